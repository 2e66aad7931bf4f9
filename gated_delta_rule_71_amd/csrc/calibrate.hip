// Calibration probe: the bf16 matrix-core rate this GPU sustains on a loop of independent
// 16x16x32 MFMAs with register operands and no memory traffic.  It is context for the roofline
// figures (the dense bf16 peak is a vendor number); it computes nothing of the method.
#include "gdr.h"
#include "gdr_common.h"
#include "mfma.h"

namespace gdr {
namespace {

constexpr int kProbeThreads = 512;  // two waves per SIMD
constexpr int kProbeChains = 8;     // independent accumulators per wave

// Every operand element is 1/16 (exact in bf16), so each MFMA adds 32 / 256 = 1/8 to each
// accumulator element: after `iters` steps a lane's sum over its 8 x 4 accumulator elements is
// exactly 4 * iters.  Wave w of workgroup b writes that sum to out[b * 8 + w].
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int64_t iters, float* out) {
  using MM = Mma<__bf16>;
  MM::F8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.0625f);
    b[e] = static_cast<__bf16>(0.0625f);
  }
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = MM::mma8(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64] = s;
}

}  // namespace
}  // namespace gdr

#define GDR_EXPORT extern "C" __attribute__((visibility("default")))

GDR_EXPORT int gdr_mfma_probe(int64_t iters, int32_t blocks, float* out, void* stream) {
  if (iters < 0 || blocks <= 0 || blocks > 65535 || out == nullptr) return GDR_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(gdr::mfma_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(gdr::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

GDR_EXPORT int64_t gdr_mfma_probe_flop(int64_t iters, int32_t blocks) {
  return iters * static_cast<int64_t>(blocks) * (gdr::kProbeThreads / 64) * gdr::kProbeChains * 16 * 16 * 32 * 2;
}
