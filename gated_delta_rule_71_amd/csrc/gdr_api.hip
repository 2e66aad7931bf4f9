// C ABI of libgdr.so: argument validation and kernel dispatch.
// Every check runs before the first HIP call, so a rejected call launches nothing.  The only
// mutable global state is the allocation-free prefill's scratch array and its per-device address.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "gdr.h"
#include "gdr_common.h"

#define GDR_EXPORT extern "C" __attribute__((visibility("default")))

namespace gdr {
template <typename IO>
hipError_t launch_decode(const IO* q, const IO* k, const IO* v, const IO* la, const IO* bg,
                         const IO* wg, float* S, IO* o, int64_t B, int64_t H, int64_t Hk,
                         int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind,
                         bool decay_first, hipStream_t stream);
template <typename IO>
hipError_t launch_prefill(const IO* q, const IO* k, const IO* v, const IO* la, const IO* bg,
                          const IO* wg, const float* S0, IO* o, float* S_T, int64_t B, int64_t T,
                          int64_t H, int64_t Hk, int64_t DK, int64_t DV, int alpha_kind,
                          int b_kind, int w_kind, bool decay_first, void* workspace,
                          hipEvent_t mark, hipStream_t stream);
bool prefill_supported(int io_dtype, int64_t DK, int64_t DV, int alpha_kind, bool decay_first);
bool backward_supported(int io_dtype_bf16, int64_t DK, int64_t DV, int alpha_kind);
size_t backward_workspace_bytes(int64_t B, int64_t H, int64_t Hk, int64_t T, int64_t DK, int64_t DV);
hipError_t launch_backward(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* la,
                           const bf16_t* bg, const bf16_t* wg, const float* S0, const bf16_t* dO,
                           const float* dST, bf16_t* dq, bf16_t* dk, bf16_t* dv, bf16_t* dla,
                           bf16_t* db, bf16_t* dw, float* dS0, int64_t B, int64_t T, int64_t H,
                           int64_t Hk, int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind,
                           bool decay_first, void* workspace, hipStream_t s);
size_t backward_tok_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV);
hipError_t launch_backward_tok(bool io_bf16, const void* q, const void* k, const void* v, const void* la,
                               const void* bg, const void* wg, const float* S0, const void* dO,
                               const float* dST, void* dq, void* dk, void* dv, void* dla, void* db,
                               void* dw, float* dS0, int64_t B, int64_t T, int64_t H, int64_t Hk,
                               int64_t DK, int64_t DV, int alpha_kind, int b_kind, int w_kind,
                               bool decay_first, void* workspace, hipStream_t s);
size_t prefill_workspace_bytes(int io_dtype, int64_t nstate, int64_t T, int64_t DK, int64_t DV,
                               int alpha_kind, int b_kind, int w_kind, bool decay_first);
}  // namespace gdr

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxRows = int64_t(1) << 48;  // batch x seqlen x heads

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

int check_problem(const gdr_problem* p) {
  if (p == nullptr) return GDR_ERR_INVALID_ARGUMENT;
  if (p->struct_size != (int32_t)sizeof(gdr_problem)) return GDR_ERR_INVALID_ARGUMENT;
  if (p->qk_heads < 0 || (p->qk_heads > 0 && p->heads % p->qk_heads != 0))
    return GDR_ERR_INVALID_ARGUMENT;
  if (p->io_dtype != GDR_BF16 && p->io_dtype != GDR_FP32) return GDR_ERR_INVALID_ARGUMENT;
  for (int32_t kind : {p->alpha_kind, p->b_kind, p->w_kind})
    if (kind < GDR_GATE_NONE || kind > GDR_GATE_CHANNEL) return GDR_ERR_INVALID_ARGUMENT;
  if (p->order != GDR_ERASE_THEN_DECAY && p->order != GDR_DECAY_THEN_ERASE)
    return GDR_ERR_INVALID_ARGUMENT;
  if (p->batch < 0 || p->heads < 0 || p->seqlen < 0 || p->dk <= 0 || p->dv <= 0)
    return GDR_ERR_INVALID_ARGUMENT;
  if (p->batch >= kMaxDim || p->heads >= kMaxDim || p->seqlen >= kMaxDim)
    return GDR_ERR_INVALID_ARGUMENT;
  if (p->dk != 16 && p->dk != 32 && p->dk != 64 && p->dk != 128 && p->dk != 256) return GDR_ERR_UNSUPPORTED;
  if (p->dv % 16 != 0 || p->dv > 256) return GDR_ERR_UNSUPPORTED;
  if (p->chunk != 0 && p->chunk != 64) return GDR_ERR_UNSUPPORTED;
  // index arithmetic inside the kernels is 64-bit; grids are 32-bit
  if (p->batch * p->heads >= kMaxDim / 64) return GDR_ERR_UNSUPPORTED;
  // byte counts of the tensors (rows x width x 4 at most) and workspaces stay far inside int64
  // (batch x heads < 2^25 and seqlen < 2^31 here, so the product itself cannot overflow)
  if (p->batch * p->heads * p->seqlen >= kMaxRows) return GDR_ERR_UNSUPPORTED;
  return GDR_OK;
}

// Pointer checks shared by both entry points.  `nt` = tokens per (batch, head).
// q / k heads of a validated problem
int64_t qk_heads(const gdr_problem* p) { return p->qk_heads > 0 ? p->qk_heads : p->heads; }

int check_tensors(const gdr_problem* p, int64_t nt, const void* q, const void* k, const void* v,
                  const void* la, const void* b, const void* w, const void* o) {
  const int64_t rows = p->batch * nt * p->heads;
  const int64_t qk_rows = p->batch * nt * qk_heads(p);
  if (rows == 0) return GDR_OK;
  if (!q || !k || !v || !o) return GDR_ERR_INVALID_ARGUMENT;
  if ((p->alpha_kind != GDR_GATE_NONE && !la) || (p->b_kind != GDR_GATE_NONE && !b) ||
      (p->w_kind != GDR_GATE_NONE && !w))
    return GDR_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q, k, v, o, p->alpha_kind ? la : nullptr, p->b_kind ? b : nullptr,
                        p->w_kind ? w : nullptr};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return GDR_ERR_MISALIGNED;
  const int64_t es = p->io_dtype == GDR_BF16 ? 2 : 4;
  auto gate_bytes = [&](int32_t kind, int64_t width) {
    return kind == GDR_GATE_SCALAR ? rows * es : rows * width * es;
  };
  const Range ro = range_of(o, rows * p->dv * es);
  const Range ins[] = {range_of(q, qk_rows * p->dk * es), range_of(k, qk_rows * p->dk * es),
                       range_of(v, rows * p->dv * es),
                       p->alpha_kind ? range_of(la, gate_bytes(p->alpha_kind, p->dk)) : Range{0, 0},
                       p->b_kind ? range_of(b, gate_bytes(p->b_kind, p->dk)) : Range{0, 0},
                       p->w_kind ? range_of(w, gate_bytes(p->w_kind, p->dv)) : Range{0, 0}};
  for (const Range& r : ins)
    if (overlaps(ro, r)) return GDR_ERR_INVALID_ARGUMENT;
  return GDR_OK;
}

const void* gate_ptr(int32_t kind, const void* ptr) { return kind == GDR_GATE_NONE ? nullptr : ptr; }

}  // namespace

GDR_EXPORT int gdr_abi_version(void) { return GDR_ABI_VERSION; }

GDR_EXPORT const char* gdr_status_string(int status) {
  switch (status) {
    case GDR_OK: return "GDR_OK: success";
    case GDR_ERR_INVALID_ARGUMENT:
      return "GDR_ERR_INVALID_ARGUMENT: NULL pointer, negative size, bad enum value, struct_size "
             "mismatch or overlapping output";
    case GDR_ERR_UNSUPPORTED:
      return "GDR_ERR_UNSUPPORTED: dk must be 16, 32, 64, 128 or 256, dv a multiple of 16 up to 256, "
             "chunk 64";
    case GDR_ERR_MISALIGNED: return "GDR_ERR_MISALIGNED: tensor pointers must be 16-byte aligned";
    case GDR_ERR_WORKSPACE_TOO_SMALL:
      return "GDR_ERR_WORKSPACE_TOO_SMALL: workspace below the query (for gdr_chunk_fwd_noalloc: the "
             "problem needs more than the library's GDR_NOALLOC_SCRATCH_BYTES array)";
    case GDR_ERR_HIP: return "GDR_ERR_HIP: the HIP runtime reported an error at launch";
    default: return "unknown gdr_status";
  }
}

GDR_EXPORT size_t gdr_chunk_fwd_workspace_bytes(const gdr_problem* p) {
  if (check_problem(p) != GDR_OK) return 0;
  return gdr::prefill_workspace_bytes(p->io_dtype, p->batch * p->heads, p->seqlen, p->dk, p->dv,
                                      p->alpha_kind, p->b_kind, p->w_kind, p->order == GDR_DECAY_THEN_ERASE);
}

namespace {
// Every check of a prefill call except those of the workspace.
int check_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
              const void* log_alpha, const void* b, const void* w, const float* S0, const void* o,
              const float* S_T) {
  int rc = check_problem(p);
  if (rc != GDR_OK) return rc;
  rc = check_tensors(p, p->seqlen, q, k, v, log_alpha, b, w, o);
  if (rc != GDR_OK) return rc;
  const int64_t nstate = p->batch * p->heads;
  if (nstate == 0) return GDR_OK;
  if ((S0 && !aligned16(S0)) || (S_T && !aligned16(S_T))) return GDR_ERR_MISALIGNED;
  const int64_t sbytes = nstate * p->dk * p->dv * 4;
  if (S0 && S_T && S0 != S_T && overlaps(range_of(S0, sbytes), range_of(S_T, sbytes)))
    return GDR_ERR_INVALID_ARGUMENT;
  const int64_t es = p->io_dtype == GDR_BF16 ? 2 : 4;
  const int64_t rows = p->batch * p->seqlen * p->heads;
  if (S_T && rows && overlaps(range_of(S_T, sbytes), range_of(o, rows * p->dv * es)))
    return GDR_ERR_INVALID_ARGUMENT;
  if (!gdr::prefill_supported(p->io_dtype, p->dk, p->dv, p->alpha_kind,
                              p->order == GDR_DECAY_THEN_ERASE))
    return GDR_ERR_UNSUPPORTED;
  return GDR_OK;
}

// The launches of a validated prefill call.
int launch_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
               const void* log_alpha, const void* b, const void* w, const float* S0, void* o,
               float* S_T, void* workspace, void* stream, void* mark) {
  if (p->batch * p->heads == 0) return GDR_OK;
  const bool decay_first = p->order == GDR_DECAY_THEN_ERASE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->io_dtype == GDR_BF16) {
    using T = gdr::bf16_t;
    e = gdr::launch_prefill<T>(
        (const T*)q, (const T*)k, (const T*)v, (const T*)gate_ptr(p->alpha_kind, log_alpha),
        (const T*)gate_ptr(p->b_kind, b), (const T*)gate_ptr(p->w_kind, w), S0, (T*)o, S_T,
        p->batch, p->seqlen, p->heads, qk_heads(p), p->dk, p->dv, p->alpha_kind, p->b_kind, p->w_kind,
        decay_first, workspace, static_cast<hipEvent_t>(mark), s);
  } else {
    e = gdr::launch_prefill<float>(
        (const float*)q, (const float*)k, (const float*)v,
        (const float*)gate_ptr(p->alpha_kind, log_alpha), (const float*)gate_ptr(p->b_kind, b),
        (const float*)gate_ptr(p->w_kind, w), S0, (float*)o, S_T, p->batch, p->seqlen, p->heads,
        qk_heads(p), p->dk, p->dv, p->alpha_kind, p->b_kind, p->w_kind, decay_first, workspace,
        static_cast<hipEvent_t>(mark), s);
  }
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
              const void* log_alpha, const void* b, const void* w, const float* S0, void* o,
              float* S_T, void* workspace, size_t workspace_bytes, void* stream, void* mark) {
  const int rc = check_fwd(p, q, k, v, log_alpha, b, w, S0, o, S_T);
  if (rc != GDR_OK) return rc;
  if (p->batch * p->heads == 0) return GDR_OK;
  const size_t need = gdr_chunk_fwd_workspace_bytes(p);
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && workspace == nullptr) return GDR_ERR_INVALID_ARGUMENT;
  if (need > 0 && !aligned16(workspace)) return GDR_ERR_MISALIGNED;
  return launch_fwd(p, q, k, v, log_alpha, b, w, S0, o, S_T, workspace, stream, mark);
}
}  // namespace

GDR_EXPORT int gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                             const void* log_alpha, const void* b, const void* w, const float* S0,
                             void* o, float* S_T, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return chunk_fwd(p, q, k, v, log_alpha, b, w, S0, o, S_T, workspace, workspace_bytes, stream,
                   nullptr);
}

GDR_EXPORT int gdr_chunk_fwd_marked(const gdr_problem* p, const void* q, const void* k,
                                    const void* v, const void* log_alpha, const void* b,
                                    const void* w, const float* S0, void* o, float* S_T,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* phase_event) {
  return chunk_fwd(p, q, k, v, log_alpha, b, w, S0, o, S_T, workspace, workspace_bytes, stream,
                   phase_event);
}

// ---- the allocation-free prefill: its workspace is a file-scope device array ----

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // GDR_NOALLOC_SCRATCH_BYTES in gdr.h
static_assert(kScratchBytes == GDR_NOALLOC_SCRATCH_BYTES, "header and library agree");

// One copy per GPU the library runs on, for the life of the process.  Host code never uses this
// name as an address: the device address comes from hipGetSymbolAddress, per device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device (NULL on failure).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

GDR_EXPORT int gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k,
                                     const void* v, const void* log_alpha, const void* b,
                                     const void* w, const float* S0, void* o, float* S_T,
                                     void* stream) {
  const int rc = check_fwd(p, q, k, v, log_alpha, b, w, S0, o, S_T);
  if (rc != GDR_OK) return rc;
  if (p->batch * p->heads == 0) return GDR_OK;
  const size_t need = gdr_chunk_fwd_workspace_bytes(p);
  if (need > kScratchBytes) return GDR_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (ws == nullptr) return GDR_ERR_HIP;
  }
  return launch_fwd(p, q, k, v, log_alpha, b, w, S0, o, S_T, ws, stream, nullptr);
}

GDR_EXPORT int gdr_decode_step(const gdr_problem* p, const void* q, const void* k, const void* v,
                               const void* log_alpha, const void* b, const void* w, float* S,
                               void* o, void* stream) {
  int rc = check_problem(p);
  if (rc != GDR_OK) return rc;
  if (p->seqlen != 1) return GDR_ERR_INVALID_ARGUMENT;
  rc = check_tensors(p, 1, q, k, v, log_alpha, b, w, o);
  if (rc != GDR_OK) return rc;
  const int64_t nstate = p->batch * p->heads;
  if (nstate == 0) return GDR_OK;
  if (!S) return GDR_ERR_INVALID_ARGUMENT;
  if (!aligned16(S)) return GDR_ERR_MISALIGNED;
  const int64_t es = p->io_dtype == GDR_BF16 ? 2 : 4;
  if (overlaps(range_of(S, nstate * p->dk * p->dv * 4), range_of(o, nstate * p->dv * es)))
    return GDR_ERR_INVALID_ARGUMENT;
  const bool decay_first = p->order == GDR_DECAY_THEN_ERASE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->io_dtype == GDR_BF16) {
    using T = gdr::bf16_t;
    e = gdr::launch_decode<T>((const T*)q, (const T*)k, (const T*)v,
                              (const T*)gate_ptr(p->alpha_kind, log_alpha),
                              (const T*)gate_ptr(p->b_kind, b), (const T*)gate_ptr(p->w_kind, w), S,
                              (T*)o, p->batch, p->heads, qk_heads(p), p->dk, p->dv, p->alpha_kind, p->b_kind,
                              p->w_kind, decay_first, s);
  } else {
    e = gdr::launch_decode<float>((const float*)q, (const float*)k, (const float*)v,
                                  (const float*)gate_ptr(p->alpha_kind, log_alpha),
                                  (const float*)gate_ptr(p->b_kind, b),
                                  (const float*)gate_ptr(p->w_kind, w), S, (float*)o, p->batch,
                                  p->heads, qk_heads(p), p->dk, p->dv, p->alpha_kind, p->b_kind, p->w_kind,
                                  decay_first, s);
  }
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

namespace {
// the chunkwise backward's shapes; every other valid problem runs the token adjoint
bool bwd_chunkwise(const gdr_problem* p) {
  return gdr::backward_supported(p->io_dtype == GDR_BF16, p->dk, p->dv, p->alpha_kind);
}
}  // namespace

GDR_EXPORT size_t gdr_chunk_bwd_workspace_bytes(const gdr_problem* p) {
  if (check_problem(p) != GDR_OK) return 0;
  if (bwd_chunkwise(p))
    return gdr::backward_workspace_bytes(p->batch, p->heads, qk_heads(p), p->seqlen, p->dk, p->dv);
  return gdr::backward_tok_workspace_bytes(p->batch, p->heads, p->seqlen, p->dk, p->dv);
}

GDR_EXPORT int gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                             const void* log_alpha, const void* b, const void* w, const float* S0,
                             const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                             void* dlog_alpha, void* db, void* dw, float* dS0, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != GDR_OK) return rc;
  // the forward's inputs against one of the outputs (dv), then every output pairwise below
  rc = check_tensors(p, p->seqlen, q, k, v, log_alpha, b, w, dv);
  if (rc != GDR_OK) return rc;
  const int64_t nstate = p->batch * p->heads;
  const int64_t rows = p->batch * p->seqlen * p->heads;
  const int64_t qk_rows = p->batch * p->seqlen * qk_heads(p);
  if (nstate == 0) return GDR_OK;
  const int64_t sbytes = nstate * p->dk * p->dv * 4;
  if (rows > 0) {
    if (!dO || !dq || !dk) return GDR_ERR_INVALID_ARGUMENT;
    if ((p->alpha_kind != GDR_GATE_NONE && !dlog_alpha) || (p->b_kind != GDR_GATE_NONE && !db) ||
        (p->w_kind != GDR_GATE_NONE && !dw))
      return GDR_ERR_INVALID_ARGUMENT;
  }
  const void* dla_ = gate_ptr(p->alpha_kind, dlog_alpha);
  const void* db_ = gate_ptr(p->b_kind, db);
  const void* dw_ = gate_ptr(p->w_kind, dw);
  for (const void* ptr : {(const void*)S0, dO, (const void*)dS_T, (const void*)dq, (const void*)dk,
                          dla_, db_, dw_, (const void*)dS0, (const void*)workspace})
    if (ptr && !aligned16(ptr)) return GDR_ERR_MISALIGNED;
  const int64_t es = p->io_dtype == GDR_BF16 ? 2 : 4;
  auto gate_bytes = [&](int32_t kind, int64_t width) {
    return kind == GDR_GATE_SCALAR ? rows * es : kind == GDR_GATE_CHANNEL ? rows * width * es : 0;
  };
  const Range outs[] = {range_of(dq, dq ? qk_rows * p->dk * es : 0), range_of(dk, dk ? qk_rows * p->dk * es : 0),
                        range_of(dv, rows * p->dv * es),
                        range_of(dla_, gate_bytes(p->alpha_kind, p->dk)),
                        range_of(db_, gate_bytes(p->b_kind, p->dk)),
                        range_of(dw_, gate_bytes(p->w_kind, p->dv)),
                        range_of(dS0, dS0 ? sbytes : 0)};
  const Range ins[] = {range_of(q, qk_rows * p->dk * es), range_of(k, qk_rows * p->dk * es),
                       range_of(v, rows * p->dv * es),
                       range_of(gate_ptr(p->alpha_kind, log_alpha), gate_bytes(p->alpha_kind, p->dk)),
                       range_of(gate_ptr(p->b_kind, b), gate_bytes(p->b_kind, p->dk)),
                       range_of(gate_ptr(p->w_kind, w), gate_bytes(p->w_kind, p->dv)),
                       range_of(S0, S0 ? sbytes : 0), range_of(dO, dO ? rows * p->dv * es : 0),
                       range_of(dS_T, dS_T ? sbytes : 0)};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return GDR_ERR_INVALID_ARGUMENT;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlaps(outs[i], outs[j])) return GDR_ERR_INVALID_ARGUMENT;
  }
  const size_t need = gdr_chunk_bwd_workspace_bytes(p);
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && workspace == nullptr) return GDR_ERR_INVALID_ARGUMENT;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool df = p->order == GDR_DECAY_THEN_ERASE;
  hipError_t e;
  if (bwd_chunkwise(p)) {
    using T = gdr::bf16_t;
    e = gdr::launch_backward(
        (const T*)q, (const T*)k, (const T*)v, (const T*)gate_ptr(p->alpha_kind, log_alpha),
        (const T*)gate_ptr(p->b_kind, b), (const T*)gate_ptr(p->w_kind, w), S0, (const T*)dO, dS_T,
        (T*)dq, (T*)dk, (T*)dv, (T*)dla_, (T*)db_, (T*)dw_, dS0, p->batch, p->seqlen, p->heads, qk_heads(p), p->dk,
        p->dv, p->alpha_kind, p->b_kind, p->w_kind, df, workspace, st);
  } else {
    e = gdr::launch_backward_tok(p->io_dtype == GDR_BF16, q, k, v, gate_ptr(p->alpha_kind, log_alpha),
                                 gate_ptr(p->b_kind, b), gate_ptr(p->w_kind, w), S0, dO, dS_T, dq, dk, dv,
                                 (void*)dla_, (void*)db_, (void*)dw_, dS0, p->batch, p->seqlen, p->heads,
                                 qk_heads(p), p->dk, p->dv, p->alpha_kind, p->b_kind, p->w_kind, df,
                                 workspace, st);
  }
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}
