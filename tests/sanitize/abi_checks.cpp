// Host-side checks of libgdr's C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// from host-only objects of the library (no device code, no GPU).  Every call below must return
// before the library makes any HIP call: invalid arguments, empty problems, undersized
// workspaces and the workspace queries.  The program prints one line per failed expectation and
// exits with the number of failures; the sanitizers abort on the first memory or UB error.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdr.h"

static int g_fail = 0;

#define EXPECT_EQ(got, want)                                                                   \
  do {                                                                                         \
    const long long g_ = (long long)(got), w_ = (long long)(want);                             \
    if (g_ != w_) {                                                                            \
      printf("FAIL %s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #got, g_, w_);      \
      ++g_fail;                                                                                \
    }                                                                                          \
  } while (0)

static gdr_problem problem(int32_t dtype, int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                           int32_t a, int32_t b, int32_t w, int32_t order) {
  gdr_problem p;
  memset(&p, 0, sizeof(p));
  p.struct_size = (int32_t)sizeof(gdr_problem);
  p.io_dtype = dtype;
  p.batch = B;
  p.heads = H;
  p.seqlen = T;
  p.dk = dk;
  p.dv = dv;
  p.chunk = 0;
  p.alpha_kind = a;
  p.b_kind = b;
  p.w_kind = w;
  p.order = order;
  p.qk_heads = 0;
  return p;
}

// 16-byte aligned host buffer with room for a small problem's tensors (never dereferenced by the
// library: it only compares addresses before rejecting the call)
struct Buf {
  unsigned char* base;
  explicit Buf(size_t n) { base = static_cast<unsigned char*>(aligned_alloc(256, n)); memset(base, 0, n); }
  ~Buf() { free(base); }
  void* at(size_t off) const { return base + off; }
};

static void status_strings() {
  for (int s = -3; s < 10; ++s) {
    const char* t = gdr_status_string(s);
    if (t == nullptr || strlen(t) == 0) {
      printf("FAIL status string %d\n", s);
      ++g_fail;
    }
  }
  EXPECT_EQ(gdr_abi_version(), GDR_ABI_VERSION);
}

// The workspace queries over every gate, order, dtype, width and a spread of sizes, including
// the largest the validation admits: they must not overflow or read past anything.
static void workspace_queries() {
  const int64_t dks[] = {8, 16, 32, 64, 96, 128, 256, 512};
  const int64_t dvs[] = {8, 16, 48, 128, 144, 256, 272};
  const int64_t sizes[][3] = {{0, 0, 0},       {1, 1, 0},          {1, 1, 1},         {1, 16, 32768},
                              {2, 32, 8192},   {4, 16, 4096},      {1, 1, (1LL << 31) - 1},
                              {1LL << 12, 1LL << 12, 1LL << 24},   {(1LL << 25) - 1, 1, 1LL << 23},
                              {1, (1LL << 25) - 1, (1LL << 23) - 1}, {-1, 1, 1}, {1, -1, 1}, {1, 1, -1},
                              {1LL << 31, 1, 1}};
  unsigned long long sink = 0;  // (wraps harmlessly)
  for (int32_t dt = 0; dt < 3; ++dt)
    for (int64_t dk : dks)
      for (int64_t dv : dvs)
        for (int32_t a = -1; a <= 3; ++a)
          for (int32_t b = 0; b <= 2; ++b)
            for (int32_t w = 0; w <= 2; ++w)
              for (int32_t order = 0; order <= 2; ++order)
                for (const auto& s : sizes) {
                  gdr_problem p = problem(dt, s[0], s[1], s[2], dk, dv, a, b, w, order);
                  sink += (unsigned long long)gdr_chunk_fwd_workspace_bytes(&p);
                  sink += (unsigned long long)gdr_chunk_bwd_workspace_bytes(&p);
                  p.qk_heads = s[1] > 1 ? 1 : 0;
                  sink += (unsigned long long)gdr_chunk_fwd_workspace_bytes(&p);
                }
  EXPECT_EQ(gdr_chunk_fwd_workspace_bytes(nullptr), 0);
  EXPECT_EQ(gdr_chunk_bwd_workspace_bytes(nullptr), 0);
  // a zero-state or one-segment segment-path problem needs no workspace; the documented formula
  // for the Gated DeltaNet-2 shape (16 states, 1024 chunks, 16 segments)
  gdr_problem p = problem(GDR_BF16, 1, 16, 32768, 128, 128, 2, 2, 2, 0);
  const unsigned long long r = 256;
  auto up = [&](unsigned long long n) { return (n + r - 1) / r * r; };
  const unsigned long long per = 16ull * 16 * 128 * 128;
  EXPECT_EQ(gdr_chunk_fwd_workspace_bytes(&p),
            2 * up(16ull * 1024 * 32 * 128 * 2) + 3 * up(per * 4) + up(per * 2));
  p.heads = 256;
  p.seqlen = 32;
  EXPECT_EQ(gdr_chunk_fwd_workspace_bytes(&p), 0);
  if (sink == 42) printf(" ");  // keep the loop's calls
}

static void invalid_calls() {
  Buf m(1 << 20);
  const size_t X = 1 << 16;  // per-tensor stride inside the buffer
  void *q = m.at(0), *k = m.at(X), *v = m.at(2 * X), *la = m.at(3 * X), *bb = m.at(4 * X), *w = m.at(5 * X);
  void* o = m.at(6 * X);
  float* S0 = static_cast<float*>(m.at(8 * X));
  float* ST = static_cast<float*>(m.at(12 * X));
  gdr_problem good = problem(GDR_BF16, 1, 1, 64, 16, 16, 2, 2, 2, 0);

  // NULL problem, wrong struct size, bad enums, negative sizes
  EXPECT_EQ(gdr_chunk_fwd(nullptr, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  gdr_problem p = good;
  p.struct_size = 8;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  p = good;
  p.io_dtype = 7;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  p = good;
  p.alpha_kind = 3;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  p = good;
  p.order = 2;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  p = good;
  p.seqlen = -1;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  p = good;
  p.qk_heads = 3;
  p.heads = 4;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  // unsupported widths and chunk, and sizes past the documented bounds
  p = good;
  p.dk = 48;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_UNSUPPORTED);
  p = good;
  p.dv = 24;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_UNSUPPORTED);
  p = good;
  p.chunk = 32;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_UNSUPPORTED);
  p = good;
  p.batch = 1 << 20;
  p.heads = 1 << 5;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_UNSUPPORTED);
  p = good;
  p.batch = 1 << 12;
  p.heads = 1 << 12;
  p.seqlen = 1 << 24;
  EXPECT_EQ(gdr_chunk_fwd(&p, q, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_UNSUPPORTED);
  // NULL tensors, a NULL gate whose kind is not NONE, misaligned pointers, o overlapping an input
  EXPECT_EQ(gdr_chunk_fwd(&good, nullptr, k, v, la, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_chunk_fwd(&good, q, k, v, nullptr, bb, w, S0, o, ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_chunk_fwd(&good, q, k, v, la, bb, w, S0, m.at(6 * X + 2), ST, nullptr, 0, nullptr), GDR_ERR_MISALIGNED);
  EXPECT_EQ(gdr_chunk_fwd(&good, q, k, v, la, bb, w, S0, m.at(2 * X + 64), ST, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_chunk_fwd(&good, q, k, v, la, bb, w, static_cast<float*>(m.at(8 * X + 4)), o, ST, nullptr, 0, nullptr),
            GDR_ERR_MISALIGNED);
  // S_T overlapping S0 without being equal to it, and S_T overlapping o
  EXPECT_EQ(gdr_chunk_fwd(&good, q, k, v, la, bb, w, S0, o, S0 + 16, nullptr, 0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_chunk_fwd(&good, q, k, v, la, bb, w, S0, o, static_cast<float*>(o), nullptr, 0, nullptr),
            GDR_ERR_INVALID_ARGUMENT);
  // empty problems launch nothing and succeed
  p = good;
  p.batch = 0;
  EXPECT_EQ(gdr_chunk_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, 0, nullptr), GDR_OK);
  EXPECT_EQ(gdr_chunk_fwd_noalloc(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, nullptr), GDR_OK);
  EXPECT_EQ(gdr_decode_step(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
            GDR_ERR_INVALID_ARGUMENT);  // decode needs seqlen == 1
  p.seqlen = 1;
  EXPECT_EQ(gdr_decode_step(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
            GDR_OK);
  // a segment-path problem with no or too small a workspace (checked before any launch).  Its
  // tensors are far larger than the buffer: the library only compares their address ranges, so
  // distinct aligned addresses 4 GiB apart stand in for them (never dereferenced)
  gdr_problem seg = problem(GDR_BF16, 1, 16, 32768, 128, 128, 2, 2, 2, 0);
  auto fake = [](int i) { return reinterpret_cast<void*>((uintptr_t)(1ull << 44) + ((uintptr_t)i << 32)); };
  void *sq = fake(0), *sk = fake(1), *sv = fake(2), *sla = fake(3), *sb = fake(4), *sw = fake(5), *so = fake(6);
  const size_t need = gdr_chunk_fwd_workspace_bytes(&seg);
  EXPECT_EQ(need > 0, 1);
  EXPECT_EQ(gdr_chunk_fwd(&seg, sq, sk, sv, sla, sb, sw, nullptr, so, nullptr, nullptr, need - 1, nullptr),
            GDR_ERR_WORKSPACE_TOO_SMALL);
  EXPECT_EQ(gdr_chunk_fwd(&seg, sq, sk, sv, sla, sb, sw, nullptr, so, nullptr, nullptr, need, nullptr),
            GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_chunk_fwd_marked(&seg, sq, sk, sv, sla, sb, sw, nullptr, so, nullptr, static_cast<unsigned char*>(fake(7)) + 1, need, nullptr,
                                 nullptr), GDR_ERR_MISALIGNED);
  // the allocation-free entry point rejects a problem needing more than its array
  EXPECT_EQ(need > GDR_NOALLOC_SCRATCH_BYTES, 1);
  EXPECT_EQ(gdr_chunk_fwd_noalloc(&seg, sq, sk, sv, sla, sb, sw, nullptr, so, nullptr, nullptr),
            GDR_ERR_WORKSPACE_TOO_SMALL);
  // decode: S missing, misaligned, overlapping o
  gdr_problem d = problem(GDR_BF16, 1, 2, 1, 16, 16, 2, 2, 2, 0);
  EXPECT_EQ(gdr_decode_step(&d, q, k, v, la, bb, w, nullptr, o, nullptr), GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_decode_step(&d, q, k, v, la, bb, w, static_cast<float*>(m.at(8 * X + 8)), o, nullptr),
            GDR_ERR_MISALIGNED);
  EXPECT_EQ(gdr_decode_step(&d, q, k, v, la, bb, w, static_cast<float*>(o), o, nullptr), GDR_ERR_INVALID_ARGUMENT);
  // backward: a per-channel decay at dk = 32 (the token adjoint) without its workspace, missing
  // outputs, outputs overlapping inputs or each other
  gdr_problem g = problem(GDR_BF16, 1, 1, 64, 32, 32, 1, 1, 1, 0);
  void *dO = m.at(7 * X), *dq = m.at(9 * X), *dk = m.at(10 * X), *dv = m.at(11 * X), *dla = m.at(13 * X);
  void *db = m.at(14 * X), *dw = m.at(15 * X);
  float* dS0 = static_cast<float*>(m.at(12 * X));
  gdr_problem gc = g;
  gc.alpha_kind = 2;
  EXPECT_EQ(gdr_chunk_bwd(&gc, q, k, v, la, bb, w, nullptr, dO, nullptr, dq, dk, dv, dla, db, dw, dS0, nullptr, 0,
                          nullptr), GDR_ERR_WORKSPACE_TOO_SMALL);
  EXPECT_EQ(gdr_chunk_bwd(&g, q, k, v, la, bb, w, nullptr, nullptr, nullptr, dq, dk, dv, dla, db, dw, dS0, nullptr,
                          0, nullptr), GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_chunk_bwd(&g, q, k, v, la, bb, w, nullptr, dO, nullptr, q, dk, dv, dla, db, dw, dS0, nullptr, 0,
                          nullptr), GDR_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(gdr_chunk_bwd(&g, q, k, v, la, bb, w, nullptr, dO, nullptr, dq, dq, dv, dla, db, dw, dS0, nullptr, 0,
                          nullptr), GDR_ERR_INVALID_ARGUMENT);
  const size_t bneed = gdr_chunk_bwd_workspace_bytes(&g);
  EXPECT_EQ(bneed > 0, 1);
  EXPECT_EQ(gdr_chunk_bwd(&g, q, k, v, la, bb, w, nullptr, dO, nullptr, dq, dk, dv, dla, db, dw, dS0, nullptr,
                          bneed - 1, nullptr), GDR_ERR_WORKSPACE_TOO_SMALL);
}

int main() {
  status_strings();
  workspace_queries();
  invalid_calls();
  printf("abi checks: %d failure(s)\n", g_fail);
  return g_fail;
}
