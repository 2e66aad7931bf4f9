/*
 * gdr.h -- C ABI of libgdr.so: the generalized gated delta-rule recurrence on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (row-vector convention, one dk x dv fp32 state S per
 * (batch, head)):
 *
 *   S_t = Diag(alpha_t) (I - k_t^T (b_t . k_t)) S_{t-1} + k_t^T (w_t . v_t)
 *   o_t = q_t S_t
 *
 * "Recurrent Memory: Write, Erase, Decay, Read", section 05 (the unified
 * equation: decay x erase x state + write) with the read of section 01; the
 * erase gate b_t (key side) and the write gate w_t (value side) are the
 * channel-wise gates of the Gated DeltaNet-2 abstract, which reduce to the
 * single beta of section 05 when b_t = w_t = beta_t.  The read sees the
 * token's own write ("How Linear Attention Remembers", Analytical Framework:
 * o_t = q_t^T S_t).  With GDR_DECAY_THEN_ERASE the decay is applied to
 * S_{t-1} before the erase reads it instead; the two orders coincide for a
 * scalar alpha.
 *
 * Special settings (same section 05): b = 0, alpha = 1 is linear attention;
 * b = w = beta, alpha = 1 is DeltaNet; b = 0 with a decay is GLA / Mamba-2;
 * scalar alpha with b = w = beta is Gated DeltaNet; per-channel alpha with
 * b = w = beta is KDA; per-channel alpha, b and w is Gated DeltaNet-2.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller, row-major and
 *   contiguous, 16-byte aligned.  The library never allocates, frees or keeps
 *   them.  Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream); outputs are valid once the stream has reached the call.
 * - Per-token tensors are laid out [B, T, H, D]: q, k [B,T,Hqk,dk] with
 *   Hqk = qk_heads (or H when that is 0); v, o [B,T,H,dv].  Gates: log_alpha [B,T,H] (SCALAR) or [B,T,H,dk]
 *   (CHANNEL); b [B,T,H] or [B,T,H,dk]; w [B,T,H] or [B,T,H,dv].  A gate of
 *   kind NONE ignores its pointer (may be NULL) and means alpha = 1, b = 0,
 *   w = 1.  Gates are given as log alpha (<= 0 for a contraction; any finite
 *   value is accepted) and as plain values for b and w (no sigmoid is applied).
 * - q, k, v, the gates and o share io_dtype (bf16 or fp32).  The state is fp32
 *   [B, H, dk, dv] (dv fastest).  Arithmetic is fp32 with bf16 (GDR_BF16) or
 *   fp32 (GDR_FP32) matrix-core operands.
 * - Validation happens before any HIP call; a call that fails validation
 *   launches nothing and touches no memory.  A failed kernel launch returns
 *   GDR_ERR_HIP.  No exception or abort crosses the ABI.  Apart from the
 *   scratch array of gdr_chunk_fwd_noalloc, the library keeps no mutable global
 *   state; concurrent calls on different streams are safe when their buffers
 *   do not overlap.
 * - NaN or Inf in the inputs propagate to the outputs; they are not detected.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 2

typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, negative size, bad enum, struct_size */
  GDR_ERR_UNSUPPORTED = 2,      /* valid but not built: dk, dv or chunk outside the list below */
  GDR_ERR_MISALIGNED = 3,       /* a tensor pointer is not 16-byte aligned */
  GDR_ERR_WORKSPACE_TOO_SMALL = 4,
  GDR_ERR_HIP = 5               /* the HIP runtime reported an error at launch */
} gdr_status;

typedef enum { GDR_BF16 = 0, GDR_FP32 = 1 } gdr_dtype;
typedef enum { GDR_GATE_NONE = 0, GDR_GATE_SCALAR = 1, GDR_GATE_CHANNEL = 2 } gdr_gate;
typedef enum { GDR_ERASE_THEN_DECAY = 0, GDR_DECAY_THEN_ERASE = 1 } gdr_order;

/* Problem description.  Set struct_size = sizeof(gdr_problem).
 * Supported by the prefill, the decode step and the backward: dk in
 * {16, 32, 64, 128, 256}, dv a multiple of 16 in [16, 256], both I/O types,
 * every gate kind and both orders (GDR_ERR_UNSUPPORTED otherwise).  chunk == 64 or 0 (the same); batch, heads >= 0; seqlen >= 0
 * (any value: a ragged last chunk is padded with identity tokens inside the
 * kernel).  Sizes: batch, heads and seqlen below 2^31 (GDR_ERR_INVALID_ARGUMENT
 * otherwise), batch * heads below 2^25 and batch * heads * seqlen below 2^48
 * (GDR_ERR_UNSUPPORTED otherwise).  The chunk length does not change the result, which equals the
 * token-by-token recurrence up to rounding; the kernels block the chunkwise
 * form in 64-token chunks, except the segment kernel, which uses 32.  Which
 * kernels run:
 *   bf16, dk = dv = 128, per-channel decay with per-channel (erase and write)
 *     or scalar (both) gates, either order, or a scalar decay with scalar
 *     erase and write gates: the segment kernel (a state's chunks split into
 *     segments run side by side, then linked);
 *   other shapes: the chunkwise kernels where their LDS layout fits (every
 *     bf16 shape except dk = 256 with a per-channel decay after the erase;
 *     fp32 at dk <= 32, and at dk = 64 with a scalar, no or decay-first
 *     decay), else the recurrence token by token with the state in
 *     registers. */
typedef struct {
  int32_t struct_size;
  int32_t io_dtype;   /* gdr_dtype */
  int64_t batch, heads, seqlen, dk, dv;
  int32_t chunk;      /* chunk length of the prefill's chunkwise form */
  int32_t alpha_kind; /* gdr_gate */
  int32_t b_kind;     /* gdr_gate */
  int32_t w_kind;     /* gdr_gate */
  int32_t order;      /* gdr_order */
  int32_t qk_heads;   /* heads of q and k: 0 = `heads`; otherwise `heads` must be a multiple of
                         it, and value head h reads q / k head h / (heads / qk_heads) (grouped
                         key / value heads) */
} gdr_problem;

/* ABI version of the loaded library (GDR_ABI_VERSION). */
int gdr_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* gdr_status_string(int status);

/* Workspace bytes gdr_chunk_fwd needs for `p` (0 when none); 0 also for an
 * invalid problem.  Each array below is rounded up to 256 bytes.
 * Segment kernel (see gdr_problem): with S = batch * heads states and
 * n = ceil(seqlen / 32) chunks each, a state's chunks split into
 * m = ceil(n / L) segments of L = ceil(n / min(n, ceil(256 / S))) chunks.
 * For m = 1 none; else two arrays of S * n * 32 * 128 bf16 (per chunk, the
 * read-outs of the segment's state from zero and of its transition), three of
 * S * m * 128 * 128 fp32 (per segment, its state from zero, its transition and
 * the state leaving the first) and one of S * m * 128 * 128 bf16 (the state
 * entering each segment).
 * Other bf16 problems with dk in {32, 64, 128} run as a chunk-local kernel
 * plus a per-state kernel that exchange per-chunk matrices through the
 * workspace; per 64-token chunk of every (batch, head) that is:
 *   scalar (or no) decay, scalar (or no) erase gate: W (64 x dk), U (64 x dv)
 *     and the masked 64 x 64 read-out matrix, all bf16, and 132 floats of gate
 *     exponentials: 128 dk + 128 dv + 8720 bytes;
 *   per-channel decay (either order): the chunk's affine map of the state,
 *     S' = diag(decay) S + A S + D with read-out O = Q S + Z: A (dk x dk),
 *     Q (64 x dk), D (dv x dk) and Z (64 x dv) in bf16, the dk chunk decays
 *     plus 4 (fp32) and a flag:
 *     2 dk^2 + 2 dk dv + 132 dk + 128 dv + 20 bytes.
 * The scalar-decay form with a per-channel erase gate, the dk = 16 and the
 * fp32 problems run as one kernel and need none.  The caller owns the buffer;
 * its contents on entry do not matter. */
size_t gdr_chunk_fwd_workspace_bytes(const gdr_problem* p);

/*
 * Chunkwise prefill: runs the recurrence over all p->seqlen tokens of every
 * (batch, head) from S0 and returns every read-out o_t and the final state.
 *   q, k, v, log_alpha, b, w   inputs as described above (device, read only)
 *   S0     [B,H,dk,dv] fp32 initial state; NULL means zeros
 *   o      [B,T,H,dv] io_dtype output; must not overlap any input
 *   S_T    [B,H,dk,dv] fp32 final state; NULL means "not needed"; may alias S0
 *          (in-place update), must not partially overlap it
 *   workspace, workspace_bytes  device scratch of at least
 *          gdr_chunk_fwd_workspace_bytes(p) bytes, 16-byte aligned (may be NULL
 *          when that is 0); GDR_ERR_WORKSPACE_TOO_SMALL when smaller.  Calls
 *          that share one workspace must not overlap in time.
 * Method: the chunkwise form the "Recurrent Memory" post points to in
 * section 03 (the erase is linear, so a chunk of tokens reassociates into
 * matrix products and one unit-lower-triangular solve) with the decay entering
 * through prefix sums of log alpha (section 04) and, for a per-channel decay,
 * folded into separate erase factors as the Gated DeltaNet-2 abstract
 * describes.  The result equals the token-by-token recurrence up to rounding.
 */
int gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                  const void* log_alpha, const void* b, const void* w, const float* S0,
                  void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdr_chunk_fwd with a timing marker.  When `phase_event` (a hipEvent_t) is
 * not NULL it is recorded on `stream` between the chunk-local kernel and the
 * per-state kernel (for the segment kernel: after it, before the kernels that
 * link the segments), or just before the one kernel of a problem that runs as
 * one.  With events recorded before and after the call, the caller can time
 * the two phases separately.  No event is recorded when the call fails
 * validation or when B * H is 0.  Otherwise identical to gdr_chunk_fwd;
 * GDR_ERR_HIP when the record fails.
 */
int gdr_chunk_fwd_marked(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* b, const void* w, const float* S0,
                         void* o, float* S_T, void* workspace, size_t workspace_bytes,
                         void* stream, void* phase_event);

/* Size of the device array gdr_chunk_fwd_noalloc takes its workspace from. */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * gdr_chunk_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, with the workspace
 * taken from a GDR_NOALLOC_SCRATCH_BYTES device array inside the library instead of a caller
 * buffer.  The library holds one such array on every GPU it runs on until the process ends; its
 * address is looked up on the first call with that GPU current.  The call allocates and frees
 * nothing.  Arguments as for gdr_chunk_fwd.
 *   GDR_ERR_WORKSPACE_TOO_SMALL  when gdr_chunk_fwd_workspace_bytes(p) exceeds
 *                                GDR_NOALLOC_SCRATCH_BYTES (nothing is launched)
 *   GDR_ERR_HIP                  when the array's address cannot be obtained
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must not be issued; calls in order on
 * one stream are safe.  The array's contents on entry do not matter.
 */
int gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k, const void* v,
                          const void* log_alpha, const void* b, const void* w, const float* S0,
                          void* o, float* S_T, void* stream);

/*
 * One decode step (p->seqlen must be 1): for every (batch, head) applies the
 * recurrence to the single token and updates S in place.
 *   q, k, v, log_alpha, b, w   [B,1,H,*] inputs (same layouts with T = 1)
 *   S      [B,H,dk,dv] fp32 state, read and overwritten in place
 *   o      [B,1,H,dv] io_dtype read-out; must not overlap any input or S
 * One pass over S: the two dk-reductions (the erase read (b . k) S and the
 * query read) share a single read of S, then the updated S is written once.
 * "Recurrent Memory", section 03 (read, delta, write back) and section 05.
 */
int gdr_decode_step(const gdr_problem* p, const void* q, const void* k, const void* v,
                    const void* log_alpha, const void* b, const void* w, float* S, void* o,
                    void* stream);

/* Workspace bytes gdr_chunk_bwd needs for `p`; 0 for an invalid problem.
 * Chunkwise adjoint (the shapes listed under gdr_chunk_bwd): per 64-token chunk
 * of every (batch, head), the chunk's affine map as for the per-channel forward
 * (2 dk^2 + 2 dk dv + 132 dk + 128 dv + 20 bytes) and five bf16 dk x dv arrays:
 * the checkpoints (the state entering the chunk and the gradient of the state
 * leaving it, each as rows and transposed) and the chunk's Q'^T dO; with
 * grouped q / k heads also dq and dk per value head (bf16 [B,T,H,dk] each).
 * Token adjoint (every other problem): the fp32 state before every 8th token of
 * every (batch, head), B * H * ceil(T / 8) * dk * dv * 4 bytes, and per block of
 * 64 value columns the fp32 column sums of four per-token row gradients,
 * ceil(dv / 64) * B * T * H * (4 dk + 4) * 4 bytes.
 * Each array is 256-byte aligned. */
size_t gdr_chunk_bwd_workspace_bytes(const gdr_problem* p);

/*
 * Gradients of a chunkwise prefill: given dO (the gradient of every read-out)
 * and dS_T (of the final state), the gradients of every input of gdr_chunk_fwd
 * with the same problem.
 *   q, k, v, log_alpha, b, w, S0   the forward's inputs (device, read only)
 *   dO     [B,T,H,dv] io_dtype gradient of o
 *   dS_T   [B,H,dk,dv] fp32 gradient of S_T; NULL means zeros
 *   dq, dk [B,T,H,dk], dv [B,T,H,dv] io_dtype outputs
 *   dlog_alpha, db, dw  io_dtype outputs shaped like log_alpha, b and w (each
 *          ignored, and may be NULL, when that gate's kind is GDR_GATE_NONE);
 *          with one shared beta passed as both b and w the caller adds db and dw
 *   dS0    [B,H,dk,dv] fp32 gradient of S0; NULL means "not needed"
 *   workspace, workspace_bytes  device scratch of at least
 *          gdr_chunk_bwd_workspace_bytes(p) bytes, 16-byte aligned; calls that
 *          share one workspace must not overlap in time.
 * Outputs must not overlap the inputs or each other.  Every valid problem is
 * supported (both I/O types, every gate kind, both orders, grouped q / k heads:
 * dq and dk are then summed over the value heads that share each q / k head).
 * Two methods, chosen by shape:
 *   Chunkwise adjoint, for bf16 with a scalar decay or none (both orders are
 *   then the same recurrence), dk in {32, 64, 128} and dv a multiple of 16 up
 *   to 256, or a per-channel decay (the Gated DeltaNet-2 and KDA gates), either
 *   order, dk = 128 and dv 64 or 128: the adjoint of the chunk form of
 *   gdr_chunk_fwd ("Recurrent Memory", sections 03 and 04).  The state at
 *   every chunk boundary by a forward pass over the chunk maps, the gradient of
 *   the state at every boundary by the transposed maps in reverse, and each
 *   chunk's input gradients from those two by matrix products, the transposed
 *   triangular solve and a suffix sum of the decay gradient inside the chunk.
 *   With a per-channel decay a chunk whose prefix sums of log alpha leave
 *   [-76, 76] (or are not finite) is differentiated token by token from its
 *   checkpoint instead, exactly for any gate values.
 *   Token adjoint, for every other problem (the all-fp32 mode, dk = 16 and
 *   256, a per-channel decay at other widths): the adjoint of the recurrence
 *   itself ("Recurrent Memory", section 05), token by token in fp32, from
 *   checkpoints of the state kept every 8 tokens.  Exact for any gate values;
 *   tens of times slower than the chunkwise adjoint.
 * Results are deterministic: every sum is taken in a fixed order.
 */
int gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                  const void* log_alpha, const void* b, const void* w, const float* S0,
                  const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                  void* dlog_alpha, void* db, void* dw, float* dS0, void* workspace,
                  size_t workspace_bytes, void* stream);

/* ---- calibration (context for the roofline figures; computes nothing of the method) ----
 * gdr_mfma_probe: launches `blocks` workgroups of 512 threads on `stream`; each wave runs
 * `iters` steps of 8 independent bf16 16x16x32 matrix-core products on register operands (no
 * memory traffic) and writes one float to out[block * 8 + wave] (exactly 4 * iters: every
 * operand element is 1/16).  `out` is a device buffer of at least 8 * blocks floats, owned by
 * the caller.  Returns GDR_ERR_INVALID_ARGUMENT for iters < 0, blocks outside [1, 65535] or a
 * NULL out, GDR_ERR_HIP if the launch fails.  gdr_mfma_probe_flop: the dense FLOP one such
 * call performs (2 x 16 x 16 x 32 per product), for a rate from the caller's timing. */
int gdr_mfma_probe(int64_t iters, int32_t blocks, float* out, void* stream);
int64_t gdr_mfma_probe_flop(int64_t iters, int32_t blocks);

#ifdef __cplusplus
}
#endif
#endif /* GDR_H_ */
