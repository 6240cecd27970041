/*
 * gdn.h — C ABI of the MI355X (gfx950) chunkwise gated delta rule forward.
 *
 * The method (state S is dv x dk, a read is o = S q):
 *
 *   predict-then-decay (GDN_PREDICT_THEN_DECAY, the default)
 *       S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} k_t) k_t^T,   o_t = scale * S_t q_t
 *     — the recurrence of the Gated DeltaNet GPU-parallelisation blog
 *       (m.lqnn.cn), section 1.2, here in the dv x dk orientation of the
 *       DeltaNet illustrated notes (stay-hungry-time.github.io/deltanet);
 *   decay-then-predict (GDN_DECAY_THEN_PREDICT)
 *       Sbar = S_{t-1} D_t,  S_t = Sbar + beta_t (v_t - Sbar k_t) k_t^T
 *     — the GDN / KDA worked examples of the illustrated notes'
 *       architectures section;
 *   D_t = alpha_t I for a scalar gate (GDN_GATE_SCALAR) or Diag(alpha_t),
 *   scaling the key-channel columns of S, for a vector gate
 *   (GDN_GATE_CHANNEL; GLA gating section and KDA paragraph of the notes).
 *
 * Layouts (row-major, contiguous, all device memory owned by the caller):
 *   q, k       [B, T, H, dk]   bf16 or fp32 (dtype)
 *   v          [B, T, H, dv]   same dtype as q, k
 *   alpha      [B, T, H] fp32 (scalar gate) or [B, T, H, dk] fp32 (channel)
 *   beta       [B, T, H] fp32
 *   state0     [B, H, dv, dk] fp32, or NULL for a zero start state
 *   out        [B, T, H, dv] fp32
 *   state_out  [B, H, dv, dk] fp32, or NULL if not wanted
 *   workspace  device scratch of at least gdn_workspace_bytes(...) bytes
 *
 * Ownership and lifetime: the library allocates no device memory and keeps no
 * state between calls (it has no mutable globals, so calls on different
 * streams or threads may run concurrently; the optional timer below is an
 * object the caller owns and passes in; gdn_chunk_fwd_noalloc alone keeps
 * the address of its static scratch array per device).  Buffers are
 * borrowed only for the work the call enqueues on `stream` (a hipStream_t;
 * NULL is the null stream).  Calls return after enqueueing; the caller
 * synchronises.  state_out may equal state0 (in-place continuation); out and
 * the workspace must not alias any input.  Two calls that share a workspace
 * must be ordered on one stream.
 *
 * Alignment: q, k, v, state0, out, state_out, a per-channel alpha and the
 * workspace must be 16-byte aligned, beta and a scalar alpha 4-byte aligned
 * (fresh device allocations are); otherwise the call returns GDN_E_ARG.
 *
 * Errors: every argument check runs on the host before anything is enqueued;
 * a failing check returns a negative status and enqueues nothing.  A HIP
 * launch error returns GDN_E_HIP.  NaN/Inf inputs are not checked; they
 * propagate.  gdn_status_str() names each status.
 *
 * Supported shapes: any B, H, T >= 0 (the last chunk may be short; the
 * kernels pad it with tokens that neither decay nor write, which is exact);
 * dk, dv in {16, 32, 48, ..., 128} (multiples of 16 up to 128); chunk in
 * {16, 32, 64}.  bf16 inputs with dk = dv in {64, 128}, chunk 64 run the MFMA
 * kernels; every other supported case runs the fp32 vector-ALU kernels.
 * Anything else returns GDN_E_UNSUPPORTED.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 };
enum gdn_gate { GDN_GATE_SCALAR = 0, GDN_GATE_CHANNEL = 1 };
enum gdn_order { GDN_PREDICT_THEN_DECAY = 0, GDN_DECAY_THEN_PREDICT = 1 };
enum gdn_status {
    GDN_OK = 0,
    GDN_E_ARG = -1,          /* NULL pointer where one is required, bad enum */
    GDN_E_SHAPE = -2,        /* negative or inconsistent size */
    GDN_E_UNSUPPORTED = -3,  /* valid but not built (dk, dv, chunk) */
    GDN_E_WORKSPACE = -4,    /* workspace NULL or smaller than required */
    GDN_E_HIP = -5,          /* a HIP call failed */
    GDN_E_SCRATCH = -6       /* larger than gdn_chunk_fwd_noalloc's static scratch */
};
enum gdn_path { GDN_PATH_VALU = 0, GDN_PATH_MFMA = 1 };
/* Backward algorithm (gdn_backward_path). */
enum gdn_bwd_path { GDN_BWD_TOKEN = 0, GDN_BWD_CHUNKED = 1 };

/*
 * gdn_chunk_fwd — chunkwise-parallel forward.
 *
 * Three chunk stages (DeltaNet illustrated notes, WY/UT section; gates as in
 * the GLA gating section): per chunk the UT transform of the lower-triangular
 * system built from beta and the gated K K^T (T' = (I + diag(beta) L)^{-1}
 * diag(beta)); the inter-chunk state recurrence
 * S_[i+1] = S_[i] Diag(b_C) + Delta^T Kbar with Delta = T'(V - (K (.) B') S_[i]^T)
 * (which is S_[i](I - W^T K) + U^T K when every gate is 1); and the fused
 * output O = (Q (.) B) S_[i]^T + P Delta.  Returns out and state_out.
 * The workspace holds per-chunk T' and gate prefixes.  The library picks the
 * schedule: when B * H heads are too few to occupy the device it may cut
 * every sequence into segments and run them side by side (the scheme of
 * gdn_seqpar_fwd; gdn_chunk_segments reports how many), which gives the same
 * results up to floating-point rounding.
 */
int gdn_chunk_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                  int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                  float scale,
                  const void* q, const void* k, const void* v,
                  const float* alpha, const float* beta, const float* state0,
                  float* out, float* state_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_raw — gdn_chunk_fwd on the model's raw projections, with the
 * step before the delta-rule core fused in (DeltaNet illustrated notes, block
 * description; the Gated DeltaNet GPU-parallelisation blog's projection
 * stage): q and k L2-normalised per (batch, token, head) along their
 * features (a zero vector stays zero), beta = sigmoid(beta_logit) and the
 * gate alpha = sigmoid(alpha_logit) (per head, or per key channel for
 * GDN_GATE_CHANNEL), then the forward.  The MFMA kernels keep the raw bf16 q
 * and k as exact matrix operands and apply 1/|q_t| and 1/|k_t| as fp32 row
 * factors beside the gate factors, and form log alpha = -softplus(-logit)
 * in stage 1 (no normalised copy is written); the vector-ALU family writes
 * the normalised fp32 inputs into the workspace first.  Same tensors, layouts,
 * alignment and statuses as gdn_chunk_fwd, with alpha_logit and beta_logit in
 * the places of alpha and beta; the workspace must hold
 * gdn_raw_workspace_bytes(...) bytes.  Raw q and k rows
 * must have L2 lengths between 2^-60 and 2^60 (or be zero).
 */
int gdn_chunk_fwd_raw(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                      int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                      float scale,
                      const void* q, const void* k, const void* v,
                      const float* alpha_logit, const float* beta_logit, const float* state0,
                      float* out, float* state_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes gdn_chunk_fwd_raw needs for these arguments (0 when they do
 * not validate).  Host only. */
size_t gdn_raw_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                               int32_t chunk, int32_t dtype, int32_t gate);

/*
 * gdn_chunk_fwd_noalloc — gdn_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same call without a workspace argument, running
 * the same kernels with the same results.  Its workspace is a static device
 * array of GDN_NOALLOC_SCRATCH_BYTES (128 MiB) that every GPU this entry point
 * runs on holds until the process ends; the first call on a device looks up
 * the array's address there (the only state the library keeps between
 * calls).  It allocates nothing and makes no hipMalloc/hipFree call.
 * Problems whose gdn_workspace_bytes(..., n_segments = 1) exceed that size
 * return GDN_E_SCRATCH before anything is enqueued (the main workload,
 * 2 x 16 heads x 8192 tokens at d = 128, needs 100.25 MiB).  Every call on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (different
 * streams, threads or processes sharing the device) race and must be
 * ordered by the caller.  Other statuses as for gdn_chunk_fwd.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gdn_chunk_fwd_noalloc(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                          int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                          float scale,
                          const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, const float* state0,
                          float* out, float* state_out, void* stream);

/*
 * gdn_recurrent_ref — the token-by-token recurrence on the GPU (fp32 state
 * held in registers, one lane per state row), the "fused recurrent" form the
 * illustrated notes compare the chunkwise algorithm against.  Same tensors
 * and layouts as gdn_chunk_fwd; needs no workspace.
 */
int gdn_recurrent_ref(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                      int32_t dtype, int32_t gate, int32_t order, float scale,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const float* state0,
                      float* out, float* state_out, void* stream);

/*
 * gdn_decode_step — one token on a persistent state, for generation: the
 * fixed-size-state recurrence of the DeltaNet illustrated notes' linear
 * attention as an RNN part, with the gated delta update above.  For every
 * (batch, head) it reads state_in, applies the update for the token
 * (q, k, v, gate, beta) in the given order, writes the new state to
 * state_out and the read o = scale * S q to out.  Equal to gdn_recurrent_ref
 * with T = 1.
 *   q, k       [B, H, dk]   bf16 or fp32 (dtype); v [B, H, dv], same dtype
 *   alpha      [B, H] fp32 (scalar gate) or [B, H, dk] fp32 (channel)
 *   beta       [B, H] fp32
 *   state_in   [B, H, dv, dk] fp32, or NULL for a zero state
 *   out        [B, H, dv] fp32
 *   state_out  [B, H, dv, dk] fp32, required; may equal state_in (in place)
 * Alignment: q and k on 8 bytes (bf16) or 16 bytes (fp32); state_in,
 * state_out and a channel alpha on 16 bytes; otherwise GDN_E_ARG.  Needs no
 * workspace.  dk, dv as for gdn_chunk_fwd; other statuses as above.
 */
int gdn_decode_step(int64_t B, int64_t H, int64_t dk, int64_t dv,
                    int32_t dtype, int32_t gate, int32_t order, float scale,
                    const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, const float* state_in,
                    float* out, float* state_out, void* stream);

/*
 * gdn_decode_step_raw — gdn_decode_step on the model's raw projections: the
 * kernel first forms the step's inputs the way the DeltaNet block does before
 * its delta-rule core (DeltaNet illustrated notes, block description): q and
 * k L2-normalised per (batch, head) along their features (a zero vector stays
 * zero), beta = sigmoid(beta_logit), and the gate alpha = sigmoid(alpha_logit)
 * (per head, or per key channel for GDN_GATE_CHANNEL), all in fp32.  Same
 * tensors, layouts, alignment and statuses as gdn_decode_step; alpha_logit and
 * beta_logit take the places of alpha and beta.
 */
int gdn_decode_step_raw(int64_t B, int64_t H, int64_t dk, int64_t dv,
                        int32_t dtype, int32_t gate, int32_t order, float scale,
                        const void* q, const void* k, const void* v,
                        const float* alpha_logit, const float* beta_logit,
                        const float* state_in, float* out, float* state_out, void* stream);

/*
 * gdn_backward — gradients of a scalar loss L through the forward pass (the
 * token recurrence of either order and gate kind above): given
 * grad_out = dL/d out and grad_state_out = dL/d S_T (NULL: zero), it writes
 * dL/dq, dL/dk, dL/dv, dL/dalpha, dL/dbeta and grad_state0 = dL/d S_0 (NULL:
 * not wanted).  The pages fix the forward recurrence only; the gradients are
 * its chain rule.  Two algorithms (gdn_backward_path says which runs):
 *   chunked (scalar gate, dk = dv in {64, 128}): the chain rule through the
 *     chunk form of the forward (DeltaNet illustrated notes, WY/UT section)
 *     with chunks of 64 tokens on fp32 matrix cores: per-chunk UT inverses
 *     and gated scores, a forward chain of chunk entry states and a reverse
 *     chain of state gradients, then every chunk's gradients in parallel;
 *   token (otherwise): the token recurrence run backwards, its states
 *     recomputed from boundary-state checkpoints every 16 tokens.
 * Both compute in fp32 and write every output once, in a fixed order
 * (repeated calls give identical results).
 *   q, k, v, alpha, beta, state0  as for gdn_chunk_fwd (state0 NULL: zero);
 *                   alpha > 0 (the chunked path takes its logarithm)
 *   grad_out        [B, T, H, dv] fp32
 *   grad_state_out  [B, H, dv, dk] fp32 or NULL
 *   grad_q, grad_k  [B, T, H, dk] fp32;  grad_v [B, T, H, dv] fp32
 *   grad_alpha      shaped as alpha, fp32;  grad_beta [B, T, H] fp32
 *   grad_state0     [B, H, dv, dk] fp32 or NULL
 *   workspace       at least gdn_backward_workspace_bytes(B, T, H, dk, dv,
 *                   gate) bytes; chunked: per (batch, head) and chunk of 64
 *                   tokens 4 (4 * 64^2 + 7 * 64 dk + 3 dk^2 + 8 * 64) bytes
 *                   (1.9 GiB on a batch of 2 x 16 heads of 8192 tokens at
 *                   d = 128); token: per (batch, head) 4 dk dv ceil(T / 16)
 *                   of checkpoints and 4 T (2 dk + 4) per block of state rows
 *                   of sums, 3 dk + 4 for a channel gate; both capped at
 *                   about 8 GiB (larger batches run in groups of heads, one
 *                   after the other); may be NULL when T = 0
 * The gradient outputs must not alias any input or each other.
 * Alignment: q and k on 8 bytes (bf16) or 16 bytes (fp32); state0,
 * grad_state_out, grad_state0, grad_q, grad_k, a channel alpha and its
 * grad_alpha, and the workspace on 16 bytes; grad_out on 16 bytes for the
 * chunked path; the rest on their element size; otherwise GDN_E_ARG.  dk, dv
 * as for gdn_chunk_fwd; other statuses as above.
 */
int gdn_backward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                 int32_t dtype, int32_t gate, int32_t order, float scale,
                 const void* q, const void* k, const void* v,
                 const float* alpha, const float* beta, const float* state0,
                 const float* grad_out, const float* grad_state_out,
                 float* grad_q, float* grad_k, float* grad_v, float* grad_alpha,
                 float* grad_beta, float* grad_state0,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes gdn_backward needs for that shape and gate kind (0 for an
 * invalid or unsupported shape or gate). */
size_t gdn_backward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    int32_t gate);

/* Which algorithm gdn_backward runs for these feature sizes and gate kind
 * (GDN_BWD_TOKEN or GDN_BWD_CHUNKED), or a negative status.  Host only. */
int gdn_backward_path(int64_t dk, int64_t dv, int32_t gate);

/*
 * gdn_seqpar_fwd — increment-and-correct sequence parallelism (How to
 * Implement Sequence Parallelism in DeltaNet, papercache notes, sections
 * "parallel algorithm derivation" and "CP=4").  The chunks of every sequence
 * are split into n_segments contiguous runs computed concurrently: run 0 from
 * the true start state; every later run g the increment state S^D from zero
 * and the scaling matrix M from I (M_[i+1] = M_[i] (Diag(b_C) - W^T Kbar),
 * which is M_[i](I - W^T K) with unit gates).  Start states are chained
 * S_start(g+1) = S^D_end(g) + S_start(g) M_end(g), and the correction
 * S_[i] = S^D_[i] + S_start M_[i] is applied to the outputs, which are
 * linear in the entry state.  n_segments = 1 is a single stream; below 1
 * the call returns GDN_E_SHAPE.  Segments
 * hold ceil(NC / n_segments) chunks (NC = ceil(T / chunk)); the last may be
 * shorter.  When B * H * n_segments (batch, head, segment) groups are too few
 * to fill the device with the MFMA family's whole-head loop (scalar gate),
 * each segment is cut further into k equal runs (k * n_segments segments in
 * all, at least 4 chunks each), as each of n_segments devices would split
 * its own share; the results are the same up to floating-point rounding.
 * Same tensors as gdn_chunk_fwd; a larger workspace.
 */
int gdn_seqpar_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                   int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                   float scale, int32_t n_segments,
                   const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* state0,
                   float* out, float* state_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes needed by gdn_seqpar_fwd with n_segments, or, for
 * n_segments = 1, by either gdn_seqpar_fwd or gdn_chunk_fwd; 0 when the
 * arguments do not validate.  Host only. */
size_t gdn_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk,
                           int64_t dv, int32_t chunk, int32_t dtype,
                           int32_t gate, int32_t n_segments);

/* Host-only argument check; GDN_OK or the status the entry points would
 * return before enqueueing anything. */
int gdn_validate(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                 int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                 int32_t n_segments);

/* Which kernel family the chunked entry points run for these arguments
 * (GDN_PATH_VALU or GDN_PATH_MFMA), or a negative status.  Host only. */
int gdn_chunk_path(int64_t dk, int64_t dv, int32_t chunk, int32_t dtype,
                   int32_t gate);

/* Number of segments gdn_chunk_fwd cuts each sequence into for these
 * arguments (1: a single stream), or a negative status.  Host only. */
int gdn_chunk_segments(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                       int32_t chunk, int32_t dtype, int32_t gate);

/* Number of segments gdn_seqpar_fwd with n_segments runs each sequence in
 * (n_segments, or a multiple of it: see gdn_seqpar_fwd), or a negative
 * status.  Host only. */
int gdn_seqpar_segments(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        int32_t chunk, int32_t dtype, int32_t gate, int32_t n_segments);

/* Static string naming a status code. */
const char* gdn_status_str(int status);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

/*
 * Optional per-kernel timing through a caller-owned timer.  The *_timed entry
 * points below are the entry points of the same name without the suffix,
 * plus a timer: they bracket every kernel they launch with HIP events
 * recorded on the call's stream and add the elapsed times to the timer's
 * record (no work is skipped or reordered; the events cost a few microseconds
 * of GPU time between kernels).  timer may be NULL (no timing).
 *
 * gdn_timer_create makes an empty timer (host memory; its HIP events are
 * created on first use, on the device current then, and destroyed with it).
 * gdn_timer_read(t, i, name, name_len, &ms, &count) waits for the recorded
 * events and returns, for the i-th distinct kernel seen (0-based), its name,
 * total milliseconds and launch count, or GDN_E_ARG past the last kernel.
 * A timer must not be used by two calls at once; distinct timers are
 * independent.  gdn_timer_destroy(NULL) is a no-op.
 */
typedef struct gdn_timer gdn_timer;
int gdn_timer_create(gdn_timer** timer);
int gdn_timer_destroy(gdn_timer* timer);
int gdn_timer_read(gdn_timer* timer, int index, char* name, size_t name_len,
                   double* total_ms, int64_t* count);

int gdn_chunk_fwd_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                        float scale,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const float* state0,
                        float* out, float* state_out,
                        void* workspace, size_t workspace_bytes, void* stream,
                        gdn_timer* timer);
int gdn_chunk_fwd_raw_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                            int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                            float scale,
                            const void* q, const void* k, const void* v,
                            const float* alpha_logit, const float* beta_logit,
                            const float* state0, float* out, float* state_out,
                            void* workspace, size_t workspace_bytes, void* stream,
                            gdn_timer* timer);
int gdn_seqpar_fwd_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                         int32_t chunk, int32_t dtype, int32_t gate, int32_t order,
                         float scale, int32_t n_segments,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const float* state0,
                         float* out, float* state_out,
                         void* workspace, size_t workspace_bytes, void* stream,
                         gdn_timer* timer);
int gdn_decode_step_timed(int64_t B, int64_t H, int64_t dk, int64_t dv,
                          int32_t dtype, int32_t gate, int32_t order, float scale,
                          const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, const float* state_in,
                          float* out, float* state_out, void* stream, gdn_timer* timer);
int gdn_backward_timed(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                       int32_t dtype, int32_t gate, int32_t order, float scale,
                       const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const float* state0,
                       const float* grad_out, const float* grad_state_out,
                       float* grad_q, float* grad_k, float* grad_v, float* grad_alpha,
                       float* grad_beta, float* grad_state0,
                       void* workspace, size_t workspace_bytes, void* stream,
                       gdn_timer* timer);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
