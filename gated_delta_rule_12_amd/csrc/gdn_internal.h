// Internal declarations shared by the HIP translation units of libgdn.
// Nothing here is part of the C ABI (include/gdn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

struct gdn_timer;  // caller-owned per-kernel timer (include/gdn.h)

namespace gdn {

// One forward problem, as the entry points received it (already validated).
struct Problem {
    int64_t B, T, H, dk, dv;
    int C;        // chunk length
    int NC;       // chunks per sequence = ceil(T / C)
    int dtype;    // GDN_F32 / GDN_BF16
    int gate;     // GDN_GATE_SCALAR / GDN_GATE_CHANNEL
    int order;    // GDN_PREDICT_THEN_DECAY / GDN_DECAY_THEN_PREDICT
    int raw;      // 1: q, k raw projections (L2-normalised on the fly, as fp32
                  // row factors) and alpha, beta logits (through a sigmoid)
    float scale;
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* s0;
    float* out;
    float* s_out;
    gdn_timer* timer;  // host object, null: no timing (never read by a kernel)
};

// Sequence-parallel split of the NC chunks of every sequence.
struct Split {
    int G;     // segments actually used (non-empty)
    int per;   // chunks per segment (the last may hold fewer)
};

inline Split make_split(int NC, int n_segments) {
    Split s;
    if (NC <= 0 || n_segments <= 1) { s.G = 1; s.per = NC > 0 ? NC : 1; return s; }
    s.per = (NC + n_segments - 1) / n_segments;
    s.G = (NC + s.per - 1) / s.per;
    return s;
}

// Byte offsets of the pieces of a workspace (all 256-byte aligned).
struct WsLayout {
    size_t prep = 0, prep_bytes = 0;     // per-chunk stage-1 results
    size_t corr = 0, corr_bytes = 0;     // seq-par: per-chunk output corrections R
    size_t sdend = 0, sdend_bytes = 0;   // seq-par: per-segment end states (S^D)
    size_t mend = 0, mend_bytes = 0;     // seq-par: per-segment end scaling matrices
    size_t sstart = 0, sstart_bytes = 0; // seq-par: per-segment true start states
    size_t sfrag = 0, sfrag_bytes = 0;   // seq-par, MFMA family: start states as bf16 hi/lo fragments
    size_t blk = 0, blk_bytes = 0;       // seq-par, whole-head path: composed maps of blocks of segments
    size_t total = 0;
};

// Kernel-family workspace layouts and launchers (each returns a hipError_t).
WsLayout valu_layout(const Problem& p, const Split& sp);
hipError_t valu_forward(const Problem& p, const Split& sp, char* ws, hipStream_t st);

WsLayout mfma_layout(const Problem& p, const Split& sp);
bool mfma_supported(int64_t dk, int64_t dv, int C, int dtype, int gate);
hipError_t mfma_forward(const Problem& p, const Split& sp, char* ws, hipStream_t st);
// Segments the MFMA family runs a forward pass in when the caller leaves the
// schedule to the library (gdn_chunk_fwd): enough (batch, head, segment)
// workgroups to occupy the device, at least kMinSegChunks chunks each; 1 for
// paths without the whole-head chunk loop.
int mfma_auto_segments(const Problem& p);
// Segments the MFMA family runs an explicit request of G in: G, or a multiple
// of it when only a finer cut fills the device with the whole-head loop.
int mfma_refine_segments(const Problem& p, int G);

hipError_t recurrent_forward(const Problem& p, hipStream_t st);
// One-token step on a persistent state (q, k, v, gates of one token; T = 1);
// prologue: q, k L2-normalised and alpha, beta through a sigmoid first.
hipError_t decode_step(const Problem& p, bool prologue, hipStream_t st);

// Sequence-parallel tail shared by both families: chain of start states and
// output correction (R_i S_start^T), then the final state.
hipError_t seqpar_finish(const Problem& p, const Split& sp, char* ws,
                         const WsLayout& L, bool mfma, hipStream_t st);
// Start-state chain alone (final_step: also the state after the last segment).
hipError_t seqpar_chain(const Problem& p, const Split& sp, char* ws, const WsLayout& L,
                        bool write_frag, bool final_step, hipStream_t st);
// MFMA output correction O_i += R_i S_start^T (gdn_mfma.hip).
hipError_t mfma_correct(const Problem& p, const Split& sp, char* ws, const WsLayout& L,
                        hipStream_t st);

// Backward pass (gdn_backward): the forward problem plus the incoming
// gradients, the gradient outputs and the checkpoint workspace.
struct BwdProblem {
    Problem p;
    const float* dout;    // [B, T, H, dv]
    const float* ds_out;  // [B, H, dv, dk] or null (zero)
    float* dq;            // [B, T, H, dk]
    float* dk;            // [B, T, H, dk]
    float* dv;            // [B, T, H, dv]
    float* dalpha;        // shaped as alpha
    float* dbeta;         // [B, T, H]
    float* ds0;           // [B, H, dv, dk] or null
    float* ckpt;          // workspace: states at every 16-token run start
    float* part;          // workspace: per (row block, token) partial sums
    int64_t bh0, nbh;     // the (batch, head) pairs of one launch
};
size_t backward_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate);
size_t backward_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate);
hipError_t backward(const BwdProblem& a, hipStream_t st);
// Chunked backward (gdn_bwd_chunk.hip): scalar gate, dk = dv in {64, 128};
// its own workspace layout, given whole.
bool chunked_backward_supported(int64_t dk, int64_t dv, int gate);
size_t chunked_backward_workspace(int64_t B, int64_t T, int64_t H, int64_t D);
hipError_t backward_chunked(const BwdProblem& a, void* workspace, hipStream_t st);

// Raw projections on the vector-ALU family: the prologue's fp32 outputs in
// the workspace (raw_inputs_bytes of it, at raw_inputs_at), then the forward
// runs on them as fp32 inputs.
struct RawInputs {
    float* q;
    float* k;
    float* v;
    float* alpha;
    float* beta;
};
size_t raw_inputs_bytes(const Problem& p);
RawInputs raw_inputs_at(const Problem& p, char* base);
hipError_t raw_prologue(const Problem& p, const RawInputs& r, hipStream_t st);

// Start state copy/zero for empty sequences (T == 0).
hipError_t copy_state(const Problem& p, hipStream_t st);

// Timing hooks: with a caller's timer, bracket a launch with HIP events on
// the launch stream (nothing otherwise).
void prof_begin(gdn_timer* t, const char* name, hipStream_t st);
void prof_end(gdn_timer* t, hipStream_t st);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace gdn

// Device helpers -----------------------------------------------------------

// The block's gate and beta from logits: sigmoid(x) = 1 / (1 + e^-x) and its
// logarithm log sigmoid(x) = -log(1 + e^-x), formed without overflow for
// either sign of x.
__device__ __forceinline__ float gdn_sigmoid(float x) { return 1.f / (1.f + expf(-x)); }
__device__ __forceinline__ float gdn_log_sigmoid(float x) {
    return x >= 0.f ? -log1pf(expf(-x)) : x - log1pf(expf(x));
}
// 1 / |x| for an L2 length squared, 0 for a zero vector (it stays zero)
__device__ __forceinline__ float gdn_inv_len(float sumsq) { return sumsq > 0.f ? rsqrtf(sumsq) : 0.f; }

__device__ __forceinline__ float gdn_bf16_to_f32(uint16_t x) {
    return __uint_as_float(uint32_t(x) << 16);
}

template <int DT>
__device__ __forceinline__ float gdn_ld(const void* p, int64_t i);

template <>
__device__ __forceinline__ float gdn_ld<0>(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float gdn_ld<1>(const void* p, int64_t i) {
    return gdn_bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Cross-lane sums on the vector ALU (DPP and the lane-swap instructions),
// not through the LDS crossbar: each step pairs lanes symmetrically, so every
// lane of a group ends with the same sum.
template <int CTRL>
__device__ __forceinline__ float gdn_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// x + (x with 16-lane rows 0 <-> 1 and 2 <-> 3 exchanged)
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x + (x with the two 32-lane halves exchanged)
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // within 8 lanes, i <-> 7 - i
constexpr int kDppMirror = 0x140;     // within 16 lanes, i <-> 15 - i
constexpr int kDppRor4 = 0x124;       // within 16 lanes, rotate by 4
constexpr int kDppRor8 = 0x128;       // within 16 lanes, rotate by 8

// sum over the LPR lanes of a row (aligned groups of LPR lanes)
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    if constexpr (LPR >= 2) x += gdn_dpp<kDppXor1>(x);
    if constexpr (LPR >= 4) x += gdn_dpp<kDppXor2>(x);
    if constexpr (LPR >= 8) x += gdn_dpp<kDppHalfMirror>(x);
    if constexpr (LPR >= 16) x += gdn_dpp<kDppMirror>(x);
    if constexpr (LPR >= 32) x = xor16_sum(x);
    return x;
}
// sum over the row groups of a wave (lanes equal modulo LPR)
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (LPR <= 4) x += gdn_dpp<kDppRor4>(x);
    if constexpr (LPR <= 8) x += gdn_dpp<kDppRor8>(x);
    if constexpr (LPR <= 16) x = xor16_sum(x);
    return xor32_sum(x);
}
