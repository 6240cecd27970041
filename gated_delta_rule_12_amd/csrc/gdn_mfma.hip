// MFMA kernels of the chunkwise gated delta rule (gfx950, bf16 inputs,
// dk = dv = D in {64, 128}, chunk C = 64, scalar or per-key-channel gate).
//
// Chunk algebra as in the vector-ALU family (gdn_valu.hip): per chunk with
// chunk-local log-gate prefix g_t (gamma_t = exp g_t), prediction prefix g'_t
// (g_{t-1} predict-then-decay, g_t decay-then-predict), entry state S (dv x dk):
//   T'    = (I + diag(beta) L)^{-1} diag(beta),  L_tj = exp(g'_t - g_j) k_t.k_j (j < t)
//   Delta = T' (V - diag(gamma') K S^T)
//   O     = scale (diag(gamma) Q S^T + P Delta),  P_tj = exp(g_t - g_j) q_t.k_j (j <= t)
//   S'    = gamma_C S + (diag(gamma_C / gamma) Delta)^T K
// (DeltaNet illustrated notes, WY/UT section: UT transform, chunk state
// passing, output; GLA gating section: gate prefixes; the scalar gate of the
// Gated DeltaNet paragraph of the architectures section).
//
// Precision: q, k, v are exact bf16 MFMA operands.  Every operand derived in
// fp32 (S, T', X, Delta, P) is split into bf16 hi + lo and multiplied as
// hi*raw + lo*raw (one raw operand) or hi*hi + hi*lo + lo*hi (two derived
// operands); accumulation is fp32.  Gate factors are applied on the fp32
// side, as ratios exp(g_t - g_j) <= 1.
//
// Stage 1, one workgroup (4 waves) per (batch, head, chunk): gate prefix,
//   Gram K K^T on MFMA, the gated UT system and its inverse in fp32 (16 x 16
//   diagonal blocks, then off-diagonal blocks by block distance), T' written
//   as bf16 hi/lo MFMA A-operand fragments.  k_prep_scalar (scalar gate;
//   the gated scores P are formed in the chunk loop) and k_prep_channel
//   (per-key-channel gate; also the log2-prefix table and P).
// Stage 2, two chunk loops.  Results in MFMA accumulator layout are fed to
//   the next product without transposition: a k-step of 32 pairs two 16-row
//   accumulator tiles, k-slot 8g+e <-> index 4g+e (e < 4) of the first tile
//   and 4g+e-4 of the second, and the other operand is read in the same slot
//   order.
// k_seg (scalar gate, enough (head, segment) workgroups to fill the device):
//   one workgroup per (batch, head, segment) holds the whole state S^T in
//   registers, wave w the value columns 16w..16w+15; sequences cut into
//   segments run as a state pass (increment S^D and scaling matrix M per
//   segment), the start-state chain (k_chain_rows: sequential, or a two-level
//   scan over blocks of segments when they are many) and an output pass from
//   the true entry states.
// k_rec_mfma (channel gate, or too few groups): one workgroup per (batch,
//   head, segment, 16-row slice of the state); wave w owns token rows
//   16w..16w+15 of every chunk product and key rows (D/4 of them) of the
//   state.  Three barriers per chunk.  Segments use increment-and-correct
//   (scaling tiles, k_chain, k_correct_mfma).
#include <type_traits>

#include "gdn_internal.h"
#include "gdn_mfma_common.h"
#include "../../include/gdn.h"

namespace gdn {
namespace {

__device__ __forceinline__ f32x4 mfma(const u16x8& a, const u16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

// x = hi + lo + O(2^-18 |x|): hi = bf16(x), lo = bf16(x - hi), both RNE.
// x - hi is exact in fp32 and is formed by one bf16 dot product per element,
// x + (-1) hi + (-0) hi' (v_dot2c_f32_bf16), instead of a shift and a
// subtraction.  The zero factors are -0: the pair (-1, +0) would be emitted as
// the inline constant -1.0, which the instruction reads as (+0, -1) (checked
// lane by lane on gfx950); (-1, -0) and (-0, -1) are encoded as literals.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(a, b);
    const bf16x2_t h = __builtin_bit_cast(bf16x2_t, hi);
    const bf16x2_t m0 = {(__bf16)-1.f, (__bf16)-0.f}, m1 = {(__bf16)-0.f, (__bf16)-1.f};
    lo = pack_bf16(__builtin_amdgcn_fdot2_f32_bf16(h, m0, a, false), __builtin_amdgcn_fdot2_f32_bf16(h, m1, b, false));
}

__device__ __forceinline__ void split4(const f32x4& x, u16x4& hi, u16x4& lo) {
    uint32_t h0, l0, h1, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    hi = __builtin_bit_cast(u16x4, uint2{h0, h1});
    lo = __builtin_bit_cast(u16x4, uint2{l0, l1});
}

__device__ __forceinline__ u16x8 cat(const u16x4& a, const u16x4& b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// stage 1: T' and the gate block per chunk-head
// ---------------------------------------------------------------------------
// Gate block (floats): [0,64) gamma_t, [64,128) gamma'_t, [128,192)
// gamma_C / gamma_t, [192,256) g_t, [256] gamma_C; for raw projections
// (gdn_chunk_fwd_raw) the row factors of the L2 norm are folded in:
// gamma_t / |q_t|, gamma'_t / |k_t|, (gamma_C / gamma_t) / |k_t|, and
// [272,336) 1 / |q_t|, [336,400) 1 / |k_t| for the scores.
constexpr int kGateFloats = 400;
constexpr int kGateRq = 272, kGateRk = 336;
constexpr int kGatePieces = 272 / 4, kGatePiecesRaw = kGateFloats / 4;  // 16-byte pieces read
// Channel gate: the C x D log2-prefix table, then (raw) 1 / |q_t|, 1 / |k_t|.
template <int D>
constexpr int kChanFloats = C * D + 2 * C;
// T' fragments kept per chunk: (m, s) with s <= m / 2 (T' is lower triangular)
constexpr int kTslots = 6;
constexpr int kTfragPerChunk = kTslots * 2 * 64;  // [slot][hi/lo][lane] of u16x8
__host__ __device__ constexpr int tslot(int m, int s) { return m < 2 ? m : 2 + 2 * (m - 2) + s; }

// The UT inverse T = (I + A)^{-1} (fp32, ut_inverse_lds: AT holds A's
// strictly lower off-diagonal blocks transposed and its diagonal blocks in
// place; T replaces the diagonal blocks and fills the lower triangle) and
// T' = T diag(beta) written as A-operand fragments, for both stage-1 kernels.
// Called by all threads of a four-wave group (it contains barriers; tid is
// the thread's index in the group); nothing is stored unless write is set.
__device__ __forceinline__ void ut_inverse_store(float* AT, const float* bsh, u16x8* dst, int tid, bool write) {
    constexpr int LDA = C + 4;
    ut_inverse_lds(AT, tid);
    // T' = T diag(beta): [slot(m, s)][hi/lo][lane] of 8 bf16; lane (row
    // 16m + lane % 16, group g), slot e -> column 32s + 4g + e (e < 4) or
    // 32s + 16 + 4g + e - 4; entries above the block diagonal are zero (the
    // tile holds A there)
    for (int f = tid; f < kTslots * 64; f += kThreads) {
        const int slot = f >> 6, lane = f & 63;
        const int m = slot < 2 ? slot : 2 + ((slot - 2) >> 1);
        const int s = slot < 2 ? 0 : ((slot - 2) & 1);
        const int t = 16 * m + (lane & 15), gg = lane >> 4;
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            // columns j0 .. j0 + 3 of row t (16-byte pieces of the tile and of beta)
            const int j0 = 32 * s + 16 * hf + 4 * gg;
            const bool up = (j0 >> 4) > m;
            f32x4 v = *reinterpret_cast<const f32x4*>(&AT[t * LDA + j0]) * *reinterpret_cast<const f32x4*>(&bsh[j0]);
            if (up) v = zero4();
            split2(v[0], v[1], hi[2 * hf], lo[2 * hf]);
            split2(v[2], v[3], hi[2 * hf + 1], lo[2 * hf + 1]);
        }
        // (non-temporal: written once here, read by the chunk loops later;
        // measured 5 % off stage 1 and nothing on the readers)
        if (write) {
            __builtin_nontemporal_store(__builtin_bit_cast(u16x8, uint4{hi[0], hi[1], hi[2], hi[3]}), &dst[(slot * 2 + 0) * 64 + lane]);
            __builtin_nontemporal_store(__builtin_bit_cast(u16x8, uint4{lo[0], lo[1], lo[2], lo[3]}), &dst[(slot * 2 + 1) * 64 + lane]);
        }
    }
}

// Stage 1 for per-key-channel gates: the gate is a vector per token and the
// chunk-local prefix becomes a C x D table, kept in log2 units
// (lam[t][a] = sum_{s <= t} log2 alpha_sa, so every ratio is one exp2) and
// stored for the chunk loop.  Intra-chunk ratios 2^{lam_t - lam_j} differ per
// channel, so they enter the MFMA operands as row and key factors about an
// anchor token, per 16-token row block (the secondary chunking of the GLA
// gating section).
template <int D>
__global__ __launch_bounds__(kThreads, 3) void k_prep_channel(Problem p, u16x8* tfrag, u16x8* pfrag,
                                                           float* gates) {
    constexpr int LDA = C + 4;
    constexpr int LDK = D + 8;
    constexpr int PPR = D / 8;
    static_assert(C * LDK * 2 <= C * LDA * 4, "K staging fits the tile");
    // one 64 x 68 fp32 tile holds in turn the prefix scan's partials, the K
    // rows (bf16, row stride LDK) and then A and T as in the scalar kernel
    __shared__ __attribute__((aligned(16))) float AT[C * LDA];
    __shared__ __attribute__((aligned(16))) float bsh[C];
    // channel log2 prefix, rows padded by 16 bytes against bank conflicts
    __shared__ __attribute__((aligned(16))) float gt[C][D + 4];
    unsigned short* Ks = reinterpret_cast<unsigned short*>(AT);

    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int64_t H = p.H, T = p.T;
    const int64_t t0 = (int64_t)i * C;
    const int nt = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t ch = ((int64_t)b * H + h) * p.NC + i;
    const unsigned short* kin = static_cast<const unsigned short*>(p.k);
    const unsigned short* qin = static_cast<const unsigned short*>(p.q);

    // K rows loaded first (rows past the end: zero) and stored once the
    // scan partials in the tile are consumed
    constexpr int KP = C * PPR / kThreads;
    u32x4 kv[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int e = tid + kThreads * k, t = e / PPR, c8 = e % PPR;
        kv[k] = u32x4{0, 0, 0, 0};
        if (t < nt) kv[k] = *reinterpret_cast<const u32x4*>(kin + (((int64_t)b * T + t0 + t) * H + h) * D + c8 * 8);
    }
    if (w == 0) {
        float bt = 0.f;
        if (l < nt) {
            bt = p.beta[((int64_t)b * T + t0 + l) * H + h];
            if (p.raw) bt = gdn_sigmoid(bt);
        }
        bsh[l] = bt;
    }
    // raw projections: 1 / |k_t| and 1 / |q_t| (each row's pieces sit on PPR
    // consecutive lanes); otherwise ones
    __shared__ float rqsh[C], rksh[C];
    if (p.raw) {
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int e = tid + kThreads * k, t = e / PPR, c8 = e % PPR;
            u32x4 qv = u32x4{0, 0, 0, 0};
            if (t < nt) qv = *reinterpret_cast<const u32x4*>(qin + (((int64_t)b * T + t0 + t) * H + h) * D + c8 * 8);
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float x = gdn_bf16_to_f32(__builtin_bit_cast(u16x8, kv[k])[e2]);
                const float y = gdn_bf16_to_f32(__builtin_bit_cast(u16x8, qv)[e2]);
                sk += x * x;
                sq += y * y;
            }
            sk = row_sum<PPR>(sk);
            sq = row_sum<PPR>(sq);
            if (c8 == 0) {
                rksh[t] = gdn_inv_len(sk);
                rqsh[t] = gdn_inv_len(sq);
            }
        }
    } else if (w == 0) {
        rksh[l] = 1.f;
        rqsh[l] = 1.f;
    }
    // log2 prefix lam[t][a] = sum_{s <= t} log2 alpha_sa (padding tokens add
    // zero): thread (group, a4) scans TPG tokens of four channels in
    // registers, then adds the totals of the earlier groups
    constexpr int A4 = D / 4, NG = kThreads / A4, TPG = C / NG;
    static_assert(NG * A4 * 4 <= C * LDA, "scan partials fit the tile");
    f32x4(*part)[A4] = reinterpret_cast<f32x4(*)[A4]>(AT);
    const int a4 = tid % A4, grp = tid / A4;
    f32x4 run = zero4(), vals[TPG];
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
        const int t = grp * TPG + u;
        if (t < nt) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(
                p.alpha + (((int64_t)b * T + t0 + t) * H + h) * D + 4 * a4);
            if (p.raw) {
                constexpr float kLog2e = 1.4426950408889634f;
                run += kLog2e * f32x4{gdn_log_sigmoid(av[0]), gdn_log_sigmoid(av[1]), gdn_log_sigmoid(av[2]),
                                      gdn_log_sigmoid(av[3])};
            } else {
                run += f32x4{__log2f(av[0]), __log2f(av[1]), __log2f(av[2]), __log2f(av[3])};
            }
        }
        vals[u] = run;
    }
    part[grp][a4] = run;
    __syncthreads();
    f32x4 off = zero4();
    for (int gg = 0; gg < grp; ++gg) off += part[gg][a4];
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
        const int t = grp * TPG + u;
        *reinterpret_cast<f32x4*>(&gt[t][4 * a4]) = vals[u] + off;
    }
    __syncthreads();  // partials consumed: the tile takes K
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int e = tid + kThreads * k, t = e / PPR, c8 = e % PPR;
        *reinterpret_cast<u32x4*>(&Ks[t * LDK + c8 * 8]) = kv[k];
    }
    // the prefix table for the chunk loop (after the K rows, whose wait on
    // the vector-memory counter would otherwise include these stores)
    {
        // (the table and the P fragments below go out non-temporally, like
        // T': written once here, read once by the chunk loop; measured
        // 245 -> 243 us here and 407 -> 400 us in the chunk loop on the
        // channel-gate workload)
        float* gdst = gates + ch * (int64_t)kChanFloats<D>;
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
            const int t = grp * TPG + u;
            __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&gt[t][4 * a4]),
                                        reinterpret_cast<f32x4*>(&gdst[t * D + 4 * a4]));
        }
        if (p.raw && w == 0) {
            gdst[C * D + l] = rqsh[l];
            gdst[C * D + C + l] = rksh[l];
        }
    }
    __syncthreads();

    // Scores with per-channel ratios 2^{lam_t - lam_j}, row block m = w,
    // every key block c <= w anchored at p = 16w - 1 (lam_{-1} = 0):
    //   P_tj = sum_a [q_ta 2^{lam_ta - lam_pa}] [k_ja 2^{lam_pa - lam_ja}]   (j <= t)
    //   L_tj = sum_a [k_ta 2^{lam'_ta - lam_pa}] [k_ja 2^{lam_pa - lam_ja}]  (j < t)
    // Row factors are at most one, key factors too off the diagonal block;
    // on it they grow with the decay across the block.  All gated operands
    // are split hi/lo; accumulators are transposed (rows j, columns t).
    const bool ptd = p.order == GDN_PREDICT_THEN_DECAY;
    const int pa = 16 * w - 1, t = 16 * w + c16;
    const int tp = ptd ? t - 1 : t;  // row of lam' (-1: zero)
    const f32x4 z4 = zero4();
    const float rq_t = rqsh[t], rk_t = rksh[t];
    u16x8 qh[D / 32], ql[D / 32], lh[D / 32], ll[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        const int a0 = 32 * s + 8 * g4;
        u16x8 qt = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (t < nt)
            qt = *reinterpret_cast<const u16x8*>(qin + (((int64_t)b * T + t0 + t) * H + h) * D + a0);
        const u16x8 kt_ = *reinterpret_cast<const u16x8*>(&Ks[t * LDK + a0]);
        const f32x4 gp0 = pa >= 0 ? *reinterpret_cast<const f32x4*>(&gt[pa][a0]) : z4;
        const f32x4 gp1 = pa >= 0 ? *reinterpret_cast<const f32x4*>(&gt[pa][a0 + 4]) : z4;
        const f32x4 gt0 = *reinterpret_cast<const f32x4*>(&gt[t][a0]);
        const f32x4 gt1 = *reinterpret_cast<const f32x4*>(&gt[t][a0 + 4]);
        const f32x4 gq0 = tp >= 0 ? *reinterpret_cast<const f32x4*>(&gt[tp][a0]) : z4;
        const f32x4 gq1 = tp >= 0 ? *reinterpret_cast<const f32x4*>(&gt[tp][a0 + 4]) : z4;
        uint32_t h1[4], l1[4], h2[4], l2[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            float xq[2], xl[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ee = e + u;
                const float g_p = ee < 4 ? gp0[ee] : gp1[ee - 4];
                xq[u] = rq_t * gdn_bf16_to_f32(qt[ee]) * __builtin_amdgcn_exp2f((ee < 4 ? gt0[ee] : gt1[ee - 4]) - g_p);
                xl[u] = rk_t * gdn_bf16_to_f32(kt_[ee]) * __builtin_amdgcn_exp2f((ee < 4 ? gq0[ee] : gq1[ee - 4]) - g_p);
            }
            split2(xq[0], xq[1], h1[e >> 1], l1[e >> 1]);
            split2(xl[0], xl[1], h2[e >> 1], l2[e >> 1]);
        }
        qh[s] = __builtin_bit_cast(u16x8, uint4{h1[0], h1[1], h1[2], h1[3]});
        ql[s] = __builtin_bit_cast(u16x8, uint4{l1[0], l1[1], l1[2], l1[3]});
        lh[s] = __builtin_bit_cast(u16x8, uint4{h2[0], h2[1], h2[2], h2[3]});
        ll[s] = __builtin_bit_cast(u16x8, uint4{l2[0], l2[1], l2[2], l2[3]});
    }
    // Past 2^92 (about e^64) of decay across the diagonal block on some
    // channel (gates far below any trained range) that block is summed
    // directly instead.
    float span = 0.f;
    for (int a = l; a < D; a += 64) span = fmaxf(span, (pa >= 0 ? gt[pa][a] : 0.f) - gt[16 * w + 15][a]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
    const bool direct = span > 92.f;

    // P blocks go out as fragment pairs as soon as a pair is complete; the A
    // blocks (rows j, column t) stay in registers until K is dead
    u16x8* pdst = pfrag + ch * kTfragPerChunk;
    f32x4 PT[4], AL[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) PT[c] = AL[c] = zero4();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c > w) continue;
        const int j = 16 * c + c16;
        f32x4 aL = zero4(), aP = zero4();
        if (c == w && direct) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jj = 16 * c + 4 * g4 + r;
                float sp = 0.f, sl = 0.f;
                if (jj <= t && t < nt) {
                    const unsigned short* qrow = qin + (((int64_t)b * T + t0 + t) * H + h) * D;
                    for (int a = 0; a < D; ++a) {
                        const float kj = gdn_bf16_to_f32(Ks[jj * LDK + a]);
                        const float lq = tp >= 0 ? gt[tp][a] : 0.f;
                        sp += gdn_bf16_to_f32(qrow[a]) * kj * __builtin_amdgcn_exp2f(gt[t][a] - gt[jj][a]);
                        sl += gdn_bf16_to_f32(Ks[t * LDK + a]) * kj * __builtin_amdgcn_exp2f(lq - gt[jj][a]);
                    }
                }
                aP[r] = rq_t * rksh[jj] * sp;
                aL[r] = rk_t * rksh[jj] * sl;
            }
        } else {
            f32x4 aP2 = zero4(), aL2 = zero4();
            const float rk_j = rksh[j];
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                const int a0 = 32 * s + 8 * g4;
                const u16x8 kj = *reinterpret_cast<const u16x8*>(&Ks[j * LDK + a0]);
                const f32x4 gp0 = pa >= 0 ? *reinterpret_cast<const f32x4*>(&gt[pa][a0]) : z4;
                const f32x4 gp1 = pa >= 0 ? *reinterpret_cast<const f32x4*>(&gt[pa][a0 + 4]) : z4;
                const f32x4 gj0 = *reinterpret_cast<const f32x4*>(&gt[j][a0]);
                const f32x4 gj1 = *reinterpret_cast<const f32x4*>(&gt[j][a0 + 4]);
                uint32_t ah[4], al[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float xa[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int ee = e + u;
                        xa[u] = rk_j * gdn_bf16_to_f32(kj[ee]) *
                                __builtin_amdgcn_exp2f((ee < 4 ? gp0[ee] : gp1[ee - 4]) - (ee < 4 ? gj0[ee] : gj1[ee - 4]));
                    }
                    split2(xa[0], xa[1], ah[e >> 1], al[e >> 1]);
                }
                const u16x8 Ah = __builtin_bit_cast(u16x8, uint4{ah[0], ah[1], ah[2], ah[3]});
                const u16x8 Al = __builtin_bit_cast(u16x8, uint4{al[0], al[1], al[2], al[3]});
                aP = mfma(Ah, qh[s], aP);
                aP2 = mfma(Ah, ql[s], aP2);
                aP = mfma(Al, qh[s], aP);
                aL = mfma(Ah, lh[s], aL);
                aL2 = mfma(Ah, ll[s], aL2);
                aL = mfma(Al, lh[s], aL);
            }
            aP += aP2;
            aL += aL2;
        }
        // accumulator lane: column t = 16w + c16, rows j = 16c + 4g4 + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jj = 16 * c + 4 * g4 + r;
            AL[c][r] = jj < t ? bsh[t] * aL[r] : 0.f;
            PT[c][r] = jj <= t ? aP[r] : 0.f;
        }
        if ((c & 1) || c == w) {
            const int s = c >> 1;
            u16x4 h0, l0, h1, l1;
            split4(PT[2 * s], h0, l0);
            split4(PT[2 * s + 1], h1, l1);
            __builtin_nontemporal_store(cat(h0, h1), &pdst[(tslot(w, s) * 2 + 0) * 64 + l]);
            __builtin_nontemporal_store(cat(l0, l1), &pdst[(tslot(w, s) * 2 + 1) * 64 + l]);
        }
    }
    __syncthreads();  // K and the prefix table are dead
    // A into the tile: blocks left of the diagonal transposed into the upper
    // triangle (A_tj at (j, t)), the diagonal block in place
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c > w) continue;
        if (c < w) {
#pragma unroll
            for (int r = 0; r < 4; ++r) AT[(16 * c + 4 * g4 + r) * LDA + t] = AL[c][r];
        } else {
            *reinterpret_cast<f32x4*>(&AT[t * LDA + 16 * c + 4 * g4]) = AL[c];
        }
    }
    __syncthreads();

    ut_inverse_store(AT, bsh, tfrag + ch * kTfragPerChunk, threadIdx.x, true);
}

// Scalar gate, stage 1 with a small LDS footprint (18.3 KiB, so eight
// workgroups of four waves share a CU, and the chunk-heads of a head count
// that is a multiple of 512 take whole rounds of the compute units): one
// 64 x 68 fp32 tile first holds the K rows
// (bf16) for the Gram product, then both the UT system A (strictly lower
// blocks stored transposed in the upper triangle, diagonal blocks in place
// until their inverse replaces them) and T = (I + A)^{-1} (lower triangle).
struct PrepScalarShared {
    float AT[C * (C + 4)];
    float gsh[C], gpsh[C], bsh[C];
    float rqsh[C], rksh[C];  // 1 / |q_t|, 1 / |k_t| (raw projections; else ones)
};
// Chunk i of head (b, h) by a four-wave group (tid: the thread's index in
// the group; every barrier is a workgroup barrier, which a second group of
// the workgroup passes with its own chunk); stores nothing unless write is set.
template <int D>
__device__ __forceinline__ void prep_scalar_chunk(const Problem& p, u16x8* tfrag, float* gates, int i, int h, int b,
                                                  PrepScalarShared& ps, int tid, bool write) {
    constexpr int LDA = C + 4;
    float* const AT = ps.AT;
    float* const gsh = ps.gsh;
    float* const gpsh = ps.gpsh;
    float* const bsh = ps.bsh;
    float* const rqsh = ps.rqsh;
    float* const rksh = ps.rksh;
    const int w = tid >> 6, l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int64_t H = p.H, T = p.T;
    const int64_t t0 = (int64_t)i * C;
    const int nt = (int)((T - t0) < C ? (T - t0) : C);
    const int64_t ch = ((int64_t)b * H + h) * p.NC + i;
    const unsigned short* kin = static_cast<const unsigned short*>(p.k);

    // K rows staged (coalesced) in the tile's own LDS, bf16 at row stride D + 8
    // (17408 bytes, the size of the fp32 tile for D = 128); rows past the
    // sequence end are zero
    constexpr int LDK = D + 8, PPR = D / 8;
    static_assert(C * LDK * 2 <= C * LDA * 4, "K staging fits the tile");
    unsigned short* Ks = reinterpret_cast<unsigned short*>(AT);
    // K rows first (every wave), then the gate prefix on wave 0, then the rows
    // go to LDS: the two global fetches overlap
    constexpr int KP = C * PPR / kThreads;
    u32x4 kv[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int e = tid + kThreads * k, t = min(e / PPR, nt - 1), c8 = e % PPR;
        kv[k] = *reinterpret_cast<const u32x4*>(kin + (((int64_t)b * T + t0 + t) * H + h) * D + c8 * 8);
    }
    // gate prefix (wave 0)
    if (w == 0) {
        float la = 0.f, bt = 0.f;
        if (l < nt) {
            const int64_t row = ((int64_t)b * T + t0 + l) * H + h;
            if (p.raw) {
                la = gdn_log_sigmoid(p.alpha[row]);
                bt = gdn_sigmoid(p.beta[row]);
            } else {
                la = __logf(p.alpha[row]);
                bt = p.beta[row];
            }
        }
        const float gv = wave_incl_scan(la, l);
        float gprev = __shfl_up(gv, 1, 64);
        if (l == 0) gprev = 0.f;
        const float gpv = p.order == GDN_PREDICT_THEN_DECAY ? gprev : gv;
        gsh[l] = gv;
        gpsh[l] = gpv;
        bsh[l] = bt;
    }
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int e = tid + kThreads * k, t = e / PPR, c8 = e % PPR;
        *reinterpret_cast<u32x4*>(&Ks[t * LDK + c8 * 8]) = t < nt ? kv[k] : u32x4{0, 0, 0, 0};
    }
    // raw projections: 1 / |k_t| and 1 / |q_t| (each row's pieces sit on PPR
    // consecutive lanes; padding rows are zero); otherwise ones
    if (p.raw) {
        const unsigned short* qin = static_cast<const unsigned short*>(p.q);
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int e = tid + kThreads * k, t = min(e / PPR, nt - 1), c8 = e % PPR;
            const u32x4 qv = *reinterpret_cast<const u32x4*>(qin + (((int64_t)b * T + t0 + t) * H + h) * D + c8 * 8);
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float x = gdn_bf16_to_f32(__builtin_bit_cast(u16x8, kv[k])[e2]);
                const float y = gdn_bf16_to_f32(__builtin_bit_cast(u16x8, qv)[e2]);
                sk += x * x;
                sq += y * y;
            }
            sk = row_sum<PPR>(sk);
            sq = row_sum<PPR>(sq);
            if (c8 == 0) {
                const bool real = e / PPR < nt;
                rksh[e / PPR] = real ? gdn_inv_len(sk) : 0.f;
                rqsh[e / PPR] = real ? gdn_inv_len(sq) : 0.f;
            }
        }
    } else if (w == 0) {
        rksh[l] = 1.f;
        rqsh[l] = 1.f;
    }
    __syncthreads();  // K rows, the gate prefix and the row factors visible
    // the gate block for the chunk loop (after the K rows, whose wait on the
    // vector-memory counter would otherwise include these stores)
    if (w == 0 && write) {
        const float gv = gsh[l], gpv = gpsh[l], gC = gsh[C - 1];
        const float rq = rqsh[l], rk = rksh[l];
        float* gb = gates + ch * kGateFloats;
        gb[l] = rq * __expf(gv);
        gb[64 + l] = rk * __expf(gpv);
        gb[128 + l] = rk * __expf(gC - gv);
        gb[192 + l] = gv;
        if (l == 0) gb[256] = __expf(gC);
        if (p.raw) {
            gb[kGateRq + l] = rq;
            gb[kGateRk + l] = rk;
        }
    }
    auto krow = [&](int m, int s) { return *reinterpret_cast<const u16x8*>(&Ks[(16 * m + c16) * LDK + 32 * s + 8 * g4]); };
    // Gram blocks (m, nb), nb <= m, dealt 3, 3, 2, 2 over the waves
    f32x4 acc[3];
    int bm[3], bn[3], nbk;
    if (w == 0) { bm[0] = 0; bn[0] = 0; bm[1] = 3; bn[1] = 0; bm[2] = 3; bn[2] = 1; nbk = 3; }
    else if (w == 1) { bm[0] = 1; bn[0] = 0; bm[1] = 1; bn[1] = 1; bm[2] = 3; bn[2] = 2; nbk = 3; }
    else if (w == 2) { bm[0] = 2; bn[0] = 0; bm[1] = 2; bn[1] = 1; bm[2] = 0; bn[2] = 0; nbk = 2; }
    else { bm[0] = 2; bn[0] = 2; bm[1] = 3; bn[1] = 3; bm[2] = 0; bn[2] = 0; nbk = 2; }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        acc[q] = zero4();
        if (q >= nbk) continue;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) acc[q] = mfma(krow(bm[q], s), krow(bn[q], s), acc[q]);
    }
    __syncthreads();  // K is dead: the tile now takes A
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        if (q >= nbk) continue;
        const int m = bm[q], nb = bn[q];
        const int j = 16 * nb + c16;
        const int t0 = 16 * m + 4 * g4;
        const f32x4 bt = *reinterpret_cast<const f32x4*>(&bsh[t0]);
        const f32x4 rkt = *reinterpret_cast<const f32x4*>(&rksh[t0]);
        const f32x4 gpt = *reinterpret_cast<const f32x4*>(&gpsh[t0]);
        const float gj = gsh[j], rkj = rksh[j];
        f32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + r;
            a[r] = j < t ? bt[r] * rkt[r] * rkj * __expf(gpt[r] - gj) * acc[q][r] : 0.f;
        }
        if (nb < m) {
            // A_tj stored at (j, t): upper triangle
            *reinterpret_cast<f32x4*>(&AT[j * LDA + 16 * m + 4 * g4]) = a;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) AT[(16 * m + 4 * g4 + r) * LDA + j] = a[r];
        }
    }
    __syncthreads();

    ut_inverse_store(AT, bsh, tfrag + ch * kTfragPerChunk, tid, write);
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_prep_scalar(Problem p, u16x8* tfrag, float* gates) {
    __shared__ __attribute__((aligned(16))) PrepScalarShared ps;
    prep_scalar_chunk<D>(p, tfrag, gates, blockIdx.x, blockIdx.y, blockIdx.z, ps, threadIdx.x, true);
}

// ---------------------------------------------------------------------------
// stage 2: the chunk loop
// ---------------------------------------------------------------------------
// Eight waves, two per SIMD, in two roles on the same token tile m = w % 4:
//   chain waves (0-3) carry the sequential path Y -> X -> Delta -> S and own
//     key rows of the state slice S^T (fp32 registers);
//   output waves (4-7) compute Z = Q S^T, the gated scores P, P Delta, write
//     the outputs, and stage the next chunks' inputs from HBM into LDS.
// Per chunk i, three barriers:
//   A: chain: Y = K S^T, X = V - diag(gamma') Y -> LDS;  output: Z = Q S^T
//   B: chain: Delta = T' X -> LDS (also Delta scaled to the chunk end);
//      gathers K^T operands.  output: store chunk i+1 inputs to the other
//      LDS buffer, start loading chunk i+2
//   C: chain: S^T <- gamma_C S^T + K^T Delta-bar, publish S^T
//      output: O = scale (diag(gamma) Z + P Delta) -> HBM
// The gated scores P of a chunk do not depend on the state; they arrive as
// A-operand fragments from the preparation kernel, like T'.
template <int D, int CH>
struct RecShared {
    static constexpr int LDK = D + 8;
    static constexpr int KS = D / 32;
    unsigned short K[2][C * LDK];
    unsigned short Q[2][C * LDK];
    unsigned short V[2][C * 16];
    // gate block, or the C x D log2-prefix table (rows padded to D + 4 floats)
    float G[2][CH ? C * (D + 4) : kGateFloats];
    float RQK[2][CH ? 2 * C : 1];  // channel gate, raw projections: 1 / |q_t|, 1 / |k_t|
    u16x4 Sf[KS][2][2][64];  // S^T fragments: [k-step][tile half][hi/lo][lane]
    u16x4 Xf[2][2][2][64];
    u16x4 Df[2][2][2][64];
    u16x4 DBf[2][2][2][64];
};
template <int D>
struct RecSharedP : RecShared<D, 0> {
    u16x8 Pf[4][2][2][64];  // P fragments of the chunk, per token tile
};

constexpr int kRecThreads = 512;
// CH = 1 (per-key-channel gates, log2 prefix lam): Y and Z take the gated
// operands K (.) 2^{lam'} and Q (.) 2^{lam}, the state update takes
// K (.) 2^{lam_C - lam} (all split hi/lo, three MFMAs per product) and the
// state decays column-wise by 2^{lam_C}; no row factors remain.
template <int D, int CH>
__global__ __launch_bounds__(kRecThreads) void k_rec_mfma(Problem p, Split sp, WsLayout L,
                                                          char* wsb, const u16x8* tfrag,
                                                          const u16x8* pfrag,
                                                          const float* gates, int ntiles,
                                                          int xcd_remap) {
    constexpr int LDK = D + 8;
    constexpr int KS = D / 32;   // k-steps over the key dimension
    constexpr int TPW = D / 64;  // 16-row key tiles of S^T owned per chain wave
    constexpr int PPR = D / 8;   // 16-byte pieces per K/Q row
    constexpr int KQP = C * PPR / kThreads;
    constexpr int GP = CH ? C * D / 4 : kGateFloats / 4;  // 16-byte pieces of gate data
    constexpr int GPT = (GP + 255) / 256;                  // pieces per output thread
    // scalar gate: the pieces actually read (the row factors only for raw projections)
    const int gp_n = CH ? GP : (p.raw ? kGatePiecesRaw : kGatePieces);
    // (the scalar gate also hands P fragments over through LDS)
    __shared__ __attribute__((aligned(16))) std::conditional_t<CH, RecShared<D, CH>, RecSharedP<D>> sh;
    const bool ptd = p.order == GDN_PREDICT_THEN_DECAY;

    // work decode; with xcd_remap the ntiles slices of one (head, segment)
    // land on one XCD (workgroups are dealt to the 8 XCDs round-robin)
    int id = blockIdx.x;
    if (xcd_remap) {
        const int xcd = id & 7, slot = id >> 3;
        id = ((slot / ntiles) * 8 + xcd) * ntiles + slot % ntiles;
    }
    const int x = id % ntiles;
    const int hg = id / ntiles;  // (b * H + h) * G + seg
    const int gseg = hg % sp.G;
    const int64_t bh = hg / sp.G;
    const int64_t H = p.H, T = p.T;
    const int b = (int)(bh / H), h = (int)(bh - (bh / H) * H);

    const int w8 = threadIdx.x >> 6;
    const bool chain = w8 < 4;
    const int w = w8 & 3;  // token tile
    const int l = threadIdx.x & 63, g4 = l >> 4, c16 = l & 15;
    const int otid = threadIdx.x - 256;  // thread index within the output group
    const int nvt = D / 16;
    const bool scaling = x >= nvt;
    if (scaling && gseg == 0) return;
    const int r0 = (scaling ? x - nvt : x) * 16;
    const int i_begin = gseg * sp.per;
    const int i_end = min(p.NC, (gseg + 1) * sp.per);
    const unsigned short* kin = static_cast<const unsigned short*>(p.k);
    const unsigned short* qin = static_cast<const unsigned short*>(p.q);
    const unsigned short* vin = static_cast<const unsigned short*>(p.v);
    const int nks = (w >> 1) + 1;  // k-steps over tokens for rows of tile w
    const int64_t row_stride = H * D;
    const int64_t chunk_stride = (int64_t)C * row_stride;

    // ---- chain-wave state: S^T slice, a-tile tau = w*TPW + u, lane (v = c16, a = 16 tau + 4 g4 + r)
    f32x4 Sacc[TPW];
    u16x8 tf_n[2][2], tf_c[2][2];
    const u16x8* tf_base = tfrag + bh * p.NC * kTfragPerChunk + l;
    auto load_tfrag = [&](int i) {
        const u16x8* tp = tf_base + (int64_t)i * kTfragPerChunk;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
                tf_n[s][hl] = s < nks ? tp[(tslot(w, s) * 2 + hl) * 64] : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    };
    auto publish_state = [&]() {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tau = w * TPW + u;
            u16x4 hi, lo;
            split4(Sacc[u], hi, lo);
            sh.Sf[tau >> 1][tau & 1][0][l] = hi;
            sh.Sf[tau >> 1][tau & 1][1][l] = lo;
        }
    };

    // ---- output-wave state
    constexpr int RPP = 256 / PPR;  // token rows per load pass of the output group
    const int trow = otid / PPR, c8 = otid % PPR;
    const int64_t kq_base = (((int64_t)b * T + trow) * H + h) * D + c8 * 8;
    const int vrow = otid >> 1, vhf = otid & 1;
    const int64_t v_base = (((int64_t)b * T + vrow) * H + h) * D + r0 + 8 * vhf;
    constexpr int GSTRIDE = CH ? kChanFloats<D> : kGateFloats;  // gate floats per chunk-head
    constexpr int LDG = D + 4;                           // LDS row stride of the channel table
    static_assert(!CH || (GP % 256 == 0 && 256 % (D / 4) == 0), "channel table staging");
    const float* g_base = gates + bh * p.NC * GSTRIDE;
    uint4 kreg[KQP], qreg[KQP], vreg;
    u32x4 greg[GPT], rqk;
    auto issue_loads = [&](int i) {
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
        const int64_t cofs = (int64_t)i * chunk_stride;
#pragma unroll
        for (int k = 0; k < KQP; ++k) {
            const bool ok = trow + RPP * k < nt;
            const int64_t off = kq_base + cofs + (int64_t)(RPP * k) * row_stride;
            kreg[k] = ok ? *reinterpret_cast<const uint4*>(kin + off) : make_uint4(0, 0, 0, 0);
            qreg[k] = ok ? *reinterpret_cast<const uint4*>(qin + off) : make_uint4(0, 0, 0, 0);
        }
        vreg = make_uint4(0, 0, 0, 0);
        if (!scaling && otid < 128 && vrow < nt)
            vreg = *reinterpret_cast<const uint4*>(vin + v_base + cofs);
        const u32x4* gsrc = reinterpret_cast<const u32x4*>(g_base + (int64_t)i * GSTRIDE) + otid;
#pragma unroll
        for (int k = 0; k < GPT; ++k)
            if (otid + 256 * k < gp_n) greg[k] = gsrc[256 * k];
        if (CH && p.raw && otid < 2 * C / 4) rqk = gsrc[C * D / 4];
    };
    auto store_loads = [&](int buf) {
#pragma unroll
        for (int k = 0; k < KQP; ++k) {
            *reinterpret_cast<uint4*>(&sh.K[buf][(trow + RPP * k) * LDK + c8 * 8]) = kreg[k];
            *reinterpret_cast<uint4*>(&sh.Q[buf][(trow + RPP * k) * LDK + c8 * 8]) = qreg[k];
        }
        if (otid < 128) *reinterpret_cast<uint4*>(&sh.V[buf][vrow * 16 + 8 * vhf]) = vreg;
        if constexpr (CH) {
            // piece q = otid + 256k holds row q / (D/4), columns 4 (q % (D/4)) ..
            float* gdst = sh.G[buf] + (otid / (D / 4)) * LDG + 4 * (otid % (D / 4));
#pragma unroll
            for (int k = 0; k < GPT; ++k)
                *reinterpret_cast<u32x4*>(gdst + k * (256 / (D / 4)) * LDG) = greg[k];
            if (p.raw && otid < 2 * C / 4) reinterpret_cast<u32x4*>(sh.RQK[buf])[otid] = rqk;
        } else {
            u32x4* gdst = reinterpret_cast<u32x4*>(sh.G[buf]) + otid;
#pragma unroll
            for (int k = 0; k < GPT; ++k)
                if (otid + 256 * k < gp_n) gdst[256 * k] = greg[k];
        }
    };
    float* corr = reinterpret_cast<float*>(wsb + L.corr);
    const int64_t out_base = (((int64_t)b * T + 16 * w + 4 * g4) * H + h) * D + r0 + c16;
    float* corr_base = corr + bh * p.NC * C * D + (int64_t)(16 * w + 4 * g4) * D + r0 + c16;
    const u16x8* pf_base = CH ? pfrag + bh * p.NC * kTfragPerChunk + l : nullptr;
    u16x8 pf[2][2];
    auto load_pfrag = [&](int i) {
        const u16x8* pp = pf_base + (int64_t)i * kTfragPerChunk;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
                pf[s][hl] = s < nks ? pp[(tslot(w, s) * 2 + hl) * 64] : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    };
    // scalar gate: the gated causal scores P_tj = exp(g_t - g_j) q_t.k_j (j <= t)
    // of token tile w from the staged K and Q rows, computed transposed (rows
    // j, columns t) so that blocks 2s and 2s + 1 form the A fragment of
    // k-step s as they stand (hi/lo split); formed by the chain wave of the
    // tile while the output waves stage inputs, handed over through LDS
    auto scores = [&](int buf) {
        // block (m, c), c <= m: rows j of tile c, columns t of tile m; the ten
        // blocks are dealt 3, 3, 2, 2 over the four chain waves
        auto pblock = [&](int m, int c) {
            const float* G = sh.G[buf];
            const int t = 16 * m + c16;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u16x8 ka = *reinterpret_cast<const u16x8*>(&sh.K[buf][(16 * c + c16) * LDK + 32 * s + 8 * g4]);
                const u16x8 qb = *reinterpret_cast<const u16x8*>(&sh.Q[buf][t * LDK + 32 * s + 8 * g4]);
                acc = mfma(ka, qb, acc);
            }
            const float gt = G[192 + t];
            const f32x4 gj = *reinterpret_cast<const f32x4*>(&G[192 + 16 * c + 4 * g4]);
            f32x4 pt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * c + 4 * g4 + r;
                pt[r] = j <= t ? acc[r] * __expf(gt - gj[r]) : 0.f;
            }
            if (p.raw) {
                const float rq = G[kGateRq + t];
                const f32x4 rk = *reinterpret_cast<const f32x4*>(&G[kGateRk + 16 * c + 4 * g4]);
                pt = rq * (pt * rk);
            }
            u16x4 hi, lo;
            split4(pt, hi, lo);
            if constexpr (!CH) {
                reinterpret_cast<u16x4*>(&sh.Pf[m][c >> 1][0][l])[c & 1] = hi;
                reinterpret_cast<u16x4*>(&sh.Pf[m][c >> 1][1][l])[c & 1] = lo;
            }
        };
        if (w == 0) { pblock(0, 0); pblock(3, 0); pblock(3, 1); }
        else if (w == 1) { pblock(1, 0); pblock(1, 1); pblock(3, 2); }
        else if (w == 2) { pblock(2, 0); pblock(2, 1); }
        else { pblock(2, 2); pblock(3, 3); }
    };
    auto emit_output = [&](int i, const f32x4& Zc, const f32x4& gam) {
        f32x4 O1 = zero4(), O2 = zero4(), O3 = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (s >= nks) continue;
            u16x8 pah, pal;
            if constexpr (CH) {
                pah = pf[s][0];
                pal = pf[s][1];
            } else {
                pah = sh.Pf[w][s][0][l];
                pal = sh.Pf[w][s][1][l];
            }
            const u16x8 dh = cat(sh.Df[s][0][0][l], sh.Df[s][1][0][l]);
            const u16x8 dlo = cat(sh.Df[s][0][1][l], sh.Df[s][1][1][l]);
            O1 = mfma(pah, dh, O1);
            O2 = mfma(pah, dlo, O2);
            O3 = mfma(pal, dh, O3);
        }
        if (scaling) {
            float* dst = corr_base + (int64_t)i * C * D;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[r * D] = p.scale * (gam[r] * Zc[r] + O1[r] + O2[r] + O3[r]);
        } else {
            const int64_t t0 = (int64_t)i * C;
            const int nt = (int)((T - t0) < C ? (T - t0) : C);
            float* dst = p.out + out_base + t0 * row_stride;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * w + 4 * g4 + r < nt)
                    dst[r * row_stride] = p.scale * (gam[r] * Zc[r] + O1[r] + O2[r] + O3[r]);
        }
    };

    // channel gate: rows of src scaled by 2^{lam[grow]} (grow = -1: by one),
    // split hi/lo, times S^T (hi/lo): 16 x 16 tile of rows 16w.. of the chunk
    auto gated_rows = [&](const unsigned short* src, const float* G, int grow, float rowf) {
        f32x4 A1 = zero4(), A2 = zero4(), A3 = zero4();
        const int t = 16 * w + c16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u16x8 shi = cat(sh.Sf[s][0][0][l], sh.Sf[s][1][0][l]);
            const u16x8 slo = cat(sh.Sf[s][0][1][l], sh.Sf[s][1][1][l]);
            const unsigned short* rr = &src[t * LDK + 32 * s + 4 * g4];
            const u16x8 raw = cat(*reinterpret_cast<const u16x4*>(rr), *reinterpret_cast<const u16x4*>(rr + 16));
            f32x4 g0 = zero4(), g1 = zero4();
            if (grow >= 0) {
                g0 = *reinterpret_cast<const f32x4*>(&G[grow * LDG + 32 * s + 4 * g4]);
                g1 = *reinterpret_cast<const f32x4*>(&G[grow * LDG + 32 * s + 16 + 4 * g4]);
            }
            uint32_t ah[4], al[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float x0 = rowf * gdn_bf16_to_f32(raw[e]) * __builtin_amdgcn_exp2f(e < 4 ? g0[e] : g1[e - 4]);
                const float x1 = rowf * gdn_bf16_to_f32(raw[e + 1]) * __builtin_amdgcn_exp2f(e < 4 ? g0[e + 1] : g1[e - 3]);
                split2(x0, x1, ah[e >> 1], al[e >> 1]);
            }
            const u16x8 Ah = __builtin_bit_cast(u16x8, uint4{ah[0], ah[1], ah[2], ah[3]});
            const u16x8 Al = __builtin_bit_cast(u16x8, uint4{al[0], al[1], al[2], al[3]});
            A1 = mfma(Ah, shi, A1);
            A2 = mfma(Ah, slo, A2);
            A3 = mfma(Al, shi, A3);
        }
        return A1 + A2 + A3;
    };

    // The two roles run separate loops with the same barrier sequence (three
    // per chunk), so neither role's loop-carried registers stay live in the
    // other's code.
    if (chain) {
        // ---- chain prologue
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int a = 16 * (w * TPW + u) + 4 * g4 + r, v = r0 + c16;
                float sv;
                if (scaling) sv = v == a ? 1.f : 0.f;
                else if (gseg == 0 && p.s0) sv = p.s0[(bh * D + v) * D + a];
                else sv = 0.f;
                Sacc[u][r] = sv;
            }
        }
        if constexpr (!CH) {
            // the never-written halves of the P fragments: blocks (0, 1), (2, 3)
            if (w == 0) {
                const u16x4 z = u16x4{0, 0, 0, 0};
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) {
                    reinterpret_cast<u16x4*>(&sh.Pf[0][0][hl][l])[1] = z;
                    reinterpret_cast<u16x4*>(&sh.Pf[2][1][hl][l])[1] = z;
                }
            }
        }
        publish_state();
        if (i_begin < i_end) {
            load_tfrag(i_begin);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) tf_c[s][hl] = tf_n[s][hl];
            if (i_begin + 1 < i_end) load_tfrag(i_begin + 1);
        }

        for (int i = i_begin; i < i_end; ++i) {
            const int cur = (i - i_begin) & 1;
            const float* G = sh.G[cur];
            __syncthreads();  // B1: state fragments and chunk i inputs visible

            // ---- phase A: Y = K S^T (channel gate: gated rows), X = V - gamma' Y
            f32x4 Xc;
            if constexpr (!CH) {
                f32x4 A1 = zero4(), A2 = zero4();
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const u16x8 shi = cat(sh.Sf[s][0][0][l], sh.Sf[s][1][0][l]);
                    const u16x8 slo = cat(sh.Sf[s][0][1][l], sh.Sf[s][1][1][l]);
                    const unsigned short* rr = &sh.K[cur][(16 * w + c16) * LDK + 32 * s + 4 * g4];
                    const u16x8 ra = cat(*reinterpret_cast<const u16x4*>(rr), *reinterpret_cast<const u16x4*>(rr + 16));
                    A1 = mfma(ra, shi, A1);
                    A2 = mfma(ra, slo, A2);
                }
                Xc = A1 + A2;
            } else {
                Xc = gated_rows(sh.K[cur], G, ptd ? 16 * w + c16 - 1 : 16 * w + c16,
                                p.raw ? sh.RQK[cur][C + 16 * w + c16] : 1.f);
            }
            {
                f32x4 gamp = f32x4{1.f, 1.f, 1.f, 1.f};
                if constexpr (!CH) gamp = *reinterpret_cast<const f32x4*>(&G[64 + 16 * w + 4 * g4]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vv = scaling ? 0.f : gdn_bf16_to_f32(sh.V[cur][(16 * w + 4 * g4 + r) * 16 + c16]);
                    Xc[r] = vv - gamp[r] * Xc[r];
                }
                u16x4 hi, lo;
                split4(Xc, hi, lo);
                sh.Xf[w >> 1][w & 1][0][l] = hi;
                sh.Xf[w >> 1][w & 1][1][l] = lo;
            }
            __syncthreads();  // B2

            // ---- phase B: Delta = T' X; K^T operands of the state update
            u16x8 kt[TPW][2], ktl[CH ? TPW : 1][2];
            {
                f32x4 D1 = zero4(), D2 = zero4(), D3 = zero4();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s >= nks) continue;
                    const u16x8 xh = cat(sh.Xf[s][0][0][l], sh.Xf[s][1][0][l]);
                    const u16x8 xl = cat(sh.Xf[s][0][1][l], sh.Xf[s][1][1][l]);
                    D1 = mfma(tf_c[s][0], xh, D1);
                    D2 = mfma(tf_c[s][0], xl, D2);
                    D3 = mfma(tf_c[s][1], xh, D3);
                }
                D1 += D2 + D3;
                u16x4 hi, lo;
                split4(D1, hi, lo);
                sh.Df[w >> 1][w & 1][0][l] = hi;
                sh.Df[w >> 1][w & 1][1][l] = lo;
                if constexpr (!CH) {
                    // Delta scaled to the chunk end (gamma_C / gamma_t per row)
                    const f32x4 rat = *reinterpret_cast<const f32x4*>(&G[128 + 16 * w + 4 * g4]);
                    split4(rat * D1, hi, lo);
                }
                sh.DBf[w >> 1][w & 1][0][l] = hi;
                sh.DBf[w >> 1][w & 1][1][l] = lo;
            }
            // K^T: rows a = 16 tau + c16, k-slots j (channel gate: K (.) 2^{lam_C - lam},
            // split hi/lo)
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int a = 16 * (w * TPW + u) + c16;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if constexpr (!CH) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 32 * s + (e < 4 ? 4 * g4 + e : 16 + 4 * g4 + e - 4);
                            kt[u][s][e] = sh.K[cur][j * LDK + a];
                        }
                    } else {
                        const float gC = G[(C - 1) * LDG + a];
                        uint32_t kh[4], kl[4];
#pragma unroll
                        for (int e = 0; e < 8; e += 2) {
                            const int j0 = 32 * s + (e < 4 ? 4 * g4 + e : 16 + 4 * g4 + e - 4);
                            const float f0 = p.raw ? sh.RQK[cur][C + j0] : 1.f;
                            const float f1 = p.raw ? sh.RQK[cur][C + j0 + 1] : 1.f;
                            const float x0 = f0 * gdn_bf16_to_f32(sh.K[cur][j0 * LDK + a]) * __builtin_amdgcn_exp2f(gC - G[j0 * LDG + a]);
                            const float x1 = f1 * gdn_bf16_to_f32(sh.K[cur][(j0 + 1) * LDK + a]) *
                                             __builtin_amdgcn_exp2f(gC - G[(j0 + 1) * LDG + a]);
                            split2(x0, x1, kh[e >> 1], kl[e >> 1]);
                        }
                        kt[u][s] = __builtin_bit_cast(u16x8, uint4{kh[0], kh[1], kh[2], kh[3]});
                        ktl[u][s] = __builtin_bit_cast(u16x8, uint4{kl[0], kl[1], kl[2], kl[3]});
                    }
                }
            }
            if constexpr (!CH) scores(cur);
            __syncthreads();  // B3

            // ---- phase C: S^T <- decay (.) S^T + K^T Delta-bar, publish
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                f32x4 acc, acc2 = zero4(), acc3 = zero4();
                if constexpr (!CH) {
                    acc = G[256] * Sacc[u];
                } else {
                    // column decay 2^{lam_C[a]} for key rows a = 16 tau + 4 g4 + r
                    const f32x4 gC = *reinterpret_cast<const f32x4*>(&G[(C - 1) * LDG + 16 * (w * TPW + u) + 4 * g4]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] = __builtin_amdgcn_exp2f(gC[r]) * Sacc[u][r];
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const u16x8 dbh = cat(sh.DBf[s][0][0][l], sh.DBf[s][1][0][l]);
                    const u16x8 dbl = cat(sh.DBf[s][0][1][l], sh.DBf[s][1][1][l]);
                    acc = mfma(kt[u][s], dbh, acc);
                    acc2 = mfma(kt[u][s], dbl, acc2);
                    if constexpr (CH) acc3 = mfma(ktl[u][s], dbh, acc3);
                }
                Sacc[u] = acc + acc2 + acc3;
            }
            publish_state();
            if (i + 1 < i_end) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl) tf_c[s][hl] = tf_n[s][hl];
                if (i + 2 < i_end) load_tfrag(i + 2);
            }
        }

        // ---- chain epilogue: the slice of the end state (or of M, or S^Delta)
        float* dst;
        if (scaling)
            dst = reinterpret_cast<float*>(wsb + L.mend) + (bh * sp.G + gseg) * D * D;
        else if (sp.G == 1)
            dst = p.s_out ? p.s_out + bh * D * D : nullptr;
        else
            dst = reinterpret_cast<float*>(wsb + L.sdend) + (bh * sp.G + gseg) * D * D;
        if (dst) {
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int a0 = 16 * (w * TPW + u) + 4 * g4;
                *reinterpret_cast<f32x4*>(&dst[(int64_t)(r0 + c16) * D + a0]) = Sacc[u];
            }
        }
    } else {
        // ---- output prologue
        if (i_begin < i_end) {
            issue_loads(i_begin);
            store_loads(0);
            if (i_begin + 1 < i_end) issue_loads(i_begin + 1);
        }
        for (int i = i_begin; i < i_end; ++i) {
            const int cur = (i - i_begin) & 1;
            const float* G = sh.G[cur];
            __syncthreads();  // B1

            // ---- phase A: Z = Q S^T (channel gate: rows Q (.) 2^{lam})
            f32x4 Zc;
            if constexpr (!CH) {
                f32x4 A1 = zero4(), A2 = zero4();
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const u16x8 shi = cat(sh.Sf[s][0][0][l], sh.Sf[s][1][0][l]);
                    const u16x8 slo = cat(sh.Sf[s][0][1][l], sh.Sf[s][1][1][l]);
                    const unsigned short* rr = &sh.Q[cur][(16 * w + c16) * LDK + 32 * s + 4 * g4];
                    const u16x8 ra = cat(*reinterpret_cast<const u16x4*>(rr), *reinterpret_cast<const u16x4*>(rr + 16));
                    A1 = mfma(ra, shi, A1);
                    A2 = mfma(ra, slo, A2);
                }
                Zc = A1 + A2;
            } else {
                Zc = gated_rows(sh.Q[cur], G, 16 * w + c16, p.raw ? sh.RQK[cur][16 * w + c16] : 1.f);
            }
            if constexpr (CH) load_pfrag(i);
            __syncthreads();  // B2

            // ---- phase B: the other LDS buffer held chunk i-1, finished before
            // B1: stage chunk i+1 there, then start loading chunk i+2
            if (i + 1 < i_end) {
                store_loads(cur ^ 1);
                if (i + 2 < i_end) issue_loads(i + 2);
            }
            __syncthreads();  // B3

            // ---- phase C: O = scale (gamma Z + P Delta)
            f32x4 gam = f32x4{1.f, 1.f, 1.f, 1.f};
            if constexpr (!CH) gam = *reinterpret_cast<const f32x4*>(&G[16 * w + 4 * g4]);
            emit_output(i, Zc, gam);
        }
    }
}

// ---------------------------------------------------------------------------
// Head-shared chunk loop for per-key-channel gates
// ---------------------------------------------------------------------------
// With a channel gate every key column decays at its own rate, so the row
// operands of the state products carry per-element factors (log2 prefix lam,
// lam' its prediction row, lam_C the chunk's last row):
//   X = (K o 2^{lam'}) S^T,   Z = (Q o 2^{lam}) S^T,
//   S^T <- diag(2^{lam_C}) S^T + (K o 2^{lam_C - lam})^T Delta
// (GLA gating section; the diagonal decay of the KDA paragraph).  The gated
// rows are the same for every value column of the head, so here they are
// formed once per chunk into LDS (bf16 hi/lo, row factors of raw projections
// folded in) and shared by the waves, where the sliced loop forms them again
// for each 16-column slice.  Two workgroups per (batch, head) split the value
// columns, so that 128 heads occupy 256 compute units; each of the two forms
// the gated rows itself.  One pass, no segments.
// Eight waves in two roles, one of each per SIMD, so that the vector-ALU
// work of one overlaps the matrix-core work of the other:
//   consumers (waves 0-3) hold 16 value columns of S^T each for every key
//     row (as in k_seg) and run the products;
//   producers (waves 4-7) load the next chunks' inputs and form their gated
//     operands, each a chunk ahead of the consumers.
// Per chunk i, three barriers:
//   B0 .. B1   consumers: X, Z, U = V - X, Delta = T' U; producers: K^T
//              fragments of chunk i from the transposed rows by exact identity
//              products (matrix-core work off the consumers' chain), written
//              in place over those rows, then the gated operands of chunk
//              i + 1 into registers;
//   B1 .. B2   consumers: state update and outputs; producers: K and Q rows,
//              V and T' of chunk i + 1 to LDS, then the loads of chunk i + 2;
//   B2 .. B0   producers: the transposed rows, P and the decay of chunk i + 1.
template <int D>
struct ChanShared {
    static constexpr int LDK = D + 8;      // row stride (bf16) of the gated rows, permuted columns
    static constexpr int LDV = D / 2 + 8;  // row stride of the workgroup's value columns
    unsigned short Kg[2][C * LDK];         // K o 2^{lam'} (row factor 1/|k| for raw projections), hi / lo
    unsigned short Qg[2][C * LDK];         // Q o 2^{lam} (1/|q|), hi / lo
    // K o 2^{lam_C - lam} (1/|k|), hi / lo; from B0 to B1 of a chunk each
    // 16-byte piece is overwritten by one lane's K^T fragment (chan_ktf_off)
    unsigned short Kt[2][C * LDK];
    unsigned short V[C * LDV];
    u16x8 Tf[kTfragPerChunk];
    u16x8 Pf[kTfragPerChunk];
    float dec[D];                          // 2^{lam_C}
};

// Where the K^T A-fragment of key tile u, token k-step s, lane l sits in a
// transposed-rows tile: in the 16-byte piece that lane loads as its operand
// for token tile 2 s + (u % 2) and key block u / 2, so that the fragments of
// the two key tiles of a block replace exactly the pieces they were made from.
template <int D>
__device__ __forceinline__ int chan_ktf_off(int u, int s, int l) {
    return (32 * s + 16 * (u & 1) + (l & 15)) * ChanShared<D>::LDK + 32 * (u >> 1) + 8 * (l >> 4);
}

template <int D>
constexpr int chan_threads() { return 4 * D; }  // D / 32 consumer waves of 16 value columns, as many producers

template <int D, bool RAW>
__global__ __launch_bounds__(chan_threads<D>(), 2) void k_chan_head(Problem p, const u16x8* tfrag,
                                                                    const u16x8* pfrag, const float* gates,
                                                                    int xcd_remap) {
    constexpr int NP = chan_threads<D>() / 2;  // threads per role
    constexpr int NW = NP / 64;
    constexpr int LDK = ChanShared<D>::LDK;
    constexpr int LDV = ChanShared<D>::LDV;
    constexpr int KS = D / 32;         // k-steps over the key dimension
    constexpr int TPW = D / 16;        // 16-row key tiles of S^T per value block
    constexpr int GPR = D / 8;         // 16-byte groups per stored row
    constexpr int RUN = C * GPR / NP;  // consecutive tokens per producer thread
    constexpr int VP = C * (D / 2) / 8 / NP;  // 16-byte value pieces per producer thread
    constexpr int TFP = kTfragPerChunk / NP;  // fragment pieces per producer thread
    static_assert(NW == 4 && RUN == 4 && VP * NP * 8 == C * D / 2 && TFP * NP == kTfragPerChunk,
                  "staging split");
    __shared__ __attribute__((aligned(16))) ChanShared<D> sh;

    // (batch, head, value half); with xcd_remap both halves of a head land on
    // one XCD (workgroups are dealt to the 8 XCDs round-robin)
    int id = blockIdx.x, half;
    if (xcd_remap) {
        const int xcd = id & 7, slot = id >> 3;
        half = slot & 1;
        id = (slot >> 1) * 8 + xcd;
    } else {
        half = id & 1;
        id >>= 1;
    }
    const int64_t bh = id;
    const int64_t H = p.H, T = p.T;
    const int b = (int)(bh / H), h = (int)(bh - (bh / H) * H);
    const int64_t row_stride = H * D;
    const int NC = p.NC;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    if (wave >= NW) {
        // ================= producers =================
        const int tid = threadIdx.x - NP;
        const int pw = tid >> 6;  // the producer wave
        const bool ptd = p.order == GDN_PREDICT_THEN_DECAY;
        const unsigned short* kin = static_cast<const unsigned short*>(p.k);
        const unsigned short* qin = static_cast<const unsigned short*>(p.q);
        const unsigned short* vin = static_cast<const unsigned short*>(p.v);
        // Rows are stored with the columns of every 32-column block permuted,
        // 16 hh + 4 g + r -> 8 g + 4 hh + r, so that a lane group's eight
        // k-slots of a k-step are 16 contiguous bytes.  Thread (run, q) takes
        // tokens RUN run .. + RUN - 1 and stored group q (key columns
        // a0 = 32 (q / 4) + 4 (q % 4) .. + 3 and a1 = a0 + 16 .. + 3), so each
        // formed group is one 16-byte store and the 16 groups of a row span
        // every LDS bank; the log2-prefix rows from one before the run (the
        // prediction rows of predict-then-decay) and the chunk's last row.
        const int q = tid % GPR, run = tid / GPR, t0r = RUN * run;
        const int a0 = 32 * (q >> 2) + 4 * (q & 3), a1 = a0 + 16;
        u32x2 kr[RUN][2], qr[RUN][2];
        u32x4 vr[VP], tr[TFP], pr[TFP], pn[TFP];
        f32x4 lam[RUN + 1][2], lamC[2], rq4, rk4;
        // loads of chunk i (all but P)
        auto issue = [&](int i) {
            const int64_t t0 = (int64_t)i * C;
            const int nt = (int)((T - t0) < C ? (T - t0) : C);
            const int64_t base = ((int64_t)b * T + t0) * row_stride + (int64_t)h * D;
#pragma unroll
            for (int j = 0; j < RUN; ++j) {
                const int t = t0r + j;
                kr[j][0] = kr[j][1] = qr[j][0] = qr[j][1] = u32x2{0, 0};
                if (t < nt) {
                    kr[j][0] = ld_g<u32x2>(kin + base + t * row_stride + a0);
                    kr[j][1] = ld_g<u32x2>(kin + base + t * row_stride + a1);
                    qr[j][0] = ld_g<u32x2>(qin + base + t * row_stride + a0);
                    qr[j][1] = ld_g<u32x2>(qin + base + t * row_stride + a1);
                }
            }
#pragma unroll
            for (int k = 0; k < VP; ++k) {
                const int e = tid + NP * k, t = e / (D / 16), c = e % (D / 16);
                vr[k] = u32x4{0, 0, 0, 0};
                if (t < nt) vr[k] = ld_g<u32x4>(vin + base + t * row_stride + (D / 2) * half + 8 * c);
            }
            const float* g = gates + (bh * NC + i) * kChanFloats<D>;
#pragma unroll
            for (int j = 0; j <= RUN; ++j) {
                const int t = t0r + j - 1;
                lam[j][0] = lam[j][1] = zero4();
                if (t >= 0 && (ptd || j > 0)) {
                    lam[j][0] = ld_g<f32x4>(g + t * D + a0);
                    lam[j][1] = ld_g<f32x4>(g + t * D + a1);
                }
            }
            lamC[0] = ld_g<f32x4>(g + (C - 1) * D + a0);
            lamC[1] = ld_g<f32x4>(g + (C - 1) * D + a1);
            if constexpr (RAW) {
                rq4 = ld_g<f32x4>(g + C * D + t0r);
                rk4 = ld_g<f32x4>(g + C * D + C + t0r);
            }
            const u32x4* tp = reinterpret_cast<const u32x4*>(tfrag + (bh * NC + i) * kTfragPerChunk);
#pragma unroll
            for (int k = 0; k < TFP; ++k) tr[k] = ld_g<u32x4>(tp + tid + NP * k);
        };
        // P of chunk i into pn (pr holds the P still to be stored)
        auto issue_p = [&](int i) {
            const u32x4* pp = reinterpret_cast<const u32x4*>(pfrag + (bh * NC + i) * kTfragPerChunk);
#pragma unroll
            for (int k = 0; k < TFP; ++k) pn[k] = ld_g<u32x4>(pp + tid + NP * k);
        };
        // element e of a stored group: column a0 + e (e < 4) or a1 + e - 4
        auto el = [](const f32x4 (&x)[2], int e) { return e < 4 ? x[0][e] : x[1][e - 4]; };
        auto elb = [](const u32x2 (&x)[2], int e) {
            return gdn_bf16_to_f32(__builtin_bit_cast(u16x4, x[e >> 2])[e & 3]);
        };
        // the three gated operands of the staged chunk, split hi/lo
        u32x4 kg[RUN][2], qg[RUN][2], kt[RUN][2];
        f32x4 dec[2];
        auto form = [&]() {
            float eprev[8];  // 2^{lam} of the row before (predict-then-decay)
#pragma unroll
            for (int e = 0; e < 8; ++e) eprev[e] = __builtin_amdgcn_exp2f(el(lam[0], e));
#pragma unroll
            for (int j = 0; j < RUN; ++j) {
                uint32_t kh[4], kl[4], qh[4], ql[4], th[4], tl[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float yk[2], yq[2], yt[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int ee = e + u;
                        const float lt = el(lam[j + 1], ee);
                        const float et = __builtin_amdgcn_exp2f(lt);
                        const float ft = __builtin_amdgcn_exp2f(el(lamC, ee) - lt);
                        float kf = elb(kr[j], ee), qf = elb(qr[j], ee);
                        if constexpr (RAW) {
                            kf *= rk4[j];
                            qf *= rq4[j];
                        }
                        yk[u] = kf * (ptd ? eprev[ee] : et);
                        yq[u] = qf * et;
                        yt[u] = kf * ft;
                        eprev[ee] = et;
                    }
                    split2(yk[0], yk[1], kh[e >> 1], kl[e >> 1]);
                    split2(yq[0], yq[1], qh[e >> 1], ql[e >> 1]);
                    split2(yt[0], yt[1], th[e >> 1], tl[e >> 1]);
                }
                kg[j][0] = u32x4{kh[0], kh[1], kh[2], kh[3]};
                kg[j][1] = u32x4{kl[0], kl[1], kl[2], kl[3]};
                qg[j][0] = u32x4{qh[0], qh[1], qh[2], qh[3]};
                qg[j][1] = u32x4{ql[0], ql[1], ql[2], ql[3]};
                kt[j][0] = u32x4{th[0], th[1], th[2], th[3]};
                kt[j][1] = u32x4{tl[0], tl[1], tl[2], tl[3]};
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dec[0][e] = __builtin_amdgcn_exp2f(lamC[0][e]);
                dec[1][e] = __builtin_amdgcn_exp2f(lamC[1][e]);
            }
        };
        // K and Q rows, V and T' (their tiles are free from B1 on)
        auto store_a = [&]() {
#pragma unroll
            for (int j = 0; j < RUN; ++j) {
                const int o = (t0r + j) * LDK + 8 * q;
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) {
                    *reinterpret_cast<u32x4*>(&sh.Kg[hl][o]) = kg[j][hl];
                    *reinterpret_cast<u32x4*>(&sh.Qg[hl][o]) = qg[j][hl];
                }
            }
#pragma unroll
            for (int k = 0; k < VP; ++k) {
                const int e = tid + NP * k, t = e / (D / 16), c = e % (D / 16);
                *reinterpret_cast<u32x4*>(&sh.V[t * LDV + 8 * c]) = vr[k];
            }
#pragma unroll
            for (int k = 0; k < TFP; ++k) reinterpret_cast<u32x4*>(sh.Tf)[tid + NP * k] = tr[k];
        };
        // the transposed operand's rows, P and the decay (free from B2 on)
        auto store_b = [&]() {
#pragma unroll
            for (int j = 0; j < RUN; ++j) {
                const int o = (t0r + j) * LDK + 8 * q;
                *reinterpret_cast<u32x4*>(&sh.Kt[0][o]) = kt[j][0];
                *reinterpret_cast<u32x4*>(&sh.Kt[1][o]) = kt[j][1];
            }
#pragma unroll
            for (int k = 0; k < TFP; ++k) reinterpret_cast<u32x4*>(sh.Pf)[tid + NP * k] = pr[k];
            if (run == 0) {
                *reinterpret_cast<f32x4*>(&sh.dec[a0]) = dec[0];
                *reinterpret_cast<f32x4*>(&sh.dec[a1]) = dec[1];
            }
        };
        // chunks past the last reload it: every step stays branch-free and
        // its results are never read
        auto clampc = [&](int i) { return i < NC ? i : NC - 1; };
        auto take_p = [&]() {
#pragma unroll
            for (int k = 0; k < TFP; ++k) pr[k] = pn[k];
        };
        if (NC > 0) {
            issue(0);
            issue_p(0);
            take_p();
            form();
            store_a();
            store_b();
            issue(clampc(1));
            issue_p(clampc(1));
            take_p();
        }
        // the loads go out while the consumers run the state update and the
        // outputs, so that no barrier waits on their issue (the compiler is
        // free to sink the formation towards the stores, which measured
        // faster than holding it before B1: the loads then have longer to
        // arrive)
        // K^T fragments of chunk i: producer wave pw takes the hi (pw even) or
        // lo rows of token tiles 2 s', 2 s' + 1 (s' = pw / 2); per key block
        // v the lane loads one piece of each token tile, and the identity
        // selecting key tile 2 v + uu turns them into that tile's A fragment
        // (exact), which goes back over the piece of token tile 2 s' + uu.
        // Only this wave reads these rows, and every store depends on all
        // the wave's loads of its block through the products.
        const int l = tid & 63, g4 = l >> 4, c16 = l & 15;
        const int hl = pw & 1, sj = pw >> 1;
        auto jobs = [&]() {
#pragma unroll
            for (int v = 0; v < TPW / 2; ++v) {
                u16x8 ka[2];
#pragma unroll
                for (int qq = 0; qq < 2; ++qq)
                    ka[qq] = *reinterpret_cast<const u16x8*>(&sh.Kt[hl][chan_ktf_off<D>(2 * v + qq, sj, l)]);
#pragma unroll
                for (int uu = 0; uu < 2; ++uu) {
                    u16x8 idf;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        idf[e] = ((e >> 2) == uu && 4 * g4 + (e & 3) == c16) ? (unsigned short)0x3F80 : (unsigned short)0;
                    u16x4 hv[2];
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq) {
                        const f32x4 d = mfma(ka[qq], idf, zero4());
#pragma unroll
                        for (int r = 0; r < 4; ++r) hv[qq][r] = (unsigned short)(__float_as_uint(d[r]) >> 16);
                    }
                    *reinterpret_cast<u16x8*>(&sh.Kt[hl][chan_ktf_off<D>(2 * v + uu, sj, l)]) = cat(hv[0], hv[1]);
                }
            }
        };
        for (int i = 0; i < NC; ++i) {
            __syncthreads();  // B0
            jobs();           // chunk i
            form();           // chunk i + 1
            __syncthreads();  // B1
            store_a();
            issue(clampc(i + 2));
            issue_p(clampc(i + 2));
            __syncthreads();  // B2
            store_b();
            take_p();
        }
        return;
    }

    // ================= consumers =================
    const int tid = threadIdx.x;
    const int w = wave;
    const int l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int vcol = (D / 2) * half + 16 * w + c16;  // the lane's value column

    // state: S^T tile u, lane (v = vcol, a = 16 u + 4 g4 + r)
    f32x4 Sacc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
        Sacc[u] = p.s0 ? ld_g<f32x4>(p.s0 + (bh * D + vcol) * D + 16 * u + 4 * g4) : zero4();

    for (int i = 0; i < NC; ++i) {
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
        __syncthreads();  // B0: chunk i staged

        // S^T as B operands of every k-step, split hi/lo
        u16x8 sbh[KS], sbl[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u16x4 h0, l0, h1, l1;
            split4(Sacc[2 * s], h0, l0);
            split4(Sacc[2 * s + 1], h1, l1);
            sbh[s] = cat(h0, h1);
            sbl[s] = cat(l0, l1);
        }
        // X = Kg S^T, Z = Qg S^T (both operands split: three products)
        f32x4 X[4], Z[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) X[m] = Z[m] = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int o = (16 * m + c16) * LDK + 32 * s + 8 * g4;
                const u16x8 kh = *reinterpret_cast<const u16x8*>(&sh.Kg[0][o]);
                const u16x8 kl = *reinterpret_cast<const u16x8*>(&sh.Kg[1][o]);
                X[m] = mfma(kh, sbh[s], X[m]);
                X[m] = mfma(kh, sbl[s], X[m]);
                X[m] = mfma(kl, sbh[s], X[m]);
                const u16x8 qh = *reinterpret_cast<const u16x8*>(&sh.Qg[0][o]);
                const u16x8 ql = *reinterpret_cast<const u16x8*>(&sh.Qg[1][o]);
                Z[m] = mfma(qh, sbh[s], Z[m]);
                Z[m] = mfma(qh, sbl[s], Z[m]);
                Z[m] = mfma(ql, sbh[s], Z[m]);
            }
        // U = V - X, split hi/lo
        u16x4 uh[4], ul[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x[r] = gdn_bf16_to_f32(sh.V[(16 * m + 4 * g4 + r) * LDV + 16 * w + c16]) - X[m][r];
            split4(x, uh[m], ul[m]);
        }
        // Delta = T' U (tile m takes k-steps s <= m / 2), split hi/lo
        u16x4 dh[4], dl[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 d1 = zero4();
#pragma unroll
            for (int s = 0; s <= (m >> 1); ++s) {
                const u16x8 th = sh.Tf[(tslot(m, s) * 2 + 0) * 64 + l];
                const u16x8 tl = sh.Tf[(tslot(m, s) * 2 + 1) * 64 + l];
                const u16x8 xh = cat(uh[2 * s], uh[2 * s + 1]);
                const u16x8 xl = cat(ul[2 * s], ul[2 * s + 1]);
                d1 = mfma(th, xh, d1);
                d1 = mfma(th, xl, d1);
                d1 = mfma(tl, xh, d1);
            }
            split4(d1, dh[m], dl[m]);
        }
        __syncthreads();  // B1: the gated rows, V and T' of chunk i are read, K^T fragments complete

        // S^T <- diag(2^{lam_C}) S^T + K^T Delta (A rows a = 16 u + c16)
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            f32x4 acc = *reinterpret_cast<const f32x4*>(&sh.dec[16 * u + 4 * g4]) * Sacc[u];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u16x8 kh = *reinterpret_cast<const u16x8*>(&sh.Kt[0][chan_ktf_off<D>(u, s, l)]);
                const u16x8 kl = *reinterpret_cast<const u16x8*>(&sh.Kt[1][chan_ktf_off<D>(u, s, l)]);
                const u16x8 bh_ = cat(dh[2 * s], dh[2 * s + 1]);
                const u16x8 bl_ = cat(dl[2 * s], dl[2 * s + 1]);
                acc = mfma(kh, bh_, acc);
                acc = mfma(kh, bl_, acc);
                acc = mfma(kl, bh_, acc);
            }
            Sacc[u] = acc;
        }
        // O = scale (Z + P Delta), rows past the sequence end dropped
        {
            float* obase = p.out + ((int64_t)b * T + t0) * row_stride + (int64_t)h * D + vcol;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 o1 = zero4();
#pragma unroll
                for (int s = 0; s <= (m >> 1); ++s) {
                    const u16x8 ph = sh.Pf[(tslot(m, s) * 2 + 0) * 64 + l];
                    const u16x8 pl = sh.Pf[(tslot(m, s) * 2 + 1) * 64 + l];
                    const u16x8 xh = cat(dh[2 * s], dh[2 * s + 1]);
                    const u16x8 xl = cat(dl[2 * s], dl[2 * s + 1]);
                    o1 = mfma(ph, xh, o1);
                    o1 = mfma(ph, xl, o1);
                    o1 = mfma(pl, xh, o1);
                }
                const f32x4 o = p.scale * (Z[m] + o1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * m + 4 * g4 + r;
                    if (t < nt) st_g<float>(obase + (int64_t)t * row_stride, o[r]);
                }
            }
        }
        __syncthreads();  // B2: K^T fragments, P and the decay of chunk i are read
    }

    if (p.s_out) {
#pragma unroll
        for (int u = 0; u < TPW; ++u)
            st_g<f32x4>(p.s_out + (bh * D + vcol) * D + 16 * u + 4 * g4, Sacc[u]);
    }
}

// ---------------------------------------------------------------------------
// Whole-head chunk loop (scalar gate)
// ---------------------------------------------------------------------------
// One workgroup per (batch, head, segment) keeps the whole state S^T (D x D,
// fp32) in registers: wave w holds value columns 16w..16w+15 for every key
// row, so each chunk's K, Q, V and T' are fetched from L2 once per head and
// shared by the D/16 waves through LDS, and no intermediate crosses waves
// (each wave's X, Delta and output columns depend only on its own slice).
// Long sequences are cut into segments run side by side in two passes, after
// the sequence-parallel notes (the state at a segment end is the increment
// from a zero start plus the entry state through the scaling matrix):
//   pass 1 (kSegState): one workgroup per segment g < G-1 runs the increment
//     S^D from zero (segment 0: from the true start state) on one half of its
//     waves and the scaling matrix M from I (the same recurrence with V = 0)
//     on the other, on the same staged chunks; end values only;
//   the start-state chain S_start(g+1) = S^D_end(g) + S_start(g) M_end(g);
//   pass 2 (kSegOut): every segment from its true entry state, with outputs.
// Per chunk: X = K S^T and Z = Q S^T (S^T split hi/lo), U = V - diag(gamma') X,
// Delta = T' U, S^T <- gamma_C S^T + K^T diag(gamma_C / gamma) Delta and
// O = scale (diag(gamma) Z + P Delta); P (gated causal scores) is formed per
// chunk by the waves together and handed over through LDS.
constexpr int kSegOut = 0, kSegState = 1;

// K and Q rows are kept with the columns of every 32-column block permuted,
// 16h + 4g + r -> 8g + 4h + r, so that the 8 key slots of lane group g of a
// k-step in the paired-tile order (4g + r of one 16-column half, then of the
// other) are 16 contiguous bytes.
template <int D, int MODE>
struct SegShared {
    static constexpr bool OUT = MODE == kSegOut;
    static constexpr int LDK = D + 8;  // row stride (bf16) of K, Q, V
    unsigned short K[C * LDK];
    unsigned short V[C * LDK];
    u16x8 KtF[D / 16][2][64];  // K^T A-fragments: [key tile][token k-step][lane]
    u16x8 Tf[kTfragPerChunk];
    float G[kGateFloats];
    unsigned short Q[OUT ? C * LDK : 8];
    u16x8 Pf[OUT ? 4 : 1][2][2][64];  // P fragments per token tile
    static constexpr int LDO = D + 4;  // row stride (fp32) of the output tile
    float O[OUT ? C * LDO : 4];
};

// KIND 0 (output pass): the state S (values from V); KIND 2 (state pass): S
// and the scaling matrix M (V = 0, identity start) in one workgroup, waves
// 0 .. NWH - 1 on S and NWH .. 2 NWH - 1 on M, sharing the staged chunk and
// the K^T fragments; KIND 3 (state pass, NV = 2): every wave holds the same
// value columns of S (slot 0) and of M (slot 1).
template <int D, int MODE, int KIND, int NV>
__device__ __forceinline__ void seg_body(const Problem& p, const Split& sp, const WsLayout& L, char* wsb,
                                         const u16x8* tfrag, const float* gates, int64_t bh, int gseg,
                                         SegShared<D, MODE>& sh) {
    constexpr bool OUT = MODE == kSegOut;
    static_assert(KIND == 0 || KIND == 2 || (KIND == 3 && NV == 2), "S alone, or S and M together");
    // KIND 3: each wave holds the same value columns of S (slot 0) and M (slot 1)
    constexpr int NWH = KIND == 3 ? D / 16 : D / (16 * NV);  // waves per state; wave w owns value columns 16 NV (w % NWH) ..
    constexpr int NW = KIND == 2 ? 2 * NWH : NWH;
    constexpr int NT = 64 * NW;
    constexpr int LDK = SegShared<D, MODE>::LDK;
    constexpr int LDO = SegShared<D, MODE>::LDO;
    constexpr int KS = D / 32;         // k-steps over the key dimension
    constexpr int TPW = D / 16;        // 16-row key tiles of S^T per value block
    constexpr int PPR = D / 8;         // 16-byte pieces per K/Q/V row
    constexpr int KP = C * PPR / NT;   // pieces per thread and matrix
    constexpr int TFP = (kTfragPerChunk + NT - 1) / NT;
    constexpr int GP = kGateFloats / 4;
    static_assert(C * PPR % NT == 0 && GP <= NT, "staging split");
    // the gate pieces read: the row factors only for raw projections
    const int gp_n = p.raw ? kGatePiecesRaw : kGatePieces;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = KIND == 2 ? w % NWH : w;                      // value block of the wave
    const bool mk = KIND == 2 && w >= NWH;                      // the wave runs M
    auto is_m = [&](int n) { return KIND == 3 ? n == 1 : mk; };  // slot n holds M
    const int l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int64_t H = p.H, T = p.T;
    const int b = (int)(bh / H), h = (int)(bh - (bh / H) * H);
    const int i_begin = gseg * sp.per;
    const int i_end = min(p.NC, (gseg + 1) * sp.per);
    const unsigned short* kin = static_cast<const unsigned short*>(p.k);
    const unsigned short* qin = static_cast<const unsigned short*>(p.q);
    const unsigned short* vin = static_cast<const unsigned short*>(p.v);
    const int64_t row_stride = H * D;

    // ---- state: value block n of the wave, S^T tile tau, lane
    // (v = 16 (NV w + n) + c16, a = 16 tau + 4 g4 + r)
    int v[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) v[n] = KIND == 3 ? 16 * wv + c16 : 16 * (NV * wv + n) + c16;
    f32x4 Sacc[NV][TPW];
    // Entry states: the caller's start state for segment 0 of a single pass;
    // with segments, every segment of the output pass reads its slot of the
    // workspace's start states (segment 0's copied there by the state pass),
    // so the start state may be the buffer the last segment's final state
    // goes to (in-place streaming) with no ordering between the workgroups
    // of the output pass.
    float* const sstart_ws = reinterpret_cast<float*>(wsb + L.sstart) + (bh * sp.G + gseg) * D * D;
    {
        const float* src = nullptr;
        if (!mk) {
            if (OUT && sp.G > 1) src = sstart_ws;
            else if (gseg == 0) src = p.s0 ? p.s0 + bh * D * D : nullptr;
        }
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int a0 = 16 * u + 4 * g4;
                if (is_m(n)) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sacc[n][u][r] = v[n] == a0 + r ? 1.f : 0.f;
                } else if (src) {
                    Sacc[n][u] = *reinterpret_cast<const f32x4*>(src + (int64_t)v[n] * D + a0);
                } else {
                    Sacc[n][u] = zero4();
                }
            }
        if (!OUT && gseg == 0) {
#pragma unroll
            for (int n = 0; n < NV; ++n)
                if (!is_m(n)) {
#pragma unroll
                    for (int u = 0; u < TPW; ++u)
                        *reinterpret_cast<f32x4*>(sstart_ws + (int64_t)v[n] * D + 16 * u + 4 * g4) = Sacc[n][u];
                }
        }
    }

    // ---- staging: chunk i+1 in registers while chunk i computes
    u32x4 kr[KP], vr[KP], qr[OUT ? KP : 1], tr[TFP], gr;
    // part mask: 1 K, 2 V, 4 Q, 8 T' fragments and gate block
    auto issue = [&](int i, int parts = 15) {
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int e = tid + NT * k, t = min(e / PPR, nt - 1), c8 = e % PPR;
            const int64_t off = (((int64_t)b * T + t0 + t) * H + h) * D + c8 * 8;
            if (parts & 1) kr[k] = *reinterpret_cast<const u32x4*>(kin + off);
            if (parts & 2) vr[k] = *reinterpret_cast<const u32x4*>(vin + off);
            if (OUT && (parts & 4)) qr[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qin + off));
        }
        if (parts & 8) {
            const u32x4* tp = reinterpret_cast<const u32x4*>(tfrag + (bh * p.NC + i) * kTfragPerChunk);
#pragma unroll
            for (int k = 0; k < TFP; ++k) tr[k] = tp[min(tid + NT * k, kTfragPerChunk - 1)];
            gr = reinterpret_cast<const u32x4*>(gates + (bh * p.NC + i) * kGateFloats)[min(tid, gp_n - 1)];
        }
    };
    auto store = [&](int i) {
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
        const u32x4 z = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int e = tid + NT * k, t = e / PPR, c8 = e % PPR;
            const bool ok = t < nt;
            *reinterpret_cast<u32x4*>(&sh.V[t * LDK + c8 * 8]) = ok ? vr[k] : z;
            // columns 8 c8 .. +3 and +4 .. +7 of block c8 / 4 go to the
            // permuted positions 16 (c8 % 2) + 4 h and that + 8, h = (c8 % 4) / 2
            const int p0 = t * LDK + 32 * (c8 >> 2) + 16 * (c8 & 1) + 4 * ((c8 >> 1) & 1);
            const u32x4 kk = ok ? kr[k] : z;
            *reinterpret_cast<u32x2*>(&sh.K[p0]) = u32x2{kk[0], kk[1]};
            *reinterpret_cast<u32x2*>(&sh.K[p0 + 8]) = u32x2{kk[2], kk[3]};
            if (OUT) {
                const u32x4 qq = ok ? qr[k] : z;
                *reinterpret_cast<u32x2*>(&sh.Q[p0]) = u32x2{qq[0], qq[1]};
                *reinterpret_cast<u32x2*>(&sh.Q[p0 + 8]) = u32x2{qq[2], qq[3]};
            }
        }
#pragma unroll
        for (int k = 0; k < TFP; ++k)
            if (kTfragPerChunk % NT == 0 || tid + NT * k < kTfragPerChunk)
                reinterpret_cast<u32x4*>(sh.Tf)[tid + NT * k] = tr[k];
        if (tid < gp_n) reinterpret_cast<u32x4*>(sh.G)[tid] = gr;
    };

    // ---- P blocks (m, c), c <= m, dealt over the waves: rows j of tile c,
    // columns t of tile m, so that blocks 2s, 2s + 1 form the A fragment of
    // k-step s as they stand; P_tj = exp(g_t - g_j) q_t.k_j (j <= t)
    auto scores = [&]() {
        for (int bi = w; bi < 10; bi += NW) {
            const int m = bi >= 6 ? 3 : bi >= 3 ? 2 : bi >= 1 ? 1 : 0;
            const int c = bi - m * (m + 1) / 2;
            const int t = 16 * m + c16;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u16x8 ka = *reinterpret_cast<const u16x8*>(&sh.K[(16 * c + c16) * LDK + 32 * s + 8 * g4]);
                const u16x8 qb = *reinterpret_cast<const u16x8*>(&sh.Q[t * LDK + 32 * s + 8 * g4]);
                acc = mfma(ka, qb, acc);
            }
            const float gt = sh.G[192 + t];
            const f32x4 gj = *reinterpret_cast<const f32x4*>(&sh.G[192 + 16 * c + 4 * g4]);
            f32x4 pt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * c + 4 * g4 + r;
                pt[r] = j <= t ? acc[r] * __expf(gt - gj[r]) : 0.f;
            }
            if (p.raw) {
                const float rq = sh.G[kGateRq + t];
                const f32x4 rk = *reinterpret_cast<const f32x4*>(&sh.G[kGateRk + 16 * c + 4 * g4]);
                pt = rq * (pt * rk);
            }
            u16x4 hi, lo;
            split4(pt, hi, lo);
            reinterpret_cast<u16x4*>(&sh.Pf[m][c >> 1][0][l])[c & 1] = hi;
            reinterpret_cast<u16x4*>(&sh.Pf[m][c >> 1][1][l])[c & 1] = lo;
        }
    };

    if constexpr (OUT) {
        // the never-written halves of the P fragments: blocks (0, 1), (2, 3)
        if (w == 0) {
            const u16x4 z = u16x4{0, 0, 0, 0};
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
                reinterpret_cast<u16x4*>(&sh.Pf[0][0][hl][l])[1] = z;
                reinterpret_cast<u16x4*>(&sh.Pf[2][1][hl][l])[1] = z;
            }
        }
    }
    // the output tile of chunk i (LDS) to HBM: 16-byte pieces of whole rows,
    // rows past the sequence end dropped.  O is written once and Q read once
    // per forward; both go with non-temporal hints, which leaves the caches
    // to K, V and T' (read by both passes) and measured 7 % off this pass
    auto flush = [&](int i) {
        constexpr int OPR = D / 4, OP = C * OPR / NT;
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
        float* obase = p.out + (((int64_t)b * T + t0) * H + h) * D;
#pragma unroll
        for (int k = 0; k < OP; ++k) {
            const int e = tid + NT * k, t = e / OPR, c4 = e % OPR;
            if (t < nt)
                __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&sh.O[t * LDO + 4 * c4]),
                                            reinterpret_cast<f32x4*>(obase + (int64_t)t * row_stride + 4 * c4));
        }
    };
    if (i_begin < i_end) {
        issue(i_begin);
        store(i_begin);
    }

    // identity B fragment selecting the key half hh of a k-step: lane (column
    // c16, slots e) is one where the slot holds key 16 hh + c16 of the block
    auto idfrag = [&](int hh) {
        u16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = ((e >> 2) == hh && 4 * g4 + (e & 3) == c16) ? (unsigned short)0x3F80 : (unsigned short)0;
        return f;
    };

    for (int i = i_begin; i < i_end; ++i) {
        __syncthreads();  // chunk i staged
        // the output pass fetches the next chunk's K and V here, its Q, T'
        // and gates after the first product and writes the previous chunk's
        // output tile after the second, so that the loads and stores of one
        // chunk (about 100 KiB per CU) do not queue up at one point and stall
        // the waves behind them
        const bool more = i + 1 < i_end;
        if constexpr (OUT)
            if (more) issue(i + 1, 3);
        if constexpr (OUT) scores();
        // K^T fragments by exact MFMA products with the identity: job (s', u)
        // turns token tiles 2s', 2s' + 1 of key tile u into the A fragment of
        // rows a = 16u + c16, k-step s' over tokens; every wave takes the same
        // number of jobs
        static_assert((2 * TPW) % NW == 0, "K^T jobs split evenly over the waves");
#pragma unroll
        for (int jj = 0; jj < 2 * TPW / NW; ++jj) {
            const int job = w + NW * jj;
            const int sp_ = job & 1, u = job >> 1;
            u16x4 half[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int m = 2 * sp_ + q;
                const u16x8 ka = *reinterpret_cast<const u16x8*>(&sh.K[(16 * m + c16) * LDK + 32 * (u >> 1) + 8 * g4]);
                const f32x4 d = mfma(ka, idfrag(u & 1), zero4());
#pragma unroll
                for (int r = 0; r < 4; ++r) half[q][r] = (unsigned short)(__float_as_uint(d[r]) >> 16);
            }
            sh.KtF[u][sp_][l] = cat(half[0], half[1]);
        }

        // S^T as B operands of every k-step (tiles 2s, 2s + 1), split hi/lo
        // (the output pass keeps them for Z; the state pass forms them per
        // k-step inside the X product)
        u16x8 sbh[NV][OUT ? KS : 1], sbl[NV][OUT ? KS : 1];
        if constexpr (OUT) {
#pragma unroll
            for (int n = 0; n < NV; ++n)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    u16x4 h0, l0, h1, l1;
                    split4(Sacc[n][2 * s], h0, l0);
                    split4(Sacc[n][2 * s + 1], h1, l1);
                    sbh[n][s] = cat(h0, h1);
                    sbl[n][s] = cat(l0, l1);
                }
        }
        // rows 16m.. of src times S^T for every value block of the wave: lane
        // (column v, rows t = 16m + 4 g4 + r); each A fragment read once
        auto times_state = [&](const unsigned short* src, int m, f32x4 (&res)[NV]) {
#pragma unroll
            for (int n = 0; n < NV; ++n) res[n] = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u16x8 ra = *reinterpret_cast<const u16x8*>(&src[(16 * m + c16) * LDK + 32 * s + 8 * g4]);
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    res[n] = mfma(ra, sbh[n][s], res[n]);
                    res[n] = mfma(ra, sbl[n][s], res[n]);
                }
            }
        };
        // X = K S^T
        f32x4 X[4][NV];
        if constexpr (OUT) {
#pragma unroll
            for (int m = 0; m < 4; ++m) times_state(sh.K, m, X[m]);
        } else {
            // k-step outer, one accumulator per tile (the other waves of the
            // SIMD hide the dependent products; this keeps the state pass's
            // registers low)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < NV; ++n) X[m][n] = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u16x8 bh_[NV], bl_[NV];
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    u16x4 h0, l0, h1, l1;
                    split4(Sacc[n][2 * s], h0, l0);
                    split4(Sacc[n][2 * s + 1], h1, l1);
                    bh_[n] = cat(h0, h1);
                    bl_[n] = cat(l0, l1);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const u16x8 ra = *reinterpret_cast<const u16x8*>(&sh.K[(16 * m + c16) * LDK + 32 * s + 8 * g4]);
#pragma unroll
                    for (int n = 0; n < NV; ++n) {
                        X[m][n] = mfma(ra, bh_[n], X[m][n]);
                        X[m][n] = mfma(ra, bl_[n], X[m][n]);
                    }
                }
            }
        }
        // (the state pass fetches the next chunk only now, so that the staging
        // registers are not live across these products)
        if constexpr (!OUT)
            if (more) issue(i + 1);
        if constexpr (OUT)
            if (more) issue(i + 1, 12);
        // U = V - diag(gamma') X, split hi/lo; Z = Q S^T (entry state of the
        // chunk) in the same loop so that its products overlap the U arithmetic
        u16x4 uh[NV][4], ul[NV][4];
        f32x4 Z[OUT ? 4 : 1][NV];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if constexpr (OUT) times_state(sh.Q, m, Z[m]);
            const f32x4 gp = *reinterpret_cast<const f32x4*>(&sh.G[64 + 16 * m + 4 * g4]);
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                f32x4 u;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vv = is_m(n) ? 0.f : gdn_bf16_to_f32(sh.V[(16 * m + 4 * g4 + r) * LDK + v[n]]);
                    u[r] = vv - gp[r] * X[m][n][r];
                }
                split4(u, uh[n][m], ul[n][m]);
            }
        }
        if constexpr (OUT)
            if (i > i_begin) flush(i - 1);
        // Delta = T' U (tile m takes k-steps s <= m / 2); Delta hi/lo for the
        // output and Delta-bar = diag(gamma_C / gamma) Delta hi/lo for the state
        u16x4 dh[NV][4], dl[NV][4], dbh[NV][4], dbl[NV][4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 d1[NV];
#pragma unroll
            for (int n = 0; n < NV; ++n) d1[n] = zero4();
#pragma unroll
            for (int s = 0; s <= (m >> 1); ++s) {
                const u16x8 th = sh.Tf[(tslot(m, s) * 2 + 0) * 64 + l];
                const u16x8 tl = sh.Tf[(tslot(m, s) * 2 + 1) * 64 + l];
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    const u16x8 xh = cat(uh[n][2 * s], uh[n][2 * s + 1]);
                    const u16x8 xl = cat(ul[n][2 * s], ul[n][2 * s + 1]);
                    d1[n] = mfma(th, xh, d1[n]);
                    d1[n] = mfma(th, xl, d1[n]);
                    d1[n] = mfma(tl, xh, d1[n]);
                }
            }
            const f32x4 rat = *reinterpret_cast<const f32x4*>(&sh.G[128 + 16 * m + 4 * g4]);
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                const f32x4 dd = d1[n];
                if constexpr (OUT) split4(dd, dh[n][m], dl[n][m]);
                split4(rat * dd, dbh[n][m], dbl[n][m]);
            }
        }
        __syncthreads();  // K^T (and P) fragments of chunk i complete

        // S^T <- gamma_C S^T + K^T Delta-bar (A operand rows a = 16 tau + c16,
        // k-slots t in the paired-tile order)
        const float gC = sh.G[256];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            f32x4 acc[NV];
#pragma unroll
            for (int n = 0; n < NV; ++n) acc[n] = gC * Sacc[n][u];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u16x8 ka = sh.KtF[u][s][l];
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    acc[n] = mfma(ka, cat(dbh[n][2 * s], dbh[n][2 * s + 1]), acc[n]);
                    acc[n] = mfma(ka, cat(dbl[n][2 * s], dbl[n][2 * s + 1]), acc[n]);
                }
            }
#pragma unroll
            for (int n = 0; n < NV; ++n) Sacc[n][u] = acc[n];
        }

        // O = scale (diag(gamma) Z + P Delta) into the LDS output tile; it goes
        // to HBM early in the next chunk (staging waits on the vector-memory
        // counter, which also counts stores)
        if constexpr (OUT) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 o1[NV];
#pragma unroll
                for (int n = 0; n < NV; ++n) o1[n] = zero4();
#pragma unroll
                for (int s = 0; s <= (m >> 1); ++s) {
                    const u16x8 ph = sh.Pf[m][s][0][l];
                    const u16x8 pl = sh.Pf[m][s][1][l];
#pragma unroll
                    for (int n = 0; n < NV; ++n) {
                        const u16x8 xh = cat(dh[n][2 * s], dh[n][2 * s + 1]);
                        const u16x8 xl = cat(dl[n][2 * s], dl[n][2 * s + 1]);
                        o1[n] = mfma(ph, xh, o1[n]);
                        o1[n] = mfma(ph, xl, o1[n]);
                        o1[n] = mfma(pl, xh, o1[n]);
                    }
                }
                const f32x4 gam = *reinterpret_cast<const f32x4*>(&sh.G[16 * m + 4 * g4]);
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    const f32x4 o = p.scale * (gam * Z[m][n] + o1[n]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sh.O[(16 * m + 4 * g4 + r) * LDO + v[n]] = o[r];
                }
            }
        }
        __syncthreads();  // every read of chunk i's inputs done, output tile complete
        if (i + 1 < i_end) store(i + 1);
    }
    if constexpr (OUT)
        if (i_begin < i_end) flush(i_end - 1);

    // ---- end value: final state (last segment of pass 2), S^D (pass 1, row
    // major) or M (pass 1, as the chain's operand fragments)
    float* dst = nullptr;
    if (OUT) {
        if (gseg == sp.G - 1 && p.s_out) dst = p.s_out + bh * D * D;
    } else {
        if (!mk) dst = reinterpret_cast<float*>(wsb + L.sdend) + (bh * sp.G + gseg) * D * D;
    }
    if (dst) {
#pragma unroll
        for (int n = 0; n < NV; ++n)
            if (!is_m(n)) {
#pragma unroll
                for (int u = 0; u < TPW; ++u)
                    *reinterpret_cast<f32x4*>(&dst[(int64_t)v[n] * D + 16 * u + 4 * g4]) = Sacc[n][u];
            }
    }
    if constexpr (!OUT) {
        if (gseg > 0) {  // (segment 0 needs no M)
            // M_end(g) goes out as the start-state chain's B operands, split
            // hi/lo: fragment (column tile nt, k-step s) holds, for lane
            // (g, c), rows 32 s + 8 g .. + 7 of column 16 nt + c.  An M wave
            // owns rows v0 .. v0 + 16 NV - 1 of every column: it puts them in
            // a private LDS tile (column-major, 16 NV floats per column) and
            // reads back runs of 8 rows of one column, one fragment slot per
            // lane, so each slot leaves as one 16-byte store per half.
            constexpr int LW = KIND == 3 ? 16 : 16 * NV;  // rows of M per wave
            static_assert(sizeof(SegShared<D, MODE>) >= sizeof(float) * NWH * D * LW, "M tiles fit");
            __syncthreads();  // the chunk loop is done with LDS
            if (KIND == 3 || mk) {
                float* Wt = reinterpret_cast<float*>(&sh) + wv * (D * LW);
#pragma unroll
                for (int n = 0; n < NV; ++n)
                    if (is_m(n)) {
                        const int col = KIND == 3 ? 0 : 16 * n;
#pragma unroll
                        for (int u = 0; u < TPW; ++u)
#pragma unroll
                            for (int r = 0; r < 4; ++r) Wt[(16 * u + 4 * g4 + r) * LW + col + c16] = Sacc[n][u][r];
                    }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const int v0 = LW * wv;
                u16x8* frag = reinterpret_cast<u16x8*>(wsb + L.mend) + (bh * sp.G + gseg) * (int64_t)(D * D / 4);
#pragma unroll
                for (int q = l; q < 2 * LW * TPW; q += 64) {  // (u, run h, column c)
                    const int c = q & 15, h = (q >> 4) % (LW / 8), u = q / (2 * LW);
                    const int vr = v0 + 8 * h, s = vr >> 5, fl = 16 * ((vr & 31) >> 3) + c;
                    const float* src = &Wt[(16 * u + c) * LW + 8 * h];
                    u16x4 h0, l0, h1, l1;
                    split4(*reinterpret_cast<const f32x4*>(src), h0, l0);
                    split4(*reinterpret_cast<const f32x4*>(src + 4), h1, l1);
                    frag[((u * KS + s) * 2 + 0) * 64 + fl] = cat(h0, h1);
                    frag[((u * KS + s) * 2 + 1) * 64 + fl] = cat(l0, l1);
                }
            }
        }
    }
}

// Start-state chain of the whole-head path, S_start(g + 1) = S^D_end(g) +
// S_start(g) M_end(g), g = 1 .. G - 2, from S_start(1) = S^D_end(0)
// (sequence-parallel notes: the state at a segment end is the increment plus
// the entry state through the scaling matrix).  Each map X -> X M + A is
// affine, and affine maps compose associatively (GDN blog, section 2.3), so
// for many segments the chain runs as a two-level scan over blocks of b
// consecutive maps:
//   compose  (blocks in parallel)  P_j = M(a) ... M(e - 1), Q_j the matching
//            addend, so that S_start(e) = S_start(a) P_j + Q_j;
//   blocks   (sequential over j)   S_start(a_{j+1}) = S_start(a_j) P_j + Q_j;
//   expand   (blocks in parallel)  the starts inside each block, one map at a
//            time from the block's start.
// That is about 3 sqrt(G) dependent steps instead of G - 2; below
// kChainBlockMin maps the plain sequential chain runs.
// Every mode is the same row chain: X <- X Mult(s) + Add(s) for s < nsteps on
// 16 rows of one head per workgroup (rows of the start state are independent
// chains), each step a 16 x D x D product on bf16 MFMA with both factors split
// hi/lo (three products, fp32 accumulate).  Mult(s + 1) and the rows of
// Add(s + 1) are fetched while step s computes.  Workgroups are dealt to the
// eight XCDs round-robin; when the count of groups that share their Mult
// matrices is a multiple of eight, each group is placed on one XCD, so that it
// shares the L2 copy (one HBM fetch per group and step).
constexpr int kChainBlockMin = 16;
enum { kChainSeq = 0, kChainCompose = 1, kChainBlocks = 2, kChainExpand = 3 };
struct ChainPlan {
    int b;   // maps per block (0: sequential chain)
    int nb;  // blocks
};
// b about sqrt(n), but no more blocks than keep one workgroup per (head,
// block, 16 rows) within the 256 CUs (the compose and expand grids run in one
// round); the plain chain when the scan would not take fewer steps
ChainPlan chain_plan(int G, int64_t heads, int D) {
    const int n = G - 2;  // maps M_end(1 .. G - 2)
    ChainPlan c{0, 0};
    if (n < kChainBlockMin) return c;
    int b = 1;
    while (b * b < n) ++b;
    const int64_t nb_cap = 256 / ((D / 16) * heads);
    if (nb_cap >= 2 && (n + b - 1) / b > nb_cap) b = (int)((n + nb_cap - 1) / nb_cap);
    const int nb = (n + b - 1) / b;
    if (2 * (b - 1) + nb >= n) return c;
    c.b = b;
    c.nb = nb;
    return c;
}

// Multipliers (M_end and the composed P_j) are stored as the MFMA B operands
// of these products, split hi/lo (fragment (column tile nt, k-step s): lane
// (g, c) holds rows 32 s + 8 g .. + 7 of column 16 nt + c), written so by the
// state pass and by the compose step; each wave loads the fragments of its
// column tiles for step s + 1 while step s computes, straight into registers.
// NR = 2 (compose): the P and the Q rows of a block in one workgroup, both
// from (I, 0) through every map of the block.
// One wave per 16-column tile of the product (D / 16 waves: two per SIMD at
// D = 128, so the matrix cores run at the two-wave rate); each step's
// multiplier fragments and addend rows are fetched two steps ahead into three
// rotating register sets.
template <int D>
constexpr int chain_threads() { return 64 * (D / 16); }
template <int D, int NR>
__global__ __launch_bounds__(chain_threads<D>()) void k_chain_rows(Problem p, Split sp, WsLayout L, char* wsb,
                                                                  int mode, ChainPlan cp) {
    constexpr int LD = D + 4;
    constexpr int KS = D / 32;           // k-steps of the product
    constexpr int NT = chain_threads<D>();
    constexpr int SP = 16 * D / 4;       // float4 pieces of 16 rows
    constexpr int SR = (SP + NT - 1) / NT;
    constexpr int NX = D / 16;           // row blocks per head
    constexpr int64_t DD = (int64_t)D * D;
    constexpr int64_t FD = DD / 4;       // u16x8 per fragment matrix (hi and lo)
    __shared__ __attribute__((aligned(16))) float Cb[2][NR][16 * LD];
    __shared__ __attribute__((aligned(16))) float SDs[2][16 * LD];
    const int64_t heads = p.B * p.H;
    const bool per_block = mode == kChainCompose || mode == kChainExpand;
    const int64_t groups = heads * (per_block ? cp.nb : 1);  // workgroups of a group share Mult
    int64_t grp;
    int x;
    if (groups % 8 == 0) {
        const int64_t slot = blockIdx.x / 8;
        grp = (slot / NX) * 8 + blockIdx.x % 8;
        x = (int)(slot % NX);
    } else {
        grp = blockIdx.x / NX;
        x = (int)(blockIdx.x % NX);
    }
    const int64_t bh = per_block ? grp / cp.nb : grp;
    const int j = per_block ? (int)(grp % cp.nb) : 0;
    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int nt = __builtin_amdgcn_readfirstlane(tid >> 6);  // the wave's column tile
    const int r0 = 16 * x;
    const float* sdend = reinterpret_cast<const float*>(wsb + L.sdend) + bh * sp.G * DD;
    const u16x8* mfr = reinterpret_cast<const u16x8*>(wsb + L.mend) + bh * sp.G * FD;
    float* sstart = reinterpret_cast<float*>(wsb + L.sstart) + bh * sp.G * DD;
    u16x8* pfr = reinterpret_cast<u16x8*>(wsb + L.blk) + bh * cp.nb * FD;
    float* qblk = reinterpret_cast<float*>(wsb + L.blk) + (heads + bh) * cp.nb * DD;

    // the job: start rows of each set (nullptr: the identity for set 0, zero
    // otherwise), step operands Mult(s) = mult0 + s FD (fragments) and Add(s)
    // = add0 + s DD (rows, last set only), X written before step s (pre),
    // after it (post), at the end (fin, rows; compose: P_j as fragments)
    const int a = 1 + j * cp.b;                               // first map of block j
    const int len = per_block ? min(cp.b, sp.G - 1 - a) : 0;  // its maps a .. a + len - 1
    const float* init[NR];
    const u16x8* mult0;
    const float* add0;
    float* pre0 = nullptr;
    float* post0 = nullptr;
    float* fin = nullptr;
    u16x8* fin_frag = nullptr;
    int64_t pre_stride = DD;
    int nsteps;
    if (mode == kChainSeq) {
        init[0] = sdend;
        nsteps = sp.G - 2;
        mult0 = mfr + FD;
        add0 = sdend + DD;
        pre0 = sstart + DD;
        fin = sstart + (sp.G - 1) * DD;
    } else if (mode == kChainCompose) {
        init[0] = nullptr;
        init[NR - 1] = nullptr;
        nsteps = len;
        mult0 = mfr + a * FD;
        add0 = sdend + a * DD;
        fin_frag = pfr + j * FD;
        fin = qblk + j * DD;
    } else if (mode == kChainBlocks) {
        init[0] = sdend;
        nsteps = cp.nb;
        mult0 = pfr;
        add0 = qblk;
        pre0 = sstart + DD;
        pre_stride = cp.b * DD;
        fin = sstart + (sp.G - 1) * DD;
    } else {
        init[0] = sstart + a * DD;
        nsteps = len - 1;
        mult0 = mfr + a * FD;
        add0 = sdend + a * DD;
        post0 = sstart + (a + 1) * DD;
    }

    // register sets: B fragments of the wave's column tile (hi and lo) and the
    // thread's pieces of the addend rows
    typedef u16x8 Frag[KS][2];
    typedef f32x4 Rows[SR];
    auto fetch = [&](int s, Frag& F, Rows& S) {
        const u16x8* M = mult0 + s * FD;
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) F[k][hl] = M[((nt * KS + k) * 2 + hl) * 64 + l];
        const f32x4* A = reinterpret_cast<const f32x4*>(add0 + s * DD + (int64_t)r0 * D);
#pragma unroll
        for (int k = 0; k < SR; ++k) S[k] = A[min(tid + NT * k, SP - 1)];
    };
    auto write_rows = [&](float* dst, const float* X) {
        float* SS = dst + (int64_t)r0 * D;
        for (int e = tid; e < SP; e += NT) {
            const int r = e / (D / 4), c4 = e % (D / 4);
            *reinterpret_cast<f32x4*>(&SS[r * D + 4 * c4]) = *reinterpret_cast<const f32x4*>(&X[r * LD + 4 * c4]);
        }
    };
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        for (int e = tid; e < SP; e += NT) {
            const int rr = e / (D / 4), c4 = e % (D / 4);
            f32x4 val;
            if (init[r]) {
                val = reinterpret_cast<const f32x4*>(init[r] + (int64_t)r0 * D)[e];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) val[i] = (r == 0 && r0 + rr == 4 * c4 + i) ? 1.f : 0.f;
            }
            *reinterpret_cast<f32x4*>(&Cb[0][r][rr * LD + 4 * c4]) = val;
        }
    }
    // the end values from X in Cb[c]
    auto finish = [&](int c) {
        if (fin) write_rows(fin, Cb[c][NR - 1]);
        if (fin_frag) {
            // P_j rows 16 x .. of block j as B fragments: k-step x / 2, lane
            // groups 2 (x % 2), 2 (x % 2) + 1
            if (tid < (D / 16) * 32) {
                const int ft = tid >> 5, hsel = (tid >> 4) & 1, cc = tid & 15;
                const int gg = 2 * (x & 1) + hsel, ks = x >> 1;
                f32x4 y0, y1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y0[e] = Cb[c][0][(8 * hsel + e) * LD + 16 * ft + cc];
                    y1[e] = Cb[c][0][(8 * hsel + 4 + e) * LD + 16 * ft + cc];
                }
                u16x4 h0, l0, h1, l1;
                split4(y0, h0, l0);
                split4(y1, h1, l1);
                fin_frag[((ft * KS + ks) * 2 + 0) * 64 + 16 * gg + cc] = cat(h0, h1);
                fin_frag[((ft * KS + ks) * 2 + 1) * 64 + 16 * gg + cc] = cat(l0, l1);
            }
        }
    };
    int cur = 0;
    // step s with its operands in (F, S); the operands of step s + 2 go to
    // (Fn, Sn), the set step s - 1 used; false once the chain is done
    auto step = [&](int s, const Frag& F, const Rows& S, Frag& Fn, Rows& Sn) {
        // every step issues a fetch (the last step's operands again near the
        // end), so that the waits below count the loads in flight exactly
        fetch(min(s + 2, nsteps - 1), Fn, Sn);
        if (s < nsteps) {
#pragma unroll
            for (int k = 0; k < SR; ++k) {
                const int e = tid + NT * k;
                if (SP % NT == 0 || e < SP)
                    *reinterpret_cast<f32x4*>(&SDs[s & 1][(e / (D / 4)) * LD + 4 * (e % (D / 4))]) = S[k];
            }
        }
        __syncthreads();  // X complete in Cb[cur]; Add(s) staged; Cb[cur ^ 1] and SDs[s ^ 1] free
        if (s < nsteps) {
            if (pre0) write_rows(pre0 + s * pre_stride, Cb[cur][0]);
        } else {
            finish(cur);
        }
        if (s > 0 && post0) write_rows(post0 + (s - 1) * DD, Cb[cur][0]);
        if (s == nsteps) return false;
        // Cb[cur ^ 1][r] = Cb[cur][r] Mult(s) (+ Add(s) for the last set) on
        // the wave's column tile
        u16x8 ah[NR][KS], al[NR][KS];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const float* A = Cb[cur][r];
                const f32x4 x0 = *reinterpret_cast<const f32x4*>(&A[c16 * LD + 32 * k + 8 * g4]);
                const f32x4 x1 = *reinterpret_cast<const f32x4*>(&A[c16 * LD + 32 * k + 8 * g4 + 4]);
                u16x4 h0, l0, h1, l1;
                split4(x0, h0, l0);
                split4(x1, h1, l1);
                ah[r][k] = cat(h0, h1);
                al[r][k] = cat(l0, l1);
            }
        f32x4 acc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = zero4();
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[NR - 1][i] = SDs[s & 1][(4 * g4 + i) * LD + 16 * nt + c16];
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                acc[r] = mfma(ah[r][k], F[k][0], acc[r]);
                acc[r] = mfma(ah[r][k], F[k][1], acc[r]);
                acc[r] = mfma(al[r][k], F[k][0], acc[r]);
            }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) Cb[cur ^ 1][r][(4 * g4 + i) * LD + 16 * nt + c16] = acc[r][i];
        cur ^= 1;
        return true;
    };
    Frag f0, f1, f2;
    Rows s0, s1, s2;
    if (nsteps <= 0) {  // no map: the end values are the start rows
        __syncthreads();
        finish(0);
        return;
    }
    fetch(0, f0, s0);
    fetch(min(1, nsteps - 1), f1, s1);
    for (int s = 0;; s += 3) {
        if (!step(s, f0, s0, f2, s2)) break;
        if (!step(s + 1, f1, s1, f0, s0)) break;
        if (!step(s + 2, f2, s2, f1, s1)) break;
    }
}

// pass 1: workgroup (head, segment g < G - 1, kind); pass 2: (head, segment)
// Value blocks (16 columns) per wave.  One: eight waves at D = 128, two per
// SIMD.  (Two blocks per wave read every shared A fragment once for twice the
// products, but leave one wave per SIMD and measured slower.)
template <int D>
constexpr int kSegNV = 1;
// threads per workgroup: one wave per value block; the state pass runs the S
// and the M chain of a segment in one workgroup (twice the waves, unless
// every wave carries both, see kSegPaired)
// The state pass at D = 128 pairs S^D and M in every wave (KIND 3): eight
// waves, each with the same 16 value columns of both, so that every shared A
// fragment read from LDS feeds two products (88.5 against 94.1 us on the main
// workload, with half the LDS operand traffic and two waves per SIMD instead
// of four).  At D = 64 the sixteen-wave form (KIND 2) stays faster.
template <int D>
constexpr bool kSegPaired = D == 128;
template <int D, int MODE>
constexpr int seg_threads() {
    return 64 * D / (16 * kSegNV<D>) * (MODE == kSegState && !kSegPaired<D> ? 2 : 1);
}
template <int D, int MODE>
constexpr int seg_waves_per_eu() { return seg_threads<D, MODE>() / 256 < 1 ? 1 : seg_threads<D, MODE>() / 256; }
// Stage 1 of the last segment's chunks of one head, inside the state pass
// (which has no workgroup for that segment, and whose (head, segment)
// workgroups leave compute units idle): the workgroup's two four-wave groups
// take the chunks two at a time, each in its own part of the LDS; a group
// with no chunk left in the last pair repeats the last chunk, storing nothing.
template <int D>
__device__ __forceinline__ void prep_last_segment(const Problem& p, const Split& sp, u16x8* tfrag, float* gates,
                                                  int64_t head, SegShared<D, kSegState>& sh) {
    static_assert(seg_threads<D, kSegState>() == 2 * kThreads, "two four-wave groups");
    static_assert(2 * sizeof(PrepScalarShared) <= sizeof(SegShared<D, kSegState>), "two stage-1 tiles fit");
    const int grp = threadIdx.x / kThreads, tid = threadIdx.x % kThreads;
    PrepScalarShared& ps = reinterpret_cast<PrepScalarShared*>(&sh)[grp];
    const int b = (int)(head / p.H), h = (int)(head % p.H);
    const int i0 = (sp.G - 1) * sp.per;
    for (int i = i0; i < p.NC; i += 2) {
        if (i > i0) __syncthreads();  // the previous pair's LDS reads are done
        const int ic = i + grp;
        prep_scalar_chunk<D>(p, tfrag, gates, min(ic, p.NC - 1), h, b, ps, tid, ic < p.NC);
    }
}

template <int D, int MODE>
__global__ __launch_bounds__((seg_threads<D, MODE>()), (seg_waves_per_eu<D, MODE>())) void k_seg(
    Problem p, Split sp, WsLayout L, char* wsb, u16x8* tfrag, float* gates) {
    constexpr int NV = kSegNV<D>;
    __shared__ __attribute__((aligned(16))) SegShared<D, MODE> sh;
    if constexpr (MODE == kSegOut) {
        const int id = blockIdx.x;
        seg_body<D, MODE, 0, NV>(p, sp, L, wsb, tfrag, gates, id / sp.G, id % sp.G, sh);
    } else {
        // workgroup (head, segment g < G - 1), then one per head for stage 1
        // of the last segment
        const int nseg = sp.G - 1;
        const int64_t nstate = p.B * p.H * (int64_t)nseg;
        if ((int64_t)blockIdx.x >= nstate) {
            prep_last_segment<D>(p, sp, tfrag, gates, (int64_t)blockIdx.x - nstate, sh);
            return;
        }
        if constexpr (kSegPaired<D>)
            seg_body<D, MODE, 3, 2>(p, sp, L, wsb, tfrag, gates, blockIdx.x / nseg, blockIdx.x % nseg, sh);
        else
            seg_body<D, MODE, 2, NV>(p, sp, L, wsb, tfrag, gates, blockIdx.x / nseg, blockIdx.x % nseg, sh);
    }
}

// ---------------------------------------------------------------------------
// sequence parallel: output correction O_i += R_i S_start(g)^T
// ---------------------------------------------------------------------------
// Computed transposed, O^T[v][t] += sum_a S_start[v][a] R[t][a]: the start
// state is the A operand (pre-split fragments written by the chain kernel),
// R the B operand (rows of R are contiguous in a).  One workgroup takes a run
// of kCorrChunks chunks of one segment; wave (tn, half) covers token tile tn
// and half of the value tiles, whose start-state fragments it keeps in
// registers for the whole run.
constexpr int kCorrChunks = 16;

template <int D>
__global__ __launch_bounds__(512) void k_correct_mfma(Problem p, Split sp, WsLayout L, char* wsb,
                                                      int runs) {
    constexpr int KS = D / 32;
    constexpr int NVT = D / 16;
    constexpr int VPW = NVT / 2;  // value tiles per wave
    const int seg = 1 + blockIdx.x / runs, run = blockIdx.x % runs;
    const int h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int tn = w & 3, vh = w >> 2;
    const int64_t H = p.H, T = p.T, bh = (int64_t)b * H + h;
    const int i0 = seg * sp.per + run * kCorrChunks;
    const int i1 = min(min(p.NC, (seg + 1) * sp.per), i0 + kCorrChunks);
    if (i0 >= i1) return;
    const u16x8* fr = reinterpret_cast<const u16x8*>(wsb + L.sfrag) + (bh * sp.G + seg) * (int64_t)NVT * KS * 2 * 64 + l;
    u16x8 ah[VPW][KS], al[VPW][KS];
#pragma unroll
    for (int q = 0; q < VPW; ++q)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int vn = vh * VPW + q;
            ah[q][s] = fr[((vn * KS + s) * 2 + 0) * 64];
            al[q][s] = fr[((vn * KS + s) * 2 + 1) * 64];
        }
    // R rows t = 16 tn + c16, columns 32s + 8 g4 .. +7, one chunk ahead
    f32x4 rx[KS], ry[KS];
    auto load_r = [&](int i) {
        i = min(i, i1 - 1);
        const float* R = reinterpret_cast<const float*>(wsb + L.corr) + (bh * p.NC + i) * C * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const float* src = R + (int64_t)(16 * tn + c16) * D + 32 * s + 8 * g4;
            rx[s] = *reinterpret_cast<const f32x4*>(src);
            ry[s] = *reinterpret_cast<const f32x4*>(src + 4);
        }
    };
    // O values of the wave's tiles (column t, rows 16 vn + 4 g4 ..), one chunk
    // ahead too; rows past the sequence end read its last row and are not stored
    const int t = 16 * tn + c16;
    f32x4 ov[VPW];
    auto load_o = [&](int i) {
        i = min(i, i1 - 1);
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
        const float* o = p.out + ((b * T + t0 + min(t, nt - 1)) * H + h) * D + 4 * g4;
#pragma unroll
        for (int q = 0; q < VPW; ++q) ov[q] = *reinterpret_cast<const f32x4*>(o + 16 * (vh * VPW + q));
    };
    load_r(i0);
    load_o(i0);
    for (int i = i0; i < i1; ++i) {
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
        f32x4 oc[VPW];
#pragma unroll
        for (int q = 0; q < VPW; ++q) oc[q] = ov[q];
        // B operands from R, split hi/lo
        u16x8 rh[KS], rl[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const f32x4 x = rx[s], y = ry[s];
            uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
            split2(x[0], x[1], h0, l0);
            split2(x[2], x[3], h1, l1);
            split2(y[0], y[1], h2, l2);
            split2(y[2], y[3], h3, l3);
            rh[s] = __builtin_bit_cast(u16x8, uint4{h0, h1, h2, h3});
            rl[s] = __builtin_bit_cast(u16x8, uint4{l0, l1, l2, l3});
        }
        load_r(i + 1);
        load_o(i + 1);
#pragma unroll
        for (int q = 0; q < VPW; ++q) {
            f32x4 a1 = zero4(), a2 = zero4(), a3 = zero4();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                a1 = mfma(ah[q][s], rh[s], a1);
                a2 = mfma(ah[q][s], rl[s], a2);
                a3 = mfma(al[q][s], rh[s], a3);
            }
            // accumulator: column t, rows v = 16 vn + 4 g4 + r
            if (t < nt) {
                float* o = p.out + ((b * T + t0 + t) * H + h) * D + 16 * (vh * VPW + q) + 4 * g4;
                *reinterpret_cast<f32x4*>(o) = oc[q] + a1 + a2 + a3;
            }
        }
    }
}

template <int D, int CH>
hipError_t launch(const Problem& p, const Split& sp, char* ws, const WsLayout& L, hipStream_t st) {
    u16x8* tfrag = reinterpret_cast<u16x8*>(ws + L.prep);
    const int64_t nch = p.B * p.H * (int64_t)p.NC;
    const size_t fbytes = align256((size_t)nch * kTfragPerChunk * sizeof(u16x8));
    // P fragments: channel gates only (the scalar-gate loop forms P itself)
    u16x8* pfrag = CH ? reinterpret_cast<u16x8*>(ws + L.prep + fbytes) : nullptr;
    float* gates = reinterpret_cast<float*>(ws + L.prep + (CH ? 2 : 1) * fbytes);
    {
        dim3 grid(p.NC, (unsigned)p.H, (unsigned)p.B);
        prof_begin(p.timer, "k_prep_mfma", st);
        if constexpr (CH)
            hipLaunchKernelGGL((k_prep_channel<D>), grid, dim3(kThreads), 0, st, p, tfrag, pfrag, gates);
        else
            hipLaunchKernelGGL((k_prep_scalar<D>), grid, dim3(kThreads), 0, st, p, tfrag, gates);
        prof_end(p.timer, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        const int ntiles = D / 16 + (sp.G > 1 ? D / 16 : 0);
        const int64_t heads = p.B * p.H * sp.G;
        const int64_t nwork = heads * ntiles;
        const int remap = (heads % 8 == 0) ? 1 : 0;
        prof_begin(p.timer, "k_rec_mfma", st);
        hipLaunchKernelGGL((k_rec_mfma<D, CH>), dim3((unsigned)nwork), dim3(kRecThreads), 0, st, p, sp, L,
                           ws, tfrag, pfrag, gates, ntiles, remap);
        prof_end(p.timer, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (sp.G > 1) return seqpar_finish(p, sp, ws, L, true, st);
    return hipSuccess;
}

// Channel gate with enough heads: stage 1, then the head-shared chunk loop
// (two workgroups per head, one pass).
template <int D>
hipError_t launch_chan(const Problem& p, char* ws, const WsLayout& L, hipStream_t st) {
    u16x8* tfrag = reinterpret_cast<u16x8*>(ws + L.prep);
    const int64_t nch = p.B * p.H * (int64_t)p.NC;
    const size_t fbytes = align256((size_t)nch * kTfragPerChunk * sizeof(u16x8));
    u16x8* pfrag = reinterpret_cast<u16x8*>(ws + L.prep + fbytes);
    float* gates = reinterpret_cast<float*>(ws + L.prep + 2 * fbytes);
    if (p.NC > 0) {
        dim3 grid(p.NC, (unsigned)p.H, (unsigned)p.B);
        prof_begin(p.timer, "k_prep_mfma", st);
        hipLaunchKernelGGL((k_prep_channel<D>), grid, dim3(kThreads), 0, st, p, tfrag, pfrag, gates);
        prof_end(p.timer, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t heads = p.B * p.H;
    const int remap = heads % 8 == 0 ? 1 : 0;
    prof_begin(p.timer, "k_chan_head", st);
    if (p.raw)
        hipLaunchKernelGGL((k_chan_head<D, true>), dim3((unsigned)(2 * heads)), dim3(chan_threads<D>()), 0, st, p,
                           tfrag, pfrag, gates, remap);
    else
        hipLaunchKernelGGL((k_chan_head<D, false>), dim3((unsigned)(2 * heads)), dim3(chan_threads<D>()), 0, st, p,
                           tfrag, pfrag, gates, remap);
    prof_end(p.timer, st);
    return hipGetLastError();
}

// Scalar gate: stage 1, then the whole-head chunk loop (two passes and the
// start-state chain when the sequence is cut into segments).
template <int D>
hipError_t launch_seg(const Problem& p, const Split& sp, char* ws, const WsLayout& L, hipStream_t st) {
    u16x8* tfrag = reinterpret_cast<u16x8*>(ws + L.prep);
    const int64_t nch = p.B * p.H * (int64_t)p.NC;
    const size_t fbytes = align256((size_t)nch * kTfragPerChunk * sizeof(u16x8));
    float* gates = reinterpret_cast<float*>(ws + L.prep + fbytes);
    // With segments, stage 1 of the last segment's chunks runs inside the
    // state pass (which does not read them), on its extra workgroups.
    const int64_t first_end = (int64_t)(sp.G - 1) * sp.per;
    const int nc_first = sp.G > 1 && first_end < p.NC ? (int)first_end : p.NC;
    if (nc_first > 0) {
        dim3 grid(nc_first, (unsigned)p.H, (unsigned)p.B);
        prof_begin(p.timer, "k_prep_mfma", st);
        hipLaunchKernelGGL((k_prep_scalar<D>), grid, dim3(kThreads), 0, st, p, tfrag, gates);
        prof_end(p.timer, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t heads = p.B * p.H;
    if (sp.G > 1) {
        prof_begin(p.timer, "k_seg_state", st);
        hipLaunchKernelGGL((k_seg<D, kSegState>), dim3((unsigned)(heads * sp.G)), dim3(seg_threads<D, kSegState>()), 0, st,
                           p, sp, L, ws, tfrag, gates);
        prof_end(p.timer, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const ChainPlan cp = chain_plan(sp.G, heads, D);
        const unsigned nx = D / 16;
        prof_begin(p.timer, "k_chain", st);
        if (cp.nb == 0) {
            hipLaunchKernelGGL((k_chain_rows<D, 1>), dim3((unsigned)(heads * nx)), dim3(chain_threads<D>()), 0, st, p, sp,
                               L, ws, (int)kChainSeq, cp);
        } else {
            hipLaunchKernelGGL((k_chain_rows<D, 2>), dim3((unsigned)(heads * cp.nb * nx)), dim3(chain_threads<D>()), 0,
                               st, p, sp, L, ws, (int)kChainCompose, cp);
            hipLaunchKernelGGL((k_chain_rows<D, 1>), dim3((unsigned)(heads * nx)), dim3(chain_threads<D>()), 0, st, p, sp,
                               L, ws, (int)kChainBlocks, cp);
            hipLaunchKernelGGL((k_chain_rows<D, 1>), dim3((unsigned)(heads * cp.nb * nx)), dim3(chain_threads<D>()), 0,
                               st, p, sp, L, ws, (int)kChainExpand, cp);
        }
        prof_end(p.timer, st);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    prof_begin(p.timer, "k_seg_out", st);
    hipLaunchKernelGGL((k_seg<D, kSegOut>), dim3((unsigned)(heads * sp.G)), dim3(seg_threads<D, kSegOut>()), 0, st, p, sp, L, ws,
                       tfrag, gates);
    prof_end(p.timer, st);
    return hipGetLastError();
}

}  // namespace

// The whole-head chunk loop (scalar gate) needs enough (head, segment)
// workgroups to occupy the device; below that the state is sliced over
// 16-column workgroups (k_rec_mfma), eight per head.
constexpr int64_t kWholeHeadMinGroups = 128;
static bool whole_head(const Problem& p, const Split& sp) {
    return p.gate == GDN_GATE_SCALAR && p.B * p.H * (int64_t)sp.G >= kWholeHeadMinGroups;
}
// The channel gate's head-shared loop (two workgroups per head, one pass) at
// dk = 128 once there are enough heads; the sliced loop otherwise and for
// segmented runs.
constexpr int64_t kChanHeadMinHeads = 64;
static bool chan_head(const Problem& p, const Split& sp) {
    return p.gate == GDN_GATE_CHANNEL && p.dk == 128 && sp.G == 1 && p.B * p.H >= kChanHeadMinHeads;
}

bool mfma_supported(int64_t dk, int64_t dv, int C_, int dtype, int gate) {
    return dtype == GDN_BF16 && (gate == GDN_GATE_SCALAR || gate == GDN_GATE_CHANNEL) &&
           C_ == C && dk == dv && (dk == 64 || dk == 128);
}

WsLayout mfma_layout(const Problem& p, const Split& sp) {
    WsLayout L;
    const int64_t nch = p.B * p.H * (int64_t)p.NC;
    L.prep = 0;
    const size_t gate_floats = p.gate == GDN_GATE_CHANNEL ? (size_t)C * p.dk + 2 * C : kGateFloats;
    L.prep_bytes = (p.gate == GDN_GATE_CHANNEL ? 2 : 1) * align256((size_t)nch * kTfragPerChunk * sizeof(u16x8)) +
                   align256((size_t)nch * gate_floats * sizeof(float));
    size_t off = L.prep_bytes;
    // the whole-head path keeps no per-chunk corrections and no start-state
    // fragments
    const bool whole = whole_head(p, sp);
    if (sp.G > 1) {
        L.corr = off;
        L.corr_bytes = whole ? 0 : align256(sizeof(float) * nch * p.C * p.dk);
        off += L.corr_bytes;
        L.sdend = off;
        L.sdend_bytes = align256(sizeof(float) * p.B * p.H * sp.G * p.dv * p.dk);
        off += L.sdend_bytes;
        L.mend = off;
        L.mend_bytes = align256(sizeof(float) * p.B * p.H * sp.G * p.dk * p.dk);
        off += L.mend_bytes;
        L.sstart = off;
        L.sstart_bytes = align256(sizeof(float) * p.B * p.H * sp.G * p.dv * p.dk);
        off += L.sstart_bytes;
        L.sfrag = off;
        L.sfrag_bytes = whole ? 0 : align256(2 * sizeof(uint16_t) * p.B * p.H * sp.G * p.dv * p.dk);
        off += L.sfrag_bytes;
        // the blocked start-state chain keeps a composed map pair per block
        const ChainPlan cp = whole ? chain_plan(sp.G, p.B * p.H, (int)p.dk) : ChainPlan{0, 0};
        L.blk = off;
        L.blk_bytes = align256(2 * sizeof(float) * p.B * p.H * cp.nb * p.dk * p.dk);
        off += L.blk_bytes;
    }
    L.total = off;
    return L;
}

hipError_t mfma_correct(const Problem& p, const Split& sp, char* ws, const WsLayout& L,
                        hipStream_t st) {
    const int runs = (sp.per + kCorrChunks - 1) / kCorrChunks;  // runs of chunks per segment
    dim3 grid((unsigned)((sp.G - 1) * runs), (unsigned)p.H, (unsigned)p.B);
    prof_begin(p.timer, "k_correct_mfma", st);
    if (p.dk == 128)
        hipLaunchKernelGGL(k_correct_mfma<128>, grid, dim3(512), 0, st, p, sp, L, ws, runs);
    else
        hipLaunchKernelGGL(k_correct_mfma<64>, grid, dim3(512), 0, st, p, sp, L, ws, runs);
    prof_end(p.timer, st);
    return hipGetLastError();
}

hipError_t mfma_forward(const Problem& p, const Split& sp, char* ws, hipStream_t st) {
    const WsLayout L = mfma_layout(p, sp);
    const bool ch = p.gate == GDN_GATE_CHANNEL;
    if (whole_head(p, sp)) return p.dk == 128 ? launch_seg<128>(p, sp, ws, L, st) : launch_seg<64>(p, sp, ws, L, st);
    if (chan_head(p, sp)) return launch_chan<128>(p, ws, L, st);
    if (p.dk == 128) return ch ? launch<128, 1>(p, sp, ws, L, st) : launch<128, 0>(p, sp, ws, L, st);
    return ch ? launch<64, 1>(p, sp, ws, L, st) : launch<64, 0>(p, sp, ws, L, st);
}

// Segments for an explicit request of G: when (batch, head, segment) groups
// are too few for the whole-head loop, each segment is cut into k equal runs
// (k G segments in all, about kTargetGroups groups, at least kMinSegChunks
// chunks each), so that the whole-head loop, whose correction is fused with
// the outputs, takes it; a request that cannot reach kWholeHeadMinGroups so
// stays as it is (the sliced loop).
int mfma_refine_segments(const Problem& p, int G) {
    constexpr int64_t kTargetGroups = 256;
    constexpr int kMinSegChunks = 4;
    if (G <= 1 || !mfma_supported(p.dk, p.dv, p.C, p.dtype, p.gate) || p.gate != GDN_GATE_SCALAR) return G;
    const Split sp = make_split(p.NC, G);
    const int64_t heads = p.B * p.H;
    if (heads <= 0 || whole_head(p, sp)) return G;
    int64_t k = (kTargetGroups + heads * sp.G - 1) / (heads * sp.G);
    const int64_t kmax = p.NC / ((int64_t)kMinSegChunks * sp.G);
    if (k > kmax) k = kmax;
    if (k < 2) return G;
    const Split fine = make_split(p.NC, (int)(k * sp.G));
    return whole_head(p, fine) ? fine.G : G;
}

int mfma_auto_segments(const Problem& p) {
    constexpr int kTargetGroups = 256;  // compute units of a gfx950 device
    constexpr int kMinSegChunks = 4;
    if (!mfma_supported(p.dk, p.dv, p.C, p.dtype, p.gate) || p.gate != GDN_GATE_SCALAR) return 1;
    const int64_t heads = p.B * p.H;
    if (heads <= 0 || p.NC <= 0) return 1;
    int64_t g = (kTargetGroups + heads - 1) / heads;
    const int64_t cap = p.NC / kMinSegChunks;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    // too few workgroups for the whole-head loop: one stream on the sliced loop
    return whole_head(p, make_split(p.NC, (int)g)) ? (int)g : 1;
}

}  // namespace gdn
