// Chunked backward of the gated delta rule (gdn_backward with a scalar gate,
// dk = dv = D in {64, 128}; the channel gate and other shapes take the token
// kernel of gdn_bwd.hip).
//
// The pages fix the forward only (the DeltaNet illustrated notes, WY/UT
// section: UT transform, chunk state passing, output; the scalar gate of the
// Gated DeltaNet paragraph); these are the chain rule through its chunk
// form.  Per chunk of C = 64 tokens with entry state S (dv x dk), chunk-local
// log-gate prefix l_t (gamma_t = e^{l_t}), prediction prefix l'_t (l_{t-1}
// predict-then-decay, l_t decay-then-predict), R_t = e^{l_{C-1} - l_t}:
//   A_tj = beta_t e^{l'_t - l_j} k_t.k_j (j < t),  T = (I + A)^{-1}
//   X = K S^T,  U = V - diag(gamma') X,  Delta = T diag(beta) U
//   O = scale (diag(gamma) Q S^T + P Delta),  P_tj = e^{l_t - l_j} q_t.k_j (j <= t)
//   S_end = gamma_{C-1} S + Delta^T diag(R) K
// and, with dO and dS_end given:
//   dDelta = scale P^T dO + diag(R) K dS_end^T,  dU' = T^T dDelta,  dV = diag(beta) dU'
//   dS = gamma_{C-1} dS_end + scale dO^T diag(gamma) Q - dU'^T diag(gamma' beta) K
//   dP = scale dO Delta^T (j <= t),  dT = dDelta U^T diag(beta),  dA = -T^T dT T^T (j < t)
//   dQ = scale diag(gamma) dO S + (dP o M) K,         M_tj = e^{l_t - l_j}
//   dK = (dP o M)^T Q - diag(gamma' beta) dU' S + diag(R) Delta dS_end + (W + W^T) K,
//        W_tj = beta_t dA_tj e^{l'_t - l_j}
//   dbeta_t = dU'_t . U_t + sum_j dA_tj Atilde_tj,     Atilde = A / beta
// The gate gradient is taken pair by pair: every product of gates above is a
// ratio e^{l_b - l_a} over the tokens a < s <= b (a = -1: from the chunk
// start), whose derivative in log alpha_s is the term itself, so
//   dlog alpha_s = sum over terms whose range holds s   (dalpha_s = that / alpha_s),
// summed as a two-dimensional prefix over a matrix V[b][a + 1] of the terms
// (pair terms dP o P, dA o A at their ranges; the boundary terms q_t.dQ_S0,
// k_t.dK_S0, gamma_{C-1} <dS_end, S> and k_j.dK_dS at theirs, the last two
// formed from the S and dS_end parts of dQ and dK).  Every addend of a sum
// for s then carries the factor alpha_s, so the division loses nothing
// where a gate is small.  l is kept as a compensated pair (hi + lo, each
// step of the prefix an error-free addition), so every ratio's exponent
// (hi_b - hi_a) + (lo_b - lo_a) is accurate to the fp32 rounding of its own
// value, not of the prefix.
//
// Three kernels, all fp32 MFMA (16 x 16 x 4, the layout of gdn_mfma_common.h;
// bf16 inputs are exact in fp32), fp32 accumulation:
//   k_bprep, one workgroup per chunk: gate prefix, Gram K K^T and Q K^T, A,
//     T by the in-LDS UT inverse; T, T^T and P^T in the workspace, with K
//     and Q as transposed fragments (K[16 tb + 4 g + q][16 m + c] per lane).
//   k_bchain, one workgroup per (head, one or two 16-row slices of the
//     state) and direction: the forward chain carries S over the chunks and stores each
//     chunk's entry state, U and Delta; the reverse chain carries dS back and
//     stores each chunk's dS_end, dDelta and dU' and writes dv and dS_0.  Rows
//     of the state are independent given T, K and the gates, so a slice holds
//     its 16 rows in registers; wave w owns key tiles of it, the token tiles
//     of the chunk products are dealt over the waves and exchanged in LDS.
//   k_bgrad, one workgroup per chunk: everything else from the stored pieces.
#include <type_traits>

#include "gdn_internal.h"
#include "gdn_mfma_common.h"
#include "../../include/gdn.h"

namespace gdn {
namespace {

constexpr int LDA = C + 4;  // row stride of C x C fp32 tiles in LDS

// acc += A B over a 16 x 16 x 16 block: a = A[c][4g .. 4g + 3] (the lane's
// row c, four consecutive contraction indices), b = B[4g .. 4g + 3][c].  An
// accumulator tile of M serves as b for M as it stands; one of M^T as a.
__device__ __forceinline__ f32x4 blk(const f32x4& a, const f32x4& b, f32x4 acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = mfma_f32(a[q], b[q], acc);
    return acc;
}

// four consecutive input-typed elements (q, k and their fragments: 8 bytes
// bf16 or 16 bytes fp32), kept as loaded until used
template <int DT>
using R4 = std::conditional_t<DT == GDN_BF16, u32x2, f32x4>;
template <int DT>
using InE = std::conditional_t<DT == GDN_BF16, uint16_t, float>;
template <int DT>
__device__ __forceinline__ R4<DT> ldr(const void* base, int64_t i) {
    return *reinterpret_cast<const R4<DT>*>(static_cast<const InE<DT>*>(base) + i);
}
template <int DT>
__device__ __forceinline__ f32x4 cvt(const R4<DT>& u) {
    if constexpr (DT == GDN_BF16) {
        return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xFFFF0000u),
                     __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xFFFF0000u)};
    } else {
        return u;
    }
}
template <int DT>
__device__ __forceinline__ f32x4 ld4in(const void* base, int64_t i) {
    return cvt<DT>(ldr<DT>(base, i));
}
// eight consecutive input-typed elements (16 bytes bf16, 32 bytes fp32)
template <int DT>
struct R8 {
    R4<DT> h[2];
};
template <int DT>
__device__ __forceinline__ R8<DT> ldr8(const void* base, int64_t i) {
    R8<DT> x;
    if constexpr (DT == GDN_BF16) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + i);
        x.h[0] = u32x2{u[0], u[1]};
        x.h[1] = u32x2{u[2], u[3]};
    } else {
        x.h[0] = ldr<DT>(base, i);
        x.h[1] = ldr<DT>(base, i + 4);
    }
    return x;
}

// Key (dk) index of row i (0..15) of key tile mi (of MT = D / 64) of wave w.
// A wave's tiles interleave in runs of four, so that a lane's rows of all of
// them are 4 MT consecutive keys and come in one load; every tiling of the
// key axis below (state tiles, K^T and Q^T fragments, the gradient kernel's
// output columns) uses this order.  Column block db of the whole axis is
// tile db % MT of wave db / MT.
template <int D>
__device__ __forceinline__ int key_of(int w, int mi, int i) {
    return (D / 4) * w + 4 * (D / 64) * (i >> 2) + 4 * mi + (i & 3);
}
template <int D>
__device__ __forceinline__ int key_col(int db, int i) {
    return key_of<D>(db / (D / 64), db % (D / 64), i);
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ float dot4(const f32x4& x, const f32x4& y) {
    return x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
}
// lower block (m, nb), nb <= m, of the 10 of a C x C tile, by index
__device__ __forceinline__ int blk_m(int i) { return i >= 6 ? 3 : i >= 3 ? 2 : i >= 1 ? 1 : 0; }
__device__ __forceinline__ int blk_n(int i) { const int m = blk_m(i); return i - m * (m + 1) / 2; }
__device__ __forceinline__ void st4f(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }

__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// Chunk gates on one wave (lane t = token t of the chunk; past the sequence
// end alpha = 1, beta = 0): the log-gate prefix as hi + lo, the prediction
// prefix, beta and alpha.
struct Gate {
    float hi, lo, phi, plo, beta, alpha;
};
__device__ __forceinline__ Gate gate_from(float alpha, float beta, int nt, int order, int lane) {
    Gate g;
    g.alpha = lane < nt ? alpha : 1.f;
    g.beta = lane < nt ? beta : 0.f;
    float hi = lane < nt ? logf(g.alpha) : 0.f, lo = 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float h2 = __shfl_up(hi, o, 64), l2 = __shfl_up(lo, o, 64);
        if (lane >= o) {
            float s, e;
            two_sum(hi, h2, s, e);
            hi = s;
            lo = (lo + l2) + e;
        }
    }
    g.hi = hi;
    g.lo = lo;
    if (order == GDN_PREDICT_THEN_DECAY) {
        g.phi = __shfl_up(hi, 1, 64);
        g.plo = __shfl_up(lo, 1, 64);
        if (lane == 0) g.phi = g.plo = 0.f;
    } else {
        g.phi = hi;
        g.plo = lo;
    }
    return g;
}
// (token rows past the sequence end are read at the last real row and
// replaced by the defaults)
__device__ __forceinline__ Gate chunk_gate(const Problem& p, int64_t row0, int nt, int lane) {
    const int64_t r = row0 + (int64_t)min(lane, nt - 1) * p.H;
    return gate_from(p.alpha[r], p.beta[r], nt, p.order, lane);
}

// Rows of a chunk's token factors (lane t: token t): the gate prefix pair,
// the prediction prefix pair, beta, gamma_t, gamma'_t and R_t = gamma_C / gamma_t.
enum { kGhi, kGlo, kGphi, kGplo, kGbeta, kGgam, kGgamp, kGR };

// e^{(hb - ha) + (lb - la)}
__device__ __forceinline__ float ratio(float hb, float lb, float ha, float la) {
    return __expf((hb - ha) + (lb - la));
}

// Per-chunk records of the workspace.  Fragment sets: [m][tp][lane][8] =
// X[16 (2 tp + e) + 4 g + q][key_col(m, c)] (e = 0, 1; q = 0..3) for X = K,
// Q; state fragments [vb][db][lane] of f32x4 = S[16 vb + 4 g + q][key_col(db, c)].
template <int D>
struct Rec {
    static constexpr int NB = D / 16;
    static constexpr size_t kTile = (size_t)C * C;          // T, T^T, P^T, Atilde^T (floats)
    static constexpr size_t kFrag = (size_t)NB * 4 * 64 * 4;  // K^T, Q^T fragments
    static constexpr size_t kState = (size_t)NB * NB * 64 * 4;
    static constexpr size_t kRows = (size_t)C * D;          // U, Delta, dDelta, dU'; E fragments
    static constexpr size_t kHf = (size_t)D * D;            // H fragments
    static constexpr size_t kGr = 8 * (size_t)C;            // gate rows
};

struct CbWs {
    float *T, *TT, *PT, *AtT;  // [chunk][C][C]
    void *KTf, *QTf;           // [chunk][fragment set], input-typed
    float *Sf, *dSf;           // [chunk][state fragments]
    float *U, *Dl, *dDl, *dUp; // [chunk][C][D]
    float *Ef, *Hf;            // [chunk][vb][jb or m][lane] of f32x4: E = scale P^T dO,
                               // H = scale Q^T diag(gamma) dO as accumulator tiles
    float* Gr;                 // [chunk][8][C]: the chunk's gate rows (kG*)
};

// ---------------------------------------------------------------------------
// k_bprep: per chunk T, T^T, P^T, Atilde^T, the K^T and Q^T fragments, and
// the reverse chain's state-independent terms E = scale P^T dO and
// H = scale Q^T diag(gamma) dO as accumulator tiles
// ---------------------------------------------------------------------------
// Work of wave w: the Gram row block m = w (tiles (w, nb), nb <= w) and the
// Q K^T column block jb = w (tiles (tb, w), tb >= w), five tiles either way;
// the P tiles it holds are the A operands of E's block row w as they stand
// (a lane holds P[16 tb + 4 g + r][16 w + c] = P^T[16 w + c][16 tb + 4 g + r]).
// LDS: the K and Q rows, later dL/d out over them; the UT system.  With
// bf16 inputs the K rows sit in the UT tile itself (A goes there once the
// Gram products are done) and dL/d out comes in two column halves, which
// keeps the workgroup at 36 KiB, four per compute unit.
template <int D, int DT>
__global__ __launch_bounds__(kThreads, DT == GDN_BF16 ? 4 : 2) void k_bprep(BwdProblem a, CbWs ws) {
    using E = std::conditional_t<DT == GDN_BF16, uint16_t, float>;
    constexpr int NB = D / 16, MT = D / 64;
    constexpr int LDK = D + (DT == GDN_BF16 ? 8 : 4);
    constexpr bool KIN = DT == GDN_BF16;  // K rows in the UT tile
    constexpr int NH = KIN ? 2 : 1;       // column parts of dL/d out
    constexpr int DH = D / NH;
    constexpr int LDD = DH + 4;
    constexpr int EP = 16 / sizeof(E);  // elements per 16-byte piece
    constexpr int PPR = D / EP;         // pieces per row
    constexpr int KQB = (KIN ? 1 : 2) * C * LDK * (int)sizeof(E);
    static_assert(C * LDD * 4 <= KQB, "dL/d out fits over the Q (and K) rows");
    static_assert(!KIN || C * LDK * (int)sizeof(E) <= C * LDA * 4, "K rows fit the UT tile");
    __shared__ __attribute__((aligned(16))) float AT[C * LDA];
    __shared__ __attribute__((aligned(16))) unsigned char kq[KQB];
    __shared__ __attribute__((aligned(16))) float ghi[C], glo[C], gphi[C], gplo[C], gbeta[C], ggam[C];
    E* Ks = KIN ? reinterpret_cast<E*>(AT) : reinterpret_cast<E*>(kq);
    E* Qs = KIN ? reinterpret_cast<E*>(kq) : Ks + C * LDK;
    float* dOs = reinterpret_cast<float*>(kq);

    const Problem& p = a.p;
    const int64_t ci = blockIdx.x;
    const int64_t bl = ci / p.NC;
    const int c = (int)(ci - bl * p.NC);
    const int64_t bh = a.bh0 + bl, b = bh / p.H, h = bh - b * p.H;
    const int64_t t0 = (int64_t)c * C;
    const int nt = (int)min<int64_t>(C, p.T - t0);
    const int64_t row0 = (b * p.T + t0) * p.H + h;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g4 = l >> 4, c16 = l & 15;

    // K and Q rows into LDS (rows past the sequence end zero)
    constexpr int KP = C * PPR / kThreads;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        const int e = tid + kThreads * i, t = e / PPR, pc = e % PPR;
        const int64_t src = (row0 + (int64_t)min(t, nt - 1) * p.H) * D + pc * EP;
        u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(p.k) + src);
        u32x4 qv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(p.q) + src);
        if (t >= nt) kv = qv = u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(&Ks[t * LDK + pc * EP]) = kv;
        *reinterpret_cast<u32x4*>(&Qs[t * LDK + pc * EP]) = qv;
    }
    if (w == 0) {
        const Gate g = chunk_gate(p, row0, nt, l);
        ghi[l] = g.hi;
        glo[l] = g.lo;
        gphi[l] = g.phi;
        gplo[l] = g.plo;
        gbeta[l] = g.beta;
        ggam[l] = __expf(g.hi + g.lo);
        // the chain kernel's gate rows
        const float hC = __shfl(g.hi, C - 1, 64), lC = __shfl(g.lo, C - 1, 64);
        float* gr = ws.Gr + ci * Rec<D>::kGr;
        gr[kGhi * C + l] = g.hi;
        gr[kGlo * C + l] = g.lo;
        gr[kGphi * C + l] = g.phi;
        gr[kGplo * C + l] = g.plo;
        gr[kGbeta * C + l] = g.beta;
        gr[kGgam * C + l] = __expf(g.hi + g.lo);
        gr[kGgamp * C + l] = __expf(g.phi + g.plo);
        gr[kGR * C + l] = ratio(hC, lC, g.hi, g.lo);
    }
    __syncthreads();

    auto row4 = [&](const E* X, int t, int d0) -> f32x4 {
        if constexpr (DT == GDN_BF16) return ld4in<DT>(X, t * LDK + d0);
        else return ld4f(X + t * LDK + d0);
    };
    // Gram row block m = w: A_tj = beta_t Atilde_tj, Atilde_tj = e^{l'_t - l_j}
    // k_t.k_j (j < t), Atilde^T[j][t] to the workspace; A goes to the tile in
    // the inverse's layout once the K rows are dead (tiles nb <= w kept)
    f32x4 av[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        av[nb] = zero4();
        if (nb > w) continue;
        const int m = w;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
            acc = blk(row4(Ks, 16 * m + c16, 16 * kb + 4 * g4), row4(Ks, 16 * nb + c16, 16 * kb + 4 * g4), acc);
        const int j = 16 * nb + c16;
        f32x4 tv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * m + 4 * g4 + r;
            tv[r] = j < t ? ratio(gphi[t], gplo[t], ghi[j], glo[j]) * acc[r] : 0.f;
            av[nb][r] = gbeta[t] * tv[r];
        }
        st4f(ws.AtT + ci * Rec<D>::kTile + j * C + 16 * m + 4 * g4, tv);
    }
    // Q K^T column block jb = w: P_tj = e^{l_t - l_j} q_t.k_j (j <= t), kept
    // (pk[tb], tb >= w) and stored as P^T[j][t]
    f32x4 pk[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        pk[tb] = zero4();
        if (tb < w) continue;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
            acc = blk(row4(Qs, 16 * tb + c16, 16 * kb + 4 * g4), row4(Ks, 16 * w + c16, 16 * kb + 4 * g4), acc);
        const int j = 16 * w + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * g4 + r;
            pk[tb][r] = j <= t ? ratio(ghi[t], glo[t], ghi[j], glo[j]) * acc[r] : 0.f;
        }
        st4f(ws.PT + ci * Rec<D>::kTile + j * C + 16 * tb + 4 * g4, pk[tb]);
    }
    // K^T and Q^T fragments (input-typed), two token blocks a lane
    for (int f = tid; f < NB * 2 * 64; f += kThreads) {
        const int ln = f & 63, mt = f >> 6, m = mt >> 1, tp = mt & 1;
        const int gg = ln >> 4, d = key_col<D>(m, ln & 15);
        E kx[8], qx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 16 * (2 * tp + (e >> 2)) + 4 * gg + (e & 3);
            kx[e] = Ks[t * LDK + d];
            qx[e] = Qs[t * LDK + d];
        }
        E* kd = static_cast<E*>(ws.KTf) + ci * Rec<D>::kFrag + (size_t)f * 8;
        E* qd = static_cast<E*>(ws.QTf) + ci * Rec<D>::kFrag + (size_t)f * 8;
        if constexpr (DT == GDN_BF16) {
            u16x8 kv, qv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kv[e] = kx[e];
                qv[e] = qx[e];
            }
            *reinterpret_cast<u16x8*>(kd) = kv;
            *reinterpret_cast<u16x8*>(qd) = qv;
        } else {
            st4f(kd, f32x4{kx[0], kx[1], kx[2], kx[3]});
            st4f(kd + 4, f32x4{kx[4], kx[5], kx[6], kx[7]});
            st4f(qd, f32x4{qx[0], qx[1], qx[2], qx[3]});
            st4f(qd + 4, f32x4{qx[4], qx[5], qx[6], qx[7]});
        }
    }
    // H's A operand Q^T[key_of(w, mi, c16)][16 tb + 4 g4 + q], before dL/d out
    // takes the Q rows' place
    f32x4 qa[MT][4];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const E x = Qs[(16 * tb + 4 * g4 + q) * LDK + key_of<D>(w, mi, c16)];
                if constexpr (DT == GDN_BF16) qa[mi][tb][q] = gdn_bf16_to_f32(x);
                else qa[mi][tb][q] = x;
            }
    // dL/d out columns DH hh .. + DH - 1 into registers (rows past the end zero)
    constexpr int OP = C * (DH / 4) / kThreads;
    f32x4 dov[OP];
    auto fetch_dout = [&](int hh) {
#pragma unroll
        for (int i = 0; i < OP; ++i) {
            const int e = tid + kThreads * i, t = e / (DH / 4), pc = e % (DH / 4);
            dov[i] = ld4f(a.dout + (row0 + (int64_t)min(t, nt - 1) * p.H) * D + DH * hh + 4 * pc);
            if (t >= nt) dov[i] = zero4();
        }
    };
    auto store_dout = [&]() {
#pragma unroll
        for (int i = 0; i < OP; ++i) {
            const int e = tid + kThreads * i, t = e / (DH / 4), pc = e % (DH / 4);
            st4f(&dOs[t * LDD + 4 * pc], dov[i]);
        }
    };
    __syncthreads();  // the K and Q rows are dead
    // A into the tile: blocks left of the diagonal transposed into the upper
    // triangle (A_tj at (j, t)), the diagonal block in place
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        if (nb > w) continue;
        const int j = 16 * nb + c16;
        if (nb < w) {
            st4f(&AT[j * LDA + 16 * w + 4 * g4], av[nb]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) AT[(16 * w + 4 * g4 + r) * LDA + j] = av[nb][r];
        }
    }
    fetch_dout(0);
    store_dout();
    __syncthreads();
    // E block row w (all value blocks) and H of the wave's key tiles
    for (int vb = 0; vb < NB; ++vb) {
        if (NH == 2 && vb == NB / 2) {
            // the second column half over the first
            fetch_dout(1);
            __syncthreads();
            store_dout();
            __syncthreads();
        }
        const int vc = 16 * (vb % (NB / NH));  // column of the value block in the staged part
        f32x4 db[4], gb[4];  // B operands dO[16 tb + 4 g4 + q][16 vb + c16], and scale gamma_t times it
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) db[tb][q] = dOs[(16 * tb + 4 * g4 + q) * LDD + vc + c16];
            gb[tb] = p.scale * *reinterpret_cast<const f32x4*>(&ggam[16 * tb + 4 * g4]) * db[tb];
        }
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            f32x4 acc = zero4();
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc = blk(qa[mi][tb], gb[tb], acc);
            st4f(ws.Hf + ci * Rec<D>::kHf + ((size_t)(vb * NB + w * MT + mi) * 64 + l) * 4, acc);
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            if (tb >= w) acc = blk(pk[tb], db[tb], acc);
        st4f(ws.Ef + ci * Rec<D>::kRows + ((size_t)(vb * 4 + w) * 64 + l) * 4, p.scale * acc);
    }
    ut_inverse_lds(AT, threadIdx.x);

    // T and T^T, row-major, zero above (below) the diagonal
    float* Tg = ws.T + ci * Rec<D>::kTile;
    float* TTg = ws.TT + ci * Rec<D>::kTile;
    for (int e = tid; e < C * C / 4; e += kThreads) {
        const int r0 = e >> 4, c0 = (e & 15) * 4;
        f32x4 x, y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = c0 + i <= r0 ? AT[r0 * LDA + c0 + i] : 0.f;   // T[r0][c0 + i]
            y[i] = r0 <= c0 + i ? AT[(c0 + i) * LDA + r0] : 0.f; // T^T[r0][c0 + i] = T[c0 + i][r0]
        }
        st4f(Tg + r0 * C + c0, x);
        st4f(TTg + r0 * C + c0, y);
    }
}

// ---------------------------------------------------------------------------
// k_bchain: the forward state chain and the reverse adjoint chain
// ---------------------------------------------------------------------------
// LDS of a chain workgroup carrying NS adjacent 16-row slices of the state.
template <int NS>
struct ChainShared {
    f32x4 red[NS][4][4][64];  // [slice][wave][token tile][lane]: partial K S^T (or K dS^T)
    f32x4 xch[NS][4][64];     // [slice][token tile][lane]: Delta R (forward) / dDelta (reverse)
    f32x4 xch2[NS][4][64];    // reverse: -gamma' beta dU'
    float vs[2][16 * NS][C + 4];  // forward: V of the slices, [chunk parity][value][token]
    float tp[4][5][16][20];   // per wave: 16 x 16 tiles being transposed for stores
    float g[2][8][C];         // [chunk parity][row kG*][token]: gate rows
};

// A chunk's gate rows in LDS (written by the preparation kernel, staged
// by the workgroup).
struct RowF {
    const float* g;  // [8][C]
    // rows of four consecutive tokens t0 .. t0 + 3
    __device__ f32x4 v4(int row, int t0) const { return *reinterpret_cast<const f32x4*>(g + row * C + t0); }
    __device__ float gC() const { return g[kGgam * C + C - 1]; }
};

// Operands of a chain step, all fetched one chunk ahead (the next chunk's
// while the current one computes), the gates and the V slices two ahead (they
// are turned into LDS rows at the end of the step before their chunk's);
// rows past the sequence end are read at the last real row and zeroed at
// use.  A chunk's workspace stores are issued at the start of the next chunk.
// Nothing a step waits for was fetched in that step: vector memory results
// count down in issue order, so waiting for a fresh fetch would wait for the
// whole prefetch.  Stores go out in 16-byte pieces after a transpose through
// the wave's own LDS tiles, at the step's start; the next chunk's fetch goes
// out after the step's second barrier, while the rest of the step computes:
// issued at the start, its twenty-odd loads of every wave of the compute
// unit queued in the vector-memory path ahead of the step's first products
// (cycle stamps: ≈3 000 cycles of a ≈14 500-cycle step; the chain measured
// 9 % faster with the later issue).  The K, K^T and T operands serve every
// slice of the workgroup: with two slices a workgroup, the compute unit
// issues half the loads for the same products.
template <int D, int DT>
struct FwdIn {
    static constexpr int MT = D / 64;
    R4<DT> kx[4][MT];    // K[16 at + c16][key_of(w, mi, 4 g4 ..)]: the K S^T operand
    f32x4 tr[4];         // T[16 w + c16][16 jb + 4 g4 ..]
    R8<DT> kt[MT][2];    // K^T fragments of the wave's key tiles, token blocks in pairs
};
template <int DT, int NS>
struct GateIn {
    f32x2 gr;            // gate rows: row tid / 32, tokens 2 (tid % 32) ..
    R4<DT> vr[NS];       // forward: V[t][r0 + 16 s + 4 p ..] of this thread's (t, p) = (tid / 4, tid % 4)
};
template <int D, int DT, int NS>
struct RevIn {
    static constexpr int MT = D / 64;
    R4<DT> kx[4][MT];
    f32x4 ef[NS];        // E tile w of each slice
    f32x4 hf[NS][MT];    // H tiles of the wave's key tiles, each slice
    f32x4 tt[4];         // T^T[16 w + c16][16 jb + 4 g4 ..]
    R8<DT> kt[MT][2];
};

template <int D, int DT, int NS>
struct ChainCtx {
    static constexpr int NB = D / 16, MT = D / 64;
    using Sh = ChainShared<NS>;
    const BwdProblem& a;
    const CbWs& ws;
    int64_t bl, b, h, bh;
    int rho, r0, w, l, g4, c16, NC, tid;  // rho: the first slice (rows r0 = 16 rho ..)
    __device__ int64_t row0(int c) const { return (b * a.p.T + (int64_t)c * C) * a.p.H + h; }
    __device__ int ntok(int c) const { return (int)min<int64_t>(C, a.p.T - (int64_t)c * C); }
    __device__ int64_t cidx(int c) const { return bl * NC + c; }
    // gate rows (and, forward, the V slices) of chunk c, clamped to a real chunk
    __device__ void load_gate(GateIn<DT, NS>& x, int c, bool fwd) const {
        c = min(max(c, 0), NC - 1);
        const int64_t r = row0(c);
        const int nt = ntok(c);
        x.gr = *reinterpret_cast<const f32x2*>(ws.Gr + cidx(c) * Rec<D>::kGr + 2 * tid);
        if (fwd) {
            const int64_t o = (r + (int64_t)min(tid >> 2, nt - 1) * a.p.H) * D + r0 + 4 * (tid & 3);
#pragma unroll
            for (int s = 0; s < NS; ++s) x.vr[s] = ldr<DT>(a.p.v, o + 16 * s);
        }
    }
    template <class In>
    __device__ void load_common(In& x, int c) const {
        const int64_t r = row0(c);
        const int nt = ntok(c);
        const int64_t ci = cidx(c);
#pragma unroll
        for (int at = 0; at < 4; ++at) {
            const int64_t o = (r + (int64_t)min(16 * at + c16, nt - 1) * a.p.H) * D + key_of<D>(w, 0, 4 * g4);
            if constexpr (MT == 2) {
                const R8<DT> k8 = ldr8<DT>(a.p.k, o);
                x.kx[at][0] = k8.h[0];
                x.kx[at][MT - 1] = k8.h[1];
            } else {
                x.kx[at][0] = ldr<DT>(a.p.k, o);
            }
        }
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
                x.kt[mi][tp] = ldr8<DT>(ws.KTf, ci * Rec<D>::kFrag + ((int64_t)((w * MT + mi) * 2 + tp) * 64 + l) * 8);
    }
    __device__ void load(FwdIn<D, DT>& x, int c) const {
        c = min(max(c, 0), NC - 1);
        load_common(x, c);
        const int64_t ci = cidx(c);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) x.tr[jb] = ld4f(ws.T + ci * Rec<D>::kTile + (16 * w + c16) * C + 16 * jb + 4 * g4);
    }
    __device__ void load(RevIn<D, DT, NS>& x, int c) const {
        c = min(max(c, 0), NC - 1);
        load_common(x, c);
        const int64_t ci = cidx(c);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            x.ef[s] = ld4f(ws.Ef + ci * Rec<D>::kRows + ((size_t)((rho + s) * 4 + w) * 64 + l) * 4);
#pragma unroll
            for (int mi = 0; mi < MT; ++mi)
                x.hf[s][mi] = ld4f(ws.Hf + ci * Rec<D>::kHf + ((size_t)((rho + s) * NB + w * MT + mi) * 64 + l) * 4);
        }
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) x.tt[jb] = ld4f(ws.TT + ci * Rec<D>::kTile + (16 * w + c16) * C + 16 * jb + 4 * g4);
    }
    // K^T fragment of key tile mi, token block tb
    template <class In>
    __device__ f32x4 ktf(const In& x, int mi, int tb) const { return cvt<DT>(x.kt[mi][tb >> 1].h[tb & 1]); }
    // partial K S^T over the wave's key tiles for every token tile and slice,
    // to LDS (each K operand converted once for every slice)
    template <class In>
    __device__ void partial_KS(Sh& sh, const In& x, const f32x4 (&St)[NS][MT], int nt) const {
#pragma unroll
        for (int at = 0; at < 4; ++at) {
            f32x4 acc[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) acc[s] = zero4();
            const float ok = 16 * at + c16 < nt ? 1.f : 0.f;
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                const f32x4 ka = ok * cvt<DT>(x.kx[at][mi]);
#pragma unroll
                for (int s = 0; s < NS; ++s) acc[s] = blk(ka, St[s][mi], acc[s]);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) sh.red[s][w][at][l] = acc[s];
        }
    }
    // the state as the gradient kernel's fragments: lane (g, c) holds
    // S[r0 + 16 s + c][key_of(w, mi, 4 g + r)], the fragment lane 16 (c / 4) + 4 g + r
    // wants it in element c % 4; transposed through the wave's tile
    __device__ void store_state(Sh& sh, float* dst, const f32x4 (&St)[NS][MT]) const {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                float(*X)[20] = sh.tp[w][mi];
#pragma unroll
                for (int r = 0; r < 4; ++r) X[4 * g4 + r][c16] = St[s][mi][r];
                const f32x4 v = *reinterpret_cast<const f32x4*>(&X[c16][4 * g4]);
                st4f(dst + ((size_t)((rho + s) * NB + w * MT + mi) * 64 + l) * 4, v);
            }
    }
    // a token tile w of a C x D row block (rows 16 w + 4 g4 + q, column
    // r0 + 16 s + c16) as 16-byte row pieces: lane l takes row l / 4, columns
    // r0 + 16 s + 4 (l % 4) ..; base points at row 0, column 0, rows ld apart
    __device__ void store_rows(Sh& sh, int slot, float* base, int64_t ld, const f32x4& x, int nvalid, int s) const {
        float(*X)[20] = sh.tp[w][slot];
#pragma unroll
        for (int q = 0; q < 4; ++q) X[4 * g4 + q][c16] = x[q];
        const int i = l >> 2, j = l & 3;
        const f32x4 v = *reinterpret_cast<const f32x4*>(&X[i][4 * j]);
        if (16 * w + i < nvalid) st4f(base + (int64_t)(16 * w + i) * ld + r0 + 16 * s + 4 * j, v);
    }
    // this thread's two gate-row entries into a parity's LDS rows
    __device__ void gates_to_lds(float* gw, const GateIn<DT, NS>& x) const {
        *reinterpret_cast<f32x2*>(gw + 2 * tid) = x.gr;
    }
    // the slices of V (this thread's four values of one token per slice)
    // into LDS, transposed to [value][token]
    __device__ void v_to_lds(Sh& sh, int buf, const GateIn<DT, NS>& x, int nt) const {
        const int t = tid >> 2, j = tid & 3;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4 v = t < nt ? cvt<DT>(x.vr[s]) : zero4();
#pragma unroll
            for (int e = 0; e < 4; ++e) sh.vs[buf][16 * s + 4 * j + e][t] = v[e];
        }
    }
};

template <int D, int DT, int NS>
__device__ void chain_forward(const ChainCtx<D, DT, NS>& cx, ChainShared<NS>& sh, f32x4 (&St)[NS][D / 64]) {
    constexpr int MT = D / 64;
    const CbWs& ws = cx.ws;
    const int w = cx.w, l = cx.l, g4 = cx.g4, c16 = cx.c16;
    // two operand sets and two gate sets that trade roles every step (no
    // copies between them, so a step waits only for the previous step's
    // fetches)
    FwdIn<D, DT> xa, xb;
    GateIn<DT, NS> ga, gb;
    cx.load(xa, 0);
    cx.load_gate(ga, 0, true);
    cx.gates_to_lds(&sh.g[0][0][0], ga);
    cx.v_to_lds(sh, 0, ga, cx.ntok(0));
    cx.load_gate(ga, 1, true);
    // the previous chunk's U and Delta tiles, stored at the next chunk's start
    // (chunk 0's slots first take zeros, overwritten in order by the same lane)
    f32x4 pU[NS], pD[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) pU[s] = pD[s] = zero4();
    int64_t pci = cx.cidx(0);
    // chunk c from cur; fetches chunk c + 1 into nxt and the gates of chunk
    // c + 2 into g2; turns g1 (chunk c + 1) into LDS rows at the end
    auto step = [&](int c, const FwdIn<D, DT>& cur, FwdIn<D, DT>& nxt, const GateIn<DT, NS>& g1, GateIn<DT, NS>& g2) {
        const RowF rf{&sh.g[c & 1][0][0]};
        const int64_t ci = cx.cidx(c);
        const int nt = cx.ntok(c);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            cx.store_rows(sh, 2, ws.U + pci * Rec<D>::kRows, D, pU[s], C, s);
            cx.store_rows(sh, 3, ws.Dl + pci * Rec<D>::kRows, D, pD[s], C, s);
        }
        cx.store_state(sh, ws.Sf + ci * Rec<D>::kState, St);
        cx.partial_KS(sh, cur, St, nt);
        __syncthreads();
        // U' tiles jb <= w and the Delta tile w = sum_jb T[w][jb] U'[jb]
        f32x4 dl[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) dl[s] = zero4();
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            if (jb > w) continue;
            const f32x4 gp = rf.v4(kGgamp, 16 * jb + 4 * g4), bt = rf.v4(kGbeta, 16 * jb + 4 * g4);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const f32x4 X = sh.red[s][0][jb][l] + sh.red[s][1][jb][l] + sh.red[s][2][jb][l] + sh.red[s][3][jb][l];
                const f32x4 U = *reinterpret_cast<const f32x4*>(&sh.vs[c & 1][16 * s + c16][16 * jb + 4 * g4]) - gp * X;
                if (jb == w) pU[s] = U;
                dl[s] = blk(cur.tr[jb], bt * U, dl[s]);
            }
        }
        const f32x4 Rw = rf.v4(kGR, 16 * w + 4 * g4);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            pD[s] = dl[s];
            sh.xch[s][w][l] = Rw * dl[s];
        }
        pci = ci;
        __syncthreads();
        cx.load(nxt, c + 1);
        cx.load_gate(g2, c + 2, true);
        // S^T <- gamma_C S^T + K^T diag(R) Delta
        const float gC = rf.gC();
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            f32x4 acc[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) acc[s] = gC * St[s][mi];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const f32x4 ka = cx.ktf(cur, mi, tb);
#pragma unroll
                for (int s = 0; s < NS; ++s) acc[s] = blk(ka, sh.xch[s][tb][l], acc[s]);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) St[s][mi] = acc[s];
        }
        // the next chunk's gate rows and V slices while the update multiplies
        // (every wave is past this chunk's first barrier, the last reader of
        // the buffers written here)
        const int nn = cx.ntok(min(c + 1, cx.NC - 1));
        cx.gates_to_lds(&sh.g[(c + 1) & 1][0][0], g1);
        cx.v_to_lds(sh, (c + 1) & 1, g1, nn);
    };
    int c = 0;
    for (; c + 1 < cx.NC; c += 2) {
        step(c, xa, xb, ga, gb);
        step(c + 1, xb, xa, gb, ga);
    }
    if (c < cx.NC) step(c, xa, xb, ga, gb);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        cx.store_rows(sh, 2, ws.U + pci * Rec<D>::kRows, D, pU[s], C, s);
        cx.store_rows(sh, 3, ws.Dl + pci * Rec<D>::kRows, D, pD[s], C, s);
    }
}

template <int D, int DT, int NS>
__device__ void chain_reverse(const ChainCtx<D, DT, NS>& cx, ChainShared<NS>& sh, f32x4 (&St)[NS][D / 64]) {
    constexpr int MT = D / 64;
    const BwdProblem& a = cx.a;
    const Problem& p = a.p;
    const CbWs& ws = cx.ws;
    const int w = cx.w, l = cx.l, g4 = cx.g4;
    RevIn<D, DT, NS> xa, xb;
    GateIn<DT, NS> ga, gb;
    cx.load(xa, cx.NC - 1);
    cx.load_gate(ga, cx.NC - 1, false);
    cx.gates_to_lds(&sh.g[(cx.NC - 1) & 1][0][0], ga);
    cx.load_gate(ga, cx.NC - 2, false);
    // the previous step's dDelta, dU' and dv tiles, stored at the next step's
    // start (the first step's slots first take zeros, then the real values)
    f32x4 pdD[NS], pdU[NS], pdv[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) pdD[s] = pdU[s] = pdv[s] = zero4();
    int64_t pci = cx.cidx(cx.NC - 1), prow = cx.row0(cx.NC - 1);
    int pnt = 0;
    // chunk c from cur; fetches chunk c - 1 into nxt and the gates of chunk
    // c - 2 into g2; turns g1 (chunk c - 1) into LDS rows at the end
    auto step = [&](int c, const RevIn<D, DT, NS>& cur, RevIn<D, DT, NS>& nxt, const GateIn<DT, NS>& g1,
                    GateIn<DT, NS>& g2) {
        const RowF rf{&sh.g[c & 1][0][0]};
        const int64_t ci = cx.cidx(c);
        const int nt = cx.ntok(c);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            cx.store_rows(sh, 2, ws.dDl + pci * Rec<D>::kRows, D, pdD[s], C, s);
            cx.store_rows(sh, 3, ws.dUp + pci * Rec<D>::kRows, D, pdU[s], C, s);
            cx.store_rows(sh, 4, a.dv + prow * D, p.H * D, pdv[s], pnt, s);
        }
        cx.store_state(sh, ws.dSf + ci * Rec<D>::kState, St);
        cx.partial_KS(sh, cur, St, nt);
        __syncthreads();
        // dDelta tile w = diag(R) K dS^T + E_w
        const f32x4 Rw = rf.v4(kGR, 16 * w + 4 * g4);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4 Y = sh.red[s][0][w][l] + sh.red[s][1][w][l] + sh.red[s][2][w][l] + sh.red[s][3][w][l];
            const f32x4 dd = Rw * Y + cur.ef[s];
            sh.xch[s][w][l] = dd;
            pdD[s] = dd;
        }
        __syncthreads();
        cx.load(nxt, c - 1);
        cx.load_gate(g2, c - 2, false);
        // dU' tile w = sum_{jb >= w} T^T[w][jb] dDelta[jb]; dv = beta dU'
        f32x4 du[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) du[s] = zero4();
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            if (jb >= w) {
#pragma unroll
                for (int s = 0; s < NS; ++s) du[s] = blk(cur.tt[jb], sh.xch[s][jb][l], du[s]);
            }
        const f32x4 bt = rf.v4(kGbeta, 16 * w + 4 * g4);
        const f32x4 mgb = -(rf.v4(kGgamp, 16 * w + 4 * g4) * bt);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            sh.xch2[s][w][l] = mgb * du[s];
            pdU[s] = du[s];
            pdv[s] = bt * du[s];
        }
        pci = ci;
        prow = cx.row0(c);
        pnt = nt;
        __syncthreads();
        // dS^T <- gamma_C dS^T + scale Q^T diag(gamma) dO - K^T diag(gamma' beta) dU'
        const float gC = rf.gC();
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            f32x4 acc[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) acc[s] = gC * St[s][mi] + cur.hf[s][mi];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const f32x4 ka = cx.ktf(cur, mi, tb);
#pragma unroll
                for (int s = 0; s < NS; ++s) acc[s] = blk(ka, sh.xch2[s][tb][l], acc[s]);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) St[s][mi] = acc[s];
        }
        // the next chunk's gate rows while the update multiplies (every wave
        // is past this chunk's first barrier, the last reader of the buffer)
        cx.gates_to_lds(&sh.g[(c + 1) & 1][0][0], g1);
    };
    int c = cx.NC - 1;
    for (; c >= 1; c -= 2) {
        step(c, xa, xb, ga, gb);
        step(c - 1, xb, xa, gb, ga);
    }
    if (c == 0) step(0, xa, xb, ga, gb);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        cx.store_rows(sh, 2, ws.dDl + pci * Rec<D>::kRows, D, pdD[s], C, s);
        cx.store_rows(sh, 3, ws.dUp + pci * Rec<D>::kRows, D, pdU[s], C, s);
        cx.store_rows(sh, 4, a.dv + prow * D, p.H * D, pdv[s], pnt, s);
    }
}

// NS adjacent 16-row slices of a head's state per workgroup and direction:
// two on heads x slices that fill the compute units that way, one otherwise.
template <int D, int DT, int NS>
__global__ __launch_bounds__(kThreads, NS == 1 ? 2 : 1) void k_bchain(BwdProblem a, CbWs ws) {
    constexpr int NB = D / 16, MT = D / 64;
    constexpr int NSL = NB / NS;  // workgroups per head and direction
    __shared__ ChainShared<NS> sh;
    const Problem& p = a.p;
    // workgroups go to the eight XCDs in turn; the logical order (head,
    // direction, slice group) is laid over them so that consecutive logical
    // indices, the 2 NSL workgroups of a head that read the same chunk
    // operands, share an XCD and its L2
    const int64_t N = 2 * a.nbh * NSL;
    const int64_t lin = N % 8 == 0 ? (blockIdx.x % 8) * (N / 8) + blockIdx.x / 8 : blockIdx.x;
    const int64_t head = lin / (2 * NSL);
    const int rem = (int)(lin - head * 2 * NSL);
    const bool rev = rem < NSL;
    ChainCtx<D, DT, NS> cx{a, ws};
    cx.bl = head;
    cx.rho = NS * (rev ? rem : rem - NSL);
    cx.r0 = 16 * cx.rho;
    cx.bh = a.bh0 + cx.bl;
    cx.b = cx.bh / p.H;
    cx.h = cx.bh - cx.b * p.H;
    const int tid = threadIdx.x;
    cx.tid = tid;
    cx.w = tid >> 6;
    cx.l = tid & 63;
    cx.g4 = cx.l >> 4;
    cx.c16 = cx.l & 15;
    cx.NC = p.NC;
    // the slices' state rows as accumulator tiles of S^T: tile mi of slice s
    // holds S[r0 + 16 s + c16][key_of(w, mi, 4 g4 + r)]
    f32x4 St[NS][MT];
    const float* init = rev ? a.ds_out : p.s0;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
            St[s][mi] = init ? ld4f(init + ((cx.bh * D + cx.r0 + 16 * s + cx.c16) * D) + key_of<D>(cx.w, mi, 4 * cx.g4))
                             : zero4();
    if (p.NC > 0) {
        if (rev) chain_reverse<D, DT, NS>(cx, sh, St);
        else chain_forward<D, DT, NS>(cx, sh, St);
    }
    if (rev && a.ds0) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int mi = 0; mi < MT; ++mi)
                st4f(a.ds0 + ((cx.bh * D + cx.r0 + 16 * s + cx.c16) * D) + key_of<D>(cx.w, mi, 4 * cx.g4), St[s][mi]);
    }
}

// Slices per chain workgroup: two once the heads' slice pairs and both
// directions still give a workgroup to every compute unit.
inline int chain_slices(int64_t nbh, int64_t D) { return nbh * (D / 16) >= 256 ? 2 : 1; }

// ---------------------------------------------------------------------------
// k_bgrad: dq, dk, dbeta and dalpha of one chunk
// ---------------------------------------------------------------------------
struct GradShared {
    float dPm[C * LDA];   // dP o M (lower triangle with the diagonal, zero above)
    float W[C * LDA];     // W + W^T
    float dT[C * LDA];    // dT (lower triangle)
    float Vm[C * LDA];    // gate terms V[b][a + 1]; then their prefix along a
    float ghi[C], glo[C], gphi[C], gplo[C], gbeta[C], galpha[C];
    float db1[C];         // dU'_t . U_t
    float db2[4][C];      // per wave: sum_j dA_tj Atilde_tj
    float vo[4][C], vx[4][C], vr[4][C];  // per wave: q.dQ_S0, k.dK_S0, k.dK_dS
    float sd[4];          // per wave: <dS_end, S>
};

// Global operands are fetched ahead of their use throughout: a job's or a
// block's whole set at once, the next phase's before the barrier that ends
// the current one, the state products' next value block while the current
// one multiplies.
template <int D, int DT>
__global__ __launch_bounds__(kThreads, 2) void k_bgrad(BwdProblem a, CbWs ws) {
    constexpr int NB = D / 16, MT = D / 64;
    __shared__ __attribute__((aligned(16))) GradShared sh;
    const Problem& p = a.p;
    const int64_t ci = blockIdx.x;
    const int64_t bl = ci / p.NC;
    const int c = (int)(ci - bl * p.NC);
    const int64_t bh = a.bh0 + bl, b = bh / p.H, h = bh - b * p.H;
    const int64_t t0 = (int64_t)c * C;
    const int nt = (int)min<int64_t>(C, p.T - t0);
    const int64_t row0 = (b * p.T + t0) * p.H + h;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const float* U = ws.U + ci * Rec<D>::kRows;
    const float* Dl = ws.Dl + ci * Rec<D>::kRows;
    const float* dDl = ws.dDl + ci * Rec<D>::kRows;
    const float* dUp = ws.dUp + ci * Rec<D>::kRows;
    const float* Tg = ws.T + ci * Rec<D>::kTile;
    const float* TTg = ws.TT + ci * Rec<D>::kTile;
    const float* PTg = ws.PT + ci * Rec<D>::kTile;
    const float* AtTg = ws.AtT + ci * Rec<D>::kTile;
    const float* Sf = ws.Sf + ci * Rec<D>::kState;
    const float* dSf = ws.dSf + ci * Rec<D>::kState;
    const InE<DT>* KTf = static_cast<const InE<DT>*>(ws.KTf) + ci * Rec<D>::kFrag;
    const InE<DT>* QTf = static_cast<const InE<DT>*>(ws.QTf) + ci * Rec<D>::kFrag;
    auto rowaddr = [&](int t) { return (row0 + (int64_t)min(t, nt - 1) * p.H) * D; };

    // ---- phase 0: gates, dU'.U, cleared sums
    if (w == 0) {
        const Gate g = chunk_gate(p, row0, nt, l);
        sh.ghi[l] = g.hi;
        sh.glo[l] = g.lo;
        sh.gphi[l] = g.phi;
        sh.gplo[l] = g.plo;
        sh.gbeta[l] = g.beta;
        sh.galpha[l] = g.alpha;
    }
    {
        const int t = tid >> 2, part = tid & 3;
        f32x4 x[NB / 2], y[NB / 2];
#pragma unroll
        for (int i = 0; i < NB / 2; ++i) {
            x[i] = ld4f(dUp + t * D + 4 * part + 16 * i);
            y[i] = ld4f(U + t * D + 4 * part + 16 * i);
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NB / 2; ++i) s += dot4(x[i], y[i]);
#pragma unroll
        for (int i = 0; i < NB / 2; ++i) {
            x[i] = ld4f(dUp + t * D + 4 * part + 16 * (i + NB / 2));
            y[i] = ld4f(U + t * D + 4 * part + 16 * (i + NB / 2));
        }
#pragma unroll
        for (int i = 0; i < NB / 2; ++i) s += dot4(x[i], y[i]);
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (part == 0) sh.db1[t] = s;
    }
    for (int e = tid; e < C * LDA; e += kThreads) sh.Vm[e] = 0.f;
    for (int e = tid; e < 4 * C; e += kThreads) (&sh.db2[0][0])[e] = 0.f;
    __syncthreads();
    auto ex = [&](int tb_, int ja) { return ratio(sh.ghi[tb_], sh.glo[tb_], sh.ghi[ja], sh.glo[ja]); };
    auto exp_ = [&](int tb_, int ja) { return ratio(sh.gphi[tb_], sh.gplo[tb_], sh.ghi[ja], sh.glo[ja]); };

    // ---- phase 1: dP = scale dO Delta^T and dT = dDelta U^T diag(beta) on
    // the lower blocks (10 each), all operands of a job fetched at once
    for (int job = w; job < 20; job += 4) {
        const int kind = job / 10, tb = blk_m(job % 10), jb = blk_n(job % 10);
        const int ta = 16 * tb + c16, ja = 16 * jb + c16;  // A-operand row, B-operand row
        const float* Ar = kind == 0 ? a.dout + rowaddr(ta) : dDl + ta * D;
        const float* Br = (kind == 0 ? Dl : U) + ja * D;
        const float ok = (kind == 0 && ta >= nt) ? 0.f : 1.f;
        f32x4 av[NB], bv[NB];
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) {
            av[vb] = ld4f(Ar + 16 * vb + 4 * g4);
            bv[vb] = ld4f(Br + 16 * vb + 4 * g4);
        }
        const f32x4 pv = kind == 0 ? ld4f(PTg + ja * C + 16 * tb + 4 * g4) : zero4();  // P[t][j], r = 0..3
        f32x4 x = zero4();
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) x = blk(ok * av[vb], bv[vb], x);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * g4 + r, j = ja;
            if (kind == 0) {
                const float dp = p.scale * x[r];
                sh.dPm[t * LDA + j] = j <= t ? dp * ex(t, j) : 0.f;
                sh.Vm[t * LDA + 1 + j] = j < t ? dp * pv[r] : 0.f;
            } else {
                sh.dT[t * LDA + j] = j <= t ? x[r] * sh.gbeta[j] : 0.f;
            }
        }
    }
    // phase 2's operands: rows of T (block bb = w), of T^T and Atilde^T
    const int bb = w;
    f32x4 trow[4], ttrow[4][4], atr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        trow[i] = ld4f(Tg + (16 * bb + c16) * C + 16 * i + 4 * g4);
        atr[i] = ld4f(AtTg + (16 * bb + c16) * C + 16 * i + 4 * g4);
#pragma unroll
        for (int k = 0; k < 4; ++k) ttrow[i][k] = ld4f(TTg + (16 * i + c16) * C + 16 * k + 4 * g4);
    }
    __syncthreads();

    // ---- phase 2: dA = -T^T (dT T^T), column block bb = w.  W + W^T: the
    // lower entry (ar, bc) and its transpose, the diagonal zero
    {
        f32x4 Z[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            Z[ib] = zero4();
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                if (ib >= bb && jb <= bb)
                    Z[ib] = blk(ld4f(&sh.dT[(16 * ib + c16) * LDA + 16 * jb + 4 * g4]), trow[jb], Z[ib]);
        }
#pragma unroll
        for (int ab = 0; ab < 4; ++ab) {
            if (ab < bb) continue;
            f32x4 dA = zero4();
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
                if (ib >= ab) dA = blk(ttrow[ab][ib], Z[ib], dA);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ar = 16 * ab + 4 * g4 + r, bc = 16 * bb + c16;
                const bool lower = ar > bc;
                const float da = -dA[r];
                const float at = lower ? atr[ab][r] : 0.f;
                const float bt = sh.gbeta[ar];
                if (lower) {
                    const int row = p.order == GDN_DECAY_THEN_PREDICT ? ar : ar - 1;
                    sh.Vm[row * LDA + 1 + bc] += da * bt * at;
                    const float wk = bt * da * exp_(ar, bc);
                    sh.W[ar * LDA + bc] = wk;
                    sh.W[bc * LDA + ar] = wk;
                } else if (ar == bc) {
                    sh.W[ar * LDA + bc] = 0.f;
                }
                const float rs = row_sum<16>(lower ? da * at : 0.f);
                if (c16 == 0) sh.db2[w][ar] = rs;
            }
        }
    }

    // ---- phase 3: dQ and dK, value-column blocks db = w MT + mi.  State
    // products first, in one pass over the value blocks vb (S with dO and
    // dU', dS_end with Delta, and <dS_end, S>), fetching block vb + 1 while
    // block vb multiplies: every state fragment is read once
    float fo[4], fu[4], fr[4], okr[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int t = 16 * tb + c16;
        okr[tb] = t < nt ? 1.f : 0.f;
        fo[tb] = p.scale * __expf(sh.ghi[t] + sh.glo[t]);
        fu[tb] = -__expf(sh.gphi[t] + sh.gplo[t]) * sh.gbeta[t];
        fr[tb] = ratio(sh.ghi[C - 1], sh.glo[C - 1], sh.ghi[t], sh.glo[t]);
    }
    struct PassIn {
        f32x4 sf[MT], dsf[MT], ao[4], au[4], ad[4];
    };
    auto fidx = [&](int vb, int mi) { return ((size_t)(vb * NB + w * MT + mi) * 64 + l) * 4; };
    auto load_pass = [&](PassIn& x, int vb) {
        vb = min(vb, NB - 1);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            x.sf[mi] = ld4f(Sf + fidx(vb, mi));
            x.dsf[mi] = ld4f(dSf + fidx(vb, mi));
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            x.ao[tb] = ld4f(a.dout + rowaddr(16 * tb + c16) + 16 * vb + 4 * g4);
            x.au[tb] = ld4f(dUp + (16 * tb + c16) * D + 16 * vb + 4 * g4);
            x.ad[tb] = ld4f(Dl + (16 * tb + c16) * D + 16 * vb + 4 * g4);
        }
    };
    PassIn pa, pa2;
    load_pass(pa, 0);
    __syncthreads();

    f32x4 aQ[4][MT], aK1[4][MT], aK2[4][MT];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) aQ[tb][mi] = aK1[tb][mi] = aK2[tb][mi] = zero4();
    float sdot = 0.f;
#pragma unroll 1
    for (int vb = 0; vb < NB; ++vb) {
        load_pass(pa2, vb + 1);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) sdot += dot4(pa.sf[mi], pa.dsf[mi]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const f32x4 Ao = (okr[tb] * fo[tb]) * pa.ao[tb];
            const f32x4 Au = fu[tb] * pa.au[tb];
            const f32x4 Ad = fr[tb] * pa.ad[tb];
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                aQ[tb][mi] = blk(Ao, pa.sf[mi], aQ[tb][mi]);
                aK1[tb][mi] = blk(Au, pa.sf[mi], aK1[tb][mi]);
                aK2[tb][mi] = blk(Ad, pa.dsf[mi], aK2[tb][mi]);
            }
        }
        pa = pa2;
    }
    // K^T and Q^T fragments of the wave's value blocks, for the rest of dQ, dK
    R8<DT> kf[MT][2], qf[MT][2];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            kf[mi][i] = ldr8<DT>(KTf, ((int64_t)((w * MT + mi) * 2 + i) * 64 + l) * 8);
            qf[mi][i] = ldr8<DT>(QTf, ((int64_t)((w * MT + mi) * 2 + i) * 64 + l) * 8);
        }
    // boundary terms: q_t . dQ_S0, k_t . dK_S0, k_t . dK_dS (rows of the
    // tiles; the Q^T and K^T fragments hold q and k in the accumulator layout:
    // Q[16 tb + 4 g4 + r][key_col(db, c16)] in element r)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        f32x4 qv[MT], kv[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            qv[mi] = cvt<DT>(qf[mi][tb >> 1].h[tb & 1]);
            kv[mi] = cvt<DT>(kf[mi][tb >> 1].h[tb & 1]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * g4 + r;
            float so = 0.f, sx = 0.f, sr = 0.f;
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                so += qv[mi][r] * aQ[tb][mi][r];
                sx += kv[mi][r] * aK1[tb][mi][r];
                sr += kv[mi][r] * aK2[tb][mi][r];
            }
            // (rows past the sequence end: their accumulators are zero or unused)
            so = row_sum<16>(t < nt ? so : 0.f);
            sx = row_sum<16>(t < nt ? sx : 0.f);
            sr = row_sum<16>(t < nt ? sr : 0.f);
            if (c16 == 0) {
                sh.vo[w][t] = so;
                sh.vx[w][t] = sx;
                sh.vr[w][t] = sr;
            }
        }
    }
    {
        float s = sdot;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
        if (l == 0) sh.sd[w] = s;
    }
    // dQ += (dP o M) K,  dK += (dP o M)^T Q + (W + W^T) K
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            const int db = w * MT + mi;
            f32x4 q = aQ[tb][mi], kk = aK1[tb][mi] + aK2[tb][mi];
#pragma unroll
            for (int jb = 0; jb <= tb; ++jb)
                q = blk(ld4f(&sh.dPm[(16 * tb + c16) * LDA + 16 * jb + 4 * g4]), cvt<DT>(kf[mi][jb >> 1].h[jb & 1]), q);
#pragma unroll
            for (int sb = tb; sb < 4; ++sb) {
                f32x4 at;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) at[qq] = sh.dPm[(16 * sb + 4 * g4 + qq) * LDA + 16 * tb + c16];
                kk = blk(at, cvt<DT>(qf[mi][sb >> 1].h[sb & 1]), kk);
            }
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
                kk = blk(ld4f(&sh.W[(16 * tb + c16) * LDA + 16 * ib + 4 * g4]), cvt<DT>(kf[mi][ib >> 1].h[ib & 1]), kk);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tb + 4 * g4 + r;
                if (t < nt) {
                    const int64_t o = (row0 + (int64_t)t * p.H) * D + key_col<D>(db, c16);
                    a.dq[o] = q[r];
                    a.dk[o] = kk[r];
                }
            }
        }
    }
    __syncthreads();

    // ---- phase 4: boundary terms into V, then dlog alpha_s = sum_{b >= s}
    // sum_{a' <= s} V[b][a'], dalpha = that / alpha, dbeta
    if (w == 0) {
        const int t = l;
        const float vo = sh.vo[0][t] + sh.vo[1][t] + sh.vo[2][t] + sh.vo[3][t];
        const int tx = p.order == GDN_DECAY_THEN_PREDICT ? t : t + 1;  // k_tx . dK_S0 lands in row t
        const float vx = tx < C ? sh.vx[0][tx] + sh.vx[1][tx] + sh.vx[2][tx] + sh.vx[3][tx] : 0.f;
        float c0 = vo + vx;
        if (t == C - 1) {
            const float sd = sh.sd[0] + sh.sd[1] + sh.sd[2] + sh.sd[3];
            c0 += __expf(sh.ghi[C - 1] + sh.glo[C - 1]) * sd;
        }
        sh.Vm[t * LDA] += c0;
        if (t < C - 1) sh.Vm[(C - 1) * LDA + 1 + t] += sh.vr[0][t] + sh.vr[1][t] + sh.vr[2][t] + sh.vr[3][t];
    }
    __syncthreads();
    {
        // inclusive prefix along each row over a' = 0 .. 63: four threads a
        // row (consecutive lanes), 16 entries each, then the parts' offsets
        const int bro = tid >> 2, part = tid & 3;
        float* row = &sh.Vm[bro * LDA + 16 * part];
        float s = 0.f;
        float pre[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s += row[i];
            pre[i] = s;
        }
        const float s1 = __shfl_up(s, 1, 64), s2 = __shfl_up(s, 2, 64), s3 = __shfl_up(s, 3, 64);
        const float off = (part >= 1 ? s1 : 0.f) + (part >= 2 ? s2 : 0.f) + (part >= 3 ? s3 : 0.f);
#pragma unroll
        for (int i = 0; i < 16; ++i) row[i] = pre[i] + off;
    }
    __syncthreads();
    {
        const int s = tid >> 2, part = tid & 3;
        float acc = 0.f;
        for (int bro = max(16 * part, s); bro < 16 * part + 16; ++bro) acc += sh.Vm[bro * LDA + s];
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        if (part == 0 && s < nt) {
            const int64_t o = row0 + (int64_t)s * p.H;
            a.dalpha[o] = acc / sh.galpha[s];
            a.dbeta[o] = sh.db1[s] + sh.db2[0][s] + sh.db2[1][s] + sh.db2[2][s] + sh.db2[3][s];
        }
    }
}

template <int D, int DT>
hipError_t launch_chunked(const BwdProblem& a, const CbWs& ws, hipStream_t st) {
    const int64_t nch = a.nbh * a.p.NC;
    prof_begin(a.p.timer, "k_bprep", st);
    hipLaunchKernelGGL((k_bprep<D, DT>), dim3((unsigned)nch), dim3(kThreads), 0, st, a, ws);
    prof_end(a.p.timer, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_begin(a.p.timer, "k_bchain", st);
    if (chain_slices(a.nbh, D) == 2)
        hipLaunchKernelGGL((k_bchain<D, DT, 2>), dim3((unsigned)(a.nbh * (D / 16))), dim3(kThreads), 0, st, a, ws);
    else
        hipLaunchKernelGGL((k_bchain<D, DT, 1>), dim3((unsigned)(2 * a.nbh * (D / 16))), dim3(kThreads), 0, st, a, ws);
    prof_end(a.p.timer, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    prof_begin(a.p.timer, "k_bgrad", st);
    hipLaunchKernelGGL((k_bgrad<D, DT>), dim3((unsigned)nch), dim3(kThreads), 0, st, a, ws);
    prof_end(a.p.timer, st);
    return hipGetLastError();
}

}  // namespace

bool chunked_backward_supported(int64_t dk, int64_t dv, int gate) {
    return gate == GDN_GATE_SCALAR && dk == dv && (dk == 64 || dk == 128);
}

// Workspace bytes per (batch, head) of the chunked backward; larger batches
// run in groups of heads so that the workspace stays within the cap.
static size_t chunked_bytes_per_head(int64_t T, int64_t D) {
    const size_t nc = (size_t)((T + C - 1) / C);
    const size_t nb = (size_t)(D / 16);
    const size_t per_chunk = sizeof(float) * (4 * (size_t)C * C + 2 * nb * 4 * 64 * 4 + 2 * nb * nb * 64 * 4 +
                                              5 * (size_t)C * D + (size_t)D * D + 8 * (size_t)C);
    return nc * per_chunk;
}
constexpr size_t kChunkedWsCap = size_t(8) << 30;
static int64_t chunked_heads_per_launch(int64_t B, int64_t T, int64_t H, int64_t D) {
    const size_t per = chunked_bytes_per_head(T, D);
    const int64_t g = per > 0 ? (int64_t)(kChunkedWsCap / per) : B * H;
    return std::max<int64_t>(1, std::min<int64_t>(B * H, g));
}

size_t chunked_backward_workspace(int64_t B, int64_t T, int64_t H, int64_t D) {
    // fifteen pieces, each 256-byte aligned
    return chunked_bytes_per_head(T, D) * (size_t)chunked_heads_per_launch(B, T, H, D) + 15 * 256;
}

hipError_t backward_chunked(const BwdProblem& a_in, void* workspace, hipStream_t st) {
    BwdProblem a0 = a_in;
    a0.p.C = C;
    a0.p.NC = (int)((a0.p.T + C - 1) / C);
    const Problem& p = a0.p;
    const int64_t D = p.dk, BH = p.B * p.H;
    if (p.T == 0) {
        // dS_0 = dS_T: the chain kernel with no chunks (its whole grid, both
        // directions, as the block order assumes; the forward half does nothing)
        BwdProblem g = a0;
        g.bh0 = 0;
        g.nbh = BH;
        CbWs ws{};
        hipLaunchKernelGGL((D == 64 ? k_bchain<64, GDN_BF16, 1> : k_bchain<128, GDN_BF16, 1>),
                           dim3((unsigned)(2 * BH * (D / 16))), dim3(kThreads), 0, st, g, ws);
        return hipGetLastError();
    }
    const int64_t gsz = chunked_heads_per_launch(p.B, p.T, p.H, D);
    const size_t nch = (size_t)gsz * (size_t)p.NC;
    const size_t nb = (size_t)(D / 16);
    char* base = static_cast<char*>(workspace);
    size_t off = 0;
    auto take = [&](size_t floats) {
        float* q = reinterpret_cast<float*>(base + off);
        off += align256(floats * sizeof(float));
        return q;
    };
    CbWs ws;
    ws.T = take(nch * C * C);
    ws.TT = take(nch * C * C);
    ws.PT = take(nch * C * C);
    ws.AtT = take(nch * C * C);
    ws.KTf = take(nch * nb * 4 * 64 * 4);  // (sized for fp32 inputs)
    ws.QTf = take(nch * nb * 4 * 64 * 4);
    ws.Sf = take(nch * nb * nb * 64 * 4);
    ws.dSf = take(nch * nb * nb * 64 * 4);
    ws.U = take(nch * C * D);
    ws.Dl = take(nch * C * D);
    ws.dDl = take(nch * C * D);
    ws.dUp = take(nch * C * D);
    ws.Ef = take(nch * C * D);
    ws.Hf = take(nch * D * D);
    ws.Gr = take(nch * 8 * C);
    for (int64_t bh0 = 0; bh0 < BH; bh0 += gsz) {
        BwdProblem g = a0;
        g.bh0 = bh0;
        g.nbh = std::min<int64_t>(gsz, BH - bh0);
        hipError_t e;
        if (D == 64) e = p.dtype == GDN_BF16 ? launch_chunked<64, GDN_BF16>(g, ws, st) : launch_chunked<64, GDN_F32>(g, ws, st);
        else e = p.dtype == GDN_BF16 ? launch_chunked<128, GDN_BF16>(g, ws, st) : launch_chunked<128, GDN_F32>(g, ws, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gdn
