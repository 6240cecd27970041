// fp32 vector-ALU kernels of the chunkwise gated delta rule (gfx950).
//
// This family runs every supported shape and both input dtypes; bf16 inputs
// are widened exactly to fp32 on load and all arithmetic is fp32.  It is the
// path for fp32 inputs and for shapes the MFMA kernels do not cover.
//
// Three launches per forward (plus two for sequence parallelism):
//   k_prep_valu  one workgroup per (batch, head, chunk): gate prefixes, the
//                UT transform T' = (I + diag(beta) L)^{-1} diag(beta), the
//                gated causal scores P, and the gated key/query operands;
//   k_rec_valu   one workgroup per (batch, head, segment, 16-row tile): the
//                sequential chunk loop carrying a 16 x dk slice of the state;
//   k_chain_valu / k_correct_valu (sequence parallel only).
//
// Chunk algebra (chunk-local gate prefix b_t = prod_{u<=t} alpha_u, b'_t the
// prefix the prediction sees: b_{t-1} predict-then-decay, b_t
// decay-then-predict; entry state S):
//   L_tj  = (k_t (.) b'_t).(k_j / b_j),  j < t
//   T'    = (I + diag(beta) L)^{-1} diag(beta)
//   Delta = T' (V - (K (.) B') S^T)
//   O     = scale ((Q (.) B) S^T + P Delta),  P_tj = (q_t (.) b_t).(k_j / b_j), j <= t
//   S'    = S Diag(b_C) + Delta^T (K (.) b_C / B)
// following the WY/UT section (U, W, T, chunk state passing, output) and the
// GLA gating section (gate prefixes, gated scores, boundary key) of the
// DeltaNet illustrated notes (stay-hungry-time.github.io/deltanet).  Every
// gate ratio is evaluated as exp(g_t - g_j) with g the chunk-local log
// prefix and t >= j, so no factor exceeds one.
#include <algorithm>

#include "gdn_internal.h"
#include "../../include/gdn.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;  // state rows per k_rec_valu workgroup

struct ValuWs {
    int64_t per_ch;  // floats per chunk-head
    int C, dk;
    __host__ __device__ float* Tp(float* base, int64_t ch) const { return base + ch * per_ch; }
    __host__ __device__ float* P(float* base, int64_t ch) const { return Tp(base, ch) + C * C; }
    __host__ __device__ float* Kp(float* base, int64_t ch) const { return P(base, ch) + C * C; }
    __host__ __device__ float* Qg(float* base, int64_t ch) const { return Kp(base, ch) + C * dk; }
    __host__ __device__ float* Kb(float* base, int64_t ch) const { return Qg(base, ch) + C * dk; }
    __host__ __device__ float* bC(float* base, int64_t ch) const { return Kb(base, ch) + C * dk; }
    __host__ __device__ float* G(float* base, int64_t ch) const { return bC(base, ch) + dk; }
};

ValuWs make_ws(const Problem& p) {
    ValuWs w;
    w.C = p.C;
    w.dk = (int)p.dk;
    w.per_ch = 2LL * p.C * p.C + 4LL * p.C * p.dk + p.dk;
    return w;
}

// ---------------------------------------------------------------------------
// stage 1: per chunk-head preparation
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_prep_valu(Problem p, ValuWs w, float* ws) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int C = p.C, dk = (int)p.dk, tid = threadIdx.x;
    const int64_t H = p.H, T = p.T;
    const int64_t ch = ((int64_t)b * H + h) * p.NC + i;
    const int64_t t0 = (int64_t)i * C;
    const int nt = (int)((T - t0) < C ? (T - t0) : C);
    const bool channel = p.gate == GDN_GATE_CHANNEL;

    extern __shared__ float smem[];
    const int kw = (dk > C ? dk : C) + 1;
    float* Ks = smem;                  // [C][dk+1]; reused as T [C][C+1]
    float* As = Ks + C * kw;           // [C][C+1]
    float* gs = As + C * (C + 1);      // scalar gates: g [C], g' [C]
    float* bs = gs + 2 * C;            // beta [C]

    float* Gl = w.G(ws, ch);           // channel gates: g [C][dk] (global)
    auto row = [&](int t) { return ((int64_t)b * T + t0 + t) * H + h; };

    for (int e = tid; e < C * dk; e += kThreads) {
        const int t = e / dk, a = e - (e / dk) * dk;
        Ks[t * (dk + 1) + a] = t < nt ? gdn_ld<DT>(p.k, row(t) * dk + a) : 0.f;
    }
    for (int t = tid; t < C; t += kThreads) bs[t] = t < nt ? p.beta[row(t)] : 0.f;

    // chunk-local log prefixes; padded tokens neither decay nor write (the
    // loops over tokens and keys below read global memory every iteration and
    // are unrolled so that several loads are in flight)
    if (!channel) {
        if (tid == 0) {
            float g = 0.f;
#pragma unroll 8
            for (int t = 0; t < C; ++t) {
                const float prev = g;
                if (t < nt) g += logf(p.alpha[row(t)]);
                gs[t] = g;
                gs[C + t] = p.order == GDN_PREDICT_THEN_DECAY ? prev : g;
            }
        }
    } else if (tid < dk) {
        float g = 0.f;
#pragma unroll 8
        for (int t = 0; t < C; ++t) {
            if (t < nt) g += logf(p.alpha[row(t) * dk + tid]);
            Gl[t * dk + tid] = g;
        }
    }
    __syncthreads();

    auto G = [&](int t, int a) -> float { return channel ? Gl[t * dk + a] : gs[t]; };
    auto GP = [&](int t, int a) -> float {
        if (!channel) return gs[C + t];
        if (p.order == GDN_PREDICT_THEN_DECAY) return t > 0 ? Gl[(t - 1) * dk + a] : 0.f;
        return Gl[t * dk + a];
    };

    // gated operands for the recurrence
    float* Kp = w.Kp(ws, ch);
    float* Qg = w.Qg(ws, ch);
    float* Kb = w.Kb(ws, ch);
    for (int e = tid; e < C * dk; e += kThreads) {
        const int t = e / dk, a = e - (e / dk) * dk;
        const float kk = Ks[t * (dk + 1) + a];
        const float qq = t < nt ? gdn_ld<DT>(p.q, row(t) * dk + a) : 0.f;
        const float gt = G(t, a);
        Kp[e] = kk * expf(GP(t, a));
        Qg[e] = qq * expf(gt);
        Kb[e] = kk * expf(G(C - 1, a) - gt);
    }
    for (int a = tid; a < dk; a += kThreads) w.bC(ws, ch)[a] = expf(G(C - 1, a));

    // L (scaled by beta) and the gated causal scores P
    float* P = w.P(ws, ch);
    for (int e = tid; e < C * C; e += kThreads) {
        const int t = e / C, j = e - (e / C) * C;
        float l = 0.f, s = 0.f;
        if (j <= t) {
#pragma unroll 8
            for (int a = 0; a < dk; ++a) {
                const float kj = Ks[j * (dk + 1) + a];
                const float qt = t < nt ? gdn_ld<DT>(p.q, row(t) * dk + a) : 0.f;
                if (channel) {
                    const float gj = G(j, a);
                    if (j < t) l += Ks[t * (dk + 1) + a] * kj * expf(GP(t, a) - gj);
                    s += qt * kj * expf(G(t, a) - gj);
                } else {
                    if (j < t) l += Ks[t * (dk + 1) + a] * kj;
                    s += qt * kj;
                }
            }
            if (!channel) {
                l *= expf(gs[C + t] - gs[j]);
                s *= expf(gs[t] - gs[j]);
            }
        }
        As[t * (C + 1) + j] = j < t ? bs[t] * l : 0.f;
        P[t * C + j] = s;
    }
    __syncthreads();

    // forward substitution: T = (I + A)^{-1}, one column per thread
    float* Ts = Ks;  // [C][C+1], K no longer needed
    for (int j = tid; j < C; j += kThreads) {
        for (int t = 0; t < C; ++t) {
            float x;
            if (t < j) {
                x = 0.f;
            } else if (t == j) {
                x = 1.f;
            } else {
                x = 0.f;
                for (int m = j; m < t; ++m) x -= As[t * (C + 1) + m] * Ts[m * (C + 1) + j];
            }
            Ts[t * (C + 1) + j] = x;
        }
    }
    __syncthreads();
    float* Tp = w.Tp(ws, ch);
    for (int e = tid; e < C * C; e += kThreads) {
        const int t = e / C, j = e - (e / C) * C;
        Tp[e] = Ts[t * (C + 1) + j] * bs[j];
    }
}

// ---------------------------------------------------------------------------
// stage 2: sequential chunk loop on a 16-row slice of the state
// ---------------------------------------------------------------------------
// Tile kinds: state tiles (rows of S, value dims) and, for segments g >= 1 of
// a sequence-parallel run, scaling tiles (rows of M, key dims, zero values,
// identity start) whose "output" is the correction operator R_i.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_rec_valu(Problem p, ValuWs w, float* ws,
                                                       Split sp, WsLayout L, char* wsb) {
    const int x = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
    const int h = hg / sp.G, g = hg - (hg / sp.G) * sp.G;
    const int dk = (int)p.dk, dv = (int)p.dv, C = p.C, tid = threadIdx.x;
    const int nvt = dv / kRows;
    const bool scaling = x >= nvt;
    if (scaling && g == 0) return;
    const int r0 = (scaling ? x - nvt : x) * kRows;
    const int64_t H = p.H, T = p.T, bh = (int64_t)b * H + h;

    extern __shared__ float smem[];
    float* Ss = smem;                       // [16][dk+1]
    float* Xs = Ss + kRows * (dk + 1);      // [C][17]
    float* Ds = Xs + C * (kRows + 1);       // [C][17]

    for (int e = tid; e < kRows * dk; e += kThreads) {
        const int r = e / dk, a = e - (e / dk) * dk;
        float s;
        if (scaling) s = (r0 + r == a) ? 1.f : 0.f;
        else if (g == 0 && p.s0) s = p.s0[(bh * dv + r0 + r) * dk + a];
        else s = 0.f;
        Ss[r * (dk + 1) + a] = s;
    }
    __syncthreads();

    float* corr = reinterpret_cast<float*>(wsb + L.corr);
    const int i_begin = g * sp.per;
    const int i_end = min(p.NC, (g + 1) * sp.per);
    // (the inner products read the chunk's operands from global memory, one
    // load an iteration: unrolled so that eight loads are in flight at once
    // instead of one round trip per term)
    for (int i = i_begin; i < i_end; ++i) {
        const int64_t ch = bh * p.NC + i;
        const int64_t t0 = (int64_t)i * C;
        const int nt = (int)((T - t0) < C ? (T - t0) : C);
        const float* Kp = w.Kp(ws, ch);
        const float* Qg = w.Qg(ws, ch);
        const float* Kb = w.Kb(ws, ch);
        const float* Tp = w.Tp(ws, ch);
        const float* P = w.P(ws, ch);
        const float* bC = w.bC(ws, ch);

        // X = V - (K (.) B') S^T
        for (int e = tid; e < C * kRows; e += kThreads) {
            const int t = e >> 4, r = e & 15;
            float y = 0.f;
#pragma unroll 8
            for (int a = 0; a < dk; ++a) y += Kp[t * dk + a] * Ss[r * (dk + 1) + a];
            float vv = 0.f;
            if (!scaling && t < nt) vv = gdn_ld<DT>(p.v, ((b * T + t0 + t) * H + h) * dv + r0 + r);
            Xs[t * (kRows + 1) + r] = vv - y;
        }
        __syncthreads();
        // Delta = T' X
        for (int e = tid; e < C * kRows; e += kThreads) {
            const int t = e >> 4, r = e & 15;
            float d = 0.f;
#pragma unroll 8
            for (int j = 0; j <= t; ++j) d += Tp[t * C + j] * Xs[j * (kRows + 1) + r];
            Ds[t * (kRows + 1) + r] = d;
        }
        __syncthreads();
        // O = scale ((Q (.) B) S^T + P Delta)
        for (int e = tid; e < C * kRows; e += kThreads) {
            const int t = e >> 4, r = e & 15;
            float o = 0.f;
#pragma unroll 8
            for (int a = 0; a < dk; ++a) o += Qg[t * dk + a] * Ss[r * (dk + 1) + a];
#pragma unroll 8
            for (int j = 0; j <= t; ++j) o += P[t * C + j] * Ds[j * (kRows + 1) + r];
            o *= p.scale;
            if (scaling) corr[ch * C * dk + (int64_t)t * dk + r0 + r] = o;
            else if (t < nt) p.out[((b * T + t0 + t) * H + h) * dv + r0 + r] = o;
        }
        __syncthreads();
        // S' = S Diag(b_C) + Delta^T Kbar
        for (int e = tid; e < kRows * dk; e += kThreads) {
            const int r = e / dk, a = e - (e / dk) * dk;
            float s = Ss[r * (dk + 1) + a] * bC[a];
#pragma unroll 8
            for (int t = 0; t < C; ++t) s += Ds[t * (kRows + 1) + r] * Kb[t * dk + a];
            Ss[r * (dk + 1) + a] = s;
        }
        __syncthreads();
    }

    float* dst;
    if (scaling) {
        dst = reinterpret_cast<float*>(wsb + L.mend) + (bh * sp.G + g) * dk * dk;
    } else if (sp.G == 1) {
        dst = p.s_out ? p.s_out + bh * dv * dk : nullptr;
    } else {
        dst = reinterpret_cast<float*>(wsb + L.sdend) + (bh * sp.G + g) * dv * dk;
    }
    if (dst) {
        for (int e = tid; e < kRows * dk; e += kThreads) {
            const int r = e / dk, a = e - (e / dk) * dk;
            dst[(int64_t)(r0 + r) * dk + a] = Ss[r * (dk + 1) + a];
        }
    }
}

}  // namespace

WsLayout valu_layout(const Problem& p, const Split& sp) {
    WsLayout L;
    const ValuWs w = make_ws(p);
    const int64_t nch = p.B * p.H * (int64_t)p.NC;
    L.prep = 0;
    L.prep_bytes = align256(sizeof(float) * w.per_ch * nch);
    size_t off = L.prep_bytes;
    if (sp.G > 1) {
        L.corr = off;
        L.corr_bytes = align256(sizeof(float) * nch * p.C * p.dk);
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
    }
    L.total = off;
    return L;
}

hipError_t valu_forward(const Problem& p, const Split& sp, char* ws, hipStream_t st) {
    const WsLayout L = valu_layout(p, sp);
    const ValuWs w = make_ws(p);
    float* wsp = reinterpret_cast<float*>(ws + L.prep);
    const int C = p.C, dk = (int)p.dk, dv = (int)p.dv;

    {
        dim3 grid(p.NC, (unsigned)p.H, (unsigned)p.B);
        const size_t kw = (size_t)(dk > C ? dk : C) + 1;
        const size_t lds = sizeof(float) * ((size_t)C * kw + (size_t)C * (C + 1) + 3 * C);
        prof_begin(p.timer, "k_prep_valu", st);
        if (p.dtype == GDN_BF16)
            hipLaunchKernelGGL(k_prep_valu<1>, grid, dim3(kThreads), lds, st, p, w, wsp);
        else
            hipLaunchKernelGGL(k_prep_valu<0>, grid, dim3(kThreads), lds, st, p, w, wsp);
        prof_end(p.timer, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        const int ntiles = dv / kRows + (sp.G > 1 ? dk / kRows : 0);
        dim3 grid(ntiles, (unsigned)(p.H * sp.G), (unsigned)p.B);
        const size_t lds = sizeof(float) * ((size_t)kRows * (dk + 1) + 2 * (size_t)C * (kRows + 1));
        prof_begin(p.timer, "k_rec_valu", st);
        if (p.dtype == GDN_BF16)
            hipLaunchKernelGGL(k_rec_valu<1>, grid, dim3(kThreads), lds, st, p, w, wsp, sp, L, ws);
        else
            hipLaunchKernelGGL(k_rec_valu<0>, grid, dim3(kThreads), lds, st, p, w, wsp, sp, L, ws);
        prof_end(p.timer, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (sp.G > 1) return seqpar_finish(p, sp, ws, L, false, st);
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// sequence-parallel tail (shared by both kernel families)
// ---------------------------------------------------------------------------
namespace {

// S_start(g+1) = S^D_end(g) + S_start(g) M_end(g), 16 state rows per block;
// rows of the start state evolve independently.  M_end(g) is staged in LDS.
// With frag != nullptr the start states are also written as bf16 hi/lo
// B-operand fragments for the MFMA correction: [n][s][hi/lo][lane] of 8
// bf16, lane (row v = 16n + lane%16, columns 32s + 8(lane/16) .. +7).
// Chain of segment start states, S_start(g + 1) = S^D_end(g) + S_start(g) M_end(g)
// (sequence-parallel notes: the true state is the increment plus the start
// state through the scaling matrix).  Rows of S chain independently, so one
// workgroup takes 16 rows of one head; each step is a 16 x dk x dk product in
// fp32 on the matrix cores (16x16x4 fp32 MFMA: instruction s contracts the
// indices 4G + s, G = lane / 16), with M_end(g + 1) fetched into registers
// while step g computes.  With write_frag the start states are also stored
// as bf16 hi/lo A-fragments for the MFMA output correction.  Without
// final_step the chain stops at the last segment's start state (the
// whole-head path runs that segment from it and ends the state itself).
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t bf16_rne(float v) {
    const uint32_t ub = __float_as_uint(v);
    return (uint16_t)((ub + 0x7FFFu + ((ub >> 16) & 1u)) >> 16);
}

constexpr int kChainMaxD = 128;
constexpr int kChainMPieces = kChainMaxD * kChainMaxD / 4 / kThreads;  // float4 of M per thread

__global__ __launch_bounds__(kThreads) void k_chain(Problem p, Split sp, WsLayout L, char* wsb,
                                                    int write_frag, int final_step) {
    const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int dk = (int)p.dk, dv = (int)p.dv, tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, g4 = l >> 4, c16 = l & 15;
    const int r0 = x * kRows;
    const int64_t bh = (int64_t)b * p.H + h;
    const float* sdend = reinterpret_cast<const float*>(wsb + L.sdend);
    const float* mend = reinterpret_cast<const float*>(wsb + L.mend);
    float* sstart = reinterpret_cast<float*>(wsb + L.sstart);
    const int ldc = dk + 1, ldm = dk + 4;

    extern __shared__ float smem[];
    float* bufA = smem;                   // [16][dk + 1]
    float* bufB = bufA + kRows * ldc;     // [16][dk + 1]
    float* Ms = bufB + kRows * ldc;       // [dk][dk + 4]
    float* Cur = bufA;
    float* Nxt = bufB;
    for (int e = tid; e < kRows * dk; e += kThreads) {
        const int r = e / dk, a = e - (e / dk) * dk;
        Cur[r * ldc + a] = sdend[(bh * sp.G + 0) * dv * dk + (int64_t)(r0 + r) * dk + a];
    }
    const int mp = dk * dk / 4;  // float4 pieces of M
    f32x4v mreg[kChainMPieces];
    auto load_m = [&](int g) {
        const f32x4v* M = reinterpret_cast<const f32x4v*>(mend + (bh * sp.G + min(g, sp.G - 1)) * dk * dk);
#pragma unroll
        for (int k = 0; k < kChainMPieces; ++k) mreg[k] = M[min(tid + kThreads * k, mp - 1)];
    };
    load_m(1);
    for (int g = 1; g < sp.G; ++g) {
        const float* SD = sdend + (bh * sp.G + g) * dv * dk;
        float* SS = sstart + (bh * sp.G + g) * dv * dk;
#pragma unroll
        for (int k = 0; k < kChainMPieces; ++k) {
            const int e = tid + kThreads * k;
            if (e < mp) {
                const int a = (4 * e) / dk, c = (4 * e) % dk;
                *reinterpret_cast<f32x4v*>(&Ms[a * ldm + c]) = mreg[k];
            }
        }
        load_m(g + 1);
        __syncthreads();  // M(g) staged, Cur = S_start(g) complete
        if (write_frag) {
            // rows r0..r0+15 as A fragments of every k-step: lane (row lane % 16,
            // keys 32s + 8 (lane / 16) ..), hi and lo halves, 16-byte stores
            const int ks = dk / 32;
            u16x8v* fr = reinterpret_cast<u16x8v*>(wsb + L.sfrag) + ((bh * sp.G + g) * (dv / 16) + x) * (int64_t)ks * 2 * 64;
            for (int f = tid; f < ks * 64; f += kThreads) {
                const int s = f >> 6, lane = f & 63;
                const int r = lane & 15, a0 = 32 * s + 8 * (lane >> 4);
                u16x8v hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = Cur[r * ldc + a0 + e];
                    const uint16_t hb = bf16_rne(v);
                    hi[e] = hb;
                    lo[e] = bf16_rne(v - __uint_as_float((uint32_t)hb << 16));
                }
                fr[(s * 2 + 0) * 64 + lane] = hi;
                fr[(s * 2 + 1) * 64 + lane] = lo;
            }
        }
        for (int e = tid; e < kRows * dk; e += kThreads) {
            const int r = e / dk, c = e - (e / dk) * dk;
            SS[(int64_t)(r0 + r) * dk + c] = Cur[r * ldc + c];
        }
        if (g == sp.G - 1 && !final_step) return;  // the last segment ends the state itself
        // Nxt = SD + Cur M: wave w takes column tiles w, w + 4, ...
        // (four independent accumulator chains, one per instruction s)
        for (int nt = w; nt < dk / 16; nt += 4) {
            f32x4v acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[0][i] = SD[(int64_t)(r0 + 4 * g4 + i) * dk + 16 * nt + c16];
                acc[1][i] = acc[2][i] = acc[3][i] = 0.f;
            }
            for (int kb = 0; kb < dk / 16; ++kb) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(Cur[c16 * ldc + 16 * kb + 4 * g4 + s],
                                                                  Ms[(16 * kb + 4 * g4 + s) * ldm + 16 * nt + c16],
                                                                  acc[s], 0, 0, 0);
            }
            const f32x4v sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) Nxt[(4 * g4 + i) * ldc + 16 * nt + c16] = sum[i];
        }
        __syncthreads();  // Nxt complete; Cur and Ms free
        float* t = Cur;
        Cur = Nxt;
        Nxt = t;
    }
    if (p.s_out) {
        for (int e = tid; e < kRows * dk; e += kThreads) {
            const int r = e / dk, a = e - (e / dk) * dk;
            p.s_out[(bh * dv + r0 + r) * dk + a] = Cur[r * ldc + a];
        }
    }
}

// O_i += R_i S_start(g)^T for the chunks of segments g >= 1.
__global__ __launch_bounds__(kThreads) void k_correct(Problem p, Split sp, WsLayout L, char* wsb) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = i / sp.per;
    if (g == 0) return;
    const int dk = (int)p.dk, dv = (int)p.dv, C = p.C, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * p.H + h, T = p.T, H = p.H;
    const int64_t ch = bh * p.NC + i, t0 = (int64_t)i * C;
    const int nt = (int)((T - t0) < C ? (T - t0) : C);
    const float* R = reinterpret_cast<const float*>(wsb + L.corr) + ch * C * dk;
    const float* SS = reinterpret_cast<const float*>(wsb + L.sstart) + (bh * sp.G + g) * dv * dk;
    for (int e = tid; e < nt * dv; e += kThreads) {
        const int t = e / dv, c = e - (e / dv) * dv;
        float s = 0.f;
        for (int a = 0; a < dk; ++a) s += R[(int64_t)t * dk + a] * SS[(int64_t)c * dk + a];
        p.out[((b * T + t0 + t) * H + h) * dv + c] += s;
    }
}

__global__ void k_copy_state(Problem p) {
    const int64_t n = p.B * p.H * p.dv * p.dk;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x)
        p.s_out[e] = p.s0 ? p.s0[e] : 0.f;
}

}  // namespace

hipError_t seqpar_chain(const Problem& p, const Split& sp, char* ws, const WsLayout& L,
                        bool write_frag, bool final_step, hipStream_t st) {
    const int dk = (int)p.dk, dv = (int)p.dv;
    dim3 grid(dv / kRows, (unsigned)p.H, (unsigned)p.B);
    const size_t lds = sizeof(float) * (2 * kRows * (dk + 1) + (size_t)dk * (dk + 4));
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_chain),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    prof_begin(p.timer, "k_chain", st);
    hipLaunchKernelGGL(k_chain, grid, dim3(kThreads), lds, st, p, sp, L, ws, write_frag ? 1 : 0,
                       final_step ? 1 : 0);
    prof_end(p.timer, st);
    return hipGetLastError();
}

hipError_t seqpar_finish(const Problem& p, const Split& sp, char* ws, const WsLayout& L,
                         bool mfma, hipStream_t st) {
    {
        hipError_t e = seqpar_chain(p, sp, ws, L, mfma, true, st);
        if (e != hipSuccess) return e;
    }
    if (mfma) return mfma_correct(p, sp, ws, L, st);
    {
        dim3 grid(p.NC, (unsigned)p.H, (unsigned)p.B);
        prof_begin(p.timer, "k_correct", st);
        hipLaunchKernelGGL(k_correct, grid, dim3(kThreads), 0, st, p, sp, L, ws);
        prof_end(p.timer, st);
        return hipGetLastError();
    }
}

// The block's prologue for raw projections on the vector-ALU family: q and k
// L2-normalised per (batch, token, head) along their features (a zero vector
// stays zero), v converted to fp32, alpha = sigmoid(alpha_logit) (per head or
// per key channel), beta = sigmoid(beta_logit), written as fp32 [B, T, H, .]
// for the forward kernels (DeltaNet illustrated notes, block description).
// One wave per (batch, token, head) row, lanes over the features.
template <int DT>
__global__ __launch_bounds__(256) void k_raw_prologue(Problem p, RawInputs r) {
    const int lane = threadIdx.x & 63;
    const int64_t rows = p.B * p.T * p.H;
    const int dk = (int)p.dk, dv = (int)p.dv;
    const bool chan = p.gate == GDN_GATE_CHANNEL;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
        float sq = 0.f, sk = 0.f;
        for (int a = lane; a < dk; a += 64) {
            const float x = gdn_ld<DT>(p.q, row * dk + a), y = gdn_ld<DT>(p.k, row * dk + a);
            sq += x * x;
            sk += y * y;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            sq += __shfl_xor(sq, o, 64);
            sk += __shfl_xor(sk, o, 64);
        }
        const float rq = gdn_inv_len(sq), rk = gdn_inv_len(sk);
        for (int a = lane; a < dk; a += 64) {
            r.q[row * dk + a] = rq * gdn_ld<DT>(p.q, row * dk + a);
            r.k[row * dk + a] = rk * gdn_ld<DT>(p.k, row * dk + a);
            if (chan) r.alpha[row * dk + a] = gdn_sigmoid(p.alpha[row * dk + a]);
        }
        for (int a = lane; a < dv; a += 64) r.v[row * dv + a] = gdn_ld<DT>(p.v, row * dv + a);
        if (lane == 0) {
            if (!chan) r.alpha[row] = gdn_sigmoid(p.alpha[row]);
            r.beta[row] = gdn_sigmoid(p.beta[row]);
        }
    }
}

size_t raw_inputs_bytes(const Problem& p) {
    const int64_t rows = p.B * p.T * p.H;
    return align256(sizeof(float) * rows * p.dk) * 2 + align256(sizeof(float) * rows * p.dv) +
           align256(sizeof(float) * rows * (p.gate == GDN_GATE_CHANNEL ? p.dk : 1)) +
           align256(sizeof(float) * rows);
}

RawInputs raw_inputs_at(const Problem& p, char* base) {
    const int64_t rows = p.B * p.T * p.H;
    RawInputs r;
    size_t off = 0;
    r.q = reinterpret_cast<float*>(base + off);
    off += align256(sizeof(float) * rows * p.dk);
    r.k = reinterpret_cast<float*>(base + off);
    off += align256(sizeof(float) * rows * p.dk);
    r.v = reinterpret_cast<float*>(base + off);
    off += align256(sizeof(float) * rows * p.dv);
    r.alpha = reinterpret_cast<float*>(base + off);
    off += align256(sizeof(float) * rows * (p.gate == GDN_GATE_CHANNEL ? p.dk : 1));
    r.beta = reinterpret_cast<float*>(base + off);
    return r;
}

hipError_t raw_prologue(const Problem& p, const RawInputs& r, hipStream_t st) {
    const int64_t rows = p.B * p.T * p.H;
    if (rows == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((rows + 3) / 4, 8192);
    prof_begin(p.timer, "k_raw_prologue", st);
    if (p.dtype == GDN_BF16)
        hipLaunchKernelGGL(k_raw_prologue<1>, dim3((unsigned)blocks), dim3(256), 0, st, p, r);
    else
        hipLaunchKernelGGL(k_raw_prologue<0>, dim3((unsigned)blocks), dim3(256), 0, st, p, r);
    prof_end(p.timer, st);
    return hipGetLastError();
}

hipError_t copy_state(const Problem& p, hipStream_t st) {
    if (!p.s_out) return hipSuccess;
    const int64_t n = p.B * p.H * p.dv * p.dk;
    if (n == 0) return hipSuccess;
    const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    prof_begin(p.timer, "k_copy_state", st);
    hipLaunchKernelGGL(k_copy_state, dim3(blocks), dim3(256), 0, st, p);
    prof_end(p.timer, st);
    return hipGetLastError();
}

}  // namespace gdn
