// Backward pass of the gated delta rule (gdn_backward): gradients of a loss
// through the forward recurrence, for both gate orderings and gate kinds.
//
// The pages give the recurrence, not its gradient (the Gated DeltaNet
// GPU-parallelisation blog, section 1.2, and the DeltaNet illustrated notes
// fix the forward; training through it is mentioned, not derived).  Here the
// chain rule is applied to one token step, row by row: rows r of the dv x dk
// state evolve independently given the token's k, gate d and beta, so with
// X_r = S_r (predict-then-decay) or S_r * d (decay-then-predict),
// p_r = X_r . k, e_r = beta (v_r - p_r) and G_r = dL/dS'_r + scale do_r q,
// gk_r = G_r . k:
//   dv_r = beta gk_r                 dbeta += gk_r (v_r - p_r)
//   dk  += e_r G_r - beta gk_r X_r   dq    += scale do_r S'_r
//   predict-then-decay: dL/dS_r = G_r * d - beta gk_r k,  dd += G_r * S_r
//   decay-then-predict: dX_r = G_r - beta gk_r k,  dL/dS_r = dX_r * d,
//                       dd += dX_r * S_r
// (dalpha = dd for a channel gate, its sum over channels for a scalar gate).
//
// Schedule (recompute from boundary-state checkpoints): a workgroup owns a
// block of state rows of one (batch, head) and works in runs of kSub tokens,
// whose inputs (q, k, gates, beta and the block's v and dL/dout) are staged
// into LDS by one coalesced load of the whole workgroup, issued while the
// previous run computes.  Phase A runs the recurrence forward over the
// sequence and stores its rows of the state at every run start in the
// workspace.  Phase B walks the runs backwards: it recomputes each run's
// states from its checkpoint into registers and carries dL/dS back through
// them.  (Checkpoints every 64 tokens, with the run starts recomputed per
// interval, took 14 % more time for a quarter of the workspace.)  The
// per-token sums over rows (dq, dk, dalpha, dbeta) are reduced within the
// workgroup through LDS and stored as one record per (row block, token) in
// the workspace; k_bwd_reduce then sums a head's row blocks into the outputs
// in a fixed order with plain coalesced accesses (fp32 atomics from every row
// block into the outputs took 2.7 ms of the main workload's 11.9).  dv is
// row-local and written directly, as is dL/dS_0.
//
// Every thread holds kRows rows as float4 pieces, LPR lanes per row (the
// layout of the decode step); a row's dot products are butterfly sums over
// its lanes on the vector ALU (DPP and lane swaps).
#include <algorithm>

#include "gdn_internal.h"
#include "../../include/gdn.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 2;    // rows per thread
constexpr int kSub = 16;    // tokens recomputed into registers at a time
constexpr int kMaxD = 128;

template <int DT>
__device__ __forceinline__ float4 ld4(const void* p, int64_t i) {
    if constexpr (DT == 0) {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    }
}

// a 16-byte load from global memory, typed so: a conditional load must not
// become a load through a pointer chosen between this address and a
// zero-filled stack slot (a generic load, which every LDS wait then waits for)
typedef float f32x4g __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ldg4(const float* p) {
    const f32x4g x = *(const __attribute__((address_space(1))) f32x4g*)(p);
    return make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float4 mul4(const float4& a, const float4& b) {
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 axpy4(float s, const float4& x, const float4& y) {  // s x + y
    return make_float4(s * x.x + y.x, s * x.y + y.y, s * x.z + y.z, s * x.w + y.w);
}
__device__ __forceinline__ float4 add4(const float4& a, const float4& b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

template <int LPR>
__device__ __forceinline__ float4 group_sum4(float4 x) {
    return make_float4(group_sum<LPR>(x.x), group_sum<LPR>(x.y), group_sum<LPR>(x.z),
                       group_sum<LPR>(x.w));
}

// one token's inputs as a thread sees them
struct Tok {
    float4 k, q, d;
    float beta;
    float v[kRows];
    float dout[kRows];
};

// LDS of a workgroup: the inputs of one run of kSub tokens (fp32), the
// per-token partial sums of a run, and the states at the runs' starts
template <int LPR, int RB>
struct BwdShared {
    static constexpr int KD = 4 * LPR;  // largest dk of this lane layout
    float tq[kSub][KD], tk[kSub][KD], td[kSub][KD];
    float tbeta[kSub], talpha[kSub];
    float tv[kSub][RB], tdo[kSub][RB];
    float4 vec[4][kSub][3][LPR];        // [wave][token][dq | dk | dd][piece]
    float sc[4][kSub][2];               // dbeta, dalpha (scalar gate)
};

template <int DT, int LPR, bool CH, bool DTPO>
struct Bwd {
    static constexpr int RPW = 64 / LPR;             // rows per wave and pass
    static constexpr int RB = 4 * RPW * kRows;       // rows per workgroup
    static constexpr int KD = 4 * LPR;
    static constexpr int QP = (kSub * KD / 4 + kThreads - 1) / kThreads;  // staged pieces per thread
    static constexpr int VP = (kSub * RB + kThreads - 1) / kThreads;
    using Sh = BwdShared<LPR, RB>;
    // (by value: a reference to the kernel argument would put it in scratch
    // memory and turn every pointer read from it into a generic one)
    const BwdProblem a;
    Sh& sh;
    int64_t b, h, bh;
    int rb, c, w, l, tid;
    bool col;
    int r[kRows], rr[kRows];
    bool on[kRows];

    __device__ Bwd(const BwdProblem& a_, Sh& sh_, int64_t bh_, int rb_) : a(a_), sh(sh_) {
        const Problem& p = a.p;
        bh = bh_;
        rb = rb_;
        b = bh / p.H;
        h = bh - b * p.H;
        tid = threadIdx.x;
        w = tid >> 6;
        l = tid & 63;
        c = l % LPR;
        col = 4 * c < p.dk;
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            rr[j] = (j * 4 + w) * RPW + l / LPR;
            r[j] = rb * RB + rr[j];
            on[j] = r[j] < p.dv;
        }
    }

    // ---- staging of a run's inputs: loads into registers, then LDS
    struct Stage {
        float4 q[QP], k[QP], d[QP];
        float beta, alpha;
        float v[VP], dout[VP];
    };
    __device__ void stage_load(Stage& s, int64_t ts, int m) const {
        const Problem& p = a.p;
        const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
        const int P4 = KD / 4;
#pragma unroll
        for (int i = 0; i < QP; ++i) {
            const int e = tid + kThreads * i, u = e / P4, c4 = e % P4;
            const bool ok = e < kSub * P4 && u < m && 4 * c4 < p.dk;
            const int64_t th = (b * p.T + ts + u) * p.H + h;
            s.q[i] = ok ? ld4<DT>(p.q, th * p.dk + 4 * c4) : z4;
            s.k[i] = ok ? ld4<DT>(p.k, th * p.dk + 4 * c4) : z4;
            if constexpr (CH) s.d[i] = ok ? *reinterpret_cast<const float4*>(p.alpha + th * p.dk + 4 * c4) : z4;
        }
        const int64_t th0 = (b * p.T + ts + (tid < m ? tid : 0)) * p.H + h;
        s.beta = tid < m ? p.beta[th0] : 0.f;
        s.alpha = (!CH && tid < m) ? p.alpha[th0] : 0.f;
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int e = tid + kThreads * i, u = e / RB, q = e % RB;
            const bool ok = e < kSub * RB && u < m && rb * RB + q < p.dv;
            const int64_t th = (b * p.T + ts + u) * p.H + h;
            s.v[i] = ok ? gdn_ld<DT>(p.v, th * p.dv + rb * RB + q) : 0.f;
            s.dout[i] = ok ? a.dout[th * p.dv + rb * RB + q] : 0.f;
        }
    }
    __device__ void stage_store(const Stage& s) const {
        const int P4 = KD / 4;
#pragma unroll
        for (int i = 0; i < QP; ++i) {
            const int e = tid + kThreads * i;
            if (e < kSub * P4) {
                const int u = e / P4, c4 = e % P4;
                *reinterpret_cast<float4*>(&sh.tq[u][4 * c4]) = s.q[i];
                *reinterpret_cast<float4*>(&sh.tk[u][4 * c4]) = s.k[i];
                if constexpr (CH) *reinterpret_cast<float4*>(&sh.td[u][4 * c4]) = s.d[i];
            }
        }
        if (tid < kSub) {
            sh.tbeta[tid] = s.beta;
            sh.talpha[tid] = s.alpha;
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int e = tid + kThreads * i;
            if (e < kSub * RB) {
                sh.tv[e / RB][e % RB] = s.v[i];
                sh.tdo[e / RB][e % RB] = s.dout[i];
            }
        }
    }

    // token u of the staged run
    __device__ Tok tok(int u) const {
        Tok x;
        x.k = *reinterpret_cast<const float4*>(&sh.tk[u][4 * c]);
        x.q = *reinterpret_cast<const float4*>(&sh.tq[u][4 * c]);
        if constexpr (CH) {
            x.d = *reinterpret_cast<const float4*>(&sh.td[u][4 * c]);
        } else {
            const float g = sh.talpha[u];
            x.d = make_float4(g, g, g, g);
        }
        x.beta = sh.tbeta[u];
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            x.v[j] = sh.tv[u][rr[j]];
            x.dout[j] = sh.tdo[u][rr[j]];
        }
        return x;
    }

    // the state after the token, from the state before it (rows of the thread)
    __device__ void step(const float4 (&S)[kRows], float4 (&Sn)[kRows], const Tok& x) const {
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            const float4 X = DTPO ? mul4(S[j], x.d) : S[j];
            const float pr = row_sum<LPR>(dot4(X, x.k));
            const float e = x.beta * (x.v[j] - pr);
            Sn[j] = axpy4(e, x.k, DTPO ? X : mul4(S[j], x.d));
        }
    }

    // the thread's piece of row j: in a [B, H, dv, dk] state tensor, and in
    // one head's state (the checkpoints)
    __device__ int64_t off(int j) const { return (bh * a.p.dv + r[j]) * a.p.dk + 4 * c; }
    __device__ int64_t roff(int j) const { return (int64_t)r[j] * a.p.dk + 4 * c; }
};

// Visits of runs of kSub tokens: phase A over runs 0 .. NR - 1, then the
// backward over runs NR - 1 .. 0.
__device__ __forceinline__ int64_t run_of(int64_t vi, int64_t NR) { return vi < NR ? vi : 2 * NR - 1 - vi; }

template <int DT, int LPR, bool CH, bool DTPO>
__global__ __launch_bounds__(kThreads) void k_backward(BwdProblem a, int nrb, int RS) {
    using K = Bwd<DT, LPR, CH, DTPO>;
    __shared__ typename K::Sh sh;
    const Problem& p = a.p;
    const int64_t bl = blockIdx.x / nrb;  // (batch, head) pair within the launch
    const int64_t bh = a.bh0 + bl;
    const K k(a, sh, bh, (int)(blockIdx.x % nrb));
    const int tid = threadIdx.x;
    const int64_t T = p.T;
    const int64_t NR = (T + kSub - 1) / kSub, NV = 2 * NR;
    const int64_t DD = p.dv * p.dk;
    float* ckpt = a.ckpt + bl * NR * DD;  // (the launch's own checkpoint region)
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);

    float4 S[kRows], Gd[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        S[j] = (k.on[j] && k.col && p.s0) ? ldg4(p.s0 + k.off(j)) : z4;
        Gd[j] = (k.on[j] && k.col && a.ds_out) ? ldg4(a.ds_out + k.off(j)) : z4;
    }
    typename K::Stage stg;
    if (NV > 0) {
        k.stage_load(stg, 0, (int)min<int64_t>(kSub, T));
        k.stage_store(stg);
    }
    __syncthreads();
    for (int64_t vi = 0; vi < NV; ++vi) {
        const bool fwd = vi < NR;
        const int64_t R = run_of(vi, NR), ts = R * kSub;
        const int m = (int)min<int64_t>(kSub, T - ts);
        // a backward visit starts from its run's checkpoint (each thread reads
        // back what it wrote; read before the next visit's inputs are
        // requested, so that waiting for it does not wait for them)
        if (!fwd) {
#pragma unroll
            for (int j = 0; j < kRows; ++j) S[j] = (k.on[j] && k.col) ? ldg4(ckpt + R * DD + k.roff(j)) : z4;
        }
        // the next visit's inputs are fetched while this one computes
        if (vi + 1 < NV) {
            const int64_t nR = run_of(vi + 1, NR);
            k.stage_load(stg, nR * kSub, (int)min<int64_t>(kSub, T - nR * kSub));
        }
        if (fwd) {
            // phase A: the run's start state, then its tokens
#pragma unroll
            for (int j = 0; j < kRows; ++j)
                if (k.on[j] && k.col) *reinterpret_cast<float4*>(ckpt + R * DD + k.roff(j)) = S[j];
            for (int u = 0; u < m; ++u) {
                float4 Sn[kRows];
                k.step(S, Sn, k.tok(u));
#pragma unroll
                for (int j = 0; j < kRows; ++j) S[j] = Sn[j];
            }
        } else {
            // backward over the run: its states into registers, St[u] before
            // token ts + u, then dL/dS carried back through them
            float4 St[kSub + 1][kRows];
#pragma unroll
            for (int j = 0; j < kRows; ++j) St[0][j] = S[j];
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                if (u < m) {
                    k.step(St[u], St[u + 1], k.tok(u));
                } else {
#pragma unroll
                    for (int j = 0; j < kRows; ++j) St[u + 1][j] = St[u][j];
                }
            }
#pragma unroll
            for (int u = kSub - 1; u >= 0; --u) {
                if (u >= m) continue;
                const int64_t th = (k.b * T + ts + u) * p.H + k.h;
                const Tok x = k.tok(u);
                float4 dkp = z4, dqp = z4, ddp = z4;
                float dbp = 0.f;
#pragma unroll
                for (int j = 0; j < kRows; ++j) {
                    const float dor = x.dout[j];
                    const float4 X = DTPO ? mul4(St[u][j], x.d) : St[u][j];
                    const float pr = row_sum<LPR>(dot4(X, x.k));
                    const float e = x.beta * (x.v[j] - pr);
                    const float4 G = axpy4(p.scale * dor, x.q, Gd[j]);
                    const float gk = row_sum<LPR>(dot4(G, x.k));
                    if (k.on[j] && k.c == 0) a.dv[th * p.dv + k.r[j]] = x.beta * gk;
                    dbp += gk * (x.v[j] - pr);
                    const float bg = x.beta * gk;
                    dkp = add4(dkp, make_float4(e * G.x - bg * X.x, e * G.y - bg * X.y, e * G.z - bg * X.z,
                                                e * G.w - bg * X.w));
                    dqp = axpy4(p.scale * dor, St[u + 1][j], dqp);
                    if constexpr (!DTPO) {
                        ddp = add4(ddp, mul4(G, St[u][j]));
                        Gd[j] = make_float4(G.x * x.d.x - bg * x.k.x, G.y * x.d.y - bg * x.k.y,
                                            G.z * x.d.z - bg * x.k.z, G.w * x.d.w - bg * x.k.w);
                    } else {
                        const float4 dX = make_float4(G.x - bg * x.k.x, G.y - bg * x.k.y, G.z - bg * x.k.z,
                                                      G.w - bg * x.k.w);
                        ddp = add4(ddp, mul4(dX, St[u][j]));
                        Gd[j] = mul4(dX, x.d);
                    }
                }
                // the wave's sums over its rows: lanes c of the first row group
                dkp = group_sum4<LPR>(dkp);
                dqp = group_sum4<LPR>(dqp);
                if constexpr (CH) ddp = group_sum4<LPR>(ddp);
                // dbp is equal on the lanes of a row: sum over row groups only
                dbp = group_sum<LPR>(dbp);
                float das = 0.f;
                if constexpr (!CH) das = group_sum<LPR>(row_sum<LPR>(ddp.x + ddp.y + ddp.z + ddp.w));
                if (k.l < LPR) {
                    sh.vec[k.w][u][0][k.c] = dqp;
                    sh.vec[k.w][u][1][k.c] = dkp;
                    if constexpr (CH) sh.vec[k.w][u][2][k.c] = ddp;
                    if (k.l == 0) {
                        sh.sc[k.w][u][0] = dbp;
                        sh.sc[k.w][u][1] = das;
                    }
                }
            }
            __syncthreads();  // the run's partial sums complete
            // workgroup sums into its records: (token, vector, piece) jobs
            const int P4 = (int)(p.dk / 4);
            const int nv = CH ? 3 : 2;
            for (int e = tid; e < m * (nv * P4 + 1); e += kThreads) {
                const int u = e / (nv * P4 + 1), f = e % (nv * P4 + 1);
                float* rec = a.part + ((bl * nrb + k.rb) * T + ts + u) * RS;
                if (f == nv * P4) {
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) {
                        s0 += sh.sc[ww][u][0];
                        s1 += sh.sc[ww][u][1];
                    }
                    *reinterpret_cast<float4*>(rec + nv * p.dk) = make_float4(s0, s1, 0.f, 0.f);
                } else {
                    const int vi2 = f / P4, c4 = f % P4;
                    float4 s = sh.vec[0][u][vi2][c4];
#pragma unroll
                    for (int ww = 1; ww < 4; ++ww) s = add4(s, sh.vec[ww][u][vi2][c4]);
                    *reinterpret_cast<float4*>(rec + vi2 * p.dk + 4 * c4) = s;
                }
            }
        }
        __syncthreads();  // the staged run (and partial sums) read
        if (vi + 1 < NV) {
            k.stage_store(stg);
            __syncthreads();
        }
    }
    if (a.ds0) {
#pragma unroll
        for (int j = 0; j < kRows; ++j)
            if (k.on[j] && k.col) *reinterpret_cast<float4*>(a.ds0 + k.off(j)) = Gd[j];
    }
}

// The row blocks' partial records of every head-token summed into the
// outputs: record = [dq | dk | dalpha (channel gate) | dbeta, dalpha (scalar)]
__global__ void k_bwd_reduce(BwdProblem a, int nrb, int RS) {
    const Problem& p = a.p;
    const bool ch = p.gate == GDN_GATE_CHANNEL;
    const int nv = ch ? 3 : 2;
    const int P4 = RS / 4;
    const int64_t n = a.nbh * p.T * P4;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int f = (int)(i % P4);
        const int64_t ht = i / P4, bl = ht / p.T, t = ht % p.T, bh = a.bh0 + bl;
        const float* src = a.part + (bl * nrb * p.T + t) * RS + 4 * f;
        float4 s = *reinterpret_cast<const float4*>(src);
        for (int r = 1; r < nrb; ++r) s = add4(s, *reinterpret_cast<const float4*>(src + (int64_t)r * p.T * RS));
        const int64_t b = bh / p.H, h = bh % p.H;
        const int64_t th = (b * p.T + t) * p.H + h;
        const int e = 4 * f;
        if (e >= nv * p.dk) {
            a.dbeta[th] = s.x;
            if (!ch) a.dalpha[th] = s.y;
        } else {
            const int vi = e / (int)p.dk, c = e % (int)p.dk;
            float* dst = (vi == 0 ? a.dq : vi == 1 ? a.dk : a.dalpha) + th * p.dk + c;
            *reinterpret_cast<float4*>(dst) = s;
        }
    }
}

int lpr_for(int64_t dk) {
    const int64_t pieces = dk / 4;  // float4 pieces per row, 4 .. 32
    return pieces <= 4 ? 4 : pieces <= 8 ? 8 : pieces <= 16 ? 16 : 32;
}
// rows per workgroup, and the stride of the per-token records of partial sums
int rows_per_block(int64_t dk) { return 4 * (64 / lpr_for(dk)) * kRows; }
int record_stride(int64_t dk, int gate) { return (gate == GDN_GATE_CHANNEL ? 3 : 2) * (int)dk + 4; }

template <int DT, int LPR, bool CH, bool DTPO>
hipError_t launch4(const BwdProblem& a, hipStream_t st) {
    constexpr int RB = Bwd<DT, LPR, CH, DTPO>::RB;
    const int nrb = (int)((a.p.dv + RB - 1) / RB);
    const int64_t grid = a.nbh * nrb;
    static_assert(RB == 4 * (64 / LPR) * kRows, "rows_per_block");
    hipLaunchKernelGGL((k_backward<DT, LPR, CH, DTPO>), dim3((unsigned)grid), dim3(kThreads), 0, st, a,
                       nrb, record_stride(a.p.dk, a.p.gate));
    return hipGetLastError();
}

template <int DT, int LPR>
hipError_t launch_lpr(const BwdProblem& a, hipStream_t st) {
    const bool ch = a.p.gate == GDN_GATE_CHANNEL, dtp = a.p.order == GDN_DECAY_THEN_PREDICT;
    if (ch) return dtp ? launch4<DT, LPR, true, true>(a, st) : launch4<DT, LPR, true, false>(a, st);
    return dtp ? launch4<DT, LPR, false, true>(a, st) : launch4<DT, LPR, false, false>(a, st);
}

template <int DT>
hipError_t launch_dt(const BwdProblem& a, hipStream_t st) {
    switch (lpr_for(a.p.dk)) {
        case 4: return launch_lpr<DT, 4>(a, st);
        case 8: return launch_lpr<DT, 8>(a, st);
        case 16: return launch_lpr<DT, 16>(a, st);
        default: return launch_lpr<DT, 32>(a, st);
    }
}

}  // namespace


// The workspace of a launch: per (batch, head) pair the checkpoints (the
// state at every run start) and the records of the row blocks' sums.  Larger
// batches run in groups of pairs, one launch pair (kernel and reduction) per
// group, so that the workspace stays within kWsCap however large the batch.
constexpr size_t kWsCap = size_t(8) << 30;
size_t ckpt_bytes_per_head(int64_t T, int64_t dk, int64_t dv) {
    return sizeof(float) * (size_t)((T + kSub - 1) / kSub) * (size_t)(dk * dv);
}
size_t part_bytes_per_head(int64_t T, int64_t dk, int64_t dv, int gate) {
    const int RB = rows_per_block(dk);
    const int64_t nrb = (dv + RB - 1) / RB;
    return sizeof(float) * (size_t)nrb * (size_t)T * (size_t)record_stride(dk, gate);
}
int64_t heads_per_launch(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate) {
    const size_t per = ckpt_bytes_per_head(T, dk, dv) + part_bytes_per_head(T, dk, dv, gate);
    const int64_t g = per > 0 ? (int64_t)(kWsCap / per) : B * H;
    return std::max<int64_t>(1, std::min<int64_t>(B * H, g));
}

size_t backward_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate) {
    return align256(ckpt_bytes_per_head(T, dk, dv) * (size_t)heads_per_launch(B, T, H, dk, dv, gate));
}

size_t backward_workspace(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate) {
    const size_t part = part_bytes_per_head(T, dk, dv, gate) * (size_t)heads_per_launch(B, T, H, dk, dv, gate);
    return backward_ckpt_bytes(B, T, H, dk, dv, gate) + align256(part);
}

hipError_t backward(const BwdProblem& a, hipStream_t st) {
    const Problem& p = a.p;
    const int RB = rows_per_block(p.dk);
    const int nrb = (int)((p.dv + RB - 1) / RB);
    const int RS = record_stride(p.dk, p.gate);
    const int64_t BH = p.B * p.H, gsz = heads_per_launch(p.B, p.T, p.H, p.dk, p.dv, p.gate);
    for (int64_t bh0 = 0; bh0 < BH; bh0 += gsz) {
        BwdProblem g = a;
        g.bh0 = bh0;
        g.nbh = std::min<int64_t>(gsz, BH - bh0);
        prof_begin(p.timer, "k_backward", st);
        hipError_t e = p.dtype == GDN_BF16 ? launch_dt<1>(g, st) : launch_dt<0>(g, st);
        prof_end(p.timer, st);
        if (e != hipSuccess) return e;
        const int64_t n = g.nbh * p.T * (RS / 4);
        if (n == 0) continue;
        const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
        prof_begin(p.timer, "k_bwd_reduce", st);
        hipLaunchKernelGGL(k_bwd_reduce, dim3((unsigned)blocks), dim3(256), 0, st, g, nrb, RS);
        prof_end(p.timer, st);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gdn
