// One-token step of the gated delta rule on a persistent state
// (gdn_decode_step).
//
// Generation runs the fixed-size-state recurrence: each new token updates
// the dv x dk state once and reads it once, at a cost that does not grow
// with the history (DeltaNet illustrated notes, the part on linear attention
// as an RNN; the per-token update is that of the Gated DeltaNet
// GPU-parallelisation blog, section 1.2, in the notes' dv x dk orientation).
//
// Given the token's k, q, gate and beta, the rows r of S (value dimensions)
// are independent:
//   predict-then-decay:  p_r = S_r . k;  S'_r = S_r D + beta (v_r - p_r) k
//   decay-then-predict:  S_r <- S_r D;  p_r = S_r . k;  S'_r = S_r + beta (v_r - p_r) k
//   o_r = scale S'_r . q
// so the step is a stream over S: 8 dk dv bytes of HBM traffic per head (read
// and write), against 4 flops per element.  LPR lanes hold one row as float4
// pieces (16-byte loads and stores; a wave covers 64 / LPR whole rows, which
// are contiguous in memory), the two dot products are reduced across the
// row's lanes by vector-ALU butterflies (row_sum), and each thread keeps kRows rows in flight so
// that enough bytes are outstanding per CU to cover the HBM latency.  The
// state is read and written with non-temporal hints: each byte is touched
// once per step, and keeping it out of the caches took a quarter less time
// than cached accesses.
//
// With the prologue (gdn_decode_step_raw) the kernel also forms the step's
// inputs from the model's raw projections, as the DeltaNet block does before
// the recurrence (DeltaNet illustrated notes, block description: per-head L2
// normalisation of q and k; the gates through a sigmoid): q <- q / |q|,
// k <- k / |k| (a zero vector stays zero), alpha <- sigmoid(alpha),
// beta <- sigmoid(beta), all in fp32.  The row's lanes hold the head's q and
// k in float4 pieces, so each norm is one more reduction over them.
#include "gdn_internal.h"
#include "../../include/gdn.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;  // rows per thread
typedef float f32x4v __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float dot4(const float4& a, const float4& b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}


// grid (row blocks, H, B); block: 4 waves, wave w covers rows
// rb RB + (j 4 + w) RPW + l / LPR for j < kRows
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

template <int LPR>
__device__ __forceinline__ float4 l2_normalised(const float4& x) {
    const float n2 = row_sum<LPR>(dot4(x, x));
    const float r = n2 > 0.f ? 1.f / __fsqrt_rn(n2) : 0.f;
    return make_float4(x.x * r, x.y * r, x.z * r, x.w * r);
}

template <int DT, int LPR, bool PRO>
__global__ __launch_bounds__(kThreads) void k_decode(Problem p) {
    constexpr int RPW = 64 / LPR;            // rows per wave and pass
    constexpr int RB = 4 * RPW * kRows;      // rows per block
    const int64_t b = blockIdx.z, h = blockIdx.y, H = p.H;
    const int64_t bh = b * H + h;
    const int dk = (int)p.dk, dv = (int)p.dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int c = l % LPR;                   // float4 piece of the row
    const bool col = 4 * c < dk;
    const bool channel = p.gate == GDN_GATE_CHANNEL;
    const bool dtp = p.order == GDN_DECAY_THEN_PREDICT;

    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 k4 = col ? ld4<DT>(p.k, bh * dk + 4 * c) : z4;
    float4 q4 = col ? ld4<DT>(p.q, bh * dk + 4 * c) : z4;
    float4 d4;
    if (channel) {
        d4 = col ? *reinterpret_cast<const float4*>(p.alpha + bh * dk + 4 * c) : z4;
        if (PRO && col) d4 = make_float4(sigmoid(d4.x), sigmoid(d4.y), sigmoid(d4.z), sigmoid(d4.w));
    } else {
        float a = p.alpha[bh];
        if (PRO) a = sigmoid(a);
        d4 = make_float4(a, a, a, a);
    }
    float beta = p.beta[bh];
    if (PRO) {
        k4 = l2_normalised<LPR>(k4);
        q4 = l2_normalised<LPR>(q4);
        beta = sigmoid(beta);
    }

    int r[kRows];
    bool on[kRows];
    float4 s[kRows];
    float vr[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        r[j] = blockIdx.x * RB + (j * 4 + w) * RPW + l / LPR;
        on[j] = r[j] < dv;
        const int64_t off = (bh * dv + r[j]) * dk + 4 * c;
        s[j] = z4;
        if (on[j] && col && p.s0) {
            const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p.s0 + off));
            s[j] = make_float4(x[0], x[1], x[2], x[3]);
        }
        vr[j] = on[j] ? gdn_ld<DT>(p.v, bh * dv + r[j]) : 0.f;
    }
    float pr[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        if (dtp) s[j] = make_float4(s[j].x * d4.x, s[j].y * d4.y, s[j].z * d4.z, s[j].w * d4.w);
        pr[j] = dot4(s[j], k4);
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) pr[j] = row_sum<LPR>(pr[j]);
    float o[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const float e = beta * (vr[j] - pr[j]);
        float4 n;
        if (dtp) {
            n = make_float4(s[j].x + e * k4.x, s[j].y + e * k4.y, s[j].z + e * k4.z, s[j].w + e * k4.w);
        } else {
            n = make_float4(s[j].x * d4.x + e * k4.x, s[j].y * d4.y + e * k4.y,
                            s[j].z * d4.z + e * k4.z, s[j].w * d4.w + e * k4.w);
        }
        s[j] = n;
        o[j] = dot4(n, q4);
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) o[j] = row_sum<LPR>(o[j]);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        if (on[j] && col) {
            const f32x4v x = {s[j].x, s[j].y, s[j].z, s[j].w};
            __builtin_nontemporal_store(x, reinterpret_cast<f32x4v*>(p.s_out + (bh * dv + r[j]) * dk + 4 * c));
        }
        if (on[j] && c == 0) p.out[bh * dv + r[j]] = p.scale * o[j];
    }
}

template <int DT, int LPR, bool PRO>
hipError_t launch_lpr(const Problem& p, hipStream_t st) {
    constexpr int RB = 4 * (64 / LPR) * kRows;
    const dim3 grid((unsigned)((p.dv + RB - 1) / RB), (unsigned)p.H, (unsigned)p.B);
    hipLaunchKernelGGL((k_decode<DT, LPR, PRO>), grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <int DT, bool PRO>
hipError_t launch_dt(const Problem& p, hipStream_t st) {
    const int64_t pieces = p.dk / 4;  // float4 pieces per row, 4 .. 32
    if (pieces <= 4) return launch_lpr<DT, 4, PRO>(p, st);
    if (pieces <= 8) return launch_lpr<DT, 8, PRO>(p, st);
    if (pieces <= 16) return launch_lpr<DT, 16, PRO>(p, st);
    return launch_lpr<DT, 32, PRO>(p, st);
}

}  // namespace

hipError_t decode_step(const Problem& p, bool prologue, hipStream_t st) {
    prof_begin(p.timer, "k_decode", st);
    hipError_t e;
    if (prologue)
        e = p.dtype == GDN_BF16 ? launch_dt<1, true>(p, st) : launch_dt<0, true>(p, st);
    else
        e = p.dtype == GDN_BF16 ? launch_dt<1, false>(p, st) : launch_dt<0, false>(p, st);
    prof_end(p.timer, st);
    return e;
}

}  // namespace gdn
