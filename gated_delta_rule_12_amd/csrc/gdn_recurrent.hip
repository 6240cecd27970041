// Token-by-token gated delta rule on the GPU (gdn_recurrent_ref).
//
// The "fused recurrent" form the DeltaNet illustrated notes compare the
// chunkwise algorithm against (WY/UT section, speed comparison): the state
// stays on chip for the whole sequence.  One lane owns one row of S (a value
// dimension) with its dk entries in registers, so the prediction S k, the
// correction and the read S q are lane-local dot products; the current
// token's k, q and gate are broadcast from LDS.  One 64-lane wave per
// (batch, head, 64-row block).
//
// Per token (state rows r, key channels c):
//   predict-then-decay:  p = S k;  S = S D + beta (v - p) k^T
//   decay-then-predict:  S = S D;  p = S k;  S = S + beta (v - p) k^T
//   o = scale * S q
#include "gdn_internal.h"
#include "../../include/gdn.h"

namespace gdn {
namespace {

constexpr int kLanes = 64;
constexpr int kStage = 16;  // tokens staged in LDS per barrier

template <int DT, int DK>
__global__ __launch_bounds__(kLanes) void k_recurrent(Problem p) {
    const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int dv = (int)p.dv;
    const int r = rb * kLanes + lane;
    const bool active = r < dv;
    const int64_t H = p.H, T = p.T, bh = (int64_t)b * H + h;
    const bool channel = p.gate == GDN_GATE_CHANNEL;
    const bool dtp = p.order == GDN_DECAY_THEN_PREDICT;

    __shared__ float ks[kStage][DK];
    __shared__ float qs[kStage][DK];
    __shared__ float as[kStage][DK];
    __shared__ float sc[kStage][2];  // scalar alpha, beta

    float S[DK];
#pragma unroll
    for (int c = 0; c < DK; ++c)
        S[c] = (active && p.s0) ? p.s0[(bh * dv + r) * DK + c] : 0.f;

    for (int64_t tb = 0; tb < T; tb += kStage) {
        const int n = (int)((T - tb) < kStage ? (T - tb) : kStage);
        __syncthreads();
        for (int e = lane; e < n * DK; e += kLanes) {
            const int j = e / DK, c = e - (e / DK) * DK;
            const int64_t row = (b * T + tb + j) * H + h;
            ks[j][c] = gdn_ld<DT>(p.k, row * DK + c);
            qs[j][c] = gdn_ld<DT>(p.q, row * DK + c);
            if (channel) as[j][c] = p.alpha[row * DK + c];
        }
        for (int j = lane; j < n; j += kLanes) {
            const int64_t row = (b * T + tb + j) * H + h;
            sc[j][0] = channel ? 1.f : p.alpha[row];
            sc[j][1] = p.beta[row];
        }
        __syncthreads();
        for (int j = 0; j < n; ++j) {
            const int64_t row = (b * T + tb + j) * H + h;
            const float vr = active ? gdn_ld<DT>(p.v, row * dv + r) : 0.f;
            const float a_s = sc[j][0], bt = sc[j][1];
            if (dtp) {
#pragma unroll
                for (int c = 0; c < DK; ++c) S[c] *= channel ? as[j][c] : a_s;
            }
            float pred = 0.f;
#pragma unroll
            for (int c = 0; c < DK; ++c) pred += S[c] * ks[j][c];
            const float e = bt * (vr - pred);
            if (!dtp) {
#pragma unroll
                for (int c = 0; c < DK; ++c) S[c] = S[c] * (channel ? as[j][c] : a_s) + e * ks[j][c];
            } else {
#pragma unroll
                for (int c = 0; c < DK; ++c) S[c] += e * ks[j][c];
            }
            float o = 0.f;
#pragma unroll
            for (int c = 0; c < DK; ++c) o += S[c] * qs[j][c];
            if (active) p.out[row * dv + r] = p.scale * o;
        }
    }
    if (active && p.s_out) {
#pragma unroll
        for (int c = 0; c < DK; ++c) p.s_out[(bh * dv + r) * DK + c] = S[c];
    }
}

template <int DT>
hipError_t launch_dt(const Problem& p, hipStream_t st) {
    dim3 grid((unsigned)((p.dv + kLanes - 1) / kLanes), (unsigned)p.H, (unsigned)p.B);
    switch (p.dk) {
#define GDN_CASE(D) \
    case D: hipLaunchKernelGGL((k_recurrent<DT, D>), grid, dim3(kLanes), 0, st, p); break;
        GDN_CASE(16) GDN_CASE(32) GDN_CASE(48) GDN_CASE(64)
        GDN_CASE(80) GDN_CASE(96) GDN_CASE(112) GDN_CASE(128)
#undef GDN_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t recurrent_forward(const Problem& p, hipStream_t st) {
    prof_begin(p.timer, "k_recurrent", st);
    hipError_t e = p.dtype == GDN_BF16 ? launch_dt<1>(p, st) : launch_dt<0>(p, st);
    prof_end(p.timer, st);
    return e;
}

}  // namespace gdn
