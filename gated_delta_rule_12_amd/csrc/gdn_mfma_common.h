// Pieces shared by the MFMA kernel files (gdn_mfma.hip, the chunked forward;
// gdn_bwd_chunk.hip, the chunked backward): vector types, the fp32 MFMA and
// its operand layout, a wave prefix sum, and the in-LDS inverse of the unit
// lower-triangular UT system.  Internal to libgdn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int C = 64;          // chunk length of the MFMA kernels
constexpr int kThreads = 256;  // four waves

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Loads and stores through the global address space.  Where the compiler
// cannot prove that a generic pointer is global it emits flat instructions,
// which count on the LDS counter too, so that every later wait for an LDS
// access (each barrier included) also waits for them to come back from
// memory; these casts keep such accesses global.
template <typename V>
__device__ __forceinline__ V ld_g(const void* p) {
    return *(const __attribute__((address_space(1))) V*)p;
}
template <typename V>
__device__ __forceinline__ void st_g(void* p, const V& x) {
    *(__attribute__((address_space(1))) V*)p = x;
}

// D += A B on a 16 x 16 x 4 fp32 tile.  Lane l = 16 g + c supplies A[c][g]
// and B[g][c]; the accumulator holds D[4 g + r][c] in element r.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// The UT inverse T = (I + A)^{-1} in fp32, in place in LDS.  On entry AT
// (C x C, row stride C + 4) holds A's strictly lower off-diagonal blocks
// transposed (block (i, k) at rows of block k, columns of block i) and A's
// diagonal blocks in place, zero on and above their diagonal; on return the
// diagonal blocks and the lower triangle hold T (unit lower triangular, exact
// zeros above the diagonal inside the diagonal blocks) and the upper
// off-diagonal blocks still hold A transposed.  Called by all threads of a
// four-wave group (it contains workgroup barriers; tid is the thread's index
// in its group of 256, so two groups of one workgroup can each invert their
// own tile, passing the same barriers).  The strictly lower
// off-diagonal blocks are free until the off-diagonal phase fills them, so
// the diagonal phase keeps each wave's power of N in one of them (row stride
// C + 4 spreads a lane group's column writes over every bank).
//   diagonal block w: (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8)
//     (N^16 = 0), three rounds of P <- P P, X <- X + X P on fp32 MFMA;
//     accumulators (lane: column c16, rows 4 g4 + i) serve as B operands as
//     they stand (instruction s contracts the indices 4G + s, G = lane / 16);
//   off-diagonal blocks by distance d: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.
__device__ __forceinline__ void ut_inverse_lds(float* AT, int tid) {
    constexpr int LDA = C + 4;
    const int w = tid >> 6, l = tid & 63, g4 = l >> 4, c16 = l & 15;
    {
        float* Xb = &AT[(16 * w) * LDA + 16 * w];
        // scratch block (1, 0), (2, 0), (3, 0) or (3, 1) for waves 0 .. 3
        float* Pw = &AT[(16 * (w < 3 ? w + 1 : 3)) * LDA + 16 * (w < 3 ? 0 : 1)];
        f32x4 pm, xm;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pm[r] = -Xb[(4 * g4 + r) * LDA + c16];
            xm[r] = (4 * g4 + r == c16 ? 1.f : 0.f) + pm[r];
        }
#pragma unroll
        for (int round = 0; round < 3; ++round) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Pw[(4 * g4 + r) * LDA + c16] = pm[r];
            f32x4 np = zero4();
#pragma unroll
            for (int q = 0; q < 4; ++q) np = mfma_f32(Pw[c16 * LDA + 4 * g4 + q], pm[q], np);
            pm = np;
#pragma unroll
            for (int r = 0; r < 4; ++r) Xb[(4 * g4 + r) * LDA + c16] = xm[r];
            f32x4 nx = xm;
#pragma unroll
            for (int q = 0; q < 4; ++q) nx = mfma_f32(Xb[c16 * LDA + 4 * g4 + q], pm[q], nx);
            xm = nx;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Xb[(4 * g4 + r) * LDA + c16] = xm[r];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        if (w < 4 - d) {
            const int jb = w, ib = w + d;
            f32x4 X = zero4();
            for (int kb = jb; kb < ib; ++kb) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    X = mfma_f32(AT[(16 * kb + 4 * g4 + q) * LDA + 16 * ib + c16],   // A_ib,kb (transposed)
                                 AT[(16 * kb + 4 * g4 + q) * LDA + 16 * jb + c16], X);  // T_kb,jb
            }
            f32x4 Tij = zero4();
#pragma unroll
            for (int q = 0; q < 4; ++q) Tij = mfma_f32(AT[(16 * ib + c16) * LDA + 16 * ib + 4 * g4 + q], X[q], Tij);
#pragma unroll
            for (int r = 0; r < 4; ++r) AT[(16 * ib + 4 * g4 + r) * LDA + 16 * jb + c16] = -Tij[r];
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace gdn
