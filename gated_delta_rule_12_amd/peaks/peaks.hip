// Achievable-peak probes for the benchmark's roofline: a plain device copy
// (HBM read + write streaming) and a loop of independent bf16 MFMAs (matrix
// core issue rate).  Not part of the gated-delta path; built into a library
// of their own and called only by the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyUnroll = 4;

// Each thread moves kCopyUnroll 16-byte pieces per grid-stride step: all
// loads first, then all stores.
__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                              int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256 * kCopyUnroll;
    for (int64_t base = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x; base < n16; base += stride) {
        u32x4 r[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + 256 * u;
            if (i < n16) r[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + 256 * u;
            if (i < n16) __builtin_nontemporal_store(r[u], dst + i);
        }
    }
}

// Eight independent accumulator chains per wave of bf16 MFMAs (SHAPE 0:
// 16x16x32, SHAPE 1: 32x32x16, 16384 and 32768 flop each); the operands
// depend on the lane so that nothing folds, and the sums are written out so
// that nothing is dropped.  Lane 0 of every wave also records the shader-clock
// cycles (s_memtime) and the 100 MHz real-time ticks (s_memrealtime) its loop
// took, into clk[2 * wave] and clk[2 * wave + 1].
template <int SHAPE>
__global__ __launch_bounds__(256) void k_mfma(float* out, unsigned long long* clk, int iters) {
    typedef float acc_t __attribute__((ext_vector_type(SHAPE ? 16 : 4)));
    const int l = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.0078125f * ((l + e) & 7));
        b[e] = (__bf16)(0.5f - 0.0078125f * ((l * 3 + e) & 7));
    }
    acc_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < (SHAPE ? 16 : 4); ++i) acc[j][i] = 0.f;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (SHAPE) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
            else acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < (SHAPE ? 16 : 4); ++i) s += acc[j][i];
    const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
    if (l == 0 && clk) {
        const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
        clk[2 * wave] = c1 - c0;
        clk[2 * wave + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" {

// Copies n_bytes (a multiple of 16, 16-byte aligned buffers) from src to dst
// on the stream.  0 on success, -1 on bad arguments, -5 on a launch error.
int gdn_peak_copy(const void* src, void* dst, size_t n_bytes, void* stream) {
    if (!src || !dst || n_bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16) return -1;
    const int64_t n16 = (int64_t)(n_bytes / 16);
    if (n16 == 0) return 0;
    int64_t blocks = (n16 + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_copy, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// blocks x 256 threads, each wave issuing 8 * iters bf16 MFMAs of shape 0
// (16 x 16 x 32) or 1 (32 x 32 x 16); out holds blocks * 256 floats, clk
// (may be null) 2 * 4 * blocks counters (cycles and 100 MHz ticks per wave).
int gdn_peak_mfma(float* out, unsigned long long* clk, int shape, int blocks, int iters, void* stream) {
    if (!out || blocks <= 0 || iters <= 0 || (shape != 0 && shape != 1)) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (shape)
        hipLaunchKernelGGL(k_mfma<1>, dim3((unsigned)blocks), dim3(256), 0, st, out, clk, iters);
    else
        hipLaunchKernelGGL(k_mfma<0>, dim3((unsigned)blocks), dim3(256), 0, st, out, clk, iters);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
