// peak.hip -- matrix-core throughput microbenchmark (a measurement aid, not
// part of the attention library: it is built into its own libfa_peak.so).
//
// Every wave runs a loop of independent 32x32 MFMA chains on operands held in
// registers: no memory traffic inside the loop, so the launch's rate is the
// matrix cores' own, at whatever clock the board holds for this work.  The
// operands are zeros, a constant or pseudo-random values near N(0, 1): on a
// power-capped board the switching activity of the operands sets the clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 pk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pk_f32x16 __attribute__((ext_vector_type(16)));
typedef float pk_f32x4 __attribute__((ext_vector_type(4)));

namespace {

// A value near N(0, 1) from a counter: an integer mix of the counter (xorshift
// and multiply rounds), then the centred, scaled sum of its four bytes
// (Irwin-Hall with n = 4, variance 4 * (256^2 - 1) / 12).
__device__ inline float near_normal(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    const float u = (float)(x & 0xffu) + (float)((x >> 8) & 0xffu) + (float)((x >> 16) & 0xffu) + (float)(x >> 24);
    return (u - 510.f) / 147.8f;
}

template <int mode>
__device__ inline float operand(uint32_t counter, float constant) {
    if constexpr (mode == 0) return 0.f;
    else if constexpr (mode == 1) return constant;
    else return near_normal(counter);
}

constexpr int kChains = 4;  // independent accumulators per wave

// bf16: v_mfma_f32_32x32x16_bf16, 32768 FLOP per wave instruction.  (The
// operand set-up is unrolled and the mode a template argument: built with a
// run-time mode and run-time element indices, the set-up compiled to select
// chains and cost about 2 ms per launch of 4096 workgroups, more than short
// loops themselves.)
template <int mode>
__global__ __launch_bounds__(256) void peak_bf16_kernel(int iters, float *out) {
    const uint32_t t = threadIdx.x + blockIdx.x * 256u;
    pk_bf16x8 a[kChains], b[kChains];
#pragma unroll
    for (int s = 0; s < kChains; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[s][i] = (__bf16)operand<mode>(t * 64u + s * 8u + i, 0.5f);
            b[s][i] = (__bf16)operand<mode>(0x9e3779b9u ^ (t * 64u + s * 8u + i), 0.25f);
        }
    pk_f32x16 c[kChains] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < kChains; ++s)
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(s + j) % kChains], b[s], c[j], 0, 0, 0);
    }
    float r = 0.f;
    for (int j = 0; j < kChains; ++j)
        for (int i = 0; i < 16; ++i) r += c[j][i];
    out[t] = r;  // keeps the chains live
}

// bf16 16x16: v_mfma_f32_16x16x32_bf16, 16384 FLOP per wave instruction
// (the same operand registers per lane as the 32x32x16 form, a quarter of
// its accumulator registers).
template <int mode>
__global__ __launch_bounds__(256) void peak_bf16_16_kernel(int iters, float *out) {
    const uint32_t t = threadIdx.x + blockIdx.x * 256u;
    pk_bf16x8 a[kChains], b[kChains];
#pragma unroll
    for (int s = 0; s < kChains; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[s][i] = (__bf16)operand<mode>(t * 64u + s * 8u + i, 0.5f);
            b[s][i] = (__bf16)operand<mode>(0x9e3779b9u ^ (t * 64u + s * 8u + i), 0.25f);
        }
    pk_f32x4 c[kChains] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < kChains; ++s)
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(s + j) % kChains], b[s], c[j], 0, 0, 0);
    }
    float r = 0.f;
    for (int j = 0; j < kChains; ++j)
        for (int i = 0; i < 4; ++i) r += c[j][i];
    out[t] = r;
}

// fp32: v_mfma_f32_32x32x2_f32, 4096 FLOP per wave instruction.
template <int mode>
__global__ __launch_bounds__(256) void peak_f32_kernel(int iters, float *out) {
    const uint32_t t = threadIdx.x + blockIdx.x * 256u;
    float a[kChains], b[kChains];
#pragma unroll
    for (int s = 0; s < kChains; ++s) {
        a[s] = operand<mode>(t * 64u + s, 0.5f);
        b[s] = operand<mode>(0x9e3779b9u ^ (t * 64u + s), 0.25f);
    }
    pk_f32x16 c[kChains] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < kChains; ++s)
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                c[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[(s + j) % kChains], b[s], c[j], 0, 0, 0);
    }
    float r = 0.f;
    for (int j = 0; j < kChains; ++j)
        for (int i = 0; i < 16; ++i) r += c[j][i];
    out[t] = r;
}

}  // namespace

extern "C" {

// FLOP one launch of fa_peak_mfma performs (0 for invalid arguments).
double fa_peak_mfma_flop(int dtype, int blocks, int iters) {
    if (dtype < 0 || dtype > 2 || blocks <= 0 || iters <= 0) return 0.0;
    const double per_instr = dtype == 1 ? 32768.0 : dtype == 2 ? 16384.0 : 4096.0;
    return (double)blocks * 4 /* waves */ * (double)iters * kChains * kChains * per_instr;
}

// Enqueue one launch on `stream`: `blocks` workgroups of 4 waves, each wave
// running `iters` rounds of kChains x kChains MFMAs of the dtype (0: fp32
// 32x32x2, 1: bf16 32x32x16, 2: bf16 16x16x32) on operands `mode` (0 zeros, 1 constant,
// 2 near N(0, 1)).  out: device buffer of blocks * 256 floats (overwritten).
// Returns 0, -1 (invalid argument) or -5 (launch refused).
int fa_peak_mfma(int dtype, int mode, int blocks, int iters, float *out, hipStream_t stream) {
    if (dtype < 0 || dtype > 2 || mode < 0 || mode > 2 || blocks <= 0 || blocks > (1 << 22) || iters <= 0 ||
        !out)
        return -1;
    const dim3 grid((unsigned)blocks), block(256);
    if (dtype == 1) {
        if (mode == 0) hipLaunchKernelGGL(peak_bf16_kernel<0>, grid, block, 0, stream, iters, out);
        else if (mode == 1) hipLaunchKernelGGL(peak_bf16_kernel<1>, grid, block, 0, stream, iters, out);
        else hipLaunchKernelGGL(peak_bf16_kernel<2>, grid, block, 0, stream, iters, out);
    } else if (dtype == 2) {
        if (mode == 0) hipLaunchKernelGGL(peak_bf16_16_kernel<0>, grid, block, 0, stream, iters, out);
        else if (mode == 1) hipLaunchKernelGGL(peak_bf16_16_kernel<1>, grid, block, 0, stream, iters, out);
        else hipLaunchKernelGGL(peak_bf16_16_kernel<2>, grid, block, 0, stream, iters, out);
    } else {
        if (mode == 0) hipLaunchKernelGGL(peak_f32_kernel<0>, grid, block, 0, stream, iters, out);
        else if (mode == 1) hipLaunchKernelGGL(peak_f32_kernel<1>, grid, block, 0, stream, iters, out);
        else hipLaunchKernelGGL(peak_f32_kernel<2>, grid, block, 0, stream, iters, out);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
