// Throughput probes (libfa_probe.so), not part of the attention library:
//   * the rate the bf16 matrix cores sustain on this GPU under a pure MFMA
//     load, and the core clock while they do -- bench.py reports it beside
//     the published 2.5 PFLOP/s peak as a measured denominator;
//   * the chip-wide rate of float32 buffer atomic adds to distinct
//     addresses -- the bound of the backward's atomic-dQ mode;
//   * the VALU cost of v_exp_f32 against v_fma_f32 (is the exponential a
//     separate pipe, and what would a polynomial 2^x on the FMA path cost).
//
// Each wave runs `iters` rounds of 16 v_mfma_f32_32x32x16_bf16 on four
// independent accumulator chains (no memory traffic inside the loop), so the
// issue rate is the matrix cores' own.  Wave 0 of workgroup 0 records
// s_memtime (core clock) and s_memrealtime (a fixed 100 MHz reference)
// before and after its loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) probe_mfma_kernel(float* out, uint64_t* clocks, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * lane + 0.01f * i);
        b[i] = (__bf16)(0.01f * i);
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the products live
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clocks[0] = t1 - t0;
        clocks[1] = r1 - r0;
    }
}

// out: grid * 256 floats; clocks: 2 uint64 (core cycles, 100 MHz ticks of
// wave 0 of workgroup 0).  Returns 0, or -7 if the launch failed.
extern "C" int fa_probe_mfma_launch(void* out, void* clocks, int grid, int iters, void* stream) {
    if (!out || !clocks || grid <= 0 || iters <= 0) return -1;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (float*)out,
                       (uint64_t*)clocks, iters);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// FLOPs one launch executes: grid * 4 waves * iters * 16 MFMAs * 32768.
extern "C" double fa_probe_mfma_flops(int grid, int iters) {
    return (double)grid * 4.0 * (double)iters * 16.0 * 32768.0;
}

// float32 atomic adds: each lane of workgroup w adds 1 to element
// (w * ITERS + i) * 256 + threadIdx.x for i < ITERS, so every add of a
// launch goes to its own address and a wave's 64 lanes to 256 contiguous
// bytes.  `buf` holds grid * kAtomicIters * 256 floats.
constexpr int kAtomicIters = 64;

__global__ void __launch_bounds__(256) probe_atomic_kernel(float* buf, uint32_t n) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(buf, (short)0, n * 4u, 0x00020000);
    for (int i = 0; i < kAtomicIters; ++i) {
        const uint32_t idx = (blockIdx.x * kAtomicIters + i) * 256u + threadIdx.x;
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(1.0f, r, idx * 4u, 0, 0);
    }
}

// buf: at least fa_probe_atomic_elems(grid) floats.  Returns 0, -1 for bad
// arguments, -7 if the launch failed.
extern "C" long fa_probe_atomic_elems(int grid) { return (long)grid * kAtomicIters * 256; }

extern "C" int fa_probe_atomic_launch(void* buf, int grid, void* stream) {
    if (!buf || grid <= 0 || fa_probe_atomic_elems(grid) * 4 > 0xffffffffL) return -1;
    hipLaunchKernelGGL(probe_atomic_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (float*)buf,
                       (uint32_t)fa_probe_atomic_elems(grid));
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// VALU issue costs: each lane runs 8 independent chains for kValuIters
// steps; a step is NE x (v_exp_f32 then one add) and NF x v_fma_f32 per
// chain.  With 8 waves per SIMD (grid = 32 workgroups per CU) the time per
// wave-step and SIMD gives the cycles each instruction holds the pipe.
constexpr int kValuIters = 2048;

template <int NE, int NF>
__global__ void __launch_bounds__(256) probe_valu_kernel(float* out, float a) {
    float x[8], y[8];
    for (int i = 0; i < 8; ++i) {
        x[i] = -0.001f * (float)(threadIdx.x + i);
        y[i] = 0.5f + 0.01f * (float)i;
    }
    for (int it = 0; it < kValuIters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int e = 0; e < NE; ++e) x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
#pragma unroll
            for (int f = 0; f < NF; ++f) y[i] = fmaf(y[i], a, 0.25f);
        }
    }
    float sum = 0.f;
    for (int i = 0; i < 8; ++i) sum += x[i] + y[i];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

// variant 0: exp + add; 1: two FMAs; 2: exp + add and two FMAs.  out: grid *
// 256 floats.  Returns the instruction counts of one wave through *n_exp,
// *n_other (adds and FMAs), 0, or -1 / -7.
extern "C" int fa_probe_valu_launch(void* out, int grid, int variant, void* stream, long* n_exp, long* n_other) {
    if (!out || grid <= 0 || variant < 0 || variant > 2 || !n_exp || !n_other) return -1;
    const long steps = (long)kValuIters * 8;
    hipStream_t s = (hipStream_t)stream;
    if (variant == 0) hipLaunchKernelGGL((probe_valu_kernel<1, 0>), dim3(grid), dim3(256), 0, s, (float*)out, 0.999f);
    if (variant == 1) hipLaunchKernelGGL((probe_valu_kernel<0, 2>), dim3(grid), dim3(256), 0, s, (float*)out, 0.999f);
    if (variant == 2) hipLaunchKernelGGL((probe_valu_kernel<1, 2>), dim3(grid), dim3(256), 0, s, (float*)out, 0.999f);
    *n_exp = variant == 1 ? 0 : steps;
    *n_other = variant == 0 ? steps : variant == 1 ? 2 * steps : 3 * steps;
    return hipGetLastError() == hipSuccess ? 0 : -7;
}
