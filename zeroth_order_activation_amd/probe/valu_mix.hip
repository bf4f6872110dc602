// Issue-rate probes for the plain vector ALU (measurement only; not part of the
// estimator library).  Each kernel runs a register-only loop of one instruction
// mix; the build counts the vector instructions of each loop body from this
// file's own gfx950 assembly, and the benchmark divides
//     instructions x 64 lanes x waves x iterations
// by the measured time: the sustained lane-op rate of that mix on the chip.
//
//   mix 0  fp32 FMA (eight independent chains)
//   mix 1  v_mad_u64_u32 (the 32x32->64 products of Philox), one xor each
//   mix 2  the transcendentals of Box-Muller (log2, sqrt, sin, cos), one product
//          per four
//   mix 3  the LM-head estimator's per-draw arithmetic for 8 channel quads per
//          lane: Philox4x32-10 (the counter's token, draw and layer uniform),
//          Box-Muller, the degree-4 expm1 polynomial weighted by p, and the
//          running sums of r a -- without the per-draw reduction, barrier and
//          reward, and without memory traffic.
//   mix 4  v_mfma_f32_32x32x16_bf16 only: eight independent accumulators per
//          wave, operands taken from `in` (the sustained matrix-core rate with
//          non-trivial data; rated in flops, not lane-ops).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dust_device.hpp"

namespace {

constexpr int kNT = 256;

__global__ void __launch_bounds__(kNT) mix_fma_kernel(const float* __restrict__ in, float* __restrict__ out, int iters) {
    const int tid = blockIdx.x * kNT + threadIdx.x;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = in[(tid + k) & 1023];
    const float a = in[1024], b = in[1025];
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = fmaf(x[k], a, b);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += x[k];
    out[tid] = s;
}

__global__ void __launch_bounds__(kNT) mix_mad64_kernel(const float* __restrict__ in, float* __restrict__ out, int iters) {
    const int tid = blockIdx.x * kNT + threadIdx.x;
    uint32_t x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __float_as_uint(in[(tid + k) & 1023]);
    const uint32_t m = __float_as_uint(in[1024]) | 1u;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint64_t p = (uint64_t)x[k] * (uint64_t)m;
                x[k] = (uint32_t)(p >> 32) ^ (uint32_t)p;
            }
    }
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s ^= x[k];
    out[tid] = __uint_as_float(s);
}

__global__ void __launch_bounds__(kNT) mix_trans_kernel(const float* __restrict__ in, float* __restrict__ out, int iters) {
    const int tid = blockIdx.x * kNT + threadIdx.x;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.25f + 0.5f * fabsf(in[(tid + k) & 1023]);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float l = __builtin_amdgcn_sqrtf(-__builtin_amdgcn_logf(x[k]));
                x[k] = __builtin_amdgcn_cosf(l) * __builtin_amdgcn_sinf(x[k]);
            }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += x[k];
    out[tid] = s;
}

__global__ void __launch_bounds__(kNT) mix_head_kernel(const float* __restrict__ in, float* __restrict__ out, int iters,
                                                       uint32_t k0, uint32_t k1) {
    constexpr int Q = 8;
    const int tid = threadIdx.x;
    const uint32_t tok = blockIdx.x, layer = 1;
    float p[Q][4], acc[Q][4];
#pragma unroll
    for (int j = 0; j < Q; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            p[j][c] = in[(tid + 4 * j + c) & 1023] * 1e-3f;
            acc[j][c] = 0.f;
        }
    const float c1 = in[1024] * 1e-3f, c2 = in[1025] * 1e-6f, c3 = in[1026] * 1e-9f;
    float r = in[1027];
    for (int i = 0; i < iters; ++i) {
        float a[Q][4];
        float sl = 0.f;
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const dust::f32x4 g = dust::gauss4_unscaled_uniform(tok, (uint32_t)(tid + j * kNT), (uint32_t)i, layer, k0, k1);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                a[j][c] = g.v[c];
                float t = fmaf(g.v[c], c3, c2);
                t = fmaf(g.v[c], t, c1);
                t = fmaf(g.v[c], t, 1.0f);
                sl = fmaf(p[j][c], g.v[c] * t, sl);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        r = fmaf(sl, 1e-3f, r * 0.5f);  // lane-local stand-in for the reward
#pragma unroll
        for (int j = 0; j < Q; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[j][c] = fmaf(r, a[j][c], acc[j][c]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < Q; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) s += acc[j][c];
    out[blockIdx.x * kNT + tid] = s;
}

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(kNT) mix_mfma_kernel(const float* __restrict__ in, float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    uint32_t ua[4], ub[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {   // bf16 pairs from the upper halves of two floats
        ua[k] = (__float_as_uint(in[(2 * (lane + 8 * k)) & 1023]) >> 16) |
                (__float_as_uint(in[(2 * (lane + 8 * k) + 1) & 1023]) & 0xFFFF0000u);
        ub[k] = (__float_as_uint(in[(2 * (lane + 8 * k) + 512) & 1023]) >> 16) |
                (__float_as_uint(in[(2 * (lane + 8 * k) + 513) & 1023]) & 0xFFFF0000u);
    }
    pbf16x8_t a, b;
    __builtin_memcpy(&a, ua, 16);
    __builtin_memcpy(&b, ub, 16);
    pf32x16_t acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    out[blockIdx.x * kNT + threadIdx.x] = s;
}

}  // namespace

// Runs mix `mix` (0..4) over `blocks` workgroups of 256 lanes with `iters` loop
// trips; `in` holds at least 1028 floats, `out` blocks*256 floats (device memory).
// Returns 0, or -1 for an unknown mix, or the HIP error of the launch.
extern "C" int dust_probe_valu_mix(int mix, int blocks, int iters, const float* in, float* out, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (blocks <= 0 || iters <= 0) return -1;
    switch (mix) {
        case 0: hipLaunchKernelGGL(mix_fma_kernel, dim3(blocks), dim3(kNT), 0, s, in, out, iters); break;
        case 1: hipLaunchKernelGGL(mix_mad64_kernel, dim3(blocks), dim3(kNT), 0, s, in, out, iters); break;
        case 2: hipLaunchKernelGGL(mix_trans_kernel, dim3(blocks), dim3(kNT), 0, s, in, out, iters); break;
        case 3: hipLaunchKernelGGL(mix_head_kernel, dim3(blocks), dim3(kNT), 0, s, in, out, iters, 0x12345678u, 0x9abcdef0u); break;
        case 4: hipLaunchKernelGGL(mix_mfma_kernel, dim3(blocks), dim3(kNT), 0, s, in, out, iters); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}
