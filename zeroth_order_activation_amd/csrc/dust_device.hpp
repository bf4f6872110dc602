// Device-side building blocks shared by the Dust kernels (gfx950, wave64).
//
// Noise: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) + Box-Muller, on
// the counter (token, channel >> 2, draw, layer) under the key (lo32(seed),
// hi32(seed)).  The pages only ask for independent Gaussian noise per token
// and channel (TL;DR page, section 1, "activation-space perturbation"); the
// stream is fixed so that the estimate is reproducible and can be split over
// draws or tokens.  The noise is produced in registers and never stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dust {

constexpr float kLog2eF = 1.4426950408889634f;

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct u32x4 {
    uint32_t x, y, z, w;
};

// Ten Philox4x32 rounds.  The counter words that are uniform across a wave
// (token, draw, layer in the head kernel) sit in c0, c2, c3, so the first
// products of the chain are scalar; the channel quad sits in c1.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)kPhiloxM0 * (uint64_t)c0;
        const uint64_t p1 = (uint64_t)kPhiloxM1 * (uint64_t)c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
    return {c0, c1, c2, c3};
}

// Box-Muller on one pair of 32-bit words: the top 24 bits of each give
// u1 in (0,1] and u2 in [0,1), both exact in fp32.
//   rho = sqrt(-2 ln u1) = sqrt(-2 ln2 * log2 u1)
//   (cos, sin)(2 pi u2): the hardware sine/cosine take their argument in
//   revolutions, so u2 is used as is.
__device__ __forceinline__ void box_muller(uint32_t we, uint32_t wo, float& c, float& s) {
    const float u1 = (float)((we >> 8) + 1u) * 0x1p-24f;
    const float u2 = (float)(wo >> 8) * 0x1p-24f;
    const float rho = __builtin_amdgcn_sqrtf(-1.3862943611198906f * __builtin_amdgcn_logf(u1));
    c = rho * __builtin_amdgcn_cosf(u2);
    s = rho * __builtin_amdgcn_sinf(u2);
}

struct f32x4 {
    float v[4];
};

// The four Gaussians of channel quad q for (token, draw).
__device__ __forceinline__ f32x4 gauss4(uint32_t token, uint32_t quad, uint32_t draw, uint32_t layer,
                                        uint32_t k0, uint32_t k1) {
    const u32x4 w = philox4x32_10(token, quad, draw, layer, k0, k1);
    f32x4 a;
    box_muller(w.x, w.y, a.v[0], a.v[1]);
    box_muller(w.z, w.w, a.v[2], a.v[3]);
    return a;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Wave64 reductions (butterfly over all 64 lanes; every lane gets the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace dust
