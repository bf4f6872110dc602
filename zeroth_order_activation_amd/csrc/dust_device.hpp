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

// Three-way xor in one VALU op (v_bitop3_b32 with the truth table of a^b^c).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Ten Philox4x32 rounds (SC'11): per round two 32x32->64 products
// (v_mad_u64_u32) and two three-way xors.  With UNIFORM3 the caller
// guarantees that c0, c2, c3 and the key are uniform across the wave (token,
// draw, layer) and only c1 (the channel quad) varies: the first three rounds
// then use plain xors so that the uniform halves stay on the scalar unit.
template <bool UNIFORM3 = false>
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)kPhiloxM0 * (uint64_t)c0;
        const uint64_t p1 = (uint64_t)kPhiloxM1 * (uint64_t)c2;
        uint32_t n0, n2;
        if (UNIFORM3 && r < 3) {
            n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
            n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        } else {
            n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
            n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        }
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
//   rho = sqrt(-2 ln u1) = sqrt(2 ln 2) * sqrt(-log2 u1)
//   (cos, sin)(2 pi u2): the hardware sine/cosine take their argument in
//   revolutions, so u2 is used as is.
// box_muller_unscaled returns the pair divided by sqrt(2 ln 2) (one product
// fewer per pair); callers fold the factor into their own constants.
constexpr float kSqrt2Ln2 = 1.1774100225154747f;

__device__ __forceinline__ void box_muller_unscaled(uint32_t we, uint32_t wo, float& c, float& s) {
    const float u1 = fmaf((float)(we >> 8), 0x1p-24f, 0x1p-24f);  // ((we>>8)+1) 2^-24, exact
    const float u2 = (float)(wo >> 8) * 0x1p-24f;
    const float rho = __builtin_amdgcn_sqrtf(-__builtin_amdgcn_logf(u1));
    c = rho * __builtin_amdgcn_cosf(u2);
    s = rho * __builtin_amdgcn_sinf(u2);
}

__device__ __forceinline__ void box_muller(uint32_t we, uint32_t wo, float& c, float& s) {
    box_muller_unscaled(we, wo, c, s);
    c *= kSqrt2Ln2;
    s *= kSqrt2Ln2;
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

// The Gaussians divided by sqrt(2 ln 2) (any counter).
__device__ __forceinline__ f32x4 gauss4_unscaled(uint32_t token, uint32_t quad, uint32_t draw, uint32_t layer,
                                                 uint32_t k0, uint32_t k1) {
    const u32x4 w = philox4x32_10(token, quad, draw, layer, k0, k1);
    f32x4 a;
    box_muller_unscaled(w.x, w.y, a.v[0], a.v[1]);
    box_muller_unscaled(w.z, w.w, a.v[2], a.v[3]);
    return a;
}

// The same Gaussians divided by sqrt(2 ln 2), for a wave whose token, draw and
// layer are uniform.
__device__ __forceinline__ f32x4 gauss4_unscaled_uniform(uint32_t token, uint32_t quad, uint32_t draw,
                                                         uint32_t layer, uint32_t k0, uint32_t k1) {
    const u32x4 w = philox4x32_10<true>(token, quad, draw, layer, k0, k1);
    f32x4 a;
    box_muller_unscaled(w.x, w.y, a.v[0], a.v[1]);
    box_muller_unscaled(w.z, w.w, a.v[2], a.v[3]);
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

// v + (v moved by one DPP pattern); rows outside ROWM add 0.
template <int CTRL, int ROWM>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWM, 0xF, false));
}
// Sum over the 64 lanes of a wave, returned wave-uniform; every lane must be
// active.  Lane pairs and quads by quad permutes, half rows and rows by the
// row mirrors, then the row sums gathered into the last row by the two row
// broadcasts and read from lane 63: VALU work only, where a butterfly of
// lane shuffles costs six dependent LDS-unit round trips.
__device__ __forceinline__ float wave_total(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror
    v = dpp_add<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// log1p(x) for a wave-uniform x > -1.  For |x| <= 1/8: log1p(x) = 2 atanh(s),
// s = x / (2 + x), |s| < 0.059, by its series through s^7 (the next term is
// below 2e-11 relative); otherwise the library function.
__device__ __forceinline__ float log1p_uniform(float x) {
    x = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
    if (fabsf(x) <= 0.125f) {
        const float s = x * __builtin_amdgcn_rcpf(2.0f + x);
        const float s2 = s * s;
        const float p = fmaf(s2, fmaf(s2, fmaf(s2, 1.0f / 7.0f, 1.0f / 5.0f), 1.0f / 3.0f), 1.0f);
        return 2.0f * s * p;
    }
    return log1pf(x);
}

}  // namespace dust
