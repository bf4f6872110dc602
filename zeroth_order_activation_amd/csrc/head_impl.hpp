// LM-head estimator on cached logits: one workgroup per token (and, for the
// LDS-staged bf16 rows feeding the outer product, a persistent form in which
// each workgroup walks many tokens, the next row loading during the stores).
//
// Method (TL;DR page "Dust: zeroth-order Transformer pretraining without
// backprop", section 1, "credit assignment without backprop" and "reducing
// interference"; news article on tahou.com, mechanism paragraph): the head is
// jittered on the cached logits z_t, only the loss is recomputed, the reward
// is the loss reduction at the token and
//     g_hat_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i).
//
// Per draw the kernel needs CE(z + sigma a) - CE(z).  With p = softmax(z) this
// is exactly  log1p(S) - sigma a_y,  S = sum_v p_v expm1(sigma a_v),  which
// avoids subtracting two losses of size ln V in fp32.  |a| <= sqrt(48 ln 2)
// by construction of the noise, so for small sigma expm1 is a short Taylor
// polynomial of degree DEG (3, 4 or 6) in x = sigma a; the host picks the
// lowest degree whose dropped terms move S by less than 2e-5 sigma (since
// sum p = 1, that bound is |x|max^(DEG+1)/(DEG+1)! e^|x|max); larger sigma uses
// the library expm1 (DEG = 0).  The noise is generated divided by sqrt(2 ln 2) (one
// product fewer per pair); the host folds that factor into sigma and the
// final scale.
//
// Layout: lane l owns channel quads q = l + j*NT (j < Q), so each load and
// store of a quad is one coalesced 16-byte (fp32) or 8-byte (bf16) access.
// The noise of the current draw and the running sum of r*a live in registers
// (for the widest rows, the running sums of the last QL quads of each lane
// live in LDS after the logit row instead, so that 4 waves per SIMD fit without
// spilling); each draw costs one workgroup reduction (two floats) and one
// barrier.
#pragma once

#include <algorithm>
#include <type_traits>

#include "dust_device.hpp"
#include "dust_internal.hpp"
#include "launch_events.hpp"

namespace dust {

constexpr float kLog2e = kLog2eF;

template <int LT>
__device__ __forceinline__ f32x4 load_quad(const void* row, int q, int V, bool vec) {
    f32x4 r;
    const float ninf = -__builtin_inff();
    if (vec) {
        if (LT == 0) {
            const float4 v = reinterpret_cast<const float4*>(row)[q];
            r.v[0] = v.x; r.v[1] = v.y; r.v[2] = v.z; r.v[3] = v.w;
        } else {
            const uint2 v = reinterpret_cast<const uint2*>(row)[q];
            r.v[0] = __uint_as_float(v.x << 16);
            r.v[1] = __uint_as_float(v.x & 0xFFFF0000u);
            r.v[2] = __uint_as_float(v.y << 16);
            r.v[3] = __uint_as_float(v.y & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int v = 4 * q + c;
            if (v < V)
                r.v[c] = LT == 0 ? reinterpret_cast<const float*>(row)[v]
                                 : bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[v]);
            else
                r.v[c] = ninf;
        }
    }
    return r;
}

// Block-wide reductions for the clean statistics (called a few times per token).
template <int NT>
__device__ __forceinline__ float block_max(float v, float* sh) {
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, sh[w]);
    return r;
}
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) r += sh[w];
    return r;
}

// Maximum over the 64 lanes of a wave, returned wave-uniform (the pattern of
// wave_total with max in place of the sum; rows a broadcast does not write keep
// -inf); every lane must be active.
template <int CTRL, int ROWM>
__device__ __forceinline__ float dpp_max(float v) {
    const int ninf = (int)0xFF800000u;
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), CTRL, ROWM, 0xF, false)));
}
__device__ __forceinline__ float wave_max_uniform(float v) {
    v = dpp_max<0xB1, 0xF>(v);
    v = dpp_max<0x4E, 0xF>(v);
    v = dpp_max<0x141, 0xF>(v);
    v = dpp_max<0x140, 0xF>(v);
    v = dpp_max<0x142, 0xA>(v);
    v = dpp_max<0x143, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Log-sum-exp statistics of a row from per-lane pairs (m, s = sum exp(z - m)):
// pairs merge as M = max(m, m'), s exp(m - M) + s' exp(m' - M); a pair with
// m = -inf (no entries) contributes nothing.  Within a wave: the maximum by
// DPP, each lane's sum rescaled to it and summed by DPP (all lanes active);
// between the waves: one LDS exchange.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    const float a = m == -__builtin_inff() ? 0.f : s * __expf(m - M);
    const float b = m2 == -__builtin_inff() ? 0.f : s2 * __expf(m2 - M);
    m = M;
    s = a + b;
}
__device__ __forceinline__ void wave_max_sumexp(float& m, float& s) {
    const float M = wave_max_uniform(m);
    s = wave_total(m == -__builtin_inff() ? 0.f : s * __expf(m - M));
    m = M;
}
template <int NT>
__device__ __forceinline__ void block_max_sumexp(float& m, float& s, float2* sh) {
    wave_max_sumexp(m, s);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = make_float2(m, s);
    __syncthreads();
    float2 r = sh[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) merge_ms(r.x, r.y, sh[w].x, sh[w].y);
    m = r.x;
    s = r.y;
}

// Two floats to a pair of bf16 (round to nearest even), the first in the low half.
typedef __bf16 hbf16x2_t __attribute__((ext_vector_type(2)));
typedef float hf32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_2(float a, float b) {
    const hf32x2_t v = {a, b};
    const hbf16x2_t h = __builtin_convertvector(v, hbf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

// expm1(sigma a) / sigma  (DEG = 4, 6)  or  expm1(sigma a)  (DEG = 0).
template <int DEG>
__device__ __forceinline__ float em1(float a, const HeadArgs& A) {
    if (DEG > 0) {
        float t = A.coef[DEG - 1];
#pragma unroll
        for (int k = DEG - 2; k >= 1; --k) t = fmaf(a, t, A.coef[k]);
        t = fmaf(a, t, 1.0f);
        return a * t;
    } else {
        return expm1f(A.sigma * a);
    }
}

// Row of LDS-staged logits (PMODE 1): stored in the logits' own type.
template <int LT>
__device__ __forceinline__ f32x4 lds_quad(const unsigned char* zl, int q) {
    f32x4 r;
    if (LT == 0) {
        const float4 v = reinterpret_cast<const float4*>(zl)[q];
        r.v[0] = v.x; r.v[1] = v.y; r.v[2] = v.z; r.v[3] = v.w;
    } else {
        const uint2 v = reinterpret_cast<const uint2*>(zl)[q];
        r.v[0] = __uint_as_float(v.x << 16);
        r.v[1] = __uint_as_float(v.x & 0xFFFF0000u);
        r.v[2] = __uint_as_float(v.y << 16);
        r.v[3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
    return r;
}

template <int NT, int Q, int LT, int PMODE, int DEG, int QL>
__global__ void __launch_bounds__(NT, (NT == 256 ? 4 : 1)) head_estimate_kernel(HeadArgs A) {
    static_assert(QL == 0 || PMODE == 1, "LDS running sums sit after the LDS logit row");
    constexpr int QR = Q - QL;  // quads whose running sums stay in registers
    constexpr int NW = NT / 64;
    constexpr bool SCHED_FENCE = Q >= 8;
    __shared__ float2 sh_ms[NW];
    __shared__ float sh_red[2][NW][2];
    extern __shared__ __align__(16) unsigned char zlds[];

    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int V = A.V;
    const int nq = (V + 3) >> 2;
    const bool vec = (V & 3) == 0;
    const void* row = reinterpret_cast<const unsigned char*>(A.logits) + (size_t)t * V * (LT == 0 ? 4 : 2);

    // ---- clean statistics: max, log-sum-exp, probabilities ---------------
    // Every quad of the lane is loaded at once (the loads are independent, so
    // their latencies overlap); PMODE 1 stages the row in LDS, padded to NT*Q
    // quads with -inf (probability 0) so the draw loop needs no bounds test.
    // One block reduction merges the per-lane (max, sum of exponentials).
    float p[PMODE == 0 ? Q : 1][4];
    float m = -__builtin_inff(), s = 0.f;
    // consume quad j of the lane: its four logits (-inf past the row)
    auto keep = [&](int j, const f32x4& z) {
        if (PMODE == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) p[PMODE == 0 ? j : 0][c] = z.v[c];
        } else {
            const int q = tid + j * NT;
            if (LT == 0) {
                reinterpret_cast<float4*>(zlds)[q] = make_float4(z.v[0], z.v[1], z.v[2], z.v[3]);
            } else {
                uint2 b;
                b.x = (__float_as_uint(z.v[0]) >> 16) | (__float_as_uint(z.v[1]) & 0xFFFF0000u);
                b.y = (__float_as_uint(z.v[2]) >> 16) | (__float_as_uint(z.v[3]) & 0xFFFF0000u);
                reinterpret_cast<uint2*>(zlds)[q] = b;
            }
        }
    };
    if (vec) {
        // uniform fast path: all quads at once, from clamped (always valid)
        // addresses, kept packed; padding is applied by select afterwards
        typedef typename std::conditional<LT == 0, float4, uint2>::type raw_t;
        raw_t raw[Q];
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const int q = tid + j * NT;
            raw[j] = reinterpret_cast<const raw_t*>(row)[q < nq ? q : nq - 1];
        }
        auto unpack = [&](int j) {
            f32x4 z;
            if (LT == 0) {
                const float4 v = *reinterpret_cast<const float4*>(&raw[j]);
                z.v[0] = v.x; z.v[1] = v.y; z.v[2] = v.z; z.v[3] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(&raw[j]);
                z.v[0] = __uint_as_float(v.x << 16);
                z.v[1] = __uint_as_float(v.x & 0xFFFF0000u);
                z.v[2] = __uint_as_float(v.y << 16);
                z.v[3] = __uint_as_float(v.y & 0xFFFF0000u);
            }
            if (tid + j * NT >= nq) z.v[0] = z.v[1] = z.v[2] = z.v[3] = -__builtin_inff();
            return z;
        };
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const f32x4 z = unpack(j);
#pragma unroll
            for (int c = 0; c < 4; ++c) m = fmaxf(m, z.v[c]);
        }
        if (m != -__builtin_inff()) {
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const f32x4 z = unpack(j);
#pragma unroll
                for (int c = 0; c < 4; ++c) s += __expf(z.v[c] - m);
            }
        }
#pragma unroll
        for (int j = 0; j < Q; ++j) keep(j, unpack(j));
    } else {
        // rows whose length is not a multiple of 4: element loads, two passes
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const int q = tid + j * NT;
            f32x4 z;
            if (q < nq) z = load_quad<LT>(row, q, V, false);
            else z.v[0] = z.v[1] = z.v[2] = z.v[3] = -__builtin_inff();
#pragma unroll
            for (int c = 0; c < 4; ++c) m = fmaxf(m, z.v[c]);
            keep(j, z);
        }
        if (m != -__builtin_inff()) {
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const int q = tid + j * NT;
                if (q >= nq) continue;
                const f32x4 z = load_quad<LT>(row, q, V, false);
#pragma unroll
                for (int c = 0; c < 4; ++c) s += __expf(z.v[c] - m);
            }
        }
    }
    block_max_sumexp<NT>(m, s, sh_ms);  // its barrier also publishes the LDS row
    const float lse = m + __logf(s);
    const float lse2 = lse * kLog2e;
    if (PMODE == 0) {
#pragma unroll
        for (int j = 0; j < Q; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) p[j][c] = __builtin_amdgcn_exp2f(fmaf(p[j][c], kLog2e, -lse2));
    }

    // ---- label owner --------------------------------------------------------
    const uint32_t y = (uint32_t)A.labels[t];
    const uint32_t qy = y >> 2, cy = y & 3u;
    const uint32_t jy = qy / NT;
    const bool owner = (qy % NT) == (uint32_t)tid && y < (uint32_t)V;

    const uint32_t tok = A.tok0 + (uint32_t)t;
    // some lane of this wave holds a quad of the row in the last quad row (uniform)
    const bool tail_live = wid * 64 + (Q - 1) * NT < nq;
    float acc[QR > 0 ? QR : 1][4];
#pragma unroll
    for (int j = 0; j < QR; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[j][c] = 0.f;
    // running sums of quads j >= QR: float4 slots [j - QR][lane] after the row
    float4* accl = reinterpret_cast<float4*>(zlds + (size_t)NT * Q * (LT == 0 ? 16 : 8));
#pragma unroll
    for (int j = 0; j < QL; ++j) accl[j * NT + tid] = make_float4(0.f, 0.f, 0.f, 0.f);

    for (int i = 0; i < A.K; ++i) {
        const uint32_t draw = A.draw0 + (uint32_t)i;
        // the lane index, opaque to the compiler inside the draw loop: the per-quad
        // indices and LDS addresses derived from it are recomputed (one or two
        // instructions each) instead of hoisted out of the loop and spilled
        int tl = tid;
        asm volatile("" : "+v"(tl));
        float a[Q][4];
        float sl = 0.f, ly = 0.f;
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            // quads past the row have probability 0: they add nothing to S, and
            // their running sums are never stored; a wave whose lanes are all past
            // the row in the last quad row skips it
            if (j == Q - 1 && !tail_live) {
#pragma unroll
                for (int c = 0; c < 4; ++c) a[j][c] = 0.f;
                continue;
            }
            const int q = tl + j * NT;
            const f32x4 g = gauss4_unscaled_uniform(tok, (uint32_t)q, draw, A.layer, A.k0, A.k1);
            f32x4 pz;
            if (PMODE == 1) pz = lds_quad<LT>(zlds, q);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                a[j][c] = g.v[c];
                const float pc = PMODE == 0 ? p[j][c] : __builtin_amdgcn_exp2f(fmaf(pz.v[c], kLog2e, -lse2));
                sl = fmaf(pc, em1<DEG>(g.v[c], A), sl);
            }
            if ((uint32_t)j == jy) {
                const float sel = cy == 0 ? a[j][0] : cy == 1 ? a[j][1] : cy == 2 ? a[j][2] : a[j][3];
                ly = owner ? sel : 0.f;
            }
            // keep the scheduler from interleaving many quads (their Philox and
            // Box-Muller temporaries would not fit next to a[] and acc[])
            if (SCHED_FENCE) __builtin_amdgcn_sched_barrier(0);
        }
        sl = wave_total(sl);
        ly = wave_total(ly);
        const int b = i & 1;
        if ((tid & 63) == 0) { sh_red[b][wid][0] = sl; sh_red[b][wid][1] = ly; }
        __syncthreads();
        float S = 0.f, LY = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) { S += sh_red[b][w][0]; LY += sh_red[b][w][1]; }
        const float r = A.sigma * LY - log1p_uniform(S * A.smul);
#pragma unroll
        for (int j = 0; j < QR; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[j][c] = fmaf(r, a[j][c], acc[j][c]);
#pragma unroll
        for (int j = QR; j < Q; ++j) {  // only this lane touches its slots: no barrier needed
            if (j == Q - 1 && !tail_live) continue;
            float4 o = accl[(j - QR) * NT + tl];
            o.x = fmaf(r, a[j][0], o.x); o.y = fmaf(r, a[j][1], o.y);
            o.z = fmaf(r, a[j][2], o.z); o.w = fmaf(r, a[j][3], o.w);
            accl[(j - QR) * NT + tl] = o;
        }
        if (tid == 0 && A.rewards) A.rewards[(size_t)i * A.T + t] = r;
    }

    // ---- g_hat_t = -(1/(K sigma)) sum_i r a ------------------------------------
    // fp32 rows and/or the bf16 pairs (hi = bf16(g), lo = bf16(g - hi)) that the
    // outer product consumes, token-major with the row zero-padded to ldp
    float* out = A.ghat ? A.ghat + (size_t)t * V : nullptr;
    uint16_t* ohi = A.ghi ? A.ghi + (size_t)t * A.ldp : nullptr;
    uint16_t* olo = A.ghi ? A.glo + (size_t)t * A.ldp : nullptr;
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const int q = tid + j * NT;
        float v[4];
        if (j < QR) {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = acc[j < QR ? j : 0][c] * A.gscale;
        } else {
            const float4 o = accl[(j - QR) * NT + tid];
            v[0] = o.x * A.gscale; v[1] = o.y * A.gscale; v[2] = o.z * A.gscale; v[3] = o.w * A.gscale;
        }
        if (ohi && 4 * (int64_t)q < A.ldp) {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = 4 * q + c < V ? v[c] : 0.f;
            uint2 h, l;
            h.x = pack_bf16_2(v[0], v[1]);
            h.y = pack_bf16_2(v[2], v[3]);
            l.x = pack_bf16_2(v[0] - __uint_as_float(h.x << 16), v[1] - __uint_as_float(h.x & 0xFFFF0000u));
            l.y = pack_bf16_2(v[2] - __uint_as_float(h.y << 16), v[3] - __uint_as_float(h.y & 0xFFFF0000u));
            *reinterpret_cast<uint2*>(ohi + 4 * q) = h;
            *reinterpret_cast<uint2*>(olo + 4 * q) = l;
        }
        if (!out || q >= nq) continue;
        if (vec) {
            reinterpret_cast<float4*>(out)[q] = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (4 * q + c < V) out[4 * q + c] = v[c];
        }
    }
}

// ---------------------------------------------------------------------------
// Persistent form of the LDS-staged variant (bf16 rows, V a multiple of 8, the
// bf16-pair output only).  Each workgroup walks the tokens t = b, b + G, ...
// with G at most one workgroup per CU.  The row of the next token goes from
// global memory straight into LDS (buffer loads into LDS: no registers) once
// the last draw of the current token is reduced -- past that barrier no wave
// reads the row again -- and lands while the running sums are scaled and the
// pairs stored.  The pair stores are buffer stores checked against the row's
// bounds, two per quad whatever the lane, so every wave knows that exactly 2Q
// memory operations follow its row loads and waits for the loads alone; the
// stores drain during the next token's draws.  The barriers wait for LDS
// operations only.  At T 8192, V 50304, K 16 this takes 5.07-5.41 ms per launch
// where one workgroup per token takes 5.42-5.53 ms on the same boxes; without
// the stores at all it would take about 4.8 ms (the stores still cost time
// once they overlap the draws, and starting the workgroups at staggered
// times, so that fewer of them store at once, made it slower).
// ---------------------------------------------------------------------------
constexpr int head_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kHeadLgkm0 = 15 | (7 << 4) | (3 << 14);   // lgkmcnt(0), vmcnt and expcnt not waited for

// Barrier for data exchanged through LDS: the wave's own LDS operations are
// complete, outstanding global memory operations are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kHeadLgkm0);
    asm volatile("s_barrier" ::: "memory");
}

// The row statistics of block_max_sumexp with a barrier that does not wait for
// global memory, the wave's slot given as a wave-uniform index.
template <int NT>
__device__ __forceinline__ void block_max_sumexp_lds(float& m, float& s, float2* sh, int wid) {
    wave_max_sumexp(m, s);
    asm volatile("" : "+s"(wid));   // the slot address is formed here, not kept live across the caller's loops
    sh[wid] = make_float2(m, s);   // the same values from every lane of the wave
    lds_barrier();
    float2 r = sh[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) merge_ms(r.x, r.y, sh[w].x, sh[w].y);
    m = r.x;
    s = r.y;
}

constexpr int kStreamNT = 1024;

// This lane's index in the workgroup (w64 = 64 x the wave's index, wave-uniform),
// recomputed where it is used: the volatile asm cannot be hoisted out of the loops,
// so no register has to hold the index (or anything derived from it) across them.
__device__ __forceinline__ int stream_tid(int w64) {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l + w64;
}

template <int Q, int DEG, int QL>
__global__ void __launch_bounds__(kStreamNT, 1) head_stream_kernel(HeadArgs A) {
    constexpr int NT = kStreamNT, NW = NT / 64, QR = Q - QL;
    constexpr int NPL = (Q * 8 + 15) / 16;   // 16-byte row pieces per lane
    constexpr int NST = 2 * Q;               // pair stores per lane and token
    constexpr bool SCHED_FENCE = Q >= 8;
    // separate LDS objects: the running sums and reduction slots provably do not
    // alias the row loads in flight
    __shared__ __align__(16) uint2 zrow[NT * Q];
    __shared__ __align__(16) float4 accl[QL > 0 ? QL * NT : 1];
    __shared__ float2 sh_ms[NW];
    __shared__ float sh_red[2][NW][2];

    const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // wave-uniform
    const int w64 = wid * 64;
    const int V = A.V;
    const int nq = V >> 2, npc = V >> 3;
    const uint32_t rowbytes = (uint32_t)V * 2u;
    const uint32_t pairbytes = (uint32_t)A.ldp * 2u;
    const bool tail_live = wid * 64 + (Q - 1) * NT < nq;

    {
        // quads past the row: -inf (probability 0); the row loads cover quads < nq exactly
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < Q; ++j)
            if (tid + j * NT >= nq) zrow[tid + j * NT] = make_uint2(0xFF80FF80u, 0xFF80FF80u);
#pragma unroll
        for (int j = 0; j < QL; ++j) accl[j * NT + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    auto issue_row = [&](int tt) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const unsigned char*>(A.logits) + (size_t)tt * rowbytes), (short)0,
            (int)rowbytes, 0x00020000);
        const int tl = stream_tid(w64);
        int wbase = w64 * 16;   // byte offset of the wave's 64 slots, formed anew for each row
        asm volatile("" : "+s"(wbase));
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int P = tl + i * NT;
            if (P < npc)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)(reinterpret_cast<unsigned char*>(zrow) +
                                                                  i * NT * 16 + wbase),
                    16, P * 16, 0, 0, 0);
        }
    };

    int t = blockIdx.x;   // the grid never exceeds T
    issue_row(t);
    __builtin_amdgcn_s_waitcnt(head_vmcnt(0));
    lds_barrier();
    for (;;) {
        // ---- clean statistics of the staged row (each lane reads its own quads)
        float m = -__builtin_inff(), s = 0.f;
        {
            const int tl = stream_tid(w64);
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const f32x4 z = lds_quad<1>(reinterpret_cast<const unsigned char*>(zrow), tl + j * NT);
#pragma unroll
                for (int c = 0; c < 4; ++c) m = fmaxf(m, z.v[c]);
            }
            if (m != -__builtin_inff()) {
#pragma unroll
                for (int j = 0; j < Q; ++j) {
                    const f32x4 z = lds_quad<1>(reinterpret_cast<const unsigned char*>(zrow), tl + j * NT);
#pragma unroll
                    for (int c = 0; c < 4; ++c) s += __expf(z.v[c] - m);
                }
            }
        }
        block_max_sumexp_lds<NT>(m, s, sh_ms, wid);
        const float lse2 = (m + __logf(s)) * kLog2e;

        // the labels are read-only here: a scalar load, which no vector-memory wait
        // (and so none of the pair stores still in flight) holds up
        const uint32_t y = (uint32_t)((const __attribute__((address_space(4))) int32_t*)A.labels)[t];
        const uint32_t qy = y >> 2, cy = y & 3u;
        const uint32_t jy = qy / NT;
        const bool owner = (qy % NT) == (uint32_t)stream_tid(w64) && y < (uint32_t)V;
        const uint32_t tok = A.tok0 + (uint32_t)t;

        float acc[QR > 0 ? QR : 1][4];
#pragma unroll
        for (int j = 0; j < QR; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[j][c] = 0.f;

        for (int i = 0; i < A.K; ++i) {
            const uint32_t draw = A.draw0 + (uint32_t)i;
            const int tl = stream_tid(w64);
            float a[Q][4];
            float sl = 0.f, ly = 0.f;
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                if (j == Q - 1 && !tail_live) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) a[j][c] = 0.f;
                    continue;
                }
                const int q = tl + j * NT;
                const f32x4 g = gauss4_unscaled_uniform(tok, (uint32_t)q, draw, A.layer, A.k0, A.k1);
                const f32x4 pz = lds_quad<1>(reinterpret_cast<const unsigned char*>(zrow), q);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    a[j][c] = g.v[c];
                    const float pc = __builtin_amdgcn_exp2f(fmaf(pz.v[c], kLog2e, -lse2));
                    sl = fmaf(pc, em1<DEG>(g.v[c], A), sl);
                }
                if ((uint32_t)j == jy) {
                    const float sel = cy == 0 ? a[j][0] : cy == 1 ? a[j][1] : cy == 2 ? a[j][2] : a[j][3];
                    ly = owner ? sel : 0.f;
                }
                if (SCHED_FENCE) __builtin_amdgcn_sched_barrier(0);
            }
            sl = wave_total(sl);
            ly = wave_total(ly);
            const int b = i & 1;
            if (tl == w64) { sh_red[b][wid][0] = sl; sh_red[b][wid][1] = ly; }
            lds_barrier();
            float S = 0.f, LY = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) { S += sh_red[b][w][0]; LY += sh_red[b][w][1]; }
            const float r = A.sigma * LY - log1p_uniform(S * A.smul);
#pragma unroll
            for (int j = 0; j < QR; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[j][c] = fmaf(r, a[j][c], acc[j][c]);
#pragma unroll
            for (int j = QR; j < Q; ++j) {
                if (j == Q - 1 && !tail_live) continue;
                float4 o = accl[(j - QR) * NT + tl];
                o.x = fmaf(r, a[j][0], o.x); o.y = fmaf(r, a[j][1], o.y);
                o.z = fmaf(r, a[j][2], o.z); o.w = fmaf(r, a[j][3], o.w);
                accl[(j - QR) * NT + tl] = o;
            }
            if (tl == 0 && A.rewards) A.rewards[(size_t)i * A.T + t] = r;
        }

        // ---- the next row into LDS: every wave is past its last read of this one
        const int tn = t + (int)gridDim.x;
        const bool more = tn < A.T;
        __builtin_amdgcn_sched_barrier(0);
        if (more) issue_row(tn);
        __builtin_amdgcn_sched_barrier(0);

        // ---- g_hat_t = -(1/(K sigma)) sum_i r a, as bf16 pairs (zero past V) -----
        {
            const int tl = stream_tid(w64);
            const __amdgpu_buffer_rsrc_t rh =
                __builtin_amdgcn_make_buffer_rsrc((void*)(A.ghi + (size_t)t * A.ldp), (short)0, (int)pairbytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t rl =
                __builtin_amdgcn_make_buffer_rsrc((void*)(A.glo + (size_t)t * A.ldp), (short)0, (int)pairbytes, 0x00020000);
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const int q = tl + j * NT;
                float v[4];
                if (j < QR) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = acc[j < QR ? j : 0][c] * A.gscale;
                } else {
                    const float4 o = accl[(j - QR) * NT + tl];
                    float z0 = 0.f;
                    asm volatile("" : "+v"(z0));
                    accl[(j - QR) * NT + tl] = make_float4(z0, z0, z0, z0);
                    v[0] = o.x * A.gscale; v[1] = o.y * A.gscale; v[2] = o.z * A.gscale; v[3] = o.w * A.gscale;
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = 4 * q + c < V ? v[c] : 0.f;
                typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
                u32x2_t h, l;
                h.x = pack_bf16_2(v[0], v[1]);
                h.y = pack_bf16_2(v[2], v[3]);
                l.x = pack_bf16_2(v[0] - __uint_as_float(h.x << 16), v[1] - __uint_as_float(h.x & 0xFFFF0000u));
                l.y = pack_bf16_2(v[2] - __uint_as_float(h.y << 16), v[3] - __uint_as_float(h.y & 0xFFFF0000u));
                // past ldp the bounds check drops the store
                __builtin_amdgcn_raw_buffer_store_b64(h, rh, q * 8, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(l, rl, q * 8, 0, 0);
            }
        }
        if (!more) break;
        t = tn;
        // this wave's row pieces have landed once at most NST operations (its
        // stores) are outstanding; the barrier then covers every wave's pieces
        __builtin_amdgcn_s_waitcnt(head_vmcnt(NST));
        lds_barrier();
    }
}

template <int Q, int DEG, int QL>
hipError_t launch_head_stream(const HeadArgs& args, hipStream_t stream) {
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int grid = (int)std::min<int64_t>(args.T, std::max(ncu, 1));
    bool timed = false;
    if ((e = launch_timer_begin(kTimedHead, stream, timed)) != hipSuccess) return e;
    hipLaunchKernelGGL((head_stream_kernel<Q, DEG, QL>), dim3(grid), dim3(kStreamNT), 0, stream, args);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_timer_end(kTimedHead, stream, timed);
}

// The persistent form applies to bf16 rows of the LDS-staged plans whose length
// is a multiple of 8, when the pairs are the only output.
inline bool head_stream_applies(const HeadPlan& P, const HeadArgs& A, int logits_dtype) {
    return logits_dtype == 1 && P.pmode == 1 && P.nt == kStreamNT && (A.V & 7) == 0 && A.ghi && A.glo && !A.ghat &&
           (A.ldp & 3) == 0;
}

template <int NT, int Q, int LT, int PMODE, int DEG, int QL>
hipError_t launch_head_variant(const HeadPlan& plan, const HeadArgs& args, hipStream_t stream) {
    auto k = head_estimate_kernel<NT, Q, LT, PMODE, DEG, QL>;
    if (plan.lds > 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds);
        if (e != hipSuccess) return e;
    }
    bool timed = false;
    hipError_t e = launch_timer_begin(kTimedHead, stream, timed);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(args.T), dim3(NT), plan.lds, stream, args);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_timer_end(kTimedHead, stream, timed);
}

// Dispatch over the compiled variants for one logits type.
template <int LT>
hipError_t dispatch_head(const HeadPlan& P, const HeadArgs& A, hipStream_t s) {
#define DUST_STREAM_CASE(Q_, QL_)                                                          \
    if (P.q == Q_ && P.ql == QL_) {                                                        \
        return P.deg == 3   ? launch_head_stream<Q_, 3, QL_>(A, s)                         \
               : P.deg == 4 ? launch_head_stream<Q_, 4, QL_>(A, s)                         \
               : P.deg == 6 ? launch_head_stream<Q_, 6, QL_>(A, s)                         \
                            : launch_head_stream<Q_, 0, QL_>(A, s);                        \
    }
    if constexpr (LT == 1) {
        if (head_stream_applies(P, A, LT)) {
            DUST_STREAM_CASE(4, 0)
            DUST_STREAM_CASE(8, 0)
            DUST_STREAM_CASE(13, 3)
            DUST_STREAM_CASE(16, 0)
        }
    }
#undef DUST_STREAM_CASE
#define DUST_HEAD_CASE(NT_, Q_, PM_, QL_)                                                  \
    if (P.nt == NT_ && P.q == Q_ && P.pmode == PM_ && P.ql == QL_) {                        \
        return P.deg == 3   ? launch_head_variant<NT_, Q_, LT, PM_, 3, QL_>(P, A, s)         \
               : P.deg == 4 ? launch_head_variant<NT_, Q_, LT, PM_, 4, QL_>(P, A, s)         \
               : P.deg == 6 ? launch_head_variant<NT_, Q_, LT, PM_, 6, QL_>(P, A, s)         \
                            : launch_head_variant<NT_, Q_, LT, PM_, 0, QL_>(P, A, s);        \
    }
    DUST_HEAD_CASE(256, 1, 0, 0)
    DUST_HEAD_CASE(256, 2, 0, 0)
    DUST_HEAD_CASE(256, 4, 0, 0)
    DUST_HEAD_CASE(256, 8, 0, 0)
    DUST_HEAD_CASE(1024, 4, 1, 0)
    DUST_HEAD_CASE(1024, 8, 1, 0)
    if constexpr (LT == 1) {  // rows past 32768 channels: bf16 only (an fp32 row would not fit in LDS)
        DUST_HEAD_CASE(1024, 13, 1, 3)
        DUST_HEAD_CASE(1024, 16, 1, 0)
    }
#undef DUST_HEAD_CASE
    return hipErrorInvalidConfiguration;
}

}  // namespace dust
