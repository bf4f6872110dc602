// LM-head estimator with a vocabulary subset per draw: one workgroup per token.
//
// Method (TL;DR page "Dust: zeroth-order Transformer pretraining without
// backprop", section 1, "reducing interference": the head is evaluated on part
// of the vocabulary per draw to save time; the subset rule is not given).
// Reading: per (token, draw) the subset S is a cyclic window of mq = m/4
// consecutive channel quads starting at o = (w * nq) >> 32, w = word 0 of
// Philox4x32-10 on the counter (token, 0xFFFFFFFF, draw, layer), plus the label.
// S is perturbed with the full estimator's noise; nothing else moves, so the
// change of the loss is exactly log1p(sum_{v in S} p_v expm1(sigma a_v)) -
// sigma a_y.  Channels are weighted by the inverse of their inclusion
// probability (nq/mq in the window, 1 for the label), which keeps
//     g_hat_v = -(1/(K sigma)) sum_i r_i a_v^(i) 1[v in S_i] / pi_v
// unbiased.  The per-draw work is mq quads instead of nq.
//
// Layout: the clean probabilities (fp32) and the running sums (fp32) of the
// row live in LDS, each with one spare quad past the row.  A workgroup holds
// four draw groups of 128 lanes that work on four draws at once; lane l of a
// group takes window positions l, l + 128, ... of its draw (the window moves,
// so the sums cannot stay in registers) and positions past the window take the
// spare quad, whose probability is 0, so the draw loop has no branches.  The
// groups' windows may overlap, so they update the running sums in turn, a
// barrier apart.  What depends on the draw
// alone -- the window offset, the label's noise, the label's loss term when the
// label lies outside the window, and the label channel's weight correction
// (weight 1 instead of nq/mq inside the window, 1 outside) -- is computed for a
// chunk of draws up front, one draw per lane, into LDS; the correction is
// summed in a register and added to the label's running sum at the end.
//
// Per draw there is one wave reduction (DPP row operations and two row
// broadcasts, no LDS round trips), one barrier that publishes the groups' wave
// sums, and the read-modify-write of the window's running sums.  The noise of
// the next draw is generated between publishing a draw's wave sum and the
// barrier, so the reduction's latency hides behind it.
#include <algorithm>

#include "dust_device.hpp"
#include "dust_internal.hpp"

namespace dust {

namespace {
constexpr int GL = 128;    // lanes per draw group
constexpr int SKC = 512;   // draws per chunk of precomputed per-draw terms
constexpr int SH = 4;      // draw groups per workgroup
constexpr float kL2e = kLog2eF;

__device__ __forceinline__ uint32_t window_offset(uint32_t tok, uint32_t draw, uint32_t layer, uint32_t k0,
                                                  uint32_t k1, uint32_t nq) {
    const u32x4 w = philox4x32_10<true>(tok, 0xFFFFFFFFu, draw, layer, k0, k1);  // every word wave-uniform
    return (uint32_t)(((uint64_t)w.x * nq) >> 32);
}

template <int DEG>
__device__ __forceinline__ float em1s(float a, const HeadArgs& A) {  // expm1(sigma a) / sigma, or expm1(sigma a)
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

template <int LT>
__device__ __forceinline__ float logit_at(const void* row, int64_t v) {
    return LT == 0 ? reinterpret_cast<const float*>(row)[v]
                   : bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[v]);
}

template <int NT>
__device__ __forceinline__ float block_reduce_max(float v, float* sh) {
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
__device__ __forceinline__ float block_reduce_sum(float v, float* sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r += sh[w];
    return r;
}

// Two floats to a pair of bf16 (round to nearest even), the first in the low half.
typedef __bf16 sbf16x2_t __attribute__((ext_vector_type(2)));
typedef float sf32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_pair(float a, float b) {
    const sf32x2_t v = {a, b};
    const sbf16x2_t h = __builtin_convertvector(v, sbf16x2_t);
    uint32_t u;
    __builtin_memcpy(&u, &h, 4);
    return u;
}

}  // namespace

// H draw groups of GL lanes each (NT = H GL lanes): group g takes draws
// g, g + H, ... of every chunk; QW window positions per lane (mq <= GL QW).
template <int LT, int DEG, int QW, int H>
__global__ void __launch_bounds__(GL * H) head_subset_kernel(HeadArgs A, int mq, float winv) {
    constexpr int NT = GL * H;
    extern __shared__ __align__(16) float lds[];
    __shared__ float sh[NT / 64];
    __shared__ float sh_red[2][H][GL / 64];
    const int t = blockIdx.x, tid = threadIdx.x;
    const int g = tid / GL, lt = tid % GL, wl = lt >> 6;  // group, lane and wave within the group
    const int V = A.V, nq = (V + 3) >> 2;
    float* P = lds;                  // [4 (nq + 1)] clean probabilities (0 past V and in the spare quad)
    float* ACC = P + 4 * (nq + 1);   // [4 (nq + 1)] running sums of r a w
    // [SKC] per draw of the current chunk: window offset (bits), the label's loss
    // term when outside the window (else 0), the label's noise, its weight correction
    float4* DR = reinterpret_cast<float4*>(ACC + 4 * (nq + 1));
    const float4* P4 = reinterpret_cast<const float4*>(P);
    float4* ACC4 = reinterpret_cast<float4*>(ACC);
    const void* row = reinterpret_cast<const unsigned char*>(A.logits) + (size_t)t * V * (LT == 0 ? 4 : 2);

    // ---- clean statistics ----------------------------------------------------
    float m = -__builtin_inff();
    for (int v = tid; v < 4 * (nq + 1); v += NT) {
        const float z = v < V ? logit_at<LT>(row, v) : -__builtin_inff();
        P[v] = z;
        ACC[v] = 0.f;
        m = fmaxf(m, z);
    }
    m = block_reduce_max<NT>(m, sh);  // its barriers publish P
    float s = 0.f;
    for (int v = tid; v < V; v += NT) s += __expf(P[v] - m);
    s = block_reduce_sum<NT>(s, sh);
    const float lse2 = (m + __logf(s)) * kL2e;
    for (int v = tid; v < 4 * (nq + 1); v += NT) P[v] = __builtin_amdgcn_exp2f(fmaf(P[v], kL2e, -lse2));
    __syncthreads();  // publishes P

    const uint32_t y = (uint32_t)A.labels[t];
    const int qy = (int)(y >> 2), cy = (int)(y & 3u);
    const uint32_t tok = A.tok0 + (uint32_t)t;
    const float cw_in = 1.0f - winv;  // label weight correction when the label is in the window
    float accy = 0.f;                 // this group's sum over its draws of r a_y (weight correction)
    const float py = P[y];            // clean probability of the label

    // One draw's window: noise a, quads q, and this lane's share of
    // sum_{v in S} p_v expm1(sigma a_v) (the label's term, when outside the
    // window, on the group's lane 0); ay, ca: the label's noise and weighted correction.
    auto gen = [&](int ii, int i0, float (&a)[QW][4], int (&q)[QW], float& ay, float& ca) -> float {
        const uint32_t draw = A.draw0 + (uint32_t)(i0 + ii);
        const float4 dr = DR[ii];
        const int o = __builtin_amdgcn_readfirstlane(__float_as_int(dr.x));
        ay = dr.z;
        ca = dr.w;
        float sl = 0.f;
#pragma unroll
        for (int k = 0; k < QW; ++k) {
            const int j = lt + k * GL;
            int qq = o + j;
            qq = qq >= nq ? qq - nq : qq;
            qq = j < mq ? qq : nq;  // past the window: the spare quad
            q[k] = qq;
            const f32x4 gv = gauss4_unscaled_uniform(tok, (uint32_t)qq, draw, A.layer, A.k0, A.k1);
            const float4 pq = P4[qq];
            const float pv[4] = {pq.x, pq.y, pq.z, pq.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                a[k][c] = gv.v[c];
                sl = fmaf(pv[c], em1s<DEG>(gv.v[c], A), sl);
            }
        }
        return sl + (lt == 0 ? dr.y : 0.f);
    };

    for (int i0 = 0; i0 < A.K; i0 += SKC) {
        const int kc = min(SKC, A.K - i0);
        __syncthreads();  // the previous chunk's terms fully used
        for (int i = tid; i < kc; i += NT) {
            const uint32_t draw = A.draw0 + (uint32_t)(i0 + i);
            const int o = (int)window_offset(tok, draw, A.layer, A.k0, A.k1, (uint32_t)nq);
            const int jy = qy - o < 0 ? qy - o + nq : qy - o;  // label quad's place in the window
            const bool in_w = jy < mq;
            // the same words and conversion as the window's path
            const u32x4 w = philox4x32_10<false>(tok, (uint32_t)qy, draw, A.layer, A.k0, A.k1);
            float gg[4];
            box_muller_unscaled(w.x, w.y, gg[0], gg[1]);
            box_muller_unscaled(w.z, w.w, gg[2], gg[3]);
            const float ay = cy == 0 ? gg[0] : cy == 1 ? gg[1] : cy == 2 ? gg[2] : gg[3];
            DR[i] = make_float4(__int_as_float(o), in_w ? 0.f : py * em1s<DEG>(ay, A), ay, (in_w ? cw_in : 1.0f) * ay);
        }
        __syncthreads();

        const int steps = (kc + H - 1) / H;
        float a[QW][4], an[QW][4];
        int q[QW], qn[QW];
        float ay, ayn, ca, can;
        float sl = gen(min(g, kc - 1), i0, a, q, ay, ca);
        float rv = 0.f;  // lane l keeps the reward of this group's step l (mod GL) until it is written
        for (int st = 0; st < steps; ++st) {
            const int ii = st * H + g;  // this group's draw
            const int b = st & 1;
            sh_red[b][g][wl] = wave_total(sl);  // every lane of the wave writes the same value
            sl = gen(min(ii + H, kc - 1), i0, an, qn, ayn, can);
            __syncthreads();  // publishes the wave sums; orders the last group's updates before group 0's
            float S = sh_red[b][g][0];
#pragma unroll
            for (int w = 1; w < GL / 64; ++w) S += sh_red[b][g][w];
            const float r0 = A.sigma * ay - log1p_uniform(S * A.smul);
            const float r = ii < kc ? r0 : 0.f;  // a group past the chunk's last draw adds nothing
            const float rw = r * winv;
            // the groups update the running sums in turn (their windows may overlap)
#pragma unroll
            for (int h = 0; h < H; ++h) {
                if (g == h) {
#pragma unroll
                    for (int k = 0; k < QW; ++k) {
                        float4 acc = ACC4[q[k]];
                        acc.x = fmaf(rw, a[k][0], acc.x);
                        acc.y = fmaf(rw, a[k][1], acc.y);
                        acc.z = fmaf(rw, a[k][2], acc.z);
                        acc.w = fmaf(rw, a[k][3], acc.w);
                        ACC4[q[k]] = acc;
                    }
                }
                if (h + 1 < H) __syncthreads();
            }
            accy = fmaf(r, ca, accy);
            rv = (st & (GL - 1)) == lt ? r : rv;
            if ((st & (GL - 1)) == GL - 1 || st == steps - 1) {  // uniform
                const int sb = (st & ~(GL - 1)) + lt;  // the step whose reward this lane holds
                const int ib = sb * H + g;
                if (A.rewards && sb <= st && ib < kc) A.rewards[(size_t)(i0 + ib) * A.T + t] = rv;
            }
#pragma unroll
            for (int k = 0; k < QW; ++k) {
                q[k] = qn[k];
#pragma unroll
                for (int c = 0; c < 4; ++c) a[k][c] = an[k][c];
            }
            ay = ayn;
            ca = can;
        }
    }
    __syncthreads();
    if (lt == 0) sh[g] = accy;
    __syncthreads();
    if (tid == 0) {
        float cy_sum = 0.f;
#pragma unroll
        for (int h = 0; h < H; ++h) cy_sum += sh[h];
        ACC[y] += cy_sum;
    }
    __syncthreads();

    // ---- g_hat_t = -(1/(K sigma)) sum_i r a w ---------------------------------
    // fp32 row and/or the bf16 pairs (hi = bf16(g), lo = bf16(g - hi)) that the
    // outer product consumes, token-major with the row zero-padded to ldp
    float* out = A.ghat ? A.ghat + (size_t)t * V : nullptr;
    uint16_t* ohi = A.ghi ? A.ghi + (size_t)t * A.ldp : nullptr;
    uint16_t* olo = A.ghi ? A.glo + (size_t)t * A.ldp : nullptr;
    const int nqo = ohi ? (int)((A.ldp + 3) / 4) : nq;
    for (int qq = tid; qq < nqo; qq += NT) {
        float v[4];
        const float4 o = qq < nq ? ACC4[qq] : make_float4(0.f, 0.f, 0.f, 0.f);
        v[0] = o.x; v[1] = o.y; v[2] = o.z; v[3] = o.w;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = 4 * qq + c < V ? v[c] * A.gscale : 0.f;
        if (ohi && 4 * (int64_t)qq < A.ldp) {
            uint2 h, l;
            h.x = pack_bf16_pair(v[0], v[1]);
            h.y = pack_bf16_pair(v[2], v[3]);
            l.x = pack_bf16_pair(v[0] - __uint_as_float(h.x << 16), v[1] - __uint_as_float(h.x & 0xFFFF0000u));
            l.y = pack_bf16_pair(v[2] - __uint_as_float(h.y << 16), v[3] - __uint_as_float(h.y & 0xFFFF0000u));
            *reinterpret_cast<uint2*>(ohi + 4 * qq) = h;
            *reinterpret_cast<uint2*>(olo + 4 * qq) = l;
        }
        if (out && qq < nq) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (4 * qq + c < V) out[4 * qq + c] = v[c];
        }
    }
}

// ---- rows beyond LDS (V > 16384): a rewards pass, then an accumulation pass ----
//
// The probabilities and the running sums of a wide row do not fit in LDS
// together.  The rewards pass recomputes p per window channel from the logits
// in global memory (below); every wave works on whole draws, so the wave's own
// reduction gives S and the draw loop has no barrier.  It writes r and the
// window offset o of every (draw, token).  The accumulation pass gives each workgroup one
// vocabulary segment of one token with the running sums in registers (lane l
// owns quads l, l + 256, ... of the segment); per draw it regenerates the
// noise of the segment's quads that lie in the window (and of the label quad),
// skipping 64-quad blocks the window misses, and adds r a / pi.  The noise is
// generated twice, once per pass.
constexpr int RNT = 256;   // rewards pass: lanes per workgroup
constexpr int BNT = 256;   // accumulation pass: lanes per workgroup
constexpr int BQS = 8;    // accumulation pass: quads per lane (segments of BNT * BQS quads)

// Quad q of a row as fp32, -inf past V (the spare quad q = nq included).
template <int LT>
__device__ __forceinline__ f32x4 global_quad(const void* row, int q, int V) {
    f32x4 z;
    if ((V & 3) == 0 && 4 * q < V) {  // whole quads: one aligned load
        if (LT == 0) {
            const float4 v = reinterpret_cast<const float4*>(row)[q];
            z.v[0] = v.x; z.v[1] = v.y; z.v[2] = v.z; z.v[3] = v.w;
        } else {
            const uint2 v = reinterpret_cast<const uint2*>(row)[q];
            z.v[0] = __uint_as_float(v.x << 16);
            z.v[1] = __uint_as_float(v.x & 0xFFFF0000u);
            z.v[2] = __uint_as_float(v.y << 16);
            z.v[3] = __uint_as_float(v.y & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) z.v[c] = 4 * q + c < V ? logit_at<LT>(row, 4 * q + c) : -__builtin_inff();
    }
    return z;
}

// Rewards pass of the wide rows: one workgroup of RNT lanes per token and no row
// in LDS, so that several tokens share a CU and hide each other's memory
// latency.  The statistics stream the row twice (maximum, then the sum of
// exponentials; the second read mostly hits the caches), RB quads per lane in
// flight at a time.  Each wave takes whole draws (wave w: draws w, w + 4, ...)
// and reads its window's logits from global memory, four quads per lane at once;
// its own DPP reduction gives S, so the draw loop has no barrier.  It writes r
// and the window offset of every (draw, token) as one pair, token-major, so the
// accumulation pass reads a token's pairs as one contiguous run (and r into the
// caller's [K, T] rewards when asked for).  A 1024-lane workgroup per token
// with the row staged in LDS (100 KB at the 243M shape: one token per CU) took
// 0.79 ms per launch there.
constexpr int RB = 8;   // quads per lane and batch of the statistics' loads

template <int LT, int DEG>
__global__ void __launch_bounds__(RNT) head_subset_rewards_kernel(HeadArgs A, int mq, float2* __restrict__ ro) {
    __shared__ float4 DR[SKC];
    __shared__ float sh[RNT / 64];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int V = A.V, nq = (V + 3) >> 2;
    const void* row = reinterpret_cast<const unsigned char*>(A.logits) + (size_t)t * V * (LT == 0 ? 4 : 2);

    // ---- clean statistics, streamed ----
    float m = -__builtin_inff();
    for (int q0 = tid; q0 < nq; q0 += RB * RNT) {
        f32x4 z[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) z[u] = global_quad<LT>(row, min(q0 + u * RNT, nq), V);
#pragma unroll
        for (int u = 0; u < RB; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) m = fmaxf(m, z[u].v[c]);
    }
    m = block_reduce_max<RNT>(m, sh);
    float s = 0.f;
    for (int q0 = tid; q0 < nq; q0 += RB * RNT) {
        f32x4 z[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) z[u] = global_quad<LT>(row, min(q0 + u * RNT, nq), V);
#pragma unroll
        for (int u = 0; u < RB; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) s += __expf(z[u].v[c] - m);
    }
    s = block_reduce_sum<RNT>(s, sh);
    const float lse2 = (m + __logf(s)) * kL2e;

    const uint32_t y = (uint32_t)A.labels[t];
    const int qy = (int)(y >> 2), cy = (int)(y & 3u);
    const uint32_t tok = A.tok0 + (uint32_t)t;
    const float py = __builtin_amdgcn_exp2f(fmaf(logit_at<LT>(row, y), kL2e, -lse2));

    for (int i0 = 0; i0 < A.K; i0 += SKC) {
        const int kc = min(SKC, A.K - i0);
        __syncthreads();  // the previous chunk's terms fully used
        for (int i = tid; i < kc; i += RNT) {
            const uint32_t draw = A.draw0 + (uint32_t)(i0 + i);
            const int o = (int)window_offset(tok, draw, A.layer, A.k0, A.k1, (uint32_t)nq);
            const int jy = qy - o < 0 ? qy - o + nq : qy - o;
            const bool in_w = jy < mq;
            const u32x4 w = philox4x32_10<false>(tok, (uint32_t)qy, draw, A.layer, A.k0, A.k1);
            float gg[4];
            box_muller_unscaled(w.x, w.y, gg[0], gg[1]);
            box_muller_unscaled(w.z, w.w, gg[2], gg[3]);
            const float ay = cy == 0 ? gg[0] : cy == 1 ? gg[1] : cy == 2 ? gg[2] : gg[3];
            DR[i] = make_float4(__int_as_float(o), in_w ? 0.f : py * em1s<DEG>(ay, A), ay, 0.f);
        }
        __syncthreads();
        for (int ii = wv; ii < kc; ii += RNT / 64) {  // wave-uniform
            const uint32_t draw = A.draw0 + (uint32_t)(i0 + ii);
            const float4 dr = DR[ii];
            const int o = __builtin_amdgcn_readfirstlane(__float_as_int(dr.x));
            float sl[4] = {0.f, 0.f, 0.f, 0.f};
            for (int j0 = 0; j0 < mq; j0 += 256) {
                int q[4];
                f32x4 z[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = j0 + 64 * u + lane;
                    int qq = o + j;
                    qq = qq >= nq ? qq - nq : qq;
                    q[u] = j < mq ? qq : nq;  // past the window: the spare quad (probability 0)
                    z[u] = global_quad<LT>(row, q[u], V);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f32x4 g = gauss4_unscaled_uniform(tok, (uint32_t)q[u], draw, A.layer, A.k0, A.k1);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        sl[u] = fmaf(__builtin_amdgcn_exp2f(fmaf(z[u].v[c], kL2e, -lse2)), em1s<DEG>(g.v[c], A),
                                     sl[u]);
                }
            }
            const float S = wave_total((sl[0] + sl[1]) + (sl[2] + sl[3])) + dr.y;
            const float r = A.sigma * dr.z - log1p_uniform(S * A.smul);
            if (lane == 0) {
                ro[(size_t)t * A.K + i0 + ii] = make_float2(r, __int_as_float(o));
                if (A.rewards) A.rewards[(size_t)(i0 + ii) * A.T + t] = r;
            }
        }
    }
}

__global__ void __launch_bounds__(BNT) head_subset_accum_kernel(HeadArgs A, int mq, float winv, int nseg,
                                                                const float2* __restrict__ ro) {
    __shared__ float2 dro[SKC];   // (r, window offset) of a chunk of draws
    const int t = blockIdx.x / nseg, sg = blockIdx.x % nseg, tid = threadIdx.x;
    const int V = A.V, nq = (V + 3) >> 2;
    const int qbase = sg * BNT * BQS + tid;
    const uint32_t y = (uint32_t)A.labels[t];
    const int qy = (int)(y >> 2), cy = (int)(y & 3u);
    const uint32_t tok = A.tok0 + (uint32_t)t;
    float acc[BQS][4];
#pragma unroll
    for (int k = 0; k < BQS; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[k][c] = 0.f;
    // this wave's 64-quad blocks start at wq0 + k BNT
    const int wq0 = sg * BNT * BQS + __builtin_amdgcn_readfirstlane(tid & ~63);
    // bit k: the blocks [wq0 + k BNT, + 64) that meet a quad range [lo, hi), all
    // wave-uniform: k BNT < hi - wq0 and k BNT > lo - wq0 - 64
    auto block_bits = [&](int lo, int hi) -> uint32_t {
        const int khi = min(BQS, max(0, (hi - wq0 + BNT - 1) >> 8));
        const int klo = max(0, ((lo - wq0 - 64) >> 8) + 1);   // arithmetic shift: floor
        return khi > klo ? ((1u << khi) - 1u) & ~((1u << klo) - 1u) : 0u;
    };
    static_assert(BNT == 256, "block_bits divides by BNT with a shift");
    // the label channel carries weight r in every draw: its running sum is kept
    // apart (accy, on the lane that owns it) and replaces that channel's window
    // sum at the end; per-block label tests in the draw loop had kept one scalar
    // mask per block live across it (scalar registers spilled)
    const int dy = qy - wq0;
    const bool lwave = dy >= 0 && dy < BQS * BNT && (dy & (BNT - 1)) < 64;   // wave-uniform
    const int ky = dy >> 8;
    const bool lowner = lwave && (threadIdx.x & 63) == (dy & 63);
    float accy = 0.f;
    // the token's (r, o) pairs staged in LDS by chunk: one coalesced read, where a
    // scalar load per draw left each wave waiting on a chain of load latencies
    for (int i0 = 0; i0 < A.K; i0 += SKC) {
      const int kc = min(SKC, A.K - i0);
      __syncthreads();  // the previous chunk fully read
      for (int i = tid; i < kc; i += BNT) dro[i] = ro[(size_t)t * A.K + i0 + i];
      __syncthreads();
      for (int i = 0; i < kc; ++i) {
        const float2 pr = dro[i];  // one address for the whole wave
        const int o = __builtin_amdgcn_readfirstlane(__float_as_int(pr.y));
        const float r = pr.x;
        const float rw = r * winv;
        const uint32_t draw = A.draw0 + (uint32_t)(i0 + i);
        // the window as [o, e1) and, when it wraps, [0, e2)
        const int e1 = min(o + mq, nq), e2 = o + mq - nq;
        // the blocks that the window or the label meet, as one mask built once per
        // draw: a few scalar instructions, where a test per block cost a dozen
        const uint32_t hits = block_bits(o, e1) | (e2 > 0 ? block_bits(0, e2) : 0u);
        if (lwave) {  // the label's noise, the same counter as its block's
            const f32x4 gy = gauss4_unscaled_uniform(tok, (uint32_t)qy, draw, A.layer, A.k0, A.k1);
            const float ay = cy == 0 ? gy.v[0] : cy == 1 ? gy.v[1] : cy == 2 ? gy.v[2] : gy.v[3];
            accy = fmaf(r, ay, accy);
        }
#pragma unroll
        for (int k = 0; k < BQS; ++k) {
            if ((hits >> k) & 1u) {  // blocks the window misses cost no vector work
                const int q = qbase + k * BNT;
                const bool in = q < nq && ((q >= o && q < e1) || q < e2);
                const f32x4 g = gauss4_unscaled_uniform(tok, (uint32_t)q, draw, A.layer, A.k0, A.k1);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[k][c] = fmaf(in ? rw : 0.f, g.v[c], acc[k][c]);   // window: nq/mq
            }
        }
      }
    }
    // the output rows formed here, opaque to the compiler: addresses derived from
    // them are not hoisted into scalar registers that would live across the draws
    uint64_t ob = (uint64_t)(uintptr_t)A.ghat, hb = (uint64_t)(uintptr_t)A.ghi, lb = (uint64_t)(uintptr_t)A.glo;
    asm volatile("" : "+s"(ob), "+s"(hb), "+s"(lb));
    float* out = ob ? reinterpret_cast<float*>(ob) + (size_t)t * V : nullptr;
    uint16_t* ohi = hb ? reinterpret_cast<uint16_t*>(hb) + (size_t)t * A.ldp : nullptr;
    uint16_t* olo = hb ? reinterpret_cast<uint16_t*>(lb) + (size_t)t * A.ldp : nullptr;
#pragma unroll
    for (int k = 0; k < BQS; ++k) {
        const int q = qbase + k * BNT;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float a = (lowner && k == ky && c == cy) ? accy : acc[k][c];   // the label: weight 1
            v[c] = 4 * q + c < V ? a * A.gscale : 0.f;
        }
        if (ohi && 4 * (int64_t)q < A.ldp) {
            uint2 h, l;
            h.x = pack_bf16_pair(v[0], v[1]);
            h.y = pack_bf16_pair(v[2], v[3]);
            l.x = pack_bf16_pair(v[0] - __uint_as_float(h.x << 16), v[1] - __uint_as_float(h.x & 0xFFFF0000u));
            l.y = pack_bf16_pair(v[2] - __uint_as_float(h.y << 16), v[3] - __uint_as_float(h.y & 0xFFFF0000u));
            *reinterpret_cast<uint2*>(ohi + 4 * q) = h;
            *reinterpret_cast<uint2*>(olo + 4 * q) = l;
        }
        if (out && q < nq) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (4 * q + c < V) out[4 * q + c] = v[c];
        }
    }
}

// P and ACC hold 4 (nq + 1) floats each, DR SKC float4s.
size_t head_subset_lds_bytes(int64_t V) { return (size_t)(8 * ((V + 3) / 4 + 1) + 4 * SKC) * sizeof(float); }


int head_subset_qw(int64_t m, int64_t V) {
    const int64_t nq = (V + 3) / 4, mq = m / 4 < nq ? m / 4 : nq;
    for (int qw : {1, 2, 4, 8, 16})
        if (mq <= (int64_t)GL * qw) return qw;
    return 0;
}

hipError_t launch_head_subset(const HeadPlan& plan, int logits_dtype, const HeadArgs& A, int64_t m, float2* ro_ws,
                              hipStream_t stream) {
    const int64_t nq = (A.V + 3) / 4, mq = m / 4 < nq ? m / 4 : nq;
    // the subset kernels come in degrees 4 and 6: degree 3 runs as 4 (a smaller
    // truncation, same coefficients)
    const int pdeg = plan.deg == 3 ? 4 : plan.deg;
    if (A.V > kSubsetLdsMaxV) {  // two passes
        const float winv = (float)((double)nq / (double)mq);
        hipError_t e = hipErrorInvalidConfiguration;
#define DUST_WIDE_CASE(LT_, DEG_)                                                                      \
        if (logits_dtype == LT_ && pdeg == DEG_) {                                                \
            hipLaunchKernelGGL((head_subset_rewards_kernel<LT_, DEG_>), dim3(A.T), dim3(RNT), 0, stream, A, \
                               (int)mq, ro_ws);                                                        \
            e = hipGetLastError();                                                                     \
        }
        DUST_WIDE_CASE(0, 4) DUST_WIDE_CASE(0, 6) DUST_WIDE_CASE(0, 0)
        DUST_WIDE_CASE(1, 4) DUST_WIDE_CASE(1, 6) DUST_WIDE_CASE(1, 0)
#undef DUST_WIDE_CASE
        if (e != hipSuccess) return e;
        const int64_t nqo = A.ghi ? std::max<int64_t>(nq, (A.ldp + 3) / 4) : nq;
        const int nseg = (int)((nqo + BNT * BQS - 1) / (BNT * BQS));
        hipLaunchKernelGGL(head_subset_accum_kernel, dim3((unsigned)(A.T * nseg)), dim3(BNT), 0, stream, A, (int)mq,
                           winv, nseg, ro_ws);
        return hipGetLastError();
    }
    const int qw = head_subset_qw(m, A.V);
    const size_t lds = head_subset_lds_bytes(A.V);
    const float winv = (float)((double)nq / (double)mq);
    hipError_t e = hipErrorInvalidConfiguration;
#define DUST_SUBSET_CASE(LT_, DEG_, QW_)                                                               \
    if (logits_dtype == LT_ && pdeg == DEG_ && qw == QW_) {                                        \
        auto k = head_subset_kernel<LT_, DEG_, QW_, SH>;                                                   \
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),                                 \
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess) \
            return e;                                                                                  \
        hipLaunchKernelGGL(k, dim3(A.T), dim3(GL * SH), lds, stream, A, (int)mq, winv);                    \
        return hipGetLastError();                                                                      \
    }
#define DUST_SUBSET_QW(LT_, DEG_)                                                                      \
    DUST_SUBSET_CASE(LT_, DEG_, 1) DUST_SUBSET_CASE(LT_, DEG_, 2) DUST_SUBSET_CASE(LT_, DEG_, 4)       \
    DUST_SUBSET_CASE(LT_, DEG_, 8) DUST_SUBSET_CASE(LT_, DEG_, 16)
    DUST_SUBSET_QW(0, 4) DUST_SUBSET_QW(0, 6) DUST_SUBSET_QW(0, 0)
    DUST_SUBSET_QW(1, 4) DUST_SUBSET_QW(1, 6) DUST_SUBSET_QW(1, 0)
#undef DUST_SUBSET_QW
#undef DUST_SUBSET_CASE
    return e;
}

}  // namespace dust
