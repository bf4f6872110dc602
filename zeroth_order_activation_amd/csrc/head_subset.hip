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
// row live in LDS; lane l takes window quads l, l + NT, ... of each draw (the
// window moves, so the sums cannot stay in registers); the label's noise for
// a chunk of draws is generated up front by all lanes into LDS, so a label
// outside the window costs no Philox inside the draw loop.
#include "dust_device.hpp"
#include "dust_internal.hpp"

namespace dust {

namespace {
constexpr int SNT = 256;    // lanes per workgroup
constexpr int SKC = 4096;   // draws per chunk of precomputed label noise
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

__device__ __forceinline__ float block_reduce_max(float v, float* sh) {
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}
__device__ __forceinline__ float block_reduce_sum(float v, float* sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}
}  // namespace

// QW: window quads per lane (mq <= SNT * QW).
template <int LT, int DEG, int QW>
__global__ void __launch_bounds__(SNT) head_subset_kernel(HeadArgs A, int mq, float winv) {
    extern __shared__ __align__(16) float lds[];
    __shared__ float sh[4];
    __shared__ float sh_red[2][4][2];
    const int t = blockIdx.x, tid = threadIdx.x, wid = tid >> 6;
    const int V = A.V, nq = (V + 3) >> 2;
    float* P = lds;               // [4 nq] clean probabilities (0 past V)
    float* ACC = lds + 4 * nq;    // [4 nq] running sums of r a w
    float* AY = ACC + 4 * nq;     // [SKC] label noise of the current chunk of draws
    const void* row = reinterpret_cast<const unsigned char*>(A.logits) + (size_t)t * V * (LT == 0 ? 4 : 2);

    // ---- clean statistics ----------------------------------------------------
    float m = -__builtin_inff();
    for (int v = tid; v < 4 * nq; v += SNT) {
        const float z = v < V ? logit_at<LT>(row, v) : -__builtin_inff();
        P[v] = z;
        ACC[v] = 0.f;
        m = fmaxf(m, z);
    }
    m = block_reduce_max(m, sh);  // its barriers publish P
    float s = 0.f;
    for (int v = tid; v < V; v += SNT) s += __expf(P[v] - m);
    s = block_reduce_sum(s, sh);
    const float lse2 = (m + __logf(s)) * kL2e;
    for (int v = tid; v < 4 * nq; v += SNT) P[v] = __builtin_amdgcn_exp2f(fmaf(P[v], kL2e, -lse2));
    // (the next barrier, in the label-noise chunk below, publishes P)

    const uint32_t y = (uint32_t)A.labels[t];
    const int qy = (int)(y >> 2), cy = (int)(y & 3u);
    const uint32_t tok = A.tok0 + (uint32_t)t;

    for (int i0 = 0; i0 < A.K; i0 += SKC) {
        const int kc = min(SKC, A.K - i0);
        __syncthreads();  // AY of the previous chunk fully used
        for (int i = tid; i < kc; i += SNT) {
            // the same words and conversion as the window's uniform-counter path
            const u32x4 w = philox4x32_10<false>(tok, (uint32_t)qy, A.draw0 + (uint32_t)(i0 + i), A.layer, A.k0, A.k1);
            float g[4];
            box_muller_unscaled(w.x, w.y, g[0], g[1]);
            box_muller_unscaled(w.z, w.w, g[2], g[3]);
            AY[i] = cy == 0 ? g[0] : cy == 1 ? g[1] : cy == 2 ? g[2] : g[3];
        }
        __syncthreads();
        for (int ii = 0; ii < kc; ++ii) {
            const int i = i0 + ii;
            const uint32_t draw = A.draw0 + (uint32_t)i;
            const int o = (int)window_offset(tok, draw, A.layer, A.k0, A.k1, (uint32_t)nq);
            const int jy = qy - o < 0 ? qy - o + nq : qy - o;  // label quad's place in the window
            const bool inw = jy < mq;                           // uniform
            float a[QW][4];
            float sl = 0.f, ly = 0.f;
#pragma unroll
            for (int k = 0; k < QW; ++k) {
                const int j = tid + k * SNT;
                if (j < mq) {
                    int q = o + j;
                    q = q >= nq ? q - nq : q;
                    const f32x4 g = gauss4_unscaled_uniform(tok, (uint32_t)q, draw, A.layer, A.k0, A.k1);
                    const float4 pq = reinterpret_cast<const float4*>(P)[q];
                    const float pv[4] = {pq.x, pq.y, pq.z, pq.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        a[k][c] = g.v[c];
                        sl = fmaf(pv[c], em1s<DEG>(g.v[c], A), sl);
                    }
                    if (j == jy) ly = cy == 0 ? g.v[0] : cy == 1 ? g.v[1] : cy == 2 ? g.v[2] : g.v[3];
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) a[k][c] = 0.f;
                }
            }
            const float ay = AY[ii];
            if (!inw && tid == 0) {  // the label alone, outside the window
                sl = fmaf(P[y], em1s<DEG>(ay, A), sl);
                ly = ay;
            }
            sl = wave_sum(sl);
            ly = wave_sum(ly);
            const int b = ii & 1;
            if ((tid & 63) == 0) { sh_red[b][wid][0] = sl; sh_red[b][wid][1] = ly; }
            __syncthreads();
            const float S = (sh_red[b][0][0] + sh_red[b][1][0]) + (sh_red[b][2][0] + sh_red[b][3][0]);
            const float LY = (sh_red[b][0][1] + sh_red[b][1][1]) + (sh_red[b][2][1] + sh_red[b][3][1]);
            const float r = A.sigma * LY - log1pf(S * A.smul);
            // running sums: each window quad belongs to one lane in this draw; the
            // barrier above separates this draw's updates from the previous one's
#pragma unroll
            for (int k = 0; k < QW; ++k) {
                const int j = tid + k * SNT;
                if (j < mq) {
                    int q = o + j;
                    q = q >= nq ? q - nq : q;
                    float4 acc = reinterpret_cast<float4*>(ACC)[q];
                    const float rw = r * winv;
                    const bool lab = j == jy;
                    acc.x = fmaf(lab && cy == 0 ? r : rw, a[k][0], acc.x);
                    acc.y = fmaf(lab && cy == 1 ? r : rw, a[k][1], acc.y);
                    acc.z = fmaf(lab && cy == 2 ? r : rw, a[k][2], acc.z);
                    acc.w = fmaf(lab && cy == 3 ? r : rw, a[k][3], acc.w);
                    reinterpret_cast<float4*>(ACC)[q] = acc;
                }
            }
            if (!inw && tid == 0) ACC[y] = fmaf(r, ay, ACC[y]);
            if (tid == 0 && A.rewards) A.rewards[(size_t)i * A.T + t] = r;
        }
    }
    __syncthreads();
    float* out = A.ghat + (size_t)t * V;
    for (int v = tid; v < V; v += SNT) out[v] = ACC[v] * A.gscale;
}

// P and ACC hold 4 nq floats each, AY SKC floats.
size_t head_subset_lds_bytes(int64_t V) { return (size_t)(8 * ((V + 3) / 4) + SKC) * sizeof(float); }

int head_subset_qw(int64_t m, int64_t V) {
    const int64_t nq = (V + 3) / 4, mq = m / 4 < nq ? m / 4 : nq;
    for (int qw : {1, 2, 4, 8, 16})
        if (mq <= (int64_t)SNT * qw) return qw;
    return 0;
}

hipError_t launch_head_subset(const HeadPlan& plan, int logits_dtype, const HeadArgs& A, int64_t m,
                              hipStream_t stream) {
    const int64_t nq = (A.V + 3) / 4, mq = m / 4 < nq ? m / 4 : nq;
    const int qw = head_subset_qw(m, A.V);
    const size_t lds = head_subset_lds_bytes(A.V);
    const float winv = (float)((double)nq / (double)mq);
    hipError_t e = hipErrorInvalidConfiguration;
#define DUST_SUBSET_CASE(LT_, DEG_, QW_)                                                               \
    if (logits_dtype == LT_ && plan.deg == DEG_ && qw == QW_) {                                        \
        auto k = head_subset_kernel<LT_, DEG_, QW_>;                                                   \
        if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),                                 \
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess) \
            return e;                                                                                  \
        hipLaunchKernelGGL(k, dim3(A.T), dim3(SNT), lds, stream, A, (int)mq, winv);                    \
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
