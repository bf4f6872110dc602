/*
 * Oracle for the Dust per-token activation-perturbation gradient estimator.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * CPU reference that the HIP path is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It shares
 * no code, header, table or helper with the HIP library.
 *
 * Everything here is fp64 unless a step of the method fixes another precision.
 *
 * Sources (the web pages about Dust, Q Labs 2026):
 *  [TLDR]  "Dust: zeroth-order Transformer pretraining without backprop"
 *          (agentlenshq.com, zh), section 1, sub-heads "activation-space
 *          perturbation" and "credit assignment without backprop": the
 *          per-token reward, the output-error estimate g_hat_t and the weight
 *          gradient G_W = sum_t g_hat_t x_t^T.
 *  [NEWS]  "Training Transformers without backprop: Dust zeroth-order
 *          breakthrough" (tahou.com, zh), mechanism paragraph: Gaussian noise
 *          added to every layer output, independently per token; LM head
 *          perturbed directly on cached logits, only the loss recomputed.
 *  [IITOG] "Dust: pretraining transformers without backpropagation"
 *          (iitog.ru, ru), paragraph on the mechanics: noise on each linear
 *          output per token, rewarded by the change of that token's loss.
 *
 * Noise stream (the pages only say "independent Gaussian per token"; the
 * counter layout below is this implementation's fixed reading, shared by the
 * HIP path through its own independent code):
 *   Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *   easy as 1, 2, 3", SC'11), key = (lo32(seed), hi32(seed)),
 *   counter = (token, channel >> 2, draw, layer).
 *   Box-Muller (1958) on each half of the 4-word output: for pair p in {0,1},
 *     u1 = ((w[2p] >> 8) + 1) * 2^-24 in (0, 1],
 *     u2 = (w[2p+1] >> 8) * 2^-24   in [0, 1),
 *     rho = sqrt(-2 ln u1),
 *     a[4q + 2p] = rho cos(2 pi u2),  a[4q + 2p + 1] = rho sin(2 pi u2).
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

/* Threads the OpenMP loops below use. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One Philox4x32 round: two 32x32->64 products, the high halves xored with
 * the other two counter words and the round key (SC'11, section 3.3). */
static void philox_round(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c[2];
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

/* Philox4x32 with 10 rounds; the key is bumped by the Weyl constants before
 * every round but the first. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        philox_round(c, k0, k1);
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* Box-Muller on one (w_even, w_odd) pair of Philox words, in fp64. */
static void box_muller(uint32_t we, uint32_t wo, double *c, double *s)
{
    const double two_m24 = 1.0 / 16777216.0;
    double u1 = (double)((we >> 8) + 1u) * two_m24;
    double u2 = (double)(wo >> 8) * two_m24;
    double rho = sqrt(-2.0 * log(u1));
    double ang = 2.0 * M_PI * u2;
    *c = rho * cos(ang);
    *s = rho * sin(ang);
}

/* The raw Philox words for channels [0, n) of one (draw, token):
 * quad q -> raw[4q .. 4q+3].  raw has 4 * ceil(n/4) entries. */
void orc_noise_raw(uint64_t seed, uint32_t layer, uint32_t draw, uint32_t token,
                   int64_t n, uint32_t *raw)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    int64_t nq = (n + 3) / 4;
    for (int64_t q = 0; q < nq; ++q) {
        uint32_t ctr[4] = {token, (uint32_t)q, draw, layer};
        orc_philox4x32_10(ctr, key, raw + 4 * q);
    }
}

/* Standard-normal noise a[c], c in [0, n), for one (draw, token). */
void orc_noise(uint64_t seed, uint32_t layer, uint32_t draw, uint32_t token,
               int64_t n, double *a)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    int64_t nq = (n + 3) / 4;
    for (int64_t q = 0; q < nq; ++q) {
        uint32_t ctr[4] = {token, (uint32_t)q, draw, layer};
        uint32_t w[4];
        double v[4];
        orc_philox4x32_10(ctr, key, w);
        box_muller(w[0], w[1], &v[0], &v[1]);
        box_muller(w[2], w[3], &v[2], &v[3]);
        for (int j = 0; j < 4; ++j)
            if (4 * q + j < n) a[4 * q + j] = v[j];
    }
}

/* Noise for a block of draws and tokens: out[(i*T + t)*n + c] =
 * a(draw_offset + i, token_offset + t, c). */
void orc_noise_block(uint64_t seed, uint32_t layer, uint32_t draw_offset, int64_t K,
                     uint32_t token_offset, int64_t T, int64_t n, double *out)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < K; ++i)
        for (int64_t t = 0; t < T; ++t)
            orc_noise(seed, layer, draw_offset + (uint32_t)i, token_offset + (uint32_t)t,
                      n, out + (i * T + t) * n);
}

/* Per-token cross-entropy of one logit row: log-sum-exp minus the label logit. */
static double row_ce(const double *z, int64_t V, int32_t y)
{
    double m = z[0];
    for (int64_t v = 1; v < V; ++v) if (z[v] > m) m = z[v];
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s += exp(z[v] - m);
    return m + log(s) - z[y];
}

/*
 * LM-head estimator on cached logits ([NEWS] mechanism; [TLDR] section 1,
 * "reducing interference": the head is jittered on cached logits and only the
 * loss is recomputed).  For every token t and draw i:
 *   z~   = z_t + sigma * a_t^(i)             (full vocabulary)
 *   r    = CE(z_t) - CE(z~)                   (loss reduction at token t)
 *   ghat_t = -(1/(K sigma)) sum_i r a_t^(i)   ([TLDR] eq. for g_hat_t)
 * Outputs: ghat [T,V]; rewards [K,T] and ce0 [T] when non-NULL.
 */
void orc_head_estimate(const double *logits, const int32_t *labels,
                       int64_t T, int64_t V, int64_t K, double sigma,
                       uint64_t seed, uint32_t layer, uint32_t token_offset,
                       uint32_t draw_offset, double *ghat, double *rewards, double *ce0)
{
    #pragma omp parallel
    {
        double *a = (double *)malloc((size_t)V * sizeof(double));
        double *zt = (double *)malloc((size_t)V * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            const double *z = logits + t * V;
            int32_t y = labels[t];
            double c0 = row_ce(z, V, y);
            if (ce0) ce0[t] = c0;
            double *g = ghat + t * V;
            for (int64_t v = 0; v < V; ++v) g[v] = 0.0;
            for (int64_t i = 0; i < K; ++i) {
                orc_noise(seed, layer, draw_offset + (uint32_t)i, token_offset + (uint32_t)t, V, a);
                for (int64_t v = 0; v < V; ++v) zt[v] = z[v] + sigma * a[v];
                double r = c0 - row_ce(zt, V, y);
                if (rewards) rewards[i * T + t] = r;
                for (int64_t v = 0; v < V; ++v) g[v] += r * a[v];
            }
            double scale = -1.0 / ((double)K * sigma);
            for (int64_t v = 0; v < V; ++v) g[v] *= scale;
        }
        free(a);
        free(zt);
    }
}


/*
 * Vocabulary-subset head estimator ([TLDR] section 1, "reducing interference":
 * only part of the vocabulary is perturbed per head draw; the pages give no
 * rule).  Reading: per (token, draw) the subset S is a window of mq = m/4
 * consecutive channel quads, cyclic over the nq = ceil(V/4) quads, at an
 * offset o drawn from word 0 of Philox4x32-10 on the counter
 * (token, 0xFFFFFFFF, draw, layer) as o = (w * nq) >> 32, plus the label.
 * The noise on S is the full estimator's a_v; outside S nothing is perturbed;
 * the loss is the plain cross-entropy of the perturbed row.  Each channel is
 * weighted by the inverse of its inclusion probability pi_v (mq/nq for window
 * channels, 1 for the label), which keeps the estimate unbiased:
 *   ghat_v = -(1/(K sigma)) sum_i r_i a_v^(i) 1[v in S_i] / pi_v.
 * With mq >= nq the window is the whole vocabulary and this is
 * orc_head_estimate.
 */
uint32_t orc_window_offset(uint64_t seed, uint32_t layer, uint32_t draw, uint32_t token, uint32_t nq)
{
    uint32_t ctr[4] = {token, 0xFFFFFFFFu, draw, layer};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return (uint32_t)(((uint64_t)out[0] * (uint64_t)nq) >> 32);
}

void orc_head_estimate_subset(const double *logits, const int32_t *labels,
                              int64_t T, int64_t V, int64_t K, int64_t m, double sigma,
                              uint64_t seed, uint32_t layer, uint32_t token_offset,
                              uint32_t draw_offset, double *ghat, double *rewards, double *ce0)
{
    const int64_t nq = (V + 3) / 4;
    const int64_t mq = m / 4 < nq ? m / 4 : nq;
    const double pi_win = (double)mq / (double)nq;
    #pragma omp parallel
    {
        double *a = (double *)malloc((size_t)V * sizeof(double));
        double *zt = (double *)malloc((size_t)V * sizeof(double));
        unsigned char *in = (unsigned char *)malloc((size_t)V);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            const double *z = logits + t * V;
            int32_t y = labels[t];
            double c0 = row_ce(z, V, y);
            if (ce0) ce0[t] = c0;
            double *g = ghat + t * V;
            for (int64_t v = 0; v < V; ++v) g[v] = 0.0;
            for (int64_t i = 0; i < K; ++i) {
                const uint32_t draw = draw_offset + (uint32_t)i, tok = token_offset + (uint32_t)t;
                const int64_t o = orc_window_offset(seed, layer, draw, tok, (uint32_t)nq);
                orc_noise(seed, layer, draw, tok, V, a);
                for (int64_t v = 0; v < V; ++v) {
                    in[v] = ((v / 4 - o + nq) % nq) < mq || v == y;
                    zt[v] = in[v] ? z[v] + sigma * a[v] : z[v];
                }
                double r = c0 - row_ce(zt, V, y);
                if (rewards) rewards[i * T + t] = r;
                for (int64_t v = 0; v < V; ++v)
                    if (in[v]) g[v] += r * a[v] / (v == y ? 1.0 : pi_win);
            }
            double scale = -1.0 / ((double)K * sigma);
            for (int64_t v = 0; v < V; ++v) g[v] *= scale;
        }
        free(a);
        free(zt);
        free(in);
    }
}

