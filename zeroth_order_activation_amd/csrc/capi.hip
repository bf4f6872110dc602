// C ABI of the Dust estimator library: argument checks, workspace layout and
// dispatch.  Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "dust.h"
#include "dust_internal.hpp"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_stage_event[4] = {nullptr, nullptr, nullptr, nullptr};

hipError_t record_stage(int stage, hipStream_t s) {
    return g_stage_event[stage] ? hipEventRecord(g_stage_event[stage], s) : hipSuccess;
}

dust_status fail(dust_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

dust_status ok() {
    g_err.clear();
    return DUST_OK;
}

dust_status device_fail(const char* what, hipError_t e) {
    return fail(DUST_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool env_flag(const char* name) {
    const char* v = std::getenv(name);
    return v && v[0] && v[0] != '0';
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Checks shared by the estimators.  Returns DUST_OK or a failure with message.
dust_status check_common(int64_t T, int64_t K, float sigma, uint32_t token_offset, uint32_t draw_offset) {
    if (T <= 0 || T > (int64_t)INT32_MAX) return fail(DUST_E_INVALID, "T must be in [1, 2^31): got %lld", (long long)T);
    if (K <= 0 || K > (int64_t)INT32_MAX) return fail(DUST_E_INVALID, "K must be in [1, 2^31): got %lld", (long long)K);
    if (!std::isfinite(sigma) || !(sigma > 0.f)) return fail(DUST_E_INVALID, "sigma must be finite and > 0: got %g", (double)sigma);
    if ((uint64_t)token_offset + (uint64_t)T > (1ull << 32))
        return fail(DUST_E_INVALID, "token_offset + T exceeds the 32-bit token counter");
    if ((uint64_t)draw_offset + (uint64_t)K > (1ull << 32))
        return fail(DUST_E_INVALID, "draw_offset + K exceeds the 32-bit draw counter");
    return DUST_OK;
}

dust_status check_labels(const int32_t* labels, int64_t T, int64_t V, hipStream_t stream) {
    if (!env_flag("DUST_DEBUG_CHECKS")) return DUST_OK;
    std::vector<int32_t> h((size_t)T);
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipMemcpy(h.data(), labels, (size_t)T * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return device_fail("label check copy", e);
    for (int64_t t = 0; t < T; ++t)
        if (h[(size_t)t] < 0 || h[(size_t)t] >= V)
            return fail(DUST_E_INVALID, "label[%lld] = %d is outside [0, %lld)", (long long)t, h[(size_t)t], (long long)V);
    return DUST_OK;
}

size_t head_ghat_bytes(int64_t T, int64_t V) { return round_up((size_t)T * (size_t)V * sizeof(float)); }

}  // namespace

extern "C" {

int dust_abi_version(void) { return DUST_ABI_VERSION; }

const char* dust_last_error(void) { return g_err.c_str(); }

dust_status dust_set_stage_event(int stage, void* event) {
    if (stage < 0 || stage > 3) return fail(DUST_E_INVALID, "dust_set_stage_event: stage must be in [0, 3]");
    g_stage_event[stage] = static_cast<hipEvent_t>(event);
    return ok();
}

dust_status dust_noise(uint64_t seed, uint32_t layer, uint32_t draw_offset, int64_t K, uint32_t token_offset,
                       int64_t T, int64_t n, uint32_t* raw, float* gauss, void* stream) {
    if (!raw && !gauss) return fail(DUST_E_INVALID, "dust_noise: raw and gauss are both NULL");
    if (T <= 0 || K <= 0 || n <= 0) return fail(DUST_E_INVALID, "dust_noise: K, T, n must be >= 1");
    if ((uint64_t)token_offset + (uint64_t)T > (1ull << 32) || (uint64_t)draw_offset + (uint64_t)K > (1ull << 32))
        return fail(DUST_E_INVALID, "dust_noise: offset + count exceeds the 32-bit counter");
    const int64_t threads = K * T * ((n + 3) / 4);
    if (K > (int64_t)INT32_MAX || T > (int64_t)INT32_MAX || threads > ((int64_t)1 << 32) - 256)
        return fail(DUST_E_UNSUPPORTED, "dust_noise: K*T*ceil(n/4) must stay below 2^32");
    hipError_t e = dust::launch_noise_export(seed, layer, draw_offset, K, token_offset, T, n, raw, gauss,
                                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("dust_noise launch", e);
    return ok();
}

size_t dust_outer_workspace_bytes(int64_t T, int64_t n, int64_t d) {
    if (T <= 0 || n <= 0 || d <= 0) return 0;
    return dust::outer_workspace_bytes(T, n, d);
}

dust_status dust_outer_product(const float* ghat, const float* x, int64_t T, int64_t n, int64_t d, float* grad_w,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (!ghat || !x || !grad_w) return fail(DUST_E_INVALID, "dust_outer_product: null tensor pointer");
    if (!aligned16(ghat) || !aligned16(x) || !aligned16(grad_w))
        return fail(DUST_E_INVALID, "dust_outer_product: tensors must be 16-byte aligned");
    if (T <= 0 || n <= 0 || d <= 0) return fail(DUST_E_INVALID, "dust_outer_product: T, n, d must be >= 1");
    if (n > 65535LL * 128 || d > 65535LL * 128) return fail(DUST_E_UNSUPPORTED, "dust_outer_product: n or d too large");
    const size_t need = dust::outer_workspace_bytes(T, n, d);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(DUST_E_WORKSPACE, "dust_outer_product: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (workspace && !aligned16(workspace)) return fail(DUST_E_INVALID, "dust_outer_product: workspace must be 16-byte aligned");
    hipError_t e = dust::launch_outer(ghat, x, T, n, d, grad_w, workspace, workspace_bytes,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("dust_outer_product launch", e);
    return ok();
}

// g_hat needs a home of its own only when the outer product takes the fp32
// path; on the bf16-pair path the estimator writes the pairs straight into the
// outer product's workspace.
static bool head_pairs_path(int64_t T, int64_t V, int64_t d) { return dust::outer_uses_pairs(T, V, d); }

// Kernel arguments shared by the head estimators.  The kernels draw the noise
// divided by sqrt(2 ln 2) and work with sigma' = sigma sqrt(2 ln 2), so that
// sigma' a' = sigma a; the final scale takes the factor back:
// g_hat = -(1/(K sigma)) sqrt(2 ln 2) sum r a'.
static dust::HeadArgs head_args(const void* logits, const int32_t* labels, float* ghat, float* rewards, int64_t T,
                                int64_t V, int64_t K, float sigma, const dust::HeadPlan& plan, uint64_t seed,
                                uint32_t layer, uint32_t token_offset, uint32_t draw_offset) {
    dust::HeadArgs A{};
    A.logits = logits;
    A.labels = labels;
    A.ghat = ghat;
    A.rewards = rewards;
    A.T = (int32_t)T;
    A.V = (int32_t)V;
    A.K = (int32_t)K;
    const double s2 = std::sqrt(2.0 * std::log(2.0));
    const double sd = (double)sigma * s2;
    A.sigma = (float)sd;
    A.smul = plan.deg > 0 ? (float)sd : 1.0f;
    A.gscale = (float)(-s2 / ((double)K * (double)sigma));
    double ck = 1.0, fact = 1.0;
    for (int k = 0; k < 8; ++k) {  // coef[k] = sd^k / (k+1)!
        fact *= (k + 1);
        A.coef[k] = (float)(ck / fact);
        ck *= sd;
    }
    A.k0 = (uint32_t)seed;
    A.k1 = (uint32_t)(seed >> 32);
    A.layer = layer;
    A.tok0 = token_offset;
    A.draw0 = draw_offset;
    return A;
}

size_t dust_head_workspace_bytes(int64_t T, int64_t V, int64_t d, int64_t K) {
    (void)K;
    if (T <= 0 || V <= 0 || d <= 0) return 0;
    return (head_pairs_path(T, V, d) ? 0 : head_ghat_bytes(T, V)) + dust::outer_workspace_bytes(T, V, d);
}

dust_status dust_estimate_head(const void* logits, int logits_dtype, const float* x, const int32_t* labels,
                               int64_t T, int64_t V, int64_t d, int64_t K, float sigma, uint64_t seed,
                               uint32_t layer, uint32_t token_offset, uint32_t draw_offset, float* grad_w,
                               float* ghat, float* rewards, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!logits || !x || !labels || !grad_w)
        return fail(DUST_E_INVALID, "dust_estimate_head: logits, x, labels and grad_w must be non-NULL");
    if (logits_dtype != DUST_F32 && logits_dtype != DUST_BF16)
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_head: logits_dtype %d is not DUST_F32 or DUST_BF16", logits_dtype);
    if (!aligned16(logits) || !aligned16(x) || !aligned16(labels) || !aligned16(grad_w) ||
        (ghat && !aligned16(ghat)) || (rewards && !aligned16(rewards)) || (workspace && !aligned16(workspace)))
        return fail(DUST_E_INVALID, "dust_estimate_head: every pointer must be 16-byte aligned");
    dust_status s = check_common(T, K, sigma, token_offset, draw_offset);
    if (s != DUST_OK) return s;
    if (V <= 0) return fail(DUST_E_INVALID, "dust_estimate_head: V must be >= 1");
    if (d <= 0) return fail(DUST_E_INVALID, "dust_estimate_head: d must be >= 1");
    if (V > 65535LL * 128 || d > 65535LL * 128) return fail(DUST_E_UNSUPPORTED, "dust_estimate_head: V or d too large");
    const dust::HeadPlan plan = dust::plan_head(V, logits_dtype, sigma);
    if (!plan.ok) return fail(DUST_E_UNSUPPORTED, "dust_estimate_head: %s", plan.why);

    const bool pairs = head_pairs_path(T, V, d);
    const size_t ghat_ws = (ghat || pairs) ? 0 : head_ghat_bytes(T, V);
    const size_t outer_ws = dust::outer_workspace_bytes(T, V, d);
    const size_t need = ghat_ws + outer_ws;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(DUST_E_WORKSPACE, "dust_estimate_head: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    s = check_labels(labels, T, V, st);
    if (s != DUST_OK) return s;

    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* g = ghat ? ghat : (pairs ? nullptr : reinterpret_cast<float*>(ws));
    void* ows = outer_ws ? ws + ghat_ws : nullptr;
    const dust::OuterPairs pr = dust::outer_ghat_pairs(T, V, d, ows);

    dust::HeadArgs A = head_args(logits, labels, g, rewards, T, V, K, sigma, plan, seed, layer, token_offset,
                                 draw_offset);
    A.ghi = pr.hi;
    A.glo = pr.lo;
    A.ldp = pr.ld;
    if (env_flag("DUST_LOG"))
        std::fprintf(stderr, "[dust] head T=%lld V=%lld d=%lld K=%lld nt=%d q=%d pmode=%d deg=%d lds=%zu\n",
                     (long long)T, (long long)V, (long long)d, (long long)K, plan.nt, plan.q, plan.pmode, plan.deg,
                     plan.lds);
    hipError_t e = dust::launch_head(plan, logits_dtype, A, st);
    if (e != hipSuccess) return device_fail("dust_estimate_head: estimator launch", e);
    if ((e = record_stage(0, st)) != hipSuccess) return device_fail("dust_estimate_head: stage event", e);
    e = dust::launch_outer(g, x, T, V, d, grad_w, ows, outer_ws, st, pr.hi != nullptr);
    if (e != hipSuccess) return device_fail("dust_estimate_head: outer-product launch", e);
    if ((e = record_stage(1, st)) != hipSuccess) return device_fail("dust_estimate_head: stage event", e);
    return ok();
}

// bytes of K*T floats or ints, padded to 256
static size_t kt_bytes(int64_t T, int64_t K) { return ((size_t)T * (size_t)K * 4 + 255) & ~(size_t)255; }

// dynamic LDS a workgroup of the wide-row subset rewards pass may take
static constexpr size_t kMaxWideLds = 160 * 1024 - 1024;

size_t dust_head_subset_workspace_bytes(int64_t T, int64_t V, int64_t d, int64_t K) {
    // the full estimator's layout (which a covering window runs); rows wider
    // than LDS add the rewards and window offsets of every (draw, token)
    const size_t base = dust_head_workspace_bytes(T, V, d, K);
    if (base == 0 || K <= 0 || V <= dust::kSubsetLdsMaxV) return base;
    return base + 2 * kt_bytes(T, K);
}

dust_status dust_estimate_head_subset(const void* logits, int logits_dtype, const float* x, const int32_t* labels,
                                      int64_t T, int64_t V, int64_t d, int64_t K, int64_t m, float sigma,
                                      uint64_t seed, uint32_t layer, uint32_t token_offset, uint32_t draw_offset,
                                      float* grad_w, float* ghat, float* rewards, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (m < 4 || m % 4 != 0)
        return fail(DUST_E_INVALID, "dust_estimate_head_subset: m must be a positive multiple of 4 (got %lld)",
                    (long long)m);
    if (V > 0 && m / 4 >= (V + 3) / 4)  // the window is the whole vocabulary
        return dust_estimate_head(logits, logits_dtype, x, labels, T, V, d, K, sigma, seed, layer, token_offset,
                                  draw_offset, grad_w, ghat, rewards, workspace, workspace_bytes, stream);
    if (!logits || !x || !labels || !grad_w)
        return fail(DUST_E_INVALID, "dust_estimate_head_subset: logits, x, labels and grad_w must be non-NULL");
    if (logits_dtype != DUST_F32 && logits_dtype != DUST_BF16)
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_head_subset: logits_dtype %d is not DUST_F32 or DUST_BF16",
                    logits_dtype);
    if (!aligned16(logits) || !aligned16(x) || !aligned16(labels) || !aligned16(grad_w) ||
        (ghat && !aligned16(ghat)) || (rewards && !aligned16(rewards)) || (workspace && !aligned16(workspace)))
        return fail(DUST_E_INVALID, "dust_estimate_head_subset: every pointer must be 16-byte aligned");
    dust_status s = check_common(T, K, sigma, token_offset, draw_offset);
    if (s != DUST_OK) return s;
    if (V <= 0) return fail(DUST_E_INVALID, "dust_estimate_head_subset: V must be >= 1");
    if (d <= 0) return fail(DUST_E_INVALID, "dust_estimate_head_subset: d must be >= 1");
    if (V > 65535LL * 128 || d > 65535LL * 128)
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_head_subset: V or d too large");
    const dust::HeadPlan plan = dust::plan_head(V, logits_dtype, sigma);  // the Taylor degree and the row limits
    if (!plan.ok) return fail(DUST_E_UNSUPPORTED, "dust_estimate_head_subset: %s", plan.why);
    const bool wide = V > dust::kSubsetLdsMaxV;
    if (wide && dust::head_subset_wide_lds_bytes(V, logits_dtype) > kMaxWideLds)
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_head_subset: the logit row does not fit in LDS");
    const bool pairs = head_pairs_path(T, V, d);
    const size_t ghat_ws = (ghat || pairs) ? 0 : head_ghat_bytes(T, V);
    const size_t outer_ws = dust::outer_workspace_bytes(T, V, d);
    const size_t kt_ws = wide ? kt_bytes(T, K) : 0;  // rewards, then window offsets
    const size_t need = ghat_ws + outer_ws + 2 * kt_ws;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(DUST_E_WORKSPACE, "dust_estimate_head_subset: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    s = check_labels(labels, T, V, st);
    if (s != DUST_OK) return s;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* g = ghat ? ghat : (pairs ? nullptr : reinterpret_cast<float*>(ws));
    void* ows = outer_ws ? ws + ghat_ws : nullptr;
    const dust::OuterPairs pr = dust::outer_ghat_pairs(T, V, d, ows);
    dust::HeadArgs A = head_args(logits, labels, g, rewards, T, V, K, sigma, plan, seed, layer, token_offset,
                                 draw_offset);
    A.ghi = pr.hi;
    A.glo = pr.lo;
    A.ldp = pr.ld;
    float* rew_ws = wide ? reinterpret_cast<float*>(ws + ghat_ws + outer_ws) : nullptr;
    int* off_ws = wide ? reinterpret_cast<int*>(ws + ghat_ws + outer_ws + kt_ws) : nullptr;
    hipError_t e = dust::launch_head_subset(plan, logits_dtype, A, m, rew_ws, off_ws, st);
    if (e != hipSuccess) return device_fail("dust_estimate_head_subset: estimator launch", e);
    if ((e = record_stage(0, st)) != hipSuccess) return device_fail("dust_estimate_head_subset: stage event", e);
    e = dust::launch_outer(g, x, T, V, d, grad_w, ows, outer_ws, st, pr.hi != nullptr);
    if (e != hipSuccess) return device_fail("dust_estimate_head_subset: outer-product launch", e);
    if ((e = record_stage(1, st)) != hipSuccess) return device_fail("dust_estimate_head_subset: stage event", e);
    return ok();
}

size_t dust_linear_workspace_bytes(int64_t T, int64_t d, int64_t n, int64_t V, int64_t K) {
    if (T <= 0 || d <= 0 || n <= 0 || V <= 0 || K <= 0) return 0;
    return dust::mlp_layout(T, d, n, V, K).total;
}

dust_status dust_estimate_linear(const float* u, const float* h, const float* x_res, const uint16_t* w2,
                                 const uint16_t* w_head, const int32_t* labels, int64_t T, int64_t d, int64_t n,
                                 int64_t V, int64_t K, float sigma, float ln_eps, uint64_t seed, uint32_t layer,
                                 uint32_t token_offset, uint32_t draw_offset, float* grad_w, float* ghat,
                                 float* rewards, void* workspace, size_t workspace_bytes, void* stream) {
    if (!u || !h || !x_res || !w2 || !w_head || !labels || !grad_w)
        return fail(DUST_E_INVALID, "dust_estimate_linear: u, h, x_res, w2, w_head, labels and grad_w must be non-NULL");
    if (!aligned16(u) || !aligned16(h) || !aligned16(x_res) || !aligned16(w2) || !aligned16(w_head) ||
        !aligned16(labels) || !aligned16(grad_w) || (ghat && !aligned16(ghat)) || (rewards && !aligned16(rewards)) ||
        (workspace && !aligned16(workspace)))
        return fail(DUST_E_INVALID, "dust_estimate_linear: every pointer must be 16-byte aligned");
    dust_status s = check_common(T, K, sigma, token_offset, draw_offset);
    if (s != DUST_OK) return s;
    if (d <= 0 || n <= 0 || V <= 0) return fail(DUST_E_INVALID, "dust_estimate_linear: d, n, V must be >= 1");
    if (!std::isfinite(ln_eps) || !(ln_eps > 0.f))
        return fail(DUST_E_INVALID, "dust_estimate_linear: ln_eps must be finite and > 0: got %g", (double)ln_eps);
    if (d != 256 && d != 512) return fail(DUST_E_UNSUPPORTED, "dust_estimate_linear: d must be 256 or 512 (got %lld)", (long long)d);
    if (n % 32 != 0) return fail(DUST_E_UNSUPPORTED, "dust_estimate_linear: n must be a multiple of 32 (got %lld)", (long long)n);
    if (V > (int64_t)INT32_MAX / 2 || n > (int64_t)INT32_MAX / 4)
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_linear: V or n too large");
    if (T * (K + 1) > ((int64_t)1 << 40)) return fail(DUST_E_UNSUPPORTED, "dust_estimate_linear: T*(K+1) too large");
    const dust::MlpLayout L = dust::mlp_layout(T, d, n, V, K);
    if (workspace == nullptr || workspace_bytes < L.total)
        return fail(DUST_E_WORKSPACE, "dust_estimate_linear: workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    s = check_labels(labels, T, V, st);
    if (s != DUST_OK) return s;
    dust::MlpArgs A{};
    A.u = u;
    A.h = h;
    A.x_res = x_res;
    A.w2 = w2;
    A.w_head = w_head;
    A.labels = labels;
    A.rewards = rewards;
    A.T = (int32_t)T;
    A.d = (int32_t)d;
    A.n = (int32_t)n;
    A.V = (int32_t)V;
    A.K = (int32_t)K;
    A.sigma = sigma;
    A.ln_eps = ln_eps;
    A.gscale = (float)(-1.0 / ((double)K * (double)sigma));
    A.k0 = (uint32_t)seed;
    A.k1 = (uint32_t)(seed >> 32);
    A.layer = layer;
    A.tok0 = token_offset;
    A.draw0 = draw_offset;
    A.stage_event = g_stage_event[0];
    A.gemm1_event = g_stage_event[2];
    A.gemm2_event = g_stage_event[3];
    if (env_flag("DUST_LOG"))
        std::fprintf(stderr, "[dust] linear T=%lld d=%lld n=%lld V=%lld K=%lld chunk=%lld vtiles=%d ws=%zu\n",
                     (long long)T, (long long)d, (long long)n, (long long)V, (long long)K, (long long)L.chunk, L.nvt,
                     L.total);
    hipError_t e = dust::launch_mlp(A, L, static_cast<unsigned char*>(workspace), ghat, grad_w, st);
    if (e != hipSuccess) return device_fail("dust_estimate_linear: launch", e);
    if ((e = record_stage(1, st)) != hipSuccess) return device_fail("dust_estimate_linear: stage event", e);
    return ok();
}

}  // extern "C"

size_t dust_attn_workspace_bytes(int proj, int64_t T, int64_t S, int64_t d, int64_t H, int64_t K) {
    if (proj < 0 || proj > 2 || T <= 0 || S <= 0 || d <= 0 || H <= 0 || K <= 0) return 0;
    return dust::attn_layout(proj, T, S, d, H, K).total;
}

size_t dust_attn_v_workspace_bytes(int64_t T, int64_t S, int64_t d, int64_t H, int64_t K) {
    return dust_attn_workspace_bytes(DUST_ATTN_V, T, S, d, H, K);
}

dust_status dust_estimate_attn(int proj, const float* q, const float* k, const float* v, const float* e,
                               const float* u, int64_t T, int64_t S, int64_t d, int64_t H, int64_t K, float sigma,
                               uint64_t seed, uint32_t layer, uint32_t token_offset, uint32_t draw_offset,
                               float* grad_w, float* ghat, float* rewards, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (proj != DUST_ATTN_Q && proj != DUST_ATTN_K && proj != DUST_ATTN_V)
        return fail(DUST_E_INVALID, "dust_estimate_attn: proj %d is not DUST_ATTN_Q, _K or _V", proj);
    if (!q || !k || !e || !u || !grad_w || (proj != DUST_ATTN_V && !v))
        return fail(DUST_E_INVALID, "dust_estimate_attn: q, k, e, u, grad_w (and v for queries and keys) must be "
                                    "non-NULL");
    if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || !aligned16(e) || !aligned16(u) ||
        !aligned16(grad_w) || (ghat && !aligned16(ghat)) || (rewards && !aligned16(rewards)) ||
        (workspace && !aligned16(workspace)))
        return fail(DUST_E_INVALID, "dust_estimate_attn: every pointer must be 16-byte aligned");
    dust_status s = check_common(T, K, sigma, token_offset, draw_offset);
    if (s != DUST_OK) return s;
    if (S <= 0 || d <= 0 || H <= 0) return fail(DUST_E_INVALID, "dust_estimate_attn: S, d and H must be >= 1");
    if (T % S != 0)
        return fail(DUST_E_INVALID, "dust_estimate_attn: T (%lld) must be a multiple of S (%lld)", (long long)T,
                    (long long)S);
    if (d != 64 * H) return fail(DUST_E_UNSUPPORTED, "dust_estimate_attn: heads of 64 channels only (d = 64 H)");
    if (S % 64 != 0 || S > 4096)
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_attn: S must be a multiple of 64 up to 4096 (got %lld)",
                    (long long)S);
    if (T > (1LL << 31) / 64 || K * T > (1LL << 31))
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_attn: T or K*T too large");
    const dust::AttnVLayout L = dust::attn_layout(proj, T, S, d, H, K);
    if (workspace == nullptr || workspace_bytes < L.total)
        return fail(DUST_E_WORKSPACE, "dust_estimate_attn: workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* rew = rewards ? rewards : reinterpret_cast<float*>(ws + L.off_rew);
    float* g = ghat ? ghat : reinterpret_cast<float*>(ws + L.off_ghat);
    hipError_t err = dust::launch_attn_rewards(proj, q, k, v, e, T, S, d, H, K, sigma, seed, layer, token_offset,
                                               draw_offset, rew, ws, L, st);
    if (err != hipSuccess) return device_fail("dust_estimate_attn: attention passes", err);
    if ((err = record_stage(2, st)) != hipSuccess) return device_fail("dust_estimate_attn: stage event", err);
    err = dust::launch_attn_v_ghat(T, d, K, sigma, seed, layer, token_offset, draw_offset, rew, g, st);
    if (err != hipSuccess) return device_fail("dust_estimate_attn: reduction launch", err);
    if ((err = record_stage(0, st)) != hipSuccess) return device_fail("dust_estimate_attn: stage event", err);
    err = dust::launch_outer(g, u, T, d, d, grad_w, ws + L.off_outer, L.total - L.off_outer, st, false);
    if (err != hipSuccess) return device_fail("dust_estimate_attn: outer-product launch", err);
    if ((err = record_stage(1, st)) != hipSuccess) return device_fail("dust_estimate_attn: stage event", err);
    return ok();
}

dust_status dust_estimate_attn_v(const float* q, const float* k, const float* e, const float* u, int64_t T,
                                 int64_t S, int64_t d, int64_t H, int64_t K, float sigma, uint64_t seed,
                                 uint32_t layer, uint32_t token_offset, uint32_t draw_offset, float* grad_w,
                                 float* ghat, float* rewards, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return dust_estimate_attn(DUST_ATTN_V, q, k, nullptr, e, u, T, S, d, H, K, sigma, seed, layer, token_offset,
                              draw_offset, grad_w, ghat, rewards, workspace, workspace_bytes, stream);
}
