// C ABI of the Dust estimator library: argument checks, workspace layout and
// dispatch.  Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "dust.h"
#include "dust_internal.hpp"
#include "launch_events.hpp"
#include "lm_internal.hpp"

namespace dust {
thread_local LaunchEvents g_kernel_events[kTimedKernels];
}

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_stage_event[8] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};

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
dust_status check_common(int64_t T, int64_t K, float sigma, uint64_t token_offset, uint32_t draw_offset) {
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

// Scratch of dust_estimate_head_noalloc: one array per GPU, part of the code object,
// so no call allocates.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns, fetched once per device with that device current.
#define DUST_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
static __device__ __align__(256) unsigned char scratch[DUST_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
dust_status scratch_for_current_device(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_fail(fn, e);
    if (dev < 0 || dev >= kMaxDevices) return fail(DUST_E_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return device_fail("hipGetSymbolAddress(scratch)", e);
        if (!p) return fail(DUST_E_DEVICE, "%s: hipGetSymbolAddress(scratch) gave NULL", fn);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DUST_OK;
}

}  // namespace

extern "C" {

int dust_abi_version(void) { return DUST_ABI_VERSION; }

const char* dust_last_error(void) { return g_err.c_str(); }

dust_status dust_set_stage_event(int stage, void* event) {
    if (stage < 0 || stage > 7) return fail(DUST_E_INVALID, "dust_set_stage_event: stage must be in [0, 7]");
    g_stage_event[stage] = static_cast<hipEvent_t>(event);
    return ok();
}

dust_status dust_set_kernel_events(int kernel, void* const* starts, void* const* ends, int capacity) {
    static thread_local std::vector<hipEvent_t> s_starts[dust::kTimedKernels], s_ends[dust::kTimedKernels];
    if (kernel < 0 || kernel >= dust::kTimedKernels)
        return fail(DUST_E_INVALID, "dust_set_kernel_events: kernel must be in [0, %d)", (int)dust::kTimedKernels);
    dust::LaunchEvents& le = dust::g_kernel_events[kernel];
    if (!starts || !ends || capacity <= 0) {
        le = dust::LaunchEvents{};
        return ok();
    }
    s_starts[kernel].assign(reinterpret_cast<hipEvent_t const*>(starts),
                            reinterpret_cast<hipEvent_t const*>(starts) + capacity);
    s_ends[kernel].assign(reinterpret_cast<hipEvent_t const*>(ends), reinterpret_cast<hipEvent_t const*>(ends) + capacity);
    le.starts = s_starts[kernel].data();
    le.ends = s_ends[kernel].data();
    le.capacity = capacity;
    le.count = 0;
    return ok();
}

int dust_kernel_event_count(int kernel) {
    return kernel >= 0 && kernel < dust::kTimedKernels ? dust::g_kernel_events[kernel].count : -1;
}

dust_status dust_noise(uint64_t seed, uint32_t layer, uint32_t draw_offset, int64_t K, uint64_t token_offset,
                       int64_t T, int64_t n, uint32_t* raw, float* gauss, void* stream) {
    if (!raw && !gauss) return fail(DUST_E_INVALID, "dust_noise: raw and gauss are both NULL");
    if (T <= 0 || K <= 0 || n <= 0) return fail(DUST_E_INVALID, "dust_noise: K, T, n must be >= 1");
    if ((uint64_t)token_offset + (uint64_t)T > (1ull << 32) || (uint64_t)draw_offset + (uint64_t)K > (1ull << 32))
        return fail(DUST_E_INVALID, "dust_noise: offset + count exceeds the 32-bit counter");
    const int64_t threads = K * T * ((n + 3) / 4);
    if (K > (int64_t)INT32_MAX || T > (int64_t)INT32_MAX || threads > ((int64_t)1 << 32) - 256)
        return fail(DUST_E_UNSUPPORTED, "dust_noise: K*T*ceil(n/4) must stay below 2^32");
    hipError_t e = dust::launch_noise_export(seed, layer, draw_offset, K, (uint32_t)token_offset, T, n, raw, gauss,
                                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("dust_noise launch", e);
    return ok();
}

dust_status dust_debug_noise(uint64_t seed, uint32_t layer, uint32_t draw, uint64_t token, int64_t n,
                             uint32_t* raw, float* gauss, void* stream) {
    if (!raw && !gauss) return fail(DUST_E_INVALID, "dust_debug_noise: raw and gauss are both NULL");
    if (n <= 0) return fail(DUST_E_INVALID, "dust_debug_noise: n must be >= 1");
    if (token >= (1ull << 32)) return fail(DUST_E_INVALID, "dust_debug_noise: token must be below 2^32");
    if (n > ((int64_t)1 << 32) - 1024) return fail(DUST_E_UNSUPPORTED, "dust_debug_noise: n too large");
    hipError_t e = dust::launch_noise_export(seed, layer, draw, 1, (uint32_t)token, 1, n, raw, gauss,
                                             static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("dust_debug_noise launch", e);
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
                                uint32_t layer, uint64_t token_offset, uint32_t draw_offset) {
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
    A.tok0 = (uint32_t)token_offset;
    A.draw0 = draw_offset;
    return A;
}

size_t dust_head_workspace_bytes(int64_t T, int64_t V, int64_t d, int64_t K) {
    (void)K;
    if (T <= 0 || V <= 0 || d <= 0) return 0;
    return (head_pairs_path(T, V, d) ? 0 : head_ghat_bytes(T, V)) + dust::outer_workspace_bytes(T, V, d);
}

// The host checks of dust_estimate_head (and of its no-allocation variant), in order;
// `fn` names the entry point in the messages.  Touches no device.
static dust_status head_checks(const char* fn, const void* logits, int logits_dtype, const float* x,
                               const int32_t* labels, int64_t T, int64_t V, int64_t d, int64_t K, float sigma,
                               uint64_t token_offset, uint32_t draw_offset, const float* grad_w, const float* ghat,
                               const float* rewards, const void* workspace, dust::HeadPlan* plan) {
    if (!logits || !x || !labels || !grad_w)
        return fail(DUST_E_INVALID, "%s: logits, x, labels and grad_w must be non-NULL", fn);
    if (logits_dtype != DUST_F32 && logits_dtype != DUST_BF16)
        return fail(DUST_E_UNSUPPORTED, "%s: logits_dtype %d is not DUST_F32 or DUST_BF16", fn, logits_dtype);
    if (!aligned16(logits) || !aligned16(x) || !aligned16(labels) || !aligned16(grad_w) ||
        (ghat && !aligned16(ghat)) || (rewards && !aligned16(rewards)) || (workspace && !aligned16(workspace)))
        return fail(DUST_E_INVALID, "%s: every pointer must be 16-byte aligned", fn);
    dust_status s = check_common(T, K, sigma, token_offset, draw_offset);
    if (s != DUST_OK) return s;
    if (V <= 0) return fail(DUST_E_INVALID, "%s: V must be >= 1", fn);
    if (d <= 0) return fail(DUST_E_INVALID, "%s: d must be >= 1", fn);
    if (V > 65535LL * 128 || d > 65535LL * 128) return fail(DUST_E_UNSUPPORTED, "%s: V or d too large", fn);
    *plan = dust::plan_head(V, logits_dtype, sigma);
    if (!plan->ok) return fail(DUST_E_UNSUPPORTED, "%s: %s", fn, plan->why);
    return DUST_OK;
}

// Workspace bytes one dust_estimate_head call needs (the g_hat rows only when the
// caller passes no ghat and the outer product does not take the bf16-pair path).
static size_t head_need_bytes(int64_t T, int64_t V, int64_t d, bool have_ghat) {
    const size_t ghat_ws = (have_ghat || head_pairs_path(T, V, d)) ? 0 : head_ghat_bytes(T, V);
    return ghat_ws + dust::outer_workspace_bytes(T, V, d);
}

dust_status dust_estimate_head(const void* logits, int logits_dtype, const float* x, const int32_t* labels,
                               int64_t T, int64_t V, int64_t d, int64_t K, float sigma, uint64_t seed,
                               uint32_t layer, uint64_t token_offset, uint32_t draw_offset, float* grad_w,
                               float* ghat, float* rewards, void* workspace, size_t workspace_bytes,
                               void* stream) {
    dust::HeadPlan plan{};
    dust_status s = head_checks("dust_estimate_head", logits, logits_dtype, x, labels, T, V, d, K, sigma,
                                token_offset, draw_offset, grad_w, ghat, rewards, workspace, &plan);
    if (s != DUST_OK) return s;

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

dust_status dust_estimate_head_noalloc(const void* logits, int logits_dtype, const float* x, const int32_t* labels,
                                       int64_t T, int64_t V, int64_t d, int64_t K, float sigma, uint64_t seed,
                                       uint32_t layer, uint64_t token_offset, uint32_t draw_offset, float* grad_w,
                                       float* ghat, float* rewards, void* stream) {
    const char* fn = "dust_estimate_head_noalloc";
    dust::HeadPlan plan{};
    dust_status s = head_checks(fn, logits, logits_dtype, x, labels, T, V, d, K, sigma, token_offset, draw_offset,
                                grad_w, ghat, rewards, nullptr, &plan);
    if (s != DUST_OK) return s;
    const size_t need = head_need_bytes(T, V, d, ghat != nullptr);
    if (need > DUST_NOALLOC_SCRATCH_BYTES)
        return fail(DUST_E_UNSUPPORTED, "%s: this shape needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use dust_estimate_head with a workspace)", fn, need, DUST_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((s = scratch_for_current_device(fn, &ws)) != DUST_OK) return s;
    // Nothing in the workspace has to start at zero: every byte the kernels read is
    // written earlier in the same call (as for a workspace fresh from an allocator).
    return dust_estimate_head(logits, logits_dtype, x, labels, T, V, d, K, sigma, seed, layer, token_offset,
                              draw_offset, grad_w, ghat, rewards, ws, DUST_NOALLOC_SCRATCH_BYTES, stream);
}

size_t dust_head_noalloc_max_bytes(void) { return DUST_NOALLOC_SCRATCH_BYTES; }

// bytes of K*T floats or ints, padded to 256
static size_t kt_bytes(int64_t T, int64_t K) { return ((size_t)T * (size_t)K * 4 + 255) & ~(size_t)255; }

size_t dust_head_subset_workspace_bytes(int64_t T, int64_t V, int64_t d, int64_t K) {
    // the full estimator's layout (which a covering window runs); rows wider
    // than LDS add the rewards and window offsets of every (draw, token)
    const size_t base = dust_head_workspace_bytes(T, V, d, K);
    if (base == 0 || K <= 0 || V <= dust::kSubsetLdsMaxV) return base;
    return base + 2 * kt_bytes(T, K);
}

dust_status dust_estimate_head_subset(const void* logits, int logits_dtype, const float* x, const int32_t* labels,
                                      int64_t T, int64_t V, int64_t d, int64_t K, int64_t m, float sigma,
                                      uint64_t seed, uint32_t layer, uint64_t token_offset, uint32_t draw_offset,
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
    const bool pairs = head_pairs_path(T, V, d);
    const size_t ghat_ws = (ghat || pairs) ? 0 : head_ghat_bytes(T, V);
    const size_t outer_ws = dust::outer_workspace_bytes(T, V, d);
    const size_t kt_ws = wide ? kt_bytes(T, K) : 0;  // twice: the (reward, window offset) pairs
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
    float2* ro_ws = wide ? reinterpret_cast<float2*>(ws + ghat_ws + outer_ws) : nullptr;   // 2 kt_ws >= 8 K T
    hipError_t e = dust::launch_head_subset(plan, logits_dtype, A, m, ro_ws, st);
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
                                 uint64_t token_offset, uint32_t draw_offset, float* grad_w, float* ghat,
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
    if (V * d >= ((int64_t)1 << 31) || n * d >= ((int64_t)1 << 31))
        return fail(DUST_E_UNSUPPORTED, "dust_estimate_linear: V*d and n*d must stay below 2^31 (W_head and W2 "
                                        "element offsets are 32-bit)");
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
    A.tok0 = (uint32_t)token_offset;
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
                               uint64_t seed, uint32_t layer, uint64_t token_offset, uint32_t draw_offset,
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
    if (H > 16) return fail(DUST_E_UNSUPPORTED, "dust_estimate_attn: at most 16 heads (got %lld)", (long long)H);
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
    hipError_t err = dust::launch_attn_rewards(proj, q, k, v, e, T, S, d, H, K, sigma, seed, layer, (uint32_t)token_offset,
                                               draw_offset, rew, ws, L, st);
    if (err != hipSuccess) return device_fail("dust_estimate_attn: attention passes", err);
    if ((err = record_stage(2, st)) != hipSuccess) return device_fail("dust_estimate_attn: stage event", err);
    err = dust::launch_attn_v_ghat(T, d, K, sigma, seed, layer, (uint32_t)token_offset, draw_offset, rew, g, st);
    if (err != hipSuccess) return device_fail("dust_estimate_attn: reduction launch", err);
    if ((err = record_stage(0, st)) != hipSuccess) return device_fail("dust_estimate_attn: stage event", err);
    err = dust::launch_outer(g, u, T, d, d, grad_w, ws + L.off_outer, L.total - L.off_outer, st, false);
    if (err != hipSuccess) return device_fail("dust_estimate_attn: outer-product launch", err);
    if ((err = record_stage(1, st)) != hipSuccess) return device_fail("dust_estimate_attn: stage event", err);
    return ok();
}

dust_status dust_estimate_attn_v(const float* q, const float* k, const float* e, const float* u, int64_t T,
                                 int64_t S, int64_t d, int64_t H, int64_t K, float sigma, uint64_t seed,
                                 uint32_t layer, uint64_t token_offset, uint32_t draw_offset, float* grad_w,
                                 float* ghat, float* rewards, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return dust_estimate_attn(DUST_ATTN_V, q, k, nullptr, e, u, T, S, d, H, K, sigma, seed, layer, token_offset,
                              draw_offset, grad_w, ghat, rewards, workspace, workspace_bytes, stream);
}

// ---- one full Dust step on a small causal LM -----------------------------------------
namespace {

constexpr uint32_t kLmLidEmb = 1, kLmLidHead = 2, kLmLidEs = 3;
constexpr int kLmMaxL = 32;
constexpr size_t kLmChunkBytes = size_t(1) << 30;  // change tensors of one chunk of draws

// noise layer word of block l's linear: 0 q, 1 k, 2 v, 3 o, 4 up, 5 down
uint32_t lm_lid(int64_t l, int kind) { return 16u * (uint32_t)(l + 1) + (uint32_t)kind; }

struct LmDims {
    int64_t V, d, H, L, n, S, B, T;
    float eps;
};

dust_status lm_check_cfg(const dust_lm_config* c, LmDims& D, const char* who) {
    if (!c) return fail(DUST_E_INVALID, "%s: cfg is NULL", who);
    if (c->H < 1 || c->H > 16 || c->d != 64 * c->H)
        return fail(DUST_E_UNSUPPORTED, "%s: heads of 64 channels, 1 <= H <= 16 and d = 64 H (got d=%d H=%d)", who,
                    c->d, c->H);
    if (c->S < 64 || c->S % 64 != 0 || c->S > 4096)
        return fail(DUST_E_UNSUPPORTED, "%s: S must be a multiple of 64 in [64, 4096] (got %d)", who, c->S);
    if (c->n < 64 || c->n % 64 != 0 || c->n > 65536)
        return fail(DUST_E_UNSUPPORTED, "%s: n must be a multiple of 64 in [64, 65536] (got %d)", who, c->n);
    if (c->V < 1 || c->V > 32768) return fail(DUST_E_UNSUPPORTED, "%s: V must be in [1, 32768] (got %d)", who, c->V);
    if (c->L < 1 || c->L > kLmMaxL) return fail(DUST_E_UNSUPPORTED, "%s: L must be in [1, 32] (got %d)", who, c->L);
    if (c->B < 1 || (int64_t)c->B * c->S > (int64_t(1) << 24))
        return fail(DUST_E_INVALID, "%s: B must be >= 1 with B S <= 2^24 (got B=%d)", who, c->B);
    if (!std::isfinite(c->ln_eps) || !(c->ln_eps > 0.f))
        return fail(DUST_E_INVALID, "%s: ln_eps must be finite and > 0", who);
    D = {c->V, c->d, c->H, c->L, c->n, c->S, c->B, (int64_t)c->B * c->S, c->ln_eps};
    return ok();
}

dust_status lm_check_hp(const dust_lm_hparams* h, const char* who, bool step) {
    if (!h) return fail(DUST_E_INVALID, "%s: hp is NULL", who);
    if (h->K < 1 || h->K > (1 << 24) || h->M < 1 || h->M > (1 << 24))
        return fail(DUST_E_INVALID, "%s: K and M must be in [1, 2^24] (got K=%d M=%d)", who, h->K, h->M);
    if (h->chunk < 0) return fail(DUST_E_INVALID, "%s: chunk must be >= 0 (got %d)", who, h->chunk);
    const float s[9] = {h->sigma_emb, h->sigma_q,    h->sigma_k,    h->sigma_v, h->sigma_o,
                        h->sigma_up,  h->sigma_down, h->sigma_head, h->sigma_es};
    for (float v : s)
        if (!std::isfinite(v) || !(v > 0.f)) return fail(DUST_E_INVALID, "%s: every sigma must be finite and > 0", who);
    if (step && !(std::isfinite(h->lr) && std::isfinite(h->lr_scalar) && std::isfinite(h->momentum)))
        return fail(DUST_E_INVALID, "%s: lr, lr_scalar and momentum must be finite", who);
    return ok();
}

struct LmParams {
    int64_t d, n, emb, pos, layer0, per_layer, head, scal, count;
    int64_t wq(int64_t l) const { return layer0 + l * per_layer; }
    int64_t wo(int64_t l) const { return wq(l) + 3 * d * d; }
    int64_t w1(int64_t l) const { return wq(l) + 4 * d * d; }
    int64_t w2(int64_t l) const { return w1(l) + n * d; }
};

LmParams lm_params(const LmDims& D) {
    LmParams P;
    P.d = D.d;
    P.n = D.n;
    P.emb = 0;
    P.pos = D.V * D.d;
    P.layer0 = P.pos + D.S * D.d;
    P.per_layer = 4 * D.d * D.d + 2 * D.n * D.d;
    P.head = P.layer0 + D.L * P.per_layer;
    P.scal = P.head + D.V * D.d;
    P.count = P.scal + 2 * D.L;
    return P;
}

struct LmLayout {
    int64_t kc;
    bool fused;                  // head change fused with its loss change (d = 64 or 128)
    int64_t vp, nseg, vseg;      // padded vocabulary, its segments for the fused kernel
    size_t HBHI, HBLO, PP, PART;
    size_t X[kLmMaxL + 1], U1[kLmMaxL], Q[kLmMaxL], Kk[kLmMaxL], Vv[kLmMaxL], O[kLmMaxL], BA[kLmMaxL], XM[kLmMaxL],
        U2[kLmMaxL], BM[kLmMaxL], Hh[kLmMaxL], Mm[kLmMaxL], MU1[kLmMaxL], RS1[kLmMaxL], MU2[kLmMaxL], RS2[kLmMaxL],
        LSE[kLmMaxL], PC[kLmMaxL], CDF[kLmMaxL], PDF[kLmMaxL], GO[kLmMaxL], GUP[kLmMaxL], GDN[kLmMaxL], WSH[kLmMaxL], WSL[kLmMaxL];
    size_t UF, MUF, RSF, Z, LSEZ, CE;
    size_t DX, DU, DQ, DK, DV, DO, DB, DH, DM, DZ;
    size_t REWS, REWES, DL, GE, E, WOT, SUB, sub_bytes, total;
};

size_t lm_rewards_count(const LmDims& D, int64_t K, int64_t M) {
    return (size_t)((5 + 3 * D.L) * K * D.T + 2 * M);
}

LmLayout lm_layout(const LmDims& D, int64_t K, int64_t M, int64_t chunk) {
    LmLayout L{};
    size_t off = 0;
    auto take = [&](int64_t floats) {
        const size_t o = off;
        off += round_up((size_t)floats * sizeof(float));
        return o;
    };
    const int64_t T = D.T, d = D.d, n = D.n;
    for (int64_t l = 0; l < D.L; ++l) {
        L.X[l] = take(T * d);
        L.U1[l] = take(T * d);
        L.Q[l] = take(T * d);
        L.Kk[l] = take(T * d);
        L.Vv[l] = take(T * d);
        L.O[l] = take(T * d);
        L.BA[l] = take(T * d);
        L.XM[l] = take(T * d);
        L.U2[l] = take(T * d);
        L.BM[l] = take(T * d);
        L.Hh[l] = take(T * n);
        L.Mm[l] = take(T * n);
        L.CDF[l] = take(T * n);  // Phi(h) and phi(h) of the clean W_1 output
        L.PDF[l] = take(T * n);
        L.MU1[l] = take(T);
        L.RS1[l] = take(T);
        L.MU2[l] = take(T);
        L.RS2[l] = take(T);
        L.LSE[l] = take(T * D.H);
        L.PC[l] = take(T * D.S * D.H);  // clean attention probabilities, [b, h, query, key]
        L.GO[l] = take(T * d);
        L.GUP[l] = take(T * n);
        L.GDN[l] = take(T * d);
        // bf16 parts of the block's weights (W_Q, W_K, W_V, W_O, W_1, W_2 as in the parameters)
        L.WSH[l] = take((4 * d * d + 2 * n * d) / 2);
        L.WSL[l] = take((4 * d * d + 2 * n * d) / 2);
    }
    L.X[D.L] = take(T * d);
    L.UF = take(T * d);
    L.MUF = take(T);
    L.RSF = take(T);
    L.Z = take(T * D.V);
    L.LSEZ = take(T);
    L.CE = take(T);
    L.fused = d == 64 || d == 128;
    L.vp = (D.V + 127) / 128 * 128;
    if (L.fused) {
        L.HBHI = take(L.vp * d / 2);
        L.HBLO = take(L.vp * d / 2);
        L.PP = take(T * L.vp);
    }
    const int64_t per_draw = T * (7 * d + 2 * n + (L.fused ? L.vp / 128 : D.V)) * (int64_t)sizeof(float);
    L.kc = std::max<int64_t>(1, std::min<int64_t>(std::max(K, 2 * M), (int64_t)kLmChunkBytes / per_draw));
    if (chunk > 0) L.kc = std::min(L.kc, chunk);
    const int64_t R = L.kc * T;
    // segments: enough workgroups (64 rows x one segment each) to fill the chip
    const int64_t tiles = L.vp / 128, rb = R / 64;
    L.nseg = std::max<int64_t>(1, std::min<int64_t>(tiles, (2048 + rb - 1) / rb));
    L.vseg = (tiles + L.nseg - 1) / L.nseg * 128;
    L.nseg = (L.vp + L.vseg - 1) / L.vseg;
    L.DX = take(R * d);
    L.DU = take(R * d);
    L.DQ = take(3 * R * d);  // D_q, D_k, D_v: three consecutive [R, d] planes (one product writes them)
    L.DK = L.DQ + (size_t)(R * d) * sizeof(float);
    L.DV = L.DK + (size_t)(R * d) * sizeof(float);
    L.DO = take(R * d);
    L.DB = take(R * d);
    L.DH = take(R * n);
    L.DM = take(R * n);
    if (L.fused)
        L.PART = take(R * L.nseg);
    else
        L.DZ = take(R * D.V);
    L.REWS = take((int64_t)lm_rewards_count(D, K, M));
    L.REWES = take(2 * M * T);
    L.DL = take(2 * M);
    L.GE = take(T * d);
    L.E = take(T * d);
    L.WOT = take(d * d);
    size_t sub = dust_head_workspace_bytes(T, D.V, d, K);
    for (int p = 0; p < 3; ++p) sub = std::max(sub, dust_attn_workspace_bytes(p, T, D.S, d, D.H, K));
    sub = std::max({sub, dust::outer_workspace_bytes(T, d, d), dust::outer_workspace_bytes(T, n, d),
                    dust::outer_workspace_bytes(T, d, n)});
    L.sub_bytes = round_up(sub);
    L.SUB = off;
    off += L.sub_bytes;
    L.total = off;
    return L;
}

struct LmRun {
    LmDims D;
    LmParams P;
    const LmLayout* L;
    unsigned char* ws;
    hipStream_t st;
    const float* prm;
    const int32_t* tok;
    const int32_t* lab;
    float* f(size_t off) const { return reinterpret_cast<float*>(ws + off); }
};

#define LM_TRY(x)                           \
    do {                                    \
        const hipError_t e_ = (x);          \
        if (e_ != hipSuccess) return e_;    \
    } while (0)

hipError_t lm_clean_forward(const LmRun& R) {
    const LmDims& D = R.D;
    const LmLayout& L = *R.L;
    const int T = (int)D.T, d = (int)D.d, n = (int)D.n;
    const hipStream_t st = R.st;
    const float* p = R.prm;
    LM_TRY(dust::lm_embed(p + R.P.emb, p + R.P.pos, R.tok, T, (int)D.S, d, (int)D.V, R.f(L.X[0]), st));
    for (int64_t l = 0; l < D.L; ++l) {
        const int64_t wq = R.P.wq(l);
        LM_TRY(dust::lm_layernorm(R.f(L.X[l]), T, d, D.eps, R.f(L.U1[l]), R.f(L.MU1[l]), R.f(L.RS1[l]), st));
        LM_TRY(dust::lm_gemm_nt(R.f(L.U1[l]), p + wq, R.f(L.Q[l]), T, d, d, nullptr, false, st));
        LM_TRY(dust::lm_gemm_nt(R.f(L.U1[l]), p + wq + D.d * D.d, R.f(L.Kk[l]), T, d, d, nullptr, false, st));
        LM_TRY(dust::lm_gemm_nt(R.f(L.U1[l]), p + wq + 2 * D.d * D.d, R.f(L.Vv[l]), T, d, d, nullptr, false, st));
        LM_TRY(dust::lm_attn_fwd(R.f(L.Q[l]), R.f(L.Kk[l]), R.f(L.Vv[l]), T, (int)D.S, (int)D.H, R.f(L.O[l]),
                                 R.f(L.LSE[l]), R.f(L.PC[l]), st));
        LM_TRY(dust::lm_gemm_nt(R.f(L.O[l]), p + R.P.wo(l), R.f(L.BA[l]), T, d, d, nullptr, false, st));
        LM_TRY(dust::lm_residual(R.f(L.X[l]), R.f(L.BA[l]), p + R.P.scal + 2 * l, D.T * D.d, R.f(L.XM[l]), st));
        LM_TRY(dust::lm_layernorm(R.f(L.XM[l]), T, d, D.eps, R.f(L.U2[l]), R.f(L.MU2[l]), R.f(L.RS2[l]), st));
        LM_TRY(dust::lm_gemm_nt(R.f(L.U2[l]), p + R.P.w1(l), R.f(L.Hh[l]), T, n, d, nullptr, false, st));
        LM_TRY(dust::lm_gelu(R.f(L.Hh[l]), D.T * D.n, R.f(L.Mm[l]), R.f(L.CDF[l]), R.f(L.PDF[l]), st));
        LM_TRY(dust::lm_gemm_nt(R.f(L.Mm[l]), p + R.P.w2(l), R.f(L.BM[l]), T, d, n, nullptr, false, st));
        LM_TRY(dust::lm_residual(R.f(L.XM[l]), R.f(L.BM[l]), p + R.P.scal + 2 * l + 1, D.T * D.d, R.f(L.X[l + 1]),
                                 st));
    }
    for (int64_t l = 0; l < D.L; ++l)  // bf16 parts of the block's weights, for the change GEMMs
        LM_TRY(dust::lm_split(p + R.P.wq(l), 1, 1, (int)R.P.per_layer, reinterpret_cast<uint16_t*>(R.ws + L.WSH[l]),
                              reinterpret_cast<uint16_t*>(R.ws + L.WSL[l]), st));
    LM_TRY(dust::lm_layernorm(R.f(L.X[D.L]), T, d, D.eps, R.f(L.UF), R.f(L.MUF), R.f(L.RSF), st));
    LM_TRY(dust::lm_gemm_nt(R.f(L.UF), p + R.P.head, R.f(L.Z), T, D.V, d, nullptr, false, st));
    if (L.fused)
        LM_TRY(dust::lm_split_frag(p + R.P.head, D.V, L.vp, d, reinterpret_cast<uint16_t*>(R.ws + L.HBHI),
                              reinterpret_cast<uint16_t*>(R.ws + L.HBLO), st));
    return dust::lm_ce(R.f(L.Z), R.lab, T, (int)D.V, R.f(L.LSEZ), R.f(L.CE), L.fused ? R.f(L.PP) : nullptr,
                       (int)L.vp, st);
}

// One chunk of kn draws (or ES members from draw0) of a pass: kind 0 emb, 1 o, 2 up,
// 3 down, 4 residual-scalar ES.  Writes the rewards -D_CE of rows i T + t to rew.
hipError_t lm_delta_chunk(const LmRun& R, int kind, int kn, uint32_t draw0, float sigma, uint32_t k0, uint32_t k1,
                          float* rew) {
    const LmDims& D = R.D;
    const LmLayout& L = *R.L;
    const hipStream_t st = R.st;
    const float* p = R.prm;
    const int T = (int)D.T, d = (int)D.d, n = (int)D.n;
    const int64_t rows = (int64_t)kn * D.T;
    const bool es = kind == 4;
    const float es_sigma = es ? sigma : 0.f;
    float *DX = R.f(L.DX), *DU = R.f(L.DU), *DQ = R.f(L.DQ), *DK = R.f(L.DK), *DV = R.f(L.DV), *DO = R.f(L.DO),
          *DB = R.f(L.DB), *DH = R.f(L.DH), *DM = R.f(L.DM), *DZ = L.fused ? nullptr : R.f(L.DZ);
    auto zero = [&](float* ptr, int64_t count) { return hipMemsetAsync(ptr, 0, (size_t)count * sizeof(float), st); };
    // bf16 parts of block l's weight at parameter offset `off`
    auto wh = [&](int64_t l, int64_t off) {
        return reinterpret_cast<const uint16_t*>(R.ws + L.WSH[l]) + (off - R.P.wq(l));
    };
    auto wl = [&](int64_t l, int64_t off) {
        return reinterpret_cast<const uint16_t*>(R.ws + L.WSL[l]) + (off - R.P.wq(l));
    };
    const int64_t qkv_plane = L.kc * D.T * D.d;  // floats from D_q to D_k and from D_k to D_v
    bool live = false;  // whether DX holds a change yet
    // the residual updates also form the following LayerNorm change in the same pass when
    // the width allows; du_ready then says that DU already holds it
    const bool fuse = dust::lm_residual_ln_fusable(d);
    bool du_ready = false;
    if (kind == 0) {
        LM_TRY(dust::lm_noise_add(DX, kn, T, d, sigma, k0, k1, kLmLidEmb, draw0, st, /*set=*/true));
        live = true;
    }
    for (int64_t l = 0; l < D.L; ++l) {
        const int64_t wq = R.P.wq(l);
        if (live) {
            if (!du_ready)
                LM_TRY(dust::lm_layernorm_delta(R.f(L.X[l]), R.f(L.MU1[l]), R.f(L.RS1[l]), DX, rows, T, d, DU, st));
            du_ready = false;
            // W_Q, W_K, W_V are consecutive rows of one [3d, d] weight and D_q, D_k, D_v
            // consecutive planes of the workspace: one product reads the change rows once
            LM_TRY(dust::lm_gemm_x3(DU, wh(l, wq), wl(l, wq), DQ, rows, 3 * d, d, st, d, qkv_plane));
            LM_TRY(dust::lm_attn_delta(R.f(L.Q[l]), R.f(L.Kk[l]), R.f(L.Vv[l]), R.f(L.O[l]), R.f(L.PC[l]), DQ, DK,
                                       DV, kn, T, (int)D.S, (int)D.H, DO, st));
            LM_TRY(dust::lm_gemm_x3(DO, wh(l, R.P.wo(l)), wl(l, R.P.wo(l)), DB, rows, d, d, st));
        } else if (es) {
            LM_TRY(zero(DB, rows * d));
        }
        // with no change yet the noise is written, not added
        if (kind == 1) LM_TRY(dust::lm_noise_add(DB, kn, T, d, sigma, k0, k1, lm_lid(l, 3), draw0, st, !live));
        if (live || kind == 1 || es) {
            if (!live) LM_TRY(zero(DX, rows * d));
            if (fuse)
                LM_TRY(dust::lm_residual_ln_delta(DX, DB, R.f(L.BA[l]), p + R.P.scal, (int)(2 * l), kn, T, d, es_sigma,
                                                  draw0, k0, k1, kLmLidEs, R.f(L.XM[l]), R.f(L.MU2[l]),
                                                  R.f(L.RS2[l]), DU, st));
            else
                LM_TRY(dust::lm_residual_delta(DX, DB, R.f(L.BA[l]), p + R.P.scal, (int)(2 * l), kn, D.T * D.d,
                                               es_sigma, draw0, k0, k1, kLmLidEs, st));
            live = true;
            du_ready = fuse;
        }
        if (live) {
            if (!du_ready)
                LM_TRY(dust::lm_layernorm_delta(R.f(L.XM[l]), R.f(L.MU2[l]), R.f(L.RS2[l]), DX, rows, T, d, DU, st));
            du_ready = false;
            LM_TRY(dust::lm_gemm_x3(DU, wh(l, R.P.w1(l)), wl(l, R.P.w1(l)), DH, rows, n, d, st));
        }
        if (kind == 2) LM_TRY(dust::lm_noise_add(DH, kn, T, n, sigma, k0, k1, lm_lid(l, 4), draw0, st, !live));
        const bool mlp = live || kind == 2;
        if (mlp) {
            LM_TRY(dust::lm_gelu_delta(R.f(L.Hh[l]), R.f(L.CDF[l]), R.f(L.PDF[l]), DH, D.T * D.n, rows * n, DM, st));
            LM_TRY(dust::lm_gemm_x3(DM, wh(l, R.P.w2(l)), wl(l, R.P.w2(l)), DB, rows, d, n, st));
        }
        if (kind == 3) LM_TRY(dust::lm_noise_add(DB, kn, T, d, sigma, k0, k1, lm_lid(l, 5), draw0, st, !mlp));
        if (mlp || kind == 3 || es) {
            if (!live) LM_TRY(zero(DX, rows * d));
            // the next LayerNorm: the next block's first, or the final one
            const bool last = l + 1 == D.L;
            const float* nx = R.f(L.X[l + 1]);
            const float* nmu = R.f(last ? L.MUF : L.MU1[l + 1]);
            const float* nrs = R.f(last ? L.RSF : L.RS1[l + 1]);
            if (fuse)
                LM_TRY(dust::lm_residual_ln_delta(DX, DB, R.f(L.BM[l]), p + R.P.scal, (int)(2 * l + 1), kn, T, d,
                                                  es_sigma, draw0, k0, k1, kLmLidEs, nx, nmu, nrs, DU, st));
            else
                LM_TRY(dust::lm_residual_delta(DX, DB, R.f(L.BM[l]), p + R.P.scal, (int)(2 * l + 1), kn, D.T * D.d,
                                               es_sigma, draw0, k0, k1, kLmLidEs, st));
            live = true;
            du_ready = fuse;
        }
    }
    if (!du_ready) LM_TRY(dust::lm_layernorm_delta(R.f(L.X[D.L]), R.f(L.MUF), R.f(L.RSF), DX, rows, T, d, DU, st));
    if (L.fused) {
        LM_TRY(dust::lm_head_delta(DU, reinterpret_cast<const uint16_t*>(R.ws + L.HBHI),
                                   reinterpret_cast<const uint16_t*>(R.ws + L.HBLO), R.f(L.PP), d, kn, T, (int)L.vp,
                                   (int)L.vseg, (int)L.nseg, R.f(L.PART), st));
        return dust::lm_head_reward(DU, p + R.P.head, R.lab, R.f(L.PART), T, (int)D.V, d, (int)L.nseg, rows, rew, st);
    }
    LM_TRY(dust::lm_gemm_nt(DU, p + R.P.head, DZ, rows, D.V, d, nullptr, false, st));
    return dust::lm_ce_delta(R.f(L.Z), R.f(L.LSEZ), DZ, R.lab, kn, T, (int)D.V, rew, st);
}

dust_status lm_prepare(const dust_lm_config* cfg, const dust_lm_hparams* hp, const float* params,
                       const int32_t* tokens, const int32_t* labels, void* workspace, size_t workspace_bytes,
                       void* stream, const char* who, bool step, LmRun& R, LmLayout& L) {
    dust_status s = lm_check_cfg(cfg, R.D, who);
    if (s != DUST_OK) return s;
    if (hp && (s = lm_check_hp(hp, who, step)) != DUST_OK) return s;
    if (!params || !tokens || !labels) return fail(DUST_E_INVALID, "%s: params, tokens and labels must be non-NULL", who);
    if (!aligned16(params)) return fail(DUST_E_INVALID, "%s: params must be 16-byte aligned", who);
    L = lm_layout(R.D, hp ? hp->K : 1, hp ? hp->M : 1, hp ? hp->chunk : 0);
    if (!workspace || workspace_bytes < L.total)
        return fail(DUST_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, L.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(DUST_E_INVALID, "%s: workspace must be 16-byte aligned", who);
    R.P = lm_params(R.D);
    R.L = &L;
    R.ws = static_cast<unsigned char*>(workspace);
    R.st = static_cast<hipStream_t>(stream);
    R.prm = params;
    R.tok = tokens;
    R.lab = labels;
    return ok();
}

}  // namespace

size_t dust_lm_param_count(const dust_lm_config* cfg) {
    LmDims D;
    if (lm_check_cfg(cfg, D, "dust_lm_param_count") != DUST_OK) return 0;
    return (size_t)lm_params(D).count;
}

size_t dust_lm_rewards_count(const dust_lm_config* cfg, const dust_lm_hparams* hp) {
    LmDims D;
    if (lm_check_cfg(cfg, D, "dust_lm_rewards_count") != DUST_OK) return 0;
    if (lm_check_hp(hp, "dust_lm_rewards_count", false) != DUST_OK) return 0;
    return lm_rewards_count(D, hp->K, hp->M);
}

size_t dust_lm_workspace_bytes(const dust_lm_config* cfg, const dust_lm_hparams* hp) {
    LmDims D;
    if (lm_check_cfg(cfg, D, "dust_lm_workspace_bytes") != DUST_OK) return 0;
    if (hp && lm_check_hp(hp, "dust_lm_workspace_bytes", false) != DUST_OK) return 0;
    return lm_layout(D, hp ? hp->K : 1, hp ? hp->M : 1, hp ? hp->chunk : 0).total;
}

dust_status dust_lm_forward(const dust_lm_config* cfg, const float* params, const int32_t* tokens,
                            const int32_t* labels, float* ce, void* workspace, size_t workspace_bytes, void* stream) {
    LmRun R;
    LmLayout L;
    dust_status s = lm_prepare(cfg, nullptr, params, tokens, labels, workspace, workspace_bytes, stream,
                               "dust_lm_forward", false, R, L);
    if (s != DUST_OK) return s;
    if (!ce) return fail(DUST_E_INVALID, "dust_lm_forward: ce must be non-NULL");
    hipError_t e = lm_clean_forward(R);
    if (e != hipSuccess) return device_fail("dust_lm_forward: forward", e);
    e = hipMemcpyAsync(ce, R.f(L.CE), (size_t)R.D.T * sizeof(float), hipMemcpyDeviceToDevice, R.st);
    if (e != hipSuccess) return device_fail("dust_lm_forward: copy", e);
    return ok();
}

dust_status dust_lm_estimate(const dust_lm_config* cfg, const dust_lm_hparams* hp, const float* params,
                             const int32_t* tokens, const int32_t* labels, uint64_t seed, float* grads,
                             float* rewards, void* workspace, size_t workspace_bytes, void* stream) {
    const char* who = "dust_lm_estimate";
    if (!hp) return fail(DUST_E_INVALID, "%s: hp is NULL", who);
    LmRun R;
    LmLayout L;
    dust_status s = lm_prepare(cfg, hp, params, tokens, labels, workspace, workspace_bytes, stream, who, false, R, L);
    if (s != DUST_OK) return s;
    if (!grads || !aligned16(grads)) return fail(DUST_E_INVALID, "%s: grads must be non-NULL and 16-byte aligned", who);
    if (rewards && !aligned16(rewards)) return fail(DUST_E_INVALID, "%s: rewards must be 16-byte aligned", who);
    if (env_flag("DUST_DEBUG_CHECKS")) {
        if ((s = check_labels(tokens, R.D.T, R.D.V, R.st)) != DUST_OK) return s;
        if ((s = check_labels(labels, R.D.T, R.D.V, R.st)) != DUST_OK) return s;
    }
    const LmDims& D = R.D;
    const LmParams& P = R.P;
    const hipStream_t st = R.st;
    const int64_t K = hp->K, M = hp->M, T = D.T, KT = K * T;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    unsigned char* sub = R.ws + L.SUB;
    float* rw = rewards ? rewards : R.f(L.REWS);
    hipError_t e = lm_clean_forward(R);
    if (e == hipSuccess) e = record_stage(4, st);
    if (e != hipSuccess) return device_fail("dust_lm_estimate: clean forward", e);
    // head on the cached logits
    s = dust_estimate_head(R.f(L.Z), DUST_F32, R.f(L.UF), labels, T, D.V, D.d, K, hp->sigma_head, seed, kLmLidHead,
                           0, 0, grads + P.head, nullptr, rw, sub, L.sub_bytes, stream);
    if (s != DUST_OK) return s;
    if ((e = record_stage(5, st)) != hipSuccess) return device_fail("dust_lm_estimate: stage event", e);
    // one pass per linear type, the network recomputed as changes
    const float sig[4] = {hp->sigma_emb, hp->sigma_o, hp->sigma_up, hp->sigma_down};
    for (int kind = 0; kind < 4; ++kind) {
        float* r = rw + (1 + kind) * KT;
        for (int64_t i0 = 0; i0 < K; i0 += L.kc) {
            const int kn = (int)std::min<int64_t>(L.kc, K - i0);
            if ((e = lm_delta_chunk(R, kind, kn, (uint32_t)i0, sig[kind], k0, k1, r + i0 * T)) != hipSuccess)
                return device_fail("dust_lm_estimate: perturbed pass", e);
        }
        const float scale = -1.0f / ((float)K * sig[kind]);
        for (int64_t l = 0; l < (kind == 0 ? 1 : D.L); ++l) {
            if (kind == 0) {
                e = dust::lm_ghat(r, (int)K, (int)T, (int)D.d, scale, k0, k1, kLmLidEmb, R.f(L.GE), st);
                if (e == hipSuccess)
                    e = dust::lm_embed_grads(R.f(L.GE), tokens, (int)T, (int)D.S, (int)D.V, (int)D.d, grads + P.emb,
                                             grads + P.pos, st);
            } else if (kind == 1) {
                e = dust::lm_ghat(r, (int)K, (int)T, (int)D.d, scale, k0, k1, lm_lid(l, 3), R.f(L.GO[l]), st);
                if (e == hipSuccess)
                    e = dust::launch_outer(R.f(L.GO[l]), R.f(L.O[l]), T, D.d, D.d, grads + P.wo(l), sub, L.sub_bytes,
                                           st, false);
            } else if (kind == 2) {
                e = dust::lm_ghat(r, (int)K, (int)T, (int)D.n, scale, k0, k1, lm_lid(l, 4), R.f(L.GUP[l]), st);
                if (e == hipSuccess)
                    e = dust::launch_outer(R.f(L.GUP[l]), R.f(L.U2[l]), T, D.n, D.d, grads + P.w1(l), sub,
                                           L.sub_bytes, st, false);
            } else {
                e = dust::lm_ghat(r, (int)K, (int)T, (int)D.d, scale, k0, k1, lm_lid(l, 5), R.f(L.GDN[l]), st);
                if (e == hipSuccess)
                    e = dust::launch_outer(R.f(L.GDN[l]), R.f(L.Mm[l]), T, D.d, D.n, grads + P.w2(l), sub,
                                           L.sub_bytes, st, false);
            }
            if (e != hipSuccess) return device_fail("dust_lm_estimate: g_hat / outer product", e);
        }
    }
    if ((e = record_stage(6, st)) != hipSuccess) return device_fail("dust_lm_estimate: stage event", e);
    // attention internals, with the error at the attention output e = g_hat_O W_O
    const float sqkv[3] = {hp->sigma_q, hp->sigma_k, hp->sigma_v};
    for (int64_t l = 0; l < D.L; ++l) {
        e = dust::lm_transpose(params + P.wo(l), (int)D.d, (int)D.d, R.f(L.WOT), st);
        if (e == hipSuccess) e = dust::lm_gemm_nt(R.f(L.GO[l]), R.f(L.WOT), R.f(L.E), T, D.d, D.d, nullptr, false, st);
        if (e != hipSuccess) return device_fail("dust_lm_estimate: attention-output error", e);
        for (int proj = 0; proj < 3; ++proj) {
            s = dust_estimate_attn(proj, R.f(L.Q[l]), R.f(L.Kk[l]), R.f(L.Vv[l]), R.f(L.E), R.f(L.U1[l]), T, D.S, D.d,
                                   D.H, K, sqkv[proj], seed, lm_lid(l, proj), 0, 0, grads + P.wq(l) + proj * D.d * D.d,
                                   nullptr, rw + (5 + 3 * l + proj) * KT, sub, L.sub_bytes, stream);
            if (s != DUST_OK) return s;
        }
    }
    if ((e = record_stage(7, st)) != hipSuccess) return device_fail("dust_lm_estimate: stage event", e);
    // residual scalars: antithetic weight-space ES
    float* res = R.f(L.REWES);
    for (int64_t m0 = 0; m0 < 2 * M; m0 += L.kc) {
        const int kn = (int)std::min<int64_t>(L.kc, 2 * M - m0);
        if ((e = lm_delta_chunk(R, 4, kn, (uint32_t)m0, hp->sigma_es, k0, k1, res + m0 * T)) != hipSuccess)
            return device_fail("dust_lm_estimate: ES pass", e);
    }
    float* dL = rewards ? rewards + (5 + 3 * D.L) * KT : R.f(L.DL);
    e = dust::lm_member_losses(res, (int)(2 * M), (int)T, dL, st);
    if (e == hipSuccess)
        e = dust::lm_es_grad(dL, (int)M, (int)(2 * D.L), 1.0f / (2.0f * (float)M * hp->sigma_es), k0, k1, kLmLidEs,
                             grads + P.scal, st);
    if (e != hipSuccess) return device_fail("dust_lm_estimate: ES gradient", e);
    return ok();
}

dust_status dust_lm_sgd(const dust_lm_config* cfg, const dust_lm_hparams* hp, float* params, float* momentum,
                        const float* grads, void* stream) {
    LmDims D;
    dust_status s = lm_check_cfg(cfg, D, "dust_lm_sgd");
    if (s != DUST_OK) return s;
    if ((s = lm_check_hp(hp, "dust_lm_sgd", true)) != DUST_OK) return s;
    if (!params || !momentum || !grads) return fail(DUST_E_INVALID, "dust_lm_sgd: params, momentum and grads must be non-NULL");
    const LmParams P = lm_params(D);
    const hipError_t e = dust::lm_sgd(params, momentum, grads, P.count, P.scal, hp->lr, hp->lr_scalar, hp->momentum,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("dust_lm_sgd", e);
    return ok();
}

dust_status dust_lm_step(const dust_lm_config* cfg, const dust_lm_hparams* hp, float* params, float* momentum,
                         const int32_t* tokens, const int32_t* labels, uint64_t seed, float* grads, float* rewards,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (!hp) return fail(DUST_E_INVALID, "dust_lm_step: hp is NULL");
    dust_status s = lm_check_hp(hp, "dust_lm_step", true);
    if (s != DUST_OK) return s;
    if (!momentum) return fail(DUST_E_INVALID, "dust_lm_step: momentum must be non-NULL");
    s = dust_lm_estimate(cfg, hp, params, tokens, labels, seed, grads, rewards, workspace, workspace_bytes, stream);
    if (s != DUST_OK) return s;
    return dust_lm_sgd(cfg, hp, params, momentum, grads, stream);
}
