// Variant planning for the LM-head estimator.
#include <cmath>

#include "dust_internal.hpp"

namespace dust {

hipError_t launch_head_f32(const HeadPlan& plan, const HeadArgs& args, hipStream_t stream);
hipError_t launch_head_bf16(const HeadPlan& plan, const HeadArgs& args, hipStream_t stream);

// Largest |a| the noise can take: sqrt(-2 ln 2^-24) = sqrt(48 ln 2).
static constexpr double kMaxAbsNoise = 5.7683;
// Dynamic LDS available to one workgroup on gfx950, minus the static arrays.
static constexpr size_t kMaxDynLds = 160 * 1024 - 1024;

HeadPlan plan_head(int64_t V, int logits_dtype, float sigma) {
    HeadPlan p{};
    p.ok = true;
    p.why = "";
    const int64_t nq = (V + 3) / 4;
    if (V <= 8192) {
        p.nt = 256;
        p.q = V <= 1024 ? 1 : V <= 2048 ? 2 : V <= 4096 ? 4 : 8;
        p.pmode = 0;
        p.lds = 0;
    } else if (V <= 65536) {
        // The noise of one draw and the running sum of r*a take 2*4*Q registers per
        // lane: 1024 lanes keep that within the 128 VGPRs of 4 waves/SIMD up to
        // Q = 8.  Up to Q = 13 (V <= 53248, bf16 rows) the running sums of 3
        // quads per lane move to LDS after the row; beyond, Q = 16 spills.
        p.ql = 0;
        if (V <= 16384) { p.nt = 1024; p.q = 4; }
        else if (V <= 32768) { p.nt = 1024; p.q = 8; }
        else if (V <= 1024 * 4 * 13 && logits_dtype == 1) { p.nt = 1024; p.q = 13; p.ql = 3; }
        else { p.nt = 1024; p.q = 16; }
        p.pmode = 1;
        if ((size_t)p.nt * p.q * (logits_dtype == 0 ? 16 : 8) + (size_t)p.ql * p.nt * 16 > kMaxDynLds) {
            p.ok = false;
            p.why = "fp32 logits with V > 32768 do not fit one workgroup's LDS; pass bf16 logits";
        }
    } else {
        p.ok = false;
        p.why = "vocabulary larger than 65536 is not supported";
    }
    // Taylor degree of expm1(x), x = sigma a, |x| <= sigma*5.7683: the dropped
    // terms move S = sum_v p_v expm1(x_v) by at most |x|^(D+1)/(D+1)! e^|x|, which
    // moves a reward (of size ~sigma) by at most as much.  The lowest degree whose
    // bound stays below 2e-5 sigma is taken (the typical change is many orders of
    // magnitude smaller: |a| reaches 5.77 with probability ~1e-7).
    const double xm = (double)sigma * kMaxAbsNoise;
    auto rem = [&](int D) {
        double f = 1.0;
        for (int k = 2; k <= D + 1; ++k) f *= k;
        return std::pow(xm, D + 1) / f * std::exp(xm);
    };
    const double tol = 2e-5 * (double)sigma;
    p.deg = rem(3) <= tol ? 3 : rem(4) <= tol ? 4 : rem(6) <= tol ? 6 : 0;
    if (p.pmode == 1) p.lds = (size_t)p.nt * p.q * (logits_dtype == 0 ? 16 : 8) + (size_t)p.ql * p.nt * 16;
    return p;
}

hipError_t launch_head(const HeadPlan& plan, int logits_dtype, const HeadArgs& args, hipStream_t stream) {
    return logits_dtype == 0 ? launch_head_f32(plan, args, stream) : launch_head_bf16(plan, args, stream);
}

}  // namespace dust
