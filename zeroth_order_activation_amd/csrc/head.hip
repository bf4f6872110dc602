// Variant planning for the LM-head estimator.
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
        // Q = 8; beyond, 768 lanes (3 waves/SIMD, 170 VGPRs) take Q = 17.
        if (V <= 16384) { p.nt = 1024; p.q = 4; }
        else if (V <= 32768) { p.nt = 1024; p.q = 8; }
        else if (V <= 768 * 4 * 17) { p.nt = 768; p.q = 17; }
        else { p.nt = 1024; p.q = 16; }
        p.pmode = 1;
        p.lds = (size_t)nq * (logits_dtype == 0 ? 16 : 8);
        if (p.lds > kMaxDynLds) {
            p.ok = false;
            p.why = "fp32 logits with V > 40896 do not fit one workgroup's LDS; pass bf16 logits";
        }
    } else {
        p.ok = false;
        p.why = "vocabulary larger than 65536 is not supported";
    }
    // expm1(x) = x(1 + x/2 + x^2/6 + x^3/24 + x^4/120) + O(x^6): the dropped part is
    // below 2^-25 of x for |x| <= 0.117.
    p.deg = ((double)sigma * kMaxAbsNoise <= 0.117) ? 5 : 0;
    return p;
}

hipError_t launch_head(const HeadPlan& plan, int logits_dtype, const HeadArgs& args, hipStream_t stream) {
    return logits_dtype == 0 ? launch_head_f32(plan, args, stream) : launch_head_bf16(plan, args, stream);
}

}  // namespace dust
