// Profiling hook: HIP events recorded around each launch of a chosen kernel, so
// that a caller can time every launch of it inside a larger call.
#pragma once

#include <hip/hip_runtime.h>

namespace dust {

// kernels that can be timed launch by launch
enum TimedKernel {
    kTimedLmGemm = 0,
    kTimedLmHead = 1,
    kTimedAttnMain = 2,
    kTimedMlpGemm1 = 3,
    kTimedMlpGemm2 = 4,
    kTimedHead = 5,
    kTimedOuter = 6,
    kTimedKernels = 7
};

struct LaunchEvents {
    hipEvent_t* starts = nullptr;
    hipEvent_t* ends = nullptr;
    int capacity = 0;
    int count = 0;
};
extern thread_local LaunchEvents g_kernel_events[kTimedKernels];

// Records the start event of the next launch of `kernel` if the hook is set and has room.
inline hipError_t launch_timer_begin(int kernel, hipStream_t s, bool& timed) {
    LaunchEvents& le = g_kernel_events[kernel];
    timed = le.starts && le.count < le.capacity;
    return timed ? hipEventRecord(le.starts[le.count], s) : hipSuccess;
}

inline hipError_t launch_timer_end(int kernel, hipStream_t s, bool timed) {
    if (!timed) return hipSuccess;
    LaunchEvents& le = g_kernel_events[kernel];
    const hipError_t e = hipEventRecord(le.ends[le.count], s);
    ++le.count;
    return e;
}

}  // namespace dust
