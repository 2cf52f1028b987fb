// Kernel launch with optional timestamps for the library's profiling scopes.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace spec {

// Timing of the launches inside one profiling scope: the scope's first launch
// records `start` as that kernel begins (then `start` is cleared), every launch
// records `stop` as its kernel ends, so `stop` holds the end of the scope's
// last kernel.  The timestamps travel in the dispatch packets themselves
// (hipExtLaunchKernel), so timing adds no work to the stream.  Set by the
// profiling scope of the enqueuing thread, null otherwise.
struct LaunchTiming {
  hipEvent_t start;
  hipEvent_t stop;
};
extern thread_local LaunchTiming* launch_timing;

}  // namespace spec

// hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...), timed when
// a profiling scope is active on this thread.
#define SPEC_LAUNCH(kernel, grid, block, shmem, stream, ...)                                  \
  do {                                                                                        \
    ::spec::LaunchTiming* spec_t_ = ::spec::launch_timing;                                    \
    if (spec_t_) {                                                                            \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, spec_t_->start, spec_t_->stop, \
                            0u, __VA_ARGS__);                                                 \
      spec_t_->start = nullptr;                                                               \
    } else {                                                                                  \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                    \
    }                                                                                         \
  } while (0)
