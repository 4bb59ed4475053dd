// Kernel launch with optional timing events.  When ev0/ev1 are given the
// launch goes through hipExtLaunchKernelGGL, which stamps the two events with
// the start and end of the kernel's own dispatch: no marker packets are added
// to the stream and the kernel's own duration is unchanged, but each stamped
// dispatch still leaves a gap of about 5 us before the next one starts, so a
// caller that wants the stream's throughput too times a sample of launches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace psw {

template <typename Kernel, typename Args>
inline void launch_timed(Kernel kernel, dim3 grid, dim3 block, void* stream, void* ev0,
                         void* ev1, const Args& args) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ev0 != nullptr && ev1 != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, static_cast<hipEvent_t>(ev0),
                          static_cast<hipEvent_t>(ev1), 0, args);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args);
}

}  // namespace psw
