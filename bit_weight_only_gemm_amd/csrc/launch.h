// launch.h -- kernel launch helper shared by the GEMM launchers: a launch that
// carries the timing events set by w4a16_set_timing_events (consumed once).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace w4a16 {

extern thread_local hipEvent_t t_ev_start, t_ev_stop;

template <typename K, typename... Args>
static void launch_timed(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         Args... args) {
  if (t_ev_start || t_ev_stop) {
    hipEvent_t a = t_ev_start, b = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, a, b, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  }
}

}  // namespace w4a16
