// Kernel launch with optional timing events carried by the dispatch itself.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kernels.hpp"

// Launch `kernel` on `stream`.  Events in `ev` (a pa::KernelEvents; either
// may be null) take the kernel's own start and end times from its dispatch
// (hipExtLaunchKernel), so timing puts nothing on the stream between this
// kernel and its neighbours; untimed launches take the plain (cheaper on the
// host) path.  A macro so that the plain path names the kernel itself.
#define PA_LAUNCH(ev, kernel, grid, block, shmem, stream, ...)                                   \
  do {                                                                                           \
    if ((ev).start || (ev).stop)                                                                 \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (ev).start, (ev).stop, 0u,        \
                            __VA_ARGS__);                                                        \
    else                                                                                         \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                        \
  } while (0)
