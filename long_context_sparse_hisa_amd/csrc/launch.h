// Launch helpers shared by the libhisa kernel sources.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace hisa {

template <class T>
struct exact {
    using type = T;
};

// Launch `kernel` with arguments converted to its exact parameter types,
// recording the optional start / stop events from the dispatch itself.
template <typename... P>
inline hipError_t launch_k(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1, typename exact<P>::type... args)
{
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev0, ev1, 0, args...);
    return hipGetLastError();
}

// The same with `lds` bytes of dynamic shared memory.
template <typename... P>
inline hipError_t launch_kl(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                            hipEvent_t ev0, hipEvent_t ev1, typename exact<P>::type... args)
{
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev0, ev1, 0, args...);
    return hipGetLastError();
}

}  // namespace hisa
