// launch.hpp -- how every kernel of the library is enqueued.
//
// hipLaunchKernel with the kernel's own parameter list, so that a caller
// gets the status of this launch alone.  Reading the runtime's last-error
// slot after a launch instead would also report an error left there by an
// earlier, unrelated HIP call of the same thread.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>

namespace trt {

// Enqueue k<<<grid, block, lds, s>>>(args...) and return the runtime's
// status for that launch.  Each argument is converted to the parameter type
// it is passed as, and the kernel receives copies of them.
template <class... P, class... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         const A&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "one value per kernel parameter");
  std::tuple<P...> vals(args...);
  void* ptrs[sizeof...(P) == 0 ? 1 : sizeof...(P)] = {};
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, lds, s);
}

}  // namespace trt
