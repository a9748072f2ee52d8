// Global-address-space pointers for device code.
#pragma once

#include <hip/hip_runtime.h>

namespace matopt {

// Pointers into device memory, as the global address space. Accesses through
// a generic pointer compile to flat instructions, which the hardware counts
// against both the vector-memory and the LDS counters, so every wait for an
// LDS read would also wait for the outstanding global loads; accesses
// through these compile to global instructions, counted against vmcnt only.
template <class T> using gmem = __attribute__((address_space(1))) T*;
template <class T> __device__ __forceinline__ gmem<T> gptr(T* p) { return (gmem<T>)p; }

}  // namespace matopt
