// csa_walk.h -- the strided element walk the kernels use to zero byte ranges
// of the gradient buffers.  Kept free of HIP headers so the same code can be
// compiled for the host by the CPU tests (tests/test_zero_walk_cpu.py), which
// check it at the edges of the 32-bit offset envelope.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define CSA_HOST_DEVICE __host__ __device__
#else
#define CSA_HOST_DEVICE
#endif

namespace csa {

// Visit the elements of E bytes that tile [begin, end): a thread starts at
// element `first` and advances by `step` elements, calling visit(byte offset)
// for each.  The loop runs over the element index, which stays below the
// element count (< 2^31 for E >= 2 and 32-bit offsets), so `index + step`
// cannot wrap for step < 2^31 and no offset outside [begin, end) is visited.
// (Stepping a byte offset by step * E instead wraps past 2^32 when the range
// ends near the top of the 32-bit offset space.)
template <uint32_t E, typename Visit>
CSA_HOST_DEVICE inline void walk_elements(uint32_t begin, uint32_t end, uint32_t first, uint32_t step,
                                          Visit&& visit) {
  if (end <= begin) return;
  const uint32_t count = (end - begin) / E;
  for (uint32_t i = first; i < count; i += step) visit(begin + i * E);
}

}  // namespace csa
