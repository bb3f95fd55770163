// LDS poisoning for test builds. Compiled with -DTTT_LDS_POISON, every kernel fills its LDS
// with all-ones words at entry, before anything else touches it: all ones is a NaN as fp32
// and as bf16, so any read of LDS that the kernel did not write first (a missing barrier, a
// wrong index, padding fed to a product) turns the outputs non-finite. In the product build
// the macros expand to nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ttt {

#ifdef TTT_LDS_POISON
__device__ __forceinline__ void lds_poison_bytes(void* p, size_t bytes) {
  unsigned* w = static_cast<unsigned*>(p);
  for (size_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xffffffffu;
}
template <class T>
__device__ __forceinline__ void lds_poison(T& obj) {
  static_assert(sizeof(T) % 4 == 0, "LDS objects are poisoned in whole words");
  lds_poison_bytes(&obj, sizeof(T));
}
#define TTT_POISON(obj) ::ttt::lds_poison(obj)
#define TTT_POISON_BYTES(ptr, bytes) ::ttt::lds_poison_bytes((ptr), (bytes))
#define TTT_POISON_DONE() __syncthreads()
#else
#define TTT_POISON(obj)
#define TTT_POISON_BYTES(ptr, bytes)
#define TTT_POISON_DONE()
#endif

}  // namespace ttt
