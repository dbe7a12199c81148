// Raw bits of one activation (a 16-bit load for bf16) and their value.  Kernels that load a
// batch of activations keep the raw bits until the value is used: a conversion right after a
// load makes the compiler wait for that load there, and loads complete in order, so the batch
// would be serialised.
#pragma once

#include "hci_internal.h"

namespace hci {

template <int ACT> struct ActRaw;
template <> struct ActRaw<HCI_F32> {
    typedef float R;
    __device__ static __forceinline__ R load(const float* p, size_t i) { return p[i]; }
    __device__ static __forceinline__ float cvt(R r) { return r; }
};
template <> struct ActRaw<HCI_BF16> {
    typedef uint32_t R;
    __device__ static __forceinline__ R load(const uint16_t* p, size_t i) { return p[i]; }
    __device__ static __forceinline__ float cvt(R r) { return __uint_as_float(r << 16); }
};

}  // namespace hci
