// Checks of the debug build (compiled with -DIDX_DEBUG; compiled away otherwise).
//
// The kernels trust what lives on the device (sequence lengths, row bounds,
// block-table entries, slots, rotary positions, sequence ids of rows): each such value
// is clamped or dropped so that no access leaves its buffer, and the rows it touches
// get unspecified results. In the debug build the kernels also OR one IDX_DBG_* bit
// per offending value into a word of device memory that belongs to the translation
// unit; the host reads the words back through idx_debug_flags. Nothing traps: a bad
// value is reported, never turned into a fault, and every result is the one the
// release build gives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/idx.h"

namespace idx {

#ifdef IDX_DEBUG
static __device__ uint32_t g_debug_word;

__device__ __forceinline__ void debug_note(bool bad, uint32_t bit) {
  if (bad) atomicOr(&g_debug_word, bit);
}

// The release build does not even evaluate the condition (an empty inline function
// still shifts the compiler's inlining choices).
#define IDX_DEBUG_NOTE(bad, bit) ::idx::debug_note((bad), (bit))

// Defines the host function `fn` that copies this translation unit's word of the
// current device to *out and, with `clear`, resets it.
#define IDX_DEBUG_READER(fn)                                               \
  hipError_t fn(uint32_t *out, bool clear) {                               \
    void *p = nullptr;                                                     \
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_word));      \
    if (e == hipSuccess) e = hipMemcpy(out, p, 4, hipMemcpyDeviceToHost);  \
    const uint32_t zero = 0;                                               \
    if (e == hipSuccess && clear) e = hipMemcpy(p, &zero, 4, hipMemcpyHostToDevice); \
    return e;                                                              \
  }
#else
#define IDX_DEBUG_NOTE(bad, bit) ((void)0)
#define IDX_DEBUG_READER(fn)
#endif

}  // namespace idx
