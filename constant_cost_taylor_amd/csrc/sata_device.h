// Device-side helpers shared by the prefill kernels (sata_prefill.hip,
// sata_prefill_b16.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sata {

// Tokens of the call window [t0, t0 + nw) that belong to a head: all nw of
// them, or, with per-head lengths, those before the head's length (a length
// is clamped to [0, n_total]).  Keys and values past it enter nothing, and
// its output rows are written as zeros.
__device__ __forceinline__ int head_tokens(const int32_t* lens, int head, int64_t t0, int nw, int64_t n_total) {
  if (!lens) return nw;
  const int64_t len = min(max(static_cast<int64_t>(lens[head]), int64_t(0)), n_total);
  return static_cast<int>(min(max(len - t0, int64_t(0)), static_cast<int64_t>(nw)));
}

}  // namespace sata
