// Device-side helpers shared by the kernels (sata_prefill.hip,
// sata_prefill_b16.hip, sata_decode.hip).  Not part of the public ABI.
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

// Max over the wave by DPP (prefix maxima within rows of 16, then across
// rows; lane 63 ends with the total), broadcast from lane 63.  Every lane of
// the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false);
  return fmaxf(x, __int_as_float(y));
}
__device__ __forceinline__ float wave_max(float x) {
  x = dpp_max<0x111>(x);   // row_shr:1
  x = dpp_max<0x112>(x);   // row_shr:2
  x = dpp_max<0x114>(x);   // row_shr:4
  x = dpp_max<0x118>(x);   // row_shr:8
  x = dpp_max<0x142>(x);   // row_bcast:15
  x = dpp_max<0x143>(x);   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

}  // namespace sata
