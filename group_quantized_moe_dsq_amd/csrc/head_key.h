// head_key.h -- the 64-bit rank key of the output-head selection and a wave
// maximum over it, shared by the selection kernels and the GEMV that can
// reduce its own outputs.
//
// Rank order ("Hand-writing a DeepSeek inference engine in pure C" §2.1: the
// output projection's logits choose the next token): larger value first,
// equal values (-0 equals +0) to the smaller index, NaN below every number.
// high word: the float's bits mapped to an unsigned integer of the same order
// (negative values complemented, positive ones with the top bit set), both
// zeros alike, NaN mapped to 0; low word: the complemented index.  Keys are
// distinct, and 0 (the padding) ranks below every real value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsq {

__device__ __forceinline__ uint64_t head_key(float v, uint32_t i) {
  uint32_t u = __float_as_uint(v);
  uint32_t h;
  if (v != v) {
    h = 0u;
  } else {
    if (v == 0.0f) u = 0u;  // -0 ranks with +0
    h = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (uint64_t(h) << 32) | uint64_t(~i);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// One step of a wave maximum: each lane compares with the lane the DPP
// control names (lanes without a source, or in rows outside ROW_MASK, keep
// their own key).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
  const int lo = int(uint32_t(v)), hi = int(uint32_t(v >> 32));
  const uint32_t olo = uint32_t(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false));
  const uint32_t ohi = uint32_t(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false));
  return umax64(v, (uint64_t(ohi) << 32) | olo);
}

// The largest key of the wave, in every lane: row shifts leave each row's
// maximum in its lane 15, the two row broadcasts carry them to lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  v = max_step<0x111, 0xf>(v);  // row_shr:1
  v = max_step<0x112, 0xf>(v);  // row_shr:2
  v = max_step<0x114, 0xf>(v);  // row_shr:4
  v = max_step<0x118, 0xf>(v);  // row_shr:8
  v = max_step<0x142, 0xa>(v);  // row_bcast:15
  v = max_step<0x143, 0xc>(v);  // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(v)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 63);
  return (uint64_t(hi) << 32) | lo;
}

}  // namespace dsq
