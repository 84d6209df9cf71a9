// common.h -- internal helpers shared by the libdsq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsq.h"

namespace dsq {

constexpr int kWave = 64;
constexpr int kMaxCus = 256;  // MI355X; grids sized per CU never assume more

// Compute units of the current device, read once per device.
inline int device_cus() {
  static int cache[64] = {0};
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return kMaxCus;
  if (cache[d] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || n <= 0)
      n = kMaxCus;
    cache[d] = n;
  }
  return cache[d];
}

__host__ __device__ inline int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

// group = 256 (4-bit only) selects the two-level super-block format: the
// metadata of a group is then a 16-byte block header (fp16 d, fp16 dmin,
// twelve bytes of 6-bit sub-block scales and mins) instead of the
// (float scale, float zero point) pair.
constexpr int kSuperGroup = 256;
__host__ __device__ inline int meta_bytes_per_group(int group) {
  return group == kSuperGroup ? 16 : 8;
}

// Byte geometry of one packed batch entry (layout version 1, see dsq.h).
struct Layout {
  int64_t row_bytes;     // K * bits / 8
  int64_t groups;        // K / group
  int64_t meta_off;      // offset of the metadata table inside an entry
  int64_t stride;        // bytes per batch entry
};

__host__ __device__ inline Layout layout_of(int bits, int group, int64_t K, int64_t N) {
  Layout L;
  L.row_bytes = K * bits / 8;
  L.groups = K / group;
  L.meta_off = align256(N * L.row_bytes);
  L.stride = L.meta_off + align256(N * L.groups * meta_bytes_per_group(group));
  return L;
}

// Pointers to one batch entry.
struct QMat {
  const uint8_t* payload;  // [N][row_bytes]
  const float2* meta;      // [N][groups] of (scale, zero point)
};

inline QMat entry(const dsq_qweight& W, int64_t b) {
  Layout L = layout_of(W.bits, W.group, W.K, W.N);
  const uint8_t* base = static_cast<const uint8_t*>(W.data) + b * L.stride;
  return QMat{base, reinterpret_cast<const float2*>(base + L.meta_off)};
}

// ---------------------------------------------------------------------------
// Wave reductions.  All lanes end up with the result.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Reduce R per-lane partial sums across the wave in one pass ("reduce
// scatter"): at step s lanes exchange half of the remaining values, so R
// values cost R-1 exchanges plus log2(64/R) for the last one.  On return,
// lane l holds the full sum of value index row_of_lane(l) = l / (64 / R).
template <int R>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[R]) {
  const int lane = threadIdx.x & 63;
  int width = R;
  int bit = 32;
  // Halve the number of live values each step while R > 1.
#pragma unroll
  for (int step = 0; (1 << step) < R; ++step) {
    const int half = width >> 1;
    const bool upper = (lane & bit) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      // keep v[i + half] on upper lanes, v[i] on lower lanes
      float keep = upper ? v[i + half] : v[i];
      float send = upper ? v[i] : v[i + half];
      v[i] = keep + __shfl_xor(send, bit);
    }
    width = half;
    bit >>= 1;
  }
  float s = v[0];
  for (; bit >= 1; bit >>= 1) s += __shfl_xor(s, bit);
  return s;
}

// Row index held by lane l after wave_reduce_scatter<R>: the bits consumed
// were 32, 16, ... (most significant first), so row = l >> (6 - log2 R) read
// with the bit order reversed into value index order.
template <int R>
__device__ __forceinline__ int reduce_scatter_row(int lane) {
  if (R == 1) return 0;
  int r = 0;
  int idxbit = R >> 1;  // first step decides the top half of the index
  int bit = 32;
  for (int w = R; w > 1; w >>= 1) {
    if (lane & bit) r += idxbit;
    idxbit >>= 1;
    bit >>= 1;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Unpacking a 16-byte chunk of codes into floats.
// INT8: 16 codes, byte order = k order.
// INT4: 32 codes; word j gives k = 8j..8j+3 from its low nibbles and
//       k = 8j+4..8j+7 from its high nibbles (layout version 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bytes4_to_float(uint32_t w, float* f) {
  f[0] = (float)(w & 0xffu);
  f[1] = (float)((w >> 8) & 0xffu);
  f[2] = (float)((w >> 16) & 0xffu);
  f[3] = (float)(w >> 24);
}

template <int BITS>
struct Codes;

template <>
struct Codes<8> {
  static constexpr int kPerChunk = 16;
  __device__ __forceinline__ static void unpack(const uint4& c, float* f) {
    bytes4_to_float(c.x, f + 0);
    bytes4_to_float(c.y, f + 4);
    bytes4_to_float(c.z, f + 8);
    bytes4_to_float(c.w, f + 12);
  }
};

template <>
struct Codes<4> {
  static constexpr int kPerChunk = 32;
  __device__ __forceinline__ static void unpack(const uint4& c, float* f) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // The empty asm hides the mask from the compiler, which would otherwise
      // fold it into one bit-field extract per code; each masked byte then
      // converts with a single v_cvt_f32_ubyteN (11 instructions per 8 codes
      // instead of 16).
      uint32_t lo = w[j] & 0x0F0F0F0Fu, hi = (w[j] >> 4) & 0x0F0F0F0Fu;
      asm("" : "+v"(lo), "+v"(hi));
      bytes4_to_float(lo, f + 8 * j);
      bytes4_to_float(hi, f + 8 * j + 4);
    }
  }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming 16-byte load (weights are read once per call).
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// Activation vectors staged in LDS.  A lane reads its 16-byte chunk's
// EPC = 16 or 32 floats (F = EPC / 4 float4 slots) as F ds_read_b128 at a
// stride of F slots between lanes; rotating each chunk's slots by its chunk
// index spreads the lanes of one read over distinct banks.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ int lds_slot(int f) {
  const int c = f / F, j = f % F;
  return c * F + ((j + (F == 4 ? (c >> 1) : c)) & (F - 1));
}

// All threads of the workgroup copy n floats (n % 4 == 0) into LDS, swizzled
// for chunks of F float4.  The caller synchronises afterwards.
template <int F>
__device__ __forceinline__ void stage_lds(const float* __restrict__ src, int n, float4* lds) {
  const float4* s4 = reinterpret_cast<const float4*>(src);
  for (int f = threadIdx.x; f < n / 4; f += blockDim.x) lds[lds_slot<F>(f)] = s4[f];
}

// ---------------------------------------------------------------------------
// Wave-wide argmax by (value desc, index desc) with DPP row shifts and row
// broadcasts; every lane returns the winner.  Lanes with index < 0 hold no
// candidate.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia > ib);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xf, false);
  // branch-free: the comparison masks combine with bitwise ops and two selects
  // (a branch per step costs exec-mask round trips)
  const bool better = (oi >= 0) & ((i < 0) | (ov > v) | ((ov == v) & (oi > i)));
  v = better ? ov : v;
  i = better ? oi : i;
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<0x111, 0xf>(v, i);  // row_shr:1
  argmax_step<0x112, 0xf>(v, i);  // row_shr:2
  argmax_step<0x114, 0xf>(v, i);  // row_shr:4
  argmax_step<0x118, 0xf>(v, i);  // row_shr:8   -> lane 15 of each row
  argmax_step<0x142, 0xa>(v, i);  // row_bcast:15 into rows 1 and 3
  argmax_step<0x143, 0xc>(v, i);  // row_bcast:31 into rows 2 and 3 -> lane 63
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

}  // namespace dsq
