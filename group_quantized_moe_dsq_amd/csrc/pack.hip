// pack.hip -- quantize fp32 weights into the device layout (version 1): the
// group format, and the two-level super-block 4-bit format (group 256).
//
// Quantization rule: "Hand-writing a DeepSeek inference engine in pure C"
// (hnwysp.cn/news/134870) §3.2: per group of `group` consecutive weights
// along K, scale = (max - min) / (2^bits - 1), zp = round(-min / scale),
// q = clamp(round(v / scale) + zp, 0, 2^bits - 1); scale and zp kept in fp32;
// INT4 stores two codes per byte.  §5.1: a zero scale is an error, reported
// through the status word instead of producing inf/NaN codes.
//
// All arithmetic is IEEE fp32: the library is compiled with correctly rounded
// fp32 division and roundf rounds half-way cases away from zero, so the codes
// are the exact ones the rule defines.
#include <float.h>

#include "common.h"
#include "internal.h"

namespace dsq {

// One thread quantizes one group.  The 64/128 inputs of a group are read as
// float4 (adjacent threads read adjacent groups); the codes are written as
// 16-byte stores and the (scale, zp) pair as one 8-byte store.
template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ src,
                                                   uint8_t* __restrict__ base, int64_t N,
                                                   int64_t K, int group, int64_t stride,
                                                   int64_t meta_off, int64_t first,
                                                   int64_t count, int32_t* __restrict__ flags) {
  const int64_t groups = K / group;
  const int64_t total = count * N * groups;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int64_t g = gid % groups;
  const int64_t rowall = gid / groups;  // b * N + n
  const int64_t n = rowall % N;
  const int64_t b = rowall / N;
  const float4* s4 = reinterpret_cast<const float4*>(src + rowall * K + g * group);
  const int nv4 = group / 4;

  // Pass 1: range and finiteness.  Comparisons as in the printed routine.
  float lo = FLT_MAX, hi = -FLT_MAX;
  bool nonfinite = false;
  for (int i = 0; i < nv4; ++i) {
    const float4 v = s4[i];
    const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      nonfinite |= !isfinite(a[j]);
      if (a[j] < lo) lo = a[j];
      if (a[j] > hi) hi = a[j];
    }
  }
  constexpr int qmax = (1 << BITS) - 1;
  constexpr float levels = float(qmax);
  int32_t flag = nonfinite ? DSQ_FLAG_NONFINITE : 0;
  float scale = 0.0f, zr = 0.0f;
  if (!flag) {
    scale = (hi - lo) / levels;
    if (!(scale > 0.0f) || !isfinite(scale)) {
      flag |= DSQ_FLAG_DEGENERATE;
    } else {
      zr = roundf(-lo / scale);
      // zp must stay an exact integer in fp32 (and inside int32)
      if (!(fabsf(zr) <= 16777216.0f)) flag |= DSQ_FLAG_DEGENERATE;
    }
  }
  if (flag) {
    scale = 0.0f;
    zr = 0.0f;
    if (flags) atomicOr(flags, flag);
  }
  const int32_t z = int32_t(zr);

  uint8_t* entry = base + (first + b) * stride;
  const int64_t row_bytes = K * BITS / 8;
  uint8_t* qrow = entry + n * row_bytes + g * group * BITS / 8;
  float2* meta = reinterpret_cast<float2*>(entry + meta_off);
  meta[n * groups + g] = make_float2(scale, zr);

  // Pass 2: codes, written 16 bytes at a time.
  auto code = [&](float v) -> uint32_t {
    if (flag) return 0u;
    int32_t q = int32_t(roundf(v / scale)) + z;
    q = q < 0 ? 0 : (q > qmax ? qmax : q);
    return uint32_t(q);
  };
  uint4* out = reinterpret_cast<uint4*>(qrow);
  if (BITS == 8) {
    for (int c = 0; c < group / 16; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = s4[c * 4 + j];
        w[j] = code(v.x) | (code(v.y) << 8) | (code(v.z) << 16) | (code(v.w) << 24);
      }
      out[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    // 32 codes per 16-byte chunk; word j covers k = 8j..8j+7 of the chunk:
    // byte i = code(8j+i) | code(8j+4+i) << 4
    for (int c = 0; c < group / 32; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 a = s4[c * 8 + 2 * j];
        const float4 h = s4[c * 8 + 2 * j + 1];
        w[j] = (code(a.x) | (code(h.x) << 4)) | ((code(a.y) | (code(h.y) << 4)) << 8) |
               ((code(a.z) | (code(h.z) << 4)) << 16) | ((code(a.w) | (code(h.w) << 4)) << 24);
      }
      out[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Two-level super-block 4-bit format (group = 256).  The block is the one
// "ds4 code walkthrough" prints in trace 4 (quant block struct sizes): fp16 d,
// fp16 dmin, 12 bytes of scales, 128 bytes of nibbles for 256 weights.  Its
// arithmetic, read from those fields: 8 sub-blocks of 32 weights, sub-block j
// with a 6-bit scale sc_j and a 6-bit min m_j, weight = d*sc_j*q - dmin*m_j.
// The quantizer applies the group rule of §3.2 level by level, in fp32 with
// roundf:
//   off_j = max(0, -min_j), step_j = (max_j + off_j) / 15,
//   d = fp16(max step / 63), dmin = fp16(max off / 63)  (round to nearest even),
//   sc_j = clamp(round(step_j / d), 0, 63), m_j = clamp(round(off_j / dmin), 0, 63),
//   q = clamp(round((w + dmin*m_j) / (d*sc_j)), 0, 15).
// A block with a NaN or infinity, or whose d or dmin overflows fp16, is
// written as zeros and flagged.
//
// One thread per block.  The codes go to the payload in the 4-bit layout of
// the group format (a 16-byte chunk is one sub-block), the 16-byte header
// (d | dmin << 16, then the 96 bits of 6-bit fields sc_0..7, m_0..7 from bit
// 0 up) to the metadata table.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f16_bits(float f) {
  const _Float16 h = static_cast<_Float16>(f);  // v_cvt_f16_f32: round to nearest even
  return uint32_t(__builtin_bit_cast(uint16_t, h));
}

__device__ __forceinline__ float f16_value(uint32_t bits) {
  return float(__builtin_bit_cast(_Float16, uint16_t(bits)));
}

__global__ __launch_bounds__(256) void pack_sb4_kernel(const float* __restrict__ src,
                                                       uint8_t* __restrict__ base, int64_t N,
                                                       int64_t K, int64_t stride,
                                                       int64_t meta_off, int64_t first,
                                                       int64_t count, int32_t* __restrict__ flags) {
  const int64_t nb = K / kSuperGroup;
  const int64_t total = count * N * nb;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int64_t blk = gid % nb;
  const int64_t rowall = gid / nb;  // b * N + n
  const int64_t n = rowall % N;
  const int64_t b = rowall / N;
  const float4* s4 = reinterpret_cast<const float4*>(src + rowall * K + blk * kSuperGroup);

  float step[8], off[8];
  float smax = 0.0f, omax = 0.0f;
  bool nonfinite = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float lo = FLT_MAX, hi = -FLT_MAX;
    for (int i = 0; i < 8; ++i) {
      const float4 v = s4[8 * j + i];
      const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nonfinite |= !isfinite(a[e]);
        if (a[e] < lo) lo = a[e];
        if (a[e] > hi) hi = a[e];
      }
    }
    off[j] = lo < 0.0f ? -lo : 0.0f;
    step[j] = (hi + off[j]) / 15.0f;
    if (step[j] > smax) smax = step[j];
    if (off[j] > omax) omax = off[j];
  }
  int32_t flag = nonfinite ? DSQ_FLAG_NONFINITE : 0;
  uint32_t d16 = 0, m16 = 0;
  if (!flag) {
    d16 = f16_bits(smax / 63.0f);
    m16 = f16_bits(omax / 63.0f);
    if ((d16 & 0x7c00u) == 0x7c00u || (m16 & 0x7c00u) == 0x7c00u) flag = DSQ_FLAG_DEGENERATE;
  }
  if (flag) {
    d16 = m16 = 0;
    if (flags) atomicOr(flags, flag);
  }
  const float df = f16_value(d16), mf = f16_value(m16);
  uint64_t lo64 = 0, hi64 = 0;  // the 96 bits of 6-bit fields
  float S[8], M[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float sc = df > 0.0f ? roundf(step[j] / df) : 0.0f;
    float mn = mf > 0.0f ? roundf(off[j] / mf) : 0.0f;
    sc = sc < 0.0f ? 0.0f : (sc > 63.0f ? 63.0f : sc);
    mn = mn < 0.0f ? 0.0f : (mn > 63.0f ? 63.0f : mn);
    S[j] = df * sc;
    M[j] = mf * mn;
    const uint64_t vs = uint64_t(sc), vm = uint64_t(mn);
    const int ps = 6 * j, pm = 6 * (8 + j);  // ps <= 42; pm = 48 .. 90
    lo64 |= vs << ps;
    if (pm + 6 <= 64) {
      lo64 |= vm << pm;
    } else if (pm >= 64) {
      hi64 |= vm << (pm - 64);
    } else {  // straddles bit 64
      lo64 |= vm << pm;
      hi64 |= vm >> (64 - pm);
    }
  }
  uint8_t* entry = base + (first + b) * stride;
  uint4* hdr = reinterpret_cast<uint4*>(entry + meta_off);
  hdr[n * nb + blk] = make_uint4(d16 | (m16 << 16), uint32_t(lo64), uint32_t(lo64 >> 32),
                                 uint32_t(hi64));

  auto code = [&](float v, int j) -> uint32_t {
    if (flag || !(S[j] > 0.0f)) return 0u;
    float q = roundf((v + M[j]) / S[j]);
    q = q < 0.0f ? 0.0f : (q > 15.0f ? 15.0f : q);
    return uint32_t(q);
  };
  // sub-block j = one 16-byte chunk; word w covers k = 8w..8w+7 of it:
  // byte i = code(8w+i) | code(8w+4+i) << 4
  uint4* out = reinterpret_cast<uint4*>(entry + n * (K / 2) + blk * (kSuperGroup / 2));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 a = s4[8 * j + 2 * q4];
      const float4 h = s4[8 * j + 2 * q4 + 1];
      w[q4] = (code(a.x, j) | (code(h.x, j) << 4)) | ((code(a.y, j) | (code(h.y, j) << 4)) << 8) |
              ((code(a.z, j) | (code(h.z, j) << 4)) << 16) |
              ((code(a.w, j) | (code(h.w, j) << 4)) << 24);
    }
    out[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_pack(const float* src, const dsq_qweight& W, int64_t first, int64_t count,
                       int32_t* flags, hipStream_t stream) {
  const Layout L = layout_of(W.bits, W.group, W.K, W.N);
  const int64_t total = count * W.N * L.groups;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  uint8_t* base = static_cast<uint8_t*>(W.data);
  if (W.group == kSuperGroup)
    hipLaunchKernelGGL(pack_sb4_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, src, base,
                       W.N, W.K, L.stride, L.meta_off, first, count, flags);
  else if (W.bits == 8)
    hipLaunchKernelGGL(pack_kernel<8>, dim3(unsigned(blocks)), dim3(256), 0, stream, src, base,
                       W.N, W.K, W.group, L.stride, L.meta_off, first, count, flags);
  else
    hipLaunchKernelGGL(pack_kernel<4>, dim3(unsigned(blocks)), dim3(256), 0, stream, src, base,
                       W.N, W.K, W.group, L.stride, L.meta_off, first, count, flags);
  return hipGetLastError();
}

}  // namespace dsq
