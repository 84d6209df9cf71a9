// pack.hip -- quantize fp32 weights into the device layout (version 1).
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

hipError_t launch_pack(const float* src, const dsq_qweight& W, int64_t first, int64_t count,
                       int32_t* flags, hipStream_t stream) {
  const Layout L = layout_of(W.bits, W.group, W.K, W.N);
  const int64_t total = count * W.N * L.groups;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  uint8_t* base = static_cast<uint8_t*>(W.data);
  if (W.bits == 8)
    hipLaunchKernelGGL(pack_kernel<8>, dim3(unsigned(blocks)), dim3(256), 0, stream, src, base,
                       W.N, W.K, W.group, L.stride, L.meta_off, first, count, flags);
  else
    hipLaunchKernelGGL(pack_kernel<4>, dim3(unsigned(blocks)), dim3(256), 0, stream, src, base,
                       W.N, W.K, W.group, L.stride, L.meta_off, first, count, flags);
  return hipGetLastError();
}

}  // namespace dsq
