// gemv_core.h -- the fused-dequant dot-product core shared by the decode
// kernels (dense GEMV, MoE gate/up + SwiGLU, MoE down + combine).
//
// y[n] = sum_k x[k] * (q[n][k] - zp) * scale  ("Hand-writing a DeepSeek
// inference engine in pure C", hnwysp.cn/news/134870, §3.2: dequantize inside
// the matmul's inner loop).
//
// A row is split into 16-byte chunks of codes; lane l of a wave owns chunks
// l, l + 64, ... (KCH of them), so one wave-wide load covers 1 KiB of one row
// and every lane sees the same K positions in every row.  The lane's slice of
// x therefore sits in registers (XSlice) and is reused across rows.  A chunk
// lies inside one quantization group, so the zero point is factored per chunk:
//   sum_c x (q - zp) s = s * (sum_c x q - zp * sum_c x)
// which costs one convert and one FMA per code plus two FMAs per chunk.
//
// RowChunks splits a step into load() and dot() so a kernel can issue the
// next step's loads before doing the current step's arithmetic.
#pragma once

#include "common.h"

namespace dsq {

template <int BITS, int KCH>
struct XSlice {
  static constexpr int EPC = Codes<BITS>::kPerChunk;
  float v[KCH][EPC];
  float s[KCH];

  // x: the K activations; chunks past nchunk read as zero.
  __device__ __forceinline__ void load(const float* __restrict__ x, int nchunk, int lane) {
    // clamped addresses and a select afterwards: every load is issued up front
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = lane + 64 * i;
      const float4* x4 = reinterpret_cast<const float4*>(x + min(c, nchunk - 1) * EPC);
      const bool keep = c < nchunk;
#pragma unroll
      for (int j = 0; j < EPC / 4; ++j) {
        const float4 t = x4[j];
        v[i][4 * j + 0] = keep ? t.x : 0.0f;
        v[i][4 * j + 1] = keep ? t.y : 0.0f;
        v[i][4 * j + 2] = keep ? t.z : 0.0f;
        v[i][4 * j + 3] = keep ? t.w : 0.0f;
      }
    }
  }
  // The same slice from a vector staged in LDS by stage_lds<EPC / 4>.
  __device__ __forceinline__ void load_lds(const float4* lds, int nchunk, int lane) {
    constexpr int F = EPC / 4;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = lane + 64 * i;
      const int cc = min(c, nchunk - 1);
      const bool keep = c < nchunk;
#pragma unroll
      for (int j = 0; j < F; ++j) {
        const float4 t = lds[lds_slot<F>(cc * F + j)];
        v[i][4 * j + 0] = keep ? t.x : 0.0f;
        v[i][4 * j + 1] = keep ? t.y : 0.0f;
        v[i][4 * j + 2] = keep ? t.z : 0.0f;
        v[i][4 * j + 3] = keep ? t.w : 0.0f;
      }
    }
  }
  // per-chunk sums of x, needed by the factored zero point
  __device__ __forceinline__ void sums() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) a += v[i][e];
      s[i] = a;
    }
  }
};

template <int BITS, int R, int KCH>
struct RowChunks {
  static constexpr int EPC = Codes<BITS>::kPerChunk;
  uint4 w[R][KCH];
  float2 m[R][KCH];

  //   prow[r] : first byte of row r's codes;  mrow[r] : row r's (scale, zp)
  __device__ __forceinline__ void load(const uint8_t* const (&prow)[R],
                                       const float2* const (&mrow)[R], int nchunk, int group,
                                       int lane) {
    // Lanes past the row's end load a valid chunk again (clamped address, no
    // branch, so every load is in flight at once); their x slice is zero, so
    // the duplicate contributes exactly zero.
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = min(lane + 64 * i, nchunk - 1);
        w[r][i] = ld_nt(reinterpret_cast<const uint4*>(prow[r]) + c);
        m[r][i] = mrow[r][(c * EPC) / group];
      }
    }
  }

  // per-lane partial sums of the R rows over this lane's chunks
  __device__ __forceinline__ void dot(const XSlice<BITS, KCH>& xs, float (&acc)[R]) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        float f[EPC];
        Codes<BITS>::unpack(w[r][i], f);
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; e += 2) {
          d0 = fmaf(xs.v[i][e], f[e], d0);
          d1 = fmaf(xs.v[i][e + 1], f[e + 1], d1);
        }
        a = fmaf(m[r][i].x, fmaf(-m[r][i].y, xs.s[i], d0 + d1), a);
      }
      acc[r] = a;
    }
  }
};

}  // namespace dsq
