// gemv_sb4.hip -- fused-dequant GEMV (M = 1) over the two-level super-block
// 4-bit format (group = 256).
//
// The block is the one "ds4 code walkthrough" prints in trace 4 (quant block
// struct sizes): fp16 d, fp16 dmin, 6-bit scales and mins of 8 sub-blocks of
// 32, 4-bit codes; a weight dequantizes to d*sc_j*q - dmin*m_j.  The matmul
// folds the dequantization into its inner loop ("Hand-writing a DeepSeek
// inference engine in pure C", hnwysp.cn/news/134870, §3.2-§3.3) and is
// HBM-bound: 0.5625 bytes per weight (codes 0.5, headers 16 B per 256).
//
// Mapping (wave64), as the group-format GEMV: a row is split into 16-byte
// chunks, lane l takes chunks l, l+64, ...; a 16-byte chunk of 4-bit codes is
// exactly one sub-block, so per chunk
//   sum x (S q - M) = S * sum x q - M * sum x,   S = d*sc_j, M = dmin*m_j,
// with sum x precomputed per lane.  The lane reads its block's 16-byte header
// (eight lanes share one, each lane loads one of its words and a DPP quad
// exchange rebuilds it) and decodes d, dmin and its two 6-bit fields with a
// few shifts.  The activation vector is staged in LDS once per workgroup and
// each lane keeps its slice in registers; the next row block's loads are
// issued before the current one's arithmetic.
#include "common.h"
#include "gemv_core.h"
#include "internal.h"

namespace dsq {

#ifndef DSQ_GEMV_SB_R
#define DSQ_GEMV_SB_R 2  // rows per wave step
#endif
#ifndef DSQ_GEMV_SB_FENCE
#define DSQ_GEMV_SB_FENCE 1  // keep each buffer's loads ahead of the arithmetic (57.5 against 59.4 us)
#endif
#if DSQ_GEMV_SB_FENCE
#define SB_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#else
#define SB_SCHED_FENCE() ((void)0)
#endif

// (S, M) of sub-block j from its block's header: x = d | dmin << 16 (fp16
// bits), then the 96 bits of 6-bit fields sc_0..7, m_0..7 (field f at bit 6f).
__device__ __forceinline__ float2 sb_scale_min(const uint4& h, int j) {
  const float d = float(__builtin_bit_cast(_Float16, uint16_t(h.x & 0xffffu)));
  const float dmin = float(__builtin_bit_cast(_Float16, uint16_t(h.x >> 16)));
  const uint64_t lo = (uint64_t(h.z) << 32) | h.y;  // bits 0..63
  const uint64_t hi = (uint64_t(h.w) << 32) | h.z;  // bits 32..95
  const int ps = 6 * j, pm = 48 + 6 * j;            // ps <= 42, pm = 48 .. 90
  const uint32_t sc = uint32_t(lo >> ps) & 63u;
  const uint32_t m = uint32_t(pm <= 58 ? (lo >> pm) : (hi >> (pm - 32))) & 63u;
  return make_float2(d * float(sc), dmin * float(m));
}

// A block header is shared by the 8 lanes of its sub-blocks, so each lane
// loads one of its four words (lane l: word l % 4) and the four lanes of a
// DPP quad hand them to each other at dot time: one register per (row,
// chunk) instead of four.  The number of chunks in a row (K/32) is a multiple
// of 8, so the lanes of a quad are all inside the row or all past its end.
// 32 codes of a chunk to floats.  The masked nibble words are passed through
// an empty asm so the compiler cannot fold the mask into per-code bit-field
// extracts: each byte then converts with one v_cvt_f32_ubyteN (1.25
// instructions per code instead of 2).
__device__ __forceinline__ void sb_unpack(const uint4& c, float* f) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t lo = w[j] & 0x0F0F0F0Fu, hi = (w[j] >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(lo), "+v"(hi));
    bytes4_to_float(lo, f + 8 * j);
    bytes4_to_float(hi, f + 8 * j + 4);
  }
}

template <int R, int KCH>
struct SbRowChunks {
  uint4 w[R][KCH];
  uint32_t hw[R][KCH];

  //   prow[r] : first byte of row r's codes;  hrow[r] : row r's block headers
  __device__ __forceinline__ void load(const uint8_t* const (&prow)[R],
                                       const uint4* const (&hrow)[R], int nchunk, int lane) {
    // lanes past the row's end re-read a valid chunk (clamped, no branch);
    // their x slice is zero, so the duplicate contributes exactly zero
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = min(lane + 64 * i, nchunk - 1);
        w[r][i] = ld_nt(reinterpret_cast<const uint4*>(prow[r]) + c);
        hw[r][i] = reinterpret_cast<const uint32_t*>(hrow[r] + (c >> 3))[lane & 3];
      }
    }
  }

  __device__ __forceinline__ static uint4 header(uint32_t v) {
    // quad_perm broadcasts of lanes 0..3 of the quad
    return make_uint4(uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x00, 0xf, 0xf, false)),
                      uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x55, 0xf, 0xf, false)),
                      uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xaa, 0xf, 0xf, false)),
                      uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xff, 0xf, 0xf, false)));
  }

  __device__ __forceinline__ void dot(const XSlice<4, KCH>& xs, int nchunk, int lane,
                                      float (&acc)[R]) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = min(lane + 64 * i, nchunk - 1);
        const float2 sm = sb_scale_min(header(hw[r][i]), c & 7);
        float f[32];
        sb_unpack(w[r][i], f);
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; e += 2) {
          d0 = fmaf(xs.v[i][e], f[e], d0);
          d1 = fmaf(xs.v[i][e + 1], f[e + 1], d1);
        }
        a = fmaf(sm.x, d0 + d1, fmaf(-sm.y, xs.s[i], a));
      }
      acc[r] = a;
    }
  }
};

// BUFS row blocks in flight per wave: 3 when every wave runs at least three
// (the loads of a row block issued two steps ahead; vocab-size matrices), 2
// otherwise: the three-buffer loop loads unconditionally (clamped), so a wave
// with one row block would fetch three (4096 x 4096: 7.2 against 5.9 us).
template <int R, int KCH, int BUFS>
__global__ __launch_bounds__(256) void gemv_sb4_kernel(const uint8_t* __restrict__ payload,
                                                       const uint4* __restrict__ hdr,
                                                       const float* __restrict__ x,
                                                       float* __restrict__ y, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int row_bytes = K / 2;
  const int nchunk = row_bytes / 16;
  const int nb = K / kSuperGroup;

  auto load = [&](SbRowChunks<R, KCH>& C, int rb) {
    const uint8_t* prow[R];
    const uint4* hrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rb * R + r, N - 1);
      prow[r] = payload + int64_t(row) * row_bytes;
      hrow[r] = hdr + int64_t(row) * nb;
    }
    C.load(prow, hrow, nchunk, lane);
  };
  XSlice<4, KCH> xs;  // this lane's slice of x, reused for every row
  auto finish = [&](const SbRowChunks<R, KCH>& C, int rb) {
    float acc[R];
    C.dot(xs, nchunk, lane, acc);
    const float tot = wave_reduce_scatter<R>(acc);
    if ((lane & (64 / R - 1)) == 0) {
      const int row = rb * R + reduce_scatter_row<R>(lane);
      if (row < N) y[row] = tot;
    }
  };

  extern __shared__ float4 xl[];
  if constexpr (BUFS == 3) {
  // Three buffers: a row block's loads are issued two steps before its
  // arithmetic.  Loads past the last row block re-read the last row (clamped
  // addresses), so every load is unconditional and the waits stay static.
  SbRowChunks<R, KCH> A, B, C;
  int rb = wave;
  load(A, rb);
  load(B, rb + nwaves);
  // every thread takes its share of x, so a wave without rows leaves only
  // after the barrier
  stage_lds<8>(x, K, xl);
  __syncthreads();
  if (rb * R >= N) return;
  xs.load_lds(xl, nchunk, lane);
  xs.sums();
  for (;; rb += 3 * nwaves) {
    load(C, rb + 2 * nwaves);
    SB_SCHED_FENCE();
    finish(A, rb);
    if ((rb + nwaves) * R >= N) break;
    load(A, rb + 3 * nwaves);
    SB_SCHED_FENCE();
    finish(B, rb + nwaves);
    if ((rb + 2 * nwaves) * R >= N) break;
    load(B, rb + 4 * nwaves);
    SB_SCHED_FENCE();
    finish(C, rb + 2 * nwaves);
    if ((rb + 3 * nwaves) * R >= N) break;
  }
  } else {
  SbRowChunks<R, KCH> A, B;
  int rb = wave;
  if (rb * R < N) load(A, rb);
  stage_lds<8>(x, K, xl);
  __syncthreads();
  xs.load_lds(xl, nchunk, lane);
  xs.sums();
  while (rb * R < N) {
    const int rb1 = rb + nwaves;
    const bool more1 = rb1 * R < N;
    if (more1) load(B, rb1);
    finish(A, rb);
    if (!more1) break;
    const int rb2 = rb1 + nwaves;
    if (rb2 * R < N) load(A, rb2);
    finish(B, rb1);
    rb = rb2;
  }
  }
}

// Rows longer than 4 chunks per lane (K > 8192): x is re-read from memory
// (L1/L2) for every chunk instead of being held in registers.
template <int R>
__global__ __launch_bounds__(256) void gemv_sb4_kernel_long(const uint8_t* __restrict__ payload,
                                                            const uint4* __restrict__ hdr,
                                                            const float* __restrict__ x,
                                                            float* __restrict__ y, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int row_bytes = K / 2;
  const int nchunk = row_bytes / 16;
  const int nb = K / kSuperGroup;
  for (int rb = wave; rb * R < N; rb += nwaves) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    for (int c = lane; c < nchunk; c += 64) {
      float xv[32];
      const float4* x4 = reinterpret_cast<const float4*>(x + c * 32);
      float xsum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 v = x4[j];
        xv[4 * j] = v.x;
        xv[4 * j + 1] = v.y;
        xv[4 * j + 2] = v.z;
        xv[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) xsum += xv[e];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(rb * R + r, N - 1);
        const uint4 wv = ld_nt(reinterpret_cast<const uint4*>(payload + int64_t(row) * row_bytes) + c);
        const float2 sm = sb_scale_min(hdr[int64_t(row) * nb + (c >> 3)], c & 7);
        float f[32];
        sb_unpack(wv, f);
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) d = fmaf(xv[e], f[e], d);
        acc[r] = fmaf(sm.x, d, fmaf(-sm.y, xsum, acc[r]));
      }
    }
    const float tot = wave_reduce_scatter<R>(acc);
    if ((lane & (64 / R - 1)) == 0) {
      const int row = rb * R + reduce_scatter_row<R>(lane);
      if (row < N) y[row] = tot;
    }
  }
}

namespace {

#ifndef DSQ_GEMV_SB_WAVES_PER_CU
#define DSQ_GEMV_SB_WAVES_PER_CU 8
#endif
constexpr int kSbMaxWaves = 256 * DSQ_GEMV_SB_WAVES_PER_CU;  // grid-stride beyond

template <int R, int KCH>
hipError_t go_sb(const uint8_t* payload, const uint4* hdr, const float* x, float* y, int N, int K,
                 hipStream_t stream) {
  const int rowblocks = (N + R - 1) / R;
  const int waves = rowblocks < kSbMaxWaves ? rowblocks : kSbMaxWaves;
  const int blocks = (waves + 3) / 4;
  if (rowblocks >= 3 * waves)
    hipLaunchKernelGGL((gemv_sb4_kernel<R, KCH, 3>), dim3(blocks), dim3(256), size_t(K) * 4,
                       stream, payload, hdr, x, y, N, K);
  else
    hipLaunchKernelGGL((gemv_sb4_kernel<R, KCH, 2>), dim3(blocks), dim3(256), size_t(K) * 4,
                       stream, payload, hdr, x, y, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_sb4(const dsq_qweight& W, int64_t expert, const float* x, float* y,
                           hipStream_t stream) {
  const Layout L = layout_of(W.bits, W.group, W.K, W.N);
  const uint8_t* base = static_cast<const uint8_t*>(W.data) + expert * L.stride;
  const uint4* hdr = reinterpret_cast<const uint4*>(base + L.meta_off);
  const int N = int(W.N), K = int(W.K);
  constexpr int R = DSQ_GEMV_SB_R;
  const int kch = (K / 32 + 63) / 64;
  switch (kch) {
    case 1: return go_sb<R, 1>(base, hdr, x, y, N, K, stream);
    case 2: return go_sb<R, 2>(base, hdr, x, y, N, K, stream);
    case 3: return go_sb<R, 3>(base, hdr, x, y, N, K, stream);
    case 4: return go_sb<R, 4>(base, hdr, x, y, N, K, stream);
    default: {
      const int rowblocks = (N + R - 1) / R;
      const int waves = rowblocks < kSbMaxWaves ? rowblocks : kSbMaxWaves;
      hipLaunchKernelGGL((gemv_sb4_kernel_long<R>), dim3((waves + 3) / 4), dim3(256), 0, stream,
                         base, hdr, x, y, N, K);
      return hipGetLastError();
    }
  }
}

}  // namespace dsq
