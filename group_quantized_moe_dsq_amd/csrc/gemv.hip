// gemv.hip -- fused-dequant GEMV for one activation vector (decode, M = 1).
//
// Computes y[n] = sum_k x[k] * (q[n][k] - zp[n][g]) * scale[n][g], the
// matmul with dequantization folded into its inner loop ("Hand-writing a
// DeepSeek inference engine in pure C", hnwysp.cn/news/134870, §3.2 and
// §3.3).  The loop is HBM-bound: every weight byte is read once.
//
// Mapping (wave64):
//   * A row is split into 16-byte chunks; lane l of a wave takes chunks
//     l, l+64, l+128, ...  A wave's load instruction therefore covers 1 KiB
//     of one row, contiguous, and every lane sees the same K positions for
//     every row, so its slice of x is loaded into registers once per wave and
//     reused for all the rows the wave visits (no LDS, no barrier).
//   * A 16-byte chunk never straddles a quantization group (groups are 32,
//     64 or 128 bytes and chunk offsets are 16-aligned), so the zero point is
//     factored per chunk:  sum_c x*(q - zp)*s = s * (sum_c x*q - zp * sum_c x)
//     with sum_c x precomputed per lane.  Per code that leaves one convert and
//     one FMA.
//   * R rows per wave step; their partial sums are reduced across the wave in
//     one reduce-scatter, after which R lanes store the R outputs.  The next
//     step's loads are issued before the current step's arithmetic.
#include <algorithm>

#include "common.h"
#include "gemv_core.h"
#include "head_key.h"
#include "internal.h"

namespace dsq {

// Launch shape (tuned on MI355X; overridable at build time for sweeps).
#ifndef DSQ_GEMV_R8
#define DSQ_GEMV_R8 2  // rows per wave step, INT8
#endif
#ifndef DSQ_GEMV_R4
#define DSQ_GEMV_R4 2  // rows per wave step, INT4
#endif
#ifndef DSQ_GEMV_WAVES_PER_CU
#define DSQ_GEMV_WAVES_PER_CU 8
#endif
#ifndef DSQ_GEMV_WAVES_PER_CU_LARGE
#define DSQ_GEMV_WAVES_PER_CU_LARGE 4  // INT8, when every wave gets >= 4 row blocks at the above
#endif
#ifndef DSQ_GEMV_WAVES_PER_CU_LARGE4
#define DSQ_GEMV_WAVES_PER_CU_LARGE4 12  // the same for INT4 (three workgroups per CU)
#endif

template <int BITS, int R, int KCH>
__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t* __restrict__ payload,
                                                   const float2* __restrict__ meta,
                                                   const float* __restrict__ x,
                                                   float* __restrict__ y, int N, int K,
                                                   int group) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int row_bytes = K / 8 * BITS;  // K is a multiple of the group
  const int nchunk = row_bytes / 16;
  const int groups = K / group;

  auto load = [&](RowChunks<BITS, R, KCH>& C, int rb) {
    const uint8_t* prow[R];
    const float2* mrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rb * R + r, N - 1);
      prow[r] = payload + int64_t(row) * row_bytes;
      mrow[r] = meta + int64_t(row) * groups;
    }
    C.load(prow, mrow, nchunk, group, lane);
  };
  XSlice<BITS, KCH> xs;  // this lane's slice of x, reused for every row
  auto finish = [&](const RowChunks<BITS, R, KCH>& C, int rb) {
    float acc[R];
    C.dot(xs, acc);
    const float tot = wave_reduce_scatter<R>(acc);
    if ((lane & (64 / R - 1)) == 0) {
      const int row = rb * R + reduce_scatter_row<R>(lane);
      if (row < N) y[row] = tot;
    }
  };

  // Two buffers: the loads of the wave's next row block are in flight while
  // the current one is dequantized and reduced.  The first weight loads are
  // issued before x is staged, so the two latencies overlap; x is read from
  // memory once per workgroup and shared through LDS.
  extern __shared__ float4 xl[];
  RowChunks<BITS, R, KCH> A, B;
  int rb = wave;
  if (rb * R < N) load(A, rb);
  stage_lds<Codes<BITS>::kPerChunk / 4>(x, K, xl);
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

// The same loop as gemv_kernel, plus every wave's best rank key (head_key.h)
// of the rows it stored, written to wkey[wave]: the output head's top-1
// without a separate pass over the logits.  (A separate kernel, so that
// gemv_kernel's code stays as tuned.)
template <int BITS, int R, int KCH>
__global__ __launch_bounds__(256) void gemv_argmax_kernel(const uint8_t* __restrict__ payload,
                                                          const float2* __restrict__ meta,
                                                          const float* __restrict__ x,
                                                          float* __restrict__ y, int N, int K,
                                                          int group, uint64_t* __restrict__ wkey) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int row_bytes = K / 8 * BITS;  // K is a multiple of the group
  const int nchunk = row_bytes / 16;
  const int groups = K / group;

  auto load = [&](RowChunks<BITS, R, KCH>& C, int rb) {
    const uint8_t* prow[R];
    const float2* mrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rb * R + r, N - 1);
      prow[r] = payload + int64_t(row) * row_bytes;
      mrow[r] = meta + int64_t(row) * groups;
    }
    C.load(prow, mrow, nchunk, group, lane);
  };
  XSlice<BITS, KCH> xs;
  uint64_t best = 0;  // the best key of the rows this lane stored
  auto finish = [&](const RowChunks<BITS, R, KCH>& C, int rb) {
    float acc[R];
    C.dot(xs, acc);
    const float tot = wave_reduce_scatter<R>(acc);
    if ((lane & (64 / R - 1)) == 0) {
      const int row = rb * R + reduce_scatter_row<R>(lane);
      if (row < N) {
        y[row] = tot;
        best = umax64(best, head_key(tot, uint32_t(row)));
      }
    }
  };

  extern __shared__ float4 xl[];
  RowChunks<BITS, R, KCH> A, B;
  int rb = wave;
  if (rb * R < N) load(A, rb);
  stage_lds<Codes<BITS>::kPerChunk / 4>(x, K, xl);
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
  const uint64_t b = wave_max_key(best);  // every lane active: the loop is wave-uniform
  if (lane == 0) wkey[wave] = b;
}

// Rows longer than KMAX chunks per lane: x is re-read from memory (L1/L2)
// for every chunk instead of being held in registers.
template <int BITS, int R>
__global__ __launch_bounds__(256) void gemv_kernel_long(const uint8_t* __restrict__ payload,
                                                        const float2* __restrict__ meta,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ y, int N, int K,
                                                        int group) {
  constexpr int EPC = Codes<BITS>::kPerChunk;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int row_bytes = K / 8 * BITS;  // K is a multiple of the group
  const int nchunk = row_bytes / 16;
  const int groups = K / group;
  for (int rb = wave; rb * R < N; rb += nwaves) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    for (int c = lane; c < nchunk; c += 64) {
      float xv[EPC];
      const float4* x4 = reinterpret_cast<const float4*>(x + c * EPC);
      float xsum = 0.0f;
#pragma unroll
      for (int j = 0; j < EPC / 4; ++j) {
        const float4 v = x4[j];
        xv[4 * j] = v.x;
        xv[4 * j + 1] = v.y;
        xv[4 * j + 2] = v.z;
        xv[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) xsum += xv[e];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(rb * R + r, N - 1);
        const uint4 wv = ld_nt(reinterpret_cast<const uint4*>(payload + int64_t(row) * row_bytes) + c);
        const float2 mv = meta[int64_t(row) * groups + (c * EPC) / group];
        float f[EPC];
        Codes<BITS>::unpack(wv, f);
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) d = fmaf(xv[e], f[e], d);
        acc[r] = fmaf(mv.x, fmaf(-mv.y, xsum, d), acc[r]);
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

// Waves launched (grid-stride beyond): large INT8 matrices run fewer, longer
// waves, each staging x once and keeping its prefetch pipeline full for
// more row blocks (vocab projection: 87.8 against 90.6 us); small ones keep
// every row block's loads in flight at once.  INT4 does about twice the
// arithmetic per byte; with two rows per step (167 VGPRs) three waves fit a
// SIMD and hide it behind each other's loads (INT4 g64 vocab projection:
// 55.5-55.8 us, against 65-67 us with one wave of four rows per SIMD).
// The grid is sized from the device's compute units (at most 256, the size
// the top-1 key workspace is built for) and, for large matrices, from the
// number of 4-wave workgroups per CU the compiled kernel actually fits
// (`occ`, from its register and LDS use): a grid that asked for more would
// run its last workgroups as a second round.
template <int BITS>
int max_waves(int rowblocks, int occ) {
  const int cus = std::min(device_cus(), kMaxCus);
  const int small = cus * DSQ_GEMV_WAVES_PER_CU;
  const int want = BITS == 8 ? DSQ_GEMV_WAVES_PER_CU_LARGE : DSQ_GEMV_WAVES_PER_CU_LARGE4;
  const int large = cus * std::max(4, std::min(want, 4 * occ));
  return rowblocks >= 4 * small ? large : small;
}

// 4-wave workgroups of `kernel` resident per CU with `lds` bytes of LDS each.
template <class Kernel>
int occupancy(Kernel kernel, size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, lds) != hipSuccess || n <= 0)
    n = 1;
  return n;
}

template <int BITS, int R, int KCH>
hipError_t go(const QMat& q, const float* x, float* y, int N, int K, int group,
              uint64_t* wkey, int64_t* nkeys, hipStream_t stream) {
  // the largest x this instance stages (KCH chunks of 16 bytes per lane)
  constexpr size_t kLds = size_t(KCH) * 64 * Codes<BITS>::kPerChunk * 4;
  static const int occ_plain = occupancy(gemv_kernel<BITS, R, KCH>, kLds);
  static const int occ_key = occupancy(gemv_argmax_kernel<BITS, R, KCH>, kLds);
  const int rowblocks = (N + R - 1) / R;
  const int mw = max_waves<BITS>(rowblocks, wkey ? occ_key : occ_plain);
  const int waves = rowblocks < mw ? rowblocks : mw;
  const int blocks = (waves + 3) / 4;
  if (wkey) {
    hipLaunchKernelGGL((gemv_argmax_kernel<BITS, R, KCH>), dim3(blocks), dim3(256),
                       size_t(K) * 4, stream, q.payload, q.meta, x, y, N, K, group, wkey);
    *nkeys = int64_t(blocks) * 4;
  } else {
    hipLaunchKernelGGL((gemv_kernel<BITS, R, KCH>), dim3(blocks), dim3(256), size_t(K) * 4,
                       stream, q.payload, q.meta, x, y, N, K, group);
  }
  return hipGetLastError();
}

template <int BITS, int R>
hipError_t go_long(const QMat& q, const float* x, float* y, int N, int K, int group,
                   hipStream_t stream) {
  static const int occ = occupancy(gemv_kernel_long<BITS, R>, 0);
  const int rowblocks = (N + R - 1) / R;
  const int mw = max_waves<BITS>(rowblocks, occ);
  const int waves = rowblocks < mw ? rowblocks : mw;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((gemv_kernel_long<BITS, R>), dim3(blocks), dim3(256), 0, stream, q.payload,
                     q.meta, x, y, N, K, group);
  return hipGetLastError();
}

// wkey: also write every wave's best key there (rows of at most 4 chunks per
// lane only; the caller checks gemv_argmax_supported) and their count to nkeys
template <int BITS>
hipError_t dispatch(const QMat& q, const float* x, float* y, int N, int K, int group,
                    uint64_t* wkey, int64_t* nkeys, hipStream_t stream) {
  const int nchunk = K / 8 * BITS / 16;
  const int kch = (nchunk + 63) / 64;
  constexpr int R = BITS == 8 ? DSQ_GEMV_R8 : DSQ_GEMV_R4;
  switch (kch) {
    case 1: return go<BITS, R, 1>(q, x, y, N, K, group, wkey, nkeys, stream);
    case 2: return go<BITS, R, 2>(q, x, y, N, K, group, wkey, nkeys, stream);
    case 3: return go<BITS, R, 3>(q, x, y, N, K, group, wkey, nkeys, stream);
    case 4: return go<BITS, R, 4>(q, x, y, N, K, group, wkey, nkeys, stream);
    default:
      if (wkey) return hipErrorNotSupported;
      return go_long<BITS, 4>(q, x, y, N, K, group, stream);
  }
}

}  // namespace

hipError_t launch_gemv(const dsq_qweight& W, int64_t expert, const float* x, float* y,
                       hipStream_t stream) {
  if (W.group == kSuperGroup) return launch_gemv_sb4(W, expert, x, y, stream);
  const QMat q = entry(W, expert);
  const int N = int(W.N), K = int(W.K);
  if (W.bits == 8) return dispatch<8>(q, x, y, N, K, W.group, nullptr, nullptr, stream);
  return dispatch<4>(q, x, y, N, K, W.group, nullptr, nullptr, stream);
}

bool gemv_argmax_supported(const dsq_qweight& W) {
  return W.group != kSuperGroup && (W.K * W.bits / 8 / 16 + 63) / 64 <= 4;
}

size_t gemv_argmax_key_bytes() {
  const int most = kMaxCus * std::max(DSQ_GEMV_WAVES_PER_CU,
                                  std::max(DSQ_GEMV_WAVES_PER_CU_LARGE,
                                           DSQ_GEMV_WAVES_PER_CU_LARGE4));
  return size_t(align256(int64_t(most + 3) * 8));
}

hipError_t launch_gemv_argmax(const dsq_qweight& W, int64_t expert, const float* x, float* y,
                              uint64_t* wkey, int64_t* nkeys, hipStream_t stream) {
  if (!gemv_argmax_supported(W)) return hipErrorNotSupported;
  const QMat q = entry(W, expert);
  const int N = int(W.N), K = int(W.K);
  if (W.bits == 8) return dispatch<8>(q, x, y, N, K, W.group, wkey, nkeys, stream);
  return dispatch<4>(q, x, y, N, K, W.group, wkey, nkeys, stream);
}

}  // namespace dsq
