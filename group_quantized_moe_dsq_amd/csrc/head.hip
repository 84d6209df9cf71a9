// head.hip -- output-head selection: the k largest of N logits.
//
// The last projection's logits choose the next token ("Hand-writing a
// DeepSeek inference engine in pure C", hnwysp.cn/news/134870, §2.1; "ds4
// code walkthrough", the session API's argmax / sample step), and the
// end-to-end check compares the argmax at every position ("Running a
// 284B-parameter LLM from 3.2 GB of RAM in plain C").  Rank order: larger
// value first, equal values (-0 equals +0) to the smaller index, NaN below
// every number.
//
// Every value becomes one 64-bit key that orders exactly like that rule:
//   high word: the float's bits mapped to an unsigned integer of the same
//              order (negative values complemented, positive ones with the
//              top bit set), both zeros mapped alike, NaN mapped to 0;
//   low word : the complemented index, so the smaller index ranks higher.
// Keys are distinct, and 0 (the padding) ranks below every real value.
//
// Selection by rounds: a workgroup keeps the best k keys of its chunk; the
// kept keys are the next round's input, until one chunk remains, whose best
// k are the answer (the top k of all values lie among every chunk's top k).
// For small k a workgroup takes the block maximum of a 4096-key chunk k times
// (the pick is removed by the one lane that holds it); for larger k it sorts
// a 1024-key chunk with a bitonic network held in registers.
#include "common.h"
#include "internal.h"
#include "head_key.h"
#include "mfma_util.h"

namespace dsq {

constexpr int kHeadChunk = 1024;      // bitonic path (k > kHeadPickMaxK)
constexpr int kHeadSortThreads = kHeadChunk / 2;  // one pair per thread and step
constexpr int kHeadThreads = 256;     // pick path
constexpr int kHeadWaves = kHeadThreads / 64;
#ifndef DSQ_HEAD_PICK_MAXK
#define DSQ_HEAD_PICK_MAXK 6  // picks cost ~1.1 us each; the sort path ~13.5 us up to k = 8
#endif
constexpr int kHeadPickMaxK = DSQ_HEAD_PICK_MAXK;
constexpr int kHeadPickPer = 16;      // keys per thread, pick path
constexpr int kHeadPickChunk = kHeadThreads * kHeadPickPer;

// Write the r-th best key of a round: FINAL as (index, value), else as a key
// of the next round's input.
template <bool FINAL>
__device__ __forceinline__ void head_emit(uint64_t key, int r, const float* __restrict__ y,
                                          uint64_t* __restrict__ out, int32_t* __restrict__ idx,
                                          float* __restrict__ val, int k) {
  if (FINAL) {
    const uint32_t i = ~uint32_t(key);
    idx[r] = int32_t(i);
    val[r] = y[i];
  } else {
    out[int64_t(blockIdx.x) * k + r] = key;
  }
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const int lo = __shfl_xor(int(uint32_t(v)), m), hi = __shfl_xor(int(uint32_t(v >> 32)), m);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = int(uint32_t(v)), hi = int(uint32_t(v >> 32));
  const uint32_t a = uint32_t(__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xf, 0xf, false));
  const uint32_t b = uint32_t(__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xf, 0xf, false));
  return (uint64_t(b) << 32) | a;
}

// The key of lane (lane ^ m).  Inside a 16-lane row the data-parallel
// primitives do it without the LDS crossbar: xor 1 and 2 are quad permutes,
// xor 8 the row rotation by 8, xor 4 the row shifts by 4 (lanes with bit 2
// clear read lane + 4, the others lane - 4); xor 16 and 32 go through
// ds_bpermute.  m is a constant after unrolling, so one branch remains.
__device__ __forceinline__ uint64_t xchg64(uint64_t v, int m, int lane) {
  if (m == 1) return dpp64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if (m == 2) return dpp64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if (m == 8) return dpp64<0x128>(v);  // row_ror:8
  if (m == 4) {
    const uint64_t up = dpp64<0x104>(v);  // row_shl:4 -> lane + 4
    const uint64_t dn = dpp64<0x114>(v);  // row_shr:4 -> lane - 4
    return (lane & 4) ? dn : up;
  }
  return shfl_xor64(v, m);
}

// One round, bitonic path.  FROM_Y: the input is the logits (keys are formed
// here), else the previous round's keys.  FINAL (one workgroup): write the k
// best as (index, value); else write them as keys to out[block][k].
//
// The chunk's 1024 keys stay in registers, thread t holding positions 2t and
// 2t + 1 (a wave owns 128 consecutive positions).  Every step of the network
// (blocks of `size` sorted in alternating direction, the last one descending)
// pairs position p with p ^ stride: stride 1 is inside a thread, strides 2 ..
// 64 pair lanes of one wave (a lane exchange, xchg64), and only strides 128 .. 512
// (6 of the 55 steps) go through LDS, each with one barrier (two LDS buffers
// alternate, so a step's writes never meet the previous step's reads).  Both
// members of a pair compute their new key from the same two keys: the lower
// position keeps the larger one in a descending block, the smaller one in an
// ascending block.
template <bool FROM_Y, bool FINAL>
__global__ __launch_bounds__(kHeadSortThreads) void head_round_kernel(const float* __restrict__ y,
                                                                      const uint64_t* __restrict__ in,
                                                                      int64_t n, int k,
                                                                      uint64_t* __restrict__ out,
                                                                      int32_t* __restrict__ idx,
                                                                      float* __restrict__ val) {
  __shared__ uint64_t s[2][kHeadChunk];
  const int t = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * kHeadChunk;
  uint64_t v[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t i = base + 2 * t + b;
    uint64_t key = 0;
    if (i < n) key = FROM_Y ? head_key(y[i], uint32_t(i)) : in[i];
    v[b] = key;
  }
  int buf = 0;
#pragma unroll
  for (int size = 2; size <= kHeadChunk; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t o[2];
      if (stride == 1) {
        o[0] = v[1];
        o[1] = v[0];
      } else if (stride <= 64) {
#pragma unroll
        for (int b = 0; b < 2; ++b) o[b] = xchg64(v[b], stride >> 1, t & 63);
      } else {
        s[buf][2 * t] = v[0];
        s[buf][2 * t + 1] = v[1];
        lds_barrier();
#pragma unroll
        for (int b = 0; b < 2; ++b) o[b] = s[buf][(2 * t + b) ^ stride];
        buf ^= 1;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int pos = 2 * t + b;
        const bool lower = (pos & stride) == 0, desc = (pos & size) == 0;
        v[b] = lower == desc ? umax64(v[b], o[b]) : umin64(v[b], o[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int r = 2 * t + b;
    if (r < k) head_emit<FINAL>(v[b], r, y, out, idx, val, k);
  }
}

// One round, pick path: k times the block maximum of the workgroup's chunk.
// Each thread holds kHeadPickPer keys (strided by the block size, so a wave's
// loads are contiguous) and keeps their maximum; a pick is the wave maxima's
// maximum, and the one thread that holds it clears that key and recomputes
// its maximum.  The wave maxima alternate between two LDS slots, so one
// barrier per pick suffices: a wave writes slot r & 1 again only after every
// wave has passed the barrier of pick r + 1, which it reaches after reading
// the slot for pick r.  The picks are kept in LDS and written after the loop.
template <bool FROM_Y, bool FINAL>
__global__ __launch_bounds__(kHeadThreads) void head_pick_kernel(const float* __restrict__ y,
                                                                 const uint64_t* __restrict__ in,
                                                                 int64_t n, int k,
                                                                 uint64_t* __restrict__ out,
                                                                 int32_t* __restrict__ idx,
                                                                 float* __restrict__ val) {
  __shared__ uint64_t wmax[2][kHeadWaves];
  __shared__ uint64_t picked[kHeadPickMaxK > 0 ? kHeadPickMaxK : 1];
  const int64_t base = int64_t(blockIdx.x) * kHeadPickChunk;
  uint64_t v[kHeadPickPer];
#pragma unroll
  for (int q = 0; q < kHeadPickPer; ++q) {
    const int64_t i = base + threadIdx.x + int64_t(q) * kHeadThreads;
    uint64_t key = 0;
    if (i < n) key = FROM_Y ? head_key(y[i], uint32_t(i)) : in[i];
    v[q] = key;
  }
  uint64_t lm = v[0];
#pragma unroll
  for (int q = 1; q < kHeadPickPer; ++q) lm = umax64(lm, v[q]);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int r = 0; r < k; ++r) {
    const uint64_t b = wave_max_key(lm);
    if (lane == 0) wmax[r & 1][wv] = b;
    lds_barrier();
    uint64_t m = wmax[r & 1][0];
#pragma unroll
    for (int w = 1; w < kHeadWaves; ++w) m = umax64(m, wmax[r & 1][w]);
    // real keys are distinct, so one thread owns m (when only padding is
    // left m is 0, and clearing zeros changes nothing)
    if (lm == m) {
      uint64_t nm = 0;
#pragma unroll
      for (int q = 0; q < kHeadPickPer; ++q) {
        v[q] = v[q] == m ? 0 : v[q];
        nm = umax64(nm, v[q]);
      }
      lm = nm;
    }
    if (threadIdx.x == 0) picked[r] = m;
  }
  lds_barrier();
  for (int r = threadIdx.x; r < k; r += kHeadThreads) head_emit<FINAL>(picked[r], r, y, out, idx, val, k);
}

namespace {

int64_t chunk_of(int32_t k) { return k <= kHeadPickMaxK ? kHeadPickChunk : kHeadChunk; }
int64_t chunks(int64_t n, int32_t k) { return (n + chunk_of(k) - 1) / chunk_of(k); }

template <bool FROM_Y, bool FINAL>
void launch_round(int64_t nb, const float* y, const uint64_t* in, int64_t n, int32_t k,
                  uint64_t* out, int32_t* idx, float* val, hipStream_t stream) {
  if (k <= kHeadPickMaxK)
    hipLaunchKernelGGL((head_pick_kernel<FROM_Y, FINAL>), dim3(unsigned(nb)), dim3(kHeadThreads),
                       0, stream, y, in, n, k, out, idx, val);
  else
    hipLaunchKernelGGL((head_round_kernel<FROM_Y, FINAL>), dim3(unsigned(nb)),
                       dim3(kHeadSortThreads), 0, stream, y, in, n, k, out, idx, val);
}

}  // namespace

size_t head_workspace(int64_t N, int32_t k) {
  // two ping-pong key buffers, each large enough for the first round's output
  // (none when one chunk holds N: 256, nonzero means supported); for k = 1 at
  // least the GEMV's per-wave keys
  size_t b = chunks(N, k) == 1 ? 256 : size_t(2) * align256(chunks(N, k) * k * 8);
  if (k == 1 && b < gemv_argmax_key_bytes()) b = gemv_argmax_key_bytes();
  return b;
}

hipError_t launch_head_from_keys(const float* y, const uint64_t* keys, int64_t n, int32_t* idx,
                                 float* val, hipStream_t stream) {
  if (n < 1 || n > kHeadPickChunk || kHeadPickMaxK < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((head_pick_kernel<false, true>), dim3(1), dim3(kHeadThreads), 0, stream, y,
                     keys, n, 1, nullptr, idx, val);
  return hipGetLastError();
}

hipError_t launch_head(const float* y, int64_t N, int32_t k, int32_t* idx, float* val,
                       void* workspace, hipStream_t stream) {
  const int64_t half = chunks(N, k) == 1 ? 0 : align256(chunks(N, k) * k * 8);
  uint64_t* buf[2] = {static_cast<uint64_t*>(workspace),
                      reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) + half)};
  int64_t n = N;
  int round = 0;
  while (true) {
    const int64_t nb = chunks(n, k);
    const uint64_t* in = round == 0 ? nullptr : buf[(round - 1) & 1];
    if (nb == 1) {
      if (round == 0) launch_round<true, true>(1, y, in, n, k, nullptr, idx, val, stream);
      else launch_round<false, true>(1, y, in, n, k, nullptr, idx, val, stream);
      return hipGetLastError();
    }
    uint64_t* out = buf[round & 1];
    if (round == 0) launch_round<true, false>(nb, y, in, n, k, out, nullptr, nullptr, stream);
    else launch_round<false, false>(nb, y, in, n, k, out, nullptr, nullptr, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    n = nb * k;
    ++round;
  }
}

}  // namespace dsq
