// route.hip -- the routing steps of the MoE layer: router logits (fp32
// weights, few token rows), softmax + top-k + renormalisation, stable
// grouping of the routed entries by expert, and the weighted combine.
//
// Method: "Hand-writing a DeepSeek inference engine in pure C"
// (hnwysp.cn/news/134870) §3.4 (softmax with the maximum subtracted), §3.5
// (router = a linear layer, top-k by a greater-first sort of (score, index)
// pairs, tokens gathered per expert, weighted sum of the expert outputs).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace dsq {

// ---------------------------------------------------------------------------
// Router logits for many tokens: logits[t][e] = X[t] . Wr[e] (+ bias[e]),
// fp32 weights.  A workgroup of 4 waves owns 4*R experts and loops over the
// tokens in tiles of MT.  K is walked in rounds of 1024: the round's
// activations of the MT tokens are staged in LDS, each lane loads 16
// consecutive weights of each of its rows once and reuses them for all MT
// tokens; partial sums are reduced across the wave in one reduce-scatter.
// (Few tokens take the router GEMV of decode.hip instead.)
// ---------------------------------------------------------------------------
struct RouterArgs {
  const float* W;   // [E][K]
  int N, K;         // N = E
  const float* X;   // [M][K]
  int64_t M;
  float* out;       // [M][N]; with ks > 1: [ks][M][N] partial sums, no bias
  const float* bias;
  int ks;           // K slices (grid y)
};

constexpr int kRound = 1024;  // K per LDS round: 64 lanes x 16

template <int R, int MT>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs p) {
  constexpr int NV = R * MT;  // outputs per wave per token tile
  __shared__ float4 xs[MT][kRound / 4];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wv) * R;
  const int nrounds = (p.K + kRound - 1) / kRound;

  for (int64_t m0 = int64_t(blockIdx.y) * MT; m0 < p.M; m0 += int64_t(gridDim.y) * MT) {
    const int mt = int(p.M - m0 < MT ? p.M - m0 : MT);
    float acc[R][MT];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[j][m] = 0.0f;

    for (int rd = 0; rd < nrounds; ++rd) {
      __syncthreads();  // previous round fully consumed
      // stage x[m][rd*1024 .. +1024) with the chunk swizzle described below
      for (int idx = threadIdx.x; idx < MT * (kRound / 4); idx += 256) {
        const int m = idx / (kRound / 4);
        const int k4 = idx % (kRound / 4);
        const int k = rd * kRound + k4 * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m < mt && k < p.K) v = *reinterpret_cast<const float4*>(p.X + (m0 + m) * p.K + k);
        // lane l's 16 values are float4 slots 4l..4l+3; rotating them by
        // (l >> 2) spreads 16 lanes' reads over distinct LDS banks
        const int l = k4 >> 2, j = k4 & 3;
        xs[m][l * 4 + ((j + (l >> 2)) & 3)] = v;
      }
      __syncthreads();
      const int chunk = rd * 64 + lane;
      if (chunk * 16 >= p.K) continue;  // this lane has no weights this round
      float wf[R][16];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = min(n0 + r, p.N - 1);
        const float4* q = reinterpret_cast<const float4*>(p.W + int64_t(n) * p.K) + chunk * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 v = q[j];
          wf[r][4 * j] = v.x;
          wf[r][4 * j + 1] = v.y;
          wf[r][4 * j + 2] = v.z;
          wf[r][4 * j + 3] = v.w;
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= mt) break;
        float xv[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 v = xs[m][lane * 4 + ((j + (lane >> 2)) & 3)];
          xv[4 * j] = v.x;
          xv[4 * j + 1] = v.y;
          xv[4 * j + 2] = v.z;
          xv[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
          float d = acc[j][m];
#pragma unroll
          for (int q = 0; q < 16; ++q) d = fmaf(xv[q], wf[j][q], d);
          acc[j][m] = d;
        }
      }
    }

    // reduce and store: value index v = r * MT + m
    float va[NV];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) va[r * MT + m] = acc[r][m];
    const float ta = wave_reduce_scatter<NV>(va);
    if ((lane & (64 / NV - 1)) == 0) {
      const int v = reduce_scatter_row<NV>(lane);
      const int r = v / MT, m = v % MT;
      const int n = n0 + r;
      if (m < mt && n < p.N) {
        float o = ta;
        if (p.bias) o += p.bias[n];
        p.out[(m0 + m) * p.N + n] = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same logits on the fp32 matrix cores (v_mfma_f32_16x16x4_f32, fp32
// products and sums).  A workgroup of NW waves owns a tile of 16 tokens x 16
// experts; wave w takes the part w of K.  Within a wave, the K range is
// walked in chunks of 16: lane group g (16 lanes) holds elements 4g .. 4g+3 of
// a chunk and MFMA u of the chunk takes element 4g + u from group g, for A
// (tokens) and B (experts) alike; the four groups of a row read 64 contiguous
// bytes per instruction.  Lane l supplies
// A[token l%16] and B[expert l%16]; its 4 results are tokens 4(l/16) .. +3 of
// expert l%16.  The waves' partial tiles meet in LDS in a fixed order.
// Requires K % (256 NW) == 0.  With few tiles, K is also split over ks
// workgroups (grid y, slice s takes K range s of ks); each writes its partial
// tile, and the top-k kernel adds the slices in order and the bias.
// ---------------------------------------------------------------------------
typedef float f32x4v __attribute__((ext_vector_type(4)));

#ifndef DSQ_ROUTER_NW
#define DSQ_ROUTER_NW 4  // waves per workgroup = ways K is split
#endif
constexpr int kRouterNW = DSQ_ROUTER_NW;

__global__ __launch_bounds__(64 * kRouterNW) void router_mfma_kernel(RouterArgs p) {
  __shared__ f32x4v part[kRouterNW][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  // tile of this workgroup; workgroup b runs on XCD b % 8: when the tile grid
  // splits evenly, XCD x takes one block of (tiles_t / 2) x (tiles_e / 4)
  // tiles, so its L2 sees a quarter of the weights and half of the tokens
  const int tiles_e = (p.N + 15) / 16;
  const int tiles_t = int((p.M + 15) / 16);
  const int blk = blockIdx.x;
  int te, tt;
  if (tiles_t % 2 == 0 && tiles_e % 4 == 0) {
    const int x = blk % 8, i = blk / 8;
    const int bw = tiles_e / 4;  // block width in expert tiles
    te = (x % 4) * bw + i % bw;
    tt = (x / 4) * (tiles_t / 2) + i / bw;
  } else {
    te = blk % tiles_e;
    tt = blk / tiles_e;
  }
  const int e0 = te * 16;
  const int64_t t0 = int64_t(tt) * 16;
  const int K = p.K, KQ = K / (kRouterNW * p.ks);  // K range per wave
  const int k0 = blockIdx.y * (K / p.ks) + wv * KQ;
  const int64_t tr = t0 + r16 < p.M ? t0 + r16 : p.M - 1;  // clamped rows: loads stay in range
  const int er = e0 + r16 < p.N ? e0 + r16 : p.N - 1;
  // lane group g holds elements 4g .. 4g+3 of every 16-element chunk of the
  // wave's K range: the four groups of a row read one contiguous 64 bytes
  const float4* xa = reinterpret_cast<const float4*>(p.X + tr * K + k0) + g;
  const float4* wb = reinterpret_cast<const float4*>(p.W + int64_t(er) * K + k0) + g;
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
  // chunks of 4 float4 per operand (16 MFMAs); four register stages, loads
  // three chunks ahead.  Chunk indices past the end are clamped, so every
  // load is unconditional and the compiler's waits stay static; the
  // multiply-adds of chunks past the end are skipped (uniform branches).
  const int nch = KQ / 64;  // chunks of 64 k (>= 1: K % (64 NW ks) == 0)
  float4 a[4][4], b[4][4];
  auto load = [&](float4 (&av)[4], float4 (&bv)[4], int c) {
    if (nch < 4 && c >= nch) return;  // short ranges: no loads past the end
    const int cc = c < nch ? c : nch - 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = xa[(cc * 4 + u) * 4];
      bv[u] = wb[(cc * 4 + u) * 4];
    }
  };
  auto mma = [&](const float4 (&av)[4], const float4 (&bv)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].x, bv[u].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].y, bv[u].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].z, bv[u].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].w, bv[u].w, acc, 0, 0, 0);
    }
  };
  // (the scheduling barriers keep each stage's loads where they are issued:
  // left alone, the scheduler sinks every load to just before its use)
  load(a[0], b[0], 0);
  load(a[1], b[1], 1);
  load(a[2], b[2], 2);
  for (int c = 0; c < nch; c += 4) {
    load(a[3], b[3], c + 3);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[0], b[0]);
    __builtin_amdgcn_sched_barrier(0);
    load(a[0], b[0], c + 4);
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < nch) mma(a[1], b[1]);
    __builtin_amdgcn_sched_barrier(0);
    load(a[1], b[1], c + 5);
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 < nch) mma(a[2], b[2]);
    __builtin_amdgcn_sched_barrier(0);
    load(a[2], b[2], c + 6);
    __builtin_amdgcn_sched_barrier(0);
    if (c + 3 < nch) mma(a[3], b[3]);
    __builtin_amdgcn_sched_barrier(0);
  }
  part[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    f32x4v v = part[0][lane];
#pragma unroll
    for (int w = 1; w < kRouterNW; ++w) v += part[w][lane];
    const int e = e0 + r16;
    if (e < p.N) {
      const bool add_bias = p.bias && p.ks == 1;
      const float b = add_bias ? p.bias[e] : 0.0f;
      float* out = p.out + int64_t(blockIdx.y) * p.M * p.N;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t t = t0 + 4 * g + q;
        if (t < p.M) out[t * p.N + e] = add_bias ? v[q] + b : v[q];
      }
    }
  }
}

#ifndef DSQ_ROUTER_R
#define DSQ_ROUTER_R 2   // experts per wave
#endif
#ifndef DSQ_ROUTER_MT
#define DSQ_ROUTER_MT 8  // tokens per tile
#endif

int router_slices(int64_t T, int32_t E, int64_t H) {
  const int64_t tiles = ((E + 15) / 16) * ((T + 15) / 16);
  if (H % (256 * kRouterNW) != 0 || tiles > int64_t(INT32_MAX)) return 0;
  int ks = 1;
  while (2 * ks <= kRouterMaxSlices && tiles * 2 * ks <= 256 && H % (64 * kRouterNW * 2 * ks) == 0)
    ks *= 2;
  return ks;
}

hipError_t launch_router(const float* X, int64_t T, const float* Wr, const float* bias,
                         int32_t E, int64_t H, float* logits, int ks, hipStream_t stream) {
  if (ks >= 1) {
    if (ks > router_slices(T, E, H)) return hipErrorInvalidValue;
    RouterArgs a{};
    a.W = Wr;
    a.N = E;
    a.K = int(H);
    a.X = X;
    a.M = T;
    a.out = logits;
    a.bias = bias;
    a.ks = ks;
    if (T == 0 || E == 0) return hipSuccess;
    hipLaunchKernelGGL(router_mfma_kernel, dim3(unsigned(((E + 15) / 16) * ((T + 15) / 16)),
                                                unsigned(ks)),
                       dim3(64 * kRouterNW), 0, stream, a);
    return hipGetLastError();
  }
  constexpr int R = DSQ_ROUTER_R, MT = DSQ_ROUTER_MT;
  RouterArgs a{};
  a.W = Wr;
  a.N = E;
  a.K = int(H);
  a.X = X;
  a.M = T;
  a.out = logits;
  a.bias = bias;
  const int rowblocks = (E + 4 * R - 1) / (4 * R);
  const int64_t tiles = (T + MT - 1) / MT;
  const int gy = int(tiles < 65535 ? tiles : 65535);
  if (rowblocks == 0 || gy == 0) return hipSuccess;
  hipLaunchKernelGGL((router_kernel<R, MT>), dim3(rowblocks, gy), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Softmax + top-k + renormalisation ("Hand-writing a DeepSeek inference
// engine in pure C" §3.4: subtract the maximum; §3.5: top-k by a greater-first
// sort of (score, index) pairs).  One wave per token; each lane holds EPL
// scores.  k rounds of a wave-wide DPP argmax with the comparator
// (score desc, index desc); lane i keeps the i-th winner.  The renormalised
// weight of a selected expert is exp(s_i - s_max) / sum_sel exp(s_j - s_max):
// the full softmax denominator cancels in p_i / sum_sel p_j.
// With nparts > 1 the input is the router's K slices [nparts][T][E]: they are
// added in slice order, then the router bias rbias, and the sums are written
// to lout (the layer's logits) before the selection.
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int nparts,
                                                   const float* __restrict__ rbias,
                                                   float* __restrict__ lout,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (t >= T) return;
  float v[EPL];
  uint64_t taken = 0;
  // all loads first (clamped addresses, no branches), then the fix-ups
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = logits[int64_t(t) * E + min(lane + 64 * j, E - 1)];
  if (nparts > 1) {
    // every slice's and the bias's loads in flight before the first add (up
    // to eight slices; more take further rounds); slices added in order
    const int64_t ps = int64_t(T) * E;
    float u[7][EPL], rb[EPL];
#pragma unroll
    for (int q = 0; q < 7; ++q)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        u[q][j] = logits[min(1 + q, nparts - 1) * ps + int64_t(t) * E + min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < EPL; ++j) rb[j] = rbias ? rbias[min(lane + 64 * j, E - 1)] : 0.0f;
#pragma unroll
    for (int q = 0; q < 7; ++q) {
      if (1 + q >= nparts) break;
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[j] += u[q][j];
    }
    for (int q = 8; q < nparts; ++q) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[j] += logits[q * ps + int64_t(t) * E + min(lane + 64 * j, E - 1)];
    }
    if (rbias) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[j] += rb[j];
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j < E) lout[int64_t(t) * E + lane + 64 * j] = v[j];
  }
  if (bias) {
    float b[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) b[j] = bias[min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] += b[j];
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    if (v[j] != v[j]) v[j] = -INFINITY;  // NaN ranks last
    if (lane + 64 * j >= E) taken |= uint64_t(1) << j;  // padding never wins
  }
  float my_val = 0.0f;
  int my_idx = 0;
  float best_val = 0.0f;
  for (int i = 0; i < k; ++i) {
    // local best among not-taken
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (!((taken >> j) & 1) && (bi < 0 || ranks_before(v[j], e, bv, bi))) {
        bv = v[j];
        bi = e;
      }
    }
    wave_argmax(bv, bi);  // DPP reduction; uniform across the wave
    if (bi >= 0 && (bi & 63) == lane) taken |= uint64_t(1) << (bi >> 6);
    if (i == 0) best_val = bv;
    if (lane == i) {
      my_val = bv;
      my_idx = bi;
    }
  }
  const float ex = lane < k ? expf(my_val - best_val) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    idx[int64_t(t) * k + lane] = my_idx;
    wout[int64_t(t) * k + lane] = ex / sum;
  }
}

namespace {

hipError_t topk_any(const float* logits, int nparts, const float* rbias, float* lout,
                    const float* bias, int64_t T, int32_t E, int32_t k, int32_t* idx, float* w,
                    hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = (T + 3) / 4;
  const int epl = (E + 63) / 64;
#define DSQ_TOPK(n)                                                                          \
  hipLaunchKernelGGL(topk_kernel<n>, dim3(unsigned(blocks)), dim3(256), 0, stream, logits,   \
                     nparts, rbias, lout, bias, int(T), E, k, idx, w)
  if (epl <= 1) DSQ_TOPK(1);
  else if (epl <= 2) DSQ_TOPK(2);
  else if (epl <= 4) DSQ_TOPK(4);
  else if (epl <= 8) DSQ_TOPK(8);
  else if (epl <= 16) DSQ_TOPK(16);
  else if (epl <= 32) DSQ_TOPK(32);
  else DSQ_TOPK(64);
#undef DSQ_TOPK
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                       int32_t* idx, float* w, hipStream_t stream) {
  return topk_any(logits, 1, nullptr, nullptr, bias, T, E, k, idx, w, stream);
}

hipError_t launch_topk_parts(const float* parts, int nparts, const float* rbias, float* logits,
                             int64_t T, int32_t E, int32_t k, int32_t* idx, float* w,
                             hipStream_t stream) {
  if (nparts < 2 || !logits) return hipErrorInvalidValue;
  return topk_any(parts, nparts, rbias, logits, nullptr, T, E, k, idx, w, stream);
}

// ---------------------------------------------------------------------------
// Grouping by expert (§3.5 of the same page: gather the tokens routed to one
// expert).  A token selects distinct experts, so an entry's rank inside its
// expert's segment is the number of earlier tokens that selected the same
// expert.  A bitmap with bit t of expert e's row set when token t chose e
// turns that into popcounts.  Integer only, so the result is exact and stable
// (ascending token order within an expert).  Entries whose expert lies
// outside [0, E) are not grouped (pos = -1).
// With `tiles`, the same pass lists the grouped GEMM's token tiles: expert
// segments cut into tiles of tpt rows, one record per tile in (active expert,
// tile) order, written by the entry that opens the tile.
// Up to kGroupSmallT tokens one workgroup does everything (the rank of an
// entry popcounts at most 8 words); beyond that three kernels keep every
// entry's rank O(1): per 32-token word the bitmap words of all experts, per
// expert the exclusive prefix of the words' popcounts, then one thread per
// entry.
// ---------------------------------------------------------------------------
constexpr int kGroupSmallT = 256;
constexpr int kGroupMaxE = 4096;

// Wave 0 scans the per-expert counts held in s_off[0..E): on return s_off[e]
// is expert e's first position (s_off[E] the total), s_act[e] its rank among
// the experts with entries and s_tile[e] its first token tile (tiles of ntpt
// rows).  With `out`, the offsets, active list and their totals (and the
// counts, when `counts` is not NULL) are written to memory as well.  The
// caller synchronises before and after.
__device__ void group_scan_experts(int E, int ntpt, int32_t* s_off, int32_t* s_act,
                                   int32_t* s_tile, bool out, int32_t* counts, int32_t* offsets,
                                   int32_t* active, int32_t* n_active, int32_t* n_tiles) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int per = (E + 63) / 64;
  const int lo = min(lane * per, E);
  const int hi = min(lo + per, E);
  int sc = 0, sa = 0, st = 0;
  for (int e = lo; e < hi; ++e) {
    sc += s_off[e];
    sa += s_off[e] > 0;
    st += (s_off[e] + ntpt - 1) / ntpt;
  }
  int ic = sc, ia = sa, it = st;  // inclusive scan across lanes
  for (int o = 1; o < 64; o <<= 1) {
    const int uc = __shfl_up(ic, o);
    const int ua = __shfl_up(ia, o);
    const int ut = __shfl_up(it, o);
    if (lane >= o) {
      ic += uc;
      ia += ua;
      it += ut;
    }
  }
  int rc = ic - sc, ra = ia - sa, rt = it - st;
  for (int e = lo; e < hi; ++e) {
    const int c = s_off[e];
    s_off[e] = rc;
    s_act[e] = ra;
    s_tile[e] = rt;
    if (out) {
      if (counts) counts[e] = c;
      offsets[e] = rc;
      if (c > 0) active[ra] = e;
    }
    rc += c;
    ra += c > 0;
    rt += (c + ntpt - 1) / ntpt;
  }
  if (lane == 63) {
    s_off[E] = ic;
    if (out) {
      offsets[E] = ic;
      *n_active = ia;
      if (n_tiles) *n_tiles = it;
    }
  }
}

// Places entry j = t * k + i of expert e at rank `rank` of its segment, and
// writes the token-tile record when the entry opens a tile.
__device__ __forceinline__ void group_place(int j, int e, int rank, const int32_t* s_off,
                                            const int32_t* s_act, const int32_t* s_tile,
                                            int tpt, int32_t* perm, int32_t* pos, int4* tiles) {
  const int p = s_off[e] + rank;
  perm[p] = j;
  pos[j] = p;
  // the activation tile index is the one the grouped GEMM's prep assigns
  // (segment start / tpt + active rank + tile)
  if (tiles && rank % tpt == 0) {
    const int c = s_off[e + 1] - s_off[e];
    const int t = rank / tpt;
    tiles[s_tile[e] + t] = make_int4(e, p, min(tpt, c - rank), s_off[e] / tpt + s_act[e] + t);
  }
}

// Few tokens: one workgroup; bitmap [E][ceil(T/32)], built with atomics, in
// LDS when it fits beside the tables (LBM; no memory round trips but the
// routing's load and the outputs' stores), else in the scratch memory.
constexpr int kGroupLdsWords = 3072;  // E * ceil(T/32): 256 experts x 256 tokens is 2048
template <bool LBM>
__global__ __launch_bounds__(1024) void group_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                     int E, uint32_t* __restrict__ bm,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ active,
                                                     int32_t* __restrict__ n_active, int tpt,
                                                     int4* __restrict__ tiles,
                                                     int32_t* __restrict__ n_tiles) {
  __shared__ int32_t s_off[kGroupMaxE + 1];
  __shared__ int32_t s_act[kGroupMaxE + 1];
  __shared__ int32_t s_tile[kGroupMaxE + 1];
  __shared__ uint32_t s_bm[LBM ? kGroupLdsWords : 1];
  // a bitmap in memory is built with device-scope atomics: read it past L1
  typedef typename std::conditional<LBM, uint32_t, volatile uint32_t>::type word_t;
  word_t* const B = LBM ? s_bm : bm;
  const int W = (T + 31) / 32;
  const int nent = T * k;
  for (int i = threadIdx.x; i < E * W; i += blockDim.x) B[i] = 0u;
  __syncthreads();
  for (int j = threadIdx.x; j < nent; j += blockDim.x) {
    const int e = idx[j];
    const int t = j / k;
    if (unsigned(e) < unsigned(E))
      atomicOr(const_cast<uint32_t*>(&B[e * W + (t >> 5)]), 1u << (t & 31));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
    const word_t* row = B + e * W;
    for (int w = 0; w < W; ++w) c += __popc(row[w]);
    s_off[e] = c;
  }
  __syncthreads();
  group_scan_experts(E, tiles ? tpt : 1, s_off, s_act, s_tile, true, counts, offsets, active,
                     n_active, tiles ? n_tiles : nullptr);
  __syncthreads();
  for (int j = threadIdx.x; j < nent; j += blockDim.x) {
    const int e = idx[j];
    if (unsigned(e) >= unsigned(E)) {
      pos[j] = -1;
      continue;
    }
    const int t = j / k;
    const word_t* row = B + e * W;
    int rank = 0;
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(row[w]);
    rank += __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
    group_place(j, e, rank, s_off, s_act, s_tile, tpt, perm, pos, tiles);
  }
}

// Many tokens, step 1: one workgroup per 32-token word w writes the bitmap
// words bm[w][e] of every expert (LDS atomics, then plain stores: no
// clearing pass, every word is written once).
__global__ __launch_bounds__(256) void group_bits_kernel(const int32_t* __restrict__ idx, int T,
                                                         int k, int E,
                                                         uint32_t* __restrict__ bm) {
  __shared__ uint32_t bits[kGroupMaxE];
  const int w = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) bits[e] = 0u;
  __syncthreads();
  const int j0 = w * 32 * k, j1 = min(T, (w + 1) * 32) * k;
  for (int j = j0 + threadIdx.x; j < j1; j += blockDim.x) {
    const int e = idx[j];
    if (unsigned(e) < unsigned(E)) atomicOr(&bits[e], 1u << ((j / k) & 31));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) bm[int64_t(w) * E + e] = bits[e];
}

// Step 2: per expert, the exclusive prefix over the words of their
// popcounts, pre[w][e], and the expert's count.  A workgroup owns 64 experts
// (one per lane); its 16 waves split the words into 16 consecutive ranges.
constexpr int kGroupPrefixWaves = 16;
__global__ __launch_bounds__(1024) void group_prefix_kernel(const uint32_t* __restrict__ bm,
                                                            int W, int E,
                                                            int32_t* __restrict__ pre,
                                                            int32_t* __restrict__ counts) {
  __shared__ int32_t part[kGroupPrefixWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int cw = (W + kGroupPrefixWaves - 1) / kGroupPrefixWaves;
  const int w0 = min(wv * cw, W), w1 = min(w0 + cw, W);
  int s = 0;
  if (e < E)
    for (int w = w0; w < w1; ++w) s += __popc(bm[int64_t(w) * E + e]);
  part[wv][lane] = s;
  __syncthreads();
  int run = 0, tot = 0;
  for (int v = 0; v < kGroupPrefixWaves; ++v) {
    const int c = part[v][lane];
    if (v < wv) run += c;
    tot += c;
  }
  if (e >= E) return;
  if (wv == 0) counts[e] = tot;
  for (int w = w0; w < w1; ++w) {
    pre[int64_t(w) * E + e] = run;
    run += __popc(bm[int64_t(w) * E + e]);
  }
}

// Step 3: every workgroup scans the expert counts itself (workgroup 0 also
// writes offsets, active list and totals), then one thread per entry ranks
// it in O(1): pre[w][e] + the popcount of the earlier tokens of its word.
__global__ __launch_bounds__(256) void group_rank_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, const uint32_t* __restrict__ bm,
    const int32_t* __restrict__ pre, const int32_t* __restrict__ cnt,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, int tpt,
    int4* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int32_t s_off[kGroupMaxE + 1];
  __shared__ int32_t s_act[kGroupMaxE + 1];
  __shared__ int32_t s_tile[kGroupMaxE + 1];
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_off[e] = cnt[e];
  __syncthreads();
  // the counts themselves were written by the previous kernel
  group_scan_experts(E, tiles ? tpt : 1, s_off, s_act, s_tile, blockIdx.x == 0, nullptr, offsets,
                     active, n_active, tiles ? n_tiles : nullptr);
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T * k) return;
  const int e = idx[j];
  if (unsigned(e) >= unsigned(E)) {
    pos[j] = -1;
    return;
  }
  const int t = j / k;
  const int64_t wi = int64_t(t >> 5) * E + e;
  const int rank = pre[wi] + __popc(bm[wi] & ((1u << (t & 31)) - 1u));
  group_place(j, e, rank, s_off, s_act, s_tile, tpt, perm, pos, tiles);
}

size_t group_scratch_words(int64_t T, int32_t E) {
  const int64_t W = (T + 31) / 32;
  return size_t(W * E * (T > kGroupSmallT ? 2 : 1));
}

hipError_t launch_group(const int32_t* idx, int64_t T, int32_t k, int32_t E, uint32_t* scratch,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                        int32_t* active, int32_t* n_active, int tpt, int4* tiles,
                        int32_t* n_tiles, hipStream_t stream) {
  if (tiles && tpt <= 0) return hipErrorInvalidValue;
  if (E <= 0 || E > kGroupMaxE || T < 0) return hipErrorInvalidValue;
  if (T <= kGroupSmallT) {
    if (int64_t(E) * ((T + 31) / 32) <= kGroupLdsWords)
      hipLaunchKernelGGL(group_kernel<true>, dim3(1), dim3(1024), 0, stream, idx, int(T), k, E,
                         scratch, counts, offsets, perm, pos, active, n_active, tpt, tiles,
                         n_tiles);
    else
      hipLaunchKernelGGL(group_kernel<false>, dim3(1), dim3(1024), 0, stream, idx, int(T), k, E,
                         scratch, counts, offsets, perm, pos, active, n_active, tpt, tiles,
                         n_tiles);
    return hipGetLastError();
  }
  const int W = int((T + 31) / 32);
  uint32_t* bm = scratch;
  int32_t* pre = reinterpret_cast<int32_t*>(scratch + int64_t(W) * E);
  hipLaunchKernelGGL(group_bits_kernel, dim3(W), dim3(256), 0, stream, idx, int(T), k, E, bm);
  hipLaunchKernelGGL(group_prefix_kernel, dim3((E + 63) / 64), dim3(64 * kGroupPrefixWaves), 0,
                     stream, bm, W, E, pre, counts);
  const int64_t nent = T * k;
  hipLaunchKernelGGL(group_rank_kernel, dim3(unsigned((nent + 255) / 256)), dim3(256), 0, stream,
                     idx, int(T), k, E, bm, pre, counts, offsets, perm, pos, active, n_active, tpt,
                     tiles, n_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weighted combine in slot order (§3.5: weighted sum of the expert outputs),
// plus the block's residual when `resid` is given (§2.1: the residual is
// added after the MoE step).  The residual element is read and Y written by
// the same thread, so Y may be the residual itself.  Slots are taken eight at
// a time: their positions and weights are loaded together, then their rows,
// so a token costs two memory round trips per eight slots, not two per slot.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 128;
constexpr int kCombineSlots = 8;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ ybuf, const int32_t* __restrict__ pos, const float* __restrict__ w,
    int T, int k, int H, const float* resid, float* Y) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // float4 index
  const int h4 = H / 4;
  if (i >= int64_t(T) * h4) return;
  const int t = int(i / h4), c = int(i % h4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < k; s0 += kCombineSlots) {
    int ps[kCombineSlots];
    float ws[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      const int s = min(s0 + u, k - 1);
      ps[u] = pos[t * k + s];
      ws[u] = w[t * k + s];
    }
    float4 v[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u)
      v[u] = reinterpret_cast<const float4*>(ybuf + int64_t(ps[u]) * H)[c];
#pragma unroll
    for (int u = 0; u < kCombineSlots; ++u) {
      if (s0 + u >= k) break;
      acc.x = fmaf(ws[u], v[u].x, acc.x);
      acc.y = fmaf(ws[u], v[u].y, acc.y);
      acc.z = fmaf(ws[u], v[u].z, acc.z);
      acc.w = fmaf(ws[u], v[u].w, acc.w);
    }
  }
  if (resid) {
    const float4 r = reinterpret_cast<const float4*>(resid + int64_t(t) * H)[c];
    acc.x = r.x + acc.x;
    acc.y = r.y + acc.y;
    acc.z = r.z + acc.z;
    acc.w = r.w + acc.w;
  }
  reinterpret_cast<float4*>(Y + int64_t(t) * H)[c] = acc;
}

hipError_t launch_combine(const float* ybuf, const int32_t* pos, const float* w, int64_t T,
                          int32_t k, int64_t H, const float* resid, float* Y,
                          hipStream_t stream) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned((n + kCombineThreads - 1) / kCombineThreads)),
                     dim3(kCombineThreads), 0, stream, ybuf, pos, w, int(T), k, int(H), resid, Y);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm of each token row before the MoE step (§2.1; epsilon from the
// model constants of "ds4 code walkthrough"): xn = (x * r) * gamma with
// r = 1 / sqrt(mean(x^2) + eps).  One workgroup per row; each thread sums the
// squares of its float4s in order, the waves' sums meet in LDS in a fixed
// order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ X,
                                                      const float* __restrict__ gamma, int H,
                                                      float eps, float* __restrict__ xn) {
  __shared__ float red[4];
  const int n4 = H / 4;
  const float4* x4 = reinterpret_cast<const float4*>(X + int64_t(blockIdx.x) * H);
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  float4* o4 = reinterpret_cast<float4*>(xn + int64_t(blockIdx.x) * H);
  float ss = 0.0f;
  for (int j = threadIdx.x; j < n4; j += 256) {
    const float4 v = x4[j];
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float r = 1.0f / sqrtf(tot / float(H) + eps);
  for (int j = threadIdx.x; j < n4; j += 256) {
    const float4 v = x4[j], g = g4[j];
    o4[j] = make_float4((v.x * r) * g.x, (v.y * r) * g.y, (v.z * r) * g.z, (v.w * r) * g.w);
  }
}

hipError_t launch_rmsnorm(const float* X, const float* gamma, int64_t T, int64_t H, float eps,
                          float* xn, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(unsigned(T)), dim3(256), 0, stream, X, gamma, int(H),
                     eps, xn);
  return hipGetLastError();
}

}  // namespace dsq
