// decode.hip -- the MoE layer for a few tokens (decode), as four launches:
//   router GEMV (fp32) -> softmax/top-k -> gate/up GEMV + SwiGLU per routing
//   slot -> down GEMV fused with the weighted combine.
//
// Method: "Hand-writing a DeepSeek inference engine in pure C"
// (hnwysp.cn/news/134870) §3.5: router = linear layer + softmax + top-k, the
// selected experts run on the token, their outputs are summed with the routing
// weights.  With a handful of tokens every (token, slot) pair is its own
// GEMV: grouping by expert only pays once experts are shared by many tokens.
// The expert form down(silu(gate) * up) is the workload's definition.
#include "common.h"
#include "gemv_core.h"
#include "internal.h"

namespace dsq {

// ---------------------------------------------------------------------------
// Router: logits[t][e] = X[t] . Wr[e] (+ bias[e]), fp32.  One workgroup per
// (expert, tile of TT tokens); its 256 threads split K (float4 granularity),
// so the 16 KiB row is read by 256 lanes at once; per-wave partials meet in
// LDS and are added in a fixed order.
// ---------------------------------------------------------------------------
template <int TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const float* __restrict__ X, int T,
                                                          const float* __restrict__ Wr,
                                                          const float* __restrict__ bias, int E,
                                                          int H, float* __restrict__ logits) {
  __shared__ float red[4][TT];
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * TT;
  const int tt = min(TT, T - t0);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n4 = H / 4;
  const float4* w4 = reinterpret_cast<const float4*>(Wr + int64_t(e) * H);
  const float4* x4 = reinterpret_cast<const float4*>(X + int64_t(t0) * H);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  // four float4 per thread in flight per iteration (H = 4096: one iteration)
  // Loads from clamped addresses (no branches, all in flight at once); a
  // duplicated weight float4 is paired with a zeroed x float4.
  for (int j0 = threadIdx.x; j0 < n4; j0 += 1024) {
    float4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = w4[min(j0 + 256 * u, n4 - 1)];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int tc = min(t, tt - 1);
      float4 xv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) xv[u] = x4[int64_t(tc) * n4 + min(j0 + 256 * u, n4 - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool keep = t < tt && j0 + 256 * u < n4;
        acc[t] = fmaf(w[u].x, keep ? xv[u].x : 0.0f, acc[t]);
        acc[t] = fmaf(w[u].y, keep ? xv[u].y : 0.0f, acc[t]);
        acc[t] = fmaf(w[u].z, keep ? xv[u].z : 0.0f, acc[t]);
        acc[t] = fmaf(w[u].w, keep ? xv[u].w : 0.0f, acc[t]);
      }
    }
  }
  const float s = wave_reduce_scatter<TT>(acc);
  if ((lane & (64 / TT - 1)) == 0) red[wv][reduce_scatter_row<TT>(lane)] = s;
  __syncthreads();
  if (threadIdx.x < tt) {
    const int t = threadIdx.x;
    float v = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    if (bias) v += bias[e];
    logits[int64_t(t0 + t) * E + e] = v;
  }
}

hipError_t launch_router_gemv(const float* X, int64_t T, const float* Wr, const float* bias,
                              int32_t E, int64_t H, float* logits, hipStream_t stream) {
  if (T <= 1) {
    hipLaunchKernelGGL(router_gemv_kernel<1>, dim3(E, unsigned(T)), dim3(256), 0, stream, X,
                       int(T), Wr, bias, E, int(H), logits);
  } else if (T <= 2) {
    hipLaunchKernelGGL(router_gemv_kernel<2>, dim3(E, 1), dim3(256), 0, stream, X, int(T), Wr,
                       bias, E, int(H), logits);
  } else if (T <= 4) {
    hipLaunchKernelGGL(router_gemv_kernel<4>, dim3(E, 1), dim3(256), 0, stream, X, int(T), Wr,
                       bias, E, int(H), logits);
  } else {
    hipLaunchKernelGGL(router_gemv_kernel<8>, dim3(E, unsigned((T + 7) / 8)), dim3(256), 0,
                       stream, X, int(T), Wr, bias, E, int(H), logits);
  }
  return hipGetLastError();
}

struct DecArgs {
  const uint8_t* gate;   // packed gate (entry 0)
  const uint8_t* up;
  const uint8_t* down;
  int64_t gu_stride, gu_meta_off;  // gate/up entry geometry (N = I, K = H)
  int64_t d_stride, d_meta_off;    // down entry geometry (N = H, K = I)
  int H, I, group, k, E;
  const float* X;        // [T][H]
  const float* logits;   // [T][E] router scores (bias included)
  int32_t* idx;          // [T][k] written by the gate/up kernel
  float* w;              // [T][k] written by the gate/up kernel
  float* hbuf;           // [T*k][I]
  float* Y;              // [T][H]
};

#ifndef DSQ_GU_RP
#define DSQ_GU_RP 2  // gate/up output rows per wave step (2 * RP weight rows)
#endif
#ifndef DSQ_GU_WAVES
#define DSQ_GU_WAVES (256 * 8)  // target waves over all slots
#endif
#ifndef DSQ_DN_R
#define DSQ_DN_R 4  // down output rows per wave
#endif

constexpr int kDecodeMaxE = 1024;  // scores per lane held in registers: 16

// ---------------------------------------------------------------------------
// Top-k of one token's E scores by one wave (softmax + top-k + renormalise,
// "Hand-writing a DeepSeek inference engine in pure C" §3.4-§3.5): k rounds
// of a DPP wave argmax with the comparator (score desc, index desc).  Returns
// the expert of rank `want` and its renormalised weight
//   exp(s_want - s_max) / sum over the k selected of exp(s - s_max).
// ---------------------------------------------------------------------------
template <int EPL>
__device__ __forceinline__ void topk_rank(const float* __restrict__ l, int E, int k, int want,
                                          int lane, int* out_e, float* out_w) {
  float v[EPL];
  uint32_t taken = 0;
  // all loads first (clamped addresses, no branches), then the fix-ups
#pragma unroll
  for (int j = 0; j < EPL; ++j) v[j] = l[min(lane + 64 * j, E - 1)];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    if (v[j] != v[j]) v[j] = -INFINITY;  // NaN ranks last
    if (e >= E) taken |= 1u << j;
  }
  float best = 0.0f, mine = 0.0f, sum = 0.0f;
  int mine_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (!((taken >> j) & 1u) && (bi < 0 || ranks_before(v[j], e, bv, bi))) {
        bv = v[j];
        bi = e;
      }
    }
    wave_argmax(bv, bi);  // uniform across the wave
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (r == 0) best = bv;
    const float ex = expf(bv - best);
    sum += ex;
    if (r == want) {
      mine = ex;
      mine_e = bi;
    }
  }
  *out_e = mine_e;
  *out_w = mine / sum;
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU: one routing slot j = t*k + i per blockIdx.y.  Wave 0
// first ranks token t's scores to find the slot's expert (the workgroups
// with blockIdx.x == 0 also publish idx/w for the down kernel).  Then each
// wave walks blocks of RP output rows n, computing gate row n and up row n
// of that expert against X[t] (staged in LDS, sliced into registers), and
// writes h[j][n] = silu(g) * u.  The next row block's loads are issued
// before the current one's math.
// ---------------------------------------------------------------------------
template <int BITS, int RP, int KCH>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(DecArgs p) {
  constexpr int NR = 2 * RP;
  extern __shared__ float4 xl[];
  __shared__ int s_e;
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.y;
  const int t = slot / p.k;
  if (threadIdx.x < 64) {
    int e;
    float wgt;
    topk_rank<kDecodeMaxE / 64>(p.logits + int64_t(t) * p.E, p.E, p.k, slot % p.k, lane, &e,
                                &wgt);
    if (lane == 0) {
      s_e = e;
      if (blockIdx.x == 0) {
        p.idx[slot] = e;
        p.w[slot] = wgt;
      }
    }
  }
  __syncthreads();
  const int e = s_e;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int row_bytes = p.H * BITS / 8;
  const int nchunk = row_bytes / 16;
  const int groups = p.H / p.group;
  const uint8_t* gbase = p.gate + int64_t(e) * p.gu_stride;
  const uint8_t* ubase = p.up + int64_t(e) * p.gu_stride;
  const float2* gmeta = reinterpret_cast<const float2*>(gbase + p.gu_meta_off);
  const float2* umeta = reinterpret_cast<const float2*>(ubase + p.gu_meta_off);

  auto load = [&](RowChunks<BITS, NR, KCH>& C, int n0) {
    const uint8_t* prow[NR];
    const float2* mrow[NR];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int n = min(n0 + r, p.I - 1);
      prow[r] = gbase + int64_t(n) * row_bytes;
      mrow[r] = gmeta + int64_t(n) * groups;
      prow[RP + r] = ubase + int64_t(n) * row_bytes;
      mrow[RP + r] = umeta + int64_t(n) * groups;
    }
    C.load(prow, mrow, nchunk, p.group, lane);
  };
  XSlice<BITS, KCH> xs;
  auto finish = [&](const RowChunks<BITS, NR, KCH>& C, int n0) {
    float acc[NR];
    C.dot(xs, acc);
    float g[RP], u[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      g[r] = acc[r];
      u[r] = acc[RP + r];
    }
    const float tg = wave_reduce_scatter<RP>(g);
    const float tu = wave_reduce_scatter<RP>(u);
    if ((lane & (64 / RP - 1)) == 0) {
      const int n = n0 + reduce_scatter_row<RP>(lane);
      if (n < p.I) p.hbuf[int64_t(slot) * p.I + n] = silu(tg) * tu;
    }
  };

  RowChunks<BITS, NR, KCH> A, B;
  const int step = nwaves * RP;
  int n0 = wave * RP;
  if (n0 < p.I) load(A, n0);
  stage_lds<Codes<BITS>::kPerChunk / 4>(p.X + int64_t(t) * p.H, p.H, xl);
  __syncthreads();
  xs.load_lds(xl, nchunk, lane);
  xs.sums();
  while (n0 < p.I) {
    const int n1 = n0 + step;
    if (n1 < p.I) load(B, n1);
    finish(A, n0);
    if (n1 >= p.I) break;
    const int n2 = n1 + step;
    if (n2 < p.I) load(A, n2);
    finish(B, n1);
    n0 = n2;
  }
}

// ---------------------------------------------------------------------------
// down + combine: one token per blockIdx.y; the token's k vectors h[t*k+i]
// are staged in LDS once per workgroup.  Each wave owns R output rows and,
// for each of the token's k slots in order, adds
//   w[t][i] * (h[t*k+i] . Wd_{idx[t][i]}[n])
// to its per-lane partial sums before one reduction per row.  The next
// slot's weights are loaded while the current slot is computed.  No atomics:
// the result is deterministic.
// ---------------------------------------------------------------------------
template <int BITS, int R, int KCH>
__global__ __launch_bounds__(256) void down_combine_kernel(DecArgs p) {
  constexpr int F = Codes<BITS>::kPerChunk / 4;
  extern __shared__ float4 hl[];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.y;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = wave * R;
  const int row_bytes = p.I * BITS / 8;
  const int nchunk = row_bytes / 16;
  const int groups = p.I / p.group;
  const bool active = n0 < p.H;

  auto load = [&](RowChunks<BITS, R, KCH>& C, int i) {
    const int e = p.idx[t * p.k + i];
    const uint8_t* dbase = p.down + int64_t(e) * p.d_stride;
    const float2* dmeta = reinterpret_cast<const float2*>(dbase + p.d_meta_off);
    const uint8_t* prow[R];
    const float2* mrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(n0 + r, p.H - 1);
      prow[r] = dbase + int64_t(n) * row_bytes;
      mrow[r] = dmeta + int64_t(n) * groups;
    }
    C.load(prow, mrow, nchunk, p.group, lane);
  };
  RowChunks<BITS, R, KCH> A, B;
  if (active) load(A, 0);
  for (int i = 0; i < p.k; ++i)
    stage_lds<F>(p.hbuf + int64_t(t * p.k + i) * p.I, p.I, hl + int64_t(i) * (p.I / 4));
  __syncthreads();
  if (!active) return;  // after the only barrier

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  auto accumulate = [&](const RowChunks<BITS, R, KCH>& C, int i) {
    XSlice<BITS, KCH> xs;
    xs.load_lds(hl + int64_t(i) * (p.I / 4), nchunk, lane);
    xs.sums();
    float part[R];
    C.dot(xs, part);
    const float wgt = p.w[t * p.k + i];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fmaf(wgt, part[r], acc[r]);
  };
  for (int i = 0; i < p.k; i += 2) {
    if (i + 1 < p.k) load(B, i + 1);
    accumulate(A, i);
    if (i + 1 >= p.k) break;
    if (i + 2 < p.k) load(A, i + 2);
    accumulate(B, i + 1);
  }
  const float s = wave_reduce_scatter<R>(acc);
  if ((lane & (64 / R - 1)) == 0) {
    const int n = n0 + reduce_scatter_row<R>(lane);
    if (n < p.H) p.Y[int64_t(t) * p.H + n] = s;
  }
}

namespace {

template <int BITS, int KCH>
hipError_t go_decode(const DecArgs& a, int64_t T, hipStream_t stream) {
  constexpr int RP = DSQ_GU_RP;
  const int64_t slots = T * a.k;
  const int rowblocks = (a.I + RP - 1) / RP;
  // Waves per slot, rounded down to whole workgroups so the grid never
  // exceeds one round of resident waves (a second round would start only when
  // the first finishes and doubles the kernel time).
  int64_t wps = DSQ_GU_WAVES / slots;
  if (wps > rowblocks) wps = rowblocks;
  int bx = int(wps / 4);
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL((gateup_gemv_kernel<BITS, RP, KCH>), dim3(bx, unsigned(slots)), dim3(256),
                     size_t(a.H) * 4, stream, a);
  return hipGetLastError();
}

template <int BITS, int KCH>
hipError_t go_down(const DecArgs& a, int64_t T, hipStream_t stream) {
  constexpr int R = DSQ_DN_R;
  const int waves = (a.H + R - 1) / R;
  const int bx = (waves + 3) / 4;
  hipLaunchKernelGGL((down_combine_kernel<BITS, R, KCH>), dim3(bx, unsigned(T)), dim3(256),
                     size_t(a.k) * a.I * 4, stream, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_gateup(const DecArgs& a, int64_t T, hipStream_t s) {
  const int kch = (a.H * BITS / 8 / 16 + 63) / 64;
  switch (kch) {
    case 1: return go_decode<BITS, 1>(a, T, s);
    case 2: return go_decode<BITS, 2>(a, T, s);
    case 3: return go_decode<BITS, 3>(a, T, s);
    case 4: return go_decode<BITS, 4>(a, T, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t dispatch_down(const DecArgs& a, int64_t T, hipStream_t s) {
  const int kch = (a.I * BITS / 8 / 16 + 63) / 64;
  switch (kch) {
    case 1: return go_down<BITS, 1>(a, T, s);
    case 2: return go_down<BITS, 2>(a, T, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// True when the decode kernels apply: a row's x slice fits the register
// budget (at most 4 chunk rounds per lane for K = H and for K = I), the
// scores of a token fit one wave's registers, and the token's k vectors h fit
// the 64 KiB of LDS the down kernel stages them in.
bool decode_supported(int bits, int64_t H, int64_t I, int32_t E, int32_t k) {
  const int64_t a = (H * bits / 8 / 16 + 63) / 64;
  const int64_t b = (I * bits / 8 / 16 + 63) / 64;
  return a <= 4 && b <= 2 && E <= kDecodeMaxE && int64_t(k) * I * 4 <= 65536 && H * 4 <= 65536;
}

hipError_t launch_moe_decode(const dsq_qweight& gate, const dsq_qweight& up,
                             const dsq_qweight& down, const float* X, int64_t T, int32_t E,
                             int32_t k, const float* logits, int32_t* idx, float* w, float* hbuf,
                             float* Y, hipStream_t stream) {
  const Layout Lgu = layout_of(gate.bits, gate.group, gate.K, gate.N);
  const Layout Ld = layout_of(down.bits, down.group, down.K, down.N);
  DecArgs a{};
  a.gate = static_cast<const uint8_t*>(gate.data);
  a.up = static_cast<const uint8_t*>(up.data);
  a.down = static_cast<const uint8_t*>(down.data);
  a.gu_stride = Lgu.stride;
  a.gu_meta_off = Lgu.meta_off;
  a.d_stride = Ld.stride;
  a.d_meta_off = Ld.meta_off;
  a.H = int(gate.K);
  a.I = int(gate.N);
  a.group = gate.group;
  a.k = k;
  a.E = E;
  a.logits = logits;
  a.X = X;
  a.idx = idx;
  a.w = w;
  a.hbuf = hbuf;
  a.Y = Y;
  hipError_t e = gate.bits == 8 ? dispatch_gateup<8>(a, T, stream) : dispatch_gateup<4>(a, T, stream);
  if (e != hipSuccess) return e;
  return gate.bits == 8 ? dispatch_down<8>(a, T, stream) : dispatch_down<4>(a, T, stream);
}

}  // namespace dsq
