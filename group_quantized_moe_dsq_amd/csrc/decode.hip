// decode.hip -- the MoE layer for a few tokens (decode), as three launches:
//   router GEMV (fp32) -> gate/up + SwiGLU per routing slot (the kernel ranks
//   the scores itself) -> down fused with the weighted combine.
//
// Method: "Hand-writing a DeepSeek inference engine in pure C"
// (hnwysp.cn/news/134870) §3.2 (dequantize inside the matmul loop), §3.5
// (router = linear layer + softmax + top-k, the selected experts run on the
// token, their outputs are summed with the routing weights).  With a handful
// of tokens every (token, slot) pair is its own matrix-vector product:
// grouping by expert only pays once experts are shared by many tokens.  The
// expert form down(silu(gate) * up) is the workload's definition.
//
// The expert products run on v_mfma_f32_16x16x32_bf16 like the grouped GEMM
// (gmm.hip): the B operand holds 16 weight rows as exact bf16 integers (INT4:
// bf16(16 + q), INT8: bf16(q)), the A operand the token's activation split
// into two bf16 parts x = hi + lo (rows 0 and 1; rows 2..15 are zero), and
// each group's zero point and scale are applied in fp32:
//   sum_k x (q - zp) s = s (sum_k x (q + o) - (zp + o) sum_k x).
// This keeps the INT4 dequantization at about one VALU operation per code
// (the fp32 FMA form needs about three, which would make decode VALU-bound).
// A workgroup of 8 waves owns one 16-row tile; its waves split K eight ways
// and meet in LDS, where the parts are added in a fixed order.
#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace dsq {

// ---------------------------------------------------------------------------
// Router: logits[t][e] = X[t] . Wr[e] (+ bias[e]), fp32.  One workgroup per
// (expert, tile of TT tokens); its 256 threads split K (float4 granularity),
// so the 16 KiB row is read by 256 lanes at once; per-wave partials meet in
// LDS and are added in a fixed order.
//
// With gamma the rows are first normalised (RMSNorm before the MoE step,
// "Hand-writing a DeepSeek inference engine in pure C" §2.1):
// xn = (x * r) * gamma, r = 1 / sqrt(mean(x^2) + eps).  Every workgroup
// computes r itself from the whole row (same code, same order, so the same
// bits everywhere), and the expert-0 workgroup of each token tile writes xn
// for the later kernels.
// ---------------------------------------------------------------------------
template <int TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const float* __restrict__ X, int T,
                                                          const float* __restrict__ Wr,
                                                          const float* __restrict__ bias, int E,
                                                          int H, float* __restrict__ logits,
                                                          const float* __restrict__ gamma,
                                                          float eps, float* __restrict__ xn) {
  __shared__ float red[4][TT];
  __shared__ float red_ss[4][TT];
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * TT;
  const int tt = min(TT, T - t0);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n4 = H / 4;
  const float4* w4 = reinterpret_cast<const float4*>(Wr + int64_t(e) * H);
  const float4* x4 = reinterpret_cast<const float4*>(X + int64_t(t0) * H);
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  float4* xn4 = reinterpret_cast<float4*>(xn + int64_t(t0) * H);
  const bool write_xn = xn != nullptr && e == 0;
  float rinv[TT];
  if (gamma) {
    float ss[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) ss[t] = 0.0f;
    for (int j0 = threadIdx.x; j0 < n4; j0 += 1024) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int tc = min(t, tt - 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 v = x4[int64_t(tc) * n4 + min(j0 + 256 * u, n4 - 1)];
          const bool keep = t < tt && j0 + 256 * u < n4;
          ss[t] = fmaf(v.x, keep ? v.x : 0.0f, ss[t]);
          ss[t] = fmaf(v.y, keep ? v.y : 0.0f, ss[t]);
          ss[t] = fmaf(v.z, keep ? v.z : 0.0f, ss[t]);
          ss[t] = fmaf(v.w, keep ? v.w : 0.0f, ss[t]);
        }
      }
    }
    const float s = wave_reduce_scatter<TT>(ss);
    if ((lane & (64 / TT - 1)) == 0) red_ss[wv][reduce_scatter_row<TT>(lane)] = s;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float tot = ((red_ss[0][t] + red_ss[1][t]) + red_ss[2][t]) + red_ss[3][t];
      rinv[t] = 1.0f / sqrtf(tot / float(H) + eps);
    }
  }
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  // four float4 per thread in flight per iteration (H = 4096: one iteration)
  // Loads from clamped addresses (no branches, all in flight at once); a
  // duplicated weight float4 is paired with a zeroed x float4.
  for (int j0 = threadIdx.x; j0 < n4; j0 += 1024) {
    float4 w[4], gv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = w4[min(j0 + 256 * u, n4 - 1)];
    if (gamma) {
#pragma unroll
      for (int u = 0; u < 4; ++u) gv[u] = g4[min(j0 + 256 * u, n4 - 1)];
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int tc = min(t, tt - 1);
      float4 xv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) xv[u] = x4[int64_t(tc) * n4 + min(j0 + 256 * u, n4 - 1)];
      if (gamma) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xv[u].x = (xv[u].x * rinv[t]) * gv[u].x;
          xv[u].y = (xv[u].y * rinv[t]) * gv[u].y;
          xv[u].z = (xv[u].z * rinv[t]) * gv[u].z;
          xv[u].w = (xv[u].w * rinv[t]) * gv[u].w;
          if (write_xn && t < tt && j0 + 256 * u < n4) xn4[int64_t(t) * n4 + j0 + 256 * u] = xv[u];
        }
      }
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
                              int32_t E, int64_t H, float* logits, const float* gamma, float eps,
                              float* xn, hipStream_t stream) {
  if (T <= 1) {
    hipLaunchKernelGGL(router_gemv_kernel<1>, dim3(E, unsigned(T)), dim3(256), 0, stream, X,
                       int(T), Wr, bias, E, int(H), logits, gamma, eps, xn);
  } else if (T <= 2) {
    hipLaunchKernelGGL(router_gemv_kernel<2>, dim3(E, 1), dim3(256), 0, stream, X, int(T), Wr,
                       bias, E, int(H), logits, gamma, eps, xn);
  } else if (T <= 4) {
    hipLaunchKernelGGL(router_gemv_kernel<4>, dim3(E, 1), dim3(256), 0, stream, X, int(T), Wr,
                       bias, E, int(H), logits, gamma, eps, xn);
  } else {
    hipLaunchKernelGGL(router_gemv_kernel<8>, dim3(E, unsigned((T + 7) / 8)), dim3(256), 0,
                       stream, X, int(T), Wr, bias, E, int(H), logits, gamma, eps, xn);
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
  const float* logits;   // [T][E] router scores (bias included), or NULL: routing given
  int32_t* idx;          // [T][k] written by the gate/up kernel (read when given)
  float* w;              // [T][k] written by the gate/up kernel (read when given)
  float* hbuf;           // [T*k][I]
  float* Y;              // [T][H]
  const float* resid;    // [T][H] added to Y, or NULL (may equal Y)
};

#ifndef DSQ_DEC_GU_DEPTH
#define DSQ_DEC_GU_DEPTH 2
#endif
#ifndef DSQ_DEC_DN_DEPTH
#define DSQ_DEC_DN_DEPTH 2
#endif
#ifndef DSQ_DEC_UB
#define DSQ_DEC_UB 4
#endif
constexpr int kDecodeMaxE = 256;  // scores per lane held in registers: 4
constexpr int kDecWaves = 8;       // waves per workgroup: the K split
constexpr int kDecUB = DSQ_DEC_UB; // gate/up units whose sums are added together

// ---------------------------------------------------------------------------
// Top-k of one token's E scores by one wave (softmax + top-k + renormalise,
// "Hand-writing a DeepSeek inference engine in pure C" §3.4-§3.5): k rounds
// of a DPP wave argmax with the comparator (score desc, index desc).  Writes
// the experts in rank order to e_out[0..k) and their renormalised weights
//   exp(s_r - s_max) / sum over the k selected of exp(s - s_max)
// to w_out[0..k) (LDS).
// ---------------------------------------------------------------------------
template <int EPL>
__device__ __forceinline__ void topk_all(const float* __restrict__ l, int E, int k, int lane,
                                         int* e_out, float* w_out) {
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
  float best = 0.0f, mine = 0.0f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      const bool better = !((taken >> j) & 1u) & ((bi < 0) | (v[j] > bv) | ((v[j] == bv) & (e > bi)));
      bv = better ? v[j] : bv;
      bi = better ? e : bi;
    }
    wave_argmax(bv, bi);  // uniform across the wave
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (r == 0) best = bv;
    if (lane == r) mine = bv;
    if (lane == 0) e_out[r] = bi;
  }
  const float ex = lane < k ? expf(mine - best) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) w_out[lane] = ex / sum;
}

// ---------------------------------------------------------------------------
// Activation parts in LDS: rows of x (fp32) -> xp[row][part][K] bf16 (part 0:
// hi = bf16(x), part 1: lo = bf16(x - hi)) and xs[row][group] = (sum of hi,
// sum of lo, 0, 0) over the group, the sums taken in double and rounded once.
// The A operand of lane (c, g4) is row c < 2 of this layout; the group-sum
// operand of lane g4 = 0 is the float4 itself, all other lanes read zeros.
// ---------------------------------------------------------------------------
// One pass of the staging: up to U segments (8 values) per thread, loads
// first (clamped addresses), converted and stored by stage_store.  A kernel
// can issue the loads early and store after other work.
constexpr int kStageU = 4;
struct StageRegs {
  float4 qa[kStageU], qb[kStageU];
};

__device__ __forceinline__ void stage_load(const float* __restrict__ src, int64_t ld,
                                           const int32_t* __restrict__ rows, int nrows, int K,
                                           int base, int nthreads, StageRegs& q) {
  const int segs = K / 8;
  const int total = nrows * segs;
#pragma unroll
  for (int u = 0; u < kStageU; ++u) {
    const int it = min(base + u * nthreads, total - 1);
    const int r = it / segs, sg = it % segs;
    const int64_t row = rows ? rows[r] : r;
    const float4* v = reinterpret_cast<const float4*>(src + row * ld + sg * 8);
    q.qa[u] = v[0];
    q.qb[u] = v[1];
  }
}

__device__ __forceinline__ void stage_store(const StageRegs& q, int nrows, int K, int G,
                                            uint16_t* xp, float4* xs, int base, int nthreads) {
  const int segs = K / 8;  // multiple of G / 8: a group's lanes are adjacent
  const int total = nrows * segs;
#pragma unroll
  for (int u = 0; u < kStageU; ++u) {
    const int it = base + u * nthreads;
    if (it >= total) break;  // whole groups leave together: total is a multiple of G / 8
    const int r = it / segs, sg = it % segs;
    const float v[8] = {q.qa[u].x, q.qa[u].y, q.qa[u].z, q.qa[u].w,
                        q.qb[u].x, q.qb[u].y, q.qb[u].z, q.qb[u].w};
    uint32_t hw[4], lw[4];
    double sh = 0.0, sl = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h0 = __bf16(v[2 * i]), h1 = __bf16(v[2 * i + 1]);
      const __bf16 l0 = __bf16(v[2 * i] - float(h0)), l1 = __bf16(v[2 * i + 1] - float(h1));
      hw[i] = uint32_t(__builtin_bit_cast(uint16_t, h0)) |
              (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
      lw[i] = uint32_t(__builtin_bit_cast(uint16_t, l0)) |
              (uint32_t(__builtin_bit_cast(uint16_t, l1)) << 16);
      sh += double(float(h0)) + double(float(h1));
      sl += double(float(l0)) + double(float(l1));
    }
    for (int o = 1; o < G / 8; o <<= 1) {
      sh += __shfl_xor(sh, o);
      sl += __shfl_xor(sl, o);
    }
    uint4* d = reinterpret_cast<uint4*>(xp + (int64_t(r) * 2) * K + sg * 8);
    d[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    d[K / 8] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    if ((sg * 8) % G == 0)
      xs[r * (K / G) + sg * 8 / G] = make_float4(float(sh), float(sl), 0.f, 0.f);
  }
}

// true when one pass (kStageU segments per thread) stages nrows rows of K
__host__ __device__ constexpr bool stage_one_pass(int64_t nrows, int64_t K, int nthreads) {
  return nrows * (K / 8) <= int64_t(kStageU) * nthreads;
}

__device__ __forceinline__ void stage_parts(const float* __restrict__ src, int64_t ld,
                                            const int32_t* __restrict__ rows, int nrows, int K,
                                            int G, uint16_t* xp, float4* xs, int tid,
                                            int nthreads) {
  const int total = nrows * (K / 8);
  for (int base = tid; base < total; base += kStageU * nthreads) {
    StageRegs q;
    stage_load(src, ld, rows, nrows, K, base, nthreads, q);
    stage_store(q, nrows, K, G, xp, xs, base, nthreads);
  }
}

// ---------------------------------------------------------------------------
// Streaming a wave's share of NT weight tiles (16 rows each) through its own
// LDS ring.  A step is 128 code bytes (L groups) of every row; step m of wave
// w is piece 8 m + w of the rows, so at each step the workgroup's eight waves
// read one contiguous kilobyte of every row together (a DRAM row is opened
// once, not once per wave).  The pieces are fetched by direct global->LDS
// loads: 16-byte chunk j of row r lands at position j ^ swz(r) of the row, so
// the MFMA operand reads (16 rows at once) fall on distinct banks; the rows'
// (scale, zp) of the step land beside them.  A ring holds DEPTH steps, chosen
// per kernel; only this wave reads its ring, so no barrier is needed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dswz(int r) { return (r >> 1) & 7; }

template <int BITS, int J, int NT>
struct DecRing {
  static constexpr int L = 1024 / (J * 32 * BITS);  // groups per step
  static constexpr int LB = J * BITS;                 // code bytes per lane, tile and group
  static constexpr int CSLOT = NT * 2048;
  static constexpr int WSLOT = CSLOT + NT * 16 * L * 8;
  static constexpr int PPR = L >= 2 ? L / 2 : 2;      // direct-load pieces per metadata row
  static constexpr int PB = L >= 2 ? 16 : 4;          // bytes per piece
  static constexpr int PER_STEP = 3 * NT;             // direct loads per step
};

// Per-lane offsets of a wave's tiles (step 0 of its share).
template <int BITS, int J, int NT>
struct DecLane {
  __amdgpu_buffer_rsrc_t rc[NT], rm[NT];
  int vdc[NT][2];
  int vdm[NT];
};

template <int BITS, int J, int NT>
__device__ __forceinline__ void dec_lane(DecLane<BITS, J, NT>& ln, const uint8_t* const (&mat)[NT],
                                         int64_t meta_off, int N, int K, int G, int row0,
                                         int s_lo, int lane) {
  using R = DecRing<BITS, J, NT>;
  const int S = K / G;
  const int64_t RB = int64_t(K) * BITS / 8;
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    ln.rc[b] = rsrc(mat[b], int64_t(N) * RB);
    ln.rm[b] = rsrc(mat[b] + meta_off, int64_t(N) * S * 8);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + (lane >> 3);
      const int n = min(row0 + r, N - 1);
      ln.vdc[b][h] = int(int64_t(n) * RB) + s_lo * (G * BITS / 8) + (((lane & 7) ^ dswz(r)) << 4);
    }
    const int n = min(row0 + lane / R::PPR, N - 1);
    ln.vdm[b] = (n * S + s_lo) * 8 + (lane % R::PPR) * R::PB;
  }
}

template <int BITS, int J, int NT, class Lane>
__device__ __forceinline__ void dec_issue(const Lane& ln, uint8_t* slot, int m, int lane) {
  using R = DecRing<BITS, J, NT>;
#pragma unroll
  for (int b = 0; b < NT; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ln.rc[b], (lds_ptr_t)(slot + b * 2048 + h * 1024),
                                               16, ln.vdc[b][h] + m * (kDecWaves * 128), 0, 0, 0);
  if (lane < 16 * R::PPR) {
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      lds_ptr_t dst = (lds_ptr_t)(slot + R::CSLOT + b * 16 * R::L * 8);
      const int off = ln.vdm[b] + m * (kDecWaves * R::L * 8);
      // the piece size as a literal (the builtin takes a constant)
      if constexpr (R::PB == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(ln.rm[b], dst, 16, off, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(ln.rm[b], dst, 4, off, 0, 0, 0);
    }
  }
}

// Products of step m of the wave's share (groups s_lo + 8 L m .. + L, s_lo =
// L w): for every group s of the step below s_hi, y[b] += the group's fp32
// correction of the MFMA sum of the activation parts (rows 0, 1 of A) times
// tile b's codes.  SHARED: every tile takes the activation xp[0] / xs[0]
// (gate and up of one slot); else tile b takes xp[b] / xs[b] (the tiles of
// different slots).
template <int BITS, int J, int NT, bool SHARED>
__device__ __forceinline__ void dec_step(const uint8_t* slot, f32x4_t (&y)[NT],
                                         const uint16_t* const (&xp)[NT],
                                         const float4* const (&xs)[NT], int K, int G, int s_lo,
                                         int s_hi, int m, int lane, const uint32_t* zeros) {
  using R = DecRing<BITS, J, NT>;
  constexpr float kOff = BITS == 4 ? 16.0f : 0.0f;
  constexpr int NA = SHARED ? 1 : NT;  // activations read per group
  const int c = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int sl = 0; sl < R::L; ++sl) {
    const int s = s_lo + m * (kDecWaves * R::L) + sl;
    if (s >= s_hi) break;  // uniform
    u32x4_t af[NA][J];
    f32x2_t xv[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int k = s * G + g4 * 8 * J + 8 * j;
        const uint16_t* src =
            c < 2 ? xp[a] + int64_t(c) * K + k : reinterpret_cast<const uint16_t*>(zeros);
        af[a][j] = *reinterpret_cast<const u32x4_t*>(src);
      }
      // the group's sums (hi, lo): read by every lane, used by lanes g4 = 0
      xv[a] = lds_read_f32x2(xs[a] + s);
    }
    const int off = sl * (G * BITS / 8) + g4 * R::LB;  // byte of the 128-byte window
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int a = SHARED ? 0 : b;
      const uint8_t* row = slot + b * 2048 + c * 128;
      uint32_t w[R::LB / 4];
      if constexpr (R::LB == 8) {
        const u32x2_t v =
            *reinterpret_cast<const u32x2_t*>(row + (((off >> 4) ^ dswz(c)) << 4) + (off & 15));
        w[0] = v[0];
        w[1] = v[1];
      } else {
#pragma unroll
        for (int h = 0; h < R::LB / 16; ++h) {
          const u32x4_t v =
              *reinterpret_cast<const u32x4_t*>(row + ((((off >> 4) + h) ^ dswz(c)) << 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) w[4 * h + i] = v[i];
        }
      }
      const f32x2_t mq =
          *reinterpret_cast<const f32x2_t*>(slot + R::CSLOT + (b * 16 + c) * R::L * 8 + sl * 8);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < J; ++j) {
        u32x4_t bq;
        if constexpr (BITS == 4) bq = int4_to_bf16(w[j]);
        else bq = int8_to_bf16(w[2 * j], w[2 * j + 1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[a][j]),
                                                      __builtin_bit_cast(bf16x8_t, bq), acc, 0, 0,
                                                      0);
      }
      const float sc = mq[0], zq = mq[1] + kOff;
      if (b == 0) {
#pragma unroll
        for (int q = 0; q < NA; ++q) lgkm_wait(xv[q]);
      }
      const float x0 = g4 == 0 ? xv[a][0] : 0.0f, x1 = g4 == 0 ? xv[a][1] : 0.0f;
      y[b][0] = fmaf(sc, fmaf(-zq, x0, acc[0]), y[b][0]);
      y[b][1] = fmaf(sc, fmaf(-zq, x1, acc[1]), y[b][1]);
    }
  }
}

// A wave's ring of streamed steps.  Steps are numbered over the wave's whole
// sequence (units one after another), so the loads of the next unit are in
// flight while the current unit is reduced.
template <int BITS, int J, int NT, int DEPTH_>
struct DecStream {
  using R = DecRing<BITS, J, NT>;
  static constexpr int DEPTH = DEPTH_;                // steps per ring
  static constexpr int BYTES = DEPTH * R::WSLOT;      // LDS per wave
  uint8_t* ring;
  int issued = 0;     // steps issued
  int consumed = 0;   // steps computed
  __device__ __forceinline__ uint8_t* slot(int g) const { return ring + (g % DEPTH) * R::WSLOT; }
  // Wait for the oldest outstanding step (the one about to be computed).
  __device__ __forceinline__ void wait_oldest() const {
    const int ahead = issued - consumed - 1;  // steps issued after it
    if (ahead >= 6) wait_vmcnt<6 * R::PER_STEP>();
    else if (ahead == 5) wait_vmcnt<5 * R::PER_STEP>();
    else if (ahead == 4) wait_vmcnt<4 * R::PER_STEP>();
    else if (ahead == 3) wait_vmcnt<3 * R::PER_STEP>();
    else if (ahead == 2) wait_vmcnt<2 * R::PER_STEP>();
    else if (ahead == 1) wait_vmcnt<R::PER_STEP>();
    else wait_vmcnt<0>();
  }
};

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Every workgroup first ranks the scores of the T tokens
// (wave t ranks token t; workgroup 0 publishes idx/w for the down kernel).
// Units (slot j = t*k + i, 16-row tile) are dealt to the workgroups in a
// fixed stride (token-major, so a workgroup restages the activation parts
// only when the token changes); within a unit, wave w streams the pieces
// w, w + 8, ... of K (L groups each) of the gate and the up tile, and the
// eight partial sums of each row meet in LDS.
// ---------------------------------------------------------------------------
template <int BITS, int J>
__global__ __launch_bounds__(512) void dec_gateup_kernel(DecArgs p, int T) {
  using R = DecRing<BITS, J, 2>;
  using St = DecStream<BITS, J, 2, DSQ_DEC_GU_DEPTH>;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  __shared__ int s_e[4 * 32];
  __shared__ float s_w[4 * 32];
  // partial sums of a batch of units, double-buffered: [batch parity][unit
  // of the batch][wave][gate | up][row]
  __shared__ float red[2][kDecUB][kDecWaves][2][16];
  __shared__ __attribute__((aligned(16))) uint32_t zeros[4];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  const int H = p.H, I = p.I, G = p.group, S = H / G, k = p.k;
  uint8_t* rings = dsm;                                                      // [8][DEPTH][WSLOT]
  uint16_t* xp = reinterpret_cast<uint16_t*>(dsm + kDecWaves * St::BYTES);    // [2][H]
  float4* xs = reinterpret_cast<float4*>(dsm + kDecWaves * St::BYTES + 4 * H);  // [S]

  if (threadIdx.x < 4) zeros[threadIdx.x] = 0u;
  // token 0's activation is loaded first and converted once the first weight
  // loads are in flight; waves 0..T-1 rank the tokens' scores meanwhile
  StageRegs x0;
  stage_load(p.X, H, nullptr, 1, H, threadIdx.x, 512, x0);
  if (p.logits) {
    if (wv < T)
      topk_all<kDecodeMaxE / 64>(p.logits + int64_t(wv) * p.E, p.E, k, lane, s_e + wv * k,
                                 s_w + wv * k);
  } else if (threadIdx.x < T * k) {
    // routing given by the caller (idx/w already in memory)
    s_e[threadIdx.x] = p.idx[threadIdx.x];
    s_w[threadIdx.x] = p.w[threadIdx.x];
  }
  __syncthreads();
  if (p.logits && blockIdx.x == 0 && threadIdx.x < T * k) {
    p.idx[threadIdx.x] = s_e[threadIdx.x];
    p.w[threadIdx.x] = s_w[threadIdx.x];
  }

  const int tiles = (I + 15) / 16;
  const int units = T * k * tiles;
  const int s_lo = wv * R::L, s_hi = S;  // the wave's first group; the row's end
  const int NS = (S + kDecWaves * R::L - 1) / (kDecWaves * R::L);  // steps per unit
  auto unit_of = [&](int j) { return int(blockIdx.x) + j * int(gridDim.x); };
  if (unit_of(0) >= units) return;

  St st;
  st.ring = rings + wv * St::BYTES;
  // lookahead position (unit index j, step m) and its lane offsets
  int lj = 0, lm = 0;
  DecLane<BITS, J, 2> ln;
  auto lane_for = [&](int j) {
    const int u = unit_of(j);
    const int e = s_e[u / tiles];
    const uint8_t* const mat[2] = {p.gate + int64_t(e) * p.gu_stride,
                                   p.up + int64_t(e) * p.gu_stride};
    dec_lane<BITS, J, 2>(ln, mat, p.gu_meta_off, I, H, G, (u % tiles) * 16, s_lo, lane);
  };
  lane_for(0);
  auto issue_next = [&]() {
    if (unit_of(lj) >= units) return;
    dec_issue<BITS, J, 2>(ln, st.slot(st.issued), lm, lane);
    ++st.issued;
    if (++lm == NS) {
      lm = 0;
      ++lj;
      if (unit_of(lj) < units) lane_for(lj);
    }
  };
  for (int d = 0; d < St::DEPTH - 1; ++d) issue_next();
  stage_store(x0, 1, H, G, xp, xs, threadIdx.x, 512);
  lds_barrier();

  // The partial sums of up to kDecUB units wait in LDS and are added after
  // one barrier per batch, so the waves stream through the batch's units
  // without meeting.  Batches alternate between two buffers: batch b's sums
  // are read (by wave 0, after barrier b) before wave 0 reaches barrier b+1,
  // which every wave passes before writing batch b+2.
  auto finish_batch = [&](int j_last) {
    lds_barrier();
    const int b = j_last / kDecUB;
    const int nu = j_last % kDecUB + 1;
    if (wv == 0) {
      for (int q = lane >> 4; q < nu; q += 4) {
        const int r = lane & 15;
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
          gs += red[b & 1][q][w][0][r];
          us += red[b & 1][q][w][1][r];
        }
        const int uq = unit_of(b * kDecUB + q);
        const int n = (uq % tiles) * 16 + r;
        if (n < I) p.hbuf[int64_t(uq / tiles) * I + n] = silu(gs) * us;
      }
    }
  };
  int staged = 0;
  int j = 0;
  for (; unit_of(j) < units; ++j) {
    const int u = unit_of(j);
    const int slot_j = u / tiles, t = slot_j / k;
    if (t != staged) {
      if (j % kDecUB != 0) finish_batch(j - 1);  // the batch ends with the token
      lds_barrier();  // the previous token's parts are no longer read
      stage_parts(p.X + int64_t(t) * H, H, nullptr, 1, H, G, xp, xs, threadIdx.x, 512);
      lds_barrier();
      staged = t;
    }
    f32x4_t y[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    for (int m = 0; m < NS; ++m) {
      issue_next();  // into the slot computed in the previous iteration
      st.wait_oldest();
      const uint16_t* const xpa[2] = {xp, xp};
      const float4* const xsa[2] = {xs, xs};
      dec_step<BITS, J, 2, true>(st.slot(st.consumed), y, xpa, xsa, H, G, s_lo, s_hi, m, lane,
                                 zeros);
      ++st.consumed;
    }
    // rows 0 and 1 of the tile are the two parts of the token's product
    if (g4 == 0) {
      red[(j / kDecUB) & 1][j % kDecUB][wv][0][c] = y[0][0] + y[0][1];
      red[(j / kDecUB) & 1][j % kDecUB][wv][1][c] = y[1][0] + y[1][1];
    }
    if (j % kDecUB == kDecUB - 1) finish_batch(j);
  }
  if (j % kDecUB != 0) finish_batch(j - 1);
}

// ---------------------------------------------------------------------------
// down + combine: Y[t][n] = sum_i w[t][i] (h[t*k+i] . Wd_{idx[t][i]}[n]).
// Units (token t, 16-row tile of H) are dealt in a fixed stride; a workgroup
// stages the token's k activation parts, wave w streams the pieces w, w + 8,
// ... of I (L groups each) of the slots' tiles, NT slots per step (NT = 2:
// slots 2i and 2i + 1 together, the same rows of two experts, so a step
// carries 4 KB of codes per wave), weights each slot's partial sum by
// w[t][i] in slot order, and the eight waves' sums meet in LDS in a fixed
// order.
// ---------------------------------------------------------------------------
template <int BITS, int J, int NT>
__device__ __forceinline__ void dec_down_body(const DecArgs& p, int T, uint8_t* dsm) {
  using R = DecRing<BITS, J, NT>;
  using St = DecStream<BITS, J, NT, DSQ_DEC_DN_DEPTH>;
  __shared__ float red[kDecWaves][16];
  __shared__ __attribute__((aligned(16))) uint32_t zeros[4];
  __shared__ int32_t s_rows[32];
  __shared__ int32_t s_e[4 * 32];  // routing of the T tokens, read once
  __shared__ float s_w[4 * 32];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  const int H = p.H, I = p.I, G = p.group, S = I / G, k = p.k;
  uint8_t* rings = dsm;                                                       // [8][DEPTH][WSLOT]
  uint16_t* hp = reinterpret_cast<uint16_t*>(dsm + kDecWaves * St::BYTES);     // [k][2][I]
  float4* hs = reinterpret_cast<float4*>(dsm + kDecWaves * St::BYTES + int64_t(k) * 4 * I);
  if (threadIdx.x < 4) zeros[threadIdx.x] = 0u;
  // the first token's activations and the routing are loaded together; the
  // activations are converted once the first weight loads are in flight
  const int t_first = int(blockIdx.x) / ((H + 15) / 16);
  StageRegs h0;  // rows t_first*k .. + k of hbuf are consecutive
  stage_load(p.hbuf + int64_t(min(t_first, T - 1)) * k * I, I, nullptr, k, I, threadIdx.x, 512,
             h0);
  if (threadIdx.x < T * k) {
    s_e[threadIdx.x] = p.idx[threadIdx.x];
    s_w[threadIdx.x] = p.w[threadIdx.x];
  }
  __syncthreads();

  const int tiles = (H + 15) / 16;
  const int units = T * tiles;
  const int s_lo = wv * R::L, s_hi = S;  // the wave's first group; the row's end
  const int NS = (S + kDecWaves * R::L - 1) / (kDecWaves * R::L);  // steps per slot
  auto unit_of = [&](int j) { return int(blockIdx.x) + j * int(gridDim.x); };
  if (unit_of(0) >= units) return;

  St st;
  st.ring = rings + wv * St::BYTES;
  // lookahead position (unit j, slot group i of NT slots, step m)
  int lj = 0, li = 0, lm = 0;
  const int kg = k / NT;  // slot groups (NT divides k)
  DecLane<BITS, J, NT> ln;
  auto lane_for = [&](int j, int i) {
    const int u = unit_of(j);
    const int t = u / tiles;
    const uint8_t* mat[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) mat[b] = p.down + int64_t(s_e[t * k + NT * i + b]) * p.d_stride;
    const uint8_t* const (&cmat)[NT] = mat;
    dec_lane<BITS, J, NT>(ln, cmat, p.d_meta_off, H, I, G, (u % tiles) * 16, s_lo, lane);
  };
  lane_for(0, 0);
  auto issue_next = [&]() {
    if (unit_of(lj) >= units) return;
    uint8_t* const sp = st.ring + (st.issued % St::DEPTH) * R::WSLOT;
    dec_issue<BITS, J, NT>(ln, sp, lm, lane);
    ++st.issued;
    if (++lm == NS) {
      lm = 0;
      if (++li == kg) {
        li = 0;
        ++lj;
      }
      if (unit_of(lj) < units) lane_for(lj, li);
    }
  };
  for (int d = 0; d < St::DEPTH - 1; ++d) issue_next();
  stage_store(h0, k, I, G, hp, hs, threadIdx.x, 512);
  lds_barrier();

  int staged = t_first;
  for (int j = 0; unit_of(j) < units; ++j) {
    const int u = unit_of(j);
    const int t = u / tiles;
    if (t != staged) {
      lds_barrier();  // the previous token's parts are no longer read
      if (threadIdx.x < k) s_rows[threadIdx.x] = t * k + threadIdx.x;
      lds_barrier();
      stage_parts(p.hbuf, I, s_rows, k, I, G, hp, hs, threadIdx.x, 512);
      lds_barrier();
      staged = t;
    }
    float yacc = 0.0f;
    for (int i = 0; i < kg; ++i) {
      f32x4_t y[NT];
      const uint16_t* xpa[NT];
      const float4* xsa[NT];
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        y[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        xpa[b] = hp + int64_t(NT * i + b) * 2 * I;
        xsa[b] = hs + int64_t(NT * i + b) * S;
      }
      const uint16_t* const (&cxp)[NT] = xpa;
      const float4* const (&cxs)[NT] = xsa;
      for (int m = 0; m < NS; ++m) {
        issue_next();  // into the slot computed in the previous iteration
        st.wait_oldest();
        dec_step<BITS, J, NT, false>(st.slot(st.consumed), y, cxp, cxs, I, G, s_lo, s_hi, m,
                                     lane, zeros);
        ++st.consumed;
      }
      // the slots' products are weighted and added in slot order
#pragma unroll
      for (int b = 0; b < NT; ++b) yacc = fmaf(s_w[t * k + NT * i + b], y[b][0] + y[b][1], yacc);
    }
    if (g4 == 0) red[wv][c] = yacc;
    lds_barrier();
    if (wv == 0 && lane < 16) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) v += red[w][lane];
      const int nn = (u % tiles) * 16 + lane;
      if (nn < H) {
        // the residual is read and Y written by the same lane, so Y may be
        // the residual itself
        if (p.resid) v = p.resid[int64_t(t) * H + nn] + v;
        p.Y[int64_t(t) * H + nn] = v;
      }
    }
    lds_barrier();
  }
}

template <int BITS, int J, int NT>
__global__ __launch_bounds__(512) void dec_down_kernel(DecArgs p, int T) {
  // The body is compiled for the device only: the host pass (which only
  // needs the launch stub) rejects its ring-load helper for the two-tile
  // instances.
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  dec_down_body<BITS, J, NT>(p, T, dsm);
#endif
}

namespace {

// dynamic LDS a down kernel may take: 160 KiB less its static tables
constexpr int kDecDownLdsMax = 160 * 1024 - 2048;

template <int BITS, int J, int NT>
hipError_t launch_down(const DecArgs& a, int64_t T, unsigned blocks, size_t lds,
                       hipStream_t stream) {
  // more than 64 KiB of dynamic LDS must be granted to the kernel explicitly
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dec_down_kernel<BITS, J, NT>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dec_down_kernel<BITS, J, NT>), dim3(blocks), dim3(512), lds, stream, a,
                     int(T));
  return hipGetLastError();
}

template <int BITS, int J>
hipError_t go_decode(const DecArgs& a, int64_t T, hipStream_t stream) {
  const int64_t gu_units = T * a.k * ((a.I + 15) / 16);
  const unsigned gb = unsigned(gu_units < 256 ? gu_units : 256);
  const size_t gu_lds = size_t(kDecWaves) * DecStream<BITS, J, 2, DSQ_DEC_GU_DEPTH>::BYTES +
                        size_t(4) * a.H +
                        size_t(a.H / a.group) * 16;
  // more than 64 KiB of dynamic LDS must be granted to the kernel explicitly
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dec_gateup_kernel<BITS, J>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(gu_lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dec_gateup_kernel<BITS, J>), dim3(gb), dim3(512), gu_lds, stream, a,
                     int(T));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t dn_units = T * ((a.H + 15) / 16);
  const unsigned db = unsigned(dn_units < 256 ? dn_units : 256);
  const size_t parts = size_t(a.k) * 4 * a.I + size_t(a.k) * (a.I / a.group) * 16;
  // INT4: slot pairs per step when k is even and their ring fits beside the
  // parts (one token, top-6: 0.5-0.65 us less per layer; INT8 measured
  // 0.7 us slower with pairs, so it keeps one slot per step)
  const size_t dn_lds2 = size_t(kDecWaves) * DecStream<BITS, J, 2, DSQ_DEC_DN_DEPTH>::BYTES + parts;
  if constexpr (BITS == 4)
    if (a.k % 2 == 0 && dn_lds2 <= size_t(kDecDownLdsMax))
      return launch_down<BITS, J, 2>(a, T, db, dn_lds2, stream);
  return launch_down<BITS, J, 1>(
      a, T, db, size_t(kDecWaves) * DecStream<BITS, J, 1, DSQ_DEC_DN_DEPTH>::BYTES + parts, stream);
}

}  // namespace

// True when the decode kernels apply: the wave rings plus one token's
// activation parts (gate/up) or its k activation parts (down) fit LDS, the
// scores of a token fit one wave's registers and k fits the rank tables.
bool decode_supported(int bits, int64_t H, int64_t I, int32_t E, int32_t k) {
  if (bits != 4 && bits != 8) return false;
  // largest rings over the supported groupings (at most 4 groups per step)
  constexpr int64_t kGuSlot = 2 * 2048 + 2 * 16 * 4 * 8, kDnSlot = 2048 + 16 * 4 * 8;
  const int64_t gu_ring = int64_t(kDecWaves) * DSQ_DEC_GU_DEPTH * kGuSlot;
  const int64_t dn_ring = int64_t(kDecWaves) * DSQ_DEC_DN_DEPTH * kDnSlot;
  const int64_t gu = gu_ring + 4 * H + (H / 64) * 16;
  const int64_t dn = dn_ring + int64_t(k) * (4 * I + (I / 64) * 16);
  // 160 KiB less each kernel's static tables
  const int64_t gu_static = int64_t(sizeof(float)) * 2 * kDecUB * kDecWaves * 2 * 16 + 2048;
  const int64_t dn_static = 2048;
  return E <= kDecodeMaxE && k <= 32 && gu <= 160 * 1024 - gu_static &&
         dn <= 160 * 1024 - dn_static && stage_one_pass(1, H, 512) && stage_one_pass(k, I, 512);
}

hipError_t launch_moe_decode(const dsq_qweight& gate, const dsq_qweight& up,
                             const dsq_qweight& down, const float* X, int64_t T, int32_t E,
                             int32_t k, const float* logits, int32_t* idx, float* w, float* hbuf,
                             float* Y, const float* resid, hipStream_t stream) {
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
  a.resid = resid;
  const bool g64 = gate.group == 64;
  if (gate.bits == 8) return g64 ? go_decode<8, 2>(a, T, stream) : go_decode<8, 4>(a, T, stream);
  return g64 ? go_decode<4, 2>(a, T, stream) : go_decode<4, 4>(a, T, stream);
}

}  // namespace dsq
