// gmm.hip -- grouped fused-dequant GEMM on bf16 MFMA for the tokens routed
// to each expert (batched decode and prefill of the routed MoE FFN).
//
// Method: "Hand-writing a DeepSeek inference engine in pure C"
// (hnwysp.cn/news/134870) §3.2 (dequantize inside the matmul loop, value =
// (q - zero_point) * scale per group), §3.3 (the matmul), §3.5 (gather the
// tokens routed to one expert and run the expert once over all of them, so
// its weights are read once per layer).  The SwiGLU expert form is the
// workload's definition.
//
// The expert weights are streamed once; the tokens of an expert are few
// (1..16 per pass), so the kernel is bound by HBM, and the dequantization
// work per weight must stay small.  v_mfma_f32_16x16x32_bf16 does the
// multiply-adds with
//   A (16 x 32) = activation rows of one token tile ("parts", below),
//   B (32 x 16) = weight codes of 16 weight rows, as exact bf16 integers,
// and the group's zero point and scale are applied in fp32 afterwards:
//   sum_k x[k] (q[k] - zp) s = s * (sum_k x[k] (q[k] + o) - (zp + o) sum_k x[k])
// with o = 16 for INT4 (the code is built as bf16(16 + q) by two byte
// permutes per 4 codes: bf16 0x4180 | q << 3) and o = 0 for INT8 (bf16(q)).
// Both products and the group sums in the MFMA are exact or carry fp32
// rounding only.
//
// Activations: the fp32 path splits every activation into two bf16 parts,
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (|x - hi - lo| <= 2^-18 |x|),
// each part its own MFMA row, and adds the two rows' results at the end; the
// bf16 path uses hi only.  A prep kernel writes the parts of every token tile
// in MFMA operand order (one 16-byte load per lane and k step) together with
// the per-group sums of each part row, which the zero-point term needs.
//
// Lane l of a wave supplies A row l % 16 and B column l % 16 for k slice
// l / 16 of every MFMA.  Within a quantization group of G = 32 J weights the
// lane's k range is the contiguous [8 J (l / 16), 8 J (l / 16) + 8 J): MFMA j
// of the group takes its 8-k piece j.  The output lane l holds column l % 16
// (one weight row: its scale and zero point are the lane's own) and rows
// 4 (l / 16) + i, i < 4.
//
// Work: a wave owns NB B tiles (SwiGLU: NB/2 gate tiles and the NB/2 up
// tiles of the same rows, so silu(g) u is formed in the lane) of one expert
// and streams the expert's codes of those rows over all of K, D quantization
// groups ahead; it processes up to NT token tiles per pass.  Waves take items
// (expert, row block) in a fixed stride so every wave gets the same count to
// within one item.
#include "common.h"
#include "internal.h"

namespace dsq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Raw buffer resource over [base, base + bytes): 32-bit lane offsets plus a
// wave-uniform offset, no 64-bit address arithmetic per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0x7fffffff ? bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(n), 0x00020000);
}

#ifndef DSQ_GMM_CODE_AUX
#define DSQ_GMM_CODE_AUX 0
#endif
constexpr int kNT = 0;                    // aux: default caching
// Codes use default caching: a 16-row tile takes 32-128 B of each row per
// group, and the rest of the 128-byte line is used by the next groups; a
// nontemporal hint drops it from L2 before they come.
constexpr int kStream = DSQ_GMM_CODE_AUX;

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 8 INT4 codes of one word of the packed layout (byte i: low nibble k = i,
// high nibble k = 4 + i) -> bf16(16 + q) for k = 0..7.
__device__ __forceinline__ u32x4_t int4_to_bf16(uint32_t w) {
  const uint32_t lo = ((w << 3) & 0x78787878u) | 0x80808080u;
  const uint32_t hi = ((w >> 1) & 0x78787878u) | 0x80808080u;
  u32x4_t d;
  d[0] = __builtin_amdgcn_perm(0x41414141u, lo, 0x04010400u);
  d[1] = __builtin_amdgcn_perm(0x41414141u, lo, 0x04030402u);
  d[2] = __builtin_amdgcn_perm(0x41414141u, hi, 0x04010400u);
  d[3] = __builtin_amdgcn_perm(0x41414141u, hi, 0x04030402u);
  return d;
}

// 8 INT8 codes (two words, k = 0..7 in byte order) -> bf16(q).
__device__ __forceinline__ u32x4_t int8_to_bf16(uint32_t w0, uint32_t w1) {
  u32x4_t d;
  d[0] = pk_bf16(float(w0 & 0xffu), float((w0 >> 8) & 0xffu));
  d[1] = pk_bf16(float((w0 >> 16) & 0xffu), float(w0 >> 24));
  d[2] = pk_bf16(float(w1 & 0xffu), float((w1 >> 8) & 0xffu));
  d[3] = pk_bf16(float((w1 >> 16) & 0xffu), float(w1 >> 24));
  return d;
}

}  // namespace

// ---------------------------------------------------------------------------
// Activation prep: token tiles of 16 part rows, per quantization group s and
// MFMA j, 64 lanes x 8 bf16 (lane = 16 * kslice + row), and the fp32 sums of
// each part row over each group.
// ---------------------------------------------------------------------------
struct GmmPrepArgs {
  const float* src;
  int64_t ld_src;
  int xrows;                // XR_DENSE / XR_GATHER / XR_SEGMENT
  const int32_t* perm;
  int top_k;
  const int32_t* active;    // NULL: dense
  const int32_t* n_active;
  const int32_t* offsets;
  int64_t M;                // dense rows
  int K, group;
  uint4* afrag;
  float* xs;
};

template <int XP>
__global__ __launch_bounds__(256) void gmm_prep_kernel(GmmPrepArgs p) {
  constexpr int TPT = 16 / XP;     // tokens per tile
  constexpr int SEGS = 256 / TPT;  // 8-wide k segments per block
  int64_t p0, M;
  int tb;
  if (p.active) {
    const int a = blockIdx.y;
    if (a >= *p.n_active) return;
    const int e = p.active[a];
    p0 = p.offsets[e];
    M = p.offsets[e + 1] - p0;
    tb = int(p0 * XP / 16) + a;
  } else {
    p0 = 0;
    M = p.M;
    tb = 0;
  }
  const int tok = threadIdx.x / SEGS, seg = threadIdx.x % SEGS;
  const int k = (blockIdx.x * SEGS + seg) * 8;
  // K is a multiple of the group and segments are group-aligned, so the lanes
  // that reduce one group below leave or stay together
  if (k >= p.K) return;
  const int G = p.group, J = G / 32, S = p.K / G;
  const int s = k / G, kk = k % G;
  const int g4 = kk / (8 * J), j = (kk % (8 * J)) / 8;
  const int ntiles = int((M * XP + 15) / 16);
  for (int t = 0; t < ntiles; ++t) {
    const int64_t m = int64_t(t) * TPT + tok;
    float v[8];
    if (m < M) {
      int64_t row;
      if (p.xrows == XR_GATHER) row = p.perm[p0 + m] / p.top_k;
      else if (p.xrows == XR_SEGMENT) row = p0 + m;
      else row = m;
      const float4* q = reinterpret_cast<const float4*>(p.src + row * p.ld_src + k);
      const float4 a = q[0], b = q[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    uint32_t hw[4], lw[4];
    double sh = 0.0, sl = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h0 = __bf16(v[2 * i]), h1 = __bf16(v[2 * i + 1]);
      hw[i] = uint32_t(__builtin_bit_cast(uint16_t, h0)) |
              (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
      sh += double(float(h0)) + double(float(h1));
      if constexpr (XP == 2) {
        const __bf16 l0 = __bf16(v[2 * i] - float(h0)), l1 = __bf16(v[2 * i + 1] - float(h1));
        lw[i] = uint32_t(__builtin_bit_cast(uint16_t, l0)) |
                (uint32_t(__builtin_bit_cast(uint16_t, l1)) << 16);
        sl += double(float(l0)) + double(float(l1));
      }
    }
    // sum over the G/8 lanes of this group (consecutive lanes)
    for (int o = 1; o < G / 8; o <<= 1) {
      sh += __shfl_xor(sh, o);
      if constexpr (XP == 2) sl += __shfl_xor(sl, o);
    }
    const int64_t blk = (int64_t(tb + t) * S + s);
#pragma unroll
    for (int part = 0; part < XP; ++part) {
      const int R = tok * XP + part;
      const uint32_t* w = part ? lw : hw;
      p.afrag[(blk * J + j) * 64 + g4 * 16 + R] = make_uint4(w[0], w[1], w[2], w[3]);
      if (kk == 0) p.xs[blk * 16 + R] = float(part ? sl : sh);
    }
  }
}

// ---------------------------------------------------------------------------
// The grouped GEMM.
// ---------------------------------------------------------------------------
struct GmmArgs {
  const uint8_t* wa;        // matrix (SwiGLU: gate), entry 0
  const uint8_t* wb;        // SwiGLU up, entry 0
  int64_t stride;           // bytes per entry
  int64_t meta_off;         // offset of the (scale, zp) table in an entry
  int N, K, group;
  int64_t expert;           // dense mode entry
  const int32_t* active;    // NULL: dense
  const int32_t* n_active;
  const int32_t* offsets;
  int64_t M;                // dense rows
  const uint4* afrag;
  int64_t afrag_bytes;
  const float* xs;
  int64_t xs_bytes;
  float* out;
  int64_t ld_out;
  int rt;                   // row blocks (items) per expert
};

// Wave-uniform state of one item (expert, row block).
struct GmmItem {
  __amdgpu_buffer_rsrc_t rca, rma, rcb, rmb;  // codes / metadata of A and B
  int64_t p0, M;                              // routed rows of the expert
  int tb;                                     // its first token tile
  int n0;                                     // first output row
};

// One pass over K for the NTT token tiles starting at tile t0 of the item.
template <int BITS, int J, int XP, int NB, int NTT, int D, bool SWIGLU>
__device__ __forceinline__ void gmm_pass(const GmmArgs& p, const GmmItem& it,
                                         __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rx,
                                         const int (&voc)[NB], const int (&vom)[NB], int t0) {
  constexpr int TPT = 16 / XP;
  constexpr float kOff = BITS == 4 ? 16.0f : 0.0f;
  constexpr int CW = J * BITS / 4;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g4 = lane >> 4;
  const int G = p.group, S = p.K / G;
  int voa[NTT], vox[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
    const int tile = it.tb + t0 + t;
    voa[t] = tile * S * J * 1024 + lane * 16;
    vox[t] = tile * S * 64 + g4 * 16;
  }
  f32x4_t y[NB][NTT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int t = 0; t < NTT; ++t) y[b][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ring of D groups of codes and metadata; activations one group ahead
  uint32_t cw[D][NB][CW];
  f32x2_t mt[D][NB];
  auto load_codes = [&](int s, uint32_t (&w)[NB][CW], f32x2_t (&m)[NB]) {
    const int so = s * (G * BITS / 8);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const __amdgpu_buffer_rsrc_t rc = (SWIGLU && b >= NB / 2) ? it.rcb : it.rca;
      const __amdgpu_buffer_rsrc_t rm = (SWIGLU && b >= NB / 2) ? it.rmb : it.rma;
      if constexpr (CW == 2) {
        const u32x2_t v = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rc, voc[b], so, kStream));
        w[b][0] = v[0];
        w[b][1] = v[1];
      } else {
#pragma unroll
        for (int h = 0; h < CW / 4; ++h) {
          const u32x4_t v = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, voc[b] + 16 * h, so, kStream));
#pragma unroll
          for (int i = 0; i < 4; ++i) w[b][4 * h + i] = v[i];
        }
      }
      m[b] = __builtin_bit_cast(f32x2_t,
                                __builtin_amdgcn_raw_buffer_load_b64(rm, vom[b], s * 8, kNT));
    }
  };
  u32x4_t af[2][NTT][J];
  f32x4_t xsum[2][NTT];
  auto load_act = [&](int s, u32x4_t (&A)[NTT][J], f32x4_t (&X)[NTT]) {
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        A[t][j] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, voa[t] + j * 1024, s * J * 1024,
                                                           kNT));
      X[t] = __builtin_bit_cast(f32x4_t,
                                __builtin_amdgcn_raw_buffer_load_b128(rx, vox[t], s * 64, kNT));
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load_codes(min(d, S - 1), cw[d], mt[d]);
  load_act(0, af[0], xsum[0]);

  for (int s0 = 0; s0 < S; s0 += 2 * D) {
#pragma unroll
    for (int u = 0; u < 2 * D; ++u) {
      const int s = s0 + u;
      if (s >= S) break;
      const int d = u % D, cur = u & 1;
      load_act(min(s + 1, S - 1), af[cur ^ 1], xsum[cur ^ 1]);
      f32x4_t acc[NB][NTT];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        u32x4_t bq[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
          if constexpr (BITS == 4) bq[j] = int4_to_bf16(cw[d][b][j]);
          else bq[j] = int8_to_bf16(cw[d][b][2 * j], cw[d][b][2 * j + 1]);
        }
#pragma unroll
        for (int t = 0; t < NTT; ++t) {
          acc[b][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < J; ++j)
            acc[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, af[cur][t][j]), __builtin_bit_cast(bf16x8_t, bq[j]),
                acc[b][t], 0, 0, 0);
        }
      }
      // zero point and scale of the group, in fp32, after all MFMAs are issued
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float sc = mt[d][b][0];
        const float zq = mt[d][b][1] + kOff;
#pragma unroll
        for (int t = 0; t < NTT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            y[b][t][i] = fmaf(sc, fmaf(-zq, xsum[cur][t][i], acc[b][t][i]), y[b][t][i]);
      }
      load_codes(min(s + D, S - 1), cw[d], mt[d]);
    }
  }

  // epilogue: rows 4 g4 + i of tile t are parts of this lane's tokens
#pragma unroll
  for (int t = 0; t < NTT; ++t) {
#pragma unroll
    for (int q = 0; q < 4 / XP; ++q) {
      const int64_t m = int64_t(t0 + t) * TPT + g4 * (4 / XP) + q;
      if (m >= it.M) continue;
      const int64_t orow = p.active ? it.p0 + m : m;
      float* o = p.out + orow * p.ld_out;
#pragma unroll
      for (int b = 0; b < (SWIGLU ? NB / 2 : NB); ++b) {
        const int n = it.n0 + b * 16 + c;
        if (n >= p.N) continue;
        float v = XP == 2 ? y[b][t][2 * q] + y[b][t][2 * q + 1] : y[b][t][q];
        if constexpr (SWIGLU) {
          const int bu = b + NB / 2;
          const float u = XP == 2 ? y[bu][t][2 * q] + y[bu][t][2 * q + 1] : y[bu][t][q];
          v = silu(v) * u;
        }
        o[n] = v;
      }
    }
  }
}

template <int BITS, int J, int XP, int NB, int NT, int D, bool SWIGLU>
__global__ __launch_bounds__(256) void gmm_kernel(GmmArgs p) {
  constexpr int ROWS = SWIGLU ? NB / 2 * 16 : NB * 16;  // output rows per item
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g4 = lane >> 4;
  const int nw = gridDim.x * 4;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // item decode and the buffer descriptors in scalar registers
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.K / p.group;
  const int64_t RB = int64_t(p.K) * BITS / 8;
  const int items = (p.active ? *p.n_active : 1) * p.rt;
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.afrag, p.afrag_bytes);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.xs, p.xs_bytes);

  for (int item = gw; item < items; item += nw) {
    const int a = item / p.rt, rblk = item % p.rt;
    GmmItem it;
    int64_t e;
    if (p.active) {
      e = p.active[a];
      it.p0 = p.offsets[e];
      it.M = p.offsets[e + 1] - it.p0;
      it.tb = int(it.p0 * XP / 16) + a;
    } else {
      e = p.expert;
      it.p0 = 0;
      it.M = p.M;
      it.tb = 0;
    }
    const uint8_t* ea = p.wa + e * p.stride;
    const uint8_t* eb = SWIGLU ? p.wb + e * p.stride : ea;
    const int64_t cbytes = int64_t(p.N) * RB, mbytes = int64_t(p.N) * S * 8;
    it.rca = rsrc(ea, cbytes);
    it.rma = rsrc(ea + p.meta_off, mbytes);
    it.rcb = rsrc(eb, cbytes);
    it.rmb = rsrc(eb + p.meta_off, mbytes);
    it.n0 = rblk * ROWS;
    int voc[NB], vom[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int nb = it.n0 + (SWIGLU ? (b % (NB / 2)) : b) * 16 + c;
      const int n = min(nb, p.N - 1);
      voc[b] = int(int64_t(n) * RB) + g4 * J * BITS;
      vom[b] = n * S * 8;
    }
    const int ntiles = int((it.M * XP + 15) / 16);
    int t0 = 0;
    for (; t0 + NT <= ntiles; t0 += NT)
      gmm_pass<BITS, J, XP, NB, NT, D, SWIGLU>(p, it, ra, rx, voc, vom, t0);
    if constexpr (NT > 1) {
      for (; t0 < ntiles; ++t0) gmm_pass<BITS, J, XP, NB, 1, D, SWIGLU>(p, it, ra, rx, voc, vom, t0);
    }
  }
}

namespace {

int tiles_bound(int64_t rows, int64_t segments, int xp) {
  return int(rows * xp / 16 + segments + 1);
}

template <int BITS, int J, int XP, bool SWIGLU>
hipError_t launch_one(const GmmArgs& a, int max_items, hipStream_t stream) {
  constexpr int NB = 4;
  constexpr int NT = XP == 2 ? 2 : 1;
  constexpr int D = J * BITS <= 16 ? 4 : 2;
  const int64_t total = int64_t(max_items) * a.rt;
  // every wave gets the same number of items to within one
  int64_t waves = total < 2048 ? total : 2048;
  const unsigned blocks = unsigned((waves + 3) / 4);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gmm_kernel<BITS, J, XP, NB, NT, D, SWIGLU>), dim3(blocks), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <int XP>
hipError_t launch_bits(const GmmArgs& a, int bits, bool swiglu, int max_items,
                       hipStream_t stream) {
  const int J = a.group / 32;
  if (bits == 4 && J == 2)
    return swiglu ? launch_one<4, 2, XP, true>(a, max_items, stream)
                  : launch_one<4, 2, XP, false>(a, max_items, stream);
  if (bits == 4 && J == 4)
    return swiglu ? launch_one<4, 4, XP, true>(a, max_items, stream)
                  : launch_one<4, 4, XP, false>(a, max_items, stream);
  if (bits == 8 && J == 2)
    return swiglu ? launch_one<8, 2, XP, true>(a, max_items, stream)
                  : launch_one<8, 2, XP, false>(a, max_items, stream);
  return swiglu ? launch_one<8, 4, XP, true>(a, max_items, stream)
                : launch_one<8, 4, XP, false>(a, max_items, stream);
}

}  // namespace

size_t gmm_act_bytes(int64_t rows, int64_t segments, int xp, int64_t K) {
  const int64_t tiles = tiles_bound(rows, segments, xp);
  return size_t(align256(tiles * K * 32));
}

size_t gmm_xs_bytes(int64_t rows, int64_t segments, int xp, int64_t K, int group) {
  const int64_t tiles = tiles_bound(rows, segments, xp);
  return size_t(align256(tiles * (K / group) * 64));
}

hipError_t launch_gmm(const dsq_qweight& A, const dsq_qweight* B, int64_t expert,
                      const Groups* grp, int xrows, const float* X, int64_t ld_x, int64_t M,
                      int xp, void* act, size_t act_bytes, float* xs, size_t xs_bytes,
                      float* out, int64_t ld_out, hipStream_t stream) {
  const Layout L = layout_of(A.bits, A.group, A.K, A.N);
  // (1) activations in operand order
  GmmPrepArgs pa{};
  pa.src = X;
  pa.ld_src = ld_x;
  pa.xrows = xrows;
  pa.K = int(A.K);
  pa.group = A.group;
  pa.afrag = static_cast<uint4*>(act);
  pa.xs = xs;
  pa.M = M;
  int items = 1;
  if (grp) {
    pa.perm = grp->perm;
    pa.top_k = grp->top_k;
    pa.active = grp->active;
    pa.n_active = grp->n_active;
    pa.offsets = grp->offsets;
    items = grp->max_items;
  }
  if (items == 0) return hipSuccess;
  const int segs = xp == 2 ? 32 : 16;
  const dim3 pgrid(unsigned((A.K / 8 + segs - 1) / segs), unsigned(items));
  if (xp == 2) hipLaunchKernelGGL(gmm_prep_kernel<2>, pgrid, dim3(256), 0, stream, pa);
  else hipLaunchKernelGGL(gmm_prep_kernel<1>, pgrid, dim3(256), 0, stream, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // (2) the GEMM
  GmmArgs a{};
  a.wa = static_cast<const uint8_t*>(A.data);
  a.wb = B ? static_cast<const uint8_t*>(B->data) : nullptr;
  a.stride = L.stride;
  a.meta_off = L.meta_off;
  a.N = int(A.N);
  a.K = int(A.K);
  a.group = A.group;
  a.expert = expert;
  a.M = M;
  if (grp) {
    a.active = grp->active;
    a.n_active = grp->n_active;
    a.offsets = grp->offsets;
  }
  a.afrag = static_cast<const uint4*>(act);
  a.afrag_bytes = int64_t(act_bytes);
  a.xs = xs;
  a.xs_bytes = int64_t(xs_bytes);
  a.out = out;
  a.ld_out = ld_out;
  const int rows = B ? 32 : 64;  // output rows per item (NB = 4 tiles of 16)
  a.rt = int((A.N + rows - 1) / rows);
  if (xp == 2) return launch_bits<2>(a, A.bits, B != nullptr, items, stream);
  return launch_bits<1>(a, A.bits, B != nullptr, items, stream);
}

}  // namespace dsq
