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
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (|x - hi - lo| <= 2^-17 |x|:
// bf16 keeps 8 significant bits, so each round-to-nearest step leaves at most
// 2^-8 of its input, and the second input is itself at most 2^-8 |x|, with
// one bit to spare from the exponent step),
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
// Work: a workgroup item is one pass of one token tile of one expert over
// 128 (SwiGLU: 128 gate and 128 up) or 256 output rows.  Each wave streams the codes of its two 16-row tiles (SwiGLU: the gate and
// the up tile of the same rows, so silu(g) u is formed in the lane) straight
// from HBM into its own LDS ring, 128 bytes of every row per step (whole cache
// lines; a 16-row operand only needs 32 bytes of a row per INT4 group), and
// the workgroup shares a ring of the token tile's activation fragments.  Three
// steps are in flight.  The routing step lists the token tiles of every
// expert; items are dealt to the workgroups in a fixed stride, so every
// workgroup runs the same number of passes to within one whatever the
// routing (an expert with many tokens is many items, not one long one).
#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace dsq {


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
  const int4* tiles;        // NULL: dense; else the token-tile table
  const int32_t* n_tiles;
  int64_t M;                // dense rows
  int K, group;
  uint4* afrag;
  float* xs;
};

template <int XP>
__global__ __launch_bounds__(256) void gmm_prep_kernel(GmmPrepArgs p) {
  constexpr int TPT = 16 / XP;     // tokens per tile
  constexpr int SEGS = 256 / TPT;  // 8-wide k segments per block
  const int tok = threadIdx.x / SEGS, seg = threadIdx.x % SEGS;
  const int k = (blockIdx.x * SEGS + seg) * 8;
  // K is a multiple of the group and segments are group-aligned, so the lanes
  // that reduce one group below leave or stay together
  if (k >= p.K) return;
  const int G = p.group, J = G / 32, S = p.K / G;
  const int s = k / G, kk = k % G;
  const int g4 = kk / (8 * J), j = (kk % (8 * J)) / 8;
  // token tiles: blockIdx.y, blockIdx.y + gridDim.y, ...
  const int ntiles = p.tiles ? *p.n_tiles : int((p.M * XP + 15) / 16);
  for (int q = blockIdx.y; q < ntiles; q += gridDim.y) {
    int64_t row0;
    int rows, atile;
    if (p.tiles) {
      const int4 v = p.tiles[q];
      row0 = v.y;
      rows = v.z;
      atile = v.w;
    } else {
      row0 = int64_t(q) * TPT;
      rows = int(min(int64_t(TPT), p.M - row0));
      atile = q;
    }
    float v[8];
    if (tok < rows) {
      const int64_t m = row0 + tok;
      const int64_t row = p.xrows == XR_GATHER ? p.perm[m] / p.top_k : m;
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
    const int64_t blk = (int64_t(atile) * S + s);
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
  const int4* tiles;        // NULL: dense; else the token-tile table (Groups::tiles)
  const int32_t* n_tiles;
  int64_t M;                // dense rows
  const uint4* afrag;
  int64_t afrag_bytes;
  const float* xs;
  int64_t xs_bytes;
  float* out;
  int64_t ld_out;
  int rt;                   // row blocks per token tile
};

// Chunk swizzle of the code tiles in LDS: 16-byte chunk j of row r sits at
// position j ^ swz(r), so the 16 rows an MFMA operand read touches fall on
// distinct banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int BITS, int J, bool SWIGLU>
#ifndef DSQ_GMM_DM
#define DSQ_GMM_DM 3
#endif
struct GmmShape {
  static constexpr int W = 8;                       // waves per workgroup
  static constexpr int NB = 2;                      // B tiles (16 rows) per wave
  static constexpr int L = 1024 / (J * 32 * BITS);  // groups per 128 code bytes of a row
  static constexpr int DM = DSQ_GMM_DM;             // ring depth in steps of L groups
  static constexpr int CSLOT = NB * 16 * 128;       // one step of a wave's codes
  static constexpr int MSLOT = NB * 16 * L * 8;     // one step of a wave's (scale, zp)
  static constexpr int PPR = L >= 2 ? L / 2 : 2;    // direct-load pieces per metadata row
  static constexpr int PB = L >= 2 ? 16 : 4;        // bytes per piece
  static constexpr int WSLOT = CSLOT + MSLOT;
  static constexpr int AFR = L * J * 1024;          // one step of activation fragments
  static constexpr int ASLOT = AFR + L * 64;        // + their group sums
  static constexpr int PER_STEP = 3 * NB + 2;       // direct loads per wave and step
  static constexpr int LDS = W * DM * WSLOT + DM * ASLOT;
  static constexpr int ROWS = SWIGLU ? W * 16 : W * NB * 16;  // output rows per item
  static_assert(L * J <= 8, "one fragment load per wave and step");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Position in a workgroup's sequence of passes.  An item is one pass: one
// token tile of one expert against ROWS output rows, MS steps over K.  Items
// are numbered (tile, row block), the tiles in table order, and dealt in a
// fixed stride, so every workgroup runs the same number of passes to within
// one however the tokens fall on the experts.
struct GmmCursor {
  int j;           // position in the workgroup's item sequence
  int item;        // global item index (>= items: exhausted)
  int m;           // step within the pass
  int atile;       // activation tile
  int rows;        // token rows of the tile
  int64_t e, row0; // expert; first output row (perm order, or dense row)
};

// Item j of this workgroup.  Workgroup b runs on XCD b % 8; the workgroups of
// one XCD take consecutive items (every row block of one or two token tiles)
// at the same time, so that XCD's L2 fetches those activation tiles once, and
// the weight rows of an expert's tiles together.
__device__ __forceinline__ int gmm_item(int j) {
  const int nb = gridDim.x, b = blockIdx.x;
  if (nb % 8 != 0) return b + j * nb;
  const int per = nb / 8;  // workgroups per XCD
  return (j * 8 + b % 8) * per + b / 8;
}

// The routing tables are read through the constant address space: with a
// workgroup-uniform index these become scalar loads, which do not queue behind
// the weight stream's outstanding vector loads (a vector load here would wait
// for the whole lookahead to land).  The tables are written before the kernel
// starts and never during it.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

template <int XP>
__device__ __forceinline__ int gmm_items(const GmmArgs& p) {
  const int tiles = p.tiles ? __builtin_amdgcn_readfirstlane(*(const_i32_ptr)p.n_tiles)
                            : int((p.M * XP + 15) / 16);
  return tiles * p.rt;
}

template <int XP>
__device__ __forceinline__ void gmm_cursor_load(const GmmArgs& p, int items, GmmCursor& cu) {
  constexpr int TPT = 16 / XP;
  cu.item = gmm_item(cu.j);
  cu.m = 0;
  if (cu.item >= items) return;
  const int q = cu.item / p.rt;
  if (p.tiles) {
    const const_i32_ptr v = (const_i32_ptr)p.tiles + 4 * int64_t(q);
    cu.e = __builtin_amdgcn_readfirstlane(v[0]);
    cu.row0 = __builtin_amdgcn_readfirstlane(v[1]);
    cu.rows = __builtin_amdgcn_readfirstlane(v[2]);
    cu.atile = __builtin_amdgcn_readfirstlane(v[3]);
  } else {
    cu.e = p.expert;
    cu.row0 = int64_t(q) * TPT;
    cu.rows = int(min(int64_t(TPT), p.M - cu.row0));
    cu.atile = q;
  }
}

// Advance by one step; returns true when a new item begins.
template <int XP>
__device__ __forceinline__ bool gmm_cursor_next(const GmmArgs& p, int items, int MS,
                                                GmmCursor& cu) {
  if (++cu.m < MS) return false;
  ++cu.j;
  gmm_cursor_load<XP>(p, items, cu);
  return true;
}

// The whole streaming loop of one workgroup.  Wave w streams the codes and
// (scale, zp) of its NB tiles (SwiGLU: the gate and the up tile of the same
// 16 rows) 128 code bytes of every row per step (L groups; whole cache lines)
// into its own LDS ring by direct global->LDS loads, and the workgroup shares
// a ring of the token tile's activation fragments and group sums.  The ring
// runs on across passes and items: a lookahead cursor issues the loads two
// steps ahead of the compute cursor, wherever those steps fall.  One barrier
// per step releases the oldest slot; nothing but the direct loads is
// outstanding across a step, so the waits are the explicit ones below.
template <int BITS, int J, int XP, bool SWIGLU>
__device__ __forceinline__ void gmm_stream(const GmmArgs& p, uint8_t* sm) {
  using Sh = GmmShape<BITS, J, SWIGLU>;
  constexpr int NB = Sh::NB, L = Sh::L, DM = Sh::DM;
  constexpr int LB = J * BITS;  // code bytes per lane, tile and group
  constexpr float kOff = BITS == 4 ? 16.0f : 0.0f;
  static_assert(DM >= 2 && DM <= 4, "waits below");
  constexpr int A = DM - 1;  // steps issued ahead of the one computed
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g4 = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* const wring = sm + wv * DM * Sh::WSLOT;
  uint8_t* const aring = sm + Sh::W * DM * Sh::WSLOT;
  const int G = p.group, S = p.K / G;
  const int MS = (S + L - 1) / L;  // steps over K
  const int64_t RB = int64_t(p.K) * BITS / 8;
  const int items = gmm_items<XP>(p);
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.afrag, p.afrag_bytes);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.xs, p.xs_bytes);
  const bool mlane = lane < 16 * Sh::PPR;
  auto wrow_of = [&](int item) {
    return (item % p.rt) * Sh::ROWS + wv * (SWIGLU ? 16 : NB * 16);
  };

  // lookahead cursor and its load state
  GmmCursor la;
  la.j = 0;
  gmm_cursor_load<XP>(p, items, la);
  if (la.item >= items) return;
  __amdgpu_buffer_rsrc_t rca, rcb, rma, rmb;
  int vdc[NB][2], vdm[NB];
  auto la_item = [&]() {
    const uint8_t* ea = p.wa + la.e * p.stride;
    const uint8_t* eb = SWIGLU ? p.wb + la.e * p.stride : ea;
    const int64_t cbytes = int64_t(p.N) * RB, mbytes = int64_t(p.N) * S * 8;
    rca = rsrc(ea, cbytes);
    rcb = rsrc(eb, cbytes);
    rma = rsrc(ea + p.meta_off, mbytes);
    rmb = rsrc(eb + p.meta_off, mbytes);
    const int wrow = wrow_of(la.item);
    // tile b of the wave: matrix B (SwiGLU up) for b = 1 in SwiGLU mode, else
    // A; rows wrow + roff .. +16 with roff = 0 (SwiGLU) or 16 b.  Codes: half
    // h -> lane reads row 8h + lane/8, global chunk (lane % 8) ^ swz(row),
    // landing at LDS chunk lane % 8 of that row.  (scale, zp): lane -> (row,
    // piece) of LDS [tile][row][L groups].
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int roff = SWIGLU ? 0 : 16 * b;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + (lane >> 3);
        const int n = min(wrow + roff + r, p.N - 1);
        vdc[b][h] = int(int64_t(n) * RB) + (((lane & 7) ^ swz(r)) << 4);
      }
      const int n = min(wrow + roff + lane / Sh::PPR, p.N - 1);
      vdm[b] = n * S * 8 + (lane % Sh::PPR) * Sh::PB;
    }
  };
  la_item();

  auto issue = [&](int slot) {
    uint8_t* ws = wring + slot * Sh::WSLOT;
    uint8_t* as = aring + slot * Sh::ASLOT;
    const int m = la.m;
    const int tile = la.atile;
    const int abase = tile * S * J * 1024, xbase = tile * S * 64;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds((SWIGLU && b == 1) ? rcb : rca,
                                                 (lds_ptr_t)(ws + b * 2048 + h * 1024), 16,
                                                 vdc[b][h] + m * 128, 0, 0, kCodeAux);
    if (mlane) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        __builtin_amdgcn_raw_ptr_buffer_load_lds((SWIGLU && b == 1) ? rmb : rma,
                                                 (lds_ptr_t)(ws + Sh::CSLOT + b * 16 * L * 8),
                                                 Sh::PB, vdm[b] + m * L * 8, 0, 0, 0);
    }
    // one activation fragment per wave (waves beyond L*J repeat one)
    const int f = wv % (L * J);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(as + f * 1024), 16,
                                             abase + (m * L * J + f) * 1024 + lane * 16, 0, 0, 0);
    if (lane < L * 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(as + Sh::AFR), 4,
                                               xbase + m * L * 64 + lane * 4, 0, 0, 0);
    if (gmm_cursor_next<XP>(p, items, MS, la) && la.item < items) la_item();
  };

  f32x4_t y[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) y[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int m, int slot) {
    const uint8_t* ws = wring + slot * Sh::WSLOT;
    const uint8_t* as = aring + slot * Sh::ASLOT;
#pragma unroll
    for (int sl = 0; sl < L; ++sl) {
      if (m * L + sl >= S) break;  // last step may be partial (uniform)
      u32x4_t af[J];
#pragma unroll
      for (int j = 0; j < J; ++j)
        af[j] = *reinterpret_cast<const u32x4_t*>(as + (sl * J + j) * 1024 + lane * 16);
      const f32x4_t xsum = *reinterpret_cast<const f32x4_t*>(as + Sh::AFR + sl * 64 + g4 * 16);
      const int off = sl * (G * BITS / 8) + g4 * LB;  // byte of the row
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint8_t* row = ws + b * 2048 + c * 128;
        uint32_t w[LB / 4];
        if constexpr (LB == 8) {
          const u32x2_t v =
              *reinterpret_cast<const u32x2_t*>(row + (((off >> 4) ^ swz(c)) << 4) + (off & 15));
          w[0] = v[0];
          w[1] = v[1];
        } else {
#pragma unroll
          for (int h = 0; h < LB / 16; ++h) {
            const u32x4_t v =
                *reinterpret_cast<const u32x4_t*>(row + ((((off >> 4) + h) ^ swz(c)) << 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * h + i] = v[i];
          }
        }
        const f32x2_t mq =
            *reinterpret_cast<const f32x2_t*>(ws + Sh::CSLOT + (b * 16 + c) * L * 8 + sl * 8);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < J; ++j) {
          u32x4_t bq;
          if constexpr (BITS == 4) bq = int4_to_bf16(w[j]);
          else bq = int8_to_bf16(w[2 * j], w[2 * j + 1]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[j]),
                                                        __builtin_bit_cast(bf16x8_t, bq), acc, 0,
                                                        0, 0);
        }
        const float sc = mq[0], zq = mq[1] + kOff;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[b][i] = fmaf(sc, fmaf(-zq, xsum[i], acc[i]), y[b][i]);
      }
    }
  };

  // compute cursor
  GmmCursor cu;
  cu.j = 0;
  gmm_cursor_load<XP>(p, items, cu);
  auto epilogue = [&]() {
    // rows 4 g4 + i of the tile are parts of this lane's tokens
    const int wrow = wrow_of(cu.item);
#pragma unroll
    for (int q = 0; q < 4 / XP; ++q) {
      const int mrow = g4 * (4 / XP) + q;
      if (mrow >= cu.rows) continue;
      float* o = p.out + (cu.row0 + mrow) * p.ld_out;
      if constexpr (SWIGLU) {
        const int n = wrow + c;
        const float gv = XP == 2 ? y[0][2 * q] + y[0][2 * q + 1] : y[0][q];
        const float uv = XP == 2 ? y[1][2 * q] + y[1][2 * q + 1] : y[1][q];
        if (n < p.N) o[n] = silu(gv) * uv;
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int n = wrow + 16 * b + c;
          const float v = XP == 2 ? y[b][2 * q] + y[b][2 * q + 1] : y[b][q];
          if (n < p.N) o[n] = v;
        }
      }
    }
  };

  // steps issued so far; at step g the steps g + 1 .. issued - 1 are in
  // flight (at most A - 1 of them when the wait comes)
  int issued = 0;
  issue(0);
  ++issued;
#pragma unroll
  for (int d = 1; d < A; ++d) {
    if (la.item < items) {
      issue(d);
      ++issued;
    }
  }
  for (int g0 = 0;; g0 += DM) {
#pragma unroll
    for (int u = 0; u < DM; ++u) {
      const int g = g0 + u;
      if (g >= issued) return;  // every issued step has been computed
      const int ahead = issued - g - 1;
      if (A >= 3 && ahead >= 2) wait_vmcnt<2 * Sh::PER_STEP>();
      else if (A >= 2 && ahead == 1) wait_vmcnt<Sh::PER_STEP>();
      else wait_vmcnt<0>();
      lds_barrier();  // all waves' loads of step g landed; step g - 1 consumed
      if (la.item < items) {
        issue((u + A) % DM);
        ++issued;
      }
      compute(cu.m, u);
      if (cu.m == MS - 1) {
        epilogue();
#pragma unroll
        for (int b = 0; b < NB; ++b) y[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      gmm_cursor_next<XP>(p, items, MS, cu);
    }
  }
}

template <int BITS, int J, int XP, bool SWIGLU>
__global__ __launch_bounds__(512) void gmm_kernel(GmmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[GmmShape<BITS, J, SWIGLU>::LDS];
  gmm_stream<BITS, J, XP, SWIGLU>(p, sm);
}

namespace {

// prep workgroups per K segment (token tiles beyond take further rounds)
constexpr int64_t kPrepMaxTileBlocks = 4096;

int tiles_bound(int64_t rows, int64_t segments, int xp) {
  return int(rows * xp / 16 + segments + 1);
}

template <int BITS, int J, int XP, bool SWIGLU>
hipError_t launch_one(const GmmArgs& a, int64_t max_tiles, hipStream_t stream) {
  const int64_t total = max_tiles * a.rt;
  // one workgroup per CU; every workgroup gets the same number of items to
  // within one
  const int64_t blocks = total < 256 ? total : 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gmm_kernel<BITS, J, XP, SWIGLU>), dim3(unsigned(blocks)), dim3(512), 0,
                     stream, a);
  return hipGetLastError();
}

template <int XP>
hipError_t launch_bits(const GmmArgs& a, int bits, bool swiglu, int64_t max_tiles,
                       hipStream_t stream) {
  const int J = a.group / 32;
  if (bits == 4 && J == 2)
    return swiglu ? launch_one<4, 2, XP, true>(a, max_tiles, stream)
                  : launch_one<4, 2, XP, false>(a, max_tiles, stream);
  if (bits == 4 && J == 4)
    return swiglu ? launch_one<4, 4, XP, true>(a, max_tiles, stream)
                  : launch_one<4, 4, XP, false>(a, max_tiles, stream);
  if (bits == 8 && J == 2)
    return swiglu ? launch_one<8, 2, XP, true>(a, max_tiles, stream)
                  : launch_one<8, 2, XP, false>(a, max_tiles, stream);
  return swiglu ? launch_one<8, 4, XP, true>(a, max_tiles, stream)
                : launch_one<8, 4, XP, false>(a, max_tiles, stream);
}

}  // namespace

int64_t gmm_tiles_bound(int64_t rows, int64_t segments, int xp) {
  return tiles_bound(rows, segments, xp);
}

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
  int64_t max_tiles = (M * xp + 15) / 16;
  if (grp) {
    pa.perm = grp->perm;
    pa.top_k = grp->top_k;
    pa.tiles = grp->tiles;
    pa.n_tiles = grp->n_tiles;
    max_tiles = grp->max_tiles;
    if (grp->max_items == 0) return hipSuccess;
  }
  if (max_tiles == 0) return hipSuccess;
  const int segs = xp == 2 ? 32 : 16;
  const dim3 pgrid(unsigned((A.K / 8 + segs - 1) / segs),
                   unsigned(max_tiles < kPrepMaxTileBlocks ? max_tiles : kPrepMaxTileBlocks));
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
    a.tiles = grp->tiles;
    a.n_tiles = grp->n_tiles;
  }
  a.afrag = static_cast<const uint4*>(act);
  a.afrag_bytes = int64_t(act_bytes);
  a.xs = xs;
  a.xs_bytes = int64_t(xs_bytes);
  a.out = out;
  a.ld_out = ld_out;
  const int rows = B ? 128 : 256;  // output rows per workgroup item
  a.rt = int((A.N + rows - 1) / rows);
  if (xp == 2) return launch_bits<2>(a, A.bits, B != nullptr, max_tiles, stream);
  return launch_bits<1>(a, A.bits, B != nullptr, max_tiles, stream);
}

}  // namespace dsq
