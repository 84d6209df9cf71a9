// gemm_mfma.hip -- dense fused-dequant GEMM on bf16 MFMA (prefill).
//
// Y[m][n] = sum_k bf16(X[m][k]) * bf16((q[n][k] - zp) * scale), fp32 sums,
// the batched form of the fused-dequant matmul ("Hand-writing a DeepSeek
// inference engine in pure C", hnwysp.cn/news/134870, §3.2-§3.3) for prompt
// tokens processed together.
//
// Two kernels (one when K is not split):
//   * gemm_mfma_kernel: one workgroup per 128x128 output tile and K slice,
//     12 waves in two roles.  Waves 0-3 only read LDS and issue MFMAs (wave
//     (wm, wn) owns 64x64 as 2x2 v_mfma_f32_32x32x16_bf16 tiles); waves 4-11
//     load the next K steps (64 k each) of X (fp32) and of the codes into
//     registers, round X to bf16, dequantize the codes to bf16 and write both
//     tiles to LDS.  Two producer waves share each SIMD with one MFMA wave,
//     so the dequant VALU work overlaps the matrix core;
//   * splitk_reduce_kernel: adds the K slices' partial tiles in slice order.
//
// The loop is bound by LDS (it accepts ~76 B/clk of writes and ~118 B/clk of
// reads per CU) and by the L2, which sees a request per cache line touched
// by a wave's load; every access is shaped to need few:
//   * X: each load instruction reads 4 whole 256-byte row pieces;
//   * W: a row's 64 codes of a step are one 64-byte (INT8) or 32-byte (INT4)
//     piece, read by 4 adjacent lanes;
//   * (scale, zp): the K slice's groups of the tile's 128 rows are copied to
//     LDS once, instead of one 8-byte read per row and step.
// LDS tiles are 128-byte rows of 16-byte chunks, chunk c of row r stored at
// c ^ (r % 8): the 8 rows an MFMA operand read serves per cycle fall on
// distinct banks.  Three step buffers let the MFMA waves read step k+1 into
// registers while the MFMAs of step k run, with one barrier per step.
//
// Split-K: the K range is cut into SK slices so that tiles * SK fills the
// 256 CUs; each slice writes an fp32 partial tile with device-scope stores,
// which write through the XCD's L2 as they go (plain stores left 16.8 MB
// dirty in the L2s at M = 256, K = N = 4096, written back only when the
// kernel ends: ~1 us more per call).  No fence or counter inside the GEMM: a
// device-scope fence writes the whole L2 back on this chip.  Workgroups are ordered so the two M tiles that share a
// W slice run on the same XCD (workgroup b runs on XCD b % 8), and each walks
// its K steps from a step rotated by its N tile, which spreads the
// workgroups of an XCD over the L2 channels.
//
// MFMA 32x32x16 operands: lane l supplies 8 bf16 of row (l % 32) of A and of
// column (l % 32) of B for k-slice (l / 32); lane l's 16 accumulators hold
// column (l % 32), rows 8 * (r / 4) + 4 * (l / 32) + (r % 4).
#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace dsq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kRowBytes = kBK * 2;  // LDS tile row: 64 bf16, chunks swizzled
constexpr int kTileBytes = kBM * kRowBytes;
constexpr int kConsumers = 4;       // MFMA waves
constexpr int kProducers = 8;       // load / dequantize waves
constexpr int kThreads = 64 * (kConsumers + kProducers);
#ifndef DSQ_GEMM_STAGES
#define DSQ_GEMM_STAGES 3
#endif
constexpr int kStages = DSQ_GEMM_STAGES;  // global-load steps in flight
constexpr int kBufs = 3;                  // LDS step buffers
// (scale, zp) of at most this many groups per row of a K slice sit in LDS;
// the row pitch (49 float2 = 98 dwords) puts the 16 rows of a wave's reads
// on distinct banks
constexpr int kMetaGroups = 48;
constexpr int kMetaPitch = kMetaGroups + 1;
#ifndef DSQ_GEMM_MAX_WG
#define DSQ_GEMM_MAX_WG 256
#endif
constexpr int kMaxWorkgroups = DSQ_GEMM_MAX_WG;  // one per CU

struct GemmArgs {
  const uint8_t* w;     // packed entry (codes)
  const float2* meta;   // its (scale, zp) table
  const float* X;       // [M][K] fp32
  float* Y;             // [M][N]
  float* partial;       // [tiles][SK][128*128] fp32 (split-K only)
  int M, N, K, lg;      // lg = log2(group)
  int SK;               // K slices
  int tiles_m, tiles_n;
};

// byte offset of 16-byte chunk c of row r in an LDS tile
__device__ __forceinline__ int chunk_off(int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); }

// Per producer thread (t = threadIdx.x - 256, 0..511) share of one K step:
//   X : rows (t / 16) + 32 j (j = 0..3), 4 fp32 at k = 4 (t % 16);
//   W : row t / 4, 16 codes at k = 16 (t % 4) (INT8: one 16-byte load, INT4:
//       one 8-byte load of two words) and the (scale, zp) of their group (a
//       step lies inside one group), read from LDS.
template <int BITS>
struct StepRegs {
  f32x4_t x[4];
  uint32_t c[BITS == 8 ? 4 : 2];
  f32x2_t m;
};

// Per-lane offsets, fixed over the K loop; a step adds wave-uniform offsets.
// An offset of 2^31 or more lies beyond every buffer (records < 2^31): the
// load returns zeros without touching memory.  Rows of X past M use it, and
// so do the loads of steps past the slice's end, which keep the count of
// loads in flight the same on every step.
constexpr uint32_t kOOB = 0x80000000u;
struct ProdLane {
  __amdgpu_buffer_rsrc_t rx, rw;
  uint32_t vx[4];  // X byte offsets of (row (t / 16) + 32 j, k = 4 (t % 16)) at k = 0
  uint32_t vw;     // code byte offset of (row t / 4, k = 16 (t % 4)) at k = 0
  const float2* ml;  // LDS (scale, zp) of row t / 4, group g_first
  int g_first;
};

template <int BITS>
__device__ __forceinline__ void load_step(const ProdLane& pl, int k0, int lg, bool live,
                                          StepRegs<BITS>& r) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r.x[j] = __builtin_bit_cast(
        f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(pl.rx, live ? pl.vx[j] : kOOB, k0 * 4, kNT));
  const uint32_t vw = live ? pl.vw : kOOB;
  if constexpr (BITS == 8) {
    const u32x4_t v = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(pl.rw, vw, k0, kNT));
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = v[i];
  } else {
    const u32x2_t v = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(pl.rw, vw, k0 / 2, kNT));
    r.c[0] = v[0];
    r.c[1] = v[1];
  }
  // the group of a step past the slice's end may lie past the staged ones
  const int g = live ? (k0 >> lg) - pl.g_first : 0;
  const float2 m = pl.ml[g];
  r.m[0] = m.x;
  r.m[1] = m.y;
}

// Round X to bf16, dequantize the codes and write both tiles of the step to LDS.
template <int BITS>
__device__ __forceinline__ void store_step(const StepRegs<BITS>& r, uint8_t* lds_a,
                                           uint8_t* lds_b) {
  const int t = threadIdx.x - 64 * kConsumers;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint2*>(lds_a + chunk_off((t >> 4) + 32 * j, (t & 15) >> 1) + 8 * (t & 1)) =
        make_uint2(pk_bf16(r.x[j][0], r.x[j][1]), pk_bf16(r.x[j][2], r.x[j][3]));
  // w = q * s - zp * s, rounded once to bf16
  const float sc = r.m[0], nzs = -r.m[1] * r.m[0];
  float f[16];
  if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[4 * i] = float(r.c[i] & 0xffu);
      f[4 * i + 1] = float((r.c[i] >> 8) & 0xffu);
      f[4 * i + 2] = float((r.c[i] >> 16) & 0xffu);
      f[4 * i + 3] = float(r.c[i] >> 24);
    }
  } else {
    // word w: byte i holds k = i (low nibble) and k = 4 + i (high nibble)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t lo = r.c[h] & 0x0F0F0F0Fu, hi = (r.c[h] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * h + i] = float((lo >> (8 * i)) & 0xffu);
        f[8 * h + 4 + i] = float((hi >> (8 * i)) & 0xffu);
      }
    }
  }
  uint32_t wv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) wv[i] = pk_bf16(fmaf(f[2 * i], sc, nzs), fmaf(f[2 * i + 1], sc, nzs));
  const int row = t >> 2, c0 = 2 * (t & 3);
  *reinterpret_cast<uint4*>(lds_b + chunk_off(row, c0)) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  *reinterpret_cast<uint4*>(lds_b + chunk_off(row, c0 + 1)) = make_uint4(wv[4], wv[5], wv[6], wv[7]);
}

// Barrier between K steps.  The scheduling fence keeps the compiler from
// hoisting the next step's conversions (which wait for its loads) above it.
__device__ __forceinline__ void step_barrier() {
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// K slice ks of SK over steps_total steps: the first steps_total % SK slices
// get one step more.
__device__ __forceinline__ void slice_range(int steps_total, int SK, int ks, int& first, int& n) {
  const int base = steps_total / SK, rem = steps_total % SK;
  n = base + (ks < rem ? 1 : 0);
  first = ks * base + min(ks, rem);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmArgs p) {
  // [buffer][A | B]: X tile and dequantized W tile of one K step, bf16
  __shared__ __attribute__((aligned(16))) uint8_t lds[kBufs][2][kTileBytes];
  __shared__ __attribute__((aligned(16))) float2 lds_meta[kBN * kMetaPitch];
  const int nblocks = gridDim.x;
  // XCD-aware order: workgroup b runs on XCD b % 8; give consecutive logical
  // work items (same K slice and N tile, different M tiles) to one XCD.
  int b = blockIdx.x;
  if (nblocks % 8 == 0) b = (blockIdx.x % 8) * (nblocks / 8) + blockIdx.x / 8;
  const int tm = b % p.tiles_m;
  const int rest = b / p.tiles_m;
  const int tn = rest % p.tiles_n;
  const int ks = rest / p.tiles_n;
  const int tile = tn * p.tiles_m + tm;
  int sfirst, steps;
  slice_range(p.K / kBK, p.SK, ks, sfirst, steps);
  const int kbeg = sfirst * kBK;
  const int rot = tn % steps;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool producer = wv >= kConsumers;

  // Step s lives in buffer s % 3.  Barriers: one before the loop ("-1") and
  // one after each phase k = 0 .. steps-2.  In phase k the consumers run the
  // MFMAs of step k and read step k+1 into registers; the producers write
  // step k+2.  Before barrier k-1 the producers have written steps <= k+1, so
  // step k+1 is readable in phase k; the buffer of step k+2 last held step
  // k-1, whose reads were issued in phase k-2 and finished before barrier k-2
  // (each barrier first waits for the wave's LDS accesses).
  if (producer) {
    const int t = threadIdx.x - 64 * kConsumers;
    ProdLane pl;
    pl.rx = rsrc(p.X, int64_t(p.M) * p.K * 4);
    pl.rw = rsrc(p.w, int64_t(p.N) * p.K * BITS / 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = tm * kBM + (t >> 4) + 32 * j;
      pl.vx[j] = m < p.M ? uint32_t((m * p.K + 4 * (t & 15)) * 4) : kOOB;
    }
    const int row = t >> 2;
    const int n = min(tn * kBN + row, p.N - 1);
    pl.vw = uint32_t(n * (p.K * BITS / 8) + 16 * (t & 3) * BITS / 8);
    // copy the slice's (scale, zp) of this row to LDS: the row's 4 lanes take
    // pairs of groups in turn; only these lanes read them back, so program
    // order within the wave is the only ordering needed
    {
      const int gpr = p.K >> p.lg;  // groups per row
      const int g_first = kbeg >> p.lg;
      const int ng = ((kbeg + steps * kBK - 1) >> p.lg) - g_first + 1;
      const __amdgpu_buffer_rsrc_t rm = rsrc(p.meta, int64_t(p.N) * gpr * 8);
      float2* dst = lds_meta + row * kMetaPitch;
      for (int c = t & 3; 2 * c < ng; c += 4) {
        const uint32_t off = uint32_t((n * gpr + g_first + 2 * c) * 8);
        if (2 * c + 1 < ng) {
          const f32x4_t v = __builtin_bit_cast(
              f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rm, off, 0, kNT));
          dst[2 * c] = make_float2(v[0], v[1]);
          dst[2 * c + 1] = make_float2(v[2], v[3]);
        } else {  // odd count: the last group alone (it may end the table)
          const f32x2_t v = __builtin_bit_cast(
              f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rm, off, 0, kNT));
          dst[2 * c] = make_float2(v[0], v[1]);
        }
      }
      pl.ml = dst;
      pl.g_first = g_first;
    }
    // K offset of the next step to load: the slice's steps starting at step
    // `rot`, wrapping to the slice start
    const int kend = kbeg + steps * kBK;
    int kl = kbeg + rot * kBK;
    auto next_k = [&]() {
      const int k = kl;
      kl += kBK;
      if (kl == kend) kl = kbeg;
      return k;
    };
    // step s is loaded into regs[s % kStages]; after it is stored, step
    // s + kStages is loaded into the same registers (loads past the slice end
    // read nothing)
    StepRegs<BITS> regs[kStages];
#pragma unroll
    for (int d = 0; d < kStages; ++d) load_step<BITS>(pl, next_k(), p.lg, d < steps, regs[d]);
    auto put = [&](StepRegs<BITS>& r, int s) {
      const int buf = s % kBufs;
      store_step<BITS>(r, lds[buf][0], lds[buf][1]);
      load_step<BITS>(pl, next_k(), p.lg, s + kStages < steps, r);
    };
    // Steps 0 and 1 before the first barrier.  Every put of the main loop
    // runs, so the count of loads in flight is the same on each step and the
    // compiler waits only for the step being stored.  A put of a step past
    // the end writes a buffer that no consumer reads again.
    put(regs[0], 0);
    put(regs[1 % kStages], 1);
    step_barrier();
    int k = 0;
    for (; k + kStages + 1 < steps; k += kStages) {
#pragma unroll
      for (int d = 0; d < kStages; ++d) {
        put(regs[(d + 2) % kStages], k + d + 2);
        step_barrier();
      }
    }
    // the last phases (fewer than kStages + 1 remain, k a multiple of kStages)
#pragma unroll
    for (int d = 0; d < kStages; ++d) {
      if (k + d < steps - 1) {  // uniform over the workgroup
        if (k + d + 2 < steps) put(regs[(d + 2) % kStages], k + d + 2);
        step_barrier();
      }
    }
    return;  // the consumer waves write the tile
  }

  const int wm = wv >> 1, wn = wv & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // fragment of slice kk (16 of the step's 64 k): A rows / B columns
  // 32 i + lane % 32 of the wave's 64, chunk 2 kk + lane / 32 (rows are
  // multiples of 8 apart from lane % 32, so the swizzle uses lane % 8)
  const int arow = (wm * 64 + (lane & 31)) * kRowBytes;
  const int brow = (wn * 64 + (lane & 31)) * kRowBytes;
  int coff[kBK / 16];
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) coff[kk] = ((2 * kk + (lane >> 5)) ^ (lane & 7)) << 4;
  bf16x8 af[kBK / 16][2], bfr[kBK / 16][2];
  auto read = [&](int buf, int kk) {
    const uint8_t* A = lds[buf][0] + arow + coff[kk];
    const uint8_t* B = lds[buf][1] + brow + coff[kk];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      af[kk][i] = *reinterpret_cast<const bf16x8*>(A + i * 32 * kRowBytes);
      bfr[kk][i] = *reinterpret_cast<const bf16x8*>(B + i * 32 * kRowBytes);
    }
  };
  step_barrier();
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) read(0, kk);
  for (int k = 0; k < steps; ++k) {
    const bool more = k + 1 < steps;
    const int nbuf = (k + 1) % kBufs;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
      if (more) read(nbuf, kk);
    }
    if (more) step_barrier();
  }

  // ---- epilogue ----
  auto out_index = [&](int i, int j, int r, int& m, int& n) {
    m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    n = wn * 64 + j * 32 + (lane & 31);
  };
  if (p.SK == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int m, n;
          out_index(i, j, r, m, n);
          m += tm * kBM;
          n += tn * kBN;
          if (m < p.M && n < p.N) p.Y[int64_t(m) * p.N + n] = acc[i][j][r];
        }
    return;
  }
  // split-K: this slice's partial tile, reduced by splitk_reduce_kernel;
  // written through to memory (device scope), read by the next kernel
  float* mine = p.partial + (int64_t(tile) * p.SK + ks) * (kBM * kBN);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m, n;
        out_index(i, j, r, m, n);
        __hip_atomic_store(mine + m * kBN + n, acc[i][j][r], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
}

// Y[m][n] = sum over slices q = 0..SK-1 (in that order) of the partial tiles.
// One thread per 4 consecutive outputs of a row (N % 4 == 0; else one);
// consecutive threads read consecutive partial floats.  The slices' loads are
// issued together, 4 at a time, before the adds.  Each partial is read once:
// non-temporal loads (0.3 us less per call at M = 256, K = N = 4096; two or
// four outputs per thread measured slower).
template <int V>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            float* __restrict__ Y, int M, int N,
                                                            int SK, int tiles_m) {
  typedef float fv __attribute__((ext_vector_type(V)));
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * V;
  if (i >= int64_t(M) * N) return;
  const int m = int(i / N), n = int(i % N);
  const int tile = (n / kBN) * tiles_m + m / kBM;
  const fv* base = reinterpret_cast<const fv*>(partial + int64_t(tile) * SK * (kBM * kBN) +
                                               (m % kBM) * kBN + (n % kBN));
  constexpr int kSlice = kBM * kBN / V;
  auto ld = [&](int q) { return __builtin_nontemporal_load(base + int64_t(q) * kSlice); };
  fv v = ld(0);
  int q = 1;
  for (; q + 4 <= SK; q += 4) {
    const fv a = ld(q), b = ld(q + 1), c = ld(q + 2), d = ld(q + 3);
    v += a;
    v += b;
    v += c;
    v += d;
  }
  for (; q < SK; ++q) v += ld(q);
  *reinterpret_cast<fv*>(Y + i) = v;
}

namespace {

struct Plan {
  int tiles_m, tiles_n, SK;
};

// groups of `group` columns that a run of `steps` K steps can touch
int span_groups(int steps, int group) {
  return (steps * kBK + group - 1) / group + (group > kBK ? 1 : 0);
}

Plan plan(int64_t M, int64_t N, int64_t K, int group) {
  Plan pl;
  pl.tiles_m = int((M + kBM - 1) / kBM);
  pl.tiles_n = int((N + kBN - 1) / kBN);
  const int64_t tiles = int64_t(pl.tiles_m) * pl.tiles_n;
  const int steps = int(K / kBK);
  // enough K slices to give every CU a workgroup (at most 16) ...
  pl.SK = 1;
  while (pl.SK < 16 && pl.SK < steps && tiles * (pl.SK + 1) <= kMaxWorkgroups) ++pl.SK;
  // ... and short enough for their groups' (scale, zp) to fit in LDS
  while (span_groups((steps + pl.SK - 1) / pl.SK, group) > kMetaGroups) ++pl.SK;
  return pl;
}

}  // namespace

bool gemm_mfma_supported(int64_t M, int64_t N, int64_t K) {
  // 32-bit buffer offsets into X and into an INT8 entry's codes
  return M * K * 4 < (int64_t(1) << 31) && N * K < (int64_t(1) << 31) && K % kBK == 0;
}

size_t gemm_mfma_workspace(int64_t M, int64_t N, int64_t K) {
  // the smallest group (64) gives the most K slices
  const Plan pl = plan(M, N, K, 64);
  const Plan p2 = plan(M, N, K, 128);
  const int64_t tiles = int64_t(pl.tiles_m) * pl.tiles_n;
  const int sk = max(pl.SK, p2.SK);
  // at least one aligned block, so that 0 can mean "unsupported"
  int64_t b = 256;
  if (sk > 1) b = align256(tiles * sk * kBM * kBN * 4);
  return size_t(b);
}

hipError_t launch_gemm_mfma(const dsq_qweight& W, int64_t expert, const float* X, float* Y,
                            int64_t M, void* workspace, hipStream_t stream) {
  const Plan pl = plan(M, W.N, W.K, W.group);
  const QMat q = entry(W, expert);
  const int64_t tiles = int64_t(pl.tiles_m) * pl.tiles_n;
  float* partial = pl.SK > 1 ? static_cast<float*>(workspace) : nullptr;
  GemmArgs a{};
  a.w = q.payload;
  a.meta = q.meta;
  a.X = X;
  a.Y = Y;
  a.partial = partial;
  a.M = int(M);
  a.N = int(W.N);
  a.K = int(W.K);
  a.lg = W.group == 128 ? 7 : 6;
  a.SK = pl.SK;
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  const unsigned blocks = unsigned(tiles * pl.SK);
  if (W.bits == 8)
    hipLaunchKernelGGL(gemm_mfma_kernel<8>, dim3(blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(gemm_mfma_kernel<4>, dim3(blocks), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.SK == 1) return e;
  const int64_t outs = M * W.N;
  if (W.N % 4 == 0)
    hipLaunchKernelGGL(splitk_reduce_kernel<4>, dim3(unsigned((outs / 4 + 255) / 256)), dim3(256),
                       0, stream, partial, Y, int(M), int(W.N), pl.SK, pl.tiles_m);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3(unsigned((outs + 255) / 256)), dim3(256), 0,
                       stream, partial, Y, int(M), int(W.N), pl.SK, pl.tiles_m);
  return hipGetLastError();
}

}  // namespace dsq
