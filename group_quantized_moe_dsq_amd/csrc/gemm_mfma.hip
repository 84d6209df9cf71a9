// gemm_mfma.hip -- dense fused-dequant GEMM on bf16 MFMA (prefill).
//
// Y[m][n] = sum_k bf16(X[m][k]) * bf16((q[n][k] - zp) * scale), fp32 sums,
// the batched form of the fused-dequant matmul ("Hand-writing a DeepSeek
// inference engine in pure C", hnwysp.cn/news/134870, §3.2-§3.3) for prompt
// tokens processed together.
//
// Tiling (gfx950, wave64):
//   * workgroup = 8 waves for a 128x128 output tile, specialised: waves 0-3
//     only read LDS and issue MFMAs (wave (wm, wn) owns 64x64 as 2x2
//     v_mfma_f32_32x32x16_bf16 tiles, 64 fp32 accumulators per lane), waves
//     4-7 only load, dequantize and fill the next LDS buffer.  One wave of
//     each kind per SIMD: the dequant VALU work overlaps the matrix core
//     instead of waiting for it in program order;
//   * K in steps of 64: the step's X tile (bf16, 128x64) and W tile (codes
//     dequantized to bf16 once per workgroup, 128x64) are written to LDS,
//     double-buffered, rows padded to 144 B so the 32 rows an MFMA operand
//     read touches fall on distinct banks; the next step's global loads are
//     in flight while the current step's MFMAs run;
//   * the global loads of the next D steps are in flight (a ring of D
//     register stages) while the current step's MFMAs run: the loaded memory
//     latency (~1.4 us) is paid once, not once per step;
//   * split-K: the K range is cut into SK slices so that tiles * SK covers
//     the 256 CUs; each slice writes an fp32 partial tile with plain stores
//     and a second kernel adds the SK partials in slice order (deterministic).
//     No fence or counter inside the GEMM: a device-scope fence writes the
//     whole L2 back on this chip and, issued by every workgroup, costs far
//     more than the extra launch;
//   * blocks are ordered so the two M tiles that share a W slice run on the
//     same XCD (workgroup b runs on XCD b % 8) and share its L2;
//   * rows of X and W are 4-8 KiB apart, so the 128 rows of one K step share
//     their low address bits (and L2 channel); each workgroup therefore walks
//     its K steps starting at a step rotated by its N tile, which spreads the
//     workgroups of an XCD over the channels instead of marching in lockstep.
//
// MFMA 32x32x16 operands: lane l supplies 8 bf16 of row (l % 32) of A and of
// column (l % 32) of B for k-slice (l / 32); lane l's 16 accumulators hold
// column (l % 32), rows 8 * (r / 4) + 4 * (l / 32) + (r % 4).
#include "common.h"
#include "internal.h"

namespace dsq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kRowBytes = kBK * 2 + 16;  // padded LDS row: 64 bf16 + 16 B
#ifndef DSQ_GEMM_STAGES
#define DSQ_GEMM_STAGES 4
#endif
constexpr int kStages = DSQ_GEMM_STAGES;  // global-load steps in flight

struct GemmArgs {
  const uint8_t* w;     // packed entry (codes)
  const float2* meta;   // its (scale, zp) table
  const __bf16* X;      // [M][K] bf16
  float* Y;             // [M][N]
  float* partial;       // [tiles][SK][128*128] fp32 (split-K only)
  int M, N, K, group;
  int SK;               // K slices
  int tiles_m, tiles_n;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = __bf16(a), y = __bf16(b);
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

// Per producer thread (t = threadIdx.x - 256) share of one K step.  Loads are
// laid out so that consecutive lanes read consecutive 16-byte chunks: one
// wave instruction then covers whole cache lines (8 rows x 128 B of X).
//   X : chunks c = t + 256 j (j < 4) of the 128 x 128 B tile: row c / 8,
//       16-byte column c % 8.
//   W : INT8 chunks c = t + 256 j (j < 2) of the 128 x 64 B tile: row c / 4,
//       16 codes at column c % 4; INT4 chunk c = t: row c / 2, 32 codes at
//       column c % 2.  Each chunk carries its row's (scale, zp).
template <int BITS>
struct StepRegs {
  static constexpr int NC = BITS == 8 ? 2 : 1;  // W chunks per thread
  uint4 x[4];
  uint4 c[NC];
  float2 m[NC];
};

template <int BITS>
__device__ __forceinline__ void load_step(const GemmArgs& p, int tm, int tn, int k0,
                                          StepRegs<BITS>& r) {
  const int t = threadIdx.x - 256;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 256 * j;
    // rows past M read row M-1 and are zeroed when stored
    const int m = min(tm * kBM + (c >> 3), p.M - 1);
    r.x[j] = *reinterpret_cast<const uint4*>(p.X + int64_t(m) * p.K + k0 + (c & 7) * 8);
  }
  const int64_t rb = int64_t(p.K) * BITS / 8;
  const int groups = p.K / p.group;
#pragma unroll
  for (int j = 0; j < StepRegs<BITS>::NC; ++j) {
    const int c = t + 256 * j;
    const int row = BITS == 8 ? (c >> 2) : (c >> 1);
    const int col = BITS == 8 ? (c & 3) : (c & 1);  // 16-byte column
    const int n = min(tn * kBN + row, p.N - 1);
    const int kc = k0 + col * (BITS == 8 ? 16 : 32);  // first k of the chunk
    r.c[j] = ld_nt(reinterpret_cast<const uint4*>(p.w + int64_t(n) * rb + int64_t(kc) * BITS / 8));
    r.m[j] = p.meta[int64_t(n) * groups + kc / p.group];
  }
}

// Dequantize and write the step to LDS (A = X tile, B = W tile).
template <int BITS>
__device__ __forceinline__ void store_step(const GemmArgs& p, int tm, const StepRegs<BITS>& r,
                                           uint8_t* lds_a, uint8_t* lds_b) {
  const int t = threadIdx.x - 256;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = t + 256 * j;
    const bool mvalid = tm * kBM + (c >> 3) < p.M;
    *reinterpret_cast<uint4*>(lds_a + (c >> 3) * kRowBytes + (c & 7) * 16) =
        mvalid ? r.x[j] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < StepRegs<BITS>::NC; ++j) {
    const int c = t + 256 * j;
    constexpr int CPC = BITS == 8 ? 16 : 32;  // codes per chunk
    float f[CPC];
    if constexpr (BITS == 8) Codes<8>::unpack(r.c[j], f);
    else Codes<4>::unpack(r.c[j], f);
    const float sc = r.m[j].x, nzs = -r.m[j].y * r.m[j].x;
    uint32_t wv[CPC / 2];
#pragma unroll
    for (int i = 0; i < CPC / 2; ++i)
      wv[i] = pack_bf16x2(fmaf(f[2 * i], sc, nzs), fmaf(f[2 * i + 1], sc, nzs));
    const int row = BITS == 8 ? (c >> 2) : (c >> 1);
    const int col = BITS == 8 ? (c & 3) : (c & 1);
    uint4* b = reinterpret_cast<uint4*>(lds_b + row * kRowBytes + col * CPC * 2);
#pragma unroll
    for (int i = 0; i < CPC / 8; ++i)
      b[i] = make_uint4(wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]);
  }
}

template <int BITS>
__global__ __launch_bounds__(512) void gemm_mfma_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kBM * kRowBytes];  // [buf][A|B]
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
  const int steps_total = p.K / kBK;
  const int steps = steps_total / p.SK;
  const int kbeg = ks * steps * kBK;
  const int rot = tn % steps;
  // K offset of the workgroup's s-th step
  auto kof = [&](int s) { return kbeg + ((s + rot) % steps) * kBK; };

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool producer = wv >= 4;

  // Both roles meet at one barrier per step.  Before barrier s the producers
  // have filled buffer s&1 with step s and the consumers have finished the
  // MFMAs of step s-1 (buffer (s-1)&1), so after it the producers may refill
  // that buffer with step s+1 while the consumers read buffer s&1.
  if (producer) {
    StepRegs<BITS> regs[kStages];
#pragma unroll
    for (int d = 0; d < kStages; ++d)
      if (d < steps) load_step<BITS>(p, tm, tn, kof(d), regs[d]);
    // step s is held in regs[s % kStages]
    for (int s0 = 0; s0 < steps; s0 += kStages) {
#pragma unroll
      for (int d = 0; d < kStages; ++d) {
        const int s = s0 + d;
        if (s >= steps) break;  // uniform over the workgroup
        store_step<BITS>(p, tm, regs[d], lds[s & 1][0], lds[s & 1][1]);
        if (s + kStages < steps) load_step<BITS>(p, tm, tn, kof(s + kStages), regs[d]);
        __syncthreads();
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
  for (int s = 0; s < steps; ++s) {
    __syncthreads();
    const uint8_t* A = lds[s & 1][0];
    const uint8_t* B = lds[s & 1][1];
    bf16x8 af[kBK / 16][2], bfr[kBK / 16][2];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int koff = kk * 32 + (lane >> 5) * 16;  // bytes within the row
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[kk][i] = *reinterpret_cast<const bf16x8*>(A + (wm * 64 + i * 32 + (lane & 31)) * kRowBytes + koff);
        bfr[kk][i] = *reinterpret_cast<const bf16x8*>(B + (wn * 64 + i * 32 + (lane & 31)) * kRowBytes + koff);
      }
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
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
  // split-K: this slice's partial tile, reduced by splitk_reduce_kernel
  float* mine = p.partial + (int64_t(tile) * p.SK + ks) * (kBM * kBN);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m, n;
        out_index(i, j, r, m, n);
        mine[m * kBN + n] = acc[i][j][r];
      }
}

// Y[m][n] = sum over slices q = 0..SK-1 (in that order) of the partial tiles.
// One thread per output; consecutive threads read consecutive partial floats.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            float* __restrict__ Y, int M, int N,
                                                            int SK, int tiles_m) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(M) * N) return;
  const int m = int(i / N), n = int(i % N);
  const int tile = (n / kBN) * tiles_m + m / kBM;
  const float* base = partial + int64_t(tile) * SK * (kBM * kBN) + (m % kBM) * kBN + (n % kBN);
  float v = base[0];
  for (int q = 1; q < SK; ++q) v += base[int64_t(q) * (kBM * kBN)];
  Y[i] = v;
}

// X (fp32) -> bf16.
__global__ __launch_bounds__(256) void prep_kernel(const float* __restrict__ x, int64_t n,
                                                   __bf16* __restrict__ out) {
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const float4 v = *reinterpret_cast<const float4*>(x + i);
    out[i] = __bf16(v.x);
    out[i + 1] = __bf16(v.y);
    out[i + 2] = __bf16(v.z);
    out[i + 3] = __bf16(v.w);
  } else {
    for (int64_t j = i; j < n; ++j) out[j] = __bf16(x[j]);
  }
}

namespace {

struct Plan {
  int tiles_m, tiles_n, SK;
};

Plan plan(int64_t M, int64_t N, int64_t K) {
  Plan pl;
  pl.tiles_m = int((M + kBM - 1) / kBM);
  pl.tiles_n = int((N + kBN - 1) / kBN);
  const int tiles = pl.tiles_m * pl.tiles_n;
  const int steps = int(K / kBK);
  pl.SK = 1;
  // largest divisor of the step count that keeps tiles * SK within 256 CUs
  for (int sk = 2; sk <= 16 && sk <= steps; ++sk)
    if (steps % sk == 0 && tiles * sk <= 256) pl.SK = sk;
  return pl;
}

}  // namespace

size_t gemm_mfma_workspace(int64_t M, int64_t N, int64_t K) {
  const Plan pl = plan(M, N, K);
  int64_t b = align256(M * K * 2);  // X in bf16
  if (pl.SK > 1) {
    const int64_t tiles = int64_t(pl.tiles_m) * pl.tiles_n;
    b += align256(tiles * pl.SK * kBM * kBN * 4);
  }
  return size_t(b);
}

hipError_t launch_gemm_mfma(const dsq_qweight& W, int64_t expert, const float* X, float* Y,
                            int64_t M, void* workspace, hipStream_t stream) {
  const Plan pl = plan(M, W.N, W.K);
  const QMat q = entry(W, expert);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  __bf16* xb = reinterpret_cast<__bf16*>(ws);
  const int64_t tiles = int64_t(pl.tiles_m) * pl.tiles_n;
  float* partial = nullptr;
  if (pl.SK > 1) partial = reinterpret_cast<float*>(ws + align256(M * W.K * 2));
  const int64_t n = M * W.K;
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(prep_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, X,
                     n, xb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmArgs a{};
  a.w = q.payload;
  a.meta = q.meta;
  a.X = xb;
  a.Y = Y;
  a.partial = partial;
  a.M = int(M);
  a.N = int(W.N);
  a.K = int(W.K);
  a.group = W.group;
  a.SK = pl.SK;
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  const unsigned blocks = unsigned(tiles * pl.SK);
  if (W.bits == 8)
    hipLaunchKernelGGL(gemm_mfma_kernel<8>, dim3(blocks), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(gemm_mfma_kernel<4>, dim3(blocks), dim3(512), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || pl.SK == 1) return e;
  const int64_t outs = M * W.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(unsigned((outs + 255) / 256)), dim3(256), 0,
                     stream, partial, Y, int(M), int(W.N), pl.SK, pl.tiles_m);
  return hipGetLastError();
}

}  // namespace dsq
