// mfma.hip -- bf16 MFMA fused-dequant GEMM for prefill-sized token counts.
//
// out[m][n] = sum_k bf16(X[m][k]) * bf16((q[n][k] - zp) * scale), products
// summed in fp32 by v_mfma_f32_16x16x32_bf16 (gfx950).  Dense or grouped by
// expert exactly like the fp32 path ("Hand-writing a DeepSeek inference
// engine in pure C", hnwysp.cn/news/134870, §3.2 fused dequant, §3.5 experts
// batched over the tokens routed to them).  The MoE gate/up form multiplies
// two matrices and writes silu(gate) * up.
//
// MFMA 16x16x32 operands: lane l supplies 8 bf16 of row (l % 16) of A and of
// column (l % 16) of B, for a k-slice chosen by l / 16; the output tile gives
// lane l column (l % 16) and rows 4 * (l / 16) + 0..3.  Any assignment of the
// 32 k-values of one instruction to (lane group, element) is correct as long
// as A and B use the same one, because the instruction sums over all of them.
// Here each lane loads 16 bytes of codes at a time (INT8: 16 codes, INT4: 32)
// and feeds them to CPL / 8 consecutive instructions.
#include "common.h"
#include "internal.h"

namespace dsq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ x, int64_t n,
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

hipError_t launch_to_bf16(const float* X, int64_t n, uint16_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(to_bf16_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream,
                     X, n, reinterpret_cast<__bf16*>(out));
  return hipGetLastError();
}

struct MfArgs {
  const uint8_t* a;
  const uint8_t* b;
  int64_t stride, meta_off;
  int N, K, group;
  int64_t expert;
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* offsets;
  const int32_t* perm;
  int top_k;
  int xrows;
  const __bf16* X;
  int64_t M;
  void* out;
  int out_bf16;
  int64_t ld_out;
};

// Dequantize the lane's 16-byte chunk of codes into bf16.
template <int BITS>
__device__ __forceinline__ void dequant_chunk(const uint4& c, float2 m, bf16x8* out) {
  constexpr int CPL = BITS == 8 ? 16 : 32;
  float f[CPL];
  if constexpr (BITS == 8) {
    Codes<8>::unpack(c, f);
  } else {
    Codes<4>::unpack(c, f);
  }
#pragma unroll
  for (int j = 0; j < CPL / 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) out[j][e] = __bf16((f[8 * j + e] - m.y) * m.x);
}

// Workgroup: 4 waves x 16 rows = 64 rows of W; token tiles of 16 * TM.
template <int BITS, int TM, bool SWIGLU>
__global__ __launch_bounds__(256) void mfma_kernel(MfArgs p) {
  constexpr int CPL = BITS == 8 ? 16 : 32;  // codes per 16-byte chunk
  constexpr int KS = 4 * CPL;               // K per step (4 lane groups)
  constexpr int NI = CPL / 8;               // MFMA instructions per step
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int n_raw = blockIdx.x * 64 + wv * 16 + col;
  const int n = min(n_raw, p.N - 1);

  int64_t e, p0, M;
  const bool moe = p.active != nullptr;
  if (moe) {
    const int a = blockIdx.y;
    if (a >= *p.n_active) return;
    e = p.active[a];
    p0 = p.offsets[e];
    M = p.offsets[e + 1] - p0;
  } else {
    e = p.expert;
    p0 = 0;
    M = p.M;
  }
  const int64_t row_bytes = int64_t(p.K) * BITS / 8;
  const int64_t groups = p.K / p.group;
  const uint8_t* arow = p.a + e * p.stride + int64_t(n) * row_bytes;
  const float2* ameta = reinterpret_cast<const float2*>(p.a + e * p.stride + p.meta_off) +
                        int64_t(n) * groups;
  const uint8_t* brow = SWIGLU ? p.b + e * p.stride + int64_t(n) * row_bytes : nullptr;
  const float2* bmeta =
      SWIGLU ? reinterpret_cast<const float2*>(p.b + e * p.stride + p.meta_off) + int64_t(n) * groups
             : nullptr;

  const int64_t mstart = moe ? 0 : int64_t(blockIdx.y) * 16 * TM;
  const int64_t mstep = moe ? 16 * TM : int64_t(gridDim.y) * 16 * TM;
  for (int64_t m0 = mstart; m0 < M; m0 += mstep) {
    // x row of token (m0 + t*16 + col) for every tile t; -1 = padding
    int64_t xrow[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int64_t m = m0 + t * 16 + col;
      if (m < M) {
        const int64_t pidx = p0 + m;
        xrow[t] = p.xrows == XR_GATHER ? int64_t(p.perm[pidx] / p.top_k) : pidx;
      } else {
        xrow[t] = -1;
      }
    }
    f32x4 acc[TM], accb[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      accb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = 0; k0 < p.K; k0 += KS) {
      const int kk = k0 + kg * CPL;  // this lane's first k
      // INT4 steps are 128 wide while K is only a multiple of 64: a lane
      // group past the end contributes zeros (its x slice is zeroed too).
      const bool live = kk < p.K;
      bf16x8 wa[NI], wb[NI];
      if (live) {
        const uint4 c = *reinterpret_cast<const uint4*>(arow + int64_t(kk) * BITS / 8);
        dequant_chunk<BITS>(c, ameta[kk / p.group], wa);
        if constexpr (SWIGLU) {
          const uint4 cb = *reinterpret_cast<const uint4*>(brow + int64_t(kk) * BITS / 8);
          dequant_chunk<BITS>(cb, bmeta[kk / p.group], wb);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            wa[j][q] = __bf16(0.0f);
            wb[j][q] = __bf16(0.0f);
          }
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        bf16x8 xa[NI];
        if (xrow[t] >= 0 && live) {
          const uint4* src = reinterpret_cast<const uint4*>(p.X + xrow[t] * p.K + kk);
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const uint4 v = src[j];
            xa[j] = *reinterpret_cast<const bf16x8*>(&v);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q) xa[j][q] = __bf16(0.0f);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], wa[j], acc[t], 0, 0, 0);
          if constexpr (SWIGLU)
            accb[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], wb[j], accb[t], 0, 0, 0);
        }
      }
    }
    // lane holds rows (tokens) 4*kg + r of each tile, column col
#pragma unroll
    for (int t = 0; t < TM; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + t * 16 + kg * 4 + r;
        if (m < M && n_raw < p.N) {
          float o = acc[t][r];
          if constexpr (SWIGLU) o = silu(o) * accb[t][r];
          const int64_t orow = p0 + m;
          if (p.out_bf16)
            reinterpret_cast<__bf16*>(p.out)[orow * p.ld_out + n_raw] = __bf16(o);
          else
            reinterpret_cast<float*>(p.out)[orow * p.ld_out + n_raw] = o;
        }
      }
    }
  }
}

hipError_t launch_mfma_gemm(const dsq_qweight& A, const dsq_qweight* B, int64_t expert,
                            const Groups* grp, int xrows, const uint16_t* Xb, int64_t M,
                            void* out, int out_bf16, int64_t ld_out, hipStream_t stream) {
  const Layout L = layout_of(A.bits, A.group, A.K, A.N);
  MfArgs a{};
  a.a = static_cast<const uint8_t*>(A.data);
  a.b = B ? static_cast<const uint8_t*>(B->data) : nullptr;
  a.stride = L.stride;
  a.meta_off = L.meta_off;
  a.N = int(A.N);
  a.K = int(A.K);
  a.group = A.group;
  a.expert = expert;
  a.xrows = xrows;
  a.X = reinterpret_cast<const __bf16*>(Xb);
  a.M = M;
  a.out = out;
  a.out_bf16 = out_bf16;
  a.ld_out = ld_out;
  constexpr int TM = 2;
  int gy = 1;
  if (grp) {
    a.active = grp->active;
    a.n_active = grp->n_active;
    a.offsets = grp->offsets;
    a.perm = grp->perm;
    a.top_k = grp->top_k;
    gy = grp->max_items;
  } else {
    const int64_t tiles = (M + 16 * TM - 1) / (16 * TM);
    gy = int(tiles < 65535 ? tiles : 65535);
  }
  const int gx = int((A.N + 63) / 64);
  if (gx == 0 || gy == 0) return hipSuccess;
  const dim3 grid(gx, gy);
  const bool sw = B != nullptr;
  if (A.bits == 8 && !sw)
    hipLaunchKernelGGL((mfma_kernel<8, TM, false>), grid, dim3(256), 0, stream, a);
  else if (A.bits == 8)
    hipLaunchKernelGGL((mfma_kernel<8, TM, true>), grid, dim3(256), 0, stream, a);
  else if (!sw)
    hipLaunchKernelGGL((mfma_kernel<4, TM, false>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((mfma_kernel<4, TM, true>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsq
