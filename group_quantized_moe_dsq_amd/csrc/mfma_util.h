// mfma_util.h -- helpers shared by the matrix-core kernels: operand vector
// types, conversion of packed codes to exact bf16 operands, raw buffer
// descriptors and explicit memory-counter waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsq {

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

constexpr int kNT = 0;  // aux of the register loads: default caching
// Cache policy of the code loads.  Each 128-byte line of codes is consumed
// whole by one direct load, yet the nontemporal hint measured ~15% slower
// than default caching on this path, so the default stays.
#ifndef DSQ_GMM_CODE_AUX
#define DSQ_GMM_CODE_AUX 0
#endif
constexpr int kCodeAux = DSQ_GMM_CODE_AUX;

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


typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most N of this wave's global loads are outstanding (loads
// complete in order for this count).  The empty asm with a memory clobber
// keeps the compiler from moving LDS reads of the data these loads bring
// above the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}

// Workgroup barrier once the wave's own LDS accesses are done.  The memory
// clobber keeps the compiler from moving LDS accesses across it; unlike
// __syncthreads() it does not wait for the wave's outstanding global loads,
// which are the prefetches this kernel keeps in flight.
// 8-byte LDS read the compiler's wait analysis does not see.  Once a direct
// global->LDS load is outstanding, the compiler puts a full vmcnt(0) wait in
// front of LDS reads it cannot prove disjoint from every such load, which
// would drain a ring's lookahead; reads whose data a stream's own explicit
// wait already covers go through here.  The value may be used only after
// lgkm_wait(v), which waits for the read and, by taking v as an operand,
// keeps every use of v behind the wait.
__device__ __forceinline__ f32x2_t lds_read_f32x2(const void* p) {
  f32x2_t v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(uint32_t(size_t((lds_ptr_t)p))) : "memory");
  return v;
}
__device__ __forceinline__ void lgkm_wait(f32x2_t& v) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v) : : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


}  // namespace dsq
