// api.hip -- the C ABI of libdsq (declared in include/dsq.h).
//
// Every entry point validates its arguments on the host first (the
// up-front shape validation of "ds4 code walkthrough", Part 1, trace 5),
// returns a status instead of exiting, allocates nothing (callers pass
// workspace; the same walkthrough forbids allocation in the token loop) and
// only enqueues work on the caller's stream (dsq_moe_ffn_cached alone waits
// for it once: the host must see the routing to fetch experts).
#include <float.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "internal.h"

using namespace dsq;

// Scratch of dsq_moe_ffn_noalloc: one fixed array per device, loaded with
// the library's code object (so no allocation at call time).  In host code
// `scratch` names a host-side stand-in, never the device address: the
// device address comes from hipGetSymbolAddress, taken once per device.
static __device__ __align__(256) uint8_t scratch[DSQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;
// Up to this many tokens the fp32 MoE runs each (token, slot) pair as its own
// GEMV instead of grouping tokens by expert.

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t lim = int64_t(1) << 62) {
  return a >= 0 && b >= 0 && (a == 0 || b <= lim / a);
}

// Shape rules of a packed weight (without the pointer).
dsq_status check_shape(int32_t bits, int32_t group, int64_t K, int64_t N, int64_t batch) {
  if (bits != 8 && bits != 4) return DSQ_ERR_INVALID_ARG;
  if (group != 64 && group != 128 && !(group == kSuperGroup && bits == 4))
    return DSQ_ERR_INVALID_ARG;
  if (K <= 0 || N <= 0 || batch <= 0) return DSQ_ERR_SHAPE;
  if (K % group != 0) return DSQ_ERR_SHAPE;
  if (K > kMaxDim || N > kMaxDim || batch > kMaxDim) return DSQ_ERR_OVERFLOW;
  if (!mul_ok(K, N) || !mul_ok(K * N, batch)) return DSQ_ERR_OVERFLOW;
  return DSQ_OK;
}

dsq_status check_qweight(const dsq_qweight* W) {
  if (!W || !W->data) return DSQ_ERR_INVALID_ARG;
  const dsq_status s = check_shape(W->bits, W->group, W->K, W->N, W->batch);
  if (s != DSQ_OK) return s;
  if (W->layout_version != DSQ_LAYOUT_VERSION || W->reserved != 0) return DSQ_ERR_LAYOUT;
  if (!aligned(W->data, 256)) return DSQ_ERR_ALIGN;
  return DSQ_OK;
}

// The matrix-core kernels (grouped GEMM, decode) address one entry's codes
// and its (scale, zp) table with 32-bit buffer offsets: an entry must stay
// below 2 GiB there (a larger one would read zeros past 2 GiB, not fault).
bool entry_fits_32(const dsq_qweight* W) {
  return layout_of(W->bits, W->group, W->K, W->N).stride <= int64_t(INT32_MAX);
}

dsq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return DSQ_OK;
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice) return DSQ_ERR_NO_DEVICE;
  return DSQ_ERR_HIP;
}

dsq_status check_device() {
  int d = -1;
  const hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) return hip_status(e) == DSQ_ERR_HIP ? DSQ_ERR_NO_DEVICE : hip_status(e);
  return DSQ_OK;
}

// Carves consecutive 256-byte aligned regions out of a workspace.
struct Carver {
  uint8_t* base;
  int64_t used = 0;
  bool overflow = false;
  explicit Carver(void* b) : base(static_cast<uint8_t*>(b)) {}
  void* take(int64_t n, int64_t elem) {
    if (!mul_ok(n, elem)) {
      overflow = true;
      return nullptr;
    }
    void* p = base ? base + used : nullptr;
    used += align256(n * elem);
    return p;
  }
};

bool use_bf16(int32_t math, int64_t M) {
  return math == DSQ_MATH_BF16_MFMA || (math == DSQ_MATH_AUTO && M >= 64);
}

struct MoeWs {
  float* logits;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
  int32_t* active;
  int32_t* n_active;
  uint32_t* bitmap;
  void* hbuf;
  float* ybuf;
  void* act;         // activations of the token tiles in MFMA operand order
  size_t act_bytes;
  float* xs;         // their per-group sums
  size_t xs_bytes;
  int4* tiles;       // token-tile table of the grouped GEMM
  int32_t* n_tiles;
  int64_t max_tiles;
  float* rparts;     // the router's K slices [ks][T][E] (ks = router_slices > 1)
};

int64_t moe_layout(void* ws, int64_t T, int32_t E, int32_t k, int64_t H, int64_t I, int group,
                   bool bf16, MoeWs* out, bool* overflow) {
  Carver c(ws);
  MoeWs m{};
  const int64_t nk = T * k;
  m.logits = static_cast<float*>(c.take(T * E, 4));
  m.idx = static_cast<int32_t*>(c.take(nk, 4));
  m.w = static_cast<float*>(c.take(nk, 4));
  m.counts = static_cast<int32_t*>(c.take(E, 4));
  m.offsets = static_cast<int32_t*>(c.take(E + 1, 4));
  m.perm = static_cast<int32_t*>(c.take(nk, 4));
  m.pos = static_cast<int32_t*>(c.take(nk, 4));
  m.active = static_cast<int32_t*>(c.take(E, 4));
  m.n_active = static_cast<int32_t*>(c.take(1, 4));
  m.bitmap = static_cast<uint32_t*>(c.take(int64_t(group_scratch_words(T, E)), 4));
  m.hbuf = c.take(nk * I, 4);
  m.ybuf = static_cast<float*>(c.take(nk * H, 4));
  // token tiles of the grouped GEMM: routed rows nk in at most min(nk, E) experts
  const int xp = bf16 ? 1 : 2;
  const int64_t kmax = H > I ? H : I;
  const int64_t segs = nk < E ? nk : E;
  m.act_bytes = gmm_act_bytes(nk, segs, xp, kmax);
  m.act = c.take(int64_t(m.act_bytes), 1);
  m.xs_bytes = gmm_xs_bytes(nk, segs, xp, kmax, group);
  m.xs = static_cast<float*>(c.take(int64_t(m.xs_bytes), 1));
  m.max_tiles = gmm_tiles_bound(nk, segs, xp);
  m.tiles = static_cast<int4*>(c.take(m.max_tiles, 16));
  m.n_tiles = static_cast<int32_t*>(c.take(1, 4));
  const int ks = router_slices(T, E, H);
  m.rparts = ks > 1 ? static_cast<float*>(c.take(int64_t(ks) * T * E, 4)) : nullptr;
  // the grouped GEMM addresses these with 32-bit offsets
  if (m.act_bytes > size_t(INT32_MAX) || m.xs_bytes > size_t(INT32_MAX)) c.overflow = true;
  if (out) *out = m;
  if (overflow) *overflow = c.overflow;
  return c.used;
}

}  // namespace

extern "C" {

const char* dsq_status_string(dsq_status s) {
  switch (s) {
    case DSQ_OK: return "DSQ_OK";
    case DSQ_ERR_INVALID_ARG: return "DSQ_ERR_INVALID_ARG: null pointer or value out of range";
    case DSQ_ERR_SHAPE: return "DSQ_ERR_SHAPE: inconsistent or unsupported shape";
    case DSQ_ERR_ALIGN: return "DSQ_ERR_ALIGN: pointer not aligned as required";
    case DSQ_ERR_WORKSPACE: return "DSQ_ERR_WORKSPACE: workspace missing or too small";
    case DSQ_ERR_UNSUPPORTED: return "DSQ_ERR_UNSUPPORTED: outside the implemented limits";
    case DSQ_ERR_NO_DEVICE: return "DSQ_ERR_NO_DEVICE: no HIP device";
    case DSQ_ERR_HIP: return "DSQ_ERR_HIP: HIP runtime or launch failure";
    case DSQ_ERR_OVERFLOW: return "DSQ_ERR_OVERFLOW: size computation overflows";
    case DSQ_ERR_LAYOUT: return "DSQ_ERR_LAYOUT: unknown packed layout version";
    default: return "unknown dsq_status";
  }
}

size_t dsq_packed_bytes(int32_t bits, int32_t group, int64_t K, int64_t N, int64_t batch) {
  if (check_shape(bits, group, K, N, batch) != DSQ_OK) return 0;
  const Layout L = layout_of(bits, group, K, N);
  if (!mul_ok(L.stride, batch)) return 0;
  return size_t(L.stride * batch);
}

dsq_status dsq_qweight_init(dsq_qweight* w, int32_t bits, int32_t group, int64_t K, int64_t N,
                            int64_t batch, void* data) {
  if (!w || !data) return DSQ_ERR_INVALID_ARG;
  const dsq_status s = check_shape(bits, group, K, N, batch);
  if (s != DSQ_OK) return s;
  if (!aligned(data, 256)) return DSQ_ERR_ALIGN;
  w->bits = bits;
  w->group = group;
  w->K = K;
  w->N = N;
  w->batch = batch;
  w->layout_version = DSQ_LAYOUT_VERSION;
  w->reserved = 0;
  w->data = data;
  return DSQ_OK;
}

dsq_status dsq_pack_weights(const float* src, const dsq_qweight* out, int64_t first,
                            int64_t count, int32_t* dev_flags, void* stream) {
  if (!src) return DSQ_ERR_INVALID_ARG;
  dsq_status s = check_qweight(out);
  if (s != DSQ_OK) return s;
  if (first < 0 || count < 0 || first > out->batch || count > out->batch - first)
    return DSQ_ERR_INVALID_ARG;
  if (!aligned(src, 16)) return DSQ_ERR_ALIGN;
  if (dev_flags && !aligned(dev_flags, 4)) return DSQ_ERR_ALIGN;
  if ((s = check_device()) != DSQ_OK) return s;
  return hip_status(launch_pack(src, *out, first, count, dev_flags, (hipStream_t)stream));
}

dsq_status dsq_gemv(const dsq_qweight* W, int64_t expert, const float* x, float* y,
                    void* stream) {
  dsq_status s = check_qweight(W);
  if (s != DSQ_OK) return s;
  if (!x || !y) return DSQ_ERR_INVALID_ARG;
  if (expert < 0 || expert >= W->batch) return DSQ_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 4)) return DSQ_ERR_ALIGN;
  if ((s = check_device()) != DSQ_OK) return s;
  return hip_status(launch_gemv(*W, expert, x, y, (hipStream_t)stream));
}

size_t dsq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t math) {
  if (M < 0 || N <= 0 || K <= 0) return 0;
  if (math != DSQ_MATH_FP32 && math != DSQ_MATH_BF16_MFMA && math != DSQ_MATH_AUTO) return 0;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || !mul_ok(M, K) || !mul_ok(M, N)) return 0;
  if (use_bf16(math, M)) return gemm_mfma_supported(M, N, K) ? gemm_mfma_workspace(M, N, K) : 0;
  if (M < 2) return 0;  // GEMV
  // fp32 path: the token tiles of the grouped GEMM (one segment), sized for
  // the smallest supported group
  const size_t a = gmm_act_bytes(M, 1, 2, K), x = gmm_xs_bytes(M, 1, 2, K, 64);
  if (a > size_t(INT32_MAX) || x > size_t(INT32_MAX)) return 0;
  return a + x;
}

dsq_status dsq_gemm(const dsq_qweight* W, int64_t expert, const float* X, float* Y, int64_t M,
                    int32_t math, void* workspace, size_t workspace_bytes, void* stream) {
  dsq_status s = check_qweight(W);
  if (s != DSQ_OK) return s;
  if (!X || !Y) return DSQ_ERR_INVALID_ARG;
  if (expert < 0 || expert >= W->batch) return DSQ_ERR_INVALID_ARG;
  if (math != DSQ_MATH_FP32 && math != DSQ_MATH_BF16_MFMA && math != DSQ_MATH_AUTO)
    return DSQ_ERR_INVALID_ARG;
  if (M < 0) return DSQ_ERR_SHAPE;
  if (M > kMaxDim || !mul_ok(M, W->K) || !mul_ok(M, W->N)) return DSQ_ERR_OVERFLOW;
  if (!aligned(X, 16) || !aligned(Y, 4)) return DSQ_ERR_ALIGN;
  const bool bf16 = use_bf16(math, M);
  if (W->group == kSuperGroup && (M >= 2 || bf16)) return DSQ_ERR_UNSUPPORTED;  // GEMV only
  if (M >= 2 && !bf16 && !entry_fits_32(W)) return DSQ_ERR_UNSUPPORTED;
  if (M >= 2 || bf16) {
    const size_t need = dsq_gemm_workspace_bytes(M, W->N, W->K, math);
    if (need == 0) return DSQ_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < need) return DSQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DSQ_ERR_ALIGN;
  }
  if (M == 0) return DSQ_OK;
  if ((s = check_device()) != DSQ_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (bf16) return hip_status(launch_gemm_mfma(*W, expert, X, Y, M, workspace, st));
  if (M == 1) return hip_status(launch_gemv(*W, expert, X, Y, st));
  const size_t act = gmm_act_bytes(M, 1, 2, W->K);
  const size_t xsb = gmm_xs_bytes(M, 1, 2, W->K, 64);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return hip_status(launch_gmm(*W, nullptr, expert, nullptr, XR_DENSE, X, W->K, M, 2, ws, act,
                               reinterpret_cast<float*>(ws + act), xsb, Y, W->N, st));
}

dsq_status dsq_moe_route_topk(const float* logits, const float* bias, int64_t T, int32_t E,
                              int32_t top_k, int32_t* idx, float* weights, void* stream) {
  if (!logits || !idx || !weights) return DSQ_ERR_INVALID_ARG;
  if (T < 0 || E <= 0 || top_k <= 0 || top_k > E) return DSQ_ERR_SHAPE;
  if (E > 4096 || top_k > 32 || T > kMaxDim) return DSQ_ERR_UNSUPPORTED;
  if (!aligned(logits, 4) || !aligned(idx, 4) || !aligned(weights, 4) ||
      (bias && !aligned(bias, 4)))
    return DSQ_ERR_ALIGN;
  if (T == 0) return DSQ_OK;
  dsq_status s = check_device();
  if (s != DSQ_OK) return s;
  return hip_status(launch_topk(logits, bias, T, E, top_k, idx, weights, (hipStream_t)stream));
}

size_t dsq_moe_group_workspace_bytes(int64_t T, int32_t E, int32_t top_k) {
  if (T < 0 || E <= 0 || top_k <= 0 || top_k > E) return 0;
  if (T > 65536 || E > 4096 || top_k > 32) return 0;
  // bitmap (+ prefixes), active list, its count
  return size_t(align256(int64_t(group_scratch_words(T, E)) * 4) + align256(int64_t(E) * 4) +
                align256(4));
}

dsq_status dsq_moe_group(const int32_t* idx, int64_t T, int32_t E, int32_t top_k,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!counts || !offsets || (T > 0 && (!idx || !perm || !pos))) return DSQ_ERR_INVALID_ARG;
  if (T < 0 || E <= 0 || top_k <= 0 || top_k > E) return DSQ_ERR_SHAPE;
  if (T > 65536 || E > 4096 || top_k > 32) return DSQ_ERR_UNSUPPORTED;
  if ((idx && !aligned(idx, 4)) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      (perm && !aligned(perm, 4)) || (pos && !aligned(pos, 4)))
    return DSQ_ERR_ALIGN;
  const size_t need = dsq_moe_group_workspace_bytes(T, E, top_k);
  if (!workspace || workspace_bytes < need) return DSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSQ_ERR_ALIGN;
  dsq_status s = check_device();
  if (s != DSQ_OK) return s;
  Carver c(workspace);
  uint32_t* scratch = static_cast<uint32_t*>(c.take(int64_t(group_scratch_words(T, E)), 4));
  int32_t* active = static_cast<int32_t*>(c.take(E, 4));
  int32_t* n_active = static_cast<int32_t*>(c.take(1, 4));
  return hip_status(launch_group(idx, T, top_k, E, scratch, counts, offsets, perm, pos, active,
                                 n_active, 1, nullptr, nullptr, (hipStream_t)stream));
}

size_t dsq_topk_workspace_bytes(int64_t N, int32_t k) {
  if (N <= 0 || N > INT32_MAX || k <= 0 || k > N || k > kHeadMaxK) return 0;
  return head_workspace(N, k);
}

dsq_status dsq_topk(const float* y, int64_t N, int32_t k, int32_t* idx, float* values,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!y || !idx || !values) return DSQ_ERR_INVALID_ARG;
  if (N <= 0 || k <= 0 || k > N) return DSQ_ERR_SHAPE;
  if (N > INT32_MAX || k > kHeadMaxK) return DSQ_ERR_UNSUPPORTED;
  if (!aligned(y, 4) || !aligned(idx, 4) || !aligned(values, 4)) return DSQ_ERR_ALIGN;
  const size_t need = head_workspace(N, k);
  if (!workspace || workspace_bytes < need) return DSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSQ_ERR_ALIGN;
  dsq_status s = check_device();
  if (s != DSQ_OK) return s;
  return hip_status(launch_head(y, N, k, idx, values, workspace, (hipStream_t)stream));
}

dsq_status dsq_gemv_topk(const dsq_qweight* W, int64_t expert, const float* x, float* y,
                         int32_t k, int32_t* idx, float* values, void* workspace,
                         size_t workspace_bytes, void* stream) {
  dsq_status s = check_qweight(W);
  if (s != DSQ_OK) return s;
  if (!x || !y || !idx || !values) return DSQ_ERR_INVALID_ARG;
  if (expert < 0 || expert >= W->batch) return DSQ_ERR_INVALID_ARG;
  if (k <= 0 || k > W->N) return DSQ_ERR_SHAPE;
  if (W->N > INT32_MAX || k > kHeadMaxK) return DSQ_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(y, 4) || !aligned(idx, 4) || !aligned(values, 4))
    return DSQ_ERR_ALIGN;
  const size_t need = head_workspace(W->N, k);
  if (!workspace || workspace_bytes < need) return DSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSQ_ERR_ALIGN;
  if ((s = check_device()) != DSQ_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (k == 1 && gemv_argmax_supported(*W)) {
    // top-1: the GEMV's waves rank their own outputs; one pick over their keys
    uint64_t* keys = static_cast<uint64_t*>(workspace);
    int64_t n = 0;
    hipError_t e = launch_gemv_argmax(*W, expert, x, y, keys, &n, st);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_head_from_keys(y, keys, n, idx, values, st));
  }
  hipError_t e = launch_gemv(*W, expert, x, y, st);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_head(y, W->N, k, idx, values, workspace, st));
}

size_t dsq_moe_workspace_bytes(int64_t T, int32_t E, int32_t top_k, int64_t H, int64_t I,
                               int32_t math) {
  if (T < 0 || E <= 0 || top_k <= 0 || top_k > E || H <= 0 || I <= 0) return 0;
  if (math != DSQ_MATH_FP32 && math != DSQ_MATH_BF16_MFMA && math != DSQ_MATH_AUTO) return 0;
  if (T > 65536 || E > 4096 || top_k > 32 || H > kMaxDim || I > kMaxDim) return 0;
  bool ovf = false;
  // the group size enters only the size of the per-group sums: size for the
  // smallest supported group
  const int64_t n = moe_layout(nullptr, T, E, top_k, H, I, 64, use_bf16(math, T), nullptr, &ovf);
  return ovf ? 0 : size_t(n);
}

}  // extern "C"

namespace {

// Shape and type rules shared by the MoE layer and the MoE block.
dsq_status check_moe(const float* X, const float* router_w, const float* bias,
                     const dsq_qweight* gate, const dsq_qweight* up, const dsq_qweight* down,
                     int64_t T, int32_t top_k, int32_t math, const float* Y,
                     const float* logits_out, const int32_t* idx_out, const float* w_out,
                     const int32_t* expert_counts_out) {
  if (!X || !router_w || !Y) return DSQ_ERR_INVALID_ARG;
  dsq_status s;
  if ((s = check_qweight(gate)) != DSQ_OK) return s;
  if ((s = check_qweight(up)) != DSQ_OK) return s;
  if ((s = check_qweight(down)) != DSQ_OK) return s;
  if (math != DSQ_MATH_FP32 && math != DSQ_MATH_BF16_MFMA && math != DSQ_MATH_AUTO)
    return DSQ_ERR_INVALID_ARG;
  const int64_t E64 = gate->batch;
  const int64_t H = gate->K, I = gate->N;
  if (up->batch != E64 || down->batch != E64) return DSQ_ERR_SHAPE;
  if (up->K != H || up->N != I || down->K != I || down->N != H) return DSQ_ERR_SHAPE;
  if (up->bits != gate->bits || down->bits != gate->bits || up->group != gate->group ||
      down->group != gate->group)
    return DSQ_ERR_SHAPE;
  if (gate->group == kSuperGroup) return DSQ_ERR_UNSUPPORTED;  // GEMV only
  if (!entry_fits_32(gate) || !entry_fits_32(down)) return DSQ_ERR_UNSUPPORTED;
  if (T < 0 || top_k <= 0 || top_k > E64) return DSQ_ERR_SHAPE;
  if (T > 65536 || E64 > 4096 || top_k > 32) return DSQ_ERR_UNSUPPORTED;
  if (!aligned(X, 16) || !aligned(router_w, 16) || !aligned(Y, 16) || (bias && !aligned(bias, 4)))
    return DSQ_ERR_ALIGN;
  if ((logits_out && !aligned(logits_out, 4)) || (idx_out && !aligned(idx_out, 4)) ||
      (w_out && !aligned(w_out, 4)) || (expert_counts_out && !aligned(expert_counts_out, 4)))
    return DSQ_ERR_ALIGN;
  return DSQ_OK;
}

// The MoE layer of the pages (§3.5) on the rows X.  With gamma the rows are
// RMS-normalised into xn first and the experts see xn (§2.1: RMSNorm before
// the MoE step); with resid the residual is added to Y.
// With given_idx/given_w the routing is given (entries index the weight
// batches, e.g. expert-cache slots): no router and no top-k run.
dsq_status run_moe(const float* X, const float* gamma, float eps, float* xn, const float* resid,
                   const float* router_w, const float* bias, const dsq_qweight& gate,
                   const dsq_qweight& up, const dsq_qweight& down, int64_t T, int32_t top_k,
                   bool bf16, float* Y, void* workspace, float* logits_out, int32_t* idx_out,
                   float* w_out, int32_t* expert_counts_out, const int32_t* given_idx,
                   const float* given_w, hipStream_t st) {
  const int32_t E = int32_t(gate.batch);
  const int64_t E64 = gate.batch, H = gate.K, I = gate.N;
  MoeWs m{};
  moe_layout(workspace, T, E, top_k, H, I, 64, bf16, &m, nullptr);
  if (logits_out) m.logits = logits_out;
  if (idx_out) m.idx = idx_out;
  if (w_out) m.w = w_out;
  if (expert_counts_out) m.counts = expert_counts_out;
  const bool given = given_idx != nullptr;
  if (given) {
    m.idx = const_cast<int32_t*>(given_idx);  // only read
    m.w = const_cast<float*>(given_w);
  }
  // the rows the experts (and a separate router) read
  const float* Xe = gamma ? xn : X;
  hipError_t e;
#define DSQ_TRY(call)                          \
  if ((e = (call)) != hipSuccess) return hip_status(e);
  if (!bf16 && T <= kDecodeMaxTokens && decode_supported(gate.bits, H, I, E, top_k)) {
    // Decode: every (token, slot) pair is its own GEMV; no grouping needed.
    // The gate/up kernel ranks the scores itself and publishes idx/w.
    if (!given)
      DSQ_TRY(launch_router_gemv(X, T, router_w, bias, E, H, m.logits, gamma, eps, xn, st));
    DSQ_TRY(launch_moe_decode(gate, up, down, Xe, T, E, top_k, given ? nullptr : m.logits, m.idx,
                              m.w, static_cast<float*>(m.hbuf), Y, resid, st));
    if (expert_counts_out) {
      DSQ_TRY(launch_group(m.idx, T, top_k, E, m.bitmap, m.counts, m.offsets, m.perm, m.pos,
                           m.active, m.n_active, 0, nullptr, nullptr, st));
    }
    return DSQ_OK;
  }
  if (!given) {
    // (0) + (1) normalisation and router logits, fp32, bias included;
    // (2) softmax + top-k + renormalisation.  Up to 32 tokens the GEMV router
    // (the norm fused in) serves the block and shapes the matrix-core router
    // does not take; otherwise the matrix-core router, its K split over
    // several workgroups when the token x expert tiles are too few to fill
    // the chip, the slices added by the top-k kernel.
    const int ks = router_slices(T, E, H);
    if (T <= 32 && (gamma || ks == 0)) {
      DSQ_TRY(launch_router_gemv(X, T, router_w, bias, E, H, m.logits, gamma, eps, xn, st));
      DSQ_TRY(launch_topk(m.logits, nullptr, T, E, top_k, m.idx, m.w, st));
    } else {
      if (gamma) DSQ_TRY(launch_rmsnorm(X, gamma, T, H, eps, xn, st));
      if (ks > 1) {
        DSQ_TRY(launch_router(Xe, T, router_w, nullptr, E, H, m.rparts, ks, st));
        DSQ_TRY(launch_topk_parts(m.rparts, ks, bias, m.logits, T, E, top_k, m.idx, m.w, st));
      } else {
        DSQ_TRY(launch_router(Xe, T, router_w, bias, E, H, m.logits, ks, st));
        DSQ_TRY(launch_topk(m.logits, nullptr, T, E, top_k, m.idx, m.w, st));
      }
    }
  }
  // (3) stable grouping by expert, and the token tiles of the grouped GEMMs
  const int xp = bf16 ? 1 : 2;
  DSQ_TRY(launch_group(m.idx, T, top_k, E, m.bitmap, m.counts, m.offsets, m.perm, m.pos, m.active,
                       m.n_active, 16 / xp, m.tiles, m.n_tiles, st));
  Groups g{};
  g.active = m.active;
  g.n_active = m.n_active;
  g.offsets = m.offsets;
  g.perm = m.perm;
  g.top_k = top_k;
  const int64_t max_items = T * top_k < E64 ? T * top_k : E64;
  g.max_items = int32_t(max_items);
  g.tiles = m.tiles;
  g.n_tiles = m.n_tiles;
  g.max_tiles = int32_t(m.max_tiles);
  // (4) expert FFNs over their token groups, (5) weighted combine (+ residual)
  float* hbuf = static_cast<float*>(m.hbuf);
  DSQ_TRY(launch_gmm(gate, &up, 0, &g, XR_GATHER, Xe, H, 0, xp, m.act, m.act_bytes, m.xs,
                     m.xs_bytes, hbuf, I, st));
  DSQ_TRY(launch_gmm(down, nullptr, 0, &g, XR_SEGMENT, hbuf, I, 0, xp, m.act, m.act_bytes, m.xs,
                     m.xs_bytes, m.ybuf, H, st));
  DSQ_TRY(launch_combine(m.ybuf, m.pos, m.w, T, top_k, H, resid, Y, st));
#undef DSQ_TRY
  return DSQ_OK;
}

}  // namespace

extern "C" {

dsq_status dsq_moe_ffn(const float* X, const float* router_w, const float* bias,
                       const dsq_qweight* gate, const dsq_qweight* up, const dsq_qweight* down,
                       int64_t T, int32_t top_k, int32_t math, float* Y, void* workspace,
                       size_t workspace_bytes, float* logits_out, int32_t* idx_out,
                       float* w_out, int32_t* expert_counts_out, void* stream) {
  dsq_status s = check_moe(X, router_w, bias, gate, up, down, T, top_k, math, Y, logits_out,
                           idx_out, w_out, expert_counts_out);
  if (s != DSQ_OK) return s;
  const size_t need =
      dsq_moe_workspace_bytes(T, int32_t(gate->batch), top_k, gate->K, gate->N, math);
  if (need == 0) return DSQ_ERR_OVERFLOW;
  if (!workspace || workspace_bytes < need) return DSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSQ_ERR_ALIGN;
  if (T == 0) return DSQ_OK;
  if ((s = check_device()) != DSQ_OK) return s;
  return run_moe(X, nullptr, 0.0f, nullptr, nullptr, router_w, bias, *gate, *up, *down, T, top_k,
                 use_bf16(math, T), Y, workspace, logits_out, idx_out, w_out, expert_counts_out,
                 nullptr, nullptr, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept for the process.
dsq_status noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int d = -1;
  const hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) return DSQ_ERR_NO_DEVICE;
  if (d < 0 || d >= kMaxDevices) return DSQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[d]) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || !p) return DSQ_ERR_HIP;
    addr[d] = p;
  }
  *out = addr[d];
  return DSQ_OK;
}

}  // namespace

extern "C" {

dsq_status dsq_moe_ffn_noalloc(const float* X, const float* router_w, const float* bias,
                               const dsq_qweight* gate, const dsq_qweight* up,
                               const dsq_qweight* down, int64_t T, int32_t top_k, int32_t math,
                               float* Y, float* logits_out, int32_t* idx_out, float* w_out,
                               int32_t* expert_counts_out, void* stream) {
  dsq_status s = check_moe(X, router_w, bias, gate, up, down, T, top_k, math, Y, logits_out,
                           idx_out, w_out, expert_counts_out);
  if (s != DSQ_OK) return s;
  const size_t need =
      dsq_moe_workspace_bytes(T, int32_t(gate->batch), top_k, gate->K, gate->N, math);
  if (need == 0) return DSQ_ERR_OVERFLOW;
  if (need > size_t(DSQ_NOALLOC_SCRATCH_BYTES)) return DSQ_ERR_WORKSPACE;
  if (T == 0) return DSQ_OK;
  if ((s = check_device()) != DSQ_OK) return s;
  void* ws = nullptr;
  if ((s = noalloc_scratch(&ws)) != DSQ_OK) return s;
  // the MoE kernels overwrite every scratch word they read, so the previous
  // call's contents need no clearing
  return run_moe(X, nullptr, 0.0f, nullptr, nullptr, router_w, bias, *gate, *up, *down, T, top_k,
                 use_bf16(math, T), Y, ws, logits_out, idx_out, w_out, expert_counts_out,
                 nullptr, nullptr, (hipStream_t)stream);
}

size_t dsq_moe_block_workspace_bytes(int64_t T, int32_t E, int32_t top_k, int64_t H, int64_t I,
                                     int32_t math) {
  const size_t moe = dsq_moe_workspace_bytes(T, E, top_k, H, I, math);
  if (moe == 0) return 0;
  // the normalised rows come first
  return size_t(align256(T * H * 4)) + moe;
}

dsq_status dsq_moe_block(const float* X, const float* norm_w, float eps, const float* router_w,
                         const float* bias, const dsq_qweight* gate, const dsq_qweight* up,
                         const dsq_qweight* down, int64_t T, int32_t top_k, int32_t math,
                         float* Y, void* workspace, size_t workspace_bytes, float* xn_out,
                         float* logits_out, int32_t* idx_out, float* w_out,
                         int32_t* expert_counts_out, void* stream) {
  dsq_status s = check_moe(X, router_w, bias, gate, up, down, T, top_k, math, Y, logits_out,
                           idx_out, w_out, expert_counts_out);
  if (s != DSQ_OK) return s;
  if (!norm_w) return DSQ_ERR_INVALID_ARG;
  if (!(eps > 0.0f) || !(eps <= FLT_MAX)) return DSQ_ERR_INVALID_ARG;  // rejects NaN too
  if (!aligned(norm_w, 16) || (xn_out && !aligned(xn_out, 16))) return DSQ_ERR_ALIGN;
  const size_t need =
      dsq_moe_block_workspace_bytes(T, int32_t(gate->batch), top_k, gate->K, gate->N, math);
  if (need == 0) return DSQ_ERR_OVERFLOW;
  if (!workspace || workspace_bytes < need) return DSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSQ_ERR_ALIGN;
  if (T == 0) return DSQ_OK;
  if ((s = check_device()) != DSQ_OK) return s;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* xn = xn_out ? xn_out : reinterpret_cast<float*>(ws);
  return run_moe(X, norm_w, eps, xn, X, router_w, bias, *gate, *up, *down, T, top_k,
                 use_bf16(math, T), Y, ws + align256(T * gate->K * 4), logits_out, idx_out, w_out,
                 expert_counts_out, nullptr, nullptr, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// Expert cache ("Running a 284B-parameter LLM from 3.2 GB of RAM in plain C":
// the router picks the experts, only those are streamed into an LRU cache).
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

int64_t entry_stride(const dsq_qweight& W) { return layout_of(W.bits, W.group, W.K, W.N).stride; }

dsq_status check_cache(const dsq_expert_cache* c) {
  if (!c || !c->host_gate || !c->host_up || !c->host_down || !c->slot_of || !c->expert_of ||
      !c->last_use || c->E < 1)
    return DSQ_ERR_INVALID_ARG;
  dsq_status s;
  if ((s = check_qweight(&c->gate)) != DSQ_OK) return s;
  if ((s = check_qweight(&c->up)) != DSQ_OK) return s;
  if ((s = check_qweight(&c->down)) != DSQ_OK) return s;
  const int64_t H = c->gate.K, I = c->gate.N, S = c->gate.batch;
  if (c->up.batch != S || c->down.batch != S || c->slots != S) return DSQ_ERR_SHAPE;
  if (c->up.K != H || c->up.N != I || c->down.K != I || c->down.N != H) return DSQ_ERR_SHAPE;
  if (c->up.bits != c->gate.bits || c->down.bits != c->gate.bits ||
      c->up.group != c->gate.group || c->down.group != c->gate.group)
    return DSQ_ERR_SHAPE;
  if (c->gate.group == kSuperGroup) return DSQ_ERR_UNSUPPORTED;
  return DSQ_OK;
}

// Maps experts[0..n) to slots as one call; fill(expert, slot) for each miss.
template <class Fill>
dsq_status cache_map(dsq_expert_cache* c, const int32_t* experts, int64_t n, int32_t* slot_out,
                     Fill&& fill) {
  // every request takes the next stamp; this call's stamps are >= first
  const uint64_t first = c->clock + 1;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t e = experts[i];
    if (e < 0 || e >= c->E) return DSQ_ERR_INVALID_ARG;
    const uint64_t now = ++c->clock;
    int32_t s = c->slot_of[e];
    if (s >= 0) {
      ++c->hits;
    } else {
      // an empty slot (stamp 0; the lowest index) first, else the least
      // recently used slot that this call has not used
      int32_t v = -1;
      uint64_t best = ~uint64_t(0);
      for (int32_t j = 0; j < c->slots; ++j) {
        const uint64_t t = c->expert_of[j] < 0 ? 0 : c->last_use[j];
        if (t < first && t < best) {
          best = t;
          v = j;
        }
      }
      if (v < 0) return DSQ_ERR_UNSUPPORTED;
      if (c->expert_of[v] >= 0) c->slot_of[c->expert_of[v]] = -1;
      c->expert_of[v] = e;
      c->slot_of[e] = v;
      s = v;
      ++c->misses;
      const dsq_status f = fill(e, v);
      if (f != DSQ_OK) return f;
    }
    c->last_use[s] = now;
    if (slot_out) slot_out[i] = s;
  }
  return DSQ_OK;
}

}  // namespace

extern "C" {

dsq_status dsq_expert_cache_init(dsq_expert_cache* cache, const dsq_qweight* gate,
                                 const dsq_qweight* up, const dsq_qweight* down,
                                 const void* host_gate, const void* host_up,
                                 const void* host_down, int32_t E, int32_t* slot_of,
                                 int32_t* expert_of, uint64_t* last_use) {
  if (!cache || !gate || !up || !down) return DSQ_ERR_INVALID_ARG;
  dsq_expert_cache c{};
  c.gate = *gate;
  c.up = *up;
  c.down = *down;
  c.host_gate = host_gate;
  c.host_up = host_up;
  c.host_down = host_down;
  c.E = E;
  c.slots = gate->batch > INT32_MAX ? -1 : int32_t(gate->batch);
  c.slot_of = slot_of;
  c.expert_of = expert_of;
  c.last_use = last_use;
  const dsq_status s = check_cache(&c);
  if (s != DSQ_OK) return s;
  for (int32_t e = 0; e < E; ++e) slot_of[e] = -1;
  for (int32_t j = 0; j < c.slots; ++j) {
    expert_of[j] = -1;
    last_use[j] = 0;
  }
  *cache = c;
  return DSQ_OK;
}

dsq_status dsq_expert_cache_plan(dsq_expert_cache* cache, const int32_t* experts, int64_t n,
                                 int32_t* slot_out, int32_t* fill_expert, int32_t* fill_slot,
                                 int64_t* n_fill) {
  dsq_status s = check_cache(cache);
  if (s != DSQ_OK) return s;
  if (n < 0 || (n > 0 && (!experts || !slot_out || !fill_expert || !fill_slot)) || !n_fill)
    return DSQ_ERR_INVALID_ARG;
  int64_t nf = 0;
  s = cache_map(cache, experts, n, slot_out, [&](int32_t e, int32_t v) {
    fill_expert[nf] = e;
    fill_slot[nf] = v;
    ++nf;
    return DSQ_OK;
  });
  *n_fill = nf;
  return s;
}

size_t dsq_moe_cached_workspace_bytes(int64_t T, int32_t E, int32_t slots, int32_t top_k,
                                      int64_t H, int64_t I, int32_t math) {
  if (E < 1 || E > 4096) return 0;
  const size_t moe = dsq_moe_workspace_bytes(T, slots, top_k, H, I, math);
  if (moe == 0) return 0;
  // router logits [T][E], expert ids, weights and slots [T][k]
  return size_t(align256(T * E * 4) + 3 * align256(T * top_k * 4)) + moe;
}

dsq_status dsq_moe_ffn_cached(const float* X, const float* router_w, const float* bias,
                              dsq_expert_cache* cache, int64_t T, int32_t top_k, int32_t math,
                              float* Y, void* workspace, size_t workspace_bytes,
                              int32_t* host_idx, int32_t* host_slots, float* logits_out,
                              int32_t* idx_out, float* w_out, void* stream) {
  dsq_status s = check_cache(cache);
  if (s != DSQ_OK) return s;
  if ((s = check_moe(X, router_w, bias, &cache->gate, &cache->up, &cache->down, T, top_k, math, Y,
                     logits_out, idx_out, w_out, nullptr)) != DSQ_OK)
    return s;
  if (top_k > cache->E) return DSQ_ERR_SHAPE;
  if (T > 0 && (!host_idx || !host_slots)) return DSQ_ERR_INVALID_ARG;
  const int32_t E = cache->E;
  const int64_t H = cache->gate.K, I = cache->gate.N;
  const size_t need = dsq_moe_cached_workspace_bytes(T, E, cache->slots, top_k, H, I, math);
  if (need == 0) return DSQ_ERR_OVERFLOW;
  if (!workspace || workspace_bytes < need) return DSQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSQ_ERR_ALIGN;
  if (T == 0) return DSQ_OK;
  if ((s = check_device()) != DSQ_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  Carver cv(workspace);
  float* logits = static_cast<float*>(cv.take(T * E, 4));
  int32_t* idx = static_cast<int32_t*>(cv.take(T * top_k, 4));
  float* w = static_cast<float*>(cv.take(T * top_k, 4));
  int32_t* slots_dev = static_cast<int32_t*>(cv.take(T * top_k, 4));
  void* moe_ws = static_cast<uint8_t*>(workspace) + cv.used;
  if (logits_out) logits = logits_out;
  if (idx_out) idx = idx_out;
  if (w_out) w = w_out;
  hipError_t e;
#define DSQ_TRY(call)                          \
  if ((e = (call)) != hipSuccess) return hip_status(e);
  // (1) routing on the GPU
  if (T <= 32) {
    DSQ_TRY(launch_router_gemv(X, T, router_w, bias, E, H, logits, nullptr, 0.0f, nullptr, st));
  } else {
    DSQ_TRY(launch_router(X, T, router_w, bias, E, H, logits,
                          router_slices(T, E, H) > 0 ? 1 : 0, st));
  }
  DSQ_TRY(launch_topk(logits, nullptr, T, E, top_k, idx, w, st));
  // (2) the host sees the routing
  const size_t nb = size_t(T * top_k) * 4;
  DSQ_TRY(hipMemcpyAsync(host_idx, idx, nb, hipMemcpyDeviceToHost, st));
  DSQ_TRY(hipStreamSynchronize(st));
  // (3) slots for the requested experts; misses copied from the host stores
  const int64_t sg = entry_stride(cache->gate), su = entry_stride(cache->up),
                sd = entry_stride(cache->down);
  s = cache_map(cache, host_idx, T * top_k, host_slots, [&](int32_t ex, int32_t v) {
    const struct {
      void* dst;
      const void* src;
      int64_t n;
    } cp[3] = {
        {static_cast<uint8_t*>(cache->gate.data) + v * sg,
         static_cast<const uint8_t*>(cache->host_gate) + ex * sg, sg},
        {static_cast<uint8_t*>(cache->up.data) + v * su,
         static_cast<const uint8_t*>(cache->host_up) + ex * su, su},
        {static_cast<uint8_t*>(cache->down.data) + v * sd,
         static_cast<const uint8_t*>(cache->host_down) + ex * sd, sd}};
    for (const auto& c : cp) {
      const hipError_t ce = hipMemcpyAsync(c.dst, c.src, size_t(c.n), hipMemcpyHostToDevice, st);
      if (ce != hipSuccess) return hip_status(ce);
      cache->bytes_copied += uint64_t(c.n);
    }
    return DSQ_OK;
  });
  if (s != DSQ_OK) return s;
  DSQ_TRY(hipMemcpyAsync(slots_dev, host_slots, nb, hipMemcpyHostToDevice, st));
#undef DSQ_TRY
  // (4) the expert FFN on the slots, routing given
  return run_moe(X, nullptr, 0.0f, nullptr, nullptr, router_w, bias, cache->gate, cache->up,
                 cache->down, T, top_k, use_bf16(math, T), Y, moe_ws, nullptr, nullptr, nullptr,
                 nullptr, slots_dev, w, st);
}

}  // extern "C"
