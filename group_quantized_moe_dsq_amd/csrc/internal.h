// internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsq.h"

namespace dsq {

hipError_t launch_pack(const float* src, const dsq_qweight& W, int64_t first, int64_t count,
                       int32_t* flags, hipStream_t stream);

// y = W[expert] x  (M = 1); the super-block format (group 256) goes to
// launch_gemv_sb4 (gemv_sb4.hip)
hipError_t launch_gemv(const dsq_qweight& W, int64_t expert, const float* x, float* y,
                       hipStream_t stream);
hipError_t launch_gemv_sb4(const dsq_qweight& W, int64_t expert, const float* x, float* y,
                           hipStream_t stream);

// Routing description for the grouped kernels.  In dense mode `active` is
// NULL and the single "expert" covers tokens 0..M-1.
struct Groups {
  const int32_t* active;    // [E] experts with tokens, ascending (NULL: dense)
  const int32_t* n_active;  // device scalar
  const int32_t* offsets;   // [E+1] segment starts in perm order
  const int32_t* perm;      // [T*k] entry j = t*k+i in (expert, j) order
  int32_t top_k;
  int32_t max_items;        // bound on the number of active experts (0: no rows)
  // token tiles in (active expert, tile) order, one record each:
  // {expert, first row in perm order, rows in the tile (<= 16 / xp),
  //  activation tile index}; count in *n_tiles, at most max_tiles
  const int4* tiles;
  const int32_t* n_tiles;
  int32_t max_tiles;
};

// Where the rows of a grouped GEMM come from:
//  dense -> X + m*K ; moe gather -> X + (perm[p]/top_k)*K ; moe segment -> X + p*K.
enum XRows { XR_DENSE = 0, XR_GATHER = 1, XR_SEGMENT = 2 };

// fp32 router: logits[t][e] = X[t] . Wr[e] (+ bias[e]), on the matrix cores with K split over ks workgroups
// (ks = router_slices(T, E, H); 0 = the VALU kernel).  ks == 1: logits
// [T][E] with the bias; ks > 1: partial sums [ks][T][E] without it, for
// launch_topk_parts.
constexpr int kRouterMaxSlices = 16;
int router_slices(int64_t T, int32_t E, int64_t H);
hipError_t launch_router(const float* X, int64_t T, const float* Wr, const float* bias,
                         int32_t E, int64_t H, float* logits, int ks, hipStream_t stream);

hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                       int32_t* idx, float* w, hipStream_t stream);
// top-k on the router's K slices: logits = sum of the slices in order + rbias
// (written out), then as launch_topk without a selection bias
hipError_t launch_topk_parts(const float* parts, int nparts, const float* rbias, float* logits,
                             int64_t T, int32_t E, int32_t k, int32_t* idx, float* w,
                             hipStream_t stream);

// Stable grouping of the T*k routing entries by expert (E <= 4096): counts,
// offsets, perm (entries in (expert, entry) order), pos (perm's inverse; -1
// for an entry whose expert is outside [0, E)), the active experts.  With
// tiles, also the token-tile table of the grouped GEMM for tiles of tpt rows
// (Groups::tiles; at most gmm_tiles_bound(T*k, min(T*k, E), 16/tpt)).
// scratch: group_scratch_words(T, E) 32-bit words (bitmap, and for many
// tokens the per-expert popcount prefixes).
size_t group_scratch_words(int64_t T, int32_t E);
hipError_t launch_group(const int32_t* idx, int64_t T, int32_t k, int32_t E, uint32_t* scratch,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                        int32_t* active, int32_t* n_active, int tpt, int4* tiles,
                        int32_t* n_tiles, hipStream_t stream);

// Y[t][n] = (resid[t][n] +) sum_i w[t][i] * ybuf[pos[t*k+i]][n]; Y may be resid
hipError_t launch_combine(const float* ybuf, const int32_t* pos, const float* w, int64_t T,
                          int32_t k, int64_t H, const float* resid, float* Y,
                          hipStream_t stream);

// xn[t] = X[t] / sqrt(mean(X[t]^2) + eps) * gamma, one workgroup per row
hipError_t launch_rmsnorm(const float* X, const float* gamma, int64_t T, int64_t H, float eps,
                          float* xn, hipStream_t stream);

// Decode path (few tokens): fp32 router GEMV, and the expert FFN per routing
// slot on the matrix cores (gate/up + SwiGLU into hbuf [T*k][I], then down
// fused with the weighted combine into Y).
// With gamma, the rows are RMS-normalised first and the normalised rows are
// written to xn (when xn is not NULL).
hipError_t launch_router_gemv(const float* X, int64_t T, const float* Wr, const float* bias,
                              int32_t E, int64_t H, float* logits, const float* gamma, float eps,
                              float* xn, hipStream_t stream);
constexpr int64_t kDecodeMaxTokens = 4;  // decode kernels: at most this many tokens
bool decode_supported(int bits, int64_t H, int64_t I, int32_t E, int32_t k);
// Ranks each token's scores itself (writing idx/w), so no separate top-k;
// with logits NULL the routing idx/w is read as given.
hipError_t launch_moe_decode(const dsq_qweight& gate, const dsq_qweight& up,
                             const dsq_qweight& down, const float* X, int64_t T, int32_t E,
                             int32_t k, const float* logits, int32_t* idx, float* w, float* hbuf,
                             float* Y, const float* resid, hipStream_t stream);

// bf16 MFMA dense GEMM (prefill): the workspace holds the fp32 partial
// tiles when the K range is split.  Supported while X and one weight entry
// stay below 2 GiB (32-bit buffer offsets).
bool gemm_mfma_supported(int64_t M, int64_t N, int64_t K);
size_t gemm_mfma_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mfma(const dsq_qweight& W, int64_t expert, const float* X, float* Y,
                            int64_t M, void* workspace, hipStream_t stream);

// Grouped fused-dequant GEMM on bf16 MFMA (tokens grouped by expert, or one
// dense matrix).  xp = 2: activations split into two bf16 parts (fp32-accurate
// results); xp = 1: activations rounded to bf16.  The prep step writes the
// activations of every token tile into `act`/`xs` (sizes from gmm_act_bytes /
// gmm_xs_bytes for `rows` routed rows in at most `segments` experts).
// out rows: dense -> m ; grouped -> p (perm order).  With B (SwiGLU up) the
// output is silu(x A^T) * (x B^T).
int64_t gmm_tiles_bound(int64_t rows, int64_t segments, int xp);
size_t gmm_act_bytes(int64_t rows, int64_t segments, int xp, int64_t K);
size_t gmm_xs_bytes(int64_t rows, int64_t segments, int xp, int64_t K, int group);
hipError_t launch_gmm(const dsq_qweight& A, const dsq_qweight* B, int64_t expert,
                      const Groups* grp, int xrows, const float* X, int64_t ld_x, int64_t M,
                      int xp, void* act, size_t act_bytes, float* xs, size_t xs_bytes,
                      float* out, int64_t ld_out, hipStream_t stream);

// GEMV that also writes every wave's best rank key (head_key.h) of its
// outputs to wkey (at most gemv_argmax_key_bytes()) and their count to
// nkeys; for the group formats with rows of at most 4 16-byte chunks per lane.
bool gemv_argmax_supported(const dsq_qweight& W);
size_t gemv_argmax_key_bytes();
hipError_t launch_gemv_argmax(const dsq_qweight& W, int64_t expert, const float* x, float* y,
                              uint64_t* wkey, int64_t* nkeys, hipStream_t stream);

// Output-head selection: the k (<= kHeadMaxK) largest of N logits in rank
// order (head.hip).  Workspace: head_workspace(N, k) bytes.
constexpr int32_t kHeadMaxK = 256;
size_t head_workspace(int64_t N, int32_t k);
hipError_t launch_head(const float* y, int64_t N, int32_t k, int32_t* idx, float* val,
                       void* workspace, hipStream_t stream);
// Top-1 from n (<= 4096) rank keys, e.g. launch_gemv_argmax's; y holds the
// values the keys index.
hipError_t launch_head_from_keys(const float* y, const uint64_t* keys, int64_t n, int32_t* idx,
                                 float* val, hipStream_t stream);

}  // namespace dsq
