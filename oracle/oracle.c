/*
 * oracle.c -- plain, slow, CPU oracle for the group-quantized matmul and the
 * routed mixture-of-experts FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header,
 * table or constant with the GPU library, and it never reads anything that the
 * GPU library wrote.
 *
 * Build: C99 + OpenMP, -O2 -ffp-contract=off, never -ffast-math (fast-math
 * would turn the fp32 divisions of the quantizer into reciprocal multiplies and
 * change quantized codes).
 *
 * Sources (cited by page title and section):
 *   [P1] "Hand-writing a DeepSeek inference engine in pure C"
 *        (hnwysp.cn/news/134870):
 *        §2.3  group-wise asymmetric quantization, group 64 or 128, dequant
 *              formula (q - zero_point) * scale;
 *        §3.2  the quantize_group routine (per-group min/max,
 *              scale = (max - min) / (2^bits - 1), zp = round(-min / scale),
 *              q = clamp(round(v / scale) + zp)); INT4 = two values per byte,
 *              same rule over 0..15; dequant fused into the matmul inner loop;
 *        §3.3  the matmul C = A * B (reduction over K);
 *        §3.4  softmax with the maximum subtracted first;
 *        §3.5  MoE router = linear layer + softmax + top-k (partial sort of
 *              (score, index) pairs, greater-first), tokens grouped per expert,
 *              weighted sum of the expert outputs;
 *        §5.1/§5.3  a zero scale is an error (assert scale != 0);
 *        §2.1  each block normalises with RMSNorm before its FFN / MoE step
 *              and adds the residual after it.
 *   [P2] "ds4 code walkthrough": the RMSNorm epsilon constant (1e-6).
 *   [P3] "Running a 284B-parameter LLM from 3.2 GB of RAM in plain C"
 *        (feinterview.poetries.top): the scalar and OpenMP CPU paths must be
 *        bitwise identical (fixed accumulator tree, no fp contraction).
 *
 * Where the pages are silent or garbled, the reading taken is stated next to
 * the code that takes it.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_FLAG_DEGENERATE 1u /* scale == 0 / not finite, or |zp| > 2^24 */
#define ORC_FLAG_NONFINITE 2u  /* a NaN or infinity among the group's inputs */

void orc_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t orc_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Canonical quantized format (the oracle's own):                            */
/*   q     : INT8 -> one byte per weight, row-major [rows][K], value 0..255   */
/*           INT4 -> [rows][K/2]; byte j of a row holds k = 2j in its low    */
/*           nibble and k = 2j+1 in its high nibble                          */
/*   scale : fp32 [rows][K/group]                                            */
/*   zp    : fp32 [rows][K/group], an exact integer                          */
/* [P1] §3.2 stores int8(q - 128); the byte used here is that byte XOR 0x80. */
/* ------------------------------------------------------------------------ */

static int32_t orc_get_q(const uint8_t* q, int64_t K, int32_t bits, int64_t r, int64_t k) {
  if (bits == 8) return (int32_t)q[r * K + k];
  uint8_t byte = q[r * (K / 2) + k / 2];
  return (k & 1) ? (int32_t)(byte >> 4) : (int32_t)(byte & 0x0F);
}

/*
 * [P1] §3.2 quantize_group, applied to every group of `group` consecutive
 * elements along K of every row.  All arithmetic is IEEE fp32, as in the
 * printed routine: scale = (max - min) / 255.0f (or / 15.0f for INT4),
 * zp = (int32) roundf(-min / scale), q = clamp((int32) roundf(v / scale) + zp,
 * 0, 2^bits - 1).  roundf rounds half-way cases away from zero.
 *
 * Flagged groups ([P1] §5.1: a zero scale must not be used) get q = 0,
 * scale = 0, zp = 0 and a nonzero gflags entry.  Returns the number of flagged
 * groups, or -1 for invalid arguments.
 */
int64_t orc_quantize(const float* w, int64_t rows, int64_t K, int32_t bits, int32_t group,
                     uint8_t* q, float* scale, float* zp, uint8_t* gflags) {
  if (!w || !q || !scale || !zp || rows < 0 || K <= 0) return -1;
  if (bits != 8 && bits != 4) return -1;
  if (group <= 0 || K % group != 0) return -1;
  if (bits == 4 && (K % 2) != 0) return -1;
  const int32_t qmax = (1 << bits) - 1;
  const float levels = (float)qmax; /* 255.0f or 15.0f */
  const int64_t ngroups = K / group;
  const int64_t row_bytes = (bits == 8) ? K : K / 2;
  int64_t nflag = 0;

#pragma omp parallel for schedule(static) reduction(+ : nflag)
  for (int64_t r = 0; r < rows; ++r) {
    memset(q + r * row_bytes, 0, (size_t)row_bytes);
    for (int64_t g = 0; g < ngroups; ++g) {
      const float* src = w + r * K + g * group;
      uint8_t flag = 0;
      float lo = FLT_MAX, hi = -FLT_MAX;
      for (int32_t i = 0; i < group; ++i) {
        float v = src[i];
        if (!isfinite(v)) flag |= ORC_FLAG_NONFINITE;
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      float s = 0.0f;
      float zr = 0.0f;
      if (!flag) {
        s = (hi - lo) / levels;
        if (!(s > 0.0f) || !isfinite(s)) {
          flag |= ORC_FLAG_DEGENERATE;
        } else {
          zr = roundf(-lo / s);
          /* zp is kept as an fp32 holding an exact integer; beyond 2^24 it
             would not be exact (and beyond 2^31 the int32 cast of the printed
             routine is undefined), so such groups are flagged instead. */
          if (!(fabsf(zr) <= 16777216.0f)) flag |= ORC_FLAG_DEGENERATE;
        }
      }
      const int64_t gi = r * ngroups + g;
      if (gflags) gflags[gi] = flag;
      if (flag) {
        scale[gi] = 0.0f;
        zp[gi] = 0.0f;
        ++nflag;
        continue;
      }
      const int32_t z = (int32_t)zr;
      scale[gi] = s;
      zp[gi] = (float)z;
      for (int32_t i = 0; i < group; ++i) {
        float v = src[i];
        int32_t qi = (int32_t)roundf(v / s) + z;
        if (qi < 0) qi = 0;
        if (qi > qmax) qi = qmax;
        const int64_t k = g * group + i;
        if (bits == 8) {
          q[r * row_bytes + k] = (uint8_t)qi;
        } else {
          uint8_t* b = q + r * row_bytes + k / 2;
          if (k & 1) *b = (uint8_t)((*b & 0x0F) | (qi << 4));
          else       *b = (uint8_t)((*b & 0xF0) | qi);
        }
      }
    }
  }
  return nflag;
}

/* [P1] §2.3: w = (q - zero_point) * scale.  In fp64 this is exact: q - zp is
   an integer below 2^25 in magnitude and scale has a 24-bit significand. */
void orc_dequant_f64(const uint8_t* q, const float* scale, const float* zp, int64_t rows,
                     int64_t K, int32_t bits, int32_t group, double* w) {
  const int64_t ngroups = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t gi = r * ngroups + k / group;
      w[r * K + k] = ((double)orc_get_q(q, K, bits, r, k) - (double)zp[gi]) * (double)scale[gi];
    }
}

/* The same formula in fp32: (float)(q - zp) is exact, so one rounding. */
void orc_dequant_f32(const uint8_t* q, const float* scale, const float* zp, int64_t rows,
                     int64_t K, int32_t bits, int32_t group, float* w) {
  const int64_t ngroups = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t gi = r * ngroups + k / group;
      w[r * K + k] = ((float)orc_get_q(q, K, bits, r, k) - zp[gi]) * scale[gi];
    }
}

/*
 * Plain reference matmul in fp64 ([P1] §3.3 semantics, with the weight stored
 * as W[N][K] so the reduction runs along a row): Y[m][n] = sum_k X[m][k] *
 * W[n][k], summed in k order.  S[m][n] = sum_k |X[m][k] * W[n][k]| is the
 * magnitude sum that scales every floating-point tolerance.  Either output
 * pointer may be NULL.
 */
void orc_matmul_f64(const double* X, int64_t M, const double* W, int64_t N, int64_t K, double* Y,
                    double* S) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double p = X[m * K + k] * W[n * K + k];
        acc += p;
        mag += fabs(p);
      }
      if (Y) Y[m * N + n] = acc;
      if (S) S[m * N + n] = mag;
    }
}

/*
 * The pages' own CPU method in fp32 ([P1] §3.2 "dequantize inside the inner
 * loop while accumulating", §3.3 OpenMP over independent outputs):
 *   Y[m][n] = sum_k X[m][k] * ((q[n][k] - zp) * scale)
 * Each product is added into one of 16 partial sums (k mod 16); the partial
 * sums are then added in a fixed pairwise tree.  Every output's arithmetic is
 * the same whatever the thread count, so the 1-thread and the OpenMP runs are
 * bitwise identical ([P3]).  Rows of X are indexed through `xrows` when it is
 * not NULL (the expert-grouped batch of [P1] §3.5).
 */
static float orc_tree16(float* a) {
  for (int w = 8; w >= 1; w >>= 1)
    for (int i = 0; i < w; ++i) a[i] = a[i] + a[i + w];
  return a[0];
}

static void orc_qdot_rows_f32(const float* X, const int64_t* xrows, int64_t M, const uint8_t* q,
                              const float* scale, const float* zp, int64_t n, int64_t K,
                              int32_t bits, int32_t group, float* out, int64_t out_stride) {
  const int64_t ngroups = K / group;
  for (int64_t m = 0; m < M; ++m) {
    const float* x = X + (xrows ? xrows[m] : m) * K;
    float part[16];
    for (int i = 0; i < 16; ++i) part[i] = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t gi = n * ngroups + k / group;
      const float wq = ((float)orc_get_q(q, K, bits, n, k) - zp[gi]) * scale[gi];
      const float p = x[k] * wq;
      part[k & 15] = part[k & 15] + p;
    }
    out[m * out_stride] = orc_tree16(part);
  }
}

void orc_qmatmul_f32(const float* X, int64_t M, const uint8_t* q, const float* scale,
                     const float* zp, int64_t N, int64_t K, int32_t bits, int32_t group,
                     float* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    orc_qdot_rows_f32(X, NULL, M, q, scale, zp, n, K, bits, group, Y + n, N);
}

/* ------------------------------------------------------------------------ */
/* Router and routing ([P1] §3.4, §3.5)                                      */
/* ------------------------------------------------------------------------ */

/* Router = linear layer ([P1] §3.5): l[t][e] = sum_h X[t][h] * Wr[e][h]
   (+ bias[e] when bias is not NULL), in fp64.  S = magnitude sums. */
void orc_router_f64(const double* X, int64_t T, const double* Wr, const double* bias, int32_t E,
                    int64_t H, double* logits, double* S) {
  orc_matmul_f64(X, T, Wr, E, H, logits, S);
  if (bias)
    for (int64_t t = 0; t < T; ++t)
      for (int32_t e = 0; e < E; ++e) logits[t * E + e] += bias[e];
}

/* "a ranks before b": larger logit first; equal logits -> larger index first,
   which is what a greater-than partial sort over (score, index) pairs gives
   ([P1] §3.5; the comparison characters were lost in extraction). */
static int orc_before(double la, int32_t ia, double lb, int32_t ib) {
  if (la != lb) return la > lb;
  return ia > ib;
}

/*
 * Softmax + top-k + renormalisation for each token.
 *   p_e = exp(l_e - max) / sum_j exp(l_j - max)      ([P1] §3.4: subtract max)
 *   idx = the k experts ranked first by orc_before, in that order ([P1] §3.5)
 *   w_i = p_{idx_i} / sum_j p_{idx_j}                 (weights sum to one)
 * Selection uses the logits themselves, as the printed route() does, so two
 * distinct logits are never merged by rounding in exp.  gap[t] (nullable) is
 * the logit distance between the k-th and the (k+1)-th ranked experts
 * (+inf when k == E); tests use it to tell near-ties apart.
 * Logits must be finite; returns -1 otherwise or for invalid arguments.
 */
int32_t orc_route(const double* logits, int64_t T, int32_t E, int32_t k, int32_t* idx, double* w,
                  double* gap) {
  if (E <= 0 || k <= 0 || k > E) return -1;
  for (int64_t i = 0; i < T * E; ++i)
    if (!isfinite(logits[i])) return -1;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  if (!taken || !p) {
    free(taken);
    free(p);
    return -1;
  }
  for (int64_t t = 0; t < T; ++t) {
    const double* l = logits + t * E;
    double mx = l[0];
    for (int32_t e = 1; e < E; ++e)
      if (l[e] > mx) mx = l[e];
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      p[e] = exp(l[e] - mx);
      z += p[e];
    }
    for (int32_t e = 0; e < E; ++e) p[e] /= z;
    memset(taken, 0, (size_t)E);
    double sel = 0.0;
    for (int32_t i = 0; i < k; ++i) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || orc_before(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      idx[t * k + i] = best;
      sel += p[best];
    }
    for (int32_t i = 0; i < k; ++i) w[t * k + i] = p[idx[t * k + i]] / sel;
    if (gap) {
      if (k == E) {
        gap[t] = INFINITY;
      } else {
        int32_t next = -1;
        for (int32_t e = 0; e < E; ++e) {
          if (taken[e]) continue;
          if (next < 0 || orc_before(l[e], e, l[next], next)) next = e;
        }
        gap[t] = l[idx[t * k + k - 1]] - l[next];
      }
    }
  }
  free(taken);
  free(p);
  return 0;
}

/*
 * Group the T*k routing entries by expert ([P1] §3.5: gather the tokens routed
 * to one expert so its weights are read once).  A stable counting sort:
 *   counts[e]  = number of entries j = t*k+i with idx[j] == e
 *   offsets[e] = sum of counts below e (offsets[E] = T*k)
 *   perm       = every entry j, ordered by (expert, j)
 */
int32_t orc_group(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t* counts,
                  int32_t* offsets, int32_t* perm) {
  const int64_t n = T * k;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t j = 0; j < n; ++j) {
    if (idx[j] < 0 || idx[j] >= E) return -1;
    counts[idx[j]]++;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!fill) return -1;
  for (int32_t e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t j = 0; j < n; ++j) perm[fill[idx[j]]++] = (int32_t)j;
  free(fill);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* One expert: SwiGLU FFN over group-quantized weights                       */
/* ------------------------------------------------------------------------ */

static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* d/dz silu(z) = s(z) * (1 + z * (1 - s(z))), s = logistic */
static double orc_dsilu(double z) {
  const double s = 1.0 / (1.0 + exp(-z));
  return s * (1.0 + z * (1.0 - s));
}

/* The two functions above, exported so that tests can pin them to closed
   forms (silu(0) = 0, silu(ln 3) = 3/4 ln 3, silu'(0) = 1/2, ...). */
double orc_silu_f64(double z) { return orc_silu(z); }
double orc_dsilu_f64(double z) { return orc_dsilu(z); }

typedef struct {
  const uint8_t* q;
  const float* scale;
  const float* zp;
} orc_qmat;

/* dot of x (fp64, length K) with the exact fp64 dequantized row n */
static void orc_qrow_dot_f64(const double* x, orc_qmat W, int64_t n, int64_t K, int32_t bits,
                             int32_t group, double* dot, double* mag) {
  const int64_t ngroups = K / group;
  double acc = 0.0, s = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const int64_t gi = n * ngroups + k / group;
    const double wv =
        ((double)orc_get_q(W.q, K, bits, n, k) - (double)W.zp[gi]) * (double)W.scale[gi];
    const double p = x[k] * wv;
    acc += p;
    s += fabs(p);
  }
  *dot = acc;
  *mag = s;
}

/*
 * One expert in fp64:  g = x Wg^T, u = x Wu^T (I outputs, K = H),
 * h = silu(g) * u, y = h Wd^T (H outputs, K = I); silu(z) = z / (1 + e^-z).
 * Expert FFN form: SwiGLU, as the workload defines (the pages only call the
 * experts feed-forward networks).
 * Tolerance helpers (all nullable):
 *   Sd[n]  = sum_j |h_j * Wd[n][j]|
 *   Pd[n]  = sum_j dh_j * |Wd[n][j]| with
 *            dh_j = |silu'(g_j) u_j| * Sg_j + |silu(g_j)| * Su_j,
 *            Sg_j, Su_j the magnitude sums of g_j and u_j: the first-order
 *            effect on y of a relative error of 1 in the gate/up sums.
 *   g, u, h (length I) are returned when their pointers are not NULL.
 */
void orc_expert_f64(const double* x, int64_t H, int64_t I, const uint8_t* gq, const float* gs,
                    const float* gz, const uint8_t* uq, const float* us, const float* uz,
                    const uint8_t* dq, const float* ds, const float* dz, int32_t bits,
                    int32_t group, double* y, double* Sd, double* Pd, double* g_out,
                    double* u_out, double* h_out) {
  orc_qmat Wg = {gq, gs, gz}, Wu = {uq, us, uz}, Wd = {dq, ds, dz};
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  double* dh = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < I; ++j) {
    double g, sg, u, su;
    orc_qrow_dot_f64(x, Wg, j, H, bits, group, &g, &sg);
    orc_qrow_dot_f64(x, Wu, j, H, bits, group, &u, &su);
    h[j] = orc_silu(g) * u;
    dh[j] = fabs(orc_dsilu(g) * u) * sg + fabs(orc_silu(g)) * su;
    if (g_out) g_out[j] = g;
    if (u_out) u_out[j] = u;
    if (h_out) h_out[j] = h[j];
  }
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < H; ++n) {
    double acc, mag;
    orc_qrow_dot_f64(h, Wd, n, I, bits, group, &acc, &mag);
    y[n] = acc;
    if (Sd) Sd[n] = mag;
    if (Pd) {
      const int64_t ngroups = I / group;
      double pm = 0.0;
      for (int64_t j = 0; j < I; ++j) {
        const int64_t gi = n * ngroups + j / group;
        const double wv =
            ((double)orc_get_q(Wd.q, I, bits, n, j) - (double)Wd.zp[gi]) * (double)Wd.scale[gi];
        pm += dh[j] * fabs(wv);
      }
      Pd[n] = pm;
    }
  }
  free(h);
  free(dh);
}

/* ------------------------------------------------------------------------ */
/* The pages' CPU MoE in fp32 (timed as the CPU baseline)                    */
/* ------------------------------------------------------------------------ */

/*
 * Token-routed MoE FFN, fp32, fused dequant (the same dot routine as
 * orc_qmatmul_f32).  Experts are passed as pointer arrays indexed by expert id
 * (entries of experts nobody selected may be NULL).  Routing (idx, w) is an
 * input.  Y[t] = sum_i w[t][i] * y_{idx[t][i]}(X[t]), summed in slot order.
 *
 * grouped = 0: loop over tokens, then over the token's k experts.
 * grouped = 1: group the entries by expert first ([P1] §3.5) and run each
 *              expert once over its batch of tokens.  Both orders perform the
 *              identical per-output arithmetic, so the outputs are bitwise
 *              equal (a test checks this).
 * h_ws must hold T*k*I floats, y_ws T*k*H floats.
 */
int32_t orc_moe_f32(const float* X, int64_t T, int64_t H, int64_t I, int32_t E, int32_t k,
                    const int32_t* idx, const float* w, const uint8_t* const* gq,
                    const float* const* gs, const float* const* gz, const uint8_t* const* uq,
                    const float* const* us, const float* const* uz, const uint8_t* const* dq,
                    const float* const* ds, const float* const* dz, int32_t bits, int32_t group,
                    int32_t grouped, float* h_ws, float* y_ws, float* Y) {
  const int64_t n = T * k;
  int64_t* xrows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  int64_t* hrows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!xrows || !hrows || !counts || !offsets || !perm) return -1;
  if (orc_group(idx, T, k, E, counts, offsets, perm) != 0) return -1;

  /* Build the batches: one per (token, slot) when token-looped, one per
     expert when grouped.  h_ws / y_ws rows are indexed by entry j = t*k+i. */
  const int64_t nb = grouped ? E : n;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t cnt, e;
    const int32_t* js;
    int32_t one;
    if (grouped) {
      e = b;
      cnt = counts[e];
      js = perm + offsets[e];
    } else {
      one = (int32_t)b;
      js = &one;
      cnt = 1;
      e = idx[b];
    }
    if (cnt == 0) continue;
    for (int64_t m = 0; m < cnt; ++m) {
      xrows[m] = js[m] / k;
      hrows[m] = js[m];
    }
    /* gate and up: outputs j' in [0, I) for every token of the batch */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < I; ++r) {
      for (int64_t m = 0; m < cnt; ++m) {
        float gv, uv;
        orc_qdot_rows_f32(X, xrows + m, 1, gq[e], gs[e], gz[e], r, H, bits, group, &gv, 1);
        orc_qdot_rows_f32(X, xrows + m, 1, uq[e], us[e], uz[e], r, H, bits, group, &uv, 1);
        const float sg = gv / (1.0f + expf(-gv));
        h_ws[hrows[m] * I + r] = sg * uv;
      }
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < H; ++r) {
      for (int64_t m = 0; m < cnt; ++m) {
        float yv;
        orc_qdot_rows_f32(h_ws, hrows + m, 1, dq[e], ds[e], dz[e], r, I, bits, group, &yv, 1);
        y_ws[hrows[m] * H + r] = yv;
      }
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < H; ++c) {
      float acc = 0.0f;
      for (int32_t i = 0; i < k; ++i) acc = acc + w[t * k + i] * y_ws[(t * k + i) * H + c];
      Y[t * H + c] = acc;
    }
  free(xrows);
  free(hrows);
  free(counts);
  free(offsets);
  free(perm);
  return 0;
}

/*
 * Output-head selection: the last projection's logits choose the next token
 * ([P1] §2.1, the pipeline ends in the output projection, logits and
 * sampling; [P2] the session API's argmax / sample step; [P3] the end-to-end
 * check compares the argmax at every position).  Returns the k largest of
 * y[0..N) in rank order:
 *   larger value first; equal values (-0 equals +0) -> smaller index first,
 *   the first maximum a plain "if (y[i] > best)" scan keeps; NaN ranks below
 *   every number (and among NaNs the smaller index first).
 * Plain k-pass selection, O(k N).  Returns -1 for invalid arguments.
 */
static int orc_head_before(float a, int64_t ia, float b, int64_t ib) {
  const int an = a != a, bn = b != b;
  if (an || bn) {
    if (an && bn) return ia < ib;
    return bn;  /* a number ranks before a NaN */
  }
  if (a != b) return a > b;
  return ia < ib;
}

int32_t orc_topk_f32(const float* y, int64_t N, int32_t k, int32_t* idx, float* val) {
  if (!y || !idx || !val || N < 1 || k < 1 || k > N) return -1;
  unsigned char* taken = (unsigned char*)calloc((size_t)N, 1);
  if (!taken) return -1;
  for (int32_t r = 0; r < k; ++r) {
    int64_t best = -1;
    for (int64_t i = 0; i < N; ++i) {
      if (taken[i]) continue;
      if (best < 0 || orc_head_before(y[i], i, y[best], best)) best = i;
    }
    taken[best] = 1;
    idx[r] = (int32_t)best;
    val[r] = y[best];
  }
  free(taken);
  return 0;
}

/*
 * RMSNorm of each row, the normalisation a block applies before its FFN
 * ("Hand-writing a DeepSeek inference engine in pure C", §2.1: every block
 * normalises with RMSNorm before the feed-forward / MoE step and adds the
 * residual after it; "ds4 code walkthrough", the model constants: epsilon
 * 1e-6).  The formula is the standard one, which the pages name but do not
 * print: out[t][h] = x[t][h] / sqrt(mean_h x[t][h]^2 + eps) * g[h], all in
 * double.  Returns -1 for invalid arguments.
 */
int32_t orc_rmsnorm_f64(const float* x, const float* g, int64_t T, int64_t H, double eps,
                        double* out) {
  if (!x || !g || !out || T < 0 || H < 1 || !(eps >= 0.0)) return -1;
  for (int64_t t = 0; t < T; ++t) {
    const float* row = x + t * H;
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h) ss += (double)row[h] * (double)row[h];
    const double rms = sqrt(ss / (double)H + eps);
    for (int64_t h = 0; h < H; ++h) out[t * H + h] = (double)row[h] / rms * (double)g[h];
  }
  return 0;
}

/*
 * Two-level "super-block" 4-bit format.  "ds4 code walkthrough", trace 4
 * (quant block struct sizes) prints the block: an fp16 d, an fp16 dmin, 12
 * bytes of scales and 128 bytes of nibbles for 256 weights, 144 bytes in all.
 * The pages fix only those fields and sizes; the arithmetic is this reading
 * of them:
 *   - a block covers 256 consecutive weights of a row (along K) in 8
 *     sub-blocks of 32;
 *   - sub-block j has a 6-bit scale sc_j and a 6-bit min m_j; the 12 bytes
 *     hold sc_0..sc_7 then m_0..m_7 as consecutive 6-bit fields of one
 *     little-endian 96-bit integer (field i at bits 6i .. 6i+5);
 *   - weight 2i is the low nibble of byte i of the 128, weight 2i+1 the high
 *     nibble (the same byte order as the 4-bit codes of the group format);
 *   - weight w of sub-block j dequantizes to d*sc_j*q - dmin*m_j.
 * Quantizer (the pages print none; this follows the group rule of [P1] §3.2
 * level by level, in fp32 with roundf):
 *   off_j = max(0, -min_j), step s_j = (max_j + off_j) / 15  (the 16 levels
 *   -off_j .. 15 s_j - off_j cover the sub-block, 0 included);
 *   d = fp16(max_j s_j / 63), dmin = fp16(max_j off_j / 63), rounded to
 *   nearest even;
 *   sc_j = clamp(round(s_j / d), 0, 63), m_j = clamp(round(off_j / dmin), 0, 63)
 *   (0 when the divisor is 0);
 *   q = clamp(round((w + dmin*m_j) / (d*sc_j)), 0, 15) (0 when d*sc_j is 0).
 * A block holding a NaN or an infinity, or whose d or dmin overflows fp16, is
 * stored as all zeros and flagged (NONFINITE / DEGENERATE).
 */
#define ORC_SB_K 256
#define ORC_SB_BYTES 144

/* fp32 -> IEEE binary16 bits, round to nearest, ties to even; subnormal
   results kept, overflow to infinity, NaN to a quiet NaN. */
uint16_t orc_f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, sizeof x);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u));
  if (ax < 0x00800000u) return (uint16_t)sign; /* fp32 subnormal: far below 2^-25 */
  const int e = (int)(ax >> 23) - 127;
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  const uint32_t mant = (ax & 0x7fffffu) | 0x800000u; /* 24-bit significand */
  const int shift = e >= -14 ? 13 : 13 + (-14 - e);   /* bits dropped */
  if (shift > 24) return (uint16_t)sign;
  uint32_t q = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  /* normal: q holds the implicit bit (0x400 .. 0x800, a carry moves the
     exponent up); subnormal: q is the fraction itself */
  const uint32_t h = e >= -14 ? ((uint32_t)(e + 14) << 10) + q : q;
  return (uint16_t)(sign | (h >= 0x7c00u ? 0x7c00u : h));
}

/* binary16 bits -> its exact value */
double orc_f16_to_f64(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);
  return (h & 0x8000u) ? -v : v;
}

static uint32_t orc_sb_field(const uint8_t* s12, int i) {
  uint32_t v = 0;
  for (int b = 0; b < 6; ++b) {
    const int bit = 6 * i + b;
    v |= (uint32_t)((s12[bit >> 3] >> (bit & 7)) & 1u) << b;
  }
  return v;
}

static void orc_sb_set_field(uint8_t* s12, int i, uint32_t v) {
  for (int b = 0; b < 6; ++b) {
    const int bit = 6 * i + b;
    if ((v >> b) & 1u) s12[bit >> 3] |= (uint8_t)(1u << (bit & 7));
  }
}

/* Quantizes w[rows][K] (K % 256 == 0) into blocks[rows][K/256][144]; flags
   gets one byte per block.  Returns the number of flagged blocks, -1 for
   invalid arguments. */
int64_t orc_sb4_quantize(const float* w, int64_t rows, int64_t K, uint8_t* blocks,
                         uint8_t* bflags) {
  if (!w || !blocks || rows < 0 || K <= 0 || K % ORC_SB_K != 0) return -1;
  const int64_t nb = K / ORC_SB_K;
  int64_t nflag = 0;
#pragma omp parallel for schedule(static) reduction(+ : nflag)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* src = w + r * K + b * ORC_SB_K;
      uint8_t* out = blocks + (r * nb + b) * ORC_SB_BYTES;
      memset(out, 0, ORC_SB_BYTES);
      uint8_t flag = 0;
      float step[8], off[8];
      float smax = 0.0f, omax = 0.0f;
      for (int j = 0; j < 8; ++j) {
        float lo = FLT_MAX, hi = -FLT_MAX;
        for (int i = 0; i < 32; ++i) {
          const float v = src[32 * j + i];
          if (!isfinite(v)) flag |= ORC_FLAG_NONFINITE;
          if (v < lo) lo = v;
          if (v > hi) hi = v;
        }
        off[j] = lo < 0.0f ? -lo : 0.0f;
        step[j] = (hi + off[j]) / 15.0f;
        if (step[j] > smax) smax = step[j];
        if (off[j] > omax) omax = off[j];
      }
      uint16_t d16 = 0, m16 = 0;
      if (!flag) {
        d16 = orc_f32_to_f16(smax / 63.0f);
        m16 = orc_f32_to_f16(omax / 63.0f);
        if ((d16 & 0x7c00u) == 0x7c00u || (m16 & 0x7c00u) == 0x7c00u) flag |= ORC_FLAG_DEGENERATE;
      }
      if (bflags) bflags[r * nb + b] = flag;
      if (flag) {
        ++nflag;
        continue; /* the block stays all zeros */
      }
      const float df = (float)orc_f16_to_f64(d16), mf = (float)orc_f16_to_f64(m16);
      out[0] = (uint8_t)(d16 & 0xff);
      out[1] = (uint8_t)(d16 >> 8);
      out[2] = (uint8_t)(m16 & 0xff);
      out[3] = (uint8_t)(m16 >> 8);
      for (int j = 0; j < 8; ++j) {
        float sc = df > 0.0f ? roundf(step[j] / df) : 0.0f;
        float mn = mf > 0.0f ? roundf(off[j] / mf) : 0.0f;
        sc = sc < 0.0f ? 0.0f : (sc > 63.0f ? 63.0f : sc);
        mn = mn < 0.0f ? 0.0f : (mn > 63.0f ? 63.0f : mn);
        orc_sb_set_field(out + 4, j, (uint32_t)sc);
        orc_sb_set_field(out + 4, 8 + j, (uint32_t)mn);
        const float S = df * sc, M = mf * mn;
        for (int i = 0; i < 32; ++i) {
          const int k = 32 * j + i;
          float q = S > 0.0f ? roundf((src[k] + M) / S) : 0.0f;
          q = q < 0.0f ? 0.0f : (q > 15.0f ? 15.0f : q);
          out[16 + k / 2] |= (uint8_t)((uint32_t)q << ((k & 1) * 4));
        }
      }
    }
  }
  return nflag;
}

/* Dequantizes blocks[rows][K/256][144] into out[rows][K] (double, exact). */
int32_t orc_sb4_dequant_f64(const uint8_t* blocks, int64_t rows, int64_t K, double* out) {
  if (!blocks || !out || rows < 0 || K <= 0 || K % ORC_SB_K != 0) return -1;
  const int64_t nb = K / ORC_SB_K;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = blocks + (r * nb + b) * ORC_SB_BYTES;
      const double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
      const double dmin = orc_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
      for (int k = 0; k < ORC_SB_K; ++k) {
        const int j = k / 32;
        const double q = (double)((blk[16 + k / 2] >> ((k & 1) * 4)) & 15u);
        out[r * K + b * ORC_SB_K + k] =
            d * (double)orc_sb_field(blk + 4, j) * q - dmin * (double)orc_sb_field(blk + 4, 8 + j);
      }
    }
  return 0;
}
