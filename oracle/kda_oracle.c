/*
 * KDA prefill oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of what the KDA prefill
 * hot path computes.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it; the product library never calls it, and the two share
 * no code.  Floating point is fp64 throughout (inputs are widened exactly), no
 * fast-math.  OpenMP only distributes independent (sequence, head) chains over
 * threads; it changes no arithmetic.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "vllm-ascend 的 KDA 状态复制 Triton 集成：PR 17301 对齐的预编译 worker
 *       生命周期方案", section "数值契约" (numerical contract: gather side,
 *       scatter side, memory and addressing).
 *  [P2] "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对",
 *       section 1.1 (the state update S_t = M_t S_{t-1} + b_t) and section 1.3
 *       (a token segment acts on the state as an affine map).
 *  The explicit transition M_t = (I - beta_t k_t k_t^T) Diag(exp g_t),
 *  b_t = beta_t k_t v_t^T and the read-out o_t = S_t^T q_t are the gated delta
 *  rule as the method defines it; [P3] "PR #33465 完整报告" (SGLang Kimi-K3 on
 *  NPU), section "关键源码片段", shows that q and k are L2-normalised first and
 *  that the read-out is scaled by K^-1/2 (passed in here as `scale`).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* State copy ([P1] "数值契约").                                               */
/*                                                                           */
/* The cache is a 4-D tensor [num_rows, H, V, K] given by a base pointer that */
/* already includes the storage offset and by four element strides.  The     */
/* oracle walks the general strides; it never assumes the row is dense.      */
/* Elements are copied as raw bits (elem_bytes = 4 for fp32, 2 for bf16).    */
/* ------------------------------------------------------------------------- */

static int64_t read_index(const void* indices, int index_is_64, int64_t i) {
  if (index_is_64) return ((const int64_t*)indices)[i];
  return (int64_t)((const int32_t*)indices)[i];
}

/* Gather: packed[i] = cache[idx_i] when 0 <= idx_i < num_rows and the row's
 * flag is true (or there are no flags); every other packed row is all zero
 * bits.  packed is [S, H, V, K] contiguous.  Duplicate indices are allowed. */
int oracle_state_gather(const void* cache, int64_t elem_bytes, int64_t num_rows, int64_t H, int64_t V,
                        int64_t K, const int64_t* strides, const void* indices, int index_is_64,
                        int64_t S, const uint8_t* flags, void* packed) {
  const char* base = (const char*)cache;
  char* dst = (char*)packed;
  for (int64_t i = 0; i < S; ++i) {
    int64_t idx = read_index(indices, index_is_64, i);
    int valid = idx >= 0 && idx < num_rows;
    int take = valid && (flags == NULL || flags[i] != 0);
    for (int64_t h = 0; h < H; ++h)
      for (int64_t v = 0; v < V; ++v)
        for (int64_t k = 0; k < K; ++k) {
          char* d = dst + (((i * H + h) * V + v) * K + k) * elem_bytes;
          if (take) {
            const char* s = base + (idx * strides[0] + h * strides[1] + v * strides[2] + k * strides[3]) * elem_bytes;
            memcpy(d, s, (size_t)elem_bytes);
          } else {
            memset(d, 0, (size_t)elem_bytes);
          }
        }
  }
  return 0;
}

/* Scatter: cache[idx_i] = packed[i] for every valid idx_i; invalid targets
 * are skipped and initial-state flags play no part.  Valid targets must be
 * unique (a caller precondition); the oracle checks it and returns -1 without
 * writing anything when two valid entries name the same row. */
int oracle_state_scatter(void* cache, int64_t elem_bytes, int64_t num_rows, int64_t H, int64_t V, int64_t K,
                         const int64_t* strides, const void* indices, int index_is_64, int64_t S,
                         const void* packed) {
  for (int64_t i = 0; i < S; ++i) {
    int64_t a = read_index(indices, index_is_64, i);
    if (a < 0 || a >= num_rows) continue;
    for (int64_t j = i + 1; j < S; ++j)
      if (read_index(indices, index_is_64, j) == a) return -1;
  }
  char* base = (char*)cache;
  const char* src = (const char*)packed;
  for (int64_t i = 0; i < S; ++i) {
    int64_t idx = read_index(indices, index_is_64, i);
    if (idx < 0 || idx >= num_rows) continue;
    for (int64_t h = 0; h < H; ++h)
      for (int64_t v = 0; v < V; ++v)
        for (int64_t k = 0; k < K; ++k) {
          char* d = base + (idx * strides[0] + h * strides[1] + v * strides[2] + k * strides[3]) * elem_bytes;
          memcpy(d, src + (((i * H + h) * V + v) * K + k) * elem_bytes, (size_t)elem_bytes);
        }
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Gated delta rule, token by token ([P2] 1.1; transition as defined above).   */
/*                                                                           */
/* Layouts (all fp64, contiguous):                                           */
/*   q, k, g : [T, H, K]    v, out : [T, H, V]    beta : [T, H]             */
/*   cu_seqlens : [N+1] token offsets of the varlen batch                    */
/*   initial, final_state : [N, H, V, K]; element (n,h,v,c) is S[c][v] of    */
/*   the K x V state of sequence n, head h.  initial may be NULL (zeros).    */
/* For each token t of a sequence, in order:                                 */
/*   q^ = q_t / sqrt(|q_t|^2 + eps), k^ likewise   (when use_l2norm)         */
/*   S  <- Diag(exp g_t) S                        (decay first)              */
/*   S  <- S - beta_t k^ (k^^T S) + beta_t k^ v_t^T  (erase, then write)     */
/*   o_t = scale * S^T q^                         (read the updated state)   */
/* The two middle lines are S_t = (I - beta k^ k^^T) Diag(exp g) S_{t-1}     */
/* + beta k^ v^T with the product applied to S column by column.            */
/* ------------------------------------------------------------------------- */

static void l2_normalise(const double* x, double* y, int64_t n, int use_l2norm, double eps) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = use_l2norm ? 1.0 / sqrt(ss + eps) : 1.0;
  for (int64_t i = 0; i < n; ++i) y[i] = x[i] * inv;
}

int oracle_kda_recurrence(int64_t N, int64_t H, int64_t K, int64_t V, const int64_t* cu_seqlens,
                          const double* q, const double* k, const double* v, const double* g,
                          const double* beta, const double* initial, double scale, int use_l2norm,
                          double eps, double* out, double* final_state, int num_threads) {
  for (int64_t n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  int64_t chains = N * H;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : 1) if (num_threads != 1)
  for (int64_t ch = 0; ch < chains; ++ch) {
    int64_t n = ch / H, h = ch % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)(K * V));   /* S[c*V + v] */
    double* qh = (double*)malloc(sizeof(double) * (size_t)K);
    double* kh = (double*)malloc(sizeof(double) * (size_t)K);
    double* u = (double*)malloc(sizeof(double) * (size_t)V);
    if (!S || !qh || !kh || !u) {
      failed = 1;
    } else {
      for (int64_t c = 0; c < K; ++c)
        for (int64_t j = 0; j < V; ++j)
          S[c * V + j] = initial ? initial[((n * H + h) * V + j) * K + c] : 0.0;
      for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
        const double* qt = q + (t * H + h) * K;
        const double* kt = k + (t * H + h) * K;
        const double* vt = v + (t * H + h) * V;
        const double* gt = g + (t * H + h) * K;
        double b = beta[t * H + h];
        l2_normalise(qt, qh, K, use_l2norm, eps);
        l2_normalise(kt, kh, K, use_l2norm, eps);
        for (int64_t c = 0; c < K; ++c) {
          double d = exp(gt[c]);
          for (int64_t j = 0; j < V; ++j) S[c * V + j] *= d;
        }
        for (int64_t j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int64_t c = 0; c < K; ++c) acc += S[c * V + j] * kh[c];
          u[j] = acc;
        }
        for (int64_t c = 0; c < K; ++c)
          for (int64_t j = 0; j < V; ++j) S[c * V + j] += b * kh[c] * (vt[j] - u[j]);
        for (int64_t j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int64_t c = 0; c < K; ++c) acc += S[c * V + j] * qh[c];
          out[(t * H + h) * V + j] = scale * acc;
        }
      }
      if (final_state)
        for (int64_t c = 0; c < K; ++c)
          for (int64_t j = 0; j < V; ++j) final_state[((n * H + h) * V + j) * K + c] = S[c * V + j];
    }
    free(S);
    free(qh);
    free(kh);
    free(u);
  }
  return failed ? -2 : 0;
}
