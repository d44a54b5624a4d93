/*
 * kda.h -- C ABI of the KDA (Kimi Delta Attention) prefill hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The prefill step has three stages:
 *   1. kda_state_gather   -- copy each request's initial recurrent state out
 *                            of indexed rows of a state cache;
 *   2. kda_chunk_prefill  -- run the chunkwise gated delta rule (chunk size
 *                            64) over a varlen batch delimited by cu_seqlens;
 *   3. kda_state_scatter  -- copy the final states back into cache rows.
 * Decode has one: kda_recurrent_decode advances each sequence by one token
 * with its state updated in place in its cache row.  Checkpoints can be
 * parked compressed: kda_ckpt_quantize_scatter / kda_ckpt_dequantize_gather
 * move states between packed buffers and an INT8 checkpoint store.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "vllm-ascend 的 KDA 状态复制 Triton 集成：PR 17301 对齐的预编译 worker
 *       生命周期方案": section "背景" (gather -> chunk math -> scatter around
 *       an unchanged chunk kernel with chunk size 64), section "数值契约"
 *       (the copy contract), section "自动分发" (the layout admissibility
 *       rule), section "启动准备" (index dtype kept as given).
 *  [P2] "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对",
 *       section 1.1 (S_t = M_t S_{t-1} + b_t) and the varlen row of the
 *       table in section 0x00 (cu_seqlens, every sequence advances its own
 *       state).
 *  [P3] "PR #33465 完整报告" (SGLang Kimi-K3 on NPU), section "关键源码片段":
 *       the prefill decomposition l2norm -> chunk-local cumulative gate sum
 *       (scaled by log2 e) -> gated K K^T -> triangular solve -> W/U
 *       recompute -> inter-chunk state recurrence -> chunk output, with scale
 *       K^-1/2 and the output allowed to reuse v's buffer.
 *
 * Conventions shared by every entry point:
 *  - Ownership: the library owns no memory (except the static scratch of
 *    kda_chunk_prefill_noalloc).  The caller allocates every buffer (device
 *    memory unless stated) and passes the HIP stream on each call; no buffer
 *    or per-call state is retained between calls (the library looks up each
 *    device's CU count, and the scratch's address, once).
 *  - stream: a hipStream_t passed as void* (NULL = the default stream).  All
 *    work is enqueued on it; no entry point synchronises the device or reads
 *    device memory on the host.
 *  - Validation is host-only and fail-closed: a bad argument returns an error
 *    status and enqueues nothing.
 *  - Errors from the HIP runtime return KDA_E_HIP; kda_last_error_detail()
 *    then names the failing call (thread-local, valid until the next call on
 *    the same thread).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;
typedef enum { KDA_I32 = 0, KDA_I64 = 1 } kda_index_t;

typedef enum {
  KDA_OK = 0,
  KDA_E_NULL = 1,        /* a required pointer is NULL                                   */
  KDA_E_DTYPE = 2,       /* dtype / index type outside the supported set                 */
  KDA_E_SHAPE = 3,       /* negative or zero size where a positive one is required       */
  KDA_E_LAYOUT = 4,      /* cache inner dims [H,V,K] are not dense                       */
  KDA_E_OVERLAP = 5,     /* cache row stride smaller than the row payload (pages overlap) */
  KDA_E_UNSUPPORTED = 6, /* a size the library has no kernel for (e.g. K > 128)          */
  KDA_E_WORKSPACE = 7,   /* workspace missing or smaller than kda_chunk_prefill_workspace_size */
  KDA_E_ALIAS = 8,       /* an output overlaps an input or another output               */
  KDA_E_HIP = 9          /* the HIP runtime reported an error                           */
} kda_status_t;

/*
 * A view of one layer's recurrent-state cache: a 4-D tensor [num_rows, H, V, K].
 * Element (r, h, v, c) is S_h[c][v] of cache row r, where S_h is the K x V
 * state of head h (state rows are laid out [H][V][K], K fastest; [P1] section
 * "自动分发" gives the [N,H,V,K] shape).
 *  data      -- address of element (0,0,0,0): the storage offset is already
 *               applied (a tensor's data_ptr()).
 *  dtype     -- KDA_F32 or KDA_BF16.
 *  stride[4] -- element strides of the four dims.
 * Admissible layouts ([P1] section "自动分发"): num_rows > 0, H, V, K > 0;
 * reading the inner dims from the back, each has size 1 or a stride equal to
 * the running payload (stride[3] = 1, stride[2] = K, stride[1] = V*K); and
 * stride[0] >= H*V*K, so rows never overlap.  The gap between a row's payload
 * and the next row is never read or written, nor is anything before data.
 */
typedef struct {
  void* data;
  kda_dtype_t dtype;
  int64_t num_rows, H, V, K;
  int64_t stride[4];
} kda_state_cache_t;

/*
 * kda_state_gather -- [P1] section "数值契约", gather side.
 * For i in [0, num_selected):
 *   packed[i] = cache row indices[i]   if 0 <= indices[i] < num_rows and
 *                                       (flags == NULL or flags[i] != 0),
 *   packed[i] = all-zero bits           otherwise.
 *  indices     -- device array of num_selected int32 (KDA_I32) or int64
 *                 (KDA_I64) values, read in their own width (no conversion).
 *                 Duplicates are allowed.
 *  flags       -- device array of num_selected bytes, or NULL (all true).
 *  packed      -- device output [num_selected, H, V, K], contiguous, in the
 *                 cache dtype; every row is written.
 * Bits are copied unchanged.  num_selected == 0 validates the cache view and
 * enqueues nothing.  Preconditions (not checked): packed does not overlap the
 * cache.  Errors: KDA_E_NULL, KDA_E_DTYPE, KDA_E_SHAPE, KDA_E_LAYOUT,
 * KDA_E_OVERLAP, KDA_E_HIP.
 */
kda_status_t kda_state_gather(const kda_state_cache_t* cache, const void* indices, kda_index_t index_type,
                              int64_t num_selected, const uint8_t* flags, void* packed, void* stream);

/*
 * kda_state_scatter -- [P1] section "数值契约", scatter side.
 * For i in [0, num_selected): if 0 <= indices[i] < num_rows, cache row
 * indices[i] = packed[i]; other entries are skipped.  Initial-state flags
 * play no part: a valid target is always written.
 *  packed      -- device input [num_selected, H, V, K], contiguous, cache
 *                 dtype (convert final states to the cache dtype first).
 * Preconditions (not checked, no device-to-host scan): valid targets are
 * unique; packed does not overlap the cache.  num_selected == 0 enqueues
 * nothing.  Errors as for kda_state_gather.
 */
kda_status_t kda_state_scatter(const kda_state_cache_t* cache, const void* indices, kda_index_t index_type,
                               int64_t num_selected, const void* packed, void* stream);

/*
 * Arguments of kda_chunk_prefill.  All pointers are device pointers to
 * contiguous row-major arrays.
 *  T, N, H, K, V   -- tokens, sequences, heads, key dim (1..128), value dim (>= 1);
 *                     H * max(K, V) <= 2^22 (else KDA_E_UNSUPPORTED).
 *  q, k            -- [T, H, K] in qkv_dtype.           v -- [T, H, V] in qkv_dtype.
 *  g               -- [T, H, K] fp32: natural-log decay per key channel; the
 *                     state is multiplied by exp(g) (g <= 0 for a decay).
 *  beta            -- [T, H] in beta_dtype (fp32 or bf16).
 *  cu_seqlens      -- [N+1] int32 token offsets; sequence n is tokens
 *                     [cu_seqlens[n], cu_seqlens[n+1]).  Precondition (not
 *                     checked on the host): cu_seqlens[0] = 0, non-decreasing,
 *                     cu_seqlens[N] = T; the kernels clamp so that bad
 *                     offsets cannot address outside [0, T).
 *  initial_state   -- [N, H, V, K] in initial_dtype, element (n,h,v,c) =
 *                     S[c][v]; or NULL for zero initial states.
 *  out             -- [T, H, V] in qkv_dtype.  It may be exactly v (the
 *                     output then overwrites v, [P3]).
 *  final_state     -- [N, H, V, K] in final_dtype, or NULL.  fp32 states are
 *                     rounded to bf16 to nearest even when final_dtype is bf16.
 *                     It may be exactly initial_state with the same dtype
 *                     (the states are then updated in place).
 *  scale           -- read-out scale ([P3] uses K^-1/2).
 *  use_qk_l2norm   -- nonzero: q and k rows are divided by sqrt(|x|^2 + 1e-6).
 *  workspace       -- device scratch of at least
 *                     kda_chunk_prefill_workspace_size(T, N, H, K, V) bytes
 *                     (may be NULL when that size is 0).
 * Aliasing (checked on the host, KDA_E_ALIAS): the outputs -- out,
 * final_state, ckpt_states and the workspace's first
 * kda_chunk_prefill_workspace_size bytes -- overlap neither each other nor
 * any input (q, k, v, g, beta, cu_seqlens, initial_state, ckpt_cu), except
 * for the two exact aliases above.
 * Per sequence n and head h, with S the K x V fp32 state, this computes for
 * each token t in order ([P2] section 1.1 and the gated delta rule):
 *   S <- (I - beta_t k_t k_t^T) Diag(exp g_t) S + beta_t k_t v_t^T
 *   out_t = scale * S^T q_t
 * evaluated chunkwise in chunks of 64 tokens aligned to each sequence start
 * ([P3]).  Sequences of length 0 pass their initial state through.
 * Precision: the state, the gate sums, the row norms, the triangular
 * inverse's diagonal blocks and every accumulation are fp32; the operands of
 * the matrix products (the gated q/k tiles, the inverse, W, U, V_new and the
 * state as a right-hand operand) are rounded to bf16 -- for fp32 q/k/v too.
 * Against an fp64 evaluation of the recurrence this gives a relative L2
 * error of about 4e-3 on outputs and final states for bf16 and fp32 inputs
 * alike (tolerance 2e-2).
 */
typedef struct {
  int64_t T, N, H, K, V;
  const void* q;
  const void* k;
  const void* v;
  kda_dtype_t qkv_dtype;
  const float* g;
  const void* beta;
  kda_dtype_t beta_dtype;
  const int32_t* cu_seqlens;
  const void* initial_state;
  kda_dtype_t initial_dtype;
  void* out;
  void* final_state;
  kda_dtype_t final_dtype;
  float scale;
  int use_qk_l2norm;
  void* workspace;
  size_t workspace_bytes;
  /* Optional chunk-boundary checkpoints (prefix states that a cache can keep
   * and later resume from; [P2] section 1.3 and section 5.2's checkpoints at
   * chunk boundaries).  With ckpt_states != NULL, for sequence n the j-th
   * checkpoint (j = 0 .. ckpt_cu[n+1]-ckpt_cu[n]-1) is the state after
   * (j+1)*ckpt_interval tokens of that sequence, written to row ckpt_cu[n]+j
   * of ckpt_states ([num_ckpt, H, V, K], ckpt_dtype, same element order as
   * final_state, rounded like final_state).  Positions past the sequence's
   * length and rows outside [0, num_ckpt) are not written; the natural
   * choice is ckpt_cu[n+1]-ckpt_cu[n] = floor(len_n / ckpt_interval).
   * Chunks never straddle a multiple of 64 tokens of a sequence, so the
   * checkpoint states are exact chunk-boundary states, and requesting them
   * does not change out or final_state.
   *  ckpt_interval -- positive multiple of 64 (ignored when ckpt_states is NULL).
   *  ckpt_cu       -- [N+1] int32 device array of checkpoint row offsets,
   *                   non-decreasing (not checked).
   *  ckpt_states   -- device output, num_ckpt rows, or NULL for none.  It must
   *                   not overlap any other argument (checked, KDA_E_ALIAS). */
  int64_t ckpt_interval;
  const int32_t* ckpt_cu;
  void* ckpt_states;
  int64_t num_ckpt;
  kda_dtype_t ckpt_dtype;
} kda_prefill_args_t;

/* Bytes of device workspace kda_chunk_prefill needs for these sizes. */
size_t kda_chunk_prefill_workspace_size(int64_t T, int64_t N, int64_t H, int64_t K, int64_t V);

/*
 * kda_chunk_prefill -- the chunkwise gated delta rule of [P3] over a varlen
 * batch; see kda_prefill_args_t for arguments and semantics.
 * N == 0 enqueues nothing.  Errors: KDA_E_NULL, KDA_E_DTYPE, KDA_E_SHAPE,
 * KDA_E_UNSUPPORTED, KDA_E_WORKSPACE, KDA_E_ALIAS, KDA_E_HIP.
 */
kda_status_t kda_chunk_prefill(const kda_prefill_args_t* args, void* stream);

/*
 * Bytes of device scratch that kda_chunk_prefill_noalloc keeps on each device
 * it runs on: 256 MiB, more than kda_chunk_prefill_workspace_size returns for
 * any sizes kda_chunk_prefill accepts.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * kda_chunk_prefill_noalloc -- kda_chunk_prefill for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics, validation and
 * kernels as kda_chunk_prefill, except that args->workspace and
 * args->workspace_bytes are ignored: the workspace is a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES inside the library, one copy per device, created
 * when the library's code is loaded on that device and held until the process
 * ends.  The call allocates and frees nothing (no hipMalloc, no hipFree, no
 * allocating library routine) and enqueues no memset.  The first call on a
 * device looks up that device's copy (hipGetSymbolAddress) with the device
 * current.
 * Calls on one device share that device's array: two calls that can overlap
 * in time on one device (different streams, or different host threads with
 * no ordering between them) race on it and give undefined results; order
 * them on one stream or with events.  Calls on different devices do not
 * interact.  Nothing is carried from one call to the next.
 * Errors: as kda_chunk_prefill, with KDA_E_WORKSPACE when
 * kda_chunk_prefill_workspace_size(T, N, H, K, V) exceeds
 * KDA_NOALLOC_SCRATCH_BYTES (no accepted size does), and KDA_E_HIP if the
 * scratch array cannot be located on the current device.
 */
kda_status_t kda_chunk_prefill_noalloc(const kda_prefill_args_t* args, void* stream);

/*
 * Arguments of kda_recurrent_decode: one new token for each of N sequences.
 * All pointers are device pointers to contiguous row-major arrays.
 *  N, H, K, V      -- sequences (= tokens), heads, key dim (1..128), value dim (>= 1);
 *                     H, V, K must equal the cache's.
 *  q, k            -- [N, H, K] in qkv_dtype.       v -- [N, H, V] in qkv_dtype.
 *  g               -- [N, H, K] fp32 natural-log decays (state multiplied by exp(g)).
 *  beta            -- [N, H] in beta_dtype.
 *  state_indices   -- [N] int32 (KDA_I32) or int64 (KDA_I64): the cache row
 *                     holding sequence n's state, read in its own width.
 *  out             -- [N, H, V] in qkv_dtype; may be exactly v.
 *  scale, use_qk_l2norm -- as for kda_chunk_prefill.
 */
typedef struct {
  int64_t N, H, K, V;
  const void* q;
  const void* k;
  const void* v;
  kda_dtype_t qkv_dtype;
  const float* g;
  const void* beta;
  kda_dtype_t beta_dtype;
  const void* state_indices;
  kda_index_t index_type;
  void* out;
  float scale;
  int use_qk_l2norm;
} kda_decode_args_t;

/*
 * kda_recurrent_decode -- one step of the gated delta rule per sequence with
 * the state updated in place in its cache row ([P2] section 1.1 for one
 * token; decode runs its own recurrent kernel on the indexed state rows, [P1]
 * section "背景" and [P3] section "实现拆解").  For each n with
 * r = state_indices[n] in [0, num_rows) and each head h, with S the K x V
 * state of cache row r, head h (element (r,h,v,c) = S[c][v]):
 *   S <- (I - beta k^ k^T) Diag(exp g) S + beta k^ v^T   (written back to row r,
 *                                                       rounded to the cache dtype)
 *   out[n,h,:] = scale * S^T q^
 * computed in fp32.  An index outside [0, num_rows) marks a padding slot: its
 * output is zero and no cache row is read or written.
 * Preconditions (not checked, no device-to-host scan): valid indices are
 * unique within one call (rows are updated concurrently).  Aliasing (checked
 * on the host, KDA_E_ALIAS): neither the cache's address span nor out
 * overlaps q, k, v, g, beta, state_indices or the other, except that out may
 * be exactly v.
 * N == 0 validates the cache view and enqueues nothing.
 * Errors: KDA_E_NULL, KDA_E_DTYPE, KDA_E_SHAPE, KDA_E_LAYOUT, KDA_E_OVERLAP,
 * KDA_E_UNSUPPORTED, KDA_E_ALIAS, KDA_E_HIP.
 */
kda_status_t kda_recurrent_decode(const kda_state_cache_t* cache, const kda_decode_args_t* args, void* stream);

/*
 * A compressed (INT8) checkpoint store for one layer ([P2] section 5.3: parked
 * checkpoints compressed to INT8 and dequantised into a fresh active slot on
 * a hit; section 6.6.2: qdata [slots, heads, d_v, d_k] int8 and scale
 * [slots, heads, 1, d_k]).
 *  qdata         -- int8 codes; element (s, h, v, c) at qdata[s*qdata_stride0 + (h*V + v)*K + c].
 *  scale         -- fp32 scales; element (s, h, c) at scale[s*scale_stride0 + h*K + c].
 *  num_slots, H, V, K -- num_slots > 0, 1 <= K <= 128, H, V > 0.
 *  qdata_stride0 >= H*V*K and scale_stride0 >= H*K (slots never overlap); the
 *  qdata and scale address ranges must be disjoint.
 */
typedef struct {
  int8_t* qdata;
  float* scale;
  int64_t num_slots, H, V, K;
  int64_t qdata_stride0, scale_stride0;
} kda_int8_store_t;

/*
 * kda_ckpt_quantize_scatter -- for i in [0, num_selected): if
 * 0 <= indices[i] < num_slots, slot indices[i] receives packed[i] quantised
 * per (head, key channel c):
 *   amax_c  = max over v of |x[v][c]|,   scale_c = amax_c / 127   (fp32 division)
 *   code    = clamp(rint(x[v][c] / scale_c), -127, 127)            (fp32 division,
 *             ties to even), code = 0 where scale_c == 0.
 * Other entries are skipped.  packed: [num_selected, H, V, K] in packed_dtype
 * (fp32 or bf16), contiguous.  Preconditions (not checked): valid slots are
 * unique; finite inputs.  The store's qdata and scale ranges must not overlap
 * packed or indices (checked, KDA_E_ALIAS).  num_selected == 0 enqueues
 * nothing.
 * Errors: KDA_E_NULL, KDA_E_DTYPE, KDA_E_SHAPE, KDA_E_OVERLAP, KDA_E_UNSUPPORTED,
 * KDA_E_ALIAS, KDA_E_HIP.
 */
kda_status_t kda_ckpt_quantize_scatter(const kda_int8_store_t* store, const void* indices, kda_index_t index_type,
                                       int64_t num_selected, const void* packed, kda_dtype_t packed_dtype,
                                       void* stream);

/*
 * kda_ckpt_dequantize_gather -- for i in [0, num_selected):
 *   packed[i][h][v][c] = code * scale_c (fp32, then rounded to packed_dtype)
 *       if 0 <= indices[i] < num_slots and (flags == NULL or flags[i] != 0),
 *   packed[i] = zeros otherwise.
 * Every row of packed is written; the result can seed kda_chunk_prefill's
 * initial_state or go to active cache rows through kda_state_scatter.  packed
 * must not overlap the store, indices or flags (checked, KDA_E_ALIAS).
 * Errors as for kda_ckpt_quantize_scatter.
 */
kda_status_t kda_ckpt_dequantize_gather(const kda_int8_store_t* store, const void* indices, kda_index_t index_type,
                                        int64_t num_selected, const uint8_t* flags, void* packed,
                                        kda_dtype_t packed_dtype, void* stream);

/* Static, human-readable name of a status code. */
const char* kda_status_string(kda_status_t status);

/* Detail of the last KDA_E_HIP on this thread ("" if none). */
const char* kda_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
