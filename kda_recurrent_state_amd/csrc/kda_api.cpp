// Host entry points of libkda: argument validation and kernel dispatch.
//
// Validation is host-only and fail-closed, as the copy contract of the page
// "vllm-ascend 的 KDA 状态复制 Triton 集成：PR 17301 对齐的预编译 worker 生命周期方案"
// asks (sections "数值契约" and "启动准备"): no device reads, no
// synchronisation, no environment scan, no conversion of int32 indices; a bad
// layout returns an error and enqueues nothing; an empty selection validates
// the cache view and enqueues nothing.
#include <string.h>

#include "internal.h"

namespace {

thread_local char g_detail[256] = "";

void set_detail(const char* what, hipError_t e) {
  const char* s = hipGetErrorString(e);
  size_t n = strlen(what);
  if (n > 100) n = 100;
  memcpy(g_detail, what, n);
  g_detail[n] = ':';
  g_detail[n + 1] = ' ';
  strncpy(g_detail + n + 2, s ? s : "?", sizeof(g_detail) - n - 3);
  g_detail[sizeof(g_detail) - 1] = 0;
}

kda_status_t hip_status(const char* what, hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  set_detail(what, e);
  return KDA_E_HIP;
}

int64_t dtype_bytes(kda_dtype_t d) { return d == KDA_F32 ? 4 : (d == KDA_BF16 ? 2 : 0); }

bool valid_dtype(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }

// Layout admissibility: 4-D, num_rows > 0, positive inner sizes, inner dims
// dense from the back (size 1 or stride = running payload), rows disjoint.
kda_status_t check_cache(const kda_state_cache_t* c, int64_t* payload_elems) {
  if (!c) return KDA_E_NULL;
  if (!valid_dtype(c->dtype)) return KDA_E_DTYPE;
  if (c->num_rows <= 0 || c->H <= 0 || c->V <= 0 || c->K <= 0) return KDA_E_SHAPE;
  const int64_t sizes[3] = {c->H, c->V, c->K};
  int64_t run = 1;
  for (int d = 2; d >= 0; --d) {
    if (sizes[d] != 1 && c->stride[d + 1] != run) return KDA_E_LAYOUT;
    if (run > ((int64_t)1 << 40) / sizes[d]) return KDA_E_SHAPE;
    run *= sizes[d];
  }
  if (c->stride[0] < run) return KDA_E_OVERLAP;
  if (c->stride[0] > ((int64_t)1 << 46) / c->num_rows) return KDA_E_SHAPE;
  if (!c->data) return KDA_E_NULL;
  *payload_elems = run;
  return KDA_OK;
}

kda_status_t copy_common(bool gather, const kda_state_cache_t* cache, const void* indices, kda_index_t it,
                         int64_t num_selected, const uint8_t* flags, void* packed, void* stream) {
  int64_t payload = 0;
  kda_status_t st = check_cache(cache, &payload);
  if (st != KDA_OK) return st;
  if (it != KDA_I32 && it != KDA_I64) return KDA_E_DTYPE;
  if (num_selected < 0) return KDA_E_SHAPE;
  if (num_selected == 0) return KDA_OK;
  if (!indices || !packed) return KDA_E_NULL;
  const int64_t eb = dtype_bytes(cache->dtype);
  hipError_t e = kda::launch_state_copy(gather, static_cast<char*>(cache->data), cache->stride[0] * eb,
                                        cache->num_rows, payload * eb, indices, it == KDA_I64, num_selected,
                                        gather ? flags : nullptr, static_cast<char*>(packed),
                                        static_cast<hipStream_t>(stream));
  return hip_status(gather ? "kda_state_gather launch" : "kda_state_scatter launch", e);
}

bool ranges_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

kda_status_t int8_common(bool quantize, const kda_int8_store_t* st, const void* indices, kda_index_t it,
                         int64_t num_selected, const uint8_t* flags, void* packed, kda_dtype_t pdt, void* stream) {
  if (!st) return KDA_E_NULL;
  if (st->num_slots <= 0 || st->H <= 0 || st->V <= 0 || st->K <= 0) return KDA_E_SHAPE;
  if (st->K > 128) return KDA_E_UNSUPPORTED;
  if (st->H * st->V > ((int64_t)1 << 40) / st->K) return KDA_E_SHAPE;
  const int64_t qpay = st->H * st->V * st->K, spay = st->H * st->K;
  if (st->qdata_stride0 < qpay || st->scale_stride0 < spay) return KDA_E_OVERLAP;
  if (st->qdata_stride0 > ((int64_t)1 << 46) / st->num_slots || st->scale_stride0 > ((int64_t)1 << 46) / st->num_slots)
    return KDA_E_SHAPE;
  if (!st->qdata || !st->scale) return KDA_E_NULL;
  if (ranges_overlap(st->qdata, (st->num_slots - 1) * st->qdata_stride0 + qpay, st->scale,
                     ((st->num_slots - 1) * st->scale_stride0 + spay) * 4))
    return KDA_E_OVERLAP;
  if (!valid_dtype(pdt)) return KDA_E_DTYPE;
  if (it != KDA_I32 && it != KDA_I64) return KDA_E_DTYPE;
  if (num_selected < 0) return KDA_E_SHAPE;
  if (num_selected == 0) return KDA_OK;
  if (!indices || !packed) return KDA_E_NULL;
  hipError_t e = kda::launch_int8_ckpt(quantize, *st, indices, it == KDA_I64, num_selected, quantize ? nullptr : flags,
                                       packed, pdt == KDA_BF16, static_cast<hipStream_t>(stream));
  return hip_status(quantize ? "kda_ckpt_quantize_scatter launch" : "kda_ckpt_dequantize_gather launch", e);
}

}  // namespace

extern "C" {

kda_status_t kda_state_gather(const kda_state_cache_t* cache, const void* indices, kda_index_t index_type,
                              int64_t num_selected, const uint8_t* flags, void* packed, void* stream) {
  return copy_common(true, cache, indices, index_type, num_selected, flags, packed, stream);
}

kda_status_t kda_state_scatter(const kda_state_cache_t* cache, const void* indices, kda_index_t index_type,
                               int64_t num_selected, const void* packed, void* stream) {
  return copy_common(false, cache, indices, index_type, num_selected, nullptr, const_cast<void*>(packed), stream);
}

size_t kda_chunk_prefill_workspace_size(int64_t T, int64_t N, int64_t H, int64_t K, int64_t V) {
  return kda::chunk_prefill_workspace_bytes(T, N, H, K, V);
}

kda_status_t kda_chunk_prefill(const kda_prefill_args_t* a, void* stream) {
  if (!a) return KDA_E_NULL;
  if (a->T < 0 || a->N < 0 || a->H <= 0 || a->K <= 0 || a->V <= 0) return KDA_E_SHAPE;
  if (a->N == 0 && a->T != 0) return KDA_E_SHAPE;
  if (!valid_dtype(a->qkv_dtype) || !valid_dtype(a->beta_dtype)) return KDA_E_DTYPE;
  if (a->initial_state && !valid_dtype(a->initial_dtype)) return KDA_E_DTYPE;
  if (a->final_state && !valid_dtype(a->final_dtype)) return KDA_E_DTYPE;
  if (a->K > 128) return KDA_E_UNSUPPORTED;
  if (a->H * (a->K > a->V ? a->K : a->V) > ((int64_t)1 << 22)) return KDA_E_UNSUPPORTED;  // 32-bit chunk offsets
  if (a->ckpt_states) {
    if (a->ckpt_interval <= 0 || a->ckpt_interval % 64 != 0 || a->num_ckpt < 0) return KDA_E_SHAPE;
    if (!a->ckpt_cu) return KDA_E_NULL;
    if (!valid_dtype(a->ckpt_dtype)) return KDA_E_DTYPE;
  }
  if (a->T > ((int64_t)1 << 40) / (a->H * (a->K > a->V ? a->K : a->V))) return KDA_E_SHAPE;
  if (a->N == 0) return KDA_OK;
  if (!a->cu_seqlens) return KDA_E_NULL;
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out)) return KDA_E_NULL;
  const size_t need = kda::chunk_prefill_workspace_bytes(a->T, a->N, a->H, a->K, a->V);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return KDA_E_WORKSPACE;
  const int64_t eb = dtype_bytes(a->qkv_dtype);
  if (a->T > 0) {
    const int64_t ob = a->T * a->H * a->V * eb;
    const int64_t kb = a->T * a->H * a->K * eb;
    if (a->out != a->v && ranges_overlap(a->out, ob, a->v, ob)) return KDA_E_ALIAS;
    if (ranges_overlap(a->out, ob, a->q, kb) || ranges_overlap(a->out, ob, a->k, kb) ||
        ranges_overlap(a->out, ob, a->g, a->T * a->H * a->K * 4))
      return KDA_E_ALIAS;
    if (a->final_state &&
        ranges_overlap(a->out, ob, a->final_state, a->N * a->H * a->V * a->K * dtype_bytes(a->final_dtype)))
      return KDA_E_ALIAS;
  }
  hipError_t e = kda::launch_chunk_prefill(*a, static_cast<hipStream_t>(stream));
  return hip_status("kda_chunk_prefill launch", e);
}

kda_status_t kda_recurrent_decode(const kda_state_cache_t* cache, const kda_decode_args_t* a, void* stream) {
  int64_t payload = 0;
  kda_status_t st = check_cache(cache, &payload);
  if (st != KDA_OK) return st;
  if (!a) return KDA_E_NULL;
  if (a->N < 0 || a->H <= 0 || a->K <= 0 || a->V <= 0) return KDA_E_SHAPE;
  if (a->H != cache->H || a->V != cache->V || a->K != cache->K) return KDA_E_SHAPE;
  if (!valid_dtype(a->qkv_dtype) || !valid_dtype(a->beta_dtype)) return KDA_E_DTYPE;
  if (a->index_type != KDA_I32 && a->index_type != KDA_I64) return KDA_E_DTYPE;
  if (a->K > 128) return KDA_E_UNSUPPORTED;
  if (a->V * a->K * 4 >= ((int64_t)1 << 31)) return KDA_E_UNSUPPORTED;  // 32-bit offsets within a head's state
  if (a->N > ((int64_t)1 << 40) / (a->H * (a->K > a->V ? a->K : a->V))) return KDA_E_SHAPE;
  if (a->N == 0) return KDA_OK;
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->state_indices || !a->out) return KDA_E_NULL;
  const int64_t eb = dtype_bytes(a->qkv_dtype);
  const int64_t ob = a->N * a->H * a->V * eb;
  const int64_t kb = a->N * a->H * a->K * eb;
  if (a->out != a->v && ranges_overlap(a->out, ob, a->v, ob)) return KDA_E_ALIAS;
  if (ranges_overlap(a->out, ob, a->q, kb) || ranges_overlap(a->out, ob, a->k, kb) ||
      ranges_overlap(a->out, ob, a->g, a->N * a->H * a->K * 4))
    return KDA_E_ALIAS;
  const int64_t span = ((cache->num_rows - 1) * cache->stride[0] + payload) * dtype_bytes(cache->dtype);
  if (ranges_overlap(a->out, ob, cache->data, span)) return KDA_E_ALIAS;
  hipError_t e = kda::launch_recurrent_decode(*cache, *a, static_cast<hipStream_t>(stream));
  return hip_status("kda_recurrent_decode launch", e);
}

kda_status_t kda_ckpt_quantize_scatter(const kda_int8_store_t* store, const void* indices, kda_index_t index_type,
                                       int64_t num_selected, const void* packed, kda_dtype_t packed_dtype,
                                       void* stream) {
  return int8_common(true, store, indices, index_type, num_selected, nullptr, const_cast<void*>(packed),
                     packed_dtype, stream);
}

kda_status_t kda_ckpt_dequantize_gather(const kda_int8_store_t* store, const void* indices, kda_index_t index_type,
                                        int64_t num_selected, const uint8_t* flags, void* packed,
                                        kda_dtype_t packed_dtype, void* stream) {
  return int8_common(false, store, indices, index_type, num_selected, flags, packed, packed_dtype, stream);
}

const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_E_NULL: return "KDA_E_NULL: a required pointer is NULL";
    case KDA_E_DTYPE: return "KDA_E_DTYPE: unsupported dtype or index type";
    case KDA_E_SHAPE: return "KDA_E_SHAPE: invalid size";
    case KDA_E_LAYOUT: return "KDA_E_LAYOUT: cache inner dims [H,V,K] are not dense";
    case KDA_E_OVERLAP: return "KDA_E_OVERLAP: cache row stride is smaller than the row payload";
    case KDA_E_UNSUPPORTED: return "KDA_E_UNSUPPORTED: no kernel for these sizes";
    case KDA_E_WORKSPACE: return "KDA_E_WORKSPACE: workspace missing or too small";
    case KDA_E_ALIAS: return "KDA_E_ALIAS: output overlaps an input";
    case KDA_E_HIP: return "KDA_E_HIP: HIP runtime error";
  }
  return "unknown kda_status_t";
}

const char* kda_last_error_detail(void) { return g_detail; }

}  // extern "C"
