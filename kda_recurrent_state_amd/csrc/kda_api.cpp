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

// A device byte range; an absent argument has p == NULL or bytes == 0.
struct Span {
  const void* p;
  int64_t bytes;
};

bool spans_overlap(const Span& a, const Span& b) {
  return a.p && b.p && a.bytes > 0 && b.bytes > 0 && ranges_overlap(a.p, a.bytes, b.p, b.bytes);
}

// Every output must be disjoint from every input and from the other outputs,
// except for the pairs (outs[i], ins[same[i]]) that are the very same range
// (same[i] < 0: no such exception).
bool alias_error(const Span* outs, const int* same, int nouts, const Span* ins, int nins) {
  for (int i = 0; i < nouts; ++i) {
    for (int j = 0; j < nins; ++j) {
      if (!spans_overlap(outs[i], ins[j])) continue;
      if (same[i] == j && outs[i].p == ins[j].p && outs[i].bytes == ins[j].bytes) continue;
      return true;
    }
    for (int j = i + 1; j < nouts; ++j)
      if (spans_overlap(outs[i], outs[j])) return true;
  }
  return false;
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
  if (num_selected > ((int64_t)1 << 40) / qpay) return KDA_E_SHAPE;
  if (num_selected == 0) return KDA_OK;
  if (!indices || !packed) return KDA_E_NULL;
  {
    const Span qd{st->qdata, (st->num_slots - 1) * st->qdata_stride0 + qpay};
    const Span sc{st->scale, ((st->num_slots - 1) * st->scale_stride0 + spay) * 4};
    const Span pk{packed, num_selected * qpay * dtype_bytes(pdt)};
    const Span ix{indices, num_selected * (it == KDA_I64 ? 8 : 4)};
    const Span fl{quantize ? nullptr : flags, num_selected};
    const int none[2] = {-1, -1};
    if (quantize) {
      const Span outs[2] = {qd, sc}, ins[2] = {pk, ix};
      if (alias_error(outs, none, 2, ins, 2)) return KDA_E_ALIAS;
    } else {
      const Span outs[1] = {pk}, ins[4] = {qd, sc, ix, fl};
      if (alias_error(outs, none, 1, ins, 4)) return KDA_E_ALIAS;
    }
  }
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

}  // extern "C"

namespace {

// Validation shared by kda_chunk_prefill and kda_chunk_prefill_noalloc: every
// check but the caller's workspace.  *need receives the workspace bytes the
// call uses; KDA_OK with a->N == 0 means there is nothing to enqueue.
kda_status_t check_prefill(const kda_prefill_args_t* a, size_t* need) {
  *need = 0;
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
  if (a->N > ((int64_t)1 << 40) / (a->H * a->V * a->K)) return KDA_E_SHAPE;
  if (a->ckpt_states && a->num_ckpt > ((int64_t)1 << 40) / (a->H * a->V * a->K)) return KDA_E_SHAPE;
  if (a->N == 0) return KDA_OK;
  if (!a->cu_seqlens) return KDA_E_NULL;
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out)) return KDA_E_NULL;
  *need = kda::chunk_prefill_workspace_bytes(a->T, a->N, a->H, a->K, a->V);
  {
    // out may be exactly v and final_state exactly initial_state (same
    // dtype); any other overlap between an output and an argument is an error
    const int64_t eb = dtype_bytes(a->qkv_dtype), TH = a->T * a->H, NHVK = a->N * a->H * a->V * a->K;
    const Span vin{a->v, TH * a->V * eb};
    const Span init{a->initial_state, a->initial_state ? NHVK * dtype_bytes(a->initial_dtype) : 0};
    const Span ins[8] = {{a->q, TH * a->K * eb},
                         {a->k, TH * a->K * eb},
                         vin,
                         {a->g, TH * a->K * 4},
                         {a->beta, TH * dtype_bytes(a->beta_dtype)},
                         {a->cu_seqlens, (a->N + 1) * 4},
                         init,
                         {a->ckpt_states ? a->ckpt_cu : nullptr, (a->N + 1) * 4}};
    const Span outs[4] = {{a->out, TH * a->V * eb},
                          {a->final_state, a->final_state ? NHVK * dtype_bytes(a->final_dtype) : 0},
                          {a->ckpt_states, a->ckpt_states ? a->num_ckpt * a->H * a->V * a->K * dtype_bytes(a->ckpt_dtype) : 0},
                          {*need > 0 ? a->workspace : nullptr, (int64_t)*need}};
    const int same[4] = {2, 6, -1, -1};
    if (alias_error(outs, same, 4, ins, 8)) return KDA_E_ALIAS;
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_prefill(const kda_prefill_args_t* a, void* stream) {
  size_t need = 0;
  const kda_status_t st = check_prefill(a, &need);
  if (st != KDA_OK || a->N == 0) return st;
  if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return KDA_E_WORKSPACE;
  hipError_t e = kda::launch_chunk_prefill(*a, static_cast<hipStream_t>(stream));
  return hip_status("kda_chunk_prefill launch", e);
}

kda_status_t kda_chunk_prefill_noalloc(const kda_prefill_args_t* a, void* stream) {
  kda_prefill_args_t b;
  size_t need = 0;
  if (a) {
    // the caller's workspace fields play no part
    b = *a;
    b.workspace = nullptr;
    b.workspace_bytes = 0;
  }
  const kda_status_t st = check_prefill(a ? &b : nullptr, &need);
  if (st != KDA_OK || b.N == 0) return st;
  if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_E_WORKSPACE;
  if (need > 0) {
    // this device's copy of the library's scratch array (set up on the first
    // call on each device)
    hipError_t e = kda::noalloc_scratch(&b.workspace);
    if (e != hipSuccess) return hip_status("kda_chunk_prefill_noalloc scratch lookup", e);
    b.workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
  }
  hipError_t e = kda::launch_chunk_prefill(b, static_cast<hipStream_t>(stream));
  return hip_status("kda_chunk_prefill_noalloc launch", e);
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
  {
    // the cache rows are updated in place; out may be exactly v; any other
    // overlap between the cache or out and an argument is an error
    const int64_t eb = dtype_bytes(a->qkv_dtype), NH = a->N * a->H;
    const Span ins[6] = {{a->q, NH * a->K * eb},
                         {a->k, NH * a->K * eb},
                         {a->v, NH * a->V * eb},
                         {a->g, NH * a->K * 4},
                         {a->beta, NH * dtype_bytes(a->beta_dtype)},
                         {a->state_indices, a->N * (a->index_type == KDA_I64 ? 8 : 4)}};
    const Span outs[2] = {{a->out, NH * a->V * eb},
                          {cache->data, ((cache->num_rows - 1) * cache->stride[0] + payload) * dtype_bytes(cache->dtype)}};
    const int same[2] = {2, -1};
    if (alias_error(outs, same, 2, ins, 6)) return KDA_E_ALIAS;
  }
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
    case KDA_E_ALIAS: return "KDA_E_ALIAS: an output overlaps an input or another output";
    case KDA_E_HIP: return "KDA_E_HIP: HIP runtime error";
  }
  return "unknown kda_status_t";
}

const char* kda_last_error_detail(void) { return g_detail; }

}  // extern "C"
