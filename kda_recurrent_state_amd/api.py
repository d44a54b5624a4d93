"""Python binding of libkda with the C ABI's names.

Argument marshalling only: tensors are described by pointer, dtype, sizes and
strides and handed to the C entry points together with the current HIP
stream.  Every step of the path runs in libkda's kernels; PyTorch supplies
device memory and streams.  A non-OK status raises :class:`KDAError`.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import KDA_BF16, KDA_F32, KDA_I32, KDA_I64, DecodeArgs, Int8Store, KDAError, PrefillArgs, StateCache

_DT = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype not in _DT:
        raise KDAError(what, 2, "dtype %s (need float32 or bfloat16)" % t.dtype)
    return _DT[t.dtype]


def _stream_handle(stream, device) -> int:
    """The given stream, or the current stream of ``device``."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _on_stream(stream, device, *tensors) -> None:
    """Tensors this binding allocated on the current stream but that a kernel
    uses on another ``stream``: tell PyTorch's caching allocator, so their
    memory is not handed out again before that stream's work is done."""
    if stream is None:
        return
    if not hasattr(stream, "cuda_stream"):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    if stream.cuda_stream == torch.cuda.current_stream(device).cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _device(*ts) -> torch.device:
    """The one device that all given tensors live on (device tensors only)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libkda works on device tensors; got a %s tensor" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("libkda arguments must share one device; got %s and %s" % (dev, t.device))
    return dev


def cache_descriptor(cache: torch.Tensor) -> StateCache:
    """Describe a 4-D [num_rows, H, V, K] cache view (storage offset included in data_ptr)."""
    if cache.dim() != 4:
        raise KDAError("kda_state_cache", 3, "cache must be 4-D [num_rows, H, V, K]")
    d = StateCache()
    d.data = cache.data_ptr()
    d.dtype = _DT.get(cache.dtype, 99)
    d.num_rows, d.H, d.V, d.K = (int(x) for x in cache.shape)
    for i, s in enumerate(cache.stride()):
        d.stride[i] = int(s)
    return d


def _index_code(indices: torch.Tensor) -> int:
    if indices.dtype == torch.int32:
        return KDA_I32
    if indices.dtype == torch.int64:
        return KDA_I64
    raise KDAError("state copy", 2, "indices must be int32 or int64")


def kda_state_gather(cache: torch.Tensor, indices: torch.Tensor, flags: Optional[torch.Tensor] = None,
                     packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """packed[i] = cache[indices[i]] if valid and flagged, else zeros (all rows written)."""
    lib = _lib.load_library()
    dev = _device(cache, indices, flags, packed)
    if indices.dim() != 1 or not indices.is_contiguous():
        raise KDAError("kda_state_gather", 3, "indices must be a contiguous 1-D tensor")
    S = indices.shape[0]
    if packed is None:
        packed = torch.empty((S,) + tuple(cache.shape[1:]), dtype=cache.dtype, device=cache.device)
        _on_stream(stream, dev, packed)
    if packed.dtype != cache.dtype or not packed.is_contiguous() or tuple(packed.shape) != (S,) + tuple(cache.shape[1:]):
        raise KDAError("kda_state_gather", 3, "packed must be a contiguous [S,H,V,K] tensor of the cache dtype")
    fptr = None
    if flags is not None:
        if flags.dtype not in (torch.bool, torch.uint8) or flags.numel() != S or not flags.is_contiguous():
            raise KDAError("kda_state_gather", 2, "flags must be a contiguous bool/uint8 tensor of length S")
        fptr = flags.data_ptr()
    d = cache_descriptor(cache)
    with torch.cuda.device(dev):
        st = lib.kda_state_gather(ctypes.byref(d), indices.data_ptr(), _index_code(indices), S, fptr,
                                  packed.data_ptr(), _stream_handle(stream, dev))
    _lib.check("kda_state_gather", st)
    return packed


def kda_state_scatter(cache: torch.Tensor, indices: torch.Tensor, packed: torch.Tensor, stream=None) -> None:
    """cache[indices[i]] = packed[i] for every valid index (flags play no part)."""
    lib = _lib.load_library()
    dev = _device(cache, indices, packed)
    if indices.dim() != 1 or not indices.is_contiguous():
        raise KDAError("kda_state_scatter", 3, "indices must be a contiguous 1-D tensor")
    S = indices.shape[0]
    if packed.dtype != cache.dtype or not packed.is_contiguous() or tuple(packed.shape) != (S,) + tuple(cache.shape[1:]):
        raise KDAError("kda_state_scatter", 3, "packed must be a contiguous [S,H,V,K] tensor of the cache dtype")
    d = cache_descriptor(cache)
    with torch.cuda.device(dev):
        st = lib.kda_state_scatter(ctypes.byref(d), indices.data_ptr(), _index_code(indices), S, packed.data_ptr(),
                                   _stream_handle(stream, dev))
    _lib.check("kda_state_scatter", st)


def kda_chunk_prefill_workspace_size(T: int, N: int, H: int, K: int, V: int) -> int:
    return int(_lib.load_library().kda_chunk_prefill_workspace_size(T, N, H, K, V))


def kda_chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                      cu_seqlens: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                      final_dtype: Optional[torch.dtype] = torch.float32, scale: Optional[float] = None,
                      use_qk_l2norm: bool = True, workspace: Optional[torch.Tensor] = None, stream=None,
                      ckpt_interval: int = 0, ckpt_cu: Optional[torch.Tensor] = None,
                      ckpt_states: Optional[torch.Tensor] = None):
    """Chunked gated delta rule over a varlen batch.

    q, k: [T,H,K]; v: [T,H,V] (fp32 or bf16, same dtype); g: [T,H,K] fp32;
    beta: [T,H]; cu_seqlens: [N+1] int32; initial_state: [N,H,V,K] or None.
    Returns (out [T,H,V], final_state [N,H,V,K] or None).  ``out`` may be ``v``.
    ``final_dtype=None`` skips the final state unless ``final_state`` is given.

    Checkpoints (optional): with ``ckpt_states`` ([num_ckpt,H,V,K], fp32 or
    bf16) and ``ckpt_cu`` ([N+1] int32, e.g. from ``checkpoint_offsets``),
    row ckpt_cu[n]+j receives the state of sequence n after
    (j+1)*ckpt_interval tokens; ckpt_interval is a positive multiple of 64.
    """
    return _prefill("kda_chunk_prefill", q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                    final_dtype, scale, use_qk_l2norm, workspace, stream, ckpt_interval, ckpt_cu, ckpt_states)


def kda_chunk_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                              beta: torch.Tensor, cu_seqlens: torch.Tensor, out: torch.Tensor,
                              initial_state: Optional[torch.Tensor] = None,
                              final_state: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                              use_qk_l2norm: bool = True, stream=None, ckpt_interval: int = 0,
                              ckpt_cu: Optional[torch.Tensor] = None, ckpt_states: Optional[torch.Tensor] = None):
    """kda_chunk_prefill that allocates nothing: ``out`` (and ``final_state``,
    if wanted) are the caller's, and the workspace is the library's static
    per-device scratch.  Calls that can overlap on one device race on that
    scratch.  Returns (out, final_state)."""
    return _prefill("kda_chunk_prefill_noalloc", q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                    None, scale, use_qk_l2norm, None, stream, ckpt_interval, ckpt_cu, ckpt_states)


def _prefill(entry, q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, final_dtype, scale,
             use_qk_l2norm, workspace, stream, ckpt_interval, ckpt_cu, ckpt_states):
    noalloc = entry == "kda_chunk_prefill_noalloc"
    lib = _lib.load_library()
    dev = _device(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, workspace, ckpt_cu, ckpt_states)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise KDAError(entry, 3, "q,k must be [T,H,K] and v [T,H,V]")
    T, H, K = (int(x) for x in q.shape)
    V = int(v.shape[2])
    N = int(cu_seqlens.numel()) - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("cu_seqlens", cu_seqlens)):
        if not t.is_contiguous():
            raise KDAError(entry, 4, "%s must be contiguous" % name)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise KDAError(entry, 2, "q, k, v must share a dtype")
    if g.dtype != torch.float32 or tuple(g.shape) != (T, H, K):
        raise KDAError(entry, 2, "g must be float32 [T,H,K]")
    if tuple(beta.shape) != (T, H):
        raise KDAError(entry, 3, "beta must be [T,H]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or N < 0:
        raise KDAError(entry, 2, "cu_seqlens must be int32 [N+1]")
    if noalloc and out is None:
        raise KDAError(entry, 1, "out must be given (the call allocates nothing)")
    made = []   # tensors allocated here (on the current stream)
    if out is None:
        out = torch.empty((T, H, V), dtype=q.dtype, device=q.device)
        made.append(out)
    if out.dtype != q.dtype or tuple(out.shape) != (T, H, V) or not out.is_contiguous():
        raise KDAError(entry, 3, "out must be a contiguous [T,H,V] tensor of q's dtype")
    if final_state is None and final_dtype is not None and N > 0:
        final_state = torch.empty((N, H, V, K), dtype=final_dtype, device=q.device)
        made.append(final_state)
    for name, s in (("initial_state", initial_state), ("final_state", final_state)):
        if s is not None and (tuple(s.shape) != (N, H, V, K) or not s.is_contiguous()):
            raise KDAError(entry, 3, "%s must be a contiguous [N,H,V,K] tensor" % name)
    if ckpt_states is not None:
        if ckpt_cu is None or ckpt_cu.dtype != torch.int32 or ckpt_cu.numel() != N + 1:
            raise KDAError(entry, 2, "ckpt_cu must be int32 [N+1]")
        if ckpt_states.dim() != 4 or tuple(ckpt_states.shape[1:]) != (H, V, K) or not ckpt_states.is_contiguous():
            raise KDAError(entry, 3, "ckpt_states must be a contiguous [num_ckpt,H,V,K] tensor")
    need = 0 if noalloc else int(lib.kda_chunk_prefill_workspace_size(T, N, H, K, V))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        made.append(workspace)
    if need > 0 and workspace.numel() * workspace.element_size() < need:
        raise KDAError(entry, 7, "workspace of %d bytes, need %d (kda_chunk_prefill_workspace_size)"
                       % (workspace.numel() * workspace.element_size(), need))
    _on_stream(stream, dev, *made)
    a = PrefillArgs()
    a.T, a.N, a.H, a.K, a.V = T, N, H, K, V
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.qkv_dtype = _dtype_code(q, "kda_chunk_prefill")
    a.g = g.data_ptr()
    a.beta = beta.data_ptr()
    a.beta_dtype = _dtype_code(beta, "kda_chunk_prefill")
    a.cu_seqlens = cu_seqlens.data_ptr()
    a.initial_state = initial_state.data_ptr() if initial_state is not None else None
    a.initial_dtype = _dtype_code(initial_state, "kda_chunk_prefill") if initial_state is not None else KDA_F32
    a.out = out.data_ptr()
    a.final_state = final_state.data_ptr() if final_state is not None else None
    a.final_dtype = _dtype_code(final_state, "kda_chunk_prefill") if final_state is not None else KDA_F32
    a.scale = float(K ** -0.5 if scale is None else scale)
    a.use_qk_l2norm = 1 if use_qk_l2norm else 0
    a.workspace = workspace.data_ptr() if (workspace is not None and need > 0) else None
    a.workspace_bytes = need if (workspace is not None and need > 0) else 0
    if ckpt_states is not None:
        a.ckpt_interval = int(ckpt_interval)
        a.ckpt_cu = ckpt_cu.data_ptr()
        a.ckpt_states = ckpt_states.data_ptr()
        a.num_ckpt = int(ckpt_states.shape[0])
        a.ckpt_dtype = _dtype_code(ckpt_states, "kda_chunk_prefill")
    with torch.cuda.device(dev):
        st = getattr(lib, entry)(ctypes.byref(a), _stream_handle(stream, dev))
    _lib.check(entry, st)
    return out, final_state


def kda_recurrent_decode(cache: torch.Tensor, state_indices: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                         v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, out: Optional[torch.Tensor] = None,
                         scale: Optional[float] = None, use_qk_l2norm: bool = True, stream=None) -> torch.Tensor:
    """One decode token per sequence; cache rows state_indices[n] updated in place.

    cache: [num_rows,H,V,K] view (fp32 or bf16, dense inner dims); state_indices:
    [N] int32/int64 (outside [0,num_rows) = padding slot: zero output, no state
    access); q, k, g: [N,H,K]; v: [N,H,V]; beta: [N,H].  Returns out [N,H,V]
    (may be ``v``).  Valid indices must be unique.
    """
    lib = _lib.load_library()
    dev = _device(cache, state_indices, q, k, v, g, beta, out)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise KDAError("kda_recurrent_decode", 3, "q,k must be [N,H,K] and v [N,H,V]")
    N, H, K = (int(x) for x in q.shape)
    V = int(v.shape[2])
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state_indices", state_indices)):
        if not t.is_contiguous():
            raise KDAError("kda_recurrent_decode", 4, "%s must be contiguous" % name)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise KDAError("kda_recurrent_decode", 2, "q, k, v must share a dtype")
    if g.dtype != torch.float32 or tuple(g.shape) != (N, H, K):
        raise KDAError("kda_recurrent_decode", 2, "g must be float32 [N,H,K]")
    if tuple(beta.shape) != (N, H):
        raise KDAError("kda_recurrent_decode", 3, "beta must be [N,H]")
    if state_indices.dim() != 1 or state_indices.numel() != N:
        raise KDAError("kda_recurrent_decode", 3, "state_indices must be [N]")
    if out is None:
        out = torch.empty((N, H, V), dtype=q.dtype, device=q.device)
        _on_stream(stream, dev, out)
    if out.dtype != q.dtype or tuple(out.shape) != (N, H, V) or not out.is_contiguous():
        raise KDAError("kda_recurrent_decode", 3, "out must be a contiguous [N,H,V] tensor of q's dtype")
    d = cache_descriptor(cache)
    a = DecodeArgs()
    a.N, a.H, a.K, a.V = N, H, K, V
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.qkv_dtype = _dtype_code(q, "kda_recurrent_decode")
    a.g = g.data_ptr()
    a.beta = beta.data_ptr()
    a.beta_dtype = _dtype_code(beta, "kda_recurrent_decode")
    a.state_indices = state_indices.data_ptr()
    a.index_type = _index_code(state_indices)
    a.out = out.data_ptr()
    a.scale = float(K ** -0.5 if scale is None else scale)
    a.use_qk_l2norm = 1 if use_qk_l2norm else 0
    with torch.cuda.device(dev):
        st = lib.kda_recurrent_decode(ctypes.byref(d), ctypes.byref(a), _stream_handle(stream, dev))
    _lib.check("kda_recurrent_decode", st)
    return out


def int8_store_descriptor(qdata: torch.Tensor, scale: torch.Tensor) -> Int8Store:
    """Describe an INT8 checkpoint store: qdata [num_slots,H,V,K] int8 and scale
    [num_slots,H,1,K] (or [num_slots,H,K]) fp32, inner dims dense, any slot stride."""
    if qdata.dim() != 4 or qdata.dtype != torch.int8:
        raise KDAError("int8 store", 2, "qdata must be an int8 [num_slots,H,V,K] tensor")
    S, H, V, K = (int(x) for x in qdata.shape)
    if scale.dtype != torch.float32 or scale.shape[0] != S or scale.numel() != S * H * K:
        raise KDAError("int8 store", 2, "scale must be float32 [num_slots,H,1,K]")
    sc = scale.reshape(S, H, K) if scale.dim() == 4 else scale
    if tuple(qdata.stride()[1:]) != (V * K, K, 1) or tuple(sc.stride()[1:]) != (K, 1):
        raise KDAError("int8 store", 4, "qdata [H,V,K] and scale [H,K] must be dense within a slot")
    d = Int8Store()
    d.qdata, d.scale = qdata.data_ptr(), scale.data_ptr()
    d.num_slots, d.H, d.V, d.K = S, H, V, K
    d.qdata_stride0, d.scale_stride0 = int(qdata.stride(0)), int(sc.stride(0))
    return d


def kda_ckpt_quantize_scatter(qdata: torch.Tensor, scale: torch.Tensor, indices: torch.Tensor, packed: torch.Tensor,
                              stream=None) -> None:
    """Slots indices[i] of the INT8 store <- quantised packed[i] (invalid slots skipped)."""
    lib = _lib.load_library()
    dev = _device(qdata, scale, indices, packed)
    if indices.dim() != 1 or not indices.is_contiguous():
        raise KDAError("kda_ckpt_quantize_scatter", 3, "indices must be a contiguous 1-D tensor")
    S = int(indices.shape[0])
    if tuple(packed.shape) != (S,) + tuple(qdata.shape[1:]) or not packed.is_contiguous():
        raise KDAError("kda_ckpt_quantize_scatter", 3, "packed must be a contiguous [S,H,V,K] tensor")
    d = int8_store_descriptor(qdata, scale)
    with torch.cuda.device(dev):
        st = lib.kda_ckpt_quantize_scatter(ctypes.byref(d), indices.data_ptr(), _index_code(indices), S,
                                           packed.data_ptr(), _dtype_code(packed, "kda_ckpt_quantize_scatter"),
                                           _stream_handle(stream, dev))
    _lib.check("kda_ckpt_quantize_scatter", st)


def kda_ckpt_dequantize_gather(qdata: torch.Tensor, scale: torch.Tensor, indices: torch.Tensor,
                               flags: Optional[torch.Tensor] = None, packed: Optional[torch.Tensor] = None,
                               dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """packed[i] = dequantised slot indices[i] if valid and flagged, else zeros."""
    lib = _lib.load_library()
    dev = _device(qdata, scale, indices, flags, packed)
    if indices.dim() != 1 or not indices.is_contiguous():
        raise KDAError("kda_ckpt_dequantize_gather", 3, "indices must be a contiguous 1-D tensor")
    S = int(indices.shape[0])
    if packed is None:
        packed = torch.empty((S,) + tuple(qdata.shape[1:]), dtype=dtype, device=qdata.device)
        _on_stream(stream, dev, packed)
    if tuple(packed.shape) != (S,) + tuple(qdata.shape[1:]) or not packed.is_contiguous():
        raise KDAError("kda_ckpt_dequantize_gather", 3, "packed must be a contiguous [S,H,V,K] tensor")
    fptr = None
    if flags is not None:
        if flags.dtype not in (torch.bool, torch.uint8) or flags.numel() != S or not flags.is_contiguous():
            raise KDAError("kda_ckpt_dequantize_gather", 2, "flags must be a contiguous bool/uint8 tensor of length S")
        fptr = flags.data_ptr()
    d = int8_store_descriptor(qdata, scale)
    with torch.cuda.device(dev):
        st = lib.kda_ckpt_dequantize_gather(ctypes.byref(d), indices.data_ptr(), _index_code(indices), S, fptr,
                                            packed.data_ptr(), _dtype_code(packed, "kda_ckpt_dequantize_gather"),
                                            _stream_handle(stream, dev))
    _lib.check("kda_ckpt_dequantize_gather", st)
    return packed


def checkpoint_offsets(lengths, interval: int):
    """Row offsets [N+1] of the chunk-boundary checkpoints of a batch: sequence
    n of length len_n owns floor(len_n / interval) rows (host-side helper)."""
    if interval <= 0 or interval % 64:
        raise ValueError("interval must be a positive multiple of 64")
    offs = [0]
    for n in lengths:
        offs.append(offs[-1] + int(n) // int(interval))
    return offs


class KDAStateCopy:
    """A cache view validated once, with a bound on the selection size.

    Mirrors the prepared-plan idea of the vllm-ascend state-copy page (section
    "启动准备"): the cache layout is checked when the object is made, and a
    launch that selects more than ``max_selected`` rows is rejected.  Nothing
    is compiled or retained beyond the tensor reference.
    """

    def __init__(self, cache: torch.Tensor, max_selected: int):
        self.cache = cache
        self.max_selected = int(max_selected)
        lib = _lib.load_library()
        d = cache_descriptor(cache)
        # validate the layout (S = 0 launches nothing)
        st = lib.kda_state_gather(ctypes.byref(d), None, KDA_I32, 0, None, None, None)
        _lib.check("KDAStateCopy", st)

    def _check(self, indices: torch.Tensor):
        if indices.numel() > self.max_selected:
            raise KDAError("KDAStateCopy", 3, "selected %d rows > max_selected %d"
                           % (indices.numel(), self.max_selected))

    def gather(self, indices, flags=None, packed=None, stream=None):
        self._check(indices)
        return kda_state_gather(self.cache, indices, flags, packed, stream)

    def scatter(self, indices, packed, stream=None):
        self._check(indices)
        kda_state_scatter(self.cache, indices, packed, stream)
