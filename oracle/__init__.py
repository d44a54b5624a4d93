"""KDA prefill oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``kda_recurrent_state_amd``) never imports it and shares no code with it.

What it provides (fp64, plain loops in ``kda_oracle.c``):

* :func:`state_gather` / :func:`state_scatter` -- the state-copy contract of
  the page "vllm-ascend 的 KDA 状态复制 Triton 集成" (section "数值契约"):
  invalid or negative indices and false flags gather zeros, scatter skips
  invalid targets and ignores flags, page gaps and storage offsets are never
  touched.  Raw bits are copied.
* :func:`kda_recurrence` -- the gated delta rule token by token,
  S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
  o_t = scale * S_t^T q_t, over a varlen batch (page
  "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对", section 1.1).
* :func:`checkpoint_states` -- states at every ``interval`` tokens of each
  sequence (prefix-boundary checkpoints), from the recurrence above.
* :func:`recurrent_decode` -- one token per sequence against indexed state
  rows (explicit-matrix form, numpy fp64); padding slots give zeros.
* :func:`int8_quantize` / :func:`int8_dequantize` and the store/load
  contracts :func:`int8_quantize_scatter` / :func:`int8_dequantize_gather`
  -- the INT8 checkpoint codec (numpy, decisions in fp32).
* :mod:`oracle.chunk_form` -- the same map evaluated through the chunk
  decomposition stages of "PR #33465 完整报告" (section "关键源码片段"), in
  fp64 numpy; used to pin the chunk formulas, never by the product path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

L2NORM_EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_state_gather.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, ctypes.c_int, i64, vp, vp]
        lib.oracle_state_gather.restype = ctypes.c_int
        lib.oracle_state_scatter.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, ctypes.c_int, i64, vp]
        lib.oracle_state_scatter.restype = ctypes.c_int
        lib.oracle_kda_recurrence.argtypes = [i64, i64, i64, i64, vp, dp, dp, dp, dp, dp, dp,
                                              ctypes.c_double, ctypes.c_int, ctypes.c_double, dp, dp,
                                              ctypes.c_int]
        lib.oracle_kda_recurrence.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _raw_dtype(elem_bytes: int):
    if elem_bytes == 4:
        return np.uint32
    if elem_bytes == 2:
        return np.uint16
    raise ValueError("elem_bytes must be 2 or 4")


def state_gather(backing: np.ndarray, offset: int, shape, strides, indices: np.ndarray,
                 flags: np.ndarray | None) -> np.ndarray:
    """Gather rows of a cache view into a packed [S,H,V,K] array of raw bits.

    ``backing`` is the whole allocation as a 1-D uint32 (fp32) or uint16
    (bf16) array; the cache view starts ``offset`` elements in and has the
    given ``shape`` (num_rows, H, V, K) and element ``strides``.
    """
    lib = _load()
    backing = np.ascontiguousarray(backing)
    eb = backing.dtype.itemsize
    nrows, H, V, K = (int(x) for x in shape)
    st = np.asarray(strides, dtype=np.int64)
    idx = np.ascontiguousarray(indices)
    if idx.dtype not in (np.int32, np.int64):
        raise TypeError("indices must be int32 or int64")
    S = idx.shape[0]
    packed = np.empty((S, H, V, K), dtype=_raw_dtype(eb))
    fl = None if flags is None else np.ascontiguousarray(flags.astype(np.uint8))
    base = backing.ctypes.data + int(offset) * eb
    rc = lib.oracle_state_gather(base, eb, nrows, H, V, K, _ptr(st), _ptr(idx), int(idx.dtype == np.int64),
                                 S, None if fl is None else _ptr(fl), _ptr(packed))
    if rc != 0:
        raise RuntimeError("oracle_state_gather failed: %d" % rc)
    return packed


def state_scatter(backing: np.ndarray, offset: int, shape, strides, indices: np.ndarray,
                  packed: np.ndarray, in_place: bool = False) -> np.ndarray:
    """Return a copy of ``backing`` with the valid packed rows written to the
    cache view (``in_place``: write into ``backing`` itself, which must be a
    contiguous array, and return it)."""
    lib = _load()
    if in_place:
        if not backing.flags.c_contiguous:
            raise ValueError("in-place scatter needs a contiguous backing array")
        out = backing
    else:
        out = np.array(backing, copy=True)
    eb = out.dtype.itemsize
    nrows, H, V, K = (int(x) for x in shape)
    st = np.asarray(strides, dtype=np.int64)
    idx = np.ascontiguousarray(indices)
    if idx.dtype not in (np.int32, np.int64):
        raise TypeError("indices must be int32 or int64")
    pk = np.ascontiguousarray(packed).view(_raw_dtype(eb))
    S = idx.shape[0]
    if pk.shape != (S, H, V, K):
        raise ValueError("packed shape mismatch")
    base = out.ctypes.data + int(offset) * eb
    rc = lib.oracle_state_scatter(base, eb, nrows, H, V, K, _ptr(st), _ptr(idx), int(idx.dtype == np.int64),
                                  S, _ptr(pk))
    if rc != 0:
        raise RuntimeError("oracle_state_scatter: duplicate valid scatter targets (precondition)")
    return out


def kda_recurrence(q, k, v, g, beta, cu_seqlens, initial=None, scale=None, use_l2norm=True,
                   eps=L2NORM_EPS, threads=1):
    """Token-by-token gated delta rule in fp64.

    q, k, g: [T,H,K]; v: [T,H,V]; beta: [T,H]; cu_seqlens: [N+1];
    initial: [N,H,V,K] or None.  ``scale`` defaults to K**-0.5.
    Returns (out [T,H,V], final_state [N,H,V,K]) as float64 arrays.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, H, K = q.shape
    V = v.shape[2]
    N = cu.shape[0] - 1
    if k.shape != (T, H, K) or g.shape != (T, H, K) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("shape mismatch")
    if N < 0 or cu[0] != 0 or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0 and end at T")
    init = None
    if initial is not None:
        init = np.ascontiguousarray(initial, dtype=np.float64)
        if init.shape != (N, H, V, K):
            raise ValueError("initial state shape mismatch")
    if scale is None:
        scale = K ** -0.5
    out = np.zeros((T, H, V), dtype=np.float64)
    fin = np.zeros((N, H, V, K), dtype=np.float64)
    rc = lib.oracle_kda_recurrence(N, H, K, V, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   None if init is None else _ptr(init), float(scale), int(bool(use_l2norm)),
                                   float(eps), _ptr(out), _ptr(fin), int(threads))
    if rc != 0:
        raise RuntimeError("oracle_kda_recurrence failed: %d" % rc)
    return out, fin


def checkpoint_states(q, k, v, g, beta, cu_seqlens, interval, initial=None, scale=None, use_l2norm=True,
                      eps=L2NORM_EPS, threads=1):
    """States at prefix boundaries, in fp64: for sequence n (length len_n) and
    j < floor(len_n / interval), row ckpt_offsets[n] + j is the state after
    (j+1)*interval tokens of that sequence (the prefix-boundary checkpoint of
    "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对", section
    1.3; section 5.2 places prefill checkpoints at chunk boundaries).

    By definition such a state is the final state of the recurrence run over
    the prefix alone.  It is computed here by running the recurrence over
    consecutive ``interval``-token pieces, each resuming from the previous
    piece's final state (the recurrence is one token at a time, so this is
    the same arithmetic as one run over the prefix).
    Returns (states [num_ckpt,H,V,K] float64, offsets list of N+1 ints).
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    N = len(cu) - 1
    T, H, K = np.shape(q)
    V = np.shape(v)[2]
    counts = [(cu[n + 1] - cu[n]) // int(interval) for n in range(N)]
    offs = [0]
    for c in counts:
        offs.append(offs[-1] + c)
    states = np.zeros((offs[-1], H, V, K), dtype=np.float64)
    cur = np.zeros((N, H, V, K), dtype=np.float64) if initial is None else np.array(initial, dtype=np.float64)
    for j in range(max(counts, default=0)):
        sel = [n for n in range(N) if counts[n] > j]
        rows = np.concatenate([np.arange(cu[n] + j * interval, cu[n] + (j + 1) * interval) for n in sel])
        pcu = np.arange(len(sel) + 1, dtype=np.int64) * int(interval)
        _, fin = kda_recurrence(np.asarray(q)[rows], np.asarray(k)[rows], np.asarray(v)[rows], np.asarray(g)[rows],
                                np.asarray(beta)[rows], pcu, cur[sel], scale=scale, use_l2norm=use_l2norm, eps=eps,
                                threads=threads)
        for i, n in enumerate(sel):
            cur[n] = fin[i]
            states[offs[n] + j] = fin[i]
    return states, offs


def recurrent_decode(rows, indices, q, k, v, g, beta, scale=None, use_l2norm=True, eps=L2NORM_EPS):
    """One decode token per sequence against indexed state rows, in fp64.

    rows: [num_rows,H,V,K] states (element (r,h,v,c) = S[c][v]); indices: [N];
    q, k, g: [N,H,K]; v: [N,H,V]; beta: [N,H].  For every n whose index r is in
    [0, num_rows) and every head, the gated delta rule of "【轻量化复刻大模型 /
    KIMI K3】KDA 对 AI Infra 的挑战与各家应对" (section 1.1) takes one step,
        S <- (I - beta k^ k^T) Diag(exp g) S + beta k^ v^T,   o = scale S^T q^,
    written here with explicit K x K matrices; other indices are padding slots
    (zero output, no row touched).  Valid indices must be unique.
    Returns (out [N,H,V] float64, new_rows [num_rows,H,V,K] float64).
    """
    new = np.array(rows, dtype=np.float64)
    idx = [int(x) for x in np.asarray(indices).tolist()]
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    R, H, V, K = new.shape
    N = len(idx)
    if scale is None:
        scale = K ** -0.5
    valid = [r for r in idx if 0 <= r < R]
    if len(set(valid)) != len(valid):
        raise ValueError("valid state indices must be unique")
    out = np.zeros((N, H, V), dtype=np.float64)
    for n, r in enumerate(idx):
        if not 0 <= r < R:
            continue
        for h in range(H):
            kh, qh = k[n, h], q[n, h]
            if use_l2norm:
                kh = kh / np.sqrt(kh @ kh + eps)
                qh = qh / np.sqrt(qh @ qh + eps)
            S = new[r, h].T                                   # K x V
            M = (np.eye(K) - beta[n, h] * np.outer(kh, kh)) @ np.diag(np.exp(g[n, h]))
            S = M @ S + beta[n, h] * np.outer(kh, v[n, h])
            out[n, h] = scale * S.T @ qh
            new[r, h] = S.T
    return out, new


def int8_quantize(states):
    """Symmetric INT8 codes of states [S,H,V,K] with one scale per (slot, head,
    key channel): scale = (max over V of |x|) / 127, code = round-half-even of
    x / scale clamped to [-127, 127], code 0 where the scale is 0 (page
    "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对", sections
    5.3 and 6.6.2: max-abs along d_v, symmetric).  The decisions are taken in
    fp32, the precision of the stored scale.  Returns (codes int8 [S,H,V,K],
    scales float32 [S,H,1,K])."""
    x = np.asarray(states, dtype=np.float32)
    amax = np.max(np.abs(x), axis=2, keepdims=True)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale)
    codes = np.clip(np.rint(x / safe), -127, 127)
    codes = np.where(scale == 0, 0, codes).astype(np.int8)
    return codes, scale


def int8_dequantize(codes, scales):
    """code * scale in fp32 ([S,H,V,K] float32)."""
    return (np.asarray(codes, dtype=np.int8).astype(np.float32) * np.asarray(scales, dtype=np.float32)).astype(
        np.float32)


def int8_quantize_scatter(qdata, scale, indices, packed):
    """Store side of the codec: slot indices[i] <- int8_quantize(packed[i]) for
    indices in [0, num_slots); others skipped (the copy contract of page
    "vllm-ascend 的 KDA 状态复制 Triton 集成", section "数值契约", applied to the
    compressed store).  qdata [num_slots,H,V,K] int8 and scale
    [num_slots,H,1,K] float32 are updated copies; returns (qdata, scale)."""
    qd = np.array(qdata, dtype=np.int8)
    sc = np.array(scale, dtype=np.float32)
    codes, scales = int8_quantize(packed)
    idx = [int(x) for x in np.asarray(indices).tolist()]
    valid = [r for r in idx if 0 <= r < qd.shape[0]]
    if len(set(valid)) != len(valid):
        raise ValueError("valid slot indices must be unique")
    for i, r in enumerate(idx):
        if 0 <= r < qd.shape[0]:
            qd[r] = codes[i]
            sc[r] = scales[i]
    return qd, sc


def int8_dequantize_gather(qdata, scale, indices, flags=None):
    """Load side: packed[i] = int8_dequantize(slot indices[i]) when the index is
    in [0, num_slots) and flags[i] (if given) is nonzero, else zeros.
    Returns float32 [S,H,V,K]."""
    qd = np.asarray(qdata, dtype=np.int8)
    idx = [int(x) for x in np.asarray(indices).tolist()]
    out = np.zeros((len(idx),) + qd.shape[1:], dtype=np.float32)
    for i, r in enumerate(idx):
        if 0 <= r < qd.shape[0] and (flags is None or int(flags[i]) != 0):
            out[i] = int8_dequantize(qd[r], np.asarray(scale)[r])
    return out


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
