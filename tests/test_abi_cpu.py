"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/kda.h, and its host-side validation rejects bad
arguments with the documented status before any HIP call is made.  Only
calls that fail validation, or that validate and enqueue nothing (an empty
selection, N == 0), are made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from kda_recurrent_state_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from kda_recurrent_state_amd import build
        build.build()
    return _lib.load_library()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "kda.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_stages():
    names = _declared_functions()
    for n in ("kda_state_gather", "kda_state_scatter", "kda_chunk_prefill"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_python_binding_uses_the_c_names():
    import kda_recurrent_state_amd as k
    for n in ("kda_state_gather", "kda_state_scatter", "kda_chunk_prefill", "kda_chunk_prefill_workspace_size",
              "kda_recurrent_decode", "kda_ckpt_quantize_scatter", "kda_ckpt_dequantize_gather"):
        assert callable(getattr(k, n))


def _cache(dtype=0, rows=4, H=2, V=3, K=4, strides=None, data=0x1000):
    from kda_recurrent_state_amd._lib import StateCache
    d = StateCache()
    d.data = data
    d.dtype = dtype
    d.num_rows, d.H, d.V, d.K = rows, H, V, K
    st = strides or (H * V * K + 16, V * K, K, 1)
    for i in range(4):
        d.stride[i] = st[i]
    return d


def _gather(lib, d, S=0, idx=None, it=0, packed=None):
    return lib.kda_state_gather(ctypes.byref(d), idx, it, S, None, packed, None)


def test_valid_layout_empty_selection_is_ok(lib):
    assert _gather(lib, _cache()) == 0
    assert lib.kda_state_scatter(ctypes.byref(_cache()), None, 1, 0, None, None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), 2),                                   # KDA_E_DTYPE
    (dict(rows=0), 3),                                    # shape[0] > 0 required
    (dict(H=0), 3),
    (dict(strides=(100, 12, 4, 2)), 4),                   # K stride != 1
    (dict(strides=(100, 12, 5, 1)), 4),                   # V stride != K
    (dict(strides=(100, 13, 4, 1)), 4),                   # H stride != V*K
    (dict(strides=(23, 12, 4, 1)), 5),                    # rows overlap (stride0 < payload)
    (dict(data=0), 1),                                    # NULL base
])
def test_layout_rejections(lib, kw, status):
    assert _gather(lib, _cache(**kw)) == status


def test_size_one_dims_may_have_any_stride(lib):
    # H == 1 and V == 1: their strides are irrelevant to density
    assert _gather(lib, _cache(H=1, V=1, K=8, strides=(8, 999, 777, 1))) == 0
    assert _gather(lib, _cache(H=1, V=1, K=8, strides=(8, 999, 777, 2))) == 4


def test_gap_is_allowed(lib):
    assert _gather(lib, _cache(strides=(24 + 4096, 12, 4, 1))) == 0


def test_bad_selection_arguments(lib):
    d = _cache()
    assert _gather(lib, d, S=-1) == 3
    assert _gather(lib, d, S=2, idx=None, packed=0x2000) == 1
    assert _gather(lib, d, S=2, idx=0x3000, packed=None) == 1
    assert _gather(lib, d, S=0, it=7) == 2
    assert lib.kda_state_gather(None, None, 0, 0, None, None, None) == 1


def _args(**kw):
    from kda_recurrent_state_amd._lib import PrefillArgs
    a = PrefillArgs()
    a.T, a.N, a.H, a.K, a.V = 10, 1, 2, 8, 8
    a.q, a.k, a.v, a.g, a.beta, a.out = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000
    a.cu_seqlens = 0x7000
    a.qkv_dtype, a.beta_dtype, a.initial_dtype, a.final_dtype = 1, 0, 0, 0
    a.scale = 0.35
    a.use_qk_l2norm = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), 3), (dict(V=0), 3), (dict(H=0), 3), (dict(T=-1), 3), (dict(N=-1), 3),
    (dict(N=0, T=5), 3),
    (dict(K=129), 6), (dict(H=1 << 20), 6),     # H * max(K, V) above 2^22
    (dict(qkv_dtype=3), 2), (dict(beta_dtype=9), 2),
    (dict(cu_seqlens=0), 1), (dict(q=0), 1), (dict(g=0), 1), (dict(out=0), 1),
    (dict(N=4, workspace=0, workspace_bytes=0), 7),
    (dict(out=0x3000 + 4), 8),                    # partial overlap with v
    (dict(out=0x1000), 8),                        # overlaps q
    (dict(ckpt_states=0x9000, ckpt_cu=0xa000, ckpt_interval=100), 3),   # not a multiple of 64
    (dict(ckpt_states=0x9000, ckpt_cu=0xa000, ckpt_interval=0), 3),
    (dict(ckpt_states=0x9000, ckpt_cu=0xa000, ckpt_interval=64, num_ckpt=-1), 3),
    (dict(ckpt_states=0x9000, ckpt_cu=0, ckpt_interval=64), 1),
    (dict(ckpt_states=0x9000, ckpt_cu=0xa000, ckpt_interval=64, ckpt_dtype=5), 2),
])
def test_prefill_rejections(lib, kw, status):
    a = _args(**kw)
    assert lib.kda_chunk_prefill(ctypes.byref(a), None) == status


@pytest.mark.parametrize("kw", [
    dict(out=0x5000 + 40),                                    # out over beta
    dict(out=0x7000 - 100),                                   # out over cu_seqlens
    dict(initial_state=0x6000 + 64),                          # initial state under out
    dict(final_state=0x1000),                                 # final state over q
    dict(final_state=0x8000, initial_state=0x8000, final_dtype=1),      # same address, other dtype
    dict(final_state=0x8000 + 4, initial_state=0x8000),       # partial overlap
    dict(ckpt_states=0x2000, ckpt_cu=0xa000, ckpt_interval=64, num_ckpt=1),   # checkpoints over k
    dict(ckpt_states=0x9000, ckpt_cu=0x6000, ckpt_interval=64, num_ckpt=1),   # ckpt_cu under out
    dict(ckpt_states=0x9000, ckpt_cu=0xa000, ckpt_interval=64, num_ckpt=1, final_state=0x9000 + 8),  # two outputs
    dict(N=2, workspace=0x3000, workspace_bytes=1 << 20),     # workspace over v
])
def test_prefill_alias_rejections(lib, kw):
    a = _args(**kw)
    assert lib.kda_chunk_prefill(ctypes.byref(a), None) == 8


@pytest.mark.parametrize("kw", [
    dict(N=2, out=0x3000),                                    # out is exactly v
    dict(N=2, final_state=0x8000, initial_state=0x8000),      # states updated in place
])
def test_prefill_exact_aliases_pass_validation(lib, kw):
    # N = 2 needs a workspace, which is checked after aliasing: the call stops
    # there, before any launch
    a = _args(**kw)
    assert lib.kda_chunk_prefill(ctypes.byref(a), None) == 7


def test_prefill_empty_batch_is_ok(lib):
    a = _args(N=0, T=0)
    assert lib.kda_chunk_prefill(ctypes.byref(a), None) == 0


def _dargs(**kw):
    from kda_recurrent_state_amd._lib import DecodeArgs
    a = DecodeArgs()
    a.N, a.H, a.K, a.V = 3, 2, 4, 3
    a.q, a.k, a.v, a.g, a.beta, a.out = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000
    a.state_indices = 0x700000
    a.qkv_dtype, a.beta_dtype, a.index_type = 1, 0, 0
    a.scale = 0.5
    a.use_qk_l2norm = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("ckw,akw,status", [
    ({}, dict(K=8), 3),                       # args disagree with the cache
    ({}, dict(N=-1), 3),
    ({}, dict(qkv_dtype=4), 2), ({}, dict(index_type=2), 2),
    (dict(K=200), dict(K=200), 6),            # K > 128
    ({}, dict(q=0), 1), ({}, dict(state_indices=0), 1), ({}, dict(out=0), 1),
    ({}, dict(out=0x300000 + 2), 8),          # partial overlap with v
    ({}, dict(out=0x200000), 8),              # overlaps k
    ({}, dict(out=0x1000 + 8), 8),            # inside the cache span
    (dict(strides=(24, 12, 3, 2)), {}, 4),    # inner dims not dense
    (dict(strides=(10, 12, 4, 1)), {}, 5),    # rows overlap
])
def test_decode_rejections(lib, ckw, akw, status):
    d = _cache(**ckw)
    a = _dargs(**akw)
    assert lib.kda_recurrent_decode(ctypes.byref(d), ctypes.byref(a), None) == status


@pytest.mark.parametrize("akw", [
    dict(out=0x500000 + 4),                   # out over beta
    dict(out=0x700000),                       # out over state_indices
    dict(q=0x1000 + 4),                       # q inside the cache span (updated in place)
    dict(state_indices=0x1000),               # indices inside the cache span
])
def test_decode_alias_rejections(lib, akw):
    d = _cache()
    a = _dargs(**akw)
    assert lib.kda_recurrent_decode(ctypes.byref(d), ctypes.byref(a), None) == 8


def test_decode_empty_batch_is_ok(lib):
    d = _cache()
    a = _dargs(N=0, q=0, k=0, v=0, g=0, beta=0, out=0, state_indices=0)
    assert lib.kda_recurrent_decode(ctypes.byref(d), ctypes.byref(a), None) == 0
    a = _dargs(out=0x300000)                  # out may be exactly v (no launch without a GPU: N=0)
    a.N = 0
    assert lib.kda_recurrent_decode(ctypes.byref(d), ctypes.byref(a), None) == 0


def _store(**kw):
    from kda_recurrent_state_amd._lib import Int8Store
    d = Int8Store()
    d.qdata, d.scale = 0x100000, 0x900000
    d.num_slots, d.H, d.V, d.K = 4, 2, 3, 8
    d.qdata_stride0, d.scale_stride0 = 2 * 3 * 8 + 8, 2 * 8
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(num_slots=0), 3), (dict(K=0), 3), (dict(V=-1), 3),
    (dict(K=130, qdata_stride0=2 * 3 * 130, scale_stride0=260), 6),
    (dict(qdata_stride0=47), 5), (dict(scale_stride0=15), 5),
    (dict(qdata=0), 1), (dict(scale=0), 1),
    (dict(scale=0x100000 + 100), 5),             # scale inside the qdata range
])
def test_int8_store_rejections(lib, kw, status):
    d = _store(**kw)
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), 0x1000, 0, 2, 0x2000, 0, None) == status
    assert lib.kda_ckpt_dequantize_gather(ctypes.byref(d), 0x1000, 0, 2, None, 0x2000, 0, None) == status


def test_int8_alias_rejections(lib):
    d = _store()
    # quantize writes the store: packed and indices must stay outside it
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), 0x1000, 0, 2, 0x100000 + 8, 0, None) == 8
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), 0x900000, 0, 2, 0x2000, 0, None) == 8
    # dequantize writes packed: the store, indices and flags must stay outside it
    assert lib.kda_ckpt_dequantize_gather(ctypes.byref(d), 0x1000, 0, 2, None, 0x900000 - 16, 0, None) == 8
    assert lib.kda_ckpt_dequantize_gather(ctypes.byref(d), 0x1000, 0, 2, 0x2000, 0x2000, 0, None) == 8
    assert lib.kda_ckpt_dequantize_gather(ctypes.byref(d), 0x2000 + 64, 0, 2, None, 0x2000, 0, None) == 8


def test_int8_selection_arguments(lib):
    d = _store()
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), 0x1000, 2, 2, 0x2000, 0, None) == 2     # index type
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), 0x1000, 0, 2, 0x2000, 7, None) == 2     # packed dtype
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), 0x1000, 0, -1, 0x2000, 0, None) == 3
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), None, 0, 2, 0x2000, 0, None) == 1
    assert lib.kda_ckpt_dequantize_gather(ctypes.byref(d), 0x1000, 0, 2, None, None, 1, None) == 1
    # an empty selection validates and enqueues nothing
    assert lib.kda_ckpt_quantize_scatter(ctypes.byref(d), None, 0, 0, None, 1, None) == 0
    assert lib.kda_ckpt_dequantize_gather(ctypes.byref(d), None, 1, 0, None, None, 0, None) == 0


def test_checkpoint_offsets_helper():
    from kda_recurrent_state_amd.api import checkpoint_offsets
    assert checkpoint_offsets([300, 64, 0, 63, 128], 64) == [0, 4, 5, 5, 5, 7]
    assert checkpoint_offsets([1000], 192) == [0, 5]
    with pytest.raises(ValueError):
        checkpoint_offsets([10], 100)


def test_workspace_size(lib):
    assert lib.kda_chunk_prefill_workspace_size(100, 1, 32, 128, 128) == 0
    # the planning kernel's sequence order (4 B per sequence) and its kernel
    # choice (4 B after it), also when 4 N is a multiple of the 256-byte
    # rounding
    for n in (2, 64, 200, 2048):
        ws = lib.kda_chunk_prefill_workspace_size(100, n, 32, 128, 128)
        assert ws >= 4 * n + 4 and ws % 256 == 0
    # more sequences than the planning kernel orders: natural order, no plan
    assert lib.kda_chunk_prefill_workspace_size(10 ** 5, 2049, 32, 128, 128) == 0


def test_status_strings(lib):
    for s in range(10):
        assert lib.kda_status_string(s)
    assert b"KDA_OK" in lib.kda_status_string(0)


def test_binding_resolves_one_device():
    """Every call runs on the device its tensors share; host tensors and
    tensors on several devices are refused before anything is launched."""
    import types
    import torch
    from kda_recurrent_state_amd import api
    d0, d1 = torch.device("cuda", 0), torch.device("cuda", 1)
    t0 = types.SimpleNamespace(is_cuda=True, device=d0)
    t1 = types.SimpleNamespace(is_cuda=True, device=d1)
    assert api._device(t0, None, t0) == d0
    with pytest.raises(ValueError, match="one device"):
        api._device(t0, t1)
    with pytest.raises(ValueError, match="device tensors"):
        api._device(t0, torch.zeros(1))


def test_binding_refuses_without_library(tmp_path):
    from kda_recurrent_state_amd import _lib
    saved = _lib._lib
    try:
        _lib._lib = None
        with pytest.raises(ImportError):
            _lib.load_library(str(tmp_path / "missing.so"))
    finally:
        _lib._lib = saved


def _noalloc_max():
    with open(os.path.join(ROOT, "include", "kda.h")) as f:
        m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    return int(m.group(1)) << int(m.group(2))


def test_noalloc_scratch_covers_every_accepted_size(lib):
    """The static scratch of kda_chunk_prefill_noalloc holds the workspace of
    every size kda_chunk_prefill accepts.  The segment maps are the largest
    part: with N*H < 256 chains the segments after each sequence's first are
    at least lc = H*T / (256 + 0.8*N*H) tokens long, so a batch has fewer than
    1.25*N + T/lc + 1 segments, i.e. at most 2.05*N*H + 256 + H < 1040
    (segment, head) slots of 3*K*V*4 bytes (K, V <= 128 on that path) --
    195 MiB; the sequence-order plan needs 4 bytes per sequence for N <= 2048."""
    import numpy as np
    mx = _noalloc_max()
    assert 1040 * 3 * 128 * 128 * 4 + 64 * 1024 <= mx
    ts = sorted(set([int(x) for x in np.geomspace(16384, 1 << 26, 300)] + [2048 * k for k in range(8, 520)]))
    worst = 0
    for H in range(1, 256):
        for N in sorted({1, 2, 3, max(1, 255 // H), max(1, 255 // H // 2)}):
            if N * H >= 256:
                continue
            for T in ts:
                worst = max(worst, lib.kda_chunk_prefill_workspace_size(T, N, H, 128, 128))
    for N in (2, 100, 2048, 2049, 5000):
        worst = max(worst, lib.kda_chunk_prefill_workspace_size(10 ** 6, N, 32, 128, 128))
    assert 0 < worst <= mx, (worst, mx)


@pytest.mark.parametrize("kw,status", [
    (dict(K=129), 6), (dict(qkv_dtype=3), 2), (dict(q=0), 1), (dict(out=0x1000), 8),
])
def test_noalloc_rejections(lib, kw, status):
    # the same validation as kda_chunk_prefill, before any HIP call
    a = _args(**kw)
    assert lib.kda_chunk_prefill_noalloc(ctypes.byref(a), None) == status


def test_noalloc_ignores_the_workspace_fields(lib):
    # N = 4 needs a workspace; the allocation-free call takes it from its own
    # scratch, so a missing caller workspace is no error -- checked here with
    # an argument that fails afterwards (NULL cu_seqlens), before any HIP call
    a = _args(N=4, workspace=0, workspace_bytes=0, cu_seqlens=0)
    assert lib.kda_chunk_prefill_noalloc(ctypes.byref(a), None) == 1
    assert lib.kda_chunk_prefill_noalloc(None, None) == 1
    assert lib.kda_chunk_prefill_noalloc(ctypes.byref(_args(N=0, T=0)), None) == 0
