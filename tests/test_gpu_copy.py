"""GPU parity of kda_state_gather / kda_state_scatter against the oracle: bit-exact.

Covers fp32/bf16 caches, int32/int64 indices, every index class, flags
(none / mixed), duplicate gather indices, a storage offset, page gaps holding
a sentinel, misaligned views (narrower vector paths), graph capture/replay
with changed index and flag values, an empty selection enqueuing nothing,
and the full-size copy workloads: fp32 [1024,32,128,128] with a 4096-element
gap (S=256) and bf16 [4096,32,128,128] whose rows span more than 4 GiB.
"""
import ctypes

import numpy as np
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _dev_backing(backing):
    import torch
    if backing.dtype == np.uint32:
        return torch.from_numpy(backing.view(np.int32).copy()).cuda()
    return torch.from_numpy(backing.view(np.int16).copy()).cuda()


def _view(back_d, off, shape, strides):
    import torch
    fdt = torch.float32 if back_d.dtype == torch.int32 else torch.bfloat16
    return torch.as_strided(back_d.view(fdt), shape, strides, off)


def _raw(t):
    import torch
    if t.dtype == torch.float32:
        return t.cpu().view(torch.int32).numpy().view(np.uint32)
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


CASES = [(dt, it, off, gap) for dt in ("f32", "bf16") for it in ("int32", "int64")
         for (off, gap) in ((0, 4096), (3, 5), (1, 1))]


@pytest.mark.parametrize("dtype,itype,offset,gap", CASES)
def test_gather_scatter_small(dtype, itype, offset, gap):
    import torch
    import kda_recurrent_state_amd as kda
    print("case: small dtype=%s itype=%s offset=%d gap=%d" % (dtype, itype, offset, gap), flush=True)
    nrows, H, V, K = 9, 2, 8, 16
    backing, off, shape, strides = wl.host_cache(nrows, H, V, K, dtype=dtype, gap=gap, offset=offset, seed=21)
    big = 2 ** 31 - 1 if itype == "int32" else 2 ** 40
    gidx = np.array([3, -1, nrows, 0, 3, big, 8, 2, 5, 7], dtype=itype)
    flags = np.array([1, 1, 1, 0, 1, 1, 1, 0, 2, 1], dtype=np.uint8)
    back_d = _dev_backing(backing)
    cache = _view(back_d, off, shape, strides)
    for fl in (None, flags):
        ref = oracle.state_gather(backing, off, shape, strides, gidx, fl)
        got = kda.kda_state_gather(cache, torch.from_numpy(gidx).cuda(),
                                   None if fl is None else torch.from_numpy(fl).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(_raw(got), ref)
    sidx = np.array([4, -1, 1, nrows, big, 8, 0], dtype=itype)
    rng = np.random.default_rng(3)
    raw_t = np.uint32 if dtype == "f32" else np.uint16
    packed = rng.integers(0, 2 ** 15, size=(len(sidx), H, V, K)).astype(raw_t)
    expect = oracle.state_scatter(backing, off, shape, strides, sidx, packed)
    pk = torch.from_numpy(packed.view(np.int32 if dtype == "f32" else np.int16)).cuda()
    pk = pk.view(torch.float32 if dtype == "f32" else torch.bfloat16)
    kda.kda_state_scatter(cache, torch.from_numpy(sidx).cuda(), pk)
    torch.cuda.synchronize()
    got_back = back_d.cpu().numpy().view(raw_t)
    assert np.array_equal(got_back, expect)


def test_state_copy_object_bounds_selection():
    import torch
    import kda_recurrent_state_amd as kda
    backing, off, shape, strides = wl.host_cache(4, 1, 4, 4, dtype="f32", gap=4, offset=0, seed=22)
    cache = _view(_dev_backing(backing), off, shape, strides)
    plan = kda.KDAStateCopy(cache, max_selected=2)
    plan.gather(torch.tensor([1, 2], dtype=torch.int32, device="cuda"))
    with pytest.raises(kda.KDAError):
        plan.gather(torch.tensor([1, 2, 3], dtype=torch.int32, device="cuda"))


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    lib.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    lib.hipGraphDestroy.argtypes = [ctypes.c_void_p]
    return lib


def test_empty_selection_enqueues_nothing():
    import torch
    import kda_recurrent_state_amd as kda
    backing, off, shape, strides = wl.host_cache(4, 2, 4, 4, dtype="bf16", gap=4, offset=2, seed=23)
    cache = _view(_dev_backing(backing), off, shape, strides)
    idx = torch.zeros(0, dtype=torch.int32, device="cuda")
    packed = torch.empty((0, 2, 4, 4), dtype=torch.bfloat16, device="cuda")
    hip = _hip()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = ctypes.c_void_p()
    assert hip.hipStreamBeginCapture(ctypes.c_void_p(s.cuda_stream), 0) == 0
    kda.kda_state_gather(cache, idx, None, packed, stream=s)
    kda.kda_state_scatter(cache, idx, packed, stream=s)
    assert hip.hipStreamEndCapture(ctypes.c_void_p(s.cuda_stream), ctypes.byref(graph)) == 0
    n = ctypes.c_size_t(99)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    hip.hipGraphDestroy(graph)
    assert n.value == 0


def test_graph_replay_with_changed_indices_and_flags():
    import torch
    import kda_recurrent_state_amd as kda
    nrows, H, V, K = 8, 2, 16, 16
    backing, off, shape, strides = wl.host_cache(nrows, H, V, K, dtype="f32", gap=64, offset=8, seed=24)
    cache = _view(_dev_backing(backing), off, shape, strides)
    idx = torch.tensor([1, 2, 3, 4], dtype=torch.int64, device="cuda")
    fl = torch.ones(4, dtype=torch.uint8, device="cuda")
    packed = torch.empty((4, H, V, K), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kda.kda_state_gather(cache, idx, fl, packed)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kda.kda_state_gather(cache, idx, fl, packed)
    settings = [([1, 2, 3, 4], [1, 1, 1, 1]), ([7, -1, 0, 7], [1, 1, 0, 1]), ([5, 6, 100, 2], [0, 1, 1, 1])]
    for rep in range(2):
        for iv, fv in settings:
            idx.copy_(torch.tensor(iv, dtype=torch.int64))
            fl.copy_(torch.tensor(fv, dtype=torch.uint8))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ref = oracle.state_gather(backing, off, shape, strides, np.array(iv, np.int64), np.array(fv, np.uint8))
            assert np.array_equal(_raw(packed), ref), (rep, iv, fv)


@pytest.mark.parametrize("itype", ["int32", "int64"])
def test_full_size_fp32_cache_with_gap(itype):
    """fp32 cache [1024,32,128,128], row stride payload+4096, S=256, 5% invalid, 10% flags false."""
    import torch
    import kda_recurrent_state_amd as kda
    print("case: fp32 [1024,32,128,128] S=256 %s" % itype, flush=True)
    nrows, H, V, K = 1024, 32, 128, 128
    back_d, off, shape, strides = wl.device_cache(nrows, H, V, K, dtype="f32", gap=wl.GAP, offset=1024, seed=25)
    backing = back_d.cpu().numpy().view(np.uint32)
    cache = _view(back_d, off, shape, strides)
    S = 256
    gidx = wl.copy_indices(26, S, nrows, 13, itype, unique=False, huge=True)
    flags = wl.copy_flags(26, S, 26)
    got = kda.kda_state_gather(cache, torch.from_numpy(gidx).cuda(), torch.from_numpy(flags).cuda())
    torch.cuda.synchronize()
    ref = oracle.state_gather(backing, off, shape, strides, gidx, flags)
    assert np.array_equal(_raw(got), ref)
    del ref
    sidx = wl.copy_indices(27, S, nrows, 13, itype, unique=True, huge=True)
    packed_bits = np.random.default_rng(28).integers(0, 2 ** 31, size=(S, H, V, K), dtype=np.int64).astype(np.uint32)
    pk = torch.from_numpy(packed_bits.view(np.int32)).cuda().view(torch.float32)
    kda.kda_state_scatter(cache, torch.from_numpy(sidx).cuda(), pk)
    torch.cuda.synchronize()
    expect = oracle.state_scatter(backing, off, shape, strides, sidx, packed_bits)
    assert np.array_equal(back_d.cpu().numpy().view(np.uint32), expect)


def test_full_size_bf16_cache_beyond_4gib():
    """bf16 cache [4096,32,128,128] + gap (span > 4 GiB); int32 indices with duplicates, rows >= 4065 included."""
    import torch
    import kda_recurrent_state_amd as kda
    print("case: bf16 [4096,32,128,128] span>4GiB", flush=True)
    nrows, H, V, K = 4096, 32, 128, 128
    back_d, off, shape, strides = wl.device_cache(nrows, H, V, K, dtype="bf16", gap=wl.GAP, offset=0, seed=29)
    assert (nrows - 1) * strides[0] * 2 > 2 ** 32
    backing = back_d.cpu().numpy().view(np.uint16)
    cache = _view(back_d, off, shape, strides)
    S = 200
    r = wl.rng(30)
    gidx = r.integers(0, nrows, size=S).astype(np.int32)
    gidx[:16] = r.integers(4065, 4096, size=16)
    gidx[16] = gidx[0]                     # a guaranteed duplicate
    gidx[17] = -1
    flags = wl.copy_flags(30, S, 20)
    got = kda.kda_state_gather(cache, torch.from_numpy(gidx).cuda(), torch.from_numpy(flags).cuda())
    torch.cuda.synchronize()
    ref = oracle.state_gather(backing, off, shape, strides, gidx, flags)
    assert np.array_equal(_raw(got), ref)
    del ref
    sidx = r.permutation(nrows)[:S].astype(np.int32)
    sidx[:16] = np.arange(4080, 4096)
    sidx[16:] = np.setdiff1d(r.permutation(4065)[:S], sidx[:16])[:S - 16]
    assert len(set(sidx.tolist())) == S
    packed_bits = r.integers(0, 2 ** 15, size=(S, H, V, K)).astype(np.uint16)
    pk = torch.from_numpy(packed_bits.view(np.int16)).cuda().view(torch.bfloat16)
    kda.kda_state_scatter(cache, torch.from_numpy(sidx).cuda(), pk)
    torch.cuda.synchronize()
    expect = oracle.state_scatter(backing, off, shape, strides, sidx, packed_bits)
    assert np.array_equal(back_d.cpu().numpy().view(np.uint16), expect)
