"""Pins for the oracle's state gather / scatter (CPU only).

The rules come from the page "vllm-ascend 的 KDA 状态复制 Triton 集成：PR 17301
对齐的预编译 worker 生命周期方案", section "数值契约" (gather side, scatter
side, memory and addressing).  Every expectation below is built with numpy
indexing written in the test itself, on tiny caches that cover every index
class, flag state, page gaps and a storage offset.
"""
import numpy as np
import pytest

import oracle
from kda_workloads import SENTINEL_BF16, SENTINEL_F32, host_cache


def _row_bits(backing, offset, strides, idx, H, V, K):
    hh, vv, kk = np.meshgrid(np.arange(H), np.arange(V), np.arange(K), indexing="ij")
    pos = offset + idx * strides[0] + hh * strides[1] + vv * strides[2] + kk * strides[3]
    return backing[pos]


CASES = []
for dt in ("f32", "bf16"):
    for it in ("int32", "int64"):
        CASES.append((dt, it))


@pytest.mark.parametrize("dtype,itype", CASES)
def test_gather_rules(dtype, itype):
    nrows, H, V, K = 6, 2, 3, 4
    backing, off, shape, strides = host_cache(nrows, H, V, K, dtype=dtype, gap=5, offset=7, seed=3)
    big = 2 ** 31 - 1 if itype == "int32" else 2 ** 40
    idx = np.array([3, -1, nrows, 0, 3, big, 5, 2, -2 ** 31 if itype == "int32" else -2 ** 40], dtype=itype)
    for flags in (None, np.array([1, 1, 1, 0, 1, 1, 7, 0, 1], np.uint8)):
        packed = oracle.state_gather(backing, off, shape, strides, idx, flags)
        assert packed.shape == (len(idx), H, V, K)
        for i, r in enumerate(idx.astype(np.int64)):
            valid = 0 <= r < nrows
            on = flags is None or flags[i] != 0
            if valid and on:
                assert np.array_equal(packed[i], _row_bits(backing, off, strides, r, H, V, K))
            else:
                assert not packed[i].any(), "invalid / flag-false rows gather all-zero bits"


@pytest.mark.parametrize("dtype,itype", CASES)
def test_scatter_rules(dtype, itype):
    nrows, H, V, K = 6, 2, 3, 4
    backing, off, shape, strides = host_cache(nrows, H, V, K, dtype=dtype, gap=5, offset=7, seed=4)
    raw = np.uint32 if dtype == "f32" else np.uint16
    big = 2 ** 31 - 1 if itype == "int32" else 2 ** 40
    idx = np.array([4, -1, 1, nrows, big, 0], dtype=itype)
    packed = np.random.default_rng(9).integers(0, 2 ** 15, size=(len(idx), H, V, K)).astype(raw)
    out = oracle.state_scatter(backing, off, shape, strides, idx, packed)
    expect = backing.copy()
    for i, r in enumerate(idx.astype(np.int64)):
        if 0 <= r < nrows:
            hh, vv, kk = np.meshgrid(np.arange(H), np.arange(V), np.arange(K), indexing="ij")
            pos = off + r * strides[0] + hh * strides[1] + vv * strides[2] + kk * strides[3]
            expect[pos] = packed[i]
    assert np.array_equal(out, expect)
    # the storage-offset prefix and every page gap keep the sentinel
    sent = SENTINEL_F32 if dtype == "f32" else SENTINEL_BF16
    payload = H * V * K
    assert (out[:off] == sent).all()
    for r in range(nrows):
        gap = out[off + r * strides[0] + payload: off + (r + 1) * strides[0]]
        assert (gap == sent).all()


def test_scatter_ignores_flags_and_rejects_duplicates():
    nrows, H, V, K = 4, 1, 2, 2
    backing, off, shape, strides = host_cache(nrows, H, V, K, gap=3, offset=2, seed=5)
    packed = np.arange(2 * H * V * K, dtype=np.uint32).reshape(2, H, V, K) + 1
    with pytest.raises(RuntimeError):
        oracle.state_scatter(backing, off, shape, strides, np.array([1, 1], np.int32), packed)
    # duplicate invalid targets are fine (they are skipped)
    out = oracle.state_scatter(backing, off, shape, strides, np.array([-1, -1], np.int32), packed)
    assert np.array_equal(out, backing)


def test_empty_selection():
    backing, off, shape, strides = host_cache(3, 1, 2, 2, gap=1, offset=1)
    p = oracle.state_gather(backing, off, shape, strides, np.zeros(0, np.int64), None)
    assert p.shape == (0, 1, 2, 2)
    out = oracle.state_scatter(backing, off, shape, strides, np.zeros(0, np.int64), p)
    assert np.array_equal(out, backing)


def test_oracle_walks_general_strides():
    """A non-dense view (V and K strides swapped) is gathered element by element."""
    nrows, H, V, K = 3, 2, 3, 4
    base = np.arange(100 + nrows * 64, dtype=np.uint32)
    strides = (64, 12, 1, 3)   # v fastest, then k
    idx = np.array([2, 0], np.int64)
    packed = oracle.state_gather(base, 10, (nrows, H, V, K), strides, idx, None)
    view = np.lib.stride_tricks.as_strided(base[10:], shape=(nrows, H, V, K),
                                           strides=tuple(s * 4 for s in strides))
    assert np.array_equal(packed, view[idx])


def test_gather_then_scatter_round_trip():
    nrows, H, V, K = 5, 2, 2, 3
    backing, off, shape, strides = host_cache(nrows, H, V, K, dtype="bf16", gap=2, offset=3, seed=6)
    idx = np.array([4, 1, 3], np.int64)
    packed = oracle.state_gather(backing, off, shape, strides, idx, None)
    out = oracle.state_scatter(backing, off, shape, strides, idx, packed)
    assert np.array_equal(out, backing)
