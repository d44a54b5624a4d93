"""Pins for the INT8 checkpoint codec of the oracle (CPU only).

Definition (page "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对",
sections 5.3 and 6.6.2): one fp32 scale per (slot, head, key channel) equal to
the max magnitude over d_v divided by 127, symmetric int8 codes, dequantised
as code * scale.  Checked against values worked by hand (ties to even, a
zero channel), exact round trips of values on the code grid, the error
bound of rounding, per-channel independence of the scales, and the
store/load index contract.
"""
import json
import os

import numpy as np
import pytest

import oracle
from kda_workloads import rng

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_example():
    with open(os.path.join(HERE, "golden", "int8_hand_example.json")) as f:
        ex = json.load(f)
    x = np.array(ex["x"], dtype=np.float32)[None, None]          # [1,1,V,K]
    codes, scale = oracle.int8_quantize(x)
    assert scale.shape == (1, 1, 1, 3)
    assert np.array_equal(scale[0, 0, 0], np.array(ex["expected"]["scale"], dtype=np.float32))
    assert np.array_equal(codes[0, 0], np.array(ex["expected"]["codes"], dtype=np.int8))
    assert np.array_equal(oracle.int8_dequantize(codes, scale)[0, 0],
                          np.array(ex["expected"]["dequantized"], dtype=np.float32))


def test_values_on_the_code_grid_round_trip_exactly():
    r = rng(1)
    S, H, V, K = 3, 2, 16, 8
    e = r.integers(-12, 6, size=(S, H, 1, K)).astype(np.float32)
    m = r.integers(-127, 128, size=(S, H, V, K)).astype(np.float32)
    m[:, :, 0, :] = np.where(r.random((S, H, K)) < 0.5, 127.0, -127.0)   # the column max sits on the grid edge
    x = m * np.exp2(e)
    codes, scale = oracle.int8_quantize(x)
    assert np.array_equal(scale, np.exp2(e))
    assert np.array_equal(codes.astype(np.float32), m)
    assert np.array_equal(oracle.int8_dequantize(codes, scale), x)


def test_rounding_error_bound_and_code_range():
    r = rng(2)
    x = (r.standard_normal((4, 3, 32, 16)) * np.exp(r.standard_normal((4, 3, 1, 16)))).astype(np.float32)
    codes, scale = oracle.int8_quantize(x)
    assert codes.min() >= -127 and codes.max() <= 127
    amax = np.max(np.abs(x), axis=2, keepdims=True)
    # the largest magnitude of every channel maps to +-127
    at_max = np.abs(x) == amax
    assert np.all(np.abs(codes[at_max]) == 127)
    err = np.abs(oracle.int8_dequantize(codes, scale).astype(np.float64) - x)
    assert np.all(err <= scale.astype(np.float64) * (0.5 + 1e-5))


def test_scales_are_per_slot_head_and_channel():
    r = rng(3)
    x = r.standard_normal((2, 3, 8, 5)).astype(np.float32)
    _, s0 = oracle.int8_quantize(x)
    y = x.copy()
    y[1, 2, :, 4] *= 10.0                           # one channel of one head of one slot
    _, s1 = oracle.int8_quantize(y)
    changed = s0 != s1
    assert changed[1, 2, 0, 4] and changed.sum() == 1
    # the max runs over d_v only: permuting rows changes no scale
    _, s2 = oracle.int8_quantize(x[:, :, ::-1, :])
    assert np.array_equal(s0, s2)


def test_store_and_load_index_contract():
    r = rng(4)
    slots, H, V, K = 6, 2, 4, 8
    qd = r.integers(-127, 128, size=(slots, H, V, K)).astype(np.int8)
    sc = r.random((slots, H, 1, K)).astype(np.float32)
    packed = r.standard_normal((4, H, V, K)).astype(np.float32)
    idx = np.array([4, -1, slots, 0])
    qd2, sc2 = oracle.int8_quantize_scatter(qd, sc, idx, packed)
    codes, scales = oracle.int8_quantize(packed)
    assert np.array_equal(qd2[4], codes[0]) and np.array_equal(sc2[0], scales[3])
    for s in (1, 2, 3, 5):                           # untouched slots
        assert np.array_equal(qd2[s], qd[s]) and np.array_equal(sc2[s], sc[s])
    out = oracle.int8_dequantize_gather(qd2, sc2, np.array([0, 7, -3, 4, 4]), flags=np.array([1, 1, 1, 0, 2]))
    assert np.array_equal(out[0], oracle.int8_dequantize(qd2[0], sc2[0]))
    assert np.all(out[1:4] == 0)
    assert np.array_equal(out[4], oracle.int8_dequantize(qd2[4], sc2[4]))
    with pytest.raises(ValueError):
        oracle.int8_quantize_scatter(qd, sc, np.array([2, 2]), packed[:2])
