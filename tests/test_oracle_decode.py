"""Pins for the decode oracle (CPU only).

oracle.recurrent_decode is one step of the gated delta rule per sequence
against indexed state rows (page "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的
挑战与各家应对", section 1.1, one token).  It is checked against values worked
by hand, against the token recurrence of the C oracle (one-token sequences
from the gathered rows), against a whole sequence decoded token by token
(decode continues prefill: section 1.3's boundary state resumes the
sequence), and against the padding-slot and uniqueness rules.
"""
import json
import os

import numpy as np
import pytest

import oracle
from kda_workloads import rng

HERE = os.path.dirname(os.path.abspath(__file__))


def _tokens(seed, N, H, K, V):
    r = rng(seed)
    q = r.standard_normal((N, H, K))
    k = r.standard_normal((N, H, K))
    v = r.standard_normal((N, H, V))
    g = -np.logaddexp(0.0, r.standard_normal((N, H, K)))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((N, H))))
    return q, k, v, g, b


def test_hand_worked_example_two_decode_steps():
    """Two decode steps on a one-row cache reproduce the paper-derived values."""
    with open(os.path.join(HERE, "golden", "hand_example_k2v2.json")) as f:
        ex = json.load(f)
    rows = np.array(ex["S0_KxV"]).T[None, None]         # [1,1,V,K]
    for t, (skey, okey) in enumerate((("S1_KxV", "o1"), ("S2_KxV", "o2"))):
        tok = ex["tokens"][t]
        out, rows = oracle.recurrent_decode(rows, [0], [[tok["q"]]], [[tok["k"]]], [[tok["v"]]], [[tok["g"]]],
                                            [[tok["beta"]]], scale=1.0, use_l2norm=False)
        np.testing.assert_allclose(rows[0, 0].T, np.array(ex["expected"][skey]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(out[0, 0], np.array(ex["expected"][okey]), rtol=0, atol=1e-14)


def test_matches_token_recurrence_from_gathered_rows():
    R, N, H, K, V = 9, 5, 3, 6, 4
    rows = rng(1).standard_normal((R, H, V, K)) * 0.5
    idx = [7, 2, 0, 5, 8]
    q, k, v, g, b = _tokens(2, N, H, K, V)
    out, new = oracle.recurrent_decode(rows, idx, q, k, v, g, b, scale=0.3)
    ro, rf = oracle.kda_recurrence(q, k, v, g, b, np.arange(N + 1), rows[idx], scale=0.3)
    assert np.abs(out - ro).max() < 1e-12
    assert np.abs(new[idx] - rf).max() < 1e-12
    untouched = [r for r in range(R) if r not in idx]
    assert np.array_equal(new[untouched], rows[untouched])


def test_decoding_a_sequence_token_by_token_equals_the_recurrence():
    T, H, K, V = 12, 2, 5, 3
    q, k, v, g, b = _tokens(3, T, H, K, V)
    s0 = rng(4).standard_normal((1, H, V, K))
    ro, rf = oracle.kda_recurrence(q, k, v, g, b, [0, T], s0)
    rows = np.concatenate([np.zeros((2, H, V, K)), s0])          # the state lives in row 2
    outs = []
    for t in range(T):
        o, rows = oracle.recurrent_decode(rows, [2], q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1])
        outs.append(o[0])
    assert np.abs(np.stack(outs) - ro).max() < 1e-12
    assert np.abs(rows[2] - rf[0]).max() < 1e-12
    assert np.array_equal(rows[:2], np.zeros((2, H, V, K)))


def test_padding_slots_give_zeros_and_touch_nothing():
    R, H, K, V = 4, 2, 3, 3
    rows = rng(5).standard_normal((R, H, V, K))
    idx = [-1, 1, 4, 10 ** 9]
    q, k, v, g, b = _tokens(6, len(idx), H, K, V)
    out, new = oracle.recurrent_decode(rows, idx, q, k, v, g, b)
    assert np.all(out[[0, 2, 3]] == 0)
    assert np.any(out[1] != 0)
    assert np.array_equal(new[[0, 2, 3]], rows[[0, 2, 3]])
    assert not np.array_equal(new[1], rows[1])


def test_duplicate_valid_indices_are_rejected():
    rows = np.zeros((3, 1, 2, 2))
    q, k, v, g, b = _tokens(7, 3, 1, 2, 2)
    with pytest.raises(ValueError):
        oracle.recurrent_decode(rows, [1, -1, 1], q, k, v, g, b)
    oracle.recurrent_decode(rows, [-1, -1, 2], q, k, v, g, b)   # repeated padding is fine
