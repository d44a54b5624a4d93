"""Pins for the fp64 recurrence oracle (CPU only).

Each test checks the oracle against something other than itself: a worked
example derived by hand, the explicit-matrix unrolled form, affine
composition, split/resume, closed forms of special cases, library routines
and invariants of the map.  Sources: page "【轻量化复刻大模型 / KIMI K3】KDA 对
AI Infra 的挑战与各家应对" -- section 1.1 (S_t = M_t S_{t-1} + b_t), section
1.3 (segment maps compose affinely, associative but not commutative), section
0x03 3.2 (the state after n tokens is F_n(...F_1(S_0))), section 0x09 9.1
(S_n = M_n...M_1 S_0 + sum_i M_n...M_{i+1} b_i); and the checkpoint/resume
reading of section 1.3 (a saved boundary state continues the sequence).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunk_form
from kda_workloads import cu_from_lengths, rng

HERE = os.path.dirname(os.path.abspath(__file__))
EPS = oracle.L2NORM_EPS


def _rand_inputs(seed, lengths, H, K, V, g_scale=1.0, beta=None, init=True):
    r = rng(seed)
    T = sum(lengths)
    q = r.standard_normal((T, H, K))
    k = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    g = -np.logaddexp(0.0, r.standard_normal((T, H, K))) * g_scale
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((T, H)))) if beta is None else np.full((T, H), beta)
    s0 = r.standard_normal((len(lengths), H, V, K)) * 0.5 if init else None
    return q, k, v, g, b, cu_from_lengths(lengths), s0


def _unit(x):
    return x / np.sqrt(np.linalg.norm(x) ** 2 + EPS)


def _relerr(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


# -----------------------------------------------------------------------------
def test_hand_worked_example():
    """Values derived on paper (tests/golden/hand_example_k2v2.json)."""
    with open(os.path.join(HERE, "golden", "hand_example_k2v2.json")) as f:
        ex = json.load(f)
    toks = ex["tokens"]
    q = np.array([[t["q"]] for t in toks])
    k = np.array([[t["k"]] for t in toks])
    v = np.array([[t["v"]] for t in toks])
    g = np.array([[t["g"]] for t in toks])
    b = np.array([[t["beta"]] for t in toks])
    s0 = np.array(ex["S0_KxV"]).T[None, None]            # [1,1,V,K]
    for T, skey, okeys in ((1, "S1_KxV", ["o1"]), (2, "S2_KxV", ["o1", "o2"])):
        out, fin = oracle.kda_recurrence(q[:T], k[:T], v[:T], g[:T], b[:T], [0, T], s0, scale=1.0,
                                         use_l2norm=False)
        np.testing.assert_allclose(fin[0, 0].T, np.array(ex["expected"][skey]), rtol=0, atol=1e-14)
        for t, key in enumerate(okeys):
            np.testing.assert_allclose(out[t, 0], np.array(ex["expected"][key]), rtol=0, atol=1e-14)


# -----------------------------------------------------------------------------
@pytest.mark.parametrize("seed,lengths,K,V", [(1, [7, 13], 3, 2), (2, [40], 5, 4), (3, [1, 2, 9], 4, 3)])
def test_explicit_matrix_unrolled_form(seed, lengths, K, V):
    """S_t = M_t...M_1 S_0 + sum_i M_t...M_{i+1} b_i with explicit K x K matrices."""
    H = 2
    q, k, v, g, b, cu, s0 = _rand_inputs(seed, lengths, H, K, V)
    scale = 0.37
    out, fin = oracle.kda_recurrence(q, k, v, g, b, cu, s0, scale=scale)
    for n in range(len(lengths)):
        for h in range(H):
            S0 = s0[n, h].T                               # K x V
            Ms, bs = [], []
            for t in range(cu[n], cu[n + 1]):
                kh = _unit(k[t, h])
                Ms.append((np.eye(K) - b[t, h] * np.outer(kh, kh)) @ np.diag(np.exp(g[t, h])))
                bs.append(b[t, h] * np.outer(kh, v[t, h]))
            for tt in range(len(Ms)):
                # S_tt = (M_tt ... M_0) S0 + sum_i (M_tt ... M_{i+1}) b_i
                St = np.zeros((K, V))
                P = np.eye(K)
                for i in range(tt, -1, -1):
                    St += P @ bs[i]
                    P = P @ Ms[i]
                St += P @ S0
                o = scale * St.T @ _unit(q[cu[n] + tt, h])
                assert _relerr(out[cu[n] + tt, h], o) < 1e-12
            assert _relerr(fin[n, h].T, St) < 1e-12


# -----------------------------------------------------------------------------
def _segment_map(q, k, v, g, b, S_vk):
    """F_C(S): run one segment from state S (given [V,K]) and return the final [V,K]."""
    T = q.shape[0]
    _, fin = oracle.kda_recurrence(q, k, v, g, b, [0, T], S_vk[None, None])
    return fin[0, 0]


def _probe_affine(q, k, v, g, b, K, V):
    """Recover (M, b) of F_C(S) = M S + b by probing with zero and unit states."""
    bvec = _segment_map(q, k, v, g, b, np.zeros((V, K))).T    # K x V
    M = np.zeros((K, K))
    for c in range(K):
        E = np.zeros((K, V))
        E[c, 0] = 1.0
        M[:, c] = (_segment_map(q, k, v, g, b, E.T).T - bvec)[:, 0]
    return M, bvec


def test_affine_composition():
    K, V = 4, 3
    q, k, v, g, b, _, _ = _rand_inputs(11, [12], 1, K, V)
    c1 = slice(0, 5)
    c2 = slice(5, 12)
    M1, b1 = _probe_affine(q[c1], k[c1], v[c1], g[c1], b[c1], K, V)
    M2, b2 = _probe_affine(q[c2], k[c2], v[c2], g[c2], b[c2], K, V)
    S = rng(12).standard_normal((K, V))
    # F is affine with the same M on every column
    f1 = _segment_map(q[c1], k[c1], v[c1], g[c1], b[c1], S.T).T
    assert _relerr(f1, M1 @ S + b1) < 1e-12
    # F_C2(F_C1(S)) = M2 M1 S + M2 b1 + b2 = one pass over C1 C2
    nested = _segment_map(q[c2], k[c2], v[c2], g[c2], b[c2], f1.T).T
    composed = M2 @ M1 @ S + M2 @ b1 + b2
    whole = _segment_map(q, k, v, g, b, S.T).T
    assert _relerr(nested, composed) < 1e-12
    assert _relerr(whole, composed) < 1e-12
    # order matters: the other order gives a different state
    swapped = M1 @ M2 @ S + M1 @ b2 + b1
    assert _relerr(swapped, composed) > 1e-3


# -----------------------------------------------------------------------------
def test_split_resume_bit_identical():
    K, V, H = 5, 3, 2
    q, k, v, g, b, _, s0 = _rand_inputs(21, [50], H, K, V)
    out, fin = oracle.kda_recurrence(q, k, v, g, b, [0, 50], s0)
    for t in range(0, 51):
        o1, f1 = oracle.kda_recurrence(q[:t], k[:t], v[:t], g[:t], b[:t], [0, t], s0)
        o2, f2 = oracle.kda_recurrence(q[t:], k[t:], v[t:], g[t:], b[t:], [0, 50 - t], f1)
        assert np.array_equal(np.concatenate([o1, o2]), out)
        assert np.array_equal(f2, fin)


# -----------------------------------------------------------------------------
def test_beta_zero_is_pure_decay():
    K, V, H = 6, 4, 2
    q, k, v, g, _, cu, s0 = _rand_inputs(31, [9, 17], H, K, V)
    b = np.zeros(q.shape[:2])
    scale = 0.5
    out, fin = oracle.kda_recurrence(q, k, v, g, b, cu, s0, scale=scale)
    for n in range(2):
        for h in range(H):
            G = np.cumsum(g[cu[n]:cu[n + 1], h], axis=0)
            for j, t in enumerate(range(cu[n], cu[n + 1])):
                St = np.exp(G[j])[:, None] * s0[n, h].T
                assert _relerr(out[t, h], scale * St.T @ _unit(q[t, h])) < 1e-13
            assert _relerr(fin[n, h].T, np.exp(G[-1])[:, None] * s0[n, h].T) < 1e-13


def test_beta_zero_no_decay_is_a_matmul():
    K, V, H = 8, 5, 3
    q, k, v, _, _, cu, s0 = _rand_inputs(32, [11], H, K, V)
    g = np.zeros_like(q)
    b = np.zeros(q.shape[:2])
    out, fin = oracle.kda_recurrence(q, k, v, g, b, cu, s0, scale=1.0)
    qn = q / np.sqrt(np.linalg.norm(q, axis=-1, keepdims=True) ** 2 + EPS)
    for h in range(H):
        expect = np.matmul(qn[:, h], s0[0, h].T)
        np.testing.assert_allclose(out[:, h], expect, rtol=1e-13, atol=1e-13)
    assert np.array_equal(fin, s0)


def test_full_decay_full_write():
    """exp(g) = 0 and beta = 1: S_t = k^_t v_t^T, o_t = scale (k^_t . q^_t) v_t."""
    K, V, H = 4, 3, 2
    q, k, v, _, _, cu, s0 = _rand_inputs(33, [10], H, K, V)
    g = np.full_like(q, -1e4)
    b = np.ones(q.shape[:2])
    out, fin = oracle.kda_recurrence(q, k, v, g, b, cu, s0, scale=0.7)
    for t in range(10):
        for h in range(H):
            kh, qh = _unit(k[t, h]), _unit(q[t, h])
            np.testing.assert_allclose(out[t, h], 0.7 * (kh @ qh) * v[t, h], rtol=1e-13, atol=1e-14)
    for h in range(H):
        np.testing.assert_allclose(fin[0, h].T, np.outer(_unit(k[9, h]), v[9, h]), rtol=1e-13, atol=1e-14)


def test_one_hot_keys_replace_rows():
    """g = 0, beta = 1, k = e_i (no normalisation): row i of S becomes v_t, other rows stay."""
    K, V = 5, 3
    r = rng(34)
    S0 = r.standard_normal((K, V))
    keys = [2, 0, 2, 4]
    T = len(keys)
    k = np.zeros((T, 1, K))
    for t, i in enumerate(keys):
        k[t, 0, i] = 1.0
    v = r.standard_normal((T, 1, V))
    q = r.standard_normal((T, 1, K))
    _, fin = oracle.kda_recurrence(q, k, v, np.zeros((T, 1, K)), np.ones((T, 1)), [0, T], S0.T[None, None],
                                   use_l2norm=False)
    expect = S0.copy()
    for t, i in enumerate(keys):
        expect[i] = v[t, 0]
    np.testing.assert_allclose(fin[0, 0].T, expect, rtol=0, atol=1e-14)


def test_single_token_direct_formula():
    K, V = 6, 4
    q, k, v, g, b, _, s0 = _rand_inputs(35, [1], 1, K, V)
    out, fin = oracle.kda_recurrence(q, k, v, g, b, [0, 1], s0, scale=1.3)
    kh = _unit(k[0, 0])
    S1 = (np.eye(K) - b[0, 0] * np.outer(kh, kh)) @ np.diag(np.exp(g[0, 0])) @ s0[0, 0].T \
        + b[0, 0] * np.outer(kh, v[0, 0])
    assert _relerr(fin[0, 0].T, S1) < 1e-14
    assert _relerr(out[0, 0], 1.3 * S1.T @ _unit(q[0, 0])) < 1e-14


def test_l2norm_matches_library_norm():
    K, V, H = 7, 3, 2
    q, k, v, g, b, cu, s0 = _rand_inputs(36, [5, 8], H, K, V)
    o1, f1 = oracle.kda_recurrence(q, k, v, g, b, cu, s0, use_l2norm=True)
    qn = q / np.sqrt(np.linalg.norm(q, axis=-1, keepdims=True) ** 2 + EPS)
    kn = k / np.sqrt(np.linalg.norm(k, axis=-1, keepdims=True) ** 2 + EPS)
    o2, f2 = oracle.kda_recurrence(qn, kn, v, g, b, cu, s0, use_l2norm=False)
    assert _relerr(o1, o2) < 1e-14 and _relerr(f1, f2) < 1e-14


def test_zero_length_sequence_is_identity():
    K, V, H = 4, 4, 2
    q, k, v, g, b, _, s0 = _rand_inputs(37, [3, 0, 5], H, K, V)
    cu = cu_from_lengths([3, 0, 5])
    _, fin = oracle.kda_recurrence(q, k, v, g, b, cu, s0)
    assert np.array_equal(fin[1], s0[1])


# -----------------------------------------------------------------------------
def test_affine_in_initial_state():
    K, V, H = 5, 4, 2
    q, k, v, g, b, cu, A = _rand_inputs(41, [6, 9], H, K, V)
    B = rng(42).standard_normal(A.shape)
    a = 0.3
    oA, fA = oracle.kda_recurrence(q, k, v, g, b, cu, A)
    oB, fB = oracle.kda_recurrence(q, k, v, g, b, cu, B)
    oM, fM = oracle.kda_recurrence(q, k, v, g, b, cu, a * A + (1 - a) * B)
    assert _relerr(oM, a * oA + (1 - a) * oB) < 1e-13
    assert _relerr(fM, a * fA + (1 - a) * fB) < 1e-13


def test_linear_in_values_from_zero_state():
    K, V, H = 5, 4, 2
    q, k, v, g, b, cu, _ = _rand_inputs(43, [6, 9], H, K, V, init=False)
    o1, f1 = oracle.kda_recurrence(q, k, v, g, b, cu, None)
    o2, f2 = oracle.kda_recurrence(q, k, 2.5 * v, g, b, cu, None)
    assert _relerr(o2, 2.5 * o1) < 1e-14 and _relerr(f2, 2.5 * f1) < 1e-14


def test_state_norm_bound():
    """beta in [0,1], g <= 0: |S_t|_F <= |S_{t-1}|_F + beta_t |v_t|."""
    K, V = 6, 5
    q, k, v, g, b, _, s0 = _rand_inputs(44, [30], 1, K, V)
    S = s0
    for t in range(30):
        _, S2 = oracle.kda_recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], [0, 1], S)
        assert np.linalg.norm(S2) <= np.linalg.norm(S) + b[t, 0] * np.linalg.norm(v[t, 0]) + 1e-12
        S = S2


def test_sequences_and_heads_are_independent():
    K, V, H = 4, 3, 3
    lengths = [5, 9, 2]
    q, k, v, g, b, cu, s0 = _rand_inputs(45, lengths, H, K, V)
    out, fin = oracle.kda_recurrence(q, k, v, g, b, cu, s0)
    perm = [2, 0, 1]
    segs = [slice(cu[n], cu[n + 1]) for n in range(3)]
    cat = lambda x: np.concatenate([x[segs[p]] for p in perm])  # noqa: E731
    hp = [1, 2, 0]
    o2, f2 = oracle.kda_recurrence(cat(q)[:, hp], cat(k)[:, hp], cat(v)[:, hp], cat(g)[:, hp], cat(b)[:, hp],
                                   cu_from_lengths([lengths[p] for p in perm]), s0[perm][:, hp])
    assert np.array_equal(o2, cat(out)[:, hp])
    assert np.array_equal(f2, fin[perm][:, hp])


def test_scale_only_scales_outputs():
    K, V, H = 4, 3, 2
    q, k, v, g, b, cu, s0 = _rand_inputs(46, [7], H, K, V)
    o1, f1 = oracle.kda_recurrence(q, k, v, g, b, cu, s0, scale=1.0)
    o2, f2 = oracle.kda_recurrence(q, k, v, g, b, cu, s0, scale=0.25)
    assert np.array_equal(f1, f2)
    assert _relerr(o2, 0.25 * o1) < 1e-15


# -----------------------------------------------------------------------------
@pytest.mark.parametrize("lengths,K,V", [([1, 63, 64, 65, 130], 8, 4), ([200], 16, 16), ([64, 3], 5, 7)])
def test_chunk_form_equals_token_recurrence(lengths, K, V):
    H = 2
    q, k, v, g, b, cu, s0 = _rand_inputs(51, lengths, H, K, V)
    for init in (s0, None):
        o1, f1 = oracle.kda_recurrence(q, k, v, g, b, cu, init)
        o2, f2 = chunk_form.kda_chunked(q, k, v, g, b, cu, init)
        assert _relerr(o2, o1) < 1e-10
        assert _relerr(f2, f1) < 1e-10


def test_chunk_form_planted_mistake_is_caught():
    """A chunk form with the decay of S_in dropped must disagree with the oracle."""
    K, V = 6, 4
    q, k, v, g, b, cu, s0 = _rand_inputs(52, [100], 1, K, V)
    o1, f1 = oracle.kda_recurrence(q, k, v, g, b, cu, s0)
    o2, f2 = chunk_form.kda_chunked(q, k, v, np.zeros_like(g), b, cu, s0)
    assert _relerr(f2, f1) > 1e-2


# -----------------------------------------------------------------------------
def _explicit_state(q, k, v, g, b, t0, t1, h, S0_kv):
    """State after tokens [t0, t1) of head h by the explicit product form."""
    K = k.shape[2]
    S = S0_kv.copy()
    for t in range(t0, t1):
        kh = _unit(k[t, h])
        M = (np.eye(K) - b[t, h] * np.outer(kh, kh)) @ np.diag(np.exp(g[t, h]))
        S = M @ S + b[t, h] * np.outer(kh, v[t, h])
    return S


@pytest.mark.parametrize("interval", [3, 4])
def test_checkpoint_states_are_prefix_states(interval):
    """Checkpoint j of sequence n is the state after (j+1)*interval of its tokens
    (section 1.3's boundary state), checked against the explicit product form
    and against one run over the prefix alone; rows follow floor(len/interval)."""
    lengths = [7, 0, 4, 9, 2]
    H, K, V = 2, 3, 2
    q, k, v, g, b, cu, s0 = _rand_inputs(31, lengths, H, K, V)
    states, offs = oracle.checkpoint_states(q, k, v, g, b, cu, interval, s0)
    assert offs == list(np.cumsum([0] + [n // interval for n in lengths]))
    assert states.shape == (offs[-1], H, V, K)
    for n, ln in enumerate(lengths):
        for j in range(ln // interval):
            t1 = cu[n] + (j + 1) * interval
            for h in range(H):
                ref = _explicit_state(q, k, v, g, b, cu[n], t1, h, s0[n, h].T)
                assert _relerr(states[offs[n] + j, h].T, ref) < 1e-12
            sl = slice(cu[n], t1)
            _, fin = oracle.kda_recurrence(q[sl], k[sl], v[sl], g[sl], b[sl], [0, t1 - cu[n]], s0[n:n + 1])
            assert np.array_equal(states[offs[n] + j], fin[0])
    # a length that is a multiple of the interval: the last checkpoint is the final state
    _, fin = oracle.kda_recurrence(q, k, v, g, b, cu, s0)
    n = lengths.index(max(lengths))
    if lengths[n] % interval == 0:
        assert np.array_equal(states[offs[n + 1] - 1], fin[n])
