"""GPU parity of kda_recurrent_decode against the fp64 decode oracle.

Outputs and the updated cache rows must be within 2e-2 relative L2 of the
oracle; every other cache row, the page gaps and the storage-offset prefix
must keep their bits.  Covers fp32/bf16 states, fp32/bf16 q/k/v, fp32/bf16
beta, int32/int64 indices with padding slots (-1, num_rows, huge), aligned
(vector) and misaligned (element) cache views, K < 16-lane slices, V above
one 128-row batch, out aliasing v, many steps in a row, prefill followed by
decode, determinism, and a full-size batch (512 sequences, H=32, K=V=128,
bf16 cache of 4096 rows spanning more than 4 GiB) checked on sampled rows.
"""
import numpy as np
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import assert_chains, bf16_tensor, ensure_built, tensor_f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _bits_to_f64(bits):
    if bits.dtype == np.uint32:
        return bits.view(np.float32).astype(np.float64)
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _dev_backing(backing):
    import torch
    if backing.dtype == np.uint32:
        return torch.from_numpy(backing.view(np.int32).copy()).cuda()
    return torch.from_numpy(backing.view(np.int16).copy()).cuda()


def _view(back_d, off, shape, strides):
    import torch
    fdt = torch.float32 if back_d.dtype == torch.int32 else torch.bfloat16
    return torch.as_strided(back_d.view(fdt), shape, strides, off)


def _rows_f64(backing, off, shape, strides):
    R, H, V, K = shape
    out = np.empty(shape, dtype=np.float64)
    for r in range(R):
        s = off + r * strides[0]
        out[r] = _bits_to_f64(backing[s:s + H * V * K]).reshape(H, V, K)
    return out


def _tokens(seed, N, H, K, V, xdt, bdt):
    """Decode-token inputs with the workload's distributions, rounded to their dtypes."""
    r = wl.rng(seed)
    q = r.standard_normal((N, H, K), dtype=np.float32)
    k = r.standard_normal((N, H, K), dtype=np.float32)
    v = r.standard_normal((N, H, V), dtype=np.float32)
    g = (-wl.softplus(r.standard_normal((N, H, K)))).astype(np.float32)
    b = wl.sigmoid(r.standard_normal((N, H))).astype(np.float32)
    host, dev = {}, {}
    for name, x, dt in (("q", q, xdt), ("k", k, xdt), ("v", v, xdt), ("beta", b, bdt)):
        if dt == "bf16":
            bits = wl.f32_to_bf16_bits(x)
            host[name] = wl.bf16_bits_to_f32(bits).astype(np.float64)
            dev[name] = bf16_tensor(bits).reshape(x.shape)
        else:
            host[name] = x.astype(np.float64)
            dev[name] = to_dev(x)
    host["g"] = g.astype(np.float64)
    dev["g"] = to_dev(g)
    return host, dev


CASES = [
    # R,  N, H,   K,   V, state, x,     beta,  index,   offset, gap
    (64, 37, 4, 128, 128, "bf16", "bf16", "f32", "int32", 0, wl.GAP),
    (64, 37, 4, 128, 128, "bf16", "bf16", "bf16", "int64", 5, 3),
    (40, 21, 2, 128, 128, "f32", "bf16", "bf16", "int64", 0, 4096),
    (40, 21, 2, 128, 128, "f32", "f32", "f32", "int32", 1, 1),
    (16, 9, 2, 64, 32, "bf16", "f32", "f32", "int32", 0, 64),
    (16, 9, 3, 48, 80, "f32", "f32", "bf16", "int64", 3, 7),
    (12, 5, 3, 128, 200, "bf16", "bf16", "f32", "int32", 0, 0),
    (8, 3, 1, 1, 1, "f32", "f32", "f32", "int32", 0, 0),
]


@pytest.mark.parametrize("R,N,H,K,V,sdt,xdt,bdt,itype,offset,gap", CASES)
def test_decode_small(R, N, H, K, V, sdt, xdt, bdt, itype, offset, gap):
    import torch
    import kda_recurrent_state_amd as kda
    print("case: decode R=%d N=%d H=%d K=%d V=%d state=%s x=%s beta=%s idx=%s off=%d gap=%d" % (
        R, N, H, K, V, sdt, xdt, bdt, itype, offset, gap), flush=True)
    backing, off, shape, strides = wl.host_cache(R, H, V, K, dtype=sdt, gap=gap, offset=offset, seed=R + N, std=0.5)
    rows0 = _rows_f64(backing, off, shape, strides)
    r = wl.rng(N * 7 + K)
    perm = r.permutation(R)[:N].astype(np.int64)
    big = 2 ** 31 - 1 if itype == "int32" else 2 ** 40
    pads = [-1, R, big]
    for i in range(0, N, 4):      # every fourth slot is padding
        perm[i] = pads[(i // 4) % 3]
    idx = perm.astype(itype)
    host, dev = _tokens(N + H, N, H, K, V, xdt, bdt)
    scale = 0.7 if K == 1 else None
    ro, rnew = oracle.recurrent_decode(rows0, idx, host["q"], host["k"], host["v"], host["g"], host["beta"],
                                       scale=scale)
    back_d = _dev_backing(backing)
    cache = _view(back_d, off, shape, strides)
    out = kda.kda_recurrent_decode(cache, torch.from_numpy(idx).cuda(), dev["q"], dev["k"], dev["v"], dev["g"],
                                   dev["beta"], scale=scale)
    torch.cuda.synchronize()
    o = tensor_f64(out)
    valid = [int(x) for x in idx if 0 <= int(x) < R]
    after = back_d.cpu().numpy().view(backing.dtype)
    rows1 = _rows_f64(after, off, shape, strides)
    # each (sequence, head): its output row and its updated state on their own
    assert_chains(o, ro, np.arange(N + 1), rows1[valid], rnew[valid])
    pad = [i for i in range(N) if not 0 <= int(idx[i]) < R]
    assert np.all(o[pad] == 0)
    # every bit outside the updated payload rows is unchanged
    mask = np.ones(backing.shape[0], dtype=bool)
    for rr in valid:
        s = off + rr * strides[0]
        mask[s:s + H * V * K] = False
    assert np.array_equal(after[mask], backing[mask])


def test_out_aliases_v_and_deterministic():
    import torch
    import kda_recurrent_state_amd as kda
    R, N, H, K, V = 32, 16, 4, 128, 128
    backing, off, shape, strides = wl.host_cache(R, H, V, K, dtype="f32", gap=64, seed=3, std=0.5)
    idx = torch.arange(3, 3 + N, dtype=torch.int32, device="cuda")
    host, dev = _tokens(9, N, H, K, V, "bf16", "f32")
    results = []
    for alias in (False, True, False):
        back_d = _dev_backing(backing)
        cache = _view(back_d, off, shape, strides)
        v = dev["v"].clone()
        o = kda.kda_recurrent_decode(cache, idx, dev["q"], dev["k"], v, dev["g"], dev["beta"],
                                     out=v if alias else None)
        torch.cuda.synchronize()
        results.append((o.clone(), back_d.clone()))
    for o, b in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(b, results[0][1])


def test_many_steps_match_the_recurrence():
    """20 decode steps of 6 sequences equal the token recurrence over 20 tokens."""
    import torch
    import kda_recurrent_state_amd as kda
    R, N, H, K, V, T = 10, 6, 2, 128, 128, 20
    backing, off, shape, strides = wl.host_cache(R, H, V, K, dtype="f32", gap=0, seed=4, std=0.5)
    rows0 = _rows_f64(backing, off, shape, strides)
    idx_np = np.array([9, 0, 4, 7, 2, 5], dtype=np.int64)
    back_d = _dev_backing(backing)
    cache = _view(back_d, off, shape, strides)
    idx = torch.from_numpy(idx_np).cuda()
    steps = [_tokens(100 + t, N, H, K, V, "bf16", "f32") for t in range(T)]
    outs = []
    for host, dev in steps:
        outs.append(tensor_f64(kda.kda_recurrent_decode(cache, idx, dev["q"], dev["k"], dev["v"], dev["g"],
                                                        dev["beta"])))
    torch.cuda.synchronize()
    # the same tokens as N sequences of T tokens each, token-major -> sequence-major
    cat = {name: np.stack([s[0][name] for s in steps], axis=1).reshape((N * T,) + steps[0][0][name].shape[1:])
           for name in ("q", "k", "v", "g", "beta")}
    ro, rf = oracle.kda_recurrence(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], np.arange(N + 1) * T,
                                   rows0[idx_np])
    got = np.stack(outs, axis=1).reshape(N * T, H, V)
    after = _rows_f64(back_d.cpu().numpy().view(np.uint32), off, shape, strides)
    assert_chains(got, ro, np.arange(N + 1) * T, after[idx_np], rf, label="20 steps: ")


def test_prefill_then_decode():
    """Prefill 130 tokens, scatter the final state into the cache, decode 3 more."""
    import torch
    import kda_recurrent_state_amd as kda
    from tests.helpers import device_inputs
    H, K, V = 4, 128, 128
    inp = wl.host_prefill_inputs([133, 70], H, K, V, dtype="bf16", seed=31, initial=False)
    lengths_pre = [130, 67]
    cu = inp["cu_seqlens"]
    pre_rows = np.concatenate([np.arange(cu[n], cu[n] + lengths_pre[n]) for n in range(2)])
    dec_rows = [[cu[n] + lengths_pre[n] + t for n in range(2)] for t in range(3)]
    d = device_inputs(inp)
    sel = torch.from_numpy(pre_rows).cuda()
    cu_pre = torch.tensor([0, 130, 197], dtype=torch.int32, device="cuda")
    _, fin = kda.kda_chunk_prefill(d["q"][sel].contiguous(), d["k"][sel].contiguous(), d["v"][sel].contiguous(),
                                   d["g"][sel].contiguous(), d["beta"][sel].contiguous(), cu_pre)
    cache = torch.zeros((5, H, V, K), dtype=torch.float32, device="cuda")
    idx = torch.tensor([3, 1], dtype=torch.int64, device="cuda")
    kda.kda_state_scatter(cache, idx, fin)
    outs = []
    for t in range(3):
        s = torch.tensor(dec_rows[t], dtype=torch.int64, device="cuda")
        outs.append(kda.kda_recurrent_decode(cache, idx, d["q"][s].contiguous(), d["k"][s].contiguous(),
                                             d["v"][s].contiguous(), d["g"][s].contiguous(),
                                             d["beta"][s].contiguous()))
    torch.cuda.synchronize()
    ro, rf = oracle.kda_recurrence(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu, None)
    # sequence-major rows of the 3 decoded tokens of each sequence
    want = np.stack([ro[dec_rows[t]] for t in range(3)], axis=1).reshape(6, H, V)
    got = np.stack([tensor_f64(o) for o in outs], axis=1).reshape(6, H, V)
    assert_chains(got, want, [0, 3, 6], tensor_f64(cache[[3, 1]]), rf, label="prefill+decode: ")


def test_full_size_sampled():
    """512 sequences, H=32, K=V=128, bf16 cache [4096,32,128,128] + gap (> 4 GiB span)."""
    import torch
    import kda_recurrent_state_amd as kda
    R, N, H, K, V = 4096, 512, 32, 128, 128
    print("case: decode full size N=%d R=%d" % (N, R), flush=True)
    back, off, shape, strides = wl.device_cache(R, H, V, K, dtype="bf16", gap=wl.GAP, offset=0, seed=51)
    cache = torch.as_strided(back.view(torch.bfloat16), shape, strides, off)
    r = wl.rng(52)
    idx_np = r.permutation(R)[:N].astype(np.int32)
    idx_np[::37] = -1                       # padding slots
    idx_np[5] = R - 1                       # the last row (highest addresses)
    host, dev = _tokens(53, N, H, K, V, "bf16", "f32")
    # 64 sequences (all heads each), the last cache row among them, and padding slots
    sample = sorted(set([5, 100, 311, 511] + list(range(0, N, 8)))) + [i for i in range(N) if idx_np[i] < 0][:2]
    pre = {i: tensor_f64(cache[int(idx_np[i])]) for i in sample if idx_np[i] >= 0}
    before = back.clone()
    out = kda.kda_recurrent_decode(cache, torch.from_numpy(idx_np).cuda(), dev["q"], dev["k"], dev["v"], dev["g"],
                                   dev["beta"])
    torch.cuda.synchronize()
    o = tensor_f64(out)
    for i in sample:
        if idx_np[i] < 0:
            assert np.all(o[i] == 0)
            continue
        ro, rnew = oracle.recurrent_decode(pre[i][None], [0], host["q"][i:i + 1], host["k"][i:i + 1],
                                           host["v"][i:i + 1], host["g"][i:i + 1], host["beta"][i:i + 1])
        assert_chains(o[i:i + 1], ro, [0, 1], tensor_f64(cache[int(idx_np[i])])[None], rnew,
                      label="seq %d row %d: " % (i, idx_np[i]))
    # rows not selected (and the gaps) keep their bits
    changed = (back != before)
    stride0 = strides[0]
    touched = torch.zeros(back.numel(), dtype=torch.bool, device="cuda")
    for rr in idx_np[idx_np >= 0].tolist():
        touched[off + rr * stride0: off + rr * stride0 + H * V * K] = True
    assert not bool((changed & ~touched).any())
    del before
