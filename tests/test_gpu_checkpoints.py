"""GPU parity of the chunk-boundary checkpoints of kda_chunk_prefill.

Checkpoint j of sequence n is the state after (j+1)*interval tokens of that
sequence (prefix-boundary checkpoints, page "【轻量化复刻大模型 / KIMI K3】KDA
对 AI Infra 的挑战与各家应对", sections 1.3 and 5.2).  Every checkpoint row is
compared with the fp64 oracle's state for that prefix (relative L2 <= 2e-2
for every (row, head) state on its own); outputs and final states must be bit-identical to a run without
checkpoints.  Covers ragged lengths, lengths below the interval, intervals
above the chunk size, bf16 checkpoints, shortened chunks under strong decay,
the segment-parallel path, row bounds, and scattering checkpoints into cache
rows.
"""
import numpy as np
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import REL_TOL, device_inputs, ensure_built, rel_l2, tensor_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _prefill(d, **kw):
    import torch
    import kda_recurrent_state_amd as kda
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 initial_state=d["initial"], **kw)
    torch.cuda.synchronize()
    return o, f


def _check_checkpoints(inp, interval, ckpt_dtype="f32"):
    import torch
    import kda_recurrent_state_amd as kda
    lengths = np.diff(inp["cu_seqlens"]).tolist()
    print("case: lengths=%s H=%d K=%d V=%d dtype=%s interval=%d ckpt=%s" % (
        lengths[:8], inp["H"], inp["K"], inp["V"], inp["dtype"], interval, ckpt_dtype), flush=True)
    d = device_inputs(inp)
    offs = kda.checkpoint_offsets(lengths, interval)
    cdt = torch.bfloat16 if ckpt_dtype == "bf16" else torch.float32
    ck = torch.full((offs[-1], inp["H"], inp["V"], inp["K"]), float("nan"), dtype=cdt, device="cuda")
    ck_cu = torch.tensor(offs, dtype=torch.int32, device="cuda")
    o1, f1 = _prefill(d, ckpt_interval=interval, ckpt_cu=ck_cu, ckpt_states=ck)
    o0, f0 = _prefill(d)
    assert torch.equal(o1, o0) and torch.equal(f1, f0)   # checkpoints do not change the run
    ref, roffs = oracle.checkpoint_states(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                          interval, inp["initial"], threads=oracle.default_threads())
    assert roffs == offs
    got = tensor_f64(ck)
    assert np.isfinite(got).all()
    # every (checkpoint row, head) state on its own
    H = inp["H"]
    err = np.sqrt(((got - ref) ** 2).reshape(offs[-1], H, -1).sum(axis=2))
    den = np.sqrt((ref ** 2).reshape(offs[-1], H, -1).sum(axis=2))
    err = err / np.where(den > 0, den, 1.0)
    worst = float(err.max()) if err.size else 0.0
    at = np.unravel_index(int(np.argmax(err)), err.shape) if err.size else None
    print("  %d checkpoints, worst (row, head) relL2 %.3e at %s" % (offs[-1], worst, at), flush=True)
    assert worst <= REL_TOL, (worst, at)
    return got, ref


@pytest.mark.parametrize("lengths,H,K,V,dtype,interval,ckpt_dtype", [
    ([300, 64, 129, 0, 700, 63], 2, 128, 128, "bf16", 64, "f32"),
    ([300, 64, 129, 0, 700], 3, 64, 48, "f32", 128, "bf16"),
    ([520, 1000, 191], 2, 32, 64, "bf16", 192, "f32"),
    ([0, 1, 64, 65, 300] + [40 + 7 * i for i in range(59)], 16, 128, 128, "bf16", 64, "bf16"),  # two chains per CU
])
def test_checkpoints_match_prefix_states(lengths, H, K, V, dtype, interval, ckpt_dtype):
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype=dtype, seed=sum(lengths) + interval)
    _check_checkpoints(inp, interval, ckpt_dtype)


def test_checkpoints_with_shortened_chunks():
    # strong decays force chunks shorter than 64; chunks still end on every
    # multiple of 64 tokens, so every checkpoint position is a chunk end
    inp = wl.host_prefill_inputs([300, 150], 2, 64, 64, dtype="bf16", seed=77)
    g = inp["g"].copy()
    g[5::37, :, ::3] = -1e4
    inp["g"] = g
    _check_checkpoints(inp, 64)


@pytest.mark.parametrize("lengths,H,K,V,interval", [
    ([20000], 2, 64, 64, 640),
    ([20000], 2, 64, 64, 2048),
    ([17000, 100, 0], 4, 128, 128, 1024),
    ([4096] * 4, 2, 64, 64, 1024),        # whole sequences (splitting would not pay)
    ([17000, 5000, 3000, 100], 2, 64, 64, 1024),  # 9, 3, 2 and 1 segments
])
def test_checkpoints_on_segmented_path(lengths, H, K, V, interval):
    import kda_recurrent_state_amd as kda
    assert kda.kda_chunk_prefill_workspace_size(sum(lengths), len(lengths), H, K, V) > 0  # segmentation is on
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=len(lengths) * 10 + interval)
    _check_checkpoints(inp, interval)


def test_checkpoint_rows_are_bounded():
    """Rows come from ckpt_cu and stop at num_ckpt; nothing else is written."""
    import torch
    inp = wl.host_prefill_inputs([256, 200, 320], 2, 64, 64, dtype="bf16", seed=78)
    d = device_inputs(inp)
    # natural counts are [4, 3, 5]; give sequence 0 two rows, sequence 1 none,
    # sequence 2 five rows of which only four fit below num_ckpt = 6
    ck_cu = torch.tensor([0, 2, 2, 7], dtype=torch.int32, device="cuda")
    buf = torch.full((8, 2, 64, 64), float("nan"), dtype=torch.float32, device="cuda")
    _prefill(d, ckpt_interval=64, ckpt_cu=ck_cu, ckpt_states=buf[:6])
    ref, offs = oracle.checkpoint_states(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                         64, inp["initial"])
    got = tensor_f64(buf)
    want = {0: ref[offs[0] + 0], 1: ref[offs[0] + 1], 2: ref[offs[2] + 0], 3: ref[offs[2] + 1],
            4: ref[offs[2] + 2], 5: ref[offs[2] + 3]}
    for r, w in want.items():
        assert rel_l2(got[r], w) <= REL_TOL, r
    assert np.isnan(got[6:]).all()


def test_checkpoints_scattered_into_cache_rows():
    """gather -> prefill with checkpoints -> scatter finals and checkpoints to
    cache rows by index: the rows hold the packed bits exactly."""
    import torch
    import kda_recurrent_state_amd as kda
    lengths, H, K, V = [200, 70, 333], 2, 128, 128
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=79, initial=False)
    d = device_inputs(inp)
    rows = 64
    backing, off, shape, strides = wl.device_cache(rows, H, V, K, dtype="f32", gap=wl.GAP, offset=3, seed=80)
    cache = torch.as_strided(backing.view(torch.float32), shape, strides, off)
    init_idx = torch.tensor([5, -1, 17], dtype=torch.int64, device="cuda")
    init = kda.kda_state_gather(cache, init_idx)
    offs = kda.checkpoint_offsets(lengths, 64)
    ck = torch.empty((offs[-1], H, V, K), dtype=torch.float32, device="cuda")
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], initial_state=init,
                                 ckpt_interval=64, ckpt_cu=torch.tensor(offs, dtype=torch.int32, device="cuda"),
                                 ckpt_states=ck)
    ck_idx = torch.arange(30, 30 + offs[-1], dtype=torch.int64, device="cuda")
    kda.kda_state_scatter(cache, ck_idx, ck)
    kda.kda_state_scatter(cache, torch.tensor([5, 9, 17], dtype=torch.int64, device="cuda"), f)
    torch.cuda.synchronize()
    assert torch.equal(cache[30:30 + offs[-1]], ck)
    assert torch.equal(cache[[5, 9, 17]], f)
    # the gathered initial states were the cache rows (zeros for the invalid index)
    init_h = tensor_f64(init)
    assert np.all(init_h[1] == 0)
    ref, _ = oracle.checkpoint_states(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"], 64,
                                      init_h)
    assert rel_l2(tensor_f64(cache[30:30 + offs[-1]]), ref) <= REL_TOL
    del backing
