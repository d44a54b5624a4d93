"""Full-size GPU parity on sampled outputs, in the launch configuration the
benchmark times.

* varlen: 16 sequences, lengths uniform in [512, 4096], H=32, K=V=128, bf16
  q/k/v, fp32 g/beta, fp32 initial states N(0, 0.1);
* long: one sequence of 65536 tokens, initial state gathered from a bf16
  cache row, final state written back as bf16 by scatter;
* end-to-end step: 200 sequences log-uniform in [64, 8192], bf16 cache
  [4096,32,128,128] with a row gap (span > 4 GiB), gather -> chunk -> scatter.

For each, whole (sequence, head) chains are recomputed by the oracle -- every
head of each sampled sequence -- and every chain on its own must be within
relative L2 2e-2 (the worst chain is printed); copies are compared
bit-exactly against the oracle, and cache rows and gaps that no valid target
names are checked unchanged.  The sampled sequences include the first and the
last ranks of the longest-first schedule.
"""
import numpy as np
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import REL_TOL, assert_chains, ensure_built, rel_l2, tensor_f64

pytestmark = pytest.mark.gpu
H, K, V = 32, 128, 128
ALL_HEADS = tuple(range(H))


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _chain_ref(inp, n, heads, init_f64=None):
    """Oracle on one sequence and a few heads, inputs copied from the device."""
    cu = inp["cu_seqlens"].cpu().numpy()
    s, e = int(cu[n]), int(cu[n + 1])
    hs = list(heads)
    sl = lambda t: t[s:e][:, hs].float().cpu().numpy().astype(np.float64)  # noqa: E731
    init = None if init_f64 is None else init_f64[None]
    return oracle.kda_recurrence(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]), sl(inp["beta"]),
                                 [0, e - s], init, threads=min(len(hs), oracle.default_threads())), (s, e)


def _check_sequence(inp, out, fin, n, init_f64=None, label=""):
    """All heads of sequence n against the oracle, chain by chain."""
    (ro, rf), (s, e) = _chain_ref(inp, n, ALL_HEADS, init_f64)
    go = tensor_f64(out[s:e])
    gf = tensor_f64(fin[n])
    assert_chains(go, ro, [0, e - s], gf[None], rf, label="%sseq %d (len %d): " % (label, n, e - s))
    return rf[0]


def schedule_ranks(lengths):
    """Sequence indices in the longest-first order the chunk kernel issues
    them (ties by index)."""
    return sorted(range(len(lengths)), key=lambda n: (-lengths[n], n))


def test_varlen_full_size_sampled():
    import torch
    import kda_recurrent_state_amd as kda
    lengths = wl.lengths_varlen(41)
    print("case: varlen lengths=%s" % lengths, flush=True)
    inp = wl.device_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=41, init_dtype="f32")
    out, fin = kda.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                     initial_state=inp["initial"])
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(fin).all()
    order = schedule_ranks(lengths)
    # the first two and the last two ranks of the schedule, and the first and
    # last sequence of the batch; all 32 heads of each
    sample = sorted(set(order[:2] + order[-2:] + [0, len(lengths) - 1]))
    for n in sample:
        init = inp["initial"][n].cpu().numpy().astype(np.float64)
        _check_sequence(inp, out, fin, n, init, label="rank %d " % order.index(n))


def test_long_sequence_full_size_sampled():
    import torch
    import kda_recurrent_state_amd as kda
    print("case: long T=65536", flush=True)
    inp = wl.device_prefill_inputs(wl.lengths_long(), H, K, V, dtype="bf16", seed=42, initial=False)
    back, off, shape, strides = wl.device_cache(4, H, V, K, dtype="bf16", gap=wl.GAP, offset=0, seed=43)
    cache = torch.as_strided(back.view(torch.bfloat16), shape, strides, off)
    before = back.cpu().numpy().view(np.uint16).copy()
    gidx = torch.tensor([1], dtype=torch.int32, device="cuda")
    flags = torch.tensor([1], dtype=torch.uint8, device="cuda")
    packed = kda.kda_state_gather(cache, gidx, flags)
    out, fin = kda.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                     initial_state=packed, final_dtype=torch.bfloat16)
    kda.kda_state_scatter(cache, torch.tensor([3], dtype=torch.int32, device="cuda"), fin)
    torch.cuda.synchronize()
    ref_pk = oracle.state_gather(before, off, shape, strides, np.array([1], np.int32), np.array([1], np.uint8))
    assert np.array_equal(packed.cpu().view(torch.int16).numpy().view(np.uint16), ref_pk)
    init64 = wl.bf16_bits_to_f32(ref_pk).reshape(1, H, V, K).astype(np.float64)
    # all 32 (sequence, head) chains of the run
    rf0 = _check_sequence(inp, out, fin, 0, init64[0])
    after = back.cpu().numpy().view(np.uint16)
    # row 3 now holds the bf16 final states; rows 0-2 and every gap are untouched
    row = lambda a, r: a[off + r * strides[0]: off + r * strides[0] + H * V * K]  # noqa: E731
    assert np.array_equal(row(after, 3), fin.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1))
    assert rel_l2(wl.bf16_bits_to_f32(row(after, 3)).reshape(H, V, K), rf0) <= REL_TOL
    for r in range(3):
        assert np.array_equal(row(after, r), row(before, r))
    mask = np.ones(after.shape[0], bool)
    for r in range(4):
        mask[off + r * strides[0]: off + r * strides[0] + H * V * K] = False
    assert np.array_equal(after[mask], before[mask])


def test_end_to_end_step_full_size_sampled():
    import torch
    import kda_recurrent_state_amd as kda
    seed = 41
    lengths = wl.lengths_e2e(seed)
    N = len(lengths)
    print("case: e2e N=%d T=%d" % (N, sum(lengths)), flush=True)
    inp = wl.device_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=seed, initial=False)
    back, off, shape, strides = wl.device_cache(4096, H, V, K, dtype="bf16", gap=wl.GAP, offset=0, seed=seed + 1)
    cache = torch.as_strided(back.view(torch.bfloat16), shape, strides, off)
    gidx, flags, sidx = wl.e2e_copy_indices(seed, N)
    before = back.cpu().numpy().view(np.uint16).copy()
    packed = kda.kda_state_gather(cache, torch.from_numpy(gidx).cuda(), torch.from_numpy(flags).cuda())
    out, fin = kda.kda_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                     initial_state=packed, final_dtype=torch.bfloat16)
    kda.kda_state_scatter(cache, torch.from_numpy(sidx).cuda(), fin)
    torch.cuda.synchronize()
    ref_pk = oracle.state_gather(before, off, shape, strides, gidx, flags)
    assert np.array_equal(packed.cpu().view(torch.int16).numpy().view(np.uint16), ref_pk)
    init64 = wl.bf16_bits_to_f32(ref_pk).reshape(N, H, V, K).astype(np.float64)
    after = back.cpu().numpy().view(np.uint16)
    order = schedule_ranks(lengths)
    # 16+ sequences, all 32 heads each: the first and last three ranks of
    # the longest-first schedule, four pairs of neighbouring ranks in its
    # middle, the sequences whose initial rows lie past 2^31 elements (0, 16:
    # the duplicate gather source), fresh (flag-false) requests, and the
    # middle and last sequence of the batch
    picks = order[:3] + order[-3:] + order[50:52] + order[97:99] + order[120:122] + order[150:152]
    picks += [0, 16, int(np.argmax(flags == 0)), int(np.nonzero(flags == 0)[0][-1]), N // 2, N - 1]
    sample = sorted(set(picks))
    assert len(sample) >= 16, sample
    for n in sample:
        rfn = _check_sequence(inp, out, fin, n, init64[n], label="rank %d " % order.index(n))
        # the scattered cache row of sequence n holds its final state
        r = int(sidx[n])
        rowbits = after[off + r * strides[0]: off + r * strides[0] + H * V * K]
        assert rel_l2(wl.bf16_bits_to_f32(rowbits).reshape(H, V, K), rfn) <= REL_TOL
    # rows no scatter target names, and every gap, are unchanged
    mask = np.ones(after.shape[0], bool)
    for r in sidx.tolist():
        mask[off + r * strides[0]: off + r * strides[0] + H * V * K] = False
    assert np.array_equal(after[mask], before[mask])
