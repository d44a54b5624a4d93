"""GPU parity of kda_chunk_prefill against the fp64 oracle (relative L2 <= 2e-2).

Small cases are compared over every element; they span several chunks and
tiles, ragged tails, K != V, V-split blocks, zero-length sequences, fp32 and
bf16 I/O, vector and element-by-element loads (odd K or V, sizes that are not
a multiple of 4, unaligned tensors), no initial state, bf16 final states, out
aliasing v, final states written in place over the initial states, strong
decays that force shorter chunks, split/resume and determinism, on both
kernels for K = V = 128 (one chain per CU, or two, as the planning kernel
chooses from the lengths once there are more chains than CUs).
"""
import numpy as np
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import assert_chains, device_inputs, ensure_built, tensor_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _run(inp, final_dtype="f32", scale=None, l2norm=True, alias=False, init_override=None):
    import torch
    import kda_recurrent_state_amd as kda
    d = device_inputs(inp)
    init = d["initial"] if init_override is None else init_override
    fdt = torch.bfloat16 if final_dtype == "bf16" else torch.float32
    out = d["v"] if alias else None
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], initial_state=init,
                                 out=out, final_dtype=fdt, scale=scale, use_qk_l2norm=l2norm)
    torch.cuda.synchronize()
    return tensor_f64(o), tensor_f64(f)


def _ref(inp, scale=None, l2norm=True):
    return oracle.kda_recurrence(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                 inp["initial"], scale=scale, use_l2norm=l2norm, threads=oracle.default_threads())


def _check(inp, **kw):
    print("case: lengths=%s H=%d K=%d V=%d dtype=%s kw=%s" % (inp["cu_seqlens"].tolist()[:8], inp["H"], inp["K"],
                                                             inp["V"], inp["dtype"], kw), flush=True)
    o, f = _run(inp, **{k: v for k, v in kw.items() if k in ("final_dtype", "scale", "l2norm", "alias")})
    ro, rf = _ref(inp, scale=kw.get("scale"), l2norm=kw.get("l2norm", True))
    # whole tensors and every (sequence, head) chain on its own
    return assert_chains(o, ro, inp["cu_seqlens"], f, rf)


def test_tiny_fp32():
    inp = wl.host_prefill_inputs(wl.lengths_tiny(), 2, 32, 32, dtype="f32", seed=41)
    _check(inp)


@pytest.mark.parametrize("K,V", [(64, 32), (32, 64), (128, 64), (128, 128), (48, 80), (128, 200), (96, 40)])
def test_shapes_k_ne_v(K, V):
    inp = wl.host_prefill_inputs([70, 130], 2, K, V, dtype="bf16", seed=K * 1000 + V)
    _check(inp)


@pytest.mark.parametrize("K,V,dtype", [(30, 50, "bf16"), (33, 17, "f32"), (126, 130, "bf16")])
def test_shapes_element_loads(K, V, dtype):
    # odd K or V take the element-by-element loads; even sizes that are not a
    # multiple of 4 take the vector loads with clamped tails
    inp = wl.host_prefill_inputs([70, 130], 2, K, V, dtype=dtype, seed=K * 1000 + V + 7)
    _check(inp)


def test_unaligned_inputs_use_element_loads():
    """q, k, v and g as views one element into larger buffers (2-byte or
    4-byte aligned), which takes the element-by-element load path."""
    import torch
    import kda_recurrent_state_amd as kda
    inp = wl.host_prefill_inputs([100, 64, 37], 2, 64, 64, dtype="bf16", seed=91)
    print("case: unaligned q/k/v/g lengths=[100, 64, 37] H=2 K=V=64 bf16", flush=True)
    d = device_inputs(inp)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        view = buf[1:].view(t.shape)
        view.copy_(t)
        return view

    o, f = kda.kda_chunk_prefill(shifted(d["q"]), shifted(d["k"]), shifted(d["v"]), shifted(d["g"]), d["beta"],
                                 d["cu_seqlens"], initial_state=d["initial"])
    torch.cuda.synchronize()
    ro, rf = _ref(inp)
    assert_chains(tensor_f64(o), ro, inp["cu_seqlens"], tensor_f64(f), rf)


@pytest.mark.parametrize("lengths,H,K,V,init_dtype", [
    ([300, 64, 129, 0], 2, 128, 128, "f32"),
    ([17000], 2, 64, 64, "bf16"),             # segment-parallel path
])
def test_final_state_in_place(lengths, H, K, V, init_dtype):
    """final_state is initial_state: every (sequence, head) state is read
    before it is overwritten, so the update may run in place."""
    import torch
    import kda_recurrent_state_amd as kda
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=sum(lengths) + 3, init_dtype=init_dtype)
    print("case: in-place states lengths=%s H=%d K=%d V=%d init=%s" % (lengths, H, K, V, init_dtype), flush=True)
    d = device_inputs(inp)
    st = d["initial"].clone()
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], initial_state=st,
                                 final_state=st)
    torch.cuda.synchronize()
    assert f.data_ptr() == st.data_ptr()
    ro, rf = _ref(inp)
    assert_chains(tensor_f64(o), ro, inp["cu_seqlens"], tensor_f64(st), rf)


@pytest.mark.parametrize("lengths,H,K,V", [
    ([70, 130, 5], 2, 128, 128),   # vector loads
    ([70, 33], 2, 33, 50),         # element-by-element loads
])
def test_bf16_beta(lengths, H, K, V):
    """beta given in bf16 (its values rounded to bf16 in the oracle's input too)."""
    import torch
    import kda_recurrent_state_amd as kda
    from tests.helpers import bf16_tensor
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=sum(lengths) + K)
    bits = wl.f32_to_bf16_bits(inp["beta"].astype(np.float32))
    inp["beta"] = wl.bf16_bits_to_f32(bits).reshape(inp["beta"].shape)
    print("case: bf16 beta lengths=%s H=%d K=%d V=%d" % (lengths, H, K, V), flush=True)
    d = device_inputs(inp)
    beta = bf16_tensor(bits).reshape(inp["beta"].shape)
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], beta, d["cu_seqlens"], initial_state=d["initial"])
    torch.cuda.synchronize()
    ro, rf = _ref(inp)
    assert_chains(tensor_f64(o), ro, inp["cu_seqlens"], tensor_f64(f), rf)


def test_bf16_ragged_varlen():
    inp = wl.host_prefill_inputs([1, 17, 64, 65, 200, 333, 128], 4, 128, 128, dtype="bf16", seed=5)
    _check(inp)


def test_many_chains_take_full_value_blocks():
    # 512 chains: twice as many workgroups as CUs
    inp = wl.host_prefill_inputs([40 + 3 * i for i in range(64)], 8, 128, 128, dtype="bf16", seed=6)
    _check(inp)


# Two chains per CU (K = V = 128, bf16 q/k/v, 1024 (sequence, head) chains
# that the planning kernel puts two to a CU): 64 ragged sequences, among them
# empty, single-token and exact chunk-multiple ones, x 16 heads.
TWO_PER_CU = [0, 1, 64, 65, 128] + [40 + 3 * i for i in range(59)]


@pytest.mark.parametrize("variant", ["plain", "bf16_final_no_initial", "alias", "no_l2norm"])
def test_two_chains_per_cu(variant):
    inp = wl.host_prefill_inputs(TWO_PER_CU, 16, 128, 128, dtype="bf16", seed=61,
                                 initial=variant != "bf16_final_no_initial")
    if variant == "no_l2norm":
        # unnormalised keys need beta * |k|^2 < 2 for a stable state: shrink k
        # (by a power of two, so the bf16 bits the device gets stay exact)
        inp["k"] = inp["k"] * np.float32(1.0 / 16.0)
        inp["k_bits"] = wl.f32_to_bf16_bits(inp["k"])
        _check(inp, scale=1.0, l2norm=False)
    elif variant == "bf16_final_no_initial":
        _check(inp, final_dtype="bf16")
    else:
        _check(inp, alias=variant == "alias")


@pytest.mark.parametrize("gval", [-30.0, -1e4])
def test_two_chains_per_cu_strong_decay(gval):
    inp = wl.host_prefill_inputs(TWO_PER_CU, 16, 128, 128, dtype="bf16", seed=62)
    g = inp["g"].copy()
    g[::7, :, ::3] = gval
    inp["g"] = g
    _check(inp)


def test_two_chains_per_cu_bf16_beta():
    import torch
    import kda_recurrent_state_amd as kda
    from tests.helpers import bf16_tensor
    inp = wl.host_prefill_inputs(TWO_PER_CU, 16, 128, 128, dtype="bf16", seed=63)
    bits = wl.f32_to_bf16_bits(inp["beta"].astype(np.float32))
    inp["beta"] = wl.bf16_bits_to_f32(bits).reshape(inp["beta"].shape)
    print("case: bf16 beta, two chains per CU", flush=True)
    d = device_inputs(inp)
    beta = bf16_tensor(bits).reshape(inp["beta"].shape)
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], beta, d["cu_seqlens"], initial_state=d["initial"])
    torch.cuda.synchronize()
    ro, rf = _ref(inp)
    assert_chains(tensor_f64(o), ro, inp["cu_seqlens"], tensor_f64(f), rf)


# More (sequence, head) chains than CUs with K = V = 128 and bf16 q/k/v: the
# planning kernel picks the chunk kernel from the lengths and writes its choice
# after the sequence order in the workspace (1: two chains per CU).
@pytest.mark.parametrize("lengths,want", [
    ([130] * 12, 1),                      # 384 chains of equal length: two per CU
    ([2000] + [64] * 11, 0),              # one long sequence: its chains alone on their CUs
    ([64 * 10] * 20 + [0, 1], 1),         # 704 chains, two empty and two single-token ones
    ([3000, 2900] + [40] * 30, 0),        # 1024 chains, two long sequences
])
def test_planned_kernel_choice(lengths, want):
    import torch
    import kda_recurrent_state_amd as kda
    H = 32
    inp = wl.host_prefill_inputs(lengths, H, 128, 128, dtype="bf16", seed=64 + len(lengths))
    print("case: planned kernel choice lengths=%s... H=%d want=%d" % (lengths[:3], H, want), flush=True)
    d = device_inputs(inp)
    N, T = len(lengths), sum(lengths)
    ws = torch.full((kda.kda_chunk_prefill_workspace_size(T, N, H, 128, 128) // 4,), -1, dtype=torch.int32,
                    device=d["q"].device)
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 initial_state=d["initial"], workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[N].item()) == want
    ro, rf = _ref(inp)
    assert_chains(tensor_f64(o), ro, inp["cu_seqlens"], tensor_f64(f), rf)


def test_two_per_cu_batches_take_the_two_chains_kernel():
    """The batches the two-chains tests (here and in test_gpu_checkpoints.py)
    rely on are planned onto that kernel."""
    import torch
    import kda_recurrent_state_amd as kda
    for lengths in (TWO_PER_CU, [0, 1, 64, 65, 300] + [40 + 7 * i for i in range(59)]):
        inp = wl.host_prefill_inputs(lengths, 16, 128, 128, dtype="bf16", seed=65)
        d = device_inputs(inp)
        N, T = len(lengths), sum(lengths)
        ws = torch.full((kda.kda_chunk_prefill_workspace_size(T, N, 16, 128, 128) // 4,), -1, dtype=torch.int32,
                        device=d["q"].device)
        kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[N].item()) == 1, lengths[:6]


def test_zero_length_sequences_pass_state_through():
    inp = wl.host_prefill_inputs([5, 0, 70, 0], 2, 64, 64, dtype="bf16", seed=7)
    o, f = _run(inp)
    ro, rf = _ref(inp)
    assert_chains(o, ro, inp["cu_seqlens"], f, rf)
    assert np.array_equal(f[1], inp["initial"][1]) and np.array_equal(f[3], inp["initial"][3])


def test_no_initial_state_and_bf16_final():
    inp = wl.host_prefill_inputs([100, 300], 2, 128, 128, dtype="bf16", seed=8, initial=False)
    _check(inp, final_dtype="bf16")


@pytest.mark.parametrize("lengths,K,V,dtype", [([90], 64, 64, "f32"), ([90, 200], 128, 128, "bf16")])
def test_scale_one_and_no_l2norm(lengths, K, V, dtype):
    inp = wl.host_prefill_inputs(lengths, 2, K, V, dtype=dtype, seed=9)
    # unnormalised keys need beta * |k|^2 < 2 for a stable state: shrink k
    # (by a power of two, so bf16 bits stay exact)
    inp["k"] = inp["k"] * np.float32(1.0 / 16.0)
    if dtype == "bf16":
        inp["k_bits"] = wl.f32_to_bf16_bits(inp["k"])
    _check(inp, scale=1.0, l2norm=False)


def test_out_aliases_v():
    inp = wl.host_prefill_inputs([64, 129], 2, 128, 128, dtype="bf16", seed=10)
    _check(inp, alias=True)


def test_single_token():
    inp = wl.host_prefill_inputs([1], 1, 128, 128, dtype="bf16", seed=11)
    _check(inp)


@pytest.mark.parametrize("gval", [-30.0, -1e4])
@pytest.mark.parametrize("lengths,H,K,V", [
    ([150, 70], 2, 64, 64),                            # K <= 64 kernel
    ([150, 70], 2, 128, 64),                           # 128-column value block, V = 64
    ([150, 70], 2, 128, 128),                          # 128-column value blocks, few chains
    ([130 + 5 * (i % 7) for i in range(64)], 8, 128, 128),  # 128-column value blocks, 512 chains
])
def test_strong_decay_uses_shorter_chunks(gval, lengths, H, K, V):
    """Gate factors past 2^+-100 make a chunk retry as shorter chunks, after
    half the waves have already issued the next chunk's loads."""
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=12)
    g = inp["g"].copy()
    g[::7, :, ::3] = gval          # some channels of some tokens decay (almost) to zero
    inp["g"] = g
    _check(inp)


def test_no_decay_full_write():
    inp = wl.host_prefill_inputs([130], 2, 64, 64, dtype="bf16", seed=13)
    inp["g"] = np.zeros_like(inp["g"])
    inp["beta"] = np.ones_like(inp["beta"])
    _check(inp)


@pytest.mark.parametrize("split", [64, 100, 1])
def test_split_and_resume(split):
    import torch
    import kda_recurrent_state_amd as kda
    inp = wl.host_prefill_inputs([256], 2, 128, 128, dtype="bf16", seed=14)
    d = device_inputs(inp)
    o_all, f_all = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                         initial_state=d["initial"])
    cu1 = torch.tensor([0, split], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, 256 - split], dtype=torch.int32, device="cuda")
    s = slice(0, split)
    t = slice(split, 256)
    o1, f1 = kda.kda_chunk_prefill(d["q"][s].contiguous(), d["k"][s].contiguous(), d["v"][s].contiguous(),
                                   d["g"][s].contiguous(), d["beta"][s].contiguous(), cu1, initial_state=d["initial"])
    o2, f2 = kda.kda_chunk_prefill(d["q"][t].contiguous(), d["k"][t].contiguous(), d["v"][t].contiguous(),
                                   d["g"][t].contiguous(), d["beta"][t].contiguous(), cu2, initial_state=f1)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    assert_chains(tensor_f64(torch.cat([o1, o2])), tensor_f64(o_all), cu, tensor_f64(f2), tensor_f64(f_all),
                  label="resumed vs whole: ")
    ro, rf = _ref(inp)
    assert_chains(tensor_f64(torch.cat([o1, o2])), ro, cu, tensor_f64(f2), rf, label="resumed vs oracle: ")


@pytest.mark.parametrize("lengths,H", [([300, 77], 4), (TWO_PER_CU, 16)])
def test_deterministic(lengths, H):
    inp = wl.host_prefill_inputs(lengths, H, 128, 128, dtype="bf16", seed=15)
    o1, f1 = _run(inp)
    o2, f2 = _run(inp)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


# --- segment-parallel path: few (sequence, head) chains and T >= 16384 ----------------
@pytest.mark.parametrize("lengths,H,K,V,dtype,init", [
    ([20000], 2, 64, 64, "bf16", False),
    ([17000, 100, 0], 4, 128, 128, "bf16", True),
    ([9000, 9001], 3, 32, 48, "f32", True),
    ([17000], 2, 30, 50, "bf16", True),   # K not a multiple of 4: element loads in the map scan
    ([4096] * 4, 2, 128, 128, "bf16", True),         # splitting would not pay: whole sequences
    ([4096, 0, 4096, 4096, 4096], 2, 64, 64, "f32", True),  # whole sequences and an empty one
    # 9, 3, 2 and 1 segments: maps and a scan, one map, a first and a last
    # segment only (no map), and a first segment that is also the last
    ([17000, 5000, 3000, 100], 2, 64, 64, "bf16", True),
    ([17000, 5000, 3000, 100], 2, 128, 128, "f32", False),
])
def test_segmented_long_sequences(lengths, H, K, V, dtype, init):
    import kda_recurrent_state_amd as kda
    T = sum(lengths)
    assert len(lengths) * H < 256 and T >= 16384
    assert kda.kda_chunk_prefill_workspace_size(T, len(lengths), H, K, V) > 0   # segmentation is on
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype=dtype, seed=T + H, initial=init)
    _check(inp, final_dtype="bf16" if init else "f32")


@pytest.mark.parametrize("lengths,H,K,V", [
    ([131072], 2, 64, 64),     # 65 segments (1664 tokens, then 2048)
    ([131072], 1, 128, 128),   # the same with 128-column value blocks
])
def test_many_segments_compose(lengths, H, K, V):
    """63 segment maps composed in order: drift in the fp32 composition of
    maps built from bf16 operands would show up here first."""
    import kda_recurrent_state_amd as kda
    T = sum(lengths)
    assert kda.kda_chunk_prefill_workspace_size(T, len(lengths), H, K, V) > 0
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=T + 7 * H + K)
    _check(inp, final_dtype="f32")


def test_side_stream_with_binding_allocations():
    """The binding allocates out, the final states and the workspace on the
    current stream; a call on another stream must keep that memory from being
    handed out again while its kernels still run (segment-parallel path, whose
    workspace carries the segment maps)."""
    import torch
    import kda_recurrent_state_amd as kda
    inp = wl.host_prefill_inputs([20000], 2, 64, 64, dtype="bf16", seed=21)
    print("case: side stream, lengths=[20000] H=2 K=V=64", flush=True)
    d = device_inputs(inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, f = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 initial_state=d["initial"], stream=side)
    # the current stream takes new memory and overwrites it while the side
    # stream is still busy
    junk = [torch.full((1 << 18,), float("nan"), device="cuda") for _ in range(64)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    ro, rf = _ref(inp)
    assert_chains(tensor_f64(o), ro, inp["cu_seqlens"], tensor_f64(f), rf)
