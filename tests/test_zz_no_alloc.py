"""The allocation-free prefill entry point (kda_chunk_prefill_noalloc) against
kda_chunk_prefill, through the C ABI: the same kernels on the same inputs
must give the same bits, and both must match the oracle chain by chain
(relative L2 <= 2e-2).  Calls in a row share the library's per-device
scratch: a large segment-parallel call, then a smaller one, then a plain
varlen call whose sequence-order plan lives in the same scratch."""
import numpy as np
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import assert_chains, device_inputs, ensure_built, tensor_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _both(lengths, H, K, V, seed):
    import torch
    import kda_recurrent_state_amd as kda
    print("case: no-alloc lengths=%s H=%d K=%d V=%d (workspace %d B)" % (
        lengths[:6], H, K, V, kda.kda_chunk_prefill_workspace_size(sum(lengths), len(lengths), H, K, V)),
        flush=True)
    inp = wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=seed)
    d = device_inputs(inp)
    o_ref, f_ref = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                         initial_state=d["initial"])
    out = torch.full_like(d["v"], float("nan"))
    fin = torch.full((len(lengths), H, V, K), float("nan"), dtype=torch.float32, device="cuda")
    o, f = kda.kda_chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], out=out,
                                         initial_state=d["initial"], final_state=fin)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and f.data_ptr() == fin.data_ptr()
    assert torch.equal(out, o_ref) and torch.equal(fin, f_ref)
    ro, rf = oracle.kda_recurrence(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                   inp["initial"], threads=oracle.default_threads())
    assert_chains(tensor_f64(out), ro, inp["cu_seqlens"], tensor_f64(fin), rf)


def test_noalloc_matches_prefill_on_calls_in_a_row():
    import kda_recurrent_state_amd as kda
    # segment-parallel path: segment tables and maps in the scratch
    assert kda.kda_chunk_prefill_workspace_size(20000, 1, 2, 64, 64) > 0
    _both([20000], 2, 64, 64, seed=301)
    # a smaller segment-parallel call over what the first one left behind
    assert kda.kda_chunk_prefill_workspace_size(17000, 1, 1, 32, 32) > 0
    _both([17000], 1, 32, 32, seed=302)
    # plain varlen call: the sequence-order plan in the scratch
    _both([300, 64, 129, 0, 7], 2, 128, 128, seed=303)
