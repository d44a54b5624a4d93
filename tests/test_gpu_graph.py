"""kda_chunk_prefill_noalloc captured in a HIP graph and replayed.

The allocation-free entry point is the one a caller under graph capture can
use.  Each case captures one call (the planning kernel, and for K = V = 128
bf16 batches with more chains than CUs both chunk kernels, one of which
returns at once; or the segment-parallel passes), then replays the graph with
two input sets copied in turn into the captured buffers, with eager calls and
synchronisations between the replays.  Every replay must give the bits of an
eager call on the same inputs (the kernels are deterministic), and the eager
results match the oracle chain by chain.
"""
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import assert_chains, device_inputs, ensure_built, tensor_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


@pytest.mark.parametrize("lengths,H,K,V", [
    ([130] * 12, 32, 128, 128),          # 384 chains of equal length: two chains per CU
    ([2000] + [64] * 11, 32, 128, 128),  # skewed: one chain per CU
    ([300, 77, 0, 5], 4, 128, 128),      # fewer chains than CUs
    ([17000], 2, 64, 64),                # segment-parallel passes and the map scan
])
def test_prefill_graph_replays(lengths, H, K, V):
    import torch
    import kda_recurrent_state_amd as kda
    print("case: graph replay lengths=%s H=%d K=%d V=%d" % (lengths[:4], H, K, V), flush=True)
    N = len(lengths)
    inps = [wl.host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=400 + i) for i in range(2)]
    devs = [device_inputs(x) for x in inps]
    names = ("q", "k", "v", "g", "beta", "cu_seqlens", "initial")

    def call(d, out, fin):
        kda.kda_chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], out=out,
                                      initial_state=d["initial"], final_state=fin)

    # eager results of both input sets
    refs = []
    for d in devs:
        o = torch.empty_like(d["v"])
        f = torch.empty((N, H, V, K), dtype=torch.float32, device="cuda")
        call(d, o, f)
        refs.append((o, f))
    torch.cuda.synchronize()
    for x, (o, f) in zip(inps, refs):
        ro, rf = oracle.kda_recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], x["initial"],
                                       threads=oracle.default_threads())
        assert_chains(tensor_f64(o), ro, x["cu_seqlens"], tensor_f64(f), rf)

    # captured buffers, holding input set 0 at capture time
    cap = {n: devs[0][n].clone() for n in names}
    out = torch.full_like(cap["v"], float("nan"))
    fin = torch.full((N, H, V, K), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(cap, out, fin)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(cap, out, fin)
    for rep in range(2):
        for i in (1, 0):
            for n in names:
                cap[n].copy_(devs[i][n])
            out.fill_(float("nan"))
            fin.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, refs[i][0]) and torch.equal(fin, refs[i][1]), (rep, i)
            # eager work on the same scratch between replays
            o2 = torch.empty_like(out)
            f2 = torch.empty_like(fin)
            call(devs[1 - i], o2, f2)
            torch.cuda.synchronize()
            assert torch.equal(o2, refs[1 - i][0]) and torch.equal(f2, refs[1 - i][1]), (rep, i, "eager")
