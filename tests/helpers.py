"""Shared helpers for the GPU parity tests (device plumbing and error norms)."""
from __future__ import annotations

import os

import numpy as np

REL_TOL = 2e-2   # relative L2 bar for outputs and final states (bf16 inputs, fp32 state)

# (test id, label, worst output chain, worst state chain) of every per-chain
# check in this process; tests/conftest.py prints them at the end of the run
CHAIN_RECORDS = []


def ensure_built():
    from kda_recurrent_state_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from kda_recurrent_state_amd import build
        build.build()


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def to_dev(x, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def bf16_tensor(bits, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def tensor_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_inputs(inp, dev="cuda"):
    """Move a host_prefill_inputs dict to the device with its exact bits."""
    import torch
    d = {}
    for name in ("q", "k", "v"):
        if inp["dtype"] == "bf16":
            d[name] = bf16_tensor(inp[name + "_bits"], dev).reshape(inp[name].shape)
        else:
            d[name] = to_dev(inp[name].astype(np.float32), dev)
    d["g"] = to_dev(inp["g"].astype(np.float32), dev)
    d["beta"] = to_dev(inp["beta"].astype(np.float32), dev)
    d["cu_seqlens"] = to_dev(inp["cu_seqlens"].astype(np.int32), dev)
    if inp.get("initial") is not None:
        if inp.get("init_dtype") == "bf16":
            d["initial"] = bf16_tensor(inp["initial_bits"], dev).reshape(inp["initial"].shape)
        else:
            d["initial"] = to_dev(inp["initial"].astype(np.float32), dev)
    else:
        d["initial"] = None
    del torch
    return d


def chain_errors(o, ro, cu, f=None, rf=None):
    """Relative L2 of every (sequence, head) chain.

    o, ro: outputs [T, H, V]; cu: [N+1] token offsets; f, rf: states
    [R, H, V, K] (optional; R final states, or any R rows of states, each
    (row, head) measured on its own).  Returns (worst_out, where_out, worst_final,
    where_final) with ``where`` = (sequence, head).  Empty sequences have no
    output chain; a chain whose reference is all zero is measured absolutely.
    """
    o = np.asarray(o, dtype=np.float64)
    ro = np.asarray(ro, dtype=np.float64)
    cu = [int(x) for x in np.asarray(cu).tolist()]
    H = o.shape[1]
    wo, at_o = 0.0, None
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        if e <= s:
            continue
        num = np.sqrt(((o[s:e] - ro[s:e]) ** 2).sum(axis=(0, 2)))
        den = np.sqrt((ro[s:e] ** 2).sum(axis=(0, 2)))
        err = num / np.where(den > 0, den, 1.0)
        h = int(np.argmax(err))
        if err[h] > wo or at_o is None:
            wo, at_o = float(err[h]), (n, h)
    wf, at_f = 0.0, None
    if f is not None:
        f = np.asarray(f, dtype=np.float64)
        f = f.reshape(f.shape[0], f.shape[1], -1)
        rf = np.asarray(rf, dtype=np.float64).reshape(f.shape)
        num = np.sqrt(((f - rf) ** 2).sum(axis=2))
        den = np.sqrt((rf ** 2).sum(axis=2))
        err = num / np.where(den > 0, den, 1.0)
        n, h = np.unravel_index(int(np.argmax(err)), err.shape)
        wf, at_f = float(err[n, h]), (int(n), int(h))
    return wo, at_o, wf, at_f


def assert_chains(o, ro, cu, f=None, rf=None, tol=REL_TOL, label=""):
    """Assert the whole-tensor and the worst per-(sequence, head) relative L2
    of outputs (and final states) are within ``tol``; print the worst chain."""
    eo = rel_l2(o, ro)
    wo, at_o, wf, at_f = chain_errors(o, ro, cu, f, rf)
    msg = "  %srelL2 out %.3e (worst chain %.3e at seq,head %s)" % (label, eo, wo, at_o)
    if f is not None:
        ef = rel_l2(f, rf)
        msg += " final %.3e (worst chain %.3e at %s)" % (ef, wf, at_f)
    print(msg, flush=True)
    test_id = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    CHAIN_RECORDS.append((test_id, label.strip(), wo, wf if f is not None else None))
    assert np.isfinite(np.asarray(o, dtype=np.float64)).all()
    assert eo <= tol, eo
    assert wo <= tol, (wo, at_o)
    if f is not None:
        assert np.isfinite(np.asarray(f, dtype=np.float64)).all()
        assert ef <= tol, ef
        assert wf <= tol, (wf, at_f)
    return wo, wf
