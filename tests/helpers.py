"""Shared helpers for the GPU parity tests (device plumbing and error norms)."""
from __future__ import annotations

import os

import numpy as np

REL_TOL = 2e-2   # relative L2 bar for outputs and final states (bf16 inputs, fp32 state)


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
