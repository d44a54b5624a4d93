"""Seeded synthetic inputs for the KDA prefill hot path.

This module only draws random inputs (and converts fp32 to bf16 bit patterns
by round-to-nearest-even); it holds none of the method's arithmetic.  The
tests, the benchmark and the oracle-side checks all take their inputs from
here, so both sides of every comparison see identical bits.

Distributions (the workloads of the KDA prefill path):

* q, k, v ~ N(0, 1), rounded to bf16 when the workload is bf16;
* g = -softplus(N(0, 1)) per (token, head, key channel), fp32, natural-log decay;
* beta = sigmoid(N(0, 1)) per (token, head), fp32;
* initial states / cache rows ~ N(0, 0.1), rounded to the cache dtype;
* cache page gaps hold a NaN sentinel bit pattern so that any stray write or
  read of a gap is visible.
"""
from __future__ import annotations

import math

import numpy as np

SENTINEL_F32 = np.uint32(0x7FA5A5A5)
SENTINEL_BF16 = np.uint16(0x7FA5)
GAP = 4096  # elements between consecutive cache rows beyond the payload


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN stays a quiet NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7F800000) == 0x7F800000
    nan &= (u & 0x007FFFFF) != 0
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------
# sequence-length recipes
# ----------------------------------------------------------------------------

def lengths_tiny():
    """Two sequences of 64 and 100 tokens."""
    return [64, 100]


def lengths_varlen(seed: int, n: int = 16, lo: int = 512, hi: int = 4096):
    """n sequences with lengths uniform on the integers [lo, hi]."""
    return [int(x) for x in rng(seed + 1000).integers(lo, hi + 1, size=n)]


def lengths_long():
    return [65536]


def lengths_e2e(seed: int, n: int = 200, lo: int = 64, hi: int = 8192):
    """n sequences with lengths log-uniform on [lo, hi], rounded to integers."""
    r = rng(seed + 2000)
    x = np.exp(r.uniform(math.log(lo), math.log(hi), size=n))
    return [int(min(hi, max(lo, round(float(v))))) for v in x]


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    if len(lengths):
        cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


# ----------------------------------------------------------------------------
# host (numpy) prefill inputs
# ----------------------------------------------------------------------------

def host_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=41, initial=True, init_dtype="f32",
                        init_std=0.1):
    """Draw a varlen prefill batch on the host.

    Returns a dict of numpy arrays.  For bf16 tensors both the bit pattern
    (``*_bits``, uint16) and its exact fp32 value are returned.
    """
    r = rng(seed)
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    N = len(lengths)
    out = {"cu_seqlens": cu, "T": T, "N": N, "H": H, "K": K, "V": V, "dtype": dtype}
    for name, last in (("q", K), ("k", K), ("v", V)):
        x = r.standard_normal((T, H, last), dtype=np.float32)
        if dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits).reshape(T, H, last)
        else:
            out[name] = x
    out["g"] = (-softplus(r.standard_normal((T, H, K), dtype=np.float32))).astype(np.float32)
    out["beta"] = sigmoid(r.standard_normal((T, H), dtype=np.float32)).astype(np.float32)
    if initial:
        s = (r.standard_normal((N, H, V, K), dtype=np.float32) * np.float32(init_std)).astype(np.float32)
        if init_dtype == "bf16":
            bits = f32_to_bf16_bits(s)
            out["initial_bits"] = bits
            out["initial"] = bf16_bits_to_f32(bits).reshape(N, H, V, K)
        else:
            out["initial"] = s
        out["init_dtype"] = init_dtype
    else:
        out["initial"] = None
        out["init_dtype"] = None
    return out


# ----------------------------------------------------------------------------
# device (torch) prefill inputs, for sizes too large to draw on the host
# ----------------------------------------------------------------------------

def device_prefill_inputs(lengths, H, K, V, dtype="bf16", seed=41, device="cuda", initial=True,
                          init_dtype="f32", init_std=0.1):
    """Same distributions as :func:`host_prefill_inputs`, drawn by torch on ``device``."""
    import torch
    import torch.nn.functional as F

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    N = len(lengths)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def normal(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    out = {"cu_seqlens": torch.from_numpy(cu).to(device), "T": T, "N": N, "H": H, "K": K, "V": V,
           "dtype": dtype, "lengths": list(lengths)}
    out["q"] = normal((T, H, K)).to(tdt)
    out["k"] = normal((T, H, K)).to(tdt)
    out["v"] = normal((T, H, V)).to(tdt)
    out["g"] = -F.softplus(normal((T, H, K)))
    out["beta"] = torch.sigmoid(normal((T, H)))
    if initial:
        s = normal((N, H, V, K)) * init_std
        out["initial"] = s.to(torch.bfloat16) if init_dtype == "bf16" else s
    else:
        out["initial"] = None
    return out


# ----------------------------------------------------------------------------
# state-cache workloads
# ----------------------------------------------------------------------------

def host_cache(num_rows, H, V, K, dtype="f32", gap=GAP, offset=0, seed=7, std=0.1):
    """A cache view inside a larger host allocation.

    Returns (backing, offset, shape, strides) with ``backing`` the raw bits of
    the whole allocation (uint32 for fp32, uint16 for bf16).  Payload elements
    are N(0, std); the storage offset prefix and every page gap hold the NaN
    sentinel.
    """
    payload = H * V * K
    stride0 = payload + gap
    total = offset + (num_rows - 1) * stride0 + payload + gap
    r = rng(seed)
    if dtype == "f32":
        backing = np.full(total, SENTINEL_F32, dtype=np.uint32)
    else:
        backing = np.full(total, SENTINEL_BF16, dtype=np.uint16)
    for row in range(num_rows):
        vals = (r.standard_normal(payload, dtype=np.float32) * np.float32(std)).astype(np.float32)
        bits = vals.view(np.uint32) if dtype == "f32" else f32_to_bf16_bits(vals)
        start = offset + row * stride0
        backing[start:start + payload] = bits
    strides = (stride0, V * K, K, 1)
    return backing, offset, (num_rows, H, V, K), strides


def copy_indices(seed, S, num_rows, n_invalid, index_dtype="int32", unique=False, huge=False):
    """S indices into [0, num_rows); exactly n_invalid of them made invalid.

    Invalid entries alternate between -1 and an out-of-range value (num_rows,
    or 2**31-1 / 2**40 when ``huge``).  With ``unique`` the valid ones are a
    seeded sample without replacement (scatter targets), else drawn with
    replacement (gather sources, duplicates allowed).
    """
    r = rng(seed)
    if unique:
        idx = r.permutation(num_rows)[:S].astype(np.int64)
    else:
        idx = r.integers(0, num_rows, size=S).astype(np.int64)
    pos = r.permutation(S)[:n_invalid]
    for j, p in enumerate(sorted(pos)):
        if j % 2 == 0:
            idx[p] = -1
        else:
            if huge:
                idx[p] = (2 ** 31 - 1) if index_dtype == "int32" else 2 ** 40
            else:
                idx[p] = num_rows
    return idx.astype(np.int32 if index_dtype == "int32" else np.int64)


def copy_flags(seed, S, n_false):
    r = rng(seed + 17)
    fl = np.ones(S, dtype=np.uint8)
    fl[r.permutation(S)[:n_false]] = 0
    return fl


def device_cache(num_rows, H, V, K, dtype="bf16", gap=GAP, offset=0, seed=7, std=0.1, device="cuda"):
    """Like :func:`host_cache` but drawn by torch on ``device`` (for multi-GiB caches).

    Returns (backing, offset, shape, strides) with ``backing`` a 1-D int32
    (fp32 cache) or int16 (bf16 cache) device tensor of raw bits.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    payload = H * V * K
    stride0 = payload + gap
    total = offset + (num_rows - 1) * stride0 + payload + gap
    if dtype == "f32":
        backing = torch.full((total,), int(SENTINEL_F32.view(np.int32)), dtype=torch.int32, device=device)
        view = backing.view(torch.float32)
    else:
        backing = torch.full((total,), int(SENTINEL_BF16.view(np.int16)), dtype=torch.int16, device=device)
        view = backing.view(torch.bfloat16)
    rows = torch.as_strided(view, (num_rows, payload), (stride0, 1), offset)
    chunk = max(1, (1 << 27) // payload)
    for r0 in range(0, num_rows, chunk):
        r1 = min(num_rows, r0 + chunk)
        vals = torch.randn((r1 - r0, payload), generator=gen, device=device, dtype=torch.float32) * std
        rows[r0:r1] = vals.to(view.dtype)
    return backing, offset, (num_rows, H, V, K), (stride0, V * K, K, 1)


def e2e_copy_indices(seed, N, num_rows=4096, high_rows=31, n_high=16):
    """Gather/scatter selection of the end-to-end prefill step.

    Gather: int32, drawn with replacement (one duplicate forced), the first
    ``n_high`` drawn from the last ``high_rows`` rows (base offset past 2^31
    elements), 10% false flags.  Scatter: N unique int32 targets, ``n_high``
    of them in the last rows.
    """
    r = rng(seed + 3)
    gidx = r.integers(0, num_rows, size=N).astype(np.int32)
    gidx[:n_high] = r.integers(num_rows - high_rows, num_rows, size=n_high)
    gidx[n_high] = gidx[0]
    flags = copy_flags(seed + 3, N, N // 10)
    sidx = np.concatenate([np.arange(num_rows - n_high, num_rows),
                           r.permutation(num_rows - high_rows)[:N - n_high]]).astype(np.int32)
    return gidx, flags, sidx
