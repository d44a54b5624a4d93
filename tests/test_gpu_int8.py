"""GPU parity of the INT8 checkpoint codec against the oracle: bit-exact.

Codes and scales written by kda_ckpt_quantize_scatter, and the states
produced by kda_ckpt_dequantize_gather, must equal the oracle's bit for bit
(the quantisation decisions are fp32 on both sides).  Slots not selected and
the gaps between slots keep their bits.  Covers fp32/bf16 packed states,
int32/int64 indices with invalid entries, flags, slot gaps, vector and
element paths (K not a multiple of 8), V above 128, values next to the
rounding boundaries of the codes with scales down to the subnormal range, a
full-size store of 256 states of [32,128,128], and a prefill that resumes
from dequantised checkpoints.
"""
import numpy as np
import pytest

import kda_workloads as wl
import oracle
from tests.helpers import REL_TOL, device_inputs, ensure_built, rel_l2, tensor_f64

pytestmark = pytest.mark.gpu

Q_SENT = -101           # int8 sentinel in unused store bytes
S_SENT = np.float32(-7.25)


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _store(slots, H, V, K, qgap, sgap, seed):
    """Device store views inside larger buffers holding sentinels; returns
    (qbuf, sbuf, qdata view, scale view, host copies of both buffers)."""
    import torch
    r = wl.rng(seed)
    qs0, ss0 = H * V * K + qgap, H * K + sgap
    qbuf_h = np.full(slots * qs0, Q_SENT, dtype=np.int8)
    sbuf_h = np.full(slots * ss0, S_SENT, dtype=np.float32)
    for s in range(slots):      # previous contents of every slot
        qbuf_h[s * qs0:s * qs0 + H * V * K] = r.integers(-127, 128, size=H * V * K)
        sbuf_h[s * ss0:s * ss0 + H * K] = r.random(H * K)
    qbuf = torch.from_numpy(qbuf_h.copy()).cuda()
    sbuf = torch.from_numpy(sbuf_h.copy()).cuda()
    qd = torch.as_strided(qbuf, (slots, H, V, K), (qs0, V * K, K, 1))
    sc = torch.as_strided(sbuf, (slots, H, 1, K), (ss0, K, K, 1))
    return qbuf, sbuf, qd, sc, qbuf_h, sbuf_h, qs0, ss0


def _host_views(qbuf_h, sbuf_h, slots, H, V, K, qs0, ss0):
    qd = np.stack([qbuf_h[s * qs0:s * qs0 + H * V * K].reshape(H, V, K) for s in range(slots)])
    sc = np.stack([sbuf_h[s * ss0:s * ss0 + H * K].reshape(H, 1, K) for s in range(slots)])
    return qd, sc


def _packed(S, H, V, K, dtype, seed):
    """States with varied per-channel magnitudes; returns (host fp32 values, device tensor)."""
    import torch
    r = wl.rng(seed)
    x = (r.standard_normal((S, H, V, K)) * np.exp(r.standard_normal((S, H, 1, K)))).astype(np.float32)
    if K > 1:
        x[0, 0, :, 1] = 0.0                  # a zero channel
    if dtype == "bf16":
        bits = wl.f32_to_bf16_bits(x)
        return wl.bf16_bits_to_f32(bits), torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return x, torch.from_numpy(x).cuda()


CASES = [
    # slots, S, H,   V,   K, packed, index, qgap, sgap
    (12, 7, 3, 128, 128, "f32", "int32", 64, 8),
    (12, 7, 3, 128, 128, "bf16", "int64", 0, 0),
    (9, 5, 2, 48, 64, "f32", "int64", 8, 4),
    (9, 5, 2, 64, 40, "bf16", "int32", 3, 1),
    (6, 4, 2, 200, 128, "f32", "int32", 16, 0),
    (6, 4, 1, 1, 1, "f32", "int32", 0, 0),
]


@pytest.mark.parametrize("slots,S,H,V,K,pdt,itype,qgap,sgap", CASES)
def test_quantize_scatter_and_dequantize_gather(slots, S, H, V, K, pdt, itype, qgap, sgap):
    import torch
    import kda_recurrent_state_amd as kda
    print("case: int8 slots=%d S=%d H=%d V=%d K=%d packed=%s idx=%s gaps=%d/%d" % (
        slots, S, H, V, K, pdt, itype, qgap, sgap), flush=True)
    qbuf, sbuf, qd, sc, qbuf_h, sbuf_h, qs0, ss0 = _store(slots, H, V, K, qgap, sgap, seed=slots + V)
    x, xd = _packed(S, H, V, K, pdt, seed=S + K)
    big = 2 ** 31 - 1 if itype == "int32" else 2 ** 40
    idx = np.array(([slots - 1, -1, 0, big, 3, slots, 2] * 2)[:S], dtype=itype)
    kda.kda_ckpt_quantize_scatter(qd, sc, torch.from_numpy(idx).cuda(), xd)
    torch.cuda.synchronize()
    q0, s0 = _host_views(qbuf_h, sbuf_h, slots, H, V, K, qs0, ss0)
    rq, rs = oracle.int8_quantize_scatter(q0, s0, idx, x)
    # expected buffers: oracle slots written into the host copies, gaps untouched
    qexp, sexp = qbuf_h.copy(), sbuf_h.copy()
    for s in range(slots):
        qexp[s * qs0:s * qs0 + H * V * K] = rq[s].reshape(-1)
        sexp[s * ss0:s * ss0 + H * K] = rs[s].reshape(-1)
    assert np.array_equal(qbuf.cpu().numpy(), qexp)
    assert np.array_equal(sbuf.cpu().numpy().view(np.uint32), sexp.view(np.uint32))
    # load back, with flags, into fp32 and bf16
    gidx = np.array([0, slots - 1, -5, 2, 1, slots + 3], dtype=itype)
    flags = np.array([1, 1, 1, 0, 1, 1], dtype=np.uint8)
    want = oracle.int8_dequantize_gather(rq, rs, gidx, flags)
    for dt in (torch.float32, torch.bfloat16):
        got = kda.kda_ckpt_dequantize_gather(qd, sc, torch.from_numpy(gidx).cuda(),
                                             flags=torch.from_numpy(flags).cuda(), dtype=dt)
        torch.cuda.synchronize()
        if dt == torch.float32:
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
        else:
            assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), wl.f32_to_bf16_bits(want))


def test_full_size_store():
    """256 states of [32,128,128] fp32 into a 1024-slot store, then loaded back."""
    import torch
    import kda_recurrent_state_amd as kda
    slots, S, H, V, K = 1024, 256, 32, 128, 128
    print("case: int8 full size slots=%d S=%d" % (slots, S), flush=True)
    qd = torch.zeros((slots, H, V, K), dtype=torch.int8, device="cuda")
    sc = torch.zeros((slots, H, 1, K), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(61)
    xd = torch.randn((S, H, V, K), generator=gen, device="cuda") * 0.1
    idx = torch.from_numpy(wl.rng(62).permutation(slots)[:S].astype(np.int64)).cuda()
    kda.kda_ckpt_quantize_scatter(qd, sc, idx, xd)
    back = kda.kda_ckpt_dequantize_gather(qd, sc, idx)
    torch.cuda.synchronize()
    x = xd.cpu().numpy()
    rq, rs = oracle.int8_quantize(x)
    sel = idx.cpu().numpy()
    assert np.array_equal(qd[idx].cpu().numpy(), rq)
    assert np.array_equal(sc[idx].cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(back.cpu().numpy().view(np.uint32), oracle.int8_dequantize(rq, rs).view(np.uint32))
    rest = np.setdiff1d(np.arange(slots), sel)
    assert not bool(qd[torch.from_numpy(rest).cuda()].any())


def test_codes_near_half_integers():
    """Values within a few ulps of (k + 1/2) * scale, where the rounding of the
    quotient decides the code, and scales from the subnormal range to 2^-120
    and beyond: codes and scales bit-exact against the oracle."""
    import torch
    import kda_recurrent_state_amd as kda
    S, H, V, K = 2, 2, 128, 128
    print("case: int8 near half-integers S=%d H=%d V=%d K=%d" % (S, H, V, K), flush=True)
    r = wl.rng(71)
    amax = np.exp(r.uniform(-60.0, 60.0, size=(S, H, 1, K))).astype(np.float32)
    amax[0, 0, 0, :8] = np.float32(1e-40) * np.arange(1, 9, dtype=np.float32)  # subnormal scales
    amax[0, 1, 0, :8] = np.float32(127.0 * 2.0 ** -120) * (1 + np.arange(8, dtype=np.float32) / 64)
    sc = (amax / np.float32(127.0)).astype(np.float32)
    k = r.integers(-127, 127, size=(S, H, V, K)).astype(np.float32) + np.float32(0.5)
    x = (k * sc).astype(np.float32)
    nudge = r.integers(-3, 4, size=x.shape)
    for step in range(1, 4):
        up, dn = nudge >= step, nudge <= -step
        x[up] = np.nextafter(x[up], np.float32(np.inf))
        x[dn] = np.nextafter(x[dn], np.float32(-np.inf))
    x = np.clip(x, -amax, amax)
    x[:, :, 0, :] = amax[:, :, 0, :]     # row 0 carries the channel maximum
    slots = 4
    qd = torch.zeros((slots, H, V, K), dtype=torch.int8, device="cuda")
    scd = torch.zeros((slots, H, 1, K), dtype=torch.float32, device="cuda")
    idx = np.array([2, 0], dtype=np.int32)
    kda.kda_ckpt_quantize_scatter(qd, scd, torch.from_numpy(idx).cuda(), torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    rq, rs = oracle.int8_quantize(x)
    assert np.array_equal(qd[torch.from_numpy(idx.astype(np.int64)).cuda()].cpu().numpy(), rq)
    assert np.array_equal(scd[torch.from_numpy(idx.astype(np.int64)).cuda()].cpu().numpy().view(np.uint32),
                          rs.view(np.uint32))


def test_prefill_resumes_from_int8_checkpoints():
    """Prefill with checkpoints -> INT8 store -> dequantised states seed the
    continuation; the result stays within the parity bar of the exact run."""
    import torch
    import kda_recurrent_state_amd as kda
    H, K, V = 4, 128, 128
    inp = wl.host_prefill_inputs([256, 320], H, K, V, dtype="bf16", seed=63, initial=True)
    d = device_inputs(inp)
    offs = kda.checkpoint_offsets([256, 320], 128)        # 2 + 2 checkpoints
    ck = torch.empty((offs[-1], H, V, K), dtype=torch.float32, device="cuda")
    kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], initial_state=d["initial"],
                          ckpt_interval=128, ckpt_cu=torch.tensor(offs, dtype=torch.int32, device="cuda"),
                          ckpt_states=ck)
    qd = torch.empty((8, H, V, K), dtype=torch.int8, device="cuda")
    sc = torch.empty((8, H, 1, K), dtype=torch.float32, device="cuda")
    slots = torch.tensor([5, 1, 6, 2], dtype=torch.int32, device="cuda")
    kda.kda_ckpt_quantize_scatter(qd, sc, slots, ck)
    # resume each sequence from its first checkpoint (128 tokens in)
    s0 = kda.kda_ckpt_dequantize_gather(qd, sc, torch.tensor([5, 6], dtype=torch.int32, device="cuda"))
    cu = inp["cu_seqlens"]
    rows = np.concatenate([np.arange(cu[0] + 128, cu[1]), np.arange(cu[1] + 128, cu[2])])
    r = torch.from_numpy(rows).cuda()
    cu2 = torch.tensor([0, 128, 320], dtype=torch.int32, device="cuda")
    o2, f2 = kda.kda_chunk_prefill(d["q"][r].contiguous(), d["k"][r].contiguous(), d["v"][r].contiguous(),
                                   d["g"][r].contiguous(), d["beta"][r].contiguous(), cu2, initial_state=s0)
    torch.cuda.synchronize()
    ro, rf = oracle.kda_recurrence(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu, inp["initial"])
    e_out, e_fin = rel_l2(tensor_f64(o2), ro[rows]), rel_l2(tensor_f64(f2), rf)
    e_ck = rel_l2(tensor_f64(s0), tensor_f64(ck[[0, 2]]))
    print("  int8 resume: checkpoint relL2 %.3e, out %.3e, final %.3e" % (e_ck, e_out, e_fin), flush=True)
    assert e_ck <= REL_TOL and e_out <= REL_TOL and e_fin <= REL_TOL
