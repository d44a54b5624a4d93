"""Host-side checks of bench.py: the multi-GPU refusal, the algorithmic byte
and flop conventions of the chunk kernel's roofline, and the percentiles."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_per_token_head():
    # q, k, v, o bf16 (256 B each), g fp32 (512 B), beta fp32 (4 B) per token-head;
    # bf16 initial + final states per (sequence, head); cu_seqlens
    assert bench.chunk_bytes_per_launch(1, 1) == 32 * 1540 + 32 * 2 * 128 * 128 * 2 + 8
    assert bench.chunk_bytes_per_launch(1000, 3) - bench.chunk_bytes_per_launch(999, 3) == 32 * 1540


def test_flop_convention():
    f = bench.chunk_flops_per_token_head()
    assert 1.38e5 < f < 1.45e5
    # the in-chunk triangles grow with the chunk length
    assert bench.chunk_flops_per_token_head(C=16) < bench.chunk_flops_per_token_head(C=64)
    # arithmetic intensity of the path (flop per algorithmic byte) is below the
    # MI355X bf16 ridge point, so the HBM roofline binds
    intensity = f / 1540
    assert intensity < bench.MFMA_BF16_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBPS * 1e9)


def test_percentiles():
    p = bench.pct([5.0, 1.0, 3.0, 2.0, 4.0])
    assert p == pytest.approx({"p10": 1.4, "p50": 3.0, "p90": 4.6})
