"""FLOP and byte accounting against numbers the pages print."""
import os

import pytest

from attention_forward_fa_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def test_counted_flops_is_two_gemms_per_head():
    # Two products per head, S = Q K^T (N x d by d x N) and O = P V (N x N by
    # N x d), each 2*M*N*K; causal counts half.
    B, H, N, d = 3, 5, 96, 64
    per_head = 2 * (2 * N * N * d)
    assert acc.counted_flops(B, H, N, d, False) == B * H * per_head
    assert acc.counted_flops(B, H, N, d, True) == B * H * per_head / 2


def test_b200_table_matches_flop_convention():
    # MFU x peak x time must equal 4 * (B*H) * S^2 * D for every printed row.
    rows = _rows("b200_attention_mfu.txt")
    assert len(rows) == 4
    for name, S, D, BH, ms, mfu in rows:
        flops = acc.counted_flops(1, int(BH), int(S), int(D), False)
        implied = float(mfu) / 100.0 * 2250e12 * float(ms) * 1e-3
        assert implied == pytest.approx(flops, rel=0.01), name
        # The factor-2 convention would be off by 2x.
        assert abs(implied / (flops / 2) - 1) > 0.5


def test_b300_harness_lines_match_accounting():
    # Reading of the blog workload: fp16, non-causal, d=128, B*H=64, N=1024.
    rows = _rows("b300_blog_harness.txt")
    assert len(rows) == 9
    flops = acc.counted_flops(1, 64, 1024, 128, False)
    four_tensors = 4 * 64 * 1024 * 128 * 2
    for version, ms, tf, gbps in rows:
        t = float(ms) * 1e-3
        # ms is printed to 3 digits: allow the rounding of the last digit.
        tol = 0.0005 / float(ms) + 1e-4
        assert acc.tflops(flops, t) == pytest.approx(float(tf), rel=tol), version
        assert acc.gib_per_s(four_tensors, t) == pytest.approx(float(gbps), rel=tol), version
        # TFLOPS and GB/s are printed from the same time: their ratio is exact.
        assert float(tf) / float(gbps) == pytest.approx(
            flops / 1e12 / (four_tensors / 2 ** 30), rel=2e-4), version


def test_algorithmic_bytes():
    B, H, N, d = 2, 16, 4096, 128
    assert acc.algorithmic_bytes(B, H, N, d, "fp16") == B * H * N * (d * 8 + 4)
    assert acc.algorithmic_bytes(B, H, N, d, "fp8") == B * H * N * (d * 5 + 4)


def test_algorithmic_bytes_bwd():
    # Q, K, V, O, dO in the input type, LSE fp32 in; dQ, dK, dV and delta fp32 out.
    B, H, N, d = 2, 16, 4096, 128
    per_row = 5 * 2 * d + 4 + 3 * 4 * d + 4
    assert acc.algorithmic_bytes_bwd(B, H, N, d, "fp16") == B * H * N * per_row
    assert acc.algorithmic_bytes_bwd(B, H, N, d, "bf16") == B * H * N * (22 * d + 8)
