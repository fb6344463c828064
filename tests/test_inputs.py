"""The seeded input generator (shared by the oracle side and the HIP side)."""
import numpy as np
import torch

from attention_forward_fa_amd import inputs
from oracle import attention as A


def test_seeded_and_deterministic():
    a = inputs.draw(1, 2, 64, 64, "fp16", False, seed=11)
    b = inputs.draw(1, 2, 64, 64, "fp16", False, seed=11)
    c = inputs.draw(1, 2, 64, 64, "fp16", False, seed=12)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert not np.array_equal(a.q, c.q)
    assert a.q.dtype == np.uint16 and a.q.shape == (1, 2, 64, 64)


def test_draw_order_and_rne_casts():
    g = torch.Generator().manual_seed(3)
    q = torch.randn((1, 1, 16, 64), generator=g)
    k = torch.randn((1, 1, 16, 64), generator=g)
    v = torch.randn((1, 1, 16, 64), generator=g)
    x = inputs.draw(1, 1, 16, 64, "bf16", True, seed=3)
    for t, bits in ((q, x.q), (k, x.k), (v, x.v)):
        ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(bits, ref)
    h = inputs.draw(1, 1, 16, 64, "fp16", False, seed=3)
    assert np.array_equal(A.decode_fp16(h.q), q.numpy().astype(np.float16).astype(np.float64))
    assert x.causal and x.scale == float(np.float32(1 / 8))


def test_fp8_per_head_quantization():
    x = inputs.draw(2, 3, 100, 64, "fp8", True, seed=5)
    g = torch.Generator().manual_seed(5)
    qf = torch.randn((2, 3, 100, 64), generator=g).numpy()
    for name, codes, ds in (("q", x.q, x.descale_q), ("k", x.k, x.descale_k),
                            ("v", x.v, x.descale_v)):
        assert codes.dtype == np.uint8 and ds.dtype == np.float32 and ds.shape == (6,)
        vals = A.decode_e4m3(codes)
        assert np.isfinite(vals).all()
        # The largest magnitude of every head maps to +-448 exactly.
        assert np.array_equal(np.abs(vals).reshape(6, -1).max(axis=1), np.full(6, 448.0))
    # Descale is amax / 448 in float32, and dequantized values track the draw
    # within e4m3's relative spacing (2^-3) plus the subnormal step.
    amax = np.abs(qf).reshape(6, -1).max(axis=1).astype(np.float32)
    assert np.array_equal(x.descale_q, (amax / np.float32(448)).astype(np.float32))
    deq = A.decode_e4m3(x.q) * x.descale_q.astype(np.float64).reshape(2, 3, 1, 1)
    err = np.abs(deq - qf)
    assert (err <= np.abs(qf) * 2.0 ** -4 + 2.0 ** -10 * x.descale_q.max()).all()


def test_configs_table():
    assert len(inputs.CONFIGS) == 5
    name, B, H, N, d, dtype, causal, seed = inputs.config(2)
    assert (B, H, N, d, dtype, causal) == (2, 16, 4096, 128, "fp16", False)
    assert inputs.config("fp8_causal_b1h32_n16384_d128")[5] == "fp8"
