"""Dot-product precision of the matrix instructions, seen through the C ABI.

A row with a single key has LSE = its one score, scale * q . k, so N = 1
exposes the score arithmetic directly: here with random operands over the
whole input range (fp8: every finite e4m3 code, from 2^-9 to 448; fp16 /
bf16: N(0, 1) times per-head powers of two), each head's error is compared
with the sum of the magnitudes of its products.  The fp16 and bf16
instructions come out within fp32 summation error; the fp8 one (K = 64 per
instruction) sums its products with a relative error of up to about 2^-12.4
of that magnitude sum, which is the bound the fp8 LSE bars of the parity
tests use (FP8_DOT_REL = 2^-12).
"""
import json
import os

import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding, inputs
from oracle import attention as oracle
from tests.test_gpu_parity import FP8_DOT_REL, announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _ratio(inp, l):
    """max over heads of |LSE - s| / (scale * sum_c |q_c k_c|), and of
    |LSE - s| / |s| (fp32 rounding reference)."""
    worst, worst_rel = 0.0, 0.0
    for f in range(inp.B * inp.H):
        q, k, _ = oracle.head_values(inp, f // inp.H, f % inp.H)
        s = inp.scale * float(q[0] @ k[0])
        mag = inp.scale * float(np.abs(q[0]) @ np.abs(k[0]))
        err = abs(float(l.reshape(-1)[f]) - s)
        worst = max(worst, err / mag)
        worst_rel = max(worst_rel, err / max(abs(s), 1e-30))
    return worst, worst_rel


def _log(name, worst):
    log = os.environ.get("FA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": name, "max_err_over_sum_abs_products": worst,
                                "log2": float(np.log2(worst)) if worst > 0 else None}) + "\n")


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_dot_error_bound(d):
    rng = np.random.default_rng(6000 + d)
    B, H, N = 1, 256, 1
    codes = rng.integers(0, 256, size=(3, B, H, N, d), dtype=np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, codes & 0xF8, codes).astype(np.uint8)
    ds = [(rng.uniform(0.5, 2.0, size=B * H)).astype(np.float32) for _ in range(3)]
    inp = inputs.AttnInputs(B, H, N, d, "fp8", False, float(np.float32(1e-3)), codes[0],
                            codes[1], codes[2], ds[0], ds[1], ds[2], 6000 + d)
    announce("fp8 dot precision " + inp.describe())
    _, l = binding.run_inputs(inp)
    torch.cuda.synchronize()
    worst, rel = _ratio(inp, l.cpu().numpy().astype(np.float64))
    announce(f"fp8 d={d}: max |LSE - s| / (scale sum|q k|) = {worst:.3e} "
             f"(2^{np.log2(worst):.2f}), max relative to |s| {rel:.3e}")
    _log(f"fp8 dot precision d={d}", worst)
    assert worst <= FP8_DOT_REL


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fp16_bf16_dot_is_fp32_exact(dtype, d):
    g = torch.Generator().manual_seed(6100 + d)
    B, H, N = 1, 256, 1
    sc = 2.0 ** torch.randint(-6, 7, (1, H, 1, 1), generator=g).float()
    q, k, v = (torch.randn((B, H, N, d), generator=g) * sc for _ in range(3))
    inp = inputs.from_float(q, k, v, dtype, False, scale=1e-2, seed=6100 + d)
    announce(f"{dtype} dot precision " + inp.describe())
    _, l = binding.run_inputs(inp)
    torch.cuda.synchronize()
    worst, rel = _ratio(inp, l.cpu().numpy().astype(np.float64))
    announce(f"{dtype} d={d}: max |LSE - s| / (scale sum|q k|) = {worst:.3e} "
             f"(2^{np.log2(max(worst, 1e-300)):.2f})")
    _log(f"{dtype} dot precision d={d}", worst)
    # fp32 summation of d exact products, then a few fp32 roundings of the
    # score: at most (d + 8) unit roundoffs of the magnitude sum
    assert worst <= (d + 8) * 2.0 ** -24
