"""Randomised parity: seeded draws of shape, head dimension, dtype, causality,
layout and entry point (fa_fwd_ex, fa_fwd_fp8_pv, fa_fwd_kvsplit,
fa_fwd_fp8_kvtile; fa_bwd; full-size fp8 grids on sampled rows),
every output against the CPU fp64 oracle with the bars of the other parity
tests.  The case lists are fixed by their seeds, so a failure names a case
that reruns exactly."""
import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding, inputs
from tests.test_gpu_parity import announce, check, to_np

pytestmark = pytest.mark.gpu

TORCH = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def _cases(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ["fp16", "bf16", "fp8"][rng.integers(3)]
        entry = ["ex", "kvsplit", "fp8_pv"][rng.integers(3)] if dtype == "fp8" else \
            ["ex", "kvsplit"][rng.integers(2)]
        out.append(dict(
            B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
            N=int(rng.choice([1, 2, 63, 64, 65, 127, 128, 129, 255, 300, 511, 513, 700, 1000,
                              1299])),
            d=int(rng.choice([64, 128])), dtype=dtype, causal=bool(rng.integers(2)),
            layout=["bhnd", "bnhd"][rng.integers(2)], entry=entry,
            min_keys=int(rng.choice([0, 1, 129, 512])), seed=3000 + i))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


@pytest.mark.parametrize("case", CASES, ids=lambda c: (
    f"{c['entry']}-{c['dtype']}-B{c['B']}H{c['H']}N{c['N']}d{c['d']}"
    f"-{'causal' if c['causal'] else 'full'}-{c['layout']}-s{c['seed']}"))
def test_random_forward(case):
    inp = inputs.draw(case["B"], case["H"], case["N"], case["d"], case["dtype"], case["causal"],
                      seed=case["seed"])
    announce(f"random {case}")
    q, k, v, ds = binding.to_device(inp)
    if case["layout"] == "bnhd":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    kw = dict(layout=case["layout"], causal=inp.causal, scale=inp.scale,
              descales=ds if inp.dtype == "fp8" else None)
    if case["entry"] == "kvsplit":
        o, l = binding.fwd_kvsplit(q, k, v, **kw)
    elif case["entry"] == "fp8_pv":
        o, l = binding.fwd_fp8_pv(q, k, v, min_keys=case["min_keys"], **kw)
    else:
        o, l = binding.fwd_ex(q, k, v, **kw)
    torch.cuda.synchronize()
    if case["layout"] == "bnhd":
        o = o.transpose(1, 2).contiguous()
    on, ln = to_np(o, l, inp)
    if case["entry"] == "fp8_pv":
        # Tiles of 128 rows whose first row sees >= min_keys keys take e4m3 P:
        # those rows get the e4m3 bound of the fp8-P V tests, the rest the
        # fixed bars.
        from tests.test_gpu_fp8pv import check_e4m3_bound
        check_e4m3_bound(inp, on, ln)
    else:
        check(inp, on, ln)


def _kvt_cases(n=16, seed=20261204):
    rng = np.random.default_rng(seed)
    return [dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                 N=int(rng.choice([1, 63, 64, 65, 129, 300, 513, 1000, 1299])),
                 d=int(rng.choice([64, 128])), causal=bool(rng.integers(2)),
                 layout=["bhnd", "bnhd"][rng.integers(2)],
                 pv_min_keys=int(rng.choice([-1, -1, 0, 129, 512])), seed=3500 + i)
            for i in range(n)]


@pytest.mark.parametrize("case", _kvt_cases(), ids=lambda c: (
    f"kvtile-B{c['B']}H{c['H']}N{c['N']}d{c['d']}-{'causal' if c['causal'] else 'full'}"
    f"-{c['layout']}-pv{c['pv_min_keys']}-s{c['seed']}"))
def test_random_kvtile(case):
    # fp8 with K and V scales per 64-key tile: P V in fp16 (pv_min_keys -1)
    # against the fp8 bars, with fp8 P V for some or all tiles against the
    # per-element e4m3 bound (which also covers the fp16-P V rows).
    from tests.test_gpu_kvtile import check_e4m3_bound_tiles, run_kvtile
    inp = inputs.draw(case["B"], case["H"], case["N"], case["d"], "fp8", case["causal"],
                      seed=case["seed"], kv_tile=binding.KV_TILE)
    announce(f"random kvtile {case}")
    o, l = to_np(*run_kvtile(inp, pv_min_keys=case["pv_min_keys"], layout=case["layout"]), inp)
    if case["pv_min_keys"] < 0:
        check(inp, o, l)
    else:
        check_e4m3_bound_tiles(inp, o, l)


def _large_fp8_cases(n=8, seed=20261205):
    """fp8 grids of at least two 256-row tiles per CU on a 256-CU MI355X:
    fp16 P V runs the 8-wave kernel (per-head or per-tile scales)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, H, N = int(rng.integers(1, 5)), int(rng.integers(8, 49)), int(rng.integers(1400, 4200))
        if B * H * ((N + 255) // 256) < 512 or B * H * N > 2_000_000:
            continue
        out.append(dict(B=B, H=H, N=N, causal=bool(rng.integers(2)),
                        layout=["bhnd", "bnhd"][rng.integers(2)],
                        kvtile=bool(rng.integers(2)), seed=3700 + len(out)))
    return out


@pytest.mark.parametrize("case", _large_fp8_cases(), ids=lambda c: (
    f"fp8large-{'kvtile' if c['kvtile'] else 'head'}-B{c['B']}H{c['H']}N{c['N']}"
    f"-{'causal' if c['causal'] else 'full'}-{c['layout']}-s{c['seed']}"))
def test_random_large_fp8(case):
    # Full-size grids, oracle on sampled heads and rows (every row would take
    # the fp64 oracle minutes).
    from tests.test_gpu_parity import _sample_rows
    from tests.test_gpu_kvtile import run_kvtile
    inp = inputs.draw(case["B"], case["H"], case["N"], 128, "fp8", case["causal"],
                      seed=case["seed"], **({"kv_tile": binding.KV_TILE} if case["kvtile"] else {}))
    announce(f"random large fp8 {case}")
    if case["kvtile"]:
        o, l = run_kvtile(inp, layout=case["layout"])
    else:
        q, k, v, ds = binding.to_device(inp)
        if case["layout"] == "bnhd":
            q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        o, l = binding.fwd_ex(q, k, v, layout=case["layout"], causal=inp.causal,
                              scale=inp.scale, descales=ds)
        torch.cuda.synchronize()
        if case["layout"] == "bnhd":
            o = o.transpose(1, 2).contiguous()
    on, ln = to_np(o, l, inp)
    BH = inp.B * inp.H
    rng = np.random.default_rng(case["seed"])
    heads = sorted({0, BH // 3, BH - 1, int(rng.integers(BH))})
    rows = np.unique(np.concatenate([_sample_rows(inp.N, seed=case["seed"], extra=12),
                                     [inp.N - 1]]))
    check(inp, on, ln, heads=heads, rows=rows)


def _bwd_cases(n=12, seed=20261203):
    rng = np.random.default_rng(seed)
    return [dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)),
                 N=int(rng.choice([1, 5, 64, 65, 127, 129, 200, 333, 513])),
                 d=int(rng.choice([64, 128])), dtype=["fp16", "bf16"][rng.integers(2)],
                 causal=bool(rng.integers(2)), seed=3100 + i) for i in range(n)]


@pytest.mark.parametrize("case", _bwd_cases(), ids=lambda c: (
    f"bwd-{c['dtype']}-B{c['B']}H{c['H']}N{c['N']}d{c['d']}"
    f"-{'causal' if c['causal'] else 'full'}-s{c['seed']}"))
def test_random_backward(case):
    from tests.test_gpu_bwd import check_grads, run_bwd
    inp = inputs.draw_bwd(case["B"], case["H"], case["N"], case["d"], case["dtype"],
                          case["causal"], seed=case["seed"])
    dq, dk, dv, delta, o = run_bwd(inp)
    check_grads(inp, (dq, dk, dv))
