"""fa_fwd_fp8_kvtile (fp8 with K and V scales per tile of 64 key rows, the
per-block K scale of the CUDA chapter's fp8 section, section 17.7 item 1)
through the C ABI, against the fp64 oracle, which dequantizes every key row
with its own tile's scale.

Bars: the fp8 bars of test_gpu_parity with P V in fp16; with P V on the fp8
matrix instructions (pv_min_keys = 0) the per-element e4m3 bound of
test_gpu_fp8pv, V taken with its per-tile scales."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding, inputs
from oracle import attention as oracle
from tests.test_gpu_parity import _sample_rows, announce, check, fp8_dot_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def run_kvtile(inp, pv_min_keys=-1, layout="bhnd"):
    announce(f"fa_fwd_fp8_kvtile pv_min_keys={pv_min_keys} layout={layout} {inp.describe()}")
    q, k, v, ds = binding.to_device(inp)
    if layout == "bnhd":
        q, k, v = (t.view(torch.uint8).permute(0, 2, 1, 3).contiguous().view(t.dtype)
                   for t in (q, k, v))
    o, l = binding.fwd_fp8_kvtile(q, k, v, ds, pv_min_keys=pv_min_keys, layout=layout,
                                  causal=inp.causal, scale=inp.scale)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.permute(0, 2, 1, 3).contiguous()
    return o, l


def check_e4m3_bound_tiles(inp, o, l, heads=None, rows=None):
    """|dO_ic| <= 2^-4 sum_j p_ij |v_jc| / l_i + 63 * 2^-17 max_j |v_jc| + 4e-3
    (each rounded probability relative 2^-4, at most 63 subnormal ones per
    block), the first term the oracle's output for |V|, plus the fp8 dot
    error's 2 E_i relative; LSE within 1e-3 + E_i."""
    o_ref, l_ref = oracle.run(inp, rows=rows, heads=heads)
    absv = dataclasses.replace(inp, v=inp.v & np.uint8(0x7F))
    a_ref, _ = oracle.run(absv, rows=rows, heads=heads)
    hsel = np.arange(inp.B * inp.H) if heads is None else np.asarray(heads)
    rsel = np.arange(inp.N) if rows is None else np.asarray(rows)
    e = fp8_dot_err(inp, hsel, rsel)[:, :, None]
    og, lg = o[hsel][:, rsel], l[hsel][:, rsel]
    assert np.isfinite(og).all() and np.isfinite(lg).all(), inp.describe()
    vmax = np.stack([np.abs(oracle.head_values(inp, f // inp.H, f % inp.H)[2]).max(axis=0)
                     for f in hsel])[:, None, :]
    bound = (2.0 ** -4 + 2 * e) * a_ref + 63 * 2.0 ** -17 * vmax + 4e-3
    d_o = np.abs(og - o_ref)
    d_l = np.abs(lg - l_ref)
    ratio = float((d_o / bound).max())
    announce(f"{inp.describe()}: max|dO|={d_o.max():.3e} max|dO|/bound={ratio:.3f} "
             f"max|dLSE|={d_l.max():.3e}")
    log = os.environ.get("FA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": "kvtile e4m3 bound " + inp.describe(),
                                "max_dO": float(d_o.max()), "max_dO_over_bound": ratio,
                                "max_dLSE": float(d_l.max())}) + "\n")
    assert ratio <= 1.0, inp.describe()
    assert (d_l <= 1e-3 + e[:, :, 0]).all(), inp.describe()


def _varied_tiles(B, H, N, d, causal, seed):
    """N(0, 1) draws whose 64-row tiles of K and V are multiplied by factors
    from 2^-3 to 2^3 (not powers of two), so the per-tile scales differ by
    up to 2^6 within a head and have mantissas of their own."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    q, k, v = (torch.randn(shape, generator=g) for _ in range(3))
    t = torch.arange(N) // binding.KV_TILE
    fk = (2.0 ** ((t % 7) - 3).float() * (1.0 + 0.37 * (t % 3).float()))[None, None, :, None]
    fv = (2.0 ** (2 - (t % 5)).float() * (1.0 + 0.21 * (t % 4).float()))[None, None, :, None]
    return inputs.from_float(q, k * fk, v * fv, "fp8", causal, seed=seed,
                             kv_tile=binding.KV_TILE)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", (1, 17, 64, 100, 129, 300))
def test_small_shapes_fp16_pv(d, causal, N):
    inp = inputs.draw(2, 3, N, d, "fp8", causal, seed=5000 + N + d, kv_tile=binding.KV_TILE)
    o, l = to_np(*run_kvtile(inp), inp)
    check(inp, o, l)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varied_tile_scales(d, causal):
    inp = _varied_tiles(2, 3, 700, d, causal, seed=5100 + d)
    assert float(inp.descale_k.max() / inp.descale_k.min()) > 16.0
    o, l = to_np(*run_kvtile(inp), inp)
    check(inp, o, l)
    o8, l8 = to_np(*run_kvtile(inp, pv_min_keys=0), inp)
    check_e4m3_bound_tiles(inp, o8, l8)


@pytest.mark.parametrize("causal", [False, True])
def test_eight_wave_kernel_ragged(causal):
    # B*H*ceil(N/256) = 576 workgroups on 256 CUs: the 8-wave d=128 kernel with
    # per-tile scales (P V in fp16), ragged last tile and last key block, tile
    # scales varied within each head.
    inp = _varied_tiles(2, 32, 2100, 128, causal, seed=5150)
    rows = np.unique(np.concatenate([_sample_rows(inp.N, seed=5150), [2047, 2048, 2099]]))
    o, l = to_np(*run_kvtile(inp), inp)
    check(inp, o, l, heads=[0, 1, 33, 63], rows=rows)


@pytest.mark.parametrize("N", (17, 129, 300))
@pytest.mark.parametrize("causal", [False, True])
def test_small_shapes_fp8_pv_within_e4m3_bound(N, causal):
    inp = inputs.draw(2, 3, N, 128, "fp8", causal, seed=5200 + N, kv_tile=binding.KV_TILE)
    o, l = to_np(*run_kvtile(inp, pv_min_keys=0), inp)
    check_e4m3_bound_tiles(inp, o, l)


def test_layout_bnhd_matches_bhnd():
    inp = inputs.draw(1, 4, 333, 128, "fp8", True, seed=5300, kv_tile=binding.KV_TILE)
    o1, l1 = run_kvtile(inp)
    o2, l2 = run_kvtile(inp, layout="bnhd")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_equal_tile_scales_match_per_head_path():
    # Every tile of a head given the head's scale: the same problem as
    # fa_fwd_fp8 with per-head scales; both within the oracle bars, and
    # within two fp16 roundings of the probabilities of each other (the
    # per-tile path rounds p times the scale's mantissa, so each side's row
    # sum is off by at most 2^-11 relative: LSE within 2^-10, O within the
    # fp16 bar).
    base = inputs.draw(1, 4, 500, 128, "fp8", True, seed=5400)
    nt = -(-base.N // binding.KV_TILE)
    tiled = dataclasses.replace(base, kv_tile=binding.KV_TILE,
                                descale_k=np.repeat(base.descale_k, nt),
                                descale_v=np.repeat(base.descale_v, nt))
    o1, l1 = to_np(*run_kvtile(tiled), tiled)
    o2, l2 = to_np(*binding.run_inputs(base), base)
    check(tiled, o1, l1)
    assert np.abs(o1 - o2).max() <= 4e-3 and np.abs(l1 - l2).max() <= 2.0 ** -10


def test_full_size_sampled():
    # The fp8 causal workload's shape [1, 32, 16384, 128], K and V quantized
    # per 64-row tile, P V in fp16 and with the fp8-P V split at 512 keys.
    inp = inputs.draw(1, 32, 16384, 128, "fp8", True, seed=5, kv_tile=binding.KV_TILE)
    heads = [0, 1, 16, 31]
    rows = np.unique(np.concatenate([_sample_rows(inp.N, seed=55), [511, 512, 640, 1024]]))
    o, l = to_np(*run_kvtile(inp), inp)
    check(inp, o, l, heads=heads, rows=rows)
    o, l = to_np(*run_kvtile(inp, pv_min_keys=512), inp)
    check(inp, o, l, heads=heads, rows=rows)
