"""fp8 inputs with P V on the fp8 matrix instructions (fa_fwd_fp8_pv) against the
CPU fp64 oracle.

Bars:
  * query tiles that keep P V in fp16 (first row sees fewer than min_keys keys)
    run the fa_fwd_fp8 kernel itself: bit-identical to it;
  * with the default min_keys = 512, every output within the fp8 bars of the
    other parity tests (max|dO| <= 3e-2, mean|dO| <= 3.75e-3, max|dLSE| <= 1e-3);
  * with min_keys = 0 (fp8 P V everywhere, rows with a handful of keys
    included) each element within the e4m3 rounding bound: every probability
    is rounded with relative error <= 2^-4 (3 fraction bits, no saturation:
    the largest of a block is scaled into (128, 256]), so
        |dO_ic| <= 2^-4 sum_j p_ij |v_jc| / l_i + 63 * 2^-17 max_j |v_jc| + 4e-3,
    where the middle term bounds the probabilities that fall below the
    normal range (at most 63 per block, each off by <= 2^-10 against a block
    maximum >= 128) and 4e-3 is the fp16 bar for the rest of the arithmetic.
    sum_j p_ij |v_jc| / l_i is the oracle's output for |V|.  LSE takes the
    unrounded row sum: max|dLSE| <= 1e-3 throughout.
"""
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


def run_pv(inp, min_keys, layout="bhnd"):
    announce(f"fa_fwd_fp8_pv min_keys={min_keys} layout={layout} {inp.describe()}")
    q, k, v, ds = binding.to_device(inp)
    if layout == "bnhd":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    o, l = binding.fwd_fp8_pv(q, k, v, min_keys=min_keys, layout=layout, causal=inp.causal,
                              scale=inp.scale, descales=ds)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.transpose(1, 2).contiguous()
    return o, l


def run_fp16_pv(inp):
    announce(f"fa_fwd_fp8 {inp.describe()}")
    o, l = binding.run_inputs(inp)
    torch.cuda.synchronize()
    return o, l


def abs_v(inp):
    """The same problem with |V| (e4m3 sign bit cleared)."""
    return inputs.AttnInputs(inp.B, inp.H, inp.N, inp.d, inp.dtype, inp.causal, inp.scale,
                             inp.q, inp.k, inp.v & np.uint8(0x7F), inp.descale_q,
                             inp.descale_k, inp.descale_v, inp.seed)


def check_e4m3_bound(inp, o, l, heads=None, rows=None):
    # The fp8 dot error on the scores (E_i per row, see test_gpu_parity) moves
    # the weights by at most 2 E_i relative and LSE by E_i.
    o_ref, l_ref = oracle.run(inp, rows=rows, heads=heads)
    a_ref, _ = oracle.run(abs_v(inp), rows=rows, heads=heads)
    hsel = np.arange(inp.B * inp.H) if heads is None else np.asarray(heads)
    rsel = np.arange(inp.N) if rows is None else np.asarray(rows)
    e = fp8_dot_err(inp, hsel, rsel)[:, :, None]
    lse_tol = 1e-3 + e[:, :, 0]
    og, lg = o[hsel][:, rsel], l[hsel][:, rsel]
    assert np.isfinite(og).all() and np.isfinite(lg).all(), inp.describe()
    v = torch.from_numpy(inp.v).view(torch.float8_e4m3fn).double().numpy()
    v = v.reshape(inp.B * inp.H, inp.N, inp.d) * inp.descale_v.astype(np.float64)[:, None, None]
    vmax = np.abs(v[hsel]).max(axis=1)[:, None, :]  # per head and column
    bound = (2.0 ** -4 + 2 * e) * a_ref + 63 * 2.0 ** -17 * vmax + 4e-3
    d_o = np.abs(og - o_ref)
    d_l = np.abs(lg - l_ref)
    ratio = float((d_o / bound).max())
    announce(f"{inp.describe()}: max|dO|={d_o.max():.3e} mean|dO|={d_o.mean():.3e} "
             f"max|dO|/bound={ratio:.3f} max|dLSE|={d_l.max():.3e}")
    log = os.environ.get("FA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": "e4m3 bound " + inp.describe(),
                                "max_dO": float(d_o.max()), "mean_dO": float(d_o.mean()),
                                "max_dO_over_bound": ratio, "max_dLSE": float(d_l.max()),
                                "rows": int(len(rsel)), "heads": int(len(hsel))}) + "\n")
    assert ratio <= 1.0, inp.describe()
    assert (d_l <= lse_tol).all(), inp.describe()
    return d_o


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_min_keys_above_n_is_fwd_fp8(d, causal):
    inp = inputs.draw(2, 3, 300, d, "fp8", causal, seed=1300 + d)
    o1, l1 = run_pv(inp, min_keys=301)
    o2, l2 = run_fp16_pv(inp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", (1, 17, 64, 100, 129, 300))
def test_all_fp8_small_shapes_within_e4m3_bound(d, causal, N):
    inp = inputs.draw(2, 3, N, d, "fp8", causal, seed=1400 + N + d)
    o, l = to_np(*run_pv(inp, min_keys=0), inp)
    check_e4m3_bound(inp, o, l)


@pytest.mark.parametrize("d", [64, 128])
def test_split_causal(d):
    # 1100 rows: tiles 0-3 (rows < 512) keep fp16 P V and match fa_fwd_fp8 bit
    # for bit; tiles 4-8 (the last one ragged) run fp8 P V within the fp8 bars.
    inp = inputs.draw(1, 3, 1100, d, "fp8", True, seed=1500 + d)
    o, l = run_pv(inp, min_keys=512)
    o16, l16 = run_fp16_pv(inp)
    assert torch.equal(o[:, :, :512].contiguous().view(torch.int16),
                       o16[:, :, :512].contiguous().view(torch.int16))
    assert torch.equal(l[:, :, :512].contiguous().view(torch.int32),
                       l16[:, :, :512].contiguous().view(torch.int32))
    assert not torch.equal(o[:, :, 512:].contiguous().view(torch.int16),
                           o16[:, :, 512:].contiguous().view(torch.int16))
    on, ln = to_np(o, l, inp)
    check(inp, on, ln)


@pytest.mark.parametrize("min_keys", [129, 130, 257])
def test_split_at_tile_boundaries(min_keys):
    # A tile takes fp8 P V when its first row (qt*128) sees >= min_keys keys,
    # i.e. qt*128 + 1 >= min_keys: 129 -> tiles from 1 on, 130 and 257 -> from 2 on
    # (257: row 256 sees 257 keys).
    inp = inputs.draw(1, 2, 400, 128, "fp8", True, seed=1550)
    o, l = run_pv(inp, min_keys=min_keys)
    o16, _ = run_fp16_pv(inp)
    first_fp8 = 128 * (1 if min_keys == 129 else 2)
    assert torch.equal(o[:, :, :first_fp8].contiguous().view(torch.int16),
                       o16[:, :, :first_fp8].contiguous().view(torch.int16))
    assert not torch.equal(o[:, :, first_fp8:first_fp8 + 128].contiguous().view(torch.int16),
                           o16[:, :, first_fp8:first_fp8 + 128].contiguous().view(torch.int16))
    on, ln = to_np(o, l, inp)
    check_e4m3_bound(inp, on, ln)


def test_noncausal_all_fp8():
    inp = inputs.draw(2, 2, 700, 128, "fp8", False, seed=1600)
    o, l = to_np(*run_pv(inp, min_keys=512), inp)
    check(inp, o, l)


@pytest.mark.parametrize("causal", [False, True])
def test_bnhd_layout_matches_bhnd(causal):
    inp = inputs.draw(2, 3, 333, 128, "fp8", causal, seed=1700)
    o1, l1 = run_pv(inp, min_keys=0)
    o2, l2 = run_pv(inp, min_keys=0, layout="bnhd")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_unit_descales():
    # No descale arrays: the e4m3 codes are the values.
    inp = inputs.draw(1, 2, 600, 64, "fp8", True, seed=1750, scale=1e-4)
    q, k, v, _ = binding.to_device(inp)
    announce("fa_fwd_fp8_pv unit descales " + inp.describe())
    o, l = binding.fwd_fp8_pv(q, k, v, min_keys=0, causal=True, scale=inp.scale)
    torch.cuda.synchronize()
    unit = np.ones(inp.B * inp.H, dtype=np.float32)
    ref = inputs.AttnInputs(inp.B, inp.H, inp.N, inp.d, "fp8", True, inp.scale, inp.q, inp.k,
                            inp.v, unit, unit, unit)
    on, ln = to_np(o, l, inp)
    # Values up to |448|: the fixed fp16 term of the bound scales with them.
    d_o = np.abs(on - oracle.run(ref)[0])
    a_ref = oracle.run(abs_v(ref))[0]
    assert (d_o <= 2.0 ** -4 * a_ref + 63 * 2.0 ** -17 * 448 + 4e-3 * 448 / 4).all()


def test_zero_q_gives_lse_of_uniform_rows():
    # Q = 0: every probability is 1 (exact in e4m3 after any power-of-two
    # scale), so fp8 P V is exact here and O is the prefix mean of V.
    B, H, N, d = 1, 2, 700, 128
    g = torch.Generator().manual_seed(31)
    q = torch.zeros((B, H, N, d))
    k = torch.randn((B, H, N, d), generator=g)
    v = torch.randn((B, H, N, d), generator=g)
    inp = inputs.from_float(q, k, v, "fp8", True)
    o, l = to_np(*run_pv(inp, min_keys=0), inp)
    check(inp, o, l)
    assert np.abs(l - np.log(np.arange(1, N + 1))[None, :]).max() <= 1e-3


def test_large_scores():
    # Scores of order 100 (past fp32 exp overflow), with the fp8 dot error of
    # such scores in the bars.
    inp = inputs.draw(1, 2, 700, 64, "fp8", False, seed=1800, scale=4.0)
    o, l = to_np(*run_pv(inp, min_keys=0), inp)
    assert float(np.abs(l).max()) > 88.0
    check_e4m3_bound(inp, o, l)


def test_config5_full_size_sampled():
    # The fp8 causal workload [1, 32, 16384, 128] at full size, default split.
    inp = inputs.draw_config(4)
    o, l = to_np(*run_pv(inp, min_keys=512), inp)
    heads = [0, 1, 16, 31]
    rows = np.unique(np.concatenate([_sample_rows(inp.N, seed=45),
                                     [511, 512, 513, 639, 640, 1023, 1024]]))
    check(inp, o, l, heads=heads, rows=rows)
    assert np.isfinite(o).all() and np.isfinite(l).all()


def test_deterministic():
    inp = inputs.draw(1, 4, 2000, 128, "fp8", True, seed=1900)
    o1, l1 = run_pv(inp, min_keys=512)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = run_pv(inp, min_keys=512)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
