"""fa_fwd_kvsplit (key ranges of long query tiles split over workgroups, then
merged through their LSE) against the CPU fp64 oracle, with the bars of the
other forward parity tests.  Every case asserts first that the library does
split it (non-zero workspace), so the chunk and merge kernels are what is
measured."""
import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding, inputs
from oracle import attention as oracle
from tests.test_gpu_parity import _sample_rows, announce, check, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


TORCH = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def ws_bytes(inp):
    return binding.kvsplit_workspace_bytes(inp.B, inp.H, inp.N, inp.d, inp.causal,
                                           TORCH[inp.dtype])


def run_split(inp, layout="bhnd", workspace=None, out=None, lse=None):
    announce(f"fa_fwd_kvsplit layout={layout} {inp.describe()}")
    q, k, v, ds = binding.to_device(inp)
    if layout == "bnhd":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    o, l = binding.fwd_kvsplit(q, k, v, layout=layout, causal=inp.causal, scale=inp.scale,
                               descales=ds if inp.dtype == "fp8" else None, out=out, lse=lse,
                               workspace=workspace)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.transpose(1, 2).contiguous()
    return o, l


def run_whole(inp):
    announce(f"fa_fwd {inp.describe()}")
    o, l = binding.run_inputs(inp)
    torch.cuda.synchronize()
    return o, l


# (B, H, N, d, dtype, causal): small enough for the whole oracle, each split
# into 5-12 chunks per long tile, ragged N.
SPLIT_CASES = [
    (1, 2, 1100, 128, "fp16", True),
    (1, 2, 1300, 128, "bf16", False),
    (1, 3, 1000, 64, "bf16", False),
    (2, 1, 777, 64, "fp16", True),
    (1, 2, 1500, 128, "fp8", True),
    (1, 2, 900, 64, "fp8", False),
    (1, 1, 2049, 128, "bf16", True),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_split_parity(case):
    B, H, N, d, dtype, causal = case
    inp = inputs.draw(B, H, N, d, dtype, causal, seed=2000 + N + d)
    assert ws_bytes(inp) > 0, "expected a split plan"
    o, l = run_split(inp)
    on, ln = to_np(o, l, inp)
    check(inp, on, ln)
    # Close to the unsplit kernels too.  They differ by more than the merge's
    # fp32 rounding: P is rounded to fp16 relative to each chunk's own running
    # max, so each side's row sum carries its own relative error of up to 2^-11
    # and the two LSEs may differ by up to 2 * 2^-11 ~ 9.8e-4.
    ow, lw = run_whole(inp)
    assert (o.float() - ow.float()).abs().max().item() <= 2e-3
    assert (l - lw).abs().max().item() <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_split_bnhd_matches_bhnd(causal):
    inp = inputs.draw(1, 3, 1111, 128, "fp16", causal, seed=2100)
    assert ws_bytes(inp) > 0
    o1, l1 = run_split(inp)
    o2, l2 = run_split(inp, layout="bnhd")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_no_split_is_fwd_ex():
    # 256 tiles of 4 groups: the plan keeps the grid whole and the call is
    # fa_fwd_ex itself.
    inp = inputs.draw(4, 16, 1024, 128, "fp16", False, seed=2200)
    assert ws_bytes(inp) == 0
    o1, l1 = run_split(inp)
    o2, l2 = run_whole(inp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("wl", [w[0] for w in inputs.SHARD_WORKLOADS])
def test_shard_workloads_sampled(wl):
    inp = inputs.draw_config(wl)
    assert ws_bytes(inp) > 0
    o, l = run_split(inp)
    on, ln = to_np(o, l, inp)
    rows = _sample_rows(inp.N, seed=2300)
    check(inp, on, ln, heads=list(range(inp.B * inp.H)), rows=rows)
    assert np.isfinite(on).all() and np.isfinite(ln).all()


def test_no_writes_outside_outputs_and_workspace():
    inp = inputs.draw(1, 2, 1100, 128, "bf16", True, seed=2400)
    need = ws_bytes(inp)
    assert need > 0
    G = 1 << 16
    wsbuf = torch.full((need + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = wsbuf[G:G + need]
    n_o = inp.B * inp.H * inp.N * inp.d
    n_l = inp.B * inp.H * inp.N
    obuf = torch.full((n_o + 2 * 4096,), 7.0, dtype=torch.float16, device="cuda")
    lbuf = torch.full((n_l + 2 * 4096,), 7.0, dtype=torch.float32, device="cuda")
    out = obuf[4096:4096 + n_o].view(inp.B, inp.H, inp.N, inp.d)
    lse = lbuf[4096:4096 + n_l].view(inp.B, inp.H, inp.N)
    run_split(inp, workspace=ws, out=out, lse=lse)
    assert torch.all(wsbuf[:G] == 0x5A) and torch.all(wsbuf[G + need:] == 0x5A)
    assert torch.all(obuf[:4096] == 7.0) and torch.all(obuf[4096 + n_o:] == 7.0)
    assert torch.all(lbuf[:4096] == 7.0) and torch.all(lbuf[4096 + n_l:] == 7.0)
    on, ln = to_np(out, lse, inp)
    check(inp, on, ln)


def test_workspace_reused_across_problems():
    # Stale partials of an earlier call must not leak into the next one.
    a = inputs.draw(1, 2, 1500, 128, "fp16", True, seed=2500)
    b = inputs.draw(1, 2, 1100, 128, "fp16", True, seed=2501)
    ws = torch.empty(max(ws_bytes(a), ws_bytes(b)), dtype=torch.uint8, device="cuda")
    oa, la = run_split(a, workspace=ws)
    ob, lb = run_split(b, workspace=ws)
    check(a, *to_np(oa, la, a))
    check(b, *to_np(ob, lb, b))


def test_deterministic():
    inp = inputs.draw(1, 4, 3000, 128, "bf16", True, seed=2600)
    assert ws_bytes(inp) > 0
    o1, l1 = run_split(inp)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = run_split(inp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_zero_q_prefix_mean():
    # Q = 0: every chunk's rows are uniform over their keys, and the merge
    # must weight chunks by their key counts: LSE = ln(i + 1).
    B, H, N, d = 1, 2, 1500, 128
    g = torch.Generator().manual_seed(27)
    q = torch.zeros((B, H, N, d))
    k = torch.randn((B, H, N, d), generator=g)
    v = torch.randn((B, H, N, d), generator=g)
    inp = inputs.from_float(q, k, v, "bf16", True)
    assert ws_bytes(inp) > 0
    o, l = to_np(*run_split(inp), inp)
    check(inp, o, l)
    assert np.abs(l - np.log(np.arange(1, N + 1))[None, :]).max() <= 1e-3


# --- fp8 P V with the split (fa_fwd_fp8_pv_kvsplit) ------------------------------

def run_pv_split(inp, min_keys, layout="bhnd"):
    announce(f"fa_fwd_fp8_pv_kvsplit min_keys={min_keys} layout={layout} {inp.describe()}")
    q, k, v, ds = binding.to_device(inp)
    if layout == "bnhd":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    o, l = binding.fwd_fp8_pv_kvsplit(q, k, v, min_keys=min_keys, layout=layout,
                                      causal=inp.causal, scale=inp.scale, descales=ds)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.transpose(1, 2).contiguous()
    return o, l


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_pv_split_causal(d):
    # 12 tiles of 128 rows: tiles 0-3 unsplit with fp16 P V (bit-identical to
    # fa_fwd_fp8_pv there), tiles 4-11 split with fp8 P V, within the fp8 bars.
    from tests.test_gpu_fp8pv import run_pv
    inp = inputs.draw(1, 2, 1500, d, "fp8", True, seed=2700 + d)
    assert ws_bytes(inp) > 0
    o, l = run_pv_split(inp, 512)
    o1, l1 = run_pv(inp, 512)
    assert torch.equal(o[:, :, :512].contiguous().view(torch.int16),
                       o1[:, :, :512].contiguous().view(torch.int16))
    check(inp, *to_np(o, l, inp))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_pv_split_all_tiles_e4m3_bound(causal):
    from tests.test_gpu_fp8pv import check_e4m3_bound
    inp = inputs.draw(1, 2, 1500, 128, "fp8", causal, seed=2750)
    assert ws_bytes(inp) > 0
    o, l = run_pv_split(inp, 0)
    check_e4m3_bound(inp, *to_np(o, l, inp))


def test_fp8_pv_split_bnhd_matches_bhnd():
    inp = inputs.draw(1, 3, 1111, 128, "fp8", True, seed=2760)
    assert ws_bytes(inp) > 0
    o1, l1 = run_pv_split(inp, 256)
    o2, l2 = run_pv_split(inp, 256, layout="bnhd")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_fp8_pv_split_shard_sampled():
    inp = inputs.draw_config("fp8_causal_b1h4_n16384_d128")
    o, l = run_pv_split(inp, 512)
    rows = np.unique(np.concatenate([_sample_rows(inp.N, seed=2800), [511, 512, 513]]))
    check(inp, *to_np(o, l, inp), heads=list(range(inp.B * inp.H)), rows=rows)


def test_binding_rejects_foreign_workspace():
    # A workspace in host memory, or strided, is refused before any launch.
    inp = inputs.draw(1, 2, 1100, 128, "fp16", True, seed=2900)
    need = ws_bytes(inp)
    assert need > 0
    q, k, v, _ = binding.to_device(inp)
    with pytest.raises(ValueError, match="device"):
        binding.fwd_kvsplit(q, k, v, causal=True, workspace=torch.empty(need, dtype=torch.uint8))
    strided = torch.empty(2 * need, dtype=torch.uint8, device="cuda")[::2]
    with pytest.raises(ValueError, match="contiguous"):
        binding.fwd_kvsplit(q, k, v, causal=True, workspace=strided)
