"""fa_fwd_ex through the C ABI: the [B, N, H, d] layout against the oracle and,
bit for bit, against the [B, H, N, d] entry points on the same values."""
import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding, inputs
from tests.test_gpu_parity import TOL, announce, check, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _to_bnhd(t):
    """[B, H, N, d] device tensor -> contiguous [B, N, H, d] with the same bits."""
    raw = t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16)
    return raw.permute(0, 2, 1, 3).contiguous().view(t.dtype)


def _run_both(inp):
    q, k, v, ds = binding.to_device(inp)
    announce("bnhd " + inp.describe())
    o_ref, l_ref = binding.run_inputs(inp)
    o, l = binding.fwd_ex(_to_bnhd(q), _to_bnhd(k), _to_bnhd(v), layout="bnhd",
                          causal=inp.causal, scale=inp.scale, descales=ds)
    torch.cuda.synchronize()
    return o.permute(0, 2, 1, 3).contiguous(), l, o_ref, l_ref


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 257])
def test_bnhd_small(dtype, d, causal, N):
    inp = inputs.draw(2, 3, N, d, dtype, causal, seed=2000 + N + d)
    o, l, o_ref, l_ref = _run_both(inp)
    # Same arithmetic in the same order: identical bits to the [B, H, N, d] path.
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32))
    on, ln = to_np(o, l, inp)
    check(inp, on, ln)


def test_bnhd_large_sampled():
    inp = inputs.draw_config(2)  # fp16 [2, 16, 4096, 128]
    o, l, o_ref, l_ref = _run_both(inp)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32))
    on, ln = to_np(o, l, inp)
    BH = inp.B * inp.H
    check(inp, on, ln, heads=[0, BH // 2, BH - 1], rows=np.array([0, 1, 255, 256, 2048, 4095]))


@pytest.mark.parametrize("causal", [False, True])
def test_bnhd_fp8_eight_wave(causal):
    # fp8 with P V in fp16 on a grid of 576 256-row tiles: the 8-wave kernel
    # in both layouts, ragged last tile.
    inp = inputs.draw(2, 32, 2100, 128, "fp8", causal, seed=2050)
    o, l, o_ref, l_ref = _run_both(inp)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32))
    on, ln = to_np(o, l, inp)
    check(inp, on, ln, heads=[0, 33, 63], rows=np.array([0, 1, 255, 256, 1024, 2047, 2048, 2099]))


def test_bhnd_ex_matches_fa_fwd():
    inp = inputs.draw(1, 4, 300, 128, "bf16", True, seed=2100)
    q, k, v, _ = binding.to_device(inp)
    o1, l1 = binding.fwd(q, k, v, causal=True, scale=inp.scale)
    o2, l2 = binding.fwd_ex(q, k, v, layout="bhnd", causal=True, scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_bnhd_no_writes_outside_outputs():
    inp = inputs.draw(2, 3, 131, 64, "fp16", True, seed=2200)
    q, k, v, _ = binding.to_device(inp)
    qb, kb, vb = _to_bnhd(q), _to_bnhd(k), _to_bnhd(v)
    n_o, n_l, G = qb.numel(), inp.B * inp.H * inp.N, 4096
    obuf = torch.full((n_o + 2 * G,), 7.0, dtype=torch.float16, device="cuda")
    lbuf = torch.full((n_l + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    out = obuf[G:G + n_o].view(qb.shape)
    lse = lbuf[G:G + n_l].view(inp.B, inp.H, inp.N)
    announce("bnhd guard " + inp.describe())
    binding.fwd_ex(qb, kb, vb, layout="bnhd", causal=True, scale=inp.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:G] == 7.0) and torch.all(obuf[G + n_o:] == 7.0)
    assert torch.all(lbuf[:G] == 7.0) and torch.all(lbuf[G + n_l:] == 7.0)
    on, ln = to_np(out.permute(0, 2, 1, 3).contiguous(), lse, inp)
    check(inp, on, ln)


@pytest.mark.parametrize("wl", [w[0] for w in inputs.EXTRA_WORKLOADS])
@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
def test_page_workloads_sampled(wl, layout):
    inp = inputs.draw_config(wl)
    q, k, v, _ = binding.to_device(inp)
    if layout == "bnhd":
        q, k, v = _to_bnhd(q), _to_bnhd(k), _to_bnhd(v)
    announce(f"{wl} {layout}")
    o, l = binding.fwd_ex(q, k, v, layout=layout, causal=inp.causal, scale=inp.scale)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.permute(0, 2, 1, 3).contiguous()
    on, ln = to_np(o, l, inp)
    BH = inp.B * inp.H
    rows = np.unique(np.array([0, 1, 127, 128, 255, inp.N // 2, inp.N - 2, inp.N - 1]))
    check(inp, on, ln, heads=sorted({0, 1, BH // 2, BH - 1}), rows=rows)
