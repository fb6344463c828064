"""fa_fwd_kvsplit_noalloc (split workspace in the library's static device
scratch) against fa_fwd_kvsplit (caller's workspace) through the C ABI: two
calls in a row, the second on a smaller problem, each bit-identical to the
caller-workspace entry point (same kernels and split plan) and within the
oracle's bars on sampled rows."""
import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding, inputs
from tests.test_gpu_parity import announce, check, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _rows(N):
    return np.unique(np.array([0, 1, 63, 64, 255, 256, N // 2, N - 65, N - 2, N - 1]))


def _one(inp, layout="bhnd"):
    announce("noalloc " + inp.describe())
    need = binding.kvsplit_workspace_bytes(inp.B, inp.H, inp.N, inp.d, inp.causal,
                                           binding.TORCH_DTYPES[inp.dtype])
    assert 0 < need <= binding.kvsplit_noalloc_max_bytes(), need  # the split path runs
    q, k, v, ds = binding.to_device(inp)
    torch.cuda.synchronize()
    o_ref, l_ref = binding.fwd_kvsplit(q, k, v, causal=inp.causal, scale=inp.scale, descales=ds)
    out = torch.full(q.shape, 7.0, dtype=torch.float16, device="cuda")
    lse = torch.full((inp.B, inp.H, inp.N), 7.0, dtype=torch.float32, device="cuda")
    o, l = binding.fwd_kvsplit_noalloc(q, k, v, causal=inp.causal, scale=inp.scale,
                                       descales=ds, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32))
    on, ln = to_np(o, l, inp)
    BH = inp.B * inp.H
    check(inp, on, ln, heads=sorted({0, BH - 1}), rows=_rows(inp.N))


def test_noalloc_two_calls_second_smaller():
    # 19 MiB of partials, then 3.2 MiB: the second call reuses the scratch the
    # first one filled.
    _one(inputs.draw(1, 3, 2500, 128, "bf16", True, seed=4100))
    _one(inputs.draw(1, 2, 1100, 128, "fp16", False, seed=4101))


def test_noalloc_fp8_then_unsplit():
    _one(inputs.draw(1, 2, 3000, 128, "fp8", True, seed=4102))
    # A problem the plan keeps whole touches no scratch and matches fa_fwd_ex.
    inp = inputs.draw(1, 2, 300, 64, "fp16", True, seed=4103)
    q, k, v, ds = binding.to_device(inp)
    o1, l1 = binding.fwd_ex(q, k, v, causal=True, scale=inp.scale)
    o2, l2 = binding.fwd_kvsplit_noalloc(q, k, v, causal=True, scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_noalloc_rejects_oversized_split():
    inp_shape = (1, 4, 16384, 128)
    need = binding.kvsplit_workspace_bytes(*inp_shape, True, torch.float8_e4m3fn)
    if need <= binding.kvsplit_noalloc_max_bytes():
        pytest.skip("this device's split plan fits the scratch")
    x = torch.zeros(inp_shape, dtype=torch.float8_e4m3fn, device="cuda")
    with pytest.raises(binding.FAError) as e:
        binding.fwd_kvsplit_noalloc(x, x, x, causal=True)
    assert e.value.status == -12
