"""fa_bwd through the C ABI against the fp64 oracle's gradients.

The GPU backward takes the GPU forward's O (fp16) and LSE, as a training step
would; the oracle differentiates the exact problem.  Bars, relative to the
size of each gradient tensor (R = the oracle's):
  max|d - R| <= TOL_MAX * Mx   and   mean|d - R| <= TOL_MEAN * Mn,
with Mx = max(max|R|, 0.1 G), Mn = max(mean|R|, 0.1 g), G and g the largest
max|.| and mean|.| over the problem's three reference gradients: a gradient
that vanishes exactly (dQ and dK at N = 1) is held to the problem's gradient
scale instead of to zero.
"""
import json
import os

import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding, inputs
from oracle import attention as oracle
from tests.test_gpu_parity import announce

pytestmark = pytest.mark.gpu

# (max, mean) relative bars per input type: 10 and 2 unit roundoffs of the
# type P and dS are rounded to before the second products (fp16 2^-11,
# bf16 2^-9); everything else is fp32.  Measured: about 0.5 u mean and up to
# 1.5 u max.
U = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -9}
TOL = {k: (10 * u, 2 * u) for k, u in U.items()}


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _up(bits, dtype):
    raw = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return raw.view(binding.TORCH_DTYPES[dtype])


def run_bwd(inp):
    q, k, v, _ = binding.to_device(inp)
    do = _up(inp.do, inp.dtype)
    announce("bwd " + inp.describe())
    o, lse = binding.fwd(q, k, v, causal=inp.causal, scale=inp.scale)
    dq, dk, dv, delta = binding.bwd(q, k, v, o, lse, do, causal=inp.causal, scale=inp.scale)
    torch.cuda.synchronize()
    return dq, dk, dv, delta, o


def check_grads(inp, got, heads=None):
    ref = oracle.run_bwd(inp, heads=heads)
    BH = inp.B * inp.H
    hsel = np.arange(BH) if heads is None else np.asarray(heads)
    tmax, tmean = TOL[inp.dtype]
    rec = {"case": "bwd " + inp.describe()}
    msgs = []
    gmax = max(np.abs(r).max() for r in ref)
    gmean = max(np.abs(r).mean() for r in ref)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = g.cpu().numpy().astype(np.float64).reshape(BH, inp.N, inp.d)[hsel]
        assert np.isfinite(g).all(), name
        err = np.abs(g - r)
        mx = err.max() / max(np.abs(r).max(), 0.1 * gmax)
        mn = err.mean() / max(np.abs(r).mean(), 0.1 * gmean)
        rec[name] = [float(mx), float(mn)]
        msgs.append(f"{name} max {mx:.2e} mean {mn:.2e}")
        assert mx <= tmax and mn <= tmean, f"{inp.describe()}: " + ", ".join(msgs)
    announce(inp.describe() + ": " + ", ".join(msgs))
    log = os.environ.get("FA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps(rec) + "\n")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 257])
def test_bwd_small(dtype, d, causal, N):
    inp = inputs.draw_bwd(2, 3, N, d, dtype, causal, seed=3000 + N + d)
    dq, dk, dv, delta, o = run_bwd(inp)
    check_grads(inp, (dq, dk, dv))
    # delta = rowsum(dO * O) against the oracle's O.  The GPU forms it from
    # the forward's O, which meets |O - O_oracle| <= 4e-3 per element and
    # 5e-4 on average, so |delta - D_oracle| <= 4e-3 sum_c |dO_ic| per row
    # (and the mean over rows within 5e-4 of the mean of sum_c |dO_ic|), plus
    # fp32 rounding of a d-term sum.
    dov = (oracle.decode_fp16(inp.do) if dtype == "fp16" else oracle.decode_bf16(inp.do))
    dov = dov.reshape(inp.B * inp.H, inp.N, inp.d)
    o_ref, _ = oracle.run(inp)
    want = (dov * o_ref).sum(-1)
    got = delta.cpu().double().numpy().reshape(inp.B * inp.H, inp.N)
    err = np.abs(got - want)
    absdo = np.abs(dov).sum(-1)
    assert (err <= 4e-3 * absdo + 1e-5).all(), float((err - 4e-3 * absdo).max())
    assert err.mean() <= 5e-4 * absdo.mean() + 1e-6, (float(err.mean()), float(absdo.mean()))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq", range(1, 8))
def test_bwd_every_block_count(d, nq):
    # The dK/dV loop is unrolled four times and runs to a multiple of four
    # blocks: query block counts 1 .. 7 (N = 64 nq - 1, the last block ragged)
    # end on every copy, with zero to three padding blocks, once or twice
    # round the loop.
    N = 64 * nq - 1
    inp = inputs.draw_bwd(1, 2, N, d, "fp16" if nq % 2 else "bf16", False, seed=3200 + nq + d)
    dq, dk, dv, _, _ = run_bwd(inp)
    check_grads(inp, (dq, dk, dv))


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "fp16")])
def test_bwd_causal_tiles_of_every_length(d, dtype):
    # Causal, N = 827: the 128-key tiles start at query blocks 0, 2, .., 12
    # and run 13, 11, 9, 7, 5, 3, 1 blocks (the dK/dV loop pads each to a
    # multiple of four); the 256-query dQ tiles end with masked blocks.
    inp = inputs.draw_bwd(1, 2, 827, d, dtype, True, seed=3300 + d)
    dq, dk, dv, _, _ = run_bwd(inp)
    check_grads(inp, (dq, dk, dv))


@pytest.mark.parametrize("dtype,causal", [("fp16", False), ("bf16", True)])
def test_bwd_medium_sampled_heads(dtype, causal):
    inp = inputs.draw_bwd(1, 8, 1500, 128, dtype, causal, seed=3100)
    dq, dk, dv, _, _ = run_bwd(inp)
    check_grads(inp, (dq, dk, dv), heads=[0, 5])


@pytest.mark.parametrize("B,H,N,dtype,causal,seed,heads", [
    (2, 16, 4096, "fp16", False, 3, [0, 31]),   # the workload bench.py --pass bwd times
    (1, 2, 8192, "bf16", True, 4, [1]),          # the causal workload's N, two of its heads
])
def test_bwd_full_size_sampled_heads(B, H, N, dtype, causal, seed, heads):
    inp = inputs.draw_bwd(B, H, N, 128, dtype, causal, seed=seed)
    dq, dk, dv, _, _ = run_bwd(inp)
    check_grads(inp, (dq, dk, dv), heads=heads)


def test_bwd_rejects_fp8():
    x = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device="cuda")
    lib = binding.load_library()
    f = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device="cuda")
    l = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    st = lib.fa_bwd(x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), l.data_ptr(),
                    x.data_ptr(), f.data_ptr(), f.data_ptr(), f.data_ptr(), l.data_ptr(),
                    1, 1, 64, 64, 0.125, 0, 2, None)
    assert binding.status_string(st) == "unknown dtype"


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_bwd_no_writes_outside_outputs(d, causal):
    # dq, dk, dv and delta carved out of larger buffers holding a sentinel:
    # the row stores of a ragged last tile (N = 333: key groups of 32 rows
    # end at 320 and 352) must leave the guard bands alone.
    inp = inputs.draw_bwd(1, 3, 333, d, "fp16", causal, seed=3400 + d)
    q, k, v, _ = binding.to_device(inp)
    do = _up(inp.do, inp.dtype)
    o, lse = binding.fwd(q, k, v, causal=causal, scale=inp.scale)
    B, H, N = inp.B, inp.H, inp.N
    G = 4096  # guard floats on each side, a multiple of 4: outputs stay 16-byte aligned
    n, nr = B * H * N * d, B * H * N
    bufs = [torch.full((n + 2 * G,), 7.0, dtype=torch.float32, device="cuda") for _ in range(3)]
    dbuf = torch.full((nr + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    dq, dk, dv = (b[G:G + n] for b in bufs)
    delta = dbuf[G:G + nr]
    lib = binding.load_library()
    st = lib.fa_bwd(binding._ptr(q), binding._ptr(k), binding._ptr(v), binding._ptr(o),
                    binding._ptr(lse), binding._ptr(do), binding._ptr(dq), binding._ptr(dk),
                    binding._ptr(dv), binding._ptr(delta), B, H, N, d, inp.scale, int(causal),
                    binding._TORCH_DTYPE_CODE[q.dtype], torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for b in bufs + [dbuf]:
        m = b.numel() - 2 * G
        assert torch.all(b[:G] == 7.0) and torch.all(b[G + m:] == 7.0)
    check_grads(inp, tuple(t.view(B, H, N, d) for t in (dq, dk, dv)))
