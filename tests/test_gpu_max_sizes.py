"""The largest problems the library accepts, checked against a closed form.

One head's rows may span at most 2^30 bytes, since buffer offsets are 32-bit,
and N may be at most 2^22. The tests below meet both limits exactly, one
per layout.

Inputs are built on the device from an index pattern. Drawing 2^29 normal
values per tensor on the host would take minutes.

With Q = 0 every score is 0. Row i's output is then the mean of V over the
keys it sees (causal: keys 0..i) and its LSE is ln(i + 1). This is the same
closed form as test_zero_q_gives_mean_of_v, at the other end of the size
range.

V[j, c] = (((37 j + 11 c + 5 h) mod 17) - 8) / 16 is exact in fp16. It
sums to 0 over any 17 consecutive keys: 37 = 3 mod 17 is prime to 17, so
those keys take every residue once. A prefix sum is therefore a short loop
over the last partial period, and a wrong row offset anywhere in the span
moves some row's mean.
"""
import numpy as np
import pytest
import torch

from attention_forward_fa_amd import binding
from tests.test_gpu_parity import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _v_pattern(N, H, d, layout):
    """fp16 V of the index pattern, [1, H, N, d] or [1, N, H, d], made on the GPU."""
    j = torch.arange(N, device="cuda", dtype=torch.int32)
    h = torch.arange(H, device="cuda", dtype=torch.int32)
    c = torch.arange(d, device="cuda", dtype=torch.int32)
    if layout == "bhnd":
        idx = 37 * j[None, None, :, None] + 11 * c[None, None, None, :] + 5 * h[None, :, None, None]
    else:
        idx = 37 * j[None, :, None, None] + 11 * c[None, None, None, :] + 5 * h[None, None, :, None]
    return ((idx % 17) - 8).to(torch.float16) / 16


def _prefix_mean(i, h, d):
    """Mean over keys 0..i of V[., c] for head h, c = 0..d-1 (whole periods sum to 0)."""
    n = i + 1
    js = np.arange(n - n % 17, n)
    c = np.arange(d)
    vals = (((37 * js[:, None] + 11 * c[None, :] + 5 * h) % 17) - 8) / 16.0
    return vals.sum(axis=0) / n


def _rows(N, seed):
    fixed = [0, 1, 15, 16, 17, 18, 63, 64, 255, 256, 257, N // 2, N - 257, N - 256, N - 65,
             N - 64, N - 2, N - 1]
    rand = np.random.default_rng(seed).integers(0, N, size=16)
    return np.unique(np.concatenate([fixed, rand]))


def _check(o_bhnd, lse, N, heads, d, seed):
    """o_bhnd: [H, N, d] fp16 on the device; lse: [H, N] fp32 on the device."""
    expect_l = np.log(np.arange(1, N + 1, dtype=np.float64))
    l = lse.double().cpu().numpy()
    assert np.abs(l - expect_l[None, :]).max() <= 1e-3
    rows = _rows(N, seed)
    rows_t = torch.from_numpy(rows).to("cuda")
    for h in heads:
        got = o_bhnd[h].index_select(0, rows_t).double().cpu().numpy()
        want = np.stack([_prefix_mean(int(i), h, d) for i in rows])
        err = float(np.abs(got - want).max())
        announce(f"max size head {h}: max|dO| over {len(rows)} rows = {err:.3e}")
        assert err <= 4e-3, (h, err)


def test_max_head_span_bnhd():
    # [B, N, H, d] = [1, 2^19, 16, 64] fp16: one head's rows span
    # N * H * d * 2 = 2^30 bytes, causal.
    N, H, d = 1 << 19, 16, 64
    announce(f"max head span bnhd N={N} H={H} d={d} causal")
    v = _v_pattern(N, H, d, "bnhd")
    q = torch.zeros_like(v)
    k = torch.zeros_like(v)
    o, lse = binding.fwd_ex(q, k, v, layout="bnhd", causal=True)
    torch.cuda.synchronize()
    del q, k, v
    _check(o[0].permute(1, 0, 2), lse[0], N, [0, 7, 15], d, seed=31)


def test_max_head_span_bnhd_fp8():
    # fp8 e4m3 [B, N, H, d] = [1, 2^19, 16, 128] (unit descales): one head's
    # rows span N * H * d = 2^30 bytes; a grid of 8-wave workgroups (P V in
    # fp16), causal.  Every multiple of 1/16 up to 1/2 is an e4m3 value.
    N, H, d = 1 << 19, 16, 128
    announce(f"max head span bnhd fp8 N={N} H={H} d={d} causal")
    v = _v_pattern(N, H, d, "bnhd").to(torch.float8_e4m3fn)
    q = torch.zeros(v.shape, dtype=torch.float8_e4m3fn, device="cuda")
    k = torch.zeros(v.shape, dtype=torch.float8_e4m3fn, device="cuda")
    o, lse = binding.fwd_ex(q, k, v, layout="bnhd", causal=True)
    torch.cuda.synchronize()
    del q, k, v
    _check(o[0].permute(1, 0, 2), lse[0], N, [0, 9, 15], d, seed=34)


def test_max_sequence_bhnd():
    # [B, H, N, d] = [1, 1, 2^22, 128] fp16: N at its limit, one head's rows
    # span N * d * 2 = 2^30 bytes, causal.
    N, H, d = 1 << 22, 1, 128
    announce(f"max sequence bhnd N={N} H={H} d={d} causal")
    v = _v_pattern(N, H, d, "bhnd")
    q = torch.zeros_like(v)
    k = torch.zeros_like(v)
    o, lse = binding.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    del q, k, v
    _check(o[0], lse[0], N, [0], d, seed=32)


def test_max_sequence_backward():
    # fa_bwd at N = 2^22 ([1, 1, 2^22, 64] fp16, causal; dV spans 2^30 bytes
    # of fp32).  With Q = K = 0 every P_ij is 1/(i + 1) for j <= i, dQ and dK
    # are exactly 0 (each is a sum of terms times K or Q), and
    # dV_j = sum_{i >= j} dO_i / (i + 1), computed here in fp64 from the end.
    # dO[i, c] = (((29 i + 7 c) mod 13) - 6) / 16 (exact in fp16).  P enters
    # dV rounded to fp16 (relative error <= 2^-11 each), so
    # |dV_j - exact| <= 2^-11 sum_{i >= j} |dO_i| / (i + 1) + fp32 summation;
    # the test allows twice the first term plus 1e-5.
    N, d = 1 << 22, 64
    announce(f"max sequence backward N={N} d={d} causal")
    v = _v_pattern(N, 1, d, "bhnd")
    q = torch.zeros_like(v)
    k = torch.zeros_like(v)
    i = torch.arange(N, device="cuda", dtype=torch.int32)[None, None, :, None]
    c = torch.arange(d, device="cuda", dtype=torch.int32)[None, None, None, :]
    do = (((29 * i + 7 * c) % 13) - 6).to(torch.float16) / 16
    o, lse = binding.fwd(q, k, v, causal=True)
    dq, dk, dv, _ = binding.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dq)) == 0 and int(torch.count_nonzero(dk)) == 0
    ii = np.arange(N, dtype=np.int64)
    w = 1.0 / (ii + 1.0)
    rows = _rows(N, seed=33)
    rows_t = torch.from_numpy(rows).to("cuda")
    got = dv[0, 0].index_select(0, rows_t).double().cpu().numpy()
    worst = 0.0
    sums = {}  # column c depends on c only through 7 c mod 13
    for col in range(d):
        key = (7 * col) % 13
        if key not in sums:
            g = ((((29 * ii + key) % 13) - 6) / 16.0) * w
            sums[key] = (np.cumsum(g[::-1])[::-1][rows],
                         2.0 * 2.0 ** -11 * np.cumsum(np.abs(g)[::-1])[::-1][rows] + 1e-5)
        exact, bound = sums[key]
        err = np.abs(got[:, col] - exact)
        worst = max(worst, float((err / bound).max()))
        assert (err <= bound).all(), (col, float(err.max()), float(bound.min()))
    announce(f"max sequence backward: max |dV - exact| / bound = {worst:.3f}")
