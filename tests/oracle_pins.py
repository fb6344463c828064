"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function raises AssertionError on failure.  They are run as
tests in test_oracle_pins.py, and again against deliberately broken copies of
the oracle (mistakes planted on the CPU) to show that each plausible mistake
trips at least one of them.

Independent references used here:
  * a 40-digit ``decimal`` brute force written with explicit loops;
  * the streaming recurrence the pages describe (running row max and row sum,
    rescale of the accumulator by exp(m_old - m_new), final division by the
    row sum) -- "第 17 章 TMA + Warp Specialization 把 FA2 写到 SOTA" §17.5;
  * the two-pass variant with the global row max fixed first --
    "Flash Attention CUDA Kernel 优化 ... G4", section "V17: Two Pass PV";
  * closed forms and invariants of softmax attention.
"""
from __future__ import annotations

import decimal
import math

import numpy as np
import torch

from oracle import attention as A


def _f16(x):
    """Round a float array to fp16-representable values (input construction)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


def _rand(shape, seed, s=1.0):
    g = torch.Generator().manual_seed(seed)
    return _f16(torch.randn(shape, generator=g).numpy() * s)


def _close(a, b, atol, rtol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    bad = ~(np.abs(a - b) <= atol + rtol * np.abs(b))
    assert not bad.any(), f"{what}: max |diff| = {np.nanmax(np.abs(a - b))}"


# ---------------------------------------------------------------------------
# Independent references.
# ---------------------------------------------------------------------------


def decimal_attention(q, k, v, scale, causal, prec=40):
    """O and LSE with 40-digit decimal arithmetic and explicit loops."""
    ctx = decimal.Context(prec=prec)
    D = decimal.Decimal
    n, d = len(q), len(q[0])
    sc = D(float(scale))
    O, L = [], []
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        s = []
        for j in keys:
            acc = D(0)
            for c in range(d):
                acc = ctx.add(acc, ctx.multiply(D(float(q[i][c])), D(float(k[j][c]))))
            s.append(ctx.multiply(sc, acc))
        m = max(s)
        w = [ctx.exp(ctx.subtract(x, m)) for x in s]
        lsum = D(0)
        for x in w:
            lsum = ctx.add(lsum, x)
        row = []
        for c in range(len(v[0])):
            acc = D(0)
            for wj, j in zip(w, keys):
                acc = ctx.add(acc, ctx.multiply(wj, D(float(v[j][c]))))
            row.append(float(ctx.divide(acc, lsum)))
        O.append(row)
        L.append(float(ctx.add(m, ctx.ln(lsum))))
    return np.array(O), np.array(L)


def streaming_attention(q, k, v, scale, causal, bc):
    """The pages' per-K/V-tile recurrence, float64, tiles of ``bc`` keys.

    Tiles wholly above the diagonal are skipped under the causal mask.
    """
    n, dv = q.shape[0], v.shape[1]
    O = np.zeros((n, dv))
    L = np.zeros(n)
    for i in range(n):
        m, l, acc = -math.inf, 0.0, np.zeros(dv)
        last = i if causal else n - 1
        for j0 in range(0, last + 1, bc):
            j1 = min(j0 + bc, last + 1)
            s = scale * (k[j0:j1] @ q[i])
            m_new = max(m, float(s.max()))
            alpha = math.exp(m - m_new) if m != -math.inf else 0.0
            p = np.exp(s - m_new)
            l = alpha * l + float(p.sum())
            acc = alpha * acc + p @ v[j0:j1]
            m = m_new
        O[i] = acc / l
        L[i] = m + math.log(l)
    return O, L


def two_pass_attention(q, k, v, scale, causal, bc):
    """Pass 1 finds each row's global max, pass 2 accumulates with it fixed."""
    n, dv = q.shape[0], v.shape[1]
    O = np.zeros((n, dv))
    L = np.zeros(n)
    for i in range(n):
        last = i if causal else n - 1
        m = -math.inf
        for j0 in range(0, last + 1, bc):
            m = max(m, float((scale * (k[j0:last + 1][:bc] @ q[i])).max()))
        l, acc = 0.0, np.zeros(dv)
        for j0 in range(0, last + 1, bc):
            j1 = min(j0 + bc, last + 1)
            p = np.exp(scale * (k[j0:j1] @ q[i]) - m)
            l += float(p.sum())
            acc += p @ v[j0:j1]
        O[i] = acc / l
        L[i] = m + math.log(l)
    return O, L


# ---------------------------------------------------------------------------
# Pins.
# ---------------------------------------------------------------------------


def pin_decimal_bruteforce():
    for seed, (n, d, causal) in enumerate([(5, 4, False), (7, 8, True), (8, 3, False),
                                           (1, 4, False), (6, 6, True)]):
        q, k, v = (_rand((n, d), 100 + 3 * seed + t) for t in range(3))
        scale = float(np.float32(1.0 / math.sqrt(d)))
        O, L = A.attention_head(q, k, v, scale, causal)
        Od, Ld = decimal_attention(q, k, v, scale, causal)
        _close(O, Od, 1e-13, 1e-13, f"O vs decimal n={n} d={d} causal={causal}")
        _close(L, Ld, 1e-13, 1e-13, f"LSE vs decimal n={n} d={d} causal={causal}")


def pin_decimal_large_scores():
    # Scores up to ~60: the max subtraction must keep exp() finite.
    n, d = 6, 4
    q, k, v = _rand((n, d), 7, 4.0), _rand((n, d), 8, 4.0), _rand((n, d), 9)
    O, L = A.attention_head(q, k, v, 2.0, False)
    Od, Ld = decimal_attention(q, k, v, 2.0, False)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    _close(O, Od, 1e-12, 1e-12, "O, large scores")
    _close(L, Ld, 1e-12, 1e-12, "LSE, large scores")


def pin_streaming_recurrence():
    n, d = 150, 16
    q, k, v = (_rand((n, d), 200 + t) for t in range(3))
    scale = 0.25
    for causal in (False, True):
        O, L = A.attention_head(q, k, v, scale, causal)
        for bc in (1, 7, 64):
            Os, Ls = streaming_attention(q, k, v, scale, causal, bc)
            _close(O, Os, 1e-12, 0, f"O vs streaming bc={bc} causal={causal}")
            _close(L, Ls, 1e-12, 1e-12, f"LSE vs streaming bc={bc} causal={causal}")


def pin_two_pass():
    n, d = 97, 8
    q, k, v = (_rand((n, d), 300 + t) for t in range(3))
    for causal in (False, True):
        O, L = A.attention_head(q, k, v, 0.3, causal)
        Ot, Lt = two_pass_attention(q, k, v, 0.3, causal, 16)
        _close(O, Ot, 1e-12, 0, f"O vs two-pass causal={causal}")
        _close(L, Lt, 1e-12, 1e-12, f"LSE vs two-pass causal={causal}")


def pin_probabilities():
    n, d = 33, 8
    q, k = _rand((n, d), 400), _rand((n, d), 401)
    for causal in (False, True):
        P = A.attention_probs(q, k, 0.5, causal)
        assert (P >= 0).all()
        _close(P.sum(axis=1), np.ones(n), 1e-14, 0, "P rows sum to 1")
        if causal:
            assert np.all(np.triu(P, 1) == 0), "causal P must vanish above the diagonal"
            assert P[0, 0] == 1.0


def pin_constant_v():
    n, d = 40, 8
    q, k = _rand((n, d), 500), _rand((n, d), 501)
    for c in (1.5, -3.25):
        v = np.full((n, d), c)
        for causal in (False, True):
            O, _ = A.attention_head(q, k, v, 0.7, causal)
            _close(O, np.full((n, d), c), 1e-13, 0, "constant V gives O = c")


def pin_zero_q():
    n, d = 37, 8
    q = np.zeros((n, d))
    k, v = _rand((n, d), 600), _rand((n, d), 601)
    O, L = A.attention_head(q, k, v, 0.9, False)
    _close(O, np.tile(v.mean(axis=0), (n, 1)), 1e-13, 0, "Q=0: O = mean of V")
    _close(L, np.full(n, math.log(n)), 1e-13, 0, "Q=0: LSE = ln N")
    O, L = A.attention_head(q, k, v, 0.9, True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    _close(O, prefix, 1e-13, 0, "Q=0 causal: O_i = mean of V[0..i]")
    _close(L, np.log(np.arange(1, n + 1)), 1e-13, 0, "Q=0 causal: LSE_i = ln(i+1)")


def pin_causal_first_row_and_prefix():
    n, d = 29, 8
    q, k, v = (_rand((n, d), 700 + t) for t in range(3))
    scale = 0.4
    O, L = A.attention_head(q, k, v, scale, True)
    assert np.array_equal(O[0], v[0]), "causal row 0 is exactly V[0]"
    _close(L[0], scale * float(q[0] @ k[0]), 1e-14, 1e-14, "causal row 0 LSE")
    for i in (1, 5, n - 1):
        Op, Lp = A.attention_head(q[: i + 1], k[: i + 1], v[: i + 1], scale, False)
        _close(O[i], Op[i], 1e-13, 0, f"causal row {i} = attention over prefix")
        _close(L[i], Lp[i], 1e-13, 0, f"causal LSE row {i}")


def pin_two_keys():
    # With two keys, O = sigma v0 + (1 - sigma) v1, sigma = 1 / (1 + e^(s1 - s0)).
    q = np.array([[1.0, 2.0]])
    k = np.array([[0.5, -1.0], [2.0, 0.25]])
    v = np.array([[3.0, -1.0], [-2.0, 4.0]])
    scale = 0.75
    s0, s1 = scale * float(q[0] @ k[0]), scale * float(q[0] @ k[1])
    sig = 1.0 / (1.0 + math.exp(s1 - s0))
    O, L = A.attention_head(np.vstack([q, q]), k, v, scale, False)
    _close(O[0], sig * v[0] + (1 - sig) * v[1], 1e-15, 1e-15, "two-key softmax")
    _close(L[0], math.log(math.exp(s0) + math.exp(s1)), 1e-15, 1e-15, "two-key LSE")


def pin_one_hot_keys():
    # Orthogonal keys k_j = lam e_j and q_i = lam e_i: s_ii = scale lam^2, s_ij = 0.
    n = d = 12
    lam, scale = 3.0, 0.5
    k = lam * np.eye(n)
    q = lam * np.eye(n)
    v = _rand((n, 5), 800)
    O, L = A.attention_head(q, k, v, scale, False)
    a = scale * lam * lam
    ea = math.exp(a)
    expect = (ea * v + (v.sum(axis=0)[None, :] - v)) / (ea + n - 1)
    _close(O, expect, 1e-13, 0, "one-hot keys closed form")
    _close(L, np.full(n, math.log(ea + n - 1)), 1e-13, 0, "one-hot keys LSE")


def pin_key_shift():
    n, d = 31, 8
    q, k, v = (_rand((n, d), 900 + t) for t in range(3))
    u = _rand((d,), 903)
    scale = 0.6
    for causal in (False, True):
        O, L = A.attention_head(q, k, v, scale, causal)
        O2, L2 = A.attention_head(q, k + u[None, :], v, scale, causal)
        _close(O2, O, 1e-12, 0, "key shift leaves O unchanged")
        _close(L2, L + scale * (q @ u), 1e-12, 0, "key shift moves LSE by scale q.u")


def pin_joint_permutation():
    n, d = 45, 8
    q, k, v = (_rand((n, d), 1000 + t) for t in range(3))
    perm = np.random.default_rng(5).permutation(n)
    O, L = A.attention_head(q, k, v, 0.5, False)
    O2, L2 = A.attention_head(q, k[perm], v[perm], 0.5, False)
    _close(O2, O, 1e-13, 0, "key/value permutation")
    _close(L2, L, 1e-13, 0, "key/value permutation LSE")


def pin_score_overflow_stress():
    # Scores reach ~1e3, beyond where exp() overflows even in float64, so the
    # row max must be subtracted before exponentiating.
    n, d = 64, 16
    q, k, v = (_rand((n, d), 1100 + t) for t in range(3))
    for causal in (False, True):
        O, L = A.attention_head(q, k, v, 100.0, causal)
        assert np.isfinite(O).all() and np.isfinite(L).all()
        assert np.abs(L).max() > 750.0
        Os, Ls = streaming_attention(q, k, v, 100.0, causal, 16)
        _close(O, Os, 1e-11, 0, "x30 scores vs streaming")
        _close(L, Ls, 1e-11, 1e-13, "x30 LSE vs streaming")


def pin_fwd_layout():
    # attention_fwd handles [B, H, N, d] head by head, rows selects query rows.
    B, H, n, d = 2, 3, 20, 4
    q, k, v = (_rand((B, H, n, d), 1200 + t) for t in range(3))
    O, L = A.attention_fwd(q, k, v, 0.5, True)
    rows = np.array([0, 3, 19])
    Or, Lr = A.attention_fwd(q, k, v, 0.5, True, rows=rows)
    for b in range(B):
        for h in range(H):
            Oh, Lh = decimal_attention(q[b, h], k[b, h], v[b, h], 0.5, True)
            _close(O[b, h], Oh, 1e-13, 1e-13, f"fwd O head {b},{h}")
            _close(L[b, h], Lh, 1e-13, 1e-13, f"fwd LSE head {b},{h}")
            _close(Or[b, h], Oh[rows], 1e-13, 1e-13, "row subset O")
            _close(Lr[b, h], Lh[rows], 1e-13, 1e-13, "row subset LSE")


def pin_lse_merge():
    # Attention over a key set split into parts merges exactly from the
    # parts' outputs: LSE = ln sum_g exp(LSE_g), O = sum_g exp(LSE_g - LSE) O_g.
    # This is the exchange a sequence split over several GPUs would use, and
    # it holds only if LSE is the natural-log sum of exp of the scaled scores.
    n, m, d = 37, 53, 8
    q = _rand((n, d), 1300)
    k, v = _rand((m, d), 1301), _rand((m, d), 1302)
    O, L = A.attention_head(q, k, v, 0.7, False)
    cuts = [0, 11, 30, m]
    parts = [A.attention_head(q, k[a:b], v[a:b], 0.7, False) for a, b in zip(cuts, cuts[1:])]
    Lm = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    Om = sum(np.exp(p[1] - Lm)[:, None] * p[0] for p in parts)
    _close(Lm, L, 1e-12, 1e-14, "merged LSE")
    _close(Om, O, 1e-12, 0, "merged O")


def _loss(q, k, v, do, scale, causal):
    O, _ = A.attention_head(q, k, v, scale, causal)
    return float(np.sum(do * O))


def pin_bwd_finite_differences():
    # Gradients of L = sum(dO * O) against central differences of the
    # (separately pinned) forward: h = 1e-5 in float64 leaves ~1e-9 of
    # truncation and rounding error.
    n, d, h = 6, 3, 1e-5
    q, k, v, do = (_rand((n, d), 1400 + t) for t in range(4))
    for causal in (False, True):
        dq, dk, dv = A.attention_bwd_head(q, k, v, do, 0.8, causal)
        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                key = name[1].lower()
                args_p[key], args_m[key] = xp, xm
                fd[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, 0.8, causal)
                           - _loss(args_m["q"], args_m["k"], args_m["v"], do, 0.8, causal)) / (2 * h)
            _close(g, fd, 1e-7, 0, f"{name} vs finite differences (causal={causal})")


def pin_bwd_invariants():
    # Shifting every key by u leaves each row's softmax unchanged, so
    # sum_j dK_j = 0; rows of P sum to 1, so sum_j dV_j = sum_i dO_i; scaling
    # Q by t is scaling S by t, as is scaling K, so sum dQ*Q = sum dK*K.
    n, d = 40, 8
    q, k, v, do = (_rand((n, d), 1500 + t) for t in range(4))
    for causal in (False, True):
        dq, dk, dv = A.attention_bwd_head(q, k, v, do, 0.6, causal)
        _close(dk.sum(axis=0), np.zeros(d), 1e-12, 0, "sum of dK")
        _close(dv.sum(axis=0), do.sum(axis=0), 1e-12, 0, "sum of dV")
        _close(np.sum(dq * q), np.sum(dk * k), 1e-11, 0, "dQ.Q = dK.K")


def pin_bwd_closed_forms():
    n, d = 30, 4
    q, k, v, do = (_rand((n, d), 1600 + t) for t in range(4))
    # Constant V: O does not depend on the scores, so dQ = dK = 0.
    vc = np.full((n, d), 0.75)
    for causal in (False, True):
        dq, dk, dv = A.attention_bwd_head(q, k, vc, do, 0.5, causal)
        _close(dq, np.zeros_like(dq), 1e-13, 0, "constant V: dQ")
        _close(dk, np.zeros_like(dk), 1e-13, 0, "constant V: dK")
    # Causal: row 0 sees key 0 alone (its softmax is constant: dQ_0 = 0), and
    # the last key is seen by the last row alone: dV_{N-1} = P_{N-1,N-1} dO_{N-1}.
    dq, dk, dv = A.attention_bwd_head(q, k, v, do, 0.5, True)
    _close(dq[0], np.zeros(d), 1e-14, 0, "causal row 0: dQ")
    s = 0.5 * (k[: n] @ q[n - 1])
    p_last = np.exp(s[n - 1] - s.max()) / np.sum(np.exp(s - s.max()))
    _close(dv[n - 1], p_last * do[n - 1], 1e-13, 0, "causal last key: dV")


def _fp8_input(B, H, N, d, seed, kv_tile=None):
    """An fp8 input set with random codes (NaN codes avoided) and distinct,
    non-power-of-two float32 descales per head (or per key tile for K, V)."""
    from attention_forward_fa_amd import inputs as I
    rng = np.random.default_rng(seed)

    def codes():
        c = rng.integers(0, 256, size=(B, H, N, d), dtype=np.uint8)
        return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)

    nt = -(-N // kv_tile) if kv_tile else 1
    ds_q = np.float32(1e-3) * (1 + np.arange(B * H, dtype=np.float32) * np.float32(0.37))
    ds_k = np.float32(7e-4) * (1 + np.arange(B * H * nt, dtype=np.float32) * np.float32(0.29))
    ds_v = np.float32(3e-3) * (1 + np.arange(B * H * nt, dtype=np.float32) * np.float32(0.53))
    return I.AttnInputs(B, H, N, d, "fp8", False, float(np.float32(0.5)), codes(), codes(),
                        codes(), ds_q.astype(np.float32), ds_k.astype(np.float32),
                        ds_v.astype(np.float32), seed, kv_tile=kv_tile)


def _fp8_values_independent(inp):
    """Dequantized Q, K, V [B][H][N][d] as nested lists: codes decoded by torch's
    float8_e4m3fn conversion, times the scale looked up element by element."""
    dec = [torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn)
           .to(torch.float64).numpy() for c in (inp.q, inp.k, inp.v)]
    nt = -(-inp.N // inp.kv_tile) if inp.kv_tile else 1
    out = []
    for which, (x, ds) in enumerate(zip(dec, (inp.descale_q, inp.descale_k, inp.descale_v))):
        t = [[[[0.0] * inp.d for _ in range(inp.N)] for _ in range(inp.H)] for _ in range(inp.B)]
        for b in range(inp.B):
            for h in range(inp.H):
                for n in range(inp.N):
                    if which > 0 and inp.kv_tile:
                        sc = float(ds[(b * inp.H + h) * nt + n // inp.kv_tile])
                    else:
                        sc = float(ds[b * inp.H + h])
                    for c in range(inp.d):
                        t[b][h][n][c] = float(x[b, h, n, c]) * sc
        out.append(t)
    return out


def pin_fp8_dequantization():
    # The fp8 path (codes x float32 scales): B = 2, H = 3 with a scale of its
    # own for every head -- and, with key tiles of 2 rows, for every K / V
    # tile -- against the 40-digit brute force on values decoded and scaled
    # independently of the oracle.  A head index taken as h*B + b, a tile index
    # taken modulo the tile count, or a scale on the wrong tensor, moves O.
    for kv_tile in (None, 2):
        inp = _fp8_input(2, 3, 5, 4, 1700 + (kv_tile or 0), kv_tile)
        O, L = A.run(inp)
        qv, kv, vv = _fp8_values_independent(inp)
        for b in range(inp.B):
            for h in range(inp.H):
                Od, Ld = decimal_attention(qv[b][h], kv[b][h], vv[b][h], inp.scale, False)
                f = b * inp.H + h
                _close(O[f], Od, 1e-12, 1e-12, f"fp8 O head {b},{h} kv_tile={kv_tile}")
                _close(L[f], Ld, 1e-12, 1e-12, f"fp8 LSE head {b},{h} kv_tile={kv_tile}")


PINS = [
    pin_decimal_bruteforce,
    pin_decimal_large_scores,
    pin_streaming_recurrence,
    pin_two_pass,
    pin_probabilities,
    pin_constant_v,
    pin_zero_q,
    pin_causal_first_row_and_prefix,
    pin_two_keys,
    pin_one_hot_keys,
    pin_key_shift,
    pin_joint_permutation,
    pin_score_overflow_stress,
    pin_fwd_layout,
    pin_lse_merge,
    pin_fp8_dequantization,
    pin_bwd_finite_differences,
    pin_bwd_invariants,
    pin_bwd_closed_forms,
]
