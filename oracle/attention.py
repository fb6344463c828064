"""CPU fp64 oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, tables or helpers); the only thing both sides have in common is the
seeded input generator, which holds none of the attention arithmetic.

What it computes, and from which passages:

* Attention output O = softmax(scale * Q K^T [+ causal mask]) V per (b, h).
  The pages describe a method that reaches exactly this function (up to
  rounding order) without ever storing the N x N score matrix:
  - "TCA 51%, MFU 不足 8%" (Zhihu), section "FA2 TCA 虚高归因": online softmax
    accumulates softmax(.)@V block by block instead of materialising [B, L, L];
  - "第 17 章 TMA + Warp Specialization 把 FA2 写到 SOTA", §17.5 (consumer warp
    group): per K/V tile, S = Q K^T, update of the running row max and row
    sum, rescale of the O accumulator, O += P V, and a final division of O by
    the row sum;
  - "Flash Attention CUDA Kernel 优化 ... G4", section "V17: Two Pass PV": the
    per-tile rescale exists only because the running max changes; with the
    global row max fixed first, accumulation is a plain sum.  All of these are
    the same function, so the oracle is that function's definition written
    out, one query row at a time, over all of its keys at once.
* Causal mask (key j kept iff j <= query i), the softmax scale and the LSE
  output are not on the pages; they follow the attention workloads'
  statement.  LSE is the natural-log log-sum-exp of the scaled, unmasked
  scores of a row: LSE_i = m_i + ln(sum_j exp(s_ij - m_i)) with m_i = max_j s_ij.

Readings where the pages are silent:
  * all arithmetic in float64 from the exact input values (fp16 / bf16 widened
    exactly; fp8 value = e4m3 code value x the float32 descale of its head, or
    of its tile of key rows for K and V, both exact in float64);
  * masked scores are -inf; a row whose keys are all masked would have no
    softmax and is reported as O = 0, LSE = -inf (cannot happen with
    N_q == N_k, because the diagonal key is always kept);
  * rows are independent: a chunk of query rows is processed at a time only
    to bound memory, each row still sees all of its keys in one reduction.

* Backward pass (gradients of a loss L given dO = dL/dO): the pages only
  name it (the Zhihu article counts it as recomputation at about 4x the
  forward FLOPs); the oracle takes the chain rule through O = P V,
  P = softmax(S), S = scale * Q K^T written out: dV = P^T dO, dP = dO V^T,
  dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik), dQ = scale dS K, dK = scale dS^T Q.

Pinned by tests/test_oracle_pins.py (40-digit decimal brute force, the
page's streaming recurrence, closed forms, invariants; central finite
differences and invariants of the gradients) and tests/test_oracle_codecs.py
(storage-format decoders).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Storage-format decoders (exact).
# ---------------------------------------------------------------------------


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bits -> float64 (exact widening)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float64.  A bf16 value is the upper half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """OCP 8-bit floating point, E4M3 ("e4m3fn"): bias 7, no infinities,
    0x7F / 0xFF are NaN, largest finite magnitude 448."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes -> float64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# Attention forward, from its definition.
# ---------------------------------------------------------------------------


def _scores(q_rows, k, scale, causal, row_index):
    """s_ij = scale * sum_c q[i, c] k[j, c]; -inf where the causal mask drops j."""
    s = scale * (q_rows @ k.T)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j > row_index[:, None], -np.inf, s)
    return s


def _softmax_rows(s):
    """Row softmax with its log-sum-exp; fully masked rows give p = 0, LSE = -inf."""
    m = np.max(s, axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    l = np.sum(w, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(finite[:, None], w / l[:, None], 0.0)
        lse = np.where(finite, m_safe + np.log(l), -np.inf)
    return p, lse


def attention_probs(q, k, scale, causal):
    """P = softmax(scale * Q K^T [+ mask]) for one head (tiny inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = np.arange(q.shape[0])
    p, _ = _softmax_rows(_scores(q, k, scale, causal, rows))
    return p


def attention_head(q, k, v, scale, causal, rows=None, chunk=256):
    """O [len(rows), d] and LSE [len(rows)] of one head, all float64.

    q, k, v: [N, d] float64.  rows: query indices to compute (default all).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64)
    for a in range(0, rows.shape[0], chunk):
        r = rows[a:a + chunk]
        p, lse[a:a + chunk] = _softmax_rows(_scores(q[r], k, scale, causal, r))
        o[a:a + chunk] = p @ v
    return o, lse


def attention_fwd(q, k, v, scale, causal, rows=None):
    """O [B, H, R, d] and LSE [B, H, R] for float64 Q, K, V of shape [B, H, N, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    R = N if rows is None else len(rows)
    o = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h], v[b, h], scale,
                                                causal, rows)
    return o, lse


# ---------------------------------------------------------------------------
# Attention backward, from the chain rule.
# ---------------------------------------------------------------------------


def _softmax_grad(p, dp):
    """dS = P * (dP - rowsum(P * dP)): the softmax Jacobian applied row by row."""
    return p * (dp - np.sum(p * dp, axis=1)[:, None])


def attention_bwd_head(q, k, v, do, scale, causal, chunk=256):
    """dQ, dK, dV [N, d] float64 of one head, for dO = dL/dO [N, d].

    Chunks of query rows are processed at a time only to bound memory; dK and
    dV sum the contributions of every chunk.
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    n = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a in range(0, n, chunk):
        r = np.arange(a, min(a + chunk, n))
        p, _ = _softmax_rows(_scores(q[r], k, scale, causal, r))
        dv += p.T @ do[r]
        ds = _softmax_grad(p, do[r] @ v.T)
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv


def head_values(inp, b, h):
    """Exact float64 (q, k, v), each [N, d], of head (b, h) of an input set.

    fp8: the value of an element is its e4m3 code value times the float32
    dequantization scale of its (b, h) head, descale_*[b*H + h].  When the
    input set has key tiles (``inp.kv_tile`` = T rows), K and V carry one scale
    per tile of T consecutive rows instead -- the per-block K scale of "第 17 章
    TMA + Warp Specialization 把 FA2 写到 SOTA" §17.7 (item 1), applied to V's
    rows in the same way: row n of head (b, h) takes descale_k[(b*H + h)*nt
    + n // T] with nt = ceil(N / T).  Q keeps its per-head scale.
    """
    if inp.dtype == "fp16":
        dec = decode_fp16
        return dec(inp.q[b, h]), dec(inp.k[b, h]), dec(inp.v[b, h])
    if inp.dtype == "bf16":
        dec = decode_bf16
        return dec(inp.q[b, h]), dec(inp.k[b, h]), dec(inp.v[b, h])
    if inp.dtype == "fp8":
        f = b * inp.H + h
        q = decode_e4m3(inp.q[b, h]) * float(np.float32(inp.descale_q[f]))
        tile = getattr(inp, "kv_tile", None)
        if not tile:
            k = decode_e4m3(inp.k[b, h]) * float(np.float32(inp.descale_k[f]))
            v = decode_e4m3(inp.v[b, h]) * float(np.float32(inp.descale_v[f]))
            return q, k, v
        nt = -(-inp.N // tile)
        row_tile = f * nt + np.arange(inp.N) // tile
        out = [q]
        for codes, ds in ((inp.k, inp.descale_k), (inp.v, inp.descale_v)):
            s = np.asarray(ds, dtype=np.float32).astype(np.float64)[row_tile]
            out.append(decode_e4m3(codes[b, h]) * s[:, None])
        return tuple(out)
    raise ValueError(f"unknown dtype {inp.dtype!r}")


def run(inp, rows=None, heads=None):
    """Oracle result for an input set: (O, LSE) as float64.

    rows: optional query-row indices (same for every head).
    heads: optional list of flat head indices b*H + h (default: all heads in
    order).  The result has shape [len(heads), R, d] and [len(heads), R].
    """
    if heads is None:
        heads = range(inp.B * inp.H)
    outs, lses = [], []
    for f in heads:
        b, h = divmod(int(f), inp.H)
        q, k, v = head_values(inp, b, h)
        o, l = attention_head(q, k, v, float(inp.scale), bool(inp.causal), rows)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def run_bwd(inp, heads=None):
    """Oracle gradients for an input set with dO (inp.do): (dQ, dK, dV) float64,
    each [len(heads), N, d] (heads: flat indices b*H + h, default all)."""
    if inp.dtype not in ("fp16", "bf16"):
        raise ValueError("the backward pass takes fp16 or bf16 inputs")
    dec = decode_fp16 if inp.dtype == "fp16" else decode_bf16
    if heads is None:
        heads = range(inp.B * inp.H)
    out = ([], [], [])
    for f in heads:
        b, h = divmod(int(f), inp.H)
        q, k, v = head_values(inp, b, h)
        g = attention_bwd_head(q, k, v, dec(inp.do[b, h]), float(inp.scale), bool(inp.causal))
        for lst, x in zip(out, g):
            lst.append(x)
    return tuple(np.stack(x) for x in out)
