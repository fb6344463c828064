"""The oracle against its pins, and planted oracle mistakes against the pins."""
import math

import numpy as np
import pytest

from oracle import attention as A
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# --- mutation check: each planted mistake must trip at least one pin -------

_orig_scores = A._scores
_orig_softmax = A._softmax_rows
_orig_head = A.attention_head


def _scores_no_scale(q_rows, k, scale, causal, row_index):
    return _orig_scores(q_rows, k, 1.0, causal, row_index)


def _scores_mask_diag(q_rows, k, scale, causal, row_index):
    s = scale * (q_rows @ k.T)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j >= row_index[:, None], -np.inf, s)
    return s


def _scores_mask_flipped(q_rows, k, scale, causal, row_index):
    s = scale * (q_rows @ k.T)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j < row_index[:, None], -np.inf, s)
    return s


def _scores_sqrt_scale(q_rows, k, scale, causal, row_index):
    return _orig_scores(q_rows, k, math.sqrt(scale), causal, row_index)


def _softmax_no_max(s):
    w = np.exp(s)
    l = w.sum(axis=1)
    return w / l[:, None], np.log(l)


def _softmax_exp_sign(s):
    m = np.max(s, axis=1)
    w = np.exp(m[:, None] - s)
    w = np.where(np.isfinite(s), w, 0.0)
    l = w.sum(axis=1)
    return w / l[:, None], m + np.log(l)


def _softmax_no_division(s):
    p, lse = _orig_softmax(s)
    m = np.max(s, axis=1)
    return np.exp(s - m[:, None]), lse


def _softmax_lse_without_max(s):
    p, lse = _orig_softmax(s)
    m = np.max(s, axis=1)
    return p, lse - m


def _softmax_lse_log2(s):
    m = np.max(s, axis=1)
    w = np.exp(s - m[:, None])
    l = w.sum(axis=1)
    return w / l[:, None], m + np.log2(l)


def _head_value_rows_reversed(q, k, v, scale, causal, rows=None, chunk=256):
    return _orig_head(q, k, np.asarray(v)[::-1].copy(), scale, causal, rows, chunk)


def _head_qk_swapped(q, k, v, scale, causal, rows=None, chunk=256):
    return _orig_head(k, q, v, scale, causal, rows, chunk)


_orig_bwd = A.attention_bwd_head


def _softmax_grad_no_rowsum(p, dp):
    return p * dp


def _softmax_grad_sign(p, dp):
    return p * (np.sum(p * dp, axis=1)[:, None] - dp)


def _bwd_dk_unscaled(q, k, v, do, scale, causal, chunk=256):
    dq, dk, dv = _orig_bwd(q, k, v, do, scale, causal, chunk)
    return dq, dk / scale, dv


def _bwd_dq_dk_swapped(q, k, v, do, scale, causal, chunk=256):
    dq, dk, dv = _orig_bwd(q, k, v, do, scale, causal, chunk)
    return dk, dq, dv


_orig_head_values = A.head_values


def _head_values_index_transposed(inp, b, h):
    # descales of head (b, h) looked up at h*B + b instead of b*H + h
    if inp.dtype != "fp8":
        return _orig_head_values(inp, b, h)
    import copy
    alt = copy.copy(inp)
    perm = np.array([hh * inp.B + bb for bb in range(inp.B) for hh in range(inp.H)])
    nt = -(-inp.N // inp.kv_tile) if inp.kv_tile else 1
    alt.descale_q = np.asarray(inp.descale_q)[perm]
    rows = (perm[:, None] * nt + np.arange(nt)[None, :]).reshape(-1)
    alt.descale_k = np.asarray(inp.descale_k)[rows]
    alt.descale_v = np.asarray(inp.descale_v)[rows]
    return _orig_head_values(alt, b, h)


def _head_values_tile_modulo(inp, b, h):
    # key tile of row n taken as n % nt instead of n // kv_tile
    if inp.dtype != "fp8" or not inp.kv_tile:
        return _orig_head_values(inp, b, h)
    q, _, _ = _orig_head_values(inp, b, h)
    nt = -(-inp.N // inp.kv_tile)
    f = b * inp.H + h
    idx = f * nt + np.arange(inp.N) % nt
    k = A.decode_e4m3(inp.k[b, h]) * np.asarray(inp.descale_k, np.float64)[idx][:, None]
    v = A.decode_e4m3(inp.v[b, h]) * np.asarray(inp.descale_v, np.float64)[idx][:, None]
    return q, k, v


def _head_values_v_scale_on_k(inp, b, h):
    # V's scale applied to K and K's to V
    q, k, v = _orig_head_values(inp, b, h)
    if inp.dtype != "fp8":
        return q, k, v
    alt = __import__("copy").copy(inp)
    alt.descale_k, alt.descale_v = inp.descale_v, inp.descale_k
    return _orig_head_values(alt, b, h)


MUTANTS = [
    ("head_values", _head_values_index_transposed),
    ("head_values", _head_values_tile_modulo),
    ("head_values", _head_values_v_scale_on_k),
    ("_scores", _scores_no_scale),
    ("_scores", _scores_sqrt_scale),
    ("_scores", _scores_mask_diag),
    ("_scores", _scores_mask_flipped),
    ("_softmax_rows", _softmax_no_max),
    ("_softmax_rows", _softmax_exp_sign),
    ("_softmax_rows", _softmax_no_division),
    ("_softmax_rows", _softmax_lse_without_max),
    ("_softmax_rows", _softmax_lse_log2),
    ("attention_head", _head_value_rows_reversed),
    ("attention_head", _head_qk_swapped),
    ("_softmax_grad", _softmax_grad_no_rowsum),
    ("_softmax_grad", _softmax_grad_sign),
    ("attention_bwd_head", _bwd_dk_unscaled),
    ("attention_bwd_head", _bwd_dq_dk_swapped),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda x: getattr(x, "__name__", x))
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(A, name, mutant)
    caught = []
    with np.errstate(all="ignore"):
        for pin in P.PINS:
            try:
                pin()
            except Exception as e:  # noqa: BLE001 - any failure counts as caught
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"planted mistake {mutant.__name__} passed every pin"
