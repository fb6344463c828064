"""Thin ctypes binding of libfa_mi355x.so (include/fa_mi355x.h).

Argument marshalling only: every step of the attention forward pass runs in
the library's HIP kernels.  torch supplies device memory and the current
stream.  There is no fallback: if the library is missing or refuses the call,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

from .build import LIB_PATH

FA_DTYPE_FP16 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_FP8_E4M3 = 2
_TORCH_DTYPE_CODE = {
    torch.float16: FA_DTYPE_FP16,
    torch.bfloat16: FA_DTYPE_BF16,
    torch.float8_e4m3fn: FA_DTYPE_FP8_E4M3,
}

# Exported symbols, with their C signatures.
_I64 = ctypes.c_int64
_P = ctypes.c_void_p
SIGNATURES = {
    "fa_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                              ctypes.c_int, ctypes.c_int, _P]),
    "fa_fwd_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                  ctypes.c_float, ctypes.c_int, _P]),
    "fa_fwd_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                 ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]),
    "fa_fwd_fp8_pv": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_int, _I64, _P]),
    "fa_fwd_fp8_kvtile": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                         ctypes.c_float, ctypes.c_int, ctypes.c_int, _I64, _P]),
    "fa_fwd_kvsplit_workspace": (ctypes.c_int64, [_I64, _I64, _I64, _I64, ctypes.c_int,
                                                   ctypes.c_int]),
    "fa_fwd_kvsplit": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                      ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _P, _I64, _P]),
    "fa_fwd_kvsplit_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                              _I64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _P]),
    "fa_fwd_kvsplit_noalloc_max_bytes": (ctypes.c_int64, []),
    "fa_fwd_fp8_pv_kvsplit": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                             _I64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                             _I64, _P, _I64, _P]),
    "fa_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                              ctypes.c_float, ctypes.c_int, ctypes.c_int, _P]),
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_abi_version": (ctypes.c_int, []),
}

_lib = None
_lock = threading.Lock()


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fa_mi355x status {status}: {message}")
        self.status = status


def load_library(path: Optional[str] = None):
    """Load libfa_mi355x.so (built in-tree by attention_forward_fa_amd.build)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        # FA_MI355X_LIBRARY names an alternative build of the same library.
        p = path or os.environ.get("FA_MI355X_LIBRARY") or LIB_PATH
        if not os.path.exists(p):
            raise FileNotFoundError(
                f"{p} is missing: build it first (python -m attention_forward_fa_amd.build)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise FAError(status, status_string(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


LAYOUTS = {"bhnd": 0, "bnhd": 1}


def _validate(q, k, v):
    if not (isinstance(q, torch.Tensor) and isinstance(k, torch.Tensor)
            and isinstance(v, torch.Tensor)):
        raise TypeError("q, k, v must be torch tensors")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one 4-d shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _TORCH_DTYPE_CODE:
        raise TypeError("q, k, v must all be float16, bfloat16 or float8_e4m3fn")
    for t in (q, k, v):
        if not t.is_cuda:
            raise ValueError("q, k, v must be device tensors")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _outputs(q, out, lse, layout="bhnd"):
    if layout == "bnhd":
        B, N, H, d = q.shape
    else:
        B, H, N, d = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != torch.float16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float16 tensor shaped like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if out.device != q.device or lse.device != q.device:
        raise ValueError("out and lse must be on the device of q, k, v")
    return out, lse


def _default_scale(d: int) -> float:
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O (fp16) and LSE (fp32) of softmax(scale Q K^T [+ causal mask]) V.

    fp8 (float8_e4m3fn) inputs are taken at unit scale; see ``fwd_fp8``.
    Runs on the current stream of q's device.
    """
    _validate(q, k, v)
    B, H, N, d = q.shape
    out, lse = _outputs(q, out, lse)
    scale = _default_scale(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                        int(bool(causal)), _TORCH_DTYPE_CODE[q.dtype], stream)
    _check(st)
    return out, lse


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, descale_q: torch.Tensor,
            descale_k: torch.Tensor, descale_v: torch.Tensor, causal: bool = False,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fp8 e4m3 attention with per-head dequantization scales (float32 [B*H])."""
    _validate(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("fwd_fp8 takes float8_e4m3fn q, k, v")
    B, H, N, d = q.shape
    for t in (descale_q, descale_k, descale_v):
        if (t.dtype != torch.float32 or t.numel() != B * H or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError("descales must be contiguous float32 device tensors of B*H values")
    out, lse = _outputs(q, out, lse)
    scale = _default_scale(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(descale_q), _ptr(descale_k),
                            _ptr(descale_v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                            int(bool(causal)), stream)
    _check(st)
    return out, lse


def _layout_shape(q, layout):
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    if layout == "bnhd":
        B, N, H, d = q.shape
    else:
        B, H, N, d = q.shape
    return B, H, N, d


def _descale_ptrs(q, descales, B, H):
    if descales is None:
        return None, None, None
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("descales apply to float8_e4m3fn inputs only")
    for t in descales:
        if (t.dtype != torch.float32 or t.numel() != B * H or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError("descales must be contiguous float32 device tensors of B*H values")
    return descales


def fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: str = "bhnd",
           causal: bool = False, scale: Optional[float] = None,
           descales: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
           out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fa_fwd_ex: q, k, v, out in [B, H, N, d] ("bhnd") or [B, N, H, d] ("bnhd");
    lse is [B, H, N] either way.  descales (fp8 only): float32 [B*H] each."""
    B, H, N, d = _layout_shape(q, layout)
    _validate(q, k, v)
    dq, dk, dv = _descale_ptrs(q, descales, B, H)
    out, lse = _outputs(q, out, lse, layout)
    scale = _default_scale(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(out),
                           _ptr(lse), B, H, N, d, scale, int(bool(causal)),
                           _TORCH_DTYPE_CODE[q.dtype], LAYOUTS[layout], stream)
    _check(st)
    return out, lse


def fwd_fp8_pv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, min_keys: int = 512,
               layout: str = "bhnd", causal: bool = False, scale: Optional[float] = None,
               descales: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
               out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fa_fwd_fp8_pv: fwd_ex for float8_e4m3fn q, k, v with P V on the fp8 matrix
    instructions for the query tiles whose first row sees at least min_keys keys."""
    B, H, N, d = _layout_shape(q, layout)
    _validate(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("fwd_fp8_pv takes float8_e4m3fn q, k, v")
    dq, dk, dv = _descale_ptrs(q, descales, B, H)
    out, lse = _outputs(q, out, lse, layout)
    scale = _default_scale(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd_fp8_pv(_ptr(q), _ptr(k), _ptr(v), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(out), _ptr(lse), B, H, N, d, scale, int(bool(causal)),
                               LAYOUTS[layout], int(min_keys), stream)
    _check(st)
    return out, lse


KV_TILE = 64  # key rows per scale of fa_fwd_fp8_kvtile


def fwd_fp8_kvtile(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   descales: Tuple[torch.Tensor, torch.Tensor, torch.Tensor],
                   pv_min_keys: int = -1, layout: str = "bhnd", causal: bool = False,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fa_fwd_fp8_kvtile: float8_e4m3fn q, k, v; descales = (per-head Q scales
    [B*H], per-tile K scales [B*H*ceil(N/64)], per-tile V scales, float32
    device tensors).  pv_min_keys < 0 keeps P V in fp16."""
    B, H, N, d = _layout_shape(q, layout)
    _validate(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("fwd_fp8_kvtile takes float8_e4m3fn q, k, v")
    nt = -(-N // KV_TILE)
    want = (B * H, B * H * nt, B * H * nt)
    if descales is None or len(descales) != 3:
        raise ValueError("fwd_fp8_kvtile needs (descale_q, descale_k, descale_v)")
    for t, n in zip(descales, want):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() != n
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"descales must be contiguous float32 device tensors of "
                             f"{want} elements")
    out, lse = _outputs(q, out, lse, layout)
    scale = _default_scale(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd_fp8_kvtile(_ptr(q), _ptr(k), _ptr(v), *(_ptr(t) for t in descales),
                                   _ptr(out), _ptr(lse), B, H, N, d, scale, int(bool(causal)),
                                   LAYOUTS[layout], int(pv_min_keys), stream)
    _check(st)
    return out, lse


def kvsplit_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool, dtype) -> int:
    """fa_fwd_kvsplit_workspace: device bytes fwd_kvsplit needs (0: it will not split)."""
    code = _TORCH_DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    n = load_library().fa_fwd_kvsplit_workspace(B, H, N, d, int(bool(causal)), code)
    if n < 0:
        _check(int(n))
    return int(n)


def _workspace(workspace, need, device):
    """The caller's workspace (a contiguous tensor on the inputs' device) and
    its size in bytes, or one allocated here when none is given."""
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError("workspace must be a tensor on the device of q, k, v")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace, workspace.numel() * workspace.element_size()


def fwd_kvsplit(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: str = "bhnd",
                causal: bool = False, scale: Optional[float] = None,
                descales: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fa_fwd_kvsplit: fwd_ex with long query tiles' key ranges split over several
    workgroups and merged.  workspace: a device tensor of at least
    kvsplit_workspace_bytes(...) bytes (allocated here when not given)."""
    B, H, N, d = _layout_shape(q, layout)
    _validate(q, k, v)
    dq, dk, dv = _descale_ptrs(q, descales, B, H)
    out, lse = _outputs(q, out, lse, layout)
    scale = _default_scale(d) if scale is None else float(scale)
    need = kvsplit_workspace_bytes(B, H, N, d, causal, q.dtype)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd_kvsplit(_ptr(q), _ptr(k), _ptr(v), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(out), _ptr(lse), B, H, N, d, scale, int(bool(causal)),
                                _TORCH_DTYPE_CODE[q.dtype], LAYOUTS[layout], _ptr(workspace),
                                ws_bytes, stream)
    _check(st)
    return out, lse


def fwd_kvsplit_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: str = "bhnd",
                        causal: bool = False, scale: Optional[float] = None,
                        descales: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fa_fwd_kvsplit_noalloc: fwd_kvsplit with the split workspace in the
    library's static device scratch (the library allocates nothing; pass out
    and lse to allocate nothing here either)."""
    B, H, N, d = _layout_shape(q, layout)
    _validate(q, k, v)
    dq, dk, dv = _descale_ptrs(q, descales, B, H)
    out, lse = _outputs(q, out, lse, layout)
    scale = _default_scale(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd_kvsplit_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dq), _ptr(dk), _ptr(dv),
                                        _ptr(out), _ptr(lse), B, H, N, d, scale,
                                        int(bool(causal)), _TORCH_DTYPE_CODE[q.dtype],
                                        LAYOUTS[layout], stream)
    _check(st)
    return out, lse


def kvsplit_noalloc_max_bytes() -> int:
    """Bytes of the static split workspace behind fwd_kvsplit_noalloc."""
    return int(load_library().fa_fwd_kvsplit_noalloc_max_bytes())


def fwd_fp8_pv_kvsplit(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, min_keys: int = 512,
                       layout: str = "bhnd", causal: bool = False,
                       scale: Optional[float] = None,
                       descales: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fa_fwd_fp8_pv_kvsplit: fwd_fp8_pv with long tiles' key ranges split over
    workgroups and merged (workspace as for fwd_kvsplit)."""
    B, H, N, d = _layout_shape(q, layout)
    _validate(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("fwd_fp8_pv_kvsplit takes float8_e4m3fn q, k, v")
    dq, dk, dv = _descale_ptrs(q, descales, B, H)
    out, lse = _outputs(q, out, lse, layout)
    scale = _default_scale(d) if scale is None else float(scale)
    need = kvsplit_workspace_bytes(B, H, N, d, causal, q.dtype)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_fwd_fp8_pv_kvsplit(_ptr(q), _ptr(k), _ptr(v), _ptr(dq), _ptr(dk), _ptr(dv),
                                       _ptr(out), _ptr(lse), B, H, N, d, scale,
                                       int(bool(causal)), LAYOUTS[layout], int(min_keys),
                                       _ptr(workspace), ws_bytes, stream)
    _check(st)
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
        dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
        dv: Optional[torch.Tensor] = None, delta: Optional[torch.Tensor] = None):
    """dQ, dK, dV (fp32 [B, H, N, d]) and delta = rowsum(dO * O) (fp32 [B, H, N])
    for fp16 / bf16 q, k, v, dout, the forward's o (fp16) and lse.  Output
    buffers may be passed in (contiguous, on q's device), else they are
    allocated."""
    _validate(q, k, v)
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("the backward pass takes float16 or bfloat16 q, k, v")
    B, H, N, d = q.shape
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_contiguous():
        raise ValueError("dout must be contiguous, shaped and typed like q")
    if o.shape != q.shape or o.dtype != torch.float16 or not o.is_contiguous():
        raise ValueError("o must be the forward's contiguous float16 output")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be the forward's contiguous float32 [B, H, N] output")
    for t in (dout, o, lse):
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")

    def out_buf(t, shape):
        if t is None:
            return torch.empty(shape, dtype=torch.float32, device=q.device)
        if (tuple(t.shape) != tuple(shape) or t.dtype != torch.float32
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"gradient outputs must be contiguous float32 {tuple(shape)} "
                             "tensors on q's device")
        return t

    dq, dk, dv = (out_buf(t, (B, H, N, d)) for t in (dq, dk, dv))
    delta = out_buf(delta, (B, H, N))
    scale = _default_scale(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(delta), B, H, N, d, scale, int(bool(causal)),
                        _TORCH_DTYPE_CODE[q.dtype], stream)
    _check(st)
    return dq, dk, dv, delta


# Storage dtype names of the input generator -> torch dtypes.
TORCH_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def to_device(inp, device="cuda"):
    """Upload an input set's storage bits as torch tensors (no conversion)."""
    import numpy as np

    def up(bits):
        raw = np.ascontiguousarray(bits)
        raw = raw.view(np.uint8) if inp.dtype == "fp8" else raw.view(np.int16)
        return torch.from_numpy(raw).to(device).view(TORCH_DTYPES[inp.dtype])
    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    ds = None
    if inp.dtype == "fp8":
        ds = tuple(torch.from_numpy(x).to(device) for x in
                   (inp.descale_q, inp.descale_k, inp.descale_v))
    return q, k, v, ds


def run_inputs(inp, device="cuda", out=None, lse=None):
    """Run the library on an input set (fp8 with its per-head descales, or
    fa_fwd_fp8_kvtile when K and V carry per-key-tile scales)."""
    q, k, v, ds = to_device(inp, device)
    if inp.dtype == "fp8" and getattr(inp, "kv_tile", None):
        if inp.kv_tile != KV_TILE:
            raise ValueError(f"the library takes key tiles of {KV_TILE} rows")
        return fwd_fp8_kvtile(q, k, v, ds, causal=inp.causal, scale=inp.scale, out=out, lse=lse)
    if inp.dtype == "fp8":
        return fwd_fp8(q, k, v, *ds, causal=inp.causal, scale=inp.scale, out=out, lse=lse)
    return fwd(q, k, v, causal=inp.causal, scale=inp.scale, out=out, lse=lse)
