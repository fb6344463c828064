"""The C-ABI library loads, exports what include/fa_mi355x.h declares and rejects
invalid arguments before any HIP call (nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

from attention_forward_fa_amd import binding
from attention_forward_fa_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH),
                                reason="library not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fa_[a-z0-9_]+)\s*\(",
                      text, flags=re.M)


def _header_constants():
    text = open(HEADER, encoding="utf-8").read()
    consts = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(FA_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}
    consts["FA_ABI_VERSION"] = int(re.search(r"#define FA_ABI_VERSION (\d+)", text).group(1))
    return consts


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) >= {"fa_fwd", "fa_fwd_fp8", "fa_status_string", "fa_abi_version"}
    lib = ctypes.CDLL(LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.SIGNATURES)


def test_abi_version_and_status_strings():
    lib = binding.load_library()
    c = _header_constants()
    assert lib.fa_abi_version() == c["FA_ABI_VERSION"]
    for name, val in c.items():
        if name.startswith("FA_ERR_") or name == "FA_OK":
            s = binding.status_string(val)
            assert s and s != "unknown status", name
    assert binding.status_string(12345) == "unknown status"


# Fake, 16-byte aligned "device" addresses: never dereferenced, because every
# call below fails validation (or is empty) before reaching the HIP runtime.
A = 0x7F0000000000
Q, K, V, O, L = A, A + 0x1000, A + 0x2000, A + 0x3000, A + 0x4000


def _call(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=256, d=64, scale=0.125, causal=0,
                dtype=0, stream=None)
    args.update(kw)
    return lib.fa_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                      args["H"], args["N"], args["d"], args["scale"], args["causal"],
                      args["dtype"], args["stream"])


def _call_fp8(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, dq=A + 0x5000, dk=A + 0x6000, dv=A + 0x7000, o=O, lse=L,
                B=1, H=2, N=256, d=128, scale=0.1, causal=1, stream=None)
    args.update(kw)
    return lib.fa_fwd_fp8(args["q"], args["k"], args["v"], args["dq"], args["dk"], args["dv"],
                          args["o"], args["lse"], args["B"], args["H"], args["N"], args["d"],
                          args["scale"], args["causal"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), "FA_ERR_NULL"),
    (dict(lse=None), "FA_ERR_NULL"),
    (dict(o=None), "FA_ERR_NULL"),
    (dict(B=-1), "FA_ERR_SHAPE"),
    (dict(N=-5), "FA_ERR_SHAPE"),
    (dict(N=1 << 25), "FA_ERR_SHAPE"),
    (dict(B=1 << 25), "FA_ERR_SHAPE"),
    (dict(B=1 << 40, H=1 << 40), "FA_ERR_SHAPE"),  # B * H would overflow int64
    (dict(B=1 << 13, H=1 << 12), "FA_ERR_SHAPE"),
    (dict(d=96), "FA_ERR_HEAD_DIM"),
    (dict(d=0), "FA_ERR_HEAD_DIM"),
    (dict(dtype=3), "FA_ERR_DTYPE"),
    (dict(dtype=-1), "FA_ERR_DTYPE"),
    (dict(q=Q + 8), "FA_ERR_ALIGN"),
    (dict(o=O + 2), "FA_ERR_ALIGN"),
    (dict(lse=L + 2), "FA_ERR_ALIGN"),
    (dict(scale=0.0), "FA_ERR_SCALE"),
    (dict(scale=-0.5), "FA_ERR_SCALE"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(causal=2), "FA_ERR_CAUSAL"),
])
def test_fa_fwd_rejects(kw, status):
    assert _call(**kw) == _header_constants()[status]


@pytest.mark.parametrize("kw,status", [
    (dict(dq=None), "FA_ERR_NULL"),
    (dict(dv=None), "FA_ERR_NULL"),
    (dict(dk=A + 0x6002), "FA_ERR_ALIGN"),
    (dict(d=32), "FA_ERR_HEAD_DIM"),
    (dict(causal=-1), "FA_ERR_CAUSAL"),
])
def test_fa_fwd_fp8_rejects(kw, status):
    assert _call_fp8(**kw) == _header_constants()[status]


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0),
                                dict(N=0, q=None, k=None, v=None, o=None, lse=None)])
def test_empty_problem_is_a_noop(kw):
    # B*H*N == 0: nothing to compute, no pointer is read, no launch.
    assert _call(**kw) == 0
    assert _call_fp8(**kw) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        binding.load_library(str(tmp_path / "missing.so"))


def _call_ex(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, dq=None, dk=None, dv=None, o=O, lse=L, B=1, H=2, N=256, d=128,
                scale=0.1, causal=0, dtype=0, layout=1, stream=None)
    args.update(kw)
    return lib.fa_fwd_ex(args["q"], args["k"], args["v"], args["dq"], args["dk"], args["dv"],
                         args["o"], args["lse"], args["B"], args["H"], args["N"], args["d"],
                         args["scale"], args["causal"], args["dtype"], args["layout"],
                         args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(layout=2), "FA_ERR_LAYOUT"),
    (dict(layout=-1), "FA_ERR_LAYOUT"),
    (dict(q=None), "FA_ERR_NULL"),
    (dict(d=96), "FA_ERR_HEAD_DIM"),
    (dict(dtype=5), "FA_ERR_DTYPE"),
    (dict(o=O + 4), "FA_ERR_ALIGN"),
    # fp8: descales all or none
    (dict(dtype=2, dq=A + 0x5000), "FA_ERR_NULL"),
    (dict(dtype=2, dq=A + 0x5000, dk=A + 0x6000), "FA_ERR_NULL"),
    (dict(dtype=2, dq=A + 0x5002, dk=A + 0x6000, dv=A + 0x7000), "FA_ERR_ALIGN"),
    # [B, N, H, d]: one head's rows span N*H*d elements, at most 2^30 bytes
    (dict(N=1 << 20, H=1 << 9, d=128, dtype=1), "FA_ERR_SHAPE"),
    (dict(N=1 << 20, H=1 << 4, d=128, dtype=2, layout=1), "FA_ERR_SHAPE"),
])
def test_fa_fwd_ex_rejects(kw, status):
    assert _call_ex(**kw) == _header_constants()[status]


def test_fa_fwd_ex_shape_limit_is_per_layout():
    # The same N*H*d that [B, N, H, d] refuses passes the size checks for
    # [B, H, N, d]; a NULL q (checked after the sizes) stops it before launch.
    big = dict(N=1 << 20, H=1 << 4, d=128, dtype=2, q=None)
    assert _call_ex(layout=1, **big) == _header_constants()["FA_ERR_SHAPE"]
    assert _call_ex(layout=0, **big) == _header_constants()["FA_ERR_NULL"]


@pytest.mark.parametrize("layout", [0, 1])
def test_fa_fwd_ex_empty_is_a_noop(layout):
    assert _call_ex(layout=layout, N=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert _call_ex(layout=layout, B=0) == 0


def _call_bwd(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, o=O, lse=L, do=A + 0x5000, dq=A + 0x6000, dk=A + 0x7000,
                dv=A + 0x8000, delta=A + 0x9000, B=1, H=2, N=256, d=128, scale=0.1, causal=1,
                dtype=0, stream=None)
    args.update(kw)
    return lib.fa_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"],
                      args["dq"], args["dk"], args["dv"], args["delta"], args["B"], args["H"],
                      args["N"], args["d"], args["scale"], args["causal"], args["dtype"],
                      args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), "FA_ERR_DTYPE"),
    (dict(dtype=7), "FA_ERR_DTYPE"),
    (dict(d=32), "FA_ERR_HEAD_DIM"),
    (dict(causal=3), "FA_ERR_CAUSAL"),
    (dict(scale=-1.0), "FA_ERR_SCALE"),
    (dict(N=-1), "FA_ERR_SHAPE"),
    (dict(N=1 << 23), "FA_ERR_SHAPE"),
    (dict(B=1 << 40, H=1 << 40), "FA_ERR_SHAPE"),  # B * H would overflow int64
    (dict(delta=None), "FA_ERR_NULL"),
    (dict(dv=None), "FA_ERR_NULL"),
    (dict(do=None), "FA_ERR_NULL"),
    (dict(lse=L + 4), "FA_ERR_ALIGN"),
    (dict(dk=A + 0x7008), "FA_ERR_ALIGN"),
])
def test_fa_bwd_rejects(kw, status):
    assert _call_bwd(**kw) == _header_constants()[status]


def test_fa_bwd_empty_is_a_noop():
    assert _call_bwd(N=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None,
                     dv=None, delta=None) == 0


def _call_pv(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, dq=None, dk=None, dv=None, o=O, lse=L, B=1, H=2, N=256, d=128,
                scale=0.1, causal=1, layout=0, min_keys=512, stream=None)
    args.update(kw)
    return lib.fa_fwd_fp8_pv(args["q"], args["k"], args["v"], args["dq"], args["dk"],
                             args["dv"], args["o"], args["lse"], args["B"], args["H"],
                             args["N"], args["d"], args["scale"], args["causal"],
                             args["layout"], args["min_keys"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(min_keys=-1), "FA_ERR_MIN_KEYS"),
    (dict(min_keys=-(1 << 40), N=0), "FA_ERR_MIN_KEYS"),
    (dict(layout=3), "FA_ERR_LAYOUT"),
    (dict(d=256), "FA_ERR_HEAD_DIM"),
    (dict(causal=2), "FA_ERR_CAUSAL"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"),
    (dict(v=None), "FA_ERR_NULL"),
    (dict(lse=L + 2), "FA_ERR_ALIGN"),
    (dict(dq=A + 0x5000), "FA_ERR_NULL"),
    (dict(dq=A + 0x5000, dk=A + 0x6000, dv=A + 0x7001), "FA_ERR_ALIGN"),
    (dict(N=1 << 20, H=1 << 4, d=128, layout=1), "FA_ERR_SHAPE"),
])
def test_fa_fwd_fp8_pv_rejects(kw, status):
    assert _call_pv(**kw) == _header_constants()[status]


@pytest.mark.parametrize("min_keys", [0, 512, 1 << 62])
def test_fa_fwd_fp8_pv_empty_is_a_noop(min_keys):
    assert _call_pv(min_keys=min_keys, N=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert _call_pv(min_keys=min_keys, H=0) == 0


# --- key-range split: the plan is host logic, visible through the workspace size ---

def _ws(B, H, N, d, causal, dtype):
    return binding.load_library().fa_fwd_kvsplit_workspace(B, H, N, d, causal, dtype)


def test_kvsplit_workspace_follows_the_plan():
    c = _header_constants()
    # Grids with at least two tiles per resident workgroup are not split.
    assert _ws(2, 16, 4096, 128, 0, 0) == 0        # 512 tiles of 256 rows
    assert _ws(1, 32, 8192, 128, 1, 1) == 0        # 1024 causal tiles
    assert _ws(1, 32, 16384, 128, 1, 2) == 0       # fp8: 4096 tiles of 128 rows
    assert _ws(4, 16, 1024, 64, 0, 0) == 0         # 512 tiles, 8 groups each: no gain
    assert _ws(1, 2, 256, 64, 0, 0) == 0           # fewer than 4 tiles per head
    # One GPU's share of the bf16 causal workload (4 of 32 heads): 32 tiles of
    # 256 rows per head, tile t spanning t + 1 groups; chunks of <= 11 groups
    # give 63 chunks per head (252 workgroups for 256 CUs), the longest tile 3.
    # Per chunk row: O in fp16 (2 d bytes) and LSE in fp32 (4 bytes).
    assert _ws(1, 4, 8192, 128, 1, 1) == 4 * 32 * 3 * 256 * (2 * 128 + 4)
    # Non-causal: split only when the whole grid leaves CUs idle.  8 heads of
    # 4096 rows (128 tiles of 256 rows) split in two chunks per tile; 16 heads
    # of 2048 rows are estimated no faster split; 4 heads of 4096 rows: 16
    # tiles of 16 groups per head, chunks of 4 groups.
    assert _ws(1, 8, 4096, 128, 0, 0) == 8 * 16 * 2 * 256 * (2 * 128 + 4)
    assert _ws(1, 16, 2048, 128, 0, 0) == 0
    assert _ws(1, 4, 4096, 128, 0, 0) == 4 * 16 * 4 * 256 * (2 * 128 + 4)
    # Invalid arguments give fa_fwd_ex's statuses; an empty problem needs nothing.
    assert _ws(1, 4, 8192, 96, 1, 1) == c["FA_ERR_HEAD_DIM"]
    assert _ws(1, 4, 8192, 128, 2, 1) == c["FA_ERR_CAUSAL"]
    assert _ws(1, 4, 8192, 128, 1, 9) == c["FA_ERR_DTYPE"]
    assert _ws(-1, 4, 8192, 128, 1, 1) == c["FA_ERR_SHAPE"]
    assert _ws(1, 4, 0, 128, 1, 1) == 0


def _call_split(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, dq=None, dk=None, dv=None, o=O, lse=L, B=1, H=4, N=8192, d=128,
                scale=0.1, causal=1, dtype=1, layout=0, ws=A + 0x10000, ws_bytes=1 << 30,
                stream=None)
    args.update(kw)
    return lib.fa_fwd_kvsplit(args["q"], args["k"], args["v"], args["dq"], args["dk"],
                              args["dv"], args["o"], args["lse"], args["B"], args["H"],
                              args["N"], args["d"], args["scale"], args["causal"],
                              args["dtype"], args["layout"], args["ws"], args["ws_bytes"],
                              args["stream"])


NEED = 4 * 32 * 3 * 256 * (2 * 128 + 4)  # bf16 causal [1, 4, 8192, 128]: O fp16 + LSE fp32 per chunk row


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), "FA_ERR_NULL"),
    (dict(ws=A + 0x10080), "FA_ERR_ALIGN"),
    (dict(ws_bytes=NEED - 1), "FA_ERR_WORKSPACE"),
    (dict(ws_bytes=-1), "FA_ERR_WORKSPACE"),
    (dict(ws_bytes=-1, N=0), "FA_ERR_WORKSPACE"),
    (dict(layout=5), "FA_ERR_LAYOUT"),
    (dict(d=80), "FA_ERR_HEAD_DIM"),
    (dict(scale=0.0), "FA_ERR_SCALE"),
    (dict(o=None), "FA_ERR_NULL"),
    (dict(dtype=2, dq=A + 0x5000), "FA_ERR_NULL"),
])
def test_fa_fwd_kvsplit_rejects(kw, status):
    assert _call_split(**kw) == _header_constants()[status]


def test_fa_fwd_kvsplit_empty_is_a_noop():
    assert _call_split(N=0, q=None, k=None, v=None, o=None, lse=None, ws=None, ws_bytes=0) == 0
    assert _call_split(B=0, ws=None, ws_bytes=0) == 0


def _call_pvsplit(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, dq=None, dk=None, dv=None, o=O, lse=L, B=1, H=4, N=16384, d=128,
                scale=0.1, causal=1, layout=0, min_keys=512, ws=A + 0x10000, ws_bytes=1 << 34,
                stream=None)
    args.update(kw)
    return lib.fa_fwd_fp8_pv_kvsplit(args["q"], args["k"], args["v"], args["dq"], args["dk"],
                                     args["dv"], args["o"], args["lse"], args["B"], args["H"],
                                     args["N"], args["d"], args["scale"], args["causal"],
                                     args["layout"], args["min_keys"], args["ws"],
                                     args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(min_keys=-1), "FA_ERR_MIN_KEYS"),
    (dict(ws_bytes=-5), "FA_ERR_WORKSPACE"),
    (dict(ws=None), "FA_ERR_NULL"),
    (dict(ws=A + 0x10010), "FA_ERR_ALIGN"),
    (dict(ws_bytes=1000), "FA_ERR_WORKSPACE"),
    (dict(layout=7), "FA_ERR_LAYOUT"),
    (dict(dq=A + 0x5000, dk=A + 0x6000), "FA_ERR_NULL"),
    (dict(lse=None), "FA_ERR_NULL"),
])
def test_fa_fwd_fp8_pv_kvsplit_rejects(kw, status):
    assert _call_pvsplit(**kw) == _header_constants()[status]


def test_fa_fwd_fp8_pv_kvsplit_empty_is_a_noop():
    assert _call_pvsplit(N=0, q=None, k=None, v=None, o=None, lse=None, ws=None,
                         ws_bytes=0) == 0


def _call_noalloc(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, dq=None, dk=None, dv=None, o=O, lse=L, B=1, H=4, N=8192, d=128,
                scale=0.1, causal=1, dtype=1, layout=0, stream=None)
    args.update(kw)
    return lib.fa_fwd_kvsplit_noalloc(args["q"], args["k"], args["v"], args["dq"], args["dk"],
                                      args["dv"], args["o"], args["lse"], args["B"], args["H"],
                                      args["N"], args["d"], args["scale"], args["causal"],
                                      args["dtype"], args["layout"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(layout=5), "FA_ERR_LAYOUT"),
    (dict(d=80), "FA_ERR_HEAD_DIM"),
    (dict(scale=0.0), "FA_ERR_SCALE"),
    (dict(o=None), "FA_ERR_NULL"),
    (dict(q=Q + 8), "FA_ERR_ALIGN"),
    (dict(dtype=2, dq=A + 0x5000), "FA_ERR_NULL"),
    # fp8 causal [1, 4, 16384, 128] splits into 81.25 MiB of partials: more
    # than the 64 MiB static scratch, refused before any launch
    (dict(dtype=2, N=16384), "FA_ERR_SCRATCH"),
])
def test_fa_fwd_kvsplit_noalloc_rejects(kw, status):
    assert _call_noalloc(**kw) == _header_constants()[status]


def test_fa_fwd_kvsplit_noalloc_empty_is_a_noop():
    assert _call_noalloc(N=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert _call_noalloc(B=0) == 0


def test_noalloc_scratch_size():
    assert binding.kvsplit_noalloc_max_bytes() == 64 << 20


def _call_kvtile(**kw):
    lib = binding.load_library()
    args = dict(q=Q, k=K, v=V, dq=A + 0x5000, dk=A + 0x6000, dv=A + 0x7000, o=O, lse=L, B=1,
                H=2, N=300, d=128, scale=0.1, causal=1, layout=0, min_keys=-1, stream=None)
    args.update(kw)
    return lib.fa_fwd_fp8_kvtile(args["q"], args["k"], args["v"], args["dq"], args["dk"],
                                 args["dv"], args["o"], args["lse"], args["B"], args["H"],
                                 args["N"], args["d"], args["scale"], args["causal"],
                                 args["layout"], args["min_keys"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dq=None), "FA_ERR_NULL"),
    (dict(dk=None), "FA_ERR_NULL"),
    (dict(dv=None), "FA_ERR_NULL"),
    (dict(dk=A + 0x6002), "FA_ERR_ALIGN"),
    (dict(layout=3), "FA_ERR_LAYOUT"),
    (dict(d=32), "FA_ERR_HEAD_DIM"),
    (dict(causal=2), "FA_ERR_CAUSAL"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"),
    (dict(lse=None), "FA_ERR_NULL"),
    (dict(o=O + 4), "FA_ERR_ALIGN"),
])
def test_fa_fwd_fp8_kvtile_rejects(kw, status):
    assert _call_kvtile(**kw) == _header_constants()[status]


def test_fa_fwd_fp8_kvtile_empty_is_a_noop():
    assert _call_kvtile(N=0, q=None, k=None, v=None, o=None, lse=None, dq=None, dk=None,
                        dv=None) == 0
