"""The product path and its boundary, on the CPU: the oracle stays test
infrastructure (no product module imports it, no HIP source includes it),
compute calls without a GPU fail loudly instead of falling back, and
bench.py keeps its one-GPU contract."""
import glob
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_forward_fa_amd")


def test_product_modules_do_not_import_the_oracle():
    code = ("import sys\n"
            "import attention_forward_fa_amd.binding, attention_forward_fa_amd.build\n"
            "import attention_forward_fa_amd.inputs, attention_forward_fa_amd.accounting\n"
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.strip()
    assert out == "[]", out


def test_product_sources_never_name_the_oracle_package():
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle)\b", re.M)
    for path in glob.glob(os.path.join(PKG, "*.py")):
        assert not pat.search(open(path).read()), path
    for path in glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*")):
        text = open(path).read()
        assert "oracle/" not in text and '#include "oracle' not in text, path


def test_bench_imports_the_oracle_only_for_the_cpu_baseline():
    src = open(os.path.join(ROOT, "bench.py")).read()
    hits = [m.start() for m in re.finditer(r"from oracle import|import oracle", src)]
    assert len(hits) == 1
    fn = src.rfind("\ndef ", 0, hits[0])
    assert "cpu_baseline" in src[fn:src.index("\n", fn + 1)], "oracle import outside the baseline leg"


def test_bench_refuses_more_than_one_gpu(capsys):
    sys.path.insert(0, ROOT)
    import bench
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour without a GPU")
def test_compute_without_a_gpu_fails_loudly():
    from attention_forward_fa_amd import binding
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16)
    with pytest.raises(Exception):
        binding.fwd(q, q, q)
