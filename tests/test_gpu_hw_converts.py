"""The kernels encode FP8 and FP4 with gfx950 conversion instructions.  This
runs the built check program, which compares those instructions with the
exact round-to-nearest-even, saturating integer encoders over every finite
fp32 input (and decoding over every e4m3 code and code pair), and expects no
mismatch."""
import os
import subprocess

import pytest

from conftest import ROOT

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

BIN = os.path.join(ROOT, "pruning_quantization_amd", "check_converts")


def test_hw_conversions_match_exact_encoders():
    assert os.path.exists(BIN), "build first: python -m pruning_quantization_amd.build"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": 0 mismatches") == 7
