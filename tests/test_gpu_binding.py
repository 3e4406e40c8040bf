"""The binding loads the library against PyTorch's HIP runtime whatever the
import order: a fresh process that loads the library before it imports
torch itself must still launch kernels on torch's streams."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = """
from bit_nf4_quantized_14_amd import capi
capi.lib()                       # before this script imports torch
import torch
w = torch.randn(128, 256, device="cuda")
t = capi.nf4_quantize(w)
out = capi.nf4_dequantize(t)
torch.cuda.synchronize()
assert out.shape == (128, 256)
print("launched")
"""


def test_library_loaded_before_torch_still_launches():
    res = subprocess.run([sys.executable, "-c", CODE], cwd=ROOT,
                         capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stderr[-2000:]
    assert "launched" in res.stdout
