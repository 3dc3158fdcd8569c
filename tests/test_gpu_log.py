"""PQL_LOG on the device: each launch is logged with the kernel the call enqueues.

PQL_LOG is read once per process, so the calls run in one child interpreter."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = """
import torch, precision_quantized_linear_amd as pql
a = torch.randn(300, 512, dtype=torch.bfloat16, device="cuda")
w = torch.randn(256, 512, dtype=torch.bfloat16, device="cuda")
wq = pql.quantize(w, "fp8_row", "weight")
pql.qgemm(pql.quantize(a, "fp8_row", "activation"), wq)
pql.qlinear(a[:4], wq)
torch.cuda.synchronize()
print("done", flush=True)
"""


def test_launch_log_names_the_kernels():
    import precision_quantized_linear_amd as pql
    env = dict(os.environ, PQL_LOG="1")
    r = subprocess.run([sys.executable, "-c", CODE], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "done", r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[pql] ")]
    assert len(lines) == 4, r.stderr
    assert lines[0].startswith("[pql] quantize FP8_ROW weight M=256 N=0 K=512 -> k_fp8_row on stream ")
    assert lines[1].startswith("[pql] quantize FP8_ROW activation M=300 N=0 K=512 -> k_fp8_row on stream ")
    gemm = pql.kernel_name("qgemm", "fp8_row", "activation", 300, 256, 512)
    assert lines[2].startswith(f"[pql] qgemm FP8_ROW M=300 N=256 K=512 -> {gemm} on stream ")
    few = pql.kernel_name("qlinear", "fp8_row", "activation", 4, 256, 512)
    assert few == "k_qlinear_few<fp8_row>"
    assert lines[3].startswith(f"[pql] qlinear FP8_ROW M=4 N=256 K=512 -> {few} on stream ")
