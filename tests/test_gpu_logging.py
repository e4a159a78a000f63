"""FAR_LOG: with the variable set, each launching call prints its shape and plan."""

import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_far_log_prints_the_plan():
    """FAR_LOG=1 makes each launching call print its shape and plan on stderr; unset,
    nothing is printed."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    code = (
        "import torch\n"
        "from residual_add_rmsnorm_fp32_amd import binding as B\n"
        "p = [torch.ones(3, 520, dtype=torch.bfloat16, device='cuda') for _ in range(2)]\n"
        "g = torch.ones(520, dtype=torch.bfloat16, device='cuda')\n"
        "B.fused_add_rmsnorm(p, p[0].clone(), g, 1e-6, quant='dynamic')\n"
        "q = [torch.ones(4096, 1028, dtype=torch.bfloat16, device='cuda') for _ in range(2)]\n"
        "gq = torch.ones(1028, dtype=torch.bfloat16, device='cuda')\n"
        "B.fused_add_rmsnorm(q, q[0].clone(), gq, 1e-6, quant='dynamic')\n"
        "torch.cuda.synchronize()\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for flag, expect in (("1", 2), ("0", 0)):
        env = dict(os.environ, FAR_LOG=flag, PYTHONPATH=root)
        print(f"[log] FAR_LOG={flag}", flush=True)
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                             env=env, timeout=300, cwd=root)
        assert res.returncode == 0, res.stderr[-2000:]
        lines = [l for l in res.stderr.splitlines() if l.startswith("far: ")]
        assert len(lines) == expect, res.stderr[-2000:]
        if expect:
            assert "T=3 H=520 P=2 bf16 quant=dynamic" in lines[0] and "-> vector" in lines[0]
            assert "residual_stores=streamed" in lines[0]  # a decode-sized batch
            # a prefill-sized batch, rows ending in a partial pack: through the cache
            assert "T=4096 H=1028 P=2" in lines[1] and "residual_stores=cached" in lines[1]
            print(f"[log] {lines[0]}\n[log] {lines[1]}", flush=True)
