"""The opt-in launch log (FIX_ATTN_LOG): a small forward and backward in a child process with the
variable set print one line per enqueued kernel, naming the entry point and the kernel; without it,
nothing."""
import os
import subprocess
import sys

import pytest

from gpu_util import needs_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = r"""
import sys, torch
sys.path.insert(0, %r)
import gated_softmax_attention_amd as F
dev = "cuda:0"
torch.manual_seed(0)
q, k, v = (torch.randn(1, 100, 2, 64, device=dev).to(torch.bfloat16) for _ in range(3))
g = torch.nn.functional.logsigmoid(torch.randn(1, 100, 2, 64, device=dev) + 2)
o, m, rstd, x = F.forward(q, k, v, g, o_norm=True)
F.backward(q, k, v, g, m, rstd, x, torch.randn_like(o), o_norm=True)
torch.cuda.synchronize()
print("child done", flush=True)
""" % ROOT


def _run(env):
    return subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True, timeout=300, env=env)


@pytest.mark.gpu
@needs_gpu
def test_launch_log():
    print("launch log: child with FIX_ATTN_LOG=1", flush=True)
    r = _run({**os.environ, "FIX_ATTN_LOG": "1"})
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[fixattn] ")]
    assert any(l.startswith("[fixattn] fix_attn_fwd: fix_fwd enqueued on stream") for l in lines), lines
    assert any(l.startswith("[fixattn] fix_attn_bwd: bwd_dkv enqueued on stream") for l in lines), lines
    assert sum(l.startswith("[fixattn] fix_attn_fwd: ") for l in lines) >= 3  # plan, gate scan, forward
    print("launch log: child without it", flush=True)
    env = dict(os.environ)
    env.pop("FIX_ATTN_LOG", None)
    r = _run(env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "[fixattn] " not in r.stderr
