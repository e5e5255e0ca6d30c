"""Input magnitudes at the edges of the fp16 operands the backward stages.

q and k reach some products rounded to fp16.  fix_attn_check_inputs reports
whether any |q| or |k| exceeds 65504 (or is infinite or NaN), the case the
kernels do not handle; magnitudes below 2^-14 are fp16 subnormals and are
handled (parity against the oracle at the usual bar, below)."""
import numpy as np
import pytest
import torch

import gated_softmax_attention_amd as F
from gpu_util import announce, custom_inputs, needs_gpu, oracle_bwd_for, oracle_fwd_for
from test_gpu_bwd import check_bwd, run_bwd
from test_gpu_fox import check as check_scalar, run as run_scalar, scalar_inputs

pytestmark = [pytest.mark.gpu, needs_gpu]


def _qkv(dtype, T=200, Hq=4, Hkv=2, dk=64, dv=64, seed=3):
    g = torch.Generator().manual_seed(seed)
    mk = lambda *s: torch.randn(*s, generator=g).to(dtype).cuda()
    return mk(1, T, Hq, dk), mk(1, T, Hkv, dk), mk(1, T, Hkv, dv)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_check_inputs_in_range(dtype):
    announce(f"check_inputs in range {dtype}")
    q, k, v = _qkv(dtype)
    assert F.check_inputs(q, k, v) == F.FIX_OK
    # the largest value in range in each type (65504 is not a bf16 value: it rounds to 65536)
    top = 65280.0 if dtype == torch.bfloat16 else 65504.0
    q.view(-1)[17] = top
    k.view(-1)[-1] = -top
    assert F.check_inputs(q, k, v) == F.FIX_OK
    q.view(-1)[17] = 65536.0
    assert F.check_inputs(q, k, v) == F.FIX_E_RANGE


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("where,val", [("q", 1.0e5), ("k", -7.0e4), ("q", float("inf")), ("k", float("nan"))])
def test_check_inputs_out_of_range(dtype, where, val):
    announce(f"check_inputs {where}={val} {dtype}")
    q, k, v = _qkv(dtype)
    (q if where == "q" else k).view(-1)[1234] = val
    assert F.check_inputs(q, k, v) == F.FIX_E_RANGE


@pytest.mark.parametrize("scalar", [False, True])
def test_small_magnitude_parity(scalar):
    """q and k scaled by 2^-16: most elements are fp16 subnormals when staged;
    forward and backward still meet the parity bar (power-of-two scaling is
    exact in bf16, so the oracle sees the same inputs)."""
    announce(f"small magnitude scalar={scalar}")
    mk = scalar_inputs if scalar else custom_inputs
    x = dict(mk(1, 300, 4, 2, 64, 64, gate=(3.0, 1.0)))
    x["q"] = x["q"] * 2.0 ** -16
    x["k"] = x["k"] * 2.0 ** -16
    if scalar:
        check_scalar(run_scalar(x), oracle_fwd_for(x), oracle_bwd_for(x))
    else:
        check_bwd(run_bwd(x), oracle_bwd_for(x))
