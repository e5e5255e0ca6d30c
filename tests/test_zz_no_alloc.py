"""The allocation-free decode step (fix_decode_step_noalloc, through the C ABI) against the
allocating one (fix_decode_step) on the same cache and query: two calls in a row, the second
with a smaller input (fewer sequences, heads and tokens), each compared element by element
(the bar of the decode tests, 1e-2 of rms on o; the two run the same kernels, so the results
are expected to be equal) and against the fp64 oracle's row."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_softmax_attention_amd as F
from gpu_util import announce, custom_inputs, err_rms, needs_gpu, oracle_fwd_for, to_dev

pytestmark = [pytest.mark.gpu, needs_gpu]
TOL = 1e-2


def _one(B, T, Hq, Hkv, dk, dv, seed):
    x = custom_inputs(B, T, Hq, Hkv, dk, dv, seed=seed, backward=False)
    wl = x["workload"]
    cap = ((T + 63) // 64) * 64
    cache = F.DecodeCache(B, cap, Hq, Hkv, dk, dv, dtype=torch.bfloat16, out_dtype=torch.float32, o_norm=True)
    cache.append(to_dev(x["k"], torch.bfloat16), to_dev(x["v"], torch.bfloat16), to_dev(x["g"], torch.float32))
    q = to_dev(x["q"][:, T - 1], torch.bfloat16)
    w = to_dev(x["w"], torch.bfloat16)
    o_ref, m_ref = cache.step(q, w)
    # poisoned outputs: the entry point must overwrite every element
    o = torch.full((B, Hq, dv), float("nan"), device="cuda")
    m = torch.full((B, Hq), float("nan"), device="cuda")
    cache.step_noalloc(q, o, m, w)
    torch.cuda.synchronize()
    got, ref = o.cpu().numpy(), o_ref.cpu().numpy()
    e = err_rms(got, ref)
    ora = oracle_fwd_for(x, window=1)["o"][:, T - 1]
    e_or = err_rms(got, ora)
    print(f"B={B} T={T} H={Hq}/{Hkv} d={dk}/{dv}: vs fix_decode_step {e:.2e} (equal: {np.array_equal(got, ref)}), "
          f"vs oracle {e_or:.2e}", flush=True)
    assert e <= TOL and e_or <= TOL
    assert torch.isfinite(m).all()
    assert torch.equal(m, m_ref)


def test_decode_step_noalloc_matches_step():
    announce("decode step without allocation: two calls, the second smaller")
    _one(4, 1000, 8, 2, 128, 128, seed=3)
    _one(2, 130, 4, 4, 64, 32, seed=4)
