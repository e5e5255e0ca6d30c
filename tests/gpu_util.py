"""Helpers shared by the GPU parity tests: device transfer, oracle calls, metrics."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
from gated_softmax_attention_amd import synth

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")


def announce(msg: str):
    """Name the case on stdout before any GPU work, so a fault can be attributed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a, dtype):
    """numpy fp32 (bf16-representable when dtype is bf16) -> CUDA tensor, exactly."""
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def device_inputs(x: dict):
    wl = x["workload"]
    dt = torch.bfloat16 if wl.in_dtype == "bf16" else torch.float32
    d = {n: to_dev(x[n], dt) for n in ("q", "k", "v", "w", "z", "dO")}
    d["g"] = to_dev(x["g"], torch.float32)
    d["g_logits"] = to_dev(x["g_logits"], torch.float32)
    d["cu_seqlens"] = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    d["dtype"] = dt
    return d


def err_rms(got, ref, mask=None, floor=0.0):
    """max |got - ref| / max(rms(ref), floor) over the entries where ref is defined (and mask).

    floor is only for references that vanish in exact arithmetic (their fp64 value is
    rounding noise); it is then the scale of the terms that cancel."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    sel = ~np.isnan(ref)
    if mask is not None:
        sel &= mask
    g, r = got[sel], ref[sel]
    assert g.size > 0, "nothing to compare"
    assert np.isfinite(g).all(), "non-finite GPU output where the oracle is defined"
    rms = np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(g - r)) / max(rms, floor, 1e-300))


def bf16_ulp(a):
    """Spacing of bf16 numbers at |a| (half of it is the worst rounding error)."""
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-38)))
    return np.exp2(e - 7)


def oracle_fwd_for(x: dict, *, o_norm=True, eps=1e-5, unit_mask=None, window=0, gate_logits=False):
    g = x["g_logits"] if gate_logits else x["g"]
    return O.oracle_fwd(x["q"], x["k"], x["v"], g, x["cu_seqlens"], eps=eps, o_norm=o_norm,
                        w=x["w"] if o_norm else None, z=x["z"], unit_mask=unit_mask, window=window,
                        gate_logits=gate_logits)


def oracle_bwd_for(x: dict, *, o_norm=True, eps=1e-5, unit_mask=None, window=0, gate_logits=False):
    g = x["g_logits"] if gate_logits else x["g"]
    return O.oracle_bwd(x["q"], x["k"], x["v"], g, x["dO"], x["cu_seqlens"], eps=eps, o_norm=o_norm,
                        w=x["w"] if o_norm else None, z=x["z"], unit_mask=unit_mask, window=window,
                        gate_logits=gate_logits)


def custom_inputs(B, T, Hq, Hkv, dk, dv, *, in_dtype="bf16", gate=(3.0, 1.5), lengths=(), o_gate=False,
                  w_kind="normal", seed=7, backward=True):
    wl = synth.Workload("custom", B, T, Hq, Hkv, dk, dv, in_dtype=in_dtype, gate_mu=gate[0], gate_sd=gate[1],
                        w_kind=w_kind, o_gate=o_gate, lengths=tuple(lengths), backward=backward)
    return synth.make_inputs(wl, seed=seed)
