"""Parity of the scalar-gate path (gate_scalar: one gate value per token and kv head).

Forward and backward have their own kernels (the decay as a logit bias); the
gate gradient is the suffix sum of row sums minus column sums of dS.  The
reference is the fp64 oracle with the same scalar gate (the oracle treats it
as the same value in every channel and sums its per-channel dg).  Bars: max
|gpu - oracle| / rms(oracle) <= 1e-2 on o, x, dq, dk, dv, dw, dz and 5e-3 on
dg; m within 1e-4 * max|m| (bf16 inputs) or 2^-9 * max|m| (fp32 inputs
staged as fp16); rstd within 1e-2 relative.  A single token (exact dq, dk
and dg vanish at eps = 0, so no relative error is defined) is checked on the
forward only; packed cases hold one-token and empty sequences.
"""
import numpy as np
import pytest
import torch

import gated_softmax_attention_amd as F
from gpu_util import announce, custom_inputs, device_inputs, err_rms, needs_gpu, oracle_bwd_for, oracle_fwd_for

pytestmark = [pytest.mark.gpu, needs_gpu]
TOL = 1e-2
TOL_DG = 5e-3


def scalar_inputs(*args, **kw):
    """Seeded inputs with the gate reduced to channel 0 of the per-channel one: [B,T,Hkv]."""
    x = custom_inputs(*args, **kw)
    x = dict(x)
    x["g"] = np.ascontiguousarray(x["g"][..., 0])
    x["g_logits"] = np.ascontiguousarray(x["g_logits"][..., 0])
    return x


def run(x, *, o_norm=True, gate_logits=False, backward=True):
    d = device_inputs(x)
    w = d["w"] if o_norm else None
    g = d["g_logits"] if gate_logits else d["g"]
    assert g.dim() == 3
    o, m, rstd, xx = F.forward(d["q"], d["k"], d["v"], g, d["cu_seqlens"], o_norm=o_norm, o_norm_weight=w,
                               o_gate=d["z"], out_dtype=torch.float32, gate_logits=gate_logits)
    out = {"o": o.cpu().numpy(), "m": m.cpu().numpy(), "rstd": rstd.cpu().numpy(), "x": xx.cpu().numpy()}
    if backward:
        o2, m2, r2, x2 = F.forward(d["q"], d["k"], d["v"], g, d["cu_seqlens"], o_norm=o_norm, o_norm_weight=w,
                                   o_gate=d["z"], gate_logits=gate_logits)
        dq, dk, dv, dg, dw, dz = F.backward(d["q"], d["k"], d["v"], g, m2, r2, x2, d["dO"], d["cu_seqlens"],
                                            o_norm=o_norm, o_norm_weight=w, o_gate=d["z"], out_dtype=torch.float32,
                                            need_dw=True, need_dz=True, gate_logits=gate_logits)
        cpu = lambda t: None if t is None else t.float().cpu().numpy()
        out.update({"dq": cpu(dq), "dk": cpu(dk), "dv": cpu(dv), "dg": cpu(dg), "dw": cpu(dw), "dz": cpu(dz)})
    torch.cuda.synchronize()
    return out


def check(got, rf, rb, *, o_norm=True, f32_inputs=False):
    e = {"o": err_rms(got["o"], rf["o"]), "x": err_rms(got["x"], rf["x"])}
    sel = ~np.isnan(rf["m"])
    m_err = float(np.max(np.abs(got["m"][sel] - rf["m"][sel])))
    if o_norm:
        e["rstd"] = float(np.max(np.abs(got["rstd"][sel] / rf["rstd"][sel] - 1)))
    if rb is not None:
        assert got["dg"].shape == rb["dg"].shape
        for n in ("dq", "dk", "dv", "dg"):
            e[n] = err_rms(got[n], rb[n])
        if got["dz"] is not None:
            e["dz"] = err_rms(got["dz"], rb["dz"])
        if o_norm:
            e["dw"] = err_rms(got["dw"], rb["dw"])
    print("errors:", {k: f"{v:.2e}" for k, v in e.items()}, f"m {m_err:.2e}", flush=True)
    for n, v in e.items():
        assert v <= (TOL_DG if n == "dg" else TOL), f"{n}: {v:.3e}"
    m_tol = 2.0 ** -9 if f32_inputs else 1e-4
    assert m_err <= m_tol * max(1.0, float(np.nanmax(np.abs(rf["m"]))))


CASES = [
    # B, T, Hq, Hkv, dk, dv, options
    (2, 300, 4, 2, 64, 64, {}),
    (1, 65, 2, 2, 128, 128, {"o_gate": True}),
    (1, 700, 4, 4, 128, 128, {"gate": (8.0, 1.0)}),
    (1, 300, 2, 1, 64, 64, {"gate": (-3.0, 1.0)}),
    (1, 591, 4, 2, 64, 64, {"lengths": (1, 0, 65, 130, 5, 300, 90)}),
    (1, 257, 2, 2, 32, 16, {"in_dtype": "f32"}),
    (1, 129, 4, 2, 16, 128, {}),
    (1, 100, 2, 1, 128, 16, {}),
    (1, 200, 8, 1, 32, 32, {}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}-T{}-H{}x{}-dk{}-dv{}".format(*c[:6]) + (
    "-" + "-".join(f"{k}" for k in c[6]) if c[6] else ""))
def test_scalar_gate(case):
    B, T, Hq, Hkv, dk, dv, opt = case
    announce(f"scalar gate {case}")
    x = scalar_inputs(B, T, Hq, Hkv, dk, dv, **opt)
    got = run(x)
    check(got, oracle_fwd_for(x), oracle_bwd_for(x), f32_inputs=opt.get("in_dtype") == "f32")


def test_scalar_gate_single_token_forward():
    announce("scalar gate single token")
    x = scalar_inputs(1, 1, 1, 1, 64, 64, backward=False)
    check(run(x, backward=False), oracle_fwd_for(x), None)


def test_scalar_gate_logits_no_norm():
    announce("scalar gate logits, no norm")
    x = scalar_inputs(2, 300, 4, 2, 64, 64, o_gate=True, gate=(2.0, 2.0))
    got = run(x, o_norm=False, gate_logits=True)
    check(got, oracle_fwd_for(x, o_norm=False, gate_logits=True), oracle_bwd_for(x, o_norm=False, gate_logits=True),
          o_norm=False)


def test_scalar_gate_full_size_sampled():
    """The training shape (B=4, T=8192, Hq=Hkv=16, d=128) with a scalar gate, as the benchmark
    runs it: o and dq on the last 256 rows, dk, dv and dg on the last 256 keys of two
    (sequence, kv head) units, from the full sequences."""
    announce("scalar gate full size")
    x = scalar_inputs(4, 8192, 16, 16, 128, 128, gate=(4.0, 2.0), seed=5)
    got = run(x)
    mask = np.zeros((4, 16), np.uint8)
    mask[0, 0] = mask[3, 15] = 1
    rf = oracle_fwd_for(x, unit_mask=mask, window=256)
    rb = oracle_bwd_for(x, unit_mask=mask, window=256)
    e = {"o": err_rms(got["o"], rf["o"])}
    for n in ("dq", "dk", "dv", "dg"):
        e[n] = err_rms(got[n], rb[n])
    print("errors:", {k: f"{v:.2e}" for k, v in e.items()}, flush=True)
    for n, v in e.items():
        assert v <= (TOL_DG if n == "dg" else TOL), f"{n}: {v:.3e}"


def test_scalar_gate_full_size_first_keys():
    """Training shape, scalar gate: dq of the first 256 rows and dk, dv of the first 256 keys
    of one unit, whose gradients gather every later query of the sequence."""
    announce("scalar gate full size, first keys")
    x = scalar_inputs(4, 8192, 16, 16, 128, 128, gate=(4.0, 2.0), seed=5)
    got = run(x)
    mask = np.zeros((4, 16), np.uint8)
    mask[2, 7] = 1
    rb = oracle_bwd_for(x, unit_mask=mask, window=-256)
    e = {n: err_rms(got[n], rb[n]) for n in ("dq", "dk", "dv")}
    print("errors:", {k: f"{v:.2e}" for k, v in e.items()}, flush=True)
    for n, v in e.items():
        assert v <= TOL, f"{n}: {v:.3e}"
