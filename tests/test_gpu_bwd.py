"""Backward parity: the HIP path against the fp64 oracle on identical seeded inputs.

Bar (fp32 outputs): max |gpu - oracle| / rms(oracle) <= 1e-2 for dq, dk, dv,
d(o_norm_weight) and d(o_gate), and <= 5e-3 for dg.
"""
import numpy as np
import pytest
import torch

import gated_softmax_attention_amd as F
from gated_softmax_attention_amd import synth
from gpu_util import (announce, custom_inputs, device_inputs, err_rms, needs_gpu, oracle_bwd_for)

pytestmark = [pytest.mark.gpu, needs_gpu]
TOL, TOL_DG = 1e-2, 5e-3


def run_bwd(x, *, o_norm=True, eps=1e-5, gate_logits=False):
    d = device_inputs(x)
    w = d["w"] if o_norm else None
    g = d["g_logits"] if gate_logits else d["g"]
    o, m, rstd, xx = F.forward(d["q"], d["k"], d["v"], g, d["cu_seqlens"], o_norm=o_norm, o_norm_weight=w,
                               o_gate=d["z"], eps=eps, gate_logits=gate_logits)
    dq, dk, dv, dg, dw, dz = F.backward(d["q"], d["k"], d["v"], g, m, rstd, xx, d["dO"], d["cu_seqlens"],
                                        o_norm=o_norm, o_norm_weight=w, o_gate=d["z"], eps=eps,
                                        out_dtype=torch.float32, need_dw=True, need_dz=True,
                                        gate_logits=gate_logits)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.float().cpu().numpy()
    return {"dq": cpu(dq), "dk": cpu(dk), "dv": cpu(dv), "dg": cpu(dg), "dw": cpu(dw), "dz": cpu(dz)}


def check_bwd(got, ref, *, check_dw=True, floors=None):
    floors = floors or {}
    e = {n: err_rms(got[n], ref[n], floor=floors.get(n, 0.0)) for n in ("dq", "dk", "dv", "dg")}
    if got["dz"] is not None:
        e["dz"] = err_rms(got["dz"], ref["dz"])
    if check_dw and got["dw"] is not None:
        e["dw"] = err_rms(got["dw"], ref["dw"])
    print("errors:", {k: f"{v:.2e}" for k, v in e.items()}, flush=True)
    for n, v in e.items():
        assert v <= (TOL_DG if n == "dg" else TOL), f"{n}: {v:.3e}"


@pytest.mark.parametrize("name", ["quick", "varlen"])
def test_bwd_config(name):
    announce(f"bwd config {name}")
    x = synth.make_inputs(name)
    check_bwd(run_bwd(x), oracle_bwd_for(x))


EDGES = [
    (1, 2, 1, 1, 64, 64, {}),
    (2, 63, 2, 1, 32, 32, {}),
    (1, 128, 2, 2, 128, 128, {}),
    (1, 129, 4, 2, 16, 128, {}),
    (1, 100, 2, 1, 128, 16, {}),
    (2, 257, 4, 4, 64, 64, {"o_gate": True}),
    (1, 300, 3, 1, 32, 64, {}),
    (1, 591, 4, 2, 64, 64, {"lengths": (1, 0, 65, 130, 5, 300, 90)}),
    (1, 300, 2, 1, 64, 64, {"gate": (-3.0, 1.0)}),
    (1, 700, 4, 2, 128, 128, {"gate": (0.0, 1.0)}),
    (1, 257, 2, 2, 32, 16, {"in_dtype": "f32"}),
    (1, 384, 2, 2, 16, 16, {}),
    (3, 170, 2, 2, 128, 64, {"o_gate": True, "gate": (1.0, 2.0)}),
    # long memory (g about -3e-4 per token): pairs two or more chunks apart carry most of
    # the weight, so the inter-chunk kernels decide the result
    (1, 1100, 4, 2, 64, 64, {"gate": (8.0, 1.0)}),
    (2, 640, 2, 1, 128, 128, {"gate": (10.0, 0.5), "o_gate": True}),
    (1, 1024, 4, 4, 32, 128, {"gate": (8.0, 1.0), "lengths": (384, 129, 511)}),
]


@pytest.mark.parametrize("case", EDGES, ids=lambda c: "B{}-T{}-H{}x{}-dk{}-dv{}".format(*c[:6]) + (
    "-" + "-".join(f"{k}" for k in c[6]) if c[6] else ""))
def test_bwd_edges(case):
    B, T, Hq, Hkv, dk, dv, extra = case
    announce(f"bwd edge {case}")
    x = custom_inputs(B, T, Hq, Hkv, dk, dv, **extra)
    check_bwd(run_bwd(x), oracle_bwd_for(x))


def _cancel_scale(x, ref):
    """rms of v (.) dv: dG = sum_h delta (.) x - v (.) dv cancels to zero in the cases below."""
    return float(np.sqrt(np.mean((x["v"].astype(np.float64) * ref["dv"]) ** 2)))


def test_bwd_infinite_gate():
    """g = -1e4: only diagonal pairs survive, so dG = delta x - v dv is exactly 0 per token;
    dg is then compared against the scale of the two cancelling terms."""
    announce("bwd g=-1e4")
    x = custom_inputs(1, 200, 2, 1, 64, 64)
    x["g"][:] = -1e4
    ref = oracle_bwd_for(x)
    check_bwd(run_bwd(x), ref, floors={"dg": _cancel_scale(x, ref)})


def test_bwd_single_token():
    """T = 1 without the norm: x = v, dv = delta, so dG (and dg) vanish exactly."""
    announce("bwd T=1")
    x = custom_inputs(2, 1, 2, 1, 64, 64)
    ref = oracle_bwd_for(x, o_norm=False)
    check_bwd(run_bwd(x, o_norm=False), ref, check_dw=False, floors={"dg": _cancel_scale(x, ref)})


def test_bwd_no_norm():
    announce("bwd o_norm off")
    x = custom_inputs(1, 333, 4, 2, 64, 32, o_gate=True)
    check_bwd(run_bwd(x, o_norm=False), oracle_bwd_for(x, o_norm=False), check_dw=False)


def test_bwd_autograd_matches_entry_points():
    """parallel_fix_attn's autograd gradients are the entry points' gradients."""
    announce("bwd autograd")
    x = custom_inputs(1, 300, 4, 2, 64, 64, o_gate=True)
    d = device_inputs(x)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "w", "z")}
    o = F.parallel_fix_attn(leaves["q"], leaves["k"], leaves["v"], leaves["g"], o_norm=True,
                            o_norm_weight=leaves["w"], o_gate=leaves["z"])
    (o.float() * d["dO"].float()).sum().backward()
    o2, m, rstd, xx = F.forward(d["q"], d["k"], d["v"], d["g"], o_norm=True, o_norm_weight=d["w"], o_gate=d["z"])
    ref = F.backward(d["q"], d["k"], d["v"], d["g"], m, rstd, xx, d["dO"], o_norm=True, o_norm_weight=d["w"],
                     o_gate=d["z"], need_dw=True, need_dz=True)
    assert torch.equal(o, o2)
    for name, r in zip(("q", "k", "v", "g", "w", "z"), ref):
        # autograd hands each gradient back in its input's dtype
        assert torch.equal(leaves[name].grad, r.to(leaves[name].dtype)), name


def test_bwd_nan_poison_determinism():
    """NaN-filled outputs and workspace are fully overwritten, and two runs give equal bits."""
    announce("bwd poison/determinism")
    x = custom_inputs(1, 700, 4, 2, 64, 64, lengths=(300, 1, 0, 399), o_gate=True)
    d = device_inputs(x)
    o, m, rstd, xx = F.forward(d["q"], d["k"], d["v"], d["g"], d["cu_seqlens"], o_norm=True, o_norm_weight=d["w"],
                               o_gate=d["z"])
    desc = F.make_desc(d["q"], d["k"], d["v"], d["cu_seqlens"], o_norm=True, out_dtype=torch.float32)
    wsb = F.fix_attn_bwd_workspace_size(desc)
    outs = []
    for _ in range(2):
        nan = float("nan")
        t = [torch.full(d[n].shape, nan, device="cuda") for n in ("q", "k", "v", "g")]
        dw = torch.full((d["v"].shape[3],), nan, device="cuda")
        dz = torch.full(d["z"].shape, nan, device="cuda")
        ws = torch.full((wsb // 4 + 1,), nan, device="cuda")
        F.fix_attn_bwd(desc, d["q"], d["k"], d["v"], d["g"], d["w"], d["z"], m, rstd, xx, d["dO"], t[0], t[1], t[2],
                       t[3], dw, dz, ws, wsb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        outs.append([a.cpu() for a in (*t, dw, dz)])
    for a, b in zip(*outs):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


def _unit_mask(wl, units):
    m = np.zeros((wl.B, wl.Hkv), np.uint8)
    for s, c in units:
        m[s, c] = 1
    return m


@pytest.mark.parametrize("name,units", [
    ("train", [(1, 2), (3, 15)]),
    ("long_d16", [(0, 1)]),
    ("long_d32", [(0, 6)]),
    ("long_d64", [(0, 2)]),
    ("long_d128", [(0, 4)]),
])
def test_bwd_full_size_sampled(name, units):
    """Full-size workloads as the benchmark runs them; the oracle recomputes dq of the last 256
    rows and dk, dv, dg of the last 256 keys of the selected (sequence, kv head) units."""
    announce(f"bwd full-size {name}")
    x = synth.make_inputs(name)
    got = run_bwd(x)
    ref = oracle_bwd_for(x, unit_mask=_unit_mask(x["workload"], units), window=256)
    check_bwd(got, ref, check_dw=False)


FIRST_KEYS = [
    ("train", [(0, 5), (2, 11)]),
    ("long_d16", [(0, 3)]),
    ("long_d32", [(0, 0)]),
    ("long_d64", [(0, 5)]),
    ("long_d128", [(0, 7)]),
]


@pytest.mark.parametrize("name,units", FIRST_KEYS)
def test_bwd_full_size_first_keys(name, units):
    """Full-size workloads as the benchmark runs them: dq of the first 256 rows and dk, dv of
    the first 256 keys of the selected units, whose gradients gather every later query (the
    inter-chunk kernels' work); the oracle computes the units' whole forward for them."""
    announce(f"bwd full-size {name}, first keys")
    x = synth.make_inputs(name)
    got = run_bwd(x)
    ref = oracle_bwd_for(x, unit_mask=_unit_mask(x["workload"], units), window=-256)
    e = {n: err_rms(got[n], ref[n]) for n in ("dq", "dk", "dv")}
    print("errors:", {k: f"{v:.2e}" for k, v in e.items()}, flush=True)
    for n, v in e.items():
        assert v <= TOL, f"{n}: {v:.3e}"


def test_bwd_full_size_dw():
    """Training shape: d(o_norm_weight) is a sum over every row of every head.  With dO zero
    outside the last 256 rows of two units (the gradient is linear in dO), only those rows
    contribute, and the oracle computes exactly them; dq, dk, dv, dg of the units are checked
    on the same input."""
    announce("bwd full-size train, dw")
    x = dict(synth.make_inputs("train"))
    wl = x["workload"]
    units = [(1, 4), (3, 9)]
    G = wl.Hq // wl.Hkv
    keep = np.zeros(x["dO"].shape, bool)
    for s_, c in units:
        keep[s_, wl.T - 256:, c * G:(c + 1) * G] = True
    x["dO"] = np.where(keep, x["dO"], 0.0).astype(x["dO"].dtype)
    x["w"] = synth.make_inputs("quick")["w"][:wl.dv].copy()  # a weight that is not all ones
    got = run_bwd(x)
    ref = oracle_bwd_for(x, unit_mask=_unit_mask(wl, units), window=256)
    check_bwd(got, ref, check_dw=True)


# The gate given as raw logits: dg is the gradient with respect to the logits.
LOGIT_CASES = [
    (1, 640, 4, 2, 64, 64, {"lengths": (100, 300, 240), "o_gate": True, "gate": (3.0, 1.5)}),
    (2, 300, 2, 2, 128, 128, {"gate": (0.0, 2.0)}),
]


@pytest.mark.parametrize("case", LOGIT_CASES, ids=lambda c: "B{}-T{}-H{}x{}-dk{}-dv{}".format(*c[:6]))
def test_bwd_gate_logits(case):
    B, T, Hq, Hkv, dk, dv, extra = case
    announce(f"bwd gate logits {case}")
    x = custom_inputs(B, T, Hq, Hkv, dk, dv, **extra)
    check_bwd(run_bwd(x, gate_logits=True), oracle_bwd_for(x, gate_logits=True))
