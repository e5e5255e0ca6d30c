"""GPU parity of the decode path (fix_decode_* through the C ABI).

The output of a decode step for the newest token t of a sequence is row t of
the forward over the tokens the cache holds, so the reference is the fp64
oracle's forward (no arithmetic of its own): all rows for small cases, and
only the last row of each sequence (window = 1) at large sizes.  Bar: max
|gpu - oracle| / rms(oracle) <= 1e-2 on o (fp32 output), and m within 1e-3
relative of the oracle's row max.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_softmax_attention_amd as F
from gpu_util import announce, custom_inputs, err_rms, needs_gpu, oracle_fwd_for, to_dev

pytestmark = [pytest.mark.gpu, needs_gpu]
TOL = 1e-2


def _dt(x):
    return torch.bfloat16 if x["workload"].in_dtype == "bf16" else torch.float32


def make_cache(x, cap, *, o_norm=True, gate_logits=False, eps=1e-5):
    wl = x["workload"]
    return F.DecodeCache(wl.B, cap, wl.Hq, wl.Hkv, wl.dk, wl.dv, dtype=_dt(x), out_dtype=torch.float32,
                         o_norm=o_norm, gate_logits=gate_logits, eps=eps)


def step(cache, x, t, *, o_norm=True):
    """Decode step with the query (and output gate) of token t of every row."""
    dt = _dt(x)
    z = None if x["z"] is None else to_dev(x["z"][:, t], dt)
    o, m = cache.step(to_dev(x["q"][:, t], dt), to_dev(x["w"], dt) if o_norm else None, z)
    torch.cuda.synchronize()
    return o.cpu().numpy(), m.cpu().numpy()


def append(cache, x, t0, t1, *, gate_logits=False, n_seq=None):
    dt = _dt(x)
    g = x["g_logits"] if gate_logits else x["g"]
    ns = None if n_seq is None else torch.tensor(n_seq, dtype=torch.int32, device="cuda")
    cache.append(to_dev(x["k"][:, t0:t1], dt), to_dev(x["v"][:, t0:t1], dt), to_dev(g[:, t0:t1], torch.float32),
                 ns)


def check(o, m, ref_o, ref_m, what):
    e = err_rms(o, ref_o)
    em = float(np.max(np.abs(m - ref_m) / np.maximum(1.0, np.abs(ref_m))))
    print(f"{what}: o err {e:.2e}, m err {em:.2e}", flush=True)
    assert e <= TOL, f"{what}: o {e:.3e}"
    assert em <= 1e-3, f"{what}: m {em:.3e}"


CASES = [
    # B, T, Hq, Hkv, dk, dv, options; positions stepped (tokens appended up to each in turn)
    ((2, 300, 4, 2, 64, 64, {}), [0, 1, 62, 63, 64, 65, 127, 128, 200, 299]),
    ((1, 200, 8, 1, 128, 128, {"o_gate": True}), [63, 64, 150, 199]),
    ((1, 160, 32, 1, 32, 128, {}), [31, 127, 159]),
    ((2, 130, 2, 2, 16, 16, {}), [0, 63, 64, 129]),
    ((1, 140, 2, 1, 128, 16, {}), [100, 139]),
    ((1, 140, 2, 2, 16, 128, {}), [64, 139]),
    ((1, 200, 4, 4, 64, 32, {"in_dtype": "f32"}), [70, 199]),
    ((1, 700, 4, 2, 128, 128, {"gate": (8.0, 1.0)}), [640, 699]),     # long memory: far chunks dominate
    ((1, 300, 2, 1, 64, 64, {"gate": (-3.0, 1.0)}), [150, 299]),      # strong forgetting
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}-T{}-H{}x{}-dk{}-dv{}".format(*c[0][:6]))
def test_decode_positions(case):
    (B, T, Hq, Hkv, dk, dv, opt), positions = case
    announce(f"decode {case}")
    x = custom_inputs(B, T, Hq, Hkv, dk, dv, backward=False, **opt)
    ref = oracle_fwd_for(x)
    cache = make_cache(x, cap=((T + 63) // 64) * 64)
    t = 0
    for p in positions:
        append(cache, x, t, p + 1)
        t = p + 1
        o, m = step(cache, x, p)
        check(o, m, ref["o"][:, p], ref["m"][:, p], f"token {p}")


def test_decode_gate_logits_no_norm():
    announce("decode gate logits, no norm")
    x = custom_inputs(2, 200, 4, 2, 64, 64, backward=False, o_gate=True, gate=(3.0, 1.5))
    ref = oracle_fwd_for(x, o_norm=False, gate_logits=True)
    cache = make_cache(x, 256, o_norm=False, gate_logits=True)
    append(cache, x, 0, 130, gate_logits=True)
    o, m = step(cache, x, 129, o_norm=False)
    check(o, m, ref["o"][:, 129], ref["m"][:, 129], "token 129")
    append(cache, x, 130, 200, gate_logits=True)
    o, m = step(cache, x, 199, o_norm=False)
    check(o, m, ref["o"][:, 199], ref["m"][:, 199], "token 199")


def test_decode_ragged_and_empty():
    """Per-sequence token counts (n_seq), one sequence left empty (o = 0, m = 0)."""
    announce("decode ragged lengths")
    x = custom_inputs(4, 260, 4, 2, 64, 64, backward=False)
    ref = oracle_fwd_for(x)
    cache = make_cache(x, 320)
    lens = [260, 1, 0, 129]
    append(cache, x, 0, 260, n_seq=lens)
    # each row's query is the one of its own newest token
    dt = _dt(x)
    q = np.stack([x["q"][b, max(L - 1, 0)] for b, L in enumerate(lens)])
    z = None
    o, m = cache.step(to_dev(q, dt), to_dev(x["w"], dt), z)
    torch.cuda.synchronize()
    o, m = o.cpu().numpy(), m.cpu().numpy()
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(o[b] == 0) and np.all(m[b] == 0), "empty sequence"
        else:
            check(o[b], m[b], ref["o"][b, L - 1], ref["m"][b, L - 1], f"row {b} token {L - 1}")


def test_decode_full_cache_drops_extra_tokens():
    announce("decode full cache")
    x = custom_inputs(1, 192, 2, 1, 64, 64, backward=False)
    ref = oracle_fwd_for(x)
    cache = make_cache(x, 128)
    append(cache, x, 0, 128)
    o1, m1 = step(cache, x, 127)
    check(o1, m1, ref["o"][:, 127], ref["m"][:, 127], "token 127")
    append(cache, x, 128, 192)  # past the capacity: dropped
    o2, m2 = step(cache, x, 127)
    assert np.array_equal(o1, o2) and np.array_equal(m1, m2)


def test_decode_reset_reuses_the_cache():
    announce("decode reset")
    x = custom_inputs(1, 100, 2, 2, 32, 32, backward=False)
    ref = oracle_fwd_for(x)
    cache = make_cache(x, 128)
    append(cache, x, 0, 100)
    cache.reset()
    append(cache, x, 0, 70)
    o, m = step(cache, x, 69)
    check(o, m, ref["o"][:, 69], ref["m"][:, 69], "token 69 after reset")


@pytest.mark.parametrize("T", [8192])
def test_decode_full_size_last_token(T):
    """The decode shape of the benchmark (B=4, Hq=Hkv=16, d=128, T tokens held),
    checked on the last row of every sequence and head."""
    announce(f"decode full size T={T}")
    x = custom_inputs(4, T, 16, 16, 128, 128, backward=False, gate=(4.0, 2.0), seed=11)
    ref = O_last_rows(x)
    cache = make_cache(x, T)
    append(cache, x, 0, T)
    o, m = step(cache, x, T - 1)
    check(o, m, ref["o"][:, T - 1], ref["m"][:, T - 1], f"token {T - 1}")


def O_last_rows(x):
    return oracle_fwd_for(x, window=1)
