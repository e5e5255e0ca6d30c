"""Checks that pin the fp64 oracle to facts outside itself.

Each function takes an oracle library handle (so the mutation tests can run
the same checks against deliberately broken builds) and returns the worst
relative error it found; the caller compares that with a tolerance.

Nothing here re-types the oracle's loops.  The checks use:
  * closed forms that the method reduces to -- no gate gives causal softmax
    attention followed by RMSNorm, because the dropped softmax denominator
    is a positive per-row scale that RMSNorm removes (FiX ICML 2026 poster
    page, abstract); a gate that is equal across channels gives forgetting
    attention, whose gate enters as an additive logit bias (Forgetting
    Transformer page, abstract); a gate at minus infinity keeps only the
    diagonal term; both are evaluated with torch's own attention routine;
  * central finite differences of the forward for every gradient;
  * structural identities (packing, GQA, scale invariance, the first token
    of a sequence never sees its own gate);
  * an independent dense fp64 reference written with torch tensor ops and
    autograd, where the decay is exp of a difference of prefix sums.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def rand_case(rng, B, T, Hq, Hkv, dk, dv, gate=(1.0, 1.0), lengths=None):
    q = rng.standard_normal((B, T, Hq, dk))
    k = rng.standard_normal((B, T, Hkv, dk))
    v = rng.standard_normal((B, T, Hkv, dv))
    g = -np.logaddexp(0.0, -(rng.standard_normal((B, T, Hkv, dv)) * gate[1] + gate[0]))
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, g, cu


def rmsnorm0(x):
    """RMSNorm without eps over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    # q [T,H,dk] etc. in numpy -> torch [1,H,T,d]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask)[None],
        is_causal=causal, scale=scale)
    return out[0].numpy().transpose(1, 0, 2)


def pin_no_gate_is_softmax_attention(lib, rng):
    """g = 0: o = RMSNorm(causal softmax attention) at eps = 0 (GQA, packed)."""
    lengths = [37, 1, 50]
    q, k, v, g, cu = rand_case(rng, 1, sum(lengths), 4, 2, 16, 24, lengths=lengths)
    g[:] = 0.0
    w = rng.standard_normal(24)
    o = O.oracle_fwd(q, k, v, g, cu, eps=0.0, w=w, lib=lib)["o"][0]
    worst = 0.0
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        kr = np.repeat(k[0, a:b], 2, axis=1)
        vr = np.repeat(v[0, a:b], 2, axis=1)
        ref = rmsnorm0(_sdpa(q[0, a:b], kr, vr, causal=True, scale=16 ** -0.5)) * w
        worst = max(worst, rel(o[a:b], ref))
    return worst


def pin_no_gate_unnormalised(lib, rng):
    """g = 0, o_norm off: x_i = softmax-attention_i * sum_j exp(s_ij - max_j s_ij)."""
    q, k, v, g, _ = rand_case(rng, 1, 40, 2, 2, 8, 8)
    g[:] = 0.0
    r = O.oracle_fwd(q, k, v, g, o_norm=False, lib=lib)
    att = _sdpa(q[0], k[0], v[0], causal=True, scale=8 ** -0.5)
    s = torch.einsum("ihd,jhd->hij", torch.from_numpy(q[0]), torch.from_numpy(k[0])) * 8 ** -0.5
    s = s.masked_fill(~torch.ones(40, 40, dtype=torch.bool).tril(), float("-inf"))
    m = s.amax(-1)
    z = torch.exp(torch.logsumexp(s, -1) - m)           # [H, T]
    ref = att * z.numpy().T[:, :, None]
    return max(rel(r["o"][0], ref), rel(r["m"][0], m.numpy().T))


def pin_scalar_gate_is_forgetting_attention(lib, rng):
    """Gate equal across channels: o = RMSNorm(softmax(s_ij + F_i - F_j) v) at eps = 0."""
    T, H = 45, 2
    q, k, v, g, _ = rand_case(rng, 1, T, H, H, 8, 12)
    f = -np.logaddexp(0.0, -rng.standard_normal((T, H)))          # per-token log forget gate
    g[0] = f[:, :, None]
    o = O.oracle_fwd(q, k, v, g, eps=0.0, lib=lib)["o"][0]
    F = np.cumsum(f, axis=0)                                       # [T, H]
    bias = F.T[:, :, None] - F.T[:, None, :]                       # [H, i, j] = F_i - F_j
    bias = np.where(np.tril(np.ones((T, T), bool))[None], bias, -np.inf)
    ref = rmsnorm0(_sdpa(q[0], k[0], v[0], mask=bias, scale=8 ** -0.5))
    return rel(o, ref)


def pin_infinite_gate_keeps_diagonal(lib, rng):
    """g -> -inf: only the j = i term survives, o_i = RMSNorm(v_i) * w * z (eps = 0)."""
    q, k, v, g, _ = rand_case(rng, 2, 20, 4, 2, 8, 16)
    g[:] = -1e4
    w = rng.standard_normal(16)
    z = rng.standard_normal((2, 20, 4, 16))
    o = O.oracle_fwd(q, k, v, g, eps=0.0, w=w, z=z, lib=lib)["o"]
    ref = rmsnorm0(np.repeat(v, 2, axis=2)) * w * z
    return rel(o, ref)


def pin_single_token(lib, rng):
    """T = 1: o = RMSNorm(v) (eps = 0) whatever q, k, g are."""
    q, k, v, g, _ = rand_case(rng, 3, 1, 2, 1, 16, 8, gate=(-3.0, 2.0))
    o = O.oracle_fwd(q, k, v, g, eps=0.0, lib=lib)["o"]
    return rel(o, rmsnorm0(np.repeat(v, 2, axis=2)))


def pin_gate_and_weight_algebra(lib, rng):
    """o(w, z) = o(1, 1) * w * z elementwise."""
    q, k, v, g, _ = rand_case(rng, 1, 30, 2, 1, 8, 8)
    w = rng.standard_normal(8)
    z = rng.standard_normal((1, 30, 2, 8))
    a = O.oracle_fwd(q, k, v, g, eps=1e-5, lib=lib)["o"]
    b = O.oracle_fwd(q, k, v, g, eps=1e-5, w=w, z=z, lib=lib)["o"]
    return rel(b, a * w * z)


def _loss(lib, args, dO, **kw):
    o = O.oracle_fwd(*args, lib=lib, **kw)["o"]
    return float(np.sum(o * dO))


def pin_finite_differences(lib, rng, eps=0.0):
    """Every gradient against central differences of sum(o * dO).

    At eps = 0 the row max drops out of o, so the frozen-max gradient is the
    true gradient; at eps > 0 the max is frozen on both sides.
    """
    lengths = [2, 5]
    q, k, v, g, cu = rand_case(rng, 1, 7, 2, 1, 3, 4, gate=(0.5, 1.0), lengths=lengths)
    w = rng.standard_normal(4)
    z = rng.standard_normal((1, 7, 2, 4))
    dO = rng.standard_normal((1, 7, 2, 4))
    base = O.oracle_fwd(q, k, v, g, cu, eps=eps, w=w, z=z, lib=lib)
    m_in = base["m"] if eps > 0 else None
    kw = dict(eps=eps, w=w, z=z, m_in=m_in)
    grads = O.oracle_bwd(q, k, v, g, dO, cu, lib=lib, **kw)
    worst = 0.0
    h = 1e-6
    for name, gname in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("w", "dw"), ("z", "dz")]:
        arrs = {"q": q, "k": k, "v": v, "g": g, "w": w, "z": z}
        fd = np.zeros_like(arrs[name])
        for idx in np.ndindex(arrs[name].shape):
            vals = []
            for sgn in (1, -1):
                a2 = {kk: vv.copy() for kk, vv in arrs.items()}
                a2[name][idx] += sgn * h
                kw2 = dict(kw, w=a2["w"], z=a2["z"])
                vals.append(_loss(lib, (a2["q"], a2["k"], a2["v"], a2["g"], cu), dO, **kw2))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        worst = max(worst, rel(grads[gname], fd))
    return worst


def pin_first_token(lib, rng):
    """dg is zero at every sequence start; o at a sequence start ignores g."""
    lengths = [9, 4, 11]
    q, k, v, g, cu = rand_case(rng, 1, 24, 2, 2, 8, 8, lengths=lengths)
    dO = rng.standard_normal((1, 24, 2, 8))
    dg = O.oracle_bwd(q, k, v, g, dO, cu, lib=lib)["dg"][0]
    scale = np.sqrt(np.mean(dg * dg))
    worst = max(np.abs(dg[cu[:-1]]).max() / scale, 0.0)
    o1 = O.oracle_fwd(q, k, v, g, cu, lib=lib)["o"][0]
    g2 = g + rng.uniform(-3, 0, g.shape)
    o2 = O.oracle_fwd(q, k, v, g2, cu, lib=lib)["o"][0]
    worst = max(worst, rel(o2[cu[:-1]], o1[cu[:-1]]))
    # and the gate is not ignored elsewhere
    assert rel(o2, o1) > 1e-3
    return worst


def pin_packing(lib, rng):
    """Packed sequences give the same results as separate calls (fwd and bwd)."""
    lengths = [13, 1, 20, 6]
    q, k, v, g, cu = rand_case(rng, 1, 40, 4, 2, 8, 12, lengths=lengths)
    dO = rng.standard_normal((1, 40, 4, 12))
    z = rng.standard_normal((1, 40, 4, 12))
    fp = O.oracle_fwd(q, k, v, g, cu, z=z, lib=lib)
    bp = O.oracle_bwd(q, k, v, g, dO, cu, z=z, lib=lib)
    worst = 0.0
    dw_sum = np.zeros(12)
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        sl = lambda t: t[:, a:b]
        f1 = O.oracle_fwd(sl(q), sl(k), sl(v), sl(g), z=sl(z), lib=lib)
        b1 = O.oracle_bwd(sl(q), sl(k), sl(v), sl(g), sl(dO), z=sl(z), lib=lib)
        worst = max(worst, rel(fp["o"][:, a:b], f1["o"]))
        for n in ("dq", "dk", "dv", "dg", "dz"):
            worst = max(worst, rel(bp[n][:, a:b], b1[n]))
        dw_sum += b1["dw"]
    return max(worst, rel(bp["dw"], dw_sum))


def pin_gqa(lib, rng):
    """GQA equals MHA with k, v, g repeated per group; kv gradients sum over the group."""
    q, k, v, g, _ = rand_case(rng, 2, 17, 6, 2, 8, 8)
    dO = rng.standard_normal((2, 17, 6, 8))
    rep = lambda t: np.repeat(t, 3, axis=2)
    fa = O.oracle_fwd(q, k, v, g, lib=lib)
    fb = O.oracle_fwd(q, rep(k), rep(v), rep(g), lib=lib)
    ba = O.oracle_bwd(q, k, v, g, dO, lib=lib)
    bb = O.oracle_bwd(q, rep(k), rep(v), rep(g), dO, lib=lib)
    grp = lambda t: t.reshape(t.shape[0], t.shape[1], 2, 3, t.shape[3]).sum(axis=3)
    worst = rel(fa["o"], fb["o"])
    worst = max(worst, rel(ba["dq"], bb["dq"]))
    for n in ("dk", "dv", "dg"):
        worst = max(worst, rel(ba[n], grp(bb[n])))
    return worst


def pin_value_scale(lib, rng):
    """eps = 0: scaling v by c > 0 leaves o unchanged and divides dv by c."""
    q, k, v, g, _ = rand_case(rng, 1, 25, 2, 1, 8, 8)
    dO = rng.standard_normal((1, 25, 2, 8))
    c = 3.7
    a = O.oracle_fwd(q, k, v, g, eps=0.0, lib=lib)["o"]
    b = O.oracle_fwd(q, k, c * v, g, eps=0.0, lib=lib)["o"]
    da = O.oracle_bwd(q, k, v, g, dO, eps=0.0, lib=lib)["dv"]
    db = O.oracle_bwd(q, k, c * v, g, dO, eps=0.0, lib=lib)["dv"]
    return max(rel(b, a), rel(db * c, da))


def dense_reference(q, k, v, g, dO, cu=None, eps=1e-5, w=None, z=None, o_norm=True):
    """Independent dense fp64 torch implementation with autograd gradients.

    Decays are exp(G_i - G_j) from a prefix sum G (inclusive), masked above the
    diagonal; the row max is excluded from differentiation.
    """
    B, T, Hq, dk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    G = Hq // Hkv
    tq, tk, tv, tg = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, g))
    tw = torch.tensor(np.ones(dv) if w is None else w, dtype=torch.float64, requires_grad=True)
    tz = None if z is None else torch.tensor(z, dtype=torch.float64, requires_grad=True)
    bounds = [(b, 0, T) for b in range(B)] if cu is None else [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    outs = torch.zeros(B, T, Hq, dv, dtype=torch.float64)
    pieces = []
    for b, a, e in bounds:
        L = e - a
        if L == 0:
            continue
        qq = tq[b, a:e]                                   # [L, Hq, dk]
        kk = tk[b, a:e].repeat_interleave(G, dim=1)       # [L, Hq, dk]
        vv = tv[b, a:e].repeat_interleave(G, dim=1)
        Gc = torch.cumsum(tg[b, a:e], dim=0).repeat_interleave(G, dim=1)   # [L, Hq, dv]
        s = torch.einsum("ihd,jhd->hij", qq, kk) * dk ** -0.5
        causal = torch.ones(L, L, dtype=torch.bool).tril()
        s = s.masked_fill(~causal, float("-inf"))
        m = s.detach().amax(-1, keepdim=True)
        P = torch.exp(s - m)                              # [Hq, L, L]
        dlog = Gc[:, None] - Gc[None, :]                  # [i, j, Hq, dv]
        dlog = dlog.masked_fill(~causal[:, :, None, None], float("-inf"))
        x = torch.einsum("hij,ijhd,jhd->ihd", P, torch.exp(dlog), vv)
        if o_norm:
            o = x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * tw
        else:
            o = x
        if tz is not None:
            o = o * tz[b, a:e]
        pieces.append((b, a, e, o))
    loss = sum((o * torch.tensor(dO[b, a:e])).sum() for b, a, e, o in pieces)
    loss.backward()
    for b, a, e, o in pieces:
        outs[b, a:e] = o.detach()
    res = {"o": outs.numpy(), "dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy(),
           "dg": tg.grad.numpy(), "dw": np.zeros(dv) if tw.grad is None else tw.grad.numpy()}
    if tz is not None:
        res["dz"] = tz.grad.numpy()
    return res


def pin_dense_reference(lib, rng, o_norm=True):
    """Oracle vs the dense autograd reference: packed, GQA, dk != dv, eps > 0, w and z."""
    lengths = [70, 1, 0, 57]
    q, k, v, g, cu = rand_case(rng, 1, 128, 4, 2, 16, 8, gate=(0.0, 1.0), lengths=lengths)
    w = rng.standard_normal(8)
    z = rng.standard_normal((1, 128, 4, 8))
    dO = rng.standard_normal((1, 128, 4, 8))
    ref = dense_reference(q, k, v, g, dO, cu, eps=1e-5, w=w, z=z, o_norm=o_norm)
    f = O.oracle_fwd(q, k, v, g, cu, eps=1e-5, w=w, z=z, o_norm=o_norm, lib=lib)
    b = O.oracle_bwd(q, k, v, g, dO, cu, eps=1e-5, w=w, z=z, o_norm=o_norm, lib=lib)
    worst = rel(f["o"], ref["o"])
    for n in ("dq", "dk", "dv", "dg", "dz"):
        worst = max(worst, rel(b[n], ref[n]))
    if o_norm:
        worst = max(worst, rel(b["dw"], ref["dw"]))
    return worst


def pin_dense_reference_vanishing_decay(lib, rng):
    """Oracle vs the dense autograd reference under gates so strong (logsigmoid of N(-30, 2), and
    -1e4 in half the channels) that the running decay product reaches exactly zero in every
    channel within a few tokens, where the oracle's walks stop, and with zeros in only some
    channels, where they must not: the shortcut must leave every output unchanged."""
    lengths = [60, 3, 61]
    q, k, v, g, cu = rand_case(rng, 1, 124, 4, 2, 16, 8, gate=(-30.0, 2.0), lengths=lengths)
    # half the channels cut off at once everywhere; in the last sequence the other half
    # forgets slowly, so the product is zero in some channels only and the walk must go on
    g[..., :4] = -1e4
    g[0, 63:, :, 4:] = -np.logaddexp(0.0, -(rng.standard_normal((61, 2, 4)) + 2.0))
    dO = rng.standard_normal((1, 124, 4, 8))
    ref = dense_reference(q, k, v, g, dO, cu, eps=1e-5)
    f = O.oracle_fwd(q, k, v, g, cu, eps=1e-5, lib=lib)
    b = O.oracle_bwd(q, k, v, g, dO, cu, eps=1e-5, lib=lib)
    worst = rel(f["o"], ref["o"])
    for n in ("dq", "dk", "dv"):
        worst = max(worst, rel(b[n], ref[n]))
    # dg is a difference of nearly equal terms here (x_t is almost v_t, dv_t almost delta_t):
    # measured against the scale of the cancelling terms, as fp64 cancellation leaves it
    scale = np.sqrt(np.mean((v * ref["dv"]) ** 2))
    return max(worst, float(np.max(np.abs(b["dg"] - ref["dg"])) / scale))


def pin_suffix_window(lib, rng):
    """The sampled (unit mask + suffix window) mode reproduces the full results there."""
    lengths = [30, 45]
    q, k, v, g, cu = rand_case(rng, 1, 75, 4, 2, 8, 8, lengths=lengths)
    dO = rng.standard_normal((1, 75, 4, 8))
    full_f = O.oracle_fwd(q, k, v, g, cu, lib=lib)
    full_b = O.oracle_bwd(q, k, v, g, dO, cu, lib=lib)
    mask = np.array([[0, 1], [1, 0]], np.uint8)
    win_f = O.oracle_fwd(q, k, v, g, cu, unit_mask=mask, window=10, lib=lib)
    win_b = O.oracle_bwd(q, k, v, g, dO, cu, unit_mask=mask, window=10, lib=lib)
    sel = np.zeros((75, 4), bool)
    sel[20:30, 2:4] = True     # sequence 0, kv head 1
    sel[65:75, 0:2] = True     # sequence 1, kv head 0
    selk = np.zeros((75, 2), bool)
    selk[20:30, 1] = True
    selk[65:75, 0] = True
    worst = rel(win_f["o"][0][sel], full_f["o"][0][sel])
    worst = max(worst, rel(win_b["dq"][0][sel], full_b["dq"][0][sel]))
    for n in ("dk", "dv", "dg"):
        worst = max(worst, rel(win_b[n][0][selk], full_b[n][0][selk]))
    assert np.isnan(win_f["o"][0][~sel]).all()
    return worst


def pin_prefix_window(lib, rng):
    """The prefix mode (window < 0) reproduces the full dq of the first rows and dk, dv of the
    first keys of the selected units, and computes nothing else."""
    lengths = [30, 45]
    q, k, v, g, cu = rand_case(rng, 1, 75, 4, 2, 8, 8, lengths=lengths)
    dO = rng.standard_normal((1, 75, 4, 8))
    full_b = O.oracle_bwd(q, k, v, g, dO, cu, lib=lib)
    mask = np.array([[0, 1], [1, 0]], np.uint8)
    pre = O.oracle_bwd(q, k, v, g, dO, cu, unit_mask=mask, window=-7, lib=lib)
    sel = np.zeros((75, 4), bool)
    sel[0:7, 2:4] = True       # sequence 0, kv head 1
    sel[30:37, 0:2] = True     # sequence 1, kv head 0
    selk = np.zeros((75, 2), bool)
    selk[0:7, 1] = True
    selk[30:37, 0] = True
    worst = rel(pre["dq"][0][sel], full_b["dq"][0][sel])
    for n in ("dk", "dv"):
        worst = max(worst, rel(pre[n][0][selk], full_b[n][0][selk]))
    assert np.isnan(pre["dq"][0][~sel]).all() and np.isnan(pre["dk"][0][~selk]).all()
    assert np.isnan(pre["dg"]).all()
    return worst


def pin_logits_finite_differences(lib, rng):
    """Gate given as raw logits x (gate = logsigmoid(x)): every gradient, dg now with respect
    to x, against central differences of sum(o * dO) at eps = 0."""
    lengths = [3, 4]
    q, k, v, _, cu = rand_case(rng, 1, 7, 2, 1, 3, 4, lengths=lengths)
    x = rng.standard_normal((1, 7, 1, 4)) * 1.5 + 0.3  # both signs: both branches of the transform
    dO = rng.standard_normal((1, 7, 2, 4))
    grads = O.oracle_bwd(q, k, v, x, dO, cu, eps=0.0, gate_logits=True, lib=lib)
    loss = lambda qq, kk, vv, xx: float(np.sum(O.oracle_fwd(qq, kk, vv, xx, cu, eps=0.0, gate_logits=True,
                                                                lib=lib)["o"] * dO))
    worst, h = 0.0, 1e-6
    arrs = {"q": q, "k": k, "v": v, "x": x}
    for name, gname in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("x", "dg")]:
        fd = np.zeros_like(arrs[name])
        for idx in np.ndindex(arrs[name].shape):
            vals = []
            for sgn in (1, -1):
                a2 = {kk: vv.copy() for kk, vv in arrs.items()}
                a2[name][idx] += sgn * h
                vals.append(loss(a2["q"], a2["k"], a2["v"], a2["x"]))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        worst = max(worst, rel(grads[gname], fd))
    return worst


def pin_logits_match_logsigmoid(lib, rng):
    """Logits x give what the log gate torch.nn.functional.logsigmoid(x) gives (forward and
    dq, dk, dv), and dg with respect to x is the log-gate dg times torch.sigmoid(-x)."""
    lengths = [11, 1, 20]
    q, k, v, _, cu = rand_case(rng, 1, 32, 4, 2, 8, 8, lengths=lengths)
    x = rng.standard_normal((1, 32, 2, 8)) * 2.0 + 1.0
    dO = rng.standard_normal((1, 32, 4, 8))
    tx = torch.from_numpy(x)
    g = torch.nn.functional.logsigmoid(tx).numpy()
    fa = O.oracle_fwd(q, k, v, x, cu, gate_logits=True, lib=lib)
    fb = O.oracle_fwd(q, k, v, g, cu, lib=lib)
    ba = O.oracle_bwd(q, k, v, x, dO, cu, gate_logits=True, lib=lib)
    bb = O.oracle_bwd(q, k, v, g, dO, cu, lib=lib)
    worst = rel(fa["o"], fb["o"])
    for n in ("dq", "dk", "dv"):
        worst = max(worst, rel(ba[n], bb[n]))
    worst = max(worst, rel(ba["dg"], bb["dg"] * torch.sigmoid(-tx).numpy()))
    return worst


def pin_scalar_gate_finite_differences(lib, rng):
    """A scalar gate (one value per token and kv head, [B,T,Hkv]), plain and as logits: its
    dg against central differences of sum(o * dO) at eps = 0."""
    lengths = [3, 5]
    q, k, v, _, cu = rand_case(rng, 1, 8, 2, 1, 3, 4, lengths=lengths)
    dO = rng.standard_normal((1, 8, 2, 4))
    worst, h = 0.0, 1e-6
    for logits in (False, True):
        x = rng.standard_normal((1, 8, 1)) * 1.5 + (0.3 if logits else -1.0)
        if not logits:
            x = -np.abs(x)  # a forget gate
        dg = O.oracle_bwd(q, k, v, x, dO, cu, eps=0.0, gate_logits=logits, lib=lib)["dg"]
        assert dg.shape == x.shape
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            vals = []
            for sgn in (1, -1):
                x2 = x.copy()
                x2[idx] += sgn * h
                vals.append(float(np.sum(O.oracle_fwd(q, k, v, x2, cu, eps=0.0, gate_logits=logits, lib=lib)["o"]
                                         * dO)))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        worst = max(worst, rel(dg, fd))
    return worst


ALL_PINS = {
    "no_gate_softmax": (pin_no_gate_is_softmax_attention, 1e-12),
    "no_gate_unnormalised": (pin_no_gate_unnormalised, 1e-12),
    "scalar_gate_fox": (pin_scalar_gate_is_forgetting_attention, 1e-12),
    "infinite_gate": (pin_infinite_gate_keeps_diagonal, 1e-12),
    "single_token": (pin_single_token, 1e-12),
    "gate_weight_algebra": (pin_gate_and_weight_algebra, 1e-12),
    "finite_diff_eps0": (lambda lib, rng: pin_finite_differences(lib, rng, 0.0), 1e-6),
    "finite_diff_eps": (lambda lib, rng: pin_finite_differences(lib, rng, 1e-3), 1e-6),
    "first_token": (pin_first_token, 1e-12),
    "packing": (pin_packing, 1e-12),
    "gqa": (pin_gqa, 1e-12),
    "value_scale": (pin_value_scale, 1e-12),
    "dense_reference": (pin_dense_reference, 1e-10),
    "dense_reference_unnormed": (lambda lib, rng: pin_dense_reference(lib, rng, False), 1e-10),
    "dense_reference_vanishing_decay": (pin_dense_reference_vanishing_decay, 1e-10),
    "suffix_window": (pin_suffix_window, 0.0),
    "prefix_window": (pin_prefix_window, 0.0),
    "logits_finite_diff": (pin_logits_finite_differences, 1e-6),
    "logits_match_logsigmoid": (pin_logits_match_logsigmoid, 1e-12),
    "scalar_gate_finite_diff": (pin_scalar_gate_finite_differences, 1e-6),
}
