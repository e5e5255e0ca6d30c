"""Seeded synthetic inputs for FiX attention workloads.

This module only draws random numbers and rounds them to the storage types
the kernels receive; it holds none of the attention arithmetic.  Both the
HIP path (tests, benchmark) and the fp64 oracle consume exactly the arrays
it returns, so the two sides always see bit-identical inputs.

Recipe (one numpy PCG64 stream per tensor, spawned from one SeedSequence in
the fixed order q, k, v, gate pre-activation, o_norm weight, o_gate, dO,
sequence lengths):
  * q, k, v ~ N(0, 1), rounded to bf16 (round-to-nearest-even) unless the
    workload keeps fp32 inputs;
  * the forget gate is g = logsigmoid(x) with x ~ N(mu, sd), evaluated in
    fp64 and stored fp32 -- a log-space gate, so g <= 0 (FiX README, "Quick
    Start": the gate is fp32 and shaped like v);
  * o_norm weight either ones or N(1, 0.1) rounded like q; o_gate ~ N(0, 1);
    dO ~ N(0, 1);
  * packed workloads draw sequence lengths in [64, 4096] that sum to T.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

MASTER_SEED = 42


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even), kept as fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def logsigmoid64(x: np.ndarray) -> np.ndarray:
    """log(1 / (1 + exp(-x))) in fp64 without overflow."""
    return -np.logaddexp(0.0, -np.asarray(x, dtype=np.float64))


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    dk: int
    dv: int
    in_dtype: str = "bf16"          # "bf16" or "f32"
    gate_mu: float = 3.0
    gate_sd: float = 1.5
    w_kind: str = "ones"            # "ones" or "normal"
    o_gate: bool = False
    varlen: bool = False
    backward: bool = True
    lengths: tuple = field(default=())  # explicit packed lengths (overrides the draw)
    index: int = 0                  # seed offset

    @property
    def Ttot(self) -> int:
        return self.B * self.T


WORKLOADS = {
    # T=256 single sequence, fp32 inputs, forward only.
    "tiny": Workload("tiny", 1, 256, 2, 2, 64, 64, in_dtype="f32", gate_mu=2.0, gate_sd=1.0,
                     backward=False, index=0),
    # The Quick Start shapes of the FiX README: GQA 8/4, d=128.
    "quick": Workload("quick", 2, 2048, 8, 4, 128, 128, gate_mu=3.0, gate_sd=1.5, w_kind="normal",
                      index=1),
    # Packed sequences (cu_seqlens) with an output gate.
    "varlen": Workload("varlen", 1, 8192, 16, 4, 64, 64, gate_mu=3.0, gate_sd=1.5, o_gate=True,
                       varlen=True, index=2),
    # Training shape: B=4, T=8192, 16 heads, d=128, near-1 gates.
    "train": Workload("train", 4, 8192, 16, 16, 128, 128, gate_mu=4.0, gate_sd=2.0, index=3),
}
for _d in (16, 32, 64, 128):
    WORKLOADS[f"long_d{_d}"] = Workload(f"long_d{_d}", 1, 32768, 32, 8, _d, _d, gate_mu=0.0,
                                        gate_sd=1.0, index=4)


def draw_lengths(rng: np.random.Generator, total: int, lo: int = 64, hi: int = 4096) -> list:
    """Lengths in [lo, hi] summing to total (the remainder never drops below lo)."""
    out, rem = [], total
    while rem > 0:
        if rem > hi:
            L = int(rng.integers(lo, min(hi, rem - lo) + 1))
        else:
            L = int(rng.integers(lo, rem + 1)) if rem > lo else rem
            if rem - L < lo:
                L = rem
        out.append(L)
        rem -= L
    return out


def make_inputs(wl: Workload | str, seed: int | None = None, **overrides) -> dict:
    """Draw every tensor of a workload.

    Returns a dict of C-contiguous numpy arrays: q [B,T,Hq,dk], k [B,T,Hkv,dk],
    v [B,T,Hkv,dv], g [B,T,Hkv,dv] (fp32), w [dv], z [B,T,Hq,dv] or None,
    dO [B,T,Hq,dv], cu_seqlens (int64 [N+1]) or None, and the workload.
    Values of bf16 tensors are bf16-representable fp32.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if overrides:
        wl = replace(wl, **overrides)
    ss = np.random.SeedSequence(MASTER_SEED + wl.index if seed is None else seed)
    rq, rk, rv, rg, rw, rz, rd, rl = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(8)]
    B, T, Hq, Hkv, dk, dv = wl.B, wl.T, wl.Hq, wl.Hkv, wl.dk, wl.dv
    cast = (lambda a: round_bf16(a)) if wl.in_dtype == "bf16" else (lambda a: np.asarray(a, np.float32))

    def normal(r, shape, mu=0.0, sd=1.0):
        return (r.standard_normal(shape, dtype=np.float64) * sd + mu).astype(np.float32)

    logits = rg.standard_normal((B, T, Hkv, dv)) * wl.gate_sd + wl.gate_mu
    out = {
        "q": cast(normal(rq, (B, T, Hq, dk))),
        "k": cast(normal(rk, (B, T, Hkv, dk))),
        "v": cast(normal(rv, (B, T, Hkv, dv))),
        "g": logsigmoid64(logits).astype(np.float32),
        # the same gate as raw logits (fp32), for callers that pass logits
        "g_logits": logits.astype(np.float32),
    }
    out["w"] = cast(normal(rw, (dv,), 1.0, 0.1)) if wl.w_kind == "normal" else np.ones(dv, np.float32)
    out["z"] = cast(normal(rz, (B, T, Hq, dv))) if wl.o_gate else None
    out["dO"] = cast(normal(rd, (B, T, Hq, dv))) if wl.backward else None
    cu = None
    if wl.lengths:
        cu = np.concatenate([[0], np.cumsum(wl.lengths)]).astype(np.int64)
    elif wl.varlen:
        cu = np.concatenate([[0], np.cumsum(draw_lengths(rl, T))]).astype(np.int64)
    if cu is not None:
        assert B == 1 and cu[-1] == T
    out["cu_seqlens"] = cu
    out["workload"] = wl
    return out


def seq_bounds(wl: Workload, cu: np.ndarray | None) -> list:
    """(start, length) of every sequence in packed token order."""
    if cu is None:
        return [(b * wl.T, wl.T) for b in range(wl.B)]
    return [(int(cu[i]), int(cu[i + 1] - cu[i])) for i in range(len(cu) - 1)]
