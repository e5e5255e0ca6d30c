"""fp64 CPU oracle for FiX parallel attention -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never loads it, and it
shares no code with the HIP library.

The arithmetic lives in ``fix_oracle.c`` (plain loops, fp64, decay as a
running product of per-token gate factors); this module only marshals numpy
arrays into it.  See the header of ``fix_oracle.c`` for the definition it
follows and the page passages it rests on (FiX repository README, section
"Quick Start"; FiX ICML 2026 poster page, abstract).

Every function here is pinned by tests under ``tests/`` that do not reuse its
code: closed forms (no gate reduces to causal softmax attention followed by
RMSNorm; a scalar gate reduces to forgetting attention; an infinitely strong
gate reduces to RMSNorm(v)), finite differences of the forward, packing and
GQA equivalences, and an independent dense fp64 autograd reference.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fix_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(out: str = _LIB, extra_flags: tuple = ()) -> str:
    """Compile ``fix_oracle.c`` with the host C compiler into ``out``."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", *extra_flags, _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    i64, f64, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    p = ctypes.c_void_p
    lib.fix_oracle_fwd.restype = i32
    lib.fix_oracle_fwd.argtypes = [i64, p, i64, i64, i64, i64, f64, f64, i32, i32,
                                   p, p, p, p, p, p, p, p, i64, p, p, p, p]
    lib.fix_oracle_bwd.restype = i32
    lib.fix_oracle_bwd.argtypes = [i64, p, i64, i64, i64, i64, f64, f64, i32, i32,
                                   p, p, p, p, p, p, p, p, p, i64, p, p, p, p, p, p]
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _gate_per_channel(g, dv):
    """A scalar gate [B,T,Hkv] as the per-channel gate it stands for ([B,T,Hkv,dv], every
    channel the same value); a per-channel gate unchanged.  Marshalling only."""
    g = np.asarray(g)
    if g.ndim == 3:
        return np.ascontiguousarray(np.broadcast_to(g[..., None], g.shape + (dv,))), True
    return g, False


def _layout(q, k, v, g, cu_seqlens):
    B, T, Hq, dk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return B, T, Hq, Hkv, dk, dv, cu


def oracle_fwd(q, k, v, g, cu_seqlens=None, *, scale=None, eps=1e-5, o_norm=True, w=None, z=None,
               m_in=None, unit_mask=None, window=0, gate_logits=False, lib=None):
    """Forward of FiX attention in fp64.

    q [B,T,Hq,dk], k [B,T,Hkv,dk], v, g [B,T,Hkv,dv], w [dv] or None, z [B,T,Hq,dv] or None.
    gate_logits: g holds raw logits x and the gate is logsigmoid(x).
    Returns dict o, x [B,T,Hq,dv], m, rstd [B,T,Hq] (float64; NaN where not computed).
    """
    lib = lib or load()
    g, _ = _gate_per_channel(g, np.asarray(v).shape[3])
    q, k, v, g, w, z = map(_f64, (q, k, v, g, w, z))
    B, T, Hq, Hkv, dk, dv, cu = _layout(q, k, v, g, cu_seqlens)
    scale = dk ** -0.5 if scale is None else float(scale)
    nseq = len(cu) - 1
    o = np.full((B, T, Hq, dv), np.nan)
    x = np.full((B, T, Hq, dv), np.nan)
    m = np.full((B, T, Hq), np.nan)
    r = np.full((B, T, Hq), np.nan)
    mi = None if m_in is None else np.ascontiguousarray(np.asarray(m_in, dtype=np.float64))
    um = None if unit_mask is None else np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8))
    st = lib.fix_oracle_fwd(nseq, _ptr(cu), Hq, Hkv, dk, dv, scale, float(eps), int(bool(o_norm)), int(bool(gate_logits)),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(w), _ptr(z), _ptr(mi), _ptr(um),
                            int(window), _ptr(o), _ptr(x), _ptr(m), _ptr(r))
    if st != 0:
        raise RuntimeError(f"fix_oracle_fwd failed with status {st}")
    return {"o": o, "x": x, "m": m, "rstd": r}


def oracle_bwd(q, k, v, g, dO, cu_seqlens=None, *, scale=None, eps=1e-5, o_norm=True, w=None, z=None,
               m_in=None, unit_mask=None, window=0, gate_logits=False, lib=None):
    """Backward of FiX attention in fp64 (row max m held constant).

    gate_logits: g holds raw logits x (the gate is logsigmoid(x)) and dg is the gradient with
    respect to x.

    window > 0: the last `window` rows and keys of every selected unit; window < 0: dq of the
    first -window rows and dk, dv of the first -window keys (dg not computed).
    Returns dict dq, dk, dv, dg, dw ([dv]; zeros without o_norm), dz (NaN where not computed).
    A scalar gate g [B,T,Hkv] stands for the same value in every channel; its dg is the
    gradient of the loss through every copy, the sum over the channels of the per-channel dg.
    """
    lib = lib or load()
    g, scalar = _gate_per_channel(g, np.asarray(v).shape[3])
    q, k, v, g, w, z, dO = map(_f64, (q, k, v, g, w, z, dO))
    B, T, Hq, Hkv, dk, dv, cu = _layout(q, k, v, g, cu_seqlens)
    scale = dk ** -0.5 if scale is None else float(scale)
    nseq = len(cu) - 1
    dq = np.full(q.shape, np.nan)
    dkk = np.full(k.shape, np.nan)
    dvv = np.full(v.shape, np.nan)
    dg = np.full(g.shape, np.nan)
    dw = np.zeros(dv)
    dz = np.full((B, T, Hq, dv), np.nan)
    mi = None if m_in is None else np.ascontiguousarray(np.asarray(m_in, dtype=np.float64))
    um = None if unit_mask is None else np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8))
    st = lib.fix_oracle_bwd(nseq, _ptr(cu), Hq, Hkv, dk, dv, scale, float(eps), int(bool(o_norm)), int(bool(gate_logits)),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(w), _ptr(z), _ptr(dO), _ptr(mi),
                            _ptr(um), int(window), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(dw),
                            _ptr(dz))
    if st != 0:
        raise RuntimeError(f"fix_oracle_bwd failed with status {st}")
    if scalar:
        dg = dg.sum(axis=-1)
    return {"dq": dq, "dk": dkk, "dv": dvv, "dg": dg, "dw": dw, "dz": dz}
