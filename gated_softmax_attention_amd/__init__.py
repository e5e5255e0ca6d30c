"""FiX parallel attention on AMD MI355X (gfx950): Python binding of libfixattn.so.

The compute runs entirely in the HIP library behind the C ABI declared in
include/fixattn.h; this module only marshals torch tensors (device memory and
the current stream) into it.  There is no fallback: if the library is absent
every call raises.

    from gated_softmax_attention_amd import parallel_fix_attn
    o = parallel_fix_attn(q, k, v, g)                       # q [B,T,Hq,dk]; k [B,T,Hkv,dk]
    o = parallel_fix_attn(q, k, v, g, cu_seqlens=cu)        # packed, B == 1
    o = parallel_fix_attn(q, k, v, g, o_norm=True, o_norm_weight=w, o_gate=z)

(argument names and shapes follow the FiX README, section "Quick Start").
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfixattn.so")

FIX_OK, FIX_E_INVALID, FIX_E_UNSUPPORTED, FIX_E_WORKSPACE, FIX_E_HIP, FIX_E_RANGE = range(6)
FIX_BF16, FIX_F32 = 0, 1


class fix_attn_desc(ctypes.Structure):
    """Mirror of the C struct fix_attn_desc (include/fixattn.h)."""
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64),
        ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("cu_seqlens", ctypes.c_void_p), ("num_seqs", ctypes.c_int64),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("scale", ctypes.c_float), ("eps", ctypes.c_float),
        ("o_norm", ctypes.c_int32), ("gate_logits", ctypes.c_int32),
        ("gate_scalar", ctypes.c_int32),
    ]


class fix_decode_desc(ctypes.Structure):
    """Mirror of the C struct fix_decode_desc (include/fixattn.h)."""
    _fields_ = [
        ("B", ctypes.c_int64), ("cap", ctypes.c_int64),
        ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("scale", ctypes.c_float), ("eps", ctypes.c_float),
        ("o_norm", ctypes.c_int32), ("gate_logits", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gated_softmax_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, D = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(fix_attn_desc)
    lib.fix_attn_validate.argtypes = [D]
    lib.fix_attn_validate.restype = ctypes.c_int
    lib.fix_attn_fwd_workspace_size.argtypes = [D]
    lib.fix_attn_fwd_workspace_size.restype = S
    lib.fix_attn_bwd_workspace_size.argtypes = [D]
    lib.fix_attn_bwd_workspace_size.restype = S
    lib.fix_attn_fwd.argtypes = [D] + [P] * 11 + [S, P]
    lib.fix_attn_fwd.restype = ctypes.c_int
    lib.fix_attn_bwd.argtypes = [D] + [P] * 17 + [S, P]
    lib.fix_attn_bwd.restype = ctypes.c_int
    DD = ctypes.POINTER(fix_decode_desc)
    lib.fix_decode_validate.argtypes = [DD]
    lib.fix_decode_validate.restype = ctypes.c_int
    lib.fix_decode_cache_size.argtypes = [DD]
    lib.fix_decode_cache_size.restype = S
    lib.fix_decode_workspace_size.argtypes = [DD]
    lib.fix_decode_workspace_size.restype = S
    lib.fix_decode_reset.argtypes = [DD, P, P]
    lib.fix_decode_reset.restype = ctypes.c_int
    lib.fix_decode_append.argtypes = [DD, P, P, P, P, ctypes.c_int64, P, P]
    lib.fix_decode_append.restype = ctypes.c_int
    lib.fix_decode_step.argtypes = [DD, P, P, P, P, P, P, P, S, P]
    lib.fix_decode_step.restype = ctypes.c_int
    lib.fix_decode_step_noalloc.argtypes = [DD, P, P, P, P, P, P, P]
    lib.fix_decode_step_noalloc.restype = ctypes.c_int
    lib.fix_attn_check_inputs.argtypes = [D, P, P, P, S, P]
    lib.fix_attn_check_inputs.restype = ctypes.c_int
    lib.fix_attn_status_string.argtypes = [ctypes.c_int]
    lib.fix_attn_status_string.restype = ctypes.c_char_p
    lib.fix_attn_last_hip_error.argtypes = []
    lib.fix_attn_last_hip_error.restype = ctypes.c_int
    lib.fix_attn_set_event_trace.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.fix_attn_set_event_trace.restype = None
    lib.fix_attn_event_trace_count.argtypes = []
    lib.fix_attn_event_trace_count.restype = ctypes.c_int
    lib.fix_attn_event_trace_label.argtypes = [ctypes.c_int]
    lib.fix_attn_event_trace_label.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library():
    """The loaded ctypes handle of libfixattn.so (raises if it is not built)."""
    return _load()


class FixAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _load()
        msg = lib.fix_attn_status_string(status).decode()
        if status == FIX_E_HIP:
            msg += f" (hipError {lib.fix_attn_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(fn, status):
    if status != FIX_OK:
        raise FixAttnError(fn, status)


# ---- thin wrappers with the C names (pointers may be torch tensors or ints) ----

def fix_attn_validate(desc: fix_attn_desc) -> int:
    return _load().fix_attn_validate(ctypes.byref(desc))


def fix_attn_fwd_workspace_size(desc: fix_attn_desc) -> int:
    return _load().fix_attn_fwd_workspace_size(ctypes.byref(desc))


def fix_attn_bwd_workspace_size(desc: fix_attn_desc) -> int:
    return _load().fix_attn_bwd_workspace_size(ctypes.byref(desc))


def fix_attn_fwd(desc, q, k, v, g, o_norm_weight, o_gate, o, m, rstd, x, ws, ws_bytes, stream):
    st = _load().fix_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o_norm_weight),
                              _ptr(o_gate), _ptr(o), _ptr(m), _ptr(rstd), _ptr(x), _ptr(ws), ws_bytes,
                              stream)
    _check("fix_attn_fwd", st)


def fix_attn_bwd(desc, q, k, v, g, o_norm_weight, o_gate, m, rstd, x, d_o, dq, dk, dv, dg, d_o_norm_weight,
                 d_o_gate, ws, ws_bytes, stream):
    st = _load().fix_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o_norm_weight),
                              _ptr(o_gate), _ptr(m), _ptr(rstd), _ptr(x), _ptr(d_o), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(dg), _ptr(d_o_norm_weight), _ptr(d_o_gate), _ptr(ws), ws_bytes,
                              stream)
    _check("fix_attn_bwd", st)


def fix_attn_check_inputs(desc, q, k, ws, ws_bytes, stream) -> int:
    """Status of the q/k range check (FIX_OK or FIX_E_RANGE; other codes as the C call)."""
    return _load().fix_attn_check_inputs(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(ws), ws_bytes, stream)


def check_inputs(q, k, v, cu_seqlens=None) -> int:
    """fix_attn_check_inputs on torch tensors (synchronizes the current stream)."""
    import torch
    desc = make_desc(q, k, v, cu_seqlens)
    ws = torch.empty(64, dtype=torch.uint8, device=q.device)
    return fix_attn_check_inputs(desc, q, k, ws, ws.numel(), torch.cuda.current_stream().cuda_stream)


def make_desc(q, k, v, cu_seqlens=None, *, o_norm=False, scale=None, eps=1e-5, out_dtype=None,
              gate_logits=False, gate_scalar=False) -> fix_attn_desc:
    """Descriptor for torch tensors q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv]."""
    import torch
    B, T, Hq, dk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    dt = {torch.bfloat16: FIX_BF16, torch.float32: FIX_F32}
    if q.dtype not in dt:
        raise ValueError(f"q, k, v must be bfloat16 or float32, got {q.dtype}")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    d = fix_attn_desc()
    d.B, d.T, d.Hq, d.Hkv, d.dk, d.dv = B, T, Hq, Hkv, dk, dv
    if cu_seqlens is not None:
        d.cu_seqlens = cu_seqlens.data_ptr()
        d.num_seqs = cu_seqlens.numel() - 1
    d.in_dtype = dt[q.dtype]
    d.out_dtype = dt[out_dtype]
    d.scale = 0.0 if scale is None else float(scale)
    d.eps = float(eps)
    d.o_norm = 1 if o_norm else 0
    d.gate_logits = 1 if gate_logits else 0
    d.gate_scalar = 1 if gate_scalar else 0
    return d


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check_inputs(q, k, v, g, cu_seqlens, o_norm_weight, o_gate):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D CUDA tensor")
    if not g.is_cuda or not g.is_contiguous() or g.dim() not in (3, 4):
        raise ValueError("g must be a contiguous CUDA tensor, [B,T,Hkv,dv] or [B,T,Hkv] (scalar gate)")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    if g.dtype != torch.float32:
        raise ValueError("the forget gate g must be float32")
    B, T, Hq, dk = q.shape
    if (k.shape[:2] != (B, T) or v.shape[:3] != k.shape[:3] or k.shape[3] != dk
            or tuple(g.shape) not in (tuple(v.shape), tuple(v.shape[:3]))):
        raise ValueError("shape mismatch among q, k, v, g")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int64 or not cu_seqlens.is_cuda or B != 1):
        raise ValueError("cu_seqlens must be an int64 CUDA tensor and requires B == 1")
    if o_norm_weight is not None and (o_norm_weight.shape != (v.shape[3],) or o_norm_weight.dtype != q.dtype):
        raise ValueError("o_norm_weight must be [dv] with the dtype of q")
    if o_gate is not None and (o_gate.shape != (B, T, Hq, v.shape[3]) or o_gate.dtype != q.dtype
                               or not o_gate.is_contiguous()):
        raise ValueError("o_gate must be a contiguous [B,T,Hq,dv] tensor with the dtype of q")


def forward(q, k, v, g, cu_seqlens=None, *, o_norm=False, o_norm_weight=None, o_gate=None, scale=None,
            eps=1e-5, out_dtype=None, save_x=True, gate_logits=False):
    """One call of fix_attn_fwd; returns (o, m, rstd, x or None).  gate_logits: g holds logits."""
    import torch
    _check_inputs(q, k, v, g, cu_seqlens, o_norm_weight, o_gate)
    desc = make_desc(q, k, v, cu_seqlens, o_norm=o_norm, scale=scale, eps=eps, out_dtype=out_dtype,
                     gate_logits=gate_logits, gate_scalar=g.dim() == 3)
    B, T, Hq, _ = q.shape
    dv = v.shape[3]
    od = q.dtype if out_dtype is None else out_dtype
    o = torch.empty(B, T, Hq, dv, dtype=od, device=q.device)
    m = torch.empty(B, T, Hq, dtype=torch.float32, device=q.device)
    rstd = torch.empty(B, T, Hq, dtype=torch.float32, device=q.device)
    x = torch.empty(B, T, Hq, dv, dtype=torch.float32, device=q.device) if save_x else None
    wsb = fix_attn_fwd_workspace_size(desc)
    if wsb == 0:
        _check("fix_attn_fwd_workspace_size", fix_attn_validate(desc))
    ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    fix_attn_fwd(desc, q, k, v, g, o_norm_weight if o_norm else None, o_gate, o, m, rstd, x, ws, wsb, _stream())
    return o, m, rstd, x


def backward(q, k, v, g, m, rstd, x, d_o, cu_seqlens=None, *, o_norm=False, o_norm_weight=None, o_gate=None,
             scale=None, eps=1e-5, out_dtype=None, need_dw=False, need_dz=False, gate_logits=False):
    """One call of fix_attn_bwd; returns (dq, dk, dv, dg, d_o_norm_weight or None, d_o_gate or None).
    gate_logits: g holds logits and dg is the gradient with respect to them."""
    import torch
    _check_inputs(q, k, v, g, cu_seqlens, o_norm_weight, o_gate)
    desc = make_desc(q, k, v, cu_seqlens, o_norm=o_norm, scale=scale, eps=eps, out_dtype=out_dtype,
                     gate_logits=gate_logits, gate_scalar=g.dim() == 3)
    od = q.dtype if out_dtype is None else out_dtype
    d_o = d_o.contiguous().to(q.dtype)
    dq = torch.empty(q.shape, dtype=od, device=q.device)
    dk = torch.empty(k.shape, dtype=od, device=q.device)
    dv = torch.empty(v.shape, dtype=od, device=q.device)
    dg = torch.empty(g.shape, dtype=torch.float32, device=q.device)
    dw = torch.empty(v.shape[3], dtype=torch.float32, device=q.device) if (need_dw and o_norm) else None
    dz = torch.empty(o_gate.shape, dtype=od, device=q.device) if (need_dz and o_gate is not None) else None
    wsb = fix_attn_bwd_workspace_size(desc)
    if wsb == 0:
        _check("fix_attn_bwd_workspace_size", fix_attn_validate(desc))
    ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    fix_attn_bwd(desc, q, k, v, g, o_norm_weight if o_norm else None, o_gate, m, rstd, x, d_o, dq, dk, dv, dg,
                 dw, dz, ws, wsb, _stream())
    return dq, dk, dv, dg, dw, dz


def _autograd_fn():
    import torch

    class FixAttnFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, g, o_norm_weight, o_gate, cu_seqlens, o_norm, scale, eps):
            o, m, rstd, x = forward(q, k, v, g, cu_seqlens, o_norm=o_norm, o_norm_weight=o_norm_weight,
                                    o_gate=o_gate, scale=scale, eps=eps, save_x=True)
            ctx.save_for_backward(q, k, v, g, o_norm_weight, o_gate, cu_seqlens, m, rstd, x)
            ctx.cfg = (o_norm, scale, eps)
            return o

        @staticmethod
        def backward(ctx, d_o):
            q, k, v, g, w, z, cu, m, rstd, x = ctx.saved_tensors
            o_norm, scale, eps = ctx.cfg
            need_dw = w is not None and ctx.needs_input_grad[4]
            need_dz = z is not None and ctx.needs_input_grad[5]
            dq, dk, dv, dg, dw, dz = backward(q, k, v, g, m, rstd, x, d_o, cu, o_norm=o_norm, o_norm_weight=w,
                                              o_gate=z, scale=scale, eps=eps, need_dw=need_dw, need_dz=need_dz)
            if dw is not None:
                dw = dw.to(w.dtype)
            return dq, dk, dv, dg, dw, dz, None, None, None, None

    return FixAttnFunction


_FN = None


def parallel_fix_attn(q, k, v, g, cu_seqlens=None, o_norm=False, o_norm_weight=None, o_gate=None, scale=None,
                      eps=1e-5):
    """FiX parallel attention (differentiable).  Shapes as in the module docstring; g is float32."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    q, k, v, g = (t.contiguous() for t in (q, k, v, g))
    if o_gate is not None:
        o_gate = o_gate.contiguous()
    return _FN.apply(q, k, v, g, o_norm_weight, o_gate, cu_seqlens, bool(o_norm), scale, float(eps))


__all__ = [
    "parallel_fix_attn", "forward", "backward", "make_desc", "library", "fix_attn_desc",
    "fix_attn_validate", "fix_attn_fwd_workspace_size", "fix_attn_bwd_workspace_size", "fix_attn_fwd",
    "fix_attn_bwd", "FixAttnError", "FIX_OK", "FIX_E_INVALID", "FIX_E_UNSUPPORTED", "FIX_E_WORKSPACE",
    "FIX_E_HIP", "FIX_E_RANGE", "FIX_BF16", "FIX_F32", "fix_attn_check_inputs",
]


class DecodeCache:
    """A key/value/gate cache for one-token decode steps (fix_decode_* in
    include/fixattn.h): the cache buffer and the step's scratch are torch
    device tensors owned by this object.

        c = DecodeCache(B, cap, Hq, Hkv, dk, dv, dtype=torch.bfloat16)
        c.append(k, v, g)           # k [B,n,Hkv,dk], v/g [B,n,Hkv,dv]
        o, m = c.step(q)            # q [B,Hq,dk] of the newest token
    """

    def __init__(self, B, cap, Hq, Hkv, dk, dv, *, dtype=None, out_dtype=None, scale=None, eps=1e-5,
                 o_norm=False, gate_logits=False, device="cuda"):
        import torch
        dtype = torch.bfloat16 if dtype is None else dtype
        dt = {torch.bfloat16: FIX_BF16, torch.float32: FIX_F32}
        self.dtype, self.out_dtype = dtype, dtype if out_dtype is None else out_dtype
        d = fix_decode_desc()
        d.B, d.cap, d.Hq, d.Hkv, d.dk, d.dv = B, cap, Hq, Hkv, dk, dv
        d.in_dtype, d.out_dtype = dt[dtype], dt[self.out_dtype]
        d.scale = 0.0 if scale is None else float(scale)
        d.eps = float(eps)
        d.o_norm = 1 if o_norm else 0
        d.gate_logits = 1 if gate_logits else 0
        lib = _load()
        _check("fix_decode_validate", lib.fix_decode_validate(ctypes.byref(d)))
        self.desc = d
        self.cache = torch.empty(lib.fix_decode_cache_size(ctypes.byref(d)), dtype=torch.uint8, device=device)
        self.ws = torch.empty(lib.fix_decode_workspace_size(ctypes.byref(d)), dtype=torch.uint8, device=device)
        self.reset()

    def reset(self):
        _check("fix_decode_reset", _load().fix_decode_reset(ctypes.byref(self.desc), _ptr(self.cache), _stream()))

    def append(self, k, v, g, n_seq=None):
        """Append n tokens per sequence (the first n_seq[b] of row b, n_seq an int32 device tensor)."""
        d = self.desc
        n = k.shape[1]
        if (tuple(k.shape) != (d.B, n, d.Hkv, d.dk) or tuple(v.shape) != (d.B, n, d.Hkv, d.dv)
                or tuple(g.shape) != (d.B, n, d.Hkv, d.dv)):
            raise ValueError("k, v, g shapes do not match the cache")
        import torch
        if k.dtype != self.dtype or v.dtype != self.dtype or g.dtype != torch.float32:
            raise ValueError("k, v must have the cache dtype and g float32")
        for t in (k, v, g):
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
        st = _load().fix_decode_append(ctypes.byref(d), _ptr(self.cache), _ptr(k), _ptr(v), _ptr(g), n,
                                       _ptr(n_seq), _stream())
        _check("fix_decode_append", st)

    def step(self, q, o_norm_weight=None, o_gate=None):
        """Output (o [B,Hq,dv], m [B,Hq]) of the newest cached token of every sequence."""
        import torch
        d = self.desc
        if tuple(q.shape) != (d.B, d.Hq, d.dk) or q.dtype != self.dtype or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B, Hq, dk] tensor of the cache dtype")
        o = torch.empty(d.B, d.Hq, d.dv, dtype=self.out_dtype, device=q.device)
        m = torch.empty(d.B, d.Hq, dtype=torch.float32, device=q.device)
        st = _load().fix_decode_step(ctypes.byref(d), _ptr(self.cache), _ptr(q),
                                     _ptr(o_norm_weight) if d.o_norm else None, _ptr(o_gate), _ptr(o), _ptr(m),
                                     _ptr(self.ws), self.ws.numel(), _stream())
        _check("fix_decode_step", st)
        return o, m

    def step_noalloc(self, q, o, m, o_norm_weight=None, o_gate=None):
        """fix_decode_step_noalloc into caller-given o [B,Hq,dv] and m [B,Hq] (or None): the same
        step with the library's own scratch, so no device memory is allocated."""
        d = self.desc
        if tuple(q.shape) != (d.B, d.Hq, d.dk) or q.dtype != self.dtype or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B, Hq, dk] tensor of the cache dtype")
        if tuple(o.shape) != (d.B, d.Hq, d.dv) or o.dtype != self.out_dtype or not o.is_contiguous():
            raise ValueError("o must be a contiguous [B, Hq, dv] tensor of the output dtype")
        st = _load().fix_decode_step_noalloc(ctypes.byref(d), _ptr(self.cache), _ptr(q),
                                             _ptr(o_norm_weight) if d.o_norm else None, _ptr(o_gate), _ptr(o),
                                             _ptr(m), _stream())
        _check("fix_decode_step_noalloc", st)
