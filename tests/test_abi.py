"""The C ABI on the host: exported symbols, descriptor validation, workspace sizing,
status strings (no GPU needed: validation makes no HIP call)."""
import ctypes
import re
import os

import pytest

import gated_softmax_attention_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fixattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fix_(?:attn|decode)_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = F.library()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fixattn.h but not exported"


def desc(**kw):
    d = F.fix_attn_desc()
    base = dict(B=2, T=100, Hq=4, Hkv=2, dk=64, dv=64, in_dtype=F.FIX_BF16, out_dtype=F.FIX_BF16, scale=0.0,
                eps=1e-5, o_norm=1)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def test_valid_descriptor():
    assert F.fix_attn_validate(desc()) == F.FIX_OK
    for dk in (16, 32, 64, 128):
        for dv in (16, 32, 64, 128):
            assert F.fix_attn_validate(desc(dk=dk, dv=dv)) == F.FIX_OK


@pytest.mark.parametrize("kw,status", [
    ({"B": 0}, F.FIX_E_INVALID), ({"T": 0}, F.FIX_E_INVALID), ({"Hq": 0}, F.FIX_E_INVALID),
    ({"Hkv": 0}, F.FIX_E_INVALID), ({"Hq": 6, "Hkv": 4}, F.FIX_E_INVALID),
    ({"in_dtype": 7}, F.FIX_E_INVALID), ({"out_dtype": -1}, F.FIX_E_INVALID),
    ({"eps": -1.0}, F.FIX_E_INVALID), ({"eps": float("nan")}, F.FIX_E_INVALID),
    ({"scale": float("inf")}, F.FIX_E_INVALID),
    ({"dk": 48}, F.FIX_E_UNSUPPORTED), ({"dv": 256}, F.FIX_E_UNSUPPORTED), ({"dk": 8}, F.FIX_E_UNSUPPORTED),
    ({"B": 1, "T": 2 ** 31}, F.FIX_E_UNSUPPORTED),
])
def test_invalid_descriptors(kw, status):
    assert F.fix_attn_validate(desc(**kw)) == status


def test_packed_descriptor_rules():
    d = desc(B=1)
    d.cu_seqlens = 0x1000  # never dereferenced on the host
    d.num_seqs = 3
    assert F.fix_attn_validate(d) == F.FIX_OK
    d.num_seqs = 0
    assert F.fix_attn_validate(d) == F.FIX_E_INVALID
    d = desc(B=2)
    d.cu_seqlens = 0x1000
    d.num_seqs = 3
    assert F.fix_attn_validate(d) == F.FIX_E_INVALID


def test_workspace_sizes():
    assert F.fix_attn_fwd_workspace_size(desc(dk=48)) == 0
    assert F.fix_attn_bwd_workspace_size(desc(B=0)) == 0
    small, large = desc(T=100), desc(T=1000)
    assert 0 < F.fix_attn_fwd_workspace_size(small) < F.fix_attn_fwd_workspace_size(large)
    assert 0 < F.fix_attn_bwd_workspace_size(small) < F.fix_attn_bwd_workspace_size(large)
    assert F.fix_attn_fwd_workspace_size(small) % 256 == 0


def test_entry_points_reject_before_launching():
    lib = F.library()
    d = desc()
    # missing required pointers: rejected on the host, nothing enqueued
    assert lib.fix_attn_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, None,
                            0, None) == F.FIX_E_INVALID
    assert lib.fix_attn_bwd(ctypes.byref(d), *([None] * 17), 0, None) == F.FIX_E_INVALID
    bad = desc(dk=48)
    assert lib.fix_attn_fwd(ctypes.byref(bad), *([None] * 10), None, 0, None) == F.FIX_E_UNSUPPORTED
    # a too-small workspace is reported as such (pointers are never dereferenced on the host)
    fake = 0x10000
    st = lib.fix_attn_fwd(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, fake, fake, None, fake, 16, None)
    assert st == F.FIX_E_WORKSPACE
    # misaligned q
    st = lib.fix_attn_fwd(ctypes.byref(d), fake + 2, fake, fake, fake, None, None, fake, fake, fake, None, fake,
                          1 << 40, None)
    assert st == F.FIX_E_INVALID


def test_check_inputs_rejects_before_launching():
    lib = F.library()
    fake = 0x10000
    assert F.fix_attn_check_inputs(desc(dk=48), fake, fake, fake, 64, None) == F.FIX_E_UNSUPPORTED
    assert F.fix_attn_check_inputs(desc(), None, fake, fake, 64, None) == F.FIX_E_INVALID
    assert F.fix_attn_check_inputs(desc(), fake, fake, None, 64, None) == F.FIX_E_INVALID
    assert F.fix_attn_check_inputs(desc(), fake, fake, fake, 4, None) == F.FIX_E_WORKSPACE
    assert b"65504" in lib.fix_attn_status_string(F.FIX_E_RANGE)


def test_status_strings():
    lib = F.library()
    for s in range(6):
        assert lib.fix_attn_status_string(s)
    assert b"head dim" in lib.fix_attn_status_string(F.FIX_E_UNSUPPORTED)
    assert lib.fix_attn_last_hip_error() == 0


def test_event_trace_setting_is_host_only():
    lib = F.library()
    lib.fix_attn_set_event_trace(None, 0)
    assert lib.fix_attn_event_trace_count() == 0
    assert lib.fix_attn_event_trace_label(1) is None


def test_descriptor_layout_matches_header(tmp_path):
    """sizeof and field offsets of fix_attn_desc in the C header equal the ctypes binding's."""
    import ctypes
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = [f[0] for f in F.fix_attn_desc._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fixattn.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(fix_attn_desc));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(fix_attn_desc, {n}));\n' for n in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(root, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(F.fix_attn_desc)] + [getattr(F.fix_attn_desc, n).offset for n in fields]
    assert got == want


def ddesc(**kw):
    d = F.fix_decode_desc()
    d.B, d.cap, d.Hq, d.Hkv, d.dk, d.dv = 2, 256, 4, 2, 64, 64
    d.in_dtype, d.out_dtype, d.eps = F.FIX_BF16, F.FIX_F32, 1e-5
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    ({}, F.FIX_OK),
    ({"cap": 100}, F.FIX_E_INVALID),           # not a multiple of 64
    ({"cap": 0}, F.FIX_E_INVALID),
    ({"Hq": 3}, F.FIX_E_INVALID),              # Hq % Hkv
    ({"eps": -1.0}, F.FIX_E_INVALID),
    ({"in_dtype": 7}, F.FIX_E_INVALID),
    ({"dk": 48}, F.FIX_E_UNSUPPORTED),
    ({"Hq": 66, "Hkv": 2}, F.FIX_E_UNSUPPORTED),  # group of 33 query heads
    ({"Hq": 64, "Hkv": 2}, F.FIX_OK),              # group of 32
    ({"cap": 1 << 30}, F.FIX_E_UNSUPPORTED),
])
def test_decode_validate(kw, status):
    lib = F.library()
    assert lib.fix_decode_validate(ctypes.byref(ddesc(**kw))) == status


def test_decode_sizes_and_host_rejections():
    lib = F.library()
    d = ddesc()
    cs, ws = lib.fix_decode_cache_size(ctypes.byref(d)), lib.fix_decode_workspace_size(ctypes.byref(d))
    # the cache holds at least the fp16 keys and chunk-end values of every token
    assert cs >= 2 * 256 * 2 * (64 + 64) * 2 and ws > 0
    assert lib.fix_decode_cache_size(ctypes.byref(ddesc(cap=512))) > cs
    assert lib.fix_decode_cache_size(ctypes.byref(ddesc(cap=100))) == 0
    fake = 0x10000
    # null or misaligned cache, bad counts, missing workspace: rejected before any launch
    assert lib.fix_decode_reset(ctypes.byref(d), None, None) == F.FIX_E_INVALID
    assert lib.fix_decode_reset(ctypes.byref(d), fake + 16, None) == F.FIX_E_INVALID
    assert lib.fix_decode_append(ctypes.byref(d), fake, fake, fake, fake, 0, None, None) == F.FIX_E_INVALID
    assert lib.fix_decode_append(ctypes.byref(d), fake, fake, fake, fake, 257, None, None) == F.FIX_E_INVALID
    assert lib.fix_decode_step(ctypes.byref(d), fake, fake, None, None, fake, None, fake, 16, None) == F.FIX_E_WORKSPACE
    assert lib.fix_decode_step(ctypes.byref(d), fake, None, None, None, fake, None, fake, ws, None) == F.FIX_E_INVALID


def test_decode_descriptor_layout_matches_header(tmp_path):
    """sizeof and field offsets of fix_decode_desc in the C header equal the ctypes binding's."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = [f[0] for f in F.fix_decode_desc._fields_]
    src = tmp_path / "dlayout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fixattn.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(fix_decode_desc));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(fix_decode_desc, {n}));\n' for n in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "dlayout"
    subprocess.run(["gcc", "-I", os.path.join(root, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(F.fix_decode_desc)] + [getattr(F.fix_decode_desc, n).offset for n in fields]
    assert got == want


def test_decode_step_noalloc_rejects_oversize():
    """The allocation-free decode step refuses, before anything runs, a shape whose scratch
    exceeds the library's per-GPU array (FIX_DECODE_SCRATCH_BYTES = 32 MiB)."""
    lib = F.library()
    d = F.fix_decode_desc()
    d.B, d.cap, d.Hq, d.Hkv, d.dk, d.dv = 256, 4096, 64, 64, 128, 128
    d.in_dtype, d.out_dtype, d.eps = F.FIX_BF16, F.FIX_F32, 1e-5
    assert lib.fix_decode_validate(ctypes.byref(d)) == F.FIX_OK
    assert lib.fix_decode_workspace_size(ctypes.byref(d)) > (32 << 20)
    st = lib.fix_decode_step_noalloc(ctypes.byref(d), None, None, None, None, None, None, None)
    assert st == F.FIX_E_WORKSPACE
