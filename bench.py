"""Benchmark of the FiX attention hot path (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = fix_attn_fwd + fix_attn_bwd over one workload (default: the
training shape, B=4, T=8192, Hq=Hkv=16, dk=dv=128, bf16 inputs and outputs,
gates logsigmoid(N(4, 2))), with inputs, outputs and workspaces resident in
HBM before the timed region; the backward returns d(o_norm_weight) (and
d(o_gate) where the workload has an output gate).  Before anything is timed
the same inputs pass a parity check against the fp64 oracle on a sampled set
of rows.  Prints one JSON line.  Throughput counts algorithmic flops
(FlashAttention convention, causal pairs only): forward 2*(dk+dv) per pair and
head, backward 2*(3*dk+2*dv).  --workload picks any of the synthetic
workloads (tiny, quick, varlen, train, long_d16 .. long_d128); tiny is
forward only.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA peak (AMD specification)

# HBM bytes per launch (the last dispatch of the run: a timed step) from rocprofv3 FETCH_SIZE /
# WRITE_SIZE runs of the training workload, scaled by a plain-copy calibration (x2.0 reads,
# x1.0 writes); valid only for the sources they were
# taken on (sha256 prefix over the files listed, the build flags included).  Reported as roofline.traffic, else null.
TRAFFIC = {
    "bwd_dkv": {"bytes": int(2 * 1221795.38 * 1024 + 551170.44 * 1024), "sha": "b116608af67edde9",
                "files": ["gated_softmax_attention_amd/csrc/bwd_kernel.h",
                          "gated_softmax_attention_amd/csrc/common.h",
                          "gated_softmax_attention_amd/csrc/launch.h",
                          "gated_softmax_attention_amd/build.py"]},
    "fox_bwd_dkv": {"bytes": int(2 * 379854.00 * 1024 + 278535.75 * 1024), "sha": "80f8e6aa85e01e1a",
                    "files": ["gated_softmax_attention_amd/csrc/fox_bwd.h",
                              "gated_softmax_attention_amd/csrc/fox_bwd_d128.hip",
                              "gated_softmax_attention_amd/csrc/common.h",
                              "gated_softmax_attention_amd/csrc/launch.h",
                              "gated_softmax_attention_amd/build.py"]},
    "decode_step": {"bytes": int(2 * 135838.875 * 1024) + 1040 * 1024, "sha": "2a43a0c324eddeff",
                    "files": ["gated_softmax_attention_amd/csrc/decode.hip",
                              "gated_softmax_attention_amd/csrc/common.h",
                              "gated_softmax_attention_amd/csrc/launch.h",
                              "gated_softmax_attention_amd/build.py"]},
}


def measured_traffic(kernel):
    import hashlib
    t = TRAFFIC.get(kernel)
    if t is None:
        return None
    h = hashlib.sha256()
    for f in t["files"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return t["bytes"] if h.hexdigest()[:16] == t["sha"] else None
METRIC = "FiX attn fwd+bwd TFLOP/s (and % MFMA peak) at T=8192 d=128 bf16, 1 GPU"
WORKLOAD = "train"


def pair_counts(lengths, cb=128):
    """Causal pairs in total and split by 128-chunk distance (0, 1, >=1, >=2)."""
    tot = same = adj = 0
    for L in lengths:
        tot += L * (L + 1) // 2
        nch = (L + cb - 1) // cb
        for I in range(nch):
            rows = min(cb, L - I * cb)
            same += rows * (rows + 1) // 2
            if I >= 1:
                adj += rows * cb
    return {"all": tot, "same": same, "adj": adj, "inter": tot - same, "far": tot - same - adj}


def hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return lib


def sample_units(wl, nseq):
    """(sequence, kv head) units checked by the parity gate: the first and the last."""
    mask = np.zeros((nseq, wl.Hkv), np.uint8)
    mask[0, 0] = mask[nseq - 1, wl.Hkv - 1] = 1
    return mask


def parity_gate(x, d, F, torch, logits=False):
    """Sampled parity against the oracle: the last 64 rows (and keys) of two (sequence, kv head)
    units, or every row of a workload the oracle runs in seconds (the forward-only one)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle as O
    from gpu_util import err_rms
    wl = x["workload"]
    cu = x["cu_seqlens"]
    nseq = wl.B if cu is None else len(cu) - 1
    full = not wl.backward
    mask = None if full else sample_units(wl, nseq)
    win = 0 if full else 64
    g = x["g_logits"] if logits else x["g"]
    o, m, rstd, xx = F.forward(d["q"], d["k"], d["v"], d["g"], d["cu"], o_norm=True, o_norm_weight=d["w"],
                               o_gate=d["z"], out_dtype=torch.float32, gate_logits=logits)
    torch.cuda.synchronize()
    rf = O.oracle_fwd(x["q"], x["k"], x["v"], g, cu, w=x["w"], z=x["z"], unit_mask=mask, window=win,
                      gate_logits=logits)
    errs = {"o": err_rms(o.cpu().numpy(), rf["o"])}
    if wl.backward:
        dq, dk, dv, dg, _, _ = F.backward(d["q"], d["k"], d["v"], d["g"], m, rstd, xx, d["dO"], d["cu"],
                                          o_norm=True, o_norm_weight=d["w"], o_gate=d["z"],
                                          out_dtype=torch.float32, gate_logits=logits)
        torch.cuda.synchronize()
        rb = O.oracle_bwd(x["q"], x["k"], x["v"], g, x["dO"], cu, w=x["w"], z=x["z"], unit_mask=mask,
                          window=win, gate_logits=logits)
        for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
            errs[n] = err_rms(t.cpu().numpy(), rb[n])
    ok = all(v <= (5e-3 if n == "dg" else 1e-2) for n, v in errs.items())
    return ok, errs


def cpu_baseline(x, logits=False):
    """The fp64 oracle, forward (+ backward), on a bounded slice of the same workload: whole
    sequences of the first batch row (or packed sequence), a few heads of one kv group."""
    import oracle as O
    wl = x["workload"]
    cu = x["cu_seqlens"]
    G = wl.Hq // wl.Hkv
    if wl.name == "train":
        nh, nk = 4, 4          # four heads of batch row 0 (about 15 s on 16 threads)
    else:
        nh, nk = min(G, 4), 1  # the first kv head and up to four of its q heads
        if wl.T >= 32768:
            nh = 1             # one head of the 32k-token sequence
    if cu is not None:
        L0 = int(cu[1])
        sl = lambda a, h: np.ascontiguousarray(a[:, :L0, :h])
        lengths = [L0]
    else:
        sl = lambda a, h: np.ascontiguousarray(a[:1, :, :h])
        lengths = [wl.T]
    q = sl(x["q"], nh)
    k, v, g = (sl(x[n], nk) for n in ("k", "v", "g_logits" if logits else "g"))
    z = None if x["z"] is None else sl(x["z"], nh)
    O.load()
    t0 = time.perf_counter()
    O.oracle_fwd(q, k, v, g, w=x["w"], z=z, gate_logits=logits)
    t1 = time.perf_counter()
    if wl.backward:
        O.oracle_bwd(q, k, v, g, sl(x["dO"], nh), w=x["w"], z=z, gate_logits=logits)
    t2 = time.perf_counter()
    pairs = sum(L * (L + 1) // 2 for L in lengths) * nh
    flops = 2 * (wl.dk + wl.dv) * pairs + (2 * (3 * wl.dk + 2 * wl.dv) * pairs if wl.backward else 0)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{nh} q head(s) of the first sequence (L={lengths[0]}, dk={wl.dk}, dv={wl.dv}): "
                      f"fwd {t1 - t0:.1f} s" + (f" + bwd {t2 - t1:.1f} s (the backward recomputes the forward)"
                                                 if wl.backward else "")}


COPY_BYTES = 1 << 30


def copy_probe(torch):
    """A plain copy of known size: each dispatch reads and writes COPY_BYTES of HBM, which
    calibrates the FETCH_SIZE / WRITE_SIZE counters against true bytes."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_BYTES, "dispatches": 3}), flush=True)


PEAK_HBM_GBS = 8000.0  # MI355X HBM3E bandwidth (AMD specification)


def decode_bench(args, x, F, torch):
    """Decode steps against a cache holding all T tokens of every sequence of the workload.

    Algorithmic bytes per step: the cached keys and values in their stored fp16 form
    (T * (dk + dv) * 2 per sequence and kv head) plus q and o; the cache's fp64 chunk
    decay prefixes (dv * 8 per 64 tokens) are extra traffic, not counted."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle as O
    from gpu_util import err_rms
    wl = x["workload"]
    B, T, Hq, Hkv, dk, dv = wl.B, wl.T, wl.Hq, wl.Hkv, wl.dk, wl.dv
    bf = torch.bfloat16
    dev = lambda a, dt=bf: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    cache = F.DecodeCache(B, T, Hq, Hkv, dk, dv, dtype=bf, out_dtype=bf, o_norm=True)
    cache.append(dev(x["k"]), dev(x["v"]), dev(x["g"], torch.float32))
    q = dev(x["q"][:, T - 1])
    w = dev(x["w"])
    torch.cuda.synchronize()
    print(f"[bench] decode cache filled: B={B} T={T} Hq={Hq} Hkv={Hkv} dk={dk} dv={dv}", file=sys.stderr, flush=True)
    # parity gate: every sequence and head, against the oracle's last row
    cf = F.DecodeCache(B, T, Hq, Hkv, dk, dv, dtype=bf, out_dtype=torch.float32, o_norm=True)
    cf.append(dev(x["k"]), dev(x["v"]), dev(x["g"], torch.float32))
    o32, m32 = cf.step(q, w)
    torch.cuda.synchronize()
    ref = O.oracle_fwd(x["q"], x["k"], x["v"], x["g"], window=1, w=x["w"])
    err = err_rms(o32.cpu().numpy(), ref["o"][:, T - 1])
    print(f"[bench] decode parity gate: {'pass' if err <= 1e-2 else 'FAIL'} o err {err:.2e}", file=sys.stderr,
          flush=True)
    if err > 1e-2:
        sys.exit(1)
    del cf
    for _ in range(args.warmup):
        cache.step(q, w)
    torch.cuda.synchronize()
    h = hip()
    lib = F.library()
    lib.fix_attn_set_event_trace.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.fix_attn_event_trace_count.restype = ctypes.c_int
    lib.fix_attn_event_trace_label.restype = ctypes.c_char_p
    lib.fix_attn_event_trace_label.argtypes = [ctypes.c_int]
    cap = 4
    evs = []
    for _ in range(args.steps):
        arr = (ctypes.c_void_p * cap)()
        for i in range(cap):
            e = ctypes.c_void_p()
            assert h.hipEventCreate(ctypes.byref(e)) == 0
            arr[i] = e
        evs.append(arr)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        lib.fix_attn_set_event_trace(ctypes.cast(evs[k], ctypes.c_void_p), cap)
        cache.step(q, w)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n = lib.fix_attn_event_trace_count()
    labels = [lib.fix_attn_event_trace_label(i).decode() for i in range(1, n)]
    lib.fix_attn_set_event_trace(None, 0)
    per = {}
    for k in range(args.steps):
        for i in range(1, n):
            t = ctypes.c_float()
            assert h.hipEventElapsedTime(ctypes.byref(t), evs[k][i - 1], evs[k][i]) == 0
            per.setdefault(labels[i - 1], []).append(t.value)
    avg = {k: sum(v) / len(v) for k, v in per.items()}
    ms = (t1 - t0) * 1e3 / args.steps
    kv_bytes = B * Hkv * T * (dk + dv) * 2
    io_bytes = B * Hq * (dk + dv) * 2
    alg = kv_bytes + io_bytes
    ach = alg / (avg["decode_step"] * 1e-3) / 1e9
    out = {
        "metric": "FiX decode step HBM GB/s (cache of T=8192 tokens per sequence, d=128, bf16)",
        "value": round(alg / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"decode: B={B} cache T={T} Hq={Hq} Hkv={Hkv} dk={dk} dv={dv}, one query per "
                               f"sequence, o_norm, bf16 in/out, cache operands fp16",
                   "alg_bytes": alg, "kernel_ms": {k: round(v, 4) for k, v in avg.items()}},
        "roofline": {"bound": "hbm", "kernel": "decode_step", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode_step"),
                     "avg_launch_ms": round(avg["decode_step"], 4)},
    }
    if not args.no_cpu_baseline:
        O.load()
        c0 = time.perf_counter()
        O.oracle_fwd(x["q"], x["k"], x["v"], x["g"], window=1, w=x["w"])
        c1 = time.perf_counter()
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        out["cpu_baseline"] = {"value": round(alg / (c1 - c0) / 1e9, 3), "unit": "GB/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"the whole step: the last row of every sequence and head, {c1 - c0:.2f} s"}
    print(json.dumps(out), flush=True)


# Exponential peak: 1024 SIMDs at 2.4 GHz, one v_exp_f32 per wave64 every 8 cycles (the
# transcendental unit handles 8 lanes a cycle), in Gexp/s.
PEAK_EXP_GEXPS = 1024 * 64 / 8 * 2.4


def peak_probe(torch):
    """Measured peaks: independent 32x32x16 bf16 products on every SIMD, independent v_exp_f32
    chains, a 16-byte-per-lane copy of 1 GiB, and the fp32 atomic dq traffic a key-stationary
    fused backward would make at the training shape (libfixprobe.so, separate from the library)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_softmax_attention_amd", "libfixprobe.so"))
    lib.fix_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fix_probe_exp.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fix_probe_copy.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    blocks = 256 * 4
    out = torch.empty(blocks * 256, device="cuda")

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = None
        for _ in range(reps):
            e0.record()
            assert fn() == 0
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        return best

    it_m, it_e = 2000, 100000
    t_m = timed(lambda: lib.fix_probe_mfma(blocks, it_m, out.data_ptr(), st))
    t_e = timed(lambda: lib.fix_probe_exp(blocks, it_e, out.data_ptr(), st))
    src = torch.ones(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    t_c = timed(lambda: lib.fix_probe_copy(256 * 8, src.data_ptr(), dst.data_ptr(), COPY_BYTES, st))
    # dq accumulation of a key-stationary fused backward at the training shape (B=4, T=8192,
    # H=16, dk=128): every (key chunk, 64-row slice) pair adds a 64 x 128 fp32 tile atomically
    lib.fix_probe_atomic_dq.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    Bq, Tq, Hq = 4, 8192, 16
    dqa = torch.zeros(Bq * Tq * Hq * 128, device="cuda")
    t_a = timed(lambda: lib.fix_probe_atomic_dq(dqa.data_ptr(), Bq, Tq, Hq, 0, st), reps=3)
    t_as = timed(lambda: lib.fix_probe_atomic_dq(dqa.data_ptr(), Bq, Tq, Hq, 1, st), reps=3)
    # LDS read bandwidth: 16-byte reads and 8-byte transposing reads, 8 waves per workgroup
    lib.fix_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lblocks, it_l = 256 * 4, 4000
    lout = torch.empty(lblocks * 512, dtype=torch.int32, device="cuda")
    t_l = [timed(lambda m=m: lib.fix_probe_lds(m, lblocks, it_l, lout.data_ptr(), st)) for m in (0, 1)]
    lds_bytes = [lblocks * 512 * it_l * 8 * w for w in (16, 8)]
    nsl = Tq // 64
    adds = Bq * Hq * sum(max(0, nsl - 2 * J) for J in range(Tq // 128)) * 64 * 128
    mfma = blocks * 4 * it_m * 4 * 32768 / t_m / 1e12
    exps = blocks * 256 * it_e * 8 / t_e / 1e9
    copy = 2 * COPY_BYTES / t_c / 1e9
    print(json.dumps({"mfma_bf16_tflops": round(mfma, 1), "mfma_frac_of_spec": round(mfma / PEAK_BF16_TFLOPS, 4),
                      "exp_gexps": round(exps, 1), "exp_frac_of_model": round(exps / PEAK_EXP_GEXPS, 4),
                      "copy_gbs": round(copy, 1), "copy_frac_of_spec": round(copy / PEAK_HBM_GBS, 4),
                      "fused_dq_atomics_ms": round(t_a * 1e3, 3), "fused_dq_atomic_bytes": adds * 4,
                      "fused_dq_atomic_gbs": round(adds * 4 / t_a / 1e9, 1),
                      "fused_dq_atomics_staggered_ms": round(t_as * 1e3, 3),
                      "lds_b128_bytes_per_clk_cu": round(lds_bytes[0] / t_l[0] / 256 / 2.4e9, 1),
                      "lds_tr_b64_bytes_per_clk_cu": round(lds_bytes[1] / t_l[1] / 256 / 2.4e9, 1),
                      "mfma_s": t_m, "exp_s": t_e, "copy_s": t_c}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=WORKLOAD,
                    help="tiny, quick, varlen, train (default), long_d16, long_d32, long_d64, long_d128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate-logits", action="store_true",
                    help="pass the gate as raw logits (logsigmoid applied inside the kernels)")
    ap.add_argument("--peak-probe", action="store_true",
                    help="only measure the matrix-product, exponential and copy peaks (libfixprobe.so)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (HBM counter calibration)")
    ap.add_argument("--scalar-gate", action="store_true",
                    help="one gate value per token and kv head (channel 0 of the workload's gate): the "
                         "logit-bias forward and backward")
    ap.add_argument("--decode", action="store_true",
                    help="time decode steps (fix_decode_step) against a cache holding the workload's T tokens")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library runs the kernels on one GPU's share and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.peak_probe:
        peak_probe(torch)
        return
    import gated_softmax_attention_amd as F
    from gated_softmax_attention_amd import synth

    x = synth.make_inputs(args.workload)
    if args.scalar_gate:
        x = dict(x)
        x["g"] = np.ascontiguousarray(x["g"][..., 0])
        x["g_logits"] = np.ascontiguousarray(x["g_logits"][..., 0])
    if args.decode:
        decode_bench(args, x, F, torch)
        return
    wl = x["workload"]
    dt = torch.bfloat16 if wl.in_dtype == "bf16" else torch.float32
    dev = lambda a, t=dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()
    d = {n: dev(x[n]) for n in ("q", "k", "v", "dO", "w", "z")}
    d["g"] = dev(x["g_logits"] if args.gate_logits else x["g"], torch.float32)
    d["cu"] = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    print(f"[bench] inputs resident: {wl}{' (gate as logits)' if args.gate_logits else ''}", file=sys.stderr,
          flush=True)

    ok, errs = parity_gate(x, d, F, torch, logits=args.gate_logits)
    print(f"[bench] parity gate: {'pass' if ok else 'FAIL'} {errs}", file=sys.stderr, flush=True)
    if not ok:
        sys.exit(1)

    B, T, Hq, dk = d["q"].shape
    Hkv, dv = d["k"].shape[2], d["v"].shape[3]
    o = torch.empty(B, T, Hq, dv, dtype=dt, device="cuda")
    m = torch.empty(B, T, Hq, device="cuda")
    rstd = torch.empty(B, T, Hq, device="cuda")
    xx = torch.empty(B, T, Hq, dv, device="cuda")
    if wl.backward:
        dq, dkk, dvv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        dg = torch.empty_like(d["g"])
        dw = torch.empty(dv, device="cuda")
        dz = None if d["z"] is None else torch.empty_like(d["z"])
    desc = F.make_desc(d["q"], d["k"], d["v"], d["cu"], o_norm=True, gate_logits=args.gate_logits,
                       gate_scalar=args.scalar_gate)
    wf, wb = F.fix_attn_fwd_workspace_size(desc), F.fix_attn_bwd_workspace_size(desc)
    ws_f = torch.empty(wf, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(wb if wl.backward else 1, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lib = F.library()

    def fwd():
        F.fix_attn_fwd(desc, d["q"], d["k"], d["v"], d["g"], d["w"], d["z"], o, m, rstd,
                       xx if wl.backward else None, ws_f, wf, stream)

    def bwd():
        F.fix_attn_bwd(desc, d["q"], d["k"], d["v"], d["g"], d["w"], d["z"], m, rstd, xx, d["dO"], dq, dkk, dvv, dg,
                       dw, dz, ws_b, wb, stream)

    for _ in range(args.warmup):
        fwd()
        if wl.backward:
            bwd()
    torch.cuda.synchronize()

    # Per-kernel events recorded by the library on its stream during the timed steps.
    h = hip()
    cap = 24
    ev = [[(ctypes.c_void_p * cap)() for _ in range(2)] for _ in range(args.steps)]
    for s_ in ev:
        for arr in s_:
            for i in range(cap):
                e = ctypes.c_void_p()
                assert h.hipEventCreate(ctypes.byref(e)) == 0
                arr[i] = e
    labels = [None, None]
    counts = [0, 0]

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        lib.fix_attn_set_event_trace(ctypes.cast(ev[k][0], ctypes.c_void_p), cap)
        fwd()
        counts[0] = lib.fix_attn_event_trace_count()
        if labels[0] is None:
            labels[0] = [lib.fix_attn_event_trace_label(i).decode() for i in range(1, counts[0])]
        if wl.backward:
            lib.fix_attn_set_event_trace(ctypes.cast(ev[k][1], ctypes.c_void_p), cap)
            bwd()
            counts[1] = lib.fix_attn_event_trace_count()
            if labels[1] is None:
                labels[1] = [lib.fix_attn_event_trace_label(i).decode() for i in range(1, counts[1])]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.fix_attn_set_event_trace(None, 0)
    ms_step = (t1 - t0) * 1e3 / args.steps

    per_kernel = {}
    side_ms = [[], []]
    for k in range(args.steps):
        for side in (0, 1) if wl.backward else (0,):
            tot = 0.0
            for i in range(1, counts[side]):
                t = ctypes.c_float()
                assert h.hipEventElapsedTime(ctypes.byref(t), ev[k][side][i - 1], ev[k][side][i]) == 0
                per_kernel.setdefault(labels[side][i - 1], []).append(t.value)
                tot += t.value
            side_ms[side].append(tot)
    avg = {n: sum(v) / len(v) for n, v in per_kernel.items()}

    cu = x["cu_seqlens"]
    lengths = [T] * B if cu is None else [int(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]
    pc = pair_counts(lengths)
    heads = Hq
    fwd_flops = 2 * (dk + dv) * pc["all"] * heads
    bwd_flops = 2 * (3 * dk + 2 * dv) * pc["all"] * heads if wl.backward else 0
    total = fwd_flops + bwd_flops
    tflops = total / (ms_step * 1e-3) / 1e12
    # Algorithmic flops per head of each kernel (its share of the 2 forward and 5 backward products)
    # and the exponentials it must evaluate (one per pair for every kernel that forms P).
    alg = {
        "fix_fwd": (2 * (dk + dv) * pc["all"], pc["all"]),
        "fox_fwd": (2 * (dk + dv) * pc["all"], pc["all"]),
        "bwd_dq": (2 * (2 * dk + dv) * pc["inter"], pc["inter"]),      # S, dP, dQ on pairs in different chunks
        "bwd_dkv": (2 * (dk + dv) * pc["far"], pc["far"]),             # dV, dK on pairs two or more chunks apart
        "bwd_intra_dq": (2 * (2 * dk + dv) * pc["same"], pc["same"]),
        "bwd_intra_dkv": (2 * (dk + dv) * (pc["same"] + pc["adj"]), pc["same"] + pc["adj"]),
        "fox_bwd_dq": (2 * (2 * dk + dv) * pc["all"], pc["all"]),      # S, dP, dQ on every pair
        "fox_bwd_dkv": (2 * (dk + dv) * pc["all"], pc["all"]),         # dV, dK on every pair
    }
    dom = max(avg, key=avg.get)
    roof = None
    if dom in alg:
        fl, npair = alg[dom]
        fl, nexp = fl * heads, npair * heads
        sec = avg[dom] * 1e-3
        t_mfma = fl / (PEAK_BF16_TFLOPS * 1e12)
        t_exp = nexp / (PEAK_EXP_GEXPS * 1e9)
        if t_exp > t_mfma:   # the exponentials, not the products, bound this kernel at its head dims
            ach = nexp / sec / 1e9
            roof = {"bound": "alu", "kernel": dom, "achieved": round(ach, 1), "peak": round(PEAK_EXP_GEXPS, 1),
                    "unit": "Gexp/s", "frac": round(ach / PEAK_EXP_GEXPS, 4),
                    "mfma_frac": round(fl / sec / 1e12 / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = fl / sec / 1e12
            roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        # the stored counts were taken on the training workload (per-channel or scalar gate as run)
        roof["traffic"] = measured_traffic(dom) if wl.name == "train" and not args.gate_logits else None
        roof["avg_launch_ms"] = round(avg[dom], 4)
    fwd_ms = sum(side_ms[0]) / len(side_ms[0])
    bwd_ms = sum(side_ms[1]) / len(side_ms[1]) if wl.backward else None
    desc_w = (f"{wl.name}: B={B} T={T}" + (f" packed {len(lengths)} seqs" if cu is not None else "")
              + f" Hq={Hq} Hkv={Hkv} dk={dk} dv={dv} {wl.in_dtype} in/{wl.in_dtype} out, "
              f"g=logsigmoid(N({wl.gate_mu},{wl.gate_sd}))"
              + (" passed as logits (logsigmoid in the kernels)" if args.gate_logits else "")
              + (", scalar per token and head (channel 0)" if args.scalar_gate else "")
              + ", o_norm" + (" with d(o_norm_weight)" if wl.backward else "")
              + (", o_gate" + (" with d(o_gate)" if wl.backward else "") if d["z"] is not None else "")
              + (", fwd+bwd" if wl.backward else ", fwd only"))
    metric = METRIC if wl.name == WORKLOAD and wl.backward else (
        f"FiX attn {'fwd+bwd' if wl.backward else 'fwd'} TFLOP/s (and % MFMA peak), workload {wl.name}, 1 GPU")
    out = {
        "metric": metric, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.in_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": desc_w,
                   "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                   "fwd_flops": fwd_flops, "bwd_flops": bwd_flops,
                   "fwd_ms": round(fwd_ms, 4), "bwd_ms": None if bwd_ms is None else round(bwd_ms, 4),
                   "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
                   "kernel_ms": {n: round(v, 4) for n, v in sorted(avg.items(), key=lambda kv: -kv[1])}},
        "roofline": roof,
    }
    if cu is not None:
        out["config"]["cu_seqlens"] = [int(c) for c in cu]
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(x, logits=args.gate_logits)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
