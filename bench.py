"""Benchmark of the FiX attention hot path (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = fix_attn_fwd + fix_attn_bwd over the training-shape workload
(B=4, T=8192, Hq=Hkv=16, dk=dv=128, bf16 inputs and outputs, gates
logsigmoid(N(4, 2))), with inputs, outputs and workspaces resident in HBM
before the timed region.  Before anything is timed the same inputs pass a
parity check against the fp64 oracle on a sampled set of rows.  Prints one
JSON line.  Throughput counts algorithmic flops (FlashAttention convention,
causal pairs only): forward 2*(dk+dv) per pair and head, backward
2*(3*dk+2*dv).
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

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this workload, scaled by
# a plain-copy calibration (x2.0 reads, x1.0 writes); valid only for the sources they were
# taken on (sha256 prefix over the files listed, the build flags included).  Reported as roofline.traffic, else null.
TRAFFIC = {
    "bwd_dkv": {"bytes": 2 * 1023348 * 1024 + 531964 * 1024, "sha": "73ac43155d216708",
                "files": ["gated_softmax_attention_amd/csrc/bwd_kernel.h",
                          "gated_softmax_attention_amd/csrc/common.h",
                          "gated_softmax_attention_amd/csrc/launch.h",
                          "gated_softmax_attention_amd/build.py"]},
    "decode_step": {"bytes": int(2 * 135774.125 * 1024) + 1040 * 1024, "sha": "ca18dcf888947a22",
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


def parity_gate(x, d, F, torch, logits=False):
    """Sampled parity against the oracle (last 64 rows of two (sequence, kv head) units)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle as O
    from gpu_util import err_rms
    o, m, rstd, xx = F.forward(d["q"], d["k"], d["v"], d["g"], o_norm=True, out_dtype=torch.float32,
                               gate_logits=logits)
    dq, dk, dv, dg, _, _ = F.backward(d["q"], d["k"], d["v"], d["g"], m, rstd, xx, d["dO"], o_norm=True,
                                      out_dtype=torch.float32, gate_logits=logits)
    torch.cuda.synchronize()
    wl = x["workload"]
    mask = np.zeros((wl.B, wl.Hkv), np.uint8)
    mask[0, 0] = mask[wl.B - 1, wl.Hkv - 1] = 1
    g = x["g_logits"] if logits else x["g"]
    rf = O.oracle_fwd(x["q"], x["k"], x["v"], g, unit_mask=mask, window=64, gate_logits=logits)
    rb = O.oracle_bwd(x["q"], x["k"], x["v"], g, x["dO"], unit_mask=mask, window=64, gate_logits=logits)
    errs = {"o": err_rms(o.cpu().numpy(), rf["o"])}
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
        errs[n] = err_rms(t.cpu().numpy(), rb[n])
    ok = all(v <= (5e-3 if n == "dg" else 1e-2) for n, v in errs.items())
    return ok, errs


def cpu_baseline(x, logits=False):
    """The fp64 oracle, fwd + bwd, on four heads of one batch row of the same workload, full length."""
    import oracle as O
    NH = 4
    sl = lambda a: np.ascontiguousarray(a[:1, :, :NH])
    q, k, v, g, dO = (sl(x[n]) for n in ("q", "k", "v", "g_logits" if logits else "g", "dO"))
    O.load()
    t0 = time.perf_counter()
    O.oracle_fwd(q, k, v, g, gate_logits=logits)
    t1 = time.perf_counter()
    O.oracle_bwd(q, k, v, g, dO, gate_logits=logits)
    t2 = time.perf_counter()
    wl = x["workload"]
    pairs = wl.T * (wl.T + 1) // 2 * NH
    flops = (2 * (wl.dk + wl.dv) + 2 * (3 * wl.dk + 2 * wl.dv)) * pairs
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"heads 0-{NH - 1} of batch row 0 of the workload: B=1 T={wl.T} H={NH} d={wl.dk}, "
                      f"fwd {t1 - t0:.1f} s + "
                      f"bwd {t2 - t1:.1f} s (the backward recomputes the forward)"}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate-logits", action="store_true",
                    help="pass the gate as raw logits (logsigmoid applied inside the kernels)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (HBM counter calibration)")
    ap.add_argument("--scalar-gate", action="store_true",
                    help="one gate value per token and kv head (channel 0 of the workload's gate): the "
                         "logit-bias forward and the broadcast backward")
    ap.add_argument("--decode", action="store_true",
                    help="time decode steps (fix_decode_step) against a cache holding the workload's T tokens")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build runs the kernel on one GPU's share and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    import gated_softmax_attention_amd as F
    from gated_softmax_attention_amd import synth

    x = synth.make_inputs(WORKLOAD)
    if args.scalar_gate:
        x = dict(x)
        x["g"] = np.ascontiguousarray(x["g"][..., 0])
        x["g_logits"] = np.ascontiguousarray(x["g_logits"][..., 0])
    if args.decode:
        decode_bench(args, x, F, torch)
        return
    wl = x["workload"]
    dev = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    d = {n: dev(x[n]) for n in ("q", "k", "v", "dO")}
    d["g"] = dev(x["g_logits"] if args.gate_logits else x["g"], torch.float32)
    print(f"[bench] inputs resident: {wl}{' (gate as logits)' if args.gate_logits else ''}", file=sys.stderr,
          flush=True)

    ok, errs = parity_gate(x, d, F, torch, logits=args.gate_logits)
    print(f"[bench] parity gate: {'pass' if ok else 'FAIL'} {errs}", file=sys.stderr, flush=True)
    if not ok:
        sys.exit(1)

    B, T, Hq, dk = d["q"].shape
    Hkv, dv = d["k"].shape[2], d["v"].shape[3]
    bf = torch.bfloat16
    o = torch.empty(B, T, Hq, dv, dtype=bf, device="cuda")
    m = torch.empty(B, T, Hq, device="cuda")
    rstd = torch.empty(B, T, Hq, device="cuda")
    xx = torch.empty(B, T, Hq, dv, device="cuda")
    dq, dkk, dvv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    dg = torch.empty_like(d["g"])
    desc = F.make_desc(d["q"], d["k"], d["v"], o_norm=True, gate_logits=args.gate_logits,
                       gate_scalar=args.scalar_gate)
    wf, wb = F.fix_attn_fwd_workspace_size(desc), F.fix_attn_bwd_workspace_size(desc)
    ws_f = torch.empty(wf, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(wb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lib = F.library()
    lib.fix_attn_set_event_trace.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.fix_attn_event_trace_count.restype = ctypes.c_int
    lib.fix_attn_event_trace_label.restype = ctypes.c_char_p
    lib.fix_attn_event_trace_label.argtypes = [ctypes.c_int]

    def step():
        F.fix_attn_fwd(desc, d["q"], d["k"], d["v"], d["g"], None, None, o, m, rstd, xx, ws_f, wf, stream)
        F.fix_attn_bwd(desc, d["q"], d["k"], d["v"], d["g"], None, None, m, rstd, xx, d["dO"], dq, dkk, dvv, dg,
                       None, None, ws_b, wb, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-kernel events recorded by the library on its stream during the timed steps.
    h = hip()
    cap = 16
    ev = [[(ctypes.c_void_p * cap)() for _ in range(2)] for _ in range(args.steps)]
    for s in ev:
        for arr in s:
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
        F.fix_attn_fwd(desc, d["q"], d["k"], d["v"], d["g"], None, None, o, m, rstd, xx, ws_f, wf, stream)
        counts[0] = lib.fix_attn_event_trace_count()
        if labels[0] is None:
            labels[0] = [lib.fix_attn_event_trace_label(i).decode() for i in range(1, counts[0])]
        lib.fix_attn_set_event_trace(ctypes.cast(ev[k][1], ctypes.c_void_p), cap)
        F.fix_attn_bwd(desc, d["q"], d["k"], d["v"], d["g"], None, None, m, rstd, xx, d["dO"], dq, dkk, dvv, dg,
                       None, None, ws_b, wb, stream)
        counts[1] = lib.fix_attn_event_trace_count()
        if labels[1] is None:
            labels[1] = [lib.fix_attn_event_trace_label(i).decode() for i in range(1, counts[1])]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.fix_attn_set_event_trace(None, 0)
    ms_step = (t1 - t0) * 1e3 / args.steps

    per_kernel = {}
    for k in range(args.steps):
        for side in (0, 1):
            for i in range(1, counts[side]):
                t = ctypes.c_float()
                assert h.hipEventElapsedTime(ctypes.byref(t), ev[k][side][i - 1], ev[k][side][i]) == 0
                per_kernel.setdefault(labels[side][i - 1], []).append(t.value)
    avg = {n: sum(v) / len(v) for n, v in per_kernel.items()}

    pc = pair_counts([T] * B)
    heads = Hq
    fwd_flops = 2 * (dk + dv) * pc["all"] * heads
    bwd_flops = 2 * (3 * dk + 2 * dv) * pc["all"] * heads
    total = fwd_flops + bwd_flops
    tflops = total / (ms_step * 1e-3) / 1e12
    # Algorithmic flops of each kernel: its share of the 2 forward and 5 backward products.
    alg = {
        "fix_fwd": fwd_flops,
        "fox_fwd": fwd_flops,
        "bwd_dq": 2 * (2 * dk + dv) * pc["inter"] * heads,        # S, dP, dQ on pairs in different chunks
        "bwd_dkv": 2 * (dk + dv) * pc["far"] * heads,             # dV, dK on pairs two or more chunks apart
        "bwd_intra_dq": 2 * (2 * dk + dv) * pc["same"] * heads,
        "bwd_intra_dkv": 2 * (dk + dv) * (pc["same"] + pc["adj"]) * heads,
    }
    dom = max(avg, key=avg.get)
    roof = None
    if dom in alg:
        ach = alg[dom] / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom),
                "avg_launch_ms": round(avg[dom], 4)}
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: B={B} T={T} Hq={Hq} Hkv={Hkv} dk={dk} dv={dv} bf16 in/out, "
                               f"g=logsigmoid(N({wl.gate_mu},{wl.gate_sd}))"
                               f"{' passed as logits (logsigmoid in the kernels)' if args.gate_logits else ''}"
                               f"{', scalar per token and head (channel 0)' if args.scalar_gate else ''}, "
                               f"o_norm, fwd+bwd",
                   "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                   "fwd_flops": fwd_flops, "bwd_flops": bwd_flops,
                   "kernel_ms": {n: round(v, 4) for n, v in sorted(avg.items(), key=lambda kv: -kv[1])}},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(x, logits=args.gate_logits)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
