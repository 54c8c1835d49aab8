#!/usr/bin/env python3
"""Benchmark of the chunked Gated DeltaNet prefill forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR --copy-mib M [--workload NAME]
    python bench.py --summarize-mfma PMC_DIR


A step is one gdn_chunk_fwd over one batch of synthetic inputs already resident in HBM (for the
mixer workload: 48 back-to-back gdn_mixer_fwd layers).  Prints ONE JSON line with tokens/s per
layer, the roofline of the dominant kernel (timed with HIP events on the launch stream, in a
separate stage-by-stage loop), the whole-path roofline, and the fp64 CPU oracle timed on the host
as a baseline.

roofline.achieved is the path's algorithmic HBM bytes of one launch (24,832 B per token at Hk=16,
Hv=32: q and k 8,192, v 8,192, g and beta 256, o 8,192; plus 64 KiB per sequence and v-head for
hT, and again for h0 if given) divided by the dominant kernel's mean launch time.  The bytes that
kernel itself moves (its inputs, the workspace records it reads, its outputs) are reported beside
it as roofline.own_io, a different and larger figure.

The second form turns two rocprofv3 counter runs of the first form (one with --pmc FETCH_SIZE,
one with --pmc WRITE_SIZE, both with --copy-mib M) into profiles/traffic_<kernel>_<workload>.json:
the counters of the dominant kernel per dispatch, each scaled by what the same counter reads for a
plain device copy of M MiB, and a hash of the kernel's sources.  A later bench run reports that
traffic in roofline.traffic only while the hash still matches.  The third form prints the MFMA
utilisation of the chunk kernels from a rocprofv3 run with --pmc SQ_VALU_MFMA_BUSY_CYCLES
SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE.

Workloads (seeded, synthetic; see gdn_inputs.py):
    t16384_h16x32    single sequence, T=16384, Hk=16, Hv=32, d=128  (default: the largest)
    t256_h4, t539_h16x32, varlen7_t677_h0, t936_h16x32, t3399_h16x32
    t16384_h2x4      T=16384 at Hk=2, Hv=4: one GPU's share when the heads are split over 8 GPUs
    mixer_t936_x48   48 GDN mixer layers at T=936, Hk=16, Hv=32, one layer per seed
                     (--fused-norm: gdn_mixer_fwd_fused_norm, the norm inside the state pass;
                     --gates: gdn_mixer_fwd_gates, g and beta made from the projections)
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
REC_BYTES = 18944             # per-(chunk, v-head) workspace record
D = 128


# ------------------------------------------------------------------------------------------------
# Algorithmic bytes and flops
# ------------------------------------------------------------------------------------------------
def n_chunks(cu):
    L = np.diff(np.asarray(cu, dtype=np.int64))
    return int(np.sum((L + 63) // 64))


def path_bytes(T, N, Hk, Hv, with_h0):
    """Minimum HBM I/O of one gdn_chunk_fwd: q,k,v,g,beta in, o out, h0 in (if any), hT out."""
    state = N * Hv * D * D * 4
    return T * (2 * Hk * D * 2 + Hv * D * 2 + Hv * 8 + Hv * D * 2) + state * (2 if with_h0 else 1)


def path_flops(T, Hk, Hv):
    """Useful flops per token per v-head: three 128x128 products (W H, K^T U~, Q H) 98,304,
    triangular 64-wide products 24,960, the 64x64 solve 2,731, K K^T + Q K^T 16,384 per k-head."""
    r = Hv // Hk
    return T * Hv * (98304 + 24960 + 2731 + 16384 / r)


def prep_bytes(T, Hk, Hv, nch):
    return T * Hk * D * 2 * 2 + T * Hv * 8 + nch * Hv * REC_BYTES


def pass_bytes(T, N, Hk, Hv, nch, with_h0):
    state = N * Hv * D * D * 4
    return (T * Hk * D * 2 * 2 + T * Hv * D * 2 + nch * Hv * REC_BYTES
            + T * Hv * D * 2 + state * (2 if with_h0 else 1))


def mixer_bytes(T, N, Hk, Hv, gates=False):
    """Algorithmic bytes of one mixer layer: qkv, conv weights, g and beta (fp32) or, with the gate
    step, a and b (bf16) and A_log, dt_bias (fp32 per head), z, y, norm weight, hT."""
    C = (2 * Hk + Hv) * D
    gate_bytes = T * Hv * 4 + Hv * 8 if gates else T * Hv * 8
    return T * C * 2 + C * 4 * 2 + gate_bytes + T * Hv * D * 2 * 2 + D * 2 + N * Hv * D * D * 4


# ------------------------------------------------------------------------------------------------
def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------
# Measured HBM traffic of the dominant kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE)
# ------------------------------------------------------------------------------------------------
KERNEL_SOURCES = {
    "state_pass": ["gated_deltanet_chunked_amd/csrc/state_pass.hip", "gated_deltanet_chunked_amd/csrc/gdn_device.h"],
    "chunk_prep": ["gated_deltanet_chunked_amd/csrc/chunk_prep.hip", "gated_deltanet_chunked_amd/csrc/gdn_device.h"],
}
KERNEL_SYMBOLS = {"state_pass": "state_pass_kernel", "chunk_prep": "chunk_prep_kernel"}


def kernel_sha(kernel):
    """Hash of the kernel's sources with comments and blank runs removed, so that an edit of the
    comments alone does not mark its counter summary as stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_path(kernel, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")


def read_counter(run_dir, counter):
    """Per-dispatch sums of `counter` (KiB) by kernel name, from a rocprofv3 csv run directory."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (name, _), v in per.items():
        by_kernel.setdefault(name, []).append(v)
    return by_kernel


def summarize_traffic(fetch_dir, write_dir, copy_mib, workload):
    out = {"workload": workload, "copy_mib": copy_mib}
    copy_bytes = copy_mib * 2 ** 20
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        by_kernel = read_counter(run_dir, counter)
        # the calibration copy: the three largest dispatches of kernels whose name says they copy
        # (input uploads share the kernel name but are far smaller than the copy)
        copies = sorted((v for n, vs in by_kernel.items() if "copy" in n.lower() for v in vs), reverse=True)[:3]
        if not copies:
            raise SystemExit(f"no copy kernel found in {run_dir}")
        copy_kib = statistics.median(copies)
        calib = copy_bytes / (copy_kib * 1024.0)
        out[counter] = {"copy_kib": copy_kib, "bytes_per_counted_byte": calib, "kernels": {}}
        for kern, sym in KERNEL_SYMBOLS.items():
            vals = [v for n, vs in by_kernel.items() if sym in n for v in vs]
            if vals:
                out[counter]["kernels"][kern] = {"dispatches": len(vals), "kib_median": statistics.median(vals),
                                                 "bytes_per_launch": statistics.median(vals) * 1024.0 * calib}
    for kern in KERNEL_SYMBOLS:
        if kern in out["FETCH_SIZE"]["kernels"] and kern in out["WRITE_SIZE"]["kernels"]:
            rec = {"kernel": kern, "workload": workload, "src_sha": kernel_sha(kern),
                   "fetch_bytes": round(out["FETCH_SIZE"]["kernels"][kern]["bytes_per_launch"]),
                   "write_bytes": round(out["WRITE_SIZE"]["kernels"][kern]["bytes_per_launch"]),
                   "fetch_calibration": out["FETCH_SIZE"]["bytes_per_counted_byte"],
                   "write_calibration": out["WRITE_SIZE"]["bytes_per_counted_byte"],
                   "dispatches": [out["FETCH_SIZE"]["kernels"][kern]["dispatches"],
                                  out["WRITE_SIZE"]["kernels"][kern]["dispatches"]]}
            rec["traffic_bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
            with open(traffic_path(kern, workload), "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
            log(f"[bench] {kern}: {rec['traffic_bytes'] / 1e6:.2f} MB per launch -> {traffic_path(kern, workload)}")


def summarize_counters(run_dir):
    """MFMA utilisation of the two chunk kernels from a rocprofv3 --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_VALU_MFMA_MOPS_F32 and
    GRBM_GUI_ACTIVE.  GRBM_GUI_ACTIVE comes summed over the 8 XCDs, so the busy fraction is
    busy / (GRBM_GUI_ACTIVE / 8 * SIMDs); a MOPS count is 512 flops.  Printed as a markdown table."""
    import csv
    import glob
    simds = 256 * 4
    per = {}
    dur = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                kern = next((k for k, sym in KERNEL_SYMBOLS.items() if sym in r["Kernel_Name"]), None)
                if kern is None:
                    continue
                key = (kern, int(r["Dispatch_Id"]))
                d = per.setdefault(key, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    print("| kernel | dispatches | MFMA busy (of all SIMD cycles) | bf16 MFMA TFLOP/s (of 2,516.6) "
          "| fp32 MFMA TFLOP/s | MFMA flops per dispatch (bf16 / fp32) | µs per dispatch under counters |")
    print("|---|---|---|---|---|---|---|")
    for kern in KERNEL_SYMBOLS:
        keys = [k for k in per if k[0] == kern]
        if not keys:
            continue
        busy = statistics.median(per[k]["SQ_VALU_MFMA_BUSY_CYCLES"] / (per[k]["GRBM_GUI_ACTIVE"] / 8 * simds)
                                 for k in keys)
        bf = statistics.median(per[k]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for k in keys)
        f32 = statistics.median(per[k]["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512 for k in keys)
        t = statistics.median(dur[k] for k in keys)
        print(f"| {kern} | {len(keys)} | {busy:.3f} | {bf / t / 1e12:.1f} ({bf / t / 1e12 / BF16_PEAK_TFLOPS:.3f}) "
              f"| {f32 / t / 1e12:.2f} | {bf / 1e9:.2f} G / {f32 / 1e9:.3f} G | {t * 1e6:.1f} |")


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None if absent or stale."""
    try:
        with open(traffic_path(kernel, workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec["traffic_bytes"] if rec.get("src_sha") == kernel_sha(kernel) else None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warmup steps, repeat the step for this long (untimed) so that the "
                         "GPU clock has left its idle state; reported as timing.settle_*")
    ap.add_argument("--workload", default="t16384_h16x32")
    ap.add_argument("--rotate-mib", type=float, default=512.0,
                    help="rotate among input copies until their footprint exceeds this (cold caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gates", action="store_true",
                    help="mixer workload: gate parameters from the projections (gdn_mixer_fwd_gates)")
    ap.add_argument("--fused-norm", action="store_true",
                    help="mixer workload: gated RMSNorm fused into the state pass (gdn_mixer_fwd_fused_norm)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on oracle time for the baseline")
    ap.add_argument("--copy-mib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration under rocprofv3)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_*.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="print the chunk kernels' MFMA utilisation from a rocprofv3 --pmc run and exit")
    args = ap.parse_args()

    if args.summarize_mfma:
        summarize_counters(args.summarize_mfma)
        return

    if args.summarize_traffic:
        if args.copy_mib <= 0:
            raise SystemExit("--summarize-traffic needs the --copy-mib the runs used")
        summarize_traffic(*args.summarize_traffic, args.copy_mib, args.workload)
        return

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "requested_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import gated_deltanet_chunked_amd as gdn
    import gdn_inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"[bench] device {props.name} CUs={props.multi_processor_count} workload={args.workload}")

    mixer = args.workload.startswith("mixer")
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    if not mixer:
        case = gi.CASES[args.workload]
        x = gi.make_case(args.workload)
        T, N, Hk, Hv = case.T, case.N, case.Hk, case.Hv
        with_h0 = x.h0 is not None
        cu_host = torch.from_numpy(x.cu.astype(np.int64))
        base = dict(q=bf(x.q), k=bf(x.k), v=bf(x.v), g=f32(x.g), beta=f32(x.beta),
                    cu=torch.from_numpy(x.cu).to(dev), h0=None if x.h0 is None else f32(x.h0))
        per_set = sum(t.numel() * t.element_size() for t in base.values() if t is not None) + \
            T * Hv * D * 2 + N * Hv * D * D * 4
        R = max(1, int(np.ceil(args.rotate_mib * 2 ** 20 / per_set)))
        ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(T, N, Hk, Hv), dtype=torch.uint8, device=dev)
        plans = []
        for r in range(R):
            s = base if r == 0 else {kk: (None if t is None else t.clone()) for kk, t in base.items()}
            plans.append(gdn.ChunkPlan(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu"], s["h0"],
                                       workspace=ws, cu_seqlens_host=cu_host))
        step = lambda i: plans[i % R].forward()
        tokens_per_step = T
        layers_per_step = 1
    else:
        T, N, Hk, Hv, LAYERS = gi.MIXER_T, 1, 16, 32, gi.MIXER_LAYERS
        with_h0 = False
        log(f"[bench] generating {LAYERS} mixer layers")
        layers = []
        for l in range(LAYERS):
            m = gi.make_mixer_inputs(100 + l)
            layers.append(dict(qkv=bf(m.qkv), conv_w=bf(m.conv_w), g=f32(m.g), beta=f32(m.beta), z=bf(m.z),
                               norm_w=bf(m.norm_w), cu=torch.from_numpy(m.cu).to(dev)))
            if args.gates:
                gt = gi.make_gate_inputs(200 + l, T, Hv)
                layers[-1].update(a=bf(gt.a), b=bf(gt.b), A_log=f32(gt.A_log), dt_bias=f32(gt.dt_bias))
        cu_host = torch.tensor([0, T], dtype=torch.int64)
        ws = torch.empty(gdn.gdn_mixer_fwd_workspace_size(T, N, Hk, Hv), dtype=torch.uint8, device=dev)
        ys = [torch.empty((T, Hv, D), dtype=torch.bfloat16, device=dev) for _ in range(LAYERS)]
        hs = [torch.empty((N, Hv, D, D), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
        R = 1

        def step(i):
            for l, L_ in enumerate(layers):
                if args.gates:
                    gdn.gdn_mixer_fwd_gates(L_["qkv"], L_["conv_w"], L_["a"], L_["b"], L_["A_log"], L_["dt_bias"],
                                            L_["z"], L_["norm_w"], L_["cu"], None, y=ys[l], hT=hs[l],
                                            workspace=ws, cu_seqlens_host=cu_host)
                else:
                    gdn.gdn_mixer_fwd(L_["qkv"], L_["conv_w"], L_["g"], L_["beta"], L_["z"], L_["norm_w"], L_["cu"],
                                      None, y=ys[l], hT=hs[l], workspace=ws, cu_seqlens_host=cu_host,
                                      fused_norm=args.fused_norm)
        tokens_per_step = T * LAYERS
        layers_per_step = LAYERS

    # ---- clock settling, warmup, timed region --------------------------------------------------
    # A GPU that has been idle starts a run at a lower clock and reaches its sustained clock only
    # after some tens of milliseconds of load (T = 16,384: 414 us per step over the first 25 steps,
    # 350 us over 200).  The step is therefore repeated, untimed, for --settle-ms first; the warmup
    # steps and the exactly --steps timed steps follow.
    t_settle = time.perf_counter()
    settle_steps = 0
    while True:
        step(settle_steps)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t_settle) * 1e3 >= args.settle_ms:
                break
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    tokens_per_s = tokens_per_step / (ms_per_step * 1e-3)   # tokens per second per layer
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall_s * 1e6 / args.steps:.1f} us)")

    # ---- per-kernel timing (HIP events on the launch stream, one stage at a time) ---------------
    stages = {}
    if not mixer:
        nch = n_chunks(x.cu)
        dur = {"chunk_prep": [], "state_pass": []}
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
        for i in range(args.steps):
            p = plans[i % R]
            ev[3 * i].record()
            p.prep()
            ev[3 * i + 1].record()
            p.state_pass()
            ev[3 * i + 2].record()
        torch.cuda.synchronize()
        for i in range(args.steps):
            dur["chunk_prep"].append(ev[3 * i].elapsed_time(ev[3 * i + 1]) * 1e3)
            dur["state_pass"].append(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) * 1e3)
        kbytes = {"chunk_prep": prep_bytes(T, Hk, Hv, nch), "state_pass": pass_bytes(T, N, Hk, Hv, nch, with_h0)}
        alg = path_bytes(T, N, Hk, Hv, with_h0)
        for kname, ds in dur.items():
            us = statistics.mean(ds)
            stages[kname] = {"us_mean": us, "us_median": statistics.median(ds), "bytes": kbytes[kname],
                             "GBps": kbytes[kname] / (us * 1e-6) / 1e9}
            log(f"[bench] {kname}: {us:.2f} us mean, {stages[kname]['GBps']:.0f} GB/s of its own I/O")
        dominant = max(stages, key=lambda k: stages[k]["us_mean"])
        dom = stages[dominant]
        ach = alg / (dom["us_mean"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(dominant, args.workload),
                    "bytes_per_launch": alg, "us_per_launch": round(dom["us_mean"], 3),
                    "own_io": {"bytes": dom["bytes"], "GBps": round(dom["GBps"], 1),
                               "frac": round(dom["GBps"] / HBM_PEAK_GBS, 4)}}
        pb, pf = path_bytes(T, N, Hk, Hv, with_h0), path_flops(T, Hk, Hv)
    else:
        pb = layers_per_step * (mixer_bytes(T, N, Hk, Hv, args.gates))
        pf = layers_per_step * (path_flops(T, Hk, Hv) + T * (2 * Hk + Hv) * D * 8)
        roofline = {"bound": "hbm", "kernel": "mixer step (48 layers)", "achieved": round(pb / (ms_per_step * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(pb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None}
    t_roof_us = max(pb / (HBM_PEAK_GBS * 1e9), pf / (BF16_PEAK_TFLOPS * 1e12)) * 1e6
    path = {"bytes": int(pb), "flops": int(pf), "t_roof_us": round(t_roof_us, 3),
            "frac": round(t_roof_us / (ms_per_step * 1e3), 4),
            "mfma_util_useful": round(pf / (ms_per_step * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}

    # ---- parity of the timed outputs against the oracle (cheap for the default workload) ------
    parity = None
    if not mixer and T <= 16384:
        import oracle
        p = plans[(args.warmup + args.steps - 1) % R]
        o_ref, h_ref = oracle.gdn_fwd(*x.f64())
        o = p.o.float().cpu().numpy()
        h = p.hT.cpu().numpy()
        parity = {"o_rel_l2": float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)),
                  "o_max_abs": float(np.abs(o - o_ref).max()),
                  "hT_rel_l2": float(np.linalg.norm(h - h_ref) / np.linalg.norm(h_ref))}

    # ---- optional plain copy kernel of known size (counter calibration) ----------------------
    if args.copy_mib > 0:
        n = int(args.copy_mib * 2 ** 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy kernel: {args.copy_mib} MiB read + {args.copy_mib} MiB written, 3 launches")

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same workload -----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.max_threads()
        if not mixer:
            f64 = x.f64()
            t0 = time.perf_counter()
            oracle.gdn_fwd(*f64)
            once = time.perf_counter() - t0
            reps = max(1, min(5, int(args.cpu_seconds / max(once, 1e-6))))
            times = [once]
            for _ in range(reps - 1):
                t0 = time.perf_counter()
                oracle.gdn_fwd(*f64)
                times.append(time.perf_counter() - t0)
            med = statistics.median(times)
            cpu = {"value": round(T / med, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                   "sample": f"whole workload ({T} tokens, {Hv} v-heads), median of {len(times)} runs, fp64"}
        else:
            m = gi.make_mixer_inputs(100)
            fb = gi.bits_to_f64
            t0 = time.perf_counter()
            oracle.mixer_fwd(fb(m.qkv), fb(m.conv_w), m.g, m.beta, fb(m.z), fb(m.norm_w), m.cu, None)
            once = time.perf_counter() - t0
            cpu = {"value": round(T / once, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                   "sample": f"one of the 48 layers ({T} tokens), fp64"}
        log(f"[bench] cpu baseline {cpu['value']} tokens/s on {threads} threads")

    cfg = {"workload": args.workload, "T": T, "N": N, "Hk": Hk, "Hv": Hv, "d": D, "chunk": 64,
           "rotating_input_sets": R, "layers_per_step": layers_per_step}
    if mixer:
        cfg["norm"] = "fused into the state pass" if args.fused_norm else "separate kernel"
        cfg["gates"] = "from the projections" if args.gates else "inputs"
    line = {"metric": "GDN prefill tokens/s per layer (Hk16/Hv32,d128) + % MFMA/HBM roofline",
            "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": cfg,
            "roofline": roofline, "cpu_baseline": cpu, "path_roofline": path, "stages": stages,
            "parity": parity, "device": {"name": props.name, "cus": props.multi_processor_count},
            "timing": {"settle_ms": round(settle_ms, 1), "settle_steps": settle_steps,
                       "note": "untimed steps before the warmup steps, until the GPU clock has settled"}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
