"""Benchmark: one quantized training step of an MLP up-projection on one
MI355X, through the library's C ABI.

Step (Quartet II linear-layer scheme: forward RTN NVFP4, backward
re-quantization along the reduction dimension with the randomized Hadamard
rotation and MS-EDEN):
  forward   qX  = RTN(X)            [32768 x 4096]   axis 0
            qW  = RTN(W)            [11008 x 4096]   axis 0
            Y   = qX qW^T           [32768 x 11008]  bf16
  backward  qdYr = MSEDEN(dY)       [32768 x 11008]  axis 0, rotation
            qWc  = MSEDEN(W)        [4096 x 11008]   axis 1, rotation
            dX   = qdYr qWc^T       [32768 x 4096]   bf16
            qdYc = MSEDEN(dY)       [11008 x 32768]  axis 1, rotation
            qXc  = MSEDEN(X)        [4096 x 32768]   axis 1, rotation
            dW   = qdYc qXc^T       [11008 x 4096]   fp32
Inputs: X ~ N(0,1), W ~ N(0, 0.02^2), dY ~ N(0, 1e-3^2), bf16, seed 4.

Reported: `value` = quantizer throughput over the six quantizations, in
algorithmic GB/s (bf16 input read once + codes + scales written once =
2.5625 bytes per element) divided by their measured time; `gemm` = the three
GEMMs' 2MNK flops over their time.  `roofline` describes the GEMM kernel
(the dominant one), `cpu_baseline` the CPU oracle on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 quantize GB/s (% HBM peak); block-scaled FP4 GEMM TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
BYTES_PER_ELEM_BF16 = 2.5625   # 2 (read) + 0.5 (codes) + 0.0625 (scales)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra configurations after the step (profiling runs: then every "
                         "k_gemm launch is one of the step's GEMMs)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="approximate budget for the CPU oracle sample (all threads and one thread)")
    ap.add_argument("--extras-only", action="store_true",
                    help="no step, no CPU baseline: only the extra configurations, each timed once as a "
                         "graph (profiling runs of the kernels outside the step)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="before the warm-up, run one plain fp32 negation of GIB GiB (reads and writes "
                         "exactly that many bytes): the reference that scales the HBM byte counters")
    ap.add_argument("--activity-from", metavar="PMC_DIR",
                    help="no benchmark: print a markdown table of the activity counters of one rocprofv3 "
                         "--pmc run of this script (GRBM_GUI_ACTIVE, SQ_* counters), per library kernel")
    ap.add_argument("--per-kernel", action="store_true",
                    help="with --activity-from: one row per kernel instance (means over its launches)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no benchmark: read two rocprofv3 --pmc outputs of this script (FETCH_SIZE, "
                         "then WRITE_SIZE, both run with the --copy-calibration given here) and write "
                         "profiles/traffic.json")
    return ap.parse_args()


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "nvfp4_bit_block_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, digest, launch_flops_or_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(kernel)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("hbm_bytes_per_launch")


COPY_KERNEL_TAG = "neg"   # the calibration kernel's name contains this


def _counter_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter):
    """kernel name -> list of per-dispatch values of `counter` (summed over
    the rows rocprofv3 writes per dispatch)."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (k, _), v in sorted(acc.items(), key=lambda kv: int(kv[0][1])):
        out.setdefault(k, []).append(v)
    return out


def write_traffic(fetch_dir, write_dir, cal_gib):
    """HBM bytes per launch of each library kernel, from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled so that the calibration copy
    reads / writes exactly its known size."""
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")
    cal = [k for k in fetch if COPY_KERNEL_TAG in k]
    if not cal:
        raise SystemExit("calibration kernel not found: run with --copy-calibration")
    if cal_gib <= 0:
        raise SystemExit("give the --copy-calibration size the counter runs used")
    cal_bytes = float(int(cal_gib * (1 << 30)) // 4 * 4)
    f_scale = cal_bytes / (fetch[cal[0]][0] * 1024.0)
    w_scale = cal_bytes / (write[cal[0]][0] * 1024.0)
    digests = {"k_gemm": source_digest("gemm.hip", "common.hpp", "kernels.hpp"),
               "k_gemm_if4": source_digest("gemm.hip", "common.hpp", "kernels.hpp"),
               "k_quant": source_digest("quantize.hip", "common.hpp", "kernels.hpp"),
               "k_eden_scales": source_digest("quantize.hip", "common.hpp", "kernels.hpp")}
    out = {"calibration": {"bytes": cal_bytes, "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
                           "kernel": cal[0]}}
    for name in fetch:
        if "nv4::" not in name:
            continue
        short = name.split("nv4::")[1].split("(")[0]
        fam = next((d for d in digests if short.startswith(d)), None)
        fb = [v * 1024.0 * f_scale for v in fetch[name]]
        wb = [v * 1024.0 * w_scale for v in write.get(name, [0.0])]
        if short.startswith("k_gemm"):
            # k_gemm<OUT_BF16, FAST, IF4>: the step's GEMMs are the NVFP4 ones
            fam_key = "k_gemm_if4" if short.replace(" ", "").endswith(",1>") else "k_gemm"
        else:
            fam_key = short
        e = out.setdefault(fam_key, {"source_digest": digests.get(fam), "instances": {}})
        e["instances"][short] = {"launches": len(fb), "fetch_bytes": [round(x) for x in fb],
                                 "write_bytes": [round(x) for x in wb]}
    for k, e in out.items():
        if k == "calibration":
            continue
        allf = [x for i in e["instances"].values() for x in i["fetch_bytes"]]
        allw = [x for i in e["instances"].values() for x in i["write_bytes"]]
        e["hbm_bytes_per_launch"] = round((sum(allf) + sum(allw)) / max(1, len(allf)))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")


def compiler_registers():
    """kernel symbol -> (VGPRs, AGPRs, SGPRs, LDS bytes) from the device
    assembly the build keeps (the compiler's resource metadata)."""
    import glob
    import re
    out = {}
    for f in glob.glob(os.path.join(ROOT, "nvfp4_bit_block_amd", "_build", "*.s")):
        name = None
        vals = {}
        for line in open(f):
            m = re.match(r"\s+\.(name|vgpr_count|agpr_count|sgpr_count|group_segment_fixed_size):\s+(\S+)", line)
            if not m:
                continue
            k, v = m.group(1), m.group(2)
            if k == "group_segment_fixed_size":
                if name and vals:
                    out[name] = vals
                vals, name = {"lds": int(v)}, None
            elif k == "name":
                name = v
            else:
                vals[k] = int(v)
            if name and "vgpr_count" in vals and "sgpr_count" in vals:
                out[name] = dict(vals)
    import subprocess
    names = list(out)
    try:
        dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout.split("\n")
    except OSError:
        dem = names
    return {d.strip(): out[n] for n, d in zip(names, dem)}


def write_activity(pmc_dir, per_kernel=False):
    """Per-dispatch activity of the library's kernels from one rocprofv3
    --pmc run, as markdown: duration, clock (GRBM_GUI_ACTIVE counts core
    clock cycles summed over the 8 XCDs; its window also covers a few
    microseconds of dispatch and drain around the kernel, so the clock is
    given only for kernels longer than 200 us), matrix-pipe busy fraction,
    vector instructions and waits per wave-cycle, and the compiler's
    register counts."""
    import csv
    import glob
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    acc = {}
    for r in csv.DictReader(open(files[0])):
        if "nv4::" not in r["Kernel_Name"]:
            continue
        key = int(r["Dispatch_Id"])
        e = acc.setdefault(key, {"name": r["Kernel_Name"], "dur": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                 "c": {}})
        e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    regs = compiler_registers()
    if per_kernel:
        # one row per instance: sums of the counters and durations over its launches
        merged = {}
        for key in sorted(acc):
            e = acc[key]
            m = merged.setdefault(e["name"], {"name": e["name"], "dur": 0, "c": {}, "n": 0, "long": 0})
            m["n"] += 1
            m["dur"] += e["dur"]
            for k, v in e["c"].items():
                m["c"][k] = m["c"].get(k, 0.0) + v
        acc = {i: m for i, m in enumerate(sorted(merged.values(), key=lambda m: -m["dur"]))}
    print("| Kernel | " + ("Launches | Mean duration (us)" if per_kernel else "Duration (us)") +
          " | Clock (GHz) | MFMA busy | VALU instr. / wave-cycle | s_waitcnt / wave-cycle "
          "| LDS wait / wave-cycle | VGPR / AGPR / LDS bytes (compiler) |")
    print("|---|---|---|---|---|---|---|---|" + ("---|" if per_kernel else ""))
    for key in sorted(acc):
        e = acc[key]
        c = e["c"]
        short = e["name"].split("nv4::")[1].split("(")[0]
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        dur = e["dur"]
        n = e.get("n", 1)
        clock = f"{cyc / (dur * 1e-9) / 1e9:.2f}" if dur / n > 200e3 and cyc else "n/a"
        busy = f"{c.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / (1024 * cyc):.3f}" if cyc else "n/a"
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        valu = f"{c.get('SQ_ACTIVE_INST_VALU', 0.0) / wc:.3f}" if wc else "n/a"
        wait = f"{c.get('SQ_WAIT_INST_ANY', 0.0) / wc:.3f}" if wc else "n/a"
        lds = f"{c.get('SQ_WAIT_INST_LDS', 0.0) / wc:.3f}" if wc else "n/a"
        rg = regs.get(e["name"].strip())
        r = f"{rg.get('vgpr_count', '?')} / {rg.get('agpr_count', 0)} / {rg.get('lds', '?')}" if rg else "?"
        head = f"{n} | {dur / n / 1e3:.1f}" if per_kernel else f"{dur / 1e3:.1f}"
        print(f"| `{short}` | {head} | {clock} | {busy} | {valu} | {wait} | {lds} | {r} |")


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.copy_calibration)
        return
    if args.activity_from:
        write_activity(args.activity_from, args.per_kernel)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the quantizers and the "
                          "GEMM are single-device kernels; run with --gpus 1"}), flush=True)
        sys.exit(2)
    import torch
    import nvfp4_bit_block_amd as nv
    from nvfp4_bit_block_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nv.lib()
    if args.extras_only:
        print(json.dumps({"extras_only": other_configs(nv, torch)}), flush=True)
        return

    T, D, O = synth.MLP_SHAPES["X"][0], synth.MLP_SHAPES["X"][1], synth.MLP_SHAPES["W"][0]
    t0 = time.time()
    rng = np.random.default_rng(4)

    def draw(shape, scale):
        a = rng.standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        g = torch.from_numpy(a).to(dev).to(torch.bfloat16)   # round to nearest even
        return a, g

    Xh, X = draw((T, D), 1.0)
    Wh, W = draw((O, D), 0.02)
    dYh, dY = draw((T, O), 1e-3)
    signs = synth.signs_from_rng(rng)
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def ws_for(rows, cols, rounding, axis):
        return torch.empty(nv.workspace_size(rows, cols, rounding, axis), dtype=torch.uint8, device=dev)

    def qt(rows_out, k):
        return nv.QTensor(torch.empty((rows_out, k // 2), dtype=torch.uint8, device=dev),
                          torch.empty((rows_out, k // 16), dtype=torch.uint8, device=dev),
                          torch.empty(1, dtype=torch.float32, device=dev))

    # preallocated outputs and workspaces: the timed region allocates nothing
    plan = [  # name, input, rounding, axis, rotation, rows_out, K
        ("qX", X, nv.RTN, 0, None, T, D),
        ("qW", W, nv.RTN, 0, None, O, D),
        ("qdYr", dY, nv.MSEDEN, 0, signs, T, O),
        ("qWc", W, nv.MSEDEN, 1, signs, D, O),
        ("qdYc", dY, nv.MSEDEN, 1, signs, O, T),
        ("qXc", X, nv.MSEDEN, 1, signs, D, T),
    ]
    outs = {n: qt(r, k) for n, _, _, _, _, r, k in plan}
    wss = {n: ws_for(x.shape[0], x.shape[1], rnd, ax) for n, x, rnd, ax, _, _, _ in plan}
    # X and W are quantized column-wise (for the gradients) right before their
    # row-wise RTN (for Y): each column-wise MS-EDEN pass also writes max|x|,
    # the row-wise RTN's tensor scale takes it, and X and W are read once
    # less than with a separate maximum pass.  The two passes over a tensor
    # run back to back, so the row pass finds part of the tensor still in the
    # 256 MB memory-side cache (all of W's 90 MB, part of X's 268 MB).
    amax = {"X": torch.zeros(1, dtype=torch.float32, device=dev),
            "W": torch.zeros(1, dtype=torch.float32, device=dev)}
    handoff = {"qXc": {"amax_out": amax["X"]}, "qWc": {"amax_out": amax["W"]},
               "qX": {"amax_in": amax["X"]}, "qW": {"amax_in": amax["W"]}}
    by_name = {e[0]: e for e in plan}
    Y = torch.empty((T, O), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((O, D), dtype=torch.float32, device=dev)
    gemms = [("Y", "qX", "qW", Y), ("dX", "qdYr", "qWc", dX), ("dW", "qdYc", "qXc", dW)]
    stream = torch.cuda.current_stream()

    def quantize(name, x, rnd, ax, sg, step):
        nv.quantize_nvfp4(x, rounding=rnd, axis=ax, rht_signs=sg, seed=1000 + len(name), stream_id=step,
                          out=outs[name], workspace=wss[name], **handoff.get(name, {}))

    ev_pool = []

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev_pool.append(e)
        return e

    def step(i, timed):
        marks = []

        def q(names):
            for n in names:
                _, x, rnd, ax, sg, _, _ = by_name[n]
                a = ev() if timed else None
                quantize(n, x, rnd, ax, sg, i)
                marks.append(("q", n, a, ev() if timed else None))

        def g(name, qa, qb, out):
            a = ev() if timed else None
            nv.gemm_nvfp4(outs[qa], outs[qb], out=out)
            marks.append(("g", name, a, ev() if timed else None))

        q(("qXc", "qX", "qWc", "qW"))     # per tensor, column-wise first: it hands max|x| on
        g("Y", "qX", "qW", Y)
        q(("qdYr",))
        g("dX", "qdYr", "qWc", dX)
        q(("qdYc",))
        g("dW", "qdYc", "qXc", dW)
        return marks

    if args.copy_calibration > 0:
        n = int(args.copy_calibration * (1 << 30)) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
        print(json.dumps({"calibration_bytes": n * 4}), file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    progress(f"{args.warmup} warm-up steps done")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    all_marks = []
    start.record(stream)
    for i in range(args.steps):
        all_marks.append(step(args.warmup + i, True))
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    progress(f"{args.steps} timed steps: {ms_per_step:.3f} ms per step")

    qms = {n: 0.0 for n, *_ in plan}
    gms = {n: 0.0 for n, *_ in gemms}
    for marks in all_marks:
        for kind, n, a, b in marks:
            (qms if kind == "q" else gms)[n] += a.elapsed_time(b)
    for d in (qms, gms):
        for n in d:
            d[n] /= args.steps
    q_elems = {n: x.numel() for n, x, *_ in plan}
    q_bytes = sum(q_elems[n] * BYTES_PER_ELEM_BF16 for n in q_elems)
    q_time_ms = sum(qms.values())
    q_gbs = q_bytes / (q_time_ms * 1e-3) / 1e9
    flops = {"Y": 2.0 * T * O * D, "dX": 2.0 * T * D * O, "dW": 2.0 * O * D * T}
    g_time_ms = sum(gms.values())
    g_tflops = sum(flops.values()) / (g_time_ms * 1e-3) / 1e12
    gemm_launch_ms = g_time_ms / 3.0
    gemm_flops_launch = flops["Y"]
    achieved = gemm_flops_launch / (gemm_launch_ms * 1e-3) / 1e12

    kernels = {}
    for n, x, rnd, ax, sg, r, k in plan:
        gbs = q_elems[n] * BYTES_PER_ELEM_BF16 / (qms[n] * 1e-3) / 1e9
        kernels[n] = {"ms": round(qms[n], 4), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                      "rounding": ["rtn", "sr", "mseden"][rnd], "axis": ax, "rotation": sg is not None,
                      "shape_in": list(x.shape)}
    for n, *_ in gemms:
        tf = flops[n] / (gms[n] * 1e-3) / 1e12
        kernels["gemm_" + n] = {"ms": round(gms[n], 4), "TFLOP/s": round(tf, 1),
                                "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 3)}

    digest = source_digest("gemm.hip", "common.hpp", "kernels.hpp")
    traffic = measured_traffic("k_gemm", digest, gemm_flops_launch)
    result = {
        "metric": METRIC,
        "value": round(q_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "mlp_up_projection_training_step", "X": [T, D], "W": [O, D],
                   "dY": [T, O], "input_dtype": "bf16", "rotation": 128,
                   "quantizations": "RTN(X,W) fwd; RHT+MS-EDEN(dY row+col, W col, X col) bwd; "
                                    "X col then X row, W col then W row: each col pass hands max|x| to its row RTN",
                   "gemms": "Y=XW^T (bf16), dX=dY W (bf16), dW=dY^T X (fp32)"},
        "hbm_frac": round(q_gbs / HBM_PEAK_GBS, 3),
        "gemm": {"value": round(g_tflops, 1), "unit": "TFLOP/s",
                 "frac": round(g_tflops / MFMA_F16_PEAK_TFLOPS, 3),
                 "dtype": "f16 MFMA on exactly dequantized FP4, f32 accumulate"},
        "roofline": {"kernel": "k_gemm", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "launch_ms": round(gemm_launch_ms, 4),
                     "flops_per_launch": gemm_flops_launch},
        "kernels": kernels,
    }

    if not args.no_extras:
        result["extras"] = extras(nv, torch, stream, X, W, dY, signs, outs, wss, args.steps)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(Xh, Wh, dYh, signs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def progress(msg):
    """A progress line on stderr (long profiling runs stay visibly alive)."""
    print(f"# {msg}", file=sys.stderr, flush=True)


MALL_BYTES = 256e6      # MI355X memory-side (Infinity) cache
ROTATE_BYTES = 600e6    # distinct bytes one rotation of copies touches


def graph_time(torch, fns, min_calls=20, replays=5):
    """GPU time per call, in ms, of the calls fns[0], fns[1], ... repeated
    round-robin: at least `min_calls` calls captured in one HIP graph (short
    calls launched one by one from Python would leave the GPU waiting on the
    host), replayed `replays` times after one untimed replay.  With several
    fns working on distinct copies of their data, each call finds its input
    evicted from the memory-side cache by the calls before it."""
    n = max(min_calls, len(fns))
    n = (n + len(fns) - 1) // len(fns) * len(fns)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            fns[i % len(fns)]()
    graph.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * n)


def n_copies(bytes_per_copy):
    """Copies of a call's data so that one round over them touches more
    than the memory-side cache holds (1 if one copy already does)."""
    if bytes_per_copy >= 2 * MALL_BYTES:
        return 1
    return max(1, int(np.ceil(ROTATE_BYTES / bytes_per_copy)))


def _q_entry(x, ms, what, copies, bytes_per_elem=BYTES_PER_ELEM_BF16):
    progress(f"{what}: {ms:.4f} ms")
    gbs = x.numel() * bytes_per_elem / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
            "shape_in": list(x.shape), "copies": copies, "what": what}


def _g_entry(flops, ms, what, copies):
    progress(f"{what}: {ms:.4f} ms")
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 3),
            "copies": copies, "what": what}


def _qbuf(nv, torch, x, axis, rounding, dev):
    R, K = (x.shape[0], x.shape[1]) if axis == 0 else (x.shape[1], x.shape[0])
    q = nv.QTensor(torch.empty((R, K // 2), dtype=torch.uint8, device=dev),
                   torch.empty((R, K // 16), dtype=torch.uint8, device=dev),
                   torch.empty(1, dtype=torch.float32, device=dev))
    w = torch.empty(nv.workspace_size(x.shape[0], x.shape[1], rounding, axis), dtype=torch.uint8, device=dev)
    return q, w


def rotating_quant(nv, torch, x, call, axis=0, rounding="rtn"):
    """GPU ms per call of call(x_i, q_i, ws_i) over enough copies (input,
    output, workspace) of x to defeat the memory-side cache; returns
    (ms, copies)."""
    dev = x.device
    per = x.numel() * (x.element_size() + 0.5625) + (x.numel() // 4 if rounding == "mseden" else 0)
    k = n_copies(per)
    xs = [x] + [x.clone() for _ in range(k - 1)]
    bufs = [_qbuf(nv, torch, x, axis, rounding, dev) for _ in range(k)]
    fns = [(lambda xi=xi, b=b: call(xi, b[0], b[1])) for xi, b in zip(xs, bufs)]
    ms = graph_time(torch, fns)
    del xs, bufs, fns
    return ms, k


def extras(nv, torch, stream, X, W, dY, signs, outs, wss, reps):
    """Options beyond the step, timed on the same inputs (not part of
    `value`): dY quantized along both axes from one read; IF4 quantization of
    X and W and the Y GEMM on IF4 operands; Four Over Six and searched block
    scales for X and W; the Y GEMM writing NVFP4.  Calls on W (90 MB, which
    the 256 MB memory-side cache would hold between calls) rotate over
    copies of it."""
    dev = X.device
    res = {}
    # dY along both axes from one read (the step quantizes it twice)
    qr, qc = outs["qdYr"], outs["qdYc"]
    wsd = torch.empty(nv.workspace_size_dual(dY.shape[0], dY.shape[1]), dtype=torch.uint8, device=dev)
    ms = graph_time(torch, [lambda: nv.quantize_nvfp4_dual(dY, rht_signs=signs, seed=1004, stream_id=0,
                                                           out_rows=qr, out_cols=qc, workspace=wsd)], min_calls=3)
    res["dY_dual_axis"] = _q_entry(dY, ms, "RHT + MS-EDEN of dY along rows and columns from one read (input once, "
                                   "two sets of codes and scales)", 1, bytes_per_elem=2.0 + 2 * 0.5625)
    res["dY_dual_axis"]["bytes_per_elem"] = 3.125
    del wsd
    # the Y GEMM with its output coded as NVFP4 in the same kernel (RTN along
    # N, the tensor scale from a first call's max |Y|), on the step's operands
    Mq, Nq, Kq = X.shape[0], W.shape[0], X.shape[1]
    ymax = torch.zeros(1, dtype=torch.float32, device=dev)
    qy = nv.QTensor(torch.empty((Mq, Nq // 2), dtype=torch.uint8, device=dev),
                    torch.empty((Mq, Nq // 16), dtype=torch.uint8, device=dev),
                    torch.ones(1, dtype=torch.float32, device=dev), nv.FORMAT_NVFP4)
    nv.gemm_nvfp4_rtn(outs["qX"], outs["qW"], qy.tensor_scale, amax_out=ymax, out=qy)
    qy.tensor_scale.copy_(ymax / 2688.0)
    ms = graph_time(torch, [lambda: nv.gemm_nvfp4_rtn(outs["qX"], outs["qW"], qy.tensor_scale, amax_out=ymax,
                                                      out=qy)], min_calls=2)
    res["gemm_Y_nvfp4_out"] = _g_entry(2.0 * Mq * Nq * Kq, ms, "Y = X W^T written as NVFP4 (RTN along N with a "
                                       "given tensor scale, max |Y| out) by the GEMM itself instead of bf16", 1)
    del qy
    # IF4 forward operands (the output buffers of the step are reused), then
    # the Y GEMM on them through the INT-flag-aware entry point
    qa = nv.quantize_if4(X, out=outs["qX"], workspace=wss["qX"])
    qb = nv.quantize_if4(W, out=outs["qW"], workspace=wss["qW"])
    Yb = torch.empty((Mq, Nq), dtype=torch.bfloat16, device=dev)
    ms = graph_time(torch, [lambda: nv.gemm_nvfp4(qa, qb, out=Yb)], min_calls=2)
    res["gemm_Y_if4"] = _g_entry(2.0 * Mq * Nq * Kq, ms, "Y = X W^T, both operands IF4 (INT-flagged blocks "
                                 "decoded by table)", 1)
    del Yb
    for name, x in (("X_if4", X), ("W_if4", W)):
        ms, k = rotating_quant(nv, torch, x, lambda xi, q, w: nv.quantize_if4(xi, out=q, workspace=w))
        res[name] = _q_entry(x, ms, "IF4 (FP4/INT4 per 16-group), axis 0", k)
    for rule, what in (("4over6", "RTN, Four Over Six block scaling, axis 0"),
                       ("search", "RTN, block scale searched over 19 E4M3 bytes, axis 0")):
        for name, x in (("X_" + rule, X), ("W_" + rule, W)):
            ms, k = rotating_quant(nv, torch, x, lambda xi, q, w, r=rule: nv.quantize_nvfp4(
                xi, scale_rule=r, out=q, workspace=w))
            res[name] = _q_entry(x, ms, what, k)
    res.update(other_configs(nv, torch))
    return res


def small_config(nv, torch):
    """The 256 x 256 fp32 correctness case (N(0,1), seed 0), RTN and SR
    (seed 0, stream 0), no rotation: a latency case.  Per call: GPU time
    back to back in a HIP graph, and the median of 200 single calls timed
    with events around each (what one call costs on an idle stream)."""
    from nvfp4_bit_block_amd import synth
    dev = torch.device("cuda:0")
    x = torch.from_numpy(synth.gaussian(256, 256, seed=0)).to(dev)
    res = {}
    for rnd in ("rtn", "sr"):
        q, w = _qbuf(nv, torch, x, 0, rnd, dev)
        call = (lambda r=rnd, q=q, w=w: nv.quantize_nvfp4(x, rounding=r, seed=0, stream_id=0, out=q, workspace=w))
        ms_graph = graph_time(torch, [call], min_calls=100)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        single = []
        for _ in range(200):
            a.record()
            call()
            b.record()
            b.synchronize()
            single.append(a.elapsed_time(b))
        res["small_256_" + rnd] = {"us_per_call_graph": round(ms_graph * 1e3, 2),
                                   "us_single_call_median": round(float(np.median(single)) * 1e3, 2),
                                   "shape_in": [256, 256], "dtype_in": "fp32",
                                   "what": f"256x256 fp32 N(0,1), {rnd.upper()}, no rotation: maximum pass "
                                           "+ coding pass"}
    return res


def other_configs(nv, torch):
    """The other workloads of the method's configurations, each on its own
    seeded inputs (synth.py), rotating over copies so that no call finds
    its data in the memory-side cache: the 256x256 correctness case
    (latency), the 4096x4096 gradient (rows, rotation: SR, MS-EDEN, and IF4
    with SR and with MS-EDEN), the 8192x8192 weight (IF4, RTN) and the weight
    gradient of a Llama-like linear (dY, X 16384x4096 column-wise with
    rotation and MS-EDEN, then dW = dY^T X, fp32)."""
    from nvfp4_bit_block_amd import synth
    dev = torch.device("cuda:0")
    res = small_config(nv, torch)
    g, gs = synth.gradient(4096, 4096, seed=1)
    G = torch.from_numpy(g).to(dev).to(torch.bfloat16)
    for rnd in ("sr", "mseden"):
        ms, k = rotating_quant(nv, torch, G, lambda xi, q, w, r=rnd: nv.quantize_nvfp4(
            xi, rounding=r, rht_signs=gs, seed=1, out=q, workspace=w), rounding=rnd)
        res["gradient_4096_" + rnd] = _q_entry(G, ms, f"4096x4096 gradient (5 % outliers x10), RHT + {rnd}, rows",
                                               k)
        ms, k = rotating_quant(nv, torch, G, lambda xi, q, w, r=rnd: nv.quantize_if4(
            xi, rounding=r, rht_signs=gs, seed=1, out=q, workspace=w), rounding=rnd)
        res["gradient_4096_if4_" + rnd] = _q_entry(G, ms, f"4096x4096 gradient, RHT + IF4 with {rnd}, rows", k)
    del G
    Wt = torch.from_numpy(synth.weight(8192, 8192, seed=2)).to(dev).to(torch.bfloat16)
    ms, k = rotating_quant(nv, torch, Wt, lambda xi, q, w: nv.quantize_if4(xi, out=q, workspace=w))
    res["weight_8192_if4"] = _q_entry(Wt, ms, "8192x8192 Student-t weight, IF4 RTN, rows", k)
    del Wt
    dy, x, ws = synth.wgrad(16384, 4096, seed=3)
    dYw = torch.from_numpy(dy).to(dev).to(torch.bfloat16)
    Xw = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    for name, t in (("wgrad_dY_cols", dYw), ("wgrad_X_cols", Xw)):
        ms, k = rotating_quant(nv, torch, t, lambda xi, q, w: nv.quantize_nvfp4(
            xi, rounding="mseden", axis=1, rht_signs=ws, seed=3, out=q, workspace=w), axis=1, rounding="mseden")
        res[name] = _q_entry(t, ms, "16384x4096, RHT + MS-EDEN along the 16384 rows (weight gradient operand)", k)
    qd = nv.quantize_nvfp4(dYw, rounding="mseden", axis=1, rht_signs=ws, seed=3)
    qx = nv.quantize_nvfp4(Xw, rounding="mseden", axis=1, rht_signs=ws, seed=3)
    ops = qd.codes.numel() + qd.scales.numel() + qx.codes.numel() + qx.scales.numel()
    k = n_copies(ops + 4096 * 4096 * 4)
    pairs = [(qd, qx)] + [(nv.QTensor(qd.codes.clone(), qd.scales.clone(), qd.tensor_scale.clone()),
                           nv.QTensor(qx.codes.clone(), qx.scales.clone(), qx.tensor_scale.clone()))
                          for _ in range(k - 1)]
    outs = [torch.empty((4096, 4096), dtype=torch.float32, device=dev) for _ in range(k)]
    ms = graph_time(torch, [(lambda a=a, b=b, o=o: nv.gemm_nvfp4(a, b, out=o)) for (a, b), o in zip(pairs, outs)])
    res["wgrad_gemm_dW"] = _g_entry(2.0 * 4096 * 4096 * 16384, ms, "dW = dY^T X [4096 x 4096], K = 16384, fp32 "
                                    "out: 256 tiles, one per CU", k)
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(Xh, Wh, dYh, signs, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same step:
    the same six quantizations restricted to slices of the inputs (each
    slice quantized as its own tensor), on all of the host's threads and on
    one thread, each the median of 3 runs; and sampled dW outputs computed
    one by one.  A calibration pass sizes the slices so that the measured
    runs take about `budget_s` seconds in all."""
    import oracle
    from nvfp4_bit_block_amd import synth
    w = oracle.signs_words(signs)
    T, D = Xh.shape
    O = Wh.shape[0]

    def jobs(rows):
        """(label, array, rounding, axis, rotation) for a slice of `rows` rows
        of the token dimension (and proportionally of W)."""
        ro = max(128, min(O, rows * O // T) // 128 * 128)
        cols = max(128, min(D, rows // 4) // 128 * 128)
        return [
            (f"X[:{rows}] RTN", Xh[:rows], oracle.RTN, 0, False),
            (f"W[:{ro}] RTN", Wh[:ro], oracle.RTN, 0, False),
            (f"dY[:{rows}] MS-EDEN+RHT rows", dYh[:rows], oracle.MSEDEN, 0, True),
            (f"W[:, :{cols}] MS-EDEN+RHT cols", Wh[:, :cols], oracle.MSEDEN, 1, True),
            (f"dY[:{rows}] MS-EDEN+RHT cols", dYh[:rows], oracle.MSEDEN, 1, True),
            (f"X[:{rows}] MS-EDEN+RHT cols", Xh[:rows], oracle.MSEDEN, 1, True),
        ]

    def run(rows):
        t_q, b_q = 0.0, 0.0
        for _, x, rnd, axis, rot in jobs(rows):
            xb = synth.to_bf16_f32(x)
            t = time.perf_counter()
            oracle.quantize(xb, rounding=rnd, axis=axis, rht_on=rot, signs_w=w if rot else None, seed=1)
            t_q += time.perf_counter() - t
            b_q += xb.size * BYTES_PER_ELEM_BF16
        return t_q, b_q

    def measured(threads, share):
        """Median of 3 runs on a slice sized to `share` of the budget."""
        oracle.set_num_threads(threads)
        t_cal, _ = run(128)
        rows = int(128 * max(1.0, share * budget_s / 3 / max(t_cal, 1e-3)))
        rows = max(128, min(T, rows // 128 * 128))
        runs = [run(rows) for _ in range(3)]
        t_med = sorted(r[0] for r in runs)[1]
        b = runs[0][1]
        return {"GB/s": b / t_med / 1e9, "rows": rows, "elements": b / BYTES_PER_ELEM_BF16,
                "labels": "; ".join(j[0] for j in jobs(rows)), "seconds": [round(r[0], 3) for r in runs]}

    t_start = time.perf_counter()
    all_threads = oracle.num_threads()
    full = measured(all_threads, 0.5)
    one = measured(1, 0.5)
    oracle.set_num_threads(all_threads)
    # GEMM: sampled output entries of dW (K = T), one by one
    qa = oracle.quantize(synth.to_bf16_f32(dYh[:, :64]), rounding=oracle.MSEDEN, axis=1, rht_on=True,
                         signs_w=w)
    qb = oracle.quantize(synth.to_bf16_f32(Xh[:, :64]), rounding=oracle.MSEDEN, axis=1, rht_on=True,
                         signs_w=w)
    rng = np.random.default_rng(0)
    n_ent = 1024
    im, in_ = rng.integers(0, 64, n_ent), rng.integers(0, 64, n_ent)
    t = time.perf_counter()
    oracle.gemm_entries(qa, qb, im, in_)
    t_g = time.perf_counter() - t
    return {"value": round(full["GB/s"], 4), "unit": "GB/s", "cores": all_threads, "kind": "oracle",
            "sample": f"quantize {full['labels']} (bf16 inputs, {full['elements'] / 1e6:.1f} M elements), "
                      f"median of 3 runs on {all_threads} threads; gemm: {n_ent} dW entries one by one (K={T})",
            "runs_s": full["seconds"],
            "value_1thread": round(one["GB/s"], 4),
            "sample_1thread": f"quantize {one['labels']} ({one['elements'] / 1e6:.1f} M elements), median of "
                              f"3 runs on 1 thread",
            "runs_1thread_s": one["seconds"],
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(),
            "gemm_TFLOP/s": round(n_ent * 2.0 * T / t_g / 1e12, 6),
            "seconds": round(time.perf_counter() - t_start, 1)}


if __name__ == "__main__":
    main()
