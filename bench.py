#!/usr/bin/env python3
"""Bench of the Q4_K x q8_K decode mat-vec on one MI355X.

One step is one pass of the hot path over one token, shaped like an FFN pair:
quantize x (f32 [1, 4096]) to q8_K, up mat-vec (Q4_K 14336 x 4096), quantize
h to q8_K, down mat-vec (Q4_K 4096 x 14336). The activation quantizations are
inside the timed region. Weights are cold: every step reads the next copy of a
rotation pool of weight pairs larger than twice the 256 MB Infinity Cache plus
the L2s, so the bytes come from HBM.

Printed (one JSON line on stdout):
  value          weight bytes of a step (2 x 33,030,144) / step time, in GB/s
  roofline       for the metric's kernel (the 14336 x 4096 up mat-vec):
                 algorithmic bytes per launch / its mean duration (the median
                 of interleaved rounds of 500 back-to-back launches on the
                 step's stream, weights rotating, after WARM_MS of the same
                 launches), against the 8 TB/s HBM peak; beside it, its
                 weight rate against the 2 GiB streaming read (the 75% bar)
                 and against the streaming read of the same 33 MB;
                 traffic from the committed rocprofv3 counter summary when it
                 matches the current kernel source
  roofline_down  the same for the 4096 x 14336 down mat-vec
  configs        every workload config timed once on this machine: the tiny and
                 4096 x 4096 Q4_K mat-vecs, the IQ4_NL 4096 x 4096 and
                 128256 x 4096 mat-vecs, the 512-token prefill product, and
                 the streaming read's fixed-cost fit t = b + bytes / rate
  cpu_baseline   the oracle on the host's cores over whole FFN pairs
  stream_read    the streaming-read ceiling measured by the library's probe
"""

from __future__ import annotations

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

METRIC = "weight GB/s and % of HBM roofline, Q4_K×q8_K GEMV 14336×4096 batch 1"
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
UP = (14336, 4096)
DOWN = (4096, 14336)
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
COUNTERS_MD = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
CSRC = os.path.join(ROOT, "quantized_decode_mat_amd", "csrc")
BUILD_SCRIPT = os.path.join(ROOT, "quantized_decode_mat_amd", "build.py")
# Each counted kernel: the name rocprofv3 reports (a prefix), the launches of a
# --counters run, its algorithmic bytes per launch, and the sources its code
# comes from (the summary is void once any of them changes).
COUNTED = {
    "gemv_q4k_up_14336x4096": (
        "void xq::(anonymous namespace)::gemv_q4k_kernel<1, 1, 4, 2, true, false, false, false>", 20,
        33030144 + 5120 + 4 * 14336, ("gemv_q4k.hip", "q4k_row.h", "xq_device.h")),
    "gemv_q4k_down_4096x14336": (
        "void xq::(anonymous namespace)::gemv_q4k_kernel<1, 4, 8, 3, true, false, false, false>", 20,
        33030144 + 17920 + 4 * 4096, ("gemv_q4k.hip", "q4k_row.h", "xq_device.h")),
    "gemv_iq4nl_head_128256x4096": (
        "void xq::(anonymous namespace)::gemv_iq4nl_resident_kernel<2, false, 0>", 8,
        295501824 + 5120 + 4 * 128256, ("gemv_iq4nl.hip", "xq_device.h")),
    "gemm_q4k_512x14336x4096": (
        "void xq::(anonymous namespace)::gemm_q4k_kernel<64, false>", 4,
        33030144 + 512 * 16 * 320 + 4 * 512 * 14336, ("gemm_q4k.hip", "xq_device.h")),
}
HEADLINE = "gemv_q4k_up_14336x4096"
# The prefill product's MFMA pass: int8 MFMA work executed (in units of 512
# ops), MFMA busy cycles summed over SIMDs, and the active cycles of the run.
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
                 "GRBM_GUI_ACTIVE")
PREFILL = ("gemm_q4k_512x14336x4096", 2 * 512 * 14336 * 4096)
XCDS, SIMDS = 8, 256 * 4
INT8_OPS_PER_CYCLE = 2 * 16 * 16 * 64 / 16   # per SIMD


# Sustained work before every timed region. After an idle spell (host-side
# input generation, a synchronize) the device needs some tens of milliseconds
# of load before its clocks settle: measured on MI355X, 50-launch windows of
# the 128256 x 4096 IQ4_NL mat-vec fell from 80.6 to 47.5 us over the first
# ~50 ms after a 2 s idle. Timing from a cold start would measure the ramp.
WARM_MS = 250.0


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10000)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps before the timed ones; more untimed steps follow "
                        "until %.0f ms of sustained work have passed" % WARM_MS)
    p.add_argument("--pool-mb", type=int, default=1100,
                   help="size of the cold-weight rotation pool")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="lower bound of the oracle's timed host work")
    p.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    p.add_argument("--suite", action="store_true",
                   help="also time the other workloads; their lines go to stderr (and to "
                        "--suite-out when given)")
    p.add_argument("--suite-out", default=None,
                   help="file that receives the suite's lines, one JSON object per line")
    p.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    p.add_argument("--counters", action="store_true",
                   help="short run for rocprofv3 --pmc: 20 up and 20 down mat-vec launches over "
                        "the cold pool, 8 IQ4_NL 128256x4096 mat-vecs, 4 small-M products, then "
                        "5 device copies and 5 streaming reads of 64 MiB (the counters' "
                        "calibration), then exit")
    p.add_argument("--trace-summary", metavar="TRACE_DIR",
                   help="read the *_kernel_trace.csv of a rocprofv3 --kernel-trace run under "
                        "TRACE_DIR and print one JSON line per kernel (calls, mean/min/max us, "
                        "mean of the last 1000 launches), then exit (no GPU needed)")
    p.add_argument("--pmc-table", nargs="+", metavar="DIR",
                   help="print a markdown table of every counter in the rocprofv3 counter CSVs under "
                        "the DIRs, per counted kernel of a --counters run, then exit (no GPU needed)")
    p.add_argument("--counters-summary", nargs="+", metavar="DIR",
                   help="FETCH_DIR WRITE_DIR [MFMA_DIR]: read the rocprofv3 CSVs of the "
                        "--counters runs (FETCH_SIZE; WRITE_SIZE; optionally " +
                        " ".join(MFMA_COUNTERS) + "), write " + os.path.relpath(COUNTERS, ROOT) +
                        " and exit (no GPU needed)")
    return p.parse_args()


def sha_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def sources_sha(files):
    """Hash of a kernel's sources and of the build script that sets its
    compiler flags: either changes the machine code the counters measured."""
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, f) for f in files] + [BUILD_SCRIPT]:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name):
    """HBM bytes per launch of a counted kernel from the committed rocprofv3
    counter summary, or None when it is missing or was taken on another
    version of the kernel's sources."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)["kernels"][name]
    except (OSError, ValueError, KeyError):
        return None, "no counter summary"
    if c.get("sources_sha256_16") != sources_sha(COUNTED[name][3]):
        return None, "counter summary predates the current kernel source"
    return int(c["hbm_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def trace_summary(trace_dir):
    """Durations (End - Start, ns) from a rocprofv3 kernel trace, one line per
    kernel and grid size (so one kernel's launch shapes stay apart)."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                grid = "x".join(r.get(k, "?") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
                per.setdefault((r["Kernel_Name"], grid), []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    for (name, grid), v in sorted(per.items(), key=lambda kv: -len(kv[1])):
        v.sort()
        d = [x[1] / 1e3 for x in v]
        last = d[-1000:]
        print(json.dumps({"kernel": name, "grid": grid, "calls": len(d),
                          "mean_us": round(sum(d) / len(d), 3), "min_us": round(min(d), 3),
                          "max_us": round(max(d), 3),
                          "last1000_mean_us": round(sum(last) / len(last), 3)}))


def counters_summary(fetch_dir, write_dir, mfma_dir=None):
    """Per-kernel HBM bytes from the two --pmc runs of `bench.py --counters`.
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read
    for the run's five 64 MiB device copies (64 MiB read, 64 MiB written)."""
    import csv
    import glob

    def load(d, counter):
        out = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == counter:
                        out.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                    float(r["Counter_Value"])))
        return sorted(out)

    def calib(rows, known_kib):
        # The run's last five device copies are the 64 MiB calibration copies.
        cp = [v for (_, nm, v) in rows if "copyBuffer" in nm][-5:]
        assert len(cp) == 5 and max(cp) - min(cp) < 0.01 * max(cp), cp
        return known_kib / (sum(cp) / len(cp))

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    fcal, wcal = calib(fetch, 65536.0), calib(write, 65536.0)
    kernels = {}
    for name, (kname, n, alg, srcs) in COUNTED.items():
        fv = [v for (_, nm, v) in fetch if nm.startswith(kname)][-n:]
        wv = [v for (_, nm, v) in write if nm.startswith(kname)][-n:]
        assert len(fv) == n and len(wv) == n, "%s: %d/%d dispatches" % (name, len(fv), len(wv))
        fk, wk = sum(fv) / n, sum(wv) / n
        hbm = fk * 1024 * fcal + wk * 1024 * wcal
        kernels[name] = {"kernel": kname, "launches": n, "fetch_size_kib_per_launch": round(fk, 3),
                         "write_size_kib_per_launch": round(wk, 3),
                         "hbm_bytes_per_launch": int(round(hbm)), "alg_bytes_per_launch": alg,
                         "traffic_over_alg": round(hbm / alg, 4),
                         "sources_sha256_16": sources_sha(srcs)}
    out = {"fetch_calibration": round(fcal, 5), "write_calibration": round(wcal, 5),
           "kernels": kernels}
    if mfma_dir:
        name, alg_ops = PREFILL
        kname, n = COUNTED[name][0], COUNTED[name][1]
        raw = {}
        for cn in MFMA_COUNTERS:
            v = [val for (_, nm, val) in load(mfma_dir, cn) if nm.startswith(kname)][-n:]
            assert len(v) == n, "%s: %d dispatches of %s" % (cn, len(v), kname)
            raw[cn] = sum(v) / n
        kernels[name]["mfma"] = {
            "per_launch": {k: round(v, 1) for k, v in raw.items()},
            "int8_ops_executed": int(raw["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512),
            "executed_over_algorithmic": round(raw["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512 / alg_ops, 4),
            # GRBM_GUI_ACTIVE sums the eight XCDs' busy cycles; MFMA busy
            # cycles sum over the 1024 SIMDs (256 CUs x 4).
            "cycles_per_xcd": round(raw["GRBM_GUI_ACTIVE"] / XCDS, 1),
            # every MFMA (int8 and the f16 min term) over the SIMD cycles
            "mfma_busy_frac": round(raw["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                    (SIMDS * raw["GRBM_GUI_ACTIVE"] / XCDS), 4),
            # the int8 MFMA share, at 2048 int8 ops per cycle per SIMD
            # (v_mfma_i32_16x16x64_i8: 2 * 16 * 16 * 64 ops in 16 cycles)
            "int8_busy_frac": round(raw["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512 / INT8_OPS_PER_CYCLE /
                                    (SIMDS * raw["GRBM_GUI_ACTIVE"] / XCDS), 4),
            # algorithmic ops over the int8 capacity of the run
            "useful_int8_frac": round(alg_ops / INT8_OPS_PER_CYCLE /
                                      (SIMDS * raw["GRBM_GUI_ACTIVE"] / XCDS), 4),
            "sources_sha256_16": sources_sha(COUNTED[name][3]),
        }
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(COUNTERS_MD, "w") as f:
        f.write(counters_markdown(out))
    print(json.dumps(out, indent=1))


def counters_markdown(out):
    """profiles/hbm_traffic_counters.md, written from the same numbers as the
    JSON next to it."""
    ks = out["kernels"]
    lines = [
        "# HBM traffic and MFMA counters: mat-vecs, IQ4_NL head and small-M product (cold weights)",
        "",
        "Generated by `bench.py --counters-summary` from the rocprofv3 counter runs below, over the committed "
        "launch sequence of `bench.py --counters` (20 up and 20 down Q4_K mat-vecs over the 1.1 GB cold pool, 8 "
        "IQ4_NL 128256x4096 mat-vecs over four rotating copies, 4 small-M products 512x14336x4096, then 5 device "
        "copies and 5 streaming reads of 64 MiB). The same numbers are in "
        "`profiles/hbm_traffic_counters.json`, which `bench.py` reads for the roofline's `traffic`.",
        "",
        "```",
        "cd /tmp && TMPDIR=/tmp timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv \\",
        "    -d $OUT/pmc_1 -o pmc -- python3 $REPO/bench.py --counters --no-cpu",
        "cd /tmp && TMPDIR=/tmp timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv \\",
        "    -d $OUT/pmc_2 -o pmc -- python3 $REPO/bench.py --counters --no-cpu",
        "cd /tmp && TMPDIR=/tmp timeout -s KILL 120 rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) + " \\",
        "    --output-format csv -d $OUT/pmc_3 -o pmc -- python3 $REPO/bench.py --counters --no-cpu",
        "python3 $REPO/bench.py --counters-summary $OUT/pmc_1 $OUT/pmc_2 $OUT/pmc_3",
        "```",
        "",
        "Calibration against the plain device copy of known size (64 MiB read and 64 MiB written per copy): "
        "FETCH_SIZE x %.5f, WRITE_SIZE x %.5f." % (out["fetch_calibration"], out["write_calibration"]),
        "",
        "| kernel | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | calibrated HBM bytes | algorithmic bytes "
        "| ratio |",
        "|---|---|---|---|---|---|",
    ]
    for name, k in ks.items():
        lines.append("| %s `%s` | %.1f | %.1f | %d | %d | %.4f |" % (
            name, k["kernel"].split("::")[-1], k["fetch_size_kib_per_launch"],
            k["write_size_kib_per_launch"], k["hbm_bytes_per_launch"], k["alg_bytes_per_launch"],
            k["traffic_over_alg"]))
    lines += ["", "Algorithmic bytes: every weight byte, the q8_K activation and the f32 output once (the "
              "product: W once, the 512-token q8_K once, Y once). Where the ratio sits above 1: the Q4_K "
              "mat-vecs' lanes each load their block's 16-byte header (the cache serves the repeats); each "
              "of the IQ4_NL head's workgroups stages the q8_K row from L2, which the non-temporal weight "
              "stream evicts; the small-M product's weight tiles re-read the 2.6 MB of activations, and the "
              "token tiles of one weight tile re-read its stage when they do not share an L2 in time."]
    pre = ks.get(PREFILL[0], {}).get("mfma")
    if pre:
        pl = pre["per_launch"]
        lines += ["", "**MFMA pass (small-M product, per launch).** SQ_INSTS_VALU_MFMA_MOPS_I8 = %d (units of "
                  "512 ops): %d int8 ops executed, %.2fx the %d algorithmic ops (the two scale planes; the "
                  "min term runs on f16 MFMA and is not counted there). SQ_VALU_MFMA_BUSY_CYCLES = %d. "
                  "GRBM_GUI_ACTIVE = %d, the eight XCDs' busy cycles summed (%.0f per XCD). All MFMA busy "
                  "%.1f%% of the SIMD cycles; int8 MFMA busy %.1f%% (at 2048 int8 ops per cycle per SIMD); "
                  "algorithmic work %.1f%% of the int8 capacity of the run." % (
                      pl["SQ_INSTS_VALU_MFMA_MOPS_I8"], pre["int8_ops_executed"],
                      pre["executed_over_algorithmic"], PREFILL[1], pl["SQ_VALU_MFMA_BUSY_CYCLES"],
                      pl["GRBM_GUI_ACTIVE"], pre["cycles_per_xcd"], 100 * pre["mfma_busy_frac"],
                      100 * pre["int8_busy_frac"], 100 * pre["useful_int8_frac"])]
    lines += ["", "Each entry carries the sha256 (first 16 hex digits) of the sources its kernel is built "
              "from and of the build script that sets the compiler flags; `bench.py` reports "
              "`traffic: null` once they differ from the committed files.", ""]
    return "\n".join(lines)


def pmc_table(dirs):
    """A markdown table of every counter found in the rocprofv3 counter CSVs
    under `dirs`, per counted kernel: the counter's value per dispatch (summed
    over the CSV's rows for that dispatch), averaged over the kernel's last n
    dispatches of the `bench.py --counters` sequence; a counter collected in
    several runs is averaged over them."""
    import csv
    import glob
    found = {}
    for d in dirs:
        per = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    key = (r["Counter_Name"], int(r["Dispatch_Id"]), r["Kernel_Name"])
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for cn in {k[0] for k in per}:
            for name, spec in COUNTED.items():
                kname, n = spec[0], spec[1]
                v = sorted((disp, val) for (c, disp, kn), val in per.items()
                           if c == cn and kn.startswith(kname))[-n:]
                if len(v) == n:
                    found.setdefault((cn, name), []).append(sum(x for _, x in v) / n)
    names = list(COUNTED)
    rows = ["| counter | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for cn in sorted({c for c, _ in found}):
        vals = []
        for name in names:
            v = found.get((cn, name))
            vals.append("{:,.0f}".format(sum(v) / len(v)) if v else "-")
        rows.append("| `%s` | %s |" % (cn, " | ".join(vals)))
    print("\n".join(rows))


def main():
    args = parse()
    if args.counters_summary:
        if len(args.counters_summary) not in (2, 3):
            sys.exit("--counters-summary takes FETCH_DIR WRITE_DIR [MFMA_DIR]")
        counters_summary(*args.counters_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_table:
        pmc_table(args.pmc_table)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_decode_mat_amd as xq
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    # ---- inputs ----
    g = wl.rng(wl.SEEDS["ffn_up"])
    w_up = wl.q4k_weights(*UP, g)
    x = wl.activations(1, UP[1], g)
    w_dn = wl.q4k_weights(*DOWN, wl.rng(wl.SEEDS["ffn_down"]))
    pair_bytes = w_up.nbytes + w_dn.nbytes
    pool = max(2, (args.pool_mb * 1000 * 1000 + pair_bytes - 1) // pair_bytes)
    log("weights %d B per pair, pool of %d pairs (%.0f MB)" % (pair_bytes, pool,
                                                             pool * pair_bytes / 1e6))
    up0 = torch.from_numpy(w_up.reshape(-1)).to(dev)
    dn0 = torch.from_numpy(w_dn.reshape(-1)).to(dev)
    ups = [up0] + [up0.clone() for _ in range(pool - 1)]
    dns = [dn0] + [dn0.clone() for _ in range(pool - 1)]
    x_d = torch.from_numpy(x.reshape(-1)).to(dev)
    xq1 = torch.empty(xq.xq_q8k_bytes(1, UP[1]), dtype=torch.uint8, device=dev)
    h = torch.empty(UP[0], dtype=torch.float32, device=dev)
    xq2 = torch.empty(xq.xq_q8k_bytes(1, DOWN[1]), dtype=torch.uint8, device=dev)
    y = torch.empty(DOWN[0], dtype=torch.float32, device=dev)
    s = stream.cuda_stream

    L = xq.lib()  # direct C calls in the timed loops: no per-call Python checks

    def step(i, s=s):
        k = i % pool
        L.xq_quantize_q8k(xq1.data_ptr(), x_d.data_ptr(), 1, UP[1], s)
        L.xq_gemv_q4k(h.data_ptr(), ups[k].data_ptr(), xq1.data_ptr(), UP[0], UP[1], s)
        L.xq_quantize_q8k(xq2.data_ptr(), h.data_ptr(), 1, DOWN[1], s)
        L.xq_gemv_q4k(y.data_ptr(), dns[k].data_ptr(), xq2.data_ptr(), DOWN[0], DOWN[1], s)

    # One checked pass through the binding (raises on any refusal).
    xq.xq_quantize_q8k(xq1, x_d, 1, UP[1])
    xq.xq_gemv_q4k(h, ups[0], xq1, UP[0], UP[1])
    xq.xq_quantize_q8k(xq2, h, 1, DOWN[1])
    xq.xq_gemv_q4k(y, dns[0], xq2, DOWN[0], DOWN[1])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    # Kept for the CPU leg, which holds this pass against the oracle before
    # any rate is printed.
    first_pass = {"xq_x": xq1.cpu().numpy().copy(), "h": h.cpu().numpy().astype(np.float64),
                  "xq_h": xq2.cpu().numpy().copy(), "y": y.cpu().numpy().astype(np.float64)}

    if args.counters:
        counters_run(torch, xq, L, dev, stream, ups, dns, xq1, xq2, h, y, x_d, pool)
        return

    # ---- headline: K plain steps ----
    for i in range(args.warmup):
        step(i)
    tw = time.perf_counter()
    nxt = _warm(torch, step, args.warmup)
    warm_ms = (time.perf_counter() - tw) * 1e3
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(nxt + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    value = pair_bytes / (ms * 1e-3) / 1e9
    log("step %.3f us (host clock %.3f us), weight %.1f GB/s" % (ms * 1e3, wall / args.steps * 1e6,
                                                               value))

    # ---- the same step in three launches: the up mat-vec quantizes its own
    # output (xq_gemv_q4k_q8k, the fused tail), beside the plain figure.
    ws_tail = _workspace(torch, dev, xq.xq_gemv_q4k_q8k_workspace_bytes(UP[0]))

    def step_fused(i, s=s):
        k = i % pool
        L.xq_quantize_q8k(xq1.data_ptr(), x_d.data_ptr(), 1, UP[1], s)
        L.xq_gemv_q4k_q8k(h.data_ptr(), xq2.data_ptr(), ups[k].data_ptr(), xq1.data_ptr(), UP[0],
                          UP[1], ws_tail.data_ptr(), ws_tail.numel(), s)
        L.xq_gemv_q4k(y.data_ptr(), dns[k].data_ptr(), xq2.data_ptr(), DOWN[0], DOWN[1], s)

    fused_us = _time_loop(torch, stream, step_fused, args.steps)
    fused = {"us_per_step": round(fused_us, 3),
             "weight_GBps": round(pair_bytes / fused_us / 1e3, 1),
             "step": "quantize x, up mat-vec quantizing its own output, down mat-vec"}
    log("fused-tail step: %s" % fused)

    # ---- the same step replayed from a HIP graph (beside the plain figure,
    # never instead of it): one graph holds one pass over the weight pool.
    # Every replay is checked against the eager result first.
    graph = graph_step(torch, step, pool, y, stream)
    log("graph replay: %s" % graph)

    # ---- per-kernel durations: each kernel of the step launched back to back
    # n_k times on the step's stream (weights still rotating through the
    # pool), one HIP event pair around the loop; mean = elapsed / n_k. This is
    # what a kernel trace averages, launch gaps aside. Each loop follows
    # WARM_MS of the same launches.
    n_k = 1000
    calls = {
        "quantize_x": lambda k: L.xq_quantize_q8k(xq1.data_ptr(), x_d.data_ptr(), 1, UP[1], s),
        "gemv_up": lambda k: L.xq_gemv_q4k(h.data_ptr(), ups[k % pool].data_ptr(),
                                           xq1.data_ptr(), UP[0], UP[1], s),
        "quantize_h": lambda k: L.xq_quantize_q8k(xq2.data_ptr(), h.data_ptr(), 1, DOWN[1], s),
        "gemv_down": lambda k: L.xq_gemv_q4k(y.data_ptr(), dns[k % pool].data_ptr(),
                                             xq2.data_ptr(), DOWN[0], DOWN[1], s),
    }
    kern_us = {}
    for nm, call in calls.items():
        kern_us[nm] = _time_loop(torch, stream, call, n_k)
    log("kernel means (us): " + ", ".join("%s %.3f" % kv for kv in kern_us.items()))

    # ---- streaming-read ceiling ----
    def stream_read(nbytes, reps):
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        sink = torch.empty(xq.xq_bench_sink_words(nbytes), dtype=torch.int32, device=dev)
        xq.xq_bench_stream_read(buf, nbytes, sink)
        torch.cuda.synchronize()
        us = _time_loop(torch, stream, lambda k: L.xq_bench_stream_read(
            buf.data_ptr(), nbytes, sink.data_ptr(), s), reps)
        r = nbytes / us / 1e3
        del buf, sink
        return r

    stream_gbps = stream_read(2 << 30, 100)
    log("streaming read, 2 GiB: %.1f GB/s" % stream_gbps)
    # Like-for-like: the probe over the same rotation pool as the up mat-vec,
    # 33 MB per launch, so launch and ramp costs weigh the same; timed against
    # the up mat-vec in interleaved ABBA rounds, whose median round of the
    # mat-vec is also the roofline's launch duration.
    sink_s = torch.empty(xq.xq_bench_sink_words(w_up.nbytes), dtype=torch.int32, device=dev)
    kern_us["gemv_up"], us_small = _abba(torch, stream, calls["gemv_up"], lambda k: L.xq_bench_stream_read(
        ups[k % pool].data_ptr(), w_up.nbytes, sink_s.data_ptr(), s), 500)
    stream_small_gbps = w_up.nbytes / us_small / 1e3
    log("streaming read, 33 MB cold: %.3f us, %.1f GB/s" % (us_small, stream_small_gbps))

    # The down mat-vec (the step's longest kernel) the same way, over its own
    # pool, against the streaming read of its 33 MB.
    sink_d = torch.empty(xq.xq_bench_sink_words(w_dn.nbytes), dtype=torch.int32, device=dev)
    kern_us["gemv_down"], us_small_dn = _abba(torch, stream, calls["gemv_down"],
                                              lambda k: L.xq_bench_stream_read(
        dns[k % pool].data_ptr(), w_dn.nbytes, sink_d.data_ptr(), s), 500)
    log("down mat-vec %.3f us; streaming read of its 33 MB %.3f us" % (kern_us["gemv_down"],
                                                                      us_small_dn))
    # The quantize kernels' GPU time: 64 launches replayed from one HIP graph
    # (an eager loop of them measures the host's launch rate instead).
    quant_graph_us = {
        "quantize_x": _graph_us(torch, lambda sc: L.xq_quantize_q8k(
            xq1.data_ptr(), x_d.data_ptr(), 1, UP[1], sc)),
        "quantize_h": _graph_us(torch, lambda sc: L.xq_quantize_q8k(
            xq2.data_ptr(), h.data_ptr(), 1, DOWN[1], sc)),
    }
    log("quantize, graph-replayed: %s" % quant_graph_us)

    # ---- rooflines of the two mat-vecs (the metric's kernel is the up) ----
    def matvec_roofline(name, counted, alg_bytes, us, us_read_same, weight_bytes):
        achieved = alg_bytes / (us * 1e-6) / 1e9
        traffic, note = traffic_from_profile(counted)
        return {
            "bound": "hbm",
            "kernel": name,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_note": note,
            "alg_bytes_per_launch": alg_bytes,
            "mean_launch_us": round(us, 3),
            # the 75% bar: weight bytes per second against the 2 GiB
            # streaming read, and against the same-size read of the same pool
            "frac_of_stream_read": round(weight_bytes / us / 1e3 / stream_gbps, 4),
            "frac_of_stream_read_same_size": round(us_read_same / us, 4),
            "stream_read_same_size_us": round(us_read_same, 3),
        }

    up_alg_bytes = w_up.nbytes + xq.xq_q8k_bytes(1, UP[1]) + 4 * UP[0]
    dn_alg_bytes = w_dn.nbytes + xq.xq_q8k_bytes(1, DOWN[1]) + 4 * DOWN[0]
    roofline = matvec_roofline("gemv_q4k 14336x4096", HEADLINE, up_alg_bytes, kern_us["gemv_up"],
                               us_small, w_up.nbytes)
    roofline_down = matvec_roofline("gemv_q4k 4096x14336", "gemv_q4k_down_4096x14336",
                                    dn_alg_bytes, kern_us["gemv_down"], us_small_dn, w_dn.nbytes)

    # ---- every workload config, each timed once on this machine ----
    del sink_s, sink_d
    configs = config_block(args, torch, xq, wl, dev, stream, stream_gbps)

    # ---- CPU baseline: the oracle over whole FFN pairs ----
    cpu = cpu_all = None
    if not args.no_cpu:
        cpu, cpu_all = cpu_legs(args, x, w_up, w_dn, pair_bytes, first_pass)
        if not cpu["parity_gate"]["passed"]:
            log("parity gate FAILED: %s" % cpu["parity_gate"])
            sys.exit(1)
        log("cpu oracle: %s" % cpu)
        log("cpu oracle, all cores: %s" % cpu_all)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_ms": round(warm_ms, 1),
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "ffn_pair_q4k_batch1",
            "up": list(UP),
            "down": list(DOWN),
            "batch": 1,
            "weight_bytes_per_step": pair_bytes,
            "weights": "cold: rotation pool of %d pairs (%.0f MB)" % (pool,
                                                                    pool * pair_bytes / 1e6),
            "step": "quantize x, up mat-vec, quantize h, down mat-vec",
        },
        "roofline": roofline,
        "roofline_down": roofline_down,
        "cpu_baseline": cpu,
        "configs": configs,
        # mat-vecs: mean of back-to-back launches on the step's stream (GPU
        # time, launches overlap their gaps); quantize: GPU time per launch
        # replayed from a HIP graph, beside the eager loop's launch interval
        "kernels_us": {"gemv_up": round(kern_us["gemv_up"], 3),
                       "gemv_down": round(kern_us["gemv_down"], 3),
                       "quantize_x_graph": round(quant_graph_us["quantize_x"], 3),
                       "quantize_h_graph": round(quant_graph_us["quantize_h"], 3)},
        "launch_interval_us": {"quantize_x": round(kern_us["quantize_x"], 3),
                               "quantize_h": round(kern_us["quantize_h"], 3)},
        "stream_read_GBps": round(stream_gbps, 1),
        "stream_read_33MB_GBps": round(stream_small_gbps, 1),
        "frac_of_stream_read": round(value / stream_gbps, 4),
        "host_us_per_step": round(wall / args.steps * 1e6, 3),
        "graph_replay": graph,
        "fused_tail_step": fused,
    }
    if cpu_all is not None:
        line["cpu_baseline_all_cores"] = cpu_all

    if args.suite:
        del ups, dns
        torch.cuda.empty_cache()
        suite(args, torch, xq, wl, dev, stream, stream_gbps)

    out = json.dumps(line)
    print(out, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(out + "\n")


def graph_step(torch, step, pool, y, stream):
    """Capture `pool` consecutive steps into one HIP graph on a side stream,
    check three replays (with eager steps between them) against the eager
    output, then time 300 replays. Returns the per-step figure, or the reason
    there is none."""
    step(0)
    torch.cuda.synchronize()
    y_eager = y.clone()
    cs = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    s_main = stream.cuda_stream
    with torch.cuda.graph(gr, stream=cs, capture_error_mode="thread_local"):
        sc = torch.cuda.current_stream().cuda_stream
        for k in range(pool):
            step(k, sc)
    torch.cuda.synchronize()
    for r in range(3):
        y.zero_()
        gr.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, y_eager):
            return {"us_per_step": None, "note": "replay %d differs from the eager step" % r}
        step(r, s_main)
        torch.cuda.synchronize()
    us = _time_loop(torch, stream, lambda i: gr.replay(), 300) / pool
    return {"us_per_step": round(us, 3), "steps_per_replay": pool,
            "note": "replays checked equal to the eager step"}


def _parity_gate(o, x, w_up, w_dn, fp):
    """One step of the GPU (its first, checked pass) against the oracle on the
    same bytes: q8_K(x) and q8_K(h) bytes 0..291 of every block equal, h and
    y within 1e-5 of the sum of |terms| per output. The second quantization
    is the oracle's of the GPU's own h, as in the parity tests."""
    def q8k_equal(a, b):
        return bool(np.array_equal(a.reshape(-1, 320)[:, :292], b.reshape(-1, 320)[:, :292]))

    def within(got, ref, T):
        return bool(np.all(np.abs(got - ref) <= 1e-5 * T)) and not np.isnan(got).any()

    xq_x = o.quantize_q8k(x)
    h_ref, Th = o.gemv_q4k(w_up, xq_x, *UP)
    xq_h = o.quantize_q8k(fp["h"].astype(np.float32).reshape(1, -1))
    y_ref, Ty = o.gemv_q4k(w_dn, xq_h, *DOWN)
    checks = {"q8k_x_bytes": q8k_equal(fp["xq_x"], xq_x), "h": within(fp["h"], h_ref, Th),
              "q8k_h_bytes": q8k_equal(fp["xq_h"], xq_h), "y": within(fp["y"], y_ref, Ty)}
    return {"passed": all(checks.values()), **checks,
            "checked": "one step (pool pair 0): q8_K bytes equal, h and y within 1e-5 T"}


def cpu_legs(args, x, w_up, w_dn, pair_bytes, first_pass):
    """The oracle, as it stands, over whole FFN pairs: single-threaded, then
    row-split over the host's cores (the same C calls on row lists, one per
    thread; ctypes drops the GIL for the call). Each leg is the median of
    three rounds that together take about args.cpu_seconds. Before the
    timing, the GPU's first step is held against the oracle (_parity_gate)."""
    import concurrent.futures as cf
    import oracle
    o = oracle.default()
    gate = _parity_gate(o, x, w_up, w_dn, first_pass)
    cores = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "16")), 16)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def pair_1():
        xq_h = o.quantize_q8k(x)
        hh, _ = o.gemv_q4k(w_up, xq_h, *UP)
        xq_h2 = o.quantize_q8k(hh.astype(np.float32).reshape(1, -1))
        o.gemv_q4k(w_dn, xq_h2, *DOWN)

    pool = cf.ThreadPoolExecutor(max_workers=cores)
    up_parts = np.array_split(np.arange(UP[0]), cores)
    dn_parts = np.array_split(np.arange(DOWN[0]), cores)

    def split_gemv(w, xq_b, shape, parts):
        outs = list(pool.map(lambda r: o.gemv_q4k(w, xq_b, *shape, rows=r)[0], parts))
        return np.concatenate(outs)

    def pair_n():
        xq_h = o.quantize_q8k(x)
        hh = split_gemv(w_up, xq_h, UP, up_parts)
        xq_h2 = o.quantize_q8k(hh.astype(np.float32).reshape(1, -1))
        split_gemv(w_dn, xq_h2, DOWN, dn_parts)

    def leg(fn, seconds):
        rates, total = [], 0
        for _ in range(3):
            reps, t0 = 0, time.perf_counter()
            while True:
                fn()
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds / 3:
                    break
            rates.append(reps * pair_bytes / el / 1e9)
            total += reps
        return sorted(rates)[1], rates, total

    v1, r1, n1 = leg(pair_1, args.cpu_seconds)
    vn, rn, nn = leg(pair_n, args.cpu_seconds / 2)
    pool.shutdown()
    sample = ("whole FFN pairs (quantize, up 14336x4096, quantize, down 4096x14336) on the "
              "plain C oracle; median of 3 rounds")
    one = {"value": round(v1, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "%d %s, single-threaded, %.0f s" % (n1, sample, args.cpu_seconds),
           "rounds_GBps": [round(r, 4) for r in r1], "cpu": model, "parity_gate": gate}
    alln = {"value": round(vn, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d %s, rows split over %d threads, %.0f s" % (
                nn, sample, cores, args.cpu_seconds / 2),
            "rounds_GBps": [round(r, 4) for r in rn], "cpu": model}
    return one, alln


def counters_run(torch, xq, L, dev, stream, ups, dns, xq1, xq2, h, y, x_d, pool):
    """Launch sequence profiled by the rocprofv3 --pmc runs: up x20, down x20
    (cold pool), IQ4_NL 128256x4096 x8 (four rotating copies), small-M
    product 512x14336x4096 x4 (rotating through the up pool), then copy x5
    and stream read x5 of 64 MiB."""
    import workloads as wl
    s = stream.cuda_stream
    L.xq_quantize_q8k(xq1.data_ptr(), x_d.data_ptr(), 1, UP[1], s)
    L.xq_quantize_q8k(xq2.data_ptr(), h.data_ptr(), 1, DOWN[1], s)
    torch.cuda.synchronize()
    for i in range(20):
        L.xq_gemv_q4k(h.data_ptr(), ups[(i + 3) % pool].data_ptr(), xq1.data_ptr(), UP[0], UP[1], s)
    for i in range(20):
        L.xq_gemv_q4k(y.data_ptr(), dns[(i + 7) % pool].data_ptr(), xq2.data_ptr(), DOWN[0],
                      DOWN[1], s)
    torch.cuda.synchronize()
    N, K = 128256, 4096
    g = wl.rng(wl.SEEDS["iq4nl_head"])
    w = torch.from_numpy(wl.iq4nl_weights(N, K, g).reshape(-1)).to(dev)
    ws = [w] + [w.clone() for _ in range(3)]
    xh = torch.from_numpy(wl.activations(1, K, g).reshape(-1)).to(dev)
    xqh = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
    L.xq_quantize_q8k(xqh.data_ptr(), xh.data_ptr(), 1, K, s)
    yh = torch.empty(N, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for i in range(8):
        L.xq_gemv_iq4nl(yh.data_ptr(), ws[i % 4].data_ptr(), xqh.data_ptr(), N, K, s)
    torch.cuda.synchronize()
    del ws, w
    M = 512
    xm = torch.from_numpy(wl.activations(M, UP[1], wl.rng(wl.SEEDS["prefill"])).reshape(-1)).to(dev)
    xqm = torch.empty(xq.xq_q8k_bytes(M, UP[1]), dtype=torch.uint8, device=dev)
    L.xq_quantize_q8k(xqm.data_ptr(), xm.data_ptr(), M, UP[1], s)
    ym = torch.empty(M * UP[0], dtype=torch.float32, device=dev)
    wsm = _workspace(torch, dev, xq.xq_gemm_q4k_small_m_workspace_bytes(M, UP[0], UP[1]))
    torch.cuda.synchronize()
    for i in range(4):
        L.xq_gemm_q4k_small_m(ym.data_ptr(), ups[(i + 11) % pool].data_ptr(), xqm.data_ptr(), M,
                              UP[0], UP[1], wsm.data_ptr(), wsm.numel(), s)
    torch.cuda.synchronize()
    n = 64 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    c = torch.empty_like(a)
    sink = torch.empty(xq.xq_bench_sink_words(n), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    for _ in range(5):
        c.copy_(a)
    for _ in range(5):
        L.xq_bench_stream_read(a.data_ptr(), n, sink.data_ptr(), s)
    torch.cuda.synchronize()
    log("counters run done")


def _graph_us(torch, launch, n=64, reps=30):
    """GPU time per launch: n launches of launch(stream_handle) captured in
    one HIP graph on a side stream, replayed reps times after one checked
    replay (one event pair around the replays)."""
    launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs, capture_error_mode="thread_local"):
        sc = torch.cuda.current_stream().cuda_stream
        for _ in range(n):
            launch(sc)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * n) * 1e3


def _matvec_entry(torch, xq, L, dev, stream, stream_gbps, call, pool, wbytes, alg_bytes, n):
    """A mat-vec timed over its rotating weight pool against the streaming
    read of the same bytes over the same pool, in interleaved ABBA rounds
    (medians): us per launch, weight GB/s, the algorithmic-bytes roofline
    fraction of 8 TB/s, and its fractions of the 2 GiB and the same-size
    streaming reads."""
    s = stream.cuda_stream
    sink = torch.empty(xq.xq_bench_sink_words(wbytes), dtype=torch.int32, device=dev)
    us, sus = _abba(torch, stream, call, lambda i: L.xq_bench_stream_read(
        pool[i % len(pool)].data_ptr(), wbytes, sink.data_ptr(), s), n)
    return {"us": round(us, 3), "weight_GBps": round(wbytes / us / 1e3, 1),
            "alg_GBps": round(alg_bytes / us / 1e3, 1),
            "frac_of_8TBps": round(alg_bytes / us / 1e3 / HBM_PEAK_GBPS, 4),
            "frac_of_stream_read": round(wbytes / us / 1e3 / stream_gbps, 4),
            "stream_read_same_size_us": round(sus, 3),
            "frac_of_stream_read_same_size": round(sus / us, 4)}


def _stream_fit(torch, xq, L, dev, stream, pool_mb):
    """The streaming read over sizes, each cold (windows rotating through a
    pool past the caches), and the fit t = b + bytes / rate that splits a
    launch's fixed cost from the rate ("25 — Writing XPU Kernels", section
    25.2: a bytes-per-second figure hides a fixed cost)."""
    s = stream.cuda_stream
    pool_bytes = (pool_mb * 1000 * 1000) // 4096 * 4096
    big = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    big.fill_(1)
    pts = []
    for sz, n in ((9437184, 1000), (33030144, 1000), (132120576, 300), (295501824, 100),
                  (1 << 30, 30)):
        nwin = max(1, pool_bytes // sz)
        sink = torch.empty(xq.xq_bench_sink_words(sz), dtype=torch.int32, device=dev)
        us = _time_loop(torch, stream, lambda i: L.xq_bench_stream_read(
            big.data_ptr() + (i % nwin) * sz, sz, sink.data_ptr(), s), n)
        pts.append((sz, us))
    del big
    torch.cuda.empty_cache()
    A = np.array([[1.0, b] for b, _ in pts])
    coef, *_ = np.linalg.lstsq(A, np.array([u for _, u in pts]), rcond=None)
    return {"points": [{"bytes": b, "us": round(u, 3), "GBps": round(b / u / 1e3, 1)}
                       for b, u in pts],
            "fit_fixed_us": round(float(coef[0]), 3),
            "fit_rate_GBps": round(1e-3 / float(coef[1]), 1),
            "windows": "rotating over %d MB" % (pool_bytes // 1000000)}


def config_block(args, torch, xq, wl, dev, stream, stream_gbps):
    """Every workload config on this machine, compactly: the tiny Q4_K mat-vec
    (launch-bound, us only), the 4096x4096 Q4_K mat-vec, the IQ4_NL 4096x4096
    and 128256x4096 mat-vecs (each against the 8 TB/s peak and the streaming
    reads), the 512-token prefill product (TOPS against the int8 peak), and
    the streaming read's fixed-cost fit. Weights are cold (rotating pools);
    the FFN pair itself is the headline and its two rooflines."""
    L = xq.lib()
    s = stream.cuda_stream
    out = {}
    t0 = time.perf_counter()

    def q4k_case(N, K, seed):
        g = wl.rng(seed)
        w = torch.from_numpy(wl.q4k_weights(N, K, g).reshape(-1)).to(dev)
        xv = torch.from_numpy(wl.activations(1, K, g).reshape(-1)).to(dev)
        return w, xv

    # c0: 256 x 1024, 147 KB of weights: launch-bound, no roofline claim.
    N, K = 256, 1024
    w, xv = q4k_case(N, K, wl.SEEDS["q4k_tiny"])
    xqb = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
    xq.xq_quantize_q8k(xqb, xv, 1, K)
    pool = _pool_copies(w, 64)
    yy = torch.empty(N, dtype=torch.float32, device=dev)
    us = _time_loop(torch, stream, lambda i: L.xq_gemv_q4k(
        yy.data_ptr(), pool[i % len(pool)].data_ptr(), xqb.data_ptr(), N, K, s), 2000)
    out["c0_q4k_256x1024"] = {"us": round(us, 3), "bound": "launch"}
    del pool, w

    # c1: 4096 x 4096 Q4_K.
    N, K = 4096, 4096
    w, xv = q4k_case(N, K, wl.SEEDS["q4k_4096"])
    xqb = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
    xq.xq_quantize_q8k(xqb, xv, 1, K)
    pool = _pool_copies(w, args.pool_mb)
    yy = torch.empty(N, dtype=torch.float32, device=dev)
    out["c1_q4k_4096x4096"] = _matvec_entry(
        torch, xq, L, dev, stream, stream_gbps, lambda i: L.xq_gemv_q4k(
            yy.data_ptr(), pool[i % len(pool)].data_ptr(), xqb.data_ptr(), N, K, s),
        pool, w.numel(), w.numel() + xq.xq_q8k_bytes(1, K) + 4 * N, 1000)
    del pool, w
    torch.cuda.empty_cache()

    # c3: IQ4_NL 4096 x 4096 and the 128256 x 4096 head.
    for key, (N, K), seed, n in (("c3_iq4nl_4096x4096", (4096, 4096), wl.SEEDS["iq4nl_4096"], 1000),
                                 ("c3_iq4nl_128256x4096", (128256, 4096), wl.SEEDS["iq4nl_head"],
                                  100)):
        g = wl.rng(seed)
        w = torch.from_numpy(wl.iq4nl_weights(N, K, g).reshape(-1)).to(dev)
        xv = torch.from_numpy(wl.activations(1, K, g).reshape(-1)).to(dev)
        xqb = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
        xq.xq_quantize_q8k(xqb, xv, 1, K)
        pool = _pool_copies(w, args.pool_mb)
        yy = torch.empty(N, dtype=torch.float32, device=dev)
        out[key] = _matvec_entry(
            torch, xq, L, dev, stream, stream_gbps, lambda i: L.xq_gemv_iq4nl(
                yy.data_ptr(), pool[i % len(pool)].data_ptr(), xqb.data_ptr(), N, K, s),
            pool, w.numel(), w.numel() + xq.xq_q8k_bytes(1, K) + 4 * N, n)
        del pool, w
        torch.cuda.empty_cache()

    # c4: the 512-token prefill product on int8 MFMA.
    M, (N, K) = 512, UP
    g = wl.rng(wl.SEEDS["prefill"])
    w = torch.from_numpy(wl.q4k_weights(N, K, g).reshape(-1)).to(dev)
    xv = torch.from_numpy(wl.activations(M, K, g).reshape(-1)).to(dev)
    xqb = torch.empty(xq.xq_q8k_bytes(M, K), dtype=torch.uint8, device=dev)
    xq.xq_quantize_q8k(xqb, xv, M, K)
    yy = torch.empty(M * N, dtype=torch.float32, device=dev)
    pool = _pool_copies(w, args.pool_mb)
    wsp = _workspace(torch, dev, xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K))
    us = _time_loop(torch, stream, lambda i: L.xq_gemm_q4k_small_m(
        yy.data_ptr(), pool[i % len(pool)].data_ptr(), xqb.data_ptr(), M, N, K, wsp.data_ptr(),
        wsp.numel(), s), 200)
    ops = 2.0 * M * N * K
    out["c4_prefill_q4k_512x14336x4096"] = {
        "us": round(us, 3), "TOPS": round(ops / us / 1e6, 1),
        "frac_of_int8_peak": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4), "bound": "mfma"}
    del pool, w, yy
    torch.cuda.empty_cache()

    out["stream_read_fit"] = _stream_fit(torch, xq, L, dev, stream, args.pool_mb)
    log("configs (%.1f s): %s" % (time.perf_counter() - t0, json.dumps(out)))
    return out


def _workspace(torch, dev, nbytes):
    """A caller-owned workspace for the library, zeroed before first use (at
    least 256 bytes, so a call that needs none still gets a valid pointer)."""
    return torch.zeros(max(256, nbytes), dtype=torch.uint8, device=dev)


def _pool_copies(t, pool_mb):
    n = max(2, (pool_mb * 1000 * 1000 + t.numel() - 1) // t.numel())
    return [t] + [t.clone() for _ in range(n - 1)]


def _warm(torch, fn, start, ms=WARM_MS):
    """Call fn(start), fn(start + 1), ... until `ms` of wall time have passed
    (a synchronize every 32 calls keeps the queue short); return the next index."""
    i = start
    t0 = time.perf_counter()
    while True:
        for _ in range(32):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return i


def _abba(torch, stream, fa, fb, n, reps=2):
    """fa and fb in interleaved rounds A B B A (`reps` times) of n calls each,
    after one warm-up, so drift of clocks or temperature falls on both alike;
    the rounds run back to back (one event between rounds, one synchronize at
    the end). Returns the median round of each, in us per call."""
    i = _warm(torch, fa, 0)
    sides = [0, 1, 1, 0] * reps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sides) + 1)]
    ev[0].record(stream)
    for r, side in enumerate(sides):
        f = fb if side else fa
        for k in range(n):
            f(i + k)
        i += n
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    ta = [ev[r].elapsed_time(ev[r + 1]) / n * 1e3 for r, sd in enumerate(sides) if sd == 0]
    tb = [ev[r].elapsed_time(ev[r + 1]) / n * 1e3 for r, sd in enumerate(sides) if sd == 1]
    return float(np.median(ta)), float(np.median(tb))


def _time_loop(torch, stream, fn, n):
    warm = _warm(torch, fn, 0)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(warm + i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e3  # us


def suite(args, torch, xq, wl, dev, stream, stream_gbps):
    """The other workloads, each timed back to back with cold weights."""
    import oracle  # noqa: F401  (the suite reports no oracle figures)
    L = xq.lib()
    s = stream.cuda_stream
    lines = []

    def emit(d):
        d["stream_read_GBps"] = round(stream_gbps, 1)
        lines.append(d)
        log("suite: " + json.dumps(d))

    def matvec_line(name, ws, wb, call, n):
        """Time `call` over the rotating pool `ws` against the streaming read
        of the same wb bytes over the same pool (like for like: same launch and
        ramp costs), in interleaved ABBA rounds, and emit both."""
        sink = torch.empty(xq.xq_bench_sink_words(wb), dtype=torch.int32, device=dev)
        us, sus = _abba(torch, stream, call, lambda i: L.xq_bench_stream_read(
            ws[i % len(ws)].data_ptr(), wb, sink.data_ptr(), s), n)
        emit({"workload": name, "us": round(us, 3), "weight_GBps": round(wb / us / 1e3, 1),
              "frac_of_8TBps": round(wb / us / 1e3 / HBM_PEAK_GBPS, 4),
              "frac_of_stream_read": round(wb / us / 1e3 / stream_gbps, 4),
              "stream_read_same_size_us": round(sus, 3),
              "frac_of_stream_read_same_size": round(sus / us, 4)})

    # The streaming read itself over sizes, and its fixed-cost fit.
    emit({"workload": "stream_read_sizes", **_stream_fit(torch, xq, L, dev, stream, args.pool_mb)})
    pool_bytes = (args.pool_mb * 1000 * 1000) // 4096 * 4096
    big = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    big.fill_(1)
    # A plain device-to-device copy of up to 1 GiB (torch's copy_, read + write).
    cb = min(1 << 30, pool_bytes)
    dst = torch.empty(cb, dtype=torch.uint8, device=dev)
    us = _time_loop(torch, stream, lambda i: dst.copy_(big[:cb]), 30)
    emit({"workload": "copy_dtod", "bytes": cb, "us": round(us, 3),
          "read_plus_write_GBps": round(2 * cb / us / 1e3, 1)})
    del big, dst
    torch.cuda.empty_cache()

    # Q4_K mat-vecs alone: 4096x4096 and the two FFN shapes.
    for name, (N, K), seed in (("q4k_4096x4096", (4096, 4096), wl.SEEDS["q4k_4096"]),
                               ("q4k_up_14336x4096", UP, wl.SEEDS["ffn_up"]),
                               ("q4k_down_4096x14336", DOWN, wl.SEEDS["ffn_down"]),
                               ("q4k_tiny_256x1024", (256, 1024), wl.SEEDS["q4k_tiny"])):
        g = wl.rng(seed)
        w = torch.from_numpy(wl.q4k_weights(N, K, g).reshape(-1)).to(dev)
        xv = torch.from_numpy(wl.activations(1, K, g).reshape(-1)).to(dev)
        xqb = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
        xq.xq_quantize_q8k(xqb, xv, 1, K)
        ws = _pool_copies(w, args.pool_mb)
        yy = torch.empty(N, dtype=torch.float32, device=dev)
        matvec_line(name, ws, w.numel(), lambda i: L.xq_gemv_q4k(
            yy.data_ptr(), ws[i % len(ws)].data_ptr(), xqb.data_ptr(), N, K, s), 1000)
        del ws, w
        torch.cuda.empty_cache()

    # IQ4_NL mat-vecs.
    for name, (N, K), seed in (("iq4nl_4096x4096", (4096, 4096), wl.SEEDS["iq4nl_4096"]),
                               ("iq4nl_head_128256x4096", (128256, 4096),
                                wl.SEEDS["iq4nl_head"])):
        g = wl.rng(seed)
        w = torch.from_numpy(wl.iq4nl_weights(N, K, g).reshape(-1)).to(dev)
        xv = torch.from_numpy(wl.activations(1, K, g).reshape(-1)).to(dev)
        xqb = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
        xq.xq_quantize_q8k(xqb, xv, 1, K)
        ws = _pool_copies(w, args.pool_mb)
        yy = torch.empty(N, dtype=torch.float32, device=dev)
        n = 1000 if N < 100000 else 200
        matvec_line(name, ws, w.numel(), lambda i: L.xq_gemv_iq4nl(
            yy.data_ptr(), ws[i % len(ws)].data_ptr(), xqb.data_ptr(), N, K, s), n)
        del ws, w
        torch.cuda.empty_cache()

    # Q4_0 mat-vecs on the same row shape (the IQ4_NL twin).
    for name, (N, K), seed in (("q4_0_4096x4096", (4096, 4096), wl.SEEDS["iq4nl_4096"]),
                               ("q4_0_head_128256x4096", (128256, 4096), wl.SEEDS["iq4nl_head"])):
        g = wl.rng(seed)
        w = torch.from_numpy(wl.iq4nl_weights(N, K, g).reshape(-1)).to(dev)
        xv = torch.from_numpy(wl.activations(1, K, g).reshape(-1)).to(dev)
        xqb = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
        xq.xq_quantize_q8k(xqb, xv, 1, K)
        ws = _pool_copies(w, args.pool_mb)
        yy = torch.empty(N, dtype=torch.float32, device=dev)
        n = 1000 if N < 100000 else 200
        matvec_line(name, ws, w.numel(), lambda i: L.xq_gemv_q4_0(
            yy.data_ptr(), ws[i % len(ws)].data_ptr(), xqb.data_ptr(), N, K, s), n)
        del ws, w
        torch.cuda.empty_cache()

    # Expert-grouped mat-vecs: one launch over a bank of small experts against
    # the per-expert dense launches it replaces (the pages' grouped dispatch,
    # "25 — Writing XPU Kernels", section 25.2.2). Slabs rotate through the pool.
    E, rows, K, ids = 64, 1408, 2048, [3, 17, 25, 40, 41, 50, 58, 63]
    used = len(ids)
    for name, wfn, nbytes, grouped, dense in (
            ("q4k_id_E64_r1408_k2048_used8", wl.q4k_weights, xq.xq_q4k_bytes,
             L.xq_gemv_q4k_id, L.xq_gemv_q4k),
            ("iq4nl_id_E64_r1408_k2048_used8", wl.iq4nl_weights, xq.xq_iq4nl_bytes,
             L.xq_gemv_iq4nl_id, L.xq_gemv_iq4nl)):
        g = wl.rng(wl.SEEDS["grouped"])
        slab = torch.from_numpy(np.concatenate(
            [wfn(rows, K, g).reshape(rows, -1) for _ in range(E)], axis=0).reshape(-1)).to(dev)
        xv = torch.from_numpy(wl.activations(1, K, g).reshape(-1)).to(dev)
        xqb = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device=dev)
        xq.xq_quantize_q8k(xqb, xv, 1, K)
        sel = torch.tensor(ids, dtype=torch.int32, device=dev)
        slabs = _pool_copies(slab, args.pool_mb)
        yy = torch.empty(used * rows, dtype=torch.float32, device=dev)
        rb = nbytes(1, K)
        us = _time_loop(torch, stream, lambda i: grouped(
            yy.data_ptr(), slabs[i % len(slabs)].data_ptr(), xqb.data_ptr(), sel.data_ptr(),
            E, used, rows, K, 0, s), 1000)

        def dense_all(i):
            base = slabs[i % len(slabs)].data_ptr()
            for kk, e in enumerate(ids):
                dense(yy.data_ptr() + 4 * kk * rows, base + e * rows * rb, xqb.data_ptr(),
                      rows, K, s)

        dus = _time_loop(torch, stream, dense_all, 300)
        wb = used * rows * rb
        emit({"workload": name, "us": round(us, 3), "weight_GBps": round(wb / us / 1e3, 1),
              "frac_of_stream_read": round(wb / us / 1e3 / stream_gbps, 4),
              "dense_launches_us": round(dus, 3), "speedup_vs_dense": round(dus / us, 3)})
        del slabs, slab
        torch.cuda.empty_cache()

    # Bind-time repack of the head's IQ4_NL file blocks (18 B each) into
    # resident rows: bytes read + written per second.
    N, K = 128256, 4096
    bpr = K // 32
    blocks = torch.from_numpy(wl.iq4nl_file_blocks(N * bpr, wl.rng(wl.SEEDS["iq4nl_head"]))
                              .reshape(-1)).to(dev)
    res = torch.empty(N * xq.iq4nl_row_bytes(bpr), dtype=torch.uint8, device=dev)
    us = _time_loop(torch, stream, lambda i: L.xq_repack_iq4nl(
        res.data_ptr(), blocks.data_ptr(), N * bpr, 0, bpr, s), 100)
    moved = blocks.numel() + res.numel()
    emit({"workload": "repack_iq4nl_head_128256x4096", "us": round(us, 3),
          "read_plus_write_GBps": round(moved / us / 1e3, 1),
          "frac_of_stream_read": round(moved / us / 1e3 / stream_gbps, 4)})
    del blocks, res
    torch.cuda.empty_cache()

    # Small-M prefill product.
    M, (N, K) = 512, UP
    g = wl.rng(wl.SEEDS["prefill"])
    w = torch.from_numpy(wl.q4k_weights(N, K, g).reshape(-1)).to(dev)
    xv = torch.from_numpy(wl.activations(M, K, g).reshape(-1)).to(dev)
    xqb = torch.empty(xq.xq_q8k_bytes(M, K), dtype=torch.uint8, device=dev)
    qus = _time_loop(torch, stream, lambda i: L.xq_quantize_q8k(
        xqb.data_ptr(), xv.data_ptr(), M, K, s), 200)
    yy = torch.empty(M * N, dtype=torch.float32, device=dev)
    ws = _pool_copies(w, args.pool_mb)
    wsp = _workspace(torch, dev, xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K))
    us = _time_loop(torch, stream, lambda i: L.xq_gemm_q4k_small_m(
        yy.data_ptr(), ws[i % len(ws)].data_ptr(), xqb.data_ptr(), M, N, K, wsp.data_ptr(),
        wsp.numel(), s), 200)
    ops = 2.0 * M * N * K
    emit({"workload": "prefill_q4k_512x14336x4096", "us": round(us, 3),
          "TOPS": round(ops / us / 1e6, 1),
          "frac_of_int8_peak": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4),
          "quantize_512x4096_us": round(qus, 3)})
    del ws, w
    torch.cuda.empty_cache()

    # The same product at other token counts: 2 and 3 tokens on the up
    # matrix (the batched mat-vec on its persistent grid), 4 and 16 (the
    # wave-split MFMA tile); 2 and 3 tokens on the down matrix (the batched
    # mat-vec with the tokens' rows in LDS), 16 (the 16-token tile on its
    # three-stage ring: 256 workgroups), 64 (the 16-token tile, four token
    # tiles) and 512 (the 64-token tile); K is split over workgroups where the tile grid cannot fill the
    # device. 320 tokens on the up matrix: 512 of its 560 tiles whole, the
    # rest split four ways in the same launch.
    for M, (N, K), seed in ((2, UP, wl.SEEDS["prefill"]), (3, UP, wl.SEEDS["prefill"]),
                            (4, UP, wl.SEEDS["prefill"]), (16, UP, wl.SEEDS["prefill"]),
                            (2, DOWN, wl.SEEDS["ffn_down"]), (3, DOWN, wl.SEEDS["ffn_down"]),
                            (16, DOWN, wl.SEEDS["ffn_down"]),
                            (320, UP, wl.SEEDS["prefill"]),
                            (64, DOWN, wl.SEEDS["ffn_down"]), (512, DOWN, wl.SEEDS["ffn_down"])):
        g = wl.rng(seed)
        w = torch.from_numpy(wl.q4k_weights(N, K, g).reshape(-1)).to(dev)
        xv = torch.from_numpy(wl.activations(M, K, g).reshape(-1)).to(dev)
        xqb = torch.empty(xq.xq_q8k_bytes(M, K), dtype=torch.uint8, device=dev)
        xq.xq_quantize_q8k(xqb, xv, M, K)
        yy = torch.empty(M * N, dtype=torch.float32, device=dev)
        ws = _pool_copies(w, args.pool_mb)
        wsp = _workspace(torch, dev, xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K))
        us = _time_loop(torch, stream, lambda i: L.xq_gemm_q4k_small_m(
            yy.data_ptr(), ws[i % len(ws)].data_ptr(), xqb.data_ptr(), M, N, K, wsp.data_ptr(),
            wsp.numel(), s), 200)
        ops = 2.0 * M * N * K
        emit({"workload": "gemm_q4k_%dx%dx%d" % (M, N, K), "us": round(us, 3),
              "TOPS": round(ops / us / 1e6, 1),
              "frac_of_int8_peak": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4),
              "weight_GBps": round(w.numel() / us / 1e3, 1)})
        del ws, w
        torch.cuda.empty_cache()

    # Grouped product (mul_mat_id): 512 tokens routed top-8 over 64 experts of
    # 1408 x 2048, one routing launch plus one product launch, against one
    # dense product per expert over its pre-gathered token rows (the gather
    # is not timed).
    E, rows, K, T, U = 64, 1408, 2048, 512, 8
    g = wl.rng(wl.SEEDS["grouped"])
    slab_np = np.concatenate([wl.q4k_weights(rows, K, g).reshape(rows, -1) for _ in range(E)],
                             axis=0)
    slab = torch.from_numpy(slab_np.reshape(-1)).to(dev)
    xv = torch.from_numpy(wl.activations(T, K, g).reshape(-1)).to(dev)
    xqb = torch.empty(xq.xq_q8k_bytes(T, K), dtype=torch.uint8, device=dev)
    xq.xq_quantize_q8k(xqb, xv, T, K)
    ids_np = np.stack([g.choice(E, size=U, replace=False) for _ in range(T)]).astype(np.int32)
    ids = torch.from_numpy(ids_np).to(dev)
    slabs = _pool_copies(slab, args.pool_mb)
    yy = torch.empty(T * U * rows, dtype=torch.float32, device=dev)
    wsr = _workspace(torch, dev, xq.xq_gemm_q4k_id_workspace_bytes(T, U, E))
    us = _time_loop(torch, stream, lambda i: L.xq_gemm_q4k_id(
        yy.data_ptr(), slabs[i % len(slabs)].data_ptr(), xqb.data_ptr(), ids.data_ptr(), T, U, E,
        rows, K, 0, wsr.data_ptr(), wsr.numel(), s), 200)
    nb8, rb = xq.xq_q8k_bytes(1, K), xq.xq_q4k_bytes(rows, K)
    xr = xqb.view(T, nb8)
    per = []
    for e in range(E):
        toks = torch.from_numpy(np.nonzero((ids_np == e).any(axis=1))[0]).to(dev)
        if len(toks):
            per.append((e, len(toks), xr[toks].contiguous(),
                        torch.empty(len(toks) * rows, dtype=torch.float32, device=dev)))

    wse = _workspace(torch, dev, max(xq.xq_gemm_q4k_small_m_workspace_bytes(m, rows, K)
                                     for _, m, _, _ in per))

    def dense_all(i):
        base = slabs[i % len(slabs)].data_ptr()
        for e, m, xe, ye in per:
            L.xq_gemm_q4k_small_m(ye.data_ptr(), base + e * rb, xe.data_ptr(), m, rows, K,
                                  wse.data_ptr(), wse.numel(), s)

    dus = _time_loop(torch, stream, dense_all, 50)
    ops = 2.0 * T * U * rows * K
    emit({"workload": "gemm_q4k_id_T512_top8_E64_r1408_k2048", "us": round(us, 3),
          "TOPS": round(ops / us / 1e6, 1), "frac_of_int8_peak": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4),
          "dense_per_expert_us": round(dus, 3), "speedup_vs_dense": round(dus / us, 3)})
    del slabs, slab
    torch.cuda.empty_cache()

    if args.suite_out:
        with open(args.suite_out, "w") as f:
            for d in lines:
                f.write(json.dumps(d) + "\n")


if __name__ == "__main__":
    main()
