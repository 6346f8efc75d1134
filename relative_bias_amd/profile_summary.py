"""Summaries of rocprofv3 output for profiles/ (host-side text processing).

    python -m relative_bias_amd.profile_summary trace WORKLOAD DIR [--steps K]
    python -m relative_bias_amd.profile_summary traffic WORKLOAD FETCH_DIR WRITE_DIR FETCH_COPY_DIR WRITE_COPY_DIR
    python -m relative_bias_amd.profile_summary mfma WORKLOAD DIR
    python -m relative_bias_amd.profile_summary l2 WORKLOAD DIR

Each DIR is the -d directory of one rocprofv3 run of bench.py made with the
command the summary records (see COMMANDS below); they run committed files
only.  The summaries land in profiles/ as <kernel>_<workload>_{trace.md,
traffic.json, mfma.json, l2.json}, stamped with bench.kernel_hash() so that bench.py
uses a traffic figure only while the kernel source is unchanged.

trace: per kernel, the calls, the median duration and the mean of the last
K dispatches (bench.py times exactly K steps after its warm-up and clock
settle, so these are the timed, steady-state calls: K = --steps for the
batched decodes, max(5, steps // 2) for the others), with min and max over
all dispatches (the early ones run before the shader clock has ramped up).

traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, two runs) of the
dominant kernel, each scaled by what the same counter reads for a plain
1 GiB device copy (bench.py --copy-calibration), to HBM bytes per launch.

mfma: SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 and
GRBM_GUI_ACTIVE of the dominant kernel: MFMA pipe busy fraction and executed
MFMA flops against the algorithmic flops.

l2: TCC_HIT_sum, TCC_MISS_sum, TCC_READ_sum and TCC_REQ_sum (one run) of the
dominant kernel: L2 requests per launch and the fraction that hit, against
the kernel's algorithmic bytes in 128-byte lines.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")

# Dominant kernel of each bench workload (name prefix as rocprofv3 prints it).
DOMINANT = {
    "batched_decode": "decode_heads_kernel", "long_decode": "decode_heads_kernel",
    "batched_decode_fp8": "decode_heads_kernel", "long_decode_fp8": "decode_heads_kernel",
    "batched_decode_alibi": "decode_heads_kernel",
    "chunked_prefill": "attn_kernel", "chunked_prefill_fp8": "attn_kernel", "chunked_prefill_alibi": "attn_kernel",
    "chunked_prefill_relbf16": "attn_kernel", "continuous_batch": "attn_kernel", "kv_write": "kv_write_kernel",
}

# bench.py times --steps calls of the batched decodes and max(5, steps // 2)
# of every other workload.
FULL_STEPS = ("batched_decode", "batched_decode_fp8")


def timed_steps(wl: str, steps: int) -> int:
    return steps if wl in FULL_STEPS else max(5, steps // 2)


COMMANDS = {
    "trace": ("rocprofv3 --kernel-trace --stats --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/prof/{wl} "
              "-o {wl} -- python3 $GRAFT_REPO_ROOT/bench.py --only {wl} --steps {steps} --warmup 3 --no-cpu"),
    "pmc": ("rocprofv3 --pmc {c} --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/pmc/{c}_{wl} -o {wl} "
            "-- python3 $GRAFT_REPO_ROOT/bench.py --only {wl} --steps 3 --warmup 1 --no-cpu"),
    "copy": ("rocprofv3 --pmc {c} --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/pmc/{c}_copy -o copy "
             "-- python3 $GRAFT_REPO_ROOT/bench.py --copy-calibration"),
    "mfma": ("rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE "
             "--output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/mfma/{wl} -o {wl} -- python3 "
             "$GRAFT_REPO_ROOT/bench.py --only {wl} --steps 3 --warmup 1 --no-cpu"),
    "l2": ("rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum TCC_READ_sum TCC_REQ_sum --output-format csv "
           "-d $GRAFT_REPO_ROOT/gpurun_out/l2/{wl} -o {wl} -- python3 $GRAFT_REPO_ROOT/bench.py --only {wl} "
           "--steps 3 --warmup 1 --no-cpu"),
}

L2_COUNTERS = ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_READ_sum", "TCC_REQ_sum")


def _kernel_hash() -> str:
    sys.path.insert(0, ROOT)
    import bench
    return bench.kernel_hash()


def _short(name: str) -> str:
    return name.replace("rpa::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def _one(dir_: str, pattern: str) -> str:
    hits = glob.glob(os.path.join(dir_, "**", pattern), recursive=True)
    if len(hits) != 1:
        raise SystemExit(f"expected one {pattern} under {dir_}, found {len(hits)}")
    return hits[0]


def trace(wl: str, dir_: str, steps: int, out_dir: str = PROFILES) -> str:
    rows = list(csv.DictReader(open(_one(dir_, "*kernel_trace.csv"))))
    per = collections.OrderedDict()
    kt = timed_steps(wl, steps)
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        if "rpa::" not in r["Kernel_Name"]:
            continue
        per.setdefault(_short(r["Kernel_Name"]), []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = [f"# rocprofv3 kernel-trace summary: {wl}", "",
           "Command (on the MI355X box, from /tmp; `$GRAFT_REPO_ROOT` is the repository root):", "", "```",
           COMMANDS["trace"].format(wl=wl, steps=steps), "```", "",
           f"kernel source hash (bench.py kernel_hash): {_kernel_hash()}", "",
           f"`timed mean` is the mean of the last {kt} dispatches of each kernel (the calls bench.py times, "
           "after its warm-up and clock settle); min and max are over all dispatches.", "",
           "| kernel | calls | median ns | timed mean ns | min ns | max ns |", "|---|---|---|---|---|---|"]
    for k, d in per.items():
        tail = d[-kt:]
        out.append(f"| {k} | {len(d)} | {statistics.median(d):.0f} | {sum(tail) / len(tail):.0f} | {min(d)} | "
                   f"{max(d)} |")
    path = os.path.join(out_dir, f"{DOMINANT[wl]}_{wl}_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    return path


def _counter(dir_: str, counter: str, kernel_prefix: str):
    per = collections.defaultdict(float)
    name = None
    for r in csv.DictReader(open(_one(dir_, "*counter_collection.csv"))):
        if r["Counter_Name"] != counter or kernel_prefix not in r["Kernel_Name"]:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        name = r["Kernel_Name"]
    if not per:
        raise SystemExit(f"no {counter} samples of {kernel_prefix} under {dir_}")
    return name, list(per.values())


def traffic(wl: str, fetch_dir: str, write_dir: str, fetch_copy: str, write_copy: str, out_dir: str = PROFILES) -> str:
    nb = 1 << 30
    _, cf = _counter(fetch_copy, "FETCH_SIZE", "copyBuffer")
    _, cw = _counter(write_copy, "WRITE_SIZE", "copyBuffer")
    ff = nb / 1024 / statistics.median(cf)
    wf = nb / 1024 / statistics.median(cw)
    name, fv = _counter(fetch_dir, "FETCH_SIZE", DOMINANT[wl])
    _, wv = _counter(write_dir, "WRITE_SIZE", DOMINANT[wl])
    fk, wk = statistics.median(fv), statistics.median(wv)
    rd, wr = int(fk * 1024 * ff), int(wk * 1024 * wf)
    j = {"kernel": _short(name), "workload": wl, "kernel_hash": _kernel_hash(),
         "fetch_size_kib_per_dispatch": fk, "write_size_kib_per_dispatch": wk,
         "copy_calibration": {"bytes_each_way": nb, "fetch_size_kib": statistics.median(cf),
                              "write_size_kib": statistics.median(cw), "fetch_factor": round(ff, 4),
                              "write_factor": round(wf, 4)},
         "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr,
         "statistic": "median over dispatches",
         "commands": [COMMANDS["copy"].format(c="FETCH_SIZE"), COMMANDS["copy"].format(c="WRITE_SIZE"),
                      COMMANDS["pmc"].format(c="FETCH_SIZE", wl=wl), COMMANDS["pmc"].format(c="WRITE_SIZE", wl=wl)],
         "dispatches_sampled": [len(fv), len(wv)]}
    path = os.path.join(out_dir, f"{DOMINANT[wl]}_{wl}_traffic.json")
    with open(path, "w") as f:
        json.dump(j, f, indent=1)
    return path


def mfma(wl: str, dir_: str) -> str:
    sys.path.insert(0, ROOT)
    import torch
    from relative_bias_amd import metrics, workloads
    per = collections.defaultdict(dict)
    dur = {}
    name = None
    for r in csv.DictReader(open(_one(dir_, "*counter_collection.csv"))):
        if DOMINANT[wl] not in r["Kernel_Name"]:
            continue
        per[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
        dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        name = r["Kernel_Name"]
    keys = ("GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES")
    med = {k: statistics.median(d[k] for d in per.values()) for k in keys}
    dns = statistics.median(dur.values())
    make = workloads.continuous_batch if wl == "continuous_batch" else workloads.chunked_prefill
    w = make(device="cpu")
    if wl.endswith("relbf16"):
        w.rel_logits = w.rel_logits.to(torch.bfloat16)
    alg = metrics.work(w)["flops"]
    per_xcd = med["GRBM_GUI_ACTIVE"] / 8
    exe = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    t = {"kernel": _short(name), "workload": wl, "kernel_hash": _kernel_hash(), "dispatches_sampled": len(per),
         "statistic": "median over dispatches",
         "counters_per_dispatch": {k: int(round(v)) for k, v in med.items()},
         "dispatch_ns_under_counters": int(round(dns)), "mfma_flops_executed": int(exe), "algorithmic_flops": int(alg),
         "executed_over_algorithmic": round(exe / alg, 4), "gui_active_cycles_per_xcd": int(round(per_xcd)),
         "shader_clock_ghz": round(per_xcd / dns, 3),
         "mfma_busy_fraction": round(med["SQ_VALU_MFMA_BUSY_CYCLES"] / (per_xcd * 1024), 4),
         "notes": "GRBM_GUI_ACTIVE is read as the sum over the 8 XCDs (per-XCD = /8); MFMA busy = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (per-XCD active cycles x 1024 SIMDs), rocprofv3's MfmaUtil; executed "
                  "MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (includes masked and padded tile work)",
         "command": COMMANDS["mfma"].format(wl=wl)}
    path = os.path.join(PROFILES, f"attn_kernel_{wl}_mfma.json")
    with open(path, "w") as f:
        json.dump(t, f, indent=1)
    return path


def l2(wl: str, dir_: str, out_dir: str = PROFILES, algorithmic_bytes: int = None) -> str:
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    name = None
    for r in csv.DictReader(open(_one(dir_, "*counter_collection.csv"))):
        if DOMINANT[wl] not in r["Kernel_Name"] or r["Counter_Name"] not in L2_COUNTERS:
            continue
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        name = r["Kernel_Name"]
    if not per:
        raise SystemExit(f"no L2 counter samples of {DOMINANT[wl]} under {dir_}")
    med = {k: statistics.median(d[k] for d in per.values()) for k in L2_COUNTERS}
    if algorithmic_bytes is None:
        sys.path.insert(0, ROOT)
        from relative_bias_amd import metrics, workloads
        make = {"continuous_batch": workloads.continuous_batch, "batched_decode": workloads.batched_decode,
                "chunked_prefill": workloads.chunked_prefill}[wl]
        algorithmic_bytes = metrics.work(make(device="cpu"))["bytes"]
    hit, miss = med["TCC_HIT_sum"], med["TCC_MISS_sum"]
    t = {"kernel": _short(name), "workload": wl, "kernel_hash": _kernel_hash(), "dispatches_sampled": len(per),
         "statistic": "median over dispatches", "counters_per_dispatch": {k: int(round(v)) for k, v in med.items()},
         "hit_fraction": round(hit / (hit + miss), 4) if hit + miss else None,
         "algorithmic_bytes": int(algorithmic_bytes),
         "algorithmic_lines_128b": int(algorithmic_bytes // 128),
         "requests_per_algorithmic_line": round(med["TCC_REQ_sum"] / (algorithmic_bytes / 128), 3),
         "notes": "TCC_* are L2 (TCC) request counts summed over the channels of every XCD; a request is one "
                  "access of up to a 128-byte line, so requests per algorithmic 128-byte line counts how often "
                  "the kernel's data passes through L2 (re-reads by the q-tiles of a request included)",
         "command": COMMANDS["l2"].format(wl=wl)}
    path = os.path.join(out_dir, f"{DOMINANT[wl]}_{wl}_l2.json")
    with open(path, "w") as f:
        json.dump(t, f, indent=1)
    return path


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("kind", choices=("trace", "traffic", "mfma", "l2"))
    ap.add_argument("workload", choices=sorted(DOMINANT))
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--steps", type=int, default=20)
    a = ap.parse_args(argv)
    if a.kind == "trace":
        print(trace(a.workload, a.dirs[0], a.steps))
    elif a.kind == "traffic":
        if len(a.dirs) != 4:
            raise SystemExit("traffic needs FETCH_DIR WRITE_DIR FETCH_COPY_DIR WRITE_COPY_DIR")
        print(traffic(a.workload, *a.dirs))
    elif a.kind == "l2":
        print(l2(a.workload, a.dirs[0]))
    else:
        print(mfma(a.workload, a.dirs[0]))
    return 0


if __name__ == "__main__":
    sys.exit(main())
