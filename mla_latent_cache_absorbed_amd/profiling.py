"""Turn rocprofv3 counter output into per-launch HBM traffic figures.

rocprofv3's FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch, summed over
the L2 channels) are scaled by what the same counters read for a plain
device-to-device copy of known size, so that the figure is in real bytes.
The result goes to ``profiles/traffic.json``, keyed by kernel and workload
and stamped with a digest of the kernel's source: ``bench.py`` reports it as
``roofline.traffic`` only while the source is unchanged.

Usage (after one counter run each, see the --help text)::

    python -m mla_latent_cache_absorbed_amd.profiling \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --copy-bytes N --workload ds2_t4k --command "..."

A second mode records the MFMA and LDS counters of one run (rocprofv3's
derived metrics MfmaUtil, MfmaFlopsBF16, LdsUtil and LdsBankConflict, and
the raw counters behind them) in ``profiles/counters.json``::

    python -m mla_latent_cache_absorbed_amd.profiling counters \\
        --pmc DIR --workload ds2_t32k --command "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_cache_absorbed_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# MFMA-busy and LDS counters per kernel and workload (same keying)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")

# step name -> (substring of the device symbol, its source files)
KERNELS = {
    "q_absorb": ("q_absorb", ("q_absorb.hip",)),
    "split_attn": ("split_attn", ("split_attn.hip",)),
    "finish": ("finish_bf16", ("finish.hip",)),
    "combine": ("combine_general", ("combine.hip",)),
    "up_project": ("up_general", ("general.hip",)),
    "oproj": ("oproj_", ("oproj.hip",)),
    "prefill_attn": ("prefill_attn", ("prefill.hip",)),
    "kv_rebuild": ("kv_rebuild", ("prefill.hip",)),
    "rope_finish": ("rope_finish", ("rope_proj.hip",)),
    "rope_rows": ("rope_rows", ("rope_proj.hip",)),
}


def _code_only(text: str) -> str:
    """C++ source without comments and blank space (the kernel sources hold
    no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kernel: str) -> str:
    """Digest of the code that determines one kernel (its source and every
    shared header, comments and layout ignored)."""
    h = hashlib.sha256()
    headers = sorted(f for f in os.listdir(CSRC) if f.endswith(".h"))
    for f in list(KERNELS[kernel][1]) + headers:
        with open(os.path.join(CSRC, f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_means(path: str, counter: str) -> dict:
    """Mean value of one counter per kernel symbol over all its dispatches
    in a rocprofv3 --output-format csv directory (or file)."""
    files = [path] if os.path.isfile(path) else glob.glob(
        os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under %s" % path)
    vals = defaultdict(list)
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") == counter:
                    vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def all_counter_means(path: str) -> dict:
    """{kernel symbol: {counter: mean over its dispatches}} of every counter
    in a rocprofv3 --output-format csv directory (or file)."""
    files = [path] if os.path.isfile(path) else glob.glob(
        os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under %s" % path)
    vals = defaultdict(lambda: defaultdict(list))
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                vals[row["Kernel_Name"]][row["Counter_Name"]].append(float(row["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}


# derived metric (rocprofv3's name) -> key in counters.json and its scale
DERIVED = {
    "MfmaUtil": ("mfma_util", 0.01),          # percent -> fraction of SIMD cycles with the MFMA busy
    "MfmaFlopsBF16": ("mfma_flops_bf16", 1.0),
    "LdsUtil": ("lds_util", 0.01),            # percent -> fraction of CU cycles with LDS indexed work
    "LdsBankConflict": ("lds_bank_conflicts_per_access", 1.0),
}


def counters_main(argv):
    ap = argparse.ArgumentParser(prog="profiling counters",
                                 description="record MFMA / LDS counters of one rocprofv3 --pmc run")
    ap.add_argument("--pmc", required=True, action="append",
                    help="rocprofv3 --pmc output directory (repeat for several passes)")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", default="", help="the profiled command, recorded verbatim")
    ap.add_argument("--out", default=COUNTERS_FILE)
    args = ap.parse_args(argv)
    merged = defaultdict(dict)
    for d in args.pmc:
        for sym, cs in all_counter_means(d).items():
            merged[sym].update(cs)
    try:
        with open(args.out) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    # where a step name covers several kernels, the one with the most MFMA
    # FLOPs (the one that does the step's arithmetic) is recorded
    chosen = {}
    for sym, cs in merged.items():
        k = short_name(sym)
        if k is None:
            continue
        if k not in chosen or cs.get("MfmaFlopsBF16", 0.0) > merged[chosen[k]].get("MfmaFlopsBF16", 0.0):
            chosen[k] = sym
    for k, sym in chosen.items():
        cs = merged[sym]
        e = {"source_digest": source_digest(k), "symbol": sym, "command": args.command}
        for name, (key, scale) in DERIVED.items():
            if name in cs:
                e[key] = cs[name] * scale
        e["raw"] = {c: v for c, v in cs.items() if c not in DERIVED}
        table.setdefault(k, {})[args.workload] = e
        print("%-11s %-14s %s" % (k, args.workload, "  ".join(
            "%s %.4g" % (key, e[key]) for _, (key, _) in DERIVED.items() if key in e)))
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")


def short_name(symbol: str):
    for k, (needle, _) in KERNELS.items():
        if needle in symbol:
            return k
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--fetch", required=True, help="rocprofv3 output of the FETCH_SIZE run")
    ap.add_argument("--write", required=True, help="rocprofv3 output of the WRITE_SIZE run")
    ap.add_argument("--copy-fetch", required=True, help="FETCH_SIZE run of bench.py --copy-calibration")
    ap.add_argument("--copy-write", required=True, help="WRITE_SIZE run of bench.py --copy-calibration")
    ap.add_argument("--copy-bytes", type=int, required=True, help="bytes read (= written) per copy")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", default="", help="the profiled command, recorded verbatim")
    ap.add_argument("--out", default=TRAFFIC_FILE)
    args = ap.parse_args()

    cf = counter_means(args.copy_fetch, "FETCH_SIZE")
    cw = counter_means(args.copy_write, "WRITE_SIZE")
    copy_kernel = max(cf, key=cf.get)  # the copy dominates that run
    f_factor = args.copy_bytes / (cf[copy_kernel] * 1024.0)
    w_factor = args.copy_bytes / (cw[copy_kernel] * 1024.0)

    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    try:
        with open(args.out) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    # a step name may cover several kernels launched once per call each (the
    # output projection's partial and slice-sum kernels): their per-dispatch
    # means add up to the bytes of one call
    per_name = {}
    for sym in fetch:
        k = short_name(sym)
        if k is None or sym not in write:
            continue
        f0, w0, fr, wr = per_name.get(k, (0.0, 0.0, 0.0, 0.0))
        per_name[k] = (f0 + fetch[sym] * 1024.0 * f_factor, w0 + write[sym] * 1024.0 * w_factor,
                       fr + fetch[sym], wr + write[sym])
    for k, (fb, wb, fraw, wraw) in per_name.items():
        table.setdefault(k, {})[args.workload] = {
            "source_digest": source_digest(k),
            "bytes_per_launch": fb + wb,
            "fetch_bytes": fb,
            "write_bytes": wb,
            "fetch_kib_raw": fraw,
            "write_kib_raw": wraw,
            "copy_kernel": copy_kernel,
            "fetch_factor": f_factor,
            "write_factor": w_factor,
            "command": args.command,
        }
        print("%-11s %-10s fetch %10.3f MB  write %10.3f MB" % (k, args.workload, fb / 1e6, wb / 1e6))
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("copy kernel %s: fetch factor %.4f, write factor %.4f" % (copy_kernel, f_factor, w_factor))


if __name__ == "__main__":
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        counters_main(sys.argv[2:])
    else:
        main()
