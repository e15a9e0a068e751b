"""Text summaries of rocprofv3 output for the library's kernels.

Two inputs are understood:

* ``--kernel-trace --stats -f csv`` output (``*_kernel_stats.csv``): per kernel
  calls, average and total duration;
* ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` runs (``*_counter_collection.csv``,
  one run per counter): HBM bytes per dispatch.  Both counters are in KiB per
  dispatch; each is divided by what the same counter reads, per byte, for a
  plain device-to-device copy of known size recorded in the same run (the
  largest ``copyBuffer`` dispatch), which calibrates it to bytes.

Usage (after copying the rocprofv3 output back):

  python -m matrix_optimizer_step_owner_amd.profiling stats KT_kernel_stats.csv \
      --command "<the profiled command>" --out profiles/<kernels>_<workload>.txt
  python -m matrix_optimizer_step_owner_amd.profiling traffic FETCH.csv WRITE.csv \
      --calib-mib 1024 --kernel update --workload block_d2048 \
      --command "<the profiled command>" --out profiles/update_kernel_block_d2048_traffic.json
  python -m matrix_optimizer_step_owner_amd.profiling counters PMC1.csv PMC2.csv \
      --calib-mib 1024 --command "<command 1>" --command "<command 2>" \
      --out profiles/counters_<workload>.txt

Any other ``--pmc`` counters in the files (GRBM_GUI_ACTIVE,
SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16, TCC_HIT_sum, ...) are
averaged per kernel kind by ``counters``.
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
from typing import Dict, List

PKG_DIR = os.path.dirname(os.path.abspath(__file__))

_NS_MODES = {"0": "gram", "1": "poly", "2": "update", "3": "final_wide", "4": "final_tall",
             "5": "syrk"}


#: HIP sources that compile into each kind of kernel (the device code whose
#: traffic a counter run measures)
_KERNEL_SOURCES = {"ns": ("common.hpp", "ns_gemm.hpp"),
                   "elementwise": ("common.hpp", "ew_kernels.hpp")}
_NS_KINDS = {"gram", "poly", "update", "final", "final_wide", "final_tall", "syrk"}


def kernel_source_hash(kind: str = "update") -> str:
    """sha256 over the HIP sources that define kernel kind ``kind`` (the NS
    product kernel for gram/poly/update/final/syrk, the elementwise kernels
    otherwise): it identifies the device code a traffic figure was taken on."""
    d = os.path.join(PKG_DIR, "csrc")
    h = hashlib.sha256()
    for name in _KERNEL_SOURCES["ns" if kind in _NS_KINDS else "elementwise"]:
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def short_name(kernel: str) -> str:
    """Library kernel kind of a demangled kernel name ('' for other kernels)."""
    m = re.search(r"ns_gemm_kernel<mfsdp::Elem(BF16|F32), (\d)>", kernel)
    if m:
        return _NS_MODES[m.group(2)] + ("" if m.group(1) == "BF16" else "_f32")
    for key, name in (("small_ns_kernel", "small"), ("momentum_kernel", "momentum"),
                      ("norm_finalize_kernel", "norm"),
                      ("adamw_kernel", "adamw"), ("apply_x0_kernel", "apply"),
                      ("mfma_probe_kernel", "mfma_loop")):
        if key in kernel:
            return name
    return ""


def kernel_stats(stats_csv: str) -> List[dict]:
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append({"kernel": r["Name"], "kind": short_name(r["Name"]),
                         "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3,
                         "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3,
                         "total_ms": float(r["TotalDurationNs"]) / 1e6,
                         "pct": float(r["Percentage"])})
    return rows


def format_stats(rows: List[dict], command: str) -> str:
    out = ["rocprofv3 --kernel-trace --stats summary", "", "command:", "  " + command, "",
           f"{'kind':12s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} "
           f"{'total ms':>10s} {'%':>6s}  kernel"]
    for r in rows:
        out.append(f"{r['kind'] or '-':12s} {r['calls']:6d} {r['avg_us']:10.2f} {r['min_us']:10.2f} "
                   f"{r['max_us']:10.2f} {r['total_ms']:10.3f} {r['pct']:6.2f}  {r['kernel'][:90]}")
    return "\n".join(out) + "\n"


def counter_by_dispatch(pmc_csv: str, counter: str) -> List[dict]:
    """Per dispatch: kernel name and the counter summed over its rows."""
    acc: Dict[int, dict] = collections.OrderedDict()
    with open(pmc_csv) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = acc.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"], "value": 0.0})
            d["value"] += float(r["Counter_Value"])
    return list(acc.values())


def traffic(fetch_csv: str, write_csv: str, calib_bytes: int, kind: str) -> dict:
    """Calibrated HBM bytes per launch of kernel kind ``kind``."""
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        ds = counter_by_dispatch(path, counter)
        copies = [d["value"] for d in ds if "copyBuffer" in d["kernel"]]
        if not copies:
            raise SystemExit(f"{path}: no copy dispatch to calibrate {counter}")
        factor = max(copies) * 1024.0 / calib_bytes
        vals = [d["value"] * 1024.0 / factor for d in ds if short_name(d["kernel"]) == kind]
        if not vals:
            raise SystemExit(f"{path}: no dispatch of kernel kind {kind!r}")
        res[counter] = {"factor": factor, "dispatches": len(vals),
                        "bytes_per_launch": sum(vals) / len(vals)}
    return res


#: XCDs (GRBM_GUI_ACTIVE is reported once per XCD) and SIMDs of an MI355X
N_XCD = 8
N_SIMD = 256 * 4
MIN_GRBM_US = 50.0


def counter_table(pmc_csvs: List[str], calib: Dict[str, float]) -> List[dict]:
    """Per kernel kind, the mean per dispatch of every counter in the files,
    the kernel duration and what follows from them: SCLK (GRBM_GUI_ACTIVE per
    XCD over the duration), MFMA busy % (busy SIMD-cycles over SIMD-cycles,
    rocprofv3's MfmaUtil), executed bf16 MFMA flops (MOPS x 512) and
    calibrated HBM bytes (FETCH_SIZE / WRITE_SIZE in KiB over ``calib``)."""
    per: Dict[int, dict] = collections.OrderedDict()
    for path in pmc_csvs:
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (path, int(r["Dispatch_Id"]))
                d = per.setdefault(key, {"kernel": r["Kernel_Name"], "c": {},
                                         "dur_ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
                d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    kinds: Dict[str, List[dict]] = collections.OrderedDict()
    for d in per.values():
        k = short_name(d["kernel"]) or ("copy" if "copyBuffer" in d["kernel"] else "")
        if k:
            kinds.setdefault(k, []).append(d)
    rows = []
    for k, ds in kinds.items():
        row = {"kind": k, "dispatches": len(ds), "avg_us": sum(d["dur_ns"] for d in ds) / len(ds) / 1e3}
        names = sorted({n for d in ds for n in d["c"]})
        for n in names:
            vals = [d["c"][n] for d in ds if n in d["c"]]
            row[n] = sum(vals) / len(vals)
        dur_s = row["avg_us"] * 1e-6
        # GRBM_GUI_ACTIVE spans the profiler's whole sampling window of a
        # dispatch (some microseconds beyond the kernel), so the derived clock
        # and busy fraction are only given for kernels of MIN_GRBM_US or more.
        if "GRBM_GUI_ACTIVE" in row and row["avg_us"] >= MIN_GRBM_US:
            cyc = row["GRBM_GUI_ACTIVE"] / N_XCD
            row["sclk_ghz"] = cyc / dur_s / 1e9
            if "SQ_VALU_MFMA_BUSY_CYCLES" in row:
                row["mfma_busy_pct"] = 100.0 * row["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in row and dur_s > 0:
            row["mfma_tflops"] = row["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / dur_s / 1e12
        if "TCC_HIT_sum" in row and "TCC_MISS_sum" in row:
            req = row["TCC_HIT_sum"] + row["TCC_MISS_sum"]
            if req > 0:
                row["l2_hit_pct"] = 100.0 * row["TCC_HIT_sum"] / req
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            if cn in row and cn in calib and dur_s > 0:
                row[cn.lower() + "_mb"] = row[cn] * 1024.0 / calib[cn] / 1e6
                row[cn.lower() + "_gbs"] = row[cn] * 1024.0 / calib[cn] / dur_s / 1e9
        rows.append(row)
    return rows


def calibration(pmc_csvs: List[str], calib_bytes: int) -> Dict[str, float]:
    """Counter units per byte of the largest plain copy dispatch in the files."""
    out = {}
    for path in pmc_csvs:
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            ds = counter_by_dispatch(path, cn)
            copies = [d["value"] for d in ds if "copyBuffer" in d["kernel"]]
            if copies:
                out[cn] = max(copies) * 1024.0 / calib_bytes
    return out


def format_counters(rows: List[dict], commands: List[str], calib: Dict[str, float]) -> str:
    out = ["rocprofv3 --pmc summary (means per dispatch)", "", "commands:"]
    out += ["  " + c for c in commands]
    out += ["", "calibration (counter KiB per byte of a plain copy): "
            + (", ".join(f"{k} {v:.3f}" for k, v in calib.items()) or "none"),
            "sclk = GRBM_GUI_ACTIVE per XCD / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /",
            f"(GRBM_GUI_ACTIVE per XCD x {N_SIMD} SIMDs).  GRBM_GUI_ACTIVE spans the profiler's",
            "dispatch window, some microseconds longer than the kernel, so both are given only",
            f"for kernels of {MIN_GRBM_US:.0f} us or more and overstate sclk (understate busy) by",
            "about that window over the duration.  L2 hit% = TCC_HIT_sum / (TCC_HIT_sum +",
            "TCC_MISS_sum), in requests.", "",
            f"{'kind':12s} {'disp':>5s} {'avg us':>9s} {'sclk GHz':>9s} {'MFMA busy%':>10s} "
            f"{'MFMA TF/s':>10s} {'fetch MB':>10s} {'write MB':>10s} {'HBM GB/s':>9s} {'L2 hit%':>8s}"]
    for r in rows:
        def f(key, fmt):
            return format(r[key], fmt) if key in r else "-"
        hbm = (r.get("fetch_size_gbs", 0.0) + r.get("write_size_gbs", 0.0)) or None
        out.append(f"{r['kind']:12s} {r['dispatches']:5d} {r['avg_us']:9.2f} {f('sclk_ghz', '9.2f'):>9s} "
                   f"{f('mfma_busy_pct', '10.1f'):>10s} {f('mfma_tflops', '10.1f'):>10s} "
                   f"{f('fetch_size_mb', '10.1f'):>10s} {f('write_size_mb', '10.1f'):>10s} "
                   f"{format(hbm, '9.0f') if hbm else '-':>9s} {f('l2_hit_pct', '8.1f'):>8s}")
    return "\n".join(out) + "\n"


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m matrix_optimizer_step_owner_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--calib-mib", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("pmc_csvs", nargs="+")
    c.add_argument("--calib-mib", type=int, default=0)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        cal = calibration(a.pmc_csvs, a.calib_mib << 20) if a.calib_mib else {}
        text = format_counters(counter_table(a.pmc_csvs, cal), a.command, cal)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
    elif a.cmd == "stats":
        text = format_stats(kernel_stats(a.stats_csv), a.command)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
    else:
        tr = traffic(a.fetch_csv, a.write_csv, a.calib_mib << 20, a.kernel)
        doc = {"kernel": a.kernel, "workload": a.workload,
               "bytes_per_launch": tr["FETCH_SIZE"]["bytes_per_launch"]
               + tr["WRITE_SIZE"]["bytes_per_launch"],
               "fetch_bytes_per_launch": tr["FETCH_SIZE"]["bytes_per_launch"],
               "write_bytes_per_launch": tr["WRITE_SIZE"]["bytes_per_launch"],
               "fetch_calibration_factor": tr["FETCH_SIZE"]["factor"],
               "write_calibration_factor": tr["WRITE_SIZE"]["factor"],
               "dispatches": tr["FETCH_SIZE"]["dispatches"],
               "source_sha256": kernel_source_hash(a.kernel),
               "command": a.command}
        with open(a.out, "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
        print(json.dumps(doc, indent=1))


if __name__ == "__main__":
    main()
