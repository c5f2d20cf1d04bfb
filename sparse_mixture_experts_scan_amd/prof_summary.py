"""Summaries of rocprofv3 output for the MoE layer's kernels.

    python -m sparse_mixture_experts_scan_amd.prof_summary \\
        --workload decode --kt <dir> --fetch <dir> --write <dir> \\
        --command-kt "<cmd>" --command-pmc "<cmd>" --out profiles/<name>.md

<dir> are rocprofv3 ``-d`` output directories (``--output-format csv``):
``--kt`` from ``--kernel-trace --stats``, ``--fetch``/``--write`` from
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of ``bench.py
--copy-calibration-mib N``, and optionally ``--dram`` from a
``--pmc TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_WRITE_DRAM_32B_sum`` run: the
L2's read and write requests to memory in 32-byte units (a 64-byte request
counts 2, a 128-byte one 4), bytes by the counters' own definition, which
cross-checks the calibrated FETCH_SIZE / WRITE_SIZE figures.  That option runs, before the timed steps, a
plain elementwise kernel that reads N MiB and writes N MiB; what the two
counters read for it gives the scale factor from counter units to bytes,
applied to every other kernel.  The per-kernel traffic is also merged into
``profiles/traffic.json`` keyed by workload and kernel, with the SHA-256 of
the code text (comments and whitespace dropped) of the kernel's source
files, so a reader can tell when the numbers no longer describe the code."""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
KERNEL_SOURCES = {
    "gateup": {"stream": ["gemm_stream.hip", "common.h", "plan.h"],
               "tile": ["gemm_tile.hip", "common.h", "plan.h"],
               "q4": ["gemm_q4.hip", "common.h", "plan.h"]},
    "down": {"stream": ["gemm_stream.hip", "common.h", "plan.h"],
             "tile": ["gemm_tile.hip", "common.h", "plan.h"],
             "q4": ["gemm_q4.hip", "common.h", "plan.h"]},
}


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_text(src: str) -> str:
    """The source with its comments removed and whitespace collapsed: what
    decides the compiled kernel (the kernel sources hold no string literals
    that contain comment markers)."""
    return " ".join(_COMMENT.sub(" ", src).split())


def source_hash(files) -> str:
    """SHA-256 over the code text of `files`, so that a change to a comment
    does not mark the recorded counters as stale."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()


def kernel_key(name: str) -> str:
    """Short role of a kernel from its demangled name."""
    if "stream_gemm_kernel" in name:
        return "gateup" if ", true," in name else "down"
    if "stream_dma_kernel" in name:
        return "gateup" if ", true>" in name else "down"
    if "tile_gemm_kernel" in name:
        return "gateup" if "<true>" in name else "down"
    if "stream_q4_kernel" in name:
        return "gateup" if ", true," in name else "down"
    if "stream_q4_dma_kernel" in name:
        return "gateup" if ", true>" in name else "down"
    for k in ("quantize_int4", "dequant_int4", "rmsnorm"):
        if k in name:
            return k
    for k in ("router_topk", "router_select", "expert_scan", "scatter_gather", "combine"):
        if k in name:
            return k
    if "elementwise" in name:
        return "elementwise"
    if "copyBuffer" in name:
        return "copyBuffer"
    return name[:40]


def read_counter(d: str, counter: str = ""):
    """{kernel_key: [value per dispatch]} and the dispatches' kernel names;
    with `counter`, only that counter's rows of a multi-counter run."""
    path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    per = defaultdict(lambda: defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        if counter and r.get("Counter_Name") != counter:
            continue
        key = kernel_key(r["Kernel_Name"])
        per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    return {k: list(v.values()) for k, v in per.items()}, names


def calibration(values, cal_mib: int, kind: str) -> float:
    """Bytes per counter unit from the reference elementwise kernel.  Its
    dispatches are: torch.zeros of the count buffer (tiny), torch.ones of the
    N MiB source (writes N MiB), and the add (reads N MiB, writes N MiB)."""
    ref = sorted(values["elementwise"])
    known = cal_mib << 20
    if kind == "fetch":
        return known / ref[-1]                    # only the add reads N MiB
    return 2 * known / sum(ref)                    # ones + add write 2 N MiB


def read_stats(d: str):
    path = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0]
    return list(csv.DictReader(open(path)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--variant", choices=("stream", "tile", "q4"), required=True)
    ap.add_argument("--kt", required=True)
    ap.add_argument("--fetch", help="FETCH_SIZE run (omit with --write for a trace-only summary)")
    ap.add_argument("--write")
    ap.add_argument("--dram", help="TCC_EA0_RDREQ_DRAM_32B_sum / TCC_EA0_WRREQ_WRITE_DRAM_32B_sum "
                                   "run (a cross-check in 32-byte units)")
    ap.add_argument("--cal-mib", type=int, default=512)
    ap.add_argument("--command-kt", required=True)
    ap.add_argument("--command-pmc", default="",
                    help="counter-run command with <COUNTER> (the counters) and <DIR> (the "
                         "output directory suffix: FETCH_SIZE, WRITE_SIZE or DRAM)")
    ap.add_argument("--title", default="MoE layer")
    ap.add_argument("--algorithmic", default="{}",
                    help="JSON {kernel: algorithmic bytes per launch} for the table")
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(PKG), "profiles",
                                                           "traffic.json"))
    a = ap.parse_args()

    stats = read_stats(a.kt)
    alg = json.loads(a.algorithmic)

    lines = [f"# rocprofv3 summary: {a.title}, workload `{a.workload}`", "",
             "Kernel trace (`--kernel-trace --stats`):", "", "```", a.command_kt, "```", "",
             "| kernel | calls | avg us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    if not a.fetch or not a.write:
        with open(a.out, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {a.out} (kernel trace only)")
        return
    fetch, names = read_counter(a.fetch)
    write, _ = read_counter(a.write)
    cf = calibration(fetch, a.cal_mib, "fetch")
    cw = calibration(write, a.cal_mib, "write")
    dram_r = dram_w = None
    if a.dram:
        dram_r, _ = read_counter(a.dram, "TCC_EA0_RDREQ_DRAM_32B_sum")
        dram_w, _ = read_counter(a.dram, "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
    lines += ["", "HBM traffic per launch (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, "
              "one run each):", "", "```",
              a.command_pmc.replace("<COUNTER>", "FETCH_SIZE").replace("<DIR>", "FETCH_SIZE"),
              a.command_pmc.replace("<COUNTER>", "WRITE_SIZE").replace("<DIR>", "WRITE_SIZE"),
              "```", "",
              f"Scale from counter units to bytes, from the reference elementwise kernel "
              f"that reads {a.cal_mib} MiB and writes {a.cal_mib} MiB: FETCH_SIZE x {cf:.4g} "
              f"B/unit, WRITE_SIZE x {cw:.4g} B/unit.", ""]
    if a.dram:
        ref_r = sorted(dram_r["elementwise"])[-1] * 32
        ref_w = sum(dram_w["elementwise"]) * 32
        known = a.cal_mib << 20
        lines += ["Cross-check (`--pmc TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_WRITE_DRAM_32B_sum`"
                  ", one run; 32 bytes per unit by the counters' definition):", "", "```",
                  a.command_pmc.replace("<COUNTER>", "TCC_EA0_RDREQ_DRAM_32B_sum "
                                        "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
                  .replace("<DIR>", "DRAM"), "```", "",
                  f"On the reference kernel these read {ref_r / known:.3f} x and write "
                  f"{ref_w / (2 * known):.3f} x its known bytes.", ""]
    lines += ["| kernel | fetch GB | write GB | DRAM read GB | DRAM write GB | algorithmic GB "
              "| traffic / algorithmic |", "|---|---|---|---|---|---|---|"]
    record = {}
    for key in ("router_topk", "router_select", "expert_scan", "scatter_gather", "gateup",
                "down", "combine"):
        if key not in fetch:
            continue
        fb = sum(fetch[key]) / len(fetch[key]) * cf
        wb = sum(write.get(key, [0.0])) / max(1, len(write.get(key, [0.0]))) * cw
        dr = dw = None
        if a.dram and key in dram_r:
            dr = sum(dram_r[key]) / len(dram_r[key]) * 32
            dws = dram_w.get(key, [0.0])
            dw = sum(dws) / max(1, len(dws)) * 32
        al = alg.get(key)
        ratio = f"{(fb + wb) / al:.2f}" if al else "-"
        fmt = (lambda v: f"{v/1e9:.4f}" if v is not None else "-")
        lines.append(f"| {key} | {fb/1e9:.4f} | {wb/1e9:.4f} | {fmt(dr)} | {fmt(dw)} | "
                     f"{al/1e9 if al else float('nan'):.4f} | {ratio} |")
        if key in KERNEL_SOURCES:
            files = KERNEL_SOURCES[key][a.variant]
            record[key] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb,
                           "source_files": files, "source_sha256": source_hash(files),
                           "profile": os.path.basename(a.out)}
            if dr is not None:
                record[key].update(dram_read_bytes=dr, dram_write_bytes=dw)
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    try:
        with open(a.traffic_json) as fh:
            db = json.load(fh)
    except FileNotFoundError:
        db = {}
    db.setdefault(a.workload, {}).update(record)
    with open(a.traffic_json, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    print(f"wrote {a.out} and {a.traffic_json}")


if __name__ == "__main__":
    main()
