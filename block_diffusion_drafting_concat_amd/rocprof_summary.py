"""Summaries of rocprofv3 output for the committed profiles.

  kernel-stats:  python -m block_diffusion_drafting_concat_amd.rocprof_summary stats <run>_kernel_stats.csv
                 prints a markdown table of per-kernel calls and durations.
  pmc:           python -m block_diffusion_drafting_concat_amd.rocprof_summary pmc <workload> \
                     <fetch>_counter_collection.csv <write>_counter_collection.csv
                 prints the JSON read by bench.py: per GEMM instance, the HBM bytes per launch
                 from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the same
                 counter reads for the largest plain device copy in the run (bench.py
                 --copy-calib copies 1 GiB), so that bytes = counter * (copy bytes / copy reading).
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SOURCES = ("block_diffusion_drafting_concat_amd/csrc/gemm.hip", "block_diffusion_drafting_concat_amd/csrc/common.h")
EPI = {"0": "kStore", "1": "kResidAdd", "2": "kSwiGLU", "3": "kArgmax", "4": "kHeadNormRope", "5": "kKvScatter"}
COPY_BYTES = 1 << 30


def source_sha(paths=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """'gemm_kernel<unsigned short, 1, 8, 1, 1, 8, (dflash::GemmEpi)3, false, true>(...)' ->
    'gemm_kernel<bf16,MT=1,CW=8,CT=1,KW=1,NCG=8,kArgmax,fp32-A>'; the tiled and wide GEMMs
    likewise; other kernels: the name without arguments."""
    m = re.search(r"gemm_kernel<([^,]+), (\d+), (\d+), (\d+), (\d+), (\d+), \(dflash::GemmEpi\)(\d), "
                  r"(true|false), (true|false)>", name)
    if m:
        dt = "bf16" if "short" in m.group(1) else "f32"
        s = (f"gemm_kernel<{dt},MT={m.group(2)},CW={m.group(3)},CT={m.group(4)},KW={m.group(5)},"
             f"NCG={m.group(6)},{EPI[m.group(7)]}")
        s += ",multi-A" if m.group(8) == "true" else ""
        return s + (",fp32-A>" if m.group(9) == "true" else ">")
    m = re.search(r"gemm_tiled_kernel<\(dflash::GemmEpi\)(\d), (true|false), (\d+), (\d+)>", name)
    if m:
        return (f"gemm_tiled_kernel<{EPI[m.group(1)]},{'hi+lo-A' if m.group(2) == 'true' else 'bf16-A'},"
                f"{m.group(3)}x{m.group(4)}>")
    m = re.search(r"gemm_wide_kernel<\(dflash::GemmEpi\)(\d), (true|false), (true|false)>", name)
    if m:
        a_kind = "bf16-A-segments" if m.group(2) == "true" else "hi+lo-A" if m.group(3) == "true" else "bf16-A"
        return f"gemm_wide_kernel<{EPI[m.group(1)]},{a_kind},256x256>"
    if name.startswith("Cijk_"):  # a library GEMM kernel (bench.py's attainable-rate check)
        return "library bf16 GEMM (" + name.split("_MT")[1].split("_")[0] + " tiles)" if "_MT" in name else name[:40]
    name = re.sub(r"^void ", "", name)
    name = name.replace("dflash::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out)


def _counter(path: str, counter: str):
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def pmc(workload: str, fetch_csv: str, write_csv: str) -> dict:
    f = _counter(fetch_csv, "FETCH_SIZE")
    w = _counter(write_csv, "WRITE_SIZE")
    copies_f = [v for k, vs in f.items() if "copyBuffer" in k for v in vs]
    copies_w = [v for k, vs in w.items() if "copyBuffer" in k for v in vs]
    if not copies_f or not copies_w:
        raise SystemExit("no device copy found: run bench.py with --copy-calib")
    kib = COPY_BYTES / 1024
    scale_f = kib / max(copies_f)
    scale_w = kib / max(copies_w)
    kernels = {}
    for k in set(f) | set(w):
        s = short_name(k)
        if not s.startswith("gemm_") and not s.startswith("attn_"):
            continue
        fk = sum(f.get(k, [0])) / max(1, len(f.get(k, [])))
        wk = sum(w.get(k, [0])) / max(1, len(w.get(k, [])))
        kernels[s] = {"fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
                      "traffic_bytes_per_launch": (fk * scale_f + wk * scale_w) * 1024,
                      "launches": len(f.get(k, []))}
    return {"workload": workload, "source_sha": source_sha(), "copy_bytes": COPY_BYTES,
            "copy_fetch_kib": max(copies_f), "copy_write_kib": max(copies_w),
            "scale_fetch": scale_f, "scale_write": scale_w, "kernels": kernels}


def counters(paths) -> str:
    """Per kernel (short name) and counter: dispatches and the mean value per dispatch, over
    every counter-collection CSV given (one rocprofv3 --pmc run each)."""
    per = defaultdict(lambda: defaultdict(list))
    for path in paths:
        for r in csv.DictReader(open(path)):
            per[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in per.values() for c in k})
    out = ["| kernel | " + " | ".join(f"{c} (dispatches, mean)" for c in names) + " |",
           "|---|" + "---:|" * len(names)]
    for k in sorted(per, key=lambda k: -max(sum(v) for v in per[k].values())):
        cells = []
        for c in names:
            v = per[k].get(c, [])
            cells.append(f"{len(v)}, {sum(v) / len(v):.4g}" if v else "")
        out.append(f"| {k} | " + " | ".join(cells) + " |")
    return "\n".join(out)


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print(stats(argv[1]))
    elif len(argv) >= 2 and argv[0] == "counters":
        print(counters(argv[1:]))
    elif len(argv) >= 4 and argv[0] == "pmc":
        print(json.dumps(pmc(argv[1], argv[2], argv[3]), indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
