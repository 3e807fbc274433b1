"""Short text summaries of rocprofv3 output (kernel statistics, HBM traffic).

    python -m dilated_sparse_attention_amd.profiling stats KERNEL_STATS_CSV \\
        --title TITLE --command CMD [--match SUBSTR ...]
    python -m dilated_sparse_attention_amd.profiling traffic \\
        --fetch COUNTER_CSV --write COUNTER_CSV --command CMD
    python -m dilated_sparse_attention_amd.profiling counters COUNTER_CSV ... \\
        --title TITLE --command CMD

``stats`` turns ``rocprofv3 --kernel-trace --stats --output-format csv``
output (``*_kernel_stats.csv``) into a markdown table.  ``traffic`` reads two
``rocprofv3 --pmc`` runs of the same program, one with ``FETCH_SIZE`` and one
with ``WRITE_SIZE`` (KiB per dispatch), and scales both by what the counters
read for a plain elementwise kernel of known size (``torch.neg`` over 1 GiB of
float32 into another 1 GiB, run by ``bench.py --copy-calibration``), giving
HBM bytes per launch for every kernel of this library.  ``counters`` reads
``rocprofv3 --pmc`` passes of SQ counters (one CSV per pass, each pass with
``SQ_WAVES``) and tabulates, per kernel of this library, the instructions a
wave issues and the share of its cycles spent issuing or waiting.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CALIBRATION_KERNEL = "neg_kernel"
CALIBRATION_BYTES = 1 << 30  # read and written, each


def kernel_sources_hash() -> str:
    """Hash of the HIP sources: a counter summary records it so that stale
    readings are not reported for a changed kernel."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """'void rat::k<128>(rat::Args)' -> 'rat::k<128>'; long library names cut."""
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, c in enumerate(name):
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == "(" and depth == 0:
            name = name[:i]
            break
    return name if len(name) <= 90 else name[:87] + "..."


def stats_table(path, title, command, match=None):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            n = short_name(r["Name"])
            if match and not any(m in n for m in match):
                continue
            rows.append((n, int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
                         float(r["Percentage"])))
    rows.sort(key=lambda x: -x[1] * x[2])
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           f"Kernel sources hash: `{kernel_sources_hash()}`", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    for n, c, a, lo, hi, p in rows:
        out.append(f"| `{n}` | {c} | {a / 1e3:.1f} | {lo / 1e3:.1f} | {hi / 1e3:.1f} | {p:.1f} |")
    return "\n".join(out) + "\n"


def _counter_means(path, counter):
    acc = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return acc


def traffic(fetch_csv, write_csv, command):
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    cal_f = [v for k, vs in fetch.items() if CALIBRATION_KERNEL in k for v in vs]
    cal_w = [v for k, vs in write.items() if CALIBRATION_KERNEL in k for v in vs]
    if not cal_f or not cal_w:
        raise SystemExit("no calibration dispatch found (run the program with --copy-calibration)")
    kib = CALIBRATION_BYTES / 1024
    f_scale = kib / (sum(cal_f) / len(cal_f))
    w_scale = kib / (sum(cal_w) / len(cal_w))
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if not name.startswith("void rat::"):
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write[name]) / len(write[name])
        kernels[short_name(name)] = {
            "dispatches": len(fetch[name]),
            "fetch_kib": fk, "write_kib": wk,
            "bytes_per_launch": (fk * f_scale + wk * w_scale) * 1024,
        }
    return {
        "command": command,
        "sources_hash": kernel_sources_hash(),
        "calibration": {"kernel": "torch.neg over 1 GiB float32 (1 GiB read + 1 GiB written)",
                        "fetch_kib_measured": sum(cal_f) / len(cal_f),
                        "write_kib_measured": sum(cal_w) / len(cal_w),
                        "fetch_scale": f_scale, "write_scale": w_scale},
        "kernels": kernels,
    }


def _all_counter_means(paths):
    """{kernel: {counter: mean over dispatches}} over several pmc passes."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Kernel_Name"].startswith("void rat::"):
                    acc[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


MFMA_FLOP_PER_INSTR = 16384      # v_mfma_f32_16x16x32_bf16, the only MFMA these kernels issue
MFMA_PEAK_FLOPS = 2.5e15          # MI355X dense bf16 MFMA
NUM_CU = 256


def _avg_duration_ns(stats_csv):
    """{kernel: average duration in ns} from a rocprofv3 kernel_stats.csv."""
    out = {}
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            out[short_name(r["Name"])] = float(r["AverageNs"])
    return out


def counters_table(paths, title, command, stats_csv=None):
    means = _all_counter_means(paths)
    dur = _avg_duration_ns(stats_csv) if stats_csv else {}
    out = [f"# {title}", "", "Commands (one rocprofv3 pass per counter set):", "", "```", command, "```", "",
           f"Kernel sources hash: `{kernel_sources_hash()}`", "",
           "Per wave: instructions issued (SQ_INSTS_* / SQ_WAVES). Issue and wait shares: SQ_ACTIVE_INST_ANY "
           "and SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES (wave-cycles). LDS conflicts: SQ_LDS_BANK_CONFLICT cycles "
           "per LDS instruction.", "",
           "MFMA utilisation: issued MFMA FLOPs (SQ_INSTS_MFMA x 16,384 per v_mfma_f32_16x16x32_bf16) over "
           "(average kernel duration from the kernel trace x 2.5 PFLOP/s); MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES "
           "over (GRBM_GUI_ACTIVE x 256 CUs), the share of CU-cycles with the matrix unit busy.", "",
           "| kernel | waves | VALU/wave | MFMA/wave | LDS/wave | SALU/wave | VMEM/wave | issuing | waiting | "
           "waiting on LDS | LDS conflict cyc/instr | avg us | MFMA util | MFMA busy |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]

    def ratio(d, a, b):
        return d[a] / d[b] if a in d and d.get(b) else float("nan")

    for k in sorted(means):
        d = means[k]
        out.append(f"| `{k}` | {d.get('SQ_WAVES', float('nan')):.0f} | {ratio(d, 'SQ_INSTS_VALU', 'SQ_WAVES'):.0f} | "
                   f"{ratio(d, 'SQ_INSTS_MFMA', 'SQ_WAVES'):.0f} | {ratio(d, 'SQ_INSTS_LDS', 'SQ_WAVES'):.0f} | "
                   f"{ratio(d, 'SQ_INSTS_SALU', 'SQ_WAVES'):.0f} | {ratio(d, 'SQ_INSTS_VMEM', 'SQ_WAVES'):.0f} | "
                   f"{ratio(d, 'SQ_ACTIVE_INST_ANY', 'SQ_WAVE_CYCLES'):.2f} | "
                   f"{ratio(d, 'SQ_WAIT_INST_ANY', 'SQ_WAVE_CYCLES'):.2f} | "
                   f"{ratio(d, 'SQ_WAIT_INST_LDS', 'SQ_WAVE_CYCLES'):.2f} | "
                   f"{ratio(d, 'SQ_LDS_BANK_CONFLICT', 'SQ_INSTS_LDS'):.2f} | "
                   f"{dur[k] / 1e3 if k in dur else float('nan'):.1f} | "
                   f"{d['SQ_INSTS_MFMA'] * MFMA_FLOP_PER_INSTR / (dur[k] * 1e-9) / MFMA_PEAK_FLOPS if k in dur and 'SQ_INSTS_MFMA' in d else float('nan'):.3f} | "
                   f"{ratio(d, 'SQ_VALU_MFMA_BUSY_CYCLES', 'GRBM_GUI_ACTIVE') / NUM_CU:.3f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--match", nargs="*", default=None)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--stats", default=None, help="kernel_stats.csv of the same workload (durations)")
    a = p.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats_table(a.csv, a.title, a.command, a.match))
    elif a.cmd == "counters":
        sys.stdout.write(counters_table(a.csv, a.title, a.command, a.stats))
    else:
        sys.stdout.write(json.dumps(traffic(a.fetch, a.write, a.command), indent=1) + "\n")


if __name__ == "__main__":
    main()
