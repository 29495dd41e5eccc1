"""Summarise rocprofv3 CSV output into the short text files kept under profiles/.

  python rocprof_summary.py trace  <kernel_stats.csv> <out.txt> --command "<command>"
  python rocprof_summary.py pmc    decode|prefill <workload> <out.txt> --fetch <csv> --write <csv>
                                   --copy-fetch <csv> --copy-write <csv> --command "<command>"
  python rocprof_summary.py sq     <kernel-needle> <out.txt> --passes <csv> [<csv> ...] --command "<command>"

`trace` keeps the kernel table (calls, average/min/max duration) of a --kernel-trace --stats
run. `pmc` turns FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the decode or prefill kernel into HBM
bytes per launch, each scaled by what the same counter reads for the plain copy kernel
(pa_copy_blocks moving 4096 blocks of 256 KiB: 2 GiB read and 2 GiB written per launch), and
records the hash of that kernel's sources so bench.py only reports the figure while those
sources are unchanged. `sq` averages the SQ_* (and GRBM_*) counters of one kernel per dispatch
over several --pmc passes and derives where its waves spend their cycles.
"""
from __future__ import annotations

import argparse
import collections
import csv
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# bytes read (= written) per copy launch: 4096 pairs x (K block + V block) of 32*32*128 fp16
COPY_BYTES = 4096 * 2 * 32 * 32 * 128 * 2


def kernel_avgs(path: str) -> dict:
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def pick(avgs: dict, needle: str) -> tuple:
    hits = [(k, v) for k, v in avgs.items() if needle in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {needle!r}, found {[h[0] for h in hits]}")
    return hits[0]


def do_trace(args) -> str:
    rows = list(csv.DictReader(open(args.stats)))
    lines = [f"command: {args.command}", "", "kernel | calls | avg us | min us | max us | % time"]
    for r in rows:
        lines.append(f"{r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f}")
    return "\n".join(lines) + "\n"


def do_pmc(args) -> str:
    import bench

    fetch = kernel_avgs(args.fetch)
    write = kernel_avgs(args.write)
    cf = pick(kernel_avgs(args.copy_fetch), "copy_blocks_kernel")[1]
    cw = pick(kernel_avgs(args.copy_write), "copy_blocks_kernel")[1]
    f_factor = COPY_BYTES / (cf * 1024)
    w_factor = COPY_BYTES / (cw * 1024)
    kind = args.kind
    if kind == "decode":
        step = bench.make_workload(args.workload, poison=False)
        alg = bench.algorithmic_bytes(step)["decode"]
        needle = "decode_"
    else:
        import workloads

        step = getattr(workloads, bench.WORKLOADS["prefill-" + args.workload][0])(poison=False)
        alg = bench.prefill_bytes(step)
        needle = "prefill_f32_kernel" if step.dtype == "f32" else "prefill_mfma_kernel"
    name, fk = pick(fetch, needle)
    _, wk = pick(write, needle)
    rd = fk * 1024 * f_factor
    wr = wk * 1024 * w_factor
    lines = [
        f"command: {args.command}",
        f"kernel: {name}",
        f"FETCH_SIZE_KiB_per_dispatch: {fk:.1f}",
        f"WRITE_SIZE_KiB_per_dispatch: {wk:.1f}",
        f"copy_kernel_FETCH_SIZE_KiB: {cf:.1f}  (known read {COPY_BYTES} B -> factor {f_factor:.4f})",
        f"copy_kernel_WRITE_SIZE_KiB: {cw:.1f}  (known write {COPY_BYTES} B -> factor {w_factor:.4f})",
        f"hbm_read_bytes_per_launch: {rd:.6g}",
        f"hbm_write_bytes_per_launch: {wr:.6g}",
        f"hbm_bytes_per_launch: {rd + wr:.6g}",
        f"algorithmic_bytes_per_launch: {alg:.6g}",
        f"traffic_over_algorithmic: {(rd + wr) / alg:.4f}",
        f"source_sha256_16: {bench.source_hash(kind)}",
    ]
    return "\n".join(lines) + "\n"


def do_sq(args) -> str:
    vals = collections.defaultdict(list)
    names = set()
    for path in args.passes:
        for r in csv.DictReader(open(path)):
            if args.needle in r["Kernel_Name"]:
                names.add(r["Kernel_Name"])
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    if len(names) != 1:
        raise SystemExit(f"expected one kernel matching {args.needle!r}, found {sorted(names)}")
    v = {k: sum(x) / len(x) for k, x in vals.items()}
    lines = [f"command: {args.command}", f"kernel: {names.pop()}",
             "counter averages per dispatch (summed over the units that report them):"]
    lines += [f"  {k}: {v[k]:.6g}" for k in sorted(v)]
    wc = v.get("SQ_WAVE_CYCLES")
    if wc:
        lines.append("share of wave cycles:")
        for k, label in (("SQ_ACTIVE_INST_ANY", "issuing any instruction"),
                         ("SQ_ACTIVE_INST_VALU", "issuing vector ALU"),
                         ("SQ_ACTIVE_INST_SCA", "issuing scalar"),
                         ("SQ_ACTIVE_INST_LDS", "issuing LDS"),
                         ("SQ_WAIT_INST_ANY", "waiting to issue (dependency or arbitration)"),
                         ("SQ_WAIT_ANY", "waiting (s_waitcnt, barrier)")):
            if k in v:
                lines.append(f"  {label}: {v[k] / wc:.3f}")
    if "SQ_INSTS_MFMA" in v and v["SQ_INSTS_MFMA"]:
        m = v["SQ_INSTS_MFMA"]
        lines.append("instructions per MFMA:")
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU", "SQ_INSTS_LDS"):
            if k in v:
                lines.append(f"  {k}: {v[k] / m:.3f}")
    if v.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in v:
        lines.append("vector ALU co-executing with MFMA, share of MFMA-busy cycles: "
                     f"{v['SQ_VALU_MFMA_COEXEC_CYCLES'] / v['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("kind", choices=["decode", "prefill"])
    p.add_argument("workload")
    p.add_argument("out")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--command"):
        p.add_argument(k, required=True)
    q = sub.add_parser("sq")
    q.add_argument("needle")
    q.add_argument("out")
    q.add_argument("--passes", nargs="+", required=True)
    q.add_argument("--command", required=True)
    args = ap.parse_args()
    text = {"trace": do_trace, "pmc": do_pmc, "sq": do_sq}[args.mode](args)
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
