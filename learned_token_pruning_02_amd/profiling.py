"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m learned_token_pruning_02_amd.profiling \
        --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --workload NAME --command "..." --out profiles/NAME

DIR arguments are rocprofv3 output directories (``--output-format csv``):
--trace from ``--kernel-trace --stats``, --fetch/--write from ``--pmc
FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of the same command, --copy-fetch /
--copy-write from the same counters on ``bench.py --copy-calibration`` (a
plain copy of exactly 512 MiB), which fixes the factor that turns each
counter into bytes.  Writes OUT_kernel_stats.md, OUT_hbm_traffic.md and
OUT_hbm_traffic.json; the JSON records the SHA-256 of each kernel's source
file so that a reader can tell whether the counters still describe the code.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# kernel-name fragment -> (short name, source file)
KERNELS = [
    ("gate_bf16_kernel", "gate", "learned_token_pruning_02_amd/csrc/gate.hip"),
    ("gate_f32_kernel", "gate", "learned_token_pruning_02_amd/csrc/gate.hip"),
    ("sel_clear_kernel", "select", "learned_token_pruning_02_amd/csrc/select.hip"),
    ("sel_hist_kernel", "select", "learned_token_pruning_02_amd/csrc/select.hip"),
    ("sel_cand_kernel", "select", "learned_token_pruning_02_amd/csrc/select.hip"),
    ("sel_compact_kernel", "select", "learned_token_pruning_02_amd/csrc/select.hip"),
    ("sel_one_kernel", "select", "learned_token_pruning_02_amd/csrc/select.hip"),
    ("sel_rank_kernel", "select", "learned_token_pruning_02_amd/csrc/select.hip"),
    ("sel_rankcount_kernel", "select", "learned_token_pruning_02_amd/csrc/select.hip"),
    ("gather_rows_kernel", "gather", "learned_token_pruning_02_amd/csrc/gather.hip"),
    ("attn_bf16_kernel", "attention", "learned_token_pruning_02_amd/csrc/attn.hip"),
    ("attn_f32_kernel", "attention", "learned_token_pruning_02_amd/csrc/attn.hip"),
    ("linear_bf16_kernel", "linear", "learned_token_pruning_02_amd/csrc/linear.hip"),
    ("rmsnorm_kernel", "layer", "learned_token_pruning_02_amd/csrc/layer.hip"),
    ("qk_norm_rope_kernel", "layer", "learned_token_pruning_02_amd/csrc/layer.hip"),
    ("silu_mul_kernel", "layer", "learned_token_pruning_02_amd/csrc/layer.hip"),
    ("kept_positions_kernel", "layer", "learned_token_pruning_02_amd/csrc/layer.hip"),
    ("bwd_dot_kernel", "backward", "learned_token_pruning_02_amd/csrc/attn_bwd.hip"),
    ("bwd_kv_kernel", "backward", "learned_token_pruning_02_amd/csrc/attn_bwd.hip"),
    ("bwd_q_kernel", "backward", "learned_token_pruning_02_amd/csrc/attn_bwd.hip"),
    ("bwd_reduce_kernel", "backward", "learned_token_pruning_02_amd/csrc/attn_bwd.hip"),
    ("gate_dz_kernel", "gate backward", "learned_token_pruning_02_amd/csrc/gate_bwd.hip"),
    ("gate_bwd_reduce_kernel", "gate backward", "learned_token_pruning_02_amd/csrc/gate_bwd.hip"),
    ("transpose_kernel", "gate backward", "learned_token_pruning_02_amd/csrc/gate_bwd.hip"),
    ("decode_chunk_kernel", "decode", "learned_token_pruning_02_amd/csrc/decode.hip"),
    ("decode_merge_kernel", "decode", "learned_token_pruning_02_amd/csrc/decode.hip"),
]
COPY_BYTES = 512 << 20


def source_sha(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short(name: str):
    """The longest kernel-name fragment of KERNELS that `name` contains (so
    that gate_bwd_reduce_kernel is not taken for bwd_reduce_kernel)."""
    best = None
    for frag, s, src in KERNELS:
        if frag in name and (best is None or len(frag) > len(best[0])):
            best = (frag, s, src)
    return best


def _csv(d: str, suffix: str):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return list(csv.DictReader(open(files[0])))


def counter_per_kernel(d: str, counter: str):
    """Mean value of `counter` per kernel (KiB per dispatch, as rocprofv3 reports)."""
    acc = collections.defaultdict(list)
    for r in _csv(d, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def copy_factor(d: str, counter: str) -> float:
    vals = counter_per_kernel(d, counter)
    best = max(vals.values())  # the 512 MiB copy dominates every other dispatch
    return COPY_BYTES / (best * 1024.0)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True, help="the profiled command, for the record")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    stats = _csv(a.trace, "kernel_stats.csv")
    # Per-call durations from the trace, for the median (the average also
    # holds the first calls, made while the chip's clocks still ramp up).
    durs = collections.defaultdict(list)
    try:
        for r in _csv(a.trace, "kernel_trace.csv"):
            durs[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    except (FileNotFoundError, KeyError, ValueError):
        durs.clear()
    lines = [f"# Kernel time: {a.workload}", "",
             "rocprofv3 kernel-trace statistics (`--kernel-trace --stats --output-format csv`); "
             "the median is over the per-call durations of the trace.", "",
             "Command (from the repository root):", "", "```", a.command, "```", "",
             "| kernel | calls | average us | median us | min us | max us | share |",
             "|---|---|---|---|---|---|---|"]
    for r in stats:
        d = sorted(durs.get(r["Name"], []))
        med = f"{d[len(d) // 2] / 1e3:.1f}" if d else "-"
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {med} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    open(a.out + "_kernel_stats.md", "w").write("\n".join(lines) + "\n")

    ff = copy_factor(a.copy_fetch, "FETCH_SIZE")
    wf = copy_factor(a.copy_write, "WRITE_SIZE")
    fetch = counter_per_kernel(a.fetch, "FETCH_SIZE")
    write = counter_per_kernel(a.write, "WRITE_SIZE")
    rec = {"workload": a.workload, "command": a.command,
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": ff, "write_factor": wf},
           "kernels": {}}
    md = [f"# HBM traffic per dispatch: {a.workload}", "",
          "rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE`, one run each, KiB per dispatch, "
          "scaled by what the same counters read for a plain 512 MiB device copy "
          "(`python bench.py --copy-calibration`).", "",
          f"Calibration: FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {wf:.3f} = bytes.", "",
          "Command (from the repository root):", "", "```", a.command, "```", "",
          "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MiB | written MiB |",
          "|---|---|---|---|---|"]
    seen = collections.Counter()
    for name in sorted(set(fetch) | set(write)):
        s = short(name)
        if s is None:
            continue
        frag, _, src = s
        # Several instantiations of one kernel template get their own keys.
        seen[frag] += 1
        key = frag if seen[frag] == 1 else f"{frag}#{seen[frag]}"
        f_kib, w_kib = fetch.get(name, 0.0), write.get(name, 0.0)
        rb, wb = f_kib * 1024 * ff, w_kib * 1024 * wf
        rec["kernels"][key] = {"source": src, "source_sha256": source_sha(src), "name": name[:120],
                               "fetch_kib": f_kib, "write_kib": w_kib,
                               "read_bytes": rb, "written_bytes": wb}
        md.append(f"| `{key}` | {f_kib:.1f} | {w_kib:.1f} | {rb / 2**20:.2f} | {wb / 2**20:.2f} |")
    open(a.out + "_hbm_traffic.md", "w").write("\n".join(md) + "\n")
    with open(a.out + "_hbm_traffic.json", "w") as f:
        json.dump(rec, f, indent=1)
    print(f"wrote {a.out}_kernel_stats.md, {a.out}_hbm_traffic.md, {a.out}_hbm_traffic.json")


if __name__ == "__main__":
    main()
