"""Summaries of rocprofv3 CSV output for the files kept under profiles/.

    python -m block_masked_causal_amd.profile_summary stats KERNEL_STATS_CSV \
        --title T --cmd "rocprofv3 ..." --out profiles/NAME.md
    python -m block_masked_causal_amd.profile_summary traffic \
        --fetch FETCH_COUNTER_CSV --write WRITE_COUNTER_CSV --plan PLAN_JSON \
        --cmd-fetch "..." --cmd-write "..." --out profiles/hbm_traffic.json
    python -m block_masked_causal_amd.profile_summary counters COUNTER_CSV \
        --plan PLAN_JSON --cmd "..." --out profiles/NAME.md

`stats` turns the --kernel-trace --stats table into markdown. `traffic` and
`counters` read --pmc runs of `bench.py --profile-pass PLAN_JSON`. That pass
first copies a buffer of known size, then launches every hot-path call once,
each right after a one-element int64 fill (the marker); PLAN_JSON lists the
calls in launch order. The dispatches between one marker and the next belong
to that call. `traffic` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
by (known bytes) / (what the counter read for the copy) and records the HBM
bytes per launch of each call with a hash of the sources that built it:
bench.py reports the figure only while those sources are unchanged.
`counters` tabulates the COUNTERS below per call, with MFMA busy =
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs).
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

_TS = ["attn_two_stream.hip", "attn_common.hpp", "mars_common.hpp"]
_DEC = ["attn_decode.hip", "mars_common.hpp"]
_LM = ["lmhead_confidence.hip", "mars_common.hpp"]
_AC = ["accept_commit.hip", "mars_common.hpp"]
_BWD = ["attn_two_stream_bwd.hip", "attn_common.hpp", "mars_common.hpp"]

# hot-path call of the profile pass -> the source files that build its kernels
SOURCES = {
    "two_stream_attention": _TS,
    "two_stream_causal_2L": _TS,
    "two_stream_attention_0.5b": _TS,
    "block_decode_attention": _DEC,
    "lmhead_confidence_fused": _LM,
    "accept_commit": _AC,
    "lmhead_gemm_plus_confidence": _LM,
    "confidence_only": _LM,
    "loop_decode_attention": _DEC,
    "loop_confidence": _LM,
    "loop_accept_commit": _AC,
    "two_stream_backward_0.5b": _BWD,
    "two_stream_backward_7b": _BWD,
    "kv_append": _AC,
    "commit_layers": _AC,
}
COPY_KERNEL = "copyBuffer"
MARKER = "FillFunctor<long>"
SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
XCCS = 8      # MI355X: 8 XCDs; each counts GRBM_GUI_ACTIVE, and the CSV holds their sum


def sources_sha256(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read() + b"\0")
    return h.hexdigest()


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= 110 else name[:107] + "..."


def stats(args) -> None:
    rows = list(csv.DictReader(open(args.csv)))
    lines = [f"# {args.title}", "", "Command (on one MI355X; $REPO is the repository root):", "",
             "```", args.cmd, "```", "",
             "rocprofv3 kernel-trace statistics (durations in microseconds):", "",
             "| kernel | calls | total us | average us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(
            f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
            f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
            f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    if args.note:
        lines += ["", args.note]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def dispatches(path: str):
    """[(dispatch id, kernel name, {counter: value})] in order (values summed over any
    dimension rows; rocprofv3's CSV already holds one chip-wide sum per counter)."""
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        key = int(r["Dispatch_Id"])
        acc[key][r["Counter_Name"]] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    return [(k, names[k], dict(acc[k])) for k in sorted(acc)]


def calibration_index(rows):
    """Index of the calibration copy: the first copy after the first marker (the pass
    creates the marker tensor, then copies the buffer of known size, then launches
    the calls, each after a marker fill)."""
    first = next((i for i, (_, n, _) in enumerate(rows) if MARKER in n), None)
    if first is None:
        raise SystemExit("no marker dispatch found")
    for i in range(first + 1, len(rows)):
        if COPY_KERNEL in rows[i][1]:
            return i
    raise SystemExit("no calibration copy dispatch found after the first marker")


def segments(rows, plan):
    """call name -> its dispatches (those after the call's marker, before the next),
    counting markers from the calibration copy on. Runtime copies (the host reading a
    status word after the last call) are not the library's and are left out."""
    out = collections.OrderedDict()
    cur = -1
    for k, name, vals in rows[calibration_index(rows) + 1:]:
        if MARKER in name:
            cur += 1
            if cur >= len(plan):
                raise SystemExit(f"more markers than calls in the plan ({len(plan)})")
            out[plan[cur]] = []
            continue
        if cur >= 0 and COPY_KERNEL not in name:
            out[plan[cur]].append((k, name, vals))
    if cur != len(plan) - 1:
        raise SystemExit(f"found {cur + 1} markers for {len(plan)} calls")
    return out


def _copy_value(rows, counter):
    return rows[calibration_index(rows)][2][counter]


def traffic(args) -> None:
    plan = json.load(open(args.plan))
    fetch = dispatches(args.fetch)
    write = dispatches(args.write)
    f_copy, w_copy = _copy_value(fetch, "FETCH_SIZE"), _copy_value(write, "WRITE_SIZE")
    copy_bytes = plan["copy_bytes"]
    f_fac = copy_bytes / (f_copy * 1024.0)
    w_fac = copy_bytes / (w_copy * 1024.0)
    fs, ws = segments(fetch, plan["calls"]), segments(write, plan["calls"])
    out = {
        "calibration": {"copy_bytes": copy_bytes, "fetch_kib": f_copy, "write_kib": w_copy,
                        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
        "command_fetch": args.cmd_fetch, "command_write": args.cmd_write, "calls": {}}
    for call in plan["calls"]:
        fk = sum(v.get("FETCH_SIZE", 0.0) for _, _, v in fs[call])
        wk = sum(v.get("WRITE_SIZE", 0.0) for _, _, v in ws[call])
        kernels = sorted({_short(n) for _, n, _ in fs[call]})
        files = SOURCES[call]
        out["calls"][call] = {
            "kernels": kernels, "dispatches": len(fs[call]), "sources": files,
            "sha256": sources_sha256(files), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
            "bytes": round(fk * 1024.0 * f_fac + wk * 1024.0 * w_fac)}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    md = ["# HBM traffic per launch of each hot-path call (bench.py --profile-pass)", "",
          "Commands (on one MI355X; $REPO is the repository root):", "", "```",
          args.cmd_fetch, args.cmd_write, "```", "",
          f"Calibration: a plain {copy_bytes} B device copy reads FETCH_SIZE = "
          f"{f_copy:.1f} KiB and WRITE_SIZE = {w_copy:.1f} KiB, so FETCH_SIZE is scaled by "
          f"{f_fac:.4f} and WRITE_SIZE by {w_fac:.4f}.", "",
          "| call | kernels | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch |",
          "|---|---|---|---|---|---|"]
    for call, e in out["calls"].items():
        md.append(f"| {call} | {'<br>'.join('`%s`' % k for k in e['kernels'])} | "
                  f"{e['dispatches']} | {e['fetch_kib']:.1f} | {e['write_kib']:.1f} | "
                  f"{e['bytes']} |")
    md += ["", f"Machine-readable copy with source hashes: {os.path.basename(args.out)} "
           "(bench.py reports a figure only while the hashed sources are unchanged).",
           "Summary written by: python -m block_masked_causal_amd.profile_summary traffic "
           "--fetch <fetch csv> --write <write csv> --plan <plan json> --cmd-fetch ... "
           f"--cmd-write ... --out {args.out}"]
    with open(os.path.splitext(args.out)[0] + ".md", "w") as f:
        f.write("\n".join(md) + "\n")


COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
            "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
            "SQ_LDS_BANK_CONFLICT"]


def counters(args) -> None:
    plan = json.load(open(args.plan))
    segs = segments(dispatches(args.csv), plan["calls"])
    lines = [f"# {args.title}", "", "Command (on one MI355X; $REPO is the repository root):", "",
             "```", args.cmd, "```", "",
             "One row per kernel dispatch of `bench.py --profile-pass` (one launch of every "
             "hot-path call). Every counter is the chip-wide sum rocprofv3 writes; each of "
             f"the {XCCS} XCCs counts GRBM_GUI_ACTIVE, so the dispatch's busy cycles are "
             f"GRBM_GUI_ACTIVE / {XCCS} (the cycles column). Derived columns:", "",
             f"- MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {SIMDS} SIMDs) x 100 "
             "(rocprofv3's MfmaUtil): the share of SIMD cycles the matrix core was busy;",
             "- MFMA GFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / 1e9 (the counter counts "
             "bf16 MFMA flops in units of 512), i.e. the flops the kernel computed, masked "
             "or not;",
             "- VALU / MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA (instructions issued);",
             f"- VALU busy % = SQ_ACTIVE_INST_VALU x 4 / (cycles x {SIMDS}) x 100 (the "
             "counter is in quad-cycles);",
             "- LDS bank-conflict cycles, summed over the chip.", "",
             "| call | kernel | cycles | MFMA busy % | MFMA GFLOP | VALU / MFMA | "
             "VALU busy % | LDS bank-conflict cycles |",
             "|---|---|---|---|---|---|---|---|"]
    for call, disp in segs.items():
        for _, name, v in disp:
            gui = v.get("GRBM_GUI_ACTIVE", 0.0) / XCCS
            busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
            nmfma = v.get("SQ_INSTS_MFMA", 0.0)
            nvalu = v.get("SQ_INSTS_VALU", 0.0)
            avalu = v.get("SQ_ACTIVE_INST_VALU", 0.0)
            pct = 100.0 * busy / (gui * SIMDS) if gui else 0.0
            vpct = 100.0 * 4.0 * avalu / (gui * SIMDS) if gui else 0.0
            ratio = f"{nvalu / nmfma:.2f}" if nmfma else "-"
            lines.append(f"| {call} | `{_short(name)}` | {gui:.0f} | {pct:.1f} | "
                         f"{mops * 512 / 1e9:.1f} | {ratio} | {vpct:.1f} | "
                         f"{v.get('SQ_LDS_BANK_CONFLICT', 0.0):.4g} |")
    if args.note:
        lines += ["", args.note]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def load_traffic(path: str):
    """call -> HBM bytes per launch, for calls whose sources are unchanged."""
    if not os.path.exists(path):
        return {}
    data = json.load(open(path))
    res = {}
    for call, e in data.get("calls", {}).items():
        try:
            if sources_sha256(e["sources"]) == e["sha256"]:
                res[call] = float(e["bytes"])
        except OSError:
            continue
    return res


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--plan", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--plan", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    args = ap.parse_args()
    {"stats": stats, "traffic": traffic, "counters": counters}[args.cmd_name](args)


if __name__ == "__main__":
    main()
