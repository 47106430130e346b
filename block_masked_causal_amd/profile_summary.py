"""Summaries of rocprofv3 CSV output for the files kept under profiles/.

    python -m block_masked_causal_amd.profile_summary stats KERNEL_STATS_CSV \
        --title T --cmd "rocprofv3 ..." --out profiles/NAME.md
    python -m block_masked_causal_amd.profile_summary traffic \
        --fetch FETCH_COUNTER_CSV --write WRITE_COUNTER_CSV --copy-bytes N \
        --cmd-fetch "..." --cmd-write "..." --out profiles/hbm_traffic.json

`stats` turns the --kernel-trace --stats table into markdown. `traffic` reads
two --pmc runs of `bench.py --profile-pass` (FETCH_SIZE, then WRITE_SIZE, in
KiB per dispatch). That pass first copies a buffer of known size, so each
counter is scaled by (known bytes) / (what the counter read for the copy). It
then launches every hot-path kernel once. The result records the HBM bytes
per launch of each hot-path call, together with a hash of the sources that
built it: bench.py reports the figure only while those sources are unchanged.
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

# hot-path call -> (source files that build it, kernel-name substrings of its dispatches)
CALLS = {
    "two_stream_attention": (["attn_two_stream.hip", "attn_common.hpp", "mars_common.hpp"],
                             ["two_stream_bf16_kernel"]),
    "block_decode_attention": (["attn_decode.hip", "mars_common.hpp"],
                               ["decode_split_kernel", "decode_merge_kernel"]),
    "lmhead_confidence_fused": (["lmhead_confidence.hip", "mars_common.hpp"],
                                ["lmhead_gemm_kernel<true, 320>",
                                 "lmhead_gemm_kernel<true, 64>", "conf_merge_wide_kernel"]),
    "lmhead_gemm_plus_confidence": (["lmhead_confidence.hip", "mars_common.hpp"],
                                    ["lmhead_gemm_kernel<false, 320>",
                                     "lmhead_gemm_kernel<false, 64>", "conf_partial_kernel",
                                     r"conf_merge_kernel\("]),
    "accept_commit": (["accept_commit.hip", "mars_common.hpp"], ["accept_commit_kernel"]),
    "kv_append": (["accept_commit.hip", "mars_common.hpp"],
                  ["kv_append_kernel", "kv_append_len_kernel"]),
    "two_stream_backward": (["attn_two_stream_bwd.hip", "attn_common.hpp", "mars_common.hpp"],
                            ["bwd_dsum_kernel", "bwd_dq_kernel", r"bwd_dkv_kernel<",
                             "bwd_dkv_reduce_kernel"]),
}
COPY_KERNEL = "copyBuffer"


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


def _per_dispatch(path: str, counter: str):
    """kernel name -> list of per-dispatch counter values (summed over dimensions)."""
    acc = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        acc[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in sorted(acc.items(), key=lambda kv: int(kv[0])):
        out[names[key]].append(v)
    return out


def traffic(args) -> None:
    fetch = _per_dispatch(args.fetch, "FETCH_SIZE")
    write = _per_dispatch(args.write, "WRITE_SIZE")

    def copy_value(table):
        vals = [v for n, vs in table.items() if COPY_KERNEL in n for v in vs]
        if not vals:
            raise SystemExit("no calibration copy dispatch found")
        return max(vals)  # the large calibration copy, not small incidental copies

    f_copy, w_copy = copy_value(fetch), copy_value(write)
    f_fac = args.copy_bytes / (f_copy * 1024.0)
    w_fac = args.copy_bytes / (w_copy * 1024.0)
    out = {
        "calibration": {"copy_bytes": args.copy_bytes, "fetch_kib": f_copy, "write_kib": w_copy,
                        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
        "command_fetch": args.cmd_fetch, "command_write": args.cmd_write, "calls": {}}
    for call, (files, pats) in CALLS.items():
        fk = wk = 0.0
        seen = []
        for pat in pats:
            fv = [v for n, vs in fetch.items() if re.search(pat, n) for v in vs]
            wv = [v for n, vs in write.items() if re.search(pat, n) for v in vs]
            if not fv or not wv:
                continue
            # one hot-path call launches each of its kernels once in the pass
            fk += sum(fv) / len(fv)
            wk += sum(wv) / len(wv)
            seen.append(pat)
        if not seen:
            continue
        out["calls"][call] = {
            "kernels": seen, "sources": files, "sha256": sources_sha256(files),
            "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
            "bytes": round(fk * 1024.0 * f_fac + wk * 1024.0 * w_fac)}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    md = [f"# HBM traffic per launch of each hot-path call (bench.py --profile-pass)", "",
          "Commands (on one MI355X; $REPO is the repository root):", "", "```",
          args.cmd_fetch, args.cmd_write, "```", "",
          f"Calibration: a plain {args.copy_bytes} B device copy reads FETCH_SIZE = "
          f"{f_copy:.1f} KiB and WRITE_SIZE = {w_copy:.1f} KiB, so FETCH_SIZE is scaled by "
          f"{f_fac:.4f} and WRITE_SIZE by {w_fac:.4f}.", "",
          "| call | kernels | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch |",
          "|---|---|---|---|---|"]
    for call, e in out["calls"].items():
        md.append(f"| {call} | {', '.join(e['kernels'])} | {e['fetch_kib']:.1f} | "
                  f"{e['write_kib']:.1f} | {e['bytes']} |")
    md += ["", f"Machine-readable copy with source hashes: {os.path.basename(args.out)} "
           "(bench.py reports a figure only while the hashed sources are unchanged).",
           "Summary written by: python -m block_masked_causal_amd.profile_summary traffic "
           "--fetch <fetch csv> --write <write csv> --copy-bytes "
           f"{args.copy_bytes} --cmd-fetch ... --cmd-write ... --out {args.out}"]
    with open(os.path.splitext(args.out)[0] + ".md", "w") as f:
        f.write("\n".join(md) + "\n")


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
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    args = ap.parse_args()
    (stats if args.cmd_name == "stats" else traffic)(args)


if __name__ == "__main__":
    main()
