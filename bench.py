#!/usr/bin/env python3
"""Benchmark of the MARS hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--profile-pass]

A step is one pass of the whole hot path over synthetic, Qwen2.5-shaped inputs
that are resident in HBM before timing starts:
  1. two-stream MARS attention forward: batch 8, L = 2048 (2L = 4096), B = 4,
     14 query / 2 KV heads, head_dim 64, bf16;
  2. one block-decode step at the Qwen2.5-7B shape: 64 sequences with cached
     prefixes U[512, 4096], B = 4 mask queries, 28/4 heads, head_dim 128:
     decode attention over the paged cache -> LM head (3584 x 152064, bf16
     weights, packed once at setup into the GEMM's tile layout) with the
     confidence reduced in the GEMM epilogue (no logits written) ->
     acceptance (tau cycling 1.0 / 0.9 / 0.7) + KV commit of the accepted
     prefix.

The headline `value` is the useful (unmasked) TFLOP/s of the two-stream
attention; `accepted_tokens_per_s` is the decode step's accepted tokens per
second over the sum of its segment times. Per-kernel times come from HIP events
recorded on the stream the kernels run on. `decode_step_unmarked` runs the
decode step again on its own with events only around the whole run, and
`kernel_ms_back_to_back` times the attention and LM-head calls launched 20
times in a row. Extras (skippable with --no-extras): the two-pass LM head
(GEMM writing fp32 logits, then the confidence kernels), the tile-skipping benefit
at the 7B two-stream shape, a 64-step batched decode loop with a live tau
switch (accepted tokens/s), the no-cache causal prefill and the paged KV
append, acceptance + commit with every row accepted, a 64-step decode loop at the 7B shape under the batch-synchronous
block cache (both batch policies), per-token commit and one-token AR, and
the CPU oracle timed on a bounded sample.
Prints one JSON line on stdout; progress goes to stderr.

`roofline.traffic` is the HBM bytes one launch moves, from two rocprofv3
counter runs of `--profile-pass` (FETCH_SIZE, then WRITE_SIZE), each scaled
by what the counter reads for a plain copy of known size; it is null when the
kernel sources changed after the counters were taken. `--profile-pass` copies
a 1 GiB buffer once and then launches every hot-path kernel once.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# workload shapes
TS = dict(batch=8, L=2048, B=4, Hq=14, Hkv=2, d=64)           # two-stream, 0.5B shape
TS7 = dict(batch=4, L=4096, B=16, Hq=28, Hkv=4, d=128)        # two-stream, 7B shape
DEC = dict(S=64, B=4, Hq=28, Hkv=4, d=128, lo=512, hi=4096, page=16)
LM = dict(D=3584, V=152064)
PRE = dict(batch=8, T=4096 + 4, Hq=14, Hkv=2, d=64)              # no-cache prefill, 0.5B
APP = dict(S=64, T=2048, Hkv=4, d=128, page=16)                  # prompt KV append, 7B
BCL = dict(S=16, B=4, B_cache=16, Hq=28, Hkv=4, d=128, lo=512, hi=2048, page=16, steps=64,
           tau=0.95)                                               # block cache, 7B, batch 16
LOOP = dict(S=256, B=8, Hq=28, Hkv=4, d=128, lo=128, hi=2048, page=16, steps=64, switch=32)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def useful_two_stream_flops(batch, L, B, Hq, d, mask_mode=0):
    """4*d flops per visible (query, key) pair per query head; every row of the
    MARS mask sees a+1 (clean) or t+1 (mask) keys, L(L+1) pairs per head; dense
    causal over 2L sees L(2L+1)."""
    pairs = L * (L + 1) if mask_mode == 0 else L * (2 * L + 1)
    return 4.0 * d * pairs * Hq * batch


def decode_flops_bytes(cache_len, B, Hq, Hkv, d):
    lens = np.asarray(cache_len, dtype=np.float64)
    keys = (B * lens + B * (B + 1) / 2).sum()         # sum over rows of visible keys
    flops = 4.0 * d * Hq * keys
    S = lens.size
    cache_bytes = lens.sum() * Hkv * d * 2 * 2         # K and V, bf16
    io_bytes = S * B * (Hq * d * 2 * 2 + Hkv * d * 2 * 2)  # q + o, k_new + v_new
    return flops, cache_bytes + io_bytes


def to_dev(t, dev):
    import torch
    if getattr(t, "bits", None) is not None:
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(dev).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(getattr(t, "f32", t))).to(dev)


class Timer:
    """Per-segment HIP event timing on the current stream."""

    def __init__(self, names):
        import torch
        self.torch = torch
        self.names = names
        self.samples = {n: [] for n in names}
        self.pending = []

    def start(self):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.marks = [ev]

    def mark(self):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.marks.append(ev)

    def stop(self):
        self.pending.append(self.marks)

    def collect(self):
        for marks in self.pending:
            for i, n in enumerate(self.names):
                self.samples[n].append(marks[i].elapsed_time(marks[i + 1]))
        self.pending = []

    def mean_ms(self, n):
        return float(np.mean(self.samples[n]))


def roofline(bound, achieved, peak, unit, traffic=None, algorithmic_bytes=None):
    r = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4),
         "traffic": None if traffic is None else int(round(traffic))}
    if algorithmic_bytes is not None:
        r["algorithmic_bytes"] = int(round(algorithmic_bytes))
    return r


def cpu_baseline(q, k, v, budget_s):
    """The oracle's two-stream attention, timed on whole heads of the 0.5B shape."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    L, B, d = TS["L"], TS["B"], TS["d"]
    t0 = time.perf_counter()
    heads = 0
    for pair in [(b, h) for b in range(TS["batch"]) for h in range(TS["Hq"])]:
        oracle.attn_two_stream(q.f32, k.f32, v.f32, L, B, pairs=[pair])
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = useful_two_stream_flops(1, L, B, heads, d)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {TS['batch'] * TS['Hq']} (batch, head) pairs of the "
                      f"two-stream 0.5B-shape attention, all {2 * L} rows, float64 numpy "
                      f"({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--profile-pass", action="store_true",
                    help="copy 1 GiB once, launch each hot-path kernel once, exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              f"(the MARS hot path here is a single-GPU build).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    import block_masked_causal_amd as mars
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    mars.lib()
    t_setup = time.perf_counter()

    # ---- inputs -------------------------------------------------------------
    log("generating two-stream inputs (0.5B shape)")
    q, k, v = synth.two_stream_qkv(1002, TS["batch"], TS["L"], TS["Hq"], TS["Hkv"], TS["d"])
    Q, K, V = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    O = torch.empty_like(Q)

    log("generating decode inputs (7B shape) and LM head")
    # the timed steps and the decode-only loop both commit
    total_steps = 2 * args.steps + args.warmup
    di = synth.decode_inputs(1004, DEC["S"], DEC["B"], DEC["Hq"], DEC["Hkv"], DEC["d"],
                             DEC["lo"], DEC["hi"], DEC["page"],
                             extra_capacity=DEC["B"] * (total_steps + 2))
    dq, dkn, dvn = to_dev(di.q, dev), to_dev(di.k_new, dev), to_dev(di.v_new, dev)
    kc, vc = to_dev(di.k_cache, dev), to_dev(di.v_cache, dev)
    bt, cl = to_dev(di.block_table, dev), to_dev(di.cache_len, dev)
    cl0 = cl.clone()
    dO = torch.empty_like(dq)
    dws = torch.empty(mars.mars_decode_workspace_bytes(DEC["S"], DEC["B"], DEC["Hq"], DEC["Hkv"],
                                                       DEC["d"], DEC["page"], di.max_pages),
                      dtype=torch.uint8, device=dev)
    N = DEC["S"] * DEC["B"]
    h, w = synth.lmhead_inputs(1004, N, LM["D"], LM["V"])
    H, W = to_dev(h, dev), to_dev(w, dev)
    del w
    # the LM-head weights are packed once, as at model load: the same products,
    # read as contiguous 20 KiB blocks per GEMM stage
    W = mars.mars_lmhead_pack(W)
    torch.cuda.synchronize()
    logits = torch.empty((N, LM["V"]), dtype=torch.float32, device=dev)
    top = torch.empty(N, dtype=torch.int32, device=dev)
    pm = torch.empty(N, dtype=torch.float32, device=dev)
    lws = torch.empty(mars.mars_lmhead_workspace_bytes(N, LM["V"]), dtype=torch.uint8,
                      device=dev)
    taus = [torch.full((DEC["S"],), t, dtype=torch.float32, device=dev) for t in (1.0, 0.9, 0.7)]
    n_acc = torch.empty(DEC["S"], dtype=torch.int32, device=dev)
    acc_ids = torch.empty((DEC["S"], DEC["B"]), dtype=torch.int32, device=dev)
    cpos = torch.empty((DEC["S"], DEC["B"]), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s")

    seg = ["two_stream", "decode_attn", "lmhead_conf", "accept_commit"]
    timer = Timer(seg)
    dec_lens = []

    def decode_part(i, mark):
        mars.mars_attn_block_decode(dq, dkn, dvn, kc, vc, bt, cl, o=dO, workspace=dws,
                                    status=status)
        mark()
        mars.mars_lmhead_confidence(H, W, None, top_id=top, p_max=pm, workspace=lws,
                                    status=status, fused=True)
        mark()
        mars.mars_accept_commit(pm.view(DEC["S"], DEC["B"]), top.view(DEC["S"], DEC["B"]),
                                taus[i % 3], dkn, dvn, kc, vc, bt, cl, n_accepted=n_acc,
                                accepted_ids=acc_ids, commit_pos=cpos, status=status)
        mark()

    def step(i, timed):
        if timed:
            timer.start()
        mars.mars_attn_two_stream(Q, K, V, TS["L"], TS["B"], o=O)
        if timed:
            timer.mark()
        decode_part(i, timer.mark if timed else (lambda: None))
        if timed:
            timer.stop()

    if args.profile_pass:
        n = 1 << 28  # float32 elements: a 1 GiB calibration copy
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        step(0, False)
        # the two-pass LM head as well (its own traffic line)
        mars.mars_lmhead_confidence(H, W, logits, top_id=top, p_max=pm, workspace=lws,
                                    status=status)
        # and the two-stream backward at the 0.5B shape
        lse = torch.empty((TS["batch"], TS["Hq"], 2 * TS["L"]), dtype=torch.float32, device=dev)
        mars.mars_attn_two_stream(Q, K, V, TS["L"], TS["B"], o=O, lse=lse)
        mars.mars_attn_two_stream_bwd(Q, K, V, O, Q, lse, TS["L"], TS["B"])
        # and one KV append at the prompt-append shape
        app = append_inputs(synth, torch, dev)
        mars.mars_kv_append(*app)
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "copy_bytes": n * 4,
                          "status_flags": int(status.item())}), flush=True)
        return

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    lens_before = cl.cpu().numpy().copy()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect()
    lens_after = cl.cpu().numpy()
    accepted = int((lens_after - lens_before).sum())
    st = int(status.item())
    if st != 0:
        log(f"WARNING: device status flags {st}")

    # The decode step again, on its own and timed as a whole: one HIP event before
    # the first step and one after the last, none between its kernels (the
    # markers between segments above add the command processor's gap to each).
    lens_dec0 = cl.cpu().numpy().copy()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        decode_part(i, lambda: None)
    e1.record()
    torch.cuda.synchronize()
    dec_whole_ms = e0.elapsed_time(e1) / args.steps
    acc_whole = int((cl.cpu().numpy() - lens_dec0).sum())

    # Each call of the step on its own, launched back to back: one event pair
    # around 20 launches (after 3 untimed), for comparison with the in-step times
    def back_to_back(fn, n=20):
        for _ in range(3):
            fn()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        for _ in range(n):
            fn()
        b_.record()
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / n

    b2b = {
        "two_stream_attention": back_to_back(
            lambda: mars.mars_attn_two_stream(Q, K, V, TS["L"], TS["B"], o=O)),
        "block_decode_attention": back_to_back(
            lambda: mars.mars_attn_block_decode(dq, dkn, dvn, kc, vc, bt, cl, o=dO,
                                                workspace=dws, status=status)),
        "lmhead_confidence_fused": back_to_back(
            lambda: mars.mars_lmhead_confidence(H, W, None, top_id=top, p_max=pm,
                                                workspace=lws, status=status, fused=True)),
    }  # (the commit kernel is shorter than a host launch, so it is not timed this way)
    if int(status.item()) != 0:
        log(f"WARNING: device status flags {int(status.item())}")

    ms_step = wall * 1e3 / args.steps
    t_ts = timer.mean_ms("two_stream")
    t_dec = timer.mean_ms("decode_attn")
    t_lm = timer.mean_ms("lmhead_conf")
    t_acc = timer.mean_ms("accept_commit")
    ts_flops = useful_two_stream_flops(TS["batch"], TS["L"], TS["B"], TS["Hq"], TS["d"])
    value = ts_flops / (t_ts * 1e-3) / 1e12
    decode_ms = t_dec + t_lm + t_acc
    acc_tok_s = accepted / (args.steps * decode_ms * 1e-3)

    mean_len = 0.5 * (lens_before + lens_after)
    dflops, dbytes = decode_flops_bytes(mean_len, DEC["B"], DEC["Hq"], DEC["Hkv"], DEC["d"])
    lm_flops = 2.0 * N * LM["D"] * LM["V"]
    nvt = (LM["V"] + 319) // 320  # 320-entry vocabulary tiles
    # fused: W and hidden read once; per-(row, vocabulary tile) partials written and merged
    lmf_bytes = LM["V"] * LM["D"] * 2 + N * LM["D"] * 2 + 2 * N * nvt * 16
    lm_bytes = LM["V"] * LM["D"] * 2 + N * LM["D"] * 2 + N * LM["V"] * 4
    commit_bytes = accepted / args.steps * DEC["Hkv"] * DEC["d"] * 2 * 2 * 2

    from block_masked_causal_amd.profile_summary import load_traffic
    traffic = load_traffic(os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    b2, L2, Hq2, Hkv2, d2 = TS["batch"], TS["L"], TS["Hq"], TS["Hkv"], TS["d"]
    ts_bytes = b2 * 2 * L2 * d2 * 2 * (2 * Hq2 + 2 * Hkv2)   # read Q, K, V; write O (bf16)
    kernels = {
        "two_stream_attention": roofline("mfma", value, PEAK_BF16_TFLOPS, "TFLOP/s",
                                         traffic.get("two_stream_attention"), ts_bytes),
        "block_decode_attention": roofline("hbm", dbytes / (t_dec * 1e-3) / 1e9, PEAK_HBM_GBS,
                                           "GB/s", traffic.get("block_decode_attention"),
                                           dbytes),
        "lmhead_confidence_fused": roofline(
            "hbm", lmf_bytes / (t_lm * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
            traffic.get("lmhead_confidence_fused"), lmf_bytes),
        "accept_commit": roofline("hbm", commit_bytes / (t_acc * 1e-3) / 1e9, PEAK_HBM_GBS,
                                  "GB/s", traffic.get("accept_commit"), commit_bytes),
    }
    kernels["block_decode_attention"]["useful_tflops"] = round(dflops / (t_dec * 1e-3) / 1e12, 3)
    kernels["lmhead_confidence_fused"]["useful_tflops"] = round(
        lm_flops / (t_lm * 1e-3) / 1e12, 3)
    times = {"two_stream_attention": t_ts, "block_decode_attention": t_dec,
             "lmhead_confidence_fused": t_lm, "accept_commit": t_acc}

    extras = {}
    if not args.no_extras:
        extras = run_extras(mars, synth, torch, dev, logits, lws, status, H, W, N, traffic)

    result = {
        "metric": "MARS-mask attention useful TFLOP/s + accepted tokens/s per decode step",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V and caches, N(0,0.02) LM head; Qwen2.5 shapes)",
        "config": {
            "workload": "two-stream MARS attention fwd b=8 2L=4096 B=4 heads 14/2 d=64 "
                        "+ block-decode step S=64 B=4 cache U[512,4096] heads 28/4 d=128 "
                        "page 16, LM head 3584x152064 with fused confidence, accept+commit",
            "two_stream": TS, "decode": DEC, "lm_head": LM,
        },
        "accepted_tokens_per_s": round(acc_tok_s, 1),
        "decode_step_ms": round(decode_ms, 4),
        "kernel_ms_back_to_back": {k: round(v, 4) for k, v in b2b.items()},
        "two_stream_back_to_back_tflops": round(ts_flops / (b2b["two_stream_attention"] * 1e-3)
                                                / 1e12, 3),
        "decode_step_unmarked": {
            "ms": round(dec_whole_ms, 4),
            "accepted_tokens_per_s": round(acc_whole / (args.steps * dec_whole_ms * 1e-3), 1),
            "note": "the same decode step run on its own, timed with one event pair around "
                    "all steps (no markers between its kernels)"},
        "kernel_ms": {k2: round(v2, 4) for k2, v2 in times.items()},
        "roofline": kernels["two_stream_attention"],
        "kernels": kernels,
        "status_flags": st,
    }
    result.update(extras)
    if not args.no_extras:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(q, k, v, args.cpu_budget)
    print(json.dumps(result), flush=True)


def run_extras(mars, synth, torch, dev, logits, lws, status, H, W, N, traffic):
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # the two-pass LM head: GEMM writing fp32 logits, then the confidence kernels
    top2 = torch.empty(N, dtype=torch.int32, device=dev)
    pm2 = torch.empty(N, dtype=torch.float32, device=dev)
    for _ in range(2):
        mars.mars_lmhead_confidence(H, W, logits, top_id=top2, p_max=pm2, workspace=lws)
    a, b = ev(), ev()
    a.record()
    for _ in range(10):
        mars.mars_lmhead_confidence(H, W, logits, top_id=top2, p_max=pm2, workspace=lws)
    b.record()
    torch.cuda.synchronize()
    t2 = a.elapsed_time(b) / 10
    b2 = LM["V"] * LM["D"] * 2 + N * LM["D"] * 2 + 2 * N * LM["V"] * 4
    out["lmhead_gemm_plus_confidence"] = {
        "ms": round(t2, 4), "useful_tflops": round(2.0 * N * LM["D"] * LM["V"] / (t2 * 1e-3)
                                                   / 1e12, 3),
        "roofline": roofline("hbm", b2 / (t2 * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
                             traffic.get("lmhead_gemm_plus_confidence"), b2)}

    # confidence alone on the same logits: splits the LM-head call into GEMM + confidence
    top = torch.empty(N, dtype=torch.int32, device=dev)
    pm = torch.empty(N, dtype=torch.float32, device=dev)
    for _ in range(2):
        mars.mars_lmhead_confidence(None, None, logits, top_id=top, p_max=pm, workspace=lws)
    a, b = ev(), ev()
    a.record()
    for _ in range(10):
        mars.mars_lmhead_confidence(None, None, logits, top_id=top, p_max=pm, workspace=lws)
    b.record()
    torch.cuda.synchronize()
    t_conf = a.elapsed_time(b) / 10
    out["confidence_only"] = {
        "rows": N, "vocab": LM["V"], "ms": round(t_conf, 4),
        "roofline": roofline("hbm", N * LM["V"] * 4 / (t_conf * 1e-3) / 1e9, PEAK_HBM_GBS,
                             "GB/s")}

    # tile skipping at the 7B two-stream shape: MARS mask vs dense causal over 2L
    log("two-stream 7B shape: MARS mask vs causal-2L")
    q, k, v = synth.two_stream_qkv(1003, TS7["batch"], TS7["L"], TS7["Hq"], TS7["Hkv"], TS7["d"])
    Q, K, V = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    del q, k, v
    O = torch.empty_like(Q)
    res = {}
    for mode in (0, 1):
        for _ in range(2):
            mars.mars_attn_two_stream(Q, K, V, TS7["L"], TS7["B"], o=O, mask_mode=mode)
        a, b = ev(), ev()
        a.record()
        for _ in range(5):
            mars.mars_attn_two_stream(Q, K, V, TS7["L"], TS7["B"], o=O, mask_mode=mode)
        b.record()
        torch.cuda.synchronize()
        res[mode] = a.elapsed_time(b) / 5
    f0 = useful_two_stream_flops(TS7["batch"], TS7["L"], TS7["B"], TS7["Hq"], TS7["d"], 0)
    f1 = useful_two_stream_flops(TS7["batch"], TS7["L"], TS7["B"], TS7["Hq"], TS7["d"], 1)
    out["two_stream_7b"] = {
        "shape": TS7, "mars_ms": round(res[0], 4), "causal_2L_ms": round(res[1], 4),
        "mars_useful_tflops": round(f0 / (res[0] * 1e-3) / 1e12, 2),
        "causal_2L_useful_tflops": round(f1 / (res[1] * 1e-3) / 1e12, 2),
        "skip_speedup": round(res[1] / res[0], 3)}
    del Q, K, V, O
    torch.cuda.empty_cache()

    # two-stream attention backward (dq, dk, dv) at both training shapes
    out["two_stream_bwd"] = two_stream_bwd(mars, synth, torch, dev, traffic)

    # no-cache causal prefill over prompt + one block of masks, and the KV append
    # that fills the paged cache from a prompt
    out["causal_prefill"] = causal_prefill(mars, synth, torch, dev, traffic)

    # acceptance + commit with every row accepted (tau = 0) at the high-load loop's
    # shape: the largest copy one call makes there
    out["accept_commit_full"] = accept_commit_full(mars, torch, dev)

    # batched decode loop with a live tau switch
    out["decode_loop"] = decode_loop(mars, synth, torch, dev, status)

    # the batch-synchronous block cache (both batch policies) beside per-token
    # commit and one-token-per-step AR decoding, on the same confidence draws
    pol = {p_: block_cache_loop(mars, synth, torch, dev, p_)
           for p_ in ("min", "wait", "per_token", "ar")}
    pol["note"] = ("per step: decode attention, confidence over the step's rows x 152064 "
                   "fp32 logits, acceptance (+ block freeze or commit); the model layers "
                   "around attention are not part of this path, so these are not the "
                   "pages' end-to-end wall-clock ratios")
    out["decode_policies"] = pol
    return out


def accept_commit_full(mars, torch, dev):
    """mars_accept_commit at S=256, B=8 (Qwen2.5-7B KV heads) with tau = 0, so every
    row is accepted and committed: 8.4 MB of K/V rows read and written per call."""
    S, B, Hkv, d, page, steps = 256, 8, 4, 128, 16, 8
    max_pages = (B * steps + page - 1) // page
    g = torch.Generator(device="cpu").manual_seed(1010)
    kc = torch.zeros(S * max_pages, Hkv, page, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(S * max_pages, Hkv, d, page, dtype=torch.bfloat16, device=dev)
    bt = torch.randperm(S * max_pages, generator=g).to(torch.int32).reshape(S, max_pages).to(dev)
    kn = torch.randn(S, B, Hkv, d, generator=g).to(torch.bfloat16).to(dev)
    vn = torch.randn(S, B, Hkv, d, generator=g).to(torch.bfloat16).to(dev)
    pm = torch.ones(S, B, dtype=torch.float32, device=dev)
    top = torch.zeros(S, B, dtype=torch.int32, device=dev)
    tau = torch.zeros(S, dtype=torch.float32, device=dev)
    cl = torch.zeros(S, dtype=torch.int32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(4):
        cl.zero_()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(steps):
            mars.mars_accept_commit(pm, top, tau, kn, vn, kc, vc, bt, cl)
        b.record()
        torch.cuda.synchronize()
        if rep > 0:
            times.append(a.elapsed_time(b) / steps)
    if int(cl.min().item()) != B * steps:
        raise RuntimeError("full-acceptance commit did not place every row")
    ms = sum(times) / len(times)
    nbytes = S * B * Hkv * d * 2 * 2 * 2  # K and V rows, read and written
    del kc, vc, bt, kn, vn
    torch.cuda.empty_cache()
    return {"shape": {"S": S, "B": B, "Hkv": Hkv, "d": d, "page": page}, "ms": round(ms, 4),
            "roofline": roofline("hbm", nbytes / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s",
                                 None, nbytes),
            "note": "tau = 0: all 8 rows of every sequence committed; one call per step"}


def two_stream_bwd(mars, synth, torch, dev, traffic):
    """Backward of the two-stream attention; useful FLOPs = 10 d per visible pair per query
    head (QK^T recomputed, dO V^T, and the dV, dK, dQ products: 2d each)."""
    res = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for name, c in (("0.5b", TS), ("7b", TS7)):
        log(f"two-stream backward, {name} shape")
        q, k, v = synth.two_stream_qkv(1006, c["batch"], c["L"], c["Hq"], c["Hkv"], c["d"])
        do, _, _ = synth.two_stream_qkv(1007, c["batch"], c["L"], c["Hq"], c["Hkv"], c["d"])
        Q, K, V, DO = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), to_dev(do, dev)
        del q, k, v, do
        o, lse = mars.mars_attn_two_stream(Q, K, V, c["L"], c["B"], return_lse=True)
        dq, dk, dv = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
        ws = torch.empty(mars.lib().mars_attn_two_stream_bwd_workspace_bytes(
            c["batch"], c["L"], c["Hq"], c["Hkv"], c["d"]), dtype=torch.uint8, device=dev)
        call = lambda: mars.mars_attn_two_stream_bwd(Q, K, V, o, DO, lse, c["L"], c["B"], dq=dq,
                                                     dk=dk, dv=dv, workspace=ws)
        for _ in range(2):
            call()
        a, b = ev(), ev()
        a.record()
        for _ in range(5):
            call()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 5
        fl = 2.5 * useful_two_stream_flops(c["batch"], c["L"], c["B"], c["Hq"], c["d"])
        tf = fl / (ms * 1e-3) / 1e12
        res[name] = {"shape": c, "ms": round(ms, 4), "useful_tflops": round(tf, 2),
                     "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                          traffic.get("two_stream_backward") if name == "0.5b"
                                          else None)}
        del Q, K, V, DO, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return res


def append_inputs(synth, torch, dev):
    """Rows to append and an empty paged cache with room for them (APP shape)."""
    a_ = APP
    di = synth.decode_inputs(1009, a_["S"], 1, a_["Hkv"], a_["Hkv"], a_["d"], 0, 0, a_["page"],
                             extra_capacity=a_["T"])
    kc, vc = to_dev(di.k_cache, dev), to_dev(di.v_cache, dev)
    bt = to_dev(di.block_table, dev)
    del di
    _, kr, vr = synth.decode_step_tensors(1009, 0, a_["S"], a_["T"], a_["Hkv"], a_["Hkv"],
                                          a_["d"])
    KR, VR = to_dev(kr, dev), to_dev(vr, dev)
    cl = torch.zeros(a_["S"], dtype=torch.int32, device=dev)
    return KR, VR, kc, vc, bt, cl


def causal_prefill(mars, synth, torch, dev, traffic):
    """Causal attention over T = prompt + B positions (useful FLOPs: 4 d per visible
    pair per query head, T (T + 1) / 2 pairs), and the paged KV append of a prompt
    (bytes: K and V rows read once and written once)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    c = PRE
    log(f"causal prefill b={c['batch']} T={c['T']} heads {c['Hq']}/{c['Hkv']} d={c['d']}")
    q, k, v = synth.sequence_qkv(1008, c["batch"], c["T"], c["Hq"], c["Hkv"], c["d"])
    Q, K, V = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    del q, k, v
    O = torch.empty_like(Q)
    for _ in range(2):
        mars.mars_attn_causal(Q, K, V, o=O)
    a, b = ev(), ev()
    a.record()
    for _ in range(5):
        mars.mars_attn_causal(Q, K, V, o=O)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    fl = 4.0 * c["d"] * c["Hq"] * c["batch"] * c["T"] * (c["T"] + 1) / 2
    tf = fl / (ms * 1e-3) / 1e12
    res = {"prefill": {"shape": c, "ms": round(ms, 4), "useful_tflops": round(tf, 2),
                       "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s")}}
    del Q, K, V, O

    a_ = APP
    log(f"KV append S={a_['S']} T={a_['T']} heads {a_['Hkv']} d={a_['d']} page {a_['page']}")
    KR, VR, kc, vc, bt, cl = append_inputs(synth, torch, dev)
    times = []
    for i in range(7):
        cl.zero_()
        a, b = ev(), ev()
        a.record()
        mars.mars_kv_append(KR, VR, kc, vc, bt, cl)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            times.append(a.elapsed_time(b))
    ms = sum(times) / len(times)
    nbytes = 2 * 2 * a_["S"] * a_["T"] * a_["Hkv"] * a_["d"] * 2
    res["kv_append"] = {"shape": a_, "ms": round(ms, 4),
                        "roofline": roofline("hbm", nbytes / (ms * 1e-3) / 1e9, PEAK_HBM_GBS,
                                             "GB/s", traffic.get("kv_append"), nbytes)}
    del KR, VR, kc, vc, bt, cl
    torch.cuda.empty_cache()
    return res


def block_cache_loop(mars, synth, torch, dev, policy):
    """Decode loop at the 7B shape under one commit policy; the same seeded
    confidence draws (planted-peak logits) drive every policy.

    "min" / "wait": the batch-synchronous block cache. Per step: block-decode
    attention over each sequence's unfrozen tokens + B masks, the block
    freeze, the confidence of the B mask rows, the batch-synchronous
    acceptance. "per_token": every accepted token is committed at once
    (block decode over B rows, confidence, accept + commit). "ar": one token
    per step (B = 1) with a KV cache. The logits and the step's Q/K/V rows
    are written outside the timed events.
    """
    c = BCL
    block = policy in ("min", "wait")
    Bm = 1 if policy == "ar" else c["B"]
    R = c["B_cache"] + Bm if block else Bm
    log(f"decode policy {policy}: S={c['S']} B={Bm} B_cache={c['B_cache']}, "
        f"{c['steps']} steps, tau {c['tau']}")
    di = synth.decode_inputs(1010, c["S"], R, c["Hq"], c["Hkv"], c["d"], c["lo"], c["hi"],
                             c["page"], extra_capacity=c["B"] * c["steps"] + c["B_cache"])
    kc, vc = to_dev(di.k_cache, dev), to_dev(di.v_cache, dev)
    bt, cl = to_dev(di.block_table, dev), to_dev(di.cache_len, dev)
    del di
    N = c["S"] * Bm
    pool = synth.PeakedLogitsPool(1010, N, LM["V"], taus=(c["tau"],))
    pool_dev = torch.from_numpy(pool.pool).to(dev)
    logits = torch.empty_like(pool_dev)
    rows = torch.arange(N, device=dev)
    tau = torch.full((c["S"],), c["tau"], dtype=torch.float32, device=dev)
    unfrozen = torch.zeros(c["S"], dtype=torch.int32, device=dev)
    toks = torch.full((c["S"], c["B_cache"]), -1, dtype=torch.int32, device=dev)
    n_rows = torch.full((c["S"],), Bm, dtype=torch.int32, device=dev)
    kept = torch.empty(c["S"], dtype=torch.int32, device=dev)
    acc_ids = torch.empty((c["S"], Bm), dtype=torch.int32, device=dev)
    cpos = torch.empty((c["S"], Bm), dtype=torch.int32, device=dev)
    o = torch.empty((c["S"], R, c["Hq"], c["d"]), dtype=torch.bfloat16, device=dev)
    dws = torch.empty(mars.mars_decode_workspace_bytes(c["S"], R, c["Hq"], c["Hkv"], c["d"],
                                                       c["page"], bt.shape[1]),
                      dtype=torch.uint8, device=dev)
    lws = torch.empty(mars.mars_lmhead_workspace_bytes(N, LM["V"]), dtype=torch.uint8, device=dev)
    top = torch.empty(N, dtype=torch.int32, device=dev)
    pm = torch.empty(N, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    total_ms, kept_total = 0.0, 0
    len0 = int(cl.sum().item())
    for step in range(c["steps"]):
        q, kn, vn = synth.decode_step_tensors(1010, step, c["S"], R, c["Hq"], c["Hkv"], c["d"])
        Q, KN, VN = to_dev(q, dev), to_dev(kn, dev), to_dev(vn, dev)
        ids, peak, _ = pool.peaks(step)
        logits.copy_(pool_dev)
        logits[rows, torch.from_numpy(ids).to(dev)] = torch.from_numpy(peak).to(dev)
        a, b = ev(), ev()
        a.record()
        if block:
            mars.mars_attn_block_decode(Q, KN, VN, kc, vc, bt, cl, n_rows=n_rows, o=o,
                                        workspace=dws, status=status)
            mars.mars_block_freeze(KN, VN, kc, vc, bt, cl, unfrozen, c["B_cache"],
                                   status=status)
        else:
            mars.mars_attn_block_decode(Q, KN, VN, kc, vc, bt, cl, o=o, workspace=dws,
                                        status=status)
        mars.mars_lmhead_confidence(None, None, logits, top_id=top, p_max=pm, workspace=lws,
                                    status=status)
        if block:
            mars.mars_block_sync_accept(pm.view(c["S"], Bm), top.view(c["S"], Bm), tau,
                                        unfrozen, toks, policy=policy, n_kept=kept,
                                        n_rows=n_rows, status=status)
        else:
            mars.mars_accept_commit(pm.view(c["S"], Bm), top.view(c["S"], Bm), tau, KN, VN, kc,
                                    vc, bt, cl, n_accepted=kept, accepted_ids=acc_ids,
                                    commit_pos=cpos, status=status)
        b.record()
        torch.cuda.synchronize()
        total_ms += a.elapsed_time(b)
        kept_total += int(kept.sum().item())
    res = {
        "config": dict(c, policy=policy, B=Bm),
        "accepted_tokens_per_s": round(kept_total / (total_ms * 1e-3), 1),
        "ms_per_step": round(total_ms / c["steps"], 4),
        "mean_kept_per_seq_per_step": round(kept_total / (c["steps"] * c["S"]), 4),
        "status_flags": int(status.item()),
    }
    if block:
        res["blocks_frozen"] = (int(cl.sum().item()) - len0) // (c["B_cache"] * c["S"])
    return res


def decode_loop(mars, synth, torch, dev, status):
    c = LOOP
    log("decode loop: S=256 B=8, 64 steps, tau 0.9 -> 0.6 at step 32")
    di = synth.decode_inputs(1005, c["S"], c["B"], c["Hq"], c["Hkv"], c["d"], c["lo"], c["hi"],
                             c["page"], extra_capacity=c["steps"] * c["B"])
    pool = synth.PeakedLogitsPool(1005, c["S"] * c["B"], LM["V"], taus=(0.9, 0.6))
    kc, vc = to_dev(di.k_cache, dev), to_dev(di.v_cache, dev)
    bt, cl = to_dev(di.block_table, dev), to_dev(di.cache_len, dev)
    del di.k_cache, di.v_cache
    pool_dev = torch.from_numpy(pool.pool).to(dev)
    logits = torch.empty_like(pool_dev)
    N = c["S"] * c["B"]
    rows = torch.arange(N, device=dev)
    tau = torch.full((c["S"],), 0.9, dtype=torch.float32, device=dev)
    o = torch.empty((c["S"], c["B"], c["Hq"], c["d"]), dtype=torch.bfloat16, device=dev)
    dws = torch.empty(mars.mars_decode_workspace_bytes(c["S"], c["B"], c["Hq"], c["Hkv"], c["d"],
                                                       c["page"], bt.shape[1]),
                      dtype=torch.uint8, device=dev)
    lws = torch.empty(mars.mars_lmhead_workspace_bytes(N, LM["V"]), dtype=torch.uint8, device=dev)
    top = torch.empty(N, dtype=torch.int32, device=dev)
    pm = torch.empty(N, dtype=torch.float32, device=dev)
    n_acc = torch.empty(c["S"], dtype=torch.int32, device=dev)
    acc_ids = torch.empty((c["S"], c["B"]), dtype=torch.int32, device=dev)
    cpos = torch.empty((c["S"], c["B"]), dtype=torch.int32, device=dev)
    total_ms = 0.0
    accepted = []
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for s in range(c["steps"]):
        if s == c["switch"]:
            tau.fill_(0.6)  # live threshold change: same buffers, no re-initialisation
        q, kn, vn = synth.decode_step_tensors(1005, s, c["S"], c["B"], c["Hq"], c["Hkv"], c["d"])
        Q, KN, VN = to_dev(q, dev), to_dev(kn, dev), to_dev(vn, dev)
        ids, peak, _ = pool.peaks(s)
        logits.copy_(pool_dev)
        logits[rows, torch.from_numpy(ids).to(dev)] = torch.from_numpy(peak).to(dev)
        a, b = ev(), ev()
        a.record()
        mars.mars_attn_block_decode(Q, KN, VN, kc, vc, bt, cl, o=o, workspace=dws, status=status)
        mars.mars_lmhead_confidence(None, None, logits, top_id=top, p_max=pm, workspace=lws,
                                    status=status)
        mars.mars_accept_commit(pm.view(c["S"], c["B"]), top.view(c["S"], c["B"]), tau, KN, VN,
                                kc, vc, bt, cl, n_accepted=n_acc, accepted_ids=acc_ids,
                                commit_pos=cpos, status=status)
        b.record()
        torch.cuda.synchronize()
        total_ms += a.elapsed_time(b)
        accepted.append(int(n_acc.sum().item()))
    acc = np.array(accepted, dtype=np.float64)
    sw = c["switch"]
    return {
        "config": {k: c[k] for k in ("S", "B", "Hq", "Hkv", "d", "page", "steps")},
        "accepted_tokens_per_s": round(acc.sum() / (total_ms * 1e-3), 1),
        "ms_per_step": round(total_ms / c["steps"], 4),
        "mean_accepted_per_seq_tau_0.9": round(acc[:sw].mean() / c["S"], 4),
        "mean_accepted_per_seq_tau_0.6": round(acc[sw:].mean() / c["S"], 4),
        "note": "per step: decode attention + confidence over 2048 x 152064 fp32 logits + "
                "accept/commit; the synthetic logits are written outside the timed events",
    }


if __name__ == "__main__":
    main()
