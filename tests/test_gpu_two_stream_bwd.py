"""GPU parity: two-stream attention backward (dq, dk, dv) against the fp64 oracle.

Inputs q, k, v, dO ~ N(0, 1) in bf16; o and lse come from the device forward.
Tolerance: max |gpu - oracle| <= 2e-2 * max(1, max |oracle|) per tensor. The
device rounds P and dS to bf16 before the P^T dO, dS^T Q and dS K products
(relative 2^-9 each), uses the bf16 forward output in rowsum(dO * O), and
rounds dq, dk, dv to bf16 (relative 2^-9 of values up to ~10 at these sizes).
"""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import bf16_bits, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def abs_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not (np.isfinite(got).all() and np.isfinite(ref).all()):
        return float("inf")
    return float(np.max(np.abs(got - ref)))


def run(seed, b, L, B, Hq, Hkv, d, mode=0, groups=None):
    """Returns ((err_dq, err_dk, err_dv), (max|dq|, max|dk|, max|dv|)) over the compared
    part: every tensor, or the given (batch, KV head) groups."""
    say(f"[bwd] seed={seed} b={b} L={L} B={B} Hq={Hq} Hkv={Hkv} d={d} mode={mode}")
    q, k, v = synth.two_stream_qkv(seed, b, L, Hq, Hkv, d, "bf16")
    do, _, _ = synth.two_stream_qkv(seed + 77, b, L, Hq, Hkv, d, "bf16")
    Q, K, V, DO = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = mars.mars_attn_two_stream(Q, K, V, L, B, mask_mode=mode, return_lse=True)
    dq, dk, dv = mars.mars_attn_two_stream_bwd(Q, K, V, o, DO, lse, L, B, mask_mode=mode)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_two_stream_backward(q.f32, k.f32, v.f32, do.f32, L, B,
                                                 mask_mode=mode, groups=groups)
    gq, gk, gv = from_dev(dq), from_dev(dk), from_dev(dv)
    if groups is None:
        parts = [(gq, rq), (gk, rk), (gv, rv)]
    else:
        g = Hq // Hkv
        sel_q = lambda x: np.stack([x[bi, :, kv * g:(kv + 1) * g] for bi, kv in groups])
        sel_kv = lambda x: np.stack([x[bi, :, kv] for bi, kv in groups])
        parts = [(sel_q(gq), sel_q(rq)), (sel_kv(gk), sel_kv(rk)), (sel_kv(gv), sel_kv(rv))]
    errs = tuple(abs_err(g_, r_) for g_, r_ in parts)
    refs = tuple(float(np.max(np.abs(r_))) for _, r_ in parts)
    say(f"[bwd]   max |err| dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}; "
        f"max |ref| dq {refs[0]:.3f} dk {refs[1]:.3f} dv {refs[2]:.3f}")
    return errs, refs


def check(errs, refs, bounds):
    """Absolute per-tensor bounds; the oracle's gradient scale they were set for must
    not have moved (a bound is only meaningful for the magnitudes it was derived from)."""
    for name, e, r, (bound, ref_max) in zip(("dq", "dk", "dv"), errs, refs, bounds):
        assert abs(r - ref_max) <= 0.01 * ref_max, (name, r, ref_max)
        assert e <= bound, (name, e, bound)


# (b, L, B, Hq, Hkv, d, mode) -> per tensor (dq, dk, dv): (absolute bound, the oracle's
# max |gradient| for these seeded inputs). Each bound is 1/50 of that magnitude.
CASES = {
    (1, 256, 4, 4, 2, 64, 0): ((0.043, 2.146), (0.069, 3.463), (0.135, 6.766)),
    (1, 200, 7, 2, 2, 64, 0): ((0.034, 1.702), (0.060, 2.984), (0.089, 4.474)),
    (1, 130, 1, 2, 1, 128, 0): ((0.065, 3.243), (0.084, 4.182), (0.145, 7.246)),
    (1, 96, 96, 2, 2, 64, 0): ((0.043, 2.175), (0.059, 2.930), (0.089, 4.473)),
    (1, 5, 2, 1, 1, 64, 0): ((0.042, 2.103), (0.030, 1.487), (0.070, 3.488)),
    (1, 200, 4, 4, 2, 128, 1): ((0.044, 2.204), (0.077, 3.871), (0.108, 5.399)),
    (2, 320, 8, 6, 3, 64, 1): ((0.057, 2.858), (0.076, 3.793), (0.115, 5.733)),
    (1, 256, 16, 8, 2, 128, 0): ((0.073, 3.629), (0.087, 4.355), (0.163, 8.166)),
    (1, 160, 16, 7, 1, 128, 0): ((0.084, 4.215), (0.126, 6.280), (0.212, 10.619)),
}
FULL_05B = ((0.061, 3.0405), (0.145, 7.2636), (0.251, 12.5279))
FULL_7B = ((0.073, 3.6721), (0.146, 7.2799), (0.267, 13.3539))
CASE_NOTES = ["several 128-row / 128-key blocks, GQA 2",
              "L not a multiple of 32: blocks straddle the streams", "B = 1", "B = L",
              "a single partial block", "causal over 2L", "batch 2, GQA 3", "GQA 4, d = 128",
              "GQA 7 (the 7B group size)"]


@pytest.mark.parametrize("case", list(CASES), ids=CASE_NOTES)
def test_bwd_matches_oracle(case):
    b, L, B, Hq, Hkv, d, mode = case
    errs, refs = run(6000 + L, b, L, B, Hq, Hkv, d, mode)
    check(errs, refs, CASES[case])


def test_bwd_deterministic():
    say("[bwd] repeat runs are bit-identical")
    L, B = 192, 4
    q, k, v = synth.two_stream_qkv(61, 1, L, 4, 2, 64, "bf16")
    do, _, _ = synth.two_stream_qkv(62, 1, L, 4, 2, 64, "bf16")
    Q, K, V, DO = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = mars.mars_attn_two_stream(Q, K, V, L, B, return_lse=True)
    a = mars.mars_attn_two_stream_bwd(Q, K, V, o, DO, lse, L, B)
    c = mars.mars_attn_two_stream_bwd(Q, K, V, o, DO, lse, L, B)
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert np.array_equal(bf16_bits(x), bf16_bits(y))


def test_full_size_qwen05b_bwd_sampled_groups():
    """batch 8, L = 2048, B = 4, 14/2 heads, d = 64: two (batch, KV head) groups."""
    errs, refs = run(1002, 8, 2048, 4, 14, 2, 64, groups=[(0, 0), (7, 1)])
    check(errs, refs, FULL_05B)


def test_full_size_qwen7b_bwd_sampled_groups():
    """batch 4, L = 4096 (2L = 8192), B = 16, 28/4 heads, d = 128: two (batch, KV head)
    groups, each 7 query heads over all 8192 rows (the launch the benchmark times)."""
    errs, refs = run(1003, 4, 4096, 16, 28, 4, 128, groups=[(0, 0), (3, 3)])
    check(errs, refs, FULL_7B)
