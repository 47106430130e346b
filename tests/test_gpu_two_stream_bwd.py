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

REL = 2e-2


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not (np.isfinite(got).all() and np.isfinite(ref).all()):
        return float("inf")
    return float(np.max(np.abs(got - ref)) / max(1.0, float(np.max(np.abs(ref)))))


def run(seed, b, L, B, Hq, Hkv, d, mode=0, groups=None):
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
        res = rel_err(gq, rq), rel_err(gk, rk), rel_err(gv, rv)
        say(f"[bwd]   normalised max errors dq {res[0]:.2e} dk {res[1]:.2e} dv {res[2]:.2e}")
        return res
    g = Hq // Hkv
    eq = max(rel_err(gq[bi, :, kv * g:(kv + 1) * g], rq[bi, :, kv * g:(kv + 1) * g])
             for bi, kv in groups)
    ek = max(rel_err(gk[bi, :, kv], rk[bi, :, kv]) for bi, kv in groups)
    ev = max(rel_err(gv[bi, :, kv], rv[bi, :, kv]) for bi, kv in groups)
    say(f"[bwd]   normalised max errors dq {eq:.2e} dk {ek:.2e} dv {ev:.2e}")
    return eq, ek, ev


@pytest.mark.parametrize("b,L,B,Hq,Hkv,d,mode", [
    (1, 256, 4, 4, 2, 64, 0),     # several 128-row / 128-key blocks, GQA 2
    (1, 200, 7, 2, 2, 64, 0),     # L not a multiple of 32: blocks straddle the streams
    (1, 130, 1, 2, 1, 128, 0),    # B = 1
    (1, 96, 96, 2, 2, 64, 0),     # B = L
    (1, 5, 2, 1, 1, 64, 0),       # a single partial block
    (1, 200, 4, 4, 2, 128, 1),    # causal over 2L
    (2, 320, 8, 6, 3, 64, 1),     # batch 2, GQA 3
    (1, 256, 16, 8, 2, 128, 0),   # GQA 4, d = 128
    (1, 160, 16, 7, 1, 128, 0),   # GQA 7 (the 7B group size)
])
def test_bwd_matches_oracle(b, L, B, Hq, Hkv, d, mode):
    eq, ek, ev = run(6000 + L, b, L, B, Hq, Hkv, d, mode)
    assert max(eq, ek, ev) <= REL, (eq, ek, ev)


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
    eq, ek, ev = run(1002, 8, 2048, 4, 14, 2, 64, groups=[(0, 0), (7, 1)])
    assert max(eq, ek, ev) <= REL, (eq, ek, ev)
