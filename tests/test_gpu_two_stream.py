"""GPU parity: two-stream MARS attention (HIP kernels vs the CPU oracle).

Tolerances (max-abs on outputs, inputs N(0, 1)): 1e-4 for the fp32 path and
2e-2 for the bf16 path; LSE within 1e-4 (fp32) and 2e-3 (bf16: scores are
exact bf16 products accumulated in fp32).
"""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import bf16_bits, from_dev, max_abs, say, to_dev

pytestmark = pytest.mark.gpu

F32_TOL, BF16_TOL = 1e-4, 2e-2


def run_case(seed, b, L, B, Hq, Hkv, d, dtype, mode=0, pairs=None, rows=None):
    say(f"[two_stream] seed={seed} b={b} L={L} B={B} Hq={Hq} Hkv={Hkv} d={d} {dtype} mode={mode}")
    q, k, v = synth.two_stream_qkv(seed, b, L, Hq, Hkv, d, dtype)
    o, lse = mars.mars_attn_two_stream(to_dev(q), to_dev(k), to_dev(v), L, B, mask_mode=mode,
                                       return_lse=True)
    torch.cuda.synchronize()
    og, lg = from_dev(o), from_dev(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), "non-finite attention output"
    ref_o, ref_l = oracle.attn_two_stream(q.f32, k.f32, v.f32, L, B, mask_mode=mode, pairs=pairs,
                                          rows=rows)
    err_o = err_l = 0.0
    for (bi, h), ro in ref_o.items():
        sel = slice(None) if rows is None else rows
        err_o = max(err_o, max_abs(og[bi, sel, h], ro))
        err_l = max(err_l, max_abs(lg[bi, h, sel], ref_l[(bi, h)]))
    return err_o, err_l, o


@pytest.mark.parametrize("b,L,B,Hq,Hkv,d", [
    (1, 64, 4, 2, 2, 32),     # the tiny fp32 configuration
    (2, 50, 3, 4, 2, 64),     # ragged 2L, B does not divide L
    (1, 40, 5, 2, 1, 128),
    (1, 7, 7, 1, 1, 32),      # B = L
])
def test_fp32_matches_oracle(b, L, B, Hq, Hkv, d):
    eo, el, _ = run_case(1000, b, L, B, Hq, Hkv, d, "f32")
    assert eo <= F32_TOL and el <= F32_TOL, (eo, el)


@pytest.mark.parametrize("b,L,B,Hq,Hkv,d,mode", [
    (2, 256, 4, 4, 2, 64, 0),    # several 128-row tiles, clean/mask pairing
    (1, 384, 16, 4, 1, 128, 0),
    (1, 200, 7, 2, 2, 64, 0),    # tile straddles the stream boundary, partial last block
    (1, 130, 1, 2, 1, 128, 0),   # B = 1: strictly earlier clean tokens plus self
    (1, 96, 96, 2, 2, 64, 0),    # B = L
    (1, 5, 2, 1, 1, 64, 0),      # a single partial tile
    (1, 200, 4, 4, 2, 128, 1),   # dense causal over 2L
    (2, 320, 8, 6, 3, 64, 1),
    # first mask block: rows with no visible key in the first staged tile while
    # other rows of the same wave do (regression: the deferred rescale once
    # produced NaN there)
    (1, 256, 4, 8, 2, 128, 0),
    (1, 128, 4, 8, 2, 64, 0),
    (1, 256, 16, 4, 1, 128, 0),
    # d = 128 with a 7-head GQA group (the 7B grouping): batch x KV heads = 8
    # takes the XCD-striped workgroup order, 1 KV head the fallback order;
    # both ragged (2L not a multiple of the 128-row workgroup tile)
    (2, 84, 4, 28, 4, 128, 0),
    (1, 100, 4, 7, 1, 128, 0),
    # d = 128 workgroups that pair clean tile i with mask tile i (L a multiple of
    # 128): blocks larger than a tile, blocks that do not divide 128, a single
    # pair, B = L (mask rows see no clean key); causal over 2L with few tiles
    (1, 512, 200, 2, 1, 128, 0),
    (1, 384, 24, 4, 2, 128, 0),
    (1, 128, 4, 7, 1, 128, 0),
    (1, 128, 128, 2, 1, 128, 0),
    (1, 3, 2, 2, 1, 128, 1),
    (2, 300, 4, 4, 2, 128, 1),
])
def test_bf16_matches_oracle(b, L, B, Hq, Hkv, d, mode):
    eo, el, _ = run_case(2000 + L, b, L, B, Hq, Hkv, d, "bf16", mode=mode)
    assert eo <= BF16_TOL and el <= 2e-3, (eo, el)


def test_bf16_clean_half_identical_in_both_mask_modes():
    say("[two_stream] clean half MARS vs causal-2L, bit-exact")
    q, k, v = synth.two_stream_qkv(5, 2, 512, 4, 2, 64, "bf16")
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    a = mars.mars_attn_two_stream(Q, K, V, 512, 4, mask_mode=0)
    c = mars.mars_attn_two_stream(Q, K, V, 512, 4, mask_mode=1)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(a[:, :512]), bf16_bits(c[:, :512]))
    assert not np.array_equal(bf16_bits(a[:, 512:]), bf16_bits(c[:, 512:]))


def test_bf16_deterministic():
    say("[two_stream] repeat runs are bit-identical")
    q, k, v = synth.two_stream_qkv(6, 1, 256, 4, 2, 128, "bf16")
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    a = mars.mars_attn_two_stream(Q, K, V, 256, 16)
    b = mars.mars_attn_two_stream(Q, K, V, 256, 16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(a), bf16_bits(b))


def test_full_size_qwen05b_shape_sampled_heads():
    """batch 8, L = 2048, B = 4, 14/2 heads, d = 64: two sampled heads, all rows."""
    pairs = synth.sample_pairs(1002, 8, 14, 2)
    eo, el, _ = run_case(1002, 8, 2048, 4, 14, 2, 64, "bf16", pairs=pairs)
    assert eo <= BF16_TOL and el <= 2e-3, (eo, el)


@pytest.mark.parametrize("mode", [0, 1])
def test_full_size_qwen7b_shape_sampled_heads(mode):
    """batch 4, L = 4096, B = 16, 28/4 heads, d = 128: two sampled heads."""
    pairs = synth.sample_pairs(1003, 4, 28, 2)
    rows = None if mode == 0 else np.concatenate([np.arange(0, 8192, 7), [8191]])
    eo, el, _ = run_case(1003, 4, 4096, 16, 28, 4, 128, "bf16", mode=mode, pairs=pairs, rows=rows)
    assert eo <= BF16_TOL and el <= 2e-3, (eo, el)
