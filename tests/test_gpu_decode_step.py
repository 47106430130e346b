"""GPU parity of the whole 7B decode step, chained as in a serving loop: block-decode
attention -> packed LM head with the confidence fused into the GEMM -> acceptance + KV
commit, three steps with tau = 1.0, 0.9, 0.7, against the oracle on sampled sequences.

64 sequences, cached prefixes U[512, 4096], B = 4 mask rows, 28/4 heads, d = 128, page
16; hidden states [256, 3584] ~ N(0, 1) and W [152064, 3584] ~ N(0, 0.02), bf16. The
random LM head gives p_max ~ 1e-3, so every tau accepts exactly one token per sequence
(the tau = 1 rule of the pages) and the commit grows each cache by one row per step.
Counts, accepted ids, commit positions, cache lengths and every committed cache byte
are bit-exact; the attention output is within 2e-2, p_max within 1e-3 relative.
"""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import DEV, from_dev, max_abs, say, to_dev

pytestmark = pytest.mark.gpu


def test_full_size_decode_step_chain():
    S, B, Hq, Hkv, D, page, V, H = 64, 4, 28, 4, 128, 16, 152064, 3584
    taus = (1.0, 0.9, 0.7)
    sample = [0, 21, 42, 63]
    say("[decode step] S=64 B=4 28/4 d=128 + LM head 3584x152064 fused, tau 1.0/0.9/0.7")
    d = synth.decode_inputs(1004, S, B, Hq, Hkv, D, 512, 4096, page,
                            extra_capacity=B * len(taus))
    h, w = synth.lmhead_inputs(1004, S * B, H, V)
    q, kn, vn = to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new)
    kc, vc, bt, cl = to_dev(d.k_cache), to_dev(d.v_cache), to_dev(d.block_table), \
        to_dev(d.cache_len)
    Wp = mars.mars_lmhead_pack(to_dev(w))
    hid = to_dev(h)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    # the oracle's LM head for the sampled sequences' rows (the hidden states are the
    # same every step, so one GEMM serves the three steps)
    rows = [s * B + r for s in sample for r in range(B)]
    ref_logits = oracle.lmhead(h.f32[rows], w.f32)
    rid, rp = oracle.confidence(ref_logits)
    del w
    # the oracle's cache: the sampled sequences' pages only
    pages = sorted(set(d.block_table[sample].ravel().tolist()))
    remap = {pg: i for i, pg in enumerate(pages)}
    sub_table = np.vectorize(remap.get)(d.block_table[sample]).astype(np.int32)
    ok, ov = d.k_cache.f32[pages], d.v_cache.f32[pages]
    olen = d.cache_len[sample].copy()

    for step, tau in enumerate(taus):
        say(f"  step {step}: tau {tau}")
        tau_d = torch.full((S,), tau, dtype=torch.float32, device=DEV)
        o = mars.mars_attn_block_decode(q, kn, vn, kc, vc, bt, cl, status=status)
        _, ids, p = mars.mars_lmhead_confidence(hid, Wp, None, fused=True, status=status)
        n, acc, pos = mars.mars_accept_commit(p.view(S, B), ids.view(S, B), tau_d, kn, vn, kc, vc,
                                              bt, cl, status=status)
        torch.cuda.synchronize()

        ro = oracle.attn_block_decode(d.q.f32[sample], d.k_new.f32[sample],
                                      d.v_new.f32[sample], ok, ov, sub_table, olen, page)
        assert max_abs(from_dev(o)[sample], ro) <= 2e-2, step

        gid = ids.cpu().numpy()[rows]
        gp = p.cpu().numpy()[rows].astype(np.float64)
        for i in range(len(rows)):
            srt = np.sort(ref_logits[i])
            if srt[-1] - srt[-2] > 2e-4:     # the argmax is unique at this precision
                assert gid[i] == rid[i], (step, i)
            else:                            # several ids are correct: the chosen one is one
                assert ref_logits[i, gid[i]] >= srt[-1] - 2e-4, (step, i)
        assert np.max(np.abs(gp / rp - 1)) <= 1e-3, step

        # acceptance and commit: both sides decide from the device's float32 p and ids
        tau_s = np.full(len(sample), tau, dtype=np.float32)
        rn, racc = oracle.accept(gp.astype(np.float32).reshape(-1, B), gid.reshape(-1, B),
                                 tau_s)
        assert (rn == 1).all(), step          # tau = 1 and a random head: one token each
        ok, ov, olen2, rpos = oracle.commit(ok, ov, sub_table, olen, d.k_new.f32[sample],
                                            d.v_new.f32[sample], rn, page)
        assert np.array_equal(n.cpu().numpy()[sample], rn), step
        assert (n.cpu().numpy() == 1).all(), step
        assert np.array_equal(acc.cpu().numpy()[sample], racc), step
        assert np.array_equal(pos.cpu().numpy()[sample], rpos), step
        assert np.array_equal(cl.cpu().numpy()[sample], olen2), step
        olen = olen2
    assert int(status.item()) == 0
    kbits = kc.cpu().view(torch.int16).numpy()[pages]
    vbits = vc.cpu().view(torch.int16).numpy()[pages]
    assert np.array_equal(kbits, synth.bf16_round(ok).view(np.int16))
    assert np.array_equal(vbits, synth.bf16_round(ov).view(np.int16))
    assert np.array_equal(cl.cpu().numpy(), d.cache_len + len(taus))
