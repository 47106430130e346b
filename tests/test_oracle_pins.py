"""The CPU oracle against what the pages and mathematics fix (no GPU needed)."""

import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import pin_checks as pc


def test_mask_hand_worked_fixtures():
    pc.check_mask_fixtures(oracle.build_mask_loops)
    pc.check_mask_fixtures(oracle.build_mask)


def test_mask_bruteforce_all_small_L_and_B():
    pc.check_mask_bruteforce(oracle.build_mask, max_L=24)


def test_mask_loop_and_grid_forms_agree():
    for L in range(1, 13):
        for B in range(1, L + 1):
            assert np.array_equal(oracle.build_mask_loops(L, B), oracle.build_mask(L, B))


def test_mask_closed_forms():
    pc.check_mask_closed_forms(oracle.build_mask)


def test_useful_pair_count_closed_forms():
    pc.check_useful_pairs(oracle.useful_pairs_two_stream)


def test_bench_useful_flops_agree_with_the_oracle_pair_count():
    import bench
    for L, B in ((5, 2), (16, 4), (12, 1), (9, 9), (4096 // 64, 16)):
        for mode in (0, 1):
            for d in (32, 64, 128):
                want = 4 * d * oracle.useful_pairs_two_stream(L, B, mode)
                assert bench.useful_two_stream_flops(1, L, B, 1, d, mode) == want


def test_mask_b1_sees_strictly_earlier_clean_tokens():
    pc.check_mask_b1(oracle.build_mask)


def test_mask_bL_is_causal_inside_mask_stream():
    pc.check_mask_bL(oracle.build_mask)


def test_ar_signal_ratio_matches_printed_table(golden_dir):
    with open(os.path.join(golden_dir, "ar_signal_ratio.json")) as f:
        g = json.load(f)
    for B, want in g["mask_only"].items():
        _, mask_only = oracle.ar_signal_ratio(64, int(B))
        assert mask_only == pytest.approx(want, abs=1e-12)
    for B, want in g["combined"].items():
        combined, _ = oracle.ar_signal_ratio(64, int(B))
        assert round(combined, g["combined_printed_decimals"][B]) == pytest.approx(want, abs=1e-12)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
def test_ar_signal_ratio_closed_form(B):
    combined, mask_only = oracle.ar_signal_ratio(64, B)
    assert combined == pytest.approx((1 + 1 / B) / 2, abs=1e-15)
    assert mask_only == pytest.approx(1 / B, abs=1e-15)


def test_clean_half_equals_plain_causal_attention():
    pc.check_clean_half_is_causal(oracle.attn_two_stream)


def test_clean_half_ignores_mask_stream_inputs():
    q, k, v = pc.rand_qkv(9, 1, 16, 2, 1, 8)
    a, _ = oracle.attn_two_stream(q, k, v, 16, 4)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 16:] += 5.0
    k2[:, 16:] -= 3.0
    v2[:, 16:] *= 7.0
    b, _ = oracle.attn_two_stream(q2, k2, v2, 16, 4)
    for key in a:
        np.testing.assert_array_equal(a[key][:16], b[key][:16])


def test_b_equals_L_mask_half_is_causal_on_mask_stream():
    pc.check_bL_mask_half_is_causal(oracle.attn_two_stream)


@pytest.mark.parametrize("L,B,mode", [(20, 3, 0), (16, 4, 0), (9, 1, 0), (7, 7, 0), (10, 4, 1)])
def test_rows_equal_softmax_over_visible_keys(L, B, mode):
    pc.check_rows_by_gather(oracle.attn_two_stream, L=L, B=B, mask_mode=mode)


def test_single_key_rows_return_their_value():
    pc.check_single_key_rows(oracle.attn_two_stream)


def test_gqa_head_mapping():
    pc.check_gqa_head_map(oracle.attn_two_stream)


def test_decode_equals_causal_attention_over_prefix_and_new_rows():
    pc.check_decode_matches_causal_sdpa(oracle.attn_block_decode)


def test_decode_equals_two_stream_mask_rows():
    pc.check_decode_equals_two_stream(oracle.attn_two_stream, oracle.attn_block_decode)


def test_confidence_closed_forms():
    pc.check_confidence_closed_forms(oracle.confidence_row)


def test_confidence_matches_library_softmax():
    pc.check_confidence_vs_torch(oracle.confidence_row)


def test_confidence_shift_invariant():
    row = np.random.default_rng(3).standard_normal(3000)
    a = oracle.confidence_row(row)
    b = oracle.confidence_row(row + 1234.5)
    assert a[0] == b[0] and a[1] == pytest.approx(b[1], rel=1e-12)


def test_peaked_logits_realise_their_target():
    pool = synth.PeakedLogitsPool(seed=11, N=32, V=20000, taus=(0.9, 0.6))
    ids, peak, target = pool.peaks(step=3)
    logits = pool.logits(step=3)
    got_ids, got_p = oracle.confidence(logits)
    assert np.array_equal(got_ids, ids.astype(np.int32))
    assert np.max(np.abs(got_p - target)) < 5e-7
    for tau in (0.9, 0.6):
        assert np.min(np.abs(got_p - tau)) > 1e-6


def test_accept_truth_table():
    pc.check_accept_truth_table(oracle.accept_count)


def test_accept_rules():
    pc.check_accept_rules(oracle.accept_count)


def test_accept_tau_one_on_real_logits_accepts_one():
    logits = synth.normal_logits(1001, 16, 1000, 3.0)
    ids, p = oracle.confidence(logits)
    n, acc = oracle.accept(p.reshape(4, 4), ids.reshape(4, 4), np.ones(4))
    assert (n == 1).all()
    assert np.array_equal(acc[:, 0], ids.reshape(4, 4)[:, 0]) and (acc[:, 1:] == -1).all()


@pytest.mark.parametrize("tau,expect", [(0.9, 1.2835), (0.6, 5.7314)])
def test_accept_mean_matches_beta51_closed_form(tau, expect):
    """p ~ Beta(5, 1) i.i.d., q = 1 - tau^5: E[n] = q(1 - q^B)/(1 - q) + (1 - q)."""
    B, S = 8, 4000
    q = 1 - tau ** 5
    closed = q * (1 - q ** B) / (1 - q) + (1 - q)
    assert closed == pytest.approx(expect, abs=1e-4)
    p = np.empty((S, B))
    for step in range(B):
        pool_p = np.random.default_rng([77, step]).random(S) ** (1 / 5)
        p[:, step] = pool_p
    n = np.array([oracle.accept_count(p[s], tau) for s in range(S)])
    se = n.std() / np.sqrt(S)
    assert abs(n.mean() - closed) < 5 * se


def test_commit_hand_worked_example():
    pc.check_commit_example(oracle.commit)


def test_commit_positions_and_growth():
    d = synth.decode_inputs(5, S=6, B=4, n_q_heads=4, n_kv_heads=2, head_dim=8, len_lo=0,
                            len_hi=20, page_size=4, extra_capacity=8, dtype="f32")
    n = np.array([1, 4, 2, 3, 1, 4], dtype=np.int32)
    kc, vc, ln, pos = oracle.commit(d.k_cache.f32, d.v_cache.f32, d.block_table, d.cache_len,
                                    d.k_new.f32, d.v_new.f32, n, 4)
    assert np.array_equal(ln, d.cache_len + n)
    for s in range(6):
        for r in range(4):
            assert pos[s, r] == (d.cache_len[s] + r if r < n[s] else -1)
    changed = (kc != d.k_cache.f32).any(axis=(1, 3)).sum()
    assert changed <= n.sum() * 1  # only committed slots can change


def test_lmhead_exact_on_small_integers():
    pc.check_lmhead_exact_integers(oracle.lmhead)


def test_generators_are_seeded_and_bf16_exact():
    a = synth.two_stream_qkv(3, 1, 8, 2, 1, 16, "bf16")
    b = synth.two_stream_qkv(3, 1, 8, 2, 1, 16, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x.bits, y.bits)
        # every float32 value is exactly representable in bfloat16
        assert not (x.f32.view(np.uint32) & 0xFFFF).any()
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to even (1.0)
    assert list(synth.bf16_bits_to_f32(synth.bf16_round(x))) == [1.0, 1.0, 1.0078125, -2.5]


# ---- attention backward ([notes] 关键设计 2: the training loss runs through the forward)

@pytest.mark.parametrize("L,B,mode", [(6, 2, 0), (5, 1, 0), (4, 4, 0), (5, 2, 1)])
def test_backward_matches_central_differences(L, B, mode):
    pc.check_backward_finite_differences(oracle.attn_two_stream, oracle.attn_two_stream_backward,
                                         L=L, B=B, mask_mode=mode)


@pytest.mark.parametrize("mode", [0, 1])
def test_backward_matches_torch_autograd(mode):
    pc.check_backward_vs_torch_autograd(oracle.attn_two_stream_backward, mask_mode=mode)


def test_backward_groups_and_row_chunks():
    pc.check_backward_groups_and_chunks(oracle.attn_two_stream_backward)


# ---- no-cache prefill: plain causal attention over any length ([gist] 4)

def test_causal_prefill_matches_sdpa():
    pc.check_causal_vs_sdpa(oracle.attn_causal)


def test_causal_prefill_equals_two_stream_mode1():
    pc.check_causal_equals_mode1(oracle.attn_causal, oracle.attn_two_stream)


def test_block_sync_hand_worked_example():
    pc.check_block_sync_example(oracle.block_sync_step)


def test_block_sync_advance_closed_forms():
    pc.check_block_sync_advance_closed_forms(oracle.block_sync_advance)


def test_block_sync_token_stream():
    pc.check_block_sync_token_stream(oracle.block_sync_step)


def test_block_freeze():
    pc.check_block_freeze(oracle.block_freeze)


def test_block_decode_rows_vs_causal():
    pc.check_block_decode_rows_vs_causal(oracle.attn_block_decode_rows, oracle.attn_causal)

