"""GPU parity: the batch-synchronous block cache (ragged block-decode rows,
batch-synchronous acceptance, block freeze) against the CPU oracle.

Attention outputs: bf16, max-abs 2e-2 (inputs N(0, 1)), as for block decode.
Counts, token ids, unfrozen counts, cache lengths and every cache byte:
bit-exact.
"""

import json
import os

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import DEV, bf16_bits, from_dev, max_abs, say, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def cache_bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("S,R,Hq,Hkv,D,page,lo,hi", [
    (4, 36, 28, 4, 128, 16, 0, 700),     # 7B heads, B_cache 32 + 4 masks: two tile groups
    (3, 20, 14, 2, 64, 16, 0, 1200),     # 0.5B heads, several cache chunks
    (5, 64, 4, 2, 128, 32, 10, 90),      # the row limit
    (2, 9, 7, 1, 64, 16, 0, 0),          # empty caches
    # 7 heads x 8 rows: two query tiles; sequences with at most 4 rows fill only the
    # first
    (6, 8, 28, 4, 128, 16, 0, 2500),
    (4, 8, 14, 2, 64, 32, 0, 1500),
])
def test_decode_rows_matches_oracle(S, R, Hq, Hkv, D, page, lo, hi):
    say(f"[block rows] S={S} R={R} Hq={Hq} Hkv={Hkv} D={D} page={page} len U[{lo},{hi}]")
    d = synth.decode_inputs(4100 + R, S, R, Hq, Hkv, D, lo, hi, page)
    rng = np.random.default_rng(4101 + R)
    n_rows = rng.integers(0, R + 1, size=S).astype(np.int32)
    n_rows[0] = R
    if S > 2:
        n_rows[1] = 0
        n_rows[2] = 1
    o = torch.full((S, R, Hq, D), 7.0, dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    mars.mars_attn_block_decode(to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), to_dev(d.k_cache),
                                to_dev(d.v_cache), to_dev(d.block_table), to_dev(d.cache_len),
                                n_rows=to_dev(n_rows), o=o, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    og = from_dev(o)
    ref = oracle.attn_block_decode_rows(d.q.f32, d.k_new.f32, d.v_new.f32, d.k_cache.f32,
                                        d.v_cache.f32, d.block_table, d.cache_len, n_rows, page)
    err = 0.0
    for s in range(S):
        Rs = int(n_rows[s])
        err = max(err, max_abs(og[s, :Rs], ref[s]))
        assert np.all(og[s, Rs:] == 7.0), "rows past n_rows were written"
    assert err <= 2e-2, err


@pytest.mark.parametrize("R", [12, 8])  # 3 query tiles; 2
def test_decode_rows_full_equals_plain_decode_bitwise(R):
    say(f"[block rows] n_rows = R = {R} everywhere vs the plain entry")
    S, Hq, Hkv, D, page = 3, 28, 4, 128, 16
    d = synth.decode_inputs(4200, S, R, Hq, Hkv, D, 100, 900, page)
    args = [to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), to_dev(d.k_cache), to_dev(d.v_cache),
            to_dev(d.block_table), to_dev(d.cache_len)]
    o1 = mars.mars_attn_block_decode(*args)
    o2 = mars.mars_attn_block_decode(*args, n_rows=torch.full((S,), R, dtype=torch.int32,
                                                              device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(o1), bf16_bits(o2))


def test_block_sync_accept_hand_worked_example():
    with open(os.path.join(GOLDEN, "block_sync_example.json")) as f:
        ex = json.load(f)
    S, B, Bc = ex["S"], ex["B"], ex["B_cache"]
    for policy in ("min", "wait"):
        say(f"[block accept] hand-worked example, policy {policy}")
        want = ex[policy]
        u = torch.zeros(S, dtype=torch.int32, device=DEV)
        toks = torch.full((S, Bc), -1, dtype=torch.int32, device=DEV)
        tau = torch.full((S,), ex["tau"], dtype=torch.float32, device=DEV)
        for t, p in enumerate(ex["p_max"]):
            ids = np.array([[100 * t + 10 * s + i for i in range(B)] for s in range(S)],
                           dtype=np.int32)
            kept, nrows = mars.mars_block_sync_accept(
                torch.tensor(p, dtype=torch.float32, device=DEV), to_dev(ids), tau, u, toks,
                policy=policy)
            torch.cuda.synchronize()
            assert kept.cpu().tolist() == want["kept"][t], (policy, t)
            assert u.cpu().tolist() == want["unfrozen"][t], (policy, t)
            assert toks.cpu().tolist() == want["block_tokens"][t], (policy, t)
            assert nrows.cpu().tolist() == [x + B for x in want["unfrozen"][t]]


@pytest.mark.parametrize("S,B,Bc,policy", [
    (7, 4, 8, "min"), (7, 4, 8, "wait"),
    (300, 8, 32, "min"), (1500, 4, 16, "wait"),   # more sequences than threads
    (64, 16, 16, "wait"),
])
def test_block_sync_accept_random_runs(S, B, Bc, policy):
    say(f"[block accept] S={S} B={B} B_cache={Bc} {policy}: 40 random steps")
    rng = np.random.default_rng(4300 + S)
    u = np.zeros(S, dtype=np.int32)
    toks = np.full((S, Bc), -1, dtype=np.int32)
    ud, td = to_dev(u), to_dev(toks)
    for t in range(40):
        p = rng.uniform(0, 1, size=(S, B)).astype(np.float32)
        p[rng.uniform(size=(S, B)) < 0.02] = np.nan
        ids = rng.integers(0, 152064, size=(S, B)).astype(np.int32)
        tau = rng.choice(np.array([0.2, 0.5, 0.9], dtype=np.float32), size=S)
        kept, nrows = mars.mars_block_sync_accept(to_dev(p), to_dev(ids), to_dev(tau), ud, td,
                                                  policy=policy)
        rk, u, toks, froze, rn = oracle.block_sync_step(p, ids, tau, u, toks, Bc, policy)
        torch.cuda.synchronize()
        assert np.array_equal(kept.cpu().numpy(), rk), t
        assert np.array_equal(ud.cpu().numpy(), u), t
        assert np.array_equal(td.cpu().numpy(), toks), t
        assert np.array_equal(nrows.cpu().numpy(), rn), t


@pytest.mark.parametrize("full", [True, False])
def test_block_freeze_matches_oracle(full):
    say(f"[block freeze] all blocks full={full}")
    S, R, Bc, Hkv, D, page = 6, 20, 16, 4, 128, 16
    d = synth.decode_inputs(4400, S, R, 2 * Hkv, Hkv, D, 0, 300, page, extra_capacity=Bc)
    u = np.full(S, Bc, dtype=np.int32)
    if not full:
        u[3] = Bc - 1
    kc, vc, cl = to_dev(d.k_cache), to_dev(d.v_cache), to_dev(d.cache_len)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    mars.mars_block_freeze(to_dev(d.k_new), to_dev(d.v_new), kc, vc, to_dev(d.block_table), cl,
                           to_dev(u), Bc, status=status)
    torch.cuda.synchronize()
    rk, rv, rl, froze = oracle.block_freeze(d.k_cache.f32, d.v_cache.f32, d.block_table,
                                            d.cache_len, d.k_new.f32, d.v_new.f32, u, Bc, page)
    assert froze == full and int(status.item()) == 0
    assert np.array_equal(cl.cpu().numpy(), rl)
    assert np.array_equal(cache_bits(kc), synth.bf16_round(rk).view(np.int16))
    assert np.array_equal(cache_bits(vc), synth.bf16_round(rv).view(np.int16))


@pytest.mark.parametrize("policy", ["min", "wait"])
def test_block_cache_loop_matches_oracle(policy):
    """Twelve steps of the whole block-cache step on the GPU (ragged attention,
    freeze, batch-synchronous acceptance), checked against the oracle after
    every step; acceptance is driven by seeded probabilities."""
    S, B, Bc, Hq, Hkv, D, page, steps = 4, 4, 8, 8, 2, 64, 16, 12
    R = Bc + B
    d = synth.decode_inputs(4500, S, R, Hq, Hkv, D, 20, 60, page,
                            extra_capacity=Bc * (steps + 1))
    kc, vc, bt = to_dev(d.k_cache), to_dev(d.v_cache), to_dev(d.block_table)
    cl = to_dev(d.cache_len)
    ud = torch.zeros(S, dtype=torch.int32, device=DEV)
    td = torch.full((S, Bc), -1, dtype=torch.int32, device=DEV)
    nr = torch.full((S,), B, dtype=torch.int32, device=DEV)
    o = torch.zeros((S, R, Hq, D), dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rkc, rvc, rcl = d.k_cache.f32, d.v_cache.f32, d.cache_len.copy()
    ru = np.zeros(S, dtype=np.int32)
    rt = np.full((S, Bc), -1, dtype=np.int32)
    rn = np.full(S, B, dtype=np.int32)
    rng = np.random.default_rng(4501)
    froze_seen = 0
    for t in range(steps):
        say(f"[block loop] {policy} step {t}")
        q, kn, vn = synth.decode_step_tensors(4502, t, S, R, Hq, Hkv, D)
        KN, VN = to_dev(kn), to_dev(vn)
        mars.mars_attn_block_decode(to_dev(q), KN, VN, kc, vc, bt, cl, n_rows=nr, o=o,
                                    status=status)
        mars.mars_block_freeze(KN, VN, kc, vc, bt, cl, ud, Bc, status=status)
        p = rng.uniform(0.3, 1.0, size=(S, B)).astype(np.float32)
        ids = rng.integers(0, 1000, size=(S, B)).astype(np.int32)
        tau = np.full(S, 0.6, dtype=np.float32)
        kept, nrows = mars.mars_block_sync_accept(to_dev(p), to_dev(ids), to_dev(tau), ud, td,
                                                  policy=policy, n_rows=nr, status=status)
        torch.cuda.synchronize()
        # oracle, same order
        ref = oracle.attn_block_decode_rows(q.f32, kn.f32, vn.f32, rkc, rvc, d.block_table, rcl,
                                            rn, page)
        rkc, rvc, rcl, froze = oracle.block_freeze(rkc, rvc, d.block_table, rcl, kn.f32, vn.f32,
                                                   ru, Bc, page)
        froze_seen += froze
        rk, ru, rt, _, rn = oracle.block_sync_step(p, ids, tau, ru, rt, Bc, policy)
        og = from_dev(o)
        for s in range(S):
            assert max_abs(og[s, :len(ref[s])], ref[s]) <= 2e-2, (t, s)
        assert int(status.item()) == 0
        assert np.array_equal(kept.cpu().numpy(), rk)
        assert np.array_equal(ud.cpu().numpy(), ru)
        assert np.array_equal(td.cpu().numpy(), rt)
        assert np.array_equal(nr.cpu().numpy(), rn)
        assert np.array_equal(cl.cpu().numpy(), rcl)
    assert froze_seen >= 1
    assert np.array_equal(cache_bits(kc), synth.bf16_round(rkc).view(np.int16))
    assert np.array_equal(cache_bits(vc), synth.bf16_round(rvc).view(np.int16))


def test_decode_rows_counts_are_clamped():
    """n_rows outside [0, R] is clamped: above R uses all R rows, below 0 none."""
    say("[block rows] n_rows clamped to [0, R]")
    S, R, Hq, Hkv, D, page = 3, 6, 4, 2, 64, 16
    d = synth.decode_inputs(4600, S, R, Hq, Hkv, D, 5, 40, page)
    args = [to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), to_dev(d.k_cache), to_dev(d.v_cache),
            to_dev(d.block_table), to_dev(d.cache_len)]
    o = torch.full((S, R, Hq, D), 3.0, dtype=torch.bfloat16, device=DEV)
    mars.mars_attn_block_decode(*args, n_rows=to_dev(np.array([R + 5, -2, 1 << 20], np.int32)),
                                o=o)
    full = mars.mars_attn_block_decode(*args)
    torch.cuda.synchronize()
    ob, fb = bf16_bits(o), bf16_bits(full)
    assert np.array_equal(ob[0], fb[0]) and np.array_equal(ob[2], fb[2])
    assert np.all(o[1].float().cpu().numpy() == 3.0)


def test_block_sync_accept_flags_out_of_range_state():
    """An unfrozen count outside [0, B_cache] raises the status flag and is
    treated as its clamp."""
    say("[block accept] corrupt unfrozen counts are flagged and clamped")
    S, B, Bc = 3, 4, 8
    p = np.full((S, B), 0.95, dtype=np.float32)
    ids = np.arange(S * B, dtype=np.int32).reshape(S, B)
    tau = np.full(S, 0.5, dtype=np.float32)
    u = np.array([-3, 2, 11], dtype=np.int32)
    toks = np.full((S, Bc), -1, dtype=np.int32)
    toks[1, :2] = [7, 8]
    toks[2, :] = np.arange(Bc)
    ud, td = to_dev(u), to_dev(toks)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kept, nrows = mars.mars_block_sync_accept(to_dev(p), to_dev(ids), to_dev(tau), ud, td,
                                              policy="wait", status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & mars.STATUS_CACHE_OVERFLOW
    rk, ru, rt, _, rn = oracle.block_sync_step(p, ids, tau, np.clip(u, 0, Bc), toks, Bc, "wait")
    assert np.array_equal(kept.cpu().numpy(), rk)
    assert np.array_equal(ud.cpu().numpy(), ru)
    assert np.array_equal(td.cpu().numpy(), rt)
    assert np.array_equal(nrows.cpu().numpy(), rn)


def test_block_freeze_flags_overflow_and_keeps_what_fits():
    say("[block freeze] a sequence without room: flagged, rows that fit are frozen")
    S, R, Bc, Hkv, D, page = 3, 12, 8, 2, 64, 16
    d = synth.decode_inputs(4700, S, R, 2 * Hkv, Hkv, D, 20, 20, page, extra_capacity=Bc)
    cap = d.max_pages * page
    lens = np.array([20, cap - 3, 20], dtype=np.int32)   # sequence 1 has room for 3 rows
    kc, vc, cl = to_dev(d.k_cache), to_dev(d.v_cache), to_dev(lens)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    mars.mars_block_freeze(to_dev(d.k_new), to_dev(d.v_new), kc, vc, to_dev(d.block_table), cl,
                           to_dev(np.full(S, Bc, np.int32)), Bc, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & mars.STATUS_CACHE_OVERFLOW
    assert list(cl.cpu().numpy()) == [20 + Bc, cap, 20 + Bc]
    rk, rv, _, _ = oracle.commit(d.k_cache.f32, d.v_cache.f32, d.block_table, lens, d.k_new.f32,
                                 d.v_new.f32, np.array([Bc, 3, Bc]), page)
    assert np.array_equal(cache_bits(kc), synth.bf16_round(rk).view(np.int16))
    assert np.array_equal(cache_bits(vc), synth.bf16_round(rv).view(np.int16))


def test_full_size_block_cache_step_sampled_sequences():
    """The benchmarked block-cache shape (Qwen2.5-7B heads, S=16, B=4, B_cache=16,
    prefixes U[512, 2048]): one step with every block full (ragged rows up to
    B_cache + B = 20, the freeze, the acceptance), the attention checked on
    sampled sequences, the integer state on all."""
    S, B, Bc, Hq, Hkv, D, page = 16, 4, 16, 28, 4, 128, 16
    R = Bc + B
    say(f"[block full size] S={S} R={R} heads {Hq}/{Hkv} d={D}")
    d = synth.decode_inputs(4800, S, R, Hq, Hkv, D, 512, 2048, page, extra_capacity=Bc)
    rng = np.random.default_rng(4801)
    u = np.full(S, Bc, dtype=np.int32)
    nrows = (u + B).astype(np.int32)
    nrows[3] = 7                                # a sequence that waits with fewer rows
    toks = rng.integers(0, 152064, size=(S, Bc)).astype(np.int32)
    kc, vc, bt, cl = to_dev(d.k_cache), to_dev(d.v_cache), to_dev(d.block_table), to_dev(d.cache_len)
    KN, VN = to_dev(d.k_new), to_dev(d.v_new)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = mars.mars_attn_block_decode(to_dev(d.q), KN, VN, kc, vc, bt, cl, n_rows=to_dev(nrows),
                                    status=status)
    ud, td = to_dev(u), to_dev(toks)
    mars.mars_block_freeze(KN, VN, kc, vc, bt, cl, ud, Bc, status=status)
    p = rng.uniform(0.0, 1.0, size=(S, B)).astype(np.float32)
    ids = rng.integers(0, 152064, size=(S, B)).astype(np.int32)
    tau = np.full(S, 0.5, dtype=np.float32)
    kept, nr = mars.mars_block_sync_accept(to_dev(p), to_dev(ids), to_dev(tau), ud, td,
                                           policy="min", status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    seqs = [0, 3, S - 1]
    ref = oracle.attn_block_decode_rows(d.q.f32, d.k_new.f32, d.v_new.f32, d.k_cache.f32,
                                        d.v_cache.f32, d.block_table, d.cache_len, nrows, page,
                                        seqs=seqs)
    for s in seqs:  # rows past nrows[s] are not written: convert only the written ones
        assert max_abs(from_dev(o[s, :nrows[s]]), ref[s]) <= 2e-2, s
    _, _, rl, froze = oracle.block_freeze(d.k_cache.f32, d.v_cache.f32, d.block_table,
                                          d.cache_len, d.k_new.f32, d.v_new.f32, u, Bc, page)
    rk, ru, rt, _, rn = oracle.block_sync_step(p, ids, tau, u, toks, Bc, "min")
    assert froze and np.array_equal(cl.cpu().numpy(), rl)
    assert np.array_equal(kept.cpu().numpy(), rk)
    assert np.array_equal(ud.cpu().numpy(), ru)
    assert np.array_equal(td.cpu().numpy(), rt)
    assert np.array_equal(nr.cpu().numpy(), rn)
