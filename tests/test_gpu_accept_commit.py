"""GPU parity: acceptance + KV commit, and the batched decode loop.

Integer results (accepted counts, accepted ids, commit positions, cache
lengths) and every committed cache byte must be bit-exact.
"""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import DEV, bf16_bits, from_dev, max_abs, say, to_dev

pytestmark = pytest.mark.gpu


def cache_bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def ref_bits(x, dtype):
    if dtype == "bf16":
        return synth.bf16_round(x).view(np.int16)
    return np.ascontiguousarray(x, dtype=np.float32).view(np.int32)


def commit_case(seed, S, B, Hkv, D, page, lo, hi, dtype, p_np, ids_np, tau_np, extra=None):
    # both sides see the same float32 probabilities and thresholds
    p_np = np.asarray(p_np, dtype=np.float32)
    tau_np = np.asarray(tau_np, dtype=np.float32)
    d = synth.decode_inputs(seed, S, B, 2 * Hkv, Hkv, D, lo, hi, page,
                            extra_capacity=B if extra is None else extra, dtype=dtype)
    kc, vc = to_dev(d.k_cache), to_dev(d.v_cache)
    bt, cl = to_dev(d.block_table), to_dev(d.cache_len)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    n, acc, pos = mars.mars_accept_commit(
        to_dev(p_np), to_dev(ids_np.astype(np.int32)), to_dev(tau_np), to_dev(d.k_new), to_dev(d.v_new), kc, vc, bt, cl,
        status=status)
    torch.cuda.synchronize()
    rn, racc = oracle.accept(p_np, ids_np, tau_np)
    rk, rv, rl, rpos = oracle.commit(d.k_cache.f32, d.v_cache.f32, d.block_table, d.cache_len,
                                     d.k_new.f32, d.v_new.f32, rn, page)
    return dict(n=n.cpu().numpy(), acc=acc.cpu().numpy(), pos=pos.cpu().numpy(),
                len=cl.cpu().numpy(), kc=cache_bits(kc), vc=cache_bits(vc),
                status=int(status.item()), rn=rn, racc=racc, rpos=rpos, rlen=rl,
                rk=ref_bits(rk, dtype), rv=ref_bits(rv, dtype))


def assert_exact(r):
    assert np.array_equal(r["n"], r["rn"])
    assert np.array_equal(r["acc"], r["racc"])
    assert np.array_equal(r["pos"], r["rpos"])
    assert np.array_equal(r["len"], r["rlen"])
    assert np.array_equal(r["kc"], r["rk"])
    assert np.array_equal(r["vc"], r["rv"])


def test_tiny_fp32_config_acceptance_and_commit():
    """16 positions = 4 sequences x B = 4, logits [16 x 1000] ~ N(0, std 3), tau 0.9."""
    say("[accept] tiny fp32 configuration")
    lg = synth.normal_logits(1001, 16, 1000, 3.0)
    _, ids, p = mars.mars_lmhead_confidence(None, None, to_dev(lg))
    rid, rp = oracle.confidence(lg)
    assert np.min(np.abs(rp - 0.9)) > 1e-6
    r = commit_case(1001, 4, 4, 2, 32, 16, 0, 32, "f32", rp.reshape(4, 4), rid.reshape(4, 4),
                    np.full(4, 0.9))
    # the device's own confidence feeds the same decision
    assert np.array_equal(ids.cpu().numpy().reshape(4, 4), rid.reshape(4, 4))
    assert_exact(r)
    assert (r["n"] == 1).all()


@pytest.mark.parametrize("dtype,Hkv,D,page", [("bf16", 4, 128, 16), ("f32", 2, 64, 32),
                                                ("bf16", 2, 8, 16), ("bf16", 4, 128, 48),
                                                # V rows staged one per pass (8 KiB rows)
                                                ("f32", 2, 2048, 16),
                                                # rows too long to stage: element path
                                                ("f32", 1, 4096, 16)])
def test_multi_accept_random_thresholds(dtype, Hkv, D, page):
    say(f"[accept] multi-accept {dtype} Hkv={Hkv} d={D} page={page}")
    S, B = 24, 8
    rng = np.random.default_rng(7)
    taus = rng.choice([0.5, 0.6, 0.9, 0.95, 1.0], size=S)
    p = rng.random((S, B)) ** 0.2
    p[np.abs(p[:, :, None] - np.array([0.5, 0.6, 0.9, 0.95, 1.0])).min(-1) < 1e-6] = 0.3
    ids = rng.integers(0, 152064, size=(S, B))
    r = commit_case(4100, S, B, Hkv, D, page, 0, 90, dtype, p, ids, taus)
    assert_exact(r)
    assert r["status"] == 0
    assert r["n"].max() > 1


def test_threshold_is_inclusive_and_nan_stops():
    say("[accept] p == tau accepted, NaN stops the scan, tau = 1 gives one token")
    S, B = 4, 4
    p = np.array([[0.9, 0.9, 0.9, 0.89],
                  [np.nan, 0.99, 0.99, 0.99],
                  [0.99, np.nan, 0.99, 0.99],
                  [0.999, 0.9999, 0.99999, 0.999999]], dtype=np.float32)
    tau = np.array([0.9, 0.5, 0.5, 1.0], dtype=np.float32)
    ids = np.arange(16).reshape(4, 4)
    d = synth.decode_inputs(1, S, B, 2, 1, 32, 0, 10, 16, extra_capacity=4)
    n, acc, pos = mars.mars_accept_commit(
        to_dev(p), to_dev(ids.astype(np.int32)), to_dev(tau), to_dev(d.k_new), to_dev(d.v_new),
        to_dev(d.k_cache), to_dev(d.v_cache), to_dev(d.block_table), to_dev(d.cache_len))
    torch.cuda.synchronize()
    assert list(n.cpu().numpy()) == [3, 1, 1, 1]
    assert list(acc.cpu().numpy()[0]) == [0, 1, 2, -1]


def test_overflow_and_bad_page_are_flagged_and_clamped():
    say("[accept] overflow / bad page: flags raised, nothing written out of bounds")
    S, B, Hkv, D, page = 3, 4, 2, 32, 16
    d = synth.decode_inputs(9, S, B, 2, Hkv, D, 5, 5, page, extra_capacity=0, dtype="bf16")
    cap = d.max_pages * page
    cl = to_dev(np.array([cap - 2, 5, 5], dtype=np.int32))   # seq 0 has room for 2 rows
    bt = to_dev(d.block_table)
    bt[1, 0] = d.num_pages                                    # seq 1 page id out of range
    kc, vc = to_dev(d.k_cache), to_dev(d.v_cache)
    before_k, before_v = cache_bits(kc), cache_bits(vc)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = np.full((S, B), 0.99, dtype=np.float32)
    n, acc, pos = mars.mars_accept_commit(
        to_dev(p), to_dev(np.zeros((S, B), np.int32)), to_dev(np.full(S, 0.5, np.float32)),
        to_dev(d.k_new), to_dev(d.v_new), kc, vc, bt, cl, status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st & mars.STATUS_CACHE_OVERFLOW and st & mars.STATUS_BAD_PAGE
    assert list(n.cpu().numpy()) == [4, 4, 4]
    assert list(cl.cpu().numpy()) == [cap, 5, 9]
    assert list(pos.cpu().numpy()[0]) == [cap - 2, cap - 1, -1, -1]
    assert (pos.cpu().numpy()[1] == -1).all()
    # sequence 1 wrote nothing
    pages1 = set(d.block_table[1].tolist()) - {d.num_pages}
    after_k = cache_bits(kc)
    for pg in pages1:
        assert np.array_equal(after_k[pg], before_k[pg])


def run_loop(seed, S, B, Hq, Hkv, D, V, lo, hi, page, steps, switch, sample=None, say_every=8):
    """The batched decode loop: decode attention, confidence, accept + commit per step.

    Returns per-step device results for the sampled sequences and the final
    device caches; the oracle replays the same steps for those sequences.
    """
    d = synth.decode_inputs(seed, S, B, Hq, Hkv, D, lo, hi, page, extra_capacity=steps * B)
    pool = synth.PeakedLogitsPool(seed, S * B, V, taus=(0.9, 0.6))
    kc, vc = to_dev(d.k_cache), to_dev(d.v_cache)
    bt, cl = to_dev(d.block_table), to_dev(d.cache_len)
    pool_dev = torch.from_numpy(pool.pool).to(DEV)
    logits = torch.empty_like(pool_dev)
    tau = to_dev(synth.tau_schedule(S, 0, switch))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    sample = list(range(S)) if sample is None else list(sample)
    rows_of = lambda s: list(range(s * B, s * B + B))
    # the oracle's view: the pages of the sampled sequences only
    pages = sorted(set(d.block_table[sample].ravel().tolist()))
    remap = {pg: i for i, pg in enumerate(pages)}
    sub_table = np.vectorize(remap.get)(d.block_table[sample]).astype(np.int32)
    ok = d.k_cache.f32[pages]
    ov = d.v_cache.f32[pages]
    olen = d.cache_len[sample].copy()
    worst = 0.0
    accepted = [0, 0]   # accepted tokens over all sequences before / after the tau switch
    for step in range(steps):
        if step == switch:
            tau.copy_(to_dev(synth.tau_schedule(S, step, switch)))  # live change, no rebuild
        q, kn, vn = synth.decode_step_tensors(seed, step, S, B, Hq, Hkv, D)
        Q, KN, VN = to_dev(q), to_dev(kn), to_dev(vn)
        ids_np, peak, _ = pool.peaks(step)
        logits.copy_(pool_dev)
        logits[torch.arange(S * B, device=DEV), torch.from_numpy(ids_np).to(DEV)] = \
            torch.from_numpy(peak).to(DEV)
        o = mars.mars_attn_block_decode(Q, KN, VN, kc, vc, bt, cl, status=status)
        _, top, pm = mars.mars_lmhead_confidence(None, None, logits, status=status)
        n, acc, pos = mars.mars_accept_commit(pm.view(S, B), top.view(S, B), tau, KN, VN, kc, vc,
                                              bt, cl, status=status)
        torch.cuda.synchronize()
        # oracle replay for the sampled sequences
        rows = sum((rows_of(s) for s in sample), [])
        lg_rows = pool.pool[rows].copy()
        lg_rows[np.arange(len(rows)), ids_np[rows]] = peak[rows]
        rid, rp = oracle.confidence(lg_rows)
        ro = oracle.attn_block_decode(q.f32[sample], kn.f32[sample], vn.f32[sample], ok, ov,
                                      sub_table, olen, page)
        tau_s = np.full(len(sample), 0.9 if step < switch else 0.6)
        rn, racc = oracle.accept(rp.reshape(-1, B), rid.reshape(-1, B), tau_s)
        ok, ov, olen2, rpos = oracle.commit(ok, ov, sub_table, olen, kn.f32[sample],
                                            vn.f32[sample], rn, page)
        worst = max(worst, max_abs(from_dev(o)[sample], ro))
        gn = n.cpu().numpy()[sample]
        assert np.array_equal(gn, rn), step
        assert np.array_equal(acc.cpu().numpy()[sample], racc), step
        assert np.array_equal(pos.cpu().numpy()[sample], rpos), step
        assert np.array_equal(cl.cpu().numpy()[sample], olen2), step
        olen = olen2
        accepted[step >= switch] += int(n.sum().item())
        if step % say_every == 0:
            say(f"  step {step}: mean accepted {float(n.float().mean()):.3f}, attn err {worst:.2e}")
    assert int(status.item()) == 0
    kbits = cache_bits(kc)[pages]
    vbits = cache_bits(vc)[pages]
    assert np.array_equal(kbits, synth.bf16_round(ok).view(np.int16))
    assert np.array_equal(vbits, synth.bf16_round(ov).view(np.int16))
    return worst, accepted


def accepted_count_law(tau, B, a=5.0):
    """Mean and variance of n = max(1, leading run of p_r >= tau) for i.i.d. p_r ~ Beta(a, 1):
    P(p >= tau) = q = 1 - tau^a, the run is k < B with probability q^k (1 - q), B with q^B."""
    q = 1.0 - tau ** a
    pmf = np.array([q ** k * (1 - q) for k in range(B)] + [q ** B])
    n = np.maximum(np.arange(B + 1), 1)
    mean = float((pmf * n).sum())
    return mean, float((pmf * n * n).sum()) - mean * mean


def test_decode_loop_small_all_sequences():
    say("[loop] S=12 B=8 V=4096, 64 steps, tau 0.9 -> 0.6 at step 32")
    worst, _ = run_loop(4200, 12, 8, 28, 4, 128, 4096, 20, 200, 16, 64, 32)
    assert worst <= 2e-2


def test_full_size_decode_loop_sampled_sequences():
    """256 sequences, B = 8, prompt lengths U[128, 2048], V = 152064, 64 steps."""
    say("[loop] full size: S=256 B=8 V=152064, 64 steps, 4 sampled sequences")
    worst, accepted = run_loop(1005, 256, 8, 28, 4, 128, 152064, 128, 2048, 16, 64, 32,
                               sample=[0, 77, 128, 255])
    assert worst <= 2e-2
    # Each phase's mean accepted count per sequence against its closed form (about 1.2835
    # at tau 0.9 and 5.7314 at tau 0.6 with B = 8): 32 steps x 256 sequences = 8192 draws
    # per phase, within five standard errors of the law's variance.
    for phase, tau in enumerate((0.9, 0.6)):
        mean, var = accepted_count_law(tau, 8)
        got = accepted[phase] / (256 * 32)
        say(f"  tau {tau}: mean accepted {got:.4f}, closed form {mean:.4f}")
        assert abs(got - mean) <= 5 * np.sqrt(var / (256 * 32)), (tau, got, mean)

