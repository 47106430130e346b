"""GPU parity: acceptance + KV commit into every layer's cache in one call.

The decision outputs (accepted counts, ids, commit positions, cache lengths)
and every cache byte of every layer must be bit-exact against the oracle's
acceptance and its commit applied layer by layer.
"""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import DEV, say, to_dev

pytestmark = pytest.mark.gpu

TAUS = np.array([0.5, 0.6, 0.9, 0.95, 1.0])


def bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def ref_bits(x, dtype):
    if dtype == "bf16":
        return synth.bf16_round(x).view(np.int16)
    return np.ascontiguousarray(x, dtype=np.float32).view(np.int32)


def beta_probs(rng, S, B):
    """p ~ Beta(5, 1), none within 1e-6 of a threshold in TAUS."""
    p = (rng.random((S, B)) ** 0.2).astype(np.float32)
    p[np.abs(p[:, :, None] - TAUS).min(-1) < 1e-6] = 0.3
    return p


@pytest.mark.parametrize("dtype,layers,S,B,Hkv,D,page", [
    ("bf16", 3, 24, 8, 4, 128, 16),
    ("f32", 2, 24, 8, 2, 64, 32),
    ("bf16", 4, 24, 8, 2, 8, 16),
    # 64 positions x 2 heads: the staged (head, row) pairs take two passes
    ("bf16", 2, 5, 64, 2, 64, 16),
    # rows too long to stage: element path
    ("f32", 2, 6, 8, 1, 4096, 16),
])
def test_layers_match_the_oracle_per_layer(dtype, layers, S, B, Hkv, D, page):
    say(f"[layers] {dtype} layers={layers} S={S} B={B} Hkv={Hkv} d={D} page={page}")
    rng = np.random.default_rng(4300 + D)
    d = synth.layered_commit_inputs(4300 + D, layers, S, B, Hkv, D, 0, 90, page,
                                    extra_capacity=B, dtype=dtype)
    p = beta_probs(rng, S, B)
    ids = rng.integers(0, 152064, size=(S, B)).astype(np.int32)
    tau = rng.choice(TAUS, size=S).astype(np.float32)
    kc, vc = to_dev(d.k_cache), to_dev(d.v_cache)
    cl = to_dev(d.cache_len)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    n, acc, pos = mars.mars_accept_commit_layers(
        to_dev(p), to_dev(ids), to_dev(tau), to_dev(d.k_new), to_dev(d.v_new), kc, vc,
        to_dev(d.block_table), cl, status=status)
    torch.cuda.synchronize()
    rn, racc = oracle.accept(p, ids, tau)
    assert np.array_equal(n.cpu().numpy(), rn)
    assert np.array_equal(acc.cpu().numpy(), racc)
    assert int(status.item()) == 0
    assert rn.max() > 1
    gk, gv = bits(kc), bits(vc)
    for layer in range(layers):
        rk, rv, rl, rpos = oracle.commit(d.k_cache.f32[layer], d.v_cache.f32[layer],
                                         d.block_table, d.cache_len, d.k_new.f32[layer],
                                         d.v_new.f32[layer], rn, page)
        assert np.array_equal(pos.cpu().numpy(), rpos)
        assert np.array_equal(cl.cpu().numpy(), rl)
        assert np.array_equal(gk[layer], ref_bits(rk, dtype)), layer
        assert np.array_equal(gv[layer], ref_bits(rv, dtype)), layer


def test_layers_agree_with_the_one_layer_call_on_overflow_and_bad_pages():
    say("[layers] overflow / bad page / NaN: same flags, lengths and bytes as one layer at a time")
    layers, S, B, Hkv, D, page = 2, 4, 4, 2, 32, 16
    d = synth.layered_commit_inputs(9, layers, S, B, Hkv, D, 5, 5, page, dtype="bf16")
    cap = d.max_pages * page
    lens = np.array([cap - 2, 5, 5, -1], dtype=np.int32)  # room for 2 rows; ok; ok; bad length
    table = d.block_table.copy()
    table[1, 0] = d.num_pages                               # sequence 1: page id out of range
    p = np.full((S, B), 0.99, dtype=np.float32)
    p[2, 2] = np.nan                                       # sequence 2 stops after 2 rows
    ids = np.arange(S * B, dtype=np.int32).reshape(S, B)
    tau = np.full(S, 0.5, dtype=np.float32)
    kc, vc = to_dev(d.k_cache), to_dev(d.v_cache)
    cl = to_dev(lens)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = mars.mars_accept_commit_layers(to_dev(p), to_dev(ids), to_dev(tau), to_dev(d.k_new),
                                         to_dev(d.v_new), kc, vc, to_dev(table), cl,
                                         status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st & mars.STATUS_CACHE_OVERFLOW and st & mars.STATUS_BAD_PAGE
    assert list(cl.cpu().numpy()) == [cap, 5, 7, -1]
    for layer in range(layers):
        kc1, vc1 = to_dev(d.k_cache)[layer].contiguous(), to_dev(d.v_cache)[layer].contiguous()
        cl1 = to_dev(lens)
        st1 = torch.zeros(1, dtype=torch.int32, device=DEV)
        one = mars.mars_accept_commit(to_dev(p), to_dev(ids), to_dev(tau),
                                      to_dev(d.k_new)[layer].contiguous(),
                                      to_dev(d.v_new)[layer].contiguous(), kc1, vc1,
                                      to_dev(table), cl1, status=st1)
        torch.cuda.synchronize()
        for a, b in zip(out, one):
            assert torch.equal(a, b)
        assert torch.equal(cl, cl1) and int(st1.item()) == st
        assert np.array_equal(bits(kc[layer]), bits(kc1)), layer
        assert np.array_equal(bits(vc[layer]), bits(vc1)), layer


def page_sums(cache):
    """Per-(layer, page) sums of the 16-bit patterns: a cheap fingerprint of every page."""
    L, P = cache.shape[0], cache.shape[1]
    return torch.stack([cache[l].view(torch.int16).reshape(P, -1).sum(dim=1, dtype=torch.int64)
                        for l in range(L)])


def test_full_size_28_layers_sampled_sequences():
    """28 layers x S = 256 x B = 8, 4 KV heads of 128, pages of 16, prompt lengths U[128, 2048].

    Two calls in a row: full acceptance (every row of every layer committed, about
    235 MB moved), then Beta(5, 1) confidences against tau = 0.9. The oracle
    replays both calls layer by layer for six sampled sequences (their pages
    only); over all sequences the committed rows must equal the new rows and no
    page outside the committed slots may change.
    """
    layers, S, B, Hkv, D, page = 28, 256, 8, 4, 128, 16
    lo, hi = 128, 2048
    rng = np.random.default_rng(1006)
    lens = rng.integers(lo, hi + 1, size=S).astype(np.int32)
    max_pages = -(-(hi + 2 * B) // page)
    num_pages = S * max_pages
    table = rng.permutation(num_pages).astype(np.int32).reshape(S, max_pages)
    say(f"[layers] full size: {layers} layers, S={S}, B={B}, {num_pages} pages per layer")
    g = torch.Generator(device=DEV)
    g.manual_seed(1006)
    kc = torch.randn((layers, num_pages, Hkv, page, D), generator=g, device=DEV,
                     dtype=torch.bfloat16)
    vc = torch.randn((layers, num_pages, Hkv, D, page), generator=g, device=DEV,
                     dtype=torch.bfloat16)
    bt, cl = to_dev(table), to_dev(lens)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    sample = [0, 1, 77, 128, 200, 255]
    pages = sorted(set(table[sample].ravel().tolist()))
    remap = {pg: i for i, pg in enumerate(pages)}
    sub_table = np.vectorize(remap.get)(table[sample]).astype(np.int32)
    pages_dev = torch.tensor(pages, device=DEV)
    olen = lens.copy()
    for call, (p, tau_v) in enumerate([(np.full((S, B), 0.99, np.float32), 0.5),
                                       (beta_probs(rng, S, B), 0.9)]):
        kn = torch.randn((layers, S, B, Hkv, D), generator=g, device=DEV, dtype=torch.bfloat16)
        vn = torch.randn((layers, S, B, Hkv, D), generator=g, device=DEV, dtype=torch.bfloat16)
        ids = rng.integers(0, 152064, size=(S, B)).astype(np.int32)
        tau = np.full(S, tau_v, dtype=np.float32)
        ok = kc[:, pages_dev].float().cpu().numpy()
        ov = vc[:, pages_dev].float().cpu().numpy()
        sums_k, sums_v = page_sums(kc), page_sums(vc)
        say(f"  call {call}: tau {tau_v}")
        n, acc, pos = mars.mars_accept_commit_layers(to_dev(p), to_dev(ids), to_dev(tau), kn, vn,
                                                     kc, vc, bt, cl, status=status)
        torch.cuda.synchronize()
        rn, racc = oracle.accept(p, ids, tau)
        assert np.array_equal(n.cpu().numpy(), rn)
        assert np.array_equal(acc.cpu().numpy(), racc)
        if call == 0:
            assert (rn == B).all()
        # positions and lengths of every sequence: the oracle's commit on a
        # one-element-per-row stand-in cache
        _, _, rl, rpos = oracle.commit(np.zeros((num_pages, 1, page, 1), np.float32),
                                       np.zeros((num_pages, 1, 1, page), np.float32), table,
                                       olen, np.zeros((S, B, 1, 1), np.float32),
                                       np.zeros((S, B, 1, 1), np.float32), rn, page)
        gpos = pos.cpu().numpy()
        assert np.array_equal(gpos, rpos)
        assert np.array_equal(cl.cpu().numpy(), rl)
        # sampled sequences: every byte of their pages, layer by layer
        knf, vnf = kn.float().cpu().numpy(), vn.float().cpu().numpy()
        gk, gv = bits(kc[:, pages_dev]), bits(vc[:, pages_dev])
        sub_len = olen[sample]
        for layer in range(layers):
            rk, rv, _, _ = oracle.commit(ok[layer], ov[layer], sub_table, sub_len,
                                         knf[layer][sample], vnf[layer][sample], rn[sample], page)
            assert np.array_equal(gk[layer], ref_bits(rk, "bf16")), (call, layer)
            assert np.array_equal(gv[layer], ref_bits(rv, "bf16")), (call, layer)
        # all sequences: committed rows hold the new rows; other pages unchanged
        s_idx, r_idx = np.nonzero(gpos >= 0)
        pp = gpos[s_idx, r_idx]
        pg = torch.from_numpy(table[s_idx, pp // page]).to(DEV).long()
        sl = torch.from_numpy(pp % page).to(DEV).long()
        si, ri = torch.from_numpy(s_idx).to(DEV), torch.from_numpy(r_idx).to(DEV)
        h = torch.arange(Hkv, device=DEV)
        dd = torch.arange(D, device=DEV)
        k_row = (pg[:, None] * Hkv + h) * page + sl[:, None]                 # [M, Hkv]
        v_el = ((pg[:, None, None] * Hkv + h[:, None]) * D + dd) * page + sl[:, None, None]
        assert torch.equal(kc.view(layers, -1, D)[:, k_row], kn[:, si, ri])
        assert torch.equal(vc.view(layers, -1)[:, v_el], vn[:, si, ri])
        touched = torch.zeros(num_pages, dtype=torch.bool, device=DEV)
        touched[pg] = True
        assert torch.equal(page_sums(kc)[:, ~touched], sums_k[:, ~touched])
        assert torch.equal(page_sums(vc)[:, ~touched], sums_v[:, ~touched])
        assert int(status.item()) == 0
        olen = rl
