"""GPU parity: the no-cache causal prefill and the KV append that fills the
block-level cache from it.

Tolerances as for the two-stream attention (max-abs, inputs N(0, 1)): 1e-4 on
the fp32 path, 2e-2 on bf16 outputs, 1e-4 / 2e-3 on the LSE. The append moves
bytes only and must be bit-exact.
"""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import DEV, bf16_bits, from_dev, max_abs, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-3)}


def causal_case(seed, b, T, Hq, Hkv, d, dtype, pairs=None, rows=None):
    say(f"[causal] seed={seed} b={b} T={T} Hq={Hq} Hkv={Hkv} d={d} {dtype}")
    q, k, v = synth.sequence_qkv(seed, b, T, Hq, Hkv, d, dtype)
    o, lse = mars.mars_attn_causal(to_dev(q), to_dev(k), to_dev(v), return_lse=True)
    torch.cuda.synchronize()
    og, lg = from_dev(o), from_dev(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), "non-finite attention output"
    if rows is None:
        ref_o, ref_l = oracle.attn_causal(q.f32, k.f32, v.f32, pairs=pairs)
        sel = slice(None)
    else:  # sampled rows: the oracle on the prefix each row needs
        hi = max(rows) + 1
        ref_o, ref_l = oracle.attn_causal(q.f32[:, :hi], k.f32[:, :hi], v.f32[:, :hi],
                                          pairs=pairs)
        ref_o = {key: val[rows] for key, val in ref_o.items()}
        ref_l = {key: val[rows] for key, val in ref_l.items()}
        sel = rows
    eo = max(max_abs(og[bi, sel, h], ro) for (bi, h), ro in ref_o.items())
    el = max(max_abs(lg[bi, h, sel], ref_l[(bi, h)]) for (bi, h) in ref_o)
    return eo, el, (q, k, v, o, lse)


@pytest.mark.parametrize("b,T,Hq,Hkv,d,dtype", [
    (1, 1, 2, 1, 64, "bf16"),      # a single position
    (1, 9, 2, 2, 32, "f32"),
    (2, 101, 4, 2, 64, "f32"),     # odd, ragged last tile
    (2, 257, 4, 2, 64, "bf16"),    # odd: one row past four full tiles
    (1, 300, 4, 1, 128, "bf16"),
    (1, 129, 6, 3, 128, "bf16"),   # GQA group 2, odd
    (3, 64, 2, 2, 64, "bf16"),     # exactly one row tile
])
def test_causal_matches_oracle(b, T, Hq, Hkv, d, dtype):
    eo, el, _ = causal_case(3100 + T, b, T, Hq, Hkv, d, dtype)
    to, tl = TOL[dtype]
    assert eo <= to and el <= tl, (eo, el)


def test_causal_even_length_is_two_stream_causal_mode_bitwise():
    # for even T the causal entry is the two-stream call in its causal mode
    # with L = T / 2: the same launch, so the same bits
    say("[causal] T=512 vs two-stream mode 1, L=256")
    q, k, v = synth.sequence_qkv(3200, 2, 512, 4, 2, 64, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o1, l1 = mars.mars_attn_causal(qd, kd, vd, return_lse=True)
    o2, l2 = mars.mars_attn_two_stream(qd, kd, vd, 256, 4, mask_mode=1, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(o1), bf16_bits(o2))
    assert torch.equal(l1, l2)


def test_full_size_prefill_sampled():
    # Qwen2.5-0.5B attention shape (14 query heads, 2 KV heads, d = 64) over a
    # prompt plus one block of [MASK] rows of odd total length; sampled
    # (batch, head) pairs and rows, including the last row
    T = 4096 + 16 + 1
    pairs = synth.sample_pairs(3300, 2, 14, 3)
    rows = [0, 1, 63, 64, 1000, 2047, 2048, 4095, 4100, T - 1]
    eo, el, _ = causal_case(3300, 2, T, 14, 2, 64, "bf16", pairs=pairs, rows=rows)
    assert eo <= 2e-2 and el <= 2e-3, (eo, el)


def cache_bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def ref_bits(x, dtype):
    if dtype == "bf16":
        return synth.bf16_round(x).view(np.int16)
    return np.ascontiguousarray(x, dtype=np.float32).view(np.int32)


@pytest.mark.parametrize("S,T,Hkv,D,page,lo,hi,dtype", [
    (3, 5, 2, 32, 16, 0, 20, "f32"),
    (4, 70, 2, 64, 16, 0, 40, "bf16"),    # more than one 64-row chunk, ragged
    (2, 130, 1, 128, 64, 3, 3, "bf16"),
    (5, 1, 3, 64, 1, 0, 9, "bf16"),       # one-slot pages
    (3, 45, 2, 64, 12, 0, 30, "bf16"),    # page size not a multiple of 8: element stores
    (2, 200, 4, 128, 16, 5, 77, "f32"),   # 32-byte V runs, unaligned start
    (64, 2048, 4, 128, 16, 0, 0, "bf16"), # the benchmarked prompt append
])
def test_append_matches_commit_of_all_rows(S, T, Hkv, D, page, lo, hi, dtype):
    say(f"[append] S={S} T={T} Hkv={Hkv} D={D} page={page} {dtype}")
    d = synth.decode_inputs(3400 + T, S, 1, Hkv, Hkv, D, lo, hi, page, extra_capacity=T,
                            dtype=dtype)
    _, kr, vr = synth.decode_step_tensors(3401, 0, S, T, Hkv, Hkv, D, dtype)
    kc, vc = to_dev(d.k_cache), to_dev(d.v_cache)
    cl = to_dev(d.cache_len)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    mars.mars_kv_append(to_dev(kr), to_dev(vr), kc, vc, to_dev(d.block_table), cl, status=status)
    torch.cuda.synchronize()
    rk, rv, rl, _ = oracle.commit(d.k_cache.f32, d.v_cache.f32, d.block_table, d.cache_len,
                                  kr.f32, vr.f32, np.full(S, T), page)
    assert int(status.item()) == 0
    assert np.array_equal(cl.cpu().numpy(), rl)
    assert np.array_equal(cache_bits(kc), ref_bits(rk, dtype))
    assert np.array_equal(cache_bits(vc), ref_bits(rv, dtype))


def test_append_overflow_and_bad_page():
    say("[append] overflow / bad page: flagged, nothing written out of place")
    S, T, Hkv, D, page = 3, 40, 2, 64, 16
    d = synth.decode_inputs(3500, S, 1, Hkv, Hkv, D, 8, 8, page, extra_capacity=T,
                            dtype="bf16")
    cap = d.max_pages * page
    lens = np.array([cap - 10, 8, 8], dtype=np.int32)   # seq 0 has room for 10 rows
    table = d.block_table.copy()
    bad_slot = (8 + 20) // page                           # seq 1: page of its row 20
    table[1, bad_slot] = -3
    _, kr, vr = synth.decode_step_tensors(3501, 0, S, T, Hkv, Hkv, D, "bf16")
    kc, vc = to_dev(d.k_cache), to_dev(d.v_cache)
    cl = to_dev(lens)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    mars.mars_kv_append(to_dev(kr), to_dev(vr), kc, vc, to_dev(table), cl, status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st & mars.STATUS_CACHE_OVERFLOW and st & mars.STATUS_BAD_PAGE
    assert list(cl.cpu().numpy()) == [cap, 8 + T, 8 + T]
    # expected: the oracle's commit with seq 0 cut at its capacity and seq 1's
    # bad page pointed at a scratch page that is then dropped
    ext = d.num_pages
    kx = np.concatenate([d.k_cache.f32, np.zeros_like(d.k_cache.f32[:1])])
    vx = np.concatenate([d.v_cache.f32, np.zeros_like(d.v_cache.f32[:1])])
    table_x = table.copy()
    table_x[1, bad_slot] = ext
    rk, rv, _, _ = oracle.commit(kx, vx, table_x, lens, kr.f32, vr.f32,
                                 np.array([10, T, T]), page)
    assert np.array_equal(cache_bits(kc), ref_bits(rk[:ext], "bf16"))
    assert np.array_equal(cache_bits(vc), ref_bits(rv[:ext], "bf16"))


@pytest.mark.parametrize("P,B,Hq,Hkv,D,page", [
    (37, 4, 4, 2, 64, 16),
    (300, 16, 14, 2, 64, 64),    # Qwen2.5-0.5B heads
    (129, 8, 28, 4, 128, 32),    # Qwen2.5-7B heads
])
def test_prefill_then_block_decode_agree(P, B, Hq, Hkv, D, page):
    """A causal pass over prompt + B [MASK] rows, and the cached route (append
    the prompt's K/V, then block-decode the B rows against it), compute the
    same B output rows."""
    say(f"[prefill->decode] P={P} B={B} Hq={Hq} Hkv={Hkv} D={D} page={page}")
    S = 2
    T = P + B
    q, k, v = synth.sequence_qkv(3600 + P, S, T, Hq, Hkv, D, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_pref = mars.mars_attn_causal(qd, kd, vd)
    max_pages = -(-P // page)
    num_pages = S * max_pages
    table = np.random.default_rng(3601).permutation(num_pages).astype(np.int32).reshape(
        S, max_pages)
    kc = torch.zeros((num_pages, Hkv, page, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((num_pages, Hkv, D, page), dtype=torch.bfloat16, device=DEV)
    cl = torch.zeros(S, dtype=torch.int32, device=DEV)
    bt = to_dev(table)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    mars.mars_kv_append(kd[:, :P].contiguous(), vd[:, :P].contiguous(), kc, vc, bt, cl,
                        status=status)
    o_dec = mars.mars_attn_block_decode(qd[:, P:].contiguous(), kd[:, P:].contiguous(),
                                        vd[:, P:].contiguous(), kc, vc, bt, cl, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert list(cl.cpu().numpy()) == [P] * S
    a = from_dev(o_pref)[:, P:]
    bdec = from_dev(o_dec)
    ref, _ = oracle.attn_causal(q.f32, k.f32, v.f32)
    for s in range(S):
        for h in range(Hq):
            r = ref[(s, h)][P:]
            assert max_abs(a[s, :, h], r) <= 2e-2
            assert max_abs(bdec[s, :, h], r) <= 2e-2
    assert max_abs(a, bdec) <= 4e-2
