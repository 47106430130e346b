"""GPU parity: block-decode attention over the paged KV cache (bf16, tol 2e-2)."""

import numpy as np
import pytest
import torch

import block_masked_causal_amd as mars
import oracle
import synth
from tests.gpu_util import DEV, from_dev, max_abs, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-2


def dev_inputs(d):
    return (to_dev(d.q), to_dev(d.k_new), to_dev(d.v_new), to_dev(d.k_cache), to_dev(d.v_cache),
            to_dev(d.block_table), to_dev(d.cache_len))


def run(seed, S, B, Hq, Hkv, D, lo, hi, page, seqs=None, lens=None):
    say(f"[decode] seed={seed} S={S} B={B} Hq={Hq} Hkv={Hkv} d={D} len=[{lo},{hi}] page={page}")
    d = synth.decode_inputs(seed, S, B, Hq, Hkv, D, lo, hi, page, extra_capacity=B)
    if lens is not None:
        d.cache_len[:] = np.asarray(lens, dtype=np.int32)
    q, kn, vn, kc, vc, bt, cl = dev_inputs(d)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = mars.mars_attn_block_decode(q, kn, vn, kc, vc, bt, cl, status=status)
    torch.cuda.synchronize()
    ref = oracle.attn_block_decode(d.q.f32, d.k_new.f32, d.v_new.f32, d.k_cache.f32,
                                   d.v_cache.f32, d.block_table, d.cache_len, page, seqs=seqs)
    og = from_dev(o)
    sel = slice(None) if seqs is None else list(seqs)
    return max_abs(og[sel], ref), int(status.item())


@pytest.mark.parametrize("S,B,Hq,Hkv,D,lo,hi,page", [
    (5, 4, 28, 4, 128, 0, 700, 16),    # ragged lengths incl. chunk tails, GQA 7
    (4, 8, 28, 4, 128, 1, 600, 16),    # B = 8: two packed query tiles
    (3, 4, 4, 2, 64, 30, 300, 32),     # d = 64, page 32
    (2, 1, 2, 1, 128, 0, 40, 16),      # B = 1
    (2, 32, 4, 1, 64, 5, 90, 16),      # B = 32, 128 packed rows
    (3, 8, 14, 2, 64, 0, 1500, 32),    # d = 64 with two query tiles (56 rows)
    # page sizes without a specialised instance: 48 (a page straddles the
    # 512-key wave boundary) and 64
    (4, 4, 28, 4, 128, 0, 2600, 48),
    (3, 8, 14, 2, 64, 0, 2600, 64),
])
def test_decode_matches_oracle(S, B, Hq, Hkv, D, lo, hi, page):
    err, st = run(3000 + S * 10 + B, S, B, Hq, Hkv, D, lo, hi, page)
    assert err <= TOL and st == 0, (err, st)


def test_decode_lengths_on_chunk_and_page_edges():
    """One query tile: 2048-key chunks split over 4 waves of 512 keys; lengths on both
    sides of page, wave and chunk boundaries."""
    lens = [0, 1, 15, 16, 31, 32, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047,
            2048, 2049]
    err, st = run(3100, len(lens), 4, 8, 2, 128, 0, 2060, 16, lens=lens)
    assert err <= TOL and st == 0, (err, st)


def test_decode_two_query_tiles_on_chunk_and_wave_edges():
    """B = 8 with 7 query heads per KV head: 56 packed rows in two query tiles, whose
    workgroup splits each 1024-key chunk between two waves of 512 keys; lengths on
    both sides of the wave and chunk boundaries."""
    lens = [0, 1, 511, 512, 513, 1023, 1024, 1025, 1535, 1536, 2047, 2048, 2049, 2600,
            8192, 9000, 12000]  # the last three: more than eight chunks
    err, st = run(3120, len(lens), 8, 28, 4, 128, 0, 12000, 16, lens=lens)
    assert err <= TOL and st == 0, (err, st)


def test_decode_more_than_eight_chunks():
    """Caches longer than eight chunks (one query tile: 4 waves x 512 keys = 2048-key
    chunks): the merge takes the chunk partials eight at a time and rescales across
    batches when a later batch raises a row's maximum (16384 keys = exactly eight
    chunks, then 9, 9, 10 and 18)."""
    lens = [16384, 16385, 18432, 20480, 36000]
    err, st = run(3400, len(lens), 4, 8, 2, 128, 0, 36000, 16, lens=lens)
    assert err <= TOL and st == 0, (err, st)


def test_decode_large_batch_on_chunk_and_wave_edges():
    """130 sequences x 8 KV heads, one packed row per KV head (2048-key chunks split
    over 4 waves of 512 keys); lengths sit on both sides of the wave, chunk and
    single-chunk boundaries."""
    rng = np.random.default_rng(3150)
    lens = rng.integers(0, 4400, size=130)
    lens[:18] = [0, 1, 511, 512, 513, 1023, 1024, 1025, 1535, 1536, 2047, 2048, 2049, 4095,
                 4096, 4097, 31, 32]
    seqs = list(range(0, 130, 9)) + list(range(1, 18))
    err, st = run(3150, 130, 1, 8, 8, 64, 0, 4400, 16, seqs=sorted(set(seqs)), lens=lens)
    assert err <= TOL and st == 0, (err, st)


def test_decode_equals_two_stream_mask_rows_on_gpu():
    """Mask rows of block b from the two-stream kernel == decode with cache = clean K/V[0:bB]."""
    L, B, Hq, Hkv, D = 256, 4, 8, 2, 128
    say("[decode] cross-check against the two-stream kernel")
    q, k, v = synth.two_stream_qkv(3200, 1, L, Hq, Hkv, D, "bf16")
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    o2 = mars.mars_attn_two_stream(Q, K, V, L, B)
    blocks = [0, 1, 17, 40, 63]
    page = 16
    max_pages = L // page
    S = len(blocks)
    num_pages = S * max_pages
    kc = torch.zeros((num_pages, Hkv, page, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((num_pages, Hkv, D, page), dtype=torch.bfloat16, device=DEV)
    table = torch.arange(num_pages, dtype=torch.int32, device=DEV).flip(0).reshape(S, max_pages)
    lens = torch.tensor([b * B for b in blocks], dtype=torch.int32, device=DEV)
    for s, b in enumerate(blocks):
        for pos in range(b * B):
            pg = int(table[s, pos // page])
            kc[pg, :, pos % page, :] = K[0, pos]
            vc[pg, :, :, pos % page] = V[0, pos]
    rows = torch.stack([torch.arange(L + b * B, L + b * B + B) for b in blocks]).to(DEV)
    qd = Q[0][rows].contiguous()
    kd = K[0][rows].contiguous()
    vd = V[0][rows].contiguous()
    od = mars.mars_attn_block_decode(qd, kd, vd, kc, vc, table, lens)
    torch.cuda.synchronize()
    want = from_dev(o2[0][rows])
    assert max_abs(from_dev(od), want) <= TOL


@pytest.mark.parametrize("bad_page", [0, 40, 100])
def test_decode_flags_bad_page_and_overflow_without_faulting(bad_page):
    """A bad page id in the first, second or fourth 512-key part of sequence 1's first
    chunk (the wave holding it flags it and masks its keys), and a cache_len longer
    than the pages sequence 2 owns."""
    say(f"[decode] status flags for a bad page id (page {bad_page}) and an over-long cache_len")
    d = synth.decode_inputs(3300, 3, 4, 8, 2, 128, 20, 1800, 16, extra_capacity=4)
    d.cache_len[:2] = [45, 1700]
    q, kn, vn, kc, vc, bt, cl = dev_inputs(d)
    bt[1, bad_page] = -5          # bad page id in sequence 1
    cl[2] = bt.shape[1] * 16 + 7  # longer than the pages sequence 2 owns
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = mars.mars_attn_block_decode(q, kn, vn, kc, vc, bt, cl, status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st & mars.STATUS_BAD_PAGE and st & mars.STATUS_CACHE_OVERFLOW
    ref = oracle.attn_block_decode(d.q.f32, d.k_new.f32, d.v_new.f32, d.k_cache.f32,
                                   d.v_cache.f32, d.block_table, d.cache_len, 16, seqs=[0])
    assert max_abs(from_dev(o)[0:1], ref) <= TOL  # untouched sequences stay exact
    # sequence 1 equals the same sequence with the bad page's 16 keys left out
    table = d.block_table.copy()
    row = table[1]
    table[1] = np.concatenate([np.delete(row, bad_page), row[bad_page:bad_page + 1]])
    lens = d.cache_len.copy()
    lens[1] -= 16
    ref1 = oracle.attn_block_decode(d.q.f32, d.k_new.f32, d.v_new.f32, d.k_cache.f32,
                                    d.v_cache.f32, table, lens, 16, seqs=[1])
    assert max_abs(from_dev(o)[1:2], ref1) <= TOL


def test_full_size_qwen7b_decode_sampled_sequences():
    """64 sequences, cached lengths U[512, 4096], B = 4, 28/4 heads, d = 128, page 16."""
    seqs = [0, 17, 40, 63]
    err, st = run(1004, 64, 4, 28, 4, 128, 512, 4096, 16, seqs=seqs)
    assert err <= TOL and st == 0, err
