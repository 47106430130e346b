"""Checks that pin the CPU oracle to facts outside itself.

Each check takes the oracle function(s) under test as arguments, so that the
mutation tests can hand in a deliberately broken copy and confirm the check
catches it. The checks rely only on: values printed on the pages, hand-worked
fixtures, closed forms derived from the mask equation, brute force on tiny
inputs, and library routines (torch CPU attention / softmax, exact integer
arithmetic in Python).
"""

from __future__ import annotations

import itertools
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_mask_fixture(name: str) -> np.ndarray:
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c == "1" for c in line])
    return np.array(rows, dtype=bool)


# ---------------------------------------------------------------- mask -----

def zero_based_visible(a: int, c: int, L: int, B: int) -> bool:
    """The 0-based interval form of the mask, written independently of the oracle."""
    if a < L:
        return c <= a
    t = a - L
    blk = t // B
    if c < L:
        return c < blk * B
    return blk * B <= c - L <= t


def check_mask_fixtures(build):
    for name, L, B in (("mask_L4_B2.txt", 4, 2), ("mask_L5_B2.txt", 5, 2)):
        want = load_mask_fixture(name)
        got = build(L, B)
        assert got.shape == want.shape, name
        assert np.array_equal(got, want), name


def check_mask_bruteforce(build, max_L: int = 24):
    for L in range(1, max_L + 1):
        for B in range(1, L + 1):
            M = build(L, B)
            n = 2 * L
            ref = np.array([[zero_based_visible(a, c, L, B) for c in range(n)]
                            for a in range(n)], dtype=bool)
            assert np.array_equal(M, ref), (L, B)


def check_mask_closed_forms(build, cases=((7, 3), (16, 4), (33, 8), (64, 16), (12, 1), (9, 9))):
    for L, B in cases:
        M = build(L, B)
        counts = M.sum(axis=1)
        # clean row a sees a + 1 keys; mask row t sees t + 1 keys, for every B
        assert np.array_equal(counts[:L], np.arange(1, L + 1)), (L, B)
        assert np.array_equal(counts[L:], np.arange(1, L + 1)), (L, B)
        assert int(M.sum()) == L * (L + 1)
        # the diagonal is always visible; no clean row ever sees the mask stream
        assert M.diagonal().all()
        assert not M[:L, L:].any()


def check_useful_pairs(count, cases=((1, 1), (5, 2), (7, 3), (16, 4), (33, 8), (12, 1),
                                      (9, 9), (64, 16), (10, 4))):
    """Visible (query, key) pairs per head: every MARS row a < L sees a + 1 keys and
    every mask row t sees t + 1 (whatever B is, B | L or not), so the mask holds
    L(L + 1) pairs; plain causal attention over 2L positions holds L(2L + 1)."""
    for L, B in cases:
        assert count(L, B, 0) == L * (L + 1), (L, B, "mars")
        assert count(L, B, 1) == L * (2 * L + 1), (L, B, "causal-2L")


def check_mask_b1(build, L: int = 11):
    M = build(L, 1)
    for t in range(L):
        vis = np.flatnonzero(M[L + t])
        want = list(range(t)) + [L + t]  # strictly earlier clean tokens, plus itself
        assert list(vis) == want, t


def check_mask_bL(build, L: int = 10):
    M = build(L, L)
    assert not M[L:, :L].any()
    assert np.array_equal(M[L:, L:], np.tril(np.ones((L, L), dtype=bool)))


# ------------------------------------------------------------ attention ----

def sdpa_causal(q, k, v, scale):
    """Library reference: torch CPU scaled_dot_product_attention, causal, float64."""
    Q = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))[None]
    K = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))[None]
    V = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))[None]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    return o[0].numpy()


def rand_qkv(seed, b, L, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, 2 * L, Hq, d)), rng.standard_normal((b, 2 * L, Hkv, d)),
            rng.standard_normal((b, 2 * L, Hkv, d)))


def check_clean_half_is_causal(attn, L=24, B=4, Hq=4, Hkv=2, d=16):
    q, k, v = rand_qkv(1, 2, L, Hq, Hkv, d)
    scale = 1.0 / np.sqrt(d)
    outs, _ = attn(q, k, v, L, B)
    g = Hq // Hkv
    for (bi, h), o in outs.items():
        ref = sdpa_causal(q[bi, :L, h], k[bi, :L, h // g], v[bi, :L, h // g], scale)
        np.testing.assert_allclose(o[:L], ref, atol=1e-12, rtol=0)


def check_bL_mask_half_is_causal(attn, L=16, Hq=2, Hkv=1, d=8):
    q, k, v = rand_qkv(2, 1, L, Hq, Hkv, d)
    scale = 1.0 / np.sqrt(d)
    outs, _ = attn(q, k, v, L, L)
    for (bi, h), o in outs.items():
        ref = sdpa_causal(q[bi, L:, h], k[bi, L:, 0], v[bi, L:, 0], scale)
        np.testing.assert_allclose(o[L:], ref, atol=1e-12, rtol=0)


def check_rows_by_gather(attn, L=20, B=3, Hq=6, Hkv=2, d=8, mask_mode=0):
    """Each output row equals torch.softmax attention over the keys it may see."""
    q, k, v = rand_qkv(3, 2, L, Hq, Hkv, d)
    scale = 0.37
    outs, lses = attn(q, k, v, L, B, scale=scale, mask_mode=mask_mode)
    g = Hq // Hkv
    for (bi, h), o in outs.items():
        for a in range(2 * L):
            if mask_mode == 0:
                keys = [c for c in range(2 * L) if zero_based_visible(a, c, L, B)]
            else:
                keys = list(range(a + 1))
            Q = torch.from_numpy(q[bi, a, h])
            K = torch.from_numpy(k[bi, keys, h // g])
            Vv = torch.from_numpy(v[bi, keys, h // g])
            s = (K @ Q) * scale
            ref = torch.softmax(s, dim=0) @ Vv
            np.testing.assert_allclose(o[a], ref.numpy(), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lses[(bi, h)][a], torch.logsumexp(s, 0).item(),
                                       atol=1e-12, rtol=0)


def check_single_key_rows(attn, L=12, B=4, d=8):
    """Clean row 0 and mask row t = 0 see exactly one key: their output is V there."""
    q, k, v = rand_qkv(4, 1, L, 1, 1, d)
    outs, _ = attn(q, k, v, L, B)
    o = outs[(0, 0)]
    np.testing.assert_allclose(o[0], v[0, 0, 0], atol=1e-14, rtol=0)
    np.testing.assert_allclose(o[L], v[0, L, 0], atol=1e-14, rtol=0)


def check_gqa_head_map(attn, L=8, B=2, d=4):
    """q-head h reads KV head h // (Hq / Hkv): equals the run with K/V repeated per head."""
    q, k, v = rand_qkv(7, 1, L, 6, 2, d)
    rep = lambda x: np.repeat(x, 3, axis=2)  # kv head j serves q heads 3j, 3j+1, 3j+2
    a, _ = attn(q, k, v, L, B)
    b, _ = attn(q, rep(k), rep(v), L, B)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], atol=1e-14, rtol=0)


# ------------------------------------------------------------- decode ------

# ---------------------------------------------------------- causal prefill -

def check_causal_vs_sdpa(causal, T=23, Hq=4, Hkv=2, d=8, seed=21):
    """Library reference: torch CPU causal scaled_dot_product_attention, any length."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, T, Hq, d))
    k = rng.standard_normal((2, T, Hkv, d))
    v = rng.standard_normal((2, T, Hkv, d))
    outs, lses = causal(q, k, v)
    g = Hq // Hkv
    for (bi, h), o in outs.items():
        np.testing.assert_allclose(o, sdpa_causal(q[bi, :, h], k[bi, :, h // g],
                                                  v[bi, :, h // g], 1 / np.sqrt(d)),
                                   atol=1e-12, rtol=0)
        # lse: natural log of the sum of exp of the scaled causal scores, row by row
        s = (q[bi, :, h] @ k[bi, :, h // g].T) / np.sqrt(d)
        ref = np.array([np.log(np.exp(s[i, :i + 1]).sum()) for i in range(T)])
        np.testing.assert_allclose(lses[(bi, h)], ref, atol=1e-12, rtol=0)


def check_causal_equals_mode1(causal, attn, L=9, Hq=2, Hkv=1, d=4, seed=22):
    """For an even length 2L the prefill equals the two-stream kernel's causal mode."""
    q, k, v = rand_qkv(seed, 1, L, Hq, Hkv, d)
    a, la = causal(q, k, v)
    b, lb = attn(q, k, v, L, 3, mask_mode=1)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], atol=1e-12, rtol=0)
        np.testing.assert_allclose(la[key], lb[key], atol=1e-12, rtol=0)


# ------------------------------------------------------- attention backward -

def _forward_full(attn, q, k, v, L, B, mask_mode):
    """The forward oracle's output as one [b, 2L, Hq, d] array."""
    outs, _ = attn(q, k, v, L, B, mask_mode=mask_mode)
    o = np.zeros(q.shape)
    for (bi, h), val in outs.items():
        o[bi, :, h] = val
    return o


def check_backward_finite_differences(attn, bwd, L=6, B=2, Hq=4, Hkv=2, d=4, mask_mode=0,
                                      seed=11):
    """dLoss/dq, dk, dv of Loss = sum(do * O(q, k, v)) against central differences
    of the (separately pinned) forward, entry by entry, in float64."""
    q, k, v = rand_qkv(seed, 1, L, Hq, Hkv, d)
    do = np.random.default_rng(seed + 1).standard_normal(q.shape)
    dq, dk, dv = bwd(q, k, v, do, L, B, mask_mode=mask_mode)
    h = 1e-5

    def loss(qq, kk, vv):
        return float(np.sum(do * _forward_full(attn, qq, kk, vv, L, B, mask_mode)))

    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{"qq": args_p["q"], "kk": args_p["k"], "vv": args_p["v"]})
                        - loss(**{"qq": args_m["q"], "kk": args_m["k"], "vv": args_m["v"]})) / (2 * h)
        np.testing.assert_allclose(grad, num, atol=1e-7, rtol=0, err_msg=f"d{name}")


def check_backward_vs_torch_autograd(bwd, L=10, B=3, Hq=6, Hkv=2, d=8, mask_mode=0, seed=12):
    """Library reference: torch CPU autograd through dense softmax attention whose mask
    is the independently written 0-based interval form (float64)."""
    q, k, v = rand_qkv(seed, 2, L, Hq, Hkv, d)
    do = np.random.default_rng(seed + 1).standard_normal(q.shape)
    n = 2 * L
    if mask_mode == 0:
        vis = np.array([[zero_based_visible(a, c, L, B) for c in range(n)] for a in range(n)])
    else:
        vis = np.tril(np.ones((n, n), dtype=bool))
    g = Hq // Hkv
    Q = torch.tensor(q, requires_grad=True)
    K = torch.tensor(k, requires_grad=True)
    V = torch.tensor(v, requires_grad=True)
    Kx = K.repeat_interleave(g, dim=2)
    Vx = V.repeat_interleave(g, dim=2)
    s = torch.einsum("bqhd,bkhd->bhqk", Q, Kx) / np.sqrt(d)
    s = s.masked_fill(~torch.from_numpy(vis), float("-inf"))
    o = torch.einsum("bhqk,bkhd->bqhd", torch.softmax(s, dim=-1), Vx)
    (o * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = bwd(q, k, v, do, L, B, mask_mode=mask_mode)
    np.testing.assert_allclose(dq, Q.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, K.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, V.grad.numpy(), atol=1e-11, rtol=0)


def check_backward_groups_and_chunks(bwd, L=9, B=2, Hq=4, Hkv=2, d=6, seed=13):
    """Restricting to one (batch, KV head) group, or processing rows in small chunks,
    gives the same numbers as the full call on the entries it fills."""
    q, k, v = rand_qkv(seed, 2, L, Hq, Hkv, d)
    do = np.random.default_rng(seed + 1).standard_normal(q.shape)
    full = bwd(q, k, v, do, L, B)
    part = bwd(q, k, v, do, L, B, groups=[(1, 0)], row_chunk=5)
    np.testing.assert_allclose(part[0][1, :, 0:2], full[0][1, :, 0:2], atol=1e-12, rtol=0)
    np.testing.assert_allclose(part[1][1, :, 0], full[1][1, :, 0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(part[2][1, :, 0], full[2][1, :, 0], atol=1e-12, rtol=0)
    assert not part[0][0].any() and not part[1][:, :, 1].any()


def paged_layout(kv_rows: np.ndarray, page_size: int, seed: int, total_pages: int | None = None):
    """Scatter logical rows [n, Hkv, d] into pages; returns (K pages, V^T pages, table)."""
    n, Hkv, d = kv_rows.shape
    pages_needed = max(1, -(-n // page_size))
    total = total_pages or pages_needed + 3
    rng = np.random.default_rng(seed)
    table = rng.permutation(total)[:pages_needed]
    K = rng.standard_normal((total, Hkv, page_size, d))
    for pos in range(n):
        K[table[pos // page_size], :, pos % page_size, :] = kv_rows[pos]
    return K, table


def check_decode_matches_causal_sdpa(decode, S=3, B=4, Hq=4, Hkv=2, d=8, page=4):
    rng = np.random.default_rng(5)
    lens = np.array([0, 5, 13])[:S]
    max_pages = 5
    num_pages = S * max_pages
    table = rng.permutation(num_pages).reshape(S, max_pages).astype(np.int32)
    Kc = rng.standard_normal((num_pages, Hkv, page, d))
    Vc = rng.standard_normal((num_pages, Hkv, d, page))
    q = rng.standard_normal((S, B, Hq, d))
    kn = rng.standard_normal((S, B, Hkv, d))
    vn = rng.standard_normal((S, B, Hkv, d))
    out = decode(q, kn, vn, Kc, Vc, table, lens, page)
    g = Hq // Hkv
    for s in range(S):
        n = int(lens[s])
        for h in range(Hq):
            kv = h // g
            keys = [Kc[table[s, p // page], kv, p % page] for p in range(n)]
            vals = [Vc[table[s, p // page], kv, :, p % page] for p in range(n)]
            Kall = np.array(keys + list(kn[s, :, kv])).reshape(n + B, d)
            Vall = np.array(vals + list(vn[s, :, kv])).reshape(n + B, d)
            # queries sit at positions n..n+B-1 of the sequence [prefix; new]
            Qall = np.concatenate([np.zeros((n, d)), q[s, :, h]], axis=0)
            ref = sdpa_causal(Qall, Kall, Vall, 1.0 / np.sqrt(d))[n:]
            np.testing.assert_allclose(out[s, :, h], ref, atol=1e-12, rtol=0)


def check_decode_equals_two_stream(attn, decode, L=24, B=4, Hq=4, Hkv=2, d=8, page=4):
    """Mask rows of block b == decode over cache = clean K/V[0:bB] + that block's rows."""
    q, k, v = rand_qkv(6, 1, L, Hq, Hkv, d)
    outs, _ = attn(q, k, v, L, B)
    nblk = L // B
    for blk in range(nblk):
        n = blk * B
        Kc, table = paged_layout(k[0, :n], page, seed=blk)
        Vrows, _ = paged_layout(v[0, :n], page, seed=blk)
        Vc = np.ascontiguousarray(Vrows.transpose(0, 1, 3, 2))
        rows = slice(L + blk * B, L + blk * B + B)
        out = decode(q[0, rows][None], k[0, rows][None], v[0, rows][None], Kc, Vc,
                     table[None].astype(np.int32), np.array([n]), page)
        for h in range(Hq):
            np.testing.assert_allclose(out[0, :, h], outs[(0, h)][rows], atol=1e-12, rtol=0)


# --------------------------------------------------------- confidence ------

def check_confidence_closed_forms(conf_row):
    V = 1000
    i, p = conf_row(np.zeros(V))
    assert i == 0 and abs(p - 1.0 / V) < 1e-15
    for a, pos in ((3.0, 17), (-2.0, 999), (10.0, 0), (-1.0, 0)):
        row = np.zeros(V)
        row[pos] = a
        i, p = conf_row(row)
        if a > 0:
            want_i, want_p = pos, np.exp(a) / (np.exp(a) + V - 1)
        else:
            want_i, want_p = (0 if pos != 0 else 1), 1.0 / (V - 1 + np.exp(a))
        assert i == want_i, (a, pos, i)
        assert abs(p - want_p) < 1e-14
    row = np.random.default_rng(0).standard_normal(V)
    row[[5, 600]] = row.max() + 1.0
    assert conf_row(row)[0] == 5  # ties go to the lowest id


def check_confidence_vs_torch(conf_row, seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        row = rng.standard_normal(5000) * rng.uniform(0.1, 6.0) + rng.uniform(-50, 50)
        i, p = conf_row(row)
        t = torch.from_numpy(row)
        assert i == int(torch.argmax(t))
        assert abs(p - torch.softmax(t, 0).max().item()) < 1e-14


# --------------------------------------------------------- acceptance -------

def leading_run_by_string(flags) -> int:
    s = "".join("1" if f else "0" for f in flags)
    return len(s) - len(s.lstrip("1"))


def check_accept_truth_table(accept_count, max_B=8):
    for B in range(1, max_B + 1):
        for flags in itertools.product((False, True), repeat=B):
            p = [0.95 if f else 0.85 for f in flags]
            want = max(1, leading_run_by_string(flags))
            assert accept_count(p, 0.9) == want, (B, flags)


def check_accept_rules(accept_count):
    assert accept_count([0.9, 0.9, 0.9], 0.9) == 3       # p == tau is accepted (>=)
    assert accept_count([0.95, 0.97, 0.5, 0.99], 0.9) == 2  # stop at the first miss
    assert accept_count([0.2, 0.99, 0.99], 0.9) == 1     # the first token is forced
    assert accept_count([0.999999, 0.9999], 1.0) == 1    # tau = 1 behaves as plain AR
    rng = np.random.default_rng(1)
    for _ in range(200):
        p = rng.random(8)
        assert accept_count(p, float(p.min())) == 8      # tau <= min p accepts all B
        taus = np.sort(rng.random(10))
        ns = [accept_count(p, t) for t in taus]
        assert all(a >= b for a, b in zip(ns, ns[1:]))   # non-increasing in tau


# ------------------------------------------------------------ commit --------

def check_commit_example(commit):
    with open(os.path.join(GOLDEN, "commit_example.json")) as f:
        ex = json.load(f)
    P, ps, Hkv, d, B = 4, ex["page_size"], 2, 3, ex["B"]
    rng = np.random.default_rng(0)
    kc = rng.standard_normal((P, Hkv, ps, d))
    vc = rng.standard_normal((P, Hkv, d, ps))
    kn = rng.standard_normal((1, B, Hkv, d))
    vn = rng.standard_normal((1, B, Hkv, d))
    table = np.array([ex["block_table"]], dtype=np.int32)
    k2, v2, ln, pos = commit(kc, vc, table, np.array([ex["cache_len"]]), kn, vn,
                             np.array([ex["n_accepted"]]), ps)
    assert list(pos[0]) == ex["commit_pos"]
    assert int(ln[0]) == ex["cache_len_after"]
    touched = set()
    for r, (pg, sl) in enumerate(zip(ex["page_of_row"], ex["slot_of_row"])):
        np.testing.assert_array_equal(k2[pg, :, sl, :], kn[0, r])
        np.testing.assert_array_equal(v2[pg, :, :, sl], vn[0, r])
        touched.add((pg, sl))
    for pg in range(P):
        for sl in range(ps):
            if (pg, sl) not in touched:
                np.testing.assert_array_equal(k2[pg, :, sl, :], kc[pg, :, sl, :])
                np.testing.assert_array_equal(v2[pg, :, :, sl], vc[pg, :, :, sl])


# ------------------------------------------------------------ LM head -------

def check_lmhead_exact_integers(lmhead):
    rng = np.random.default_rng(0)
    N, D, V = 3, 7, 5
    h = rng.integers(-8, 9, size=(N, D))
    w = rng.integers(-8, 9, size=(V, D))
    got = lmhead(h.astype(np.float32), w.astype(np.float32))
    assert got.shape == (N, V)
    for n in range(N):
        for vv in range(V):
            assert got[n, vv] == sum(int(h[n, k]) * int(w[vv, k]) for k in range(D))


# ------------------------------------------------ batch-synchronous block cache ----

def check_block_sync_example(step):
    """The hand-worked four-step example, both policies."""
    with open(os.path.join(GOLDEN, "block_sync_example.json")) as f:
        ex = json.load(f)
    S, B, Bc = ex["S"], ex["B"], ex["B_cache"]
    tau = np.full(S, ex["tau"], dtype=np.float32)
    for policy in ("min", "wait"):
        want = ex[policy]
        u = np.zeros(S, dtype=np.int32)
        toks = np.full((S, Bc), -1, dtype=np.int32)
        for t, p in enumerate(ex["p_max"]):
            ids = np.array([[100 * t + 10 * s + i for i in range(B)] for s in range(S)],
                           dtype=np.int32)
            keep, u, toks, froze, nrows = step(np.array(p, dtype=np.float32), ids, tau, u, toks,
                                               Bc, policy)
            assert froze == want["froze"][t], (policy, t)
            assert list(keep) == want["kept"][t], (policy, t, list(keep))
            assert list(u) == want["unfrozen"][t], (policy, t, list(u))
            assert toks.tolist() == want["block_tokens"][t], (policy, t)
            assert list(nrows) == [x + B for x in want["unfrozen"][t]]


def check_block_sync_advance_closed_forms(advance):
    rng = np.random.default_rng(11)
    for _ in range(300):
        S = int(rng.integers(1, 7))
        Bc = int(rng.integers(1, 33))
        n = rng.integers(1, 9, size=S)
        u = rng.integers(0, Bc + 1, size=S)
        room = Bc - u
        w = advance(n, u, Bc, "wait")
        m = advance(n, u, Bc, "min")
        # never past the block boundary, never more than accepted, never negative
        for a in (w, m):
            assert np.all(a >= 0) and np.all(a <= room) and np.all(a <= n)
        # with room for every accepted token, "wait" is plain per-sequence acceptance
        ok = room >= n
        assert np.array_equal(w[ok], n[ok])
        # "min" keeps the batch minimum wherever the block has room for it
        fit = room >= n.min()
        assert np.all(m[fit] == n.min())
        assert np.array_equal(m[~fit], room[~fit])
        # one sequence: the two policies coincide
        if S == 1:
            assert np.array_equal(w, m)
        # equal progress stays equal under "min"
        ue = np.full(S, u[0])
        me = advance(n, ue, Bc, "min")
        assert np.all(me == me[0])


def check_block_sync_token_stream(step):
    """Random runs: each sequence's token stream (frozen blocks, then the open
    block) is the concatenation of its kept ids; under "min" the batch stays
    in step; a block freezes exactly when every sequence has filled it."""
    rng = np.random.default_rng(12)
    for policy in ("min", "wait"):
        for _ in range(20):
            S = int(rng.integers(1, 6))
            B = int(rng.integers(1, 6))
            Bc = int(rng.integers(1, 9))
            u = np.zeros(S, dtype=np.int32)
            toks = np.full((S, Bc), -1, dtype=np.int32)
            frozen = [[] for _ in range(S)]
            kept_all = [[] for _ in range(S)]
            for t in range(30):
                p = rng.uniform(0, 1, size=(S, B)).astype(np.float32)
                ids = rng.integers(0, 1000, size=(S, B)).astype(np.int32)
                tau = np.full(S, 0.3, dtype=np.float32)
                full_before = bool(np.all(u == Bc))
                before = toks.copy()
                keep, u, toks, froze, _ = step(p, ids, tau, u, toks, Bc, policy)
                assert froze == full_before
                if froze:
                    for s in range(S):
                        frozen[s] += before[s].tolist()
                for s in range(S):
                    kept_all[s] += ids[s, :keep[s]].tolist()
                assert np.all(u <= Bc)
                if policy == "min":
                    assert np.all(u == u[0]) and np.all(keep == keep[0])
                for s in range(S):
                    assert frozen[s] + toks[s, :u[s]].tolist() == kept_all[s]
                    assert np.all(toks[s, u[s]:] == -1)


def check_block_freeze(freeze):
    """All blocks full: rows 0..B_cache-1 land at positions cache_len + r, by a
    plain loop over rows here; any block not full: nothing changes."""
    rng = np.random.default_rng(13)
    S, R, Hkv, d, ps, Bc, P = 3, 7, 2, 3, 4, 5, 12
    kc = rng.standard_normal((P, Hkv, ps, d))
    vc = rng.standard_normal((P, Hkv, d, ps))
    table = rng.permutation(P).astype(np.int32).reshape(S, 4)
    lens = np.array([0, 3, 8], dtype=np.int32)
    kr = rng.standard_normal((S, R, Hkv, d))
    vr = rng.standard_normal((S, R, Hkv, d))
    k2, v2, l2, froze = freeze(kc, vc, table, lens, kr, vr, np.array([Bc, Bc, Bc]), Bc, ps)
    assert froze and list(l2) == [Bc, 3 + Bc, 8 + Bc]
    kw, vw = kc.copy(), vc.copy()
    for s in range(S):
        for r in range(Bc):
            pos = lens[s] + r
            kw[table[s, pos // ps], :, pos % ps, :] = kr[s, r]
            vw[table[s, pos // ps], :, :, pos % ps] = vr[s, r]
    np.testing.assert_array_equal(k2, kw)
    np.testing.assert_array_equal(v2, vw)
    k3, v3, l3, froze = freeze(kc, vc, table, lens, kr, vr, np.array([Bc, Bc - 1, Bc]), Bc, ps)
    assert not froze and np.array_equal(l3, lens)
    np.testing.assert_array_equal(k3, kc)
    np.testing.assert_array_equal(v3, vc)


def check_block_decode_rows_vs_causal(fn, attn_causal):
    """Row r of a sequence with n frozen prefix rows is position n + r of plain
    causal attention over prefix + new rows (the prefix written into pages by
    a plain loop here); rows past n_rows[s] play no part."""
    rng = np.random.default_rng(14)
    S, R, Hq, Hkv, d, ps = 3, 6, 4, 2, 8, 4
    lens = np.array([0, 5, 9], dtype=np.int32)
    n_rows = np.array([6, 2, 4], dtype=np.int32)
    max_pages = 4
    table = rng.permutation(S * max_pages).astype(np.int32).reshape(S, max_pages)
    kc = rng.standard_normal((S * max_pages, Hkv, ps, d))
    vc = rng.standard_normal((S * max_pages, Hkv, d, ps))
    q = rng.standard_normal((S, R, Hq, d))
    kn = rng.standard_normal((S, R, Hkv, d))
    vn = rng.standard_normal((S, R, Hkv, d))
    kfull = [rng.standard_normal((int(lens[s]), Hkv, d)) for s in range(S)]
    vfull = [rng.standard_normal((int(lens[s]), Hkv, d)) for s in range(S)]
    for s in range(S):
        for pos in range(int(lens[s])):
            kc[table[s, pos // ps], :, pos % ps, :] = kfull[s][pos]
            vc[table[s, pos // ps], :, :, pos % ps] = vfull[s][pos]
    out = fn(q, kn, vn, kc, vc, table, lens, n_rows, ps)
    for s in range(S):
        n, Rs = int(lens[s]), int(n_rows[s])
        assert out[s].shape == (Rs, Hq, d)
        K = np.concatenate([kfull[s], kn[s, :Rs]])[None]
        V = np.concatenate([vfull[s], vn[s, :Rs]])[None]
        Q = np.concatenate([rng.standard_normal((n, Hq, d)), q[s, :Rs]])[None]
        ref, _ = attn_causal(Q, K, V)
        for h in range(Hq):
            np.testing.assert_allclose(out[s][:, h], ref[(0, h)][n:], rtol=1e-12, atol=1e-12)

