"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each mutant is a copy of an oracle function with one deliberate error: an
off-by-one in the block index, a dropped or loosened mask case, the wrong GQA
head map, a strict comparison, a missing floor, a shifted commit position, the
wrong tie-break, a transposed operand. Every one must be rejected by at least
one of the pin checks that the oracle itself passes.
"""

import numpy as np
import pytest

import oracle
from oracle import mars_oracle as om
from tests import pin_checks as pc

_build_mask = om.build_mask  # the unmutated original, captured before any patching


def _fails(check, *args, **kw):
    try:
        check(*args, **kw)
    except (AssertionError, IndexError, ValueError):
        return True
    return False


# -- mask mutants ------------------------------------------------------------

def mask_ceil_on_zero_based(L, B):
    n = 2 * L
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bi, bjm, bjc = -(-(i - L) // B), -(-(j - L) // B), -(-j // B)  # 0-based with ceil
    return (((i < L) & (j < L) & (j <= i)) | ((i >= L) & (j >= L) & (bi == bjm) & (j <= i))
            | ((i >= L) & (j < L) & (bjc < bi)))


def mask_case3_le(L, B):
    M = _build_mask(L, B)
    n = 2 * L
    for i in range(L + 1, n + 1):
        for j in range(1, L + 1):
            if om.beta(j, B) <= om.beta(i - L, B):
                M[i - 1, j - 1] = True
    return M


def mask_bidirectional_block(L, B):
    M = _build_mask(L, B)
    n = 2 * L
    for i in range(L + 1, n + 1):
        for j in range(L + 1, n + 1):
            if om.beta(i - L, B) == om.beta(j - L, B):
                M[i - 1, j - 1] = True
    return M


def mask_no_self(L, B):
    M = _build_mask(L, B)
    for a in range(L, 2 * L):
        M[a, a] = False
    return M


@pytest.mark.parametrize("mutant", [mask_ceil_on_zero_based, mask_case3_le,
                                    mask_bidirectional_block, mask_no_self])
def test_mask_mutants_are_caught(mutant):
    caught = (_fails(pc.check_mask_fixtures, mutant)
              or _fails(pc.check_mask_bruteforce, mutant, max_L=8)
              or _fails(pc.check_mask_closed_forms, mutant))
    assert caught


# -- attention mutants ---------------------------------------------------------

def test_wrong_gqa_map_is_caught(monkeypatch):
    def attn_mod_heads(q, k, v, L, B, scale=None, mask_mode=0, pairs=None, **kw):
        b, n, Hq, d = q.shape
        Hkv = k.shape[2]
        outs, lses = {}, {}
        for bi in range(b):
            for h in range(Hq):
                kk = np.repeat(k[:, :, [h % Hkv]], Hq, axis=2)  # h % Hkv instead of h // g
                vv = np.repeat(v[:, :, [h % Hkv]], Hq, axis=2)
                o, l = oracle.attn_two_stream(q, kk, vv, L, B, scale, mask_mode, pairs=[(bi, h)])
                outs[(bi, h)], lses[(bi, h)] = o[(bi, h)], l[(bi, h)]
        return outs, lses
    assert _fails(pc.check_clean_half_is_causal, attn_mod_heads)


def test_missing_scale_is_caught():
    def attn_noscale(q, k, v, L, B, scale=None, mask_mode=0, **kw):
        return oracle.attn_two_stream(q, k, v, L, B, scale=1.0, mask_mode=mask_mode, **kw)
    assert _fails(pc.check_clean_half_is_causal, attn_noscale)


def test_attention_with_mutant_mask_is_caught(monkeypatch):
    monkeypatch.setattr(om, "build_mask", mask_bidirectional_block)
    assert _fails(pc.check_rows_by_gather, oracle.attn_two_stream)


def test_decode_without_causal_new_rows_is_caught():
    def decode_full_block(q, k_new, v_new, k_cache, v_cache, table, lens, page, scale=None, seqs=None):
        S, B, Hq, d = q.shape
        Hkv = k_new.shape[2]
        g = Hq // Hkv
        out = np.empty((S, B, Hq, d))
        for s in range(S):
            n = int(lens[s])
            for kv in range(Hkv):
                Kp = om.gather_prefix(k_cache, table, s, n, page, kv, False)
                Vp = om.gather_prefix(v_cache, table, s, n, page, kv, True)
                K = np.concatenate([Kp, k_new[s, :, kv]])
                V = np.concatenate([Vp, v_new[s, :, kv]])
                for h in range(kv * g, (kv + 1) * g):
                    out[s, :, h], _ = om._softmax_attend(q[s, :, h], K, V, np.ones((B, n + B), bool),
                                                          1 / np.sqrt(d))
        return out
    assert _fails(pc.check_decode_matches_causal_sdpa, decode_full_block)


def test_decode_reading_v_untransposed_is_caught():
    def decode_v_as_k_layout(q, k_new, v_new, k_cache, v_cache, table, lens, page, **kw):
        vc = np.ascontiguousarray(v_cache.reshape(k_cache.shape))  # ignores the V^T page layout
        vt = np.ascontiguousarray(vc.transpose(0, 1, 3, 2))
        return oracle.attn_block_decode(q, k_new, v_new, k_cache, vt, table, lens, page)
    assert _fails(pc.check_decode_matches_causal_sdpa, decode_v_as_k_layout)


# -- confidence / acceptance / commit / lm-head mutants -------------------------

def test_last_index_tie_break_is_caught():
    def conf_last(row):
        row = np.asarray(row, dtype=np.float64)
        m = row.max()
        return int(np.flatnonzero(row == m)[-1]), float(1 / np.exp(row - m).sum())
    assert _fails(pc.check_confidence_closed_forms, conf_last)


def test_softmax_without_max_subtraction_in_log_domain_is_caught():
    def conf_wrong(row):
        row = np.asarray(row, dtype=np.float64)
        return int(np.argmax(row)), float(np.exp(row.max()) / np.exp(row).sum() * 1.0001)
    assert _fails(pc.check_confidence_vs_torch, conf_wrong)


def accept_strict(p, tau):
    n = 0
    while n < len(p) and p[n] > tau:
        n += 1
    return max(n, 1)


def accept_no_floor(p, tau):
    n = 0
    while n < len(p) and p[n] >= tau:
        n += 1
    return n


def accept_force_then_scan(p, tau):
    n = 1
    while n < len(p) and p[n] >= tau:
        n += 1
    return n


@pytest.mark.parametrize("mutant", [accept_strict, accept_no_floor, accept_force_then_scan])
def test_accept_mutants_are_caught(mutant):
    assert _fails(pc.check_accept_truth_table, mutant) or _fails(pc.check_accept_rules, mutant)


def test_commit_off_by_one_is_caught():
    def commit_shifted(kc, vc, table, lens, kn, vn, n, ps):
        return oracle.commit(kc, vc, table, np.asarray(lens) + 1, kn, vn, n, ps)
    assert _fails(pc.check_commit_example, commit_shifted)


def test_lmhead_transposed_is_caught():
    assert _fails(pc.check_lmhead_exact_integers, lambda h, w: (np.asarray(w, np.float64) @ np.asarray(h, np.float64).T))


# -- attention backward mutants ------------------------------------------------

def _bwd_mutant(kind):
    """A copy of the backward oracle with one planted mistake."""
    def bwd(q, k, v, do, L, B, scale=None, mask_mode=0, groups=None, row_chunk=1024):
        q = np.asarray(q)
        b, n, Hq, d = q.shape
        Hkv = k.shape[2]
        g = Hq // Hkv
        sc = 1.0 / np.sqrt(d) if scale is None else scale
        M = _build_mask(L, B) if mask_mode == 0 else om.causal_mask(n)
        dq = np.zeros((b, n, Hq, d))
        dk = np.zeros((b, n, Hkv, d))
        dv = np.zeros((b, n, Hkv, d))
        for bi in range(b):
            for h in range(Hq):
                kv = h // g
                K, V = k[bi, :, kv], v[bi, :, kv]
                Q, dO = q[bi, :, h], do[bi, :, h]
                s = np.where(M, (Q @ K.T) * sc, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = dO @ V.T
                if kind == "no_rowsum":
                    ds = p * dp
                else:
                    ds = p * (dp - (dO * (p @ V)).sum(axis=1, keepdims=True))
                dq[bi, :, h] = sc * (ds @ K)
                if kind == "gqa_first_head" and h % g:
                    continue
                dk[bi, :, kv] += (ds.T @ Q) * (1.0 if kind == "dk_unscaled" else sc)
                dv[bi, :, kv] += (ds.T @ dO) if kind == "dv_uses_ds" else (p.T @ dO)
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", ["no_rowsum", "dk_unscaled", "gqa_first_head", "dv_uses_ds"])
def test_backward_mutants_are_caught(kind):
    m = _bwd_mutant(kind)
    assert _fails(pc.check_backward_finite_differences, oracle.attn_two_stream, m, L=4, B=2,
                  Hq=2, Hkv=1, d=3)
    assert _fails(pc.check_backward_vs_torch_autograd, m)


def test_causal_prefill_mutants_are_caught():
    def causal_strict(q, k, v, scale=None, pairs=None):
        # a row may not see itself (the diagonal dropped); row 0 then sees key 0 only
        q = np.asarray(q)
        b, n, Hq, d = q.shape
        g = Hq // k.shape[2]
        sc = 1.0 / np.sqrt(d) if scale is None else scale
        M = np.tril(np.ones((n, n), dtype=bool), -1)
        M[0, 0] = True
        outs, lses = {}, {}
        for bi in range(b):
            for h in range(Hq):
                outs[(bi, h)], lses[(bi, h)] = om._softmax_attend(
                    q[bi, :, h], k[bi, :, h // g], v[bi, :, h // g], M, sc)
        return outs, lses

    def causal_unscaled(q, k, v, scale=None, pairs=None):
        return oracle.attn_causal(q, k, v, scale=1.0, pairs=pairs)

    assert _fails(pc.check_causal_vs_sdpa, causal_strict)
    assert _fails(pc.check_causal_vs_sdpa, causal_unscaled)


# -- batch-synchronous block cache mutants ------------------------------------

def _advance_mutant(kind):
    def adv(n_accepted, unfrozen, B_cache, policy="min"):
        n = np.asarray(n_accepted, dtype=np.int64)
        room = B_cache - np.asarray(unfrozen, dtype=np.int64)
        if kind == "room_plus_one":
            room = room + 1
        if policy == "min":
            pick = n.max() if kind == "max_not_min" else n.min()
            keep = pick if kind == "no_cap" else np.minimum(pick, room)
            keep = np.broadcast_to(keep, n.shape)
        else:
            keep = n if kind == "no_cap" else np.minimum(n, room)
        return np.asarray(keep, dtype=np.int32)
    return adv


@pytest.mark.parametrize("kind", ["max_not_min", "no_cap", "room_plus_one"])
def test_block_sync_advance_mutants_are_caught(kind, monkeypatch):
    adv = _advance_mutant(kind)
    assert _fails(pc.check_block_sync_advance_closed_forms, adv)
    monkeypatch.setattr(om, "block_sync_advance", adv)
    assert _fails(pc.check_block_sync_example, om.block_sync_step)


def _step_mutant(kind):
    def step(p_max, top_id, tau, unfrozen, block_tokens, B_cache, policy="min"):
        S, B = np.asarray(p_max).shape
        u = np.array(unfrozen, dtype=np.int32, copy=True)
        toks = np.array(block_tokens, dtype=np.int32, copy=True)
        full = np.any(u == B_cache) if kind == "freeze_on_any" else np.all(u == B_cache)
        froze = bool(full)
        if froze and kind != "no_reset":
            u[:] = 0
            toks[:] = -1
        n, _ = oracle.accept(p_max, top_id, tau)
        keep = oracle.block_sync_advance(n, u, B_cache, policy)
        for s in range(S):
            for i in range(int(keep[s])):
                at = i if kind == "write_at_zero" else u[s] + i
                if at < B_cache:
                    toks[s, at] = top_id[s][i]
            u[s] += keep[s]
        return keep, u, toks, froze, u + B
    return step


@pytest.mark.parametrize("kind", ["freeze_on_any", "no_reset", "write_at_zero"])
def test_block_sync_step_mutants_are_caught(kind):
    step = _step_mutant(kind)
    assert _fails(pc.check_block_sync_example, step)
    assert _fails(pc.check_block_sync_token_stream, step)


def test_block_freeze_on_any_full_is_caught():
    def freeze(k_cache, v_cache, block_table, cache_len, k_rows, v_rows, unfrozen, B_cache,
               page_size):
        if not np.any(np.asarray(unfrozen) == B_cache):
            return k_cache.copy(), v_cache.copy(), cache_len.copy(), False
        S = k_rows.shape[0]
        kc, vc, ln, _ = oracle.commit(k_cache, v_cache, block_table, cache_len,
                                      k_rows[:, :B_cache], v_rows[:, :B_cache],
                                      np.full(S, B_cache), page_size)
        return kc, vc, ln, True
    assert _fails(pc.check_block_freeze, freeze)


def test_block_decode_rows_mutants_are_caught():
    def all_rows(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_rows, page_size):
        full = oracle.attn_block_decode(q, k_new, v_new, k_cache, v_cache, block_table,
                                        cache_len, page_size)
        return {s: full[s] for s in range(q.shape[0])}

    def short_prefix(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_rows,
                     page_size):
        return oracle.attn_block_decode_rows(q, k_new, v_new, k_cache, v_cache, block_table,
                                             np.maximum(np.asarray(cache_len) - 1, 0), n_rows,
                                             page_size)
    assert _fails(pc.check_block_decode_rows_vs_causal, all_rows, oracle.attn_causal)
    assert _fails(pc.check_block_decode_rows_vs_causal, short_prefix, oracle.attn_causal)


def test_useful_pair_count_mutants_are_caught():
    def ignores_mode(L, B, mask_mode=0):
        return oracle.useful_pairs_two_stream(L, B, 0)

    def causal_over_L(L, B, mask_mode=0):
        return int(om.causal_mask(L).sum()) if mask_mode else oracle.useful_pairs_two_stream(L, B)

    def from_mask(mutant):
        def count(L, B, mask_mode=0):
            if mask_mode:
                return oracle.useful_pairs_two_stream(L, B, 1)
            return int(mutant(L, B).sum())
        count.__name__ = mutant.__name__
        return count

    for m in (ignores_mode, causal_over_L, from_mask(mask_case3_le), from_mask(mask_no_self)):
        assert _fails(pc.check_useful_pairs, m), m.__name__
