"""Plain CPU oracle for the MARS hot path (TEST INFRASTRUCTURE ONLY).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module. The product path never calls it: it shares no code,
constants or helpers with the HIP library, and it imports nothing from it.

Everything is computed in float64 from the exact values the device receives
(bfloat16 inputs are upcast exactly), directly from the definitions on the
pages, with no tiling, fusion or reordering beyond what those definitions
state.

Pages cited (all titled "MARS: Enabling Autoregressive Models Multi-Token
Generation", by Jin, Wang, Luo and Sun):
  [notes]  the papernotes.org notes (NeurIPS 2026 entry), sections
           整体框架 (overall framework), 关键设计 1-4 (key designs 1-4),
           主实验 / 消融实验 tables;
  [gist]   the gist.science English explainer, sections 2A-2D and 4;
  [abs]    the chatpaper.ai abstract.

Readings taken where the pages are silent (each also listed in the design
notes): 0-based arrays, 1-based formulas; a mask row sees itself; softmax scale
1/sqrt(d); q-head h uses KV head floor(h / (Hq / Hkv)); confidence is the
temperature-1 softmax maximum over the full vocabulary with ties resolved to
the lowest token id; "at least one token" means n = max(1, leading run);
comparisons are p >= tau.

Parity-pin status: every function below is pinned by tests other than itself
(brute force, closed forms, library routines, printed values, central finite
differences for the attention gradient), useful_pairs_two_stream included (the
closed forms L(L+1) and L(2L+1)). None is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Two-stream structured mask            [notes] 关键设计 1, equation for M_ij
# ---------------------------------------------------------------------------


def beta(t: int, B: int) -> int:
    """Block index beta(t) = ceil(t / B) of a 1-based position t ([notes] 关键设计 1)."""
    return -(-t // B)


def build_mask_loops(L: int, B: int) -> np.ndarray:
    """The 2L x 2L visibility matrix, one entry at a time (tiny L only).

    Entry [i-1, j-1] is True where M_ij = 0 (visible) and False where
    M_ij = -inf, with i, j 1-based positions in z = [x; x~] and the four cases
    of the mask equation in [notes] 关键设计 1:
      1. i, j <= L and j <= i                          (clean stream, causal)
      2. i, j > L, beta(i-L) = beta(j-L), j <= i       (mask stream, causal in block)
      3. i > L, j <= L, beta(j) < beta(i-L)            (mask row sees earlier clean blocks)
      4. otherwise masked.
    """
    n = 2 * L
    M = np.zeros((n, n), dtype=bool)
    for i in range(1, n + 1):
        for j in range(1, n + 1):
            if i <= L and j <= L and j <= i:
                M[i - 1, j - 1] = True
            elif i > L and j > L and beta(i - L, B) == beta(j - L, B) and j <= i:
                M[i - 1, j - 1] = True
            elif i > L and j <= L and beta(j, B) < beta(i - L, B):
                M[i - 1, j - 1] = True
    return M


def build_mask(L: int, B: int) -> np.ndarray:
    """The same four cases as `build_mask_loops`, evaluated on whole index grids."""
    n = 2 * L
    i = np.arange(1, n + 1, dtype=np.int64)[:, None]
    j = np.arange(1, n + 1, dtype=np.int64)[None, :]
    bi = -(-(i - L) // B)   # beta(i - L), meaningful where i > L
    bj_m = -(-(j - L) // B)  # beta(j - L), meaningful where j > L
    bj_c = -(-j // B)        # beta(j), meaningful where j <= L
    case1 = (i <= L) & (j <= L) & (j <= i)
    case2 = (i > L) & (j > L) & (bi == bj_m) & (j <= i)
    case3 = (i > L) & (j <= L) & (bj_c < bi)
    return case1 | case2 | case3


def causal_mask(n: int) -> np.ndarray:
    """Plain causal visibility over n positions (the dense causal-2L comparison)."""
    return np.tril(np.ones((n, n), dtype=bool))


def ar_signal_ratio(L: int, B: int) -> tuple[float, float]:
    """AR-signal fractions from mask counts ([notes] 关键设计 2; 消融实验 table).

    A row carries an "AR signal" when its visible set holds no [MASK] key other
    than the row itself, i.e. it predicts from a fully clean context. Returns
    (combined, mask_only): the share of such rows among all 2L rows, and among
    the L mask-stream rows alone.
    """
    M = build_mask(L, B)
    n = 2 * L
    clean_ctx = 0
    mask_rows_clean_ctx = 0
    for a in range(n):
        vis = np.nonzero(M[a])[0]
        mask_keys = vis[vis >= L]
        others = mask_keys[mask_keys != a]
        if others.size == 0:
            clean_ctx += 1
            if a >= L:
                mask_rows_clean_ctx += 1
    return clean_ctx / n, mask_rows_clean_ctx / L


# ---------------------------------------------------------------------------
# Attention                              [notes] 整体框架, 关键设计 1
# ---------------------------------------------------------------------------


def _softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray,
                    scale: float):
    """Dense masked softmax attention for one head: rows q [r, d], keys k/v [c, d]."""
    s = (q @ k.T) * scale
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    out = (e / z) @ v
    lse = (m + np.log(z))[:, 0]
    return out, lse


def attn_two_stream(q, k, v, L: int, B: int, scale: float | None = None,
                    mask_mode: int = 0, pairs=None, rows=None, row_chunk: int = 1024):
    """Two-stream attention over z = [x; x~] under the explicit 2L x 2L mask.

    q [b, 2L, Hq, d], k/v [b, 2L, Hkv, d]. mask_mode 0 uses the MARS mask
    (`build_mask`), 1 plain causal over all 2L positions. `pairs` restricts the
    work to a list of (batch, q_head) pairs, `rows` to a list of query rows.
    Returns (out, lse) dicts keyed by pair: out [rows, d] float64 and the
    natural-log sum-exp of the scaled scores per row.
    """
    q = np.asarray(q)
    b, n, Hq, d = q.shape
    Hkv = k.shape[2]
    assert n == 2 * L and Hq % Hkv == 0
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    M = build_mask(L, B) if mask_mode == 0 else causal_mask(n)
    if pairs is None:
        pairs = [(bi, h) for bi in range(b) for h in range(Hq)]
    row_idx = np.arange(n) if rows is None else np.asarray(rows)
    outs, lses = {}, {}
    for (bi, h) in pairs:
        kv = h // g
        K = np.asarray(k[bi, :, kv, :], dtype=np.float64)
        Vv = np.asarray(v[bi, :, kv, :], dtype=np.float64)
        o = np.empty((row_idx.size, d))
        l = np.empty(row_idx.size)
        for s0 in range(0, row_idx.size, row_chunk):
            r = row_idx[s0:s0 + row_chunk]
            Q = np.asarray(q[bi, r, h, :], dtype=np.float64)
            o[s0:s0 + r.size], l[s0:s0 + r.size] = _softmax_attend(Q, K, Vv, M[r], scale)
        outs[(bi, h)], lses[(bi, h)] = o, l
    return outs, lses


def attn_causal(q, k, v, scale: float | None = None, pairs=None):
    """Plain causal attention over T positions (the no-cache prefill path: every step
    recomputes the whole sequence, prompt plus the B [MASK] rows, causally; [gist] 4
    and the notes' wall-clock table for the no-cache setting).

    q [b, T, Hq, d], k/v [b, T, Hkv, d]. Returns (out, lse) dicts keyed by
    (batch, q_head), as attn_two_stream.
    """
    q = np.asarray(q)
    b, n, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    M = causal_mask(n)
    if pairs is None:
        pairs = [(bi, h) for bi in range(b) for h in range(Hq)]
    outs, lses = {}, {}
    for (bi, h) in pairs:
        K = np.asarray(k[bi, :, h // g, :], dtype=np.float64)
        Vv = np.asarray(v[bi, :, h // g, :], dtype=np.float64)
        Q = np.asarray(q[bi, :, h, :], dtype=np.float64)
        outs[(bi, h)], lses[(bi, h)] = _softmax_attend(Q, K, Vv, M, scale)
    return outs, lses


def attn_two_stream_backward(q, k, v, do, L: int, B: int, scale: float | None = None,
                             mask_mode: int = 0, groups=None, row_chunk: int = 1024):
    """Gradients of `attn_two_stream` with respect to q, k and v, given do = dLoss/dO.

    The pages train the model on L_mask + L_AR through this attention ([notes]
    关键设计 2; [gist] 2B), so its gradient is that of the forward's definition,
    by the chain rule. Per query head, with S = scale * Q K^T masked by M,
    P = softmax over each row of S, O = P V:
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(dO * O))
        dQ = scale * dS K
        dK = scale * dS^T Q
    and a KV head collects dK, dV from every query head that reads it.

    q, do [b, 2L, Hq, d]; k, v [b, 2L, Hkv, d]. `groups` restricts the work to
    a list of (batch, kv_head): dq of that group's query heads and dk, dv of
    that KV head are filled, everything else stays zero. Rows are processed in
    chunks of `row_chunk` (the sums over rows are unchanged by that split).
    Returns float64 arrays dq [b, 2L, Hq, d], dk, dv [b, 2L, Hkv, d].
    """
    q = np.asarray(q)
    b, n, Hq, d = q.shape
    Hkv = k.shape[2]
    assert n == 2 * L and Hq % Hkv == 0
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    M = build_mask(L, B) if mask_mode == 0 else causal_mask(n)
    if groups is None:
        groups = [(bi, kv) for bi in range(b) for kv in range(Hkv)]
    dq = np.zeros((b, n, Hq, d))
    dk = np.zeros((b, n, Hkv, d))
    dv = np.zeros((b, n, Hkv, d))
    for (bi, kv) in groups:
        K = np.asarray(k[bi, :, kv, :], dtype=np.float64)
        Vv = np.asarray(v[bi, :, kv, :], dtype=np.float64)
        for h in range(kv * g, (kv + 1) * g):
            for r0 in range(0, n, row_chunk):
                r = np.arange(r0, min(n, r0 + row_chunk))
                Q = np.asarray(q[bi, r, h, :], dtype=np.float64)
                dO = np.asarray(do[bi, r, h, :], dtype=np.float64)
                s = np.where(M[r], (Q @ K.T) * scale, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                o = p @ Vv
                dp = dO @ Vv.T
                ds = p * (dp - (dO * o).sum(axis=1, keepdims=True))
                dq[bi, r, h, :] = scale * (ds @ K)
                dk[bi, :, kv, :] += scale * (ds.T @ Q)
                dv[bi, :, kv, :] += p.T @ dO
    return dq, dk, dv


def gather_prefix(cache: np.ndarray, block_table: np.ndarray, s: int, length: int,
                  page_size: int, kv_head: int, transposed: bool) -> np.ndarray:
    """Logical cache rows 0..length-1 of sequence s for one KV head, as [length, d].

    Position pos lives in page block_table[s, pos // page_size] at slot
    pos % page_size. K pages are [pages, Hkv, page, d]; V pages (transposed=True)
    are [pages, Hkv, d, page].
    """
    pos = np.arange(length)
    pages = block_table[s, pos // page_size]
    slots = pos % page_size
    if transposed:
        return np.asarray(cache[pages, kv_head, :, slots], dtype=np.float64)
    return np.asarray(cache[pages, kv_head, slots, :], dtype=np.float64)


def attn_block_decode(q, k_new, v_new, k_cache, v_cache, block_table, cache_len,
                      page_size: int, scale: float | None = None, seqs=None):
    """Block-decode attention ([gist] 2C-2D; [notes] 关键设计 3-4).

    Each sequence s appends B [MASK] query rows. Row r (0-based) attends to the
    cached prefix rows 0..cache_len[s]-1 and to the new rows 0..r (causal among
    the B new rows). q [S, B, Hq, d]; k_new/v_new [S, B, Hkv, d]; K cache
    [pages, Hkv, page, d]; V cache [pages, Hkv, d, page]. Returns out
    [len(seqs), B, Hq, d] float64.
    """
    S, B, Hq, d = q.shape
    Hkv = k_new.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if seqs is None:
        seqs = range(S)
    seqs = list(seqs)
    out = np.empty((len(seqs), B, Hq, d))
    for si, s in enumerate(seqs):
        n = int(cache_len[s])
        for kv in range(Hkv):
            Kp = gather_prefix(k_cache, block_table, s, n, page_size, kv, False)
            Vp = gather_prefix(v_cache, block_table, s, n, page_size, kv, True)
            Kn = np.asarray(k_new[s, :, kv, :], dtype=np.float64)
            Vn = np.asarray(v_new[s, :, kv, :], dtype=np.float64)
            Kall = np.concatenate([Kp, Kn], axis=0)
            Vall = np.concatenate([Vp, Vn], axis=0)
            vis = np.zeros((B, n + B), dtype=bool)
            for r in range(B):
                vis[r, :n + r + 1] = True
            for h in range(kv * g, (kv + 1) * g):
                Q = np.asarray(q[s, :, h, :], dtype=np.float64)
                out[si, :, h, :], _ = _softmax_attend(Q, Kall, Vall, vis, scale)
    return out


# ---------------------------------------------------------------------------
# LM head, confidence, acceptance, commit   [gist] 2C; [notes] 关键设计 3-4
# ---------------------------------------------------------------------------


def lmhead(hidden, w) -> np.ndarray:
    """logits = hidden @ W^T in float64 (the unchanged LM head, [gist] section 3)."""
    return np.asarray(hidden, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def confidence_row(row) -> tuple[int, float]:
    """(argmax id, max softmax probability) of one logit row.

    max_v p(x_t = v) at temperature 1 ([notes] 关键设计 3); the id is the first
    (lowest) index attaining the maximum logit. p = 1 / sum_v exp(l_v - m).
    """
    row = np.asarray(row, dtype=np.float64)
    if not np.all(np.isfinite(row)):
        raise ValueError("the oracle's confidence is defined for finite logits only")
    m = row.max()
    idx = int(np.flatnonzero(row == m)[0])
    return idx, float(1.0 / np.exp(row - m).sum())


def confidence(logits) -> tuple[np.ndarray, np.ndarray]:
    """Per-row (top_id int32, p_max float64) of logits [N, V]."""
    logits = np.asarray(logits)
    ids = np.empty(logits.shape[0], dtype=np.int32)
    ps = np.empty(logits.shape[0], dtype=np.float64)
    for r in range(logits.shape[0]):
        ids[r], ps[r] = confidence_row(logits[r])
    return ids, ps


def accept_count(p_row, tau: float) -> int:
    """Accepted tokens of one step ([gist] 2C; [notes] 关键设计 3).

    Scan left to right, accepting while p >= tau; stop at the first position
    below tau; always accept at least the first token.
    """
    n = 0
    while n < len(p_row) and p_row[n] >= tau:
        n += 1
    return max(n, 1)


def accept(p_max, top_id, tau):
    """Per-sequence acceptance over p_max/top_id [S, B] and tau [S].

    Returns (n_accepted [S] int32, accepted_ids [S, B] int32 padded with -1).
    """
    p_max = np.asarray(p_max)
    S, B = p_max.shape
    n_acc = np.empty(S, dtype=np.int32)
    ids = np.full((S, B), -1, dtype=np.int32)
    for s in range(S):
        n = accept_count(p_max[s], float(tau[s]))
        n_acc[s] = n
        ids[s, :n] = top_id[s, :n]
    return n_acc, ids


def commit(k_cache, v_cache, block_table, cache_len, k_new, v_new, n_accepted,
           page_size: int):
    """Append the accepted prefix of each sequence's new K/V rows to the paged cache.

    Works in place on copies of the caches and lengths and returns
    (k_cache, v_cache, cache_len, commit_pos). Row r < n of sequence s goes to
    position pos = cache_len[s] + r, i.e. page block_table[s, pos // page_size],
    slot pos % page_size; then cache_len[s] grows by n ([gist] 2D; [notes]
    关键设计 4: accepted tokens join the persistent prefix cache). commit_pos
    [S, B] holds pos, or -1 for rows not committed.
    """
    k_cache = np.array(k_cache, copy=True)
    v_cache = np.array(v_cache, copy=True)
    cache_len = np.array(cache_len, copy=True)
    S, B = k_new.shape[0], k_new.shape[1]
    commit_pos = np.full((S, B), -1, dtype=np.int32)
    for s in range(S):
        base = int(cache_len[s])
        for r in range(int(n_accepted[s])):
            pos = base + r
            page = block_table[s, pos // page_size]
            slot = pos % page_size
            k_cache[page, :, slot, :] = k_new[s, r]
            v_cache[page, :, :, slot] = v_new[s, r]
            commit_pos[s, r] = pos
        cache_len[s] = base + int(n_accepted[s])
    return k_cache, v_cache, cache_len, commit_pos


# ---------------------------------------------------------------------------
# Batch-synchronous block cache                     [notes] 关键设计 4; [gist] 2D
# ---------------------------------------------------------------------------
#
# Reading taken (the pages describe the policy in two sentences that are read
# here as one rule): the persistent prefix cache grows only by whole blocks of
# B_cache tokens, and only once every sequence of the batch has filled the
# block; until then the tokens accepted since the last frozen block are
# re-fed to every forward (their K/V are recomputed), ahead of the B [MASK]
# rows. Policy "min" (the default): each step the whole batch advances by the
# smallest accepted count of the step, capped at the block boundary. Policy
# "wait": each sequence advances by its own count, capped at the boundary,
# where a faster sequence waits (advances by 0) until the batch has filled the
# block. The forward after the block fills has the B_cache block tokens as its
# first rows; that forward freezes them into the cache.


def attn_block_decode_rows(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_rows,
                           page_size: int, scale: float | None = None, seqs=None):
    """Block-decode attention with a per-sequence count of new rows.

    Under the block cache a step's forward takes, for sequence s, the u_s
    tokens not yet frozen followed by the B [MASK] rows: n_rows[s] = u_s + B
    rows out of the R rows that q/k_new/v_new [S, R, ...] hold. Row r <
    n_rows[s] attends to the frozen prefix (cache_len[s] rows) and to new rows
    0..r. Returns {s: out [n_rows[s], Hq, d]} (float64).
    """
    S = q.shape[0]
    if seqs is None:
        seqs = range(S)
    out = {}
    for s in seqs:
        R = int(n_rows[s])
        if R == 0:
            out[s] = np.zeros((0, q.shape[2], q.shape[3]))
            continue
        out[s] = attn_block_decode(q[s:s + 1, :R], k_new[s:s + 1, :R], v_new[s:s + 1, :R],
                                   k_cache, v_cache, block_table[s:s + 1], cache_len[s:s + 1],
                                   page_size, scale)[0]
    return out


def block_sync_advance(n_accepted, unfrozen, B_cache: int, policy: str = "min"):
    """Tokens each sequence keeps this step under the batch-synchronous block cache.

    n_accepted [S]: the step's accepted counts (accept_count); unfrozen [S]:
    tokens accepted since the last frozen block (0..B_cache). "min": every
    sequence keeps min over the batch of n_accepted, but no more than the room
    left in its block; "wait": each keeps its own count, but no more than the
    room left in its block.
    """
    n = np.asarray(n_accepted, dtype=np.int64)
    room = B_cache - np.asarray(unfrozen, dtype=np.int64)
    if policy == "min":
        keep = np.minimum(n.min(), room)
    elif policy == "wait":
        keep = np.minimum(n, room)
    else:
        raise ValueError(f"policy must be 'min' or 'wait', got {policy!r}")
    return keep.astype(np.int32)


def block_sync_step(p_max, top_id, tau, unfrozen, block_tokens, B_cache: int,
                    policy: str = "min"):
    """Acceptance under the batch-synchronous block cache, for one step.

    1. If every sequence's block was full when this step's forward ran, that
       forward froze the block: the unfrozen count restarts at 0.
    2. Each sequence's accepted count n_s follows the threshold rule
       (accept_count); the batch policy turns it into the kept count a_s.
    3. The a_s kept tokens (the first a_s top ids) join the unfrozen block.

    Returns (kept [S], unfrozen [S], block_tokens [S, B_cache] padded with -1,
    froze: bool, n_rows_next [S] = unfrozen + B).
    """
    S, B = np.asarray(p_max).shape
    u = np.array(unfrozen, dtype=np.int32, copy=True)
    toks = np.array(block_tokens, dtype=np.int32, copy=True)
    froze = bool(np.all(u == B_cache))
    if froze:
        u[:] = 0
        toks[:] = -1
    n, _ = accept(p_max, top_id, tau)
    keep = block_sync_advance(n, u, B_cache, policy)
    for s in range(S):
        for i in range(int(keep[s])):
            toks[s, u[s] + i] = top_id[s][i]
        u[s] += keep[s]
    return keep, u, toks, froze, u + B


def block_freeze(k_cache, v_cache, block_table, cache_len, k_rows, v_rows, unfrozen,
                 B_cache: int, page_size: int):
    """Freeze the block into the persistent cache when every sequence has filled it.

    k_rows/v_rows [S, R, Hkv, d] are the K/V of a forward whose first B_cache
    rows per sequence are the block's tokens. If every unfrozen count equals
    B_cache, those rows are appended to the paged cache (commit of B_cache rows
    per sequence); otherwise nothing changes. Returns (k_cache, v_cache,
    cache_len, froze).
    """
    if not np.all(np.asarray(unfrozen) == B_cache):
        return (np.array(k_cache, copy=True), np.array(v_cache, copy=True),
                np.array(cache_len, copy=True), False)
    S = k_rows.shape[0]
    kc, vc, ln, _ = commit(k_cache, v_cache, block_table, cache_len, k_rows[:, :B_cache],
                           v_rows[:, :B_cache], np.full(S, B_cache), page_size)
    return kc, vc, ln, True


def useful_pairs_two_stream(L: int, B: int, mask_mode: int = 0) -> int:
    """Number of visible (query, key) pairs per head under the explicit mask
    ([notes] 关键设计 1); mask_mode 1 counts plain causal attention over 2L."""
    M = build_mask(L, B) if mask_mode == 0 else causal_mask(2 * L)
    return int(M.sum())
