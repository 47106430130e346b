"""Thin torch-facing binding of the four MARS entry points.

Each function checks that the tensors are on the GPU, contiguous and of the
expected dtype, allocates outputs when the caller did not pass them, and calls
the C function of the same name on the current HIP stream. All arithmetic
happens in the library's kernels; nothing here computes a result.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import MARS_BF16, MARS_F32, check

_DT = {torch.float32: MARS_F32, torch.bfloat16: MARS_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")


def mars_attn_two_stream(q, k, v, L: int, B: int, *, o=None, lse=None, return_lse=False,
                         softmax_scale: float = 0.0, mask_mode: int = 0, stream=None):
    """Two-stream MARS attention over z = [x; x~].

    q [b, 2L, Hq, d], k/v [b, 2L, Hkv, d] (bf16 or fp32). Returns o (and lse
    [b, Hq, 2L] fp32 when return_lse or lse is given).
    """
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dt, 4)
    b, n2, Hq, d = q.shape
    Hkv = k.shape[2]
    if n2 != 2 * L or k.shape != (b, n2, Hkv, d) or v.shape != k.shape:
        raise ValueError("shapes must be q [b,2L,Hq,d], k/v [b,2L,Hkv,d]")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", dt)
    if lse is None and return_lse:
        lse = torch.empty((b, Hq, n2), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    code = _lib.lib().mars_attn_two_stream(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, L, B, Hq, Hkv, d,
        _DT.get(dt, -1), float(softmax_scale), int(mask_mode), _stream(stream))
    check("mars_attn_two_stream", code)
    return (o, lse) if lse is not None else o


def mars_attn_causal(q, k, v, *, o=None, lse=None, return_lse=False,
                     softmax_scale: float = 0.0, stream=None):
    """Causal attention over T positions (no-cache prefill). q [b, T, Hq, d],
    k/v [b, T, Hkv, d]; returns o (and lse [b, Hq, T] when asked)."""
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dt, 4)
    b, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (b, T, Hkv, d) or v.shape != k.shape:
        raise ValueError("shapes must be q [b,T,Hq,d], k/v [b,T,Hkv,d]")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", dt)
    if lse is None and return_lse:
        lse = torch.empty((b, Hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    code = _lib.lib().mars_attn_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, T, Hq,
                                       Hkv, d, _DT.get(dt, -1), float(softmax_scale),
                                       _stream(stream))
    check("mars_attn_causal", code)
    return (o, lse) if lse is not None else o


def mars_kv_append(k_rows, v_rows, k_cache, v_cache, block_table, cache_len, *, status=None,
                   stream=None):
    """Append k_rows/v_rows [S, T, Hkv, d] to the paged cache at cache_len; cache_len
    is advanced in place. Cache layouts as for mars_attn_block_decode."""
    dt = k_rows.dtype
    for t, n in ((k_rows, "k_rows"), (v_rows, "v_rows"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, n, dt, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_len, "cache_len", torch.int32, 1)
    S, T, Hkv, d = k_rows.shape
    num_pages, _, page, _ = k_cache.shape
    if v_rows.shape != k_rows.shape or tuple(v_cache.shape) != (num_pages, Hkv, d, page):
        raise ValueError("v_rows as k_rows; k_cache [pages,Hkv,page,d], v_cache [pages,Hkv,d,page]")
    code = _lib.lib().mars_kv_append(_ptr(k_rows), _ptr(v_rows), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_table), _ptr(cache_len), S, T, Hkv, d, page,
                                     block_table.shape[1], num_pages, _DT.get(dt, -1),
                                     _ptr(status), _stream(stream))
    check("mars_kv_append", code)


def mars_attn_two_stream_bwd(q, k, v, o, d_o, lse, L: int, B: int, *, dq=None, dk=None,
                             dv=None, workspace=None, softmax_scale: float = 0.0,
                             mask_mode: int = 0, stream=None):
    """Backward of mars_attn_two_stream (bf16): returns (dq, dk, dv). o and lse are the
    forward's outputs for the same inputs; d_o is dLoss/dO [b, 2L, Hq, d]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")):
        _need(t, n, torch.bfloat16, 4)
    b, n2, Hq, d = q.shape
    Hkv = k.shape[2]
    if (n2 != 2 * L or k.shape != (b, n2, Hkv, d) or v.shape != k.shape or o.shape != q.shape
            or d_o.shape != q.shape):
        raise ValueError("shapes must be q/o/d_o [b,2L,Hq,d], k/v [b,2L,Hkv,d]")
    _need(lse, "lse", torch.float32, 3)
    if tuple(lse.shape) != (b, Hq, n2):
        raise ValueError("lse must be [b, Hq, 2L]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, torch.bfloat16, 4)
    need = int(_lib.lib().mars_attn_two_stream_bwd_workspace_bytes(b, L, Hq, Hkv, d))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    code = _lib.lib().mars_attn_two_stream_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        b, L, B, Hq, Hkv, d, _DT[torch.bfloat16], float(softmax_scale), int(mask_mode),
        _ptr(workspace), workspace.numel(), _stream(stream))
    check("mars_attn_two_stream_bwd", code)
    return dq, dk, dv


def mars_decode_workspace_bytes(S, B, n_q_heads, n_kv_heads, head_dim, page_size, max_pages):
    return int(_lib.lib().mars_decode_workspace_bytes(S, B, n_q_heads, n_kv_heads, head_dim,
                                                      page_size, max_pages))


def mars_attn_block_decode(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, *,
                           n_rows=None, o=None, workspace=None, status=None,
                           softmax_scale: float = 0.0, stream=None):
    """Block-decode attention. q [S,B,Hq,d]; k_new/v_new [S,B,Hkv,d]; K cache
    [pages,Hkv,page,d]; V cache [pages,Hkv,d,page]; block_table [S,max_pages];
    cache_len [S] (all on the GPU). Returns o [S,B,Hq,d]. With n_rows (int32 [S],
    on the GPU), sequence s uses only its first n_rows[s] rows (the block-cache
    form); output rows past them are left as they were."""
    dt = q.dtype
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, n, dt, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_len, "cache_len", torch.int32, 1)
    S, B, Hq, d = q.shape
    Hkv = k_new.shape[2]
    num_pages, _, page, _ = k_cache.shape
    max_pages = block_table.shape[1]
    if v_cache.shape != (num_pages, Hkv, d, page) or k_cache.shape != (num_pages, Hkv, page, d):
        raise ValueError("K cache must be [pages,Hkv,page,d] and V cache [pages,Hkv,d,page]")
    if o is None:
        o = torch.empty_like(q)
    need = mars_decode_workspace_bytes(S, B, Hq, Hkv, d, page, max_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if n_rows is None:
        code = _lib.lib().mars_attn_block_decode(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(cache_len), _ptr(o), S, B, Hq, Hkv, d, page, max_pages, num_pages,
            _DT.get(dt, -1), float(softmax_scale), _ptr(workspace), workspace.numel(),
            _ptr(status), _stream(stream))
        check("mars_attn_block_decode", code)
        return o
    _need(n_rows, "n_rows", torch.int32, 1)
    code = _lib.lib().mars_attn_block_decode_rows(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(cache_len), _ptr(n_rows), _ptr(o), S, B, Hq, Hkv, d, page, max_pages, num_pages,
        _DT.get(dt, -1), float(softmax_scale), _ptr(workspace), workspace.numel(), _ptr(status),
        _stream(stream))
    check("mars_attn_block_decode_rows", code)
    return o


_POLICY = {"min": 0, "wait": 1}


def mars_block_sync_accept(p_max, top_id, tau, unfrozen, block_tokens, *, policy="min",
                           n_kept=None, n_rows=None, status=None, stream=None):
    """Acceptance under the batch-synchronous block cache. p_max/top_id [S,B], tau [S];
    unfrozen [S] and block_tokens [S,B_cache] (int32) are updated in place.
    Returns (n_kept [S], n_rows [S]) (int32)."""
    _need(p_max, "p_max", torch.float32, 2)
    _need(top_id, "top_id", torch.int32, 2)
    _need(tau, "tau", torch.float32, 1)
    _need(unfrozen, "unfrozen", torch.int32, 1)
    _need(block_tokens, "block_tokens", torch.int32, 2)
    S, B = p_max.shape
    Bc = block_tokens.shape[1]
    if n_kept is None:
        n_kept = torch.empty(S, dtype=torch.int32, device=p_max.device)
    if n_rows is None:
        n_rows = torch.empty(S, dtype=torch.int32, device=p_max.device)
    code = _lib.lib().mars_block_sync_accept(
        _ptr(p_max), _ptr(top_id), _ptr(tau), _ptr(unfrozen), _ptr(block_tokens), _ptr(n_kept),
        _ptr(n_rows), S, B, Bc, _POLICY.get(policy, -1), _ptr(status), _stream(stream))
    check("mars_block_sync_accept", code)
    return n_kept, n_rows


def mars_block_freeze(k_rows, v_rows, k_cache, v_cache, block_table, cache_len, unfrozen,
                      B_cache: int, *, status=None, stream=None):
    """Append rows 0..B_cache-1 of k_rows/v_rows [S,R,Hkv,d] to the paged cache if every
    unfrozen[s] == B_cache (decided on the GPU); cache_len grows by B_cache then."""
    dt = k_rows.dtype
    for t, n in ((k_rows, "k_rows"), (v_rows, "v_rows"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, n, dt, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_len, "cache_len", torch.int32, 1)
    _need(unfrozen, "unfrozen", torch.int32, 1)
    S, R, Hkv, d = k_rows.shape
    num_pages, _, page, _ = k_cache.shape
    code = _lib.lib().mars_block_freeze(
        _ptr(k_rows), _ptr(v_rows), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(cache_len), _ptr(unfrozen), S, R, int(B_cache), Hkv, d, page,
        block_table.shape[1], num_pages, _DT.get(dt, -1), _ptr(status), _stream(stream))
    check("mars_block_freeze", code)


def mars_lmhead_workspace_bytes(N, V):
    return int(_lib.lib().mars_lmhead_workspace_bytes(N, V))


class PackedLMHead:
    """LM-head weights in the GEMM's tile layout (from mars_lmhead_pack)."""

    def __init__(self, data, vocab: int, dim: int):
        self.data, self.vocab, self.dim = data, vocab, dim


def mars_lmhead_pack(w_lm, *, stream=None) -> PackedLMHead:
    """Pack W [V, D] bf16 once for mars_lmhead_confidence (same results, contiguous
    weight reads)."""
    _need(w_lm, "w_lm", torch.bfloat16, 2)
    V, D = w_lm.shape
    n = int(_lib.lib().mars_lmhead_packed_bytes(D, V))
    if n == 0:
        raise ValueError("packing needs D >= 32, D % 32 == 0, V >= 4 and V % 4 == 0")
    data = torch.empty(n // 2, dtype=torch.bfloat16, device=w_lm.device)
    check("mars_lmhead_pack", _lib.lib().mars_lmhead_pack(_ptr(w_lm), _ptr(data), D, V,
                                                            _stream(stream)))
    return PackedLMHead(data, V, D)


def mars_lmhead_confidence(hidden, w_lm, logits=None, *, top_id=None, p_max=None,
                           workspace=None, status=None, stream=None, fused=False):
    """LM head + confidence. With hidden [N,D] bf16 and w_lm [V,D] bf16 (or a
    PackedLMHead), writes fp32 logits [N,V] (or, with fused=True, writes no logits and
    returns None for them); with hidden None, `logits` is the input. Returns (logits,
    top_id int32 [N], p_max fp32 [N])."""
    packed = isinstance(w_lm, PackedLMHead)
    if hidden is not None:
        _need(hidden, "hidden", torch.bfloat16, 2)
        N, D = hidden.shape
        if packed:
            _need(w_lm.data, "w_lm", torch.bfloat16, 1)
            V = w_lm.vocab
            if w_lm.dim != D:
                raise ValueError("packed LM head has a different hidden size")
        else:
            _need(w_lm, "w_lm", torch.bfloat16, 2)
            V = w_lm.shape[0]
            if w_lm.shape[1] != D:
                raise ValueError("w_lm must be [V, D]")
        if fused:
            if logits is not None:
                raise ValueError("fused=True writes no logits; pass logits=None")
        elif logits is None:
            logits = torch.empty((N, V), dtype=torch.float32, device=hidden.device)
        dev = hidden.device
    else:
        if logits is None or fused:
            raise ValueError("logits are required (and fused is off) when hidden is None")
        D = 0
    if logits is not None:
        _need(logits, "logits", torch.float32, 2)
        N, V = logits.shape
        dev = logits.device
    if top_id is None:
        top_id = torch.empty(N, dtype=torch.int32, device=dev)
    if p_max is None:
        p_max = torch.empty(N, dtype=torch.float32, device=dev)
    need = mars_lmhead_workspace_bytes(N, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if packed:
        if hidden is None:
            raise ValueError("a packed LM head needs hidden states")
        code = _lib.lib().mars_lmhead_confidence_packed(
            _ptr(hidden), _ptr(w_lm.data), _ptr(logits), N, D, V, _ptr(top_id), _ptr(p_max),
            _ptr(workspace), workspace.numel(), _ptr(status), _stream(stream))
        check("mars_lmhead_confidence_packed", code)
        return logits, top_id, p_max
    code = _lib.lib().mars_lmhead_confidence(
        _ptr(hidden), _ptr(w_lm), _ptr(logits), N, D, V, _ptr(top_id), _ptr(p_max),
        _ptr(workspace), workspace.numel(), _ptr(status), _stream(stream))
    check("mars_lmhead_confidence", code)
    return logits, top_id, p_max


def mars_accept_commit(p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table,
                       cache_len, *, n_accepted=None, accepted_ids=None, commit_pos=None,
                       status=None, stream=None):
    """Acceptance + KV commit. p_max [S,B] fp32, top_id [S,B] int32, tau [S] fp32,
    k_new/v_new [S,B,Hkv,d]; caches as for decode; cache_len updated in place.
    Returns (n_accepted [S], accepted_ids [S,B], commit_pos [S,B])."""
    _need(p_max, "p_max", torch.float32, 2)
    _need(top_id, "top_id", torch.int32, 2)
    _need(tau, "tau", torch.float32, 1)
    dt = k_new.dtype
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, dt, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_len, "cache_len", torch.int32, 1)
    S, B = p_max.shape
    _, _, Hkv, d = k_new.shape
    num_pages, _, page, _ = k_cache.shape
    max_pages = block_table.shape[1]
    dev = p_max.device
    if n_accepted is None:
        n_accepted = torch.empty(S, dtype=torch.int32, device=dev)
    if accepted_ids is None:
        accepted_ids = torch.empty((S, B), dtype=torch.int32, device=dev)
    if commit_pos is None:
        commit_pos = torch.empty((S, B), dtype=torch.int32, device=dev)
    code = _lib.lib().mars_accept_commit(
        _ptr(p_max), _ptr(top_id), _ptr(tau), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), _ptr(cache_len), _ptr(n_accepted), _ptr(accepted_ids),
        _ptr(commit_pos), S, B, Hkv, d, page, max_pages, num_pages, _DT.get(dt, -1),
        _ptr(status), _stream(stream))
    check("mars_accept_commit", code)
    return n_accepted, accepted_ids, commit_pos
