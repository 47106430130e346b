"""Thin torch-facing binding of the MARS entry points.

Each function checks every tensor it is given: type, dtype, rank, contiguity,
the full shape against the sizes it implies for the other tensors, workspace
sizes, and last that every tensor lives on the GPU. A mismatch raises
ValueError (TypeError for a non-tensor) before the library is called, so a
wrongly shaped buffer can never reach a kernel. Outputs the caller did not
pass are allocated, and the C function of the same name is called on the
current HIP stream. All arithmetic happens in the library's kernels; nothing
here computes a result.
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


def _need(t, name, dtype=None, ndim=None, shape=None):
    """Type, dtype, rank, contiguity and (optionally) the exact shape of one tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(t, name, dtype=None, ndim=None, shape=None):
    if t is not None:
        _need(t, name, dtype, ndim, shape)


def _status(status):
    if status is not None:
        _need(status, "status", torch.int32)
        if status.numel() < 1:
            raise ValueError("status must hold at least one int32")


def _workspace(ws, need, name="workspace"):
    _need(ws, name, torch.uint8)
    if ws.numel() < need:
        raise ValueError(f"{name} holds {ws.numel()} bytes; this call needs {need}")


def _on_gpu(**tensors):
    """Last check before a library call: every given tensor is on one GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other tensors on {dev}")


def _paged_cache(k_cache, v_cache, dt, Hkv, d):
    """K cache [pages, Hkv, page, d] and V cache [pages, Hkv, d, page] matching Hkv, d."""
    _need(k_cache, "k_cache", dt, 4)
    num_pages, hk, page, dk = k_cache.shape
    if hk != Hkv or dk != d:
        raise ValueError(f"k_cache must be [pages, {Hkv}, page, {d}] (got {tuple(k_cache.shape)})")
    _need(v_cache, "v_cache", dt, 4, (num_pages, Hkv, d, page))
    return num_pages, page


def mars_attn_two_stream(q, k, v, L: int, B: int, *, o=None, lse=None, return_lse=False,
                         softmax_scale: float = 0.0, mask_mode: int = 0, stream=None):
    """Two-stream MARS attention over z = [x; x~].

    q [b, 2L, Hq, d], k/v [b, 2L, Hkv, d] (bf16 or fp32). Returns o (and lse
    [b, Hq, 2L] fp32 when return_lse or lse is given).
    """
    dt = q.dtype
    _need(q, "q", dt, 4)
    b, n2, Hq, d = q.shape
    _need(k, "k", dt, 4)
    Hkv = k.shape[2]
    if n2 != 2 * L:
        raise ValueError(f"q must hold 2L = {2 * L} positions (got {n2})")
    _need(k, "k", dt, 4, (b, n2, Hkv, d))
    _need(v, "v", dt, 4, (b, n2, Hkv, d))
    _opt(o, "o", dt, 4, q.shape)
    _opt(lse, "lse", torch.float32, 3, (b, Hq, n2))
    _on_gpu(q=q, k=k, v=v, o=o, lse=lse)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((b, Hq, n2), dtype=torch.float32, device=q.device)
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
    _need(q, "q", dt, 4)
    b, T, Hq, d = q.shape
    _need(k, "k", dt, 4)
    Hkv = k.shape[2]
    _need(k, "k", dt, 4, (b, T, Hkv, d))
    _need(v, "v", dt, 4, (b, T, Hkv, d))
    _opt(o, "o", dt, 4, q.shape)
    _opt(lse, "lse", torch.float32, 3, (b, Hq, T))
    _on_gpu(q=q, k=k, v=v, o=o, lse=lse)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((b, Hq, T), dtype=torch.float32, device=q.device)
    code = _lib.lib().mars_attn_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, T, Hq,
                                       Hkv, d, _DT.get(dt, -1), float(softmax_scale),
                                       _stream(stream))
    check("mars_attn_causal", code)
    return (o, lse) if lse is not None else o


def _append_args(k_rows, v_rows, k_cache, v_cache, block_table, cache_len, status):
    dt = k_rows.dtype
    _need(k_rows, "k_rows", dt, 4)
    S, T, Hkv, d = k_rows.shape
    _need(v_rows, "v_rows", dt, 4, (S, T, Hkv, d))
    num_pages, page = _paged_cache(k_cache, v_cache, dt, Hkv, d)
    _need(block_table, "block_table", torch.int32, 2)
    if block_table.shape[0] != S:
        raise ValueError(f"block_table must have {S} rows (got {block_table.shape[0]})")
    _need(cache_len, "cache_len", torch.int32, 1, (S,))
    _status(status)
    return dt, S, T, Hkv, d, num_pages, page


def mars_kv_append(k_rows, v_rows, k_cache, v_cache, block_table, cache_len, *, status=None,
                   stream=None):
    """Append k_rows/v_rows [S, T, Hkv, d] to the paged cache at cache_len; cache_len
    is advanced in place. Cache layouts as for mars_attn_block_decode."""
    dt, S, T, Hkv, d, num_pages, page = _append_args(k_rows, v_rows, k_cache, v_cache,
                                                     block_table, cache_len, status)
    _on_gpu(k_rows=k_rows, v_rows=v_rows, k_cache=k_cache, v_cache=v_cache,
            block_table=block_table, cache_len=cache_len, status=status)
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
    bf = torch.bfloat16
    _need(q, "q", bf, 4)
    b, n2, Hq, d = q.shape
    _need(k, "k", bf, 4)
    Hkv = k.shape[2]
    if n2 != 2 * L:
        raise ValueError(f"q must hold 2L = {2 * L} positions (got {n2})")
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, bf, 4, (b, n2, Hkv, d))
    for t, n in ((o, "o"), (d_o, "d_o")):
        _need(t, n, bf, 4, q.shape)
    _need(lse, "lse", torch.float32, 3, (b, Hq, n2))
    _opt(dq, "dq", bf, 4, q.shape)
    _opt(dk, "dk", bf, 4, k.shape)
    _opt(dv, "dv", bf, 4, k.shape)
    need = int(_lib.lib().mars_attn_two_stream_bwd_workspace_bytes(b, L, Hq, Hkv, d))
    if workspace is not None:
        _workspace(workspace, need)
    _on_gpu(q=q, k=k, v=v, o=o, d_o=d_o, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    code = _lib.lib().mars_attn_two_stream_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        b, L, B, Hq, Hkv, d, _DT[bf], float(softmax_scale), int(mask_mode),
        _ptr(workspace), workspace.numel(), _stream(stream))
    check("mars_attn_two_stream_bwd", code)
    return dq, dk, dv


def mars_decode_workspace_bytes(S, B, n_q_heads, n_kv_heads, head_dim, page_size, max_pages):
    return int(_lib.lib().mars_decode_workspace_bytes(S, B, n_q_heads, n_kv_heads, head_dim,
                                                      page_size, max_pages))


def _decode_args(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_rows, o, status):
    dt = q.dtype
    _need(q, "q", dt, 4)
    S, B, Hq, d = q.shape
    _need(k_new, "k_new", dt, 4)
    Hkv = k_new.shape[2]
    _need(k_new, "k_new", dt, 4, (S, B, Hkv, d))
    _need(v_new, "v_new", dt, 4, (S, B, Hkv, d))
    num_pages, page = _paged_cache(k_cache, v_cache, dt, Hkv, d)
    _need(block_table, "block_table", torch.int32, 2)
    if block_table.shape[0] != S:
        raise ValueError(f"block_table must have {S} rows (got {block_table.shape[0]})")
    _need(cache_len, "cache_len", torch.int32, 1, (S,))
    _opt(n_rows, "n_rows", torch.int32, 1, (S,))
    _opt(o, "o", dt, 4, q.shape)
    _status(status)
    return dt, S, B, Hq, Hkv, d, num_pages, page, block_table.shape[1]


def mars_attn_block_decode(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, *,
                           n_rows=None, o=None, workspace=None, status=None,
                           softmax_scale: float = 0.0, stream=None):
    """Block-decode attention. q [S,B,Hq,d]; k_new/v_new [S,B,Hkv,d]; K cache
    [pages,Hkv,page,d]; V cache [pages,Hkv,d,page]; block_table [S,max_pages];
    cache_len [S] (all on the GPU). Returns o [S,B,Hq,d]. With n_rows (int32 [S],
    on the GPU), sequence s uses only its first n_rows[s] rows (the block-cache
    form); output rows past them are left as they were."""
    dt, S, B, Hq, Hkv, d, num_pages, page, max_pages = _decode_args(
        q, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_rows, o, status)
    need = mars_decode_workspace_bytes(S, B, Hq, Hkv, d, page, max_pages)
    if workspace is not None:
        _workspace(workspace, need)
    _on_gpu(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
            block_table=block_table, cache_len=cache_len, n_rows=n_rows, o=o,
            workspace=workspace, status=status)
    if o is None:
        o = torch.empty_like(q)
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
    S, B = p_max.shape
    _need(top_id, "top_id", torch.int32, 2, (S, B))
    _need(tau, "tau", torch.float32, 1, (S,))
    _need(unfrozen, "unfrozen", torch.int32, 1, (S,))
    _need(block_tokens, "block_tokens", torch.int32, 2)
    if block_tokens.shape[0] != S:
        raise ValueError(f"block_tokens must have {S} rows (got {block_tokens.shape[0]})")
    Bc = block_tokens.shape[1]
    _opt(n_kept, "n_kept", torch.int32, 1, (S,))
    _opt(n_rows, "n_rows", torch.int32, 1, (S,))
    _status(status)
    _on_gpu(p_max=p_max, top_id=top_id, tau=tau, unfrozen=unfrozen, block_tokens=block_tokens,
            n_kept=n_kept, n_rows=n_rows, status=status)
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
    dt, S, R, Hkv, d, num_pages, page = _append_args(k_rows, v_rows, k_cache, v_cache,
                                                     block_table, cache_len, status)
    _need(unfrozen, "unfrozen", torch.int32, 1, (S,))
    _on_gpu(k_rows=k_rows, v_rows=v_rows, k_cache=k_cache, v_cache=v_cache,
            block_table=block_table, cache_len=cache_len, unfrozen=unfrozen, status=status)
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
    _on_gpu(w_lm=w_lm)
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
    wdata = None
    if hidden is not None:
        _need(hidden, "hidden", torch.bfloat16, 2)
        N, D = hidden.shape
        if packed:
            wdata = w_lm.data
            V = w_lm.vocab
            if w_lm.dim != D:
                raise ValueError("packed LM head has a different hidden size")
            _need(wdata, "w_lm", torch.bfloat16, 1)
            if wdata.numel() * 2 < int(_lib.lib().mars_lmhead_packed_bytes(D, V)):
                raise ValueError("packed LM head buffer is smaller than its layout")
        else:
            wdata = w_lm
            _need(w_lm, "w_lm", torch.bfloat16, 2)
            V = w_lm.shape[0]
            if w_lm.shape[1] != D:
                raise ValueError(f"w_lm must be [V, {D}] (got {tuple(w_lm.shape)})")
        if fused:
            if logits is not None:
                raise ValueError("fused=True writes no logits; pass logits=None")
        else:
            _opt(logits, "logits", torch.float32, 2, (N, V))
    else:
        if logits is None or fused:
            raise ValueError("logits are required (and fused is off) when hidden is None")
        if packed:
            raise ValueError("a packed LM head needs hidden states")
        _need(logits, "logits", torch.float32, 2)
        N, V = logits.shape
    _opt(top_id, "top_id", torch.int32, 1, (N,))
    _opt(p_max, "p_max", torch.float32, 1, (N,))
    need = mars_lmhead_workspace_bytes(N, V)
    if workspace is not None:
        _workspace(workspace, need)
    _status(status)
    _on_gpu(hidden=hidden, w_lm=wdata, logits=logits, top_id=top_id, p_max=p_max,
            workspace=workspace, status=status)
    dev = hidden.device if hidden is not None else logits.device
    if logits is None and not fused:
        logits = torch.empty((N, V), dtype=torch.float32, device=dev)
    if top_id is None:
        top_id = torch.empty(N, dtype=torch.int32, device=dev)
    if p_max is None:
        p_max = torch.empty(N, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if packed:
        code = _lib.lib().mars_lmhead_confidence_packed(
            _ptr(hidden), _ptr(wdata), _ptr(logits), N, D, V, _ptr(top_id), _ptr(p_max),
            _ptr(workspace), workspace.numel(), _ptr(status), _stream(stream))
        check("mars_lmhead_confidence_packed", code)
        return logits, top_id, p_max
    code = _lib.lib().mars_lmhead_confidence(
        _ptr(hidden), _ptr(wdata), _ptr(logits), N, D if hidden is not None else 0, V,
        _ptr(top_id), _ptr(p_max), _ptr(workspace), workspace.numel(), _ptr(status),
        _stream(stream))
    check("mars_lmhead_confidence", code)
    return logits, top_id, p_max


def _commit_args(p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table, cache_len,
                 n_accepted, accepted_ids, commit_pos, status, layered):
    """Shape checks of the commit calls; returns (S, B, Hkv, d, page, num_pages, layers)."""
    _need(p_max, "p_max", torch.float32, 2)
    S, B = p_max.shape
    _need(top_id, "top_id", torch.int32, 2, (S, B))
    _need(tau, "tau", torch.float32, 1, (S,))
    dt = k_new.dtype
    if layered:
        _need(k_new, "k_new", dt, 5)
        layers, Hkv, d = k_new.shape[0], k_new.shape[3], k_new.shape[4]
        rows = (layers, S, B, Hkv, d)
        _need(k_cache, "k_cache", dt, 5)
        if k_cache.shape[0] != layers:
            raise ValueError(f"k_cache must hold {layers} layers (got {k_cache.shape[0]})")
        _need(v_cache, "v_cache", dt, 5)
        if v_cache.shape[0] != layers:
            raise ValueError(f"v_cache must hold {layers} layers (got {v_cache.shape[0]})")
        num_pages, page = _paged_cache(k_cache[0], v_cache[0], dt, Hkv, d)
    else:
        _need(k_new, "k_new", dt, 4)
        layers, Hkv, d = 1, k_new.shape[2], k_new.shape[3]
        rows = (S, B, Hkv, d)
        num_pages, page = _paged_cache(k_cache, v_cache, dt, Hkv, d)
    _need(k_new, "k_new", dt, len(rows), rows)
    _need(v_new, "v_new", dt, len(rows), rows)
    _need(block_table, "block_table", torch.int32, 2)
    if block_table.shape[0] != S:
        raise ValueError(f"block_table must have {S} rows (got {block_table.shape[0]})")
    _need(cache_len, "cache_len", torch.int32, 1, (S,))
    _opt(n_accepted, "n_accepted", torch.int32, 1, (S,))
    _opt(accepted_ids, "accepted_ids", torch.int32, 2, (S, B))
    _opt(commit_pos, "commit_pos", torch.int32, 2, (S, B))
    _status(status)
    _on_gpu(p_max=p_max, top_id=top_id, tau=tau, k_new=k_new, v_new=v_new, k_cache=k_cache,
            v_cache=v_cache, block_table=block_table, cache_len=cache_len,
            n_accepted=n_accepted, accepted_ids=accepted_ids, commit_pos=commit_pos,
            status=status)
    return S, B, Hkv, d, page, num_pages, layers


def _commit_outputs(p_max, n_accepted, accepted_ids, commit_pos):
    S, B = p_max.shape
    dev = p_max.device
    if n_accepted is None:
        n_accepted = torch.empty(S, dtype=torch.int32, device=dev)
    if accepted_ids is None:
        accepted_ids = torch.empty((S, B), dtype=torch.int32, device=dev)
    if commit_pos is None:
        commit_pos = torch.empty((S, B), dtype=torch.int32, device=dev)
    return n_accepted, accepted_ids, commit_pos


def mars_accept_commit(p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table,
                       cache_len, *, n_accepted=None, accepted_ids=None, commit_pos=None,
                       status=None, stream=None):
    """Acceptance + KV commit. p_max [S,B] fp32, top_id [S,B] int32, tau [S] fp32,
    k_new/v_new [S,B,Hkv,d]; caches as for decode; cache_len updated in place.
    Returns (n_accepted [S], accepted_ids [S,B], commit_pos [S,B])."""
    S, B, Hkv, d, page, num_pages, _ = _commit_args(
        p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_accepted,
        accepted_ids, commit_pos, status, layered=False)
    n_accepted, accepted_ids, commit_pos = _commit_outputs(p_max, n_accepted, accepted_ids,
                                                           commit_pos)
    code = _lib.lib().mars_accept_commit(
        _ptr(p_max), _ptr(top_id), _ptr(tau), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), _ptr(cache_len), _ptr(n_accepted), _ptr(accepted_ids),
        _ptr(commit_pos), S, B, Hkv, d, page, block_table.shape[1], num_pages,
        _DT.get(k_new.dtype, -1), _ptr(status), _stream(stream))
    check("mars_accept_commit", code)
    return n_accepted, accepted_ids, commit_pos


def mars_accept_commit_layers(p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table,
                              cache_len, *, n_accepted=None, accepted_ids=None, commit_pos=None,
                              status=None, stream=None):
    """As mars_accept_commit, committing into every layer: k_new/v_new
    [layers,S,B,Hkv,d], k_cache [layers,pages,Hkv,page,d], v_cache
    [layers,pages,Hkv,d,page]; one block table and cache_len for all layers.
    Returns (n_accepted [S], accepted_ids [S,B], commit_pos [S,B])."""
    S, B, Hkv, d, page, num_pages, layers = _commit_args(
        p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_accepted,
        accepted_ids, commit_pos, status, layered=True)
    n_accepted, accepted_ids, commit_pos = _commit_outputs(p_max, n_accepted, accepted_ids,
                                                           commit_pos)
    code = _lib.lib().mars_accept_commit_layers(
        _ptr(p_max), _ptr(top_id), _ptr(tau), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), _ptr(cache_len), _ptr(n_accepted), _ptr(accepted_ids),
        _ptr(commit_pos), layers, S, B, Hkv, d, page, block_table.shape[1], num_pages,
        _DT.get(k_new.dtype, -1), _ptr(status), _stream(stream))
    check("mars_accept_commit_layers", code)
    return n_accepted, accepted_ids, commit_pos


def mars_lmhead_confidence_noalloc(hidden, w_lm, logits=None, *, top_id=None, p_max=None,
                                   status=None, stream=None, fused=False):
    """As mars_lmhead_confidence (row-major w_lm [V, D], or hidden None with `logits`
    as the input), with no workspace: the library keeps the partials in its own
    fixed device array (for callers that cannot allocate device memory). Pass
    top_id and p_max to allocate nothing here either. Returns (logits, top_id, p_max)."""
    if isinstance(w_lm, PackedLMHead):
        raise ValueError("the no-workspace call takes row-major weights [V, D]")
    if hidden is not None:
        _need(hidden, "hidden", torch.bfloat16, 2)
        N, D = hidden.shape
        _need(w_lm, "w_lm", torch.bfloat16, 2)
        V = w_lm.shape[0]
        if w_lm.shape[1] != D:
            raise ValueError(f"w_lm must be [V, {D}] (got {tuple(w_lm.shape)})")
        if fused:
            if logits is not None:
                raise ValueError("fused=True writes no logits; pass logits=None")
        else:
            _opt(logits, "logits", torch.float32, 2, (N, V))
    else:
        if logits is None or fused:
            raise ValueError("logits are required (and fused is off) when hidden is None")
        _need(logits, "logits", torch.float32, 2)
        N, V = logits.shape
        D = 0
    _opt(top_id, "top_id", torch.int32, 1, (N,))
    _opt(p_max, "p_max", torch.float32, 1, (N,))
    _status(status)
    _on_gpu(hidden=hidden, w_lm=w_lm if hidden is not None else None, logits=logits,
            top_id=top_id, p_max=p_max, status=status)
    dev = hidden.device if hidden is not None else logits.device
    if logits is None and not fused:
        logits = torch.empty((N, V), dtype=torch.float32, device=dev)
    if top_id is None:
        top_id = torch.empty(N, dtype=torch.int32, device=dev)
    if p_max is None:
        p_max = torch.empty(N, dtype=torch.float32, device=dev)
    code = _lib.lib().mars_lmhead_confidence_noalloc(
        _ptr(hidden), _ptr(w_lm) if hidden is not None else None, _ptr(logits), N, D, V,
        _ptr(top_id), _ptr(p_max), _ptr(status), _stream(stream))
    check("mars_lmhead_confidence_noalloc", code)
    return logits, top_id, p_max
