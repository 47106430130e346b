"""The C-ABI library: loads, exports every declared symbol, rejects bad arguments
on the host (no GPU needed: every call here fails its checks before any launch)."""

import ctypes
import os
import re

import pytest

import block_masked_causal_amd as mars
from block_masked_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mars.h")

# A fake, 16-byte-aligned device address. It is only ever passed to calls that
# must be rejected by a host-side check before any kernel is enqueued.
FAKE = 0x7F0000000000
MIS = FAKE + 8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mars_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 8
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must match the header"


def test_version_and_strerror():
    assert mars.lib().mars_version() >= 100
    for code in range(0, -8, -1):
        assert mars.strerror(code) != "unknown error code"
    assert mars.strerror(-99) == "unknown error code"


def ts(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, batch=1, L=64, B=4, Hq=2, Hkv=2, d=32,
       dtype=0, mode=0):
    return mars.lib().mars_attn_two_stream(q, k, v, o, lse, batch, L, B, Hq, Hkv, d, dtype,
                                           0.0, mode, None)


def test_two_stream_argument_checks():
    assert ts(q=None) == _lib.MARS_ERR_NULL
    assert ts(dtype=7) == _lib.MARS_ERR_DTYPE
    assert ts(B=0) == _lib.MARS_ERR_SHAPE
    assert ts(B=65) == _lib.MARS_ERR_SHAPE          # B > L
    assert ts(Hq=3, Hkv=2) == _lib.MARS_ERR_SHAPE   # Hq % Hkv != 0
    assert ts(mode=2) == _lib.MARS_ERR_SHAPE
    assert ts(q=MIS) == _lib.MARS_ERR_ALIGN
    assert ts(lse=MIS) == _lib.MARS_ERR_ALIGN
    assert ts(d=48) == _lib.MARS_ERR_UNSUPPORTED
    assert ts(d=32, dtype=1) == _lib.MARS_ERR_UNSUPPORTED  # bf16 path: d in {64, 128}


def dec(S=2, B=4, Hq=4, Hkv=2, d=128, page=16, max_pages=4, num_pages=8, dtype=1, ws=FAKE,
        ws_bytes=1 << 30, q=FAKE, table=FAKE):
    return mars.lib().mars_attn_block_decode(q, FAKE, FAKE, FAKE, FAKE, table, FAKE, FAKE, S, B,
                                             Hq, Hkv, d, page, max_pages, num_pages, dtype, 0.0,
                                             ws, ws_bytes, None, None)


def bwd(dtype=1, d=64, ws=FAKE, ws_bytes=1 << 20, q=FAKE, B=4, L=16, mode=0):
    return mars.lib().mars_attn_two_stream_bwd(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                               1, L, B, 4, 2, d, dtype, 0.0, mode, ws, ws_bytes,
                                               None)


def test_two_stream_bwd_argument_checks():
    # every case is rejected before any launch: the fake addresses are never used
    assert bwd(q=None) == _lib.MARS_ERR_NULL
    assert bwd(dtype=0) == _lib.MARS_ERR_DTYPE            # fp32 has no backward
    assert bwd(d=32) == _lib.MARS_ERR_UNSUPPORTED
    assert bwd(B=17) == _lib.MARS_ERR_SHAPE               # B > L
    assert bwd(mode=2) == _lib.MARS_ERR_SHAPE
    assert bwd(q=MIS) == _lib.MARS_ERR_ALIGN
    need = mars.lib().mars_attn_two_stream_bwd_workspace_bytes(1, 16, 4, 2, 64)
    rows = 1 * 32 * 4
    assert need == rows * 4 + 2 * rows * 64 * 4               # rowsum, dK and dV partials
    assert mars.lib().mars_attn_two_stream_bwd_workspace_bytes(1, 16, 2, 2, 64) == 256
    assert mars.lib().mars_attn_two_stream_bwd_workspace_bytes(1, 16, 3, 2, 64) == 0
    assert bwd(ws_bytes=need - 1) == _lib.MARS_ERR_WORKSPACE
    assert bwd(ws=None) == _lib.MARS_ERR_WORKSPACE


def test_causal_and_append_argument_checks():
    L_ = mars.lib()
    # rejected before any launch
    assert L_.mars_attn_causal(None, FAKE, FAKE, FAKE, None, 1, 9, 2, 1, 64, 1, 0.0,
                               None) == _lib.MARS_ERR_NULL
    assert L_.mars_attn_causal(FAKE, FAKE, FAKE, FAKE, None, 1, 0, 2, 1, 64, 1, 0.0,
                               None) == _lib.MARS_ERR_SHAPE
    assert L_.mars_attn_causal(FAKE, FAKE, FAKE, FAKE, None, 1, 9, 3, 2, 64, 1, 0.0,
                               None) == _lib.MARS_ERR_SHAPE
    assert L_.mars_attn_causal(FAKE, FAKE, FAKE, FAKE, None, 1, 9, 2, 1, 64, 7, 0.0,
                               None) == _lib.MARS_ERR_DTYPE
    assert L_.mars_attn_causal(MIS, FAKE, FAKE, FAKE, None, 1, 9, 2, 1, 64, 1, 0.0,
                               None) == _lib.MARS_ERR_ALIGN
    ap = lambda **kw: L_.mars_kv_append(kw.get("k", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE,
                                        kw.get("S", 2), kw.get("T", 5), 2, kw.get("d", 64),
                                        16, 4, 8, kw.get("dt", 1), None, None)
    assert ap(k=None) == _lib.MARS_ERR_NULL
    assert ap(T=0) == _lib.MARS_ERR_SHAPE
    assert ap(d=12) == _lib.MARS_ERR_SHAPE
    assert ap(dt=5) == _lib.MARS_ERR_DTYPE
    assert ap(k=MIS) == _lib.MARS_ERR_ALIGN
    assert ap(d=512) == _lib.MARS_ERR_UNSUPPORTED          # 1 KiB V rows exceed the staging


def test_decode_argument_checks():
    assert dec(q=None) == _lib.MARS_ERR_NULL
    assert dec(dtype=5) == _lib.MARS_ERR_DTYPE
    assert dec(B=65) == _lib.MARS_ERR_SHAPE                 # more than 64 new rows
    assert dec(Hq=6, Hkv=4) == _lib.MARS_ERR_SHAPE          # heads not a multiple
    assert dec(page=8) == _lib.MARS_ERR_SHAPE
    assert dec(page=24) == _lib.MARS_ERR_SHAPE
    assert dec(num_pages=0) == _lib.MARS_ERR_SHAPE
    assert dec(dtype=0) == _lib.MARS_ERR_UNSUPPORTED
    assert dec(d=96) == _lib.MARS_ERR_UNSUPPORTED
    assert dec(table=MIS) == _lib.MARS_ERR_ALIGN
    need = mars.mars_decode_workspace_bytes(2, 4, 4, 2, 128, 16, 4)
    assert need > 0
    assert dec(ws_bytes=need - 1) == _lib.MARS_ERR_WORKSPACE
    assert dec(ws=None) == _lib.MARS_ERR_WORKSPACE
    assert mars.mars_decode_workspace_bytes(2, 4, 4, 2, 96, 16, 4) == 0


def test_block_cache_argument_checks():
    L_ = mars.lib()
    rows = lambda **kw: L_.mars_attn_block_decode_rows(
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("n_rows", FAKE), FAKE, 2,
        kw.get("R", 8), 4, 2, 128, 16, 4, 8, 1, 0.0, FAKE, kw.get("ws_bytes", 1 << 30), None,
        None)
    assert rows(n_rows=None) == _lib.MARS_ERR_NULL
    assert rows(R=65) == _lib.MARS_ERR_SHAPE
    assert rows(n_rows=MIS) == _lib.MARS_ERR_ALIGN
    assert rows(ws_bytes=16) == _lib.MARS_ERR_WORKSPACE
    acc = lambda **kw: L_.mars_block_sync_accept(
        kw.get("p", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("S", 4), kw.get("B", 4),
        kw.get("Bc", 16), kw.get("policy", 0), None, None)
    assert acc(p=None) == _lib.MARS_ERR_NULL
    assert acc(B=65) == _lib.MARS_ERR_SHAPE
    assert acc(Bc=0) == _lib.MARS_ERR_SHAPE
    assert acc(policy=2) == _lib.MARS_ERR_SHAPE
    assert acc(S=0) == _lib.MARS_ERR_SHAPE
    frz = lambda **kw: L_.mars_block_freeze(
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("u", FAKE), 2, kw.get("R", 20),
        kw.get("Bc", 16), 2, kw.get("d", 64), 16, 4, 8, kw.get("dt", 1), None, None)
    assert frz(u=None) == _lib.MARS_ERR_NULL
    assert frz(Bc=21) == _lib.MARS_ERR_SHAPE                # block larger than the rows
    assert frz(Bc=0) == _lib.MARS_ERR_SHAPE
    assert frz(dt=3) == _lib.MARS_ERR_DTYPE
    assert frz(d=1024) == _lib.MARS_ERR_UNSUPPORTED
    assert frz(u=MIS) == _lib.MARS_ERR_ALIGN


def test_decode_workspace_grows_with_capacity():
    a = mars.mars_decode_workspace_bytes(64, 4, 28, 4, 128, 16, 64)
    b = mars.mars_decode_workspace_bytes(64, 4, 28, 4, 128, 16, 257)
    assert 0 < a < b


def lm(hidden=FAKE, w=FAKE, logits=FAKE, N=16, D=64, V=1000, ws=FAKE, ws_bytes=1 << 20):
    return mars.lib().mars_lmhead_confidence(hidden, w, logits, N, D, V, FAKE, FAKE, ws, ws_bytes,
                                             None, None)


def test_lmhead_argument_checks():
    # logits may be omitted only with an LM head (fused form); every case below is
    # rejected before any launch, so the fake addresses are never dereferenced
    assert lm(hidden=None, w=None, logits=None) == _lib.MARS_ERR_NULL
    assert mars.lib().mars_lmhead_confidence(FAKE, FAKE, None, 16, 64, 1000, None, FAKE, FAKE,
                                             1 << 20, None, None) == _lib.MARS_ERR_NULL
    assert lm(w=None) == _lib.MARS_ERR_NULL
    assert lm(V=1002) == _lib.MARS_ERR_SHAPE      # V % 4 != 0
    assert lm(D=48) == _lib.MARS_ERR_SHAPE        # D % 32 != 0 with an LM head
    assert lm(N=0) == _lib.MARS_ERR_SHAPE
    assert lm(logits=MIS) == _lib.MARS_ERR_ALIGN
    need = mars.mars_lmhead_workspace_bytes(16, 1000)
    assert need > 0
    assert lm(ws_bytes=need - 1) == _lib.MARS_ERR_WORKSPACE
    assert mars.mars_lmhead_workspace_bytes(16, 1001) == 0


def test_lmhead_packing_argument_checks():
    L_ = mars.lib()
    assert L_.mars_lmhead_packed_bytes(3584, 152064) == 476 * 320 * 3584 * 2
    assert L_.mars_lmhead_packed_bytes(64, 1000) == 4 * 320 * 64 * 2   # padded to 1280 rows
    assert L_.mars_lmhead_packed_bytes(48, 1000) == 0                   # D % 32 != 0
    assert L_.mars_lmhead_packed_bytes(64, 1002) == 0                   # V % 4 != 0
    assert L_.mars_lmhead_pack(None, FAKE, 64, 1000, None) == _lib.MARS_ERR_NULL
    assert L_.mars_lmhead_pack(FAKE, FAKE, 48, 1000, None) == _lib.MARS_ERR_SHAPE
    assert L_.mars_lmhead_pack(MIS, FAKE, 64, 1000, None) == _lib.MARS_ERR_ALIGN
    pk = lambda **kw: L_.mars_lmhead_confidence_packed(
        kw.get("h", FAKE), kw.get("w", FAKE), None, 16, kw.get("D", 64), 1000, FAKE, FAKE,
        FAKE, kw.get("ws", 1 << 20), None, None)
    assert pk(h=None) == _lib.MARS_ERR_NULL      # a packed head needs hidden states
    assert pk(w=None) == _lib.MARS_ERR_NULL
    assert pk(D=48) == _lib.MARS_ERR_SHAPE
    assert pk(ws=16) == _lib.MARS_ERR_WORKSPACE


def ac(p=FAKE, S=4, B=4, Hkv=2, d=32, page=16, max_pages=4, num_pages=16, dtype=1, kc=FAKE):
    return mars.lib().mars_accept_commit(p, FAKE, FAKE, FAKE, FAKE, kc, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, S, B, Hkv, d, page, max_pages, num_pages,
                                         dtype, None, None)


def test_accept_commit_argument_checks():
    assert ac(p=None) == _lib.MARS_ERR_NULL
    assert ac(dtype=3) == _lib.MARS_ERR_DTYPE
    assert ac(B=0) == _lib.MARS_ERR_SHAPE
    assert ac(B=65) == _lib.MARS_ERR_SHAPE
    assert ac(d=12) == _lib.MARS_ERR_SHAPE
    assert ac(num_pages=0) == _lib.MARS_ERR_SHAPE
    assert ac(kc=MIS) == _lib.MARS_ERR_ALIGN


def acl(layers=2, S=4, B=4, kc=FAKE):
    return mars.lib().mars_accept_commit_layers(FAKE, FAKE, FAKE, FAKE, FAKE, kc, FAKE, FAKE,
                                                FAKE, FAKE, FAKE, FAKE, layers, S, B, 2, 32, 16,
                                                4, 16, 1, None, None)


def test_layered_commit_argument_checks():
    assert acl(layers=0) == _lib.MARS_ERR_SHAPE
    assert acl(layers=65536) == _lib.MARS_ERR_SHAPE
    assert acl(B=65) == _lib.MARS_ERR_SHAPE
    assert acl(kc=MIS) == _lib.MARS_ERR_ALIGN
    assert acl(kc=None) == _lib.MARS_ERR_NULL


def test_binding_rejects_cpu_tensors_before_calling():
    import torch
    q = torch.zeros(1, 8, 2, 32)
    with pytest.raises(ValueError):
        mars.mars_attn_two_stream(q, q, q, 4, 2)


def _cpu(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _shape_error(fn, *args, match, **kw):
    """The call must fail on the named shape check, not on the GPU-residency check
    that comes last (these tensors live on the CPU)."""
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def _gpu_error(fn, *args, **kw):
    """Shapes are right: the only complaint left is that the tensors are on the CPU."""
    with pytest.raises(ValueError, match="GPU tensor"):
        fn(*args, **kw)


def _decode_set(S=2, B=4, Hq=4, Hkv=2, d=64, pages=6, page=16, max_pages=3):
    import torch
    return dict(q=_cpu((S, B, Hq, d)), k_new=_cpu((S, B, Hkv, d)), v_new=_cpu((S, B, Hkv, d)),
                k_cache=_cpu((pages, Hkv, page, d)), v_cache=_cpu((pages, Hkv, d, page)),
                block_table=_cpu((S, max_pages), torch.int32), cache_len=_cpu((S,), torch.int32))


def test_binding_checks_every_shape_of_the_decode_call():
    import torch
    a = _decode_set()
    call = lambda **kw: mars.mars_attn_block_decode(*[{**a, **kw}[n] for n in (
        "q", "k_new", "v_new", "k_cache", "v_cache", "block_table", "cache_len")],
        **{k: v for k, v in kw.items() if k in ("o", "n_rows", "workspace", "status")})
    _gpu_error(call)
    _shape_error(call, match="o must have shape", o=_cpu((2, 4, 4, 32)))
    _shape_error(call, match="k_new must have shape", k_new=_cpu((2, 3, 2, 64)))
    _shape_error(call, match="v_new must have shape", v_new=_cpu((2, 4, 1, 64)))
    _shape_error(call, match="k_cache must be", k_cache=_cpu((6, 2, 16, 32)))
    _shape_error(call, match="v_cache must have shape", v_cache=_cpu((6, 2, 16, 64)))
    _shape_error(call, match="block_table must have 2 rows",
                 block_table=_cpu((3, 3), torch.int32))
    _shape_error(call, match="cache_len must have shape", cache_len=_cpu((3,), torch.int32))
    _shape_error(call, match="n_rows must have shape", n_rows=_cpu((1,), torch.int32))
    _shape_error(call, match="workspace holds", workspace=_cpu((16,), torch.uint8))
    _shape_error(call, match="status must hold", status=_cpu((0,), torch.int32))


def test_binding_checks_every_shape_of_accept_commit():
    import torch
    a = _decode_set(B=4)
    S, B = 2, 4
    base = dict(p_max=_cpu((S, B), torch.float32), top_id=_cpu((S, B), torch.int32),
                tau=_cpu((S,), torch.float32), k_new=a["k_new"], v_new=a["v_new"],
                k_cache=a["k_cache"], v_cache=a["v_cache"], block_table=a["block_table"],
                cache_len=a["cache_len"])
    names = list(base)

    def call(**kw):
        args = {**base, **kw}
        outs = {k: v for k, v in kw.items() if k in ("n_accepted", "accepted_ids",
                                                      "commit_pos", "status")}
        return mars.mars_accept_commit(*[args[n] for n in names], **outs)

    _gpu_error(call)
    _shape_error(call, match="top_id must have shape", top_id=_cpu((S, B + 1), torch.int32))
    _shape_error(call, match="tau must have shape", tau=_cpu((S + 1,), torch.float32))
    _shape_error(call, match="cache_len must have shape", cache_len=_cpu((1,), torch.int32))
    _shape_error(call, match="block_table must have 2 rows",
                 block_table=_cpu((1, 3), torch.int32))
    _shape_error(call, match="k_new must have shape", k_new=_cpu((S, B - 1, 2, 64)))
    _shape_error(call, match="v_new must have shape", v_new=_cpu((S, B, 2, 32)))
    _shape_error(call, match="k_cache must be", k_cache=_cpu((6, 1, 16, 64)))
    _shape_error(call, match="v_cache must have shape", v_cache=_cpu((6, 2, 16, 64)))
    _shape_error(call, match="n_accepted must have shape",
                 n_accepted=_cpu((S + 1,), torch.int32))
    _shape_error(call, match="accepted_ids must have shape",
                 accepted_ids=_cpu((S, B - 1), torch.int32))
    _shape_error(call, match="commit_pos must have shape",
                 commit_pos=_cpu((S, 1), torch.int32))


def test_binding_checks_shapes_of_append_freeze_and_block_sync():
    import torch
    S, T, Hkv, d = 2, 5, 2, 64
    kr, vr = _cpu((S, T, Hkv, d)), _cpu((S, T, Hkv, d))
    kc, vc = _cpu((6, Hkv, 16, d)), _cpu((6, Hkv, d, 16))
    bt, cl = _cpu((S, 3), torch.int32), _cpu((S,), torch.int32)
    _gpu_error(mars.mars_kv_append, kr, vr, kc, vc, bt, cl)
    _shape_error(mars.mars_kv_append, kr, _cpu((S, T - 1, Hkv, d)), kc, vc, bt, cl,
                 match="v_rows must have shape")
    _shape_error(mars.mars_kv_append, kr, vr, kc, _cpu((6, Hkv, 16, d)), bt, cl,
                 match="v_cache must have shape")
    _shape_error(mars.mars_kv_append, kr, vr, kc, vc, bt, _cpu((S + 2,), torch.int32),
                 match="cache_len must have shape")
    un = _cpu((S,), torch.int32)
    _gpu_error(mars.mars_block_freeze, kr, vr, kc, vc, bt, cl, un, 4)
    _shape_error(mars.mars_block_freeze, kr, vr, kc, vc, bt, cl, _cpu((S + 1,), torch.int32),
                 4, match="unfrozen must have shape")
    _shape_error(mars.mars_block_freeze, kr, vr, kc, vc, _cpu((S + 1, 3), torch.int32), cl,
                 un, 4, match="block_table must have")
    pm, ids, tau = _cpu((S, 4), torch.float32), _cpu((S, 4), torch.int32), _cpu((S,),
                                                                               torch.float32)
    toks = _cpu((S, 8), torch.int32)
    _gpu_error(mars.mars_block_sync_accept, pm, ids, tau, un, toks)
    _shape_error(mars.mars_block_sync_accept, pm, ids, _cpu((1,), torch.float32), un, toks,
                 match="tau must have shape")
    _shape_error(mars.mars_block_sync_accept, pm, ids, tau, un, _cpu((S + 1, 8), torch.int32),
                 match="block_tokens must have")
    _shape_error(mars.mars_block_sync_accept, pm, ids, tau, un, toks,
                 n_rows=_cpu((S + 1,), torch.int32), match="n_rows must have shape")


def test_binding_checks_shapes_of_attention_calls():
    import torch
    b, L, Hq, Hkv, d = 1, 8, 4, 2, 64
    q, k = _cpu((b, 2 * L, Hq, d)), _cpu((b, 2 * L, Hkv, d))
    _gpu_error(mars.mars_attn_two_stream, q, k, k, L, 2)
    _shape_error(mars.mars_attn_two_stream, q, k, k, L + 1, 2, match="2L")
    _shape_error(mars.mars_attn_two_stream, q, k, _cpu((b, 2 * L, Hkv, 32)), L, 2,
                 match="v must have shape")
    _shape_error(mars.mars_attn_two_stream, q, k, k, L, 2, o=_cpu((b, 2 * L, Hq, 32)),
                 match="o must have shape")
    _shape_error(mars.mars_attn_two_stream, q, k, k, L, 2,
                 lse=_cpu((b, Hq, L), torch.float32), match="lse must have shape")
    _shape_error(mars.mars_attn_causal, q, k, k, o=_cpu((b, 2 * L, Hq + 1, d)),
                 match="o must have shape")
    lse = _cpu((b, Hq, 2 * L), torch.float32)
    _gpu_error(mars.mars_attn_two_stream_bwd, q, k, k, q, q, lse, L, 2)
    _shape_error(mars.mars_attn_two_stream_bwd, q, k, k, q, q, lse, L, 2,
                 dk=_cpu((b, 2 * L, Hq, d)), match="dk must have shape")
    _shape_error(mars.mars_attn_two_stream_bwd, q, k, k, q, q, lse, L, 2,
                 workspace=_cpu((8,), torch.uint8), match="workspace holds")
    _shape_error(mars.mars_attn_two_stream_bwd, q, k, k, _cpu((b, 2 * L, Hq, 32)), q, lse, L,
                 2, match="o must have shape")


def test_binding_checks_shapes_of_the_lm_head_call():
    import torch
    N, D, V = 4, 64, 128
    h, w = _cpu((N, D)), _cpu((V, D))
    _gpu_error(mars.mars_lmhead_confidence, h, w)
    _shape_error(mars.mars_lmhead_confidence, h, _cpu((V, D + 32)), match="w_lm must be")
    _shape_error(mars.mars_lmhead_confidence, h, w, _cpu((N, V + 4), torch.float32),
                 match="logits must have shape")
    _shape_error(mars.mars_lmhead_confidence, h, w, top_id=_cpu((N + 1,), torch.int32),
                 match="top_id must have shape")
    _shape_error(mars.mars_lmhead_confidence, h, w, p_max=_cpu((N - 1,), torch.float32),
                 match="p_max must have shape")
    _shape_error(mars.mars_lmhead_confidence, None, None, _cpu((N, V), torch.float32),
                 workspace=_cpu((1,), torch.uint8), match="workspace holds")


def test_oracle_is_not_imported_by_the_package():
    import sys
    for name in list(sys.modules):
        if name == "oracle" or name.startswith("oracle."):
            mod = sys.modules[name]
            del mod
    import importlib
    importlib.reload(mars)
    pkg_dir = os.path.dirname(mars.__file__)
    for fn in os.listdir(pkg_dir):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg_dir, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn


def test_binding_checks_every_shape_of_the_layered_commit():
    import torch
    S, B, Hkv, d, L = 2, 4, 2, 64, 3
    base = dict(p_max=_cpu((S, B), torch.float32), top_id=_cpu((S, B), torch.int32),
                tau=_cpu((S,), torch.float32), k_new=_cpu((L, S, B, Hkv, d)),
                v_new=_cpu((L, S, B, Hkv, d)), k_cache=_cpu((L, 6, Hkv, 16, d)),
                v_cache=_cpu((L, 6, Hkv, d, 16)), block_table=_cpu((S, 3), torch.int32),
                cache_len=_cpu((S,), torch.int32))
    names = list(base)

    def call(**kw):
        args = {**base, **kw}
        outs = {k: v for k, v in kw.items() if k in ("n_accepted", "accepted_ids",
                                                      "commit_pos", "status")}
        return mars.mars_accept_commit_layers(*[args[n] for n in names], **outs)

    _gpu_error(call)
    _shape_error(call, match="k_new must have 5 dims", k_new=_cpu((S, B, Hkv, d)))
    _shape_error(call, match="v_new must have shape", v_new=_cpu((L - 1, S, B, Hkv, d)))
    _shape_error(call, match="k_cache must hold 3 layers", k_cache=_cpu((2, 6, Hkv, 16, d)))
    _shape_error(call, match="v_cache must hold 3 layers", v_cache=_cpu((2, 6, Hkv, d, 16)))
    _shape_error(call, match="v_cache must have shape", v_cache=_cpu((L, 6, Hkv, 16, d)))
    _shape_error(call, match="k_cache must be", k_cache=_cpu((L, 6, 1, 16, d)))
    _shape_error(call, match="block_table must have 2 rows",
                 block_table=_cpu((1, 3), torch.int32))
    _shape_error(call, match="commit_pos must have shape",
                 commit_pos=_cpu((S, 1), torch.int32))
