"""The C ABI: the library loads, exports every entry point include/focus.h declares, and rejects
every bad-argument class on the host, before any launch (so these run without a GPU).

Fake device pointers below are never dereferenced: each call fails validation first.
"""
import ctypes
import math
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "focus.h")
OK, ARG, SHAPE, UNSUP, ALIGN, WS = 0, -1, -2, -3, -4, -5
P = 4096          # an aligned fake pointer
MIS = 4096 + 2    # misaligned for every buffer kind
BIG = 1 << 40     # a workspace size large enough for any case here


@pytest.fixture(scope="module")
def lib():
    from learned_centroid_gated_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfocus.so not built (run __graft_entry__.build())")
    return _lib.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(focus_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) == 24, names
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.focus_version() >= 100
    for code in (OK, ARG, SHAPE, UNSUP, ALIGN, WS, -6, -7):
        assert lib.focus_status_string(code).decode().startswith("FOCUS_")
    assert b"UNKNOWN" in lib.focus_status_string(-99)


def _assign(lib, hidden=P, w=P, c=P, n=128, d=64, dg=16, K=8, top_k=2, iters=3, groups=P, v=P,
            ws=P, wsb=BIG):
    return lib.focus_assign(hidden, w, c, n, d, dg, K, top_k, iters, groups, v, ws, wsb, None)


def test_assign_validation(lib):
    assert _assign(lib, n=-1) == ARG
    assert _assign(lib, dg=0) == ARG
    assert _assign(lib, dg=2048) == ARG
    assert _assign(lib, iters=-1) == ARG
    assert _assign(lib, K=0) == ARG
    assert _assign(lib, K=2000) == ARG
    assert _assign(lib, top_k=0) == ARG
    assert _assign(lib, top_k=9, K=8) == ARG
    assert _assign(lib, top_k=9, K=16) == UNSUP
    assert _assign(lib, d=66) == UNSUP
    assert _assign(lib, dg=18) == UNSUP
    assert _assign(lib, n=1 << 30, top_k=2) == SHAPE
    assert _assign(lib, hidden=None) == ARG
    assert _assign(lib, groups=None) == ARG
    assert _assign(lib, hidden=MIS) == ALIGN
    assert _assign(lib, v=MIS) == ALIGN
    assert _assign(lib, ws=MIS) == ALIGN
    assert _assign(lib, ws=None) == WS
    assert _assign(lib, wsb=16) == WS
    assert _assign(lib, n=0, hidden=None, groups=None) == OK  # empty: nothing enqueued


def test_assign_workspace_size(lib):
    f = lib.focus_assign_workspace_size
    assert f(-1, 8, 8, 8) == 0
    a, b = f(1000, 768, 64, 16), f(2000, 768, 64, 16)
    assert 0 < a < b
    # the scores alone take n * K floats
    assert f(1 << 20, 4096, 128, 256) >= (1 << 20) * 256 * 4


def _bucket(lib, groups=P, batch=1, n=100, K=8, top_k=2, off=P, idx=P, slot=P, ws=P, wsb=BIG):
    return lib.focus_bucket(groups, batch, n, K, top_k, off, idx, slot, ws, wsb, None)


def test_bucket_validation(lib):
    assert _bucket(lib, batch=0) == ARG
    assert _bucket(lib, n=-5) == ARG
    assert _bucket(lib, K=0) == ARG
    assert _bucket(lib, top_k=9, K=16) == UNSUP
    assert _bucket(lib, top_k=3, K=2) == ARG
    assert _bucket(lib, n=1 << 31, top_k=1) == SHAPE
    assert _bucket(lib, off=None) == ARG
    assert _bucket(lib, idx=None) == ARG
    assert _bucket(lib, slot=MIS) == ALIGN
    assert _bucket(lib, wsb=0) == WS
    assert lib.focus_bucket_workspace_size(2, 1000, 16, 2) >= 2 * 16 * 4 * 4


def _attn(lib, q=P, k=P, v=P, n=256, Hq=8, Hkv=2, dh=128, groups=P, off=P, idx=P, slot=P, K=8,
          top_k=2, window=16, scale=0.0, out=P, lse=P, ws=P, wsb=BIG):
    return lib.focus_attention(q, k, v, n, Hq, Hkv, dh, groups, off, idx, slot, K, top_k, window,
                               scale, out, lse, ws, wsb, None)


def test_attention_validation(lib):
    assert _attn(lib, n=-1) == ARG
    assert _attn(lib, window=-1) == ARG
    assert _attn(lib, Hq=6, Hkv=4) == ARG
    assert _attn(lib, Hq=6, Hkv=2) == UNSUP   # G = 3
    assert _attn(lib, Hq=64, Hkv=2) == UNSUP  # G = 32
    assert _attn(lib, dh=96) == UNSUP
    assert _attn(lib, top_k=5, K=8) == UNSUP
    assert _attn(lib, top_k=9, K=8) == ARG
    assert _attn(lib, scale=math.nan) == ARG
    assert _attn(lib, scale=math.inf) == ARG
    assert _attn(lib, n=1 << 30, top_k=2) == SHAPE
    assert _attn(lib, q=None) == ARG
    assert _attn(lib, slot=None) == ARG
    assert _attn(lib, lse=MIS) == ALIGN
    assert _attn(lib, wsb=1) == WS
    assert _attn(lib, n=0, q=None) == OK


def test_attention_workspace_size(lib):
    f = lib.focus_attention_workspace_size
    n, Hq, Hkv, dh, K, k = 131072, 64, 8, 128, 128, 2
    # gathered K/V (bf16), fp16 group partials, their log-sum-exp and the key records
    floor = n * k * 2 * Hkv * dh * 2 + n * k * Hq * dh * 2 + n * k * Hq * 4 + n * k * 16
    assert f(n, Hq, Hkv, dh, K, k) >= floor


def _append(lib, ng=P, ln=P, B=4, L=1024, K=16, top_k=2, oi=P, ii=P + 65536, oo=P + 4096,
            io=P + 131072):
    return lib.focus_bucket_append(ng, ln, B, L, K, top_k, oi, ii, oo, io, None)


def test_bucket_append_validation(lib):
    assert _append(lib, B=0) == ARG
    assert _append(lib, L=0) == ARG
    assert _append(lib, K=0) == ARG
    assert _append(lib, top_k=9, K=16) == UNSUP
    assert _append(lib, L=1 << 30, top_k=4) == SHAPE
    assert _append(lib, ng=None) == ARG
    assert _append(lib, ln=None) == ARG
    assert _append(lib, oo=P) == ARG          # in place is refused
    assert _append(lib, io=P + 65536) == ARG
    assert _append(lib, ln=MIS) == ALIGN
    assert _append(lib, io=MIS) == ALIGN


def _soft(lib, q=P, k=P, v=P, n=256, Hq=8, Hkv=2, dh=128, g=P, K=16, top_k=2, window=32,
          lam=10.0, scale=0.0, out=P, lse=P):
    return lib.focus_soft_attention(q, k, v, n, Hq, Hkv, dh, g, K, top_k, window, lam, scale, out,
                                    lse, None)


def test_soft_attention_validation(lib):
    assert _soft(lib, n=-1) == ARG
    assert _soft(lib, window=-1) == ARG
    assert _soft(lib, lam=math.nan) == ARG
    assert _soft(lib, lam=math.inf) == ARG
    assert _soft(lib, scale=math.nan) == ARG
    assert _soft(lib, Hq=6, Hkv=4) == ARG
    assert _soft(lib, Hq=6, Hkv=2) == UNSUP
    assert _soft(lib, dh=96) == UNSUP
    assert _soft(lib, K=0) == ARG
    assert _soft(lib, top_k=5, K=16) == UNSUP
    assert _soft(lib, n=1 << 30, top_k=2) == SHAPE
    assert _soft(lib, q=None) == ARG
    assert _soft(lib, g=None) == ARG
    assert _soft(lib, lse=None) == ARG
    assert _soft(lib, k=MIS) == ALIGN
    assert _soft(lib, out=MIS) == ALIGN
    assert _soft(lib, n=0, q=None) == OK  # empty: nothing enqueued


def _asym(lib, q=P, k=P, v=P, n=256, Hq=8, Hkv=2, dh=128, qo=P, qi=P, qs=P, top_k=2, ko=P, ki=P,
          ks=P, K=16, window=64, scale=0.0, out=P, lse=P, ws=P, wsb=BIG):
    return lib.focus_attention_asym(q, k, v, n, Hq, Hkv, dh, qo, qi, qs, top_k, ko, ki, ks, K,
                                    window, scale, out, lse, ws, wsb, None)


def test_attention_asym_validation(lib):
    assert _asym(lib, n=-1) == ARG
    assert _asym(lib, window=-1) == ARG
    assert _asym(lib, scale=math.nan) == ARG
    assert _asym(lib, Hq=6, Hkv=4) == ARG
    assert _asym(lib, Hq=6, Hkv=2) == UNSUP
    assert _asym(lib, dh=96) == UNSUP
    assert _asym(lib, K=0) == ARG
    assert _asym(lib, top_k=5, K=16) == UNSUP
    assert _asym(lib, n=1 << 30, top_k=2) == SHAPE
    for name in ("q", "qo", "qi", "qs", "ko", "ki", "ks", "out", "lse"):
        assert _asym(lib, **{name: None}) == ARG, name
    assert _asym(lib, v=MIS) == ALIGN
    assert _asym(lib, ki=P + 2) == ALIGN
    assert _asym(lib, ws=None) == WS
    assert _asym(lib, wsb=16) == WS
    assert _asym(lib, n=0, q=None) == OK  # empty: nothing enqueued
    small = lib.focus_attention_asym_workspace_size(1000, 8, 2, 128, 16, 2)
    sym = lib.focus_attention_workspace_size(1000, 8, 2, 128, 16, 2)
    assert 0 < small < sym  # K/V gathered once per token, not once per membership
    assert lib.focus_attention_asym_workspace_size(-1, 8, 2, 128, 16, 2) == 0


def _decode(lib, q=P, qg=P, kc=P, vc=P, ln=P, cg=P, co=P, ci=P, B=4, L=1024, Hq=8, Hkv=2, dh=128,
            K=16, top_k=2, window=64, scale=0.0, out=P, lse=P, ws=P, wsb=BIG):
    return lib.focus_decode(q, qg, kc, vc, ln, cg, co, ci, B, L, Hq, Hkv, dh, K, top_k, window,
                            scale, out, lse, ws, wsb, None)


def test_decode_validation(lib):
    assert _decode(lib, B=-1) == ARG
    assert _decode(lib, L=0) == ARG
    assert _decode(lib, window=-3) == ARG
    assert _decode(lib, dh=32) == UNSUP
    assert _decode(lib, top_k=5) == UNSUP
    assert _decode(lib, L=1 << 31, top_k=1) == SHAPE
    assert _decode(lib, cg=None) == ARG
    assert _decode(lib, ci=MIS) == ALIGN
    assert _decode(lib, wsb=0) == WS
    assert _decode(lib, B=0, q=None) == OK


@pytest.mark.gpu
def test_python_binding_checks_dtypes():
    import torch
    import learned_centroid_gated_amd as F
    with pytest.raises(TypeError):
        F.focus_bucket(torch.zeros(8, 2, dtype=torch.int64, device="cuda"), 4)


def _paged(lib, q=P, qg=P, kp=P, vp=P, npages=64, page=16, table=P, pps=8, ln=P, cg=P, co=P,
           ci=P, B=4, Hq=8, Hkv=2, dh=128, K=16, top_k=2, window=64, scale=0.0, out=P, lse=P,
           ws=P, wsb=BIG):
    return lib.focus_decode_paged(q, qg, kp, vp, npages, page, table, pps, ln, cg, co, ci, B, Hq,
                                  Hkv, dh, K, top_k, window, scale, out, lse, ws, wsb, None)


def test_decode_paged_validation(lib):
    assert _paged(lib, B=-1) == ARG
    assert _paged(lib, npages=0) == ARG
    assert _paged(lib, page=0) == ARG
    assert _paged(lib, pps=0) == ARG
    assert _paged(lib, window=-1) == ARG
    assert _paged(lib, dh=32) == UNSUP
    assert _paged(lib, top_k=5, K=16) == UNSUP
    assert _paged(lib, npages=(1 << 27) + 1, page=16) == SHAPE  # pool rows past 2^31
    assert _paged(lib, pps=1 << 27, page=16) == SHAPE
    assert _paged(lib, pps=1 << 26, page=16, top_k=2) == SHAPE  # Lmax * top_k past 2^31
    for name in ("q", "qg", "kp", "vp", "table", "ln", "cg", "co", "ci", "out", "lse"):
        assert _paged(lib, **{name: None}) == ARG, name
    assert _paged(lib, kp=MIS) == ALIGN
    assert _paged(lib, table=P + 2) == ALIGN
    assert _paged(lib, ws=None) == WS
    assert _paged(lib, wsb=16) == WS
    assert _paged(lib, B=0, q=None) == OK


def test_slots_validation(lib):
    fb = lambda off=P, idx=P, B=4, L=1024, K=16, k=2, cap=64, sl=P, sp=P, ov=P: \
        lib.focus_slots_from_bucket(off, idx, B, L, K, k, cap, sl, sp, ov, None)
    assert fb(B=0) == ARG
    assert fb(L=0) == ARG
    assert fb(cap=0) == ARG
    assert fb(K=0) == ARG
    assert fb(k=9) == UNSUP
    assert fb(B=70000) == SHAPE
    assert fb(K=1024, cap=1 << 21) == SHAPE
    for name in ("off", "idx", "sl", "sp", "ov"):
        assert fb(**{name: None}) == ARG, name
    assert fb(sp=P + 2) == ALIGN
    ap = lambda ng=P, ln=P, B=4, K=16, k=2, cap=64, sl=P, sp=P, ov=P: \
        lib.focus_slots_append(ng, ln, B, K, k, cap, sl, sp, ov, None)
    assert ap(B=0) == ARG
    assert ap(cap=0) == ARG
    assert ap(K=1024, cap=1 << 21) == SHAPE
    for name in ("ng", "ln", "sl", "sp", "ov"):
        assert ap(**{name: None}) == ARG, name
    assert ap(ov=P + 1) == ALIGN


def _dslots(lib, q=P, qg=P, kp=P, vp=P, npages=64, page=16, table=P, pps=8, ln=P, cg=P, sl=P,
            sp=P, cap=64, B=4, Hq=8, Hkv=2, dh=128, K=16, top_k=2, window=64, scale=0.0, out=P,
            lse=P, ws=P, wsb=BIG):
    return lib.focus_decode_slots(q, qg, kp, vp, npages, page, table, pps, ln, cg, sl, sp, cap, B,
                                  Hq, Hkv, dh, K, top_k, window, scale, out, lse, ws, wsb, None)


def test_decode_slots_validation(lib):
    assert _dslots(lib, B=-1) == ARG
    assert _dslots(lib, cap=0) == ARG
    assert _dslots(lib, page=0) == ARG
    assert _dslots(lib, dh=32) == UNSUP
    assert _dslots(lib, K=1024, cap=1 << 21) == SHAPE
    assert _dslots(lib, npages=(1 << 27) + 1, page=16) == SHAPE
    for name in ("q", "qg", "kp", "vp", "table", "ln", "cg", "sl", "sp", "out", "lse"):
        assert _dslots(lib, **{name: None}) == ARG, name
    assert _dslots(lib, sp=P + 2) == ALIGN
    assert _dslots(lib, ws=None) == WS
    assert _dslots(lib, wsb=16) == WS
    assert _dslots(lib, B=0, q=None) == OK


def _noalloc(lib, q=P, qg=P, kc=P, vc=P, ln=P, cg=P, co=P, ci=P, B=4, L=1024, Hq=8, Hkv=2,
             dh=128, K=16, top_k=2, window=64, scale=0.0, out=P, lse=P):
    return lib.focus_decode_noalloc(q, qg, kc, vc, ln, cg, co, ci, B, L, Hq, Hkv, dh, K, top_k,
                                    window, scale, out, lse, None)


def test_decode_pieces_follow_the_batch(lib):
    """Decode cuts each sequence's key list into pieces so that the partial kernel gets at most
    512 blocks (two per compute unit), at most 256 pieces per sequence. With 32 query heads in
    8 kv groups of d_head 128 a block serves all heads of one sequence, so the partials
    (Hq * pieces * (4 d_head + 8) bytes per sequence) fill the same workspace for every batch
    whose pieces times sequences is 512, half of it for one sequence (256 pieces), and grow
    with the batch past 512 sequences (one piece each)."""
    ws = lambda B: lib.focus_decode_workspace_size(B, 65536, 32, 8, 128, 64, 2)
    per_piece = 32 * (4 * 128 + 8)
    for B in (2, 4, 8, 16, 64, 128, 256, 512):
        assert ws(B) == 512 * per_piece, B
    assert ws(1) == 256 * per_piece
    assert ws(100) == 100 * 5 * per_piece
    assert ws(1000) == 1000 * per_piece


def test_decode_noalloc_validation(lib):
    """The allocation-free decode refuses what focus_decode refuses, and every call whose
    scratch would exceed the fixed array, before touching the device."""
    cap = lib.focus_decode_noalloc_scratch_bytes()
    assert cap == 64 << 20
    assert _noalloc(lib, B=-1) == ARG
    assert _noalloc(lib, L=0) == ARG
    assert _noalloc(lib, dh=32) == UNSUP
    assert _noalloc(lib, top_k=5) == UNSUP
    assert _noalloc(lib, L=1 << 31, top_k=1) == SHAPE
    for name in ("q", "qg", "kc", "vc", "ln", "cg", "co", "ci", "out", "lse"):
        assert _noalloc(lib, **{name: None}) == ARG, name
    assert _noalloc(lib, ci=MIS) == ALIGN
    assert _noalloc(lib, B=0, q=None) == OK
    # the scratch holds the pieces' partials: the 64 x 65536 decode and 2048 sequences (one
    # piece each) fit, while the partials of 4096 sequences of 32 heads do not
    ws = lib.focus_decode_workspace_size
    assert ws(64, 65536, 32, 8, 128, 64, 2) <= ws(2048, 65536, 32, 8, 128, 64, 2) <= cap
    assert cap < ws(4096, 1024, 32, 8, 128, 64, 2)
    assert _noalloc(lib, B=4096, L=1024, Hq=32, Hkv=8, K=64) == -7


def _train_args(**over):
    a = dict(h=P, w=P, c=P, n=256, d=64, dg=16, K=8, iters=2, q=P, k=P, v=P, Hq=8, Hkv=2, dh=128,
             window=16, lam=4.0, scale=0.0)
    a.update(over)
    return a


def _train_fwd(lib, out=P, lse=P, ws=P, wsb=BIG, **over):
    a = _train_args(**over)
    return lib.focus_soft_train_forward(a["h"], a["w"], a["c"], a["n"], a["d"], a["dg"], a["K"],
                                        a["iters"], a["q"], a["k"], a["v"], a["Hq"], a["Hkv"],
                                        a["dh"], a["window"], a["lam"], a["scale"], out, lse, ws,
                                        wsb, None)


def _train_bwd(lib, out=P, lse=P, dout=P, dc=P, dw=P, dh_out=P, ws=P, wsb=BIG, **over):
    a = _train_args(**over)
    return lib.focus_soft_train_backward(a["h"], a["w"], a["c"], a["n"], a["d"], a["dg"], a["K"],
                                         a["iters"], a["q"], a["k"], a["v"], a["Hq"], a["Hkv"],
                                         a["dh"], a["window"], a["lam"], a["scale"], out, lse,
                                         dout, dc, dw, dh_out, ws, wsb, None)


@pytest.mark.parametrize("call", [_train_fwd, _train_bwd])
def test_soft_train_validation(lib, call):
    assert call(lib, n=-1) == ARG
    assert call(lib, window=-1) == ARG
    assert call(lib, iters=-1) == ARG
    assert call(lib, iters=65) == ARG
    assert call(lib, lam=math.nan) == ARG
    assert call(lib, lam=math.inf) == ARG
    assert call(lib, scale=math.nan) == ARG
    assert call(lib, K=0) == ARG
    assert call(lib, K=129) == UNSUP
    assert call(lib, d=66) == UNSUP
    assert call(lib, dg=18) == UNSUP
    assert call(lib, dg=2048) == ARG
    assert call(lib, Hq=6, Hkv=4) == ARG
    assert call(lib, Hq=6, Hkv=2) == UNSUP
    assert call(lib, dh=96) == UNSUP
    assert call(lib, n=1 << 26, Hq=64, Hkv=8) == SHAPE
    for name in ("h", "w", "c", "q", "k", "v"):
        assert call(lib, **{name: None}) == ARG, name
    assert call(lib, k=MIS) == ALIGN
    assert call(lib, ws=None) == WS
    assert call(lib, wsb=64) == WS
    assert call(lib, out=None) == ARG


def test_soft_train_backward_outputs(lib):
    assert _train_bwd(lib, dc=None) == ARG
    assert _train_bwd(lib, dw=None) == ARG
    assert _train_bwd(lib, dout=None) == ARG
    assert _train_bwd(lib, lse=None) == ARG
    assert _train_bwd(lib, dc=P + 2) == ALIGN
    assert _train_bwd(lib, dout=MIS) == ALIGN
    f = lib.focus_soft_train_workspace_size
    assert f(-1, 64, 16, 8, 8, 2) == 0
    # the scores, the soft assignment's planes and the backward's per-token buffers at least
    assert f(32768, 4096, 128, 64, 32, 3) >= 32768 * (64 * 4 * 3 + 64 * 2 * 2 + 32 * 4 + 128 * 8)
