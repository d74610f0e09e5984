"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before anything reaches a device.  CPU only: every
call here fails validation, so no kernel is launched."""
import ctypes as C
import os
import re

import pytest

from orthogonal_reparameterized_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "poetx.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libpoetx.so not built")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(poetx_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = _lib.lib()
    syms = declared_symbols()
    assert len(syms) >= 11
    for s in syms:
        assert hasattr(L, s), s
        assert s in _lib.SIGNATURES, s
    assert set(_lib.SIGNATURES) == set(syms)
    assert L.poetx_abi_version() == 2


def test_status_strings():
    L = _lib.lib()
    assert L.poetx_status_str(0) == b"POETX_OK"
    assert L.poetx_status_str(3) == b"POETX_ERR_WORKSPACE"
    assert L.poetx_status_str(99) == b"POETX_UNKNOWN_STATUS"


FAKE = C.c_void_p(0x10000)      # aligned, never dereferenced: every call fails first
MISALIGNED = C.c_void_p(0x10002)


def test_cnp_argument_errors():
    L = _lib.lib()
    ok_args = lambda **kw: dict(dict(nblk=4, b=32, k=4, theta=FAKE, G=FAKE, GT=None, dt=1,
                                     ws=None, wsb=0, s=None), **kw)
    call = lambda a: L.poetx_cnp_fwd(a["nblk"], a["b"], a["k"], a["theta"], a["G"], a["GT"],
                                     a["dt"], a["ws"], a["wsb"], a["s"])
    assert call(ok_args(b=7)) == 1
    assert call(ok_args(nblk=0)) == 1
    assert call(ok_args(k=-1)) == 1
    assert call(ok_args(k=9)) == 1
    assert call(ok_args(theta=None)) == 1
    assert b"theta" in L.poetx_last_error()
    assert call(ok_args(G=MISALIGNED)) == 1
    assert b"aligned" in L.poetx_last_error()
    assert call(ok_args(dt=0, b=128)) == 2          # float32 blocks above 64
    assert call(ok_args(dt=5)) == 1
    # bf16 b=256 needs a workspace
    need = L.poetx_cnp_workspace_bytes(4, 256, 4, 0, 1)
    assert need >= 4 * 256 * 256 * 2
    assert call(ok_args(b=256, ws=FAKE, wsb=need - 1)) == 3
    assert L.poetx_cnp_bwd(4, 256, 4, FAKE, FAKE, FAKE, 0, 1, FAKE,
                           L.poetx_cnp_workspace_bytes(4, 256, 4, 1, 1) - 1, None) == 3
    assert L.poetx_cnp_bwd(4, 32, 4, FAKE, None, FAKE, 0, 0, FAKE, 1 << 20, None) == 1
    # the backward after the forward checks its arguments the same way
    assert L.poetx_cnp_bwd_after_fwd(4, 256, 4, FAKE, FAKE, FAKE, 0, 1, FAKE,
                                     L.poetx_cnp_workspace_bytes(4, 256, 4, 1, 1) - 1, None) == 3
    assert b"poetx_cnp_bwd_after_fwd" in L.poetx_last_error()
    assert L.poetx_cnp_bwd_after_fwd(4, 256, 4, FAKE, None, FAKE, 0, 1, FAKE, 1 << 30, None) == 1
    assert L.poetx_cnp_bwd_after_fwd(4, 7, 4, FAKE, FAKE, FAKE, 0, 1, FAKE, 1 << 30, None) == 1
    assert L.poetx_cnp_workspace_bytes(4, 7, 4, 0, 1) == 0


def test_layer_argument_errors():
    L = _lib.lib()
    good = _lib.Shape(4096, 4096, 256, 4, 8192, 1)
    assert L.poetx_workspace_bytes(C.byref(good), 0) > 0
    assert L.poetx_workspace_bytes(C.byref(good), 1) > 0
    assert L.poetx_saved_bytes(C.byref(good)) >= 8192 * (4096 + 4096) * 2
    bad = [
        _lib.Shape(4000, 4096, 256, 4, 8192, 1),   # m % b
        _lib.Shape(4096, 4096, 100, 4, 8192, 1),   # b
        _lib.Shape(4096, 4096, 256, 4, 0, 1),      # T
        _lib.Shape(4096, 4096, 256, -1, 8192, 1),  # k
        _lib.Shape(4096, 4096, 256, 4, 8192, 3),   # dtype
    ]
    for sh in bad:
        assert L.poetx_workspace_bytes(C.byref(sh), 0) == 0
        assert L.poetx_saved_bytes(C.byref(sh)) == 0
        st = L.poetx_layer_fwd(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, 1 << 40, None)
        assert st == 1, L.poetx_last_error()
    f32big = _lib.Shape(4096, 4096, 256, 4, 64, 0)
    assert L.poetx_layer_fwd(C.byref(f32big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, 1 << 40, None) == 2
    # workspace too small
    need = L.poetx_workspace_bytes(C.byref(good), 0)
    assert L.poetx_layer_fwd(C.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, need - 1, None) == 3
    need = L.poetx_workspace_bytes(C.byref(good), 1)
    bwd = lambda W0f=FAKE, W0fT=FAKE, GT_R=FAKE, ws=need: L.poetx_layer_bwd(
        C.byref(good), FAKE, FAKE, GT_R, W0f, W0fT, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
        None)
    assert bwd(ws=need - 1) == 3
    # null pointers are named
    assert bwd(GT_R=None) == 1
    assert b"GT_R" in L.poetx_last_error()
    # the backward takes the forward's W0f; its transpose is optional (the
    # dense product then reads W0f K-major): W0f alone passes every check
    # and stops only at the workspace
    assert bwd(W0fT=None, ws=need - 1) == 3
    assert bwd(W0f=None) == 1
    assert b"W0f" in L.poetx_last_error()
    assert bwd(W0fT=MISALIGNED) == 1
    assert L.poetx_fold_perm(0, 4, 1, FAKE, FAKE, FAKE, FAKE, None, None, None, None) == 1
    assert L.poetx_fold_perm(4, 4, 1, FAKE, None, FAKE, FAKE, None, None, None, None) == 1


def test_xmem_argument_errors_and_sizes():
    L = _lib.lib()
    good = _lib.Shape(4096, 4096, 256, 4, 8192, 1)
    fast, mem = L.poetx_saved_bytes(C.byref(good)), L.poetx_saved_bytes_xmem(C.byref(good))
    assert mem > 0 and fast - mem >= 8192 * 4096 * 2   # Z is not kept
    for which in (2, 3):
        assert L.poetx_workspace_bytes(C.byref(good), which) > \
            L.poetx_workspace_bytes(C.byref(good), which - 2)
    assert L.poetx_workspace_bytes(C.byref(good), 5) == 0
    need = L.poetx_workspace_bytes(C.byref(good), 2)
    assert L.poetx_layer_fwd_xmem(C.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, need - 1, None) == 3
    need = L.poetx_workspace_bytes(C.byref(good), 3)
    # the recompute needs G_P and W0f
    assert L.poetx_layer_bwd_xmem(C.byref(good), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 1
    assert b"G_P" in L.poetx_last_error()
    assert L.poetx_layer_bwd_xmem(C.byref(good), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 1
    assert b"W0f" in L.poetx_last_error()
    assert L.poetx_layer_bwd_xmem(C.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == 3


def test_fused_gather_switch_sizes_the_workspace():
    """poetx_set_fused_gather returns the previous setting; the one-pass
    form needs room for G in fragment order (W b bf16 per side) where it
    applies (bf16, b = 256, gathered width a multiple of 512 up to 4096)."""
    L = _lib.lib()
    square = _lib.Shape(4096, 4096, 256, 4, 8192, 1)
    mid = _lib.Shape(2048, 2048, 128, 4, 4096, 1)
    up = _lib.Shape(14336, 4096, 256, 4, 16384, 1)
    prev = L.poetx_set_fused_gather(0)
    try:
        sizes = {}
        for on in (0, 1):
            assert L.poetx_set_fused_gather(on) == 0   # was off (set above, then on = 0)
            sizes[on] = {nm: [L.poetx_workspace_bytes(C.byref(sh), w) for w in range(4)]
                         for nm, sh in (("square", square), ("mid", mid), ("up", up))}
        assert L.poetx_set_fused_gather(0) == 1
        g = 4096 * 256 * 2
        assert [b - a for a, b in zip(sizes[0]["square"], sizes[1]["square"])] == [g] * 4
        assert sizes[0]["mid"] == sizes[1]["mid"]          # b = 128: never one pass
        # mlp_up: the forward side (n = 4096) only; m = 14336 is too wide, so
        # the backward grows only in the memory-saving mode (recompute of V)
        d = [b - a for a, b in zip(sizes[0]["up"], sizes[1]["up"])]
        assert d == [g, 0, g, g]
    finally:
        L.poetx_set_fused_gather(prev)


def test_binding_rejects_host_tensors():
    import torch
    from orthogonal_reparameterized_02_amd import poetx as P
    th = torch.zeros(2, 32 * 31 // 2)
    G = torch.zeros(2, 32, 32)
    with pytest.raises(ValueError, match="GPU tensor"):
        P.poetx_cnp_fwd(th, 32, 4, G)


def test_merge_argument_errors():
    L = _lib.lib()
    good = _lib.Shape(4096, 4096, 256, 4, 8192, 1)
    need = L.poetx_workspace_bytes(C.byref(good), 4)
    assert need >= 2 * 4096 * 4096 * 2
    OUT = C.c_void_p(0x20000)
    assert L.poetx_merge(C.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, OUT, FAKE, need - 1,
                         None) == 3
    assert L.poetx_merge(C.byref(good), FAKE, None, FAKE, FAKE, FAKE, OUT, FAKE, need,
                         None) == 1
    assert b"G_R" in L.poetx_last_error()
    # the output may not alias the folded weight
    assert L.poetx_merge(C.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                         None) == 1
    assert b"alias" in L.poetx_last_error()


def test_xq_argument_errors():
    L = _lib.lib()
    assert L.poetx_dequant(64, 24, FAKE, FAKE, 1, FAKE, None) == 1      # cols % 16
    assert L.poetx_dequant(64, 32, MISALIGNED, FAKE, 1, FAKE, None) == 1
    assert L.poetx_dequant(64, 32, FAKE, None, 1, FAKE, None) == 1
    assert L.poetx_fold_scale(0, FAKE, FAKE, FAKE, None) == 1
    assert L.poetx_fold_scale(16, FAKE, None, FAKE, None) == 1
    assert L.poetx_fold_perm(4, 4, 3, FAKE, FAKE, FAKE, FAKE, None, None, None, None) == 1


def test_int8_layer_argument_errors():
    L = _lib.lib()
    good = _lib.Shape(4096, 4096, 256, 4, 8192, 1)
    need_f = L.poetx_workspace_bytes(C.byref(good), 0)
    need_b = L.poetx_workspace_bytes(C.byref(good), 1)
    fwd = lambda sh, qf=FAKE, sf=FAKE, ws=need_f, xmem=0: L.poetx_layer_fwd_q(
        C.byref(sh), FAKE, FAKE, FAKE, qf, sf, FAKE, FAKE, FAKE, FAKE, FAKE, ws, xmem, None)
    bwd = lambda sh, gp=None, qf=None, qft=FAKE, sf=FAKE, ws=need_b, xmem=0: L.poetx_layer_bwd_q(
        C.byref(sh), FAKE, gp, FAKE, FAKE, qf, qft, sf, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        ws, xmem, None)
    # the int8 weight runs on bf16 MFMA kernels with whole 256-column tiles
    assert fwd(_lib.Shape(4096, 4096, 32, 4, 64, 0)) == 2
    assert b"bf16" in L.poetx_last_error()
    assert fwd(_lib.Shape(4096, 4224, 128, 4, 64, 1)) == 2
    assert fwd(_lib.Shape(4096, 4096, 32, 4, 64, 1)) == 2
    assert fwd(good, sf=None) == 1
    assert fwd(good, qf=None) == 1
    assert b"q_f" in L.poetx_last_error()
    assert fwd(good, ws=need_f - 1) == 3
    assert fwd(good, ws=L.poetx_workspace_bytes(C.byref(good), 2) - 1, xmem=1) == 3
    assert bwd(_lib.Shape(4096, 4096, 32, 4, 64, 0)) == 2
    assert bwd(good, qft=None) == 1
    assert b"q_fT" in L.poetx_last_error()
    assert bwd(good, sf=None) == 1
    assert bwd(good, ws=need_b - 1) == 3
    # the memory-saving mode recomputes Z: it needs G_P and q_f
    need_bx = L.poetx_workspace_bytes(C.byref(good), 3)
    assert bwd(good, ws=need_bx, xmem=1) == 1
    assert b"G_P" in L.poetx_last_error()
    assert bwd(good, gp=FAKE, ws=need_bx, xmem=1) == 1
    assert b"q_f" in L.poetx_last_error()
