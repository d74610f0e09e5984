"""Python binding of libpoetx.so with the C ABI's names.

Argument marshalling only: every tensor must already live on the GPU,
contiguous, in the storage type the call expects; the functions check that on
the host (so no host pointer ever reaches a kernel), pass raw pointers and the
current HIP stream, and raise PoetxError on a non-OK status.  No arithmetic of
the layer happens here.  See include/poetx.h for the meaning of each argument.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from ._lib import BF16, F32, I8, PoetxError, Shape, check, lib  # noqa: F401

_DT = {F32: torch.float32, BF16: torch.bfloat16}


def act_of(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported activation dtype {dtype}")


def _stream(stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return C.c_void_p(t.data_ptr())


def _ws(ws: Optional[torch.Tensor], need: int, name="ws"):
    if need == 0 and ws is None:
        return None, 0
    if ws is None:
        raise ValueError(f"{name}: {need} bytes of workspace required")
    p = _dev(ws, name)
    return p, ws.numel() * ws.element_size()


def shape(m: int, n: int, b: int, k: int, T: int, act: int) -> Shape:
    return Shape(m, n, b, k, T, act)


def poetx_set_fused_gather(on: bool) -> bool:
    """Select the one-pass gather + block products for later layer calls
    (set it before sizing workspaces); returns the previous setting."""
    return bool(lib().poetx_set_fused_gather(1 if on else 0))


def poetx_cnp_workspace_bytes(nblk: int, b: int, k: int, which: int, act: int) -> int:
    return lib().poetx_cnp_workspace_bytes(nblk, b, k, which, act)


def poetx_workspace_bytes(sh: Shape, which: int) -> int:
    return lib().poetx_workspace_bytes(C.byref(sh), which)


def poetx_saved_bytes(sh: Shape) -> int:
    return lib().poetx_saved_bytes(C.byref(sh))


def poetx_saved_bytes_xmem(sh: Shape) -> int:
    return lib().poetx_saved_bytes_xmem(C.byref(sh))


def poetx_cnp_fwd(theta: torch.Tensor, b: int, k: int, G: torch.Tensor,
                  GT: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    nblk = theta.shape[0]
    act = act_of(G.dtype)
    tb = b * (b - 1) // 2
    need = poetx_cnp_workspace_bytes(nblk, b, k, 0, act)
    wp, wb = _ws(ws, need)
    check("poetx_cnp_fwd", lib().poetx_cnp_fwd(
        nblk, b, k, _dev(theta, "theta", torch.float32, nblk * tb), _dev(G, "G", None, nblk * b * b),
        _dev(GT, "GT", G.dtype, nblk * b * b, optional=True), act, wp, wb, _stream(stream)))


def poetx_cnp_fwd_noalloc(theta: torch.Tensor, b: int, k: int, G: torch.Tensor,
                          GT: Optional[torch.Tensor] = None, stream=None) -> None:
    """poetx_cnp_fwd without a workspace: the library's own per-GPU scratch
    array holds the unpacked Q (calls that overlap on one GPU race)."""
    nblk = theta.shape[0]
    act = act_of(G.dtype)
    tb = b * (b - 1) // 2
    check("poetx_cnp_fwd_noalloc", lib().poetx_cnp_fwd_noalloc(
        nblk, b, k, _dev(theta, "theta", torch.float32, nblk * tb), _dev(G, "G", None, nblk * b * b),
        _dev(GT, "GT", G.dtype, nblk * b * b, optional=True), act, _stream(stream)))


def poetx_cnp_bwd(theta: torch.Tensor, dG: torch.Tensor, b: int, k: int, dtheta: torch.Tensor,
                  prec: int, accumulate: bool = False, ws: Optional[torch.Tensor] = None,
                  stream=None, after_fwd: bool = False) -> None:
    """after_fwd: call poetx_cnp_bwd_after_fwd (ws last served poetx_cnp_fwd
    with this theta and still holds its unpacked Q)."""
    nblk = theta.shape[0]
    tb = b * (b - 1) // 2
    need = poetx_cnp_workspace_bytes(nblk, b, k, 1, prec)
    wp, wb = _ws(ws, need)
    name = "poetx_cnp_bwd_after_fwd" if after_fwd else "poetx_cnp_bwd"
    check(name, getattr(lib(), name)(
        nblk, b, k, _dev(theta, "theta", torch.float32, nblk * tb),
        _dev(dG, "dG", torch.float32, nblk * b * b), _dev(dtheta, "dtheta", torch.float32, nblk * tb),
        int(bool(accumulate)), prec, wp, wb, _stream(stream)))


def poetx_fold_perm(W0: torch.Tensor, perm_R: torch.Tensor, perm_P: torch.Tensor,
                    W0f: torch.Tensor, W0fT: Optional[torch.Tensor] = None,
                    perm_R_inv: Optional[torch.Tensor] = None,
                    perm_P_inv: Optional[torch.Tensor] = None, stream=None) -> None:
    m, n = W0.shape
    dt = I8 if W0.dtype == torch.int8 else act_of(W0.dtype)
    check("poetx_fold_perm", lib().poetx_fold_perm(
        m, n, dt, _dev(W0, "W0"), _dev(perm_R, "perm_R", torch.int32, m),
        _dev(perm_P, "perm_P", torch.int32, n), _dev(W0f, "W0f", W0.dtype, m * n),
        _dev(W0fT, "W0fT", W0.dtype, m * n, optional=True),
        _dev(perm_R_inv, "perm_R_inv", torch.int32, m, optional=True),
        _dev(perm_P_inv, "perm_P_inv", torch.int32, n, optional=True), _stream(stream)))


def poetx_layer_fwd(sh: Shape, x, G_P, G_R, W0f, perm_P, perm_R_inv, y, saved, ws,
                    stream=None) -> None:
    dt = _DT[sh.act]
    m, n, b, T = sh.m, sh.n, sh.b, sh.T
    need_ws, need_saved = poetx_workspace_bytes(sh, 0), poetx_saved_bytes(sh)
    wp, wb = _ws(ws, need_ws)
    if saved.numel() * saved.element_size() < need_saved:
        raise ValueError(f"saved: {need_saved} bytes required")
    check("poetx_layer_fwd", lib().poetx_layer_fwd(
        C.byref(sh), _dev(x, "x", dt, T * n), _dev(G_P, "G_P", dt, n * b),
        _dev(G_R, "G_R", dt, m * b), _dev(W0f, "W0f", dt, m * n),
        _dev(perm_P, "perm_P", torch.int32, n), _dev(perm_R_inv, "perm_R_inv", torch.int32, m),
        _dev(y, "y", dt, T * m), _dev(saved, "saved"), wp, wb, _stream(stream)))


def poetx_layer_bwd(sh: Shape, dy, GT_P, GT_R, W0f, W0fT, perm_P_inv, perm_R, saved, dx, dG_P,
                    dG_R, ws, stream=None) -> None:
    """W0fT may be None: the dense product then reads W0f K-major."""
    dt = _DT[sh.act]
    m, n, b, T = sh.m, sh.n, sh.b, sh.T
    need_ws, need_saved = poetx_workspace_bytes(sh, 1), poetx_saved_bytes(sh)
    wp, wb = _ws(ws, need_ws)
    if saved.numel() * saved.element_size() < need_saved:
        raise ValueError(f"saved: {need_saved} bytes required")
    check("poetx_layer_bwd", lib().poetx_layer_bwd(
        C.byref(sh), _dev(dy, "dy", dt, T * m), _dev(GT_P, "GT_P", dt, n * b),
        _dev(GT_R, "GT_R", dt, m * b), _dev(W0f, "W0f", dt, m * n),
        _dev(W0fT, "W0fT", dt, m * n, optional=True),
        _dev(perm_P_inv, "perm_P_inv", torch.int32, n), _dev(perm_R, "perm_R", torch.int32, m),
        _dev(saved, "saved"), _dev(dx, "dx", dt, T * n), _dev(dG_P, "dG_P", torch.float32, n * b),
        _dev(dG_R, "dG_R", torch.float32, m * b), wp, wb, _stream(stream)))


def poetx_layer_fwd_xmem(sh: Shape, x, G_P, G_R, W0f, perm_P, perm_R_inv, y, saved, ws,
                         stream=None) -> None:
    dt = _DT[sh.act]
    m, n, b, T = sh.m, sh.n, sh.b, sh.T
    need_ws, need_saved = poetx_workspace_bytes(sh, 2), poetx_saved_bytes_xmem(sh)
    wp, wb = _ws(ws, need_ws)
    if saved.numel() * saved.element_size() < need_saved:
        raise ValueError(f"saved: {need_saved} bytes required")
    check("poetx_layer_fwd_xmem", lib().poetx_layer_fwd_xmem(
        C.byref(sh), _dev(x, "x", dt, T * n), _dev(G_P, "G_P", dt, n * b),
        _dev(G_R, "G_R", dt, m * b), _dev(W0f, "W0f", dt, m * n),
        _dev(perm_P, "perm_P", torch.int32, n), _dev(perm_R_inv, "perm_R_inv", torch.int32, m),
        _dev(y, "y", dt, T * m), _dev(saved, "saved"), wp, wb, _stream(stream)))


def poetx_layer_bwd_xmem(sh: Shape, dy, G_P, GT_P, GT_R, W0f, W0fT, perm_P_inv, perm_R, saved,
                         dx, dG_P, dG_R, ws, stream=None) -> None:
    dt = _DT[sh.act]
    m, n, b, T = sh.m, sh.n, sh.b, sh.T
    need_ws, need_saved = poetx_workspace_bytes(sh, 3), poetx_saved_bytes_xmem(sh)
    wp, wb = _ws(ws, need_ws)
    if saved.numel() * saved.element_size() < need_saved:
        raise ValueError(f"saved: {need_saved} bytes required")
    check("poetx_layer_bwd_xmem", lib().poetx_layer_bwd_xmem(
        C.byref(sh), _dev(dy, "dy", dt, T * m), _dev(G_P, "G_P", dt, n * b),
        _dev(GT_P, "GT_P", dt, n * b), _dev(GT_R, "GT_R", dt, m * b),
        _dev(W0f, "W0f", dt, m * n), _dev(W0fT, "W0fT", dt, m * n, optional=True),
        _dev(perm_P_inv, "perm_P_inv", torch.int32, n), _dev(perm_R, "perm_R", torch.int32, m),
        _dev(saved, "saved"), _dev(dx, "dx", dt, T * n), _dev(dG_P, "dG_P", torch.float32, n * b),
        _dev(dG_R, "dG_R", torch.float32, m * b), wp, wb, _stream(stream)))


def poetx_layer_fwd_q(sh: Shape, x, G_P, G_R, q_f, s_f, perm_P, perm_R_inv, y, saved, ws,
                      xmem: bool = False, stream=None) -> None:
    """The forward pass on an int8 base weight W0f = diag(s_f) q_f."""
    dt = _DT[sh.act]
    m, n, b, T = sh.m, sh.n, sh.b, sh.T
    need_ws = poetx_workspace_bytes(sh, 2 if xmem else 0)
    need_saved = poetx_saved_bytes_xmem(sh) if xmem else poetx_saved_bytes(sh)
    wp, wb = _ws(ws, need_ws)
    if saved.numel() * saved.element_size() < need_saved:
        raise ValueError(f"saved: {need_saved} bytes required")
    check("poetx_layer_fwd_q", lib().poetx_layer_fwd_q(
        C.byref(sh), _dev(x, "x", dt, T * n), _dev(G_P, "G_P", dt, n * b),
        _dev(G_R, "G_R", dt, m * b), _dev(q_f, "q_f", torch.int8, m * n),
        _dev(s_f, "s_f", torch.float32, m), _dev(perm_P, "perm_P", torch.int32, n),
        _dev(perm_R_inv, "perm_R_inv", torch.int32, m), _dev(y, "y", dt, T * m),
        _dev(saved, "saved"), wp, wb, int(bool(xmem)), _stream(stream)))


def poetx_layer_bwd_q(sh: Shape, dy, G_P, GT_P, GT_R, q_f, q_fT, s_f, perm_P_inv, perm_R, saved,
                      dx, dG_P, dG_R, ws, xmem: bool = False, stream=None) -> None:
    """The backward pass on an int8 base weight (G_P and q_f are read only
    with xmem and may be None otherwise)."""
    dt = _DT[sh.act]
    m, n, b, T = sh.m, sh.n, sh.b, sh.T
    need_ws = poetx_workspace_bytes(sh, 3 if xmem else 1)
    need_saved = poetx_saved_bytes_xmem(sh) if xmem else poetx_saved_bytes(sh)
    wp, wb = _ws(ws, need_ws)
    if saved.numel() * saved.element_size() < need_saved:
        raise ValueError(f"saved: {need_saved} bytes required")
    check("poetx_layer_bwd_q", lib().poetx_layer_bwd_q(
        C.byref(sh), _dev(dy, "dy", dt, T * m), _dev(G_P, "G_P", dt, n * b, optional=not xmem),
        _dev(GT_P, "GT_P", dt, n * b), _dev(GT_R, "GT_R", dt, m * b),
        _dev(q_f, "q_f", torch.int8, m * n, optional=not xmem),
        _dev(q_fT, "q_fT", torch.int8, m * n), _dev(s_f, "s_f", torch.float32, m),
        _dev(perm_P_inv, "perm_P_inv", torch.int32, n), _dev(perm_R, "perm_R", torch.int32, m),
        _dev(saved, "saved"), _dev(dx, "dx", dt, T * n), _dev(dG_P, "dG_P", torch.float32, n * b),
        _dev(dG_R, "dG_R", torch.float32, m * b), wp, wb, int(bool(xmem)), _stream(stream)))


def poetx_merge(sh: Shape, W0f, G_R, GT_P, perm_R_inv, perm_P_inv, W0_out, ws,
                stream=None) -> None:
    """W0_out = R W0 P, the weight the current transforms represent."""
    dt = _DT[sh.act]
    m, n, b = sh.m, sh.n, sh.b
    wp, wb = _ws(ws, poetx_workspace_bytes(sh, 4))
    check("poetx_merge", lib().poetx_merge(
        C.byref(sh), _dev(W0f, "W0f", dt, m * n), _dev(G_R, "G_R", dt, m * b),
        _dev(GT_P, "GT_P", dt, n * b), _dev(perm_R_inv, "perm_R_inv", torch.int32, m),
        _dev(perm_P_inv, "perm_P_inv", torch.int32, n), _dev(W0_out, "W0_out", dt, m * n),
        wp, wb, _stream(stream)))


def poetx_fold_scale(s, perm_R, s_f, stream=None) -> None:
    """s_f[i] = s[perm_R[i]] (the per-row scales of an int8 base weight)."""
    m = perm_R.numel()
    check("poetx_fold_scale", lib().poetx_fold_scale(
        m, _dev(s, "s", torch.float32, m), _dev(perm_R, "perm_R", torch.int32, m),
        _dev(s_f, "s_f", torch.float32, m), _stream(stream)))


def poetx_dequant(q, scale, per_row: bool, out, stream=None) -> None:
    """out = bf16(scale * q) for int8 q [rows][cols], scale by row or column."""
    rows, cols = q.shape
    check("poetx_dequant", lib().poetx_dequant(
        rows, cols, _dev(q, "q", torch.int8, rows * cols),
        _dev(scale, "scale", torch.float32, rows if per_row else cols), int(bool(per_row)),
        _dev(out, "out", torch.bfloat16, rows * cols), _stream(stream)))
