"""A POET-X layer driven through libpoetx.so.

`POETXLayer` owns every device buffer of one layer shape (the folded weight,
the orthogonal blocks, saved activations, workspaces, gradients) and runs the
forward pass, the backward pass, or one whole training step of the layer
through the C ABI on the current HIP stream.  `POETXLinear` wraps it as a
torch.nn.Module whose packed parameters get gradients through autograd.
PyTorch supplies device memory and streams only.
"""
from __future__ import annotations

import torch

from . import poetx as P

_DT = {P.F32: torch.float32, P.BF16: torch.bfloat16}


def _bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


class POETXLayer:
    """Buffers and calls for one (m, n, b, k, T, dtype) layer."""

    def __init__(self, m: int, n: int, b: int, k: int, T: int, act: int, device="cuda",
                 xmem: bool = False, xq: bool = False, keep_w0ft: bool = False):
        """xmem: keep only U for the backward pass and recompute Z there
        (the memory-saving mode) instead of keeping U and Z.
        xq: the base weight is int8 with per-row scales (load_q); the dense
        products read the folded int8 weight directly and no bf16 copy of
        it is kept (W0f and W0fT are None).
        keep_w0ft: also keep the folded weight transposed (W0fT) for the
        backward's dense product; by default it reads W0f itself, so the
        fixed weight is held once (same results, bit for bit)."""
        self.m, self.n, self.b, self.k, self.T, self.act = m, n, b, k, T, act
        self.xmem, self.xq = xmem, xq
        if xq and act != P.BF16:
            raise ValueError("the int8 base weight is expanded to bf16: act must be BF16")
        self.sh = P.shape(m, n, b, k, T, act)
        dt = self.dtype = _DT[act]
        dev = self.device = torch.device(device)
        nP, nR = n // b, m // b
        self.nP, self.nR = nP, nR
        e = lambda *s, d=dt: torch.empty(*s, dtype=d, device=dev)
        self.W0f = None if xq else e(m, n)
        self.W0fT = e(n, m) if keep_w0ft and not xq else None
        if xq:
            self.qf, self.qfT = e(m, n, d=torch.int8), e(n, m, d=torch.int8)
            self.s_f = e(m, d=torch.float32)
        self.perm_P = e(n, d=torch.int32)
        self.perm_R = e(m, d=torch.int32)
        self.perm_P_inv = e(n, d=torch.int32)
        self.perm_R_inv = e(m, d=torch.int32)
        # Both sides share one block array (P blocks first, then R), so one
        # Cayley-Neumann call covers the nP + nR blocks of a step; the
        # per-side tensors are views.
        nb = nP + nR
        tb = b * (b - 1) // 2
        self.G, self.GT = e(nb, b, b), e(nb, b, b)
        self.G_P, self.G_R = self.G[:nP], self.G[nP:]
        self.GT_P, self.GT_R = self.GT[:nP], self.GT[nP:]
        self.y = e(T, m)
        self.dx = e(T, n)
        self.dG = e(nb, b, b, d=torch.float32)
        self.dG_P, self.dG_R = self.dG[:nP], self.dG[nP:]
        self.theta = torch.zeros(nb, tb, dtype=torch.float32, device=dev)
        self.theta_P, self.theta_R = self.theta[:nP], self.theta[nP:]
        self.dtheta = e(nb, tb, d=torch.float32)
        self.dtheta_P, self.dtheta_R = self.dtheta[:nP], self.dtheta[nP:]
        if xmem:
            self.saved = _bytes(P.poetx_saved_bytes_xmem(self.sh), dev)
            self.ws_fwd = _bytes(P.poetx_workspace_bytes(self.sh, 2), dev)
            self.ws_bwd = _bytes(P.poetx_workspace_bytes(self.sh, 3), dev)
        else:
            self.saved = _bytes(P.poetx_saved_bytes(self.sh), dev)
            self.ws_fwd = _bytes(P.poetx_workspace_bytes(self.sh, 0), dev)
            self.ws_bwd = _bytes(P.poetx_workspace_bytes(self.sh, 1), dev)
        # one CNP workspace for both calls (the backward's size covers the
        # forward's): the backward then reuses the Q the forward unpacked
        self.ws_cnp = _bytes(P.poetx_cnp_workspace_bytes(nb, b, k, 1, act), dev)
        self._q_ready = False

    # -- set-up, once per inner loop (untimed) --------------------------------
    def load(self, W0: torch.Tensor, theta_P: torch.Tensor, theta_R: torch.Tensor,
             perm_P: torch.Tensor, perm_R: torch.Tensor) -> None:
        self.perm_P.copy_(perm_P)
        self.perm_R.copy_(perm_R)
        W0 = W0.to(self.device, self.dtype).contiguous()
        P.poetx_fold_perm(W0, self.perm_R, self.perm_P, self.W0f, self.W0fT,
                          self.perm_R_inv, self.perm_P_inv)
        self.set_theta(theta_P, theta_R)

    def merge(self, out: torch.Tensor = None) -> torch.Tensor:
        """The weight R W0 P that the current theta and permutations
        represent (G from the latest cnp()), as an [m, n] tensor."""
        if self.xq:
            raise NotImplementedError("merging into an int8 base weight needs a new "
                                      "quantization; not provided")
        if out is None:
            out = torch.empty(self.m, self.n, dtype=self.dtype, device=self.device)
        ws = _bytes(P.poetx_workspace_bytes(self.sh, 4), self.device)
        P.poetx_merge(self.sh, self.W0f, self.G_R, self.GT_P, self.perm_R_inv, self.perm_P_inv,
                      out, ws)
        return out

    def load_q(self, q: torch.Tensor, s: torch.Tensor, theta_P: torch.Tensor,
               theta_R: torch.Tensor, perm_P: torch.Tensor, perm_R: torch.Tensor) -> None:
        """Set-up for an int8 base weight W0 = s[:, None] * q (xq layers)."""
        assert self.xq
        self.perm_P.copy_(perm_P)
        self.perm_R.copy_(perm_R)
        P.poetx_fold_perm(q.to(self.device, torch.int8).contiguous(), self.perm_R, self.perm_P,
                          self.qf, self.qfT, self.perm_R_inv, self.perm_P_inv)
        P.poetx_fold_scale(s.to(self.device, torch.float32).contiguous(), self.perm_R, self.s_f)
        self.set_theta(theta_P, theta_R)

    def set_theta(self, theta_P: torch.Tensor, theta_R: torch.Tensor) -> None:
        self.theta_P.copy_(theta_P)
        self.theta_R.copy_(theta_R)
        self._q_ready = False

    # -- the hot path ---------------------------------------------------------
    def cnp(self) -> None:
        """G, G^T of every block of both sides, in one call."""
        P.poetx_cnp_fwd(self.theta, self.b, self.k, self.G, self.GT, self.ws_cnp)
        self._q_ready = True

    def cnp_bwd(self) -> None:
        """dtheta of both sides from dG, in one call (reusing the forward's
        unpacked Q when theta has not changed since cnp())."""
        P.poetx_cnp_bwd(self.theta, self.dG, self.b, self.k, self.dtheta, self.act,
                        ws=self.ws_cnp, after_fwd=self._q_ready)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        self.cnp()
        self.layer_fwd(x)
        return self.y

    def layer_fwd(self, x: torch.Tensor) -> None:
        """The layer forward alone (G_P, G_R already formed)."""
        if self.xq:
            P.poetx_layer_fwd_q(self.sh, x, self.G_P, self.G_R, self.qf, self.s_f, self.perm_P,
                                self.perm_R_inv, self.y, self.saved, self.ws_fwd, self.xmem)
            return
        fwd = P.poetx_layer_fwd_xmem if self.xmem else P.poetx_layer_fwd
        fwd(self.sh, x, self.G_P, self.G_R, self.W0f, self.perm_P, self.perm_R_inv, self.y,
            self.saved, self.ws_fwd)

    def layer_bwd(self, dy: torch.Tensor) -> None:
        """The layer backward alone (dx, dG_P, dG_R)."""
        if self.xq:
            P.poetx_layer_bwd_q(self.sh, dy, self.G_P, self.GT_P, self.GT_R, self.qf, self.qfT,
                                self.s_f, self.perm_P_inv, self.perm_R, self.saved, self.dx,
                                self.dG_P, self.dG_R, self.ws_bwd, self.xmem)
        elif self.xmem:
            P.poetx_layer_bwd_xmem(self.sh, dy, self.G_P, self.GT_P, self.GT_R, self.W0f,
                                   self.W0fT, self.perm_P_inv, self.perm_R, self.saved, self.dx,
                                   self.dG_P, self.dG_R, self.ws_bwd)
        else:
            P.poetx_layer_bwd(self.sh, dy, self.GT_P, self.GT_R, self.W0f, self.W0fT,
                              self.perm_P_inv, self.perm_R, self.saved, self.dx, self.dG_P,
                              self.dG_R, self.ws_bwd)

    def backward(self, dy: torch.Tensor):
        self.layer_bwd(dy)
        self.cnp_bwd()
        return self.dx, self.dtheta_P, self.dtheta_R

    def step(self, x: torch.Tensor, dy: torch.Tensor):
        """One training step of the layer: every stage of the hot path."""
        self.forward(x)
        return self.backward(dy)


class _POETXFn(torch.autograd.Function):
    """One call of the layer.  Every forward call owns its G, G^T, saved
    activations, CNP workspace (which keeps the call's unpacked Q) and
    a snapshot of theta, all from torch's caching allocator, so forwards may
    run back to back before their backwards (micro-batch accumulation,
    weight tying) and each backward sees its own forward's state."""

    @staticmethod
    def forward(ctx, x, theta_P, theta_R, mod: "POETXLinear"):
        n, m, b, k, act = mod.n, mod.m, mod.b, mod.k, mod.act
        if x.shape[-1] != n:
            raise ValueError(f"x has {x.shape[-1]} features, the layer takes n={n}")
        if x.dtype != mod.dtype:
            raise ValueError(f"x has dtype {x.dtype}, the layer computes in {mod.dtype}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, n).contiguous()
        T = x2.shape[0]
        if T < 1:
            raise ValueError("x holds no tokens")
        dev, dt = x2.device, mod.dtype
        sh = P.shape(m, n, b, k, T, act)
        nP = n // b
        theta = torch.cat([theta_P.detach(), theta_R.detach()]).to(torch.float32).contiguous()
        nb = theta.shape[0]
        G = torch.empty(nb, b, b, dtype=dt, device=dev)
        GT = torch.empty_like(G)
        ws_cnp = _bytes(P.poetx_cnp_workspace_bytes(nb, b, k, 1, act), dev)
        P.poetx_cnp_fwd(theta, b, k, G, GT, ws_cnp)
        y = torch.empty(T, m, dtype=dt, device=dev)
        saved = _bytes(P.poetx_saved_bytes(sh), dev)
        ws = _bytes(P.poetx_workspace_bytes(sh, 0), dev)
        P.poetx_layer_fwd(sh, x2, G[:nP], G[nP:], mod.W0f, mod.perm_P, mod.perm_R_inv, y, saved,
                          ws)
        del ws, G
        ctx.mod, ctx.sh, ctx.lead = mod, sh, lead
        ctx.state = (theta, GT, saved, ws_cnp)
        return y.reshape(*lead, m)

    @staticmethod
    def backward(ctx, dy):
        mod, sh = ctx.mod, ctx.sh
        theta, GT, saved, ws_cnp = ctx.state
        ctx.state = None
        n, m, b, k, act, T = mod.n, mod.m, mod.b, mod.k, mod.act, sh.T
        dev = dy.device
        dy2 = dy.reshape(T, m).to(mod.dtype).contiguous()
        nP = n // b
        dx = torch.empty(T, n, dtype=mod.dtype, device=dev)
        dG = torch.empty(theta.shape[0], b, b, dtype=torch.float32, device=dev)
        ws = _bytes(P.poetx_workspace_bytes(sh, 1), dev)
        P.poetx_layer_bwd(sh, dy2, GT[:nP], GT[nP:], mod.W0f, None, mod.perm_P_inv, mod.perm_R,
                          saved, dx, dG[:nP], dG[nP:], ws)
        del ws
        dtheta = torch.empty_like(theta)
        # ws_cnp still holds this call's own unpacked Q
        P.poetx_cnp_bwd(theta, dG, b, k, dtheta, act, ws=ws_cnp, after_fwd=True)
        return dx.reshape(*ctx.lead, n), dtheta[:nP], dtheta[nP:], None


class POETXLinear(torch.nn.Module):
    """y = x (R W0 P)^T with a fixed random W0 and CNP-parameterized R, P.

    theta_P / theta_R start at 0 (R = P = I, the layer equals W0).
    `start_inner_loop()` draws new permutations and folds them into W0;
    `end_inner_loop()` merges the learned transforms into W0 first.
    x is [..., n] in the layer's dtype, any number of tokens per call; each
    call is independent of the others (see _POETXFn).
    """

    def __init__(self, n: int, m: int, b: int, k: int, dtype=torch.bfloat16, seed: int = 0,
                 device="cuda"):
        super().__init__()
        self.n, self.m, self.b, self.k = n, m, b, k
        self.act, self.dtype = P.act_of(dtype), dtype
        # shape checks of the library (T is free here, 1 stands in)
        if P.poetx_saved_bytes(P.shape(m, n, b, k, 1, self.act)) == 0:
            raise ValueError(f"unsupported layer m={m} n={n} b={b} k={k} {dtype}: "
                             + P.lib().poetx_last_error().decode())
        g = torch.Generator().manual_seed(seed)
        self.register_buffer("W0", (torch.randn(m, n, generator=g) / n ** 0.5).to(dtype).to(device))
        tb = b * (b - 1) // 2
        self.theta_P = torch.nn.Parameter(torch.zeros(n // b, tb, device=device))
        self.theta_R = torch.nn.Parameter(torch.zeros(m // b, tb, device=device))
        e = lambda *s, d=dtype: torch.empty(*s, dtype=d, device=device)
        self.W0f = e(m, n)
        self.perm_P, self.perm_R = e(n, d=torch.int32), e(m, d=torch.int32)
        self.perm_P_inv, self.perm_R_inv = e(n, d=torch.int32), e(m, d=torch.int32)
        self._gen = g
        self.start_inner_loop()

    def start_inner_loop(self) -> None:
        """Draw new permutations and fold them into the weight."""
        self.perm_P.copy_(torch.randperm(self.n, generator=self._gen).to(torch.int32))
        self.perm_R.copy_(torch.randperm(self.m, generator=self._gen).to(torch.int32))
        P.poetx_fold_perm(self.W0, self.perm_R, self.perm_P, self.W0f, None,
                          self.perm_R_inv, self.perm_P_inv)

    @torch.no_grad()
    def end_inner_loop(self) -> None:
        """Merge the learned transforms into the weight (W0 <- R W0 P), reset
        theta to 0 (R = P = I) and start a new inner loop with new
        permutations; the layer's function is unchanged by the merge."""
        n, m, b, k, act = self.n, self.m, self.b, self.k, self.act
        theta = torch.cat([self.theta_P, self.theta_R]).float().contiguous()
        nb, nP = theta.shape[0], n // b
        G = torch.empty(nb, b, b, dtype=self.dtype, device=theta.device)
        GT = torch.empty_like(G)
        P.poetx_cnp_fwd(theta, b, k, G, GT, _bytes(P.poetx_cnp_workspace_bytes(nb, b, k, 0, act),
                                                   theta.device))
        sh = P.shape(m, n, b, k, 1, act)
        W = torch.empty(m, n, dtype=self.dtype, device=theta.device)
        P.poetx_merge(sh, self.W0f, G[nP:], GT[:nP], self.perm_R_inv, self.perm_P_inv, W,
                      _bytes(P.poetx_workspace_bytes(sh, 4), theta.device))
        self.W0.copy_(W)
        self.theta_P.zero_()
        self.theta_R.zero_()
        self.start_inner_loop()

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return _POETXFn.apply(x, self.theta_P, self.theta_R, self)
