"""Float64 CPU oracle for the POET-X reparameterized linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  It shares no code with the HIP
library: plain NumPy in float64, written to be checked by eye against the
pages, with no blocking, fusion or reordering beyond what the definitions
state.

Sources (pages, by title):
  [POET]    "Reparameterized LLM Training via Orthogonal Equivalence
            Transformation" (chatpaper.ai), Abstract: each weight is
            W = R W0 P with two learnable orthogonal matrices R, P and a fixed
            random W0; orthogonal R, P keep the singular values of W0.
  [X-zh]    "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
            Transformation" (gist.science, Chinese), technical summary
            sections 2.1-2.5.
  [X-it]    the same title (gist.science, Italian), "Sommario tecnico" section 2.

Conventions (readings where the pages are silent; each listed in the design
notes):
  * Q = U - U^T where U is strictly upper triangular holding the packed
    parameters row by row over i < j (numpy.triu_indices(b, 1) order);
    b(b-1)/2 parameters per block ([X-zh] 2.4, [X-it] 2).
  * Cayley-Neumann parameterization: the pages name it without printing it.
    Reading: the Cayley transform (I+Q)(I-Q)^{-1} with the inverse replaced by
    its Neumann series cut after Q^k:  G = (I+Q)(I + Q + ... + Q^k).
  * Permutation matrix of an index map pi: Pi[i, pi[i]] = 1, so (Pi v)_i =
    v[pi[i]].  R = Pi_R^T BD(G_R) Pi_R and P = Pi_P^T BD(G_P) Pi_P, where BD is
    block diagonal with block j acting on coordinates [j b, (j+1) b)
    ([X-zh] 2.2 and 2.3: random permutations inside the orthogonal matrices,
    block-diagonal structure).
  * Layout: x [T, n] token-major, W0 [m, n] stored [out, in], y = x W^T [T, m].
  * The two permutations next to W0 fold into W0f = Pi_R W0 Pi_P^T, i.e.
    W0f[i, j] = W0[pi_R[i], pi_P[j]] ([X-zh] 2.2 "permutation reduction").

Parity: every function here is pinned by the CPU tests (closed forms, special
cases, brute force, finite differences); see tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

CHUNK = 2048  # tokens per chunk for the large GEMMs (memory only)


# --------------------------------------------------------------------------
# packed skew-symmetric parameters  ([X-zh] 2.4 storage; [X-it] 2 CNP bullet)
# --------------------------------------------------------------------------
def tri_count(b: int) -> int:
    """Parameters per block: the strict upper triangle, b(b-1)/2."""
    return b * (b - 1) // 2


def skew_from_packed(theta: np.ndarray, b: int) -> np.ndarray:
    """Q with Q[i, j] = theta[t(i, j)], Q[j, i] = -theta[t(i, j)] for i < j."""
    theta = np.asarray(theta, dtype=np.float64)
    assert theta.shape == (tri_count(b),)
    U = np.zeros((b, b))
    U[np.triu_indices(b, 1)] = theta
    return U - U.T


def pack_upper(M: np.ndarray) -> np.ndarray:
    """The strict upper triangle of M, row by row."""
    b = M.shape[0]
    return np.asarray(M, dtype=np.float64)[np.triu_indices(b, 1)].copy()


# --------------------------------------------------------------------------
# Cayley-Neumann parameterization ([X-zh] 2.4; [X-it] 2)
# --------------------------------------------------------------------------
def cnp_block(Q: np.ndarray, k: int) -> np.ndarray:
    """G = (I + Q) S with S = I + Q + ... + Q^k, by repeated multiplication."""
    b = Q.shape[0]
    I = np.eye(b)
    S = I.copy()
    Pp = I.copy()
    for _ in range(k):
        Pp = Pp @ Q
        S = S + Pp
    return (I + Q) @ S


def cnp_fwd(theta: np.ndarray, b: int, k: int) -> np.ndarray:
    """theta [N, b(b-1)/2] -> G [N, b, b] (float64)."""
    theta = np.asarray(theta, dtype=np.float64)
    return np.stack([cnp_block(skew_from_packed(t, b), k) for t in theta])


def cnp_bwd_block(Q: np.ndarray, k: int, dG: np.ndarray) -> np.ndarray:
    """Gradient of <dG, G(Q)> with respect to the packed parameters.

    With G = (I+Q) S and S = sum_{p<=k} Q^p, a perturbation dQ gives
      delta G = dQ S + (I+Q) sum_{p=1..k} sum_{a=0..p-1} Q^a dQ Q^{p-1-a},
    so the gradient with respect to the full matrix Q is
      gQ = dG S^T + sum_{p=1..k} sum_{a=0..p-1} (Q^T)^a M (Q^T)^{p-1-a},
      M  = (I+Q)^T dG.
    Q = U - U^T with U holding the parameters, so d/dtheta = triu1(gQ - gQ^T).
    """
    b = Q.shape[0]
    I = np.eye(b)
    powers_T = [I]                       # (Q^T)^a, a = 0..k-1
    for _ in range(max(k - 1, 0)):
        powers_T.append(powers_T[-1] @ Q.T)
    S = I.copy()
    Pp = I.copy()
    for _ in range(k):
        Pp = Pp @ Q
        S = S + Pp
    M = (I + Q).T @ dG
    gQ = dG @ S.T
    for p in range(1, k + 1):
        for a in range(p):
            gQ = gQ + powers_T[a] @ M @ powers_T[p - 1 - a]
    return pack_upper(gQ - gQ.T)


def cnp_bwd(theta: np.ndarray, dG: np.ndarray, b: int, k: int) -> np.ndarray:
    """theta [N, t_b], dG [N, b, b] -> dtheta [N, t_b] (float64)."""
    theta = np.asarray(theta, dtype=np.float64)
    return np.stack([cnp_bwd_block(skew_from_packed(t, b), k, np.asarray(g, np.float64))
                     for t, g in zip(theta, dG)])


def cayley_exact(Q: np.ndarray) -> np.ndarray:
    """Exact Cayley transform C = (I - Q)^{-1} (I + Q), by a LAPACK solve."""
    b = Q.shape[0]
    I = np.eye(b)
    return np.linalg.solve(I - Q, I + Q)


# --------------------------------------------------------------------------
# permutations as index maps ([X-zh] 2.2; [X-it] 2 "Ottimizzazione delle
# Permutazioni")
# --------------------------------------------------------------------------
def inverse_perm(pi: np.ndarray) -> np.ndarray:
    """inv[pi[i]] = i."""
    pi = np.asarray(pi)
    inv = np.empty_like(pi)
    for i, p in enumerate(pi.tolist()):
        inv[p] = i
    return inv


def is_permutation(pi: np.ndarray, n: int) -> bool:
    pi = np.asarray(pi)
    return pi.shape == (n,) and np.array_equal(np.sort(pi), np.arange(n))


def fold_perm(W0: np.ndarray, perm_R: np.ndarray, perm_P: np.ndarray):
    """W0f[i, j] = W0[pi_R[i], pi_P[j]] (= Pi_R W0 Pi_P^T), plus the inverse
    maps.  Pure data movement, so it is exact in any storage type."""
    W0f = np.asarray(W0)[np.asarray(perm_R)][:, np.asarray(perm_P)]
    return W0f, inverse_perm(perm_R), inverse_perm(perm_P)


# --------------------------------------------------------------------------
# the orthogonal factors, applied through index maps
# --------------------------------------------------------------------------
def apply_R_left(G_R: np.ndarray, perm_R: np.ndarray, X: np.ndarray) -> np.ndarray:
    """R X with R = Pi_R^T BD(G_R) Pi_R, for X with m rows."""
    b = G_R.shape[1]
    Y = X[perm_R]                               # Pi_R X
    Z = np.empty_like(Y)
    for i, G in enumerate(G_R):                 # BD(G_R) (Pi_R X)
        Z[i * b:(i + 1) * b] = G @ Y[i * b:(i + 1) * b]
    out = np.empty_like(Z)
    out[perm_R] = Z                             # Pi_R^T (...)
    return out


def apply_P_right(X: np.ndarray, G_P: np.ndarray, perm_P: np.ndarray) -> np.ndarray:
    """X P with P = Pi_P^T BD(G_P) Pi_P, for X with n columns."""
    b = G_P.shape[1]
    Y = X[:, perm_P]                            # X Pi_P^T
    Z = np.empty_like(Y)
    for j, G in enumerate(G_P):                 # (X Pi_P^T) BD(G_P)
        Z[:, j * b:(j + 1) * b] = Y[:, j * b:(j + 1) * b] @ G
    out = np.empty_like(Z)
    out[:, perm_P] = Z                          # (...) Pi_P
    return out


def weight(W0, G_R, G_P, perm_R, perm_P) -> np.ndarray:
    """W = R W0 P ([POET] Abstract)."""
    W0 = np.asarray(W0, dtype=np.float64)
    return apply_P_right(apply_R_left(G_R, perm_R, W0), G_P, perm_P)


# --------------------------------------------------------------------------
# the layer: plain definition y = x W^T and its gradients
# --------------------------------------------------------------------------
def layer_fwd(x, W0, theta_P, theta_R, perm_P, perm_R, b, k):
    """y = x (R W0 P)^T in float64.  Returns y and the weight W."""
    G_P = cnp_fwd(theta_P, b, k)
    G_R = cnp_fwd(theta_R, b, k)
    W = weight(W0, G_R, G_P, perm_R, perm_P)
    x = np.asarray(x, dtype=np.float64)
    y = np.empty((x.shape[0], W.shape[0]))
    for s in range(0, x.shape[0], CHUNK):
        y[s:s + CHUNK] = x[s:s + CHUNK] @ W.T
    return y, W


def layer_bwd(x, dy, W0, theta_P, theta_R, perm_P, perm_R, b, k):
    """Gradients of L with dL/dy = dy, for y = x W^T, W = R W0 P.

    dx = dy W;  dW = dy^T x;  dR = dW (W0 P)^T;  dP = (R W0)^T dW.
    R = Pi_R^T BD(G_R) Pi_R gives dBD_R = Pi_R dR Pi_R^T, whose diagonal
    blocks are dG_R (likewise for P).  Only those blocks are formed:
      dG_R[i] = dW[pi_R[I]] (W0 P)[pi_R[I]]^T,   I = [i b, (i+1) b)
      dG_P[j] = (R W0)[:, pi_P[J]]^T dW[:, pi_P[J]].
    W0 is fixed and gets no gradient ([POET] Abstract).
    Returns dict with dx, dtheta_P, dtheta_R, dG_P, dG_R.
    """
    G_P = cnp_fwd(theta_P, b, k)
    G_R = cnp_fwd(theta_R, b, k)
    W0 = np.asarray(W0, dtype=np.float64)
    RW0 = apply_R_left(G_R, perm_R, W0)
    W0P = apply_P_right(W0, G_P, perm_P)
    W = apply_P_right(RW0, G_P, perm_P)
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    m, n = W.shape
    dx = np.empty((x.shape[0], n))
    dW = np.zeros((m, n))
    for s in range(0, x.shape[0], CHUNK):
        dx[s:s + CHUNK] = dy[s:s + CHUNK] @ W
        dW += dy[s:s + CHUNK].T @ x[s:s + CHUNK]
    dG_R = np.stack([dW[perm_R[i * b:(i + 1) * b]] @ W0P[perm_R[i * b:(i + 1) * b]].T
                     for i in range(m // b)])
    dG_P = np.stack([RW0[:, perm_P[j * b:(j + 1) * b]].T @ dW[:, perm_P[j * b:(j + 1) * b]]
                     for j in range(n // b)])
    return {
        "dx": dx,
        "dG_P": dG_P,
        "dG_R": dG_R,
        "dtheta_P": cnp_bwd(theta_P, dG_P, b, k),
        "dtheta_R": cnp_bwd(theta_R, dG_R, b, k),
    }


# --------------------------------------------------------------------------
# bilinear probes of dG, for token counts where dG itself is too costly
# --------------------------------------------------------------------------
def dG_probes(x, dy, W0, G_P, G_R, perm_P, perm_R, u_P, v_P, u_R, v_R):
    """u^T dG v for every block and probe pair, without forming dG.

    With U = x[:, pi_P], V_j = U_j G_Pj^T, Z = V W0f^T, dS = dy[:, pi_R],
    dZ_i = dS_i G_Ri, dV = dZ W0f (the input-centric form, [X-zh] 2.1-2.3):
      dG_Ri = sum_t dS_i[t]^T Z_i[t]   ->  u^T dG_Ri v = sum_t (dS_i[t].u)(Z_i[t].v)
      dG_Pj = sum_t dV_j[t]^T U_j[t]   ->  u^T dG_Pj v = sum_t (dV_j[t].u)(U_j[t].v)
    Each per-token dot product is linear in x[t] or dy[t], so it is x[t] or
    dy[t] against one fixed vector, found by pulling the probe back through
    the layer's maps:
      Z_i[t].v  = V[t].(W0f_i^T v)  = sum_j U_j[t].(G_Pj^T w_j) = x[t].rx
      dS_i[t].u = dy[t].ry          (u placed at columns pi_R[i b + c])
      U_j[t].v  = x[t].rx'          (v placed at columns pi_P[j b + c])
      dV_j[t].u = dZ[t].(W0f_{:,j} u) = sum_i dS_i[t].(G_Ri s_i) = dy[t].ry'
    so every probe of every block is one column of x @ Rx times one column
    of dy @ Ry, summed over tokens.  u_P, v_P: [probes, N_P, b];
    u_R, v_R: [probes, N_R, b].  Returns (probes_P [probes, N_P],
    probes_R [probes, N_R]) in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    perm_P = np.asarray(perm_P)
    perm_R = np.asarray(perm_R)
    W0f, _, _ = fold_perm(np.asarray(W0, dtype=np.float64), perm_R, perm_P)
    m, n = W0f.shape
    b = G_P.shape[1]
    npr, nP, nR = u_P.shape[0], n // b, m // b
    Rx = np.zeros((n, npr * (nR + nP)))   # columns: R-side Z.v, then P-side U.v
    Ry = np.zeros((m, npr * (nR + nP)))   # columns: R-side dS.u, then P-side dV.u
    col = 0
    for q in range(npr):
        for i in range(nR):
            I = slice(i * b, (i + 1) * b)
            w = W0f[I].T @ v_R[q, i]                       # n, in U coordinates
            r = np.concatenate([G_P[j].T @ w[j * b:(j + 1) * b] for j in range(nP)])
            Rx[perm_P, col] = r                            # U[t].r = x[t].Rx[:, col]
            Ry[perm_R[I], col] = u_R[q, i]                 # dS_i[t].u = dy[t].Ry[:, col]
            col += 1
    for q in range(npr):
        for j in range(nP):
            J = slice(j * b, (j + 1) * b)
            Rx[perm_P[J], col] = v_P[q, j]                 # U_j[t].v
            s_ = W0f[:, J] @ u_P[q, j]                     # m, in dZ coordinates
            r = np.concatenate([G_R[i] @ s_[i * b:(i + 1) * b] for i in range(nR)])
            Ry[perm_R, col] = r                            # dS[t].r = dy[t].Ry[:, col]
            col += 1
    acc = np.zeros(col)
    for s0 in range(0, x.shape[0], CHUNK):
        acc += np.sum((x[s0:s0 + CHUNK] @ Rx) * (dy[s0:s0 + CHUNK] @ Ry), axis=0)
    probes_R = acc[:npr * nR].reshape(npr, nR)
    probes_P = acc[npr * nR:].reshape(npr, nP)
    return probes_P, probes_R


# --------------------------------------------------------------------------
# second formulation: input-centric with two permutations folded into W0
# ([X-zh] 2.1 "input-centric", 2.2 "4 -> 2 permutations", 2.3 batched blocks)
# --------------------------------------------------------------------------
def layer_fwd_input_centric(x, W0f, G_P, G_R, perm_P, perm_R):
    """U = x[:, pi_P]; V_j = U_j G_Pj^T; Z = V W0f^T; S_i = Z_i G_Ri^T;
    y[:, pi_R] = S.  Same result as layer_fwd up to rounding."""
    b = G_P.shape[1]
    x = np.asarray(x, dtype=np.float64)
    U = x[:, perm_P]
    V = np.empty_like(U)
    for j, G in enumerate(G_P):
        V[:, j * b:(j + 1) * b] = U[:, j * b:(j + 1) * b] @ G.T
    Z = V @ np.asarray(W0f, dtype=np.float64).T
    S = np.empty_like(Z)
    for i, G in enumerate(G_R):
        S[:, i * b:(i + 1) * b] = Z[:, i * b:(i + 1) * b] @ G.T
    y = np.empty_like(S)
    y[:, perm_R] = S
    return y


# --------------------------------------------------------------------------
# explicit dense matrices (tiny sizes only), as original POET built them
# --------------------------------------------------------------------------
def perm_matrix(pi: np.ndarray) -> np.ndarray:
    n = len(pi)
    M = np.zeros((n, n))
    M[np.arange(n), np.asarray(pi)] = 1.0
    return M


def block_diag_dense(G: np.ndarray) -> np.ndarray:
    nblk, b, _ = G.shape
    M = np.zeros((nblk * b, nblk * b))
    for j in range(nblk):
        M[j * b:(j + 1) * b, j * b:(j + 1) * b] = G[j]
    return M


def orthogonal_dense(G: np.ndarray, pi: np.ndarray) -> np.ndarray:
    """Pi^T BD(G) Pi as a dense matrix."""
    Pm = perm_matrix(pi)
    return Pm.T @ block_diag_dense(G) @ Pm


def weight_dense(W0, G_R, G_P, perm_R, perm_P) -> np.ndarray:
    return orthogonal_dense(G_R, perm_R) @ np.asarray(W0, np.float64) @ orthogonal_dense(G_P, perm_P)


# --------------------------------------------------------------------------
# comparison metric used by the parity tests
# --------------------------------------------------------------------------
def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F in float64 (the plain difference when ref
    is all zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.sqrt(np.sum(ref * ref))
    num = np.sqrt(np.sum((got - ref) * (got - ref)))
    return float(num / (den if den > 0 else 1.0))


def max_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over all elements, in float64 (the plain
    largest difference when ref is all zero).  One wrong element among many
    shows here at full size, where a norm over the whole tensor dilutes it."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def rel_fro_slices(got: np.ndarray, ref: np.ndarray, axis: int = 0) -> np.ndarray:
    """rel_fro of every slice along `axis`: entry i compares
    got.take(i, axis) with ref.take(i, axis).  axis 0 of a [N, ...] block
    tensor gives one figure per orthogonal block (each block is an
    independent matrix, [X-zh] 2.3); axis 0 / 1 of a token-major [T, w]
    activation gives one per token / per feature."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rest = tuple(a for a in range(got.ndim) if a != axis)   # summed within each slice
    diff = got - ref
    num = np.sqrt(np.sum(diff * diff, axis=rest))
    den = np.sqrt(np.sum(ref * ref, axis=rest))
    return num / np.where(den > 0, den, 1.0)


# --------------------------------------------------------------------------
# int8 base weight ([X-zh] 2.6; [X-it] 2: training on a quantized base
# model, dequantized when needed)
# --------------------------------------------------------------------------
def dequant_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The float64 weight an int8 matrix q with one scale per output row
    stands for: W0[i, j] = s[i] * q[i, j] (exact in float64)."""
    q = np.asarray(q)
    s = np.asarray(s)
    assert q.ndim == 2 and s.shape == (q.shape[0],)
    return s.astype(np.float64)[:, None] * q.astype(np.float64)
