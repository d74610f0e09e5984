"""GPU parity: the HIP path through the C ABI against the float64 oracle on
the same seeded inputs.  Index work must be bit-exact.  Floating point is
held to 1e-5 (float32) or 2e-2 (bf16 storage) on every figure check_close
takes: relative Frobenius error of the whole tensor, of each block (G, dG,
dtheta), of each token row and feature column (y, dx), and
max |gpu - ref| / max |ref|."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, act_of, bits, check_close, check_layer, raw, to_dev, to_f64
from orthogonal_reparameterized_02_amd import inputs as I
from orthogonal_reparameterized_02_amd import poetx as P
from orthogonal_reparameterized_02_amd.layer import POETXLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()  # a missing library fails loudly here


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ fold
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m,n", [(96, 160), (1, 7), (2048, 2048), (14336, 4096)])
def test_fold_bit_exact(dtype, m, n):
    say(f"fold {dtype} {m}x{n}")
    rng = np.random.default_rng(m * 7 + n)
    w = rng.standard_normal((m, n)).astype(np.float32)
    W0 = I.bf16_round_bits(w) if dtype == "bf16" else w
    pR, pP = rng.permutation(m).astype(np.int32), rng.permutation(n).astype(np.int32)
    ref, iR, iP = O.fold_perm(W0, pR, pP)
    dW0 = to_dev(W0)
    W0f, W0fT = torch.empty_like(dW0), torch.empty(n, m, dtype=dW0.dtype, device="cuda")
    iRd = torch.empty(m, dtype=torch.int32, device="cuda")
    iPd = torch.empty(n, dtype=torch.int32, device="cuda")
    P.poetx_fold_perm(dW0, to_dev(pR), to_dev(pP), W0f, W0fT, iRd, iPd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(W0f), raw(ref))
    np.testing.assert_array_equal(bits(W0fT), raw(ref.T))
    np.testing.assert_array_equal(iRd.cpu().numpy(), iR)
    np.testing.assert_array_equal(iPd.cpu().numpy(), iP)


# ------------------------------------------------------------------ CNP
CNP_CASES = [  # nblk, b, k, dtype, sigma
    (8, 32, 4, "f32", 0.02),
    (5, 64, 3, "f32", 0.02),
    (3, 16, 0, "f32", 0.1),
    (4, 8, 2, "bf16", 0.05),
    (3, 64, 4, "bf16", 0.02),
    (4, 64, 0, "bf16", 0.02),
    (4, 64, 1, "bf16", 0.02),
    (16, 128, 4, "bf16", 0.01),
    (32, 256, 4, "bf16", 0.01),
    (5, 256, 2, "bf16", 0.01),
    (3, 512, 5, "bf16", 0.005),
    (37, 512, 5, "bf16", 0.005),   # six panels a block: four of 96 columns, two of 64
    (40, 512, 1, "bf16", 0.005),   # the same, a single step
    (74, 512, 5, "bf16", 0.005),   # 128-column panels for 64 blocks, 64-column ones for 10
    (65, 512, 3, "bf16", 0.005),   # the same split with a single 64-column block
    (64, 512, 4, "bf16", 0.005),   # exactly one round of wide panels, no tail
    (1, 512, 2, "bf16", 0.005),    # one block: narrow panels only
    (2, 512, 0, "bf16", 0.005),
    (2, 512, 1, "bf16", 0.005),
]


def _cnp_inputs(nblk, b, sigma, seed):
    rng = np.random.default_rng(seed)
    th = (rng.standard_normal((nblk, b * (b - 1) // 2)) * sigma).astype(np.float32)
    dG = rng.standard_normal((nblk, b, b)).astype(np.float32)
    return th, dG


@pytest.mark.parametrize("nblk,b,k,dtype,sigma", CNP_CASES)
def test_cnp_fwd(nblk, b, k, dtype, sigma):
    say(f"cnp_fwd nblk={nblk} b={b} k={k} {dtype}")
    th, _ = _cnp_inputs(nblk, b, sigma, b + k)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    G = torch.empty(nblk, b, b, dtype=tdt, device="cuda")
    GT = torch.empty_like(G)
    ws = torch.empty(max(16, P.poetx_cnp_workspace_bytes(nblk, b, k, 0, act_of(dtype))),
                     dtype=torch.uint8, device="cuda")
    P.poetx_cnp_fwd(to_dev(th), b, k, G, GT, ws)
    torch.cuda.synchronize()
    ref = O.cnp_fwd(th.astype(np.float64), b, k)
    check_close("G", to_f64(G), ref, TOL[dtype], blocks=True, log=say)
    np.testing.assert_array_equal(bits(GT), bits(G).transpose(0, 2, 1))


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("nblk,b,k,dtype,sigma", CNP_CASES)
def test_cnp_bwd(nblk, b, k, dtype, sigma, accumulate):
    say(f"cnp_bwd nblk={nblk} b={b} k={k} {dtype} acc={accumulate}")
    th, dG = _cnp_inputs(nblk, b, sigma, 1000 + b + k)
    tb = b * (b - 1) // 2
    prior = np.random.default_rng(5).standard_normal((nblk, tb)).astype(np.float32)
    dth = to_dev(prior.copy())
    ws = torch.empty(max(16, P.poetx_cnp_workspace_bytes(nblk, b, k, 1, act_of(dtype))),
                     dtype=torch.uint8, device="cuda")
    P.poetx_cnp_bwd(to_dev(th), to_dev(dG), b, k, dth, act_of(dtype), accumulate, ws)
    torch.cuda.synchronize()
    ref = O.cnp_bwd(th.astype(np.float64), dG.astype(np.float64), b, k)
    got = to_f64(dth)
    if accumulate:
        got = got - prior.astype(np.float64)
    check_close("dtheta", got, ref, TOL[dtype], blocks=True, log=say)


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("nblk,b,k,dtype,sigma", [(32, 256, 4, "bf16", 0.01), (16, 128, 4, "bf16", 0.01),
                                                  (3, 512, 5, "bf16", 0.005), (5, 64, 3, "f32", 0.02)])
def test_cnp_bwd_after_fwd_bitwise(nblk, b, k, dtype, sigma, accumulate):
    """The backward that reuses the forward's unpacked Q (the workspace
    that served poetx_cnp_fwd) gives poetx_cnp_bwd's dtheta bit for bit."""
    say(f"cnp_bwd_after_fwd nblk={nblk} b={b} k={k} {dtype} acc={accumulate}")
    th, dG = _cnp_inputs(nblk, b, sigma, 2000 + b + k)
    tb = b * (b - 1) // 2
    prior = np.random.default_rng(6).standard_normal((nblk, tb)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    G = torch.empty(nblk, b, b, dtype=tdt, device="cuda")
    ws = torch.empty(max(16, P.poetx_cnp_workspace_bytes(nblk, b, k, 1, act_of(dtype))),
                     dtype=torch.uint8, device="cuda")
    th_d, dG_d = to_dev(th), to_dev(dG)
    outs = []
    for after in (False, True):
        ws.fill_(0x5A)  # the reuse must not depend on anything but the forward's writes
        P.poetx_cnp_fwd(th_d, b, k, G, None, ws)
        dth = to_dev(prior.copy())
        P.poetx_cnp_bwd(th_d, dG_d, b, k, dth, act_of(dtype), accumulate, ws, after_fwd=after)
        torch.cuda.synchronize()
        outs.append(bits(dth).copy())
    np.testing.assert_array_equal(outs[0], outs[1])


# ------------------------------------------------------------------ the layer
def run_layer(cfg, d, T):
    L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype))
    L.load(to_dev(d["W0"]), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
           to_dev(d["perm_P"]), to_dev(d["perm_R"]))
    x, dy = to_dev(d["x"]), to_dev(d["dy"])
    L.step(x, dy)
    torch.cuda.synchronize()
    return L


def layer_out(L, rows=None):
    """The layer's outputs as float64 host arrays (y and dx restricted to
    `rows` when given)."""
    sel = (lambda t: t) if rows is None else (lambda t: t[torch.as_tensor(rows, device="cuda")])
    return {"y": to_f64(sel(L.y)), "dx": to_f64(sel(L.dx)), "dG_P": to_f64(L.dG_P),
            "dG_R": to_f64(L.dG_R), "dtheta_P": to_f64(L.dtheta_P), "dtheta_R": to_f64(L.dtheta_R)}


SMALL_T = {"probe": 64, "mid": 200, "square": 96, "mlp_up": 64, "mlp13b": 40}


@pytest.mark.parametrize("name", [c.name for c in I.CONFIGS])
def test_layer_parity_small_T(name):
    """Every config's layer shape at a token count the oracle finishes in
    seconds (not a multiple of any tile size where possible)."""
    cfg = I.CONFIG_BY_NAME[name]
    T = SMALL_T[name]
    say(f"layer {name} T={T}")
    d = I.make_inputs(cfg, seed=11, T=T)
    L = run_layer(cfg, d, T)
    y_ref, _ = O.layer_fwd(d["x64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                           d["perm_R"], cfg.b, cfg.k)
    g = O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    check_layer(layer_out(L), dict(g, y=y_ref), TOL[cfg.dtype], log=say)


@pytest.mark.parametrize("name,T,k", [("square", 1, 4), ("square", 257, 4), ("mid", 33, 0),
                                      ("mid", 4063, 4), ("mlp_up", 4100, 4), ("mlp13b", 1, 5),
                                      ("probe", 1, 0)])
def test_layer_edge_cases(name, T, k):
    """One token, a ragged tail just past a 256-token tile, a ragged last
    tile on the 256 x 256 dense path (mid, 128 tiles), uneven token splits
    of the 56-block pass and the joint 72-block dG reduction (mlp_up), and
    k = 0 (G = I + Q): every output against the oracle."""
    base = I.CONFIG_BY_NAME[name]
    cfg = I.LayerConfig(base.name, base.m, base.n, base.b, k, T, base.dtype, base.sigma)
    say(f"edge {name} T={T} k={k}")
    d = I.make_inputs(cfg, seed=17, T=T)
    L = run_layer(cfg, d, T)
    y_ref, _ = O.layer_fwd(d["x64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                           d["perm_R"], cfg.b, cfg.k)
    g = O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    check_layer(layer_out(L), dict(g, y=y_ref), TOL[cfg.dtype], log=say)


@pytest.mark.parametrize("name", ["mid", "square", "mlp_up", "mlp13b"])
def test_layer_parity_full_size(name):
    """Full token count, the launch configuration the bench times: sampled
    rows of y and dx against the oracle row by row, and the whole dtheta
    (a reduction over every token) against the full oracle."""
    cfg = I.CONFIG_BY_NAME[name]
    say(f"layer full {name} T={cfg.T}")
    d = I.make_inputs(cfg, seed=0)
    L = run_layer(cfg, d, cfg.T)
    rows = np.sort(np.random.default_rng(1).choice(cfg.T, 48, replace=False))
    rows[-1] = cfg.T - 1
    G_P = O.cnp_fwd(d["theta_P64"], cfg.b, cfg.k)
    G_R = O.cnp_fwd(d["theta_R64"], cfg.b, cfg.k)
    W = O.weight(d["W064"], G_R, G_P, d["perm_R"], d["perm_P"])
    ref = {"y": d["x64"][rows] @ W.T, "dx": d["dy64"][rows] @ W}
    del W
    g = O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    ref.update({nm: g[nm] for nm in ("dG_P", "dG_R", "dtheta_P", "dtheta_R")})
    check_layer(layer_out(L, rows), ref, TOL[cfg.dtype], log=say)


@pytest.mark.parametrize("dtype,b", [("bf16", 256), ("bf16", 128), ("bf16", 32), ("f32", 32)])
def test_pure_permutation_layer_bit_exact(dtype, b):
    """theta = 0 and W0 a permutation matrix: every output is one exact
    product, so y is a column permutation of x and dx one of dy, bitwise."""
    say(f"pure permutation {dtype} b={b}")
    m = n = 2 * max(b, 64)
    T = 130
    rng = np.random.default_rng(b)
    sigma = rng.permutation(n)
    W0 = np.zeros((m, n), np.float32)
    W0[np.arange(m), sigma] = 1.0
    x = rng.standard_normal((T, n)).astype(np.float32)
    dy = rng.standard_normal((T, m)).astype(np.float32)
    st = (lambda a: I.bf16_round_bits(a)) if dtype == "bf16" else (lambda a: a)
    tb = b * (b - 1) // 2
    L = POETXLayer(m, n, b, 4, T, act_of(dtype))
    L.load(to_dev(st(W0)), torch.zeros(n // b, tb, device="cuda"),
           torch.zeros(m // b, tb, device="cuda"),
           to_dev(rng.permutation(n).astype(np.int32)), to_dev(rng.permutation(m).astype(np.int32)))
    L.step(to_dev(st(x)), to_dev(st(dy)))
    torch.cuda.synchronize()
    xs, dys = st(x), st(dy)
    # y[t][i] = x[t][sigma[i]];  dx[t][j] = dy[t][sigma^{-1}[j]]
    y_ref, _ = O.layer_fwd(I.to_f64(xs, dtype), I.to_f64(st(W0), dtype),
                           np.zeros((n // b, tb)), np.zeros((m // b, tb)),
                           np.arange(n), np.arange(m), b, 4)
    np.testing.assert_array_equal(bits(L.y), raw(xs[:, sigma]))
    np.testing.assert_array_equal(to_f64(L.y), y_ref)
    np.testing.assert_array_equal(bits(L.dx), raw(dys[:, O.inverse_perm(sigma)]))


def test_repeat_runs_bitwise_equal():
    cfg = I.CONFIG_BY_NAME["square"]
    d = I.make_inputs(cfg, seed=2, T=512)
    L = run_layer(cfg, d, 512)
    first = [bits(t).copy() for t in (L.y, L.dx, L.dtheta_P, L.dtheta_R)]
    L.step(to_dev(d["x"]), to_dev(d["dy"]))
    torch.cuda.synchronize()
    for a, t in zip(first, (L.y, L.dx, L.dtheta_P, L.dtheta_R)):
        np.testing.assert_array_equal(a, bits(t))


# ------------------------------------------------------------------ one copy of the weight
KMAJOR_CASES = [("probe", 64, None), ("mid", 200, None), ("square", 96, None),
                ("square", 8192, None), ("mlp_up", 64, None), ("mlp13b", 40, None),
                ("b64_narrow", 100, I.LayerConfig("b64_narrow", 256, 192, 64, 4, 100, "bf16", 0.02))]


@pytest.mark.parametrize("name,T,cfg", KMAJOR_CASES)
def test_backward_reads_w0f_itself(name, T, cfg):
    """The backward's dense product dV = dZ W0f read straight from W0f
    (K-major: the layer holds one copy of the fixed weight) equals the read
    from a transposed copy bit for bit, on every kernel path: the fused
    b = 256 and b = 128 epilogues, the unfused b = 512 product, the fp32
    and narrow-width portable kernels; the memory-saving mode likewise."""
    cfg = cfg or I.CONFIG_BY_NAME[name]
    say(f"K-major W0f {cfg.name} T={T}")
    d = I.make_inputs(cfg, seed=25, T=T)
    for xmem in (False, True):
        outs = []
        for keep in (True, False):
            L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype), xmem=xmem,
                           keep_w0ft=keep)
            assert (L.W0fT is not None) == keep
            L.load(to_dev(d["W0"]), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
                   to_dev(d["perm_P"]), to_dev(d["perm_R"]))
            L.step(to_dev(d["x"]), to_dev(d["dy"]))
            torch.cuda.synchronize()
            outs.append([bits(t).copy() for t in (L.dx, L.dG_P, L.dG_R, L.dtheta_P, L.dtheta_R)])
            del L
        for a, b in zip(*outs):
            np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------ xmem mode
@pytest.mark.parametrize("name,T", [("probe", 64), ("mid", 200), ("square", 96),
                                    ("mlp13b", 40), ("square", 8192), ("mlp_up", 600)])
def test_xmem_bitwise_equals_xfast(name, T):
    """The memory-saving mode keeps only U and recomputes Z in the backward
    with the forward's own kernels, so every output equals the default
    mode's bit for bit; its saved buffer is T*m elements smaller."""
    cfg = I.CONFIG_BY_NAME[name]
    say(f"xmem {name} T={T}")
    d = I.make_inputs(cfg, seed=21, T=T)
    outs = []
    for xmem in (False, True):
        L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype), xmem=xmem)
        L.load(to_dev(d["W0"]), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
               to_dev(d["perm_P"]), to_dev(d["perm_R"]))
        L.step(to_dev(d["x"]), to_dev(d["dy"]))
        torch.cuda.synchronize()
        outs.append([bits(t).copy() for t in (L.y, L.dx, L.dG_P, L.dG_R, L.dtheta_P, L.dtheta_R)])
        if xmem:
            es = 2 if cfg.dtype == "bf16" else 4
            assert (P.poetx_saved_bytes(L.sh) - P.poetx_saved_bytes_xmem(L.sh)) >= T * cfg.m * es
        del L
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("T", [72, 600])
def test_xmem_parity_small_T(T):
    """The memory-saving mode against the oracle directly (T = 600: the
    joint dG reduction over three token splits, the last one ragged)."""
    cfg = I.CONFIG_BY_NAME["square"]
    say(f"xmem parity square T={T}")
    d = I.make_inputs(cfg, seed=23, T=T)
    L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype), xmem=True)
    L.load(to_dev(d["W0"]), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
           to_dev(d["perm_P"]), to_dev(d["perm_R"]))
    L.step(to_dev(d["x"]), to_dev(d["dy"]))
    torch.cuda.synchronize()
    y_ref, _ = O.layer_fwd(d["x64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                           d["perm_R"], cfg.b, cfg.k)
    g = O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    check_layer(layer_out(L), dict(g, y=y_ref), TOL[cfg.dtype], log=say)


# ------------------------------------------------------------------ merge
@pytest.mark.parametrize("name", ["probe", "mid", "square", "mlp_up", "mlp13b"])
def test_merge_matches_oracle_weight(name):
    """poetx_merge returns R W0 P (the oracle's explicit weight); mlp_up's
    56 R-side blocks take the block kernel's one-round token split."""
    cfg = I.CONFIG_BY_NAME[name]
    say(f"merge {name}")
    d = I.make_inputs(cfg, seed=31, T=8, want=("W0", "theta_P", "theta_R", "perm_P", "perm_R"))
    L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, 8, act_of(cfg.dtype))
    L.load(to_dev(d["W0"]), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
           to_dev(d["perm_P"]), to_dev(d["perm_R"]))
    L.cnp()
    W = L.merge()
    torch.cuda.synchronize()
    G_P = O.cnp_fwd(d["theta_P64"], cfg.b, cfg.k)
    G_R = O.cnp_fwd(d["theta_R64"], cfg.b, cfg.k)
    ref = O.weight(d["W064"], G_R, G_P, d["perm_R"], d["perm_P"])
    check_close("W", to_f64(W), ref, TOL[cfg.dtype], rows=True, cols=True, log=say)


@pytest.mark.parametrize("name", ["probe", "square"])
def test_merge_at_identity_bit_exact(name):
    """theta = 0 makes R = P = I: the merge gives back W0 bit for bit."""
    cfg = I.CONFIG_BY_NAME[name]
    d = I.make_inputs(cfg, seed=33, T=8, want=("W0", "perm_P", "perm_R"))
    L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, 8, act_of(cfg.dtype))
    tb = cfg.tri
    L.load(to_dev(d["W0"]), torch.zeros(cfg.n_P, tb, device="cuda"),
           torch.zeros(cfg.n_R, tb, device="cuda"), to_dev(d["perm_P"]), to_dev(d["perm_R"]))
    L.cnp()
    W = L.merge()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(W), raw(d["W0"]))


def test_end_inner_loop_keeps_the_function():
    """Merge, reset theta to 0 and redraw the permutations: the layer
    computes the same function as before (to bf16 rounding)."""
    from orthogonal_reparameterized_02_amd.layer import POETXLinear
    torch.manual_seed(1)
    mod = POETXLinear(n=512, m=768, b=128, k=4, dtype=torch.bfloat16, seed=4)
    with torch.no_grad():
        mod.theta_P.normal_(0, 0.02)
        mod.theta_R.normal_(0, 0.02)
    x = torch.randn(64, 512, device="cuda").to(torch.bfloat16)
    with torch.no_grad():
        y0 = mod(x).float().cpu().numpy().astype(np.float64)
        perm_before = mod.perm_P.clone()
        mod.end_inner_loop()
        assert float(mod.theta_P.abs().max()) == 0.0 and float(mod.theta_R.abs().max()) == 0.0
        assert not torch.equal(perm_before, mod.perm_P)
        y1 = mod(x).float().cpu().numpy().astype(np.float64)
    check_close("y after the merge", y1, y0, TOL["bf16"], rows=True, cols=True, log=say)


# ------------------------------------------------------------------ POET-XQ
def test_fold_int8_and_scales_bit_exact():
    rng = np.random.default_rng(41)
    m, n = 768, 512
    q = rng.integers(-127, 128, size=(m, n)).astype(np.int8)
    s = rng.uniform(0.001, 0.01, size=m).astype(np.float32)
    pR, pP = rng.permutation(m).astype(np.int32), rng.permutation(n).astype(np.int32)
    qf = torch.empty(m, n, dtype=torch.int8, device="cuda")
    qfT = torch.empty(n, m, dtype=torch.int8, device="cuda")
    sf = torch.empty(m, dtype=torch.float32, device="cuda")
    P.poetx_fold_perm(to_dev(q), to_dev(pR), to_dev(pP), qf, qfT)
    P.poetx_fold_scale(to_dev(s), to_dev(pR), sf)
    torch.cuda.synchronize()
    ref, _, _ = O.fold_perm(q, pR, pP)
    np.testing.assert_array_equal(qf.cpu().numpy(), ref)
    np.testing.assert_array_equal(qfT.cpu().numpy(), ref.T)
    np.testing.assert_array_equal(sf.cpu().numpy(), s[pR])


@pytest.mark.parametrize("per_row", [True, False])
def test_dequant_bit_exact(per_row):
    """bf16(s * q) with one float32 multiply and round-to-nearest-even."""
    rng = np.random.default_rng(43)
    rows, cols = 320, 448
    q = rng.integers(-127, 128, size=(rows, cols)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-1, size=rows if per_row else cols).astype(np.float32)
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    P.poetx_dequant(to_dev(q), to_dev(s), per_row, out)
    torch.cuda.synchronize()
    sb = s[:, None] if per_row else s[None, :]
    ref = I.bf16_round_bits((sb * q.astype(np.float32)).astype(np.float32))
    np.testing.assert_array_equal(bits(out), ref)


def _xq_layer(cfg, d, T, xmem=False):
    q, sc = I.quantize_rows_int8(d["W064"])
    L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype), xq=True, xmem=xmem)
    assert L.W0f is None and L.W0fT is None          # no bf16 copy of the weight
    L.load_q(to_dev(q), to_dev(sc), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
             to_dev(d["perm_P"]), to_dev(d["perm_R"]))
    L.step(to_dev(d["x"]), to_dev(d["dy"]))
    torch.cuda.synchronize()
    return L, O.dequant_rows(q, sc)


@pytest.mark.parametrize("name,T", [("mid", 200), ("square", 96), ("mlp_up", 64), ("mlp13b", 40),
                                    ("square", 600)])
def test_xq_layer_parity_small_T(name, T):
    """The layer on an int8 base weight, read by the dense kernels as int8
    and widened in their operand path, against the oracle on the weight the
    int8 pair represents (every workload shape; b = 128 and 256 carry the
    block epilogue, b = 512 the separate block products)."""
    cfg = I.CONFIG_BY_NAME[name]
    say(f"xq {name} T={T}")
    d = I.make_inputs(cfg, seed=45, T=T)
    L, W0q = _xq_layer(cfg, d, T)
    y_ref, _ = O.layer_fwd(d["x64"], W0q, d["theta_P64"], d["theta_R64"], d["perm_P"],
                           d["perm_R"], cfg.b, cfg.k)
    g = O.layer_bwd(d["x64"], d["dy64"], W0q, d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    check_layer(layer_out(L), dict(g, y=y_ref), TOL[cfg.dtype], log=say)


@pytest.mark.parametrize("name,T", [("square", 96), ("mid", 200), ("mlp13b", 40)])
def test_xq_xmem_bitwise_equals_xq(name, T):
    """The memory-saving mode on the int8 weight recomputes Z with the
    forward's own int8 kernel: every output equals the default mode's."""
    cfg = I.CONFIG_BY_NAME[name]
    say(f"xq xmem {name} T={T}")
    d = I.make_inputs(cfg, seed=47, T=T)
    outs = []
    for xmem in (False, True):
        L, _ = _xq_layer(cfg, d, T, xmem=xmem)
        outs.append([bits(t).copy() for t in (L.y, L.dx, L.dG_P, L.dG_R, L.dtheta_P, L.dtheta_R)])
        del L
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_xq_layer_full_size():
    cfg = I.CONFIG_BY_NAME["square"]
    d = I.make_inputs(cfg, seed=0)
    L, W0q = _xq_layer(cfg, d, cfg.T)
    rows = np.sort(np.random.default_rng(3).choice(cfg.T, 32, replace=False))
    G_P = O.cnp_fwd(d["theta_P64"], cfg.b, cfg.k)
    G_R = O.cnp_fwd(d["theta_R64"], cfg.b, cfg.k)
    W = O.weight(W0q, G_R, G_P, d["perm_R"], d["perm_P"])
    ref = {"y": d["x64"][rows] @ W.T, "dx": d["dy64"][rows] @ W}
    del W
    g = O.layer_bwd(d["x64"], d["dy64"], W0q, d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    ref.update({nm: g[nm] for nm in ("dG_P", "dG_R", "dtheta_P", "dtheta_R")})
    check_layer(layer_out(L, rows), ref, TOL["bf16"], log=say)


def test_graph_replays_match_eager():
    """The whole step captured as one HIP graph: every replay, with other
    eager work and synchronizations in between, equals the eager step bit
    for bit (the step records no memset nodes)."""
    cfg = I.CONFIG_BY_NAME["square"]
    T = 512
    d = I.make_inputs(cfg, seed=51, T=T)
    L = run_layer(cfg, d, T)
    ref = [bits(t).copy() for t in (L.y, L.dx, L.dtheta_P, L.dtheta_R)]
    other = run_layer(cfg, I.make_inputs(cfg, seed=52, T=T), T)
    x, dy = to_dev(d["x"]), to_dev(d["dy"])
    L.step(x, dy)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.step(x, dy)
    torch.cuda.synchronize()
    for i in range(3):
        other.step(to_dev(I.make_inputs(cfg, seed=60 + i, T=T, want=("x",))["x"]),
                   to_dev(d["dy"]))          # eager work between replays
        torch.cuda.synchronize()
        for t in (L.y, L.dx, L.dtheta_P, L.dtheta_R):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, t in zip(ref, (L.y, L.dx, L.dtheta_P, L.dtheta_R)):
            np.testing.assert_array_equal(a, bits(t))


def test_autograd_module_matches_layer():
    from orthogonal_reparameterized_02_amd.layer import POETXLinear
    torch.manual_seed(0)
    mod = POETXLinear(n=512, m=768, b=128, k=4, dtype=torch.bfloat16, seed=3)
    with torch.no_grad():
        mod.theta_P.normal_(0, 0.01)
        mod.theta_R.normal_(0, 0.01)
    x = torch.randn(64, 512, device="cuda").to(torch.bfloat16).requires_grad_(True)
    y = mod(x)
    dy = torch.randn_like(y)
    y.backward(dy)
    torch.cuda.synchronize()
    pP, pR = mod.perm_P.cpu().numpy(), mod.perm_R.cpu().numpy()
    W0 = to_f64(mod.W0)
    ref_y, _ = O.layer_fwd(to_f64(x), W0, to_f64(mod.theta_P), to_f64(mod.theta_R), pP, pR, 128, 4)
    g = O.layer_bwd(to_f64(x), to_f64(dy), W0, to_f64(mod.theta_P), to_f64(mod.theta_R), pP, pR,
                    128, 4)
    check_layer({"y": to_f64(y), "dx": to_f64(x.grad), "dtheta_P": to_f64(mod.theta_P.grad),
                 "dtheta_R": to_f64(mod.theta_R.grad)}, dict(g, y=ref_y), TOL["bf16"], log=say)


def test_autograd_module_is_reentrant():
    """Two forwards of different token counts (one with a leading batch
    axis), both before either backward, then one backward over both: y, dx
    of each call against the oracle, and the theta gradients against the
    oracle's over all tokens of both calls (dG sums over tokens and dtheta
    is linear in dG, so the two calls' gradients add)."""
    from orthogonal_reparameterized_02_amd.layer import POETXLinear
    torch.manual_seed(2)
    mod = POETXLinear(n=512, m=768, b=128, k=4, dtype=torch.bfloat16, seed=5)
    with torch.no_grad():
        mod.theta_P.normal_(0, 0.01)
        mod.theta_R.normal_(0, 0.01)
    x1 = torch.randn(2, 40, 512, device="cuda").to(torch.bfloat16).requires_grad_(True)
    x2 = torch.randn(72, 512, device="cuda").to(torch.bfloat16).requires_grad_(True)
    y1 = mod(x1)
    y2 = mod(x2)
    assert y1.shape == (2, 40, 768) and y2.shape == (72, 768)
    dy1, dy2 = torch.randn_like(y1), torch.randn_like(y2)
    torch.autograd.backward([y1, y2], [dy1, dy2])
    torch.cuda.synchronize()
    pP, pR = mod.perm_P.cpu().numpy(), mod.perm_R.cpu().numpy()
    W0, thP, thR = to_f64(mod.W0), to_f64(mod.theta_P), to_f64(mod.theta_R)
    xs = [to_f64(x1).reshape(80, 512), to_f64(x2)]
    dys = [to_f64(dy1).reshape(80, 768), to_f64(dy2)]
    for xx, dd, y, gx in ((xs[0], dys[0], y1, x1.grad), (xs[1], dys[1], y2, x2.grad)):
        ref_y, _ = O.layer_fwd(xx, W0, thP, thR, pP, pR, 128, 4)
        g = O.layer_bwd(xx, dd, W0, thP, thR, pP, pR, 128, 4)
        check_layer({"y": to_f64(y).reshape(xx.shape[0], 768),
                     "dx": to_f64(gx).reshape(xx.shape[0], 512)},
                    dict(g, y=ref_y), TOL["bf16"], log=say)
    g = O.layer_bwd(np.concatenate(xs), np.concatenate(dys), W0, thP, thR, pP, pR, 128, 4)
    check_layer({"dtheta_P": to_f64(mod.theta_P.grad), "dtheta_R": to_f64(mod.theta_R.grad)},
                g, TOL["bf16"], log=say)
    with pytest.raises(ValueError, match="features"):
        mod(torch.zeros(4, 256, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="dtype"):
        mod(torch.zeros(4, 512, dtype=torch.float32, device="cuda"))
