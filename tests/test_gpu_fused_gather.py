"""The one-pass gather + block products (poetx_set_fused_gather): the same
layer calls with the input-side gather read straight into the block
products' operands.  Against the float64 oracle on every output; the
gathered U and dS bit-exact; the memory-saving and int8-weight variants on
top of it; and the two settings against each other."""
import contextlib
import sys

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, act_of, bits, check_layer, raw, to_dev, to_f64
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


@contextlib.contextmanager
def fused(on=True):
    prev = P.poetx_set_fused_gather(on)
    try:
        yield
    finally:
        P.poetx_set_fused_gather(prev)


def make_layer(cfg, d, T, xmem=False):
    L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype), xmem=xmem)
    L.load(to_dev(d["W0"]), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
           to_dev(d["perm_P"]), to_dev(d["perm_R"]))
    return L


def layer_out(L, rows=None):
    sel = (lambda t: t) if rows is None else (lambda t: t[torch.as_tensor(rows, device="cuda")])
    return {"y": to_f64(sel(L.y)), "dx": to_f64(sel(L.dx)), "dG_P": to_f64(L.dG_P),
            "dG_R": to_f64(L.dG_R), "dtheta_P": to_f64(L.dtheta_P), "dtheta_R": to_f64(L.dtheta_R)}


def gathered(buf: torch.Tensor, T: int, width: int) -> np.ndarray:
    """The first T x width bf16 values of a byte buffer, as raw bits."""
    return bits(buf[: T * width * 2].view(torch.bfloat16).view(T, width))


@pytest.mark.parametrize("name,T", [("square", 96), ("square", 257), ("square", 1),
                                    ("mlp_up", 64), ("mid", 200)])
def test_fused_layer_parity_and_exact_gathers(name, T):
    """Every output against the oracle; U = x[:, pi_P] (saved for the
    backward) and dS = dy[:, pi_R] bit for bit.  square: both sides take
    the one-pass form (T = 1 and 257: a single token and a ragged last
    32-token group); mlp_up: the forward only (m = 14336 is too wide);
    mid: neither (b = 128), which must be unaffected."""
    cfg = I.CONFIG_BY_NAME[name]
    say(f"fused gather {name} T={T}")
    d = I.make_inputs(cfg, seed=31, T=T)
    with fused():
        L = make_layer(cfg, d, T)
        L.step(to_dev(d["x"]), to_dev(d["dy"]))
        torch.cuda.synchronize()
    y_ref, _ = O.layer_fwd(d["x64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                           d["perm_R"], cfg.b, cfg.k)
    g = O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    check_layer(layer_out(L), dict(g, y=y_ref), TOL[cfg.dtype], log=say)
    np.testing.assert_array_equal(gathered(L.saved, T, cfg.n), raw(d["x"])[:, d["perm_P"]])
    np.testing.assert_array_equal(gathered(L.ws_bwd, T, cfg.m), raw(d["dy"])[:, d["perm_R"]])


def test_fused_layer_full_size_square():
    """The square workload at its full 8192 tokens (one 32-token group per
    CU): sampled rows of y and dx, and every dtheta, against the oracle."""
    cfg = I.CONFIG_BY_NAME["square"]
    say(f"fused gather full square T={cfg.T}")
    d = I.make_inputs(cfg, seed=0)
    with fused():
        L = make_layer(cfg, d, cfg.T)
        L.step(to_dev(d["x"]), to_dev(d["dy"]))
        torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(3).choice(cfg.T, 48, replace=False))
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


def test_fused_pure_permutation_bit_exact():
    """theta = 0 and W0 a permutation matrix: every product is exact, so
    y and dx are column permutations of x and dy, bitwise, through the
    one-pass form (m = n = 512, b = 256: two blocks, six of eight waves
    without a block)."""
    m = n = 512
    b, T = 256, 130
    rng = np.random.default_rng(256)
    sigma = rng.permutation(n)
    W0 = np.zeros((m, n), np.float32)
    W0[np.arange(m), sigma] = 1.0
    st = I.bf16_round_bits
    x = rng.standard_normal((T, n)).astype(np.float32)
    dy = rng.standard_normal((T, m)).astype(np.float32)
    tb = b * (b - 1) // 2
    with fused():
        L = POETXLayer(m, n, b, 4, T, act_of("bf16"))
        L.load(to_dev(st(W0)), torch.zeros(n // b, tb, device="cuda"),
               torch.zeros(m // b, tb, device="cuda"),
               to_dev(rng.permutation(n).astype(np.int32)),
               to_dev(rng.permutation(m).astype(np.int32)))
        L.step(to_dev(st(x)), to_dev(st(dy)))
        torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(L.y), raw(st(x)[:, sigma]))
    np.testing.assert_array_equal(bits(L.dx), raw(st(dy)[:, O.inverse_perm(sigma)]))


@pytest.mark.parametrize("T", [96, 600])
def test_fused_xmem_bitwise_equals_fused_xfast(T):
    """With the one-pass form, the memory-saving backward recomputes V with
    the same kernel (identity map), so every output equals the default
    mode's bit for bit."""
    cfg = I.CONFIG_BY_NAME["square"]
    say(f"fused gather xmem square T={T}")
    d = I.make_inputs(cfg, seed=33, T=T)
    outs = []
    with fused():
        for xmem in (False, True):
            L = make_layer(cfg, d, T, xmem=xmem)
            L.step(to_dev(d["x"]), to_dev(d["dy"]))
            torch.cuda.synchronize()
            outs.append([bits(t).copy() for t in (L.y, L.dx, L.dG_P, L.dG_R, L.dtheta_P,
                                                  L.dtheta_R)])
            del L
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_fused_xq_parity():
    """The int8 base weight: the backward's per-column weight scale is
    applied inside the one-pass R-side block products."""
    cfg = I.CONFIG_BY_NAME["square"]
    T = 96
    say(f"fused gather xq square T={T}")
    d = I.make_inputs(cfg, seed=35, T=T)
    q, sc = I.quantize_rows_int8(d["W064"])
    with fused():
        L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype), xq=True)
        L.load_q(to_dev(q), to_dev(sc), to_dev(d["theta_P"]), to_dev(d["theta_R"]),
                 to_dev(d["perm_P"]), to_dev(d["perm_R"]))
        L.step(to_dev(d["x"]), to_dev(d["dy"]))
        torch.cuda.synchronize()
    W0q = O.dequant_rows(q, sc)
    y_ref, _ = O.layer_fwd(d["x64"], W0q, d["theta_P64"], d["theta_R64"], d["perm_P"],
                           d["perm_R"], cfg.b, cfg.k)
    g = O.layer_bwd(d["x64"], d["dy64"], W0q, d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    check_layer(layer_out(L), dict(g, y=y_ref), TOL[cfg.dtype], log=say)


def test_fused_and_two_pass_agree():
    """The two settings on the same inputs: the saved U identical, every
    output equal to rounding (relative Frobenius 1e-2 of bf16 storage; the
    block products only sum in a different order)."""
    cfg = I.CONFIG_BY_NAME["square"]
    T = 512
    say(f"fused vs two-pass square T={T}")
    d = I.make_inputs(cfg, seed=37, T=T)
    res = []
    for on in (False, True):
        with fused(on):
            L = make_layer(cfg, d, T)
            L.step(to_dev(d["x"]), to_dev(d["dy"]))
            torch.cuda.synchronize()
        res.append((gathered(L.saved, T, cfg.n).copy(), layer_out(L)))
        del L
    np.testing.assert_array_equal(res[0][0], res[1][0])
    for nm, a in res[0][1].items():
        b = res[1][1][nm]
        err = np.linalg.norm(a - b) / np.linalg.norm(a)
        say(f"  {nm}: {err:.2e}")
        assert err <= 1e-2, (nm, err)

