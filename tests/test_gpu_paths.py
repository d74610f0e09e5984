"""GPU parity on launch paths the workload tests do not reach: the dG token
reduction forced into several splits because one split of the widest operand
would pass the 2^31-byte range of a buffer resource, and bf16 layers with
block sizes below 128 (the register-staged MFMA kernels for b = 64, the
portable kernels below)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, act_of, check_close, check_layer, to_dev, to_f64
from orthogonal_reparameterized_02_amd import inputs as I
from orthogonal_reparameterized_02_amd import poetx as P
from orthogonal_reparameterized_02_amd.layer import POETXLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _layer(cfg, T):
    return POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, T, act_of(cfg.dtype))


def _load(L, d):
    L.load(to_dev(d["W0"]), to_dev(d["theta_P"]), to_dev(d["theta_R"]), to_dev(d["perm_P"]),
           to_dev(d["perm_R"]))


def _outputs(L, rows):
    r = torch.as_tensor(rows, device="cuda")
    return {"y": to_f64(L.y[r]), "dx": to_f64(L.dx[r]), "dG_P": to_f64(L.dG_P),
            "dG_R": to_f64(L.dG_R), "dtheta_P": to_f64(L.dtheta_P),
            "dtheta_R": to_f64(L.dtheta_R)}


def _row_refs(cfg, d, rows, W0=None):
    G_P = O.cnp_fwd(d["theta_P64"], cfg.b, cfg.k)
    G_R = O.cnp_fwd(d["theta_R64"], cfg.b, cfg.k)
    W = O.weight(d["W064"] if W0 is None else W0, G_R, G_P, d["perm_R"], d["perm_P"])
    return {"y": d["x64"][rows] @ W.T, "dx": d["dy64"][rows] @ W}, G_P, G_R


def _sample_rows(T, count, seed):
    rows = np.sort(np.random.default_rng(seed).choice(T, count, replace=False))
    rows[0], rows[-1] = 0, T - 1
    return rows


@pytest.mark.timeout(600)
def test_dG_forced_token_splits_narrow_full_oracle():
    """m = 15872 (31 blocks), n = 512 (1 block), b = 512, k = 5,
    T = 69632: the 32 blocks x 4 tiles of the joint dG launch would need no
    token split, but one split of the 15872-wide operands would span
    69632 * 15872 * 2 > 2^31 bytes, so the reduction takes two splits with
    fp32 partials.  n = 512 keeps the full float64 oracle affordable: every
    block of dG and dtheta against it, and sampled rows of y and dx."""
    cfg = I.LayerConfig("split_narrow", 15872, 512, 512, 5, 69632, "bf16", 0.005)
    assert cfg.T * cfg.m * 2 >= 2 ** 31
    say(f"forced splits {cfg}")
    d = I.make_inputs(cfg, seed=71)
    L = _layer(cfg, cfg.T)
    _load(L, d)
    L.step(to_dev(d["x"]), to_dev(d["dy"]))
    torch.cuda.synchronize()
    rows = _sample_rows(cfg.T, 48, 5)
    out = _outputs(L, rows)
    del L
    torch.cuda.empty_cache()
    ref, _, _ = _row_refs(cfg, d, rows)
    g = O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
    ref.update({nm: g[nm] for nm in ("dG_P", "dG_R", "dtheta_P", "dtheta_R")})
    check_layer(out, ref, TOL["bf16"], log=say)


@pytest.mark.timeout(900)
def test_dG_forced_token_splits_mlp13b_large_T():
    """The Llama-13B MLP shape (m = 13824, n = 5120, b = 512, k = 5; its 37
    blocks x 4 tiles need no token split) at T = 81920, where one split of
    the 13824-wide operands would span 81920 * 13824 * 2 > 2^31 bytes.
    Against the float64 oracle: sampled rows of y and dx, four bilinear
    probes u^T dG v of every block (O.dG_probes, without forming dG), and
    dtheta against the oracle's CNP backward of the GPU's own dG.  The
    reduction is a sum over tokens, so dG also equals the sum of the dG of
    the two halves of the token range, each run on its own (one split each,
    no partials)."""
    base = I.CONFIG_BY_NAME["mlp13b"]
    T = 81920
    cfg = I.LayerConfig(base.name, base.m, base.n, base.b, base.k, T, base.dtype, base.sigma)
    assert T * cfg.m * 2 >= 2 ** 31 and (T // 2) * cfg.m * 2 < 2 ** 31
    say(f"forced splits mlp13b T={T}")
    d = I.make_inputs(cfg, seed=73)
    x, dy = to_dev(d["x"]), to_dev(d["dy"])
    L = _layer(cfg, T)
    _load(L, d)
    L.step(x, dy)
    torch.cuda.synchronize()
    rows = _sample_rows(T, 48, 7)
    out = _outputs(L, rows)
    del L
    torch.cuda.empty_cache()
    # the two halves of the token range, one launch each
    H = T // 2
    Lh = _layer(cfg, H)
    _load(Lh, d)
    halves = []
    for h in range(2):
        Lh.step(x[h * H:(h + 1) * H].contiguous(), dy[h * H:(h + 1) * H].contiguous())
        torch.cuda.synchronize()
        halves.append((to_f64(Lh.dG_P), to_f64(Lh.dG_R)))
    del Lh, x, dy
    torch.cuda.empty_cache()
    for nm, s, tot in (("dG_P", 0, out["dG_P"]), ("dG_R", 1, out["dG_R"])):
        check_close(nm + " = sum of the halves", tot, halves[0][s] + halves[1][s], 1e-6,
                    blocks=True, log=say)
    # the oracle
    ref, G_P, G_R = _row_refs(cfg, d, rows)
    for nm in ("y", "dx"):
        check_close(nm, out[nm], ref[nm], TOL["bf16"], rows=True, cols=True, log=say)
    rng = np.random.default_rng(75)
    npr = 4
    u_P, v_P = rng.standard_normal((2, npr, cfg.n_P, cfg.b))
    u_R, v_R = rng.standard_normal((2, npr, cfg.n_R, cfg.b))
    pP, pR = O.dG_probes(d["x64"], d["dy64"], d["W064"], G_P, G_R, d["perm_P"], d["perm_R"],
                         u_P, v_P, u_R, v_R)
    gP = np.einsum("qjr,jrc,qjc->qj", u_P, out["dG_P"], v_P)
    gR = np.einsum("qir,irc,qic->qi", u_R, out["dG_R"], v_R)
    # per block: the four probes as one vector (axis 1 of [probes, blocks])
    check_close("u^T dG_P v", gP, pP, TOL["bf16"], cols=False, log=say)
    check_close("u^T dG_R v", gR, pR, TOL["bf16"], log=say)
    for name, got, want in (("probe block P", gP, pP), ("probe block R", gR, pR)):
        worst = float(O.rel_fro_slices(got, want, 1).max())
        say(f"  {name}: worst block {worst:.2e}")
        assert worst <= TOL["bf16"], (name, worst)
    for nm, th, s in (("dtheta_P", d["theta_P64"], "dG_P"), ("dtheta_R", d["theta_R64"], "dG_R")):
        check_close(nm + " (CNP backward of the GPU's dG)", out[nm],
                    O.cnp_bwd(th, out[s], cfg.b, cfg.k), TOL["bf16"], blocks=True, log=say)


SMALL_B = [  # name, m, n, b, k, T, dtype, sigma
    ("bf16_b64", 768, 512, 64, 4, 200, "bf16", 0.02),
    ("bf16_b64_split", 768, 512, 64, 4, 1000, "bf16", 0.02),   # joint dG launch, 4 token splits
    ("bf16_b16", 256, 192, 16, 4, 100, "bf16", 0.05),
    ("bf16_b8", 128, 64, 8, 3, 70, "bf16", 0.05),
    ("f32_b64", 384, 256, 64, 4, 96, "f32", 0.02),
    ("f32_b16", 192, 128, 16, 2, 50, "f32", 0.05),
]


@pytest.mark.parametrize("name,m,n,b,k,T,dtype,sigma", SMALL_B)
def test_layer_small_block_sizes(name, m, n, b, k, T, dtype, sigma):
    """Block sizes the workloads do not use, against the oracle: bf16 b = 64
    takes the register-staged MFMA products and the b = 64 reductions (one
    launch per side, or the joint launch once the tokens are split), bf16
    b = 16 and 8 and float32 layers take the portable kernels."""
    cfg = I.LayerConfig(name, m, n, b, k, T, dtype, sigma)
    say(f"small b {cfg}")
    d = I.make_inputs(cfg, seed=77, T=T)
    L = _layer(cfg, T)
    _load(L, d)
    L.step(to_dev(d["x"]), to_dev(d["dy"]))
    torch.cuda.synchronize()
    y_ref, _ = O.layer_fwd(d["x64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                           d["perm_R"], b, k)
    g = O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], b, k)
    out = {"y": to_f64(L.y), "dx": to_f64(L.dx), "dG_P": to_f64(L.dG_P), "dG_R": to_f64(L.dG_R),
           "dtheta_P": to_f64(L.dtheta_P), "dtheta_R": to_f64(L.dtheta_R)}
    check_layer(out, dict(g, y=y_ref), TOL[dtype], log=say)
