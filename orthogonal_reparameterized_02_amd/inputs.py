"""Seeded synthetic inputs for the POET-X layer, shared by the tests, the bench
and the smoke check.

This module only draws random numbers and rounds them to their storage type;
it holds none of the layer's arithmetic.  Both the HIP path and the float64
oracle consume exactly the arrays produced here.

Workloads (shapes of the Llama layers the POET-X pages train; the pages train
on C4 text at sequence length 1024, and Gaussian activations of the same
shape stand in for it):

  name      m      n     b   k     T   storage  theta sigma
  probe     256    256   32  4    64   fp32     0.02
  mid       2048   2048  128 4  4096   bf16     0.01
  square    4096   4096  256 4  8192   bf16     0.01   (headline)
  mlp_up    14336  4096  256 4 16384   bf16     0.01
  mlp13b    13824  5120  512 5  8192   bf16     0.005

Distributions: W0 ~ N(0, 1/n) (fixed random weight), x ~ N(0, 1),
dL/dy ~ N(0, 1), theta ~ N(0, sigma^2) in fp32, pi_P / pi_R uniform random
permutations.  Draws are made in float64 from numpy's PCG64 streams spawned
from SeedSequence(seed) in the order W0, theta_P, theta_R, pi_P, pi_R, x, dy,
cast to fp32, then (for bf16 tensors) rounded to bf16 with round-to-nearest-
even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    m: int          # outputs (rows of W0)
    n: int          # inputs (columns of W0)
    b: int          # orthogonal block size
    k: int          # Neumann order (highest power kept)
    T: int          # tokens
    dtype: str      # storage type of x, W0, y, dy, dx and G: "f32" | "bf16"
    sigma: float    # std of the packed skew parameters

    @property
    def n_P(self) -> int:
        return self.n // self.b

    @property
    def n_R(self) -> int:
        return self.m // self.b

    @property
    def tri(self) -> int:
        return self.b * (self.b - 1) // 2


CONFIGS = (
    LayerConfig("probe", 256, 256, 32, 4, 64, "f32", 0.02),
    LayerConfig("mid", 2048, 2048, 128, 4, 4096, "bf16", 0.01),
    LayerConfig("square", 4096, 4096, 256, 4, 8192, "bf16", 0.01),
    LayerConfig("mlp_up", 14336, 4096, 256, 4, 16384, "bf16", 0.01),
    LayerConfig("mlp13b", 13824, 5120, 512, 5, 8192, "bf16", 0.005),
)
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


def bf16_round_bits(a32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16.  Inputs here are finite."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a64: np.ndarray, dtype: str):
    """Return (storage array, exact float64 view of the stored values)."""
    a32 = a64.astype(np.float32)
    if dtype == "f32":
        return a32, a32.astype(np.float64)
    if dtype == "bf16":
        bits = bf16_round_bits(a32)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(dtype)


def make_inputs(cfg: LayerConfig, seed: int = 0, T: int | None = None,
                want=("W0", "theta_P", "theta_R", "perm_P", "perm_R", "x", "dy"),
                f64: bool = True) -> Dict[str, np.ndarray]:
    """Draw the layer's inputs for `cfg`.

    Returns storage arrays under their names (uint16 bit patterns for bf16,
    float32 otherwise; theta float32; permutations int32) and, when `f64`,
    the exact float64 values of the stored tensors under "<name>64".
    `T` overrides the token count; the rows of x and dy are drawn in order,
    so a smaller T yields the leading rows of the full-size draw.
    """
    T = cfg.T if T is None else T
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(7)
    names = ("W0", "theta_P", "theta_R", "perm_P", "perm_R", "x", "dy")
    rng = {nm: np.random.Generator(np.random.PCG64(kid)) for nm, kid in zip(names, kids)}
    out: Dict[str, np.ndarray] = {}
    if "W0" in want:
        w = rng["W0"].standard_normal((cfg.m, cfg.n)) * (1.0 / np.sqrt(cfg.n))
        out["W0"], w64 = _store(w, cfg.dtype)
        if f64:
            out["W064"] = w64
        del w
    for nm, nblk in (("theta_P", cfg.n_P), ("theta_R", cfg.n_R)):
        if nm in want:
            th = (rng[nm].standard_normal((nblk, cfg.tri)) * cfg.sigma).astype(np.float32)
            out[nm] = th
            if f64:
                out[nm + "64"] = th.astype(np.float64)
    if "perm_P" in want:
        out["perm_P"] = rng["perm_P"].permutation(cfg.n).astype(np.int32)
    if "perm_R" in want:
        out["perm_R"] = rng["perm_R"].permutation(cfg.m).astype(np.int32)
    for nm, width in (("x", cfg.n), ("dy", cfg.m)):
        if nm in want:
            a = rng[nm].standard_normal((T, width))
            out[nm], a64 = _store(a, cfg.dtype)
            if f64:
                out[nm + "64"] = a64
            del a
    return out


def to_f64(storage: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a storage array (bf16 bit patterns or float32)."""
    if dtype == "bf16" or storage.dtype == np.uint16:
        return bf16_bits_to_f32(storage).astype(np.float64)
    return storage.astype(np.float64)


def quantize_rows_int8(w: np.ndarray):
    """An INT8 base weight as it would arrive for POET-XQ: symmetric per-row
    quantization, s[i] = max_j |w[i, j]| / 127 (float32) and
    q = round(w / s) clipped to [-127, 127] (int8).  The weight it represents
    is s[:, None] * q, exactly representable in float64."""
    w = np.asarray(w, dtype=np.float64)
    s = (np.abs(w).max(axis=1) / 127.0).astype(np.float32)
    s[s == 0] = 1.0
    q = np.clip(np.rint(w / s.astype(np.float64)[:, None]), -127, 127).astype(np.int8)
    return q, s

