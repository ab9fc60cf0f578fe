"""Seeded synthetic inputs for the routed-branch forward.

This module only draws random numbers: it holds none of the method's
arithmetic, and both the HIP path's callers and the CPU oracle's callers take
their inputs from it.

The pages train their routers on a text corpus and report latency for a
batch of "4096 inputs" on a model whose layer shapes they do not print.  No
weights or data are available here, so Gaussian parameters stand in for the
trained ones and a clustered token distribution stands in for skewed trained
routing.  Recipe (per tensor, per block of rows, its own torch generator
seeded from numpy's SeedSequence([seed, tensor id, block])):

* x ~ N(0, 1)  (or the clustered mixture below),
* W, V, W_r, W_c ~ N(0, 1/d),
* draws are float32; bf16 workloads round them to nearest-even once.
* clustered x: 32 centres c_k = z_k / |z_k| with z_k ~ N(0, I_d), a uniform
  cluster id per token, and x_t = c_u + (0.1 / sqrt(d)) * eps_t, so the
  noise norm is about 0.1 around unit-norm centres.

Generation runs on the device the caller names; the same seed gives the same
values on the same device type (CPU and GPU generators differ, so CPU-side
checks of GPU-generated inputs copy those inputs back).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

ROWS_PER_BLOCK = 65536
_TID = {"x": 0, "Wr": 1, "Wc": 2, "W": 3, "V": 4, "centres": 5, "cluster": 6, "dy": 7, "Wg": 8, "Wu": 9, "Wd": 10}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    L: int
    d: int
    Nr: int
    Nc: int
    K: int
    B: int
    dtype: str = "bf16"  # "f32" or "bf16"
    x_dist: str = "normal"  # "normal" or "clustered"
    note: str = ""

    @property
    def N(self) -> int:
        return self.Nr * self.Nc

    @property
    def M(self) -> int:
        return self.L * self.K

    @property
    def G(self) -> int:
        return -(-self.N // self.B)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def describe(self) -> dict:
        return dict(workload=self.name, L=self.L, d=self.d, N_r=self.Nr,
                    N_c=self.Nc, N=self.N, K=self.K, B=self.B,
                    dtype=self.dtype, x=self.x_dist)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_L64_N1024_d64_f32", 64, 64, 32, 32, 16, 16, "f32",
                 note="small grid, brute-force top-K feasible"),
        Workload("L4096_N280900_d768", 4096, 768, 530, 530, 64, 64),
        Workload("L4096_N1048576_d1024", 4096, 1024, 1024, 1024, 128, 128),
        Workload("L4096_N1700416_d2048", 4096, 2048, 1304, 1304, 128, 128,
                 note="1.7M atomic experts, 4096 tokens"),
        Workload("skewed_L16384_N1700416_d2048", 16384, 2048, 1304, 1304, 256,
                 256, x_dist="clustered",
                 note="32 token clusters pile tasks onto few experts"),
    ]
}
TINY = "tiny_L64_N1024_d64_f32"
HEADLINE = "L4096_N1700416_d2048"


def _block_seed(seed: int, tensor: str, block: int) -> int:
    s = np.random.SeedSequence([seed, _TID[tensor], block]).generate_state(2)
    return (int(s[0]) << 31) ^ int(s[1])


def _gen(device) -> torch.Generator:
    return torch.Generator(device=device)


def normal_rows(tensor: str, rows: int, cols: int, std: float, seed: int,
                device="cpu", out_dtype=torch.float32) -> torch.Tensor:
    """rows x cols draws of N(0, std^2), blockwise-seeded, cast once."""
    out = torch.empty((rows, cols), dtype=out_dtype, device=device)
    g = _gen(device)
    for b, r0 in enumerate(range(0, rows, ROWS_PER_BLOCK)):
        r1 = min(rows, r0 + ROWS_PER_BLOCK)
        g.manual_seed(_block_seed(seed, tensor, b))
        blk = torch.randn((r1 - r0, cols), generator=g, device=device,
                          dtype=torch.float32)
        if std != 1.0:
            blk.mul_(std)
        out[r0:r1].copy_(blk)  # round-to-nearest-even for bf16
    return out


def clustered_x(L: int, d: int, seed: int, device="cpu", out_dtype=torch.float32,
                n_clusters: int = 32, noise_norm: float = 0.1) -> torch.Tensor:
    z = normal_rows("centres", n_clusters, d, 1.0, seed, device)
    centres = z / z.norm(dim=1, keepdim=True)
    g = _gen(device)
    g.manual_seed(_block_seed(seed, "cluster", 0))
    u = torch.randint(0, n_clusters, (L,), generator=g, device=device)
    eps = normal_rows("x", L, d, 1.0, seed, device)
    x = centres[u] + (noise_norm / math.sqrt(d)) * eps
    return x.to(out_dtype)


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> dict:
    """x [L,d], Wr [N_r,d], Wc [N_c,d], W [N,d], V [N,d] in w's dtype."""
    dt = w.torch_dtype
    std = 1.0 / math.sqrt(w.d)
    if w.x_dist == "clustered":
        x = clustered_x(w.L, w.d, seed, device, dt)
    else:
        x = normal_rows("x", w.L, w.d, 1.0, seed, device, dt)
    return dict(
        x=x,
        Wr=normal_rows("Wr", w.Nr, w.d, std, seed, device, dt),
        Wc=normal_rows("Wc", w.Nc, w.d, std, seed, device, dt),
        W=normal_rows("W", w.N, w.d, std, seed, device, dt),
        V=normal_rows("V", w.N, w.d, std, seed, device, dt),
    )


def mlp_hidden(d: int) -> int:
    """Hidden width of the shared SwiGLU MLP: 8d/3 rounded up to 128."""
    return -(-8 * d // (3 * 128)) * 128


def mlp_weights(L_unused, d: int, F: int, dtype: str = "bf16", seed: int = 0,
                device="cpu") -> dict:
    """Wg, Wu [F, d] ~ N(0, 1/d) and Wd [d, F] ~ N(0, 1/F), in the given dtype."""
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    return dict(
        Wg=normal_rows("Wg", F, d, 1.0 / math.sqrt(d), seed, device, dt),
        Wu=normal_rows("Wu", F, d, 1.0 / math.sqrt(d), seed, device, dt),
        Wd=normal_rows("Wd", d, F, 1.0 / math.sqrt(F), seed, device, dt),
    )


def upstream_grad(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """dy [L, d] fp32 ~ N(0, 1/d): the gradient arriving at the branch output
    (a unit-variance loss gradient spread over d outputs)."""
    return normal_rows("dy", w.L, w.d, 1.0 / math.sqrt(w.d), seed, device)


def make_case(L, d, Nr, Nc, K, B, dtype="f32", seed=0, device="cpu",
              x_dist="normal") -> tuple:
    """An ad-hoc workload (tests of ragged sizes and edge cases)."""
    w = Workload(f"case_L{L}_d{d}_{Nr}x{Nc}_K{K}_B{B}_{dtype}", L, d, Nr, Nc,
                 K, B, dtype, x_dist)
    return w, make_inputs(w, seed, device)


def quantised_logit_case(L, d, Nr, Nc, seed=0, levels=4):
    """Inputs whose logits take few distinct values, to force exact ties.

    x is one-hot per token and the router rows hold small integers, so every
    logit is an integer in [0, levels) and many grid sums tie exactly.
    Float64 numpy arrays (for the CPU oracle's tie tests).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    x = np.zeros((L, d))
    x[np.arange(L), rng.integers(0, d, L)] = 1.0
    Wr = rng.integers(0, levels, (Nr, d)).astype(np.float64)
    Wc = rng.integers(0, levels, (Nc, d)).astype(np.float64)
    return x, Wr, Wc
