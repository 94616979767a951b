"""Seeded synthetic inputs for the sparse-linear attention forward.

This module only draws random numbers and lays them out; it holds none of the
attention method's arithmetic (no pooling, scoring, selection or attention).
Both the HIP path (through the tests and bench.py) and the CPU oracle consume
what it produces, so the two always see identical bits.

Workloads (the shapes of the pages' own workloads):

* ``tiny_sla``     B1 H1 N1024 d64, fp32, i.i.d. N(0,1) Q, K, V.
* ``wan13b_sla``   Wan2.1-1.3B-shaped video DiT layer: 12 heads, d128, tokens on a
                   21x30x52 latent grid (32760 tokens, padded to 32768), bf16.
* ``salad``        same tensors as ``wan13b_sla`` plus a per-head gate vector.
* ``nsa_prefill``  N65536, 16 query heads sharing one KV head, d128, bf16, noise
                   plus a per-position low-rank drift.
* ``wan14b_sla``   Wan-14B-shaped layer: 40 heads, 21x45x80 grid (75600 tokens,
                   padded to 75648), bf16.

Video-shaped generator (the pages evaluate on Wan2.1 video DiT attention; its
activations need model weights, so random Fourier features of the normalised
latent coordinates stand in for them): with x = (t/(T-1), h/(H-1), w/(W-1)),
F_m(x) = sqrt(2) cos(2 pi omega_m . x + beta_m), m = 1..32, omega_m ~ N(0, 3^2 I),
beta_m ~ U[0, 2 pi); per head Q = F W_q + 0.3 eps, K = F W_k + 0.3 eps with
W ~ N(0, 1/32) of shape 32 x d and eps ~ N(0, 1); V ~ N(0, 1).  Rows past the
valid length are zero.

Drift generator (NSA-style prefill): X = eps + G(p) U with
G_m(p) = sqrt(2) cos(2 pi 2^m p / N + beta_m), m = 0..7, U ~ N(0, 1/8) of shape 8 x d,
drawn separately for every query head, for K and for V.

All draws use numpy's PCG64 with the stated seed, in the order documented in
each generator, in float32 (float64 for the few frequency/phase parameters),
then are rounded once to bf16 (round-to-nearest-even) for bf16 workloads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int            # padded length, a multiple of 64
    Nv: int           # valid length
    d: int
    dtype: str        # "bf16" or "f32"
    mode: str         # "sla", "salad" or "nsa"
    seed: int
    kh_bp: int = 0    # critical share in basis points (sla, salad)
    kl_bp: int = 0    # negligible share in basis points (sla)
    causal: bool = False
    n_sel: int = 0    # selected blocks per query block (nsa)
    window: int = 0   # sliding window in tokens (nsa)
    grid: Optional[Tuple[int, int, int]] = None   # (T, H, W) latent grid (video)
    gate_seed: Optional[int] = None               # salad gate vector seed
    generator: str = "iid"                        # "iid", "video" or "drift"

    @property
    def nb(self) -> int:
        return self.N // BLOCK

    def dense_flops(self) -> float:
        """Dense-equivalent attention FLOPs: 4 B Hq Nv^2 d, halved when causal."""
        f = 4.0 * self.B * self.Hq * float(self.Nv) ** 2 * self.d
        return f / 2.0 if self.causal else f


def _pad_to_block(n: int) -> int:
    return ((n + BLOCK - 1) // BLOCK) * BLOCK


def video_workload(name, grid, heads, seed, mode="sla", kh_bp=500, kl_bp=8500, gate_seed=None, d=128):
    Nv = grid[0] * grid[1] * grid[2]
    return Workload(name=name, B=1, Hq=heads, Hkv=heads, N=_pad_to_block(Nv), Nv=Nv, d=d,
                    dtype="bf16", mode=mode, seed=seed, kh_bp=kh_bp, kl_bp=kl_bp, grid=grid,
                    gate_seed=gate_seed, generator="video")


WORKLOADS = {
    "tiny_sla": Workload(name="tiny_sla", B=1, Hq=1, Hkv=1, N=1024, Nv=1024, d=64, dtype="f32",
                         mode="sla", seed=1, kh_bp=2500, kl_bp=5000, generator="iid"),
    "wan13b_sla": video_workload("wan13b_sla", (21, 30, 52), 12, seed=2),
    "salad": video_workload("salad", (21, 30, 52), 12, seed=2, mode="salad", kh_bp=1000, kl_bp=0,
                            gate_seed=3),
    "nsa_prefill": Workload(name="nsa_prefill", B=1, Hq=16, Hkv=1, N=65536, Nv=65536, d=128,
                            dtype="bf16", mode="nsa", seed=4, causal=True, n_sel=16, window=512,
                            generator="drift"),
    "wan14b_sla": video_workload("wan14b_sla", (21, 45, 80), 40, seed=5),
}


def _to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _video_tensors(w: Workload):
    T, Hh, W = w.grid
    rng = np.random.Generator(np.random.PCG64(w.seed))
    omega = rng.normal(0.0, 3.0, size=(32, 3))
    beta = rng.uniform(0.0, 2.0 * math.pi, size=32)
    tt, hh, ww = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    x = np.stack([tt.ravel() / max(T - 1, 1), hh.ravel() / max(Hh - 1, 1),
                  ww.ravel() / max(W - 1, 1)], axis=1)                 # row-major (t, h, w)
    F = (math.sqrt(2.0) * np.cos(2.0 * math.pi * (x @ omega.T) + beta)).astype(np.float32)
    shape = (w.B, w.Hq, w.N, w.d)
    tq = torch.zeros(shape, dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    tk, tv = torch.zeros_like(tq), torch.zeros_like(tq)
    sd = math.sqrt(1.0 / 32.0)
    for b in range(w.B):
        for h in range(w.Hq):
            Wq = rng.normal(0.0, sd, size=(32, w.d)).astype(np.float32)
            Wk = rng.normal(0.0, sd, size=(32, w.d)).astype(np.float32)
            eq = rng.standard_normal((w.Nv, w.d), dtype=np.float32)
            ek = rng.standard_normal((w.Nv, w.d), dtype=np.float32)
            vv = rng.standard_normal((w.Nv, w.d), dtype=np.float32)
            tq[b, h, :w.Nv] = _to_dtype(F @ Wq + np.float32(0.3) * eq, w.dtype)
            tk[b, h, :w.Nv] = _to_dtype(F @ Wk + np.float32(0.3) * ek, w.dtype)
            tv[b, h, :w.Nv] = _to_dtype(vv, w.dtype)
    return tq, tk, tv


def _drift_tensor(rng, heads, w: Workload):
    out = torch.zeros((w.B, heads, w.N, w.d), dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    p = np.arange(w.Nv, dtype=np.float64)
    for b in range(w.B):
        for h in range(heads):
            beta = rng.uniform(0.0, 2.0 * math.pi, size=8)
            U = rng.normal(0.0, math.sqrt(1.0 / 8.0), size=(8, w.d)).astype(np.float32)
            eps = rng.standard_normal((w.Nv, w.d), dtype=np.float32)
            G = (math.sqrt(2.0) * np.cos(2.0 * math.pi * np.outer(p, 2.0 ** np.arange(8)) / w.N
                                         + beta)).astype(np.float32)
            out[b, h, :w.Nv] = _to_dtype(eps + G @ U, w.dtype)
    return out


def _drift_tensors(w: Workload):
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = _drift_tensor(rng, w.Hq, w)
    k = _drift_tensor(rng, w.Hkv, w)
    v = _drift_tensor(rng, w.Hkv, w)
    return q, k, v


def _iid_tensors(w: Workload):
    rng = np.random.Generator(np.random.PCG64(w.seed))
    tensors = []
    for heads in (w.Hq, w.Hkv, w.Hkv):
        t = torch.zeros((w.B, heads, w.N, w.d), dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32)
        a = rng.standard_normal((w.B, heads, w.Nv, w.d), dtype=np.float32)
        t[:, :, :w.Nv] = _to_dtype(a, w.dtype)
        tensors.append(t)
    return tuple(tensors)


def gate_vector(w: Workload) -> torch.Tensor:
    """Per-head gate weights w_g ~ N(0, 1/d), shape [Hq, d], float32."""
    rng = np.random.Generator(np.random.PCG64(w.gate_seed if w.gate_seed is not None else w.seed + 1))
    return torch.from_numpy(rng.normal(0.0, math.sqrt(1.0 / w.d), size=(w.Hq, w.d)).astype(np.float32))


def make_inputs(w: Workload):
    """Return (q, k, v, w_gate_or_None) as CPU torch tensors in layout [B, H, N, d]."""
    if w.generator == "video":
        q, k, v = _video_tensors(w)
    elif w.generator == "drift":
        q, k, v = _drift_tensors(w)
    else:
        q, k, v = _iid_tensors(w)
    wg = gate_vector(w) if w.mode == "salad" else None
    return q, k, v, wg


def scaled(w: Workload, name: str, **changes) -> Workload:
    """A smaller variant of a workload (for parity at sizes the oracle finishes quickly)."""
    if "grid" in changes and "Nv" not in changes:
        g = changes["grid"]
        nv = g[0] * g[1] * g[2]
        changes["Nv"] = nv
        changes["N"] = _pad_to_block(nv)
    return dataclasses.replace(w, name=name, **changes)
