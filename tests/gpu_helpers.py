"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI binding and the
CPU oracle on the same seeded inputs, and compare.  Inputs flow oracle -> GPU only (the
oracle's block maps may be uploaded to drive sla_attn_fwd); nothing computed on the GPU is
ever fed to the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_oracle as orc
from workloads import BLOCK, make_inputs

REL_L2 = 1e-2      # output tolerance, bf16 I/O with fp32 accumulation
MAX_ABS = 3e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def to_dev(a, dtype=torch.int32):
    return torch.as_tensor(np.asarray(a)).to(device="cuda", dtype=dtype)


def oracle_for(w, q, k, v, wg):
    return orc.Forward(host(q), host(k), host(v), n_valid=w.Nv, mode=w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp,
                       n_sel=w.n_sel, window=w.window, w_gate=None if wg is None else wg.numpy())


def layer_for(w, q, k, v, wg):
    return sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp,
                          n_sel=w.n_sel, window=w.window, w_gate=wg)


def make_case(w, proj_w=None, proj_b=None, smooth_k=False, training=False):
    """Seeded inputs of workload w, the oracle Forward and the library layer, both with the given
    Proj weights (float32 numpy) and smooth-K setting (training: the layer keeps what its backward
    needs)."""
    q, k, v, wg = make_inputs(w)
    f = orc.Forward(host(q), host(k), host(v), n_valid=w.Nv, mode=w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp,
                    n_sel=w.n_sel, window=w.window, w_gate=None if wg is None else wg.numpy(),
                    proj_w=proj_w, proj_b=proj_b, smooth_k=smooth_k)
    t = lambda x: None if x is None else torch.as_tensor(x)
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp,
                           n_sel=w.n_sel, window=w.window, w_gate=wg, proj_w=t(proj_w), proj_b=t(proj_b),
                           smooth_k=smooth_k, training=training)
    return q, k, v, wg, f, layer


def gpu_map_rows(maps, rows_idx):
    """Per-row (crit list, flags, marg list, counts) for the given flat row indices."""
    cr = maps["crit_rowptr"].cpu().numpy()
    ci = maps["crit_idx"].cpu().numpy()
    cf = maps["crit_flags"].cpu().numpy()
    mr = maps["marg_rowptr"].cpu().numpy() if "marg_rowptr" in maps else None
    mi = maps["marg_idx"].cpu().numpy() if "marg_idx" in maps else None
    rc = maps["row_counts"].cpu().numpy()
    out = {}
    for r in rows_idx:
        crit = ci[cr[r]:cr[r + 1]].tolist()
        flags = cf[cr[r]:cr[r + 1]].tolist()
        marg = mi[mr[r]:mr[r + 1]].tolist() if mr is not None else None
        out[r] = (crit, flags, marg, tuple(rc[r].tolist()))
    return out


def compare_outputs(o_gpu: np.ndarray, o_ref: np.ndarray, what: str):
    """rel-L2 over all compared rows and max-abs, the stated output tolerance."""
    diff = o_gpu.astype(np.float64) - o_ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(o_ref), 1e-30)
    mx = np.abs(diff).max() if diff.size else 0.0
    say(f"  {what}: rel-L2 {rel:.3e}, max-abs {mx:.3e}")
    assert rel <= REL_L2, f"{what}: rel-L2 {rel} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max-abs {mx} > {MAX_ABS}"
    return rel, mx


def oracle_csr(f: orc.Forward):
    """The oracle's own block map of every row as device CSR tensors (oracle -> GPU input)."""
    Hs = f.Hkv if f.group_sum else f.Hq
    maps = {}
    for b in range(f.B):
        for h in range(Hs):
            for i in range(f.nb):
                maps[(b, h, i)] = f.map_row(b, h, i)
    csr = orc.to_csr(maps, f.B, Hs, f.nb)
    csr["marg_bits"] = marg_bits_of(maps, f.B, Hs, f.nb, f.nb)
    # index arrays get at least one element (a device pointer is required even for empty lists)
    pad = lambda v: v if np.asarray(v).size else np.zeros(1, np.asarray(v).dtype)
    dev = {k: to_dev(pad(v), torch.uint8 if k == "crit_flags" else torch.int32) for k, v in csr.items()}
    return dev, maps


def marg_bits_of(maps, B, Hs, nqb, nkb):
    """Bit masks of the marginal lists: block j is bit j % 32 of word j / 32 (int32 view)."""
    nw = (nkb + 31) // 32
    bits = np.zeros((B * Hs * nqb, nw), dtype=np.uint32)
    r = 0
    for b in range(B):
        for h in range(Hs):
            for i in range(nqb):
                for j in maps[(b, h, i)]["marg"]:
                    bits[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
                r += 1
    return bits.view(np.int32)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)
