"""Independent reference forms used to pin the oracle (CPU only, float64).

Each function here computes a special case of the method in a different way from
the oracle: dense attention through torch's scaled_dot_product_attention, linear
attention in its quadratic kernel-attention form (never through per-block states),
and block classifications by counting ranks (never by sorting).
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

BLOCK = 64


def as_t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def sdpa(q, k, v, scale, mask=None, causal=False):
    """Softmax attention via torch SDPA in float64.  q [..., Lq, d], k, v [..., Lk, d]; mask True = attend."""
    q, k, v = as_t(q), as_t(k), as_t(v)
    m = None if mask is None else torch.as_tensor(mask, dtype=torch.bool)
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=m, is_causal=causal, scale=scale)
    return out.numpy()


def elu1(x):
    """phi = elu + 1 through torch's ELU."""
    return (F.elu(as_t(x)) + 1.0).numpy()


def kernel_linear_attention(q, k, v, mask=None):
    """sum_s sim(q_t, k_s) v_s / sum_s sim(q_t, k_s) with sim = phi(q).phi(k), over masked keys."""
    pq, pk = elu1(q), elu1(k)
    A = pq @ pk.T
    if mask is not None:
        A = np.where(mask, A, 0.0)
    den = A.sum(axis=1)
    out = (A @ np.asarray(v, dtype=np.float64)) / np.where(den == 0, 1.0, den)[:, None]
    return np.where((den == 0)[:, None], 0.0, out)


def beats(a, ja, b, jb):
    """True iff candidate (score a, index ja) ranks above (score b, index jb)."""
    an, bn = math.isnan(a), math.isnan(b)
    if an != bn:
        return bn
    if an and bn:
        return ja < jb
    if a != b:            # -0.0 == +0.0 here
        return a > b
    return ja < jb


def ranks(row):
    """Rank of every candidate = number of candidates that beat it (0 = most important)."""
    row = [float(x) for x in row]
    n = len(row)
    return [sum(1 for jp in range(n) if jp != j and beats(row[jp], jp, row[j], j)) for j in range(n)]


def brute_classes(row, n_h, n_l):
    r = ranks(row)
    nb = len(row)
    crit = [j for j in range(nb) if r[j] < n_h]
    negl = [j for j in range(nb) if r[j] >= nb - n_l]
    marg = [j for j in range(nb) if n_h <= r[j] < nb - n_l]
    return crit, marg, negl


def brute_token_masks(maps_rows, nqb, N, n_valid):
    """Token masks [nqb*64, N] of the critical and marginal blocks of each query block row."""
    crit = np.zeros((N, N), dtype=bool)
    marg = np.zeros((N, N), dtype=bool)
    for i in range(nqb):
        c, m, _ = maps_rows[i]
        for j in c:
            crit[BLOCK * i:BLOCK * (i + 1), BLOCK * j:BLOCK * (j + 1)] = True
        for j in m:
            marg[BLOCK * i:BLOCK * (i + 1), BLOCK * j:BLOCK * (j + 1)] = True
    crit[:, n_valid:] = False
    marg[:, n_valid:] = False
    return crit, marg


def parse_json_scores(vals):
    out = []
    for v in vals:
        if v is None:
            out.append(float("nan"))
        elif v == "-inf":
            out.append(float("-inf"))
        elif v == "-0":
            out.append(-0.0)
        else:
            out.append(float(v))
    return np.asarray(out, dtype=np.float32)
