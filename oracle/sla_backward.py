"""CPU oracle for the gradients of the SLA forward (dQ, dK, dV).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  The product path never calls it.

The pages train SLA by fine-tuning (SLA analysis page for arXiv 2509.24006: the
Proj layer and the linear path need fine-tuning), so the layer needs its
backward; the pages print no backward, so this oracle takes the plainest one:
the exact gradient of the forward the pages define, through both branches,
obtained by automatic differentiation of that forward written out in float64
torch operations.

Readings (also listed in the design notes):
  * the block map is a piecewise-constant function of Q and K (it changes only
    where two pooled scores swap order), so it is held fixed: the gradient flows
    through the critical softmax branch and the marginal linear branch only,
    never through pooling, scores or classification;
  * Proj (when given) is part of the forward, so dQ, dK, dV see it, and its
    weight and bias get their own gradients (summed over every valid row of the
    heads that share them);
  * padded positions (>= n_valid) get zero gradient;
  * smooth-K (when on) shifts the keys of the linear branch by their mean over
    the valid rows inside the differentiated forward, so dK carries the
    gradient through that mean as well.

The forward here restates the numpy oracle's steps with masks: a query row
attends with one softmax to the keys of its critical blocks (s < n_valid), and
gets the linear term phi(q)^T (sum of H_j) / (phi(q) . sum of z_j) over its
marginal blocks j, with H_j = phi(K_j)^T V_j and z_j = sum phi(K_j) over the
valid rows of block j.  The SALAD variant replaces the marginal term by the gated
linear attention over all valid keys (and w_gate gets its gradient); the NSA
variant attends causally to its selected blocks and window, with the query heads
of a GQA group sharing one selection and one KV head (so dK and dV sum over the
group's heads).  Its output is checked against the numpy oracle, and its
gradients against central finite differences of the numpy oracle.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

BLOCK = 64


def _phi(x: torch.Tensor) -> torch.Tensor:
    """elu + 1, written by cases (x + 1 above zero, exp(x) otherwise)."""
    return torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))


def forward_torch(Q, K, V, maps: Dict, n_valid: int, scale: float, proj_w=None, proj_b=None,
                  blocks: Optional[set] = None, smooth_k: bool = False, mode: str = "sla", w_gate=None,
                  window: int = 0, group_map: bool = False) -> torch.Tensor:
    """Layer output [B, Hq, N, d] for a fixed block map, in float64 torch ops (differentiable).

    Q: float64 [B, Hq, N, d]; K, V: float64 [B, Hkv, N, d], query head h reads KV head
    h // (Hq / Hkv) (GQA when Hkv < Hq).
    maps[(b, m, i)]: dict with the ascending lists "crit" and "marg" (and, causal, "flags") of query
    block i of map head m: m = h // (Hq / Hkv) when group_map (the heads of a GQA group share one
    selection), else m = h.
    mode: "sla"   critical softmax + marginal linear (+ Proj);
          "salad" critical softmax + sigmoid(q . w_gate[h]) times linear attention over all valid
                  keys (SALAD page, method framework: a parallel linear branch mixed by an
                  input-dependent gate);
          "nsa"   causal: query row t attends to key s of a listed block iff s < n_valid, s <= t,
                  and (the block is a selected one, flag bit 0, or t - s < window); no linear branch.
    blocks: if given, only these (b, h, i) query blocks (h a query head) are computed, the others
    output 0 (so a loss over them is exact for every input row it depends on).
    """
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    nb = N // BLOCK
    tok = torch.arange(N)
    valid_k = tok < n_valid
    rows = []
    for b in range(B):
        heads = []
        for h in range(Hq):
            if blocks is not None and not any((b, h, i) in blocks for i in range(nb)):
                heads.append(torch.zeros_like(Q[b, h]))
                continue
            g = h // G
            mh = g if group_map else h
            q, k, v = Q[b, h], K[b, g], V[b, g]
            kl = k - k[:n_valid].mean(dim=0) if smooth_k else k   # keys of the linear branch
            pk = _phi(kl) * valid_k[:, None]                      # padded keys contribute nothing
            if mode == "salad":
                H_all = pk.T @ v                                  # over all valid keys, [d, d]
                z_all = pk.sum(dim=0)
            blocks_out = []
            for i in range(nb):
                qi = q[BLOCK * i:BLOCK * (i + 1)]
                if blocks is not None and (b, h, i) not in blocks:
                    blocks_out.append(torch.zeros_like(qi))
                    continue
                m = maps[(b, mh, i)]
                # sparse branch: one softmax over the allowed keys of the listed blocks
                if m["crit"]:
                    keys = torch.cat([torch.arange(BLOCK * j, BLOCK * (j + 1)) for j in m["crit"]])
                    allowed = (keys < n_valid)[None, :].expand(BLOCK, -1).clone()
                    if mode == "nsa":
                        t_ = BLOCK * i + torch.arange(BLOCK)[:, None]
                        s_ = keys[None, :]
                        sel = torch.cat([torch.full((BLOCK,), (f & 1) == 1) for f in m["flags"]])[None, :]
                        allowed &= (s_ <= t_) & (sel | (t_ - s_ < window))
                    has = allowed.any(dim=1)
                    x = (qi @ k[keys].T) * scale
                    x = torch.where(allowed, x, torch.full_like(x, -torch.inf))
                    # rows with no allowed key output 0 (their softmax is not formed)
                    xs = torch.where(has[:, None], x, torch.zeros_like(x))
                    p = torch.softmax(xs, dim=1) * allowed
                    o = torch.where(has[:, None], p @ v[keys], torch.zeros_like(qi))
                else:
                    o = torch.zeros_like(qi)
                ol = torch.zeros_like(qi)
                if mode == "sla" and m["marg"]:
                    sel = torch.zeros(N, dtype=torch.bool)
                    for j in m["marg"]:
                        sel[BLOCK * j:BLOCK * (j + 1)] = True
                    Hs = pk[sel].T @ v[sel]                           # sum of H_j, [d, d]
                    zs = pk[sel].sum(dim=0)                           # sum of z_j, [d]
                    pq = _phi(qi)
                    ol = (pq @ Hs) / (pq @ zs)[:, None]
                elif mode == "salad":
                    pq = _phi(qi)
                    gate = torch.sigmoid(qi @ w_gate[h])
                    ol = gate[:, None] * (pq @ H_all) / (pq @ z_all)[:, None]
                if proj_w is not None:
                    W = proj_w[h] if proj_w.dim() == 3 else proj_w
                    ol = ol @ W.T
                    if proj_b is not None:
                        ol = ol + (proj_b[h] if proj_b.dim() == 2 else proj_b)
                blocks_out.append(o + ol)
            out = torch.cat(blocks_out, dim=0)
            heads.append(out * (tok < n_valid)[:, None])              # padded query rows are 0
        rows.append(torch.stack(heads))
    return torch.stack(rows)


def gradients(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, maps: Dict, n_valid: int,
              scale: float, proj_w=None, proj_b=None, blocks: Optional[set] = None, smooth_k: bool = False,
              with_proj_grads: bool = False, mode: str = "sla", w_gate=None, window: int = 0,
              group_map: bool = False):
    """(O, dQ, dK, dV) as float64 numpy arrays: the output and the gradient of sum(dO * O);
    with with_proj_grads also (dW, db) of the Proj weight and bias (db None without a bias);
    in mode "salad" also dw_gate (last).

    With `blocks`, the loss covers only those query blocks (see forward_torch).
    """
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    q, k, v = t(Q), t(K), t(V)
    pw = None if proj_w is None else t(proj_w)
    pb = None if proj_b is None else t(proj_b)
    wg = None if w_gate is None else t(w_gate)
    O = forward_torch(q, k, v, maps, n_valid, scale, pw, pb, blocks, smooth_k, mode, wg, window, group_map)
    O.backward(torch.tensor(np.asarray(dO, dtype=np.float64)))
    out = (O.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy())
    if with_proj_grads:
        out = out + (None if pw is None else pw.grad.numpy(), None if pb is None else pb.grad.numpy())
    if mode == "salad":
        out = out + (wg.grad.numpy(),)
    return out
