"""CPU oracle for the sparse-linear hybrid attention forward (SLA, SALAD, NSA-selected).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  The product path (the
block_sparse_linear_mean_amd package and its HIP library) never calls it, and
this module imports nothing from the product path.

It is a plain, slow, step-by-step float64 implementation of what the method
computes, in the order the pages describe it:

  1. predict:  mean-pool Q and K over 64-token blocks, score the pooled blocks,
     softmax each score row (the prediction step of SpargeAttn / SLA:
     "2025稀疏注意力架构综述", section 11 "SpargeAttn", prediction formulas;
     the SLA analysis page for arXiv 2509.24006, critique of the mean-pooled
     compressed prediction that turns N x N into an (N/b)^2 classification);
  2. classify: per query-block row, top k_h% key blocks are critical, bottom k_l%
     negligible, the rest marginal (SLA analysis page, comparison with
     LongCat-Video BSA and with Kimi Linear: three classes per Q-K block pair;
     "2025稀疏注意力架构综述", section 10 "SLA", core idea);
  3. execute:  critical pairs get exact softmax attention, marginal pairs get
     linear attention with phi = elu + 1 through per-key-block states
     H_j = phi(K_j)^T V_j and z_j = sum phi(K_j), negligible pairs are skipped
     (SLA analysis page: FlashAttn + linear attention per block pair, the
     marginal cost is O(N d^2));
  4. combine:  O = O^s + Proj(O^l) (SLA analysis page, the zero-initialised Proj
     remark).  Proj is the identity unless a weight is given; a given Proj is a
     linear layer on each output row, x W^T + b.

Smooth-K (SLA analysis page, the remark that the open-source code zero-means K,
a step the paper does not mention): optionally the keys of the linear branch are
replaced by K - mean(K), the mean over the valid tokens of each (batch, KV head).

Variants: SALAD adds a linear branch over all keys in parallel with the sparse
branch and mixes it with an input-dependent gate (SALAD page, method
framework); the NSA-style selected branch picks 16 blocks of 64 keys per query
block plus a 512-token sliding window under a causal mask, with the query heads
of a GQA group sharing one selection ("Sparse Attention 方法综述", section 2 NSA,
key-parameter table; "2025稀疏注意力架构综述", section 1 GQA and section 2 NSA
operator design).

Precision.  All arithmetic is float64.  Two values are stored at float32 because
that is the precision the library's boundary stores them in, and the block
classification is decided on them: the pooled vectors (the exact block mean,
rounded once to float32) and the pooled scores (scale * q_pool . k_pool in
float64 from the float32 pooled vectors, rounded once to float32).  The
classification compares those float32 scores.

Readings where the pages are silent (each also listed in the design notes):
  * scale = 1/sqrt(d) rounded to float32, for pooled and exact scores alike;
  * ranking uses the scores, not their softmax (same order, softmax is monotone);
  * counts: n_h = ceil(kh_bp * nb / 10000) (0 iff kh_bp = 0), n_l = min(floor(kl_bp * nb / 10000), nb - n_h);
  * one total order per row: score descending, then block index ascending;
    -0.0 equals +0.0; NaN ranks below everything;
  * CSR lists are in ascending block order;
  * keys and queries at positions >= n_valid are padding: excluded from the pooled
    means, from both branches, and padded query rows output 0;
  * phi(x) = x + 1 for x > 0, exp(x) otherwise; no epsilon in the linear
    denominator; an empty marginal set gives a zero linear term;
  * SALAD gate = sigmoid(q_t . w_g) per token from the raw query row; its linear
    branch covers all valid keys; nothing is negligible;
  * NSA: group score = scale * (sum over the group's heads of q_pool) . k_pool,
    candidates j <= i, selected = top min(n_sel, i+1), window = key s with
    0 <= t - s < window, one softmax over (selected or window) and causal keys.
  * Proj: weight W [d, d] (one for all heads) or [Hq, d, d] (one per head), bias
    b [d] or [Hq, d] or none; applied to O^l of every valid row of an SLA output,
    also where the row has no marginal block (O^l = 0 there, so the row gets b);
  * smooth-K shifts the keys of the linear branch only (the key states H_j, z_j).
    The softmax branch and the pooled ranking are unchanged by it in exact
    arithmetic: subtracting one vector from every key adds the same amount to
    every logit of a query row (and to every pooled score of a row).
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

BLOCK = 64
F64 = np.float64
F32 = np.float32


# ----------------------------------------------------------------------------- helpers

def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32, returned as a Python float."""
    return float(np.float32(1.0 / math.sqrt(d)))


def block_counts(nb: int, kh_bp: int, kl_bp: int) -> Tuple[int, int]:
    """Number of critical and negligible key blocks per row for nb candidates.

    The pages give only percentages (k_h%, k_l%); a fixed-budget top-k keeps the
    same number per row ("深度调研：面向长上下文的次二次稀疏注意力", reading notes on
    fixed-budget top-k).  Reading: integer basis points, critical rounded up,
    negligible rounded down, so at least k_h% is exact and at most k_l% dropped.
    """
    n_h = 0 if kh_bp <= 0 else min(nb, -(-kh_bp * nb // 10000))
    n_l = min(max(kl_bp, 0) * nb // 10000, nb - n_h)
    return n_h, n_l


def phi(x: np.ndarray) -> np.ndarray:
    """elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=F64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def window_blocks(i: int, window: int) -> List[int]:
    """Key blocks that hold a key s with 0 <= t - s < window for some t in query block i."""
    if window <= 0:
        return []
    reach = (window + BLOCK - 2) // BLOCK
    return list(range(max(0, i - reach), i + 1))


# ----------------------------------------------------------------------------- step 1: predict

def pool_block(X_head: np.ndarray, i: int, n_valid: int) -> np.ndarray:
    """Mean of the valid rows of block i of one head ([N, d] array), float64."""
    lo, hi = BLOCK * i, min(BLOCK * (i + 1), n_valid)
    return X_head[lo:hi].astype(F64).sum(axis=0) / float(hi - lo)


def pool(X: np.ndarray, n_valid: int) -> np.ndarray:
    """Block means of X [B, H, N, d] over 64-row blocks, rounded once to float32."""
    B, H, N, d = X.shape
    nb = N // BLOCK
    out = np.empty((B, H, nb, d), dtype=F32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                out[b, h, i] = pool_block(X[b, h], i, n_valid).astype(F32)
    return out


def scores_row(q_vec_f32: np.ndarray, k_pool_head_f32: np.ndarray, scale: float) -> np.ndarray:
    """One row of pooled scores: scale * (q . k_j) for every key block j, float64."""
    return (k_pool_head_f32.astype(F64) @ q_vec_f32.astype(F64)) * float(scale)


def pooled_scores(q_pool: np.ndarray, k_pool: np.ndarray, scale: float,
                  group_sum: bool = False, causal: bool = False) -> np.ndarray:
    """Pooled score matrices, float32 [B, Hs, nb, nb] (Hs = Hkv if group_sum else Hq).

    Without group_sum, query head h is scored against its own KV head h // (Hq/Hkv).
    With group_sum, the pooled queries of a GQA group's heads are summed first (float64)
    and scored against the group's KV head.  Causal: entries j > i are -inf.
    """
    B, Hq, nb, d = q_pool.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    Hs = Hkv if group_sum else Hq
    S = np.empty((B, Hs, nb, nb), dtype=F32)
    for b in range(B):
        for hs in range(Hs):
            if group_sum:
                qh = q_pool[b, hs * G:(hs + 1) * G].astype(F64).sum(axis=0)
                kh = k_pool[b, hs]
            else:
                qh = q_pool[b, hs].astype(F64)
                kh = k_pool[b, hs // G]
            for i in range(nb):
                row = (kh.astype(F64) @ qh[i]) * float(scale)
                S[b, hs, i] = row.astype(F32)
            if causal:
                S[b, hs][np.triu(np.ones((nb, nb), dtype=bool), k=1)] = -np.inf
    return S


def score_probs(S: np.ndarray) -> np.ndarray:
    """Row softmax of the pooled scores over each row's candidates (-inf excluded), float32."""
    X = S.astype(F64)
    m = np.max(X, axis=-1, keepdims=True)
    E = np.exp(X - m)
    return (E / E.sum(axis=-1, keepdims=True)).astype(F32)


# ----------------------------------------------------------------------------- step 2: classify

def rank_order(s_row: np.ndarray) -> np.ndarray:
    """Candidate indices from most to least important: score descending, index ascending.

    -0.0 and +0.0 compare equal (so their order falls to the index); NaN ranks last.
    """
    s = np.asarray(s_row, dtype=F64)
    neg = np.where(np.isnan(s), np.inf, -s)          # NaN after every finite and -inf score
    nan_last = np.isnan(s).astype(np.int8)
    idx = np.arange(len(s))
    return np.lexsort((idx, neg, nan_last))


def classify_row(s_row: np.ndarray, n_h: int, n_l: int):
    """(critical, marginal, negligible) block lists of one non-causal row, each ascending."""
    order = rank_order(s_row)
    nb = len(order)
    crit = sorted(order[:n_h].tolist())
    negl = sorted(order[nb - n_l:].tolist()) if n_l > 0 else []
    marg = sorted(order[n_h:nb - n_l].tolist())
    return crit, marg, negl


def select_row_causal(s_row: np.ndarray, i: int, n_sel: int, window: int):
    """NSA-style row i: top min(n_sel, i+1) of the causal candidates j <= i, united with the
    window blocks.  Returns (blocks ascending, flags, negligible) with flag bit 0 = selected,
    bit 1 = window block."""
    cand = np.asarray(s_row[: i + 1])
    order = rank_order(cand)
    sel = set(order[: min(n_sel, i + 1)].tolist())
    win = set(window_blocks(i, window))
    blocks = sorted(sel | win)
    flags = [(1 if j in sel else 0) | (2 if j in win else 0) for j in blocks]
    negl = sorted(set(range(i + 1)) - set(blocks))
    return blocks, flags, negl


def block_map_rows(S: np.ndarray, rows: Iterable[Tuple[int, int, int]], *, n_h: int = 0, n_l: int = 0,
                   causal: bool = False, n_sel: int = 0, window: int = 0) -> Dict:
    """Block map for the given (b, hs, i) rows of score matrices S [B, Hs, nqb, nkb]."""
    out = {}
    for (b, hs, i) in rows:
        row = S[b, hs, i]
        if causal:
            blocks, flags, negl = select_row_causal(row, i, n_sel, window)
            out[(b, hs, i)] = dict(crit=blocks, flags=flags, marg=[], negl=negl)
        else:
            crit, marg, negl = classify_row(row, n_h, n_l)
            out[(b, hs, i)] = dict(crit=crit, flags=[1] * len(crit), marg=marg, negl=negl)
    return out


def block_map(S: np.ndarray, **kw) -> Dict:
    """Block map of every row of S [B, Hs, nqb, nkb] (see block_map_rows)."""
    B, Hs, nqb, _ = S.shape
    rows = [(b, h, i) for b in range(B) for h in range(Hs) for i in range(nqb)]
    return block_map_rows(S, rows, **kw)


def to_csr(maps: Dict, B: int, Hs: int, nqb: int):
    """Flatten per-row lists into CSR arrays (rows ordered b, hs, i)."""
    crit_ptr, marg_ptr, crit_idx, marg_idx, flags, counts = [0], [0], [], [], [], []
    for b in range(B):
        for h in range(Hs):
            for i in range(nqb):
                m = maps[(b, h, i)]
                crit_idx += m["crit"]
                flags += m["flags"]
                marg_idx += m["marg"]
                crit_ptr.append(len(crit_idx))
                marg_ptr.append(len(marg_idx))
                counts.append((len(m["crit"]), len(m["marg"]), len(m["negl"])))
    as32 = lambda a: np.asarray(a, dtype=np.int32)
    return dict(crit_rowptr=as32(crit_ptr), crit_idx=as32(crit_idx), crit_flags=np.asarray(flags, np.uint8),
                marg_rowptr=as32(marg_ptr), marg_idx=as32(marg_idx), row_counts=as32(counts).reshape(-1, 3))


# ----------------------------------------------------------------------------- step 3: execute

def key_mean(K_head: np.ndarray, n_valid: int) -> np.ndarray:
    """Smooth-K shift of one head: the mean over its valid key rows (float64, [d])."""
    return K_head[:n_valid].astype(F64).mean(axis=0)


def kv_state(K_head: np.ndarray, V_head: np.ndarray, j: int, n_valid: int, shift=None):
    """H_j = phi(K_j)^T V_j (d x d) and z_j = sum_s phi(K_j[s]) over the valid rows of key block j.

    With `shift` (smooth-K) the keys are K_j - shift before phi.
    """
    lo, hi = BLOCK * j, min(BLOCK * (j + 1), n_valid)
    Kj = K_head[lo:hi].astype(F64)
    if shift is not None:
        Kj = Kj - shift
    pk = phi(Kj)
    return pk.T @ V_head[lo:hi].astype(F64), pk.sum(axis=0)


def kv_states(K: np.ndarray, V: np.ndarray, n_valid: int, smooth_k: bool = False):
    """All per-block states: H [B, Hkv, nb, d, d], z [B, Hkv, nb, d], float64."""
    B, Hkv, N, d = K.shape
    nb = N // BLOCK
    H = np.zeros((B, Hkv, nb, d, d), dtype=F64)
    z = np.zeros((B, Hkv, nb, d), dtype=F64)
    for b in range(B):
        for h in range(Hkv):
            shift = key_mean(K[b, h], n_valid) if smooth_k else None
            for j in range(nb):
                if BLOCK * j < n_valid:
                    H[b, h, j], z[b, h, j] = kv_state(K[b, h], V[b, h], j, n_valid, shift)
    return H, z


def sparse_block(Qi: np.ndarray, t0: int, K_head: np.ndarray, V_head: np.ndarray, blocks: List[int],
                 flags: List[int], n_valid: int, scale: float, causal: bool, window: int) -> np.ndarray:
    """Exact softmax attention of query rows t0..t0+len(Qi)-1 over the allowed keys of `blocks`.

    Allowed keys: s < n_valid in a listed block; when causal also s <= t and (the block is a
    selected one or t - s < window).  A row with no allowed key gets 0.
    """
    nq, d = Qi.shape
    if not blocks:
        return np.zeros((nq, d), dtype=F64)
    keys = np.concatenate([np.arange(BLOCK * j, BLOCK * (j + 1)) for j in blocks])
    kflag = np.concatenate([np.full(BLOCK, f) for f in flags])
    t = t0 + np.arange(nq)[:, None]
    s = keys[None, :]
    allowed = np.broadcast_to(s < n_valid, (nq, len(keys))).copy()
    if causal:
        allowed &= (s <= t) & (((kflag[None, :] & 1) == 1) | (t - s < window))
    X = (Qi.astype(F64) @ K_head[keys].astype(F64).T) * float(scale)
    X = np.where(allowed, X, -np.inf)
    has = allowed.any(axis=1)
    m = np.where(has, X.max(axis=1), 0.0)
    P = np.where(allowed, np.exp(X - m[:, None]), 0.0)
    l = P.sum(axis=1)
    O = P @ V_head[keys].astype(F64)
    return np.where(has[:, None], O / np.where(has, l, 1.0)[:, None], 0.0)


def linear_block(Qi: np.ndarray, Hsum: np.ndarray, zsum: np.ndarray) -> np.ndarray:
    """phi(q)^T Hsum / (phi(q) . zsum) for each query row."""
    pq = phi(Qi)
    return (pq @ Hsum) / (pq @ zsum)[:, None]


def project(O_lin: np.ndarray, W: np.ndarray, bias=None) -> np.ndarray:
    """The learned projection of the linear branch on each row: O_lin W^T (+ bias)."""
    out = O_lin @ np.asarray(W, dtype=F64).T
    return out if bias is None else out + np.asarray(bias, dtype=F64)


def sigmoid(x):
    """1 / (1 + exp(-x)); exp overflow for very negative x correctly gives 0."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=F64)))


# ----------------------------------------------------------------------------- full forward

class Forward:
    """Step-by-step forward for one problem; rows are computed on request and cached per head.

    mode: "sla" (critical + marginal linear + skip), "salad" (top blocks + gated linear over all
    keys) or "nsa" (causal selected + window, maps shared by a GQA group, no linear branch).
    """

    def __init__(self, Q, K, V, *, n_valid: int, mode: str, kh_bp: int = 0, kl_bp: int = 0,
                 n_sel: int = 0, window: int = 0, w_gate=None, scale: Optional[float] = None,
                 proj_w=None, proj_b=None, smooth_k: bool = False):
        self.Q, self.K, self.V = Q, K, V
        self.B, self.Hq, self.N, self.d = Q.shape
        self.Hkv = K.shape[1]
        self.G = self.Hq // self.Hkv
        self.nb = self.N // BLOCK
        self.n_valid = n_valid
        self.mode = mode
        self.causal = mode == "nsa"
        self.group_sum = mode == "nsa"
        self.n_sel, self.window = n_sel, window
        self.scale = default_scale(self.d) if scale is None else float(scale)
        self.w_gate = None if w_gate is None else np.asarray(w_gate, dtype=F64)
        self.proj_w = None if proj_w is None else np.asarray(proj_w, dtype=F64)
        self.proj_b = None if proj_b is None else np.asarray(proj_b, dtype=F64)
        if self.proj_w is None and self.proj_b is not None:
            raise ValueError("a Proj bias needs a Proj weight")
        if self.proj_w is not None and mode != "sla":
            raise ValueError("Proj applies to the SLA linear branch")
        self.smooth_k = smooth_k
        if mode == "sla":
            self.n_h, self.n_l = block_counts(self.nb, kh_bp, kl_bp)
        elif mode == "salad":
            self.n_h, self.n_l = block_counts(self.nb, kh_bp, 0)
        else:
            self.n_h, self.n_l = 0, 0
        self._kpool: Dict = {}
        self._H: Dict = {}
        self._Hall: Dict = {}

    # -- caches per KV head
    def k_pool_head(self, b, hk):
        key = (b, hk)
        if key not in self._kpool:
            self._kpool[key] = np.stack([pool_block(self.K[b, hk], j, self.n_valid).astype(F32)
                                         for j in range(self.nb)])
        return self._kpool[key]

    def state(self, b, hk, j):
        key = (b, hk, j)
        if key not in self._H:
            shift = key_mean(self.K[b, hk], self.n_valid) if self.smooth_k else None
            self._H[key] = kv_state(self.K[b, hk], self.V[b, hk], j, self.n_valid, shift)
        return self._H[key]

    def proj_head(self, h):
        """(W, b) of head h's projection; W None = identity."""
        if self.proj_w is None:
            return None, None
        W = self.proj_w[h] if self.proj_w.ndim == 3 else self.proj_w
        bias = None
        if self.proj_b is not None:
            bias = self.proj_b[h] if self.proj_b.ndim == 2 else self.proj_b
        return W, bias

    def global_state(self, b, hk):
        key = (b, hk)
        if key not in self._Hall:
            Hs = np.zeros((self.d, self.d))
            zs = np.zeros(self.d)
            for j in range(self.nb):
                if BLOCK * j < self.n_valid:
                    H, z = self.state(b, hk, j)
                    Hs += H
                    zs += z
            self._Hall[key] = (Hs, zs)
        return self._Hall[key]

    # -- steps for one map row
    def map_head(self, h):
        return h // self.G if self.group_sum else h

    def pooled_query(self, b, hs, i) -> np.ndarray:
        if self.group_sum:
            return np.stack([pool_block(self.Q[b, h], i, self.n_valid).astype(F32)
                             for h in range(hs * self.G, (hs + 1) * self.G)]).astype(F64).sum(axis=0)
        return pool_block(self.Q[b, hs], i, self.n_valid).astype(F32)

    def score_row(self, b, hs, i) -> np.ndarray:
        hk = hs if self.group_sum else hs // self.G
        row = scores_row(self.pooled_query(b, hs, i), self.k_pool_head(b, hk), self.scale).astype(F32)
        if self.causal:
            row[i + 1:] = -np.inf
        return row

    def map_row(self, b, hs, i) -> Dict:
        row = self.score_row(b, hs, i)
        if self.causal:
            blocks, flags, negl = select_row_causal(row, i, self.n_sel, self.window)
            return dict(crit=blocks, flags=flags, marg=[], negl=negl, scores=row)
        crit, marg, negl = classify_row(row, self.n_h, self.n_l)
        if self.mode == "salad":
            negl = []
        return dict(crit=crit, flags=[1] * len(crit), marg=marg, negl=negl, scores=row)

    # -- output rows of query block i of head h
    def output_block(self, b, h, i, m: Optional[Dict] = None) -> np.ndarray:
        hk = h // self.G
        if m is None:
            m = self.map_row(b, self.map_head(h), i)
        t0 = BLOCK * i
        Qi = self.Q[b, h, t0:t0 + BLOCK].astype(F64)
        O = sparse_block(Qi, t0, self.K[b, hk], self.V[b, hk], m["crit"], m["flags"], self.n_valid,
                         self.scale, self.causal, self.window)
        if self.mode == "sla":
            O_lin = np.zeros_like(O)
            if m["marg"]:
                Hs = np.zeros((self.d, self.d))
                zs = np.zeros(self.d)
                for j in m["marg"]:
                    H, z = self.state(b, hk, j)
                    Hs += H
                    zs += z
                O_lin = linear_block(Qi, Hs, zs)
            W, bias = self.proj_head(h)
            if W is not None:
                O_lin = project(O_lin, W, bias)
            O = O + O_lin
        elif self.mode == "salad":
            Hs, zs = self.global_state(b, hk)
            gate = sigmoid(Qi @ self.w_gate[h])
            O = O + gate[:, None] * linear_block(Qi, Hs, zs)
        valid = (t0 + np.arange(BLOCK)) < self.n_valid
        return np.where(valid[:, None], O, 0.0)

    def output(self) -> np.ndarray:
        O = np.zeros((self.B, self.Hq, self.N, self.d), dtype=F64)
        for b in range(self.B):
            for h in range(self.Hq):
                for i in range(self.nb):
                    O[b, h, BLOCK * i:BLOCK * (i + 1)] = self.output_block(b, h, i)
        return O

    def maps(self) -> Dict:
        Hs = self.Hkv if self.group_sum else self.Hq
        return {(b, h, i): self.map_row(b, h, i)
                for b in range(self.B) for h in range(Hs) for i in range(self.nb)}


def forward(Q, K, V, **kw) -> np.ndarray:
    """Full output O [B, Hq, N, d] (float64) of the forward described in the module docstring."""
    return Forward(Q, K, V, **kw).output()


# ----------------------------------------------------------------------------- NSA, three branches

def compress_kv(X_head: np.ndarray, n_valid: int, block: int, stride: int) -> np.ndarray:
    """Compressed tokens of one head (NSA's compressed branch: windows of `block` tokens every
    `stride` tokens, "Sparse Attention 方法综述" section 2 and its key-parameter table): token m is
    the mean of rows m*stride .. m*stride + block - 1, for every window inside the valid rows;
    float64 [M, d] with M = (n_valid - block) // stride + 1 (0 if n_valid < block)."""
    if n_valid < block:
        return np.zeros((0, X_head.shape[1]), dtype=F64)
    M = (n_valid - block) // stride + 1
    return np.stack([X_head[m * stride:m * stride + block].astype(F64).mean(axis=0) for m in range(M)])


def softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query row over the given keys; 0 when there are none."""
    if len(keys) == 0:
        return np.zeros(vals.shape[1], dtype=F64)
    x = (keys.astype(F64) @ q.astype(F64)) * float(scale)
    p = np.exp(x - x.max())
    return (p @ vals.astype(F64)) / p.sum()


def nsa3_forward(Q, K, V, *, n_valid: int, n_sel: int, window: int, cmp_block: int, cmp_stride: int,
                 w_gates, scale: Optional[float] = None, heads: Optional[Iterable[int]] = None,
                 rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """NSA with its three parallel branches ("Sparse Attention 方法综述", section 2 NSA: compressed,
    selected and sliding-window branches, merged), output [B, Hq, N, d] float64.

    For query row t of head h (KV head g = h // (Hq/Hkv)), each branch is its own softmax attention:
      compressed: over the compressed tokens m whose window ends at or before t
                  (m * cmp_stride + cmp_block - 1 <= t);
      selected:   over the keys s <= t of the row's selected blocks, the top min(n_sel, i+1) causal
                  blocks of the GQA group's pooled scores (the NSA selection of Forward, no window);
      window:     over the keys 0 <= t - s < window;
    an empty branch gives 0.  O_t = sum over branches b of sigmoid(q_t . w_gates[b, h]) * O_b,
    w_gates [3, Hq, d] in the order (compressed, selected, window).  Rows t >= n_valid are 0.
    heads / rows: compute only these query heads and rows (the others stay 0).
    """
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    sel_fwd = Forward(Q, K, V, n_valid=n_valid, mode="nsa", n_sel=n_sel, window=0, scale=scale)
    sc = sel_fwd.scale
    W = np.asarray(w_gates, dtype=F64)
    O = np.zeros((B, Hq, N, d), dtype=F64)
    for b in range(B):
        for g in range(Hkv):
            Kg, Vg = K[b, g].astype(F64), V[b, g].astype(F64)
            Kc = compress_kv(K[b, g], n_valid, cmp_block, cmp_stride)
            Vc = compress_kv(V[b, g], n_valid, cmp_block, cmp_stride)
            hs = [h for h in range(g * G, (g + 1) * G) if heads is None or h in set(heads)]
            if not hs:
                continue
            ts = [t for t in (range(n_valid) if rows is None else rows) if t < n_valid]
            sel_rows = {i: sel_fwd.map_row(b, g, i)["crit"] for i in sorted({t // BLOCK for t in ts})}
            for h in hs:
                for t in ts:
                    q = Q[b, h, t].astype(F64)
                    n_c = max(0, min(len(Kc), (t - cmp_block + 1) // cmp_stride + 1)) if t >= cmp_block - 1 else 0
                    o_c = softmax_attend(q, Kc[:n_c], Vc[:n_c], sc)
                    sel_keys = [s for j in sel_rows[t // BLOCK] for s in range(BLOCK * j, BLOCK * (j + 1))
                                if s <= t and s < n_valid]
                    o_s = softmax_attend(q, Kg[sel_keys], Vg[sel_keys], sc)
                    lo = max(0, t - window + 1)
                    o_w = softmax_attend(q, Kg[lo:t + 1], Vg[lo:t + 1], sc) if window > 0 else np.zeros(d)
                    gates = sigmoid(W[:, h] @ q)
                    O[b, h, t] = gates[0] * o_c + gates[1] * o_s + gates[2] * o_w
    return O
