"""Pins of the CPU oracle against things other than itself (CPU only, no GPU).

Every check compares the oracle with a closed form, a library routine on a special
case, a brute-force definition, a hand-worked golden fixture, or an invariant of
the method, so that a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import sla_oracle as orc
from tests import refs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


def bf16_round(a):
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def rand_qkv(B, Hq, Hkv, N, d, seed, n_valid=None, garbage=False):
    r = np.random.default_rng(seed)
    Q = bf16_round(r.standard_normal((B, Hq, N, d)))
    K = bf16_round(r.standard_normal((B, Hkv, N, d)))
    V = bf16_round(r.standard_normal((B, Hkv, N, d)))
    if n_valid is not None and n_valid < N:
        for X in (Q, K, V):
            X[:, :, n_valid:] = (r.standard_normal(X[:, :, n_valid:].shape) * 7.0 + 3.0) if garbage else 0.0
    return Q, K, V


# ----------------------------------------------------------------------------- counts and phi

def test_counts_golden():
    data = json.load(open(os.path.join(GOLDEN, "counts.json")))
    for c in data["cases"]:
        assert orc.block_counts(c["nb"], c["kh_bp"], c["kl_bp"]) == (c["n_h"], c["n_l"]), c["what"]


def test_phi_is_elu_plus_one():
    x = np.linspace(-6, 6, 1001)
    assert np.allclose(orc.phi(x), refs.elu1(x), rtol=0, atol=1e-15)
    assert orc.phi(0.0) == 1.0 and orc.phi(1.0) == 2.0 and orc.phi(-1.0) == math.exp(-1.0)
    assert np.all(orc.phi(x) > 0)


# ----------------------------------------------------------------------------- pooling and scores

def test_pool_constant_blocks_and_padding():
    N, d, nv = 256, 16, 256 - 24
    consts = rng0.standard_normal((4, d)).astype(np.float32)
    X = np.repeat(consts, 64, axis=0)[None, None].copy()
    X[0, 0, nv:] = 1e3 * rng0.standard_normal((N - nv, d))     # padding garbage
    P = orc.pool(X, nv)
    assert P.shape == (1, 1, 4, d)
    assert np.array_equal(P[0, 0], consts)


def test_pool_matches_blockwise_mean_of_valid_rows():
    N, d, nv = 320, 8, 300
    X = bf16_round(rng0.standard_normal((1, 2, N, d)))
    P = orc.pool(X, nv)
    for i in range(5):
        hi = min(64 * i + 64, nv)
        ref = np.mean(X[0, 1, 64 * i:hi].astype(np.float64), axis=0)
        assert np.allclose(P[0, 1, i], ref, rtol=1e-7, atol=0)


def test_scores_closed_form_and_probs():
    d = 32
    cq = np.array([1.0, -2.0, 0.5, 4.0], np.float32)
    ck = np.array([0.25, 2.0, -1.0, 8.0], np.float32)
    qp = (cq[:, None] * np.ones((4, d), np.float32))[None, None]
    kp = (ck[:, None] * np.ones((4, d), np.float32))[None, None]
    scale = 0.125
    S = orc.pooled_scores(qp, kp, scale)
    expect = (scale * d * np.outer(cq.astype(np.float64), ck)).astype(np.float32)   # exact powers of two
    assert np.array_equal(S[0, 0], expect)
    P = orc.score_probs(S)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-6)
    assert np.array_equal(P.argmax(-1), S.argmax(-1))


def test_default_scale_is_sdpa_default_on_exact_attention():
    """The oracle's default scale against torch SDPA's own default (scale=None, 1/sqrt(d)): an
    all-critical SLA forward with no scale given must be dense attention at SDPA's default."""
    import torch
    import torch.nn.functional as F
    for d in (16, 64):
        N = 192
        Q, K, V = rand_qkv(1, 1, 1, N, d, seed=60 + d)
        O = orc.forward(Q, K, V, n_valid=N, mode="sla", kh_bp=10000, kl_bp=0)
        t = lambda x: torch.as_tensor(x[0, 0].astype(np.float64))
        ref = F.scaled_dot_product_attention(t(Q), t(K), t(V)).numpy()      # SDPA picks its own scale
        # the oracle rounds 1/sqrt(d) to float32 once: relative effect on the logits <= 2^-24
        assert np.allclose(O[0, 0], ref, rtol=1e-6, atol=1e-7)
        for wrong in (1.0 / d, math.sqrt(d), 1.0):
            bad = F.scaled_dot_product_attention(t(Q), t(K), t(V), scale=wrong).numpy()
            assert not np.allclose(O[0, 0], bad, rtol=1e-3, atol=1e-3)


def test_score_probs_are_attention_weights_of_pooled_vectors():
    """Row softmax of the pooled scores at the default scale against (a) torch SDPA's attention
    weights over the pooled vectors (values = identity, SDPA's own default scale) and (b)
    torch.softmax over rows with causal -inf entries."""
    import torch
    import torch.nn.functional as F
    r = np.random.default_rng(61)
    nb, d = 12, 32
    qp = r.standard_normal((1, 1, nb, d)).astype(np.float32)
    kp = r.standard_normal((1, 1, nb, d)).astype(np.float32)
    S = orc.pooled_scores(qp, kp, orc.default_scale(d))
    P = orc.score_probs(S)
    eye = torch.eye(nb, dtype=torch.float64)
    W = F.scaled_dot_product_attention(torch.as_tensor(qp[0, 0].astype(np.float64)),
                                       torch.as_tensor(kp[0, 0].astype(np.float64)), eye).numpy()
    assert np.allclose(P[0, 0], W, rtol=2e-6, atol=1e-7)
    # softmax at another temperature is far from it
    assert not np.allclose(orc.score_probs(2.0 * S)[0, 0], W, rtol=1e-2, atol=1e-3)
    # causal rows: -inf entries get probability 0, the rest a softmax over the finite entries
    Sc = orc.pooled_scores(qp, kp, orc.default_scale(d), causal=True)
    Pc = orc.score_probs(Sc)
    ref = torch.softmax(torch.as_tensor(Sc[0, 0].astype(np.float64)), dim=-1).numpy()
    assert np.allclose(Pc[0, 0], ref, rtol=2e-6, atol=1e-7)
    assert np.all(Pc[0, 0][np.triu_indices(nb, 1)] == 0.0)
    assert np.allclose(Pc[0, 0, 0, 0], 1.0)


def test_group_scores_are_sum_of_head_scores():
    B, Hq, Hkv, nb, d = 1, 4, 2, 6, 16
    qp = rng0.standard_normal((B, Hq, nb, d)).astype(np.float32)
    kp = rng0.standard_normal((B, Hkv, nb, d)).astype(np.float32)
    Sg = orc.pooled_scores(qp, kp, 0.25, group_sum=True)
    for g in range(Hkv):
        ref = sum(qp[0, h].astype(np.float64) @ kp[0, g].astype(np.float64).T for h in (2 * g, 2 * g + 1)) * 0.25
        assert np.allclose(Sg[0, g], ref, rtol=2e-7, atol=1e-7)
    Sc = orc.pooled_scores(qp, kp, 0.25, group_sum=True, causal=True)
    iu = np.triu_indices(nb, 1)
    assert np.all(np.isneginf(Sc[0, 0][iu]))
    il = np.tril_indices(nb)
    assert np.array_equal(Sc[0, 0][il], Sg[0, 0][il])


# ----------------------------------------------------------------------------- block maps

def test_block_map_golden_ties():
    data = json.load(open(os.path.join(GOLDEN, "block_map_ties.json")))
    row = refs.parse_json_scores(data["scores"])
    for c in data["cases"]:
        crit, marg, negl = orc.classify_row(row, c["n_h"], c["n_l"])
        assert (crit, marg, negl) == (c["crit"], c["marg"], c["negl"]), c


def test_nsa_select_golden():
    data = json.load(open(os.path.join(GOLDEN, "nsa_select.json")))
    for r in data["rows"]:
        row = refs.parse_json_scores(r["scores"])
        blocks, flags, negl = orc.select_row_causal(row, r["i"], r["n_sel"], r["window"])
        assert (blocks, flags, negl) == (r["blocks"], r["flags"], r["negl"]), r


@pytest.mark.parametrize("seed", range(6))
def test_block_map_brute_force_with_ties(seed):
    r = np.random.default_rng(seed)
    nb = int(r.integers(3, 40))
    levels = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 3.0], np.float32)
    for _ in range(20):
        row = r.choice(levels, size=nb).astype(np.float32)
        if r.random() < 0.3:
            row[r.integers(0, nb)] = np.nan
        n_h, n_l = orc.block_counts(nb, int(r.integers(0, 10001)), int(r.integers(0, 10001)))
        assert orc.classify_row(row, n_h, n_l) == refs.brute_classes(row, n_h, n_l)


def test_block_map_invariants_tiny_workload():
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["tiny_sla"]
    q, k, v, _ = make_inputs(w)
    Q, K = q.numpy(), k.numpy()
    S = orc.pooled_scores(orc.pool(Q, w.Nv), orc.pool(K, w.Nv), orc.default_scale(w.d))
    n_h, n_l = orc.block_counts(w.nb, w.kh_bp, w.kl_bp)
    maps = orc.block_map(S, n_h=n_h, n_l=n_l)
    for (b, h, i), m in maps.items():
        c, mg, ng = m["crit"], m["marg"], m["negl"]
        assert len(c) == n_h and len(ng) == n_l and len(c) + len(mg) + len(ng) == w.nb
        assert not (set(c) & set(mg)) and not (set(mg) & set(ng)) and not (set(c) & set(ng))
        s = S[b, h, i]
        if mg:
            assert s[c].min() >= s[mg].max()
        if ng:
            assert s[mg].min() >= s[ng].max() and s[c].min() >= s[ng].max()
        assert (c, mg, ng) == tuple(refs.brute_classes(s, n_h, n_l))
    csr = orc.to_csr(maps, 1, 1, w.nb)
    assert csr["crit_rowptr"][-1] == w.nb * n_h and csr["marg_rowptr"][-1] == w.nb * (w.nb - n_h - n_l)


# ----------------------------------------------------------------------------- linear states

def test_kv_states_sum_to_global_closed_form():
    Q, K, V = rand_qkv(1, 1, 1, 320, 16, seed=3, n_valid=290, garbage=True)
    H, z = orc.kv_states(K, V, 290)
    pk = refs.elu1(K[0, 0, :290])
    assert np.allclose(H[0, 0].sum(0), pk.T @ V[0, 0, :290].astype(np.float64), rtol=1e-12, atol=1e-10)
    assert np.allclose(z[0, 0].sum(0), pk.sum(0), rtol=1e-12)
    # H_j is phi(K)^T V, not V^T phi(K): check one block against an explicit sum of outer products
    j = 1
    ref = sum(np.outer(pk[s], V[0, 0, s]) for s in range(64 * j, 64 * j + 64))
    assert np.allclose(H[0, 0, j], ref, rtol=1e-12, atol=1e-10)


# ----------------------------------------------------------------------------- outputs: special cases

def _valid_sdpa(Q, K, V, nv, scale, **kw):
    return refs.sdpa(Q[:nv], K[:nv], V[:nv], scale, **kw)


@pytest.mark.parametrize("N,nv", [(256, 256), (320, 289)])
def test_all_critical_equals_dense_attention(N, nv):
    d = 32
    Q, K, V = rand_qkv(1, 2, 2, N, d, seed=5, n_valid=nv, garbage=True)
    O = orc.forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=10000, kl_bp=3000)
    sc = orc.default_scale(d)
    for h in range(2):
        ref = _valid_sdpa(Q[0, h], K[0, h], V[0, h], nv, sc)
        assert np.allclose(O[0, h, :nv], ref, rtol=1e-10, atol=1e-12)
        assert np.all(O[0, h, nv:] == 0.0)


@pytest.mark.parametrize("N,nv", [(256, 256), (320, 300)])
def test_nothing_critical_equals_closed_form_linear_attention(N, nv):
    d = 16
    Q, K, V = rand_qkv(1, 1, 1, N, d, seed=7, n_valid=nv, garbage=True)
    O = orc.forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=0, kl_bp=0)
    ref = refs.kernel_linear_attention(Q[0, 0, :nv], K[0, 0, :nv], V[0, 0, :nv])
    assert np.allclose(O[0, 0, :nv], ref, rtol=1e-10, atol=1e-12)
    assert np.all(O[0, 0, nv:] == 0.0)


# ----------------------------------------------------------------------------- Proj and smooth-K

def _linear_layer(x, W, b):
    """torch's Linear convention (x W^T + b), as a library routine."""
    import torch
    return torch.nn.functional.linear(torch.as_tensor(x), torch.as_tensor(np.asarray(W, np.float64)),
                                      None if b is None else torch.as_tensor(np.asarray(b, np.float64))).numpy()


def test_proj_all_marginal_is_projected_closed_form_linear_attention():
    N, nv, d, H = 256, 230, 16, 2
    Q, K, V = rand_qkv(1, H, H, N, d, seed=21, n_valid=nv, garbage=True)
    r = np.random.default_rng(22)
    W, b = r.standard_normal((H, d, d)) / 4.0, r.standard_normal((H, d))
    O = orc.forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=0, kl_bp=0, proj_w=W, proj_b=b)
    for h in range(H):
        la = refs.kernel_linear_attention(Q[0, h, :nv], K[0, h, :nv], V[0, h, :nv])
        assert np.allclose(O[0, h, :nv], _linear_layer(la, W[h], b[h]), rtol=1e-10, atol=1e-12)
        assert np.all(O[0, h, nv:] == 0.0)
    # one weight shared by all heads, no bias
    O1 = orc.forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=0, kl_bp=0, proj_w=W[1])
    la = refs.kernel_linear_attention(Q[0, 0, :nv], K[0, 0, :nv], V[0, 0, :nv])
    assert np.allclose(O1[0, 0, :nv], _linear_layer(la, W[1], None), rtol=1e-10, atol=1e-12)


def test_zero_proj_weight_leaves_sparse_branch_plus_bias():
    N, nv, d = 384, 350, 16
    Q, K, V = rand_qkv(1, 2, 1, N, d, seed=23, n_valid=nv, garbage=True)
    b = np.random.default_rng(24).standard_normal(d)
    kw = dict(n_valid=nv, mode="sla", kh_bp=2500)
    O = orc.forward(Q, K, V, kl_bp=3000, proj_w=np.zeros((d, d)), proj_b=b, **kw)
    O_sparse = orc.forward(Q, K, V, kl_bp=10000, **kw)     # every non-critical block negligible
    assert np.allclose(O[:, :, :nv], O_sparse[:, :, :nv] + b, rtol=1e-12, atol=1e-12)
    assert np.all(O[:, :, nv:] == 0.0)


def test_identity_proj_equals_no_proj():
    N, nv, d = 320, 320, 16
    Q, K, V = rand_qkv(1, 1, 1, N, d, seed=25)
    kw = dict(n_valid=nv, mode="sla", kh_bp=2500, kl_bp=2500)
    assert np.allclose(orc.forward(Q, K, V, proj_w=np.eye(d), **kw), orc.forward(Q, K, V, **kw),
                       rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("N,nv", [(256, 256), (320, 300)])
def test_smooth_k_all_marginal_is_linear_attention_of_centred_keys(N, nv):
    d = 16
    Q, K, V = rand_qkv(1, 1, 1, N, d, seed=26, n_valid=nv, garbage=True)
    K = K + 0.7      # a non-zero key mean
    O = orc.forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=0, kl_bp=0, smooth_k=True)
    Kc = K[0, 0, :nv] - np.mean(K[0, 0, :nv], axis=0, dtype=np.float64)     # padding excluded
    ref = refs.kernel_linear_attention(Q[0, 0, :nv], Kc, V[0, 0, :nv])
    assert np.allclose(O[0, 0, :nv], ref, rtol=1e-10, atol=1e-12)
    assert not np.allclose(ref, refs.kernel_linear_attention(Q[0, 0, :nv], K[0, 0, :nv], V[0, 0, :nv]),
                           rtol=1e-3, atol=1e-3)
    assert np.all(O[0, 0, nv:] == 0.0)


def test_smooth_k_leaves_softmax_branch_and_salad_gates_centred_linear_branch():
    N, nv, d = 256, 250, 16
    Q, K, V = rand_qkv(1, 1, 1, N, d, seed=27, n_valid=nv, garbage=True)
    K = K - 0.5
    sc = orc.default_scale(d)
    dense = _valid_sdpa(Q[0, 0], K[0, 0], V[0, 0], nv, sc)
    Kc = K[0, 0, :nv] - np.mean(K[0, 0, :nv], axis=0, dtype=np.float64)
    # premise of the reading: one shift of every key leaves softmax attention unchanged
    assert np.allclose(refs.sdpa(Q[0, 0, :nv], Kc, V[0, 0, :nv], sc), dense, rtol=1e-10, atol=1e-12)
    O = orc.forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=10000, kl_bp=0, smooth_k=True)
    assert np.allclose(O[0, 0, :nv], dense, rtol=1e-10, atol=1e-12)
    Os = orc.forward(Q, K, V, n_valid=nv, mode="salad", kh_bp=10000, w_gate=np.zeros((1, d)), smooth_k=True)
    ref = dense + 0.5 * refs.kernel_linear_attention(Q[0, 0, :nv], Kc, V[0, 0, :nv])
    assert np.allclose(Os[0, 0, :nv], ref, rtol=1e-10, atol=1e-12)


def test_everything_negligible_gives_zero():
    Q, K, V = rand_qkv(1, 1, 1, 192, 8, seed=8)
    O = orc.forward(Q, K, V, n_valid=192, mode="sla", kh_bp=0, kl_bp=10000)
    assert np.all(O == 0.0)


@pytest.mark.parametrize("seed", [11, 12])
def test_generic_sla_equals_masked_softmax_plus_masked_kernel_attention(seed):
    N, nv, d, Hq, Hkv = 384, 370, 16, 2, 1
    Q, K, V = rand_qkv(1, Hq, Hkv, N, d, seed=seed, n_valid=nv, garbage=True)
    kh, kl = 2500, 4000
    O = orc.forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=kh, kl_bp=kl)
    sc = orc.default_scale(d)
    S = orc.pooled_scores(orc.pool(Q, nv), orc.pool(K, nv), sc)
    nb = N // 64
    n_h, n_l = orc.block_counts(nb, kh, kl)
    for h in range(Hq):
        rows = [refs.brute_classes(S[0, h, i], n_h, n_l) for i in range(nb)]
        cm, mm = refs.brute_token_masks(rows, nb, N, nv)
        ref = np.zeros((N, d))
        qv, kv_, vv = Q[0, h], K[0, 0], V[0, 0]
        ref += refs.sdpa(qv, kv_, vv, sc, mask=cm)
        ref += refs.kernel_linear_attention(qv, kv_, vv, mask=mm)
        assert np.allclose(O[0, h, :nv], ref[:nv], rtol=1e-9, atol=1e-11)


def test_linearity_in_v_and_padding_invariance():
    N, nv, d = 320, 301, 16
    Q, K, V = rand_qkv(1, 1, 1, N, d, seed=13, n_valid=nv)
    kw = dict(n_valid=nv, mode="sla", kh_bp=2500, kl_bp=3000)
    O1 = orc.forward(Q, K, V, **kw)
    O2 = orc.forward(Q, K, 2.0 * V, **kw)
    assert np.array_equal(O2, 2.0 * O1)
    Qg, Kg, Vg = (X.copy() for X in (Q, K, V))
    for X in (Qg, Kg, Vg):
        X[:, :, nv:] = 55.0
    assert np.array_equal(orc.forward(Qg, Kg, Vg, **kw), O1)


def test_key_block_permutation_equivariance():
    N, d = 384, 16
    Q, K, V = rand_qkv(1, 1, 1, N, d, seed=17)
    kw = dict(n_valid=N, mode="sla", kh_bp=3400, kl_bp=3300)
    f = orc.Forward(Q, K, V, **kw)
    perm = np.array([3, 0, 5, 1, 4, 2])
    tok = np.concatenate([np.arange(64 * p, 64 * p + 64) for p in perm])
    Kp, Vp = K[:, :, tok].copy(), V[:, :, tok].copy()
    g = orc.Forward(Q, Kp, Vp, **kw)
    inv = np.argsort(perm)
    for i in range(6):
        a, b = f.map_row(0, 0, i), g.map_row(0, 0, i)
        assert sorted(perm[b["crit"]].tolist()) == a["crit"]
        assert sorted(perm[b["marg"]].tolist()) == a["marg"]
    assert np.allclose(f.output(), g.output(), rtol=1e-12, atol=1e-13)
    assert inv is not None


# ----------------------------------------------------------------------------- SALAD

def test_salad_zero_gate_weights_half_linear_plus_dense():
    N, nv, d = 256, 250, 16
    Q, K, V = rand_qkv(1, 2, 2, N, d, seed=19, n_valid=nv, garbage=True)
    wg = np.zeros((2, d))
    O = orc.forward(Q, K, V, n_valid=nv, mode="salad", kh_bp=10000, w_gate=wg)
    sc = orc.default_scale(d)
    for h in range(2):
        ref = _valid_sdpa(Q[0, h], K[0, h], V[0, h], nv, sc) + \
            0.5 * refs.kernel_linear_attention(Q[0, h, :nv], K[0, h, :nv], V[0, h, :nv])
        assert np.allclose(O[0, h, :nv], ref, rtol=1e-10, atol=1e-12)


def test_salad_gate_limits_and_top_blocks():
    import torch
    N, d = 320, 16
    Q, K, V = rand_qkv(1, 1, 1, N, d, seed=23)
    sc = orc.default_scale(d)
    lin = refs.kernel_linear_attention(Q[0, 0], K[0, 0], V[0, 0])
    # a huge gate vector along the sign of each query row's first coordinate drives the gate to 0 or 1
    wg = np.zeros((1, d)); wg[0, 0] = 1e4
    f = orc.Forward(Q, K, V, n_valid=N, mode="salad", kh_bp=4000, w_gate=wg)
    O = f.output()
    S = orc.pooled_scores(orc.pool(Q, N), orc.pool(K, N), sc)
    n_h, _ = orc.block_counts(5, 4000, 0)
    rows = [refs.brute_classes(S[0, 0, i], n_h, 0) for i in range(5)]
    cm, _ = refs.brute_token_masks(rows, 5, N, N)
    sparse = refs.sdpa(Q[0, 0], K[0, 0], V[0, 0], sc, mask=cm)
    gate = torch.sigmoid(torch.as_tensor(Q[0, 0].astype(np.float64) @ wg[0])).numpy()
    assert set(np.round(gate[np.abs(Q[0, 0, :, 0]) > 0.01], 12)) <= {0.0, 1.0}
    assert np.allclose(O[0, 0], sparse + gate[:, None] * lin, rtol=1e-10, atol=1e-12)
    pos = Q[0, 0, :, 0] > 0.01
    assert np.allclose(O[0, 0][pos], (sparse + lin)[pos], rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------- NSA-style selected + window

def _expand(K, G):
    return np.repeat(K, G, axis=0)


def test_nsa_short_sequence_is_dense_causal_gqa():
    N, d, Hq = 512, 16, 4       # 8 blocks <= 16 selected: every causal block is selected
    Q, K, V = rand_qkv(1, Hq, 1, N, d, seed=29)
    O = orc.forward(Q, K, V, n_valid=N, mode="nsa", n_sel=16, window=128)
    ref = refs.sdpa(Q[0], _expand(K[0], Hq), _expand(V[0], Hq), orc.default_scale(d), causal=True)
    assert np.allclose(O[0], ref, rtol=1e-10, atol=1e-12)


def test_nsa_no_selection_is_sliding_window():
    N, d, Hq, w = 640, 16, 2, 100
    Q, K, V = rand_qkv(1, Hq, 1, N, d, seed=31)
    O = orc.forward(Q, K, V, n_valid=N, mode="nsa", n_sel=0, window=w)
    t = np.arange(N)[:, None]
    s = np.arange(N)[None, :]
    band = (t - s >= 0) & (t - s < w)
    ref = refs.sdpa(Q[0], _expand(K[0], Hq), _expand(V[0], Hq), orc.default_scale(d), mask=band)
    assert np.allclose(O[0], ref, rtol=1e-10, atol=1e-12)


def test_nsa_selection_only_and_selected_token_budget():
    N, d, Hq, n_sel = 1536, 16, 2, 16      # 24 blocks: rows i >= 16 select 16 of i+1
    Q, K, V = rand_qkv(1, Hq, 1, N, d, seed=37)
    f = orc.Forward(Q, K, V, n_valid=N, mode="nsa", n_sel=n_sel, window=0)
    O = f.output()
    sc = orc.default_scale(d)
    S = orc.pooled_scores(orc.pool(Q, N), orc.pool(K, N), sc, group_sum=True, causal=True)
    mask = np.zeros((N, N), bool)
    for i in range(24):
        r = refs.ranks(S[0, 0, i, :i + 1])
        sel = [j for j in range(i + 1) if r[j] < min(n_sel, i + 1)]
        for j in sel:
            mask[64 * i:64 * i + 64, 64 * j:64 * j + 64] = True
        if i >= 16:
            # 16 selected blocks of 64 keys: the last query row of the block attends 1024 tokens
            assert len(sel) * 64 == 1024
    mask &= np.tril(np.ones((N, N), bool))
    ref = refs.sdpa(Q[0], _expand(K[0], Hq), _expand(V[0], Hq), sc, mask=mask)
    assert np.allclose(O[0], ref, rtol=1e-10, atol=1e-12)


def test_nsa_selected_union_window_counts():
    N, d, Hq = 2048, 8, 2
    Q, K, V = rand_qkv(1, Hq, 1, N, d, seed=41)
    f = orc.Forward(Q, K, V, n_valid=N, mode="nsa", n_sel=16, window=512)
    for i in range(32):
        m = f.map_row(0, 0, i)
        assert m["crit"] == sorted(m["crit"])
        assert len(m["crit"]) + len(m["negl"]) == i + 1
        if i >= 16:
            assert 16 <= len(m["crit"]) <= 25
            assert sum(1 for fl in m["flags"] if fl & 1) == 16
        assert [j for j, fl in zip(m["crit"], m["flags"]) if fl & 2] == list(range(max(0, i - 8), i + 1))
