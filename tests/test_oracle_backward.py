"""Pins of the gradient oracle (CPU only): its forward against the numpy oracle, its gradients
against central finite differences of the numpy oracle, and the all-critical special case
against torch SDPA's own autograd."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import sla_backward as bwd
from oracle import sla_oracle as orc
from tests.test_oracle import rand_qkv


def _setup(seed, N=256, nv=240, d=8, H=2, kh=2500, kl=2500, proj=False):
    Q, K, V = rand_qkv(1, H, H, N, d, seed=seed, n_valid=nv, garbage=True)
    r = np.random.default_rng(seed + 100)
    dO = r.standard_normal(Q.shape)
    pw = pb = None
    if proj:
        pw, pb = r.standard_normal((H, d, d)) / np.sqrt(d), r.standard_normal((H, d))
    f = orc.Forward(Q, K, V, n_valid=nv, mode="sla", kh_bp=kh, kl_bp=kl, proj_w=pw, proj_b=pb)
    return Q, K, V, dO, f, f.maps(), pw, pb


def _numpy_loss(f, maps, dO, Q, K, V):
    """sum(dO * O) of the numpy oracle with the block map held fixed."""
    g = orc.Forward(Q, K, V, n_valid=f.n_valid, mode="sla", kh_bp=0, kl_bp=0, proj_w=f.proj_w, proj_b=f.proj_b)
    tot = 0.0
    for (b, h, i), m in maps.items():
        tot += float(np.sum(dO[b, h, 64 * i:64 * (i + 1)] * g.output_block(b, h, i, m)))
    return tot


@pytest.mark.parametrize("proj", [False, True])
def test_forward_matches_numpy_oracle(proj):
    Q, K, V, dO, f, maps, pw, pb = _setup(31, proj=proj)
    O, *_ = bwd.gradients(Q, K, V, dO, maps, f.n_valid, f.scale, pw, pb)
    assert np.allclose(O, f.output(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed,proj", [(32, False), (33, True)])
def test_gradients_match_finite_differences(seed, proj):
    Q, K, V, dO, f, maps, pw, pb = _setup(seed, proj=proj)
    n_crit = sum(len(m["crit"]) for m in maps.values())
    n_marg = sum(len(m["marg"]) for m in maps.values())
    assert n_crit and n_marg            # both branches carry gradient
    _, dQ, dK, dV = bwd.gradients(Q, K, V, dO, maps, f.n_valid, f.scale, pw, pb)
    r = np.random.default_rng(seed)
    eps = 1e-6
    for X, G, name in [(Q, dQ, "Q"), (K, dK, "K"), (V, dV, "V")]:
        for _ in range(12):
            idx = (0, r.integers(2), r.integers(f.n_valid), r.integers(X.shape[-1]))
            Xp, Xm = X.astype(np.float64).copy(), X.astype(np.float64).copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = {"Q": Q, "K": K, "V": V}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Xp, Xm
            fd = (_numpy_loss(f, maps, dO, **args_p) - _numpy_loss(f, maps, dO, **args_m)) / (2 * eps)
            assert abs(fd - G[idx]) <= 1e-6 * (1.0 + abs(fd)), (name, idx, fd, G[idx])
        assert np.all(G[:, :, f.n_valid:] == 0.0), f"padded rows of d{name} must be zero"


def test_all_critical_gradients_equal_sdpa_autograd():
    N, nv, d, H = 256, 230, 16, 2
    Q, K, V, dO, f, maps, _, _ = _setup(34, N=N, nv=nv, d=d, H=H, kh=10000, kl=0)
    _, dQ, dK, dV = bwd.gradients(Q, K, V, dO, maps, nv, f.scale)
    for h in range(H):
        q, k, v = (torch.tensor(np.asarray(X[0, h, :nv], np.float64), requires_grad=True) for X in (Q, K, V))
        o = F.scaled_dot_product_attention(q, k, v, scale=f.scale)
        o.backward(torch.tensor(dO[0, h, :nv]))
        for G, ref in [(dQ, q.grad), (dK, k.grad), (dV, v.grad)]:
            assert np.allclose(G[0, h, :nv], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_nothing_critical_gradients_equal_closed_form_linear_autograd():
    N, nv, d = 192, 180, 8
    Q, K, V, dO, f, maps, _, _ = _setup(35, N=N, nv=nv, d=d, H=1, kh=0, kl=0)
    _, dQ, dK, dV = bwd.gradients(Q, K, V, dO, maps, nv, f.scale)
    q, k, v = (torch.tensor(np.asarray(X[0, 0, :nv], np.float64), requires_grad=True) for X in (Q, K, V))
    pq, pk = F.elu(q) + 1.0, F.elu(k) + 1.0
    A = pq @ pk.T
    o = (A @ v) / A.sum(dim=1, keepdim=True)
    o.backward(torch.tensor(dO[0, 0, :nv]))
    for G, ref in [(dQ, q.grad), (dK, k.grad), (dV, v.grad)]:
        assert np.allclose(G[0, 0, :nv], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_restricted_blocks_give_the_rows_they_cover():
    """A loss over some query blocks only: dQ rows of those blocks, and dK/dV rows of a key block
    used only by those blocks, equal the full gradient's rows."""
    Q, K, V, dO, f, maps, _, _ = _setup(36)
    _, dQ, dK, dV = bwd.gradients(Q, K, V, dO, maps, f.n_valid, f.scale)
    j = 1
    users = {key for key, m in maps.items() if key[1] == 0 and (j in m["crit"] or j in m["marg"])}
    assert users
    _, dQr, dKr, dVr = bwd.gradients(Q, K, V, dO, maps, f.n_valid, f.scale, blocks=users)
    for (b, h, i) in users:
        assert np.allclose(dQr[b, h, 64 * i:64 * i + 64], dQ[b, h, 64 * i:64 * i + 64], rtol=1e-12, atol=1e-14)
    assert np.allclose(dKr[0, 0, 64 * j:64 * j + 64], dK[0, 0, 64 * j:64 * j + 64], rtol=1e-12, atol=1e-14)
    assert np.allclose(dVr[0, 0, 64 * j:64 * j + 64], dV[0, 0, 64 * j:64 * j + 64], rtol=1e-12, atol=1e-14)
    assert not dQr[0, 1].any()


@pytest.mark.parametrize("shared_w", [False, True])
def test_proj_weight_and_smooth_k_gradients_match_finite_differences(shared_w):
    """Proj weight / bias gradients and smooth-K key gradients against central differences of the
    numpy oracle (smooth-K makes every key's gradient depend on the mean over the valid keys)."""
    N, nv, d, H = 256, 240, 8, 2
    Q, K, V = rand_qkv(1, H, H, N, d, seed=37, n_valid=nv, garbage=True)
    K = K + 0.3
    r = np.random.default_rng(38)
    W = r.standard_normal((d, d) if shared_w else (H, d, d)) / np.sqrt(d)
    b = r.standard_normal(d if shared_w else (H, d))
    dO = r.standard_normal(Q.shape)
    kw = dict(n_valid=nv, mode="sla", kh_bp=2500, kl_bp=2500)
    f = orc.Forward(Q, K, V, proj_w=W, proj_b=b, smooth_k=True, **kw)
    maps = f.maps()
    O, dQ, dK, dV, dW, db = bwd.gradients(Q, K, V, dO, maps, nv, f.scale, W, b, smooth_k=True,
                                          with_proj_grads=True)
    assert np.allclose(O, f.output(), rtol=1e-12, atol=1e-13)

    def loss(Qx=Q, Kx=K, Vx=V, Wx=W, bx=b):
        g = orc.Forward(Qx, Kx, Vx, proj_w=Wx, proj_b=bx, smooth_k=True, **kw)
        return sum(float(np.sum(dO[bb, h, 64 * i:64 * i + 64] * g.output_block(bb, h, i, m)))
                   for (bb, h, i), m in maps.items())
    eps = 1e-6
    for _ in range(6):
        idx = tuple(int(r.integers(s_)) for s_ in W.shape)
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += eps
        Wm[idx] -= eps
        fd = (loss(Wx=Wp) - loss(Wx=Wm)) / (2 * eps)
        assert abs(fd - dW[idx]) <= 1e-6 * (1 + abs(fd)), ("W", idx, fd, dW[idx])
        bidx = tuple(int(r.integers(s_)) for s_ in b.shape)
        bp, bm = b.copy(), b.copy()
        bp[bidx] += eps
        bm[bidx] -= eps
        fd = (loss(bx=bp) - loss(bx=bm)) / (2 * eps)
        assert abs(fd - db[bidx]) <= 1e-6 * (1 + abs(fd)), ("b", bidx, fd, db[bidx])
        kidx = (0, int(r.integers(H)), int(r.integers(nv)), int(r.integers(d)))
        Kp, Km = K.astype(np.float64).copy(), K.astype(np.float64).copy()
        Kp[kidx] += eps
        Km[kidx] -= eps
        fd = (loss(Kx=Kp) - loss(Kx=Km)) / (2 * eps)
        assert abs(fd - dK[kidx]) <= 1e-6 * (1 + abs(fd)), ("K", kidx, fd, dK[kidx])
    assert np.all(dK[:, :, nv:] == 0.0)


# ----------------------------------------------------------------------------- SALAD and NSA (GQA)

def _mode_loss(kw, maps, dO, Q, K, V, G=1, group_map=False):
    """sum(dO * O) of the numpy oracle in any mode, with the block map held fixed."""
    g = orc.Forward(Q, K, V, **kw)
    Hq = Q.shape[1]
    tot = 0.0
    for b in range(Q.shape[0]):
        for h in range(Hq):
            mh = h // G if group_map else h
            for i in range(Q.shape[2] // 64):
                tot += float(np.sum(dO[b, h, 64 * i:64 * (i + 1)] * g.output_block(b, h, i, maps[(b, mh, i)])))
    return tot


def _fd_check(loss, arrays, grads, r, n=10, name_of=None):
    eps = 1e-6
    for name, X in arrays.items():
        G = grads[name]
        for _ in range(n):
            idx = tuple(int(r.integers(s_)) for s_ in X.shape)
            Xp, Xm = X.astype(np.float64).copy(), X.astype(np.float64).copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            fd = (loss(**{name: Xp}) - loss(**{name: Xm})) / (2 * eps)
            assert abs(fd - G[idx]) <= 1e-6 * (1.0 + abs(fd)), (name, idx, fd, G[idx])


@pytest.mark.parametrize("smooth_k", [False, True])
def test_salad_gradients_match_finite_differences(smooth_k):
    """SALAD: the sparse branch plus sigmoid(q . w_g) times linear attention over all valid keys;
    dQ, dK, dV and the gate weights' gradient against central differences of the numpy oracle."""
    N, nv, d, H = 256, 236, 8, 2
    Q, K, V = rand_qkv(1, H, H, N, d, seed=51, n_valid=nv, garbage=True)
    K = K + 0.2
    r = np.random.default_rng(52)
    wg = r.standard_normal((H, d)) / np.sqrt(d)
    dO = r.standard_normal(Q.shape)
    kw = dict(n_valid=nv, mode="salad", kh_bp=2500, w_gate=wg, smooth_k=smooth_k)
    f = orc.Forward(Q, K, V, **kw)
    maps = f.maps()
    O, dQ, dK, dV, dwg = bwd.gradients(Q, K, V, dO, maps, nv, f.scale, smooth_k=smooth_k, mode="salad", w_gate=wg)
    assert np.allclose(O, f.output(), rtol=1e-12, atol=1e-13)

    def loss(Q=Q, K=K, V=V, wg=wg):
        return _mode_loss(dict(kw, w_gate=wg), maps, dO, Q, K, V)
    _fd_check(loss, {"Q": Q, "K": K, "V": V, "wg": wg}, {"Q": dQ, "K": dK, "V": dV, "wg": dwg}, r)
    for G in (dQ, dK, dV):
        assert np.all(G[:, :, nv:] == 0.0)


def test_nsa_gqa_gradients_match_finite_differences():
    """NSA-style causal selection shared by a GQA group (4 query heads on 2 KV heads), with a
    window: dQ, and dK / dV summed over the group's heads, against central differences."""
    N, nv, d, Hq, Hkv = 640, 630, 8, 4, 2
    Q, K, V = rand_qkv(1, Hq, Hkv, N, d, seed=53, n_valid=nv, garbage=True)
    r = np.random.default_rng(54)
    dO = r.standard_normal(Q.shape)
    kw = dict(n_valid=nv, mode="nsa", n_sel=3, window=100)
    f = orc.Forward(Q, K, V, **kw)
    maps = f.maps()
    assert any(len(m["crit"]) > 3 for m in maps.values())          # window blocks beside the selection
    O, dQ, dK, dV = bwd.gradients(Q, K, V, dO, maps, nv, f.scale, mode="nsa", window=100, group_map=True)
    assert np.allclose(O, f.output(), rtol=1e-12, atol=1e-13)

    def loss(Q=Q, K=K, V=V):
        return _mode_loss(kw, maps, dO, Q, K, V, G=2, group_map=True)
    _fd_check(loss, {"Q": Q, "K": K, "V": V}, {"Q": dQ, "K": dK, "V": dV}, r)
    for G in (dQ, dK, dV):
        assert np.all(G[:, :, nv:] == 0.0)


def test_nsa_short_sequence_gradients_equal_causal_sdpa_autograd():
    """Every causal block selected (8 blocks <= 16): causal GQA attention, whose gradients torch's
    SDPA autograd gives (K and V repeated over the group, so their gradients sum over it)."""
    N, d, Hq = 512, 16, 4
    Q, K, V = rand_qkv(1, Hq, 1, N, d, seed=55)
    dO = np.random.default_rng(56).standard_normal(Q.shape)
    f = orc.Forward(Q, K, V, n_valid=N, mode="nsa", n_sel=16, window=128)
    _, dQ, dK, dV = bwd.gradients(Q, K, V, dO, f.maps(), N, f.scale, mode="nsa", window=128, group_map=True)
    q, k, v = (torch.tensor(np.asarray(X[0], np.float64), requires_grad=True) for X in (Q, K, V))
    o = F.scaled_dot_product_attention(q, k.expand(Hq, -1, -1), v.expand(Hq, -1, -1), is_causal=True, scale=f.scale)
    o.backward(torch.tensor(dO[0]))
    for G, ref in [(dQ, q.grad), (dK, k.grad), (dV, v.grad)]:
        assert np.allclose(G[0], ref.numpy(), rtol=1e-9, atol=1e-11)
