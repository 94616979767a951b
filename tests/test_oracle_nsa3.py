"""Pins of the three-branch NSA oracle (CPU only): the compressed tokens against a library sliding
window mean, and the merged output against its three branches computed independently (torch SDPA
over the compressed tokens with the window-end mask, SDPA with a band mask for the window branch,
the pinned selection-only NSA forward for the selected branch), combined with torch's sigmoid."""
import numpy as np
import pytest
import torch

from oracle import sla_oracle as orc
from tests import refs
from tests.test_oracle import rand_qkv


def _sdpa_rows(q, k, v, mask, scale):
    """SDPA per row; rows with no allowed key give 0."""
    out = np.zeros((q.shape[0], v.shape[1]))
    has = mask.any(axis=1)
    if has.any():
        out[has] = refs.sdpa(q[has], k, v, scale, mask=mask[has])
    return out


@pytest.mark.parametrize("nv,block,stride", [(300, 32, 16), (64, 32, 16), (31, 32, 16), (200, 16, 16)])
def test_compressed_tokens_are_sliding_window_means(nv, block, stride):
    r = np.random.default_rng(nv)
    X = r.standard_normal((320, 8))
    got = orc.compress_kv(X, nv, block, stride)
    if nv < block:
        assert got.shape == (0, 8)
        return
    ref = np.lib.stride_tricks.sliding_window_view(X[:nv], block, axis=0)[::stride].mean(axis=-1)
    assert got.shape == ref.shape and np.allclose(got, ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("seed,zero_gates", [(41, True), (42, False)])
def test_three_branch_merge_matches_its_branches(seed, zero_gates):
    N, nv, d, Hq, Hkv = 320, 300, 16, 4, 1
    n_sel, window, block, stride = 2, 100, 32, 16
    Q, K, V = rand_qkv(1, Hq, Hkv, N, d, seed=seed, n_valid=nv, garbage=True)
    r = np.random.default_rng(seed)
    W = np.zeros((3, Hq, d)) if zero_gates else r.standard_normal((3, Hq, d)) / 4.0
    O = orc.nsa3_forward(Q, K, V, n_valid=nv, n_sel=n_sel, window=window, cmp_block=block, cmp_stride=stride,
                         w_gates=W)
    sc = orc.default_scale(d)
    O_sel = orc.Forward(Q, K, V, n_valid=nv, mode="nsa", n_sel=n_sel, window=0).output()
    t = np.arange(nv)[:, None]
    s = np.arange(nv)[None, :]
    band = (s <= t) & (t - s < window)
    Kc = np.lib.stride_tricks.sliding_window_view(K[0, 0, :nv], block, axis=0)[::stride].mean(axis=-1)
    Vc = np.lib.stride_tricks.sliding_window_view(V[0, 0, :nv], block, axis=0)[::stride].mean(axis=-1)
    m = np.arange(len(Kc))[None, :]
    cmask = m * stride + block - 1 <= t
    for h in range(Hq):
        q = Q[0, h, :nv].astype(np.float64)
        o_w = _sdpa_rows(q, K[0, 0, :nv], V[0, 0, :nv], band, sc)
        o_c = _sdpa_rows(q, Kc, Vc, cmask, sc)
        g = torch.sigmoid(torch.as_tensor(np.einsum("bd,td->tb", W[:, h], q))).numpy()
        ref = g[:, 0:1] * o_c + g[:, 1:2] * O_sel[0, h, :nv] + g[:, 2:3] * o_w
        assert np.allclose(O[0, h, :nv], ref, rtol=1e-10, atol=1e-12)
        assert np.all(O[0, h, nv:] == 0.0)
        if zero_gates:
            assert np.allclose(O[0, h, :nv], 0.5 * (o_c + O_sel[0, h, :nv] + o_w), rtol=1e-10, atol=1e-12)
