"""The seeded synthetic inputs (CPU): shapes, padding, block counts of the five configurations,
determinism, and the statistics the generator recipes imply.

Recipe statistics: video features F_m = sqrt(2) cos(.) have unit mean square, so F W with
W ~ N(0, 1/32) over 32 features has unit variance and Q = F W + 0.3 eps has variance 1.09;
the drift tensors eps + G U (G_m = sqrt(2) cos(.), U ~ N(0, 1/8) over 8 rows) have variance 2;
V and the i.i.d. tensors are N(0, 1); the SALAD gate vector is N(0, 1/d).
"""
import math

import numpy as np
import pytest
import torch

from oracle import sla_oracle as orc
from workloads import WORKLOADS, make_inputs, scaled


@pytest.mark.parametrize("name,N,Nv,nb,n_h,n_l", [
    ("tiny_sla", 1024, 1024, 16, 4, 8),
    ("wan13b_sla", 32768, 32760, 512, 26, 435),
    ("salad", 32768, 32760, 512, 52, 0),
    ("wan14b_sla", 75648, 75600, 1182, 60, 1004),
])
def test_config_shapes_and_counts(name, N, Nv, nb, n_h, n_l):
    w = WORKLOADS[name]
    assert (w.N, w.Nv, w.nb) == (N, Nv, nb)
    assert orc.block_counts(w.nb, w.kh_bp, w.kl_bp) == (n_h, n_l)


def test_nsa_config():
    w = WORKLOADS["nsa_prefill"]
    assert (w.B, w.Hq, w.Hkv, w.N, w.Nv, w.d, w.dtype) == (1, 16, 1, 65536, 65536, 128, "bf16")
    assert w.causal and (w.n_sel, w.window) == (16, 512)
    assert w.dense_flops() == pytest.approx(2.0 * 16 * 65536 ** 2 * 128)


def _std(t, nv):
    return float(t[:, :, :nv].float().std())


def test_video_generator():
    w = scaled(WORKLOADS["wan13b_sla"], "small_video", grid=(3, 10, 13), Hq=3, Hkv=3)
    q, k, v, wg = make_inputs(w)
    assert wg is None
    assert q.shape == (1, 3, w.N, 128) and q.dtype == torch.bfloat16 and w.N == 448 and w.Nv == 390
    for t in (q, k, v):
        assert not t[:, :, w.Nv:].any()                       # padded rows are zero
    q2, k2, v2, _ = make_inputs(w)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    assert _std(v, w.Nv) == pytest.approx(1.0, rel=0.05)
    assert abs(float(v[:, :, :w.Nv].float().mean())) < 0.02
    assert _std(q, w.Nv) == pytest.approx(math.sqrt(1.09), rel=0.15)
    assert _std(k, w.Nv) == pytest.approx(math.sqrt(1.09), rel=0.15)
    # the features vary smoothly over the grid, so neighbouring tokens' queries are alike (the
    # mean dot product of consecutive rows); V is i.i.d. noise (its mean dot product is near 0)
    nb_dot = lambda t: float((t[0, 0, :w.Nv - 1].float() * t[0, 0, 1:w.Nv].float()).sum(1).mean())
    assert nb_dot(q) > 10.0 and nb_dot(k) > 10.0
    assert abs(nb_dot(v)) < 5.0


def test_salad_shares_the_video_tensors():
    grid = (2, 6, 11)
    a = make_inputs(scaled(WORKLOADS["wan13b_sla"], "a", grid=grid, Hq=2, Hkv=2))
    b = make_inputs(scaled(WORKLOADS["salad"], "b", grid=grid, Hq=2, Hkv=2))
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    wg = b[3]
    assert wg.shape == (2, 128) and wg.dtype == torch.float32
    full = make_inputs(scaled(WORKLOADS["salad"], "c", grid=grid))[3]   # 12 heads x 128
    assert float(full.std()) == pytest.approx(1.0 / math.sqrt(128), rel=0.1)


def test_drift_generator():
    w = scaled(WORKLOADS["nsa_prefill"], "small_drift", N=2048, Nv=2000)
    q, k, v, wg = make_inputs(w)
    assert q.shape == (1, 16, 2048, 128) and k.shape == v.shape == (1, 1, 2048, 128)
    for t in (q, k, v):
        assert not t[:, :, w.Nv:].any()
    assert _std(q, w.Nv) == pytest.approx(math.sqrt(2.0), rel=0.15)
    # the drift G U varies slowly along the sequence: neighbouring rows share it
    km = k[0, 0, :w.Nv].float()
    assert float((km[:-1] * km[1:]).sum(1).mean()) > 64.0        # ~ d * Var(G U) = 128


def test_iid_generator():
    q, k, v, _ = make_inputs(WORKLOADS["tiny_sla"])
    assert q.dtype == torch.float32 and q.shape == (1, 1, 1024, 64)
    for t in (q, k, v):
        assert float(t.std()) == pytest.approx(1.0, rel=0.05)
    assert not torch.equal(q, k) and not torch.equal(k, v)
    x = np.concatenate([t.numpy().ravel() for t in (q, k, v)])
    assert abs(float(np.corrcoef(x[:-1], x[1:])[0, 1])) < 0.02   # independent draws
