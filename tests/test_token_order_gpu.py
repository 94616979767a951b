"""GPU parity of token reordering (sla_permute_rows, through the C-ABI) and of the layer run in a
Hilbert token order, against the oracle: gathers and scatters bit-exact; the reordered layer's
output (scattered back) within rel-L2 1e-2 / max-abs 3e-2 of the oracle run on the reordered
inputs and restored; its block map identical to the oracle's map of the reordered inputs; its
backward within the backward bars."""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_backward as obwd
from oracle import sla_oracle as orc
from oracle import token_order as tor
from tests.gpu_helpers import compare_outputs, gpu_map_rows, host, say
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("dtype,d,grid,N", [(torch.bfloat16, 128, (3, 7, 9), 192), (torch.float32, 64, (2, 5, 6), 64),
                                            (torch.bfloat16, 64, (4, 6, 10), 256), (torch.float32, 128, (1, 8, 8), 64)])
def test_permute_rows_bit_exact(dtype, d, grid, N):
    say(f"[permute rows] {dtype} d={d} grid={grid} N={N}")
    nv = int(np.prod(grid))
    assert N - 64 < nv <= N
    order = tor.hilbert_order(*grid)
    r = np.random.default_rng(nv)
    X = torch.from_numpy(r.standard_normal((2, 3, N, d)).astype(np.float32)).to(dtype)
    base = torch.empty((2, 5, N, d), dtype=dtype)        # a strided view: heads 1..3 of 5
    base[:, 1:4] = X
    Xd = base.cuda()[:, 1:4]
    od = torch.from_numpy(order.astype(np.int32)).cuda()
    G = sla.sla_permute_rows(Xd, od)
    torch.cuda.synchronize()
    Xn = X.float().numpy()
    assert np.array_equal(G.float().cpu().numpy(), tor.reorder(Xn, order))
    R = sla.sla_permute_rows(G, od, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(R.float().cpu().numpy(), Xn)


def _reordered_case(w):
    q, k, v, wg = make_inputs(w)
    order = tor.hilbert_order(*w.grid)
    Qr, Kr, Vr = (tor.reorder(x.float().numpy(), order) for x in (q, k, v))
    f = orc.Forward(Qr, Kr, Vr, n_valid=w.Nv, mode=w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp)
    return q, k, v, order, f


def test_layer_in_hilbert_order():
    w = scaled(WORKLOADS["wan13b_sla"], "med_sla_hilbert", grid=(5, 18, 46), Hq=2, Hkv=2, kh_bp=2500, kl_bp=5000)
    say("[layer in Hilbert order] med_sla")
    q, k, v, order, f = _reordered_case(w)
    od = torch.from_numpy(order.astype(np.int32))
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "sla", kh_bp=w.kh_bp, kl_bp=w.kl_bp,
                           token_order=od, training=True)
    O = host(layer.run())
    torch.cuda.synchronize()
    got = gpu_map_rows(layer.maps, range(w.Hq * f.nb))
    for r_, (crit, _, marg, _) in got.items():
        h, i = divmod(r_, f.nb)
        m = f.map_row(0, h, i)
        assert crit == m["crit"] and marg == m["marg"], (h, i)
    ref = tor.restore(f.output(), order)
    compare_outputs(O[:, :, :w.Nv], ref[:, :, :w.Nv], "Hilbert-ordered layer")
    assert not O[:, :, w.Nv:].any()
    # backward through the order: gradients of the reordered problem, scattered back
    r = np.random.default_rng(5)
    dO = torch.from_numpy(r.standard_normal(q.shape).astype(np.float32)).to(q.dtype)
    dq, dk, dv = layer.backward(dO.cuda())
    torch.cuda.synchronize()
    maps = f.maps()
    _, gq, gk, gv = obwd.gradients(f.Q, f.K, f.V, tor.reorder(host(dO).astype(np.float64), order), maps, w.Nv,
                                   f.scale)
    for got_, ref_, what in zip((dq, dk, dv), (gq, gk, gv), ("dQ", "dK", "dV")):
        g_ = host(got_)[:, :, :w.Nv].astype(np.float64)
        r_ = tor.restore(ref_, order)[:, :, :w.Nv]
        rel = np.linalg.norm(g_ - r_) / np.linalg.norm(r_)
        say(f"  {what}: rel-L2 {rel:.3e}")
        assert rel <= 1e-2, what
