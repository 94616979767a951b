"""GPU parity at batch size 2 (every other test runs one sequence): the layer end to end for the
SLA, GQA SLA, SALAD and NSA modes, three-branch NSA, the layer in Hilbert token order and the
backward, against the oracle, with the block maps equal to the oracle's own.  Catches any
per-sequence indexing mistake (batch strides, map rows, per-sequence workspace slices)."""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_backward as obwd
from oracle import sla_oracle as orc
from oracle import token_order as tor
from tests.gpu_helpers import compare_outputs, gpu_map_rows, host, layer_for, oracle_for, say, to_dev
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    "b2_sla": scaled(W["wan13b_sla"], "b2_sla", B=2, grid=(3, 10, 30), Hq=2, Hkv=2, kh_bp=2500, kl_bp=5000),
    "b2_gqa_sla": scaled(W["tiny_sla"], "b2_gqa_sla", B=2, Hq=4, Hkv=2, N=640, Nv=610, d=128, dtype="bf16",
                         kh_bp=3000, kl_bp=4000),
    "b2_salad": scaled(W["salad"], "b2_salad", B=2, grid=(3, 10, 30), Hq=2, Hkv=2),
    "b2_nsa": scaled(W["nsa_prefill"], "b2_nsa", B=2, N=1280, Nv=1250, Hq=8),
}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _check_maps(w, f, layer):
    Hs = f.Hkv if f.group_sum else f.Hq
    got = gpu_map_rows(layer.maps, range(w.B * Hs * f.nb))
    for r_, (crit, flags, marg, _) in got.items():
        b, rem = divmod(r_, Hs * f.nb)
        h, i = divmod(rem, f.nb)
        m = f.map_row(b, h, i)
        assert crit == m["crit"] and flags == m["flags"], (b, h, i)
        if marg is not None and f.mode == "sla":
            assert marg == m["marg"], (b, h, i)


@pytest.mark.parametrize("name", list(CASES))
def test_batch2_layer(name):
    w = CASES[name]
    say(f"[batch 2] {name}")
    q, k, v, wg = make_inputs(w)
    assert w.B == 2 and not torch.equal(q[0], q[1])
    layer = layer_for(w, q, k, v, wg)
    O = host(layer.run())
    torch.cuda.synchronize()
    f = oracle_for(w, q, k, v, wg)
    _check_maps(w, f, layer)
    compare_outputs(O[:, :, :w.Nv], f.output()[:, :, :w.Nv], name)
    assert not O[:, :, w.Nv:].any()


def test_batch2_backward_and_token_order():
    w = CASES["b2_sla"]
    say("[batch 2] backward in Hilbert token order")
    q, k, v, _ = make_inputs(w)
    order = tor.hilbert_order(*w.grid)
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "sla", kh_bp=w.kh_bp, kl_bp=w.kl_bp,
                           token_order=torch.from_numpy(order.astype(np.int32)), training=True)
    O = host(layer.run())
    r = np.random.default_rng(21)
    dO = torch.from_numpy(r.standard_normal(q.shape).astype(np.float32)).to(q.dtype)
    dq, dk, dv = layer.backward(dO.cuda())
    torch.cuda.synchronize()
    Qr, Kr, Vr = (tor.reorder(x.float().numpy(), order) for x in (q, k, v))
    f = orc.Forward(Qr, Kr, Vr, n_valid=w.Nv, mode="sla", kh_bp=w.kh_bp, kl_bp=w.kl_bp)
    compare_outputs(O[:, :, :w.Nv], tor.restore(f.output(), order)[:, :, :w.Nv], "batch 2 Hilbert order")
    _, gq, gk, gv = obwd.gradients(f.Q, f.K, f.V, tor.reorder(host(dO).astype(np.float64), order), f.maps(),
                                   w.Nv, f.scale)
    for got_, ref_, what in zip((dq, dk, dv), (gq, gk, gv), ("dQ", "dK", "dV")):
        g_ = host(got_)[:, :, :w.Nv].astype(np.float64)
        r_ = tor.restore(ref_, order)[:, :, :w.Nv]
        rel = np.linalg.norm(g_ - r_) / np.linalg.norm(r_)
        say(f"  {what}: rel-L2 {rel:.3e}")
        assert rel <= 1e-2, what


def test_batch2_nsa_three_branches():
    w = CASES["b2_nsa"]
    say("[batch 2] three-branch NSA")
    q, k, v, _ = make_inputs(w)
    wg = (np.random.default_rng(5).standard_normal((3, w.Hq, w.d)) / np.sqrt(w.d)).astype(np.float32)
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "nsa", n_sel=w.n_sel, window=0)
    layer.pool_scores()
    layer.block_map()
    O = host(sla.sla_nsa3_fwd(layer.q, layer.k, layer.v, w.Nv, layer.maps, to_dev(wg, torch.float32), window=512,
                              out_dtype=torch.float32))
    torch.cuda.synchronize()
    Q, K, V = (host(x) for x in (q, k, v))
    ref = orc.nsa3_forward(Q, K, V, n_valid=w.Nv, n_sel=w.n_sel, window=512, cmp_block=32, cmp_stride=16,
                           w_gates=wg)
    compare_outputs(O[:, :, :w.Nv], ref[:, :, :w.Nv], "batch 2 nsa3")
