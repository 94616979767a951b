"""GPU test of SlaForward.capture: the layer forward recorded into one HIP graph.

Every replay must give the eager forward's output bit for bit (the same kernels on the same
inputs; no pass clears memory with a memset, so nothing depends on replaying memset nodes).
The replays are interleaved with eager work of another layer and host synchronisations, and a
replay after new inputs are copied into the captured input tensors must match an eager forward
of those inputs.  Cases: the small fp32 SLA layer, a bf16 SLA layer with GQA and a ragged tail,
SALAD, and the NSA-style causal map with head pairs.
"""
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from tests.gpu_helpers import say
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    "tiny_sla": W["tiny_sla"],
    "gqa_sla_bf16": scaled(W["tiny_sla"], "graph_gqa", Hq=4, Hkv=2, N=1280, Nv=1250, d=128, dtype="bf16",
                           kh_bp=2500, kl_bp=5000),
    "salad": scaled(W["salad"], "graph_salad", grid=(3, 10, 30), Hq=2, Hkv=2),
    "nsa_pairs": scaled(W["nsa_prefill"], "graph_nsa", N=1024, Nv=1000, Hq=4, Hkv=1, n_sel=3, window=150),
}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def layer_of(w, q, k, v, wg):
    return sla.SlaForward(q, k, v, w.Nv, w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp, n_sel=w.n_sel, window=w.window,
                          w_gate=None if wg is None else wg.cuda())


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    w = CASES[name]
    say(f"[graph] {name}")
    q, k, v, wg = (None if x is None else x.cuda() for x in make_inputs(w))
    layer = layer_of(w, q, k, v, wg)
    ref = layer.run().clone()
    other = layer_of(w, q.clone(), k.clone(), v.clone(), wg)   # eager work between the replays
    graph = layer.capture()
    for rep in range(3):
        layer.out.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, ref), f"replay {rep} differs from the eager forward"
        other.run()
        torch.cuda.synchronize()
    # new inputs in the captured tensors: the replay computes their forward
    g = torch.Generator(device="cpu").manual_seed(17)
    for x in (q, k, v):
        x.copy_((torch.randn(x.shape, generator=g) * 0.5).to(x.dtype))
        x[:, :, w.Nv:] = 0
    graph.replay()
    fresh = layer_of(w, q.clone(), k.clone(), v.clone(), wg).run()
    torch.cuda.synchronize()
    assert torch.equal(layer.out, fresh), "replay on new inputs differs from their eager forward"
    assert not torch.equal(layer.out, ref)
