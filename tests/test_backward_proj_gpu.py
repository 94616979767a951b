"""GPU parity of the SLA backward with the learned Proj and smooth-K (sla_attn_bwd through the
C-ABI) against the gradient oracle: dQ, dK, dV and the Proj weight and bias gradients of
sum(dO * O) on the oracle's block map, every valid row, rel-L2 <= 1e-2 and max-abs <= 3e-2 of the
largest reference magnitude per gradient.

Error sources beyond the plain backward: the Proj weight and the linear-branch output enter the
products as bf16 (2^-9 relative each) and dW sums a few thousand such products per entry in fp32;
the smooth-K key shift is the fp32 mean of the pooled block means.  Padded rows of dO are set to
5: they must leave every gradient (dW and db included) unchanged.
"""
import numpy as np
import pytest
import torch

from oracle import sla_backward as obwd
from tests.gpu_helpers import host, make_case, oracle_csr, say
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

W = WORKLOADS
MED = dict(grid=(5, 18, 46), Hq=2, Hkv=2, kh_bp=2500, kl_bp=5000)
# name: (workload, Proj per head (None: no Proj), bias, smooth-K)
CASES = {
    "tiny_shared_bias_smoothk": (W["tiny_sla"], False, True, True),
    "med_per_head_bias_smoothk": (scaled(W["wan13b_sla"], "med_sla", **MED), True, True, True),
    "med_smoothk_only": (scaled(W["wan13b_sla"], "med_sla", **MED), None, False, True),
    "med_shared_nobias": (scaled(W["wan13b_sla"], "med_sla", **MED), False, False, False),
    "med_d64_per_head_f32": (scaled(W["wan13b_sla"], "med_sla_d64", grid=(4, 9, 20), Hq=2, Hkv=2, d=64,
                                    dtype="f32", kh_bp=1500, kl_bp=6000), True, True, True),
    "b2_shared_bias_smoothk": (scaled(W["wan13b_sla"], "b2_sla", B=2, grid=(3, 10, 30), Hq=2, Hkv=2, kh_bp=2500,
                                      kl_bp=5000), False, True, True),
    # GQA (two query heads per KV head, maps per query head): dW per query head, the key side's state
    # gradients summed over the group's heads
    "gqa_per_head_bias_smoothk": (scaled(W["tiny_sla"], "gqa_bp", Hq=4, Hkv=2, N=1280, Nv=1250, d=128,
                                         dtype="bf16", kh_bp=2500, kl_bp=5000), True, True, True),
    "all_linear_proj": (scaled(W["wan13b_sla"], "med_all_linear", grid=(3, 10, 30), Hq=1, Hkv=1, kh_bp=0, kl_bp=0),
                        True, True, True),
    "all_crit_proj": (scaled(W["wan13b_sla"], "med_all_crit", grid=(3, 10, 30), Hq=1, Hkv=1, kh_bp=10000, kl_bp=0),
                      False, True, True),
}
REL_L2, MAX_ABS_FRAC = 1e-2, 3e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def proj_weights(w, per_head, bias, seed):
    if per_head is None:
        return None, None
    r = np.random.default_rng(seed)
    shape = (w.Hq, w.d, w.d) if per_head else (w.d, w.d)
    Wp = (r.standard_normal(shape) / np.sqrt(w.d)).astype(np.float32)
    bp = (0.5 * r.standard_normal(shape[:-1])).astype(np.float32) if bias else None
    return Wp, bp


def check(got, ref, what):
    got = got.astype(np.float64)
    diff = got - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(diff).max() / max(np.abs(ref).max(), 1e-30)
    say(f"  {what}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
    assert rel <= REL_L2, (what, rel)
    assert mx <= MAX_ABS_FRAC, (what, mx)


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_proj_smoothk(name):
    w, per_head, bias, smooth_k = CASES[name]
    say(f"[backward, Proj {per_head} bias {bias} smooth-K {smooth_k}] {name}")
    Wp, bp = proj_weights(w, per_head, bias, 31)
    q, k, v, wg, f, layer = make_case(w, proj_w=Wp, proj_b=bp, smooth_k=smooth_k, training=True)
    csr, maps = oracle_csr(f)
    r = np.random.default_rng(77)
    dO = torch.from_numpy(r.standard_normal(q.shape).astype(np.float32)).to(q.dtype)
    dO[:, :, w.Nv:] = 5.0
    layer.pool_scores()
    layer.kv_reduce()
    layer.marginal_states(maps=csr)
    O = host(layer.attention(maps=csr))
    g = layer.backward(dO.cuda(), maps=csr)
    torch.cuda.synchronize()
    ref = obwd.gradients(f.Q, f.K, f.V, host(dO).astype(np.float64), maps, w.Nv, f.scale, proj_w=Wp, proj_b=bp,
                         smooth_k=smooth_k, with_proj_grads=True)
    nv = w.Nv
    check(O[:, :, :nv], ref[0][:, :, :nv], "O")
    for got_, ref_, what in zip(g[:3], ref[1:4], ("dQ", "dK", "dV")):
        gh = host(got_)
        check(gh[:, :, :nv], ref_[:, :, :nv], what)
        assert not gh[:, :, nv:].any(), f"padded rows of {what} must be zero"
    if per_head is None:
        assert len(g) == 3
        return
    dW, db = g[3], g[4]
    check(host(dW), ref[4], "dW")
    if bias:
        check(host(db), ref[5], "db")
    else:
        assert db is None
