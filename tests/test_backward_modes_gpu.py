"""GPU parity of the backward of the SALAD and NSA-style forwards and of GQA maps
(sla_attn_bwd_ext through the C-ABI) against the gradient oracle.

The forward runs in training mode on the oracle's block map; dQ, dK, dV (and dw_gate for the
gated SALAD branch) of sum(dO * O) are compared with autograd of the float64 forward, itself
pinned by central finite differences of the numpy oracle, over every valid row.  The bar is the
one of the SLA backward (rel-L2 <= 1e-2 per gradient, max-abs <= 3e-2 of the largest magnitude):
the same bf16 matrix-core operands with fp32 accumulation.  dw_gate sums dlogit q over every
valid row of a head, so it is held to the same relative bar.
"""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_backward as obwd
from tests.gpu_helpers import host, make_case, oracle_csr, say
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    # SALAD: top 10% critical blocks plus the gated linear branch over all keys
    "med_salad": (scaled(W["salad"], "med_salad", grid=(5, 18, 46), Hq=2, Hkv=2), False),
    "med_salad_smoothk": (scaled(W["salad"], "med_salad_smoothk", grid=(4, 9, 20), Hq=2, Hkv=2, d=64), True),
    # SALAD with two query heads per KV head (per-head maps, one all-key state per KV head)
    "gqa_salad": (scaled(W["tiny_sla"], "gqa_salad", mode="salad", Hq=4, Hkv=2, N=1280, Nv=1250, d=128,
                         dtype="bf16", kh_bp=2000, kl_bp=0, gate_seed=7), False),
    # SLA with GQA and per-head maps (dH of a KV head sums its query heads' state gradients)
    "gqa_sla": (scaled(W["tiny_sla"], "gqa_sla", Hq=4, Hkv=2, N=1280, Nv=1250, d=128, dtype="bf16",
                       kh_bp=3000, kl_bp=4000), False),
    "gqa_sla_smoothk_f32": (scaled(W["tiny_sla"], "gqa_sla_smoothk_f32", Hq=2, Hkv=1, N=1024, Nv=1000, d=64,
                                   kh_bp=2500, kl_bp=5000), True),
    # NSA-style causal maps shared by the group: 16 query heads on one KV head, 16 selected
    # blocks and a 512-token window, a ragged tail
    "med_nsa": (scaled(W["nsa_prefill"], "med_nsa", N=4160, Nv=4150), False),
    # a window that ends inside a block, two KV heads
    "nsa_gqa_win200": (scaled(W["nsa_prefill"], "nsa_gqa_win200", N=2048, Nv=2000, Hq=4, Hkv=2, n_sel=4,
                              window=200), False),
    # two sequences: the split dK/dV partials and the gate gradient sum over the batch
    "nsa_gqa_b2": (scaled(W["nsa_prefill"], "nsa_gqa_b2", B=2, N=1024, Nv=1000, Hq=4, Hkv=1, n_sel=3,
                          window=150), False),
    "gqa_salad_b2": (scaled(W["tiny_sla"], "gqa_salad_b2", mode="salad", B=2, Hq=4, Hkv=2, N=640, Nv=600,
                            d=64, dtype="bf16", kh_bp=2000, kl_bp=0, gate_seed=11), False),
    # selection only (no window), fp32 inputs, d = 64
    "nsa_sel_only_f32_d64": (scaled(W["nsa_prefill"], "nsa_sel_only_f32_d64", N=1024, Nv=1000, Hq=2, Hkv=1,
                                    d=64, dtype="f32", n_sel=3, window=0), False),
}
REL_L2, MAX_ABS_FRAC = 1e-2, 3e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


_cache = {}


def run_case(name):
    """GPU gradients, oracle gradients and context for one case, built once."""
    if name in _cache:
        return _cache[name]
    w, smooth_k = CASES[name]
    q, k, v, wg, f, layer = make_case(w, smooth_k=smooth_k, training=True)
    csr, maps = oracle_csr(f)
    r = np.random.default_rng(123)
    dO = torch.from_numpy(r.standard_normal(q.shape).astype(np.float32)).to(q.dtype)
    dO[:, :, w.Nv:] = 5.0                              # padded rows of dO must not matter
    layer.pool_scores()
    layer.kv_reduce()
    if w.mode == "sla":
        layer.marginal_states(maps=csr)
    layer.attention(maps=csr)
    got = layer.backward(dO.cuda(), maps=csr)
    torch.cuda.synchronize()
    got = tuple(host(x) for x in got)
    ref = obwd.gradients(f.Q, f.K, f.V, host(dO).astype(np.float64), maps, w.Nv, f.scale, smooth_k=smooth_k,
                         mode=w.mode, w_gate=None if wg is None else wg.numpy(), window=w.window,
                         group_map=w.mode == "nsa")
    _cache[name] = (w, layer, dO, csr, got, ref)
    return _cache[name]


def check(g_, r_, what, nv=None):
    sl = (slice(None), slice(None), slice(0, nv)) if nv is not None else (slice(None),)
    diff = g_[sl].astype(np.float64) - r_[sl]
    rel = np.linalg.norm(diff) / max(np.linalg.norm(r_[sl]), 1e-30)
    mx = np.abs(diff).max() / max(np.abs(r_[sl]).max(), 1e-30)
    say(f"  {what}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
    assert rel <= REL_L2, (what, rel)
    assert mx <= MAX_ABS_FRAC, (what, mx)


@pytest.mark.parametrize("name", list(CASES))
def test_gradients(name):
    say(f"[backward] {name}")
    w, layer, dO, csr, got, ref = run_case(name)
    nv = w.Nv
    assert got[0].shape == (w.B, w.Hq, w.N, w.d) and got[1].shape == (w.B, w.Hkv, w.N, w.d)
    for g_, r_, what in zip(got[:3], ref[1:4], ("dQ", "dK", "dV")):
        check(g_, r_, what, nv)
        assert not g_[:, :, nv:].any(), f"padded rows of {what} must be zero"
    if w.mode == "salad":
        check(got[3], ref[4], "dw_gate")


@pytest.mark.parametrize("name", ["med_salad", "nsa_gqa_win200"])
def test_backward_is_deterministic(name):
    say(f"[backward determinism] {name}")
    w, layer, dO, csr, got, ref = run_case(name)
    again = layer.backward(dO.cuda(), maps=csr)
    torch.cuda.synchronize()
    for a, b_ in zip(again, got):
        assert np.array_equal(host(a), b_)


def test_mha_entry_matches_extended_entry():
    """sla_attn_bwd is the row-states mode of sla_attn_bwd_ext: bit-identical gradients."""
    say("[backward entry points] gqa_sla_smoothk_f32 as MHA")
    w = scaled(W["tiny_sla"], "mha_sla", Hq=2, Hkv=2, N=1024, Nv=1000, d=64, kh_bp=2500, kl_bp=5000)
    q, k, v, wg, f, layer = make_case(w, smooth_k=True, training=True)
    csr, maps = oracle_csr(f)
    dO = torch.from_numpy(np.random.default_rng(5).standard_normal(q.shape).astype(np.float32)).cuda()
    layer.pool_scores()
    layer.kv_reduce()
    S, u = layer.marginal_states(maps=csr)
    O = layer.attention(maps=csr)
    ext = layer.backward(dO, maps=csr)
    mha = sla.sla_attn_bwd(layer.q, layer.k, layer.v, O, dO, layer.lse, w.Nv, csr, S, u, scale=layer.scale,
                           k_shift=layer.k_mean)
    torch.cuda.synchronize()
    for a, b_ in zip(ext, mha):
        assert torch.equal(a, b_)
