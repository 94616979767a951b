"""GPU parity of the learned Proj on the linear branch and of smooth-K, through the C-ABI.

Proj (O = O_s + O_l W^T + b, weights shared or per head) and the smooth-K key shift (keys of
the linear branch minus their mean over the valid tokens of each head) are compared with the
oracle on seeded inputs and random weights: the key mean to fp32 rounding of the pooled block
means it is taken from, the shifted key states within bf16-operand rounding, and outputs within
rel-L2 1e-2 and max-abs 3e-2 over every valid row (given the oracle's block map).
"""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_oracle as orc
from tests.gpu_helpers import compare_outputs, host, make_case, oracle_csr, say
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    "tiny_sla": W["tiny_sla"],
    "med_sla": scaled(W["wan13b_sla"], "med_sla", grid=(5, 18, 46), Hq=2, Hkv=2, kh_bp=2500, kl_bp=5000),
    "med_sla_d64": scaled(W["wan13b_sla"], "med_sla_d64", grid=(4, 9, 20), Hq=2, Hkv=2, d=64, kh_bp=1500,
                          kl_bp=6000),
    "med_gqa_sla": scaled(W["tiny_sla"], "med_gqa_sla", Hq=4, Hkv=2, N=1280, Nv=1250, d=128, dtype="bf16",
                          kh_bp=3000, kl_bp=4000),
    "med_salad": scaled(W["salad"], "med_salad", grid=(5, 18, 46), Hq=2, Hkv=2),
}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def proj_weights(w, per_head, bias, seed):
    r = np.random.default_rng(seed)
    shape = (w.Hq, w.d, w.d) if per_head else (w.d, w.d)
    Wp = (r.standard_normal(shape) / np.sqrt(w.d)).astype(np.float32)
    bp = None
    if bias:
        bp = (0.5 * r.standard_normal(shape[:-1])).astype(np.float32)
    return Wp, bp


@pytest.mark.parametrize("name", list(CASES))
def test_key_mean(name):
    say(f"[key mean] {name}")
    w = CASES[name]
    q, k, v, wg, f, layer = make_case(w)
    out = layer.pool_scores()
    km = host(sla.sla_key_mean(out["k_pool"], w.Nv))
    torch.cuda.synchronize()
    kp = host(out["k_pool"])
    ref = np.stack([np.stack([orc.key_mean(f.K[b, g], w.Nv) for g in range(f.Hkv)]) for b in range(f.B)])
    # taken from the fp32-rounded block means: error <= 2^-24 max|k_pool| per term, plus the final rounding
    err = np.abs(km.astype(np.float64) - ref).max()
    say(f"  max-abs {err:.2e}")
    assert err <= 2.0 ** -22 * (np.abs(kp).max() + np.abs(ref).max())


@pytest.mark.parametrize("name", ["tiny_sla", "med_sla", "med_sla_d64", "med_gqa_sla"])
def test_shifted_key_states(name):
    say(f"[smooth-K key states] {name}")
    w = CASES[name]
    q, k, v, wg, f, layer = make_case(w)
    out = layer.pool_scores()
    km = sla.sla_key_mean(out["k_pool"], w.Nv)
    kv = sla.sla_linear_kv_reduce(layer.k, layer.v, w.Nv, per_block=True, want_all=True, k_shift=km)
    torch.cuda.synchronize()
    H, z = orc.kv_states(f.K, f.V, w.Nv, smooth_k=True)
    H = np.swapaxes(H, -1, -2)      # the library stores each state V-feature major, [c][r]
    for got, ref, what, bound in [(kv["H"], H, "H", 5e-3), (kv["z"], z, "z", 3e-3),
                                  (kv["H_all"], H.sum(2), "H_all", 3e-3), (kv["z_all"], z.sum(2), "z_all", 3e-3)]:
        g = host(got).astype(np.float64)
        rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
        say(f"  {what}: rel-L2 {rel:.2e}")
        # as for the unshifted states: bf16 operands (and bf16 per-block storage)
        assert rel < bound, what


PROJ_CASES = [("med_sla", True, True, False), ("med_sla", False, False, True), ("med_sla_d64", True, True, True),
              ("med_gqa_sla", True, True, True), ("tiny_sla", False, True, True)]


@pytest.mark.parametrize("name,per_head,bias,smooth", PROJ_CASES)
def test_sla_proj_smooth_k_given_oracle_map(name, per_head, bias, smooth):
    say(f"[Proj / smooth-K] {name} per_head={per_head} bias={bias} smooth_k={smooth}")
    w = CASES[name]
    Wp, bp = proj_weights(w, per_head, bias, seed=7 + len(name))
    q, k, v, wg, f, layer = make_case(w, proj_w=Wp, proj_b=bp, smooth_k=smooth)
    csr, _ = oracle_csr(f)
    layer.pool_scores()
    layer.kv_reduce()
    layer.marginal_states(maps=csr)
    O = host(layer.attention(maps=csr))
    torch.cuda.synchronize()
    ref = f.output()
    compare_outputs(O[:, :, :w.Nv], ref[:, :, :w.Nv], name)
    assert not O[:, :, w.Nv:].any(), "padded query rows must be zero"
    # the one-call marginal mode runs the same epilogue
    O1 = sla.sla_attn_fwd(layer.q, layer.k, layer.v, w.Nv, csr, lin_mode=sla.SLA_LIN_MARGINAL, H=layer.kv["H"],
                          z=layer.kv["z"], proj_w=layer.proj_w, proj_b=layer.proj_b)
    torch.cuda.synchronize()
    compare_outputs(host(O1)[:, :, :w.Nv], ref[:, :, :w.Nv], name + " one call")


def test_zero_proj_weight_is_sparse_branch_plus_bias():
    say("[Proj W = 0] med_sla")
    w = CASES["med_sla"]
    bp = np.linspace(-1.0, 1.0, w.d).astype(np.float32)
    q, k, v, wg, f, layer = make_case(w, proj_w=np.zeros((w.d, w.d), np.float32), proj_b=bp)
    O = host(layer.run())
    torch.cuda.synchronize()
    ws = scaled(w, "med_sla_sparse_only", kl_bp=10000)      # every non-critical block negligible
    _, _, _, _, fs, layer_s = make_case(ws)
    Os = host(layer_s.run())
    torch.cuda.synchronize()
    # same inputs and critical lists: W = 0 leaves the sparse branch plus b, up to the two bf16
    # output roundings (half an ulp each, 2^-8 relative)
    err = np.abs(O[:, :, :w.Nv] - Os[:, :, :w.Nv] - bp).max()
    say(f"  max-abs vs sparse branch + b: {err:.2e}")
    assert err <= 2.0 ** -7 * (np.abs(Os).max() + np.abs(bp).max())


def test_salad_smooth_k_end_to_end():
    say("[smooth-K] med_salad end to end")
    w = CASES["med_salad"]
    q, k, v, wg, f, layer = make_case(w, smooth_k=True)
    O = host(layer.run())
    torch.cuda.synchronize()
    compare_outputs(O[:, :, :w.Nv], f.output()[:, :, :w.Nv], "med_salad smooth-K")
