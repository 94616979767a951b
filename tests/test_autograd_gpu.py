"""GPU tests of sla_attention, the differentiable layer forward (torch autograd over
SlaForward.run and sla_attn_bwd_ext through the C-ABI).

For each case the layer also runs directly (SlaForward with training=True, then backward());
its block map is checked equal to the oracle's own map, its output and gradients against the
gradient oracle (autograd of the float64 forward on that map, pinned by finite differences of
the numpy oracle) at the backward's bar (rel-L2 <= 1e-2, max-abs <= 3e-2 of the largest
magnitude), and the autograd path must reproduce the direct path bit for bit: the same kernels
on the same inputs, deterministic.  Cases: SLA with a per-head Proj weight and bias (gradients for
q, k, v, proj_w, proj_b), SALAD with GQA (q, k, v, w_gate), the NSA-style causal map with a
window (q, k, v).
"""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_backward as obwd
from tests.gpu_helpers import host, make_case, oracle_csr, say
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    "sla_proj_per_head": scaled(W["wan13b_sla"], "ag_sla", grid=(3, 10, 30), Hq=2, Hkv=2, kh_bp=2500, kl_bp=5000),
    "salad_gqa": scaled(W["tiny_sla"], "ag_salad", mode="salad", B=2, Hq=4, Hkv=2, N=640, Nv=600, d=64,
                        dtype="bf16", kh_bp=2000, kl_bp=0, gate_seed=11),
    "nsa_window": scaled(W["nsa_prefill"], "ag_nsa", N=2048, Nv=2000, Hq=4, Hkv=2, n_sel=4, window=200),
}
REL_L2, MAX_ABS_FRAC = 1e-2, 3e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def check(got, ref, what):
    diff = got.astype(np.float64) - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(diff).max() / max(np.abs(ref).max(), 1e-30)
    say(f"  {what}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
    assert rel <= REL_L2, (what, rel)
    assert mx <= MAX_ABS_FRAC, (what, mx)


@pytest.mark.parametrize("name", list(CASES))
def test_autograd_matches_direct_backward_and_oracle(name):
    w = CASES[name]
    say(f"[sla_attention autograd] {name}")
    Wp = bp = None
    if w.mode == "sla":
        r = np.random.default_rng(41)
        Wp = (r.standard_normal((w.Hq, w.d, w.d)) / np.sqrt(w.d)).astype(np.float32)
        bp = (0.5 * r.standard_normal((w.Hq, w.d))).astype(np.float32)
    q, k, v, wg, f, layer = make_case(w, proj_w=Wp, proj_b=bp, training=True)
    csr, maps = oracle_csr(f)
    r = np.random.default_rng(99)
    dO = torch.from_numpy(r.standard_normal(q.shape).astype(np.float32)).to(q.dtype)
    dO[:, :, w.Nv:] = 5.0                              # padded rows of dO must not matter
    dO = dO.cuda()

    # the direct path: its own map (equal to the oracle's), output and gradients
    out_d = layer.run()
    g_d = layer.backward(dO)
    torch.cuda.synchronize()
    for key in ("crit_rowptr", "crit_idx", "crit_flags"):
        n = int(layer.maps["crit_rowptr"][-1])
        a, b_ = layer.maps[key], csr[key]
        if key != "crit_rowptr":
            a, b_ = a[:n], b_[:n]
        assert torch.equal(a.cpu(), b_.cpu()), f"{key} differs from the oracle's map"

    # the autograd path on leaf tensors
    leaf = lambda x: None if x is None else x.detach().clone().cuda().requires_grad_(True)
    qa, ka, va = leaf(q), leaf(k), leaf(v)
    wga = leaf(wg)
    pwa, pba = leaf(None if Wp is None else torch.from_numpy(Wp)), leaf(None if bp is None else torch.from_numpy(bp))
    out_a = sla.sla_attention(qa, ka, va, w.Nv, w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp, n_sel=w.n_sel,
                              window=w.window, w_gate=wga, proj_w=pwa, proj_b=pba)
    assert out_a.requires_grad and out_a.dtype == q.dtype and out_a.shape == q.shape
    out_a.backward(dO)
    torch.cuda.synchronize()
    assert torch.equal(out_a.detach(), out_d), "autograd forward differs from SlaForward.run"
    assert qa.grad.dtype == q.dtype and ka.grad.shape == k.shape and va.grad.shape == v.shape
    for got, ref, what in zip((qa.grad, ka.grad, va.grad), g_d[:3], ("dQ", "dK", "dV")):
        assert torch.equal(got, ref.to(got.dtype)), f"autograd {what} differs from SlaForward.backward"
    extra = list(g_d[3:])
    if Wp is not None:
        assert torch.equal(pwa.grad, extra[0]) and torch.equal(pba.grad, extra[1])
    if wg is not None:
        assert torch.equal(wga.grad.cpu(), extra[-1].cpu())

    # the direct path against the gradient oracle on the same (oracle) map
    ref = obwd.gradients(f.Q, f.K, f.V, host(dO).astype(np.float64), maps, w.Nv, f.scale, proj_w=Wp, proj_b=bp,
                         with_proj_grads=Wp is not None, mode=w.mode, w_gate=None if wg is None else wg.numpy(),
                         window=w.window, group_map=w.mode == "nsa")
    nv = w.Nv
    check(host(out_d)[:, :, :nv], ref[0][:, :, :nv], "O")
    for got, r_, what in zip(g_d[:3], ref[1:4], ("dQ", "dK", "dV")):
        gh = host(got)
        check(gh[:, :, :nv], r_[:, :, :nv], what)
        assert not gh[:, :, nv:].any(), f"padded rows of {what} must be zero"
    if Wp is not None:
        check(host(extra[0]), ref[4], "dW")
        check(host(extra[1]), ref[5], "db")
    if wg is not None:
        check(host(extra[-1]), ref[-1], "dw_gate")


def test_autograd_catches_an_inplace_change_of_the_output():
    w = CASES["nsa_window"]
    say("[sla_attention autograd] in-place change of the output")
    q, k, v, _ = make_inputs(w)
    qa = q.cuda().requires_grad_(True)
    out = sla.sla_attention(qa, k.cuda(), v.cuda(), w.Nv, "nsa", n_sel=w.n_sel, window=w.window)
    out.add_(1.0)
    with pytest.raises(RuntimeError):
        out.backward(torch.ones_like(out))


def test_no_grad_gives_the_same_output():
    """Without anything to differentiate the plain forward runs: the same bits, no graph."""
    w = CASES["salad_gqa"]
    say("[sla_attention autograd] no_grad")
    q, k, v, wg = make_inputs(w)
    args = (q.cuda(), k.cuda(), v.cuda(), w.Nv, "salad")
    kw = dict(kh_bp=w.kh_bp, w_gate=wg.cuda())
    with torch.no_grad():
        plain = sla.sla_attention(*args, **kw)
    qa = args[0].clone().requires_grad_(True)
    tracked = sla.sla_attention(qa, *args[1:], **kw)
    torch.cuda.synchronize()
    assert not plain.requires_grad and tracked.requires_grad
    assert torch.equal(plain, tracked.detach())


def test_autograd_with_smooth_k_and_token_order_matches_direct():
    """The options pass through: smooth-K and a Hilbert token order (the library's own order of the
    latent grid), gradients bit for bit those of SlaForward.backward."""
    w = scaled(W["wan13b_sla"], "ag_sla_order", grid=(3, 10, 30), Hq=2, Hkv=2, kh_bp=2500, kl_bp=5000)
    say("[sla_attention autograd] smooth-K + token order")
    q, k, v, _ = make_inputs(w)
    order = sla.sla_hilbert_order(*w.grid)
    kw = dict(kh_bp=w.kh_bp, kl_bp=w.kl_bp, smooth_k=True, token_order=order)
    dO = torch.from_numpy(np.random.default_rng(5).standard_normal(q.shape).astype(np.float32)).to(q.dtype).cuda()
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "sla", training=True, **kw)
    out_d = layer.run()
    g_d = layer.backward(dO)
    leaf = lambda x: x.detach().clone().cuda().requires_grad_(True)
    qa, ka, va = leaf(q), leaf(k), leaf(v)
    out_a = sla.sla_attention(qa, ka, va, w.Nv, "sla", **kw)
    out_a.backward(dO)
    torch.cuda.synchronize()
    assert torch.equal(out_a.detach(), out_d)
    for got, ref in zip((qa.grad, ka.grad, va.grad), g_d[:3]):
        assert torch.equal(got, ref.to(got.dtype))
