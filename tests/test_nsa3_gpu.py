"""GPU parity of three-branch NSA (sla_nsa3_fwd, through the C-ABI) against the oracle.

Medium cases compare every valid row (rel-L2 <= 1e-2, max-abs <= 3e-2), with the selection map
built by the library from the oracle's own group-summed scores (bit-exact map parity is covered by
the block-map tests) and checked equal to the oracle's selection; the full 65536-token prefill
compares sampled rows of sampled heads.  Gate weights are seeded random (and zero in one case).
"""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_oracle as orc
from tests.gpu_helpers import MAX_ABS, REL_L2, compare_outputs, gpu_map_rows, host, say, to_dev
from workloads import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


W0 = WORKLOADS["nsa_prefill"]
CASES = {
    "med_nsa3": (scaled(W0, "med_nsa3", N=4160, Nv=4150), 512, False),
    "med_nsa3_hq4": (scaled(W0, "med_nsa3_hq4", N=2048, Nv=2048, Hq=4), 512, False),
    "med_nsa3_nowin_zero_gates": (scaled(W0, "med_nsa3_nw", N=1280, Nv=1250, Hq=4), 0, True),
    "med_nsa3_d64_f32": (scaled(W0, "med_nsa3_d64", N=1024, Nv=1000, Hq=4, d=64, dtype="f32"), 200, False),
    "short_nsa3": (scaled(W0, "short_nsa3", N=64, Nv=20, Hq=4), 512, False),
}


def gate_weights(w, zero, seed):
    if zero:
        return np.zeros((3, w.Hq, w.d), np.float32)
    return (np.random.default_rng(seed).standard_normal((3, w.Hq, w.d)) / np.sqrt(w.d)).astype(np.float32)


def run_gpu(w, q, k, v, wg, window):
    """The layer's selection (pool + scores + causal top-n_sel map without window), then the three branches."""
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "nsa", n_sel=w.n_sel, window=0)
    layer.pool_scores()
    layer.block_map()
    out = sla.sla_nsa3_fwd(layer.q, layer.k, layer.v, w.Nv, layer.maps, to_dev(wg, torch.float32), window=window,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    return layer, host(out)


@pytest.mark.parametrize("name", list(CASES))
def test_nsa3_medium(name):
    w, window, zero = CASES[name]
    say(f"[nsa3] {name}: Hq {w.Hq} N {w.N} n_valid {w.Nv} d {w.d} window {window}")
    q, k, v, _ = make_inputs(w)
    wg = gate_weights(w, zero, 11)
    layer, O = run_gpu(w, q, k, v, wg, window)
    Q, K, V = (host(x) for x in (q, k, v))
    f = orc.Forward(Q, K, V, n_valid=w.Nv, mode="nsa", n_sel=w.n_sel, window=0)
    got = gpu_map_rows(layer.maps, range(w.Hkv * f.nb))
    for r_, (crit, flags, _, _) in got.items():
        g, i = divmod(r_, f.nb)
        assert crit == f.map_row(0, g, i)["crit"], (g, i)
    ref = orc.nsa3_forward(Q, K, V, n_valid=w.Nv, n_sel=w.n_sel, window=window, cmp_block=32, cmp_stride=16,
                           w_gates=wg)
    compare_outputs(O[:, :, :w.Nv], ref[:, :, :w.Nv], name)
    assert not O[:, :, w.Nv:].any()


def test_nsa3_full_prefill_sampled():
    w = W0
    say("[nsa3 full size] nsa_prefill: generating inputs")
    q, k, v, _ = make_inputs(w)
    wg = gate_weights(w, False, 12)
    layer, O = run_gpu(w, q, k, v, wg, 512)
    Q, K, V = (host(x) for x in (q, k, v))
    r = np.random.default_rng(13)
    rows = sorted(set([0, 1, 30, 31, 47, 63, 64, 511, 512, 513, 4095, w.Nv - 1] + r.integers(0, w.Nv, 20).tolist()))
    heads = [0, 7, 15]
    say(f"[nsa3 full size] oracle on {len(rows)} rows x {len(heads)} heads")
    ref = orc.nsa3_forward(Q, K, V, n_valid=w.Nv, n_sel=w.n_sel, window=512, cmp_block=32, cmp_stride=16,
                           w_gates=wg, heads=heads, rows=rows)
    got = O[:, heads][:, :, rows]
    exp = ref[:, heads][:, :, rows]
    d_ = got.astype(np.float64) - exp
    rel = np.linalg.norm(d_) / np.linalg.norm(exp)
    mx = np.abs(d_).max()
    say(f"  sampled rows: rel-L2 {rel:.3e}, max-abs {mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS
    assert np.isfinite(O).all()
