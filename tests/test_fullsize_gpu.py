"""Full-size parity, in the launch configuration bench.py times (SlaForward.run on the whole
workload): sampled query blocks are recomputed one by one by the oracle, and properties that
hold at any size are checked on every row.

Sampled blocks: first, second, middle, the last two (the last one holds the padding), and
two seeded random ones, on the first, middle and last head.
"""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from oracle import sla_backward as obwd
from oracle import sla_oracle as orc
from tests.gpu_helpers import (MAX_ABS, REL_L2, gpu_map_rows, host, layer_for, oracle_for, say,
                               ulp_distance)
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def sample_blocks(nb, seed):
    r = np.random.default_rng(seed)
    return sorted(set([0, 1, nb // 2, nb - 2, nb - 1] + r.integers(0, nb, 2).tolist()))


def check_all_rows(w, f, layer):
    """Properties of every map row and of the whole output."""
    Hs = f.Hkv if f.group_sum else f.Hq
    rows = w.B * Hs * f.nb
    cr = layer.maps["crit_rowptr"].cpu().numpy().astype(np.int64)
    ci = layer.maps["crit_idx"].cpu().numpy()[:cr[-1]]
    cf = layer.maps["crit_flags"].cpu().numpy()[:cr[-1]]
    rc = layer.maps["row_counts"].cpu().numpy()
    assert cr[0] == 0 and np.all(np.diff(cr) == rc[:, 0])
    i_of_row = np.tile(np.arange(f.nb), w.B * Hs)
    if f.causal:
        assert np.all(rc.sum(1) == i_of_row + 1)
        assert np.all(rc[:, 0] >= np.minimum(i_of_row + 1, f.n_sel))
        assert np.all(rc[:, 0] <= np.minimum(i_of_row + 1, f.n_sel + 9))
    else:
        assert np.all(rc.sum(1) == f.nb)
        assert np.all(rc[:, 0] == f.n_h)
    # ascending, in range, causal
    row_of = np.repeat(np.arange(rows), np.diff(cr))
    same = row_of[1:] == row_of[:-1]
    assert np.all(ci[1:][same] > ci[:-1][same])
    assert ci[:cr[-1]].min() >= 0 and ci[:cr[-1]].max() < f.nb
    if f.causal:
        assert np.all(ci[:cr[-1]] <= i_of_row[row_of])
        assert np.all((cf[:cr[-1]] >= 1) & (cf[:cr[-1]] <= 3))
    if "marg_idx" in layer.maps:
        mr = layer.maps["marg_rowptr"].cpu().numpy().astype(np.int64)
        mi = layer.maps["marg_idx"].cpu().numpy()
        assert np.all(np.diff(mr) == rc[:, 1])
        # disjoint critical / marginal per row: mark per-row membership
        mark = np.zeros((rows, f.nb), np.int8)
        mark[row_of, ci[:cr[-1]]] += 1
        mrow = np.repeat(np.arange(rows), np.diff(mr))
        mark[mrow, mi[:mr[-1]]] += 1
        assert mark.max() == 1


@pytest.mark.parametrize("name", ["wan13b_sla", "salad", "nsa_prefill", "wan14b_sla"])
def test_full_size_sampled(name):
    w = WORKLOADS[name]
    say(f"[full size] {name}: generating inputs")
    q, k, v, wg = make_inputs(w)
    layer = layer_for(w, q, k, v, wg)
    say(f"[full size] {name}: running the layer")
    O = layer.run()
    torch.cuda.synchronize()
    f = oracle_for(w, q, k, v, wg)
    del q, k, v
    say(f"[full size] {name}: whole-map properties")
    check_all_rows(w, f, layer)
    Og = layer.out
    assert torch.isfinite(Og).all()
    assert not Og[:, :, w.Nv:].any()
    Hs = f.Hkv if f.group_sum else f.Hq
    scores = layer.pool["scores"]
    heads = sorted(set([0, w.Hq // 2, w.Hq - 1]))
    diffs, refs_ = [], []
    n_rows = 0
    for h in heads:
        hs = f.map_head(h)
        blocks = sample_blocks(f.nb, 1000 * h + w.seed)
        got_rows = gpu_map_rows(layer.maps, [hs * f.nb + i for i in blocks])
        for i in blocks:
            m = f.map_row(0, hs, i)
            srow = host(scores[0, hs, i])
            fin = np.isfinite(m["scores"])
            assert np.array_equal(np.isfinite(srow), fin)
            assert ulp_distance(srow[fin], m["scores"][fin]).max() <= 1
            crit, flags, marg, counts = got_rows[hs * f.nb + i]
            assert crit == m["crit"] and flags == m["flags"], (h, i)
            if marg is not None and not f.mode == "salad":
                assert marg == m["marg"], (h, i)
            ref = f.output_block(0, h, i, m)
            got = host(Og[0, h, 64 * i:64 * i + 64]).astype(np.float64)
            diffs.append(got - ref)
            refs_.append(ref)
            n_rows += 1
    d = np.concatenate(diffs)
    r = np.concatenate(refs_)
    rel = np.linalg.norm(d) / np.linalg.norm(r)
    mx = np.abs(d).max()
    say(f"  {name}: {n_rows} sampled blocks, rel-L2 {rel:.3e}, max-abs {mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def test_full_size_backward_sampled():
    """The backward at the wan13b layer, in the configuration bench.py --backward times: dQ rows of
    sampled query blocks and dK / dV rows of sampled key blocks, each recomputed by the gradient
    oracle from exactly the query blocks that depend on them, on the first and last head."""
    w = WORKLOADS["wan13b_sla"]
    say("[full size backward] generating inputs")
    q, k, v, wg = make_inputs(w)
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "sla", kh_bp=w.kh_bp, kl_bp=w.kl_bp, training=True)
    layer.run()
    r = np.random.default_rng(w.seed + 17)
    dO = torch.from_numpy(r.standard_normal(q.shape, dtype=np.float32)).to(torch.bfloat16)
    dq, dk, dv = layer.backward(dO.cuda())
    torch.cuda.synchronize()
    f = oracle_for(w, q, k, v, wg)
    nb, nv = f.nb, w.Nv
    for h in [0, w.Hq - 1]:
        say(f"[full size backward] head {h}: oracle map")
        maps_h = {(0, 0, i): f.map_row(0, h, i) for i in range(nb)}
        got_rows = gpu_map_rows(layer.maps, [h * nb + i for i in range(nb)])
        for i in range(nb):
            crit, _, marg, _ = got_rows[h * nb + i]
            assert crit == maps_h[(0, 0, i)]["crit"] and marg == maps_h[(0, 0, i)]["marg"], (h, i)
        Qh, Kh, Vh = (X[:, h:h + 1] for X in (f.Q, f.K, f.V))
        dOh = host(dO[:, h:h + 1]).astype(np.float64)
        gq, gk, gv = (host(X[0, h]) for X in (dq, dk, dv))
        diffs = {"dQ": [], "dK": [], "dV": []}
        refs_ = {"dQ": [], "dK": [], "dV": []}
        qblocks = sample_blocks(nb, 7 + h)
        _, dQr, _, _ = obwd.gradients(Qh, Kh, Vh, dOh, maps_h, nv, f.scale, blocks={(0, 0, i) for i in qblocks})
        for i in qblocks:
            rows = slice(64 * i, min(64 * i + 64, nv))
            diffs["dQ"].append(gq[rows] - dQr[0, 0, rows])
            refs_["dQ"].append(dQr[0, 0, rows])
        for j in [0, nb // 2, nb - 1]:
            users = {key for key, m in maps_h.items() if j in m["crit"] or j in m["marg"]}
            say(f"  key block {j}: {len(users)} query blocks use it")
            _, _, dKr, dVr = obwd.gradients(Qh, Kh, Vh, dOh, maps_h, nv, f.scale, blocks=users)
            rows = slice(64 * j, min(64 * j + 64, nv))
            for name, g_, r_ in (("dK", gk, dKr), ("dV", gv, dVr)):
                diffs[name].append(g_[rows] - r_[0, 0, rows])
                refs_[name].append(r_[0, 0, rows])
        for name in diffs:
            d_ = np.concatenate(diffs[name])
            r_ = np.concatenate(refs_[name])
            rel = np.linalg.norm(d_) / np.linalg.norm(r_)
            mx = np.abs(d_).max() / np.abs(r_).max()
            say(f"  head {h} {name}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
            assert rel <= REL_L2 and mx <= 3e-2, (h, name)
    assert not dq[:, :, nv:].any() and not dk[:, :, nv:].any() and not dv[:, :, nv:].any()
