"""Full-size parity, in the launch configuration bench.py times (SlaForward.run on the whole
workload).

Every row of every workload: pooled scores within one fp32 ulp of the oracle's, and the block map
(critical lists and flags, marginal lists and bit masks, row counts) bit for bit against the
oracle's classification of the same scores, plus properties that hold at any size.  Outputs: every
valid row of wan13b_sla, salad and nsa_prefill recomputed by the oracle; for wan14b_sla every valid
row of four of its 40 heads and sampled query blocks of the middle head (first, second, middle, the
last two (the last one holds the padding), and two seeded random ones).  Backward: wan13b_sla and
salad on every valid row of two heads, nsa_prefill on sampled blocks.
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


def marg_bits_from_csr(rowptr, idx, rows, nkb):
    """Bit masks (bit j % 32 of word j / 32) of CSR marginal lists, as int32 words."""
    bits = np.zeros((rows, (nkb + 31) // 32), dtype=np.uint32)
    n = int(rowptr[-1])
    row_of = np.repeat(np.arange(rows), np.diff(rowptr))
    j = np.asarray(idx[:n], dtype=np.int64)
    np.bitwise_or.at(bits, (row_of, j // 32), (np.uint32(1) << (j % 32).astype(np.uint32)))
    return bits.view(np.int32)


def check_maps_every_row(w, f, layer):
    """Every row: the pooled scores against the oracle's (within one fp32 ulp), and the GPU's block
    map bit for bit against the oracle's classification of the GPU's own scores (the scores the map
    was built from).  Returns the oracle's per-row maps (used for the output comparison)."""
    Hs = f.Hkv if f.group_sum else f.Hq
    rows = w.B * Hs * f.nb
    Sg = host(layer.pool["scores"])
    say(f"  oracle pooling and scores of all {rows} rows")
    S_own = orc.pooled_scores(orc.pool(f.Q, w.Nv), orc.pool(f.K, w.Nv), f.scale, group_sum=f.group_sum,
                              causal=f.causal)
    assert np.array_equal(np.isneginf(Sg), np.isneginf(S_own))
    fin = np.isfinite(S_own)
    ulp = ulp_distance(Sg[fin], S_own[fin])
    say(f"  scores: {np.count_nonzero(ulp)} of {ulp.size} differ, max {ulp.max()} ulp")
    assert ulp.max() <= 1
    say(f"  oracle classification of every row of the GPU's scores")
    maps = orc.block_map(Sg, n_h=f.n_sel if f.causal else f.n_h, n_l=f.n_l, causal=f.causal, n_sel=f.n_sel,
                         window=f.window)
    ref = orc.to_csr(maps, w.B, Hs, f.nb)
    cr = layer.maps["crit_rowptr"].cpu().numpy()
    n = int(cr[-1])
    assert np.array_equal(cr, ref["crit_rowptr"])
    assert np.array_equal(layer.maps["crit_idx"].cpu().numpy()[:n], ref["crit_idx"])
    assert np.array_equal(layer.maps["crit_flags"].cpu().numpy()[:n], ref["crit_flags"])
    assert np.array_equal(layer.maps["row_counts"].cpu().numpy(), ref["row_counts"])
    if "marg_rowptr" in layer.maps:
        mr = layer.maps["marg_rowptr"].cpu().numpy()
        assert np.array_equal(mr, ref["marg_rowptr"])
        assert np.array_equal(layer.maps["marg_idx"].cpu().numpy()[:int(mr[-1])], ref["marg_idx"])
        assert np.array_equal(layer.maps["marg_bits"].cpu().numpy(),
                              marg_bits_from_csr(ref["marg_rowptr"], ref["marg_idx"], rows, f.nb))
    say(f"  block map: all {rows} rows bit-exact ({n} critical entries)")
    # diagnostic: rows whose map would change if the oracle used its own scores
    changed = 0
    for r in np.flatnonzero((np.where(fin, Sg, 0) != np.where(fin, S_own, 0)).reshape(rows, -1).any(1)):
        b, rem = divmod(int(r), Hs * f.nb)
        h, i = divmod(rem, f.nb)
        if f.map_row(b, h, i)["crit"] != maps[(b, h, i)]["crit"]:
            changed += 1
    say(f"  rows whose map differs under the oracle's own scores: {changed}")
    return maps


FULL_OUTPUT = {"wan13b_sla", "salad", "nsa_prefill"}     # every valid row recomputed by the oracle
# wan14b: every valid row of these heads, sampled query blocks of the middle head
FULL_HEADS = {"wan14b_sla": [0, 13, 26, 39]}


@pytest.mark.parametrize("name", ["wan13b_sla", "salad", "nsa_prefill", "wan14b_sla"])
def test_full_size(name):
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
    say(f"[full size] {name}: block maps of every row")
    maps = check_maps_every_row(w, f, layer)
    Og = layer.out
    assert torch.isfinite(Og).all()
    assert not Og[:, :, w.Nv:].any()
    if name in FULL_OUTPUT:
        heads = list(range(w.Hq))
        blocks_of = lambda h: list(range(f.nb))
    else:
        heads = sorted(set([0, w.Hq // 2, w.Hq - 1] + FULL_HEADS[name]))
        blocks_of = lambda h: (list(range(f.nb)) if h in FULL_HEADS[name]
                               else sample_blocks(f.nb, 1000 * h + w.seed))
    diffs, refs_ = [], []
    n_rows = 0
    for h in heads:
        hs = f.map_head(h)
        Oh = host(Og[0, h]).astype(np.float64)
        for i in blocks_of(h):
            ref = f.output_block(0, h, i, maps[(0, hs, i)])
            hi = min(64, w.Nv - 64 * i)
            diffs.append(Oh[64 * i:64 * i + hi] - ref[:hi])
            refs_.append(ref[:hi])
            n_rows += hi
        if name in FULL_OUTPUT or h in FULL_HEADS.get(name, []):
            f._H.clear()          # the per-block states of this head are not needed again
    d = np.concatenate(diffs)
    r = np.concatenate(refs_)
    rel = np.linalg.norm(d) / np.linalg.norm(r)
    mx = np.abs(d).max()
    say(f"  {name}: {n_rows} valid rows compared, rel-L2 {rel:.3e}, max-abs {mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS


def test_full_size_backward():
    """The backward at the wan13b layer, in the configuration bench.py --backward times: every valid row
    of dQ, dK and dV against the gradient oracle on the first and last head (the oracle recomputes the
    whole head: its critical softmax branch and its marginal linear branch)."""
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
        say(f"[full size backward] head {h}: oracle gradients of every row")
        _, dQr, dKr, dVr = obwd.gradients(Qh, Kh, Vh, dOh, maps_h, nv, f.scale)
        for name, g_, r_ in (("dQ", dq, dQr), ("dK", dk, dKr), ("dV", dv, dVr)):
            rel, mx = _rel(host(g_[0, h, :nv]).astype(np.float64) - r_[0, 0, :nv], r_[0, 0, :nv])
            say(f"  head {h} {name}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref| ({nv} rows)")
            assert rel <= REL_L2 and mx <= 3e-2, (h, name)
    assert not dq[:, :, nv:].any() and not dk[:, :, nv:].any() and not dv[:, :, nv:].any()


def _rel(d_, r_):
    return np.linalg.norm(d_) / np.linalg.norm(r_), np.abs(d_).max() / np.abs(r_).max()


def test_full_size_backward_salad():
    """The SALAD backward at full size (sla_attn_bwd_ext, gated all-key branch): every valid row of
    dQ, dK, dV and the head's dw_g against the gradient oracle, on the first and last head (each key
    block's gradient depends on every query block through the all-key state, so the whole head is
    recomputed)."""
    w = WORKLOADS["salad"]
    say("[full size backward, salad] generating inputs")
    q, k, v, wg = make_inputs(w)
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "salad", kh_bp=w.kh_bp, w_gate=wg, training=True)
    layer.run()
    r = np.random.default_rng(w.seed + 19)
    dO = torch.from_numpy(r.standard_normal(q.shape, dtype=np.float32)).to(torch.bfloat16)
    dq, dk, dv, dwg = layer.backward(dO.cuda())
    torch.cuda.synchronize()
    f = oracle_for(w, q, k, v, wg)
    nb, nv = f.nb, w.Nv
    for h in [0, w.Hq - 1]:
        maps_h = {(0, 0, i): f.map_row(0, h, i) for i in range(nb)}
        got_rows = gpu_map_rows(layer.maps, [h * nb + i for i in range(nb)])
        for i in range(nb):
            assert got_rows[h * nb + i][0] == maps_h[(0, 0, i)]["crit"], (h, i)
        say(f"[full size backward, salad] head {h}: gradient oracle over the whole head")
        Qh, Kh, Vh = (X[:, h:h + 1] for X in (f.Q, f.K, f.V))
        dOh = host(dO[:, h:h + 1]).astype(np.float64)
        _, dQr, dKr, dVr, dWr = obwd.gradients(Qh, Kh, Vh, dOh, maps_h, nv, f.scale, mode="salad",
                                               w_gate=wg.numpy()[h:h + 1])
        for name, g_, r_ in (("dQ", dq, dQr), ("dK", dk, dKr), ("dV", dv, dVr)):
            rel, mx = _rel(host(g_[0, h, :nv]).astype(np.float64) - r_[0, 0, :nv], r_[0, 0, :nv])
            say(f"  head {h} {name}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
            assert rel <= REL_L2 and mx <= 3e-2, (h, name)
        rel, mx = _rel(host(dwg[h]).astype(np.float64) - dWr[0], dWr[0])
        say(f"  head {h} dw_g: rel-L2 {rel:.3e}, max-abs {mx:.3e}")
        assert rel <= REL_L2 and mx <= 3e-2
    assert not dq[:, :, nv:].any() and not dk[:, :, nv:].any() and not dv[:, :, nv:].any()


def test_full_size_backward_nsa():
    """The NSA-style backward at the full prefill (16 query heads on one KV head, causal selected +
    window maps shared by the group; sla_attn_bwd_ext with the key blocks' heads split over
    workgroups): dQ rows of sampled query blocks on two query heads, and dK / dV rows of sampled key
    blocks recomputed from every (query head, query block) that lists them."""
    w = WORKLOADS["nsa_prefill"]
    say("[full size backward, nsa] generating inputs")
    q, k, v, wg = make_inputs(w)
    layer = sla.SlaForward(q.cuda(), k.cuda(), v.cuda(), w.Nv, "nsa", n_sel=w.n_sel, window=w.window, training=True)
    layer.run()
    r = np.random.default_rng(w.seed + 23)
    dO = torch.from_numpy(r.standard_normal(q.shape, dtype=np.float32)).to(torch.bfloat16)
    dq, dk, dv = layer.backward(dO.cuda())
    torch.cuda.synchronize()
    f = oracle_for(w, q, k, v, wg)
    nb, nv = f.nb, w.Nv
    maps = {(0, 0, i): f.map_row(0, 0, i) for i in range(nb)}
    got_rows = gpu_map_rows(layer.maps, list(range(nb)))
    for i in range(nb):
        assert got_rows[i][0] == maps[(0, 0, i)]["crit"] and got_rows[i][1] == maps[(0, 0, i)]["flags"], i
    dOn = host(dO).astype(np.float64)
    heads = [0, w.Hq - 1]
    qblocks = sample_blocks(nb, 31)
    say(f"[full size backward, nsa] dQ of query blocks {qblocks} on heads {heads}")
    _, dQr, _, _ = obwd.gradients(f.Q, f.K, f.V, dOn, maps, nv, f.scale, mode="nsa", window=w.window,
                                  group_map=True, blocks={(0, h, i) for h in heads for i in qblocks})
    users_of = {j: [i for i in range(nb) if j in maps[(0, 0, i)]["crit"]] for j in range(nb)}
    # the last block (listed only by itself) and the two least-listed of 12 seeded candidates
    cand = sorted(set(np.random.default_rng(37).integers(0, nb - 1, 12).tolist()))
    kblocks = [nb - 1] + sorted(cand, key=lambda j: (len(users_of[j]), j))[:2]
    diffs = {"dQ": [], "dK": [], "dV": []}
    refs_ = {"dQ": [], "dK": [], "dV": []}
    gq, gk, gv = host(dq), host(dk), host(dv)
    for h in heads:
        for i in qblocks:
            rows = slice(64 * i, min(64 * i + 64, nv))
            diffs["dQ"].append(gq[0, h, rows] - dQr[0, h, rows])
            refs_["dQ"].append(dQr[0, h, rows])
    for j in kblocks:
        users = {(0, h, i) for h in range(w.Hq) for i in users_of[j]}
        say(f"  key block {j}: {len(users_of[j])} query blocks x {w.Hq} heads list it")
        _, _, dKr, dVr = obwd.gradients(f.Q, f.K, f.V, dOn, maps, nv, f.scale, mode="nsa", window=w.window,
                                        group_map=True, blocks=users)
        rows = slice(64 * j, min(64 * j + 64, nv))
        for name, g_, r_ in (("dK", gk, dKr), ("dV", gv, dVr)):
            diffs[name].append(g_[0, 0, rows] - r_[0, 0, rows])
            refs_[name].append(r_[0, 0, rows])
    for name in diffs:
        rel, mx = _rel(np.concatenate(diffs[name]), np.concatenate(refs_[name]))
        say(f"  {name}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
        assert rel <= REL_L2 and mx <= 3e-2, name
