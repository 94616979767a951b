"""GPU parity at the degenerate sizes: one 64-token block, a single valid token, a last block with
one valid row, a map with empty marginal lists, and the SALAD / NSA-style modes at one and two
blocks — the whole layer (end to end) and its backward against the oracles, every valid row — and
at the maximum length (4096 key blocks).

The layer's own block map is checked against the oracle's map row for row first; the backward runs
on the oracle's map (as the other backward tests do).  Bars: the output tolerance of the forward
tests, and rel-L2 <= 1e-2 / max-abs <= 3e-2 of the largest gradient for the backward.

One degenerate case is held to a different bar, for a reason the backward shares with every
FlashAttention-style backward: D_t = dO_t . O_t is formed from the stored output.  When a query
block's only critical block holds a single valid key, its softmax is constant and dS = P (dP - D)
vanishes in exact arithmetic, so the block's true dQ is its small linear-branch part and whatever
dP - D leaves over shows up in full.  dP is a matrix-core product of bf16 operands, so D is formed
from dO rounded the same way (fp32 inputs: the cancellation is then exact, checked here at the
ordinary bar).  With a bf16 output the stored O = O_s + O_l is itself rounded after the linear term
is added, so D = dO . (O - O_l) keeps that rounding: a rank-one term along the one key, measured to
match this prediction to 0.1%.  That bf16 case is checked against the case's gradient scale:
max-abs <= 1e-2 of its largest gradient for dQ and dK.
"""
import numpy as np
import pytest
import torch

from oracle import sla_backward as obwd
from tests.gpu_helpers import compare_outputs, gpu_map_rows, host, make_case, oracle_csr, say
from workloads import WORKLOADS, scaled

pytestmark = pytest.mark.gpu

W = WORKLOADS
T = W["tiny_sla"]
CASES = {
    # one block, one valid token: the only key block is critical, nothing marginal
    "one_token_f32_d64": scaled(T, "one_token_f32_d64", N=64, Nv=1, d=64, kh_bp=2500, kl_bp=5000),
    # one full block, bf16, d 128
    "one_block_bf16": scaled(T, "one_block_bf16", N=64, Nv=64, d=128, dtype="bf16", kh_bp=2500, kl_bp=5000),
    # two blocks, the second with one valid row; one critical, one marginal block per row (query
    # block 0's only critical key is token 64)
    "two_blocks_ragged": scaled(T, "two_blocks_ragged", N=128, Nv=65, d=128, kh_bp=5000, kl_bp=0),
    "two_blocks_ragged_bf16": scaled(T, "two_blocks_ragged_bf16", N=128, Nv=65, d=128, dtype="bf16", kh_bp=5000,
                                     kl_bp=0),
    # two blocks, one critical and one negligible: every marginal list is empty
    "no_marginal": scaled(T, "no_marginal", N=128, Nv=100, d=64, kh_bp=5000, kl_bp=5000),
    # SALAD (gated all-key linear) with GQA at one and two blocks
    "salad_one_block": scaled(T, "salad_one_block", mode="salad", N=64, Nv=30, Hq=2, Hkv=1, d=128,
                              dtype="bf16", kh_bp=10000, kl_bp=0, gate_seed=5),
    "salad_two_blocks": scaled(T, "salad_two_blocks", mode="salad", N=128, Nv=70, Hq=2, Hkv=2, d=64,
                               kh_bp=5000, kl_bp=0, gate_seed=6),
    # NSA-style causal maps at one and two blocks (every block selected, the window inside the block)
    "nsa_one_block": scaled(W["nsa_prefill"], "nsa_one_block", N=64, Nv=50, Hq=2, Hkv=1, n_sel=16, window=512),
    "nsa_two_blocks_win": scaled(W["nsa_prefill"], "nsa_two_blocks_win", N=128, Nv=128, Hq=4, Hkv=2, n_sel=1,
                                 window=20),
    # head pairs (an even group shares each staged tile) at d 64 in bf16, a ragged tail
    "nsa_pairs_bf16_d64": scaled(W["nsa_prefill"], "nsa_pairs_bf16_d64", N=320, Nv=300, Hq=4, Hkv=2, d=64,
                                 n_sel=2, window=100),
}
REL_L2_G, MAX_ABS_G = 1e-2, 3e-2
# bf16 cases whose dQ / dK carry the single-key rounding term described above
SINGLE_KEY_BF16 = {"two_blocks_ragged_bf16"}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("name", list(CASES))
def test_layer_end_to_end(name):
    w = CASES[name]
    say(f"[edge forward] {name}: N {w.N}, n_valid {w.Nv}, Hq {w.Hq}, Hkv {w.Hkv}, d {w.d}, {w.dtype}, {w.mode}")
    q, k, v, wg, f, layer = make_case(w)
    O = host(layer.run())
    torch.cuda.synchronize()
    Hs = f.Hkv if f.group_sum else f.Hq
    got = gpu_map_rows(layer.maps, range(w.B * Hs * f.nb))
    for r, (crit, flags, marg, counts) in got.items():
        b, rem = divmod(r, Hs * f.nb)
        h, i = divmod(rem, f.nb)
        m = f.map_row(b, h, i)
        assert crit == m["crit"], (r, crit, m["crit"])
        if marg is not None:
            assert marg == m["marg"], (r, marg, m["marg"])
    assert np.all(np.isfinite(O))
    assert not O[:, :, w.Nv:].any(), "padded rows must be zero"
    compare_outputs(O[:, :, :w.Nv], f.output()[:, :, :w.Nv], name)


@pytest.mark.parametrize("name", list(CASES))
def test_backward(name):
    w = CASES[name]
    say(f"[edge backward] {name}")
    q, k, v, wg, f, layer = make_case(w, training=True)
    csr, maps = oracle_csr(f)
    dO = torch.from_numpy(np.random.default_rng(7).standard_normal(q.shape).astype(np.float32)).to(q.dtype)
    dO[:, :, w.Nv:] = 3.0                              # padded rows of dO must not matter
    layer.pool_scores()
    layer.kv_reduce()
    if w.mode == "sla":
        layer.marginal_states(maps=csr)
    layer.attention(maps=csr)
    got = tuple(host(x) for x in layer.backward(dO.cuda(), maps=csr))
    torch.cuda.synchronize()
    ref = obwd.gradients(f.Q, f.K, f.V, host(dO).astype(np.float64), maps, w.Nv, f.scale, mode=w.mode,
                         w_gate=None if wg is None else wg.numpy(), window=w.window, group_map=w.mode == "nsa")
    nv = w.Nv
    names = ("dQ", "dK", "dV") + (("dw_gate",) if w.mode == "salad" else ())
    refs_ = ref[1:4] + ((ref[4],) if w.mode == "salad" else ())
    rows = (slice(None), slice(None), slice(0, nv))
    gscale = max(np.abs(r_[rows]).max() for r_ in ref[1:4])     # the case's largest gradient
    for g_, r_, what in zip(got, refs_, names):
        sl = (slice(None),) if what == "dw_gate" else rows
        diff = g_[sl].astype(np.float64) - r_[sl]
        rmax = np.abs(r_[sl]).max()
        if name in SINGLE_KEY_BF16 and what in ("dQ", "dK"):
            mx = np.abs(diff).max() / gscale
            rel = np.linalg.norm(diff) / max(np.linalg.norm(r_[sl]), 1e-30)
            say(f"  {what}: max-abs {mx:.3e} of the largest gradient (rel-L2 {rel:.3e} of its own, single-key term)")
            assert mx <= 1e-2, (what, mx)
        elif rmax > 1e-6 * gscale:
            rel = np.linalg.norm(diff) / np.linalg.norm(r_[sl])
            mx = np.abs(diff).max() / rmax
            say(f"  {what}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
            assert rel <= REL_L2_G and mx <= MAX_ABS_G, (what, rel, mx)
        else:
            # an exactly vanishing gradient (a single key: the softmax is constant): what the GPU
            # returns must be rounding-sized next to the case's other gradients
            mx = np.abs(diff).max() / gscale
            say(f"  {what}: reference 0, max |GPU| {mx:.3e} of the largest gradient")
            assert mx <= 1e-2, (what, mx)
        if what != "dw_gate":
            assert not g_[:, :, nv:].any(), f"padded rows of {what} must be zero"


def test_maximum_length():
    """The longest sequence the library takes (4096 key blocks: N = 262144) on one head, bf16 d 128,
    5% critical / 85% negligible: every map row against the oracle's classification of the GPU's
    scores, sampled output blocks (first, second, middle, last two) against the oracle, and the
    backward's dQ on two of those blocks (every key block's gradient is covered at smaller sizes)."""
    from tests.test_fullsize_gpu import check_maps_every_row
    w = scaled(T, "max_len", N=262144, Nv=262144 - 37, d=128, dtype="bf16", kh_bp=500, kl_bp=8500, seed=13)
    say(f"[edge maximum] N {w.N} n_valid {w.Nv}: inputs and the layer")
    q, k, v, wg, f, layer = make_case(w, training=True)
    O = layer.run()
    torch.cuda.synchronize()
    assert f.nb == 4096
    maps = check_maps_every_row(w, f, layer)
    Oh = host(O[0, 0]).astype(np.float64)
    assert np.all(np.isfinite(Oh)) and not Oh[w.Nv:].any()
    blocks = [0, 1, f.nb // 2, f.nb - 2, f.nb - 1]
    got, refs_ = [], []
    for i in blocks:
        ref = f.output_block(0, 0, i, maps[(0, 0, i)])
        hi = min(64, w.Nv - 64 * i)
        got.append(Oh[64 * i:64 * i + hi])
        refs_.append(ref[:hi])
    compare_outputs(np.concatenate(got), np.concatenate(refs_), "max_len sampled blocks")
    say("[edge maximum] backward")
    dO = torch.from_numpy(np.random.default_rng(3).standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16)
    dq, dk, dv = (host(x) for x in layer.backward(dO.cuda()))
    torch.cuda.synchronize()
    for g_ in (dq, dk, dv):
        assert np.all(np.isfinite(g_)) and not g_[:, :, w.Nv:].any()
    qblocks = [1, f.nb - 1]
    _, dQr, _, _ = obwd.gradients(f.Q, f.K, f.V, host(dO).astype(np.float64), maps, w.Nv, f.scale,
                                  blocks={(0, 0, i) for i in qblocks})
    for i in qblocks:
        rows = slice(64 * i, min(64 * i + 64, w.Nv))
        diff = dq[0, 0, rows].astype(np.float64) - dQr[0, 0, rows]
        rel = np.linalg.norm(diff) / np.linalg.norm(dQr[0, 0, rows])
        mx = np.abs(diff).max() / np.abs(dQr[0, 0, rows]).max()
        say(f"  dQ of query block {i}: rel-L2 {rel:.3e}, max-abs {mx:.3e} of max |ref|")
        assert rel <= REL_L2_G and mx <= MAX_ABS_G


def _random_cases(n, seed):
    """Seeded random configurations: batch, heads and grouping, length and its ragged tail, head
    size, dtype, mode and shares (each a valid call of the library)."""
    r = np.random.default_rng(seed)
    out = {}
    for c in range(n):
        mode = ["sla", "salad", "nsa"][c % 3]
        Hkv = int(r.integers(1, 3))
        Hq = Hkv * int(r.choice([1, 2])) if mode != "sla" else Hkv
        nb = int(r.integers(1, 13))
        N = 64 * nb
        Nv = N - int(r.integers(0, 64))
        d = int(r.choice([64, 128]))
        dtype = str(r.choice(["bf16", "f32"]))
        B = int(r.choice([1, 2]))
        name = f"rand{c}_{mode}"
        if mode == "nsa":
            w = scaled(W["nsa_prefill"], name, B=B, Hq=Hq, Hkv=Hkv, N=N, Nv=Nv, d=d, dtype=dtype,
                       n_sel=int(r.integers(1, 5)), window=int(r.choice([0, 37, 200])), seed=100 + c)
        else:
            kh = int(r.integers(0, 10001))
            kl = int(r.integers(0, 10001 - kh)) if mode == "sla" else 0
            w = scaled(T, name, mode=mode, B=B, Hq=Hq, Hkv=Hkv, N=N, Nv=Nv, d=d, dtype=dtype, kh_bp=kh, kl_bp=kl,
                       seed=100 + c, gate_seed=200 + c if mode == "salad" else None)
        out[name] = w
    return out


RANDOM = _random_cases(12, 2024)


@pytest.mark.parametrize("name", list(RANDOM))
def test_random_shapes(name):
    """Forward end to end and backward of a seeded random configuration against the oracles."""
    w = RANDOM[name]
    say(f"[edge random] {name}: B {w.B} Hq {w.Hq} Hkv {w.Hkv} N {w.N} n_valid {w.Nv} d {w.d} {w.dtype} "
        f"kh {w.kh_bp} kl {w.kl_bp} n_sel {w.n_sel} window {w.window}")
    q, k, v, wg, f, layer = make_case(w, training=True)
    O = host(layer.run())
    torch.cuda.synchronize()
    assert np.all(np.isfinite(O)) and not O[:, :, w.Nv:].any()
    compare_outputs(O[:, :, :w.Nv], f.output()[:, :, :w.Nv], name)
    Hs = f.Hkv if f.group_sum else f.Hq
    maps = {(b, h, i): f.map_row(b, h, i) for b in range(w.B) for h in range(Hs) for i in range(f.nb)}
    dO = torch.from_numpy(np.random.default_rng(9).standard_normal(q.shape).astype(np.float32)).to(q.dtype)
    got = tuple(host(x) for x in layer.backward(dO.cuda()))
    torch.cuda.synchronize()
    ref = obwd.gradients(f.Q, f.K, f.V, host(dO).astype(np.float64), maps, w.Nv, f.scale, mode=w.mode,
                         w_gate=None if wg is None else wg.numpy(), window=w.window, group_map=w.mode == "nsa")
    rows = (slice(None), slice(None), slice(0, w.Nv))
    gscale = max(np.abs(r_[rows]).max() for r_ in ref[1:4])
    for g_, r_, what in zip(got[:3], ref[1:4], ("dQ", "dK", "dV")):
        diff = g_[rows].astype(np.float64) - r_[rows]
        # max-abs against the case's largest gradient (a single-key row can leave the bf16 term of
        # R28 in a small gradient), rel-L2 at the ordinary bar (none of these cases has such a row)
        mx = np.abs(diff).max() / gscale
        rel = np.linalg.norm(diff) / max(np.linalg.norm(r_[rows]), 1e-30)
        say(f"  {what}: max-abs {mx:.3e} of the largest gradient, rel-L2 {rel:.3e}")
        assert mx <= 1e-2 and rel <= REL_L2_G, (what, mx, rel)
        assert not g_[:, :, w.Nv:].any()
