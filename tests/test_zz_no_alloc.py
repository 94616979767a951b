"""The allocation-free block map (sla_block_map_noalloc, static device scratch) against
sla_block_map with a caller workspace, through the C-ABI: two calls in a row, the second on a
smaller input (the scratch keeps the first call's contents), causal and non-causal maps, outputs
bit for bit."""
import numpy as np
import pytest
import torch

import block_sparse_linear_mean_amd as sla
from tests.gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu


def _scores(B, Hs, nb, seed, causal):
    r = np.random.default_rng(seed)
    S = r.choice(np.array([-1.0, -0.0, 0.0, 0.25, 0.25, 2.0, 3.5], np.float32), size=(B, Hs, nb, nb))
    S = S.astype(np.float32)
    S[r.random(S.shape) < 0.02] = np.nan
    if causal:
        iu = np.triu_indices(nb, 1)
        S[:, :, iu[0], iu[1]] = -np.inf
    return to_dev(S, torch.float32)


def _same(a, b, causal):
    n = int(a["crit_rowptr"][-1].item())
    assert torch.equal(a["crit_rowptr"], b["crit_rowptr"])
    assert torch.equal(a["crit_idx"][:n], b["crit_idx"][:n])
    assert torch.equal(a["crit_flags"][:n], b["crit_flags"][:n])
    assert torch.equal(a["row_counts"], b["row_counts"])
    if not causal:
        m = int(a["marg_rowptr"][-1].item())
        assert torch.equal(a["marg_rowptr"], b["marg_rowptr"])
        assert torch.equal(a["marg_idx"][:m], b["marg_idx"][:m])
        assert torch.equal(a["marg_bits"], b["marg_bits"])
    return n


def test_noalloc_causal_two_calls():
    assert torch.cuda.is_available()
    # (B, Hs, nb, n_sel, window): the second call is smaller, with a shorter row capacity
    for k, (B, Hs, nb, n_sel, window) in enumerate([(1, 3, 300, 16, 512), (1, 1, 70, 4, 100)]):
        say(f"[no-alloc causal] call {k}: B={B} Hs={Hs} nb={nb} n_sel={n_sel} window={window}")
        S = _scores(B, Hs, nb, 100 + k, True)
        ref = sla.sla_block_map(S, n_sel, 0, causal=True, window=window)
        got = sla.sla_block_map_noalloc(S, n_sel, 0, causal=True, window=window)
        torch.cuda.synchronize()
        n = _same(got, ref, True)
        say(f"  {n} entries equal")


def test_noalloc_noncausal_two_calls():
    for k, (B, Hs, nb, nc, nn) in enumerate([(2, 2, 200, 26, 120), (1, 1, 65, 5, 30)]):
        say(f"[no-alloc non-causal] call {k}: B={B} Hs={Hs} nb={nb}")
        S = _scores(B, Hs, nb, 200 + k, False)
        ref = sla.sla_block_map(S, nc, nn)
        got = sla.sla_block_map_noalloc(S, nc, nn)
        torch.cuda.synchronize()
        _same(got, ref, False)


def test_noalloc_rejects_oversize():
    """A causal map whose padded lists exceed the 16 MiB scratch is refused before any launch."""
    S = torch.zeros(16, device="cuda")
    cap = sla.sla_block_map_capacity(1, 64, 4096, 4096, 16, 0, 1, 512, 0)
    p = S.data_ptr()
    rc = sla.lib().sla_block_map_noalloc(p, 1, 64, 4096, 4096, 16, 0, 1, 512, p, p, None, cap, None, None, 0, None,
                                         p, None)
    assert rc == 8    # SLA_ERR_WORKSPACE
