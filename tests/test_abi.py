"""The C-ABI library loads, exports every symbol include/sla.h declares, and rejects invalid
arguments on the host with the documented status codes.  CPU only: no call here reaches a
kernel launch (every call either launches nothing or fails validation first)."""
import ctypes
import json
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")

sla = pytest.importorskip("block_sparse_linear_mean_amd")
from block_sparse_linear_mean_amd import _lib  # noqa: E402

OK, ENULL, ESHAPE, EALIGN, ERANGE, EUNSUP, ECAP, EHIP, EWS = range(9)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsla.so is not built: run python -m block_sparse_linear_mean_amd.build")
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sla_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"libsla.so does not export {n}"
    assert set(names) == set(_lib._SIGS), "binding signatures and header declarations differ"


def test_version_and_status_strings(L):
    assert sla.sla_abi_version() == 6
    for s in range(9):
        assert len(sla.sla_status_str(s)) > 0
    assert sla.sla_status_str(12345) == "unknown status"


def test_counts_match_golden(L):
    data = json.load(open(os.path.join(ROOT, "tests", "golden", "counts.json")))
    for c in data["cases"]:
        assert sla.sla_counts(c["nb"], c["kh_bp"], c["kl_bp"]) == (c["n_h"], c["n_l"]), c["what"]
    with pytest.raises(sla.SlaError):
        sla.sla_counts(0, 100, 100)
    with pytest.raises(sla.SlaError):
        sla.sla_counts(10, 10001, 0)


def test_capacities_and_workspaces(L):
    # non-causal maps are exact
    assert sla.sla_block_map_capacity(1, 12, 512, 512, 26, 435, 0, 0, 0) == 12 * 512 * 26
    assert sla.sla_block_map_capacity(1, 12, 512, 512, 26, 435, 0, 0, 1) == 12 * 512 * 51
    assert sla.sla_block_map_capacity(1, 1, 16, 16, 10, 10, 0, 0, 0) == -1
    # causal: row i holds at most min(i + 1, 16 + 9) blocks
    nb = 1024
    ub = sum(min(i + 1, 25) for i in range(nb))
    assert sla.sla_block_map_capacity(1, 1, nb, nb, 16, 0, 1, 512, 0) == ub
    assert sla.sla_block_map_capacity(1, 1, nb, nb, 16, 0, 1, 512, 1) == 0
    assert sla.sla_block_map_workspace_bytes(1, 1, nb, nb, 16, 0, 512) == 0
    assert sla.sla_block_map_workspace_bytes(1, 1, nb, nb, 16, 1, 512) >= nb * 25 * 5
    assert sla.sla_attn_workspace_bytes(1, 12, 512, 128, _lib.SLA_LIN_MARGINAL) == 12 * 512 * (128 * 128 * 2 + 128 * 4)
    assert sla.sla_attn_workspace_bytes(1, 12, 512, 128, _lib.SLA_LIN_NONE) == 0
    assert sla.sla_kv_reduce_workspace_bytes(1, 12, 32768, 128, 1, 0) == 0
    # 12 heads x 512 blocks: runs of 12 blocks would make 43 x 12 = 516 workgroups, one more wave than
    # the 512 that run at once, so runs of 13 blocks: 40 fp32 partial states per head
    assert sla.sla_kv_reduce_workspace_bytes(1, 12, 32768, 128, 1, 1) == 12 * 40 * (128 * 128 + 128) * 4
    assert sla.sla_kv_reduce_workspace_bytes(1, 12, 32768, 128, 0, 1) == 12 * 40 * (128 * 128 + 128) * 4
    # runs stay within 4 .. 32 blocks
    assert sla.sla_kv_reduce_workspace_bytes(1, 1, 4096, 64, 1, 1) == 1 * 16 * (64 * 64 + 64) * 4
    assert sla.sla_kv_reduce_workspace_bytes(1, 64, 262144, 64, 1, 1) == 64 * 128 * (64 * 64 + 64) * 4


def desc(ptr=0x10000, dtype=0, B=1, H=2, N=256, d=128, sB=None, sH=None, sN=None):
    sN = d if sN is None else sN
    sH = N * sN if sH is None else sH
    sB = H * sH if sB is None else sB
    return _lib.SlaTensor(ctypes.c_void_p(ptr), dtype, B, H, N, d, sB, sH, sN)


P = ctypes.c_void_p(0x20000)   # a fake, 16-byte aligned device address: never dereferenced


def pool_call(L, q, k, n_valid=256, scale=0.1, qp=P, kp=P, sc=P):
    return L.sla_pool_scores(ctypes.byref(q), ctypes.byref(k), n_valid, 0, 0, scale, 0, qp, kp, sc, None, None, 0, None)


def test_pool_scores_validation(L):
    good = desc()
    assert pool_call(L, desc(ptr=0), good) == ENULL
    assert pool_call(L, good, good, qp=None) == ENULL
    assert pool_call(L, good, good, qp=ctypes.c_void_p(0x20004)) == EALIGN   # pooled vectors are read 16 bytes at a time
    assert pool_call(L, good, good, kp=ctypes.c_void_p(0x20008)) == EALIGN
    assert pool_call(L, desc(d=96), desc(d=96)) == EUNSUP
    assert pool_call(L, desc(dtype=7), good) == EUNSUP
    assert pool_call(L, desc(N=200), desc(N=200)) == ESHAPE
    assert pool_call(L, desc(ptr=0x10008), good) == EALIGN
    assert pool_call(L, desc(sN=132), desc(sN=132)) == EALIGN
    assert pool_call(L, good, desc(N=512)) == ESHAPE
    assert pool_call(L, desc(H=3), desc(H=2)) == ESHAPE
    assert pool_call(L, good, good, n_valid=192) == ERANGE      # more than one partial block
    assert pool_call(L, good, good, n_valid=257) == ERANGE
    assert pool_call(L, good, good, scale=0.0) == ERANGE
    assert pool_call(L, good, good, scale=float("nan")) == ERANGE
    assert pool_call(L, desc(N=64 * 4097), desc(N=64 * 4097)) == EUNSUP
    # group-summed scores of a GQA group need the workspace for the group sums
    q4, k1 = desc(H=4), desc(H=1)
    assert L.sla_pool_scores(ctypes.byref(q4), ctypes.byref(k1), 256, 1, 1, 0.1, 0, P, P, P, None, None, 0, None) == EWS
    assert L.sla_pool_scores(ctypes.byref(q4), ctypes.byref(k1), 256, 1, 1, 0.1, 1, P, P, P, None, None, 0, None) == EWS
    assert L.sla_pool_scores_workspace_bytes(1, 4, 1, 256, 128, 1) == 4 * 128 * 8
    assert L.sla_pool_scores_workspace_bytes(1, 4, 1, 256, 128, 0) == 0


def test_block_map_validation(L):
    def call(scores=P, B=1, Hs=1, nqb=16, nkb=16, nc=4, nn=8, causal=0, win=0, crp=P, ci=P, ccap=64,
             mrp=P, mi=P, mcap=64, rc=P, ws=None, wsb=0, bits=None):
        return L.sla_block_map(scores, B, Hs, nqb, nkb, nc, nn, causal, win, crp, ci, None, ccap, mrp, mi, mcap,
                               bits, rc, ws, wsb, None)
    assert call(scores=None) == ENULL
    assert call(crp=None) == ENULL
    assert call(rc=None) == ENULL
    assert call(mrp=None) == ENULL            # marginal pointers must come together
    assert call(nqb=0) == ESHAPE
    assert call(nkb=5000) == EUNSUP
    assert call(nc=-1) == ERANGE
    assert call(nc=10, nn=10) == ERANGE
    assert call(ccap=63) == ECAP
    assert call(mcap=63) == ECAP
    assert call(causal=1, nqb=16, nkb=15) == ESHAPE
    assert call(causal=1, nc=4, win=128, ccap=10) == ECAP
    assert call(causal=1, nc=4, win=128, ccap=1000) == EWS        # workspace missing
    assert call(causal=1, nc=4, win=128, ccap=1000, ws=P, wsb=1) == EWS
    assert call(causal=1, nc=4, win=128, ccap=1000, ws=P, wsb=1 << 20, bits=P) == EUNSUP


def test_block_map_noalloc_validation(L):
    """The allocation-free block map checks its arguments like sla_block_map, and rejects causal maps
    whose padded lists exceed its 16 MiB device scratch, all before any HIP call."""
    def call(scores=P, B=1, Hs=1, nqb=16, nkb=16, nc=4, nn=8, causal=0, win=0, crp=P, ci=P, ccap=64,
             mrp=P, mi=P, mcap=64, rc=P, bits=None):
        return L.sla_block_map_noalloc(scores, B, Hs, nqb, nkb, nc, nn, causal, win, crp, ci, None, ccap, mrp, mi,
                                       mcap, bits, rc, None)
    assert call(scores=None) == ENULL
    assert call(rc=None) == ENULL
    assert call(mrp=None) == ENULL
    assert call(nqb=0) == ESHAPE
    assert call(nkb=5000) == EUNSUP
    assert call(nc=10, nn=10) == ERANGE
    assert call(ccap=63) == ECAP
    assert call(causal=1, nqb=16, nkb=15) == ESHAPE
    assert call(causal=1, nc=4, win=128, ccap=1000, bits=P) == EUNSUP
    # 64 heads x 4096 query blocks x 25 entries x 5 bytes > 16 MiB of scratch
    big = dict(causal=1, Hs=64, nqb=4096, nkb=4096, nc=16, win=512)
    cap = L.sla_block_map_capacity(1, 64, 4096, 4096, 16, 0, 1, 512, 0)
    assert L.sla_block_map_workspace_bytes(1, 64, 4096, 4096, 16, 1, 512) > 16 << 20
    assert call(ccap=cap, **big) == EWS


def test_kv_reduce_validation(L):
    k = desc()
    def call(kk=k, vv=k, nv=256, H=P, z=P, Ha=None, za=None, ws=None, wsb=0, shift=None, kp=None):
        return L.sla_linear_kv_reduce(ctypes.byref(kk), ctypes.byref(vv), nv, shift, H, z, Ha, za, kp, ws, wsb, None)
    assert call(H=None, z=None) == ENULL
    assert call(z=None) == ENULL
    assert call(Ha=P, za=None) == ENULL
    assert call(vv=desc(H=3)) == ESHAPE
    assert call(vv=desc(dtype=1)) == ESHAPE
    assert call(nv=0) == ERANGE
    assert call(H=None, z=None, Ha=P, za=P) == EWS
    assert call(shift=ctypes.c_void_p(0x20004)) == EALIGN
    assert call(kp=ctypes.c_void_p(0x20004)) == EALIGN
    assert call(kp=P, H=None, z=None) == ENULL               # the key block means come with a state output


def test_key_mean_validation(L):
    def call(kp=P, B=1, Hkv=2, nkb=4, d=128, nv=256, out=P):
        return L.sla_key_mean(kp, B, Hkv, nkb, d, nv, out, None)
    assert call(kp=None) == ENULL
    assert call(out=None) == ENULL
    assert call(d=96) == ESHAPE
    assert call(nkb=0) == ESHAPE
    assert call(nv=192) == ERANGE
    assert call(nv=257) == ERANGE
    assert call(out=ctypes.c_void_p(0x20004)) == EALIGN


def test_marginal_states_validation(L):
    def call(H=P, z=P, B=1, Hq=2, Hkv=1, nqb=4, nkb=4, d=128, bits=P, S=P, u=P):
        return L.sla_marginal_states(H, z, B, Hq, Hkv, nqb, nkb, d, 0, bits, S, u, None)
    assert call(H=None) == ENULL
    assert call(bits=None) == ENULL
    assert call(Hq=3, Hkv=2) == ESHAPE
    assert call(d=96) == EUNSUP
    assert call(S=ctypes.c_void_p(0x20004)) == EALIGN


def test_attn_fwd_validation(L):
    q = desc()
    def call(qq=q, kk=q, vv=q, nv=256, scale=0.1, causal=0, win=0, group=0, crp=P, ci=P, cf=None, mb=None,
             lin=0, H=None, z=None, Ha=None, za=None, wg=None, out=P, odt=0, ws=None, wsb=0, pw=None, pb=None,
             ph=0):
        return L.sla_attn_fwd(ctypes.byref(qq), ctypes.byref(kk), ctypes.byref(vv), nv, scale, causal, win, group,
                              crp, ci, cf, mb, lin, H, z, Ha, za, wg, pw, pb, ph, out, odt, None, ws, wsb, None)
    assert call(out=None) == ENULL
    assert call(crp=None) == ENULL
    assert call(causal=1) == ENULL                   # causal needs the flags
    assert call(causal=1, cf=P, lin=1) == EUNSUP     # no linear branch under a causal mask
    assert call(lin=1) == ENULL                      # marginal mode needs H, z and the marginal bit masks
    assert call(lin=1, H=P, z=P, mb=P) == EWS
    assert call(lin=2) == ENULL
    assert call(lin=3) == ENULL                      # precomputed row states needed
    assert call(lin=3, H=ctypes.c_void_p(0x20004), z=P) == EALIGN
    assert call(lin=4) == EUNSUP
    assert call(odt=5) == EUNSUP
    assert call(out=ctypes.c_void_p(0x20002)) == EALIGN
    assert call(kk=desc(H=3), vv=desc(H=3)) == ESHAPE
    assert call(vv=desc(H=1)) == ESHAPE
    assert call(win=-1) == ERANGE
    assert call(nv=64) == ERANGE
    assert call(pb=P) == ENULL                       # a Proj bias needs the weight
    assert call(pw=P, ph=1) == EUNSUP                # Proj is for the SLA linear branch only
    assert call(lin=3, H=P, z=P, pw=P, ph=3) == ESHAPE
    assert call(lin=3, H=P, z=P, pw=ctypes.c_void_p(0x20004), ph=1) == EALIGN


def test_attn_bwd_validation(L):
    q = desc()
    def call(qq=q, kk=q, vv=q, oo=q, gg=q, lse=P, nv=256, scale=0.1, crp=P, ci=P, mb=P, S=P, u=P, ks=None,
             pw=None, pb=None, ph=0, dq=P, dk=P, dv=P, dw=None, db=None, ws=None, wsb=0):
        return L.sla_attn_bwd(ctypes.byref(qq), ctypes.byref(kk), ctypes.byref(vv), ctypes.byref(oo),
                              ctypes.byref(gg), lse, nv, scale, crp, ci, mb, S, u, ks, pw, pb, ph, dq, dk, dv, dw,
                              db, ws, wsb, None)
    assert call(lse=None) == ENULL
    assert call(mb=None) == ENULL
    assert call(dq=None) == ENULL
    assert call(kk=desc(H=1), vv=desc(H=1)) == EUNSUP          # one KV head per query head only
    assert call(oo=desc(dtype=1)) == ESHAPE
    assert call(gg=desc(N=512)) == ESHAPE
    assert call(nv=100) == ERANGE
    assert call(scale=-1.0) == ERANGE
    assert call(dk=ctypes.c_void_p(0x20004)) == EALIGN
    assert call() == EWS                                       # workspace missing
    assert call(ws=P, wsb=16) == EWS
    assert call(pb=P) == ENULL                                 # Proj bias without the weight
    assert call(dw=P) == ENULL                                 # Proj gradient without the weight
    assert call(pw=P, ph=1) == ENULL                           # Proj needs its weight gradient
    assert call(pw=P, ph=3, dw=P) == ESHAPE                    # proj_heads is 1 or H
    assert call(pw=P, ph=2, dw=ctypes.c_void_p(0x20004)) == EALIGN
    assert call(ks=ctypes.c_void_p(0x20004)) == EALIGN
    assert call(pw=P, ph=1, dw=P, ws=P, wsb=L.sla_attn_bwd_workspace_bytes(1, 2, 256, 128, 0)) == EWS
    assert L.sla_attn_bwd_workspace_bytes(1, 2, 256, 128, 0) > 0
    assert L.sla_attn_bwd_workspace_bytes(1, 2, 256, 128, 1) > L.sla_attn_bwd_workspace_bytes(1, 2, 256, 128, 0)
    assert L.sla_attn_bwd_workspace_bytes(1, 2, 256, 128, 3) == 0
    assert L.sla_attn_bwd_workspace_bytes(1, 2, 100, 128, 0) == 0


def test_attn_bwd_ext_validation(L):
    q = desc(H=4)
    kv = desc(H=2)
    ROW, NONE, GATED = 3, 0, 2
    def call(qq=q, kk=kv, vv=kv, oo=q, gg=q, lse=P, nv=256, scale=0.1, lin=NONE, causal=0, win=0, gm=0, crp=P,
             ci=P, cf=None, mb=None, S=None, u=None, Ha=None, za=None, wg=None, ks=None, pw=None, pb=None, ph=0,
             dq=P, dk=P, dv=P, dw=None, db=None, dwg=None, ws=None, wsb=0):
        return L.sla_attn_bwd_ext(ctypes.byref(qq), ctypes.byref(kk), ctypes.byref(vv), ctypes.byref(oo),
                                  ctypes.byref(gg), lse, nv, scale, lin, causal, win, gm, crp, ci, cf, mb, S, u, Ha,
                                  za, wg, ks, pw, pb, ph, dq, dk, dv, dw, db, dwg, ws, wsb, None)
    assert call(kk=desc(H=3), vv=desc(H=3)) == ESHAPE           # Hq not a multiple of Hkv
    assert call(vv=desc(H=4)) == ESHAPE                         # K and V disagree
    assert call(lin=1 + 8) == EUNSUP                            # unknown linear mode
    assert call(lin=ROW, causal=1, cf=P) == EUNSUP              # a linear branch is non-causal
    assert call(lin=GATED, gm=1) == EUNSUP                      # ... and takes per-head maps
    assert call(causal=1) == ENULL                              # causal maps need their flags
    assert call(causal=1, cf=P, win=-1) == ERANGE
    assert call(lin=ROW) == ENULL                               # row states and masks
    assert call(lin=ROW, mb=P, S=P, u=ctypes.c_void_p(0x20004)) == EALIGN
    assert call(lin=GATED, Ha=P, za=P, wg=P) == ENULL           # the gate gradient is required
    assert call(dwg=P) == ENULL                                 # ... and only with the gate
    assert call(pw=P, ph=1, dw=P) == EUNSUP                     # Proj belongs to the row-states mode
    assert call(ks=P) == EUNSUP                                 # smooth-K needs a linear branch
    assert call() == EWS
    need = L.sla_attn_bwd_ext_workspace_bytes(1, 4, 2, 256, 128, NONE, 1, 1, 0)
    assert call(causal=1, cf=P, gm=1, ws=P, wsb=need - 1) == EWS
    assert need > 0
    assert L.sla_attn_bwd_ext_workspace_bytes(1, 4, 2, 256, 128, ROW, 0, 0, 0) > need
    assert L.sla_attn_bwd_ext_workspace_bytes(1, 4, 2, 256, 128, GATED, 0, 0, 0) > need
    assert L.sla_attn_bwd_ext_workspace_bytes(1, 4, 3, 256, 128, NONE, 0, 0, 0) == 0
    assert L.sla_attn_bwd_ext_workspace_bytes(1, 4, 2, 256, 128, ROW, 1, 0, 0) == 0
    assert L.sla_attn_bwd_ext_workspace_bytes(1, 4, 2, 256, 128, GATED, 0, 0, 1) == 0
    # the MHA entry point is the row-states mode of the extended one
    assert (L.sla_attn_bwd_workspace_bytes(1, 2, 256, 128, 1)
            == L.sla_attn_bwd_ext_workspace_bytes(1, 2, 2, 256, 128, ROW, 0, 0, 1))


def test_nsa3_validation(L):
    q = desc(H=4)
    kv = desc(H=1)
    def call(qq=q, kk=kv, vv=kv, nv=256, scale=0.1, rp=P, ci=P, cf=P, win=512, blk=32, st=16, wg=P, out=P, odt=0,
             ws=None, wsb=0):
        return L.sla_nsa3_fwd(ctypes.byref(qq), ctypes.byref(kk), ctypes.byref(vv), nv, scale, rp, ci, cf, win, blk, st,
                              wg, out, odt, ws, wsb, None)
    assert call(wg=None) == ENULL
    assert call(cf=None) == ENULL
    assert call(kk=desc(H=3), vv=desc(H=3)) == ESHAPE
    assert call(blk=0) == ERANGE
    assert call(st=0) == ERANGE
    assert call(win=-1) == ERANGE
    assert call(odt=3) == EUNSUP
    assert call(wg=ctypes.c_void_p(0x20004)) == EALIGN
    assert call() == EWS
    assert L.sla_nsa3_workspace_bytes(1, 4, 1, 256, 128, 0, 256, 512, 32, 16) > 0
    assert L.sla_nsa3_workspace_bytes(1, 4, 3, 256, 128, 0, 256, 512, 32, 16) == 0


def test_layer_fuses_key_pooling_only_when_exact(L):
    """The layer takes the key block means from the key-state pass only when that pass runs without a
    shift on bf16 K (exact fp64 block sums, so the same bits as the pooling pass); host logic only:
    constructing the layer on CPU tensors launches nothing."""
    def layer(dtype, mode="sla", smooth_k=False):
        x = torch.zeros((1, 1, 256, 64), dtype=dtype)
        wg = torch.zeros((1, 64)) if mode == "salad" else None
        return sla.SlaForward(x, x, x, 256, mode, kh_bp=2500, kl_bp=5000, n_sel=2, window=64, smooth_k=smooth_k,
                              w_gate=wg)
    assert layer(torch.bfloat16).fuse_key_pooling
    assert layer(torch.bfloat16, mode="salad").fuse_key_pooling
    assert not layer(torch.float32).fuse_key_pooling
    assert not layer(torch.bfloat16, smooth_k=True).fuse_key_pooling
    assert not layer(torch.bfloat16, mode="nsa").fuse_key_pooling


def test_differentiable_layer_fails_loudly_without_the_gpu(L):
    """sla_attention has no CPU fallback: on CPU tensors the first library call refuses them."""
    x = torch.zeros((1, 1, 256, 64), dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError, match="GPU tensors"):
        sla.sla_attention(x, x, x, 256, "sla", kh_bp=2500, kl_bp=5000)
