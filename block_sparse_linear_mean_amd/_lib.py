"""ctypes binding of libsla (include/sla.h): argument marshalling only.

Every step of the forward runs in the HIP library; this module checks tensor
placement, allocates outputs with torch on the tensors' device, passes raw device
pointers, strides and torch's current HIP stream, and turns status codes into
exceptions.  It fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint8, c_void_p
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsla.so")

SLA_BF16, SLA_F32 = 0, 1
SLA_LIN_NONE, SLA_LIN_MARGINAL, SLA_LIN_GLOBAL_GATED, SLA_LIN_ROW_STATES = 0, 1, 2, 3
BLOCK = 64


class SlaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class SlaTensor(ctypes.Structure):
    _fields_ = [("ptr", c_void_p), ("dtype", c_int32), ("B", c_int32), ("H", c_int32), ("N", c_int32),
                ("d", c_int32), ("sB", c_int64), ("sH", c_int64), ("sN", c_int64)]


_lib = None
_P = c_void_p
_I32P = POINTER(c_int32)

_SIGS = {
    "sla_abi_version": (c_int32, []),
    "sla_status_str": (c_char_p, [c_int32]),
    "sla_counts": (c_int32, [c_int32, c_int32, c_int32, _I32P, _I32P]),
    "sla_pool_scores": (c_int32, [POINTER(SlaTensor), POINTER(SlaTensor), c_int32, c_int32, c_int32, c_float,
                                  c_int32, _P, _P, _P, _P, _P, c_size_t, _P]),
    "sla_pool_scores_workspace_bytes": (c_size_t, [c_int32] * 6),
    "sla_block_map_capacity": (c_int64, [c_int32] * 9),
    "sla_block_map_workspace_bytes": (c_size_t, [c_int32] * 7),
    "sla_block_map": (c_int32, [_P, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                _P, _P, _P, c_int64, _P, _P, c_int64, _P, _P, _P, c_size_t, _P]),
    "sla_block_map_noalloc": (c_int32, [_P, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                        c_int32, _P, _P, _P, c_int64, _P, _P, c_int64, _P, _P, _P]),
    "sla_kv_reduce_workspace_bytes": (c_size_t, [c_int32] * 6),
    "sla_key_mean": (c_int32, [_P, c_int32, c_int32, c_int32, c_int32, c_int32, _P, _P]),
    "sla_linear_kv_reduce": (c_int32, [POINTER(SlaTensor), POINTER(SlaTensor), c_int32, _P, _P, _P, _P, _P, _P,
                                       _P, c_size_t, _P]),
    "sla_marginal_states": (c_int32, [_P, _P, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                      _P, _P, _P, _P]),
    "sla_attn_workspace_bytes": (c_size_t, [c_int32] * 5),
    "sla_attn_fwd": (c_int32, [POINTER(SlaTensor), POINTER(SlaTensor), POINTER(SlaTensor), c_int32, c_float,
                               c_int32, c_int32, c_int32, _P, _P, _P, _P, c_int32, _P, _P, _P, _P, _P,
                               _P, _P, c_int32, _P, c_int32, _P, _P, c_size_t, _P]),
    "sla_nsa3_workspace_bytes": (c_size_t, [c_int32] * 10),
    "sla_nsa3_fwd": (c_int32, [POINTER(SlaTensor)] * 3 + [c_int32, c_float, _P, _P, _P, c_int32, c_int32, c_int32, _P,
                                                          _P, c_int32, _P, c_size_t, _P]),
    "sla_hilbert_order": (c_int32, [c_int32, c_int32, c_int32, _P]),
    "sla_permute_rows": (c_int32, [POINTER(SlaTensor), _P, c_int32, c_int32, _P, _P]),
    "sla_attn_bwd_workspace_bytes": (c_size_t, [c_int32] * 5),
    "sla_attn_bwd": (c_int32, [POINTER(SlaTensor)] * 5 + [_P, c_int32, c_float, _P, _P, _P, _P, _P, _P, _P, _P,
                                                          c_int32, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "sla_attn_bwd_ext_workspace_bytes": (c_size_t, [c_int32] * 9),
    "sla_attn_bwd_ext": (c_int32, [POINTER(SlaTensor)] * 5 + [_P, c_int32, c_float, c_int32, c_int32, c_int32,
                                                              c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                              _P, c_int32, _P, _P, _P, _P, _P, _P, _P, c_size_t,
                                                              _P]),
}


def lib():
    """The loaded library (ctypes.CDLL).  Raises if libsla.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libsla.so not built at {LIB_PATH}: run `python -m block_sparse_linear_mean_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise SlaError(fn, status, lib().sla_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libsla calls take GPU tensors")


def tensor_desc(x: torch.Tensor) -> SlaTensor:
    """Descriptor of a [B, H, N, d] bf16/fp32 tensor with unit d-stride."""
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("expected a [B, H, N, d] tensor with unit stride along d")
    if x.dtype == torch.bfloat16:
        dt = SLA_BF16
    elif x.dtype == torch.float32:
        dt = SLA_F32
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    B, H, N, d = x.shape
    return SlaTensor(c_void_p(x.data_ptr()), dt, B, H, N, d, x.stride(0), x.stride(1), x.stride(2))


# ----------------------------------------------------------------------------- host-only calls

def sla_abi_version() -> int:
    return lib().sla_abi_version()


def sla_status_str(status: int) -> str:
    return lib().sla_status_str(status).decode()


def sla_counts(nb: int, kh_bp: int, kl_bp: int):
    a, b = c_int32(), c_int32()
    _check("sla_counts", lib().sla_counts(nb, kh_bp, kl_bp, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def sla_block_map_capacity(B, Hs, nqb, nkb, n_crit, n_negl, causal, window, which) -> int:
    return lib().sla_block_map_capacity(B, Hs, nqb, nkb, n_crit, n_negl, int(causal), window, which)


def sla_block_map_workspace_bytes(B, Hs, nqb, nkb, n_crit, causal, window) -> int:
    return lib().sla_block_map_workspace_bytes(B, Hs, nqb, nkb, n_crit, int(causal), window)


def sla_kv_reduce_workspace_bytes(B, Hkv, N, d, want_blocks, want_all) -> int:
    return lib().sla_kv_reduce_workspace_bytes(B, Hkv, N, d, int(want_blocks), int(want_all))


def sla_attn_workspace_bytes(B, Hs, nqb, d, lin_mode) -> int:
    return lib().sla_attn_workspace_bytes(B, Hs, nqb, d, lin_mode)


# ----------------------------------------------------------------------------- GPU calls

def sla_pool_scores(q, k, n_valid, group_sum=False, causal=False, scale=None, want_probs=False, out=None,
                    k_pooled=False, q_pooled=False, want_scores=True):
    """Returns dict(q_pool, k_pool, scores[, probs]); `out` may hold preallocated tensors.

    k_pooled: out["k_pool"] already holds the key block means (sla_linear_kv_reduce's k_pool output);
    q_pooled: out["q_pool"] already holds the query block means; want_scores=False: pooling only.
    """
    _require_gpu(q, k)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nb = N // BLOCK
    Hs = Hkv if group_sum else Hq
    scale = (1.0 / d ** 0.5) if scale is None else scale
    if out is None:
        f = dict(device=q.device, dtype=torch.float32)
        out = dict(q_pool=torch.empty((B, Hq, nb, d), **f), k_pool=torch.empty((B, Hkv, nb, d), **f),
                   scores=torch.empty((B, Hs, nb, nb), **f))
        if want_probs:
            out["probs"] = torch.empty((B, Hs, nb, nb), **f)
    ws = int(lib().sla_pool_scores_workspace_bytes(B, Hq, Hkv, N, d, int(group_sum)))
    if ws and (out.get("workspace") is None or out["workspace"].numel() < ws):
        out["workspace"] = torch.empty(ws, device=q.device, dtype=torch.uint8)
    qd, kd = tensor_desc(q), tensor_desc(k)
    pooled = (1 if k_pooled else 0) | (2 if q_pooled else 0)
    _check("sla_pool_scores", lib().sla_pool_scores(
        ctypes.byref(qd), ctypes.byref(kd), n_valid, int(group_sum), int(causal), float(scale), pooled,
        _ptr(out["q_pool"]), _ptr(out["k_pool"]), _ptr(out["scores"]) if want_scores else None,
        _ptr(out.get("probs")) if want_scores else None, _ptr(out.get("workspace")), ws, _stream(q.device)))
    return out


def alloc_block_map(B, Hs, nqb, nkb, n_crit, n_negl, causal, window, device, want_marg=True):
    rows = B * Hs * nqb
    cc = sla_block_map_capacity(B, Hs, nqb, nkb, n_crit, n_negl, causal, window, 0)
    mc = sla_block_map_capacity(B, Hs, nqb, nkb, n_crit, n_negl, causal, window, 1) if want_marg else 0
    if cc < 0 or mc < 0:
        raise ValueError("invalid block-map sizes")
    i32 = dict(device=device, dtype=torch.int32)
    m = dict(crit_rowptr=torch.empty(rows + 1, **i32), crit_idx=torch.empty(max(cc, 1), **i32),
             crit_flags=torch.empty(max(cc, 1), device=device, dtype=torch.uint8),
             row_counts=torch.empty((rows, 3), **i32), crit_cap=cc, marg_cap=mc)
    if want_marg and not causal:
        m["marg_rowptr"] = torch.empty(rows + 1, **i32)
        m["marg_idx"] = torch.empty(max(mc, 1), **i32)
        m["marg_bits"] = torch.empty((rows, (nkb + 31) // 32), **i32)   # uint32 bit masks
    ws = sla_block_map_workspace_bytes(B, Hs, nqb, nkb, n_crit, causal, window)
    m["workspace"] = torch.empty(max(ws, 16), device=device, dtype=torch.uint8) if ws else None
    m["workspace_bytes"] = ws
    return m


def sla_block_map(scores, n_crit, n_negl=0, causal=False, window=0, want_marg=True, out=None):
    """Block map of scores [B, Hs, nqb, nkb]; returns the dict of CSR tensors."""
    _require_gpu(scores)
    B, Hs, nqb, nkb = scores.shape
    if out is None:
        out = alloc_block_map(B, Hs, nqb, nkb, n_crit, n_negl, causal, window, scores.device, want_marg)
    _check("sla_block_map", lib().sla_block_map(
        _ptr(scores), B, Hs, nqb, nkb, n_crit, n_negl, int(causal), window,
        _ptr(out["crit_rowptr"]), _ptr(out["crit_idx"]), _ptr(out["crit_flags"]), out["crit_cap"],
        _ptr(out.get("marg_rowptr")), _ptr(out.get("marg_idx")), out["marg_cap"], _ptr(out.get("marg_bits")),
        _ptr(out["row_counts"]), _ptr(out["workspace"]), out["workspace_bytes"], _stream(scores.device)))
    return out


def sla_block_map_noalloc(scores, n_crit, n_negl=0, causal=False, window=0, want_marg=True, out=None):
    """sla_block_map without a workspace (the library's static device scratch serves the causal
    path); out: the dict of alloc_block_map (its workspace entry is not used)."""
    _require_gpu(scores)
    B, Hs, nqb, nkb = scores.shape
    if out is None:
        out = alloc_block_map(B, Hs, nqb, nkb, n_crit, n_negl, causal, window, scores.device, want_marg)
    _check("sla_block_map_noalloc", lib().sla_block_map_noalloc(
        _ptr(scores), B, Hs, nqb, nkb, n_crit, n_negl, int(causal), window,
        _ptr(out["crit_rowptr"]), _ptr(out["crit_idx"]), _ptr(out["crit_flags"]), out["crit_cap"],
        _ptr(out.get("marg_rowptr")), _ptr(out.get("marg_idx")), out["marg_cap"], _ptr(out.get("marg_bits")),
        _ptr(out["row_counts"]), _stream(scores.device)))
    return out


def sla_key_mean(k_pool, n_valid, out=None):
    """Smooth-K shift [B, Hkv, d] fp32: the mean of the valid key rows, from the block means k_pool."""
    _require_gpu(k_pool)
    B, Hkv, nb, d = k_pool.shape
    if out is None:
        out = torch.empty((B, Hkv, d), device=k_pool.device, dtype=torch.float32)
    _check("sla_key_mean", lib().sla_key_mean(_ptr(k_pool), B, Hkv, nb, d, n_valid, _ptr(out),
                                              _stream(k_pool.device)))
    return out


def sla_linear_kv_reduce(k, v, n_valid, per_block=True, want_all=False, out=None, k_shift=None, k_pool=None):
    """Returns dict(H, z[, H_all, z_all]): per-block states H in bf16, everything else fp32.

    k_shift [B, Hkv, d] fp32 (smooth-K, e.g. from sla_key_mean): states of phi(K - k_shift).
    k_pool [B, Hkv, nb, d] fp32 (optional output): also the key block means of the prediction step.
    """
    _require_gpu(k, v)
    if k_shift is not None and (k_shift.dtype != torch.float32 or not k_shift.is_contiguous()):
        raise ValueError("k_shift must be a contiguous float32 [B, Hkv, d] tensor")
    B, Hkv, N, d = k.shape
    nb = N // BLOCK
    if k_pool is not None and (k_pool.dtype != torch.float32 or not k_pool.is_contiguous()
                               or tuple(k_pool.shape) != (B, Hkv, nb, d)):
        raise ValueError("k_pool must be a contiguous float32 [B, Hkv, nb, d] tensor")
    if out is None:
        f = dict(device=k.device, dtype=torch.float32)
        out = {}
        if per_block:
            out["H"] = torch.empty((B, Hkv, nb, d, d), device=k.device, dtype=torch.bfloat16)
            out["z"] = torch.empty((B, Hkv, nb, d), **f)
        if want_all:
            out["H_all"] = torch.empty((B, Hkv, d, d), **f)
            out["z_all"] = torch.empty((B, Hkv, d), **f)
        ws = sla_kv_reduce_workspace_bytes(B, Hkv, N, d, per_block, want_all)
        out["workspace"] = torch.empty(ws, device=k.device, dtype=torch.uint8) if ws else None
        out["workspace_bytes"] = ws
    kd, vd = tensor_desc(k), tensor_desc(v)
    _check("sla_linear_kv_reduce", lib().sla_linear_kv_reduce(
        ctypes.byref(kd), ctypes.byref(vd), n_valid, _ptr(k_shift), _ptr(out.get("H")), _ptr(out.get("z")),
        _ptr(out.get("H_all")), _ptr(out.get("z_all")), _ptr(k_pool), _ptr(out.get("workspace")),
        out.get("workspace_bytes", 0), _stream(k.device)))
    return out


def sla_marginal_states(H, z, Hq, group_map, marg_bits, out=None):
    """Per-row marginal sums of the bf16 states H: S bf16 [rows, d, d] in H's [c][r] layout, u fp32 [rows, d]."""
    _require_gpu(H, z, marg_bits)
    if H.dtype != torch.bfloat16:
        raise ValueError("H must be the bf16 per-block states of sla_linear_kv_reduce")
    B, Hkv, nb, d, _ = H.shape
    Hs = Hkv if group_map else Hq
    rows = B * Hs * nb
    if out is None:
        S = torch.empty((rows, d, d), device=H.device, dtype=torch.bfloat16)
        u = torch.empty((rows, d), device=H.device, dtype=torch.float32)
    else:
        S, u = out
    _check("sla_marginal_states", lib().sla_marginal_states(
        _ptr(H), _ptr(z), B, Hq, Hkv, nb, nb, d, int(group_map), _ptr(marg_bits), _ptr(S), _ptr(u),
        _stream(H.device)))
    return S, u


def sla_attn_fwd(q, k, v, n_valid, maps, lin_mode=SLA_LIN_NONE, scale=None, causal=False, window=0,
                 group_map=False, H=None, z=None, H_all=None, z_all=None, w_gate=None, out=None,
                 out_dtype=None, workspace=None, proj_w=None, proj_b=None, lse=None):
    """Attention output [B, Hq, N, d]; `maps` is the dict returned by sla_block_map.

    lse: optional float32 [B, Hq, N] output, the log-sum-exp of each row's sparse logits (for sla_attn_bwd).

    proj_w [d, d] or [Hq, d, d] fp32 (out x in) and proj_b [d] or [Hq, d]: the learned
    projection of the SLA linear branch (None = identity).
    """
    _require_gpu(q, k, v)
    B, Hq, N, d = q.shape
    proj_heads = 0
    if proj_w is not None:
        if proj_w.dtype != torch.float32 or not proj_w.is_contiguous() or proj_w.shape[-2:] != (d, d):
            raise ValueError("proj_w must be a contiguous float32 [d, d] or [Hq, d, d] tensor")
        proj_heads = 1 if proj_w.dim() == 2 else proj_w.shape[0]
        if proj_b is not None and (proj_b.dtype != torch.float32 or not proj_b.is_contiguous()
                                   or proj_b.numel() != proj_heads * d):
            raise ValueError("proj_b must be a contiguous float32 tensor with one d-vector per weight")
    scale = (1.0 / d ** 0.5) if scale is None else scale
    if out is None:
        out = torch.empty(q.shape, device=q.device, dtype=out_dtype or q.dtype)
    odt = SLA_F32 if out.dtype == torch.float32 else SLA_BF16
    Hs = k.shape[1] if group_map else Hq
    ws_bytes = sla_attn_workspace_bytes(B, Hs, N // BLOCK, d, lin_mode)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    qd, kd, vd = tensor_desc(q), tensor_desc(k), tensor_desc(v)
    _check("sla_attn_fwd", lib().sla_attn_fwd(
        ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), n_valid, float(scale), int(causal), window,
        int(group_map), _ptr(maps["crit_rowptr"]), _ptr(maps["crit_idx"]), _ptr(maps.get("crit_flags")),
        _ptr(maps.get("marg_bits")), lin_mode, _ptr(H), _ptr(z), _ptr(H_all),
        _ptr(z_all), _ptr(w_gate), _ptr(proj_w), _ptr(proj_b), proj_heads, _ptr(out), odt, _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(q.device)))
    return out


def sla_attn_bwd_workspace_bytes(B, H, N, d, proj_heads=0) -> int:
    return int(lib().sla_attn_bwd_workspace_bytes(B, H, N, d, proj_heads))


def sla_attn_bwd(q, k, v, o, dout, lse, n_valid, maps, S, u, scale=None, grads=None, workspace=None, k_shift=None,
                 proj_w=None, proj_b=None, proj_grads=None):
    """(dq, dk, dv) fp32 [B, H, N, d]: gradients of sum(dout * o) for the SLA forward with the same map;
    with proj_w, (dq, dk, dv, dW, db) with dW shaped like proj_w and db like it without the last axis
    (db None when there is no bias and proj_grads does not supply one).

    o and lse come from sla_attn_fwd; S, u are that map's per-row marginal sums (sla_marginal_states).
    k_shift: the smooth-K key mean [B, H, d] fp32 given to the forward (None: smooth-K off).
    proj_w, proj_b: the forward's Proj weight and bias (None: identity).
    """
    _require_gpu(q, k, v, o, dout, lse)
    B, H, N, d = q.shape
    scale = (1.0 / d ** 0.5) if scale is None else scale
    if grads is None:
        grads = tuple(torch.empty((B, H, N, d), device=q.device, dtype=torch.float32) for _ in range(3))
    proj_heads = 0
    dW = db = None
    if proj_w is not None:
        if proj_w.dtype != torch.float32 or not proj_w.is_contiguous() or proj_w.shape[-2:] != (d, d):
            raise ValueError("proj_w must be a contiguous float32 [d, d] or [H, d, d] tensor")
        proj_heads = 1 if proj_w.dim() == 2 else proj_w.shape[0]
        if proj_grads is not None:
            dW, db = proj_grads
        else:
            dW = torch.empty_like(proj_w)
            db = None if proj_b is None else torch.empty(proj_w.shape[:-1], device=q.device, dtype=torch.float32)
    elif proj_b is not None:
        raise ValueError("proj_b without proj_w")
    if k_shift is not None and (k_shift.dtype != torch.float32 or not k_shift.is_contiguous()
                                or tuple(k_shift.shape) != (B, H, d)):
        raise ValueError("k_shift must be a contiguous float32 [B, H, d] tensor")
    ws_bytes = sla_attn_bwd_workspace_bytes(B, H, N, d, proj_heads)
    if workspace is None:
        workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    descs = [tensor_desc(x) for x in (q, k, v, o, dout)]
    dq, dk, dv = grads
    _check("sla_attn_bwd", lib().sla_attn_bwd(
        *[ctypes.byref(x) for x in descs], _ptr(lse), n_valid, float(scale), _ptr(maps["crit_rowptr"]),
        _ptr(maps["crit_idx"]), _ptr(maps["marg_bits"]), _ptr(S), _ptr(u), _ptr(k_shift), _ptr(proj_w),
        _ptr(proj_b), proj_heads, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW), _ptr(db), _ptr(workspace), ws_bytes,
        _stream(q.device)))
    if proj_w is not None:
        return dq, dk, dv, dW, db
    return dq, dk, dv


def sla_attn_bwd_ext_workspace_bytes(B, Hq, Hkv, N, d, lin_mode, causal=False, group_map=False,
                                     proj_heads=0) -> int:
    return int(lib().sla_attn_bwd_ext_workspace_bytes(B, Hq, Hkv, N, d, lin_mode, int(causal), int(group_map),
                                                      proj_heads))


def sla_attn_bwd_ext(q, k, v, o, dout, lse, n_valid, maps, lin_mode, scale=None, causal=False, window=0,
                     group_map=False, S=None, u=None, H_all=None, z_all=None, w_gate=None, k_shift=None,
                     proj_w=None, proj_b=None, grads=None, proj_grads=None, dw_gate=None, workspace=None):
    """Gradients of sum(dout * o) for every sla_attn_fwd mode, fixed map: (dq [B, Hq, N, d],
    dk, dv [B, Hkv, N, d]) fp32, then (dW, db) with proj_w, then dw_gate [Hq, d] when gated.

    lin_mode SLA_LIN_ROW_STATES: S, u the map's per-row marginal sums, maps["marg_bits"] its masks;
    SLA_LIN_GLOBAL_GATED: H_all, z_all from sla_linear_kv_reduce and w_gate [Hq, d];
    SLA_LIN_NONE: no linear branch (causal maps with window tokens, shared by a GQA group with
    group_map).  k_shift [B, Hkv, d]: the smooth-K key mean given to the forward.
    """
    _require_gpu(q, k, v, o, dout, lse)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = (1.0 / d ** 0.5) if scale is None else scale
    f32 = dict(device=q.device, dtype=torch.float32)
    if grads is None:
        grads = (torch.empty((B, Hq, N, d), **f32), torch.empty((B, Hkv, N, d), **f32),
                 torch.empty((B, Hkv, N, d), **f32))
    proj_heads = 0
    dW = db = None
    if proj_w is not None:
        if proj_w.dtype != torch.float32 or not proj_w.is_contiguous() or proj_w.shape[-2:] != (d, d):
            raise ValueError("proj_w must be a contiguous float32 [d, d] or [Hq, d, d] tensor")
        proj_heads = 1 if proj_w.dim() == 2 else proj_w.shape[0]
        if proj_grads is not None:
            dW, db = proj_grads
        else:
            dW = torch.empty_like(proj_w)
            db = None if proj_b is None else torch.empty(proj_w.shape[:-1], **f32)
    elif proj_b is not None:
        raise ValueError("proj_b without proj_w")
    gated = lin_mode == SLA_LIN_GLOBAL_GATED
    if gated and dw_gate is None:
        dw_gate = torch.empty((Hq, d), **f32)
    if k_shift is not None and (k_shift.dtype != torch.float32 or not k_shift.is_contiguous()
                                or tuple(k_shift.shape) != (B, Hkv, d)):
        raise ValueError("k_shift must be a contiguous float32 [B, Hkv, d] tensor")
    ws_bytes = sla_attn_bwd_ext_workspace_bytes(B, Hq, Hkv, N, d, lin_mode, causal, group_map, proj_heads)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    descs = [tensor_desc(x) for x in (q, k, v, o, dout)]
    dq, dk, dv = grads
    _check("sla_attn_bwd_ext", lib().sla_attn_bwd_ext(
        *[ctypes.byref(x) for x in descs], _ptr(lse), n_valid, float(scale), lin_mode, int(causal), int(window),
        int(group_map), _ptr(maps["crit_rowptr"]), _ptr(maps["crit_idx"]), _ptr(maps.get("crit_flags")),
        _ptr(maps.get("marg_bits")), _ptr(S), _ptr(u), _ptr(H_all), _ptr(z_all), _ptr(w_gate), _ptr(k_shift),
        _ptr(proj_w), _ptr(proj_b), proj_heads, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW), _ptr(db), _ptr(dw_gate),
        _ptr(workspace), workspace.numel(), _stream(q.device)))
    out = (dq, dk, dv)
    if proj_w is not None:
        out = out + (dW, db)
    if gated:
        out = out + (dw_gate,)
    return out


def sla_hilbert_order(T, H, W) -> torch.Tensor:
    """Host int32 tensor [T*H*W]: row-major token indices in the order of a 3-D Hilbert curve."""
    out = torch.empty(T * H * W, dtype=torch.int32)
    _check("sla_hilbert_order", lib().sla_hilbert_order(T, H, W, ctypes.c_void_p(out.data_ptr())))
    return out


def sla_permute_rows(x, order, inverse=False, out=None):
    """Gather (inverse=False) or scatter rows of x [B, H, N, d] by a device int32 order of n_order rows."""
    _require_gpu(x, order)
    if out is None:
        out = torch.empty(x.shape, device=x.device, dtype=x.dtype)
    _check("sla_permute_rows", lib().sla_permute_rows(ctypes.byref(tensor_desc(x)), _ptr(order), order.numel(),
                                                      int(inverse), _ptr(out), _stream(x.device)))
    return out


def sla_nsa3_workspace_bytes(B, Hq, Hkv, N, d, dtype, n_valid, window, cmp_block, cmp_stride) -> int:
    return int(lib().sla_nsa3_workspace_bytes(B, Hq, Hkv, N, d, dtype, n_valid, window, cmp_block, cmp_stride))


def sla_nsa3_fwd(q, k, v, n_valid, sel_maps, w_gates, window=512, cmp_block=32, cmp_stride=16, scale=None,
                 out=None, out_dtype=None, workspace=None):
    """Three-branch NSA output [B, Hq, N, d]: gated compressed + selected + window attention.

    sel_maps: the causal selection map of sla_block_map (group-summed scores, window 0);
    w_gates: float32 [3, Hq, d] gate weights (compressed, selected, window).
    """
    _require_gpu(q, k, v, w_gates)
    B, Hq, N, d = q.shape
    scale = (1.0 / d ** 0.5) if scale is None else scale
    if out is None:
        out = torch.empty(q.shape, device=q.device, dtype=out_dtype or q.dtype)
    odt = SLA_F32 if out.dtype == torch.float32 else SLA_BF16
    dt = SLA_BF16 if q.dtype == torch.bfloat16 else SLA_F32
    ws = sla_nsa3_workspace_bytes(B, Hq, k.shape[1], N, d, dt, n_valid, window, cmp_block, cmp_stride)
    if workspace is None:
        workspace = torch.empty(ws, device=q.device, dtype=torch.uint8)
    qd, kd, vd = tensor_desc(q), tensor_desc(k), tensor_desc(v)
    _check("sla_nsa3_fwd", lib().sla_nsa3_fwd(
        ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), n_valid, float(scale), _ptr(sel_maps["crit_rowptr"]),
        _ptr(sel_maps["crit_idx"]), _ptr(sel_maps["crit_flags"]), window, cmp_block, cmp_stride, _ptr(w_gates),
        _ptr(out), odt, _ptr(workspace), ws, _stream(q.device)))
    return out