"""Sparse-linear hybrid attention forward (SLA, SALAD, NSA-style selected blocks) on MI355X.

The compute runs in libsla (HIP, gfx950); this package is its Python binding.
Entry points keep the C names (see include/sla.h):

    sla_pool_scores      block mean pooling of Q, K and pooled scores
    sla_key_mean         smooth-K shift (mean key of each head) from the pooled key blocks
    sla_block_map        critical / marginal / negligible classification as CSR lists
    sla_block_map_noalloc  the same without a workspace (static device scratch), for callers that cannot allocate
    sla_linear_kv_reduce per-key-block linear states H_j = phi(K_j)^T V_j, z_j
    sla_marginal_states  per-row sums of the marginal states (also done inside sla_attn_fwd)
    sla_attn_fwd         block-sparse softmax attention + fused linear epilogue
    sla_attn_bwd         dQ, dK, dV of the SLA layer for a fixed block map
    sla_attn_bwd_ext     the same for every forward mode (SALAD gate, NSA causal maps, GQA)
    sla_hilbert_order    token order of a video latent grid along a 3-D Hilbert curve (host)
    sla_nsa3_fwd         NSA with compressed, selected and window branches, gated
    sla_permute_rows     apply / undo a token order on [B, H, N, d] rows

`SlaForward` strings the four calls into one layer forward with every buffer
allocated up front, so a step launches kernels only.  `sla_attention` is the same forward as a
differentiable function (torch autograd, gradients through sla_attn_bwd_ext).
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import (  # noqa: F401
    BLOCK, SLA_BF16, SLA_F32, SLA_LIN_GLOBAL_GATED, SLA_LIN_MARGINAL, SLA_LIN_NONE, SLA_LIN_ROW_STATES, SlaError, alloc_block_map,
    lib, sla_abi_version, sla_attn_bwd, sla_attn_bwd_ext, sla_attn_bwd_ext_workspace_bytes,
    sla_attn_bwd_workspace_bytes, sla_attn_fwd, sla_attn_workspace_bytes,
    sla_hilbert_order, sla_nsa3_fwd, sla_nsa3_workspace_bytes, sla_permute_rows, sla_block_map, sla_block_map_capacity,
    sla_block_map_noalloc,
    sla_block_map_workspace_bytes, sla_counts, sla_key_mean, sla_kv_reduce_workspace_bytes, sla_linear_kv_reduce,
    sla_marginal_states, sla_pool_scores, sla_status_str, tensor_desc,
)


class SlaForward:
    """One attention-layer forward through libsla with preallocated buffers.

    mode "sla":   top kh_bp critical, bottom kl_bp negligible, linear attention on marginal blocks.
    mode "salad": top kh_bp sparse blocks plus the gated linear branch over all keys (w_gate [Hq, d]).
    mode "nsa":   causal, GQA-shared selection of n_sel blocks plus a window of `window` tokens.
    proj_w / proj_b (sla mode): the learned projection of the linear branch, [d, d] or [Hq, d, d]
    (out x in) and [d] or [Hq, d]; None = identity.  smooth_k (sla and salad modes): the linear
    branch uses the keys minus their mean over the valid tokens of each head.
    token_order: optional int32 order of the n_valid tokens (e.g. sla_hilbert_order of the latent
    grid): Q, K, V are gathered into that order before the layer and the output is scattered back.
    """

    def __init__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_valid: int, mode: str,
                 kh_bp: int = 0, kl_bp: int = 0, n_sel: int = 0, window: int = 0,
                 w_gate: Optional[torch.Tensor] = None, scale: Optional[float] = None, out_dtype=None,
                 proj_w: Optional[torch.Tensor] = None, proj_b: Optional[torch.Tensor] = None,
                 smooth_k: bool = False, training: bool = False, token_order: Optional[torch.Tensor] = None):
        self.order = None
        self.q_in, self.k_in, self.v_in = q, k, v
        if token_order is not None:
            if token_order.numel() != n_valid:
                raise ValueError("token_order must order the n_valid tokens")
            self.order = token_order.to(device=q.device, dtype=torch.int32).contiguous()
            q, k, v = (torch.empty(x.shape, device=x.device, dtype=x.dtype) for x in (q, k, v))
        self.q, self.k, self.v = q, k, v
        self.n_valid = n_valid
        self.mode = mode
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        nb = N // BLOCK
        self.scale = (1.0 / d ** 0.5) if scale is None else scale
        self.window = 0
        if mode == "sla":
            self.n_crit, self.n_negl = sla_counts(nb, kh_bp, kl_bp)
            self.causal, self.group = False, False
            self.lin = SLA_LIN_MARGINAL
        elif mode == "salad":
            self.n_crit, _ = sla_counts(nb, kh_bp, 0)
            self.n_negl = 0
            self.causal, self.group = False, False
            self.lin = SLA_LIN_GLOBAL_GATED
            if w_gate is None:
                raise ValueError("salad mode needs w_gate [Hq, d]")
        elif mode == "nsa":
            self.n_crit, self.n_negl = n_sel, 0
            self.causal, self.group = True, True
            self.window = window
            self.lin = SLA_LIN_NONE
        else:
            raise ValueError(f"unknown mode {mode}")
        self.w_gate = None if w_gate is None else w_gate.to(device=q.device, dtype=torch.float32).contiguous()
        if (proj_w is not None or proj_b is not None) and mode != "sla":
            raise ValueError("proj_w / proj_b apply to the sla mode's linear branch")
        if proj_w is None and proj_b is not None:
            raise ValueError("proj_b needs proj_w")
        as32 = lambda x: None if x is None else x.to(device=q.device, dtype=torch.float32).contiguous()
        self.proj_w, self.proj_b = as32(proj_w), as32(proj_b)
        if smooth_k and mode == "nsa":
            raise ValueError("smooth_k applies to a linear branch (sla or salad mode)")
        self.smooth_k = smooth_k
        dev = q.device
        f = dict(device=dev, dtype=torch.float32)
        Hs = Hkv if self.group else Hq
        self.pool = dict(q_pool=torch.empty((B, Hq, nb, d), **f), k_pool=torch.empty((B, Hkv, nb, d), **f),
                         scores=torch.empty((B, Hs, nb, nb), **f))
        self.maps = alloc_block_map(B, Hs, nb, nb, self.n_crit, self.n_negl, self.causal, self.window, dev,
                                    want_marg=self.lin == SLA_LIN_MARGINAL)
        self.kv = {}
        if self.lin == SLA_LIN_MARGINAL:
            self.kv = dict(H=torch.empty((B, Hkv, nb, d, d), device=dev, dtype=torch.bfloat16),
                           z=torch.empty((B, Hkv, nb, d), **f),
                           workspace=None, workspace_bytes=0)
        elif self.lin == SLA_LIN_GLOBAL_GATED:
            ws = sla_kv_reduce_workspace_bytes(B, Hkv, N, d, False, True)
            self.kv = dict(H_all=torch.empty((B, Hkv, d, d), **f), z_all=torch.empty((B, Hkv, d), **f),
                           workspace=torch.empty(ws, device=dev, dtype=torch.uint8), workspace_bytes=ws)
        self.k_mean = torch.empty((B, Hkv, d), **f) if smooth_k else None
        # The key-state pass reads K anyway: when it runs without a shift, it also writes the key
        # block means, and the pooling pass reads only Q.  For bf16 K (exact fp64 block sums) the
        # means are the pooling pass's bit for bit, so the block map does not change.
        self.fuse_key_pooling = self.lin != SLA_LIN_NONE and not smooth_k and k.dtype == torch.bfloat16
        # training: the forward also writes each row's log-sum-exp, which backward() reads
        self.lse = torch.empty((B, Hq, N), **f) if training else None
        self.bwd_ws = None
        self.row_states = None
        if self.lin == SLA_LIN_MARGINAL:
            # per-row marginal sums, filled by sla_marginal_states before the attention call
            self.row_states = (torch.empty((B * Hs * nb, d, d), device=dev, dtype=torch.bfloat16),
                               torch.empty((B * Hs * nb, d), **f))
        self.out = torch.empty(q.shape, device=dev, dtype=out_dtype or q.dtype)
        # with a token order the layer writes its output in that order, then scatters it back
        self.out_ordered = self.out if self.order is None else torch.empty_like(self.out)

    def reorder(self):
        """Gather Q, K, V into the token order (no-op without one)."""
        if self.order is not None:
            for src, dst in ((self.q_in, self.q), (self.k_in, self.k), (self.v_in, self.v)):
                sla_permute_rows(src, self.order, out=dst)

    def restore(self):
        """Scatter the output back to the original token order (no-op without one)."""
        if self.order is not None:
            sla_permute_rows(self.out_ordered, self.order, inverse=True, out=self.out)
        return self.out

    def pool_scores(self, k_pooled: bool = False):
        """Pooled Q and K and the pooled scores; k_pooled: the key block means are already in
        self.pool["k_pool"] (from kv_reduce(k_pool=True)), so only Q is pooled."""
        return sla_pool_scores(self.q, self.k, self.n_valid, group_sum=self.group, causal=self.causal,
                               scale=self.scale, out=self.pool, k_pooled=k_pooled)

    def pooling(self, k_pooled: bool = False):
        """The pooling half of pool_scores: block means of Q (and of K unless k_pooled)."""
        return sla_pool_scores(self.q, self.k, self.n_valid, group_sum=self.group, causal=self.causal,
                               scale=self.scale, out=self.pool, k_pooled=k_pooled, want_scores=False)

    def scoring(self):
        """The scoring half of pool_scores, from the block means pooling() (and kv_reduce) wrote."""
        return sla_pool_scores(self.q, self.k, self.n_valid, group_sum=self.group, causal=self.causal,
                               scale=self.scale, out=self.pool, k_pooled=True, q_pooled=True)

    def block_map(self):
        return sla_block_map(self.pool["scores"], self.n_crit, self.n_negl, causal=self.causal,
                             window=self.window, out=self.maps)

    def kv_reduce(self, k_pool: bool = False):
        """Linear-branch key states (after pool_scores when smooth_k: the shift comes from k_pool).
        k_pool: also write the key block means into self.pool["k_pool"] (K is read once for both)."""
        if self.lin != SLA_LIN_NONE:
            if self.smooth_k:
                sla_key_mean(self.pool["k_pool"], self.n_valid, out=self.k_mean)
            sla_linear_kv_reduce(self.k, self.v, self.n_valid, out=self.kv, k_shift=self.k_mean,
                                 k_pool=self.pool["k_pool"] if k_pool else None)
        return self.kv

    def marginal_states(self, maps=None):
        """Per-row sums of the marginal key states (SLA mode only)."""
        if self.lin == SLA_LIN_MARGINAL:
            m = maps or self.maps
            sla_marginal_states(self.kv["H"], self.kv["z"], self.q.shape[1], self.group, m["marg_bits"],
                                out=self.row_states)
        return self.row_states

    def attention(self, maps=None):
        kv = self.kv
        if self.lin == SLA_LIN_MARGINAL:
            S, u = self.row_states
            return sla_attn_fwd(self.q, self.k, self.v, self.n_valid, maps or self.maps,
                                lin_mode=SLA_LIN_ROW_STATES, scale=self.scale, H=S, z=u, out=self.out_ordered,
                                proj_w=self.proj_w, proj_b=self.proj_b, lse=self.lse)
        return sla_attn_fwd(self.q, self.k, self.v, self.n_valid, maps or self.maps, lin_mode=self.lin,
                            scale=self.scale, causal=self.causal, window=self.window, group_map=self.group,
                            H_all=kv.get("H_all"), z_all=kv.get("z_all"), w_gate=self.w_gate, out=self.out_ordered,
                            lse=self.lse)

    def backward(self, dout: torch.Tensor, maps=None, grads=None):
        """Gradients of sum(dout * out) after run() (or attention()) with training=True, for the same
        block map: (dq, dk, dv) fp32 (dk, dv per KV head); sla mode with a Proj weight adds (dW, db),
        db None without a bias; salad mode adds dw_gate [Hq, d]."""
        if self.lse is None:
            raise ValueError("construct the layer with training=True to keep what the backward needs")
        proj_heads = 0 if self.proj_w is None else (1 if self.proj_w.dim() == 2 else self.proj_w.shape[0])
        lin = SLA_LIN_ROW_STATES if self.lin == SLA_LIN_MARGINAL else self.lin
        B, Hq, N, d = self.q.shape
        Hkv = self.k.shape[1]
        if self.bwd_ws is None:
            ws = sla_attn_bwd_ext_workspace_bytes(B, Hq, Hkv, N, d, lin, self.causal, self.group, proj_heads)
            self.bwd_ws = torch.empty(max(ws, 1), device=self.q.device, dtype=torch.uint8)
        S, u = self.row_states if self.row_states is not None else (None, None)
        extra = dict(scale=self.scale, causal=self.causal, window=self.window, group_map=self.group, S=S, u=u,
                     H_all=self.kv.get("H_all"), z_all=self.kv.get("z_all"),
                     w_gate=self.w_gate if lin == SLA_LIN_GLOBAL_GATED else None, k_shift=self.k_mean,
                     proj_w=self.proj_w, proj_b=self.proj_b, workspace=self.bwd_ws)
        if self.order is None:
            return sla_attn_bwd_ext(self.q, self.k, self.v, self.out, dout, self.lse, self.n_valid,
                                    maps or self.maps, lin, grads=grads, **extra)
        # in the token order, then scattered back (the order is a permutation: its gradient is the inverse)
        dout_r = sla_permute_rows(dout, self.order)
        g_r = sla_attn_bwd_ext(self.q, self.k, self.v, self.out_ordered, dout_r, self.lse, self.n_valid,
                               maps or self.maps, lin, **extra)
        if grads is None:
            grads = tuple(torch.empty_like(x) for x in g_r[:3])
        for src, dst in zip(g_r[:3], grads):
            sla_permute_rows(src, self.order, inverse=True, out=dst)
        return tuple(grads) + tuple(g_r[3:])

    def capture(self) -> "torch.cuda.CUDAGraph":
        """Record one run() into a HIP graph and return it; graph.replay() then launches the whole
        forward from the host at once (launch-bound sizes, serving loops).  The graph reads the
        layer's input tensors and writes self.out: copy new inputs into q, k, v (as given to the
        constructor) before a replay.  Every buffer is allocated by the constructor and no pass
        clears memory with a memset, so replays recompute everything from the inputs."""
        dev = self.q.device
        main = torch.cuda.current_stream(dev)
        warm = torch.cuda.Stream(device=dev)
        warm.wait_stream(main)
        with torch.cuda.stream(warm):          # first calls (library load, workspaces) off the capture
            self.run()
        main.wait_stream(warm)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run()
        return graph

    def run(self, overlap: bool = False, events=None) -> torch.Tensor:
        """One full forward: (token order,) pool, scores, block map, linear states, marginal sums,
        attention (, order undone).  With fuse_key_pooling the pooling pass reads only Q, and the linear
        key states, which follow it, also write the key block means that the scores use.

        overlap: the linear key states depend only on K and V (and, with smooth-K, on the pooled
        keys), so they can run on a second stream while the scores and the block map run; the
        marginal sums follow on that stream once the map is there, and the attention waits for them.
        (Measured at the wan13b layer: under 1% faster, the overlapped passes sharing HBM.)
        events: optional dict pass name -> (start, end) torch.cuda.Event pairs, recorded around each
        pass on the stream it runs on.
        """
        def timed(name, fn):
            if events is not None and name in events:
                events[name][0].record()
                fn()
                events[name][1].record()
            else:
                fn()
        timed("reorder", self.reorder)
        if self.fuse_key_pooling and not overlap:
            # Q's block means first: the pass reads Q only, and the key-state pass's writes of
            # the per-block states are still draining from the caches when the next pass runs
            timed("pool", lambda: self.pooling(k_pooled=True))
            timed("kv_reduce", lambda: self.kv_reduce(k_pool=True))
            timed("scores", self.scoring)
            for name in ("block_map", "marginal_states", "attention"):
                timed(name, getattr(self, name))
            timed("restore", self.restore)
            return self.out
        if not overlap or self.lin == SLA_LIN_NONE:
            timed("pool", self.pooling)
            timed("scores", self.scoring)
            for name in ("block_map", "kv_reduce", "marginal_states", "attention"):
                timed(name, getattr(self, name))
            timed("restore", self.restore)
            return self.out
        if getattr(self, "_side", None) is None:
            self._side = torch.cuda.Stream(device=self.q.device)
            self._ev = [torch.cuda.Event() for _ in range(3)]
        main, side = torch.cuda.current_stream(self.q.device), self._side
        e_in, e_map, e_marg = self._ev
        if not self.smooth_k:
            e_in.record(main)                  # inputs (and their reorder) are ready
        timed("pool", self.pooling)
        if self.smooth_k:
            e_in.record(main)                  # the key shift needs the pooled keys
        timed("scores", self.scoring)
        with torch.cuda.stream(side):
            side.wait_event(e_in)
            timed("kv_reduce", self.kv_reduce)
        timed("block_map", self.block_map)
        e_map.record(main)
        with torch.cuda.stream(side):
            side.wait_event(e_map)
            timed("marginal_states", self.marginal_states)
            e_marg.record(side)
        main.wait_event(e_marg)
        timed("attention", self.attention)
        timed("restore", self.restore)
        return self.out


class _SlaAttention(torch.autograd.Function):
    """Autograd glue: forward = SlaForward(training=True).run(), backward = its backward() for the
    forward's own block map (the map is a discrete function of the inputs; like every top-k
    selection it passes no gradient)."""

    @staticmethod
    def forward(ctx, q, k, v, w_gate, proj_w, proj_b, cfg):
        layer = SlaForward(q.detach(), k.detach(), v.detach(), training=True,
                           w_gate=None if w_gate is None else w_gate.detach(),
                           proj_w=None if proj_w is None else proj_w.detach(),
                           proj_b=None if proj_b is None else proj_b.detach(), **cfg)
        out = layer.run()
        ctx.layer = layer
        ctx.dtypes = tuple(None if x is None else x.dtype for x in (q, k, v, w_gate, proj_w, proj_b))
        ctx.save_for_backward(out)      # an in-place change of the output is caught before backward
        return out

    @staticmethod
    def backward(ctx, dout):
        ctx.saved_tensors               # version check of the output
        layer = ctx.layer
        g = layer.backward(dout.to(layer.q.dtype).contiguous())
        dq, dk, dv = g[:3]
        dW = db = dwg = None
        if layer.proj_w is not None:
            dW, db = g[3], g[4]
        if layer.lin == SLA_LIN_GLOBAL_GATED:
            dwg = g[-1]
        grads = (dq, dk, dv, dwg, dW, db)
        return tuple(None if x is None or t is None else x.to(t) for x, t in zip(grads, ctx.dtypes)) + (None,)


def sla_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_valid: int, mode: str = "sla", *,
                  kh_bp: int = 0, kl_bp: int = 0, n_sel: int = 0, window: int = 0,
                  w_gate: Optional[torch.Tensor] = None, proj_w: Optional[torch.Tensor] = None,
                  proj_b: Optional[torch.Tensor] = None, smooth_k: bool = False, scale: Optional[float] = None,
                  token_order: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Differentiable layer forward: the output of SlaForward(...).run() for these arguments, with
    gradients for q, k, v and, where given, w_gate (salad), proj_w and proj_b (sla) through libsla's
    backward.  Shapes and modes as in SlaForward: q [B, Hq, N, d], k and v [B, Hkv, N, d] on the GPU,
    N a multiple of 64, N - 64 < n_valid <= N; rows past n_valid get zero output and zero gradient.
    Each call builds the layer's buffers; for repeated steps of one shape keep a SlaForward instead."""
    cfg = dict(n_valid=n_valid, mode=mode, kh_bp=kh_bp, kl_bp=kl_bp, n_sel=n_sel, window=window,
               smooth_k=smooth_k, scale=scale, token_order=token_order)
    tensors = (q, k, v, w_gate, proj_w, proj_b)
    if not (torch.is_grad_enabled() and any(x is not None and x.requires_grad for x in tensors)):
        # nothing to differentiate: the plain forward, without keeping what the backward needs
        return SlaForward(q, k, v, w_gate=w_gate, proj_w=proj_w, proj_b=proj_b, **cfg).run()
    return _SlaAttention.apply(*tensors, cfg)
