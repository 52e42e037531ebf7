"""Training-side wrappers over the C ABI: a 2:4 sparse linear layer with an
optional low-rank adapter, its autograd function, and AdamW on its compressed
values.

Orchestration only: every arithmetic step runs in libslope.so through the
binding in this package (the forward product with the fused adapter term, the
double-pruned dX product with the adapter's dX term, the weight gradient at the
static mask, the adapter gradients, the optimizer step fused with the double
prune and the rewrite of both GEMM operands, and the operand packing).  torch
provides device memory, streams and the autograd graph.

Layer state, per SLoPe (explainer 2.A and 2.B; discussion page, "Memory
Footprint Reduction During Pretraining and Inference" and "Choice of
Optimizer"):

    values  [N, K/2]        kept weights of W_s (an nn.Parameter; its .grad is
                            the weight gradient in the same slot order)
    meta    [N, K/32] int32 positions of the kept weights (static mask)
    packed_s                W_s in tile-chunk form, the forward's operand
    packed_dpT              the double-pruned transposed weight W_dp^T, kept
                            only in tile-chunk form (the dX product's operand)
    L [K, r], R [r, N]      the adapter (nn.Parameters), when rank > 0

Formats: bf16 or fp16 weights and activations (one format per layer), with K
and N multiples of 16 (the packed operand format).
"""
from __future__ import annotations

import torch

from . import (slope_adamw, slope_adamw_double_prune_packed, slope_double_prune_packed, slope_lowrank_grads_packed,
               slope_lowrank_grads_workspace_bytes, slope_lowrank_workspace_bytes, slope_masked_wgrad_packed,
               slope_pack_sparse, slope_pack_tokens, slope_packed_sparse_bytes, slope_packed_tokens_bytes,
               slope_prune_compress24, slope_spmm_bwd_dx_packed, slope_spmm_bwd_dx_packed_tokens,
               slope_spmm_fwd_packed, slope_wgrad_split_workspace_bytes)

__all__ = ["SparseLinear", "SparseAdamW", "training_state_bytes"]


def _bytes(n, device):
    return torch.empty(max(16, n), dtype=torch.uint8, device=device)


class _SparseLinearFn(torch.autograd.Function):
    """Y = X . W_s^T (+ (X . L) . R); gradients dX (through W_dp), dW at the
    static mask, dL and dR."""

    @staticmethod
    def forward(ctx, X, values, L, R, layer):
        T = X.shape[0]
        N, K, r = layer.out_features, layer.in_features, layer.rank
        Y = torch.empty((T, N), dtype=X.dtype, device=X.device)
        ws = None
        if r > 0:
            ws = _bytes(slope_lowrank_workspace_bytes(T, K, r, N), X.device)
            slope_spmm_fwd_packed(X, layer.packed_s, N, Y, L=L, R=R, workspace=ws)
        else:
            slope_spmm_fwd_packed(X, layer.packed_s, N, Y)
        ctx.layer, ctx.ws = layer, ws
        ctx.save_for_backward(X, L, R)
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, L, R = ctx.saved_tensors
        layer = ctx.layer
        dY = dY.contiguous()
        T = X.shape[0]
        N, K, r = layer.out_features, layer.in_features, layer.rank
        need_x, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        need_a = r > 0 and (ctx.needs_input_grad[2] or ctx.needs_input_grad[3])
        dX = dW = dL = dR = None
        ws_bwd = None
        # the weight gradients read X and dY as token chunks: the dX product
        # writes dY's while it streams dY; X's come from the packing pass (a
        # forward that wrote them would hold a second copy of X until here)
        dYp = _bytes(slope_packed_tokens_bytes(T, N), dY.device) if need_w or need_a else None
        if need_x:
            dX = torch.empty((T, K), dtype=dY.dtype, device=dY.device)
            if r > 0:
                ws_bwd = _bytes(slope_lowrank_workspace_bytes(T, N, r, K), dY.device)
            if dYp is not None:
                slope_spmm_bwd_dx_packed_tokens(dY, layer.packed_dpT, K, dX, dYp, L=L if r > 0 else None,
                                                R=R if r > 0 else None, workspace=ws_bwd)
            else:
                slope_spmm_bwd_dx_packed(dY, layer.packed_dpT, K, dX, L=L if r > 0 else None,
                                         R=R if r > 0 else None, workspace=ws_bwd)
        elif dYp is not None:
            slope_pack_tokens(dY, dYp)
        if need_w or need_a:
            Xp = _bytes(slope_packed_tokens_bytes(T, K), X.device)
            slope_pack_tokens(X, Xp)
            if need_w:
                dW = torch.empty_like(layer.values)
                wsp = _bytes(slope_wgrad_split_workspace_bytes(T, N, K), X.device)
                slope_masked_wgrad_packed(dYp, Xp, T, N, K, layer.meta, dW, in_dtype=X.dtype, split_workspace=wsp)
            if need_a:
                dL, dR = torch.empty_like(L), torch.empty_like(R)
                wsg = _bytes(slope_lowrank_grads_workspace_bytes(T, K, r, N), X.device)
                slope_lowrank_grads_packed(X, dY, Xp, dYp, L, R, wsg, dL, dR, fwd_workspace=ctx.ws,
                                           bwd_workspace=ws_bwd)
        ctx.ws = None
        return dX, dW, dL, dR, None


class SparseLinear(torch.nn.Module):
    """2:4 sparse linear layer y = x . W_s^T (+ (x . L) . R), built from a
    dense bf16 or fp16 weight [out_features, in_features] on the GPU: magnitude
    2:4 pruning along the input dimension (the mask is fixed from then on),
    compression, the double-pruned transposed copy and the packed operands."""

    def __init__(self, weight: torch.Tensor, L: torch.Tensor | None = None, R: torch.Tensor | None = None):
        super().__init__()
        if weight.dtype not in (torch.bfloat16, torch.float16) or not weight.is_cuda or weight.dim() != 2:
            raise ValueError("weight must be a 2-D bfloat16 or float16 GPU tensor [out_features, in_features]")
        N, K = weight.shape
        if K % 16 or N % 16:
            raise ValueError("in_features and out_features must be multiples of 16")
        if (L is None) != (R is None):
            raise ValueError("give both adapter factors L [K, r] and R [r, N], or neither")
        dev, dt = weight.device, weight.dtype
        self.in_features, self.out_features = K, N
        weight = weight.contiguous()
        # one pass: magnitude 2:4 mask, compressed values and metadata, and
        # W_s's tile chunks (no dense mask is materialised)
        values = torch.empty((N, K // 2), dtype=dt, device=dev)
        meta = torch.empty((N, (K // 4 + 7) // 8), dtype=torch.int32, device=dev)
        packed_s = _bytes(slope_packed_sparse_bytes(N, K), dev)
        slope_prune_compress24(weight, values, meta, packed=packed_s)
        self.values = torch.nn.Parameter(values)
        self.register_buffer("meta", meta)
        self.register_buffer("packed_s", packed_s)
        self.register_buffer("packed_dpT", _bytes(slope_packed_sparse_bytes(K, N), dev))
        if L is not None:
            if L.shape[0] != K or R.shape[1] != N or L.shape[1] != R.shape[0]:
                raise ValueError("adapter shapes must be L [K, r] and R [r, N]")
            self.L = torch.nn.Parameter(L.detach().to(dt).contiguous())
            self.R = torch.nn.Parameter(R.detach().to(dt).contiguous())
            self.rank = L.shape[1]
        else:
            self.L = self.R = None
            self.rank = 0
        slope_double_prune_packed(self.values, self.meta, N, K, self.packed_dpT)

    @torch.no_grad()
    def refresh(self) -> None:
        """Re-derive both GEMM operands from the current values: W_s's tile
        chunks and the double-pruned W_dp^T's (needed after changing `values`
        by other means than SparseAdamW)."""
        N, K = self.out_features, self.in_features
        slope_pack_sparse(self.values, self.meta, N, K, self.packed_s)
        slope_double_prune_packed(self.values, self.meta, N, K, self.packed_dpT)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features or x.dtype != self.values.dtype:
            raise ValueError("input must have in_features columns and the layer's format")
        lead = x.shape[:-1]
        y = _SparseLinearFn.apply(x.reshape(-1, self.in_features).contiguous(), self.values, self.L, self.R, self)
        return y.reshape(*lead, self.out_features)


class SparseAdamW(torch.optim.Optimizer):
    """AdamW for SparseLinear layers (and any other bf16 / fp32 parameters).

    The compressed values of each layer are updated by the fused kernel that
    also rewrites them inside W_s's tile chunks and re-derives the
    double-pruned transposed weight's tile chunks, so both GEMM operands are
    current after one pass; other parameters (the adapter factors) take the
    elementwise kernel.  Moments are fp32, two per stored value: the
    optimizer state of a 2:4 weight is half that of a dense one."""

    def __init__(self, modules, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, extra_params=()):
        modules = list(modules)
        self._layer_of = {}
        params = []
        for m in modules:
            for layer in (m.modules() if isinstance(m, torch.nn.Module) else [m]):
                if isinstance(layer, SparseLinear):
                    self._layer_of[layer.values] = layer
        for m in modules:
            params.extend(p for p in m.parameters() if p.requires_grad)
        params.extend(extra_params)
        seen, uniq = set(), []
        for p in params:
            if id(p) not in seen:
                seen.add(id(p))
                uniq.append(p)
        super().__init__(uniq, dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay))

    @torch.no_grad()
    def step(self, closure=None):
        loss = closure() if closure is not None else None
        for group in self.param_groups:
            b1, b2 = group["betas"]
            hp = dict(lr=group["lr"], beta1=b1, beta2=b2, eps=group["eps"], weight_decay=group["weight_decay"])
            for p in group["params"]:
                if p.grad is None:
                    continue
                st = self.state[p]
                if not st:
                    st["step"] = 0
                    st["exp_avg"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                    st["exp_avg_sq"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                st["step"] += 1
                g = p.grad.contiguous()
                layer = self._layer_of.get(p)
                if layer is not None:
                    slope_adamw_double_prune_packed(p, layer.meta, g, st["exp_avg"], st["exp_avg_sq"],
                                                    layer.out_features, layer.in_features, layer.packed_s,
                                                    layer.packed_dpT, st["step"], **hp)
                else:
                    slope_adamw(p, g, st["exp_avg"], st["exp_avg_sq"], st["step"], **hp)
        return loss


def training_state_bytes(layer: SparseLinear, optimizer: SparseAdamW | None = None) -> dict:
    """Bytes the layer's training state occupies on the GPU, next to a dense
    bf16 layer of the same shape trained with AdamW (weight, gradient, two fp32
    moments).  `canonical` counts what the pages' accounting counts: the
    compressed weight, its double-pruned copy (held only as tile chunks, 1.125
    bytes per weight up to the chunks' padding), the gradient at the kept
    weights and two moments per kept weight; no separate binary mask is kept
    (the metadata is the mask).  `with_packed_operands` adds W_s's tile-chunk
    copy, the forward's operand."""
    def nb(t):
        return 0 if t is None else t.numel() * t.element_size()
    N, K = layer.out_features, layer.in_features
    vals = layer.values
    grad = vals.numel() * vals.element_size()
    if optimizer is not None and vals in optimizer.state and optimizer.state[vals]:
        moments = nb(optimizer.state[vals]["exp_avg"]) + nb(optimizer.state[vals]["exp_avg_sq"])
    else:
        moments = 2 * 4 * vals.numel()
    canonical = nb(vals) + nb(layer.meta) + nb(layer.packed_dpT) + grad + moments
    dense = N * K * (2 + 2 + 4 + 4)
    packed = canonical + nb(layer.packed_s)
    return {"canonical": canonical, "with_packed_operands": packed, "dense_adamw": dense,
            "canonical_ratio": canonical / dense, "with_packed_ratio": packed / dense}
