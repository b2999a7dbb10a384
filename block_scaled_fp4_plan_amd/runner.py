"""Buffer management around the C entry points (torch supplies device memory and the stream).

Nothing here computes: each helper allocates the tensors a call needs and invokes the library.
"""

from dataclasses import dataclass

import torch

from . import (
    BFP4_FORMAT_MXFP4,
    BFP4_FORMAT_NVFP4,
    BFP4_WEIGHTS_BF16,
    BFP4_WEIGHTS_F32,
    BFP4_ACT_RELU2,
    BFP4_ACT_SWIGLU,
    GATED_ACTS,
    BFP4_SCALE_PER_GROUP,
    BFP4_SCALE_PER_ROW,
    bfp4_check_plan,
    bfp4_check_topk_ids,
    bfp4_fused_moe_nvfp4,
    bfp4_fused_moe_nvfp4_noalloc,
    bfp4_fused_moe_mx,
    bfp4_fused_moe_w4a16,
    bfp4_moe_plan,
    bfp4_moe_plan_quantize,
    bfp4_panel_bytes,
    bfp4_plan_capacity,
    bfp4_plan_workspace_size,
    bfp4_prepare_weights,
    bfp4_prepare_weights_mxfp4,
    bfp4_quantize_mxfp4,
    bfp4_quantize_mxfp8,
    bfp4_quantize_nvfp4,
    bfp4_quantize_workspace_size,
    bfp4_workspace_size,
    bfp4_workspace_size_mx,
    bfp4_workspace_size_w4a16,
)


def weights_dtype(topk_weights):
    """BFP4_WEIGHTS_* code of a routing-weight tensor (FP32 or BF16)."""
    if topk_weights.dtype == torch.float32:
        return BFP4_WEIGHTS_F32
    if topk_weights.dtype == torch.bfloat16:
        return BFP4_WEIGHTS_BF16
    raise TypeError("routing weights must be float32 or bfloat16, not %s" % topk_weights.dtype)


def _bytes(n, device):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def quantize(x_bf16, mode=BFP4_SCALE_PER_ROW, group_rows=0, fixed_encode_scale=1.0, stream=None):
    """NVFP4 of a 2-D BF16 tensor; returns (q [R, C/2] u8, sf [R, C/16] u8, dec f32)."""
    rows, cols = x_bf16.shape
    dev = x_bf16.device
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    nd = rows if mode == BFP4_SCALE_PER_ROW else (rows // group_rows if group_rows else 1)
    dec = torch.empty(max(nd, 1), dtype=torch.float32, device=dev)
    wsb = bfp4_quantize_workspace_size(rows, mode, group_rows)
    ws = _bytes(wsb, dev)
    bfp4_quantize_nvfp4(x_bf16, rows, cols, x_bf16.stride(0), mode, group_rows, fixed_encode_scale,
                        q, sf, dec, ws, wsb, stream)
    return q, sf, dec


@dataclass
class PreparedWeights:
    panels: torch.Tensor
    panels_bytes: int
    alpha1_gate: torch.Tensor
    alpha1_up: torch.Tensor
    alpha2: torch.Tensor
    num_local_experts: int
    H: int
    I: int
    gated: bool
    fmt: int = 0              # BFP4_FORMAT_NVFP4 or BFP4_FORMAT_MXFP4


def prepare_weights_mxfp4(w1_bf16, w2_bf16, gated=True, keep_linear=False, stream=None):
    """MXFP4 (E8M0 scales per 32 values) of BF16 stacks W1 [E, N1, H] and W2 [E, H, I], then the
    panel layout, for the weight-only mode (alphas of 1).  Returns PreparedWeights (and the
    linear MXFP4 tensors when keep_linear)."""
    E, N1, H = w1_bf16.shape
    I = w2_bf16.shape[2]
    dev = w1_bf16.device
    q1 = torch.empty((E * N1, H // 2), dtype=torch.uint8, device=dev)
    s1 = torch.empty((E * N1, H // 32), dtype=torch.uint8, device=dev)
    q2 = torch.empty((E * H, I // 2), dtype=torch.uint8, device=dev)
    s2 = torch.empty((E * H, I // 32), dtype=torch.uint8, device=dev)
    w1 = w1_bf16.reshape(E * N1, H)
    w2 = w2_bf16.reshape(E * H, I)
    bfp4_quantize_mxfp4(w1, E * N1, H, w1.stride(0), q1, s1, stream)
    bfp4_quantize_mxfp4(w2, E * H, I, w2.stride(0), q2, s2, stream)
    nb = bfp4_panel_bytes(E, H, I, int(gated))
    panels = _bytes(nb, dev)
    bfp4_prepare_weights_mxfp4(q1, s1, q2, s2, E, H, I, int(gated), panels, nb, stream)
    ones = torch.ones(E, dtype=torch.float32, device=dev)
    pw = PreparedWeights(panels, nb, ones, ones.clone(), ones.clone(), E, H, I, gated,
                         BFP4_FORMAT_MXFP4)
    if keep_linear:
        return pw, (q1.reshape(E, N1, H // 2), s1.reshape(E, N1, H // 32),
                    q2.reshape(E, H, I // 2), s2.reshape(E, H, I // 32))
    return pw


def prepare_weights(w1_bf16, w2_bf16, gated=True, keep_linear=False, stream=None):
    """Per-expert NVFP4 of BF16 stacks W1 [E, N1, H] ([gate; up] when gated) and W2 [E, H, I],
    then the gfx950 panel layout.  Returns PreparedWeights (and the linear NVFP4 tensors when
    keep_linear)."""
    E, N1, H = w1_bf16.shape
    I = w2_bf16.shape[2]
    dev = w1_bf16.device
    q1, s1, a1 = quantize(w1_bf16.reshape(E * N1, H), BFP4_SCALE_PER_GROUP, N1, stream=stream)
    q2, s2, a2 = quantize(w2_bf16.reshape(E * H, I), BFP4_SCALE_PER_GROUP, H, stream=stream)
    nb = bfp4_panel_bytes(E, H, I, int(gated))
    panels = _bytes(nb, dev)
    bfp4_prepare_weights(q1, s1, q2, s2, E, H, I, int(gated), panels, nb, stream)
    pw = PreparedWeights(panels, nb, a1, a1.clone(), a2, E, H, I, gated)
    if keep_linear:
        return pw, (q1.reshape(E, N1, H // 2), s1.reshape(E, N1, H // 16),
                    q2.reshape(E, H, I // 2), s2.reshape(E, H, I // 16))
    return pw


class MoePlanBuffers:
    """Plan arrays for fixed (M, top_k, num_local_experts, block_m)."""

    def __init__(self, M, top_k, num_local_experts, block_m, device):
        self.M, self.top_k, self.nloc, self.block_m = M, top_k, num_local_experts, block_m
        self.capacity = bfp4_plan_capacity(M, top_k, num_local_experts, block_m)
        cap = max(self.capacity, 1)
        self.sorted_token_ids = torch.empty(cap, dtype=torch.int32, device=device)
        self.expert_ids = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=device)
        self.num_tokens_post_padded = torch.empty(1, dtype=torch.int32, device=device)
        self.token_to_row = torch.empty((max(M, 1), top_k), dtype=torch.int32, device=device)
        self.ws_bytes = bfp4_plan_workspace_size(M, top_k, num_local_experts)
        self.ws = _bytes(self.ws_bytes, device)

    def build(self, topk_ids, num_experts, local_expert_offset=0, stream=None):
        bfp4_moe_plan(topk_ids, self.M, self.top_k, num_experts, local_expert_offset, self.nloc,
                      self.block_m, self.sorted_token_ids, self.expert_ids,
                      self.num_tokens_post_padded, self.token_to_row, self.capacity, self.ws,
                      self.ws_bytes, stream)
        return self


    def check(self, stream=None):
        """Debug validation of the plan arrays (bfp4_check_plan); waits for the stream and returns
        (bad entries, bad blocks, bad extent)."""
        report = torch.empty(3, dtype=torch.int32, device=self.sorted_token_ids.device)
        bfp4_check_plan(self.sorted_token_ids, self.expert_ids, self.num_tokens_post_padded,
                        self.capacity, self.M, self.top_k, self.nloc, self.block_m, report, stream)
        torch.cuda.synchronize(report.device)
        return tuple(int(v) for v in report.cpu())


def check_topk_ids(topk_ids, num_experts, stream=None):
    """Debug validation of a routing (bfp4_check_topk_ids); waits for the stream and returns
    (tokens with a repeated expert, ids outside [-1, num_experts), first such token or None)."""
    M, top_k = topk_ids.shape
    report = torch.empty(3, dtype=torch.int32, device=topk_ids.device)
    bfp4_check_topk_ids(topk_ids, M, top_k, num_experts, report, stream)
    torch.cuda.synchronize(report.device)
    dup, bad, first = (int(v) for v in report.cpu())
    return dup, bad, (None if first == 0x7FFFFFFF else first)


class MoeForward:
    """One forward: plan, per-token activation quantization, fused experts (+ finalize)."""

    def __init__(self, weights: PreparedWeights, M, top_k, num_experts, block_m,
                 local_expert_offset=0, do_finalize=True, device="cuda", act=None,
                 noalloc=False):
        """act: a BFP4_ACT_* code; by default SwiGLU for gated weights, squared ReLU otherwise.
        noalloc: call bfp4_fused_moe_nvfp4_noalloc (the library's static scratch) instead of
        passing a workspace."""
        if act is None:
            act = BFP4_ACT_SWIGLU if weights.gated else BFP4_ACT_RELU2
        if (act in GATED_ACTS) != bool(weights.gated):
            raise ValueError("activation %d does not match the weights' gating" % act)
        if weights.fmt != BFP4_FORMAT_NVFP4:
            raise ValueError("the NVFP4 x NVFP4 forward needs NVFP4 weights")
        self.act = act
        self.w = weights
        self.M, self.top_k, self.E, self.block_m = M, top_k, num_experts, block_m
        self.offset = local_expert_offset
        self.do_finalize = do_finalize
        self.plan = MoePlanBuffers(M, top_k, weights.num_local_experts, block_m, device)
        H, I = weights.H, weights.I
        self.a_q = torch.empty((max(M, 1), H // 2), dtype=torch.uint8, device=device)
        self.a_sf = torch.empty((max(M, 1), H // 16), dtype=torch.uint8, device=device)
        self.a_dec = torch.empty(max(M, 1), dtype=torch.float32, device=device)
        self.noalloc = noalloc
        self.ws_bytes = bfp4_workspace_size(M, H, I, top_k, weights.num_local_experts, block_m,
                                            int(do_finalize))
        self.ws = None if noalloc else _bytes(self.ws_bytes + 256, device)
        self.gemm2_out = None
        if not do_finalize:
            self.gemm2_out = torch.empty((max(self.plan.capacity, 1), H), dtype=torch.bfloat16,
                                         device=device)

    def __call__(self, x_bf16, topk_ids, topk_weights, out=None, debug=None, weights=None,
                 stream=None, c2=1.0, routed_scaling_factor=1.0):
        w = self.w if weights is None else weights
        M, H, I = self.M, w.H, w.I
        pl = self.plan
        # routing plan and activation quantization (one launch at decode sizes)
        bfp4_moe_plan_quantize(topk_ids, M, self.top_k, self.E, self.offset, pl.nloc,
                               self.block_m, pl.sorted_token_ids, pl.expert_ids,
                               pl.num_tokens_post_padded, pl.token_to_row, pl.capacity, pl.ws,
                               pl.ws_bytes, x_bf16, H, x_bf16.stride(0), self.a_q, self.a_sf,
                               self.a_dec, stream)
        if out is None and self.do_finalize:
            out = torch.zeros((M, H), dtype=torch.bfloat16, device=x_bf16.device)
        act = self.act
        if (act in GATED_ACTS) != bool(w.gated):
            raise ValueError("activation %d does not match the weights' gating" % act)
        pl = self.plan
        args = (self.a_q, self.a_sf, self.a_dec, w.panels, w.panels_bytes, w.alpha1_gate,
                w.alpha1_up, w.alpha2, c2, pl.sorted_token_ids, pl.expert_ids,
                pl.num_tokens_post_padded, pl.token_to_row, pl.capacity, topk_weights,
                weights_dtype(topk_weights), M, H, I, w.num_local_experts, self.top_k,
                self.block_m, act, routed_scaling_factor, int(self.do_finalize), out,
                self.gemm2_out, debug)
        if self.noalloc:
            bfp4_fused_moe_nvfp4_noalloc(*args, stream)
        else:
            bfp4_fused_moe_nvfp4(*args, self.ws, self.ws_bytes, stream)
        return out if self.do_finalize else (self.gemm2_out, topk_weights, pl.token_to_row)


class MoeForwardW4A16:
    """One forward of the NVFP4 weight-only mode on BF16 activations (decode plans, block_m <=
    32): routing plan, then bfp4_fused_moe_w4a16 (no activation quantization)."""

    def __init__(self, weights: PreparedWeights, M, top_k, num_experts, block_m,
                 local_expert_offset=0, do_finalize=True, device="cuda", act=None):
        if act is None:
            act = BFP4_ACT_SWIGLU if weights.gated else BFP4_ACT_RELU2
        if (act in GATED_ACTS) != bool(weights.gated):
            raise ValueError("activation %d does not match the weights' gating" % act)
        self.act = act
        self.w = weights
        self.M, self.top_k, self.E, self.block_m = M, top_k, num_experts, block_m
        self.offset = local_expert_offset
        self.do_finalize = do_finalize
        self.plan = MoePlanBuffers(M, top_k, weights.num_local_experts, block_m, device)
        self.ws_bytes = bfp4_workspace_size_w4a16(M, weights.H, weights.I, top_k,
                                                  weights.num_local_experts, block_m,
                                                  int(do_finalize))
        self.ws = _bytes(self.ws_bytes + 256, device)
        self.gemm2_out = None
        if not do_finalize:
            self.gemm2_out = torch.empty((max(self.plan.capacity, 1), weights.H),
                                         dtype=torch.bfloat16, device=device)

    def __call__(self, x_bf16, topk_ids, topk_weights, out=None, debug=None, weights=None,
                 stream=None, routed_scaling_factor=1.0):
        w = self.w if weights is None else weights
        M, H, I = self.M, w.H, w.I
        self.plan.build(topk_ids, self.E, self.offset, stream)
        if out is None and self.do_finalize:
            out = torch.zeros((M, H), dtype=torch.bfloat16, device=x_bf16.device)
        pl = self.plan
        bfp4_fused_moe_w4a16(x_bf16, x_bf16.stride(0), w.panels, w.panels_bytes, w.fmt,
                             w.alpha1_gate,
                             w.alpha1_up, w.alpha2, pl.sorted_token_ids, pl.expert_ids,
                             pl.num_tokens_post_padded, pl.token_to_row, pl.capacity,
                             topk_weights, weights_dtype(topk_weights), M, H, I,
                             w.num_local_experts, self.top_k, self.block_m, self.act,
                             routed_scaling_factor, int(self.do_finalize), out, self.gemm2_out,
                             debug, self.ws, self.ws_bytes, stream)
        return out if self.do_finalize else (self.gemm2_out, topk_weights, pl.token_to_row)


def quantize_mxfp8(x_bf16, stream=None):
    """MXFP8 of a 2-D BF16 tensor; returns (q [R, C] u8 E4M3, sf [R, C/32] u8 E8M0)."""
    rows, cols = x_bf16.shape
    dev = x_bf16.device
    q = torch.empty((max(rows, 1), cols), dtype=torch.uint8, device=dev)
    sf = torch.empty((max(rows, 1), cols // 32), dtype=torch.uint8, device=dev)
    bfp4_quantize_mxfp8(x_bf16, rows, cols, x_bf16.stride(0), q, sf, stream)
    return q, sf


class MoeForwardMX:
    """One forward of the MX mode: routing plan, MXFP8 activation quantization, fused experts on
    MXFP4 weights (+ finalize); decode kernels for block_m <= 32, tiled kernels above."""

    def __init__(self, weights: PreparedWeights, M, top_k, num_experts, block_m,
                 local_expert_offset=0, do_finalize=True, device="cuda", act=None):
        if act is None:
            act = BFP4_ACT_SWIGLU if weights.gated else BFP4_ACT_RELU2
        if (act in GATED_ACTS) != bool(weights.gated):
            raise ValueError("activation %d does not match the weights' gating" % act)
        if weights.fmt != BFP4_FORMAT_MXFP4:
            raise ValueError("the MX mode needs MXFP4 weights")
        self.act = act
        self.w = weights
        self.M, self.top_k, self.E, self.block_m = M, top_k, num_experts, block_m
        self.offset = local_expert_offset
        self.do_finalize = do_finalize
        self.plan = MoePlanBuffers(M, top_k, weights.num_local_experts, block_m, device)
        H = weights.H
        self.a_q = torch.empty((max(M, 1), H), dtype=torch.uint8, device=device)
        self.a_sf = torch.empty((max(M, 1), H // 32), dtype=torch.uint8, device=device)
        self.ws_bytes = bfp4_workspace_size_mx(M, H, weights.I, top_k, weights.num_local_experts,
                                               block_m, int(do_finalize))
        self.ws = _bytes(self.ws_bytes + 256, device)
        self.gemm2_out = None
        if not do_finalize:
            self.gemm2_out = torch.empty((max(self.plan.capacity, 1), H), dtype=torch.bfloat16,
                                         device=device)

    def __call__(self, x_bf16, topk_ids, topk_weights, out=None, debug=None, weights=None,
                 stream=None, routed_scaling_factor=1.0):
        w = self.w if weights is None else weights
        M, H, I = self.M, w.H, w.I
        self.plan.build(topk_ids, self.E, self.offset, stream)
        if M:
            bfp4_quantize_mxfp8(x_bf16, M, H, x_bf16.stride(0), self.a_q, self.a_sf, stream)
        if out is None and self.do_finalize:
            out = torch.zeros((M, H), dtype=torch.bfloat16, device=x_bf16.device)
        pl = self.plan
        bfp4_fused_moe_mx(self.a_q, self.a_sf, w.panels, w.panels_bytes, pl.sorted_token_ids,
                          pl.expert_ids, pl.num_tokens_post_padded, pl.token_to_row, pl.capacity,
                          topk_weights, weights_dtype(topk_weights), M, H, I,
                          w.num_local_experts, self.top_k, self.block_m, self.act,
                          routed_scaling_factor, int(self.do_finalize), out, self.gemm2_out,
                          debug, self.ws, self.ws_bytes, stream)
        return out if self.do_finalize else (self.gemm2_out, topk_weights, pl.token_to_row)
