"""The layer as a sequence of separate C-ABI calls, with every intermediate
kept in its own buffer (for inspection, per-op timing and op-by-op checks).

With the defaults the ops are exactly the kernels moe_forward_chunked runs
on the M tokens as one chunk, in its order: the input quant fused into the
permute (moe_quant_permute), the gate/up GEMM writing h, a separate SiLU-mul
requant, the down GEMM and the unpermute (plus the standalone count, which
the forward does inside the permute).  Where the forward takes the
small-tile GEMMs (moe_forward_plan_info), so do the ops; a GEMM whose K the
plan cuts leaves its partial slabs in part13 / part2 (h or y unwritten),
and the requant or unpermute after it reads them.  reduce=True runs the down GEMM with the weight-and-reduce in its
epilogue (moe_grouped_gemm_fp8_weight_reduce) instead of the last two.  fused_input=False runs the input quant and the permute as two
calls instead, keeping a_q / a_s; fused=True uses the gate/up GEMM fused with
the SiLU-mul requant (moe_grouped_gemm_fp8_act_quant), so h never reaches
memory.  The forward call runs on one reused workspace; this form trades
memory for visibility.
"""
from __future__ import annotations

from collections import OrderedDict

import torch

from . import _lib


class StepBuffers:
    """Buffers of one pass over M tokens.  plan_problem: the forward problem
    whose chunk plan the ops follow (default: the M tokens as one chunk; a
    chunk of a chunked forward passes the whole problem)."""

    def __init__(self, layer, M: int, topk: int, device="cuda:0", plan_problem=None):
        K, N, El = layer.K, layer.N, layer.El
        self.M, self.topk = M, topk
        self.plan = _lib.moe_forward_plan_info(plan_problem if plan_problem is not None
                                               else layer.problem(M, topk, 0, 0))
        self.cap = _lib.moe_max_rows(M, topk, El, layer.align)
        cap = self.cap
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)
        u8, f32, i32, b16 = torch.uint8, torch.float32, torch.int32, torch.int16
        self.a_q, self.a_s = e((M, K), u8), e((M, K // 128), f32)
        self.a_perm, self.a_perm_s = e((cap, K), u8), e((cap, K // 128), f32)
        self.counts, self.offsets = e((El,), i32), e((El + 1,), i32)
        self.inv_perm, self.row_src = e((M, topk), i32), e((cap,), i32)
        self.permute_ws = e((_lib.moe_permute_workspace_size(M, topk, El),), u8)
        self.h = e((cap, 2 * N), b16)
        self.act_q, self.act_s = e((cap, N), u8), e((cap, N // 128), f32)
        self.y = e((cap, K), b16)
        self.out = e((M, K), b16)
        self.count_only = e((El,), i32)
        self.red_cnt = e((M, -(-K // 256)), i32)
        pr = max(self.plan["part_rows"], 1)
        self.part13 = e((self.plan["nsplit_w13"], pr, 2 * N), f32) if self.plan["nsplit_w13"] > 1 else None
        self.part2 = e((self.plan["nsplit_w2"], pr, K), f32) if self.plan["nsplit_w2"] > 1 else None
        self.info13, self.info2 = e((1,), i32), e((1,), i32)


def step_ops(layer, x, topk_ids, topk_weights, apply_on_input: int, b: StepBuffers, fused: bool = False,
             fused_input: bool = True, reduce: bool = False):
    """Ordered {name: thunk}; running them in order computes the layer into b.out."""
    Eg, El, K, N, A = layer.Eg, layer.El, layer.K, layer.N, layer.align
    emap = layer.expert_map
    ops = OrderedDict()
    ops["count"] = lambda: _lib.moe_count(topk_ids, emap, Eg, El, b.count_only)
    if fused_input:
        ops["quant_permute"] = lambda: _lib.moe_quant_permute(x, topk_ids, topk_weights, apply_on_input, emap, Eg,
                                                              El, A, b.cap, b.a_perm, b.a_perm_s, b.counts,
                                                              b.offsets, b.inv_perm, b.row_src, b.permute_ws)
    else:
        ops["input_quant"] = lambda: _lib.moe_act_quant(x, K, _lib.MOE_ACT_IDENTITY, b.a_q, b.a_s)
        ops["permute"] = lambda: _lib.moe_permute(b.a_q, b.a_s, topk_ids, topk_weights, apply_on_input, emap, Eg,
                                                  El, A, b.cap, b.a_perm, b.a_perm_s, b.counts, b.offsets,
                                                  b.inv_perm, b.row_src, b.permute_ws)
    if fused:
        ops["gemm_w13_act"] = lambda: _lib.moe_grouped_gemm_fp8_act_quant(b.a_perm, b.a_perm_s, layer.w13,
                                                                          layer.w13_s, b.offsets, b.counts,
                                                                          b.act_q, b.act_s)
    elif b.plan["small_tiles"]:
        ns13 = b.plan["nsplit_w13"]
        ops["gemm_w13"] = lambda: _lib.moe_grouped_gemm_fp8_small(b.a_perm, b.a_perm_s, layer.w13, layer.w13_s,
                                                                  b.offsets, b.counts, out=b.h, part=b.part13,
                                                                  nsplit=ns13, info=b.info13)
        if b.part13 is not None:
            ops["silu_mul_quant"] = lambda: _lib.moe_act_quant_partials(b.part13, b.info13, N, b.cap, b.offsets,
                                                                        b.counts, b.act_q, b.act_s)
        else:
            ops["silu_mul_quant"] = lambda: _lib.moe_act_quant(b.h, N, _lib.MOE_ACT_SILU_MUL, b.act_q, b.act_s,
                                                               b.offsets, b.counts, El)
    else:
        ops["gemm_w13"] = lambda: _lib.moe_grouped_gemm_fp8(b.a_perm, b.a_perm_s, layer.w13, layer.w13_s,
                                                            b.offsets, b.counts, b.h)
        ops["silu_mul_quant"] = lambda: _lib.moe_act_quant(b.h, N, _lib.MOE_ACT_SILU_MUL, b.act_q, b.act_s,
                                                           b.offsets, b.counts, El)
    if reduce:
        ops["gemm_w2_reduce"] = lambda: _lib.moe_grouped_gemm_fp8_weight_reduce(
            b.act_q, b.act_s, layer.w2, layer.w2_s, b.offsets, b.counts, b.row_src, b.inv_perm, topk_weights,
            apply_on_input, b.y, b.red_cnt, b.out)
        return ops
    if b.plan["small_tiles"]:
        ns2 = b.plan["nsplit_w2"]
        ops["gemm_w2"] = lambda: _lib.moe_grouped_gemm_fp8_small(b.act_q, b.act_s, layer.w2, layer.w2_s, b.offsets,
                                                                 b.counts, out=b.y, part=b.part2, nsplit=ns2,
                                                                 info=b.info2)
    else:
        ops["gemm_w2"] = lambda: _lib.moe_grouped_gemm_fp8(b.act_q, b.act_s, layer.w2, layer.w2_s, b.offsets,
                                                           b.counts, b.y)
    if b.part2 is not None:
        ops["unpermute"] = lambda: _lib.moe_unpermute_partials(b.part2, b.info2, b.offsets, b.counts, b.cap,
                                                               b.inv_perm, topk_weights, apply_on_input, b.out)
    else:
        ops["unpermute"] = lambda: _lib.moe_unpermute_weight_reduce(b.y, b.inv_perm, topk_weights,
                                                                    apply_on_input, b.out)
    return ops


def run_steps(layer, x, topk_ids, topk_weights, apply_on_input: int = 0, b: StepBuffers = None,
              fused: bool = False, fused_input: bool = True, reduce: bool = False):
    if b is None:
        b = StepBuffers(layer, x.shape[0], topk_ids.shape[1], x.device)
    for fn in step_ops(layer, x, topk_ids, topk_weights, apply_on_input, b, fused, fused_input, reduce).values():
        fn()
    return b
