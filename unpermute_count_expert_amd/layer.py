"""Device-resident MoE expert layer over the C ABI.

Holds one GPU's local expert weights (fp8 e4m3 codes + 128x128 fp32 block
scales) and a workspace sized once for the largest chunk; forward() is one
moe_forward_chunked call on the current stream.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


class MoeLayer:
    def __init__(self, w13: torch.Tensor, w13_s: torch.Tensor, w2: torch.Tensor, w2_s: torch.Tensor,
                 num_global_experts: int, expert_map: Optional[torch.Tensor] = None, align: int = 128):
        assert w13.is_cuda and w13.dtype == torch.uint8 and w13.dim() == 3
        self.El, twoN, self.K = w13.shape
        self.N = twoN // 2
        assert w2.shape == (self.El, self.K, self.N)
        self.w13, self.w13_s, self.w2, self.w2_s = w13, w13_s, w2, w2_s
        self.Eg = num_global_experts
        self.expert_map = expert_map
        self.align = align
        self._ws = None
        self._ws_key = None

    def problem(self, M: int, topk: int, chunk_size: int = 0, apply_on_input: int = 0):
        return _lib.problem(M, self.K, self.N, topk, self.Eg, self.El, self.align, apply_on_input,
                            chunk_size)

    def workspace(self, p) -> torch.Tensor:
        n = _lib.moe_forward_workspace_size(p)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.w13.device)
        return self._ws

    def forward(self, x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                chunk_size: int = 0, apply_on_input: int = 0, out: Optional[torch.Tensor] = None,
                per_chunk_counts: Optional[torch.Tensor] = None) -> torch.Tensor:
        M = x.shape[0]
        p = self.problem(M, topk_ids.shape[1], chunk_size, apply_on_input)
        ws = self.workspace(p)
        if out is None:
            out = torch.empty((M, self.K), dtype=torch.int16, device=x.device)  # bf16 bits
        _lib.moe_forward_chunked(p, x, topk_ids, topk_weights, self.expert_map, self.w13, self.w13_s,
                                 self.w2, self.w2_s, out, ws, per_chunk_counts)
        return out
