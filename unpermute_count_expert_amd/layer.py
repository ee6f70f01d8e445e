"""Device-resident MoE expert layer over the C ABI.

Holds one GPU's local expert weights (fp8 e4m3 codes + 128x128 fp32 block
scales) and a workspace sized once for the largest chunk; forward() is one
moe_forward_chunked call on the current stream.

Every tensor is checked (dtype, contiguity, shape against the weights, one
device) before its pointer reaches the library: ids must be int32 (torch.topk
returns int64, which the kernels would read as pairs of int32), router
weights float32, tokens bf16 (or their int16 bits) of width K.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


class MoeLayer:
    def __init__(self, w13: torch.Tensor, w13_s: torch.Tensor, w2: torch.Tensor, w2_s: torch.Tensor,
                 num_global_experts: int, expert_map: Optional[torch.Tensor] = None, align: int = 128):
        _lib.check_arg(w13, "w13", _lib.E4M3, (None, None, None))
        self.El, twoN, self.K = w13.shape
        if twoN % 256 or self.K % 128:
            raise ValueError(f"w13 has shape {tuple(w13.shape)}; expected (El, 2N, K) with N and K "
                             "multiples of 128")
        self.N = twoN // 2
        _lib.check_arg(w13_s, "w13_s", _lib.F32, (self.El, twoN // 128, self.K // 128))
        _lib.check_arg(w2, "w2", _lib.E4M3, (self.El, self.K, self.N))
        _lib.check_arg(w2_s, "w2_s", _lib.F32, (self.El, self.K // 128, self.N // 128))
        _lib.check_arg(expert_map, "expert_map", _lib.I32, (num_global_experts,), optional=True)
        devs = {t.device for t in (w13, w13_s, w2, w2_s, expert_map) if t is not None}
        if len(devs) != 1:
            raise ValueError(f"the weights are on several devices: {sorted(map(str, devs))}")
        self.device = devs.pop()
        self.w13, self.w13_s, self.w2, self.w2_s = w13, w13_s, w2, w2_s
        self.Eg = num_global_experts
        self.expert_map = expert_map
        self.align = align
        self._ws = None

    def problem(self, M: int, topk: int, chunk_size: int = 0, apply_on_input: int = 0):
        return _lib.problem(M, self.K, self.N, topk, self.Eg, self.El, self.align, apply_on_input,
                            chunk_size)

    def workspace(self, p) -> torch.Tensor:
        n = _lib.moe_forward_workspace_size(p)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws

    def forward(self, x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                chunk_size: int = 0, apply_on_input: int = 0, out: Optional[torch.Tensor] = None,
                per_chunk_counts: Optional[torch.Tensor] = None) -> torch.Tensor:
        _lib.check_arg(x, "x", _lib.BF16, (None, self.K))
        _lib.check_arg(topk_ids, "topk_ids", _lib.I32, (x.shape[0], None))
        M, topk = topk_ids.shape
        p = self.problem(M, topk, chunk_size, apply_on_input)
        if out is None:
            out = torch.empty((M, self.K), dtype=torch.int16, device=x.device)  # bf16 bits
        _lib.check_forward_args(p, x, topk_ids, topk_weights, self.expert_map, self.w13, self.w13_s, self.w2,
                                self.w2_s, out, per_chunk_counts)
        _lib.check_device(x, topk_ids, topk_weights, out, per_chunk_counts, self.w13)
        ws = self.workspace(p)
        _lib.moe_forward_chunked(p, x, topk_ids, topk_weights, self.expert_map, self.w13, self.w13_s,
                                 self.w2, self.w2_s, out, ws, per_chunk_counts)
        return out
