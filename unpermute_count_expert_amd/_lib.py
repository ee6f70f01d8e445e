"""Thin ctypes binding over libmoe_hip.so (include/moe.h).

Argument marshalling only: each function passes device pointers, sizes and
the current HIP stream to the C ABI and raises MoeError on a non-OK status.
All arithmetic runs in the library's gfx950 kernels.  There is no fallback:
if the library is missing the import of this module fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_hip.so")

MOE_ACT_IDENTITY = 0
MOE_ACT_SILU_MUL = 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_WORKSPACE_TOO_SMALL",
          4: "MOE_ERR_UNSUPPORTED_DEVICE", 5: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


class MoeProblem(C.Structure):
    _fields_ = [("M", C.c_int64), ("K", C.c_int32), ("N", C.c_int32), ("topk", C.c_int32),
                ("num_global_experts", C.c_int32), ("num_local_experts", C.c_int32),
                ("align", C.c_int32), ("apply_router_weight_on_input", C.c_int32),
                ("chunk_size", C.c_int64)]


EXPORTS = ["moe_status_string", "moe_last_error", "moe_max_rows", "moe_grouped_gemm_tile_rows",
           "moe_forward_workspace_size",
           "moe_permute_workspace_size", "moe_count", "moe_permute", "moe_grouped_gemm_fp8",
           "moe_grouped_gemm_fp8_act_quant", "moe_act_quant", "moe_quant_permute", "moe_unpermute_weight_reduce",
           "moe_forward_chunked"]

_lib = None


def load() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950)")
        L = C.CDLL(LIB_PATH)
        P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.moe_status_string.argtypes = [C.c_int]; L.moe_status_string.restype = C.c_char_p
        L.moe_last_error.argtypes = []; L.moe_last_error.restype = C.c_char_p
        L.moe_max_rows.argtypes = [I64, I32, I32, I32]; L.moe_max_rows.restype = I64
        L.moe_grouped_gemm_tile_rows.argtypes = [I64, I32]; L.moe_grouped_gemm_tile_rows.restype = I32
        L.moe_forward_workspace_size.argtypes = [C.POINTER(MoeProblem), C.POINTER(SZ)]
        L.moe_permute_workspace_size.argtypes = [I64, I32, I32, C.POINTER(SZ)]
        L.moe_count.argtypes = [P, I64, P, I32, I32, P, P, P]
        L.moe_permute.argtypes = [P, P, P, P, I32, I64, I32, I32, P, I32, I32, I32, I64,
                                  P, P, P, P, P, P, P, SZ, P]
        L.moe_quant_permute.argtypes = [P, P, P, I32, I64, I32, I32, P, I32, I32, I32, I64,
                                        P, P, P, P, P, P, P, SZ, P]
        L.moe_grouped_gemm_fp8.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, P, P]
        L.moe_grouped_gemm_fp8_act_quant.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, P, P, P]
        L.moe_act_quant.argtypes = [P, I64, I32, I32, P, P, I32, P, P, P]
        L.moe_unpermute_weight_reduce.argtypes = [P, I64, P, P, I64, I32, I32, I32, P, P]
        L.moe_forward_chunked.argtypes = [C.POINTER(MoeProblem), P, P, P, P, P, P, P, P, P, P, SZ,
                                          P, P]
        for name in EXPORTS:
            if name not in ("moe_status_string", "moe_last_error", "moe_max_rows", "moe_grouped_gemm_tile_rows"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int, where: str):
    if rc != 0:
        detail = load().moe_last_error().decode(errors="replace")
        raise MoeError(rc, where, detail)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def moe_max_rows(Mc: int, topk: int, El: int, align: int = 128) -> int:
    return int(load().moe_max_rows(Mc, topk, El, align))


def moe_grouped_gemm_tile_rows(rows_hint: int, El: int) -> int:
    return int(load().moe_grouped_gemm_tile_rows(rows_hint, El))


def problem(M, K, N, topk, Eg, El, align=128, apply_on_input=0, chunk_size=0) -> MoeProblem:
    return MoeProblem(M, K, N, topk, Eg, El, align, apply_on_input, chunk_size)


def moe_forward_workspace_size(p: MoeProblem) -> int:
    n = C.c_size_t(0)
    _check(load().moe_forward_workspace_size(C.byref(p), C.byref(n)), "moe_forward_workspace_size")
    return int(n.value)


def moe_permute_workspace_size(Mc: int, topk: int, El: int) -> int:
    n = C.c_size_t(0)
    _check(load().moe_permute_workspace_size(Mc, topk, El, C.byref(n)), "moe_permute_workspace_size")
    return int(n.value)


def moe_count(topk_ids, expert_map, Eg, El, counts, invalid_ids=None, stream=None):
    _check(load().moe_count(_ptr(topk_ids), topk_ids.numel(), _ptr(expert_map), Eg, El, _ptr(counts),
                            _ptr(invalid_ids), _stream(stream)), "moe_count")


def moe_permute(a_q, a_s, topk_ids, topk_weights, apply_on_input, expert_map, Eg, El, align, cap_rows,
                a_perm, a_perm_s, counts, expert_offsets, inv_perm, row_src, workspace, stream=None):
    Mc, K = a_q.shape
    topk = topk_ids.shape[1]
    _check(load().moe_permute(_ptr(a_q), _ptr(a_s), _ptr(topk_ids), _ptr(topk_weights), apply_on_input,
                              Mc, K, topk, _ptr(expert_map), Eg, El, align, cap_rows, _ptr(a_perm),
                              _ptr(a_perm_s), _ptr(counts), _ptr(expert_offsets), _ptr(inv_perm),
                              _ptr(row_src), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)), "moe_permute")


def moe_quant_permute(x, topk_ids, topk_weights, apply_on_input, expert_map, Eg, El, align, cap_rows,
                      a_perm, a_perm_s, counts, expert_offsets, inv_perm, row_src, workspace, stream=None):
    Mc, K = x.shape
    topk = topk_ids.shape[1]
    _check(load().moe_quant_permute(_ptr(x), _ptr(topk_ids), _ptr(topk_weights), apply_on_input,
                                    Mc, K, topk, _ptr(expert_map), Eg, El, align, cap_rows, _ptr(a_perm),
                                    _ptr(a_perm_s), _ptr(counts), _ptr(expert_offsets), _ptr(inv_perm),
                                    _ptr(row_src), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "moe_quant_permute")


def moe_grouped_gemm_fp8(a, a_s, w, w_s, expert_offsets, counts, out, stream=None):
    cap_rows, k_in = a.shape
    El, n_out, _ = w.shape
    _check(load().moe_grouped_gemm_fp8(_ptr(a), _ptr(a_s), _ptr(w), _ptr(w_s), _ptr(expert_offsets),
                                       _ptr(counts), El, cap_rows, n_out, k_in, _ptr(out),
                                       _stream(stream)), "moe_grouped_gemm_fp8")


def moe_grouped_gemm_fp8_act_quant(a, a_s, w13, w13_s, expert_offsets, counts, q, q_s, stream=None):
    cap_rows, k_in = a.shape
    El, two_n, _ = w13.shape
    _check(load().moe_grouped_gemm_fp8_act_quant(_ptr(a), _ptr(a_s), _ptr(w13), _ptr(w13_s),
                                                 _ptr(expert_offsets), _ptr(counts), El, cap_rows, two_n // 2,
                                                 k_in, _ptr(q), _ptr(q_s), _stream(stream)),
           "moe_grouped_gemm_fp8_act_quant")


def moe_act_quant(inp, n, mode, q, q_s, expert_offsets=None, counts=None, El=0, stream=None):
    rows = inp.shape[0]
    _check(load().moe_act_quant(_ptr(inp), rows, n, mode, _ptr(expert_offsets), _ptr(counts), El,
                                _ptr(q), _ptr(q_s), _stream(stream)), "moe_act_quant")


def moe_unpermute_weight_reduce(y, inv_perm, topk_weights, apply_on_input, out, stream=None):
    y_rows, K = y.shape
    Mc, topk = inv_perm.shape
    _check(load().moe_unpermute_weight_reduce(_ptr(y), y_rows, _ptr(inv_perm), _ptr(topk_weights), Mc, K,
                                              topk, apply_on_input, _ptr(out), _stream(stream)),
           "moe_unpermute_weight_reduce")


def moe_forward_chunked(p: MoeProblem, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out,
                        workspace, per_chunk_counts=None, stream=None):
    _check(load().moe_forward_chunked(C.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                      _ptr(expert_map), _ptr(w13), _ptr(w13_s), _ptr(w2), _ptr(w2_s),
                                      _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _ptr(per_chunk_counts), _stream(stream)), "moe_forward_chunked")
