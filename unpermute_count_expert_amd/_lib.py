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
MOE_STREAM_READ, MOE_STREAM_WRITE_NT, MOE_STREAM_COPY, MOE_STREAM_WRITE = 0, 1, 2, 3
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
           "moe_forward_workspace_size", "moe_forward_workspace_slices",
           "moe_permute_workspace_size", "moe_count", "moe_permute", "moe_grouped_gemm_fp8",
           "moe_grouped_gemm_fp8_act_quant", "moe_act_quant", "moe_quant_permute", "moe_unpermute_weight_reduce",
           "moe_forward_chunked", "moe_forward_chunked_noalloc", "moe_noalloc_scratch_bytes", "moe_hbm_stream",
           "moe_batched_workspace_size", "moe_experts_batched_masked", "moe_grouped_gemm_fp8_weight_reduce",
           "moe_grouped_gemm_fp8_small", "moe_act_quant_partials", "moe_unpermute_partials",
           "moe_forward_plan_info"]

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
        L.moe_forward_workspace_slices.argtypes = [C.POINTER(MoeProblem), C.POINTER(SZ), C.POINTER(SZ), I32,
                                                   C.POINTER(I32)]
        L.moe_count.argtypes = [P, I64, P, I32, I32, P, P, P]
        L.moe_permute.argtypes = [P, P, P, P, I32, I64, I32, I32, P, I32, I32, I32, I64,
                                  P, P, P, P, P, P, P, SZ, P]
        L.moe_quant_permute.argtypes = [P, P, P, I32, I64, I32, I32, P, I32, I32, I32, I64,
                                        P, P, P, P, P, P, P, SZ, P]
        L.moe_grouped_gemm_fp8.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, P, P]
        L.moe_grouped_gemm_fp8_act_quant.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, P, P, P]
        L.moe_act_quant.argtypes = [P, I64, I32, I32, P, P, I32, P, P, P]
        L.moe_unpermute_weight_reduce.argtypes = [P, I64, P, P, I64, I32, I32, I32, P, P]
        L.moe_grouped_gemm_fp8_small.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, P, P, I64, I32, P, P]
        L.moe_act_quant_partials.argtypes = [P, P, I64, I32, I64, I32, P, P, I32, P, P, P]
        L.moe_unpermute_partials.argtypes = [P, P, I64, I32, P, P, I32, I64, P, P, I64, I32, I32, I32, P, P]
        L.moe_forward_plan_info.argtypes = [C.POINTER(MoeProblem), C.POINTER(I32), C.POINTER(I32),
                                            C.POINTER(I32), C.POINTER(I64), C.POINTER(I32)]
        L.moe_forward_chunked.argtypes = [C.POINTER(MoeProblem), P, P, P, P, P, P, P, P, P, P, SZ,
                                          P, P]
        L.moe_forward_chunked_noalloc.argtypes = [C.POINTER(MoeProblem), P, P, P, P, P, P, P, P, P, P, P]
        L.moe_hbm_stream.argtypes = [I32, P, P, SZ, P]
        L.moe_grouped_gemm_fp8_weight_reduce.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, P, P, P, I32, I64, I32,
                                                         P, P, P, P]
        L.moe_batched_workspace_size.argtypes = [I32, I64, I32, C.POINTER(SZ)]
        L.moe_experts_batched_masked.argtypes = [P, P, P, I32, I64, I32, I32, P, P, P, P, P, P, SZ, P]
        L.moe_noalloc_scratch_bytes.argtypes = []; L.moe_noalloc_scratch_bytes.restype = SZ
        for name in EXPORTS:
            if name not in ("moe_status_string", "moe_last_error", "moe_max_rows", "moe_grouped_gemm_tile_rows",
                            "moe_noalloc_scratch_bytes"):
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


# ---- argument checks -----------------------------------------------------------
# The C ABI sees raw pointers only, so a tensor of the wrong dtype, shape or
# layout would be read with the wrong strides or past its end.  Every wrapper
# below checks dtype, contiguity and shape first, then that every tensor sits
# on the current CUDA device, and raises before anything reaches the library.
BF16 = (torch.int16, torch.bfloat16)          # bf16 values or their raw bits
E4M3 = (torch.uint8, torch.float8_e4m3fn)     # e4m3 codes
I32 = (torch.int32,)
F32 = (torch.float32,)


def check_arg(t, name: str, dtypes, shape=None, min_rows=None, optional=False):
    """dtype in dtypes, contiguous, and shape == `shape` (None entries match
    any size; with min_rows the first dimension may be larger than
    shape[0] if it is at least min_rows)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None:
        got = tuple(t.shape)
        ok = len(got) == len(shape)
        for i, (g_, w_) in enumerate(zip(got, shape)):
            if i == 0 and min_rows is not None:
                ok = ok and g_ >= min_rows
            elif w_ is not None:
                ok = ok and g_ == w_
        if not ok:
            want = tuple("*" if w_ is None else w_ for w_ in shape)
            extra = f" (first dimension >= {min_rows})" if min_rows is not None else ""
            raise ValueError(f"{name} has shape {got}; expected {want}{extra}")


def check_device(*tensors):
    """Every given tensor is on the current CUDA device (the library runs on
    the current device)."""
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"a tensor is on {t.device}; the library needs tensors on the current CUDA device")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"a tensor is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


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


def moe_forward_workspace_slices(p: MoeProblem):
    """[(offset, bytes)] of the slices moe_forward_chunked carves from its
    workspace; the bytes between a slice's end and the next offset are a
    guard band no kernel touches."""
    n = C.c_int32(0)
    _check(load().moe_forward_workspace_slices(C.byref(p), None, None, 0, C.byref(n)), "moe_forward_workspace_slices")
    offs = (C.c_size_t * max(n.value, 1))()
    lens = (C.c_size_t * max(n.value, 1))()
    _check(load().moe_forward_workspace_slices(C.byref(p), offs, lens, n.value, C.byref(n)),
           "moe_forward_workspace_slices")
    return [(int(offs[i]), int(lens[i])) for i in range(n.value)]


def moe_permute_workspace_size(Mc: int, topk: int, El: int) -> int:
    n = C.c_size_t(0)
    _check(load().moe_permute_workspace_size(Mc, topk, El, C.byref(n)), "moe_permute_workspace_size")
    return int(n.value)


def moe_count(topk_ids, expert_map, Eg, El, counts, invalid_ids=None, stream=None):
    check_arg(topk_ids, "topk_ids", I32)
    check_arg(expert_map, "expert_map", I32, (Eg,), optional=True)
    check_arg(counts, "counts", I32, (El,))
    check_arg(invalid_ids, "invalid_ids", I32, (1,), optional=True)
    check_device(topk_ids, expert_map, counts, invalid_ids)
    _check(load().moe_count(_ptr(topk_ids), topk_ids.numel(), _ptr(expert_map), Eg, El, _ptr(counts),
                            _ptr(invalid_ids), _stream(stream)), "moe_count")


def _check_permute_outputs(Mc, K, topk, El, cap_rows, a_perm, a_perm_s, counts, expert_offsets, inv_perm,
                           row_src, workspace):
    check_arg(a_perm, "a_perm", E4M3, (None, K), min_rows=cap_rows)
    check_arg(a_perm_s, "a_perm_s", F32, (None, K // 128), min_rows=cap_rows)
    check_arg(counts, "counts", I32, (El,))
    check_arg(expert_offsets, "expert_offsets", I32, (El + 1,))
    check_arg(inv_perm, "inv_perm", I32, (Mc, topk))
    check_arg(row_src, "row_src", I32, (None,), min_rows=cap_rows)
    check_arg(workspace, "workspace", (torch.uint8, torch.int32))


def moe_permute(a_q, a_s, topk_ids, topk_weights, apply_on_input, expert_map, Eg, El, align, cap_rows,
                a_perm, a_perm_s, counts, expert_offsets, inv_perm, row_src, workspace, stream=None):
    check_arg(a_q, "a_q", E4M3, (None, None))
    Mc, K = a_q.shape
    check_arg(a_s, "a_s", F32, (Mc, K // 128))
    check_arg(topk_ids, "topk_ids", I32, (Mc, None))
    topk = topk_ids.shape[1]
    check_arg(topk_weights, "topk_weights", F32, (Mc, topk), optional=not apply_on_input)
    check_arg(expert_map, "expert_map", I32, (Eg,), optional=True)
    _check_permute_outputs(Mc, K, topk, El, cap_rows, a_perm, a_perm_s, counts, expert_offsets, inv_perm,
                           row_src, workspace)
    check_device(a_q, a_s, topk_ids, topk_weights, expert_map, a_perm, a_perm_s, counts, expert_offsets,
                 inv_perm, row_src, workspace)
    _check(load().moe_permute(_ptr(a_q), _ptr(a_s), _ptr(topk_ids), _ptr(topk_weights), apply_on_input,
                              Mc, K, topk, _ptr(expert_map), Eg, El, align, cap_rows, _ptr(a_perm),
                              _ptr(a_perm_s), _ptr(counts), _ptr(expert_offsets), _ptr(inv_perm),
                              _ptr(row_src), _ptr(workspace), _nbytes(workspace), _stream(stream)), "moe_permute")


def moe_quant_permute(x, topk_ids, topk_weights, apply_on_input, expert_map, Eg, El, align, cap_rows,
                      a_perm, a_perm_s, counts, expert_offsets, inv_perm, row_src, workspace, stream=None):
    check_arg(x, "x", BF16, (None, None))
    Mc, K = x.shape
    check_arg(topk_ids, "topk_ids", I32, (Mc, None))
    topk = topk_ids.shape[1]
    check_arg(topk_weights, "topk_weights", F32, (Mc, topk), optional=not apply_on_input)
    check_arg(expert_map, "expert_map", I32, (Eg,), optional=True)
    _check_permute_outputs(Mc, K, topk, El, cap_rows, a_perm, a_perm_s, counts, expert_offsets, inv_perm,
                           row_src, workspace)
    check_device(x, topk_ids, topk_weights, expert_map, a_perm, a_perm_s, counts, expert_offsets, inv_perm,
                 row_src, workspace)
    _check(load().moe_quant_permute(_ptr(x), _ptr(topk_ids), _ptr(topk_weights), apply_on_input,
                                    Mc, K, topk, _ptr(expert_map), Eg, El, align, cap_rows, _ptr(a_perm),
                                    _ptr(a_perm_s), _ptr(counts), _ptr(expert_offsets), _ptr(inv_perm),
                                    _ptr(row_src), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "moe_quant_permute")


def _check_gemm_operands(a, a_s, w, w_s, expert_offsets, counts):
    check_arg(a, "a", E4M3, (None, None))
    cap_rows, k_in = a.shape
    check_arg(a_s, "a_s", F32, (cap_rows, k_in // 128))
    check_arg(w, "w", E4M3, (None, None, k_in))
    El, n_out, _ = w.shape
    check_arg(w_s, "w_s", F32, (El, n_out // 128, k_in // 128))
    check_arg(expert_offsets, "expert_offsets", I32, (El + 1,))
    check_arg(counts, "counts", I32, (El,))
    return cap_rows, k_in, El, n_out


def moe_grouped_gemm_fp8(a, a_s, w, w_s, expert_offsets, counts, out, stream=None):
    cap_rows, k_in, El, n_out = _check_gemm_operands(a, a_s, w, w_s, expert_offsets, counts)
    check_arg(out, "out", BF16, (cap_rows, n_out))
    check_device(a, a_s, w, w_s, expert_offsets, counts, out)
    _check(load().moe_grouped_gemm_fp8(_ptr(a), _ptr(a_s), _ptr(w), _ptr(w_s), _ptr(expert_offsets),
                                       _ptr(counts), El, cap_rows, n_out, k_in, _ptr(out),
                                       _stream(stream)), "moe_grouped_gemm_fp8")


def moe_grouped_gemm_fp8_act_quant(a, a_s, w13, w13_s, expert_offsets, counts, q, q_s, stream=None):
    cap_rows, k_in, El, two_n = _check_gemm_operands(a, a_s, w13, w13_s, expert_offsets, counts)
    check_arg(q, "q", E4M3, (cap_rows, two_n // 2))
    check_arg(q_s, "q_s", F32, (cap_rows, two_n // 256))
    check_device(a, a_s, w13, w13_s, expert_offsets, counts, q, q_s)
    _check(load().moe_grouped_gemm_fp8_act_quant(_ptr(a), _ptr(a_s), _ptr(w13), _ptr(w13_s),
                                                 _ptr(expert_offsets), _ptr(counts), El, cap_rows, two_n // 2,
                                                 k_in, _ptr(q), _ptr(q_s), _stream(stream)),
           "moe_grouped_gemm_fp8_act_quant")


def moe_act_quant(inp, n, mode, q, q_s, expert_offsets=None, counts=None, El=0, stream=None):
    width = n if mode == MOE_ACT_IDENTITY else 2 * n
    check_arg(inp, "in", BF16, (None, width))
    rows = inp.shape[0]
    check_arg(q, "q", E4M3, (rows, n))
    check_arg(q_s, "q_s", F32, (rows, n // 128))
    check_arg(expert_offsets, "expert_offsets", I32, (El + 1,), optional=True)
    check_arg(counts, "counts", I32, (El,), optional=True)
    check_device(inp, q, q_s, expert_offsets, counts)
    _check(load().moe_act_quant(_ptr(inp), rows, n, mode, _ptr(expert_offsets), _ptr(counts), El,
                                _ptr(q), _ptr(q_s), _stream(stream)), "moe_act_quant")


def moe_unpermute_weight_reduce(y, inv_perm, topk_weights, apply_on_input, out, stream=None):
    check_arg(y, "y", BF16, (None, None))
    y_rows, K = y.shape
    check_arg(inv_perm, "inv_perm", I32, (None, None))
    Mc, topk = inv_perm.shape
    check_arg(topk_weights, "topk_weights", F32, (Mc, topk), optional=bool(apply_on_input))
    check_arg(out, "out", BF16, (Mc, K))
    check_device(y, inv_perm, topk_weights, out)
    _check(load().moe_unpermute_weight_reduce(_ptr(y), y_rows, _ptr(inv_perm), _ptr(topk_weights), Mc, K,
                                              topk, apply_on_input, _ptr(out), _stream(stream)),
           "moe_unpermute_weight_reduce")


def moe_grouped_gemm_fp8_small(a, a_s, w, w_s, expert_offsets, counts, out=None, part=None, nsplit=1, info=None,
                               stream=None):
    """The small-chunk GEMM: bf16 out (part None), or fp32 partial slabs
    part [nsplit, part_rows, n_out] and the segment count used in info [1]."""
    cap_rows, k_in, El, n_out = _check_gemm_operands(a, a_s, w, w_s, expert_offsets, counts)
    if part is None:
        check_arg(out, "out", BF16, (cap_rows, n_out))
        part_rows = 0
    else:
        check_arg(part, "part", F32, (nsplit, None, n_out))
        check_arg(info, "info", I32, (1,), min_rows=1)
        part_rows = part.shape[1]
    check_device(a, a_s, w, w_s, expert_offsets, counts, out, part, info)
    _check(load().moe_grouped_gemm_fp8_small(_ptr(a), _ptr(a_s), _ptr(w), _ptr(w_s), _ptr(expert_offsets),
                                             _ptr(counts), El, cap_rows, n_out, k_in, _ptr(out), _ptr(part),
                                             part_rows, nsplit, _ptr(info), _stream(stream)),
           "moe_grouped_gemm_fp8_small")


def moe_act_quant_partials(part, info, n, rows, expert_offsets, counts, q, q_s, stream=None):
    """SiLU-mul requant of h given as the small GEMM's partial slabs
    part [nsplit, part_rows, 2n]; q [rows, n], q_s [rows, n/128]."""
    check_arg(part, "part", F32, (None, None, 2 * n))
    nsplit, part_rows, _ = part.shape
    check_arg(info, "info", I32, (1,))
    check_arg(expert_offsets, "expert_offsets", I32, (None,))
    El = expert_offsets.shape[0] - 1
    check_arg(counts, "counts", I32, (El,))
    check_arg(q, "q", E4M3, (rows, n))
    check_arg(q_s, "q_s", F32, (rows, n // 128))
    check_device(part, info, expert_offsets, counts, q, q_s)
    _check(load().moe_act_quant_partials(_ptr(part), _ptr(info), part_rows, nsplit, rows, n, _ptr(expert_offsets),
                                         _ptr(counts), El, _ptr(q), _ptr(q_s), _stream(stream)),
           "moe_act_quant_partials")


def moe_unpermute_partials(part, info, expert_offsets, counts, y_rows, inv_perm, topk_weights, apply_on_input, out,
                           stream=None):
    """Unpermute with weight-and-reduce of y given as the small GEMM's partial
    slabs part [nsplit, part_rows, K]; out [Mc, K]."""
    check_arg(part, "part", F32, (None, None, None))
    nsplit, part_rows, K = part.shape
    check_arg(info, "info", I32, (1,))
    check_arg(expert_offsets, "expert_offsets", I32, (None,))
    El = expert_offsets.shape[0] - 1
    check_arg(counts, "counts", I32, (El,))
    check_arg(inv_perm, "inv_perm", I32, (None, None))
    Mc, topk = inv_perm.shape
    check_arg(topk_weights, "topk_weights", F32, (Mc, topk), optional=bool(apply_on_input))
    check_arg(out, "out", BF16, (Mc, K))
    check_device(part, info, expert_offsets, counts, inv_perm, topk_weights, out)
    _check(load().moe_unpermute_partials(_ptr(part), _ptr(info), part_rows, nsplit, _ptr(expert_offsets),
                                         _ptr(counts), El, y_rows, _ptr(inv_perm), _ptr(topk_weights), Mc, K, topk,
                                         apply_on_input, _ptr(out), _stream(stream)),
           "moe_unpermute_partials")


def moe_forward_plan_info(p: MoeProblem) -> dict:
    """How moe_forward_chunked runs p: small_tiles, nsplit_w13, nsplit_w2,
    part_rows, lanes."""
    v = [C.c_int32(), C.c_int32(), C.c_int32(), C.c_int64(), C.c_int32()]
    _check(load().moe_forward_plan_info(C.byref(p), *[C.byref(x) for x in v]), "moe_forward_plan_info")
    return dict(small_tiles=bool(v[0].value), nsplit_w13=v[1].value, nsplit_w2=v[2].value, part_rows=v[3].value,
                lanes=v[4].value)


def check_forward_args(p: MoeProblem, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out,
                       per_chunk_counts=None):
    """dtype, layout and shape checks of moe_forward_chunked's tensors
    against the problem p (no device check)."""
    M, K, N, T, El, Eg = p.M, p.K, p.N, p.topk, p.num_local_experts, p.num_global_experts
    check_arg(x, "x", BF16, (M, K))
    check_arg(topk_ids, "topk_ids", I32, (M, T))
    check_arg(topk_weights, "topk_weights", F32, (M, T))
    check_arg(expert_map, "expert_map", I32, (Eg,), optional=True)
    check_arg(w13, "w13", E4M3, (El, 2 * N, K))
    check_arg(w13_s, "w13_s", F32, (El, 2 * N // 128, K // 128))
    check_arg(w2, "w2", E4M3, (El, K, N))
    check_arg(w2_s, "w2_s", F32, (El, K // 128, N // 128))
    check_arg(out, "out", BF16, (M, K))
    cs = M if (p.chunk_size <= 0 or p.chunk_size >= M) else p.chunk_size
    nch = -(-M // cs) if M > 0 else 0
    check_arg(per_chunk_counts, "per_chunk_counts", I32, (nch, El), optional=True)


def moe_forward_chunked(p: MoeProblem, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out,
                        workspace, per_chunk_counts=None, stream=None):
    check_forward_args(p, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out, per_chunk_counts)
    check_arg(workspace, "workspace", (torch.uint8,))
    check_device(x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out, workspace, per_chunk_counts)
    _check(load().moe_forward_chunked(C.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                      _ptr(expert_map), _ptr(w13), _ptr(w13_s), _ptr(w2), _ptr(w2_s),
                                      _ptr(out), _ptr(workspace), _nbytes(workspace),
                                      _ptr(per_chunk_counts), _stream(stream)), "moe_forward_chunked")


def moe_noalloc_scratch_bytes() -> int:
    return int(load().moe_noalloc_scratch_bytes())


def moe_forward_chunked_noalloc(p: MoeProblem, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out,
                                per_chunk_counts=None, stream=None):
    """moe_forward_chunked with the workspace taken from the library's fixed
    per-GPU scratch array: nothing is allocated (see include/moe.h)."""
    check_forward_args(p, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out, per_chunk_counts)
    check_device(x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out, per_chunk_counts)
    _check(load().moe_forward_chunked_noalloc(C.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                              _ptr(expert_map), _ptr(w13), _ptr(w13_s), _ptr(w2), _ptr(w2_s),
                                              _ptr(out), _ptr(per_chunk_counts), _stream(stream)),
           "moe_forward_chunked_noalloc")


def moe_hbm_stream(mode: int, src, dst, nbytes: int, stream=None):
    """A plain HBM read / write / copy stream of nbytes (a measured ceiling)."""
    check_arg(dst, "dst", (torch.uint8,))
    check_arg(src, "src", (torch.uint8,), optional=True)
    if dst.numel() < (16 if mode == MOE_STREAM_READ else nbytes) or (src is not None and src.numel() < nbytes):
        raise ValueError("buffers smaller than the stream")
    check_device(src, dst)
    _check(load().moe_hbm_stream(mode, _ptr(src), _ptr(dst), nbytes, _stream(stream)), "moe_hbm_stream")


def moe_batched_workspace_size(El: int, max_tokens: int, N: int) -> int:
    n = C.c_size_t(0)
    _check(load().moe_batched_workspace_size(El, max_tokens, N, C.byref(n)), "moe_batched_workspace_size")
    return int(n.value)


def moe_experts_batched_masked(a_q, a_s, counts, w13, w13_s, w2, w2_s, out, workspace, stream=None):
    """The experts on the batched, masked layout: a_q [El, max_tokens, K],
    counts [El] valid rows per slot -> out [El, max_tokens, K] bf16."""
    check_arg(a_q, "a_q", E4M3, (None, None, None))
    El, max_tokens, K = a_q.shape
    check_arg(a_s, "a_s", F32, (El, max_tokens, K // 128))
    check_arg(counts, "counts", I32, (El,))
    check_arg(w13, "w13", E4M3, (El, None, K))
    N = w13.shape[1] // 2
    check_arg(w13_s, "w13_s", F32, (El, 2 * N // 128, K // 128))
    check_arg(w2, "w2", E4M3, (El, K, N))
    check_arg(w2_s, "w2_s", F32, (El, K // 128, N // 128))
    check_arg(out, "out", BF16, (El, max_tokens, K))
    check_arg(workspace, "workspace", (torch.uint8,))
    check_device(a_q, a_s, counts, w13, w13_s, w2, w2_s, out, workspace)
    _check(load().moe_experts_batched_masked(_ptr(a_q), _ptr(a_s), _ptr(counts), El, max_tokens, K, N, _ptr(w13),
                                             _ptr(w13_s), _ptr(w2), _ptr(w2_s), _ptr(out), _ptr(workspace),
                                             _nbytes(workspace), _stream(stream)), "moe_experts_batched_masked")


def moe_grouped_gemm_fp8_weight_reduce(a, a_s, w, w_s, expert_offsets, counts, row_src, inv_perm, topk_weights,
                                       apply_on_input, y, counters, out, stream=None):
    """The down GEMM with the unpermute's weight-and-reduce in its epilogue:
    y = GEMM(a, w) on the valid rows and out [Mc, n_out] = the weighted sum of
    each token's rows of y (the same bits as the two separate calls)."""
    cap_rows, k_in, El, n_out = _check_gemm_operands(a, a_s, w, w_s, expert_offsets, counts)
    check_arg(row_src, "row_src", I32, (None,), min_rows=cap_rows)
    check_arg(inv_perm, "inv_perm", I32, (None, None))
    Mc, topk = inv_perm.shape
    check_arg(topk_weights, "topk_weights", F32, (Mc, topk), optional=bool(apply_on_input))
    check_arg(y, "y", BF16, (cap_rows, n_out))
    check_arg(counters, "counters", I32, (Mc, (n_out + 255) // 256))
    check_arg(out, "out", BF16, (Mc, n_out))
    check_device(a, a_s, w, w_s, expert_offsets, counts, row_src, inv_perm, topk_weights, y, counters, out)
    _check(load().moe_grouped_gemm_fp8_weight_reduce(_ptr(a), _ptr(a_s), _ptr(w), _ptr(w_s), _ptr(expert_offsets),
                                                     _ptr(counts), El, cap_rows, n_out, k_in, _ptr(row_src),
                                                     _ptr(inv_perm), _ptr(topk_weights), apply_on_input, Mc, topk,
                                                     _ptr(y), _ptr(counters), _ptr(out), _stream(stream)),
           "moe_grouped_gemm_fp8_weight_reduce")
