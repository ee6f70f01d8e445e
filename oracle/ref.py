"""ctypes wrapper over oracle/libmoe_ref.so (test infrastructure).

Every function takes and returns numpy arrays; the arithmetic all lives in
moe_ref.c.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_REF_LIB: another build of the same source (the sanitizer test loads one
# built with AddressSanitizer and UndefinedBehaviorSanitizer)
_LIB_PATH = os.environ.get("MOE_REF_LIB") or os.path.join(_HERE, "libmoe_ref.so")
_lib = None

GROUP = 128


class OracleError(RuntimeError):
    pass


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        _lib = C.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


P = C.c_void_p
I32, I64, F32 = C.c_int32, C.c_int64, C.c_float


def _declare(L):
    L.moe_ref_bf16_from_f32.argtypes = [F32]; L.moe_ref_bf16_from_f32.restype = C.c_uint16
    L.moe_ref_bf16_from_f64.argtypes = [C.c_double]; L.moe_ref_bf16_from_f64.restype = C.c_uint16
    L.moe_ref_e4m3_from_f32.argtypes = [F32]; L.moe_ref_e4m3_from_f32.restype = C.c_uint8
    L.moe_ref_e4m3_value.argtypes = [C.c_uint8]; L.moe_ref_e4m3_value.restype = C.c_double
    L.moe_ref_exp_spec.argtypes = [F32]; L.moe_ref_exp_spec.restype = F32
    L.moe_ref_quant_group.argtypes = [P, P, P]; L.moe_ref_quant_group.restype = None
    L.moe_ref_loc.argtypes = [I32, P, I32, I32]; L.moe_ref_loc.restype = C.c_int
    L.moe_ref_count.argtypes = [P, I64, P, I32, I32, P, P]; L.moe_ref_count.restype = C.c_int
    L.moe_ref_max_rows.argtypes = [I64, I32, I32, I32]; L.moe_ref_max_rows.restype = I64
    L.moe_ref_act_quant_identity.argtypes = [P, I64, I32, P, P]
    L.moe_ref_act_quant_identity.restype = C.c_int
    L.moe_ref_permute.argtypes = [P, P, P, P, I32, I64, I32, I32, P, I32, I32, I32, I64,
                                  P, P, P, P, P, P]
    L.moe_ref_permute.restype = C.c_int
    L.moe_ref_gemm_rows.argtypes = [P, P, P, I64, P, P, I32, I32, I32, P]
    L.moe_ref_gemm_rows.restype = C.c_int
    L.moe_ref_grouped_gemm.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, P]
    L.moe_ref_grouped_gemm.restype = C.c_int
    L.moe_ref_silu_mul_quant.argtypes = [P, I64, I32, P, P, I32, P, P]
    L.moe_ref_silu_mul_quant.restype = C.c_int
    L.moe_ref_unpermute.argtypes = [P, P, P, I64, I32, I32, I32, P]
    L.moe_ref_unpermute.restype = C.c_int
    L.moe_ref_forward_chunked.argtypes = [I64, I32, I32, I32, I32, I32, I32, I32, I64,
                                          P, P, P, P, P, P, P, P, P, P]
    L.moe_ref_forward_chunked.restype = C.c_int
    L.moe_ref_num_threads.argtypes = []; L.moe_ref_num_threads.restype = C.c_int


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


# ---- scalar numerics -------------------------------------------------------
def bf16_from_f32(v: float) -> int:
    return int(lib().moe_ref_bf16_from_f32(float(v)))


def bf16_from_f64(v: float) -> int:
    return int(lib().moe_ref_bf16_from_f64(float(v)))


def e4m3_from_f32(v: float) -> int:
    return int(lib().moe_ref_e4m3_from_f32(float(v)))


def e4m3_value(q: int) -> float:
    return float(lib().moe_ref_e4m3_value(int(q) & 0xFF))


def exp_spec(x: float) -> float:
    return float(lib().moe_ref_exp_spec(float(x)))


def quant_group(v: np.ndarray):
    v = _c(v, np.float32)
    assert v.shape == (GROUP,)
    q = np.empty(GROUP, np.uint8)
    s = np.empty(1, np.float32)
    lib().moe_ref_quant_group(_p(v), _p(q), _p(s))
    return q, s[0]


def loc(i: int, expert_map, Eg: int, El: int) -> int:
    m = _c(expert_map, np.int32)
    return int(lib().moe_ref_loc(int(i), _p(m), Eg, El))


def num_threads() -> int:
    return int(lib().moe_ref_num_threads())


def max_rows(Mc, topk, El, align=128) -> int:
    return int(lib().moe_ref_max_rows(Mc, topk, El, align))


# ---- ops -------------------------------------------------------------------
def count(topk_ids, expert_map, Eg, El):
    ids = _c(topk_ids, np.int32)
    m = _c(expert_map, np.int32)
    counts = np.zeros(El, np.int32)
    bad = np.zeros(1, np.int32)
    _check(lib().moe_ref_count(_p(ids), ids.size, _p(m), Eg, El, _p(counts), _p(bad)), "count")
    return counts, int(bad[0])


def act_quant_identity(x_bits: np.ndarray):
    x = _c(x_bits, np.uint16)
    rows, n = x.shape
    q = np.empty((rows, n), np.uint8)
    s = np.empty((rows, n // GROUP), np.float32)
    _check(lib().moe_ref_act_quant_identity(_p(x), rows, n, _p(q), _p(s)), "act_quant_identity")
    return q, s


def permute(a_q, a_s, topk_ids, topk_weights, apply_on_input, expert_map, Eg, El, align=128,
            cap_rows=None):
    a_q = _c(a_q, np.uint8); a_s = _c(a_s, np.float32)
    ids = _c(topk_ids, np.int32); w = _c(topk_weights, np.float32); m = _c(expert_map, np.int32)
    Mc, K = a_q.shape
    T = ids.shape[1]
    cap = max_rows(Mc, T, El, align) if cap_rows is None else cap_rows
    a_perm = np.empty((cap, K), np.uint8)
    a_perm_s = np.empty((cap, K // GROUP), np.float32)
    counts = np.empty(El, np.int32)
    offs = np.empty(El + 1, np.int32)
    inv = np.empty((Mc, T), np.int32)
    rsrc = np.empty(cap, np.int32)
    _check(lib().moe_ref_permute(_p(a_q), _p(a_s), _p(ids), _p(w), int(apply_on_input), Mc, K, T,
                                 _p(m), Eg, El, align, cap, _p(a_perm), _p(a_perm_s), _p(counts),
                                 _p(offs), _p(inv), _p(rsrc)), "permute")
    return dict(a_perm=a_perm, a_perm_s=a_perm_s, counts=counts, expert_offsets=offs,
                inv_perm=inv, row_src=rsrc, cap_rows=cap)


def gemm_rows(a, a_s, row_expert, w, w_s):
    a = _c(a, np.uint8); a_s = _c(a_s, np.float32); ex = _c(row_expert, np.int32)
    w = _c(w, np.uint8); w_s = _c(w_s, np.float32)
    rows, k_in = a.shape
    El, n_out, _ = w.shape
    out = np.empty((rows, n_out), np.uint16)
    _check(lib().moe_ref_gemm_rows(_p(a), _p(a_s), _p(ex), rows, _p(w), _p(w_s), El, n_out, k_in,
                                   _p(out)), "gemm_rows")
    return out


def grouped_gemm(a, a_s, w, w_s, expert_offsets, counts):
    a = _c(a, np.uint8); a_s = _c(a_s, np.float32); w = _c(w, np.uint8); w_s = _c(w_s, np.float32)
    offs = _c(expert_offsets, np.int32); cnt = _c(counts, np.int32)
    cap, k_in = a.shape
    El, n_out, _ = w.shape
    out = np.empty((cap, n_out), np.uint16)
    _check(lib().moe_ref_grouped_gemm(_p(a), _p(a_s), _p(w), _p(w_s), _p(offs), _p(cnt), El, cap,
                                      n_out, k_in, _p(out)), "grouped_gemm")
    return out


def silu_mul_quant(h, expert_offsets=None, counts=None, El=0):
    h = _c(h, np.uint16)
    rows, two_n = h.shape
    n = two_n // 2
    offs = _c(expert_offsets, np.int32); cnt = _c(counts, np.int32)
    q = np.empty((rows, n), np.uint8)
    s = np.empty((rows, n // GROUP), np.float32)
    _check(lib().moe_ref_silu_mul_quant(_p(h), rows, n, _p(offs), _p(cnt), El, _p(q), _p(s)),
           "silu_mul_quant")
    return q, s


def unpermute(y, inv_perm, topk_weights, apply_on_input):
    y = _c(y, np.uint16); inv = _c(inv_perm, np.int32); w = _c(topk_weights, np.float32)
    Mc, T = inv.shape
    K = y.shape[1]
    out = np.empty((Mc, K), np.uint16)
    _check(lib().moe_ref_unpermute(_p(y), _p(inv), _p(w), Mc, K, T, int(apply_on_input), _p(out)),
           "unpermute")
    return out


def forward_chunked(x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, Eg,
                    apply_on_input=0, chunk_size=0, align=128, want_counts=False):
    x = _c(x, np.uint16); ids = _c(topk_ids, np.int32); w = _c(topk_weights, np.float32)
    m = _c(expert_map, np.int32)
    w13 = _c(w13, np.uint8); w13_s = _c(w13_s, np.float32)
    w2 = _c(w2, np.uint8); w2_s = _c(w2_s, np.float32)
    M, K = x.shape
    T = ids.shape[1]
    El, twoN, _ = w13.shape
    N = twoN // 2
    cs = M if (chunk_size <= 0 or chunk_size >= M) else chunk_size
    nch = (M + cs - 1) // cs if M > 0 else 0
    out = np.empty((M, K), np.uint16)
    pcc = np.empty((max(nch, 1), El), np.int32) if want_counts else None
    _check(lib().moe_ref_forward_chunked(M, K, N, T, Eg, El, align, int(apply_on_input), chunk_size,
                                         _p(x), _p(ids), _p(w), _p(m), _p(w13), _p(w13_s), _p(w2),
                                         _p(w2_s), _p(out), _p(pcc)), "forward_chunked")
    if want_counts:
        return out, pcc[:nch]
    return out
