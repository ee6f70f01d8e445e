"""The C-ABI library loads, exports every entry point its header declares, and
rejects bad arguments on the host (no GPU work is enqueued by these calls)."""
import ctypes as C
import os
import re

import pytest

import unpermute_count_expert_amd as moe
from unpermute_count_expert_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert "moe_forward_chunked" in names and len(names) >= 11
    L = moe.load()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(_lib.EXPORTS)


def test_status_strings():
    L = moe.load()
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"


def test_max_rows_bound():
    assert moe.moe_max_rows(16384, 8, 128, 128) == 131072 + 128 * 127
    assert moe.moe_max_rows(1, 8, 64, 16) == 8 + 8 * 15
    assert moe.moe_max_rows(0, 8, 64, 128) == 0
    assert moe.moe_max_rows(10, 2, 8, 48) == -1


def test_gemm_tile_rows_choice():
    # 256-row tiles once the experts average 256 rows, 128-row tiles below
    assert moe.moe_grouped_gemm_tile_rows(16384 * 8, 128) == 256
    assert moe.moe_grouped_gemm_tile_rows(4096 * 8, 128) == 256
    assert moe.moe_grouped_gemm_tile_rows(4096 * 8 - 1, 128) == 128
    assert moe.moe_grouped_gemm_tile_rows(64 * 8, 64) == 128
    assert moe.moe_grouped_gemm_tile_rows(0, 8) == 128
    assert moe.moe_grouped_gemm_tile_rows(1000, 0) == -1


def test_workspace_size_monotone_in_chunk():
    full = moe.moe_forward_workspace_size(moe.problem(8192, 2048, 768, 8, 128, 64, chunk_size=0))
    small = moe.moe_forward_workspace_size(moe.problem(8192, 2048, 768, 8, 128, 64, chunk_size=64))
    assert 0 < small < full


@pytest.mark.parametrize("kw,status", [
    (dict(K=200), 2), (dict(N=100), 2), (dict(topk=0), 2), (dict(El=0), 2), (dict(El=2000), 2),
    (dict(align=48), 2), (dict(on=2), 1),
])
def test_problem_validation(kw, status):
    a = dict(M=64, K=256, N=128, topk=2, Eg=8, El=8, align=128, on=0)
    a.update(kw)
    p = moe.problem(a["M"], a["K"], a["N"], a["topk"], a["Eg"], a["El"], a["align"], a["on"])
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_workspace_size(p)
    assert ei.value.status == status


def _raw(name):
    return getattr(moe.load(), name)


def test_entry_points_reject_bad_arguments_before_any_launch():
    # pointers are never dereferenced on these paths: validation fails first
    fake = C.c_void_p(0x10000)
    L = moe.load()
    assert L.moe_count(fake, 16, None, 8, 0, fake, None, None) == 2               # El = 0
    assert L.moe_count(fake, 16, None, 8, 9, fake, None, None) == 2               # El > Eg, no map
    assert L.moe_count(None, 16, None, 8, 8, fake, None, None) == 1               # null ids
    # permute: cap_rows below the bound
    cap = moe.moe_max_rows(10, 2, 8, 128)
    assert L.moe_permute(fake, fake, fake, None, 0, 10, 256, 2, None, 8, 8, 128, cap - 1, fake, fake,
                         fake, fake, fake, fake, fake, 1 << 20, None) == 3
    # permute: workspace too small
    assert L.moe_permute(fake, fake, fake, None, 0, 10, 256, 2, None, 8, 8, 128, cap, fake, fake,
                         fake, fake, fake, fake, fake, 0, None) == 3
    # gemm: n_out not a multiple of 128
    assert L.moe_grouped_gemm_fp8(fake, fake, fake, fake, fake, fake, 4, 512, 100, 256, fake, None) == 2
    # act quant: bad mode, and offsets without counts
    assert L.moe_act_quant(fake, 4, 128, 7, None, None, 0, fake, fake, None) == 1
    assert L.moe_act_quant(fake, 4, 128, 0, fake, None, 4, fake, fake, None) == 1
    # unpermute: out overlapping y
    assert L.moe_unpermute_weight_reduce(fake, 10, fake, fake, 4, 128, 2, 0, fake, None) == 1
    # misaligned pointer
    assert L.moe_unpermute_weight_reduce(fake, 10, C.c_void_p(0x10004), fake, 4, 128, 2, 0,
                                         C.c_void_p(0x900000), None) == 1


def test_forward_rejects_small_workspace_and_overlap():
    L = moe.load()
    p = moe.problem(64, 256, 128, 2, 8, 8)
    need = moe.moe_forward_workspace_size(p)
    fake = C.c_void_p(0x100000)
    ws = C.c_void_p(0x40000000)
    out = C.c_void_p(0x80000000)
    args = [C.byref(p), fake, fake, fake, None, fake, fake, fake, fake]
    assert L.moe_forward_chunked(*args, out, ws, need - 1, None, None) == 3
    assert L.moe_forward_chunked(*args, C.c_void_p(0x40000000 + 256), ws, need, None, None) == 1
    assert b"overlaps" in L.moe_last_error()
