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


# ---- the Python binding checks every tensor before a pointer reaches the C ABI
import torch  # noqa: E402


def _cpu_layer(El=4, K=256, N=128, Eg=8, emap=None):
    z = lambda *s: torch.zeros(s, dtype=torch.uint8)
    f = lambda *s: torch.ones(s, dtype=torch.float32)
    return moe.MoeLayer(z(El, 2 * N, K), f(El, 2 * N // 128, K // 128), z(El, K, N), f(El, K // 128, N // 128),
                        Eg, emap)


def _good_call(M=10, K=256, T=2):
    return dict(x=torch.zeros((M, K), dtype=torch.int16), topk_ids=torch.zeros((M, T), dtype=torch.int32),
                topk_weights=torch.ones((M, T), dtype=torch.float32))


@pytest.mark.parametrize("bad,exc,match", [
    ("ids_int64", TypeError, "topk_ids has dtype torch.int64"),
    ("weights_f64", TypeError, "topk_weights has dtype torch.float64"),
    ("weights_shape", ValueError, "topk_weights has shape"),
    ("x_noncontig", ValueError, "x must be contiguous"),
    ("x_width", ValueError, "x has shape"),
    ("x_float", TypeError, "x has dtype torch.float32"),
    ("ids_rows", ValueError, "topk_ids has shape"),
    ("out_shape", ValueError, "out has shape"),
    ("pcc_shape", ValueError, "per_chunk_counts has shape"),
])
def test_layer_forward_rejects_bad_tensors(bad, exc, match):
    layer = _cpu_layer()
    a = _good_call()
    kw = {}
    if bad == "ids_int64":
        a["topk_ids"] = a["topk_ids"].long()
    elif bad == "weights_f64":
        a["topk_weights"] = a["topk_weights"].double()
    elif bad == "weights_shape":
        a["topk_weights"] = torch.ones((10, 3), dtype=torch.float32)
    elif bad == "x_noncontig":
        a["x"] = torch.zeros((256, 10), dtype=torch.int16).t()
    elif bad == "x_width":
        a["x"] = torch.zeros((10, 128), dtype=torch.int16)
    elif bad == "x_float":
        a["x"] = torch.zeros((10, 256), dtype=torch.float32)
    elif bad == "ids_rows":
        a["topk_ids"] = torch.zeros((9, 2), dtype=torch.int32)
    elif bad == "out_shape":
        kw["out"] = torch.zeros((10, 128), dtype=torch.int16)
    elif bad == "pcc_shape":
        kw["chunk_size"] = 4
        kw["per_chunk_counts"] = torch.zeros((2, 4), dtype=torch.int32)   # 3 chunks of 4 tokens
    with pytest.raises(exc, match=match):
        layer.forward(a["x"], a["topk_ids"], a["topk_weights"], **kw)


def test_layer_forward_needs_tensors_on_the_gpu():
    # well-formed tensors still never reach the library from host memory
    layer = _cpu_layer()
    a = _good_call()
    with pytest.raises(ValueError, match="current CUDA device"):
        layer.forward(a["x"], a["topk_ids"], a["topk_weights"])


@pytest.mark.parametrize("bad,exc,match", [
    ("w13_float", TypeError, "w13 has dtype"),
    ("w13_s_shape", ValueError, "w13_s has shape"),
    ("w2_shape", ValueError, "w2 has shape"),
    ("w2_s_dtype", TypeError, "w2_s has dtype"),
    ("map_int64", TypeError, "expert_map has dtype"),
    ("map_len", ValueError, "expert_map has shape"),
])
def test_layer_rejects_bad_weights(bad, exc, match):
    El, K, N, Eg = 4, 256, 128, 8
    w13 = torch.zeros((El, 2 * N, K), dtype=torch.uint8)
    w13_s = torch.ones((El, 2, 2), dtype=torch.float32)
    w2 = torch.zeros((El, K, N), dtype=torch.uint8)
    w2_s = torch.ones((El, 2, 1), dtype=torch.float32)
    emap = None
    if bad == "w13_float":
        w13 = w13.float()
    elif bad == "w13_s_shape":
        w13_s = torch.ones((El, 2, 1), dtype=torch.float32)
    elif bad == "w2_shape":
        w2 = torch.zeros((El, N, K), dtype=torch.uint8)
    elif bad == "w2_s_dtype":
        w2_s = w2_s.half()
    elif bad == "map_int64":
        emap = torch.zeros(Eg, dtype=torch.int64)
    elif bad == "map_len":
        emap = torch.zeros(Eg + 1, dtype=torch.int32)
    with pytest.raises(exc, match=match):
        moe.MoeLayer(w13, w13_s, w2, w2_s, Eg, emap)


def test_small_gemm_and_partial_wrappers_check_before_calling():
    t = lambda shape, dt: torch.zeros(shape, dtype=dt)
    u8, f32, i32, b16 = torch.uint8, torch.float32, torch.int32, torch.int16
    a, a_s = t((100, 256), u8), t((100, 2), f32)
    w, w_s = t((4, 512, 256), u8), t((4, 4, 2), f32)
    offs, cnt = t((5,), i32), t((4,), i32)
    with pytest.raises(ValueError, match="out"):
        moe.moe_grouped_gemm_fp8_small(a, a_s, w, w_s, offs, cnt, out=t((100, 256), b16))
    with pytest.raises(ValueError, match="part"):
        moe.moe_grouped_gemm_fp8_small(a, a_s, w, w_s, offs, cnt, part=t((3, 50, 512), f32), nsplit=2,
                                       info=t((1,), i32))
    with pytest.raises(ValueError, match="info"):
        moe.moe_grouped_gemm_fp8_small(a, a_s, w, w_s, offs, cnt, part=t((2, 50, 512), f32), nsplit=2)
    with pytest.raises(ValueError, match="q"):
        moe.moe_act_quant_partials(t((2, 50, 512), f32), t((1,), i32), 256, 100, offs, cnt, t((100, 128), u8),
                                   t((100, 2), f32))
    with pytest.raises(TypeError, match="part"):
        moe.moe_unpermute_partials(t((2, 50, 256), b16), t((1,), i32), offs, cnt, 100, t((8, 4), i32),
                                   t((8, 4), f32), 0, t((8, 256), b16))
    with pytest.raises(ValueError, match="out"):
        moe.moe_unpermute_partials(t((2, 50, 256), f32), t((1,), i32), offs, cnt, 100, t((8, 4), i32),
                                   t((8, 4), f32), 0, t((8, 128), b16))


def test_op_wrappers_check_before_calling():
    cap, k_in, El, n_out = 300, 256, 3, 384
    a = torch.zeros((cap, k_in), dtype=torch.uint8)
    a_s = torch.ones((cap, 2), dtype=torch.float32)
    w = torch.zeros((El, n_out, k_in), dtype=torch.uint8)
    w_s = torch.ones((El, 3, 2), dtype=torch.float32)
    offs = torch.zeros(El + 1, dtype=torch.int32)
    cnt = torch.zeros(El, dtype=torch.int32)
    out = torch.zeros((cap, n_out), dtype=torch.int16)
    with pytest.raises(ValueError, match="a_s has shape"):
        moe.moe_grouped_gemm_fp8(a, a_s[:, :1].contiguous(), w, w_s, offs, cnt, out)
    with pytest.raises(ValueError, match="expert_offsets has shape"):
        moe.moe_grouped_gemm_fp8(a, a_s, w, w_s, offs[:El].contiguous(), cnt, out)
    with pytest.raises(ValueError, match="out has shape"):
        moe.moe_grouped_gemm_fp8(a, a_s, w, w_s, offs, cnt, out[:, :128].contiguous())
    with pytest.raises(ValueError, match="current CUDA device"):
        moe.moe_grouped_gemm_fp8(a, a_s, w, w_s, offs, cnt, out)
    y = torch.zeros((50, 256), dtype=torch.int16)
    with pytest.raises(TypeError, match="inv_perm has dtype torch.int64"):
        moe.moe_unpermute_weight_reduce(y, torch.zeros((10, 2), dtype=torch.int64),
                                        torch.ones((10, 2)), 0, torch.zeros((10, 256), dtype=torch.int16))
    with pytest.raises(ValueError, match="q_s has shape"):
        moe.moe_act_quant(y, 128, moe.MOE_ACT_SILU_MUL, torch.zeros((50, 128), dtype=torch.uint8),
                          torch.zeros((50, 2), dtype=torch.float32))
    with pytest.raises(ValueError, match="a_perm has shape"):
        moe.moe_quant_permute(torch.zeros((10, 256), dtype=torch.int16), torch.zeros((10, 2), dtype=torch.int32),
                              None, 0, None, 8, 8, 128, 100, torch.zeros((99, 256), dtype=torch.uint8),
                              torch.zeros((100, 2)), torch.zeros(8, dtype=torch.int32),
                              torch.zeros(9, dtype=torch.int32), torch.zeros((10, 2), dtype=torch.int32),
                              torch.zeros(100, dtype=torch.int32), torch.zeros(256, dtype=torch.uint8))


def test_forward_workspace_slices_leave_guard_bands():
    for p in (moe.problem(8192, 2048, 768, 8, 128, 64, chunk_size=64), moe.problem(130, 256, 128, 3, 16, 8),
              moe.problem(1, 128, 128, 1, 4, 4)):
        sl = moe.moe_forward_workspace_slices(p)
        total = moe.moe_forward_workspace_size(p)
        lanes = moe.moe_forward_plan_info(p)["lanes"]
        assert len(sl) == 10 * lanes
        ends = [o + n for o, n in sl]
        nxt = [o for o, _ in sl[1:]] + [total]
        for i, ((o, n), e, q) in enumerate(zip(sl, ends, nxt)):
            # the partial sums (slice 8 of a lane) are empty when neither GEMM cuts K
            assert o % 256 == 0 and (n > 0 or i % 10 == 8)
            assert q - e >= 256, "no guard band after a slice"
        if lanes == 2:   # the second lane repeats the first's layout
            assert [n for _, n in sl[10:]] == [n for _, n in sl[:10]]
            assert sl[10][0] - sl[0][0] == total // 2
    # 64-token chunks cut the gate/up GEMM's K; 1-group K and N cut neither
    assert moe.moe_forward_workspace_slices(moe.problem(8192, 2048, 768, 8, 128, 64, chunk_size=64))[8][1] > 0
    assert moe.moe_forward_workspace_slices(moe.problem(1, 128, 128, 1, 4, 4))[8][1] == 0


@pytest.mark.parametrize("args,want", [
    # 64 tokens, topk 4, 64 local experts: small tiles, w13 K (16 groups) in two, w2 K (6 groups) whole
    (dict(M=64, K=2048, N=768, topk=4, Eg=128, El=64), dict(small_tiles=True, nsplit_w13=2, nsplit_w2=1,
                                                          part_rows=256, lanes=1)),
    # 8192 tokens in chunks of 64: the same per chunk, and three lanes
    (dict(M=8192, K=2048, N=768, topk=8, Eg=128, El=64, chunk_size=64),
     dict(small_tiles=True, nsplit_w13=2, nsplit_w2=1, part_rows=512, lanes=3)),
    # two chunks: two lanes
    (dict(M=130, K=2048, N=768, topk=8, Eg=128, El=64, chunk_size=128),
     dict(small_tiles=True, nsplit_w13=2, nsplit_w2=1, part_rows=1024, lanes=2)),
    # a down projection of 16 groups is cut too
    (dict(M=64, K=2048, N=2048, topk=2, Eg=64, El=16), dict(small_tiles=True, nsplit_w13=2, nsplit_w2=2,
                                                          part_rows=128, lanes=1)),
    # the same layer with 64 experts all local: 64 touched experts x 16 gate/up
    # n-tiles fill the chip, so the larger tiles, K whole
    (dict(M=64, K=2048, N=2048, topk=8, Eg=64, El=64), dict(small_tiles=False, nsplit_w13=1, nsplit_w2=1,
                                                          part_rows=0, lanes=1)),
    # 64 tokens, topk 8, all 128 experts local: ~126 touched experts x 6 tiles
    (dict(M=64, K=2048, N=768, topk=8, Eg=128, El=128), dict(small_tiles=False, nsplit_w13=1, nsplit_w2=1,
                                                           part_rows=0, lanes=1)),
    # 384 tokens over 64 of 128 experts (48 pairs per local expert): small tiles
    (dict(M=384, K=2048, N=768, topk=8, Eg=128, El=64), dict(small_tiles=True, nsplit_w13=2, nsplit_w2=1,
                                                           part_rows=3072, lanes=1)),
    # 512 tokens: past 48 pairs per local expert
    (dict(M=512, K=2048, N=768, topk=8, Eg=128, El=64), dict(small_tiles=False, nsplit_w13=1, nsplit_w2=1,
                                                           part_rows=0, lanes=1)),
    # 4096 tokens, topk 8, 128 experts (256 rows each): the 128/256-row GEMMs, K whole
    (dict(M=4096, K=2048, N=768, topk=8, Eg=128, El=128), dict(small_tiles=False, nsplit_w13=1, nsplit_w2=1,
                                                             part_rows=0, lanes=1)),
    # tiny K: small tiles without a cut
    (dict(M=64, K=256, N=128, topk=2, Eg=8, El=8), dict(small_tiles=True, nsplit_w13=1, nsplit_w2=1,
                                                      part_rows=0, lanes=1)),
])
def test_forward_plan_info(args, want):
    a = dict(args)
    p = moe.problem(a.pop("M"), a.pop("K"), a.pop("N"), a.pop("topk"), a.pop("Eg"), a.pop("El"), **a)
    assert moe.moe_forward_plan_info(p) == want


def test_noalloc_plan_stays_in_one_lane():
    # chunked problems need two lanes' slices from moe_forward_chunked but one
    # from the scratch of the no-alloc entry: its size check uses one lane
    p = moe.problem(8192, 2048, 768, 8, 128, 64, chunk_size=64)
    assert moe.moe_forward_plan_info(p)["lanes"] == 3
    sl = moe.moe_forward_workspace_slices(p)
    assert moe.moe_forward_workspace_size(p) == 3 * sl[10][0]


def test_noalloc_forward_rejects_a_problem_beyond_the_scratch():
    # the size check comes before any device call: these pointers are never used
    L = moe.load()
    assert moe._lib.moe_noalloc_scratch_bytes() == 256 << 20
    big = moe.problem(65536, 2048, 768, 8, 128, 128)
    assert moe.moe_forward_workspace_size(big) > moe._lib.moe_noalloc_scratch_bytes()
    fake = C.c_void_p(0x100000)
    out = C.c_void_p(0x4000000000)
    args = [fake, fake, fake, None, fake, fake, fake, fake, out, None, None]
    assert L.moe_forward_chunked_noalloc(C.byref(big), *args) == 3
    assert b"scratch" in L.moe_last_error()
    # the same problem in chunks small enough for the array passes the size check
    # (one lane of slices: the no-alloc entry runs the chunks in order)
    small = moe.problem(65536, 2048, 768, 8, 128, 128, chunk_size=1024)
    one_lane = moe.moe_forward_workspace_size(small) // moe.moe_forward_plan_info(small)["lanes"]
    assert one_lane <= moe._lib.moe_noalloc_scratch_bytes()
