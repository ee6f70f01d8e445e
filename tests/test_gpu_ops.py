"""Per-op parity of the gfx950 kernels (through the C ABI) with the CPU oracle.

Same seeded inputs on both sides.  Bit-exact: counts, offsets, inv_perm,
row_src, permuted rows and scales, act-quant codes and scales, unpermute.
GEMM: on layer-like data (N(0,1) tokens in 1x128 groups, N(0, 0.02) weights
in 128x128 blocks) within 1e-3 + 1e-2|ref| of the oracle; on uniform random
full-range codes within the bound the fp8 MFMA's block-aligned summation
allows (2^-12 of the absolute-term sum, see gpu_helpers.gemm_tolerance); and
bit-exact against an int64 matmul in the integer special case.
"""
import numpy as np
import pytest
import torch

import oracle
import unpermute_count_expert_amd as moe
from unpermute_count_expert_amd import generators as gen
from tests.gpu_helpers import (DEV, announce, assert_bf16_close, assert_gemm_close, dev, empty, filled, host, partial_rows,
                               valid_rows)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- act quant
def _gpu_quant_identity(x_bits):
    rows, n = x_bits.shape
    q = empty((rows, n), torch.uint8)
    s = empty((rows, n // 128), torch.float32)
    moe.moe_act_quant(dev(x_bits), n, moe.MOE_ACT_IDENTITY, q, s)
    return host(q), host(s)


def test_e4m3_every_bf16_value_through_identity_quant():
    """Groups anchored by 448 have scale 448/448 = 1, so each code is e4m3(v)
    of the bf16 input itself: every finite bf16 pattern with |v| <= 448, and
    NaNs, are encoded exactly as the oracle encodes them."""
    announce("e4m3 all-bf16 anchored")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = (pats.astype(np.uint32) << 16).view(np.float32)
    keep = np.isnan(v) | (np.abs(v) <= 448)
    pats = pats[keep]
    pad = (-len(pats)) % 127
    pats = np.concatenate([pats, np.zeros(pad, np.uint16)]).reshape(-1, 127)
    anchor = np.full((pats.shape[0], 1), 0x43E0, np.uint16)   # bf16 448.0
    x = np.concatenate([anchor, pats], axis=1)                 # rows of one group
    q, s = _gpu_quant_identity(x)
    qr, sr = oracle.act_quant_identity(x)
    np.testing.assert_array_equal(s, sr)
    assert np.all(s == 1.0)
    np.testing.assert_array_equal(q, qr)


def test_identity_quant_all_bf16_patterns_shuffled():
    announce("identity quant shuffled patterns")
    rng = np.random.default_rng(0)
    pats = rng.permutation(np.arange(65536, dtype=np.uint32)).astype(np.uint16)
    x = pats.reshape(-1, 256)
    q, s = _gpu_quant_identity(x)
    qr, sr = oracle.act_quant_identity(x)
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(q, qr)


@pytest.mark.parametrize("rows,n,scale", [(1, 128, 1.0), (37, 384, 1e-3), (4096, 2048, 1.0),
                                          (16384, 2048, 3.0)])
def test_identity_quant_parity(rows, n, scale):
    announce("identity quant", rows, n, scale)
    rng = np.random.default_rng(rows + n)
    x = gen.bf16_bits((rng.standard_normal((rows, n)) * scale).astype(np.float32))
    q, s = _gpu_quant_identity(x)
    qr, sr = oracle.act_quant_identity(x)
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(q, qr)


@pytest.mark.parametrize("masked,rows,n", [(False, 1000, 768), (True, 1000, 768), (False, 24, 32768)])
def test_silu_mul_quant_parity(masked, rows, n):
    announce("silu quant masked" if masked else "silu quant", rows, n)
    rng = np.random.default_rng(5)
    h = gen.bf16_bits((rng.standard_normal((rows, 2 * n)) * 4).astype(np.float32))
    # a few extreme gates: large positive / negative, exp clamp region, zeros
    h[0, :8] = gen.bf16_bits(np.array([100, -100, 88.5, -87, 0, -0.0, 1e-30, -3e4], np.float32))
    offs = cnt = None
    El = 0
    if masked:
        cnt = np.array([1, 0, 129, 300, 7], np.int32)
        offs = np.concatenate([[0], np.cumsum(128 * ((cnt + 127) // 128))]).astype(np.int32)
        El = len(cnt)
        assert offs[-1] <= rows
    q = filled((rows, n), torch.uint8, 0xAB)
    s = filled((rows, n // 128), torch.float32, -7.0)
    moe.moe_act_quant(dev(h), n, moe.MOE_ACT_SILU_MUL, q, s,
                      dev(offs) if masked else None, dev(cnt) if masked else None, El)
    qg, sg = host(q), host(s)
    qr, sr = oracle.silu_mul_quant(h, offs, cnt, El)
    rows_v = valid_rows(offs, cnt) if masked else np.arange(rows)
    np.testing.assert_array_equal(sg[rows_v], sr[rows_v])
    np.testing.assert_array_equal(qg[rows_v], qr[rows_v])
    if masked:
        other = np.setdiff1d(np.arange(rows), rows_v)
        assert np.all(qg[other] == 0xAB) and np.all(sg[other] == -7.0)


@pytest.mark.parametrize("offs,cnt", [
    # all but expert 1 run past their slots; the last slot ends past the rows
    ([0, 128, 256, 256, 512, 750], [200, 5, 40, 300, 250]),
    # inconsistent offsets: slots that go backwards and overlap
    ([0, 400, 100, 650, 50, 700], [500, 300, 600, 100, 900]),
])
def test_silu_mul_quant_counts_cut_at_the_slot(offs, cnt):
    """Counts that run past their expert's slot (into the next slot or past
    the array) are cut there, and inconsistent offsets stay in bounds: the
    rows written are exactly those of the cut slots, each with the oracle's
    codes for that row, and nothing else is touched."""
    announce("silu quant cut counts", offs, cnt)
    rng = np.random.default_rng(11)
    rows, n = 700, 256
    h = gen.bf16_bits((rng.standard_normal((rows, 2 * n)) * 4).astype(np.float32))
    offs = np.asarray(offs, np.int32)
    cnt = np.asarray(cnt, np.int32)
    El = len(cnt)
    lo = np.minimum(offs[:-1], rows)
    hi = np.minimum(np.minimum(lo + cnt, rows), np.maximum(offs[1:], lo))
    cut = (hi - lo).astype(np.int32)
    q = filled((rows, n), torch.uint8, 0xAB)
    s = filled((rows, n // 128), torch.float32, -7.0)
    moe.moe_act_quant(dev(h), n, moe.MOE_ACT_SILU_MUL, q, s, dev(offs), dev(cnt), El)
    qg, sg = host(q), host(s)
    # every row's codes depend on that row only: the oracle on all rows
    qr, sr = oracle.silu_mul_quant(h)
    rows_v = np.unique(valid_rows(lo, cut))
    np.testing.assert_array_equal(sg[rows_v], sr[rows_v])
    np.testing.assert_array_equal(qg[rows_v], qr[rows_v])
    other = np.setdiff1d(np.arange(rows), rows_v)
    assert np.all(qg[other] == 0xAB) and np.all(sg[other] == -7.0)


@pytest.mark.parametrize("up,n", [("one", 128), ("random", 128), ("one", 8192), ("random", 8192)])
def test_silu_mul_quant_every_bf16_gate(up, n):
    """Every one of the 65536 bf16 gate patterns (zeros, subnormals, the
    tabulated range, huge values, infinities, NaNs), sorted and shuffled into
    groups, with up = 1 or random: codes and scales bit-exact with the
    oracle's SiLU formula.  n = 128 gives 1024 groups (SiLU by the formula);
    n = 8192 gives 65536 groups, enough rows for the kernel's SiLU table."""
    announce("silu quant all bf16 gates", up, n)
    rng = np.random.default_rng(11)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    reps = 2 if n == 128 else 128
    gates = np.concatenate([pats] + [rng.permutation(pats) for _ in range(reps - 1)]).reshape(-1, n)
    if up == "one":
        ups = np.full(gates.shape, 0x3F80, np.uint16)
    else:
        ups = gen.bf16_bits(rng.standard_normal(gates.shape).astype(np.float32))
    h = np.concatenate([gates, ups], axis=1)
    rows, n = gates.shape
    q = filled((rows, n), torch.uint8, 0xAB)
    sc = filled((rows, n // 128), torch.float32, -7.0)
    moe.moe_act_quant(dev(h), n, moe.MOE_ACT_SILU_MUL, q, sc)
    qr, sr = oracle.silu_mul_quant(h, None, None, 0)
    np.testing.assert_array_equal(host(sc), sr)
    np.testing.assert_array_equal(host(q), qr)


# ---------------------------------------------------------------- count
@pytest.mark.parametrize("M,T,Eg,El,mapped,p_neg,p_bad", [
    (64, 4, 128, 64, True, 0.0, 0.0),
    (16384, 8, 128, 128, False, 0.0, 0.0),
    (1000, 6, 256, 256, False, 0.05, 0.02),
    (333, 2, 16, 1, True, 0.1, 0.05),
    (1 << 21, 8, 128, 128, False, 0.0, 0.0),     # 2^24 pairs (64 MiB of ids)
    ((1 << 22) + 3, 8, 128, 128, False, 0.01, 0.01),   # several batch pairs per lane, ragged tail
    (20000, 8, 1024, 1024, False, 0.01, 0.01),   # 16 slots per expert
    (4096, 8, 4096, 1000, True, 0.02, 0.02),     # a map too long for LDS
    (777, 3, 64, 63, True, 0.0, 0.0),            # odd El: the last expert alone
])
@pytest.mark.parametrize("offset", [0, 1])       # 1: counts only 4-byte aligned
def test_count_parity(M, T, Eg, El, mapped, p_neg, p_bad, offset):
    if offset and M > 100000:
        pytest.skip("the alignment case runs on the small shapes")
    announce("count", M, T, Eg, El, mapped, offset)
    rng = np.random.default_rng(M + El)
    ids = gen.random_ids(rng, M, T, Eg, p_neg, p_bad)
    emap = None
    if mapped:
        emap = np.full(Eg, -1, np.int32)
        emap[rng.permutation(Eg)[:El]] = np.arange(El, dtype=np.int32)
    counts = filled((El + offset,), torch.int32, 12345)[offset:]
    bad = filled((1,), torch.int32, 999)
    moe.moe_count(dev(ids), dev(emap) if mapped else None, Eg, El, counts, bad)
    cr, br = oracle.count(ids, emap, Eg, El)
    np.testing.assert_array_equal(host(counts), cr)
    assert int(host(bad)[0]) == br


def test_count_all_dropped():
    announce("count all dropped")
    ids = np.full((50, 4), -1, np.int32)
    counts = filled((8,), torch.int32, 7)
    moe.moe_count(dev(ids), None, 8, 8, counts)
    assert np.all(host(counts) == 0)


# ---------------------------------------------------------------- permute
def _gpu_permute(a_q, a_s, ids, w, on_input, emap, Eg, El, align):
    Mc, K = a_q.shape
    T = ids.shape[1]
    cap = moe.moe_max_rows(Mc, T, El, align)
    ws = empty((moe.moe_permute_workspace_size(Mc, T, El),), torch.uint8)
    a_perm = filled((cap, K), torch.uint8, 0)
    a_perm_s = filled((cap, K // 128), torch.float32, 0)
    counts = empty((El,), torch.int32)
    offs = empty((El + 1,), torch.int32)
    inv = filled((Mc, T), torch.int32, -77)
    rsrc = filled((cap,), torch.int32, -77)
    moe.moe_permute(dev(a_q), dev(a_s), dev(ids), dev(w), on_input, dev(emap) if emap is not None else None,
                    Eg, El, align, cap, a_perm, a_perm_s, counts, offs, inv, rsrc, ws)
    return dict(a_perm=host(a_perm), a_perm_s=host(a_perm_s), counts=host(counts),
                expert_offsets=host(offs), inv_perm=host(inv), row_src=host(rsrc), cap_rows=cap)


def _check_permute(g, r):
    for k in ("counts", "expert_offsets", "inv_perm", "row_src"):
        np.testing.assert_array_equal(g[k], r[k], err_msg=k)
    rows = valid_rows(r["expert_offsets"], r["counts"])
    np.testing.assert_array_equal(g["a_perm"][rows], r["a_perm"][rows])
    np.testing.assert_array_equal(g["a_perm_s"][rows], r["a_perm_s"][rows])


@pytest.mark.parametrize("M,K,T,Eg,El,mapped,align,on_input,routing", [
    (77, 256, 4, 32, 12, True, 128, 0, "random"),
    (77, 256, 4, 32, 12, True, 16, 1, "random"),
    (300, 384, 3, 20, 20, False, 32, 0, "random"),
    (257, 128, 1, 8, 8, False, 64, 1, "random"),
    (64, 2048, 4, 128, 64, True, 128, 0, "uniform"),       # profiling shape
    (16384, 2048, 8, 128, 128, False, 128, 0, "uniform"),  # large batch
    (16384, 2048, 8, 128, 128, False, 128, 1, "hot"),
    (3, 256, 256, 300, 300, False, 16, 0, "random"),       # topk 256 (one token per block)
    (2500, 2048, 8, 128, 128, False, 128, 1, "uniform"),   # 79 pair blocks x 6 uneven K slices
    (512, 256, 8, 64, 40, True, 32, 0, "random"),          # 16 pair blocks: counted in the scatter
    (513, 256, 8, 64, 40, True, 32, 1, "random"),          # 17: histogram and column scan
    (100, 256, 4, 5000, 64, True, 16, 0, "random"),        # expert map too large for LDS
    (1100, 256, 4, 3000, 48, True, 32, 1, "random"),       # the same, 18 pair blocks: histogram path
    (0, 256, 4, 32, 12, True, 16, 0, "random"),            # an empty chunk: counts and offsets only
    (300, 256, 8, 1024, 1024, False, 16, 1, "random"),     # 1024 experts, counted in the scatter
    (2000, 256, 8, 1024, 1024, False, 16, 0, "random"),    # 1024 experts, histogram path
])
def test_permute_parity(M, K, T, Eg, El, mapped, align, on_input, routing):
    announce("permute", M, K, T, Eg, El, mapped, align, on_input, routing)
    rng = np.random.default_rng(M * 7 + T)
    a_q = gen.random_codes(rng, (M, K))
    a_s = rng.uniform(0.01, 2, (M, K // 128)).astype(np.float32)
    if routing == "random":
        ids = gen.random_ids(rng, M, T, Eg, 0.05, 0.02)
    else:
        cfg = gen.small_config(M=M, K=K, N=128, Eg=Eg, El=El, topk=T,
                               routing="softmax" if routing == "uniform" else "hot", seed=M)
        ids, _, _ = gen.routing(rng, cfg)
    w = rng.uniform(0, 1, (M, T)).astype(np.float32)
    emap = None
    if mapped:
        emap = np.full(Eg, -1, np.int32)
        emap[Eg - El:] = np.arange(El, dtype=np.int32)
    g = _gpu_permute(a_q, a_s, ids, w, on_input, emap, Eg, El, align)
    r = oracle.permute(a_q, a_s, ids, w, on_input, emap, Eg, El, align)
    _check_permute(g, r)


def _gpu_quant_permute(x, ids, w, on_input, emap, Eg, El, align):
    Mc, K = x.shape
    T = ids.shape[1]
    cap = moe.moe_max_rows(Mc, T, El, align)
    ws = empty((moe.moe_permute_workspace_size(Mc, T, El),), torch.uint8)
    a_perm = filled((cap, K), torch.uint8, 0xA5)
    a_perm_s = filled((cap, K // 128), torch.float32, -7.0)
    counts = empty((El,), torch.int32)
    offs = empty((El + 1,), torch.int32)
    inv = filled((Mc, T), torch.int32, -77)
    rsrc = filled((cap,), torch.int32, -77)
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda:0")
    moe.moe_quant_permute(xd, dev(ids), dev(w), on_input, dev(emap) if emap is not None else None,
                          Eg, El, align, cap, a_perm, a_perm_s, counts, offs, inv, rsrc, ws)
    return dict(a_perm=host(a_perm), a_perm_s=host(a_perm_s), counts=host(counts),
                expert_offsets=host(offs), inv_perm=host(inv), row_src=host(rsrc), cap_rows=cap)


@pytest.mark.parametrize("M,K,T,Eg,El,mapped,align,on_input,routing,special", [
    (77, 256, 4, 32, 12, True, 128, 0, "random", False),
    (77, 384, 4, 32, 12, True, 16, 1, "random", True),       # 3 groups a token, NaN/Inf/zero rows
    (300, 640, 3, 20, 20, False, 32, 1, "random", False),    # 5 groups a token
    (64, 2048, 4, 128, 64, True, 128, 0, "uniform", False),  # profiling shape
    (16384, 2048, 8, 128, 128, False, 128, 1, "uniform", False),
    (3, 128, 256, 300, 300, False, 16, 0, "random", True),   # topk 256, one group a token
    (2500, 2048, 8, 128, 128, False, 128, 0, "uniform", False),  # 79 pair blocks x 6 uneven K slices
    (130, 2048, 8, 128, 64, True, 128, 0, "uniform", True),  # 5 pair blocks x 16 K slices
    (512, 384, 8, 64, 40, True, 64, 1, "random", False),     # 16 pair blocks: counted in the scatter
    (513, 384, 8, 64, 40, True, 64, 0, "random", False),     # 17: histogram and column scan
    (100, 256, 4, 5000, 64, True, 16, 1, "random", False),   # expert map too large for LDS
    (1100, 384, 4, 3000, 48, True, 32, 0, "random", False),  # the same, 18 pair blocks: histogram path
    (0, 256, 4, 32, 12, True, 16, 0, "random", False),       # an empty chunk: counts and offsets only
    (400, 256, 8, 1024, 1000, True, 16, 0, "random", False),  # 1000 local experts, counted in the scatter
])
def test_quant_permute_parity(M, K, T, Eg, El, mapped, align, on_input, routing, special):
    """The input quant fused into the permute: bit-exact with the oracle's
    identity quant followed by its permute (codes, scales, offsets, inverse
    and source indices); padding rows are not written."""
    announce("quant permute", M, K, T, Eg, El, mapped, align, on_input, routing, special)
    rng = np.random.default_rng(M * 5 + K)
    xf = (rng.standard_normal((M, K)) * rng.uniform(1e-3, 3, (M, 1))).astype(np.float32)
    if special:
        xf[0, :] = 0.0
        xf[-1, 5] = np.nan
        xf[M // 2, 130 % K] = -np.inf
        xf[M // 2, 7] = 1e30
    x = gen.bf16_bits(xf)
    if routing == "random":
        ids = gen.random_ids(rng, M, T, Eg, 0.05, 0.02)
    else:
        cfg = gen.small_config(M=M, K=K, N=128, Eg=Eg, El=El, topk=T, routing="softmax", seed=M)
        ids, _, _ = gen.routing(rng, cfg)
    w = rng.uniform(0, 1, (M, T)).astype(np.float32)
    emap = None
    if mapped:
        emap = np.full(Eg, -1, np.int32)
        emap[Eg - El:] = np.arange(El, dtype=np.int32)
    g = _gpu_quant_permute(x, ids, w, on_input, emap, Eg, El, align)
    a_q, a_s = oracle.act_quant_identity(x)
    r = oracle.permute(a_q, a_s, ids, w, on_input, emap, Eg, El, align)
    _check_permute(g, r)
    rows = valid_rows(r["expert_offsets"], r["counts"])
    pad = np.setdiff1d(np.arange(g["cap_rows"]), rows)
    assert (g["a_perm"][pad] == 0xA5).all() and (g["a_perm_s"][pad] == -7.0).all(), "padding row written"


def test_permute_single_expert_takes_everything():
    announce("permute single expert")
    rng = np.random.default_rng(1)
    M, K, T = 500, 128, 4
    a_q = gen.random_codes(rng, (M, K))
    a_s = rng.uniform(0.5, 1, (M, 1)).astype(np.float32)
    ids = np.full((M, T), 3, np.int32)
    w = np.ones((M, T), np.float32)
    g = _gpu_permute(a_q, a_s, ids, w, 0, None, 8, 8, 128)
    r = oracle.permute(a_q, a_s, ids, w, 0, None, 8, 8, 128)
    _check_permute(g, r)


# ---------------------------------------------------------------- grouped GEMM
def _gpu_gemm(a, a_s, w, w_s, offs, cnt):
    cap, k_in = a.shape
    El, n_out, _ = w.shape
    out = filled((cap, n_out), "bf16", 0x7FC1)
    moe.moe_grouped_gemm_fp8(dev(a), dev(a_s), dev(w), dev(w_s), dev(offs), dev(cnt), out)
    return host(out, bf16=True)


def _segments(counts, align):
    counts = np.asarray(counts, np.int32)
    offs = np.concatenate([[0], np.cumsum(align * ((counts + align - 1) // align))]).astype(np.int32)
    return offs, counts


@pytest.mark.parametrize("counts,tile", [([1, 130, 0, 257, 64], 128),
                                         ([1, 300, 0, 513, 129], 256)])
def test_gemm_integer_case_bit_exact(counts, tile):
    """Codes in {0, +1, -1} with unit scales: every partial and total is an
    integer of magnitude <= 256, so the result is exact and must equal an
    int64 matmul bit for bit, on both output-tile shapes."""
    announce("gemm integer", counts, tile)
    rng = np.random.default_rng(4)
    El, n_out, k_in = 5, 384, 256
    offs, cnt = _segments(counts, 128)
    cap = int(offs[-1]) + 40
    assert moe.moe_grouped_gemm_tile_rows(cap, El) == tile
    pm1 = np.array([0x00, 0x38, 0xB8], np.uint8)
    a_i = rng.integers(-1, 2, (cap, k_in))
    w_i = rng.integers(-1, 2, (El, n_out, k_in))
    a = pm1[np.where(a_i < 0, 2, a_i)]
    w = pm1[np.where(w_i < 0, 2, w_i)]
    a_s = np.ones((cap, k_in // 128), np.float32)
    w_s = np.ones((El, n_out // 128, k_in // 128), np.float32)
    out = _gpu_gemm(a, a_s, w, w_s, offs, cnt)
    for e in range(El):
        r = np.arange(offs[e], offs[e] + cnt[e])
        want = a_i[r].astype(np.int64) @ w_i[e].T.astype(np.int64)
        got = (out[r].astype(np.uint32) << 16).view(np.float32)
        np.testing.assert_array_equal(got, want.astype(np.float32))
    # rows outside the valid segments are not written
    untouched = np.setdiff1d(np.arange(cap), valid_rows(offs, cnt))
    assert np.all(out[untouched] == 0x7FC1)


def test_mfma_fp8_summation_is_block_aligned():
    """Characterises the in-instruction summation of the 16x16x128 fp8 MFMA
    that the GEMM promotes to fp32 once per 128-group.  Small products alone
    (subnormal, min-normal, 1/8, 1) sum exactly; next to two cancelling
    products of 448*448 in the same block of 8 K-positions, unit products are
    lost while they survive next to 32*448.  The loss stays within 2^-12 of
    the sum of absolute products."""
    announce("mfma summation probe")
    K, N = 128, 128
    smalls = [0x38, 0x20, 0x08, 0x01]          # 1, 1/8, 2^-6, 2^-9
    a = np.zeros((16, K), np.uint8)
    w = np.full((1, N, K), 0x38, np.uint8)     # every column all ones ...
    w[0, 0, 0], w[0, 0, 1] = 0x7E, 0xFE        # ... col 0: +448, -448 at k=0,1
    w[0, 1, 64], w[0, 1, 127] = 0x7E, 0xFE     # ... col 1: +448, -448 at k=64,127
    for i, sm in enumerate(smalls):
        a[i, :] = sm
        a[i, 0] = a[i, 1] = 0x7E
        a[4 + i, :] = sm
        a[4 + i, 64] = a[4 + i, 127] = 0x7E
        a[8 + i, :] = sm
    for i, big in enumerate([0x78, 0x70, 0x68, 0x60]):   # 256, 128, 64, 32
        a[12 + i, :] = 0x38
        a[12 + i, 0] = a[12 + i, 1] = big
    ones = lambda *s: np.ones(s, np.float32)
    offs, cnt = np.array([0, 16], np.int32), np.array([16], np.int32)
    out = _gpu_gemm(a, ones(16, 1), w, ones(1, 1, 1), offs, cnt)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = (oracle.grouped_gemm(a, ones(16, 1), w, ones(1, 1, 1), offs, cnt).astype(np.uint32) << 16
           ).view(np.float32).astype(np.float64)
    absterm = (np.abs(_spec_values()[a]) @ np.abs(_spec_values()[w[0]]).T)
    np.testing.assert_array_equal(got[8:12, :3], ref[8:12, :3])      # small products only: exact
    assert got[15, 0] == ref[15, 0] == 126.0                          # 32*448 neighbours: exact
    assert got[0, 0] < ref[0, 0]                                      # 448*448 neighbours: low bits lost
    err = np.abs(got[:, :4] - ref[:, :4])
    ulp = np.spacing(np.abs(ref[:, :4]).astype(np.float32)).astype(np.float64) * 65536
    assert np.all(err <= 2.0 ** -12 * absterm[:, :4] + ulp)
    print("mfma probe: unit products next to +-448*448 sum to", got[0, 0], "of", ref[0, 0], flush=True)


def _spec_values():
    from tests.test_oracle_numerics import SPEC
    return SPEC


@pytest.mark.parametrize("El,n_out,k_in,counts,align,tile", [
    (4, 256, 512, [1, 127, 128, 300], 128, 128),
    (3, 384, 256, [17, 0, 250], 16, 128),
    (6, 128, 1024, [5, 33, 64, 1, 0, 129], 32, 128),
    (2, 1536, 2048, [200, 77], 128, 128),
    # 256-row tiles: a full tile, tails of 1..255 rows, the second 128-row
    # half of a tile empty or partial, a 128-column last n-tile
    (3, 384, 768, [600, 1, 300], 128, 256),
    (2, 1536, 2048, [513, 256], 128, 256),
    (4, 640, 384, [0, 129, 767, 64], 64, 256),
    # the largest k_in and n_out the library takes, and a long K loop on 256-row tiles
    (1, 128, 65536, [33], 16, 128),
    (1, 32768, 128, [70], 16, 128),
    (1, 32768, 128, [600], 128, 256),
    (2, 256, 16384, [300, 40], 128, 256),
])
def test_gemm_random_parity(El, n_out, k_in, counts, align, tile):
    announce("gemm random", El, n_out, k_in, counts, align, tile)
    rng = np.random.default_rng(n_out + k_in)
    offs, cnt = _segments(counts, align)
    cap = int(offs[-1]) + 3
    assert moe.moe_grouped_gemm_tile_rows(cap, El) == tile
    a = gen.random_codes(rng, (cap, k_in))
    w = gen.random_codes(rng, (El, n_out, k_in))
    a_s = rng.uniform(1e-3, 1, (cap, k_in // 128)).astype(np.float32)
    w_s = rng.uniform(1e-3, 1, (El, n_out // 128, k_in // 128)).astype(np.float32)
    out = _gpu_gemm(a, a_s, w, w_s, offs, cnt)
    ref = oracle.grouped_gemm(a, a_s, w, w_s, offs, cnt)
    absterm = oracle.grouped_gemm(a & 0x7F, a_s, w & 0x7F, w_s, offs, cnt)  # sum of |terms|
    rows = valid_rows(offs, cnt)
    assert_gemm_close(out[rows], ref[rows], absterm[rows], "gemm")
    untouched = np.setdiff1d(np.arange(cap), rows)
    assert np.all(out[untouched] == 0x7FC1)


@pytest.mark.parametrize("El,hi,n_out,k_in,tile,data", [
    (64, 300, 2048, 512, 128, "codes"),    # ~900 128-row tiles (3 LDS stages)
    (48, 700, 2048, 512, 256, "codes"),    # ~620 256-row tiles (2 LDS stages)
    (64, 300, 2048, 512, 128, "layer"),
    (48, 700, 2048, 512, 256, "layer"),
    (1024, 20, 256, 256, 128, "codes"),     # 1024 experts: the prologue's scans at full width
])
def test_gemm_full_grid_every_row(El, hi, n_out, k_in, tile, data):
    """Several times more tiles than the persistent grid has blocks, over
    many experts of uneven size (some empty, some exact tile multiples), with
    a K loop of four steps: every block walks many tiles, its DMA stream runs
    ahead across tile and expert boundaries, and every valid row is compared
    with the oracle.  "codes": uniform random e4m3 codes and scales, within
    the GEMM bound for full-range codes; "layer": activations and weights
    drawn and quantised like the layer's (N(0,1) tokens in 1x128 groups,
    N(0, 0.02) weights in 128x128 blocks), within 1e-3 + 1e-2|ref|."""
    announce("gemm full grid", El, hi, n_out, k_in, tile, data)
    rng = np.random.default_rng(El * 1000 + hi + (data == "layer"))
    cnt = rng.integers(0, hi + 1, El).astype(np.int32)
    cnt[::9] = 0
    cnt[1::11] = tile
    cnt[2::13] = 2 * tile
    offs, cnt = _segments(cnt, 128)
    cap = int(offs[-1]) + 5
    assert moe.moe_grouped_gemm_tile_rows(cap, El) == tile
    mt = int(((cnt + tile - 1) // tile).sum())
    assert mt * (n_out // 256) >= 2 * 256, "not enough tiles to exercise the persistent walk"
    if data == "codes":
        a = gen.random_codes(rng, (cap, k_in))
        w = gen.random_codes(rng, (El, n_out, k_in))
        a_s = rng.uniform(1e-3, 1, (cap, k_in // 128)).astype(np.float32)
        w_s = rng.uniform(1e-3, 1, (El, n_out // 128, k_in // 128)).astype(np.float32)
    else:
        a, a_s = oracle.act_quant_identity(gen.bf16_bits(rng.standard_normal((cap, k_in), dtype=np.float32)))
        w, w_s = gen.block_weights(rng, El, n_out, k_in)
    out = _gpu_gemm(a, a_s, w, w_s, offs, cnt)
    ref = oracle.grouped_gemm(a, a_s, w, w_s, offs, cnt)
    rows = valid_rows(offs, cnt)
    if data == "codes":
        absterm = oracle.grouped_gemm(a & 0x7F, a_s, w & 0x7F, w_s, offs, cnt)
        assert_gemm_close(out[rows], ref[rows], absterm[rows], "gemm full grid")
    else:
        assert_bf16_close(out[rows], ref[rows], "gemm full grid")
    assert np.all(out[np.setdiff1d(np.arange(cap), rows)] == 0x7FC1)


def _small_operands(rng, El, hi, n_out, k_in, align=16):
    cnt = rng.integers(0, hi + 1, El).astype(np.int32)
    cnt[::7] = 0
    offs, cnt = _segments(cnt, align)
    cap = int(offs[-1]) + 3
    a, a_s = oracle.act_quant_identity(gen.bf16_bits(rng.standard_normal((cap, k_in), dtype=np.float32)))
    w, w_s = gen.block_weights(rng, El, n_out, k_in)
    return a, a_s, w, w_s, offs, cnt, cap


def _num_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("El,hi,n_out,k_in,nsplit", [
    (64, 4, 1536, 2048, 2),     # 64-token decode chunk, gate/up: K cut in two
    (64, 4, 1536, 2048, 8),     # eight segments of two groups
    (16, 90, 512, 1024, 4),     # experts past one 64-row tile
    (8, 3, 256, 2048, 1),       # one slab: whole-K sums
    (40, 20, 768, 768, 3),      # down-projection K (6 groups) cut in three
    (300, 30, 2048, 512, 2),    # tiles enough for four rounds: K kept whole
    (1024, 2, 256, 256, 2),     # 1024 experts: the prologue's scans at full width
])
def test_small_gemm_and_partials(El, hi, n_out, k_in, nsplit):
    """moe_grouped_gemm_fp8_small on layer-like data: without part, the bits
    of moe_grouped_gemm_fp8 on every valid row and no other row written;
    with part, info reports the cut (nsplit while the 64-row tiles fill
    fewer than four rounds of the CUs, else 1), the slabs' sum in slab
    order rounded to bf16 is within 1e-3 + 1e-2|ref| of the oracle's exact
    GEMM (and is the plain GEMM's bits with one slab), and no slab row past
    the valid rows is written."""
    announce("small gemm", El, hi, n_out, k_in, nsplit)
    rng = np.random.default_rng(El * 7 + hi + nsplit)
    a, a_s, w, w_s, offs, cnt, cap = _small_operands(rng, El, hi, n_out, k_in)
    rows = valid_rows(offs, cnt)
    plain = _gpu_gemm(a, a_s, w, w_s, offs, cnt)
    A, As, W, Ws, O, Cn = dev(a), dev(a_s), dev(w), dev(w_s), dev(offs), dev(cnt)
    out = filled((cap, n_out), "bf16", 0x7FC1)
    moe.moe_grouped_gemm_fp8_small(A, As, W, Ws, O, Cn, out=out)
    o = host(out, bf16=True)
    np.testing.assert_array_equal(o[rows], plain[rows])
    assert np.all(o[np.setdiff1d(np.arange(cap), rows)] == 0x7FC1), "a row that is not valid was written"
    pr = len(rows) + 5
    part = filled((nsplit, pr, n_out), torch.float32, -3.0)
    info = filled((1,), torch.int32, -1)
    moe.moe_grouped_gemm_fp8_small(A, As, W, Ws, O, Cn, part=part, nsplit=nsplit, info=info)
    tiles = int(((cnt + 63) // 64).sum()) * -(-n_out // 256)
    want = nsplit if tiles < 4 * _num_cus() else 1
    assert int(host(info)[0]) == want
    h = partial_rows(part, info, offs, cnt, cap)
    ref = oracle.grouped_gemm(a, a_s, w, w_s, offs, cnt)
    assert_bf16_close(h[rows], ref[rows], "small gemm partials")
    if want == 1:
        np.testing.assert_array_equal(h[rows], plain[rows])
    p = host(part)
    assert np.all(p[:want, len(rows):] == -3.0), "a slab row past the valid rows was written"


@pytest.mark.parametrize("El,hi,n,nsplit,short", [(64, 4, 768, 2, False), (16, 90, 256, 4, False),
                                                  (8, 3, 128, 8, False), (30, 10, 384, 1, False),
                                                  (16, 90, 256, 4, True)])
def test_act_quant_and_unpermute_from_partials(El, hi, n, nsplit, short):
    """The SiLU-mul requant and the unpermute that read the small GEMM's
    partial slabs give the bits of moe_act_quant / the unpermute run on the
    slabs' bf16 sum (formed on the host in slab order), on every valid row
    and token, and leave rows that are not valid alone.  short: the requant
    is given slabs of only half the valid rows (its grid is sized by them),
    and the rows past them read as zero."""
    announce("partials consumers", El, hi, n, nsplit, short)
    rng = np.random.default_rng(El + hi + n + nsplit)
    k_in = 1024
    # the gate/up GEMM: 2n outputs as partial slabs
    a, a_s, w, w_s, offs, cnt, cap = _small_operands(rng, El, hi, 2 * n, k_in)
    rows = valid_rows(offs, cnt)
    A, As, W, Ws, O, Cn = dev(a), dev(a_s), dev(w), dev(w_s), dev(offs), dev(cnt)
    part = filled((nsplit, max(len(rows), 1), 2 * n), torch.float32, 0.0)
    info = filled((1,), torch.int32, -1)
    moe.moe_grouped_gemm_fp8_small(A, As, W, Ws, O, Cn, part=part, nsplit=nsplit, info=info)
    h = partial_rows(part, info, offs, cnt, cap)
    part_q, h_q = part, h
    if short:
        pr = max(1, len(rows) // 2)
        part_q = part[:, :pr].contiguous()
        h_q = h.copy()
        h_q[rows[pr:]] = 0
    q1, s1 = filled((cap, n), torch.uint8, 0xA5), filled((cap, n // 128), torch.float32, -7.0)
    moe.moe_act_quant_partials(part_q, info, n, cap, O, Cn, q1, s1)
    q2, s2 = filled((cap, n), torch.uint8, 0), filled((cap, n // 128), torch.float32, 0.0)
    moe.moe_act_quant(dev(h_q), n, moe.MOE_ACT_SILU_MUL, q2, s2, O, Cn, El)
    q1, s1, q2, s2 = host(q1), host(s1), host(q2), host(s2)
    np.testing.assert_array_equal(q1[rows], q2[rows])
    np.testing.assert_array_equal(s1[rows], s2[rows])
    pad = np.setdiff1d(np.arange(cap), rows)
    assert (q1[pad] == 0xA5).all() and (s1[pad] == -7.0).all(), "the requant wrote a row that is not valid"
    # the unpermute: every valid row is one (token, k) pair, some pairs -1
    topk = 4
    Mc = max(1, -(-len(rows) // topk) + 2)
    inv = np.full(Mc * topk, -1, np.int32)
    slots = rng.choice(Mc * topk, len(rows), replace=False)
    inv[slots] = rng.permutation(rows).astype(np.int32)
    inv = inv.reshape(Mc, topk)
    tw = rng.uniform(0.05, 1.0, (Mc, topk)).astype(np.float32)
    K = 2 * n   # the slabs' width serves as the output width
    for on_input in (0, 1):
        o1 = filled((Mc, K), "bf16", 0x7FC1)
        moe.moe_unpermute_partials(part, info, O, Cn, cap, dev(inv), dev(tw), on_input, o1)
        o2 = filled((Mc, K), "bf16", 0)
        moe.moe_unpermute_weight_reduce(dev(h), dev(inv), dev(tw), on_input, o2)
        np.testing.assert_array_equal(host(o1, bf16=True), host(o2, bf16=True))


@pytest.mark.parametrize("El,max_tokens,n_out,k_in,tile", [
    (16, 16, 768, 2048, 128),     # decode-sized slots: 0..16 rows per expert
    (6, 300, 384, 768, 256),      # slots longer than a 256-row tile
    (4, 512, 256, 512, 256),
])
def test_gemm_masked_batched_layout(El, max_tokens, n_out, k_in, tile):
    """The batched, masked layout [E, max_tokens, K] with a valid-row count
    per expert (low-latency dispatch, vLLM PR #20903 Purpose) is the grouped
    GEMM with expert_offsets[e] = e * max_tokens: slots need not be packed or
    aligned.  Counts include an empty and a full slot; the SiLU-mul requant
    is checked on the same layout."""
    announce("gemm masked batched", El, max_tokens, n_out, k_in, tile)
    rng = np.random.default_rng(El * max_tokens)
    cnt = rng.integers(0, max_tokens + 1, El).astype(np.int32)
    cnt[0], cnt[-1] = 0, max_tokens
    offs = (np.arange(El + 1) * max_tokens).astype(np.int32)
    cap = El * max_tokens
    assert moe.moe_grouped_gemm_tile_rows(cap, El) == tile
    a = gen.random_codes(rng, (cap, k_in))
    w = gen.random_codes(rng, (El, n_out, k_in))
    a_s = rng.uniform(1e-3, 1, (cap, k_in // 128)).astype(np.float32)
    w_s = rng.uniform(1e-3, 1, (El, n_out // 128, k_in // 128)).astype(np.float32)
    out = _gpu_gemm(a, a_s, w, w_s, offs, cnt)
    ref = oracle.grouped_gemm(a, a_s, w, w_s, offs, cnt)
    absterm = oracle.grouped_gemm(a & 0x7F, a_s, w & 0x7F, w_s, offs, cnt)
    rows = valid_rows(offs, cnt)
    assert_gemm_close(out[rows], ref[rows], absterm[rows], "gemm masked")
    assert np.all(out[np.setdiff1d(np.arange(cap), rows)] == 0x7FC1)
    # SiLU-mul requant over the same slots, on the oracle's own GEMM output
    # (the act width is n_out / 2 rounded down to whole groups)
    n = (n_out // 2) // 128 * 128
    h = np.ascontiguousarray(ref[:, :2 * n])
    q = filled((cap, n), torch.uint8, 0xAB)
    s = filled((cap, n // 128), torch.float32, -7.0)
    moe.moe_act_quant(dev(h), n, moe.MOE_ACT_SILU_MUL, q, s, dev(offs), dev(cnt), El)
    qr, sr = oracle.silu_mul_quant(h, offs, cnt, El)
    qg, sg = host(q), host(s)
    np.testing.assert_array_equal(sg[rows], sr[rows])
    np.testing.assert_array_equal(qg[rows], qr[rows])
    other = np.setdiff1d(np.arange(cap), rows)
    assert np.all(qg[other] == 0xAB) and np.all(sg[other] == -7.0)


# ---------------------------------------------------------------- unpermute
def test_unpermute_empty_y_gives_zero():
    """With no rows in y every pair is dropped, so every token's output is +0,
    also where each token's columns are split over several waves (few tokens,
    K past whole 512-column slabs)."""
    announce("unpermute empty y")
    rng = np.random.default_rng(31)
    M, K, T = 37, 2176, 8
    y = np.zeros((0, K), np.uint16)
    inv = rng.integers(0, 500, (M, T)).astype(np.int32)
    w = rng.uniform(0, 1, (M, T)).astype(np.float32)
    out = filled((M, K), "bf16", 0x7FC1)
    moe.moe_unpermute_weight_reduce(dev(y), dev(inv), dev(w), 0, out)
    got = host(out, bf16=True)
    assert np.all(got == 0)
    np.testing.assert_array_equal(got, oracle.unpermute(y, np.full((M, T), -1, np.int32), w, 0))


@pytest.mark.parametrize("M,K,T,on_input", [(1, 128, 1, 0), (513, 2048, 8, 0), (100, 384, 3, 1),
                                            (16384, 2048, 8, 0),
                                            (77, 2176, 8, 1),     # a second, partial pass of slabs
                                            (37, 640, 12, 0),     # more than eight rows a token
                                            (20, 2176, 20, 1)])
def test_unpermute_parity(M, K, T, on_input):
    announce("unpermute", M, K, T, on_input)
    rng = np.random.default_rng(M + K)
    R = M * T + 50
    y = gen.bf16_bits(rng.standard_normal((R, K)).astype(np.float32))
    inv = rng.permutation(R)[:M * T].reshape(M, T).astype(np.int32)
    inv[rng.random((M, T)) < 0.1] = -1
    # indices past the rows of y are never read; they count as dropped pairs
    oob = rng.random((M, T)) < 0.05
    inv_gpu = np.where(oob, R + 7, inv).astype(np.int32)
    inv_ref = np.where(oob, -1, inv).astype(np.int32)
    w = rng.uniform(0, 1, (M, T)).astype(np.float32)
    out = filled((M, K), "bf16", 0x7FC1)
    moe.moe_unpermute_weight_reduce(dev(y), dev(inv_gpu), dev(w), on_input, out)
    got = host(out, bf16=True)
    ref = oracle.unpermute(y, inv_ref, w, on_input)
    np.testing.assert_array_equal(got, ref)   # same fmaf order on both sides


# ------------------------------------------------- batched, masked experts
@pytest.mark.parametrize("El,max_tokens,K,N", [
    (16, 16, 2048, 768),     # decode-sized slots at the layer's shape
    (8, 300, 512, 256),      # slots longer than a 256-row tile
    (64, 1, 256, 128),       # one token per slot
])
def test_batched_masked_experts_parity(El, max_tokens, K, N):
    """moe_experts_batched_masked (the experts on the [El, max_tokens, K]
    layout of low-latency dispatch) computes the same bits as the op chain
    on the same slots: GEMM w13, the masked SiLU-mul requant, GEMM w2 with
    expert_offsets[e] = e * max_tokens and the counts cut at the slot.  The
    chain's steps against the oracle: h and y within 1e-3 + 1e-2|ref|, the act
    codes bit-exact given the GPU's h.  Slots: empty, full, over-full (cut)."""
    announce("batched masked experts", El, max_tokens, K, N)
    rng = np.random.default_rng(El * 7 + max_tokens)
    cnt = rng.integers(0, max_tokens + 1, El).astype(np.int32)
    cnt[0], cnt[-1] = 0, max_tokens
    cnt[1] = max_tokens + 9                      # cut at the slot
    cut = np.minimum(cnt, max_tokens).astype(np.int32)
    rows = El * max_tokens
    a, a_s = oracle.act_quant_identity(gen.bf16_bits(rng.standard_normal((rows, K), dtype=np.float32)))
    w13, w13_s = gen.block_weights(rng, El, 2 * N, K)
    w2, w2_s = gen.block_weights(rng, El, K, N)
    offs = (np.arange(El + 1) * max_tokens).astype(np.int32)
    d = dict(a=dev(a), a_s=dev(a_s), w13=dev(w13), w13_s=dev(w13_s), w2=dev(w2), w2_s=dev(w2_s))
    out = filled((El, max_tokens, K), "bf16", 0x7FC1)
    ws = empty((moe._lib.moe_batched_workspace_size(El, max_tokens, N),), torch.uint8)
    moe._lib.moe_experts_batched_masked(d["a"].view(El, max_tokens, K), d["a_s"].view(El, max_tokens, K // 128),
                                        dev(cnt), d["w13"], d["w13_s"], d["w2"], d["w2_s"], out, ws)
    got = host(out, bf16=True).reshape(rows, K)
    # the op chain on the cut slots
    h = filled((rows, 2 * N), "bf16", 0)
    moe.moe_grouped_gemm_fp8(d["a"], d["a_s"], d["w13"], d["w13_s"], dev(offs), dev(cut), h)
    q = filled((rows, N), torch.uint8, 0)
    s = filled((rows, N // 128), torch.float32, 0)
    moe.moe_act_quant(h, N, moe.MOE_ACT_SILU_MUL, q, s, dev(offs), dev(cut), El)
    y = filled((rows, K), "bf16", 0x7FC1)
    moe.moe_grouped_gemm_fp8(q, s, d["w2"], d["w2_s"], dev(offs), dev(cut), y)
    valid = valid_rows(offs, cut)
    np.testing.assert_array_equal(got[valid], host(y, bf16=True)[valid])
    assert np.all(got[np.setdiff1d(np.arange(rows), valid)] == 0x7FC1), "a row past a slot's count was written"
    # the chain against the oracle
    hg, qg, sg = host(h, bf16=True), host(q), host(s)
    h_ref = oracle.grouped_gemm(a, a_s, w13, w13_s, offs, cut)
    assert_bf16_close(hg[valid], h_ref[valid], "batched h")
    qr, sr = oracle.silu_mul_quant(hg, offs, cut, El)
    np.testing.assert_array_equal(qg[valid], qr[valid])
    np.testing.assert_array_equal(sg[valid], sr[valid])
    y_ref = oracle.grouped_gemm(qg, sg, w2, w2_s, offs, cut)
    assert_bf16_close(got[valid], y_ref[valid], "batched out")


# ------------------------------------------------------------ HBM streams
def test_hbm_streams_move_every_byte():
    """The measured-ceiling streams: the copy reproduces its source exactly
    (including a tail that is not a whole grid stride), and both writes touch
    every byte."""
    announce("hbm streams")
    n = (3 << 20) + 48
    src = torch.from_numpy(np.random.default_rng(3).integers(0, 256, n, dtype=np.uint8)).to(DEV)
    dst = filled((n,), torch.uint8, 0)
    moe._lib.moe_hbm_stream(moe._lib.MOE_STREAM_COPY, src, dst, n)
    np.testing.assert_array_equal(host(dst), host(src))
    for mode in (moe._lib.MOE_STREAM_WRITE_NT, moe._lib.MOE_STREAM_WRITE):
        dst.fill_(0)
        moe._lib.moe_hbm_stream(mode, None, dst, n)
        assert (host(dst) != 0).all()
    sink = filled((16,), torch.uint8, 0)
    moe._lib.moe_hbm_stream(moe._lib.MOE_STREAM_READ, src, sink, n)
    torch.cuda.synchronize()
