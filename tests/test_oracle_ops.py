"""Pins for the oracle's operations: count, permute, GEMM, unpermute, whole layer.

Each op is checked against a second formulation written here (enumeration,
numpy.bincount, a stable argsort, an int64 matmul, float64 matmuls over
dequantised operands) or against invariants the method fixes (counts sum
to the local pairs; permute then unpermute with unit weights and an
identity expert returns topk*x; chunked equals unchunked).
"""
import numpy as np
import pytest
import torch

import oracle
from unpermute_count_expert_amd import generators as gen
from tests.test_oracle_numerics import SPEC, brute_e4m3


def loc_py(ids, expert_map, Eg, El):
    ids = np.asarray(ids, np.int64)
    ok = (ids >= 0) & (ids < Eg)
    if expert_map is None:
        e = np.where(ok & (ids < El), ids, -1)
    else:
        e = np.where(ok, np.asarray(expert_map)[np.clip(ids, 0, Eg - 1)], -1)
        e = np.where((e >= 0) & (e < El), e, -1)
    return e


def bf16_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_via_torch(v):
    # used only where v is exactly representable in fp32 (no double rounding)
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --- count -------------------------------------------------------------------------
@pytest.mark.parametrize("Eg,El,mapped", [(8, 8, False), (128, 64, True), (16, 5, False), (1, 1, False),
                                          (256, 256, False)])
def test_count_against_enumeration_and_bincount(Eg, El, mapped):
    rng = np.random.default_rng(Eg * 7 + El)
    M, T = 97, 6
    ids = gen.random_ids(rng, M, T, Eg, p_minus1=0.05, p_invalid=0.03)
    emap = None
    if mapped:
        emap = np.full(Eg, -1, np.int32)
        emap[Eg - El:] = np.arange(El)
    counts, bad = oracle.count(ids, emap, Eg, El)
    # enumeration
    want = np.zeros(El, np.int64)
    nbad = 0
    for i in ids.reshape(-1):
        if i < -1 or i >= Eg:
            nbad += 1
            continue
        if i == -1:
            continue
        e = emap[i] if emap is not None else (i if i < El else -1)
        if e >= 0:
            want[e] += 1
    np.testing.assert_array_equal(counts, want)
    assert bad == nbad
    e = loc_py(ids, emap, Eg, El).reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(e[e >= 0], minlength=El))
    assert counts.sum() == (e >= 0).sum()


def test_count_all_dropped_and_single_expert():
    ids = np.full((10, 4), -1, np.int32)
    c, bad = oracle.count(ids, None, 8, 8)
    assert c.sum() == 0 and bad == 0
    ids = np.full((10, 4), 3, np.int32)
    c, _ = oracle.count(ids, None, 8, 8)
    assert c[3] == 40 and c.sum() == 40


# --- permute -------------------------------------------------------------------------
def _perm_inputs(seed, M, K, T, Eg, El, mapped):
    rng = np.random.default_rng(seed)
    a_q = gen.random_codes(rng, (M, K))
    a_s = rng.uniform(0.01, 2, (M, K // 128)).astype(np.float32)
    ids = gen.random_ids(rng, M, T, Eg, p_minus1=0.05, p_invalid=0.02)
    w = rng.uniform(0, 1, (M, T)).astype(np.float32)
    emap = None
    if mapped:
        emap = np.full(Eg, -1, np.int32)
        emap[rng.permutation(Eg)[:El]] = np.arange(El)
    return a_q, a_s, ids, w, emap


@pytest.mark.parametrize("align", [16, 32, 64, 128])
@pytest.mark.parametrize("on_input", [0, 1])
def test_permute_against_stable_argsort(align, on_input):
    M, K, T, Eg, El = 77, 256, 4, 32, 12
    a_q, a_s, ids, w, emap = _perm_inputs(align + on_input, M, K, T, Eg, El, True)
    r = oracle.permute(a_q, a_s, ids, w, on_input, emap, Eg, El, align)
    e = loc_py(ids, emap, Eg, El).reshape(-1)
    counts = np.bincount(e[e >= 0], minlength=El)
    np.testing.assert_array_equal(r["counts"], counts)
    seg = align * ((counts + align - 1) // align)
    offs = np.concatenate([[0], np.cumsum(seg)])
    np.testing.assert_array_equal(r["expert_offsets"], offs)
    # second formulation: a stable sort of the flat pairs by local expert
    flat = np.arange(M * T)
    valid = flat[e >= 0]
    order = valid[np.argsort(e[valid], kind="stable")]
    inv = np.full(M * T, -1, np.int64)
    pos = 0
    for x in range(El):
        for j in range(counts[x]):
            inv[order[pos]] = offs[x] + j
            pos += 1
    np.testing.assert_array_equal(r["inv_perm"].reshape(-1), inv)
    rs = np.full(r["cap_rows"], -1)
    rs[inv[inv >= 0]] = flat[inv >= 0] // T
    np.testing.assert_array_equal(r["row_src"], rs)
    for f in flat[inv >= 0]:
        t, k = divmod(f, T)
        row = inv[f]
        np.testing.assert_array_equal(r["a_perm"][row], a_q[t])
        want_s = a_s[t] * w[t, k] if on_input else a_s[t]
        np.testing.assert_array_equal(r["a_perm_s"][row], want_s.astype(np.float32))
    # every expert segment is ordered by token; padding rows are marked -1
    for x in range(El):
        src = r["row_src"][offs[x]:offs[x] + counts[x]]
        assert np.all(np.diff(src) >= 0)
        assert np.all(r["row_src"][offs[x] + counts[x]:offs[x + 1]] == -1)


def test_permute_capacity_error():
    a_q, a_s, ids, w, emap = _perm_inputs(0, 10, 128, 2, 8, 8, False)
    cap = oracle.max_rows(10, 2, 8, 128)
    with pytest.raises(oracle.OracleError):
        oracle.permute(a_q, a_s, ids, w, 0, None, 8, 8, 128, cap_rows=cap - 1)
    with pytest.raises(oracle.OracleError):
        oracle.permute(a_q, a_s, ids, w, 0, None, 8, 8, 48)


# --- GEMM -------------------------------------------------------------------------------
def test_gemm_integer_case_matches_int64_matmul():
    rng = np.random.default_rng(4)
    El, n_out, k_in, rows = 3, 256, 256, 50
    pm1 = np.array([0x00, 0x38, 0xB8], np.uint8)          # 0, +1, -1
    a_i = rng.integers(-1, 2, (rows, k_in))
    w_i = rng.integers(-1, 2, (El, n_out, k_in))
    a = pm1[np.where(a_i < 0, 2, a_i)]
    w = pm1[np.where(w_i < 0, 2, w_i)]
    a_s = np.ones((rows, k_in // 128), np.float32)
    w_s = np.ones((El, n_out // 128, k_in // 128), np.float32)
    ex = rng.integers(0, El, rows).astype(np.int32)
    out = oracle.gemm_rows(a, a_s, ex, w, w_s)
    want = np.einsum("rk,rnk->rn", a_i.astype(np.int64), w_i[ex].astype(np.int64))
    assert np.abs(want).max() <= 256
    np.testing.assert_array_equal(bf16_to_f64(out), want.astype(np.float64))


def _deq_rows(a, a_s):
    rows, k = a.shape
    return (SPEC[a].reshape(rows, k // 128, 128) * a_s.astype(np.float64)[:, :, None]).reshape(rows, k)


def _deq_w(w, w_s):
    E, n, k = w.shape
    v = SPEC[w].reshape(E, n // 128, 128, k // 128, 128)
    return (v * w_s.astype(np.float64)[:, :, None, :, None]).reshape(E, n, k)


def test_gemm_general_against_float64_matmul():
    rng = np.random.default_rng(12)
    El, n_out, k_in, rows = 4, 384, 512, 60
    a = gen.random_codes(rng, (rows, k_in))
    w = gen.random_codes(rng, (El, n_out, k_in))
    a_s = rng.uniform(1e-3, 1, (rows, k_in // 128)).astype(np.float32)
    w_s = rng.uniform(1e-3, 1, (El, n_out // 128, k_in // 128)).astype(np.float32)
    ex = rng.integers(0, El, rows).astype(np.int32)
    out = bf16_to_f64(oracle.gemm_rows(a, a_s, ex, w, w_s))
    A = _deq_rows(a, a_s)
    W = _deq_w(w, w_s)
    ref = np.einsum("rk,rnk->rn", A, W[ex])
    # one bf16 rounding of an (almost) exact value: within half a bf16 ulp
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 2 ** 16
    assert np.all(np.abs(out - ref) <= 0.5 * ulp + 1e-300)
    # a transposed weight or a wrong scale block would not be within that
    ref_bad = np.einsum("rk,rnk->rn", A, _deq_w(w, w_s[:, ::-1, :].copy())[ex])
    assert np.abs(out - ref_bad).max() > 100 * (0.5 * ulp).max()


def test_grouped_gemm_uses_segment_experts_and_zeroes_padding():
    rng = np.random.default_rng(2)
    El, n_out, k_in = 3, 128, 256
    counts = np.array([5, 0, 130], np.int32)
    offs = np.array([0, 128, 128, 384], np.int32)
    cap = 400
    a = gen.random_codes(rng, (cap, k_in))
    a_s = rng.uniform(0.1, 1, (cap, 2)).astype(np.float32)
    w = gen.random_codes(rng, (El, n_out, k_in))
    w_s = rng.uniform(0.1, 1, (El, 1, 2)).astype(np.float32)
    out = oracle.grouped_gemm(a, a_s, w, w_s, offs, counts)
    rows = np.r_[0:5, 128:258]
    ex = np.r_[[0] * 5, [2] * 130].astype(np.int32)
    np.testing.assert_array_equal(out[rows], oracle.gemm_rows(a[rows], a_s[rows], ex, w, w_s))
    mask = np.ones(cap, bool)
    mask[rows] = False
    assert np.all(out[mask] == 0)


# --- unpermute ------------------------------------------------------------------------------
def test_unpermute_topk1_unit_weight_is_copy():
    rng = np.random.default_rng(0)
    y = rng.integers(0, 0x7F00, (50, 256), dtype=np.uint16)
    inv = rng.permutation(50)[:30].reshape(30, 1).astype(np.int32)
    out = oracle.unpermute(y, inv, np.ones((30, 1), np.float32), 0)
    np.testing.assert_array_equal(out, y[inv[:, 0]])


def test_unpermute_exact_sums_and_dropped_pairs():
    rng = np.random.default_rng(1)
    M, T, K, R = 40, 4, 128, 200
    yv = rng.integers(-64, 64, (R, K)).astype(np.float32) / 8       # exact in bf16
    y = f64_to_bf16_via_torch(yv)
    inv = rng.integers(-1, R, (M, T)).astype(np.int32)
    w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], np.float32), (M, T))
    out = bf16_to_f64(oracle.unpermute(y, inv, w, 0))
    ref = np.zeros((M, K))
    for t in range(M):
        for k in range(T):
            if inv[t, k] >= 0:
                ref[t] += w[t, k] * yv[inv[t, k]]
    ref_b = bf16_to_f64(f64_to_bf16_via_torch(ref))    # ref is exact in fp32
    np.testing.assert_array_equal(out, ref_b)
    # on-input mode ignores the weights (they were folded into the scales)
    out1 = bf16_to_f64(oracle.unpermute(y, inv, w * 0 + 3, 1))
    ref1 = np.zeros((M, K))
    for t in range(M):
        for k in range(T):
            if inv[t, k] >= 0:
                ref1[t] += yv[inv[t, k]]
    np.testing.assert_array_equal(out1, bf16_to_f64(f64_to_bf16_via_torch(ref1)))


@pytest.mark.parametrize("mapped", [False, True])
def test_permute_then_unpermute_identity_expert(mapped):
    """Unit weights + identity expert y = bf16(dec(a_perm)*a_perm_s) give
    out[t] = bf16(n_t * bf16(x_hat[t])), i.e. topk * x when all experts are local."""
    rng = np.random.default_rng(5)
    M, K, T, Eg, El = 90, 256, 4, 16, (8 if mapped else 16)
    x = gen.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    ids = np.stack([rng.permutation(Eg)[:T] for _ in range(M)]).astype(np.int32)
    emap = None
    if mapped:
        emap = np.full(Eg, -1, np.int32)
        emap[8:] = np.arange(8)
    a_q, a_s = oracle.act_quant_identity(x)
    r = oracle.permute(a_q, a_s, ids, np.ones((M, T), np.float32), 0, emap, Eg, El)
    yv = _deq_rows(r["a_perm"], r["a_perm_s"])
    y = f64_to_bf16_via_torch(yv.astype(np.float32))
    out = oracle.unpermute(y, r["inv_perm"], np.ones((M, T), np.float32), 0)
    xhat = bf16_to_f64(f64_to_bf16_via_torch(_deq_rows(a_q, a_s).astype(np.float32)))
    n_t = (loc_py(ids, emap, Eg, El) >= 0).sum(axis=1)
    np.testing.assert_array_equal(bf16_to_f64(out), bf16_to_f64(f64_to_bf16_via_torch(n_t[:, None] * xhat)))
    if not mapped:
        assert np.all(n_t == T)


# --- whole layer ------------------------------------------------------------------------------
def _small(M=130, K=256, N=128, Eg=16, El=16, T=4, routing="softmax", seed=3, ep=None):
    cfg = gen.small_config(M=M, K=K, N=N, Eg=Eg, El=El, topk=T, routing=routing, seed=seed,
                           ep_rank_of_2=ep)
    return gen.make_inputs(cfg)


def _fwd(inp, **kw):
    return oracle.forward_chunked(inp.x, inp.topk_ids, inp.topk_weights, inp.expert_map, inp.w13,
                                  inp.w13_s, inp.w2, inp.w2_s, inp.cfg.Eg, **kw)


@pytest.mark.parametrize("on_input", [0, 1])
def test_chunked_equals_unchunked(on_input):
    inp = _small(routing="zipf", El=8, Eg=16, ep=1, seed=8)
    full, c_full = _fwd(inp, apply_on_input=on_input, want_counts=True)
    for cs in (128, 64, 7, 1):
        out, pcc = _fwd(inp, apply_on_input=on_input, chunk_size=cs, want_counts=True)
        np.testing.assert_array_equal(out, full)
        nch = -(-inp.cfg.M // cs)
        assert pcc.shape == (nch, 8)
        e = loc_py(inp.topk_ids, inp.expert_map, 16, 8)
        for c in range(nch):
            ec = e[c * cs:(c + 1) * cs].reshape(-1)
            np.testing.assert_array_equal(pcc[c], np.bincount(ec[ec >= 0], minlength=8))
        np.testing.assert_array_equal(pcc.sum(axis=0), c_full[0])


def test_chunk_tail_130_by_128():
    inp = _small(M=130, routing="zipf", El=8, Eg=16, ep=1, seed=41)
    out, pcc = _fwd(inp, chunk_size=128, want_counts=True)
    assert pcc.shape[0] == 2
    e = loc_py(inp.topk_ids[128:], inp.expert_map, 16, 8).reshape(-1)
    np.testing.assert_array_equal(pcc[1], np.bincount(e[e >= 0], minlength=8))
    np.testing.assert_array_equal(out, _fwd(inp))


def _brute_quant_rows(v):
    """float64/fp32 re-derivation of the 1x128 group quantiser with a brute-force code search."""
    rows, n = v.shape
    g = v.reshape(rows, n // 128, 128).astype(np.float32)
    d = np.maximum(np.abs(g).max(axis=2), np.float32(1e-10)).astype(np.float32)
    s = (d / np.float32(448)).astype(np.float32)
    inv = (np.float32(448) / d).astype(np.float32)
    t = (g * inv[:, :, None]).astype(np.float32)
    q = brute_e4m3(t.reshape(-1)).reshape(rows, n // 128, 128)
    return (SPEC[q] * s.astype(np.float64)[:, :, None]).reshape(rows, n)


@pytest.mark.parametrize("on_input", [0, 1])
def test_whole_layer_tiny_against_float64_brute_force(on_input):
    """The tiny layer (M=64, K=256, N=128, 8 experts, topk=2) recomputed pair by
    pair in float64 from dequantised operands."""
    cfg = gen.CONFIGS["C1"]
    inp = gen.make_inputs(cfg)
    out = bf16_to_f64(_fwd(inp, apply_on_input=on_input))
    M, K, N, T = cfg.M, cfg.K, cfg.N, cfg.topk
    xhat = _brute_quant_rows(bf16_to_f64(inp.x))
    W13 = _deq_w(inp.w13, inp.w13_s)
    W2 = _deq_w(inp.w2, inp.w2_s)
    ref = np.zeros((M, K))
    for t in range(M):
        for k in range(T):
            e = int(inp.topk_ids[t, k])
            wk = np.float64(inp.topk_weights[t, k])
            xin = xhat[t] * wk if on_input else xhat[t]
            h = bf16_to_f64(f64_to_bf16_via_torch((W13[e] @ xin).astype(np.float32)))
            g, u = h[:N], h[N:]
            act = g / (1 + np.exp(-g)) * u
            act = bf16_to_f64(f64_to_bf16_via_torch(act.astype(np.float32)))
            aq = _brute_quant_rows(act[None, :])[0]
            y = bf16_to_f64(f64_to_bf16_via_torch((W2[e] @ aq).astype(np.float32)))
            ref[t] += (1.0 if on_input else wk) * y
    err = np.abs(out - ref)
    assert np.all(err <= 1e-3 + 1e-2 * np.abs(ref)), err.max()


def test_forward_rejects_bad_shapes():
    inp = _small(M=8, K=256, N=128)
    with pytest.raises(oracle.OracleError):
        oracle.forward_chunked(inp.x[:, :200].copy(), inp.topk_ids, inp.topk_weights, None,
                               inp.w13[:, :, :200].copy(), inp.w13_s, inp.w2, inp.w2_s, 16)
    with pytest.raises(oracle.OracleError):
        _fwd(inp, align=48)


def test_zero_tokens_and_all_nonlocal():
    inp = _small(M=20, El=8, Eg=16, ep=1)
    ids = inp.topk_ids.copy()
    ids[:] = 0          # expert 0 is owned by the other rank -> dropped
    out = oracle.forward_chunked(inp.x, ids, inp.topk_weights, inp.expert_map, inp.w13, inp.w13_s,
                                 inp.w2, inp.w2_s, 16)
    assert np.all(out == 0)
