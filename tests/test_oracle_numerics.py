"""Pins for the oracle's numerics (bf16, E4M3FN, exp, group quantiser, SiLU).

Each check compares the oracle with something other than itself: the OCP
OFP8 table (golden fixtures), an exhaustive brute-force nearest-code search
written here, torch's own casts, float64 math and Fraction arithmetic.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --- an independent E4M3FN table, from the format definition --------------
def spec_e4m3_values():
    """value of every code: bias 7, 3 mantissa bits, exp 0 subnormal, S.1111.111 NaN."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m / 512.0
        else:
            vals[c] = sign * (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


SPEC = spec_e4m3_values()
POS = SPEC[:0x7F]  # finite non-negative magnitudes, codes 0x00..0x7E ascending


def brute_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest finite code by exhaustive search; ties to the even code; saturating."""
    v = v.astype(np.float64)
    out = np.empty(v.shape, np.uint8)
    nan = np.isnan(v)
    sign = np.signbit(v)
    a = np.minimum(np.abs(np.where(nan, 0, v)), 448.0)
    d = np.abs(a[:, None] - POS[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer an even code (even mantissa)
    even = cand & ((np.arange(0x7F) % 2) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)
    out[:] = pick | np.where(sign, 0x80, 0).astype(np.uint8)
    out[nan] = (0x7F | np.where(sign[nan], 0x80, 0)).astype(np.uint8)
    return out


def oracle_e4m3(v):
    return np.array([oracle.e4m3_from_f32(float(x)) for x in np.asarray(v, np.float32)], np.uint8)


def all_bf16_as_f32():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


def read_fixture(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --- E4M3FN ------------------------------------------------------------------
def test_e4m3_golden_table():
    for code_hex, val in read_fixture("e4m3fn_ocp.txt"):
        c = int(code_hex, 16)
        got = oracle.e4m3_value(c)
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))
            assert oracle.e4m3_from_f32(float(val)) == c


def test_e4m3_golden_rounding():
    for val, code_hex in read_fixture("e4m3fn_saturating_rounding.txt"):
        assert oracle.e4m3_from_f32(float(val)) == int(code_hex, 16), val


def test_e4m3_decode_matches_format_definition():
    for c in range(256):
        a, b = oracle.e4m3_value(c), SPEC[c]
        assert (math.isnan(a) and math.isnan(b)) or a == b


def test_e4m3_exhaustive_over_bf16_inputs():
    v = all_bf16_as_f32()
    np.testing.assert_array_equal(oracle_e4m3(v), brute_e4m3(v))


def test_e4m3_random_fp32_inputs():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14, 10, 60000)).astype(np.float32)
    v = np.where(rng.random(60000) < 0.5, -mag, mag).astype(np.float32)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = np.concatenate([v, bits])
    np.testing.assert_array_equal(oracle_e4m3(v), brute_e4m3(v))


def test_e4m3_matches_torch_cast_on_clamped_inputs():
    v = all_bf16_as_f32()
    v = v[~np.isnan(v)]
    vc = np.clip(v, -448, 448).astype(np.float32)
    t = torch.from_numpy(vc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle_e4m3(v), t)


# --- bf16 ----------------------------------------------------------------------
def test_bf16_from_f32_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x807FFFFF,
                        0x3F808000, 0x3F818000, 0x3F80FFFF, 0x7F800000, 0xFF800000], np.uint32)
    bits = np.concatenate([bits, special])
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_f32(float(x)) for x in v], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_bf16_nan_stays_nan():
    for b in (0x7FC00000, 0x7F800001, 0xFFC00000):
        x = np.array([b], np.uint32).view(np.float32)[0]
        out = oracle.bf16_from_f32(float(x))
        assert (out & 0x7F80) == 0x7F80 and (out & 0x7F) != 0


def _nearest_bf16_fraction(x: Fraction) -> float:
    """Brute force: the two bf16 neighbours of x by exact rational arithmetic."""
    if x == 0:
        return 0.0
    a = abs(x)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (max(e, -126) - 7)
    lo = (a // step) * step
    hi = lo + step
    dl, dh = a - lo, hi - a
    if dl < dh:
        r = lo
    elif dh < dl:
        r = hi
    else:
        r = lo if (lo / step) % 2 == 0 else hi
    r = float(r)
    return -r if x < 0 else r


def test_bf16_from_f64_single_rounding():
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(1500) * np.exp2(rng.uniform(-30, 30, 1500)))
    # halfway points of bf16 and points just off them (double rounding traps)
    for b in rng.integers(0x3000, 0x5000, 300):
        lo = float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(int(b) + 1) << 16], np.uint32).view(np.float32)[0])
        mid = (lo + hi) / 2
        vals += [mid, mid + (hi - lo) * 2.0 ** -30, mid - (hi - lo) * 2.0 ** -30]
    for v in vals:
        want = _nearest_bf16_fraction(Fraction(v))
        got_bits = oracle.bf16_from_f64(v)
        got = float(np.array([got_bits << 16], np.uint32).view(np.float32)[0])
        assert got == want, (v, got, want)


# --- exp_spec ------------------------------------------------------------------
def test_exp_spec_accuracy_against_float64():
    xs = np.concatenate([np.linspace(-86, 88, 40001), np.linspace(-1, 1, 4001)]).astype(np.float32)
    got = np.array([oracle.exp_spec(float(x)) for x in xs], np.float64)
    ref = np.exp(xs.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(got - ref) / ulp
    assert err.max() <= 2.0, err.max()


def test_exp_spec_special_points():
    assert oracle.exp_spec(0.0) == 1.0
    # clamped ends stay finite and normal
    assert oracle.exp_spec(1000.0) == oracle.exp_spec(88.0) and math.isfinite(oracle.exp_spec(1000.0))
    assert oracle.exp_spec(-1000.0) == oracle.exp_spec(-86.0) > 2.0 ** -126


# --- group quantiser -------------------------------------------------------------
@pytest.mark.parametrize("scale", [1e-6, 1e-2, 1.0, 37.0, 1e5])
def test_quant_group_invariants(scale):
    rng = np.random.default_rng(int(scale * 1000) % 2**31)
    for _ in range(50):
        v = (rng.standard_normal(128) * scale).astype(np.float32)
        q, s = oracle.quant_group(v)
        dec = SPEC[q]
        amax = np.float32(np.abs(v).max())
        d = max(amax, np.float32(1e-10))
        assert s == np.float32(d) / np.float32(448.0)
        assert np.abs(dec).max() == 448.0
        inv = np.float32(448.0) / np.float32(d)
        t = (v * inv).astype(np.float32)
        # each code is the nearest E4M3 value of v*inv ...
        np.testing.assert_array_equal(q, brute_e4m3(t))
        # ... so the dequantised group is within half an E4M3 step (times s)
        half_step = np.where(np.abs(t) < 2 ** -6, 2.0 ** -10,
                             2.0 ** (np.floor(np.log2(np.maximum(np.abs(t), 2 ** -6))) - 4))
        err = np.abs(dec * np.float64(s) - v.astype(np.float64))
        bound = (half_step + 448 * 2.0 ** -22) * np.float64(s)
        assert np.all(err <= bound)


def test_quant_group_all_zero():
    q, s = oracle.quant_group(np.zeros(128, np.float32))
    assert np.all(q == 0)
    assert s == np.float32(1e-10) / np.float32(448.0)


# --- SiLU-and-mul ----------------------------------------------------------------
def test_silu_mul_quant_against_float64():
    rng = np.random.default_rng(9)
    rows, n = 40, 256
    h = torch.from_numpy((rng.standard_normal((rows, 2 * n)) * 3).astype(np.float32)).to(torch.bfloat16)
    hb = h.view(torch.int16).numpy().view(np.uint16)
    q, s = oracle.silu_mul_quant(hb)
    hf = h.to(torch.float64)
    g, u = hf[:, :n], hf[:, n:]
    act = (torch.nn.functional.silu(g) * u).numpy()
    dec = SPEC[q].reshape(rows, n // 128, 128) * s[:, :, None]
    dec = dec.reshape(rows, n)
    # error budget: bf16 rounding of act (2^-8 relative) + half an e4m3 step
    # of the group (2^-4 relative to the element, at most 2^-4*448*s absolute)
    bound = np.abs(act) * 2.0 ** -8 + np.repeat(s, 128, axis=1) * 448 * 2.0 ** -4 + 1e-30
    assert np.all(np.abs(dec - act) <= bound)
    # the gate half is the one passed through SiLU: swapping the halves breaks it
    act_swapped = (torch.nn.functional.silu(u) * g).numpy()
    assert np.abs(dec - act_swapped).max() > 10 * np.abs(dec - act).max()


def test_silu_mul_quant_rows_masked_by_offsets():
    rng = np.random.default_rng(1)
    h = rng.integers(0, 0x3F00, (300, 256), dtype=np.uint16)
    offs = np.array([0, 128, 128, 256], np.int32)
    counts = np.array([5, 0, 100], np.int32)
    q, s = oracle.silu_mul_quant(h, offs, counts, 3)
    qa, sa = oracle.silu_mul_quant(h)
    valid = np.zeros(300, bool)
    valid[0:5] = True
    valid[128:228] = True
    np.testing.assert_array_equal(q[valid], qa[valid])
    np.testing.assert_array_equal(s[valid], sa[valid])
    assert np.all(q[~valid] == 0) and np.all(s[~valid] == 0)


def test_quant_group_skips_quiet_and_signalling_nans():
    v = np.linspace(-3, 3, 128).astype(np.float32)
    bits = v.view(np.uint32).copy()
    bits[5] = 0x7FC00000   # quiet NaN
    bits[9] = 0x7F800001   # signalling NaN
    bits[77] = 0xFFA00000  # negative signalling NaN
    w = bits.view(np.float32)
    q, s = oracle.quant_group(w)
    finite = np.ones(128, bool)
    finite[[5, 9, 77]] = False
    assert s == np.float32(np.abs(v[finite]).max()) / np.float32(448)
    assert q[5] == 0x7F and q[9] == 0x7F and q[77] == 0xFF
    q2, _ = oracle.quant_group(np.where(finite, v, 0).astype(np.float32))
    np.testing.assert_array_equal(q[finite], q2[finite])
