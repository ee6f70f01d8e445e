"""Helpers shared by the GPU parity tests: device transfer and comparisons."""
import json
import os
import sys

import numpy as np
import torch

DEV = "cuda:0"
RTOL, ATOL = 1e-2, 1e-3   # bf16 outputs: |gpu - ref| <= ATOL + RTOL*|ref|


# Parity statistics of the layer tests (outputs beyond the tolerance, code
# flips), printed in pytest's terminal summary and, when MOE_PARITY_RECORD
# names a file, written there as JSON lines.
PARITY_RECORD = []


def record(**stats):
    PARITY_RECORD.append(stats)
    path = os.environ.get("MOE_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(stats) + "\n")


def tight_excess(got_bits, ref_bits):
    """(number of outputs beyond ATOL + RTOL|ref|, number compared, largest
    |gpu - ref| / (ATOL + RTOL|ref|)); NaN pairs count as equal."""
    g, r = bf16_f64(got_bits), bf16_f64(ref_bits)
    tol = ATOL + RTOL * np.abs(r)
    ratio = np.abs(g - r) / tol
    ratio[np.isnan(g) & np.isnan(r)] = 0.0
    ratio[np.isnan(ratio)] = np.inf
    return int((ratio > 1.0).sum()), int(ratio.size), float(ratio.max()) if ratio.size else 0.0


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


# bf16 travels as raw 16-bit patterns: numpy uint16 on the host, torch int16
# on the device (only data_ptr() is handed to the library).
def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a.copy()).to(DEV)


def host(t: torch.Tensor, bf16=False) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(np.uint16) if (bf16 or t.dtype == torch.int16) else a


def empty(shape, dtype) -> torch.Tensor:
    if dtype == "bf16":
        dtype = torch.int16
    return torch.empty(shape, dtype=dtype, device=DEV)


def filled(shape, dtype, v) -> torch.Tensor:
    if dtype == "bf16":
        dtype = torch.int16
    return torch.full(shape, v, dtype=dtype, device=DEV)


def bf16_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what=""):
    g, r = bf16_f64(got), bf16_f64(ref)
    bad = ~(np.abs(g - r) <= ATOL + RTOL * np.abs(r))
    bad &= ~(np.isnan(g) & np.isnan(r))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first {idx.tolist()} "
                             f"got {g[tuple(idx[0])]} ref {r[tuple(idx[0])]}")


def valid_rows(offsets: np.ndarray, counts: np.ndarray) -> np.ndarray:
    return np.concatenate([np.arange(offsets[e], offsets[e] + counts[e]) for e in range(len(counts))]
                          + [np.zeros(0, np.int64)]).astype(np.int64)


def partial_rows(part: torch.Tensor, info: torch.Tensor, offsets: np.ndarray, counts: np.ndarray,
                 cap: int) -> np.ndarray:
    """bf16 bits [cap, n] of the rows a small-tile GEMM left as partial slabs
    part [nsplit, part_rows, n]: the fp32 sum of the first S = info[0] slabs
    in slab order, rounded to nearest-even bf16, at the valid rows (place v
    is the v-th valid row in expert order); the other rows are 0."""
    p = host(part)
    S = int(host(info)[0])
    assert 1 <= S <= p.shape[0], f"segment count {S} outside 1..{p.shape[0]}"
    acc = p[0].astype(np.float32).copy()
    for sg in range(1, S):
        acc = (acc + p[sg]).astype(np.float32)
    bits = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rows = valid_rows(offsets, counts)
    out = np.zeros((cap, p.shape[2]), np.uint16)
    out[rows] = bits[:len(rows)]
    return out


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """bf16 spacing at |v| (as float64)."""
    a = np.abs(np.asarray(v, np.float64)).astype(np.float32)
    return np.spacing(a).astype(np.float64) * 65536.0


def gemm_tolerance(ref_bits: np.ndarray, absterm_bits: np.ndarray) -> np.ndarray:
    """Allowed |gpu - ref| for a block-scaled fp8 GEMM output.

    The GPU sums each 128-group inside the fp8 MFMA and folds the groups with
    fp32 FMAs, so its error scales with the sum of the absolute terms
    T = sum_g s_g sum_k |a_k w_k|, not with |ref|: where terms cancel, |ref|
    can be tiny while the error is not.  The gfx950 fp8 MFMA sums its 128
    products in blocks of 8 aligned to the block's largest product, keeping
    about 14 bits below it (test_mfma_fp8_summation_is_block_aligned), so a
    small product next to a large one loses its low bits; random full-range
    codes show errors up to ~2^-14 T.  The bound is 2^-12 T plus the two bf16
    roundings; the benchmark spec's tolerance 1e-3 + 1e-2|ref| is always allowed."""
    ref = bf16_f64(ref_bits)
    T = bf16_f64(absterm_bits) * 1.01
    return np.maximum(ATOL + RTOL * np.abs(ref), 2.0 ** -12 * T + bf16_ulp(np.abs(ref) + 2.0 ** -12 * T))


def assert_gemm_close(got_bits, ref_bits, absterm_bits, what=""):
    g, r = bf16_f64(got_bits), bf16_f64(ref_bits)
    tol = gemm_tolerance(ref_bits, absterm_bits)
    bad = ~(np.abs(g - r) <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        i0 = tuple(idx[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside the GEMM bound; first {idx.tolist()} "
                             f"got {g[i0]} ref {r[i0]} tol {tol[i0]}")
