"""Benchmark of the MI355X fused MoE expert layer (one GPU).

Default workload: the large-batch layer, M=16384 tokens, hidden K=2048,
intermediate N=768, 128 local experts, topk=8, uniform softmax-topk routing,
fp8 e4m3 weights with 128x128 fp32 block scales, bf16 in/out.  One step is
one moe_forward_chunked call over the whole batch (input quant, count,
permute, GEMM w13, SiLU-mul requant, GEMM w2, unpermute-reduce), inputs
already resident in HBM.

Prints one JSON line: tokens/s for the layer (steps back to back), the step
time distribution warm and cold (caches flushed before each step), per-op
times measured in place (median, p10, p90, and cold), GEMM TFLOP/s, per-op
algorithmic GB/s (and the GEMM w13 fused with the SiLU-mul requant, timed
on the same buffers), the roofline of the dominant kernel (GEMM w13), the count
on a 2^24-pair case, a measured HBM copy ceiling, the CPU oracle timed on a
bounded sample of the same workload, and (with --other-layers) short step
timings of the other layer configurations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import unpermute_count_expert_amd as moe  # noqa: E402
from unpermute_count_expert_amd import generators as gen  # noqa: E402
from unpermute_count_expert_amd.pipeline import StepBuffers, step_ops  # noqa: E402

METRIC = "MoE layer tokens/s; grouped-GEMM fp8 TFLOP/s; scatter/gather HBM GB/s"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w13_traffic.json")
GEMM_SRC = os.path.join(ROOT, "unpermute_count_expert_amd", "csrc", "gemm_fp8.hip")


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a.copy()).to("cuda:0")


def gemm_source_hash() -> str:
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per GEMM-w13 launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return t.get("bytes_per_launch")


def timed(fn, iters, stream):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters  # ms


def stats(ms_list):
    a = np.asarray(ms_list, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


class Flusher:
    """Writes a 512 MiB buffer, more than the MALL (256 MB) and the L2s hold,
    so that the next kernel starts with cold caches."""

    def __init__(self):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        self.v = 0

    def __call__(self):
        self.v = (self.v + 1) & 0xFF
        self.buf.fill_(self.v)


def per_op_times(layer, d, on_input, iters, stream, only=None, flush=None, fused_input=True):
    """Times each op of the pipeline through its own C-ABI entry point (the
    kernels the fused call runs, plus the standalone count).  Each of `iters`
    passes runs the whole sequence with a HIP event recorded on the launching
    stream before and after every op, so every op is timed in place, between
    its real neighbours; with `flush`, the caches are flushed (untimed) before
    every op.  With `only`, the ops before it run once to fill its inputs and
    only it is launched repeatedly (so a profiler sees no other launch of the
    same kernel).  fused_input=False times the input quant and the permute as
    the two separate calls (not the forward's path).  Returns {op: [ms per
    pass]}."""
    if only in ("input_quant", "permute"):
        fused_input = False
    b = StepBuffers(layer, d["x"].shape[0], d["ids"].shape[1])
    ops = step_ops(layer, d["x"], d["ids"], d["w"], on_input, b, fused=(only == "gemm_w13_act"),
                   fused_input=fused_input, reduce=(only == "gemm_w2_reduce"))
    names = list(ops)
    if only is not None:
        names = names[:names.index(only) + 1]
    for name in names:          # fill every buffer once, in order
        ops[name]()
    torch.cuda.synchronize()
    if only is not None:
        res = {only: [timed(ops[only], iters, stream)]}
    else:
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
               for _ in range(iters)]
        for it in range(iters):
            for i, name in enumerate(names):
                if flush is not None:
                    flush()
                evs[it][i][0].record(stream)
                ops[name]()
                evs[it][i][1].record(stream)
        torch.cuda.synchronize()
        res = {name: [evs[it][i][0].elapsed_time(evs[it][i][1]) for it in range(iters)]
               for i, name in enumerate(names)}
    return res, b.counts.cpu().numpy(), int(b.offsets[-1].item())


def count_scaled(iters, stream):
    """moe_count on 2^24 (token, k) pairs (2^21 tokens x top-8 over 128
    experts, 64 MiB of ids): the layer's own count moves 0.5 MB, too little
    for bandwidth to show.  Timed as calls back to back (20 per event pair,
    the figure GB/s is taken from) and one call per event pair (which adds
    the events' own gaps to a call of a few tens of microseconds).  The
    calls cycle over six copies of the ids (384 MiB, more than the 256 MB
    MALL), so each call reads ids that four other calls' reads have passed
    since its copy was last read."""
    g = torch.Generator(device="cpu").manual_seed(7)
    ids = torch.randint(0, 128, (1 << 21, 8), generator=g, dtype=torch.int32).to("cuda:0")
    copies = [ids] + [ids.clone() for _ in range(5)]
    counts = torch.empty(128, dtype=torch.int32, device="cuda:0")
    nxt = [0]

    def fn():
        moe._lib.moe_count(copies[nxt[0]], None, 128, 128, counts)
        nxt[0] = (nxt[0] + 1) % len(copies)

    fn()
    torch.cuda.synchronize()
    st = stats([timed(fn, 20, stream) for _ in range(iters)])
    st["GB/s"] = round(4 * (1 << 24) / (st["median"] * 1e-3) / 1e9, 1)
    st["hbm_frac"] = round(st["GB/s"] / PEAK_HBM_GBS, 4)
    st["one_call_per_event_pair_ms"] = round(float(np.median([timed(fn, 1, stream) for _ in range(iters)])), 5)
    st["note"] = ("median of %d groups of 20 back-to-back calls over 6 copies of the ids (each call: a clear "
                  "kernel and the count kernel)" % iters)
    return st


def ceilings(iters, stream):
    """Measured HBM ceilings on this GPU: the library's plain streams over
    1 GiB (16-byte accesses, eight in flight per lane, one block per CU): a
    read, a write with non-temporal stores, a write with ordinary stores, and
    a copy (read + write); plus torch's copy_ of the same size for
    reference."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    res = {}
    for name, mode, moved in (("read", moe._lib.MOE_STREAM_READ, n), ("write_nt", moe._lib.MOE_STREAM_WRITE_NT, n),
                              ("write", moe._lib.MOE_STREAM_WRITE, n), ("copy", moe._lib.MOE_STREAM_COPY, 2 * n)):
        fn = lambda: moe._lib.moe_hbm_stream(mode, a, b, n)
        fn()
        st = stats([timed(fn, 1, stream) for _ in range(iters)])
        res[name + "_GB/s"] = round(moved / (st["median"] * 1e-3) / 1e9, 1)
    cp = stats([timed(lambda: b.copy_(a), 1, stream) for _ in range(iters)])
    res["torch_copy_GB/s"] = round(2 * n / (cp["median"] * 1e-3) / 1e9, 1)
    res["note"] = "1 GiB streams, median of %d; copy counts read + written bytes" % iters
    return res


def batched_masked(iters, stream):
    """moe_experts_batched_masked at a decode size: 256 tokens x top-8 routed
    uniformly over 128 experts, the 64 of them local to this GPU (EP rank 1 of
    2), so ~1024 rows over 64 slots of max_tokens = 64; K = 2048, N = 768."""
    rng = np.random.default_rng(12)
    El, max_tokens, K, N = 64, 64, 2048, 768
    ids = np.argsort(-rng.standard_normal((256, 128)), axis=1)[:, :8]
    cnt = np.bincount(ids[ids >= 64] - 64, minlength=El).astype(np.int32)
    rows = El * max_tokens
    a = torch.from_numpy(rng.integers(0, 0x7E, (El, max_tokens, K), dtype=np.uint8)).to("cuda:0")
    a_s = torch.full((El, max_tokens, K // 128), 0.01, dtype=torch.float32, device="cuda:0")
    w13, w13_s = gen.block_weights(rng, El, 2 * N, K)
    w2, w2_s = gen.block_weights(rng, El, K, N)
    w13, w13_s, w2, w2_s = dev(w13), dev(w13_s), dev(w2), dev(w2_s)
    out = torch.empty((El, max_tokens, K), dtype=torch.int16, device="cuda:0")
    ws = torch.empty(moe._lib.moe_batched_workspace_size(El, max_tokens, N), dtype=torch.uint8, device="cuda:0")
    counts = dev(cnt)
    fn = lambda: moe._lib.moe_experts_batched_masked(a, a_s, counts, w13, w13_s, w2, w2_s, out, ws)
    for _ in range(200):
        fn()
    st = stats([timed(fn, 1, stream) for _ in range(iters)])
    P = int(cnt.sum())
    wbytes = 2 * N * K + K * N
    ne = int((cnt > 0).sum())
    return {"workload": f"{El} local experts x {max_tokens} slots, {P} routed rows (256 tokens x top-8 over 128 "
                        f"experts), K={K} N={N}", "ms": st["median"], "p10": st["p10"], "p90": st["p90"],
            "weight_GB/s": round(ne * wbytes / (st["median"] * 1e-3) / 1e9, 1),
            "TFLOP/s": round(2.0 * P * (2 * N * K + K * N) / (st["median"] * 1e-3) / 1e12, 1)}


def small_chunk_ops(iters, stream, name="C2"):
    """The 64-token profiling layer (one chunk, 64 of 128 experts local, top-4)
    op by op through the same kernels the forward runs on it (the small-tile
    GEMMs, the gate/up GEMM's K cut into partial slabs): each op timed in
    place as in per_op_times, after ~0.2 s of warm passes.  At this size the
    GEMMs stream every non-empty expert's weights once, so their roofline is
    those bytes at the 8 TB/s HBM peak."""
    c = gen.CONFIGS[name]
    inp = gen.make_inputs(c)
    layer = moe.MoeLayer(dev(inp.w13), dev(inp.w13_s), dev(inp.w2), dev(inp.w2_s), c.Eg,
                         dev(inp.expert_map) if inp.expert_map is not None else None, c.align)
    d = {"x": dev(inp.x), "ids": dev(inp.topk_ids), "w": dev(inp.topk_weights)}
    t0 = time.time()
    while time.time() - t0 < 0.2:
        per_op_times(layer, d, 0, 5, stream)
    res, counts, _ = per_op_times(layer, d, 0, iters, stream)
    plan = moe.moe_forward_plan_info(layer.problem(c.M, c.topk, 0, 0))
    ne = int((counts > 0).sum())
    wb = {"gemm_w13": ne * 2 * c.N * c.K, "gemm_w2": ne * c.K * c.N}
    ops = {}
    for k, v in res.items():
        if k == "count":
            continue
        m = float(np.median(v))
        e = {"ms": round(m, 5)}
        if k in wb:
            e["weight_MB"] = round(wb[k] / 1e6, 1)
            e["weight_GB/s"] = round(wb[k] / (m * 1e-3) / 1e9, 1)
            e["hbm_frac"] = round(wb[k] / (m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        ops[k] = e
    return {"workload": f"{name}: M={c.M} K={c.K} N={c.N} E={c.El}/{c.Eg} topk={c.topk}, {int(counts.sum())} routed rows "
                        f"over {ne} experts", "plan": plan, "ops": ops,
            "note": "each op between HIP events, so every op's time includes its launch; the forward runs them back to back"}


def algorithmic(cfg, counts: np.ndarray, R: int):
    M, K, N, T = cfg.M, cfg.K, cfg.N, cfg.topk
    P = int(counts.sum())
    Ene = int((counts > 0).sum())
    g1_flops = 2.0 * P * (2 * N) * K
    g2_flops = 2.0 * P * K * N
    by = {
        "count": 4 * M * T + 4 * cfg.El,
        "input_quant": 2 * M * K + M * K + 4 * M * K / 128,
        # the input quant fused into the permute: bf16 x read once
        "quant_permute": 2 * M * K + P * K + 4 * P * K / 128 + 8 * M * T + 4 * R,
        "permute": M * K + 4 * M * K / 128 + P * K + 4 * P * K / 128 + 8 * M * T + 4 * R,
        "gemm_w13": P * K + Ene * 2 * N * K + 4 * P * N + 4 * P * K / 128 + 4 * Ene * (2 * N // 128) * (K // 128),
        # fused with the SiLU-mul requant: h never reaches memory
        "gemm_w13_act": P * K + Ene * 2 * N * K + P * N + 4 * P * N / 128 + 4 * P * K / 128
                        + 4 * Ene * (2 * N // 128) * (K // 128),
        "silu_mul_quant": 4 * P * N + P * N + 4 * P * N / 128,
        "gemm_w2": P * N + Ene * K * N + 2 * P * K + 4 * P * N / 128 + 4 * Ene * (K // 128) * (N // 128),
        "unpermute": 2 * P * K + 8 * M * T + 2 * M * K,
    }
    # (read, written) bytes of the memory-bound ops
    rw = {
        "quant_permute": (2 * M * K + 8 * M * T, P * K + 4 * P * K / 128 + 4 * M * T + 4 * R),
        "silu_mul_quant": (4 * P * N, P * N + 4 * P * N / 128),
        "unpermute": (2 * P * K + 8 * M * T, 2 * M * K),
    }
    return P, Ene, g1_flops, g2_flops, by, rw


def cpu_baseline(inp, on_input, target_s=15.0):
    """The oracle (plain C, OpenMP over rows) on the first S tokens of the
    same workload; S grows geometrically until one run takes about target_s."""
    import oracle
    cfg = inp.cfg

    def run(S):
        t0 = time.perf_counter()
        oracle.forward_chunked(inp.x[:S], inp.topk_ids[:S], inp.topk_weights[:S], inp.expert_map, inp.w13,
                               inp.w13_s, inp.w2, inp.w2_s, cfg.Eg, apply_on_input=on_input, align=cfg.align)
        return time.perf_counter() - t0

    S = 32
    while True:
        ts = run(S)
        if ts >= 0.5 * target_s or S >= cfg.M:
            break
        S = int(min(cfg.M, max(2 * S, S * target_s / max(ts, 1e-3))))
    return {"value": round(S / ts, 2), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {S} of {cfg.M} tokens of the same layer (all {cfg.El} experts' weights), "
                      f"{ts:.1f} s"}


def other_layers(names, warm_s=0.15, timed_s=0.1):
    """Step time of the fused forward on the other layer configurations (hot
    routing, router weight on input, the 4096-token prefill chunk, the
    8192-token layer in chunks of 64 with 64 of 128 experts local, and the
    64-token profiling shape), each on its own seeded inputs: warm-up for
    about warm_s seconds (the clock settles after ~0.1 s of load), then about
    timed_s seconds of steps timed, at least 3 of each."""
    res = {}
    stream = torch.cuda.current_stream()
    for name in names:
        c = gen.CONFIGS[name]
        inp = gen.make_inputs(c)
        emap = dev(inp.expert_map) if inp.expert_map is not None else None
        layer = moe.MoeLayer(dev(inp.w13), dev(inp.w13_s), dev(inp.w2), dev(inp.w2_s), c.Eg, emap, c.align)
        x, ids, w = dev(inp.x), dev(inp.topk_ids), dev(inp.topk_weights)
        out = torch.empty((c.M, c.K), dtype=torch.int16, device="cuda:0")
        fn = lambda: layer.forward(x, ids, w, chunk_size=c.chunk_size, apply_on_input=c.apply_router_weight_on_input,
                                   out=out)
        probe = timed(fn, 1, stream)   # one step, to size the loops
        for _ in range(max(3, int(warm_s / (probe * 1e-3)))):
            fn()
        torch.cuda.synchronize()
        ms = timed(fn, max(3, int(timed_s / (probe * 1e-3))), stream)
        res[name] = {"workload": f"M={c.M} chunk={c.chunk_size} K={c.K} N={c.N} E={c.El}/{c.Eg} topk={c.topk} "
                                 f"routing={c.routing} on_input={c.apply_router_weight_on_input}",
                     "ms_per_step": round(ms, 5), "tokens/s": round(c.M / (ms * 1e-3), 1)}
        del layer, x, ids, w, out
    return res


def copy_calibration(iters):
    """A plain device copy of known size (256 MiB read + 256 MiB written),
    for scaling HBM byte counters."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    ms = timed(lambda: b.copy_(a), iters, stream)
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "ms": round(ms, 5),
                      "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clock settles only after ~0.1 s of continuous load, so the
    # default warm-up runs 100 layer calls (~0.1 s) before the 100 timed ones
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="C5u", choices=sorted(gen.CONFIGS))
    ap.add_argument("--op-iters", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-layers", action="store_true",
                    help="skip the short runs of the other layer configurations")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--profile-op", default=None,
                    help="time only this op (count, quant_permute, input_quant, permute, gemm_w13, silu_mul_quant, "
                         "gemm_w2, unpermute, gemm_w13_act: the fused gate/up variant, or gemm_w2_reduce: the down GEMM with "
                         "the weight-and-reduce), 'count_scaled' (moe_count on 2^24 pairs) or 'copy'; for "
                         "profiler runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU expert-parallel path is not part of it)", file=sys.stderr)
        sys.exit(2)

    if args.profile_op == "copy":
        copy_calibration(args.op_iters)
        return
    if args.profile_op == "count_scaled":
        st = count_scaled(args.op_iters, torch.cuda.current_stream())
        print(json.dumps({"mode": "profile_op", "op": "count_scaled", **st}), flush=True)
        return
    cfg = gen.CONFIGS[args.config]
    on_input = cfg.apply_router_weight_on_input
    t_gen = time.perf_counter()
    inp = gen.make_inputs(cfg)
    t_gen = time.perf_counter() - t_gen
    d = dict(x=dev(inp.x), ids=dev(inp.topk_ids), w=dev(inp.topk_weights),
             emap=dev(inp.expert_map) if inp.expert_map is not None else None)
    layer = moe.MoeLayer(dev(inp.w13), dev(inp.w13_s), dev(inp.w2), dev(inp.w2_s), cfg.Eg, d["emap"], cfg.align)
    stream = torch.cuda.current_stream()
    out = torch.empty((cfg.M, cfg.K), dtype=torch.int16, device="cuda:0")

    def step():
        layer.forward(d["x"], d["ids"], d["w"], chunk_size=cfg.chunk_size, apply_on_input=on_input, out=out)

    if args.profile_op is not None:
        ops, counts, R = per_op_times(layer, d, on_input, args.op_iters, stream, only=args.profile_op)
        print(json.dumps({"mode": "profile_op", "op": args.profile_op, "iters": args.op_iters,
                          "ms": round(ops[args.profile_op][0], 5), "config": cfg.name}), flush=True)
        return

    # the GPU reaches its sustained clock only after ~0.1 s of load: layer
    # steps for 0.3 s first, then the per-op measurements, then the W warm-up
    # and K timed layer steps
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.3:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    ops, counts, R = per_op_times(layer, d, on_input, args.op_iters, stream)
    flush = Flusher()
    ops_cold, _, _ = per_op_times(layer, d, on_input, args.op_iters, stream, flush=flush)
    fused, _, _ = per_op_times(layer, d, on_input, args.op_iters, stream, only="gemm_w13_act")
    reduced, _, _ = per_op_times(layer, d, on_input, args.op_iters, stream, only="gemm_w2_reduce")
    unfused_in, _, _ = per_op_times(layer, d, on_input, args.op_iters, stream, fused_input=False)
    count_big = count_scaled(args.op_iters, stream)
    ceil = ceilings(5, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for k in range(args.steps):
        step()
        evs[k + 1].record(stream)
    evs[-1].synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm = [evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)]
    ms = evs[0].elapsed_time(evs[-1]) / args.steps

    cold = []
    for _ in range(args.steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        cold.append(e0.elapsed_time(e1))

    P, Ene, g1f, g2f, by, rw = algorithmic(cfg, counts, R)
    ops_out = {}
    for name in ops:
        st = stats(ops[name])
        t = st["median"]
        rec = {"ms": t, "p10": st["p10"], "p90": st["p90"], "GB/s": round(by[name] / (t * 1e-3) / 1e9, 1)}
        rec["hbm_frac"] = round(rec["GB/s"] / PEAK_HBM_GBS, 4)
        if name in ("gemm_w13", "gemm_w13_act"):
            rec["TFLOP/s"] = round(g1f / (t * 1e-3) / 1e12, 1)
        if name == "gemm_w2":
            rec["TFLOP/s"] = round(g2f / (t * 1e-3) / 1e12, 1)
        if name in rw:
            # the time the same bytes take on the measured streams: reads at
            # the read stream's rate, writes at the non-temporal write stream's
            floor = rw[name][0] / (ceil["read_GB/s"] * 1e9) + rw[name][1] / (ceil["write_nt_GB/s"] * 1e9)
            rec["read_MB"], rec["write_MB"] = round(rw[name][0] / 1e6, 1), round(rw[name][1] / 1e6, 1)
            rec["measured_stream_floor_ms"] = round(floor * 1e3, 5)
            rec["frac_of_measured_streams"] = round(floor * 1e3 / t, 4)
        tc = stats(ops_cold[name])["median"]
        rec["cold_ms"] = tc
        rec["cold_GB/s"] = round(by[name] / (tc * 1e-3) / 1e9, 1)
        ops_out[name] = rec
    tf = fused["gemm_w13_act"][0]
    ops_out["gemm_w13_act (fused variant, not on the forward path)"] = {
        "ms": round(tf, 5), "GB/s": round(by["gemm_w13_act"] / (tf * 1e-3) / 1e9, 1),
        "TFLOP/s": round(g1f / (tf * 1e-3) / 1e12, 1)}
    tr = reduced["gemm_w2_reduce"][0]
    ops_out["gemm_w2_reduce (w2 with the weight-and-reduce in its epilogue, not on the forward path)"] = {
        "ms": round(tr, 5), "vs_gemm_w2_plus_unpermute_ms": round(stats(ops["gemm_w2"])["median"]
                                                                  + stats(ops["unpermute"])["median"], 5)}
    for name in ("input_quant", "permute"):
        tu = stats(unfused_in[name])["median"]
        ops_out[name + " (separate call, not on the forward path)"] = {
            "ms": tu, "GB/s": round(by[name] / (tu * 1e-3) / 1e9, 1)}
    t_g1 = stats(ops["gemm_w13"])["median"]
    achieved = g1f / (t_g1 * 1e-3) / 1e12
    t_g2 = stats(ops["gemm_w2"])["median"]
    gemm_both = (g1f + g2f) / ((t_g1 + t_g2) * 1e-3) / 1e12
    traffic = measured_traffic()
    wst, cst = stats(warm), stats(cold)
    line = {
        "metric": METRIC,
        "value": round(cfg.M / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: M={cfg.M} K={cfg.K} N={cfg.N} E={cfg.El}/{cfg.Eg} "
                               f"topk={cfg.topk} routing={cfg.routing} on_input={on_input}",
                   "M": cfg.M, "K": cfg.K, "N": cfg.N, "experts": cfg.El, "topk": cfg.topk,
                   "chunk_size": cfg.chunk_size, "align": cfg.align, "pairs": P, "padded_rows": R},
        "roofline": {"bound": "mfma", "kernel": "grouped GEMM w13 (k_grouped_gemm<false, 8>, 256x256 tiles)",
                     "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic},
        "step": {"warm": wst, "cold": cst, "cold_tokens/s": round(cfg.M / (cst["median"] * 1e-3), 1),
                 "note": "warm: steps back to back; cold: a 512 MiB write before each step (untimed)"},
        "gemm_tflops_both": round(gemm_both, 1),
        "gemm_frac_both": round(gemm_both / PEAK_FP8_TFLOPS, 4),
        "ops": ops_out,
        "count_scaled_2^24_pairs": count_big,
        "ceilings": ceil,
        "batched_masked_experts": batched_masked(args.op_iters, stream),
        "small_chunk_ops": small_chunk_ops(args.op_iters, stream),
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(t_gen, 1),
    }
    if not args.no_other_layers:
        line["other_layers"] = other_layers([n for n in ("C5h", "C5u_on", "C3", "C4", "C2") if n != cfg.name])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, on_input, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
