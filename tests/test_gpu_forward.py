"""Whole-layer parity: moe_forward_chunked on the GPU against the oracle.

Small layers are compared in full; the full-size layers (prefill 4096 and
large batch 16384 tokens) on sampled tokens, which the oracle computes on
their own (a token's output depends only on its own row, ids and weights).
Per-chunk counts are compared bit for bit; chunked GPU runs are compared
with the unchunked GPU run.
"""
import numpy as np
import pytest
import torch

import oracle
import unpermute_count_expert_amd as moe
from unpermute_count_expert_amd import generators as gen
from tests.gpu_helpers import announce, assert_bf16_close, dev, filled, host

pytestmark = pytest.mark.gpu


_INPUTS = {}


def _inputs(key):
    """make_inputs for a named config; the weight-sharing on/off variants of
    one seed reuse the same arrays."""
    cfg = gen.CONFIGS[key]
    k = (cfg.seed, cfg.M, cfg.routing)
    if k not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[k] = gen.make_inputs(cfg)
    inp = _INPUTS[k]
    return gen.LayerInputs(cfg, inp.x, inp.topk_ids, inp.topk_weights, inp.expert_map, inp.w13,
                           inp.w13_s, inp.w2, inp.w2_s, inp.extra)


def _layer(inp):
    emap = dev(inp.expert_map) if inp.expert_map is not None else None
    return moe.MoeLayer(dev(inp.w13), dev(inp.w13_s), dev(inp.w2), dev(inp.w2_s), inp.cfg.Eg, emap,
                        inp.cfg.align)


def _gpu_forward(layer, inp, chunk_size, on_input, want_counts=False, x=None, ids=None, w=None):
    x = dev(inp.x) if x is None else x
    ids = dev(inp.topk_ids) if ids is None else ids
    w = dev(inp.topk_weights) if w is None else w
    M = x.shape[0]
    cs = M if chunk_size <= 0 or chunk_size >= M else chunk_size
    nch = -(-M // cs)
    pcc = filled((nch, layer.El), torch.int32, -5) if want_counts else None
    out = layer.forward(x, ids, w, chunk_size=chunk_size, apply_on_input=on_input, per_chunk_counts=pcc)
    return host(out, bf16=True), (host(pcc) if want_counts else None)


def _oracle_forward(inp, chunk_size, on_input, rows=None):
    x, ids, w = inp.x, inp.topk_ids, inp.topk_weights
    if rows is not None:
        x, ids, w = x[rows], ids[rows], w[rows]
    return oracle.forward_chunked(x, ids, w, inp.expert_map, inp.w13, inp.w13_s, inp.w2, inp.w2_s,
                                  inp.cfg.Eg, apply_on_input=on_input, chunk_size=chunk_size,
                                  align=inp.cfg.align, want_counts=True)


SMALL = [
    ("C1", gen.CONFIGS["C1"], 0),
    ("C1_on", gen.CONFIGS["C1"], 1),
    ("small_chunked", gen.small_config(M=300, K=512, N=256, Eg=32, El=16, topk=4, chunk_size=64,
                                       routing="zipf", seed=21, ep_rank_of_2=1), 0),
    ("small_align16", gen.small_config(M=150, K=256, N=384, Eg=16, El=16, topk=3, chunk_size=0,
                                       routing="softmax", seed=22, align=16), 1),
    ("C2_profiling", gen.CONFIGS["C2"], 0),
    ("C4b_tail_130_by_128", gen.CONFIGS["C4b"], 0),
]


@pytest.mark.parametrize("name,cfg,on_input", SMALL, ids=[s[0] for s in SMALL])
def test_forward_small_full_parity(name, cfg, on_input):
    announce("forward", name, on_input)
    inp = gen.make_inputs(cfg)
    layer = _layer(inp)
    got, pcc = _gpu_forward(layer, inp, cfg.chunk_size, on_input, want_counts=True)
    ref, pcc_ref = _oracle_forward(inp, cfg.chunk_size, on_input)
    np.testing.assert_array_equal(pcc, pcc_ref)
    assert_bf16_close(got, ref, name)
    if cfg.chunk_size and cfg.chunk_size < cfg.M:
        whole, _ = _gpu_forward(layer, inp, 0, on_input)
        np.testing.assert_array_equal(got, whole)   # rows are independent: no split-K


def _sample_rows(M, rng, n=48):
    picks = np.unique(np.concatenate([[0, 1, M // 2, M - 2, M - 1], rng.choice(M, n, replace=False)]))
    return picks.astype(np.int64)


LARGE = [("C3_prefill", "C3", 0), ("C5u", "C5u", 0), ("C5u_on", "C5u_on", 1), ("C5h", "C5h", 0),
         ("C5h_on", "C5h_on", 1)]


@pytest.mark.parametrize("name,key,on_input", LARGE, ids=[s[0] for s in LARGE])
def test_forward_large_sampled_parity(name, key, on_input):
    announce("forward sampled", name)
    cfg = gen.CONFIGS[key]
    inp = _inputs(key)
    layer = _layer(inp)
    got, pcc = _gpu_forward(layer, inp, 0, on_input, want_counts=True)
    counts_ref, _ = oracle.count(inp.topk_ids, inp.expert_map, cfg.Eg, cfg.El)
    np.testing.assert_array_equal(pcc[0], counts_ref)
    rows = _sample_rows(cfg.M, np.random.default_rng(cfg.seed))
    ref, _ = _oracle_forward(inp, 0, on_input, rows)
    assert_bf16_close(got[rows], ref, name)


def test_forward_chunk_stress_zipf():
    """8192 tokens in chunks of 64 with Zipf routing over 64 local of 128
    experts: per-chunk counts bit for bit (including zero-count experts),
    sampled tokens against the oracle, and chunked == unchunked on the GPU."""
    announce("forward chunk stress C4")
    cfg = gen.CONFIGS["C4"]
    inp = gen.make_inputs(cfg)
    layer = _layer(inp)
    got, pcc = _gpu_forward(layer, inp, cfg.chunk_size, 0, want_counts=True)
    nch = cfg.M // cfg.chunk_size
    for c in range(nch):
        ids_c = inp.topk_ids[c * 64:(c + 1) * 64]
        np.testing.assert_array_equal(pcc[c], oracle.count(ids_c, inp.expert_map, cfg.Eg, cfg.El)[0])
    assert (pcc == 0).sum() > 0, "some local expert must get no tokens in some chunk"
    rows = _sample_rows(cfg.M, np.random.default_rng(4), 40)
    ref, _ = _oracle_forward(inp, 0, 0, rows)
    assert_bf16_close(got[rows], ref, "C4")
    whole, _ = _gpu_forward(layer, inp, 0, 0)
    np.testing.assert_array_equal(got, whole)


def test_forward_all_pairs_nonlocal_gives_zero():
    announce("forward all non-local")
    cfg = gen.small_config(M=70, K=256, N=128, Eg=16, El=8, topk=2, routing="softmax", seed=3,
                           ep_rank_of_2=1)
    inp = gen.make_inputs(cfg)
    ids = np.where(inp.topk_ids >= 8, inp.topk_ids - 8, inp.topk_ids).astype(np.int32)  # all < 8: remote
    got, _ = _gpu_forward(_layer(inp), inp, 0, 0, ids=dev(ids))
    assert np.all(got == 0)


def test_forward_m1_and_empty():
    announce("forward M=1")
    cfg = gen.small_config(M=1, K=128, N=128, Eg=4, El=4, topk=1, routing="softmax", seed=9)
    inp = gen.make_inputs(cfg)
    layer = _layer(inp)
    got, _ = _gpu_forward(layer, inp, 1, 0)
    ref, _ = _oracle_forward(inp, 1, 0)
    assert_bf16_close(got, ref, "M=1")
    out = layer.forward(dev(inp.x[:0]), dev(inp.topk_ids[:0]), dev(inp.topk_weights[:0]))
    assert out.shape == (0, 128)


def test_forward_is_deterministic():
    announce("forward determinism")
    cfg = gen.small_config(M=512, K=512, N=256, Eg=32, El=32, topk=4, routing="zipf", seed=5)
    inp = gen.make_inputs(cfg)
    layer = _layer(inp)
    a, _ = _gpu_forward(layer, inp, 0, 0)
    b, _ = _gpu_forward(layer, inp, 0, 0)
    np.testing.assert_array_equal(a, b)
