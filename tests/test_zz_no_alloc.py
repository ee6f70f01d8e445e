"""moe_forward_chunked_noalloc (the forward for callers that cannot allocate:
its workspace is the library's fixed per-GPU scratch array) against
moe_forward_chunked with a caller workspace, through the C ABI: the same
kernels, so the same bits, on two calls in a row where the second is smaller
(the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import unpermute_count_expert_amd as moe
from unpermute_count_expert_amd import generators as gen
from tests.gpu_helpers import announce, dev, filled, host

pytestmark = pytest.mark.gpu


def _layer(inp):
    emap = dev(inp.expert_map) if inp.expert_map is not None else None
    return moe.MoeLayer(dev(inp.w13), dev(inp.w13_s), dev(inp.w2), dev(inp.w2_s), inp.cfg.Eg, emap, inp.cfg.align)


def _both(layer, inp, M, chunk_size, on_input):
    x, ids, w = dev(inp.x[:M]), dev(inp.topk_ids[:M]), dev(inp.topk_weights[:M])
    p = layer.problem(M, inp.cfg.topk, chunk_size, on_input)
    nch = -(-M // (M if chunk_size <= 0 or chunk_size >= M else chunk_size))
    assert moe.moe_forward_workspace_size(p) <= moe._lib.moe_noalloc_scratch_bytes()
    pcc_ref = filled((nch, layer.El), torch.int32, -3)
    ref = layer.forward(x, ids, w, chunk_size=chunk_size, apply_on_input=on_input, per_chunk_counts=pcc_ref)
    out = filled((M, layer.K), "bf16", 0x7FC1)
    pcc = filled((nch, layer.El), torch.int32, -5)
    moe._lib.moe_forward_chunked_noalloc(p, x, ids, w, layer.expert_map, layer.w13, layer.w13_s, layer.w2,
                                         layer.w2_s, out, pcc)
    np.testing.assert_array_equal(host(out, bf16=True), host(ref, bf16=True))
    np.testing.assert_array_equal(host(pcc), host(pcc_ref))


@pytest.mark.parametrize("name,cfg,first,second", [
    # 130 tokens in chunks of 128 (a 2-token tail), then 61 tokens in one chunk
    ("C4b", gen.CONFIGS["C4b"], (130, 128, 0), (61, 0, 0)),
    # 1000 hot-routed tokens in chunks of 300 with 64-row alignment, then 77
    # tokens with the router weight applied on the input
    ("hot_align64", gen.small_config(M=1000, K=1024, N=512, Eg=64, El=64, topk=6, chunk_size=300,
                                     routing="hot", seed=25, align=64), (1000, 300, 0), (77, 0, 1)),
])
def test_noalloc_forward_matches_workspace_forward(name, cfg, first, second):
    announce("noalloc forward", name)
    inp = gen.make_inputs(cfg)
    layer = _layer(inp)
    _both(layer, inp, *first)
    _both(layer, inp, *second)
