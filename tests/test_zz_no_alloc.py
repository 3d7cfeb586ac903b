"""The allocation-free decode entry point (qa_paged_attention_decode_noalloc,
split partials in the library's static device scratch) against the
workspace call qa_paged_attention_decode: bit-identical outputs on two calls
in a row, the second smaller than the first, and within the decode tolerance
of the oracle. Runs alone in a fresh process as well as after the other GPU
tests (the scratch keeps the previous call's partials; nothing in it has to
start at zero)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import PagedSpec, paged_inputs
from tests.gpu_helpers import say, dev_bits, gpu_cache, oracle_cache, assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_quantize_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


CALLS = [
    # (name, seed, contexts, G, Hkv, d, INT8 V, splits): the second call is smaller
    ("larger", 71, [5000, 17, 3000, 1, 4096, 800], 6, 4, 256, True, 8),
    ("smaller", 72, [900, 33], 6, 4, 256, True, 8),
    ("auto splits", 73, [20000], 6, 4, 256, False, 0),
    ("auto splits, smaller", 74, [1500, 64], 6, 4, 256, False, 0),
]


def _run(qa, inp, splits):
    spec = inp.spec
    kc, ks, vc, vs = gpu_cache(qa, inp, spec.v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q, spec.dtype))
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    want = qa.paged_attention_decode(q8, qs, kc, ks, vc, vs, tables, lens, num_splits=splits)
    got = qa.paged_attention_decode_noalloc(q8, qs, kc, ks, vc, vs, tables, lens, num_splits=splits)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("pair", [(0, 1), (2, 3)], ids=["explicit splits", "auto splits"])
def test_noalloc_decode_two_calls(qa, pair):
    for i in pair:
        name, seed, ctx, G, Hkv, d, v_int8, splits = CALLS[i]
        say(f"noalloc decode: {name} contexts={ctx} splits={splits}")
        spec = PagedSpec("noalloc", seed, len(ctx), G * Hkv, Hkv, d, ctx, [1] * len(ctx), k_bias_std=2.0,
                         v_int8=v_int8, pool_blocks=sum(-(-c // 16) for c in ctx) + 5)
        inp = paged_inputs(spec)
        got, want = _run(qa, inp, splits)
        assert torch.equal(got, want), f"{name}: the allocation-free call differs from the workspace call"
        ref = oracle.paged_decode(*oracle.quantize_q(inp.q, spec.dtype), oracle_cache(inp, v_int8), inp.block_tables,
                                  inp.context_lens, Hkv)
        assert_close(got.cpu().numpy(), ref, f"noalloc {name}")


def test_noalloc_rejects_partials_beyond_the_scratch(qa):
    ctx = [64] * 70
    spec = PagedSpec("noalloc_big", 75, len(ctx), 24, 4, 256, ctx, [1] * len(ctx), pool_blocks=300)
    inp = paged_inputs(spec, seqs=[])
    kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, 4, 256, torch.bfloat16)
    q8 = torch.zeros((70, 24, 256), dtype=torch.int8, device="cuda")
    qs = torch.zeros((70, 24), dtype=torch.float32, device="cuda")
    with pytest.raises(qa.QAttnError, match="static decode scratch"):
        qa.paged_attention_decode_noalloc(q8, qs, kc, ks, vc, vs, torch.from_numpy(inp.block_tables).cuda(),
                                          torch.from_numpy(inp.context_lens).cuda(), num_splits=64)
