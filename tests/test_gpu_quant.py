"""GPU parity, bit-exact: query quantization, cache writing, the INT32 QK
accumulators of the decode kernel, and the SageAttention preprocessing."""
import numpy as np
import pytest
import torch

import oracle
from workloads import (PagedSpec, DenseSpec, paged_inputs, dense_inputs, to_bf16_bits, to_f16_bits,
                       tiny_decode, qwen27b_decode, batched_splitk_decode, chunked_prefill, dense_sage)
from tests.gpu_helpers import say, dev_bits, gpu_cache, oracle_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_quantize_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _q_bits(T, H, d, dtype, seed):
    x = np.random.default_rng(seed).standard_normal((T, H, d)).astype(np.float32)
    x[0, 0] = 0.0                                   # zero row
    if T > 1:
        x[1, 0] = 0.0
        x[1, 0, :8] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, 126.5, -1.5]   # s = 1 exactly: ties
    if T > 2:
        x[2, 0] *= 1e-30 if dtype == "bf16" else 1e-4   # tiny magnitudes
    if T > 3:
        x[3, 0] *= 1e4 if dtype == "bf16" else 100.0
    if T > 4 and dtype == "bf16":
        x[4, 0] *= 1e-37                            # the row scale is an fp32 subnormal
    return to_bf16_bits(x) if dtype == "bf16" else to_f16_bits(x)


QSHAPES = [(1, 6, 64), (1, 24, 256), (32, 24, 256), (2048, 24, 256), (7, 3, 128), (5, 16, 64), (4099, 6, 128)]


@pytest.mark.parametrize("shape", QSHAPES, ids=[f"{t}x{h}x{d}" for t, h, d in QSHAPES])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_quantize_q_bit_exact(qa, shape, dtype):
    T, H, d = shape
    say(f"quantize_q {dtype} {shape}")
    bits = _q_bits(T, H, d, dtype, seed=T * 31 + H + d)
    q8, qs = qa.quantize_q(dev_bits(bits, dtype))
    torch.cuda.synchronize()
    w8, ws = oracle.quantize_q(bits, dtype)
    assert np.array_equal(q8.cpu().numpy(), w8)
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), ws.view(np.uint32))


def test_quantize_q_strided_view(qa):
    say("quantize_q strided view")
    bits = _q_bits(9, 4, 256, "bf16", 5)
    big = dev_bits(np.concatenate([bits, bits[:, :, :128]], axis=2), "bf16")   # [9, 4, 384]
    view = big[:, :, :256]
    q8, qs = qa.quantize_q(view)
    w8, ws = oracle.quantize_q(bits, "bf16")
    assert np.array_equal(q8.cpu().numpy(), w8) and np.array_equal(qs.cpu().numpy(), ws)


def test_quantize_q_empty(qa):
    q8, qs = qa.quantize_q(torch.empty((0, 24, 256), dtype=torch.bfloat16, device="cuda"))
    assert q8.shape == (0, 24, 256) and qs.shape == (0, 24)


KV_CASES = [
    dict(d=64, G=6, Hkv=1, ctx=[256], v_int8=False),
    dict(d=256, G=6, Hkv=4, ctx=[300, 17], v_int8=False),
    dict(d=256, G=6, Hkv=4, ctx=[130, 1, 45], v_int8=True),
    dict(d=128, G=2, Hkv=3, ctx=[77], v_int8=True),
]


@pytest.mark.parametrize("case", KV_CASES, ids=lambda c: f"d{c['d']}_Hkv{c['Hkv']}_{'i8' if c['v_int8'] else 'bf16'}V")
def test_write_kv_cache_bit_exact(qa, case):
    say(f"write_kv_cache {case}")
    spec = PagedSpec("kv", 61, len(case["ctx"]), case["G"] * case["Hkv"], case["Hkv"], case["d"], case["ctx"],
                     [1] * len(case["ctx"]), k_bias_std=2.0, v_int8=case["v_int8"], pool_blocks=64)
    inp = paged_inputs(spec)
    slots = inp.slot_mapping.copy()
    slots[5::7] = -1                                # skipped tokens
    inp.slot_mapping = slots
    kc, ks, vc, vs = gpu_cache(qa, inp, case["v_int8"])
    torch.cuda.synchronize()
    want = oracle_cache(inp, case["v_int8"])
    assert np.array_equal(kc.cpu().numpy(), want["k_cache"])
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), want["k_scale"].view(np.uint32))
    if case["v_int8"]:
        assert np.array_equal(vc.cpu().numpy(), want["v_cache"])
        assert np.array_equal(vs.cpu().numpy().view(np.uint32), want["v_scale"].view(np.uint32))
    else:
        assert np.array_equal(vc.cpu().view(torch.int16).numpy().view(np.uint16), want["v_cache"])


QK_CASES = [(64, 6, 1, [256]), (64, 3, 2, [1, 15, 16, 17, 33]), (128, 16, 2, [97, 40]),
            (256, 6, 4, [1000, 31]), (256, 1, 2, [64, 65]), (256, 8, 1, [4096])]


@pytest.mark.parametrize("case", QK_CASES, ids=lambda c: f"d{c[0]}_G{c[1]}_Hkv{c[2]}_n{len(c[3])}")
def test_debug_qk_int32_bit_exact(qa, case):
    d, G, Hkv, ctx = case
    say(f"debug_paged_qk_int32 {case}")
    spec = PagedSpec("qk", 71 + d, len(ctx), G * Hkv, Hkv, d, ctx, [1] * len(ctx), k_bias_std=2.0,
                     pool_blocks=sum(-(-c // 16) for c in ctx) + 5)
    inp = paged_inputs(spec)
    kc, ks, vc, vs = gpu_cache(qa, inp, False)
    q8, _ = qa.quantize_q(dev_bits(inp.q))
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    acc = qa.debug_paged_qk_int32(q8, kc, tables, lens, fill=-7).cpu().numpy()
    c = oracle_cache(inp, False)
    w8, _ = oracle.quantize_q(inp.q)
    want = oracle.paged_qk_int32(w8, c, inp.block_tables, inp.context_lens, Hkv)
    for s, n in enumerate(ctx):
        assert np.array_equal(acc[s, :, :n], want[s]), f"seq {s}"
        assert np.all(acc[s, :, n:] == -7)            # past the context: untouched


def test_int32_bound_through_gpu(qa):
    # all codes +-127 at d = 256: the printed bound 256*127*127 exactly
    say("int32 bound via debug export")
    d = 256
    k = to_bf16_bits(np.full((16, 1, d), 0.5, np.float32))
    kc, ks, vc, vs = qa.alloc_kv_cache(1, 1, d, torch.bfloat16)
    qa.write_kv_cache(dev_bits(k), dev_bits(k), torch.arange(16, dtype=torch.int64, device="cuda"), kc, ks, vc, vs)
    q = np.full((1, 2, d), 3.0, np.float32)
    q[0, 1] = -3.0
    q8, _ = qa.quantize_q(dev_bits(to_bf16_bits(q)))
    acc = qa.debug_paged_qk_int32(q8, kc, torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                                  torch.tensor([16], dtype=torch.int32, device="cuda")).cpu().numpy()
    assert np.all(acc[0, 0, :16] == 4129024) and np.all(acc[0, 1, :16] == -4129024)


DENSE_Q = [(1, 200, 200, 2, 2, 64, "f16", True), (2, 300, 257, 4, 2, 128, "f16", True),
           (1, 130, 70, 2, 1, 256, "bf16", True), (2, 129, 129, 3, 3, 128, "f16", False),
           (1, 1, 1, 1, 1, 64, "f16", True)]


@pytest.mark.parametrize("case", DENSE_Q, ids=lambda c: f"B{c[0]}_N{c[1]}x{c[2]}_H{c[3]}/{c[4]}_d{c[5]}_{c[6]}_s{int(c[7])}")
def test_sage_quantize_bit_exact(qa, case):
    B, Nq, Nk, Hq, Hkv, d, dt, smooth = case
    say(f"dense_sage_quantize {case}")
    spec = DenseSpec("dq", 81 + d, B, Hq, Hkv, Nq, Nk, d, k_bias_std=3.0, dtype=dt)
    inp = dense_inputs(spec)
    got = qa.dense_sage_quantize(dev_bits(inp.q, dt), dev_bits(inp.k, dt), smooth_k=smooth)
    torch.cuda.synchronize()
    want = oracle.sage_quantize(inp.q, inp.k, dt, smooth_k=smooth)
    for key in ("q_i8", "k_i8"):
        assert np.array_equal(got[key].cpu().numpy(), want[key]), key
    for key in ("q_scale", "k_scale", "k_mean"):
        assert np.array_equal(got[key].cpu().numpy().view(np.uint32), want[key].view(np.uint32)), key


@pytest.mark.slow
def test_sage_quantize_full_size(qa):
    spec = dense_sage()
    say(f"dense_sage_quantize full size {spec}")
    inp = dense_inputs(spec)
    got = qa.dense_sage_quantize(dev_bits(inp.q, "f16"), dev_bits(inp.k, "f16"))
    torch.cuda.synchronize()
    want = oracle.sage_quantize(inp.q, inp.k, "f16")
    for key in ("q_i8", "k_i8"):
        assert np.array_equal(got[key].cpu().numpy(), want[key]), key
    for key in ("q_scale", "k_scale", "k_mean"):
        assert np.array_equal(got[key].cpu().numpy().view(np.uint32), want[key].view(np.uint32)), key


@pytest.mark.parametrize("mk", [tiny_decode, qwen27b_decode, chunked_prefill], ids=lambda f: f.__name__)
def test_named_workload_caches_bit_exact(qa, mk):
    spec = mk()
    say(f"cache + quantize_q at full size: {spec.name}")
    inp = paged_inputs(spec)
    kc, ks, vc, vs = gpu_cache(qa, inp, spec.v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q))
    torch.cuda.synchronize()
    want = oracle_cache(inp, spec.v_int8)
    w8, wsc = oracle.quantize_q(inp.q)
    assert np.array_equal(q8.cpu().numpy(), w8) and np.array_equal(qs.cpu().numpy(), wsc)
    assert np.array_equal(kc.cpu().numpy(), want["k_cache"])
    assert np.array_equal(ks.cpu().numpy(), want["k_scale"])
    assert np.array_equal(vc.cpu().view(torch.int16).numpy().view(np.uint16), want["v_cache"])


@pytest.mark.parametrize("v_int8", [False, True])
def test_fused_producer_bit_exact(qa, v_int8):
    spec = PagedSpec("prod", 91, 2, 24, 4, 256, [300, 40], [5, 1], k_bias_std=2.0, v_int8=v_int8, pool_blocks=30)
    say(f"quantize_q_write_kv v_int8={v_int8}")
    inp = paged_inputs(spec)
    kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, 4, 256, torch.int8 if v_int8 else torch.bfloat16)
    q8, qs = qa.quantize_q_write_kv(dev_bits(inp.q), dev_bits(inp.k), dev_bits(inp.v),
                                    torch.from_numpy(inp.slot_mapping).cuda(), kc, ks, vc, vs)
    torch.cuda.synchronize()
    w8, wsc = oracle.quantize_q(inp.q)
    want = oracle_cache(inp, v_int8)
    assert np.array_equal(q8.cpu().numpy(), w8) and np.array_equal(qs.cpu().numpy(), wsc)
    assert np.array_equal(kc.cpu().numpy(), want["k_cache"])
    assert np.array_equal(ks.cpu().numpy(), want["k_scale"])
    if v_int8:
        assert np.array_equal(vc.cpu().numpy(), want["v_cache"])
        assert np.array_equal(vs.cpu().numpy(), want["v_scale"])
    else:
        assert np.array_equal(vc.cpu().view(torch.int16).numpy().view(np.uint16), want["v_cache"])


ROPE_CASES = [
    # (d, rot_dim, neox, dtype, v_int8)
    (256, 64, True, "bf16", False),     # partial rotary, as in models that rotate a quarter of the head
    (256, 256, False, "bf16", True),
    (128, 128, True, "f16", False),
    (64, 32, False, "f16", True),
    (64, 64, True, "bf16", False),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: f"d{c[0]}_rot{c[1]}_{'neox' if c[2] else 'gptj'}_{c[3]}_{'i8V' if c[4] else '16V'}")
def test_rope_producer_bit_exact(qa, case):
    """RoPE + query quantization + cache write in one launch: codes, scales
    and every cache byte equal the oracle's (rotation in fp32 with one
    rounding per operation, then the row rule)."""
    from workloads import rope_table
    d, rot, neox, dt, v_int8 = case
    say(f"rope producer {case}")
    T, Hq, Hkv, nb = 37, 6, 2, 8
    q = _q_bits(T, Hq, d, dt, 301 + d)
    k = _q_bits(T, Hkv, d, dt, 302 + d)
    v = _q_bits(T, Hkv, d, dt, 303 + d)
    rng = np.random.default_rng(d + rot)
    pos = rng.integers(0, 4096, T).astype(np.int64)
    pos[:3] = [0, 1, 4095]
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[5] = -1                                      # skipped token
    tab = rope_table(4096, rot)
    kc, ks, vc, vs = qa.alloc_kv_cache(nb, Hkv, d, torch.int8 if v_int8 else (torch.bfloat16 if dt == "bf16" else torch.float16))
    q8, qs = qa.quantize_q_write_kv(dev_bits(q, dt), dev_bits(k, dt), dev_bits(v, dt), torch.from_numpy(slots).cuda(),
                                    kc, ks, vc, vs, rope=(torch.from_numpy(pos).cuda(), torch.from_numpy(tab).cuda(),
                                                          rot, neox))
    torch.cuda.synchronize()
    w8, wsc = oracle.rope_quantize_q(q, dt, pos, tab, rot, neox)
    assert np.array_equal(q8.cpu().numpy(), w8), "query codes"
    assert np.array_equal(qs.cpu().numpy(), wsc), "query scales"
    want = oracle.rope_write_kv_cache(k, v, dt, slots, nb, pos, tab, rot, neox, v_int8=v_int8)
    assert np.array_equal(kc.cpu().numpy(), want["k_cache"]), "K cache"
    assert np.array_equal(ks.cpu().numpy(), want["k_scale"]), "K scales"
    if v_int8:
        assert np.array_equal(vc.cpu().numpy(), want["v_cache"])
        assert np.array_equal(vs.cpu().numpy(), want["v_scale"])
    else:
        assert np.array_equal(vc.cpu().view(torch.int16).numpy().view(np.uint16), want["v_cache"])
