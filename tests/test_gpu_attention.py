"""GPU parity for the attention outputs against the oracle's fp64 result:
relative L2 <= 1e-3 and max abs <= 2e-3 (fp32 output). Decode (split and
unsplit, bf16 and INT8 V), chunked prefill and dense SageAttention-style."""
import numpy as np
import pytest
import torch

import oracle
from workloads import (PagedSpec, DenseSpec, VarlenSpec, paged_inputs, dense_inputs, dense_zero_scale_inputs,
                       varlen_inputs, tiny_decode, qwen27b_decode, batched_splitk_decode, chunked_prefill, dense_sage)
from tests.gpu_helpers import say, dev_bits, gpu_cache, oracle_cache, assert_close, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import quantized_attention_quantize_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _decode_run(qa, inp, splits, out_dtype=torch.float32, seqs=None):
    spec = inp.spec
    kc, ks, vc, vs = gpu_cache(qa, inp, spec.v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q, spec.dtype))
    out = qa.paged_attention_decode(q8, qs, kc, ks, vc, vs, torch.from_numpy(inp.block_tables).cuda(),
                                    torch.from_numpy(inp.context_lens).cuda(), num_splits=splits,
                                    out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def _decode_oracle(inp, heads=None, seqs=None):
    spec = inp.spec
    c = oracle_cache(inp, spec.v_int8)
    w8, ws = oracle.quantize_q(inp.q, spec.dtype)
    lens = inp.context_lens.copy()
    if seqs is not None:
        lens = np.where(np.isin(np.arange(len(lens)), seqs), lens, 0)
    return oracle.paged_decode(w8, ws, c, inp.block_tables, lens, spec.num_kv_heads, heads=heads)


DECODE = [
    # (d, G, Hkv, contexts, v_int8)
    (64, 6, 1, [256], False),
    (64, 1, 2, [1, 15, 16, 17], False),
    (128, 2, 2, [97, 300], True),
    (128, 8, 1, [1000], False),
    (256, 6, 4, [17, 1024, 555], False),
    (256, 6, 4, [1, 2049, 64], True),
    (256, 16, 1, [700], True),
    (64, 6, 2, [0, 40], False),
]


@pytest.mark.parametrize("splits", [1, 3, 8, 0])
@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"d{c[0]}_G{c[1]}_Hkv{c[2]}_{'i8V' if c[4] else 'bf16V'}_{'-'.join(map(str, c[3]))}")
def test_decode_parity(qa, case, splits):
    d, G, Hkv, ctx, v_int8 = case
    say(f"decode {case} splits={splits}")
    spec = PagedSpec("dec", 101 + d + G, len(ctx), G * Hkv, Hkv, d, ctx, [1] * len(ctx), k_bias_std=2.0,
                     v_int8=v_int8, pool_blocks=sum(-(-c // 16) for c in ctx) + 3)
    inp = paged_inputs(spec)
    got = _decode_run(qa, inp, splits).cpu().numpy()
    want = _decode_oracle(inp)
    assert_close(got, want, f"decode splits={splits}")
    for s, c in enumerate(ctx):
        if c == 0:
            assert np.all(got[s] == 0)


def test_decode_tiny_full(qa):
    spec = tiny_decode()
    say(f"decode full size {spec.name}")
    inp = paged_inputs(spec)
    want = _decode_oracle(inp)
    for splits in (1, 2, 0):
        assert_close(_decode_run(qa, inp, splits).cpu().numpy(), want, f"{spec.name} splits={splits}")


def test_decode_qwen27b_full(qa):
    spec = qwen27b_decode()
    say(f"decode full size {spec.name}")
    inp = paged_inputs(spec)
    want = _decode_oracle(inp)
    for splits in (0, 1, 16):
        got = _decode_run(qa, inp, splits).cpu().numpy()
        assert_close(got, want, f"{spec.name} splits={splits}")
    # reported: error of the quantized method against unquantized fp64 attention
    widen = oracle.widen
    q = widen(inp.q, "bf16").astype(np.float64)[0]
    k = widen(inp.k, "bf16").astype(np.float64)
    v = widen(inp.v, "bf16").astype(np.float64)
    ref = np.stack([oracle.attention_fp64(q[h:h + 1], k[:, h // 6], v[:, h // 6], 1 / 16.0)[0] for h in range(24)])
    say(f"  vs unquantized fp64: rel_l2={rel_l2(got[0], ref):.3e}")


def test_decode_batched_splitk_full(qa):
    spec = batched_splitk_decode()
    say(f"decode full size {spec.name}: contexts {spec.context_lens[:6]}...")
    inp = paged_inputs(spec)
    got = _decode_run(qa, inp, spec.num_splits).cpu().numpy()
    sample = [0, 7, int(np.argmax(spec.context_lens)), int(np.argmin(spec.context_lens)), 31]
    want = _decode_oracle(inp, seqs=sample)
    assert_close(got[sample], want[sample], f"{spec.name} sampled seqs {sample}")


def test_decode_bf16_output(qa):
    spec = PagedSpec("dec_bf16", 5, 2, 12, 2, 128, [333, 64], [1, 1], k_bias_std=2.0, pool_blocks=30)
    say("decode bf16 output")
    inp = paged_inputs(spec)
    got = _decode_run(qa, inp, 4, torch.bfloat16).float().cpu().numpy()
    want = _decode_oracle(inp)
    ulp = np.abs(want) * 2.0 ** -8
    assert np.all(np.abs(got - want) <= ulp + 2e-4)


def test_decode_deterministic(qa):
    spec = PagedSpec("det", 9, 3, 24, 4, 256, [4000, 100, 2500], [1, 1, 1], k_bias_std=2.0, v_int8=True)
    say("decode determinism")
    inp = paged_inputs(spec)
    a = _decode_run(qa, inp, 8)
    b = _decode_run(qa, inp, 8)
    assert torch.equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("v_int8,splits", [(False, 8), (True, 5), (False, 1)])
def test_decode_phases_match_single_call(qa, v_int8, splits):
    """_partials then _combine equals the single decode call bit for bit."""
    spec = PagedSpec("phases", 10, 3, 24, 4, 256, [3000, 17, 1600], [1, 1, 1], k_bias_std=2.0, v_int8=v_int8)
    say(f"decode phases v_int8={v_int8} splits={splits}")
    inp = paged_inputs(spec)
    kc, ks, vc, vs = gpu_cache(qa, inp, v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q, spec.dtype))
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    whole = qa.paged_attention_decode(q8, qs, kc, ks, vc, vs, tables, lens, num_splits=splits)
    out, ws, p = qa.paged_attention_decode_partials(q8, qs, kc, ks, vc, vs, tables, lens, num_splits=splits)
    qa.paged_attention_decode_combine(p, ws, out)
    torch.cuda.synchronize()
    assert torch.equal(whole, out)


STEP_CASES = [
    # (v_int8, splits, context lens, dtype)
    (False, 8, [3000, 17, 1600], "bf16"),
    (False, 0, [4096, 32, 1], "bf16"),
    (False, 1, [700, 33], "bf16"),
    (True, 5, [3000, 17, 1600], "bf16"),
    (True, 0, [257, 2048], "f16"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", STEP_CASES)
def test_decode_step_matches_producer_then_decode(qa, case):
    """qa_paged_decode_step == qa_quantize_q_write_kv + qa_paged_attention_decode,
    bit for bit: output and every cache byte."""
    v_int8, splits, ctx, dt = case
    spec = PagedSpec("step", 12, len(ctx), 24, 4, 256, ctx, [1] * len(ctx), k_bias_std=2.0, v_int8=v_int8,
                     dtype=dt)
    say(f"decode step {case}")
    inp = paged_inputs(spec)
    last = inp.cu_seqlens_kv[1:] - 1                      # each sequence's new token
    hist = inp.slot_mapping.copy()
    hist[last] = -1
    kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, 4, 256, torch.int8 if v_int8 else torch.bfloat16)
    qa.write_kv_cache(dev_bits(inp.k, dt), dev_bits(inp.v, dt), torch.from_numpy(hist).cuda(), kc, ks, vc, vs)
    q = dev_bits(inp.q, dt)
    k_new, v_new = dev_bits(inp.k[last], dt), dev_bits(inp.v[last], dt)
    slots = torch.from_numpy(inp.slot_mapping[last].copy()).cuda()
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    c1 = [t if t is None else t.clone() for t in (kc, ks, vc, vs)]
    c2 = [t if t is None else t.clone() for t in (kc, ks, vc, vs)]
    q8, qs = qa.quantize_q_write_kv(q, k_new, v_new, slots, *c1)
    ref = qa.paged_attention_decode(q8, qs, *c1, tables, lens, num_splits=splits)
    got = qa.paged_decode_step(q, k_new, v_new, slots, *c2, tables, lens, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for a, b in zip(c1, c2):
        assert a is b is None or torch.equal(a, b)


ROPE_STEP_CASES = [
    # (v_int8, splits, context lens, dtype, rot_dim, neox)
    (False, 8, [3000, 17, 1600], "bf16", 64, True),
    (True, 0, [257, 2048], "f16", 256, False),
    (False, 1, [700, 33], "bf16", 128, True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", ROPE_STEP_CASES)
def test_decode_step_rope(qa, case):
    """The step with rotary embedding (rotation, quantization, cache write
    and attention in the split kernel) equals the rotary producer followed
    by the decode call bit for bit (output and cache bytes), and the oracle
    (rotate, quantize, write, decode) within tolerance."""
    from workloads import rope_table
    v_int8, splits, ctx, dt, rot, neox = case
    spec = PagedSpec("step_rope", 14, len(ctx), 24, 4, 256, ctx, [1] * len(ctx), k_bias_std=2.0, v_int8=v_int8,
                     dtype=dt)
    say(f"decode step rope {case}")
    inp = paged_inputs(spec)
    last = inp.cu_seqlens_kv[1:] - 1
    hist = inp.slot_mapping.copy()
    hist[last] = -1
    kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, 4, 256, torch.int8 if v_int8 else torch.bfloat16)
    qa.write_kv_cache(dev_bits(inp.k, dt), dev_bits(inp.v, dt), torch.from_numpy(hist).cuda(), kc, ks, vc, vs)
    q = dev_bits(inp.q, dt)
    k_new, v_new = dev_bits(inp.k[last], dt), dev_bits(inp.v[last], dt)
    slots = torch.from_numpy(inp.slot_mapping[last].copy()).cuda()
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    pos = (inp.context_lens - 1).astype(np.int64)
    tab = rope_table(4096, rot)
    rope = (torch.from_numpy(pos).cuda(), torch.from_numpy(tab).cuda(), rot, neox)
    c1 = [t if t is None else t.clone() for t in (kc, ks, vc, vs)]
    c2 = [t if t is None else t.clone() for t in (kc, ks, vc, vs)]
    q8, qs = qa.quantize_q_write_kv(q, k_new, v_new, slots, *c1, rope=rope)
    ref = qa.paged_attention_decode(q8, qs, *c1, tables, lens, num_splits=splits)
    got = qa.paged_decode_step(q, k_new, v_new, slots, *c2, tables, lens, num_splits=splits, rope=rope)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for a, b in zip(c1, c2):
        assert a is b is None or torch.equal(a, b)
    caches = oracle.write_kv_cache(inp.k, inp.v, dt, hist, spec.num_blocks, v_int8=v_int8)
    caches = oracle.rope_write_kv_cache(inp.k[last], inp.v[last], dt, inp.slot_mapping[last], spec.num_blocks, pos, tab,
                                        rot, neox, v_int8=v_int8, caches=caches)
    w8, wsc = oracle.rope_quantize_q(inp.q, dt, pos, tab, rot, neox)
    assert np.array_equal(q8.cpu().numpy(), w8)
    want = oracle.paged_decode(w8, wsc, caches, inp.block_tables, inp.context_lens, 4)
    assert_close(got.cpu().numpy(), want, "decode step rope")


@pytest.mark.gpu
def test_decode_step_unwritten_slot(qa):
    """A negative slot writes nothing; both paths then read the cached value."""
    spec = PagedSpec("step_neg", 13, 2, 24, 4, 256, [900, 40], [1, 1], k_bias_std=2.0)
    inp = paged_inputs(spec)
    last = inp.cu_seqlens_kv[1:] - 1
    kc, ks, vc, vs = gpu_cache(qa, inp, False)          # every token, the new ones included
    q = dev_bits(inp.q)
    k_new = torch.zeros((2, 4, 256), dtype=torch.bfloat16, device="cuda")   # must not be used
    slots = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    before = [t if t is None else t.clone() for t in (kc, ks, vc, vs)]
    q8, qs = qa.quantize_q(q)
    ref = qa.paged_attention_decode(q8, qs, kc, ks, vc, vs, tables, lens, num_splits=4)
    got = qa.paged_decode_step(q, k_new, k_new, slots, kc, ks, vc, vs, tables, lens, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for a, b in zip(before, (kc, ks, vc, vs)):
        assert a is b is None or torch.equal(a, b)


# ---------------------------------------------------------------------------
# multi-token decode (T new query tokens per sequence in the decode kernel)
# ---------------------------------------------------------------------------

MT_CASES = [
    # (d, G, Hkv, T, contexts, v_int8, splits)
    (256, 6, 4, 2, [3000, 17, 1600], False, 0),
    (256, 6, 2, 2, [500, 2], True, 8),
    (128, 4, 2, 4, [700, 33], False, 3),
    (64, 1, 2, 16, [300, 16, 5], False, 0),     # context 5 < 16 tokens: early tokens see nothing
    (64, 8, 1, 2, [129], True, 1),              # one split: the kernel writes the output
    (128, 16, 1, 1, [640], False, 0),
]


def _mt_run(qa, inp, T, splits):
    spec = inp.spec
    kc, ks, vc, vs = gpu_cache(qa, inp, spec.v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q, spec.dtype))
    S, Hq, d = spec.num_seqs, spec.num_q_heads, spec.head_dim
    out = qa.paged_attention_decode_mt(q8.view(S, T, Hq, d), qs.view(S, T, Hq), kc, ks, vc, vs,
                                       torch.from_numpy(inp.block_tables).cuda(),
                                       torch.from_numpy(inp.context_lens).cuda(), num_splits=splits)
    torch.cuda.synchronize()
    return out, (q8, qs, kc, ks, vc, vs)


@pytest.mark.parametrize("case", MT_CASES, ids=lambda c: f"d{c[0]}_G{c[1]}_Hkv{c[2]}_T{c[3]}_{'i8V' if c[5] else 'bf16V'}_S{c[6]}")
def test_decode_mt_parity(qa, case):
    d, G, Hkv, T, ctx, v_int8, splits = case
    say(f"multi-token decode {case}")
    spec = PagedSpec("mt", 501 + d + G + T, len(ctx), G * Hkv, Hkv, d, ctx, [T] * len(ctx), k_bias_std=2.0,
                     v_int8=v_int8, pool_blocks=sum(-(-c // 16) for c in ctx) + 4)
    inp = paged_inputs(spec)
    got, _ = _mt_run(qa, inp, T, splits)
    want = _prefill_oracle(inp).reshape(got.shape)
    assert_close(got.cpu().numpy(), want, "multi-token decode")


def test_decode_mt_one_token_is_decode(qa):
    """T = 1 gives qa_paged_attention_decode's result bit for bit."""
    spec = PagedSpec("mt1", 77, 3, 24, 4, 256, [1500, 40, 999], [1, 1, 1], k_bias_std=2.0)
    inp = paged_inputs(spec)
    got, (q8, qs, kc, ks, vc, vs) = _mt_run(qa, inp, 1, 0)
    ref = qa.paged_attention_decode(q8, qs, kc, ks, vc, vs, torch.from_numpy(inp.block_tables).cuda(),
                                    torch.from_numpy(inp.context_lens).cuda())
    torch.cuda.synchronize()
    assert torch.equal(got.view(ref.shape), ref)


# ---------------------------------------------------------------------------
# chunked prefill
# ---------------------------------------------------------------------------

def _prefill_run(qa, inp, out_dtype=torch.float32):
    spec = inp.spec
    kc, ks, vc, vs = gpu_cache(qa, inp, spec.v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q, spec.dtype))
    out = qa.chunked_prefill_attention(q8, qs, torch.from_numpy(inp.cu_seqlens_q).cuda(),
                                       torch.from_numpy(inp.context_lens).cuda(), kc, ks, vc, vs,
                                       torch.from_numpy(inp.block_tables).cuda(), max(spec.query_lens),
                                       out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def _prefill_oracle(inp, rows=None, heads=None):
    spec = inp.spec
    c = oracle_cache(inp, spec.v_int8)
    w8, ws = oracle.quantize_q(inp.q, spec.dtype)
    return oracle.chunked_prefill(w8, ws, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables,
                                  spec.num_kv_heads, rows=rows, heads=heads)


PREFILL = [
    # (d, G, Hkv, contexts, query_lens, v_int8)
    (64, 6, 1, [50, 37], [20, 37], False),
    (64, 1, 2, [1, 17, 300], [1, 5, 130], False),
    (128, 2, 2, [257, 129], [200, 129], True),
    (256, 6, 4, [600], [260], False),
    (256, 6, 2, [140, 33], [140, 1], True),
    (256, 3, 1, [100], [0], False),
    # workgroups of packed (token, head) rows that start and end inside a token
    (256, 5, 1, [300, 90], [250, 7], False),
    (128, 3, 2, [190, 64], [190, 50], False),
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: f"d{c[0]}_G{c[1]}_Hkv{c[2]}_{'i8V' if c[5] else 'bf16V'}_{'-'.join(map(str, c[3]))}")
def test_prefill_parity(qa, case):
    d, G, Hkv, ctx, ql, v_int8 = case
    say(f"prefill {case}")
    spec = PagedSpec("pf", 201 + d + G, len(ctx), G * Hkv, Hkv, d, ctx, ql, k_bias_std=2.0, v_int8=v_int8,
                     pool_blocks=sum(-(-c // 16) for c in ctx) + 4)
    inp = paged_inputs(spec)
    if spec.total_q == 0:
        return
    got = _prefill_run(qa, inp).cpu().numpy()
    assert_close(got, _prefill_oracle(inp), "prefill")


def test_prefill_full_size_sampled(qa):
    spec = chunked_prefill()
    say(f"prefill full size {spec.name}")
    inp = paged_inputs(spec)
    got = _prefill_run(qa, inp).cpu().numpy()
    rows = [0, 1, 127, 128, 1000, 1500, 2046, 2047]
    want = _prefill_oracle(inp, rows=rows)
    assert_close(got[rows], want[rows], f"{spec.name} rows {rows}")


# chunked prefill with V converted once into a workspace: the same output as
# the plain entry bit for bit (a workspace full of NaN bytes beforehand, so a
# read of any unwritten byte would show), the oracle's within tolerance, and
# the workspace holding each context's V rounded to fp16


def _prefill_ws_run(qa, inp, out_dtype=torch.float32):
    spec = inp.spec
    kc, ks, vc, vs = gpu_cache(qa, inp, spec.v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q, spec.dtype))
    args = (q8, qs, torch.from_numpy(inp.cu_seqlens_q).cuda(), torch.from_numpy(inp.context_lens).cuda(), kc, ks,
            vc, vs, torch.from_numpy(inp.block_tables).cuda(), max(spec.query_lens))
    p = qa.prefill_params(q8, args[3], kc, vc, args[8], args[9], out_dtype=out_dtype)
    ws = qa.chunked_prefill_ws_workspace(p)
    assert ws.numel() == spec.num_seqs * inp.block_tables.shape[1] * spec.num_kv_heads * spec.head_dim * 32
    ws.fill_(0xFF)
    got = qa.chunked_prefill_attention_ws(*args, out_dtype=out_dtype, workspace=ws)
    plain = qa.chunked_prefill_attention(*args, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return got, plain, ws, vc, vs


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: f"d{c[0]}_G{c[1]}_Hkv{c[2]}_{'i8V' if c[5] else 'bf16V'}_{'-'.join(map(str, c[3]))}")
def test_prefill_ws_parity(qa, case):
    d, G, Hkv, ctx, ql, v_int8 = case
    say(f"prefill ws {case}")
    spec = PagedSpec("pfw", 201 + d + G, len(ctx), G * Hkv, Hkv, d, ctx, ql, k_bias_std=2.0, v_int8=v_int8,
                     pool_blocks=sum(-(-c // 16) for c in ctx) + 4)
    inp = paged_inputs(spec)
    if spec.total_q == 0:
        return
    got, plain, ws, vc, _ = _prefill_ws_run(qa, inp)
    assert torch.equal(got, plain)
    assert_close(got.cpu().numpy(), _prefill_oracle(inp), "prefill ws")
    # the workspace: V of every block of the context, fp16 [seq, block, Hkv, d, 16]
    nb = inp.block_tables.shape[1]
    w = ws.view(torch.float16).view(spec.num_seqs, nb, Hkv, d, 16).cpu()
    vcache = vc.cpu().float() if not v_int8 else vc.cpu().to(torch.float32)
    for s_, c in enumerate(ctx):
        for j in range(-(-c // 16)):
            want = vcache[int(inp.block_tables[s_, j])].to(torch.float16).clone()
            n_in = min(16, c - 16 * j)
            want[..., n_in:] = 0
            assert torch.equal(w[s_, j], want), (s_, j)


def test_prefill_ws_bf16_output(qa):
    spec = PagedSpec("pfwb", 77, 2, 12, 2, 128, [333, 70], [160, 70], k_bias_std=2.0, pool_blocks=40)
    got, plain, _, _, _ = _prefill_ws_run(qa, paged_inputs(spec), out_dtype=torch.bfloat16)
    assert torch.equal(got, plain)


def test_prefill_ws_full_size(qa):
    spec = chunked_prefill()
    say(f"prefill ws full size {spec.name}")
    inp = paged_inputs(spec)
    got, plain, _, _, _ = _prefill_ws_run(qa, inp)
    assert torch.equal(got, plain)
    rows = [0, 2047]
    want = _prefill_oracle(inp, rows=rows)
    assert_close(got.cpu().numpy()[rows], want[rows], f"{spec.name} ws rows {rows}")


# ---------------------------------------------------------------------------
# chunked prefill with the P.V product in FP8 (E4M3): the tolerance model of
# the dense FP8 path below (sigma of the difference to the plain definition),
# and the E4M3 V codes and channel scales the call leaves in its workspace,
# bit-exact against the oracle's
# ---------------------------------------------------------------------------

def _prefill_fp8_run(qa, inp, out_dtype=torch.float32):
    spec = inp.spec
    kc, ks, vc, vs = gpu_cache(qa, inp, spec.v_int8)
    q8, qs = qa.quantize_q(dev_bits(inp.q, spec.dtype))
    tables = torch.from_numpy(inp.block_tables).cuda()
    ctx = torch.from_numpy(inp.context_lens).cuda()
    p = qa.prefill_params(q8, ctx, kc, vc, tables, max(spec.query_lens), out_dtype=out_dtype)
    ws = qa.chunked_prefill_fp8pv_workspace(p)
    out = qa.chunked_prefill_attention_fp8pv(q8, qs, torch.from_numpy(inp.cu_seqlens_q).cuda(), ctx, kc, ks, vc, vs,
                                             tables, max(spec.query_lens), out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out, ws


def _prefill_fp8_oracle(inp, rows=None):
    spec = inp.spec
    c = oracle_cache(inp, spec.v_int8)
    w8, wsc = oracle.quantize_q(inp.q, spec.dtype)
    return oracle.chunked_prefill_fp8pv(w8, wsc, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables,
                                        spec.num_kv_heads, rows=rows, return_sigma=True)


def _fp8_workspace_values(ws, spec, inp_blocks):
    """E4M3 values [S, T*128, Hkv, d] and scales [S, Hkv, d] from the
    workspace layout of qa_chunked_prefill_attention_fp8pv (inp_blocks: the
    block-table width, max_blocks_per_seq)."""
    S, Hkv, d = spec.num_seqs, spec.num_kv_heads, spec.head_dim
    T = -(-inp_blocks * 16 // 128)
    raw = ws.cpu().numpy()
    nv8 = S * T * Hkv * 128 * d
    v8 = raw[:nv8].reshape(S, T, Hkv, 4, d, 32)
    key = np.arange(128)
    ch = np.arange(d)
    j, h, e = key // 32, (key % 32) // 16, key % 16
    byte = 16 * (h[:, None] ^ ((ch[None, :] >> 3) & 1)) + e[:, None]        # [128, d]
    codes = v8[:, :, :, j[:, None], ch[None, :], byte]                         # [S, T, Hkv, 128, d]
    codes = codes.transpose(0, 1, 3, 2, 4).reshape(S, T * 128, Hkv, d)
    off = -(-nv8 // 256) * 256
    sc = raw[off:off + S * Hkv * d * 4].view(np.float32).reshape(S, Hkv, d)
    return oracle.e4m3_decode(codes), sc


PREFILL_FP8 = PREFILL + [
    # several 128-key tiles with a ragged tail, history plus a chunk
    (256, 6, 2, [1000], [300], False),
    (256, 6, 1, [385, 129], [128, 129], True),
]


@pytest.mark.parametrize("case", PREFILL_FP8, ids=lambda c: f"d{c[0]}_G{c[1]}_Hkv{c[2]}_{'i8V' if c[5] else 'bf16V'}_{'-'.join(map(str, c[3]))}")
def test_prefill_fp8pv_parity(qa, case):
    d, G, Hkv, ctx, ql, v_int8 = case
    say(f"prefill fp8 P.V {case}")
    spec = PagedSpec("pf8", 231 + d + G, len(ctx), G * Hkv, Hkv, d, ctx, ql, k_bias_std=2.0, v_int8=v_int8,
                     pool_blocks=sum(-(-c // 16) for c in ctx) + 4)
    inp = paged_inputs(spec)
    if spec.total_q == 0:
        return
    got, ws = _prefill_fp8_run(qa, inp)
    want, sig = _prefill_fp8_oracle(inp)
    _fp8_close(got.cpu().numpy(), want, sig, "prefill fp8 P.V vs oracle")
    # the workspace: E4M3 V values and channel scales of every (sequence, KV head)
    vals, sc = _fp8_workspace_values(ws, spec, inp.block_tables.shape[1])
    c = oracle_cache(inp, v_int8)
    for s_, n in enumerate(ctx):
        for h in range(Hkv):
            codes, wsc = oracle.paged_v_fp8(c, inp.block_tables, s_, n, h, len(ctx), Hkv, d)
            if n > 0:
                np.testing.assert_array_equal(sc[s_, h], wsc)
            np.testing.assert_array_equal(vals[s_, :n, h], oracle.e4m3_decode(codes))
            tail = -(-n // 128) * 128
            assert np.all(vals[s_, n:tail, h] == 0)


def test_prefill_fp8pv_bf16_output(qa):
    spec = PagedSpec("pf8b", 241, 1, 12, 2, 128, [300], [100], k_bias_std=2.0)
    inp = paged_inputs(spec)
    got, _ = _prefill_fp8_run(qa, inp, out_dtype=torch.bfloat16)
    want, sig = _prefill_fp8_oracle(inp)
    g = got.float().cpu().numpy()
    # bf16 output: the rounding (2^-9 relative) joins the E4M3 deviation
    _fp8_close(g, want, np.sqrt(sig ** 2 + (np.abs(want) * 2.0 ** -9) ** 2), "prefill fp8 P.V bf16 out")


def test_prefill_fp8pv_full_size_sampled(qa):
    spec = chunked_prefill()
    say(f"prefill fp8 P.V full size {spec.name}")
    inp = paged_inputs(spec)
    got, _ = _prefill_fp8_run(qa, inp)
    rows = [0, 1, 127, 128, 1000, 1500, 2046, 2047]
    want, sig = _prefill_fp8_oracle(inp, rows=rows)
    _fp8_close(got.cpu().numpy()[rows], want[rows], sig[rows], f"{spec.name} fp8 P.V rows {rows}")
    ref = _prefill_oracle(inp, rows=rows)
    say(f"  fp8 P.V vs 16-bit P definition: rel_l2={rel_l2(got.cpu().numpy()[rows], ref[rows]):.3e}")


# ---------------------------------------------------------------------------
# dense SageAttention-style
# ---------------------------------------------------------------------------

DENSE = [
    # (B, Nq, Nk, Hq, Hkv, d, dtype, causal)
    (1, 200, 200, 2, 2, 64, "f16", False),
    (1, 200, 200, 2, 2, 64, "f16", True),
    (2, 300, 257, 4, 2, 128, "f16", True),
    (2, 129, 400, 2, 2, 128, "bf16", False),
    (1, 256, 256, 2, 1, 256, "f16", True),
    (1, 1, 1, 1, 1, 64, "f16", False),
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: f"B{c[0]}_{c[1]}x{c[2]}_H{c[3]}/{c[4]}_d{c[5]}_{c[6]}_{'causal' if c[7] else 'full'}")
def test_dense_parity(qa, case):
    B, Nq, Nk, Hq, Hkv, d, dt, causal = case
    say(f"dense {case}")
    spec = DenseSpec("dn", 301 + d, B, Hq, Hkv, Nq, Nk, d, k_bias_std=3.0, dtype=dt)
    inp = dense_inputs(spec)
    got = qa.dense_sage_attention(dev_bits(inp.q, dt), dev_bits(inp.k, dt), dev_bits(inp.v, dt),
                                  is_causal=causal).cpu().numpy()
    quant = oracle.sage_quantize(inp.q, inp.k, dt)
    want = oracle.dense_sage_attention(quant, inp.v, dt, causal=causal)
    assert_close(got, want, "dense")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_zero_scales(qa, causal, dt):
    """Zero key-block scales (constant keys) and a zero query block: finite
    output equal to the oracle's (uniform attention for those rows)."""
    say(f"dense zero scales causal={causal} {dt}")
    inp = dense_zero_scale_inputs(N=300, d=128, dtype=dt)
    got = qa.dense_sage_attention(dev_bits(inp.q, dt), dev_bits(inp.k, dt), dev_bits(inp.v, dt),
                                  is_causal=causal).cpu().numpy()
    assert np.all(np.isfinite(got))
    want = oracle.dense_sage_attention(oracle.sage_quantize(inp.q, inp.k, dt), inp.v, dt, causal=causal)
    assert_close(got, want, "dense zero scales")


@pytest.mark.parametrize("scale", [1.5, 12.0])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_large_magnitude(qa, causal, scale):
    """Q and K scaled up so that the per-tile score factor crosses (1.5) or
    far exceeds (12) the bound under which the kernel folds its accumulator
    offset into the exponent's constant; both ways must match the oracle."""
    say(f"dense large magnitude scale={scale} causal={causal}")
    spec = DenseSpec("dn_big", 407, 1, 2, 2, 300, 300, 128, k_bias_std=3.0, dtype="f16")
    inp = dense_inputs(spec)

    def scaled(bits):
        return (bits.view(np.float16).astype(np.float32) * scale).astype(np.float16).view(np.uint16)
    q, k = scaled(inp.q), scaled(inp.k)
    got = qa.dense_sage_attention(dev_bits(q, "f16"), dev_bits(k, "f16"), dev_bits(inp.v, "f16"),
                                  is_causal=causal).cpu().numpy()
    want = oracle.dense_sage_attention(oracle.sage_quantize(q, k, "f16"), inp.v, "f16", causal=causal)
    assert_close(got, want, f"dense x{scale}")


@pytest.mark.parametrize("causal", [False, True])
def test_dense_full_size_sampled(qa, causal):
    spec = dense_sage()
    say(f"dense full size {spec.name} causal={causal}")
    inp = dense_inputs(spec)
    got = qa.dense_sage_attention(dev_bits(inp.q, "f16"), dev_bits(inp.k, "f16"), dev_bits(inp.v, "f16"),
                                  is_causal=causal)
    torch.cuda.synchronize()
    quant = oracle.sage_quantize(inp.q, inp.k, "f16")
    rows = np.array([0, 1, 127, 128, 4095, 8191])
    want = oracle.dense_sage_attention(quant, inp.v, "f16", causal=causal, rows=rows, heads=[0, 17, 31])
    g = got.cpu().numpy()
    for b in range(2):
        for h in (0, 17, 31):
            assert_close(g[b, rows, h], want[b, rows, h], f"dense b={b} h={h}")


# the dense call with its options: HND layout, smooth_v, LSE output
DENSE_EX = [
    # (B, Nq, Nk, Hq, Hkv, d, dtype, causal)
    (1, 200, 200, 2, 2, 64, "f16", False),
    (2, 300, 257, 4, 2, 128, "bf16", True),      # causal with Nq > Nk: 43 rows see no key
    (1, 129, 400, 6, 1, 256, "f16", True),
    (2, 77, 150, 4, 4, 128, "f16", False),
]


def _lse_close(got, want, what):
    dead = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), dead), f"{what}: rows without keys differ"
    err = np.abs(got[~dead] - want[~dead])
    assert err.size == 0 or err.max() <= 1e-3 * max(1.0, np.abs(want[~dead]).max()), \
        f"{what}: LSE error {err.max():.3g}"


@pytest.mark.parametrize("smooth_k", [True, False])
@pytest.mark.parametrize("smooth_v", [True, False])
@pytest.mark.parametrize("case", DENSE_EX, ids=lambda c: f"B{c[0]}_{c[1]}x{c[2]}_H{c[3]}/{c[4]}_d{c[5]}_{c[6]}_{'causal' if c[7] else 'full'}")
def test_dense_options_parity(qa, case, smooth_v, smooth_k):
    """Output and LSE of the options call against the oracle's whole dense
    forward, in both layouts; the HND result must be the NHD one transposed,
    bit for bit (same arithmetic, other strides)."""
    B, Nq, Nk, Hq, Hkv, d, dt, causal = case
    say(f"dense options {case} smooth_v={smooth_v} smooth_k={smooth_k}")
    spec = DenseSpec("dn_ex", 509 + d, B, Hq, Hkv, Nq, Nk, d, k_bias_std=3.0, dtype=dt, v_bias_std=2.0)
    inp = dense_inputs(spec)
    q, k, v = dev_bits(inp.q, dt), dev_bits(inp.k, dt), dev_bits(inp.v, dt)
    out_n, lse_n = qa.dense_sage_attention_ex(q, k, v, "NHD", is_causal=causal, smooth_k=smooth_k,
                                              smooth_v=smooth_v, return_lse=True)
    hnd = lambda t: t.transpose(1, 2).contiguous()
    out_h, lse_h = qa.dense_sage_attention_ex(hnd(q), hnd(k), hnd(v), "HND", is_causal=causal,
                                              smooth_k=smooth_k, smooth_v=smooth_v, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_h.transpose(1, 2), out_n), "HND output differs from NHD"
    assert torch.equal(lse_h, lse_n), "HND LSE differs from NHD"
    want, want_lse = oracle.sage_forward(inp.q, inp.k, inp.v, dt, causal=causal, smooth_k=smooth_k,
                                         smooth_v=smooth_v, return_lse=True)
    assert_close(out_n.cpu().numpy(), want, "dense options")
    _lse_close(lse_n.cpu().numpy(), want_lse, "dense options LSE")
    if not smooth_v:   # the plain call is the options call without options
        plain = qa.dense_sage_attention(q, k, v, is_causal=causal, smooth_k=smooth_k)
        assert torch.equal(plain, out_n)


@pytest.mark.parametrize("pv_fp8", [False, True])
@pytest.mark.parametrize("case", [(2, 300, 257, 4, 2, 128, "bf16", True), (1, 200, 333, 2, 2, 64, "f16", False),
                                  (1, 129, 400, 6, 1, 256, "f16", True), (2, 1, 70, 2, 1, 128, "bf16", False)],
                         ids=lambda c: f"B{c[0]}_{c[1]}x{c[2]}_H{c[3]}/{c[4]}_d{c[5]}_{c[6]}_{'causal' if c[7] else 'full'}")
def test_dense_query_blocks_in_kernel(qa, case, pv_fp8):
    """The attention kernel quantizes its 128-row query blocks itself, except
    when the smooth_k LSE correction asks for the separate query pass (whose
    codes the preprocessing tests pin to the oracle's bit for bit); the LSE
    output changes nothing else, so both calls give the same output bit for
    bit."""
    B, Nq, Nk, Hq, Hkv, d, dt, causal = case
    if pv_fp8 and d > 128:
        pytest.skip("FP8 P.V: head_dim 64 or 128")
    say(f"dense query blocks in the kernel {case} pv_fp8={pv_fp8}")
    spec = DenseSpec("dn_qk", 733 + d, B, Hq, Hkv, Nq, Nk, d, k_bias_std=3.0, dtype=dt)
    inp = dense_inputs(spec)
    q, k, v = dev_bits(inp.q, dt), dev_bits(inp.k, dt), dev_bits(inp.v, dt)
    fused = qa.dense_sage_attention_ex(q, k, v, is_causal=causal, smooth_k=True, pv_fp8=pv_fp8)
    separate, _ = qa.dense_sage_attention_ex(q, k, v, is_causal=causal, smooth_k=True, pv_fp8=pv_fp8,
                                             return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(fused, separate)


def _zero_mean_v_bits(seq_lens, H, d, seed):
    """fp16 V rows k/64 (|k| <= 256) whose every sequence has channel sums of
    exactly 0 (the second half of its rows negates the first, a last odd row
    is 0): the smooth_v mean is exactly 0 in any summation order, so smooth_v
    leaves the output unchanged bit for bit."""
    rng = np.random.default_rng(seed)
    parts = []
    for L in seq_lens:
        half = rng.integers(-256, 257, size=(L // 2, H, d)) / 64.0
        rows = np.concatenate([half, -half[rng.permutation(L // 2)], np.zeros((L % 2, H, d))])
        parts.append(rows[rng.permutation(L)] if L else rows)
    return np.concatenate(parts).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("case", [(2, 200, 256, 4, 2, 128, True), (1, 130, 500, 2, 2, 64, False),
                                  (1, 129, 193, 6, 1, 256, True), (2, 64, 64, 2, 1, 128, False),
                                  (2, 70, 1, 2, 1, 64, False)],
                         ids=lambda c: f"B{c[0]}_{c[1]}x{c[2]}_H{c[3]}/{c[4]}_d{c[5]}_{'causal' if c[6] else 'full'}")
def test_dense_token_order_v(qa, case):
    """fp16 V without smooth_v: the attention kernel copies V tiles in token
    order (a partial last tile re-reads the last row, where P is 0) and forms its P.V operands with transposing LDS reads. With channel
    sums of exactly 0, the smooth_v call (which takes the V block pass: the
    same fp16 values in the other layout, mean 0) must give the same output
    bit for bit; each sequence must equal its one-sequence varlen call; and
    the output must match the oracle."""
    B, Nq, Nk, Hq, Hkv, d, causal = case
    say(f"dense token-order V {case}")
    spec = DenseSpec("dn_vt", 877 + d, B, Hq, Hkv, Nq, Nk, d, k_bias_std=3.0, dtype="f16")
    inp = dense_inputs(spec)
    vbits = _zero_mean_v_bits([Nk] * B, Hkv, d, 5 + d).reshape(B, Nk, Hkv, d)
    q, k, v = dev_bits(inp.q, "f16"), dev_bits(inp.k, "f16"), dev_bits(vbits, "f16")
    out = qa.dense_sage_attention(q, k, v, is_causal=causal)
    blocks = qa.dense_sage_attention_ex(q, k, v, is_causal=causal, smooth_v=True)
    torch.cuda.synchronize()
    assert torch.equal(out, blocks), "token-order V against the V block pass"
    for b in range(B):
        cq = torch.tensor([0, Nq], dtype=torch.int32, device="cuda")
        ck = torch.tensor([0, Nk], dtype=torch.int32, device="cuda")
        one = qa.dense_sage_attention_varlen(q[b].contiguous(), k[b].contiguous(), v[b].contiguous(), cq, ck, Nq, Nk,
                                             is_causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(one, out[b]), f"sequence {b}"
    want = oracle.sage_forward(inp.q, inp.k, vbits, "f16", causal=causal)
    assert_close(out.cpu().numpy(), want, "dense token-order V")


@pytest.mark.parametrize("case", [([200, 7, 0, 129], [256, 64, 30, 1], 4, 2, 128, True),
                                  ([65, 300], [63, 191], 2, 1, 64, False),
                                  ([33, 1, 97], [130, 5, 97], 2, 2, 256, True)],
                         ids=lambda c: f"{'-'.join(map(str, c[0]))}_on_{'-'.join(map(str, c[1]))}_H{c[2]}/{c[3]}_d{c[4]}")
def test_dense_varlen_token_order_v(qa, case):
    """Packed fp16 sequences of ragged lengths (partial last tiles, a
    sequence without queries): token-order V (each sequence's rows from its
    own offset) against the smooth_v call's V block pass on channel sums of
    exactly 0, bit for bit, and against the oracle."""
    seq_q, seq_k, Hq, Hkv, d, causal = case
    say(f"dense varlen token-order V {case}")
    spec = VarlenSpec("vl_vt", 91 + d, seq_q, seq_k, Hq, Hkv, d, dtype="f16")
    inp = varlen_inputs(spec)
    vbits = _zero_mean_v_bits(seq_k, Hkv, d, 9 + d)
    cu_q, cu_k = torch.from_numpy(inp.cu_q).cuda(), torch.from_numpy(inp.cu_k).cuda()
    q, k, v = dev_bits(inp.q, "f16"), dev_bits(inp.k, "f16"), dev_bits(vbits, "f16")
    run = lambda sv: qa.dense_sage_attention_varlen(q, k, v, cu_q, cu_k, max(seq_q), max(seq_k), is_causal=causal,
                                                    smooth_v=sv)
    out, blocks = run(False), run(True)
    torch.cuda.synchronize()
    assert torch.equal(out, blocks), "token-order V against the V block pass"
    want = oracle.sage_varlen_forward(inp.q, inp.k, vbits, inp.cu_q, inp.cu_k, "f16", causal=causal)
    assert_close(out.cpu().numpy(), want, "dense varlen token-order V")


def test_dense_options_full_size_sampled(qa):
    """The dense workload (2 x 8192 x 32 heads, d 128) through the options
    call in HND with smooth_v and the LSE, sampled rows and heads against the
    oracle's steps (quantize, smooth V, attend, add the mean back, correct
    the LSE)."""
    spec = dense_sage()
    say(f"dense options full size {spec.name}")
    inp = dense_inputs(spec)
    hnd = lambda bits: dev_bits(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)), "f16")
    out, lse = qa.dense_sage_attention_ex(hnd(inp.q), hnd(inp.k), hnd(inp.v), "HND", is_causal=True,
                                          smooth_v=True, return_lse=True)
    torch.cuda.synchronize()
    quant = oracle.sage_quantize(inp.q, inp.k, "f16")
    vb, mu = oracle.sage_smooth_v(inp.v, "f16")
    rows, heads = np.array([0, 1, 127, 128, 4095, 8191]), [0, 17, 31]
    want, want_lse = oracle.dense_sage_attention(quant, vb, "f16", causal=True, rows=rows, heads=heads,
                                                 return_lse=True)
    corr = oracle.sage_lse_correction(inp.q, quant["k_mean"], "f16")
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(2):
        for h in heads:
            assert_close(o[b, h, rows], want[b, rows, h] + mu[b, h // (spec.num_q_heads // spec.num_kv_heads)],
                         f"dense options b={b} h={h}")
            _lse_close(l[b, h, rows], want_lse[b, h, rows] + corr[b, h, rows], f"dense options LSE b={b} h={h}")


# FP8 (E4M3) P.V against the oracle's plain definition (P8 = E4M3(448
# exp(s - m)) at the exact row maximum m). The kernel rounds P from a lazily
# moved reference instead (56 exp(s - m'), m' <= m), so the two results
# differ by independent E4M3 roundings; the oracle returns the standard
# deviation sigma of that difference per element and per LSE (2^-4 relative
# per normal E4M3 value, 2^-10 absolute per subnormal one, propagated through
# the normalized sum). The bar: no element beyond 6 sigma and an RMS of
# |difference| / sigma of at most 1, with a floor for the fp32 arithmetic
# (rows that see one key have sigma 0).
FP8_MAX_Z, FP8_RMS_Z = 6.0, 1.0

FP8_CASES = [
    # (B, Nq, Nk, Hq, Hkv, d, dtype, causal, smooth_v)
    (1, 200, 200, 2, 2, 64, "f16", False, False),
    (2, 300, 257, 4, 2, 128, "bf16", True, True),
    (1, 129, 400, 6, 1, 128, "f16", True, False),
    (2, 77, 150, 4, 4, 64, "f16", False, True),
]


def _fp8_close(got, want, sig, what):
    got, want, sig = (np.asarray(x, np.float64) for x in (got, want, sig))
    floor = 2e-6 * float(np.max(np.abs(want))) + 1e-7
    z = np.abs(got - want) / np.maximum(sig, floor)
    zmax, zrms = float(np.max(z)), float(np.sqrt(np.mean(z ** 2)))
    say(f"  {what}: rel_l2={rel_l2(got, want):.3e} max|d|/sigma={zmax:.2f} rms|d|/sigma={zrms:.3f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert zmax <= FP8_MAX_Z and zrms <= FP8_RMS_Z, f"{what}: max z {zmax:.2f}, rms z {zrms:.3f}"


def _fp8_lse_close(got, want, sig, what):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    _fp8_close(got[fin], want[fin], sig[fin] + 1e-6 * np.abs(want[fin]), what)


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: f"B{c[0]}_{c[1]}x{c[2]}_H{c[3]}/{c[4]}_d{c[5]}_{c[6]}_{'causal' if c[7] else 'full'}{'_sv' if c[8] else ''}")
def test_dense_fp8pv_parity(qa, case):
    B, Nq, Nk, Hq, Hkv, d, dt, causal, smooth_v = case
    say(f"dense fp8 P.V {case}")
    spec = DenseSpec("dn_fp8", 611 + d, B, Hq, Hkv, Nq, Nk, d, k_bias_std=3.0, dtype=dt, v_bias_std=2.0)
    inp = dense_inputs(spec)
    out, lse = qa.dense_sage_attention_ex(dev_bits(inp.q, dt), dev_bits(inp.k, dt), dev_bits(inp.v, dt),
                                          is_causal=causal, smooth_v=smooth_v, return_lse=True, pv_fp8=True)
    torch.cuda.synchronize()
    quant = oracle.sage_quantize(inp.q, inp.k, dt)
    want, want_lse, sig, sig_lse = oracle.dense_sage_attention_fp8pv(quant, inp.v, dt, causal=causal,
                                                                     smooth_v=smooth_v, return_sigma=True)
    got = out.cpu().numpy()
    _fp8_close(got, want, sig, "fp8 P.V vs oracle")
    corr = oracle.sage_lse_correction(inp.q, quant["k_mean"], dt)
    _fp8_lse_close(lse.cpu().numpy().astype(np.float64), want_lse + corr, sig_lse, "fp8 P.V LSE")
    exact = oracle.sage_forward(inp.q, inp.k, inp.v, dt, causal=causal, smooth_v=smooth_v)
    r = rel_l2(got, exact)
    say(f"  fp8 P.V vs 16-bit P path: rel_l2={r:.3e}")
    assert r < 3e-2
    # reported: error against fp64 attention of the unquantized inputs
    qv, kv, vv = (oracle.widen(x, dt).astype(np.float64) for x in (inp.q, inp.k, inp.v))
    G = Hq // Hkv
    vis = (np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)) if causal else None
    ref = np.stack([np.stack([oracle.attention_fp64(qv[b, :, h], kv[b, :, h // G], vv[b, :, h // G], d ** -0.5, vis)
                              for h in range(Hq)], axis=1) for b in range(B)])
    live = np.isfinite(want_lse).transpose(0, 2, 1)[..., None]
    say(f"  fp8 P.V vs unquantized fp64 attention: rel_l2={rel_l2(np.where(live, got, 0), np.where(live, ref, 0)):.3e}")


def test_dense_fp8pv_full_size_sampled(qa):
    spec = dense_sage()
    say(f"dense fp8 P.V full size {spec.name}")
    inp = dense_inputs(spec)
    out = qa.dense_sage_attention_ex(dev_bits(inp.q, "f16"), dev_bits(inp.k, "f16"), dev_bits(inp.v, "f16"),
                                     is_causal=True, pv_fp8=True)
    torch.cuda.synchronize()
    quant = oracle.sage_quantize(inp.q, inp.k, "f16")
    rows = np.array([0, 1, 127, 128, 4095, 8191])
    want, _, sig, _ = oracle.dense_sage_attention_fp8pv(quant, inp.v, "f16", causal=True, rows=rows,
                                                        heads=[0, 17, 31], return_sigma=True)
    g = out.cpu().numpy()
    for b in range(2):
        for h in (0, 17, 31):
            _fp8_close(g[b, rows, h], want[b, rows, h], sig[b, rows, h], f"fp8 P.V b={b} h={h}")


def test_dense_fp8pv_varlen_matches_one_sequence_calls(qa):
    spec = VarlenSpec("vl8", 93, [130, 7, 300], [200, 7, 260], 4, 2, 128, dtype="bf16", v_bias_std=2.0)
    inp = varlen_inputs(spec)
    say("dense fp8 P.V varlen")
    dt = "bf16"
    cu_q, cu_k = torch.from_numpy(inp.cu_q).cuda(), torch.from_numpy(inp.cu_k).cuda()
    out = qa.dense_sage_attention_varlen(dev_bits(inp.q, dt), dev_bits(inp.k, dt), dev_bits(inp.v, dt), cu_q, cu_k,
                                         300, 260, is_causal=True, pv_fp8=True)
    for b in range(3):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        one = qa.dense_sage_attention_ex(dev_bits(inp.q[None, q0:q1], dt), dev_bits(inp.k[None, k0:k1], dt),
                                         dev_bits(inp.v[None, k0:k1], dt), is_causal=True, pv_fp8=True)
        assert torch.equal(one[0], out[q0:q1]), f"sequence {b}"


# packed variable-length dense
VARLEN = [
    # (seq_q, seq_k, Hq, Hkv, d, dtype, causal, smooth_v)
    ([1, 50, 64, 97, 128, 300], [1, 50, 64, 97, 128, 300], 4, 2, 128, "f16", True, True),
    ([130, 7, 0, 260], [200, 7, 30, 260], 8, 1, 64, "bf16", False, False),
    ([300, 5, 16], [100, 0, 16], 2, 2, 256, "f16", True, True),     # Nq > Nk, a sequence without keys
    ([129, 255, 1], [513, 64, 2], 6, 2, 128, "bf16", True, False),
]


def _varlen_run(qa, inp, causal, smooth_v):
    sp = inp.spec
    dt = sp.dtype
    cu_q, cu_k = torch.from_numpy(inp.cu_q).cuda(), torch.from_numpy(inp.cu_k).cuda()
    return qa.dense_sage_attention_varlen(dev_bits(inp.q, dt), dev_bits(inp.k, dt), dev_bits(inp.v, dt), cu_q, cu_k,
                                          max(sp.seq_q), max(sp.seq_k), is_causal=causal, smooth_v=smooth_v,
                                          return_lse=True)


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"{'-'.join(map(str, c[0]))}_on_{'-'.join(map(str, c[1]))}_H{c[2]}/{c[3]}_d{c[4]}_{c[5]}_{'causal' if c[6] else 'full'}{'_sv' if c[7] else ''}")
def test_dense_varlen_parity(qa, case):
    """Packed sequences in one batched call: output and LSE against the
    oracle's per-sequence forward, and every sequence bit-identical to the
    one-sequence options call on its slice."""
    seq_q, seq_k, Hq, Hkv, d, dt, causal, smooth_v = case
    say(f"dense varlen {case}")
    spec = VarlenSpec("vl", 71 + d, seq_q, seq_k, Hq, Hkv, d, dtype=dt, v_bias_std=2.0)
    inp = varlen_inputs(spec)
    out, lse = _varlen_run(qa, inp, causal, smooth_v)
    torch.cuda.synchronize()
    want, want_lse = oracle.sage_varlen_forward(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, dt, causal=causal,
                                                smooth_v=smooth_v, return_lse=True)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert_close(o, want, "dense varlen")
    _lse_close(l, want_lse, "dense varlen LSE")
    for b in range(len(seq_q)):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        if q1 == q0 or k1 == k0:
            continue
        one, one_lse = qa.dense_sage_attention_ex(dev_bits(inp.q[None, q0:q1], dt), dev_bits(inp.k[None, k0:k1], dt),
                                                  dev_bits(inp.v[None, k0:k1], dt), is_causal=causal,
                                                  smooth_v=smooth_v, return_lse=True)
        assert torch.equal(one[0], out[q0:q1]), f"sequence {b} differs from its one-sequence call"
        assert torch.equal(one_lse[0], lse[:, q0:q1]), f"sequence {b} LSE differs"


def test_dense_varlen_extreme_mix_sampled(qa):
    """Lengths 1 : 8192 in one call (the pages' extreme varlen mix): the
    short sequences in full and sampled rows of the long one against the
    oracle's steps on that slice."""
    spec = VarlenSpec("vl_mix", 83, [1, 8192, 33], [1, 8192, 40], 4, 4, 128, dtype="f16")
    inp = varlen_inputs(spec)
    say("dense varlen 1 : 8192 mix")
    out, lse = _varlen_run(qa, inp, True, False)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for b in (0, 2):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        w, wl = oracle.sage_forward(inp.q[None, q0:q1], inp.k[None, k0:k1], inp.v[None, k0:k1], "f16", causal=True,
                                    return_lse=True)
        assert_close(o[q0:q1], w[0], f"varlen sequence {b}")
        _lse_close(l[:, q0:q1], wl[0], f"varlen sequence {b} LSE")
    q0, k0 = inp.cu_q[1], inp.cu_k[1]
    quant = oracle.sage_quantize(inp.q[None, q0:q0 + 8192], inp.k[None, k0:k0 + 8192], "f16")
    rows = np.array([0, 127, 128, 4000, 8191])
    w, wl = oracle.dense_sage_attention(quant, inp.v[None, k0:k0 + 8192], "f16", causal=True, rows=rows,
                                        heads=[0, 3], return_lse=True)
    corr = oracle.sage_lse_correction(inp.q[None, q0:q0 + 8192], quant["k_mean"], "f16")
    for h in (0, 3):
        assert_close(o[q0 + rows, h], w[0, rows, h], f"varlen long sequence head {h}")
        _lse_close(l[h, q0 + rows], wl[0, h, rows] + corr[0, h, rows], f"varlen long sequence LSE head {h}")


def test_decode_workspace_reuse_across_calls(qa):
    # one workspace serves calls with different split counts; partials left
    # by earlier calls must not leak into later results
    say("decode workspace reuse")
    spec = PagedSpec("reuse", 17, 3, 24, 4, 256, [3000, 77, 1500], [1, 1, 1], k_bias_std=2.0)
    inp = paged_inputs(spec)
    kc, ks, vc, vs = gpu_cache(qa, inp, False)
    q8, qs = qa.quantize_q(dev_bits(inp.q))
    tables = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.context_lens).cuda()
    big = qa.decode_params(3, 24, 4, 256, inp.block_tables.shape[1], spec.num_blocks, num_splits=64)
    ws = qa.decode_workspace(big)
    want = _decode_oracle(inp)
    for S in (64, 7, 64, 2, 13):
        out = qa.paged_attention_decode(q8, qs, kc, ks, vc, vs, tables, lens, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), want, f"reuse S={S}")


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_dense_and_varlen_are_deterministic(qa, pv_fp8):
    """Repeat calls give bit-identical outputs and LSE (no atomics in any
    reduction): dense causal with smooth_v, and a varlen batch."""
    say(f"dense determinism fp8={pv_fp8}")
    spec = DenseSpec("dn_det", 711, 2, 4, 2, 300, 257, 128, k_bias_std=3.0, dtype="bf16", v_bias_std=1.0)
    inp = dense_inputs(spec)
    q, k, v = (dev_bits(x, "bf16") for x in (inp.q, inp.k, inp.v))
    runs = [qa.dense_sage_attention_ex(q, k, v, is_causal=True, smooth_v=True, return_lse=True, pv_fp8=pv_fp8)
            for _ in range(5)]
    vs = VarlenSpec("vl_det", 712, [130, 1, 260], [200, 9, 260], 4, 2, 128, dtype="bf16")
    vin = varlen_inputs(vs)
    cu_q, cu_k = torch.from_numpy(vin.cu_q).cuda(), torch.from_numpy(vin.cu_k).cuda()
    vq, vk, vv = (dev_bits(x, "bf16") for x in (vin.q, vin.k, vin.v))
    vruns = [qa.dense_sage_attention_varlen(vq, vk, vv, cu_q, cu_k, 260, 260, is_causal=True, return_lse=True,
                                            pv_fp8=pv_fp8) for _ in range(5)]
    torch.cuda.synchronize()
    for o, l in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(l, runs[0][1])
    for o, l in vruns[1:]:
        assert torch.equal(o, vruns[0][0]) and torch.equal(l, vruns[0][1])
