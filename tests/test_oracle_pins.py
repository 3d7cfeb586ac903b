"""Pins for the CPU oracle: each check ties the oracle to something other
than itself (values the pages print, closed forms, brute force, textbook
attention through scipy, structural invariants). CPU only."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
import oracle as oq
from workloads import (PagedSpec, DenseSpec, VarlenSpec, paged_inputs, dense_inputs, dense_zero_scale_inputs,
                       varlen_inputs, rope_table, to_bf16_bits, to_f16_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _nearest_f32(fr: Fraction) -> np.float32:
    """Nearest float32 to an exact rational (ties to even), found by exact
    comparison of the neighbours of a float64 guess."""
    g = np.float32(float(fr))
    cands = [np.nextafter(g, np.float32(-np.inf)), g, np.nextafter(g, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


# --------------------------------------------------------------------------
# quantization
# --------------------------------------------------------------------------

def test_quant_worked_ties_from_golden():
    rows = _golden("quant_ties.txt")
    x = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1]) for r in rows])
    assert np.array_equal(oq.widen(to_bf16_bits(x), "bf16"), x)  # exact in bf16
    q, s = oracle.quant_rows(x[None])
    assert s[0] == np.float32(1.0)
    assert np.array_equal(q[0].astype(int), want)


def test_quant_scale_is_correctly_rounded_division():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((200, 64)).astype(np.float32) * rng.uniform(1e-3, 1e3, (200, 1)).astype(np.float32)
    _, s = oracle.quant_rows(x)
    for i in range(x.shape[0]):
        amax = Fraction(float(np.max(np.abs(x[i]))))
        assert s[i] == _nearest_f32(amax / 127)


def test_quant_codes_match_exact_rounding_of_fp32_quotient():
    # code = round-half-even of the fp32 quotient x/s; the quotient itself is
    # the float32 nearest to the exact rational x/s.
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 32)).astype(np.float32) * 3
    q, s = oracle.quant_rows(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            quo = _nearest_f32(Fraction(float(x[i, j])) / Fraction(float(s[i])))
            want = max(-127, min(127, round(Fraction(float(quo)))))  # Python round: ties to even
            assert int(q[i, j]) == want


def test_quant_near_ties_against_fp64_quotient():
    # Inputs built to land within a few ulps of k + 1/2 after division by the
    # row scale, where a reciprocal-multiply or a wrong rounding mode shows.
    # Reference route: for fp32 operands the fp64 quotient rounded once to
    # fp32 equals the correctly rounded fp32 quotient.
    rng = np.random.default_rng(14)
    n_rows = 400
    amax = (rng.uniform(0.5, 2.0, n_rows) * 2.0 ** rng.integers(-20, 20, n_rows)).astype(np.float32)
    s_ref = (amax.astype(np.float64) / 127.0).astype(np.float32)
    k = rng.integers(-125, 125, (n_rows, 255))
    x = ((k + 0.5) * s_ref[:, None].astype(np.float64)).astype(np.float32)
    for _ in range(3):
        step = rng.integers(-1, 2, x.shape)
        x = np.where(step > 0, np.nextafter(x, np.float32(np.inf)),
                     np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
    rows = np.concatenate([amax[:, None], x], axis=1)
    q, s = oracle.quant_rows(rows)
    assert np.array_equal(s, s_ref)
    quo = (rows.astype(np.float64) / s_ref[:, None].astype(np.float64)).astype(np.float32)
    want = np.clip(np.rint(quo), -127, 127)
    assert np.array_equal(q.astype(np.float64), want)


def test_quant_properties():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((500, 256)) * rng.uniform(0.01, 100, (500, 1))).astype(np.float32)
    q, s = oracle.quant_rows(x)
    assert q.min() >= -127 and q.max() <= 127
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(500), am]) == 127)
    assert np.all(np.sign(q[np.arange(500), am]) == np.sign(x[np.arange(500), am]))
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None])
    assert np.all(err <= s[:, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -20))


def test_quant_zero_row_and_signed_zero():
    x = np.zeros((2, 64), np.float32)
    x[1] = -0.0
    q, s = oracle.quant_rows(x)
    assert np.all(q == 0) and np.all(s == 0)


def test_quant_tiny_values_fp16_subnormal():
    x = np.array([[6e-8, -1.2e-7, 3e-8, 0.0]], np.float32)
    x = oq.widen(to_f16_bits(x), "f16")[None][0]
    q, s = oracle.quant_rows(x)
    assert s[0] > 0 and abs(int(q[0, 1])) == 127


def test_widen_bf16_and_f16_exact():
    v = np.array([1.0, -2.5, 3.140625, 65504.0, 1e-3], np.float32)
    bb = to_bf16_bits(v)
    assert np.array_equal(oq.widen(bb, "bf16"), np.array([1.0, -2.5, 3.140625, 65536.0, 0.00099945068359375], np.float32))
    hb = to_f16_bits(v)
    assert np.array_equal(oq.widen(hb, "f16"), v.astype(np.float16).astype(np.float32))


# --------------------------------------------------------------------------
# cache layout
# --------------------------------------------------------------------------

def _small_spec(**kw):
    base = dict(name="t", seed=21, num_seqs=3, num_q_heads=6, num_kv_heads=2, head_dim=64,
                context_lens=[17, 1, 40], query_lens=[1, 1, 1], k_bias_std=2.0)
    base.update(kw)
    return PagedSpec(**base)


@pytest.mark.parametrize("v_int8", [False, True])
def test_cache_layout_elementwise(v_int8):
    spec = _small_spec(v_int8=v_int8, pool_blocks=9)
    inp = paged_inputs(spec)
    c = oracle.write_kv_cache(inp.k, inp.v, "bf16", inp.slot_mapping, spec.num_blocks, v_int8)
    kq, ks = oracle.quant_rows(oq.widen(inp.k, "bf16"))
    vq, vs = oracle.quant_rows(oq.widen(inp.v, "bf16"))
    # [QK-MMAC] §3 layout: [block, kv_head, head_dim/16, block_size, 16]
    for t in range(inp.k.shape[0]):
        slot = int(inp.slot_mapping[t])
        b, o = slot // 16, slot % 16
        for h in range(spec.num_kv_heads):
            assert c["k_scale"][b, h, o] == ks[t, h]
            for i in range(spec.head_dim):
                assert c["k_cache"][b, h, i // 16, o, i % 16] == kq[t, h, i]
                if v_int8:
                    assert c["v_cache"][b, h, i, o] == vq[t, h, i]
                else:
                    assert c["v_cache"][b, h, i, o] == inp.v[t, h, i]
            if v_int8:
                assert c["v_scale"][b, h, o] == vs[t, h]


def test_cache_negative_slot_skipped():
    spec = _small_spec()
    inp = paged_inputs(spec)
    slots = inp.slot_mapping.copy()
    slots[::2] = -1
    c = oracle.write_kv_cache(inp.k, inp.v, "bf16", slots, spec.num_blocks)
    for t in range(0, inp.k.shape[0], 2):
        b, o = inp.slot_mapping[t] // 16, inp.slot_mapping[t] % 16
        assert np.all(c["k_cache"][b, :, :, o, :] == 0) and np.all(c["k_scale"][b, :, o] == 0)


# --------------------------------------------------------------------------
# INT32 QK
# --------------------------------------------------------------------------

@pytest.mark.parametrize("row", _golden("int32_bound.txt"))
def test_int32_bound_from_golden(row):
    d, bound = int(row[0]), int(row[1])
    assert bound == d * 127 * 127
    spec = PagedSpec("b", 1, 1, 2, 1, d, [16], [1])
    k = to_bf16_bits(np.full((16, 1, d), 0.75, np.float32))
    v = np.zeros_like(k)
    slots = np.arange(16)
    c = oracle.write_kv_cache(k, v, "bf16", slots, 1)
    q = np.stack([np.full((2, d), 127, np.int8)])
    q[0, 1] = -127
    acc = oracle.paged_qk_int32(q, c, np.zeros((1, 1), np.int32), [16], 1)[0]
    assert np.all(acc[0] == bound) and np.all(acc[1] == -bound)
    assert bound < 2 ** 24 < 2 ** 31 - 1


@pytest.mark.parametrize("ctx", [1, 15, 16, 17, 33])
def test_qk_brute_force_int64(ctx):
    spec = PagedSpec("bf", 5 + ctx, 2, 6, 2, 64, [ctx, 33], [1, 1], k_bias_std=2.0, pool_blocks=7)
    inp = paged_inputs(spec)
    c = oracle.write_kv_cache(inp.k, inp.v, "bf16", inp.slot_mapping, spec.num_blocks)
    q_i8, _ = oracle.quantize_q(inp.q)
    kq, _ = oracle.quant_rows(oq.widen(inp.k, "bf16"))
    accs = oracle.paged_qk_int32(q_i8, c, inp.block_tables, inp.context_lens, 2)
    for s in range(2):
        base = int(inp.cu_seqlens_kv[s])
        for h in range(6):
            for t in range(int(inp.context_lens[s])):
                want = 0
                for i in range(64):
                    want += int(q_i8[s, h, i]) * int(kq[base + t, h // 3, i])
                assert accs[s][h, t] == want


# --------------------------------------------------------------------------
# decode attention
# --------------------------------------------------------------------------

def _textbook_decode(inp, spec, v_int8):
    """softmax(Qdeq Kdeq^T / sqrt d) Vdeq per sequence from the UNPAGED token
    arrays, with scipy's softmax; no block table involved."""
    q_i8, q_s = oracle.quantize_q(inp.q)
    kq, ks = oracle.quant_rows(oq.widen(inp.k, "bf16"))
    if v_int8:
        vq, vs = oracle.quant_rows(oq.widen(inp.v, "bf16"))
        vd = vq.astype(np.float64) * vs[..., None]
    else:
        vd = oq.widen(inp.v, "bf16").astype(np.float64)
    G = spec.group
    out = np.zeros(q_i8.shape, np.float64)
    for s in range(spec.num_seqs):
        a, b = int(inp.cu_seqlens_kv[s]), int(inp.cu_seqlens_kv[s + 1])
        if b == a:
            continue
        for h in range(spec.num_q_heads):
            qd = q_i8[s, h].astype(np.float64) * float(q_s[s, h])
            kd = kq[a:b, h // G].astype(np.float64) * ks[a:b, h // G, None]
            p = sp_softmax(kd @ qd / math.sqrt(spec.head_dim))
            out[s, h] = p @ vd[a:b, h // G]
    return out


def _decode_setup(spec):
    inp = paged_inputs(spec)
    c = oracle.write_kv_cache(inp.k, inp.v, "bf16", inp.slot_mapping, spec.num_blocks, spec.v_int8)
    q_i8, q_s = oracle.quantize_q(inp.q)
    return inp, c, q_i8, q_s


@pytest.mark.parametrize("G,d,v_int8", [(1, 64, False), (2, 128, True), (6, 64, False), (6, 256, True), (16, 64, False)])
def test_decode_equals_textbook_attention_of_dequantized(G, d, v_int8):
    spec = _small_spec(num_q_heads=2 * G, num_kv_heads=2, head_dim=d, v_int8=v_int8,
                       context_lens=[17, 1, 100], pool_blocks=20)
    inp, c, q_i8, q_s = _decode_setup(spec)
    got = oracle.paged_decode(q_i8, q_s, c, inp.block_tables, inp.context_lens, 2)
    want = _textbook_decode(inp, spec, v_int8)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_decode_softmax_rows_sum_to_one_via_one_hot_v():
    # V[t] = e_t makes the output row equal the probability row.
    ctx, d = 40, 64
    spec = PagedSpec("oh", 31, 1, 6, 1, d, [ctx], [1], k_bias_std=1.0, pool_blocks=5)
    inp = paged_inputs(spec)
    v = np.zeros((ctx, 1, d), np.float32)
    v[np.arange(ctx), 0, np.arange(ctx)] = 1.0
    c = oracle.write_kv_cache(inp.k, to_bf16_bits(v), "bf16", inp.slot_mapping, spec.num_blocks)
    q_i8, q_s = oracle.quantize_q(inp.q)
    out = oracle.paged_decode(q_i8, q_s, c, inp.block_tables, inp.context_lens, 1)[0]
    np.testing.assert_allclose(out.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(out[:, :ctx] > 0) and np.all(out[:, ctx:] == 0)
    # the probabilities themselves: scipy softmax of brute-force scores
    acc = oracle.paged_qk_int32(q_i8, c, inp.block_tables, inp.context_lens, 1)[0]
    kq, ks = oracle.quant_rows(oq.widen(inp.k, "bf16"))
    sc = acc * q_s[0][:, None].astype(np.float64) * ks[:, 0][None].astype(np.float64) / 8.0
    np.testing.assert_allclose(out[:, :ctx], sp_softmax(sc, axis=1), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("S", [1, 2, 8, 33])
def test_split_equals_unsplit(S):
    spec = _small_spec(num_q_heads=12, num_kv_heads=2, head_dim=64, context_lens=[17, 1, 300],
                       v_int8=True, pool_blocks=30)
    inp, c, q_i8, q_s = _decode_setup(spec)
    a = oracle.paged_decode(q_i8, q_s, c, inp.block_tables, inp.context_lens, 2)
    b = oracle.paged_decode_split(q_i8, q_s, c, inp.block_tables, inp.context_lens, 2, S)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)


def test_split_segments_cover_context():
    split_segments = oracle.split_segments
    for ctx in [0, 1, 15, 16, 17, 255, 256, 1000]:
        for S in [1, 2, 3, 8, 33]:
            segs = split_segments(ctx, S)
            assert len(segs) == S
            covered = [t for a, b in segs for t in range(a, b)]
            assert covered == list(range(ctx))
            assert all(a % 16 == 0 for a, b in segs if b > a)


def test_decode_empty_context_is_zero():
    spec = _small_spec(context_lens=[0, 5, 0], pool_blocks=3)
    inp, c, q_i8, q_s = _decode_setup(spec)
    out = oracle.paged_decode(q_i8, q_s, c, inp.block_tables, inp.context_lens, 2)
    assert np.all(out[0] == 0) and np.all(out[2] == 0) and np.all(np.isfinite(out))


def test_decode_single_token_returns_its_value():
    spec = _small_spec(context_lens=[1, 1, 1], pool_blocks=3)
    inp, c, q_i8, q_s = _decode_setup(spec)
    out = oracle.paged_decode(q_i8, q_s, c, inp.block_tables, inp.context_lens, 2)
    vv = oq.widen(inp.v, "bf16").astype(np.float64)
    for s in range(3):
        for h in range(6):
            np.testing.assert_array_equal(out[s, h], vv[s, h // 3])


def test_decode_scale_recovery_is_before_softmax():
    # doubling every K scale must change probabilities, not just rescale
    # the scores after softmax ([QK-MMAC] §1).
    spec = _small_spec(context_lens=[64, 64, 64], pool_blocks=12)
    inp, c, q_i8, q_s = _decode_setup(spec)
    a = oracle.paged_decode(q_i8, q_s, c, inp.block_tables, inp.context_lens, 2)
    c2 = dict(c)
    c2["k_scale"] = c["k_scale"] * np.float32(2)
    b = oracle.paged_decode(q_i8, q_s, c2, inp.block_tables, inp.context_lens, 2)
    assert np.max(np.abs(a - b)) > 1e-3
    b2 = oracle.paged_decode(q_i8, q_s, c, inp.block_tables, inp.context_lens, 2, scale=2 / 8.0)
    np.testing.assert_allclose(b, b2, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# chunked prefill
# --------------------------------------------------------------------------

def _prefill_setup(ctxs, qls, G=3, d=64, seed=41):
    spec = PagedSpec("pf", seed, len(ctxs), 2 * G, 2, d, ctxs, qls, k_bias_std=2.0)
    inp = paged_inputs(spec)
    c = oracle.write_kv_cache(inp.k, inp.v, "bf16", inp.slot_mapping, spec.num_blocks)
    q_i8, q_s = oracle.quantize_q(inp.q)
    return spec, inp, c, q_i8, q_s


def test_prefill_equals_textbook_masked_attention():
    spec, inp, c, q_i8, q_s = _prefill_setup([50, 37], [20, 37])
    got = oracle.chunked_prefill(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c,
                                 inp.block_tables, 2)
    kq, ks = oracle.quant_rows(oq.widen(inp.k, "bf16"))
    vd = oq.widen(inp.v, "bf16").astype(np.float64)
    G = spec.group
    for s in range(2):
        a, b = int(inp.cu_seqlens_kv[s]), int(inp.cu_seqlens_kv[s + 1])
        qa, qb = int(inp.cu_seqlens_q[s]), int(inp.cu_seqlens_q[s + 1])
        ctx, tq = b - a, qb - qa
        for i in range(tq):
            pos = ctx - tq + i
            for h in range(spec.num_q_heads):
                qd = q_i8[qa + i, h].astype(np.float64) * float(q_s[qa + i, h])
                kd = kq[a:a + pos + 1, h // G].astype(np.float64) * ks[a:a + pos + 1, h // G, None]
                p = sp_softmax(kd @ qd / 8.0)
                np.testing.assert_allclose(got[qa + i, h], p @ vd[a:a + pos + 1, h // G],
                                           rtol=1e-12, atol=1e-13)


def test_prefill_last_row_equals_decode_and_first_row_of_fresh_chunk():
    spec, inp, c, q_i8, q_s = _prefill_setup([70], [70])
    got = oracle.chunked_prefill(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c,
                                 inp.block_tables, 2)
    # last chunk row sees the whole context = a decode step with that query
    dec = oracle.paged_decode(q_i8[-1:], q_s[-1:], c, inp.block_tables, inp.context_lens, 2)
    np.testing.assert_allclose(got[-1], dec[0], rtol=1e-12, atol=1e-14)
    # with no history, the first row sees only key 0: output = V[0] exactly
    vv = oq.widen(inp.v, "bf16").astype(np.float64)
    for h in range(6):
        np.testing.assert_array_equal(got[0, h], vv[0, h // 3])


def test_multi_token_decode_equals_per_token_decodes():
    """A T-token step (the chunk form of the prefill oracle, T tokens per
    sequence) equals T one-token decodes, token j with the context cut after
    its own position ctx - T + j: pins the causal offset the multi-token
    decode kernel applies per query column. Contexts shorter than T leave
    the earliest tokens with no key (zeros)."""
    T = 4
    ctx = [40, 17, 3]
    spec = PagedSpec("mtp", 91, len(ctx), 8, 2, 64, ctx, [T] * len(ctx), k_bias_std=2.0)
    inp = paged_inputs(spec)
    c = oracle.write_kv_cache(inp.k, inp.v, "bf16", inp.slot_mapping, spec.num_blocks)
    q_i8, q_s = oracle.quantize_q(inp.q)
    got = oracle.chunked_prefill(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2)
    for s_, cl in enumerate(ctx):
        for j in range(T):
            r = s_ * T + j
            lens = np.zeros(len(ctx), np.int32)
            lens[s_] = max(cl - T + j + 1, 0)
            dec = oracle.paged_decode(np.repeat(q_i8[r:r + 1], len(ctx), 0), np.repeat(q_s[r:r + 1], len(ctx), 0),
                                      c, inp.block_tables, lens, 2)
            np.testing.assert_allclose(got[r], dec[s_], rtol=1e-12, atol=1e-14)
    assert np.all(got[2 * T:2 * T + 1] == 0)          # sequence 2 (ctx 3): token 0 sits at position -1


def test_prefill_row_subset_matches_full():
    spec, inp, c, q_i8, q_s = _prefill_setup([90], [33])
    full = oracle.chunked_prefill(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2)
    part = oracle.chunked_prefill(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2,
                                  rows=[0, 7, 32], heads=[1, 4])
    for r in [0, 7, 32]:
        for h in [1, 4]:
            np.testing.assert_array_equal(part[r, h], full[r, h])


# --------------------------------------------------------------------------
# dense SageAttention-style path
# --------------------------------------------------------------------------

def _dense(B=1, H=2, Hkv=2, N=200, Nk=None, d=64, dtype="f16", seed=51, bias=3.0):
    spec = DenseSpec("d", seed, B, H, Hkv, N, Nk or N, d, k_bias_std=bias, dtype=dtype)
    return spec, dense_inputs(spec)


def test_sage_mean_is_exact_sum():
    spec, inp = _dense(N=300)
    qz = oracle.sage_quantize(inp.q, inp.k, "f16")
    k = oq.widen(inp.k, "f16")
    for h in range(2):
        for ch in range(0, 64, 7):
            tot = sum(Fraction(float(x)) for x in k[0, :, h, ch])
            assert qz["k_mean"][0, h, ch] == np.float32(float(tot / 300))


def test_sage_per_block_scales_brute_force():
    spec, inp = _dense(N=200)
    qz = oracle.sage_quantize(inp.q, inp.k, "f16")
    q = oq.widen(inp.q, "f16")
    ks = (oq.widen(inp.k, "f16") - qz["k_mean"][:, None]).astype(np.float32)
    for h in range(2):
        for j, (a, b) in enumerate([(0, 128), (128, 200)]):
            amax = max(abs(float(x)) for x in q[0, a:b, h].ravel())
            assert qz["q_scale"][0, h, j] == _nearest_f32(Fraction(amax) / 127)
        for j, (a, b) in enumerate([(0, 64), (64, 128), (128, 192), (192, 200)]):
            amax = max(abs(float(x)) for x in ks[0, a:b, h].ravel())
            assert qz["k_scale"][0, h, j] == _nearest_f32(Fraction(amax) / 127)
            blk = ks[0, a:b, h]
            codes = qz["k_i8"][0, a:b, h]
            assert np.max(np.abs(codes)) == 127
            assert np.all(np.abs(blk - codes * qz["k_scale"][0, h, j]) <= qz["k_scale"][0, h, j] * 0.50001)


@pytest.mark.parametrize("causal,Nk", [(False, None), (True, None), (True, 260), (False, 70)])
def test_dense_equals_textbook_attention_of_dequantized(causal, Nk):
    spec, inp = _dense(B=2, H=4, Hkv=2, N=150, Nk=Nk)
    qz = oracle.sage_quantize(inp.q, inp.k, "f16")
    got = oracle.dense_sage_attention(qz, inp.v, "f16", causal=causal)
    Nq, Nk_ = spec.seq_q, spec.seq_k
    v = oq.widen(inp.v, "f16").astype(np.float64)
    for b in range(2):
        for h in range(4):
            kvh = h // 2
            qd = qz["q_i8"][b, :, h].astype(np.float64) * np.repeat(qz["q_scale"][b, h], 128)[:Nq, None]
            kd = qz["k_i8"][b, :, kvh].astype(np.float64) * np.repeat(qz["k_scale"][b, kvh], 64)[:Nk_, None]
            s = qd @ kd.T / 8.0
            if causal:
                s = np.where(np.arange(Nk_)[None] <= np.arange(Nq)[:, None] + (Nk_ - Nq), s, -np.inf)
            p = sp_softmax(s, axis=1)
            p = np.nan_to_num(p)
            np.testing.assert_allclose(got[b, :, h], p @ v[b, :, kvh], rtol=1e-12, atol=1e-13)


def test_dense_causal_first_row_is_first_value():
    spec, inp = _dense(N=130)
    qz = oracle.sage_quantize(inp.q, inp.k, "f16")
    got = oracle.dense_sage_attention(qz, inp.v, "f16", causal=True)
    v = oq.widen(inp.v, "f16").astype(np.float64)
    np.testing.assert_array_equal(got[0, 0], v[0, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_dense_zero_scales_give_uniform_attention(causal):
    # a zero K' block scale or a zero query-block scale makes every score of
    # that row 0: the output is the plain mean of V over the visible keys
    inp = dense_zero_scale_inputs()
    spec = inp.spec
    qz = oracle.sage_quantize(inp.q, inp.k, "f16")
    assert np.all(qz["k_scale"][:, 0] == 0) and np.all(qz["k_i8"][:, :, 0] == 0)
    assert np.all(qz["q_scale"][:, 1, 1] == 0)
    got = oracle.dense_sage_attention(qz, inp.v, "f16", causal=causal)
    assert np.all(np.isfinite(got))
    v = oq.widen(inp.v, "f16").astype(np.float64)[0]
    N = spec.seq_k
    cnt = np.arange(1, N + 1)[:, None, None] if causal else N
    mean = (np.cumsum(v, axis=0) / cnt) if causal else np.broadcast_to(v.mean(axis=0), v.shape)
    for h in (0, 1):   # query heads of KV head 0
        np.testing.assert_allclose(got[0, :, h], mean[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got[0, 128:256, 1], mean[128:256, 0], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal,Nk", [(False, None), (True, None), (True, 90)])
def test_lse_of_equal_scores_is_log_of_visible_count(causal, Nk):
    """Zero queries make every score 0, so each row's LSE is ln(#visible keys)
    exactly (-inf for a row that sees none): bottom-right causal rows see
    i + 1 + (Nk - Nq) keys."""
    spec, inp = _dense(B=1, H=2, Hkv=1, N=130, Nk=Nk)
    q0 = np.zeros_like(inp.q)
    out, lse = oracle.sage_forward(q0, inp.k, inp.v, "f16", causal=causal, return_lse=True)
    Nq, Nk_ = spec.seq_q, spec.seq_k
    cnt = np.minimum(np.arange(Nq) + 1 + (Nk_ - Nq), Nk_) if causal else np.full(Nq, Nk_)
    want = np.where(cnt > 0, np.log(np.maximum(cnt, 1).astype(np.float64)), -np.inf)
    for h in range(2):
        np.testing.assert_allclose(lse[0, h], want, rtol=0, atol=1e-13)


def test_lse_correction_restores_constant_key_scores():
    """Keys equal to a constant c at every token: smooth_k removes them
    entirely (K' = 0, all smoothed scores 0), and the corrected LSE must be
    the unsmoothed one, q.c*scale + ln(#visible), in closed form."""
    spec, inp = _dense(B=1, H=4, Hkv=2, N=100, d=64)
    k = np.broadcast_to(inp.k[:, :1], inp.k.shape).copy()           # token 0's row everywhere
    out, lse = oracle.sage_forward(inp.q, k, inp.v, "f16", causal=True, return_lse=True)
    q = oq.widen(inp.q, "f16").astype(np.float64)
    c = oq.widen(k, "f16").astype(np.float64)[0, 0]                # [Hkv, d]
    for h in range(4):
        want = (q[0, :, h] @ c[h // 2]) / 8.0 + np.log(np.arange(1, 101, dtype=np.float64))
        np.testing.assert_allclose(lse[0, h], want, rtol=1e-12, atol=1e-12)


def test_lse_equals_direct_sum_over_scores():
    """The LSE is ln(sum exp) of the same recovered scores the softmax uses:
    exp(lse) equals the brute-force sum of exp(score) (fp64), and with
    smooth_k off no correction is added."""
    spec, inp = _dense(B=1, H=2, Hkv=2, N=70, d=64)
    qz = oracle.sage_quantize(inp.q, inp.k, "f16", smooth_k=False)
    _, lse = oracle.sage_forward(inp.q, inp.k, inp.v, "f16", smooth_k=False, return_lse=True)
    for h in range(2):
        qd = qz["q_i8"][0, :, h].astype(np.float64) * qz["q_scale"][0, h, 0]
        s = np.zeros((70, 70))
        for j in range(70):
            kd = qz["k_i8"][0, j, h].astype(np.float64) * qz["k_scale"][0, h, j // 64]
            s[:, j] = (qd @ kd) / 8.0
        np.testing.assert_allclose(np.exp(lse[0, h]), np.exp(s).sum(axis=1), rtol=1e-12)


def test_smooth_v_adds_the_mean_back():
    """With V carrying a large channel bias, smooth_v (subtract the mean,
    attend, add it back) reproduces the unsmoothed output within the fp16
    rounding of V' = V - mu (half an fp16 ulp of |V'| per element, averaged
    by the softmax), while forgetting the add-back would be off by mu."""
    spec, inp = _dense(B=1, H=2, Hkv=2, N=120, d=64)
    v = oq.widen(inp.v, "f16") + np.float32(6.0) * (np.arange(64, dtype=np.float32) % 3 - 1)
    vb = v.astype(np.float16).view(np.uint16)
    for causal in (False, True):
        a = oracle.sage_forward(inp.q, inp.k, vb, "f16", causal=causal)
        b = oracle.sage_forward(inp.q, inp.k, vb, "f16", causal=causal, smooth_v=True)
        vp, mu = oracle.sage_smooth_v(vb, "f16")
        bound = np.max(np.abs(oq.widen(vp, "f16"))) * 2.0 ** -11 + 1e-12
        assert np.max(np.abs(a - b)) <= bound
        assert np.max(np.abs(mu)) > 100 * bound            # the add-back is what makes them agree
    # the mean is the exact fp64 mean rounded to fp32
    exact = oq.widen(vb, "f16").astype(np.float64).sum(axis=1) / 120.0
    np.testing.assert_array_equal(mu, exact.astype(np.float32))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_the_batched_forward(causal):
    """Packing B equal-length sequences row after row and attending them as
    varlen gives the batched forward (outputs [B, N, H, d] -> [B*N, H, d],
    LSE [B, H, N] -> [H, B*N]); query and key lengths differ, so an offset
    taken from the wrong side shows."""
    spec, inp = _dense(B=3, H=4, Hkv=2, N=150, Nk=170, d=64)
    want, wl = oracle.sage_forward(inp.q, inp.k, inp.v, "f16", causal=causal, smooth_v=True, return_lse=True)
    cu_q, cu_k = [0, 150, 300, 450], [0, 170, 340, 510]
    got, gl = oracle.sage_varlen_forward(inp.q.reshape(450, 4, 64), inp.k.reshape(510, 2, 64),
                                         inp.v.reshape(510, 2, 64), cu_q, cu_k, "f16", causal=causal,
                                         smooth_v=True, return_lse=True)
    np.testing.assert_allclose(got, want.reshape(450, 4, 64), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gl, wl.transpose(1, 0, 2).reshape(4, 450), rtol=1e-12, atol=1e-13)


def test_varlen_sequences_are_independent():
    """A sequence's rows do not change when its neighbours' values change
    (its means, block scales and softmax are its own); a sequence with no
    keys gets zero rows and an LSE of -inf; one with no queries adds no rows."""
    spec = VarlenSpec("vl", 61, [40, 0, 130, 7, 5], [90, 30, 130, 7, 0], 4, 2, 64, v_bias_std=2.0)
    inp = varlen_inputs(spec)
    run = lambda k, v: oracle.sage_varlen_forward(inp.q, k, v, inp.cu_q, inp.cu_k, "f16", causal=True,
                                                  smooth_v=True, return_lse=True)
    out, lse = run(inp.k, inp.v)
    rows0, rows2, rows3 = slice(0, 40), slice(40, 170), slice(170, 177)
    k2 = inp.k.copy()
    k2[:90] = to_f16_bits(oq.widen(k2[:90], "f16") * np.float32(3.0) + np.float32(1.0))   # keys of sequence 0
    out2, lse2 = run(k2, inp.v)
    assert not np.allclose(out[rows0], out2[rows0])           # the change shows where it belongs
    np.testing.assert_array_equal(out2[40:], out[40:])        # and nowhere else
    np.testing.assert_array_equal(lse2[:, 40:], lse[:, 40:])
    v2 = inp.v.copy()
    v2[120:250] = to_f16_bits(oq.widen(v2[120:250], "f16") - np.float32(5.0))           # values of sequence 2
    out3, _ = run(inp.k, v2)
    assert not np.allclose(out[rows2], out3[rows2])
    np.testing.assert_array_equal(out3[rows0], out[rows0])
    np.testing.assert_array_equal(out3[rows3], out[rows3])
    np.testing.assert_array_equal(out[177:], 0.0)                # sequence 4: no keys
    assert np.all(np.isneginf(lse[:, 177:]))
    assert np.all(np.isfinite(lse[:, :177]))
    # the one-sequence forward on each slice
    for b, (q0, q1, k0, k1) in enumerate([(0, 40, 0, 90), (40, 170, 120, 250), (170, 177, 250, 257)]):
        one = oracle.sage_forward(inp.q[None, q0:q1], inp.k[None, k0:k1], inp.v[None, k0:k1], "f16", causal=True,
                                  smooth_v=True)
        np.testing.assert_array_equal(out[q0:q1], one[0])


def test_smoothing_leaves_unquantized_attention_unchanged():
    # softmax is invariant to adding q.mu to every score of a row
    spec, inp = _dense(N=100, d=64)
    q = oq.widen(inp.q, "f16").astype(np.float64)[0, :, 0]
    k = oq.widen(inp.k, "f16").astype(np.float64)[0, :, 0]
    v = oq.widen(inp.v, "f16").astype(np.float64)[0, :, 0]
    mu = k.mean(axis=0)
    a = sp_softmax(q @ k.T / 8.0, axis=1) @ v
    b = sp_softmax(q @ (k - mu).T / 8.0, axis=1) @ v
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_smoothing_reduces_quantization_error():
    # with a strong channel bias, smoothing K lowers the error against
    # unquantized attention ([SAGE-MACA] presents smooth_k as outlier removal)
    spec, inp = _dense(N=256, d=64, bias=6.0)
    ref = np.zeros((256, 2, 64))
    q = oq.widen(inp.q, "f16").astype(np.float64)[0]
    k = oq.widen(inp.k, "f16").astype(np.float64)[0]
    v = oq.widen(inp.v, "f16").astype(np.float64)[0]
    for h in range(2):
        ref[:, h] = sp_softmax(q[:, h] @ k[:, h].T / 8.0, axis=1) @ v[:, h]
    errs = []
    for smooth in (False, True):
        qz = oracle.sage_quantize(inp.q, inp.k, "f16", smooth_k=smooth)
        o = oracle.dense_sage_attention(qz, inp.v, "f16")[0]
        errs.append(np.linalg.norm(o - ref) / np.linalg.norm(ref))
    assert errs[1] < errs[0]


def test_attention_fp64_matches_scipy():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 20, 16))
    got = oracle.attention_fp64(q, k, v, 0.25)
    np.testing.assert_allclose(got, sp_softmax(q @ k.T * 0.25, axis=1) @ v, rtol=1e-13)


# --------------------------------------------------------------------------
# rotary embedding in the producer


def _rope_x(T=6, H=3, d=64, seed=91, scale=1.0):
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal((T, H, d)).astype(np.float32) * np.float32(scale))


@pytest.mark.parametrize("neox", [True, False])
def test_rope_position_zero_is_identity(neox):
    x = _rope_x()
    tab = rope_table(16, 64)
    np.testing.assert_array_equal(oracle.apply_rope(x, "bf16", np.zeros(6, np.int64), tab, 64, neox),
                                  oq.widen(x, "bf16"))


@pytest.mark.parametrize("neox", [True, False])
def test_rope_pairs_rotate_as_complex_numbers(neox):
    """Each channel pair (a, b) with frequency i becomes (a + ib) e^(i theta)
    (complex128 product; fp32 rounding bound), channels past rot_dim are
    untouched (partial rotary, 32 of 64)."""
    x = _rope_x(T=8)
    tab = rope_table(5000, 32)
    pos = np.array([0, 1, 2, 17, 100, 999, 4095, 4999])
    got = oracle.apply_rope(x, "bf16", pos, tab, 32, neox)
    xv = oq.widen(x, "bf16").astype(np.float64)
    ia = np.arange(16) if neox else np.arange(0, 32, 2)
    ib = ia + 16 if neox else ia + 1
    z = (xv[..., ia] + 1j * xv[..., ib]) * (tab[pos, :16].astype(np.float64) + 1j * tab[pos, 16:].astype(np.float64))[:, None, :]
    bound = 2.0 ** -22 * (np.abs(xv[..., ia]) + np.abs(xv[..., ib]))
    assert np.all(np.abs(got[..., ia] - z.real) <= bound)
    assert np.all(np.abs(got[..., ib] - z.imag) <= bound)
    np.testing.assert_array_equal(got[..., 32:], oq.widen(x, "bf16")[..., 32:])


def test_rope_interleaved_is_half_pairing_of_permuted_channels():
    x = _rope_x()
    tab = rope_table(300, 64)
    pos = np.array([3, 5, 8, 13, 21, 299])
    perm = np.concatenate([np.arange(0, 64, 2), np.arange(1, 64, 2)])   # interleaved -> halves
    a = oracle.apply_rope(x, "bf16", pos, tab, 64, neox=False)
    b = oracle.apply_rope(x[..., perm], "bf16", pos, tab, 64, neox=True)
    np.testing.assert_array_equal(a[..., perm], b)


@pytest.mark.parametrize("neox", [True, False])
def test_rope_dot_products_depend_on_position_difference(neox):
    q, k = _rope_x(T=1, H=1, seed=5), _rope_x(T=1, H=1, seed=6)
    tab = rope_table(4096, 64, base=1e4)
    dots = []
    for m, n in [(40, 10), (47, 17), (3030, 3000)]:
        qr = oracle.apply_rope(q, "bf16", [m], tab, 64, neox).astype(np.float64)
        kr = oracle.apply_rope(k, "bf16", [n], tab, 64, neox).astype(np.float64)
        dots.append(float(np.sum(qr * kr)))
    np.testing.assert_allclose(dots[1:], dots[0], rtol=2e-5, atol=2e-5)
    unrot = float(np.sum(oq.widen(q, "bf16").astype(np.float64) * oq.widen(k, "bf16")))
    assert abs(dots[0] - unrot) > 1e-3                       # the rotation does change it


def test_rope_cache_write_holds_rotated_keys():
    """The K cache written by the rotary producer dequantizes to the rotated
    keys within half a quantization step; at position 0 it is the plain
    write byte for byte."""
    k, v = _rope_x(T=20, H=2, seed=7, scale=3.0), _rope_x(T=20, H=2, seed=8)
    tab = rope_table(64, 64)
    slots = np.arange(20) + 5
    pos = np.arange(20) * 3 + 1
    c = oracle.rope_write_kv_cache(k, v, "bf16", slots, 4, pos, tab, 64, neox=True)
    kq, sk, _ = oracle.gather_kv(c, np.array([0, 1, 2, 3]), 25, 1)
    rot = oracle.apply_rope(k, "bf16", pos, tab, 64, True)[:, 1]
    err = np.abs(kq[5:].astype(np.float64) * sk[5:, None] - rot)
    assert np.all(err <= sk[5:, None] * 0.5 * (1 + 1e-6))
    assert np.max(np.abs(rot - oq.widen(k, "bf16")[:, 1])) > 10 * np.max(sk)   # and rotation is visible
    c0 = oracle.rope_write_kv_cache(k, v, "bf16", slots, 4, np.zeros(20, np.int64), tab, 64)
    c1 = oracle.write_kv_cache(k, v, "bf16", slots, 4)
    for key in ("k_cache", "k_scale", "v_cache"):
        np.testing.assert_array_equal(c0[key], c1[key])



# --------------------------------------------------------------------------
# FP8 (E4M3) P.V


def test_e4m3_landmarks_ties_and_saturation():
    dec = oracle.e4m3_decode
    assert dec(0x38) == 1.0 and dec(0x7E) == 448.0 and dec(0x01) == 2.0 ** -9 and dec(0x08) == 2.0 ** -6
    assert dec(0x07) == 7 * 2.0 ** -9 and np.isnan(dec(0x7F)) and dec(0xB8) == -1.0
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(dec(finite)), finite)
    # midpoints go to the even code
    assert oracle.e4m3_encode(1.0625) == 0x38 and oracle.e4m3_encode(1.1875) == 0x3A
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00 and oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert oracle.e4m3_encode(460.0) == 0x7E and oracle.e4m3_encode(-1e-12) == 0x80


def test_e4m3_matches_torch_conversion():
    import torch
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * 60, rng.standard_normal(50000) * 1e-3,
                        np.float32(2.0) ** np.arange(-12, 9)]).astype(np.float32)
    got = oracle.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, want)


def _fp8_case(N=200, Nk=None, d=64, causal=False, seed=77, vfun=None):
    spec, inp = _dense(N=N, Nk=Nk, d=d, seed=seed)
    v = inp.v if vfun is None else to_f16_bits(vfun(oq.widen(inp.v, "f16")))
    quant = oracle.sage_quantize(inp.q, inp.k, "f16")
    return inp, quant, v


def test_fp8pv_constant_values_come_back():
    # every token holds the same V row: whatever P is, the output is that row
    c = (np.arange(64, dtype=np.float32) - 20.0) * np.float32(0.37)
    inp, quant, v = _fp8_case(N=150, vfun=lambda x: np.broadcast_to(c, x.shape).copy())
    out = oracle.dense_sage_attention_fp8pv(quant, v, "f16", causal=True)
    cv = oq.widen(to_f16_bits(c), "f16").astype(np.float64)
    np.testing.assert_allclose(out, np.broadcast_to(cv, out.shape), rtol=2e-7, atol=1e-12)


def _int_dot_scores(quant, b, row, keys, h=0):
    q = quant["q_i8"][b, row, h].astype(np.float64)
    k = quant["k_i8"][b, keys, h].astype(np.float64)
    return (k @ q) * float(quant["q_scale"][b, h, row // 128]) * quant["k_scale"][b, h, np.asarray(keys) // 64] / 8.0


def test_fp8pv_one_visible_key_and_two_key_closed_form():
    inp, quant, v = _fp8_case(N=130, causal=True)
    out = oracle.dense_sage_attention_fp8pv(quant, v, "f16", causal=True)
    v8, sv = oracle.v_fp8_per_channel(oq.widen(v, "f16"))
    # row 0 sees key 0 only: its FP8-rounded value times the channel scale
    np.testing.assert_allclose(out[0, 0], v8[0, 0] * sv[0], rtol=1e-12)
    # row 1 sees keys 0 and 1: P8 = E4M3(448 exp(s - m)) with m their maximum
    s = _int_dot_scores(quant, 0, 1, [0, 1])
    p = oracle.e4m3_round(448.0 * np.exp(s - s.max()))
    assert p.max() == 448.0
    want = (p[0] * v8[0, 0, 0] + p[1] * v8[0, 1, 0]) / p.sum() * sv[0, 0]
    np.testing.assert_allclose(out[0, 1, 0], want, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8pv_lse_of_equal_scores_is_log_of_visible_count(causal):
    """Zero queries: every score is 0, every P8 is E4M3(448) = 448, so the
    LSE is ln(#visible) exactly and the output is the plain mean of the
    FP8-rounded V over the visible keys."""
    spec, inp = _dense(B=1, H=2, Hkv=2, N=100, Nk=130, d=64)
    quant = oracle.sage_quantize(np.zeros_like(inp.q), inp.k, "f16")
    out, lse = oracle.dense_sage_attention_fp8pv(quant, inp.v, "f16", causal=causal, return_lse=True)
    cnt = np.minimum(np.arange(100) + 1 + 30, 130) if causal else np.full(100, 130)
    for h in range(2):
        np.testing.assert_allclose(lse[0, h], np.log(cnt.astype(np.float64)), rtol=0, atol=1e-13)
    v8, sv = oracle.v_fp8_per_channel(oq.widen(inp.v, "f16"))
    cs = np.cumsum(v8[0], axis=0)                                  # [Nk, H, d]
    mean = cs[cnt - 1] / cnt[:, None, None] * sv[0][None]
    np.testing.assert_allclose(out[0], mean, rtol=1e-12, atol=1e-14)


def test_fp8pv_is_within_fp8_error_of_the_16bit_path():
    """Against the exact-P path: relative L2 of order the E4M3 step (2^-4
    per rounded term, averaged over keys) and not identical."""
    inp, quant, v = _fp8_case(N=300, Nk=260, causal=False, vfun=lambda x: x + np.float32(0.5))
    for causal in (False, True):
        a = oracle.dense_sage_attention_fp8pv(quant, v, "f16", causal=causal)
        b = oracle.dense_sage_attention(quant, v, "f16", causal=causal)
        r = np.linalg.norm(a - b) / np.linalg.norm(b)
        assert 1e-4 < r < 3e-2, r


def _fp8_tolerance_stats(a, b, sig, floor):
    d = np.abs(a - b)
    z = d / np.maximum(sig, floor)
    return d, z


@pytest.mark.parametrize("causal,smooth_v", [(False, False), (True, True)])
def test_fp8pv_tolerance_model_covers_lazy_references(causal, smooth_v):
    """The tolerance model of the plain definition (sigma, sigma_lse): a
    tiled implementation that rounds P from a lazily moved reference (the
    model or_dense_attention_fp8pv_lazy: 64-key tiles, slack 3, 16-row
    groups deciding together) stays within 6 sigma of the definition on every
    element and within 1 sigma in RMS, and the model is not vacuous (the two
    do differ, by more than 5% of sigma in RMS)."""
    inp, quant, v = _fp8_case(N=400, Nk=420, causal=causal, vfun=lambda x: x + np.float32(0.3))
    out, lse, sig, sig_l = oracle.dense_sage_attention_fp8pv(quant, v, "f16", causal=causal, smooth_v=smooth_v,
                                                              return_sigma=True)
    lazy, lazy_lse = oracle.dense_sage_attention_fp8pv_lazy(quant, v, "f16", causal=causal, smooth_v=smooth_v,
                                                            return_lse=True)
    floor = 1e-9 * np.max(np.abs(out))
    d, z = _fp8_tolerance_stats(lazy, out, sig, floor)
    assert np.max(z) <= 6.0, np.max(z)
    rms = float(np.sqrt(np.mean(z ** 2)))
    assert 0.05 < rms <= 1.0, rms
    dl = np.abs(lazy_lse - lse)
    zl = dl / np.maximum(sig_l, 1e-12)
    assert np.max(zl) <= 6.0 and float(np.sqrt(np.mean(zl ** 2))) <= 1.0


def test_fp8pv_tolerance_model_is_calibrated_by_random_references():
    """Independent of any tiling: each key's P rounded at a random reference
    m' in [m - 3 ln 2, m] (P8' = E4M3(56 exp(s - m')), scaled back by
    exp(m' - m)), computed here with the pinned codec, against the plain
    definition. sigma bounds each rounding by its largest error (2^-4
    relative); for mantissas spread over [1, 2) the RMS error is about 0.71
    of that, so |difference| / sigma must have an RMS near 0.7 (0.6 .. 0.82
    over 256 rows x 64 channels; a sigma off by sqrt(2) lands outside) and
    no element beyond 6; the LSE likewise (0.5 .. 0.85 over 256 rows)."""
    inp, quant, v = _fp8_case(N=256, Nk=300, d=64, seed=78)
    out, lse, sig, sig_l = oracle.dense_sage_attention_fp8pv(quant, v, "f16", return_sigma=True)
    v8, sv = oracle.v_fp8_per_channel(oq.widen(v, "f16"))
    rng = np.random.default_rng(9)
    zs, zl = [], []
    for row in range(256):
        s = _int_dot_scores(quant, 0, row, list(range(300)))
        m = s.max()
        mp = m - rng.uniform(0.0, 3.0 * np.log(2.0), size=300)
        p = oracle.e4m3_round(56.0 * np.exp(s - mp)) * np.exp(mp - m)
        alt = (p @ v8[0, :, 0]) / p.sum() * sv[0, 0]
        zs.append(np.abs(alt - out[0, row, 0]) / np.maximum(sig[0, row, 0], 1e-12))
        zl.append(abs(m + np.log(p.sum() / 56.0) - lse[0, 0, row]) / sig_l[0, 0, row])
    zs, zl = np.concatenate(zs), np.array(zl)
    assert np.max(zs) <= 6.0 and np.max(zl) <= 6.0, (np.max(zs), np.max(zl))
    rms, rms_l = float(np.sqrt(np.mean(zs ** 2))), float(np.sqrt(np.mean(zl ** 2)))
    assert 0.6 <= rms <= 0.82, rms
    assert 0.5 <= rms_l <= 0.85, rms_l


def test_v_fp8_per_channel_codes():
    """Every channel's largest magnitude maps to 448; all values are E4M3
    values; each is within half an E4M3 step of V / s."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((2, 90, 3, 64)) * rng.uniform(0.1, 30, (1, 1, 3, 64))).astype(np.float32)
    v[:, :, 1, 7] = 0.0                                   # an all-zero channel: scale 0, codes 0
    vals, s = oracle.v_fp8_per_channel(v)
    np.testing.assert_array_equal(oracle.e4m3_round(vals), vals)
    amax = np.abs(vals).max(axis=1)
    assert np.all((amax == 448.0) | (s == 0)) and s[0, 1, 7] == 0 and np.all(vals[:, :, 1, 7] == 0)
    r = v / np.where(s > 0, s, 1)[:, None]
    step = np.where(np.abs(r) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(vals - r) <= step / 2 * (1 + 1e-9))


# --------------------------------------------------------------------------
# chunked prefill with the P.V product in FP8 (E4M3)
# --------------------------------------------------------------------------

def _prefill_fp8_setup(ctxs, qls, G=3, d=64, seed=43, v_int8=False, vfun=None):
    spec = PagedSpec("pf8", seed, len(ctxs), 2 * G, 2, d, ctxs, qls, k_bias_std=2.0, v_int8=v_int8)
    inp = paged_inputs(spec)
    v = inp.v if vfun is None else to_bf16_bits(vfun(oq.widen(inp.v, "bf16")))
    c = oracle.write_kv_cache(inp.k, v, "bf16", inp.slot_mapping, spec.num_blocks, v_int8)
    q_i8, q_s = oracle.quantize_q(inp.q)
    return spec, inp, c, q_i8, q_s, v


def _token_v_values(inp, v_bits, s, v_int8):
    """fp32 V of sequence s's tokens from the unpaged arrays ([ctx, Hkv, d]):
    16-bit V exactly, INT8 V as fl32(code * scale) of its row quantization."""
    a, b = int(inp.cu_seqlens_kv[s]), int(inp.cu_seqlens_kv[s + 1])
    v = oq.widen(v_bits[a:b], "bf16")
    if v_int8:
        vq, vs = oracle.quant_rows(v)
        v = (vq.astype(np.float32) * vs[..., None]).astype(np.float32)
    return v


@pytest.mark.parametrize("v_int8", [False, True])
def test_prefill_fp8_v_codes_are_per_channel_over_the_whole_context(v_int8):
    """The paged V codes and scales of a (sequence, KV head) equal the
    per-channel E4M3 of that sequence's unpaged token values (every cached
    token counts, not only those a row sees)."""
    spec, inp, c, q_i8, q_s, v = _prefill_fp8_setup([70, 33], [20, 33], v_int8=v_int8)
    for s_ in range(2):
        vals = _token_v_values(inp, v, s_, v_int8)
        want_v, want_s = oracle.v_fp8_per_channel(vals[None])
        for h in range(2):
            codes, sc = oracle.paged_v_fp8(c, inp.block_tables, s_, int(inp.context_lens[s_]), h, 2, 2,
                                           spec.head_dim)
            np.testing.assert_array_equal(sc, want_s[0, h])
            np.testing.assert_array_equal(oracle.e4m3_decode(codes), want_v[0, :, h])


def test_prefill_fp8_first_rows_of_a_fresh_chunk_closed_form():
    """No history: row 0 sees key 0 only (out = V8[0] s); row 1 sees keys 0
    and 1 with P8 = E4M3(448 exp(s - m)) at their exact maximum."""
    spec, inp, c, q_i8, q_s, v = _prefill_fp8_setup([40], [40])
    out = oracle.chunked_prefill_fp8pv(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2)
    kq, ks = oracle.quant_rows(oq.widen(inp.k, "bf16"))
    for h in range(6):
        codes, sc = oracle.paged_v_fp8(c, inp.block_tables, 0, 40, h // 3, 1, 2, 64)
        v8 = oracle.e4m3_decode(codes)
        np.testing.assert_allclose(out[0, h], v8[0] * sc, rtol=1e-15, atol=0)
        qd = q_i8[1, h].astype(np.float64) * float(q_s[1, h])
        sco = np.array([kq[t, h // 3].astype(np.float64) @ qd * float(ks[t, h // 3]) / 8.0 for t in (0, 1)])
        p = oracle.e4m3_round(448.0 * np.exp(sco - sco.max()))
        want = (p[0] * v8[0] + p[1] * v8[1]) / p.sum() * sc
        np.testing.assert_allclose(out[1, h], want, rtol=1e-12, atol=1e-15)


def test_prefill_fp8_zero_queries_give_the_mean_of_the_visible_rounded_values():
    """Zero queries: all scores 0, every P8 = 448, so row i of a chunk of Tq
    on ctx tokens is the mean of V8 s over keys 0 .. ctx - Tq + i (pins the
    bottom-right causal offset and the key count)."""
    spec, inp, c, q_i8, q_s, v = _prefill_fp8_setup([90, 21], [30, 21])
    q0 = np.zeros_like(q_i8)
    out = oracle.chunked_prefill_fp8pv(q0, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2)
    for s_, (ctx, tq) in enumerate([(90, 30), (21, 21)]):
        qa = int(inp.cu_seqlens_q[s_])
        for kvh in range(2):
            codes, sc = oracle.paged_v_fp8(c, inp.block_tables, s_, ctx, kvh, 2, 2, 64)
            cs = np.cumsum(oracle.e4m3_decode(codes), axis=0)
            for i in range(tq):
                nvis = ctx - tq + i + 1
                for h in range(3 * kvh, 3 * kvh + 3):
                    np.testing.assert_allclose(out[qa + i, h], cs[nvis - 1] / nvis * sc, rtol=1e-12, atol=1e-15)


def test_prefill_fp8_a_late_key_sets_the_channel_scale():
    """A large value on channel 5 at the last token (seen by the last row
    only) sets that channel's scale for every row: row 0 of the chunk reads
    its channel-5 value rounded on that coarse grid, away from the exact one."""
    def vfun(x):
        x = x.copy()
        x[-1, :, 5] = np.float32(900.0)
        return x
    spec, inp, c, q_i8, q_s, v = _prefill_fp8_setup([48], [48], vfun=vfun)
    out = oracle.chunked_prefill_fp8pv(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2)
    vals = _token_v_values(inp, v, 0, False)
    sc5 = np.float32(np.abs(vals[:, 0, 5]).max() / np.float32(448.0))
    want = oracle.e4m3_round(np.float64(np.float32(vals[0, 0, 5] / sc5))) * np.float64(sc5)
    assert out[0, 0, 5] == pytest.approx(want, rel=1e-15)
    assert abs(out[0, 0, 5] - vals[0, 0, 5]) > 1e-3


def test_prefill_fp8_is_within_fp8_error_of_the_16bit_path():
    """Against the exact-P prefill: relative L2 of order the E4M3 step and
    not identical (V offset by 0.5, so that outputs are not averages near 0)."""
    spec, inp, c, q_i8, q_s, v = _prefill_fp8_setup([300, 130], [64, 130], d=128, vfun=lambda x: x + np.float32(0.5))
    a = oracle.chunked_prefill_fp8pv(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2)
    b = oracle.chunked_prefill(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2)
    r = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 1e-4 < r < 3e-2, r


def test_prefill_fp8_tolerance_model_is_calibrated_by_random_references():
    """As for the dense FP8 path: each key's P rounded at a random reference
    m' in [m - 3 ln 2, m] (scaled back), against the plain definition, lands
    within 6 sigma everywhere with an RMS z near 0.7."""
    spec, inp, c, q_i8, q_s, v = _prefill_fp8_setup([260], [60], G=1, seed=47)
    out, sig = oracle.chunked_prefill_fp8pv(q_i8, q_s, inp.cu_seqlens_q, inp.context_lens, c, inp.block_tables, 2,
                                            return_sigma=True)
    kq, ks = oracle.quant_rows(oq.widen(inp.k, "bf16"))
    codes, sc = oracle.paged_v_fp8(c, inp.block_tables, 0, 260, 0, 1, 2, 64)
    v8 = oracle.e4m3_decode(codes)
    rng = np.random.default_rng(11)
    zs = []
    for i in range(60):
        nvis = 200 + i + 1
        qd = q_i8[i, 0].astype(np.float64) * float(q_s[i, 0])
        sco = (kq[:nvis, 0].astype(np.float64) @ qd) * ks[:nvis, 0].astype(np.float64) / 8.0
        m = sco.max()
        mp = m - rng.uniform(0.0, 3.0 * np.log(2.0), size=nvis)
        p = oracle.e4m3_round(56.0 * np.exp(sco - mp)) * np.exp(mp - m)
        alt = (p @ v8[:nvis]) / p.sum() * sc
        zs.append(np.abs(alt - out[i, 0]) / np.maximum(sig[i, 0], 1e-12))
    zs = np.concatenate(zs)
    assert np.max(zs) <= 6.0, np.max(zs)
    rms = float(np.sqrt(np.mean(zs ** 2)))
    assert 0.6 <= rms <= 0.82, rms


def test_f32_to_f16_bits_matches_numpy_rounding():
    """fp32 -> fp16 (the V' operand of smooth_v) equals numpy's
    round-to-nearest-even cast, including subnormals, ties, the largest
    finite value and overflow."""
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-9, 5.2, 300000)).astype(np.float32)
    edge = np.float32([0.0, -0.0, 65504, 65519.99, 65520, 70000, -65520, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25,
                       2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11), 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1e-45])
    x = np.concatenate([x, edge])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_f16_bits(x), want)
