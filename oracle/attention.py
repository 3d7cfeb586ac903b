"""Oracle: INT8-QK attention with score recovery, softmax and P.V in fp64.

Test infrastructure only (see the package docstring).

Integer products. The QK accumulator is an exact integer dot product of
INT8 codes. It is computed here as an fp64 matrix product: every term is an
integer of magnitude <= 127*127, and the sum over head_dim <= 256 terms stays
below 256*127*127 = 4,129,024 < 2^53 ([QK-MMAC] §2.1 prints this bound), so
every partial sum is exactly representable and the result equals the
integer dot product in any summation order. A pin test checks it against
int64 brute force.
"""
from __future__ import annotations

import math

import numpy as np

from .quant import BLOCK, gather_kv, widen


def default_scale(head_dim: int) -> float:
    """softmax scale 1/sqrt(d) ([QK-MMAC] §1; [SAGE-MACA] advanced options)."""
    return 1.0 / math.sqrt(head_dim)


def _scale(scale, head_dim):
    """A positive caller scale is taken as given (fp32 on the GPU side, so the
    fp32 value is what both sides use); otherwise 1/sqrt(d)."""
    if scale is not None and scale > 0:
        return float(np.float32(scale))
    return default_scale(head_dim)


def _int_dot(a_i8: np.ndarray, b_i8: np.ndarray) -> np.ndarray:
    """Exact integer a @ b.T for INT8 code matrices (see module docstring)."""
    return a_i8.astype(np.float64) @ b_i8.astype(np.float64).T


def _softmax_pv(s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Two-pass softmax over the last axis of s (masked entries are -inf) and
    the product with v, in fp64. A row with no visible key gives zeros."""
    out = np.zeros(s.shape[:-1] + (v.shape[-1],), np.float64)
    if s.shape[-1] == 0:
        return out
    m = np.max(s, axis=-1, keepdims=True)
    live = np.isfinite(m[..., 0])
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    o = (p @ v) / np.where(l > 0, l, 1.0)
    out[live] = o[live]
    return out


def _logsumexp_rows(s: np.ndarray) -> np.ndarray:
    """ln(sum_j exp(s_j)) per row of s (masked entries -inf) in fp64, as
    m + ln(sum_j exp(s_j - m)); a row with no visible entry gives -inf."""
    if s.shape[-1] == 0:
        return np.full(s.shape[:-1], -np.inf)
    m = np.max(s, axis=-1)
    live = np.isfinite(m)
    mm = np.where(live, m, 0.0)
    l = np.exp(s - mm[..., None]).sum(axis=-1)
    return np.where(live, mm + np.log(np.where(l > 0, l, 1.0)), -np.inf)


def paged_qk_int32(q_i8, caches, block_tables, context_lens, num_kv_heads):
    """INT32 QK accumulators of decode: one query token per sequence.

    [QK-MMAC] §2.1-2.2: rows are query heads, columns are history tokens,
    acc[h][t] = sum_i Qq[h][i] * Kq_t[i], with K_t fetched through the block
    table ([QK-MMAC] §3) from KV head h // G ([QK-MMAC] §5.2 mapping).
    Returns a list with one int64 array [Hq, ctx] per sequence.
    """
    S, Hq, d = q_i8.shape
    G = Hq // num_kv_heads
    out = []
    for s in range(S):
        ctx = int(context_lens[s])
        acc = np.zeros((Hq, ctx), np.int64)
        for kvh in range(num_kv_heads):
            kq, _, _ = gather_kv(caches, block_tables[s], ctx, kvh)
            acc[kvh * G:(kvh + 1) * G] = _int_dot(q_i8[s, kvh * G:(kvh + 1) * G], kq).astype(np.int64)
        out.append(acc)
    return out


def _decode_scores(q_i8, q_scale, kq, sk, scale):
    """[QK-MMAC] §1: score = acc * sQ(query token, query head) * sK(key token,
    KV head) * softmax_scale, recovered per element before the softmax."""
    acc = _int_dot(q_i8, kq)                                       # [G, ctx]
    return acc * q_scale.astype(np.float64)[:, None] * sk.astype(np.float64)[None, :] * scale


def paged_decode(q_i8, q_scale, caches, block_tables, context_lens, num_kv_heads,
                 scale=None, v_dtype="bf16", heads=None):
    """Decode attention, one query token per sequence, unsplit reference.

    q_i8 [S, Hq, d], q_scale [S, Hq]. Keys t < ctx are visible. Softmax and
    P.V in fp64 with V dequantized exactly (bf16 value, or code * sV).
    A sequence with ctx == 0 yields zeros. ``heads`` optionally limits the
    query heads computed (others stay zero). Returns fp64 [S, Hq, d].
    """
    S, Hq, d = q_i8.shape
    G = Hq // num_kv_heads
    sc = _scale(scale, d)
    out = np.zeros((S, Hq, d), np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        for kvh in range(num_kv_heads):
            hs = [h for h in range(kvh * G, (kvh + 1) * G) if heads is None or h in heads]
            if not hs:
                continue
            kq, sk, v = gather_kv(caches, block_tables[s], ctx, kvh, v_dtype)
            sc_rows = _decode_scores(q_i8[s, hs], q_scale[s, hs], kq, sk, sc)
            out[s, hs] = _softmax_pv(sc_rows, v)
    return out


def split_segments(ctx: int, num_splits: int):
    """Block-aligned split-K segments: L = 16 * ceil(ceil(ctx/16) / S);
    segment j covers [j*L, min((j+1)*L, ctx)), possibly empty.
    ([QK-MMAC] §4 splits long decode contexts into segments; the exact cut
    is this library's reading.)"""
    nblk = -(-ctx // BLOCK)
    L = BLOCK * max(-(-nblk // num_splits), 1)
    return [(j * L, min((j + 1) * L, ctx)) for j in range(num_splits)]


def paged_decode_split(q_i8, q_scale, caches, block_tables, context_lens, num_kv_heads,
                       num_splits, scale=None, v_dtype="bf16"):
    """Split-K decode then combine, for self-checking the combine algebra.

    Each segment j yields (m_j, l_j, O_j) with m_j the segment max score,
    l_j = sum exp(s - m_j), O_j = sum exp(s - m_j) v (unnormalized); an empty
    segment yields (-inf, 0, 0). Combine: M = max m_j, w_j = exp(m_j - M),
    O = sum w_j O_j / sum w_j l_j.
    """
    S, Hq, d = q_i8.shape
    G = Hq // num_kv_heads
    sc = _scale(scale, d)
    out = np.zeros((S, Hq, d), np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        for kvh in range(num_kv_heads):
            hs = slice(kvh * G, (kvh + 1) * G)
            kq, sk, v = gather_kv(caches, block_tables[s], ctx, kvh, v_dtype)
            sc_rows = _decode_scores(q_i8[s, hs], q_scale[s, hs], kq, sk, sc)
            ms, ls, os_ = [], [], []
            for a, b in split_segments(ctx, num_splits):
                if b <= a:
                    ms.append(np.full(G, -np.inf)); ls.append(np.zeros(G)); os_.append(np.zeros((G, d)))
                    continue
                seg = sc_rows[:, a:b]
                m = seg.max(axis=1)
                p = np.exp(seg - m[:, None])
                ms.append(m); ls.append(p.sum(axis=1)); os_.append(p @ v[a:b])
            M = np.max(np.stack(ms), axis=0)
            w = [np.exp(m - M) for m in ms]
            num = sum(wj[:, None] * oj for wj, oj in zip(w, os_))
            den = sum(wj * lj for wj, lj in zip(w, ls))
            out[s, hs] = num / den[:, None]
    return out


def chunked_prefill(q_i8, q_scale, cu_seqlens_q, context_lens, caches, block_tables,
                    num_kv_heads, scale=None, v_dtype="bf16", rows=None, heads=None):
    """Chunked prefill over a paged history ([QK-MMAC] §5.2).

    Sequence s has Tq = cu[s+1] - cu[s] new query tokens, the last Tq of its
    ctx = context_lens[s] cached tokens. Query i of the chunk sits at absolute
    position ctx - Tq + i and sees keys t <= that position (history first,
    then causal within the chunk). Rows are query tokens; the KV head is
    q_head // G. ``rows`` (global query indices) and ``heads`` restrict the
    outputs computed. Returns fp64 [Tq_total, Hq, d].
    """
    T, Hq, d = q_i8.shape
    G = Hq // num_kv_heads
    sc = _scale(scale, d)
    out = np.zeros((T, Hq, d), np.float64)
    want = None if rows is None else set(int(r) for r in rows)
    for s in range(len(context_lens)):
        a, b = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        ctx, tq = int(context_lens[s]), b - a
        sel = [i for i in range(a, b) if want is None or i in want]
        if not sel or ctx == 0:
            continue
        sel = np.asarray(sel)
        pos = ctx - tq + (sel - a)                                     # absolute positions
        visible = np.arange(ctx)[None, :] <= pos[:, None]              # [rows, ctx]
        for kvh in range(num_kv_heads):
            kq, sk, v = gather_kv(caches, block_tables[s], ctx, kvh, v_dtype)
            for h in range(kvh * G, (kvh + 1) * G):
                if heads is not None and h not in heads:
                    continue
                acc = _int_dot(q_i8[sel, h], kq)                        # [rows, ctx]
                s_ = acc * q_scale[sel, h].astype(np.float64)[:, None] * sk.astype(np.float64)[None, :] * sc
                s_ = np.where(visible, s_, -np.inf)
                out[sel, h] = _softmax_pv(s_, v)
    return out


def dense_sage_attention(quant, v_bits, dtype="f16", causal=False, scale=None,
                         q_block=128, k_block=64, rows=None, heads=None, batches=None,
                         return_lse=False):
    """SageAttention-style dense attention on pre-quantized NHD inputs.

    ``quant`` is the dict from ``sage_quantize``. [SAGE-MACA] (compute
    pipeline of the attention kernel): INT8 QK to INT32, scaled by the
    query-block scale, the key-block scale and the softmax scale; online
    softmax; P.V with fp16 V. Here the softmax and P.V are exact fp64 on the
    same recovered scores. Causal: query i sees key j <= i + (Nk - Nq)
    (bottom-right alignment; identical to top-left when Nq == Nk).
    Returns fp64 [B, Nq, Hq, d]; with ``return_lse`` also the natural-log
    sum of exponentials of each row's visible scores, fp64 [B, Hq, Nq] (-inf
    for a row that sees no key): [SAGE-MACA] feature matrix "LSE return".
    """
    q_i8, k_i8 = quant["q_i8"], quant["k_i8"]
    B, Nq, Hq, d = q_i8.shape
    Nk, Hkv = k_i8.shape[1], k_i8.shape[2]
    G = Hq // Hkv
    sc = _scale(scale, d)
    v = widen(v_bits, dtype).astype(np.float64)
    out = np.zeros((B, Nq, Hq, d), np.float64)
    lse = np.full((B, Hq, Nq), -np.inf)
    qr = np.arange(Nq) if rows is None else np.asarray(rows)
    qblk = qr // q_block
    kblk = np.arange(Nk) // k_block
    vis = None
    if causal:
        vis = np.arange(Nk)[None, :] <= (qr[:, None] + (Nk - Nq))
    for b in range(B):
        if batches is not None and b not in batches:
            continue
        for h in range(Hq):
            if heads is not None and h not in heads:
                continue
            kvh = h // G
            acc = _int_dot(q_i8[b, qr, h], k_i8[b, :, kvh])
            s_ = (acc * quant["q_scale"][b, h, qblk].astype(np.float64)[:, None]
                  * quant["k_scale"][b, kvh, kblk].astype(np.float64)[None, :] * sc)
            if vis is not None:
                s_ = np.where(vis, s_, -np.inf)
            out[b, qr, h] = _softmax_pv(s_, v[b, :, kvh])
            if return_lse:
                lse[b, h, qr] = _logsumexp_rows(s_)
    return (out, lse) if return_lse else out


def sage_smooth_v(v_bits, dtype="f16"):
    """V mean fusion ([SAGE-MACA] feature matrix "smooth_v"; the V mean
    subtraction kernel; compute-pipeline step 8 adds the mean back).

    The pages fix neither precision; reading taken, as for smooth_k: the
    per-(b, h, c) sum over all N tokens in fp64, divided by N in fp64 and
    rounded to fp32 (mu_v); V' = fl16(fl32(V) - mu_v), i.e. the fp32
    difference rounded to the fp16 operand of the P.V product. Since every
    softmax row sums to 1, attention(P, V) = attention(P, V') + mu_v up to
    the fp16 rounding of V'. Returns (V' as fp16 bit patterns, mu_v fp32
    [B, Hkv, d])."""
    v = widen(v_bits, dtype)
    B, N, H, d = v.shape
    if N > 0:
        mu = (v.astype(np.float64).sum(axis=1) / np.float64(N)).astype(np.float32)
    else:
        mu = np.zeros((B, H, d), np.float32)
    vp = (v - mu[:, None, :, :]).astype(np.float32)
    return vp.astype(np.float16).view(np.uint16), mu


def sage_lse_correction(q_bits, k_mean, dtype="f16", scale=None):
    """smooth_k shifts every score of query row i by -q_i . mu * scale
    (K' = K - mu), so the LSE of the smoothed scores is corrected by adding
    it back ([SAGE-MACA] feature matrix: smooth_k "with LSE correction"):
    corr[b, h, i] = scale * sum_c q[b, i, h, c] * mu[b, h // G, c], with the
    unquantized q (fp32 values) and mu (fp32), evaluated in fp64.
    Returns fp64 [B, Hq, Nq]."""
    q = widen(q_bits, dtype).astype(np.float64)
    B, Nq, Hq, d = q.shape
    Hkv = k_mean.shape[1]
    G = Hq // Hkv
    sc = _scale(scale, d)
    mu = np.repeat(np.asarray(k_mean, np.float64), G, axis=1)        # [B, Hq, d]
    return np.einsum("bnhc,bhc->bhn", q, mu) * sc


def sage_forward(q_bits, k_bits, v_bits, dtype="f16", causal=False, smooth_k=True, smooth_v=False,
                 return_lse=False, scale=None):
    """The whole dense call with its options ([SAGE-MACA] API: smooth_k,
    smooth_v, return_lse; NHD inputs, the HND layout is the same tensors
    transposed): quantize (smooth_k), optionally smooth V, attend, add the V
    mean back on rows that see a key, and correct the LSE for the K mean.
    Returns out fp64 [B, Nq, Hq, d] (and lse fp64 [B, Hq, Nq])."""
    from .quant import sage_quantize
    quant = sage_quantize(q_bits, k_bits, dtype, smooth_k=smooth_k)
    vb, vdt = v_bits, dtype
    if smooth_v:
        vb, mu_v = sage_smooth_v(v_bits, dtype)
        vdt = "f16"
    out, lse = dense_sage_attention(quant, vb, vdt, causal=causal, scale=scale, return_lse=True)
    if smooth_v:
        B, Nq, Hq, d = out.shape
        G = Hq // mu_v.shape[1]
        mu = np.repeat(mu_v.astype(np.float64), G, axis=1)            # [B, Hq, d]
        live = np.isfinite(lse).transpose(0, 2, 1)[..., None]         # [B, Nq, Hq, 1]
        out = out + np.where(live, mu[:, None, :, :], 0.0)
    if smooth_k:
        lse = lse + sage_lse_correction(q_bits, quant["k_mean"], dtype, scale)
    return (out, lse) if return_lse else out


def sage_varlen_forward(q_bits, k_bits, v_bits, cu_seqlens_q, cu_seqlens_k, dtype="f16", causal=False,
                        smooth_k=True, smooth_v=False, return_lse=False, scale=None):
    """Variable-length dense forward on packed rows ([SAGE-MACA] API
    sageattn_varlen; its implementation section: every batch element is
    sliced out and attended on its own). q [total_q, Hq, d], k and v
    [total_k, Hkv, d]; sequence b is rows cu_q[b]:cu_q[b+1] of q and
    cu_k[b]:cu_k[b+1] of k and v, attended exactly as a one-sequence
    ``sage_forward`` (its own smoothing means, its own 128/64-row quantization
    blocks, causal alignment within the sequence). Returns out fp64
    [total_q, Hq, d] (and lse fp64 [Hq, total_q])."""
    q = np.asarray(q_bits)
    k = np.asarray(k_bits)
    v = np.asarray(v_bits)
    cq = np.asarray(cu_seqlens_q, np.int64)
    ck = np.asarray(cu_seqlens_k, np.int64)
    Tq, Hq, d = q.shape
    out = np.zeros((Tq, Hq, d), np.float64)
    lse = np.full((Hq, Tq), -np.inf)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0:
            continue
        o, l = sage_forward(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], dtype, causal=causal,
                            smooth_k=smooth_k, smooth_v=smooth_v, return_lse=True, scale=scale)
        out[q0:q1] = o[0]
        lse[:, q0:q1] = l[0]
    return (out, lse) if return_lse else out


def attention_fp64(q, k, v, scale, visible=None):
    """Textbook softmax(q k^T * scale) v in fp64 for [N, d] operands, with an
    optional boolean visibility mask [Nq, Nk]. Used for pins and for the
    error of the quantized method against unquantized attention."""
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    return _softmax_pv(s, np.asarray(v, np.float64))
