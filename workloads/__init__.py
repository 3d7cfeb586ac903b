"""Seeded synthetic workloads for INT8-QK paged and dense attention.

This module only draws inputs. It holds none of the method's arithmetic:
no quantization, no scores, no softmax. It is shared by the CPU oracle
tests and the GPU path (tests, benchmark), so both sides consume the
same bit patterns.

Every draw comes from ``numpy.random.default_rng`` seeded with a tuple
``(config_seed, stream, index)``, so one sequence's data can be
regenerated without drawing the others.

Distributions follow the workloads the pages measure on: Qwen3.5-27B
attention shapes (24 query heads, 4 KV heads, head_dim 256) and the
SageAttention dense setting. Real activations are not available, so K
gets a per-(head, channel) bias to imitate the channel outliers that
motivate smoothing. "N(0, s)" is read as standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_SIZE = 16

# ---------------------------------------------------------------------------
# float32 draws -> 16-bit storage formats (round to nearest even)
# ---------------------------------------------------------------------------


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    raw 16-bit patterns as uint16. Inputs are finite draws."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (numpy's cast is round-to-nearest-even);
    return the raw 16-bit patterns as uint16."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit patterns to float32 (for reporting only)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    raise ValueError(dtype)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else to_f16_bits(x)


# ---------------------------------------------------------------------------
# Paged workloads (decode and chunked prefill)
# ---------------------------------------------------------------------------


@dataclass
class PagedSpec:
    """Shape of a paged-attention workload."""
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context_lens: list            # KV length per sequence (incl. new tokens)
    query_lens: list              # new query tokens per sequence (1 = decode)
    k_bias_std: float = 0.0       # std of the per-(kv head, channel) K bias
    v_int8: bool = False          # V cache stored as INT8 + per-token scale
    num_splits: int = 1
    dtype: str = "bf16"
    pool_blocks: Optional[int] = None   # physical pool; default = blocks needed

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def blocks_per_seq(self) -> list:
        return [-(-c // BLOCK_SIZE) for c in self.context_lens]

    @property
    def max_blocks_per_seq(self) -> int:
        return max(max(self.blocks_per_seq), 1)

    @property
    def num_blocks(self) -> int:
        need = sum(self.blocks_per_seq)
        return max(self.pool_blocks or need, need, 1)

    @property
    def total_q(self) -> int:
        return int(sum(self.query_lens))


@dataclass
class PagedInputs:
    spec: PagedSpec
    q: np.ndarray                 # [total_q, Hq, d] uint16 bits
    k: np.ndarray                 # [total_kv, Hkv, d] uint16 bits (all tokens of all seqs)
    v: np.ndarray                 # [total_kv, Hkv, d] uint16 bits
    slot_mapping: np.ndarray      # [total_kv] int64: block * 16 + offset
    block_tables: np.ndarray      # [num_seqs, max_blocks_per_seq] int32
    context_lens: np.ndarray      # [num_seqs] int32
    cu_seqlens_q: np.ndarray      # [num_seqs + 1] int32
    cu_seqlens_kv: np.ndarray     # [num_seqs + 1] int64 (token offsets into k/v)
    k_bias: np.ndarray = field(default=None)  # [Hkv, d] float32 (reporting)


def paged_inputs(spec: PagedSpec, seqs: Optional[list] = None) -> PagedInputs:
    """Draw a paged workload. Block tables are slices of one seeded
    permutation of the physical pool, so logical blocks of one sequence
    land on scattered physical blocks.

    ``seqs`` restricts the K/V/Q draws to a subset of sequences (others are
    left as zeros); tables and lengths are always complete. Each sequence
    uses its own generator stream, so a subset equals the full draw there.
    """
    S, Hq, Hkv, d = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    assert len(spec.context_lens) == S and len(spec.query_lens) == S
    nb = spec.num_blocks
    perm = _rng(spec.seed, 0).permutation(nb).astype(np.int32)
    mb = spec.max_blocks_per_seq
    tables = np.zeros((S, mb), np.int32)
    pos = 0
    for s, nbs in enumerate(spec.blocks_per_seq):
        tables[s, :nbs] = perm[pos:pos + nbs]
        pos += nbs
    bias = (_rng(spec.seed, 1).standard_normal((Hkv, d), dtype=np.float32)
            * np.float32(spec.k_bias_std)).astype(np.float32)
    ctx = np.asarray(spec.context_lens, np.int64)
    cu_kv = np.zeros(S + 1, np.int64)
    cu_kv[1:] = np.cumsum(ctx)
    cu_q = np.zeros(S + 1, np.int32)
    cu_q[1:] = np.cumsum(np.asarray(spec.query_lens, np.int64))
    total_kv = int(cu_kv[-1])
    k = np.zeros((total_kv, Hkv, d), np.uint16)
    v = np.zeros((total_kv, Hkv, d), np.uint16)
    q = np.zeros((int(cu_q[-1]), Hq, d), np.uint16)
    slots = np.zeros(total_kv, np.int64)
    for s in range(S):
        c = int(ctx[s])
        t = np.arange(c, dtype=np.int64)
        slots[cu_kv[s]:cu_kv[s + 1]] = tables[s, t // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + t % BLOCK_SIZE
        if seqs is not None and s not in seqs:
            continue
        g = _rng(spec.seed, 2, s)
        kf = g.standard_normal((c, Hkv, d), dtype=np.float32)
        kf += bias[None]
        k[cu_kv[s]:cu_kv[s + 1]] = _store(kf, spec.dtype)
        del kf
        v[cu_kv[s]:cu_kv[s + 1]] = _store(g.standard_normal((c, Hkv, d), dtype=np.float32), spec.dtype)
        q[cu_q[s]:cu_q[s + 1]] = _store(
            g.standard_normal((spec.query_lens[s], Hq, d), dtype=np.float32), spec.dtype)
    return PagedInputs(spec, q, k, v, slots, tables, ctx.astype(np.int32), cu_q, cu_kv, bias)


# ---------------------------------------------------------------------------
# Dense (SageAttention-style) workloads
# ---------------------------------------------------------------------------


@dataclass
class DenseSpec:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    k_bias_std: float = 0.0
    dtype: str = "f16"
    layout: str = "NHD"
    v_bias_std: float = 0.0   # per-(KV head, channel) offset of V, drawn from its own stream


@dataclass
class DenseInputs:
    spec: DenseSpec
    q: np.ndarray   # NHD: [B, Nq, Hq, d] uint16 bits
    k: np.ndarray   # [B, Nk, Hkv, d]
    v: np.ndarray   # [B, Nk, Hkv, d]


def dense_inputs(spec: DenseSpec) -> DenseInputs:
    """Q ~ N(0,1); K ~ N(0,1) + bias[head, channel], bias ~ N(0, k_bias_std);
    V ~ N(0,1) (+ a per-(head, channel) offset ~ N(0, v_bias_std) when that is
    set). Stored NHD (batch, seq, head, dim)."""
    B, Hq, Hkv, d = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    bias = _rng(spec.seed, 1).standard_normal((Hkv, d), dtype=np.float32) * np.float32(spec.k_bias_std)
    vbias = _rng(spec.seed, 3).standard_normal((Hkv, d), dtype=np.float32) * np.float32(spec.v_bias_std)
    q = np.empty((B, spec.seq_q, Hq, d), np.uint16)
    k = np.empty((B, spec.seq_k, Hkv, d), np.uint16)
    v = np.empty((B, spec.seq_k, Hkv, d), np.uint16)
    for b in range(B):
        g = _rng(spec.seed, 2, b)
        q[b] = _store(g.standard_normal((spec.seq_q, Hq, d), dtype=np.float32), spec.dtype)
        k[b] = _store(g.standard_normal((spec.seq_k, Hkv, d), dtype=np.float32) + bias[None], spec.dtype)
        vx = g.standard_normal((spec.seq_k, Hkv, d), dtype=np.float32)
        v[b] = _store(vx + vbias[None] if spec.v_bias_std else vx, spec.dtype)
    return DenseInputs(spec, q, k, v)


@dataclass
class VarlenSpec:
    """Packed variable-length dense inputs: sequence b has seq_q[b] query
    rows and seq_k[b] key/value rows."""
    name: str
    seed: int
    seq_q: list
    seq_k: list
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    k_bias_std: float = 3.0
    dtype: str = "f16"
    v_bias_std: float = 0.0


@dataclass
class VarlenInputs:
    spec: VarlenSpec
    q: np.ndarray       # [total_q, Hq, d] uint16 bits
    k: np.ndarray       # [total_k, Hkv, d]
    v: np.ndarray
    cu_q: np.ndarray    # [B+1] int32 row offsets
    cu_k: np.ndarray


def varlen_inputs(spec: VarlenSpec) -> VarlenInputs:
    """The dense recipe per sequence (Q ~ N(0,1); K ~ N(0,1) + a per-(head,
    channel) bias shared by all sequences; V ~ N(0,1) + optional offset),
    packed row after row."""
    Hq, Hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    bias = _rng(spec.seed, 1).standard_normal((Hkv, d), dtype=np.float32) * np.float32(spec.k_bias_std)
    vbias = _rng(spec.seed, 3).standard_normal((Hkv, d), dtype=np.float32) * np.float32(spec.v_bias_std)
    qs, ks, vs = [], [], []
    for b, (nq, nk) in enumerate(zip(spec.seq_q, spec.seq_k)):
        g = _rng(spec.seed, 2, b)
        qs.append(_store(g.standard_normal((nq, Hq, d), dtype=np.float32), spec.dtype))
        ks.append(_store(g.standard_normal((nk, Hkv, d), dtype=np.float32) + bias[None], spec.dtype))
        vx = g.standard_normal((nk, Hkv, d), dtype=np.float32)
        vs.append(_store(vx + vbias[None] if spec.v_bias_std else vx, spec.dtype))
    cu = lambda n: np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    cat = lambda xs, H: np.concatenate(xs) if xs else np.zeros((0, H, d), np.uint16)
    return VarlenInputs(spec, cat(qs, Hq), cat(ks, Hkv), cat(vs, Hkv), cu(spec.seq_q), cu(spec.seq_k))


def rope_table(max_position: int, rot_dim: int, base: float = 1.0e6) -> np.ndarray:
    """Rotary-embedding input table [max_position, rot_dim] fp32: cos(p * w_i)
    in columns [0, rot_dim/2), sin(p * w_i) in [rot_dim/2, rot_dim), with
    w_i = base^(-2i / rot_dim), evaluated in fp64 and rounded to fp32. The
    pages give no rotary parameters; base 1e6 is a stand-in."""
    half = rot_dim // 2
    w = base ** (-np.arange(half, dtype=np.float64) * 2.0 / rot_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def dense_zero_scale_inputs(N: int = 200, d: int = 64, dtype: str = "f16") -> DenseInputs:
    """Degenerate dense inputs: KV head 0 holds the same key at every position
    (smoothing then leaves all-zero keys, so every key-block scale is 0) and
    query head 1 has an all-zero block of query rows 128..255 (query scale 0).
    B 1, 4 query heads over 2 KV heads."""
    spec = DenseSpec("dense_zero_scale", 41, 1, 4, 2, N, N, d, k_bias_std=1.0, dtype=dtype)
    inp = dense_inputs(spec)
    inp.k[:, :, 0, :] = inp.k[:, :1, 0, :]
    inp.q[:, 128:256, 1, :] = 0
    return inp


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------


def tiny_decode() -> PagedSpec:
    """Batch 1, one query token, 6 query heads over 1 KV head, head_dim 64,
    context 256: 16 blocks of 16 tokens in permuted order."""
    return PagedSpec("tiny_decode", 1, 1, 6, 1, 64, [256], [1])


def qwen27b_decode(context: int = 32768) -> PagedSpec:
    """Qwen3.5-27B full-attention shape: 24 query heads, 4 KV heads (GQA 6:1),
    head_dim 256, one query token over `context` cached tokens. K has a
    per-channel bias of std 2. The pool holds exactly the blocks in use."""
    return PagedSpec("qwen27b_decode", 2, 1, 24, 4, 256, [context], [1], k_bias_std=2.0)


def batched_splitk_decode(num_seqs: int = 32, lo: int = 1024, hi: int = 32768,
                          num_splits: int = 8) -> PagedSpec:
    """32 sequences with context lengths uniform on [1024, 32768] (integers, so
    most tails are partial blocks), 24/4 heads, head_dim 256, INT8 K and V,
    8 split-K segments per sequence."""
    ctx = _rng(3, 9).integers(lo, hi + 1, size=num_seqs).tolist()
    return PagedSpec("batched_splitk_decode", 3, num_seqs, 24, 4, 256, ctx, [1] * num_seqs,
                     k_bias_std=2.0, v_int8=True, num_splits=num_splits)


def chunked_prefill(history: int = 16384, chunk: int = 2048) -> PagedSpec:
    """One sequence: `chunk` new query tokens after `history` cached tokens;
    the KV length is history + chunk and the chunk attends causally."""
    return PagedSpec("chunked_prefill", 4, 1, 24, 4, 256, [history + chunk], [chunk], k_bias_std=2.0)


def dense_sage(seq: int = 8192, batch: int = 2, heads: int = 32, head_dim: int = 128) -> DenseSpec:
    """SageAttention-style dense forward: batch 2, 32 heads (1:1), seq 8192,
    head_dim 128, NHD, fp16 Q/K/V; K has a per-channel bias of std 3."""
    return DenseSpec("dense_sage", 5, batch, heads, heads, seq, seq, head_dim, k_bias_std=3.0)
