"""CPU oracle for INT8-QK quantized attention: TEST INFRASTRUCTURE ONLY.

The oracle is plain C++17 (quant.cpp, attention.cpp, sage.cpp; interface
oracle.h) built with g++ -O2 -fno-fast-math -ffp-contract=off into
liboracle.so. This module only marshals numpy arrays to it through ctypes:
every step of the arithmetic runs in the C++ code. Only the test suite, the
smoke check in __graft_entry__ and the CPU-baseline leg of bench.py import
it. The GPU library never imports, links or calls it, and it shares no code
with the GPU path: the only common module is the seeded input generator
(workloads/), which holds none of the method's arithmetic.

Sources (the pages this work follows):

* [QK-MMAC] "gfx936 DCU上实现INT8 QK MMAC：分页访存、Fragment映射与GQA适配"
  (INT8 QK MMAC on the gfx936 DCU: paged access, fragment mapping and GQA).
* [SAGE-MACA] "SageAttention — MetaX MXMACA 平台移植版 (v3.0.0)" README.

Precision: quantization follows the pages in IEEE fp32 (one correctly
rounded operation per step, round-half-even). Everything after the INT32
accumulator (score recovery, softmax, P.V) is fp64, since the pages fix no
precision there.

Parity status, function by function (pins live in tests/test_oracle_pins.py,
planted mistakes in tests/test_oracle_mutations.py):

* quant_rows, quantize_q, write_kv_cache, gather_kv, sage_quantize: pinned
  (worked rounding ties, correctly rounded scale, arg-max maps to +-127,
  error bound, zero rows, element-wise layout, brute force per block, exact
  smoothing mean).
* paged_qk_int32: pinned (INT32 bound 256*127*127, brute force in int64).
* paged_decode, paged_decode_split, split_segments, chunked_prefill,
  dense_sage_attention: pinned (rows sum to one, equality with a textbook
  fp64 attention of the dequantized tensors through scipy, split = unsplit,
  smoothing invariance, causal structure).
* sage_smooth_v, sage_lse_correction, sage_forward, sage_varlen_forward:
  pinned (closed forms for the LSE, the V mean added back, equal-length
  varlen = batched, independence of sequences).
* apply_rope, rope_quantize_q, rope_write_kv_cache: pinned (identity at
  position 0, complex multiplication, pairing equivalence, relative
  position property).
* e4m3_encode / e4m3_decode, f32_to_f16_bits: pinned (landmark values, ties,
  saturation, torch's float8_e4m3fn and numpy's float16 conversions).
* v_fp8_per_channel, dense_sage_attention_fp8pv: pinned (constant V comes
  back exactly; one visible key; a two-key closed form; equal scores give
  ln(#visible); within the E4M3 error of the 16-bit path; the tolerance
  model matched by randomized references).
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DT = {"bf16": 0, "f16": 1}
BLOCK = 16

_vp, _i32, _i64, _f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double


class _Paged(ctypes.Structure):
    _fields_ = [("k_cache", _vp), ("k_scale", _vp), ("v_cache", _vp), ("v_scale", _vp), ("v_dtype", _i32),
                ("tables", _vp), ("max_blocks", _i32), ("num_seqs", _i32), ("Hq", _i32), ("Hkv", _i32),
                ("d", _i32)]


class _Dense(ctypes.Structure):
    _fields_ = [("B", _i32), ("Nq", _i32), ("Nk", _i32), ("Hq", _i32), ("Hkv", _i32), ("d", _i32),
                ("q_block", _i32), ("k_block", _i32)]


_P = ctypes.POINTER
_SIGS = {
    "or_widen": [_vp, _i32, _i64, _vp],
    "or_f32_to_f16_bits": [_vp, _i64, _vp],
    "or_e4m3_encode": [_vp, _i64, _vp],
    "or_e4m3_decode": [_vp, _i64, _vp],
    "or_quant_rows": [_vp, _i64, _i64, _vp, _vp],
    "or_write_kv": [_vp, _vp, _i32, _i32, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp],
    "or_gather_kv": [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp],
    "or_apply_rope": [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _i32, _vp],
    "or_paged_qk_int32": [_P(_Paged), _vp, _vp, _vp],
    "or_paged_decode": [_P(_Paged), _vp, _vp, _vp, _f64, _vp, _vp],
    "or_split_segments": [_i32, _i32, _vp],
    "or_paged_decode_split": [_P(_Paged), _vp, _vp, _vp, _f64, _i32, _vp],
    "or_chunked_prefill": [_P(_Paged), _vp, _vp, _vp, _vp, _i64, _f64, _vp, _vp, _vp],
    "or_attention_fp64": [_vp, _vp, _vp, _i64, _i64, _i32, _f64, _vp, _vp],
    "or_paged_v_fp8": [_P(_Paged), _i32, _i32, _i32, _vp, _vp],
    "or_chunked_prefill_fp8pv": [_P(_Paged), _vp, _vp, _vp, _vp, _i64, _f64, _vp, _vp, _vp, _vp],
    "or_set_num_threads": [_i32],
    "or_max_threads": [],
    "or_sage_quantize": [_P(_Dense), _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp],
    "or_dense_attention": [_P(_Dense), _vp, _vp, _vp, _vp, _vp, _i32, _f64, _vp, _i64, _vp, _vp, _vp, _vp],
    "or_sage_smooth_v": [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp],
    "or_sage_lse_correction": [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _f64, _vp],
    "or_sage_forward": [_P(_Dense), _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f64, _vp, _vp],
    "or_sage_varlen_forward": [_vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f64, _vp,
                               _vp],
    "or_v_fp8_per_channel": [_vp, _i32, _i32, _i32, _i32, _vp, _vp],
    "or_dense_attention_fp8pv": [_P(_Dense), _vp, _vp, _vp, _vp, _vp, _i32, _f64, _i32, _vp, _i64, _vp, _vp, _vp,
                                 _vp, _vp],
    "or_dense_attention_fp8pv_lazy": [_P(_Dense), _vp, _vp, _vp, _vp, _vp, _i32, _f64, _i32, _i32, _f64, _i32,
                                      _vp, _vp],
}


def build_library(src_dir: str = _HERE, out: str = LIB_PATH) -> str:
    """Compile the C++ sources of src_dir into `out` (oracle/build.py)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("oracle_build", os.path.join(_HERE, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build(src_dir, out)


def load_library(path: str):
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = None
        fn.argtypes = args
    lib.or_max_threads.restype = _i32
    return lib


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (results do not depend on it)."""
    _L().or_set_num_threads(int(n))


def max_threads() -> int:
    return int(_L().or_max_threads())


_lib = None


def _stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    built = os.path.getmtime(LIB_PATH)
    srcs = [f for f in os.listdir(_HERE) if f.endswith((".cpp", ".h"))]
    return any(os.path.getmtime(os.path.join(_HERE, f)) > built for f in srcs)


def _L():
    global _lib
    if _lib is None:
        if _stale():
            build_library()
        _lib = load_library(LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Run the oracle from another build of its sources (the mutation tests
    use this for builds with a planted mistake)."""
    global _lib
    saved = _lib
    _lib = load_library(path)
    try:
        yield
    finally:
        _lib = saved


# ---- marshalling helpers ------------------------------------------------------

def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


def _mask(sel, n):
    """Boolean selection as a uint8 mask of length n (None = everything)."""
    if sel is None:
        return None
    m = np.zeros(n, np.uint8)
    m[np.asarray(list(sel), np.int64)] = 1
    return m


def _scale_arg(scale):
    return float(scale) if scale is not None and scale > 0 else 0.0


def default_scale(head_dim: int) -> float:
    """softmax scale 1/sqrt(d) ([QK-MMAC] §1; [SAGE-MACA] advanced options)."""
    return 1.0 / math.sqrt(head_dim)


# ---- storage formats ----------------------------------------------------------

def widen(bits, dtype: str) -> np.ndarray:
    """16-bit storage patterns (bf16 or f16) -> the fp32 values they denote."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float32)
    _L().or_widen(_p(b), _DT[dtype], b.size, _p(out))
    return out


def f32_to_f16_bits(x) -> np.ndarray:
    """fp32 values -> nearest IEEE binary16 (ties to even) as uint16 bits."""
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint16)
    _L().or_f32_to_f16_bits(_p(a), a.size, _p(out))
    return out


def e4m3_encode(x) -> np.ndarray:
    """float values -> E4M3 codes (uint8): nearest finite value, ties to the
    even code, magnitudes above 448 to 448, the sign kept."""
    a = _c(x, np.float64)
    out = np.empty(a.shape, np.uint8)
    _L().or_e4m3_encode(_p(a), a.size, _p(out))
    return out


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes -> float64 values (NaN for the two NaN codes)."""
    a = _c(codes, np.uint8)
    out = np.empty(a.shape, np.float64)
    _L().or_e4m3_decode(_p(a), a.size, _p(out))
    return out


def e4m3_round(x) -> np.ndarray:
    """The E4M3 value nearest to x (float64)."""
    return e4m3_decode(e4m3_encode(x))


# ---- quantization and the paged cache -----------------------------------------

def quant_rows(x):
    """Symmetric INT8 of each row (last axis): s = fl32(max|x| / 127),
    q = clamp(rne(fl32(x / s)), -127, 127); s = 0 and zero codes for an
    all-zero row ([QK-MMAC] §4, §2.1). Returns (codes int8, scales fp32)."""
    a = _c(x, np.float32)
    n = a.shape[-1]
    rows = a.size // n if n else 0
    q = np.empty(a.shape, np.int8)
    s = np.empty(a.shape[:-1], np.float32)
    _L().or_quant_rows(_p(a), rows, n, _p(q), _p(s))
    return q, s


def quantize_q(q_bits, dtype: str = "bf16"):
    """Per-(token, query head) quantization of Q [T, Hq, d] ([QK-MMAC] §1,
    §4). Returns (q_i8 [T, Hq, d], q_scale [T, Hq])."""
    return quant_rows(widen(q_bits, dtype))


def _new_caches(num_blocks, H, d, v_int8):
    return {
        "k_cache": np.zeros((num_blocks, H, d // 16, BLOCK, 16), np.int8),
        "k_scale": np.zeros((num_blocks, H, BLOCK), np.float32),
        "v_cache": np.zeros((num_blocks, H, d, BLOCK), np.int8 if v_int8 else np.uint16),
        "v_scale": np.zeros((num_blocks, H, BLOCK), np.float32) if v_int8 else None,
    }


def write_kv_values(k_vals, v_bits, dtype, slot_mapping, num_blocks, v_int8=False, caches=None):
    """Quantize fp32 K values (and V if v_int8) per (token, KV head) and
    scatter them into the paged cache ([QK-MMAC] §1, §3). ``caches`` (a dict
    from an earlier call) is updated in place; otherwise zero caches are made."""
    k = _c(k_vals, np.float32)
    T, H, d = k.shape
    if caches is None:
        caches = _new_caches(num_blocks, H, d, v_int8)
    v = _c(v_bits, np.uint16)
    slots = _c(slot_mapping, np.int64)
    for key in ("k_cache", "k_scale", "v_cache", "v_scale"):
        if caches[key] is not None:
            assert caches[key].flags.c_contiguous
    _L().or_write_kv(_p(k), _p(v), _DT[dtype], int(v_int8), _p(slots), T, H, d, _p(caches["k_cache"]),
                     _p(caches["k_scale"]), _p(caches["v_cache"]), _p(caches["v_scale"]))
    return caches


def write_kv_cache(k_bits, v_bits, dtype, slot_mapping, num_blocks, v_int8=False, caches=None):
    """write_kv_values of the 16-bit K inputs."""
    return write_kv_values(widen(k_bits, dtype), v_bits, dtype, slot_mapping, num_blocks, v_int8, caches)


def gather_kv(caches, table_row, ctx, kv_head, v_dtype="bf16"):
    """A sequence's first ``ctx`` tokens of one KV head read back through its
    block table ([QK-MMAC] §3). Returns (Kq [ctx, d] int8, sK [ctx] fp32,
    V [ctx, d] fp64 dequantized)."""
    kc = caches["k_cache"]
    H, d = kc.shape[1], kc.shape[2] * 16
    tab = _c(table_row, np.int32)
    kq = np.empty((ctx, d), np.int8)
    sk = np.empty(ctx, np.float32)
    v = np.empty((ctx, d), np.float64)
    _L().or_gather_kv(_p(kc), _p(caches["k_scale"]), _p(caches["v_cache"]), _p(caches.get("v_scale")),
                      _DT[v_dtype], H, d, _p(tab), int(ctx), int(kv_head), _p(kq), _p(sk), _p(v))
    return kq, sk, v


def apply_rope(x_bits, dtype, positions, cos_sin, rot_dim, neox=True):
    """Rotary embedding of [T, H, d] 16-bit inputs by the table rows of their
    positions, in fp32 without fused operations; returns fp32 [T, H, d]."""
    x = _c(x_bits, np.uint16)
    T, H, d = x.shape
    pos = _c(positions, np.int64)
    cs = _c(cos_sin, np.float32)
    out = np.empty(x.shape, np.float32)
    _L().or_apply_rope(_p(x), _DT[dtype], T, H, d, _p(pos), _p(cs), int(rot_dim), int(bool(neox)), _p(out))
    return out


def rope_quantize_q(q_bits, dtype, positions, cos_sin, rot_dim, neox=True):
    """Per-(token, head) INT8 of the rotated query. Returns (q_i8, q_scale)."""
    return quant_rows(apply_rope(q_bits, dtype, positions, cos_sin, rot_dim, neox))


def rope_write_kv_cache(k_bits, v_bits, dtype, slot_mapping, num_blocks, positions, cos_sin, rot_dim,
                        neox=True, v_int8=False, caches=None):
    """write_kv_cache with K rotated first (V as given)."""
    return write_kv_values(apply_rope(k_bits, dtype, positions, cos_sin, rot_dim, neox), v_bits, dtype,
                           slot_mapping, num_blocks, v_int8, caches)


# ---- paged attention -----------------------------------------------------------

def _paged(caches, block_tables, num_seqs, Hq, Hkv, d, v_dtype):
    tab = _c(block_tables, np.int32)
    keep = [tab]
    st = _Paged(_p(caches["k_cache"]), _p(caches["k_scale"]), _p(caches["v_cache"]), _p(caches.get("v_scale")),
                _DT[v_dtype], _p(tab), tab.shape[1] if tab.ndim == 2 else 1, num_seqs, Hq, Hkv, d)
    return st, keep


def paged_qk_int32(q_i8, caches, block_tables, context_lens, num_kv_heads):
    """INT32 QK accumulators of decode, one query token per sequence
    ([QK-MMAC] §2.1-§2.2): a list with one int64 array [Hq, ctx] per sequence."""
    q = _c(q_i8, np.int8)
    S, Hq, d = q.shape
    ctx = _c(context_lens, np.int32)
    st, keep = _paged(caches, block_tables, S, Hq, num_kv_heads, d, "bf16")
    acc = np.empty(int(sum(int(c) for c in ctx)) * Hq, np.int64)
    _L().or_paged_qk_int32(ctypes.byref(st), _p(q), _p(ctx), _p(acc))
    out, base = [], 0
    for c in ctx:
        out.append(acc[base:base + Hq * int(c)].reshape(Hq, int(c)))
        base += Hq * int(c)
    return out


def paged_decode(q_i8, q_scale, caches, block_tables, context_lens, num_kv_heads, scale=None, v_dtype="bf16",
                 heads=None):
    """Decode attention, one query token per sequence, unsplit ([QK-MMAC]
    §1-§5.1). ``heads`` limits the query heads computed (others zero).
    Returns fp64 [S, Hq, d]."""
    q = _c(q_i8, np.int8)
    S, Hq, d = q.shape
    qs = _c(q_scale, np.float32)
    ctx = _c(context_lens, np.int32)
    st, keep = _paged(caches, block_tables, S, Hq, num_kv_heads, d, v_dtype)
    hm = _mask(heads, Hq)
    out = np.empty((S, Hq, d), np.float64)
    _L().or_paged_decode(ctypes.byref(st), _p(q), _p(qs), _p(ctx), _scale_arg(scale), _p(hm), _p(out))
    return out


def split_segments(ctx: int, num_splits: int):
    """Split-K segments of a context: a list of (start, end) token ranges."""
    b = np.empty(2 * num_splits, np.int32)
    _L().or_split_segments(int(ctx), int(num_splits), _p(b))
    return [(int(b[2 * j]), int(b[2 * j + 1])) for j in range(num_splits)]


def paged_decode_split(q_i8, q_scale, caches, block_tables, context_lens, num_kv_heads, num_splits, scale=None,
                       v_dtype="bf16"):
    """Split-K decode and the merge of the segments ([QK-MMAC] §4)."""
    q = _c(q_i8, np.int8)
    S, Hq, d = q.shape
    qs = _c(q_scale, np.float32)
    ctx = _c(context_lens, np.int32)
    st, keep = _paged(caches, block_tables, S, Hq, num_kv_heads, d, v_dtype)
    out = np.empty((S, Hq, d), np.float64)
    _L().or_paged_decode_split(ctypes.byref(st), _p(q), _p(qs), _p(ctx), _scale_arg(scale), int(num_splits), _p(out))
    return out


def chunked_prefill(q_i8, q_scale, cu_seqlens_q, context_lens, caches, block_tables, num_kv_heads, scale=None,
                    v_dtype="bf16", rows=None, heads=None):
    """Chunked prefill over a paged history ([QK-MMAC] §5.2): query i of a
    chunk of Tq tokens sits at position ctx - Tq + i and sees keys up to it.
    ``rows`` (global query indices) and ``heads`` restrict the outputs.
    Returns fp64 [Tq_total, Hq, d]."""
    q = _c(q_i8, np.int8)
    T, Hq, d = q.shape
    qs = _c(q_scale, np.float32)
    cu = _c(cu_seqlens_q, np.int32)
    ctx = _c(context_lens, np.int32)
    st, keep = _paged(caches, block_tables, len(ctx), Hq, num_kv_heads, d, v_dtype)
    rm, hm = _mask(rows, T), _mask(heads, Hq)
    out = np.empty((T, Hq, d), np.float64)
    _L().or_chunked_prefill(ctypes.byref(st), _p(q), _p(qs), _p(cu), _p(ctx), T, _scale_arg(scale), _p(rm), _p(hm),
                            _p(out))
    return out


def paged_v_fp8(caches, block_tables, seq, ctx, kv_head, num_seqs, num_kv_heads, d, v_dtype="bf16"):
    """E4M3 codes [ctx, d] (uint8) and channel scales [d] (fp32) of the V of
    one (sequence, KV head) for the FP8 P.V product."""
    st, keep = _paged(caches, block_tables, num_seqs, num_kv_heads, num_kv_heads, d, v_dtype)
    codes = np.empty((int(ctx), d), np.uint8)
    scales = np.empty(d, np.float32)
    _L().or_paged_v_fp8(ctypes.byref(st), int(seq), int(ctx), int(kv_head), _p(codes), _p(scales))
    return codes, scales


def chunked_prefill_fp8pv(q_i8, q_scale, cu_seqlens_q, context_lens, caches, block_tables, num_kv_heads,
                          scale=None, v_dtype="bf16", rows=None, heads=None, return_sigma=False):
    """Chunked prefill with the P.V product in FP8 (E4M3): V per (sequence,
    KV head, channel) scaled to E4M3 over the sequence's cached tokens, per
    row P8 = E4M3(448 exp(s - m)) at the exact maximum m, out = sum P8 V8 /
    sum P8 * s_c. Returns fp64 [Tq_total, Hq, d]; with return_sigma also the
    standard deviations of the lazily referenced implementation."""
    q = _c(q_i8, np.int8)
    T, Hq, d = q.shape
    qs = _c(q_scale, np.float32)
    cu = _c(cu_seqlens_q, np.int32)
    ctx = _c(context_lens, np.int32)
    st, keep = _paged(caches, block_tables, len(ctx), Hq, num_kv_heads, d, v_dtype)
    rm, hm = _mask(rows, T), _mask(heads, Hq)
    out = np.empty((T, Hq, d), np.float64)
    sig = np.empty_like(out) if return_sigma else None
    _L().or_chunked_prefill_fp8pv(ctypes.byref(st), _p(q), _p(qs), _p(cu), _p(ctx), T, _scale_arg(scale), _p(rm),
                                  _p(hm), _p(out), _p(sig))
    return (out, sig) if return_sigma else out


def attention_fp64(q, k, v, scale, visible=None):
    """Textbook softmax(q k^T * scale) v in fp64 for [N, d] operands with an
    optional boolean visibility mask [Nq, Nk]."""
    q, k, v = _c(q, np.float64), _c(k, np.float64), _c(v, np.float64)
    vis = None if visible is None else _c(np.broadcast_to(visible, (q.shape[0], k.shape[0])), np.uint8)
    out = np.empty((q.shape[0], v.shape[1]), np.float64)
    _L().or_attention_fp64(_p(q), _p(k), _p(v), q.shape[0], k.shape[0], q.shape[1], float(scale), _p(vis), _p(out))
    return out


# ---- dense SageAttention-style path ---------------------------------------------

def _dense(B, Nq, Nk, Hq, Hkv, d, q_block=128, k_block=64):
    return _Dense(B, Nq, Nk, Hq, Hkv, d, q_block, k_block)


def sage_quantize(q_bits, k_bits, dtype="f16", smooth_k=True, q_block=128, k_block=64):
    """smooth_k and per-block INT8 of dense NHD Q [B, Nq, Hq, d] and K
    [B, Nk, Hkv, d] ([SAGE-MACA] quantization kernels, per_block). Returns
    dict q_i8, q_scale [B, Hq, ceil(Nq/qb)], k_i8, k_scale [B, Hkv,
    ceil(Nk/kb)], k_mean [B, Hkv, d]."""
    q, k = _c(q_bits, np.uint16), _c(k_bits, np.uint16)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = _dense(B, Nq, Nk, Hq, Hkv, d, q_block, k_block)
    res = {
        "q_i8": np.empty(q.shape, np.int8),
        "q_scale": np.empty((B, Hq, -(-Nq // q_block)), np.float32),
        "k_i8": np.empty(k.shape, np.int8),
        "k_scale": np.empty((B, Hkv, -(-Nk // k_block)), np.float32),
        "k_mean": np.empty((B, Hkv, d), np.float32),
    }
    _L().or_sage_quantize(ctypes.byref(g), _p(q), _p(k), _DT[dtype], int(bool(smooth_k)), _p(res["q_i8"]),
                          _p(res["q_scale"]), _p(res["k_i8"]), _p(res["k_scale"]), _p(res["k_mean"]))
    return res


def _quant_geometry(quant, q_block, k_block):
    q_i8, k_i8 = quant["q_i8"], quant["k_i8"]
    B, Nq, Hq, d = q_i8.shape
    Nk, Hkv = k_i8.shape[1], k_i8.shape[2]
    arrs = [_c(quant[n], t) for n, t in (("q_i8", np.int8), ("q_scale", np.float32), ("k_i8", np.int8),
                                          ("k_scale", np.float32))]
    return _dense(B, Nq, Nk, Hq, Hkv, d, q_block, k_block), arrs


def dense_sage_attention(quant, v_bits, dtype="f16", causal=False, scale=None, q_block=128, k_block=64, rows=None,
                         heads=None, batches=None, return_lse=False):
    """Dense attention on pre-quantized NHD inputs (the dict of
    sage_quantize): INT8 QK with block scales, exact softmax and P.V in fp64
    ([SAGE-MACA] attention pipeline). Causal: bottom-right alignment.
    Returns fp64 [B, Nq, Hq, d] (and lse [B, Hq, Nq] with return_lse)."""
    g, (q8, qs, k8, ks) = _quant_geometry(quant, q_block, k_block)
    v = _c(widen(v_bits, dtype), np.float64)
    r = None if rows is None else _c(rows, np.int64)
    hm, bm = _mask(heads, g.Hq), _mask(batches, g.B)
    out = np.empty((g.B, g.Nq, g.Hq, g.d), np.float64)
    lse = np.empty((g.B, g.Hq, g.Nq), np.float64)
    _L().or_dense_attention(ctypes.byref(g), _p(q8), _p(qs), _p(k8), _p(ks), _p(v), int(bool(causal)),
                            _scale_arg(scale), _p(r), 0 if r is None else r.size, _p(hm), _p(bm), _p(out), _p(lse))
    return (out, lse) if return_lse else out


def sage_smooth_v(v_bits, dtype="f16"):
    """smooth_v ([SAGE-MACA] feature matrix): returns (V' = fl16(fl32(V) -
    mu_v) as fp16 bits, mu_v fp32 [B, Hkv, d])."""
    v = _c(v_bits, np.uint16)
    B, N, H, d = v.shape
    vp = np.empty(v.shape, np.uint16)
    mu = np.empty((B, H, d), np.float32)
    _L().or_sage_smooth_v(_p(v), _DT[dtype], B, N, H, d, _p(vp), _p(mu))
    return vp, mu


def sage_lse_correction(q_bits, k_mean, dtype="f16", scale=None):
    """The smooth_k LSE correction scale * q . mu per row: fp64 [B, Hq, Nq]."""
    q = _c(q_bits, np.uint16)
    B, Nq, Hq, d = q.shape
    mu = _c(k_mean, np.float32)
    out = np.empty((B, Hq, Nq), np.float64)
    _L().or_sage_lse_correction(_p(q), _DT[dtype], _p(mu), B, Nq, Hq, mu.shape[1], d, _scale_arg(scale), _p(out))
    return out


def sage_forward(q_bits, k_bits, v_bits, dtype="f16", causal=False, smooth_k=True, smooth_v=False,
                 return_lse=False, scale=None):
    """The whole dense call with its options ([SAGE-MACA] API: smooth_k,
    smooth_v, return_lse). Returns out fp64 [B, Nq, Hq, d] (and lse fp64
    [B, Hq, Nq])."""
    q, k, v = _c(q_bits, np.uint16), _c(k_bits, np.uint16), _c(v_bits, np.uint16)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = _dense(B, Nq, Nk, Hq, Hkv, d)
    out = np.empty((B, Nq, Hq, d), np.float64)
    lse = np.empty((B, Hq, Nq), np.float64)
    _L().or_sage_forward(ctypes.byref(g), _p(q), _p(k), _p(v), _DT[dtype], int(bool(causal)), int(bool(smooth_k)),
                         int(bool(smooth_v)), _scale_arg(scale), _p(out), _p(lse))
    return (out, lse) if return_lse else out


def sage_varlen_forward(q_bits, k_bits, v_bits, cu_seqlens_q, cu_seqlens_k, dtype="f16", causal=False,
                        smooth_k=True, smooth_v=False, return_lse=False, scale=None):
    """Variable-length dense forward on packed rows ([SAGE-MACA]
    sageattn_varlen): each sequence attended as a one-sequence sage_forward.
    Returns out fp64 [total_q, Hq, d] (and lse fp64 [Hq, total_q])."""
    q, k, v = _c(q_bits, np.uint16), _c(k_bits, np.uint16), _c(v_bits, np.uint16)
    cq, ck = _c(cu_seqlens_q, np.int32), _c(cu_seqlens_k, np.int32)
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.empty((Tq, Hq, d), np.float64)
    lse = np.empty((Hq, Tq), np.float64)
    _L().or_sage_varlen_forward(_p(q), _p(k), _p(v), _DT[dtype], _p(cq), _p(ck), len(cq) - 1, Hq, Hkv, d,
                                int(bool(causal)), int(bool(smooth_k)), int(bool(smooth_v)), _scale_arg(scale), _p(out),
                                _p(lse))
    return (out, lse) if return_lse else out


# ---- FP8 (E4M3) P.V -----------------------------------------------------------

def v_fp8_per_channel(v_vals):
    """Per-(batch, KV head, channel) E4M3 of V over its tokens:
    s_c = fl32(max|V| / 448), values E4M3(fl32(V / s_c)). v_vals fp32
    [B, N, H, d]. Returns (values fp64, scales fp32 [B, H, d])."""
    v = _c(v_vals, np.float32)
    B, N, H, d = v.shape
    vals = np.empty(v.shape, np.float64)
    s = np.empty((B, H, d), np.float32)
    _L().or_v_fp8_per_channel(_p(v), B, N, H, d, _p(vals), _p(s))
    return vals, s


def dense_sage_attention_fp8pv(quant, v_bits, dtype="f16", causal=False, scale=None, smooth_v=False, rows=None,
                               heads=None, return_lse=False, return_sigma=False):
    """Dense attention with the P.V product in FP8 (E4M3), the plain
    definition: per row the exact maximum m of its scores and
    P8 = E4M3(448 exp(s - m)); V per channel in E4M3; out = sum P8 V8 /
    sum P8 * s_c (+ mu_v with smooth_v). Returns out fp64 [B, Nq, Hq, d];
    with return_lse also lse [B, Hq, Nq]; with return_sigma the tuple
    (out, lse, sigma [B, Nq, Hq, d], sigma_lse [B, Hq, Nq]): the standard
    deviations of an implementation that rounds P from a lazily moved
    reference (see or_dense_attention_fp8pv)."""
    g, (q8, qs, k8, ks) = _quant_geometry(quant, 128, 64)
    v = _c(widen(v_bits, dtype), np.float32)
    r = None if rows is None else _c(rows, np.int64)
    hm = _mask(heads, g.Hq)
    out = np.empty((g.B, g.Nq, g.Hq, g.d), np.float64)
    lse = np.empty((g.B, g.Hq, g.Nq), np.float64)
    sig = np.empty_like(out) if return_sigma else None
    sig_l = np.empty_like(lse) if return_sigma else None
    _L().or_dense_attention_fp8pv(ctypes.byref(g), _p(q8), _p(qs), _p(k8), _p(ks), _p(v), int(bool(causal)),
                                  _scale_arg(scale), int(bool(smooth_v)), _p(r), 0 if r is None else r.size, _p(hm),
                                  _p(out), _p(lse), _p(sig), _p(sig_l))
    if return_sigma:
        return out, lse, sig, sig_l
    return (out, lse) if return_lse else out


def dense_sage_attention_fp8pv_lazy(quant, v_bits, dtype="f16", causal=False, scale=None, smooth_v=False, tile=64,
                                    slack=3.0, group=16, return_lse=False):
    """A model of a tiled FP8 P.V implementation (reference moved lazily per
    group of rows): used to check the tolerance model, not a definition."""
    g, (q8, qs, k8, ks) = _quant_geometry(quant, 128, 64)
    v = _c(widen(v_bits, dtype), np.float32)
    out = np.empty((g.B, g.Nq, g.Hq, g.d), np.float64)
    lse = np.empty((g.B, g.Hq, g.Nq), np.float64)
    _L().or_dense_attention_fp8pv_lazy(ctypes.byref(g), _p(q8), _p(qs), _p(k8), _p(ks), _p(v), int(bool(causal)),
                                       _scale_arg(scale), int(bool(smooth_v)), int(tile), float(slack), int(group),
                                       _p(out), _p(lse))
    return (out, lse) if return_lse else out


__all__ = [
    "widen", "f32_to_f16_bits", "quant_rows", "quantize_q", "write_kv_cache", "write_kv_values", "gather_kv",
    "apply_rope", "rope_quantize_q", "rope_write_kv_cache",
    "e4m3_encode", "e4m3_decode", "e4m3_round", "v_fp8_per_channel", "dense_sage_attention_fp8pv",
    "dense_sage_attention_fp8pv_lazy",
    "paged_qk_int32", "paged_decode", "paged_decode_split", "split_segments", "chunked_prefill",
    "paged_v_fp8", "chunked_prefill_fp8pv",
    "dense_sage_attention", "attention_fp64", "default_scale",
    "sage_quantize", "sage_smooth_v", "sage_lse_correction", "sage_forward", "sage_varlen_forward",
    "build_library", "load_library", "use_library", "set_num_threads", "max_threads",
]
