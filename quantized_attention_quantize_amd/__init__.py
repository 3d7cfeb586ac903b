"""Python binding of libqattn (INT8-QK quantized attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/qattn.h. Tensors are torch
device tensors; the calls queue work on the current torch stream. Output
tensors are allocated here with torch (plumbing), and the library itself
never allocates.

If the compiled library is missing this module raises at import: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libqattn.so not found at {LIB_PATH}; build it with "
        "`python quantized_attention_quantize_amd/build.py` (hipcc, gfx950)")

lib = ctypes.CDLL(LIB_PATH)

# ---- C types ---------------------------------------------------------------
QA_OK, QA_ERR_INVALID_ARG, QA_ERR_UNSUPPORTED, QA_ERR_WORKSPACE_TOO_SMALL, QA_ERR_HIP = range(5)
QA_DT_BF16, QA_DT_F16, QA_DT_F32, QA_DT_I8 = range(4)
SAGE_Q_BLOCK, SAGE_K_BLOCK = 128, 64

_c_void_p, _i32, _i64, _f32, _size = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class DecodeParams(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("block_size", _i32), ("max_blocks_per_seq", _i32), ("num_blocks", _i64),
                ("v_cache_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("softmax_scale", _f32),
                ("num_splits", _i32)]


class PrefillParams(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("block_size", _i32), ("max_blocks_per_seq", _i32), ("num_blocks", _i64), ("total_q", _i64),
                ("max_seqlen_q", _i32), ("v_cache_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("softmax_scale", _f32)]


class DenseParams(ctypes.Structure):
    _fields_ = [("batch", _i32), ("seq_q", _i32), ("seq_k", _i32), ("num_q_heads", _i32),
                ("num_kv_heads", _i32), ("head_dim", _i32), ("dtype", ctypes.c_int), ("smooth_k", _i32),
                ("is_causal", _i32), ("softmax_scale", _f32), ("out_dtype", ctypes.c_int)]


class RopeParams(ctypes.Structure):
    _fields_ = [("positions", _c_void_p), ("cos_sin", _c_void_p), ("rot_dim", _i32), ("neox", _i32)]


class VarlenParams(ctypes.Structure):
    _fields_ = [("batch", _i32), ("total_q", _i64), ("total_k", _i64), ("max_seqlen_q", _i32),
                ("max_seqlen_k", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("dtype", ctypes.c_int), ("smooth_k", _i32), ("smooth_v", _i32), ("is_causal", _i32),
                ("softmax_scale", _f32), ("out_dtype", ctypes.c_int), ("pv_fp8", _i32)]


class DenseOptions(ctypes.Structure):
    _fields_ = [("layout", _i32), ("smooth_v", _i32), ("pv_fp8", _i32)]


QA_LAYOUT_NHD, QA_LAYOUT_HND = 0, 1
_LAYOUTS = {"NHD": QA_LAYOUT_NHD, "HND": QA_LAYOUT_HND}

_P = ctypes.POINTER
_STEP_ARGS = ([_P(DecodeParams), _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i64, _i64, ctypes.c_int]
              + [_c_void_p] * 8 + [_size, _c_void_p, _c_void_p])

_SIGS = {
    "qa_abi_version": (ctypes.c_int, []),
    "qa_last_error": (ctypes.c_char_p, []),
    "qa_quantize_q": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i32, _i32, _i64, _i64, _c_void_p,
                                      _c_void_p, _c_void_p]),
    "qa_write_kv_cache": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i32, _i32, _i64, _i64,
                                          _c_void_p, _i64, _i32, _c_void_p, _c_void_p, _c_void_p, ctypes.c_int,
                                          _c_void_p, _c_void_p]),
    "qa_quantize_q_write_kv": (ctypes.c_int, [_c_void_p, _i64, _i32, _i64, _i64, _c_void_p, _c_void_p, _i64,
                                               _i32, _i64, _i64, _c_void_p, ctypes.c_int, _i32, _i64, _i32,
                                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                               ctypes.c_int, _c_void_p, _c_void_p]),
    "qa_rope_quantize_q_write_kv": (ctypes.c_int, [_P(RopeParams), _c_void_p, _i64, _i32, _i64, _i64, _c_void_p,
                                                    _c_void_p, _i64, _i32, _i64, _i64, _c_void_p, ctypes.c_int,
                                                    _i32, _i64, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                    _c_void_p, ctypes.c_int, _c_void_p, _c_void_p]),
    "qa_paged_decode_num_splits": (_i32, [_P(DecodeParams)]),
    "qa_paged_decode_step": (ctypes.c_int, _STEP_ARGS),
    "qa_paged_decode_step_rope": (ctypes.c_int, [_P(RopeParams)] + _STEP_ARGS),
    "qa_paged_decode_step_partials": (ctypes.c_int, _STEP_ARGS),
    "qa_paged_decode_workspace_bytes": (_size, [_P(DecodeParams)]),
    "qa_paged_decode_workspace_size": (_size, [_P(DecodeParams)]),
    "qa_paged_attention_decode": (ctypes.c_int, [_P(DecodeParams)] + [_c_void_p] * 9 + [_size, _c_void_p,
                                                                                           _c_void_p]),
    "qa_paged_attention_decode_partials": (ctypes.c_int, [_P(DecodeParams)] + [_c_void_p] * 9 +
                                           [_size, _c_void_p, _c_void_p]),
    "qa_paged_attention_decode_combine": (ctypes.c_int, [_P(DecodeParams), _c_void_p, _size, _c_void_p, _c_void_p]),
    "qa_paged_attention_decode_noalloc": (ctypes.c_int, [_P(DecodeParams)] + [_c_void_p] * 9 + [_c_void_p]),
    "qa_paged_decode_mt_workspace_size": (_size, [_P(DecodeParams), _i32]),
    "qa_paged_attention_decode_mt": (ctypes.c_int, [_P(DecodeParams), _i32] + [_c_void_p] * 9 +
                                     [_size, _c_void_p, _c_void_p]),
    "qa_debug_paged_qk_int32": (ctypes.c_int, [_P(DecodeParams)] + [_c_void_p] * 6),
    "qa_chunked_prefill_attention": (ctypes.c_int, [_P(PrefillParams)] + [_c_void_p] * 11),
    "qa_chunked_prefill_ws_workspace_bytes": (_size, [_P(PrefillParams)]),
    "qa_chunked_prefill_attention_ws": (ctypes.c_int, [_P(PrefillParams)] + [_c_void_p] * 10 +
                                        [_size, _c_void_p, _c_void_p]),
    "qa_chunked_prefill_fp8pv_workspace_bytes": (_size, [_P(PrefillParams)]),
    "qa_chunked_prefill_attention_fp8pv": (ctypes.c_int, [_P(PrefillParams)] + [_c_void_p] * 10 +
                                           [_size, _c_void_p, _c_void_p]),
    "qa_dense_sage_quantize_workspace_size": (_size, [_P(DenseParams)]),
    "qa_dense_sage_quantize": (ctypes.c_int, [_P(DenseParams)] + [_c_void_p] * 8 + [_size, _c_void_p]),
    "qa_dense_sage_workspace_bytes": (_size, [_P(DenseParams)]),
    "qa_dense_sage_workspace_size": (_size, [_P(DenseParams)]),
    "qa_dense_sage_attention": (ctypes.c_int, [_P(DenseParams)] + [_c_void_p] * 4 + [_size, _c_void_p,
                                                                                        _c_void_p]),
    "qa_dense_sage_ex_workspace_size": (_size, [_P(DenseParams), _P(DenseOptions)]),
    "qa_dense_sage_attention_ex": (ctypes.c_int, [_P(DenseParams), _P(DenseOptions)] + [_c_void_p] * 4 +
                                   [_size, _c_void_p, _c_void_p, _c_void_p]),
    "qa_dense_sage_varlen_workspace_size": (_size, [_P(VarlenParams)]),
    "qa_dense_sage_attention_varlen": (ctypes.c_int, [_P(VarlenParams)] + [_c_void_p] * 6 +
                                       [_size, _c_void_p, _c_void_p, _c_void_p]),
}
for _name, (_res, _args) in _SIGS.items():
    try:
        _fn = getattr(lib, _name)
    except AttributeError as e:
        raise ImportError(f"{LIB_PATH} lacks {_name}: the library is stale, rebuild it with "
                          "`python quantized_attention_quantize_amd/build.py`") from e
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class QAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qattn status {status}: {msg}")
        self.status = status


def _check(status: int):
    if status != QA_OK:
        raise QAttnError(status, lib.qa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.dtype) -> int:
    return {torch.bfloat16: QA_DT_BF16, torch.float16: QA_DT_F16, torch.float32: QA_DT_F32,
            torch.int8: QA_DT_I8}[t]


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


# ---- entry points ------------------------------------------------------------

def quantize_q(q: torch.Tensor):
    """q [T, H, d] bf16/f16 (innermost dim contiguous) -> (q_i8 [T, H, d], q_scale [T, H])."""
    _require_cuda(q)
    T, H, d = q.shape
    q_i8 = torch.empty((T, H, d), dtype=torch.int8, device=q.device)
    q_scale = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if q.stride(2) != 1:
        raise ValueError("innermost dimension of q must be contiguous")
    _check(lib.qa_quantize_q(_ptr(q), _dt(q.dtype), T, H, d, q.stride(0), q.stride(1), _ptr(q_i8),
                             _ptr(q_scale), _stream()))
    return q_i8, q_scale


def alloc_kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, v_dtype: torch.dtype,
                   device="cuda", zero: bool = True):
    """Cache tensors in the library's layout (see include/qattn.h)."""
    mk = torch.zeros if zero else torch.empty
    k_cache = mk((num_blocks, num_kv_heads, head_dim // 16, 16, 16), dtype=torch.int8, device=device)
    k_scale = mk((num_blocks, num_kv_heads, 16), dtype=torch.float32, device=device)
    v_cache = mk((num_blocks, num_kv_heads, head_dim, 16), dtype=v_dtype, device=device)
    v_scale = mk((num_blocks, num_kv_heads, 16), dtype=torch.float32, device=device) \
        if v_dtype == torch.int8 else None
    return k_cache, k_scale, v_cache, v_scale


def write_kv_cache(k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale=None):
    """Quantize K (and V if v_cache is int8) per (token, KV head) into the paged cache."""
    _require_cuda(k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale)
    T, H, d = k.shape
    if k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError("k and v must share strides with a contiguous innermost dim")
    _check(lib.qa_write_kv_cache(_ptr(k), _ptr(v), _dt(k.dtype), T, H, d, k.stride(0), k.stride(1),
                                 _ptr(slot_mapping), k_cache.shape[0], 16, _ptr(k_cache), _ptr(k_scale),
                                 _ptr(v_cache), _dt(v_cache.dtype), _ptr(v_scale), _stream()))


def quantize_q_write_kv(q, k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale=None, q_i8=None,
                        q_scale=None, rope=None):
    """Fused producer: quantize q [Tq, Hq, d] and write k/v [Tk, Hkv, d] into the
    cache in one launch. With rope = (positions int64 [T], cos_sin fp32
    [max_position, rot_dim], rot_dim, neox), q and k are rotated first (one
    launch for all three). Returns (q_i8, q_scale)."""
    _require_cuda(q, k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale)
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    if q_i8 is None:
        q_i8 = torch.empty((Tq, Hq, d), dtype=torch.int8, device=q.device)
    if q_scale is None:
        q_scale = torch.empty((Tq, Hq), dtype=torch.float32, device=q.device)
    if k.stride() != v.stride() or k.stride(2) != 1 or q.stride(2) != 1:
        raise ValueError("k and v must share strides; innermost dims must be contiguous")
    args = (_ptr(q), Tq, Hq, q.stride(0), q.stride(1), _ptr(k), _ptr(v), Tk, Hkv, k.stride(0), k.stride(1),
            _ptr(slot_mapping), _dt(q.dtype), d, k_cache.shape[0], 16, _ptr(q_i8), _ptr(q_scale), _ptr(k_cache),
            _ptr(k_scale), _ptr(v_cache), _dt(v_cache.dtype), _ptr(v_scale), _stream())
    if rope is None:
        _check(lib.qa_quantize_q_write_kv(*args))
    else:
        _check(lib.qa_rope_quantize_q_write_kv(ctypes.byref(_rope_params(rope)), *args))
    return q_i8, q_scale


def decode_params(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, num_blocks,
                  v_int8=False, out_dtype=torch.float32, softmax_scale=0.0, num_splits=0) -> DecodeParams:
    return DecodeParams(num_seqs, num_q_heads, num_kv_heads, head_dim, 16, max_blocks_per_seq, num_blocks,
                        QA_DT_I8 if v_int8 else QA_DT_BF16, _dt(out_dtype), softmax_scale, num_splits)


def decode_num_splits(p: DecodeParams) -> int:
    return lib.qa_paged_decode_num_splits(ctypes.byref(p))


def decode_workspace(p: DecodeParams, device="cuda") -> torch.Tensor:
    """Decode workspace (split-K partials; no initialization needed)."""
    n = lib.qa_paged_decode_workspace_bytes(ctypes.byref(p))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _decode(entry, q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, num_kv_heads,
            softmax_scale, num_splits, out_dtype, workspace, out):
    _require_cuda(q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens)
    S, Hq, d = q_i8.shape
    Hkv = num_kv_heads or k_cache.shape[1]
    p = decode_params(S, Hq, Hkv, d, block_tables.shape[1], k_cache.shape[0], v_cache.dtype == torch.int8,
                      out_dtype, softmax_scale, num_splits)
    if workspace is None:
        workspace = decode_workspace(p, q_i8.device)
    if out is None:
        out = torch.empty((S, Hq, d), dtype=out_dtype, device=q_i8.device)
    _check(entry(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                 _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), _ptr(workspace), workspace.numel(),
                 _ptr(out), _stream()))
    return out, workspace, p


def paged_attention_decode(q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens,
                           num_kv_heads=None, softmax_scale=0.0, num_splits=0, out_dtype=torch.float32,
                           workspace=None, out=None):
    """Decode attention; returns out [num_seqs, Hq, d]."""
    return _decode(lib.qa_paged_attention_decode, q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables,
                   context_lens, num_kv_heads, softmax_scale, num_splits, out_dtype, workspace, out)[0]


def paged_attention_decode_noalloc(q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens,
                                   num_kv_heads=None, softmax_scale=0.0, num_splits=0, out_dtype=torch.float32,
                                   out=None):
    """Decode attention through the allocation-free entry point (split
    partials in the library's static device scratch); same result as
    paged_attention_decode. Returns out [num_seqs, Hq, d]."""
    _require_cuda(q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens, out)
    S, Hq, d = q_i8.shape
    Hkv = num_kv_heads or k_cache.shape[1]
    p = decode_params(S, Hq, Hkv, d, block_tables.shape[1], k_cache.shape[0], v_cache.dtype == torch.int8,
                      out_dtype, softmax_scale, num_splits)
    if out is None:
        out = torch.empty((S, Hq, d), dtype=out_dtype, device=q_i8.device)
    _check(lib.qa_paged_attention_decode_noalloc(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(k_cache),
                                                 _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(block_tables),
                                                 _ptr(context_lens), _ptr(out), _stream()))
    return out


def paged_attention_decode_partials(q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens,
                                    num_kv_heads=None, softmax_scale=0.0, num_splits=0, out_dtype=torch.float32,
                                    workspace=None, out=None):
    """First phase of decode (the split kernel). Returns (out, workspace,
    params); pass the last two to paged_attention_decode_combine."""
    return _decode(lib.qa_paged_attention_decode_partials, q_i8, q_scale, k_cache, k_scale, v_cache, v_scale,
                   block_tables, context_lens, num_kv_heads, softmax_scale, num_splits, out_dtype, workspace, out)


def paged_attention_decode_combine(params, workspace, out):
    """Second phase of decode: merge the split partials into out."""
    _require_cuda(workspace, out)
    _check(lib.qa_paged_attention_decode_combine(ctypes.byref(params), _ptr(workspace), workspace.numel(),
                                                 _ptr(out), _stream()))
    return out


def paged_attention_decode_mt(q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens,
                              num_kv_heads=None, softmax_scale=0.0, num_splits=0, out_dtype=torch.float32,
                              workspace=None, out=None):
    """Multi-token decode: q_i8 [num_seqs, T, Hq, d], q_scale [num_seqs, T, Hq];
    token j of sequence s sits at position context_lens[s] - T + j. Returns
    out [num_seqs, T, Hq, d]."""
    _require_cuda(q_i8, q_scale, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens)
    S, T, Hq, d = q_i8.shape
    Hkv = num_kv_heads or k_cache.shape[1]
    p = decode_params(S, Hq, Hkv, d, block_tables.shape[1], k_cache.shape[0], v_cache.dtype == torch.int8,
                      out_dtype, softmax_scale, num_splits)
    if workspace is None:
        n = lib.qa_paged_decode_mt_workspace_size(ctypes.byref(p), T)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q_i8.device)
    if out is None:
        out = torch.empty((S, T, Hq, d), dtype=out_dtype, device=q_i8.device)
    _check(lib.qa_paged_attention_decode_mt(ctypes.byref(p), T, _ptr(q_i8), _ptr(q_scale), _ptr(k_cache),
                                            _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(block_tables),
                                            _ptr(context_lens), _ptr(workspace), workspace.numel(), _ptr(out),
                                            _stream()))
    return out


def _rope_params(rope):
    positions, cos_sin, rot_dim, neox = rope
    _require_cuda(positions, cos_sin)
    if positions.dtype != torch.int64 or cos_sin.dtype != torch.float32 or not cos_sin.is_contiguous():
        raise ValueError("positions must be int64 and cos_sin contiguous fp32")
    return RopeParams(_ptr(positions), _ptr(cos_sin), rot_dim, int(bool(neox)))


def paged_decode_step(q, k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens,
                      num_kv_heads=None, softmax_scale=0.0, num_splits=0, out_dtype=torch.float32,
                      workspace=None, out=None, rope=None):
    """One decode step in one call: quantize q [num_seqs, Hq, d], write the new
    token's k/v [num_seqs, Hkv, d] at slot_mapping, and attend over the cache
    (context_lens include the new token). With rope = (positions int64
    [num_seqs], cos_sin, rot_dim, neox) q and k are rotated first, in the
    same kernel. Returns out [num_seqs, Hq, d]."""
    _require_cuda(q, k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale, block_tables, context_lens)
    S, Hq, d = q.shape
    Hkv = num_kv_heads or k_cache.shape[1]
    if k.stride() != v.stride() or k.stride(2) != 1 or q.stride(2) != 1:
        raise ValueError("k and v must share strides; innermost dims must be contiguous")
    p = decode_params(S, Hq, Hkv, d, block_tables.shape[1], k_cache.shape[0], v_cache.dtype == torch.int8,
                      out_dtype, softmax_scale, num_splits)
    if workspace is None:
        workspace = decode_workspace(p, q.device)
    if out is None:
        out = torch.empty((S, Hq, d), dtype=out_dtype, device=q.device)
    args = (ctypes.byref(p), _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
            _dt(q.dtype), _ptr(slot_mapping), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
            _ptr(block_tables), _ptr(context_lens), _ptr(workspace), workspace.numel(), _ptr(out), _stream())
    if rope is None:
        _check(lib.qa_paged_decode_step(*args))
    else:
        _check(lib.qa_paged_decode_step_rope(ctypes.byref(_rope_params(rope)), *args))
    return out


def debug_paged_qk_int32(q_i8, k_cache, block_tables, context_lens, num_kv_heads=None, fill=0):
    """INT32 QK accumulators of the decode kernel: [num_seqs, Hq, max_blocks*16]."""
    _require_cuda(q_i8, k_cache, block_tables, context_lens)
    S, Hq, d = q_i8.shape
    Hkv = num_kv_heads or k_cache.shape[1]
    p = decode_params(S, Hq, Hkv, d, block_tables.shape[1], k_cache.shape[0])
    acc = torch.full((S, Hq, block_tables.shape[1] * 16), fill, dtype=torch.int32, device=q_i8.device)
    _check(lib.qa_debug_paged_qk_int32(ctypes.byref(p), _ptr(q_i8), _ptr(k_cache), _ptr(block_tables),
                                       _ptr(context_lens), _ptr(acc), _stream()))
    return acc


def prefill_params(q_i8, context_lens, k_cache, v_cache, block_tables, max_seqlen_q, num_kv_heads=None,
                   softmax_scale=0.0, out_dtype=torch.float32) -> PrefillParams:
    T, Hq, d = q_i8.shape
    Hkv = num_kv_heads or k_cache.shape[1]
    return PrefillParams(context_lens.shape[0], Hq, Hkv, d, 16, block_tables.shape[1], k_cache.shape[0], T,
                         int(max_seqlen_q), QA_DT_I8 if v_cache.dtype == torch.int8 else QA_DT_BF16,
                         _dt(out_dtype), softmax_scale)


def chunked_prefill_attention(q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale,
                              block_tables, max_seqlen_q, num_kv_heads=None, softmax_scale=0.0,
                              out_dtype=torch.float32, out=None):
    """Chunked prefill over the paged cache; returns out [total_q, Hq, d]."""
    _require_cuda(q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale, block_tables)
    p = prefill_params(q_i8, context_lens, k_cache, v_cache, block_tables, max_seqlen_q, num_kv_heads,
                       softmax_scale, out_dtype)
    if out is None:
        out = torch.empty(q_i8.shape, dtype=out_dtype, device=q_i8.device)
    _check(lib.qa_chunked_prefill_attention(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(cu_seqlens_q),
                                            _ptr(context_lens), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                                            _ptr(v_scale), _ptr(block_tables), _ptr(out), _stream()))
    return out


def chunked_prefill_ws_workspace(p: PrefillParams):
    """A device workspace for qa_chunked_prefill_attention_ws."""
    return torch.empty(lib.qa_chunked_prefill_ws_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8,
                       device="cuda")


def chunked_prefill_attention_ws(q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale,
                                 block_tables, max_seqlen_q, num_kv_heads=None, softmax_scale=0.0,
                                 out_dtype=torch.float32, workspace=None, out=None):
    """chunked_prefill_attention with V converted once into a workspace
    (allocated when None); the output is the same bit for bit."""
    _require_cuda(q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale, block_tables)
    p = prefill_params(q_i8, context_lens, k_cache, v_cache, block_tables, max_seqlen_q, num_kv_heads,
                       softmax_scale, out_dtype)
    if workspace is None:
        workspace = chunked_prefill_ws_workspace(p)
    if out is None:
        out = torch.empty(q_i8.shape, dtype=out_dtype, device=q_i8.device)
    _check(lib.qa_chunked_prefill_attention_ws(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(cu_seqlens_q),
                                               _ptr(context_lens), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                                               _ptr(v_scale), _ptr(block_tables), _ptr(workspace),
                                               workspace.numel(), _ptr(out), _stream()))
    return out


def chunked_prefill_fp8pv_workspace(p: PrefillParams):
    """A device workspace for qa_chunked_prefill_attention_fp8pv."""
    return torch.empty(lib.qa_chunked_prefill_fp8pv_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8,
                       device="cuda")


def chunked_prefill_attention_fp8pv(q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale,
                                    block_tables, max_seqlen_q, num_kv_heads=None, softmax_scale=0.0,
                                    out_dtype=torch.float32, workspace=None, out=None):
    """Chunked prefill with the P.V product in FP8 (E4M3); returns out
    [total_q, Hq, d]. The workspace (allocated when None) holds the E4M3 V
    tiles and channel scales afterwards (include/qattn.h)."""
    _require_cuda(q_i8, q_scale, cu_seqlens_q, context_lens, k_cache, k_scale, v_cache, v_scale, block_tables)
    p = prefill_params(q_i8, context_lens, k_cache, v_cache, block_tables, max_seqlen_q, num_kv_heads,
                       softmax_scale, out_dtype)
    if workspace is None:
        workspace = chunked_prefill_fp8pv_workspace(p)
    if out is None:
        out = torch.empty(q_i8.shape, dtype=out_dtype, device=q_i8.device)
    _check(lib.qa_chunked_prefill_attention_fp8pv(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(cu_seqlens_q),
                                                  _ptr(context_lens), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                                                  _ptr(v_scale), _ptr(block_tables), _ptr(workspace),
                                                  workspace.numel(), _ptr(out), _stream()))
    return out


def dense_params(q, k, smooth_k=True, is_causal=False, softmax_scale=0.0, out_dtype=None) -> DenseParams:
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    return DenseParams(B, Nq, Nk, Hq, Hkv, d, _dt(q.dtype), int(bool(smooth_k)), int(bool(is_causal)),
                       softmax_scale, _dt(out_dtype or torch.float32))


def dense_sage_quantize(q, k, smooth_k=True):
    """NHD q, k -> dict(q_i8, q_scale, k_i8, k_scale, k_mean) (SageAttention-style preprocessing)."""
    _require_cuda(q, k)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    p = dense_params(q, k, smooth_k)
    dev = q.device
    res = {
        "q_i8": torch.empty((B, Nq, Hq, d), dtype=torch.int8, device=dev),
        "q_scale": torch.empty((B, Hq, -(-Nq // SAGE_Q_BLOCK)), dtype=torch.float32, device=dev),
        "k_i8": torch.empty((B, Nk, Hkv, d), dtype=torch.int8, device=dev),
        "k_scale": torch.empty((B, Hkv, -(-Nk // SAGE_K_BLOCK)), dtype=torch.float32, device=dev),
        "k_mean": torch.empty((B, Hkv, d), dtype=torch.float32, device=dev),
    }
    ws = torch.empty(max(lib.qa_dense_sage_quantize_workspace_size(ctypes.byref(p)), 16), dtype=torch.uint8,
                     device=dev)
    _check(lib.qa_dense_sage_quantize(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(res["q_i8"]), _ptr(res["q_scale"]),
                                      _ptr(res["k_i8"]), _ptr(res["k_scale"]), _ptr(res["k_mean"]), _ptr(ws),
                                      ws.numel(), _stream()))
    return res


def dense_sage_workspace(p: DenseParams, device="cuda") -> torch.Tensor:
    return torch.empty(max(lib.qa_dense_sage_workspace_bytes(ctypes.byref(p)), 16), dtype=torch.uint8, device=device)


def dense_sage_attention(q, k, v, is_causal=False, smooth_k=True, softmax_scale=0.0, out_dtype=torch.float32,
                         workspace=None, out=None):
    """SageAttention-style dense forward on NHD tensors; returns out [B, Nq, Hq, d]."""
    _require_cuda(q, k, v)
    p = dense_params(q, k, smooth_k, is_causal, softmax_scale, out_dtype)
    if workspace is None:
        workspace = dense_sage_workspace(p, q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check(lib.qa_dense_sage_attention(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(workspace),
                                       workspace.numel(), _ptr(out), _stream()))
    return out


def dense_sage_attention_ex(q, k, v, tensor_layout="NHD", is_causal=False, smooth_k=True, smooth_v=False,
                            return_lse=False, softmax_scale=0.0, out_dtype=torch.float32, workspace=None,
                            out=None, lse=None, pv_fp8=False):
    """The dense forward with its options: tensor_layout "NHD" ([B, N, H, d])
    or "HND" ([B, H, N, d]) for q, k, v and out; smooth_v; return_lse (fp32
    [B, Hq, Nq], natural log, corrected for the K mean under smooth_k);
    pv_fp8 (the P.V product in FP8 E4M3, head_dim 64 or 128).
    Returns out, or (out, lse) with return_lse."""
    _require_cuda(q, k, v)
    if tensor_layout not in _LAYOUTS:
        raise ValueError(f"tensor_layout must be NHD or HND, not {tensor_layout!r}")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k and v must be contiguous in their layout")
    if tensor_layout == "HND":
        B, Hq, Nq, d = q.shape
        Hkv, Nk = k.shape[1], k.shape[2]
    else:
        B, Nq, Hq, d = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
    p = DenseParams(B, Nq, Nk, Hq, Hkv, d, _dt(q.dtype), int(bool(smooth_k)), int(bool(is_causal)),
                    softmax_scale, _dt(out_dtype))
    o = DenseOptions(_LAYOUTS[tensor_layout], int(bool(smooth_v)), int(bool(pv_fp8)))
    if workspace is None:
        workspace = torch.empty(max(lib.qa_dense_sage_ex_workspace_size(ctypes.byref(p), ctypes.byref(o)), 16),
                                dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check(lib.qa_dense_sage_attention_ex(ctypes.byref(p), ctypes.byref(o), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(workspace), workspace.numel(), _ptr(out),
                                          _ptr(lse) if return_lse else None, _stream()))
    return (out, lse) if return_lse else out


def varlen_params(q, k, max_seqlen_q, max_seqlen_k, batch, is_causal=False, smooth_k=True, smooth_v=False,
                  softmax_scale=0.0, out_dtype=torch.float32, pv_fp8=False) -> VarlenParams:
    return VarlenParams(batch, q.shape[0], k.shape[0], max_seqlen_q, max_seqlen_k, q.shape[1], k.shape[1],
                        q.shape[2], _dt(q.dtype), int(bool(smooth_k)), int(bool(smooth_v)), int(bool(is_causal)),
                        softmax_scale, _dt(out_dtype), int(bool(pv_fp8)))


def dense_sage_attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, is_causal=False,
                                smooth_k=True, smooth_v=False, return_lse=False, softmax_scale=0.0,
                                out_dtype=torch.float32, workspace=None, out=None, lse=None, pv_fp8=False):
    """Packed variable-length dense forward: q [total_q, Hq, d], k and v
    [total_k, Hkv, d]; cu_seqlens_q/k int32 [B+1] on the GPU. Returns out
    [total_q, Hq, d], or (out, lse [Hq, total_q]) with return_lse."""
    _require_cuda(q, k, v, cu_seqlens_q, cu_seqlens_k)
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k and v must be contiguous")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    batch = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    p = varlen_params(q, k, max_seqlen_q, max_seqlen_k, batch, is_causal, smooth_k, smooth_v, softmax_scale,
                      out_dtype, pv_fp8)
    if workspace is None:
        workspace = torch.empty(max(lib.qa_dense_sage_varlen_workspace_size(ctypes.byref(p)), 16),
                                dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    _check(lib.qa_dense_sage_attention_varlen(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                              _ptr(cu_seqlens_k), _ptr(workspace), workspace.numel(), _ptr(out),
                                              _ptr(lse) if return_lse else None, _stream()))
    return (out, lse) if return_lse else out
