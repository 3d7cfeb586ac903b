"""C ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments on the host before any
HIP call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qattn.h")


@pytest.fixture(scope="module")
def qa():
    lib_path = os.path.join(ROOT, "quantized_attention_quantize_amd", "libqattn.so")
    if not os.path.exists(lib_path):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "qa_build", os.path.join(ROOT, "quantized_attention_quantize_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import quantized_attention_quantize_amd as m
    return m


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qa_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(qa):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(qa.lib, n), f"missing export {n}"
    assert set(names) == set(qa.EXPORTED)


def _param_counts():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(qa_[a-z0-9_]+)\s*\(([^()]*)\)\s*;", src):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_header(qa):
    counts = _param_counts()
    assert set(counts) == set(qa.EXPORTED)
    for name, (_, args) in qa._SIGS.items():
        assert len(args) == counts[name], f"{name}: binding passes {len(args)} arguments, header declares {counts[name]}"


def test_abi_version(qa):
    assert qa.lib.qa_abi_version() == 1


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first


def test_quantize_q_rejects(qa):
    L = qa.lib
    assert L.qa_quantize_q(FAKE, qa.QA_DT_BF16, 4, 2, 96, 192, 96, FAKE, FAKE, None) == qa.QA_ERR_UNSUPPORTED
    assert b"head_dim 96" in L.qa_last_error()
    assert L.qa_quantize_q(FAKE, qa.QA_DT_F32, 4, 2, 64, 128, 64, FAKE, FAKE, None) == qa.QA_ERR_UNSUPPORTED
    assert L.qa_quantize_q(None, qa.QA_DT_BF16, 4, 2, 64, 128, 64, FAKE, FAKE, None) == qa.QA_ERR_INVALID_ARG
    assert L.qa_quantize_q(FAKE, qa.QA_DT_BF16, -1, 2, 64, 128, 64, FAKE, FAKE, None) == qa.QA_ERR_INVALID_ARG
    assert L.qa_quantize_q(FAKE, qa.QA_DT_BF16, 4, 2, 64, 129, 64, FAKE, FAKE, None) == qa.QA_ERR_INVALID_ARG
    # zero tokens is a no-op even with null pointers
    assert L.qa_quantize_q(None, qa.QA_DT_BF16, 0, 2, 64, 128, 64, None, None, None) == qa.QA_OK


def test_write_kv_cache_rejects(qa):
    L = qa.lib
    args = [FAKE, FAKE, qa.QA_DT_BF16, 8, 2, 64, 128, 64, FAKE, 4, 16, FAKE, FAKE, FAKE, qa.QA_DT_BF16, None, None]
    a = list(args); a[10] = 32
    assert L.qa_write_kv_cache(*a) == qa.QA_ERR_UNSUPPORTED
    a = list(args); a[14] = qa.QA_DT_I8
    assert L.qa_write_kv_cache(*a) == qa.QA_ERR_INVALID_ARG   # INT8 V without v_scale
    a = list(args); a[14] = qa.QA_DT_F16
    assert L.qa_write_kv_cache(*a) == qa.QA_ERR_UNSUPPORTED
    a = list(args); a[8] = None
    assert L.qa_write_kv_cache(*a) == qa.QA_ERR_INVALID_ARG


def _dp(qa, **kw):
    p = qa.decode_params(2, 24, 4, 256, 64, 1000)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_decode_validation(qa):
    L = qa.lib
    call = lambda p, ws_bytes=0, ws=FAKE: L.qa_paged_attention_decode(
        ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, ws_bytes, FAKE, None)
    assert call(_dp(qa, head_dim=96)) == qa.QA_ERR_UNSUPPORTED
    assert call(_dp(qa, block_size=32)) == qa.QA_ERR_UNSUPPORTED
    assert call(_dp(qa, num_q_heads=68, num_kv_heads=4)) == qa.QA_ERR_UNSUPPORTED      # group 17
    assert call(_dp(qa, num_q_heads=25)) == qa.QA_ERR_INVALID_ARG                      # not a multiple
    assert call(_dp(qa, v_cache_dtype=qa.QA_DT_F16)) == qa.QA_ERR_UNSUPPORTED
    assert call(_dp(qa, v_cache_dtype=qa.QA_DT_I8)) == qa.QA_ERR_INVALID_ARG           # v_scale missing
    assert call(_dp(qa, out_dtype=qa.QA_DT_F16)) == qa.QA_ERR_UNSUPPORTED
    p = _dp(qa, num_splits=8)
    need = L.qa_paged_decode_workspace_bytes(ctypes.byref(p))
    al = lambda x: (x + 255) // 256 * 256
    assert need == al(2 * 24 * 8 * 256 * 4) + al(2 * 24 * 8 * 2 * 4)   # partial O + (max, sum)
    assert call(p, need - 1) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert b"needed" in L.qa_last_error()
    assert L.qa_paged_decode_workspace_bytes(ctypes.byref(_dp(qa, num_splits=1))) == 0


def test_decode_step_validation(qa):
    L = qa.lib
    p = _dp(qa, num_splits=8)
    need = L.qa_paged_decode_workspace_bytes(ctypes.byref(p))
    for fn in (L.qa_paged_decode_step, L.qa_paged_decode_step_partials):
        call = lambda p, dt=qa.QA_DT_BF16, ws_bytes=need, q=FAKE, vs=None: fn(
            ctypes.byref(p), q, 6144, 256, FAKE, FAKE, 1024, 256, dt, FAKE, FAKE, FAKE, FAKE, vs, FAKE, FAKE,
            FAKE, ws_bytes, FAKE, None)
        assert call(p, dt=qa.QA_DT_F32) == qa.QA_ERR_UNSUPPORTED
        assert call(p, dt=qa.QA_DT_F16) == qa.QA_ERR_UNSUPPORTED          # bf16 V cache needs bf16 inputs
        assert call(p, ws_bytes=need - 1) == qa.QA_ERR_WORKSPACE_TOO_SMALL
        assert call(p, q=None) == qa.QA_ERR_INVALID_ARG
        assert call(_dp(qa, v_cache_dtype=qa.QA_DT_I8), dt=qa.QA_DT_F16) == qa.QA_ERR_INVALID_ARG   # v_scale
        assert call(_dp(qa, head_dim=96)) == qa.QA_ERR_UNSUPPORTED


def test_decode_phase_validation(qa):
    L = qa.lib
    p = _dp(qa, num_splits=8)
    need = L.qa_paged_decode_workspace_bytes(ctypes.byref(p))
    part = lambda p, ws_bytes, *ptrs: L.qa_paged_attention_decode_partials(
        ctypes.byref(p), *ptrs, FAKE, ws_bytes, FAKE, None)
    assert part(p, need - 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert part(p, need, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE) == qa.QA_ERR_INVALID_ARG
    assert part(_dp(qa, head_dim=96), need, *([FAKE] * 5), None, FAKE, FAKE) == qa.QA_ERR_UNSUPPORTED
    # combine needs only the workspace and the output
    assert L.qa_paged_attention_decode_combine(ctypes.byref(p), FAKE, need - 1, FAKE, None) == \
        qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert L.qa_paged_attention_decode_combine(ctypes.byref(p), None, need, FAKE, None) == qa.QA_ERR_INVALID_ARG
    assert L.qa_paged_attention_decode_combine(ctypes.byref(p), FAKE, need, None, None) == qa.QA_ERR_INVALID_ARG


def test_decode_split_heuristic(qa):
    f = lambda S, Hkv, mb: qa.lib.qa_paged_decode_num_splits(ctypes.byref(qa.decode_params(S, 6 * Hkv, Hkv, 256, mb, 10)))
    assert f(1, 4, 2048) == 64           # one long sequence: one workgroup per CU
    assert f(32, 4, 2048) == 4           # several sequences: two workgroups per CU
    assert f(1, 1, 64) == 4              # short context: at least 16 blocks per split
    assert f(1, 1, 4) == 1
    assert f(200, 4, 2048) == 1
    assert f(64, 4, 2048) == 2


def test_prefill_and_dense_validation(qa):
    L = qa.lib
    p = qa.PrefillParams(1, 24, 4, 256, 16, 100, 1000, 10, 10, qa.QA_DT_BF16, qa.QA_DT_F32, 0.0)
    p.head_dim = 80
    assert L.qa_chunked_prefill_attention(ctypes.byref(p), *([FAKE] * 10), None) == qa.QA_ERR_UNSUPPORTED
    p.head_dim = 256
    assert L.qa_chunked_prefill_attention(ctypes.byref(p), FAKE, FAKE, None, *([FAKE] * 7), None) == \
        qa.QA_ERR_INVALID_ARG
    d = qa.DenseParams(2, 100, 100, 8, 3, 128, qa.QA_DT_F16, 1, 0, 0.0, qa.QA_DT_F32)
    assert L.qa_dense_sage_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE, None) == \
        qa.QA_ERR_INVALID_ARG                                                   # 8 % 3 != 0
    d.num_kv_heads = 4
    need = L.qa_dense_sage_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert L.qa_dense_sage_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, need - 1, FAKE, None) == \
        qa.QA_ERR_WORKSPACE_TOO_SMALL
    d.dtype = qa.QA_DT_F32
    assert L.qa_dense_sage_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, need, FAKE, None) == \
        qa.QA_ERR_UNSUPPORTED


def test_prefill_fp8pv_validation_and_workspace(qa):
    """The FP8 P.V prefill: the same shape and pointer checks as the 16-bit
    entry, a workspace of E4M3 tiles (128 keys x head_dim bytes per tile, KV
    head and sequence), channel scales and partial maxima, and a refusal of
    a smaller workspace."""
    L = qa.lib
    p = qa.PrefillParams(2, 24, 4, 256, 16, 100, 1000, 10, 10, qa.QA_DT_BF16, qa.QA_DT_F32, 0.0)
    need = L.qa_chunked_prefill_fp8pv_workspace_bytes(ctypes.byref(p))
    tiles = -(-100 * 16 // 128)
    v8 = 2 * tiles * 4 * 128 * 256
    al = lambda x: -(-x // 256) * 256
    assert need == al(al(al(v8) + 2 * 4 * 256 * 4) + 2 * 4 * 32 * 256 * 4)
    call = lambda p, ws=FAKE, nb=need, q=FAKE: L.qa_chunked_prefill_attention_fp8pv(
        ctypes.byref(p), q, *([FAKE] * 6), None, FAKE, ws, nb, FAKE, None)   # v_scale NULL
    assert call(p, nb=need - 1) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert call(p, ws=None) == qa.QA_ERR_INVALID_ARG
    assert call(p, q=None) == qa.QA_ERR_INVALID_ARG
    p.head_dim = 80
    assert L.qa_chunked_prefill_fp8pv_workspace_bytes(ctypes.byref(p)) == 0
    assert call(p) == qa.QA_ERR_UNSUPPORTED
    p.head_dim = 256
    p.v_cache_dtype = qa.QA_DT_I8
    assert call(p) == qa.QA_ERR_INVALID_ARG                # INT8 V needs v_scale
    p.num_seqs = 0
    assert L.qa_chunked_prefill_attention_fp8pv(ctypes.byref(p), *([None] * 10), 0, None, None) == qa.QA_OK


def test_prefill_ws_validation_and_workspace(qa):
    """The prefill with V converted into a workspace: the 16-bit entry's
    checks, a workspace of one fp16 V block (head_dim x 16) per logical block,
    KV head and sequence, and a refusal of a smaller or missing one."""
    L = qa.lib
    p = qa.PrefillParams(3, 24, 4, 128, 16, 100, 1000, 10, 10, qa.QA_DT_BF16, qa.QA_DT_F32, 0.0)
    need = L.qa_chunked_prefill_ws_workspace_bytes(ctypes.byref(p))
    assert need == 3 * 100 * 4 * 128 * 16 * 2
    call = lambda p, ws=FAKE, nb=need, q=FAKE: L.qa_chunked_prefill_attention_ws(
        ctypes.byref(p), q, *([FAKE] * 6), None, FAKE, ws, nb, FAKE, None)   # v_scale NULL
    assert call(p, nb=need - 1) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert call(p, ws=None) == qa.QA_ERR_INVALID_ARG
    assert call(p, ws=ctypes.c_void_p(0x10008)) == qa.QA_ERR_INVALID_ARG   # not 16-byte aligned
    assert call(p, q=None) == qa.QA_ERR_INVALID_ARG
    p.head_dim = 96
    assert L.qa_chunked_prefill_ws_workspace_bytes(ctypes.byref(p)) == 0
    assert call(p) == qa.QA_ERR_UNSUPPORTED
    p.head_dim = 128
    p.v_cache_dtype = qa.QA_DT_I8
    assert call(p) == qa.QA_ERR_INVALID_ARG                # INT8 V needs v_scale
    p.num_seqs = 0
    assert L.qa_chunked_prefill_attention_ws(ctypes.byref(p), *([None] * 10), 0, None, None) == qa.QA_OK


def test_dense_options_validation(qa):
    L = qa.lib
    d = qa.DenseParams(2, 100, 90, 8, 4, 128, qa.QA_DT_BF16, 1, 0, 0.0, qa.QA_DT_F32)
    o = qa.DenseOptions(qa.QA_LAYOUT_HND, 1, 0)
    plain = L.qa_dense_sage_workspace_bytes(ctypes.byref(d))
    need = L.qa_dense_sage_ex_workspace_size(ctypes.byref(d), ctypes.byref(o))
    # the options call adds the V mean (2 x 4 x 128 fp32) and the LSE correction (2 x 8 x 100 fp32)
    assert need == plain + 4096 + 6400
    assert L.qa_dense_sage_ex_workspace_size(ctypes.byref(d), None) == need
    ex = lambda opts, ws_bytes, lse: L.qa_dense_sage_attention_ex(
        ctypes.byref(d), opts, FAKE, FAKE, FAKE, FAKE, ws_bytes, FAKE, lse, None)
    assert ex(ctypes.byref(o), need - 1, FAKE) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert ex(None, plain, None) == qa.QA_ERR_WORKSPACE_TOO_SMALL      # the plain call's size is not enough
    assert ex(ctypes.byref(o), need, ctypes.c_void_p(0x10002)) == qa.QA_ERR_INVALID_ARG  # lse not 4-byte aligned
    assert b"lse" in L.qa_last_error()
    o.pv_fp8 = 1                                           # FP8 P.V: E4M3 V blocks of 64 keys + channel scales
    need8 = L.qa_dense_sage_ex_workspace_size(ctypes.byref(d), ctypes.byref(o))
    # 90 keys: 6 blocks of 16 (fp16) give way to 2 blocks of 64 (E4M3), plus 2 x 4 x 128 fp32 channel scales
    assert need8 == need - 2 * 6 * 4 * 128 * 16 * 2 + 2 * 2 * 4 * 128 * 64 + 2 * 4 * 128 * 4
    d.head_dim = 256
    assert ex(ctypes.byref(o), 1 << 40, None) == qa.QA_ERR_UNSUPPORTED
    d.head_dim, o.pv_fp8 = 128, 0
    o.layout = 7
    assert ex(ctypes.byref(o), need, None) == qa.QA_ERR_INVALID_ARG
    assert b"layout 7" in L.qa_last_error()
    assert L.qa_dense_sage_attention_ex(ctypes.byref(d), ctypes.byref(o), FAKE, None, FAKE, FAKE, need, FAKE,
                                        None, None) == qa.QA_ERR_INVALID_ARG


def test_dense_varlen_validation(qa):
    L = qa.lib
    p = qa.VarlenParams(3, 700, 900, 400, 500, 8, 2, 128, qa.QA_DT_F16, 1, 1, 1, 0.0, qa.QA_DT_F32, 0)
    need = L.qa_dense_sage_varlen_workspace_size(ctypes.byref(p))
    # packed blocks: 900/16 + 3 = 59 K blocks of 2 x 128 x 16 (int8 codes + fp16 V); Q codes 700 x 8 x 128
    assert need >= 700 * 8 * 128 + 59 * 2 * 128 * 16 * 3
    call = lambda ws_bytes, *ptrs: L.qa_dense_sage_attention_varlen(ctypes.byref(p), *ptrs, FAKE, ws_bytes, FAKE,
                                                                    None, None)
    assert call(need - 1, FAKE, FAKE, FAKE, FAKE, FAKE) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert call(need, FAKE, FAKE, FAKE, None, FAKE) == qa.QA_ERR_INVALID_ARG              # no cu_seqlens_q
    assert call(need, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10002)) == qa.QA_ERR_INVALID_ARG  # misaligned
    p.num_kv_heads = 3
    assert call(need, FAKE, FAKE, FAKE, FAKE, FAKE) == qa.QA_ERR_INVALID_ARG              # 8 % 3
    p.num_kv_heads, p.head_dim = 2, 96
    assert call(need, FAKE, FAKE, FAKE, FAKE, FAKE) == qa.QA_ERR_UNSUPPORTED
    p.head_dim, p.total_q = 128, -1
    assert call(need, FAKE, FAKE, FAKE, FAKE, FAKE) == qa.QA_ERR_INVALID_ARG
    p.total_q, p.batch = 700, 0
    assert call(0, None, None, None, None, None) == qa.QA_OK                              # nothing to do


def test_rope_producer_validation(qa):
    L = qa.lib
    args = lambda d: (FAKE, 4, 8, 8 * d, d, FAKE, FAKE, 4, 2, 2 * d, d, FAKE, qa.QA_DT_BF16, d, 10, 16,
                      FAKE, FAKE, FAKE, FAKE, FAKE, qa.QA_DT_BF16, None, None)
    r = qa.RopeParams(FAKE, FAKE, 64, 1)
    for rot in (0, 63, 130):
        r.rot_dim = rot
        assert L.qa_rope_quantize_q_write_kv(ctypes.byref(r), *args(128)) == qa.QA_ERR_INVALID_ARG
        assert b"rot_dim" in L.qa_last_error()
    r.rot_dim, r.positions = 64, None
    assert L.qa_rope_quantize_q_write_kv(ctypes.byref(r), *args(128)) == qa.QA_ERR_INVALID_ARG
    assert L.qa_rope_quantize_q_write_kv(None, *args(128)) == qa.QA_ERR_INVALID_ARG
    r.positions = FAKE
    assert L.qa_rope_quantize_q_write_kv(ctypes.byref(r), *args(96)) == qa.QA_ERR_UNSUPPORTED   # head_dim 96
    # the step with rotary embedding checks rope before anything is launched
    p = qa.decode_params(2, 24, 4, 256, 100, 1000)
    step = lambda rp: L.qa_paged_decode_step_rope(rp, ctypes.byref(p), FAKE, 6144, 256, FAKE, FAKE, 1024, 256,
                                                  qa.QA_DT_BF16, *([FAKE] * 8), 1 << 30, FAKE, None)
    assert step(None) == qa.QA_ERR_INVALID_ARG
    r.rot_dim = 258
    assert step(ctypes.byref(r)) == qa.QA_ERR_INVALID_ARG


def test_last_error_is_thread_local(qa):
    import threading
    L = qa.lib
    L.qa_quantize_q(FAKE, qa.QA_DT_BF16, 4, 2, 96, 192, 96, FAKE, FAKE, None)
    seen = {}

    def other():
        L.qa_quantize_q(None, qa.QA_DT_BF16, 4, 2, 64, 128, 64, FAKE, FAKE, None)
        seen["msg"] = L.qa_last_error()
    t = threading.Thread(target=other)
    t.start(); t.join()
    assert b"null" in seen["msg"]
    assert b"head_dim 96" in L.qa_last_error()


PROBE_HEADER = os.path.join(ROOT, "include", "qa_probe.h")


def test_probe_library_exports_and_rejects():
    """The measurement probes (qa_probe.h) load, export what the header
    declares and reject bad arguments on the host."""
    from quantized_attention_quantize_amd import probes
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(qa_probe_[a-z0-9_]+)\s*\(", src)))
    assert declared == sorted(probes.EXPORTED)
    L = probes.lib
    assert L.qa_probe_stream_read(None, 16, 4, FAKE, None) == 1
    assert L.qa_probe_stream_read(FAKE, 15, 4, FAKE, None) == 1        # not a multiple of 16
    assert L.qa_probe_stream_read(FAKE, 16, 0, FAKE, None) == 1
    assert L.qa_probe_stream_read(FAKE, 16, 70000, FAKE, None) == 1
    assert L.qa_probe_stream_read(FAKE, 0, 4, FAKE, None) == 0         # nothing to read
    assert L.qa_probe_mfma(9, 10, 4, FAKE, None) == 1
    assert L.qa_probe_mfma(-1, 10, 4, FAKE, None) == 1
    assert L.qa_probe_mfma(0, 0, 4, FAKE, None) == 1
    assert L.qa_probe_mfma(0, 10, 4, None, None) == 1
    assert L.qa_probe_valu(2, 10, 4, FAKE, None) == 1
    assert L.qa_probe_valu(-1, 10, 4, FAKE, None) == 1
    assert L.qa_probe_valu(0, 0, 4, FAKE, None) == 1
    assert L.qa_probe_valu(1, 10, 0, FAKE, None) == 1
    assert L.qa_probe_valu(1, 10, 65536, FAKE, None) == 1
    assert L.qa_probe_valu(0, 10, 4, None, None) == 1


def test_decode_mt_validation(qa):
    L = qa.lib
    p = _dp(qa, num_splits=8)                        # 24 query heads over 4 KV heads: G = 6
    call = lambda p, T, ws_bytes=1 << 30: L.qa_paged_attention_decode_mt(
        ctypes.byref(p), T, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws_bytes, FAKE, None)
    assert call(p, 0) == qa.QA_ERR_INVALID_ARG
    assert call(p, 3) == qa.QA_ERR_UNSUPPORTED       # 6 x 3 > 16 columns
    need = L.qa_paged_decode_mt_workspace_size(ctypes.byref(p), 2)
    al = lambda x: (x + 255) // 256 * 256
    assert need == al(2 * 2 * 24 * 8 * 256 * 4) + al(2 * 2 * 24 * 8 * 2 * 4)
    assert L.qa_paged_decode_mt_workspace_size(ctypes.byref(p), 1) == L.qa_paged_decode_workspace_bytes(ctypes.byref(p))
    assert L.qa_paged_decode_mt_workspace_size(ctypes.byref(p), 3) == 0
    assert call(p, 2, need - 1) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert call(_dp(qa, head_dim=96), 1) == qa.QA_ERR_UNSUPPORTED
    assert L.qa_paged_attention_decode_mt(ctypes.byref(p), 2, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                          FAKE, need, FAKE, None) == qa.QA_ERR_INVALID_ARG


def test_workspace_bytes_names_and_their_aliases(qa):
    """The workspace queries under their fixed names (..._bytes); the earlier
    ..._size names return the same values, also 0 for rejected parameters."""
    L = qa.lib
    for S in (0, 1, 8, 64):
        p = _dp(qa, num_splits=S)
        assert L.qa_paged_decode_workspace_bytes(ctypes.byref(p)) == L.qa_paged_decode_workspace_size(ctypes.byref(p))
    p = _dp(qa, head_dim=96)
    assert L.qa_paged_decode_workspace_bytes(ctypes.byref(p)) == 0 == L.qa_paged_decode_workspace_size(ctypes.byref(p))
    for causal in (0, 1):
        d = qa.DenseParams(2, 300, 200, 8, 4, 128, qa.QA_DT_F16, 1, causal, 0.0, qa.QA_DT_F32)
        n = L.qa_dense_sage_workspace_bytes(ctypes.byref(d))
        assert n > 0 and n == L.qa_dense_sage_workspace_size(ctypes.byref(d))
    d.head_dim = 80
    assert L.qa_dense_sage_workspace_bytes(ctypes.byref(d)) == 0


def test_decode_noalloc_validation(qa):
    """The allocation-free decode rejects, on the host and before any HIP call,
    parameters whose split partials do not fit the static scratch, and the
    same bad arguments as the workspace call."""
    L = qa.lib
    assert qa.lib is not None
    call = lambda p, q=FAKE, vs=None: L.qa_paged_attention_decode_noalloc(
        ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, vs, FAKE, FAKE, FAKE, None)
    big = _dp(qa, num_seqs=64, num_splits=64)
    need = L.qa_paged_decode_workspace_bytes(ctypes.byref(big))
    assert need > (16 << 20)
    assert call(big) == qa.QA_ERR_WORKSPACE_TOO_SMALL
    assert b"static decode scratch" in L.qa_last_error()
    ok = _dp(qa, num_seqs=32, num_splits=8)
    assert L.qa_paged_decode_workspace_bytes(ctypes.byref(ok)) <= (16 << 20)
    assert call(ok, q=None) == qa.QA_ERR_INVALID_ARG
    assert call(_dp(qa, v_cache_dtype=qa.QA_DT_I8)) == qa.QA_ERR_INVALID_ARG      # v_scale missing
    assert call(_dp(qa, head_dim=96)) == qa.QA_ERR_UNSUPPORTED
    assert L.qa_paged_attention_decode_noalloc(ctypes.byref(_dp(qa, num_seqs=0)), *([None] * 10)) == qa.QA_OK
