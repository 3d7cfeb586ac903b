"""CPU oracle for INT8-QK quantized attention: TEST INFRASTRUCTURE ONLY.

This package is the slow, plain definition of what the GPU library
computes. Only the test suite, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import it. The GPU library never
imports, links or calls it, and it shares no code with the GPU path: the
only common module is the seeded input generator, which holds none of the
method's arithmetic.

Sources (the three pages this work follows):

* [QK-MMAC] "INT8 QK MMAC on the gfx936 DCU: paged access, fragment
  mapping and GQA" (forum article, second of a series).
* [LP-NEG] "Dynamic INT8 GEMM and FP8 KV-cache attention on gfx936"
  (forum article reporting negative low-precision results).
* [SAGE-MACA] "SageAttention - MetaX MXMACA port (v3.0.0)" README.

Precision: quantization follows the pages in IEEE fp32 (one correctly
rounded operation per step, round-half-even). Everything after the INT32
accumulator (score recovery, softmax, P.V) is done in fp64, since the pages
fix no precision there.

Parity status, function by function (pins live in tests/test_oracle_pins.py):

* quant_rows, quantize_q, write_kv_cache, sage_quantize: pinned (worked
  rounding ties, arg-max maps to +-127, error bound, zero rows, layout
  round trip, brute force per block, smoothing mean exactness).
* paged_qk_int32: pinned (INT32 bound 256*127*127, brute force in int64).
* paged_decode, paged_decode_split, chunked_prefill, dense_sage_attention:
  pinned (rows sum to one, equality with a textbook fp64 attention of the
  dequantized tensors, split = unsplit, smoothing invariance, causal
  structure).
* sage_smooth_v, sage_lse_correction, sage_forward (smooth_v, LSE): pinned
  (closed forms: LSE of equal scores is ln(#visible); constant keys make the
  corrected LSE q.c*scale + ln(#visible); the V mean added back reproduces
  the unsmoothed output within the fp16 rounding of V').
* apply_rope, rope_quantize_q, rope_write_kv_cache: pinned (position 0 is
  the identity; pairs rotate as complex numbers times e^(i theta); the
  interleaved pairing is the half pairing of permuted channels; channels
  past rot_dim pass through; rotated dot products depend only on the
  position difference).
* e4m3_encode / e4m3_decode: pinned (the format's landmark values, ties to
  even at midpoints, saturation, and torch's float8_e4m3fn conversion).
* dense_sage_attention_fp8pv: pinned (constant V comes back exactly; one
  visible key returns its FP8-rounded value; a two-key closed form through
  the pinned codec; rescaling across tiles; within the FP8 error bound of
  the 16-bit P path).
* sage_varlen_forward: pinned (equal lengths reproduce the batched forward;
  a sequence's rows do not depend on its neighbours; empty sequences).
"""
from .quant import (widen, quant_rows, quantize_q, write_kv_cache, write_kv_values, sage_quantize,
                    gather_kv)
from .rope import apply_rope, rope_quantize_q, rope_write_kv_cache
from .fp8 import e4m3_encode, e4m3_decode, e4m3_round, v_fp8_per_channel, dense_sage_attention_fp8pv
from .attention import (paged_qk_int32, paged_decode, paged_decode_split,
                        chunked_prefill, dense_sage_attention, attention_fp64,
                        default_scale, sage_smooth_v, sage_lse_correction, sage_forward,
                        sage_varlen_forward)

__all__ = [
    "widen", "quant_rows", "quantize_q", "write_kv_cache", "write_kv_values", "sage_quantize", "gather_kv",
    "apply_rope", "rope_quantize_q", "rope_write_kv_cache",
    "e4m3_encode", "e4m3_decode", "e4m3_round", "v_fp8_per_channel", "dense_sage_attention_fp8pv",
    "paged_qk_int32", "paged_decode", "paged_decode_split", "chunked_prefill",
    "dense_sage_attention", "attention_fp64", "default_scale",
    "sage_smooth_v", "sage_lse_correction", "sage_forward", "sage_varlen_forward",
]
