"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library's full pipeline, and compare with the oracle."""
import sys

import numpy as np
import torch

import oracle
from workloads import PagedInputs

# Output tolerance against the oracle's fp64 result (fp32 output).
REL_L2 = 1e-3
MAX_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bits(bits: np.ndarray, dtype: str = "bf16") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def rel_l2(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def assert_close(got, want, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, want)
    m = float(np.max(np.abs(got - want))) if got.size else 0.0
    say(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= REL_L2, f"{what}: rel L2 {r:.3e} > {REL_L2}"
    assert m <= MAX_ABS, f"{what}: max abs {m:.3e} > {MAX_ABS}"


def gpu_cache(qa, inp: PagedInputs, v_int8: bool):
    """Write all tokens of a paged workload into a fresh GPU cache."""
    spec = inp.spec
    kc, ks, vc, vs = qa.alloc_kv_cache(spec.num_blocks, spec.num_kv_heads, spec.head_dim,
                                       torch.int8 if v_int8 else torch.bfloat16)
    if inp.k.shape[0]:
        qa.write_kv_cache(dev_bits(inp.k, spec.dtype), dev_bits(inp.v, spec.dtype),
                          torch.from_numpy(inp.slot_mapping).cuda(), kc, ks, vc, vs)
    return kc, ks, vc, vs


def oracle_cache(inp: PagedInputs, v_int8: bool):
    spec = inp.spec
    return oracle.write_kv_cache(inp.k, inp.v, spec.dtype, inp.slot_mapping, spec.num_blocks, v_int8)
