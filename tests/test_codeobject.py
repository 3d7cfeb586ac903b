"""The device code this repository builds, read back from libqattn.so (CPU
only): the hot kernels contain the matrix instructions the design relies on,
the decode kernels use no scratch memory, the dense tile loops keep a single
vector-memory wait and no scratch access, and no packed fp32 arithmetic was
generated (the build disables it). Uses the ROCm LLVM tools on our own
build's code objects; skipped where they are missing."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_attention_quantize_amd", "libqattn.so")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = {t: os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")}
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


@pytest.fixture(scope="module")
def disassembly():
    """(opcode set per kernel, instruction list per kernel); an instruction is
    (address, opcode, operand text, branch target address or None)."""
    if not os.path.exists(LIB):
        pytest.skip("libqattn.so not built")
    for t in TOOLS.values():
        if not os.path.exists(t):
            pytest.skip(f"{t} missing")
    out, listing = {}, {}
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fat.bin")
        subprocess.run([TOOLS["llvm-objcopy"], "--dump-section", f".hip_fatbin={fat}", LIB, os.path.join(d, "x")],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        assert starts, "no offload bundle in .hip_fatbin"
        for i, s in enumerate(starts):
            piece = data[s:starts[i + 1] if i + 1 < len(starts) else len(data)]
            b = os.path.join(d, f"b{i}.bundle")
            co = os.path.join(d, f"b{i}.co")
            open(b, "wb").write(piece)
            r = subprocess.run([TOOLS["clang-offload-bundler"], "--unbundle", "--type=o", f"--input={b}",
                                "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], capture_output=True)
            if r.returncode != 0 or not os.path.exists(co) or os.path.getsize(co) == 0:
                continue
            dis = subprocess.run([TOOLS["llvm-objdump"], "-d", "--mcpu=gfx950", co], check=True,
                                 capture_output=True, text=True).stdout
            name = None
            for line in dis.splitlines():
                m = re.match(r"^([0-9a-f]+) <(\S+)>:", line)
                if m:
                    name, base = m.group(2), int(m.group(1), 16)
                    out[name], listing[name] = set(), []
                    continue
                if name is not None:
                    t = line.strip().split()
                    if t and re.match(r"^[sv]_|^global_|^buffer_|^ds_|^scratch_|^flat_", t[0]):
                        out[name].add(t[0])
                        a = re.search(r"// ([0-9A-Fa-f]+):", line)
                        tg = re.search(r"<" + re.escape(name) + r"\+0x([0-9a-f]+)>", line)
                        if a:
                            listing[name].append((int(a.group(1), 16), t[0], line.split("//")[0],
                                                  base + int(tg.group(1), 16) if tg else None))
    assert out, "no gfx950 code object found"
    return out, listing


@pytest.fixture(scope="module")
def kernels(disassembly):
    return disassembly[0]


def _has(ins, op):
    return any(x == op or x.startswith(op + "_") for x in ins)


def _with(kernels, part):
    ks = {n: ins for n, ins in kernels.items() if part in n}
    assert ks, f"no kernel named like {part}"
    return ks


def test_decode_kernels_use_int8_and_bf16_matrix_units_and_no_scratch(kernels):
    ks = _with(kernels, "k_decode")
    assert any(_has(i, "v_mfma_i32_16x16x64_i8") and _has(i, "v_mfma_f32_16x16x32_bf16") for i in ks.values())
    for n, ins in ks.items():
        assert not any(x.startswith("scratch_") for x in ins), f"{n} spills to scratch"


def test_flash_kernels_use_the_matrix_units(kernels):
    ks = _with(kernels, "k_flash")
    assert all(_has(i, "v_mfma_i32_16x16x64_i8") for i in ks.values())        # INT8 QK in every variant
    assert any(_has(i, "v_mfma_f32_16x16x32_f16") for i in ks.values())       # fp16 P.V
    fp8 = [i for i in ks.values() if _has(i, "v_mfma_f32_32x32x64_f8f6f4")]   # FP8 P.V
    assert fp8 and all(_has(i, "v_cvt_pk_fp8_f32") and _has(i, "v_permlane16_swap_b32") for i in fp8)


def test_no_packed_fp32_arithmetic(kernels):
    bad = {n: sorted(x for x in ins if x.startswith(("v_pk_fma_f32", "v_pk_add_f32", "v_pk_mul_f32")))
           for n, ins in kernels.items()}
    bad = {n: v for n, v in bad.items() if v}
    assert not bad, bad


def _main_loop(ins):
    """The instructions of the loop (a backward branch's range) that holds the
    most matrix instructions."""
    best, best_n = [], -1
    for addr, op, _, tgt in ins:
        if op.startswith(("s_cbranch", "s_branch")) and tgt is not None and tgt < addr:
            body = [x for x in ins if tgt <= x[0] <= addr]
            n = sum(1 for x in body if x[1].startswith("v_mfma"))
            if n > best_n:
                best, best_n = body, n
    return best


def test_dense_tile_loops_wait_once_for_memory(disassembly):
    """The dense kernels copy the next tile global -> LDS while computing on
    the current one; the end-of-tile wait before the barrier must be the
    loop's only vector-memory wait (any other one also waits for the copies
    in flight), and the loop must not reload spilled registers."""
    dense = {n: ins for n, ins in disassembly[1].items()
             if re.search(r"k_flashILi\d+ELi\d+ELi\d+ELi\d+ELb1E", n)}
    assert len(dense) >= 10, sorted(dense)
    for n, ins in dense.items():
        body = _main_loop(ins)
        assert body, f"{n}: no loop found"
        waits = [x[2].strip() for x in body if x[1] == "s_waitcnt" and "vmcnt" in x[2]]
        assert len(waits) == 1, (n, waits)
        assert not [x for x in body if x[1].startswith("scratch_")], f"{n} touches scratch in its tile loop"


def test_lds_dma_never_directly_follows_an_m0_write(disassembly):
    """GFX9 parts, gfx950 included, need one wait state between an SALU write
    of M0 and an LDS-DMA load (global_load_lds_*, buffer_load_* ... lds) that
    takes its LDS address from M0. Every such load in the library must be
    separated from the instruction that writes M0 by at least one other
    instruction (the copies issue an s_nop)."""
    n_dma = 0
    for name, ins in disassembly[1].items():
        for prev, cur in zip(ins, ins[1:]):
            is_dma = cur[1].startswith("global_load_lds") or (cur[1].startswith("buffer_load") and " lds" in cur[2])
            if not is_dma:
                continue
            n_dma += 1
            writes_m0 = re.match(r"\s*s_\w+\s+m0\b", prev[2]) is not None
            assert not writes_m0, f"{name} @{cur[0]:#x}: {cur[1]} right after '{prev[2].strip()}'"
    assert n_dma > 0, "no LDS-DMA loads found: the dense and 12-wave prefill kernels use them"


def test_fp8_prefill_tile_loops_wait_once_for_memory(disassembly):
    """As for the dense kernels: the FP8 P.V prefill copies the next K and V8
    tiles global -> LDS during the current one, so its tile loop must hold a
    single vector-memory wait and touch no scratch (a spill reload would wait
    for the copies in flight)."""
    ks = {n: ins for n, ins in disassembly[1].items() if "k_prefill8" in n}
    assert len(ks) == 3, sorted(ks)
    for n, ins in ks.items():
        body = _main_loop(ins)
        assert body, f"{n}: no loop found"
        waits = [x[2].strip() for x in body if x[1] == "s_waitcnt" and "vmcnt" in x[2]]
        assert len(waits) == 1, (n, waits)
        assert not [x for x in body if x[1].startswith("scratch_")], f"{n} touches scratch in its tile loop"


def test_lds_dma_bases_are_not_sign_extended(disassembly):
    """The LDS-DMA copies take a 64-bit scalar base assembled from two 32-bit
    halves; a sign-extended low half (s_bfe_i64 ..., 0x200000 before the OR)
    turns every base whose bit 31 is set into an illegal address. No kernel
    that issues LDS-DMA loads may sign-extend a 32-bit value to 64 bits."""
    for name, ins in disassembly[1].items():
        if not any(x[1].startswith("global_load_lds") for x in ins):
            continue
        bad = [x[2].strip() for x in ins if x[1] == "s_bfe_i64"]
        assert not bad, (name, bad[:3])
