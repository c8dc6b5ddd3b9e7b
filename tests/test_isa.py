"""Checks of the gfx950 machine code of the built library (no GPU needed).

The device code objects are taken out of our own libfp4moe.so (the
.hip_fatbin section holds one offload bundle per source file), disassembled
with the ROCm LLVM tools, and checked for:
  * the instructions each hot kernel is designed around (scaled MFMA, LDS-DMA,
    the gfx950 FP4 conversions, the f16 MFMA of the NVFP4 path);
  * no register spills to scratch inside the hot loops;
  * no packed fp32 arithmetic anywhere (the build disables it);
  * no write through the scalar data cache anywhere.
"""

import functools
import os
import re
import subprocess
import tempfile

import pytest
import yaml

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_scaled_fp4_moe_amd", "libfp4moe.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


@functools.lru_cache(maxsize=1)
def kernels():
    """{kernel symbol: (list of instruction lines, metadata dict)} of every kernel."""
    tools = ["llvm-objcopy", "clang-offload-bundler", "llvm-objdump", "llvm-readelf"]
    if not os.path.exists(LIB) or not all(os.path.exists(os.path.join(LLVM, t)) for t in tools):
        pytest.skip("library or ROCm LLVM tools not available")
    out = {}
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        f".hip_fatbin={fat}", LIB], check=True, capture_output=True)
        blob = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), blob)]
        for i, s in enumerate(starts):
            e = starts[i + 1] if i + 1 < len(starts) else len(blob)
            b, co = os.path.join(d, f"b{i}.bin"), os.path.join(d, f"c{i}.o")
            open(b, "wb").write(blob[s:e])
            subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                            f"--targets={TARGET}", f"--input={b}", f"--output={co}"],
                           check=True, capture_output=True)
            dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn",
                                  co], check=True, capture_output=True, text=True).stdout
            notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co],
                                   check=True, capture_output=True, text=True).stdout
            meta = {}
            m = re.search(r"^\s*---\s*$(.*?)^\s*\.\.\.\s*$", notes, flags=re.M | re.S)
            if m:
                for k in yaml.safe_load(m.group(1)).get("amdhsa.kernels", []):
                    meta[k[".name"]] = k
            cur = None
            for line in dis.splitlines():
                lab = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
                if lab:
                    cur = lab.group(1)
                    out.setdefault(cur, ([], meta.get(cur, {})))
                elif cur and line.startswith("\t"):
                    out[cur][0].append(line.strip())
    assert out, "no kernels found"
    return out


def find(prefix):
    ks = kernels()
    names = [n for n in ks if n.startswith(prefix)]
    assert names, f"no kernel {prefix}"
    return names


def mnemonics(name):
    return {ln.split()[0] for ln in kernels()[name][0] if ln}


HOT = {
    # decode GEMMs: MXFP4 decoded to bf16 by the gfx950 conversion, bf16 MFMA
    "_ZN6fp4moe14dq_gemm_kernelILi0ELi0ELi1ELi1ELi4ELi2ELi4ELi4E":
        ["v_cvt_scalef32_pk_bf16_fp4", "v_mfma_f32_16x16x32_bf16"],
    "_ZN6fp4moe14dq_gemm_kernelILi0ELi0ELi2ELi1ELi4ELi2ELi4ELi4E":
        ["v_cvt_scalef32_pk_bf16_fp4", "v_mfma_f32_16x16x32_bf16"],
    # prefill / dense / FP8-weight tiles: scaled MFMA fed by LDS-DMA; stage 1
    # also quantizes h with the FP4 conversion
    "_ZN6fp4moe23mx_dma_wide_gemm_kernelILi1ELb0E":
        ["v_mfma_scale_f32_32x32x64_f8f6f4", "global_load_lds_dwordx4", "v_cvt_scalef32_pk_fp4_f32"],
    "_ZN6fp4moe23mx_dma_wide_gemm_kernelILi2ELb0E":
        ["v_mfma_scale_f32_32x32x64_f8f6f4", "global_load_lds_dwordx4"],
    "_ZN6fp4moe23mx_dma_wide_gemm_kernelILi1ELb1E":
        ["v_mfma_scale_f32_32x32x64_f8f6f4", "global_load_lds_dwordx4"],
    "_ZN6fp4moe23mx_dma_wide_gemm_kernelILi2ELb1E":
        ["v_mfma_scale_f32_32x32x64_f8f6f4", "global_load_lds_dwordx4"],
    # NVFP4 with f16 activations: f16 decode and the 32x32x16 f16 MFMA
    "_ZN6fp4moe15dqt_gemm_kernelILi1ELi2ELi1ELi3ELi4ELi8E":
        ["v_mfma_f32_32x32x16_f16", "v_cvt_scalef32_pk_f16_fp4", "v_pk_mul_f16",
         "global_load_lds_dwordx4"],
    "_ZN6fp4moe15dqt_gemm_kernelILi1ELi2ELi2ELi3ELi4ELi8E":
        ["v_mfma_f32_32x32x16_f16", "v_cvt_scalef32_pk_f16_fp4", "v_pk_mul_f16"],
    # NVFP4 in 128-row tiles: f16 decode in registers, 32x32x16 f16 MFMA
    "_ZN6fp4moe12_GLOBAL__N_117nvf16_gemm_kernelILi1ELi8E":
        ["v_mfma_f32_32x32x16_f16", "v_cvt_scalef32_pk_f16_fp4", "v_pk_mul_f16"],
    "_ZN6fp4moe12_GLOBAL__N_117nvf16_gemm_kernelILi2ELi8E":
        ["v_mfma_f32_32x32x16_f16", "v_cvt_scalef32_pk_f16_fp4", "v_pk_mul_f16"],
    # activation quantization: E2M1 codes by the hardware conversion
    "_ZN6fp4moe18mxfp4_quant_kernelILb1E": ["v_cvt_scalef32_pk_fp4_f32"],
    "_ZN6fp4moe18mxfp4_quant_kernelILb0E": ["v_cvt_scalef32_pk_fp4_f32"],
    # exact MXFP4 -> FP8: byte lookup by v_perm
    "_ZN6fp4moe16mx_to_fp8_kernelILi8E": ["v_perm_b32"],
    # routing: DPP wavefront maximum
    "_ZN6fp4moe20route_permute_kernelILi6E": ["v_max_u32_dpp"],
    "_ZN6fp4moe12route_kernelILi6E": ["v_max_u32_dpp"],
}


@pytest.mark.parametrize("prefix", sorted(HOT))
def test_hot_kernel_instructions(prefix):
    for name in find(prefix):
        have = mnemonics(name)
        missing = [m for m in HOT[prefix] if m not in have]
        assert not missing, f"{name} lacks {missing}"


def _innermost_mfma_loops(lines):
    """(first, last) line indices of every innermost loop (a backward branch
    whose body holds no other backward branch) that contains an MFMA."""
    addr = []
    for ln in lines:
        m = re.search(r"//\s*([0-9A-Fa-f]+):", ln)
        addr.append(int(m.group(1), 16) if m else None)
    base = next(a for a in addr if a is not None)
    loops = []
    for i, ln in enumerate(lines):
        if not ln.startswith("s_cbranch") and not ln.startswith("s_branch"):
            continue
        m = re.search(r"<[^>+]*\+0x([0-9a-fA-F]+)>", ln)
        if not m or addr[i] is None:
            continue
        target = base + int(m.group(1), 16)
        if target >= addr[i]:
            continue
        j = next(k for k, a in enumerate(addr) if a is not None and a >= target)
        loops.append((j, i))
    inner = [(j, i) for j, i in loops
             if not any(j < j2 and i2 < i for j2, i2 in loops if (j2, i2) != (j, i))]
    return [(j, i) for j, i in inner if any(ln.startswith("v_mfma") for ln in lines[j:i + 1])]


@pytest.mark.parametrize("prefix", sorted(HOT))
def test_hot_loops_do_not_spill(prefix):
    """No scratch access inside a GEMM kernel's innermost loops that hold its
    MFMAs (a spill reload there would wait for every copy in flight; a few
    between work items are harmless) and at most 64 bytes of scratch per lane;
    the kernels without MFMAs use no scratch at all."""
    for name in find(prefix):
        lines, meta = kernels()[name]
        assert meta, f"no metadata for {name}"
        if any(ln.startswith("v_mfma") for ln in lines):
            loops = _innermost_mfma_loops(lines)
            assert loops, f"{name}: no MFMA loop found"
            for j, i in loops:
                inner = [ln for ln in lines[j:i + 1] if ln.startswith("scratch_")]
                assert not inner, f"{name}: {inner[:3]}"
            assert meta.get(".private_segment_fixed_size", 0) <= 64, name
        else:
            assert meta.get(".private_segment_fixed_size", 0) == 0, name
            assert meta.get(".vgpr_spill_count", 0) == 0, name


def test_no_packed_fp32_arithmetic():
    bad = re.compile(r"^v_pk_(add|mul|fma)_f32\b")
    hits = [(n, ln) for n, (lines, _) in kernels().items() for ln in lines if bad.match(ln)]
    assert not hits, hits[:5]


def test_no_scalar_cache_writes():
    bad = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|"
                     r"dcache_discard)")
    hits = [(n, ln) for n, (lines, _) in kernels().items() for ln in lines if bad.match(ln)]
    assert not hits, hits[:5]


def _reg_range(tok):
    """'v[4:7]' -> ('v', 4, 7); 'v12' -> ('v', 12, 12); otherwise None."""
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok) or re.match(r"^([va])(\d+)()$", tok)
    if not m:
        return None
    lo = int(m.group(2))
    return m.group(1), lo, int(m.group(3)) if m.group(3) else lo


def test_mfma_destination_disjoint_from_sources():
    """Every FP8 / FP6 / FP4-operand MFMA of every kernel (the scaled and the
    f8f6f4 forms) writes a register range that overlaps neither its A nor its B
    operand: such MFMAs generated with an overlapping destination gave wrong
    results, so the kernels keep them apart and this guards against a compiler
    or flag change that would not.  The bf16 / f16 MFMAs are left to the
    compiler, whose instruction definitions let a four-register result take the
    registers of a source it last reads (their results are parity-tested)."""
    bad, n = [], 0
    for name, (lines, _) in kernels().items():
        for ln in lines:
            if not ln.startswith("v_mfma"):
                continue
            if not re.search(r"f8f6f4|fp8|bf8|_scale_", ln.split()[0]):
                continue
            ops = [t.strip() for t in ln.split("//")[0].split(None, 1)[1].split(",")]
            dst, a, b = (_reg_range(ops[0].split()[0]), _reg_range(ops[1]), _reg_range(ops[2]))
            assert dst and a and b, f"{name}: cannot parse {ln}"
            n += 1
            for src in (a, b):
                if src[0] == dst[0] and src[1] <= dst[2] and dst[1] <= src[2]:
                    bad.append((name, ln))
    assert n > 0
    assert not bad, bad[:3]
