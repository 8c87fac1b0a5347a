"""The gfx950 machine code of this repository's own build (CPU only).

The matrix instruction a GEMM uses decides its peak, and scratch memory or
register spills would silently cost bandwidth, so these tests read the AMD
code objects that the build put into int4_w4a4_quantized_amd/_build/*.o
(extracted with llvm-objdump --offloading, disassembled for gfx950) and check:

- the FP6 GEMM runs v_mfma_scale_f32_16x16x128_f8f6f4 with both operands FP6
  E2M3 (cbsz:2 blgp:2) and the packed-int4 GEMM runs v_mfma_i32_16x16x64_i8;
- the FP6 quantiser packs its codes with the hardware FP6 converter;
- no kernel of the library uses scratch memory or spills vector registers, and the
  large FP6 GEMM tile fits two waves per SIMD (at most 256 VGPRs);
- gfx950 has no int4 matrix instruction: the assembler rejects the int4
  MFMA spellings (and the RDNA int4 WMMA, which it accepts for gfx1100), while
  it accepts the int8 and f8f6f4 forms written the same way. This is why the
  s4 x s4 product is carried by the int8 and FP6 matrix instructions ([PR #63]
  Description uses int4 tensor cores, which this part does not have).
"""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJDIR = os.path.join(ROOT, "int4_w4a4_quantized_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} not found")
    return path


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    """{object name: (disassembly, kernel metadata text)} for every built source."""
    objs = sorted(glob.glob(os.path.join(OBJDIR, "*.o")))
    if not objs:
        pytest.fail("no built objects in int4_w4a4_quantized_amd/_build: run __graft_entry__.build()")
    objdump, readelf = _tool("llvm-objdump"), _tool("llvm-readelf")
    out = {}
    tmp = tmp_path_factory.mktemp("isa")
    for obj in objs:
        local = tmp / os.path.basename(obj)
        shutil.copy(obj, local)
        subprocess.run([objdump, "--offloading", str(local)], check=True, capture_output=True, cwd=tmp)
        co = f"{local}.0.{TARGET}"
        if not os.path.exists(co):
            continue  # a host-only object (the C ABI layer)
        dis = subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True, capture_output=True,
                             text=True).stdout
        notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True, text=True).stdout
        out[os.path.splitext(os.path.basename(obj))[0]] = (dis, notes)
    return out


def _kernels(notes):
    """(name, private segment bytes, vgpr count, vgpr spills, sgpr spills) of each kernel in the metadata."""
    res = []
    for block in notes.split(".name:")[1:]:
        name = block.split()[0]

        def field(key):
            m = re.search(r"\." + key + r":\s+(\d+)", block)
            return int(m.group(1)) if m else None
        res.append((name, field("private_segment_fixed_size"), field("vgpr_count"), field("vgpr_spill_count"),
                    field("sgpr_spill_count")))
    return res


def test_fp6_gemm_uses_fp6_matrix_instruction(code_objects):
    dis, _ = code_objects["gemm_fp6"]
    mfma = [l for l in dis.splitlines() if "v_mfma_scale_f32_16x16x128_f8f6f4" in l]
    assert len(mfma) >= 27
    assert all("cbsz:2" in l and "blgp:2" in l for l in mfma), "an FP6 GEMM MFMA with non-FP6 operands"


def test_int4_gemm_uses_int8_matrix_instruction(code_objects):
    dis, _ = code_objects["gemm"]
    assert dis.count("v_mfma_i32_16x16x64_i8") >= 27


def test_fp6_quantiser_uses_hardware_converter(code_objects):
    dis, _ = code_objects["rotate_quant"]
    assert "v_cvt_scalef32_2xpk16_fp6_f32" in dis


def test_no_scratch_no_vgpr_spills(code_objects):
    """No kernel has a private (scratch) segment or spills vector registers. A
    scalar register spill, which the compiler parks in lanes of a vector
    register (no memory traffic), is allowed where the metadata still shows no
    private segment (a few skinny-kernel instances for 64-row activations have
    one)."""
    seen = 0
    sgpr_spillers = set()
    for obj, (_, notes) in code_objects.items():
        for name, priv, vgpr, vspill, sspill in _kernels(notes):
            seen += 1
            assert priv == 0, f"{obj}: {name} uses {priv} bytes of scratch"
            assert vspill == 0, f"{obj}: {name} spills vector registers"
            assert vgpr is not None and vgpr <= 512, f"{obj}: {name} has {vgpr} VGPRs"
            if sspill:
                sgpr_spillers.add(name)
    assert seen >= 20
    assert len(sgpr_spillers) < seen // 10, sgpr_spillers


def test_large_fp6_tile_fits_two_waves_per_simd(code_objects):
    _, notes = code_objects["gemm_fp6"]
    big = [k for k in _kernels(notes) if "ILi288ELi192E" in k[0]]
    # int32 store, bf16 epilogue, bf16 epilogue + LoRA; FP6 images and compact ones
    assert len(big) == 6
    for name, _, vgpr, _, _ in big:
        assert vgpr <= 256, f"{name}: {vgpr} VGPRs leave room for one wave per SIMD"


def _assembles(line, cpu):
    mc = _tool("llvm-mc")
    r = subprocess.run([mc, "-arch=amdgcn", f"-mcpu={cpu}", "-show-encoding"], input=line + "\n",
                       capture_output=True, text=True)
    return r.returncode == 0 and "encoding:" in r.stdout


def test_gfx950_has_no_int4_matrix_instruction():
    # the int8 and f8f6f4 forms assemble: the operand syntax below is right
    assert _assembles("v_mfma_i32_16x16x64_i8 v[0:3], v[4:7], v[8:11], v[0:3]", "gfx950")
    assert _assembles("v_mfma_i32_32x32x32_i8 v[0:15], v[16:19], v[20:23], v[0:15]", "gfx950")
    assert _assembles("v_mfma_scale_f32_16x16x128_f8f6f4 v[0:3], v[4:9], v[10:15], v[0:3], v16, v17 "
                      "op_sel_hi:[0,0,0] cbsz:2 blgp:2", "gfx950")
    # every int4 spelling of the same shapes is rejected
    for line in ("v_mfma_i32_16x16x64_i4 v[0:3], v[4:7], v[8:11], v[0:3]",
                 "v_mfma_i32_16x16x128_i4 v[0:3], v[4:7], v[8:11], v[0:3]",
                 "v_mfma_i32_32x32x64_i4 v[0:15], v[16:19], v[20:23], v[0:15]",
                 "v_mfma_i32_16x16x32_i4 v[0:3], v[4:5], v[8:9], v[0:3]"):
        assert not _assembles(line, "gfx950"), line
    # the RDNA3 int4 WMMA exists (gfx1100 accepts it) but not on gfx950
    wmma = "v_wmma_i32_16x16x16_iu4 v[0:7], v[8:9], v[10:11], v[0:7]"
    assert _assembles(wmma, "gfx1100")
    assert not _assembles(wmma, "gfx950")
