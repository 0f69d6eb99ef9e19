"""Structural checks of the gfx950 code the decode kernel compiles to (CPU only:
hipcc cross-compiles). They guard the properties the kernel's speed depends on
and that a source change could silently lose:
  * every asynchronous global->LDS copy takes its base address from SGPRs,
  * the page loop waits for copies with one bounded vmcnt wait and never drains
    all of them (no vmcnt(0) inside the loop),
  * no packed-FP32 VALU instruction is generated,
  * no spills to scratch memory."""
import os
import re
import shutil
import subprocess

import pytest

from bit_paged_kv_nvfp4_amd import build as B

HIPCC = B.HIPCC


def _asm(tmp_path, src):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, *[f for f in B.FLAGS if f not in ("-shared", "-fPIC")], "-I", B.INCLUDE, "-I", B.CSRC,
           "--cuda-device-only", "-S", "-o", str(out), src]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _function(asm, name):
    """Body of the kernel whose mangled name holds `name` (a length-prefixed
    identifier, e.g. 14k_decode_split), up to the end of the function."""
    m = re.search(rf"^(_Z\S*{name}\S*):", asm, flags=re.M)
    assert m, name
    start = m.end()
    end = asm.index(".Lfunc_end", start)
    return asm[start:end]


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    return _asm(tmp_path_factory.mktemp("isa"), os.path.join(B.CSRC, "decode.hip"))


# the NVFP4 kernel and the FP8 baseline's instance of the same template
KERNELS = ["14k_decode_split", "18k_decode_split_fp8"]


@pytest.mark.parametrize("kernel", KERNELS)
def test_copies_use_sgpr_base(decode_asm, kernel):
    body = _function(decode_asm, kernel)
    copies = re.findall(r"global_load_lds_dword\S*\s+([^\n]+)", body)
    assert copies, "no asynchronous copies found"
    for operands in copies:
        assert re.search(r",\s*s\[\d+:\d+\]", operands), operands


def _blocks(body):
    """Basic blocks as (label, annotation, text); the annotation is the comment
    lines the compiler puts on and after the label (loop membership)."""
    out = []
    parts = re.split(r"^(\.LBB\d+_\d+):", body, flags=re.M)
    for label, rest in zip(parts[1::2], parts[2::2]):
        lines = rest.split("\n")
        note = [lines[0]]
        k = 1
        while k < len(lines) and lines[k].strip().startswith(";"):
            note.append(lines[k])
            k += 1
        out.append((label, "\n".join(note), "\n".join(lines[k:])))
    return out


def _innermost_loops(body):
    """{header: text of the loop's blocks} for loops no other loop nests in; a
    block belongs to loop X when its annotation says "in Loop: Header=X" or it is
    X's header."""
    blocks = _blocks(body)
    headers = {lab for lab, note, _ in blocks if "Loop Header" in note}
    parents = set(re.findall(r"Parent Loop (BB\d+_\d+)", "\n".join(n for _, n, _ in blocks)))
    # labels read ".LBB0_7"; annotations name the same block "BB0_7"
    inner = {h for h in headers if h[2:] not in parents}
    loops = {}
    for lab, note, text in blocks:
        m = re.search(r"in Loop: Header=(BB\d+_\d+)", note)
        owner = lab if lab in inner else (".L" + m.group(1) if m else None)
        if owner in inner:
            loops[owner] = loops.get(owner, "") + text
    return loops


@pytest.mark.parametrize("kernel", KERNELS)
def test_page_loop_never_drains_copies(decode_asm, kernel):
    body = _function(decode_asm, kernel)
    # the page loops: innermost loops that issue copies and run the MFMAs
    page_loops = [t for t in _innermost_loops(body).values() if "v_mfma" in t and "global_load_lds" in t]
    assert page_loops, "page loop not found"
    for loop in page_loops:
        waits = re.findall(r"s_waitcnt vmcnt\((\d+)\)", loop)
        assert waits and all(int(w) > 0 for w in waits), waits


@pytest.mark.parametrize("kernel,max_vgprs", [(KERNELS[0], 128), (KERNELS[1], 256)])
def test_waves_per_simd(decode_asm, kernel, max_vgprs):
    # the persistent grids: four NVFP4 workgroups of four waves per CU (four waves
    # per SIMD), four FP8 workgroups of two waves (two per SIMD)
    body_start = re.search(rf"^_Z\S*{kernel}\S*:", decode_asm, flags=re.M).start()
    meta = decode_asm[body_start:]
    vgprs = int(re.search(r"; NumVgprs:\s*(\d+)", meta).group(1))
    assert vgprs <= max_vgprs, vgprs


def test_no_packed_fp32_and_no_scratch(decode_asm):
    assert not re.search(r"v_pk_(add|mul|fma)_f32", decode_asm)
    for m in re.finditer(r"ScratchSize:\s*(\d+)", decode_asm):
        assert int(m.group(1)) == 0


@pytest.mark.parametrize("kernel", KERNELS)
def test_no_cache_wide_fences(decode_asm, kernel):
    """No device-scope acquire or release in the kernel: each would write back or
    invalidate a whole L2 per workgroup while the other workgroups of its XCD
    still stream (measured with a device-scope counter at workgroup exit: +37 us
    per launch)."""
    body = _function(decode_asm, kernel)
    assert not re.search(r"^\s*buffer_(wbl2|inv)\b", body, flags=re.M)


# ---- every source of the library ---------------------------------------------
@pytest.fixture(scope="module")
def all_asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa_all")
    return {src: _asm(d, os.path.join(B.CSRC, src)) for src in B.SOURCES}


def test_no_packed_fp32_and_no_scratch_anywhere(all_asm):
    """No packed-FP32 VALU instruction in any kernel of the library (the build
    turns the feature off), and no kernel spills to scratch."""
    for src, asm in all_asm.items():
        assert not re.search(r"v_pk_(add|mul|fma)_f32", asm), src
        for m in re.finditer(r"ScratchSize:\s*(\d+)", asm):
            assert int(m.group(1)) == 0, src


def test_quantize_encodes_with_the_fp4_conversion(all_asm):
    """The quantize kernel's fast encode: a NaN-propagating max for amax and the
    hardware f32 -> fp4 conversion of the corrected quotients (eight conversions
    per 16-value block, on each of its code paths)."""
    body = _function(all_asm["quantize.hip"], "10k_quantize")
    assert re.search(r"v_maximum3_f32", body)
    assert len(re.findall(r"v_cvt_scalef32_pk_fp4_f32", body)) >= 8


def test_dequant_has_no_mixed_fma(all_asm):
    """The dequant kernels' f16 and bf16 values are each one rounding of an exact
    product, and the sign of a zero product must survive. A multiply followed by
    the f16 rounding, left visible to the compiler, was once selected as one mixed
    fma (v_fma_mixlo_f16) with a +0 addend, which turns the product of a -0 code
    into +0 (the tiled workspace's V went through it); the V product now passes
    through an opaque register. No mixed fma may appear in any dequant kernel."""
    asm = all_asm["dequant.hip"]
    for kernel in ("9k_dequant", "15k_dequant_tiled"):
        body = _function(asm, kernel)
        assert not re.search(r"v_fma_mix(lo|hi)?_f16|v_mad_mix", body), kernel
