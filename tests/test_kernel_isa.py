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
    m = re.search(rf"^(_Z\S*{name}\S*):", asm, flags=re.M)
    assert m, name
    start = m.end()
    end = asm.index("s_endpgm", start)
    return asm[start:end]


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    return _asm(tmp_path_factory.mktemp("isa"), os.path.join(B.CSRC, "decode.hip"))


def test_copies_use_sgpr_base(decode_asm):
    body = _function(decode_asm, "k_decode_split")
    copies = re.findall(r"global_load_lds_dword\S*\s+([^\n]+)", body)
    assert copies, "no asynchronous copies found"
    for operands in copies:
        assert re.search(r",\s*s\[\d+:\d+\]", operands), operands


def _loops(body):
    """(header label, loop text) of every loop, the text running from the header
    to the branch back to it."""
    out = []
    # the "Loop Header" note sits on the label's line or on the comment line after it
    for head in re.findall(r"(\.LBB\d+_\d+):[^\n]*(?:\n\s*;[^\n]*)?Loop Header", body):
        text = body[body.index(head + ":"):]
        back = re.search(rf"s_c?branch\w*\s+{re.escape(head)}\b", text)
        out.append((head, text[:back.end()] if back else text))
    return out


def test_page_loop_never_drains_copies(decode_asm):
    body = _function(decode_asm, "k_decode_split")
    # the page loop: the innermost loop that issues copies and runs the MFMAs
    page_loops = [t for _, t in _loops(body) if "v_mfma" in t and "global_load_lds" in t]
    assert page_loops, "page loop not found"
    loop = min(page_loops, key=len)
    waits = re.findall(r"s_waitcnt vmcnt\((\d+)\)", loop)
    assert waits and all(int(w) > 0 for w in waits), waits


def test_four_waves_per_simd(decode_asm):
    # the persistent grid launches four workgroups of four waves per CU
    body_start = re.search(r"^_Z\S*k_decode_split\S*:", decode_asm, flags=re.M).start()
    meta = decode_asm[body_start:]
    vgprs = int(re.search(r"; NumVgprs:\s*(\d+)", meta).group(1))
    assert vgprs <= 128, vgprs


def test_no_packed_fp32_and_no_scratch(decode_asm):
    assert not re.search(r"v_pk_(add|mul|fma)_f32", decode_asm)
    for m in re.finditer(r"ScratchSize:\s*(\d+)", decode_asm):
        assert int(m.group(1)) == 0
