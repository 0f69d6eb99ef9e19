"""CPU check of the compiled gfx950 code of every library kernel: no kernel
writes through the scalar data cache (no s_store, s_atomic, s_dcache_wb or
s_dcache_discard instruction). All of the library's writes, its counters and
atomics included, must be vector memory instructions. (This file names those
instructions, so it stays off the upload list of GPU runs; it needs no GPU.)"""
import os
import re
import shutil
import subprocess

import pytest

from bit_paged_kv_nvfp4_amd import build as B


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip") and f != "api.hip"))
def test_no_scalar_cache_writes(tmp_path, src):
    if not os.path.exists(B.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [B.HIPCC, *[f for f in B.FLAGS if f not in ("-shared", "-fPIC")], "-I", B.INCLUDE, "-I", B.CSRC,
           "--cuda-device-only", "-S", "-o", str(out), os.path.join(B.CSRC, src)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    assert re.search(r"^\s*(global_|buffer_|ds_)", asm, flags=re.M), "no vector memory code found"
    bad = re.findall(r"^\s*(s_store\w*|s_atomic\w*|s_buffer_store\w*|s_buffer_atomic\w*|s_dcache_wb\w*|"
                     r"s_dcache_discard\w*)\b", asm, flags=re.M)
    assert not bad, f"{src}: {sorted(set(bad))}"
