"""The LDS-direct loads write the M0 register inside inline asm that the
compiler does not see as an M0 user (exact_attention_23_amd/csrc/fa_device.hpp,
dma_to_lds). That is only safe while nothing else in the kernels uses M0. This
test compiles every HIP source of the library to gfx950 assembly, as the
build does, and fails if M0 appears anywhere except in those three-instruction
sequences (s_mov_b32 m0, s_nop 0, buffer_load_dword* ... lds), or if any
instruction that reads M0 implicitly (indirect register moves, GPR indexing,
messages, GWS and ordered-append LDS operations, LDS-direct and parameter
loads) is emitted. Runs on the CPU; hipcc cross-compiles without a GPU."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_23_amd import build

IMPLICIT_M0 = re.compile(r"\b(s_movrel\w*|v_movrel\w*|s_set_gpr_idx\w*|s_sendmsg\w*|ds_gws\w*|"
                         r"ds_append|ds_consume|ds_ordered\w*|lds_direct\w*|lds_param\w*|"
                         r"v_interp\w*|s_sleep_var)\b")


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++20", "--cuda-device-only",
           "-S", "-o", out, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form=1", src]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    with open(out, encoding="utf-8") as f:
        return f.read()


def _instructions(text: str):
    for line in text.splitlines():
        line = line.split(";")[0].strip()
        if line and not line.startswith((".", "//")) and not line.endswith(":"):
            yield line


def m0_violations(text: str):
    """Lines that use M0 outside the DMA sequences, and the number of DMA
    sequences seen."""
    ins = list(_instructions(text))
    bad, seqs = [], 0
    i = 0
    while i < len(ins):
        line = ins[i]
        if IMPLICIT_M0.search(line):
            bad.append(line)
        elif re.search(r"\bm0\b", line):
            ok = (re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", line) is not None and i + 2 < len(ins)
                  and ins[i + 1] == "s_nop 0"
                  and re.match(r"buffer_load_dword\w* .* lds$", ins[i + 2]) is not None)
            if ok:
                seqs += 1
                i += 3
                continue
            bad.append(line)
        i += 1
    return bad, seqs


def test_checker_catches_planted_uses():
    good = "s_mov_b32 m0, s4\ns_nop 0\nbuffer_load_dwordx4 v1, s[0:3], 0 offen lds\n"
    assert m0_violations(good) == ([], 1)
    assert m0_violations(good + "s_mov_b32 m0, s5\nv_add_f32 v1, v2, v3\n")[0]
    assert m0_violations(good + "v_movrels_b32 v0, v1\n")[0]
    assert m0_violations(good + "s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)\n")[0]
    assert m0_violations("s_mov_b32 m0, -1\nds_read_b32 v0, v1\n")[0]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_other_m0_use_in_library_assembly():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            texts = list(ex.map(lambda s: (s, _asm(s, tmp)), build.SOURCES))
    total = 0
    for src, text in texts:
        bad, seqs = m0_violations(text)
        assert not bad, f"{os.path.basename(src)}: M0 used outside the DMA sequences: {bad[:5]}"
        total += seqs
    assert total > 0, "no DMA sequence found: the check would be vacuous"
