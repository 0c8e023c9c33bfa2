"""Checks on the built gfx950 device code (no GPU needed: hipcc cross-compiles).

The split-KV attention kernel issues its direct global->LDS loads from inline
asm that writes M0 (the LDS destination register of those loads).  The
compiler reserves M0 and does not honour a clobber of it: if it kept a value
of its own in M0 across such a statement, that value would be overwritten
silently.  So every kernel that contains the asm must leave M0 to the asm
alone.  This test compiles kernels.hip to device assembly with the library's
own flags and checks that, and that the asm blocks still hold what they
should (M0 set, then the load, in one block).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

M0 = re.compile(r"(?<![\w])m0(?![\w])")


def _device_asm(tmp_path):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    from block_diffusion_drafter_context_amd import build as b
    out = tmp_path / "kernels.s"
    cmd = [HIPCC] + b.HIP_FLAGS + ["--cuda-device-only", "-S", "-I", b.INCLUDE,
                                   os.path.join(b.CSRC, "kernels.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return out.read_text()


def _functions(asm):
    """{mangled kernel name: [(in_asm_block, instruction text)]}"""
    funcs, cur, in_asm = {}, None, False
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur, in_asm = m.group(1), False
            funcs[cur] = []
            continue
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if cur is None or not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        funcs[cur].append((in_asm, s.split(";")[0].strip()))
    return funcs


def test_m0_left_to_the_lds_dma_asm(tmp_path):
    funcs = _functions(_device_asm(tmp_path))
    users = {n: ins for n, ins in funcs.items()
             if any(a and "global_load_lds" in t for a, t in ins)}
    # the attention kernels (every dtype, head size and mask mode) use it
    assert sum("attn_split_kernel" in n for n in users) >= 8, sorted(users)[:4]
    for name, ins in users.items():
        compiler_m0 = [t for a, t in ins if not a and M0.search(t)]
        assert not compiler_m0, f"{name}: compiler-generated M0 use next to the LDS DMA asm: {compiler_m0[:3]}"
        # within the asm: each load directly follows its own M0 write
        block = [t for a, t in ins if a]
        for i, t in enumerate(block):
            if "global_load_lds" in t:
                assert i >= 2 and block[i - 2].startswith("s_mov_b32 m0,"), f"{name}: {block[max(0, i - 2):i + 1]}"
