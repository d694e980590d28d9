"""Checks on the gfx950 assembly of the kernels (host only: hipcc
cross-compiles without a GPU).

Each kernel source is compiled to assembly with the library's own flags and
every kernel in it is checked for properties the design relies on:

* no scratch (register spills), apart from a few known, bounded cases (stored
  before the key loop and reloaded in the epilogue);
* no packed fp32 instructions (the build disables them);
* M0 written only inside the inline assembly of the direct-to-LDS loads, so
  the value those loads depend on is never clobbered by compiler-generated
  code;
* no writes through the scalar data cache (stores, atomics, write-back) --
  vector stores only.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from exact_io_aware_attn_amd import build as B

KERNEL_SOURCES = ("attn_fwd_bf16.hip", "attn_fwd_pipe.hip", "attn_fwd_wide.hip", "attn_fwd_splitd.hip",
                  "attn_fwd_splitd8.hip", "attn_fwd_tiled.hip", "attn_merge.hip", "attn_quant.hip", "attn_bwd.hip",
                  "attn_fwd_p8.hip")

# kernels allowed a small spill: (source, kernel name fragment) -> max bytes
# (Q takes D/8 or D/4 VGPRs and O every accumulation register at these D)
KNOWN_SCRATCH = {
    # one 64-bit value kept across the key loop at three waves per SIMD
    # (168 of 170 VGPRs): stored before the loop, reloaded after it
    ("attn_fwd_bf16.hip", "attn_fwd_bf16_kernelILi128ELi32E"): 12,
    ("attn_fwd_wide.hip", "attn_fwd_wide_kernelILi512E"): 24,
    # backward dK/dV at D = 512, one wave per SIMD with all 512 registers
    # taken: values stored before and reloaded after each query-tile loop,
    # plus one dword reloaded per tile
    ("attn_bwd.hip", "attn_bwd_dkdv_split_kernelILi512E"): 204,
    ("attn_bwd.hip", "attn_bwd_dkdv_split_kernelILi448E"): 96,
}

SCALAR_WRITE = re.compile(r"\bs_(store|buffer_store|scratch_store|dcache_wb|dcache_discard|atomic|buffer_atomic)")
PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
M0 = re.compile(r"\bm0\b")


def _hipcc():
    return B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    hipcc = _hipcc()
    if not hipcc:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa")

    def compile_one(name):
        dst = os.path.join(out, name + ".s")
        cmd = [hipcc, *B.COMMON_FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, name), "-o", dst]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return name, dst

    with cf.ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
        return dict(ex.map(compile_one, KERNEL_SOURCES))


def kernels(path):
    """Per kernel: scratch bytes and the code lines outside/inside inline asm."""
    res, cur, in_asm = {}, None, False
    with open(path) as f:
        for line in f:
            m = re.match(r"^(_Z\S+):", line)
            if m:
                cur = m.group(1)
                res[cur] = {"scratch": None, "code": [], "asm": []}
                in_asm = False
                continue
            if cur is None:
                continue
            if ";;#ASMSTART" in line:
                in_asm = True
            elif ";;#ASMEND" in line:
                in_asm = False
            m = re.match(r"^; ScratchSize: (\d+)", line)
            if m and res[cur]["scratch"] is None:
                res[cur]["scratch"] = int(m.group(1))
            code = line.split(";")[0].strip()
            if code:
                res[cur]["asm" if in_asm else "code"].append(code)
    return res


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_kernel_assembly(assembly, src):
    ks = kernels(assembly[src])
    assert ks, f"no kernels found in {src}"
    for name, k in ks.items():
        assert k["scratch"] is not None, name
        limit = 0
        for (s, frag), lim in KNOWN_SCRATCH.items():
            if s == src and frag in name:
                limit = lim
        assert k["scratch"] <= limit, f"{name}: {k['scratch']} bytes of scratch"
        for line in k["code"] + k["asm"]:
            assert not SCALAR_WRITE.search(line), f"{name}: scalar-cache write: {line}"
            assert not PACKED_F32.search(line), f"{name}: packed fp32: {line}"
        for line in k["code"]:
            assert not M0.search(line), f"{name}: M0 used outside the direct-to-LDS asm: {line}"


def test_direct_to_lds_kernels_write_m0_only_in_asm(assembly):
    # the kernels that stream K/V with direct-to-LDS loads set M0 in their asm
    for src in ("attn_fwd_pipe.hip", "attn_fwd_wide.hip", "attn_fwd_splitd.hip", "attn_fwd_splitd8.hip"):
        for name, k in kernels(assembly[src]).items():
            assert any(M0.search(l) for l in k["asm"]), f"{name}: no M0 write in its direct-to-LDS asm"
            assert any("lds" in l and "buffer_load" in l for l in k["asm"]), name
