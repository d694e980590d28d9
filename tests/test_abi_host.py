"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

The library must load, export every function ``include/attn.h`` declares,
and reject invalid arguments with the documented codes before anything is
enqueued (validation returns before any HIP call).
"""
import ctypes
import os
import re
import subprocess

import pytest

from exact_io_aware_attn_amd import attn as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 1 << 20  # an aligned, never-dereferenced address: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(A.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    L = A.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings_and_version():
    L = A.lib()
    assert L.attn_status_string(0) == b"ATTN_OK"
    assert L.attn_status_string(1) == b"ATTN_ERR_INVALID_ARG"
    assert L.attn_status_string(2) == b"ATTN_ERR_UNSUPPORTED"
    assert L.attn_status_string(3) == b"ATTN_ERR_HIP"
    assert L.attn_status_string(99) == b"ATTN_UNKNOWN_STATUS"
    assert L.attn_version() >= 100


def call(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, D=128, causal=0,
         scale=0.1, dtype=A.ATTN_BF16):
    return A.raw_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None),
    dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Nq=0), dict(Nkv=0), dict(D=0), dict(B=-3),
    dict(Hq=6, Hkv=4), dict(scale=float("inf")), dict(scale=float("nan")), dict(dtype=7),
    dict(q=FAKE + 8), dict(o=FAKE + 2), dict(lse=FAKE + 1),
])
def test_invalid_arguments(kw):
    assert call(**kw) == A.ATTN_ERR_INVALID_ARG
    assert A.lib().attn_last_error() != b""


@pytest.mark.parametrize("kw", [
    dict(D=48), dict(D=1056), dict(D=2048), dict(D=288), dict(D=352),
    dict(D=256, dtype=A.ATTN_F32), dict(D=96, dtype=A.ATTN_FP8_E4M3), dict(D=512, dtype=A.ATTN_FP8_E4M3),
    dict(D=512, dtype=A.ATTN_F32),
    dict(Nkv=(1 << 31) // 256, D=128),            # K slab reaches 2^31 bytes
    dict(Nq=1 << 24, D=128),                       # Q slab reaches 2^31 bytes
])
def test_unsupported(kw):
    assert call(**kw) == A.ATTN_ERR_UNSUPPORTED


def test_fp8_descale_alignment():
    st = A.raw_fwd_fp8(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 2, 64, 64, 128, 0, 0.1, FAKE + 2, None, None)
    assert st == A.ATTN_ERR_INVALID_ARG


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(A, "_lib", None)
    monkeypatch.setattr(A, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(A.AttnError):
        A.lib()
