"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

The library must load, export every function ``include/attn.h`` declares,
and reject invalid arguments with the documented codes before anything is
enqueued (validation returns before any HIP call).  On a machine with no GPU
a fully valid call returns ATTN_ERR_HIP (skipped where a GPU is visible).
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
    dict(D=48), dict(D=1056), dict(D=2048), dict(D=1000),
    dict(D=256, dtype=A.ATTN_F32), dict(D=96, dtype=A.ATTN_FP8_E4M3), dict(D=512, dtype=A.ATTN_FP8_E4M3),
    dict(D=512, dtype=A.ATTN_F32),
    dict(Nkv=(1 << 31) // 256, D=128),            # K slab reaches 2^31 bytes
    dict(Nq=1 << 24, D=128),                       # Q slab reaches 2^31 bytes
])
def test_unsupported(kw):
    assert call(**kw) == A.ATTN_ERR_UNSUPPORTED


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is visible: this call on fake pointers would launch")
@pytest.mark.parametrize("D", [128, 288, 1024])
def test_valid_call_without_a_device_reports_hip_error(D):
    # every argument valid, no GPU in the machine: the launch fails in the
    # HIP runtime, which the ABI reports as ATTN_ERR_HIP with its message
    assert call(D=D) == A.ATTN_ERR_HIP
    assert b"device" in A.lib().attn_last_error()


def test_fp8_descale_alignment():
    st = A.raw_fwd_fp8(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 2, 64, 64, 128, 0, 0.1, FAKE + 2, None, None)
    assert st == A.ATTN_ERR_INVALID_ARG


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(A, "_lib", None)
    monkeypatch.setattr(A, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(A.AttnError):
        A.lib()


# ---------------------------------------------------------------------------
# key ranges, merge and split-KV: validation only (every call below fails
# before anything is enqueued)
# ---------------------------------------------------------------------------

def call_partial(lse=FAKE, kv_begin=0, kv_end=64, Nkv=64, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=2, Hkv=2, Nq=64, D=128, causal=0, scale=0.1,
             dtype=A.ATTN_BF16)
    a.update(kw)
    return A.lib().attn_fwd_partial(a["q"], a["k"], a["v"], a["o"], lse, a["B"], a["Hq"], a["Hkv"], a["Nq"], Nkv,
                                    a["D"], a["causal"], a["scale"], a["dtype"], kv_begin, kv_end,
                                    a.get("dq"), None, None, None)


@pytest.mark.parametrize("kw", [
    dict(lse=None), dict(kv_begin=-1), dict(kv_begin=10, kv_end=5), dict(kv_end=65), dict(q=None),
    dict(B=0), dict(Hq=3, Hkv=2), dict(dq=FAKE),                 # descale with a bf16 dtype
    dict(dq=FAKE + 2, dtype=A.ATTN_FP8_E4M3),                    # misaligned descale
])
def test_partial_invalid_arguments(kw):
    assert call_partial(**kw) == A.ATTN_ERR_INVALID_ARG
    assert A.lib().attn_last_error() != b""


def call_merge(o_parts=FAKE, lse_parts=FAKE, n_parts=2, o=FAKE, lse=None, B=1, Hq=2, Nq=16, D=128,
               out_dtype=A.ATTN_BF16):
    return A.lib().attn_merge(o_parts, lse_parts, n_parts, o, lse, B, Hq, Nq, D, out_dtype, None)


@pytest.mark.parametrize("kw", [
    dict(o_parts=None), dict(lse_parts=None), dict(o=None), dict(n_parts=0), dict(Nq=0), dict(D=0),
    dict(out_dtype=A.ATTN_FP8_E4M3), dict(out_dtype=9), dict(o_parts=FAKE + 4), dict(o=FAKE + 8),
    dict(lse_parts=FAKE + 2), dict(lse=FAKE + 1),
])
def test_merge_invalid_arguments(kw):
    assert call_merge(**kw) == A.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("D", [48, 1056])
def test_merge_unsupported(D):
    assert call_merge(D=D) == A.ATTN_ERR_UNSUPPORTED


def test_splitkv_workspace_size():
    f = A.lib().attn_splitkv_workspace_bytes
    # per part: float32 O rounded up to 256 bytes, then float32 LSE likewise
    assert f(1, 2, 3, 32, 1) == (1 * 2 * 3 * 32 * 4 + 255) // 256 * 256 + 256
    assert f(2, 4, 100, 128, 5) == 5 * ((2 * 4 * 100 * 128 * 4 + 255) // 256 * 256 + (2 * 4 * 100 * 4 + 255) // 256 * 256)
    assert f(0, 2, 3, 32, 1) == 0 and f(1, 2, 3, 32, 0) == 0


def call_splitkv(n_splits=4, ws=FAKE, ws_bytes=1 << 40, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, D=128, causal=0,
             scale=0.1, dtype=A.ATTN_BF16)
    a.update(kw)
    return A.lib().attn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                    a["Nkv"], a["D"], a["causal"], a["scale"], a["dtype"], a.get("dq"), None, None,
                                    n_splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(n_splits=0), dict(n_splits=5000), dict(ws=None), dict(ws_bytes=100), dict(ws=FAKE + 16),
    dict(Nq=0), dict(q=None), dict(scale=float("nan")), dict(Hq=3, Hkv=2), dict(dq=FAKE),
    dict(dq=FAKE + 2, dtype=A.ATTN_FP8_E4M3),
])
def test_splitkv_invalid_arguments(kw):
    assert call_splitkv(**kw) == A.ATTN_ERR_INVALID_ARG


def quant(x=FAKE, codes=FAKE, desc=FAKE, B=1, H=2, N=100, D=128, signs=None):
    return A.lib().attn_quantize_fp8(x, codes, desc, B, H, N, D, signs, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(codes=None), dict(desc=None), dict(B=0), dict(H=0), dict(N=0), dict(D=0), dict(N=-1),
    dict(x=FAKE + 2), dict(codes=FAKE + 8), dict(desc=FAKE + 2),
])
def test_quantize_invalid_arguments(kw):
    assert quant(**kw) == A.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("D", [32, 96, 192, 512])
def test_quantize_unsupported_head_dim(D):
    assert quant(D=D) == A.ATTN_ERR_UNSUPPORTED


def blocks(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, D=128, causal=0,
           scale=0.1, dq=FAKE, dk=FAKE, dv=FAKE):
    return A.lib().attn_fwd_fp8_blocks(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dq, dk, dv, None)


@pytest.mark.parametrize("kw", [
    dict(dq=None), dict(dk=None), dict(dv=None), dict(q=None), dict(B=0), dict(Hq=3, Hkv=2),
    dict(scale=float("nan")), dict(q=FAKE + 8),
])
def test_blocks_invalid_arguments(kw):
    assert blocks(**kw) == A.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=96), dict(D=512), dict(D=32), dict(scale=0.0), dict(scale=-0.5)])
def test_blocks_unsupported(kw):
    assert blocks(**kw) == A.ATTN_ERR_UNSUPPORTED


def bwd_call(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=2, Hkv=2,
             Nq=64, Nkv=64, D=128, causal=0, scale=0.1, dtype=A.ATTN_BF16, ws=FAKE, ws_bytes=1 << 20):
    return A.lib().attn_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, ws,
                            ws_bytes, None)


def test_bwd_workspace_size():
    assert A.bwd_workspace_bytes(2, 3, 100) == 2 * ((2 * 3 * 100 * 4 + 255) // 256 * 256)
    assert A.bwd_workspace_bytes(0, 3, 100) == 0


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(lse=None), dict(do=None), dict(dq=None), dict(dk=None), dict(dv=None), dict(ws=None),
    dict(ws_bytes=16), dict(B=0), dict(Hq=3, Hkv=2), dict(scale=float("nan")), dict(dtype=9), dict(q=FAKE + 8),
    dict(lse=FAKE + 2), dict(ws=FAKE + 4),
])
def test_bwd_invalid_arguments(kw):
    assert bwd_call(**kw) == A.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=96), dict(D=160), dict(D=576), dict(D=1024), dict(dtype=A.ATTN_F32), dict(dtype=A.ATTN_FP8_E4M3)])
def test_bwd_unsupported(kw):
    assert bwd_call(**kw) == A.ATTN_ERR_UNSUPPORTED


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.mark.skipif(_gpu_visible(), reason="a GPU is visible: the call would launch")
def test_valid_call_without_device_returns_hip_error():
    # Arguments pass validation, so the call reaches the launch, which fails
    # without a device: ATTN_ERR_HIP, with the HIP error in the message.
    st = call(B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, D=128)
    assert st == A.ATTN_ERR_HIP
    assert b"launch failed" in A.lib().attn_last_error()


def test_binding_output_buffer_checks():
    import torch
    dev = torch.device("cpu")
    shape = (1, 2, 8, 64)
    good = torch.empty(shape, dtype=torch.bfloat16)
    assert A._buffer(good, "out", shape, torch.bfloat16, dev) is good
    assert A._buffer(None, "out", shape, torch.bfloat16, dev).shape == shape
    with pytest.raises(ValueError, match="shape"):
        A._buffer(torch.empty((1, 2, 7, 64), dtype=torch.bfloat16), "out", shape, torch.bfloat16, dev)
    with pytest.raises(ValueError, match="dtype"):
        A._buffer(torch.empty(shape, dtype=torch.float32), "out", shape, torch.bfloat16, dev)
    with pytest.raises(ValueError, match="contiguous"):
        A._buffer(torch.empty((1, 2, 64, 8), dtype=torch.bfloat16).transpose(2, 3), "out", shape, torch.bfloat16,
                  dev)
    with pytest.raises(ValueError, match="expected meta"):
        A._buffer(good, "out", shape, torch.bfloat16, torch.device("meta"))
    ws = torch.empty(100, dtype=torch.uint8)
    assert A._workspace(ws, 100, dev) is ws
    with pytest.raises(ValueError, match="needed"):
        A._workspace(ws, 101, dev)
    assert A._workspace(torch.empty(30, dtype=torch.float32), 120, dev).numel() == 30


def noalloc(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, D=128, causal=0,
            scale=0.1, dtype=A.ATTN_BF16, n_splits=2):
    return A.lib().attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype,
                                            None, None, None, n_splits, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(o=None), dict(q=FAKE + 8), dict(B=0), dict(Hq=3, Hkv=2), dict(Hkv=0),
    dict(scale=float("nan")), dict(dtype=9), dict(n_splits=0), dict(n_splits=5000),
])
def test_noalloc_invalid_arguments(kw):
    assert noalloc(**kw) == A.ATTN_ERR_INVALID_ARG
    assert A.lib().attn_last_error() != b""


def test_noalloc_scratch_limit():
    # 32 heads x 4096 rows x 128 x 4 bytes x 8 splits = 512 MiB of partials
    assert A.splitkv_workspace_bytes(1, 32, 4096, 128, 8) > A.NOALLOC_SCRATCH_BYTES
    assert noalloc(Hq=32, Hkv=8, Nq=4096, Nkv=4096, n_splits=8) == A.ATTN_ERR_UNSUPPORTED
    assert b"scratch" in A.lib().attn_last_error()
    hdr = open(HEADER).read()
    assert re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", hdr)
    assert A.NOALLOC_SCRATCH_BYTES == 64 << 20


@pytest.mark.skipif(_gpu_visible(), reason="a GPU is visible: the call would launch")
def test_noalloc_without_device_returns_hip_error():
    assert noalloc() == A.ATTN_ERR_HIP


def test_last_error_is_per_thread():
    """attn_last_error describes the last failure on the calling thread: two
    threads failing in different ways at the same time (ctypes releases the
    interpreter lock around each call) each read back their own message, and
    a thread that has not failed reads an empty string."""
    import threading
    L = A.lib()
    errors = []
    start = threading.Barrier(2)

    def worker(kw, expect_status, expect_text):
        try:
            start.wait()
            for _ in range(2000):
                assert call(**kw) == expect_status
                msg = L.attn_last_error().decode()
                assert expect_text in msg, msg
        except Exception as e:  # reported below
            errors.append(e)

    t1 = threading.Thread(target=worker, args=(dict(D=48), A.ATTN_ERR_UNSUPPORTED, "D=48"))
    t2 = threading.Thread(target=worker, args=(dict(Hq=6, Hkv=4), A.ATTN_ERR_INVALID_ARG, "Hq"))
    t1.start(); t2.start(); t1.join(); t2.join()
    assert not errors, errors[0]

    fresh = []
    t3 = threading.Thread(target=lambda: fresh.append(L.attn_last_error()))
    t3.start(); t3.join()
    assert fresh == [b""]
