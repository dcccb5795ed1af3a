"""The C-ABI library loads and exports every function include/ttt.h declares (no GPU needed).

Only host-side paths are exercised here: symbol lookup, the status strings, and argument
validation that ttt_create / ttt_test_gemm perform before touching a device.
"""
import ctypes
import os
import re

import pytest

import test_long_context_chunk_amd as ttt
from test_long_context_chunk_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ttt_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ttt.lib_path()):
        pytest.fail("the HIP library is not built (run python -m test_long_context_chunk_amd.build)")
    return ttt.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["ttt_create", "ttt_prefill_chunks", "ttt_token_losses", "ttt_fast_weights", "ttt_destroy"]:
        assert must in names
    assert set(names) == set(B.SIGNATURES), "binding signatures and header disagree"


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in B.STATUS:
        s = lib.ttt_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.ttt_status_string(123) == b"unknown status"


def test_config_struct_layout_matches_header():
    # int32 x 10, int64, float x 4 -> 40 + 8 + 16 bytes
    assert ctypes.sizeof(B.Config) == 64
    assert B.Config.max_tokens.offset == 40
    assert ctypes.sizeof(B.Weights) == 5 * ctypes.sizeof(ctypes.c_void_p)


def _cfg(**kw):
    base = dict(abi_version=B.ABI_VERSION, vocab=256, d_model=64, d_hidden=256, n_blocks=1, mlp=0,
                norm=0, precision=0, chunk=1, reserved=0, max_tokens=128, lr=0.1, clip=0.0,
                rms_eps=1e-6, reserved_f=0.0)
    base.update(kw)
    return B.Config(**base)


@pytest.mark.parametrize("bad", [
    dict(abi_version=99), dict(vocab=1), dict(vocab=250), dict(d_model=60), dict(d_hidden=12),
    dict(n_blocks=-1), dict(mlp=7), dict(norm=3), dict(precision=5), dict(chunk=0),
    dict(max_tokens=0), dict(max_tokens=130, chunk=4), dict(lr=-1.0), dict(reserved=1),
    dict(mlp=1, n_blocks=2), dict(norm=1, rms_eps=0.0), dict(clip=float("nan")),
])
def test_create_rejects_bad_config_before_touching_a_device(lib, bad):
    cfg = _cfg(**bad)
    dummy = (ctypes.c_void_p * 1)(1)
    w = B.Weights(1, 1, ctypes.cast(dummy, ctypes.POINTER(ctypes.c_void_p)), None,
                  ctypes.cast(dummy, ctypes.POINTER(ctypes.c_void_p)))
    out = ctypes.c_void_p(12345)
    assert lib.ttt_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out)) == -1
    assert out.value is None


def test_create_rejects_missing_weights(lib):
    cfg = _cfg()
    w = B.Weights(None, None, None, None, None)
    out = ctypes.c_void_p()
    assert lib.ttt_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out)) == -1


@pytest.mark.parametrize("streams,chunk,max_tokens", [
    (0, 64, 128), (-3, 64, 128), (4097, 64, 128),  # stream count outside [1, TTT_MAX_STREAMS]
    (2, 1, 128), (3, 96, 192),                      # several streams need whole 64-row groups
    (64, 65536, 65536),                             # more than 2^21 rows per step
])
def test_create_batch_rejects_bad_stream_counts_before_touching_a_device(lib, streams, chunk, max_tokens):
    cfg = _cfg(chunk=chunk, max_tokens=max_tokens)
    dummy = (ctypes.c_void_p * 1)(1)
    w = B.Weights(1, 1, ctypes.cast(dummy, ctypes.POINTER(ctypes.c_void_p)), None,
                  ctypes.cast(dummy, ctypes.POINTER(ctypes.c_void_p)))
    out = ctypes.c_void_p(12345)
    assert lib.ttt_create_batch(ctypes.byref(cfg), ctypes.byref(w), streams, None, ctypes.byref(out)) == -1
    assert out.value is None


@pytest.mark.parametrize("ms,win,heads,reserved,mlp,prec,d,ptrs", [
    (12, 0, 0, 0, 0, 1, 128, True),    # static hidden size not a multiple of 8
    (4, 0, 0, 0, 0, 1, 128, True),     # below 8
    (16, 0, 0, 1, 0, 1, 128, True),    # reserved field set
    (16, 0, 0, 0, 1, 1, 128, True),    # static MLP with the SwiGLU block
    (16, 0, 0, 0, 0, 1, 128, False),   # missing weight arrays
    (0, 64, 1, 0, 0, 0, 128, True),    # attention in fp32
    (0, 64, 2, 0, 0, 1, 128, True),    # heads of 64, not 128
    (0, 64, 0, 0, 0, 1, 128, True),    # no heads
    (0, 64, 1, 0, 0, 1, 128, False),   # missing attention weights
    (0, -1, 1, 0, 0, 1, 128, True),    # negative window
])
def test_create_ext_rejects_bad_extensions_before_touching_a_device(lib, ms, win, heads, reserved, mlp, prec, d,
                                                                     ptrs):
    cfg = _cfg(mlp=mlp, precision=prec, d_model=d)
    dummy = (ctypes.c_void_p * 1)(1)
    arr = ctypes.cast(dummy, ctypes.POINTER(ctypes.c_void_p))
    w = B.Weights(1, 1, arr, arr if mlp == 1 else None, arr)
    p = arr if ptrs else None
    ext = B.BlockExt(ms, win, heads, reserved, p, p, p, p, p, p)
    out = ctypes.c_void_p(12345)
    assert lib.ttt_create_ext(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ext), 1, None, ctypes.byref(out)) == -1
    assert out.value is None


def test_block_ext_struct_layout_matches_header():
    assert B.BlockExt.ws1.offset == 16
    assert B.BlockExt.wo.offset == 16 + 5 * ctypes.sizeof(ctypes.c_void_p)
    assert ctypes.sizeof(B.BlockExt) == 16 + 6 * ctypes.sizeof(ctypes.c_void_p)


def test_null_context_calls_are_rejected(lib):
    assert lib.ttt_prefill_chunks(None, None, 8) == -1
    assert lib.ttt_token_losses(None, None, 0, 0) == -1
    assert lib.ttt_sync(None) == -1
    assert lib.ttt_destroy(None) == 0
    assert lib.ttt_tokens_consumed(None) == -1
    assert lib.ttt_decode(None, None, 1, None, None) == -1
    assert lib.ttt_decode_pending(None) == -1
    assert lib.ttt_profile_period(None, 1) == -1
    assert lib.ttt_streams(None) == -1
    assert lib.ttt_prefill_batch(None, None, 9, 8) == -1
    assert lib.ttt_stream_token_losses(None, 0, None, 0, 0) == -1
    assert lib.ttt_stream_token_argmax(None, 0, None, 0, 0) == -1
    assert lib.ttt_stream_chunk_stats(None, 0, None, 0, 0) == -1
    assert lib.ttt_stream_fast_weights(None, 0, 0, 2, 0, None) == -1


def test_gemm_hook_validates_shapes(lib):
    # K not a multiple of the 16-byte operand chunk
    assert lib.ttt_test_gemm(1, 1, 8, 1, 8, 1, 8, 4, 4, 6, None) == -1
    assert lib.ttt_test_gemm(0, 1, 8, 1, 8, 1, 8, 4, 4, 6, None) == -1
    assert lib.ttt_test_gemm(7, 1, 8, 1, 8, 1, 8, 4, 4, 8, None) == -1
    # the gradient hook: K not a multiple of 64, M not a multiple of 8 (token-major), a bad
    # layout flag, NULL operands
    assert lib.ttt_test_grad(1, 64, 1, 64, 1, 64, 1, 64, 64, 32, 1, None) == -1
    assert lib.ttt_test_grad(1, 64, 1, 64, 1, 64, 1, 60, 64, 64, 1, None) == -1
    assert lib.ttt_test_grad(1, 64, 1, 64, 1, 64, 1, 64, 64, 64, 2, None) == -1
    assert lib.ttt_test_grad(None, 64, 1, 64, 1, 64, 1, 64, 64, 64, 1, None) == -1
    # the two-weight hook: K not a multiple of 8, splits out of range, a NULL second weight
    assert lib.ttt_test_gemm_pair(1, 8, 1, 8, 1, 8, 1, 8, 4, 4, 6, 1, 0, None) == -1
    assert lib.ttt_test_gemm_pair(1, 8, 1, 8, 1, 8, 1, 8, 4, 4, 8, 0, 0, None) == -1
    assert lib.ttt_test_gemm_pair(1, 8, 1, 8, 1, 8, 1, 8, 4, 4, 8, 9, 0, None) == -1
    assert lib.ttt_test_gemm_pair(1, 8, 1, 8, None, 8, 1, 8, 4, 4, 8, 1, 0, None) == -1
    assert lib.ttt_test_gemm_pair(1, 8, 1, 8, 1, 8, 1, 8, 4, 4, 8, 1, 3, None) == -1


def test_kernel_kind_names_match_the_header():
    """The binding's kind names index the per-kind arrays that ttt_profile_read fills."""
    import re
    from test_long_context_chunk_amd import _binding
    hdr = open(os.path.join(ROOT, "include", "ttt.h")).read()
    kinds = re.findall(r"TTT_K_(\w+) = (\d+),", hdr)
    count = int(re.search(r"TTT_K_COUNT = (\d+)", hdr).group(1))
    assert [int(v) for _, v in kinds] == list(range(count))
    assert len(_binding.KERNEL_KINDS) == count


def test_a_missing_library_raises_instead_of_falling_back(tmp_path):
    """No compute path exists outside the HIP library: loading one that is not there raises."""
    with pytest.raises(RuntimeError, match="not built"):
        B.load_library(str(tmp_path / "libttt_missing.so"))
