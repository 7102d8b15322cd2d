"""The C-ABI library on a host without a GPU: it loads, exports every entry
point include/moe_mxfp4.h declares, and rejects bad arguments before it
touches the device (CPU only; no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")
from mxfp4_routed_expert_02_amd._binding import LIB_PATH as LIB  # noqa: E402 (the sanitized build under MOE_SANITIZE=1)

OK, INVALID, UNSUPPORTED, WS_SMALL, HIPERR, SCRATCH_SMALL = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail("libmoe_mxfp4.so is not built (run __graft_entry__.build())")
    from mxfp4_routed_expert_02_amd import _binding

    return _binding.lib()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ("moe_route_topk", "moe_group_rows", "moe_expert_ffn_mxfp4", "moe_combine"):
        assert f in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in range(6):
        assert L.moe_status_string(s).startswith(b"MOE_")


def test_workspace_bytes_ranges(L):
    assert L.moe_workspace_bytes(1, 16, 896, 7168, 1536) >= 16 * 1536 * 4
    assert L.moe_workspace_bytes(512, 16, 896, 7168, 1536) >= 8192 * 1536 * 4
    assert L.moe_workspace_bytes(1, 0, 896, 7168, 1536) == 0
    assert L.moe_workspace_bytes(1, 16, 896, 7100, 1536) == 0  # H not a multiple of 32
    assert L.moe_workspace_bytes(1, 16, 5000, 7168, 1536) == 0  # E above the maximum
    assert L.moe_workspace_bytes(1, 33, 896, 7168, 1536) == 0  # k above the maximum


FAKE = 0x10000  # a 16-byte aligned non-null pointer value; never dereferenced


def test_route_rejects_bad_arguments(L):
    assert L.moe_route_topk(None, 1, 8, 2, FAKE, FAKE, None) == INVALID
    assert L.moe_route_topk(FAKE, -1, 8, 2, FAKE, FAKE, None) == INVALID
    assert L.moe_route_topk(FAKE, 1, 8, 9, FAKE, FAKE, None) == INVALID  # k > E
    assert L.moe_route_topk(FAKE, 1, 64, 33, FAKE, FAKE, None) == INVALID  # k > 32
    assert L.moe_route_topk(FAKE, 1, 0, 1, FAKE, FAKE, None) == INVALID
    assert L.moe_route_topk(FAKE, 1, 4097, 1, FAKE, FAKE, None) == INVALID


def test_group_rejects_bad_arguments(L):
    assert L.moe_group_rows(FAKE, 1, 2, 8, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID
    assert L.moe_group_rows(FAKE, 1, 0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID
    assert L.moe_group_rows(FAKE, 1, 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID
    # more than 512 rows need the chunk counts in the workspace
    need = L.moe_workspace_bytes(512, 16, 896, 7168, 1536)
    assert need >= (32 * 896 + 8192) * 4
    assert L.moe_group_rows(FAKE, 512, 16, 896, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, None) == WS_SMALL
    assert L.moe_group_rows(FAKE, 512, 16, 896, FAKE, FAKE, FAKE, FAKE, None, need, None) == INVALID
    assert L.moe_group_rows(FAKE, 512, 16, 896, FAKE, FAKE, FAKE, FAKE, FAKE + 4, need, None) == INVALID


def _weights(H=256, I=128, E=8, misalign=0, stride=None, scale_misalign=0):
    from mxfp4_routed_expert_02_amd._binding import MoeWeights

    sb = 3 * (I * H // 2 + I * H // 32)
    return MoeWeights(FAKE + misalign, FAKE, FAKE, FAKE, FAKE, FAKE + scale_misalign, sb if stride is None else stride,
                      E, H, I)


def test_ffn_rejects_bad_arguments(L):
    big = 1 << 30
    w = _weights()
    assert L.moe_expert_ffn_mxfp4(None, 4, 2, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == INVALID
    assert L.moe_expert_ffn_mxfp4(FAKE + 2, 4, 2, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, big,
                                  None) == INVALID  # x misaligned
    assert L.moe_expert_ffn_mxfp4(FAKE, 4, 2, None, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == INVALID
    bad = _weights(misalign=8)
    assert L.moe_expert_ffn_mxfp4(FAKE, 4, 2, ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == INVALID
    bad = _weights(H=250)
    assert L.moe_expert_ffn_mxfp4(FAKE, 4, 2, ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == INVALID
    bad = _weights(stride=100)
    assert L.moe_expert_ffn_mxfp4(FAKE, 4, 2, ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == INVALID
    bad = _weights(scale_misalign=2)  # down_s not 4-byte aligned
    assert L.moe_expert_ffn_mxfp4(FAKE, 4, 2, ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == INVALID
    assert L.moe_expert_ffn_mxfp4(FAKE, 4, 2, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                                  None) == WS_SMALL


def test_combine_and_rescale_reject_bad_arguments(L):
    assert L.moe_combine(FAKE, FAKE, FAKE, 1, 2, 64, None, None) == INVALID
    assert L.moe_combine(FAKE + 4, FAKE, FAKE, 1, 2, 64, FAKE, None) == INVALID
    assert L.moe_combine(FAKE, FAKE, FAKE, 1, 2, 0, FAKE, None) == INVALID
    assert L.moe_rms_rescale_bf16(FAKE, 1, 0, 1e-6, FAKE, None) == INVALID
    assert L.moe_rms_rescale_bf16(FAKE, 1, 64, -1.0, FAKE, None) == INVALID
    assert L.moe_rms_rescale_bf16(FAKE, 1, 48, 1e-6, FAKE, None) == INVALID  # H not a multiple of 32
    assert L.moe_rms_rescale_bf16(FAKE + 4, 1, 64, 1e-6, FAKE, None) == INVALID  # y not 16-byte aligned


def test_router_logits_validation(L):
    assert L.moe_router_logits(FAKE, 1, 7168, FAKE, 896, FAKE, None) == HIPERR  # valid args, no GPU here
    assert L.moe_router_logits(FAKE, -1, 7168, FAKE, 896, FAKE, None) == INVALID
    assert L.moe_router_logits(FAKE, 1, 7100, FAKE, 896, FAKE, None) == INVALID  # H not a multiple of 32
    assert L.moe_router_logits(FAKE, 1, 7168, FAKE, 0, FAKE, None) == INVALID
    assert L.moe_router_logits(FAKE, 1, 7168, FAKE, 5000, FAKE, None) == INVALID
    assert L.moe_router_logits(None, 1, 7168, FAKE, 896, FAKE, None) == INVALID
    assert L.moe_router_logits(FAKE + 8, 1, 7168, FAKE, 896, FAKE, None) == INVALID  # x not 16-byte aligned
    assert L.moe_router_logits(FAKE, 1, 7168, FAKE + 4, 896, FAKE, None) == INVALID  # w not 16-byte aligned
    assert L.moe_router_logits(None, 0, 7168, None, 896, None, None) == HIPERR  # empty batch: nothing to check


def test_valid_call_without_gpu_reports_hip_error(L):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path only")
    assert L.moe_route_topk(FAKE, 1, 8, 2, FAKE, FAKE, None) == HIPERR


def test_fused_calls_validation(L):
    # moe_route_group_one: nulls, k out of range
    assert L.moe_route_group_one(None, 896, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert L.moe_route_group_one(FAKE, 896, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert L.moe_route_group_one(FAKE, 8, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert L.moe_route_group_one(FAKE, 896, 33, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert L.moe_route_group_one(FAKE, 896, 16, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == INVALID
    # moe_combine_rms_bf16: H not a multiple of 32, misaligned x_next, negative eps, nulls
    assert L.moe_combine_rms_bf16(FAKE, FAKE, FAKE, 1, 16, 100, 1e-6, FAKE, FAKE, None) == INVALID
    assert L.moe_combine_rms_bf16(FAKE, FAKE, FAKE, 1, 16, 7168, 1e-6, FAKE, FAKE + 2, None) == INVALID
    assert L.moe_combine_rms_bf16(FAKE, FAKE, FAKE, 1, 16, 7168, -1.0, FAKE, FAKE, None) == INVALID
    assert L.moe_combine_rms_bf16(FAKE, None, FAKE, 1, 16, 7168, 1e-6, FAKE, FAKE, None) == INVALID
    assert L.moe_combine_rms_bf16(FAKE + 4, FAKE, FAKE, 1, 16, 7168, 1e-6, FAKE, FAKE, None) == INVALID



def test_ffn_combine_rejects_bad_arguments(L):
    big = 1 << 30
    w = _weights()
    f = L.moe_expert_ffn_combine_mxfp4
    ok = (FAKE, 1, 16, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None)
    for i in (0, 7, 8, 10, 11):  # x, topk_weights, row_pos, out, workspace null
        args = list(ok)
        args[i] = None
        assert f(*args) == INVALID, i
    args = list(ok)
    args[10] = FAKE + 4  # out misaligned
    assert f(*args) == INVALID
    args = list(ok)
    args[2] = 33  # k above the maximum
    assert f(*args) == INVALID
    bad = _weights(H=250)
    args = list(ok)
    args[3] = ctypes.byref(bad)
    assert f(*args) == INVALID
    args = list(ok)
    args[12] = 16
    assert f(*args) == WS_SMALL


def test_decode_layer_rejects_bad_arguments(L):
    big = 1 << 30
    w = _weights()
    f = L.moe_decode_layer_mxfp4
    ok = [FAKE, FAKE, 2, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None]
    for i in (0, 1, 4, 5, 6, 7, 8, 9, 10, 11, 12):  # every pointer
        args = list(ok)
        args[i] = None
        assert f(*args) == INVALID, i
    for i, v in ((1, FAKE + 2), (10, FAKE + 4), (11, FAKE + 8), (2, 0), (2, 9), (2, 33)):  # k > E = 8
        args = list(ok)
        args[i] = v
        assert f(*args) == INVALID, (i, v)
    args = list(ok)
    args[13] = 16
    assert f(*args) == WS_SMALL


def test_decode_layer_rms_rejects_bad_arguments(L):
    big = 1 << 30
    w = _weights()
    f = L.moe_decode_layer_rms_mxfp4
    ok = [FAKE, FAKE, ctypes.c_float(1e-6), FAKE, 2, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
          FAKE, big, None]
    for i in (0, 1, 3, 6, 7, 8, 9, 10, 11, 12, 13, 14):  # every pointer
        args = list(ok)
        args[i] = None
        assert f(*args) == INVALID, i
    for i, v in ((1, FAKE + 4), (3, FAKE + 8), (2, ctypes.c_float(-1.0)), (4, 0), (4, 9)):
        args = list(ok)
        args[i] = v
        assert f(*args) == INVALID, (i, v)
    args = list(ok)
    args[15] = 16
    assert f(*args) == WS_SMALL


def test_bench_refuses_more_than_one_gpu():
    """bench.py times one GPU; asked for more it exits with status 2 and a
    message, before touching a device."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("k", [0, -1, 33, 897])
def test_decode_shape_rejects_bad_k(L, k):
    """At the decode shape (H 7168, I 1536, E 896) the fused one-token calls
    take their own launch path; a k outside 1..min(E, 32) must still be
    rejected before anything is enqueued (here: INVALID, not the HIP error
    a valid call gets on a host without a GPU)."""
    big = 1 << 34
    w = _weights(H=7168, I=1536, E=896)
    dl = L.moe_decode_layer_mxfp4
    args = [FAKE, FAKE, k, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None]
    assert dl(*args) == INVALID
    args[2] = 16
    assert dl(*args) == HIPERR  # the same call with a valid k passes validation
    rms = L.moe_decode_layer_rms_mxfp4
    args = [FAKE, FAKE, ctypes.c_float(1e-6), FAKE, k, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, big, None]
    assert rms(*args) == INVALID
    args[4] = 16
    assert rms(*args) == HIPERR
    fc = L.moe_expert_ffn_combine_mxfp4
    args = [FAKE, 1, k, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None]
    assert fc(*args) == INVALID
    args[2] = 16
    assert fc(*args) == HIPERR
    assert L.moe_route_group_one(FAKE, 896, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID


def test_decode_layer_noalloc_validation(L):
    """The allocation-free decode call: the same argument checks as
    moe_decode_layer_mxfp4, and shapes whose scratch (k * I fp32) exceeds the
    library's static buffer are refused with their own status, before any
    device call."""
    f = L.moe_decode_layer_mxfp4_noalloc
    w = _weights(H=7168, I=1536, E=896)
    ok = [FAKE, FAKE, 16, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    assert f(*ok) == HIPERR  # valid: only the missing device stops it
    for i in (0, 1, 4, 5, 6, 7, 8, 9, 10, 11):  # every pointer
        args = list(ok)
        args[i] = None
        assert f(*args) == INVALID, i
    for k in (0, -1, 33, 897):
        args = list(ok)
        args[2] = k
        assert f(*args) == INVALID, k
    args = list(ok)
    args[10] = FAKE + 4  # y_rows misaligned
    assert f(*args) == INVALID
    big = _weights(H=7168, I=16384, E=896)  # 32 * 16384 * 4 bytes = 2 MiB of scratch
    args = list(ok)
    args[2], args[3] = 32, ctypes.byref(big)
    assert f(*args) == SCRATCH_SMALL
    args[2] = 16  # 1 MiB: fits exactly
    assert f(*args) == HIPERR
    assert L.moe_status_string(SCRATCH_SMALL).startswith(b"MOE_ERR_SCRATCH_TOO_SMALL")
