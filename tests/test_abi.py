"""The C-ABI library loads and exports every entry point its header declares; argument
checks that fail before any HIP call return the documented status codes (CPU only: none of
these calls reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_mi355x.h")


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import ssm_sequence_models_amd as s
    return s._lib


def test_header_declares_the_boundary():
    names = _declared_functions()
    for f in ("ssm_conv1d_fwd", "ssm_conv1d_update", "ssm_scan_fwd", "ssm_conv_scan_fwd",
              "ssm_step", "ssm_scan_workspace_size", "ssm_abi_version", "ssm_status_string",
              "ssm_last_error", "ssm_conv1d_bwd", "ssm_conv1d_bwd_workspace_size",
              "ssm_scan_bwd_initial_state", "ssm_conv_scan_fwd_pooled",
              "ssm_conv_scan_fwd_pooled_workspace_size", "ssm_state_stats_update",
              "ssm_initial_state_noise", "ssm_state_reset", "ssm_scan_fwd_vector_decay"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert lib.ssm_abi_version() == 4
    texts = [lib.ssm_status_string(code) for code in range(6)]
    assert all(texts) and len(set(texts)) == 6 and b"unknown status" not in texts
    for code in (-1, 6, 1 << 30):
        assert lib.ssm_status_string(code) == b"unknown status"


def test_workspace_query():
    import ssm_sequence_models_amd as s
    # chunked path: per (row, chunk of 64, group): C 16 KiB + B^T 16 KiB + G 16 KiB
    assert s.workspace_size(4, 8192, 64, 64, 1, 128) == 4 * 128 * 48 * 1024
    assert s.workspace_size(2, 65, 4, 64, 2, 128) == 2 * 2 * 2 * 48 * 1024
    # few heads on a long row: 5 segments of 410 chunks (256 CUs / 48 heads, at least 16
    # chunks each), plus each segment's entry state [P, N] fp32 and decay product
    assert s.workspace_size(1, 131072, 48, 64, 1, 128) == 2048 * 48 * 1024 + 48 * 5 * (64 * 128 + 1) * 4
    # general shapes: room for the conv output of the fused call
    import torch
    assert s.workspace_size(1, 64, 1, 4, 1, 4, torch.float32) == 64 * 12 * 4
    assert s.workspace_size(0, 64, 1, 4, 1, 4) == 0
    # conv backward: one fp32 partial (dw_0 .. dw_{K-1}, dbias) per (row, 64-token run, channel)
    assert s.conv1d_bwd_workspace_size(4, 8192, 4352, 4) == 4 * 128 * 4352 * 5 * 4
    assert s.conv1d_bwd_workspace_size(2, 65, 3, 2) == 2 * 2 * 3 * 3 * 4
    assert s.conv1d_bwd_workspace_size(2, 0, 3, 4) == 0
    # prefill on the pools: the scan's workspace, then the dense conv history [B, C, K-1] and
    # the dense SSM state [B, H, P, N] fp32, each rounded up to 256 bytes
    C = 64 * 64 + 2 * 128
    assert s.conv_scan_fwd_pooled_workspace_size(4, 8192, 64, 64, 1, 128, 4) == (
        s.workspace_size(4, 8192, 64, 64, 1, 128) + (4 * C * 3 * 2 + 255) // 256 * 256
        + 4 * 64 * 64 * 128 * 4)


def _c(v):
    return ctypes.c_void_p(v)


def test_argument_errors_return_status(lib):
    dummy = _c(256)  # never dereferenced: every call below fails its host-side checks
    # width outside [2, 8]
    assert lib.ssm_conv1d_fwd(dummy, dummy, None, None, None, None, dummy, 1, 4, 8, 9, 1, 0,
                              None) == 2
    # bad dtype / activation
    assert lib.ssm_conv1d_fwd(dummy, dummy, None, None, None, None, dummy, 1, 4, 8, 4, 7, 0,
                              None) == 1
    assert lib.ssm_conv1d_fwd(dummy, dummy, None, None, None, None, dummy, 1, 4, 8, 4, 1, 5,
                              None) == 1
    # NULL required pointer
    assert lib.ssm_conv1d_fwd(None, dummy, None, None, None, None, dummy, 1, 4, 8, 4, 1, 0,
                              None) == 1
    assert b"x is NULL" in lib.ssm_last_error()
    # misaligned bf16 pointer
    assert lib.ssm_conv1d_fwd(_c(257), dummy, None, None, None, None, dummy, 1, 4, 8, 4, 1, 0,
                              None) == 3
    # state_len < width - 1
    assert lib.ssm_conv1d_update(dummy, dummy, dummy, None, None, None, dummy, 2, 8, 1, 4, 2,
                                 4, 1, 0, None) == 1
    # nheads not a multiple of ngroups
    assert lib.ssm_scan_fwd(dummy, dummy, dummy, dummy, dummy, None, None, None, dummy, 1, 64,
                            3, 64, 2, 128, 1, None, 0, None) == 1
    # chunked path without workspace
    assert lib.ssm_scan_fwd(dummy, dummy, dummy, dummy, dummy, None, None, None, dummy, 1, 64,
                            4, 64, 1, 128, 1, None, 0, None) == 4
    # unsupported state size for the general path
    assert lib.ssm_step(dummy, 0, 0, 1, dummy, dummy, dummy, 0, 0, 1, dummy, 0, 0, 1, dummy,
                        None, dummy, 1, 1, 1, 4, 1, 6, 4, 0, None) == 2
    # conv backward: width outside [2, 8]; NULL dw; workspace too small
    assert lib.ssm_conv1d_bwd(dummy, dummy, None, None, None, dummy, None, dummy, None, dummy,
                              None, dummy, 1 << 20, 1, 4, 8, 1, 1, 0, None) == 2
    assert lib.ssm_conv1d_bwd(dummy, dummy, None, None, None, dummy, None, dummy, None, None,
                              None, dummy, 1 << 20, 1, 4, 8, 4, 1, 0, None) == 1
    assert lib.ssm_conv1d_bwd(dummy, dummy, None, None, None, dummy, None, dummy, None, dummy,
                              None, dummy, 16, 1, 4, 8, 4, 1, 0, None) == 4
    # initial-state gradient: nheads not a multiple of ngroups; NULL output
    assert lib.ssm_scan_bwd_initial_state(dummy, dummy, dummy, dummy, None, None, dummy, 1, 64,
                                          3, 64, 2, 128, 1, None) == 1
    assert lib.ssm_scan_bwd_initial_state(dummy, dummy, dummy, dummy, None, None, None, 1, 64,
                                          4, 64, 1, 128, 1, None) == 1
    # prefill on the pools: state_len < width - 1; NULL ssm pool; NULL y; workspace too small
    pooled = lambda y, pool, state_len, ws_bytes: lib.ssm_conv_scan_fwd_pooled(
        dummy, dummy, None, dummy, dummy, dummy, pool, None, None, None, y, 1, 64, 4, 64, 1, 128,
        4, state_len, 2, 1, 1, dummy, ws_bytes, None)
    assert pooled(dummy, dummy, 2, 1 << 30) == 1
    assert pooled(dummy, None, 4, 1 << 30) == 1 and b"ssm_state is NULL" in lib.ssm_last_error()
    assert pooled(None, dummy, 4, 1 << 30) == 1 and b"y is NULL" in lib.ssm_last_error()
    assert pooled(dummy, dummy, 4, 16) == 4
    # initial-state distributions: NULL mean; mean without var; odd row size; NaN p; NaN beta
    assert lib.ssm_state_stats_update(dummy, 2, 4, 8, 16, 0.1, None, dummy, None) == 1
    assert lib.ssm_state_stats_update(dummy, 2, 4, 8, 16, float("nan"), dummy, dummy, None) == 1
    assert lib.ssm_initial_state_noise(dummy, 2, 4, 8, 16, dummy, None, 1.0, 0, 0, None) == 1
    assert lib.ssm_initial_state_noise(_c(258), 2, 4, 8, 16, None, None, 1.0, 0, 0, None) == 3
    assert lib.ssm_state_reset(dummy, dummy, None, 4, 7, 0.1, 0, 0, None) == 1
    assert lib.ssm_state_reset(dummy, dummy, None, 4, 8, float("nan"), 0, 0, None) == 1
    assert lib.ssm_state_reset(_c(257), dummy, None, 4, 8, 0.1, 0, 0, None) == 3
    assert lib.ssm_state_stats_update(None, 0, 4, 8, 16, 0.1, None, None, None) == 0
    assert lib.ssm_initial_state_noise(None, 0, 4, 8, 16, None, None, 1.0, 0, 0, None) == 0
    assert lib.ssm_state_reset(None, None, None, 0, 8, 0.1, 0, 0, None) == 0
    # vector decay: both decay forms / neither; A_vec without dt; state not 16-byte aligned
    vd = lambda dt, ld, av, init: lib.ssm_scan_fwd_vector_decay(
        dummy, dt, ld, av, dummy, dummy, init, None, None, dummy, 1, 8, 4, 16, 1, 32, 1, None)
    assert vd(dummy, dummy, dummy, None) == 1
    assert vd(dummy, None, None, None) == 1
    assert vd(None, None, dummy, None) == 1
    assert vd(dummy, dummy, None, _c(260)) == 3
    # allocation-free prefill: sizes beyond its static scratch; argument errors come first
    assert lib.ssm_conv_scan_fwd_noalloc(dummy, dummy, None, None, None, dummy, dummy, None,
                                         None, None, dummy, 1, 131072, 48, 64, 1, 128, 4, 1, 1,
                                         None) == 4
    assert b"bytes of scratch" in lib.ssm_last_error()
    assert lib.ssm_conv_scan_fwd_noalloc(dummy, dummy, None, None, None, dummy, dummy, None,
                                         None, None, dummy, 1, 64, 3, 64, 2, 128, 4, 1, 1,
                                         None) == 1
    assert lib.ssm_noalloc_scratch_bytes() == 32 << 20
    # streaming copy: negative size, overlapping ranges (rejected before any launch)
    assert lib.ssm_stream_copy(dummy, dummy, -1, None) == 1
    assert lib.ssm_stream_copy(_c(256), _c(300), 100, None) == 1
    assert b"overlap" in lib.ssm_last_error()
    assert lib.ssm_stream_copy(None, dummy, 16, None) == 1
    # zero-sized work is a no-op that succeeds without touching the device
    assert lib.ssm_stream_copy(None, None, 0, None) == 0
    assert lib.ssm_conv1d_update(None, None, None, None, None, None, None, 0, 8, 1, 4, 3, 4, 1,
                                 0, None) == 0
    assert lib.ssm_step(None, 0, 0, 1, None, None, None, 0, 0, 1, None, 0, 0, 1, None, None,
                        None, 3, 0, 2, 4, 1, 8, 4, 0, None) == 0


def test_check_distinct_slots():
    """The optional host check for pooled calls: two active rows naming one slot is an error;
    rows outside [0, n_slots) are padding and may repeat."""
    import torch
    import ssm_sequence_models_amd as s
    s.check_distinct_slots(None, 4)
    s.check_distinct_slots(torch.tensor([3, 0, 2, 1], dtype=torch.int32), 4)
    s.check_distinct_slots(torch.tensor([-1, 2, -1, 4, 4, 0], dtype=torch.int32), 4)
    with pytest.raises(ValueError, match=r"slot\(s\) \[2\]"):
        s.check_distinct_slots(torch.tensor([2, 0, 2, -1], dtype=torch.int32), 4, "idx")
    with pytest.raises(ValueError, match=r"\[0, 3\]"):
        s.check_distinct_slots(torch.tensor([3, 0, 3, 0, 1], dtype=torch.int32), 4)
