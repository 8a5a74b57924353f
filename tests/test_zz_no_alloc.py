"""The allocation-free fused prefill (ssm_conv_scan_fwd_noalloc, working in the library's
static per-GPU scratch) against the workspace entry point ssm_conv_scan_fwd on the same
inputs: two calls in a row, the second smaller and on the segment path, so stale scratch from
the first call would show; the first also against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bitexact, assert_close, dev

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
P, N, G, K = 64, 128, 1, 4


def _case(Bsz, L, H, seed, packed):
    C = H * P + 2 * G * N
    g = torch.Generator().manual_seed(seed)
    xBC = torch.randn(Bsz, L, C, generator=g).to(BF16)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    dt = torch.nn.functional.softplus(torch.randn(Bsz, L, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * float(np.log(16.0)))
    cinit = torch.randn(Bsz, C, K - 1, generator=g).to(BF16)
    sinit = torch.randn(Bsz, H, P, N, generator=g)
    seq = None
    if packed:  # rows of three packed sequences with ragged boundaries
        cuts = sorted(torch.randint(1, L, (2,), generator=g).tolist())
        seq = torch.zeros(Bsz, L, dtype=torch.int32)
        seq[:, cuts[0]:] = 1
        seq[:, cuts[1]:] = 2
    return [xBC, w, b, dt, A, cinit, sinit, seq]


def _both(case, H):
    import ssm_sequence_models_amd as ssm
    xBC, w, b, dt, A, cinit, sinit, seq = [dev(t) for t in case]
    Bsz, L, C = xBC.shape
    ref = ssm.conv_scan_fwd(xBC, w, b, dt, A, H, P, G, N, conv_initial_state=cinit,
                            initial_state=sinit, seq_idx=seq)
    y = torch.full((Bsz, L, H, P), float("nan"), dtype=BF16, device="cuda")
    cf = torch.full((Bsz, C, K - 1), float("nan"), dtype=BF16, device="cuda")
    sf = torch.full((Bsz, H, P, N), float("nan"), dtype=torch.float32, device="cuda")
    out = ssm.conv_scan_fwd_noalloc(xBC, w, b, dt, A, H, P, G, N, y, conv_final_state=cf,
                                    final_state=sf, conv_initial_state=cinit,
                                    initial_state=sinit, seq_idx=seq)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_workspace_entry_point_two_calls():
    import ssm_sequence_models_amd as ssm
    assert ssm.noalloc_scratch_bytes() == 32 << 20
    # call 1: 3 rows x 1100 tokens (17 full chunks + a ragged tail), 6 heads, packed rows
    H1 = 6
    c1 = _case(3, 1100, H1, 95, packed=True)
    assert ssm.workspace_size(3, 1100, H1, P, G, N) <= ssm.noalloc_scratch_bytes()
    ref, out = _both(c1, H1)
    for r, o, what in zip(ref, out, ("y", "conv final state", "final state")):
        assert_bitexact(o, r, f"call 1 {what}")
    xBC, w, b, dt, A, cinit, sinit, seq = c1
    ry, rc, rs = oracle.conv_scan_fwd(xBC, w, b, cinit, dt, A, sinit, seq, H1, P, G, N)
    assert_close(out[0], ry, "call 1 y vs oracle")
    assert_close(out[2], rs, "call 1 final state vs oracle")
    assert_bitexact(out[1], torch.from_numpy(np.asarray(rc, dtype=np.float32)).to(BF16),
                    "call 1 conv final state vs oracle")
    # call 2: one row of 2100 tokens, 1 head -- smaller, and with so few blocks that the row
    # is split into two segments whose states also live in the scratch
    H2 = 1
    c2 = _case(1, 2100, H2, 96, packed=False)
    assert ssm.workspace_size(1, 2100, H2, P, G, N) < ssm.workspace_size(3, 1100, H1, P, G, N)
    assert c2[0].numel() < c1[0].numel()
    ref, out = _both(c2, H2)
    for r, o, what in zip(ref, out, ("y", "conv final state", "final state")):
        assert_bitexact(o, r, f"call 2 {what}")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """One 131072-token row of 48 heads needs 104 MiB of scratch: refused before any launch,
    and the outputs are left as they were."""
    import ssm_sequence_models_amd as ssm
    lib = ssm._lib
    Bsz, L, H = 1, 131072, 48
    need = ssm.workspace_size(Bsz, L, H, P, G, N)
    assert need > ssm.noalloc_scratch_bytes()
    y = torch.zeros(16, dtype=BF16, device="cuda")  # never written: the size check comes first
    p = torch.zeros(16, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.ssm_conv_scan_fwd_noalloc(y.data_ptr(), p.data_ptr(), None, None, None,
                                       p.data_ptr(), p.data_ptr(), None, None, None, y.data_ptr(),
                                       Bsz, L, H, P, G, N, K, ssm.SSM_BF16, 1, stream)
    assert st == 4
    assert b"bytes of scratch" in lib.ssm_last_error()
    torch.cuda.synchronize()
    assert not y.any() and not p.any()
