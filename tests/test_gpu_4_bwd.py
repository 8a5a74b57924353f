"""GPU parity of the backward entry points with state gradients (through the C-ABI) against
the fp64 oracle: ssm_conv1d_bwd (dx, dS, dw, dbias) and ssm_scan_bwd_initial_state (dh_{-1}),
element by element within the floating-point tolerance, plus the chunked-training chains."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_close, dev

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
ODT = {BF16: "bf16", F32: "f32"}


def _conv_inputs(B, L, C, K, dtype, seed, with_init=True, with_dF=True, segs=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, L, C, generator=g).to(dtype)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    init = torch.randn(B, C, K - 1, generator=g).to(dtype) if with_init else None
    dy = torch.randn(B, L, C, generator=g).to(dtype)
    dF = torch.randn(B, C, K - 1, generator=g).to(dtype) if with_dF else None
    seq = workloads.packed_seq_idx(B, L, seed + 3, segs) if segs and L > segs else None
    return x, w, b, init, dy, dF, seq


CONV_CASES = [
    # B, L, C, K, dtype, act, init, dF, segments
    (2, 200, 96, 4, BF16, "silu", True, True, 3),    # ragged runs, packed sequences
    (1, 257, 40, 3, F32, "silu", False, True, 0),
    (2, 130, 64, 8, BF16, "silu", True, False, 2),
    (1, 65, 5, 2, F32, "none", True, True, 0),
    (2, 3, 8, 4, BF16, "silu", True, True, 0),        # L = K-1
    (2, 2, 8, 4, F32, "none", True, True, 0),         # L < K-1: dS takes part of dF
    (1, 1, 4, 5, F32, "silu", True, True, 0),
    (3, 64, 33, 4, BF16, "none", False, False, 0),    # exactly one run
    (2, 150, 18, 4, BF16, "silu", True, True, 2),     # C % 4 = 2: vector path, partial wavefront
    (1, 150, 10, 2, BF16, "silu", True, True, 0),     # narrowest conv on the vector path
    (1, 300, 12, 8, BF16, "none", True, True, 3),     # widest: head and tail steps of K-1 = 7
]


@pytest.mark.parametrize("B,L,C,K,dtype,act,with_init,with_dF,segs", CONV_CASES)
def test_conv1d_bwd_matches_oracle(B, L, C, K, dtype, act, with_init, with_dF, segs):
    import ssm_sequence_models_amd as ssm
    x, w, b, init, dy, dF, seq = _conv_inputs(B, L, C, K, dtype, seed=B + 3 * L + C + K,
                                              with_init=with_init, with_dF=with_dF, segs=segs)
    dx, dS, dw, db = ssm.conv1d_bwd(dev(x), dev(w), dev(b), dev(dy), initial_state=dev(init),
                                    dfinal_state=dev(dF), seq_idx=dev(seq), activation=act)
    torch.cuda.synchronize()
    rdx, rdS, rdw, rdb = oracle.conv1d_bwd(x, w, b, init, seq, dy, dF, act=act,
                                           dx_dtype=ODT[dtype], dstate_dtype=ODT[dtype])
    assert_close(dx, rdx, "dx")
    assert_close(dS, rdS, "dS")
    assert_close(dw, rdw, "dw")
    assert_close(db, rdb, "dbias")


def test_conv1d_bwd_len0():
    import ssm_sequence_models_amd as ssm
    x, w, b, init, dy, dF, _ = _conv_inputs(2, 0, 8, 4, BF16, seed=5)
    dx, dS, dw, db = ssm.conv1d_bwd(dev(x), dev(w), dev(b), dev(dy), initial_state=dev(init),
                                    dfinal_state=dev(dF), activation="silu")
    torch.cuda.synchronize()
    assert torch.equal(dS.cpu(), dF), "L = 0: F is S itself, so dS = dF"
    assert float(dw.abs().max()) == 0.0 and float(db.abs().max()) == 0.0


def test_conv1d_bwd_chunked_chain_equals_whole():
    """Chunked training: with S_B = F_A, chunk B's dS passed as chunk A's dF reproduces the
    whole row's gradients (dw, dbias add)."""
    import ssm_sequence_models_amd as ssm
    B, L, C, K, cut = 2, 300, 48, 4, 137
    x, w, b, init, dy, dF, _ = _conv_inputs(B, L, C, K, F32, seed=9)
    d = lambda t: dev(t)
    wx, wS, ww, wb = ssm.conv1d_bwd(d(x), d(w), d(b), d(dy), initial_state=d(init),
                                    dfinal_state=d(dF), activation="silu")
    _, FA = ssm.conv1d_fwd(d(x[:, :cut].contiguous()), d(w), d(b), initial_state=d(init),
                           activation="silu")
    bx, bS, bw, bb = ssm.conv1d_bwd(d(x[:, cut:].contiguous()), d(w), d(b),
                                    d(dy[:, cut:].contiguous()), initial_state=FA,
                                    dfinal_state=d(dF), activation="silu")
    ax, aS, aw, ab = ssm.conv1d_bwd(d(x[:, :cut].contiguous()), d(w), d(b),
                                    d(dy[:, :cut].contiguous()), initial_state=d(init),
                                    dfinal_state=bS, activation="silu")
    torch.cuda.synchronize()
    assert_close(torch.cat([ax, bx], dim=1), wx.cpu().double().numpy(), "dx (chunked)")
    assert_close(aS, wS.cpu().double().numpy(), "dS (chunked)")
    assert_close(aw + bw, ww.cpu().double().numpy(), "dw (chunked)")
    assert_close(ab + bb, wb.cpu().double().numpy(), "dbias (chunked)")


def _h0_inputs(b, L, H, P, N, G, dtype, seed, with_dF=True, segs=0, slow=False):
    g = torch.Generator().manual_seed(seed)
    if slow:  # decays that keep h_{-1} alive over the whole row
        dt = torch.rand(b, L, H, generator=g) * 0.02
        A = -torch.rand(H, generator=g) * 0.5
    else:
        dt = torch.nn.functional.softplus(torch.randn(b, L, H, generator=g) - 2.0)
        A = -torch.exp(torch.rand(H, generator=g) * float(np.log(16.0)))
    Cm = torch.randn(b, L, G, N, generator=g).to(dtype)
    dy = torch.randn(b, L, H, P, generator=g).to(dtype)
    dF = torch.randn(b, H, P, N, generator=g) if with_dF else None
    seq = workloads.packed_seq_idx(b, L, seed + 3, segs) if segs and L > segs else None
    return dt, A, Cm, dy, dF, seq


H0_CASES = [
    # b, L, H, P, N, G, dtype, dF, segments, slow decays
    (2, 300, 4, 64, 128, 1, BF16, True, 0, False),   # matrix-core path, ragged last chunk
    (1, 1000, 2, 64, 128, 1, BF16, True, 0, True),   # every chunk contributes
    (2, 200, 4, 64, 128, 2, BF16, False, 3, True),   # packed sequences: cut at the first change
    (1, 64, 2, 64, 128, 1, BF16, True, 0, True),     # exactly one chunk
    (2, 50, 3, 4, 8, 1, F32, True, 0, True),         # general shapes
    (1, 90, 2, 16, 32, 2, BF16, True, 2, True),
]


@pytest.mark.parametrize("b,L,H,P,N,G,dtype,with_dF,segs,slow", H0_CASES)
def test_scan_bwd_initial_state_matches_oracle(b, L, H, P, N, G, dtype, with_dF, segs, slow):
    import ssm_sequence_models_amd as ssm
    dt, A, Cm, dy, dF, seq = _h0_inputs(b, L, H, P, N, G, dtype, seed=b + L + H + P,
                                        with_dF=with_dF, segs=segs, slow=slow)
    dh0 = ssm.scan_bwd_initial_state(dev(dt), dev(A), dev(Cm), dev(dy), dfinal_state=dev(dF),
                                     seq_idx=dev(seq))
    torch.cuda.synchronize()
    ref = oracle.scan_bwd_h0(dt, A, Cm, seq, dy, dF, P, out_dtype="f32")
    assert_close(dh0, ref, "dh0")


def test_scan_bwd_initial_state_inplace_len0_and_chain():
    """L = 0 gives dF back; the output may be dF itself; chunk B's result passed as chunk A's
    dF equals the whole row's."""
    import ssm_sequence_models_amd as ssm
    b, L, H, P, N, G, cut = 2, 260, 2, 64, 128, 1, 100
    dt, A, Cm, dy, dF, _ = _h0_inputs(b, L, H, P, N, G, BF16, seed=77, slow=True)
    z = ssm.scan_bwd_initial_state(dev(dt[:, :0].contiguous()), dev(A), dev(Cm[:, :0].contiguous()),
                                   dev(dy[:, :0].contiguous()), dfinal_state=dev(dF))
    whole = ssm.scan_bwd_initial_state(dev(dt), dev(A), dev(Cm), dev(dy), dfinal_state=dev(dF))
    st = dev(dF).clone()
    ssm.scan_bwd_initial_state(dev(dt[:, cut:].contiguous()), dev(A), dev(Cm[:, cut:].contiguous()),
                               dev(dy[:, cut:].contiguous()), dfinal_state=st, out=st)
    ssm.scan_bwd_initial_state(dev(dt[:, :cut].contiguous()), dev(A), dev(Cm[:, :cut].contiguous()),
                               dev(dy[:, :cut].contiguous()), dfinal_state=st, out=st)
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), dF), "L = 0 returns dF"
    assert_close(st, whole.cpu().double().numpy(), "dh0 (chunked, in place)")
    ref = oracle.scan_bwd_h0(dt, A, Cm, None, dy, dF, P, out_dtype="f32")
    assert_close(whole, ref, "dh0")
