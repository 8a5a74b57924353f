"""GPU parity of ssm_conv_scan_fwd_pooled (the fused prefill on the decode pools) against the
fp64 oracle, and its continuity with the decode path: a prefill chain, and a prefill followed
by decode steps, equal one whole prefill."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bitexact, assert_close, dev

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
ODT = {BF16: "bf16", F32: "f32"}


def _layer(B, L, H, P, N, G, K, dtype, seed):
    C = H * P + 2 * G * N
    g = torch.Generator().manual_seed(seed)
    xBC = torch.randn(B, L, C, generator=g).to(dtype)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    dt = torch.nn.functional.softplus(torch.randn(B, L, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * float(np.log(16.0)))
    return xBC, w, b, dt, A, C, g


POOL_CASES = [
    # B, L, H, P, N, G, K, dtype, n_slots, state_len, circular, indices, segments
    (2, 200, 4, 64, 128, 1, 4, BF16, 4, 8, True, [3, 1], 0),
    (2, 150, 2, 64, 128, 1, 4, BF16, 3, 3, True, [0, 2], 2),
    (2, 130, 4, 64, 128, 2, 3, BF16, 2, 6, False, None, 0),
    (3, 70, 2, 64, 128, 1, 4, BF16, 3, 4, True, [2, 7, 0], 0),   # row 1: slot out of range
    (2, 40, 2, 16, 32, 1, 4, F32, 3, 5, True, [1, 2], 0),        # general shapes
    (2, 2, 2, 64, 128, 1, 4, BF16, 2, 4, True, [1, 0], 0),       # L < K-1
    (2, 2, 2, 64, 128, 1, 4, BF16, 3, 5, False, [2, 0], 0),      # linear, L < state_len
    (3, 90, 2, 64, 128, 1, 4, BF16, 4, 4, False, [3, 1, 0], 2),  # linear, packed rows
    # long rows over few heads run as segments (a state pass, then the output pass that
    # composes each segment's entry state), which read and write the pool rows in place
    (1, 4096, 2, 64, 128, 1, 4, BF16, 3, 4, True, [2], 0),
    (2, 2048, 1, 64, 128, 1, 4, BF16, 3, 4, True, [5, 1], 2),   # row 0: slot out of range
]


@pytest.mark.parametrize("B,L,H,P,N,G,K,dtype,n_slots,S_len,circular,indices,segs", POOL_CASES)
def test_conv_scan_fwd_pooled_matches_oracle(B, L, H, P, N, G, K, dtype, n_slots, S_len, circular,
                                             indices, segs):
    import ssm_sequence_models_amd as ssm
    xBC, w, b, dt, A, C, g = _layer(B, L, H, P, N, G, K, dtype, seed=B + L + H + K + S_len)
    conv_pool = torch.randn(n_slots, C, S_len, generator=g).to(dtype)
    ssm_pool = torch.randn(n_slots, H, P, N, generator=g)
    idx = None if indices is None else torch.tensor(indices, dtype=torch.int32)
    seqlens = torch.randint(0, 1000, (B,), generator=g).to(torch.int32) if circular else None
    seq = workloads.packed_seq_idx(B, L, 5, segs) if segs else None
    cp, sp = dev(conv_pool).clone(), dev(ssm_pool).clone()
    y = ssm.conv_scan_fwd_pooled(dev(xBC), dev(w), dev(b), dev(dt), dev(A), cp, sp, H, P, G, N,
                                 state_indices=dev(idx), cache_seqlens=dev(seqlens),
                                 seq_idx=dev(seq))
    torch.cuda.synchronize()
    ry, rcp, rsp = oracle.conv_scan_fwd_pooled(xBC, w, b, dt, A, conv_pool, ssm_pool, idx, seqlens,
                                               seq, H, P, G, N, act="silu", out_dtype=ODT[dtype],
                                               state_dtype="f32")
    assert_close(y, ry, "y")
    assert_bitexact(cp, torch.from_numpy(rcp).to(dtype), "conv pool")
    assert_close(sp, rsp, "ssm pool")


def test_pooled_prefill_chain_and_decode_continue_one_request():
    """Row 0 on slot 2, row 1 on slot 0: prefill L1 tokens into the pools, prefill the next L2,
    then decode the rest token by token with decode_step; every output equals one whole
    conv_scan_fwd from zero states."""
    import ssm_sequence_models_amd as ssm
    B, L, H, P, N, G, K = 2, 230, 2, 64, 128, 1, 4
    L1, L2, S_len = 100, 90, 6
    xBC, w, b, dt, A, C, _ = _layer(B, L, H, P, N, G, K, BF16, seed=23)
    d = dev
    y_whole, _, _ = ssm.conv_scan_fwd(d(xBC), d(w), d(b), d(dt), d(A), H, P, G, N)
    cp = torch.zeros(3, C, S_len, dtype=BF16, device="cuda")
    sp = torch.zeros(3, H, P, N, device="cuda")
    idx = torch.tensor([2, 0], dtype=torch.int32, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    ys = []
    for a, e in ((0, L1), (L1, L1 + L2)):
        ys.append(ssm.conv_scan_fwd_pooled(d(xBC[:, a:e].contiguous()), d(w), d(b),
                                           d(dt[:, a:e].contiguous()), d(A), cp, sp, H, P, G, N,
                                           state_indices=idx, cache_seqlens=pos))
        pos += e - a
    for t in range(L1 + L2, L):
        xn = d(xBC[:, t, :, None].contiguous())
        ys.append(ssm.decode_step(xn, cp, d(w), d(b), d(dt[:, t:t + 1].contiguous()), d(A), sp,
                                  H, P, G, N, conv_state_indices=idx, cache_seqlens=pos,
                                  state_indices=idx))
        pos += 1
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=1)
    assert_close(y, y_whole.cpu().double().numpy(), "y (pooled prefill chain + decode)")
