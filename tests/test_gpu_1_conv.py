"""GPU parity of ssm_conv1d_fwd and ssm_conv1d_update against the fp64 oracle.

Outputs within |g - o| <= 1e-3 + 2e-2 |o|; bf16 prefill outputs also bit-exact (the kernel
rounds as the exact conv value rounds); conv states (raw input copies) and pool contents
bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bitexact, assert_close, dev

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
ODT = {BF16: "bf16", F32: "f32"}


def _conv_inputs(B, L, C, K, dtype, seed, with_init=True, seq_segments=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, L, C, generator=g).to(dtype)
    w = (torch.rand(C, K, generator=g) - 0.5)
    b = (torch.rand(C, generator=g) - 0.5)
    init = torch.randn(B, C, K - 1, generator=g).to(dtype) if with_init else None
    seq = workloads.packed_seq_idx(B, L, seed + 1, seq_segments) if seq_segments and L > seq_segments else None
    return x, w, b, init, seq


CASES = [
    # B, L, C, K, dtype, init, segments, act
    (1, 64, 12, 4, F32, True, 0, "silu"),     # the tiny layer's 4 + 2*4 channels
    (1, 64, 12, 4, F32, True, 0, None),
    (2, 200, 264, 4, BF16, True, 0, "silu"),  # 2-channel vector path, ragged token runs
    (2, 130, 36, 4, BF16, True, 0, "silu"),   # 9 threads per row: a partial wavefront
    (1, 96, 24, 4, BF16, False, 0, None),     # vector path, identity, no initial state
    (2, 200, 264, 4, BF16, True, 4, "silu"),  # packed sequences
    (1, 77, 13, 3, BF16, True, 3, None),      # odd channel count: scalar path
    (2, 70, 18, 4, BF16, True, 2, "silu"),    # C % 4 = 2: vector path, one partial wavefront
    (1, 100, 24, 8, BF16, True, 0, "silu"),   # widest conv over whole runs after the first
    (1, 70, 20, 2, BF16, True, 2, None),      # narrowest conv, vector path, packed sequences
    (3, 2, 16, 4, BF16, True, 0, "silu"),     # L < K-1: F keeps state entries
    (2, 1, 8, 2, F32, False, 0, None),
    (2, 45, 40, 8, BF16, True, 2, "silu"),    # widest conv
    (1, 33, 20, 5, F32, True, 0, "silu"),
]


@pytest.mark.parametrize("B,L,C,K,dtype,with_init,segs,act", CASES)
def test_conv1d_fwd_matches_oracle(B, L, C, K, dtype, with_init, segs, act):
    import ssm_sequence_models_amd as ssm
    x, w, b, init, seq = _conv_inputs(B, L, C, K, dtype, seed=B * 1000 + L + C + K,
                                      with_init=with_init, seq_segments=segs)
    out, fin = ssm.conv1d_fwd(dev(x), dev(w), dev(b), dev(init), dev(seq), act)
    torch.cuda.synchronize()
    ref, rfin = oracle.conv1d_fwd(x, w, b, init, seq, act=act or "none", out_dtype=ODT[dtype])
    assert_close(out, ref, "conv out")
    if dtype == BF16:
        assert_bitexact(out, torch.from_numpy(np.ascontiguousarray(ref)).to(BF16), "conv out (bf16)")
    assert_bitexact(fin, torch.from_numpy(rfin).to(dtype), "conv final state")


def test_conv1d_fwd_layer1p3b_sampled_channels():
    """The 1.3B-like layer's conv at full size (B 4, L 8192, 4352 channels, K 4, SiLU, state
    in / out): bf16 outputs and final states bit-exact on a sample of channels spread over the
    row, including the last ones."""
    import ssm_sequence_models_amd as ssm
    cfg = workloads.CONFIGS["layer1p3b"]
    s = workloads.shape_of("layer1p3b")
    w, b, _ = workloads.layer_params(s, cfg["seed"])
    inp = workloads.prefill_inputs(s, cfg["seed"], with_random_init=True)
    x, init = inp["xBC"], inp["conv_init"]
    out, fin = ssm.conv1d_fwd(dev(x), dev(w), dev(b), dev(init), None, "silu")
    torch.cuda.synchronize()
    chans = torch.tensor(sorted(set(list(range(0, s.C, 97)) + [1, 2, 3, s.C - 4, s.C - 3,
                                                               s.C - 2, s.C - 1])))
    ref, rfin = oracle.conv1d_fwd(x[:, :, chans], w[chans], b[chans], init[:, chans], None,
                                  act="silu", out_dtype="bf16")
    assert_bitexact(out[:, :, dev(chans)], torch.from_numpy(np.ascontiguousarray(ref)).to(BF16),
                    "conv out (sampled channels)")
    assert_bitexact(fin[:, dev(chans)], torch.from_numpy(rfin).to(BF16), "conv final state")


def test_conv1d_fwd_len0_and_inplace_state():
    import ssm_sequence_models_amd as ssm
    x, w, b, init, _ = _conv_inputs(2, 0, 16, 4, BF16, seed=5)
    _, fin = ssm.conv1d_fwd(dev(x), dev(w), dev(b), dev(init))
    assert_bitexact(fin, init, "L = 0 passes the state through")
    _, fin0 = ssm.conv1d_fwd(dev(x), dev(w), dev(b), None)
    assert_bitexact(fin0, torch.zeros_like(init), "L = 0 without state gives zeros")
    # in place: final_state is the initial_state tensor, over several token tiles
    x, w, b, init, _ = _conv_inputs(2, 100, 24, 4, BF16, seed=6)
    st = dev(init).clone()
    out, _ = ssm.conv1d_fwd(dev(x), dev(w), dev(b), st, final_state=st, activation="silu")
    ref, rfin = oracle.conv1d_fwd(x, w, b, init, act="silu", out_dtype="bf16")
    assert_close(out, ref, "in-place conv out")
    assert_bitexact(st, torch.from_numpy(rfin).to(BF16), "in-place conv state")


def test_conv1d_fwd_chunk_continuation():
    """S_B = F_A: two calls equal one (causal-conv1d ch. 7, chunked training)."""
    import ssm_sequence_models_amd as ssm
    x, w, b, init, _ = _conv_inputs(2, 150, 64, 4, BF16, seed=7)
    X, W, Bb, S = dev(x), dev(w), dev(b), dev(init)
    full, ffin = ssm.conv1d_fwd(X, W, Bb, S, activation="silu")
    for cut in (0, 1, 2, 33, 149, 150):
        oa, fa = ssm.conv1d_fwd(X[:, :cut].contiguous(), W, Bb, S, activation="silu")
        ob, fb = ssm.conv1d_fwd(X[:, cut:].contiguous(), W, Bb, fa, activation="silu")
        assert_bitexact(torch.cat([oa, ob], 1), full, f"chunked conv, cut {cut}")
        assert_bitexact(fb, ffin, f"chunked conv state, cut {cut}")


def _decode_case(L_new, dtype=BF16, R=256, n_slots=512, C=4352, state_len=4, K=4, seed=6,
                 circular=True):
    if C == 4352 and state_len == 4:
        d = workloads.decode_inputs(L_new=L_new, seed=seed, R=R, n_slots=n_slots,
                                    with_ssm_pool=False)
        return (d["x_new"].to(dtype), d["conv_pool"].to(dtype), d["conv_w"][:, :K].contiguous(),
                d["conv_b"], d["indices"], d["cache_seqlens"] if circular else None)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(R, C, L_new, generator=g).to(dtype)
    pool = torch.randn(n_slots, C, state_len, generator=g).to(dtype)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    idx = torch.randperm(n_slots, generator=g)[:R].to(torch.int32)
    seqlens = torch.randint(0, 100001, (R,), generator=g).to(torch.int32) if circular else None
    return x, pool, w, b, idx, seqlens


@pytest.mark.parametrize("L_new", [1, 4])
def test_conv1d_update_decode_layer(L_new):
    """The 1.3B-like decode layer: 256 requests in a 512-slot pool, state_len 4, circular
    cache_seqlens up to 100000."""
    import ssm_sequence_models_amd as ssm
    x, pool, w, b, idx, seqlens = _decode_case(L_new)
    P = dev(pool)
    S = dev(seqlens)
    before = S.clone()
    out = ssm.conv1d_update(dev(x), P, dev(w), dev(b), dev(idx), S, "silu")
    torch.cuda.synchronize()
    ref, rpool = oracle.conv1d_update(x, pool, w, b, idx, seqlens, act="silu", out_dtype="bf16")
    assert_close(out, ref, "decode conv out")
    assert_bitexact(P, torch.from_numpy(rpool).to(BF16), "conv pool after update")
    assert_bitexact(S, before, "cache_seqlens is not advanced")


@pytest.mark.parametrize("state_len,circular,L_new,dtype", [
    (3, False, 1, BF16), (9, False, 2, BF16), (4, True, 6, BF16), (5, True, 3, F32),
    (3, True, 1, F32), (7, False, 9, F32)])
def test_conv1d_update_modes(state_len, circular, L_new, dtype):
    import ssm_sequence_models_amd as ssm
    x, pool, w, b, idx, seqlens = _decode_case(L_new, dtype, R=6, n_slots=9, C=264,
                                               state_len=state_len, seed=11, circular=circular)
    idx = torch.tensor([3, -1, 8, 9, 0, 5], dtype=torch.int32)  # two rows out of range
    if circular:
        seqlens = torch.tensor([0, 1, 2, 5, 100001, 7], dtype=torch.int32)  # incl. p < K-1
    P = dev(pool)
    out = ssm.conv1d_update(dev(x), P, dev(w), dev(b), dev(idx), dev(seqlens), "silu")
    torch.cuda.synchronize()
    ref, rpool = oracle.conv1d_update(x, pool, w, b, idx, seqlens, act="silu",
                                      out_dtype=ODT[dtype])
    assert_close(out, ref, "conv update out")
    assert np.all(ref[1] == 0) and np.all(ref[3] == 0)
    assert_bitexact(P, torch.from_numpy(rpool).to(dtype), "conv pool")
