"""GPU edge cases of the boundary: inputs whose storage is not 16-byte aligned (the chunked
path needs 16-byte rows, so these take the token-sequential path and must give the same
results), and NaN inputs, which must reach every output that depends on them."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, cpu64, dev

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _offset_copy(t, elems=1):
    """The same values in a buffer that starts `elems` elements past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 16, dtype=t.dtype, device="cuda")
    v = buf[elems:elems + t.numel()].view(t.shape)
    v.copy_(t.to("cuda"))
    assert v.data_ptr() % 16 != 0
    return v


@pytest.mark.parametrize("which", ["B", "C", "x", "all"])
def test_scan_fwd_misaligned_inputs_match_oracle(which):
    import ssm_sequence_models_amd as ssm
    Bsz, L, H, P, N, G = 2, 150, 2, 64, 128, 1
    g = torch.Generator().manual_seed(90)
    x = torch.randn(Bsz, L, H, P, generator=g).to(BF16)
    dt = torch.nn.functional.softplus(torch.randn(Bsz, L, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * float(np.log(16.0)))
    Bm = torch.randn(Bsz, L, G, N, generator=g).to(BF16)
    Cm = torch.randn(Bsz, L, G, N, generator=g).to(BF16)
    h0 = torch.randn(Bsz, H, P, N, generator=g)
    xd = _offset_copy(x) if which in ("x", "all") else dev(x)
    Bd = _offset_copy(Bm) if which in ("B", "all") else dev(Bm)
    Cd = _offset_copy(Cm) if which in ("C", "all") else dev(Cm)
    ws = torch.empty(ssm.workspace_size(Bsz, L, H, P, G, N), dtype=torch.uint8, device="cuda")
    y, fin = ssm.scan_fwd(xd, dev(dt), dev(A), Bd, Cd, initial_state=dev(h0), workspace=ws)
    torch.cuda.synchronize()
    ry, rf = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, None, out_dtype="bf16", state_dtype="f32")
    assert_close(y, ry, f"y (misaligned {which})")
    assert_close(fin, rf, f"final state (misaligned {which})")


def _fused_case(Bsz, L, H, seed):
    P, N, G, K = 64, 128, 1, 4
    C = H * P + 2 * G * N
    g = torch.Generator().manual_seed(seed)
    xBC = torch.randn(Bsz, L, C, generator=g).to(BF16)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    dt = torch.nn.functional.softplus(torch.randn(Bsz, L, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * float(np.log(16.0)))
    cinit = torch.randn(Bsz, C, K - 1, generator=g).to(BF16)
    sinit = torch.randn(Bsz, H, P, N, generator=g)
    return xBC, w, b, dt, A, cinit, sinit, (P, N, G, K)


def test_conv_scan_fwd_nan_input_reaches_its_outputs():
    """A NaN in one x channel of one token and a NaN in one B channel of a later token: every
    y element and final-state element the oracle computes as NaN is NaN on the GPU, and the
    rows and heads the NaNs cannot reach match the oracle.  (Within the chunk of a NaN x, the
    GPU may also make earlier tokens of that channel NaN: the intra-chunk product multiplies
    the masked, zero entries of M by it.)"""
    import ssm_sequence_models_amd as ssm
    Bsz, L, H = 2, 200, 3
    xBC, w, b, dt, A, cinit, sinit, (P, N, G, K) = _fused_case(Bsz, L, H, 91)
    hx, px, tx = 1, 5, 70          # x channel of head 1, channel 5, token 70 (row 0)
    tb = 150                       # B channel 3 at token 150 (row 1): reaches all heads of row 1
    xBC[0, tx, hx * P + px] = float("nan")
    xBC[1, tb, H * P + 3] = float("nan")
    y, cf, sf = ssm.conv_scan_fwd(dev(xBC), dev(w), dev(b), dev(dt), dev(A), H, P, G, N,
                                  conv_initial_state=dev(cinit), initial_state=dev(sinit))
    torch.cuda.synchronize()
    ry, rc, rs = oracle.conv_scan_fwd(xBC, w, b, cinit, dt, A, sinit, None, H, P, G, N)
    gy, gs = cpu64(y), cpu64(sf)
    ry, rs = np.asarray(ry, dtype=np.float64), np.asarray(rs, dtype=np.float64)
    assert np.isnan(ry).any() and np.isnan(rs).any()
    assert np.isnan(gy[np.isnan(ry)]).all(), "a NaN the oracle propagates to y is missing"
    assert np.isnan(gs[np.isnan(rs)]).all(), "a NaN the oracle propagates to the state is missing"
    # untouched: row 0 heads 0 and 2; row 0 head 1 other channels; row 1 before the B NaN's chunk
    for sel, what in (((0, slice(None), 0), "row 0 head 0"), ((0, slice(None), 2), "row 0 head 2"),
                      ((1, slice(0, 128), slice(None)), "row 1 before token 128")):
        assert_close(y.cpu()[sel], ry[sel], f"y {what}")
    other = [p for p in range(P) if p != px]
    assert_close(y.cpu()[0, :, hx][:, other], ry[0, :, hx][:, other], "y row 0 head 1 other channels")
    assert_close(sf.cpu()[0, 0], rs[0, 0], "state row 0 head 0")
    # the conv state is a raw copy of the last inputs: bit-exact, NaN included
    assert torch.equal(torch.isnan(cf.cpu().float()), torch.from_numpy(np.isnan(np.asarray(rc, dtype=np.float64))))


def test_decode_step_nan_input_matches_oracle_positions():
    """Decode (token by token): a NaN in one request's new x channel makes exactly the outputs
    and state entries the oracle makes NaN, and every other request matches the oracle."""
    import ssm_sequence_models_amd as ssm
    R, S, H, P, N, G, K, sl = 8, 16, 2, 64, 128, 1, 4, 4
    C = H * P + 2 * G * N
    g = torch.Generator().manual_seed(92)
    x = torch.randn(R, C, 2, generator=g).to(BF16)
    x[3, 7, 0] = float("nan")
    pool = torch.randn(S, C, sl, generator=g).to(BF16)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    dt = torch.nn.functional.softplus(torch.randn(R, 2, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * float(np.log(16.0)))
    spool = torch.randn(S, H, P, N, generator=g)
    idx = torch.randperm(S, generator=g)[:R].to(torch.int32)
    seqlens = torch.randint(0, 1000, (R,), generator=g).to(torch.int32)
    cp, sp = dev(pool).clone(), dev(spool).clone()
    y = ssm.decode_step(dev(x), cp, dev(w), dev(b), dev(dt), dev(A), sp, H, P, G, N,
                        conv_state_indices=dev(idx), cache_seqlens=dev(seqlens))
    torch.cuda.synchronize()
    co, rpool = oracle.conv1d_update(x, pool, w, b, idx, seqlens, act="silu", out_dtype="bf16")
    co = torch.from_numpy(np.asarray(co)).to(BF16)
    xs = co[:, :H * P, :].transpose(1, 2).reshape(R, 2, H, P)
    Bs = co[:, H * P:H * P + N, :].transpose(1, 2).reshape(R, 2, 1, N)
    Cs = co[:, H * P + N:, :].transpose(1, 2).reshape(R, 2, 1, N)
    ry, rpool_s = oracle.step(xs, dt, A, Bs, Cs, spool, idx, out_dtype="bf16", state_dtype="f32")
    gy, ry = cpu64(y), np.asarray(ry, dtype=np.float64)
    assert np.isnan(ry).any()
    assert np.array_equal(np.isnan(gy), np.isnan(ry)), "NaN positions of y differ"
    fin = np.isfinite(ry)
    assert_close(gy[fin], ry[fin], "finite y")
    gps, rps = cpu64(sp), np.asarray(rpool_s, dtype=np.float64)
    assert np.array_equal(np.isnan(gps), np.isnan(rps)), "NaN positions of the state pool differ"
    fin = np.isfinite(rps)
    assert_close(gps[fin], rps[fin], "finite state pool entries")


def test_debug_checks_reject_shared_slots(monkeypatch):
    """With the optional host check on, two active rows naming one pool slot raise ValueError
    before anything is launched, and the pools are left as they were; rows outside the pool
    (padding) may repeat."""
    import ssm_sequence_models_amd as ssm
    monkeypatch.setattr(ssm, "DEBUG_CHECKS", True)
    R, S, H, P, N, G, K, sl = 4, 8, 2, 64, 128, 1, 4, 4
    C = H * P + 2 * G * N
    g = torch.Generator().manual_seed(93)
    x = dev(torch.randn(R, C, 1, generator=g).to(BF16))
    pool = dev(torch.randn(S, C, sl, generator=g).to(BF16))
    w, b = dev(torch.rand(C, K, generator=g) - 0.5), dev(torch.rand(C, generator=g) - 0.5)
    dt = dev(torch.rand(R, 1, H, generator=g))
    A = dev(-torch.rand(H, generator=g))
    spool = dev(torch.randn(S, H, P, N, generator=g))
    before_c, before_s = pool.clone(), spool.clone()
    bad = dev(torch.tensor([5, 1, 5, 2], dtype=torch.int32))
    with pytest.raises(ValueError, match="used by more than one"):
        ssm.conv1d_update(x, pool, w, b, conv_state_indices=bad, activation="silu")
    with pytest.raises(ValueError, match="used by more than one"):
        ssm.decode_step(x, pool, w, b, dt, A, spool, H, P, G, N, conv_state_indices=bad)
    torch.cuda.synchronize()
    assert torch.equal(pool, before_c) and torch.equal(spool, before_s)
    padded = dev(torch.tensor([-1, 1, -1, 2], dtype=torch.int32))
    ssm.decode_step(x, pool, w, b, dt, A, spool, H, P, G, N, conv_state_indices=padded)
    torch.cuda.synchronize()


@pytest.mark.parametrize("nbytes,src_off,dst_off", [
    (1 << 20, 0, 0), ((1 << 20) + 7, 0, 0), (4096 * 1024 + 48, 16, 32),   # 16-byte path + tail
    (1000, 1, 0), (33, 0, 3), (1, 5, 9),                                  # byte path
])
def test_stream_copy_copies_every_byte(nbytes, src_off, dst_off):
    """The benchmark's streaming copy reference: dst equals src byte for byte, and the bytes
    around dst are untouched."""
    import ssm_sequence_models_amd as ssm
    g = torch.Generator().manual_seed(nbytes)
    src_buf = torch.randint(0, 256, (nbytes + 64,), generator=g, dtype=torch.uint8).to("cuda")
    dst_buf = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    src = src_buf[src_off:src_off + nbytes]
    dst = dst_buf[dst_off:dst_off + nbytes]
    ssm.stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), src.cpu())
    assert (dst_buf[:dst_off].cpu() == 0xA5).all() and (dst_buf[dst_off + nbytes:].cpu() == 0xA5).all()

