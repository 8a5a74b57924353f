"""GPU parity at the full layer sizes, in the launch configuration the benchmark times.

The GPU runs every head / request; the oracle recomputes a sample of them one by one (heads,
channels and requests are independent, so the sample's oracle outputs are exact for those
elements).  Chained calls are also checked against one call (state passing)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bitexact, assert_close, dev, oracle_conv_scan_heads

pytestmark = pytest.mark.gpu


def _full_states(s, heads, chans, conv_vals, ssm_vals):
    """Full-size state tensors holding the oracle's values on the sampled heads/channels."""
    conv = torch.zeros(s.B, s.C, s.K - 1, dtype=torch.float64)
    conv[:, torch.tensor(chans)] = torch.from_numpy(conv_vals)
    ssm = torch.zeros(s.B, s.H, s.P, s.N, dtype=torch.float64)
    ssm[:, torch.tensor(heads)] = torch.from_numpy(ssm_vals)
    return conv, ssm


def test_layer1p3b_state_passing_and_packed():
    """1.3B-like layer (B 4, L 8192, 64 heads x 64, N 128): initial conv / SSM states are the
    final states of a preceding seed-2 run; also the packed variant with 4 segments."""
    import ssm_sequence_models_amd as ssm
    cfg = workloads.CONFIGS["layer1p3b"]
    s = workloads.shape_of("layer1p3b")
    w, b, A = workloads.layer_params(s, cfg["seed"])
    pre = workloads.prefill_inputs(s, cfg["pre_seed"])
    main = workloads.prefill_inputs(s, cfg["seed"])
    heads = [0, 37, 63]
    W, Bb, AA = dev(w), dev(b), dev(A)
    # GPU: preceding run from zero state, then the measured run from its final states
    _, cf2, sf2 = ssm.conv_scan_fwd(dev(pre["xBC"]), W, Bb, dev(pre["dt"]), AA, s.H, s.P, s.G,
                                    s.N)
    xm, dm = dev(main["xBC"]), dev(main["dt"])
    y3, cf3, sf3 = ssm.conv_scan_fwd(xm, W, Bb, dm, AA, s.H, s.P, s.G, s.N,
                                     conv_initial_state=cf2, initial_state=sf2)
    torch.cuda.synchronize()
    # oracle on the sampled heads
    _, of2, oc2, chans = oracle_conv_scan_heads(pre["xBC"], w, b, None, pre["dt"], A, None, None,
                                                s.H, s.P, s.G, s.N, heads)
    cinit, sinit = _full_states(s, heads, chans, oc2, of2)
    oy3, of3, oc3, _ = oracle_conv_scan_heads(main["xBC"], w, b, cinit.to(torch.bfloat16),
                                              main["dt"], A, sinit, None, s.H, s.P, s.G, s.N,
                                              heads)
    hi = torch.tensor(heads)
    assert_close(sf2[:, hi], of2, "pre-run final state")
    assert_close(y3[:, :, hi], oy3, "y")
    assert_close(sf3[:, hi], of3, "final state")
    assert_bitexact(cf3[:, torch.tensor(chans)], torch.from_numpy(oc3).to(torch.bfloat16),
                    "conv final state (sampled channels)")
    # every channel's conv final state is the raw tail of xBC (L >= K-1)
    assert_bitexact(cf3, main["xBC"][:, -(s.K - 1):, :].transpose(1, 2), "conv final state")

    # packed variant: seq_idx with 4 segments per row, same initial states
    seq = workloads.packed_seq_idx(s.B, s.L, cfg["packed_seed"])
    yp, _, sfp = ssm.conv_scan_fwd(xm, W, Bb, dm, AA, s.H, s.P, s.G, s.N,
                                   conv_initial_state=cf2, initial_state=sf2, seq_idx=dev(seq))
    torch.cuda.synchronize()
    oyp, ofp, _, _ = oracle_conv_scan_heads(main["xBC"], w, b, cinit.to(torch.bfloat16),
                                            main["dt"], A, sinit, seq, s.H, s.P, s.G, s.N, heads)
    assert_close(yp[:, :, hi], oyp, "packed y")
    assert_close(sfp[:, hi], ofp, "packed final state")


def test_layer370m_zero_state():
    import ssm_sequence_models_amd as ssm
    cfg = workloads.CONFIGS["layer370m"]
    s = workloads.shape_of("layer370m")
    w, b, A = workloads.layer_params(s, cfg["seed"])
    inp = workloads.prefill_inputs(s, cfg["seed"])
    y, cf, sf = ssm.conv_scan_fwd(dev(inp["xBC"]), dev(w), dev(b), dev(inp["dt"]), dev(A), s.H,
                                  s.P, s.G, s.N)
    torch.cuda.synchronize()
    heads = [0, 19, 31]
    oy, of, oc, chans = oracle_conv_scan_heads(inp["xBC"], w, b, None, inp["dt"], A, None, None,
                                               s.H, s.P, s.G, s.N, heads)
    hi = torch.tensor(heads)
    assert_close(y[:, :, hi], oy, "y")
    assert_close(sf[:, hi], of, "final state")
    assert_bitexact(cf[:, torch.tensor(chans)], torch.from_numpy(oc).to(torch.bfloat16),
                    "conv final state")


def test_layer780m_chained_calls_equal_one_call():
    """131072 tokens as 64 chained 2048-token calls (S_{k+1} = F_k in place) against one
    full-length call, and one head against the oracle over the whole length."""
    import ssm_sequence_models_amd as ssm
    cfg = workloads.CONFIGS["layer780m"]
    s = workloads.shape_of("layer780m")
    w, b, A = workloads.layer_params(s, cfg["seed"])
    inp = workloads.prefill_inputs(s, cfg["seed"])
    X, D, W, Bb, AA = dev(inp["xBC"]), dev(inp["dt"]), dev(w), dev(b), dev(A)
    y, cf, sf = ssm.conv_scan_fwd(X, W, Bb, D, AA, s.H, s.P, s.G, s.N)
    cs = torch.zeros(s.B, s.C, s.K - 1, dtype=torch.bfloat16, device="cuda")
    ss = torch.zeros(s.B, s.H, s.P, s.N, dtype=torch.float32, device="cuda")
    yc = torch.empty_like(y)
    T = cfg["chunk_len"]
    ws = torch.empty(ssm.workspace_size(s.B, T, s.H, s.P, s.G, s.N), dtype=torch.uint8,
                     device="cuda")
    for k in range(s.L // T):
        sl = slice(k * T, (k + 1) * T)
        ssm.conv_scan_fwd(X[:, sl], W, Bb, D[:, sl], AA, s.H, s.P, s.G, s.N,
                          conv_initial_state=cs, initial_state=ss, conv_final_state=cs,
                          final_state=ss, y=yc[:, sl], workspace=ws)
    torch.cuda.synchronize()
    assert_close(yc, y.float(), "chained y vs one call")
    assert_close(ss, sf, "chained final state vs one call")
    assert_bitexact(cs, cf, "chained conv state vs one call")
    heads = [5]
    oy, of, _, _ = oracle_conv_scan_heads(inp["xBC"], w, b, None, inp["dt"], A, None, None,
                                          s.H, s.P, s.G, s.N, heads)
    assert_close(y[:, :, 5:6], oy, "y vs oracle (head 5)")
    assert_close(sf[:, 5:6], of, "final state vs oracle (head 5)")


@pytest.mark.parametrize("L_new", [1, 4])
def test_decode_layer(L_new):
    """256 requests, 512-slot conv and SSM pools (1.3B-like dims), state_len 4 circular."""
    import ssm_sequence_models_amd as ssm
    d = workloads.decode_inputs(L_new=L_new)
    c = d["cfg"]
    H, P, N, G = c["H"], c["P"], c["N"], c["G"]
    CP, SP = dev(d["conv_pool"]), dev(d["ssm_pool"])
    y = ssm.decode_step(dev(d["x_new"]), CP, dev(d["conv_w"]), dev(d["conv_b"]), dev(d["dt"]),
                        dev(d["A"]), SP, H, P, G, N, conv_state_indices=dev(d["indices"]),
                        cache_seqlens=dev(d["cache_seqlens"]))
    torch.cuda.synchronize()
    idx = d["indices"]
    # untouched slots of both pools are bit-identical
    used = torch.zeros(c["n_slots"], dtype=torch.bool)
    used[idx.long()] = True
    assert_bitexact(SP[~used.cuda()], d["ssm_pool"][~used], "untouched SSM slots")
    assert_bitexact(CP[~used.cuda()], d["conv_pool"][~used], "untouched conv slots")
    # oracle on 16 sampled requests
    rows = torch.tensor([0, 1, 2, 50, 77, 100, 128, 150, 199, 200, 210, 230, 240, 250, 254, 255])
    ridx = idx[rows]
    co, rcp = oracle.conv1d_update(d["x_new"][rows], d["conv_pool"], d["conv_w"], d["conv_b"],
                                   ridx, d["cache_seqlens"][rows], act="silu", out_dtype="bf16")
    R = len(rows)
    xs = co[:, :H * P].transpose(0, 2, 1).reshape(R, L_new, H, P)
    Bs = co[:, H * P:H * P + N].transpose(0, 2, 1).reshape(R, L_new, 1, N)
    Cs = co[:, H * P + N:].transpose(0, 2, 1).reshape(R, L_new, 1, N)
    sub_pool = d["ssm_pool"][ridx.long()]
    ry, rsp = oracle.step(xs, d["dt"][rows], d["A"], Bs, Cs, sub_pool,
                          torch.arange(R, dtype=torch.int32), out_dtype="bf16", state_dtype="f32")
    assert_close(y[rows.cuda()], ry, "decode y (sampled requests)")
    assert_close(SP[ridx.long().cuda()], rsp, "SSM slots (sampled requests)")
    assert_bitexact(CP[ridx.long().cuda()], torch.from_numpy(rcp[ridx.long()]).to(torch.bfloat16),
                    "conv slots (sampled requests)")
