"""GPU parity of ssm_scan_fwd_vector_decay (the scan with a diagonal, per-state-dimension
transition) against the fp64 oracle through the C-ABI: gate and rate forms, with and without
dt, initial states, packed sequences, general shapes, and the 1.3B-like shape on sampled
heads."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_close, dev

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
ODT = {BF16: "bf16", F32: "f32"}


def _inputs(B, L, H, P, N, G, dtype, seed, form, with_dt, with_init, segs):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, L, H, P, generator=g).to(dtype)
    Bm = torch.randn(B, L, G, N, generator=g).to(dtype)
    Cm = torch.randn(B, L, G, N, generator=g).to(dtype)
    dt = torch.nn.functional.softplus(torch.randn(B, L, H, generator=g) - 2.0) if with_dt else None
    gate = workloads.vector_decay_gates(B, L, H, N, seed + 1) if form == "gate" else None
    Av = workloads.vector_decay_rates(H, N, seed + 2) if form == "rate" else None
    h0 = torch.randn(B, H, P, N, generator=g) if with_init else None
    seq = workloads.packed_seq_idx(B, L, seed + 3, segs) if segs else None
    return x, Bm, Cm, dt, gate, Av, h0, seq


CASES = [
    # B, L, H, P, N, G, dtype, form, dt, init, segments
    (2, 300, 4, 64, 128, 1, BF16, "gate", True, True, 0),
    (2, 300, 4, 64, 128, 1, BF16, "gate", False, True, 3),   # GLA-like: no dt, packed rows
    (1, 200, 4, 64, 64, 2, BF16, "rate", True, False, 0),    # per-dimension rates x dt
    (2, 100, 4, 16, 32, 2, F32, "gate", True, True, 2),
    (1, 77, 3, 4, 8, 1, F32, "rate", True, True, 0),
    (2, 1, 2, 64, 128, 1, BF16, "gate", True, True, 0),      # one token
    (2, 150, 4, 64, 128, 1, BF16, "rate", True, True, 3),    # rates, resets folded into a_t = 0
    (1, 70, 2, 64, 128, 1, F32, "gate", True, True, 2),      # fp32: the general kernel
    # the chunked kernel: two groups, exactly one chunk, one token past a chunk
    (2, 130, 4, 64, 128, 2, BF16, "gate", True, True, 2),
    (1, 64, 3, 64, 128, 1, BF16, "gate", False, False, 0),
    (2, 65, 2, 64, 128, 1, BF16, "gate", True, True, 0),
]


@pytest.mark.parametrize("B,L,H,P,N,G,dtype,form,with_dt,with_init,segs", CASES)
def test_scan_fwd_vector_decay_matches_oracle(B, L, H, P, N, G, dtype, form, with_dt, with_init,
                                               segs):
    import ssm_sequence_models_amd as ssm
    x, Bm, Cm, dt, gate, Av, h0, seq = _inputs(B, L, H, P, N, G, dtype, B + L + H + N, form,
                                               with_dt, with_init, segs)
    y, fin = ssm.scan_fwd_vector_decay(dev(x), dev(Bm), dev(Cm), log_decay=dev(gate),
                                       A_vec=dev(Av), dt=dev(dt), initial_state=dev(h0),
                                       seq_idx=dev(seq))
    torch.cuda.synchronize()
    ry, rfin = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, A_vec=Av, init_state=h0,
                                      seq_idx=seq, out_dtype=ODT[dtype], state_dtype="f32")
    assert_close(y, ry, "y")
    assert_close(fin, rfin, "final state")


def test_scan_fwd_vector_decay_len0_inplace_and_chain():
    """L = 0 returns the initial state; the final state may overwrite the initial state; two
    chained calls equal one."""
    import ssm_sequence_models_amd as ssm
    x, Bm, Cm, dt, gate, _, h0, _ = _inputs(2, 260, 4, 64, 128, 1, BF16, 5, "gate", True, True, 0)
    d = dev
    _, f0 = ssm.scan_fwd_vector_decay(d(x[:, :0].contiguous()), d(Bm[:, :0].contiguous()),
                                      d(Cm[:, :0].contiguous()), log_decay=d(gate[:, :0].contiguous()),
                                      dt=d(dt[:, :0].contiguous()), initial_state=d(h0))
    yw, fw = ssm.scan_fwd_vector_decay(d(x), d(Bm), d(Cm), log_decay=d(gate), dt=d(dt),
                                       initial_state=d(h0))
    st = d(h0).clone()
    ys = []
    for a, e in ((0, 111), (111, 260)):
        sl = lambda t: d(t[:, a:e].contiguous())
        yc, _ = ssm.scan_fwd_vector_decay(sl(x), sl(Bm), sl(Cm), log_decay=sl(gate), dt=sl(dt),
                                          initial_state=st, final_state=st)
        ys.append(yc)
    torch.cuda.synchronize()
    assert torch.equal(f0.cpu(), h0), "L = 0: the final state is the initial state"
    assert_close(torch.cat(ys, dim=1), yw.cpu().double().numpy(), "y (chained)")
    assert_close(st, fw.cpu().double().numpy(), "final state (chained, in place)")


def test_scan_fwd_vector_decay_full_size_sampled_heads():
    """The 1.3B-like shape (B 4, L 8192, 64 heads x 64, N 128) with GLA-like gates, initial
    states; heads 0 and 37 of every row checked against the oracle (heads are independent and
    share B / C with G = 1, so the oracle sees only those heads' inputs)."""
    import ssm_sequence_models_amd as ssm
    B, L, H, P, N = 4, 8192, 64, 64, 128
    g = torch.Generator(device="cuda").manual_seed(41)
    x = torch.randn(B, L, H, P, generator=g, device="cuda").to(BF16)
    Bm = torch.randn(B, L, 1, N, generator=g, device="cuda").to(BF16)
    Cm = torch.randn(B, L, 1, N, generator=g, device="cuda").to(BF16)
    dt = torch.nn.functional.softplus(torch.randn(B, L, H, generator=g, device="cuda") - 2.0)
    gate = workloads.vector_decay_gates(B, L, H, N, 42, device="cuda")
    h0 = torch.randn(B, H, P, N, generator=g, device="cuda")
    y, fin = ssm.scan_fwd_vector_decay(x, Bm, Cm, log_decay=gate, dt=dt, initial_state=h0)
    torch.cuda.synchronize()
    heads = [0, 37]
    cpu = lambda t: t.cpu()
    ry, rfin = oracle.scan_fwd_vdecay(cpu(x[:, :, heads]), cpu(dt[:, :, heads]), cpu(Bm), cpu(Cm),
                                      log_decay=cpu(gate[:, :, heads]), init_state=cpu(h0[:, heads]),
                                      out_dtype="bf16", state_dtype="f32")
    assert_close(y[:, :, heads], ry, "y (sampled heads)")
    assert_close(fin[:, heads], rfin, "final state (sampled heads)")


# The chunked (matrix-core) kernel takes the gate form with bf16, 64 channels and 128
# dimensions; a chunk whose summed log decay leaves its range runs token by token.  These rows
# mix such chunks with ordinary ones: gates scaled up over a stretch of the row (fast decays,
# one token's gate alone below the bound), with and without packed sequences and dt.
FALLBACK_CASES = [
    # B, L, H, scale, stretch (first, last token), dt, segments
    (2, 333, 3, 60.0, (64, 200), True, 0),
    (1, 256, 2, 200.0, (0, 256), False, 3),
    (2, 190, 2, 1000.0, (100, 101), True, 2),
]


@pytest.mark.parametrize("B,L,H,scale,stretch,with_dt,segs", FALLBACK_CASES)
def test_scan_fwd_vector_decay_fast_decay_chunks(B, L, H, scale, stretch, with_dt, segs):
    import ssm_sequence_models_amd as ssm
    x, Bm, Cm, dt, gate, _, h0, seq = _inputs(B, L, H, 64, 128, 1, BF16, 7 + L, "gate", with_dt,
                                              True, segs)
    gate = gate.clone()
    gate[:, stretch[0]:stretch[1]] *= scale
    y, fin = ssm.scan_fwd_vector_decay(dev(x), dev(Bm), dev(Cm), log_decay=dev(gate), dt=dev(dt),
                                       initial_state=dev(h0), seq_idx=dev(seq))
    torch.cuda.synchronize()
    ry, rfin = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, init_state=h0, seq_idx=seq,
                                      out_dtype="bf16", state_dtype="f32")
    assert_close(y, ry, "y")
    assert_close(fin, rfin, "final state")


def test_scan_fwd_vector_decay_nan_gate_propagates():
    """A NaN gate at token t of one dimension reaches that dimension's state from t on, as in
    the recurrence itself; the other rows and heads stay finite and match the oracle."""
    import ssm_sequence_models_amd as ssm
    x, Bm, Cm, dt, gate, _, h0, _ = _inputs(2, 150, 2, 64, 128, 1, BF16, 19, "gate", True, True, 0)
    gate = gate.clone()
    gate[0, 70, 1, 5] = float("nan")
    y, fin = ssm.scan_fwd_vector_decay(dev(x), dev(Bm), dev(Cm), log_decay=dev(gate), dt=dev(dt),
                                       initial_state=dev(h0))
    torch.cuda.synchronize()
    ry, rfin = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, init_state=h0,
                                      out_dtype="bf16", state_dtype="f32")
    yc, fc = y.cpu().float(), fin.cpu()
    ry_t, rf_t = torch.from_numpy(np.asarray(ry)).float(), torch.from_numpy(np.asarray(rfin)).float()
    assert torch.equal(torch.isnan(yc), torch.isnan(ry_t)), "NaN pattern of y"
    assert torch.equal(torch.isnan(fc), torch.isnan(rf_t)), "NaN pattern of the final state"
    ok = ~torch.isnan(ry_t)
    assert_close(torch.where(ok, yc, torch.zeros_like(yc)), torch.where(ok, ry_t, torch.zeros_like(ry_t)).double().numpy(), "finite y")


def test_scan_fwd_vector_decay_starts_at_chunk_edges():
    """Sequence starts at tokens 64 and 128 (the first tokens of chunks 1 and 2 of the chunked
    kernel), at 129 and at 191 (a chunk's last token): the state must be zero before each."""
    import ssm_sequence_models_amd as ssm
    x, Bm, Cm, dt, gate, _, h0, _ = _inputs(2, 200, 2, 64, 128, 1, BF16, 23, "gate", True, True, 0)
    seq = torch.zeros(2, 200, dtype=torch.int32)
    for t in (64, 128, 129, 191):
        seq[:, t:] += 1
    seq[1, 192:] += 1  # row 1 also starts one at 192
    y, fin = ssm.scan_fwd_vector_decay(dev(x), dev(Bm), dev(Cm), log_decay=dev(gate), dt=dev(dt),
                                       initial_state=dev(h0), seq_idx=dev(seq))
    torch.cuda.synchronize()
    ry, rfin = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, init_state=h0, seq_idx=seq,
                                      out_dtype="bf16", state_dtype="f32")
    assert_close(y, ry, "y")
    assert_close(fin, rfin, "final state")
