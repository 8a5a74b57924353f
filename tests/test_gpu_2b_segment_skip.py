"""GPU parity of long rows that run as segments, where each segment's state-only pass may
start late: the tokens before the last chunk whose remaining log-decay sum to the segment end
is below -208 reach the segment's end state with a factor below 1e-90 (length-generalization
notes Sec. 2.5, the initial-state increment; Sec. 2.1 Eq. (1)).  The cases force that start
(fast decays), keep it off (slow decays), and check the two guards on the skipped tokens: a NaN
step size there must still reach every later output, and a positive dt A there keeps the
whole segment.  Compared element by element with the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, cpu64, dev

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _long_row(L, H, seed, dt_val, A_vals):
    """One row of L tokens, H heads (P 64, N 128, G 1, K 4): with B * H = 2 and L = 4096 the
    call runs as 16 segments of 4 chunks."""
    P, N, G, K = 64, 128, 1, 4
    C = H * P + 2 * G * N
    g = torch.Generator().manual_seed(seed)
    xBC = torch.randn(1, L, C, generator=g).to(BF16)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    dt = torch.full((1, L, H), float(dt_val))
    A = torch.tensor(A_vals, dtype=torch.float32)
    cinit = torch.randn(1, C, K - 1, generator=g).to(BF16)
    sinit = torch.randn(1, H, P, N, generator=g)
    return xBC, w, b, dt, A, cinit, sinit, (P, N, G)


def _run(xBC, w, b, dt, A, cinit, sinit, H, P, N, G):
    import ssm_sequence_models_amd as ssm
    y, _, sf = ssm.conv_scan_fwd(dev(xBC), dev(w), dev(b), dev(dt), dev(A), H, P, G, N,
                                 conv_initial_state=dev(cinit), initial_state=dev(sinit))
    torch.cuda.synchronize()
    ry, _, rs = oracle.conv_scan_fwd(xBC, w, b, cinit, dt, A, sinit, None, H, P, G, N)
    return y, sf, ry, rs


@pytest.mark.parametrize("dt_val,A_vals", [
    (1.0, [-16.0, -0.01]),   # head 0: -16 per token, the state pass keeps 1 of 4 chunks;
                             # head 1: -0.01 per token, never below -208 within a segment
    (0.5, [-3.0, -2.0]),     # head 0: -1.5 per token, it keeps 3 of 4 chunks; head 1: -1 per
                             # token, below -208 only from the segment's first chunk (keeps 4)
])
def test_segments_with_late_state_pass_match_oracle(dt_val, A_vals):
    xBC, w, b, dt, A, cinit, sinit, (P, N, G) = _long_row(4096, 2, 61, dt_val, A_vals)
    y, sf, ry, rs = _run(xBC, w, b, dt, A, cinit, sinit, 2, P, N, G)
    assert_close(y, ry, "y")
    assert_close(sf, rs, "final state")


def test_segments_with_mixed_decays_match_oracle():
    """Per-token step sizes that vary by orders of magnitude (some segments cross, some do not,
    at different chunks)."""
    xBC, w, b, dt, A, cinit, sinit, (P, N, G) = _long_row(4096, 2, 62, 1.0, [-3.0, -0.5])
    g = torch.Generator().manual_seed(63)
    dt = torch.exp(torch.rand(1, 4096, 2, generator=g) * 8.0 - 7.0)   # 1e-3 .. 3
    y, sf, ry, rs = _run(xBC, w, b, dt, A, cinit, sinit, 2, P, N, G)
    assert_close(y, ry, "y")
    assert_close(sf, rs, "final state")


def test_nan_step_in_a_skippable_range_reaches_later_outputs():
    """A NaN dt at token 5 of head 0 (inside the part of segment 0 a fast decay would let the
    state pass skip): the segment is kept, and y and the final state are NaN exactly where the
    oracle's are; head 1 and head 0's first five tokens match."""
    xBC, w, b, dt, A, cinit, sinit, (P, N, G) = _long_row(4096, 2, 64, 1.0, [-16.0, -0.01])
    dt[0, 5, 0] = float("nan")
    y, sf, ry, rs = _run(xBC, w, b, dt, A, cinit, sinit, 2, P, N, G)
    gy, gs = cpu64(y), cpu64(sf)
    ry, rs = np.asarray(ry, dtype=np.float64), np.asarray(rs, dtype=np.float64)
    assert np.isnan(ry[0, 5:, 0]).all() and np.isnan(rs[0, 0]).all()
    assert np.array_equal(np.isnan(gy), np.isnan(ry)), "NaN positions of y differ"
    assert np.array_equal(np.isnan(gs), np.isnan(rs)), "NaN positions of the final state differ"
    assert_close(gy[0, :, 1], ry[0, :, 1], "y head 1")
    assert_close(gy[0, :5, 0], ry[0, :5, 0], "y head 0 before the NaN")
    assert_close(gs[0, 1], rs[0, 1], "final state head 1")


def test_positive_log_decay_in_a_skippable_range_keeps_the_segment():
    """dt < 0 at one early token of a segment (dt A > 0 there): the bound on the skipped
    tokens' factors no longer holds, so the state pass runs the whole segment."""
    xBC, w, b, dt, A, cinit, sinit, (P, N, G) = _long_row(4096, 2, 65, 1.0, [-16.0, -0.01])
    for t in (3, 260, 1030):     # early tokens of segments 0, 1 and 4
        dt[0, t, 0] = -0.05      # dt A = +0.8
    y, sf, ry, rs = _run(xBC, w, b, dt, A, cinit, sinit, 2, P, N, G)
    assert_close(y, ry, "y")
    assert_close(sf, rs, "final state")
