"""GPU parity of the initial-state distributions for training (length-generalization notes
Sec. 2.6) against the fp64 oracle, through the C-ABI: the Fitted Noise statistics update,
Random / Fitted noise initial states (same Philox4x64-10 stream, Box-Muller in fp32 on the
GPU), and State Passing's reset (decisions bit-exact, rows copied or zeroed exactly)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev

pytestmark = pytest.mark.gpu


def _final_states(shape, seed, offset=0.0):
    g = torch.Generator().manual_seed(seed)
    B, H, P, N = shape
    scale = torch.rand(1, H, 1, 1, generator=g) * 3 + 0.05
    shift = torch.randn(1, H, 1, 1, generator=g) * 2 + offset
    return torch.randn(shape, generator=g) * scale + shift


STATS_CASES = [
    ((4, 64, 64, 128), 0.0),     # the 1.3B layer's final states
    ((2, 6, 3, 5), 0.0),         # P N not a multiple of 4
    ((3, 4, 16, 32), 1e4),       # a large common offset (the variance stays exact)
    ((1, 1, 1, 1), 0.0),         # one element: variance 0
]


@pytest.mark.parametrize("shape,offset", STATS_CASES)
def test_state_stats_update_matches_oracle(shape, offset):
    import ssm_sequence_models_amd as ssm
    H = shape[1]
    fin = _final_states(shape, seed=sum(shape), offset=offset)
    g = torch.Generator().manual_seed(3)
    m0 = torch.randn(H, generator=g)
    v0 = torch.rand(H, generator=g) + 0.1
    m, v = dev(m0).clone(), dev(v0).clone()
    rm, rv = m0.double().numpy(), v0.double().numpy()
    for step in range(2):  # two updates in a row, the second from the first's output
        ssm.state_stats_update(dev(fin), m, v, beta=0.1)
        rm, rv = oracle.state_stats_update(fin, rm, rv, beta=0.1, out_dtype="f32")
    torch.cuda.synchronize()
    gm, gv = m.cpu().double().numpy(), v.cpu().double().numpy()
    np.testing.assert_allclose(gm, rm, rtol=1e-6, atol=1e-6 * (1 + np.abs(offset)))
    np.testing.assert_allclose(gv, rv, rtol=1e-6, atol=1e-12)


def test_state_stats_update_unaligned_and_empty():
    import ssm_sequence_models_amd as ssm
    shape = (2, 3, 8, 8)
    fin = _final_states(shape, seed=5)
    buf = torch.zeros(fin.numel() + 1, device="cuda")
    buf[1:] = dev(fin).reshape(-1)
    view = buf[1:].view(shape)  # 4-byte aligned only: the scalar path
    m, v = torch.zeros(3, device="cuda"), torch.zeros(3, device="cuda")
    ssm.state_stats_update(view, m, v, beta=0.1)
    rm, rv = oracle.state_stats_update(fin, np.zeros(3), np.zeros(3), beta=0.1, out_dtype="f32")
    m2, v2 = m.clone(), v.clone()
    ssm.state_stats_update(torch.empty(0, 3, 8, 8, device="cuda"), m2, v2, beta=0.1)
    torch.cuda.synchronize()
    np.testing.assert_allclose(m.cpu().double().numpy(), rm, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(v.cpu().double().numpy(), rv, rtol=1e-6, atol=1e-12)
    assert torch.equal(m2, m) and torch.equal(v2, v), "batch 0 leaves the statistics unchanged"


NOISE_CASES = [
    ((4, 64, 64, 128), True),
    ((4, 8, 64, 128), False),
    ((1, 3, 5, 7), True),        # 105 elements: a ragged last Philox block
    ((2, 2, 1, 3), False),
]


@pytest.mark.parametrize("shape,fitted", NOISE_CASES)
def test_initial_state_noise_matches_oracle(shape, fitted):
    import ssm_sequence_models_amd as ssm
    B, H, P, N = shape
    g = torch.Generator().manual_seed(B * H + P)
    mean = torch.randn(H, generator=g) * 2 if fitted else None
    var = torch.rand(H, generator=g) * 3 + 0.01 if fitted else None
    sigma, seed, off = 0.75, 0x5EED0000 + H, 12 + N
    out = ssm.initial_state_noise(B, H, P, N, mean=dev(mean), var=dev(var), sigma=sigma,
                                  seed=seed, offset=off)
    again = ssm.initial_state_noise(B, H, P, N, mean=dev(mean), var=dev(var), sigma=sigma,
                                    seed=seed, offset=off)
    other = ssm.initial_state_noise(B, H, P, N, mean=dev(mean), var=dev(var), sigma=sigma,
                                    seed=seed, offset=off + 1)
    torch.cuda.synchronize()
    ref = oracle.initial_state_noise(shape, mean=mean, var=var, sigma=sigma, seed=seed,
                                     offset=off, out_dtype="f64")
    got = out.cpu().double().numpy()
    # fp32 Box-Muller: |z| <= 5.8, its absolute error below 2e-6 (log, sqrt and sincospi at
    # about one ulp each); the fitted value adds mean's rounding
    if fitted:
        scale = (np.abs(mean.double().numpy()) + np.sqrt(var.double().numpy()) * 6)[None, :, None, None]
    else:
        scale = np.full((1, 1, 1, 1), sigma * 6)
    err = np.abs(got - ref)
    assert np.all(err <= 2e-6 * scale), float((err / scale).max())
    assert torch.equal(out, again), "same seed and offset: same draws"
    assert not torch.equal(out, other)


RESET_CASES = [
    ((1000, 4352, 3), torch.bfloat16, 0.1),   # conv states of the 1.3B layer: 16-byte units
    ((1000, 8, 16, 32), torch.float32, 0.1),  # SSM states
    ((257, 3, 3), torch.bfloat16, 0.5),       # 18-byte rows: 2-byte units
    ((64, 5), torch.float32, 0.0),
    ((64, 5), torch.float32, 1.0),
]


@pytest.mark.parametrize("shape,dtype,p", RESET_CASES)
def test_state_reset_matches_oracle(shape, dtype, p):
    import ssm_sequence_models_amd as ssm
    g = torch.Generator().manual_seed(shape[0])
    st = torch.randn(shape, generator=g).to(dtype)
    seed, off = 77, 9
    out, mask = ssm.state_reset(dev(st), p=p, seed=seed, offset=off)
    inplace = dev(st).clone()
    _, mask2 = ssm.state_reset(inplace, p=p, seed=seed, offset=off, out=inplace)
    torch.cuda.synchronize()
    ref, rmask = oracle.state_reset(st, p=p, seed=seed, offset=off)
    assert np.array_equal(mask.cpu().numpy(), rmask), "reset decisions"
    assert np.array_equal(mask2.cpu().numpy(), rmask)
    want = torch.from_numpy(ref).to(dtype)
    assert torch.equal(out.cpu(), want)
    assert torch.equal(inplace.cpu(), want)


def test_state_reset_same_rows_for_conv_and_ssm_states():
    import ssm_sequence_models_amd as ssm
    B = 300
    conv = torch.randn(B, 4352, 3, device="cuda").to(torch.bfloat16)
    st = torch.randn(B, 64, 64, 128, device="cuda")
    _, m1 = ssm.state_reset(conv, p=0.1, seed=3, offset=41)
    _, m2 = ssm.state_reset(st, p=0.1, seed=3, offset=41, out=st)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2)
    z = m2.bool()
    assert float(st[z].abs().max()) == 0.0 if bool(z.any()) else True
    assert bool((st[~z].abs().amax(dim=(1, 2, 3)) > 0).all())
