"""The decode step as one call (ssm_decode_step) against its definition as two calls,
ssm_conv1d_update then ssm_step on the channel ranges of the conv output: y, the conv outputs
and both pools bit for bit, for circular and linear caches, several widths, group counts and
state sizes, with rows whose slots lie outside a pool and SSM slots that differ from the conv
slots.  The two-call composition is itself checked against the fp64 oracle by the decode
tests."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _case(R, S, H, P, N, G, K, sl, L, seed, circular=True, split_slots=False):
    C = H * P + 2 * G * N
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(R, C, L, generator=g).to(BF16)
    pool = torch.randn(S, C, sl, generator=g).to(BF16)
    w = torch.rand(C, K, generator=g) - 0.5
    b = torch.rand(C, generator=g) - 0.5
    dt = torch.nn.functional.softplus(torch.randn(R, L, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * float(np.log(16.0)))
    spool = torch.randn(S, H, P, N, generator=g)
    idx = torch.randperm(S, generator=g)[:R].to(torch.int32)
    idx[1] = S + 3          # a row outside the conv pool
    sidx = None
    if split_slots:
        sidx = torch.randperm(S, generator=g)[:R].to(torch.int32)
        sidx[2] = -1        # a row outside the SSM pool
    seqlens = torch.randint(0, 1000, (R,), generator=g).to(torch.int32) if circular else None
    return dict(x=x, pool=pool, w=w, b=b, dt=dt, A=A, spool=spool, idx=idx, sidx=sidx,
                seqlens=seqlens, dims=(H, P, G, N))


def _bits(t):
    return t.view(torch.int16) if t.dtype == BF16 else t.view(torch.int32)


def _run(c, fused):
    import ssm_sequence_models_amd as ssm
    H, P, G, N = c["dims"]
    d = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    pool, spool = d["pool"].clone(), d["spool"].clone()
    R, C, L = d["x"].shape
    if fused:
        co = torch.empty_like(d["x"])
        y = ssm.decode_step(d["x"], pool, d["w"], d["b"], d["dt"], d["A"], spool, H, P, G, N,
                            conv_state_indices=d["idx"], cache_seqlens=d["seqlens"],
                            state_indices=d["sidx"], conv_out=co)
    else:
        co = ssm.conv1d_update(d["x"], pool, d["w"], d["b"], conv_state_indices=d["idx"],
                               cache_seqlens=d["seqlens"], activation="silu")
        HP, GN = H * P, G * N
        y = ssm.step(co[:, :HP, :].transpose(1, 2), d["dt"], d["A"], co[:, HP:HP + GN, :].transpose(1, 2),
                     co[:, HP + GN:, :].transpose(1, 2), spool,
                     d["sidx"] if d["sidx"] is not None else d["idx"])
    torch.cuda.synchronize()
    return y.cpu(), co.cpu(), pool.cpu(), spool.cpu()


CASES = {
    "1p3b_dims_Lnew1": dict(R=6, S=12, H=4, P=64, N=128, G=1, K=4, sl=4, L=1),
    "groups2_K3_Lnew2": dict(R=5, S=9, H=4, P=64, N=128, G=2, K=3, sl=6, L=2),
    "K6_window8_Lnew2": dict(R=4, S=8, H=2, P=64, N=64, G=1, K=6, sl=8, L=2),
    "small_state_P32_N16": dict(R=7, S=10, H=3, P=32, N=16, G=1, K=4, sl=5, L=2),
    "full_ring_Lnew4": dict(R=5, S=8, H=2, P=64, N=128, G=1, K=4, sl=4, L=4),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("split_slots", [False, True])
def test_decode_step_equals_two_calls(name, split_slots):
    c = _case(**CASES[name], seed=100 + len(name), split_slots=split_slots)
    for got, ref, what in zip(_run(c, True), _run(c, False), ("y", "conv_out", "conv pool", "ssm pool")):
        assert torch.equal(_bits(got), _bits(ref)), f"{name}: {what} differs"


def test_decode_step_linear_layout_equals_two_calls():
    c = _case(R=5, S=8, H=2, P=64, N=128, G=1, K=4, sl=5, L=1, seed=120, circular=False,
              split_slots=True)
    for got, ref, what in zip(_run(c, True), _run(c, False), ("y", "conv_out", "conv pool", "ssm pool")):
        assert torch.equal(_bits(got), _bits(ref)), f"linear layout: {what} differs"
