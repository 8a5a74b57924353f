"""Helpers shared by the GPU parity tests: the tolerance, device transfer, and oracle runs on
a sampled subset of heads / channels (every head and channel is independent, so a subset of
the inputs gives exactly the oracle's outputs for that subset)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# bf16-input, fp32-state outputs and final states: |gpu - oracle| <= ABS + REL * |oracle|
TOL_ABS = 1e-3
TOL_REL = 2e-2


def cpu64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_close(gpu, ref, what: str, abs_tol: float = TOL_ABS, rel_tol: float = TOL_REL):
    g = cpu64(gpu)
    r = cpu64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    err = np.abs(g - r)
    bound = abs_tol + rel_tol * np.abs(r)
    bad = err > bound
    if bad.any():
        ratio = (err / bound).max()
        idx = np.unravel_index(np.argmax(err / bound), g.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} elements out of tolerance; "
                             f"worst ratio {ratio:.3g} at {idx}: gpu {g[idx]!r} oracle {r[idx]!r}")


def assert_bitexact(gpu, ref, what: str):
    g = gpu.detach().cpu() if isinstance(gpu, torch.Tensor) else torch.as_tensor(gpu)
    r = ref.detach().cpu() if isinstance(ref, torch.Tensor) else torch.as_tensor(ref)
    if g.dtype != r.dtype:
        g, r = g.to(torch.float64), r.to(torch.float64)
    neq = (g != r) & ~(torch.isnan(g.float()) & torch.isnan(r.float())) if g.is_floating_point() \
        else (g != r)
    n = int(neq.sum())
    assert n == 0, f"{what}: {n} of {g.numel()} elements differ"


def dev(t):
    return None if t is None else t.to("cuda")


def oracle_conv_scan_heads(xBC, conv_w, conv_b, conv_init, dt, A, ssm_init, seq_idx, H, P, G,
                           N, heads, act="silu", out_dtype="bf16"):
    """Oracle of the fused prefill restricted to `heads` (G = 1): conv over those heads' x
    channels and all B / C channels, then the scan of those heads.

    Returns (y [B, L, len(heads), P], ssm_final [B, len(heads), P, N],
             conv_final [B, len(chans), K-1], chans)."""
    assert G == 1
    HP = H * P
    chans = [h * P + p for h in heads for p in range(P)] + list(range(HP, HP + 2 * N))
    ci = torch.tensor(chans)
    xs = xBC[:, :, ci]
    ws = conv_w[ci]
    bs = None if conv_b is None else conv_b[ci]
    ins = None if conv_init is None else conv_init[:, ci]
    conv_out, conv_fin = oracle.conv1d_fwd(xs, ws, bs, ins, seq_idx, act=act, out_dtype=out_dtype)
    nh = len(heads)
    Bsz, L = conv_out.shape[:2]
    x = conv_out[:, :, :nh * P].reshape(Bsz, L, nh, P)
    Bm = conv_out[:, :, nh * P:nh * P + N].reshape(Bsz, L, 1, N)
    Cm = conv_out[:, :, nh * P + N:].reshape(Bsz, L, 1, N)
    hi = torch.tensor(heads)
    init = None if ssm_init is None else ssm_init[:, hi]
    y, fin = oracle.scan_fwd(x, dt[:, :, hi], A[hi], Bm, Cm, init, seq_idx, out_dtype=out_dtype,
                             state_dtype="f32")
    return y, fin, conv_fin, chans
