"""Seeded synthetic inputs for the SSM scan + causal conv1d path.

This module only draws random numbers: it holds none of the method's arithmetic, and it is
the one piece shared by the oracle side and the HIP side (tests, smoke check, benchmark).
Everything is generated on the CPU with a seeded ``torch.Generator``, so both sides see
bit-identical inputs.

The pages measure on public corpora and trained models that are not available here; these
synthetic inputs stand in for them.  Layer shapes follow the Mamba-2 370M / 780M / 1.3B
models and the 2K-128K context lengths of the length-generalization reading notes (Sec. 4,
Fig. 5 / Fig. 1 settings); the decode pool follows the causal-conv1d tutorial ch. 7
(state_len, cache_seqlens, conv_state_indices).

Distributions (fixed recipe):
  x, B, C channels (xBC)  ~ N(0, 1), stored as bf16 (fp32 for the tiny case)
  dt                      = softplus(N(0, 1) - 2), fp32           (mean ~0.18)
  A (one per head)        = -exp(U(log 1, log 16)), fp32
  conv weight, bias       ~ U(-0.5, 0.5) = U(-1/sqrt(K), 1/sqrt(K)) for K = 4, fp32
  packed seq_idx          3 distinct cut points uniform in 1 .. L-1 per row -> ids 0..3
  per-dimension log gates = logsigmoid(N(0, 1)) / 16, fp32 (mean ~ -0.05; the data-dependent
                            gates of the diagonal-transition models, with the normaliser 16
                            gated linear attention uses)
  per-dimension rates     = -exp(U(log 1, log 16)) per (head, state dimension), fp32
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

# Named workloads.  Sizes are the layer shapes described above.
CONFIGS = {
    # tiny case: 1 head, headdim 4, state 4, fp32; random initial states
    "tiny": dict(B=1, L=64, H=1, P=4, N=4, G=1, K=4, dtype="f32", seed=0, init="random"),
    # Mamba-2 370M-like layer: d_inner 2048 = 32 heads x 64, zero initial state
    "layer370m": dict(B=8, L=2048, H=32, P=64, N=128, G=1, K=4, dtype="bf16", seed=1,
                      init="zero"),
    # Mamba-2 1.3B-like layer: d_inner 4096 = 64 heads x 64, initial states = final states
    # of a preceding 8192-token run drawn with seed 2 (state passing)
    "layer1p3b": dict(B=4, L=8192, H=64, P=64, N=128, G=1, K=4, dtype="bf16", seed=3,
                      init="passed", pre_seed=2, packed_seed=4),
    # Mamba-2 780M-like layer: d_inner 3072 = 48 heads x 64, 131072 tokens, zero initial
    # state, also processed as 64 chained 2048-token calls
    "layer780m": dict(B=1, L=131072, H=48, P=64, N=128, G=1, K=4, dtype="bf16", seed=5,
                      init="zero", chunk_len=2048),
}

DECODE = dict(R=256, n_slots=512, H=64, P=64, N=128, G=1, K=4, state_len=4, dtype="bf16",
              seed=6, max_seqlen=100000)

TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Shape:
    B: int
    L: int
    H: int
    P: int
    N: int
    G: int
    K: int
    dtype: str

    @property
    def C(self) -> int:
        """conv channels, in x | B | C order"""
        return self.H * self.P + 2 * self.G * self.N


def shape_of(name: str, **overrides) -> Shape:
    cfg = dict(CONFIGS[name])
    s = Shape(B=cfg["B"], L=cfg["L"], H=cfg["H"], P=cfg["P"], N=cfg["N"], G=cfg["G"],
              K=cfg["K"], dtype=cfg["dtype"])
    return replace(s, **overrides) if overrides else s


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, dtype) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(TORCH_DTYPE[dtype])


def _softplus_shifted(shape, g) -> torch.Tensor:
    z = torch.randn(shape, generator=g, dtype=torch.float32) - 2.0
    return torch.nn.functional.softplus(z).contiguous()


def _neg_exp_uniform(H, g) -> torch.Tensor:
    u = torch.rand(H, generator=g, dtype=torch.float32) * (math.log(16.0) - math.log(1.0))
    return (-torch.exp(u)).contiguous()


def _uniform(shape, g, lo, hi) -> torch.Tensor:
    return (torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo).contiguous()


def conv_params(C: int, K: int, seed: int):
    """conv weight [C, K] and bias [C], U(-0.5, 0.5) fp32 (shared by all calls of a layer)."""
    g = _gen(seed * 1000 + 17)
    w = _uniform((C, K), g, -0.5, 0.5)
    b = _uniform((C,), g, -0.5, 0.5)
    return w, b


def layer_params(s: Shape, seed: int):
    """Per-layer parameters: conv weight/bias and A [H]."""
    w, b = conv_params(s.C, s.K, seed)
    A = _neg_exp_uniform(s.H, _gen(seed * 1000 + 29))
    return w, b, A


def prefill_inputs(s: Shape, seed: int, with_random_init: bool = False) -> dict:
    """Activations for one prefill call: xBC [B, L, C], dt [B, L, H] and, when asked,
    random N(0, 1) initial states (conv [B, C, K-1] in the input dtype, SSM [B, H, P, N]
    fp32)."""
    g = _gen(seed)
    out = {
        "xBC": _normal((s.B, s.L, s.C), g, s.dtype).contiguous(),
        "dt": _softplus_shifted((s.B, s.L, s.H), g),
    }
    if with_random_init:
        out["conv_init"] = _normal((s.B, s.C, s.K - 1), g, s.dtype).contiguous()
        out["ssm_init"] = torch.randn((s.B, s.H, s.P, s.N), generator=g,
                                      dtype=torch.float32).contiguous()
    return out


def packed_seq_idx(B: int, L: int, seed: int, n_segments: int = 4) -> torch.Tensor:
    """seq_idx [B, L] int32 marking n_segments packed sequences of random lengths: per row,
    n_segments - 1 distinct cut points drawn uniformly from 1 .. L-1."""
    g = _gen(seed)
    rows = []
    for _ in range(B):
        cuts = torch.randperm(L - 1, generator=g)[: n_segments - 1] + 1
        cuts, _ = torch.sort(cuts)
        ids = torch.zeros(L, dtype=torch.int32)
        for c in cuts.tolist():
            ids[c:] += 1
        rows.append(ids)
    return torch.stack(rows).contiguous()


def decode_inputs(L_new: int = 1, seed: int | None = None, R: int | None = None,
                  n_slots: int | None = None, H: int | None = None, P: int | None = None,
                  N: int | None = None, G: int | None = None, with_ssm_pool: bool = True,
                  max_seqlen: int | None = None) -> dict:
    """One decode step for R requests mapped into n_slots-slot pools.

    conv pool [n_slots, C, state_len] bf16 ~ N(0, 1); SSM pool [n_slots, H, P, N] fp32 ~
    N(0, 1); indices = randperm(n_slots)[:R] (distinct, shared by both pools);
    cache_seqlens ~ U{0 .. max_seqlen}; x_new [R, C, L_new] bf16 ~ N(0, 1) (the conv input);
    dt [R, L_new, H] as in prefill."""
    d = dict(DECODE)
    for k, v in (("seed", seed), ("R", R), ("n_slots", n_slots), ("H", H), ("P", P),
                 ("N", N), ("G", G), ("max_seqlen", max_seqlen)):
        if v is not None:
            d[k] = v
    C = d["H"] * d["P"] + 2 * d["G"] * d["N"]
    g = _gen(d["seed"])
    out = {
        "cfg": dict(d, C=C, L_new=L_new),
        "conv_pool": _normal((d["n_slots"], C, d["state_len"]), g, d["dtype"]).contiguous(),
        "indices": torch.randperm(d["n_slots"], generator=g)[: d["R"]].to(torch.int32)
        .contiguous(),
        "cache_seqlens": torch.randint(0, d["max_seqlen"] + 1, (d["R"],), generator=g,
                                       dtype=torch.int64).to(torch.int32).contiguous(),
        "x_new": _normal((d["R"], C, L_new), g, d["dtype"]).contiguous(),
        "dt": _softplus_shifted((d["R"], L_new, d["H"]), g),
    }
    if with_ssm_pool:
        out["ssm_pool"] = torch.randn((d["n_slots"], d["H"], d["P"], d["N"]), generator=g,
                                      dtype=torch.float32).contiguous()
    w, b = conv_params(C, d["K"], d["seed"])
    out["conv_w"], out["conv_b"] = w, b
    out["A"] = _neg_exp_uniform(d["H"], _gen(d["seed"] * 1000 + 29))
    return out


def vector_decay_gates(B: int, L: int, H: int, N: int, seed: int,
                       device: str | torch.device = "cpu") -> torch.Tensor:
    """log_decay [B, L, H, N] fp32 = logsigmoid(N(0, 1)) / 16 (generated on `device` with a
    generator seeded there, so large tensors need not cross the bus)."""
    g = torch.Generator(device=device).manual_seed(seed)
    z = torch.randn(B, L, H, N, generator=g, device=device)
    return torch.nn.functional.logsigmoid(z) / 16.0


def vector_decay_rates(H: int, N: int, seed: int) -> torch.Tensor:
    """A_vec [H, N] fp32 = -exp(U(log 1, log 16)): one rate per head and state dimension."""
    g = _gen(seed)
    return -torch.exp(torch.rand(H, N, generator=g) * math.log(16.0))
