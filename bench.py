"""Benchmark of the fused SSM scan + causal conv1d prefill on one MI355X.

A step is one pass of the whole hot path over one batch: ssm_conv_scan_fwd on a Mamba-2
1.3B-like layer (batch 4 x 8192 tokens, 64 heads x headdim 64, state 128, conv width 4 over
4352 x|B|C channels, bf16 activations, fp32 states) whose initial conv / SSM states are the
final states of a preceding 8192-token call (state passing).  Inputs are seeded synthetic
tensors already resident in HBM.

Prints one JSON line: whole-job tokens/s, the roofline of the dominant kernel (the chunked
scan main kernel; its launch time comes from HIP events the library records around it on the
call's stream, in a separate instrumented pass) and the fp64 CPU oracle timed on the host
cores on the same workload.  Before every timed step (the headline's and every other entry
point's) a 512 MiB buffer is written, outside the timed interval, so no timed call finds its
inputs in the 256 MB last-level cache; each step is timed by events on the launch stream.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
# MFMAs the main kernel issues per (batch row, head, 64-token chunk): 4 consumer waves x (12
# intra-chunk + 32 initial-state + 32 state-update), each a 16x16x32 bf16 product
MFMA_PER_CHUNK_HEAD = 4 * (12 + 32 + 32)
FLOP_PER_MFMA = 2 * 16 * 16 * 32
METRIC = "SSM scan+conv tokens/sec (B×L, 1.3B layer, L=8K) and % HBM/MFMA roofline"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(s):
    """Bytes the fused prefill must move at least once (inputs read, outputs written)."""
    tok = s.B * s.L
    per_tok = s.C * 2 + s.H * 4 + s.H * s.P * 2          # xBC in, dt in, y out
    states = 2 * s.B * s.H * s.P * s.N * 4 + 2 * s.B * s.C * (s.K - 1) * 2
    main_per_tok = s.H * s.P * 2 + s.H * 4 + s.H * s.P * 2  # x channels, dt, y
    main_states = 2 * s.B * s.H * s.P * s.N * 4 + 2 * s.B * s.H * s.P * (s.K - 1) * 2
    return tok * per_tok + states, tok * main_per_tok + main_states


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("ssd.hip", "internal.h"):
        with open(os.path.join(ROOT, "ssm_sequence_models_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the main kernel from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "ssd_main_layer1p3b_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


_FLUSH = {}


def cache_flush(torch):
    """Write 512 MiB (twice the MI355X last-level cache) on the current stream."""
    buf = _FLUSH.get("buf")
    if buf is None:
        buf = _FLUSH["buf"] = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    _FLUSH["v"] = (_FLUSH.get("v", 0) + 1) & 0xFF
    buf.fill_(_FLUSH["v"])


def _time_steps(torch, fn, reps, flush=True):
    """Per-call milliseconds of fn() for reps calls, each bracketed by events on torch's
    current stream (the library launches on that stream), with the cache flush before each
    call outside the bracket."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        if flush:
            cache_flush(torch)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def _time_gpu(torch, fn, reps, warm=2):
    """Mean milliseconds of fn() over reps calls (cache flushed before each, see _time_steps)."""
    for _ in range(warm):
        fn()
    t = _time_steps(torch, fn, reps)
    return sum(t) / len(t)


def copy_bandwidth(torch, ssm):
    """Read + write bandwidth (GB/s) of two plain 1 GiB device-to-device copies: the runtime's
    own (torch's copy_) and the library's streaming copy (non-temporal 16-byte accesses, which
    outruns the runtime's on this GPU).  The faster is the reference for the fractions below,
    beside the 8 TB/s peak: what streaming code reaches on this machine."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    rt = 2 * n / (_time_gpu(torch, lambda: dst.copy_(src), 5) * 1e-3) / 1e9
    st = 2 * n / (_time_gpu(torch, lambda: ssm.stream_copy(src, dst), 5) * 1e-3) / 1e9
    del src, dst
    return max(rt, st), {"runtime_copy_GBs": rt, "stream_copy_GBs": st}


def other_ops(torch, ssm, workloads, copy_GBs, only=None):
    """Achieved bandwidth of the other entry points on their workloads: the unfused conv at the
    1.3B shape, the decode step (conv update + SSM step, 256 requests, L_new 1 and 4), the
    1.3B-like prefill with packed sequences, the 370M-like prefill, the 131072-token
    780M-like call, the chunked prefill on the decode pools, the initial-state distributions
    for training, the per-dimension (vector) decay scan, and the backward entry points (conv with state gradients, the scan's
    initial-state gradient) at the 1.3B shape.  Seeded
    inputs drawn on the GPU (timing only; parity is the test suite's job)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    res = []

    def timed(key, fn, reps, warm=2):
        """_time_gpu for the entry points `only` selects (all when None); None otherwise: their
        inputs are still drawn, so the random streams of the later ones do not change."""
        return _time_gpu(torch, fn, reps, warm) if only is None or key in only else None

    def rep(op, workload, ms, tokens, nbytes, extra=None):
        if ms is None:
            return
        res.append({"op": op, "workload": workload, "ms": ms, "tokens_per_s": tokens / (ms * 1e-3),
                    "algorithmic_bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                    "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "frac_of_copy": nbytes / (ms * 1e-3) / 1e9 / copy_GBs, **(extra or {})})

    def prefill_inputs(s, seed):
        g.manual_seed(seed)
        x = torch.randn(s.B, s.L, s.C, generator=g, device=dev).to(torch.bfloat16)
        dt = torch.nn.functional.softplus(torch.randn(s.B, s.L, s.H, generator=g, device=dev) - 2)
        w = (torch.rand(s.C, s.K, generator=g, device=dev) - 0.5).contiguous()
        b = torch.rand(s.C, generator=g, device=dev) - 0.5
        A = -torch.exp(torch.rand(s.H, generator=g, device=dev) * math.log(16.0))
        return x, dt.contiguous(), w, b, A

    # unfused conv at the 1.3B shape, with conv states in and out
    s = workloads.shape_of("layer1p3b")
    x, dt, w, b, A = prefill_inputs(s, 11)
    init = torch.zeros(s.B, s.C, s.K - 1, dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(x)
    fin = torch.empty_like(init)
    ms = timed("conv1d_fwd", lambda: ssm.conv1d_fwd(x, w, b, initial_state=init, activation="silu",
                                                  final_state=fin, out=out), 10)
    rep("conv1d_fwd", f"B{s.B} L{s.L} C{s.C} K{s.K} bf16 SiLU, states in/out", ms, s.B * s.L,
        2 * s.B * s.L * s.C * 2 + 2 * s.B * s.C * (s.K - 1) * 2 + s.C * (s.K + 1) * 4)
    del x, out

    # the same 1.3B layer packed with 4 sequences per row (seq_idx), zero initial states
    x, dt, w, b, A = prefill_inputs(s, 14)
    seq = workloads.packed_seq_idx(s.B, s.L, 4).to(dev)
    ws = torch.empty(ssm.workspace_size(s.B, s.L, s.H, s.P, s.G, s.N), dtype=torch.uint8, device=dev)
    ms = timed("packed1p3b", lambda: ssm.conv_scan_fwd(x, w, b, dt, A, s.H, s.P, s.G, s.N, seq_idx=seq,
                                                     workspace=ws), 10)
    nb = (s.B * s.L * (s.C * 2 + s.H * 4 + s.H * s.P * 2 + 4) + s.B * s.H * s.P * s.N * 4
          + s.B * s.C * (s.K - 1) * 2)
    rep("conv_scan_fwd", f"1.3B-like layer B{s.B} L{s.L} H{s.H}x{s.P} N{s.N}, 4 packed sequences per "
        "row (seq_idx), zero initial state", ms, s.B * s.L, nb)
    del x, ws

    # 370M-like prefill, zero initial states
    s = workloads.shape_of("layer370m")
    x, dt, w, b, A = prefill_inputs(s, 12)
    ws = torch.empty(ssm.workspace_size(s.B, s.L, s.H, s.P, s.G, s.N), dtype=torch.uint8, device=dev)
    ms = timed("layer370m", lambda: ssm.conv_scan_fwd(x, w, b, dt, A, s.H, s.P, s.G, s.N, workspace=ws), 10)
    nb = s.B * s.L * (s.C * 2 + s.H * 4 + s.H * s.P * 2) + s.B * s.H * s.P * s.N * 4 + s.B * s.C * (s.K - 1) * 2
    rep("conv_scan_fwd", f"370M-like layer B{s.B} L{s.L} H{s.H}x{s.P} N{s.N}, zero initial state", ms,
        s.B * s.L, nb)
    del x, ws

    # 780M-like layer, one 131072-token call
    s = workloads.shape_of("layer780m")
    x, dt, w, b, A = prefill_inputs(s, 13)
    ws = torch.empty(ssm.workspace_size(s.B, s.L, s.H, s.P, s.G, s.N), dtype=torch.uint8, device=dev)
    ms = timed("layer780m", lambda: ssm.conv_scan_fwd(x, w, b, dt, A, s.H, s.P, s.G, s.N, workspace=ws), 3, 1)
    nb = s.B * s.L * (s.C * 2 + s.H * 4 + s.H * s.P * 2) + s.B * s.H * s.P * s.N * 4 + s.B * s.C * (s.K - 1) * 2
    rep("conv_scan_fwd", f"780M-like layer B{s.B} L{s.L} H{s.H}x{s.P} N{s.N}, one call", ms, s.B * s.L, nb)
    del x, ws

    # 780M-like layer as 64 chained 2048-token calls, each call's final states written in place
    # over its initial states (state passing / truncated BPTT over one long sequence)
    Lc = workloads.CONFIGS["layer780m"]["chunk_len"]
    x, dt, w, b, A = prefill_inputs(s, 13)
    ncalls = s.L // Lc
    xs = [x[:, i * Lc:(i + 1) * Lc].contiguous() for i in range(ncalls)]
    dts = [dt[:, i * Lc:(i + 1) * Lc].contiguous() for i in range(ncalls)]
    del x, dt
    ws = torch.empty(ssm.workspace_size(s.B, Lc, s.H, s.P, s.G, s.N), dtype=torch.uint8, device=dev)
    cst = torch.zeros(s.B, s.C, s.K - 1, dtype=torch.bfloat16, device=dev)
    sst = torch.zeros(s.B, s.H, s.P, s.N, device=dev)
    yc = torch.empty(s.B, Lc, s.H, s.P, dtype=torch.bfloat16, device=dev)

    def chain():
        for i in range(ncalls):
            ssm.conv_scan_fwd(xs[i], w, b, dts[i], A, s.H, s.P, s.G, s.N, conv_initial_state=cst,
                              initial_state=sst, conv_final_state=cst, final_state=sst, y=yc,
                              workspace=ws)
    ms = timed("layer780m_chained", chain, 3, 1)
    per_call = (s.B * Lc * (s.C * 2 + s.H * 4 + s.H * s.P * 2) + 2 * s.B * s.H * s.P * s.N * 4
                + 2 * s.B * s.C * (s.K - 1) * 2)
    rep("conv_scan_fwd", f"780M-like layer B{s.B} L{s.L} H{s.H}x{s.P} N{s.N} as {ncalls} chained "
        f"{Lc}-token calls, states passed in place", ms, s.B * s.L, ncalls * per_call,
        {"calls": ncalls, "ms_per_call": ms / ncalls} if ms is not None else None)
    del xs, dts, ws, yc

    # decode step: conv update + SSM step on 512-slot pools, 256 requests
    d = workloads.DECODE
    H, P, N, G, K = d["H"], d["P"], d["N"], d["G"], d["K"]
    C = H * P + 2 * G * N
    R, S = d["R"], d["n_slots"]
    g.manual_seed(14)
    conv_pool = torch.randn(S, C, d["state_len"], generator=g, device=dev).to(torch.bfloat16)
    ssm_pool = torch.randn(S, H, P, N, generator=g, device=dev)
    idx = torch.randperm(S, generator=g, device=dev)[:R].to(torch.int32)
    seqlens = torch.randint(0, d["max_seqlen"] + 1, (R,), generator=g, device=dev).to(torch.int32)
    w = (torch.rand(C, K, generator=g, device=dev) - 0.5).contiguous()
    b = torch.rand(C, generator=g, device=dev) - 0.5
    A = -torch.exp(torch.rand(H, generator=g, device=dev) * math.log(16.0))
    for L_new in (1, 4):
        xn = torch.randn(R, C, L_new, generator=g, device=dev).to(torch.bfloat16)
        dtn = torch.nn.functional.softplus(torch.randn(R, L_new, H, generator=g, device=dev) - 2).contiguous()
        ms = timed("decode", lambda: ssm.decode_step(xn, conv_pool, w, b, dtn, A, ssm_pool, H, P, G, N,
                                                       conv_state_indices=idx, cache_seqlens=seqlens), 20)
        nb = (2 * R * H * P * N * 4 + 2 * R * C * d["state_len"] * 2 + 3 * R * C * L_new * 2
              + R * L_new * H * 4 + R * L_new * H * P * 2)
        rep("decode_step", f"{R} requests, {S}-slot pools (1.3B dims), L_new {L_new}", ms, R * L_new, nb)
    del conv_pool, ssm_pool

    # chunked prefill on the decode pools (continuous batching): 16 requests each add a
    # 2048-token chunk, states read from and written back to their ring-buffer slots
    R, Lp = 16, 2048
    g.manual_seed(17)
    conv_pool = torch.randn(S, C, d["state_len"], generator=g, device=dev).to(torch.bfloat16)
    ssm_pool = torch.randn(S, H, P, N, generator=g, device=dev)
    idx = torch.randperm(S, generator=g, device=dev)[:R].to(torch.int32)
    seqlens = torch.randint(0, d["max_seqlen"] + 1, (R,), generator=g, device=dev).to(torch.int32)
    xp = torch.randn(R, Lp, C, generator=g, device=dev).to(torch.bfloat16)
    dtp = torch.nn.functional.softplus(torch.randn(R, Lp, H, generator=g, device=dev) - 2).contiguous()
    yp = torch.empty(R, Lp, H, P, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ssm.conv_scan_fwd_pooled_workspace_size(R, Lp, H, P, G, N, K) + 256,
                     dtype=torch.uint8, device=dev)
    ms = timed("pooled", lambda: ssm.conv_scan_fwd_pooled(
        xp, w, b, dtp, A, conv_pool, ssm_pool, H, P, G, N, state_indices=idx,
        cache_seqlens=seqlens, y=yp, workspace=ws), 10)
    nb = (R * Lp * (C * 2 + H * 4 + H * P * 2) + 2 * R * H * P * N * 4
          + R * C * (K - 1 + min(Lp, d["state_len"])) * 2)
    rep("conv_scan_fwd_pooled", f"{R} requests x {Lp}-token chunk into {S}-slot pools (1.3B dims, "
        "ring layout)", ms, R * Lp, nb)
    del conv_pool, ssm_pool, xp, yp, ws

    # initial-state distributions for training on 64 carried SSM states of the 1.3B layer
    # (64 x 64 heads x 64 x 128 fp32 = 128 MiB): the Fitted Noise statistics update, Fitted
    # Noise sampling, and State Passing's reset (out of place)
    Rs = 64
    g.manual_seed(18)
    st = torch.randn(Rs, H, P, N, generator=g, device=dev)
    mean, var = torch.zeros(H, device=dev), torch.ones(H, device=dev)
    nbs = Rs * H * P * N * 4
    ms = timed("init_state", lambda: ssm.state_stats_update(st, mean, var, beta=0.1), 10)
    rep("state_stats_update", f"{Rs} x H{H}x{P} N{N} fp32 final states, per-head mean / variance",
        ms, Rs, nbs)
    noise = torch.empty_like(st)
    ms = timed("init_state", lambda: ssm.initial_state_noise(Rs, H, P, N, mean=mean, var=var, seed=1,
                                                          offset=2, out=noise), 10)
    rep("initial_state_noise", f"{Rs} x H{H}x{P} N{N} fp32, Fitted Noise (Philox4x64-10)", ms, Rs,
        nbs)
    kept = torch.empty_like(st)
    mask = torch.empty(Rs, dtype=torch.uint8, device=dev)
    ms = timed("init_state", lambda: ssm.state_reset(st, p=0.1, seed=1, offset=3, out=kept, mask=mask), 10)
    rep("state_reset", f"{Rs} x H{H}x{P} N{N} fp32, p 0.1, out of place", ms, Rs, 2 * nbs)
    del st, noise, kept

    # the scan with a diagonal, per-state-dimension transition at the 1.3B-like shape:
    # GLA-like data-dependent log gates [B, L, H, N] fp32 (1 GiB, most of the bytes), dt,
    # initial and final states
    s = workloads.shape_of("layer1p3b")
    g.manual_seed(19)
    xv = torch.randn(s.B, s.L, s.H, s.P, generator=g, device=dev).to(torch.bfloat16)
    Bv = torch.randn(s.B, s.L, 1, s.N, generator=g, device=dev).to(torch.bfloat16)
    Cv = torch.randn(s.B, s.L, 1, s.N, generator=g, device=dev).to(torch.bfloat16)
    dtv = torch.nn.functional.softplus(torch.randn(s.B, s.L, s.H, generator=g, device=dev) - 2)
    gate = workloads.vector_decay_gates(s.B, s.L, s.H, s.N, 20, device=dev)
    h0 = torch.randn(s.B, s.H, s.P, s.N, generator=g, device=dev)
    yv = torch.empty_like(xv)
    fv = torch.empty_like(h0)
    ms = timed("vector_decay", lambda: ssm.scan_fwd_vector_decay(xv, Bv, Cv, log_decay=gate, dt=dtv,
                                                            initial_state=h0, final_state=fv,
                                                            y=yv), 5)
    nb = (s.B * s.L * (2 * s.H * s.P * 2 + s.H * s.N * 4 + 2 * s.N * 2 + s.H * 4)
          + 2 * s.B * s.H * s.P * s.N * 4)
    # the gate form runs chunked on the matrix cores (64-token chunks): per (row, head, chunk)
    # 10 tiles x 12 MFMAs for the intra-chunk matrix and 4 waves x 92 for the inter / intra /
    # state products, 16x16x32 bf16 (16,384 flops each, hi / lo splits included).  Context: the
    # token-sequential form's issue floor (3 fp32 instructions per token, channel and
    # dimension at 64 lanes per CU per clock) is what this form is not bound by.
    n_chunk = (s.L + 63) // 64
    mfma_flops = s.B * s.H * n_chunk * (10 * 12 + 4 * 92) * 16384
    elems = s.B * s.L * s.H * s.P * s.N
    floor_ms = 3 * elems / (256 * 64 * 2.4e9) * 1e3
    rep("scan_fwd_vector_decay", f"1.3B-like B{s.B} L{s.L} H{s.H}x{s.P} N{s.N} bf16, per-dimension "
        "log gates [B, L, H, N] fp32, dt, initial / final state (chunked on the matrix cores)", ms,
        s.B * s.L, nb,
        {"bound": "hbm", "mfma_issued_flops": mfma_flops,
         "mfma_achieved_TFLOPs": mfma_flops / (ms * 1e-3) / 1e12,
         "mfma_frac": mfma_flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
         "token_form_issue_floor_ms": floor_ms} if ms is not None else None)
    del xv, Bv, Cv, dtv, gate, yv

    # backward of the unfused conv at the 1.3B shape, with state gradients
    s = workloads.shape_of("layer1p3b")
    x, dt, w, b, A = prefill_inputs(s, 15)
    g.manual_seed(16)
    dy = torch.randn(s.B, s.L, s.C, generator=g, device=dev).to(torch.bfloat16)
    init = torch.randn(s.B, s.C, s.K - 1, generator=g, device=dev).to(torch.bfloat16)
    dF = torch.randn(s.B, s.C, s.K - 1, generator=g, device=dev).to(torch.bfloat16)
    dx, dS = torch.empty_like(x), torch.empty_like(init)
    dw = torch.empty(s.C, s.K, device=dev)
    dbias = torch.empty(s.C, device=dev)
    ws = torch.empty(ssm.conv1d_bwd_workspace_size(s.B, s.L, s.C, s.K), dtype=torch.uint8, device=dev)
    ms = timed("conv1d_bwd", lambda: ssm.conv1d_bwd(x, w, b, dy, initial_state=init, dfinal_state=dF,
                                                  activation="silu", dx=dx, dinitial_state=dS,
                                                  dweight=dw, dbias=dbias, workspace=ws), 10)
    rep("conv1d_bwd", f"B{s.B} L{s.L} C{s.C} K{s.K} bf16 SiLU: dx, dS, dw, dbias", ms, s.B * s.L,
        3 * s.B * s.L * s.C * 2 + 3 * s.B * s.C * (s.K - 1) * 2 + 2 * s.C * (s.K + 1) * 4)
    del x, dy, dx, ws

    # initial-state gradient at the 1.3B shape: (a) the layer's dt / A, where the decay product
    # underflows within a few hundred tokens and the kernel stops there; (b) slow decays that
    # keep every token in play (a full pass over dy and C)
    Cm = torch.randn(s.B, s.L, s.G, s.N, generator=g, device=dev).to(torch.bfloat16)
    dyh = torch.randn(s.B, s.L, s.H, s.P, generator=g, device=dev).to(torch.bfloat16)
    dFh = torch.randn(s.B, s.H, s.P, s.N, generator=g, device=dev)
    dh0 = torch.empty_like(dFh)
    for label, dts, As in (("layer dt / A (stops where the decay underflows)", dt, A),
                           ("dt 0.01, A -0.05 (every token)", torch.full_like(dt, 0.01),
                            torch.full_like(A, -0.05))):
        ms = timed("scan_bwd", lambda: ssm.scan_bwd_initial_state(dts, As, Cm, dyh, dfinal_state=dFh,
                                                                  out=dh0), 10)
        # tokens a (b, h) block must read: up to the chunk where 2^(cum log2 e) underflows in fp32
        cum = torch.cumsum(dts.double() * As.double(), dim=1) * (1.0 / math.log(2.0))
        under = (cum < -150.0)
        first = torch.where(under.any(dim=1), under.float().argmax(dim=1), torch.full_like(under[:, 0], s.L, dtype=torch.long))
        toks = float(torch.clamp((first // 64 + 1) * 64, max=s.L).sum())
        nb = toks * (s.P * 2 + s.N * 2 + 4) + 2 * s.B * s.H * s.P * s.N * 4
        rep("scan_bwd_initial_state", f"B{s.B} L{s.L} H{s.H}x{s.P} N{s.N} bf16, {label}; "
            f"{toks / (s.B * s.H):.0f} tokens read per (row, head)", ms, s.B * s.L, nb)
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def environment(torch):
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "rocm": rocm,
            "gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "cpu_model": cpu_model(),
            "cache_flush_bytes": 512 << 20}


def cpu_baseline(s, w, b, A, inp, cinit, sinit):
    import oracle
    t0 = time.perf_counter()
    oracle.conv_scan_fwd(inp["xBC"], w, b, cinit, inp["dt"], A, sinit, None, s.H, s.P, s.G, s.N)
    dt = time.perf_counter() - t0
    return {"value": s.B * s.L / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"one whole step (batch {s.B} x {s.L} tokens, all {s.H} heads), "
                      f"fp64 C oracle, {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-ops", action="store_true",
                    help="skip the bandwidth figures of the other entry points")
    ap.add_argument("--ops", default=None,
                    help="comma-separated subset of the other entry points to time (conv1d_fwd, "
                         "packed1p3b, layer370m, layer780m, layer780m_chained, decode, pooled, "
                         "init_state, vector_decay, conv1d_bwd, scan_bwd); default all")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times), the reference "
                         "the HBM traffic counters are scaled by")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU part); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    import ssm_sequence_models_amd as ssm
    import workloads

    cfg = workloads.CONFIGS["layer1p3b"]
    s = workloads.shape_of("layer1p3b")
    dev = torch.device("cuda:0")
    w, b, A = workloads.layer_params(s, cfg["seed"])
    pre = workloads.prefill_inputs(s, cfg["pre_seed"])
    inp = workloads.prefill_inputs(s, cfg["seed"])
    W, Bb, AA = w.to(dev), b.to(dev), A.to(dev)
    X, D = inp["xBC"].to(dev), inp["dt"].to(dev)
    ws = torch.empty(ssm.workspace_size(s.B, s.L, s.H, s.P, s.G, s.N), dtype=torch.uint8,
                     device=dev)
    log("bench: preceding call for the initial states")
    _, cinit, sinit = ssm.conv_scan_fwd(pre["xBC"].to(dev), W, Bb, pre["dt"].to(dev), AA, s.H,
                                        s.P, s.G, s.N, workspace=ws)
    y = torch.empty(s.B, s.L, s.H, s.P, dtype=torch.bfloat16, device=dev)
    cfin = torch.empty_like(cinit)
    sfin = torch.empty_like(sinit)

    def step():
        ssm.conv_scan_fwd(X, W, Bb, D, AA, s.H, s.P, s.G, s.N, conv_initial_state=cinit,
                          initial_state=sinit, conv_final_state=cfin, final_state=sfin, y=y,
                          workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done; timing {args.steps}")
    # the timed steps: library timing off, the cache flushed before each step (outside its
    # events), the whole loop bracketed by device synchronisation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = _time_steps(torch, step, args.steps)
    wall = time.perf_counter() - t0
    ms_per_step = sum(step_ms) / len(step_ms)
    step_ms = sorted(step_ms)
    # a separate instrumented pass for the main kernel's own duration (the library records
    # HIP events around its launch on the call's stream)
    ssm.timing_read()  # clear
    ssm.timing_enable(True)
    _time_steps(torch, step, args.steps)
    ssm.timing_enable(False)
    main_ms, launches = ssm.timing_read()
    assert launches == args.steps, (launches, args.steps)
    main_ms_avg = main_ms / launches
    tokens = s.B * s.L
    op_bytes, main_bytes = algorithmic_bytes(s)
    achieved = main_bytes / (main_ms_avg * 1e-3) / 1e9
    log(f"bench: {ms_per_step:.4f} ms/step, main kernel {main_ms_avg:.4f} ms")
    n_chunks = (s.L + 63) // 64
    mfma_flops = s.B * s.H * n_chunks * MFMA_PER_CHUNK_HEAD * FLOP_PER_MFMA
    copy_GBs, copy_detail = copy_bandwidth(torch, ssm)

    result = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": step_ms[len(step_ms) // 2],
        "ms_per_step_min": step_ms[0],
        "wall_ms_per_step_incl_cache_flush": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mamba2-1.3b-like layer prefill with state passing: fused causal "
                               "conv1d (width 4, 4352 x|B|C channels, SiLU) + selective scan",
                   "batch": s.B, "seq_len": s.L, "nheads": s.H, "headdim": s.P,
                   "dstate": s.N, "ngroups": s.G, "conv_width": s.K,
                   "initial_state": "final states of a preceding 8192-token call"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "ssd_main_kernel", "kernel_ms": main_ms_avg,
                     "algorithmic_bytes_per_launch": main_bytes,
                     "copy_GBs": copy_GBs, **copy_detail, "frac_of_copy": achieved / copy_GBs},
        "mfma": {"kernel": "ssd_main_kernel", "issued_flops_per_launch": mfma_flops,
                 "achieved_TFLOPs": mfma_flops / (main_ms_avg * 1e-3) / 1e12,
                 "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                 "frac": mfma_flops / (main_ms_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                 "note": "bf16 MFMA flops issued, the hi/lo split of fp32 operands included"},
        "op_roofline": {"algorithmic_bytes": op_bytes, "ms": ms_per_step,
                        "achieved_GBs": op_bytes / (ms_per_step * 1e-3) / 1e9,
                        "frac": op_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "cpu_baseline": None,
        "other_ops": None,
        "environment": environment(torch),
    }
    if not args.no_other_ops:
        log("bench: other entry points")
        result["other_ops"] = other_ops(torch, ssm, workloads, copy_GBs,
                                        args.ops.split(",") if args.ops else None)
    if not args.no_cpu_baseline:
        log("bench: fp64 oracle on the host (cpu baseline)")
        result["cpu_baseline"] = cpu_baseline(s, w, b, A, inp, cinit.cpu(), sinit.cpu())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
