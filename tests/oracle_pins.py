"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each ``check_*`` takes the oracle's ctypes library (so the same checks can be run against
deliberately broken copies of the oracle) and raises AssertionError on a mismatch.  None of
them re-types the oracle's own loop: they use the pages' worked examples, closed forms,
brute-force unrollings, library routines (torch fp64 conv1d / cumsum / silu / bf16 cast) and
invariants.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------------------
# causal conv1d with state
# ------------------------------------------------------------------------------------------

def check_conv_worked_example_k4(lib):
    """causal-conv1d ch. 7, extended-sequence section: K = 4, S = [a,b,c], x = [d]."""
    g = _golden("conv_state_k4.json")
    sym = g["symbols"]
    K = g["K"]
    S = np.array([[[sym[s] for s in g["S"]]]])           # [1, 1, 3]
    x = np.array([[[sym[s]] for s in g["x"]]])           # [1, 1, 1]
    w = np.array([[1.0, 10.0, 100.0, 1000.0]])           # distinct decimal digits per tap
    out, fin = oracle.conv1d_fwd(x, w, None, S, lib=lib)
    window = [sym[s] for s in g["window"]]
    expect_z = sum(w[0, k] * window[k] for k in range(K))
    assert out[0, 0, 0] == expect_z, (out, expect_z)
    expect_F = [sym[s] for s in g["F"]]
    assert fin[0, 0].tolist() == expect_F, fin
    wrong = [sym[s] if isinstance(s, str) else s for s in g["wrong_zero_padded_F"]]
    assert fin[0, 0].tolist() != wrong


def check_conv_single_token_k3(lib):
    """causal-conv1d ch. 7, single-token chunk example (forward): z and F = [b, c]."""
    g = _golden("conv_single_token_k3.json")
    sym = g["symbols"]
    S = np.array([[[sym["a"], sym["b"]]]])
    x = np.array([[[sym["c"]]]])
    w = np.array([g["w"]])
    out, fin = oracle.conv1d_fwd(x, w, np.array([g["beta"]]), S, lib=lib)
    assert out[0, 0, 0] == g["z"], out
    assert fin[0, 0].tolist() == [sym[s] for s in g["F"]], fin


def check_conv_matches_torch(lib):
    """General case against torch fp64 conv1d (cross-correlation, groups = C) over
    cat(S, x): the extended-sequence definition is exactly that library routine."""
    r = _rng(1)
    for (B, L, C, K) in [(2, 37, 5, 4), (1, 9, 3, 2), (3, 20, 4, 3), (1, 2, 6, 4)]:
        x = r.standard_normal((B, L, C))
        w = r.standard_normal((C, K))
        bias = r.standard_normal(C)
        S = r.standard_normal((B, C, K - 1))
        out, fin = oracle.conv1d_fwd(x, w, bias, S, lib=lib)
        u = torch.cat([torch.from_numpy(S), torch.from_numpy(x).transpose(1, 2)], dim=2)
        ref = torch.nn.functional.conv1d(u, torch.from_numpy(w)[:, None, :],
                                         torch.from_numpy(bias), groups=C)
        np.testing.assert_allclose(out, ref.transpose(1, 2).numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(fin, u[:, :, L:L + K - 1].numpy())
        # absent state means zeros
        out0, _ = oracle.conv1d_fwd(x, w, bias, None, lib=lib)
        u0 = torch.cat([torch.zeros(B, C, K - 1, dtype=torch.float64),
                        torch.from_numpy(x).transpose(1, 2)], dim=2)
        ref0 = torch.nn.functional.conv1d(u0, torch.from_numpy(w)[:, None, :],
                                          torch.from_numpy(bias), groups=C)
        np.testing.assert_allclose(out0, ref0.transpose(1, 2).numpy(), rtol=1e-12, atol=1e-12)


def check_conv_silu_matches_torch(lib):
    """phi = SiLU against torch fp64 silu (identity tap w = [0, .., 0, 1], no bias)."""
    r = _rng(2)
    x = r.standard_normal((2, 50, 3)) * 6.0
    w = np.zeros((3, 4))
    w[:, 3] = 1.0
    out, _ = oracle.conv1d_fwd(x, w, None, None, act="silu", lib=lib)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-300)


def check_conv_short_chunks_keep_state(lib):
    """L < K-1: F still holds entries of S (extended-sequence section)."""
    K = 4
    S = np.array([[[11.0, 12.0, 13.0]]])
    w = np.ones((1, K))
    for L in (0, 1, 2):
        x = np.arange(1, L + 1, dtype=np.float64).reshape(1, L, 1)
        _, fin = oracle.conv1d_fwd(x, w, None, S, lib=lib)
        u = [11.0, 12.0, 13.0] + list(range(1, L + 1))
        assert fin[0, 0].tolist() == u[L:L + K - 1], (L, fin)


def check_conv_chunk_continuation(lib):
    """Running chunk A then chunk B with S_B = F_A equals the full run (ch. 7, 'chunked
    training and truncated backprop'), for every split point, bit-exact in fp64."""
    r = _rng(3)
    B, L, C, K = 2, 11, 3, 4
    x = r.standard_normal((B, L, C))
    w = r.standard_normal((C, K))
    bias = r.standard_normal(C)
    S = r.standard_normal((B, C, K - 1))
    full, ffin = oracle.conv1d_fwd(x, w, bias, S, act="silu", lib=lib)
    for cut in range(0, L + 1):
        oa, fa = oracle.conv1d_fwd(x[:, :cut], w, bias, S, act="silu", lib=lib)
        ob, fb = oracle.conv1d_fwd(x[:, cut:], w, bias, fa, act="silu", lib=lib)
        np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), full)
        np.testing.assert_array_equal(fb, ffin)


def check_conv_seq_idx_segments(lib):
    """Packed sequences with distinct (monotone) ids equal separate runs: the first segment
    continues from S, later ones start from zero history (ch. 7, 'packed-sequence
    boundaries')."""
    r = _rng(4)
    B, L, C, K = 1, 23, 3, 4
    x = r.standard_normal((B, L, C))
    w = r.standard_normal((C, K))
    bias = r.standard_normal(C)
    S = r.standard_normal((B, C, K - 1))
    bounds = [0, 1, 7, 9, 23]       # segments of length 1, 6, 2, 14
    seq = np.zeros((B, L), dtype=np.int32)
    for i in range(len(bounds) - 1):
        seq[0, bounds[i]:bounds[i + 1]] = i
    out, fin = oracle.conv1d_fwd(x, w, bias, S, seq_idx=seq, act="silu", lib=lib)
    for i in range(len(bounds) - 1):
        a, b = bounds[i], bounds[i + 1]
        ref, _ = oracle.conv1d_fwd(x[:, a:b], w, bias, S if i == 0 else None, act="silu",
                                   lib=lib)
        np.testing.assert_array_equal(out[:, a:b], ref)
    # the final state is the unmasked raw tail
    np.testing.assert_array_equal(fin[0], x[0, L - (K - 1):].T)


def check_conv_seq_idx_reuse_caveat(lib):
    """ids A, B, A with a short B: identity equality does not see the reset, so the second
    A segment still reads the first A's tail (the page's stated caveat)."""
    K = 4
    x = np.array([[[1.0], [2.0], [3.0], [100.0], [5.0]]])     # ids 0 0 0 1 0
    seq = np.array([[0, 0, 0, 1, 0]], dtype=np.int32)
    w = np.array([[1.0, 10.0, 1000.0, 10000.0]])
    out, _ = oracle.conv1d_fwd(x, w, None, None, seq_idx=seq, lib=lib)
    # token 4 (id 0): window u[4..7] = x[1], x[2], x[3], x[4]; x[3] (id 1) masked
    assert out[0, 4, 0] == 1.0 * 2.0 + 10.0 * 3.0 + 10000.0 * 5.0, out[0, :, 0]
    # token 3 (id 1): only itself
    assert out[0, 3, 0] == 10000.0 * 100.0


# ------------------------------------------------------------------------------------------
# conv decode update
# ------------------------------------------------------------------------------------------

def check_ring_buffer_worked_example(lib):
    """ch. 7 circular mode: K = 3, S_len = 4, p = 5 -> history in slots 3 and 0, the new
    input goes to slot 1."""
    g = _golden("ring_buffer_k3.json")
    K, S_len, p = g["K"], g["state_len"], g["p"]
    pool = np.array([[[10.0, 20.0, 30.0, 40.0]]])            # slot s holds 10*(s+1)
    w = np.array([[1.0, 100.0, 10000.0]])                    # w0 oldest .. w2 current
    x = np.array([[[7.0]]])
    out, newpool = oracle.conv1d_update(x, pool, w, None, None, np.array([p], np.int32),
                                        lib=lib)
    older, newer = g["history_slots"]                        # logical 3 -> slot 3, 4 -> 0
    expect = w[0, 0] * pool[0, 0, older] + w[0, 1] * pool[0, 0, newer] + w[0, 2] * 7.0
    assert out[0, 0, 0] == expect, (out, expect)
    ws = g["write_slot"]
    after = pool[0, 0].copy()
    after[ws] = 7.0
    np.testing.assert_array_equal(newpool[0, 0], after)


def check_ring_wraps_backwards(lib):
    """Circular mode before K-1 tokens were written (p < K-1): history j sits in slot
    (p - j) mod S_len taken as a non-negative remainder (the page's slot rule; what such
    never-written slots hold is the caller's business)."""
    K, S_len, p = 4, 4, 1
    pool = np.array([[[10.0, 20.0, 30.0, 40.0]]])
    w = np.array([[1.0, 100.0, 10000.0, 0.0]])               # oldest .. newest history
    out, newpool = oracle.conv1d_update(np.array([[[5.0]]]), pool, w, None, None,
                                        np.array([p], np.int32), lib=lib)
    # j = 3, 2, 1 steps back -> slots (1-3) mod 4 = 2, (1-2) mod 4 = 3, (1-1) mod 4 = 0
    assert out[0, 0, 0] == 1.0 * 30.0 + 100.0 * 40.0 + 10000.0 * 10.0, out
    assert newpool[0, 0].tolist() == [10.0, 5.0, 30.0, 40.0]


def _write_history(pool_row, hist, state_len):
    """Place a logical history (positions 0 .. len-1) into a circular row."""
    for q, v in enumerate(hist):
        pool_row[q % state_len] = v


def check_update_equals_fwd(lib):
    """Decode update over [history, new tokens] equals conv1d_fwd with the last K-1
    history inputs as S, in circular and linear modes, for L_new in {1, 3, 4}; the pool then
    holds the raw inputs x (never y)."""
    r = _rng(5)
    C, K = 3, 4
    w = r.standard_normal((C, K))
    bias = r.standard_normal(C)
    for S_len in (3, 4, 6):
        for p in (3, 5, 9, 12):
            for L_new in (1, 3, 4):
                hist = r.standard_normal((C, p))
                x = r.standard_normal((1, C, L_new))
                pool = r.standard_normal((2, C, S_len))      # slot 1 is the request's
                for c in range(C):
                    _write_history(pool[1, c], hist[c], S_len)
                out, newpool = oracle.conv1d_update(x, pool, w, bias, np.array([1], np.int32),
                                                    np.array([p], np.int32), act="silu",
                                                    lib=lib)
                S = hist[:, p - (K - 1):][None]
                ref, _ = oracle.conv1d_fwd(x.transpose(0, 2, 1), w, bias, S, act="silu",
                                           lib=lib)
                np.testing.assert_array_equal(out, ref.transpose(0, 2, 1))
                expect_row = pool[1].copy()
                for c in range(C):
                    _write_history(expect_row[c], list(hist[c]) + list(x[0, c]), S_len)
                np.testing.assert_array_equal(newpool[1], expect_row)
                np.testing.assert_array_equal(newpool[0], pool[0])   # untouched slot
                # linear mode: the row holds the newest S_len inputs, oldest first
                lin = np.stack([np.concatenate([np.zeros(S_len), hist[c]])[-S_len:]
                                for c in range(C)])
                pool_l = pool.copy()
                pool_l[1] = lin
                out_l, newpool_l = oracle.conv1d_update(x, pool_l, w, bias,
                                                        np.array([1], np.int32), None,
                                                        act="silu", lib=lib)
                np.testing.assert_array_equal(out_l, out)
                for c in range(C):
                    seq = list(lin[c]) + list(x[0, c])
                    np.testing.assert_array_equal(newpool_l[1, c], seq[-S_len:])


def check_update_state_len_invariance(lib):
    """A linear cache longer than K-1 does not change the receptive field (ch. 7, 'the
    physical cache may exceed the minimal history')."""
    r = _rng(6)
    C, K = 4, 4
    w = r.standard_normal((C, K))
    x = r.standard_normal((2, C, 2))
    tail = r.standard_normal((2, C, K - 1))
    short = tail.copy()
    long_ = np.concatenate([r.standard_normal((2, C, 6)), tail], axis=2)   # K + 5 = 9
    o1, _ = oracle.conv1d_update(x, short, w, lib=lib)
    o2, _ = oracle.conv1d_update(x, long_, w, lib=lib)
    np.testing.assert_array_equal(o1, o2)


def check_update_indices_and_range(lib):
    """conv_state_indices maps rows to slots; out-of-range rows are skipped with zero
    outputs; untouched slots stay bit-identical; cache_seqlens is not advanced."""
    r = _rng(7)
    C, K, S_len, n_slots = 3, 4, 4, 6
    w = r.standard_normal((C, K))
    pool = r.standard_normal((n_slots, C, S_len))
    x = r.standard_normal((4, C, 2))
    idx = np.array([4, -1, 1, n_slots], np.int32)
    seqlens = np.array([7, 3, 0, 2], np.int32)
    seqlens_before = seqlens.copy()
    out, newpool = oracle.conv1d_update(x, pool, w, None, idx, seqlens, lib=lib)
    assert np.all(out[1] == 0) and np.all(out[3] == 0)
    np.testing.assert_array_equal(seqlens, seqlens_before)
    for s in (0, 2, 3, 5):
        np.testing.assert_array_equal(newpool[s], pool[s])
    # row 0 -> slot 4 behaves like a single request on slot 0 of a one-slot pool
    o0, p0 = oracle.conv1d_update(x[:1], pool[4:5], w, None, None, seqlens[:1], lib=lib)
    np.testing.assert_array_equal(out[0], o0[0])
    np.testing.assert_array_equal(newpool[4], p0[0])


# ------------------------------------------------------------------------------------------
# scan
# ------------------------------------------------------------------------------------------

def _scalar_ar1_inputs(n_chains_b, H, P, L, a, sigma0=None, seed=8):
    r = _rng(seed)
    x = r.standard_normal((n_chains_b, L, H, P))
    dt = np.ones((n_chains_b, L, H))
    A = np.full(H, math.log(a))
    ones = np.ones((n_chains_b, L, 1, 1))
    init = None
    if sigma0 is not None:
        init = r.standard_normal((n_chains_b, H, P, 1)) * sigma0
    return x, dt, A, ones, init


def check_scan_variance_closed_form(lib):
    """Sec. 2.4 teaching example: h_t = a h_{t-1} + x_t, h_{-1} = 0 has
    Var(h_t) = (1 - a^(2(t+1))) / (1 - a^2); at a = 0.99 the page prints ~47.4 % of the
    steady state after 32 tokens and near-steady after 512.  Monte Carlo over 262,144
    chains (dt = 1, A = ln a, B = C = 1, N = 1), within 4 standard errors."""
    g = _golden("variance_ar1.json")
    a = g["a"]
    vinf = 1.0 / (1.0 - a * a)

    def ratio(t):
        return (1.0 - a ** (2 * (t + 1))) / (1.0 - a * a) / vinf

    t32 = g["after_32_tokens_t_index"]
    assert round(ratio(t32), g["printed_digits"]) == g["after_32_tokens_ratio_printed"]
    assert ratio(g["after_512_tokens_t_index"]) > g["after_512_tokens_min_ratio"]
    # 64 x 64 x 64 = 262,144 chains over 32 tokens
    x, dt, A, ones, _ = _scalar_ar1_inputs(64, 64, 64, 32, a)
    y, fin = oracle.scan_fwd(x, dt, A, ones, ones, lib=lib)
    M = y.shape[0] * y.shape[2] * y.shape[3]
    se = math.sqrt(2.0 / M)
    for t in (0, 7, t32):
        est = y[:, t].var() / vinf
        assert abs(est / ratio(t) - 1.0) < 4 * se, (t, est, ratio(t))
    # the final state is h_{L-1}
    np.testing.assert_array_equal(fin[..., 0], y[:, -1])
    # near-steady after 512 tokens (65,536 chains), and a non-zero initial state
    # h_{-1} ~ N(0, s0^2) adds a^(2(t+1)) s0^2
    s0 = 3.0
    x, dt, A, ones, init = _scalar_ar1_inputs(16, 64, 64, 512, a, sigma0=s0, seed=9)
    y, _ = oracle.scan_fwd(x, dt, A, ones, ones, init_state=init, lib=lib)
    M = y.shape[0] * y.shape[2] * y.shape[3]
    se = math.sqrt(2.0 / M)
    for t in (0, 31, 511):
        expect = ratio(t) * vinf + a ** (2 * (t + 1)) * s0 * s0
        assert abs(y[:, t].var() / expect - 1.0) < 4 * se, (t, y[:, t].var(), expect)


def _bruteforce_eq4(x, dt, A, Bm, Cm, h0):
    """Sec. 2.5 Eq. (4), written out with explicit time-ordered products:
    y_t = C_t^T sum_{s<=t} (prod_{tau=s+1..t} a_tau) B_s dt_s x_s
          + C_t^T (prod_{tau=0..t} a_tau) h_{-1}."""
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    y = np.zeros((B, L, H, P))
    for b in range(B):
        for h in range(H):
            g = h * G // H
            a = [math.exp(dt[b, tau, h] * A[h]) for tau in range(L)]
            for t in range(L):
                for p in range(P):
                    tot = 0.0
                    for s in range(t + 1):
                        prod = 1.0
                        for tau in range(s + 1, t + 1):
                            prod *= a[tau]
                        cb = sum(Cm[b, t, g, n] * Bm[b, s, g, n] for n in range(N))
                        tot += prod * cb * dt[b, s, h] * x[b, s, h, p]
                    if h0 is not None:
                        prod = 1.0
                        for tau in range(0, t + 1):
                            prod *= a[tau]
                        tot += prod * sum(Cm[b, t, g, n] * h0[b, h, p, n] for n in range(N))
                    y[b, t, h, p] = tot
    return y


def _small_scan_inputs(seed, B=2, L=9, H=4, P=3, N=5, G=2):
    r = _rng(seed)
    x = r.standard_normal((B, L, H, P))
    dt = np.log1p(np.exp(r.standard_normal((B, L, H)) - 1.0))
    A = -np.exp(r.uniform(0.0, math.log(4.0), H))
    Bm = r.standard_normal((B, L, G, N))
    Cm = r.standard_normal((B, L, G, N))
    h0 = r.standard_normal((B, H, P, N))
    return x, dt, A, Bm, Cm, h0


def check_scan_bruteforce_eq4(lib):
    """The recurrence equals the explicit Eq. (4) unrolling (tiny shapes, G = 2 groups)."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(10)
    y, _ = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, lib=lib)
    ref = _bruteforce_eq4(x, dt, A, Bm, Cm, h0)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def check_scan_initial_state_term(lib):
    """With x = 0 only the initial-state term of Eq. (4) remains:
    y_t = C_t^T (prod_{tau<=t} a_tau) h_{-1}; the final state is (prod a) h_{-1}."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(11, B=2, L=6, H=3, P=2, N=4, G=1)
    x[:] = 0.0
    y, fin = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, lib=lib)
    B, L, H, P = x.shape
    for b in range(B):
        for h in range(H):
            prod = 1.0
            for t in range(L):
                prod *= math.exp(dt[b, t, h] * A[h])
                for p in range(P):
                    expect = prod * float(np.dot(Cm[b, t, 0], h0[b, h, p]))
                    assert abs(y[b, t, h, p] - expect) <= 1e-12 * (1 + abs(expect))
            np.testing.assert_allclose(fin[b, h], prod * h0[b, h], rtol=1e-12)


def check_scan_superposition(lib):
    """Affine in (x, h_{-1}): y(x, h0) = y(x, 0) + y(0, h0) (the split of Eq. (4))."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(12, B=2, L=15, H=4, P=3, N=6, G=1)
    y, f = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, lib=lib)
    y1, f1 = oracle.scan_fwd(x, dt, A, Bm, Cm, None, lib=lib)
    y2, f2 = oracle.scan_fwd(np.zeros_like(x), dt, A, Bm, Cm, h0, lib=lib)
    np.testing.assert_allclose(y, y1 + y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f, f1 + f2, rtol=1e-12, atol=1e-12)


def check_scan_special_cases(lib):
    """A = 0 (a = 1): the state is h_{-1} plus the running sum of dt x B (torch cumsum), and
    a perturbation of h_{-1} persists unchanged.  A -> -inf (a = 0): y_t = dt_t x_t C_t.B_t."""
    x, dt, _, Bm, Cm, h0 = _small_scan_inputs(13, B=2, L=12, H=3, P=2, N=4, G=1)
    A0 = np.zeros(3)
    y, fin = oracle.scan_fwd(x, dt, A0, Bm, Cm, h0, lib=lib)
    xt = torch.from_numpy(x)
    inc = torch.einsum("blh,blhp,bln->blhpn", torch.from_numpy(dt), xt,
                       torch.from_numpy(Bm[:, :, 0]))
    st = torch.cumsum(inc, dim=1) + torch.from_numpy(h0)[:, None]
    ref = torch.einsum("blhpn,bln->blhp", st, torch.from_numpy(Cm[:, :, 0])).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(fin, st[:, -1].numpy(), rtol=1e-12, atol=1e-12)
    delta = np.zeros_like(h0)
    delta[0, 1, 1, 2] = 0.5
    _, fin2 = oracle.scan_fwd(x, dt, A0, Bm, Cm, h0 + delta, lib=lib)
    np.testing.assert_allclose(fin2 - fin, delta, atol=1e-12)
    Aneg = np.full(3, -1e300)
    y, _ = oracle.scan_fwd(x, dt, Aneg, Bm, Cm, h0, lib=lib)
    cb = np.einsum("bln,bln->bl", Cm[:, :, 0], Bm[:, :, 0])
    ref = dt[..., None] * x * cb[:, :, None, None]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def check_scan_chunk_continuation(lib):
    """State passing: scan(A) then scan(B, h_{-1} = final_A) equals the full scan, for every
    split point, bit-exact in fp64 (Sec. 2.6 SP / TBTT)."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(14, B=2, L=10, H=2, P=3, N=4, G=1)
    full, ffin = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, lib=lib)
    for cut in range(0, 11):
        ya, fa = oracle.scan_fwd(x[:, :cut], dt[:, :cut], A, Bm[:, :cut], Cm[:, :cut], h0,
                                 lib=lib)
        yb, fb = oracle.scan_fwd(x[:, cut:], dt[:, cut:], A, Bm[:, cut:], Cm[:, cut:], fa,
                                 lib=lib)
        np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), full)
        np.testing.assert_array_equal(fb, ffin)


def check_scan_seq_idx_segments(lib):
    """Packed sequences: monotone ids equal separate runs, the first from h_{-1} and the
    rest from zero; the final state is the last segment's."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(15, B=1, L=17, H=2, P=2, N=3, G=1)
    bounds = [0, 5, 6, 12, 17]
    seq = np.zeros((1, 17), np.int32)
    for i in range(4):
        seq[0, bounds[i]:bounds[i + 1]] = i
    y, fin = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, seq_idx=seq, lib=lib)
    for i in range(4):
        a, b = bounds[i], bounds[i + 1]
        ref, rf = oracle.scan_fwd(x[:, a:b], dt[:, a:b], A, Bm[:, a:b], Cm[:, a:b],
                                  h0 if i == 0 else None, lib=lib)
        np.testing.assert_array_equal(y[:, a:b], ref)
    np.testing.assert_array_equal(fin, rf)


def check_step_equals_scan(lib):
    """Decode step == scan: one call over all tokens is bit-exact, token-by-token calls with
    fp64 pool storage are bit-exact too; slots are addressed through indices; an
    out-of-range slot is skipped (zero y, pool untouched)."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(16, B=2, L=7, H=4, P=3, N=5, G=2)
    y, fin = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, lib=lib)
    n_slots = 5
    pool = _rng(17).standard_normal((n_slots, 4, 3, 5))
    idx = np.array([3, 0], np.int32)
    pool[idx] = h0
    ys, newpool = oracle.step(x, dt, A, Bm, Cm, pool, idx, lib=lib)
    np.testing.assert_array_equal(ys, y)
    np.testing.assert_array_equal(newpool[idx], fin)
    for s in (1, 2, 4):
        np.testing.assert_array_equal(newpool[s], pool[s])
    cur = pool.copy()
    for t in range(7):
        yt, cur = oracle.step(x[:, t:t + 1], dt[:, t:t + 1], A, Bm[:, t:t + 1],
                              Cm[:, t:t + 1], cur, idx, lib=lib)
        np.testing.assert_array_equal(yt[:, 0], y[:, t])
    np.testing.assert_array_equal(cur[idx], fin)
    yo, po = oracle.step(x, dt, A, Bm, Cm, pool, np.array([-1, 5], np.int32), lib=lib)
    assert np.all(yo == 0)
    np.testing.assert_array_equal(po, pool)


# ------------------------------------------------------------------------------------------
# rounding
# ------------------------------------------------------------------------------------------

def check_round_bf16(lib):
    """Nearest-even bfloat16 rounding against torch's fp32 -> bf16 cast (for fp32-exact
    values), plus ties, subnormals and overflow."""
    r = _rng(18)
    v = np.concatenate([r.standard_normal(4000) * 10.0 ** r.integers(-30, 30, 4000),
                        r.standard_normal(200) * 1e-39])
    v32 = v.astype(np.float32)
    ours = np.array([lib.orc_round(float(t), 2) for t in v32.astype(np.float64)])
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    ties = {1.0 + 2.0 ** -8: 1.0, 1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,
            -(1.0 + 2.0 ** -8): -1.0, 2.0 ** -133 * 1.5: 2.0 ** -132}
    for k, e in ties.items():
        assert lib.orc_round(k, 2) == e, (k, lib.orc_round(k, 2), e)
    assert math.isinf(lib.orc_round(3.5e38, 2))
    assert lib.orc_round(1.0 + 2.0 ** -30, 1) == 1.0


# ------------------------------------------------------------------------------------------
# backward with state gradients
# ------------------------------------------------------------------------------------------

def check_conv_bwd_single_token_k3(lib):
    """causal-conv1d ch. 7, single-token chunk example (backward): dS = [w0 d, w1 d + q0],
    dx = [w2 d + q1]; dw = d [a, b, c], dbeta = d (identity phi, so delta = dy)."""
    g = _golden("conv_bwd_single_token_k3.json")
    sym = g["symbols"]
    S = np.array([[[sym["a"], sym["b"]]]])
    x = np.array([[[sym["c"]]]])
    w = np.array([g["w"]])
    dy = np.array([[[g["delta"]]]])
    q = np.array([[g["q"]]])
    dx, dS, dw, db = oracle.conv1d_bwd(x, w, np.array([g["beta"]]), S, None, dy, q, lib=lib)
    assert dS[0, 0].tolist() == g["dS"], dS
    assert dx[0, :, 0].tolist() == g["dx"], dx
    assert dw[0].tolist() == g["dw"], dw
    assert db.tolist() == [g["dbeta"]], db


def _conv_loss(x, w, b, S, seq, dy, q, act, lib):
    out, fin = oracle.conv1d_fwd(x, w, b, S, seq, act=act, lib=lib)
    return float((out * dy).sum() + (fin * q).sum())


def check_conv_bwd_finite_differences(lib):
    """Every gradient of the conv (dx, dS, dw, dbeta) against central differences of the
    oracle's own forward on L = sum dy * out + sum q * F, with SiLU, packed sequences and an
    initial state (the mathematics of the derivative, not the page's formula re-typed)."""
    r = _rng(31)
    B, L, C, K = 2, 9, 3, 4
    x = r.normal(size=(B, L, C))
    w = r.normal(size=(C, K))
    b = r.normal(size=(C,))
    S = r.normal(size=(B, C, K - 1))
    seq = np.array([[0, 0, 0, 1, 1, 1, 1, 2, 2], [5, 5, 5, 5, 5, 5, 5, 5, 5]], np.int32)
    dy = r.normal(size=(B, L, C))
    q = r.normal(size=(B, C, K - 1))
    for act in ("none", "silu"):
        dx, dS, dw, db = oracle.conv1d_bwd(x, w, b, S, seq, dy, q, act=act, lib=lib)
        eps = 1e-5
        for arr, grad in ((x, dx), (S, dS), (w, dw), (b, db)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                keep = arr[idx]
                arr[idx] = keep + eps
                lp = _conv_loss(x, w, b, S, seq, dy, q, act, lib)
                arr[idx] = keep - eps
                lm = _conv_loss(x, w, b, S, seq, dy, q, act, lib)
                arr[idx] = keep
                num[idx] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7)


def check_conv_bwd_chunking(lib):
    """Chunked training ([CC] 'chunked training and truncated back-propagation'): with
    S_B = F_A, passing dS_B back as dF_A reproduces the whole sequence's gradients, for every
    split point (dw and dbeta add over the chunks)."""
    r = _rng(32)
    B, L, C, K = 2, 11, 2, 4
    x = r.normal(size=(B, L, C))
    w = r.normal(size=(C, K))
    b = r.normal(size=(C,))
    S = r.normal(size=(B, C, K - 1))
    dy = r.normal(size=(B, L, C))
    q = r.normal(size=(B, C, K - 1))
    dx, dS, dw, db = oracle.conv1d_bwd(x, w, b, S, None, dy, q, act="silu", lib=lib)
    for cut in range(0, L + 1):
        _, FA = oracle.conv1d_fwd(x[:, :cut], w, b, S, act="silu", lib=lib)
        dxB, dSB, dwB, dbB = oracle.conv1d_bwd(x[:, cut:], w, b, FA, None, dy[:, cut:], q,
                                               act="silu", lib=lib)
        dxA, dSA, dwA, dbA = oracle.conv1d_bwd(x[:, :cut], w, b, S, None, dy[:, :cut], dSB,
                                               act="silu", lib=lib)
        np.testing.assert_allclose(np.concatenate([dxA, dxB], axis=1), dx, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dSA, dS, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dwA + dwB, dw, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dbA + dbB, db, rtol=1e-12, atol=1e-12)


def _scan_loss(x, dt, A, Bm, Cm, h0, seq, dy, dF, lib):
    y, fin = oracle.scan_fwd(x, dt, A, Bm, Cm, h0, seq_idx=seq, lib=lib)
    return float((y * dy).sum() + (fin * dF).sum())


def check_scan_bwd_h0_finite_differences(lib):
    """dh_{-1} against central differences of the oracle's forward scan on
    L = sum dy * y + sum dF * h_final (L is linear in h_{-1}, so the differences are exact
    up to rounding), with and without packed sequences (a reset cuts h_{-1} off)."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(33, B=2, L=9, H=4, P=3, N=5, G=2)
    r = _rng(34)
    dy = r.normal(size=x.shape)
    dF = r.normal(size=h0.shape)
    P = x.shape[3]
    for seq in (None, np.array([[0, 0, 0, 0, 1, 1, 1, 1, 1], [3] * 9], np.int32)):
        dh0 = oracle.scan_bwd_h0(dt, A, Cm, seq, dy, dF, P, lib=lib)
        num = np.zeros_like(h0)
        for idx in np.ndindex(h0.shape):
            keep = h0[idx]
            h0[idx] = keep + 0.5
            lp = _scan_loss(x, dt, A, Bm, Cm, h0, seq, dy, dF, lib)
            h0[idx] = keep - 0.5
            lm = _scan_loss(x, dt, A, Bm, Cm, h0, seq, dy, dF, lib)
            h0[idx] = keep
            num[idx] = lp - lm
        np.testing.assert_allclose(dh0, num, rtol=1e-9, atol=1e-9)


def check_scan_bwd_h0_chunking(lib):
    """State passing in the backward direction: the whole sequence's dh_{-1} equals chunk A's
    with dF_A = chunk B's dh_{-1} (itself taking the external dF), for every split point."""
    x, dt, A, Bm, Cm, h0 = _small_scan_inputs(35, B=2, L=10, H=2, P=3, N=4, G=1)
    r = _rng(36)
    dy = r.normal(size=x.shape)
    dF = r.normal(size=h0.shape)
    P = x.shape[3]
    full = oracle.scan_bwd_h0(dt, A, Cm, None, dy, dF, P, lib=lib)
    for cut in range(0, 11):
        dB = oracle.scan_bwd_h0(dt[:, cut:], A, Cm[:, cut:], None, dy[:, cut:], dF, P, lib=lib)
        dA = oracle.scan_bwd_h0(dt[:, :cut], A, Cm[:, :cut], None, dy[:, :cut], dB, P, lib=lib)
        np.testing.assert_allclose(dA, full, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------
# the prefill on the decode pools
# ------------------------------------------------------------------------------------------

def _pooled_layer(seed, B=2, L=11, H=2, P=3, N=4, G=1, K=4):
    r = _rng(seed)
    C = H * P + 2 * G * N
    xBC = r.normal(size=(B, L, C))
    w = r.uniform(-0.5, 0.5, size=(C, K))
    b = r.uniform(-0.5, 0.5, size=(C,))
    dt = np.log1p(np.exp(r.normal(size=(B, L, H)) - 2.0))
    A = -np.exp(r.uniform(0.0, np.log(16.0), size=(H,)))
    return xBC, w, b, dt, A, (H, P, G, N, K, C)


def check_pooled_prefill_chain_equals_whole(lib):
    """Continuing one request's history ([CC] ch. 7): pooled prefills of x[:L1] and then x[L1:]
    (ring position advanced by L1 between them, circular and linear layouts) give the whole
    prefill's outputs, SSM final state and raw-input history."""
    xBC, w, b, dt, A, (H, P, G, N, K, C) = _pooled_layer(41)
    B, L = xBC.shape[:2]
    y_whole, _, fin_whole = oracle.conv_scan_fwd(xBC, w, b, None, dt, A, None, None, H, P, G, N,
                                                 act="silu", out_dtype="f64", state_dtype="f64",
                                                 lib=lib)
    for S_len, circular in ((5, True), (K - 1, True), (6, False)):
        for L1 in (0, 1, 2, 7, L):
            cp = np.zeros((B, C, S_len))
            sp = np.zeros((B, H, P, N))
            seq0 = np.zeros(B, np.int32) if circular else None
            ya, cp, sp = oracle.conv_scan_fwd_pooled(xBC[:, :L1], w, b, dt[:, :L1], A, cp, sp, None,
                                                     seq0, None, H, P, G, N, out_dtype="f64",
                                                     state_dtype="f64", lib=lib)
            seq1 = np.full(B, L1, np.int32) if circular else None
            yb, cp, sp = oracle.conv_scan_fwd_pooled(xBC[:, L1:], w, b, dt[:, L1:], A, cp, sp, None,
                                                     seq1, None, H, P, G, N, out_dtype="f64",
                                                     state_dtype="f64", lib=lib)
            np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y_whole, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(sp, fin_whole, rtol=1e-12, atol=1e-12)
            for j in range(1, min(S_len, L) + 1):   # the last inputs sit where the ring says
                slot = (L - j) % S_len if circular else S_len - j
                np.testing.assert_array_equal(cp[:, :, slot], xBC[:, L - j, :])


def check_pooled_prefill_then_decode(lib):
    """Prefill into the pools, then decode the rest one token at a time with the oracle's own
    conv1d_update (circular, ring position advanced by the caller) and step on the same pools:
    the outputs equal the whole prefill's (the pool layout is the decode path's)."""
    xBC, w, b, dt, A, (H, P, G, N, K, C) = _pooled_layer(42, B=2, L=9)
    B, L = xBC.shape[:2]
    S_len, L1 = 5, 4
    idx = np.array([2, 0], np.int32)                   # rows on slots 2 and 0 of 3
    y_whole, _, _ = oracle.conv_scan_fwd(xBC, w, b, None, dt, A, None, None, H, P, G, N,
                                         act="silu", out_dtype="f64", state_dtype="f64", lib=lib)
    cp = np.zeros((3, C, S_len))
    sp = np.zeros((3, H, P, N))
    ya, cp, sp = oracle.conv_scan_fwd_pooled(xBC[:, :L1], w, b, dt[:, :L1], A, cp, sp, idx,
                                             np.zeros(B, np.int32), None, H, P, G, N,
                                             out_dtype="f64", state_dtype="f64", lib=lib)
    np.testing.assert_allclose(ya, y_whole[:, :L1], rtol=1e-12, atol=1e-12)
    for t in range(L1, L):
        out, cp = oracle.conv1d_update(xBC[:, t, :, None], cp, w, b, idx,
                                       np.full(B, t, np.int32), act="silu", lib=lib)
        o = out[:, :, 0]
        xs = o[:, :H * P].reshape(B, 1, H, P)
        Bs = o[:, H * P:H * P + G * N].reshape(B, 1, G, N)
        Cs = o[:, H * P + G * N:].reshape(B, 1, G, N)
        yt, sp = oracle.step(xs, dt[:, t:t + 1], A, Bs, Cs, sp, idx, lib=lib)
        np.testing.assert_allclose(yt[:, 0], y_whole[:, t], rtol=1e-12, atol=1e-12)


def check_pooled_prefill_ring_example(lib):
    """ch. 7 circular mode, K = 3, S_len = 4, p = 5: a one-token prefill reads its history
    from slots 3 and 0 and writes the new input to slot 1; another row's slot, an
    out-of-range row (zero states, nothing stored)."""
    g = _golden("ring_buffer_k3.json")
    K, S_len, p = g["K"], g["state_len"], g["p"]
    H, P, G, N = 1, 1, 1, 1
    C = H * P + 2 * G * N
    cp = np.zeros((2, C, S_len))
    cp[1, 0] = [10.0, 20.0, 30.0, 40.0]                 # slot 1, x channel: 10 (s + 1)
    sp = np.zeros((2, H, P, N))
    w = np.zeros((C, K))
    w[0] = [1.0, 100.0, 10000.0]                          # w0 oldest .. w2 current
    w[1, K - 1] = w[2, K - 1] = 1.0                       # B_t = C_t = their current input
    xBC = np.zeros((2, 1, C))
    xBC[:, 0, 0] = 7.0
    xBC[:, 0, 1] = xBC[:, 0, 2] = 1.0
    dt = np.ones((2, 1, H))
    A = np.array([-1.0])
    idx = np.array([1, 5], np.int32)                      # row 1: slot 5 of 2, out of range
    y, cp2, sp2 = oracle.conv_scan_fwd_pooled(xBC, w, None, dt, A, cp, sp, idx,
                                              np.array([p, p], np.int32), None, H, P, G, N,
                                              act="none", out_dtype="f64", state_dtype="f64",
                                              lib=lib)
    # y_0 = C (dt x B) = the conv output of the x channel over the ring's history
    older, newer = g["history_slots"]
    expect_z = w[0, 0] * cp[1, 0, older] + w[0, 1] * cp[1, 0, newer] + w[0, 2] * 7.0
    assert y[0, 0, 0, 0] == expect_z, (y, expect_z)
    after = cp[1, 0].copy()
    after[g["write_slot"]] = 7.0
    np.testing.assert_array_equal(cp2[1, 0], after)
    np.testing.assert_array_equal(cp2[0], cp[0])          # slot 0 untouched
    np.testing.assert_array_equal(sp2[0], sp[0])
    # the out-of-range row ran from zero states: its y is the plain prefill's
    y0, _, _ = oracle.conv_scan_fwd(xBC[1:], w, None, None, dt[1:], A, None, None, H, P, G, N,
                                    act="none", out_dtype="f64", state_dtype="f64", lib=lib)
    np.testing.assert_array_equal(y[1:], y0)


# ------------------------------------------------------------------------------------------
# initial-state distributions for training (reading notes Sec. 2.6)
# ------------------------------------------------------------------------------------------

def check_philox_matches_numpy(lib):
    """Philox4x64-10 against numpy's implementation of the same published generator
    (numpy.random.Philox): numpy advances its 256-bit counter before each block, so its
    stream from counter c is the blocks of c + 1, c + 2, ..."""
    for key, ctr in (([0, 0], [0, 0, 0, 0]), ([5, 7], [0, 0, 0, 0]),
                     ([2**64 - 1, 12345], [41, 9, 0, 0]), ([0x243F6A8885A308D3, 1], [7, 0, 3, 2**63])):
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                              counter=np.array(ctr, dtype=np.uint64))
        raw = [int(v) for v in bg.random_raw(12)]
        for i in range(3):
            c = list(ctr)
            c[0] += i + 1
            got = oracle.philox4x64_10(c, key, lib=lib)
            assert got == raw[4 * i:4 * i + 4], (key, ctr, i, [hex(v) for v in got])


def check_box_muller_closed_form(lib):
    """r = sqrt(-2 ln u1), angle 2 pi u2: u1 = e^(-1/2) gives r = 1, so u2 = 0, 1/4, 1/2, 3/4
    give the points (1, 0), (0, 1), (-1, 0), (0, -1); u1 = 1 gives the origin."""
    u1 = math.exp(-0.5)
    for u2, (c, s_) in ((0.0, (1.0, 0.0)), (0.25, (0.0, 1.0)), (0.5, (-1.0, 0.0)),
                        (0.75, (0.0, -1.0))):
        z0, z1 = oracle.box_muller(u1, u2, lib=lib)
        assert abs(z0 - c) < 1e-12 and abs(z1 - s_) < 1e-12, (u2, z0, z1)
    z0, z1 = oracle.box_muller(1.0, 0.3, lib=lib)
    assert z0 == 0.0 and z1 == 0.0
    z0, z1 = oracle.box_muller(math.exp(-2.0), 0.125, lib=lib)  # r = 2 at 45 degrees
    assert abs(z0 - math.sqrt(2.0)) < 1e-12 and abs(z1 - math.sqrt(2.0)) < 1e-12


def check_random_noise_is_normal(lib):
    """Random Noise: every element an independent N(0, sigma^2) draw -- the sample mean and
    variance within their sampling error, a Kolmogorov-Smirnov test against scipy's normal
    CDF, no correlation between neighbouring elements (the two branches of one pair, and the
    pairs of one block), a fresh stream for another offset and the same values for the same
    seed and offset."""
    from scipy import stats
    sigma, shape = 2.5, (4, 8, 64, 128)
    z = oracle.initial_state_noise(shape, sigma=sigma, seed=1234, offset=7, out_dtype="f64",
                                   lib=lib).ravel()
    n = z.size
    assert abs(z.mean()) < 5 * sigma / math.sqrt(n), z.mean()
    assert abs(z.var() / sigma**2 - 1.0) < 5 * math.sqrt(2.0 / n), z.var()
    assert stats.kstest(z / sigma, "norm").pvalue > 1e-4
    for lag in (1, 2, 3, 4):
        r = np.corrcoef(z[:-lag], z[lag:])[0, 1]
        assert abs(r) < 5 / math.sqrt(n), (lag, r)
    z2 = oracle.initial_state_noise(shape, sigma=sigma, seed=1234, offset=8, out_dtype="f64",
                                    lib=lib).ravel()
    assert abs(np.corrcoef(z, z2)[0, 1]) < 5 / math.sqrt(n)
    z3 = oracle.initial_state_noise(shape, sigma=sigma, seed=1234, offset=7, out_dtype="f64",
                                    lib=lib).ravel()
    assert np.array_equal(z, z3)


def check_fitted_noise_per_head(lib):
    """Fitted Noise: head h's elements are N(mean[h], var[h]) draws (per-head sample mean and
    variance within their sampling error)."""
    B, H, P, N = 4, 6, 32, 64
    mean = np.array([0.0, 1.5, -3.0, 0.25, 10.0, -0.5])
    var = np.array([1.0, 0.01, 4.0, 2.5, 0.5, 9.0])
    z = oracle.initial_state_noise((B, H, P, N), mean=mean, var=var, seed=99, offset=3,
                                   out_dtype="f64", lib=lib)
    n = B * P * N
    for h in range(H):
        v = z[:, h].ravel()
        sd = math.sqrt(var[h])
        assert abs(v.mean() - mean[h]) < 5 * sd / math.sqrt(n), (h, v.mean())
        assert abs(v.var() / var[h] - 1.0) < 5 * math.sqrt(2.0 / n), (h, v.var())


def check_state_stats_update(lib):
    """Fitted Noise statistics, Eqs. (5)-(6) with beta = 0.1: the new batch's statistics carry
    weight 0.9 (the page stresses this).  Mean and Variance per head over rows, channels and
    state dimension against numpy's mean / var (population); repeated updates with one final
    state from zero statistics follow m (1 - 0.1^k); a constant state has variance 0; a large
    common offset does not disturb the variance."""
    rng = _rng(61)
    B, H, P, N = 3, 4, 8, 16
    fin = rng.normal(size=(B, H, P, N)) * np.array([1.0, 0.1, 3.0, 0.5])[None, :, None, None] \
        + np.array([0.0, 2.0, -1.0, 1e4])[None, :, None, None]
    m0, v0 = rng.normal(size=H), rng.uniform(0.1, 2.0, size=H)
    m, v = oracle.state_stats_update(fin, m0, v0, beta=0.1, out_dtype="f64", lib=lib)
    ref_m = fin.mean(axis=(0, 2, 3))
    ref_v = fin.var(axis=(0, 2, 3))
    np.testing.assert_allclose(m, 0.9 * ref_m + 0.1 * m0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v, 0.9 * ref_v + 0.1 * v0, rtol=1e-9, atol=1e-12)
    m, v = np.zeros(H), np.zeros(H)
    for k in range(1, 6):
        m, v = oracle.state_stats_update(fin, m, v, beta=0.1, out_dtype="f64", lib=lib)
        np.testing.assert_allclose(m, ref_m * (1 - 0.1**k), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(v, ref_v * (1 - 0.1**k), rtol=1e-9, atol=1e-12)
    const = np.full((2, H, P, N), 3.25)
    m, v = oracle.state_stats_update(const, np.zeros(H), np.zeros(H), beta=0.1, out_dtype="f64",
                                     lib=lib)
    assert np.all(v == 0.0) and np.allclose(m, 0.9 * 3.25, rtol=1e-15)


def check_state_reset(lib):
    """State Passing's reset: p = 0 copies every row, p = 1 zeroes every row; at p = 0.1 the
    zeroed fraction over 200000 rows lies within five binomial standard deviations, zeroed
    rows are all zero and the others unchanged; the decisions depend on the row only (the
    same for a conv-state tensor and an SSM-state tensor with the same seed and offset)."""
    rng = _rng(62)
    st = rng.normal(size=(64, 3, 5))
    d0, m0 = oracle.state_reset(st, p=0.0, seed=5, offset=1, lib=lib)
    assert m0.sum() == 0 and np.array_equal(d0, st)
    d1, m1 = oracle.state_reset(st, p=1.0, seed=5, offset=1, lib=lib)
    assert m1.sum() == 64 and not d1.any()
    R = 200000
    big = rng.normal(size=(R, 2)) + 1.0
    d, m = oracle.state_reset(big, p=0.1, seed=11, offset=4, lib=lib)
    frac = m.mean()
    assert abs(frac - 0.1) < 5 * math.sqrt(0.1 * 0.9 / R), frac
    z = m.astype(bool)
    assert not d[z].any() and np.array_equal(d[~z], big[~z])
    _, m_other = oracle.state_reset(rng.normal(size=(R, 7)), p=0.1, seed=11, offset=4, lib=lib)
    assert np.array_equal(m, m_other)
    _, m_next = oracle.state_reset(big, p=0.1, seed=11, offset=5, lib=lib)
    agree = (m == m_next).mean()
    assert abs(agree - 0.82) < 0.01, agree  # independent draws agree with probability 0.82


# ------------------------------------------------------------------------------------------
# the scan with a diagonal (per-state-dimension) transition (reading notes Sec. 2.1, 2.5)
# ------------------------------------------------------------------------------------------

def _vdecay_inputs(seed, B=2, L=9, H=4, P=3, N=5, G=2):
    rng = _rng(seed)
    x = rng.normal(size=(B, L, H, P))
    dt = rng.uniform(0.05, 0.6, size=(B, L, H))
    Bm = rng.normal(size=(B, L, G, N))
    Cm = rng.normal(size=(B, L, G, N))
    gate = -rng.uniform(0.01, 1.5, size=(B, L, H, N))
    h0 = rng.normal(size=(B, H, P, N))
    return x, dt, Bm, Cm, gate, h0


def check_vdecay_bruteforce_eq4(lib):
    """Eq. (4) with diagonal transitions, written as explicit per-dimension products: h_t[p, n]
    = sum_s (prod_{s<tau<=t} a_tau[n]) u_s x_s[p] B_s[n] + (prod_{tau<=t} a_tau[n]) h_{-1}[p, n],
    y_t = C_t . h_t (G = 2 groups)."""
    x, dt, Bm, Cm, gate, h0 = _vdecay_inputs(71)
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    y, fin = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, init_state=h0, lib=lib)
    a = np.exp(gate)
    ref_y = np.zeros_like(y)
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            for t in range(L):
                st = np.prod(a[b, :t + 1, h, :], axis=0)[None, :] * h0[b, h]
                for s_ in range(t + 1):
                    prod = np.prod(a[b, s_ + 1:t + 1, h, :], axis=0)
                    st = st + prod[None, :] * dt[b, s_, h] * np.outer(x[b, s_, h], Bm[b, s_, g])
                ref_y[b, t, h] = st @ Cm[b, t, g]
                if t == L - 1:
                    np.testing.assert_allclose(fin[b, h], st, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, ref_y, rtol=1e-12, atol=1e-12)


def check_vdecay_uniform_gate_is_scalar_scan(lib):
    """A gate equal in every state dimension, log a_t[n] = dt_t A_h, is the scalar-decay scan."""
    x, dt, Bm, Cm, _, h0 = _vdecay_inputs(72)
    H, N = x.shape[2], Bm.shape[3]
    A = -_rng(73).uniform(0.2, 3.0, size=H)
    gate = np.repeat((dt * A[None, None, :])[..., None], N, axis=3)
    y, fin = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, init_state=h0, lib=lib)
    ry, rfin = oracle.scan_fwd(x, dt, A, Bm, Cm, init_state=h0, lib=lib)
    np.testing.assert_allclose(y, ry, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(fin, rfin, rtol=1e-13, atol=1e-13)


def check_vdecay_rate_form_is_gate_form(lib):
    """The per-dimension rate form (a_t[n] = exp(dt_t A[h, n])) is the gate form with
    log a = dt A."""
    x, dt, Bm, Cm, _, h0 = _vdecay_inputs(74)
    H, N = x.shape[2], Bm.shape[3]
    Av = -_rng(75).uniform(0.1, 4.0, size=(H, N))
    y1, f1 = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, A_vec=Av, init_state=h0, lib=lib)
    y2, f2 = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=dt[..., None] * Av[None, None],
                                    init_state=h0, lib=lib)
    np.testing.assert_allclose(y1, y2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(f1, f2, rtol=1e-14, atol=1e-14)


def check_vdecay_constant_rates_lfilter(lib):
    """Time-constant decays a_n and no dt: every (p, n) is a first-order IIR filter, so the
    state is scipy.signal.lfilter([1], [1, -a_n], x_t[p] B_t[n]) started from a_n h_{-1}."""
    from scipy.signal import lfilter
    rng = _rng(76)
    B, L, H, P, N, G = 1, 40, 2, 3, 6, 1
    x = rng.normal(size=(B, L, H, P))
    Bm, Cm = rng.normal(size=(B, L, G, N)), rng.normal(size=(B, L, G, N))
    an = rng.uniform(0.3, 0.99, size=(H, N))
    gate = np.broadcast_to(np.log(an)[None, None], (B, L, H, N)).copy()
    h0 = rng.normal(size=(B, H, P, N))
    y, fin = oracle.scan_fwd_vdecay(x, None, Bm, Cm, log_decay=gate, init_state=h0, lib=lib)
    for h in range(H):
        st = np.zeros((L, P, N))
        for p in range(P):
            for n in range(N):
                st[:, p, n] = lfilter([1.0], [1.0, -an[h, n]], x[0, :, h, p] * Bm[0, :, 0, n],
                                      zi=[an[h, n] * h0[0, h, p, n]])[0]
        np.testing.assert_allclose(y[0, :, h], np.einsum("tpn,tn->tp", st, Cm[0, :, 0]),
                                   rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(fin[0, h], st[-1], rtol=1e-11, atol=1e-11)


def check_vdecay_chunks_and_resets(lib):
    """Chunk continuation (final state of A = initial state of B, every split point) and
    packed sequences (a row cut by seq_idx = separate rows, each from zero)."""
    x, dt, Bm, Cm, gate, h0 = _vdecay_inputs(77, B=1, L=12)
    y, fin = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, init_state=h0, lib=lib)
    for cut in range(1, 12):
        ya, fa = oracle.scan_fwd_vdecay(x[:, :cut], dt[:, :cut], Bm[:, :cut], Cm[:, :cut],
                                        log_decay=gate[:, :cut], init_state=h0, lib=lib)
        yb, fb = oracle.scan_fwd_vdecay(x[:, cut:], dt[:, cut:], Bm[:, cut:], Cm[:, cut:],
                                        log_decay=gate[:, cut:], init_state=fa, lib=lib)
        np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fb, fin, rtol=1e-12, atol=1e-12)
    seq = np.array([[0] * 5 + [1] * 7], dtype=np.int32)
    ys, _ = oracle.scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=gate, init_state=h0, seq_idx=seq,
                                   lib=lib)
    y2, _ = oracle.scan_fwd_vdecay(x[:, 5:], dt[:, 5:], Bm[:, 5:], Cm[:, 5:],
                                   log_decay=gate[:, 5:], lib=lib)
    np.testing.assert_allclose(ys[:, :5], y[:, :5], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ys[:, 5:], y2, rtol=1e-13, atol=1e-13)


ALL_CHECKS = [
    check_conv_worked_example_k4,
    check_conv_single_token_k3,
    check_conv_matches_torch,
    check_conv_silu_matches_torch,
    check_conv_short_chunks_keep_state,
    check_conv_chunk_continuation,
    check_conv_seq_idx_segments,
    check_conv_seq_idx_reuse_caveat,
    check_ring_buffer_worked_example,
    check_ring_wraps_backwards,
    check_update_equals_fwd,
    check_update_state_len_invariance,
    check_update_indices_and_range,
    check_scan_bruteforce_eq4,
    check_scan_initial_state_term,
    check_scan_superposition,
    check_scan_special_cases,
    check_scan_chunk_continuation,
    check_scan_seq_idx_segments,
    check_step_equals_scan,
    check_round_bf16,
    check_conv_bwd_single_token_k3,
    check_conv_bwd_finite_differences,
    check_conv_bwd_chunking,
    check_scan_bwd_h0_finite_differences,
    check_scan_bwd_h0_chunking,
    check_pooled_prefill_chain_equals_whole,
    check_pooled_prefill_then_decode,
    check_pooled_prefill_ring_example,
    check_philox_matches_numpy,
    check_box_muller_closed_form,
    check_random_noise_is_normal,
    check_fitted_noise_per_head,
    check_state_stats_update,
    check_state_reset,
    check_vdecay_bruteforce_eq4,
    check_vdecay_uniform_gate_is_scalar_scan,
    check_vdecay_rate_form_is_gate_form,
    check_vdecay_constant_rates_lfilter,
    check_vdecay_chunks_and_resets,
    # last: the Monte Carlo pin is the slowest, and the mutant test stops at the first failure
    check_scan_variance_closed_form,
]
