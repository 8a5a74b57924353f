"""fp64 CPU oracle for the SSM scan + causal conv1d path -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``ssm_sequence_models_amd``) never does, and the
two share no code: this package wraps ``ssm_oracle.c`` (plain C, double precision, written
straight from the definitions on the pages) through ctypes.

Every function takes CPU arrays (numpy or torch, any float dtype; bf16 and fp32 widen to
fp64 exactly), returns new numpy float64 arrays, and never modifies its inputs.  Outputs are
rounded once to the storage type named by ``out_dtype`` ("bf16", "f32" or "f64").

Definitions followed (page title and section):
  * conv1d_fwd      causal-conv1d tutorial ch. 7, "defining the state through the extended
                    sequence" and "packed-sequence boundaries";
  * conv1d_update   same chapter, "single-token update maths", "the physical cache may exceed
                    the minimal history", "state indices for continuous batching";
  * scan_fwd, step  length-generalization reading notes, Sec. 2.1 Eq. (1) and Sec. 2.5
                    Eq. (4), with the initial state in and the final state out (Sec. 2.6);
  * conv_scan_fwd   conv1d_fwd (phi applied, output rounded to the input dtype) followed by
                    the split into x | B | C channels and scan_fwd;
  * conv1d_bwd      causal-conv1d tutorial ch. 7, "backward with states, a unified derivation"
                    (du over the extended sequence, dS, dx, dw, dbeta) and "chunked training";
  * scan_bwd_h0     the gradient of the initial state through Eq. (4) of the reading notes
                    (Sec. 2.5), with the final state's gradient added (Sec. 2.6);
  * conv_scan_fwd_pooled  conv_scan_fwd with its states taken from and returned to the decode
                    pools (tutorial ch. 7: the physical cache, circular mode, state indices);
  * scan_fwd_vdecay the scan with a diagonal (per-state-dimension) transition, Eq. (1) with
                    A_t = diag(a_t), from log gates or from dt times a per-dimension rate;
  * state_stats_update, initial_state_noise, state_reset  the initial-state distributions of
                    the reading notes' Sec. 2.6 (Fitted Noise Eqs. (5)-(6), Random Noise, State
                    Passing's reset), drawing from Philox4x64-10 (Salmon et al., SC 2011).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssm_oracle.so")
_lock = threading.Lock()
_lib = None

ROUND = {"f64": 0, "f32": 1, "bf16": 2}
ACT = {"none": 0, "silu": 1}

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fp contraction)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def load_library(path: str):
    lib = ctypes.CDLL(path)
    lib.orc_round.restype = ctypes.c_double
    lib.orc_round.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_conv1d_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _ip, _dp, _i64, _i64, _i64, _i64,
                                   ctypes.c_int, ctypes.c_int]
    lib.orc_conv1d_update.argtypes = [_dp, _dp, _dp, _dp, _ip, _ip, _dp, _i64, _i64, _i64, _i64,
                                      _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.orc_scan_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip, _dp, _i64, _i64, _i64,
                                 _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.orc_step.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, _dp, _i64, _i64, _i64, _i64,
                             _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.orc_conv1d_bwd.argtypes = [_dp, _dp, _dp, _dp, _ip, _dp, _dp, _dp, _dp, _dp, _dp, _i64,
                                   _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int]
    lib.orc_scan_bwd_h0.argtypes = [_dp, _dp, _dp, _ip, _dp, _dp, _dp, _i64, _i64, _i64, _i64,
                                    _i64, _i64, ctypes.c_int]
    for f in ("orc_conv1d_fwd", "orc_conv1d_update", "orc_scan_fwd", "orc_step",
              "orc_conv1d_bwd", "orc_scan_bwd_h0"):
        getattr(lib, f).restype = ctypes.c_int
    lib.orc_scan_fwd_vdecay.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ip, _dp, _i64,
                                        _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    _u64 = ctypes.c_uint64
    _u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.orc_philox4x64_10.argtypes = [_u64p, _u64p, _u64p]
    lib.orc_box_muller.argtypes = [ctypes.c_double, ctypes.c_double, _dp]
    lib.orc_state_stats_update.argtypes = [_dp, _i64, _i64, _i64, _i64, ctypes.c_double, _dp,
                                           _dp, ctypes.c_int]
    lib.orc_initial_state_noise.argtypes = [_dp, _i64, _i64, _i64, _i64, _dp, _dp,
                                            ctypes.c_double, _u64, _u64, ctypes.c_int]
    lib.orc_state_reset.argtypes = [_dp, _dp, ctypes.POINTER(ctypes.c_uint8), _i64, _i64,
                                    ctypes.c_double, _u64, _u64]
    return lib


def _get():
    global _lib
    with _lock:
        if _lib is None:
            # ORACLE_LIB_PATH: a separately built copy (the sanitizer build of the oracle)
            path = os.environ.get("ORACLE_LIB_PATH")
            _lib = load_library(path if path else build())
        return _lib


def max_threads() -> int:
    return int(_get().orc_max_threads())


def _f64(a):
    """Widen a CPU array (numpy or torch, any float dtype) to a contiguous float64 array."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().cpu().to(torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a, t=_dp):
    return None if a is None else a.ctypes.data_as(t)


def round_to(a, out_dtype: str) -> np.ndarray:
    """Round every element once to ``out_dtype`` (nearest even)."""
    lib = _get()
    arr = _f64(a)
    flat = arr.reshape(-1)
    out = np.empty_like(flat)
    mode = ROUND[out_dtype]
    for i in range(flat.size):
        out[i] = lib.orc_round(float(flat[i]), mode)
    return out.reshape(arr.shape)


def conv1d_fwd(x, w, bias=None, init_state=None, seq_idx=None, act="none", out_dtype="f64",
               lib=None):
    """x [B, L, C]; w [C, K]; bias [C]; init_state [B, C, K-1]; seq_idx [B, L].

    Returns (out [B, L, C], final_state [B, C, K-1])."""
    lib = lib or _get()
    x, w, bias, init_state = _f64(x), _f64(w), _f64(bias), _f64(init_state)
    seq_idx = _i32(seq_idx)
    B, L, C = x.shape
    K = w.shape[1]
    out = np.zeros((B, L, C))
    fin = np.zeros((B, C, K - 1))
    lib.orc_conv1d_fwd(_p(x), _p(w), _p(bias), _p(init_state), _p(fin), _p(seq_idx, _ip),
                       _p(out), B, L, C, K, ACT[act], ROUND[out_dtype])
    return out, fin


def conv1d_update(x, pool, w, bias=None, indices=None, cache_seqlens=None, act="none",
                  out_dtype="f64", lib=None):
    """x [B, C, L_new]; pool [n_slots, C, state_len]; indices, cache_seqlens [B].

    Returns (out [B, C, L_new], new_pool)."""
    lib = lib or _get()
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    pool = _f64(pool).copy()
    indices, cache_seqlens = _i32(indices), _i32(cache_seqlens)
    B, C, L_new = x.shape
    n_slots, _, state_len = pool.shape
    K = w.shape[1]
    out = np.zeros((B, C, L_new))
    lib.orc_conv1d_update(_p(x), _p(pool), _p(w), _p(bias), _p(indices, _ip),
                          _p(cache_seqlens, _ip), _p(out), B, C, L_new, K, state_len, n_slots,
                          ACT[act], ROUND[out_dtype])
    return out, pool


def scan_fwd(x, dt, A, Bm, Cm, init_state=None, seq_idx=None, out_dtype="f64",
             state_dtype="f64", lib=None):
    """x [B, L, H, P]; dt [B, L, H]; A [H]; Bm, Cm [B, L, G, N]; init_state [B, H, P, N].

    Returns (y [B, L, H, P], final_state [B, H, P, N])."""
    lib = lib or _get()
    x, dt, A, Bm, Cm, init_state = (_f64(v) for v in (x, dt, A, Bm, Cm, init_state))
    seq_idx = _i32(seq_idx)
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    y = np.zeros((B, L, H, P))
    fin = np.zeros((B, H, P, N))
    lib.orc_scan_fwd(_p(x), _p(dt), _p(A), _p(Bm), _p(Cm), _p(init_state), _p(fin),
                     _p(seq_idx, _ip), _p(y), B, L, H, P, G, N, ROUND[out_dtype],
                     ROUND[state_dtype])
    return y, fin


def conv1d_bwd(x, w, bias, init_state, seq_idx, dy, dfinal, act="none", dx_dtype="f64",
               dstate_dtype="f64", dw_dtype="f64", lib=None):
    """Backward of conv1d_fwd with state gradients.  x, dy [B, L, C]; w [C, K]; bias [C];
    init_state, dfinal [B, C, K-1] (None = zero); seq_idx [B, L].

    Returns (dx [B, L, C], dinit [B, C, K-1], dw [C, K], dbias [C])."""
    lib = lib or _get()
    x, w, bias, init_state, dy, dfinal = (_f64(v) for v in (x, w, bias, init_state, dy, dfinal))
    seq_idx = _i32(seq_idx)
    B, L, C = x.shape
    K = w.shape[1]
    dx = np.zeros((B, L, C))
    dinit = np.zeros((B, C, K - 1))
    dw = np.zeros((C, K))
    dbias = np.zeros((C,))
    lib.orc_conv1d_bwd(_p(x), _p(w), _p(bias), _p(init_state), _p(seq_idx, _ip), _p(dy),
                       _p(dfinal), _p(dx), _p(dinit), _p(dw), _p(dbias), B, L, C, K, ACT[act],
                       ROUND[dx_dtype], ROUND[dstate_dtype], ROUND[dw_dtype])
    return dx, dinit, dw, dbias


def scan_bwd_h0(dt, A, Cm, seq_idx, dy, dfinal, P, out_dtype="f64", lib=None):
    """Gradient of the initial state: dt [B, L, H]; A [H]; Cm [B, L, G, N]; dy [B, L, H, P];
    dfinal [B, H, P, N] (None = zero); seq_idx [B, L].  Returns dh0 [B, H, P, N]."""
    lib = lib or _get()
    dt, A, Cm, dy, dfinal = (_f64(v) for v in (dt, A, Cm, dy, dfinal))
    seq_idx = _i32(seq_idx)
    B, L, H = dt.shape
    G, N = Cm.shape[2], Cm.shape[3]
    dh0 = np.zeros((B, H, P, N))
    lib.orc_scan_bwd_h0(_p(dt), _p(A), _p(Cm), _p(seq_idx, _ip), _p(dy), _p(dfinal), _p(dh0),
                        B, L, H, P, G, N, ROUND[out_dtype])
    return dh0


def conv_scan_fwd_pooled(xBC, conv_w, conv_bias, dt, A, conv_pool, ssm_pool, indices,
                         cache_seqlens, seq_idx, H, P, G, N, act="silu", out_dtype="f64",
                         state_dtype="f64", lib=None):
    """The fused prefill on decode pools (causal-conv1d tutorial ch. 7: the physical cache,
    the circular mode's slot p mod S_len and history (p - j) mod S_len, state indices; the
    closing distinction between another request's history, packed samples and continuing one
    request's history).  Row b takes slot s = indices[b] (b if None): its conv history is the
    pool's (circular: slots (p - j) mod S_len for j = K-1 .. 1, p = cache_seqlens[b]; linear:
    the row's last K-1), its SSM initial state pool[s]; after conv_scan_fwd, the row's new raw
    inputs go where conv1d_update would put them and pool[s] takes the final state.  Rows
    with an out-of-range slot run from zero states and store nothing.

    Returns (y [B, L, H, P], new conv pool, new ssm pool); the inputs are not modified."""
    lib = lib or _get()
    xBC = _f64(xBC)
    conv_pool = np.array(_f64(conv_pool), copy=True)
    ssm_pool = np.array(_f64(ssm_pool), copy=True)
    B, L, C = xBC.shape
    K = np.asarray(conv_w).shape[1]
    S_len = conv_pool.shape[2]
    n_slots = conv_pool.shape[0]
    idx = None if indices is None else np.asarray(indices).astype(np.int64)
    p_of = None if cache_seqlens is None else np.asarray(cache_seqlens).astype(np.int64)
    ys = []
    for b in range(B):
        s = b if idx is None else int(idx[b])
        ok = 0 <= s < n_slots
        hist = np.zeros((1, C, K - 1))
        h0 = np.zeros((1, H, P, N))
        if ok:
            for j in range(K - 1):  # oldest first: j steps ... 1 step back
                back = (K - 1) - j
                slot = (int(p_of[b]) - back) % S_len if p_of is not None else S_len - back
                hist[0, :, j] = conv_pool[s, :, slot]
            h0[0] = ssm_pool[s]
        seq = None if seq_idx is None else np.asarray(seq_idx)[b:b + 1]
        y, _, fin = conv_scan_fwd(xBC[b:b + 1], conv_w, conv_bias, hist, _f64(dt)[b:b + 1], A, h0,
                                  seq, H, P, G, N, act=act, out_dtype=out_dtype,
                                  state_dtype=state_dtype, lib=lib)
        ys.append(y)
        if ok:
            if p_of is not None:
                for t in range(L):
                    conv_pool[s, :, (int(p_of[b]) + t) % S_len] = xBC[b, t, :]
            else:
                row = np.concatenate([conv_pool[s], xBC[b].T], axis=1)
                conv_pool[s] = row[:, -S_len:]
            ssm_pool[s] = fin[0]
    return np.concatenate(ys, axis=0), conv_pool, ssm_pool


def step(x, dt, A, Bm, Cm, pool, indices=None, out_dtype="f64", state_dtype="f64", lib=None):
    """x [B, L_new, H, P]; dt [B, L_new, H]; Bm, Cm [B, L_new, G, N];
    pool [n_slots, H, P, N]; indices [B].

    Returns (y [B, L_new, H, P], new_pool)."""
    lib = lib or _get()
    x, dt, A, Bm, Cm = (_f64(v) for v in (x, dt, A, Bm, Cm))
    pool = _f64(pool).copy()
    indices = _i32(indices)
    B, L_new, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    n_slots = pool.shape[0]
    y = np.zeros((B, L_new, H, P))
    lib.orc_step(_p(x), _p(dt), _p(A), _p(Bm), _p(Cm), _p(pool), _p(indices, _ip), _p(y), B,
                 L_new, H, P, G, N, n_slots, ROUND[out_dtype], ROUND[state_dtype])
    return y, pool


def conv_scan_fwd(xBC, conv_w, conv_bias, conv_init, dt, A, ssm_init, seq_idx, H, P, G, N,
                  act="silu", out_dtype="bf16", state_dtype="f32", lib=None):
    """The fused prefill: conv1d_fwd over the x | B | C channels of xBC [B, L, H*P + 2*G*N]
    (phi applied, output rounded to the input dtype ``out_dtype``), split, then scan_fwd.

    Returns (y [B, L, H, P], conv_final [B, C, K-1], ssm_final [B, H, P, N])."""
    conv_out, conv_fin = conv1d_fwd(xBC, conv_w, conv_bias, conv_init, seq_idx, act=act,
                                    out_dtype=out_dtype, lib=lib)
    B, L, Ctot = conv_out.shape
    assert Ctot == H * P + 2 * G * N
    x = conv_out[:, :, :H * P].reshape(B, L, H, P)
    Bm = conv_out[:, :, H * P:H * P + G * N].reshape(B, L, G, N)
    Cm = conv_out[:, :, H * P + G * N:].reshape(B, L, G, N)
    y, ssm_fin = scan_fwd(x, dt, A, Bm, Cm, ssm_init, seq_idx, out_dtype=out_dtype,
                          state_dtype=state_dtype, lib=lib)
    return y, conv_fin, ssm_fin


def philox4x64_10(counter, key, lib=None):
    """Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2,
    3", SC 2011): four 64-bit counter words and two key words to four output words."""
    lib = lib or _get()
    c = (ctypes.c_uint64 * 4)(*[int(v) for v in counter])
    k = (ctypes.c_uint64 * 2)(*[int(v) for v in key])
    o = (ctypes.c_uint64 * 4)()
    lib.orc_philox4x64_10(c, k, o)
    return [int(v) for v in o]


def box_muller(u1, u2, lib=None):
    """(r cos 2 pi u2, r sin 2 pi u2), r = sqrt(-2 ln u1)."""
    lib = lib or _get()
    o = (ctypes.c_double * 2)()
    lib.orc_box_muller(float(u1), float(u2), o)
    return o[0], o[1]


def state_stats_update(final_state, mean, var, beta=0.1, out_dtype="f32", lib=None):
    """Fitted Noise statistics (reading notes Sec. 2.6, Eqs. (5)-(6)): per head, the batch's
    Mean and (population) Variance of final_state [B, H, P, N] over rows, channels and state
    dimension, blended as (1 - beta) new + beta old.  Returns new (mean [H], var [H])."""
    lib = lib or _get()
    fin = _f64(final_state)
    B, H, P, N = fin.shape
    m = np.array(_f64(mean), copy=True)
    v = np.array(_f64(var), copy=True)
    lib.orc_state_stats_update(_p(fin), B, H, P, N, float(beta), _p(m), _p(v), ROUND[out_dtype])
    return m, v


def initial_state_noise(shape, mean=None, var=None, sigma=1.0, seed=0, offset=0,
                        out_dtype="f32", lib=None):
    """Noise initial states (reading notes Sec. 2.6): Fitted Noise N(mean[h], var[h]) per head
    when mean / var are given, Random Noise N(0, sigma^2) otherwise; shape (B, H, P, N)."""
    lib = lib or _get()
    B, H, P, N = shape
    out = np.zeros((B, H, P, N))
    m = None if mean is None else _f64(mean)
    v = None if var is None else _f64(var)
    lib.orc_initial_state_noise(_p(out), B, H, P, N, _p(m), _p(v), float(sigma), int(seed),
                                int(offset), ROUND[out_dtype])
    return out


def state_reset(state, p=0.1, seed=0, offset=0, lib=None):
    """State Passing's occasional reset (reading notes Sec. 2.6): each row of state [B, ...]
    is zeroed with probability p.  Returns (new state, mask [B] uint8: 1 = zeroed)."""
    lib = lib or _get()
    src = _f64(state)
    B = src.shape[0]
    per = int(np.prod(src.shape[1:])) if src.ndim > 1 else 1
    dst = np.zeros_like(src)
    mask = np.zeros(B, dtype=np.uint8)
    lib.orc_state_reset(_p(src), _p(dst), mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), B,
                        per, float(p), int(seed), int(offset))
    return dst, mask


def scan_fwd_vdecay(x, dt, Bm, Cm, log_decay=None, A_vec=None, init_state=None, seq_idx=None,
                    out_dtype="f64", state_dtype="f64", lib=None):
    """The scan with a diagonal transition A_t = diag(a_t) (reading notes Sec. 2.1 Eq. (1),
    Sec. 2.5).  x [B, L, H, P]; dt [B, L, H] or None (= 1); Bm, Cm [B, L, G, N]; log a_t from
    log_decay [B, L, H, N], else dt * A_vec [H, N].

    Returns (y [B, L, H, P], final_state [B, H, P, N])."""
    lib = lib or _get()
    x, dt, Bm, Cm, ld, Av, init_state = (_f64(v) for v in (x, dt, Bm, Cm, log_decay, A_vec,
                                                             init_state))
    seq_idx = _i32(seq_idx)
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert (ld is None) != (Av is None), "give log_decay or A_vec"
    assert ld is not None or dt is not None, "A_vec needs dt"
    y = np.zeros((B, L, H, P))
    fin = np.zeros((B, H, P, N))
    lib.orc_scan_fwd_vdecay(_p(x), _p(dt), _p(ld), _p(Av), _p(Bm), _p(Cm), _p(init_state),
                            _p(fin), _p(seq_idx, _ip), _p(y), B, L, H, P, G, N, ROUND[out_dtype],
                            ROUND[state_dtype])
    return y, fin
