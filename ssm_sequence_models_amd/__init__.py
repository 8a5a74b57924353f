"""Thin Python binding of libssm_mi355x.so (the C ABI in include/ssm_mi355x.h).

Argument marshalling only: this module checks devices / dtypes / shapes of torch tensors,
allocates outputs and workspaces with torch (device memory and streams are PyTorch's
plumbing), and calls the C entry point of the same name on the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no fallback, and the
import fails loudly if the library has not been built.

Sources of the operations (page title and section): the length-generalization reading
notes on arXiv:2507.02782v2, Sec. 2.1 Eq. (1), Sec. 2.5 Eq. (4), Sec. 2.6 (scan with
initial / final state); the causal-conv1d tutorial ch. 7 (conv state S / F, decode update,
cache_seqlens, conv_state_indices, seq_idx, and the backward with state gradients).
"""
from __future__ import annotations

import ctypes
import os

import torch  # must precede the library load: it binds the process's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSM_LIB_PATH selects another build of the same sources (the host-sanitizer build of the
# argument checks runs the ABI tests against one)
LIB_PATH = os.environ.get("SSM_LIB_PATH") or os.path.join(_HERE, "libssm_mi355x.so")

SSM_F32, SSM_BF16 = 0, 1
ACT = {None: 0, "none": 0, "silu": 1}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "misaligned pointer",
           4: "workspace", 5: "HIP error"}


# Debug checks of caller contracts the kernels do not verify (they cost a device-to-host
# copy): with SSM_DEBUG_CHECKS=1 in the environment (or DEBUG_CHECKS = True), the calls that
# update state pools refuse two active rows on one slot (causal-conv1d ch. 7, state indices
# for continuous batching: a duplicate is a caller error, undefined in the kernels).
DEBUG_CHECKS = os.environ.get("SSM_DEBUG_CHECKS", "") == "1"


def check_distinct_slots(indices, n_slots: int, name: str = "indices") -> None:
    """Raise ValueError if two entries of `indices` inside [0, n_slots) are equal (rows
    outside that range are skipped by the kernels and may repeat)."""
    if indices is None:
        return
    v = indices.detach().to("cpu").to(torch.int64)
    v = v[(v >= 0) & (v < n_slots)]
    if v.numel() != torch.unique(v).numel():
        vals, counts = torch.unique(v, return_counts=True)
        raise ValueError(f"{name}: slot(s) {vals[counts > 1].tolist()} used by more than one "
                         "active row")


class SSMError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {detail}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python ssm_sequence_models_amd/build.py "
            "or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32p, fp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    ci = ctypes.c_int
    lib.ssm_abi_version.restype = ci
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_status_string.argtypes = [ci]
    lib.ssm_conv1d_fwd.argtypes = [vp, fp, fp, vp, vp, i32p, vp, i64, i64, i64, i64, ci, ci, vp]
    lib.ssm_conv1d_update.argtypes = [vp, vp, fp, fp, i32p, i32p, vp, i64, i64, i64, i64, i64,
                                      i64, ci, ci, vp]
    lib.ssm_scan_workspace_size.restype = ctypes.c_size_t
    lib.ssm_scan_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, ci]
    lib.ssm_scan_fwd.argtypes = [vp, fp, fp, vp, vp, fp, fp, i32p, vp, i64, i64, i64, i64, i64,
                                 i64, ci, vp, ctypes.c_size_t, vp]
    lib.ssm_conv_scan_fwd.argtypes = [vp, fp, fp, vp, vp, fp, fp, fp, fp, i32p, vp, i64, i64, i64,
                                      i64, i64, i64, i64, ci, ci, vp, ctypes.c_size_t, vp]
    lib.ssm_conv_scan_fwd_noalloc.argtypes = [vp, fp, fp, vp, vp, fp, fp, fp, fp, i32p, vp, i64,
                                              i64, i64, i64, i64, i64, i64, ci, ci, vp]
    lib.ssm_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.ssm_noalloc_scratch_bytes.argtypes = []
    lib.ssm_step.argtypes = [vp, i64, i64, i64, fp, fp, vp, i64, i64, i64, vp, i64, i64, i64, fp,
                             i32p, vp, i64, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.ssm_decode_step.argtypes = [vp, vp, fp, fp, i32p, i32p, fp, fp, fp, i32p, vp, vp, i64,
                                    i64, i64, i64, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    lib.ssm_conv1d_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssm_conv1d_bwd_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.ssm_conv1d_bwd.argtypes = [vp, fp, fp, vp, i32p, vp, vp, vp, vp, fp, fp, vp,
                                   ctypes.c_size_t, i64, i64, i64, i64, ci, ci, vp]
    lib.ssm_scan_bwd_initial_state.argtypes = [fp, fp, vp, vp, i32p, fp, fp, i64, i64, i64, i64,
                                               i64, i64, ci, vp]
    lib.ssm_conv_scan_fwd_pooled_workspace_size.restype = ctypes.c_size_t
    lib.ssm_conv_scan_fwd_pooled_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i64, ci]
    lib.ssm_conv_scan_fwd_pooled.argtypes = [vp, fp, fp, fp, fp, vp, fp, i32p, i32p, i32p, vp,
                                             i64, i64, i64, i64, i64, i64, i64, i64, i64, ci, ci,
                                             vp, ctypes.c_size_t, vp]
    lib.ssm_scan_fwd_vector_decay.argtypes = [vp, fp, fp, fp, vp, vp, fp, fp, i32p, vp, i64, i64,
                                              i64, i64, i64, i64, ci, vp]
    u64 = ctypes.c_uint64
    lib.ssm_state_stats_update.argtypes = [fp, i64, i64, i64, i64, ctypes.c_float, fp, fp, vp]
    lib.ssm_initial_state_noise.argtypes = [fp, i64, i64, i64, i64, fp, fp, ctypes.c_float, u64,
                                            u64, vp]
    lib.ssm_state_reset.argtypes = [vp, vp, vp, i64, i64, ctypes.c_double, u64, u64, vp]
    lib.ssm_stream_copy.argtypes = [vp, vp, i64, vp]
    lib.ssm_timing_enable.argtypes = [ci]
    lib.ssm_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    for f in ("ssm_conv1d_fwd", "ssm_conv1d_update", "ssm_scan_fwd", "ssm_conv_scan_fwd",
              "ssm_conv_scan_fwd_noalloc", "ssm_step", "ssm_decode_step", "ssm_conv1d_bwd", "ssm_scan_bwd_initial_state",
              "ssm_conv_scan_fwd_pooled", "ssm_state_stats_update", "ssm_scan_fwd_vector_decay",
              "ssm_initial_state_noise", "ssm_state_reset", "ssm_stream_copy",
              "ssm_timing_enable", "ssm_timing_read"):
        getattr(lib, f).restype = ci
    return lib


_lib = _load()


def abi_version() -> int:
    return int(_lib.ssm_abi_version())


def _check(fn: str, status: int):
    if status != 0:
        raise SSMError(fn, status, _lib.ssm_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    if t.dtype == torch.float32:
        return SSM_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None, contiguous=True):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate, dtype=torch.bfloat16) -> int:
    code = SSM_BF16 if dtype == torch.bfloat16 else SSM_F32
    return int(_lib.ssm_scan_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate,
                                            code))


def _workspace(ws, nbytes, device):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace must hold {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


def conv1d_fwd(x, weight, bias=None, initial_state=None, seq_idx=None, activation=None,
               return_final_state=True, final_state=None, out=None):
    """x [B, L, C] (bf16 / fp32, channel-last); weight [C, K] fp32; bias [C] fp32;
    initial_state [B, C, K-1]; seq_idx [B, L] int32.  Returns (out, final_state)."""
    B, L, C = x.shape
    K = weight.shape[1]
    _need(x, "x")
    _need(weight, "weight", torch.float32, (C, K))
    _need(bias, "bias", torch.float32, (C,))
    _need(initial_state, "initial_state", x.dtype, (B, C, K - 1))
    _need(seq_idx, "seq_idx", torch.int32, (B, L))
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, (B, L, C))
    if final_state is None and return_final_state:
        final_state = torch.empty((B, C, K - 1), dtype=x.dtype, device=x.device)
    _need(final_state, "final_state", x.dtype, (B, C, K - 1))
    _check("ssm_conv1d_fwd", _lib.ssm_conv1d_fwd(
        _ptr(x), _ptr(weight), _ptr(bias), _ptr(initial_state), _ptr(final_state), _ptr(seq_idx),
        _ptr(out), B, L, C, K, _dtype_code(x), ACT[activation], _stream()))
    return out, final_state


def conv_scan_fwd_pooled(xBC, conv_weight, conv_bias, dt, A, conv_state, ssm_state, nheads,
                         headdim, ngroups, dstate, state_indices=None, cache_seqlens=None,
                         seq_idx=None, activation="silu", y=None, workspace=None):
    """The fused prefill on the decode pools: row b's initial conv history and SSM state come
    from slot state_indices[b] (ring position cache_seqlens[b], or the linear layout), and its
    new raw inputs and final state go back there.  conv_state [n_slots, C_conv, state_len]
    (xBC's dtype) and ssm_state [n_slots, H, P, N] fp32 update in place; cache_seqlens is not
    advanced.  Returns y [b, L, H, P]."""
    b, L, C_conv = xBC.shape
    K = conv_weight.shape[1]
    n_slots, _, state_len = conv_state.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    _need(xBC, "xBC")
    _need(conv_weight, "conv_weight", torch.float32, (C_conv, K))
    _need(conv_bias, "conv_bias", torch.float32, (C_conv,))
    _need(dt, "dt", torch.float32, (b, L, H))
    _need(A, "A", torch.float32, (H,))
    _need(conv_state, "conv_state", xBC.dtype, (n_slots, C_conv, state_len))
    _need(ssm_state, "ssm_state", torch.float32, (n_slots, H, P, N))
    _need(state_indices, "state_indices", torch.int32, (b,))
    if DEBUG_CHECKS:
        check_distinct_slots(state_indices, ssm_state.shape[0], "state_indices")
    _need(cache_seqlens, "cache_seqlens", torch.int32, (b,))
    _need(seq_idx, "seq_idx", torch.int32, (b, L))
    if y is None:
        y = torch.empty((b, L, H, P), dtype=xBC.dtype, device=xBC.device)
    _need(y, "y", xBC.dtype, (b, L, H, P))
    nbytes = int(_lib.ssm_conv_scan_fwd_pooled_workspace_size(b, L, H, P, G, N, K, _dtype_code(xBC)))
    if workspace is None:
        workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=xBC.device)
    off = (-workspace.data_ptr()) % 256
    if workspace.numel() - off < nbytes:
        raise ValueError(f"workspace must hold {nbytes} bytes past a 256-byte boundary")
    _check("ssm_conv_scan_fwd_pooled", _lib.ssm_conv_scan_fwd_pooled(
        _ptr(xBC), _ptr(conv_weight), _ptr(conv_bias), _ptr(dt), _ptr(A), _ptr(conv_state),
        _ptr(ssm_state), _ptr(state_indices), _ptr(cache_seqlens), _ptr(seq_idx), _ptr(y), b, L,
        H, P, G, N, K, state_len, n_slots, _dtype_code(xBC), ACT[activation],
        ctypes.c_void_p(workspace.data_ptr() + off), workspace.numel() - off, _stream()))
    return y


def conv_scan_fwd_pooled_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate, width,
                                        dtype=torch.bfloat16) -> int:
    code = SSM_BF16 if dtype == torch.bfloat16 else SSM_F32
    return int(_lib.ssm_conv_scan_fwd_pooled_workspace_size(batch, seqlen, nheads, headdim, ngroups,
                                                            dstate, width, code))


def scan_fwd_vector_decay(x, B, C, log_decay=None, A_vec=None, dt=None, initial_state=None,
                          seq_idx=None, return_final_state=True, final_state=None, y=None):
    """The scan with a diagonal transition, one decay per state dimension (length-
    generalization notes Sec. 2.1 Eq. (1) with A_t = diag(a_t), Sec. 2.5): log a_t[n] from
    log_decay [b, L, H, N] fp32, or dt * A_vec [H, N].  x [b, L, H, P]; B, C [b, L, G, N];
    dt [b, L, H] fp32 or None (= 1).  Returns (y [b, L, H, P], final_state or None)."""
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _need(x, "x")
    _need(B, "B", x.dtype, (bsz, L, G, N))
    _need(C, "C", x.dtype, (bsz, L, G, N))
    _need(log_decay, "log_decay", torch.float32, (bsz, L, H, N))
    _need(A_vec, "A_vec", torch.float32, (H, N))
    _need(dt, "dt", torch.float32, (bsz, L, H))
    _need(initial_state, "initial_state", torch.float32, (bsz, H, P, N))
    _need(seq_idx, "seq_idx", torch.int32, (bsz, L))
    if y is None:
        y = torch.empty((bsz, L, H, P), dtype=x.dtype, device=x.device)
    _need(y, "y", x.dtype, (bsz, L, H, P))
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=x.device)
    _need(final_state, "final_state", torch.float32, (bsz, H, P, N))
    _check("ssm_scan_fwd_vector_decay", _lib.ssm_scan_fwd_vector_decay(
        _ptr(x), _ptr(dt), _ptr(log_decay), _ptr(A_vec), _ptr(B), _ptr(C), _ptr(initial_state),
        _ptr(final_state), _ptr(seq_idx), _ptr(y), bsz, L, H, P, G, N, _dtype_code(x),
        _stream()))
    return y, final_state

def state_stats_update(final_state, mean, var, beta=0.1):
    """Fitted Noise statistics (length-generalization notes Sec. 2.6, Eqs. (5)-(6)): per head,
    mean <- (1 - beta) Mean(final_state) + beta mean, var likewise with the population
    variance, over batch rows, channels and state dimension.  final_state [b, H, P, N] fp32;
    mean, var [H] fp32, updated in place and returned."""
    b, H, P, N = final_state.shape
    _need(final_state, "final_state", torch.float32)
    _need(mean, "mean", torch.float32, (H,))
    _need(var, "var", torch.float32, (H,))
    _check("ssm_state_stats_update", _lib.ssm_state_stats_update(
        _ptr(final_state), b, H, P, N, float(beta), _ptr(mean), _ptr(var), _stream()))
    return mean, var


def initial_state_noise(batch, nheads, headdim, dstate, mean=None, var=None, sigma=1.0, seed=0,
                        offset=0, out=None, device="cuda"):
    """Noise initial states (Sec. 2.6): Fitted Noise N(mean[h], var[h]) per head when mean and
    var [H] are given, Random Noise N(0, sigma^2) otherwise, drawn from Philox4x64-10 with
    (seed, offset).  Returns out [batch, H, P, N] fp32."""
    shape = (batch, nheads, headdim, dstate)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=device)
    _need(out, "out", torch.float32, shape)
    _need(mean, "mean", torch.float32, (nheads,))
    _need(var, "var", torch.float32, (nheads,))
    _check("ssm_initial_state_noise", _lib.ssm_initial_state_noise(
        _ptr(out), batch, nheads, headdim, dstate, _ptr(mean), _ptr(var), float(sigma),
        int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), _stream()))
    return out


def state_reset(state, p=0.1, seed=0, offset=0, out=None, mask=None):
    """State Passing's occasional reset (Sec. 2.6): each row of state [b, ...] (any dtype) is
    zeroed with probability p, decided by (seed, offset, row) alone.  out may be state itself.
    Returns (out, mask [b] uint8, 1 = zeroed)."""
    b = state.shape[0]
    _need(state, "state")
    if out is None:
        out = torch.empty_like(state)
    _need(out, "out", state.dtype, tuple(state.shape))
    if mask is None:
        mask = torch.empty(b, dtype=torch.uint8, device=state.device)
    _need(mask, "mask", torch.uint8, (b,))
    row_bytes = state[0].numel() * state.element_size() if b > 0 else 0
    _check("ssm_state_reset", _lib.ssm_state_reset(
        _ptr(state), _ptr(out), _ptr(mask), b, row_bytes, float(p), int(seed) & (2**64 - 1),
        int(offset) & (2**64 - 1), _stream()))
    return out, mask

def conv1d_bwd(x, weight, bias, dout, initial_state=None, dfinal_state=None, seq_idx=None,
               activation=None, dx=None, dinitial_state=None, dweight=None, dbias=None,
               workspace=None):
    """Backward of conv1d_fwd with state gradients.  x, dout [B, L, C]; weight [C, K] fp32;
    bias [C] fp32 or None; initial_state, dfinal_state [B, C, K-1] (None = zero); seq_idx
    [B, L] int32.  Returns (dx [B, L, C], dinitial_state [B, C, K-1], dweight [C, K] fp32,
    dbias [C] fp32)."""
    B, L, C = x.shape
    K = weight.shape[1]
    _need(x, "x")
    _need(weight, "weight", torch.float32, (C, K))
    _need(bias, "bias", torch.float32, (C,))
    _need(dout, "dout", x.dtype, (B, L, C))
    _need(initial_state, "initial_state", x.dtype, (B, C, K - 1))
    _need(dfinal_state, "dfinal_state", x.dtype, (B, C, K - 1))
    _need(seq_idx, "seq_idx", torch.int32, (B, L))
    if dx is None:
        dx = torch.empty_like(x)
    if dinitial_state is None:
        dinitial_state = torch.empty((B, C, K - 1), dtype=x.dtype, device=x.device)
    if dweight is None:
        dweight = torch.empty((C, K), dtype=torch.float32, device=x.device)
    if dbias is None:
        dbias = torch.empty((C,), dtype=torch.float32, device=x.device)
    _need(dx, "dx", x.dtype, (B, L, C))
    _need(dinitial_state, "dinitial_state", x.dtype, (B, C, K - 1))
    _need(dweight, "dweight", torch.float32, (C, K))
    _need(dbias, "dbias", torch.float32, (C,))
    nbytes = int(_lib.ssm_conv1d_bwd_workspace_size(B, L, C, K))
    ws, wsb = _workspace(workspace, nbytes, x.device)
    _check("ssm_conv1d_bwd", _lib.ssm_conv1d_bwd(
        _ptr(x), _ptr(weight), _ptr(bias), _ptr(initial_state), _ptr(seq_idx), _ptr(dout),
        _ptr(dfinal_state), _ptr(dx), _ptr(dinitial_state), _ptr(dweight), _ptr(dbias),
        _ptr(ws), wsb, B, L, C, K, _dtype_code(x), ACT[activation], _stream()))
    return dx, dinitial_state, dweight, dbias


def conv1d_bwd_workspace_size(batch, seqlen, channels, width) -> int:
    return int(_lib.ssm_conv1d_bwd_workspace_size(batch, seqlen, channels, width))


def scan_bwd_initial_state(dt, A, C, dy, dfinal_state=None, seq_idx=None, out=None):
    """Gradient of the scan's initial state.  dt [b, L, H] fp32; A [H] fp32; C [b, L, G, N];
    dy [b, L, H, P] (C's dtype); dfinal_state [b, H, P, N] fp32 or None; seq_idx [b, L]
    int32.  Returns dinitial_state [b, H, P, N] fp32 (out may be dfinal_state itself)."""
    b, L, H, P = dy.shape
    G, N = C.shape[2], C.shape[3]
    _need(dt, "dt", torch.float32, (b, L, H))
    _need(A, "A", torch.float32, (H,))
    _need(C, "C", dy.dtype, (b, L, G, N))
    _need(dy, "dy")
    _need(dfinal_state, "dfinal_state", torch.float32, (b, H, P, N))
    _need(seq_idx, "seq_idx", torch.int32, (b, L))
    if out is None:
        out = torch.empty((b, H, P, N), dtype=torch.float32, device=dy.device)
    _need(out, "out", torch.float32, (b, H, P, N))
    _check("ssm_scan_bwd_initial_state", _lib.ssm_scan_bwd_initial_state(
        _ptr(dt), _ptr(A), _ptr(C), _ptr(dy), _ptr(seq_idx), _ptr(dfinal_state), _ptr(out),
        b, L, H, P, G, N, _dtype_code(dy), _stream()))
    return out


def conv1d_update(x, conv_state, weight, bias=None, conv_state_indices=None,
                  cache_seqlens=None, activation=None, out=None):
    """x [B, C, L_new]; conv_state [n_slots, C, state_len] (updated in place);
    conv_state_indices, cache_seqlens [B] int32 (cache_seqlens is not advanced).
    Returns out [B, C, L_new]."""
    B, C, L_new = x.shape
    n_slots, _, state_len = conv_state.shape
    K = weight.shape[1]
    _need(x, "x")
    _need(conv_state, "conv_state", x.dtype, (n_slots, C, state_len))
    _need(weight, "weight", torch.float32, (C, K))
    _need(bias, "bias", torch.float32, (C,))
    _need(conv_state_indices, "conv_state_indices", torch.int32, (B,))
    if DEBUG_CHECKS:
        check_distinct_slots(conv_state_indices, conv_state.shape[0], "conv_state_indices")
    _need(cache_seqlens, "cache_seqlens", torch.int32, (B,))
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, (B, C, L_new))
    _check("ssm_conv1d_update", _lib.ssm_conv1d_update(
        _ptr(x), _ptr(conv_state), _ptr(weight), _ptr(bias), _ptr(conv_state_indices),
        _ptr(cache_seqlens), _ptr(out), B, C, L_new, K, state_len, n_slots, _dtype_code(x),
        ACT[activation], _stream()))
    return out


def scan_fwd(x, dt, A, B, C, initial_state=None, seq_idx=None, return_final_state=True,
             final_state=None, y=None, workspace=None):
    """x [b, L, H, P]; dt [b, L, H] fp32; A [H] fp32; B, C [b, L, G, N]; initial_state
    [b, H, P, N] fp32 (may be the same tensor as final_state).  Returns (y, final_state)."""
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _need(x, "x")
    _need(dt, "dt", torch.float32, (bsz, L, H))
    _need(A, "A", torch.float32, (H,))
    _need(B, "B", x.dtype, (bsz, L, G, N))
    _need(C, "C", x.dtype, (bsz, L, G, N))
    _need(initial_state, "initial_state", torch.float32, (bsz, H, P, N))
    _need(seq_idx, "seq_idx", torch.int32, (bsz, L))
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, (bsz, L, H, P))
    if final_state is None and return_final_state:
        final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=x.device)
    _need(final_state, "final_state", torch.float32, (bsz, H, P, N))
    ws, nbytes = _workspace(workspace, workspace_size(bsz, L, H, P, G, N, x.dtype), x.device)
    _check("ssm_scan_fwd", _lib.ssm_scan_fwd(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(initial_state), _ptr(final_state),
        _ptr(seq_idx), _ptr(y), bsz, L, H, P, G, N, _dtype_code(x), _ptr(ws), nbytes, _stream()))
    return y, final_state


def conv_scan_fwd(xBC, conv_weight, conv_bias, dt, A, nheads, headdim, ngroups, dstate,
                  conv_initial_state=None, initial_state=None, seq_idx=None,
                  activation="silu", return_final_states=True, conv_final_state=None,
                  final_state=None, y=None, workspace=None):
    """The fused prefill.  xBC [b, L, H*P + 2*G*N] (x | B | C channels); conv_weight
    [C_conv, K] fp32; conv_bias [C_conv]; dt [b, L, H]; A [H]; conv states [b, C_conv, K-1];
    SSM states [b, H, P, N] fp32.  Returns (y [b, L, H, P], conv_final_state, final_state)."""
    bsz, L, Cc = xBC.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    if Cc != H * P + 2 * G * N:
        raise ValueError("xBC channel count must be nheads*headdim + 2*ngroups*dstate")
    K = conv_weight.shape[1]
    _need(xBC, "xBC")
    _need(conv_weight, "conv_weight", torch.float32, (Cc, K))
    _need(conv_bias, "conv_bias", torch.float32, (Cc,))
    _need(conv_initial_state, "conv_initial_state", xBC.dtype, (bsz, Cc, K - 1))
    _need(dt, "dt", torch.float32, (bsz, L, H))
    _need(A, "A", torch.float32, (H,))
    _need(initial_state, "initial_state", torch.float32, (bsz, H, P, N))
    _need(seq_idx, "seq_idx", torch.int32, (bsz, L))
    if y is None:
        y = torch.empty((bsz, L, H, P), dtype=xBC.dtype, device=xBC.device)
    _need(y, "y", xBC.dtype, (bsz, L, H, P))
    if return_final_states:
        if conv_final_state is None:
            conv_final_state = torch.empty((bsz, Cc, K - 1), dtype=xBC.dtype, device=xBC.device)
        if final_state is None:
            final_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=xBC.device)
    _need(conv_final_state, "conv_final_state", xBC.dtype, (bsz, Cc, K - 1))
    _need(final_state, "final_state", torch.float32, (bsz, H, P, N))
    ws, nbytes = _workspace(workspace, workspace_size(bsz, L, H, P, G, N, xBC.dtype), xBC.device)
    _check("ssm_conv_scan_fwd", _lib.ssm_conv_scan_fwd(
        _ptr(xBC), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_initial_state),
        _ptr(conv_final_state), _ptr(dt), _ptr(A), _ptr(initial_state), _ptr(final_state),
        _ptr(seq_idx), _ptr(y), bsz, L, H, P, G, N, K, _dtype_code(xBC), ACT[activation], _ptr(ws),
        nbytes, _stream()))
    return y, conv_final_state, final_state


def noalloc_scratch_bytes() -> int:
    """Bytes of the library's static per-GPU scratch that conv_scan_fwd_noalloc works in."""
    return int(_lib.ssm_noalloc_scratch_bytes())


def conv_scan_fwd_noalloc(xBC, conv_weight, conv_bias, dt, A, nheads, headdim, ngroups, dstate,
                          y, conv_final_state=None, final_state=None, conv_initial_state=None,
                          initial_state=None, seq_idx=None, activation="silu"):
    """conv_scan_fwd without a workspace: the library works in its static per-GPU scratch
    (noalloc_scratch_bytes()), so nothing is allocated; the caller passes y and the final-state
    buffers it wants (None: not written).  Calls that may overlap on one GPU race on the
    scratch; sizes needing more scratch raise SSMError (status SSM_ERR_WORKSPACE)."""
    bsz, L, Cc = xBC.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    if Cc != H * P + 2 * G * N:
        raise ValueError("xBC channel count must be nheads*headdim + 2*ngroups*dstate")
    K = conv_weight.shape[1]
    if y is None:
        raise ValueError("y is required: this call allocates nothing")
    _need(xBC, "xBC")
    _need(conv_weight, "conv_weight", torch.float32, (Cc, K))
    _need(conv_bias, "conv_bias", torch.float32, (Cc,))
    _need(conv_initial_state, "conv_initial_state", xBC.dtype, (bsz, Cc, K - 1))
    _need(dt, "dt", torch.float32, (bsz, L, H))
    _need(A, "A", torch.float32, (H,))
    _need(initial_state, "initial_state", torch.float32, (bsz, H, P, N))
    _need(seq_idx, "seq_idx", torch.int32, (bsz, L))
    _need(y, "y", xBC.dtype, (bsz, L, H, P))
    _need(conv_final_state, "conv_final_state", xBC.dtype, (bsz, Cc, K - 1))
    _need(final_state, "final_state", torch.float32, (bsz, H, P, N))
    _check("ssm_conv_scan_fwd_noalloc", _lib.ssm_conv_scan_fwd_noalloc(
        _ptr(xBC), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_initial_state),
        _ptr(conv_final_state), _ptr(dt), _ptr(A), _ptr(initial_state), _ptr(final_state),
        _ptr(seq_idx), _ptr(y), bsz, L, H, P, G, N, K, _dtype_code(xBC), ACT[activation],
        _stream()))
    return y, conv_final_state, final_state


def step(x, dt, A, B, C, state, state_indices=None, y=None, nheads=None, ngroups=None):
    """Decode update of a state pool.  x [b, n_new, H*P], B / C [b, n_new, G*N] -- any
    strides (e.g. channel ranges of the [b, C_conv, n_new] conv-update output, transposed);
    dt [b, n_new, H] fp32; state [n_slots, H, P, N] fp32 (updated in place);
    state_indices [b] int32.  Returns y [b, n_new, H, P]."""
    n_slots, H, P, N = state.shape
    bsz, n_new, HP = x.shape
    if B.dim() != 3 or B.shape[2] % N != 0:
        raise ValueError(f"B must be [b, n_new, G*N] with N = {N} (the state's last dimension)")
    G = B.shape[2] // N
    if HP != H * P or C.shape != B.shape or B.shape[:2] != x.shape[:2]:
        raise ValueError("x must be [b, n_new, H*P] and B, C [b, n_new, G*N]")
    if nheads is not None and nheads != H:
        raise ValueError(f"nheads {nheads} does not match the state's {H} heads")
    if ngroups is not None and ngroups != G:
        raise ValueError(f"ngroups {ngroups} does not match B's width {B.shape[2]} / N {N}")
    if H % G != 0:
        raise ValueError(f"nheads {H} must be a multiple of ngroups {G}")
    for t, name in ((x, "x"), (B, "B"), (C, "C")):
        _need(t, name, contiguous=False)
    _need(dt, "dt", torch.float32, (bsz, n_new, H))
    _need(A, "A", torch.float32, (H,))
    _need(state, "state", torch.float32)
    _need(state_indices, "state_indices", torch.int32, (bsz,))
    if DEBUG_CHECKS:
        check_distinct_slots(state_indices, n_slots, "state_indices")
    if y is None:
        y = torch.empty((bsz, n_new, H, P), dtype=x.dtype, device=x.device)
    _need(y, "y", x.dtype, (bsz, n_new, H, P))
    sx, sb, sc = x.stride(), B.stride(), C.stride()
    _check("ssm_step", _lib.ssm_step(
        _ptr(x), sx[0], sx[1], sx[2], _ptr(dt), _ptr(A), _ptr(B), sb[0], sb[1], sb[2], _ptr(C),
        sc[0], sc[1], sc[2], _ptr(state), _ptr(state_indices), _ptr(y), bsz, n_new, H, P, G, N,
        n_slots, _dtype_code(x), _stream()))
    return y


def decode_step(x_new, conv_state, conv_weight, conv_bias, dt, A, ssm_state, nheads, headdim,
                ngroups, dstate, conv_state_indices=None, cache_seqlens=None,
                state_indices=None, activation="silu", conv_out=None, y=None):
    """One decode step on the pools (ssm_decode_step): the conv update over x_new
    [b, C_conv, n_new], then the SSM step reading the x | B | C channel ranges of its output.
    Both pools update in place; cache_seqlens is not advanced.  state_indices defaults to
    conv_state_indices.  Returns y [b, n_new, H, P]."""
    bsz, C, n_new = x_new.shape
    H, P, G, N = nheads, headdim, ngroups, dstate
    if C != H * P + 2 * G * N:
        raise ValueError("x_new channel count must be nheads*headdim + 2*ngroups*dstate")
    n_cslots, _, state_len = conv_state.shape
    K = conv_weight.shape[1]
    _need(x_new, "x_new")
    _need(conv_state, "conv_state", x_new.dtype, (n_cslots, C, state_len))
    _need(conv_weight, "conv_weight", torch.float32, (C, K))
    _need(conv_bias, "conv_bias", torch.float32, (C,))
    _need(dt, "dt", torch.float32, (bsz, n_new, H))
    _need(A, "A", torch.float32, (H,))
    if ssm_state.dim() != 4 or tuple(ssm_state.shape[1:]) != (H, P, N):
        raise ValueError(f"ssm_state must be [n_slots, {H}, {P}, {N}]")
    _need(ssm_state, "ssm_state", torch.float32)
    _need(conv_state_indices, "conv_state_indices", torch.int32, (bsz,))
    _need(cache_seqlens, "cache_seqlens", torch.int32, (bsz,))
    _need(state_indices, "state_indices", torch.int32, (bsz,))
    if DEBUG_CHECKS:
        check_distinct_slots(conv_state_indices, n_cslots, "conv_state_indices")
        check_distinct_slots(state_indices if state_indices is not None else conv_state_indices,
                             ssm_state.shape[0], "state_indices")
    if conv_out is None:
        conv_out = torch.empty_like(x_new)
    _need(conv_out, "conv_out", x_new.dtype, (bsz, C, n_new))
    if y is None:
        y = torch.empty((bsz, n_new, H, P), dtype=x_new.dtype, device=x_new.device)
    _need(y, "y", x_new.dtype, (bsz, n_new, H, P))
    _check("ssm_decode_step", _lib.ssm_decode_step(
        _ptr(x_new), _ptr(conv_state), _ptr(conv_weight), _ptr(conv_bias),
        _ptr(conv_state_indices), _ptr(cache_seqlens), _ptr(dt), _ptr(A), _ptr(ssm_state),
        _ptr(state_indices), _ptr(conv_out), _ptr(y), bsz, n_new, H, P, G, N, K, state_len,
        n_cslots, ssm_state.shape[0], _dtype_code(x_new), ACT[activation], _stream()))
    return y


def stream_copy(src, dst):
    """dst <- src (same number of bytes, no overlap) with the library's streaming copy: the
    bandwidth reference of the benchmark, not part of the method."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("stream_copy: src and dst differ in size")
    _need(src, "src")
    _need(dst, "dst")
    _check("ssm_stream_copy", _lib.ssm_stream_copy(_ptr(src), _ptr(dst), nb, _stream()))
    return dst


def timing_enable(enable: bool = True):
    _check("ssm_timing_enable", _lib.ssm_timing_enable(1 if enable else 0))


def timing_read():
    """(summed main-kernel milliseconds, launches) since the last read."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check("ssm_timing_read", _lib.ssm_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
