"""Thin Python binding of libkda.so (ctypes).

Argument marshalling only: every step of the operator runs in the HIP kernels
behind the C ABI (include/kda.h).  PyTorch provides device memory and the
current stream; nothing here computes any part of the result.  If the built
library is missing the import fails loudly: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK = 0
KDA_F32 = 0
KDA_BF16 = 1

STATUS_NAMES = {
    0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
    4: "KDA_ERR_ALIGN", 5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_HIP",
}

EXPORTED = (
    "kda_abi_version",
    "kda_chunk_prefill_workspace_size",
    "kda_chunk_prefill",
    "kda_chunk_prefill_snapshots",
    "kda_chunk_prefill_varlen_workspace_size",
    "kda_chunk_prefill_varlen",
    "kda_decode_step",
    "kda_decode_pool",
    "kda_chunk_prefill_scalar_gate",
    "kda_chunk_prefill_varlen_scalar_gate",
    "kda_decode_step_scalar_gate",
    "kda_chunk_backward_workspace_size",
    "kda_chunk_backward",
    "kda_chunk_prefill_varlen_snapshots",
    "kda_chunk_backward_varlen_workspace_size",
    "kda_chunk_backward_varlen",
    "kda_chunk_backward_scalar_gate",
    "kda_chunk_backward_varlen_scalar_gate",
    "kda_status_string",
    "kda_last_error_message",
    "kda_internal_set_tuning",
    "kda_chunk_prefill_noalloc",
)


class KDAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m gated_delta_rule_diag_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_abi_version.restype = i
    lib.kda_abi_version.argtypes = []
    lib.kda_chunk_prefill_workspace_size.restype = sz
    lib.kda_chunk_prefill_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.kda_chunk_prefill.restype = i
    lib.kda_chunk_prefill.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_chunk_prefill_snapshots.restype = i
    lib.kda_chunk_prefill_snapshots.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp,
                                                i, vp, vp, sz, vp]
    lib.kda_chunk_prefill_varlen_workspace_size.restype = sz
    lib.kda_chunk_prefill_varlen_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.kda_chunk_prefill_varlen.restype = i
    lib.kda_chunk_prefill_varlen.argtypes = [i, i, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp,
                                             vp, sz, vp]
    lib.kda_decode_step.restype = i
    lib.kda_decode_step.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_chunk_prefill_scalar_gate.restype = i
    lib.kda_chunk_prefill_scalar_gate.argtypes = list(lib.kda_chunk_prefill.argtypes)
    lib.kda_chunk_prefill_varlen_scalar_gate.restype = i
    lib.kda_chunk_prefill_varlen_scalar_gate.argtypes = list(lib.kda_chunk_prefill_varlen.argtypes)
    lib.kda_decode_step_scalar_gate.restype = i
    lib.kda_decode_step_scalar_gate.argtypes = list(lib.kda_decode_step.argtypes)
    lib.kda_chunk_backward_workspace_size.restype = sz
    lib.kda_chunk_backward_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.kda_chunk_backward.restype = i
    lib.kda_chunk_backward.argtypes = [i, i, i, i, i, i, i] + [vp] * 15 + [sz, vp]
    lib.kda_chunk_backward_varlen_workspace_size.restype = sz
    lib.kda_chunk_backward_varlen_workspace_size.argtypes = [i] * 7
    lib.kda_chunk_backward_varlen.restype = i
    lib.kda_chunk_backward_varlen.argtypes = [i, i, vp, i, i, i, i, i, i] + [vp] * 15 + [sz, vp]
    lib.kda_chunk_backward_scalar_gate.restype = i
    lib.kda_chunk_backward_scalar_gate.argtypes = lib.kda_chunk_backward.argtypes
    lib.kda_chunk_backward_varlen_scalar_gate.restype = i
    lib.kda_chunk_backward_varlen_scalar_gate.argtypes = lib.kda_chunk_backward_varlen.argtypes
    lib.kda_chunk_prefill_varlen_snapshots.restype = i
    lib.kda_chunk_prefill_varlen_snapshots.argtypes = [i, i, vp, i, i, i, i, i] + [vp] * 8 + \
        [i, vp, i, vp, vp, sz, vp]
    lib.kda_decode_pool.restype = i
    lib.kda_decode_pool.argtypes = [i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, i, vp, vp, vp]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i]
    lib.kda_last_error_message.restype = ctypes.c_char_p
    lib.kda_last_error_message.argtypes = []
    lib.kda_internal_set_tuning.restype = i
    lib.kda_internal_set_tuning.argtypes = [i, i, i, i]
    lib.kda_chunk_prefill_noalloc.restype = i
    lib.kda_chunk_prefill_noalloc.argtypes = [i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    return lib


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


_TUNING = {"prefill_form": 0, "prefill_nsub": 0, "prefill_seg": 0, "bwd_window": 0}
_FORMS = {"auto": 0, "fused": 1, "split": 2, "staged": 2}


def set_tuning(**kw):
    """Internal (tests and measurements): kda_internal_set_tuning for the
    given knobs, the others kept.  prefill_form takes "auto", "fused" or
    "split"/"staged"; the numbers take 0 for the choice by shape.  Called
    with no argument, restores every choice by shape."""
    state = dict(_TUNING) if kw else {k: 0 for k in _TUNING}
    for k, v in kw.items():
        if k not in _TUNING:
            raise TypeError(f"unknown tuning knob {k}")
        state[k] = _FORMS[v] if k == "prefill_form" and isinstance(v, str) else int(v)
    _check(lib().kda_internal_set_tuning(state["prefill_form"], state["prefill_nsub"],
                                         state["prefill_seg"], state["bwd_window"]))
    _TUNING.update(state)


def _check(status):
    if status != KDA_OK:
        raise KDAError(status, lib().kda_last_error_message().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _in_dtype(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise ValueError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def chunk_prefill(q, k, v, alpha, beta, initial_state=None, output_final_state=True, chunk=64,
                  out=None, final_state=None, workspace=None):
    """KDA chunked prefill, fixed length.

    q, k: [B,T,H,DK], v: [B,T,H,DV] (bfloat16 or float32, same dtype);
    alpha: [B,T,H,DK] float32 (per-channel decay), or [B,T,H] for the scalar
    gate of Gated DeltaNet; beta: [B,T,H] float32;
    initial_state: [B,H,DK,DV] float32 or None (zeros).
    Returns (o [B,T,H,DV] float32, final_state [B,H,DK,DV] float32 or None).
    """
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, DK))
    _need(v, "v", q.dtype, (B, T, H, DV))
    scalar = alpha.dim() == 3
    _need(alpha, "alpha", torch.float32, (B, T, H) if scalar else (B, T, H, DK))
    _need(beta, "beta", torch.float32, (B, T, H))
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (B, H, DK, DV))
    dev = q.device
    o = out if out is not None else torch.empty((B, T, H, DV), device=dev, dtype=torch.float32)
    _need(o, "out", torch.float32, (B, T, H, DV))
    st = None
    if output_final_state:
        st = final_state if final_state is not None else torch.empty(
            (B, H, DK, DV), device=dev, dtype=torch.float32)
        _need(st, "final_state", torch.float32, (B, H, DK, DV))
    wsz = lib().kda_chunk_prefill_workspace_size(B, T, H, DK, DV, chunk)
    if wsz and workspace is None:
        workspace = torch.empty(wsz, device=dev, dtype=torch.uint8)
    fn = lib().kda_chunk_prefill_scalar_gate if scalar else lib().kda_chunk_prefill
    _check(fn(
        B, T, H, DK, DV, chunk, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(initial_state), _ptr(o), _ptr(st), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev)))
    return o, st


def chunk_prefill_snapshots(q, k, v, alpha, beta, every, initial_state=None,
                            output_final_state=True, chunk=64, out=None, final_state=None,
                            snapshots=None, workspace=None):
    """KDA chunked prefill that also returns the state after every ``every``-th
    chunk of 64 tokens (prefix caching).

    Arguments as for :func:`chunk_prefill`.  Returns (o, final_state, snapshots)
    with snapshots [B, T // (64 * every), H, DK, DV] float32: entry j is the
    state after the first 64 * every * (j + 1) tokens of each sequence.
    """
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, DK))
    _need(v, "v", q.dtype, (B, T, H, DV))
    _need(alpha, "alpha", torch.float32, (B, T, H, DK))
    _need(beta, "beta", torch.float32, (B, T, H))
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (B, H, DK, DV))
    if every < 1:
        raise ValueError("every must be >= 1")
    dev = q.device
    o = out if out is not None else torch.empty((B, T, H, DV), device=dev, dtype=torch.float32)
    _need(o, "out", torch.float32, (B, T, H, DV))
    st = None
    if output_final_state:
        st = final_state if final_state is not None else torch.empty(
            (B, H, DK, DV), device=dev, dtype=torch.float32)
        _need(st, "final_state", torch.float32, (B, H, DK, DV))
    ns = T // (chunk * every)
    snaps = snapshots if snapshots is not None else torch.empty(
        (B, ns, H, DK, DV), device=dev, dtype=torch.float32)
    _need(snaps, "snapshots", torch.float32, (B, ns, H, DK, DV))
    wsz = lib().kda_chunk_prefill_workspace_size(B, T, H, DK, DV, chunk)
    if wsz and workspace is None:
        workspace = torch.empty(wsz, device=dev, dtype=torch.uint8)
    _check(lib().kda_chunk_prefill_snapshots(
        B, T, H, DK, DV, chunk, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(initial_state), _ptr(o), _ptr(st), every, _ptr(snaps), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev)))
    return o, st, snaps


def chunk_prefill_varlen(q, k, v, alpha, beta, cu_seqlens, initial_state=None,
                         output_final_state=True, chunk=64, out=None, final_state=None,
                         workspace=None):
    """KDA chunked prefill over packed sequences.

    q, k: [T_total,H,DK], v: [T_total,H,DV]; alpha [T_total,H,DK] (or [T_total,H]
    for a scalar gate); beta [T_total,H];
    cu_seqlens: int32 device tensor [N+1]; initial_state [N,H,DK,DV] or None.
    Returns (o [T_total,H,DV], final_state [N,H,DK,DV] or None).
    """
    Tt, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (Tt, H, DK))
    _need(v, "v", q.dtype, (Tt, H, DV))
    scalar = alpha.dim() == 2
    _need(alpha, "alpha", torch.float32, (Tt, H) if scalar else (Tt, H, DK))
    _need(beta, "beta", torch.float32, (Tt, H))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, DK, DV))
    dev = q.device
    o = out if out is not None else torch.empty((Tt, H, DV), device=dev, dtype=torch.float32)
    _need(o, "out", torch.float32, (Tt, H, DV))
    st = None
    if output_final_state:
        st = final_state if final_state is not None else torch.empty(
            (N, H, DK, DV), device=dev, dtype=torch.float32)
        _need(st, "final_state", torch.float32, (N, H, DK, DV))
    wsz = lib().kda_chunk_prefill_varlen_workspace_size(N, Tt, H, DK, DV, chunk)
    if wsz and workspace is None:
        workspace = torch.empty(wsz, device=dev, dtype=torch.uint8)
    fn = lib().kda_chunk_prefill_varlen_scalar_gate if scalar else lib().kda_chunk_prefill_varlen
    _check(fn(
        N, Tt, _ptr(cu_seqlens), H, DK, DV, chunk, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(st), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev)))
    return o, st


def decode_step(q, k, v, alpha, beta, state, out=None):
    """One recurrent decode step; ``state`` [N,H,DK,DV] float32 is updated in place.

    q, k: [N,H,DK], v: [N,H,DV]; alpha [N,H,DK] (or [N,H] for a scalar gate);
    beta [N,H].  Returns o [N,H,DV].
    """
    N, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (N, H, DK))
    _need(v, "v", q.dtype, (N, H, DV))
    scalar = alpha.dim() == 2
    _need(alpha, "alpha", torch.float32, (N, H) if scalar else (N, H, DK))
    _need(beta, "beta", torch.float32, (N, H))
    _need(state, "state", torch.float32, (N, H, DK, DV))
    dev = q.device
    o = out if out is not None else torch.empty((N, H, DV), device=dev, dtype=torch.float32)
    _need(o, "out", torch.float32, (N, H, DV))
    fn = lib().kda_decode_step_scalar_gate if scalar else lib().kda_decode_step
    _check(fn(N, H, DK, DV, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state),
              _ptr(o), _stream(dev)))
    return o


def decode_pool(q, k, v, alpha, beta, state_pool, state_idx=None, num_tokens=None,
                return_token_states=False, out=None, token_states=None):
    """Decode of up to L tokens per sequence with states in a pool.

    q, k, alpha: [N,L,H,DK]; v: [N,L,H,DV]; beta: [N,L,H];
    state_pool: [P,H,DK,DV] float32, updated in place;
    state_idx: int32 device tensor [N] or None (slot n; P >= N); a slot outside
    [0, P) marks a padding row (its outputs are 0, the pool is untouched);
    num_tokens: int32 device tensor [N] or None (all L).
    Returns (o [N,L,H,DV], token_states [N,L,H,DK,DV] or None).
    """
    N, L, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (N, L, H, DK))
    _need(v, "v", q.dtype, (N, L, H, DV))
    _need(alpha, "alpha", torch.float32, (N, L, H, DK))
    _need(beta, "beta", torch.float32, (N, L, H))
    _need(state_pool, "state_pool", torch.float32)
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, DK, DV):
        raise ValueError(f"state_pool must have shape [P,{H},{DK},{DV}], got {tuple(state_pool.shape)}")
    if state_idx is not None:
        _need(state_idx, "state_idx", torch.int32, (N,))
    if num_tokens is not None:
        _need(num_tokens, "num_tokens", torch.int32, (N,))
    dev = q.device
    o = out if out is not None else torch.empty((N, L, H, DV), device=dev, dtype=torch.float32)
    _need(o, "out", torch.float32, (N, L, H, DV))
    ts = None
    if return_token_states:
        ts = token_states if token_states is not None else torch.empty(
            (N, L, H, DK, DV), device=dev, dtype=torch.float32)
        _need(ts, "token_states", torch.float32, (N, L, H, DK, DV))
    _check(lib().kda_decode_pool(
        N, L, H, DK, DV, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_idx),
        _ptr(num_tokens), _ptr(state_pool), state_pool.shape[0], _ptr(o), _ptr(ts), _stream(dev)))
    return o, ts


def chunk_backward(q, k, v, alpha, beta, d_o, initial_state=None, d_final_state=None,
                   chunk=64, workspace=None):
    """Gradients of L = sum(o * d_o) + sum(S_T * d_final_state) for the
    fixed-length prefill.

    Inputs as for :func:`chunk_prefill` (alpha [B,T,H,DK], or [B,T,H] for a
    scalar gate, whose gradient then has that shape); d_o [B,T,H,DV] float32;
    d_final_state [B,H,DK,DV] float32 or None.
    Returns (dq, dk, dv, dalpha, dbeta, d_initial_state), all float32.
    """
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, DK))
    _need(v, "v", q.dtype, (B, T, H, DV))
    sg = alpha.dim() == 3
    _need(alpha, "alpha", torch.float32, (B, T, H) if sg else (B, T, H, DK))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(d_o, "d_o", torch.float32, (B, T, H, DV))
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (B, H, DK, DV))
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", torch.float32, (B, H, DK, DV))
    dev = q.device
    f32 = dict(device=dev, dtype=torch.float32)
    dq, dk = (torch.empty((B, T, H, DK), **f32) for _ in range(2))
    dal = torch.empty((B, T, H) if sg else (B, T, H, DK), **f32)
    dv = torch.empty((B, T, H, DV), **f32)
    db = torch.empty((B, T, H), **f32)
    ds0 = torch.empty((B, H, DK, DV), **f32)
    wsz = lib().kda_chunk_backward_workspace_size(B, T, H, DK, DV, chunk)
    if wsz and workspace is None:
        workspace = torch.empty(wsz, device=dev, dtype=torch.uint8)
    fn = lib().kda_chunk_backward_scalar_gate if sg else lib().kda_chunk_backward
    _check(fn(
        B, T, H, DK, DV, chunk, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dal), _ptr(db), _ptr(ds0), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev)))
    return dq, dk, dv, dal, db, ds0


def chunk_prefill_varlen_snapshots(q, k, v, alpha, beta, cu_seqlens, every, initial_state=None,
                                   output_final_state=True, chunk=64, snap_offsets=None,
                                   out=None, final_state=None, snapshots=None, workspace=None,
                                   num_snapshots=None):
    """Packed variable-length prefill that also returns each sequence's state
    after every ``every``-th chunk of 64 tokens.

    Arguments as for :func:`chunk_prefill_varlen`.  ``snap_offsets`` (int32
    device [N+1]) places sequence n's snapshots at rows snap_offsets[n] ..; by
    default it is built on the device from the sequence lengths
    (floor(len_n / (64 every)) rows each, in order).  The host never reads
    device data: ``snapshots`` (or ``num_snapshots``) gives the number of rows;
    by default T_total // (64 every) rows, a bound of what the sequences
    produce that the host knows without reading cu_seqlens (rows from
    snap_offsets[N] on are then not written).
    Returns (o, final_state, snapshots [rows, H, DK, DV], snap_offsets).
    """
    Tt, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (Tt, H, DK))
    _need(v, "v", q.dtype, (Tt, H, DV))
    _need(alpha, "alpha", torch.float32, (Tt, H, DK))
    _need(beta, "beta", torch.float32, (Tt, H))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if every < 1:
        raise ValueError("every must be >= 1")
    N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, DK, DV))
    dev = q.device
    if snap_offsets is None:
        # device ops only (asynchronous, no host copy)
        per = torch.div(cu_seqlens[1:] - cu_seqlens[:-1], chunk * every, rounding_mode="floor")
        snap_offsets = torch.zeros(N + 1, dtype=torch.int32, device=dev)
        snap_offsets[1:] = torch.cumsum(per, 0)
    else:
        _need(snap_offsets, "snap_offsets", torch.int32, (N + 1,))
    if snapshots is not None:
        rows = snapshots.shape[0]
    elif num_snapshots is not None:
        rows = int(num_snapshots)
    else:
        rows = Tt // (chunk * every)
    o = out if out is not None else torch.empty((Tt, H, DV), device=dev, dtype=torch.float32)
    _need(o, "out", torch.float32, (Tt, H, DV))
    st = None
    if output_final_state:
        st = final_state if final_state is not None else torch.empty(
            (N, H, DK, DV), device=dev, dtype=torch.float32)
        _need(st, "final_state", torch.float32, (N, H, DK, DV))
    snaps = snapshots if snapshots is not None else torch.empty(
        (rows, H, DK, DV), device=dev, dtype=torch.float32)
    _need(snaps, "snapshots", torch.float32)
    if snaps.dim() != 4 or tuple(snaps.shape[1:]) != (H, DK, DV):
        raise ValueError(f"snapshots must have shape [rows,{H},{DK},{DV}]")
    wsz = lib().kda_chunk_prefill_varlen_workspace_size(N, Tt, H, DK, DV, chunk)
    if wsz and workspace is None:
        workspace = torch.empty(wsz, device=dev, dtype=torch.uint8)
    _check(lib().kda_chunk_prefill_varlen_snapshots(
        N, Tt, _ptr(cu_seqlens), H, DK, DV, chunk, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(st), every, _ptr(snap_offsets),
        snaps.shape[0], _ptr(snaps), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev)))
    return o, st, snaps, snap_offsets


def chunk_backward_varlen(q, k, v, alpha, beta, cu_seqlens, d_o, initial_state=None,
                          d_final_state=None, chunk=64, workspace=None, max_seqlen=None):
    """Gradients of L = sum(o * d_o) + sum(S_T * d_final_state) for the packed
    variable-length prefill (per-channel alpha).

    Inputs as for :func:`chunk_prefill_varlen` (alpha [T_total,H,DK], or
    [T_total,H] for a scalar gate); d_o [T_total,H,DV] float32;
    d_final_state [N,H,DK,DV] float32 or None; max_seqlen (required): the
    longest sequence's length as a host int, as varlen attention interfaces
    take it (the host never reads cu_seqlens), or 0 if unknown.
    Returns (dq, dk, dv, dalpha, dbeta, d_initial_state), all float32.
    """
    Tt, H, DK = q.shape
    DV = v.shape[-1]
    dt = _in_dtype(q)
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (Tt, H, DK))
    _need(v, "v", q.dtype, (Tt, H, DV))
    sg = alpha.dim() == 2
    _need(alpha, "alpha", torch.float32, (Tt, H) if sg else (Tt, H, DK))
    _need(beta, "beta", torch.float32, (Tt, H))
    _need(d_o, "d_o", torch.float32, (Tt, H, DV))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, DK, DV))
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", torch.float32, (N, H, DK, DV))
    dev = q.device
    f32 = dict(device=dev, dtype=torch.float32)
    dq, dk = (torch.empty((Tt, H, DK), **f32) for _ in range(2))
    dal = torch.empty((Tt, H) if sg else (Tt, H, DK), **f32)
    dv = torch.empty((Tt, H, DV), **f32)
    db = torch.empty((Tt, H), **f32)
    ds0 = torch.empty((N, H, DK, DV), **f32)
    if max_seqlen is None:
        raise ValueError("max_seqlen is required: the longest sequence's length as a host int "
                         "(0 if unknown: still correct, the library then assumes T_total and "
                         "runs more reverse-pass windows)")
    wsz = lib().kda_chunk_backward_varlen_workspace_size(N, Tt, max_seqlen, H, DK, DV, chunk)
    if wsz and workspace is None:
        workspace = torch.empty(wsz, device=dev, dtype=torch.uint8)
    fn = lib().kda_chunk_backward_varlen_scalar_gate if sg else lib().kda_chunk_backward_varlen
    _check(fn(
        N, Tt, _ptr(cu_seqlens), max_seqlen, H, DK, DV, chunk, dt, _ptr(q), _ptr(k), _ptr(v),
        _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dal), _ptr(db), _ptr(ds0), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(dev)))
    return dq, dk, dv, dal, db, ds0
