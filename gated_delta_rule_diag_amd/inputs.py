"""Seeded synthetic KDA workloads.

This module only draws and rounds numbers: it holds none of the operator's
arithmetic, so the fp64 oracle and the HIP path can both be fed from it
without sharing any code that decides a result.

Recipe (one independent numpy stream per (config c, sequence/batch n, head h)):
    rng = numpy.random.default_rng([20261203, c, n, h])
    draw, in this order:  q [L,DK], k [L,DK], v [L,DV] ~ N(0,1) (fp64),
                          z [L] ~ N(0,1),  u [L,DK] ~ U(-5,-1)
    q, k  <- row-wise L2-normalised in fp64, rounded to fp32 (nearest-even),
             then to bf16 (nearest-even) when the workload is bf16
    v     <- rounded the same way
    beta  = sigmoid(z)          rounded to fp32
    alpha = exp(-exp(u))        rounded to fp32, so alpha in (0.692, 0.9933)

Large packed workloads (hundreds of millions of token-heads) are drawn on the
device instead, with a seeded torch Philox generator per head and the same
distributions (normalisation in fp32); see ``device_head_inputs``.
"""

from __future__ import annotations

import numpy as np

SEED = 20261203

__all__ = [
    "SEED",
    "round_bf16",
    "bf16_bits",
    "head_inputs",
    "batch_inputs",
    "packed_inputs",
    "varlen_lengths",
    "decode_inputs",
    "decode_prefix",
    "device_head_inputs",
]


def round_bf16(x):
    """Round fp32 values to the nearest bf16 (ties to even); result as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x):
    """Bit patterns (uint16) of fp32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _round(x64, dtype):
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return round_bf16(x32)
    if dtype == "f32":
        return x32
    raise ValueError(dtype)


def head_inputs(c, n, h, L, DK, DV, dtype, sub=None):
    """Inputs of one (sequence, head) stream: L tokens.

    Returns fp32 arrays q [L,DK], k [L,DK], v [L,DV], alpha [L,DK], beta [L]
    (bf16 workloads hold bf16-exact values in q, k, v).  ``sub`` selects an
    extra sub-stream index (used for decode prefixes).
    """
    key = [SEED, c, n, h] if sub is None else [SEED, c, n, h, sub]
    rng = np.random.default_rng(key)
    q = rng.standard_normal((L, DK))
    k = rng.standard_normal((L, DK))
    v = rng.standard_normal((L, DV))
    z = rng.standard_normal(L)
    u = rng.uniform(-5.0, -1.0, size=(L, DK))
    q = q / np.linalg.norm(q, axis=1, keepdims=True)
    k = k / np.linalg.norm(k, axis=1, keepdims=True)
    beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    alpha = np.exp(-np.exp(u)).astype(np.float32)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype), alpha, beta


def batch_inputs(c, B, T, H, DK, DV, dtype, heads=None):
    """Fixed-length batch in the operator's token-major layout.

    Returns q, k, alpha [B,T,H,DK], v [B,T,H,DV], beta [B,T,H] (fp32 arrays).
    With ``heads`` given, only those heads are drawn (others stay zero).
    """
    q = np.zeros((B, T, H, DK), np.float32)
    k = np.zeros((B, T, H, DK), np.float32)
    a = np.ones((B, T, H, DK), np.float32)
    v = np.zeros((B, T, H, DV), np.float32)
    be = np.zeros((B, T, H), np.float32)
    for b in range(B):
        for h in range(H) if heads is None else heads:
            qq, kk, vv, aa, bb = head_inputs(c, b, h, T, DK, DV, dtype)
            q[b, :, h], k[b, :, h], v[b, :, h], a[b, :, h], be[b, :, h] = qq, kk, vv, aa, bb
    return q, k, v, a, be


def varlen_lengths(c, N, lo, hi):
    """Sequence lengths ~ U{lo..hi}, seeded by [20261203, c, 999]."""
    rng = np.random.default_rng([SEED, c, 999])
    return rng.integers(lo, hi + 1, size=N).astype(np.int64)


def packed_inputs(c, lengths, H, DK, DV, dtype, heads=None):
    """Packed varlen workload: sequence n draws from stream (c, n, h).

    Returns q, k, alpha [T_total,H,DK], v [T_total,H,DV], beta [T_total,H]
    and cu_seqlens (int32 [N+1]).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    Tt = int(cu[-1])
    q = np.zeros((Tt, H, DK), np.float32)
    k = np.zeros((Tt, H, DK), np.float32)
    a = np.ones((Tt, H, DK), np.float32)
    v = np.zeros((Tt, H, DV), np.float32)
    be = np.zeros((Tt, H), np.float32)
    for n, L in enumerate(lengths):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(H) if heads is None else heads:
            qq, kk, vv, aa, bb = head_inputs(c, n, h, int(L), DK, DV, dtype)
            q[s:e, h], k[s:e, h], v[s:e, h], a[s:e, h], be[s:e, h] = qq, kk, vv, aa, bb
    return q, k, v, a, be, cu.astype(np.int32)


def decode_inputs(c, N, H, DK, DV, dtype):
    """The decode token of every (sequence, head): stream (c, n, h), L = 1.

    Returns q, k, alpha [N,H,DK], v [N,H,DV], beta [N,H].
    """
    q = np.zeros((N, H, DK), np.float32)
    k = np.zeros((N, H, DK), np.float32)
    a = np.zeros((N, H, DK), np.float32)
    v = np.zeros((N, H, DV), np.float32)
    be = np.zeros((N, H), np.float32)
    for n in range(N):
        for h in range(H):
            qq, kk, vv, aa, bb = head_inputs(c, n, h, 1, DK, DV, dtype)
            q[n, h], k[n, h], v[n, h], a[n, h], be[n, h] = qq[0], kk[0], vv[0], aa[0], bb[0]
    return q, k, v, a, be


def decode_prefix(c, n, h, L0, DK, DV, dtype):
    """The L0 tokens that precede the decode token of (n, h): sub-stream 1."""
    return head_inputs(c, n, h, L0, DK, DV, dtype, sub=1)


def device_head_inputs(c, n, h, L, DK, DV, device, torch_dtype):
    """Same distributions, drawn on ``device`` by a seeded torch generator.

    Used for packed workloads too large to draw on the host.  Returns torch
    tensors q, k [L,DK] and v [L,DV] in ``torch_dtype``; alpha [L,DK] and
    beta [L] in fp32.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((((SEED * 1000003 + c) * 1000003 + n) * 1000003 + h) % (1 << 63))
    f32 = torch.float32
    q = torch.randn((L, DK), generator=g, device=device, dtype=f32)
    k = torch.randn((L, DK), generator=g, device=device, dtype=f32)
    v = torch.randn((L, DV), generator=g, device=device, dtype=f32)
    z = torch.randn((L,), generator=g, device=device, dtype=f32)
    u = torch.rand((L, DK), generator=g, device=device, dtype=f32) * 4.0 - 5.0
    q = q / q.norm(dim=1, keepdim=True)
    k = k / k.norm(dim=1, keepdim=True)
    beta = torch.sigmoid(z)
    alpha = torch.exp(-torch.exp(u))
    return q.to(torch_dtype), k.to(torch_dtype), v.to(torch_dtype), alpha, beta
