"""GPU parity of the scalar-gate (Gated DeltaNet) forms: prefill (both
forms, fixed and varlen) and decode against the fp64 Gated DeltaNet oracle,
and bitwise equality with the per-channel entry points given the gate
broadcast over the key channels."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host, random_state, tdtype
from oracle import gdn_backward, gdn_recurrent, max_rel_err

pytestmark = pytest.mark.gpu

PATHS = ["fused", "split"]


def gate_of(a):
    """One gate per token and head: the first channel's seeded alpha."""
    return np.ascontiguousarray(a[..., 0])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dt,T,dk,dv", [("bf16", 200, 128, 128), ("bf16", 64, 64, 64),
                                        ("f32", 130, 128, 64), ("bf16", 17, 64, 128),
                                        ("f32", 256, 64, 64)])
def test_scalar_gate_prefill_matches_oracle(dt, T, dk, dv, path, monkeypatch):
    kda.set_tuning(prefill_form=path)
    B, H = 2, 3
    flush(f"[scalar gate] prefill B={B} T={T} H={H} DK={dk} DV={dv} {dt} path={path}")
    q, k, v, a, b = I.batch_inputs(600 + T, B, T, H, dk, dv, dt)
    g = gate_of(a)
    S0 = random_state(np.random.default_rng(T), (B, H, dk, dv))
    o_ref, S_ref = gdn_recurrent(q, k, v, g, b, S0)
    td = tdtype(dt)
    x = (dev(q, td), dev(k, td), dev(v, td))
    o, S = kda.chunk_prefill(*x, dev(g), dev(b), dev(S0))
    ob, Sb = kda.chunk_prefill(*x, dev(np.broadcast_to(g[..., None], a.shape)), dev(b), dev(S0))
    torch.cuda.synchronize()
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL[dt] and es <= TOL[dt]
    assert torch.equal(o, ob) and torch.equal(S, Sb)


def test_scalar_gate_varlen_matches_oracle():
    H, D = 2, 128
    lengths = [70, 0, 5, 200, 64]
    flush(f"[scalar gate] varlen lengths={lengths} H={H} d={D} bf16")
    q, k, v, a, b, cu = I.packed_inputs(610, np.array(lengths), H, D, D, "bf16")
    cu = np.asarray(cu, dtype=np.int64)
    g = gate_of(a)
    S0 = random_state(np.random.default_rng(3), (len(lengths), H, D, D))
    bf = torch.bfloat16
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, S = kda.chunk_prefill_varlen(dev(q, bf), dev(k, bf), dev(v, bf), dev(g), dev(b), cu_d,
                                    dev(S0))
    torch.cuda.synchronize()
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        o_ref, S_ref = gdn_recurrent(q[None, s:e], k[None, s:e], v[None, s:e], g[None, s:e],
                                     b[None, s:e], S0[n:n + 1])
        assert max_rel_err(host(o)[s:e], o_ref[0]) <= TOL["bf16"], n
        assert max_rel_err(host(S)[n], S_ref[0]) <= TOL["bf16"], n


@pytest.mark.parametrize("dt,dk,dv", [("bf16", 128, 128), ("f32", 64, 128)])
def test_scalar_gate_decode_matches_oracle(dt, dk, dv):
    N, H = 6, 4
    flush(f"[scalar gate] decode N={N} H={H} DK={dk} DV={dv} {dt}")
    q, k, v, a, b = I.decode_inputs(620, N, H, dk, dv, dt)
    g = gate_of(a)
    S0 = random_state(np.random.default_rng(9), (N, H, dk, dv))
    td = tdtype(dt)
    S, Sb = dev(S0), dev(S0)
    x = (dev(q, td), dev(k, td), dev(v, td))
    o = kda.decode_step(*x, dev(g), dev(b), S)
    ob = kda.decode_step(*x, dev(np.broadcast_to(g[..., None], a.shape)), dev(b), Sb)
    torch.cuda.synchronize()
    o_ref, S_ref = gdn_recurrent(q[:, None], k[:, None], v[:, None], g[:, None], b[:, None], S0)
    assert max_rel_err(host(o), o_ref[:, 0]) <= TOL[dt]
    assert max_rel_err(host(S), S_ref) <= TOL[dt]
    assert torch.equal(o, ob) and torch.equal(S, Sb)


@pytest.mark.parametrize("path", PATHS)
def test_scalar_gate_prefill_b1_h32_t8192_head_subset(path, monkeypatch):
    """The B=1, H=32, T=8192, d=128 bf16 prefill shape with a
    scalar gate; heads {0, 31} against the oracle."""
    kda.set_tuning(prefill_form=path)
    B, T, H, D = 1, 8192, 32, 128
    flush(f"[scalar gate] prefill B={B} T={T} H={H} d={D} bf16 path={path}")
    heads = [0, 31]
    q, k, v, a, b = I.batch_inputs(630, B, T, H, D, D, "bf16", heads=heads)
    g = gate_of(a)
    bf = torch.bfloat16
    o, S = kda.chunk_prefill(dev(q, bf), dev(k, bf), dev(v, bf), dev(g), dev(b))
    torch.cuda.synchronize()
    o_ref, S_ref = gdn_recurrent(q[:, :, heads], k[:, :, heads], v[:, :, heads], g[:, :, heads],
                                 b[:, :, heads])
    eo = max_rel_err(host(o)[:, :, heads], o_ref)
    es = max_rel_err(host(S)[:, heads], S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


GRADS = ("dq", "dk", "dv", "dgate", "dbeta", "dS0")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dt,T,d", [("bf16", 200, 128), ("f32", 130, 64), ("bf16", 37, 64)])
def test_scalar_gate_backward_matches_oracle(dt, T, d, path, monkeypatch):
    """Gradients of the scalar-gate prefill (the gate's: one value per
    token-head) against the fp64 oracle, with an initial state and a
    final-state gradient."""
    kda.set_tuning(prefill_form=path)
    B, H = 2, 3
    flush(f"[scalar gate] backward B={B} T={T} H={H} d={d} {dt} path={path}")
    q, k, v, a, b = I.batch_inputs(620 + T, B, T, H, d, d, dt)
    g = gate_of(a)
    rng = np.random.default_rng(T)
    do = rng.standard_normal((B, T, H, d)).astype(np.float32)
    S0 = random_state(rng, (B, H, d, d))
    dST = random_state(rng, (B, H, d, d))
    td = tdtype(dt)
    got = kda.chunk_backward(dev(q, td), dev(k, td), dev(v, td), dev(g), dev(b), dev(do), dev(S0),
                             dev(dST))
    torch.cuda.synchronize()
    assert tuple(got[3].shape) == (B, T, H)
    ref = gdn_backward(q, k, v, g, b, S0, do, dST)
    errs = {n: max_rel_err(host(x), r) for n, x, r in zip(GRADS, got, ref)}
    flush("    " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    assert max(errs.values()) <= TOL[dt], errs


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_scalar_gate_backward_varlen_matches_oracle(dt, d):
    """Packed sequences (empty, short, ragged) with a scalar gate: every
    gradient against the per-sequence oracle."""
    lengths = [70, 0, 5, 128, 33]
    H = 2
    flush(f"[scalar gate] backward varlen lengths={lengths} H={H} d={d} {dt}")
    q, k, v, a, b, cu = I.packed_inputs(640, lengths, H, d, d, dt)
    g = gate_of(a)
    rng = np.random.default_rng(641)
    do = rng.standard_normal((int(cu[-1]), H, d)).astype(np.float32)
    S0 = random_state(rng, (len(lengths), H, d, d))
    dST = random_state(rng, (len(lengths), H, d, d))
    td = tdtype(dt)
    got = kda.chunk_backward_varlen(dev(q, td), dev(k, td), dev(v, td), dev(g), dev(b),
                                    torch.from_numpy(cu).cuda(), dev(do), dev(S0), dev(dST),
                                    max_seqlen=max(lengths))
    torch.cuda.synchronize()
    got = [host(x) for x in got]
    parts = [[] for _ in range(6)]
    for n in range(len(lengths)):
        s_, e_ = cu[n], cu[n + 1]
        sl = lambda x: x[None, s_:e_]  # noqa: E731
        r = gdn_backward(sl(q), sl(k), sl(v), sl(g), sl(b), S0[n:n + 1], sl(do), dST[n:n + 1])
        for i in range(6):
            parts[i].append(r[i][0])
    ref = [np.concatenate(x) for x in parts[:5]] + [np.stack(parts[5])]
    errs = {n: max_rel_err(x, r) for n, x, r in zip(GRADS, got, ref)}
    flush("    " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    assert max(errs.values()) <= TOL[dt], errs


@pytest.mark.parametrize("window", ["1", "2"])
def test_scalar_gate_backward_varlen_windows_are_exact(window, monkeypatch):
    """A scalar gate with the reverse pass in windows of 1 or 2 chunks: bit for
    bit the single-window result (the adjoint carried between windows, the
    gate's gradient summed over the channels within each chunk)."""
    lengths = [150, 0, 64, 3, 129]
    H, d = 2, 64
    flush(f"[scalar gate] backward varlen windows of {window} chunks lengths={lengths}")
    q, k, v, a, b, cu = I.packed_inputs(650, lengths, H, d, d, "bf16")
    g = gate_of(a)
    rng = np.random.default_rng(651)
    do = rng.standard_normal((int(cu[-1]), H, d)).astype(np.float32)
    S0 = random_state(rng, (len(lengths), H, d, d))
    dST = random_state(rng, (len(lengths), H, d, d))
    td = tdtype("bf16")
    x = (dev(q, td), dev(k, td), dev(v, td), dev(g), dev(b), torch.from_numpy(cu).cuda(), dev(do),
         dev(S0), dev(dST))
    ref = kda.chunk_backward_varlen(*x, max_seqlen=max(lengths))
    kda.set_tuning(bwd_window=window)
    got = kda.chunk_backward_varlen(*x, max_seqlen=max(lengths))
    kda.set_tuning(bwd_window=0)
    torch.cuda.synchronize()
    for n, u, w in zip(GRADS, got, ref):
        assert torch.equal(u, w), n
