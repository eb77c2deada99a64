"""GPU parity of the backward pass against the fp64 oracle's reverse mode:
every gradient (q, k, v, alpha, beta, initial state) with and without an
initial state and a final-state gradient, both forward forms feeding the
checkpoints, ragged last chunks, and the 8192-token 32-head shape."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host, random_state, tdtype
from oracle import kda_backward, kda_recurrent, max_rel_err

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def run_case(B, T, H, dk, dv, dt, c, with_state, heads=None):
    q, k, v, a, b = I.batch_inputs(c, B, T, H, dk, dv, dt)
    rng = np.random.default_rng(c)
    do = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    S0 = random_state(rng, (B, H, dk, dv)) if with_state else None
    dST = random_state(rng, (B, H, dk, dv)) if with_state else None
    td = tdtype(dt)
    got = kda.chunk_backward(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b), dev(do),
                             None if S0 is None else dev(S0), None if dST is None else dev(dST))
    torch.cuda.synchronize()
    got = [host(g) for g in got]
    if heads is not None:
        sel = lambda x: x[:, :, heads]  # noqa: E731
        ref = kda_backward(sel(q), sel(k), sel(v), sel(a), b[:, :, heads], None, sel(do), None)
        got = [g[:, :, heads] if g.ndim == 4 and g.shape[1] == T else
               (g[:, :, heads] if g.ndim == 3 else g[:, heads]) for g in got]
    else:
        ref = kda_backward(q, k, v, a, b, S0, do, dST)
    errs = {n: max_rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    flush("    " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    return errs


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_backward_matches_oracle(dt, d, T, path, monkeypatch):
    kda.set_tuning(prefill_form=path)
    flush(f"[backward] B=2 T={T} H=3 d={d} {dt} path={path}")
    errs = run_case(2, T, 3, d, d, dt, 700 + T, with_state=True)
    assert max(errs.values()) <= TOL[dt], errs


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_backward_rectangular_zero_state(dk, dv):
    flush(f"[backward] B=1 T=130 H=2 DK={dk} DV={dv} bf16, zero state, no final-state gradient")
    errs = run_case(1, 130, 2, dk, dv, "bf16", 710, with_state=False)
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_is_deterministic():
    B, T, H, D = 1, 300, 4, 128
    flush(f"[backward] determinism B={B} T={T} H={H} d={D}")
    q, k, v, a, b = I.batch_inputs(720, B, T, H, D, D, "bf16")
    do = np.random.default_rng(1).standard_normal((B, T, H, D)).astype(np.float32)
    bf = torch.bfloat16
    x = (dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), dev(do))
    g1 = kda.chunk_backward(*x)
    g2 = kda.chunk_backward(*x)
    torch.cuda.synchronize()
    for u, w in zip(g1, g2):
        assert torch.equal(u, w)


def test_backward_b1_h32_t8192_head_subset():
    """The B=1, H=32, T=8192, d=128 bf16 prefill shape; heads {0, 31} against the oracle."""
    flush("[backward] B=1 T=8192 H=32 d=128 bf16, heads 0 and 31")
    errs = run_case(1, 8192, 32, 128, 128, "bf16", 730, with_state=False, heads=[0, 31])
    assert max(errs.values()) <= TOL["bf16"], errs


def varlen_backward_reference(q, k, v, a, b, cu, do, S0, dST):
    """Per-sequence oracle gradients, packed in sequence order."""
    outs = [[] for _ in range(6)]
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        sl = lambda x: x[None, s:e]  # noqa: E731
        g = kda_backward(sl(q), sl(k), sl(v), sl(a), sl(b), S0[n:n + 1], sl(do), dST[n:n + 1])
        for i in range(5):
            outs[i].append(g[i][0])
        outs[5].append(g[5][0])
    return [np.concatenate(o) for o in outs[:5]] + [np.stack(outs[5])]


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_backward_varlen_matches_oracle(dt, d):
    """Packed sequences of mixed lengths (empty, shorter than a chunk, exactly
    one chunk, ragged multi-chunk), random initial states and final-state
    gradients: every gradient against the per-sequence oracle."""
    lengths = [37, 0, 64, 1, 200, 129]
    H = 3
    flush(f"[backward] varlen lengths={lengths} H={H} d={d} {dt}")
    q, k, v, a, b, cu = I.packed_inputs(730, lengths, H, d, d, dt)
    rng = np.random.default_rng(731)
    do = rng.standard_normal((int(cu[-1]), H, d)).astype(np.float32)
    S0 = random_state(rng, (len(lengths), H, d, d))
    dST = random_state(rng, (len(lengths), H, d, d))
    td = tdtype(dt)
    got = kda.chunk_backward_varlen(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b),
                                    torch.from_numpy(cu).cuda(), dev(do), dev(S0), dev(dST),
                                    max_seqlen=max(lengths))
    torch.cuda.synchronize()
    got = [host(g) for g in got]
    ref = varlen_backward_reference(q, k, v, a, b, cu, do, S0, dST)
    errs = {n: max_rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    flush("    " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    assert max(errs.values()) <= TOL[dt], errs
    # the empty sequence passes the final-state gradient through unchanged
    assert np.array_equal(got[5][1], dST[1].astype(np.float32))


def test_backward_varlen_equals_fixed_length_call(monkeypatch):
    """Equal-length packed sequences give the fixed-length backward (both
    forwards in the one-kernel form, so the checkpoints agree)."""
    kda.set_tuning(prefill_form="fused")
    B, T, H, D = 3, 150, 2, 128
    flush(f"[backward] varlen == fixed B={B} T={T} H={H} d={D}")
    q, k, v, a, b = I.batch_inputs(740, B, T, H, D, D, "bf16")
    do = np.random.default_rng(741).standard_normal((B, T, H, D)).astype(np.float32)
    S0 = random_state(np.random.default_rng(742), (B, H, D, D))
    bf = torch.bfloat16
    x = [dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), dev(do)]
    g_fix = kda.chunk_backward(*x[:5], x[5], dev(S0), None)
    flat = [t.reshape(B * T, *t.shape[2:]).contiguous() for t in x]
    cu = torch.tensor([0, T, 2 * T, 3 * T], dtype=torch.int32, device="cuda")
    g_var = kda.chunk_backward_varlen(*flat[:5], cu, flat[5], dev(S0), None, max_seqlen=T)
    torch.cuda.synchronize()
    for gf, gv in zip(g_fix[:5], g_var[:5]):
        err = max_rel_err(host(gv), host(gf).reshape(host(gv).shape))
        assert err <= 1e-6, err
    assert max_rel_err(host(g_var[5]), host(g_fix[5])) <= 1e-6


@pytest.mark.parametrize("varlen", [False, True])
def test_backward_without_tokens_passes_state_gradient(varlen):
    """T = 0: the initial state's gradient is the final state's."""
    N, H, D = 2, 3, 64
    flush(f"[backward] no tokens N={N} H={H} d={D} varlen={varlen}")
    dST = random_state(np.random.default_rng(750), (N, H, D, D))
    e = torch.empty((0, H, D), device="cuda", dtype=torch.float32)
    if varlen:
        cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
        g = kda.chunk_backward_varlen(e, e, e, e, torch.empty((0, H), device="cuda"), cu, e,
                                      None, dev(dST), max_seqlen=0)
    else:
        e4 = torch.empty((N, 0, H, D), device="cuda", dtype=torch.float32)
        g = kda.chunk_backward(e4, e4, e4, e4, torch.empty((N, 0, H), device="cuda"), e4, None,
                               dev(dST))
    torch.cuda.synchronize()
    assert torch.equal(g[5], dev(dST))


@pytest.mark.parametrize("window", ["1", "3"])
def test_backward_windows_are_exact(window, monkeypatch):
    """The reverse pass in windows of 1 or 3 chunks (the adjoint carried
    between launches, each window's first chunk recomputed from its
    checkpoint) gives bit for bit the single-window result."""
    B, T, H, D = 2, 200, 3, 128
    flush(f"[backward] windows of {window} chunks B={B} T={T} H={H} d={D}")
    q, k, v, a, b = I.batch_inputs(760, B, T, H, D, D, "bf16")
    rng = np.random.default_rng(761)
    do = rng.standard_normal((B, T, H, D)).astype(np.float32)
    S0 = random_state(rng, (B, H, D, D))
    dST = random_state(rng, (B, H, D, D))
    bf = torch.bfloat16
    x = (dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), dev(do), dev(S0), dev(dST))
    ref = kda.chunk_backward(*x)
    kda.set_tuning(bwd_window=window)
    got = kda.chunk_backward(*x)
    g_gate = kda.chunk_backward(*x[:3], x[3][..., 0].contiguous(), *x[4:])
    kda.set_tuning(bwd_window=0)
    r_gate = kda.chunk_backward(*x[:3], x[3][..., 0].contiguous(), *x[4:])
    torch.cuda.synchronize()
    for n, u, w in zip(NAMES, got, ref):
        assert torch.equal(u, w), n
    for n, u, w in zip(NAMES, g_gate, r_gate):
        assert torch.equal(u, w), n


@pytest.mark.parametrize("window,max_seqlen", [("1", 200), ("2", 0), ("1", 0)])
def test_backward_varlen_windows_are_exact(window, max_seqlen, monkeypatch):
    """Packed sequences in windows (with the longest length given, or unknown:
    then windows past every sequence's start do nothing) against the
    single-window call, bit for bit, and against the oracle."""
    lengths = [37, 0, 64, 1, 200, 129]
    H, D = 2, 64
    flush(f"[backward] varlen windows of {window} chunks, max_seqlen={max_seqlen} lengths={lengths}")
    q, k, v, a, b, cu = I.packed_inputs(770, lengths, H, D, D, "f32")
    rng = np.random.default_rng(771)
    do = rng.standard_normal((int(cu[-1]), H, D)).astype(np.float32)
    S0 = random_state(rng, (len(lengths), H, D, D))
    dST = random_state(rng, (len(lengths), H, D, D))
    x = (dev(q), dev(k), dev(v), dev(a), dev(b), torch.from_numpy(cu).cuda(), dev(do), dev(S0),
         dev(dST))
    ref = kda.chunk_backward_varlen(*x, max_seqlen=0)   # unknown: T_total assumed
    kda.set_tuning(bwd_window=window)
    got = kda.chunk_backward_varlen(*x, max_seqlen=max_seqlen)
    kda.set_tuning(bwd_window=0)
    torch.cuda.synchronize()
    for n, u, w in zip(NAMES, got, ref):
        assert torch.equal(u, w), n
    oref = varlen_backward_reference(q, k, v, a, b, cu, do, S0, dST)
    errs = {n: max_rel_err(host(u), r) for n, u, r in zip(NAMES, got, oref)}
    assert max(errs.values()) <= TOL["f32"], errs


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_at_the_decay_domain_edge(dt):
    """Strong decay, alpha ~ U[0.07, 0.2]: the backward's relative decays reach
    ~1e36 within a chunk (the same factoring as the forward).  Every gradient
    against the oracle."""
    B, T, H, D = 1, 200, 2, 64
    flush(f"[backward] alpha in [0.07, 0.2] T={T} {dt}")
    q, k, v, _, b = I.batch_inputs(890, B, T, H, D, D, dt)
    rng = np.random.default_rng(891)
    a = rng.uniform(0.07, 0.2, (B, T, H, D)).astype(np.float32)
    do = rng.standard_normal((B, T, H, D)).astype(np.float32)
    S0 = random_state(rng, (B, H, D, D))
    dST = random_state(rng, (B, H, D, D))
    td = tdtype(dt)
    got = kda.chunk_backward(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b), dev(do),
                             dev(S0), dev(dST))
    torch.cuda.synchronize()
    got = [host(g) for g in got]
    ref = kda_backward(q, k, v, a, b, S0, do, dST)
    errs = {n: max_rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    flush("    " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    assert all(np.isfinite(g).all() for g in got) and max(errs.values()) <= TOL[dt], errs


def test_prefill_and_backward_with_beta_outside_0_1():
    """beta ~ U[-0.5, 1.5] (any finite beta keeps I + Diag(beta) X unit lower
    triangular): the prefill's output and state and every gradient against
    the oracle."""
    B, T, H, D = 1, 150, 2, 64
    flush(f"[backward] beta in [-0.5, 1.5] T={T} f32")
    q, k, v, a, _ = I.batch_inputs(895, B, T, H, D, D, "f32")
    rng = np.random.default_rng(896)
    b = rng.uniform(-0.5, 1.5, (B, T, H)).astype(np.float32)
    do = rng.standard_normal((B, T, H, D)).astype(np.float32)
    S0 = random_state(rng, (B, H, D, D))
    dST = random_state(rng, (B, H, D, D))
    x = (dev(q), dev(k), dev(v), dev(a), dev(b))
    o, S = kda.chunk_prefill(*x, dev(S0))
    got = kda.chunk_backward(*x, dev(do), dev(S0), dev(dST))
    torch.cuda.synchronize()
    ro, rS = kda_recurrent(q, k, v, a, b, S0)
    ref = kda_backward(q, k, v, a, b, S0, do, dST)
    errs = {"o": max_rel_err(host(o), ro), "S": max_rel_err(host(S), rS)}
    errs.update({n: max_rel_err(host(g), r) for n, g, r in zip(NAMES, got, ref)})
    flush("    " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    assert max(errs.values()) <= TOL["f32"], errs


@pytest.mark.parametrize("window", [None, "1"])
def test_backward_varlen_rectangular(window, monkeypatch):
    """Packed sequences with d_k = 64, d_v = 128 (four waves per chain
    workgroup, eight value slabs), in one window or in windows of one chunk:
    every gradient against the per-sequence oracle."""
    lengths = [70, 0, 128, 5, 193]
    H, dk, dv = 2, 64, 128
    flush(f"[backward] varlen rectangular dk={dk} dv={dv} window={window} lengths={lengths}")
    q, k, v, a, b, cu = I.packed_inputs(900, lengths, H, dk, dv, "bf16")
    rng = np.random.default_rng(901)
    do = rng.standard_normal((int(cu[-1]), H, dv)).astype(np.float32)
    S0 = random_state(rng, (len(lengths), H, dk, dv))
    dST = random_state(rng, (len(lengths), H, dk, dv))
    td = tdtype("bf16")
    if window:
        kda.set_tuning(bwd_window=window)
    got = kda.chunk_backward_varlen(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b),
                                    torch.from_numpy(cu).cuda(), dev(do), dev(S0), dev(dST),
                                    max_seqlen=max(lengths))
    torch.cuda.synchronize()
    ref = varlen_backward_reference(q, k, v, a, b, cu, do, S0, dST)
    errs = {n: max_rel_err(host(g), r) for n, g, r in zip(NAMES, got, ref)}
    flush("    " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_varlen_max_seqlen_below_the_longest():
    """max_seqlen below the longest sequence (one window of 2 chunks, so no
    adjoint carry buffer): the call completes, sequences that fit get every
    gradient, and a longer sequence gets the right gradients on its last two
    chunks (the header: earlier tokens and its initial-state gradient are not
    written)."""
    lengths = [130, 40, 300]
    H, d = 2, 64
    flush(f"[backward] varlen max_seqlen=100 below the longest, lengths={lengths} H={H} d={d}")
    q, k, v, a, b, cu = I.packed_inputs(780, lengths, H, d, d, "f32")
    rng = np.random.default_rng(781)
    do = rng.standard_normal((int(cu[-1]), H, d)).astype(np.float32)
    S0 = random_state(rng, (len(lengths), H, d, d))
    dST = random_state(rng, (len(lengths), H, d, d))
    got = kda.chunk_backward_varlen(dev(q), dev(k), dev(v), dev(a), dev(b),
                                    torch.from_numpy(cu).cuda(), dev(do), dev(S0), dev(dST),
                                    max_seqlen=100)
    torch.cuda.synchronize()
    got = [host(g) for g in got]
    for n, first in [(0, 64), (1, 0), (2, 192)]:   # first token whose chunk is covered
        s_, e_ = int(cu[n]), int(cu[n + 1])
        sl = lambda x: x[None, s_:e_]  # noqa: E731
        ref = kda_backward(sl(q), sl(k), sl(v), sl(a), sl(b), S0[n:n + 1], sl(do), dST[n:n + 1])
        for nm, g, r in zip(NAMES[:5], got[:5], ref[:5]):
            err = max_rel_err(g[s_ + first:e_], r[0, first:])
            assert err <= TOL["f32"], (n, nm, err)
        if first == 0:
            assert max_rel_err(got[5][n], ref[5][0]) <= TOL["f32"], n
