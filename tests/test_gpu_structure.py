"""GPU structural checks: state orientation and carry at long context
(needle retrieval), state carried across calls, prefill -> decode, packed
sequences == separate calls, determinism, containment of a NaN to its own
(sequence, head), in-place state update, empty inputs.

These are the failure modes the pages warn about for KDA serving: a
recurrent-state layout error in chunked prefill that broke long-context
retrieval while short prompts looked fine ("Kimi Linear、独自の土俵でFull
Attentionを上回る" (remio.ai), risk section), and the recommendation to test
long-prefill retrieval, batched decoding and state behaviour across chunk
boundaries."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host, random_state
from oracle import kda_recurrent, kda_recurrent_varlen, max_rel_err

pytestmark = pytest.mark.gpu
bf = torch.bfloat16


def needle_inputs(T, p, H, D, c):
    """Key e_0 carries a needle written at position p with beta = 1; channel 0
    never decays and no other key touches it; every later query is e_0."""
    q, k, v, a, b = I.batch_inputs(c, 1, T, H, D, D, "bf16")
    k[..., 0] = 0.0
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = I.round_bf16(k)
    a[..., 0] = 1.0
    k[0, p] = 0.0
    k[0, p, :, 0] = 1.0
    b[0, p] = 1.0
    q[0, p + 1:] = 0.0
    q[0, p + 1:, :, 0] = 1.0
    return q, k, v, a, b


@pytest.mark.parametrize("T,p,H", [(4096, 3, 4), (65536, 37, 4), (262144, 131071, 4), (1048576, 700001, 2)])
def test_needle_retrieval_long_context(T, p, H):
    D = 128
    flush(f"[needle] T={T} p={p} H={H}")
    q, k, v, a, b = needle_inputs(T, p, H, D, 700 + p % 7)
    o, S = kda.chunk_prefill(dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b))
    torch.cuda.synchronize()
    on = host(o)[0]
    want = np.broadcast_to(v[0, p][None], (T - p - 1, H, D))
    err = max_rel_err(on[p + 1:], want)
    flush(f"    needle err {err:.2e}")
    assert err <= TOL["bf16"]
    # the state's key-channel-0 row holds the needle (row = key channel)
    assert max_rel_err(host(S)[0, :, 0, :], v[0, p]) <= TOL["bf16"]


def test_split_calls_equal_one_call():
    """prefill(T1) then prefill(T2 | S) == prefill(T1 + T2), with T1 not a
    multiple of the chunk length."""
    B, H, D, T1, T2 = 2, 3, 128, 77, 200
    q, k, v, a, b = I.batch_inputs(800, B, T1 + T2, H, D, D, "bf16")
    S0 = random_state(np.random.default_rng(1), (B, H, D, D))
    t = lambda x, dt=torch.float32: dev(x, dt)  # noqa: E731
    o_full, S_full = kda.chunk_prefill(t(q, bf), t(k, bf), t(v, bf), t(a), t(b), t(S0))
    sl = lambda x, s: np.ascontiguousarray(x[:, s])  # noqa: E731
    s1, s2 = slice(0, T1), slice(T1, T1 + T2)
    o1, S1 = kda.chunk_prefill(t(sl(q, s1), bf), t(sl(k, s1), bf), t(sl(v, s1), bf), t(sl(a, s1)),
                               t(sl(b, s1)), t(S0))
    o2, S2 = kda.chunk_prefill(t(sl(q, s2), bf), t(sl(k, s2), bf), t(sl(v, s2), bf), t(sl(a, s2)),
                               t(sl(b, s2)), S1)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_recurrent(q, k, v, a, b, S0)
    assert max_rel_err(np.concatenate([host(o1), host(o2)], axis=1), o_ref) <= TOL["bf16"]
    assert max_rel_err(host(S2), S_ref) <= TOL["bf16"]
    assert max_rel_err(host(S2), host(S_full)) <= TOL["bf16"]
    assert max_rel_err(np.concatenate([host(o1), host(o2)], axis=1), host(o_full)) <= TOL["bf16"]


def test_prefill_then_decode_equals_longer_prefill():
    B, H, D, T = 3, 2, 128, 130
    q, k, v, a, b = I.batch_inputs(801, B, T + 1, H, D, D, "bf16")
    t = lambda x, dt=torch.float32: dev(x, dt)  # noqa: E731
    o_full, S_full = kda.chunk_prefill(t(q, bf), t(k, bf), t(v, bf), t(a), t(b))
    _, S = kda.chunk_prefill(t(q[:, :T], bf), t(k[:, :T], bf), t(v[:, :T], bf), t(a[:, :T]), t(b[:, :T]))
    od = kda.decode_step(t(q[:, T], bf), t(k[:, T], bf), t(v[:, T], bf), t(a[:, T]), t(b[:, T]), S)
    torch.cuda.synchronize()
    assert max_rel_err(host(od), host(o_full)[:, T]) <= TOL["bf16"]
    assert max_rel_err(host(S), host(S_full)) <= TOL["bf16"]


def test_varlen_equals_separate_calls_and_permutes(monkeypatch):
    """Packed varlen == one fixed-length call per sequence, bitwise, when both
    run the one-kernel form (the staged form computes the same products in
    another order: equal up to rounding); permuting the sequences permutes the
    results."""
    lengths = [300, 64, 0, 1, 129, 65]
    H, D = 2, 128
    q, k, v, a, b, cu = I.packed_inputs(802, lengths, H, D, D, "bf16")
    S0 = random_state(np.random.default_rng(2), (len(lengths), H, D, D))
    t = lambda x, dt=torch.float32: dev(x, dt)  # noqa: E731
    o, S = kda.chunk_prefill_varlen(t(q, bf), t(k, bf), t(v, bf), t(a), t(b),
                                    torch.from_numpy(cu).cuda(), t(S0))
    torch.cuda.synchronize()
    on, Sn = host(o), host(S)
    for n, L in enumerate(lengths):
        s, e = int(cu[n]), int(cu[n + 1])
        if L == 0:
            np.testing.assert_array_equal(Sn[n], S0[n])  # passes the state through
            continue
        args = (t(q[None, s:e], bf), t(k[None, s:e], bf), t(v[None, s:e], bf),
                t(a[None, s:e]), t(b[None, s:e]), t(S0[n:n + 1]))
        kda.set_tuning(prefill_form="fused")
        o1, S1 = kda.chunk_prefill(*args)
        torch.cuda.synchronize()
        # the same kernels on the same data: identical results
        np.testing.assert_array_equal(host(o1)[0], on[s:e])
        np.testing.assert_array_equal(host(S1)[0], Sn[n])
        kda.set_tuning(prefill_form="split")
        o2, S2 = kda.chunk_prefill(*args)
        torch.cuda.synchronize()
        assert max_rel_err(host(o2)[0], on[s:e]) <= 1e-4
        assert max_rel_err(host(S2)[0], Sn[n]) <= 1e-4
        kda.set_tuning(prefill_form="auto")
    perm = [4, 0, 5, 2, 1, 3]
    pl = [lengths[i] for i in perm]
    pcu = np.concatenate([[0], np.cumsum(pl)]).astype(np.int32)
    sl = lambda x: np.concatenate([x[cu[i]:cu[i + 1]] for i in perm], axis=0)  # noqa: E731
    op, Sp = kda.chunk_prefill_varlen(t(sl(q), bf), t(sl(k), bf), t(sl(v), bf), t(sl(a)), t(sl(b)),
                                      torch.from_numpy(pcu).cuda(), t(S0[perm]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(op), sl(on))
    np.testing.assert_array_equal(host(Sp), Sn[perm])
    o_ref, S_ref = kda_recurrent_varlen(q, k, v, a, b, cu, S0)
    assert max_rel_err(on, o_ref) <= TOL["bf16"] and max_rel_err(Sn, S_ref) <= TOL["bf16"]


@pytest.mark.parametrize("path", ["fused", "split"])
def test_deterministic_bitwise(path, monkeypatch):
    kda.set_tuning(prefill_form=path)
    q, k, v, a, b = I.batch_inputs(803, 1, 1000, 8, 128, 128, "bf16")
    args = (dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b))
    o1, S1 = kda.chunk_prefill(*args)
    o2, S2 = kda.chunk_prefill(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    st1 = S1.clone()
    st2 = S1.clone()
    d = I.decode_inputs(803, 1, 8, 128, 128, "bf16")
    da = (dev(d[0], bf), dev(d[1], bf), dev(d[2], bf), dev(d[3]), dev(d[4]))
    x1 = kda.decode_step(*da, st1)
    x2 = kda.decode_step(*da, st2)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2) and torch.equal(st1, st2)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_nan_stays_in_its_own_sequence_and_head(path, monkeypatch):
    kda.set_tuning(prefill_form=path)
    B, T, H, D = 3, 150, 4, 128
    q, k, v, a, b = I.batch_inputs(804, B, T, H, D, D, "bf16")
    v = v.copy()
    v[1, 70, 2, 5] = np.nan
    o, S = kda.chunk_prefill(dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b))
    torch.cuda.synchronize()
    on, Sn = host(o), host(S)
    bad = np.zeros((B, H), bool)
    bad[1, 2] = True
    for bb in range(B):
        for h in range(H):
            finite = np.isfinite(on[bb, :, h]).all() and np.isfinite(Sn[bb, h]).all()
            assert finite != bad[bb, h], (bb, h)
    # Chunks before the NaN's chunk (tokens 0..63) are untouched; inside its
    # own chunk the dense chunk products (0 * NaN = NaN) spread it to earlier
    # tokens too, as the chunk form computes a chunk's tokens together.
    assert np.isfinite(on[1, :64, 2]).all()


def test_in_place_state_and_zero_length():
    B, T, H, D = 2, 100, 2, 64
    q, k, v, a, b = I.batch_inputs(805, B, T, H, D, D, "bf16")
    S0 = random_state(np.random.default_rng(3), (B, H, D, D))
    st = dev(S0)
    o, S = kda.chunk_prefill(dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), st, final_state=st)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_recurrent(q, k, v, a, b, S0)
    assert S.data_ptr() == st.data_ptr()
    assert max_rel_err(host(st), S_ref) <= TOL["bf16"] and max_rel_err(host(o), o_ref) <= TOL["bf16"]
    # T = 0: the state passes through unchanged, nothing is written to o
    z = lambda *s: torch.zeros(s, device="cuda", dtype=bf)  # noqa: E731
    zf = lambda *s: torch.zeros(s, device="cuda")  # noqa: E731
    o0, S1 = kda.chunk_prefill(z(B, 0, H, D), z(B, 0, H, D), z(B, 0, H, D), zf(B, 0, H, D), zf(B, 0, H), dev(S0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(S1), S0)


def test_binding_rejects_bad_arguments():
    x = torch.zeros((1, 64, 2, 96), device="cuda", dtype=bf)
    a = torch.zeros((1, 64, 2, 96), device="cuda")
    b = torch.zeros((1, 64, 2), device="cuda")
    with pytest.raises(kda.KDAError, match="KDA_ERR_UNSUPPORTED"):
        kda.chunk_prefill(x, x, x, a, b)
    with pytest.raises(ValueError):
        kda.chunk_prefill(x.float(), x, x, a, b)


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prefill_at_the_decay_domain_edge(path, dt, monkeypatch):
    """Strong decay, alpha ~ U[0.07, 0.2] on every channel: the product over
    32 tokens reaches ~1e-37, the edge of the data domain the header states
    (the decays are factored through each chunk's row 31).  Output and final
    state against the oracle."""
    kda.set_tuning(prefill_form=path)
    B, T, H, D = 1, 300, 2, 64
    flush(f"[domain] prefill alpha in [0.07, 0.2] T={T} {dt} {path}")
    q, k, v, _, b = I.batch_inputs(880, B, T, H, D, D, dt)
    a = np.random.default_rng(881).uniform(0.07, 0.2, (B, T, H, D)).astype(np.float32)
    S0 = random_state(np.random.default_rng(882), (B, H, D, D))
    td = torch.float32 if dt == "f32" else bf
    o, S = kda.chunk_prefill(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b), dev(S0))
    torch.cuda.synchronize()
    ro, rS = kda_recurrent(q, k, v, a, b, S0)
    e = (max_rel_err(host(o), ro), max_rel_err(host(S), rS))
    flush(f"    o={e[0]:.1e} S={e[1]:.1e}")
    assert np.isfinite(host(o)).all() and max(e) <= TOL[dt], e
