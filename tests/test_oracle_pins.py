"""Pins for the fp64 oracle: every check compares it with something other
than itself (closed forms, special cases that reduce to DeltaNet, Gated
DeltaNet and linear attention, exact-rational brute force through dense
transition matrices, hand-derived values, invariants).

Sources: "Kimi Delta Attention 徹底解説" (tech-tide.dev) sections
"なぜ今「線形アテンション」なのか" and "Kimi Delta Attention の仕組み";
"Kimi Linear、独自の土俵でFull Attentionを上回る" (remio.ai) sections
"Kimi Linearがより賢いRecurrent Memoryを使う方法" and
"オープンコード…リスク" (state layout, chunk boundaries, batching, needle).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (gdn_backward, gdn_recurrent, kda_backward, kda_chunked, kda_decode_pool,
                    kda_decode_step, kda_recurrent, kda_recurrent_snapshots, kda_recurrent_varlen,
                    max_rel_err)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, T, H, DK, DV, s0=True):
    q = rng.standard_normal((B, T, H, DK))
    k = rng.standard_normal((B, T, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    a = np.exp(-np.exp(rng.uniform(-5, -1, (B, T, H, DK))))
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, DK, DV)) if s0 else None
    return q, k, v, a, b, S0


# ---------------------------------------------------------------- golden ---
def test_golden_hand_worked():
    """Hand-derived values (fixture cites its derivation from the explainer's
    definition of the recurrence)."""
    with open(os.path.join(GOLDEN, "hand_worked_kda.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        q = np.array(case["q"], float)[None, :, None, :]
        k = np.array(case["k"], float)[None, :, None, :]
        v = np.array(case["v"], float)[None, :, None, :]
        a = np.array(case["alpha"], float)[None, :, None, :]
        b = np.array(case["beta"], float)[None, :, None]
        S0 = np.array(case["S0"], float)[None, None]
        o, S = kda_recurrent(q, k, v, a, b, S0)
        np.testing.assert_allclose(o[0, :, 0], np.array(case["o"], float), rtol=0, atol=1e-15)
        np.testing.assert_allclose(S[0, 0], np.array(case["S_final"], float), rtol=0, atol=1e-15)


# ------------------------------------------------------------------- P1 ---
@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 300])
def test_p1_chunk_form_equals_recurrence(chunk):
    """The chunked regrouping reaches the token recurrence's result (the
    explainer: both modes come from one formulation), for any chunk size,
    partial last chunk and a non-zero incoming state."""
    rng = np.random.default_rng(1)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, 203, 2, 12, 9)
    o_r, S_r = kda_recurrent(q, k, v, a, b, S0)
    o_c, S_c = kda_chunked(q, k, v, a, b, S0, chunk=chunk)
    assert max_rel_err(o_c, o_r) < 1e-12
    assert max_rel_err(S_c, S_r) < 1e-12


# ------------------------------------------------------------------- P2 ---
def test_p2_beta_zero_is_decay_only():
    """beta = 0 writes nothing: only the channel-wise forget acts, so
    S_T = Diag(prod_t alpha_t) S0 and o_t = (Diag(gamma_t) S0)^T q_t."""
    rng = np.random.default_rng(2)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 40, 3, 8, 5)
    b[:] = 0.0
    o, S = kda_recurrent(q, k, v, a, b, S0)
    gam = np.cumprod(a, axis=1)  # [B,T,H,DK]
    o_cf = np.einsum("bthk,bhkv,bthk->bthv", gam, S0, q)
    S_cf = gam[:, -1][..., None] * S0
    assert max_rel_err(o, o_cf) < 1e-13
    assert max_rel_err(S, S_cf) < 1e-13


def test_p2_decay_acts_on_key_channels():
    """One channel forgets completely fast, the rest keep: only that row of S
    shrinks (the gate is per key channel, i.e. per row of S)."""
    DK, DV, T = 4, 3, 5
    S0 = np.arange(1, DK * DV + 1, dtype=float).reshape(1, 1, DK, DV)
    a = np.ones((1, T, 1, DK))
    a[..., 2] = 0.5
    q = np.zeros((1, T, 1, DK))
    k = np.zeros((1, T, 1, DK))
    k[..., 0] = 1.0
    v = np.zeros((1, T, 1, DV))
    b = np.zeros((1, T, 1))
    _, S = kda_recurrent(q, k, v, a, b, S0)
    expect = S0.copy()
    expect[0, 0, 2] *= 0.5 ** T
    np.testing.assert_array_equal(S, expect)


# ------------------------------------------------------------------- P3 ---
def test_p3_delta_rule_exact_replacement():
    """alpha = 1, beta = 1 (DeltaNet): after writing v under a unit key the
    state returns exactly v for that key, and rewriting a key replaces its
    value instead of adding to it (the explainer's contrast of additive
    linear attention with the delta rule)."""
    rng = np.random.default_rng(3)
    DK, DV = 16, 6
    Q, _ = np.linalg.qr(rng.standard_normal((DK, DK)))
    keys = Q.T[:5]                      # 5 orthonormal keys
    vals = rng.standard_normal((5, DV))
    newv = rng.standard_normal(DV)
    seq_k = np.concatenate([keys, keys[1:2]])          # rewrite key 1 at the end
    seq_v = np.concatenate([vals, newv[None]])
    T = len(seq_k)
    k = seq_k[None, :, None, :]
    v = seq_v[None, :, None, :]
    a = np.ones((1, T, 1, DK))
    b = np.ones((1, T, 1))
    q = k.copy()
    o, S = kda_recurrent(q, k, v, a, b)
    # reading with the key just written returns the value just written
    np.testing.assert_allclose(o[0, :, 0], seq_v, atol=1e-13)
    # afterwards: key 1 holds the new value only, other keys keep theirs
    expect = vals.copy()
    expect[1] = newv
    np.testing.assert_allclose(keys @ S[0, 0], expect, atol=1e-13)


def test_p3_prediction_error_is_zero_after_write():
    """With alpha = 1, beta = 1 and a unit key, S_t^T k_t = v_t for any prior
    state: the write removes the whole prediction error."""
    rng = np.random.default_rng(31)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 1, 4, 10, 7)
    a[:] = 1.0
    b[:] = 1.0
    _, S = kda_recurrent(q, k, v, a, b, S0)
    np.testing.assert_allclose(np.einsum("bhkv,bhk->bhv", S, k[:, 0]), v[:, 0], atol=1e-13)


# ------------------------------------------------------------------- P4 ---
def test_p4_scalar_gate_is_gated_deltanet():
    """With alpha_t the same for every channel, KDA is Gated DeltaNet:
    S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T (decay the
    whole state by one scalar, then the delta write)."""
    rng = np.random.default_rng(4)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 30, 2, 8, 5)
    sc = a[..., :1]
    a = np.broadcast_to(sc, a.shape).copy()
    o, S = kda_recurrent(q, k, v, a, b, S0)
    DK = q.shape[-1]
    for h in range(2):
        St = S0[0, h].copy()
        for t in range(30):
            kt = k[0, t, h]
            M = sc[0, t, h, 0] * (np.eye(DK) - b[0, t, h] * np.outer(kt, kt))
            St = M @ St + b[0, t, h] * np.outer(kt, v[0, t, h])
            np.testing.assert_allclose(o[0, t, h], St.T @ q[0, t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


def test_p4_gdn_oracle_dense_transition():
    """The scalar-gate oracle against the dense transition written out:
    S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t;
    with a gate that varies across tokens and heads."""
    rng = np.random.default_rng(41)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, 25, 3, 6, 4)
    g = a[..., 0]
    o, S = gdn_recurrent(q, k, v, g, b, S0)
    DK = q.shape[-1]
    for bb in range(2):
        for h in range(3):
            St = S0[bb, h].copy()
            for t in range(25):
                kt = k[bb, t, h]
                St = g[bb, t, h] * (np.eye(DK) - b[bb, t, h] * np.outer(kt, kt)) @ St \
                    + b[bb, t, h] * np.outer(kt, v[bb, t, h])
                np.testing.assert_allclose(o[bb, t, h], St.T @ q[bb, t, h], atol=1e-12)
            np.testing.assert_allclose(S[bb, h], St, atol=1e-12)


def test_p4_gdn_oracle_gate_one_is_deltanet_and_zero_write_is_decay():
    """gate = 1: DeltaNet (exact replacement under unit keys); beta = 0: the
    state is the product of the gates times S0."""
    rng = np.random.default_rng(42)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 12, 2, 5, 3)
    g = a[..., 0]
    _, S = gdn_recurrent(q, k, v, g, np.zeros_like(b), S0)
    np.testing.assert_allclose(S, np.prod(g, axis=1)[..., None, None] * S0, rtol=1e-13)
    Q, _ = np.linalg.qr(rng.standard_normal((5, 5)))
    kk = np.broadcast_to(Q.T[None, :, None, :], (1, 5, 2, 5)).copy()
    vv = rng.standard_normal((1, 5, 2, 3))
    o, _ = gdn_recurrent(kk, kk, vv, np.ones((1, 5, 2)), np.ones((1, 5, 2)))
    np.testing.assert_allclose(o, vv, atol=1e-13)


# ------------------------------------------------------------------- P5 ---
def test_p5_orthogonal_keys_reduce_to_linear_attention():
    """alpha = 1 and mutually orthogonal keys (not unit length): the delta
    rule never sees a prediction, so KDA is linear attention,
    o_t = sum_{i<=t} beta_i <k_i|q_t> v_i (the re-association of the
    explainer's linear-attention section)."""
    rng = np.random.default_rng(5)
    DK, DV, T = 12, 4, 9
    Q, _ = np.linalg.qr(rng.standard_normal((DK, DK)))
    keys = Q.T[:T] * rng.uniform(0.5, 2.0, (T, 1))
    q = rng.standard_normal((1, T, 1, DK))
    v = rng.standard_normal((1, T, 1, DV))
    b = rng.uniform(0.1, 1.0, (1, T, 1))
    a = np.ones((1, T, 1, DK))
    o, _ = kda_recurrent(q, keys[None, :, None, :], v, a, b)
    for t in range(T):
        ref = sum(b[0, i, 0] * (keys[i] @ q[0, t, 0]) * v[0, i, 0] for i in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], ref, atol=1e-13)


# ------------------------------------------------------------------- P6 ---
def _dyadic(rng, shape, choices):
    return np.array([Fraction(choices[i]) for i in rng.integers(0, len(choices), size=int(np.prod(shape)))],
                    dtype=object).reshape(shape)


def _brute_transitions(q, k, v, a, b, S0):
    """Multiply out S_t = A_t S_{t-1} + beta_t k_t v_t^T with the explicit
    d_k x d_k transition A_t = Diag(alpha_t) - beta_t k_t (alpha_t * k_t)^T
    (the diagonal-plus-low-rank transition), in whatever number type the
    arrays hold."""
    T, DK = k.shape
    S = S0.copy()
    outs = []
    for t in range(T):
        A = np.zeros((DK, DK), dtype=object)
        for i in range(DK):
            for j in range(DK):
                A[i, j] = (a[t, i] if i == j else 0) - b[t] * k[t, i] * a[t, j] * k[t, j]
        S = A.dot(S) + b[t] * np.outer(k[t], v[t])
        outs.append(S.T.dot(q[t]))
    return np.array(outs), S


def test_p6_exact_rational_brute_force():
    """Exact arithmetic on dyadic inputs (T <= 16, d = 4): the fp64 oracle
    must agree with the exact dense-transition product to rounding."""
    rng = np.random.default_rng(6)
    T, DK, DV = 16, 4, 3
    vals = ["-1", "-1/2", "-1/4", "0", "1/4", "1/2", "3/4", "1"]
    q = _dyadic(rng, (T, DK), vals)
    k = _dyadic(rng, (T, DK), vals)
    v = _dyadic(rng, (T, DV), vals + ["2", "-3"])
    a = _dyadic(rng, (T, DK), ["1/4", "1/2", "3/4", "7/8", "1"])
    b = _dyadic(rng, (T,), ["0", "1/4", "1/2", "1", "3/2"])
    S0 = _dyadic(rng, (DK, DV), vals)
    o_ex, S_ex = _brute_transitions(q, k, v, a, b, S0)
    f = lambda x: np.array(x, dtype=float)  # noqa: E731
    o, S = kda_recurrent(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                         f(a)[None, :, None], f(b)[None, :, None], f(S0)[None, None])
    o_ex, S_ex = f(o_ex), f(S_ex)
    assert max_rel_err(o[0, :, 0], o_ex) < 1e-14
    assert max_rel_err(S[0, 0], S_ex) < 1e-14


def test_p6_dense_transition_fp64_d64():
    """The same dense-transition route in fp64 at d = 64."""
    rng = np.random.default_rng(61)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 12, 1, 64, 64)
    o, S = kda_recurrent(q, k, v, a, b, S0)
    S_ref = S0[0, 0]
    for t in range(12):
        kt, at, bt = k[0, t, 0], a[0, t, 0], b[0, t, 0]
        A = np.diag(at) - bt * np.outer(kt, at * kt)
        S_ref = A @ S_ref + bt * np.outer(kt, v[0, t, 0])
        np.testing.assert_allclose(o[0, t, 0], S_ref.T @ q[0, t, 0], rtol=0, atol=1e-12)
    assert max_rel_err(S[0, 0], S_ref) < 1e-13


# ------------------------------------------------------------------- P7 ---
def test_p7_linear_in_values_and_state():
    """For fixed keys, gates and queries, (V, S0) -> (O, S_T) is linear."""
    rng = np.random.default_rng(7)
    q, k, v1, a, b, S1 = rand_inputs(rng, 1, 50, 2, 8, 6)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    c1, c2 = 0.7, -1.9
    o1, T1 = kda_recurrent(q, k, v1, a, b, S1)
    o2, T2 = kda_recurrent(q, k, v2, a, b, S2)
    o3, T3 = kda_recurrent(q, k, c1 * v1 + c2 * v2, a, b, c1 * S1 + c2 * S2)
    assert max_rel_err(o3, c1 * o1 + c2 * o2) < 1e-12
    assert max_rel_err(T3, c1 * T1 + c2 * T2) < 1e-12


# ------------------------------------------------------------------- P8 ---
def needle_inputs(T, p, DK, DV, rng):
    """Needle under key e_0 at position p; channel 0 never decays and no other
    key touches it.  Any read with q = e_0 after p must return the needle."""
    q, k, v, a, b, _ = rand_inputs(rng, 1, T, 1, DK, DV, s0=False)
    k[..., 0] = 0.0
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    a[..., 0] = 1.0
    k[0, p, 0] = 0.0
    k[0, p, 0, 0] = 1.0
    b[0, p, 0] = 1.0
    q[0, p + 1:, 0] = 0.0
    q[0, p + 1:, 0, 0] = 1.0
    return q, k, v, a, b


def test_p8_needle_retrieval_and_orientation():
    """A needle written early is read back exactly at every later position
    (the long-context retrieval failure that a transposed state layout caused
    in a serving stack); reading a column instead of a row fails this."""
    rng = np.random.default_rng(8)
    T, p, DK, DV = 3000, 17, 8, 5
    q, k, v, a, b = needle_inputs(T, p, DK, DV, rng)
    o, S = kda_recurrent(q, k, v, a, b)
    np.testing.assert_array_equal(o[0, p + 1:, 0], np.broadcast_to(v[0, p, 0], (T - p - 1, DV)))
    np.testing.assert_array_equal(S[0, 0, 0], v[0, p, 0])


# ------------------------------------------------------------------- P9 ---
def test_p9_split_calls_and_prefill_then_decode():
    """State carried across calls: prefill(T1) then prefill(T2 | S) equals
    prefill(T1+T2); prefill(T) then one decode step equals prefill(T+1) at
    token T+1 (checked through the independent chunk form)."""
    rng = np.random.default_rng(9)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, 130, 2, 8, 6)
    o_full, S_full = kda_chunked(q, k, v, a, b, S0, chunk=64)
    o1, S1 = kda_recurrent(q[:, :77], k[:, :77], v[:, :77], a[:, :77], b[:, :77], S0)
    o2, S2 = kda_recurrent(q[:, 77:129], k[:, 77:129], v[:, 77:129], a[:, 77:129], b[:, 77:129], S1)
    od, Sd = kda_decode_step(q[:, 129], k[:, 129], v[:, 129], a[:, 129], b[:, 129], S2)
    assert max_rel_err(np.concatenate([o1, o2, od[:, None]], axis=1), o_full) < 1e-12
    assert max_rel_err(Sd, S_full) < 1e-12


# ------------------------------------------------------------------ P10 ---
def test_p10_varlen_equals_separate_and_permutes():
    """Packed sequences behave as separate calls (nothing crosses a sequence
    boundary), zero-length sequences pass their state through, and permuting
    the packed sequences permutes the outputs."""
    rng = np.random.default_rng(10)
    lens = [5, 0, 70, 1, 64, 33]
    H, DK, DV = 2, 8, 4
    parts = [rand_inputs(rng, 1, L, H, DK, DV) for L in lens]
    cat = lambda i: np.concatenate([p[i][0] for p in parts], axis=0)  # noqa: E731
    q, k, v, a = cat(0), cat(1), cat(2), cat(3)
    b = np.concatenate([p[4][0] for p in parts], axis=0)
    S0 = np.concatenate([p[5] for p in parts], axis=0)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = kda_recurrent_varlen(q, k, v, a, b, cu, S0)
    for n, p in enumerate(parts):
        on, Sn = kda_chunked(*p[:5], p[5], chunk=16)
        assert max_rel_err(o[cu[n]:cu[n + 1]], on[0]) < 1e-12
        assert max_rel_err(S[n], Sn[0]) < 1e-12
    np.testing.assert_array_equal(S[1], S0[1])
    perm = [3, 0, 5, 2, 1, 4]
    pl = [lens[i] for i in perm]
    pcu = np.concatenate([[0], np.cumsum(pl)])
    sl = lambda x: np.concatenate([x[cu[i]:cu[i + 1]] for i in perm], axis=0)  # noqa: E731
    op, Sp = kda_recurrent_varlen(sl(q), sl(k), sl(v), sl(a), sl(b), pcu, S0[perm])
    np.testing.assert_array_equal(op, sl(o))
    np.testing.assert_array_equal(Sp, S[perm])


# -------------------------------------------------------------- domain ---
# ------------------------------------------------------------------ P11 ---
def test_p11_snapshots_one_hot_keys_closed_form():
    """alpha = 1, beta = 1, one-hot keys e_c: each write replaces row c of the
    state with the value written, so the state after any prefix is known in
    closed form (row c = value of the last token keyed c, else the initial
    row).  Snapshot j must be that state after exactly L (j + 1) tokens,
    L = chunk * every; the ragged tail gets no snapshot."""
    rng = np.random.default_rng(11)
    B, H, DK, DV, chunk, every = 2, 2, 6, 5, 4, 2
    L = chunk * every
    T = 3 * L + 5
    ch = rng.integers(0, DK, (B, T, H))
    k = np.zeros((B, T, H, DK))
    for b_ in range(B):
        for t in range(T):
            for h in range(H):
                k[b_, t, h, ch[b_, t, h]] = 1.0
    v = rng.standard_normal((B, T, H, DV))
    q = rng.standard_normal((B, T, H, DK))
    a = np.ones((B, T, H, DK))
    bt = np.ones((B, T, H))
    S0 = rng.standard_normal((B, H, DK, DV))
    o, ST, snaps = kda_recurrent_snapshots(q, k, v, a, bt, every, S0, chunk=chunk)
    assert snaps.shape == (B, 3, H, DK, DV)
    for b_ in range(B):
        for h in range(H):
            S = S0[b_, h].copy()
            for t in range(T):
                S[ch[b_, t, h]] = v[b_, t, h]       # the replacement, written out
                np.testing.assert_allclose(o[b_, t, h], q[b_, t, h] @ S, atol=1e-13)
                if (t + 1) % L == 0:
                    np.testing.assert_allclose(snaps[b_, (t + 1) // L - 1, h], S, atol=1e-13)
            np.testing.assert_allclose(ST[b_, h], S, atol=1e-13)


def test_p11_snapshots_beta_zero_is_decayed_initial_state():
    """beta = 0: snapshot j = Diag(prod of alpha over the first L (j + 1)
    tokens) S0, per sequence and head."""
    rng = np.random.default_rng(12)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, 70, 3, 5, 4)
    b[:] = 0.0
    _, _, snaps = kda_recurrent_snapshots(q, k, v, a, b, 1, S0, chunk=16)
    assert snaps.shape == (2, 4, 3, 5, 4)
    for j in range(4):
        decay = np.prod(a[:, : 16 * (j + 1)], axis=1)          # [B,H,DK]
        np.testing.assert_allclose(snaps[:, j], decay[..., None] * S0, rtol=1e-13, atol=1e-15)


def test_p11_snapshots_match_chunk_form_on_prefixes():
    """Snapshot j equals the final state of the independent chunk form run on
    the prefix of L (j + 1) tokens; o and the final state equal the chunk form
    over the whole sequence; resuming the chunk form from snapshot j
    reproduces the outputs of the remaining tokens."""
    rng = np.random.default_rng(13)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, 200, 2, 8, 6)
    every, chunk = 2, 16
    L = every * chunk
    o, ST, snaps = kda_recurrent_snapshots(q, k, v, a, b, every, S0, chunk=chunk)
    assert snaps.shape[1] == 200 // L == 6
    for j in range(6):
        e = L * (j + 1)
        _, Sp = kda_chunked(q[:, :e], k[:, :e], v[:, :e], a[:, :e], b[:, :e], S0, chunk=chunk)
        assert max_rel_err(snaps[:, j], Sp) < 1e-12
    o_c, S_c = kda_chunked(q, k, v, a, b, S0, chunk=chunk)
    assert max_rel_err(o, o_c) < 1e-12 and max_rel_err(ST, S_c) < 1e-12
    e = 3 * L
    o_r, S_r = kda_chunked(q[:, e:], k[:, e:], v[:, e:], a[:, e:], b[:, e:], snaps[:, 2], chunk=chunk)
    assert max_rel_err(o_r, o_c[:, e:]) < 1e-12 and max_rel_err(S_r, S_c) < 1e-12


def test_p11_snapshot_count_and_arguments():
    rng = np.random.default_rng(14)
    q, k, v, a, b, _ = rand_inputs(rng, 1, 63, 1, 4, 4, s0=False)
    assert kda_recurrent_snapshots(q, k, v, a, b, 1)[2].shape == (1, 0, 1, 4, 4)
    assert kda_recurrent_snapshots(q, k, v, a, b, 1, chunk=21)[2].shape == (1, 3, 1, 4, 4)
    with pytest.raises(ValueError):
        kda_recurrent_snapshots(q, k, v, a, b, 0)


# ------------------------------------------------------------------ P12 ---
def test_p12_pool_one_hot_keys_closed_form():
    """alpha = 1, beta = 1, one-hot keys (each write replaces one row of the
    state): pool slots, padding rows (negative or out-of-range slot), per-
    sequence token counts, outputs and per-token states in closed form;
    slots nobody references stay bit-identical."""
    rng = np.random.default_rng(21)
    N, L, H, DK, DV, P = 4, 3, 2, 5, 4, 6
    idx = np.array([3, -1, 0, 9])
    lens = np.array([3, 2, 1, 3])
    ch = rng.integers(0, DK, (N, L, H))
    k = np.zeros((N, L, H, DK))
    for n in range(N):
        for j in range(L):
            for h in range(H):
                k[n, j, h, ch[n, j, h]] = 1.0
    q = rng.standard_normal((N, L, H, DK))
    v = rng.standard_normal((N, L, H, DV))
    a = np.ones((N, L, H, DK))
    b = np.ones((N, L, H))
    pool = rng.standard_normal((P, H, DK, DV))
    o, new_pool, st = kda_decode_pool(q, k, v, a, b, pool, idx, lens)
    expect_pool = pool.copy()
    for n in range(N):
        if not 0 <= idx[n] < P:
            assert np.all(o[n] == 0) and np.all(np.isnan(st[n]))
            continue
        for h in range(H):
            S = pool[idx[n], h].copy()
            for j in range(L):
                if j >= lens[n]:
                    assert np.all(o[n, j, h] == 0) and np.all(np.isnan(st[n, j, h]))
                    continue
                S[ch[n, j, h]] = v[n, j, h]             # the replacement, written out
                np.testing.assert_allclose(o[n, j, h], q[n, j, h] @ S, atol=1e-13)
                np.testing.assert_allclose(st[n, j, h], S, atol=1e-13)
            expect_pool[idx[n], h] = S
    np.testing.assert_allclose(new_pool, expect_pool, atol=1e-13)
    for s_ in (1, 2, 4, 5):
        np.testing.assert_array_equal(new_pool[s_], pool[s_])


def test_p12_pool_beta_zero_is_decay():
    """beta = 0: after j + 1 tokens slot s holds Diag(prod alpha) pool[s] and
    o_j reads that state."""
    rng = np.random.default_rng(22)
    N, L, H, DK, DV, P = 3, 4, 2, 6, 5, 3
    q = rng.standard_normal((N, L, H, DK))
    k = rng.standard_normal((N, L, H, DK))
    v = rng.standard_normal((N, L, H, DV))
    a = np.exp(-np.exp(rng.uniform(-5, -1, (N, L, H, DK))))
    b = np.zeros((N, L, H))
    pool = rng.standard_normal((P, H, DK, DV))
    idx = np.array([2, 0, 1])
    o, new_pool, st = kda_decode_pool(q, k, v, a, b, pool, idx)
    for n in range(N):
        for j in range(L):
            S = np.prod(a[n, : j + 1], axis=0)[..., None] * pool[idx[n]]
            np.testing.assert_allclose(st[n, j], S, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(o[n, j], np.einsum("hkv,hk->hv", S, q[n, j]), rtol=1e-12,
                                       atol=1e-14)
        np.testing.assert_allclose(new_pool[idx[n]], st[n, L - 1], rtol=0, atol=0)


def test_p12_pool_matches_chunk_form_on_gathered_states():
    """Each sequence's tokens run from its gathered slot through the
    independent chunk form give the same outputs and final states."""
    rng = np.random.default_rng(23)
    N, L, H, DK, DV, P = 5, 6, 2, 8, 6, 8
    q, k, v, a, b, _ = rand_inputs(rng, N, L, H, DK, DV, s0=False)
    pool = rng.standard_normal((P, H, DK, DV))
    idx = rng.permutation(P)[:N]
    o, new_pool, _ = kda_decode_pool(q, k, v, a, b, pool, idx)
    o_c, S_c = kda_chunked(q, k, v, a, b, pool[idx], chunk=4)
    assert max_rel_err(o, o_c) < 1e-12 and max_rel_err(new_pool[idx], S_c) < 1e-12


def test_p12_tokens_past_count_are_ignored_and_duplicates_rejected():
    rng = np.random.default_rng(24)
    N, L, H, DK, DV = 3, 5, 1, 4, 4
    q, k, v, a, b, _ = rand_inputs(rng, N, L, H, DK, DV, s0=False)
    pool = rng.standard_normal((N, H, DK, DV))
    lens = np.array([2, 5, 0])
    r1 = kda_decode_pool(q, k, v, a, b, pool, None, lens)
    q2, v2 = q.copy(), v.copy()
    q2[0, 2:] += 1.0
    v2[2] -= 3.0
    r2 = kda_decode_pool(q2, k, v2, a, b, pool, None, lens)
    for x, y in zip(r1, r2):
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(r1[1][2], pool[2])       # zero tokens: slot untouched
    with pytest.raises(ValueError):
        kda_decode_pool(q, k, v, a, b, pool, [0, 1, 0])


# ------------------------------------------------------------------ P13 ---
def _torch_loss_grads(q, k, v, a, b, S0, do, dST):
    """fp64 torch autograd through a recurrence written with torch ops (the
    dense transition form, independent of the oracle's code)."""
    import torch

    t = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for n, x in dict(q=q, k=k, v=v, a=a, b=b, S0=S0).items()}
    B, T, H, DK = q.shape
    S = t["S0"]
    eye = torch.eye(DK, dtype=torch.float64)
    loss = 0.0
    for s_ in range(T):
        kt = t["k"][:, s_]                                            # [B,H,DK]
        M = eye - t["b"][:, s_, :, None, None] * kt[..., :, None] * kt[..., None, :]
        S = M @ (t["a"][:, s_, ..., None] * S) + \
            t["b"][:, s_, :, None, None] * kt[..., :, None] * t["v"][:, s_][..., None, :]
        o = torch.einsum("bhkv,bhk->bhv", S, t["q"][:, s_])
        loss = loss + (o * torch.tensor(do[:, s_])).sum()
    loss = loss + (S * torch.tensor(dST)).sum()
    loss.backward()
    return [t[n].grad.numpy() for n in ("q", "k", "v", "a", "b", "S0")]


def test_p13_backward_matches_torch_autograd():
    """The hand-written reverse mode against fp64 autograd of the dense
    transition form S_t = (I - b k k^T) Diag(a) S + b k v^T."""
    rng = np.random.default_rng(51)
    q, k, v, a, b, S0 = rand_inputs(rng, 2, 23, 2, 5, 4)
    do = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)
    got = kda_backward(q, k, v, a, b, S0, do, dST)
    ref = _torch_loss_grads(q, k, v, a, b, S0, do, dST)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")):
        assert max_rel_err(g, r) < 1e-12, name


def test_p13_backward_finite_differences():
    """Central differences of L = sum(o do) + sum(S_T dST) on sampled
    coordinates of every input."""
    rng = np.random.default_rng(52)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 9, 1, 4, 3)
    do = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)

    def loss(q_, k_, v_, a_, b_, S0_):
        o, S = kda_recurrent(q_, k_, v_, a_, b_, S0_)
        return float(np.sum(o * do) + np.sum(S * dST))

    grads = kda_backward(q, k, v, a, b, S0, do, dST)
    args = [q, k, v, a, b, S0]
    h = 1e-6
    for i, (x, g) in enumerate(zip(args, grads)):
        for idx in list(np.ndindex(x.shape))[:: max(1, x.size // 7)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[i], am[i] = xp, xm
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-6 * max(1.0, abs(fd)), (i, idx, fd, g[idx])


def test_p13_backward_beta_zero_closed_form():
    """beta = 0: v and k do not reach the output (dv = dk = 0, dbeta from the
    error term), and dS0 = sum_t Diag(prod_{s<=t} a_s) q_t do_t^T + Diag(prod a) dST."""
    rng = np.random.default_rng(53)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 11, 2, 5, 3)
    b[:] = 0.0
    do = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)
    dq, dk, dv, da, db, dS0 = kda_backward(q, k, v, a, b, S0, do, dST)
    assert np.all(dv == 0) and np.all(dk == 0)
    cum = np.cumprod(a, axis=1)                                   # [B,T,H,DK]
    expect = np.einsum("bthk,bthv->bhkv", cum * q, do) + cum[:, -1][..., None] * dST
    np.testing.assert_allclose(dS0, expect, rtol=1e-12, atol=1e-12)
    # dq_t = S_t do_t with S_t = Diag(prod a) S0
    np.testing.assert_allclose(dq, np.einsum("bthk,bhkv,bthv->bthk", cum, S0, do), rtol=1e-12,
                               atol=1e-12)


# ------------------------------------------------------------------ P14 ---
def test_p14_scalar_gate_backward_finite_differences():
    """gdn_backward against central differences of the separately written
    scalar-gate recurrence gdn_recurrent, on sampled coordinates of every
    input (the gate's gradient is the one that differs from KDA's)."""
    rng = np.random.default_rng(54)
    q, k, v, a, b, S0 = rand_inputs(rng, 1, 9, 2, 4, 3)
    g = a[..., 0].copy()                                    # one gate per token-head
    do = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)

    def loss(q_, k_, v_, g_, b_, S0_):
        o, S = gdn_recurrent(q_, k_, v_, g_, b_, S0_)
        return float(np.sum(o * do) + np.sum(S * dST))

    grads = gdn_backward(q, k, v, g, b, S0, do, dST)
    assert grads[3].shape == g.shape
    args = [q, k, v, g, b, S0]
    h = 1e-6
    for i, (x, gr) in enumerate(zip(args, grads)):
        for idx in list(np.ndindex(x.shape))[:: max(1, x.size // 7)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[i], am[i] = xp, xm
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            assert abs(fd - gr[idx]) < 1e-6 * max(1.0, abs(fd)), (i, idx, fd, gr[idx])


def test_alpha_domain_is_checked():
    z = np.zeros((1, 2, 1, 2))
    with pytest.raises(ValueError):
        kda_recurrent(z, z, z, np.full((1, 2, 1, 2), 1.5), np.zeros((1, 2, 1)))
    with pytest.raises(ValueError):
        kda_recurrent(z, z, z, np.zeros((1, 2, 1, 2)), np.zeros((1, 2, 1)))


def test_max_rel_err_definition():
    ref = np.array([0.0, 2.0, -4.0])
    assert max_rel_err(ref, ref) == 0.0
    assert max_rel_err(ref + np.array([0.0, 0.0, 0.004]), ref) == pytest.approx(0.001)
    assert max_rel_err(np.array([0.0, np.nan, 0.0]), ref) == float("inf")
