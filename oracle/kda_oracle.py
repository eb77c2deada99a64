"""fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Sources (web pages; cited by title and section):

* [EXPLAINER] "Kimi Delta Attention 徹底解説 — 1M文脈で6倍速・KVキャッシュ75%削減を
  実現した線形アテンションの正体" (tech-tide.dev, 2026-07-29).
  - section "なぜ今「線形アテンション」なのか": linear attention folds the past
    into a fixed-size state by re-associating (|v><k|)|q> = <k|q>|v>; purely
    additive writes make memories interfere.
  - section "Kimi Delta Attention の仕組み — 「忘れ方」を鍛える":
      * DeltaNet queries the state with the new key, and writes only the error
        delta = beta * (v - S|k>), beta being a write strength (beta = 1 replaces
        the stored value, small beta overwrites gently);
      * Gated DeltaNet first decays the whole state by a scalar gate alpha and
        only then writes ("forget, then remember");
      * KDA promotes the gate to a diagonal matrix Diag(alpha), so every state
        channel has its own forget rate;
      * decode is a token-by-token recurrence, prefill is the same computation
        regrouped into chunked matrix products: both come from one formulation.
* [NEWS] "Kimi Linear、独自の土俵でFull Attentionを上回る" (remio.ai), section
  "Kimi Linearがより賢いRecurrent Memoryを使う方法": the finer gate depends on
  the current token (so alpha is given per token), and the chunkwise algorithm
  uses a diagonal-plus-low-rank transition.

Readings taken where the pages are silent:

* State orientation: S is d_k x d_v, row i = key channel, column j = value
  channel.  The explainer writes S|k> (a d_v x d_k map); S here is its
  transpose, so the prediction is S^T k.  Same mathematics.
* Diag(alpha_t) scales the key channels (rows of S).
* Order inside one token: decay first, then predict S^T k from the decayed
  state, then write; the output o_t = S_t^T q_t reads the state after token
  t's write.  No 1/sqrt(d_k) scale on q.
* alpha must lie in (0, 1]; beta may be any finite real.
* Heads and sequences are independent.  The initial state is zero unless given.

Parity: pinned by tests/test_oracle_pins.py (closed forms, special cases that
reduce to DeltaNet / Gated DeltaNet / linear attention, exact-rational brute
force with dense transition matrices, hand-derived golden values, linearity,
needle retrieval, split consistency, varlen packing).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kda_recurrent",
    "kda_recurrent_varlen",
    "kda_recurrent_snapshots",
    "gdn_recurrent",
    "kda_backward",
    "kda_decode_step",
    "kda_decode_pool",
    "kda_chunked",
    "max_rel_err",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check_alpha(alpha):
    a = _f64(alpha)
    if a.size and not (np.all(a > 0.0) and np.all(a <= 1.0)):
        raise ValueError("alpha must lie in (0, 1]")
    return a


def kda_recurrent(q, k, v, alpha, beta, S0=None):
    """Token recurrence of KDA, fixed-length batch.

    Shapes: q, k, alpha [B,T,H,DK]; v [B,T,H,DV]; beta [B,T,H];
    S0 [B,H,DK,DV] or None (zeros).  Returns (o [B,T,H,DV], S_T [B,H,DK,DV]),
    both fp64.

    Per token, per (batch, head), as in [EXPLAINER] "Kimi Delta Attention の仕組み":
      1. S <- Diag(alpha_t) S                      (channel-wise forget, first)
      2. S <- S + beta_t k_t (v_t - S^T k_t)^T      (delta-rule write)
      3. o_t = S^T q_t                               (read after the write)
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    alpha = _check_alpha(alpha)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    assert k.shape == (B, T, H, DK) and alpha.shape == (B, T, H, DK)
    assert v.shape == (B, T, H, DV) and beta.shape == (B, T, H)
    S = np.zeros((B, H, DK, DV)) if S0 is None else _f64(S0).copy()
    assert S.shape == (B, H, DK, DV)
    o = np.zeros((B, T, H, DV))
    for t in range(T):
        a_t = alpha[:, t]            # [B,H,DK]
        k_t = k[:, t]                # [B,H,DK]
        v_t = v[:, t]                # [B,H,DV]
        b_t = beta[:, t]             # [B,H]
        # 1. forget: every key channel (row of S) scaled by its own alpha.
        S = a_t[..., :, None] * S
        # 2. predict the value stored under k_t, then write the error.
        pred = np.einsum("bhkv,bhk->bhv", S, k_t)
        delta = b_t[..., None] * (v_t - pred)
        S = S + k_t[..., :, None] * delta[..., None, :]
        # 3. read.
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


def gdn_recurrent(q, k, v, gate, beta, S0=None):
    """Gated DeltaNet: the scalar-gate case KDA generalises ([EXPLAINER]
    "Kimi Delta Attention の仕組み": Gated DeltaNet decays the whole state by
    one scalar before the delta write; KDA turns that scalar into a diagonal).

    Shapes: q, k [B,T,H,DK]; v [B,T,H,DV]; gate, beta [B,T,H];
    S0 [B,H,DK,DV] or None.  Per token: S <- gate_t S; then the delta write
    and the read exactly as in kda_recurrent.  Returns (o, S_T) in fp64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    g = _check_alpha(gate)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    assert g.shape == (B, T, H) and beta.shape == (B, T, H)
    S = np.zeros((B, H, DK, DV)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, T, H, DV))
    for t in range(T):
        S = g[:, t, :, None, None] * S                       # one scalar per head
        pred = np.einsum("bhkv,bhk->bhv", S, k[:, t])
        S = S + k[:, t, :, :, None] * (beta[:, t, :, None] * (v[:, t] - pred))[..., None, :]
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


def kda_backward(q, k, v, alpha, beta, S0, do, dST=None):
    """Gradients of L = sum(o * do) + sum(S_T * dST) through the token
    recurrence (the chunk algorithm was designed for training as well
    ([NEWS] section "Kimi Linearがより賢いRecurrent Memoryを使う方法"); its
    gradient is that of the recurrence it regroups).

    Shapes as in kda_recurrent; do [B,T,H,DV]; dST [B,H,DK,DV] or None;
    S0 [B,H,DK,DV] or None.  Returns (dq, dk, dv, dalpha, dbeta, dS0), fp64.

    Reverse mode of each token's steps, written out.  Forward, per token:
        St = Diag(a) S;  p = St^T k;  u = b (v - p);  S' = St + k u^T;  o = S'^T q.
    With G the adjoint of S' (it includes o's term q do^T):
        dq = S' do;  du = G^T k;  dv = b du;  db = du . (v - p);  dp = -b du;
        dSt = G + k dp^T;  dk = G u + St dp;  da = rowsum(dSt * S);  G_prev = Diag(a) dSt.
    The forward states are recomputed and kept for the whole sequence.
    """
    q, k, v, beta, do = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(do)
    a = _check_alpha(alpha)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    S = np.zeros((B, H, DK, DV)) if S0 is None else _f64(S0).copy()
    states = np.zeros((T + 1, B, H, DK, DV))
    states[0] = S
    for t in range(T):
        St = a[:, t, ..., None] * S
        p = np.einsum("bhkv,bhk->bhv", St, k[:, t])
        u = beta[:, t, :, None] * (v[:, t] - p)
        S = St + k[:, t, ..., None] * u[..., None, :]
        states[t + 1] = S
    G = np.zeros((B, H, DK, DV)) if dST is None else _f64(dST).copy()
    dq, dk, da = np.zeros_like(q), np.zeros_like(k), np.zeros_like(a)
    dv, db = np.zeros_like(v), np.zeros_like(beta)
    for t in range(T - 1, -1, -1):
        Sp = states[t]                                   # state before token t
        St = a[:, t, ..., None] * Sp
        p = np.einsum("bhkv,bhk->bhv", St, k[:, t])
        u = beta[:, t, :, None] * (v[:, t] - p)
        Sn = states[t + 1]
        G = G + q[:, t, ..., None] * do[:, t, :, :][..., None, :]   # o_t = S'^T q_t
        dq[:, t] = np.einsum("bhkv,bhv->bhk", Sn, do[:, t])
        du = np.einsum("bhkv,bhk->bhv", G, k[:, t])
        dv[:, t] = beta[:, t, :, None] * du
        db[:, t] = np.sum(du * (v[:, t] - p), axis=-1)
        dp = -beta[:, t, :, None] * du
        dSt = G + k[:, t, ..., None] * dp[..., None, :]
        dk[:, t] = np.einsum("bhkv,bhv->bhk", G, u) + np.einsum("bhkv,bhv->bhk", St, dp)
        da[:, t] = np.sum(dSt * Sp, axis=-1)
        G = a[:, t, ..., None] * dSt
    return dq, dk, dv, da, db, G


def gdn_backward(q, k, v, gate, beta, S0, do, dST=None):
    """Gradients for the scalar-gate (Gated DeltaNet) recurrence of
    gdn_recurrent: the same loss as kda_backward.  A scalar gate is KDA's
    diagonal gate with every channel equal ([EXPLAINER] "Kimi Delta Attention
    の仕組み"), so by the chain rule its gradient is the sum over channels of
    the per-channel gate gradient; the other gradients are KDA's.

    Shapes as in gdn_recurrent; returns (dq, dk, dv, dgate [B,T,H], dbeta,
    dS0) in fp64.
    """
    g = _check_alpha(gate)
    DK = np.shape(q)[-1]
    dq, dk, dv, da, db, dS0 = kda_backward(q, k, v, np.repeat(g[..., None], DK, axis=-1), beta,
                                           S0, do, dST)
    return dq, dk, dv, da.sum(axis=-1), db, dS0


def kda_recurrent_varlen(q, k, v, alpha, beta, cu_seqlens, S0=None):
    """Packed variable-length prefill: sequence n owns tokens
    [cu_seqlens[n], cu_seqlens[n+1]) of the packed token axis.

    Shapes: q, k, alpha [T_total,H,DK]; v [T_total,H,DV]; beta [T_total,H];
    cu_seqlens [N+1] non-decreasing, cu_seqlens[0] == 0,
    cu_seqlens[N] == T_total; S0 [N,H,DK,DV] or None.
    Returns (o [T_total,H,DV], S_final [N,H,DK,DV]).  Each sequence starts
    from its own initial state; a length-0 sequence passes its state through.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    Ttot, H, DK = np.shape(q)
    DV = np.shape(v)[-1]
    if cu[0] != 0 or cu[-1] != Ttot or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T_total")
    o = np.zeros((Ttot, H, DV))
    Sf = np.zeros((N, H, DK, DV))
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        s0 = None if S0 is None else _f64(S0)[n : n + 1]
        on, Sn = kda_recurrent(
            _f64(q)[None, s:e], _f64(k)[None, s:e], _f64(v)[None, s:e],
            _f64(alpha)[None, s:e], _f64(beta)[None, s:e], s0,
        )
        o[s:e] = on[0]
        Sf[n] = Sn[0]
    return o, Sf


def kda_recurrent_snapshots(q, k, v, alpha, beta, every, S0=None, chunk=64):
    """Token recurrence that also records the state at block boundaries, for
    prefix caching: serving stacks keep a KDA sequence's state at block
    boundaries so that a later request sharing the prefix resumes from it
    ("Kimi Linearは広がりつつある：検証できるすべてのモデルが実際にKDAを実行する"
    (orcarouter.ai), section "既に起こった採用はサービングスタックの中にあります";
    [NEWS] section "オープンコードにより主張は検証可能になる": the state across
    chunk boundaries is what a deployment must test).

    With L = chunk * every, snapshot j (j = 0 .. T // L - 1) is by definition
    the state after the first L * (j + 1) tokens, i.e. the final state that
    kda_recurrent returns for that prefix; a tail shorter than L gets none.
    The recurrence is sequential, so it runs block by block carrying S.
    Returns (o [B,T,H,DV], S_T [B,H,DK,DV], snaps [B, T // L, H, DK, DV]).
    """
    q, k, v, alpha, beta = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta)
    if every < 1 or chunk < 1:
        raise ValueError("every and chunk must be >= 1")
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    L = chunk * every
    snaps = np.zeros((B, T // L, H, DK, DV))
    o = np.zeros((B, T, H, DV))
    S = np.zeros((B, H, DK, DV)) if S0 is None else _f64(S0).copy()
    for s in range(0, T, L):
        e = min(s + L, T)
        o[:, s:e], S = kda_recurrent(q[:, s:e], k[:, s:e], v[:, s:e], alpha[:, s:e],
                                     beta[:, s:e], S)
        if e - s == L:
            snaps[:, s // L] = S
    return o, S, snaps


def kda_decode_step(q, k, v, alpha, beta, S):
    """One recurrent decode step for N independent (sequence, head) states.

    Shapes: q, k, alpha [N,H,DK]; v [N,H,DV]; beta [N,H]; S [N,H,DK,DV].
    Returns (o [N,H,DV], S_new [N,H,DK,DV]).  It is the token recurrence with
    T = 1 (the explainer's "few lines" decode mode).
    """
    o, Sn = kda_recurrent(
        _f64(q)[:, None], _f64(k)[:, None], _f64(v)[:, None],
        _f64(alpha)[:, None], _f64(beta)[:, None], S,
    )
    return o[:, 0], Sn


def kda_decode_pool(q, k, v, alpha, beta, pool, state_idx=None, num_tokens=None):
    """Decode of up to L tokens per sequence with the states kept in a pool
    (continuous batching; verification of speculative drafts).  Deployment
    tools must support continuous batching and speculative decoding without
    breaking KDA's state handling ([NEWS] section "Kimi Linearリリース後に注目
    すべき点"); decode itself is the token recurrence ([EXPLAINER]).

    Shapes: q, k, alpha [N,L,H,DK]; v [N,L,H,DV]; beta [N,L,H];
    pool [P,H,DK,DV]; state_idx [N] ints or None (sequence n uses slot n);
    num_tokens [N] ints or None (all L).  Sequence n with slot
    s = state_idx[n] in [0, P) runs the recurrence over its first
    len_n = min(max(num_tokens[n], 0), L) tokens starting from pool[s]; the
    pool slot then holds the state after the last of them.  Any other slot
    value marks a padding row.  Returns
      o            [N,L,H,DV]      outputs; 0 for padding rows and unprocessed tokens
      new_pool     [P,H,DK,DV]     the pool after the call (untouched slots copied)
      token_states [N,L,H,DK,DV]   state after each processed token (NaN elsewhere)
    Slots referenced by two sequences are an error (the order would matter).
    """
    q, k, v, alpha, beta = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta)
    N, L, H, DK = q.shape
    DV = v.shape[-1]
    pool = _f64(pool)
    P = pool.shape[0]
    idx = np.arange(N) if state_idx is None else np.asarray(state_idx, dtype=np.int64)
    lens = np.full(N, L) if num_tokens is None else np.clip(np.asarray(num_tokens), 0, L)
    valid = (idx >= 0) & (idx < P)
    if len(set(idx[valid].tolist())) != int(valid.sum()):
        raise ValueError("a pool slot is referenced by two sequences")
    o = np.zeros((N, L, H, DV))
    new_pool = pool.copy()
    states = np.full((N, L, H, DK, DV), np.nan)
    for n in range(N):
        if not valid[n] or lens[n] == 0:
            continue
        e = int(lens[n])
        sl = slice(n, n + 1)
        # states after every token = snapshots with an interval of one token
        on, Sn, sn = kda_recurrent_snapshots(q[sl, :e], k[sl, :e], v[sl, :e], alpha[sl, :e],
                                             beta[sl, :e], 1, pool[idx[n]][None], chunk=1)
        o[n, :e] = on[0]
        states[n, :e] = sn[0]
        new_pool[idx[n]] = Sn[0]
    return o, new_pool, states


def kda_chunked(q, k, v, alpha, beta, S0=None, chunk=64):
    """The chunk form of the same recurrence, in fp64 (no blocking beyond it).

    This is the "large matrix products" regrouping the explainer names and the
    diagonal-plus-low-rank transition of [NEWS]; the pages print no formula for
    it, so it is written from this derivation (exact in real arithmetic).
    Within one chunk of n tokens with incoming state S0, g_r = sum_{s<=r} ln
    alpha_s (per key channel), and the per-token write u_r = beta_r (v_r -
    (Diag(alpha_r) S_{r-1})^T k_r) satisfies S_r = Diag(alpha_r) S_{r-1} + k_r u_r^T.
    Unrolling gives
        (I + A) U = Diag(beta) (V - K_g S0),  A[r,i] = beta_r sum_c k_rc k_ic e^{g_rc - g_ic}, i < r
        O   = Q_g S0 + P U,                   P[r,i] = sum_c q_rc k_ic e^{g_rc - g_ic},       i <= r
        S_n = Diag(e^{g_n}) S0 + K_hat^T U,   K_hat[i] = k_i * e^{g_n - g_i}
    with K_g = K * e^{g}, Q_g = Q * e^{g}.  Used only to pin that the chunk
    regrouping equals the token recurrence; it is never a parity reference.
    Shapes as in kda_recurrent.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    alpha = _check_alpha(alpha)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    S = np.zeros((B, H, DK, DV)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, T, H, DV))
    for b in range(B):
        for h in range(H):
            Sbh = S[b, h]
            for c0 in range(0, T, chunk):
                c1 = min(c0 + chunk, T)
                n = c1 - c0
                Q = q[b, c0:c1, h]
                K = k[b, c0:c1, h]
                V = v[b, c0:c1, h]
                bt = beta[b, c0:c1, h]
                g = np.cumsum(np.log(alpha[b, c0:c1, h]), axis=0)   # [n, DK]
                # decay between positions r >= i, per channel: e^{g_r - g_i}
                D = np.exp(g[:, None, :] - g[None, :, :])           # [n, n, DK]
                low_strict = np.tril(np.ones((n, n)), -1)
                low = np.tril(np.ones((n, n)))
                A = bt[:, None] * np.einsum("rc,ic,ric->ri", K, K, D) * low_strict
                P = np.einsum("rc,ic,ric->ri", Q, K, D) * low
                Kg = K * np.exp(g)
                Qg = Q * np.exp(g)
                Khat = K * np.exp(g[-1][None, :] - g)
                U = np.linalg.solve(np.eye(n) + A, bt[:, None] * (V - Kg @ Sbh))
                o[b, c0:c1, h] = Qg @ Sbh + P @ U
                Sbh = np.exp(g[-1])[:, None] * Sbh + Khat.T @ U
            S[b, h] = Sbh
    return o, S


def max_rel_err(got, ref):
    """Normwise max relative error: max|got - ref| / max|ref|.

    Element-wise relative error is undefined where ref is ~0, so the error of
    a whole output tensor is measured against its largest reference entry.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if not np.isfinite(num):
        return float("inf")
    if den == 0.0:
        return float(num)
    return float(num / den)
