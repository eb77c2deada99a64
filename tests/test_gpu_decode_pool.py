"""GPU parity of the pooled multi-token decode (continuous batching and
speculative-draft verification): outputs, the pool after the call and the
per-token states against the fp64 oracle, with padding rows, per-sequence
token counts and permuted slots."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host, tdtype
from oracle import kda_decode_pool, kda_decode_step, kda_recurrent, max_rel_err

pytestmark = pytest.mark.gpu


def pool_inputs(rng, N, L, H, DK, DV, dt):
    """Unit-norm q, k; alpha = exp(-exp(U(-5,-1))); beta = sigmoid(N(0,1));
    q, k, v rounded to the input dtype (the oracle sees the same values)."""
    from gated_delta_rule_diag_amd.inputs import round_bf16

    q = rng.standard_normal((N, L, H, DK))
    k = rng.standard_normal((N, L, H, DK))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, L, H, DV))
    a = np.exp(-np.exp(rng.uniform(-5, -1, (N, L, H, DK)))).astype(np.float32)
    b = (1 / (1 + np.exp(-rng.standard_normal((N, L, H))))).astype(np.float32)
    r = (lambda x: round_bf16(x.astype(np.float32))) if dt == "bf16" else (lambda x: x.astype(np.float32))
    return r(q), r(k), r(v), a, b


@pytest.mark.parametrize("L", [1, 3, 8])
@pytest.mark.parametrize("dt,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("f32", 128, 64),
                                      ("f32", 64, 128)])
def test_decode_pool_matches_oracle(dt, dk, dv, L):
    """N=7 sequences over a pool of 10 slots (permuted; one padding row with
    slot -1, one with slot 13 >= pool size), token counts in [0, L]."""
    N, H, P = 7, 3, 10
    flush(f"[decode_pool] N={N} L={L} H={H} DK={dk} DV={dv} {dt} pool={P}")
    rng = np.random.default_rng([L, dk, dv])
    q, k, v, a, b = pool_inputs(rng, N, L, H, dk, dv, dt)
    pool0 = (0.5 * rng.standard_normal((P, H, dk, dv))).astype(np.float32)
    idx = np.concatenate([rng.permutation(P)[: N - 2], [-1, 13]]).astype(np.int32)
    rng.shuffle(idx)
    lens = rng.integers(0, L + 1, N).astype(np.int32)
    lens[0] = L
    o_ref, pool_ref, st_ref = kda_decode_pool(q, k, v, a, b, pool0, idx, lens)
    td = tdtype(dt)
    pool = dev(pool0)
    o, st = kda.decode_pool(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b), pool,
                            torch.from_numpy(idx).cuda(), torch.from_numpy(lens).cuda(),
                            return_token_states=True)
    torch.cuda.synchronize()
    go, gp, gs = host(o), host(pool), host(st)
    eo, ep = max_rel_err(go, o_ref), max_rel_err(gp, pool_ref)
    done = ~np.isnan(st_ref[..., 0, 0, 0])          # [N, L]: processed tokens
    es = max_rel_err(gs[done], st_ref[done])
    flush(f"    err o={eo:.2e} pool={ep:.2e} token_states={es:.2e}")
    assert eo <= TOL[dt] and ep <= TOL[dt] and es <= TOL[dt]
    # rows that are not processed are exactly zero; untouched slots are unchanged
    assert np.all(go[~done] == 0)
    touched = {int(idx[n]) for n in range(N) if 0 <= idx[n] < P and lens[n] > 0}
    for s_ in range(P):
        if s_ not in touched:
            assert np.array_equal(gp[s_], pool0[s_].astype(np.float64)), s_


def test_decode_pool_single_token_equals_decode_step():
    """L = 1, no index, no counts: the same step as kda_decode_step."""
    N, H, D = 16, 4, 128
    flush(f"[decode_pool] L=1 vs decode_step N={N} H={H} d={D}")
    rng = np.random.default_rng(31)
    q, k, v, a, b = pool_inputs(rng, N, 1, H, D, D, "bf16")
    S0 = (0.5 * rng.standard_normal((N, H, D, D))).astype(np.float32)
    bf = torch.bfloat16
    x = [dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b)]
    S1, S2 = dev(S0), dev(S0)
    o1 = kda.decode_step(*[t[:, 0].contiguous() for t in x], S1)
    o2, _ = kda.decode_pool(*x, S2)
    torch.cuda.synchronize()
    assert max_rel_err(host(o2)[:, 0], host(o1)) <= 1e-6
    assert max_rel_err(host(S2), host(S1)) <= 1e-6
    o_ref, S_ref = kda_decode_step(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], S0)
    assert max_rel_err(host(o2)[:, 0], o_ref) <= TOL["bf16"]


def test_decode_pool_eight_tokens_equal_prefill():
    """Eight draft tokens from pool slots equal a prefill of the same eight
    tokens from the same states."""
    N, L, H, D, P = 5, 8, 2, 128, 9
    flush(f"[decode_pool] L=8 vs prefill N={N} H={H} d={D}")
    rng = np.random.default_rng(32)
    q, k, v, a, b = pool_inputs(rng, N, L, H, D, D, "bf16")
    pool0 = (0.5 * rng.standard_normal((P, H, D, D))).astype(np.float32)
    idx = rng.permutation(P)[:N].astype(np.int32)
    bf = torch.bfloat16
    x = [dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b)]
    pool = dev(pool0)
    o, _ = kda.decode_pool(*x, pool, torch.from_numpy(idx).cuda())
    op, Sp = kda.chunk_prefill(*x, dev(pool0[idx]))
    torch.cuda.synchronize()
    assert max_rel_err(host(o), host(op)) <= 1e-5
    assert max_rel_err(host(pool)[idx], host(Sp)) <= 1e-5
    o_ref, S_ref = kda_recurrent(q, k, v, a, b, pool0[idx])
    assert max_rel_err(host(o), o_ref) <= TOL["bf16"]


def test_decode_pool_padding_only_and_zero_tokens():
    """Every row padding (state_idx all -1) or every count 0: outputs are 0 and
    the pool is untouched."""
    N, L, H, D, P = 4, 2, 2, 64, 4
    flush(f"[decode_pool] padding only N={N} L={L} H={H} d={D}")
    rng = np.random.default_rng(33)
    q, k, v, a, b = pool_inputs(rng, N, L, H, D, D, "f32")
    pool0 = rng.standard_normal((P, H, D, D)).astype(np.float32)
    x = [dev(q), dev(k), dev(v), dev(a), dev(b)]
    pool = dev(pool0)
    o, _ = kda.decode_pool(*x, pool, torch.full((N,), -1, dtype=torch.int32, device="cuda"))
    o2, _ = kda.decode_pool(*x, pool, None, torch.zeros(N, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0 and torch.count_nonzero(o2) == 0
    assert np.array_equal(host(pool), pool0.astype(np.float64))
