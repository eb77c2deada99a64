"""kda_chunk_prefill_noalloc, the prefill for callers that cannot allocate:
called through the C ABI and checked against kda_chunk_prefill with a
workspace, on two calls in a row, the second with a smaller input (the static
scratch keeps the first call's contents)."""

import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host, random_state, tdtype
from oracle import kda_recurrent, max_rel_err

pytestmark = pytest.mark.gpu


def noalloc(q, k, v, a, b, S0):
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    o = torch.empty((B, T, H, DV), device="cuda", dtype=torch.float32)
    S = torch.empty((B, H, DK, DV), device="cuda", dtype=torch.float32)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = kda.lib().kda_chunk_prefill_noalloc(
        B, T, H, DK, DV, 64, kda._in_dtype(q), p(q), p(k), p(v), p(a), p(b), p(S0), p(o), p(S),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, kda.lib().kda_last_error_message().decode()
    return o, S


@pytest.mark.parametrize("cases", [
    # (B, T, H, d, dtype, seed): the staged form (B*H < 128) in segments that
    # fit the scratch, then a smaller call
    [(1, 8192, 32, 128, "bf16", 1), (1, 1000, 4, 64, "f32", 901)],
])
def test_noalloc_prefill_matches_workspace_call(cases):
    for B, T, H, d, dt, seed in cases:
        flush(f"[noalloc] B={B} T={T} H={H} d={d} {dt}")
        q, k, v, a, b = I.batch_inputs(seed, B, T, H, d, d, dt)
        S0 = random_state(np.random.default_rng(seed), (B, H, d, d))
        td = tdtype(dt)
        x = (dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b), dev(S0))
        assert kda.lib().kda_chunk_prefill_workspace_size(B, T, H, d, d, 64) > 0
        o_ref, S_ref = kda.chunk_prefill(*x)
        o, S = noalloc(*x)
        torch.cuda.synchronize()
        # the same kernels on the same chunks, only the segments differ: bit
        # for bit, and within the bar of the oracle on two heads
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
        hs = [0, H - 1]
        ro, rS = kda_recurrent(q[:, :, hs], k[:, :, hs], v[:, :, hs], a[:, :, hs], b[:, :, hs],
                               S0[:, hs])
        e = (max_rel_err(host(o)[:, :, hs], ro), max_rel_err(host(S)[:, hs], rS))
        flush(f"    bitwise equal to the workspace call; oracle o={e[0]:.1e} S={e[1]:.1e}")
        assert max(e) <= TOL[dt], e
