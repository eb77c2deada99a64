"""The entry points under HIP graph capture (torch.cuda.CUDAGraph): the
captured decode step, staged prefill and backward are replayed several times, with the
program's own eager work and synchronisations between replays, and every
replay is checked against the eager result.  None of the kernels records a
memset or allocates, so the captured launches are plain kernel nodes."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import dev, flush, random_state

pytestmark = pytest.mark.gpu


def test_decode_step_replays_match_eager():
    N, H, D = 8, 4, 128
    flush(f"[graph] decode N={N} H={H} d={D}: 4 replays")
    q, k, v, a, b = I.decode_inputs(800, N, H, D, D, "bf16")
    S0 = random_state(np.random.default_rng(1), (N, H, D, D))
    bf = torch.bfloat16
    x = [dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b)]
    state = dev(S0)
    out = torch.empty((N, H, D), device="cuda")
    # eager reference: four consecutive steps from S0
    S_ref = dev(S0)
    o_ref, S_after = [], []
    for _ in range(4):
        o_ref.append(kda.decode_step(*x, S_ref).clone())
        S_after.append(S_ref.clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.decode_step(*x, state, out)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    state.copy_(dev(S0))
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        kda.decode_step(*x, state, out)
    state.copy_(dev(S0))
    torch.cuda.synchronize()
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref[i]), i
        assert torch.equal(state, S_after[i]), i
        _ = (x[3] * 2).sum()                     # unrelated eager work between replays
        torch.cuda.synchronize()


def test_staged_prefill_replays_match_eager():
    B, T, H, D = 1, 640, 4, 128
    flush(f"[graph] staged prefill B={B} T={T} H={H} d={D}: 3 replays")
    q, k, v, a, b = I.batch_inputs(801, B, T, H, D, D, "bf16")
    bf = torch.bfloat16
    x = [dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b)]
    S0 = dev(random_state(np.random.default_rng(2), (B, H, D, D)))
    ws = torch.empty(kda.lib().kda_chunk_prefill_workspace_size(B, T, H, D, D, 64), device="cuda",
                     dtype=torch.uint8)
    assert ws.numel() > 0                        # the two-kernel form with a workspace
    o_ref, S_ref = kda.chunk_prefill(*x, S0)
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.chunk_prefill(*x, S0, True, 64, o, S, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.chunk_prefill(*x, S0, True, 64, o, S, ws)
    for i in range(3):
        o.zero_()
        S.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), i


@pytest.mark.parametrize("window", [None, "1"])
def test_backward_replays_match_eager(window, monkeypatch):
    """The backward call (forward with checkpoints, the reverse walk, the
    reductions; with windows of one chunk, one walk and reduction per chunk
    with the adjoint carried in the workspace) captured once and replayed;
    every replay equals the eager call."""
    if window:
        kda.set_tuning(bwd_window=window)
    B, T, H, D = 1, 200, 3, 128
    flush(f"[graph] backward B={B} T={T} H={H} d={D} window={window}: 3 replays")
    q, k, v, a, b = I.batch_inputs(802, B, T, H, D, D, "bf16")
    rng = np.random.default_rng(803)
    do = rng.standard_normal((B, T, H, D)).astype(np.float32)
    S0 = random_state(rng, (B, H, D, D))
    bf = torch.bfloat16
    x = [dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), dev(do), dev(S0)]
    ws = torch.empty(kda.lib().kda_chunk_backward_workspace_size(B, T, H, D, D, 64),
                     device="cuda", dtype=torch.uint8)
    ref = kda.chunk_backward(*x, workspace=ws)
    torch.cuda.synchronize()
    ref = [r.clone() for r in ref]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.chunk_backward(*x, workspace=ws)     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = kda.chunk_backward(*x, workspace=ws)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        for u, w in zip(out, ref):
            assert torch.equal(u, w), i
        _ = (x[3] * 2).sum()                     # unrelated eager work between replays
        torch.cuda.synchronize()


def test_varlen_snapshots_and_backward_replay_match_eager():
    """Packed-sequence calls under capture: the snapshot prefill (default
    offsets built on the device) and the backward (max_seqlen from the host)
    read no device data on the host, so both capture as plain launches; three
    replays, each checked bit for bit against the eager calls."""
    lengths = [70, 0, 5, 200, 64]
    H, D = 2, 128
    flush(f"[graph] varlen snapshots + backward lengths={lengths} H={H} d={D}: 3 replays")
    q, k, v, a, b, cu = I.packed_inputs(804, lengths, H, D, D, "bf16")
    rng = np.random.default_rng(805)
    do = rng.standard_normal(v.shape).astype(np.float32)
    S0 = random_state(rng, (len(lengths), H, D, D))
    bf = torch.bfloat16
    x = [dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b)]
    cu_d = torch.from_numpy(cu).cuda()
    ml = max(lengths)
    ws = torch.empty(kda.lib().kda_chunk_backward_varlen_workspace_size(
        len(lengths), int(cu[-1]), ml, H, D, D, 64), device="cuda", dtype=torch.uint8)
    ref_p = [t.clone() for t in kda.chunk_prefill_varlen_snapshots(*x, cu_d, 1, dev(S0))]
    ref_b = [t.clone() for t in kda.chunk_backward_varlen(*x, cu_d, dev(do), dev(S0), None,
                                                          max_seqlen=ml, workspace=ws)]
    torch.cuda.synchronize()

    def calls():
        p = kda.chunk_prefill_varlen_snapshots(*x, cu_d, 1, dev_S0)
        g_ = kda.chunk_backward_varlen(*x, cu_d, dev_do, dev_S0, None, max_seqlen=ml, workspace=ws)
        return p, g_

    dev_S0, dev_do = dev(S0), dev(do)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_p, out_b = calls()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        rows = sum(n // 64 for n in lengths)     # snapshot rows the sequences write
        for j, (u, w) in enumerate(zip(out_p, ref_p)):
            assert torch.equal(u[:rows] if j == 2 else u, w[:rows] if j == 2 else w), ("prefill", i)
        for u, w in zip(out_b, ref_b):
            assert torch.equal(u, w), ("backward", i)
        _ = (x[3] * 2).sum()                     # unrelated eager work between replays
        torch.cuda.synchronize()
