"""GPU parity of the prefill with state snapshots at chunk boundaries (prefix
caching): snapshots, outputs and final states against the fp64 oracle, in
both prefill forms, and the exact-resume property a prefix cache relies on."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host, random_state, tdtype
from oracle import kda_recurrent_snapshots, max_rel_err

pytestmark = pytest.mark.gpu

PATHS = ["fused", "split"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("every", [1, 2, 5])
@pytest.mark.parametrize("dt,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("f32", 128, 64)])
def test_snapshots_match_oracle(dt, dk, dv, every, path, monkeypatch):
    """B=2, H=3, T=337 (5 full chunks and a ragged tail of 17 tokens), random
    initial state: T // (64 every) snapshots, o and the final state."""
    kda.set_tuning(prefill_form=path)
    B, T, H = 2, 337, 3
    flush(f"[snapshots] B={B} T={T} H={H} DK={dk} DV={dv} {dt} every={every} path={path}")
    q, k, v, a, b = I.batch_inputs(500 + every, B, T, H, dk, dv, dt)
    S0 = random_state(np.random.default_rng(every), (B, H, dk, dv))
    o_ref, S_ref, sn_ref = kda_recurrent_snapshots(q, k, v, a, b, every, S0)
    td = tdtype(dt)
    o, S, sn = kda.chunk_prefill_snapshots(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b),
                                           every, dev(S0))
    torch.cuda.synchronize()
    assert tuple(sn.shape) == (B, T // (64 * every), H, dk, dv)
    eo, es, en = (max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref),
                  max_rel_err(host(sn), sn_ref))
    flush(f"    err o={eo:.2e} S={es:.2e} snapshots={en:.2e}")
    assert eo <= TOL[dt] and es <= TOL[dt] and en <= TOL[dt]
    # each snapshot on its own (a late one must not hide an early one's error)
    for j in range(sn.shape[1]):
        assert max_rel_err(host(sn[:, j]), sn_ref[:, j]) <= TOL[dt]


@pytest.mark.parametrize("path", PATHS)
def test_snapshot_call_matches_plain_prefill_bitwise(path, monkeypatch):
    """The snapshot kernels compute o and the final state exactly as the plain
    prefill does (the snapshots are extra stores only)."""
    kda.set_tuning(prefill_form=path)
    B, T, H, D = 1, 64 * 7 + 9, 4, 128
    flush(f"[snapshots] bitwise vs plain prefill B={B} T={T} H={H} d={D} path={path}")
    q, k, v, a, b = I.batch_inputs(510, B, T, H, D, D, "bf16")
    S0 = random_state(np.random.default_rng(5), (B, H, D, D))
    bf = torch.bfloat16
    args = (dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b))
    o1, S1 = kda.chunk_prefill(*args, dev(S0))
    o2, S2, sn = kda.chunk_prefill_snapshots(*args, 3, dev(S0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert sn.shape[1] == 2


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_resume_from_snapshot_is_exact(dt, path, monkeypatch):
    """A prefix cache hit: prefill started from snapshot j over the tokens
    after it reproduces the full run's outputs and final state bit for bit
    (same chunk alignment, same arithmetic).  The last snapshot of a sequence
    whose length is a multiple of the interval is its final state."""
    kda.set_tuning(prefill_form=path)
    B, T, H, D, every = 2, 64 * 6, 3, 128, 2
    flush(f"[snapshots] resume B={B} T={T} H={H} d={D} {dt} every={every} path={path}")
    q, k, v, a, b = I.batch_inputs(520, B, T, H, D, D, dt)
    td = tdtype(dt)
    x = [dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b)]
    o, S, sn = kda.chunk_prefill_snapshots(*x, every)
    torch.cuda.synchronize()
    assert sn.shape[1] == 3
    assert torch.equal(sn[:, 2], S)
    for j in range(2):
        t0 = 64 * every * (j + 1)
        tail = [t[:, t0:].contiguous() for t in x]
        o_r, S_r = kda.chunk_prefill(*tail, sn[:, j].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o_r, o[:, t0:]) and torch.equal(S_r, S), j


def test_snapshots_without_full_interval():
    """T shorter than one interval: no snapshot, the call is a plain prefill."""
    B, T, H, D = 1, 100, 2, 64
    flush(f"[snapshots] none B={B} T={T} H={H} d={D} every=2")
    q, k, v, a, b = I.batch_inputs(530, B, T, H, D, D, "bf16")
    bf = torch.bfloat16
    args = (dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b))
    o, S, sn = kda.chunk_prefill_snapshots(*args, 2)
    o1, S1 = kda.chunk_prefill(*args)
    torch.cuda.synchronize()
    assert sn.shape == (1, 0, 2, 64, 64)
    assert torch.equal(o, o1) and torch.equal(S, S1)


@pytest.mark.parametrize("seg", [1, 2])
def test_snapshots_across_staged_segments(seg, monkeypatch):
    """Staged form processed in segments of `seg` chunks (state carried
    between launches): snapshots still land at the right boundaries."""
    kda.set_tuning(prefill_form="split")
    kda.set_tuning(prefill_seg=seg)
    B, T, H, D, every = 1, 64 * 7 + 30, 2, 128, 3
    flush(f"[snapshots] segments seg={seg} B={B} T={T} H={H} d={D} every={every}")
    q, k, v, a, b = I.batch_inputs(540, B, T, H, D, D, "bf16")
    S0 = random_state(np.random.default_rng(8), (B, H, D, D))
    o_ref, S_ref, sn_ref = kda_recurrent_snapshots(q, k, v, a, b, every, S0)
    bf = torch.bfloat16
    o, S, sn = kda.chunk_prefill_snapshots(dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b),
                                           every, dev(S0))
    torch.cuda.synchronize()
    assert sn.shape[1] == 2
    eo, es, en = (max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref),
                  max_rel_err(host(sn), sn_ref))
    flush(f"    err o={eo:.2e} S={es:.2e} snapshots={en:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and en <= TOL["bf16"]


def varlen_snapshot_reference(q, k, v, a, b, cu, every, S0):
    """Per-sequence oracle snapshots, packed in sequence order."""
    o, S, rows = [], [], []
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        on, Sn, sn = kda_recurrent_snapshots(q[None, s:e], k[None, s:e], v[None, s:e],
                                             a[None, s:e], b[None, s:e], every, S0[n:n + 1])
        o.append(on[0]); S.append(Sn[0]); rows.append(sn[0])
    return np.concatenate(o), np.stack(S), np.concatenate(rows)


@pytest.mark.parametrize("every", [1, 2])
@pytest.mark.parametrize("dt,dk,dv", [("bf16", 128, 128), ("f32", 64, 64)])
def test_varlen_snapshots_match_oracle(dt, dk, dv, every):
    """Packed sequences of mixed lengths (empty, shorter than one interval,
    exact multiples, ragged tails): each sequence's snapshots land at its own
    rows, and o and the final states match the plain varlen prefill."""
    lengths = [5, 0, 200, 64, 128, 33, 257]
    H = 3
    flush(f"[snapshots] varlen lengths={lengths} H={H} DK={dk} DV={dv} {dt} every={every}")
    q, k, v, a, b, cu = I.packed_inputs(550 + every, lengths, H, dk, dv, dt)
    S0 = random_state(np.random.default_rng(11), (len(lengths), H, dk, dv))
    o_ref, S_ref, sn_ref = varlen_snapshot_reference(q, k, v, a, b, cu, every, S0)
    td = tdtype(dt)
    x = (dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b), torch.from_numpy(cu).cuda())
    o, S, sn, offs = kda.chunk_prefill_varlen_snapshots(*x, every, dev(S0))
    o1, S1 = kda.chunk_prefill_varlen(*x, dev(S0))
    torch.cuda.synchronize()
    per = [n // (64 * every) for n in lengths]
    assert offs.cpu().tolist() == list(np.concatenate([[0], np.cumsum(per)]))
    # rows: the bound T_total // (64 every), known on the host without reading
    # the lengths; the sequences fill the first sum(per)
    assert sn.shape[0] == sum(lengths) // (64 * every) and sum(per) == sn_ref.shape[0]
    assert torch.equal(o, o1) and torch.equal(S, S1)
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL[dt] and es <= TOL[dt]
    for r in range(sum(per)):
        assert max_rel_err(host(sn[r]), sn_ref[r]) <= TOL[dt], r


def test_varlen_snapshots_follow_given_offsets():
    """Caller-chosen offsets: rows the offsets leave out keep their contents,
    a sequence given fewer rows than it has boundaries writes only those, and
    device offsets that point past num_snapshots write nothing there."""
    lengths = [130, 260, 70]          # 2, 4 and 1 boundaries at every=1
    H, d = 2, 64
    flush(f"[snapshots] varlen given offsets lengths={lengths} H={H} d={d}")
    q, k, v, a, b, cu = I.packed_inputs(560, lengths, H, d, d, "bf16")
    S0 = np.zeros((3, H, d, d))
    _, _, sn_ref = varlen_snapshot_reference(q, k, v, a, b, cu, 1, S0)   # rows 0-1, 2-5, 6
    bf = torch.bfloat16
    x = (dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), torch.from_numpy(cu).cuda())
    # sequence 0 -> rows 1..2; sequence 1 -> rows 4..5 only (2 of its 4);
    # sequence 2 -> row 6, but only 6 rows are passed (a view of the first 6
    # of 8), so row 6 is out of range and skipped
    offs = torch.tensor([1, 4, 6, 9], dtype=torch.int32, device="cuda")
    sent = torch.full((8, H, d, d), -7.0, device="cuda")
    kda.chunk_prefill_varlen_snapshots(*x, 1, snap_offsets=offs, snapshots=sent[:6])
    torch.cuda.synchronize()
    got = host(sent)
    untouched = [0, 3, 6, 7]
    assert (got[untouched] == -7.0).all()
    for row, ref in [(1, 0), (2, 1), (4, 2), (5, 3)]:
        assert max_rel_err(got[row], sn_ref[ref]) <= TOL["bf16"], row
