"""GPU parity at the five workloads' full sizes, in the launch
configuration bench.py times.  Where the oracle cannot run every (sequence,
head) in seconds, a seeded subset of heads is checked element by element."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host
from oracle import (kda_backward, kda_decode_pool, kda_decode_step, kda_recurrent,
                    kda_recurrent_snapshots, kda_recurrent_varlen, max_rel_err)

pytestmark = pytest.mark.gpu


_CFG1 = {}


def _cfg1_inputs():
    """Inputs of the B=1, H=32, T=8192, d=128 bf16 workload (drawn once)."""
    if "in" not in _CFG1:
        _CFG1["in"] = I.batch_inputs(1, 1, 8192, 32, 128, 128, "bf16")
    return _CFG1["in"]


def _cfg1_oracle():
    """Inputs and oracle result of the B=1, H=32, T=8192, d=128 workload
    (computed once, shared by both prefill forms)."""
    if "ref" not in _CFG1:
        _CFG1["ref"] = kda_recurrent(*_cfg1_inputs())
    return _CFG1["in"], _CFG1["ref"]


@pytest.mark.parametrize("path", ["split", "fused"])
def test_prefill_bf16_b1_h32_t8192_full(path, monkeypatch):
    """B=1, H=32, T=8192, d=128, bf16 q/k/v, zero initial state: every head,
    in both prefill forms (the staged form is the default at this size)."""
    kda.set_tuning(prefill_form=path)
    flush(f"[config] prefill B=1 H=32 T=8192 d=128 bf16 (all heads) path={path}")
    (q, k, v, a, b), (o_ref, S_ref) = _cfg1_oracle()
    bf = torch.bfloat16
    o, S = kda.chunk_prefill(dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b))
    torch.cuda.synchronize()
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("path", ["split", "fused"])
def test_prefill_snapshots_b1_h32_t8192_head_subset(path, monkeypatch):
    """The B=1, H=32, T=8192, d=128 bf16 prefill with a state snapshot every
    16 chunks (1024 tokens): 8 snapshots per head.  Heads {0, 13, 31} are
    checked against the oracle's snapshots; o and the final state of the
    snapshot call equal the plain prefill's bit for bit."""
    kda.set_tuning(prefill_form=path)
    flush(f"[config] prefill+snapshots B=1 H=32 T=8192 d=128 bf16 every=16 path={path}")
    q, k, v, a, b = _cfg1_inputs()
    bf = torch.bfloat16
    x = (dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b))
    o, S, sn = kda.chunk_prefill_snapshots(*x, 16)
    o1, S1 = kda.chunk_prefill(*x)
    torch.cuda.synchronize()
    assert tuple(sn.shape) == (1, 8, 32, 128, 128)
    assert torch.equal(o, o1) and torch.equal(S, S1)
    assert torch.equal(sn[:, 7], S)
    heads = [0, 13, 31]
    _, _, sn_ref = kda_recurrent_snapshots(q[:, :, heads], k[:, :, heads], v[:, :, heads],
                                           a[:, :, heads], b[:, :, heads], 16)
    errs = [max_rel_err(host(sn[:, j][:, heads]), sn_ref[:, j]) for j in range(8)]
    flush("    snapshot errors " + " ".join(f"{e:.1e}" for e in errs))
    assert max(errs) <= TOL["bf16"]


def test_decode_n256_h32_full():
    """One decode step for 256 sequences x 32 heads (fp32 state, 537 MB, in
    place).  Every pair is checked.  Sequences 0, 97 and 255 start from
    oracle prefill end-states of 128 seeded tokens; the others from seeded
    random states."""
    N, H, D, L0 = 256, 32, 128, 128
    flush("[config] decode N=256 H=32 d=128 bf16 (all pairs)")
    q, k, v, a, b = I.decode_inputs(2, N, H, D, D, "bf16")
    rng = np.random.default_rng([I.SEED, 2, 7])
    S0 = (0.3 * rng.standard_normal((N, H, D, D))).astype(np.float32)
    for n in (0, 97, 255):
        for h in range(H):
            pq, pk, pv, pa, pb = I.decode_prefix(2, n, h, L0, D, D, "bf16")
            _, Sp = kda_recurrent(pq[None, :, None], pk[None, :, None], pv[None, :, None],
                                  pa[None, :, None], pb[None, :, None])
            S0[n, h] = Sp[0, 0].astype(np.float32)
    bf = torch.bfloat16
    S = dev(S0)
    o = kda.decode_step(dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), S)
    torch.cuda.synchronize()
    o_ref, S_ref = kda_decode_step(q, k, v, a, b, S0)
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    # the oracle-prefilled sequences on their own
    sel = [0, 97, 255]
    assert max_rel_err(host(o)[sel], o_ref[sel]) <= TOL["bf16"]


@pytest.mark.parametrize("L", [1, 4])
def test_decode_pool_n256_h32_full(L):
    """The decode workload's batch (256 sequences x 32 heads, d=128, bf16) as
    continuous batching over a pool of 512 states in permuted slots: L=1 (one
    token each) and L=4 (speculative drafts).  Every pair and every pool slot
    is checked."""
    N, H, D, P = 256, 32, 128, 512
    flush(f"[config] decode pool N=256 L={L} H=32 d=128 bf16 pool=512")
    rng = np.random.default_rng([I.SEED, 5, L])
    q, k, v, a, b = (x.reshape((N, L) + x.shape[1:]) for x in I.decode_inputs(5 + L, N * L, H, D, D, "bf16"))
    pool0 = (0.3 * rng.standard_normal((P, H, D, D), dtype=np.float32))
    idx = rng.permutation(P)[:N].astype(np.int32)
    bf = torch.bfloat16
    pool = dev(pool0)
    o, _ = kda.decode_pool(dev(q, bf), dev(k, bf), dev(v, bf), dev(a), dev(b), pool,
                           torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    o_ref, pool_ref, _ = kda_decode_pool(q, k, v, a, b, pool0, idx)
    eo, ep = max_rel_err(host(o), o_ref), max_rel_err(host(pool)[idx], pool_ref[idx])
    flush(f"    err o={eo:.2e} pool={ep:.2e}")
    assert eo <= TOL["bf16"] and ep <= TOL["bf16"]
    rest = np.setdiff1d(np.arange(P), idx)
    assert torch.equal(pool[torch.from_numpy(rest).cuda()], dev(pool0[rest]))


def _device_packed(c, lengths, H, D, dt):
    """Packed varlen workload drawn on the device (per (sequence, head) seeded
    torch streams), with cu_seqlens."""
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    Tt = int(cu[-1])
    q = torch.empty((Tt, H, D), device="cuda", dtype=dt)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    a = torch.empty((Tt, H, D), device="cuda", dtype=torch.float32)
    b = torch.empty((Tt, H), device="cuda", dtype=torch.float32)
    for n, L in enumerate(lengths):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            qq, kk, vv, aa, bb = I.device_head_inputs(c, n, h, int(L), D, D, "cuda", dt)
            q[s:e, h], k[s:e, h], v[s:e, h], a[s:e, h], b[s:e, h] = qq, kk, vv, aa, bb
    return q, k, v, a, b, cu


def test_varlen_n64_h32_lengths_512_16384_head_subset():
    """64 packed sequences, lengths ~U[512, 16384] (seeded), H=32, d=128,
    bf16, zero initial states.  Heads {0, 17, 31} of every sequence are
    checked against the oracle."""
    H, D = 32, 128
    lengths = I.varlen_lengths(3, 64, 512, 16384)
    flush(f"[config] varlen N=64 total={int(lengths.sum())} H=32 d=128 bf16")
    q, k, v, a, b, cu = _device_packed(3, lengths, H, D, torch.bfloat16)
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, S = kda.chunk_prefill_varlen(q, k, v, a, b, cu_d)
    torch.cuda.synchronize()
    heads = [0, 17, 31]
    f = lambda t: t[:, heads].float().cpu().numpy()  # noqa: E731
    o_ref, S_ref = kda_recurrent_varlen(f(q), f(k), f(v), f(a), b[:, heads].cpu().numpy(), cu)
    eo = max_rel_err(o[:, heads].cpu().numpy(), o_ref)
    es = max_rel_err(S[:, heads].cpu().numpy(), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_backward_varlen_n64_h32_sequence_head_subset():
    """The backward pass of the 64-sequence packed workload (576,952 tokens,
    H=32, d=128, bf16; the reverse pass in windows of chunks): every gradient
    of the three shortest sequences on heads {0, 31} against the oracle's
    reverse mode (which keeps every token state, hence the short ones), and
    the longest sequence (16,278 tokens: 37 windows of the reverse pass) on
    head 0."""
    H, D = 32, 128
    lengths = I.varlen_lengths(3, 64, 512, 16384)
    Tt = int(lengths.sum())
    flush(f"[config] backward varlen N=64 total={Tt} H=32 d=128 bf16")
    q, k, v, a, b, cu = _device_packed(3, lengths, H, D, torch.bfloat16)
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(I.SEED + 31)
    do = torch.randn((Tt, H, D), generator=gen, device="cuda")
    grads = kda.chunk_backward_varlen(q, k, v, a, b, cu_d, do, max_seqlen=int(lengths.max()))
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dalpha", "dbeta")
    cases = [(int(n), [0, 31]) for n in np.argsort(lengths)[:3]] + [(int(np.argmax(lengths)), [0])]
    for n, heads in cases:
        s_, e_ = int(cu[n]), int(cu[n + 1])
        f = lambda t: t[s_:e_][:, heads].float().cpu().numpy()[None]  # noqa: E731
        ref = kda_backward(f(q), f(k), f(v), f(a), f(b), None, f(do), None)
        errs = {nm: max_rel_err(f(g)[0], r[0]) for nm, g, r in zip(names, grads[:5], ref[:5])}
        errs["dS0"] = max_rel_err(grads[5][n, heads].cpu().numpy(), ref[5][0])
        flush(f"    sequence {n} (length {e_ - s_}): " +
              " ".join(f"{nm}={e:.1e}" for nm, e in errs.items()))
        assert max(errs.values()) <= TOL["bf16"], (n, errs)
    del grads


def test_long_context_1m_prefill_then_1024_decode_steps_head_subset():
    """B=1, H=32, d=128, T=1,048,576 bf16 prefill, then 1024 recurrent decode
    steps from the resulting state.  Heads {0, 31}: the final prefill state,
    the outputs of every prefill token and of all decode steps are checked
    against the oracle run over the whole sequence."""
    T, H, D, ND = 1 << 20, 32, 128, 1024
    flush("[config] long context: prefill T=1048576 H=32 d=128 bf16 + 1024 decode steps")
    dt = torch.bfloat16
    heads = [0, 31]
    # all heads on the device; the checked heads are copied back for the oracle
    q = torch.empty((1, T, H, D), device="cuda", dtype=dt)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    a = torch.empty((1, T, H, D), device="cuda", dtype=torch.float32)
    b = torch.empty((1, T, H), device="cuda", dtype=torch.float32)
    for h in range(H):
        qq, kk, vv, aa, bb = I.device_head_inputs(4, 0, h, T + ND, D, D, "cuda", dt)
        q[0, :, h], k[0, :, h], v[0, :, h], a[0, :, h], b[0, :, h] = qq[:T], kk[:T], vv[:T], aa[:T], bb[:T]
        if h in heads:
            tail = (qq[T:], kk[T:], vv[T:], aa[T:], bb[T:])
            if h == heads[0]:
                dec = {h: tail}
            else:
                dec[h] = tail
    o, S = kda.chunk_prefill(q, k, v, a, b)
    torch.cuda.synchronize()
    flush("    prefill done")
    # decode: the checked heads carry their own stream; other heads get copies
    od = []
    for s in range(ND):
        dq = torch.stack([dec[heads[0]][0][s]] * H)[None].contiguous()
        dk = torch.stack([dec[heads[0]][1][s]] * H)[None].contiguous()
        dv = torch.stack([dec[heads[0]][2][s]] * H)[None].contiguous()
        da = torch.stack([dec[heads[0]][3][s]] * H)[None].contiguous()
        db = torch.stack([dec[heads[0]][4][s]] * H)[None].contiguous()
        for hh in heads[1:]:
            dq[0, hh], dk[0, hh], dv[0, hh] = dec[hh][0][s], dec[hh][1][s], dec[hh][2][s]
            da[0, hh], db[0, hh] = dec[hh][3][s], dec[hh][4][s]
        od.append(kda.decode_step(dq, dk, dv, da, db, S).clone())
    torch.cuda.synchronize()
    flush("    decode done")
    # oracle over the whole sequence for the checked heads (vectorised over them)
    fq = lambda t: t[0, :, heads].float().cpu().numpy()[None]  # noqa: E731
    o_ref, S_ref = kda_recurrent(fq(q), fq(k), fq(v), fq(a), b[0, :, heads].cpu().numpy()[None])
    flush("    oracle prefill done")
    d = [torch.stack([dec[hh][i] for hh in heads], dim=1).float().cpu().numpy()[None] for i in range(5)]
    od_ref, Sd_ref = kda_recurrent(d[0], d[1], d[2], d[3], d[4], S_ref)
    gS = host(S)[0, heads]
    e_state = max_rel_err(gS, Sd_ref[0])
    e_pre = max_rel_err(o[0][:, heads].cpu().numpy(), o_ref[0])
    e_dec = max_rel_err(np.stack([x[0, heads].cpu().numpy() for x in od]), od_ref[0])
    flush(f"    heads {heads}: prefill o (all {T} tokens)={e_pre:.2e} decode o={e_dec:.2e} final S={e_state:.2e}")
    assert e_pre <= TOL["bf16"] and e_dec <= TOL["bf16"] and e_state <= TOL["bf16"]
