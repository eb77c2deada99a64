"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on
the same seeded inputs, element by element, at sizes that span several
chunks, ragged tails and every slab width.  Bar: normwise max relative error
<= 2e-3 for bf16 q/k/v and <= 1e-5 for fp32 q/k/v."""

import numpy as np
import pytest
import torch

from gated_delta_rule_diag_amd import inputs as I
from gated_delta_rule_diag_amd import kda
from kda_testlib import TOL, dev, flush, host, random_state, tdtype
from oracle import kda_decode_step, kda_recurrent, kda_recurrent_varlen, max_rel_err

pytestmark = pytest.mark.gpu


def prefill_case(B, T, H, DK, DV, dt, c, with_state, seed=0):
    flush(f"[prefill] B={B} T={T} H={H} DK={DK} DV={DV} {dt} c={c} S0={with_state}")
    q, k, v, a, b = I.batch_inputs(c, B, T, H, DK, DV, dt)
    S0 = random_state(np.random.default_rng(seed), (B, H, DK, DV)) if with_state else None
    o_ref, S_ref = kda_recurrent(q, k, v, a, b, S0)
    td = tdtype(dt)
    o, S = kda.chunk_prefill(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b),
                             None if S0 is None else dev(S0))
    torch.cuda.synchronize()
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    return eo, es


def test_prefill_fp32_small_config():
    """B=1, H=2, T=256, d=64, fp32 inputs, zero initial state (bar 1e-5)."""
    eo, es = prefill_case(1, 256, 2, 64, 64, "f32", c=0, with_state=False)
    assert eo <= TOL["f32"] and es <= TOL["f32"]


PATHS = ["fused", "split"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 15, 63, 64, 65, 127, 200, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_bf16_shapes(T, d, path, monkeypatch):
    """Both prefill forms: the one-kernel form and the staged form (per-chunk
    operands computed for all chunks first, then the state pass)."""
    kda.set_tuning(prefill_form=path)
    eo, es = prefill_case(2, T, 3, d, d, "bf16", c=100 + T, with_state=True, seed=T)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 65, 200])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
def test_prefill_fp32_shapes(T, dk, dv, path, monkeypatch):
    kda.set_tuning(prefill_form=path)
    eo, es = prefill_case(1, T, 2, dk, dv, "f32", c=200 + T, with_state=True, seed=T)
    assert eo <= TOL["f32"] and es <= TOL["f32"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_prefill_bf16_rectangular(dk, dv, path, monkeypatch):
    kda.set_tuning(prefill_form=path)
    eo, es = prefill_case(2, 130, 2, dk, dv, "bf16", c=300, with_state=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("nsub", [1, 2, 4, 8])
def test_prefill_every_slab_width(nsub, path, monkeypatch):
    """The sequential pass is split into value slabs of 16*nsub columns; every
    width gives the oracle's result, in both prefill forms."""
    kda.set_tuning(prefill_nsub=nsub)
    kda.set_tuning(prefill_form=path)
    eo, es = prefill_case(1, 190, 2, 128, 128, "bf16", c=400, with_state=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("seg", [1, 2, 3])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_split_segments(seg, dt, monkeypatch):
    """The staged form processes long sequences in segments of chunks, the
    state carried between segments in the workspace: any segment length gives
    the oracle's result (7 chunks, ragged tail, nonzero initial state)."""
    kda.set_tuning(prefill_form="split")
    kda.set_tuning(prefill_seg=seg)
    eo, es = prefill_case(2, 7 * 64 - 9, 2, 128, 128, dt, c=410 + seg, with_state=True, seed=seg)
    assert eo <= TOL[dt] and es <= TOL[dt]


@pytest.mark.parametrize("path", PATHS)
def test_prefill_paths_agree_on_config_shape(path, monkeypatch):
    """B=1, H=32, T=1000, d=128, bf16 (32 heads, as in the 8192-token workload): both forms
    against the oracle."""
    kda.set_tuning(prefill_form=path)
    eo, es = prefill_case(1, 1000, 32, 128, 128, "bf16", c=420, with_state=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_varlen_small():
    lengths = [5, 0, 70, 1, 64, 130, 33]
    H, d = 3, 128
    flush(f"[varlen] lengths={lengths}")
    q, k, v, a, b, cu = I.packed_inputs(500, lengths, H, d, d, "bf16")
    S0 = random_state(np.random.default_rng(5), (len(lengths), H, d, d))
    o_ref, S_ref = kda_recurrent_varlen(q, k, v, a, b, cu, S0)
    td = torch.bfloat16
    o, S = kda.chunk_prefill_varlen(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b),
                                    torch.from_numpy(cu).cuda(), dev(S0))
    torch.cuda.synchronize()
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("N", [256, 257])
def test_varlen_many_sequences_ranked_and_unranked(N):
    """Packed batches of up to 256 sequences are taken longest first (each
    workgroup ranks the lengths on the device), larger ones in pack order:
    both sides of the limit, with many equal lengths and empty sequences,
    against the oracle."""
    lengths = np.random.default_rng(N).integers(0, 100, N)
    H, d = 1, 64
    flush(f"[varlen] N={N} sequences, {int(lengths.sum())} tokens, {int((lengths == 0).sum())} empty")
    q, k, v, a, b, cu = I.packed_inputs(510, lengths, H, d, d, "f32")
    S0 = random_state(np.random.default_rng(511), (N, H, d, d))
    o_ref, S_ref = kda_recurrent_varlen(q, k, v, a, b, cu, S0)
    o, S = kda.chunk_prefill_varlen(dev(q), dev(k), dev(v), dev(a), dev(b), torch.from_numpy(cu).cuda(),
                                    dev(S0))
    torch.cuda.synchronize()
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


@pytest.mark.parametrize("N,H,DK,DV,dt", [(3, 2, 64, 64, "f32"), (5, 3, 128, 128, "bf16"),
                                          (2, 4, 128, 64, "bf16"), (2, 2, 64, 128, "f32")])
def test_decode_small(N, H, DK, DV, dt):
    flush(f"[decode] N={N} H={H} DK={DK} DV={DV} {dt}")
    q, k, v, a, b = I.decode_inputs(600, N, H, DK, DV, dt)
    S0 = random_state(np.random.default_rng(N), (N, H, DK, DV))
    o_ref, S_ref = kda_decode_step(q, k, v, a, b, S0)
    td = tdtype(dt)
    S = dev(S0)
    o = kda.decode_step(dev(q, td), dev(k, td), dev(v, td), dev(a), dev(b), S)
    torch.cuda.synchronize()
    eo, es = max_rel_err(host(o), o_ref), max_rel_err(host(S), S_ref)
    flush(f"    err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL[dt] and es <= TOL[dt]
