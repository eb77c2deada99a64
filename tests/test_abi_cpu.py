"""C ABI checks that run without a GPU: the library loads, exports every
symbol include/kda.h declares, and rejects invalid arguments on the host
(before any HIP call, so nothing is enqueued).  Device pointers below are
fake addresses: the host code never dereferences them."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# KDA_ABI_LIB: another build of the same sources (the sanitizer build runs
# this file against its own library).
LIB = os.environ.get("KDA_ABI_LIB") or os.path.join(ROOT, "gated_delta_rule_diag_amd", "libkda.so")
HEADER = os.path.join(ROOT, "include", "kda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libkda.so not built")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, HIP = range(8)


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_diag_amd.kda import load_library

    return load_library(LIB)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name


def test_binding_lists_every_declared_symbol():
    from gated_delta_rule_diag_amd.kda import EXPORTED

    assert sorted(EXPORTED) == declared_functions()


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() >> 16 == 1
    for s, name in enumerate(["KDA_OK", "KDA_ERR_NULL", "KDA_ERR_SHAPE", "KDA_ERR_DTYPE",
                              "KDA_ERR_ALIGN", "KDA_ERR_UNSUPPORTED", "KDA_ERR_WORKSPACE",
                              "KDA_ERR_HIP"]):
        assert lib.kda_status_string(s).decode() == name


P = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(12)]  # distinct, 16-byte aligned


def prefill(lib, B=1, T=64, H=2, DK=64, DV=64, chunk=64, dt=1, ptrs=None, ws=None, wsb=0):
    q, k, v, a, b, s_in, o, s_out = ptrs or P[:8]
    return lib.kda_chunk_prefill(B, T, H, DK, DV, chunk, dt, q, k, v, a, b, s_in, o, s_out, ws, wsb,
                                 None)


def test_prefill_argument_errors(lib):
    assert prefill(lib, DK=96) == UNSUP
    assert prefill(lib, DV=32) == UNSUP
    assert prefill(lib, chunk=32) == UNSUP
    assert prefill(lib, dt=7) == DTYPE
    assert prefill(lib, T=-1) == SHAPE
    assert prefill(lib, H=65537) == UNSUP      # 32-bit row offsets inside a chunk
    assert prefill(lib, H=-2) == SHAPE
    p = list(P[:8])
    p[0] = None
    assert prefill(lib, ptrs=p) == NULL
    p = list(P[:8])
    p[3] = ctypes.c_void_p(0x100004)
    assert prefill(lib, ptrs=p) == ALIGN
    assert "alpha" in lib.kda_last_error_message().decode()
    # o overlapping v
    p = list(P[:8])
    p[6] = ctypes.c_void_p(P[2].value + 64)
    assert prefill(lib, ptrs=p) == SHAPE
    # state_out overlapping q (but state_out == state_in is fine: not an error here,
    # checked without launching by using an empty batch)
    p = list(P[:8])
    p[7] = P[0]
    assert prefill(lib, ptrs=p) == SHAPE


def test_prefill_empty_is_ok_without_launch(lib):
    # B = 0 or H = 0: nothing to do, nothing launched.
    assert prefill(lib, B=0) == OK
    assert prefill(lib, H=0) == OK
    p = list(P[:8])
    p[7] = p[5]  # in place
    assert prefill(lib, B=0, ptrs=p) == OK


def test_workspace_size_queries(lib, monkeypatch):
    # staged form (few chains): one slot per (chunk, sequence, head) holding
    # W, Qg [64 x DK], Kg [DK x 64], P [64 x 64], Uv [64 x DV] at 4 bytes per
    # element, plus gamma_n [DK]
    slot = lambda dk, dv=128: 4 * (3 * 64 * dk + 64 * 64 + 64 * dv + dk)  # noqa: E731
    assert slot(128) == 147968 and slot(64, 64) == 82176
    # segments: at most floor(160 MiB / (pairs * slot)) chunks, the chunks
    # split into equal segments; a state is carried between segments
    def seg(pairs, nchunks, dk=128, dv=128):
        cap = max(1, (160 << 20) // (pairs * slot(dk, dv)))
        if cap >= nchunks:
            return nchunks
        nseg = -(-nchunks // cap)
        return -(-nchunks // nseg)

    def ws(pairs, nchunks, dk=128, dv=128):
        s = seg(pairs, nchunks, dk, dv)
        return pairs * s * slot(dk, dv) + (pairs * dk * dv * 4 if s < nchunks else 0)

    assert seg(32, 128) == 32                      # B=1, H=32, T=8192: 4 segments of 32
    assert lib.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128, 64) == \
        32 * 32 * slot(128) + 32 * 128 * 128 * 4
    assert lib.kda_chunk_prefill_workspace_size(2, 130, 3, 64, 128, 64) == 6 * 3 * slot(64)
    assert lib.kda_chunk_prefill_workspace_size(1, 1 << 20, 32, 128, 128, 64) == ws(32, 1 << 14)
    assert lib.kda_chunk_prefill_workspace_size(1, 4096, 8, 128, 128, 64) == ws(8, 64)
    assert ws(8, 64) == 8 * 64 * slot(128)         # fits: one segment, no carried state
    assert lib.kda_internal_set_tuning(0, 0, 5, 0) == OK    # 5 chunks per segment
    assert lib.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128, 64) == \
        32 * 5 * slot(128) + 32 * 128 * 128 * 4
    assert lib.kda_internal_set_tuning(0, 0, 0, 0) == OK
    # one chunk, many chains, varlen, unsupported sizes: no workspace
    assert lib.kda_chunk_prefill_workspace_size(1, 64, 32, 128, 128, 64) == 0
    assert lib.kda_chunk_prefill_workspace_size(4, 8192, 32, 128, 128, 64) == 0
    assert lib.kda_chunk_prefill_varlen_workspace_size(64, 540000, 32, 128, 128, 64) == 0
    assert lib.kda_chunk_prefill_workspace_size(1, 64, 2, 96, 64, 64) == 0
    assert lib.kda_internal_set_tuning(1, 0, 0, 0) == OK    # one-kernel form
    assert lib.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128, 64) == 0
    assert lib.kda_internal_set_tuning(2, 0, 0, 0) == OK    # staged form
    assert lib.kda_chunk_prefill_workspace_size(4, 8192, 32, 128, 128, 64) == ws(128, 128)
    assert lib.kda_internal_set_tuning(0, 0, 0, 0) == OK
    # out-of-range overrides are refused and change nothing
    assert lib.kda_internal_set_tuning(3, 0, 0, 0) == SHAPE
    assert lib.kda_internal_set_tuning(0, 3, 0, 0) == SHAPE
    assert lib.kda_internal_set_tuning(0, 0, -1, 0) == SHAPE
    assert lib.kda_internal_set_tuning(0, 0, 0, -2) == SHAPE
    assert lib.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128, 64) == \
        32 * 32 * slot(128) + 32 * 128 * 128 * 4
    # a call that needs a workspace is refused without one, or with one too small
    # (B=1, T=130, H=2, d=64: 3 chunks x 2 chains)
    need = 2 * 3 * slot(64, 64)
    assert lib.kda_chunk_prefill_workspace_size(1, 130, 2, 64, 64, 64) == need
    assert prefill(lib, T=130) == WS
    assert prefill(lib, T=130, ws=P[9], wsb=need - 1) == WS
    assert "workspace" in lib.kda_last_error_message().decode()
    assert prefill(lib, T=130, ws=ctypes.c_void_p(P[9].value + 8), wsb=need) == ALIGN


def test_snapshot_argument_errors(lib):
    # B=1, T=128, H=2, d=64: two chunks x two chains, staged form (workspace
    # 2 * 2 * 82176 bytes); snapshots [1, 2, 2, 64, 64] float = 64 KiB
    need = lib.kda_chunk_prefill_workspace_size(1, 128, 2, 64, 64, 64)
    assert need == 4 * 82176

    def call(B=1, T=128, H=2, DK=64, every=1, snap=P[10], ws=P[9], wsb=need, ptrs=None):
        return lib.kda_chunk_prefill_snapshots(B, T, H, DK, 64, 64, 1, *(ptrs or P[:8]), every, snap,
                                               ws, wsb, None)

    assert call(every=0) == SHAPE
    assert call(every=-3) == SHAPE
    assert call(DK=96) == UNSUP
    assert call(snap=None) == NULL
    assert "snapshots" in lib.kda_last_error_message().decode()
    assert call(snap=ctypes.c_void_p(P[10].value + 4)) == ALIGN
    assert call(snap=ctypes.c_void_p(P[6].value + 4096)) == SHAPE      # inside o
    assert call(snap=ctypes.c_void_p(P[0].value - 4096)) == SHAPE      # runs into q
    assert call(ws=ctypes.c_void_p(P[10].value + 65536 - 16)) == SHAPE  # workspace over snapshots
    assert call(ws=None) == WS
    # nothing to write: B = 0, or H = 0
    assert call(B=0, snap=None) == OK
    assert call(H=0, snap=None) == OK


def test_workspace_must_not_overlap_arguments(lib):
    need = lib.kda_chunk_prefill_workspace_size(1, 130, 2, 64, 64, 64)
    assert prefill(lib, T=130, ws=ctypes.c_void_p(P[6].value + 256), wsb=need) == SHAPE
    assert "workspace" in lib.kda_last_error_message().decode()
    assert prefill(lib, T=130, ws=ctypes.c_void_p(P[0].value - 256), wsb=need) == SHAPE


def test_varlen_argument_errors(lib):
    def call(N=2, Tt=100, cu=P[8], H=2, DK=128, DV=128, chunk=64, dt=1):
        return lib.kda_chunk_prefill_varlen(N, Tt, cu, H, DK, DV, chunk, dt, *P[:8], None, 0, None)

    assert call(cu=None) == NULL
    assert call(cu=ctypes.c_void_p(0x100002)) == ALIGN
    assert call(N=-1) == SHAPE
    assert call(DK=32) == UNSUP
    assert call(chunk=128) == UNSUP
    assert call(N=0, Tt=0) == OK


def test_varlen_snapshot_argument_errors(lib):
    # N=2, T_total=100, H=2, d=64; 2 snapshot rows of [2, 64, 64] float = 64 KiB.
    # The packed form needs no workspace.  No call below reaches a launch.
    need = lib.kda_chunk_prefill_varlen_workspace_size(2, 100, 2, 64, 64, 64)
    assert need == 0

    def call(N=2, Tt=100, cu=P[8], every=1, offs=P[11], rows=2, snap=P[10], ws=P[9], wsb=need):
        return lib.kda_chunk_prefill_varlen_snapshots(N, Tt, cu, 2, 64, 64, 64, 1, *P[:8], every,
                                                      offs, rows, snap, ws, wsb, None)

    assert call(every=0) == SHAPE
    assert call(rows=-1) == SHAPE
    assert call(offs=None) == NULL
    assert "snap_offsets" in lib.kda_last_error_message().decode()
    assert call(offs=ctypes.c_void_p(P[11].value + 2)) == ALIGN
    assert call(cu=None) == NULL
    assert call(snap=None) == NULL
    assert call(snap=ctypes.c_void_p(P[10].value + 4)) == ALIGN
    assert call(snap=ctypes.c_void_p(P[6].value + 4096)) == SHAPE      # inside o
    assert call(snap=ctypes.c_void_p(P[8].value - 4096)) == SHAPE      # runs into cu_seqlens
    assert call(offs=ctypes.c_void_p(P[10].value + 4096)) == SHAPE     # offsets inside snapshots
    # no rows: snapshots may be NULL; N = 0 needs no offsets
    assert call(rows=0, snap=None, ws=None, wsb=0, N=0, Tt=0, offs=None, cu=None) == OK


def test_decode_argument_errors(lib):
    def call(N=4, H=2, DK=128, DV=128, dt=1, ptrs=None):
        q, k, v, a, b, s, o = ptrs or P[:7]
        return lib.kda_decode_step(N, H, DK, DV, dt, q, k, v, a, b, s, o, None)

    assert call(DK=100) == UNSUP
    assert call(dt=3) == DTYPE
    assert call(N=-4) == SHAPE
    p = list(P[:7])
    p[5] = None
    assert call(ptrs=p) == NULL
    p = list(P[:7])
    p[6] = ctypes.c_void_p(P[5].value + 16)  # o inside the state
    assert call(ptrs=p) == SHAPE
    p = list(P[:7])
    p[2] = ctypes.c_void_p(0x100008)
    assert call(ptrs=p) == ALIGN
    assert call(N=0) == OK


def test_scalar_gate_argument_errors(lib):
    # the gate is [B,T,H] floats: an o placed right after a [B,T,H,DK]-sized
    # alpha region would overlap a per-channel alpha but not the gate
    B, T, H, DK = 1, 64, 2, 64
    gate_bytes = B * T * H * 4
    p = list(P[:8])
    p[6] = ctypes.c_void_p(P[3].value + gate_bytes)          # o just after the gate
    args = (B, T, H, DK, 64, 64, 1)
    assert lib.kda_chunk_prefill(*args, *p, None, 0, None) == SHAPE
    p[6] = ctypes.c_void_p(P[3].value + gate_bytes - 16)     # o over the gate's end
    assert lib.kda_chunk_prefill_scalar_gate(*args, *p, None, 0, None) == SHAPE
    assert lib.kda_chunk_prefill_scalar_gate(1, 64, 2, 96, 64, 64, 1, *P[:8], None, 0, None) == UNSUP
    assert lib.kda_chunk_prefill_scalar_gate(0, 64, 2, 64, 64, 64, 1, *P[:8], None, 0, None) == OK
    assert lib.kda_chunk_prefill_varlen_scalar_gate(2, 100, None, 2, 64, 64, 64, 1, *P[:8], None, 0,
                                                    None) == NULL
    assert lib.kda_decode_step_scalar_gate(4, 2, 64, 64, 9, *P[:7], None) == DTYPE
    d = list(P[:7])
    d[6] = ctypes.c_void_p(P[3].value + 4 * 2 * 4 - 16)       # o over the [4,2] gate
    assert lib.kda_decode_step_scalar_gate(4, 2, 64, 64, 1, *d, None) == SHAPE
    assert lib.kda_decode_step_scalar_gate(0, 2, 64, 64, 1, *P[:7], None) == OK


def test_backward_argument_errors(lib):
    # B=1, T=64, H=2, d=64 (f32): rows = 128
    need = lib.kda_chunk_backward_workspace_size(1, 64, 2, 64, 64, 64)
    # the window buffers of one chunk for the 2 heads (A_c, b_c, dS', M, P/X,
    # Vn and the 93 rows of decays: 64^2 + 2 * 64^2 + 64^2 + 64^2 + 64 * 64 +
    # 93 * 64 floats each), one snapshot per sequence-head
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    win = 2 * (6 * 64 * 64 + 93 * 64) * 4
    assert need == al(win) + al(2 * 64 * 64 * 4)
    assert lib.kda_chunk_backward_workspace_size(1, 64, 2, 96, 64, 64) == 0
    big = ctypes.c_void_p(0x40000000)
    Q = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(14)]

    def call(T=64, DK=64, dt=0, ptrs=None, ws=big, wsb=need):
        return lib.kda_chunk_backward(1, T, 2, DK, 64, 64, dt, *(ptrs or Q), ws, wsb, None)

    assert call(DK=32) == UNSUP
    assert call(dt=4) == DTYPE
    assert call(T=-1) == SHAPE
    p = list(Q)
    p[5] = None                                    # state_in may be NULL ...
    p[0] = None                                    # ... q may not
    assert call(ptrs=p) == NULL
    p = list(Q)
    p[9] = ctypes.c_void_p(Q[9].value + 8)         # dk misaligned
    assert call(ptrs=p) == ALIGN
    p = list(Q)
    p[8] = ctypes.c_void_p(Q[6].value + 64)        # dq over d_o
    assert call(ptrs=p) == SHAPE
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=ctypes.c_void_p(Q[0].value)) == SHAPE   # workspace over q
    p = list(Q)
    p[13] = None                                   # T = 0 and no d_state_in: nothing to do
    assert call(T=0, ptrs=p) == OK


def test_backward_varlen_argument_errors(lib, monkeypatch):
    # N=3 sequences, T_total=200 tokens, longest 100, H=2, d=64 (f32): the
    # reverse pass's buffers cover a window of chunks counted from each
    # sequence's end, N * H * (DK^2 + 2 DK DV + 2 * 64^2 + 64 DV + 93 DK)
    # floats per chunk of the window (at most 4 GiB, here every chunk:
    # ceil(100 / 64) = 2); snapshot rows T_total // 64 = 3 (chunk j of the
    # sequence starting at token s is row s // 64 + j)
    per_chunk = 3 * 2 * (6 * 64 * 64 + 93 * 64) * 4
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    rest = al(3 * 2 * 64 * 64 * 4)
    need = lib.kda_chunk_backward_varlen_workspace_size(3, 200, 100, 2, 64, 64, 64)
    assert need == al(2 * per_chunk) + rest
    # max_seqlen unknown (0): T_total is assumed, 4 chunks
    assert lib.kda_chunk_backward_varlen_workspace_size(3, 200, 0, 2, 64, 64, 64) == \
        al(4 * per_chunk) + rest
    # one chunk per window: two windows, and the adjoint carried between them
    assert lib.kda_internal_set_tuning(0, 0, 0, 1) == OK
    assert lib.kda_chunk_backward_varlen_workspace_size(3, 200, 100, 2, 64, 64, 64) == \
        al(per_chunk) + rest + al(3 * 2 * 64 * 64 * 4)
    assert lib.kda_internal_set_tuning(0, 0, 0, 0) == OK
    # max_seqlen below the longest sequence (not checked): one window of
    # ceil(64 / 64) = 1 chunk and no carried adjoint (nothing to carry into)
    assert lib.kda_chunk_backward_varlen_workspace_size(3, 200, 64, 2, 64, 64, 64) == \
        al(per_chunk) + rest
    assert lib.kda_chunk_backward_varlen_workspace_size(3, 200, 100, 2, 96, 64, 64) == 0
    assert lib.kda_chunk_backward_varlen_workspace_size(3, 0, 0, 2, 64, 64, 64) == 0
    big = ctypes.c_void_p(0x40000000)
    Q = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(14)]
    cu = ctypes.c_void_p(0x2000000)

    def call(N=3, Tt=200, cu=cu, DK=64, ptrs=None, ws=big, wsb=need):
        return lib.kda_chunk_backward_varlen(N, Tt, cu, 100, 2, DK, 64, 64, 0, *(ptrs or Q), ws,
                                             wsb, None)

    assert call(N=-1) == SHAPE
    assert call(Tt=-5) == SHAPE
    assert call(cu=None) == NULL
    assert "cu_seqlens" in lib.kda_last_error_message().decode()
    assert call(cu=ctypes.c_void_p(cu.value + 2)) == ALIGN
    assert call(DK=32) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    p = list(Q)
    p[8] = ctypes.c_void_p(Q[6].value + 64)        # dq over d_o
    assert call(ptrs=p) == SHAPE
    assert call(cu=ctypes.c_void_p(Q[8].value + 64)) == SHAPE   # dq over cu_seqlens
    assert call(N=0, cu=None) == OK
    p = list(Q)
    p[13] = None
    assert call(Tt=0, ptrs=p) == OK                # no tokens, no d_state_in: nothing to do


def test_backward_scalar_gate_argument_errors(lib):
    # B=1, T=64, H=2, d=64 (f32); the gate and its gradient are [B,T,H]
    need = lib.kda_chunk_backward_workspace_size(1, 64, 2, 64, 64, 64)
    big = ctypes.c_void_p(0x40000000)
    Q = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(14)]

    def call(T=64, DK=64, ptrs=None, ws=big, wsb=need):
        return lib.kda_chunk_backward_scalar_gate(1, T, 2, DK, 64, 64, 0, *(ptrs or Q), ws, wsb,
                                                  None)

    assert call(DK=32) == UNSUP
    assert call(T=-1) == SHAPE
    p = list(Q)
    p[3] = None                                    # gate
    assert call(ptrs=p) == NULL
    assert call(ws=None) == WS
    # a [B,T,H] gate is 512 bytes: dgate 256 bytes past its start overlaps it
    p = list(Q)
    p[9] = ctypes.c_void_p(Q[3].value + 256)
    assert call(ptrs=p) == SHAPE
    p = list(Q)
    p[13] = None
    assert call(T=0, ptrs=p) == OK

    def vcall(N=2, Tt=100, cu=ctypes.c_void_p(0x2000000), wsb=1 << 30):
        return lib.kda_chunk_backward_varlen_scalar_gate(N, Tt, cu, 0, 2, 64, 64, 64, 0, *Q, big,
                                                         wsb, None)

    assert vcall(cu=None) == NULL
    assert vcall(cu=ctypes.c_void_p(0x2000002)) == ALIGN
    assert vcall(N=-1) == SHAPE
    assert vcall(wsb=16) == WS


def test_decode_pool_argument_errors(lib):
    def call(N=4, L=2, H=2, DK=128, DV=128, dt=1, idx=P[9], ntok=P[10], pool=P[5], P_=8, o=P[6],
             ts=None, ptrs=None):
        q, k, v, a, b = ptrs or P[:5]
        return lib.kda_decode_pool(N, L, H, DK, DV, dt, q, k, v, a, b, idx, ntok, pool, P_, o, ts,
                                   None)

    assert call(L=0) == UNSUP
    assert call(L=65) == UNSUP
    assert call(DV=96) == UNSUP
    assert call(dt=5) == DTYPE
    assert call(N=-1) == SHAPE
    assert call(P_=-1) == SHAPE
    assert call(idx=None, P_=3) == SHAPE                 # slot n needs pool_size >= N
    assert call(pool=None) == NULL
    assert call(o=None) == NULL
    assert call(idx=ctypes.c_void_p(P[9].value + 2)) == ALIGN
    assert call(ts=ctypes.c_void_p(P[11].value + 8)) == ALIGN
    assert call(o=ctypes.c_void_p(P[2].value + 16)) == SHAPE           # o over v
    assert call(pool=ctypes.c_void_p(P[0].value + 1024)) == SHAPE      # pool over q
    assert call(ts=ctypes.c_void_p(P[6].value + 1024)) == SHAPE        # token states over o
    assert call(o=ctypes.c_void_p(P[9].value)) == SHAPE                # o over state_idx
    assert call(N=0) == OK
    assert call(H=0) == OK


def test_binding_fails_loudly_without_library(tmp_path):
    from gated_delta_rule_diag_amd.kda import load_library

    with pytest.raises(ImportError):
        load_library(str(tmp_path / "missing.so"))


def test_noalloc_prefill_rejects_what_the_scratch_cannot_hold(lib):
    # 512 (sequence, head) pairs forced into the staged form: one chunk of
    # slots (512 * 147,968 B) and the carried state exceed the 64 MiB static
    # scratch; refused on the host, nothing enqueued
    # (distinct tensors, far enough apart not to overlap at these sizes)
    q, k, v, a, b, s_in, o, s_out = [ctypes.c_void_p(0x100000000 * (i + 1)) for i in range(8)]
    assert lib.kda_internal_set_tuning(2, 0, 0, 0) == OK
    try:
        st = lib.kda_chunk_prefill_noalloc(4, 128, 128, 128, 128, 64, 1, q, k, v, a, b, s_in, o,
                                           s_out, None)
        assert st == UNSUP
        assert "scratch" in lib.kda_last_error_message().decode()
    finally:
        assert lib.kda_internal_set_tuning(0, 0, 0, 0) == OK
    # argument errors as for kda_chunk_prefill; nothing to do for B = 0
    assert lib.kda_chunk_prefill_noalloc(1, 64, 2, 96, 64, 64, 1, q, k, v, a, b, s_in, o, s_out,
                                         None) == UNSUP
    assert lib.kda_chunk_prefill_noalloc(1, 64, 2, 64, 64, 32, 1, q, k, v, a, b, s_in, o, s_out,
                                         None) == UNSUP
    assert lib.kda_chunk_prefill_noalloc(-1, 64, 2, 64, 64, 64, 1, q, k, v, a, b, s_in, o, s_out,
                                         None) == SHAPE
    assert lib.kda_chunk_prefill_noalloc(0, 64, 2, 64, 64, 64, 1, q, k, v, a, b, s_in, o, s_out,
                                         None) == OK


def test_bench_blob_ids_match_git_hash_object():
    """bench.py names the measured files by their git blob ids: the same ids
    `git hash-object` gives (checked where git and the history are present)."""
    import shutil
    import subprocess

    import bench

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    ids = bench.source_blob_ids(root)
    assert "gated_delta_rule_diag_amd/csrc/kda_prefill.hip" in ids and "include/kda.h" in ids
    if shutil.which("git") is None or not os.path.isdir(os.path.join(root, ".git")):
        pytest.skip("no git history here")
    for rel, blob in ids.items():
        out = subprocess.run(["git", "-C", root, "hash-object", rel], capture_output=True, text=True)
        assert out.returncode == 0 and out.stdout.strip()[:12] == blob, rel
