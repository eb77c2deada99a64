"""Kimi Delta Attention (KDA) operator for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (``include/kda.h``, ``libkda.so``)
with a thin ctypes binding:

    chunk_prefill(q, k, v, alpha, beta, initial_state=None) -> (o, final_state)
    chunk_prefill_snapshots(q, k, v, alpha, beta, every, initial_state=None)
        -> (o, final_state, snapshots)
    chunk_prefill_varlen(q, k, v, alpha, beta, cu_seqlens, initial_state=None)
    decode_step(q, k, v, alpha, beta, state) -> o        (state updated in place)
    chunk_backward(q, k, v, alpha, beta, d_o, initial_state=None, d_final_state=None)
        -> (dq, dk, dv, dalpha, dbeta, d_initial_state)
    decode_pool(q, k, v, alpha, beta, state_pool, state_idx=None, num_tokens=None)
        -> (o, token_states)                             (L tokens per sequence, pooled states)

The binding is imported lazily so that ``gated_delta_rule_diag_amd.inputs``
(seeded workload generation, numpy only) does not need torch.
"""

__all__ = ["chunk_prefill", "chunk_prefill_snapshots", "chunk_prefill_varlen", "decode_step",
           "decode_pool", "chunk_backward", "KDAError"]


def __getattr__(name):
    if name in __all__:
        from . import kda

        return getattr(kda, name)
    raise AttributeError(name)
