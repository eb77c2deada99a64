"""Plain, slow, fp64 CPU oracle for the Kimi Delta Attention (KDA) operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (``gated_delta_rule_diag_amd``) and imports nothing from it.
"""

from .kda_oracle import (  # noqa: F401
    kda_recurrent,
    kda_recurrent_varlen,
    kda_recurrent_snapshots,
    gdn_recurrent,
    kda_backward,
    gdn_backward,
    kda_decode_step,
    kda_decode_pool,
    kda_chunked,
    max_rel_err,
)
