"""Oracle package: plain fp64 CPU reference of rational-softmax attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
Pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_pins.py``.
"""
from .ra_oracle import (  # noqa: F401
    SUPPORT_WIDTH,
    causal_offset,
    ra_attention_bwd,
    ra_attention_decode,
    ra_attention_fwd,
    ra_attention_rope_bwd,
    ra_attention_rope_fwd,
    ra_phi,
    ra_softmax_rows,
    ra_softmax_rows_bwd,
    rope_neox,
)
