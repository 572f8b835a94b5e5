"""CPU oracle for the QSA hot path -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never calls it.  See ``qsa_oracle.c`` for the definitions it follows.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    pool,
    pool_rmsnorm,
    rope_rows,
    scores,
    select,
    score_rows,
    k_blocks,
    index_rows,
    attend_rows,
    prefill_rows,
    decode,
    index_at,
    score_at,
    attend_at,
    attend_shared,
    attend_backward,
    distill_rows,
    pool_backward,
)
