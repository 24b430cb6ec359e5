"""Float64 CPU oracle for batched lossless draft verification and the SSD / Saguaro pieces.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. It shares no code with the HIP library, and the library never calls it.
Every function is pinned by ``tests/test_oracle_pins.py`` against facts the pages or mathematics fix
(closed forms, library routines, exact enumeration, brute force); none is "parity unpinned".
"""
from .ssd_oracle import (  # noqa: F401
    SampleResult,
    VerifyResult,
    all_hit_probability,
    backup_crossover,
    batch_speedup,
    branch_layout,
    cache_keys,
    cache_lookup,
    fanout,
    geometric_pk,
    logits_f64,
    saguaro,
    saguaro_sample,
    softmax_t,
    ssd_round,
    topf,
    verify_batch,
    verify_sequence,
)
