"""fp64 CPU oracle for zero-copy host-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
package.  The product path (``decode_attention_host_amd``) never imports it and
shares no code with it: no kernels, headers, helpers, tables or constants.

Everything here is the plain definition, written out in float64 (numpy) with a
pure-Python scalar twin in :mod:`oracle.brute` for tiny shapes.

Parity pins: every function below is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants and brute force (see that file's cases).
"""
from .dkv_oracle import (  # noqa: F401
    bf16_to_f64,
    bf16_rne_bits,
    rope_inv_freq,
    rope_neox,
    project,
    attention,
    attention_subset,
    merge_lse,
    contig_split_point,
    contig_slot,
    paged_slot,
    decode_sequence,
    decode_sequence_split,
    decode_batch,
    prefill_sequence,
    append_expected_rows,
    linear,
    linear_split_rows,
    linear_split,
)
