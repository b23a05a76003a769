"""CPU oracle for the paged KV-cache hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and this
package imports nothing from the product path.

See ``oracle.paged_attention`` for the definitions and their citations.
"""

from .paged_attention import (  # noqa: F401
    BF16,
    FP32,
    append_kv,
    attention_rows,
    bits_to_f64,
    copy_blocks,
    decode,
    gather_sequence,
    prefill,
    query_position,
    visible_keys,
)
