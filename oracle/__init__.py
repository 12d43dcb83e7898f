"""CPU oracles for MLA speculative-decoding verify attention, KV compaction and step metadata (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP path.
"""
from .mla_verify_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    merge_partials,
    split_bounds,
    verify_attention,
    verify_attention_rows,
    verify_attention_split,
    visible_count,
)
from .kv_compact_oracle import compact_rows  # noqa: F401,E402
from .metadata_oracle import build_step_metadata  # noqa: F401,E402
