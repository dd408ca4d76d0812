"""fp64 CPU oracle for EAGLE target-verify attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The HIP library never does, and the oracle imports nothing
from the library.
"""

from .verify_attn_oracle import (  # noqa: F401
    allclose_report,
    attend,
    bf16_to_f64,
    block_table,
    decode_kv,
    e4m3fn_to_f64,
    lse_merge,
    problem_fields,
    run,
    run_block_table,
    run_split,
    translate_slots,
    verify_attention,
    verify_attention_split,
    visible_keys,
)
