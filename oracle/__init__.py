"""CPU oracle for the DuoLM multi-item-scoring (MIS) ranker forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of the benchmark use it.  It shares no code with the HIP
library and imports nothing from it.

It is plain NumPy in float64, written for a reader to check against the pages
by eye: no blocking, no fusion, no reordering beyond the definitions.
"""
from .ranker import (  # noqa: F401
    OracleModel,
    attention,
    brute_force_independent,
    decode_incremental,
    decoder_forward,
    embed_rows,
    layer_stages,
    mlp_swiglu,
    oracle_mis,
    oracle_mis_packed,
    pair_count,
    rmsnorm,
    rope_rotate,
    score_head,
    tree_mask,
    widen_bf16,
    widen_f16,
)
from .export import (  # noqa: F401
    export_table,
    interface_vectors,
    midpoint_distance,
    reference_scale,
    rms,
    to_fp16_bits,
)
