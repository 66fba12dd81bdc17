"""CPU oracle for attention-score KV selection and compaction.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import or run anything in this package.
The GPU library and its Python binding never import it, and it imports
nothing from them; the only shared code is the seeded input generator
(``synth``), which holds none of the method's arithmetic.

Everything here is the plain, dense, slow definition written out in float64
numpy (the int4 rule is evaluated in float32 because its codes are decided in
float32; see ``quant_int4``).  See ``reference`` for the per-function sources.

Pin status: every public function is pinned by ``tests/test_oracle_pins.py``
(closed forms, brute force, invariants, the pages' printed memory figures).
No function is "parity unpinned".
"""
from .reference import (  # noqa: F401
    default_scale,
    logits,
    softmax_rows,
    head_scores,
    max_pool,
    select,
    select_head_adaptive,
    compact_flat,
    compact_rows,
    layer_end_compress,
    kara_scores,
    kara_select,
    window_sums,
    route_tiers,
    quant_int4,
    dequant_int4,
    round_bf16,
    pack_nibbles,
    tier_outputs,
    cache_bytes,
    TIER_FULL,
    TIER_QUANT,
    TIER_EVICT,
    quant_lowbit,
    pack_codes,
    unpack_codes,
    qevict_windows,
    qevict_init,
    qevict_step,
)
