"""CPU oracle for xKV (cross-layer low-rank KV compression + Selective Reconstruction).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (``kv_cache_cross_amd``) never imports it and has no CPU
fallback.  The oracle shares no code with the HIP path; the only module both
use is ``synth`` (seeded input generation, no method arithmetic).

Everything is plain NumPy in float64.  Inputs stored in bf16/fp32 are widened
exactly before use.  Pins that tie each function to the pages or to the
mathematics live in ``tests/test_oracle_*.py``.  Nothing in this package is
"parity unpinned".
"""
from .xkv_ref import (  # noqa: F401
    ROPE_THETA,
    rope,
    group_matrix,
    gram,
    eig_desc,
    compress_group,
    reconstruct_layer,
    landmarks,
    append_tokens,
    candidate_chunks,
    landmark_scores,
    select_topk,
    attended_positions,
    sr_decode_layer,
    dense_decode,
    numerical_rank,
    effective_rank,
    ner,
    energy_rank,
    allocate_ranks,
)
