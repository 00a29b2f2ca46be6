"""Plain CPU oracle of the KV-cache compression hot path (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP implementation in
``sparse_decode_amd`` and never imports it.
"""
from .ref import (  # noqa: F401
    block_landmarks,
    block_retrieval,
    block_scores,
    build,
    cache_bytes,
    decode,
    expand_blocks,
    gather,
    query_similarity,
    score_window,
    select_core,
    select_topk,
    set_threads,
    speculative_step,
)
