"""specverify: the speculative-decoding verification step on AMD MI355X.

The computation lives in libspecverify.so (hand-written gfx950 HIP kernels
behind the C ABI of include/specverify.h); this package is its thin Python
binding plus the seeded synthetic workload generators.
"""
from ._abi import (  # noqa: F401
    FLAG_RECORDS_READY, FLAG_TOPP_TARGET_ONLY, MAX_SHARDS, POISON_BF16, ROW_BAD_ACCEPTED,
    ROW_BAD_K, ROW_BAD_PAGES, ROW_BAD_TEMPERATURE, ROW_BAD_TOKEN, ROW_BAD_TOP_P,
    ROW_FREE_OVERFLOW, ROW_NO_FINITE, ROW_NONFINITE_LOGIT, RollbackCall, ShardedCall,
    SpecVerifyError, VerifyCall, advance_offset, close_round, draft_sample, draft_sample_sharded,
    dynamic_k, dynk_state, kv_rollback, library, shard_bounds, timing_enable, timing_read,
    verify_greedy, verify_sample, verify_sample_noalloc, verify_sample_sharded,
    noalloc_scratch_bytes,
)
