"""MI355X-native paged KV-cache write and paged decode attention.

The compute lives in ``libpcache.so`` (hand-written HIP for gfx950, C ABI in
``include/pc.h``); this package only binds it.  Entry points mirror the C names:

* ``reshape_and_cache``        -- scatter new K/V rows through ``slot_mapping``;
* ``paged_attention_decode``   -- one-pass decode, or the 512-token split partials;
* ``paged_attention_reduce``   -- log-sum-exp merge of the partials;
* ``paged_attention_decode_prefix`` -- the split path's partials for sequences sharing a
  prefix, each shared tile read once for many sequences;
* ``paged_attention_plan``     -- the planner's choice between the two paths;
* ``paged_attention_plan_lens`` -- the same choice from the host's sequence lengths;
* ``reshape_and_cache_fp8`` / ``paged_attention_decode_fp8`` -- the same over an
  8-bit (OCP E4M3) pool with per-kv-head scales;
* ``paged_attention_varlen``   -- several query tokens per request (chunked
  prefill, speculative decode), causal, over the same pool;
* ``reshape_and_cache_decode`` -- a decode step's write and decode in one launch;
* ``paged_attention_split_noalloc`` -- the split decode and its reduce with the
  partials in the library's own device buffer, for callers that cannot allocate;
* ``stream_read``              -- measurement aid: one plain read of a buffer (the
  yardstick the benchmark quotes the decode's HBM rate against);
* ``gather_read``              -- measurement aid: the K/V tiles a decode of a batch
  reads, loads only.
"""

from ._native import (  # noqa: F401
    GATHER_SINK_WORDS,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    PARTITION_SIZE,
    PagedCacheError,
    abi_version,
    gather_read,
    library,
    paged_attention_decode,
    paged_attention_decode_prefix,
    paged_attention_decode_fp8,
    paged_attention_plan,
    paged_attention_plan_lens,
    paged_attention_reduce,
    paged_attention_split_noalloc,
    paged_attention_varlen,
    reshape_and_cache,
    reshape_and_cache_decode,
    reshape_and_cache_fp8,
    status_string,
    stream_read,
)
