"""Oracle for the paged KV-cache hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation (numpy, fp64 for every
floating-point step) of what the hot path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path (``paged_kv_cache_38_amd``)
and imports nothing from it; the product path never calls it.

The oracle does not emulate paging, splitting or tiling.  Paged attention is
defined to give exactly the result of ordinary softmax attention over each
request's keys and values laid out contiguously in logical order (the vLLM-Omni
design notes, "Dense and paged representation"; the SGLang encoder-decoder
post, "Approach 2: gather and go ragged").  So the oracle resolves every
logical token to its slot, gathers, and attends in fp64.

Sources, cited by short name throughout:

* [XPU]     "Enabling Encoder-Decoder Models on Intel XPU in SGLang: A KV-Cache
            Story" (skrohit.github.io)
* [OMNI]    "Scheduler-Managed Paged KV Cache" (vLLM-Omni design documents)
* [MINI]    "The KV pool, the page table and the token pool" (mini-sglang from
            Scratch, Stage 1)
* [BACKEND] "AttentionBackend" (SGLang FlashInfer-MLA / FlashMLA backend notes)

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, brute force on tiny inputs, a library routine and
invariants; none is "parity unpinned".
"""
from .numerics import bf16_bits_to_f64, to_f64, f64_to_bf16_bits  # noqa: F401
from .pool import (  # noqa: F401
    kv_bytes_per_token,
    tokens_that_fit,
    pool_shape,
    per_token_shape,
    page_of,
    offset_of,
    store,
)
from .indices import (  # noqa: F401
    ceil_div,
    ceil_align,
    page_ids_from_token_table,
    build_csr,
    build_block_table,
    last_page_len,
    slots_from_token_table,
    slots_from_pages,
    slots_from_csr,
    slots_from_block_table,
    qo_indptr,
    token_indptr,
    in_page_contiguous,
)
from .attention import attend, paged_attention, merge_partials, gather, span_segments  # noqa: F401
from .alloc import (  # noqa: F401
    FreeRing,
    new_pages_needed,
    alloc,
    alloc_extend,
    alloc_decode,
    free_pages,
    pages_of_slots,
    write_req_to_token,
)
from .enc_cache import (  # noqa: F401
    write_blocks,
    merge_blocks,
    fill_counts,
    check_filled,
)
