"""Reference oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the tests, the graft entry's smoke check and the benchmark's
CPU-baseline leg do.  It is a plain, slow, obviously correct CPU model written
from the pages, in float64 for the attention arithmetic, and it shares no code
with the HIP library or its binding.

Sources (four web pages about the PagedAttention / vLLM paper):
  [P1] lain42.top reading note on "Efficient Memory Management for Large
       Language Model Serving with PagedAttention" (abstract + summary).
  [P2] aiplusplus.yigather.com explainer "PagedAttention: bringing the OS
       virtual-memory idea into LLM inference" (sections: core idea, key
       technical points 1-4).
  [P3] auturnal.com analytical guide "paged-attention-serving" (sections 1-6,
       "Equations and derivations" Eq. (1)-(3), "Worked calculation",
       "Verification protocol").
  [P4] cayang0802.github.io blog "paged-attention" (KV block / block table
       figure, sharing, preemption).

Modules:
  closed_forms  Eq. (1)-(3) of [P3]: KV bytes, allocated slots, tail waste,
                slot utilisation.
  allocator     block pool with a FIFO free queue, refcounts, fork, free,
                copy-on-write appends, swapping to a host tier, prefix keys
                and rollback by truncation.
  cache         the physical cache layout, scatter of token K/V into slots,
                whole-block copies and the gather through a block table.
  attention     contiguous scaled dot-product attention in float64, the paged
                variant (gather, then contiguous), the split-context
                log-sum-exp combination, and runs of causal queries per
                sequence (prefill, speculative verification).
  run           replays a workload's allocator script with the pieces above.

Every function here is pinned by CPU tests against values printed on the pages,
closed forms, special cases and invariants; none is marked "parity unpinned".
"""

from . import closed_forms, allocator, cache, attention, run  # noqa: F401
