"""Plain CPU oracle for KV compaction of a page_size = 1 latent cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only tests and the benchmark's checks do.  It shares no code with the HIP
kernels.

What it computes.  magik.net, "The Moment of Truth" (sections "The Broader
Context: From Kernel to System" and "Conclusion: A Pivotal Moment of
Validation") names KV defragmentation as a next step after the verify kernel
and graph capture, without describing it.  With page_size = 1 every token's
latent row sits in its own scattered slot ("The Decisive A/B", "The Context").
Reading taken here (the plainest one): defragmenting a request's cache copies
its rows, in key order, into one contiguous range of destination slots and
gives the request new slot indices pointing at that range.  The row bytes are
copied unchanged, so any attention computed over the new slots equals the one
over the old slots (the result does not depend on where the rows sit).
"""
from __future__ import annotations

import numpy as np


def compact_rows(kv_pool: np.ndarray, slot_idx: np.ndarray, dst_pool: np.ndarray, dst_first: int):
    """Copy row kv_pool[slot_idx[j]] to dst_pool[dst_first + j] for every j, in order.

    kv_pool, dst_pool: [slots, row] arrays of any dtype (bf16 kept as uint16 bits);
    dst_pool is modified in place and returned.  Returns (dst_pool, new_slot_idx)
    with new_slot_idx[j] = dst_first + j (int32).  Rows of dst_pool outside
    [dst_first, dst_first + len(slot_idx)) are left as they were.
    """
    slot_idx = np.asarray(slot_idx)
    n = len(slot_idx)
    if dst_first < 0 or dst_first + n > dst_pool.shape[0]:
        raise ValueError("destination range outside the destination pool")
    for j in range(n):
        dst_pool[dst_first + j] = kv_pool[int(slot_idx[j])]
    new_slot_idx = np.arange(dst_first, dst_first + n, dtype=np.int64).astype(np.int32)
    return dst_pool, new_slot_idx
