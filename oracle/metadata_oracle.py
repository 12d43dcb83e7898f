"""Plain CPU oracle for the per-step metadata of a verify call.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only tests and the benchmark's checks do.  It shares no code with the HIP
kernels.

What it computes.  magik.net, "The Moment of Truth": the short-context loss
is put down to host-side marshaling that builds the kernel's index arrays
and copies them to the GPU once per layer; the remedies named are building
the combined indices once per step ("Interpreting the Crossover: The
Marshaling Tax"), making the call capturable by overriding the metadata
replay logic with pre-allocated static buffers ("The Thinking Process"), and
a marshaling kernel that runs on the GPU ("Assumptions and Their Validity").
Reading taken here: the serving side keeps a request-to-token table whose
row r lists, in position order, the cache slot of every token of the request
held in row r (page_size = 1).  For one step over `batch` requests, request
b sits in table row req_ids[b], has prefix_lens[b] tokens cached before this
step and draft_lens[b] draft tokens whose rows are already written at the
next positions.  The verify call then needs
    seq_lens[b] = prefix_lens[b] + draft_lens[b]
    q_lens[b]   = draft_lens[b]
    slot_idx    = the first seq_lens[b] entries of row req_ids[b], for b in order.
A step whose inputs are out of range (a row id outside the table, a negative
length, a sequence longer than a table row, more slots than the output holds)
yields status != 0 and all-zero lengths, so that a verify call on it does
nothing; the status bits are 1 (row id), 2 (negative length), 4 (longer than a
row), 8 (total over capacity).
"""
from __future__ import annotations

import numpy as np

ERR_ROW = 1
ERR_NEGATIVE = 2
ERR_TOO_LONG = 4
ERR_CAPACITY = 8


def build_step_metadata(req_to_token: np.ndarray, req_ids, prefix_lens, draft_lens, slot_capacity: int):
    """Returns (slot_idx int32 [total], seq_lens int32 [B], q_lens int32 [B], status int).

    On status != 0, seq_lens and q_lens are all zero and slot_idx is empty.
    """
    rows, width = req_to_token.shape
    batch = len(req_ids)
    status = 0
    seq = []
    for b in range(batch):
        r, p, d = int(req_ids[b]), int(prefix_lens[b]), int(draft_lens[b])
        if r < 0 or r >= rows:
            status |= ERR_ROW
        if p < 0 or d < 0:
            status |= ERR_NEGATIVE
        if p + d > width:
            status |= ERR_TOO_LONG
        seq.append(p + d)
    if status == 0 and sum(seq) > slot_capacity:
        status |= ERR_CAPACITY
    if status != 0:
        zeros = np.zeros(batch, dtype=np.int32)
        return np.zeros(0, dtype=np.int32), zeros, zeros.copy(), status
    slot_idx = []
    for b in range(batch):
        row = int(req_ids[b])
        for j in range(seq[b]):
            slot_idx.append(int(req_to_token[row, j]))
    return (np.array(slot_idx, dtype=np.int32), np.array(seq, dtype=np.int32),
            np.array([int(d) for d in draft_lens], dtype=np.int32), 0)
