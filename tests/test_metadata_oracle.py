"""Pins for the step-metadata oracle: closed forms on a patterned table, the status bits, and
the end-to-end property that verify attention over the built metadata equals attention over
metadata written out by hand.  CPU only."""
import numpy as np
import pytest

import oracle
from oracle import metadata_oracle as mo
from speculative_decode_mla_amd import inputs as I


def _table(rows=12, width=300):
    r = np.arange(rows, dtype=np.int64)[:, None]
    j = np.arange(width, dtype=np.int64)[None, :]
    return (r * 100_000 + j).astype(np.int32)  # entry (r, j) names its own row and position


def test_closed_form_on_a_patterned_table():
    t = _table()
    ids, pre, dr = [7, 2, 11, 0], [10, 0, 250, 33], [3, 5, 0, 16]
    slots, seq, ql, st = mo.build_step_metadata(t, ids, pre, dr, 10_000)
    assert st == 0
    assert seq.tolist() == [13, 5, 250, 49] and ql.tolist() == dr
    want = [r * 100_000 + j for r, p, d in zip(ids, pre, dr) for j in range(p + d)]
    assert slots.tolist() == want


def test_zero_length_requests_and_empty_batch():
    t = _table()
    slots, seq, ql, st = mo.build_step_metadata(t, [3, 4, 5], [0, 6, 0], [0, 2, 0], 100)
    assert st == 0 and seq.tolist() == [0, 8, 0] and slots.tolist() == [400_000 + j for j in range(8)]
    slots, seq, ql, st = mo.build_step_metadata(t, [], [], [], 100)
    assert st == 0 and len(slots) == len(seq) == 0


@pytest.mark.parametrize("ids,pre,dr,cap,bits", [
    ([12], [0], [1], 100, mo.ERR_ROW),
    ([-1], [0], [1], 100, mo.ERR_ROW),
    ([1], [-1], [1], 100, mo.ERR_NEGATIVE),
    ([1], [299], [2], 1000, mo.ERR_TOO_LONG),
    ([1, 2], [100, 100], [1, 1], 201, mo.ERR_CAPACITY),
    ([12, 1], [-5, 299], [0, 2], 1000, mo.ERR_ROW | mo.ERR_NEGATIVE | mo.ERR_TOO_LONG),
])
def test_status_bits_and_zeroed_lengths(ids, pre, dr, cap, bits):
    slots, seq, ql, st = mo.build_step_metadata(_table(), ids, pre, dr, cap)
    assert st == bits
    assert len(slots) == 0 and not seq.any() and not ql.any()


def test_capacity_is_inclusive():
    _, seq, _, st = mo.build_step_metadata(_table(), [1, 2], [100, 100], [1, 0], 201)
    assert st == 0 and seq.sum() == 201


def test_verify_over_built_metadata_equals_handwritten():
    """Place two requests' rows at table positions, build the metadata, run the verify oracle."""
    rng = np.random.default_rng(3)
    x = I.make_custom(rng, [40, 25], [3, 5], 2, 300)
    table = np.full((4, 64), -1, dtype=np.int32)
    table[2, :40] = x.slot_idx[:40]
    table[0, :25] = x.slot_idx[40:]
    slots, seq, ql, st = mo.build_step_metadata(table, [2, 0], [37, 20], [3, 5], 1000)
    assert st == 0
    pool = x.pool()
    a = oracle.verify_attention(x.q, pool, x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    b = oracle.verify_attention(x.q, pool, slots, seq, ql, x.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _mut_drafts_not_counted(req_to_token, req_ids, prefix_lens, draft_lens, cap):
    return _orig(req_to_token, req_ids, prefix_lens, [0] * len(draft_lens), cap)[0:1] + \
        _orig(req_to_token, req_ids, prefix_lens, draft_lens, cap)[1:]


def _mut_row_by_batch_index(req_to_token, req_ids, prefix_lens, draft_lens, cap):
    return _orig(req_to_token, list(range(len(req_ids))), prefix_lens, draft_lens, cap)


def _mut_no_capacity_check(req_to_token, req_ids, prefix_lens, draft_lens, cap):
    return _orig(req_to_token, req_ids, prefix_lens, draft_lens, 1 << 40)


_orig = mo.build_step_metadata


@pytest.mark.parametrize("mutant,pin", [
    (_mut_drafts_not_counted, lambda: test_closed_form_on_a_patterned_table()),
    (_mut_row_by_batch_index, lambda: test_closed_form_on_a_patterned_table()),
    (_mut_no_capacity_check, lambda: test_status_bits_and_zeroed_lengths([1, 2], [100, 100], [1, 1], 201,
                                                                          mo.ERR_CAPACITY)),
])
def test_planted_mistakes_are_caught(monkeypatch, mutant, pin):
    monkeypatch.setattr(mo, "build_step_metadata", mutant)
    with pytest.raises(AssertionError):
        pin()
