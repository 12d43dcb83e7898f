"""Pins for the KV-compaction oracle: closed forms for every copied byte, the untouched rows,
the new slot indices, and the invariance of verify attention under the move.  CPU only."""
import numpy as np
import pytest

import oracle
from oracle import kv_compact_oracle as kc
from speculative_decode_mla_amd import inputs as I

ROW = I.D_QK


def _patterned_pool(n_slots):
    """Row s, column c holds (7*s + c) mod 2^16: every byte's source is recoverable by formula."""
    s = np.arange(n_slots, dtype=np.int64)[:, None]
    c = np.arange(ROW, dtype=np.int64)[None, :]
    return ((7 * s + c) & 0xFFFF).astype(np.uint16)


def _case(seed, n, n_slots=4096, dst_slots=3000, dst_first=100):
    rng = np.random.default_rng(seed)
    slots = rng.permutation(n_slots)[:n].astype(np.int32)
    src = _patterned_pool(n_slots)
    dst = np.full((dst_slots, ROW), 0xBEEF, dtype=np.uint16)
    return src, slots, dst, dst_first


@pytest.mark.parametrize("seed,n", [(0, 1), (1, 37), (2, 1000)])
def test_every_copied_row_matches_its_formula(seed, n):
    src, slots, dst, first = _case(seed, n)
    out, new = kc.compact_rows(src, slots, dst, first)
    c = np.arange(ROW, dtype=np.int64)
    for j in range(n):
        want = ((7 * int(slots[j]) + c) & 0xFFFF).astype(np.uint16)
        assert np.array_equal(out[first + j], want), j
    assert np.array_equal(new, np.arange(first, first + n, dtype=np.int32))


def test_rows_outside_the_range_are_untouched():
    src, slots, dst, first = _case(3, 50)
    out, _ = kc.compact_rows(src, slots, dst, first)
    assert np.all(out[:first] == 0xBEEF)
    assert np.all(out[first + 50:] == 0xBEEF)


def test_empty_and_bad_ranges():
    src, slots, dst, first = _case(4, 0)
    out, new = kc.compact_rows(src, slots, dst.copy(), first)
    assert np.array_equal(out, dst) and len(new) == 0
    src, slots, dst, _ = _case(5, 10, dst_slots=20)
    with pytest.raises(ValueError):
        kc.compact_rows(src, slots, dst, 11)
    with pytest.raises(ValueError):
        kc.compact_rows(src, slots, dst, -1)


def test_verify_attention_unchanged_by_the_move():
    """The defining property: attention over the compacted rows equals attention over the originals."""
    rng = np.random.default_rng(11)
    x = I.make_custom(rng, [70, 9], [4, 2], 3, 400)
    pool = x.pool()
    ref_o, ref_l = oracle.verify_attention(x.q, pool, x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    dst = np.full((200, ROW), I.BF16_QNAN, dtype=np.uint16)
    dst, new = kc.compact_rows(pool, x.slot_idx, dst, 5)
    o, l = oracle.verify_attention(x.q, dst, new, x.seq_lens, x.q_lens, x.scale)
    assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)


# planted mistakes in the oracle must trip a pin
def _mut_reversed(kv_pool, slot_idx, dst_pool, dst_first):
    n = len(slot_idx)
    for j in range(n):
        dst_pool[dst_first + j] = kv_pool[int(slot_idx[n - 1 - j])]
    return dst_pool, np.arange(dst_first, dst_first + n, dtype=np.int32)


def _mut_off_by_one(kv_pool, slot_idx, dst_pool, dst_first):
    n = len(slot_idx)
    for j in range(n):
        dst_pool[dst_first + j + 1 if j + 1 < n else dst_first + j] = kv_pool[int(slot_idx[j])]
    return dst_pool, np.arange(dst_first, dst_first + n, dtype=np.int32)


def _mut_index_as_slot(kv_pool, slot_idx, dst_pool, dst_first):
    n = len(slot_idx)
    for j in range(n):
        dst_pool[dst_first + j] = kv_pool[j]
    return dst_pool, np.arange(dst_first, dst_first + n, dtype=np.int32)


@pytest.mark.parametrize("mutant", [_mut_reversed, _mut_off_by_one, _mut_index_as_slot])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(kc, "compact_rows", mutant)
    with pytest.raises(AssertionError):
        test_every_copied_row_matches_its_formula(1, 37)
