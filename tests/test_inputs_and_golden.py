"""Generator determinism and the frozen oracle answer on the tiny workload."""
import json
import os

import numpy as np

import oracle
from speculative_decode_mla_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))


def test_seed5_ragged_lengths():
    rng = np.random.default_rng(5)
    lens = I.ragged_lengths(rng, 16, 1024, 65536)
    assert lens.tolist() == [29126, 29484, 8731, 3361, 1281, 5044, 5599, 1236, 1254, 65312, 15438, 2716,
                             6250, 58865, 42822, 34287]
    assert int(lens.sum()) == 310806


def test_generator_is_deterministic_and_distinct_slots():
    a = I.make_custom(np.random.default_rng(3), [100, 50], [4, 2], 2, 1000)
    b = I.make_custom(np.random.default_rng(3), [100, 50], [4, 2], 2, 1000)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.kv_rows, b.kv_rows)
    assert np.array_equal(a.slot_idx, b.slot_idx)
    assert len(np.unique(a.slot_idx)) == 150
    pool = a.pool()
    assert np.all(pool[np.setdiff1d(np.arange(1000), a.slot_idx)] == I.BF16_QNAN)


def test_tiny_golden_unchanged():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        g = json.load(f)
    x = I.make_inputs("tiny")
    out, lse = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    assert np.max(np.abs(lse - np.array(g["lse"]))) < 1e-12
    assert np.max(np.abs(out.sum(axis=2) - np.array(g["out_row_sums"]))) < 1e-10
    for key, vals in g["out_samples"].items():
        t, h = map(int, key.split(","))
        assert np.max(np.abs(out[t, h, :16] - np.array(vals))) < 1e-12
