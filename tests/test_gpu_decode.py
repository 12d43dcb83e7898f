"""GPU parity for q_len = 1 decode steps (and other requests of at most 64 rows), which run the
two-stream form of kernel 1 (or, at few splits, the four-stream form), and the same cases in the
four-stream form: against the fp64 oracle, max |out err| <= 1e-2, max |lse err| <= 1e-3.
All calls go through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
from speculative_decode_mla_amd import inputs as I
from tests.gpu_helpers import LSE_TOL, OUT_TOL, DeviceInputs, bf16_to_f64, max_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decode_mla_amd import api as A
    return A


def _run_check(api, x, nsplit, label, max_q=None, form=0):
    d = DeviceInputs(x)
    h = api.MlaVerify(x.heads, len(x.seq_lens), max_q or int(max(1, x.q_lens.max())), nsplit, x.num_slots, x.scale,
                      form=form)
    out, lse = d.run(h, nsplit)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    print(f"{label} form={form} nsplit={nsplit}: max|out err|={eo:.3e} max|lse err|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL
    return out, lse


CASES = [
    # (seed, seq_lens, q_lens, heads, nsplit)
    (50, [1000], [1], 64, 4),
    (51, [33], [1], 64, 1),            # two tiles: each stream one
    (52, [31], [1], 64, 1),            # one tile: the second stream has none (empty partial)
    (53, [290], [1], 64, 2),           # ten tiles
    (54, [257, 1, 4000, 64], [1, 1, 1, 1], 64, 8),  # ragged batch, a one-key request
    (55, [700, 1500], [2, 1], 32, 4),  # 64 rows from two draft tokens x 32 heads
    (56, [999], [1], 48, 3),           # 48 rows: a part-filled group
    (57, [8 * 32 * 3 + 5], [1], 64, 3),  # 25 tiles over three splits: odd tile counts per split
]


# 0: the library's choice (the four-stream form for most of these few-split cases, the two-stream form
# past it); 2: the two-stream form; 3: the four-stream form (in which the cases above hold one, two,
# three or four streams with keys, and one-key requests)
DECODE_FORMS = [0, 2, 3]


@pytest.mark.parametrize("form", DECODE_FORMS)
@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit", CASES)
def test_decode_cases(api, seed, lens, qlens, heads, nsplit, form):
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, int(sum(lens)) * 2 + 64)
    _run_check(api, x, nsplit, f"decode case {seed}", form=form)


@pytest.mark.parametrize("form", DECODE_FORMS)
def test_decode_split_count_does_not_change_result(api, form):
    x = I.make_custom(np.random.default_rng(58), [5000], [1], 64, 12000)
    outs = []
    for ns in (1, 3, 16, 64):
        out, _ = _run_check(api, x, ns, "decode split-count", max_q=1, form=form)
        outs.append(bf16_to_f64(out))
    assert max(np.max(np.abs(o - outs[0])) for o in outs) <= OUT_TOL


@pytest.mark.parametrize("factor,lo,hi", [
    (2.5, 80, 64 + 96 - 12),    # ~100 nats above the rest: within the reference's 64-binade headroom
    (3.0, 64 + 96 + 4, 64 + 128 - 12),  # the row sum passes 2^96: exact redo
    (3.6, 64 + 128 + 4, 1e9),   # 2^(x - m_ref) overflows fp32: exact redo
])
def test_decode_overflow_fallback_rows(api, factor, lo, hi):
    """A key far above its row's other scores, in the second stream's tiles: within the headroom it
    is just a dominant key; past it the row goes through the exact redo over the whole split (the two
    streams are merged before the write)."""
    x = I.make_custom(np.random.default_rng(59), [3000], [1], 64, 6000)
    # key 2920 sits in tile 91: local tile 91 of the one split (nsplit 1) and 29 of the third split
    # (nsplit 3 -> splits start at tiles 0, 31, 62), odd in both, so the second stream takes it (in the
    # four-stream form it is in half tile 182 of the one split and 58 of the third: the third stream).
    # It is head 7's query with the span of the other 63 heads' queries projected out, times
    # `factor`: far above the rest for head 7, ~0 for every other head, and its v (dims 0..511)
    # stays ~factor * N(0,1), so head 7 is the only row it moves.
    qh = oracle.bf16_bits_to_f64(x.q[0])
    others = np.delete(qh, 7, axis=0)
    coef, *_ = np.linalg.lstsq(others.T, qh[7], rcond=None)
    perp = qh[7] - others.T @ coef
    x.kv_rows[2920] = I.f32_to_bf16_bits((factor * perp).astype(np.float32))
    qv = qh[7]
    sc = x.scale * (oracle.bf16_bits_to_f64(x.kv_rows[:3000]) @ qv) / math.log(2.0)
    margin = float(sc[2920] - np.max(np.delete(sc, 2920)))
    assert lo < margin < hi, margin
    for form in DECODE_FORMS:
        _run_check(api, x, 3, f"decode planted x{factor}", form=form)
        _run_check(api, x, 1, f"decode planted x{factor}", form=form)


@pytest.mark.parametrize("workload", ["decode64k", "decode_batch16"])
def test_decode_full_size_parity(api, workload):
    """The decode workloads at their full sizes and split counts: whole out and lse against the oracle."""
    w = I.WORKLOADS[workload]
    x = I.make_inputs(workload)
    print(f"{workload}: B={w.batch} sum(L)={int(x.seq_lens.sum())} nsplit={w.nsplit}", flush=True)
    d = DeviceInputs(x)
    h = api.MlaVerify(x.heads, w.batch, 1, w.nsplit, x.num_slots, x.scale)
    out, lse = d.run(h, w.nsplit)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attention(x.q, x.sparse_pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ro, rl)
    print(f"{workload} nsplit={w.nsplit}: max|out err|={eo:.3e} max|lse err|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL
    del d, h
    torch.cuda.empty_cache()
