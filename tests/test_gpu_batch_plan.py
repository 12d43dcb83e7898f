"""GPU parity for batches of 2..64 requests, which kernel 1 spreads over the CUs by the range plan:
the tiles of all requests in one sequence, cut into equal chunks, one piece of work per request a
chunk touches.  Every case is checked element by element against the fp64 oracle (max |out err|
<= 1e-2, max |lse err| <= 1e-3); the cases reach the plan's corners: chunks that end inside a
request, requests without rows, row groups a request does not fill, a split count too small for
an even share (the chunk length is raised), one split per request (one chunk for the whole batch),
and the largest batch the plan takes.  All calls go through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_mla_amd import inputs as I
from tests.gpu_helpers import LSE_TOL, OUT_TOL, DeviceInputs, max_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decode_mla_amd import api as A
    return A


def _handle(api, x, nsplit, max_q=None, form=0):
    return api.MlaVerify(x.heads, len(x.seq_lens), max_q or int(max(1, x.q_lens.max())), nsplit, x.num_slots, x.scale,
                         form=form)


def _oracle(x):
    return oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)


def _lens(rng, n, lo, hi):
    return [int(v) for v in rng.integers(lo, hi, n)]


CASES = [
    # (label, seed, seq_lens, q_lens, heads, nsplit)
    ("two requests, chunk ends inside the first", 50, [3000, 40], [16, 16], 16, 32),
    ("short and long, few splits", 51, [5000, 33, 700, 1], [4, 4, 4, 1], 32, 3),
    ("a request without rows", 52, [900, 400, 1200], [8, 0, 8], 16, 8),
    ("ragged row groups", 53, [600, 500, 800], [16, 2, 9], 64, 16),
    ("one split per request", 54, [1500, 300, 2200, 64], [8, 3, 8, 8], 16, 1),
    ("two splits: chunk length raised", 55, [4000, 3000, 100, 50, 2500, 10, 900], [4] * 7, 32, 2),
    ("draft block spans a chunk edge", 56, [1030, 1030], [16, 16], 8, 64),
]


@pytest.mark.parametrize("label,seed,lens,qlens,heads,nsplit", CASES, ids=[c[0] for c in CASES])
def test_batch_cases(api, label, seed, lens, qlens, heads, nsplit):
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, int(sum(lens)) * 2 + 64)
    print(f"{label}: B={len(lens)} H={heads} nsplit={nsplit}", flush=True)
    d = DeviceInputs(x)
    out, lse = d.run(_handle(api, x, nsplit), nsplit)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle(x)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    print(f"  max|out err|={eo:.3e} max|lse err|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL


def test_largest_batch(api):
    """64 requests (the most the plan holds), lengths from 1 to 3,000, 0..4 draft tokens each,
    32 heads: one row group, so 256 workers (32 per XCD)."""
    rng = np.random.default_rng(57)
    lens = _lens(rng, 64, 1, 3000)
    qlens = [int(min(l, q)) for l, q in zip(lens, rng.integers(0, 5, 64))]
    x = I.make_custom(rng, lens, qlens, 32, int(sum(lens)) + 1000)
    d = DeviceInputs(x)
    out, lse = d.run(_handle(api, x, 16, max_q=4), 16)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle(x)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    print(f"B=64: max|out err|={eo:.3e} max|lse err|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL


def test_past_the_plan_per_split(api):
    """65 requests take the per-request splits instead; there a request's result does not depend
    on the rest of the batch, so it equals the request run alone bit for bit (both calls pinned to
    the 128-row form: alone, the request's few workgroups would otherwise take the two-stream form)."""
    rng = np.random.default_rng(58)
    lens = _lens(rng, 65, 20, 1500)
    qlens = [int(min(l, 3)) for l in lens]
    x = I.make_custom(rng, lens, qlens, 32, int(sum(lens)) + 500)
    d = DeviceInputs(x)
    out, lse = d.run(_handle(api, x, 8, max_q=3, form=1), 8)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle(x)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    assert eo <= OUT_TOL and el <= LSE_TOL
    b = 40
    k0, q0 = int(sum(lens[:b])), int(sum(qlens[:b]))
    y = I.VerifyInputs(q=x.q[q0:q0 + qlens[b]], kv_rows=x.kv_rows[k0:k0 + lens[b]],
                       slot_idx=x.slot_idx[k0:k0 + lens[b]], seq_lens=x.seq_lens[b:b + 1],
                       q_lens=x.q_lens[b:b + 1], num_slots=x.num_slots, heads=32)
    e = DeviceInputs(y)
    o1, l1 = e.run(_handle(api, y, 8, max_q=3, form=1), 8)
    torch.cuda.synchronize()
    assert torch.equal(out[q0:q0 + qlens[b]], o1) and torch.equal(lse[q0:q0 + qlens[b]], l1)


def test_one_handle_two_batches(api):
    """A long batch, then a short one with fewer pieces, on one handle: the merge reads only the
    partials the second call wrote."""
    x = I.make_custom(np.random.default_rng(59), [6000, 2500, 4000], [16, 16, 16], 16, 30000)
    y = I.make_custom(np.random.default_rng(60), [300, 90, 1000], [16, 5, 16], 16, 30000)
    h = _handle(api, x, 32)
    DeviceInputs(x).run(h, 32)
    dy = DeviceInputs(y)
    out, lse = dy.run(h, 32)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle(y)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    assert eo <= OUT_TOL and el <= LSE_TOL


@pytest.mark.parametrize("lens,qlens", [([40, 0, 300], [0, 0, 0]), ([0, 0], [0, 0])],
                         ids=["no draft tokens", "no keys"])
def test_empty_batch_writes_nothing(api, lens, qlens):
    """A batch with no rows: the plan has no tiles, no workgroup does any work, nothing is written.
    Called through the C ABI with small non-empty buffers (the binding refuses empty tensors)."""
    import ctypes

    from speculative_decode_mla_amd import _lib
    dev = "cuda"
    H = 64
    q = torch.zeros((4, H, I.D_QK), dtype=torch.bfloat16, device=dev)
    pool = torch.zeros((512, I.D_QK), dtype=torch.bfloat16, device=dev)
    slot_idx = torch.zeros(max(1, sum(lens)), dtype=torch.int32, device=dev)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    q_lens = torch.tensor(qlens, dtype=torch.int32, device=dev)
    out = torch.full((4, H, I.D_V), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((4, H), 7.0, dtype=torch.float32, device=dev)
    h = api.MlaVerify(H, len(lens), 16, 8, 512, I.SM_SCALE)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = _lib.load().mla_verify_run(h._h, P(q), P(pool), P(slot_idx), P(seq_lens), P(q_lens), P(out), P(lse), 8,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == _lib.MLA_OK
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
