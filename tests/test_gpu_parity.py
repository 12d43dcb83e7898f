"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Bar (from the tolerance on bf16 outputs and fp32 log-sum-exp): max |out err| <= 1e-2,
max |lse err| <= 1e-3, element by element.  All calls go through the C ABI.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from speculative_decode_mla_amd import inputs as I
from tests.gpu_helpers import LSE_TOL, OUT_TOL, DeviceInputs, bf16_to_f64, max_errors, poison_workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decode_mla_amd import api as A
    return A


# Kernel-1 layouts: 1 = 128-row workgroups (range plan for batches of 2..64), 2 = two-stream 64-row
# workgroups, 3 = four-stream 32-row workgroups.  Tests that pin one run it under each.
FORMS = [1, 2, 3]


def _handle(api, x, nsplit, max_q=None, form=0):
    return api.MlaVerify(x.heads, len(x.seq_lens), max_q or int(max(1, x.q_lens.max())), nsplit, x.num_slots, x.scale,
                         form=form)


def _check(api, x, nsplit, label="", form=0):
    d = DeviceInputs(x)
    h = _handle(api, x, nsplit, form=form)
    out, lse = d.run(h, nsplit)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    print(f"{label} form={form} nsplit={nsplit}: max|out err|={eo:.3e} max|lse err|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL
    return d, h


def test_tiny_workload(api):
    _check(api, I.make_inputs("tiny"), 1, "tiny")


CASES = [
    # (seed, seq_lens, q_lens, heads, nsplit)
    (20, [1000], [8], 64, 4),
    (21, [130, 64, 1, 700], [3, 1, 1, 16], 8, 3),
    (22, [65], [4], 2, 2),              # the second split holds only draft keys: fully masked rows
    (23, [1], [1], 64, 1),              # one key: out is that v row
    (24, [50, 20], [0, 5], 16, 2),      # a request with no draft tokens
    (25, [300], [7], 5, 2),             # 35 rows: a partly filled wave
    (26, [300], [16], 64, 2),           # 1024 rows: eight row groups
    (27, [4096 + 37], [16], 16, 8),     # ragged last tile
    (28, [64, 128, 192], [16, 16, 16], 4, 32),  # more splits than tiles
    (29, [900], [5], 40, 4),            # 200 rows: a ragged last row group in every form
    (41, [2000], [16], 128, 8),         # 128 heads: 2,048 rows, 16 (or 32) row groups
    (42, [900, 1300], [16, 8], 128, 4),  # 128 heads in the range plan: 16 workers of 16 row groups
    (46, [16], [16], 64, 2),            # every key is a draft key: draft t sees keys 0..t only
    (47, [40, 16, 3], [16, 16, 3], 16, 4),  # the same inside a batch, next to a longer request
]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit", CASES)
def test_small_cases(api, seed, lens, qlens, heads, nsplit, form):
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, int(sum(lens)) * 2 + 64)
    _check(api, x, nsplit, f"case{seed}", form)


# Short requests with few keys per row, where single keys can carry most of a row's weight and the
# output entries reach a few units: the bf16 output's own rounding is then up to 2^-8 of the value,
# and the split partials must not add a second rounding of the same size (they are fp16).  Shapes
# drawn once from a fixed generator (lengths 20..1500, 1..16 draft tokens, 8/16/64 heads, 1..32
# splits), plus the shape on which bf16 partials came to 1.06e-2.
def _random_short_cases():
    rng = np.random.default_rng(2024)
    cases = [(62, [500], [16], 64, 32)]
    for i in range(10):
        L = int(rng.integers(20, 1500))
        cases.append((300 + i, [L], [int(min(L, rng.integers(1, 17)))], int(rng.choice([8, 16, 64])),
                      int(rng.choice([1, 2, 4, 8, 16, 32]))))
    return cases


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit", _random_short_cases())
def test_short_requests_whole_tensor(api, seed, lens, qlens, heads, nsplit, form):
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, 2 * int(sum(lens)) + 64)
    _check(api, x, nsplit, f"short{seed} L={lens[0]} Q={qlens[0]} H={heads}", form)


# Random batches, drawn once from a fixed generator: 1..8 requests with lengths 1..2,500 (ragged
# last tiles, requests shorter than their draft block), 0..16 draft tokens each, 1..128 heads,
# 1..48 splits, and each kernel-1 form (0: the library's choice, including the range plan for
# batches of 2..64 requests).  Whole out and lse tensors against the oracle.
def _random_batch_cases():
    rng = np.random.default_rng(7777)
    cases = []
    for i in range(16):
        B = int(rng.integers(1, 9))
        lens = [int(v) for v in rng.integers(1, 2501, B)]
        qlens = [int(min(L, rng.integers(0, 17))) for L in lens]
        if max(qlens) == 0:
            qlens[0] = 1
        cases.append((500 + i, lens, qlens, int(rng.choice([1, 3, 16, 48, 64, 128])),
                      int(rng.choice([1, 2, 3, 5, 8, 16, 32, 48])), int(rng.choice([0, 1, 2]))))
    return cases


@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit,form", _random_batch_cases())
def test_random_batches_whole_tensor(api, seed, lens, qlens, heads, nsplit, form):
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, 2 * int(sum(lens)) + 64)
    _check(api, x, nsplit, f"batch{seed} B={len(lens)} H={heads}", form)


@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit", [c[:5] for c in _random_batch_cases()])
def test_random_batches_four_stream(api, seed, lens, qlens, heads, nsplit):
    """The same random batches in the four-stream form."""
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, 2 * int(sum(lens)) + 64)
    _check(api, x, nsplit, f"batch{seed} B={len(lens)} H={heads}", 3)


def test_ctx4k_workload(api):
    _check(api, I.make_inputs("ctx4k"), 8, "ctx4k")


def _check_full(api, x, nsplit, label):
    """Whole out and lse tensors against the oracle, element by element (the oracle reads the pool
    through a sparse view, so the unreferenced rows of a multi-GB pool are never materialised)."""
    print(f"{label}: B={len(x.seq_lens)} H={x.heads} sum(L)={int(x.seq_lens.sum())} nsplit={nsplit}", flush=True)
    d = DeviceInputs(x)
    h = _handle(api, x, nsplit)
    out, lse = d.run(h, nsplit)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.verify_attention(x.q, x.sparse_pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    print(f"{label}: {ref_o.shape[0] * ref_o.shape[1]} rows, max|out err|={eo:.3e} max|lse err|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL
    del d, h
    torch.cuda.empty_cache()


@pytest.mark.parametrize("workload", ["ctx23k", "ctx64k", "ctx91k", "batch16", "ctx64k_sink"])
def test_full_size_parity(api, workload):
    """The large workloads at their full sizes and split counts, as the benchmark runs them: every
    (token, head) row of out and lse against the oracle."""
    _check_full(api, I.make_inputs(workload), I.WORKLOADS[workload].nsplit, workload)


def test_long_context_parity(api):
    """262,144 keys (past the largest workload) at nsplit 64, whole tensors against the oracle."""
    _check_full(api, I.make_custom(np.random.default_rng(48), [1 << 18], [16], 64, 1 << 19), 64, "ctx256k")


@pytest.mark.parametrize("form", FORMS)
def test_pool_edge_slots(api, form):
    """Slot indices at the first and the last row of the pool (the gather's address range ends)."""
    x = I.make_custom(np.random.default_rng(49), [700, 300], [8, 8], 16, 2000)
    s = x.slot_idx.copy()
    for want, pos in ((0, 5), (x.num_slots - 1, len(s) - 1)):  # swap so the slots stay distinct
        j = np.nonzero(s == want)[0]
        if len(j):
            s[j[0]] = s[pos]
        s[pos] = want
    y = I.VerifyInputs(q=x.q, kv_rows=x.kv_rows, slot_idx=s, seq_lens=x.seq_lens, q_lens=x.q_lens,
                       num_slots=x.num_slots, heads=x.heads)
    _check(api, y, 4, "pool-edge", form)


@pytest.mark.parametrize("form", FORMS)
def test_single_key_is_exact(api, form):
    x = I.make_custom(np.random.default_rng(30), [1], [1], 64, 100)
    d = DeviceInputs(x)
    out, lse = d.run(_handle(api, x, 1, form=form), 1)
    torch.cuda.synchronize()
    v = torch.from_numpy(x.kv_rows[0, :512].view(np.int16).copy()).view(torch.bfloat16)
    assert torch.equal(out.cpu()[0], v.expand(64, 512))


@pytest.mark.parametrize("form", FORMS)
def test_split_count_does_not_change_result(api, form):
    x = I.make_custom(np.random.default_rng(31), [3000, 900], [16, 9], 32, 10000)
    d = DeviceInputs(x)
    h = _handle(api, x, 32, form=form)
    ref_o, ref_l = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    outs = []
    for ns in (1, 2, 5, 32, 7):
        out, lse = d.run(h, ns)
        torch.cuda.synchronize()
        eo, el = max_errors(out, lse, ref_o, ref_l)
        assert eo <= OUT_TOL and el <= LSE_TOL, (ns, eo, el)
        outs.append(bf16_to_f64(out))
    assert max(np.max(np.abs(o - outs[0])) for o in outs) <= OUT_TOL


def test_slot_permutation_is_bitwise(api):
    x = I.make_custom(np.random.default_rng(32), [777, 300], [8, 8], 16, 5000)
    d1 = DeviceInputs(x)
    h = _handle(api, x, 4)
    o1, l1 = (t.clone() for t in d1.run(h, 4))
    perm = np.random.default_rng(33).permutation(x.num_slots)
    y = I.VerifyInputs(q=x.q, kv_rows=x.kv_rows, slot_idx=perm[x.slot_idx].astype(np.int32),
                       seq_lens=x.seq_lens, q_lens=x.q_lens, num_slots=x.num_slots, heads=x.heads)
    d2 = DeviceInputs(y)
    o2, l2 = d2.run(h, 4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit,member", [
    (34, [500, 1200, 90], [4, 16, 2], 8, 6, 1),          # range plan without the flag
    (67, [3000, 20000, 700, 65], [16, 16, 16, 9], 64, 32, 1),  # 128-row form per request
    (68, [9000, 400], [16, 16], 64, 8, 0),               # two-stream form chosen as for one request
    (69, [2000, 3000], [1, 1], 64, 16, 1),               # decode rows
])
def test_batch_invariant_request_is_bitwise_alone(api, seed, lens, qlens, heads, nsplit, member):
    """With MLA_VERIFY_FLAG_BATCH_INVARIANT a request's out and lse are bit for bit the same alone
    (a one-request handle) and inside a batch (the batch-composition pin, bitwise)."""
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, int(sum(lens)) * 2 + 64)
    max_q = int(max(qlens))
    d = DeviceInputs(x)
    h = api.MlaVerify(heads, len(lens), max_q, nsplit, x.num_slots, x.scale, batch_invariant=True)
    out, lse = d.run(h, nsplit)
    torch.cuda.synchronize()
    ko = int(sum(lens[:member]))
    qo = int(sum(qlens[:member]))
    L, Q = lens[member], qlens[member]
    y = I.VerifyInputs(q=x.q[qo:qo + Q], kv_rows=x.kv_rows[ko:ko + L], slot_idx=x.slot_idx[ko:ko + L],
                       seq_lens=x.seq_lens[member:member + 1], q_lens=x.q_lens[member:member + 1],
                       num_slots=x.num_slots, heads=heads)
    e = DeviceInputs(y)
    o1, l1 = e.run(api.MlaVerify(heads, 1, max_q, nsplit, x.num_slots, x.scale, batch_invariant=True), nsplit)
    torch.cuda.synchronize()
    assert torch.equal(out[qo:qo + Q].view(torch.int16), o1.view(torch.int16))
    assert torch.equal(lse[qo:qo + Q], l1)
    ref_o, ref_l = oracle.verify_attention(y.q, y.pool(), y.slot_idx, y.seq_lens, y.q_lens, y.scale)
    eo, el = max_errors(o1, l1, ref_o, ref_l)
    assert eo <= OUT_TOL and el <= LSE_TOL


def test_request_alone_equals_request_in_batch(api):
    x = I.make_custom(np.random.default_rng(34), [500, 1200, 90], [4, 16, 2], 8, 4000)
    d = DeviceInputs(x)
    out, lse = d.run(_handle(api, x, 6, max_q=16), 6)
    torch.cuda.synchronize()
    # request 1 alone, same slots and values
    y = I.VerifyInputs(q=x.q[4:20], kv_rows=x.kv_rows[500:1700], slot_idx=x.slot_idx[500:1700],
                       seq_lens=x.seq_lens[1:2], q_lens=x.q_lens[1:2], num_slots=x.num_slots, heads=8)
    e = DeviceInputs(y)
    o1, l1 = e.run(_handle(api, y, 6, max_q=16), 6)
    torch.cuda.synchronize()
    # A batch of 2..64 requests is spread by the range plan, which cuts a request's keys where the
    # batch's chunks fall, so the two calls agree to rounding; each is held to the oracle.
    ref_o, ref_l = oracle.verify_attention(y.q, y.pool(), y.slot_idx, y.seq_lens, y.q_lens, y.scale)
    for o_, l_ in ((out[4:20], lse[4:20]), (o1, l1)):
        eo, el = max_errors(o_, l_, ref_o, ref_l)
        assert eo <= OUT_TOL and el <= LSE_TOL


def planted_margin_log2(x, t, h, key):
    """How far (in log2 units) the score of `key` for row (t, h) of request 0 lies above that row's
    highest score over every other visible key.  Kernel 1's reference for a row is the highest score
    of one tile of the split (at most that highest score) plus 64 binades, so a margin past 64 + 96
    sends the row's sum past 2^96 (the exact redo) and one past 64 + 128 overflows the key's
    2^(x - m_ref); below about 64 + 96 - 12 (N(0,1) scores: a tile's max lies within a few log2 units
    of the row's) the row stays within the headroom."""
    L, Q = int(x.seq_lens[0]), int(x.q_lens[0])
    n = L - Q + t + 1
    qv = oracle.bf16_bits_to_f64(x.q[t, h])
    k = oracle.bf16_bits_to_f64(x.kv_rows[:n])
    sc = x.scale * (k @ qv) / math.log(2.0)
    return float(sc[key] - np.max(np.delete(sc, key)))


def plant_key_for_row(x, t, h, key, factor):
    """Key `key` of request 0 becomes `factor` times row (t, h)'s query with the span of the request's
    other rows' queries projected out: it scores ~factor * 26 nats for that row and ~0 for every other
    row, so no other row's output is pulled toward its (large) V row, whose bf16 rounding alone would
    exceed the 1e-2 bar."""
    Q = int(x.q_lens[0])
    qh = oracle.bf16_bits_to_f64(x.q[:Q].reshape(Q * x.heads, -1))
    r = t * x.heads + h
    others = np.delete(qh, r, axis=0)
    coef, *_ = np.linalg.lstsq(others.T, qh[r], rcond=None)
    perp = qh[r] - others.T @ coef
    x.kv_rows[key] = I.f32_to_bf16_bits((factor * perp).astype(np.float32))


@pytest.mark.parametrize("form", FORMS)
def test_dominant_key_within_headroom(api, form):
    """A key ~100 log2 units above the rest of its row stays within the 64-binade headroom of the
    fixed reference: no redo, and the row still matches the oracle."""
    x = I.make_custom(np.random.default_rng(35), [2000], [4], 8, 4000)
    plant_key_for_row(x, 0, 3, 1500, 1.8)
    assert 80 < planted_margin_log2(x, 0, 3, 1500) < 64 + 96 - 12
    _check(api, x, 2, "headroom", form)
    _check(api, x, 1, "headroom", form)


@pytest.mark.parametrize("form", FORMS)
def test_overflow_fallback_rows(api, form):
    """A key ~173 log2 units (~120 nats) above the rest of its row: its p passes 2^96 relative to the
    reference, so the row goes through the exact redo."""
    x = I.make_custom(np.random.default_rng(35), [2000], [4], 8, 4000)
    plant_key_for_row(x, 0, 3, 1500, 3.15)
    m = planted_margin_log2(x, 0, 3, 1500)
    assert 64 + 96 + 4 < m < 64 + 128 - 12, m
    _check(api, x, 2, "overflow", form)
    _check(api, x, 1, "overflow", form)


@pytest.mark.parametrize("form", FORMS)
def test_overflow_to_inf_fallback_rows(api, form):
    """A key so far above the rest of its row that 2^(x - m_ref) overflows fp32: without the exact
    redo the row would come out inf/NaN."""
    x = I.make_custom(np.random.default_rng(39), [3000], [4], 8, 6000)
    plant_key_for_row(x, 2, 5, 2900, 4.3)
    assert planted_margin_log2(x, 2, 5, 2900) > 64 + 128 + 4
    _check(api, x, 3, "overflow-inf", form)
    _check(api, x, 1, "overflow-inf", form)


# with 60 rows: 6 splits take the 4-group merge, 80 and 300 the column-sliced one (300: more
# splits than threads), 1100 (more than the sliced form holds in LDS) the 16-group one
@pytest.mark.parametrize("S", [6, 80, 300, 1100])
def test_merge_kernel_alone(api, S):
    x = I.make_custom(np.random.default_rng(36), [400, 37], [5, 3], 6, 1000)
    ref_o, ref_l, o_part, l_part = oracle.verify_attention_split(
        x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale, S, return_partials=True)
    B, H, maxq = 2, 6, 5
    rows = maxq * H
    op = np.zeros((B, S, rows, 512), np.float32)
    lp = np.full((B, S, rows), -np.inf, np.float32)
    tok = 0
    for b, Q in enumerate(x.q_lens.tolist()):
        for t in range(Q):
            for h in range(H):
                op[b, :, t * H + h] = o_part[tok + t, h]
                lp[b, :, t * H + h] = l_part[tok + t, h]
        tok += Q
    dev = "cuda"
    out = torch.empty((8, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((8, H), dtype=torch.float32, device=dev)
    api.merge(torch.from_numpy(op).to(dev), torch.from_numpy(lp).to(dev), torch.from_numpy(x.q_lens).to(dev), out, lse)
    torch.cuda.synchronize()
    eo, el = max_errors(out, lse, ref_o, ref_l)
    assert eo <= OUT_TOL and el <= LSE_TOL


@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit,form", [
    (60, [9000], [16], 64, 32, 0),               # one request, 32 x 8 row groups: 128-row form
    (61, [5000], [16], 64, 16, 0),               # one request, 16 x 8 row groups: two-stream form (automatic)
    (62, [3000, 1000, 37], [16, 16, 5], 16, 8, 0),  # three requests: the range plan
    (63, [4000, 700], [1, 1], 64, 32, 0),        # a decode step: 64 rows per request, two-stream form
    (64, [2500, 90, 1], [9, 3, 1], 24, 6, 1),    # ragged, forced 128-row form
    (65, [2500, 90, 1], [9, 3, 1], 24, 6, 2),    # ragged, forced two-stream form
    (66, [3000], [4], 8, 64, 0),                 # more splits asked for than the request fills
    (67, [4096], [8], 64, 8, 0),                 # one request, 8 x 16 row groups: four-stream form (automatic)
    (68, [4000], [1], 64, 16, 0),                # a decode step at few splits: four-stream form (automatic)
    (69, [2500, 90, 1], [9, 3, 1], 24, 6, 3),    # ragged, forced four-stream form (streams without keys)
], ids=["128-row", "two-stream", "range plan", "decode", "ragged 128-row", "ragged two-stream", "unused splits",
        "four-stream", "decode four-stream", "ragged four-stream"])
def test_nan_workspace_is_not_read(api, seed, lens, qlens, heads, nsplit, form):
    """The split workspace filled with NaN before the call: every partial the merge reads must have
    been written by the same call, so out and lse come out finite and match the oracle."""
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, int(sum(lens)) * 2 + 64)
    d = DeviceInputs(x)
    h = _handle(api, x, nsplit, form=form)
    poison_workspace(h)
    out, lse = d.run(h, nsplit)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())
    ref_o, ref_l = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    print(f"NaN workspace case {seed}: max|out err|={eo:.3e} max|lse err|={el:.3e}", flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL


def test_stale_workspace_is_not_read(api):
    """A call with more splits, then one with fewer and shorter requests, on one handle."""
    x = I.make_custom(np.random.default_rng(37), [5000], [16], 16, 12000)
    y = I.make_custom(np.random.default_rng(38), [700], [16], 16, 12000)
    h = _handle(api, x, 32)
    DeviceInputs(x).run(h, 32)
    dy = DeviceInputs(y)
    out, lse = dy.run(h, 3)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.verify_attention(y.q, y.pool(), y.slot_idx, y.seq_lens, y.q_lens, y.scale)
    eo, el = max_errors(out, lse, ref_o, ref_l)
    assert eo <= OUT_TOL and el <= LSE_TOL


@pytest.mark.parametrize("seed,lens,qlens,heads,nsplit", [
    (39, [3000, 1000], [16, 16], 16, 8),   # two requests: the range plan
    (43, [5000], [16], 64, 16),            # one request, 16 x 8 row groups: the two-stream form (automatic)
    (44, [9000], [16], 64, 32),            # one request, 32 x 8 row groups: the 128-row form
    (45, [4000, 700], [1, 1], 64, 32),     # a decode step: 64 rows per request, the two-stream form
    (46, [4096], [8], 64, 8),              # one request, 8 x 16 row groups: the four-stream form (automatic)
], ids=["range plan", "two-stream", "128-row", "decode", "four-stream"])
def test_graph_replay_matches_eager(api, seed, lens, qlens, heads, nsplit):
    x = I.make_custom(np.random.default_rng(seed), lens, qlens, heads, int(sum(lens)) * 2 + 64)
    d = DeviceInputs(x)
    h = _handle(api, x, nsplit)
    out_e, lse_e = (t.clone() for t in d.run(h, nsplit))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.run(h, nsplit)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.run(h, nsplit)
    for i in range(4):
        d.out.fill_(0)
        d.lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, out_e) and torch.equal(d.lse, lse_e), f"replay {i}"
        # eager work between replays
        d.run(h, nsplit)
        torch.cuda.synchronize()


def test_run_to_run_bitwise(api):
    x = I.make_inputs("ctx4k")
    d = DeviceInputs(x)
    h = _handle(api, x, 8)
    o1, l1 = (t.clone() for t in d.run(h, 8))
    o2, l2 = d.run(h, 8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_error_codes(api):
    from speculative_decode_mla_amd import _lib
    x = I.make_custom(np.random.default_rng(40), [100], [4], 4, 200)
    d = DeviceInputs(x)
    h = _handle(api, x, 4)
    with pytest.raises(_lib.MlaVerifyError) as e:
        d.run(h, 5)
    assert e.value.status == _lib.MLA_ERR_INVALID_ARGUMENT
    with pytest.raises(_lib.MlaVerifyError) as e:
        d.run(h, 0)
    assert e.value.status == _lib.MLA_ERR_INVALID_ARGUMENT
    lib = _lib.load()
    import ctypes
    misaligned = ctypes.c_void_p(d.q.data_ptr() + 2)
    st = lib.mla_verify_run(h._h, misaligned, ctypes.c_void_p(d.pool.data_ptr()), ctypes.c_void_p(d.slot_idx.data_ptr()),
                            ctypes.c_void_p(d.seq_lens.data_ptr()), ctypes.c_void_p(d.q_lens.data_ptr()),
                            ctypes.c_void_p(d.out.data_ptr()), ctypes.c_void_p(d.lse.data_ptr()), 1, None)
    assert st == _lib.MLA_ERR_INVALID_ARGUMENT
