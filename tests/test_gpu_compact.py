"""GPU parity for KV compaction (bit-exact: it is byte work) and for verify attention over the
compacted rows (bitwise equal to the scattered rows).  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_mla_amd import inputs as I
from tests.gpu_helpers import DeviceInputs

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decode_mla_amd import api as A
    return A


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,dst_first", [(1, 0), (31, 5), (32, 0), (33, 40), (1000, 123), (4097, 7)])
def test_compact_matches_oracle(api, n, dst_first):
    rng = np.random.default_rng(1000 + n)
    n_slots, dst_slots = 8192, n + dst_first + 50
    src = rng.integers(0, 1 << 16, size=(n_slots, I.D_QK), dtype=np.uint16)
    slots = rng.permutation(n_slots)[:n].astype(np.int32)
    dst0 = np.full((dst_slots, I.D_QK), SENTINEL, dtype=np.uint16)
    want, want_idx = oracle.compact_rows(src, slots, dst0.copy(), dst_first)
    d_src, d_dst = _dev(src), _dev(dst0)
    d_slots = torch.from_numpy(slots).cuda()
    d_new = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    print(f"compact n={n} dst_first={dst_first}", flush=True)
    api.compact(d_src, d_slots, d_dst, dst_first, d_new)
    torch.cuda.synchronize()
    assert np.array_equal(_host(d_dst), want)
    assert np.array_equal(d_new.cpu().numpy(), want_idx)


def test_compact_empty_is_a_no_op(api):
    d_src = torch.zeros((16, I.D_QK), dtype=torch.bfloat16, device="cuda")
    d_dst = _dev(np.full((4, I.D_QK), SENTINEL, dtype=np.uint16))
    api.compact(d_src, torch.zeros((0,), dtype=torch.int32, device="cuda"), d_dst, 0)
    torch.cuda.synchronize()
    assert np.all(_host(d_dst) == SENTINEL)


def test_compact_within_one_pool(api):
    """Rows scattered over the lower half of a pool move to a free range in its upper half."""
    rng = np.random.default_rng(5)
    pool = np.full((4096, I.D_QK), SENTINEL, dtype=np.uint16)
    slots = rng.permutation(2048)[:700].astype(np.int32)
    pool[slots] = rng.integers(0, 1 << 16, size=(700, I.D_QK), dtype=np.uint16)
    want, _ = oracle.compact_rows(pool, slots, pool.copy(), 3000)
    d_pool = _dev(pool)
    api.compact(d_pool, torch.from_numpy(slots).cuda(), d_pool, 3000)
    torch.cuda.synchronize()
    assert np.array_equal(_host(d_pool), want)


@pytest.mark.parametrize("workload", ["ctx4k", "ctx64k"])
def test_verify_over_compacted_rows_is_bitwise_equal(api, workload):
    """Full-size: the compacted pool holds exactly the request's rows in key order (closed form:
    the generator's kv_rows), and verify attention over it returns the scattered pool's result bit for bit."""
    x = I.make_inputs(workload)
    w = I.WORKLOADS[workload]
    d = DeviceInputs(x)
    n = len(x.slot_idx)
    dst = torch.empty((n, I.D_QK), dtype=torch.bfloat16, device="cuda")
    new = torch.empty((n,), dtype=torch.int32, device="cuda")
    print(f"compact {workload}: {n} rows", flush=True)
    api.compact(d.pool, d.slot_idx, dst, 0, new)
    torch.cuda.synchronize()
    assert np.array_equal(_host(dst), x.kv_rows)
    assert np.array_equal(new.cpu().numpy(), np.arange(n, dtype=np.int32))
    h = api.MlaVerify(x.heads, len(x.seq_lens), int(x.q_lens.max()), w.nsplit, x.num_slots, x.scale)
    out_a, lse_a = d.run(h, w.nsplit)
    out_a, lse_a = out_a.clone(), lse_a.clone()
    h.run(d.q, dst, new, d.seq_lens, d.q_lens, d.out, d.lse, w.nsplit)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), d.out.view(torch.int16))
    assert torch.equal(lse_a, d.lse)
