"""GPU parity for the device-side step metadata (bit-exact: integer work), and the captured
step it enables: metadata built and consumed inside one graph, replayed with new lengths.
All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_mla_amd import inputs as I
from tests.gpu_helpers import DeviceInputs

pytestmark = pytest.mark.gpu

SENTINEL = -12345


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decode_mla_amd import api as A
    return A


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _build(api, table, ids, pre, dr, cap, width=None):
    B = len(ids)
    out = dict(slot_idx=torch.full((cap,), SENTINEL, dtype=torch.int32, device="cuda"),
               seq_lens=torch.full((max(B, 1),), SENTINEL, dtype=torch.int32, device="cuda"),
               q_lens=torch.full((max(B, 1),), SENTINEL, dtype=torch.int32, device="cuda"),
               status=torch.full((1,), SENTINEL, dtype=torch.int32, device="cuda"))
    api.build_metadata(_i32(table), _i32(ids), _i32(pre), _i32(dr), out["slot_idx"], out["seq_lens"],
                       out["q_lens"], out["status"], table_width=width)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _check(api, table, ids, pre, dr, cap, label):
    print(f"metadata {label}: B={len(ids)} cap={cap}", flush=True)
    got = _build(api, table, ids, pre, dr, cap)
    slots, seq, ql, st = oracle.build_step_metadata(table, ids, pre, dr, cap)
    B = len(ids)
    assert int(got["status"][0]) == st
    assert np.array_equal(got["seq_lens"][:B], seq) and np.array_equal(got["q_lens"][:B], ql)
    assert np.array_equal(got["slot_idx"][:len(slots)], slots)
    assert np.all(got["slot_idx"][len(slots):] == SENTINEL)  # nothing written past the step's slots


def _random_table(rng, rows, width):
    return rng.integers(0, 1 << 30, size=(rows, width), dtype=np.int64).astype(np.int32)


@pytest.mark.parametrize("seed,B,rows,width", [(0, 1, 4, 300), (1, 4, 12, 300), (2, 37, 64, 2000),
                                               (3, 1024, 1100, 64)])
def test_metadata_matches_oracle(api, seed, B, rows, width):
    rng = np.random.default_rng(seed)
    table = _random_table(rng, rows, width)
    ids = rng.permutation(rows)[:B]
    dr = rng.integers(0, 17, B)
    pre = np.array([rng.integers(0, width - d + 1) for d in dr])
    pre[::5] = 0  # some requests with no prefix, some with no drafts
    dr[1::7] = 0
    _check(api, table, ids, pre, dr, int((pre + dr).sum()) + 3, f"seed {seed}")


def test_metadata_many_blocks(api):
    """A step larger than one workgroup's share: the batch-16 lengths, 310,806 slots."""
    x = I.make_inputs("batch16")
    width = int(x.seq_lens.max())
    table = np.full((20, width), -1, dtype=np.int32)
    ids = np.array([19 - b for b in range(16)])
    ko = np.concatenate([[0], np.cumsum(x.seq_lens)])
    for b in range(16):
        table[ids[b], :x.seq_lens[b]] = x.slot_idx[ko[b]:ko[b + 1]]
    pre = x.seq_lens - x.q_lens
    got = _build(api, table, ids, pre, x.q_lens, 1 << 22)
    assert int(got["status"][0]) == 0
    assert np.array_equal(got["slot_idx"][:len(x.slot_idx)], x.slot_idx)
    assert np.array_equal(got["seq_lens"][:16], x.seq_lens) and np.array_equal(got["q_lens"][:16], x.q_lens)


@pytest.mark.parametrize("ids,pre,dr,cap", [
    ([12], [0], [1], 100), ([-1], [0], [1], 100), ([1], [-1], [1], 100), ([1], [299], [2], 1000),
    ([1, 2], [100, 100], [1, 1], 201), ([12, 1], [-5, 299], [0, 2], 1000), ([1, 2], [100, 100], [1, 0], 201)])
def test_metadata_status(api, ids, pre, dr, cap):
    table = (np.arange(12)[:, None] * 100_000 + np.arange(300)[None, :]).astype(np.int32)
    _check(api, table, np.array(ids), np.array(pre), np.array(dr), cap, f"status {ids} {pre} {dr} {cap}")


def test_empty_batch(api):
    table = np.zeros((2, 8), dtype=np.int32)
    got = _build(api, table, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), 16)
    assert int(got["status"][0]) == 0 and np.all(got["slot_idx"] == SENTINEL)


def test_captured_step_with_device_metadata(api):
    """Metadata build + verify captured once; replays with new lengths written into the same static
    buffers give, bit for bit, what an eager call on host-built metadata gives."""
    rng = np.random.default_rng(9)
    H, B, qmax, width = 16, 3, 6, 700
    lens_all = [600, 450, 700]
    x = I.make_custom(rng, lens_all, [qmax] * B, H, 4096)
    d = DeviceInputs(x)
    table = np.full((5, width), 0, dtype=np.int32)
    ids = np.array([4, 0, 2])
    ko = np.concatenate([[0], np.cumsum(x.seq_lens)])
    for b in range(B):
        table[ids[b], :x.seq_lens[b]] = x.slot_idx[ko[b]:ko[b + 1]]
    t_table, t_ids = _i32(table), _i32(ids)
    t_pre, t_dr = _i32(np.zeros(B)), _i32(np.zeros(B))
    slot_idx = torch.zeros((4096,), dtype=torch.int32, device="cuda")
    seq_lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    q_lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    h = api.MlaVerify(H, B, qmax, 4, x.num_slots, x.scale)
    steps = [([500, 300, 694], [6, 2, 6]), ([100, 440, 650], [1, 6, 0]), ([594, 444, 600], [6, 6, 6])]
    # q rows of each step: the first q_lens[b] draft rows of request b, requests in order
    def q_of(dr):
        rows, qo = [], 0
        for b in range(B):
            rows.append(x.q[qo:qo + dr[b]])
            qo += qmax
        return np.concatenate(rows)
    t_q = torch.zeros((B * qmax, H, I.D_QK), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B * qmax, H, I.D_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B * qmax, H), dtype=torch.float32, device="cuda")

    def step():
        api.build_metadata(t_table, t_ids, t_pre, t_dr, slot_idx, seq_lens, q_lens, status)
        h.run(t_q, d.pool, slot_idx, seq_lens, q_lens, out, lse, 4)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for pre, dr in steps:
        n_q = int(sum(dr))
        qs = q_of(dr)
        t_q[:n_q] = torch.from_numpy(qs.view(np.int16)).cuda().view(torch.bfloat16)
        t_pre.copy_(_i32(pre))
        t_dr.copy_(_i32(dr))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        got_o, got_l = out[:n_q].clone(), lse[:n_q].clone()
        # eager call on host-built metadata
        hs, hseq, hql, hst = oracle.build_step_metadata(table, ids, pre, dr, 4096)
        e_out = torch.zeros_like(out)
        e_lse = torch.zeros_like(lse)
        h.run(t_q, d.pool, _i32(hs), _i32(hseq), _i32(hql), e_out, e_lse, 4)
        torch.cuda.synchronize()
        assert torch.equal(got_o.view(torch.int16), e_out[:n_q].view(torch.int16))
        assert torch.equal(got_l, e_lse[:n_q])
        # and the oracle agrees on the step's result
        ro, rl = oracle.verify_attention(qs, x.pool(), hs, hseq, hql, x.scale)
        assert float(np.max(np.abs(got_o.float().cpu().numpy() - ro))) <= 1e-2
        assert float(np.max(np.abs(got_l.cpu().numpy() - rl))) <= 1e-3
