"""Pins that tie the fp64 oracle to what the definition fixes, independent of the oracle's own code.

Each pin reaches the expected value by another route: a closed form, a library
routine (torch's float64 scaled-dot-product attention, scipy's logsumexp), an
invariant of the definition, or exact bf16 values written out by hand.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import mla_verify_oracle as om
from speculative_decode_mla_amd import inputs as I

SCALE = 1.0 / math.sqrt(192.0)


def _small(seed, lens, qlens, heads=3, slots=None):
    rng = np.random.default_rng(seed)
    slots = slots or int(sum(lens)) * 3 + 7
    return I.make_custom(rng, lens, qlens, heads, slots)


def _run(x, split=None):
    pool = x.pool()
    if split is None:
        return oracle.verify_attention(x.q, pool, x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    return oracle.verify_attention_split(x.q, pool, x.slot_idx, x.seq_lens, x.q_lens, x.scale, split)


# --- bf16 decode: exact values written out by hand -------------------------------------------------

def test_bf16_decode_hand_values():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x4049, 0x0000, 0x8000, 0x0001, 0x7F7F, 0x7F80, 0xFF80],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.5, 3.140625, 0.0, -0.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127,
            math.inf, -math.inf]
    got = oracle.bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    finite = np.isfinite(t)
    assert np.array_equal(got[finite], t[finite])
    assert np.array_equal(np.isnan(got), np.isnan(t))


def test_generator_bf16_encode_matches_torch_rne():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.f32_to_bf16_bits(x), want)


# --- P-1: the whole definition against library routines ---------------------------------------------

def _dense_reference_torch(x):
    """Per request: gather with numpy fancy indexing, then torch float64 SDPA with an explicit mask."""
    pool = x.pool()
    outs, lses = [], []
    ko = qo = 0
    for L, Q in zip(x.seq_lens.tolist(), x.q_lens.tolist()):
        k = torch.from_numpy(pool[x.slot_idx[ko:ko + L]].view(np.int16).copy()).view(torch.bfloat16).double()
        q = torch.from_numpy(x.q[qo:qo + Q].view(np.int16).copy()).view(torch.bfloat16).double()  # [Q,H,576]
        q = q.permute(1, 0, 2)                                   # [H, Q, 576]
        kk = k.unsqueeze(0).expand(q.shape[0], L, 576)
        vv = k[:, :512].unsqueeze(0).expand(q.shape[0], L, 512)
        pos_q = torch.arange(Q).unsqueeze(1) + (L - Q)
        pos_k = torch.arange(L).unsqueeze(0)
        mask = pos_k <= pos_q                                     # [Q, L] True = attend
        o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=SCALE)
        s = (q @ kk.transpose(1, 2)) * SCALE
        s = s.masked_fill(~mask, -math.inf)
        lse = torch.logsumexp(s, dim=-1)                          # [H, Q]
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(lse.T.numpy())
        ko += L
        qo += Q
    return np.concatenate(outs), np.concatenate(lses)


@pytest.mark.parametrize("seed,lens,qlens,heads", [
    (0, [9], [4], 3), (1, [1, 5, 17], [1, 2, 4], 2), (2, [33, 8], [3, 8], 4), (3, [64], [16], 1),
])
def test_p1_matches_torch_sdpa(seed, lens, qlens, heads):
    x = _small(seed, lens, qlens, heads)
    out, lse = _run(x)
    ro, rl = _dense_reference_torch(x)
    assert np.max(np.abs(out - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


def test_p1_scipy_logsumexp_rows():
    x = _small(11, [40], [5], 2)
    out, lse = _run(x)
    pool = x.pool()
    k = oracle.bf16_bits_to_f64(pool[x.slot_idx])
    for t in range(5):
        for h in range(2):
            q = oracle.bf16_bits_to_f64(x.q[t, h])
            s = np.array([math.fsum(q[d] * k[j, d] for d in range(576)) for j in range(40 - 5 + t + 1)]) * SCALE
            assert abs(lse[t, h] - logsumexp(s)) < 1e-12


# --- P-2: one context token ------------------------------------------------------------------------

def test_p2_single_token_returns_v_row():
    x = _small(4, [1], [1], 5)
    out, lse = _run(x)
    row = oracle.bf16_bits_to_f64(x.kv_rows[0])
    for h in range(5):
        assert np.array_equal(out[0, h], row[:512])
        q = oracle.bf16_bits_to_f64(x.q[0, h])
        assert abs(lse[0, h] - SCALE * math.fsum(q * row)) < 1e-12


# --- P-3: identical scores -> mean of the visible V rows --------------------------------------------

def test_p3_zero_query_gives_prefix_means():
    x = _small(5, [30], [6], 2)
    x.q[:] = 0
    out, lse = _run(x)
    v = oracle.bf16_bits_to_f64(x.kv_rows)[:, :512]
    for t in range(6):
        n = 30 - 6 + t + 1
        assert np.max(np.abs(out[t] - v[:n].mean(axis=0))) < 1e-12
        assert np.max(np.abs(lse[t] - math.log(n))) < 1e-12


def test_p3_shared_rope_dims_give_equal_scores():
    x = _small(6, [20], [4], 3)
    x.kv_rows[:, 512:] = x.kv_rows[0, 512:]      # every key shares the rope dims
    x.q[:, :, :512] = 0                          # q only sees the rope dims
    out, lse = _run(x)
    v = oracle.bf16_bits_to_f64(x.kv_rows)[:, :512]
    rope = oracle.bf16_bits_to_f64(x.kv_rows[0, 512:])
    for t in range(4):
        n = 20 - 4 + t + 1
        for h in range(3):
            s = SCALE * math.fsum(oracle.bf16_bits_to_f64(x.q[t, h, 512:]) * rope)
            assert np.max(np.abs(out[t, h] - v[:n].mean(axis=0))) < 1e-12
            assert abs(lse[t, h] - (s + math.log(n))) < 1e-12


# --- P-4: slot placement does not matter ------------------------------------------------------------

def test_p4_slot_permutation_invariance():
    x = _small(7, [25, 13], [3, 2], 2)
    out, lse = _run(x)
    rng = np.random.default_rng(99)
    perm = rng.permutation(x.num_slots)
    y = I.VerifyInputs(q=x.q, kv_rows=x.kv_rows, slot_idx=perm[x.slot_idx].astype(np.int32),
                       seq_lens=x.seq_lens, q_lens=x.q_lens, num_slots=x.num_slots, heads=x.heads)
    out2, lse2 = _run(y)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_p4_unreferenced_rows_are_never_read():
    x = _small(8, [12], [3], 2)
    out, lse = _run(x)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))  # the pool holds NaN everywhere else


# --- P-5: split + reduce equals the unsplit result ----------------------------------------------------

@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 8, 16, 32, 80])
def test_p5_split_equals_unsplit(nsplit):
    x = _small(9, [37, 5, 64], [4, 5, 16], 2)
    out, lse = _run(x)
    out2, lse2 = _run(x, split=nsplit)
    assert np.max(np.abs(out - out2)) < 1e-12
    assert np.max(np.abs(lse - lse2)) < 1e-12


def test_p5_merge_of_empty_partials():
    o = np.zeros((3, 2, 512))
    l = np.full((3, 2), -np.inf)
    out, lse = oracle.merge_partials(o, l)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# --- P-6: the causal boundary -------------------------------------------------------------------------

def test_p6_first_masked_key_does_not_move_output():
    L, Q = 24, 4
    x = _small(10, [L], [Q], 3)
    base_out, base_lse = _run(x)
    # spike the draft row that token 0 must not see (absolute key L - Q + 1) toward token 1's query
    j = L - Q + 1
    x.kv_rows[j] = I.f32_to_bf16_bits(8.0 * oracle.bf16_bits_to_f64(x.q[1, 0]).astype(np.float32))
    out, lse = _run(x)
    assert np.array_equal(out[0], base_out[0]) and np.array_equal(lse[0], base_lse[0])
    assert np.max(np.abs(out[1] - base_out[1])) > 1e-3     # token 1 sees it
    assert lse[1, 0] > base_lse[1, 0] + 5


def test_p6_own_row_is_visible():
    L, Q = 10, 3
    x = _small(12, [L], [Q], 1)
    base_out, _ = _run(x)
    x.kv_rows[L - Q] = I.f32_to_bf16_bits(8.0 * oracle.bf16_bits_to_f64(x.q[0, 0]).astype(np.float32))
    out, _ = _run(x)
    assert np.max(np.abs(out[0] - base_out[0])) > 1e-3


# --- P-8: two keys in closed form -----------------------------------------------------------------------

def test_p8_two_key_closed_form():
    x = _small(13, [2], [1], 2)
    out, lse = _run(x)
    k = oracle.bf16_bits_to_f64(x.kv_rows)
    for h in range(2):
        q = oracle.bf16_bits_to_f64(x.q[0, h])
        s0 = SCALE * math.fsum(q * k[0])
        s1 = SCALE * math.fsum(q * k[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        want = w0 * k[0, :512] + w1 * k[1, :512]
        assert np.max(np.abs(out[0, h] - want)) < 1e-12
        assert abs(lse[0, h] - np.logaddexp(s0, s1)) < 1e-12


# --- sampled rows agree with the full evaluation ---------------------------------------------------------

def test_rows_mode_matches_full():
    x = _small(14, [50, 20], [5, 3], 3)
    out, lse = _run(x)
    rows = [(0, 0), (4, 2), (5, 1), (7, 0), (2, 1)]
    o2, l2 = oracle.verify_attention_rows(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale, rows)
    for i, (t, h) in enumerate(rows):
        assert np.max(np.abs(o2[i] - out[t, h])) < 1e-13 and abs(l2[i] - lse[t, h]) < 1e-13


# --- planted mistakes in the oracle must trip at least one pin --------------------------------------------

def _pins_pass():
    checks = [
        lambda: test_p1_matches_torch_sdpa(2, [33, 8], [3, 8], 4),
        test_p2_single_token_returns_v_row,
        test_p3_zero_query_gives_prefix_means,
        lambda: test_p5_split_equals_unsplit(3),
        test_p6_first_masked_key_does_not_move_output,
        test_p8_two_key_closed_form,
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


_ORIG_ATTEND = om._attend
_ORIG_MERGE = om.merge_partials


def _gather_transposed(kv_pool, slot_idx, start, count):
    # the gathered [count, 576] block read back as if it were stored [576, count]
    rows = om.bf16_bits_to_f64(kv_pool[np.asarray(slot_idx[start:start + count], dtype=np.int64)])
    return rows.reshape(om.D_QK, count).T.copy()


MUTANTS = {
    "transposed key operand (rows read as columns)": ("_gather_keys", _gather_transposed),
    "base-2 LSE": ("_attend", lambda q, k, scale: (lambda o, l: (o, l / math.log(2.0)))(*_ORIG_ATTEND(q, k, scale))),
    "last split dropped in the merge": ("merge_partials", lambda o, l: _ORIG_MERGE(o[:-1], l[:-1])),
    "mask off by one (drop own row)": ("visible_count", lambda L, Q, t: L - Q + t),
    "mask off by one (see next draft)": ("visible_count", lambda L, Q, t: min(L, L - Q + t + 2)),
    "no causal mask": ("visible_count", lambda L, Q, t: L),
    "wrong scale (1/sqrt(576))": ("_scores", lambda q, k, scale: (q @ k.T) / math.sqrt(576)),
    "rope dims dropped from the score": ("_scores", lambda q, k, scale: scale * (q[:, :512] @ k[:, :512].T)),
    "max not subtracted consistently": ("_softmax_stats",
                                       lambda s: (np.exp(s), s.max(-1), np.exp(s).sum(-1))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(om, attr, fn)
    assert not _pins_pass(), f"pins did not catch: {name}"


def test_pins_pass_unmutated():
    assert _pins_pass()
