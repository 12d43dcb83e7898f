"""The debug build of the library (libmla_verify_debug.so, MLA_VERIFY_DEBUG): device-visible
arguments that break the contract -- a slot outside the pool, a negative length, a q_len past its
request's length -- are replaced before any memory access and recorded in the handle's flag word.
Every case below keeps each access inside the caller's buffers only because the debug build
clamps; none of them is run on the release build.  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_mla_amd import inputs as I
from tests.gpu_helpers import LSE_TOL, OUT_TOL, DeviceInputs, bits_to_bf16, max_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decode_mla_amd import api as A
    from speculative_decode_mla_amd import _lib
    if not __import__("os").path.exists(_lib.DEBUG_LIB_PATH):
        pytest.skip("debug library not built")
    return A


def _lib():
    from speculative_decode_mla_amd import _lib as L
    return L


def _run(api, h, q, pool, slots, seq, ql, t_q, heads, nsplit):
    out = torch.empty((t_q, heads, I.D_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((t_q, heads), dtype=torch.float32, device="cuda")
    h.run(q, pool, slots, seq, ql, out, lse, nsplit)
    torch.cuda.synchronize()
    return out, lse


def test_valid_call_sets_no_flag_and_matches_release(api):
    x = I.make_custom(np.random.default_rng(80), [2000, 300], [16, 4], 16, 5000)
    d = DeviceInputs(x)
    rel = api.MlaVerify(x.heads, 2, 16, 8, x.num_slots, x.scale)
    dbg = api.MlaVerify(x.heads, 2, 16, 8, x.num_slots, x.scale, debug=True)
    o1, l1 = (t.clone() for t in d.run(rel, 8))
    o2, l2 = d.run(dbg, 8)
    torch.cuda.synchronize()
    assert dbg.debug_flags() == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    with pytest.raises(_lib().MlaVerifyError) as e:
        rel.debug_flags()
    assert e.value.status == _lib().MLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("form", [1, 2, 3])
def test_slot_outside_the_pool_is_clamped_and_flagged(api, form):
    """Slots past the pool's end and negative slots read the pool's last and first rows instead
    (which hold finite rows here): the result equals the oracle over the clamped slot list."""
    N = 4096
    rng = np.random.default_rng(81)
    x = I.make_custom(rng, [700, 300], [8, 8], 16, N - 2)        # slots in [0, N - 2): rows 0 .. N-3
    slots = (x.slot_idx + 1).astype(np.int32)                     # shift into [1, N - 1): rows 0 and N-1 free
    pool = np.full((N, I.D_QK), I.BF16_QNAN, dtype=np.uint16)
    pool[slots] = x.kv_rows
    pool[0] = I.f32_to_bf16_bits(rng.standard_normal(I.D_QK, dtype=np.float32))
    pool[N - 1] = I.f32_to_bf16_bits(rng.standard_normal(I.D_QK, dtype=np.float32))
    bad = slots.copy()
    bad[[3, 100, 699]] = [N, N + 12345, 2**31 - 1]                # past the end (request 0)
    bad[[5, 702]] = [-1, -(2**31)]                                # negative (requests 0 and 1)
    clamped = np.clip(bad.astype(np.int64), 0, N - 1).astype(np.int32)
    dev = "cuda"
    q = bits_to_bf16(x.q, dev)
    dpool = bits_to_bf16(pool, dev)
    seq = torch.from_numpy(x.seq_lens).to(dev)
    ql = torch.from_numpy(x.q_lens).to(dev)
    h = api.MlaVerify(16, 2, 8, 4, N, x.scale, form=form, debug=True)
    assert h.debug_flags() == 0
    out, lse = _run(api, h, q, dpool, torch.from_numpy(bad).to(dev), seq, ql, 16, 16, 4)
    assert h.debug_flags() == _lib().DEBUG_SLOT_OUT_OF_RANGE
    ro, rl = oracle.verify_attention(x.q, pool, clamped, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ro, rl)
    assert eo <= OUT_TOL and el <= LSE_TOL
    # the flag word was cleared by the read: a valid call leaves it at zero
    _run(api, h, q, dpool, torch.from_numpy(slots).to(dev), seq, ql, 16, 16, 4)
    assert h.debug_flags() == 0


def test_negative_length_reads_as_zero_and_is_flagged(api):
    """seq_lens[1] = -5: request 1 has no keys and no rows; the others are unaffected."""
    x = I.make_custom(np.random.default_rng(82), [700, 0, 300], [8, 0, 8], 16, 3000)
    d = DeviceInputs(x)
    seq = x.seq_lens.copy()
    seq[1] = -5
    h = api.MlaVerify(16, 3, 8, 4, x.num_slots, x.scale, debug=True)
    out, lse = _run(api, h, d.q, d.pool, d.slot_idx, torch.from_numpy(seq).cuda(), d.q_lens, 16, 16, 4)
    assert h.debug_flags() == _lib().DEBUG_NEGATIVE_LENGTH
    ro, rl = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ro, rl)
    assert eo <= OUT_TOL and el <= LSE_TOL


@pytest.mark.parametrize("qlen", [5, -2])
def test_q_len_outside_its_range_is_clamped_and_flagged(api, qlen):
    """q_lens[1] past seq_lens[1] = 3 (or negative): clamped to 3 (or 0), like the release build,
    and flagged."""
    want = 3 if qlen > 0 else 0
    x = I.make_custom(np.random.default_rng(83), [400, 3], [8, want], 16, 1000)
    d = DeviceInputs(x)
    ql = x.q_lens.copy()
    ql[1] = qlen
    h = api.MlaVerify(16, 2, 8, 2, x.num_slots, x.scale, debug=True)
    out, lse = _run(api, h, d.q, d.pool, d.slot_idx, d.seq_lens, torch.from_numpy(ql).cuda(), 8 + want, 16, 2)
    assert h.debug_flags() == _lib().DEBUG_Q_LEN_OUT_OF_RANGE
    ro, rl = oracle.verify_attention(x.q, x.pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ro, rl)
    assert eo <= OUT_TOL and el <= LSE_TOL
