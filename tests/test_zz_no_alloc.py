"""The entry point that allocates nothing (mla_verify_run_noalloc): its split partials live in the
library's fixed per-GPU scratch array instead of a handle's workspace.  Through the C ABI, each
call must equal mla_verify_run on a handle of the same config bit for bit, over consecutive calls
whose inputs shrink (the array keeps the previous call's partials), and the oracle to the parity
bar (max |out err| <= 1e-2, max |lse err| <= 1e-3)."""
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


def _compare(api, x, nsplit, label):
    print(f"noalloc {label}: B={len(x.seq_lens)} H={x.heads} L={x.seq_lens.tolist()} nsplit={nsplit}", flush=True)
    B, max_q = len(x.seq_lens), int(max(1, x.q_lens.max()))
    d = DeviceInputs(x)
    h = api.MlaVerify(x.heads, B, max_q, nsplit, x.num_slots, x.scale)
    o_ref, l_ref = (t.clone() for t in d.run(h, nsplit))
    torch.cuda.synchronize()
    h.close()
    d.out.fill_(0)
    d.lse.fill_(0)
    out, lse = api.run_noalloc(d.q, d.pool, d.slot_idx, d.seq_lens, d.q_lens, d.out, d.lse, nsplit,
                               x.heads, B, max_q, nsplit, x.num_slots, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref), label
    ro, rl = oracle.verify_attention(x.q, x.sparse_pool(), x.slot_idx, x.seq_lens, x.q_lens, x.scale)
    eo, el = max_errors(out, lse, ro, rl)
    print(f"noalloc {label}: bitwise equal to the handle call; max|out err|={eo:.3e} max|lse err|={el:.3e}",
          flush=True)
    assert eo <= OUT_TOL and el <= LSE_TOL


def test_noalloc_equals_handle_call_on_shrinking_calls(api):
    # 1,024 rows at nsplit 32 (32.1 MiB of partials, the 128-row form), then a smaller batch through
    # the range plan, then a decode step at nsplit 256 (two-stream form) and at nsplit 16 (four-stream
    # form), then the first shape again
    big = I.make_custom(np.random.default_rng(70), [9000], [16], 64, 20000)
    _compare(api, big, 32, "one request, 128-row form")
    _compare(api, I.make_custom(np.random.default_rng(71), [700, 300, 41], [8, 8, 3], 16, 3000), 4, "batch, range plan")
    _compare(api, I.make_custom(np.random.default_rng(72), [4000], [1], 64, 9000), 256, "decode step")
    _compare(api, I.make_custom(np.random.default_rng(74), [3000], [1], 64, 7000), 16, "decode step, four streams")
    _compare(api, big, 32, "one request again")


def test_noalloc_rejects_a_call_past_its_scratch(api):
    from speculative_decode_mla_amd import _lib
    x = I.make_custom(np.random.default_rng(73), [300], [16], 64, 1000)
    d = DeviceInputs(x)
    with pytest.raises(_lib.MlaVerifyError) as e:  # 1,024 rows x 48 splits: 48.2 MiB
        api.run_noalloc(d.q, d.pool, d.slot_idx, d.seq_lens, d.q_lens, d.out, d.lse, 48, 64, 1, 16, 48,
                        x.num_slots, x.scale)
    assert e.value.status == _lib.MLA_ERR_SCRATCH_TOO_SMALL
