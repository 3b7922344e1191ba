"""hs2_decode_block_noalloc, through the C ABI: the decode step with the
library's own scratch array as its workspace, for callers that cannot
allocate.  Its outputs must equal hs2_decode_block's (no score output) bit
for bit, on two calls in a row, the second on a smaller batch (the scratch
keeps the first call's contents), and meet the oracle's bars."""

import numpy as np
import pytest
import torch

from long_context_kv_hs2_amd import hs2, inputs
from tests import parity

pytestmark = pytest.mark.gpu


def _one_call(d):
    t = parity.to_device(d)
    blk = hs2.DecodeBlock(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], t["k_scale"],
                          t["v_scale"], t["max_context"], with_score=False)
    blk()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in blk.outputs().items() if v is not None}
    for k, v in blk.outputs().items():
        if v is not None:
            v.fill_(-7)  # the no-alloc call must write every output itself
    torch.cuda.synchronize()
    hs2.decode_block_noalloc(blk)
    torch.cuda.synchronize()
    got = blk.outputs()
    for key, ref in want.items():
        assert torch.equal(got[key], ref), f"{key} differs from hs2_decode_block's"
    return got


def test_noalloc_equals_decode_block_twice_second_smaller():
    first = dict(lengths=[131072, 20000, 3000, 1153], n_sparse=4, kv="bf16", seed=101, needles=64)
    second = dict(lengths=[5000, 1200], n_sparse=2, kv="fp8_e4m3", seed=102, needles=16)
    for case in (first, second):
        print(f"case: no-alloc decode {case}", flush=True)
        d = inputs.make_decode(**case)
        out = _one_call(d)
        w = parity.check_decode(d, out)
        print(f"worst {w}", flush=True)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    lib = hs2.load()
    d = hs2.make_desc(64, 64 * 262144, 262144, 4)
    assert lib.hs2_decode_workspace_bytes(d) > hs2.NOALLOC_SCRATCH_BYTES
    z = torch.zeros(16, dtype=torch.int64, device="cuda")
    f = torch.zeros(16, dtype=torch.float32, device="cuda")
    p = lambda t: t.data_ptr()
    st = lib.hs2_decode_block_noalloc(d, p(z), p(z), p(z), None, None, p(f), p(f), p(f), p(f), p(z), p(z), None)
    assert st == 2 and "scratch" in lib.hs2_last_error_message().decode()
