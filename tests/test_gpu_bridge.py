"""GPU parity of the KV-Bridging GEMM on small and ragged shapes (every
element checked against the oracle)."""

import numpy as np
import pytest
import torch

from long_context_kv_hs2_amd import hs2, inputs
from tests import parity

pytestmark = pytest.mark.gpu


def to_dev(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("tokens,d_model,n_bridged", [(1000, 256, 2), (128, 64, 1), (1, 4096, 3), (5000, 4096, 4)])
def test_bridge_small_shapes(tokens, d_model, n_bridged):
    print(f"case: bridge T={tokens} d_model={d_model} n_bridged={n_bridged}", flush=True)
    br = inputs.make_bridge(tokens=tokens, d_model=d_model, n_bridged=n_bridged, seed=tokens + d_model)
    k_out, v_out = hs2.bridge_kv(to_dev(br["h"]), [to_dev(w) for w in br["w_k"]], [to_dev(w) for w in br["w_v"]])
    torch.cuda.synchronize()
    rows = np.arange(tokens)
    for l in range(n_bridged):
        for w_bits, out in ((br["w_k"][l], k_out[l]), (br["w_v"][l], v_out[l])):
            parity.check_bridge(br["h"], w_bits, out.view(torch.int16).cpu().numpy().view(np.uint16), rows)


def test_bridge_zero_tokens():
    h = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda")
    w = [torch.zeros((4096, 128), dtype=torch.bfloat16, device="cuda")]
    k_out, v_out = hs2.bridge_kv(h, w, w)
    torch.cuda.synchronize()
    assert k_out[0].shape == (0, 128)


def test_bridge_one_hot_weights_copy_columns():
    rng = np.random.default_rng(3)
    tokens, d_model = 777, 512
    br = inputs.make_bridge(tokens=tokens, d_model=d_model, n_bridged=1, seed=9)
    cols = rng.integers(0, d_model, size=128)
    w = np.zeros((d_model, 128), np.float32)
    w[cols, np.arange(128)] = 1.0
    wb = inputs.to_bf16_bits(w)
    k_out, _ = hs2.bridge_kv(to_dev(br["h"]), [to_dev(wb)], [to_dev(wb)])
    torch.cuda.synchronize()
    got = k_out[0].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, br["h"][:, cols])
