"""The parity rules themselves, on the CPU: the bridge checks take their
references from the oracle and accept an fp32-accumulated result, and they
reject a result with a planted systematic error."""

import numpy as np
import pytest

from oracle import hs2_oracle as O
from tests import parity


def _case(seed=0, t=96, d=512):
    rng = np.random.default_rng(seed)
    h = O.f64_to_bf16_bits(rng.standard_normal((t, d)) / np.sqrt(d))
    w = O.f64_to_bf16_bits(rng.standard_normal((d, 128)) / np.sqrt(d))
    # an fp32 accumulation of the exact products, as a GPU GEMM does (not the oracle)
    acc = (O.bf16_bits_to_f64(h).astype(np.float32) @ O.bf16_bits_to_f64(w).astype(np.float32)).astype(np.float64)
    return h, w, acc


def test_bridge_check_accepts_fp32_accumulation():
    h, w, acc = _case()
    rows = np.arange(h.shape[0])
    worst, frac1 = parity.check_bridge(h, w, O.f64_to_bf16_bits(acc), rows)
    assert worst <= 2 and frac1 >= 0.999


def test_bridge_check_rejects_truncation_and_offsets():
    h, w, acc = _case(1)
    rows = np.arange(h.shape[0])
    good = O.f64_to_bf16_bits(acc)
    bumped = (good.astype(np.int32) + np.where(good & 0x8000, -2, 2)).astype(np.uint16)  # 2 ulps toward +-inf everywhere
    with pytest.raises(AssertionError):
        parity.check_bridge(h, w, bumped, rows)
    trunc = (np.ascontiguousarray(acc.astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)  # round toward 0
    with pytest.raises(AssertionError):
        parity.check_bridge(h, w, trunc, rows)


def test_bridge_fp8_check_accepts_and_rejects():
    h, w, acc = _case(2)
    rows = np.arange(h.shape[0])
    codes, scale = O.quantize_rows_e4m3(acc.astype(np.float32).astype(np.float64))
    same, rel = parity.check_bridge_fp8(h, w, codes, scale, rows)
    assert same >= 0.995
    shifted = codes.copy()
    shifted[::7] = np.where(shifted[::7] & 0x7F < 0x7D, shifted[::7] + 2, shifted[::7])  # two steps up
    with pytest.raises(AssertionError):
        parity.check_bridge_fp8(h, w, shifted, scale, rows)
    with pytest.raises(AssertionError):
        parity.check_bridge_fp8(h, w, codes, scale * np.float32(1.001), rows)


def test_fp32_logit_band_is_below_the_tie_band_at_workload_magnitudes():
    assert parity.fp32_logit_band(5.0) < O.BAND_REL
    assert parity.fp32_logit_band(360.0) > O.BAND_REL
