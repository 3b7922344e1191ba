"""Pins of the oracle's Self-Decoder sliding-window attention over a ring
buffer: against attention over the last positions of a linear cache whose
rows were appended one decode step at a time, against torch's
scaled_dot_product_attention with a sliding-window mask, and closed cases;
planted mistakes in copies must fail a pin."""

import math

import numpy as np
import pytest
import torch

from oracle import hs2_oracle as O


def decode_appends(k_lin, v_lin, window):
    """The ring after appending positions 0..L-1 one step at a time, each
    overwriting the oldest row once the ring is full."""
    ring_k = np.full((window, k_lin.shape[1]), np.nan)
    ring_v = np.full((window, v_lin.shape[1]), np.nan)
    oldest = 0
    for p in range(k_lin.shape[0]):
        if p < window:
            ring_k[p], ring_v[p] = k_lin[p], v_lin[p]
        else:
            ring_k[oldest], ring_v[oldest] = k_lin[p], v_lin[p]
            oldest = (oldest + 1) % window
    return ring_k, ring_v


def sdpa_window(q, k_lin, v_lin, window):
    length = k_lin.shape[0]
    allowed = torch.zeros(1, length, dtype=torch.bool)
    allowed[0, max(0, length - window):] = True
    tq = torch.from_numpy(q)[None, :, None, :]
    tk = torch.from_numpy(k_lin)[None, None].expand(1, q.shape[0], length, k_lin.shape[1]).contiguous()
    tv = torch.from_numpy(v_lin)[None, None].expand(1, q.shape[0], length, v_lin.shape[1]).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed)[0, :, 0].numpy()


def swa_pin(swa):
    rng = np.random.default_rng(31)
    ok = True
    for length, window in [(5, 8), (8, 8), (9, 8), (37, 8), (300, 128), (129, 128)]:
        q = rng.standard_normal((16, 32))
        k_lin = rng.standard_normal((length, 32))
        v_lin = rng.standard_normal((length, 32))
        ring_k, ring_v = decode_appends(k_lin, v_lin, window)
        got = swa(q, np.nan_to_num(ring_k), np.nan_to_num(ring_v), length, window)
        ok = ok and np.allclose(got, sdpa_window(q, k_lin, v_lin, window), rtol=1e-12, atol=1e-13)
    return ok


def test_swa_matches_windowed_sdpa_on_appended_ring():
    assert swa_pin(O.swa_attention)


@pytest.mark.parametrize("length", [1, 50, 128])
def test_short_context_is_full_attention(length):
    rng = np.random.default_rng(length)
    q = rng.standard_normal((16, 128))
    ring_k = rng.standard_normal((128, 128))
    ring_v = rng.standard_normal((128, 128))
    want, _ = O.full_attention(q, ring_k[:length], ring_v[:length])
    np.testing.assert_allclose(O.swa_attention(q, ring_k, ring_v, length), want, rtol=0, atol=1e-15)


def test_full_ring_is_order_free_and_constant_keys_average():
    # Once the window is full, every ring row is in it: the output is the
    # attention over all 128 rows whatever the current position; with equal
    # keys it is the mean of the values.
    rng = np.random.default_rng(2)
    q = rng.standard_normal((16, 128))
    ring_v = rng.standard_normal((128, 128))
    ring_k = np.tile(rng.standard_normal(128), (128, 1))
    for length in (128, 129, 1000, 1 << 20):
        np.testing.assert_allclose(O.swa_attention(q, ring_k, ring_v, length), np.tile(ring_v.mean(axis=0), (16, 1)),
                                   rtol=0, atol=1e-13)


def test_empty_sequence_gives_zeros():
    assert not O.swa_attention(np.ones((16, 128)), np.ones((128, 128)), np.ones((128, 128)), 0).any()


def test_swa_pin_catches_planted_mistakes():
    def window_too_long(q, rk, rv, length, window):
        slots = np.arange(max(0, length - window - 1), length) % window  # one position too many
        return O.full_attention(q, rk[slots], rv[slots])[0]

    def wrong_slot(q, rk, rv, length, window):
        slots = (np.arange(max(0, length - window), length) + 1) % window
        return O.full_attention(q, rk[slots], rv[slots])[0]

    def no_scale(q, rk, rv, length, window):
        slots = O.swa_ring_slots(length, window)
        lg = rk[slots] @ q.T
        e = np.exp(lg - lg.max(axis=0))
        return (e / e.sum(axis=0)).T @ rv[slots]

    for wrong in (window_too_long, wrong_slot, no_scale):
        assert not swa_pin(wrong), wrong.__name__
