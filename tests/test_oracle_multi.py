"""Pins of the oracle's multi-token decode (several query tokens of a
sequence in one step, each causal over its own prefix with its own
selection): against torch's scaled_dot_product_attention with a causal
mask, a causality invariant, and the last token's plain single-token decode;
planted mistakes in copies must fail a pin."""

import numpy as np
import pytest
import torch

from oracle import hs2_oracle as O


def case(rng, length, n_tok, n_s=2):
    q = rng.standard_normal((n_tok, 16, 128))
    qs = rng.standard_normal((n_s, n_tok, 16, 128))
    k = rng.standard_normal((length, 128))
    v = rng.standard_normal((length, 128))
    return q, qs, k, v


def sdpa_causal(q, k, v):
    """Full-layer outputs of T queries at the last T positions, causal."""
    n_tok, length = q.shape[0], k.shape[0]
    allowed = torch.zeros(n_tok, length, dtype=torch.bool)
    for t in range(n_tok):
        allowed[t, : length - n_tok + t + 1] = True
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]            # [1, H, T, D]
    tk = torch.from_numpy(k)[None, None].expand(1, 16, length, 128).contiguous()
    tv = torch.from_numpy(v)[None, None].expand(1, 16, length, 128).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed)
    return o[0].permute(1, 0, 2).numpy()                       # [T, H, D]


def full_pin(multi):
    rng = np.random.default_rng(12)
    ok = True
    for length, n_tok in [(40, 4), (1300, 3), (5000, 8)]:
        q, qs, k, v = case(rng, length, n_tok)
        got = np.stack([r["o_full"] for r in multi(q, qs, k, v)])
        ok = ok and np.allclose(got, sdpa_causal(q, k, v), rtol=1e-11, atol=1e-12)
    return ok


def causal_pin(multi):
    rng = np.random.default_rng(13)
    q, qs, k, v = case(rng, 3000, 4)
    base = multi(q, qs, k, v)
    ok = True
    for t in range(4):
        k2, v2 = k.copy(), v.copy()
        k2[3000 - 4 + t + 1:] += 5.0  # rows after token t's position
        v2[3000 - 4 + t + 1:] -= 5.0
        r = multi(q, qs, k2, v2)[t]
        ok = ok and np.array_equal(r["sel"], base[t]["sel"]) and np.allclose(r["o_sparse"], base[t]["o_sparse"],
                                                                              rtol=0, atol=1e-13)
    return ok


def test_full_layer_matches_causal_sdpa():
    assert full_pin(O.decode_multi_sequence)


def test_causal_prefixes():
    assert causal_pin(O.decode_multi_sequence)


@pytest.mark.parametrize("length", [100, 2000])
def test_last_token_is_the_single_token_decode(length):
    rng = np.random.default_rng(length)
    q, qs, k, v = case(rng, length, 5)
    last = O.decode_multi_sequence(q, qs, k, v)[-1]
    one = O.decode_sequence(q[-1], qs[:, -1], k, v)
    np.testing.assert_array_equal(last["sel"], one["sel"])
    np.testing.assert_allclose(last["o_sparse"], one["o_sparse"], rtol=0, atol=0)


def test_tokens_before_the_start_are_empty():
    rng = np.random.default_rng(1)
    q, qs, k, v = case(rng, 3, 5)
    r = O.decode_multi_sequence(q, qs, k, v)
    assert r[0] is None and r[1] is None and r[2]["sel"].tolist() == [0]


def test_multi_pins_catch_planted_mistakes():
    def off_by_one(q, qs, k, v, window=128, top_k=1024):
        n_tok, length = q.shape[0], k.shape[0]
        return [O.decode_sequence(q[t], qs[:, t], k[:length - n_tok + t], v[:length - n_tok + t])
                for t in range(n_tok)]

    def not_causal(q, qs, k, v, window=128, top_k=1024):
        return [O.decode_sequence(q[t], qs[:, t], k, v) for t in range(q.shape[0])]

    assert not full_pin(off_by_one)
    assert not full_pin(not_causal) and not causal_pin(not_causal)
