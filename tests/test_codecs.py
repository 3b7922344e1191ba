"""Pins of the oracle's stored-value codecs and of its bridge projection."""

import math

import numpy as np
import pytest
import torch

from oracle import hs2_oracle as O


def _expr(s):
    return float(eval(s, {"__builtins__": {}}, {"nan": math.nan}))  # fixture arithmetic only


def test_e4m3_table_matches_spec_landmarks(golden):
    table = O.e4m3_value_table()
    for ln in golden("e4m3_spec_values.txt"):
        code, val = ln.split(None, 1)
        want = _expr(val)
        got = table[int(code, 16)]
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_value_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_with_scale():
    codes = np.array([[0x38, 0x7E, 0x01]], dtype=np.uint8)
    out = O.decode_kv(codes, "fp8_e4m3", np.array([0.5], dtype=np.float32))
    np.testing.assert_array_equal(out, [[0.5, 224.0, 2.0 ** -10]])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_rne_hand_cases(golden):
    for ln in golden("bf16_rne_cases.txt"):
        # the fixture has two expressions separated by runs of spaces
        raw = ln.split("  ")
        exprs = [r.strip() for r in raw if r.strip()]
        x, want = _expr(exprs[0]), _expr(exprs[1])
        bits = O.f64_to_bf16_bits(np.array([x]))
        assert O.bf16_bits_to_f64(bits)[0] == want, ln


def test_bf16_rne_matches_torch_on_binary32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    # add exact halfway points: a random bf16 value plus half its spacing
    base = (rng.standard_normal(2000).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    x = np.concatenate([x, (base.view(np.uint32) | 0x8000).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ bridge

def _bits(x):
    return O.f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_bridge_one_hot_columns_pick_hidden_columns():
    rng = np.random.default_rng(2)
    t, dm = 40, 64
    h = _bits(rng.standard_normal((t, dm)))
    cols = rng.integers(0, dm, size=128)
    w = np.zeros((dm, 128)); w[cols, np.arange(128)] = 1.0
    ks, vs = O.bridge_kv(h, [_bits(w)], [_bits(2 * w)])
    hf = O.bf16_bits_to_f64(h)
    np.testing.assert_array_equal(ks[0], hf[:, cols])
    np.testing.assert_array_equal(vs[0], 2 * hf[:, cols])


def test_bridge_zero_weights_give_zero():
    rng = np.random.default_rng(3)
    h = _bits(rng.standard_normal((16, 32)))
    ks, vs = O.bridge_kv(h, [_bits(np.zeros((32, 128)))] * 2, [_bits(np.zeros((32, 128)))] * 2)
    assert all(np.all(k == 0) for k in ks) and all(np.all(v == 0) for v in vs)


def test_bridge_brute_force_tiny():
    rng = np.random.default_rng(4)
    t, dm = 3, 5
    h = _bits(rng.standard_normal((t, dm)))
    wk = [_bits(rng.standard_normal((dm, 128))) for _ in range(2)]
    wv = [_bits(rng.standard_normal((dm, 128))) for _ in range(2)]
    ks, vs = O.bridge_kv(h, wk, wv)
    hf = O.bf16_bits_to_f64(h)
    for layer in range(2):
        for which, out in ((wk, ks), (wv, vs)):
            w = O.bf16_bits_to_f64(which[layer])
            for i in range(t):
                for j in range(128):
                    acc = 0.0
                    for c in range(dm):
                        acc += hf[i, c] * w[c, j]
                    assert abs(out[layer][i, j] - acc) <= 1e-12 * (1 + abs(acc))


def test_bridge_rows_subset_matches_full():
    rng = np.random.default_rng(5)
    h = _bits(rng.standard_normal((50, 64)))
    w = [_bits(rng.standard_normal((64, 128)))]
    full, _ = O.bridge_kv(h, w, w)
    rows = np.array([0, 7, 49])
    part, _ = O.bridge_kv(h, w, w, rows=rows)
    np.testing.assert_array_equal(part[0], full[0][rows])


def test_e4m3_encode_hand_cases(golden):
    for ln in golden("e4m3_rounding_cases.txt"):
        x, code = ln.split("#")[0].split()[:-1], ln.split("#")[0].split()[-1]
        val = _expr(" ".join(x))
        got = int(O.f64_to_e4m3(np.array([val]))[0])
        assert got == int(code, 16), (ln, hex(got))


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_bytes_to_f64(codes)
    np.testing.assert_array_equal(O.f64_to_e4m3(vals), codes)


def test_e4m3_encode_matches_torch_within_range():
    # torch's float8_e4m3fn cast rounds to nearest even; within +-448 (where
    # no saturation question arises) the two encoders must agree everywhere.
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000) * 40.0, rng.standard_normal(50000) * 2.0 ** -7,
                        (np.arange(-2000, 2000) + 0.5) * 2.0 ** -9])
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.f64_to_e4m3(x)
    zero = (ref & 0x7F) == 0
    assert np.array_equal(got[~zero], ref[~zero])
    assert np.array_equal(got[zero] & 0x7F, ref[zero] & 0x7F)  # signed zeros aside


def test_quantize_rows_closed_forms():
    x = np.array([[3.0] * 128, [0.0] * 128, [-5.0] + [1.0] * 127], dtype=np.float64)
    codes, scale = O.quantize_rows_e4m3(x)
    assert scale.dtype == np.float32
    np.testing.assert_array_equal(scale, np.float32([3.0 / 448, 1.0, 5.0 / 448]))
    assert (codes[0] == 0x7E).all()          # every value is the row maximum: 448 * scale
    assert (codes[1] == 0x00).all()          # an all-zero row: scale 1, code 0
    assert codes[2, 0] == 0xFE                # the largest magnitude maps to -448
    # 1 / (5/448) = 89.6, between 88 (0x6B) and 96 (0x6C), nearer 88
    assert (codes[2, 1:] == 0x6B).all()
    back = O.e4m3_bytes_to_f64(codes) * scale.astype(np.float64)[:, None]
    np.testing.assert_allclose(back[0], 3.0, rtol=1e-7)
    np.testing.assert_allclose(back[2, 0], -5.0, rtol=1e-7)


def test_bridge_fp8_one_hot_columns():
    # One-hot W: K_l = the selected columns of H, then quantised per row;
    # compare with quantising those columns directly.
    rng = np.random.default_rng(7)
    h = O.f64_to_bf16_bits(rng.standard_normal((40, 256)) * 0.1)
    w = np.zeros((256, 128))
    cols = rng.permutation(256)[:128]
    w[cols, np.arange(128)] = 1.0
    wb = O.f64_to_bf16_bits(w)
    (kq,), (vq,) = O.bridge_kv_fp8(h, [wb], [wb])
    want = O.quantize_rows_e4m3(O.bf16_bits_to_f64(h)[:, cols])
    np.testing.assert_array_equal(kq[0], want[0])
    np.testing.assert_array_equal(kq[1], want[1])
    np.testing.assert_array_equal(vq[0], want[0])
