"""The seeded input generators: determinism, shapes and workload structure."""

import numpy as np
import pytest

from long_context_kv_hs2_amd import inputs
from oracle import hs2_oracle as O


def test_deterministic_per_seed():
    a = inputs.make_decode(lengths=[500, 2000], n_sparse=2, seed=11, needles=16)
    b = inputs.make_decode(lengths=[500, 2000], n_sparse=2, seed=11, needles=16)
    c = inputs.make_decode(lengths=[500, 2000], n_sparse=2, seed=12, needles=16)
    for key in ("k", "v", "q_full", "q_sparse", "seq_offsets"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["k"], c["k"])


def test_shapes_and_offsets():
    d = inputs.make_decode(lengths=[1, 129, 3000], n_sparse=3, seed=1)
    assert d["seq_offsets"].tolist() == [0, 1, 130, 3130]
    assert d["k"].shape == (3130, 128) and d["k"].dtype == np.uint16
    assert d["q_full"].shape == (3, 16, 128) and d["q_full"].dtype == np.float32
    assert d["q_sparse"].shape == (3, 3, 16, 128)


def test_needles_planted_before_window_and_aligned_with_mean_query():
    d = inputs.make_decode(lengths=[4096], n_sparse=1, seed=3, needles=64)
    pos = d["needles"][0]
    assert pos.shape[0] == 64 and np.unique(pos).shape[0] == 64
    assert pos.max() < 4096 - 128
    k = O.bf16_bits_to_f64(d["k"])
    qbar = d["q_full"][0].astype(np.float64).mean(axis=0)
    u = qbar / np.linalg.norm(qbar)
    proj = k @ u
    others = np.setdiff1d(np.arange(4096), pos)
    assert abs(proj[pos].mean() - 3.0) < 0.4 and abs(proj[others].mean()) < 0.1


def test_fp8_quantisation_per_token():
    d = inputs.make_decode(lengths=[2000], n_sparse=1, kv="fp8_e4m3", seed=5)
    assert d["k"].dtype == np.uint8 and d["k_scale"].shape == (2000,)
    vals = O.e4m3_bytes_to_f64(d["k"])
    assert not np.isnan(vals).any()
    assert np.abs(vals).max() <= 448.0
    # each row reaches the top of the E4M3 range
    assert np.all(np.abs(vals).max(axis=1) >= 416.0)


def test_burst_needles_structure():
    cfg = inputs.WORKLOAD_RECIPES[3]
    rng = np.random.default_rng(0)
    pos = inputs._needle_positions(rng, cfg, 1 << 20, None)
    assert pos.shape[0] == 1024
    runs = np.split(pos, np.nonzero(np.diff(pos) != 1)[0] + 1)
    assert sum(r.shape[0] for r in runs) == 1024
    assert all(r.shape[0] % 128 == 0 for r in runs)  # bursts of 128 (adjacent bursts may touch)
    assert pos.max() < (1 << 20) - 256


def test_agent_spans_and_lengths():
    rng = np.random.default_rng(1)
    lens = inputs.agent_lengths(rng, 1000, 2048, 262144)
    assert lens.min() >= 2048 and lens.max() <= 262144
    # log-uniform: the median sits near the geometric mean
    assert abs(np.log(np.median(lens)) - 0.5 * (np.log(2048) + np.log(262144))) < 0.3
    spans = inputs.agent_spans(rng, 50000)
    assert spans[0][0] == "action" and spans[-1][2] == 50000
    for a, b in zip(spans, spans[1:]):
        assert a[2] == b[1] and a[0] != b[0]
    for kind, s, e in spans[:-1]:
        n = e - s
        assert (16 <= n <= 64) if kind == "action" else (2048 <= n <= 32768)


def test_agent_needles_only_in_observations():
    cfg = inputs.WORKLOAD_RECIPES[4]
    rng = np.random.default_rng(2)
    spans = inputs.agent_spans(rng, 40000)
    pos = inputs._needle_positions(rng, cfg, 40000, spans)
    assert pos.shape[0] == round(40000 / 512)
    obs = np.zeros(40000, bool)
    for kind, s, e in spans:
        if kind == "obs":
            obs[s:e] = True
    assert obs[pos].all() and pos.max() < 40000 - 128
