"""Pins of the oracle's gen-1 (block-level) selection, the ablation
comparator of the token-level one.

Checked against a hand-worked fixture, brute-force enumeration over block
subsets, the block-size-1 special case (which is the token-level rule),
closed forms, and invariants; planted mistakes in copies must fail a pin.
"""

import itertools

import numpy as np
import pytest

from oracle import hs2_oracle as O


def fixture(golden):
    return dict(ln.split(None, 1) for ln in golden("block_selection_worked.txt"))


def test_worked_block_fixture(golden):
    kv = fixture(golden)
    score = np.array([float(x) for x in kv["scores"].split()])
    got = O.select_blocks(score, window=int(kv["window"]), top_k=int(kv["top_k"]), block=int(kv["block"]))
    assert got["sel"].tolist() == [int(x) for x in kv["sel"].split()]
    assert got["s_k"] == float(kv["s_k"])
    assert got["band_blocks"].tolist() == [int(x) for x in kv["band_blocks"].split()]
    tok = O.select_tokens(score, window=int(kv["window"]), top_k=int(kv["top_k"]))
    assert tok["sel"].tolist() == [int(x) for x in kv["token_sel"].split()]


def block_dominance_ok(sums, chosen, domain):
    """Every chosen block beats every other candidate: larger sum, or an equal
    sum and a lower index."""
    for a in chosen:
        for b in domain:
            if b in chosen:
                continue
            if not (sums[a] > sums[b] or (sums[a] == sums[b] and a < b)):
                return False
    return True


def brute_blocks(score, window, top_k, block):
    n = len(score)
    if n <= window + top_k:
        return list(range(n))
    nb = (n - window) // block
    sums = [sum(int(score[i * block + j]) for j in range(block)) for i in range(nb)]  # exact integers
    good = [c for c in itertools.combinations(range(nb), top_k // block) if block_dominance_ok(sums, c, range(nb))]
    assert len(good) == 1
    pos = [i * block + j for i in good[0] for j in range(block)]
    return sorted(pos + list(range(n - window, n)))


@pytest.mark.parametrize("seed", range(16))
def test_block_selection_against_subset_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    block, window, top_k = 2, 2, 4
    n = int(rng.integers(7, 16))
    score = rng.integers(0, 3, size=n).astype(np.float64)  # many exact ties between block sums
    got = O.select_blocks(score, window=window, top_k=top_k, block=block)
    assert got["sel"].tolist() == brute_blocks(score, window, top_k, block)


@pytest.mark.parametrize("length", [1153, 1500, 4099, 9000])
def test_block_size_one_is_the_token_rule(length):
    rng = np.random.default_rng(length)
    score = rng.random(length) ** 4
    score[rng.integers(0, length, 50)] = 0.5  # some exact ties
    np.testing.assert_array_equal(O.select_blocks(score, block=1)["sel"], O.select_tokens(score)["sel"])


def test_constant_scores_take_the_first_blocks():
    n = 5000
    got = O.select_blocks(np.full(n, 16.0 / n))
    np.testing.assert_array_equal(got["sel"], np.concatenate([np.arange(1024), np.arange(n - 128, n)]))


def test_one_heavy_token_brings_its_whole_block():
    n = 20000
    rng = np.random.default_rng(5)
    score = rng.random(n) * 1e-6
    score[3000] = 1.0
    sel = set(O.select_blocks(score)["sel"].tolist())
    assert set(range(2944, 3008)) <= sel  # block 46 = [2944, 3008) holds position 3000


@pytest.mark.parametrize("length", [0, 1, 128, 129, 1152])
def test_short_contexts_select_everything(length):
    np.testing.assert_array_equal(O.select_blocks(np.ones(length))["sel"], np.arange(length))


def test_first_length_past_the_budget_leaves_the_partial_block_out():
    # L = 1153: 1025 positions before the window hold 16 complete blocks and
    # one position (1024) that belongs to no candidate block.
    got = O.select_blocks(np.ones(1153))["sel"]
    np.testing.assert_array_equal(got, np.concatenate([np.arange(1024), np.arange(1025, 1153)]))


@pytest.mark.parametrize("length", [1216, 3000, 70001])
def test_block_selection_invariants(length):
    rng = np.random.default_rng(length + 1)
    score = rng.exponential(size=length)
    got = O.select_blocks(score)
    sel = got["sel"]
    assert sel.shape[0] == 1152 and np.all(np.diff(sel) > 0)
    assert set(range(length - 128, length)) <= set(sel.tolist())
    outside = sel[sel < length - 128]
    nb = (length - 128) // 64
    blocks = np.unique(outside // 64)
    assert blocks.shape[0] == 16 and blocks.max() < nb
    np.testing.assert_array_equal(np.sort(outside), (blocks[:, None] * 64 + np.arange(64)).ravel())
    # every chosen block's sum is at least every other candidate's
    sums = np.array([score[64 * i:64 * i + 64].sum() for i in range(nb)])
    assert sums[blocks].min() >= np.delete(sums, blocks).max()


def test_block_decode_of_short_context_equals_full():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((16, 128))
    k = rng.standard_normal((900, 128))
    v = rng.standard_normal((900, 128))
    r = O.decode_sequence(q, q[None], k, v, selection="block")
    np.testing.assert_allclose(r["o_sparse"][0], r["o_full"], rtol=0, atol=1e-14)


def _fixture_and_brute_pin(select, golden):
    kv = fixture(golden)
    score = np.array([float(x) for x in kv["scores"].split()])
    ok = select(score, window=2, top_k=4, block=2)["sel"].tolist() == [int(x) for x in kv["sel"].split()]
    for seed in range(16):
        rng = np.random.default_rng(100 + seed)
        n = int(rng.integers(7, 16))
        s = rng.integers(0, 3, size=n).astype(np.float64)
        ok = ok and select(s, window=2, top_k=4, block=2)["sel"].tolist() == brute_blocks(s, 2, 4, 2)
    return ok


def test_block_pins_catch_planted_mistakes(golden):
    assert _fixture_and_brute_pin(O.select_blocks, golden)

    def ties_high(score, window, top_k, block):
        n = len(score)
        nb = (n - window) // block
        bs = np.asarray(score[:nb * block]).reshape(nb, block).sum(axis=1)
        top = np.lexsort((-np.arange(nb), -bs))[:top_k // block]
        return {"sel": np.sort(np.concatenate([(top[:, None] * block + np.arange(block)).ravel(),
                                               np.arange(n - window, n)]))}

    def aligned_to_window(score, window, top_k, block):
        n = len(score)
        c = n - window
        nb = c // block
        start = c - nb * block  # blocks end at the window instead of starting at 0
        bs = np.asarray(score[start:c]).reshape(nb, block).sum(axis=1)
        top = np.lexsort((np.arange(nb), -bs))[:top_k // block]
        return {"sel": np.sort(np.concatenate([(start + top[:, None] * block + np.arange(block)).ravel(),
                                               np.arange(c, n)]))}

    def max_pooled(score, window, top_k, block):
        n = len(score)
        nb = (n - window) // block
        bs = np.asarray(score[:nb * block]).reshape(nb, block).max(axis=1)
        top = np.lexsort((np.arange(nb), -bs))[:top_k // block]
        return {"sel": np.sort(np.concatenate([(top[:, None] * block + np.arange(block)).ravel(),
                                               np.arange(n - window, n)]))}

    for wrong in (ties_high, aligned_to_window, max_pooled):
        assert not _fixture_and_brute_pin(wrong, golden), wrong.__name__
