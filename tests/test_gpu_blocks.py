"""GPU parity of the gen-1 (block-level) selection, the ablation comparator:
exact on given scores, and the hybrid block with gen-1 selection against the
oracle."""

import numpy as np
import pytest
import torch

from long_context_kv_hs2_amd import hs2, inputs
from oracle import hs2_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu


def run_block_select(lengths, scores):
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    t_offs = torch.from_numpy(offs).cuda()
    t_score = torch.from_numpy(scores.astype(np.float32)).cuda()
    sel, cnt = hs2.block_select(t_offs, t_score, len(lengths), int(max(lengths)) if len(lengths) else 0)
    torch.cuda.synchronize()
    return offs, sel.cpu().numpy(), cnt.cpu().numpy()


LENGTHS = [0, 5, 1152, 1153, 1216, 1217, 5000, 70001, 131072]


@pytest.mark.parametrize("kind", ["integers", "constant", "descending"])
def test_block_select_exact_on_given_scores(kind):
    # Scores whose block sums are exact in fp32 (small integers, or equal
    # powers of two), with heavy ties: the list must match bit for bit.
    print(f"case: block select, {kind} scores, lengths {LENGTHS}", flush=True)
    rng = np.random.default_rng(3)
    n = sum(LENGTHS)
    if kind == "integers":
        scores = rng.integers(0, 4, size=n).astype(np.float32)
    elif kind == "constant":
        scores = np.full(n, 0.25, dtype=np.float32)
    else:
        scores = np.concatenate([np.arange(l, 0, -1) for l in LENGTHS]).astype(np.float32) if n else np.zeros(0)
    offs, sel, cnt = run_block_select(LENGTHS, scores)
    for b, length in enumerate(LENGTHS):
        ref = O.select_blocks(scores[offs[b]:offs[b + 1]].astype(np.float64))
        assert cnt[b] == min(length, 1152)
        np.testing.assert_array_equal(sel[b, :cnt[b]], ref["sel"], err_msg=f"{kind} L={length}")
        assert np.all(sel[b, cnt[b]:] == -1)


def test_block_select_random_scores_outside_band():
    lengths = [3000, 131072, 40000, 1048576]
    print(f"case: block select, exponential scores, lengths {lengths}", flush=True)
    rng = np.random.default_rng(4)
    scores = (rng.exponential(size=sum(lengths)) * 1e-5).astype(np.float32)
    offs, sel, cnt = run_block_select(lengths, scores)
    for b, length in enumerate(lengths):
        ref = O.select_blocks(scores[offs[b]:offs[b + 1]].astype(np.float64))
        parity.check_selection(sel[b], int(cnt[b]), length, ref)


def test_block_select_empty_batch_and_zero_tokens():
    offs, sel, cnt = run_block_select([0, 0, 0], np.zeros(0, dtype=np.float32))
    assert np.all(cnt == 0) and np.all(sel == -1)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_hybrid_block_with_block_selection(kv):
    lengths = [300, 1500, 4000, 20000, 0, 70000]
    print(f"case: gen-1 hybrid block, {kv}, lengths {lengths}", flush=True)
    d = inputs.make_decode(lengths=lengths, n_sparse=3, kv=kv, seed=17, needles=40)
    t = parity.to_device(d)
    blk = hs2.BlockSelectDecode(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], t["k_scale"],
                                t["v_scale"], t["max_context"])
    blk()
    torch.cuda.synchronize()
    w = parity.check_decode(d, blk.outputs(), selection="block")
    print(f"worst {w}", flush=True)


def run_gen1(d):
    t = parity.to_device(d)
    g1 = hs2.DecodeBlock(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], t["k_scale"], t["v_scale"],
                         t["max_context"], selection="block")
    g1()
    torch.cuda.synchronize()
    return t, g1


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_gen1_call_from_tile_sums(kv):
    # hs2_decode_block_gen1 (block sums from the full pass's per-tile head
    # sums, no per-token scores) against the oracle, and against the
    # three-call route through per-token scores on the same inputs: the full
    # layer bit for bit (same arithmetic, same merge), the lists equal away
    # from near-ties, and the sparse outputs bit for bit where the lists are.
    lengths = [300, 1152, 1153, 1216, 1217, 1280, 1500, 4000, 20000, 0, 70000, 5000]
    print(f"case: gen-1 call from tile sums, {kv}, lengths {lengths}", flush=True)
    d = inputs.make_decode(lengths=lengths, n_sparse=3, kv=kv, seed=19, needles=40)
    t, g1 = run_gen1(d)
    w = parity.check_decode(d, g1.outputs(), selection="block")
    print(f"worst {w}", flush=True)
    blk = hs2.BlockSelectDecode(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], t["k_scale"],
                                t["v_scale"], t["max_context"])
    blk()
    torch.cuda.synchronize()
    assert torch.equal(g1.o_full, blk.o_full)
    assert torch.equal(g1.sel_count, blk.sel_count)
    same = 0
    for b in range(len(lengths)):
        if torch.equal(g1.sel_idx[b], blk.sel_idx[b]):
            same += 1
            assert torch.equal(g1.o_sparse[:, b], blk.o_sparse[:, b])
    assert same >= len(lengths) - 1, f"only {same} of {len(lengths)} lists agree"


@pytest.mark.parametrize("workload", [2, 3, 4])
def test_gen1_call_full_size(workload):
    # The gen-1 line the benchmark times, at the full workload sizes, every
    # sequence against the oracle's block rule.
    print(f"case: gen-1 call, workload {workload}; oracle on every sequence", flush=True)
    d = inputs.make_decode(workload)
    _, g1 = run_gen1(d)
    out = {k: (v.clone() if v is not None else None) for k, v in g1.outputs().items()}
    g1()  # a second call on the same workspace gives the same results
    torch.cuda.synchronize()
    for key in ("o_full", "o_sparse", "sel_idx", "sel_count"):
        assert torch.equal(out[key], g1.outputs()[key]), f"{key} differs on the second call"
    w = parity.check_decode(d, out, selection="block")
    print(f"worst {w}", flush=True)


def test_block_selection_differs_from_token_selection():
    # On a needle workload the two rules pick different lists (the ablation's
    # point); both are checked against their own oracle above.
    d = inputs.make_decode(lengths=[20000], n_sparse=1, seed=18, needles=40)
    t = parity.to_device(d)
    blk = hs2.BlockSelectDecode(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], None, None,
                                t["max_context"])
    blk()
    tok = hs2.decode_block(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], max_context=t["max_context"])
    torch.cuda.synchronize()
    a = set(blk.sel_idx[0].cpu().numpy().tolist())
    b = set(tok["sel_idx"][0].cpu().numpy().tolist())
    assert len(a ^ b) > 0
    assert torch.equal(blk.o_full, tok["o_full"])  # the full layer is the same call


def test_block_select_past_256_candidates():
    # Over 1M tokens a thread ranks several 16-block groups.  Here thread 0's
    # four groups (0, 1024, 2048, 3072) hold the largest block sums and groups
    # 1..15 the next ones, so 19 groups reach the threshold: 304 candidates,
    # the workgroup-wide sort.  Block sums are exact in fp32.
    length = 4 * 1024 * 1024 + 1000
    print(f"case: block select, {length} tokens, 304 candidates", flush=True)
    score = np.zeros(length, dtype=np.float32)
    for g in (0, 1024, 2048, 3072):
        score[g * 1024:(g + 1) * 1024] = 1000.0 / 64
    score[1024:16 * 1024] = 500.0 / 64
    offs, sel, cnt = run_block_select([length], score)
    ref = O.select_blocks(score.astype(np.float64))
    assert cnt[0] == 1152
    np.testing.assert_array_equal(sel[0], ref["sel"])
