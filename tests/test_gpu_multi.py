"""GPU parity of multi-token decode (each query token a decode step over its
causal prefix, with its own selection) against the oracle."""

import numpy as np
import pytest
import torch

from long_context_kv_hs2_amd import hs2, inputs
from oracle import hs2_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu


def multi_inputs(lengths, n_query, kv, seed, n_s=2):
    d = inputs.make_decode(lengths=lengths, n_sparse=n_s, kv=kv, seed=seed, needles=32)
    rng = np.random.default_rng(seed + 1)
    b = len(lengths)
    d["q_full_m"] = rng.standard_normal((b, n_query, 16, 128), dtype=np.float32)
    d["q_sparse_m"] = rng.standard_normal((n_s, b, n_query, 16, 128), dtype=np.float32)
    return d


def run_multi(d):
    t = parity.to_device(d)
    m = hs2.MultiDecode(t["seq_offsets"], t["k"], t["v"], torch.from_numpy(d["q_full_m"]).cuda(),
                        torch.from_numpy(d["q_sparse_m"]).cuda(), t["k_scale"], t["v_scale"], t["max_context"])
    m()
    torch.cuda.synchronize()
    return m


def check_multi(d, m):
    kv = d["kv"]
    tol = parity.TOL[kv]
    offs = d["seq_offsets"]
    n_query = d["q_full_m"].shape[1]
    o_full, o_sparse = m.o_full.cpu().numpy(), m.o_sparse.cpu().numpy()
    sel, cnt = m.sel_idx.cpu().numpy(), m.sel_count.cpu().numpy()
    worst = 0.0
    for b in range(offs.shape[0] - 1):
        a, e = int(offs[b]), int(offs[b + 1])
        ks = None if d["k_scale"] is None else d["k_scale"][a:e]
        vs = None if d["v_scale"] is None else d["v_scale"][a:e]
        kf, vf = O.decode_kv(d["k"][a:e], kv, ks), O.decode_kv(d["v"][a:e], kv, vs)
        refs = O.decode_multi_sequence(d["q_full_m"][b].astype(np.float64), d["q_sparse_m"][:, b].astype(np.float64),
                                       kf, vf)
        for t, ref in enumerate(refs):
            if ref is None:
                assert cnt[b, t] == 0 and np.all(sel[b, t] == -1) and not o_full[b, t].any()
                assert not o_sparse[:, b, t].any()
                continue
            length = (e - a) - n_query + t + 1
            got = parity.check_selection(sel[b, t], int(cnt[b, t]), length, ref)
            err = parity.max_abs_rel(o_full[b, t], ref["o_full"])
            assert err <= tol, f"o_full b={b} t={t}: {err:.3e}"
            ref_sparse = ref["o_sparse"]
            if not np.array_equal(got, ref["sel"]):
                n = length
                ref_sparse = O.decode_sequence(d["q_full_m"][b, t].astype(np.float64),
                                               d["q_sparse_m"][:, b, t].astype(np.float64), kf[:n], vf[:n],
                                               sel_override=got)["o_sparse"]
            for layer in range(ref_sparse.shape[0]):
                err2 = parity.max_abs_rel(o_sparse[layer, b, t], ref_sparse[layer])
                assert err2 <= tol, f"o_sparse b={b} t={t} layer {layer}: {err2:.3e}"
            worst = max(worst, err, err2)
    return worst


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_multi_token_matches_oracle(kv):
    # 515 (bf16, chunk 256) and 899 (E4M3, chunk 448): the first token's prefix
    # ends on a chunk boundary, so the later tokens' prefixes reach one chunk
    # further than the shared pass deals (their empty partial).
    lengths = [3000, 2, 0, 129, 20000, 1153, 515, 899]
    print(f"case: multi-token decode, T=4, {kv}, lengths {lengths}", flush=True)
    d = multi_inputs(lengths, 4, kv, seed=91)
    print(f"worst {check_multi(d, run_multi(d))}", flush=True)


@pytest.mark.parametrize("n_query", [2, 3])
def test_multi_token_two_and_three_tokens(n_query):
    # The group sizes below four take their own kernel instances.
    lengths = [2000, 1, 515, 7000]
    print(f"case: multi-token decode, T={n_query}, lengths {lengths}", flush=True)
    d = multi_inputs(lengths, n_query, "bf16", seed=94 + n_query)
    check_multi(d, run_multi(d))


def test_multi_token_sixteen_tokens():
    lengths = [5000, 300, 16]
    print(f"case: multi-token decode, T=16, lengths {lengths}", flush=True)
    d = multi_inputs(lengths, 16, "bf16", seed=92)
    check_multi(d, run_multi(d))


@pytest.mark.parametrize("lengths", [[7000, 0, 1500, 40000], [100003] * 16])
def test_one_query_token_is_the_hybrid_block(lengths):
    # T = 1: the virtual batch is the batch itself, so every output equals
    # hs2_decode_block's bit for bit.  16 x 100003 is a bf16 batch of equal
    # lengths with 16 chunks a sequence and ~98 rounds: both passes deal the
    # last tiles to the even-XCD workgroups only, ending on a partial round.
    print(f"case: multi-token decode with T=1 vs the hybrid block, lengths {lengths[:4]} x{len(lengths)}", flush=True)
    d = multi_inputs(lengths, 1, "bf16", seed=93)
    m = run_multi(d)
    t = parity.to_device(d)
    blk = hs2.decode_block(t["seq_offsets"], t["k"], t["v"], torch.from_numpy(d["q_full_m"][:, 0]).cuda(),
                           torch.from_numpy(d["q_sparse_m"][:, :, 0]).contiguous().cuda(), max_context=t["max_context"],
                           with_score=False)
    torch.cuda.synchronize()
    assert torch.equal(m.o_full[:, 0], blk["o_full"])
    assert torch.equal(m.o_sparse[:, :, 0], blk["o_sparse"])
    assert torch.equal(m.sel_idx[:, 0], blk["sel_idx"]) and torch.equal(m.sel_count[:, 0], blk["sel_count"])
