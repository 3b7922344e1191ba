"""GPU parity of the Self-Decoder layers at decode: the sliding-window layer
over a ring buffer (with and without writing the current token's rows) and
the full-attention-only call, against the oracle."""

import math

import numpy as np
import pytest
import torch

from long_context_kv_hs2_amd import hs2, inputs
from oracle import hs2_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu


def make_ring(rng, batch, window, fp8):
    bits = inputs.to_bf16_bits(rng.standard_normal((batch * window, 128), dtype=np.float32))
    if fp8:
        codes, scale = inputs.quantize_e4m3_per_token(bits)
        return codes.reshape(batch, window, 128), scale.reshape(batch, window)
    return bits.reshape(batch, window, 128), None


def dev_rows(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def run_swa_case(lengths, window, fp8, write_new, seed):
    rng = np.random.default_rng(seed)
    batch = len(lengths)
    rk, rks = make_ring(rng, batch, window, fp8)
    rv, rvs = make_ring(rng, batch, window, fp8)
    q = rng.standard_normal((batch, 16, 128), dtype=np.float32)
    kn = kns = vn = vns = None
    if write_new:
        kn, kns = make_ring(rng, batch, 1, fp8)
        vn, vns = make_ring(rng, batch, 1, fp8)
        kn, vn = kn[:, 0], vn[:, 0]
        kns, vns = (kns[:, 0], vns[:, 0]) if fp8 else (None, None)
    t = dict(lengths=torch.tensor(lengths, dtype=torch.int64).cuda(), rk=dev_rows(rk), rv=dev_rows(rv),
             q=torch.from_numpy(q).cuda())
    o = hs2.swa_decode(t["lengths"], t["rk"], t["rv"], t["q"],
                       dev_rows(rks) if fp8 else None, dev_rows(rvs) if fp8 else None,
                       dev_rows(kn) if write_new else None, dev_rows(vn) if write_new else None,
                       dev_rows(kns) if (write_new and fp8) else None, dev_rows(vns) if (write_new and fp8) else None)
    torch.cuda.synchronize()
    got_o = o.cpu().numpy()
    host = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.cpu().numpy()
    got_rk, got_rv = host(t["rk"]), host(t["rv"])
    kv = "fp8_e4m3" if fp8 else "bf16"
    tol = parity.TOL[kv]
    worst = 0.0
    for b, length in enumerate(lengths):
        want_k, want_v = rk[b].copy(), rv[b].copy()
        want_ks = rks[b].copy() if fp8 else None
        want_vs = rvs[b].copy() if fp8 else None
        if write_new and length > 0:
            slot = (length - 1) % window
            want_k[slot], want_v[slot] = kn[b], vn[b]
            if fp8:
                want_ks[slot], want_vs[slot] = kns[b], vns[b]
        np.testing.assert_array_equal(got_rk[b], want_k)  # the current rows, and nothing else, written
        np.testing.assert_array_equal(got_rv[b], want_v)
        if length == 0:
            assert not got_o[b].any()
            continue
        kf = O.decode_kv(want_k, kv, want_ks)
        vf = O.decode_kv(want_v, kv, want_vs)
        ref = O.swa_attention(q[b].astype(np.float64), kf, vf, length, window)
        err = parity.max_abs_rel(got_o[b], ref)
        assert err <= tol, f"seq {b} (L={length}): {err:.3e} > {tol}"
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("write_new", [False, True])
def test_swa_decode_window_128(fp8, write_new):
    lengths = [0, 1, 50, 127, 128, 129, 5000, 1 << 20]
    print(f"case: swa decode, window 128, fp8 {fp8}, write {write_new}", flush=True)
    run_swa_case(lengths, 128, fp8, write_new, seed=11 + 2 * fp8 + write_new)


@pytest.mark.parametrize("window", [1, 100, 200, 300, 640, 1152])
def test_swa_decode_other_windows(window):
    lengths = [window - 1, window, window + 1, 3 * window + 7, 1]
    print(f"case: swa decode, window {window}", flush=True)
    run_swa_case(lengths, window, False, True, seed=window)


def test_swa_decode_large_batch():
    rng = np.random.default_rng(5)
    lengths = rng.integers(0, 400, size=300).tolist()
    print("case: swa decode, batch 300", flush=True)
    run_swa_case(lengths, 128, True, True, seed=5)


def test_swa_decode_empty_batch():
    z = torch.zeros((0, 128, 128), dtype=torch.bfloat16, device="cuda")
    o = hs2.swa_decode(torch.zeros(0, dtype=torch.int64, device="cuda"), z, z.clone(),
                       torch.zeros((0, 16, 128), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert o.shape == (0, 16, 128)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_full_decode_alone(kv):
    # The full-attention-only call runs the same pass as the hybrid block's
    # full layer: equal outputs bit for bit, and the oracle's full attention.
    lengths = [3000, 0, 129, 70000, 5]
    print(f"case: full decode alone, {kv}, lengths {lengths}", flush=True)
    d = inputs.make_decode(lengths=lengths, n_sparse=1, kv=kv, seed=23, needles=10)
    t = parity.to_device(d)
    o = hs2.full_decode(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["k_scale"], t["v_scale"], t["max_context"])
    blk = hs2.decode_block(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], t["k_scale"],
                           t["v_scale"], t["max_context"], with_score=False)
    torch.cuda.synchronize()
    assert torch.equal(o, blk["o_full"])
    got = o.cpu().numpy()
    offs = d["seq_offsets"]
    for b in range(len(lengths)):
        a, e = int(offs[b]), int(offs[b + 1])
        if e == a:
            assert not got[b].any()
            continue
        ks = None if d["k_scale"] is None else d["k_scale"][a:e]
        vs = None if d["v_scale"] is None else d["v_scale"][a:e]
        ref, _ = O.full_attention(d["q_full"][b].astype(np.float64), O.decode_kv(d["k"][a:e], kv, ks),
                                  O.decode_kv(d["v"][a:e], kv, vs))
        assert parity.max_abs_rel(got[b], ref) <= parity.TOL[kv]


def test_full_decode_writes_only_its_partials():
    # Full attention alone keeps no score bounds, statistics or selection
    # state: past the split-K partials (at most B * ceil(max_context / 256)
    # partials of 2080 floats, chunks being at least 256 tokens) the
    # workspace is left as it was.
    lengths = [20000, 3000, 0, 9000]
    print(f"case: full decode workspace use, lengths {lengths}", flush=True)
    d = inputs.make_decode(lengths=lengths, n_sparse=1, seed=29, needles=10)
    t = parity.to_device(d)
    desc = hs2.make_desc(len(lengths), sum(lengths), t["max_context"], 0)
    ws = torch.full((hs2.decode_workspace_bytes(desc),), 0xA5, dtype=torch.uint8, device="cuda")
    o = hs2.full_decode(t["seq_offsets"], t["k"], t["v"], t["q_full"], max_context=t["max_context"], workspace=ws)
    torch.cuda.synchronize()
    partial_bytes = len(lengths) * -(-t["max_context"] // 256) * 2080 * 4
    start = -(-partial_bytes // 256) * 256
    rest = ws[start:].cpu().numpy()
    assert rest.size > 0 and np.all(rest == 0xA5), f"{int((rest != 0xA5).sum())} bytes written past the partials"
    blk = hs2.decode_block(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"],
                           max_context=t["max_context"], with_score=False)
    torch.cuda.synchronize()
    assert torch.equal(o, blk["o_full"])
