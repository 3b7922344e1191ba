"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one DecodeBlock call, no score output), every sequence
against the oracle (one by one).  A second call with the score output must
give bitwise the same results, and its scores are checked as a diagnostic."""

import sys

import numpy as np
import pytest
import torch

from long_context_kv_hs2_amd import hs2, inputs
from oracle import hs2_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_workload(d, seqs):
    t = parity.to_device(d)
    blk = hs2.DecodeBlock(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], t["k_scale"],
                          t["v_scale"], t["max_context"], with_score=False)
    blk()
    torch.cuda.synchronize()
    bench_out = {k: (v.clone() if v is not None else None) for k, v in blk.outputs().items()}
    scored = hs2.DecodeBlock(t["seq_offsets"], t["k"], t["v"], t["q_full"], t["q_sparse"], t["k_scale"],
                             t["v_scale"], t["max_context"], with_score=True)
    scored()
    torch.cuda.synchronize()
    out = scored.outputs()
    for key in ("o_full", "o_sparse", "sel_idx", "sel_count"):
        assert torch.equal(bench_out[key], out[key]), f"{key} differs with the score output on"
    del t, blk
    w = parity.check_decode(d, out, seqs=seqs)
    torch.cuda.empty_cache()
    return w, out


def test_workload2_b32_ctx128k_bf16():
    say("case: workload 2 (B=32, 131072, bf16); oracle on every sequence")
    d = inputs.make_decode(2)
    w, out = run_workload(d, None)
    counts = out["sel_count"].cpu().numpy()
    assert np.all(counts == 1152)
    say(f"worst {w}")


def test_workload3_b4_ctx1m_fp8():
    say("case: workload 3 (B=4, 1048576, fp8 e4m3); oracle on every sequence")
    d = inputs.make_decode(3)
    w, _ = run_workload(d, None)
    say(f"worst {w}")


def test_workload4_b64_ragged_agent_mix():
    d = inputs.make_decode(4)
    lens = np.diff(d["seq_offsets"])
    say(f"case: workload 4 (B=64 ragged, N={lens.sum()}, L {lens.min()}..{lens.max()}); oracle on every sequence")
    w, _ = run_workload(d, None)
    say(f"worst {w}")


def test_workload5_fp8_bridge_then_decode():
    # The bridge written as the FP8 cache (E4M3 + per-token scales), then the
    # decode over it for one bridged layer (8 x 32768 packed).
    say("case: workload 5 FP8 bridge (262144 x 4096 -> 3 x (K, V) E4M3), sampled rows, then decode")
    br = inputs.make_bridge()
    dev = "cuda"
    h = torch.from_numpy(br["h"].view(np.int16)).view(torch.bfloat16).to(dev)
    wk = [torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev) for w in br["w_k"]]
    wv = [torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev) for w in br["w_v"]]
    k_c, k_s, v_c, v_s = hs2.bridge_kv_fp8(h, wk, wv)
    torch.cuda.synchronize()
    del h
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(262144, 1500, replace=False), np.arange(64),
                                     262144 - 1 - np.arange(64)]))
    for l in range(3):
        for name, w_bits, c, s in (("K", br["w_k"][l], k_c[l], k_s[l]), ("V", br["w_v"][l], v_c[l], v_s[l])):
            same, rel = parity.check_bridge_fp8(br["h"], w_bits, c.cpu().numpy(), s.cpu().numpy(), rows)
            say(f"fp8 bridge layer {l} {name}: {same:.5f} codes equal, scales within {rel:.2e}")
    del br
    queries = inputs.make_bridge_queries()
    offs = np.arange(9, dtype=np.int64) * 32768
    for l in range(3):
        d = dict(seq_offsets=offs, k=k_c[l].cpu().numpy(), v=v_c[l].cpu().numpy(), k_scale=k_s[l].cpu().numpy(),
                 v_scale=v_s[l].cpu().numpy(), q_full=queries[l][0], q_sparse=queries[l][1], kv="fp8_e4m3")
        say(f"case: workload 5 decode over the FP8 bridged cache, layer {l}; oracle on every sequence")
        w, _ = run_workload(d, None)
        say(f"worst {w}")


def test_workload5_bridge_then_decode():
    say("case: workload 5 bridge (262144 x 4096 -> 3 x (K, V)), sampled rows")
    br = inputs.make_bridge()
    dev = "cuda"
    h = torch.from_numpy(br["h"].view(np.int16)).view(torch.bfloat16).to(dev)
    wk = [torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev) for w in br["w_k"]]
    wv = [torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev) for w in br["w_v"]]
    k_out, v_out = hs2.bridge_kv(h, wk, wv)
    torch.cuda.synchronize()
    del h
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(262144, 1500, replace=False), np.arange(128),
                                     262144 - 1 - np.arange(128)]))
    for l in range(3):
        for name, w_bits, out_t in (("K", br["w_k"][l], k_out[l]), ("V", br["w_v"][l], v_out[l])):
            got = out_t.view(torch.int16).cpu().numpy().view(np.uint16)
            worst, frac1 = parity.check_bridge(br["h"], w_bits, got, rows)
            say(f"bridge layer {l} {name}: worst {worst} ulp, {frac1:.5f} within 1 ulp")
    del br
    # decode per bridged layer over the GPU-built cache (8 x 32768 packed)
    queries = inputs.make_bridge_queries()
    offs = np.arange(9, dtype=np.int64) * 32768
    for l in range(3):
        kb = k_out[l].view(torch.int16).cpu().numpy().view(np.uint16)
        vb = v_out[l].view(torch.int16).cpu().numpy().view(np.uint16)
        d = dict(seq_offsets=offs, k=kb, v=vb, k_scale=None, v_scale=None, q_full=queries[l][0],
                 q_sparse=queries[l][1], kv="bf16")
        say(f"case: workload 5 decode, bridged layer {l}; oracle on every sequence")
        w, _ = run_workload(d, None)
        say(f"worst {w}")
