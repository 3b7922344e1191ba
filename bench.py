"""Benchmark: hybrid-block decode tokens/s on one MI355X.

A step is one hs2_decode_block call over one batch: the full-attention layer
over every context token, the per-token score and the token selection, and
the sparse layers over the selected rows.  Inputs are resident in HBM before
the timed region.  Default workload: 32 sequences x 131072 tokens, bf16 MQA
cache (16 query heads, head_dim 128), window 128 + top-1024, 4 sparse layers;
the same line then carries the metric's 1M-token half (4 sequences x 1048576
tokens, E4M3 cache with per-token scales), timed the same way, as
``roofline_ctx1m_fp8``.

The roofline object covers the full layer and its score (K1 + K1b): the
split-K partial pass and the launch that merges it and runs the selection's
first pass over the score bounds.  Algorithmic bytes per launch = N x 512 B
(each K and V row read once; 264 B with E4M3 and its two scales) + B x 16 KiB
(the query and the output), divided by the two kernels' mean duration per
step, measured live with HIP events recorded by the library on the launch
stream during the timed steps.  ``k1_alone`` gives the partial pass by
itself.  ``traffic`` is the two kernels' HBM bytes per launch from the
rocprofv3 FETCH_SIZE/WRITE_SIZE runs summarised under profiles/ (scaled by a
1 GiB copy), or null when their sources changed since they were taken.

The cpu_baseline leg times the fp64 oracle on a bounded sample of the same
workload (whole sequences, one after another, until about 15 s have passed).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 2|3|4|5] [--selection token|block|block-scores]

``--tokens T`` (T > 1) times multi-token decode on the same cache: T query
tokens per sequence, each over its causal prefix with its own selection.
``--part self-decoder`` times the model's front half at decode on the same
batch: its one full-attention layer and 24 sliding-window layers (window 128).
``--selection block`` times the same workload through the gen-1 (block-level)
selection instead, the comparator of the pages' ablation: hs2_decode_block_gen1,
whose full pass keeps per-tile head sums of its weights and whose merge
launch forms the block sums from them.  ``--selection block-scores`` times the
three-call route through every per-token score (hs2_full_decode_score,
hs2_block_select, then the sparse layers).
Each line also carries per-launch percentiles, a "cold" full-pass time (after
1 GiB of writes has evicted the caches), the clock levels sampled during the
timed steps, and the device.

Workload 5 times the KV-Bridging projection (262144 x 4096 hidden states into
3 layers' K and V, one bf16 MFMA GEMM) and then each bridged layer's decode
step (8 sequences x 32768 tokens over the bridged cache); its roofline is the
GEMM's against the dense bf16 MFMA peak, and its value the decode tokens/s
through the 3 bridged hybrid blocks.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = {2: "profiles/full_partial_b32_ctx128k_bf16_hbm_traffic.md",
                   3: "profiles/full_partial_b4_ctx1m_fp8_hbm_traffic.md"}
# the kernel and what sets its launch (chunk size, grid)
KERNEL_SOURCES = ("long_context_kv_hs2_amd/csrc/full_decode.hip", "long_context_kv_hs2_amd/csrc/hs2_device.h",
                  "long_context_kv_hs2_amd/csrc/hs2_internal.h", "long_context_kv_hs2_amd/csrc/hs2_api.hip",
                  "long_context_kv_hs2_amd/csrc/topk_select.hip", "long_context_kv_hs2_amd/csrc/merge.h")
METRIC = "hybrid-block decode tokens/s at 128K/1M ctx; achieved HBM GB/s vs peak"
WORKLOADS = {2: "b32_ctx128k_bf16", 3: "b4_ctx1m_fp8", 4: "b64_ragged_2k_256k_bf16",
             5: "bridge_262144x4096_3layers_then_b8x32k_decode"}
MFMA_BF16_PEAK_TFLOPS = 2500.0
KV_ROW_BYTES = {"bf16": 2 * 2 * 128, "fp8_e4m3": 2 * 128 + 2 * 4}  # K+V (+ per-token scales)


def measured_traffic(workload):
    """HBM bytes per launch of the full-attention pass from the committed
    rocprofv3 counter summary, or None when there is none for this workload or
    the kernel source changed since the counters were taken."""
    import hashlib

    path = TRAFFIC_PROFILE.get(workload)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    text = open(os.path.join(ROOT, path), encoding="utf-8").read()
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
    sha = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in KERNEL_SOURCES)).hexdigest()
    if fields.get("source_sha256", "").strip() != sha:
        return None
    return int(fields["traffic_bytes_per_launch"])


def pct(x):
    """Mean, p10, median and p90 (ms) of per-call durations."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return None
    return {"mean": round(float(x.mean()), 5), "p10": round(float(np.percentile(x, 10)), 5),
            "median": round(float(np.median(x)), 5), "p90": round(float(np.percentile(x, 90)), 5), "n": int(x.size)}


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "clock_khz": getattr(p, "clock_rate", None), "hip": torch.version.hip, "torch": torch.__version__}


def cold_full_pass(torch, hs2, step, dev, reps=5):
    """The full pass right after 1 GiB of writes (more than the 256 MB
    Infinity Cache and the L2s hold), so its K/V reads start cold."""
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    k1, both = [], []
    for i in range(reps):
        scratch.fill_(i + 1)
        torch.cuda.synchronize()
        hs2.stage_timing(True, full_pass_only=True)
        step()
        torch.cuda.synchronize()
        hs2.stage_timing(False)
        calls = hs2.stage_timing_read_calls()
        k1.extend(calls[:, 0].tolist())
        both.extend((calls[:, 0] + calls[:, 1]).tolist())
    del scratch
    return {"k1": pct(k1), "k1_k1b": pct(both)}


def cpu_baseline(d, budget_s=15.0):
    """Time the oracle on whole sequences of this workload until `budget_s`."""
    from oracle import hs2_oracle as O  # the oracle is only ever run here, for the baseline

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    offs = d["seq_offsets"]
    done, tokens, t0 = 0, 0, time.perf_counter()
    for b in range(offs.shape[0] - 1):
        a, e = int(offs[b]), int(offs[b + 1])
        ks = None if d["k_scale"] is None else d["k_scale"][a:e]
        vs = None if d["v_scale"] is None else d["v_scale"][a:e]
        k = O.decode_kv(d["k"][a:e], d["kv"], ks)
        v = O.decode_kv(d["v"][a:e], d["kv"], vs)
        O.decode_sequence(d["q_full"][b].astype(np.float64), d["q_sparse"][:, b].astype(np.float64), k, v)
        done += 1
        tokens += e - a
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {offs.shape[0] - 1} sequences ({tokens} context tokens), fp64 numpy, "
                      f"one decode step each, {dt:.1f} s"}


def bench_bridge(args, torch, hs2, inputs, dev):
    br = inputs.make_bridge()
    t_rows, d_model = br["h"].shape
    bits = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    h = bits(br["h"])
    wk = [bits(w) for w in br["w_k"]]
    wv = [bits(w) for w in br["w_v"]]
    n_l = len(wk)
    k_out = [torch.empty((t_rows, 128), dtype=torch.bfloat16, device=dev) for _ in range(n_l)]
    v_out = [torch.empty((t_rows, 128), dtype=torch.bfloat16, device=dev) for _ in range(n_l)]
    ws = torch.empty(hs2.bridge_workspace_bytes(t_rows, d_model, n_l), dtype=torch.uint8, device=dev)
    queries = inputs.make_bridge_queries()
    batch = queries[0][0].shape[0]
    offs = torch.arange(batch + 1, dtype=torch.int64, device=dev) * (t_rows // batch)
    blocks = [hs2.DecodeBlock(offs, k_out[l], v_out[l], torch.from_numpy(queries[l][0]).to(dev),
                              torch.from_numpy(queries[l][1]).to(dev), None, None, t_rows // batch)
              for l in range(n_l)]

    # The weights are packed once per weight set (outside the timed region);
    # each timed call is the GEMM alone.
    packed = hs2.bridge_pack_weights(wk, wv)

    def bridge():
        hs2.bridge_kv_packed(h, packed, n_l, k_out, v_out)

    settle(args, torch, bridge)
    for _ in range(args.warmup):
        bridge()
        for blk in blocks:
            blk()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        bridge()
    e1.record()
    torch.cuda.synchronize()
    bridge_ms = e0.elapsed_time(e1) / args.steps
    # The per-call entry point, which packs the weights into its workspace
    # every time (diagnostic).
    e0.record()
    for _ in range(args.steps):
        hs2.bridge_kv(h, wk, wv, k_out, v_out, ws)
    e1.record()
    torch.cuda.synchronize()
    bridge_per_call_ms = e0.elapsed_time(e1) / args.steps
    # The same projection written as the E4M3 cache with per-token scales
    # (diagnostic line: its own buffers, timed the same way).
    k8 = [torch.empty((t_rows, 128), dtype=torch.uint8, device=dev) for _ in range(n_l)]
    v8 = [torch.empty((t_rows, 128), dtype=torch.uint8, device=dev) for _ in range(n_l)]
    ks8 = [torch.empty((t_rows,), dtype=torch.float32, device=dev) for _ in range(n_l)]
    vs8 = [torch.empty((t_rows,), dtype=torch.float32, device=dev) for _ in range(n_l)]

    def bridge_fp8():
        hs2.bridge_kv_packed(h, packed, n_l, k8, v8, ks8, vs8, fp8=True)

    for _ in range(min(args.warmup, 5)):
        bridge_fp8()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        bridge_fp8()
    e1.record()
    torch.cuda.synchronize()
    bridge_fp8_ms = e0.elapsed_time(e1) / args.steps
    blocks8 = [hs2.DecodeBlock(offs, k8[l], v8[l], torch.from_numpy(queries[l][0]).to(dev),
                               torch.from_numpy(queries[l][1]).to(dev), ks8[l], vs8[l], t_rows // batch)
               for l in range(n_l)]
    for _ in range(min(args.warmup, 5)):
        for blk in blocks8:
            blk()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for blk in blocks8:
            blk()
    torch.cuda.synchronize()
    decode_fp8_ms = (time.perf_counter() - t0) / args.steps * 1e3
    # Decode-time bridging: the current token's hidden row of each of the
    # batch's sequences projected into the 3 bridged layers' caches.
    h_step = h[:batch].contiguous()
    aws = torch.empty(hs2.load().hs2_bridge_append_workspace_bytes(batch, d_model, 128, n_l), dtype=torch.uint8,
                      device=dev)

    def time_append(kc, vc, ksc, vsc):
        for _ in range(5):
            hs2.bridge_append(offs, h_step, wk, wv, kc, vc, ksc, vsc, aws)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            hs2.bridge_append(offs, h_step, wk, wv, kc, vc, ksc, vsc, aws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    append_fp8_ms = time_append(k8, v8, ks8, vs8)
    del blocks8, k8, v8, ks8, vs8
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for blk in blocks:
            blk()
    torch.cuda.synchronize()
    decode_s = (time.perf_counter() - t0) / args.steps
    append_ms = time_append(k_out, v_out, None, None)
    # Per-stage breakdown (diagnostic), from extra untimed steps.
    hs2.stage_timing(True)
    hs2.stage_timing_read()
    for _ in range(min(args.steps, 20)):
        for blk in blocks:
            blk()
    torch.cuda.synchronize()
    hs2.stage_timing(False)
    stages, _ = hs2.stage_timing_read()
    flops = 2.0 * t_rows * d_model * 2 * n_l * 128
    tflops = flops / (bridge_ms * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": batch / decode_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": decode_s * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOADS[5], "tokens": t_rows, "d_model": d_model, "bridged_layers": n_l,
                   "decode_batch": batch, "context_per_sequence": t_rows // batch, "n_sparse_layers": 4},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "bridge_gemm_kernel (hs2_bridge_kv_packed)", "alg_flops_per_launch": flops,
                     "mean_launch_ms": bridge_ms},
        "device": device_info(torch),
        "bridge_ms": bridge_ms,
        "bridge_fp8_ms": bridge_fp8_ms,
        "bridge_per_call_packing_ms": bridge_per_call_ms,
        "fp8_cache_decode_ms_per_step": decode_fp8_ms,
        "decode_bridge_append_ms": {"bf16": append_ms, "fp8_e4m3": append_fp8_ms, "rows": batch,
                                    "weight_bytes": 2 * n_l * d_model * 128 * 2},
        "decode_stages_ms_per_layer": {k: round(v, 5) for k, v in stages.items()},
    }


def bench_self_decoder(args, torch, hs2, inputs, dev):
    """The Self-Decoder's attention at decode on a workload's batch: its one
    full-attention layer over the whole context (hs2_full_decode) and 24
    sliding-window layers (window 128, one ring per layer; hs2_swa_decode,
    each also writing the current token's rows), per decode step."""
    d = inputs.make_decode(args.workload)
    kv = d["kv"]
    offs = torch.from_numpy(d["seq_offsets"]).to(dev)
    if kv == "bf16":
        k = torch.from_numpy(d["k"].view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(d["v"].view(np.int16)).view(torch.bfloat16).to(dev)
        ks = vs = None
    else:
        k, v = torch.from_numpy(d["k"]).to(dev), torch.from_numpy(d["v"]).to(dev)
        ks, vs = torch.from_numpy(d["k_scale"]).to(dev), torch.from_numpy(d["v_scale"]).to(dev)
    q_full = torch.from_numpy(d["q_full"]).to(dev)
    lens = np.diff(d["seq_offsets"])
    batch, n_tokens, n_swa, window = int(lens.shape[0]), int(lens.sum()), 24, 128
    desc = hs2.make_desc(batch, n_tokens, int(lens.max()), 0, hs2.kv_dtype_of(k))
    ws = torch.empty(hs2.decode_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    o_full = torch.empty((batch, 16, 128), dtype=torch.float32, device=dev)
    g = torch.Generator(device="cpu").manual_seed(7)
    rings = [(torch.randn((batch, window, 128), generator=g).to(torch.bfloat16).to(dev),
              torch.randn((batch, window, 128), generator=g).to(torch.bfloat16).to(dev)) for _ in range(n_swa)]
    new_k = torch.randn((batch, 128), generator=g).to(torch.bfloat16).to(dev)
    new_v = torch.randn((batch, 128), generator=g).to(torch.bfloat16).to(dev)
    q_swa = torch.randn((n_swa, batch, 16, 128), generator=g).to(dev)
    lengths = torch.from_numpy(lens.astype(np.int64)).to(dev)
    o_swa = torch.empty((batch, 16, 128), dtype=torch.float32, device=dev)

    def step(marks=None):
        hs2.full_decode(offs, k, v, q_full, ks, vs, int(lens.max()), o_full, ws)
        if marks:
            marks[0].record()
        for layer in range(n_swa):
            hs2.swa_decode(lengths, rings[layer][0], rings[layer][1], q_swa[layer], k_new=new_k, v_new=new_v,
                           o=o_swa)
        if marks:
            marks[1].record()

    settle(args, torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hs2.stage_timing(True, full_pass_only=True)
    hs2.stage_timing_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    hs2.stage_timing(False)
    k1 = hs2.stage_timing_read_calls()[:, 0]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    swa_ms = []
    for _ in range(min(args.steps, 20)):
        step(marks)
        torch.cuda.synchronize()
        swa_ms.append(marks[0].elapsed_time(marks[1]) / n_swa)
    alg_bytes = n_tokens * KV_ROW_BYTES[kv] + batch * 16 * 128 * 4
    k1_ms = float(k1.mean())
    achieved = alg_bytes / (k1_ms * 1e-3) / 1e9
    return {
        "metric": "self-decoder attention tokens/s (1 full-attention + 24 sliding-window layers per step)",
        "value": batch * args.steps / dt, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dt * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if kv == "bf16" else "fp8_e4m3", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload] + "_self_decoder", "batch": batch, "context_tokens": n_tokens,
                   "full_layers": 1, "swa_layers": n_swa, "swa_window": window, "swa_kv": "bf16"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "full_partial_kernel (hs2_full_decode)", "alg_bytes_per_launch": alg_bytes,
                     "mean_launch_ms": k1_ms, "launch_ms": pct(k1)},
        "swa_layer_ms": pct(swa_ms),
        "swa_alg_bytes_per_layer": batch * window * 2 * 128 * 2 + batch * 2 * 16 * 128 * 4,
        "device": device_info(torch),
    }


def bench_multi(args, torch, hs2, inputs, dev):
    """Multi-token decode on a workload's cache: T query tokens per sequence,
    each a decode step over its causal prefix with its own selection."""
    d = inputs.make_decode(args.workload)
    kv = d["kv"]
    offs = torch.from_numpy(d["seq_offsets"]).to(dev)
    if kv == "bf16":
        k = torch.from_numpy(d["k"].view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(d["v"].view(np.int16)).view(torch.bfloat16).to(dev)
        ks = vs = None
    else:
        k, v = torch.from_numpy(d["k"]).to(dev), torch.from_numpy(d["v"]).to(dev)
        ks, vs = torch.from_numpy(d["k_scale"]).to(dev), torch.from_numpy(d["v_scale"]).to(dev)
    lens = np.diff(d["seq_offsets"])
    batch, n_tokens, t_q = int(lens.shape[0]), int(lens.sum()), args.tokens
    n_s = d["q_sparse"].shape[0]
    g = torch.Generator(device="cpu").manual_seed(11)
    q_full = torch.randn((batch, t_q, 16, 128), generator=g).to(dev)
    q_sparse = torch.randn((n_s, batch, t_q, 16, 128), generator=g).to(dev)
    step = hs2.MultiDecode(offs, k, v, q_full, q_sparse, ks, vs, int(lens.max()))
    settle(args, torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hs2.stage_timing(True, full_pass_only=True)
    hs2.stage_timing_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    hs2.stage_timing(False)
    k1 = hs2.stage_timing_read_calls()[:, 0]
    hs2.stage_timing(True)
    for _ in range(min(args.steps, 20)):
        step()
    torch.cuda.synchronize()
    hs2.stage_timing(False)
    calls = hs2.stage_timing_read_calls()
    stage_pct = {name: pct(calls[:, i]) for i, name in enumerate(hs2.STAGE_NAMES)}
    # algorithmic bytes: every K/V row once for all T tokens (a multi-query pass
    # would read no more), plus the T tokens' queries
    alg_bytes = n_tokens * KV_ROW_BYTES[kv] + batch * t_q * 16 * 128 * 4
    k1_ms = float(k1.mean())
    achieved = alg_bytes / (k1_ms * 1e-3) / 1e9
    return {
        "metric": METRIC + " (multi-token step)", "value": batch * t_q * args.steps / dt, "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if kv == "bf16" else "fp8_e4m3", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload] + f"_multi{t_q}", "batch": batch, "query_tokens": t_q,
                   "context_tokens": n_tokens, "kv_cache": kv, "n_sparse_layers": n_s},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "full_multi_kernel (the B x T causal prefixes, each K/V row read once per group of 4 tokens)", "alg_bytes_per_launch": alg_bytes,
                     "mean_launch_ms": k1_ms, "launch_ms": pct(k1)},
        "stages_ms_percentiles": stage_pct,
        "device": device_info(torch),
    }


def load_cache(torch, d, dev):
    """Device K/V (and scales) of a decode batch from the input generator."""
    if d["kv"] == "bf16":
        k = torch.from_numpy(d["k"].view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(d["v"].view(np.int16)).view(torch.bfloat16).to(dev)
        return k, v, None, None
    return (torch.from_numpy(d["k"]).to(dev), torch.from_numpy(d["v"]).to(dev),
            torch.from_numpy(d["k_scale"]).to(dev), torch.from_numpy(d["v_scale"]).to(dev))


def clock_levels():
    """The active shader, memory and fabric clock levels (the entries marked
    '*' in the driver's pp_dpm_* tables), or None where not readable."""
    import glob

    out = {}
    for name in ("sclk", "mclk", "fclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{name}")):
            try:
                text = open(path, encoding="utf-8").read()
            except OSError:
                continue
            act = [ln.split(":", 1)[1].strip().rstrip("*").strip() for ln in text.splitlines() if ln.endswith("*")]
            if act:
                out[name] = act[0]
                break
    return out or None


def settle(args, torch, step):
    """Untimed steps for ``--settle-ms`` of wall time before the warmup steps:
    after the host has kept the GPU idle (input generation, the CPU
    baseline), the shader clock starts low and takes longer than a few short
    warmup steps to rise (1.4 GHz against 2.1 GHz measured after 5 steps of
    the default line), which slows the E4M3 pass by ~15%; the timed steps
    should see the clocks a decode loop runs at.  Returns the steps run."""
    n = 0
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def hybrid_block_line(args, torch, hs2, d, dev, workload, selection="token", with_cpu=True):
    """Time hs2_decode_block (or the gen-1 line) on one decode batch; returns
    the JSON fields of its line."""
    kv = d["kv"]
    offs_t = torch.from_numpy(d["seq_offsets"]).to(dev)
    k, v, ks, vs = load_cache(torch, d, dev)
    q_full = torch.from_numpy(d["q_full"]).to(dev)
    q_sparse = torch.from_numpy(d["q_sparse"]).to(dev)
    lens = np.diff(d["seq_offsets"])
    batch, n_tokens = int(lens.shape[0]), int(lens.sum())
    if selection == "block-scores":
        blk = hs2.BlockSelectDecode(offs_t, k, v, q_full, q_sparse, ks, vs, int(lens.max()))
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    else:
        blk = hs2.DecodeBlock(offs_t, k, v, q_full, q_sparse, ks, vs, int(lens.max()), with_score=False,
                              selection=selection)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    settle_steps = settle(args, torch, blk)
    for _ in range(args.warmup):
        blk()
    torch.cuda.synchronize()
    # Timed region: HIP events around the full pass and its merge (the
    # roofline's kernels) only; every extra marker would add ~1.5 us a step.
    hs2.stage_timing(True, full_pass_only=True)
    hs2.stage_timing_read()  # clear
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        blk()
    clocks = clock_levels()  # sampled while the timed steps run
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    hs2.stage_timing(False)
    calls = hs2.stage_timing_read_calls()
    k1_calls, k1b_calls = calls[:, 0], calls[:, 1]
    n_rec = int(k1_calls.shape[0])
    # Per-stage breakdown (diagnostic), from extra untimed steps.
    hs2.stage_timing(True)
    extra = []
    for _ in range(min(args.steps, 20)):
        if selection == "block-scores":
            blk(marks)
            torch.cuda.synchronize()
            extra.append((marks[0].elapsed_time(marks[1]), marks[1].elapsed_time(marks[2])))
        else:
            blk()
    torch.cuda.synchronize()
    hs2.stage_timing(False)
    calls = hs2.stage_timing_read_calls()
    stage_pct = {name: pct(calls[:, i]) for i, name in enumerate(hs2.STAGE_NAMES)}
    stages = {name: (stage_pct[name] or {}).get("mean", 0.0) for name in hs2.STAGE_NAMES}
    if selection == "block-scores":
        # hs2_full_decode_score records partial pass, merge and score pass; the
        # block selection and the sparse layers are separate calls
        stage_pct = {"full_partial": stage_pct["full_partial"], "full_merge": stage_pct["full_merge"],
                     "score_pass": stage_pct["score_select"], "block_select": pct([e[0] for e in extra]),
                     "sparse": pct([e[1] for e in extra])}
        stages = {name: val["mean"] for name, val in stage_pct.items()}
    cold = cold_full_pass(torch, hs2, blk, dev)

    ms_per_step = dt * 1e3 / args.steps
    alg_bytes = n_tokens * KV_ROW_BYTES[kv] + batch * 2 * 16 * 128 * 4  # K/V once, query and output per sequence
    both = k1_calls + k1b_calls
    t_both, t_k1 = float(both.mean()), float(k1_calls.mean())
    achieved = alg_bytes / (t_both * 1e-3) / 1e9
    k1_achieved = alg_bytes / (t_k1 * 1e-3) / 1e9
    name = {"token": "full_partial_kernel + merge_bound_hist_kernel (the full layer and its score bounds, K1 + K1b)",
            "block": "full_partial_kernel + merge_block_pool_kernel (the full layer, its per-tile head sums and the "
                     "block sums)",
            "block-scores": "full_partial_kernel + merge_kernel (the full layer keeping every logit; the score pass "
                            "is apart)"}[selection]
    return {
        "value": batch * args.steps / dt,
        "ms_per_step": ms_per_step,
        "dtype": "bf16" if kv == "bf16" else "fp8_e4m3",
        "config": {"workload": WORKLOADS[workload], "batch": batch, "context_tokens": n_tokens,
                   "max_context": int(lens.max()), "kv_cache": kv, "q_heads": 16, "kv_heads": 1,
                   "head_dim": 128, "window": 128, "top_k": 1024, "n_sparse_layers": int(q_sparse.shape[0]),
                   "selection": {"token": "token", "block": "block64 (gen-1 comparator) from tile sums",
                                 "block-scores": "block64 (gen-1 comparator) from per-token scores"}[selection]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(workload) if selection == "token" else None,
                     "kernel": name, "alg_bytes_per_launch": alg_bytes, "mean_launch_ms": t_both,
                     "launch_ms": pct(both),
                     "k1_alone": {"kernel": "full_partial_kernel", "mean_launch_ms": t_k1,
                                  "launch_ms": pct(k1_calls), "achieved": k1_achieved,
                                  "frac": k1_achieved / HBM_PEAK_GBS}},
        "stages_ms": {k2: round(v2, 5) for k2, v2 in stages.items()},  # untimed extra steps
        "stages_ms_percentiles": stage_pct,
        "cold_full_partial_ms": cold,
        "stage_calls_timed": n_rec,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "clocks_during_timed_steps": clocks,
        **({"cpu_baseline": cpu_baseline(d)} if with_cpu else {}),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOADS))
    ap.add_argument("--part", choices=("hybrid-block", "self-decoder"), default="hybrid-block",
                    help="self-decoder: the front half's attention (1 full + 24 sliding-window layers)")
    ap.add_argument("--tokens", type=int, default=1,
                    help="query tokens per sequence and step (above 1: the multi-token decode line)")
    ap.add_argument("--selection", choices=("token", "block", "block-scores"), default="token",
                    help="token: the method's selection; block: the gen-1 64-token-block comparator "
                         "(block sums from tile sums); block-scores: the same through per-token scores")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-1m", action="store_true",
                    help="workload 2 only: skip the second (1M-token E4M3) roofline object")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for this long before the warmup steps (clock settling; 0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy before the timed region (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the decode batch would shard by sequence with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_kv_hs2_amd import hs2, inputs

    hs2.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == 5:
        print(json.dumps(bench_bridge(args, torch, hs2, inputs, dev)), flush=True)
        return
    if args.tokens > 1:
        print(json.dumps(bench_multi(args, torch, hs2, inputs, dev)), flush=True)
        return
    if args.part == "self-decoder":
        print(json.dumps(bench_self_decoder(args, torch, hs2, inputs, dev)), flush=True)
        return
    d = inputs.make_decode(args.workload)
    line = hybrid_block_line(args, torch, hs2, d, dev, args.workload, args.selection, with_cpu=False)
    result = {"metric": METRIC, "value": line.pop("value"), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": line.pop("ms_per_step"), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": line.pop("dtype"), "data": "synthetic"}
    result.update(line)
    if args.workload == 2 and args.selection == "token" and not args.no_1m:
        # The metric's 1M-token half: 4 sequences x 1048576 tokens, E4M3 cache
        # with per-token scales, timed the same way (its own warmup and steps).
        torch.cuda.empty_cache()
        d3 = inputs.make_decode(3)
        sub = hybrid_block_line(args, torch, hs2, d3, dev, 3, "token", with_cpu=False)
        del d3
        result["roofline_ctx1m_fp8"] = dict(sub["roofline"], workload=sub["config"]["workload"],
                                            tokens_per_s=sub["value"], ms_per_step=sub["ms_per_step"],
                                            steps=args.steps, warmup=args.warmup, dtype=sub["dtype"],
                                            stages_ms=sub["stages_ms"], cold_full_partial_ms=sub["cold_full_partial_ms"])
    result["device"] = device_info(torch)
    if not args.no_cpu_baseline and args.selection == "token":
        result["cpu_baseline"] = cpu_baseline(d)  # after every GPU timing: the host work idles the GPU
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
