"""Seeded synthetic inputs for the hybrid-block decode path and the bridge.

This module produces DATA only: random queries, keys, values and hidden
states with the shapes, value distributions and structure of the workloads,
stored in the formats the kernels read (bfloat16 bit patterns, or OCP E4M3
codes with per-token fp32 scales).  It holds none of the method's arithmetic:
no attention, score, selection or projection.  Both the GPU path (through
the tests and the benchmark) and the CPU oracle consume what it returns.

Recipe (per sequence, each from its own child of
``SeedSequence(1000 + workload)`` so sequences can be generated in parallel):

1. q_full  fp32 N(0,1) [16, 128]
2. K       fp32 N(0,1) [L, 128]
3. needles: rows of K replaced by 3 * qbar / |qbar| + eps, eps ~ N(0, I),
   qbar = mean of the 16 full-layer query heads; needles lie before the
   final 128-token window
4. K rounded to bfloat16 (round-to-nearest-even)
5. V       fp32 N(0,1), rounded to bfloat16
6. q_sparse fp32 N(0,1) [n_s, 16, 128]

For the FP8 cache the bfloat16 K and V are quantised per token, K and V
separately: scale = amax / 448 (1 when the row is all zero), code =
E4M3(value / scale) with round-to-nearest-even, clamped to +-448.

The stand-ins: the pages evaluate trained models on long-context retrieval
suites; these inputs reproduce only the shape of such work (context lengths
of 4K, 128K, 1M and a ragged 2K-256K agent mix, a few relevant keys hidden in
long tool-output spans).
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

N_Q_HEADS = 16
HEAD_DIM = 128
WINDOW = 128
TOP_K = 1024
D_MODEL = 4096
N_BRIDGED = 3

# Workload table.  "needles" is a count per sequence, or a rule name.
WORKLOAD_RECIPES = {
    1: dict(name="b1_ctx4k_bf16", batch=1, lengths="fixed", ctx=4096, kv="bf16", n_sparse=3,
            needles=64, needle_mode="uniform"),
    2: dict(name="b32_ctx128k_bf16", batch=32, lengths="fixed", ctx=131072, kv="bf16", n_sparse=4,
            needles=256, needle_mode="uniform"),
    3: dict(name="b4_ctx1m_fp8", batch=4, lengths="fixed", ctx=1048576, kv="fp8_e4m3", n_sparse=4,
            needles=1024, needle_mode="bursts"),
    4: dict(name="b64_ragged_2k_256k_bf16", batch=64, lengths="agent", ctx_min=2048, ctx_max=262144,
            kv="bf16", n_sparse=4, needle_mode="agent"),
    5: dict(name="bridge_262144x4096_3layers_b8x32k", batch=8, lengths="fixed", ctx=32768, kv="bf16",
            n_sparse=4, needles=0, needle_mode="none", tokens=262144, d_model=D_MODEL, n_bridged=N_BRIDGED),
}

_POOL = 8


def _threads() -> int:
    try:
        import os
        return max(1, min(_POOL, len(os.sched_getaffinity(0))))
    except Exception:
        return 4


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def quantize_e4m3_per_token(bits_bf16: np.ndarray):
    """bfloat16 rows [L, D] -> (E4M3 codes uint8 [L, D], fp32 scale [L])."""
    x = bf16_bits_to_f32(bits_bf16)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def agent_lengths(rng: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths log-uniform in [lo, hi]."""
    u = rng.uniform(math.log(lo), math.log(hi), size=batch)
    return np.floor(np.exp(u)).astype(np.int64)


def agent_spans(rng: np.random.Generator, length: int):
    """Alternating (kind, start, end) spans, action first: action U{16..64},
    observation U{2048..32768}, the last span cut at ``length``."""
    spans, pos, action = [], 0, True
    while pos < length:
        n = int(rng.integers(16, 65)) if action else int(rng.integers(2048, 32769))
        end = min(length, pos + n)
        spans.append(("action" if action else "obs", pos, end))
        pos, action = end, not action
    return spans


def _needle_rows(rng, q_full, count):
    qbar = q_full.mean(axis=0)
    direction = (3.0 * qbar / np.linalg.norm(qbar)).astype(np.float32)
    return direction[None, :] + rng.standard_normal((count, HEAD_DIM), dtype=np.float32)


def _needle_positions(rng, cfg, length, spans):
    mode = cfg["needle_mode"]
    limit = length - WINDOW
    if mode == "none" or limit <= 0:
        return np.zeros(0, dtype=np.int64)
    if mode == "uniform":
        count = min(cfg["needles"], limit)
        return np.sort(rng.choice(limit, size=count, replace=False)).astype(np.int64)
    if mode == "bursts":
        n_bursts, burst = 8, cfg["needles"] // 8
        # burst starts uniform in [0, L - 256 - burst], redrawn until no two overlap
        hi = length - 2 * WINDOW - burst
        if hi < n_bursts * burst:
            raise ValueError("context too short for the burst layout")
        while True:
            starts = np.sort(rng.integers(0, hi + 1, size=n_bursts))
            if np.all(np.diff(starts) >= burst):
                break
        pos = (starts[:, None] + np.arange(burst)[None, :]).reshape(-1)
        return pos.astype(np.int64)
    if mode == "agent":
        obs = np.concatenate([np.arange(s, min(e, limit)) for kind, s, e in spans
                              if kind == "obs" and s < limit] or [np.zeros(0, dtype=np.int64)])
        count = min(int(round(length / 512)), obs.shape[0])
        return np.sort(rng.choice(obs, size=count, replace=False)).astype(np.int64)
    raise ValueError(mode)


def _one_sequence(seed_seq, cfg, length, n_sparse, spans):
    rng = np.random.default_rng(seed_seq)
    q_full = rng.standard_normal((N_Q_HEADS, HEAD_DIM), dtype=np.float32)
    k = rng.standard_normal((length, HEAD_DIM), dtype=np.float32)
    needles = _needle_positions(rng, cfg, length, spans)
    if needles.shape[0]:
        k[needles] = _needle_rows(rng, q_full, needles.shape[0])
    k_bits = to_bf16_bits(k)
    del k
    v_bits = to_bf16_bits(rng.standard_normal((length, HEAD_DIM), dtype=np.float32))
    q_sparse = rng.standard_normal((n_sparse, N_Q_HEADS, HEAD_DIM), dtype=np.float32)
    return q_full, k_bits, v_bits, q_sparse, needles


def make_decode(workload: int = None, *, lengths=None, n_sparse=None, kv=None, seed=None,
                needles=None, needle_mode=None):
    """Build one decode batch.

    Either a workload id from WORKLOAD_RECIPES, or custom ``lengths`` (a list of
    context lengths) with ``n_sparse``, ``kv`` ("bf16" | "fp8_e4m3"), ``seed``
    and optional needle settings (used by the tests for small and ragged
    cases).  Returns a dict of host arrays:

    seq_offsets int64 [B+1]; k, v uint16 [N, 128] (bf16 bits) or uint8 (E4M3
    codes); k_scale, v_scale fp32 [N] or None; q_full fp32 [B, 16, 128];
    q_sparse fp32 [n_s, B, 16, 128]; needles list of int64 arrays; kv str.
    """
    if workload is not None:
        cfg = dict(WORKLOAD_RECIPES[workload])
        base_seed = 1000 + workload if seed is None else seed
    else:
        cfg = dict(batch=len(lengths), lengths="custom", kv=kv or "bf16", n_sparse=n_sparse or 0,
                   needles=needles if needles is not None else 0,
                   needle_mode=needle_mode or ("uniform" if needles else "none"))
        base_seed = 7 if seed is None else seed
    root = np.random.SeedSequence(base_seed)
    len_seq, kids_seq = root.spawn(2)
    len_rng = np.random.default_rng(len_seq)
    b = cfg["batch"]
    if cfg["lengths"] == "fixed":
        lens = np.full(b, cfg["ctx"], dtype=np.int64)
    elif cfg["lengths"] == "agent":
        lens = agent_lengths(len_rng, b, cfg["ctx_min"], cfg["ctx_max"])
    else:
        lens = np.asarray(lengths, dtype=np.int64)
    spans = [agent_spans(len_rng, int(l)) if cfg["needle_mode"] == "agent" else None for l in lens]
    n_s = cfg["n_sparse"]
    kids = kids_seq.spawn(b)
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda i: _one_sequence(kids[i], cfg, int(lens[i]), n_s, spans[i]), range(b)))
    offs = np.zeros(b + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    n = int(offs[-1])
    k = np.empty((n, HEAD_DIM), dtype=np.uint16)
    v = np.empty((n, HEAD_DIM), dtype=np.uint16)
    for i, p in enumerate(parts):
        k[offs[i]:offs[i + 1]] = p[1]
        v[offs[i]:offs[i + 1]] = p[2]
    q_full = np.stack([p[0] for p in parts]) if b else np.zeros((0, N_Q_HEADS, HEAD_DIM), np.float32)
    q_sparse = (np.stack([p[3] for p in parts], axis=1) if b
                else np.zeros((n_s, 0, N_Q_HEADS, HEAD_DIM), np.float32))
    out = dict(seq_offsets=offs, q_full=np.ascontiguousarray(q_full),
               q_sparse=np.ascontiguousarray(q_sparse), needles=[p[4] for p in parts],
               kv=cfg["kv"], k_scale=None, v_scale=None, spans=spans)
    del parts
    if cfg["kv"] == "fp8_e4m3":
        k8, ks = quantize_e4m3_per_token(k)
        del k
        v8, vs = quantize_e4m3_per_token(v)
        del v
        out.update(k=k8, v=v8, k_scale=ks, v_scale=vs)
    else:
        out.update(k=k, v=v)
    return out


def make_bridge(tokens: int = 262144, d_model: int = D_MODEL, n_bridged: int = N_BRIDGED,
                seed: int = 1005, block_rows: int = 16384):
    """Hidden states and bridge weights: H [T, d_model] and every W_k, W_v
    [d_model, 128], all bfloat16 N(0, 1/d_model), as uint16 bit patterns.
    H is generated in row blocks, each from its own child seed."""
    root = np.random.SeedSequence(seed)
    w_seq, h_seq = root.spawn(2)
    w_rng = np.random.default_rng(w_seq)
    std = np.float32(1.0 / math.sqrt(d_model))
    w_k = [to_bf16_bits(w_rng.standard_normal((d_model, HEAD_DIM), dtype=np.float32) * std)
           for _ in range(n_bridged)]
    w_v = [to_bf16_bits(w_rng.standard_normal((d_model, HEAD_DIM), dtype=np.float32) * std)
           for _ in range(n_bridged)]
    h = np.empty((tokens, d_model), dtype=np.uint16)
    n_blocks = (tokens + block_rows - 1) // block_rows
    kids = h_seq.spawn(max(n_blocks, 1))

    def fill(i):
        a, e = i * block_rows, min(tokens, (i + 1) * block_rows)
        rng = np.random.default_rng(kids[i])
        h[a:e] = to_bf16_bits(rng.standard_normal((e - a, d_model), dtype=np.float32) * std)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n_blocks)))
    return dict(h=h, w_k=w_k, w_v=w_v)


def make_bridge_queries(batch: int = 8, n_sparse: int = 4, n_bridged: int = N_BRIDGED, seed: int = 2005):
    """Per bridged layer: q_full [B, 16, 128] and q_sparse [n_s, B, 16, 128],
    fp32 N(0,1)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    out = []
    for _ in range(n_bridged):
        qf = rng.standard_normal((batch, N_Q_HEADS, HEAD_DIM), dtype=np.float32)
        qs = rng.standard_normal((n_sparse, batch, N_Q_HEADS, HEAD_DIM), dtype=np.float32)
        out.append((qf, qs))
    return out
