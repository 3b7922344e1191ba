"""fp64 CPU oracle: what one HySparse2 hybrid block computes at decode, and the
KV-Bridging projection that builds its cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy in float64,
one sequence at a time, no blocking, fusion or reordering beyond what the
definitions state.  Page abbreviations [zh] [en] [pt] [fr] [ko] are defined in
``oracle/__init__.py``.

The pages describe the method in prose only.  Where they leave a step open the
plainest reading is taken; each such reading is named where it is used:

* softmax scale 1/sqrt(head_dim), no bias, sink or cap (pages silent);
* the per-token score is the sum over the query heads of that head's softmax
  probability over the whole context ([en] paragraph on keeping a few
  full-attention layers: they hand complete attention scores to the sparse
  layers; [fr] "Ce que fait HySparse2": the full layer picks positions from its
  attention scores while it computes);
* the 128 most recent positions, the current token included, are always kept
  and the top-1024 are taken from the positions before them ([zh] paragraph on
  the forced recent window; [fr] and [ko] "Ce que fait" / "한 일": 128 recent
  plus 1024 outside the window);
* ties are broken by the lower position;
* a context of at most 128 + 1024 tokens selects every token;
* the sparse layers own no KV: they read the full layer's cache at the selected
  positions and renormalise their softmax over those positions only ([fr]
  "Ce que fait HySparse2": the sparse layers reuse the full layer's KV cache
  and selection indices; [en] paragraph on KV Reuse);
* one selection per sequence under MQA (one KV head) ([fr] "Les chiffres
  mesures": HySparse2 uses a more compact MQA setting);
* the bridge is a plain product of the shared hidden state with each bridged
  layer's own W_k and W_v, no norm, bias or rotary step ([ko] "한 일": one
  source hidden state, independent K/V projections per target layer);
* gen-1 block selection (the ablation comparator): 64-token blocks aligned
  to position 0, block score = sum of its token scores, 16 blocks plus the
  window under the same budget;
* a Self-Decoder sliding-window layer attends to the 128 most recent
  positions (no window size is given; the pages' local window is used),
  kept in a ring buffer at slot position mod 128;
* several query tokens of a sequence in one step (speculative verification,
  which the pages do not describe for HySparse2): each token is a decode step
  of its own over its causal prefix, with its own selection.
"""

from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128
N_Q_HEADS = 16
WINDOW = 128  # [zh] forced recent window paragraph; [fr]/[ko] "Ce que fait"/"한 일"
TOP_K = 1024  # same passages: 1024 tokens from before the window
BAND_REL = 1e-5  # relative band around the k-th score inside which ties may differ
BLOCK = 64  # gen-1 HySparse's selection unit ([en] paragraph on how the sparse layers select)
SWA_WINDOW = 128  # Self-Decoder sliding window: the pages give none; their local window (128) is taken


# --------------------------------------------------------------------------
# Stored-value codecs, written from the format definitions.
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    bfloat16 is the upper half of an IEEE binary32 word, so shifting the 16
    bits into the top of a 32-bit word gives the binary32 value exactly.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16, round-to-nearest-even, in one step.

    bfloat16 keeps 8 significant bits and binary32's exponent range.  For a
    value in [2^E, 2^(E+1)) the spacing is 2^(E-7); below the smallest normal
    2^-126 the spacing stays 2^-133.  The value is divided by its spacing,
    rounded half-to-even (numpy.rint), and multiplied back; both scalings are
    exact powers of two, so the single rounding is the only one.  The rounded
    value is a binary32 number, whose top 16 bits are the bfloat16 pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])  # x = f * 2^e, 0.5 <= |f| < 1, so E = e - 1
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    out[nz] = np.rint(x[nz] / quantum) * quantum
    out[~nz] = x[~nz]
    with np.errstate(over="ignore"):
        f32 = out.astype(np.float32)  # exact: every bfloat16 value is a binary32 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def e4m3_value_table() -> np.ndarray:
    """The 256 values of the OCP 8-bit floating point format E4M3 (float64).

    Per the OCP 8-bit Floating Point Specification: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    m * 2^-9; S.1111.111 is NaN; there are no infinities, so S.1111.000 to
    S.1111.110 are the normal values 256..448.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = math.nan
        elif exp_field == 0:
            table[code] = sign * mant * 2.0 ** -9
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


_E4M3 = e4m3_value_table()


def e4m3_bytes_to_f64(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> exact float64 values by table lookup."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def f64_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float64 values to OCP E4M3 codes (uint8): the nearest of the
    format's finite values, ties to the even code (the one whose mantissa
    field is even), magnitudes beyond 448 saturating to +-448.

    Written from the format definition (see ``e4m3_value_table``); the sign
    is kept, so a negative value that rounds to zero gives the code of -0.  The 127
    non-negative finite values, codes 0x00..0x7E, increase with the code, so
    the two candidates around |x| are adjacent codes.  Saturation is the
    reading taken for a cache encoder (the pages say only "FP8 cache").
    """
    x = np.asarray(x, dtype=np.float64)
    pos = _E4M3[:0x7F]  # codes 0x00..0x7E, increasing
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)  # the sign survives rounding to 0


def quantize_rows_e4m3(x: np.ndarray):
    """Per-row E4M3 with an fp32 scale, the FP8 cache layout the decode path
    reads ([en] paragraph on cost and [pt]: the 1M-token footprints assume an
    FP8 cache; the per-token scale is the reading taken): scale = (largest
    |value| of the row) / 448, stored as fp32 (1 for an all-zero row), and
    codes = E4M3(value / scale) with the stored scale.  Returns (codes uint8
    [rows, cols], scales float32 [rows])."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    codes = f64_to_e4m3(x / scale.astype(np.float64)[:, None])
    return codes, scale


def decode_kv(raw: np.ndarray, kv_dtype: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Stored cache rows -> exact float64 rows.

    ``kv_dtype`` is ``"bf16"`` (raw = uint16 bit patterns, [L, D]) or
    ``"fp8_e4m3"`` (raw = uint8 codes [L, D] and ``scale`` = per-token fp32
    scale [L]; the value is code_value * scale).  The FP8 cache is the one the
    pages quote their 1M-token footprints with ([en] paragraph on cost; [pt]);
    the per-token fp32 scale is the reading of "FP8 cache" taken here.
    """
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8_e4m3":
        assert scale is not None
        return e4m3_bytes_to_f64(raw) * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]
    raise ValueError(kv_dtype)


# --------------------------------------------------------------------------
# The hybrid block at decode.
# --------------------------------------------------------------------------

def full_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Full attention of one decode query over the whole context.

    q [H, D], k and v [L, D] (float64).  Logits are (k q^T) / sqrt(D); each head
    takes the softmax over all L positions; the output is the probability-
    weighted sum of the value rows.  Returns (o [H, D], p [L, H]).

    [fr] "Ce que fait HySparse2" / [ko] "한 일": the first layer of a hybrid
    block is a full-attention layer over the shared cache.
    """
    d = q.shape[-1]
    logits = (k @ q.T) / math.sqrt(d)  # [L, H]
    m = logits.max(axis=0, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=0, keepdims=True)
    p = e / z
    o = p.T @ v  # [H, D]
    return o, p


def swa_ring_slots(length: int, window: int = SWA_WINDOW) -> np.ndarray:
    """Ring slots holding the positions a sliding window of ``window`` covers
    at decode, position p being kept in slot p mod window: positions
    [max(0, L - window), L), in position order."""
    return np.arange(max(0, length - window), length) % window


def swa_attention(q: np.ndarray, ring_k: np.ndarray, ring_v: np.ndarray, length: int,
                  window: int = SWA_WINDOW) -> np.ndarray:
    """One Self-Decoder sliding-window attention layer at decode.

    The front half of the model (the Self-Decoder) mixes full-attention and
    sliding-window layers ([fr] "Ce que fait HySparse2"; [en] paragraph on
    the self-decoder and cross-decoder split).  At decode a window layer
    attends to the ``window`` most recent positions, current token included,
    which a ring buffer of ``window`` rows holds (the reading taken: the
    pages give no window size, so the local window they do give, 128, is
    used).  q [H, D]; ring_k, ring_v [window, D] decoded float64 rows;
    length = positions so far (the current token included).  Returns
    o [H, D]; a sequence with no positions gives zeros.
    """
    if length == 0:
        return np.zeros_like(q, dtype=np.float64)
    slots = swa_ring_slots(length, window)
    o, _ = full_attention(q, ring_k[slots], ring_v[slots])
    return o


def token_scores(p: np.ndarray) -> np.ndarray:
    """Per-token score: the sum over query heads of the softmax probability.

    p [L, H] -> score [L].  The full-attention layer's attention scores pick
    the positions ([en] paragraph on keeping a few full-attention layers;
    [fr] "Ce que fait HySparse2").  Summing the per-head probabilities is the
    reading taken for several query heads sharing one KV head.
    """
    return p.sum(axis=1)


def select_tokens(score: np.ndarray, window: int = WINDOW, top_k: int = TOP_K):
    """Token-level selection: the recent window plus the top-k before it.

    score [L] -> dict(sel, s_k, band):

    * ``sel``: ascending positions.  If L <= window + top_k every position.
      Otherwise the last ``window`` positions, always, plus the ``top_k``
      positions of [0, L - window) with the largest score, ties to the lower
      position.
    * ``s_k``: the k-th largest out-of-window score (None when all are taken).
    * ``band``: out-of-window positions whose score is within BAND_REL * s_k
      of s_k; a selection may legitimately differ from this one only there.

    [zh] paragraph on the forced recent window (keep the latest 128, then pick
    1024 from earlier context); [fr] "Ce que fait HySparse2" (token granularity;
    128 most recent always in, plus 1024 outside the window); [en] paragraph on
    token-level selection.
    """
    score = np.asarray(score, dtype=np.float64)
    n = score.shape[0]
    if n <= window + top_k:
        return {"sel": np.arange(n, dtype=np.int64), "s_k": None, "band": np.zeros(0, dtype=np.int64)}
    c = n - window
    s_c = score[:c]
    pos = np.arange(c)
    order = np.lexsort((pos, -s_c))  # primary: score descending; secondary: position ascending
    top = order[:top_k]
    sel = np.sort(np.concatenate([top, np.arange(c, n)]))
    s_k = float(s_c[order[top_k - 1]])
    band = np.nonzero(np.abs(s_c - s_k) <= BAND_REL * s_k)[0]
    return {"sel": sel.astype(np.int64), "s_k": s_k, "band": band.astype(np.int64)}


def select_blocks(score: np.ndarray, window: int = WINDOW, top_k: int = TOP_K, block: int = BLOCK):
    """Gen-1 (block-level) selection under the same budget, the ablation
    comparator of ``select_tokens``.

    The previous generation picked whole 64-token blocks, so one relevant
    token costs its block's share of the budget; the ablation keeps the
    backbone and the attention budget and changes only the granularity
    ([en] paragraphs on how the sparse layers select and on the ablation;
    [zh] paragraph on block versus token selection; [fr] "Ce que fait
    HySparse2").  Readings, where the pages are silent:

    * blocks are [64 i, 64 i + 64), aligned to position 0; the candidates are
      the complete blocks that end before the window, i = 0 .. (L - window) // 64 - 1;
    * a block's score is the sum of its positions' scores (its share of the
      attention mass);
    * the budget is the token-level one: the window, plus top_k // 64 blocks,
      ranked by block score descending, ties to the lower block;
    * L <= window + top_k selects every position, as at token level.

    score [L] -> dict(sel, s_k, band, band_blocks, block_scores) with ``sel``
    ascending positions, ``s_k`` the last chosen block's score, and
    ``band``/``band_blocks`` the positions/indices of the candidate blocks whose
    score is within BAND_REL * s_k of s_k (where a selection may differ).
    """
    score = np.asarray(score, dtype=np.float64)
    n = score.shape[0]
    none = np.zeros(0, dtype=np.int64)
    if n <= window + top_k:
        return {"sel": np.arange(n, dtype=np.int64), "s_k": None, "band": none, "band_blocks": none,
                "block_scores": np.zeros(0)}
    nb = (n - window) // block
    bs = score[:nb * block].reshape(nb, block).sum(axis=1)
    kb = top_k // block
    order = np.lexsort((np.arange(nb), -bs))  # block score descending, then block index ascending
    top = order[:kb]
    pos = (top[:, None] * block + np.arange(block)[None, :]).ravel()
    sel = np.sort(np.concatenate([pos, np.arange(n - window, n)]))
    s_k = float(bs[order[kb - 1]])
    band_blocks = np.nonzero(np.abs(bs - s_k) <= BAND_REL * s_k)[0]
    band = (band_blocks[:, None] * block + np.arange(block)[None, :]).ravel()
    return {"sel": sel.astype(np.int64), "s_k": s_k, "band": band.astype(np.int64),
            "band_blocks": band_blocks.astype(np.int64), "block_scores": bs}


def sparse_attention(q: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray) -> np.ndarray:
    """One sparse layer: attention of its own query over the selected rows only.

    q [H, D]; k_sel, v_sel [S, D] are the full layer's cache rows at the selected
    positions (KV Reuse: the sparse layer has no KV of its own).  The softmax is
    taken over the S selected positions.  [fr] "Ce que fait HySparse2";
    [ko] "한 일"; [en] paragraph on token-level selection.
    """
    o, _ = full_attention(q, k_sel, v_sel)
    return o


def decode_sequence(q_full: np.ndarray, q_sparse: np.ndarray, k: np.ndarray, v: np.ndarray,
                    window: int = WINDOW, top_k: int = TOP_K, sel_override=None, selection: str = "token"):
    """One sequence through one hybrid block at decode.

    q_full [H, D]; q_sparse [n_s, H, D]; k, v [L, D] decoded float64 rows.
    Steps: full attention and scores, selection ("token": ``select_tokens``;
    "block": the gen-1 comparator ``select_blocks``), then every sparse layer
    over the same selection.  ``sel_override`` (ascending positions) replaces
    the oracle's own selection in the sparse step; tests use it when a GPU
    list differs from this one only inside the tie band.
    """
    o_full, p = full_attention(q_full, k, v)
    score = token_scores(p)
    if selection == "token":
        s = select_tokens(score, window, top_k)
    elif selection == "block":
        s = select_blocks(score, window, top_k)
    else:
        raise ValueError(f"unknown selection {selection!r}")
    sel = s["sel"] if sel_override is None else np.asarray(sel_override, dtype=np.int64)
    ks, vs = k[sel], v[sel]
    o_sparse = np.stack([sparse_attention(q_sparse[l], ks, vs) for l in range(q_sparse.shape[0])]) \
        if q_sparse.shape[0] else np.zeros((0,) + q_full.shape)
    return {"o_full": o_full, "score": score, "sel": s["sel"], "s_k": s["s_k"],
            "band": s["band"], "o_sparse": o_sparse}


def decode_multi_sequence(q_full: np.ndarray, q_sparse: np.ndarray, k: np.ndarray, v: np.ndarray,
                          window: int = WINDOW, top_k: int = TOP_K):
    """Several query tokens of one sequence in one decode step (speculative
    verification).  The pages name no multi-token rule for HySparse2; the
    reading taken: the T tokens occupy the last T positions of the cache and
    token t, at position L - T + t, is a decode step of its own over the
    prefix [0, L - T + t] (causal), with its own selection.

    q_full [T, H, D]; q_sparse [n_s, T, H, D]; k, v [L, D] decoded rows.
    Returns a list of T per-token dicts (see ``decode_sequence``); a token
    whose position is below 0 (L < T) gets None.
    """
    n_tok, length = q_full.shape[0], k.shape[0]
    out = []
    for t in range(n_tok):
        n = length - n_tok + t + 1
        if n <= 0:
            out.append(None)
            continue
        out.append(decode_sequence(q_full[t], q_sparse[:, t], k[:n], v[:n], window, top_k))
    return out


def decode_block(seq_offsets, k_raw, v_raw, q_full, q_sparse, kv_dtype="bf16",
                 k_scale=None, v_scale=None, seqs=None, window=WINDOW, top_k=TOP_K, selection="token"):
    """The hybrid block for a packed batch, one sequence at a time.

    seq_offsets [B+1] (packed rows), k_raw/v_raw [N, D] stored values,
    q_full [B, H, D] fp32, q_sparse [n_s, B, H, D] fp32.  ``seqs`` restricts
    the work to some sequences (full-size tests sample a few).  Returns a list
    of per-sequence dicts (see ``decode_sequence``), None for skipped ones.
    """
    offs = np.asarray(seq_offsets, dtype=np.int64)
    b_count = offs.shape[0] - 1
    want = range(b_count) if seqs is None else seqs
    out = [None] * b_count
    for b in want:
        a, e = int(offs[b]), int(offs[b + 1])
        ks = None if k_scale is None else k_scale[a:e]
        vs = None if v_scale is None else v_scale[a:e]
        k = decode_kv(k_raw[a:e], kv_dtype, ks)
        v = decode_kv(v_raw[a:e], kv_dtype, vs)
        qf = np.asarray(q_full[b], dtype=np.float64)
        qs = np.asarray(q_sparse[:, b], dtype=np.float64)
        out[b] = decode_sequence(qf, qs, k, v, window, top_k, selection=selection)
    return out


# --------------------------------------------------------------------------
# KV Bridging.
# --------------------------------------------------------------------------

def bridge_kv(h_bits: np.ndarray, w_k_bits, w_v_bits, rows=None):
    """KV-Bridging projection: K_l = H W_k[l], V_l = H W_v[l] in float64.

    h_bits [T, d_model] and each W [d_model, D] are bfloat16 bit patterns.
    Every bridged full-attention layer builds its own K/V from the same
    source hidden state with its own projections ([ko] "한 일"; [fr] "Ce que
    fait HySparse2"; [en] paragraph on KV Bridging).  ``rows`` restricts the
    product to some rows of H.  Returns (list of K_l, list of V_l) in float64;
    the stored bfloat16 reference is ``f64_to_bf16_bits`` of these.
    """
    h = bf16_bits_to_f64(h_bits if rows is None else h_bits[rows])
    ks = [h @ bf16_bits_to_f64(w) for w in w_k_bits]
    vs = [h @ bf16_bits_to_f64(w) for w in w_v_bits]
    return ks, vs


def bridge_kv_fp8(h_bits: np.ndarray, w_k_bits, w_v_bits, rows=None):
    """The bridge projection stored as the FP8 cache: ``bridge_kv``'s float64
    products, each row quantised by ``quantize_rows_e4m3``.  Returns
    (list of (codes, scales) for K_l, the same for V_l)."""
    ks, vs = bridge_kv(h_bits, w_k_bits, w_v_bits, rows)
    return [quantize_rows_e4m3(k) for k in ks], [quantize_rows_e4m3(v) for v in vs]
