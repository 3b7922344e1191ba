"""Parity rules between the HIP path and the fp64 oracle (test infrastructure).

* selection: count min(L, 1152); ascending, unique, in range; the whole
  window present; equal to the oracle's list except for positions inside the
  oracle's tie band (|score - s_k| <= 1e-5 * s_k);
* o_full, o_sparse: max|gpu - ref| / max|ref| per tensor <= 2e-3 (bf16 KV)
  or 2e-2 (fp8 KV); when the GPU list differs from the oracle's inside the
  band, the sparse reference is recomputed by the oracle with the GPU's list;
* score (diagnostic): max_j |gpu - ref| / max(ref_j, s_k), the per-token
  relative error floored at the k-th score (what decides the selection),
  at most half the tie band (5e-6).
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import hs2_oracle as O

TOL = {"bf16": 2e-3, "fp8_e4m3": 2e-2}


def to_device(d, device="cuda"):
    """Host arrays from long_context_kv_hs2_amd.inputs -> device tensors."""
    t = {}
    t["seq_offsets"] = torch.from_numpy(d["seq_offsets"]).to(device)
    if d["kv"] == "bf16":
        t["k"] = torch.from_numpy(d["k"].view(np.int16)).view(torch.bfloat16).to(device)
        t["v"] = torch.from_numpy(d["v"].view(np.int16)).view(torch.bfloat16).to(device)
        t["k_scale"] = t["v_scale"] = None
    else:
        t["k"] = torch.from_numpy(d["k"]).to(device)
        t["v"] = torch.from_numpy(d["v"]).to(device)
        t["k_scale"] = torch.from_numpy(d["k_scale"]).to(device)
        t["v_scale"] = torch.from_numpy(d["v_scale"]).to(device)
    t["q_full"] = torch.from_numpy(d["q_full"]).to(device)
    t["q_sparse"] = torch.from_numpy(d["q_sparse"]).to(device) if d["q_sparse"].shape[0] else None
    lens = np.diff(d["seq_offsets"])
    t["max_context"] = int(lens.max()) if lens.shape[0] else 0
    return t


def max_abs_rel(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    diff = np.abs(np.asarray(got, dtype=np.float64) - ref).max()
    return float(diff / den) if den > 0 else float(diff)


def check_selection(sel_gpu, count, length, ref, band_rel=None):
    """Returns the GPU list (ascending positions); raises on a violation.
    band_rel: a wider relative tie band than the oracle's 1e-5 (peaked
    attention, where fp32 logits cannot resolve 1e-5; see fp32_logit_band)."""
    want = min(length, 1152)
    assert count == want, f"count {count} != {want} (L={length})"
    got = np.asarray(sel_gpu[:count], dtype=np.int64)
    assert np.all(sel_gpu[count:] == -1), "padding must be -1"
    if count:
        assert np.all(np.diff(got) > 0), "not strictly ascending"
        assert got[0] >= 0 and got[-1] < length, "out of range"
    window = np.arange(max(0, length - 128), length)
    assert np.isin(window, got).all(), "window not fully selected"
    diff = np.setxor1d(got, ref["sel"])
    band = ref["band"]
    if band_rel is not None:
        s_k = ref["s_k"]
        band = np.nonzero(np.abs(ref["score"][:max(0, length - 128)] - s_k) <= band_rel * s_k)[0]
    outside = np.setdiff1d(diff, band)
    assert outside.shape[0] == 0, f"selection differs outside the tie band at {outside[:10]} (L={length})"
    return got


def fp32_logit_band(max_abs_logit_log2):
    """Relative precision of an fp32 score when logits reach
    ``max_abs_logit_log2`` (log2 units) in magnitude: 2^-19 |l|.  A logit is
    built from exact products (the query split into three exact bf16 parts)
    by 12 fp32 accumulations (3 parts x 4 MFMA steps), each rounding by at
    most half an ulp of the running sum, so it is within about 12 * 2^-24 |l|;
    a probability exp2(l - M) / Z carries the errors of l and of the head's
    maximum M: relative 2 ln2 * 12 * 2^-24 |l| < 2^-19 |l|.  This worst case
    stays below the 1e-5 tie band only for |l| under ~5; at the workloads'
    magnitudes (|l| within ~10) the measured score errors are ~1.5e-6, while
    peaked attention (|l| in the hundreds) goes well past the band."""
    return 2.0 ** -19 * float(max_abs_logit_log2)


def max_abs_logit_log2(d, b):
    """max_{h,j} |q_h . k_j| / sqrt(128) * log2(e) of sequence b (oracle's decode of the cache)."""
    a, e = int(d["seq_offsets"][b]), int(d["seq_offsets"][b + 1])
    ks = None if d["k_scale"] is None else d["k_scale"][a:e]
    k = O.decode_kv(d["k"][a:e], d["kv"], ks)
    return float(np.abs(k @ d["q_full"][b].astype(np.float64).T).max()) / np.sqrt(128.0) * np.log2(np.e)


def check_decode(d, out, seqs=None, tol=None, score_tol=5e-6, oracle_cache=None, selection="token",
                 band_rel=None):
    """Compare GPU outputs (dict of tensors) with the oracle on `seqs`.

    Returns a dict of the worst errors seen.  ``oracle_cache`` may hold
    per-sequence oracle results already computed (keyed by sequence).
    ``selection`` names the oracle's rule ("token", or "block" for gen-1).
    ``band_rel`` (a dict by sequence, or one float) widens the tie band
    (see fp32_logit_band); worst["outside_std_band"] counts the sequences
    whose list differs from the oracle's outside the standard 1e-5 band."""
    kv = d["kv"]
    tol = TOL[kv] if tol is None else tol
    offs = d["seq_offsets"]
    b_count = offs.shape[0] - 1
    seqs = range(b_count) if seqs is None else seqs
    o_full = out["o_full"].cpu().numpy()
    o_sparse = out["o_sparse"].cpu().numpy() if out["o_sparse"] is not None else None
    sel_idx = out["sel_idx"].cpu().numpy()
    sel_count = out["sel_count"].cpu().numpy()
    score = out["score"].cpu().numpy() if out.get("score") is not None else None
    worst = dict(o_full=0.0, o_sparse=0.0, score=0.0, band_diffs=0, outside_std_band=0)
    for b in seqs:
        a, e = int(offs[b]), int(offs[b + 1])
        length = e - a
        if length == 0:
            assert sel_count[b] == 0 and np.all(sel_idx[b] == -1)
            assert np.all(o_full[b] == 0)
            if o_sparse is not None:
                assert np.all(o_sparse[:, b] == 0)
            continue
        if oracle_cache is not None and b in oracle_cache:
            ref = oracle_cache[b]
        else:
            ks = None if d["k_scale"] is None else d["k_scale"][a:e]
            vs = None if d["v_scale"] is None else d["v_scale"][a:e]
            kf = O.decode_kv(d["k"][a:e], kv, ks)
            vf = O.decode_kv(d["v"][a:e], kv, vs)
            ref = O.decode_sequence(d["q_full"][b].astype(np.float64), d["q_sparse"][:, b].astype(np.float64), kf, vf,
                                    selection=selection)
            ref["_k"], ref["_v"] = kf, vf
            if oracle_cache is not None:
                oracle_cache[b] = ref
        err = max_abs_rel(o_full[b], ref["o_full"])
        assert err <= tol, f"o_full seq {b}: {err:.3e} > {tol}"
        worst["o_full"] = max(worst["o_full"], err)
        brel = band_rel.get(b) if isinstance(band_rel, dict) else band_rel
        got = check_selection(sel_idx[b], int(sel_count[b]), length, ref, brel)
        if brel is not None and np.setdiff1d(np.setxor1d(got, ref["sel"]), ref["band"]).shape[0]:
            worst["outside_std_band"] += 1
        if score is not None:
            s_k = O.select_tokens(ref["score"])["s_k"] or ref["score"].max()  # the token-level k-th score
            den = np.maximum(ref["score"], s_k)
            serr = float((np.abs(score[a:e].astype(np.float64) - ref["score"]) / den).max())
            stol = score_tol.get(b) if isinstance(score_tol, dict) else score_tol
            assert serr <= stol, f"score seq {b}: {serr:.3e} (relative, floored at s_k) > {stol}"
            worst["score"] = max(worst["score"], serr)
        if o_sparse is not None:
            ref_sparse = ref["o_sparse"]
            if not np.array_equal(got, ref["sel"]):
                worst["band_diffs"] += 1
                redo = O.decode_sequence(d["q_full"][b].astype(np.float64), d["q_sparse"][:, b].astype(np.float64),
                                         ref["_k"], ref["_v"], sel_override=got)
                ref_sparse = redo["o_sparse"]
            for layer in range(ref_sparse.shape[0]):
                err = max_abs_rel(o_sparse[layer, b], ref_sparse[layer])
                assert err <= tol, f"o_sparse layer {layer} seq {b}: {err:.3e} > {tol}"
                worst["o_sparse"] = max(worst["o_sparse"], err)
    return worst


def bf16_ordinal(bits):
    """bf16 bit patterns -> integers ordered like the values (adjacent values
    differ by 1), so a difference in ordinals counts ulps."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _accumulation_bound(h_bits, w_bits, rows):
    """sum_k |h_ik w_kj| and gamma_n = n u / (1 - n u) (u = 2^-24): the
    textbook bound on fp32 accumulation of n exact products is
    gamma_n * sum|h w|.  Test-side error bound only; the reference values
    come from the oracle."""
    h = np.abs(O.bf16_bits_to_f64(h_bits[rows]))
    w = np.abs(O.bf16_bits_to_f64(w_bits))
    n = h.shape[1]
    u = 2.0 ** -24
    return h @ w, n * u / (1 - n * u)


def check_bridge(h_bits, w_bits, out_bits, rows):
    """Bridge outputs (bf16 bits [T, 128]) for the given rows against the
    oracle.  Element-wise bound from the arithmetic: fp32 accumulation of
    d_model exact bf16 products is within gamma_n * sum|h w| of the exact sum
    (gamma_n = n u / (1 - n u), u = 2^-24), and the final rounding to bf16
    adds at most one bf16 ulp.  Also: at most 0.1 % of the elements (at least
    one, for small samples) more than one ulp from the correctly rounded value
    (elements with a large sum|h w| against a small value may miss by two
    within the bound above), and at least 99 % of them equal to it (samples of
    1000 or more): a guard against a systematic error such as truncation.
    No max-abs-relative bar: bf16 output alone is off by up to
    half an ulp, 2^-9 of the largest element, which a 2e-3 bar would not
    reliably admit.  Returns (worst ulps, fraction within 1 ulp)."""
    (ref,), _ = O.bridge_kv(h_bits, [w_bits], [], rows=rows)  # the oracle's float64 product
    abs_sum, gamma = _accumulation_bound(h_bits, w_bits, rows)
    got_bits = out_bits[rows]
    got = O.bf16_bits_to_f64(got_bits)
    mag = np.abs(ref) + gamma * abs_sum
    with np.errstate(divide="ignore"):
        ulp = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.where(mag > 0, mag, 1.0))).astype(int), -126) - 7)
    bound = ulp + gamma * abs_sum
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        msg = (f"{int(bad.sum())} of {err.size} elements beyond the bound; worst at {i}: got {got[i]!r} "
               f"ref {ref[i]!r} bound {bound[i]:.3e} abs_sum {abs_sum[i]:.3e}; "
               f"max err/abs_sum {float((err / np.maximum(abs_sum, 1e-300)).max()):.3e}")
        print(msg, flush=True)
        raise AssertionError(msg)
    ulps = np.abs(bf16_ordinal(got_bits) - bf16_ordinal(O.f64_to_bf16_bits(ref)))
    frac1 = float((ulps <= 1).mean())
    allowed = max(1, int(0.001 * ulps.size))
    assert int((ulps > 1).sum()) <= allowed, f"only {frac1:.5f} of elements within 1 ulp"
    # Rounding to nearest: an fp32 accumulation error is far below half a bf16
    # ulp for nearly every element, so nearly all equal the correctly rounded
    # value; a directed rounding (truncation) misses about half of them while
    # staying within one ulp.
    if ulps.size >= 1000:
        frac0 = float((ulps == 0).mean())
        assert frac0 >= 0.99, f"only {frac0:.5f} of elements equal the correctly rounded value"
    return int(ulps.max()), frac1


def e4m3_ordinal(codes):
    """E4M3 codes -> integers in value order (sign-magnitude; both zeros 0)."""
    c = np.asarray(codes, dtype=np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_bridge_fp8(h_bits, w_bits, codes, scales, rows):
    """FP8 bridge outputs (E4M3 codes [T, 128], fp32 scales [T]) for the given
    rows against the oracle's quantisation of the float64 products.  The GPU
    quantises its fp32 products, each within gamma_n * sum|h w| of the exact
    value (see check_bridge), so its row maxima, hence its scales, differ
    from the oracle's by at most that much relative to the row maximum plus
    one fp32 rounding; and a code can differ only where a value sits within
    that error of a rounding boundary: there by one step of the code order.
    Bar: scales within that relative bound, every code within one step, at
    least 99.5 % of the codes equal.  Returns (fraction of equal codes,
    worst relative scale difference)."""
    (ref,), _ = O.bridge_kv(h_bits, [w_bits], [], rows=rows)
    ((ref_codes, ref_scale),), _ = O.bridge_kv_fp8(h_bits, [w_bits], [], rows=rows)  # the oracle's FP8 cache rows
    abs_sum, gamma = _accumulation_bound(h_bits, w_bits, rows)
    got_codes = np.asarray(codes)[rows]
    got_scale = np.asarray(scales)[rows].astype(np.float64)
    amax = np.abs(ref).max(axis=1)
    rel_bound = np.where(amax > 0, gamma * abs_sum.max(axis=1) / np.where(amax > 0, amax, 1.0), 0.0) + 2.0 ** -22
    rel = np.abs(got_scale - ref_scale.astype(np.float64)) / ref_scale.astype(np.float64)
    assert (rel <= rel_bound).all(), f"scale off by {rel.max():.3e} (bound {rel_bound[rel.argmax()]:.3e})"
    steps = np.abs(e4m3_ordinal(got_codes) - e4m3_ordinal(ref_codes))
    assert steps.max() <= 1, f"a code {steps.max()} steps from the oracle's"
    same = float((steps == 0).mean())
    assert same >= 0.995, f"only {same:.5f} of the codes equal the oracle's"
    return same, float(rel.max())
