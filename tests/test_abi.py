"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status before any HIP call
(so these run without a GPU)."""

import ctypes
import math
import os
import re

import pytest

from long_context_kv_hs2_amd import hs2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hs2.LIB_PATH), reason="libhs2.so not built")

INVALID, UNSUPPORTED, SMALL_WS = 1, 2, 3
FAKE = 0x10000  # a 256-byte aligned non-null address; never dereferenced on the error paths


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(hs2.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(hs2.EXPORTED)


def desc(**kw):
    base = dict(batch=2, total_tokens=5000, max_context=4000, n_sparse_layers=2)
    base.update(kw)
    return hs2.make_desc(**base)


def call_decode(d, ws_bytes=None, **ptrs):
    lib = hs2.load()
    p = dict(seq=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, qf=FAKE, qs=FAKE, of=FAKE, os_=FAKE, si=FAKE, sc=FAKE,
             score=None, ws=FAKE)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.hs2_decode_workspace_bytes(ctypes.byref(d)) if d is not None else 0
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.hs2_decode_block(None if d is None else ctypes.byref(d), v(p["seq"]), v(p["k"]), v(p["v"]),
                                v(p["ks"]), v(p["vs"]), v(p["qf"]), v(p["qs"]), v(p["of"]), v(p["os_"]),
                                v(p["si"]), v(p["sc"]), v(p["score"]), v(p["ws"]), ws_bytes, None)


def test_workspace_query():
    lib = hs2.load()
    d = desc()
    n = lib.hs2_decode_workspace_bytes(ctypes.byref(d))
    n_score = lib.hs2_decode_score_workspace_bytes(ctypes.byref(d))
    # without a score output: no logit spill; the score calls add exactly the
    # 64 B a token of every full-layer logit (rounded to the 256-byte layout)
    assert n_score - n == (5000 * 64 + 255) // 256 * 256
    for q in (lib.hs2_decode_workspace_bytes, lib.hs2_decode_score_workspace_bytes):
        assert q(ctypes.byref(desc(head_dim=64))) == 0
        assert q(None) == 0


def test_workspace_sizes_at_the_bench_shape():
    # 32 x 131072 tokens, bf16, 4 sparse layers: the default path (no score
    # output) needs no room for the 268 MB of logits
    lib = hs2.load()
    d = hs2.make_desc(32, 32 * 131072, 131072, 4)
    n = lib.hs2_decode_workspace_bytes(ctypes.byref(d))
    n_score = lib.hs2_decode_score_workspace_bytes(ctypes.byref(d))
    assert n_score - n >= 32 * 131072 * 64
    assert n < 96 * 2 ** 20


def test_score_output_needs_the_score_workspace():
    lib = hs2.load()
    d = desc()
    n = lib.hs2_decode_workspace_bytes(ctypes.byref(d))
    n_score = lib.hs2_decode_score_workspace_bytes(ctypes.byref(d))
    assert call_decode(d, ws_bytes=n, score=FAKE) == SMALL_WS
    assert "workspace" in lib.hs2_last_error_message().decode()
    assert call_decode(d, ws_bytes=n_score - 1, score=FAKE) == SMALL_WS
    v = ctypes.c_void_p
    assert lib.hs2_full_decode_score(ctypes.byref(d), v(FAKE), v(FAKE), v(FAKE), None, None, v(FAKE), v(FAKE),
                                     v(FAKE), v(FAKE), n, None) == SMALL_WS


@pytest.mark.parametrize("field,value,status", [
    ("n_q_heads", 8, UNSUPPORTED), ("head_dim", 64, UNSUPPORTED), ("window", 64, UNSUPPORTED),
    ("top_k", 512, UNSUPPORTED), ("n_sparse_layers", 9, UNSUPPORTED), ("n_sparse_layers", -1, UNSUPPORTED),
    ("batch", -1, INVALID), ("kv_dtype", 7, INVALID), ("softmax_scale", 0.0, INVALID),
    ("softmax_scale", math.inf, INVALID), ("total_tokens", -1, INVALID), ("max_context", (1 << 24) + 1, UNSUPPORTED),
    ("total_tokens", 9000, INVALID),
])
def test_bad_descriptor(field, value, status):
    d = desc()
    setattr(d, field, value)
    assert call_decode(d, ws_bytes=1 << 40) == status


@pytest.mark.parametrize("name", ["seq", "k", "v", "qf", "qs", "of", "os_", "si", "sc", "ws"])
def test_null_pointer(name):
    assert call_decode(desc(), **{name: None}) == INVALID
    assert hs2.load().hs2_last_error_message().decode()


def test_null_descriptor():
    assert call_decode(None) == INVALID


@pytest.mark.parametrize("name,addr", [("k", FAKE + 8), ("qf", FAKE + 4), ("ws", FAKE + 128), ("seq", FAKE + 4)])
def test_misaligned(name, addr):
    assert call_decode(desc(), **{name: addr}) == INVALID


def test_workspace_too_small():
    d = desc()
    n = hs2.load().hs2_decode_workspace_bytes(ctypes.byref(d))
    assert call_decode(d, ws_bytes=n - 1) == SMALL_WS


def test_scales_must_match_dtype():
    assert call_decode(desc(kv_dtype=1)) == INVALID            # fp8 without scales
    assert call_decode(desc(kv_dtype=0), ks=FAKE, vs=FAKE) == INVALID  # bf16 with scales


def test_sparse_pointers_optional_without_sparse_layers():
    # n_s = 0: q_sparse and o_sparse may be NULL; the call must still fail on
    # the NULL workspace, proving it got past the sparse-pointer checks.
    assert call_decode(desc(n_sparse_layers=0), qs=None, os_=None, ws=None) == INVALID
    msg = hs2.load().hs2_last_error_message().decode()
    assert "workspace" in msg


def test_bridge_validation():
    lib = hs2.load()
    arr = ctypes.c_void_p * 1
    one = arr(FAKE)
    assert lib.hs2_bridge_workspace_bytes(1000, 4096, 128, 3) == 6 * 128 * 4096 * 2
    assert lib.hs2_bridge_workspace_bytes(1000, 100, 128, 3) == 0
    assert lib.hs2_bridge_kv(10, 4096, 64, 1, FAKE, one, one, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert lib.hs2_bridge_kv(10, 4000, 128, 1, FAKE, one, one, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert lib.hs2_bridge_kv(10, 4096, 128, 5, FAKE, one, one, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert lib.hs2_bridge_kv(-1, 4096, 128, 1, FAKE, one, one, one, one, FAKE, 1 << 30, None) == INVALID
    assert lib.hs2_bridge_kv(10, 4096, 128, 1, None, one, one, one, one, FAKE, 1 << 30, None) == INVALID
    assert lib.hs2_bridge_kv(10, 4096, 128, 1, FAKE, one, one, one, one, FAKE, 100, None) == SMALL_WS
    assert lib.hs2_bridge_kv(10, 4096, 128, 1, FAKE, one, one, None, one, FAKE, 1 << 30, None) == INVALID


def test_bridge_packed_validation():
    # Pack-once entry points: shape, pointer and size checks before any HIP call.
    lib = hs2.load()
    arr = ctypes.c_void_p * 1
    one = arr(FAKE)
    need = lib.hs2_bridge_packed_weight_bytes(4096, 128, 3)
    assert need == 6 * 128 * 4096 * 2
    assert lib.hs2_bridge_packed_weight_bytes(100, 128, 3) == 0
    pack = lib.hs2_bridge_pack_weights
    assert pack(4096, 64, 1, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert pack(4000, 128, 1, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert pack(4096, 128, 5, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert pack(4096, 128, 1, None, one, FAKE, 1 << 30, None) == INVALID
    assert pack(4096, 128, 1, one, arr(None), FAKE, 1 << 30, None) == INVALID
    assert pack(4096, 128, 1, one, one, FAKE, 100, None) == SMALL_WS
    assert pack(4096, 128, 1, one, one, FAKE + 16, 1 << 30, None) == INVALID  # packed not 256-byte aligned
    run = lib.hs2_bridge_kv_packed
    assert run(10, 4096, 128, 1, 7, FAKE, FAKE, one, None, one, None, None) == UNSUPPORTED  # kv_dtype
    assert run(10, 4096, 64, 1, hs2.KV_BF16, FAKE, FAKE, one, None, one, None, None) == UNSUPPORTED
    assert run(-1, 4096, 128, 1, hs2.KV_BF16, FAKE, FAKE, one, None, one, None, None) == INVALID
    assert run(10, 4096, 128, 1, hs2.KV_BF16, None, FAKE, one, None, one, None, None) == INVALID
    assert run(10, 4096, 128, 1, hs2.KV_BF16, FAKE, None, one, None, one, None, None) == INVALID
    assert run(10, 4096, 128, 1, hs2.KV_BF16, FAKE, FAKE, None, None, one, None, None) == INVALID
    assert run(10, 4096, 128, 1, hs2.KV_FP8_E4M3, FAKE, FAKE, one, None, one, one, None) == INVALID  # scales
    assert run(10, 4096, 128, 1, hs2.KV_FP8_E4M3, FAKE, FAKE, one, arr(FAKE + 2), one, one, None) == INVALID


def test_bridge_append_validation():
    lib = hs2.load()
    one = (ctypes.c_void_p * 1)(FAKE)
    ws = lib.hs2_bridge_append_workspace_bytes(8, 4096, 128, 1)
    assert ws == 32 * 8 * 2 * 128 * 4
    assert lib.hs2_bridge_append_workspace_bytes(8, 4000, 128, 1) == 0
    assert lib.hs2_bridge_append_workspace_bytes(8, 4096, 128, 5) == 0
    ok = dict(batch=8, d=4096, hd=128, nb=1, kv=0)

    def call(batch=8, d=4096, hd=128, nb=1, kv=0, offs=FAKE, total=100, hidden=FAKE, wk=one, wv=one, kc=one,
             vc=one, ks=None, vs=None, w=FAKE, nbytes=ws):
        return lib.hs2_bridge_append(batch, d, hd, nb, kv, offs, total, hidden, wk, wv, kc, vc, ks, vs, w, nbytes,
                                     None)

    assert call(batch=-1) == INVALID
    assert call(hd=64) == UNSUPPORTED
    assert call(d=4000) == UNSUPPORTED
    assert call(d=32768) == UNSUPPORTED
    assert call(nb=0) == UNSUPPORTED
    assert call(kv=7) == INVALID
    assert call(offs=None) == INVALID
    assert call(hidden=None) == INVALID
    assert call(kc=None) == INVALID
    assert call(kv=1) == INVALID            # E4M3 without scale arrays
    assert call(ks=one, vs=one) == INVALID  # bf16 with scale arrays
    assert call(nbytes=ws - 1) == SMALL_WS
    assert call(total=-1) == INVALID


def test_swa_and_full_decode_validation():
    lib = hs2.load()

    def swa(batch=4, window=128, kv=0, scale=0.088, lengths=FAKE, rk=FAKE, rv=FAKE, rks=None, rvs=None, kn=None,
            vn=None, kns=None, vns=None, q=FAKE, o=FAKE):
        return lib.hs2_swa_decode(batch, window, kv, scale, lengths, rk, rv, rks, rvs, kn, vn, kns, vns, q, o, None)

    assert swa(batch=-1) == INVALID
    assert swa(window=0) == UNSUPPORTED
    assert swa(window=2000) == UNSUPPORTED
    assert swa(kv=3) == INVALID
    assert swa(scale=0.0) == INVALID
    assert swa(lengths=None) == INVALID
    assert swa(rk=None) == INVALID
    assert swa(q=None) == INVALID
    assert swa(kv=1) == INVALID               # E4M3 ring without scales
    assert swa(rks=FAKE, rvs=FAKE) == INVALID  # bf16 ring with scales
    assert swa(kn=FAKE) == INVALID            # k_new without v_new
    assert swa(kn=FAKE + 4, vn=FAKE) == INVALID  # current rows not 16-byte aligned
    assert swa(batch=0, lengths=None, rk=None, rv=None, q=None, o=None) == 0  # nothing to do
    d = desc()
    n = lib.hs2_decode_workspace_bytes(ctypes.byref(d))
    assert lib.hs2_full_decode(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, n, None) == INVALID
    assert lib.hs2_full_decode(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, n - 256,
                               None) == SMALL_WS


def test_decode_multi_validation():
    lib = hs2.load()
    d = desc()
    n = lib.hs2_decode_multi_workspace_bytes(ctypes.byref(d), 4)
    assert n > lib.hs2_decode_workspace_bytes(ctypes.byref(d))
    assert lib.hs2_decode_multi_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.hs2_decode_multi_workspace_bytes(ctypes.byref(d), 17) == 0

    def call(t=4, offs=FAKE, k=FAKE, q=FAKE, qs=FAKE, o=FAKE, os_=FAKE, si=FAKE, sc=FAKE, nbytes=n):
        return lib.hs2_decode_multi(ctypes.byref(d), t, offs, k, k, None, None, q, qs, o, os_, si, sc, FAKE, nbytes,
                                    None)

    assert call(t=0) == UNSUPPORTED
    assert call(t=17) == UNSUPPORTED
    assert call(offs=None) == INVALID
    assert call(q=None) == INVALID
    assert call(qs=None) == INVALID
    assert call(si=None) == INVALID
    assert call(nbytes=n - 1) == SMALL_WS


def test_stage_calls_validate():
    lib = hs2.load()
    d = desc()
    n = lib.hs2_decode_workspace_bytes(ctypes.byref(d))
    assert lib.hs2_topk_select(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, n, None) == INVALID
    assert lib.hs2_block_select(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, n, None) == INVALID
    assert lib.hs2_block_select(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, n, None) == INVALID
    assert lib.hs2_block_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, n - 256, None) == SMALL_WS
    bad = desc()
    bad.top_k = 512
    assert lib.hs2_block_select(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, n, None) == UNSUPPORTED
    assert lib.hs2_full_decode_score(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, n,
                                     None) == INVALID
    assert lib.hs2_sparse_decode(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, FAKE, FAKE, n,
                                 None) == INVALID


def test_gen1_block_call_validates():
    # hs2_decode_block_gen1: hs2_decode_block's checks, on the workspace
    # without the score spill (it keeps per-tile sums, not every logit)
    lib = hs2.load()
    v = ctypes.c_void_p
    d = desc()
    n = lib.hs2_decode_workspace_bytes(ctypes.byref(d))

    def call(dd=d, seq=FAKE, qf=FAKE, qs=FAKE, si=FAKE, nbytes=n, ws=FAKE):
        return lib.hs2_decode_block_gen1(ctypes.byref(dd) if dd is not None else None, v(seq), v(FAKE), v(FAKE),
                                         None, None, v(qf), v(qs), v(FAKE), v(FAKE), v(si), v(FAKE), v(ws),
                                         nbytes, None)

    assert call(dd=None) == INVALID
    assert call(seq=None) == INVALID
    assert call(seq=FAKE + 4) == INVALID
    assert call(qf=None) == INVALID
    assert call(qs=None) == INVALID
    assert call(si=None) == INVALID
    assert call(nbytes=n - 1) == SMALL_WS
    assert call(ws=FAKE + 16) == INVALID
    assert call(dd=desc(head_dim=64)) == UNSUPPORTED
    bad = desc()
    bad.top_k = 512
    assert call(dd=bad) == UNSUPPORTED
    assert lib.hs2_decode_score_workspace_bytes(ctypes.byref(d)) > n  # the spill is not needed here


def test_status_strings():
    lib = hs2.load()
    assert lib.hs2_status_string(0) == b"HS2_OK"
    assert lib.hs2_status_string(3) == b"HS2_ERR_WORKSPACE_TOO_SMALL"
    assert lib.hs2_status_string(99) == b"HS2_UNKNOWN_STATUS"


def test_stage_timing_modes():
    # mode 0 off, 1 every stage, 2 the full pass only; nothing recorded yet,
    # so reading makes no HIP call and returns zeros.
    lib = hs2.load()
    assert lib.hs2_stage_timing_enable(3) == INVALID
    assert lib.hs2_stage_timing_enable(-1) == INVALID
    for mode in (2, 1, 0):
        assert lib.hs2_stage_timing_enable(mode) == 0
    out = (ctypes.c_float * hs2.N_STAGES)()
    n = ctypes.c_int32(-1)
    assert lib.hs2_stage_timing_read(out, ctypes.byref(n)) == 0
    assert n.value == 0 and list(out) == [0.0] * hs2.N_STAGES
    assert lib.hs2_stage_timing_read(None, ctypes.byref(n)) == INVALID
    per = (ctypes.c_float * (4 * hs2.N_STAGES))()
    n.value = -1
    assert lib.hs2_stage_timing_read_calls(per, 4, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.hs2_stage_timing_read_calls(None, 4, ctypes.byref(n)) == INVALID
    assert lib.hs2_stage_timing_read_calls(per, -1, ctypes.byref(n)) == INVALID
    assert hs2.stage_timing_read_calls().shape == (0, hs2.N_STAGES)


def test_bridge_fp8_validation():
    # E4M3 outputs: the same checks as the bf16 call, plus the scale arrays
    # (NULL array, NULL or misaligned entry); nothing reaches the GPU.
    lib = hs2.load()
    arr = ctypes.c_void_p * 1
    one = arr(FAKE)
    f = lib.hs2_bridge_kv_fp8
    assert f(10, 4096, 64, 1, FAKE, one, one, one, one, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert f(10, 4096, 128, 5, FAKE, one, one, one, one, one, one, FAKE, 1 << 30, None) == UNSUPPORTED
    assert f(10, 4096, 128, 1, FAKE, one, one, one, None, one, one, FAKE, 1 << 30, None) == INVALID
    assert f(10, 4096, 128, 1, FAKE, one, one, one, one, one, None, FAKE, 1 << 30, None) == INVALID
    assert f(10, 4096, 128, 1, FAKE, one, one, one, arr(None), one, one, FAKE, 1 << 30, None) == INVALID
    assert f(10, 4096, 128, 1, FAKE, one, one, one, arr(FAKE + 2), one, one, FAKE, 1 << 30, None) == INVALID
    assert f(10, 4096, 128, 1, FAKE, one, one, one, one, one, one, FAKE, 100, None) == SMALL_WS


def test_noalloc_validation_before_any_hip_call():
    lib = hs2.load()
    v = ctypes.c_void_p

    def call(d, qf=FAKE, seq=FAKE):
        return lib.hs2_decode_block_noalloc(ctypes.byref(d), v(seq), v(FAKE), v(FAKE), None, None, v(qf), v(FAKE),
                                            v(FAKE), v(FAKE), v(FAKE), v(FAKE), None)

    big = hs2.make_desc(64, 64 * 262144, 262144, 4)
    assert lib.hs2_decode_workspace_bytes(ctypes.byref(big)) > hs2.NOALLOC_SCRATCH_BYTES
    assert call(big) == UNSUPPORTED
    assert "scratch" in lib.hs2_last_error_message().decode()
    assert call(desc(), qf=None) == INVALID
    assert call(desc(), seq=FAKE + 4) == INVALID
    assert call(desc(head_dim=64)) == UNSUPPORTED
    # the workloads it is sized for fit
    for b, n, lmax, kv in ((32, 32 * 131072, 131072, 0), (4, 4 * 1048576, 1048576, 1), (8, 262144, 32768, 0)):
        d = hs2.make_desc(b, n, lmax, 4, kv)
        assert lib.hs2_decode_workspace_bytes(ctypes.byref(d)) <= hs2.NOALLOC_SCRATCH_BYTES
