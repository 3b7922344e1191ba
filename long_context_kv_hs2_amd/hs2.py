"""ctypes binding of libhs2.so (include/hs2.h).

Argument marshalling only: torch tensors supply device memory (outputs and
workspace are allocated with torch) and the current HIP stream; every step of
the path runs in the library's kernels.  The first call loads the library and
raises if it is missing; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhs2.so")

HS2_OK = 0
KV_BF16 = 0
KV_FP8_E4M3 = 1
N_STAGES = 4
STAGE_NAMES = ("full_partial", "full_merge", "score_select", "sparse")

EXPORTED = (
    "hs2_decode_workspace_bytes", "hs2_decode_score_workspace_bytes", "hs2_decode_block", "hs2_decode_block_noalloc", "hs2_decode_block_gen1", "hs2_full_decode_score", "hs2_topk_select", "hs2_block_select",
    "hs2_sparse_decode", "hs2_bridge_workspace_bytes", "hs2_bridge_kv", "hs2_bridge_kv_fp8",
    "hs2_bridge_packed_weight_bytes", "hs2_bridge_pack_weights", "hs2_bridge_kv_packed",
    "hs2_bridge_append_workspace_bytes", "hs2_bridge_append", "hs2_full_decode", "hs2_swa_decode",
    "hs2_decode_multi_workspace_bytes", "hs2_decode_multi", "hs2_stage_timing_enable",
    "hs2_stage_timing_read", "hs2_stage_timing_read_calls", "hs2_status_string", "hs2_last_error_message",
)


class Hs2Error(RuntimeError):
    pass


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_sparse_layers", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("total_tokens", ctypes.c_int64),
        ("max_context", ctypes.c_int64),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load libhs2.so and declare its signatures (no HIP call happens here)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise Hs2Error(f"{path} is not built: run `python -m long_context_kv_hs2_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    dp = ctypes.POINTER(DecodeDesc)
    lib.hs2_decode_workspace_bytes.argtypes = [dp]
    lib.hs2_decode_workspace_bytes.restype = sz
    lib.hs2_decode_score_workspace_bytes.argtypes = [dp]
    lib.hs2_decode_score_workspace_bytes.restype = sz
    lib.hs2_decode_block.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_decode_block.restype = ctypes.c_int
    lib.hs2_decode_block_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hs2_decode_block_noalloc.restype = ctypes.c_int
    lib.hs2_decode_block_gen1.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_decode_block_gen1.restype = ctypes.c_int
    lib.hs2_full_decode_score.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_full_decode_score.restype = ctypes.c_int
    lib.hs2_topk_select.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_topk_select.restype = ctypes.c_int
    lib.hs2_block_select.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_block_select.restype = ctypes.c_int
    lib.hs2_sparse_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_sparse_decode.restype = ctypes.c_int
    lib.hs2_bridge_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.hs2_bridge_workspace_bytes.restype = sz
    lib.hs2_bridge_kv.argtypes = [i64, i32, i32, i32, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                  ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, vp]
    lib.hs2_bridge_kv.restype = ctypes.c_int
    lib.hs2_bridge_kv_fp8.argtypes = [i64, i32, i32, i32, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                      ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                      vp, sz, vp]
    lib.hs2_bridge_kv_fp8.restype = ctypes.c_int
    lib.hs2_bridge_packed_weight_bytes.argtypes = [i32, i32, i32]
    lib.hs2_bridge_packed_weight_bytes.restype = sz
    lib.hs2_bridge_pack_weights.argtypes = [i32, i32, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, vp]
    lib.hs2_bridge_pack_weights.restype = ctypes.c_int
    lib.hs2_bridge_kv_packed.argtypes = [i64, i32, i32, i32, i32, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                         ctypes.POINTER(vp), ctypes.POINTER(vp), vp]
    lib.hs2_bridge_kv_packed.restype = ctypes.c_int
    lib.hs2_bridge_append_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.hs2_bridge_append_workspace_bytes.restype = sz
    pp = ctypes.POINTER(vp)
    lib.hs2_bridge_append.argtypes = [i32, i32, i32, i32, i32, vp, i64, vp, pp, pp, pp, pp, pp, pp, vp, sz, vp]
    lib.hs2_bridge_append.restype = ctypes.c_int
    lib.hs2_decode_multi_workspace_bytes.argtypes = [dp, i32]
    lib.hs2_decode_multi_workspace_bytes.restype = sz
    lib.hs2_decode_multi.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_decode_multi.restype = ctypes.c_int
    lib.hs2_full_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs2_full_decode.restype = ctypes.c_int
    lib.hs2_swa_decode.argtypes = [i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hs2_swa_decode.restype = ctypes.c_int
    lib.hs2_stage_timing_enable.argtypes = [i32]
    lib.hs2_stage_timing_enable.restype = ctypes.c_int
    lib.hs2_stage_timing_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.hs2_stage_timing_read.restype = ctypes.c_int
    lib.hs2_stage_timing_read_calls.argtypes = [ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
    lib.hs2_stage_timing_read_calls.restype = ctypes.c_int
    lib.hs2_status_string.argtypes = [ctypes.c_int]
    lib.hs2_status_string.restype = ctypes.c_char_p
    lib.hs2_last_error_message.argtypes = []
    lib.hs2_last_error_message.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int):
    if status != HS2_OK:
        lib = load()
        raise Hs2Error(f"{lib.hs2_status_string(status).decode()}: {lib.hs2_last_error_message().decode()}")


def make_desc(batch, total_tokens, max_context, n_sparse_layers, kv_dtype=KV_BF16, n_q_heads=16, head_dim=128,
              window=128, top_k=1024, softmax_scale=None) -> DecodeDesc:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return DecodeDesc(batch, n_q_heads, head_dim, window, top_k, n_sparse_layers, kv_dtype,
                      softmax_scale, total_tokens, max_context)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def decode_workspace_bytes(desc: DecodeDesc, with_score: bool = False) -> int:
    """Workspace bytes for desc; with_score: for the calls that return per-token scores."""
    if with_score:
        return load().hs2_decode_score_workspace_bytes(ctypes.byref(desc))
    return load().hs2_decode_workspace_bytes(ctypes.byref(desc))


def _workspace(nbytes, device, workspace=None):
    if workspace is not None and workspace.numel() >= nbytes:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def kv_dtype_of(k: torch.Tensor) -> int:
    return KV_FP8_E4M3 if k.dtype in (torch.uint8, torch.float8_e4m3fn) else KV_BF16


class DecodeBlock:
    """Reusable decode call: holds the descriptor, outputs and workspace so
    repeated steps (benchmarks) allocate nothing.  selection="block" calls
    hs2_decode_block_gen1 (gen-1 block selection, no per-token scores)."""

    def __init__(self, seq_offsets, k, v, q_full, q_sparse, k_scale=None, v_scale=None, max_context=None,
                 with_score=False, total_tokens=None, selection="token"):
        if selection not in ("token", "block"):
            raise ValueError(f"selection {selection!r}: 'token' or 'block'")
        if selection == "block" and with_score:
            raise ValueError("the gen-1 call returns no per-token scores")
        self.selection = selection
        dev = k.device
        self.seq_offsets, self.k, self.v, self.k_scale, self.v_scale = seq_offsets, k, v, k_scale, v_scale
        self.q_full, self.q_sparse = q_full, q_sparse
        batch = q_full.shape[0]
        n_s = 0 if q_sparse is None else q_sparse.shape[0]
        if max_context is None:
            max_context = int((seq_offsets[1:] - seq_offsets[:-1]).max().item()) if batch else 0
        total = k.shape[0] if total_tokens is None else total_tokens
        self.desc = make_desc(batch, total, max_context, n_s, kv_dtype_of(k))
        self.o_full = torch.empty((batch, 16, 128), dtype=torch.float32, device=dev)
        self.o_sparse = torch.empty((n_s, batch, 16, 128), dtype=torch.float32, device=dev) if n_s else None
        self.sel_idx = torch.empty((batch, 1152), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((batch,), dtype=torch.int32, device=dev)
        self.score = torch.empty((k.shape[0],), dtype=torch.float32, device=dev) if with_score else None
        self.workspace = _workspace(decode_workspace_bytes(self.desc, with_score), dev)

    def __call__(self):
        if self.selection == "block":
            check(load().hs2_decode_block_gen1(
                ctypes.byref(self.desc), _ptr(self.seq_offsets), _ptr(self.k), _ptr(self.v), _ptr(self.k_scale),
                _ptr(self.v_scale), _ptr(self.q_full), _ptr(self.q_sparse), _ptr(self.o_full),
                _ptr(self.o_sparse), _ptr(self.sel_idx), _ptr(self.sel_count), _ptr(self.workspace),
                self.workspace.numel(), _stream()))
            return self
        check(load().hs2_decode_block(
            ctypes.byref(self.desc), _ptr(self.seq_offsets), _ptr(self.k), _ptr(self.v), _ptr(self.k_scale),
            _ptr(self.v_scale), _ptr(self.q_full), _ptr(self.q_sparse), _ptr(self.o_full), _ptr(self.o_sparse),
            _ptr(self.sel_idx), _ptr(self.sel_count), _ptr(self.score), _ptr(self.workspace),
            self.workspace.numel(), _stream()))
        return self

    def outputs(self):
        return dict(o_full=self.o_full, o_sparse=self.o_sparse, sel_idx=self.sel_idx,
                    sel_count=self.sel_count, score=self.score)


class MultiDecode:
    """Multi-token decode step: q_full [B, T, 16, 128], q_sparse [n_s, B, T,
    16, 128]; each token decodes over its causal prefix with its own
    selection.  Holds outputs and workspace across calls."""

    def __init__(self, seq_offsets, k, v, q_full, q_sparse, k_scale=None, v_scale=None, max_context=None):
        dev = k.device
        self.seq_offsets, self.k, self.v, self.k_scale, self.v_scale = seq_offsets, k, v, k_scale, v_scale
        self.q_full, self.q_sparse = q_full, q_sparse
        batch, self.n_query = q_full.shape[0], q_full.shape[1]
        n_s = 0 if q_sparse is None else q_sparse.shape[0]
        if max_context is None:
            max_context = int((seq_offsets[1:] - seq_offsets[:-1]).max().item()) if batch else 0
        self.desc = make_desc(batch, k.shape[0], max_context, n_s, kv_dtype_of(k))
        t = self.n_query
        self.o_full = torch.empty((batch, t, 16, 128), dtype=torch.float32, device=dev)
        self.o_sparse = torch.empty((n_s, batch, t, 16, 128), dtype=torch.float32, device=dev) if n_s else None
        self.sel_idx = torch.empty((batch, t, 1152), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((batch, t), dtype=torch.int32, device=dev)
        need = load().hs2_decode_multi_workspace_bytes(ctypes.byref(self.desc), t)
        self.workspace = _workspace(need, dev)

    def __call__(self):
        check(load().hs2_decode_multi(
            ctypes.byref(self.desc), self.n_query, _ptr(self.seq_offsets), _ptr(self.k), _ptr(self.v),
            _ptr(self.k_scale), _ptr(self.v_scale), _ptr(self.q_full), _ptr(self.q_sparse), _ptr(self.o_full),
            _ptr(self.o_sparse), _ptr(self.sel_idx), _ptr(self.sel_count), _ptr(self.workspace),
            self.workspace.numel(), _stream()))
        return self


NOALLOC_SCRATCH_BYTES = 96 << 20


def decode_block_noalloc(blk: "DecodeBlock"):
    """hs2_decode_block_noalloc on a DecodeBlock's inputs and outputs (its
    own workspace is not used: the library's scratch array is)."""
    check(load().hs2_decode_block_noalloc(
        ctypes.byref(blk.desc), _ptr(blk.seq_offsets), _ptr(blk.k), _ptr(blk.v), _ptr(blk.k_scale),
        _ptr(blk.v_scale), _ptr(blk.q_full), _ptr(blk.q_sparse), _ptr(blk.o_full), _ptr(blk.o_sparse),
        _ptr(blk.sel_idx), _ptr(blk.sel_count), _stream()))
    return blk


def decode_block(seq_offsets, k, v, q_full, q_sparse, k_scale=None, v_scale=None, max_context=None,
                 with_score=True):
    """One hybrid-block decode step; returns a dict of output tensors."""
    return DecodeBlock(seq_offsets, k, v, q_full, q_sparse, k_scale, v_scale, max_context, with_score)().outputs()


def full_decode_score(seq_offsets, k, v, q_full, k_scale=None, v_scale=None, max_context=None):
    dev = k.device
    batch = q_full.shape[0]
    if max_context is None:
        max_context = int((seq_offsets[1:] - seq_offsets[:-1]).max().item()) if batch else 0
    desc = make_desc(batch, k.shape[0], max_context, 0, kv_dtype_of(k))
    o_full = torch.empty((batch, 16, 128), dtype=torch.float32, device=dev)
    score = torch.empty((k.shape[0],), dtype=torch.float32, device=dev)
    ws = _workspace(decode_workspace_bytes(desc, with_score=True), dev)
    check(load().hs2_full_decode_score(ctypes.byref(desc), _ptr(seq_offsets), _ptr(k), _ptr(v), _ptr(k_scale),
                                       _ptr(v_scale), _ptr(q_full), _ptr(o_full), _ptr(score), _ptr(ws),
                                       ws.numel(), _stream()))
    return o_full, score


def topk_select(seq_offsets, score, batch, max_context):
    dev = score.device
    desc = make_desc(batch, score.shape[0], max_context, 0)
    sel_idx = torch.empty((batch, 1152), dtype=torch.int32, device=dev)
    sel_count = torch.empty((batch,), dtype=torch.int32, device=dev)
    ws = _workspace(decode_workspace_bytes(desc), dev)
    check(load().hs2_topk_select(ctypes.byref(desc), _ptr(seq_offsets), _ptr(score), _ptr(sel_idx),
                                 _ptr(sel_count), _ptr(ws), ws.numel(), _stream()))
    return sel_idx, sel_count


def block_select(seq_offsets, score, batch, max_context):
    """Gen-1 block-level selection (16 blocks of 64 + the window) from given scores."""
    dev = score.device
    desc = make_desc(batch, score.shape[0], max_context, 0)
    sel_idx = torch.empty((batch, 1152), dtype=torch.int32, device=dev)
    sel_count = torch.empty((batch,), dtype=torch.int32, device=dev)
    ws = _workspace(decode_workspace_bytes(desc), dev)
    check(load().hs2_block_select(ctypes.byref(desc), _ptr(seq_offsets), _ptr(score), _ptr(sel_idx),
                                  _ptr(sel_count), _ptr(ws), ws.numel(), _stream()))
    return sel_idx, sel_count


class BlockSelectDecode:
    """The hybrid block with gen-1 selection, as three stage calls sharing one
    workspace and fixed outputs: full attention with scores, block selection,
    then the sparse layers over that list."""

    def __init__(self, seq_offsets, k, v, q_full, q_sparse, k_scale=None, v_scale=None, max_context=None):
        dev = k.device
        self.seq_offsets, self.k, self.v, self.k_scale, self.v_scale = seq_offsets, k, v, k_scale, v_scale
        self.q_full, self.q_sparse = q_full, q_sparse
        batch = q_full.shape[0]
        n_s = 0 if q_sparse is None else q_sparse.shape[0]
        if max_context is None:
            max_context = int((seq_offsets[1:] - seq_offsets[:-1]).max().item()) if batch else 0
        self.desc = make_desc(batch, k.shape[0], max_context, n_s, kv_dtype_of(k))
        self.o_full = torch.empty((batch, 16, 128), dtype=torch.float32, device=dev)
        self.o_sparse = torch.empty((n_s, batch, 16, 128), dtype=torch.float32, device=dev) if n_s else None
        self.sel_idx = torch.empty((batch, 1152), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((batch,), dtype=torch.int32, device=dev)
        self.score = torch.empty((k.shape[0],), dtype=torch.float32, device=dev)
        self.workspace = _workspace(decode_workspace_bytes(self.desc, with_score=True), dev)

    def __call__(self, marks=None):
        """marks: optional three torch.cuda.Event recorded before the block
        selection, between it and the sparse layers, and after them."""
        lib, d, ws, st = load(), ctypes.byref(self.desc), _ptr(self.workspace), _stream()
        n = self.workspace.numel()
        check(lib.hs2_full_decode_score(d, _ptr(self.seq_offsets), _ptr(self.k), _ptr(self.v), _ptr(self.k_scale),
                                        _ptr(self.v_scale), _ptr(self.q_full), _ptr(self.o_full), _ptr(self.score),
                                        ws, n, st))
        if marks:
            marks[0].record()
        check(lib.hs2_block_select(d, _ptr(self.seq_offsets), _ptr(self.score), _ptr(self.sel_idx),
                                   _ptr(self.sel_count), ws, n, st))
        if marks:
            marks[1].record()
        if self.desc.n_sparse_layers:
            check(lib.hs2_sparse_decode(d, _ptr(self.seq_offsets), _ptr(self.k), _ptr(self.v), _ptr(self.k_scale),
                                        _ptr(self.v_scale), _ptr(self.q_sparse), _ptr(self.sel_idx),
                                        _ptr(self.sel_count), _ptr(self.o_sparse), ws, n, st))
        if marks:
            marks[2].record()
        return self

    def outputs(self):
        return dict(o_full=self.o_full, o_sparse=self.o_sparse, sel_idx=self.sel_idx,
                    sel_count=self.sel_count, score=self.score)


def sparse_decode(seq_offsets, k, v, q_sparse, sel_idx, sel_count, k_scale=None, v_scale=None, max_context=None):
    dev = k.device
    n_s, batch = q_sparse.shape[0], q_sparse.shape[1]
    if max_context is None:
        max_context = int((seq_offsets[1:] - seq_offsets[:-1]).max().item()) if batch else 0
    desc = make_desc(batch, k.shape[0], max_context, n_s, kv_dtype_of(k))
    o_sparse = torch.empty((n_s, batch, 16, 128), dtype=torch.float32, device=dev)
    ws = _workspace(decode_workspace_bytes(desc), dev)
    check(load().hs2_sparse_decode(ctypes.byref(desc), _ptr(seq_offsets), _ptr(k), _ptr(v), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(q_sparse), _ptr(sel_idx), _ptr(sel_count), _ptr(o_sparse),
                                   _ptr(ws), ws.numel(), _stream()))
    return o_sparse


def bridge_workspace_bytes(n_tokens, d_model, n_bridged, head_dim=128) -> int:
    return load().hs2_bridge_workspace_bytes(n_tokens, d_model, head_dim, n_bridged)


def bridge_kv(hidden, w_k, w_v, k_out=None, v_out=None, workspace=None):
    """K_l = hidden . w_k[l], V_l = hidden . w_v[l] (bf16 in/out, fp32 accumulate)."""
    dev = hidden.device
    t, d_model = hidden.shape
    n = len(w_k)
    if k_out is None:
        k_out = [torch.empty((t, 128), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    if v_out is None:
        v_out = [torch.empty((t, 128), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    arr = ctypes.c_void_p * n
    ws = _workspace(bridge_workspace_bytes(t, d_model, n), dev, workspace)
    check(load().hs2_bridge_kv(t, d_model, 128, n, _ptr(hidden), arr(*[w.data_ptr() for w in w_k]),
                               arr(*[w.data_ptr() for w in w_v]), arr(*[o.data_ptr() for o in k_out]),
                               arr(*[o.data_ptr() for o in v_out]), _ptr(ws), ws.numel(), _stream()))
    return k_out, v_out


def bridge_kv_fp8(hidden, w_k, w_v, k_out=None, k_sc=None, v_out=None, v_sc=None, workspace=None):
    """The bridge projection stored as E4M3 with per-token fp32 scales:
    returns (k_codes, k_scales, v_codes, v_scales), lists of uint8 [T, 128]
    and fp32 [T] tensors, one per bridged layer (allocated when not given)."""
    dev = hidden.device
    t, d_model = hidden.shape
    n = len(w_k)
    new = lambda shape, dt: [torch.empty(shape, dtype=dt, device=dev) for _ in range(n)]
    k_out = new((t, 128), torch.uint8) if k_out is None else k_out
    v_out = new((t, 128), torch.uint8) if v_out is None else v_out
    k_sc = new((t,), torch.float32) if k_sc is None else k_sc
    v_sc = new((t,), torch.float32) if v_sc is None else v_sc
    arr = ctypes.c_void_p * n
    ws = _workspace(bridge_workspace_bytes(t, d_model, n), dev, workspace)
    check(load().hs2_bridge_kv_fp8(t, d_model, 128, n, _ptr(hidden), arr(*[w.data_ptr() for w in w_k]),
                                   arr(*[w.data_ptr() for w in w_v]), arr(*[o.data_ptr() for o in k_out]),
                                   arr(*[o.data_ptr() for o in k_sc]), arr(*[o.data_ptr() for o in v_out]),
                                   arr(*[o.data_ptr() for o in v_sc]), _ptr(ws), ws.numel(), _stream()))
    return k_out, k_sc, v_out, v_sc


def bridge_pack_weights(w_k, w_v, packed=None):
    """Pack the bridge weights once (uint8 device buffer, allocated when not
    given) for bridge_kv_packed."""
    dev = w_k[0].device
    d_model = w_k[0].shape[0]
    n = len(w_k)
    need = load().hs2_bridge_packed_weight_bytes(d_model, 128, n)
    packed = _workspace(need, dev, packed)
    arr = ctypes.c_void_p * n
    check(load().hs2_bridge_pack_weights(d_model, 128, n, arr(*[w.data_ptr() for w in w_k]),
                                         arr(*[w.data_ptr() for w in w_v]), _ptr(packed), packed.numel(), _stream()))
    return packed


def bridge_kv_packed(hidden, packed, n_bridged, k_out=None, v_out=None, k_sc=None, v_sc=None, fp8=False):
    """The bridge projection from packed weights: (k_out, v_out) as bridge_kv,
    or (k_codes, k_scales, v_codes, v_scales) as bridge_kv_fp8 when fp8."""
    dev = hidden.device
    t, d_model = hidden.shape
    n = n_bridged
    new = lambda shape, dt: [torch.empty(shape, dtype=dt, device=dev) for _ in range(n)]
    code = torch.uint8 if fp8 else torch.bfloat16
    k_out = new((t, 128), code) if k_out is None else k_out
    v_out = new((t, 128), code) if v_out is None else v_out
    if fp8:
        k_sc = new((t,), torch.float32) if k_sc is None else k_sc
        v_sc = new((t,), torch.float32) if v_sc is None else v_sc
    arr = ctypes.c_void_p * n
    ptrs = lambda ts: arr(*[x.data_ptr() for x in ts]) if ts is not None else None
    check(load().hs2_bridge_kv_packed(t, d_model, 128, n, KV_FP8_E4M3 if fp8 else KV_BF16, _ptr(hidden), _ptr(packed),
                                      ptrs(k_out), ptrs(k_sc), ptrs(v_out), ptrs(v_sc), _stream()))
    return (k_out, k_sc, v_out, v_sc) if fp8 else (k_out, v_out)


def bridge_append(seq_offsets, hidden, w_k, w_v, k_cache, v_cache, k_scale=None, v_scale=None, workspace=None):
    """Project each sequence's current hidden row (bf16 [B, d_model]) by every
    bridged layer's W_k, W_v and write it at row seq_offsets[b+1]-1 of the
    layer's cache (bf16, or uint8 E4M3 codes with fp32 per-token scales)."""
    dev = hidden.device
    batch, d_model = hidden.shape
    n = len(w_k)
    fp8 = k_cache[0].dtype == torch.uint8
    arr = ctypes.c_void_p * n
    need = load().hs2_bridge_append_workspace_bytes(batch, d_model, 128, n)
    ws = _workspace(need, dev, workspace)
    ptrs = lambda ts: arr(*[t.data_ptr() for t in ts]) if ts is not None else None
    check(load().hs2_bridge_append(batch, d_model, 128, n, KV_FP8_E4M3 if fp8 else KV_BF16, _ptr(seq_offsets),
                                   k_cache[0].shape[0], _ptr(hidden), ptrs(w_k), ptrs(w_v), ptrs(k_cache),
                                   ptrs(v_cache), ptrs(k_scale), ptrs(v_scale), _ptr(ws), ws.numel(), _stream()))


def full_decode(seq_offsets, k, v, q_full, k_scale=None, v_scale=None, max_context=None, o_full=None,
                workspace=None):
    """Full attention alone (the Self-Decoder's full-attention layer): o_full."""
    dev = k.device
    batch = q_full.shape[0]
    if max_context is None:
        max_context = int((seq_offsets[1:] - seq_offsets[:-1]).max().item()) if batch else 0
    desc = make_desc(batch, k.shape[0], max_context, 0, kv_dtype_of(k))
    o_full = torch.empty((batch, 16, 128), dtype=torch.float32, device=dev) if o_full is None else o_full
    ws = _workspace(decode_workspace_bytes(desc), dev, workspace)
    check(load().hs2_full_decode(ctypes.byref(desc), _ptr(seq_offsets), _ptr(k), _ptr(v), _ptr(k_scale),
                                 _ptr(v_scale), _ptr(q_full), _ptr(o_full), _ptr(ws), ws.numel(), _stream()))
    return o_full


def swa_decode(lengths, ring_k, ring_v, q, ring_k_scale=None, ring_v_scale=None, k_new=None, v_new=None,
               k_new_scale=None, v_new_scale=None, o=None, softmax_scale=None):
    """One sliding-window layer over ring caches [B, window, 128] (bf16, or
    uint8 E4M3 codes with [B, window] scales); with k_new/v_new the current
    rows are attended and stored into their slot.  Returns o [B, 16, 128] fp32."""
    batch, window = ring_k.shape[0], ring_k.shape[1]
    dev = ring_k.device
    fp8 = ring_k.dtype == torch.uint8
    o = torch.empty((batch, 16, 128), dtype=torch.float32, device=dev) if o is None else o
    scale = 1.0 / math.sqrt(128) if softmax_scale is None else softmax_scale
    check(load().hs2_swa_decode(batch, window, KV_FP8_E4M3 if fp8 else KV_BF16, scale, _ptr(lengths), _ptr(ring_k),
                                _ptr(ring_v), _ptr(ring_k_scale), _ptr(ring_v_scale), _ptr(k_new), _ptr(v_new),
                                _ptr(k_new_scale), _ptr(v_new_scale), _ptr(q), _ptr(o), _stream()))
    return o


def stage_timing(on: bool, full_pass_only: bool = False):
    """Record HIP events around the decode stages (or only around the full pass)."""
    check(load().hs2_stage_timing_enable(0 if not on else 2 if full_pass_only else 1))


def stage_timing_read_calls(max_calls: int = 1024):
    """Per-call stage durations (ms) since the last read: float32 [n_calls, 4]."""
    import numpy as np
    buf = (ctypes.c_float * (max_calls * N_STAGES))()
    n = ctypes.c_int32(0)
    check(load().hs2_stage_timing_read_calls(buf, max_calls, ctypes.byref(n)))
    return np.frombuffer(buf, dtype=np.float32).reshape(max_calls, N_STAGES)[:min(n.value, max_calls)].copy()


def stage_timing_read():
    """Mean ms per stage over the calls recorded since the last read."""
    out = (ctypes.c_float * N_STAGES)()
    n = ctypes.c_int32(0)
    check(load().hs2_stage_timing_read(out, ctypes.byref(n)))
    return dict(zip(STAGE_NAMES, list(out))), n.value
