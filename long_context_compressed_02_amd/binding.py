"""Thin ctypes binding of libdsv4attn.so (argument marshalling only).

Every function has the name of its C entry point and forwards to it; torch
tensors are passed as raw device pointers, the stream defaults to torch's
current stream.  A non-zero status raises ``Dsv4Error``.  All arithmetic of the
method runs in the HIP kernels: nothing here computes attention, scores or
entries.  The library must have been built (``python -m
long_context_compressed_02_amd.build``); importing without it fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsv4attn.so")

DSV4_OK, DSV4_ERR_INVALID_ARG, DSV4_ERR_UNSUPPORTED, DSV4_ERR_WORKSPACE, DSV4_ERR_LAUNCH, DSV4_ERR_HIP = range(6)
DSV4_CSA, DSV4_HCA = 0, 1
DSV4_STORE_FP32, DSV4_STORE_FP8, DSV4_STORE_MXFP4 = 0, 1, 2
DSV4_DT_F32, DSV4_DT_BF16, DSV4_DT_F64 = 0, 1, 2
DSV4_POLICY_AUTO, DSV4_POLICY_HI, DSV4_POLICY_LO = 0, 1, 2
DSV4_TARGET_ENTRY, DSV4_TARGET_INDEX_KEY, DSV4_TARGET_WINDOW = 0, 1, 2
DSV4_BLOCK_TOKENS = 128
DSV4_K_COMPRESS, DSV4_K_INDEX_SCORE, DSV4_K_TOPK, DSV4_K_ATTEND, DSV4_K_PROJ, DSV4_K_MX, DSV4_K_COUNT = range(7)

EXPORTS = [
    "dsv4_status_string", "dsv4_get_layout", "dsv4_workspace_bytes", "dsv4_compress_kv_decode",
    "dsv4_compress_kv_prefill", "dsv4_index_topk_decode", "dsv4_index_topk_prefill",
    "dsv4_csa_attend_decode", "dsv4_hca_attend_decode", "dsv4_csa_attend_prefill",
    "dsv4_hca_attend_prefill", "dsv4_cache_write_entries", "dsv4_state_write_tokens",
    "dsv4_timer_enable", "dsv4_timer_read", "dsv4_topk_rows_ws_bytes", "dsv4_topk_rows", "dsv4_out_proj",
    "dsv4_out_proj_pack", "dsv4_cache_dump_bytes", "dsv4_cache_dump", "dsv4_cache_load",
    "dsv4_mx_pack_bytes", "dsv4_mx_pack_weight", "dsv4_mx_linear", "dsv4_index_q_proj_ws_bytes",
    "dsv4_index_q_proj", "dsv4_cache_read_entries", "dsv4_index_topk_decode_noalloc", "dsv4_kv_proj_ws_bytes",
    "dsv4_kv_proj", "dsv4_index_scores_layout",
]
DSV4_NOALLOC_SCRATCH_BYTES = 32 << 20


class Dsv4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


class Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("d", "d_rope", "n_heads", "window", "m_csa", "w_csa", "m_hca",
                                              "idx_heads", "idx_dim", "topk", "kv_store", "idx_store",
                                              "act_dtype")] + [("rope_base", ctypes.c_float),
                                                               ("softmax_scale", ctypes.c_float)]


class Cache(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_req", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("n_blocks", ctypes.c_int32), ("entries", ctypes.c_void_p), ("index_keys", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("block_table", ctypes.c_void_p)]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("record_bytes", "entries_per_block", "entry_block_bytes",
                                              "index_key_bytes", "index_block_bytes", "state_bytes",
                                              "pending_offset", "pending_slots", "pending_token_floats")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m long_context_compressed_02_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        cp, kp = ctypes.POINTER(Cfg), ctypes.POINTER(Cache)
        L.dsv4_status_string.restype = ctypes.c_char_p
        L.dsv4_status_string.argtypes = [i32]
        sig = {
            "dsv4_get_layout": [cp, i32, ctypes.POINTER(Layout)],
            "dsv4_workspace_bytes": [cp, i32, i32, ctypes.POINTER(i64)],
            "dsv4_index_scores_layout": [cp, kp, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)],
            "dsv4_compress_kv_decode": [cp, kp, vp, vp, vp, vp, vp, vp, i32, vp],
            "dsv4_compress_kv_prefill": [cp, kp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp],
            "dsv4_index_topk_decode": [cp, kp, vp, vp, vp, vp, i32, vp, vp, i64, vp],
            "dsv4_index_topk_decode_noalloc": [cp, kp, vp, vp, vp, vp, i32, vp, vp],
            "dsv4_index_topk_prefill": [cp, kp, vp, vp, vp, vp, vp, i32, i32, vp, vp, i64, vp],
            "dsv4_csa_attend_decode": [cp, kp, vp, vp, vp, vp, vp, vp, i32, i32, vp],
            "dsv4_hca_attend_decode": [cp, kp, vp, vp, vp, vp, vp, i32, i32, vp],
            "dsv4_csa_attend_prefill": [cp, kp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp],
            "dsv4_hca_attend_prefill": [cp, kp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp],
            "dsv4_cache_write_entries": [cp, kp, i32, vp, vp, i32, vp, vp],
            "dsv4_cache_read_entries": [cp, kp, i32, vp, vp, i32, vp, i32, vp],
            "dsv4_state_write_tokens": [cp, kp, i32, i32, i32, vp, vp, vp, vp, vp],
            "dsv4_topk_rows_ws_bytes": [i32, i32, i32, ctypes.POINTER(i64)],
            "dsv4_topk_rows": [vp, i64, vp, i32, i32, i32, vp, vp, i64, vp],
            "dsv4_out_proj": [cp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp],
            "dsv4_out_proj_pack": [cp, i32, i32, i32, vp, vp, vp, vp, vp],
            "dsv4_cache_dump_bytes": [cp, i32, i32, ctypes.POINTER(i64)],
            "dsv4_cache_dump": [cp, kp, i32, i32, vp, i64, vp],
            "dsv4_cache_load": [cp, kp, i32, i32, vp, i64, vp],
            "dsv4_mx_pack_bytes": [i32, i32, i32, ctypes.POINTER(i64)],
            "dsv4_mx_pack_weight": [vp, i32, i32, vp, i64, vp],
            "dsv4_mx_linear": [vp, i32, i32, vp, i32, vp, i64, vp, i32, vp],
            "dsv4_index_q_proj_ws_bytes": [cp, i32, i32, i32, ctypes.POINTER(i64)],
            "dsv4_index_q_proj": [cp, vp, i32, i32, i32, vp, vp, vp, i64, vp, vp],
            "dsv4_kv_proj_ws_bytes": [cp, i32, i32, ctypes.POINTER(i64)],
            "dsv4_kv_proj": [cp, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp],
            "dsv4_timer_enable": [i32, i32],
            "dsv4_timer_read": [i32, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = i32
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().dsv4_status_string(s).decode()


def _ck(fn: str, s: int):
    if s != DSV4_OK:
        raise Dsv4Error(fn, s)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# --------------------------------------------------------------------- config / layout
def make_cfg(d=512, d_rope=64, n_heads=128, window=128, m_csa=4, w_csa=8, m_hca=128, idx_heads=64,
             idx_dim=128, topk=1024, kv_store=DSV4_STORE_FP8, idx_store=DSV4_STORE_FP8,
             act_dtype=DSV4_DT_BF16, rope_base=10000.0, softmax_scale=None) -> Cfg:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    return Cfg(d, d_rope, n_heads, window, m_csa, w_csa, m_hca, idx_heads, idx_dim, topk, kv_store,
               idx_store, act_dtype, rope_base, softmax_scale)


def dsv4_get_layout(cfg: Cfg, kind: int) -> Layout:
    out = Layout()
    _ck("dsv4_get_layout", lib().dsv4_get_layout(ctypes.byref(cfg), kind, ctypes.byref(out)))
    return out


def dsv4_workspace_bytes(cfg: Cfg, n_queries: int, max_entries: int) -> int:
    out = ctypes.c_int64()
    _ck("dsv4_workspace_bytes", lib().dsv4_workspace_bytes(ctypes.byref(cfg), n_queries, max_entries,
                                                           ctypes.byref(out)))
    return out.value


class LayerCache:
    """Device memory of one layer's cache (torch tensors) and its C descriptor.

    block_table: int32 tensor [n_req, max_blocks] on the device."""

    def __init__(self, cfg: Cfg, kind: int, n_req: int, max_blocks: int, n_blocks: int, block_table,
                 device="cuda"):
        self.cfg, self.kind = cfg, kind
        self.layout = dsv4_get_layout(cfg, kind)
        lay = self.layout
        self.entries = torch.zeros(n_blocks * lay.entry_block_bytes, dtype=torch.uint8, device=device)
        self.index_keys = (torch.zeros(n_blocks * lay.index_block_bytes, dtype=torch.uint8, device=device)
                           if kind == DSV4_CSA else None)
        self.state = torch.zeros(n_req * lay.state_bytes, dtype=torch.uint8, device=device)
        self.block_table = block_table
        self.c = Cache(kind, n_req, max_blocks, n_blocks, self.entries.data_ptr(),
                       None if self.index_keys is None else self.index_keys.data_ptr(),
                       self.state.data_ptr(), block_table.data_ptr())


# --------------------------------------------------------------------- entry points
def dsv4_index_scores_layout(cfg, cache: LayerCache, n_queries: int, prefill: bool):
    """(byte offset, row stride in floats) of the score rows an index call leaves in its workspace."""
    off, ld = ctypes.c_int64(), ctypes.c_int64()
    _ck("dsv4_index_scores_layout", lib().dsv4_index_scores_layout(
        ctypes.byref(cfg), ctypes.byref(cache.c), n_queries, 1 if prefill else 0, ctypes.byref(off), ctypes.byref(ld)))
    return off.value, ld.value


def dsv4_compress_kv_decode(cfg, cache: LayerCache, kv, gate, kI, gI, req, pos, stream=None):
    _ck("dsv4_compress_kv_decode", lib().dsv4_compress_kv_decode(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(kv), _p(gate), _p(kI), _p(gI), _p(req), _p(pos),
        req.shape[0], _stream(stream)))


def dsv4_compress_kv_prefill(cfg, cache: LayerCache, kv, gate, kI, gI, cu_seqlens, req, pos0, total_tokens,
                             win_out, stream=None):
    _ck("dsv4_compress_kv_prefill", lib().dsv4_compress_kv_prefill(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(kv), _p(gate), _p(kI), _p(gI), _p(cu_seqlens), _p(req),
        _p(pos0), req.shape[0], total_tokens, _p(win_out), _stream(stream)))


def dsv4_index_topk_decode(cfg, cache: LayerCache, qI, w, req, pos, topk_out, ws, stream=None):
    _ck("dsv4_index_topk_decode", lib().dsv4_index_topk_decode(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(qI), _p(w), _p(req), _p(pos), req.shape[0], _p(topk_out),
        _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dsv4_index_topk_decode_noalloc(cfg, cache: LayerCache, qI, w, req, pos, topk_out, stream=None):
    _ck("dsv4_index_topk_decode_noalloc", lib().dsv4_index_topk_decode_noalloc(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(qI), _p(w), _p(req), _p(pos), req.shape[0], _p(topk_out),
        _stream(stream)))


def dsv4_index_topk_prefill(cfg, cache: LayerCache, qI, w, cu_seqlens, req, pos0, total_tokens, topk_out, ws,
                            stream=None):
    _ck("dsv4_index_topk_prefill", lib().dsv4_index_topk_prefill(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(qI), _p(w), _p(cu_seqlens), _p(req), _p(pos0),
        req.shape[0], total_tokens, _p(topk_out), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dsv4_csa_attend_decode(cfg, cache: LayerCache, q, req, pos, topk_idx, sinks, out,
                           policy=DSV4_POLICY_AUTO, stream=None):
    _ck("dsv4_csa_attend_decode", lib().dsv4_csa_attend_decode(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(q), _p(req), _p(pos), _p(topk_idx), _p(sinks), _p(out),
        req.shape[0], policy, _stream(stream)))


def dsv4_hca_attend_decode(cfg, cache: LayerCache, q, req, pos, sinks, out, policy=DSV4_POLICY_AUTO,
                           stream=None):
    _ck("dsv4_hca_attend_decode", lib().dsv4_hca_attend_decode(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(q), _p(req), _p(pos), _p(sinks), _p(out), req.shape[0],
        policy, _stream(stream)))


def dsv4_csa_attend_prefill(cfg, cache: LayerCache, q, cu_seqlens, req, pos0, total_tokens, topk_idx, win,
                            sinks, out, stream=None):
    _ck("dsv4_csa_attend_prefill", lib().dsv4_csa_attend_prefill(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(q), _p(cu_seqlens), _p(req), _p(pos0), req.shape[0],
        total_tokens, _p(topk_idx), _p(win), _p(sinks), _p(out), _stream(stream)))


def dsv4_hca_attend_prefill(cfg, cache: LayerCache, q, cu_seqlens, req, pos0, total_tokens, win, sinks, out,
                            stream=None):
    _ck("dsv4_hca_attend_prefill", lib().dsv4_hca_attend_prefill(
        ctypes.byref(cfg), ctypes.byref(cache.c), _p(q), _p(cu_seqlens), _p(req), _p(pos0), req.shape[0],
        total_tokens, _p(win), _p(sinks), _p(out), _stream(stream)))


def dsv4_cache_write_entries(cfg, cache: LayerCache, target, req, entry, values, stream=None):
    _ck("dsv4_cache_write_entries", lib().dsv4_cache_write_entries(
        ctypes.byref(cfg), ctypes.byref(cache.c), target, _p(req), _p(entry), req.shape[0], _p(values),
        _stream(stream)))


def dsv4_cache_read_entries(cfg, cache: LayerCache, target, req, idx, out, stream=None):
    """out: float32 or float64 device tensor [n, dim] receiving the decoded stored values."""
    dt = {torch.float32: DSV4_DT_F32, torch.float64: DSV4_DT_F64}[out.dtype]
    _ck("dsv4_cache_read_entries", lib().dsv4_cache_read_entries(
        ctypes.byref(cfg), ctypes.byref(cache.c), target, _p(req), _p(idx), req.shape[0], _p(out), dt,
        _stream(stream)))


def dsv4_state_write_tokens(cfg, cache: LayerCache, req: int, pos0: int, kv, gate, kI=None, gI=None,
                            stream=None):
    _ck("dsv4_state_write_tokens", lib().dsv4_state_write_tokens(
        ctypes.byref(cfg), ctypes.byref(cache.c), req, pos0, kv.shape[0], _p(kv), _p(gate), _p(kI), _p(gI),
        _stream(stream)))


def dsv4_cache_dump_bytes(cfg, kind: int, n_tokens: int) -> int:
    out = ctypes.c_int64()
    _ck("dsv4_cache_dump_bytes", lib().dsv4_cache_dump_bytes(ctypes.byref(cfg), kind, n_tokens, ctypes.byref(out)))
    return out.value


def dsv4_cache_dump(cfg, cache: LayerCache, req: int, n_tokens: int, buf, stream=None):
    """buf: uint8 device tensor of at least dsv4_cache_dump_bytes bytes."""
    _ck("dsv4_cache_dump", lib().dsv4_cache_dump(ctypes.byref(cfg), ctypes.byref(cache.c), req, n_tokens, _p(buf),
                                                 buf.numel() * buf.element_size(), _stream(stream)))


def dsv4_cache_load(cfg, cache: LayerCache, req: int, n_tokens: int, buf, stream=None):
    _ck("dsv4_cache_load", lib().dsv4_cache_load(ctypes.byref(cfg), ctypes.byref(cache.c), req, n_tokens, _p(buf),
                                                 buf.numel() * buf.element_size(), _stream(stream)))


def dsv4_topk_rows_ws_bytes(n_rows: int, max_n: int, k: int) -> int:
    out = ctypes.c_int64()
    _ck("dsv4_topk_rows_ws_bytes", lib().dsv4_topk_rows_ws_bytes(n_rows, max_n, k, ctypes.byref(out)))
    return out.value


def dsv4_topk_rows(scores, n, max_n: int, k: int, out, ws, stream=None):
    """scores: fp32 [n_rows, ld] (row stride ld); n: int32 [n_rows]; out: int32 [n_rows, k]."""
    _ck("dsv4_topk_rows", lib().dsv4_topk_rows(
        _p(scores), scores.stride(0), _p(n), n.shape[0], max_n, k, _p(out), _p(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def dsv4_out_proj(cfg, groups: int, rank: int, hidden: int, o, w1p, w2p, y_ws, out, stream=None):
    """o: bf16 [T, n_heads, d]; w1p, w2p: the weights packed by dsv4_out_proj_pack;
    y_ws: bf16 [T, groups*rank]; out: bf16 [T, hidden]."""
    _ck("dsv4_out_proj", lib().dsv4_out_proj(ctypes.byref(cfg), groups, rank, hidden, _p(o), _p(w1p), _p(w2p),
                                             _p(y_ws), _p(out), o.shape[0], _stream(stream)))


def dsv4_out_proj_pack(cfg, groups: int, rank: int, hidden: int, w1, w2, w1p, w2p, stream=None):
    """w1: bf16 [groups, rank, n_heads/groups*d]; w2: bf16 [hidden, groups*rank]; w1p, w2p: same sizes."""
    _ck("dsv4_out_proj_pack", lib().dsv4_out_proj_pack(ctypes.byref(cfg), groups, rank, hidden, _p(w1), _p(w2),
                                                       _p(w1p), _p(w2p), _stream(stream)))


def dsv4_mx_pack_bytes(rows: int, K: int, fp8: bool) -> int:
    out = ctypes.c_int64()
    _ck("dsv4_mx_pack_bytes", lib().dsv4_mx_pack_bytes(rows, K, int(fp8), ctypes.byref(out)))
    return out.value


def dsv4_mx_pack_weight(w, wp, stream=None):
    """w: bf16 [N, K]; wp: uint8 device tensor of dsv4_mx_pack_bytes(N, K, False) bytes."""
    _ck("dsv4_mx_pack_weight", lib().dsv4_mx_pack_weight(_p(w), w.shape[0], w.shape[1], _p(wp),
                                                         wp.numel() * wp.element_size(), _stream(stream)))


def dsv4_mx_linear(x, wp, N: int, ws, out, stream=None):
    """x: bf16 [M, K]; wp: packed MXFP4 weights [N, K]; ws: uint8 workspace of
    dsv4_mx_pack_bytes(M, K, True) bytes; out: fp32 or bf16 [M, N]."""
    import torch
    dt = DSV4_DT_F32 if out.dtype == torch.float32 else DSV4_DT_BF16
    _ck("dsv4_mx_linear", lib().dsv4_mx_linear(_p(x), x.shape[0], x.shape[1], _p(wp), N, _p(ws),
                                               ws.numel() * ws.element_size(), _p(out), dt, _stream(stream)))


def dsv4_index_q_proj_ws_bytes(cfg, T: int, hidden: int, dc: int) -> int:
    out = ctypes.c_int64()
    _ck("dsv4_index_q_proj_ws_bytes", lib().dsv4_index_q_proj_ws_bytes(ctypes.byref(cfg), T, hidden, dc,
                                                                       ctypes.byref(out)))
    return out.value


def dsv4_index_q_proj(cfg, x, dc: int, wdq_p, wuq_p, ws, qI, stream=None):
    """x: bf16 [T, hidden]; wdq_p, wuq_p: packed MXFP4 weights; ws: uint8 workspace;
    qI: [T, idx_heads, idx_dim] in the act dtype."""
    _ck("dsv4_index_q_proj", lib().dsv4_index_q_proj(ctypes.byref(cfg), _p(x), x.shape[0], x.shape[1], dc,
                                                     _p(wdq_p), _p(wuq_p), _p(ws), ws.numel() * ws.element_size(),
                                                     _p(qI), _stream(stream)))


def dsv4_kv_proj_ws_bytes(cfg, T: int, hidden: int) -> int:
    out = ctypes.c_int64()
    _ck("dsv4_kv_proj_ws_bytes", lib().dsv4_kv_proj_ws_bytes(ctypes.byref(cfg), T, hidden, ctypes.byref(out)))
    return out.value


def dsv4_kv_proj(cfg, kind: int, x, wkv_p, wg_p, wki_p, wgi_p, ww_p, kv, gate, kI, gI, w, ws, stream=None):
    """x bf16 [T, hidden]; packed weights (None where absent); outputs as documented."""
    T, hidden = x.shape
    _ck("dsv4_kv_proj", lib().dsv4_kv_proj(
        ctypes.byref(cfg), kind, _p(x), T, hidden, _p(wkv_p), _p(wg_p), _p(wki_p), _p(wgi_p), _p(ww_p), _p(kv),
        _p(gate), _p(kI), _p(gI), _p(w), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dsv4_timer_enable(kernel_id: int, on: bool = True):
    _ck("dsv4_timer_enable", lib().dsv4_timer_enable(kernel_id, int(on)))


def dsv4_timer_read(kernel_id: int, reset: bool = True):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _ck("dsv4_timer_read", lib().dsv4_timer_read(kernel_id, int(reset), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
