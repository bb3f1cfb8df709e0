"""CPU oracle for the CSA/HCA compressed-attention hot path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this module.  It composes the fp64 C primitives of
``dsv4_oracle.c`` into the method, step by step in the pages' order:

  1. raw window records: RoPE at the token's own position, then storage
     quantisation (vastsailsolution.com V4 article, paragraphs after the HCA
     section: window of the last 128 raw tokens; RoPE on the last 64 dims;
     BF16 RoPE dims + FP8 rest);
  2. CSA entries: every m=4 tokens, overlapping window of 8 tokens (same
     article, CSA section; hwcomputing.csdn.net article section 二, CSA step 1);
  3. HCA entries: every m'=128 tokens, no overlap (vastsailsolution.com, HCA
     section; hwcomputing.csdn.net section 二, HCA);
  4. indexer scores of the compressed index keys (vastsailsolution.com, CSA
     section, paragraph on the indexer; xiaoyuzhoufm.com summary 1.1, "CSA
     then applies DSA");
  5. top-k (same CSA section: the 512 / 1024 most relevant entries);
  6. MQA over the selected / all entries plus the window, with a per-head
     sink logit in the denominator (vastsailsolution.com, sink paragraph).

Readings taken where the pages are silent are stated at each function.  It
shares no code with the HIP library and never imports it.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsv4_oracle.c")
_SO = os.path.join(_HERE, "libdsv4_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp-contract off: no fused multiply-add)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        dp = ctypes.POINTER(ctypes.c_double)
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_bf16_round.restype = ctypes.c_float
        L.orc_bf16_round.argtypes = [ctypes.c_float]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e2m1_encode.argtypes = [ctypes.c_float]
        L.orc_mx_exponent.restype = ctypes.c_int
        L.orc_mx_exponent.argtypes = [ctypes.c_float]
        L.orc_store_rows.argtypes = [dp, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp]
        L.orc_rope_rows.argtypes = [dp, ctypes.c_long, ctypes.c_int, ctypes.c_int, dp, ctypes.c_double]
        L.orc_pool_entries.argtypes = [dp, dp, ctypes.c_int, ctypes.POINTER(ctypes.c_long),
                                       ctypes.POINTER(ctypes.c_int), ctypes.c_long, dp]
        L.orc_index_scores.argtypes = [dp, dp, ctypes.c_int, ctypes.c_int, dp, ctypes.c_long, dp]
        L.orc_topk.argtypes = [dp, ctypes.c_long, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)]
        L.orc_attend.argtypes = [dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_double, dp,
                                 ctypes.c_long, dp, dp]
        L.orc_out_proj.argtypes = [dp, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp,
                                   ctypes.c_int, dp, dp]
        L.orc_mxfp8_rows.argtypes = [dp, ctypes.c_long, ctypes.c_int, dp]
        _lib = L
    return _lib


def _dp(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------------------
# configuration (plain numbers; the oracle keeps its own copy of the shape)
# ---------------------------------------------------------------------------
@dataclass
class OCfg:
    d: int = 512            # head dim (the pages: raised to 512)
    d_rope: int = 64        # RoPE dims, the LAST d_rope of d
    n_heads: int = 128      # query heads sharing one KV head
    window: int = 128       # raw sliding window W
    m_csa: int = 4          # CSA stride m
    w_csa: int = 8          # CSA overlapped window (reading: 2m, backward overlap)
    m_hca: int = 128        # HCA stride m' (no overlap)
    idx_heads: int = 64
    idx_dim: int = 128
    topk: int = 1024
    kv_mode: int = 1        # 0: fp32 storage, 1: FP8 E4M3 (one scale) + BF16 RoPE dims
    idx_mode: int = 1       # 0: fp32 index keys / queries, 1: FP8 E4M3 with one scale per row,
                            # 2: MXFP4 (E2M1 codes, one power-of-two scale per 32 dims)
    rope_base: float = 10000.0
    tau: float = field(default=float("nan"))  # softmax scale, default 1/sqrt(d)

    def __post_init__(self):
        if math.isnan(self.tau):
            self.tau = 1.0 / math.sqrt(self.d)


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------
def num_threads() -> int:
    return lib().orc_num_threads()


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e4m3_encode(y: float) -> int:
    return lib().orc_e4m3_encode(y)


def bf16_round(x: float) -> float:
    return lib().orc_bf16_round(x)


def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(code)


def e2m1_encode(y: float) -> int:
    return lib().orc_e2m1_encode(y)


def mx_exponent(amax: float) -> int:
    return lib().orc_mx_exponent(amax)


def store_records(x, cfg: OCfg) -> np.ndarray:
    """KV record storage: fp8 first d - d_rope dims (one scale), bf16 RoPE dims."""
    x = _f64(x).reshape(-1, cfg.d)
    out = np.empty_like(x)
    lib().orc_store_rows(_dp(x), x.shape[0], cfg.d, cfg.d - cfg.d_rope, cfg.kv_mode, _dp(out))
    return out


def store_index_rows(x, cfg: OCfg) -> np.ndarray:
    """Index keys and index queries: all idx_dim dims FP8 with one scale per row
    (idx_mode 1), or MXFP4 with one power-of-two scale per 32 dims (idx_mode 2)."""
    x = _f64(x).reshape(-1, cfg.idx_dim)
    out = np.empty_like(x)
    lib().orc_store_rows(_dp(x), x.shape[0], cfg.idx_dim, cfg.idx_dim, cfg.idx_mode, _dp(out))
    return out


def rope(x, pos, cfg: OCfg) -> np.ndarray:
    """Rotate the last d_rope dims of each row (rows x d) by its position."""
    x = _f64(x).reshape(-1, cfg.d).copy()
    p = _f64(np.broadcast_to(np.asarray(pos, dtype=np.float64), (x.shape[0],)).copy())
    lib().orc_rope_rows(_dp(x), x.shape[0], cfg.d, cfg.d_rope, _dp(p), cfg.rope_base)
    return x


def pool(kv, gate, first, count) -> np.ndarray:
    """Gated softmax pooling of token ranges [first[e], first[e]+count[e])."""
    kv = _f64(kv)
    gate = _f64(gate)
    dim = kv.shape[1]
    first = np.ascontiguousarray(np.asarray(first, dtype=np.int64))
    count = np.ascontiguousarray(np.asarray(count, dtype=np.int32))
    n = first.shape[0]
    out = np.empty((n, dim), dtype=np.float64)
    if n:
        assert (first >= 0).all() and (first + count <= kv.shape[0]).all()
        lib().orc_pool_entries(_dp(kv), _dp(gate), dim,
                               first.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                               count.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), n, _dp(out))
    return out


def index_scores(qI_stored, w, keys_stored) -> np.ndarray:
    q = _f64(qI_stored)
    H, D = q.shape
    w = _f64(w).reshape(H)
    k = _f64(keys_stored).reshape(-1, D)
    out = np.empty(k.shape[0], dtype=np.float64)
    if k.shape[0]:
        lib().orc_index_scores(_dp(q), _dp(w), H, D, _dp(k), k.shape[0], _dp(out))
    return out


def topk(scores, k: int) -> np.ndarray:
    s = _f64(scores).reshape(-1)
    out = np.empty(k, dtype=np.int32)
    lib().orc_topk(_dp(s), s.shape[0], k, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return out


def attend(q_rot, sinks, recs, tau: float, return_sink_mass: bool = False):
    q = _f64(q_rot)
    H, d = q.shape
    z = _f64(sinks).reshape(H)
    r = _f64(recs).reshape(-1, d)
    out = np.empty((H, d), dtype=np.float64)
    sm = np.empty(H, dtype=np.float64)
    lib().orc_attend(_dp(q), _dp(z), H, d, tau, _dp(r), r.shape[0], _dp(out), _dp(sm))
    return (out, sm) if return_sink_mass else out


def mxfp8_rows(x) -> np.ndarray:
    """Rows as MXFP8: E4M3 values with one power-of-two scale per 32 dims."""
    x = _f64(x)
    x2 = x.reshape(-1, x.shape[-1])
    out = np.empty_like(x2)
    lib().orc_mxfp8_rows(_dp(np.ascontiguousarray(x2)), x2.shape[0], x2.shape[1], _dp(out))
    return out.reshape(x.shape)


def mxfp4_rows(x) -> np.ndarray:
    """Rows as MXFP4: E2M1 values with one power-of-two scale per 32 dims."""
    x = _f64(x)
    x2 = np.ascontiguousarray(x.reshape(-1, x.shape[-1]))
    out = np.empty_like(x2)
    lib().orc_store_rows(_dp(x2), x2.shape[0], x2.shape[1], x2.shape[1], 2, _dp(out))
    return out.reshape(x.shape)


def mx_linear(x, w) -> np.ndarray:
    """A projection on the indexer's low-precision path (vastsailsolution.com
    CSA section: the query is first projected down to d_c = 1024, then up to
    the index heads; rqlyzj.com FP4 QAT section and xiaoyuzhoufm.com 2.1: this
    path runs in FP4).  Reading: weights w [N, K] stored MXFP4, activations x
    [M, K] quantised to MXFP8 on the fly, out = x_q . w_q^T summed in fp64."""
    return mxfp8_rows(x) @ mxfp4_rows(w).T


def out_proj(o, w1, w2):
    """Grouped output projection (rqlyzj.com article, section on depth
    compensation): o [T, G*gd] (each row the heads' outputs, group-major),
    w1 [G, r, gd], w2 [hidden, G*r].  Returns (y [T, G*r] rounded to bf16,
    out [T, hidden])."""
    w1 = _f64(w1)
    G, r, gd = w1.shape
    w2 = _f64(w2)
    hidden = w2.shape[0]
    assert w2.shape[1] == G * r
    o = _f64(o).reshape(-1, G * gd)
    T = o.shape[0]
    y = np.empty((T, G * r), dtype=np.float64)
    out = np.empty((T, hidden), dtype=np.float64)
    if T:
        lib().orc_out_proj(_dp(o), T, G, gd, r, _dp(w1), _dp(w2), hidden, _dp(y), _dp(out))
    return y, out


# ---------------------------------------------------------------------------
# the method's index arithmetic (readings of the pages)
# ---------------------------------------------------------------------------
def csa_entry_tokens(j: int, cfg: OCfg):
    """Tokens pooled into CSA entry j: its own m tokens and the w-m tokens before
    them (backward overlap), clipped at position 0."""
    lo = cfg.m_csa * j - (cfg.w_csa - cfg.m_csa)
    return max(0, lo), cfg.m_csa * j + cfg.m_csa


def hca_entry_tokens(j: int, cfg: OCfg):
    return cfg.m_hca * j, cfg.m_hca * (j + 1)


def entry_position(kind: str, j: int, cfg: OCfg) -> int:
    """RoPE position of an entry: the last token of its block."""
    m = cfg.m_csa if kind == "csa" else cfg.m_hca
    return m * j + m - 1


def n_visible(kind: str, t: int, cfg: OCfg) -> int:
    """Entries whose block is complete at position t (last token <= t)."""
    m = cfg.m_csa if kind == "csa" else cfg.m_hca
    return (t + 1) // m


def window_tokens(t: int, cfg: OCfg) -> range:
    """The last W raw tokens including the current one."""
    return range(max(0, t - cfg.window + 1), t + 1)


# ---------------------------------------------------------------------------
# stored objects
# ---------------------------------------------------------------------------
def window_records(kv_tokens, positions, cfg: OCfg) -> np.ndarray:
    """Stored raw-window records of tokens (rows of kv) at the given positions."""
    return store_records(rope(kv_tokens, positions, cfg), cfg)


def entries_from_pool(kind: str, kv, gate, js, cfg: OCfg, token0: int = 0) -> np.ndarray:
    """Stored entries js computed from raw tokens; row i of kv/gate is the token
    at position token0 + i and must cover every pooled token."""
    rng = csa_entry_tokens if kind == "csa" else hca_entry_tokens
    js = list(js)
    first = [rng(j, cfg)[0] - token0 for j in js]
    count = [rng(j, cfg)[1] - rng(j, cfg)[0] for j in js]
    e = pool(kv, gate, first, count)
    pos = [entry_position(kind, j, cfg) for j in js]
    return store_records(rope(e, pos, cfg), cfg)


def index_keys_from_pool(kI, gI, js, cfg: OCfg, token0: int = 0) -> np.ndarray:
    """Compressed index keys: same pooling as CSA entries, no RoPE, FP8 rows."""
    js = list(js)
    first = [csa_entry_tokens(j, cfg)[0] - token0 for j in js]
    count = [csa_entry_tokens(j, cfg)[1] - csa_entry_tokens(j, cfg)[0] for j in js]
    return store_index_rows(pool(kI, gI, first, count), cfg)


def entries_from_values(kind: str, values, js, cfg: OCfg) -> np.ndarray:
    """Stored entries for directly supplied pre-RoPE entry vectors."""
    pos = [entry_position(kind, j, cfg) for j in js]
    return store_records(rope(values, pos, cfg), cfg)


# ---------------------------------------------------------------------------
# one query
# ---------------------------------------------------------------------------
def query_rot(q, t: int, cfg: OCfg) -> np.ndarray:
    """Query heads (H x d) rotated at position t in fp64 (no storage rounding)."""
    return rope(q, t, cfg)


def csa_select(t: int, qI, w, keys_stored, cfg: OCfg):
    """Indexer + top-k for query position t over the visible stored keys."""
    n = n_visible("csa", t, cfg)
    q_st = store_index_rows(qI, cfg)
    w = np.ones(cfg.idx_heads) if w is None else w
    s = index_scores(q_st, w, keys_stored[:n])
    return topk(s, cfg.topk), s


def csa_query(t: int, q, qI, w, sinks, entries_stored, keys_stored, window_of, cfg: OCfg,
              return_scores: bool = False):
    """Output (H x d) and top-k indices of CSA query at position t.

    window_of(s) returns the stored record of raw token s."""
    idx, s = csa_select(t, qI, w, keys_stored, cfg)
    sel = [int(j) for j in idx if j >= 0]
    win = [window_of(u) for u in window_tokens(t, cfg)]
    recs = np.concatenate([entries_stored[sel].reshape(-1, cfg.d)] +
                          [np.asarray(win).reshape(-1, cfg.d)])
    o = attend(query_rot(q, t, cfg), sinks, recs, cfg.tau)
    return (o, idx, s) if return_scores else (o, idx)


def hca_query(t: int, q, sinks, entries_stored, window_of, cfg: OCfg):
    n = n_visible("hca", t, cfg)
    win = [window_of(u) for u in window_tokens(t, cfg)]
    recs = np.concatenate([entries_stored[:n].reshape(-1, cfg.d), np.asarray(win).reshape(-1, cfg.d)])
    return attend(query_rot(q, t, cfg), sinks, recs, cfg.tau)


# ---------------------------------------------------------------------------
# a whole layer over one sequence starting at position 0 (token level)
# ---------------------------------------------------------------------------
def csa_layer(kv, gate, kI, gI, q, qI, w, sinks, query_positions, cfg: OCfg):
    """kv, gate: T x d; kI, gI: T x idx_dim; q[t]: H x d; qI[t]: H_I x idx_dim;
    w[t]: H_I.  Returns outputs [len(query_positions), H, d] and top-k lists."""
    T = kv.shape[0]
    nE = T // cfg.m_csa
    ents = entries_from_pool("csa", kv, gate, range(nE), cfg)
    keys = index_keys_from_pool(kI, gI, range(nE), cfg)
    win = window_records(kv, np.arange(T), cfg)
    outs, idxs = [], []
    for i, t in enumerate(query_positions):
        o, idx = csa_query(t, q[i], qI[i], None if w is None else w[i], sinks, ents, keys,
                           lambda u: win[u], cfg)
        outs.append(o)
        idxs.append(idx)
    return np.stack(outs), np.stack(idxs)


def hca_layer(kv, gate, q, sinks, query_positions, cfg: OCfg):
    T = kv.shape[0]
    nE = T // cfg.m_hca
    ents = entries_from_pool("hca", kv, gate, range(nE), cfg)
    win = window_records(kv, np.arange(T), cfg)
    return np.stack([hca_query(t, q[i], sinks, ents, lambda u: win[u], cfg)
                     for i, t in enumerate(query_positions)])
