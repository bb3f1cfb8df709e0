"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds workload shapes and random-number generation only; it does
none of the method's arithmetic.  Both the CPU oracle (through the tests and
the benchmark's CPU leg) and the HIP path consume the arrays it returns.

Every tensor is drawn from ``numpy.random.default_rng([workload_id, tensor_id])``
so that any consumer can regenerate exactly the same values.  Activations are
returned as float32; a consumer that feeds bf16 to the GPU rounds them with
torch and hands the same rounded values to the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids (second seed word)
T_X, T_WQ, T_WKV, T_WG, T_WQI, T_WW, T_WKI, T_WGI = range(8)
T_SINK, T_Q, T_QI, T_W, T_KV, T_GATE, T_KI, T_GI = range(8, 16)
T_ENT, T_KEY, T_WIN, T_PERM = range(16, 20)


@dataclass
class Workload:
    wid: int
    name: str
    d: int = 512
    d_rope: int = 64
    n_heads: int = 128
    window: int = 128
    m_csa: int = 4
    w_csa: int = 8
    m_hca: int = 128
    idx_heads: int = 64
    idx_dim: int = 128
    topk: int = 1024
    batch: int = 1
    ctx: list = field(default_factory=list)      # tokens already cached per request
    hidden: int = 0
    chunk: int = 0
    act: str = "bf16"
    store: str = "fp8"

    def shape(self) -> dict:
        return dict(d=self.d, d_rope=self.d_rope, n_heads=self.n_heads, window=self.window,
                    m_csa=self.m_csa, w_csa=self.w_csa, m_hca=self.m_hca,
                    idx_heads=self.idx_heads, idx_dim=self.idx_dim, topk=self.topk)


# The five workloads: a tiny CSA layer (prefill + decode), HCA decode at 64K,
# CSA decode at the V4-Pro shape at 128K, a CSA prefill chunk on a 256K prefix,
# and a mixed-length CSA+HCA layer pair reaching 1M tokens.
TINY_CSA = Workload(1, "tiny_csa_1k", d=64, d_rope=16, n_heads=8, window=16, idx_heads=4,
                    idx_dim=32, topk=32, batch=1, ctx=[1024], hidden=256, act="f32", store="fp32")
HCA_DECODE_64K = Workload(2, "hca_decode_b16_64k", batch=16, ctx=[65536] * 16)
CSA_DECODE_128K = Workload(3, "csa_decode_b32_128k", batch=32, ctx=[131072] * 32)
CSA_PREFILL_8K = Workload(4, "csa_prefill_8k_on_256k", topk=512, batch=1, ctx=[262144],
                          hidden=7168, chunk=8192)
PAIR_DECODE_1M = Workload(5, "csa_hca_pair_decode_1m_mixed", batch=4,
                          ctx=[1048576, 524288, 65536, 4096])

ALL = [TINY_CSA, HCA_DECODE_64K, CSA_DECODE_128K, CSA_PREFILL_8K, PAIR_DECODE_1M]


def rng(wid: int, tid: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([wid, tid, sub])


def normal(wid: int, tid: int, shape, std: float = 1.0, sub: int = 0) -> np.ndarray:
    a = rng(wid, tid, sub).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def sinks(w: Workload) -> np.ndarray:
    """Per-head sink logits ~ N(0, 1)."""
    return normal(w.wid, T_SINK, (w.n_heads,))


def decode_queries(w: Workload, n: int, sub: int = 0):
    """q [n, H, d] ~ N(0,1); index queries qI [n, H_I, d_I] ~ N(0,1);
    index head weights w [n, H_I] ~ N(0, 1/H_I)."""
    q = normal(w.wid, T_Q, (n, w.n_heads, w.d), sub=sub)
    qI = normal(w.wid, T_QI, (n, w.idx_heads, w.idx_dim), sub=sub)
    wt = normal(w.wid, T_W, (n, w.idx_heads), std=1.0 / np.sqrt(w.idx_heads), sub=sub)
    return q, qI, wt


def new_tokens(w: Workload, n: int, sub: int = 0):
    """Raw per-token compressor inputs: kv, gate [n, d]; kI, gI [n, d_I]."""
    kv = normal(w.wid, T_KV, (n, w.d), sub=sub)
    gate = normal(w.wid, T_GATE, (n, w.d), sub=sub)
    kI = normal(w.wid, T_KI, (n, w.idx_dim), sub=sub)
    gI = normal(w.wid, T_GI, (n, w.idx_dim), sub=sub)
    return kv, gate, kI, gI


def entries(w: Workload, req: int, n: int, kind: int = 0) -> np.ndarray:
    """Pre-RoPE compressed-entry vectors [n, d] ~ N(0,1) for request req
    (kind 0: CSA layer, 1: HCA layer)."""
    return normal(w.wid, T_ENT, (n, w.d), sub=2 * req + kind)


def index_keys(w: Workload, req: int, n: int) -> np.ndarray:
    """Compressed index-key vectors [n, d_I] ~ N(0,1)."""
    return normal(w.wid, T_KEY, (n, w.idx_dim), sub=req)


def clustered_index_keys(w: Workload, req: int, n: int, qI: np.ndarray, runs: int = 64,
                         run_len: int = 16) -> np.ndarray:
    """Index keys with `runs` runs of `run_len` contiguous entries correlated with
    the request's first index-query head (retrieval-like locality and margin)."""
    k = index_keys(w, req, n)
    g = rng(w.wid, T_KEY, 1000 + req)
    starts = g.choice(max(1, n // run_len), size=min(runs, max(1, n // run_len)), replace=False) * run_len
    for s in starts:
        e = min(n, s + run_len)
        k[s:e] = 0.5 * k[s:e] + 2.0 * qI[0][None, :]
    return k


def window_tokens(w: Workload, req: int, n: int, kind: int = 0):
    """Raw tokens of a prefix tail (kv, gate, kI, gI) for the state cache."""
    sub = 2 * req + kind
    return (normal(w.wid, T_WIN, (n, w.d), sub=sub),
            normal(w.wid, T_WIN, (n, w.d), sub=100000 + sub),
            normal(w.wid, T_WIN, (n, w.idx_dim), sub=200000 + sub),
            normal(w.wid, T_WIN, (n, w.idx_dim), sub=300000 + sub))


def tiny_hidden(w: Workload = TINY_CSA, steps: int = 16):
    """Tiny layer: hidden states x [T, hidden] ~ N(0,1) and projection weights
    ~ N(0, 1/hidden) for q, kv, gate, qI, w, kI, gI (the projections themselves
    run outside the library)."""
    T = w.ctx[0] + steps
    h = w.hidden
    s = 1.0 / np.sqrt(h)
    return dict(
        x=normal(w.wid, T_X, (T, h)),
        Wq=normal(w.wid, T_WQ, (h, w.n_heads * w.d), std=s),
        Wkv=normal(w.wid, T_WKV, (h, w.d), std=s),
        Wg=normal(w.wid, T_WG, (h, w.d), std=s),
        WqI=normal(w.wid, T_WQI, (h, w.idx_heads * w.idx_dim), std=s),
        Ww=normal(w.wid, T_WW, (h, w.idx_heads), std=s),
        WkI=normal(w.wid, T_WKI, (h, w.idx_dim), std=s),
        WgI=normal(w.wid, T_WGI, (h, w.idx_dim), std=s),
        sinks=sinks(w),
    )


def permutation(wid: int, n: int, sub: int = 0) -> np.ndarray:
    return rng(wid, T_PERM, sub).permutation(n)


T_SCORE = 20
SCORE_KINDS = ("normal", "ties", "crowded", "constant", "special", "allnan", "wide", "huge")


def score_row(kind: str, n: int, seed: int) -> np.ndarray:
    """A float32 row of n scores for the selection tests: 'normal' N(0,1);
    'ties' integers 0..49; 'crowded' integers 0..2; 'constant' all 1.5;
    'special' N(0,1) with NaN, +-inf and +-0 sprinkled in; 'allnan';
    'wide' log-normal with sigma 10 (a huge dynamic range); 'huge' values near
    +-3e38 (their range overflows fp32)."""
    g = np.random.default_rng([0, T_SCORE, SCORE_KINDS.index(kind), seed])
    if kind == "normal":
        x = g.standard_normal(n)
    elif kind == "ties":
        x = g.integers(0, 50, n).astype(np.float64)
    elif kind == "crowded":
        x = g.integers(0, 3, n).astype(np.float64)
    elif kind == "constant":
        x = np.full(n, 1.5)
    elif kind == "special":
        x = g.standard_normal(n)
        u = g.random(n)
        x[u < 0.10] = np.nan
        x[(u >= 0.10) & (u < 0.12)] = np.inf
        x[(u >= 0.12) & (u < 0.14)] = -np.inf
        x[(u >= 0.14) & (u < 0.17)] = 0.0
        x[(u >= 0.17) & (u < 0.20)] = -0.0
    elif kind == "allnan":
        x = np.full(n, np.nan)
    elif kind == "wide":
        x = g.lognormal(0.0, 10.0, n) * np.where(g.random(n) < 0.3, -1.0, 1.0)
    elif kind == "huge":
        x = np.where(g.random(n) < 0.5, -3e38, 3e38) * g.uniform(0.5, 1.0, n)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)
