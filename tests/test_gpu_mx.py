"""GPU parity of the indexer's low-precision linear layers (MXFP4 weights,
MXFP8 activations) against the CPU oracle, through the C ABI.

Tolerances, from the arithmetic: both sides quantise the same bf16 values with
the same rules, so the codes and scales agree exactly (checked directly on the
packed weights) and the products of codes are exact; what differs is only the
summation -- the matrix cores' against the oracle's fp64.  One scaled 128-term
step of the matrix core lands within about 1.2e-4 of the step's sum of
|products| from the exact sum (measured on single instructions with random
E4M3 / E2M1 codes and scales: the instruction's internal rounding, coarser than
a sequential fp32 sum), and the steps are added in fp32.  So |gpu - ref| is
held below 2^-12 of sum_k |x_q w_q|.  Where the GPU rounds to bf16 (the query path's d_c summary) the two
agree exactly except near a rounding boundary."""
import numpy as np
import pytest
import torch

from long_context_compressed_02_amd import binding as B
from long_context_compressed_02_amd import synth
from oracle import oracle as O
from tests import helpers as Hh

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2.0 ** -12


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def _f64(t):
    return t.to(torch.float64).cpu().numpy()


def _pack(w):
    N, K = w.shape
    wp = torch.empty(B.dsv4_mx_pack_bytes(N, K, False), dtype=torch.uint8, device=DEV)
    B.dsv4_mx_pack_weight(w, wp)
    return wp


def _linear(x, wp, N, out_dtype=torch.float32):
    M, K = x.shape
    ws = torch.empty(max(B.dsv4_mx_pack_bytes(M, K, True), 256), dtype=torch.uint8, device=DEV)
    out = torch.empty((M, N), dtype=out_dtype, device=DEV)
    B.dsv4_mx_linear(x, wp, N, ws, out)
    torch.cuda.synchronize()
    return out


def _check_f32(out, x, w, rows=None):
    """out fp32 against the oracle in fp64 with the summation bound above."""
    xs = _f64(x) if rows is None else _f64(x[rows])
    ref = O.mx_linear(xs, _f64(w))
    mag = np.abs(O.mxfp8_rows(xs)) @ np.abs(O.mxfp4_rows(_f64(w))).T
    g = _f64(out) if rows is None else _f64(out[rows])
    err = np.abs(g - ref)
    bad = err > TOL * mag + 1e-37
    print(f"  max err / bound {np.max(err / (TOL * mag + 1e-37)):.3f}", flush=True)
    assert not bad.any(), (np.argwhere(bad)[:5], g[bad][:5], ref[bad][:5])


def test_mx_weight_pack_layout():
    """The packed MXFP4 weights decode, through the documented layout, to exactly
    the oracle's MXFP4 rows (codes, nibble order and scales)."""
    g = np.random.default_rng(3)
    N, K = 48, 384                                   # 3 row blocks, 3 k-steps (a partial group of 4)
    w = g.standard_normal((N, K)).astype(np.float32) * g.lognormal(0, 2, (N, 1)).astype(np.float32)
    w[5] = 0.0                                        # a zero row
    w[7, 40:72] *= 1e-30                              # tiny blocks
    wt = _bf16(w)
    wp = _pack(wt).cpu().numpy()
    nks, nq = K // 128, (K // 128 + 3) // 4
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    dec = np.zeros((N, K))
    code_bytes = (N // 16) * nks * 1024
    for rb in range(N // 16):
        for ks in range(nks):
            for lane in range(64):
                n, k0 = 16 * rb + lane % 16, 128 * ks + 32 * (lane // 16)
                by = wp[(rb * nks + ks) * 1024 + 16 * lane:][:16]
                sc = wp[code_bytes + (rb * nq + ks // 4) * 256 + 4 * lane + ks % 4]
                for i in range(16):
                    for half in range(2):
                        c = (by[i] >> (4 * half)) & 15
                        v = (-1.0 if c & 8 else 1.0) * mags[c & 7]
                        dec[n, k0 + 2 * i + half] = v * 2.0 ** (int(sc) - 127)
    assert np.array_equal(dec, O.mxfp4_rows(_f64(wt)))


@pytest.mark.parametrize("N", [48, 256])
@pytest.mark.parametrize("K", [128, 384, 1024])
def test_mx_linear_small_ragged(K, N):
    # N = 48: 3 column blocks, a ragged column tile of the 128x128 tiling;
    # N = 256: above 64 rows the 256x256 LDS-staged tiling (one, three or
    # eight k-steps; 257 and 300 rows: a ragged second row tile)
    g = np.random.default_rng([5, K, N])
    w = _bf16(g.standard_normal((N, K)) / np.sqrt(K))
    wp = _pack(w)
    for M in (1, 20, 37, 64, 256, 257, 300):          # every tiling and quantiser split, ragged rows
        x = g.standard_normal((M, K)).astype(np.float32) * g.lognormal(0, 2, (M, 1)).astype(np.float32)
        x[M // 2] = 0.0                               # a zero row
        if M > 2:
            x[1, :32] *= 1e30                         # saturating / extreme blocks
            x[2, 32:64] *= 1e-30
        xt = _bf16(x)
        out = _linear(xt, wp, N)
        _check_f32(out, xt, w)
        assert (out[M // 2] == 0).all()


@pytest.mark.parametrize("M, N, K", [(1300, 256, 384), (4100, 4096, 128)])
def test_mx_linear_lds_tile_groups(M, N, K):
    # The LDS-staged tilings over several groups of four row tiles (the XCD
    # tile order), the last row tile ragged: 1300 x 256 takes 256x128 tiles
    # (12 of them, too few for 256-wide ones), 4100 x 4096 the 256x256 tiles
    # (17 x 16 = 272 of them).  Every row against the oracle; the last 100
    # rows bitwise the same in a launch of their own (the 64-row tilings).
    g = np.random.default_rng([8, M, N])
    w = _bf16(g.standard_normal((N, K)) / np.sqrt(K))
    wp = _pack(w)
    x = _bf16(g.standard_normal((M, K)) * g.lognormal(0, 1, (M, 1)))
    print(f"mx_linear LDS tile groups M={M} N={N} K={K}", flush=True)
    out = _linear(x, wp, N)
    _check_f32(out, x, w)
    tail = _linear(x[M - 100:].contiguous(), wp, N)
    assert torch.equal(tail.view(torch.int32), out[M - 100:].view(torch.int32))


def test_mx_linear_batch_invariance_and_bf16_out():
    g = np.random.default_rng(9)
    N, K = 256, 1024
    w = _bf16(g.standard_normal((N, K)) / 32)
    wp = _pack(w)
    x = _bf16(g.standard_normal((300, K)))
    big = _linear(x, wp, N)
    for M, off in ((1, 17), (20, 100), (64, 200)):
        part = _linear(x[off:off + M].contiguous(), wp, N)
        assert torch.equal(part.view(torch.int32), big[off:off + M].view(torch.int32)), M
    # bf16 output: the fp32 result rounded to nearest even
    bo = _linear(x, wp, N, torch.bfloat16)
    assert torch.equal(bo.view(torch.int16), big.to(torch.bfloat16).view(torch.int16))


def test_mx_linear_argument_checks():
    w = torch.zeros((48, 256), dtype=torch.bfloat16, device=DEV)
    wp = _pack(w)
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(B.dsv4_mx_pack_bytes(4, 256, True), dtype=torch.uint8, device=DEV)
    out = torch.empty((4, 48), dtype=torch.float32, device=DEV)
    for bad_k in (200, 0):                                    # K not a positive multiple of 128
        st = B.lib().dsv4_mx_linear(x.data_ptr(), 4, bad_k, wp.data_ptr(), 48, ws.data_ptr(), ws.numel(),
                                    out.data_ptr(), B.DSV4_DT_F32, None)
        assert st == B.DSV4_ERR_INVALID_ARG
    st = B.lib().dsv4_mx_linear(x.data_ptr(), 4, 256, wp.data_ptr(), 40, ws.data_ptr(), ws.numel(), out.data_ptr(),
                                B.DSV4_DT_F32, None)
    assert st == B.DSV4_ERR_INVALID_ARG                       # N not a multiple of 16
    st = B.lib().dsv4_mx_linear(x.data_ptr(), 4, 256, wp.data_ptr(), 48, ws.data_ptr(), ws.numel() - 1,
                                out.data_ptr(), B.DSV4_DT_F32, None)
    assert st == B.DSV4_ERR_WORKSPACE
    st = B.lib().dsv4_mx_linear(x.data_ptr(), 4, 256, wp.data_ptr(), 48, ws.data_ptr() + 16, ws.numel(),
                                out.data_ptr(), B.DSV4_DT_F32, None)
    assert st == B.DSV4_ERR_WORKSPACE                         # misaligned workspace
    assert B.lib().dsv4_mx_linear(x.data_ptr(), 0, 256, wp.data_ptr(), 48, None, 0, None, B.DSV4_DT_F32,
                                  None) == B.DSV4_OK            # empty batch
    torch.cuda.synchronize()


def _q_proj(cfg, x, dc, wdq_p, wuq_p, act):
    T, hidden = x.shape
    ws = torch.empty(B.dsv4_index_q_proj_ws_bytes(cfg, T, hidden, dc), dtype=torch.uint8, device=DEV)
    qI = torch.empty((T, cfg.idx_heads, cfg.idx_dim), dtype=act, device=DEV)
    B.dsv4_index_q_proj(cfg, x, dc, wdq_p, wuq_p, ws, qI)
    torch.cuda.synchronize()
    cq = ws[: T * dc * 2].view(torch.bfloat16).view(T, dc)
    return cq, qI


def _check_q_proj(x, cq, qI, wdq, wuq, rows):
    """Stage 1: the GPU's bf16 summary against the oracle's fp64 sum: equal to it
    rounded to bf16 but for a few elements near a rounding boundary (or, after
    cancellation, near zero), and always within half a bf16 step plus the
    summation bound.  Stage 2 from the GPU's summary
    (so a one-step difference upstream does not blur it): the summation bound."""
    xs = _f64(x[rows])
    ref1 = O.mx_linear(xs, _f64(wdq))
    ref1b = torch.from_numpy(ref1).to(torch.bfloat16).to(torch.float64).numpy()
    c = _f64(cq[rows])
    diff = c != ref1b
    assert diff.mean() <= 1e-2, diff.mean()
    # the GPU's sum within the summation bound, then rounded to bf16 (half a step)
    assert (np.abs(c - ref1) <= 2.0 ** -8 * np.abs(ref1) + TOL * (np.abs(O.mxfp8_rows(xs)) @
                                                                      np.abs(O.mxfp4_rows(_f64(wdq))).T)).all()
    q = _f64(qI[rows]).reshape(len(rows), -1)
    ref2 = O.mx_linear(c, _f64(wuq))
    mag = np.abs(O.mxfp8_rows(c)) @ np.abs(O.mxfp4_rows(_f64(wuq))).T
    ratio = np.abs(q - ref2) / (TOL * mag + 1e-37)
    print(f"  summaries differing: {diff.sum()} of {diff.size}; stage-2 err / bound {ratio.max():.3f}", flush=True)
    assert ratio.max() <= 1.0


def test_index_q_proj_tiny():
    """Tiny indexer (4 heads x 32) on hidden 256 -> d_c 128, both tilings."""
    cfg, oc = Hh.cfgs(dict(synth.TINY_CSA.shape()), act=B.DSV4_DT_F32)
    assert (oc.idx_heads, oc.idx_dim) == (4, 32)
    hidden, dc = 256, 128
    g = np.random.default_rng(11)
    wdq = _bf16(g.standard_normal((dc, hidden)) / 16)
    wuq = _bf16(g.standard_normal((4 * 32, dc)) / 11)
    wdq_p, wuq_p = _pack(wdq), _pack(wuq)
    for T in (3, 100):
        x = _bf16(g.standard_normal((T, hidden)))
        cq, qI = _q_proj(cfg, x, dc, wdq_p, wuq_p, torch.float32)
        _check_q_proj(x, cq, qI, wdq, wuq, list(range(T)))


def test_index_q_proj_production_shape():
    """x [T, 7168] -> d_c 1024 -> 64 x 128, at a decode batch (32) and a prefill
    chunk (8192 tokens, sampled rows), and bitwise the same for the same tokens
    in both."""
    cfg, oc = Hh.cfgs(dict(synth.CSA_DECODE_128K.shape()), act=B.DSV4_DT_F32)
    hidden, dc = 7168, 1024
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    wdq = (torch.randn((dc, hidden), generator=g, device=DEV) / hidden ** 0.5).to(torch.bfloat16)
    wuq = (torch.randn((cfg.idx_heads * cfg.idx_dim, dc), generator=g, device=DEV) / dc ** 0.5).to(torch.bfloat16)
    wdq_p, wuq_p = _pack(wdq), _pack(wuq)
    x = torch.randn((8192, hidden), generator=g, device=DEV).to(torch.bfloat16)
    cq, qI = _q_proj(cfg, x, dc, wdq_p, wuq_p, torch.float32)
    rows = [0, 1, 777, 4096, 8191]
    _check_q_proj(x, cq, qI, wdq, wuq, rows)
    cq_s, qI_s = _q_proj(cfg, x[4000:4032].contiguous(), dc, wdq_p, wuq_p, torch.float32)
    _check_q_proj(x[4000:4032], cq_s, qI_s, wdq, wuq, [0, 31])
    assert torch.equal(qI_s.view(torch.int32), qI[4000:4032].view(torch.int32))
    assert torch.equal(cq_s.view(torch.int16), cq[4000:4032].view(torch.int16))
    # bf16 query output (the act dtype the scorer takes at bf16): the fp32 result rounded
    cfgb, _ = Hh.cfgs(dict(synth.CSA_DECODE_128K.shape()), act=B.DSV4_DT_BF16)
    _, qIb = _q_proj(cfgb, x[4000:4032].contiguous(), dc, wdq_p, wuq_p, torch.bfloat16)
    assert torch.equal(qIb.view(torch.int16), qI_s.to(torch.bfloat16).view(torch.int16))


def test_index_q_proj_feeds_the_indexer():
    """The query path's output, in its [T][heads][dims] bf16 layout, is what the
    decode indexer takes: the top-k of the path's queries equals the oracle's
    selection computed from the same queries (read back) over the same keys."""
    k = 1024
    shape = dict(synth.CSA_DECODE_128K.shape())
    cfg, oc = Hh.cfgs(shape, topk=k)                          # bf16 activations, FP8 index rows
    ctx = [5000, 40001]
    bt, nb, mb = Hh.block_table(ctx, extra_blocks=3, seed=4)
    cache = B.LayerCache(cfg, B.DSV4_CSA, len(ctx), mb, nb, bt)
    keys = []
    for r, c in enumerate(ctx):
        n = c // 4
        kv = synth.index_keys(synth.CSA_DECODE_128K, 70 + r, n)[:n]
        keys.append(O.store_index_rows(kv, oc))
        B.dsv4_cache_write_entries(cfg, cache, B.DSV4_TARGET_INDEX_KEY, Hh.i32([r] * n), Hh.i32(range(n)),
                                   torch.from_numpy(kv).to(DEV))
    hidden, dc = 7168, 1024
    g = torch.Generator(device=DEV)
    g.manual_seed(23)
    wdq = (torch.randn((dc, hidden), generator=g, device=DEV) / hidden ** 0.5).to(torch.bfloat16)
    wuq = (torch.randn((oc.idx_heads * oc.idx_dim, dc), generator=g, device=DEV) / dc ** 0.5).to(torch.bfloat16)
    x = torch.randn((len(ctx), hidden), generator=g, device=DEV).to(torch.bfloat16)
    _, qI = _q_proj(cfg, x, dc, _pack(wdq), _pack(wuq), torch.bfloat16)
    w = torch.rand((len(ctx), oc.idx_heads), generator=g, device=DEV) / 8
    out = torch.empty((len(ctx), k), dtype=torch.int32, device=DEV)
    ws = torch.empty(B.dsv4_workspace_bytes(cfg, len(ctx), cache.c.max_blocks * 32), dtype=torch.uint8, device=DEV)
    pos = [c - 1 for c in ctx]
    B.dsv4_index_topk_decode(cfg, cache, qI, w, Hh.i32(range(len(ctx))), Hh.i32(pos), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    qx = qI.to(torch.float64).cpu().numpy()
    wx = w.to(torch.float64).cpu().numpy()
    swaps = 0
    for r in range(len(ctx)):
        idx, s = O.csa_select(pos[r], qx[r], wx[r], keys[r], oc)
        swaps += Hh.topk_match(got[r], idx, s, k)
    assert swaps <= 2


# ------------------------------------------------------------------ projections feeding the compressors
def _kv_proj_case(shape, T, hidden, seed, kind=B.DSV4_CSA, with_w=True):
    cfg, oc = Hh.cfgs(shape)
    g = np.random.default_rng([31, seed])
    s = 1.0 / np.sqrt(hidden)
    csa = kind == B.DSV4_CSA
    W = {"kv": _bf16(g.standard_normal((oc.d, hidden)) * s), "g": _bf16(g.standard_normal((oc.d, hidden)) * s)}
    if csa:
        W["kI"] = _bf16(g.standard_normal((oc.idx_dim, hidden)) * s)
        W["gI"] = _bf16(g.standard_normal((oc.idx_dim, hidden)) * s)
        if with_w:
            W["w"] = _bf16(g.standard_normal((oc.idx_heads, hidden)) * s / 8)
    P = {k: _pack(v) for k, v in W.items()}
    x = _bf16(g.standard_normal((T, hidden)))
    return cfg, oc, W, P, x


def _kv_proj(cfg, kind, x, P, oc):
    T, hidden = x.shape
    csa = kind == B.DSV4_CSA
    out = {"kv": torch.empty((T, oc.d), dtype=torch.bfloat16, device=DEV),
           "g": torch.empty((T, oc.d), dtype=torch.bfloat16, device=DEV)}
    if csa:
        out["kI"] = torch.empty((T, oc.idx_dim), dtype=torch.bfloat16, device=DEV)
        out["gI"] = torch.empty((T, oc.idx_dim), dtype=torch.bfloat16, device=DEV)
        if "w" in P:
            out["w"] = torch.empty((T, oc.idx_heads), dtype=torch.float32, device=DEV)
    ws = torch.empty(B.dsv4_kv_proj_ws_bytes(cfg, T, hidden), dtype=torch.uint8, device=DEV)
    B.dsv4_kv_proj(cfg, kind, x, P["kv"], P["g"], P.get("kI"), P.get("gI"), P.get("w"), out["kv"], out["g"],
                   out.get("kI"), out.get("gI"), out.get("w"), ws)
    torch.cuda.synchronize()
    return out


def _check_bf16(out, x, w):
    """bf16 outputs: the fp32 result (within the summation bound) rounded to
    nearest even -- at most half a bf16 step (2^-8 of the value) more."""
    xs = _f64(x)
    ref = O.mx_linear(xs, _f64(w))
    mag = np.abs(O.mxfp8_rows(xs)) @ np.abs(O.mxfp4_rows(_f64(w))).T
    err = np.abs(_f64(out) - ref)
    bound = TOL * mag + 2.0 ** -8 * (np.abs(ref) + TOL * mag) + 1e-37
    print(f"  max err / bound {np.max(err / bound):.3f}", flush=True)
    assert (err <= bound).all()


@pytest.mark.parametrize("kind", [B.DSV4_CSA, B.DSV4_HCA], ids=["csa", "hca"])
def test_kv_proj_production_shape(kind):
    """V4-Pro widths (hidden 7168 -> kv, gate 512; kI, gI 128; w 64 heads) on
    MXFP4 weights and MXFP8 activations against the oracle's MX linear map; a
    token's outputs are the same bytes alone and inside the batch."""
    shape = synth.CSA_DECODE_128K.shape()
    T, hidden = 300, 7168
    cfg, oc, W, P, x = _kv_proj_case(shape, T, hidden, 1, kind)
    out = _kv_proj(cfg, kind, x, P, oc)
    for k, o in out.items():
        print(f"  {k}:", end="", flush=True)
        if k == "w":
            _check_f32(o, x, W[k])
        else:
            _check_bf16(o, x, W[k])
    for M, off in ((1, 0), (32, 100), (7, 293)):
        part = _kv_proj(cfg, kind, x[off:off + M].contiguous(), P, oc)
        for k in out:
            assert torch.equal(part[k].view(torch.int16), out[k][off:off + M].view(torch.int16)), (k, M)


def test_kv_proj_feeds_the_compressor_and_indexer():
    """The projections' outputs go straight into the compressor (prefill of a
    300-token chunk, then one decode step) and the decode indexer: the cache
    holds the same bytes as when the same values come from the host, its
    entries and index keys are the oracle's compression of those values (up to
    rounding-boundary flips), and the top-k equals the oracle's selection with
    the projected head weights."""
    shape = dict(synth.CSA_DECODE_128K.shape())
    T, hidden = 301, 1024
    cfg, oc, W, P, x = _kv_proj_case(shape, T, hidden, 2)
    out = _kv_proj(cfg, B.DSV4_CSA, x, P, oc)
    C = T - 1
    bt, nb, mb = Hh.block_table([T], seed=11)
    caches = [B.LayerCache(cfg, B.DSV4_CSA, 1, mb, nb, bt) for _ in range(2)]
    feeds = [out, {k: v.cpu().to(DEV) for k, v in out.items()}]   # the same values through host memory
    cu, r0, p0 = Hh.i32([0, C]), Hh.i32([0]), Hh.i32([0])
    for cache, f in zip(caches, feeds):
        win = torch.empty((C + oc.window) * cache.layout.record_bytes, dtype=torch.uint8, device=DEV)
        B.dsv4_compress_kv_prefill(cfg, cache, f["kv"][:C].contiguous(), f["g"][:C].contiguous(),
                                   f["kI"][:C].contiguous(), f["gI"][:C].contiguous(), cu, r0, p0, C, win)
        B.dsv4_compress_kv_decode(cfg, cache, f["kv"][C:], f["g"][C:], f["kI"][C:], f["gI"][C:], r0, Hh.i32([C]))
    torch.cuda.synchronize()
    for a in ("entries", "index_keys", "state"):
        assert torch.equal(getattr(caches[0], a), getattr(caches[1], a)), a
    vals = {k: _f64(v) for k, v in out.items()}
    ne = T // oc.m_csa
    ents = O.entries_from_pool("csa", vals["kv"], vals["g"], range(ne), oc)
    keys = O.index_keys_from_pool(vals["kI"], vals["gI"], range(ne), oc)
    Hh.assert_records_close(Hh.read_back(cfg, caches[0], B.DSV4_TARGET_ENTRY, 0, range(ne)), ents, oc.d_rope)
    keys_gpu = Hh.read_back(cfg, caches[0], B.DSV4_TARGET_INDEX_KEY, 0, range(ne))
    Hh.assert_records_close(keys_gpu, keys, 0)
    # the indexer of the last token with the projected head weights
    _, qI, _ = synth.decode_queries(synth.CSA_DECODE_128K, 1, sub=77)
    qIt, qIx = Hh.act_tensor(qI, B.DSV4_DT_BF16)
    oc_k = O.OCfg(**{**shape, "topk": 32})
    cfg_k, _ = Hh.cfgs(shape, topk=32)
    ws = torch.empty(B.dsv4_workspace_bytes(cfg_k, 1, mb * 32), dtype=torch.uint8, device=DEV)
    tk = torch.empty((1, 32), dtype=torch.int32, device=DEV)
    B.dsv4_index_topk_decode(cfg_k, caches[0], qIt, out["w"][C:].contiguous(), r0, Hh.i32([C]), tk, ws)
    torch.cuda.synchronize()
    idx, s = O.csa_select(C, qIx[0], vals["w"][C], keys_gpu, oc_k)
    Hh.topk_match(tk.cpu().numpy()[0], idx, s, 32)


def test_kv_proj_argument_checks():
    shape = synth.CSA_DECODE_128K.shape()
    cfg, oc, W, P, x = _kv_proj_case(shape, 4, 256, 3)
    ws = torch.empty(B.dsv4_kv_proj_ws_bytes(cfg, 4, 256), dtype=torch.uint8, device=DEV)
    o = {k: torch.empty((4, 512), dtype=torch.bfloat16, device=DEV) for k in ("kv", "g", "kI", "gI")}
    wout = torch.empty((4, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(B.Dsv4Error):          # HCA takes no index-key projections
        B.dsv4_kv_proj(cfg, B.DSV4_HCA, x, P["kv"], P["g"], P["kI"], P["gI"], None, o["kv"], o["g"], o["kI"],
                       o["gI"], None, ws)
    with pytest.raises(B.Dsv4Error):          # CSA needs them
        B.dsv4_kv_proj(cfg, B.DSV4_CSA, x, P["kv"], P["g"], None, None, None, o["kv"], o["g"], None, None, None, ws)
    with pytest.raises(B.Dsv4Error):          # head weights need both the packed weight and the output
        B.dsv4_kv_proj(cfg, B.DSV4_CSA, x, P["kv"], P["g"], P["kI"], P["gI"], P["w"], o["kv"], o["g"], o["kI"],
                       o["gI"], None, ws)
    with pytest.raises(B.Dsv4Error):          # a short workspace
        B.dsv4_kv_proj(cfg, B.DSV4_CSA, x, P["kv"], P["g"], P["kI"], P["gI"], P["w"], o["kv"], o["g"], o["kI"],
                       o["gI"], wout, ws[:128])
