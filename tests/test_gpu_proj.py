"""GPU parity of the grouped output projection against the CPU oracle (through
the C ABI), and its batch invariance: a token's output is bitwise the same
alone, in a decode-sized batch and in a prefill-sized batch (the two tilings).

Tolerance, from the arithmetic: the group summaries are bf16 on both sides --
the GPU rounds its fp32 sum, the oracle its fp64 sum (through fp32) -- so they
agree exactly except where the two sums straddle a rounding boundary, then by
one bf16 step, plus the fp32 sum's own error, at most K * 2^-24 * sum|o w|
over the K = (H/G) d products (it matters where the sum cancels to near
zero).  The output is the GPU's fp32 sum rounded to bf16 (2^-9
relative) against the oracle's fp64 sum: per token, max |gpu - ref| is held
below 2^-7 of the row's largest magnitude."""
import numpy as np
import pytest
import torch

from long_context_compressed_02_amd import binding as B
from oracle import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(T, H, d, G, r, hidden, seed):
    g = np.random.default_rng([31, seed])
    gd = H // G * d
    o = g.standard_normal((T, H, d), dtype=np.float32)
    w1 = g.standard_normal((G, r, gd), dtype=np.float32) / np.float32(np.sqrt(gd))
    w2 = g.standard_normal((hidden, G * r), dtype=np.float32) / np.float32(np.sqrt(G * r))
    bf = lambda a: torch.from_numpy(a).to(DEV).to(torch.bfloat16)
    return bf(o), bf(w1), bf(w2)


_packed = {}


def _run(cfg, G, r, hidden, o, w1, w2):
    key = (w1.data_ptr(), w2.data_ptr())
    if key not in _packed:
        w1p, w2p = torch.empty_like(w1), torch.empty_like(w2)
        B.dsv4_out_proj_pack(cfg, G, r, hidden, w1, w2, w1p, w2p)
        _packed.clear()
        _packed[key] = (w1, w2, w1p, w2p)
    w1p, w2p = _packed[key][2:]
    T = o.shape[0]
    y = torch.empty((T, G * r), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((T, hidden), dtype=torch.bfloat16, device=DEV)
    B.dsv4_out_proj(cfg, G, r, hidden, o, w1p, w2p, y, out)
    torch.cuda.synchronize()
    return y, out


def test_out_proj_pack_layout():
    """The packed order, element by element against the documented formula."""
    cfg = B.make_cfg(d=64, d_rope=16, n_heads=32)
    G, r, hidden = 4, 128, 256
    gd = 32 // G * 64
    w1 = torch.arange(G * r * gd, dtype=torch.int32).remainder(30011).to(torch.bfloat16).view(G, r, gd).to(DEV)
    w2 = torch.arange(hidden * G * r, dtype=torch.int32).remainder(30011).to(torch.bfloat16).view(hidden, G * r).to(DEV)
    w1p, w2p = torch.empty_like(w1), torch.empty_like(w2)
    B.dsv4_out_proj_pack(cfg, G, r, hidden, w1, w2, w1p, w2p)
    torch.cuda.synchronize()
    for W, P in ((w2.cpu(), w2p.cpu().view(-1)), (w1[2].cpu(), w1p[2].cpu().view(-1))):
        N, K = W.shape
        n0, k0, l, e = np.meshgrid(np.arange(0, N, 16), np.arange(0, K, 32), np.arange(64), np.arange(8),
                                   indexing="ij")
        pos = ((n0 // 16) * (K // 32) + k0 // 32) * 512 + 8 * l + e
        ref = W[torch.from_numpy((n0 + l % 16).ravel()), torch.from_numpy((k0 + 8 * (l // 16) + e).ravel())]
        assert torch.equal(P[torch.from_numpy(pos.ravel())], ref)


def _check(y, out, o, w1, w2, rows):
    f64 = lambda t: t.to(torch.float64).cpu().numpy()
    yr, outr = O.out_proj(f64(o[rows]).reshape(len(rows), -1), f64(w1), f64(w2))
    yg, og = f64(y[rows]), f64(out[rows])
    diff = yg != yr
    assert diff.mean() <= 1e-3, diff.mean()
    if diff.any():   # one bf16 step (2^-7 relative to the larger of the two) and the fp32 sum's error
        a, b = yg[diff], yr[diff]
        K = o.shape[1] // w1.shape[0] * o.shape[2]
        mag = O.out_proj(np.abs(f64(o[rows]).reshape(len(rows), -1)), np.abs(f64(w1)), np.abs(f64(w2)))[0][diff]
        assert (np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) * 1.0001 + K * 2.0 ** -24 * mag).all()
    err = np.abs(og - outr).max(axis=1) / np.abs(outr).max(axis=1)
    print(f"  summaries differing: {diff.sum()} of {diff.size}; output max rel err {err.max():.2e}", flush=True)
    assert err.max() <= 2.0 ** -7, err.max()


def test_out_proj_small_ragged():
    H, d, G, r, hidden = 32, 64, 4, 128, 256
    cfg = B.make_cfg(d=d, d_rope=16, n_heads=H)
    for T in (1, 37, 300):                    # both tilings, ragged row counts
        o, w1, w2 = _case(T, H, d, G, r, hidden, T)
        y, out = _run(cfg, G, r, hidden, o, w1, w2)
        _check(y, out, o, w1, w2, list(range(T)))


def test_out_proj_lds_tiling_ragged_rows():
    # Above 256 rows with N a multiple of 256 both products take the 256x256
    # LDS-staged tiles.  1300 rows are 6 row tiles (the last one ragged): one
    # full group of four row tiles in the XCD tile order and a partial one of
    # two; every row against the oracle, and a 300-row slice bitwise the same
    # in the 300-row launch (two row tiles, one group).
    H, d, G, r, hidden = 32, 64, 4, 256, 512
    cfg = B.make_cfg(d=d, d_rope=16, n_heads=H)
    o, w1, w2 = _case(1300, H, d, G, r, hidden, 77)
    print("out_proj LDS tiling 1300 rows", flush=True)
    y, out = _run(cfg, G, r, hidden, o, w1, w2)
    _check(y, out, o, w1, w2, list(range(1300)))
    ys, outs = _run(cfg, G, r, hidden, o[1000:].contiguous(), w1, w2)
    assert torch.equal(outs.view(torch.int16), out[1000:].view(torch.int16))
    assert torch.equal(ys.view(torch.int16), y[1000:].view(torch.int16))


def test_out_proj_production_shape_and_invariance():
    """128 heads x 512 -> 16 groups of rank 1024 -> 7168: decode batch 32 and a
    600-row batch holding the same 32 tokens at other positions."""
    H, d, G, r, hidden = 128, 512, 16, 1024, 7168
    cfg = B.make_cfg()
    o, w1, w2 = _case(32, H, d, G, r, hidden, 99)
    y, out = _run(cfg, G, r, hidden, o, w1, w2)
    _check(y, out, o, w1, w2, [0, 1, 17, 31])
    # alone
    y1, out1 = _run(cfg, G, r, hidden, o[5:6].contiguous(), w1, w2)
    assert torch.equal(out1[0].view(torch.int16), out[5].view(torch.int16))
    assert torch.equal(y1[0].view(torch.int16), y[5].view(torch.int16))
    # inside a large batch (the other tiling), scattered among other tokens
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    big = torch.randn((600, H, d), generator=g, device=DEV).to(torch.bfloat16)
    where = torch.randperm(600, generator=torch.Generator().manual_seed(3))[:32].to(DEV)
    big[where] = o
    yb, outb = _run(cfg, G, r, hidden, big, w1, w2)
    assert torch.equal(outb[where].view(torch.int16), out.view(torch.int16))
    assert torch.equal(yb[where].view(torch.int16), y.view(torch.int16))


def test_out_proj_argument_checks():
    cfg = B.make_cfg()
    o = torch.empty((4, 128, 512), dtype=torch.bfloat16, device=DEV)
    w1 = torch.empty((16, 1024, 4096), dtype=torch.bfloat16, device=DEV)
    w2 = torch.empty((7168, 16 * 1024), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((4, 16 * 1024), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((4, 7168), dtype=torch.bfloat16, device=DEV)
    for G, r, hidden in [(3, 1024, 7168), (16, 1000, 7168), (16, 1024, 7000), (0, 1024, 7168)]:
        with pytest.raises(B.Dsv4Error) as e:
            B.dsv4_out_proj(cfg, G, r, hidden, o, w1, w2, y, out)
        assert e.value.status == B.DSV4_ERR_INVALID_ARG
    with pytest.raises(B.Dsv4Error) as e:
        B.dsv4_out_proj(B.make_cfg(act_dtype=B.DSV4_DT_F32), 16, 1024, 7168, o, w1, w2, y, out)
    assert e.value.status == B.DSV4_ERR_UNSUPPORTED


def test_out_proj_takes_the_attention_output():
    """The CSA decode attention's bf16 output ([queries][128 heads][512]) goes
    straight into the grouped output projection; compared with the oracle's
    projection of that same output (read back)."""
    from tests import test_gpu_decode as D
    from long_context_compressed_02_amd import synth
    from tests import helpers as Hh
    ctx = [1000, 5000, 4097]
    cfg, oc, cache, _, _ = D._fill_attention_case(B.DSV4_CSA, ctx, seed=6)
    nq = len(ctx)
    pos = [c - 1 for c in ctx]
    q, _, _ = synth.decode_queries(synth.CSA_DECODE_128K, nq, sub=6)
    qt, _ = Hh.act_tensor(q, B.DSV4_DT_BF16)
    st = torch.from_numpy(synth.sinks(synth.CSA_DECODE_128K)).to(DEV)
    topk = np.stack([D._random_topk(O.n_visible("csa", p, oc), oc.topk, 300 + i) for i, p in enumerate(pos)])
    o = torch.empty((nq, oc.n_heads, oc.d), dtype=torch.bfloat16, device=DEV)
    B.dsv4_csa_attend_decode(cfg, cache, qt, Hh.i32(range(nq)), Hh.i32(pos), Hh.i32(topk), st, o)
    G, r, hidden = 16, 1024, 7168
    _, w1, w2 = _case(1, oc.n_heads, oc.d, G, r, hidden, 41)
    y, out = _run(cfg, G, r, hidden, o, w1, w2)
    _check(y, out, o, w1, w2, list(range(nq)))
