"""GPU: the indexer's prefill path scores a query bit for bit as its decode
path does.  The prefill chunk's queries are also run as decode steps of their
requests at their positions (the same keys, activations and head weights);
both calls' score rows are read back from their workspaces through
dsv4_index_scores_layout and compared as bit patterns, and the two top-k
lists must then be equal.  The chunk spans two requests (so prefill
workgroups hold rows of both), prefixes that end inside a cache block, and
key ranges that end in a partial tile."""
import numpy as np
import pytest
import torch

from long_context_compressed_02_amd import binding as B
from long_context_compressed_02_amd import synth
from tests import helpers as Hh

pytestmark = pytest.mark.gpu

PROD = dict(synth.CSA_DECODE_128K.shape())


def _score_bits(ws, off, ld, n, counts):
    rows = ws[off:off + 4 * n * ld].view(torch.int32).view(n, ld).cpu().numpy()
    return [rows[i, :counts[i]] for i in range(n)]


@pytest.mark.parametrize("act", [B.DSV4_DT_BF16, B.DSV4_DT_F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("idx", [B.DSV4_STORE_FP8, B.DSV4_STORE_MXFP4], ids=["fp8", "mxfp4"])
def test_prefill_scores_bitwise_decode(idx, act):
    cfg, oc = Hh.cfgs(PROD, topk=256, idx_store=idx, act=act)
    pre, new = [16384, 9001], [100, 93]          # prefix tokens and chunk queries per request
    ctx = [p + c for p, c in zip(pre, new)]
    bt, nb, mb = Hh.block_table(ctx, extra_blocks=2, seed=9)
    cache = B.LayerCache(cfg, B.DSV4_CSA, len(ctx), mb, nb, bt)
    for r, c in enumerate(ctx):
        n = c // oc.m_csa
        kv = synth.index_keys(synth.CSA_DECODE_128K, 70 + r, n)
        B.dsv4_cache_write_entries(cfg, cache, B.DSV4_TARGET_INDEX_KEY, Hh.i32([r] * n), Hh.i32(range(n)),
                                   torch.from_numpy(kv).to(Hh.DEV))
    T = sum(new)
    g = np.random.default_rng(12)
    qI = g.standard_normal((T, oc.idx_heads, oc.idx_dim), dtype=np.float32)
    w = (g.standard_normal((T, oc.idx_heads)) / 8).astype(np.float32)
    qIt, _ = Hh.act_tensor(qI, act)
    wt = torch.from_numpy(w).to(Hh.DEV)
    req = np.repeat(np.arange(len(new)), new)
    pos = np.concatenate([np.arange(p, p + c) for p, c in zip(pre, new)])
    counts = [(int(t) + 1) // oc.m_csa for t in pos]
    nmax = mb * (128 // oc.m_csa)
    k = oc.topk
    print(f"  scores {idx} {act}: {T} queries, {min(counts)}..{max(counts)} visible keys", flush=True)
    # the chunk as a prefill call whose workspace holds all its queries
    ws_p = torch.empty(B.dsv4_workspace_bytes(cfg, T, nmax), dtype=torch.uint8, device=Hh.DEV)
    tk_p = torch.empty((T, k), dtype=torch.int32, device=Hh.DEV)
    B.dsv4_index_topk_prefill(cfg, cache, qIt, wt, Hh.i32([0, new[0], T]), Hh.i32(range(len(new))), Hh.i32(pre), T,
                              tk_p, ws_p)
    # the same queries as decode steps
    ws_d = torch.empty(B.dsv4_workspace_bytes(cfg, T, nmax), dtype=torch.uint8, device=Hh.DEV)
    tk_d = torch.empty_like(tk_p)
    B.dsv4_index_topk_decode(cfg, cache, qIt, wt, Hh.i32(req), Hh.i32(pos), tk_d, ws_d)
    torch.cuda.synchronize()
    op, lp = B.dsv4_index_scores_layout(cfg, cache, T, True)
    od, ld = B.dsv4_index_scores_layout(cfg, cache, T, False)
    sp = _score_bits(ws_p, op, lp, T, counts)
    sd = _score_bits(ws_d, od, ld, T, counts)
    bad = [i for i in range(T) if not np.array_equal(sp[i], sd[i])]
    assert not bad, (len(bad), bad[:5])
    vals = np.concatenate(sd).view(np.float32)
    assert np.isfinite(vals).all() and (vals != 0).mean() > 0.9   # real scores were compared
    assert np.array_equal(tk_p.cpu().numpy(), tk_d.cpu().numpy())
