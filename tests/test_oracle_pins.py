"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is a closed form, a library routine on a special case, a hand-worked
value from ``tests/golden`` or a property the mathematics fixes, chosen so that
a dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats
def test_e4m3_all_codes_match_torch_and_round_trip():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = O.e4m3_decode(c)
        if c & 0x7F == 0x7F:
            assert math.isnan(v) and math.isnan(ref[c])
            continue
        assert v == ref[c], c
        assert O.e4m3_encode(v) == c, c


def test_e4m3_encode_matches_torch_cast_incl_ties():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000),
                        rng.normal(0, 0.01, 2000)]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties)
    vals = np.array([O.e4m3_decode(c) for c in range(127)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert (got == ref).all()


def test_e4m3_hand_cases():
    for y, code in gold("hand_cases.json")["e4m3_encode"]["cases"]:
        assert O.e4m3_encode(y) == code, y


def test_bf16_round_matches_torch_and_hand():
    for x, r in gold("hand_cases.json")["bf16_round"]["cases"]:
        assert O.bf16_round(x) == r
    rng = np.random.default_rng(3)
    x = rng.normal(0, 10, 5000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([O.bf16_round(float(v)) for v in x], dtype=np.float32)
    assert (got == ref).all()


def test_e2m1_table_and_hand_cases():
    g = gold("hand_cases.json")["e2m1"]
    for c in range(16):
        v = O.e2m1_decode(c)
        assert v == g["decode"][c] and math.copysign(1, v) == math.copysign(1, g["decode"][c]), c
        assert O.e2m1_encode(v) == c, c
    for y, code in g["encode"]:
        assert O.e2m1_encode(y) == code, y


def test_e2m1_encode_is_nearest_by_search():
    """Brute force: the nearest of the 8 magnitudes, ties to the even mantissa
    bit (bit 0 of the code), saturating past 6."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rng = np.random.default_rng(5)
    ys = np.concatenate([np.arange(-8.0, 8.0 + 1e-9, 1.0 / 64), rng.uniform(-7, 7, 3000),
                         [(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])]]).astype(np.float32)
    for y in ys:
        a = abs(float(y))
        dist = [abs(a - m) for m in mags]
        best = min(dist)
        cand = [c for c in range(8) if dist[c] == best]
        c = cand[0] if len(cand) == 1 else [k for k in cand if k % 2 == 0][0]
        want = c | (8 if math.copysign(1, float(y)) < 0 else 0)
        assert O.e2m1_encode(float(y)) == want, float(y)


def test_mx_exponent_rule():
    for amax, x in [(1.0, -2), (6.0, 0), (7.99, 0), (8.0, 1), (0.3, -4), (0.25, -4), (0.0, -127),
                    (2.0 ** -130, -127), (3.0e38, 125)]:
        assert O.mx_exponent(amax) == x, amax
    rng = np.random.default_rng(9)
    for a in rng.lognormal(0, 4, 2000).astype(np.float32):
        x = O.mx_exponent(float(a))
        # the block's largest magnitude lands in [4, 8) after scaling (largest E2M1 binade)
        assert 4.0 <= float(a) / 2.0 ** x < 8.0


def test_mxfp4_store_rows_hand_and_bounds():
    cfg = O.OCfg(idx_dim=32, idx_heads=4, idx_mode=2)
    for case in gold("hand_cases.json")["mx_block"]["cases"]:
        x = np.zeros(32)
        x[:len(case["x"])] = case["x"]
        st = O.store_index_rows(x, cfg)[0]
        assert list(st[:len(case["expect"])]) == case["expect"]
        assert (st[len(case["expect"]):] == 0).all()
    # 128-dim rows: four independent blocks; every stored value is an E2M1
    # value times its block's scale, within half a code step of the input
    cfg = O.OCfg(idx_dim=128, idx_mode=2)
    rng = np.random.default_rng(13)
    x = rng.normal(0, 1, (200, 128)) * rng.lognormal(0, 2, (200, 1))
    st = O.store_index_rows(x, cfg)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for r in range(200):
        for b in range(4):
            xb = x[r, 32 * b:32 * b + 32].astype(np.float32).astype(np.float64)
            e = O.mx_exponent(float(np.abs(xb).max()))
            y = st[r, 32 * b:32 * b + 32] / 2.0 ** e
            assert np.isin(np.abs(y), mags).all()
            u = np.abs(xb) / 2.0 ** e
            step = np.where(u < 2, 0.5, np.where(u < 4, 1.0, 2.0))
            err = np.abs(np.abs(y) - np.minimum(u, 6.0))
            assert (err <= step / 2 + 1e-12).all()
            assert (np.sign(y) * np.sign(xb) >= 0).all()
    # a block's scale does not depend on the other blocks of the row
    x2 = x.copy()
    x2[:, 32:] *= 1000.0
    assert np.array_equal(O.store_index_rows(x2, cfg)[:, :32], st[:, :32])


def test_store_records_structure():
    cfg = O.OCfg(d=64, d_rope=16, n_heads=8)
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, (50, 64))
    st = O.store_records(x, cfg)
    n8 = 48
    for r in range(50):
        amax = np.float32(np.abs(x[r, :n8]).astype(np.float32).max())
        scale = np.float32(amax / np.float32(448.0))
        codes = st[r, :n8] / np.float64(scale)
        # every fp8 value is an E4M3 value times the shared scale
        e4 = torch.from_numpy(codes.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        assert np.array_equal(e4, codes)
        # the largest magnitude maps to the top code
        assert np.abs(codes).max() == 448.0
        # relative error of an E4M3 rounding is at most 2^-4 (normal range)
        big = np.abs(x[r, :n8]) > 8 * scale * 2.0 ** -6
        assert (np.abs(st[r, :n8][big] - x[r, :n8][big]) <= np.abs(x[r, :n8][big]) * 2.0 ** -4 + 1e-12).all()
        # RoPE dims are bf16 of the fp32 value
        ref = torch.from_numpy(x[r, n8:].astype(np.float32)).to(torch.bfloat16).double().numpy()
        assert np.array_equal(st[r, n8:], ref)
    # fp32 storage mode is plain fp32 rounding
    cfg0 = O.OCfg(d=64, d_rope=16, n_heads=8, kv_mode=0)
    assert np.array_equal(O.store_records(x, cfg0), x.astype(np.float32).astype(np.float64))
    # all-zero record stores zeros
    assert not O.store_records(np.zeros((1, 64)), cfg).any()


def test_record_bytes_nearly_half():
    g = gold("record_bytes.json")
    fp8 = g["d"] - g["d_rope"]
    bf = 2 * g["d_rope"]
    assert (fp8, bf) == (g["fp8_bytes"], g["bf16_rope_bytes"])
    assert (fp8 + bf) / (2 * g["d"]) == g["ratio"]


# ---------------------------------------------------------------- RoPE
def test_rope_hand_position_1():
    h = gold("hand_cases.json")["rope_position_1"]
    cfg = O.OCfg(d=4, d_rope=4, n_heads=1, rope_base=h["base"])
    got = O.rope(np.array([h["x"]]), h["pos"], cfg)[0]
    assert np.allclose(got, h["expect"], rtol=0, atol=1e-15)


def test_rope_properties():
    cfg = O.OCfg(d=64, d_rope=16, n_heads=1)
    rng = np.random.default_rng(5)
    x, y = rng.normal(size=(2, 64))
    # position 0 is the identity; only the last d_rope dims move
    assert np.array_equal(O.rope(x[None], 0, cfg)[0], x)
    rx = O.rope(x[None], 777, cfg)[0]
    assert np.array_equal(rx[:48], x[:48])
    # norm preserved per pair
    assert np.allclose(np.hypot(rx[48::2], rx[49::2]), np.hypot(x[48::2], x[49::2]), rtol=1e-13)
    # inner products depend only on the position difference
    for a, b in [(3, 10), (1000, 1007), (123456, 123463)]:
        l = O.rope(x[None], a, cfg)[0] @ O.rope(y[None], b, cfg)[0]
        r = O.rope(x[None], 0, cfg)[0] @ O.rope(y[None], b - a, cfg)[0]
        assert abs(l - r) < 1e-9
    # a rotation by -p undoes a rotation by p
    back = O.rope(O.rope(x[None], 4242, cfg), -4242, cfg)[0]
    assert np.allclose(back, x, atol=1e-12)


# ---------------------------------------------------------------- compressor
def test_pool_hand_two_tokens():
    h = gold("hand_cases.json")["two_token_pool"]
    got = O.pool(np.array(h["kv"]), np.array(h["gate"]), [0], [2])[0]
    assert np.allclose(got, h["expect"], atol=1e-14)


def test_pool_equal_gates_is_mean_and_dominant_gate_selects():
    rng = np.random.default_rng(9)
    kv = rng.normal(size=(8, 32))
    g = np.full((8, 32), 0.3)
    assert np.allclose(O.pool(kv, g, [0], [8])[0], kv.mean(axis=0), atol=1e-14)
    g2 = rng.normal(size=(8, 32))
    g2[5, :] = 800.0
    assert np.allclose(O.pool(kv, g2, [0], [8])[0], kv[5], atol=1e-12)
    # per-channel independence and shift invariance of the gate
    g3 = g2.copy()
    g3[:, 7] += 11.0
    a, b = O.pool(kv, g2, [0], [8])[0], O.pool(kv, g3, [0], [8])[0]
    assert np.allclose(a, b, atol=1e-12)
    g4 = rng.normal(size=(8, 32))
    g5 = g4.copy()
    g5[2, 3] += 1.0
    a, b = O.pool(kv, g4, [0], [8])[0], O.pool(kv, g5, [0], [8])[0]
    assert np.array_equal(np.delete(a, 3), np.delete(b, 3)) and a[3] != b[3]
    # a convex combination stays within the per-channel range
    e = O.pool(kv, g4, [0], [8])[0]
    assert (e <= kv.max(0) + 1e-12).all() and (e >= kv.min(0) - 1e-12).all()


def test_entry_counts_and_token_ranges():
    g = gold("entry_counts.json")
    cfg = O.OCfg()
    for c in g["cases"]:
        t = c["tokens"] - 1          # last position of a sequence of that length
        assert O.n_visible("csa", t, cfg) == c["csa_entries"]
        assert O.n_visible("hca", t, cfg) == c["hca_entries"]
        if "hca_below" in c:
            assert c["hca_entries"] < c["hca_below"]
    for j, lo, hi in g["csa_token_ranges"]["cases"]:
        assert O.csa_entry_tokens(j, cfg) == (lo, hi)
    assert O.hca_entry_tokens(3, cfg) == (384, 512)


def test_overlap_membership_by_planted_gate():
    """A token dominating its gate shows up in exactly the entries whose
    (backward-overlapped) window contains it: floor(s/4) and floor(s/4)+1."""
    cfg = O.OCfg(d=16, d_rope=8, n_heads=1, kv_mode=0)
    rng = np.random.default_rng(1)
    T = 40
    kv = rng.normal(size=(T, 16))
    gate = rng.normal(size=(T, 16)) * 0.1
    s = 13
    gate[s] = 900.0
    js = range(T // 4)
    pooled = O.pool(kv, gate, [O.csa_entry_tokens(j, cfg)[0] for j in js],
                    [O.csa_entry_tokens(j, cfg)[1] - O.csa_entry_tokens(j, cfg)[0] for j in js])
    hit = [j for j in js if np.allclose(pooled[j], kv[s], atol=1e-9)]
    assert hit == [s // 4, s // 4 + 1]


# ---------------------------------------------------------------- indexer
def test_index_scores_single_head_is_relu_dot():
    rng = np.random.default_rng(2)
    q = rng.normal(size=(1, 24))
    k = rng.normal(size=(50, 24))
    got = O.index_scores(q, np.ones(1), k)
    ref = np.maximum(0.0, np.dot(k, q[0]))
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    assert (got >= 0).all() and (got == 0).any()


def test_index_scores_properties():
    rng = np.random.default_rng(4)
    H, D, N = 3, 5, 7                        # non-square on purpose
    q = rng.normal(size=(H, D))
    k = rng.normal(size=(N, D))
    w1, w2 = rng.normal(size=H), rng.normal(size=H)
    s1, s2 = O.index_scores(q, w1, k), O.index_scores(q, w2, k)
    assert np.allclose(O.index_scores(q, w1 + w2, k), s1 + s2, atol=1e-12)      # linear in w
    assert np.allclose(O.index_scores(2.5 * q, w1, k), 2.5 * s1, atol=1e-12)    # ReLU is positively homogeneous
    perm = [2, 0, 1]
    assert np.allclose(O.index_scores(q[perm], w1[perm], k), s1, atol=1e-12)   # head order is irrelevant
    # a head whose dot products are all negative contributes nothing
    qn = np.vstack([q, -k.sum(0) * 100])
    kk = k.copy()
    qn[-1] = -np.abs(qn[-1])
    kk = np.abs(kk)
    assert np.allclose(O.index_scores(qn, np.r_[w1, 5.0], kk), O.index_scores(q, w1, kk), atol=1e-12)
    # each head sees the key through a dot product: single key, single head,
    # zero out dims one at a time
    e = O.index_scores(np.eye(D)[None, 3], np.ones(1), k)
    assert np.allclose(e, np.maximum(0, k[:, 3]))


# ---------------------------------------------------------------- top-k
def test_topk_hand_and_lexsort():
    h = gold("hand_cases.json")["topk_ties"]
    for k, exp in h["cases"]:
        assert O.topk(h["scores"], k).tolist() == exp
    rng = np.random.default_rng(8)
    for N, k in [(1000, 37), (4096, 512), (5, 5), (1, 3)]:
        s = np.round(rng.normal(size=N), 1)                       # many ties
        order = np.lexsort((np.arange(N), -s))
        ref = np.sort(order[:min(k, N)])
        got = O.topk(s, k)
        assert got[:len(ref)].tolist() == ref.tolist()
        assert (got[len(ref):] == -1).all()


def test_topk_nan_lowest():
    s = np.array([np.nan, 1.0, -5.0, np.nan, 0.0])
    assert O.topk(s, 3).tolist() == [1, 2, 4]


# ---------------------------------------------------------------- attention
def test_attend_hand_sink_half():
    h = gold("hand_cases.json")["sink_half"]
    v = np.array([h["v"]])
    q = np.zeros((1, 4))
    o, sm = O.attend(q, [h["sink"]], v, 1.0, return_sink_mass=True)
    assert np.allclose(o[0], h["expect"], atol=1e-15) and abs(sm[0] - h["sink_mass"]) < 1e-15


def test_attend_sink_limits_and_single_record():
    rng = np.random.default_rng(6)
    q = rng.normal(size=(4, 16))
    r = rng.normal(size=(9, 16))
    # no sink: one record -> the record itself
    o = O.attend(q, np.full(4, -np.inf), r[:1], 0.25)
    assert np.allclose(o, np.broadcast_to(r[0], (4, 16)), atol=1e-15)
    # a huge sink absorbs all mass
    o, sm = O.attend(q, np.full(4, 1e4), r, 0.25, return_sink_mass=True)
    assert np.abs(o).max() < 1e-300 and np.allclose(sm, 1.0)
    # sink mass + attention mass = 1 for a finite sink, checked from outside:
    # o computed with sink z equals (1 - sink_mass) * o computed without sink
    z = rng.normal(size=4)
    o1, sm1 = O.attend(q, z, r, 0.25, return_sink_mass=True)
    o0 = O.attend(q, np.full(4, -np.inf), r, 0.25)
    assert np.allclose(o1, (1 - sm1)[:, None] * o0, atol=1e-13)
    lg = 0.25 * q @ r.T
    assert np.allclose(sm1, np.exp(z) / (np.exp(z) + np.exp(lg).sum(1)), rtol=1e-12)


def test_attend_without_sink_is_sdpa():
    rng = np.random.default_rng(12)
    H, d, n = 6, 32, 21
    q = rng.normal(size=(H, d))
    r = rng.normal(size=(n, d))
    tau = 1 / math.sqrt(d)
    got = O.attend(q, np.full(H, -np.inf), r, tau)
    qt = torch.from_numpy(q)[None, :, None, :]                        # [1, H, 1, d]
    kt = torch.from_numpy(r)[None, None].expand(1, H, n, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=tau)[0, :, 0].numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- composition
def _sdpa_causal(qrot, recs, t, tau):
    qt = torch.from_numpy(qrot)[None, :, None, :]
    kt = torch.from_numpy(recs[: t + 1])[None, None].expand(1, qrot.shape[0], t + 1, recs.shape[1])
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=tau)[0, :, 0].numpy()


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_layer_reduces_to_dense_causal_mqa(kind):
    """m=1, window of compression 1, top-k >= T and no raw window: every token is
    its own entry, all are selected, so the layer is dense causal MQA over the
    stored tokens (sink removed)."""
    T, H, d = 24, 4, 32
    cfg = O.OCfg(d=d, d_rope=8, n_heads=H, window=0, m_csa=1, w_csa=1, m_hca=1,
                 idx_heads=2, idx_dim=16, topk=64)
    rng = np.random.default_rng(21)
    kv = rng.normal(size=(T, d))
    gate = rng.normal(size=(T, d))
    kI, gI = rng.normal(size=(2, T, 16))
    q = rng.normal(size=(T, H, d))
    qI = rng.normal(size=(T, 2, 16))
    sinks = np.full(H, -np.inf)
    pos = list(range(T))
    if kind == "csa":
        outs, idx = O.csa_layer(kv, gate, kI, gI, q, qI, None, sinks, pos, cfg)
        for t in pos:
            assert idx[t][: t + 1].tolist() == list(range(t + 1))
    else:
        outs = O.hca_layer(kv, gate, q, sinks, pos, cfg)
    recs = O.window_records(kv, np.arange(T), cfg)
    for t in pos:
        ref = _sdpa_causal(O.query_rot(q[t], t, cfg), recs, t, cfg.tau)
        assert np.allclose(outs[t], ref, rtol=1e-11, atol=1e-12), t


def test_early_positions_attend_window_only():
    """Before the first block completes (t < m-1) CSA sees only its window."""
    cfg = O.OCfg(d=32, d_rope=8, n_heads=2, window=16, idx_heads=2, idx_dim=16, topk=8)
    rng = np.random.default_rng(22)
    T = 3
    kv, gate = rng.normal(size=(2, T, 32))
    kI, gI = rng.normal(size=(2, T, 16))
    q = rng.normal(size=(T, 2, 32))
    qI = rng.normal(size=(T, 2, 16))
    outs, idx = O.csa_layer(kv, gate, kI, gI, q, qI, None, np.full(2, -np.inf), [0, 1, 2], cfg)
    recs = O.window_records(kv, np.arange(T), cfg)
    for t in range(T):
        assert (idx[t] == -1).all()
        assert np.allclose(outs[t], _sdpa_causal(O.query_rot(q[t], t, cfg), recs, t, cfg.tau), atol=1e-12)


def test_planted_key_is_selected_first():
    cfg = O.OCfg(d=32, d_rope=8, n_heads=2, idx_heads=4, idx_dim=16, topk=3)
    rng = np.random.default_rng(23)
    keys = O.store_index_rows(rng.normal(size=(200, 16)), cfg)
    qI = rng.normal(size=(4, 16))
    keys[77] = O.store_index_rows(qI[0][None] * 10, cfg)[0]
    w = np.array([1.0, 0.0, 0.0, 0.0])
    idx, s = O.csa_select(4 * 200 - 1, qI, w, keys, cfg)
    assert 77 in idx.tolist() and np.argmax(s) == 77


def _np_rotate(x, pos, d_rope, base=10000.0):
    """Interleaved-pair rotation of the last d_rope dims, written out with
    numpy's cos/sin (independent of the oracle's C routine)."""
    y = np.array(x, dtype=np.float64)
    n = y.shape[-1]
    for i in range(d_rope // 2):
        th = base ** (-2.0 * i / d_rope)
        c, s = np.cos(pos * th), np.sin(pos * th)
        a, b = y[n - d_rope + 2 * i].copy(), y[n - d_rope + 2 * i + 1].copy()
        y[n - d_rope + 2 * i] = a * c - b * s
        y[n - d_rope + 2 * i + 1] = a * s + b * c
    return y


@pytest.mark.parametrize("kind,m", [("csa", 4), ("hca", 128)])
def test_entry_rope_position_is_block_end(kind, m):
    """A compressed entry is rotated at the last token of its block, m*j + m-1
    (the reading of the partial-RoPE paragraph, which leaves the position
    open).  Checked through both oracle paths that store entries -- directly
    supplied vectors and pooled tokens -- against a numpy rotation; the first
    and one-past-last token of the block give visibly different vectors, so
    the pin fails for either of those readings."""
    cfg = O.OCfg(d=32, d_rope=16, n_heads=1, m_csa=4, w_csa=8, m_hca=128, kv_mode=0)
    rng = np.random.default_rng(31)
    js = [0, 1, 5, 37]
    vals = rng.normal(size=(len(js), 32))
    got = O.entries_from_values(kind, vals, js, cfg)
    for i, j in enumerate(js):
        ref = _np_rotate(vals[i], m * j + m - 1, 16)
        assert np.allclose(got[i], ref, rtol=0, atol=1e-6 * np.abs(ref).max()), (kind, j)
        for wrong in (m * j, m * j + m):
            alt = _np_rotate(vals[i], wrong, 16)
            assert np.abs(got[i] - alt).max() > 1e-3, (kind, j, wrong)
    # pooled entries: equal gates make the pooled vector the window's mean
    # (numpy), which is then rotated at the block end
    w = cfg.w_csa if kind == "csa" else m
    T = m * (max(js) + 1)
    kv = rng.normal(size=(T, 32))
    gate = np.zeros((T, 32))
    pooled = O.entries_from_pool(kind, kv, gate, js, cfg)
    for i, j in enumerate(js):
        lo = max(0, m * j + m - w)
        ref = _np_rotate(kv[lo:m * j + m].mean(axis=0), m * j + m - 1, 16)
        assert np.allclose(pooled[i], ref, rtol=0, atol=1e-6 * np.abs(ref).max()), (kind, j)
        assert np.abs(pooled[i] - _np_rotate(kv[lo:m * j + m].mean(axis=0), m * j, 16)).max() > 1e-3


def test_csa_layer_attends_entries_at_block_end_positions():
    """Composition at m = 4: with no raw window and every entry selected, a
    query at t attends exactly the rotated entries; the expected output is
    written out with numpy (mean-pooled entries rotated at 4j+3, the query
    rotated at t, softmax over tau * q.k with no sink)."""
    d, H = 32, 2
    cfg = O.OCfg(d=d, d_rope=16, n_heads=H, window=0, m_csa=4, w_csa=8, idx_heads=2, idx_dim=16,
                 topk=64, kv_mode=0, idx_mode=0)
    rng = np.random.default_rng(33)
    T = 24
    kv = rng.normal(size=(T, d))
    gate = np.zeros((T, d))
    kI, gI = rng.normal(size=(T, 16)), np.zeros((T, 16))
    q = rng.normal(size=(T, H, d))
    qI = rng.normal(size=(T, 2, 16))
    pos = [7, 15, 23]
    outs, _ = O.csa_layer(kv, gate, kI, gI, q[pos], qI[pos], None, np.full(H, -np.inf), pos, cfg)
    for n, t in enumerate(pos):
        ents = np.stack([_np_rotate(kv[max(0, 4 * j - 4):4 * j + 4].mean(axis=0), 4 * j + 3, 16)
                         for j in range((t + 1) // 4)])
        for h in range(H):
            qr = _np_rotate(q[t, h], t, 16)
            lg = cfg.tau * ents @ qr
            p = np.exp(lg - lg.max())
            ref = (p[:, None] * ents).sum(0) / p.sum()
            assert np.allclose(outs[n, h], ref, rtol=0, atol=1e-6), (t, h)


def test_window_membership():
    cfg = O.OCfg(window=128)
    assert list(O.window_tokens(0, cfg)) == [0]
    assert list(O.window_tokens(127, cfg)) == list(range(128))
    assert list(O.window_tokens(1000, cfg)) == list(range(873, 1001))


# ----------------------------------------------------------------- grouped output projection
def _int_case(T, G, gd, r, hidden, seed):
    """Small-integer inputs: every fp64 sum is exact, so any order agrees."""
    g = np.random.default_rng(seed)
    o = g.integers(-8, 9, (T, G * gd)).astype(np.float64)
    w1 = g.integers(-8, 9, (G, r, gd)).astype(np.float64)
    w2 = g.integers(-4, 5, (hidden, G * r)).astype(np.float64)
    return o, w1, w2


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float32).to(torch.bfloat16).to(
        torch.float64).numpy()


def test_out_proj_is_block_diagonal_product():
    """The grouped form equals one product with the block-diagonal matrix of
    the groups' maps, the summary rounded to bf16 (torch's rounding)."""
    o, w1, w2 = _int_case(7, 4, 24, 16, 40, 1)
    G, r, gd = w1.shape
    bd = np.zeros((G * r, G * gd))
    for k in range(G):
        bd[k * r:(k + 1) * r, k * gd:(k + 1) * gd] = w1[k]
    y_ref = _bf16(o @ bd.T)
    y, out = O.out_proj(o, w1, w2)
    assert np.array_equal(y, y_ref)
    assert np.array_equal(out, y_ref @ w2.T)
    # the rounding matters here: the summaries exceed bf16's 8-bit significand
    assert not np.array_equal(y, o @ bd.T)


def test_out_proj_special_cases():
    # one group: two plain products
    o, w1, w2 = _int_case(5, 1, 32, 8, 12, 2)
    y, out = O.out_proj(o, w1, w2)
    assert np.array_equal(out, _bf16(o @ w1[0].T) @ w2.T)
    # identity group maps: the summary is the input itself (exact in bf16)
    o, _, w2 = _int_case(3, 3, 16, 16, 10, 3)
    eye = np.broadcast_to(np.eye(16), (3, 16, 16)).copy()
    y, out = O.out_proj(o, eye, w2)
    assert np.array_equal(y, o) and np.array_equal(out, o @ w2.T)
    # relabelling the groups (heads, group maps and the columns of W2 alike)
    # leaves the output unchanged
    o, w1, w2 = _int_case(6, 4, 8, 4, 9, 4)
    perm = [2, 0, 3, 1]
    o_p = o.reshape(6, 4, 8)[:, perm].reshape(6, 32)
    w2_p = w2.reshape(9, 4, 4)[:, perm].reshape(9, 16)
    assert np.array_equal(O.out_proj(o_p, w1[perm], w2_p)[1], O.out_proj(o, w1, w2)[1])
    # zero rows stay zero; scaling W2 scales the output
    o[2] = 0.0
    _, out = O.out_proj(o, w1, w2)
    assert (out[2] == 0).all()
    assert np.array_equal(O.out_proj(o, w1, 2.0 * w2)[1], 2.0 * out)


# ----------------------------------------------------------------- MX linear (indexer path)
def test_mxfp8_rows_rule_and_bounds():
    # hand block: amax 3.0 -> floor(log2 3) - 8 = -7, scale 2^-7: 3.0 -> 384 (an E4M3
    # value), 1.01 -> 129.28 -> 128 (step 16 in [128, 256)), 0.1 -> 12.8 -> 13
    # (step 1 in [8, 16)) -> 13/128
    x = np.zeros(32)
    x[:3] = [3.0, 1.01, 0.1]
    st = O.mxfp8_rows(x[None])[0]
    assert list(st[:3]) == [3.0, 1.0, 13.0 / 128] and (st[3:] == 0).all()
    # saturation: amax 1.9 -> x = -8, 1.9 * 256 = 486.4 > 448 -> 448 / 256
    assert O.mxfp8_rows(np.array([[1.9] + [0.0] * 31]))[0, 0] == 448.0 / 256
    rng = np.random.default_rng(21)
    x = rng.standard_normal((100, 96)) * rng.lognormal(0, 3, (100, 1))
    st = O.mxfp8_rows(x)
    for r in range(100):
        for b in range(3):
            xb = x[r, 32 * b:32 * b + 32].astype(np.float32).astype(np.float64)
            amax = np.abs(xb).max()
            e = int(np.floor(np.log2(amax))) - 8
            y = st[r, 32 * b:32 * b + 32] / 2.0 ** e
            # every value an E4M3 value (torch's cast is exact on representable values)
            assert np.array_equal(torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy(), y)
            # and the nearest one (torch's RNE cast) of the scaled input, saturated at 448
            u = np.clip(xb / 2.0 ** e, -448, 448)
            ref = torch.from_numpy(u).to(torch.float8_e4m3fn).to(torch.float64).numpy()
            assert np.array_equal(y, ref)


def test_mx_linear_exact_on_representable_inputs():
    """Inputs already exact in MXFP8 / MXFP4 pass the quantisers unchanged, so
    the linear map is the plain product (numpy, exact on small integers)."""
    rng = np.random.default_rng(23)
    # activations: integers |v| <= 14 with a 14 in every block -> scale 2^-5, v * 32 in
    # E4M3 (a 15 would not be: 480 > 448 saturates to 448, the price of the
    # floor(log2 amax) - 8 rule, pinned below)
    x = rng.integers(-14, 15, (9, 64)).astype(np.float64)
    x[:, ::32] = 14.0
    # weights: E2M1 magnitudes times 2^0 with a 6 (or 4) leading every block -> scale 2^0
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    w = mags[rng.integers(0, 8, (24, 64))] * rng.choice([-1.0, 1.0], (24, 64))
    w[:, ::32] = 6.0
    assert np.array_equal(O.mxfp8_rows(x), x) and np.array_equal(O.mxfp4_rows(w), w)
    assert np.array_equal(O.mx_linear(x, w), x @ w.T)
    y = np.zeros((1, 32))
    y[0, :2] = [15.0, 1.0]
    assert list(O.mxfp8_rows(y)[0, :2]) == [14.0, 1.0]
    # and a block's quantisation does not depend on the others
    x2 = x.copy()
    x2[:, 32:] *= 1024.0
    assert np.array_equal(O.mxfp8_rows(x2)[:, :32], O.mxfp8_rows(x)[:, :32])
