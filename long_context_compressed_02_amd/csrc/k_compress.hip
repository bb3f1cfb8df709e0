// k_compress.hip -- append + block compressor (decode and prefill), and cache
// fill kernels, for gfx950.
//
// What is computed (vastsailsolution.com V4 article, CSA / HCA sections and the
// cache paragraphs; rqlyzj.com section 01): every new raw token is rotated
// (RoPE on its last d_rope dims at its own position) and stored in the
// per-request window ring; its raw values wait in the pending ring until the
// block of its layer's stride completes.  A completed block j is merged into
// one entry: per channel, softmax over the window's tokens of the gate logits,
// weighted sum of kv; RoPE at the block's last token; stored as E4M3 + scale
// (non-RoPE dims) and BF16 (RoPE dims).  CSA layers also form the index key
// the same way from (kI, gI), without RoPE.
//
// Layout of work: a 64-lane wave owns one stored vector (record or key); lane l
// holds d/64 consecutive dims, so RoPE pairs, the amax reduction and the code
// writes stay inside the wave.  Pooling is per channel and uses one shared
// routine (pool_channel) in both paths, so prefilled entries are bitwise equal
// to entries built token by token.
#include "common.h"

namespace dsv4 {

// ---------------------------------------------------------------- stored vectors
// Store a record held by one wave (lane l owns dims [l*VPL, (l+1)*VPL)).
// cs: cos/sin of the position per RoPE pair if already computed (LDS), else
// computed here.
template <int D, int DR>
__device__ void store_record(const Lay &L, float (&x)[(D / 64) > 0 ? D / 64 : 1], int64_t pos,
                             uint8_t *dst, const float2 *cs = nullptr) {
    constexpr int VPL = D / 64;
    constexpr int DN = D - DR;
    const int lane = threadIdx.x & 63;
    const int d0 = lane * VPL;
    // RoPE on the last DR dims: pairs (2i, 2i+1)
    if constexpr (VPL >= 2) {
#pragma unroll
        for (int v = 0; v < VPL; v += 2) {
            int dd = d0 + v;
            if (dd >= DN) {
                float c, s;
                if (cs) {
                    c = cs[(dd - DN) / 2].x;
                    s = cs[(dd - DN) / 2].y;
                } else {
                    rope_cs(L, pos, (dd - DN) / 2, c, s);
                }
                float a = x[v], b = x[v + 1];
                x[v] = a * c - b * s;
                x[v + 1] = a * s + b * c;
            }
        }
    } else {
        float other = __shfl_xor(x[0], 1);
        if (d0 >= DN) {
            float c, s;
            rope_cs(L, pos, (d0 - DN) / 2, c, s);
            if ((lane & 1) == 0) x[0] = x[0] * c - other * s;
            else x[0] = other * s + x[0] * c;
        }
    }
    if (L.kv_store == DSV4_STORE_FP32) {
        float *o = (float *)dst;
#pragma unroll
        for (int v = 0; v < VPL; ++v) o[d0 + v] = x[v];
        return;
    }
    float am = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        if (d0 + v < DN) am = fmaxf(am, fabsf(x[v]));
    am = wave_max(am);
    float scale = 1.0f, inv = 1.0f;
    if (am >= 1e-30f) {
        scale = am / 448.0f;
        inv = 448.0f / am;
    }
    if (d0 < DN) {
        if constexpr (VPL == 8) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) w0 |= fp8_code(x[v] * inv) << (8 * v);
#pragma unroll
            for (int v = 0; v < 4; ++v) w1 |= fp8_code(x[4 + v] * inv) << (8 * v);
            *(uint2 *)(dst + d0) = make_uint2(w0, w1);
        } else {
#pragma unroll
            for (int v = 0; v < VPL; ++v) dst[d0 + v] = (uint8_t)fp8_code(x[v] * inv);
        }
    } else {
        uint16_t *r = (uint16_t *)(dst + L.rope_off);
#pragma unroll
        for (int v = 0; v < VPL; ++v) r[d0 + v - DN] = bf16_bits(x[v]);
    }
    if (lane == 0) *(float *)(dst + L.scale_off) = scale;
    // padding after the scale is written as zeros: a stored record is a pure
    // function of its inputs, whichever path wrote it
    for (int off = L.scale_off + 4 + 4 * lane; off < L.rec_bytes; off += 256) *(uint32_t *)(dst + off) = 0u;
}

// Store an index key (dI <= 128 values) held by one wave: lane l owns dims
// [l*KPL, l*KPL+KPL) with KPL = 2 (values past dI are ignored).  The 4-byte
// scale slot holds the fp32 scale (FP8) or the four E8M0 block scales (MXFP4).
__device__ void store_index_key(const Lay &L, const float (&x)[2], uint8_t *key, float *scale_slot) {
    const int lane = threadIdx.x & 63;
    const int d0 = lane * 2;
    if (L.idx_store == DSV4_STORE_FP32) {
        float *o = (float *)key;
        if (d0 < L.dI) o[d0] = x[0];
        if (d0 + 1 < L.dI) o[d0 + 1] = x[1];
        return;
    }
    if (L.idx_store == DSV4_STORE_MXFP4) {            // codes, then the key's word of block scales
        uint32_t scales;
        const uint32_t byte = mx4_row(x[0], x[1], d0 < L.dI, d0 + 1 < L.dI, &scales);
        if (d0 < L.dI) key[lane] = (uint8_t)byte;
        if (lane == 0) *(uint32_t *)scale_slot = scales;
        return;
    }
    float am = 0.0f;
    if (d0 < L.dI) am = fabsf(x[0]);
    if (d0 + 1 < L.dI) am = fmaxf(am, fabsf(x[1]));
    am = wave_max(am);
    float scale = 1.0f, inv = 1.0f;
    if (am >= 1e-30f) {
        scale = am / 448.0f;
        inv = 448.0f / am;
    }
    if (d0 < L.dI) {
        uint32_t c0 = fp8_code(x[0] * inv), c1 = fp8_code(x[1] * inv);
        *(uint16_t *)(key + d0) = (uint16_t)(c0 | (c1 << 8));
    }
    if (lane == 0) *scale_slot = scale;
}

__device__ __forceinline__ uint8_t *entry_ptr(const Lay &L, const dsv4_cache &C, int r, int64_t j) {
    int64_t bid = block_id(C.block_table, C.max_blocks, C.n_blocks, r, (j * L.m) / kBlockTokens);
    if (bid < 0) return nullptr;
    return (uint8_t *)C.entries + bid * L.entry_block_bytes + (j % L.epb) * L.rec_bytes;
}

__device__ __forceinline__ uint8_t *key_ptr(const Lay &L, const dsv4_cache &C, int r, int64_t j,
                                            float **scale_slot) {
    int64_t bid = block_id(C.block_table, C.max_blocks, C.n_blocks, r, (j * L.m) / kBlockTokens);
    if (bid < 0) return nullptr;
    uint8_t *blk = (uint8_t *)C.index_keys + bid * L.index_block_bytes;
    *scale_slot = (float *)(blk + L.key_scale_off) + (j % L.epb);
    return blk + (j % L.epb) * L.key_bytes;
}

__device__ __forceinline__ uint8_t *state_ptr(const Lay &L, const dsv4_cache &C, int r) {
    return (uint8_t *)C.state + (int64_t)r * L.state_bytes;
}

// ---------------------------------------------------------------- decode
// One workgroup (256 threads) per request.  Everything the step reads -- the
// new token's kv / gate / kI / gI and, when a block completes and its window
// is short (CSA: 8 tokens), the window's older tokens from the pending ring --
// is loaded into LDS in one batch of loads, so the step waits on memory once;
// the pooled entry, the window record and the ring push are then formed from
// LDS.  (A long window -- HCA, 128 tokens, one entry per 128 steps -- is pooled
// straight from the ring.)
constexpr int kStageWin = 8;           // window tokens staged in LDS
constexpr int kStageFloats = 2 * 512 + 2 * 128;   // floats of one staged token (d <= 512, idx_dim <= 128)


template <int D, int DR>
__global__ __launch_bounds__(256) void k_compress_decode(Lay L, dsv4_cache C, const void *kv,
                                                         const void *gate, const void *kI,
                                                         const void *gI, const int32_t *req,
                                                         const int32_t *pos) {
    constexpr int VPL = D / 64 > 0 ? D / 64 : 1;
    __shared__ float tokbuf[kStageWin][kStageFloats];
    __shared__ float pooled[D + 128];
    __shared__ float2 cs_tab[DR / 2];                // cos/sin of position t (window record and entry)
    const int b = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const bool csa = L.kind == DSV4_CSA;
    const int dI = csa ? L.dI : 0;
    // the new token's channels depend on the batch slot alone: loaded first,
    // beside the request and position (one memory round trip less), channel
    // c = tid + 256u of [kv D][gate D][kI dI][gI dI]
    auto in_tok = [&](int c) {
        if (c < D) return load_act(kv, (int64_t)b * D + c, L.act);
        if (c < 2 * D) return load_act(gate, (int64_t)b * D + c - D, L.act);
        if (c < 2 * D + dI) return load_act(kI, (int64_t)b * dI + c - 2 * D, L.act);
        return load_act(gI, (int64_t)b * dI + c - 2 * D - dI, L.act);
    };
    constexpr int U = (kStageFloats + 255) / 256;
    float vn[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = tid + 256 * u;
        vn[u] = c < L.pend_tok_floats ? in_tok(c) : 0.0f;
    }
    const int r = req[b];
    const int64_t t = pos[b];
    if (r < 0 || r >= C.n_req || t < 0 || t >= (int64_t)C.max_blocks * kBlockTokens) return;
    uint8_t *st = state_ptr(L, C, r);
    float *pend = (float *)(st + L.pend_off);
    const int ptf = L.pend_tok_floats;               // [kv D][gate D][kI dI][gI dI]
    const bool emit = ((t + 1) % L.m) == 0;
    const int64_t j = (t + 1) / L.m - 1;
    const int64_t s0 = emit ? (j * L.m - (L.wc - L.m) > 0 ? j * L.m - (L.wc - L.m) : 0) : 0;
    const int n = emit ? (int)(t - s0 + 1) : 1;
    const bool staged = emit && n <= kStageWin;
    float *newtok = tokbuf[staged ? n - 1 : 0];      // the new token, in ring layout
    // the block of a completed entry (and of its index key), read with the
    // token loads below rather than after the pooling: one memory round trip
    const int64_t ebid = emit ? block_id(C.block_table, C.max_blocks, C.n_blocks, r, (j * L.m) / kBlockTokens) : -1;

    // 1. cos/sin of position t (the window record and the entry both sit
    // there), on the last wave while the others start their loads
    if (tid >= 192 && tid - 192 < DR / 2) {
        float c, sn;
        rope_cs_theta(theta_lane(L, DR / 2), t, c, sn);
        cs_tab[tid - 192] = make_float2(c, sn);
    }
    // 2. one batch of loads into LDS: token slot s of the window (the new one
    // last; its channels were loaded above), channel c = tid + 256u
    {
        const int nold = staged ? n - 1 : 0;         // older window tokens staged
        float v[kStageWin][U];
#pragma unroll
        for (int s = 0; s < kStageWin; ++s) {
            if (s < nold) {                          // (wave-uniform)
                const float *src = pend + ((s0 + s) % L.pend_slots) * ptf;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = tid + 256 * u;
                    v[s][u] = c < ptf ? src[c] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int s = 0; s < kStageWin; ++s)
            if (s < nold) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (tid + 256 * u < ptf) tokbuf[s][tid + 256 * u] = v[s][u];
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (tid + 256 * u < ptf) newtok[tid + 256 * u] = vn[u];
    }
    __syncthreads();

    // 2. pool the completed block (per channel: softmax over the window's gate
    // logits, weighted sum of kv)
    if (emit) {
        for (int c = tid; c < D + dI; c += 256) {
            const bool isk = c >= D;
            const int cc = isk ? c - D : c;
            const int voff = isk ? 2 * D + cc : cc;
            const int goff = isk ? 2 * D + dI + cc : D + cc;
            if (staged) {
                pooled[c] = pool_channel(n, [&](int s, float &v, float &g) {
                    v = tokbuf[s][voff];
                    g = tokbuf[s][goff];
                });
            } else {
                pooled[c] = pool_channel(n, [&](int s, float &v, float &g) {
                    const int64_t p = s0 + s;
                    if (p == t) {
                        v = newtok[voff];
                        g = newtok[goff];
                    } else {
                        const float *tok = pend + (p % L.pend_slots) * ptf;
                        v = tok[voff];
                        g = tok[goff];
                    }
                });
            }
        }
    }
    __syncthreads();
    // 3. push the raw token into the pending ring
    {
        float *tok = pend + (t % L.pend_slots) * ptf;
        for (int c = tid; c < ptf; c += 256) tok[c] = newtok[c];
    }
    // 4. window record of the new token (wave 0)
    if (wave == 0 && L.W > 0) {
        float x[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) x[v] = newtok[lane * VPL + v];
        store_record<D, DR>(L, x, t, st + (t % L.W) * L.rec_bytes, cs_tab);
    }
    // 5. the completed entry (wave 1) and its index key (wave 2)
    if (emit && wave == 1) {
        uint8_t *dst = ebid >= 0 ? (uint8_t *)C.entries + ebid * L.entry_block_bytes + (j % L.epb) * L.rec_bytes
                                 : nullptr;
        if (dst) {
            float x[VPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) x[v] = pooled[lane * VPL + v];
            store_record<D, DR>(L, x, t, dst, cs_tab);   // entry position m*j+m-1 = t
        }
    }
    if (emit && csa && wave == 2) {
        float *ss = nullptr;
        uint8_t *dst = nullptr;
        if (ebid >= 0) {
            uint8_t *blk = (uint8_t *)C.index_keys + ebid * L.index_block_bytes;
            ss = (float *)(blk + L.key_scale_off) + (j % L.epb);
            dst = blk + (j % L.epb) * L.key_bytes;
        }
        if (dst) {
            float x[2];
            x[0] = (2 * lane < dI) ? pooled[D + 2 * lane] : 0.0f;
            x[1] = (2 * lane + 1 < dI) ? pooled[D + 2 * lane + 1] : 0.0f;
            store_index_key(L, x, dst, ss);
        }
    }
}

// ---------------------------------------------------------------- prefill
__device__ __forceinline__ int find_seq(const int32_t *cu, int n_seq, int64_t gi) {
    int lo = 0, hi = n_seq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= gi) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Copy the stored window records of positions pos0-W .. pos0-1 out of the ring
// into the first W slots of the sequence's window buffer.  One WG per sequence.
__global__ __launch_bounds__(256) void k_prefill_oldwin(Lay L, dsv4_cache C, const int32_t *cu,
                                                        const int32_t *req, const int32_t *pos0,
                                                        int n_seq, uint8_t *win) {
    const int i = blockIdx.x;
    const int r = req[i];
    const int64_t p0 = pos0[i];
    if (r < 0 || r >= C.n_req || p0 < 0) return;
    const uint8_t *ring = state_ptr(L, C, r);
    uint8_t *dst = win + ((int64_t)cu[i] + (int64_t)i * L.W) * L.rec_bytes;
    const int cpr = L.rec_bytes / 16;
    for (int c = threadIdx.x; c < L.W * cpr; c += 256) {
        int u = c / cpr, o = (c % cpr) * 16;
        int64_t p = p0 - L.W + u;
        if (p < 0) continue;
        *(uint4 *)(dst + (int64_t)u * L.rec_bytes + o) = *(const uint4 *)(ring + (p % L.W) * L.rec_bytes + o);
    }
}

// One wave per token: its window record, and the entry (and index key) it
// completes, if any.  4 waves per WG.
template <int D, int DR>
__global__ __launch_bounds__(256) void k_prefill_tokens(Lay L, dsv4_cache C, const void *kv,
                                                        const void *gate, const void *kI,
                                                        const void *gI, const int32_t *cu,
                                                        const int32_t *req, const int32_t *pos0,
                                                        int n_seq, int total, uint8_t *win) {
    constexpr int VPL = D / 64 > 0 ? D / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int64_t gi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gi >= total) return;
    const int i = find_seq(cu, n_seq, gi);
    const int r = req[i];
    const int64_t p0 = pos0[i];
    if (r < 0 || r >= C.n_req || p0 < 0) return;
    const int64_t t = p0 + (gi - cu[i]);
    if (t >= (int64_t)C.max_blocks * kBlockTokens) return;
    const bool csa = L.kind == DSV4_CSA;
    const int dI = csa ? L.dI : 0;
    // window record of token t
    {
        float x[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) x[v] = load_act(kv, gi * D + lane * VPL + v, L.act);
        uint8_t *dst = win + ((int64_t)cu[i] + (int64_t)i * L.W + L.W + (gi - cu[i])) * L.rec_bytes;
        store_record<D, DR>(L, x, t, dst);
    }
    if (((t + 1) % L.m) != 0) return;
    const int64_t j = (t + 1) / L.m - 1;
    const int64_t s0 = j * L.m - (L.wc - L.m) > 0 ? j * L.m - (L.wc - L.m) : 0;
    const int n = (int)(t - s0 + 1);
    const float *pend = (const float *)(state_ptr(L, C, r) + L.pend_off);
    const int ptf = L.pend_tok_floats;
    const int64_t row0 = cu[i];
    auto pool_dim = [&](const void *vin, const void *gin, int dim, int voff, int goff, int cc) {
        return pool_channel(n, [&](int s, float &v, float &g) {
            int64_t p = s0 + s;
            if (p >= p0) {
                v = load_act(vin, (row0 + (p - p0)) * dim + cc, L.act);
                g = load_act(gin, (row0 + (p - p0)) * dim + cc, L.act);
            } else {
                const float *tok = pend + (p % L.pend_slots) * ptf;
                v = tok[voff + cc];
                g = tok[goff + cc];
            }
        });
    };
    {
        float x[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) x[v] = pool_dim(kv, gate, D, 0, D, lane * VPL + v);
        uint8_t *dst = entry_ptr(L, C, r, j);
        if (dst) store_record<D, DR>(L, x, t, dst);
    }
    if (csa) {
        float x[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            int cc = 2 * lane + v;
            x[v] = cc < dI ? pool_dim(kI, gI, dI, 2 * D, 2 * D + dI, cc) : 0.0f;
        }
        float *ss = nullptr;
        uint8_t *dst = key_ptr(L, C, r, j, &ss);
        if (dst) store_index_key(L, x, dst, ss);
    }
}

// After the chunk: the ring keeps the chunk's last W records (copied from the
// window buffer) and the pending ring its last pend_slots raw tokens.
__global__ __launch_bounds__(256) void k_prefill_commit(Lay L, dsv4_cache C, const void *kv,
                                                        const void *gate, const void *kI,
                                                        const void *gI, const int32_t *cu,
                                                        const int32_t *req, const int32_t *pos0,
                                                        int n_seq, const uint8_t *win) {
    const int i = blockIdx.y;
    const int r = req[i];
    const int64_t p0 = pos0[i];
    if (r < 0 || r >= C.n_req || p0 < 0) return;
    const int64_t len = cu[i + 1] - cu[i];
    uint8_t *st = state_ptr(L, C, r);
    const int dI = L.kind == DSV4_CSA ? L.dI : 0;
    const int D = L.d;
    // window ring
    if (L.W > 0) {
        const int64_t nw = len < L.W ? len : L.W;
        const int cpr = L.rec_bytes / 16;
        const uint8_t *src = win + ((int64_t)cu[i] + (int64_t)i * L.W + L.W + (len - nw)) * L.rec_bytes;
        for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nw * cpr; c += (int64_t)gridDim.x * 256) {
            int64_t u = c / cpr;
            int o = (int)(c % cpr) * 16;
            int64_t p = p0 + len - nw + u;
            *(uint4 *)(st + (p % L.W) * L.rec_bytes + o) = *(const uint4 *)(src + u * L.rec_bytes + o);
        }
    }
    // pending ring
    {
        const int64_t np = len < L.pend_slots ? len : L.pend_slots;
        const int ptf = L.pend_tok_floats;
        float *pend = (float *)(st + L.pend_off);
        for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < np * ptf; c += (int64_t)gridDim.x * 256) {
            int64_t u = c / ptf;
            int f = (int)(c % ptf);
            int64_t row = cu[i] + len - np + u;
            int64_t p = p0 + len - np + u;
            float v;
            if (f < D) v = load_act(kv, row * D + f, L.act);
            else if (f < 2 * D) v = load_act(gate, row * D + f - D, L.act);
            else if (f < 2 * D + dI) v = load_act(kI, row * dI + f - 2 * D, L.act);
            else v = load_act(gI, row * dI + f - 2 * D - dI, L.act);
            pend[(p % L.pend_slots) * ptf + f] = v;
        }
    }
}

// ---------------------------------------------------------------- cache fill
// One wave per item: an entry record (RoPE at its block-end position) or an
// index key, from fp32 values.
template <int D, int DR>
__global__ __launch_bounds__(256) void k_write_entries(Lay L, dsv4_cache C, int target,
                                                       const int32_t *req, const int32_t *ent,
                                                       int n, const float *vals) {
    constexpr int VPL = D / 64 > 0 ? D / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (it >= n) return;
    const int r = req[it];
    const int64_t j = ent[it];
    if (r < 0 || r >= C.n_req || j < 0) return;
    if (target == DSV4_TARGET_ENTRY) {
        uint8_t *dst = entry_ptr(L, C, r, j);
        if (!dst) return;
        float x[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) x[v] = vals[it * D + lane * VPL + v];
        store_record<D, DR>(L, x, j * L.m + L.m - 1, dst);
    } else {
        float *ss = nullptr;
        uint8_t *dst = key_ptr(L, C, r, j, &ss);
        if (!dst) return;
        float x[2];
        x[0] = 2 * lane < L.dI ? vals[it * L.dI + 2 * lane] : 0.0f;
        x[1] = 2 * lane + 1 < L.dI ? vals[it * L.dI + 2 * lane + 1] : 0.0f;
        store_index_key(L, x, dst, ss);
    }
}

// Raw prefix tokens into the state cache (window ring + pending ring).
template <int D, int DR>
__global__ __launch_bounds__(256) void k_state_tokens(Lay L, dsv4_cache C, int r, int64_t p0, int n,
                                                      const void *kv, const void *gate, const void *kI,
                                                      const void *gI) {
    constexpr int VPL = D / 64 > 0 ? D / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= n) return;
    const int64_t p = p0 + u;
    uint8_t *st = state_ptr(L, C, r);
    const int dI = L.kind == DSV4_CSA ? L.dI : 0;
    if (L.W > 0 && u >= n - L.W) {
        float x[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) x[v] = load_act(kv, u * D + lane * VPL + v, L.act);
        store_record<D, DR>(L, x, p, st + (p % L.W) * L.rec_bytes);
    }
    if (u >= n - L.pend_slots) {
        float *tok = (float *)(st + L.pend_off) + (p % L.pend_slots) * L.pend_tok_floats;
        for (int f = lane; f < L.pend_tok_floats; f += 64) {
            float v;
            if (f < D) v = load_act(kv, u * D + f, L.act);
            else if (f < 2 * D) v = load_act(gate, u * D + f - D, L.act);
            else if (f < 2 * D + dI) v = load_act(kI, u * dI + f - 2 * D, L.act);
            else v = load_act(gI, u * dI + f - 2 * D - dI, L.act);
            tok[f] = v;
        }
    }
}

// ---------------------------------------------------------------- launchers
template <int D, int DR>
static hipError_t launch_compress_decode_t(const Lay &L, const dsv4_cache &C, const void *kv,
                                           const void *gate, const void *kI, const void *gI,
                                           const int32_t *req, const int32_t *pos, int B,
                                           hipStream_t s) {
    hipLaunchKernelGGL((k_compress_decode<D, DR>), dim3(B), dim3(256), 0, s, L, C, kv, gate, kI, gI,
                       req, pos);
    return hipGetLastError();
}

hipError_t launch_compress_decode(const Lay &L, const dsv4_cache &C, const void *kv, const void *gate,
                                  const void *kI, const void *gI, const int32_t *req,
                                  const int32_t *pos, int B, hipStream_t s) {
    if (L.d == 512) return launch_compress_decode_t<512, 64>(L, C, kv, gate, kI, gI, req, pos, B, s);
    return launch_compress_decode_t<64, 16>(L, C, kv, gate, kI, gI, req, pos, B, s);
}

hipError_t launch_compress_prefill(const Lay &L, const dsv4_cache &C, const void *kv, const void *gate,
                                   const void *kI, const void *gI, const int32_t *cu,
                                   const int32_t *req, const int32_t *pos0, int n_seq, int total,
                                   uint8_t *win, hipStream_t s) {
    if (L.W > 0) {
        hipLaunchKernelGGL(k_prefill_oldwin, dim3(n_seq), dim3(256), 0, s, L, C, cu, req, pos0, n_seq, win);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 g((total + 3) / 4);
    if (L.d == 512)
        hipLaunchKernelGGL((k_prefill_tokens<512, 64>), g, dim3(256), 0, s, L, C, kv, gate, kI, gI, cu,
                           req, pos0, n_seq, total, win);
    else
        hipLaunchKernelGGL((k_prefill_tokens<64, 16>), g, dim3(256), 0, s, L, C, kv, gate, kI, gI, cu,
                           req, pos0, n_seq, total, win);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_prefill_commit, dim3(8, n_seq), dim3(256), 0, s, L, C, kv, gate, kI, gI, cu,
                       req, pos0, n_seq, win);
    return hipGetLastError();
}

hipError_t launch_write_entries(const Lay &L, const dsv4_cache &C, int target, const int32_t *req,
                                const int32_t *ent, int n, const float *vals, hipStream_t s) {
    dim3 g((n + 3) / 4);
    if (L.d == 512)
        hipLaunchKernelGGL((k_write_entries<512, 64>), g, dim3(256), 0, s, L, C, target, req, ent, n, vals);
    else
        hipLaunchKernelGGL((k_write_entries<64, 16>), g, dim3(256), 0, s, L, C, target, req, ent, n, vals);
    return hipGetLastError();
}

hipError_t launch_state_tokens(const Lay &L, const dsv4_cache &C, int r, int64_t p0, int n,
                               const void *kv, const void *gate, const void *kI, const void *gI,
                               hipStream_t s) {
    dim3 g((n + 3) / 4);
    if (L.d == 512)
        hipLaunchKernelGGL((k_state_tokens<512, 64>), g, dim3(256), 0, s, L, C, r, p0, n, kv, gate, kI, gI);
    else
        hipLaunchKernelGGL((k_state_tokens<64, 16>), g, dim3(256), 0, s, L, C, r, p0, n, kv, gate, kI, gI);
    return hipGetLastError();
}

}  // namespace dsv4
