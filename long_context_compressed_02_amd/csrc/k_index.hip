// k_index.hip -- lightning-indexer scoring and exact top-k for gfx950.
//
// What is computed (vastsailsolution.com V4 article, CSA section, indexer
// paragraph; xiaoyuzhoufm.com summary 1.1: CSA applies DSA over the compressed
// entries): for a query at position t and each visible compressed index key
// k_j (j < floor((t+1)/m)),
//     I[j] = sum_h w_h * max(0, qI_h . k_j)
// with qI and k_j stored as E4M3 codes times one fp32 scale per row.  Since the
// scales are positive, I[j] = s_j * sum_h (w_h * s_h) * max(0, c_h . c_j): the
// code dot products run on the fp8 MFMA (v_mfma 16x16x128 f8f6f4, exact
// products, fp32 accumulation), and the head reduction is a fixed-order sum.
// Then the min(k, N) largest scores by (score desc, index asc), emitted in
// ascending index order (the CSA section: keep the 512 / 1024 most relevant
// entries).
//
// Decode scoring is HBM-bound (132 B of key + scale per key and query): one
// wave streams 64 keys straight into MFMA B-operand registers (no LDS), four
// waves per workgroup, many workgroups per request.  Top-k is a deterministic
// radix select (11/11/10-bit digits, exact integer histograms) followed by an
// index-ordered compaction with wave ballots.
#include "launch.h"

namespace dsv4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- query quantisation
// One wave per (query, head) row: E4M3 codes (zero-padded to 128 bytes) and
// wq = w * scale.  Same decision rule as the stored index keys.
__global__ __launch_bounds__(256) void k_quant_index_q(Lay L, const void *qI, const float *w,
                                                       int rows, uint8_t *q8, float *wq) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int dI = L.dI;
    float x0 = 2 * lane < dI ? load_act(qI, row * dI + 2 * lane, L.act) : 0.0f;
    float x1 = 2 * lane + 1 < dI ? load_act(qI, row * dI + 2 * lane + 1, L.act) : 0.0f;
    float am = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    float scale = 1.0f, inv = 1.0f;
    if (am >= 1e-30f) {
        scale = am / 448.0f;
        inv = 448.0f / am;
    }
    uint32_t c0 = 2 * lane < dI ? fp8_code(x0 * inv) : 0u;
    uint32_t c1 = 2 * lane + 1 < dI ? fp8_code(x1 * inv) : 0u;
    *(uint16_t *)(q8 + row * 128 + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) wq[row] = (w ? w[row] : 1.0f) * scale;
}

// ---------------------------------------------------------------- decode scoring
// grid: (ceil(Nmax / kKeysPerWG), n_queries); block 256 = 4 waves, each
// streaming kKeysPerWave keys as 16-key sub-blocks, loads for the next group of
// four sub-blocks in flight while the current group is on the MFMA.
constexpr int kKeysPerWave = 256;
constexpr int kKeysPerWG = 4 * kKeysPerWave;

// HB: 16-row blocks of index heads (idx_heads <= 16*HB); FULL: idx_dim == 128
// (no padded operand bytes).  Both are compile-time so that the loads and the
// four MFMAs of a sub-block are straight-line code the compiler can pipeline.
template <int HB, bool FULL>
__global__ __launch_bounds__(256) void k_index_score_decode(Lay L, dsv4_cache C, const uint8_t *q8,
                                                            const float *wq, const int32_t *req,
                                                            const int32_t *pos, float *scores,
                                                            int64_t ld) {
    const int q = blockIdx.y;
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);    // wave-uniform (scalar)
    const int r = req[q];
    const int t = pos[q];
    if (r < 0 || r >= C.n_req || t < 0 || (int64_t)t >= (int64_t)C.max_blocks * kBlockTokens) return;
    const int N = (t + 1) / L.m;
    const int k0 = (blockIdx.x * 4 + wave) * kKeysPerWave;
    if (k0 >= N) return;
    const int dI = L.dI;
    // k-order of the 16x16x128 operands: lane group g holds bytes [16g, 16g+16)
    // and [64+16g, 64+16g+16) of a row, so each 16-byte load instruction of a
    // wave reads 64 contiguous bytes of every key row (same order on both sides).
    const int o0 = 16 * g, o1 = 64 + 16 * g;
    const bool v0 = FULL || o0 < dI, v1 = FULL || o1 < dI;   // chunks holding real bytes
    const i32x4 z4 = {0, 0, 0, 0};
    // A operand: query codes (zero-padded to 128 bytes per row), rows = index heads
    i32x8 A[HB];
    float wl[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int row = hb * 16 + c16;
        const bool ok = row < L.HI;
        const uint8_t *p = q8 + ((int64_t)q * L.HI + (ok ? row : 0)) * 128;
        i32x8 a;
        a.lo = *(const i32x4 *)(p + o0);
        a.hi = *(const i32x4 *)(p + o1);
        A[hb] = ok ? a : (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hb * 16 + 4 * g + i;
            wl[hb][i] = h < L.HI ? wq[(int64_t)q * L.HI + h] : 0.0f;
        }
    }
    const int32_t *btr = C.block_table + (int64_t)r * C.max_blocks;
    const int lane_off = c16 * L.key_bytes;
    const uint8_t *pool = (const uint8_t *)C.index_keys;
    // B operands: 16-key sub-blocks, each inside one 128-token cache block, so
    // its block lookup is a wave-uniform scalar load; lane = key (c16).  An
    // unmapped block reads block 0 and is masked by its zero scale.
    auto load_sb = [&](int kb, i32x8 &Bk, float &sk) {
        const int kc = kb < N ? kb : k0;                       // stay in mapped memory past the end
        const int bid = __builtin_amdgcn_readfirstlane(btr[(kc * L.m) / kBlockTokens]);
        const bool okb = bid >= 0 && bid < C.n_blocks && kb < N;
        const uint8_t *base = pool + (int64_t)(okb ? bid : 0) * L.index_block_bytes;
        const int slot0 = kc % L.epb;
        const uint8_t *p = base + slot0 * L.key_bytes + lane_off;
        if constexpr (FULL) {
            Bk.lo = *(const i32x4 *)(p + o0);
            Bk.hi = *(const i32x4 *)(p + o1);
        } else {
            // short keys: read inside the key (offset 0) and zero the padding
            const i32x4 l0 = *(const i32x4 *)(p + (v0 ? o0 : 0));
            const i32x4 l1 = *(const i32x4 *)(p + (v1 ? o1 : 0));
            Bk.lo = v0 ? l0 : z4;
            Bk.hi = v1 ? l1 : z4;
        }
        const float s = ((const float *)(base + L.key_scale_off))[slot0 + c16];
        sk = okb ? s : 0.0f;
    };
    float *srow = scores + (int64_t)q * ld;
    auto score_sb = [&](int kb, const i32x8 &Bk, float sk) {
        f32x4 acc[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
            acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[hb], Bk, (f32x4){0.0f, 0.0f, 0.0f, 0.0f},
                                                                       0, 0, 0, 127, 0, 127);
        float part = 0.0f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) part = part + fmaxf(acc[hb][i], 0.0f) * wl[hb][i];
        part = part + __shfl_xor(part, 16);
        part = part + __shfl_xor(part, 32);
        if (g == 0 && kb + c16 < N) srow[kb + c16] = sk * part;
    };
    constexpr int GS = 2;                          // sub-blocks per pipeline group
    constexpr int NG = kKeysPerWave / 16 / GS;
    i32x8 B0[GS], B1[GS];
    float s0[GS], s1[GS];
#pragma unroll
    for (int i = 0; i < GS; ++i) load_sb(k0 + 16 * i, B0[i], s0[i]);
#pragma unroll
    for (int grp = 0; grp < NG; grp += 2) {
        const int kg = k0 + grp * GS * 16;
        if (kg >= N) break;                        // wave-uniform
#pragma unroll
        for (int i = 0; i < GS; ++i) load_sb(kg + GS * 16 + 16 * i, B1[i], s1[i]);
#pragma unroll
        for (int i = 0; i < GS; ++i) score_sb(kg + 16 * i, B0[i], s0[i]);
        const int kh = kg + GS * 16;
        if (kh >= N) break;
        if (grp + 2 < NG) {
#pragma unroll
            for (int i = 0; i < GS; ++i) load_sb(kh + GS * 16 + 16 * i, B0[i], s0[i]);
        }
#pragma unroll
        for (int i = 0; i < GS; ++i) score_sb(kh + 16 * i, B1[i], s1[i]);
    }
}

// ---------------------------------------------------------------- top-k
// Order-preserving key of a score: larger score -> larger key; -0 == +0; NaN
// below everything.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Exclusive scan of one value per thread over the workgroup (fixed order).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *sh_w, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh_w[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int w = 0; w < kTopkWaves; ++w) {
            uint32_t c = sh_w[w];
            sh_w[w] = s;
            s += c;
        }
        *total = s;
    }
    __syncthreads();
    uint32_t r = sh_w[wave] + x - v;
    __syncthreads();
    return r;
}

struct TopkShared {
    uint32_t hist[2048];
    uint32_t sh_w[kTopkWaves];
    uint32_t wave_gt[kTopkWaves], wave_eq[kTopkWaves];
    uint32_t wave_sel_base[kTopkWaves], wave_eq_base[kTopkWaves];
    uint32_t total;
    uint32_t found_bin, found_before;
};

// Select from keys[0..n) (LDS) the k largest by (key desc, position asc);
// out_pos(i, p) is called for the i-th selected element (ascending position p).
// Returns the number selected (min(k, n)).  Called by all threads.
template <typename Out>
__device__ int select_topk(const uint32_t *keys, int n, int k, TopkShared &S, Out out_pos) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n <= k) {
        for (int p = tid; p < n; p += kTopkThreads) out_pos(p, p);
        return n;
    }
    // radix select of the k-th largest key
    uint32_t prefix = 0, pmask = 0, rem = (uint32_t)k;
    const int shifts[3] = {21, 10, 0};
    const int bitsv[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = shifts[pass], nb = 1 << bitsv[pass];
        for (int b = tid; b < nb; b += kTopkThreads) S.hist[b] = 0;
        __syncthreads();
        for (int p = tid; p < n; p += kTopkThreads) {
            uint32_t u = keys[p];
            if ((u & pmask) == prefix) atomicAdd(&S.hist[(u >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
        // counts from the top bin down: thread owns reversed bins [2*tid, 2*tid+2)
        uint32_t c0 = 0, c1 = 0;
        const int rb0 = 2 * tid, rb1 = 2 * tid + 1;
        if (rb0 < nb) c0 = S.hist[nb - 1 - rb0];
        if (rb1 < nb) c1 = S.hist[nb - 1 - rb1];
        uint32_t before = block_exclusive_scan(c0 + c1, S.sh_w, &S.total);
        if (rb0 < nb && before < rem && rem <= before + c0) {
            S.found_bin = nb - 1 - rb0;
            S.found_before = before;
        }
        if (rb1 < nb && before + c0 < rem && rem <= before + c0 + c1) {
            S.found_bin = nb - 1 - rb1;
            S.found_before = before + c0;
        }
        __syncthreads();
        prefix |= S.found_bin << sh;
        pmask |= (uint32_t)(nb - 1) << sh;
        rem -= S.found_before;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t need_eq = rem;
    // compaction in position order: each wave owns a contiguous chunk
    const int chunk = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
    const int lo = wave * chunk, hi = min(n, lo + chunk);
    uint32_t gt = 0, eq = 0;
    for (int base = lo; base < hi; base += 64) {
        int p = base + lane;
        uint32_t u = p < hi ? keys[p] : 0u;
        bool vg = p < hi && u > T, ve = p < hi && u == T;
        gt += __popcll(__ballot(vg));
        eq += __popcll(__ballot(ve));
    }
    if (lane == 0) {
        S.wave_gt[wave] = gt;
        S.wave_eq[wave] = eq;
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t sb = 0, eb = 0;
        for (int w = 0; w < kTopkWaves; ++w) {
            S.wave_sel_base[w] = sb;
            S.wave_eq_base[w] = eb;
            uint32_t take = eb >= need_eq ? 0u : min(S.wave_eq[w], need_eq - eb);
            sb += S.wave_gt[w] + take;
            eb += S.wave_eq[w];
        }
    }
    __syncthreads();
    uint32_t sb = S.wave_sel_base[wave], eb = S.wave_eq_base[wave];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = lo; base < hi; base += 64) {
        int p = base + lane;
        uint32_t u = p < hi ? keys[p] : 0u;
        bool vg = p < hi && u > T, ve = p < hi && u == T;
        uint64_t me = __ballot(ve);
        uint32_t rank = eb + __popcll(me & below);
        bool sel = vg || (ve && rank < need_eq);
        uint64_t ms = __ballot(sel);
        if (sel) out_pos((int)(sb + __popcll(ms & below)), p);
        sb += __popcll(ms);
        eb += __popcll(me);
    }
    return k;
}

// Segment pass: grid (S_max, n_queries).  Each workgroup stages one segment of
// a query's scores as keys in LDS and selects its local top-k.  A query with a
// single segment writes its final (ascending, -1 padded) list directly;
// otherwise the segment's candidates go to the workspace for the merge pass.
__global__ __launch_bounds__(kTopkThreads) void k_topk_segment(Lay L, const int32_t *req,
                                                               const int32_t *pos, int n_req_cache,
                                                               int64_t max_tokens, const float *scores, int64_t ld,
                                                               int seg, int k, int32_t *out,
                                                               int32_t *cand_idx, uint32_t *cand_key,
                                                               int s_max) {
    extern __shared__ uint32_t dyn[];
    __shared__ TopkShared S;
    const int q = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
    const int r = req[q];
    const int64_t t = pos[q];
    const bool okq = !(r < 0 || r >= n_req_cache || t < 0 || t >= max_tokens);
    const int64_t N = okq ? (t + 1) / L.m : 0;
    const int nseg = N <= seg ? 1 : (int)((N + seg - 1) / seg);
    if (s >= nseg) return;
    const int64_t lo = (int64_t)s * seg;
    const int n = (int)min((int64_t)seg, N - lo);
    const float *src = scores + (int64_t)q * ld + lo;
    uint32_t *keys = dyn;
    for (int p = tid; p < n; p += kTopkThreads) keys[p] = score_key(src[p]);
    __syncthreads();
    if (nseg == 1) {
        int32_t *o = out + (int64_t)q * k;
        int got = select_topk(keys, n, k, S, [&](int i, int p) { o[i] = p; });
        for (int i = got + tid; i < k; i += kTopkThreads) o[i] = -1;
    } else {
        int32_t *ci = cand_idx + ((int64_t)q * s_max + s) * k;
        uint32_t *ck = cand_key + ((int64_t)q * s_max + s) * k;
        select_topk(keys, n, k, S, [&](int i, int p) {
            ci[i] = (int32_t)(lo + p);
            ck[i] = keys[p];
        });
    }
}

// Merge pass: one workgroup per query with more than one segment.  Candidates
// of all segments, concatenated in segment order (ascending entry index), are
// staged and the same selection is run over them.
__global__ __launch_bounds__(kTopkThreads) void k_topk_merge(Lay L, const int32_t *req,
                                                             const int32_t *pos, int n_req_cache,
                                                             int64_t max_tokens, int seg, int k, int32_t *out,
                                                             const int32_t *cand_idx,
                                                             const uint32_t *cand_key, int s_max) {
    extern __shared__ uint32_t dyn[];
    __shared__ TopkShared S;
    const int q = blockIdx.x, tid = threadIdx.x;
    const int r = req[q];
    const int64_t t = pos[q];
    if (r < 0 || r >= n_req_cache || t < 0 || t >= max_tokens) return;
    const int64_t N = (t + 1) / L.m;
    if (N <= seg) return;
    const int nseg = (int)((N + seg - 1) / seg);
    uint32_t *keys = dyn;
    int32_t *cidx = (int32_t *)(dyn + s_max * k);
    int n = 0;
    for (int s = 0; s < nseg; ++s) {
        const int ns = (int)min((int64_t)k, min((int64_t)seg, N - (int64_t)s * seg));
        const int64_t base = ((int64_t)q * s_max + s) * k;
        for (int i = tid; i < ns; i += kTopkThreads) {
            keys[n + i] = cand_key[base + i];
            cidx[n + i] = cand_idx[base + i];
        }
        n += ns;
    }
    __syncthreads();
    int32_t *o = out + (int64_t)q * k;
    int got = select_topk(keys, n, k, S, [&](int i, int p) { o[i] = cidx[p]; });
    for (int i = got + tid; i < k; i += kTopkThreads) o[i] = -1;
}

// ---------------------------------------------------------------- launchers
// Workspace layout for n queries, Nmax entries: q8 [n][HI][128] | wq [n][HI] |
// scores [n][Nmax] | cand_idx [n][S][k] | cand_key [n][S][k].


static inline int64_t al256(int64_t x) { return (x + 255) & ~(int64_t)255; }

int topk_segment_len(int k, int64_t nmax, int nq, int cus) {
    // One workgroup per segment; a query with more than one segment is merged
    // from its segments' candidates (s_max * k <= 16384 keys in LDS).  Small
    // batches use shorter segments so that the selection spreads over the CUs.
    int64_t want = nq > 0 ? (cus + nq - 1) / nq : 1;
    int64_t cap = 16384 / k;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    int64_t seg = (nmax + want - 1) / want;
    seg = (seg + 1023) / 1024 * 1024;
    if (seg < 4096) seg = 4096;
    while ((nmax + seg - 1) / seg * (int64_t)k > 16384) seg += 1024;
    return (int)seg;
}

int64_t index_ws_bytes(const Lay &L, int n, int64_t nmax, IndexWs *w, uint8_t *base) {
    const int seg = topk_segment_len(L.topk, nmax, n, 256);
    const int s_max = nmax <= seg ? 1 : (int)((nmax + seg - 1) / seg);
    int64_t off = 0;
    int64_t o_q8 = off; off = al256(off + (int64_t)n * L.HI * 128);
    int64_t o_wq = off; off = al256(off + (int64_t)n * L.HI * 4);
    int64_t o_sc = off; off = al256(off + (int64_t)n * nmax * 4);
    int64_t o_ci = off, o_ck = off;
    if (s_max > 1) {
        o_ci = off; off = al256(off + (int64_t)n * s_max * L.topk * 4);
        o_ck = off; off = al256(off + (int64_t)n * s_max * L.topk * 4);
    }
    if (w) {
        w->q8 = base + o_q8;
        w->wq = (float *)(base + o_wq);
        w->scores = (float *)(base + o_sc);
        w->cand_idx = (int32_t *)(base + o_ci);
        w->cand_key = (uint32_t *)(base + o_ck);
        w->ld = nmax;
        w->seg = seg;
        w->s_max = s_max;
    }
    return off;
}

// Per-query (request, position) rows for the packed queries of a prefill chunk.
__global__ void k_expand_queries(const int32_t *cu, const int32_t *req, const int32_t *pos0, int n_seq,
                                 int total, int32_t *req_q, int32_t *pos_q) {
    const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gi >= total) return;
    int lo = 0, hi = n_seq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= gi) lo = mid;
        else hi = mid - 1;
    }
    const int64_t p0 = pos0[lo];
    req_q[gi] = req[lo];
    pos_q[gi] = p0 < 0 ? -1 : (int32_t)(p0 + (gi - cu[lo]));
}

hipError_t launch_expand_queries(const int32_t *cu, const int32_t *req, const int32_t *pos0, int n_seq,
                                 int total, int32_t *req_q, int32_t *pos_q, hipStream_t s) {
    hipLaunchKernelGGL(k_expand_queries, dim3((total + 255) / 256), dim3(256), 0, s, cu, req, pos0, n_seq,
                       total, req_q, pos_q);
    return hipGetLastError();
}

hipError_t launch_quant_q(const Lay &L, const void *qI, const float *w, int rows, const IndexWs &ws,
                          hipStream_t s) {
    hipLaunchKernelGGL(k_quant_index_q, dim3((rows + 3) / 4), dim3(256), 0, s, L, qI, w, rows, ws.q8, ws.wq);
    return hipGetLastError();
}

hipError_t launch_score_decode(const Lay &L, const dsv4_cache &C, const int32_t *req, const int32_t *pos,
                               int n, const IndexWs &ws, hipStream_t s) {
    dim3 g((unsigned)((ws.ld + kKeysPerWG - 1) / kKeysPerWG), n);
    const int hb = (L.HI + 15) / 16;
    const bool full = L.dI == 128;
#define DSV4_SCORE(HBV, FV) \
    hipLaunchKernelGGL((k_index_score_decode<HBV, FV>), g, dim3(256), 0, s, L, C, ws.q8, ws.wq, req, pos, ws.scores, ws.ld)
    if (full) {
        if (hb == 4) DSV4_SCORE(4, true);
        else if (hb == 3) DSV4_SCORE(3, true);
        else if (hb == 2) DSV4_SCORE(2, true);
        else DSV4_SCORE(1, true);
    } else {
        if (hb == 4) DSV4_SCORE(4, false);
        else if (hb == 3) DSV4_SCORE(3, false);
        else if (hb == 2) DSV4_SCORE(2, false);
        else DSV4_SCORE(1, false);
    }
#undef DSV4_SCORE
    return hipGetLastError();
}

hipError_t launch_topk(const Lay &L, const dsv4_cache &C, const int32_t *req, const int32_t *pos, int n,
                       const IndexWs &ws, int32_t *out, hipStream_t s) {
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void *)k_topk_segment, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           32768 * 4);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)k_topk_merge, hipFuncAttributeMaxDynamicSharedMemorySize, 16384 * 8);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    size_t lds = (size_t)ws.seg * 4;
    hipLaunchKernelGGL(k_topk_segment, dim3(ws.s_max, n), dim3(kTopkThreads), lds, s, L, req, pos, C.n_req,
                       (int64_t)C.max_blocks * kBlockTokens, ws.scores, ws.ld, ws.seg, L.topk, out, ws.cand_idx, ws.cand_key, ws.s_max);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ws.s_max <= 1) return e;
    size_t lds2 = (size_t)ws.s_max * L.topk * 8;
    hipLaunchKernelGGL(k_topk_merge, dim3(n), dim3(kTopkThreads), lds2, s, L, req, pos, C.n_req,
                       (int64_t)C.max_blocks * kBlockTokens, ws.seg,
                       L.topk, out, ws.cand_idx, ws.cand_key, ws.s_max);
    return hipGetLastError();
}

}  // namespace dsv4
