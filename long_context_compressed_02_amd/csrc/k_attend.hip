// k_attend.hip -- single-KV-head MQA with raw window and per-head sink over
// FP8/BF16 records, for gfx950 (CSA sparse gather and HCA dense; decode and
// prefill).
//
// What is computed (vastsailsolution.com V4 article: CSA section -- MQA over the
// selected compressed entries plus the 128 most recent raw tokens; HCA section
// -- the same over all entries; sink paragraph -- a learnable per-head logit
// added only to the softmax denominator): for query position t, head h,
//     l_i = tau * qrot_h . v_i ,  M = max(z_h, max_i l_i)
//     o_h = sum_i e^(l_i - M) v_i / (e^(z_h - M) + sum_i e^(l_i - M))
// with each stored record v_i serving as key and value, qrot the query rotated
// at t on its last d_rope dims.
//
// Design (MI355X): records are staged 64 at a time in LDS exactly as they sit
// in HBM (640 B rows, padded by 16 B against bank conflicts).  A wave owns a
// 16-head group; both contractions run on v_mfma_f32_16x16x32_bf16:
//   S^T = K . Q^T  (A = 16 records x 32 dims read with ds_read_b64 and
//                   converted fp8 -> bf16 exactly; B = the rotated query held
//                   in registers for the whole kernel)
//   O^T += V^T . P^T (A = 16 dims x 32 records read with the gfx950 LDS
//                   transpose loads ds_read_b64_tr_b8 / _tr_b16 straight from
//                   the row-major records; B = P from the S^T registers)
// The FP8 scale stays outside the MFMA: logits use s_i * (q_n . c_i) + q_r . r_i,
// and the P operand of the non-RoPE columns carries p_i * s_i.
//
// Batch invariance and the two kernels (m.youleyou.com, "what was sacrificed";
// hwcomputing.csdn.net section 四): there is no split over records -- every
// head's reduction runs over its query's record list in one fixed order with
// a fixed tile of 64 records.  HI (for a saturated GPU) runs one workgroup per
// (query, 64 heads): each of its 4 waves owns a 16-head group end to end (all
// 4 record blocks of S, all 32 dim blocks of O), so a staged tile feeds 64
// heads.  LO (for an unsaturated GPU) runs one workgroup per (query, 16-head
// group): its 4 waves split the group's work (wave w does record block w of S
// and dim blocks [8w, 8w+8) of O) and exchange logits through LDS, giving 8
// workgroups per query; those 8 sit on one XCD so the gathered records are
// fetched into one L2.  Every head sees the same MFMA instructions on the same
// operands and the same scalar code in the same order, so HI and LO agree bit
// for bit, whatever the batch.
//
// Latency: all record addresses of a query (top-k index -> block table ->
// record) are resolved once into an LDS locator array before the tile loop,
// and tiles are prefetched two deep into registers.
#include "launch.h"

namespace dsv4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 *lds_i32x2_p;
typedef __attribute__((address_space(3))) i16x4 *lds_i16x4_p;

constexpr int kTile = 64;   // records per online-softmax step (fixed: part of the reduction order)



__device__ __forceinline__ bf16x8 cvt8(uint32_t lo, uint32_t hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
    return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
    union { uint4 u; bf16x8 b; } x;
    x.u = u;
    return x.b;
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ __bf16 f2bf(float f) { return (__bf16)f; }

struct QueryInfo {
    int r;
    int64_t t;
    int64_t n_ent;      // visible entries (HCA) / selected list length (CSA)
    int64_t n_vis;      // visible entries
    int n_win;
    int64_t n_list;
    int64_t win_base;   // prefill: record index of position pos0 - W in the window buffer
    int64_t pos0;
    int qrow;           // row of q / out / topk
    bool ok;
};

template <bool CSA, bool PREFILL>
__device__ __forceinline__ QueryInfo query_info(const AttnArgs &A, int qi) {
    QueryInfo Q;
    const Lay &L = A.L;
    Q.qrow = qi;
    Q.ok = false;
    if constexpr (PREFILL) {
        int lo = 0, hi = A.n_seq - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (A.cu[mid] <= qi) lo = mid;
            else hi = mid - 1;
        }
        Q.r = A.req[lo];
        Q.pos0 = A.pos0[lo];
        Q.t = Q.pos0 + (qi - A.cu[lo]);
        Q.win_base = (int64_t)A.cu[lo] + (int64_t)lo * L.W;
        if (Q.pos0 < 0) return Q;
    } else {
        Q.r = A.req[qi];
        Q.t = A.pos[qi];
        Q.pos0 = 0;
        Q.win_base = 0;
    }
    if (Q.r < 0 || Q.r >= A.C.n_req || Q.t < 0 || Q.t >= (int64_t)A.C.max_blocks * kBlockTokens) return Q;
    Q.n_vis = (Q.t + 1) / L.m;
    if constexpr (CSA) Q.n_ent = Q.n_vis < L.topk ? Q.n_vis : L.topk;
    else Q.n_ent = Q.n_vis;
    Q.n_win = L.W > 0 ? (int)(Q.t + 1 < L.W ? Q.t + 1 : L.W) : 0;
    Q.n_list = Q.n_ent + Q.n_win;
    Q.ok = true;
    return Q;
}

// Record locator of list element p (entries first, then window tokens):
//   >= 0        classic-cache record index (block id * entries_per_block + slot)
//   -1 - w      window record w (decode: ring slot; prefill: window-buffer index)
//   kMasked     masked (invalid index or unmapped block)
constexpr int32_t kMasked = INT32_MIN;

template <bool CSA, bool PREFILL>
__device__ __forceinline__ int32_t record_loc(const AttnArgs &A, const QueryInfo &Q, int64_t p) {
    const Lay &L = A.L;
    if (p < Q.n_ent) {
        int64_t j = p;
        if constexpr (CSA) {
            j = A.topk[(int64_t)Q.qrow * L.topk + p];
            if (j < 0 || j >= Q.n_vis) return kMasked;
        }
        int64_t bid = block_id(A.C.block_table, A.C.max_blocks, A.C.n_blocks, Q.r, (j * L.m) / kBlockTokens);
        if (bid < 0) return kMasked;
        return (int32_t)(bid * L.epb + (j % L.epb));
    }
    int64_t u = p - Q.n_ent;
    if (u >= Q.n_win) return kMasked;
    int64_t s = Q.t - Q.n_win + 1 + u;
    if constexpr (PREFILL) return (int32_t)(-1 - (Q.win_base + (s - (Q.pos0 - L.W))));
    return (int32_t)(-1 - (s % L.W));
}

template <bool PREFILL>
__device__ __forceinline__ const uint8_t *loc_addr(const AttnArgs &A, const QueryInfo &Q, int32_t loc) {
    const Lay &L = A.L;
    if (loc >= 0) return (const uint8_t *)A.C.entries + (int64_t)loc * L.rec_bytes;
    const int64_t w = -1 - (int64_t)loc;
    if constexpr (PREFILL) return A.win + w * L.rec_bytes;
    return (const uint8_t *)A.C.state + (int64_t)Q.r * L.state_bytes + w * L.rec_bytes;
}

// G head groups per workgroup, R waves per head group: HI = (4, 2), LO = (1, 4).
template <int D, int DR, int G, int R, bool CSA, bool PREFILL>
__global__ __launch_bounds__(64 * G * R) void k_attend(AttnArgs A) {
    constexpr int NT = 64 * G * R;
    constexpr bool HI = G > 1;
    constexpr int RBW = 4 / R;                   // record blocks of S per wave
    constexpr int DN = D - DR;
    constexpr int REC = ((DN + 2 * DR + 4) + 63) / 64 * 64;   // stored record stride in HBM
    // LDS row: the record dequantised to bf16 codes (E4M3 -> bf16 is exact; the
    // scale stays separate): [DN bf16 | DR bf16 | fp32 scale | pad]
    constexpr int ROPE_OFF = 2 * DN, SCALE_OFF = 2 * D;
    constexpr int RS = (2 * D + 4 + 15) / 16 * 16 + 16;     // 16 B pad against bank conflicts
    constexpr int NCH = DN / 16;                 // HBM chunks of E4M3 codes
    constexpr int RCH = DR / 8;                  // HBM chunks of bf16 RoPE dims
    constexpr int LCH = NCH + RCH + 1;           // chunks loaded per record (codes, RoPE, scale)
    constexpr int SCALE_OFF_HBM = DN + 2 * DR;   // 16-byte aligned: DN, DR multiples of 16
    static_assert(SCALE_OFF_HBM % 16 == 0, "scale chunk alignment");
    constexpr int KN = (DN + 31) / 32, KR = (DR + 31) / 32;
    constexpr int DBN = DN / 16, DBR = DR / 16, DB = DBN + DBR;
    constexpr int TPR = NT / kTile;              // loader threads per record
    constexpr int CPT = (LCH + TPR - 1) / TPR;   // 16-byte chunks per thread per tile
    constexpr int DBW = (DB + R - 1) / R;        // dim blocks of O held per wave

    __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * RS];
    __shared__ float sS[G][4][16][17];            // logits exchanged between a group's waves
    __shared__ int32_t safe_sh;
    __shared__ float2 rope_tab[DR / 2];          // cos/sin of this query's position per RoPE pair
    extern __shared__ int32_t locs[];            // [n_list] record locators of this query

    const Lay &L = A.L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;

    // ---- which query and head group (the workgroups of one query share an
    // XCD: workgroups are dealt round-robin over the 8 XCDs)
    const int lin = blockIdx.x, x8 = lin & 7, u8 = lin >> 3;
    const int parts = A.nhg / G;                 // workgroups per query
    const int qi = (u8 / parts) * 8 + x8;
    const int gl = wave / R, role = wave % R;    // head group within the workgroup, role in it
    const int hg = (u8 % parts) * G + gl;
    if (qi >= A.nq) return;
    const QueryInfo Q = query_info<CSA, PREFILL>(A, qi);
    if (!Q.ok) return;
    const int head = hg * 16 + c16;
    const bool head_ok = hg < A.nhg && head < L.H;

    // ---- resolve every record of the list once
    for (int64_t p = tid; p < Q.n_list; p += NT) locs[p] = record_loc<CSA, PREFILL>(A, Q, p);
    __syncthreads();
    if (tid < DR / 2) {
        float c, sn;
        rope_cs(L, Q.t, tid, c, sn);
        rope_tab[tid] = make_float2(c, sn);
    }
    if (tid == 0) {
        int32_t sf = kMasked;
        for (int64_t p = Q.n_list - 1; p >= 0; --p)
            if (locs[p] != kMasked) {
                sf = locs[p];
                break;
            }
        safe_sh = sf;
    }

    __syncthreads();
    // ---- query fragments (B operand of S^T = K Q^T): lane = head, items = 8 dims
    bf16x8 Qn[KN], Qr[KR];
    {
        const int64_t qbase = ((int64_t)Q.qrow * L.H + head) * D;
        // 8 consecutive dims of this lane's head as fp32 (one or two 16-byte loads)
        auto q8 = [&](int dd, float (&v)[8]) {
            if (L.act == DSV4_DT_BF16) {
                const uint4 u = *(const uint4 *)((const uint16_t *)A.q + qbase + dd);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = __uint_as_float(w[j] << 16);
                    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                }
            } else {
                const float4 a = *(const float4 *)((const float *)A.q + qbase + dd);
                const float4 b = *(const float4 *)((const float *)A.q + qbase + dd + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            }
        };
#pragma unroll
        for (int ks = 0; ks < KN; ++ks) {
            const int dd = ks * 32 + 8 * g;
            float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (head_ok && dd < DN) q8(dd, v);
            bf16x8 f;
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = f2bf(v[j]);
            Qn[ks] = f;
        }
#pragma unroll
        for (int ks = 0; ks < KR; ++ks) {
            const int uu = ks * 32 + 8 * g;
            float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (head_ok && uu < DR) q8(DN + uu, v);
            bf16x8 f;
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                float a = 0.0f, b = 0.0f;
                if (uu + j < DR) {
                    const float2 cs = rope_tab[(uu + j) / 2];
                    a = v[j] * cs.x - v[j + 1] * cs.y;
                    b = v[j] * cs.y + v[j + 1] * cs.x;
                }
                f[j] = f2bf(a);
                f[j + 1] = f2bf(b);
            }
            Qr[ks] = f;
        }
    }
    const int32_t safe = safe_sh;

    // ---- running softmax state (lane's head) and output accumulators O^T
    // softmax in base 2: logits carry tau*log2(e), exp is v_exp_f32
    const float tau2 = L.tau * 1.4426950408889634f;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 O[DBW];
#pragma unroll
    for (int i = 0; i < DBW; ++i) O[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    const int db0 = role * DBW;
    const int64_t ntiles = (Q.n_list + kTile - 1) / kTile;

    // loader: thread tid fetches chunks (tid % TPR) + TPR*i of record tid / TPR
    const int ld_rec = tid / TPR, ld_c0 = tid % TPR;
    auto load = [&](uint4 (&pre)[CPT], int64_t tl) {
        const int64_t p = tl * kTile + ld_rec;
        int32_t lc = p < Q.n_list ? locs[p] : kMasked;
        if (lc == kMasked) lc = safe;
        if (lc == kMasked) {
#pragma unroll
            for (int i = 0; i < CPT; ++i) pre[i] = make_uint4(0, 0, 0, 0);
            return;
        }
        const uint4 *src = (const uint4 *)loc_addr<PREFILL>(A, Q, lc);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = ld_c0 + i * TPR;
            if (c < LCH) pre[i] = src[c < NCH + RCH ? c : (SCALE_OFF_HBM / 16)];
        }
    };

    auto compute = [&](int64_t tl) {
        auto valid = [&](int rr) {
            const int64_t p = tl * kTile + rr;
            return p < Q.n_list && locs[p] != kMasked;
        };
        // ---- S^T = K Q^T for the record blocks this wave owns
        float lg[4][4];
        auto qk_block = [&](int rb, float (&out)[4]) {
            const int rec = rb * 16 + c16;                 // A-operand row: record
            const uint8_t *row = tile + rec * RS;
            f32x4 an = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KN; ++ks) {
                const int d0 = ks * 32 + 8 * g;
                bf16x8 a = as_bf16x8(make_uint4(0, 0, 0, 0));
                if (d0 < DN) a = *(const bf16x8 *)(row + 2 * d0);
                an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Qn[ks], an, 0, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < KR; ++ks) {
                const int u0 = ks * 32 + 8 * g;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (u0 < DR) v = *(const uint4 *)(row + ROPE_OFF + 2 * u0);
                ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(v), Qr[ks], ar, 0, 0, 0);
            }
            // output lane = head, items = records rb*16 + 4g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = rb * 16 + 4 * g + i;
                const float sc = *(const float *)(tile + rr * RS + SCALE_OFF);
                const float z = tau2 * (sc * an[i] + ar[i]);
                out[i] = valid(rr) ? z : -INFINITY;
            }
        };
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
            const int rb = role * RBW + i;
            float mine[4];
            qk_block(rb, mine);
#pragma unroll
            for (int e = 0; e < 4; ++e) sS[gl][rb][4 * g + e][c16] = mine[e];
        }
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) lg[rb][i] = sS[gl][rb][4 * g + i][c16];

        // ---- online softmax for the lane's head (identical code in HI and LO)
        float tmax = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, lg[rb][i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        float alpha = 1.0f;
        float p[4][4];
        if (m_new == -INFINITY) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[rb][i] = 0.0f;
        } else {
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[rb][i] = __builtin_amdgcn_exp2f(lg[rb][i] - m_new);
        }
        float ps = 0.0f;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ps = ps + p[rb][i];
        ps = ps + __shfl_xor(ps, 16);
        ps = ps + __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < DBW; ++i) O[i] = O[i] * alpha;

        // ---- O^T += V^T P^T, two k-steps of 32 records
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // B operand: lane = head, items j <-> record ks*32 + (j<4 ? 4g+j : 16+4g+j-4)
            bf16x8 Pn, Pr;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int rb = 2 * ks + (j >> 2), i = j & 3;
                const int rr = rb * 16 + 4 * g + i;
                const float sc = *(const float *)(tile + rr * RS + SCALE_OFF);
                Pn[j] = f2bf(p[rb][i] * sc);
                Pr[j] = f2bf(p[rb][i]);
            }
            // transpose-read addresses: lanes 4r..4r+3 of group g -> record of row r
            const int r16 = c16 >> 2, q16 = c16 & 3;
            const int rec16a = ks * 32 + 4 * g + r16;
            const int rec16b = ks * 32 + 16 + 4 * g + r16;
#pragma unroll
            for (int ii = 0; ii < DBW; ++ii) {
                const int db = db0 + ii;
                if (db >= DB) break;
                // dims db*16 .. db*16+15 of the bf16 row (non-RoPE dims first, then RoPE)
                const int cb = db * 16 + 4 * q16;
                i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(tile + rec16a * RS + 2 * cb));
                i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(tile + rec16b * RS + 2 * cb));
                union { i16x4 s[2]; bf16x8 b; } cv;
                cv.s[0] = lo;
                cv.s[1] = hi;
                O[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, db < DBN ? Pn : Pr, O[ii], 0, 0, 0);
            }
        }
    };

    auto step = [&](uint4 (&pre)[CPT], int64_t tl) {
        __syncthreads();                                   // previous tile fully consumed
        uint8_t *row = tile + ld_rec * RS;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = ld_c0 + i * TPR;
            if (c < NCH) {                       // 16 codes -> 16 bf16
                const bf16x8 lo8 = cvt8(pre[i].x, pre[i].y), hi8 = cvt8(pre[i].z, pre[i].w);
                *(bf16x8 *)(row + 32 * c) = lo8;
                *(bf16x8 *)(row + 32 * c + 16) = hi8;
            } else if (c < NCH + RCH) {          // RoPE dims, already bf16
                *(uint4 *)(row + ROPE_OFF + 16 * (c - NCH)) = pre[i];
            } else if (c == NCH + RCH) {         // scale
                *(float *)(row + SCALE_OFF) = __uint_as_float(pre[i].x);
            }
        }
        __syncthreads();                                   // tile visible
        if (tl + 2 < ntiles) load(pre, tl + 2);            // two tiles in flight during compute
        compute(tl);
    };

    uint4 pre0[CPT], pre1[CPT];
    if (ntiles > 0) load(pre0, 0);
    if (ntiles > 1) load(pre1, 1);
    for (int64_t tl = 0; tl < ntiles; tl += 2) {
        step(pre0, tl);
        if (tl + 1 < ntiles) step(pre1, tl + 1);
    }

    // ---- sink and normalisation; output rows d = db*16 + 4g + i of head `head`
    if (!head_ok) return;
    const float z = A.sinks[head] * 1.4426950408889634f;
    const float M = fmaxf(m_run, z);
    const float f = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    const float den = l_run * f + ((z == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - M));
    const float cf = den > 0.0f ? f / den : 0.0f;
    const int64_t obase = ((int64_t)Q.qrow * L.H + head) * D;
#pragma unroll
    for (int ii = 0; ii < DBW; ++ii) {
        const int db = db0 + ii;
        if (db >= DB) break;
        const int dd = db * 16 + 4 * g;
        if (L.act == DSV4_DT_BF16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 v = {f2bf(O[ii][0] * cf), f2bf(O[ii][1] * cf), f2bf(O[ii][2] * cf), f2bf(O[ii][3] * cf)};
            *(bf16x4 *)((uint16_t *)A.out + obase + dd) = v;
        } else {
            *(float4 *)((float *)A.out + obase + dd) =
                make_float4(O[ii][0] * cf, O[ii][1] * cf, O[ii][2] * cf, O[ii][3] * cf);
        }
    }
}

// ---------------------------------------------------------------- launchers
int64_t attend_list_max(const Lay &L, const dsv4_cache &C, bool csa) {
    return (csa ? (int64_t)L.topk : (int64_t)C.max_blocks * L.epb) + L.W;
}

template <int D, int DR, int G, int R, bool CSA, bool PREFILL>
static hipError_t launch_gr(const AttnArgs &A, hipStream_t s) {
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)k_attend<D, DR, G, R, CSA, PREFILL>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kAttendMaxLocBytes);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const size_t lds = (size_t)attend_list_max(A.L, A.C, CSA) * 4;
    const int groups = (A.nq + 7) / 8;
    hipLaunchKernelGGL((k_attend<D, DR, G, R, CSA, PREFILL>), dim3(groups * 8 * (A.nhg / G)), dim3(64 * G * R), lds,
                       s, A);
    return hipGetLastError();
}

template <int D, int DR, bool CSA, bool PREFILL>
static hipError_t launch_t(const AttnArgs &A, bool hi, hipStream_t s) {
    return hi ? launch_gr<D, DR, 4, 2, CSA, PREFILL>(A, s) : launch_gr<D, DR, 1, 4, CSA, PREFILL>(A, s);
}

hipError_t launch_attend(const AttnArgs &A, bool csa, bool prefill, bool hi, hipStream_t s) {
    if (A.L.d == 512) {
        if (csa) return prefill ? launch_t<512, 64, true, true>(A, hi, s) : launch_t<512, 64, true, false>(A, hi, s);
        return prefill ? launch_t<512, 64, false, true>(A, hi, s) : launch_t<512, 64, false, false>(A, hi, s);
    }
    if (csa) return prefill ? launch_t<64, 16, true, true>(A, hi, s) : launch_t<64, 16, true, false>(A, hi, s);
    return prefill ? launch_t<64, 16, false, true>(A, hi, s) : launch_t<64, 16, false, false>(A, hi, s);
}

}  // namespace dsv4
