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
// Design (MI355X): both contractions run on v_mfma_f32_16x16x32_bf16:
//   S^T = K . Q^T  (A = 16 records x 32 dims: E4M3 codes read from LDS and
//                   converted to bf16 exactly; B = the rotated query, held in
//                   registers for the whole kernel)
//   O^T += V^T . P^T (A = 16 dims x 32 records read with the gfx950 LDS
//                   transpose loads ds_read_b64_tr_b8 / _tr_b16 straight from
//                   the row-major records; B = P from the S^T registers)
// The FP8 scale stays outside the MFMA: logits use s_i * (q_n . c_i) + q_r . r_i,
// and the P operand of the non-RoPE columns carries p_i * s_i.  Records are
// gathered 32 at a time (whole 128-byte lines per load) into LDS rows padded
// and shifted against bank conflicts.
//
// Batch invariance and the two kernels (m.youleyou.com, "what was sacrificed";
// hwcomputing.csdn.net section 四): nothing is split across workgroups -- each
// (query, 16-head group) is reduced by one workgroup in a fixed order that
// depends on nothing but the query (see the decomposition below), so a
// query's output is bitwise the same whatever the batch.  Two kernels run
// that decomposition: k_attend_lo (for an unsaturated GPU) gives the
// workgroup 4 waves, one per subset, each over all dims; k_attend (HI, for a
// saturated GPU) gives it 2 waves, one per dim part, that take the subsets one
// after another, so that several workgroups share a compute unit.  Both sum
// every logit from the same partial dot products and fold the subsets in the
// same order: they agree bit for bit.  The 8 workgroups of a query are placed
// on one XCD, so its gathered records are fetched into one L2.
//
// Latency: all record addresses of a query (top-k index -> block table ->
// record) are resolved once into an LDS locator array before the chunk loop,
// and the next chunk's loads are in flight while the current one is computed.
#include <type_traits>

#include "launch.h"

#include <mutex>

namespace dsv4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 *lds_i32x2_p;
typedef __attribute__((address_space(3))) i16x4 *lds_i16x4_p;





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
    int wb;             // decode: ring slot of the oldest window token, (t - n_win + 1) mod W
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
    Q.n_vis = (Q.t + 1) >> __builtin_ctz((uint32_t)L.m);   // (m is a power of two)
    if constexpr (CSA) Q.n_ent = Q.n_vis < L.topk ? Q.n_vis : L.topk;
    else Q.n_ent = Q.n_vis;
    Q.n_win = L.W > 0 ? (int)(Q.t + 1 < L.W ? Q.t + 1 : L.W) : 0;
    Q.n_list = Q.n_ent + Q.n_win;
    // (t < 2^31: a 32-bit remainder, taken once; window positions then add to it)
    Q.wb = !PREFILL && L.W > 0 ? (int)((uint32_t)(Q.t - Q.n_win + 1) % (uint32_t)L.W) : 0;
    Q.ok = true;
    return Q;
}

// Record locator of list element p.  The list is the window tokens first
// (oldest first), then the entries (CSA: in top-k order; HCA: in index
// order), so the records a query's first chunks need are known from its
// position alone, before any top-k or block-table read.
//   >= 0        classic-cache record index (block id * entries_per_block + slot)
//   -1 - w      window record w (decode: ring slot; prefill: window-buffer index)
//   kMasked     masked (invalid index or unmapped block)
constexpr int32_t kMasked = INT32_MIN;

template <bool PREFILL>
__device__ __forceinline__ int32_t window_loc(const AttnArgs &A, const QueryInfo &Q, int64_t p) {
    if constexpr (PREFILL) {
        const int64_t s = Q.t - Q.n_win + 1 + p;         // the token of window position p < n_win
        return (int32_t)(-1 - (Q.win_base + (s - (Q.pos0 - A.L.W))));
    }
    const int x = Q.wb + (int)p;                         // its ring slot: 0 <= p < n_win <= W
    return (int32_t)(-1 - (x >= A.L.W ? x - A.L.W : x));
}

template <bool CSA, bool PREFILL>
__device__ __forceinline__ int32_t record_loc(const AttnArgs &A, const QueryInfo &Q, int64_t p) {
    const Lay &L = A.L;
    if (p < Q.n_win) return window_loc<PREFILL>(A, Q, p);
    const int64_t e = p - Q.n_win;
    if (e >= Q.n_ent) return kMasked;
    int64_t j = e;
    if constexpr (CSA) {
        j = A.topk[(int64_t)Q.qrow * L.topk + e];
        if (j < 0 || j >= Q.n_vis) return kMasked;
    }
    int64_t bid = block_id(A.C.block_table, A.C.max_blocks, A.C.n_blocks, Q.r, (j * L.m) / kBlockTokens);
    if (bid < 0) return kMasked;
    return (int32_t)(bid * L.epb + (j & (L.epb - 1)));  // (entries per block: a power of two)
}

template <bool PREFILL>
__device__ __forceinline__ const uint8_t *loc_addr(const AttnArgs &A, const QueryInfo &Q, int32_t loc) {
    const Lay &L = A.L;
    if (loc >= 0) return (const uint8_t *)A.C.entries + (int64_t)loc * L.rec_bytes;
    const int64_t w = -1 - (int64_t)loc;
    if constexpr (PREFILL) return A.win + w * L.rec_bytes;
    return (const uint8_t *)A.C.state + (int64_t)Q.r * L.state_bytes + w * L.rec_bytes;
}

// ---------------------------------------------------------------- the kernel
// Decomposition of one (query, 16-head group).  The record list is cut into
// chunks of 32 records; chunk c belongs to subset c mod 4, and each subset is
// reduced on its own (online softmax over its chunks in increasing order).
// The dims are cut into 2 parts: part dq owns MFMA code pairs
// [QPP*dq, QPP*dq + QPP) of the logits and dim blocks [DBQ*dq, DBQ*dq + DBQ)
// of the output; the last part also owns the RoPE part of the logits.  A
// chunk's logits are the fixed-order sum of the parts' partial dot products:
//     l = tau * (s * (a0 + a1) + r)
// (a_q: code dims of part q, s: the record's scale, r: RoPE dims).  The four
// subset states are then folded left to right:
//     acc = s0;  acc = fold(acc, s1);  acc = fold(acc, s2);  acc = fold(acc, s3)
// HI (2 waves: the parts) runs the subsets one after another and folds in
// registers; k_attend_lo below runs them at once and folds through LDS.
constexpr int kChunk = 32;     // records per chunk (the k of one PV MFMA)
constexpr int kSubsets = 4;
constexpr int kParts = 2;     // dim parts (each wave holds one part of the output)

template <int N>
struct AttnState {
    float m, l;                // running max / sum of the lane's head (base-2 logits)
    f32x4 O[N];                // O^T of this quarter's dim blocks: dims 16*db + 4g + i
};

template <int N>
__device__ __forceinline__ void state_clear(AttnState<N> &s) {
    s.m = -INFINITY;
    s.l = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) s.O[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
}

// The running max of a subset's online softmax moves only when a chunk's
// largest logit exceeds it by more than 8 (base-2 units), so most chunks keep
// alpha = 1 and skip rescaling the accumulators; the weights 2^(l - m) then
// stay below 2^8, well inside bf16 and fp32.  The result is the same softmax
// (the common factor cancels in the final normalisation).
__device__ __forceinline__ float lazy_max(float m, float cmax) {
    return (m == -INFINITY || cmax > m + 8.0f) ? fmaxf(m, cmax) : m;
}

// fold(a, b): the two partial softmaxes rescaled to their common max.
__device__ __forceinline__ void fold_scales(float ma, float la, float mb, float lb, float &m, float &l,
                                            float &fa, float &fb) {
    m = fmaxf(ma, mb);
    fa = ma == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ma - m);
    fb = mb == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mb - m);
    l = la * fa + lb * fb;
}
__device__ __forceinline__ f32x4 fold_o(const f32x4 &a, float fa, const f32x4 &b, float fb) {
    return a * fa + b * fb;
}

// Max / sum over the four lanes of a head (lanes c16, c16+16, c16+32, c16+48)
// with the gfx950 row-swap permutes (VALU, no LDS).
__device__ __forceinline__ float head_max(float v) {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float head_sum(float v) {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Shapes shared by the kernel and its launcher.
template <int D, int DR>
struct AttnShape {
    static constexpr int DN = D - DR;
    static constexpr int NCH = DN / 16;                 // 16-byte pieces of E4M3 codes (16 dims each)
    static constexpr int RCH = DR / 8;                  // 16-byte pieces of BF16 RoPE dims (8 dims each)
    static constexpr int CREC = NCH + RCH + 1;          // + the piece holding the fp32 scale
    static constexpr int REC = (DN + 2 * DR + 4 + 63) / 64 * 64;   // stored record stride in HBM
    static constexpr int PPR = REC / 16;                // pieces per stored record (padding included)
    static constexpr int LW = REC % 128 == 0 ? 8 : 4;   // lanes per record in one load: a 128 (64)-byte line
    static constexpr int RPI = 64 / LW;                 // records per load instruction
    static constexpr int NLD = kChunk * PPR / 64;       // load instructions per chunk
    static constexpr int RS = PPR + 1;                  // LDS row stride in pieces (odd)
    static constexpr int SWZ = 4;                       // records 16..31 shifted by SWZ pieces
    static constexpr int BUF = (kChunk * RS + SWZ) * 16;   // LDS bytes of one chunk buffer
    static constexpr int KP = (NCH + 3) / 4;            // logits: MFMA pairs over the code pieces
    static constexpr int KR = (RCH + 3) / 4;            // logits: MFMAs over the RoPE pieces
    static constexpr int QPP = (KP + kParts - 1) / kParts;   // code pairs per dim part
    static constexpr int NDB = NCH + DR / 16;           // 16-dim blocks of the output
    static constexpr int DBQ = (NDB + kParts - 1) / kParts;  // output dim blocks per dim part
    static constexpr int XW = 2 * 4 * 64;               // floats of one part's partial logits
    static_assert(DN % 16 == 0 && DR % 16 == 0, "dims in whole 16-dim blocks");
    static_assert(NLD % kParts == 0, "a chunk's loads split evenly over the dim parts");
};

// NSW subset waves per dim part (1: the HI kernel, 2 waves).  Two waves per
// SIMD: the compiler fits the kernel into 256 registers (spilling a few
// dozen), and the second resident wave hides the chunk loop's latencies --
// measured on the 8K prefill chunk, 4.5 ms against 7.6 ms at one wave per
// SIMD (three per SIMD spill far more: 12.7 ms).
template <int D, int DR, int NSW, bool CSA, bool PREFILL>
__global__ __launch_bounds__(64 * kParts * NSW) __attribute__((amdgpu_waves_per_eu(2))) void k_attend(AttnArgs A) {
    using Sh = AttnShape<D, DR>;
    constexpr int NT = 64 * kParts * NSW;
    constexpr int NCH = Sh::NCH, RCH = Sh::RCH, CREC = Sh::CREC, PPR = Sh::PPR, LW = Sh::LW, RPI = Sh::RPI;
    constexpr int NLD = Sh::NLD, LDQ = NLD / kParts, RS = Sh::RS, SWZ = Sh::SWZ, BUF = Sh::BUF;
    constexpr int KP = Sh::KP, KR = Sh::KR, QPP = Sh::QPP, NDB = Sh::NDB, DBQ = Sh::DBQ, XW = Sh::XW;
    constexpr int DN = Sh::DN;

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ float2 rope_tab[DR / 2];
    __shared__ int32_t safe_sh;

    const Lay &L = A.L;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar registers)
    const int dq = wave % kParts, sw = wave / kParts;   // dim part, subset wave

    // ---- which query and head group (the 8 workgroups of a query are dealt
    // onto one XCD: workgroup ids go round-robin over the 8 XCDs)
    const int lin = blockIdx.x, x8 = lin & 7, u8 = lin >> 3;
    const int qi = (u8 / A.nhg) * 8 + x8;
    const int hg = u8 % A.nhg;
    if (qi >= A.nq) return;
    const QueryInfo Q = query_info<CSA, PREFILL>(A, qi);
    if (!Q.ok) return;
    const int head = hg * 16 + c16;
    const bool head_ok = head < L.H;

    // LDS: record locators, NSW chunk buffers, NSW partial-logit exchanges.
    // LO's final fold reuses the same bytes.
    int32_t *locs = (int32_t *)smem;
    const int loc_bytes = ((int)Q.n_list * 4 + 15) / 16 * 16;
    uint32_t *vmask = (uint32_t *)(smem + loc_bytes);   // [chunk]: bit r = record r usable
    const int head_bytes = loc_bytes + (((int)Q.n_list + kChunk - 1) / kChunk * 4 + 15) / 16 * 16;
    uint8_t *buf = smem + head_bytes + sw * BUF;
    float *xch = (float *)(smem + head_bytes + NSW * BUF) + sw * (kParts + 1) * XW;

    // ---- resolve every record of the list once; any valid record stands in
    // for masked ones (its bytes are loaded, its weight is 0)
    if (tid == 0) safe_sh = -1;
    __syncthreads();
    int32_t last_ok = -1;
    for (int64_t p0 = (int64_t)wave * 64; p0 < Q.n_list; p0 += NT) {   // wave-uniform: 64 consecutive records
        const int64_t p = p0 + lane;
        const int32_t lc = p < Q.n_list ? record_loc<CSA, PREFILL>(A, Q, p) : kMasked;
        if (p < Q.n_list) locs[p] = lc;
        if (lc != kMasked) last_ok = (int32_t)p;
        const uint64_t vb = __builtin_amdgcn_ballot_w64(lc != kMasked);
        if (lane == 0) {
            vmask[p0 / kChunk] = (uint32_t)vb;
            if (p0 + kChunk < Q.n_list) vmask[p0 / kChunk + 1] = (uint32_t)(vb >> 32);
        }
    }
    if (last_ok >= 0) atomicMax(&safe_sh, last_ok);
    if (tid < DR / 2) {
        float c, sn;
        rope_cs_theta(theta_lane(L, DR / 2), Q.t, c, sn);   // (lane l: theta_l from scalar reads)
        rope_tab[tid] = make_float2(c, sn);
    }
    __syncthreads();
    const int32_t safe = safe_sh >= 0 ? locs[safe_sh] : kMasked;
    const int n_list = (int)Q.n_list;                // (lists are far below 2^31 records)
    const int nchunks = safe == kMasked ? 0 : (n_list + kChunk - 1) / kChunk;

    static_assert(kParts == 2, "the part dispatch below covers two parts");
    // Everything below is compiled once per dim part (DQ), so that every LDS
    // and register index is a compile-time offset from a few lane bases.
    auto part_body = [&](auto dqc) {
        constexpr int DQ = decltype(dqc)::value;
        // ---- query fragments of this dim part (B operand of S^T = K Q^T), lane
        // (head c16, group g): code pair kp reads piece 4kp+g, dims 16(4kp+g) +
        // [0,8) and [8,16); RoPE step ks reads RoPE piece 4ks+g, rotated at t.
        bf16x8 Qn[QPP][2], Qr[KR];
        {
            const int64_t qbase = ((int64_t)Q.qrow * L.H + head) * D;
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
            for (int e = 0; e < QPP; ++e) {
                const int kp = QPP * DQ + e, ch = 4 * kp + g;
    #pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    if (head_ok && kp < KP && ch < NCH) q8(16 * ch + 8 * h, v);
                    bf16x8 f;
    #pragma unroll
                    for (int j = 0; j < 8; ++j) f[j] = f2bf(v[j]);
                    Qn[e][h] = f;
                }
            }
    #pragma unroll
            for (int ks = 0; ks < KR; ++ks) {
                const int ch = 4 * ks + g;
                float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (head_ok && DQ == kParts - 1 && ch < RCH) q8(DN + 8 * ch, v);
                bf16x8 f;
    #pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    float a = 0.0f, b = 0.0f;
                    if (ch < RCH) {
                        const float2 cs = rope_tab[(8 * ch + j) / 2];
                        a = v[j] * cs.x - v[j + 1] * cs.y;
                        b = v[j] * cs.y + v[j + 1] * cs.x;
                    }
                    f[j] = f2bf(a);
                    f[j + 1] = f2bf(b);
                }
                Qr[ks] = f;
            }
        }
        const float tau2 = L.tau * 1.4426950408889634f;   // logits in base 2

        // ---- chunk loads: the chunk's NLD loads are split over its part waves; in load i, lane l fetches piece LW*(i mod PPR/LW) + l%LW of record
        // RPI*(i / (PPR/LW)) + l/LW, so every load reads whole lines of RPI
        // records.  In LDS piece c of record r sits at r*RS + c (+SWZ for records
        // 16..31), which keeps the MFMA operand reads free of bank conflicts.
        const int ld_a = lane / LW, ld_b = lane % LW;
        auto slot = [&](int c, int r) { return buf + (r * RS + c + (r >> 4) * SWZ) * 16; };
        auto issue = [&](u32x4 (&pre)[LDQ], int ck) {
    #pragma unroll
            for (int e = 0; e < LDQ; ++e) {
                const int i = LDQ * DQ + e;
                const int r = RPI * (i / (PPR / LW)) + ld_a, c = LW * (i % (PPR / LW)) + ld_b;
                const int p = ck * kChunk + r;
                int32_t lc = locs[p < n_list ? p : n_list - 1];   // (no branch around the LDS read)
                if (p >= n_list || lc == kMasked) lc = safe;
                pre[e] = *(const u32x4 *)(loc_addr<PREFILL>(A, Q, lc) + 16 * c);
            }
        };
        auto stage = [&](const u32x4 (&pre)[LDQ]) {
    #pragma unroll
            for (int e = 0; e < LDQ; ++e) {
                const int i = LDQ * DQ + e;
                const int r = RPI * (i / (PPR / LW)) + ld_a, c = LW * (i % (PPR / LW)) + ld_b;
                *(u32x4 *)slot(c, r) = pre[e];
            }
        };

        // ---- this part's partial logits of a staged chunk: code dims of its
        // pairs (raw, scale not applied) and, in the last part, the RoPE dims;
        // rows = records 16rb + 4g + i, lane column = head c16
        auto partial = [&](float (&an)[2][4], float (&ar)[2][4]) {
    #pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, b = {0.0f, 0.0f, 0.0f, 0.0f};
    #pragma unroll
                for (int e = 0; e < QPP; ++e) {
                    const int kp = QPP * DQ + e, ch = 4 * kp + g;
                    if (kp < KP) {
                        u32x4 u = {0, 0, 0, 0};
                        if (NCH % 4 == 0 || ch < NCH) u = *(const u32x4 *)slot(ch, 16 * rb + c16);
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(u[0], u[1]), Qn[e][0], a, 0, 0, 0);
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(u[2], u[3]), Qn[e][1], a, 0, 0, 0);
                    }
                }
                if (DQ == kParts - 1) {
    #pragma unroll
                    for (int ks = 0; ks < KR; ++ks) {
                        const int ch = 4 * ks + g;
                        u32x4 u = {0, 0, 0, 0};
                        if (RCH % 4 == 0 || ch < RCH) u = *(const u32x4 *)slot(NCH + ch, 16 * rb + c16);
                        union { u32x4 v; bf16x8 b; } cv;
                        cv.v = u;
                        b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Qr[ks], b, 0, 0, 0);
                    }
                }
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    an[rb][i] = a[i];
                    ar[rb][i] = b[i];
                }
                __builtin_amdgcn_sched_barrier(0);   // one record block's operands at a time
            }
        };

        // ---- the rest of a chunk step, after the partials are exchanged: logits,
        // online softmax, O^T += V^T P^T on this part's dim blocks
        auto finish = [&](auto &S, int ck) {
            constexpr int NO = sizeof(S.O) / sizeof(S.O[0]);
            float lg[2][4], sc[2][4];
            const uint32_t vm = vmask[ck];
    #pragma unroll
            for (int rb = 0; rb < 2; ++rb)
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + 4 * g + i, k = (rb * 4 + i) * 64 + lane;
                    const bool ok = (vm >> r) & 1u;
                    sc[rb][i] = *(const float *)slot(CREC - 1, r);
                    float a = xch[k];
    #pragma unroll
                    for (int q = 1; q < kParts; ++q) a = a + xch[q * XW + k];
                    lg[rb][i] = ok ? tau2 * (sc[rb][i] * a + xch[kParts * XW + k]) : -INFINITY;
                }
            float cmax = -INFINITY;
    #pragma unroll
            for (int rb = 0; rb < 2; ++rb)
    #pragma unroll
                for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, lg[rb][i]);
            cmax = head_max(cmax);
            const float m_new = lazy_max(S.m, cmax);
            float p[2][4];
            float alpha = 1.0f;
            if (m_new == -INFINITY) {
    #pragma unroll
                for (int rb = 0; rb < 2; ++rb)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) p[rb][i] = 0.0f;
            } else {
                alpha = __builtin_amdgcn_exp2f(S.m - m_new);
    #pragma unroll
                for (int rb = 0; rb < 2; ++rb)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) p[rb][i] = __builtin_amdgcn_exp2f(lg[rb][i] - m_new);
            }
            float ps = 0.0f;
    #pragma unroll
            for (int rb = 0; rb < 2; ++rb)
    #pragma unroll
                for (int i = 0; i < 4; ++i) ps = ps + p[rb][i];
            ps = head_sum(ps);
            S.l = S.l * alpha + ps;
            S.m = m_new;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {   // alpha == 1 leaves O as it is
    #pragma unroll
                for (int i = 0; i < NO; ++i) S.O[i] = S.O[i] * alpha;
            }
            // k-slot j of lane group g is record 4g+j (j < 4) or 16+4g+(j-4): the
            // S^T rows this lane holds
            bf16x8 Pn, Pr;
    #pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int rb = j >> 2, i = j & 3;
                Pn[j] = f2bf(p[rb][i] * sc[rb][i]);
                Pr[j] = f2bf(p[rb][i]);
            }
            // code dims: ds_read_b64_tr_b8 -- lanes 2j, 2j+1 of the group address
            // row j (the record of k-slot j), 8 bytes each; lane c16 receives dim
            // c16 of the 8 records.  RoPE dims (bf16): ds_read_b64_tr_b16 -- lanes
            // 4r..4r+3 address row r (record 4g+r, resp. 16+4g+r), 4 dims each.
            const int trow = c16 >> 1, thalf = c16 & 1;
            const int trec = (trow < 4 ? 0 : 16) + 4 * g + (trow & 3);
            const int r16 = c16 >> 2, q16 = c16 & 3;
    #pragma unroll
            for (int ii = 0; ii < NO; ++ii) {
                if (ii % 4 == 0) __builtin_amdgcn_sched_barrier(0);   // bound the operands in flight
                const int db = DBQ * DQ + ii;
                if (db < NCH) {
                    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_p)(slot(db, trec) + 8 * thalf));
                    S.O[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8((uint32_t)v[0], (uint32_t)v[1]), Pn, S.O[ii], 0,
                                                                      0, 0);
                } else if (db < NDB) {
                    const int ch = NCH + 2 * (db - NCH) + (q16 >> 1);
                    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(slot(ch, 4 * g + r16) + 8 * (q16 & 1)));
                    i16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(slot(ch, 16 + 4 * g + r16) + 8 * (q16 & 1)));
                    union { i16x4 s[2]; bf16x8 b; } cv;
                    cv.s[0] = lo;
                    cv.s[1] = hi;
                    S.O[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Pr, S.O[ii], 0, 0, 0);
                }
            }
        };

        // ---- one chunk step of every subset wave: stage, exchange partials, finish.
        // ck < 0: this subset has no chunk at this step (the wave still takes part
        // in the workgroup barriers).
        auto step = [&](auto &S, int ck, u32x4 (&pre)[LDQ], int next) {
            __syncthreads();                             // the buffer's previous chunk is consumed
            if (ck >= 0) stage(pre);
            if (next >= 0) issue(pre, next);             // in flight during this step's compute
            __syncthreads();                             // staged chunk visible
            if (ck >= 0) {
                float an[2][4], ar[2][4];
                partial(an, ar);
    #pragma unroll
                for (int rb = 0; rb < 2; ++rb)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int k = (rb * 4 + i) * 64 + lane;
                        xch[DQ * XW + k] = an[rb][i];
                        if (DQ == kParts - 1) xch[kParts * XW + k] = ar[rb][i];
                    }
            }
            __syncthreads();                             // partials visible
            if (ck >= 0) finish(S, ck);
        };

        // ---- output rows d = 16db + 4g + i of head `head`, with the sink:
        // out = O * f / (l * f + 2^(z - M)),  f = 2^(m - M),  M = max(m, z)
        const int64_t obase = ((int64_t)Q.qrow * L.H + head) * D;
        // (the normalisation is computed once: with the output stores in
        // between, the compiler re-read the sink for every block, each read
        // waiting for the stores before it)
        auto out_scale = [&](float m, float l) {
            const float z = A.sinks[head] * 1.4426950408889634f;
            const float M = fmaxf(m, z);
            const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
            const float den = l * f + ((z == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - M));
            return den > 0.0f ? f / den : 0.0f;
        };
        auto emit = [&](float cf, int db, const f32x4 &o) {
            const int dd = db * 16 + 4 * g;
            if (L.act == DSV4_DT_BF16) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                const bf16x4 v = {f2bf(o[0] * cf), f2bf(o[1] * cf), f2bf(o[2] * cf), f2bf(o[3] * cf)};
                *(bf16x4 *)((uint16_t *)A.out + obase + dd) = v;
            } else {
                *(float4 *)((float *)A.out + obase + dd) = make_float4(o[0] * cf, o[1] * cf, o[2] * cf, o[3] * cf);
            }
        };

        u32x4 pre[LDQ];
        {
            // the subsets one after another on the same 2 waves
            AttnState<DBQ> acc, cur;
            state_clear(acc);
            int first = -1;                              // first chunk in processing order
            for (int s = 0; s < kSubsets && first < 0; ++s)
                if (s < nchunks) first = s;
            if (first >= 0) issue(pre, first);
    #pragma unroll 1
            for (int s = 0; s < kSubsets; ++s) {
                state_clear(cur);
    #pragma unroll 1
                for (int ck = s; ck < nchunks; ck += kSubsets) {
                    int next = ck + kSubsets;
                    if (next >= nchunks) {               // the next subset's first chunk
                        next = -1;
                        for (int s2 = s + 1; s2 < kSubsets && next < 0; ++s2)
                            if (s2 < nchunks) next = s2;
                    }
                    step(cur, ck, pre, next);
                }
                if (s == 0) {
                    acc = cur;
                } else {
                    float m, l, fa, fb;
                    fold_scales(acc.m, acc.l, cur.m, cur.l, m, l, fa, fb);
    #pragma unroll
                    for (int i = 0; i < DBQ; ++i) acc.O[i] = fold_o(acc.O[i], fa, cur.O[i], fb);
                    acc.m = m;
                    acc.l = l;
                }
            }
            if (head_ok) {
                const float cf = out_scale(acc.m, acc.l);
    #pragma unroll
                for (int i = 0; i < DBQ; ++i)
                    if (DBQ * DQ + i < NDB) emit(cf, DBQ * DQ + i, acc.O[i]);
            }
        }
    };
    if (dq == 0) part_body(std::integral_constant<int, 0>());
    else part_body(std::integral_constant<int, kParts - 1>());

}

// ---------------------------------------------------------------- the LO kernel
// Same decomposition and the same operations as k_attend, laid out for an
// unsaturated GPU: one workgroup of four waves per (query, 16-head group),
// wave s reducing subset s over all dims.  A wave stages its chunks through
// its own LDS buffer and exchanges nothing with the other waves until the
// final fold, so its chunk loop has no workgroup barrier, and it keeps the
// loads of its next two chunks in flight.  Its logits are summed from the
// same partial dot products as k_attend's dim parts (chain q over the code
// pairs [QPP*q, QPP*q + QPP), then a0 + a1, then the scale and the RoPE
// chain), so the two kernels agree bit for bit.
template <int D, int DR>
struct LoShape {
    using Sh = AttnShape<D, DR>;
    // per-wave LDS: locators [cpw][32] | valid masks [cpw] | RoPE table | chunk buffer
    static __host__ __device__ int wave_bytes(int cpw) {
        return cpw * kChunk * 4 + (cpw * 4 + 15) / 16 * 16 + (DR / 2 * 8 + 15) / 16 * 16 + Sh::BUF;
    }
    static constexpr int FOLD = kSubsets * 64 * 8 + kSubsets * Sh::NDB * 64 * 16;
    // the workgroup's 16 query rows (fp32 at most), rows padded by one piece
    static constexpr int QROW = D * 4 + 16;
    static constexpr int QBYTES = 16 * QROW;
};

constexpr int kLoPrefetch = 2;
constexpr int kLo8Group = 8;              // transposed reads per group in the eight-wave kernel

__device__ __forceinline__ void wave_lds_fence() {
    // the wave's LDS accesses are performed in order; this keeps the compiler
    // from moving one lane's LDS reads above another lane's writes
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

template <int D, int DR, bool CSA, bool PREFILL>
__global__ __launch_bounds__(64 * kSubsets) void k_attend_lo(AttnArgs A) {
    using Sh = AttnShape<D, DR>;
    constexpr int NCH = Sh::NCH, RCH = Sh::RCH, CREC = Sh::CREC, PPR = Sh::PPR, LW = Sh::LW, RPI = Sh::RPI;
    constexpr int NLD = Sh::NLD, RS = Sh::RS, SWZ = Sh::SWZ;
    constexpr int KP = Sh::KP, KR = Sh::KR, QPP = Sh::QPP, NDB = Sh::NDB, DN = Sh::DN;
    constexpr int RES = 8;                               // locators per lane per resolution batch
    constexpr int PFD = kLoPrefetch;                     // chunks of loads in flight per wave

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const Lay &L = A.L;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int sw = __builtin_amdgcn_readfirstlane(tid >> 6);   // subset of this wave

    const int lin = blockIdx.x, x8 = lin & 7, u8 = lin >> 3;
    const int qi = (u8 / A.nhg) * 8 + x8;
    const int hg = u8 % A.nhg;
    if (qi >= A.nq) return;
    // (CSA) the top-k indices of this wave's first resolution batch depend on
    // the query row alone once the window is full (list position p holds
    // top-k position p - W): read them now, beside the request and position,
    // instead of one round trip later (positions outside the row are
    // clamped; only those inside the list are used, and a query whose window
    // is not full reads its row again below)
    int32_t jpre[RES];
    if constexpr (CSA) {
#pragma unroll
        for (int u = 0; u < RES; ++u) {
            const int e = 64 * u + lane;
            const int p = (sw + kSubsets * (e >> 5)) * kChunk + (e & 31) - L.W;
            jpre[u] = A.topk[(int64_t)qi * L.topk + (p < 0 ? 0 : p < L.topk ? p : L.topk - 1)];
        }
    }
    const QueryInfo Q = query_info<CSA, PREFILL>(A, qi);
    if (!Q.ok) return;
    const int head = hg * 16 + c16;
    const bool head_ok = head < L.H;
    const int n_list = (int)Q.n_list;
    const int nchunks = (n_list + kChunk - 1) / kChunk;
    const int cpw = (nchunks + kSubsets - 1) / kSubsets;                    // chunks of wave 0 (the most)
    int mine = sw < nchunks ? (nchunks - 1 - sw) / kSubsets + 1 : 0;        // chunks sw, sw+4, ...
    uint8_t *wb = smem + sw * LoShape<D, DR>::wave_bytes(cpw);
    int32_t *locs = (int32_t *)wb;                                          // [t][32]: chunk sw + 4t
    uint32_t *vmask = (uint32_t *)(wb + cpw * kChunk * 4);
    float2 *rtab = (float2 *)(wb + cpw * kChunk * 4 + (cpw * 4 + 15) / 16 * 16);
    uint8_t *buf = (uint8_t *)rtab + (DR / 2 * 8 + 15) / 16 * 16;

    // ---- the query: the workgroup's 16 rows are fetched once (each thread a
    // few 16-byte pieces, clamped to the last head) and parked in LDS after
    // the locators resolve; rows are padded by one piece, so the fragment
    // reads below hit distinct banks
    const int ab = L.act == DSV4_DT_BF16 ? 2 : 4;
    const int qrow_bytes = D * ab;                       // bytes of one query row
    constexpr int QPT = (16 * D * 4 / 16 + 64 * kSubsets - 1) / (64 * kSubsets);   // pieces per thread (fp32 bound)
    uint8_t *qlds = smem + kSubsets * LoShape<D, DR>::wave_bytes(cpw);
    const int npc = qrow_bytes;                          // 16-byte pieces of the 16 rows
    u32x4 qpc[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int pc = tid + 64 * kSubsets * i;          // piece index over the 16 rows
        const int hr = pc / (qrow_bytes / 16), off = (pc % (qrow_bytes / 16)) * 16;
        const int hq = hg * 16 + hr < L.H ? hg * 16 + hr : L.H - 1;
        if (pc < npc)
            qpc[i] = *(const u32x4 *)((const uint8_t *)A.q + ((int64_t)Q.qrow * L.H + hq) * qrow_bytes + off);
    }

    // ---- locators of this wave's records, RES per lane per batch: the top-k
    // reads of a batch, then its block-table reads, each all in flight at
    // once (indices are clamped instead of branched around).  A masked record
    // is replaced by a stand-in that is always valid and finite -- the
    // query's own window record -- and keeps weight 0 through the valid mask.
    const int64_t n_ent = Q.n_ent, n_win = Q.n_win;
    const int32_t own = n_win > 0 ? window_loc<PREFILL>(A, Q, n_win - 1) : kMasked;
    int32_t first_ok = -1;                               // (no window: the wave's first valid record stands in)
    auto resolve = [&](int t_lo, int t_hi) {             // chunk ordinals [t_lo, t_hi) of this wave
        for (int e0 = t_lo * kChunk; e0 < t_hi * kChunk; e0 += 64 * RES) {
            // entries in this batch at all?  (wave-uniform: the window needs no reads)
            const bool any_ent = n_ent > 0 && (int64_t)(sw + kSubsets * ((e0 + 64 * RES - 1) >> 5)) * kChunk + 31 >= n_win;
            int64_t p[RES], j[RES];
            int32_t bid[RES];
#pragma unroll
            for (int u = 0; u < RES; ++u) {
                const int e = e0 + 64 * u + lane;
                p[u] = (int64_t)(sw + kSubsets * (e >> 5)) * kChunk + (e & 31);
                if (e >= t_hi * kChunk) p[u] = Q.n_list;   // past the range: masked
                j[u] = p[u];
                bid[u] = -1;
            }
            if (any_ent) {
                if constexpr (CSA) {
                    if (e0 == 0 && n_win == L.W) {       // the pre-read row (uniform)
#pragma unroll
                        for (int u = 0; u < RES; ++u) j[u] = jpre[u];
                    } else {
#pragma unroll
                        for (int u = 0; u < RES; ++u) {
                            const int64_t e = p[u] - n_win;
                            const int64_t pc = e < 0 ? 0 : e < n_ent ? e : n_ent - 1;
                            j[u] = A.topk[(int64_t)Q.qrow * L.topk + pc];
                        }
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < RES; ++u) j[u] = p[u] - n_win;
                }
#pragma unroll
                for (int u = 0; u < RES; ++u) {
                    const bool ent = p[u] >= n_win && p[u] - n_win < n_ent && j[u] >= 0 && j[u] < Q.n_vis;
                    const int64_t blk = ent ? (j[u] * L.m) / kBlockTokens : 0;
                    bid[u] = A.C.block_table[(int64_t)Q.r * A.C.max_blocks + blk];
                }
            }
            int32_t lc[RES];
#pragma unroll
            for (int u = 0; u < RES; ++u) {
                const bool ent = p[u] >= n_win && p[u] - n_win < n_ent && j[u] >= 0 && j[u] < Q.n_vis;
                const int32_t l_ent =
                    (ent && bid[u] >= 0 && bid[u] < A.C.n_blocks) ? (int32_t)(bid[u] * L.epb + (j[u] & (L.epb - 1))) : kMasked;
                lc[u] = p[u] < n_win ? window_loc<PREFILL>(A, Q, p[u]) : l_ent;
            }
#pragma unroll
            for (int u = 0; u < RES; ++u) {
                const int e = e0 + 64 * u + lane;
                const uint64_t vb = __builtin_amdgcn_ballot_w64(lc[u] != kMasked);
                if (first_ok < 0 && vb != 0)
                    first_ok = __builtin_amdgcn_readlane(lc[u], (int)__builtin_ctzll(vb));
                if (e < t_hi * kChunk) locs[e] = lc[u] != kMasked ? lc[u] : own;
                const int t0 = (e0 + 64 * u) >> 5;
                if (lane == 0) {
                    if (t0 < t_hi) vmask[t0] = (uint32_t)vb;
                    if (t0 + 1 < t_hi) vmask[t0 + 1] = (uint32_t)(vb >> 32);
                }
            }
        }
    };

    // ---- chunk loads, all NLD of a chunk on this wave.  When the code and
    // RoPE pieces each come in whole groups of four, a chunk is loaded in the
    // logits' operand layout -- lane (g, c16) holds pieces 4k+g of record
    // 16rb+c16, load rb*KPR+k -- and the logits take their key operands from
    // those registers; LDS then holds the chunk only for the transposed reads
    // of O^T += V^T P^T (and the scales).  Otherwise the loads follow k_attend's
    // line-wise pattern and both products read the chunk from LDS.
    constexpr bool REGQK = NCH % 4 == 0 && RCH % 4 == 0;
    constexpr int KPR = PPR / 4;                         // loads per record block (operand layout)
    static_assert(PPR % 4 == 0 && NLD == 2 * KPR, "two record blocks of KPR loads per chunk");
    const int ld_a = lane / LW, ld_b = lane % LW;
    auto slot = [&](int c, int r) { return buf + (r * RS + c + (r >> 4) * SWZ) * 16; };
    auto piece_rc = [&](int i, int &r, int &c) {
        if constexpr (REGQK) {
            r = 16 * (i / KPR) + c16;
            c = 4 * (i % KPR) + g;
        } else {
            r = RPI * (i / (PPR / LW)) + ld_a;
            c = LW * (i % (PPR / LW)) + ld_b;
        }
    };
    auto issue = [&](u32x4 (&pre)[NLD], int t) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            int r, c;
            piece_rc(i, r, c);
            pre[i] = *(const u32x4 *)(loc_addr<PREFILL>(A, Q, locs[t * kChunk + r]) + 16 * c);
        }
    };
    auto stage = [&](const u32x4 (&pre)[NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            int r, c;
            piece_rc(i, r, c);
            *(u32x4 *)slot(c, r) = pre[i];
        }
    };
    u32x4 R0[NLD], R1[PFD == 2 ? NLD : 1];
    resolve(0, mine);
    if (own == kMasked) {                                // no window (W = 0)
        if (first_ok < 0) mine = 0;                      // nothing valid: the subset contributes nothing
        wave_lds_fence();
        for (int e = lane; e < mine * kChunk; e += 64)
            if (locs[e] == kMasked) locs[e] = first_ok;
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int pc = tid + 64 * kSubsets * i;
        const int hr = pc / (qrow_bytes / 16), off = (pc % (qrow_bytes / 16)) * 16;
        if (pc < npc) *(u32x4 *)(qlds + hr * LoShape<D, DR>::QROW + off) = qpc[i];
    }
    __syncthreads();                                     // query rows and this wave's locators visible
    if (mine > 0) issue(R0, 0);
    if constexpr (PFD == 2)
        if (mine > 1) issue(R1, 1);
    // query fragments of head c16 from LDS: code pair kp holds piece 4kp+g
    // (bf16 queries are the MFMA operand bits as they are)
    const uint8_t *qh = qlds + c16 * LoShape<D, DR>::QROW;
    auto q8 = [&](int dd, float (&v)[8]) {               // 8 query values from dim dd
        if (L.act == DSV4_DT_BF16) {
            const u32x4 u = *(const u32x4 *)(qh + dd * 2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = __uint_as_float(u[j] << 16);
                v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
            }
        } else {
            const u32x4 a = *(const u32x4 *)(qh + dd * 4), b = *(const u32x4 *)(qh + dd * 4 + 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = __uint_as_float(a[j]);
                v[4 + j] = __uint_as_float(b[j]);
            }
        }
    };
    bf16x8 Qn[KP][2];
#pragma unroll
    for (int kp = 0; kp < KP; ++kp)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ch = 4 * kp + g;
            bf16x8 f;
            if (L.act == DSV4_DT_BF16) {
                u32x4 u = {0, 0, 0, 0};
                if (NCH % 4 == 0 || ch < NCH) u = *(const u32x4 *)(qh + (16 * ch + 8 * h) * 2);
                union { u32x4 v; bf16x8 b; } cv;
                cv.v = u;
                f = cv.b;
            } else {
                float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (NCH % 4 == 0 || ch < NCH) q8(16 * ch + 8 * h, v);
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] = f2bf(v[j]);
            }
            Qn[kp][h] = f;
        }
    if (lane < DR / 2) {
        float c, sn;
        rope_cs_theta(theta_lane(L, DR / 2), Q.t, c, sn);   // (lane l: theta_l from scalar reads)
        rtab[lane] = make_float2(c, sn);
    }
    wave_lds_fence();

    // ---- RoPE query fragments, rotated at t (the code fragments are above):
    // code pair kp holds piece 4kp+g, RoPE step ks RoPE piece 4ks+g
    bf16x8 Qr[KR];
#pragma unroll
    for (int ks = 0; ks < KR; ++ks) {
        const int ch = 4 * ks + g;
        float qr[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (RCH % 4 == 0 || ch < RCH) q8(DN + 8 * ch, qr);
        bf16x8 f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            float a = 0.0f, b = 0.0f;
            if (ch < RCH) {
                const float2 cs = rtab[(8 * ch + j) / 2];
                a = qr[j] * cs.x - qr[j + 1] * cs.y;
                b = qr[j] * cs.y + qr[j + 1] * cs.x;
            }
            f[j] = f2bf(a);
            f[j + 1] = f2bf(b);
        }
        Qr[ks] = f;
    }
    const float tau2 = L.tau * 1.4426950408889634f;   // logits in base 2

    // ---- one chunk: logits from the partial chains, online softmax, O^T += V^T P^T
    AttnState<NDB> S;
    state_clear(S);
    auto compute = [&](int t, u32x4 (&pre)[NLD], bool refill) {
        float lg[2][4], sc[2][4];
        float dot[2][4], dr[2][4];
        const uint32_t vm = vmask[t];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            // all of the block's operand pieces first (from the registers, or
            // from LDS with their latencies overlapped), then the chains
            // interleaved: chain q keeps its pairs in order
            u32x4 u[KP], ur[KR];
#pragma unroll
            for (int kp = 0; kp < KP; ++kp) {
                const int ch = 4 * kp + g;
                u[kp] = (u32x4){0, 0, 0, 0};
                if constexpr (REGQK) u[kp] = pre[rb * KPR + kp];
                else if (NCH % 4 == 0 || ch < NCH) u[kp] = *(const u32x4 *)slot(ch, 16 * rb + c16);
            }
#pragma unroll
            for (int ks = 0; ks < KR; ++ks) {
                const int ch = 4 * ks + g;
                ur[ks] = (u32x4){0, 0, 0, 0};
                if constexpr (REGQK) ur[ks] = pre[rb * KPR + NCH / 4 + ks];
                else if (RCH % 4 == 0 || ch < RCH) ur[ks] = *(const u32x4 *)slot(NCH + ch, 16 * rb + c16);
            }
            f32x4 x[kParts], xr = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int q = 0; q < kParts; ++q) x[q] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < QPP; ++e)
#pragma unroll
                for (int q = 0; q < kParts; ++q) {
                    const int kp = QPP * q + e;
                    if (kp < KP) {
                        x[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(u[kp][0], u[kp][1]), Qn[kp][0], x[q], 0, 0, 0);
                        x[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(u[kp][2], u[kp][3]), Qn[kp][1], x[q], 0, 0, 0);
                    }
                }
#pragma unroll
            for (int ks = 0; ks < KR; ++ks) {
                union { u32x4 v; bf16x8 b; } cv;
                cv.v = ur[ks];
                xr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Qr[ks], xr, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float a = x[0][i];
#pragma unroll
                for (int q = 1; q < kParts; ++q) a = a + x[q][i];
                dot[rb][i] = a;
                dr[rb][i] = xr[i];
            }
            __builtin_amdgcn_sched_barrier(0);   // one record block's operands at a time
        }
        if constexpr (REGQK) {                   // the registers are free: next loads, then the staged chunk
            if (refill) issue(pre, t + PFD);
            wave_lds_fence();
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rb + 4 * g + i;
                const bool ok = (vm >> r) & 1u;
                sc[rb][i] = *(const float *)slot(CREC - 1, r);
                lg[rb][i] = ok ? tau2 * (sc[rb][i] * dot[rb][i] + dr[rb][i]) : -INFINITY;
            }
        float cmax = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, lg[rb][i]);
        cmax = head_max(cmax);
        const float m_new = lazy_max(S.m, cmax);
        float p[2][4];
        float alpha = 1.0f;
        if (m_new == -INFINITY) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[rb][i] = 0.0f;
        } else {
            alpha = __builtin_amdgcn_exp2f(S.m - m_new);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[rb][i] = __builtin_amdgcn_exp2f(lg[rb][i] - m_new);
        }
        float ps = 0.0f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ps = ps + p[rb][i];
        ps = head_sum(ps);
        S.l = S.l * alpha + ps;
        S.m = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int i = 0; i < NDB; ++i) S.O[i] = S.O[i] * alpha;
        }
        bf16x8 Pn, Pr;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int rb = j >> 2, i = j & 3;
            Pn[j] = f2bf(p[rb][i] * sc[rb][i]);
            Pr[j] = f2bf(p[rb][i]);
        }
        const int trow = c16 >> 1, thalf = c16 & 1;
        const int trec = (trow < 4 ? 0 : 16) + 4 * g + (trow & 3);
        const int r16 = c16 >> 2, q16 = c16 & 3;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            if (db % 4 == 0) __builtin_amdgcn_sched_barrier(0);   // bound the operands in flight
            if (db < NCH) {
                const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_p)(slot(db, trec) + 8 * thalf));
                S.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8((uint32_t)v[0], (uint32_t)v[1]), Pn, S.O[db], 0,
                                                                  0, 0);
            } else {
                const int ch = NCH + 2 * (db - NCH) + (q16 >> 1);
                i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(slot(ch, 4 * g + r16) + 8 * (q16 & 1)));
                i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(slot(ch, 16 + 4 * g + r16) + 8 * (q16 & 1)));
                union { i16x4 s[2]; bf16x8 b; } cv;
                cv.s[0] = lo;
                cv.s[1] = hi;
                S.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Pr, S.O[db], 0, 0, 0);
            }
        }
    };
    auto step = [&](u32x4 (&pre)[NLD], int t) {
        wave_lds_fence();                    // the previous chunk's reads come first
        stage(pre);
        if constexpr (!REGQK) {
            if (t + PFD < mine) issue(pre, t + PFD);
            wave_lds_fence();                // staged chunk visible to the whole wave
        }
        compute(t, pre, t + PFD < mine);
    };
    if constexpr (PFD == 2) {
#pragma unroll 1
        for (int t = 0; t < mine; t += 2) {
            step(R0, t);
            if (t + 1 < mine) step(R1, t + 1);
        }
    } else {
#pragma unroll 1
        for (int t = 0; t < mine; ++t) step(R0, t);
    }

    // ---- fold the four subset states left to right through LDS (the same
    // operations as k_attend's sequential fold); wave s emits dim blocks s, s+4, ...
    __syncthreads();
    float2 *ml = (float2 *)smem;                                 // [subset][64]
    f32x4 *ob = (f32x4 *)(smem + kSubsets * 64 * 8);             // [subset][NDB][64]
    ml[sw * 64 + lane] = make_float2(S.m, S.l);
#pragma unroll
    for (int b = 0; b < NDB; ++b) ob[(sw * NDB + b) * 64 + lane] = S.O[b];
    __syncthreads();
    float m = ml[lane].x, l = ml[lane].y;
    float fw[kSubsets][2];
#pragma unroll
    for (int s = 1; s < kSubsets; ++s) {
        const float2 b = ml[s * 64 + lane];
        float mm, ll, fa, fb;
        fold_scales(m, l, b.x, b.y, mm, ll, fa, fb);
        fw[s][0] = fa;
        fw[s][1] = fb;
        m = mm;
        l = ll;
    }
    if (!head_ok) return;
    const float z = A.sinks[head] * 1.4426950408889634f;
    const float M = fmaxf(m, z);
    const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    const float den = l * f + ((z == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - M));
    const float cf = den > 0.0f ? f / den : 0.0f;
    const int64_t obase = ((int64_t)Q.qrow * L.H + head) * D;
#pragma unroll
    for (int b = sw; b < NDB; b += kSubsets) {
        f32x4 o = ob[b * 64 + lane];
#pragma unroll
        for (int s = 1; s < kSubsets; ++s) o = fold_o(o, fw[s][0], ob[(s * NDB + b) * 64 + lane], fw[s][1]);
        const int dd = b * 16 + 4 * g;
        if (L.act == DSV4_DT_BF16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 v = {f2bf(o[0] * cf), f2bf(o[1] * cf), f2bf(o[2] * cf), f2bf(o[3] * cf)};
            *(bf16x4 *)((uint16_t *)A.out + obase + dd) = v;
        } else {
            *(float4 *)((float *)A.out + obase + dd) = make_float4(o[0] * cf, o[1] * cf, o[2] * cf, o[3] * cf);
        }
    }
}

// ---------------------------------------------------------------- the LO kernel, eight waves (d = 512)
// The same decomposition and operations once more, on eight waves per (query,
// 16-head group): wave (s, q) reduces subset s over dim part q.  A part's code
// pairs of the logits and its dim blocks of the output cover the same 16-byte
// pieces of a record (part 0: the code pieces [0, 4*QPP); part 1: the other
// code pieces, the RoPE pieces and the scale), so a wave loads only its own
// pieces -- into registers in the logits' operand layout, the key operands of
// S^T = K Q^T taken straight from them, and then into its own LDS buffer for
// the transposed reads of O^T += V^T P^T.  The two parts of a subset exchange
// their partial logits (part 1 also the RoPE logits and the record scales)
// through LDS, and both run the same online softmax on the same logits.  With
// 64 accumulator registers a wave (its 16 dim blocks), two waves share each
// SIMD.  Subsets 0-1 and 2-3 run half a chunk step apart (one workgroup
// barrier between the halves), so while one wave of a SIMD runs its softmax
// and O^T += V^T P^T the other runs its logits.  Every load a wave makes is
// issued unconditionally (a step past the subset's end reads a harmless
// stand-in address and is not consumed), which keeps the compiler's
// memory-counter waits exact: a step waits for its own chunk only, with the
// next one still in flight.  Every logit, weight and accumulator takes the
// operations of k_attend's dim parts in the same order, so the kernels agree
// bit for bit.
template <int D, int DR>
struct Lo8Shape {
    using Sh = AttnShape<D, DR>;
    static constexpr int KPR = Sh::PPR / 4;                  // piece groups per record (group k: pieces 4k..4k+3)
    static constexpr int G1 = Sh::QPP;                      // part 0: groups [0, G1); part 1: [G1, KPR)
    static constexpr int NG0 = G1, NG1 = KPR - G1;          // piece groups of each part per record block
    static constexpr int NST0 = G1, NST1 = Sh::KP + Sh::KR - G1;   // groups each part stages for its dim blocks
    static constexpr int RS0 = 4 * NST0 + 1, RS1 = 4 * NST1 + 1;  // LDS row strides in pieces (odd)
    // records 16..31 shifted by 8 pieces (32 banks): the transposed reads of a
    // half-wave (records 4g..4g+3 and 16+4g.. of two lane groups) then fall on
    // distinct banks (a shift of 4 made them collide pairwise)
    static constexpr int SWZ = 8;
    static constexpr int BUF0 = (kChunk * RS0 + SWZ) * 16, BUF1 = (kChunk * RS1 + SWZ) * 16;
    static constexpr int XWF = 8 * 64;                     // floats of one partial-logit array
    static constexpr int XSLOT = 3 * XWF + kChunk;         // a0, a1, RoPE logits, the chunk's 32 scales
    static constexpr int MAXC = 16;                         // chunks per subset (one locator batch)
    static constexpr int LOC = MAXC * kChunk * 4 + MAXC * 4;   // a subset's locators and valid masks
    static constexpr int RT = DR / 2 * 8;                   // the RoPE table (part 1 of each subset)
    static constexpr int XOFF = kSubsets * (BUF0 + BUF1);
    static constexpr int LOFF = XOFF + kSubsets * XSLOT * 4;
    static constexpr int STREAM = LOFF + kSubsets * (LOC + RT);
    static constexpr int FOLD = kSubsets * 64 * 8 + kSubsets * Sh::NDB * 64 * 16;
    static constexpr int LDS = STREAM > FOLD ? STREAM : FOLD;
    static constexpr int MAX_LIST = kSubsets * MAXC * kChunk;   // longest record list it takes
    static_assert(Sh::NCH % 4 == 0 && Sh::RCH % 4 == 0 && Sh::PPR % 4 == 0, "pieces in whole groups of four");
    static_assert(Sh::DBQ == 4 * Sh::QPP, "a part's dim blocks are the pieces of its code pairs");
    static_assert(Sh::KP + Sh::KR < KPR, "the scale piece follows the RoPE pieces");
    static_assert(BUF0 % 16 == 0 && BUF1 % 16 == 0 && (XSLOT * 4) % 16 == 0 && (LOC + RT) % 16 == 0, "alignment");
    static_assert(kSubsets == 4, "two groups of two subsets");
};

template <int D, int DR, bool CSA, bool PREFILL, bool F32A>
__global__ __launch_bounds__(64 * kSubsets * kParts) void k_attend_lo8(AttnArgs A) {
    using Sh = AttnShape<D, DR>;
    using S8 = Lo8Shape<D, DR>;
    constexpr int NCH = Sh::NCH, RCH = Sh::RCH, KP = Sh::KP, KR = Sh::KR, QPP = Sh::QPP, NDB = Sh::NDB;
    constexpr int DBQ = Sh::DBQ, DN = Sh::DN, G1 = S8::G1, XWF = S8::XWF, SWZ = S8::SWZ, MAXC = S8::MAXC;
    constexpr int RESH = MAXC * kChunk / 64 / kParts;    // locators per lane each part resolves
    static_assert(RESH * 64 * kParts == MAXC * kChunk, "the parts split the locator batch");

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const Lay &L = A.L;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;                           // 0: subsets 0-1; 1: subsets 2-3, half a step later
    const int sw = 2 * grp + ((wave >> 1) & 1);          // subset (the dim part is wave & 1)

    const int lin = blockIdx.x, x8 = lin & 7, u8 = lin >> 3;
    const int qi = (u8 / A.nhg) * 8 + x8;
    const int hg = u8 % A.nhg;
    if (qi >= A.nq) return;
    const int head = hg * 16 + c16;
    const bool head_ok = head < L.H;

    static_assert(kParts == 2, "the part dispatch below covers two parts");
    auto part_body = [&](auto dqc) {
        constexpr int DQ = decltype(dqc)::value;
        constexpr int NG = DQ == 0 ? S8::NG0 : S8::NG1;  // piece groups per record block
        constexpr int NGL = DQ == 0 ? NG : NG - 1;       // 16-byte loads per record block (part 1: + the scale)
        constexpr int GB = DQ == 0 ? 0 : G1;             // first piece group
        constexpr int NST = DQ == 0 ? S8::NST0 : S8::NST1;
        constexpr int RS = DQ == 0 ? S8::RS0 : S8::RS1;
        constexpr int NPAIR = DQ == 0 ? QPP : KP - QPP;  // code pairs of this part's logits
        constexpr int NQ = 2 * NPAIR + (DQ == 1 ? KR : 0);   // query pieces of 8 dims
        uint8_t *buf = smem + sw * (S8::BUF0 + S8::BUF1) + (DQ == 0 ? 0 : S8::BUF0);
        float *xs = (float *)(smem + S8::XOFF) + sw * S8::XSLOT;             // the subset's exchange slot
        uint8_t *sl = smem + S8::LOFF + sw * (S8::LOC + S8::RT);
        int32_t *locs = (int32_t *)sl;                                      // [t][32]: chunk sw + 4t
        uint32_t *vmask = (uint32_t *)(sl + MAXC * kChunk * 4);
        float2 *rtab = (float2 *)(sl + S8::LOC);

        constexpr bool f32act = F32A;                    // fp32 activations (else bf16)
        constexpr int ab = f32act ? 4 : 2;
        const uint8_t *qrow = (const uint8_t *)A.q + ((int64_t)qi * L.H + (head_ok ? head : L.H - 1)) * D * ab;
        // ---- the query pieces of this part, first of all (their addresses
        // need only the workgroup's query and head group): code pair kp, half h
        // reads dims 16(4kp+g) + 8h .. +8; RoPE step ks reads dims DN +
        // 8(4ks+g) .. +8.  bf16 rows take one 16-byte load a piece, fp32 rows
        // two.  Measured 0.5 us faster per launch than issuing them behind the
        // block-table reads.
        u32x4 qa[NQ], qb[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int dd = i < 2 * NPAIR ? 16 * (4 * (QPP * DQ + i / 2) + g) + 8 * (i & 1)
                                         : DN + 8 * (4 * (i - 2 * NPAIR) + g);
            const uint8_t *pa = qrow + dd * ab;
            qa[i] = *(const u32x4 *)pa;
            if constexpr (f32act) qb[i] = *(const u32x4 *)(pa + 16);
        }
        // (CSA) the top-k indices of this part's half of the subset's records,
        // read beside the request and position: once the window is full, list
        // position p holds top-k position p - W (positions outside the row are
        // clamped and not used; a query whose window is not full reads its row
        // again below)
        int32_t jpre[RESH];
        if constexpr (CSA) {
#pragma unroll
            for (int u = 0; u < RESH; ++u) {
                const int e = 64 * (RESH * DQ + u) + lane;
                const int p = (sw + kSubsets * (e >> 5)) * kChunk + (e & 31) - L.W;
                jpre[u] = A.topk[(int64_t)qi * L.topk + (p < 0 ? 0 : p < L.topk ? p : L.topk - 1)];
            }
        }
        // (CSA) and the top-k indices of the lane's two records of the
        // subset's second chunk (list chunk sw + 4), which the fast start
        // below resolves per lane
        int32_t t1[2] = {0, 0};
        if constexpr (CSA) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int p = (sw + kSubsets) * kChunk + 16 * rb + c16 - L.W;
                t1[rb] = A.topk[(int64_t)qi * L.topk + (p < 0 ? 0 : p < L.topk ? p : L.topk - 1)];
            }
        }
        const QueryInfo Q = query_info<CSA, PREFILL>(A, qi);
        if (!Q.ok) return;                               // (the whole workgroup)
        const int n_list = (int)Q.n_list;
        const int n_win = Q.n_win;
        // Fast start (a full window of four chunks): a subset's first chunk is
        // window records, known from the position alone, and each lane resolves
        // its two records of the second chunk itself, so both chunks' loads go
        // out before the loop without waiting for the shared locators; those
        // become visible at the first step's barrier.  (Uniform per workgroup.)
        const bool fast = n_win == L.W && L.W == kSubsets * kChunk;
        const int nchunks = (n_list + kChunk - 1) / kChunk;
        const int cpw = (nchunks + kSubsets - 1) / kSubsets;                 // chunks of subset 0 (the most)
        int mine = sw < nchunks ? (nchunks - 1 - sw) / kSubsets + 1 : 0;     // chunks sw, sw+4, ...
        // the stand-in for masked records (always valid and finite): the
        // query's own window record, else (no window) the subset's first valid
        // record, found below
        int32_t stand = n_win > 0 ? window_loc<PREFILL>(A, Q, n_win - 1) : kMasked;
        // loads of a step past the subset's end read the query row instead
        // (valid memory; such a step's results are never consumed)
        const uint8_t *qsafe = qrow;
        // ---- this part's loads of chunk t: lane (g, c16) fetches piece 4k+g of
        // record 16rb+c16 for the part's groups k (part 1: the scale as one
        // word, the rest of its group being padding)
        auto locs_of = [&](int t, int32_t (&lc)[2]) {   // the lane's records of chunk t (rb = 0, 1)
            const int tt = t < mine ? t : 0;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) lc[rb] = locs[tt * kChunk + 16 * rb + c16];
        };
        auto issue = [&](u32x4 (&pre)[2 * NGL], uint32_t (&scl)[2], int t, const int32_t (&lcs)[2]) {
            const bool in = t < mine;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int32_t lc = lcs[rb] == kMasked ? stand : lcs[rb];
                const uint8_t *rec = in ? loc_addr<PREFILL>(A, Q, lc) : qsafe;
                const uint8_t *pc = rec + 16 * g;
#pragma unroll
                for (int k = 0; k < NGL; ++k) pre[rb * NGL + k] = *(const u32x4 *)(pc + 64 * (GB + k));
                if constexpr (DQ == 1) scl[rb] = *(const uint32_t *)(rec + 16 * (Sh::CREC - 1));
            }
        };
        u32x4 R0[2 * NGL], R1[2 * NGL];
        uint32_t C0[2], C1[2];

        // ---- locators of the subset's records: this part resolves chunk
        // ordinals [8 DQ, 8 DQ + 8) -- its top-k reads, then its block-table
        // reads, all in flight at once -- into the subset's shared array
        {
            const int64_t n_ent = Q.n_ent;
            int32_t p[RESH], j[RESH], bid[RESH];
#pragma unroll
            for (int u = 0; u < RESH; ++u) {
                const int e = 64 * (RESH * DQ + u) + lane;
                p[u] = (sw + kSubsets * (e >> 5)) * kChunk + (e & 31);
                if (e >= mine * kChunk) p[u] = n_list;                       // past the subset: masked
            }
            if constexpr (CSA) {
                if (n_win != L.W) {                      // (window not full: the row again, at p - n_win)
#pragma unroll
                    for (int u = 0; u < RESH; ++u) {
                        const int64_t en = (int64_t)p[u] - n_win;
                        jpre[u] = A.topk[(int64_t)qi * L.topk + (en < 0 ? 0 : en < n_ent ? en : n_ent - 1)];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < RESH; ++u) {
                const int64_t en = (int64_t)p[u] - n_win;                    // entry position
                j[u] = (int32_t)en;
                if constexpr (CSA) j[u] = jpre[u];
                const bool ent = en >= 0 && en < n_ent && j[u] >= 0 && j[u] < Q.n_vis;
                const int64_t blk = ent ? ((int64_t)j[u] * L.m) / kBlockTokens : 0;
                bid[u] = A.C.block_table[(int64_t)Q.r * A.C.max_blocks + blk];
            }
            // the lane's second-chunk records (fast start): their block-table reads
            int32_t j1[2], bt1[2];
            bool ok1[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int64_t en = (int64_t)(sw + kSubsets) * kChunk + 16 * rb + c16 - n_win;
                j1[rb] = CSA ? t1[rb] : (int32_t)en;
                ok1[rb] = en >= 0 && en < n_ent && j1[rb] >= 0 && j1[rb] < Q.n_vis;
                const int64_t blk = ok1[rb] ? ((int64_t)j1[rb] * L.m) / kBlockTokens : 0;
                bt1[rb] = A.C.block_table[(int64_t)Q.r * A.C.max_blocks + blk];
            }
            // fast start: the first chunk's loads go out now, behind the
            // block-table reads (loads complete in order: waiting for the block
            // table does not wait for them), then the second chunk's, once its
            // block ids are in
            if (fast) {
                int32_t l0[2], l1[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) l0[rb] = window_loc<PREFILL>(A, Q, sw * kChunk + 16 * rb + c16);
                issue(R0, C0, 0, l0);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    l1[rb] = (ok1[rb] && bt1[rb] >= 0 && bt1[rb] < A.C.n_blocks) ? (int32_t)(bt1[rb] * L.epb + (j1[rb] & (L.epb - 1)))
                                                                                 : kMasked;
                issue(R1, C1, 1, l1);
            }
#pragma unroll
            for (int u = 0; u < RESH; ++u) {
                const int e = 64 * (RESH * DQ + u) + lane;
                const int64_t en = (int64_t)p[u] - n_win;
                const bool ent = en >= 0 && en < n_ent && j[u] >= 0 && j[u] < Q.n_vis;
                const int32_t l_ent =
                    (ent && bid[u] >= 0 && bid[u] < A.C.n_blocks) ? (int32_t)(bid[u] * L.epb + (j[u] & (L.epb - 1))) : kMasked;
                const int32_t lc = p[u] < n_win ? window_loc<PREFILL>(A, Q, p[u]) : l_ent;
                const uint64_t vb = __builtin_amdgcn_ballot_w64(lc != kMasked);
                if (e < mine * kChunk) locs[e] = lc;
                const int t0 = 2 * (RESH * DQ + u);       // the two chunk ordinals of this locator row
                if (lane == 0) {
                    if (t0 < mine) vmask[t0] = (uint32_t)vb;
                    if (t0 + 1 < mine) vmask[t0 + 1] = (uint32_t)(vb >> 32);
                }
            }
        }
        if constexpr (DQ == 1) {
            if (lane < DR / 2) {
                float c, sn;
                rope_cs_theta(theta_lane(L, DR / 2), Q.t, c, sn);   // (lane l: theta_l from scalar reads)
                rtab[lane] = make_float2(c, sn);
            }
        }
        wave_lds_fence();                                // (the RoPE table: this wave's own)
        if (!fast) {                                     // (uniform: every wave of the workgroup)
            __syncthreads();                             // locators and masks visible
            if (stand == kMasked) {                      // no window: the subset's first valid record
                int c = 0;
                while (c < mine && vmask[c] == 0) ++c;
                if (c < mine) stand = locs[c * kChunk + __builtin_ctz(vmask[c])];
                else mine = 0;                           // nothing valid: the subset contributes nothing
            }
            int32_t l0[2], l1[2];
            locs_of(0, l0);
            locs_of(1, l1);
            issue(R0, C0, 0, l0);
            issue(R1, C1, 1, l1);
        }

        // ---- query fragments (B operand of S^T = K Q^T); RoPE ones rotated at t
        auto piece8 = [&](int i, float (&v)[8]) {
            if (!f32act) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = __uint_as_float(qa[i][j] << 16);
                    v[2 * j + 1] = __uint_as_float(qa[i][j] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = __uint_as_float(qa[i][j]);
                    v[4 + j] = __uint_as_float(qb[i][j]);
                }
            }
        };
        bf16x8 Qn[NPAIR][2];
#pragma unroll
        for (int e = 0; e < NPAIR; ++e)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float v[8];
                piece8(2 * e + h, v);
                bf16x8 f;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) f[jj] = f2bf(v[jj]);
                Qn[e][h] = f;
            }
        bf16x8 Qr[DQ == 1 ? KR : 1];
        if constexpr (DQ == 1) {
#pragma unroll
            for (int ks = 0; ks < KR; ++ks) {
                const int ch = 4 * ks + g;
                float v[8];
                piece8(2 * NPAIR + ks, v);
                bf16x8 f;
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    float a = 0.0f, b = 0.0f;
                    if (ch < RCH) {
                        const float2 cs = rtab[(8 * ch + jj) / 2];
                        a = v[jj] * cs.x - v[jj + 1] * cs.y;
                        b = v[jj] * cs.y + v[jj + 1] * cs.x;
                    }
                    f[jj] = f2bf(a);
                    f[jj + 1] = f2bf(b);
                }
                Qr[ks] = f;
            }
        }
        const float tau2 = L.tau * 1.4426950408889634f;   // logits in base 2
        auto slot = [&](int c, int r) { return buf + (r * RS + c + (r >> 4) * SWZ) * 16; };   // c: the part's piece

        // ---- first half of a chunk step: this part's partial logits from the
        // registers, into the exchange slot; the pieces staged for O^T += V^T P^T;
        // the loads of chunk t+2 into the freed registers
        // First half of a chunk step: this part's partial logits from the
        // registers, into the exchange slot; each piece group, once its MFMAs
        // have it, staged for O^T += V^T P^T and its registers refilled with
        // chunk t+2's group at once -- the refill loads trickle out between
        // the MFMAs instead of queueing in one burst.  Every step runs it (a
        // step past the subset's end computes on the stand-in rows and is
        // not consumed): the loads stay unconditional and in order.
        // (REFILL false: the first step, whose refill goes out after its barrier)
        auto produce = [&](auto refill_c, u32x4 (&pre)[2 * NGL], uint32_t (&scl)[2], int t) {
            constexpr bool REFILL = decltype(refill_c)::value;
            int32_t lnext[2];
            locs_of(t + 2, lnext);
            const bool in2 = t + 2 < mine;
            const uint8_t *rc[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int32_t lc = lnext[rb] == kMasked ? stand : lnext[rb];
                rc[rb] = in2 ? loc_addr<PREFILL>(A, Q, lc) : qsafe;
            }
            wave_lds_fence();                            // the previous chunk's transposed reads come first
            auto refill = [&](int k) {                   // stage group k of both record blocks, load its successor
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    if (k < NST) *(u32x4 *)slot(4 * k + g, 16 * rb + c16) = pre[rb * NGL + k];
                    if constexpr (REFILL) pre[rb * NGL + k] = *(const u32x4 *)(rc[rb] + 16 * g + 64 * (GB + k));
                }
            };
            // the two record blocks' chains interleaved; each keeps its pairs in order
            f32x4 a[2], b[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) a[rb] = b[rb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < NPAIR; ++e) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        const u32x4 u = pre[rb * NGL + e];
                        a[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8(u[2 * h], u[2 * h + 1]), Qn[e][h], a[rb], 0,
                                                                        0, 0);
                    }
                refill(e);
            }
            if constexpr (DQ == 1) {
#pragma unroll
                for (int ks = 0; ks < KR; ++ks) {
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        union { u32x4 v; bf16x8 b; } cv;
                        cv.v = pre[rb * NGL + (KP - G1) + ks];
                        b[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Qr[ks], b[rb], 0, 0, 0);
                    }
                    refill((KP - G1) + ks);
                }
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int k = (rb * 64 + lane) * 4;      // [rb][lane][i]: one 16-byte piece a lane
                if constexpr (DQ == 0) {
                    *(f32x4 *)(xs + k) = a[rb];
                } else {
                    *(f32x4 *)(xs + XWF + k) = a[rb];
                    *(f32x4 *)(xs + 2 * XWF + k) = b[rb];
                    if (g == 0) xs[3 * XWF + 16 * rb + c16] = __uint_as_float(scl[rb]);   // the record scales
                }
            }
            if constexpr (DQ == 1 && REFILL) {           // the next scales, once these are written out
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) scl[rb] = *(const uint32_t *)(rc[rb] + 16 * (Sh::CREC - 1));
            }
        };

        // ---- second half: logits from both parts' partials, online softmax,
        // O^T += V^T P^T on this part's dim blocks
        AttnState<DBQ> S;
        state_clear(S);
        auto softmax = [&](int t, bf16x8 &Pn, bf16x8 &Pr) {
            float lg[2][4], sc[2][4];
            const uint32_t vmg = vmask[t] >> (4 * g);     // bit 16rb+i: record 16rb+4g+i usable
            f32x4 x0[2], x1[2], xr[2], xc[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int k = (rb * 64 + lane) * 4;
                x0[rb] = *(const f32x4 *)(xs + k);
                x1[rb] = *(const f32x4 *)(xs + XWF + k);
                xr[rb] = *(const f32x4 *)(xs + 2 * XWF + k);
                xc[rb] = *(const f32x4 *)(xs + 3 * XWF + 16 * rb + 4 * g);   // scales of records 16rb+4g+i
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = (vmg >> (16 * rb + i)) & 1u;
                    sc[rb][i] = xc[rb][i];
                    const float a = x0[rb][i] + x1[rb][i];
                    const float v = tau2 * (sc[rb][i] * a + xr[rb][i]);
                    lg[rb][i] = ok ? v : -INFINITY;
                }
            float cmax = -INFINITY;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, lg[rb][i]);
            cmax = head_max(cmax);
            const float m_new = lazy_max(S.m, cmax);
            float p[2][4];
            float alpha = 1.0f;
            if (m_new == -INFINITY) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) p[rb][i] = 0.0f;
            } else {
                alpha = __builtin_amdgcn_exp2f(S.m - m_new);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) p[rb][i] = __builtin_amdgcn_exp2f(lg[rb][i] - m_new);
            }
            float ps = 0.0f;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) ps = ps + p[rb][i];
            ps = head_sum(ps);
            S.l = S.l * alpha + ps;
            S.m = m_new;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                for (int i = 0; i < DBQ; ++i) S.O[i] = S.O[i] * alpha;
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int rb = jj >> 2, i = jj & 3;
                Pn[jj] = f2bf(p[rb][i] * sc[rb][i]);
                Pr[jj] = f2bf(p[rb][i]);
            }
        };
        auto pv = [&](const bf16x8 &Pn, const bf16x8 &Pr) {
            const int trow = c16 >> 1, thalf = c16 & 1;
            const int trec = (trow < 4 ? 0 : 16) + 4 * g + (trow & 3);
            const int r16 = c16 >> 2, q16 = c16 & 3;
#pragma unroll
            for (int ii = 0; ii < DBQ; ++ii) {
                if (ii % kLo8Group == 0) __builtin_amdgcn_sched_barrier(0);   // bound the operands in flight
                const int db = DBQ * DQ + ii;
                if (db < NCH) {
                    const i32x2 v =
                        __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_p)(slot(db - 4 * GB, trec) + 8 * thalf));
                    S.O[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt8((uint32_t)v[0], (uint32_t)v[1]), Pn, S.O[ii], 0,
                                                                      0, 0);
                } else if (db < NDB) {
                    const int ch = NCH + 2 * (db - NCH) + (q16 >> 1) - 4 * GB;
                    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(slot(ch, 4 * g + r16) + 8 * (q16 & 1)));
                    i16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(slot(ch, 16 + 4 * g + r16) + 8 * (q16 & 1)));
                    union { i16x4 s[2]; bf16x8 b; } cv;
                    cv.s[0] = lo;
                    cv.s[1] = hi;
                    S.O[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Pr, S.O[ii], 0, 0, 0);
                }
            }
        };

        // every wave takes part in every barrier: the second group enters the
        // step sequence one barrier later, and the first leaves one later
        auto step = [&](u32x4 (&pre)[2 * NGL], uint32_t (&scl)[2], int t) {
            produce(std::true_type(), pre, scl, t);
            __syncthreads();                             // both parts' partials of chunk t visible
            if (t < mine) {
                bf16x8 Pn, Pr;
                softmax(t, Pn, Pr);
                pv(Pn, Pr);
            }
            __syncthreads();                             // the exchange slot is free again
        };
        // The first step refills after its exchange barrier (the shared
        // locators of chunk 2 are visible from there on); the others run in
        // pairs, an odd count ending with a step no subset consumes.
        if (grp == 1) __syncthreads();
        {
            produce(std::false_type(), R0, C0, 0);
            __syncthreads();                             // partials (and the locators) visible
            if (0 < mine) {
                bf16x8 Pn, Pr;
                softmax(0, Pn, Pr);
                pv(Pn, Pr);
            }
            int32_t l2[2];
            locs_of(2, l2);
            issue(R0, C0, 2, l2);
            __syncthreads();                             // the exchange slot is free again
        }
#pragma unroll 1
        for (int t = 1; t < cpw; t += 2) {
            step(R1, C1, t);
            step(R0, C0, t + 1);
        }
        if (grp == 0) __syncthreads();

        // ---- fold the four subset states left to right through LDS (the
        // operations of k_attend's sequential fold); wave (s, q) emits dim
        // blocks DBQ*q + s, +4, ... of its part
        __syncthreads();
        float2 *ml = (float2 *)smem;                             // [subset][64]
        f32x4 *ob = (f32x4 *)(smem + kSubsets * 64 * 8);         // [subset][NDB][64]
        if constexpr (DQ == 0) ml[sw * 64 + lane] = make_float2(S.m, S.l);
#pragma unroll
        for (int i = 0; i < DBQ; ++i) ob[(sw * NDB + DBQ * DQ + i) * 64 + lane] = S.O[i];
        __syncthreads();
        float m = ml[lane].x, l = ml[lane].y;
        float fw[kSubsets][2];
#pragma unroll
        for (int s = 1; s < kSubsets; ++s) {
            const float2 b = ml[s * 64 + lane];
            float mm, ll, fa, fb;
            fold_scales(m, l, b.x, b.y, mm, ll, fa, fb);
            fw[s][0] = fa;
            fw[s][1] = fb;
            m = mm;
            l = ll;
        }
        if (!head_ok) return;
        const float z = A.sinks[head] * 1.4426950408889634f;
        const float M = fmaxf(m, z);
        const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
        const float den = l * f + ((z == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - M));
        const float cf = den > 0.0f ? f / den : 0.0f;
        const int64_t obase = ((int64_t)Q.qrow * L.H + head) * D;
#pragma unroll
        for (int b = DBQ * DQ + sw; b < DBQ * DQ + DBQ; b += kSubsets) {
            f32x4 o = ob[b * 64 + lane];
#pragma unroll
            for (int s = 1; s < kSubsets; ++s) o = fold_o(o, fw[s][0], ob[(s * NDB + b) * 64 + lane], fw[s][1]);
            const int dd = b * 16 + 4 * g;
            if constexpr (!F32A) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                const bf16x4 v = {f2bf(o[0] * cf), f2bf(o[1] * cf), f2bf(o[2] * cf), f2bf(o[3] * cf)};
                *(bf16x4 *)((uint16_t *)A.out + obase + dd) = v;
            } else {
                *(float4 *)((float *)A.out + obase + dd) = make_float4(o[0] * cf, o[1] * cf, o[2] * cf, o[3] * cf);
            }
        }
    };
    if ((wave & 1) == 0) part_body(std::integral_constant<int, 0>());
    else part_body(std::integral_constant<int, 1>());
}

// ---------------------------------------------------------------- the HI kernel, shared records (d = 512)
// For a saturated GPU (prefill chunks, large batches): one workgroup of eight
// waves per (query, four 16-head groups), wave (h, q) reducing head group h
// over dim part q with the subsets one after another, exactly as k_attend's
// two waves do -- the same partial dot products in the same order, the same
// exchange, online softmax and left-to-right fold -- so the kernels agree bit
// for bit.  What changes is where the records come from: a chunk is loaded
// once per workgroup by all its threads, its E4M3 codes converted to bf16 once
// (exactly) and staged in LDS, and the four head groups' waves read it there:
// the key operands of S^T = K Q^T as 16-byte reads, the transposed operands of
// O^T += V^T P^T with ds_read_b64_tr_b16 for every dim.  Two chunk buffers:
// while one chunk is computed on, the next is converted into the other buffer
// and the one after that is loaded.  (Measured on the 8K prefill chunk: 3.69
// ms against 4.42 ms for k_attend; with two head groups per workgroup, two
// workgroups sharing a compute unit, 3.84 ms.)
template <int D, int DR>
struct HqShape {
    using Sh = AttnShape<D, DR>;
    static constexpr int NHQ = 4;                              // head groups per workgroup
    static constexpr int NT = 64 * kParts * NHQ;               // threads
    static constexpr int TPR = NT / kChunk;                    // staging threads per record
    static constexpr int NLP = 32 / TPR + 1;                   // pieces each loads: 32 / TPR, then one of 32..CREC-1
    static constexpr int BPR = 2 * Sh::NCH + Sh::RCH;          // bf16 pieces of a staged record
    // A record's row holds its BPR pieces; piece c of record r sits at column
    // c ^ swz(r), swz(r) = 2 (r mod 8) + (r / 8 mod 2).  With 64 LDS banks (16
    // pieces) the 16 records a key-operand read serves per clock then cover
    // all banks, and so do the 8 records x 2 pieces of a transposed read.
    static constexpr int RSH = BPR;
    static constexpr int BUFH = kChunk * RSH * 16;             // one chunk buffer
    static constexpr int XOFF = 2 * BUFH + 2 * kChunk * 4;     // the buffers, then their record scales
    static constexpr int LOFF = XOFF + NHQ * (kParts + 1) * Sh::XW * 4;
    static __host__ __device__ int64_t lds_bytes(int64_t list_max) {
        return LOFF + (list_max * 4 + 15) / 16 * 16 + ((list_max + kChunk - 1) / kChunk * 4 + 15) / 16 * 16;
    }
    static_assert(Sh::CREC > 32 && Sh::CREC - 32 <= TPR, "the last load of each thread covers pieces 32..CREC-1");
    static_assert(BPR % 16 == 0, "the column swizzle stays inside the row");
    static_assert(BUFH % 16 == 0 && XOFF % 16 == 0 && LOFF % 16 == 0, "alignment");
};

template <int D, int DR, bool CSA, bool PREFILL, bool F32A>
__global__ __launch_bounds__((HqShape<D, DR>::NT)) __attribute__((amdgpu_waves_per_eu(2))) void k_attend_hq(AttnArgs A) {
    using Sh = AttnShape<D, DR>;
    using HS = HqShape<D, DR>;
    constexpr int NCH = Sh::NCH, RCH = Sh::RCH, CREC = Sh::CREC, KP = Sh::KP, KR = Sh::KR, QPP = Sh::QPP;
    constexpr int NDB = Sh::NDB, DBQ = Sh::DBQ, XW = Sh::XW, DN = Sh::DN, NHQ = HS::NHQ;
    constexpr int RSH = HS::RSH, BUFH = HS::BUFH, TPR = HS::TPR, NLP = HS::NLP;
    constexpr int NT = HS::NT;

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ float2 rope_tab[DR / 2];
    __shared__ int32_t safe_sh;

    const Lay &L = A.L;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar registers)
    const int dq = wave & 1, hq = wave >> 1;                      // dim part, head group in the workgroup

    // ---- which query and head groups (a query's workgroups are dealt onto
    // one XCD: workgroup ids go round-robin over the 8 XCDs)
    const int nhq = (A.nhg + NHQ - 1) / NHQ;
    const int lin = blockIdx.x, x8 = lin & 7, u8 = lin >> 3;
    const int qi = (u8 / nhq) * 8 + x8;
    const int hg = (u8 % nhq) * NHQ + hq;
    if (qi >= A.nq) return;
    const QueryInfo Q = query_info<CSA, PREFILL>(A, qi);
    if (!Q.ok) return;
    const int head = hg * 16 + c16;
    const bool head_ok = hg < A.nhg && head < L.H;

    // LDS: two chunk buffers (bf16 records), their scales, one partial-logit
    // exchange per head group, the record locators and valid masks
    float *scl = (float *)(smem + 2 * BUFH);                     // [buffer][record]
    float *xch = (float *)(smem + HS::XOFF) + hq * (kParts + 1) * XW;
    int32_t *locs = (int32_t *)(smem + HS::LOFF);
    const int loc_bytes = ((int)Q.n_list * 4 + 15) / 16 * 16;
    uint32_t *vmask = (uint32_t *)(smem + HS::LOFF + loc_bytes);   // [chunk]: bit r = record r usable

    // ---- resolve every record of the list once; any valid record stands in
    // for masked ones (its bytes are loaded, its weight is 0)
    if (tid == 0) safe_sh = -1;
    __syncthreads();
    int32_t last_ok = -1;
    for (int64_t p0 = (int64_t)wave * 64; p0 < Q.n_list; p0 += NT) {   // wave-uniform: 64 consecutive records
        const int64_t p = p0 + lane;
        const int32_t lc = p < Q.n_list ? record_loc<CSA, PREFILL>(A, Q, p) : kMasked;
        if (p < Q.n_list) locs[p] = lc;
        if (lc != kMasked) last_ok = (int32_t)p;
        const uint64_t vb = __builtin_amdgcn_ballot_w64(lc != kMasked);
        if (lane == 0) {
            vmask[p0 / kChunk] = (uint32_t)vb;
            if (p0 + kChunk < Q.n_list) vmask[p0 / kChunk + 1] = (uint32_t)(vb >> 32);
        }
    }
    if (last_ok >= 0) atomicMax(&safe_sh, last_ok);
    if (tid < DR / 2) {
        float c, sn;
        rope_cs_theta(theta_lane(L, DR / 2), Q.t, c, sn);   // (lane l: theta_l from scalar reads)
        rope_tab[tid] = make_float2(c, sn);
    }
    __syncthreads();
    const int32_t safe = safe_sh >= 0 ? locs[safe_sh] : kMasked;
    const int n_list = (int)Q.n_list;                // (lists are far below 2^31 records)
    const int nchunks = safe == kMasked ? 0 : (n_list + kChunk - 1) / kChunk;

    // ---- chunk staging by all threads: thread t loads pieces j + TPR k
    // (k < 32 / TPR) and 32 + min(j, CREC - 33) of record t / TPR (j = t mod
    // TPR; the last load of threads j > CREC - 33 repeats the scale piece and
    // is not stored), converts the code pieces to bf16 and writes them to the
    // chunk buffer: bf16 piece 2c + h of a record holds dims 16c + 8h .. +8 of
    // code piece c, bf16 piece 2 NCH + k its RoPE piece k
    const int sr = tid / TPR, sj = tid % TPR;
    auto piece_of = [&](int k) { return k < NLP - 1 ? sj + TPR * k : 32 + (sj < CREC - 33 ? sj : CREC - 33); };
    auto hslot = [&](int b, int c, int r) {
        return smem + b * BUFH + (r * RSH + (c ^ (2 * (r & 7) + ((r >> 3) & 1)))) * 16;
    };
    auto issue = [&](u32x4 (&pre)[NLP], int ck) {
        const int p = ck * kChunk + sr;
        int32_t lc = locs[p < n_list ? p : n_list - 1];   // (no branch around the LDS read)
        if (p >= n_list || lc == kMasked) lc = safe;
        const uint8_t *rec = loc_addr<PREFILL>(A, Q, lc);
#pragma unroll
        for (int k = 0; k < NLP; ++k) pre[k] = *(const u32x4 *)(rec + 16 * piece_of(k));
    };
    auto stage = [&](const u32x4 (&pre)[NLP], int b) {
#pragma unroll
        for (int k = 0; k < NLP; ++k) {
            const int pc = piece_of(k);
            const u32x4 u = pre[k];
            if (pc < NCH) {
                union { bf16x8 b; u32x4 v; } lo, hi;
                lo.b = cvt8(u[0], u[1]);
                hi.b = cvt8(u[2], u[3]);
                // threads of odd record / upper half store their odd piece
                // first: each store of 16 lanes then spreads over the banks
                const bool sw8 = ((sj >= TPR / 2) ^ (sr & 1)) != 0;
                *(u32x4 *)hslot(b, 2 * pc + (sw8 ? 1 : 0), sr) = sw8 ? hi.v : lo.v;
                *(u32x4 *)hslot(b, 2 * pc + (sw8 ? 0 : 1), sr) = sw8 ? lo.v : hi.v;
            } else if (pc < NCH + RCH) {
                *(u32x4 *)hslot(b, NCH + pc, sr) = u;
            } else if (k == NLP - 1 && sj == CREC - 33) {
                scl[b * kChunk + sr] = __uint_as_float(u[0]);
            }
        }
    };

    static_assert(kParts == 2, "the part dispatch below covers two parts");
    auto part_body = [&](auto dqc) {
        constexpr int DQ = decltype(dqc)::value;
        // ---- query fragments of this dim part (B operand of S^T = K Q^T), lane
        // (head c16, group g): code pair kp reads piece 4kp+g, dims 16(4kp+g) +
        // [0,8) and [8,16); RoPE step ks reads RoPE piece 4ks+g, rotated at t.
        bf16x8 Qn[QPP][2], Qr[KR];
        {
            const int64_t qbase = ((int64_t)Q.qrow * L.H + (head_ok ? head : 0)) * D;
            auto q8 = [&](int dd, float (&v)[8]) {
                if constexpr (!F32A) {
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
            for (int e = 0; e < QPP; ++e) {
                const int kp = QPP * DQ + e, ch = 4 * kp + g;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    if (head_ok && kp < KP && ch < NCH) q8(16 * ch + 8 * h, v);
                    bf16x8 f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) f[j] = f2bf(v[j]);
                    Qn[e][h] = f;
                }
            }
#pragma unroll
            for (int ks = 0; ks < KR; ++ks) {
                const int ch = 4 * ks + g;
                float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (head_ok && DQ == kParts - 1 && ch < RCH) q8(DN + 8 * ch, v);
                bf16x8 f;
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    float a = 0.0f, b = 0.0f;
                    if (ch < RCH) {
                        const float2 cs = rope_tab[(8 * ch + j) / 2];
                        a = v[j] * cs.x - v[j + 1] * cs.y;
                        b = v[j] * cs.y + v[j + 1] * cs.x;
                    }
                    f[j] = f2bf(a);
                    f[j + 1] = f2bf(b);
                }
                Qr[ks] = f;
            }
        }
        const float tau2 = L.tau * 1.4426950408889634f;   // logits in base 2

        // ---- this part's partial logits of the chunk in buffer b (k_attend's
        // chains: code pairs in order, then the RoPE steps); rows = records
        // 16rb + 4g + i, lane column = head c16
        auto partial = [&](float (&an)[2][4], float (&ar)[2][4], int b) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, bb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int e = 0; e < QPP; ++e) {
                    const int kp = QPP * DQ + e, ch = 4 * kp + g;
                    if (kp < KP) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            union { u32x4 v; bf16x8 b; } cv;
                            cv.v = (u32x4){0, 0, 0, 0};
                            if (NCH % 4 == 0 || ch < NCH) cv.v = *(const u32x4 *)hslot(b, 2 * ch + h, 16 * rb + c16);
                            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Qn[e][h], a, 0, 0, 0);
                        }
                    }
                }
                if (DQ == kParts - 1) {
#pragma unroll
                    for (int ks = 0; ks < KR; ++ks) {
                        const int ch = 4 * ks + g;
                        union { u32x4 v; bf16x8 b; } cv;
                        cv.v = (u32x4){0, 0, 0, 0};
                        if (RCH % 4 == 0 || ch < RCH) cv.v = *(const u32x4 *)hslot(b, 2 * NCH + ch, 16 * rb + c16);
                        bb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, Qr[ks], bb, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    an[rb][i] = a[i];
                    ar[rb][i] = bb[i];
                }
                __builtin_amdgcn_sched_barrier(0);   // one record block's operands at a time
            }
        };

        // ---- the rest of a chunk step, after the partials are exchanged: logits,
        // online softmax, O^T += V^T P^T on this part's dim blocks
        auto finish = [&](auto &S, int ck, int b) {
            constexpr int NO = sizeof(S.O) / sizeof(S.O[0]);
            float lg[2][4], sc[2][4];
            const uint32_t vmg = vmask[ck] >> (4 * g);   // bit 16rb+i: record 16rb+4g+i usable
            f32x4 xa[kParts][2], xr[2], xc[2];            // one 16-byte read per array and record block
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int k = (rb * 64 + lane) * 4;      // [rb][lane][i]
#pragma unroll
                for (int q = 0; q < kParts; ++q) xa[q][rb] = *(const f32x4 *)(xch + q * XW + k);
                xr[rb] = *(const f32x4 *)(xch + kParts * XW + k);
                xc[rb] = *(const f32x4 *)(scl + b * kChunk + 16 * rb + 4 * g);   // scales of records 16rb+4g+i
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = (vmg >> (16 * rb + i)) & 1u;
                    sc[rb][i] = xc[rb][i];
                    float a = xa[0][rb][i];
#pragma unroll
                    for (int q = 1; q < kParts; ++q) a = a + xa[q][rb][i];
                    lg[rb][i] = ok ? tau2 * (sc[rb][i] * a + xr[rb][i]) : -INFINITY;
                }
            float cmax = -INFINITY;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, lg[rb][i]);
            cmax = head_max(cmax);
            const float m_new = lazy_max(S.m, cmax);
            float p[2][4];
            float alpha = 1.0f;
            if (m_new == -INFINITY) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) p[rb][i] = 0.0f;
            } else {
                alpha = __builtin_amdgcn_exp2f(S.m - m_new);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) p[rb][i] = __builtin_amdgcn_exp2f(lg[rb][i] - m_new);
            }
            float ps = 0.0f;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) ps = ps + p[rb][i];
            ps = head_sum(ps);
            S.l = S.l * alpha + ps;
            S.m = m_new;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {   // alpha == 1 leaves O as it is
#pragma unroll
                for (int i = 0; i < NO; ++i) S.O[i] = S.O[i] * alpha;
            }
            // k-slot j of lane group g is record 4g+j (j < 4) or 16+4g+(j-4)
            bf16x8 Pn, Pr;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int rb = j >> 2, i = j & 3;
                Pn[j] = f2bf(p[rb][i] * sc[rb][i]);
                Pr[j] = f2bf(p[rb][i]);
            }
            // every dim from the bf16 rows: ds_read_b64_tr_b16 -- lanes 4r..4r+3
            // address row r (record 4g+r, resp. 16+4g+r), 4 dims each; lane c16
            // receives dim 16db + c16 of the 4 records
            const int r16 = c16 >> 2, q16 = c16 & 3;
#pragma unroll
            for (int ii = 0; ii < NO; ++ii) {
                if (ii % 8 == 0) __builtin_amdgcn_sched_barrier(0);   // bound the operands in flight
                const int db = DBQ * DQ + ii;
                if (db < NDB) {
                    const int ch = 2 * db + (q16 >> 1);
                    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(hslot(b, ch, 4 * g + r16) + 8 * (q16 & 1)));
                    i16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(hslot(b, ch, 16 + 4 * g + r16) + 8 * (q16 & 1)));
                    union { i16x4 s[2]; bf16x8 b; } cv;
                    cv.s[0] = lo;
                    cv.s[1] = hi;
                    S.O[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv.b, db < NCH ? Pn : Pr, S.O[ii], 0, 0, 0);
                }
            }
        };

        // ---- output rows d = 16db + 4g + i of head `head`, with the sink:
        // out = O * f / (l * f + 2^(z - M)),  f = 2^(m - M),  M = max(m, z)
        const int64_t obase = ((int64_t)Q.qrow * L.H + head) * D;
        // (the normalisation is computed once: with the output stores in
        // between, the compiler re-read the sink for every block, each read
        // waiting for the stores before it)
        auto out_scale = [&](float m, float l) {
            const float z = A.sinks[head] * 1.4426950408889634f;
            const float M = fmaxf(m, z);
            const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
            const float den = l * f + ((z == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - M));
            return den > 0.0f ? f / den : 0.0f;
        };
        auto emit = [&](float cf, int db, const f32x4 &o) {
            const int dd = db * 16 + 4 * g;
            if constexpr (!F32A) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                const bf16x4 v = {f2bf(o[0] * cf), f2bf(o[1] * cf), f2bf(o[2] * cf), f2bf(o[3] * cf)};
                *(bf16x4 *)((uint16_t *)A.out + obase + dd) = v;
            } else {
                *(float4 *)((float *)A.out + obase + dd) = make_float4(o[0] * cf, o[1] * cf, o[2] * cf, o[3] * cf);
            }
        };

        // ---- the chunks in processing order: subset 0 (chunks 0, 4, 8, ...),
        // then subsets 1, 2, 3, each subset's state folded into the
        // accumulated one after its last chunk (empty subsets too, as k_attend
        // folds them).  The accumulated state is not touched inside a
        // subset's loop, so it is the one the compiler keeps out of registers
        // there.
        auto next_of = [&](int ck) {
            if (ck + kSubsets < nchunks) return ck + kSubsets;
            for (int s = ck % kSubsets + 1; s < kSubsets; ++s)
                if (s < nchunks) return s;
            return -1;
        };
        AttnState<DBQ> acc, cur;
        state_clear(acc);
        u32x4 pre[NLP];
        int cn = nchunks > 0 ? 0 : -1;                   // the next chunk to compute
        int cn1 = cn >= 0 ? next_of(cn) : -1;            // and the one after it
        if (cn >= 0) {
            issue(pre, cn);
            stage(pre, 0);
        }
        if (cn1 >= 0) issue(pre, cn1);
        __syncthreads();                                 // the first chunk staged
        int b = 0;
#pragma unroll 1
        for (int s = 0; s < kSubsets; ++s) {
            state_clear(cur);
#pragma unroll 1
            for (int ck = s; ck < nchunks; ck += kSubsets) {
                const int cn2 = cn1 >= 0 ? next_of(cn1) : -1;
                float an[2][4], ar[2][4];
                partial(an, ar, b);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const int k = (rb * 64 + lane) * 4;  // [rb][lane][i]: one 16-byte write a lane
                    *(f32x4 *)(xch + DQ * XW + k) = (f32x4){an[rb][0], an[rb][1], an[rb][2], an[rb][3]};
                    if (DQ == kParts - 1)
                        *(f32x4 *)(xch + kParts * XW + k) = (f32x4){ar[rb][0], ar[rb][1], ar[rb][2], ar[rb][3]};
                }
                if (cn1 >= 0) stage(pre, b ^ 1);         // the next chunk into the other buffer
                if (cn2 >= 0) issue(pre, cn2);           // and the one after on its way
                __syncthreads();                         // partials and the next chunk visible
                finish(cur, ck, b);
                __syncthreads();                         // buffer b and the exchange are free again
                b ^= 1;
                cn1 = cn2;
            }
            if (s == 0) {
                acc = cur;
            } else {
                float m, l, fa, fb;
                fold_scales(acc.m, acc.l, cur.m, cur.l, m, l, fa, fb);
#pragma unroll
                for (int i = 0; i < DBQ; ++i) acc.O[i] = fold_o(acc.O[i], fa, cur.O[i], fb);
                acc.m = m;
                acc.l = l;
            }
        }
        if (head_ok) {
            const float cf = out_scale(acc.m, acc.l);
#pragma unroll
            for (int i = 0; i < DBQ; ++i)
                if (DBQ * DQ + i < NDB) emit(cf, DBQ * DQ + i, acc.O[i]);
        }
    };
    if (dq == 0) part_body(std::integral_constant<int, 0>());
    else part_body(std::integral_constant<int, kParts - 1>());
}

// ---------------------------------------------------------------- fp32 records
// Records stored as d fp32 values (the reference-precision storage mode): one
// wave per (query, head), lane l holding dims [l*VPL, l*VPL + VPL).  The
// records are taken one at a time in list order (selected entries ascending,
// then the window); each logit is the wave's fixed-order sum of its fp32
// products, and an online softmax (base 2) folds it in.  Nothing depends on
// the batch or on the decode policy: both policies run this kernel.
template <int D, int DR, bool CSA, bool PREFILL>
__global__ __launch_bounds__(256) void k_attend_f32(AttnArgs A) {
    constexpr int VPL = D / 64;
    constexpr int DN = D - DR;
    const Lay &L = A.L;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)A.nq * L.H) return;
    const int qi = (int)(item / L.H), head = (int)(item % L.H);
    const QueryInfo Q = query_info<CSA, PREFILL>(A, qi);
    if (!Q.ok) return;
    const int d0 = lane * VPL;
    // the query head, rotated at t on its last DR dims (pairs stay in a lane)
    float q[VPL];
    const int64_t qb = ((int64_t)Q.qrow * L.H + head) * D + d0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) q[v] = load_act(A.q, qb + v, L.act);
    if constexpr (VPL >= 2) {
#pragma unroll
        for (int v = 0; v < VPL; v += 2)
            if (d0 + v >= DN) {
                float c, s;
                rope_cs(L, Q.t, (d0 + v - DN) / 2, c, s);
                const float a = q[v], b = q[v + 1];
                q[v] = a * c - b * s;
                q[v + 1] = a * s + b * c;
            }
    } else {
        const float other = __shfl_xor(q[0], 1);
        if (d0 >= DN) {
            float c, s;
            rope_cs(L, Q.t, (d0 - DN) / 2, c, s);
            q[0] = (lane & 1) == 0 ? q[0] * c - other * s : other * s + q[0] * c;
        }
    }
    const float tau2 = L.tau * 1.4426950408889634f;
    float m = -INFINITY, l = 0.0f, o[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) o[v] = 0.0f;
    for (int64_t p = 0; p < Q.n_list; ++p) {
        const int32_t lc = record_loc<CSA, PREFILL>(A, Q, p);
        if (lc == kMasked) continue;                       // (wave-uniform)
        const float *rec = (const float *)loc_addr<PREFILL>(A, Q, lc) + d0;
        float x[VPL], dot = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            x[v] = rec[v];
            dot = __builtin_fmaf(q[v], x[v], dot);
        }
        // wave sum, fixed tree: row-local shifts, then across rows
#pragma unroll
        for (int o2 = 1; o2 < 64; o2 <<= 1) dot = dot + __shfl_xor(dot, o2);
        const float lg = tau2 * dot;
        const float mn = fmaxf(m, lg);
        const float alpha = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        const float pe = __builtin_amdgcn_exp2f(lg - mn);
        l = l * alpha + pe;
#pragma unroll
        for (int v = 0; v < VPL; ++v) o[v] = o[v] * alpha + pe * x[v];
        m = mn;
    }
    const float z = A.sinks[head] * 1.4426950408889634f;
    const float M = fmaxf(m, z);
    const float f = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    const float den = l * f + (z == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(z - M));
    const float cf = den > 0.0f ? f / den : 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const float r = o[v] * cf;
        if (L.act == DSV4_DT_BF16) ((uint16_t *)A.out)[qb + v] = bf16_bits(r);
        else ((float *)A.out)[qb + v] = r;
    }
}

template <int D, int DR>
static hipError_t launch_f32_t(const AttnArgs &A, bool csa, bool prefill, hipStream_t s) {
    const dim3 g((unsigned)(((int64_t)A.nq * A.L.H + 3) / 4));
    if (csa) {
        if (prefill) hipLaunchKernelGGL((k_attend_f32<D, DR, true, true>), g, dim3(256), 0, s, A);
        else hipLaunchKernelGGL((k_attend_f32<D, DR, true, false>), g, dim3(256), 0, s, A);
    } else {
        if (prefill) hipLaunchKernelGGL((k_attend_f32<D, DR, false, true>), g, dim3(256), 0, s, A);
        else hipLaunchKernelGGL((k_attend_f32<D, DR, false, false>), g, dim3(256), 0, s, A);
    }
    return hipGetLastError();
}

hipError_t launch_attend_f32(const AttnArgs &A, bool csa, bool prefill, hipStream_t s) {
    if (A.L.d == 512) return launch_f32_t<512, 64>(A, csa, prefill, s);
    return launch_f32_t<64, 16>(A, csa, prefill, s);
}

// ---------------------------------------------------------------- launchers
int64_t attend_list_max(const Lay &L, const dsv4_cache &C, bool csa) {
    return (csa ? (int64_t)L.topk : (int64_t)C.max_blocks * L.epb) + L.W;
}

template <int D, int DR, int NSW>
int64_t attend_lds_bytes(int64_t list_max) {
    using Sh = AttnShape<D, DR>;
    const int64_t stream = (list_max * 4 + 15) / 16 * 16 + ((list_max + kChunk - 1) / kChunk * 4 + 15) / 16 * 16 +
                           (int64_t)NSW * Sh::BUF + (int64_t)NSW * (kParts + 1) * Sh::XW * 4;
    constexpr int NWV = kParts * NSW;
    const int64_t fold = NSW == 1 ? 0 : NWV * 64 * 8 + (int64_t)NWV * Sh::DBQ * 64 * 16;
    return stream > fold ? stream : fold;
}

template <int D, int DR>
int64_t attend_lo_lds_bytes(int64_t list_max) {
    const int64_t nch = (list_max + kChunk - 1) / kChunk, cpw = (nch + kSubsets - 1) / kSubsets;
    const int64_t stream = kSubsets * (int64_t)LoShape<D, DR>::wave_bytes((int)cpw) + LoShape<D, DR>::QBYTES;
    return stream > LoShape<D, DR>::FOLD ? stream : LoShape<D, DR>::FOLD;
}

int64_t attend_lds_max(const Lay &L, int64_t list_max) {
    const int64_t lo = L.d == 512 ? attend_lo_lds_bytes<512, 64>(list_max) : attend_lo_lds_bytes<64, 16>(list_max);
    const int64_t hi = L.d == 512 ? HqShape<512, 64>::lds_bytes(list_max) : attend_lds_bytes<64, 16, 1>(list_max);
    return lo > hi ? lo : hi;
}

// Raise a kernel's dynamic-LDS limit to at least `bytes`.  The limit only
// grows, under one lock shared by all kernels, so callers on several threads
// never lower it beneath a launch that needs more.  `lim` is the kernel's own
// record (a static of its launcher's template instance).
static std::mutex g_lds_mu;
static hipError_t raise_lds_limit(const void *fn, int64_t bytes, int64_t &lim) {
    std::lock_guard<std::mutex> lk(g_lds_mu);
    if (lim >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    lim = bytes;
    return hipSuccess;
}

template <int D, int DR, int NSW, bool CSA, bool PREFILL>
static hipError_t launch_gr(const AttnArgs &A, hipStream_t s) {
    static int64_t lim = 0;
    const int64_t lds = attend_lds_bytes<D, DR, NSW>(attend_list_max(A.L, A.C, CSA));
    hipError_t e = raise_lds_limit((const void *)k_attend<D, DR, NSW, CSA, PREFILL>, lds, lim);
    if (e != hipSuccess) return e;
    const int groups = (A.nq + 7) / 8;
    hipLaunchKernelGGL((k_attend<D, DR, NSW, CSA, PREFILL>), dim3(groups * 8 * A.nhg), dim3(64 * kParts * NSW),
                       (size_t)lds, s, A);
    return hipGetLastError();
}

template <int D, int DR, bool CSA, bool PREFILL>
static hipError_t launch_lo(const AttnArgs &A, hipStream_t s) {
    static int64_t lim = 0;
    const int64_t lds = attend_lo_lds_bytes<D, DR>(attend_list_max(A.L, A.C, CSA));
    hipError_t e = raise_lds_limit((const void *)k_attend_lo<D, DR, CSA, PREFILL>, lds, lim);
    if (e != hipSuccess) return e;
    const int groups = (A.nq + 7) / 8;
    hipLaunchKernelGGL((k_attend_lo<D, DR, CSA, PREFILL>), dim3(groups * 8 * A.nhg), dim3(64 * kSubsets), (size_t)lds,
                       s, A);
    return hipGetLastError();
}

template <int D, int DR, bool CSA, bool PREFILL, bool F32A>
static hipError_t launch_hq(const AttnArgs &A, hipStream_t s) {
    static int64_t lim = 0;
    const int64_t lds = HqShape<D, DR>::lds_bytes(attend_list_max(A.L, A.C, CSA));
    hipError_t e = raise_lds_limit((const void *)k_attend_hq<D, DR, CSA, PREFILL, F32A>, lds, lim);
    if (e != hipSuccess) return e;
    const int groups = (A.nq + 7) / 8;
    const int nhq = (A.nhg + HqShape<D, DR>::NHQ - 1) / HqShape<D, DR>::NHQ;
    hipLaunchKernelGGL((k_attend_hq<D, DR, CSA, PREFILL, F32A>), dim3(groups * 8 * nhq), dim3(HqShape<D, DR>::NT),
                       (size_t)lds, s, A);
    return hipGetLastError();
}

template <int D, int DR, bool CSA, bool PREFILL, bool F32A>
static hipError_t launch_lo8(const AttnArgs &A, hipStream_t s) {
    static int64_t lim = 0;
    constexpr int64_t lds = Lo8Shape<D, DR>::LDS;
    hipError_t e = raise_lds_limit((const void *)k_attend_lo8<D, DR, CSA, PREFILL, F32A>, lds, lim);
    if (e != hipSuccess) return e;
    const int groups = (A.nq + 7) / 8;
    hipLaunchKernelGGL((k_attend_lo8<D, DR, CSA, PREFILL, F32A>), dim3(groups * 8 * A.nhg),
                       dim3(64 * kSubsets * kParts), (size_t)lds, s, A);
    return hipGetLastError();
}

// LO: the eight-wave kernel where the record list fits its locator batch (the
// V4 shape), else the four-wave one.
template <int D, int DR, bool CSA, bool PREFILL>
static hipError_t launch_t(const AttnArgs &A, bool hi, hipStream_t s) {
    if (hi) {
        if constexpr (D == 512)
            return A.L.act == DSV4_DT_BF16 ? launch_hq<D, DR, CSA, PREFILL, false>(A, s)
                                           : launch_hq<D, DR, CSA, PREFILL, true>(A, s);
        return launch_gr<D, DR, 1, CSA, PREFILL>(A, s);
    }
    if constexpr (D == 512)
        if (attend_list_max(A.L, A.C, CSA) <= Lo8Shape<D, DR>::MAX_LIST)
            return A.L.act == DSV4_DT_BF16 ? launch_lo8<D, DR, CSA, PREFILL, false>(A, s)
                                           : launch_lo8<D, DR, CSA, PREFILL, true>(A, s);
    return launch_lo<D, DR, CSA, PREFILL>(A, s);
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
