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
// wave streams 256 keys straight into MFMA B-operand registers (no LDS), four
// waves per workgroup, many workgroups per request.  Top-k is an exact
// selection spread over 4096-score segments (histogram, boundary bin, split,
// final merge), so one query's selection runs on many compute units.
#include <string.h>

#include "launch.h"

namespace dsv4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- query quantisation
// One (query, head) row held by a wave, lane l holding values 2l and 2l+1
// (zero past dI), into a 128-byte slot: E4M3 codes (zero-padded to 128 bytes)
// and wq = w * scale, or (MXFP4) 64 bytes of E2M1 codes (zero past dI), the
// word of E8M0 block scales at byte 64, and wq = w.  Same decision rule as the
// stored index keys.  Returns wq (every lane); the slot may be global or LDS.
// MX: the rows are MXFP4 (else E4M3).
template <bool MX>
__device__ __forceinline__ float quant_q_row(const Lay &L, float x0, float x1, float wrow, uint8_t *slot) {
    const int lane = threadIdx.x & 63;
    const int dI = L.dI;
    if constexpr (MX) {
        uint32_t scales;
        const uint32_t byte = mx4_row(x0, x1, 2 * lane < dI, 2 * lane + 1 < dI, &scales);
        slot[lane] = (uint8_t)byte;
        if (lane == 0) *(uint32_t *)(slot + 64) = scales;
        return wrow;
    }
    const float am = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const bool nz = am >= 1e-30f;                  // (a row of zeros keeps scale 1)
    const float scale = nz ? am / 448.0f : 1.0f;
    const float inv = nz ? 448.0f / am : 1.0f;
    uint32_t c0 = 2 * lane < dI ? fp8_code(x0 * inv) : 0u;
    uint32_t c1 = 2 * lane + 1 < dI ? fp8_code(x1 * inv) : 0u;
    *(uint16_t *)(slot + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
    return wrow * scale;
}

// The lane's two values of row `row` of qI (zero past dI).  Two 4-byte loads
// whatever the activation type (a bf16 pair is one word, read twice; an fp32
// pair two), at addresses clamped into the row for lanes past its end: no
// load sits under a branch, so the compiler's memory-counter waits stay exact.
__device__ __forceinline__ void load_q_pair(const Lay &L, const void *qI, int64_t row, float &x0, float &x1) {
    const int lane = threadIdx.x & 63;
    const int dI = L.dI;
    const bool f32 = L.act != DSV4_DT_BF16;
    const int64_t i = row * dI + (2 * lane < dI ? 2 * lane : 0);
    const uint32_t *p = (const uint32_t *)((const uint8_t *)qI + i * (f32 ? 4 : 2));
    const uint32_t u0 = p[0], u1 = p[f32 ? 1 : 0];
    x0 = __uint_as_float(f32 ? u0 : u0 << 16);
    x1 = __uint_as_float(f32 ? u1 : u0 & 0xffff0000u);
    x0 = 2 * lane < dI ? x0 : 0.0f;
    x1 = 2 * lane + 1 < dI ? x1 : 0.0f;
}

// kQuantRows (query, head) rows a wave, one after another, their loads issued
// first (prefill batches; decode quantises inside the scoring kernel).  With
// one row a wave the waves did too little to cover their start.
constexpr int kQuantRows = 8;
__global__ __launch_bounds__(256) void k_quant_index_q(Lay L, const void *qI, const float *w,
                                                       int rows, uint8_t *q8, float *wq) {
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kQuantRows;
    if (row0 >= rows) return;
    float x0[kQuantRows], x1[kQuantRows], wr[kQuantRows];
#pragma unroll
    for (int i = 0; i < kQuantRows; ++i) {          // (rows past the end re-read the last one, never stored)
        const int64_t row = row0 + i < rows ? row0 + i : rows - 1;
        load_q_pair(L, qI, row, x0[i], x1[i]);
        wr[i] = w ? w[row] : 1.0f;
    }
#pragma unroll
    for (int i = 0; i < kQuantRows; ++i) {
        const int64_t row = row0 + i;
        if (row >= rows) break;                      // (wave-uniform)
        const float v = L.idx_store == DSV4_STORE_MXFP4 ? quant_q_row<true>(L, x0[i], x1[i], wr[i], q8 + row * 128)
                                                        : quant_q_row<false>(L, x0[i], x1[i], wr[i], q8 + row * 128);
        if ((threadIdx.x & 63) == 0) wq[row] = v;
    }
}

// p(l) + p(l^16) + p(l^32) + p(l^48) as (p(l) + p(l^16)) + (p(l^32) + p(l^48)):
// the sum of a key's partial scores over the four lane groups, on the gfx950
// row-swap permutes (VALU, no LDS).
__device__ __forceinline__ float group_sum4(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Four partial sums at once: lane group g of the result holds the sum over
// the four lane groups of v_g, added exactly as group_sum4 adds it, (v(g0) +
// v(g1)) + (v(g2) + v(g3)).  The row-swap permutes exchange two registers at
// a time, so the four take three permutes and three adds (group_sum4 takes
// two and two each).
__device__ __forceinline__ float group_sum4x4(float v0, float v1, float v2, float v3) {
    // rows (2k, 2k+1): v0 -> [v0 r0, v1 r0, v0 r2, v1 r2], v1 -> [v0 r1, v1 r1, v0 r3, v1 r3]
    const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
    const float a = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);   // [v0 r0+r1, v1 r0+r1, v0 r2+r3, v1 r2+r3]
    const float c = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
    // rows 2, 3 of a <-> rows 0, 1 of c: [a r0, a r1, c r0, c r1] and [a r2, a r3, c r2, c r3]
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(c), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// The weighted ReLU term of a head: w * max(0, x) + acc in one rounding (fma).
// max(0, x) is taken on the bits (integer max with 0: a negative float is a
// negative integer), one instruction where a float max would also canonicalise
// its operand.
__device__ __forceinline__ float relu_fma(float x, float w, float acc) {
    return __builtin_fmaf(__int_as_float(max(__float_as_int(x), 0)), w, acc);
}

// Order-preserving key of a score: larger score -> larger key; -0 == +0; NaN
// below everything.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- decode scoring
// grid: (ceil(Nmax / kKeysPerWG), n_queries); block 256 = 4 waves, each
// streaming kKeysPerWave keys as 16-key sub-blocks, loads for the next group of
// four sub-blocks in flight while the current group is on the MFMA.
constexpr int kKeysPerWave = 256;
constexpr int kKeysPerWG = 4 * kKeysPerWave;
static_assert(kKeysPerWave % 64 == 0, "scoring ranges are whole pipeline groups");

// HB: 16-row blocks of index heads (idx_heads <= 16*HB); FULL: idx_dim == 128
// (no padded operand bytes); F4: MXFP4 rows (E2M1 operands, the E8M0 block
// scales applied by the MFMA itself).  All are compile-time so that the loads
// and the MFMAs of a sub-block are straight-line code the compiler can pipeline.
//
// MXFP4: lane group g holds the 32 dims [32g, 32g+32) of a row -- 16 bytes,
// one MX block -- and passes that block's E8M0 byte as its scale operand, so
// the MFMA returns sum_b 2^(xq_b + xk_b) * (codes of block b . codes of block
// b) (exact products, fp32 sums): the dot product of the stored values.  The
// head weights then apply as they are (wq = w).
// The query rows are quantised inside the kernel, with the decision rule of
// k_quant_index_q (so the same codes and weights), into LDS while the first
// keys are already on their way: E4M3 rows by four threads each (32 dims a
// thread, the row maximum over the four), MXFP4 rows by wave w < HB for heads
// [16w, 16w+16) in the separate quantiser's lane layout.
template <int HB, bool FULL, bool F4>
__global__ __launch_bounds__(256) void k_index_score_decode(Lay L, dsv4_cache C, const void *qI,
                                                            const float *w, const int32_t *req,
                                                            const int32_t *pos, float *scores,
                                                            int64_t ld, uint2 *wr, int nwr) {
    const int q = blockIdx.y;
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);    // wave-uniform (scalar)
    // this wave's query rows first (their addresses need nothing else)
    // (MXFP4) wave w < HB holds heads [16w, 16w+16), two values a lane, the
    // layout of the separate quantiser; (E4M3) thread 4h + c holds dims
    // [32c, 32c+32) of head h: eight 16-byte loads (a bf16 quarter row takes
    // four, read twice), every address clamped into the query's rows
    constexpr int NQL = F4 ? 16 : 8;
    float qx0[F4 ? 16 : 1], qx1[F4 ? 16 : 1];
    u32x4 qv[F4 ? 1 : 8];
    if constexpr (F4) {
#pragma unroll
        for (int i = 0; i < NQL; ++i) {
            const int h = (wave < HB ? wave * 16 : 0) + i;
            load_q_pair(L, qI, (int64_t)q * L.HI + (h < L.HI ? h : 0), qx0[i], qx1[i]);
        }
    } else {
        const int h = threadIdx.x >> 2, c = threadIdx.x & 3;
        const bool f32 = L.act != DSV4_DT_BF16;
        const int64_t e0 = ((int64_t)q * L.HI + (h < L.HI ? h : 0)) * L.dI + (32 * c < L.dI ? 32 * c : 0);
        const uint8_t *p = (const uint8_t *)qI + e0 * (f32 ? 4 : 2);
#pragma unroll
        for (int k = 0; k < 8; ++k) qv[k] = *(const u32x4 *)(p + 16 * (f32 ? k : (k & 3)));
    }
    const int r = req[q];
    const int t = pos[q];
    if (r < 0 || r >= C.n_req || t < 0 || (int64_t)t >= (int64_t)C.max_blocks * kBlockTokens) return;
    const int N = (t + 1) >> __builtin_ctz((uint32_t)L.m);   // (m is a power of two)
    const int k0 = (blockIdx.x * 4 + wave) * kKeysPerWave;
    const int dI = L.dI;
    // k-order of the 16x16x128 operands: lane group g holds bytes [16g, 16g+16)
    // and [64+16g, 64+16g+16) of a row, so each 16-byte load instruction of a
    // wave reads 64 contiguous bytes of every key row (same order on both sides).
    const int o0 = 16 * g, o1 = 64 + 16 * g;
    const bool v0 = FULL || o0 < dI, v1 = FULL || o1 < dI;   // chunks holding real bytes
    const i32x4 z4 = {0, 0, 0, 0};
    // the quantised query rows (filled below): codes in LDS, the head weights
    // times the row scales in LDS, and the A operands read back from there
    __shared__ __attribute__((aligned(16))) uint8_t qsl[HB * 16 * 128];
    __shared__ f32x4 wls[HB * 4];                  // [hb][g]: heads hb*16 + 4g + i
    i32x8 A[HB];                                   // rows = index heads (zero past idx_heads)
    uint32_t sa[HB];                               // (MXFP4) the lane's block scale per head block
    const int32_t *btr = C.block_table + (int64_t)r * C.max_blocks;
    const int lane_off = c16 * L.key_bytes;
    const uint8_t *pool = (const uint8_t *)C.index_keys;
    // the block ids of this wave's key range, one per lane, read once up front
    // (a per-sub-block lookup would make every group of key loads wait for
    // the previous one: loads complete in order)
    // key index -> cache block and slot: the stride m and the entries per block
    // 128/m are powers of two, so these are shifts and masks of non-negative
    // values (scalar work per sub-block, shared by the compute unit's waves)
    const uint32_t lgb = (uint32_t)__builtin_ctz((uint32_t)L.epb);   // key k is in block k >> lgb
    const uint32_t slot_mask = (uint32_t)L.epb - 1u;
    const int blk0 = (int)((uint32_t)k0 >> lgb);
    const int btv = blk0 + lane < C.max_blocks ? btr[blk0 + lane] : -1;
    // B operands: 16-key sub-blocks, each inside one 128-token cache block
    // (lane = key c16).  An unmapped block reads block 0 and is masked by its
    // zero scale.
    auto load_sb = [&](int kb, i32x8 &Bk, float &sk, uint32_t &sb) {
        const int kc = kb < N ? kb : k0;                       // stay in mapped memory past the end
        const int blk = (int)((uint32_t)kc >> lgb);
        const int bi = blk - blk0;                             // wave-uniform
        const int bid = bi < 64 ? __builtin_amdgcn_readlane(btv, bi)   // (ranges of 64+ blocks: strides >= 32)
                                : __builtin_amdgcn_readfirstlane(btr[blk]);
        const bool okb = bid >= 0 && bid < C.n_blocks && kb < N;
        const uint8_t *base = pool + (int64_t)(okb ? bid : 0) * L.index_block_bytes;
        const int slot0 = (int)((uint32_t)kc & slot_mask);
        const uint8_t *p = base + slot0 * L.key_bytes + lane_off;
        if constexpr (F4) {
            // block g of the key: 16 bytes (zero when the key has no block g)
            const bool vg = FULL || 16 * g < L.key_bytes;
            const i32x4 l0 = *(const i32x4 *)(p + (vg ? 16 * g : 0));
            Bk.lo = vg ? l0 : z4;
            Bk.hi = z4;
            const uint32_t w = ((const uint32_t *)(base + L.key_scale_off))[slot0 + c16];
            sb = (w >> (8 * g)) & 0xffu;
            sk = okb ? 1.0f : 0.0f;
            return;
        }
        sb = 127u;
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
    uint32_t kmn = 0xffffffffu, kmx = 0u;          // key range of the finite scores this lane writes
    auto score_sb = [&](int kb, const i32x8 &Bk, float sk, uint32_t sb) {
        f32x4 acc[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            if constexpr (F4)
                acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A[hb], Bk, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, (int)sa[hb], 0, (int)sb);
            else
                acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A[hb], Bk, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
        }
        __builtin_amdgcn_sched_barrier(0);         // the products back to back, each into its own registers
        float part = 0.0f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const f32x4 w4 = wls[hb * 4 + g];
#pragma unroll
            for (int i = 0; i < 4; ++i) part = relu_fma(acc[hb][i], w4[i], part);
        }
        part = group_sum4(part);
        if (g == 0 && kb + c16 < N) {
            const float v = sk * part;
            srow[kb + c16] = v;
            if (fabsf(v) < INFINITY) {
                const uint32_t u = score_key(v);
                kmn = min(kmn, u);
                kmx = max(kmx, u);
            }
        }
    };
    constexpr int GS = 2;                          // sub-blocks per pipeline group
    constexpr int NG = kKeysPerWave / 16 / GS;
    i32x8 B0[GS], B1[GS];
    float s0[GS], s1[GS];
    uint32_t e0[GS], e1[GS];
#pragma unroll
    for (int i = 0; i < GS; ++i) load_sb(k0 + 16 * i, B0[i], s0[i], e0[i]);
    // ---- the query rows: codes and weighted scales into LDS (rows past
    // idx_heads get weight 0 and are never read)
    if constexpr (F4) {
        if (wave < HB) {                           // (uniform)
#pragma unroll
            for (int i = 0; i < NQL; ++i) {
                const int h = wave * 16 + i;
                float v = 0.0f;
                if (h < L.HI) {                    // (uniform)
                    const int64_t row = (int64_t)q * L.HI + h;
                    v = quant_q_row<true>(L, qx0[i], qx1[i], w ? w[row] : 1.0f, qsl + h * 128);
                }
                if (lane == 0) ((float *)wls)[h] = v;
            }
        }
    } else {
        // E4M3, the decision rule of quant_q_row: the row's largest magnitude
        // (max over its four threads: exact in any order), scale = amax / 448,
        // codes of x * (448 / amax), wq = w * scale
        const int h = threadIdx.x >> 2, c = threadIdx.x & 3;
        const bool f32 = L.act != DSV4_DT_BF16;
        float x[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const uint32_t wf = qv[k >> 2][k & 3];                  // fp32: value k
            const uint32_t wb = qv[k >> 3][(k >> 1) & 3];           // bf16: value k in half k & 1
            const float v = __uint_as_float(f32 ? wf : ((k & 1) ? (wb & 0xffff0000u) : (wb << 16)));
            x[k] = 32 * c + k < dI ? v : 0.0f;
        }
        float am = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) am = fmaxf(am, fabsf(x[k]));
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        const bool nz = am >= 1e-30f;
        const float scale = nz ? am / 448.0f : 1.0f;
        const float inv = nz ? 448.0f / am : 1.0f;
        if (h < HB * 16) {
            uint32_t wd[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t u = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int d = 32 * c + 4 * k + b;
                    u |= (d < dI ? fp8_code(x[4 * k + b] * inv) : 0u) << (8 * b);
                }
                wd[k] = u;
            }
            uint4 *dst = (uint4 *)(qsl + h * 128 + 32 * c);
            dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
            if (c == 0) ((float *)wls)[h] = h < L.HI ? (w ? w[(int64_t)q * L.HI + h] : 1.0f) * scale : 0.0f;
        }
    }
    __syncthreads();
    // A operand: query codes (zero-padded to 128 bytes per row)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int row = hb * 16 + c16;
        const bool ok = row < L.HI;
        const uint8_t *p = qsl + (ok ? row : 0) * 128;
        i32x8 a;
        if constexpr (F4) {
            a.lo = *(const i32x4 *)(p + 16 * g);
            a.hi = z4;
            sa[hb] = ok ? (*(const uint32_t *)(p + 64) >> (8 * g)) & 0xffu : 0u;
        } else {
            a.lo = *(const i32x4 *)(p + o0);
            a.hi = *(const i32x4 *)(p + o1);
            sa[hb] = 127u;
        }
        A[hb] = ok ? a : (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
    if (k0 >= N) return;                           // (after the barrier: every wave takes part in it)
#pragma unroll
    for (int grp = 0; grp < NG; grp += 2) {
        const int kg = k0 + grp * GS * 16;
        if (kg >= N) break;                        // wave-uniform
#pragma unroll
        for (int i = 0; i < GS; ++i) load_sb(kg + GS * 16 + 16 * i, B1[i], s1[i], e1[i]);
#pragma unroll
        for (int i = 0; i < GS; ++i) score_sb(kg + 16 * i, B0[i], s0[i], e0[i]);
        const int kh = kg + GS * 16;
        if (kh >= N) break;
        if (grp + 2 < NG) {
#pragma unroll
            for (int i = 0; i < GS; ++i) load_sb(kh + GS * 16 + 16 * i, B0[i], s0[i], e0[i]);
        }
#pragma unroll
        for (int i = 0; i < GS; ++i) score_sb(kh + 16 * i, B1[i], s1[i], e1[i]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, o));
        kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, o));
    }
    // every wave with keys records its extremes (kmx == 0: no finite score)
    if (lane == 0) wr[(int64_t)q * nwr + k0 / kKeysPerWave] = make_uint2(kmn, kmx);
}

// ---------------------------------------------------------------- fp32 index rows
// Index keys stored as fp32 (the reference-precision storage mode) and the
// queries taken as given: grid (nwr / 4, n), one wave per 256 keys of a query
// (the score record the top-k passes read), lane l scoring keys k0 + 4l + c.
// Per key the head dot products are fp32 fma chains in dim order, ReLU and the
// head weights folded in head order; the workgroup's query rows and weights
// sit in LDS.  Decode and prefill queries take the same kernel.
__global__ __launch_bounds__(256) void k_index_score_f32(Lay L, dsv4_cache C, const void *qI, const float *w,
                                                         const int32_t *req, const int32_t *pos, float *scores,
                                                         int64_t ld, uint2 *wr, int nwr) {
    __shared__ float qs[64 * 128];
    __shared__ float ws_[64];
    const int q = blockIdx.y, lane = threadIdx.x & 63;
    const int HI = L.HI, dI = L.dI;
    for (int i = threadIdx.x; i < HI * dI; i += 256) qs[i] = load_act(qI, (int64_t)q * HI * dI + i, L.act);
    if (threadIdx.x < HI) ws_[threadIdx.x] = w ? w[(int64_t)q * HI + threadIdx.x] : 1.0f;
    __syncthreads();
    const int r = req[q];
    const int t = pos[q];
    if (r < 0 || r >= C.n_req || t < 0 || (int64_t)t >= (int64_t)C.max_blocks * kBlockTokens) return;
    const int N = (t + 1) / L.m;
    const int k0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kKeysPerWave;
    if (k0 >= N) return;
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
        const int j = k0 + 4 * lane + c;
        if (j >= N) break;
        const int64_t bid = block_id(C.block_table, C.max_blocks, C.n_blocks, r, ((int64_t)j * L.m) / kBlockTokens);
        float v = 0.0f;
        if (bid >= 0) {
            const float *key =
                (const float *)((const uint8_t *)C.index_keys + bid * L.index_block_bytes + (j % L.epb) * L.key_bytes);
            float acc = 0.0f;
            for (int h = 0; h < HI; ++h) {
                float dot = 0.0f;
                for (int e = 0; e < dI; ++e) dot = __builtin_fmaf(qs[h * dI + e], key[e], dot);
                acc = __builtin_fmaf(fmaxf(dot, 0.0f), ws_[h], acc);
            }
            v = acc;
        }
        scores[(int64_t)q * ld + j] = v;
        if (fabsf(v) < INFINITY) {
            const uint32_t u = score_key(v);
            mn = min(mn, u);
            mx = max(mx, u);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    }
    if (lane == 0) wr[(int64_t)q * nwr + k0 / kKeysPerWave] = make_uint2(mn, mx);
}

// ---------------------------------------------------------------- prefill scoring
// The queries of a prefill chunk read the same keys.  A workgroup scores
// kPfRows consecutive query rows (kPfWaveRows per wave) against kPfKeys keys,
// staged kPfChunk keys at a time through two LDS tiles: the next tile's loads
// are in flight while the current one is scored, and every staged key serves
// all rows of the workgroup.  A (row, 16-key sub-block) score takes exactly
// the decode scorer's operations, so a prefilled query scores bitwise like a
// decode step.  Rows of several requests in one workgroup are taken one
// request at a time.  The kernel asks the compiler for three waves per SIMD;
// the full-width variants (128-dim rows) need more registers than that allows
// (E4M3 254, MXFP4 228) and run two, which their LDS tiles allow anyway.
constexpr int kPfWaveRows = 2;
constexpr int kPfRows = 4 * kPfWaveRows;
constexpr int kPfKeys = 2048;
constexpr int kPfChunk = kKeysPerWave;                 // keys per tile (one extremes record per row)
constexpr int kPfRowBytes = 128 + 16;                  // LDS bytes per key: codes + one piece (bank shift)
static_assert(kPfKeys % kPfChunk == 0, "whole tiles per workgroup");

// LDS the prefill scorer needs beyond its static arrays: the block ids of its key range.
int64_t score_prefill_dyn_lds(const Lay &L) { return ((int64_t)kPfKeys * L.m / kBlockTokens + 2) * 4; }

template <int HB, bool FULL, bool F4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_index_score_prefill(Lay L, dsv4_cache C, const uint8_t *q8,
                                                             const float *wq, const int32_t *req,
                                                             const int32_t *pos, int n, float *scores,
                                                             int64_t ld, uint2 *wr, int nwr) {
    constexpr int QW = kPfWaveRows;
    __shared__ __attribute__((aligned(16))) uint8_t tile[2][kPfChunk * kPfRowBytes];
    __shared__ float tsc[2][kPfChunk];                 // key scale (FP8), or 1 / 0: key mapped or not (MXFP4)
    __shared__ uint32_t tsw[F4 ? 2 : 1][F4 ? kPfChunk : 1];   // (MXFP4) the keys' words of block scales
    __shared__ f32x4 wls[kPfRows][HB * 4];             // [row][hb][g]: heads hb*16 + 4g + i
    extern __shared__ int32_t btl[];                     // block ids of the key range
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // wave-uniform (scalar)
    const int row0 = blockIdx.y * kPfRows;
    const int kbeg = blockIdx.x * kPfKeys;
    const int dI = L.dI;
    for (int i = tid; i < kPfRows * HB * 16; i += 256) {
        const int rr = i / (HB * 16), h = i % (HB * 16), qi = row0 + rr;
        ((float *)wls[rr])[h] = (qi < n && h < L.HI) ? wq[(int64_t)qi * L.HI + h] : 0.0f;
    }
    if (!FULL) {                                         // code bytes past dI stay zero
        for (int i = tid; i < 2 * kPfChunk * kPfRowBytes / 16; i += 256) ((i32x4 *)tile)[i] = (i32x4){0, 0, 0, 0};
    }
    // the rows' requests and visible key counts (0: nothing to score)
    int rq[kPfRows], Nq[kPfRows];
#pragma unroll
    for (int i = 0; i < kPfRows; ++i) {
        const int qi = row0 + i;
        rq[i] = -1;
        Nq[i] = 0;
        if (qi < n) {
            const int r = req[qi], t = pos[qi];
            if (r >= 0 && r < C.n_req && t >= 0 && (int64_t)t < (int64_t)C.max_blocks * kBlockTokens) {
                rq[i] = r;
                Nq[i] = (t + 1) / L.m;
            }
        }
    }
    const int blk0 = (kbeg * L.m) / kBlockTokens;
    const int nbl = (kPfKeys * L.m) / kBlockTokens + 2;
    const uint8_t *pool = (const uint8_t *)C.index_keys;
    constexpr int PKMAX = F4 ? 4 : 8;                    // 16-byte pieces of a key (at most 64 / 128 bytes)
    const int PK = L.key_bytes / 16;
    int done = 0;
#pragma unroll
    for (int i = 0; i < kPfRows; ++i)
        if (Nq[i] <= kbeg) done |= 1 << i;
#pragma unroll 1
    while (done != (1 << kPfRows) - 1) {                 // one request per pass (workgroup-uniform)
        int R = -1;
#pragma unroll
        for (int i = kPfRows - 1; i >= 0; --i)
            if (!((done >> i) & 1)) R = rq[i];
        int act = 0, Nmax = 0;
#pragma unroll
        for (int i = 0; i < kPfRows; ++i)
            if (!((done >> i) & 1) && rq[i] == R) {
                act |= 1 << i;
                Nmax = Nq[i] > Nmax ? Nq[i] : Nmax;
            }
        done |= act;
        const int kend = kbeg + kPfKeys < Nmax ? kbeg + kPfKeys : Nmax;
        const int nch = (kend - kbeg + kPfChunk - 1) / kPfChunk;
        __syncthreads();                                 // the previous pass is done with the tiles and btl
        const int32_t *btr = C.block_table + (int64_t)R * C.max_blocks;
        for (int i = tid; i < nbl; i += 256) btl[i] = blk0 + i < C.max_blocks ? btr[blk0 + i] : -1;
        __syncthreads();
        // A operands of this wave's rows
        const int wr0 = wave * QW;                       // first row (within the workgroup) of this wave
        i32x8 A[QW][HB];
        uint32_t sa[QW][HB];                             // (MXFP4) the lane's block scale
#pragma unroll
        for (int i = 0; i < QW; ++i)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                const int hrow = hb * 16 + c16;
                const bool ok = ((act >> (wr0 + i)) & 1) && hrow < L.HI;
                const uint8_t *p = q8 + ((int64_t)(ok ? row0 + wr0 + i : 0) * L.HI + (ok ? hrow : 0)) * 128;
                i32x8 a;
                a.lo = *(const i32x4 *)(p + 16 * g);
                if constexpr (F4) {
                    a.hi = (i32x4){0, 0, 0, 0};
                    sa[i][hb] = ok ? (*(const uint32_t *)(p + 64) >> (8 * g)) & 0xffu : 0u;
                } else {
                    a.hi = *(const i32x4 *)(p + 64 + 16 * g);
                    sa[i][hb] = 127u;
                }
                A[i][hb] = ok ? a : (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
            }
        // one tile's loads: thread piece tid + 256u is piece (u mod PK) of key (tid + 256u) / PK;
        // thread tid also fetches key tid's scale.  Keys past the end, or in
        // unmapped blocks, read block 0 and get scale 0.
        // DMA (full-width E4M3 keys): the codes go straight into LDS
        // (global_load_lds, 16 bytes a lane): wave w's load u fills the 64
        // consecutive 16-byte slots (9w + u) * 64 + lane of the tile, whose rows
        // are 9 slots (a key's 8 pieces and the pad slot, which takes piece 0
        // again and is never read).  No staging registers: they hold the head
        // weights instead.
        constexpr bool DMA = FULL && !F4;
        constexpr int SLOTS = kPfRowBytes / 16;
        static_assert(!DMA || (kPfChunk * SLOTS) % 256 == 0, "the waves' loads cover the tile's slots");
        i32x4 stg[DMA ? 1 : PKMAX];
        float stg_s;
        uint32_t stg_w = 0;
        // key k (>= 0) sits in block k >> lgb at slot k & slot_mask: the
        // entries per block, 128 / m, are a power of two (divisions by the
        // layout's runtime values took a few dozen instructions a key)
        const uint32_t lgb = (uint32_t)__builtin_ctz((uint32_t)L.epb);
        const uint32_t slot_mask = (uint32_t)L.epb - 1u;
        auto load_tile = [&](int kc0, int tb) {
            if constexpr (DMA) {
#pragma unroll
                for (int u = 0; u < kPfChunk * SLOTS / 256; ++u) {
                    const int sl = (wave * (kPfChunk * SLOTS / 256) + u) * 64 + lane;
                    const int kk = sl / SLOTS, pp = sl % SLOTS, k = kc0 + kk;
                    const int bid = k < Nmax ? btl[(int)((uint32_t)k >> lgb) - blk0] : -1;
                    const bool ok = bid >= 0 && bid < C.n_blocks;
                    const uint8_t *src = pool + (ok ? (int64_t)bid * L.index_block_bytes +
                                                          (int)((uint32_t)k & slot_mask) * L.key_bytes + (pp < 8 ? pp : 0) * 16
                                                    : 0);
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void *)src,
                        (__attribute__((address_space(3))) void *)(tile[tb] + (sl - lane) * 16), 16, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < PKMAX; ++u) {
                if (DMA || u >= PK) break;
                const int pc = tid + 256 * u, kk = pc / PK, off = (pc % PK) * 16, k = kc0 + kk;
                const int bid = k < Nmax ? btl[(int)((uint32_t)k >> lgb) - blk0] : -1;
                const bool ok = bid >= 0 && bid < C.n_blocks;
                const uint8_t *src =
                    pool + (ok ? (int64_t)bid * L.index_block_bytes + (int)((uint32_t)k & slot_mask) * L.key_bytes + off : 0);
                stg[u] = *(const i32x4 *)src;
            }
            const int k = kc0 + tid;
            const int bid = k < Nmax ? btl[(int)((uint32_t)k >> lgb) - blk0] : -1;
            const bool ok = bid >= 0 && bid < C.n_blocks;
            const uint32_t sv = *(const uint32_t *)(pool + (ok ? (int64_t)bid * L.index_block_bytes + L.key_scale_off +
                                                                  (int)((uint32_t)k & slot_mask) * 4 : 0));
            if constexpr (F4) {
                stg_s = ok ? 1.0f : 0.0f;
                stg_w = sv;
            } else {
                stg_s = ok ? __uint_as_float(sv) : 0.0f;
            }
        };
        auto store_tile = [&](int b) {
#pragma unroll
            for (int u = 0; u < PKMAX; ++u) {
                if (DMA || u >= PK) break;
                const int pc = tid + 256 * u, kk = pc / PK, off = (pc % PK) * 16;
                *(i32x4 *)(tile[b] + kk * kPfRowBytes + off) = stg[u];
            }
            tsc[b][tid] = stg_s;
            if constexpr (F4) tsw[b][tid] = stg_w;
        };
        // Two 16-key sub-blocks of the wave's two rows per step: the four
        // partial sums are reduced together (group_sum4x4), after which lane
        // group g holds sub-block g / 2 of row g % 2, and every lane scores its
        // own key (the sum, scale and extremes of a key are the decode
        // scorer's, operation for operation).  Rows inactive or past their
        // visible keys store nothing.
        static_assert(QW == 2, "two rows a wave: the four lane groups take two rows of two sub-blocks");
        static_assert((kPfChunk / 16) % 2 == 0, "sub-blocks in pairs inside a tile");
        uint32_t kmn = 0xffffffffu, kmx = 0u;            // extremes of the lane's row (g % 2)
        // The lane's head weights held in registers for the pass (MXFP4 rows,
        // and E4M3 rows whose tiles are copied without staging registers): the
        // same 32 values serve every sub-block, and read from LDS per
        // sub-block they were four times the key operand's LDS bytes.
        constexpr bool WREG = F4 || DMA;
        f32x4 wreg[WREG ? 2 : 1][WREG ? HB : 1];
        if constexpr (WREG) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) wreg[ii][hb] = wls[wr0 + ii][hb * 4 + g];
        }
        // MXFP4 rows: a sub-block's eight products, then their epilogue
        auto partials = [&](int b, int sb, float (&part)[2]) {
            i32x8 Bk;
            const uint8_t *kr = tile[b] + (sb * 16 + c16) * kPfRowBytes;
            Bk.lo = *(const i32x4 *)(kr + 16 * g);
            uint32_t sbk = 127u;
            if constexpr (F4) {
                Bk.hi = (i32x4){0, 0, 0, 0};
                sbk = (tsw[b][sb * 16 + c16] >> (8 * g)) & 0xffu;
            } else {
                Bk.hi = *(const i32x4 *)(kr + 64 + 16 * g);
            }
            f32x4 acc[2][HB];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    if constexpr (F4)
                        acc[ii][hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            A[ii][hb], Bk, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, (int)sa[ii][hb], 0, (int)sbk);
                    else
                        acc[ii][hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            A[ii][hb], Bk, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
                }
            // the eight products issue back to back into their own registers:
            // left to itself the compiler reused two accumulators, so each
            // product waited for the previous one's epilogue
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                part[ii] = 0.0f;
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    f32x4 w4;
                    if constexpr (WREG) w4 = wreg[ii][hb];
                    else w4 = wls[wr0 + ii][hb * 4 + g];
#pragma unroll
                    for (int j = 0; j < 4; ++j) part[ii] = relu_fma(acc[ii][hb][j], w4[j], part[ii]);
                }
            }
        };
        const int ls = g >> 1, lr = g & 1, lrw = wr0 + lr;   // the lane's sub-block (of the pair) and row
        const bool lact = ((act >> lrw) & 1) != 0;
        const int lN = Nq[lrw];
        float *lsrow = scores + (int64_t)(row0 + lrw) * ld;
        // E4M3 rows: a sub-block's key operand, and the products of one row
        // of the wave with it (HB MFMAs)
        auto load_b = [&](int b, int sb, i32x8 &Bk) {
            const uint8_t *kr = tile[b] + (sb * 16 + c16) * kPfRowBytes;
            Bk.lo = *(const i32x4 *)(kr + 16 * g);
            Bk.hi = *(const i32x4 *)(kr + 64 + 16 * g);
        };
        auto mma = [&](const i32x8 &Bk, int ii, f32x4 (&acc)[HB]) {
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
                acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A[ii][hb], Bk, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
        };
        // ReLU and head weight of those products, summed in head order (the
        // decode scorer's chain)
        auto epi = [&](const f32x4 (&acc)[HB], int ii) {
            float part = 0.0f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                f32x4 w4;
                if constexpr (WREG) w4 = wreg[ii][hb];
                else w4 = wls[wr0 + ii][hb * 4 + g];
#pragma unroll
                for (int j = 0; j < 4; ++j) part = relu_fma(acc[hb][j], w4[j], part);
            }
            return part;
        };
        // Software pipeline over (sub-block, row) halves: each stage issues
        // the next half's products between the epilogue instructions of the
        // current one (one MFMA per eight VALU operations), so one wave feeds
        // the matrix unit and the VALU together (only in part: each of these
        // MFMAs holds the VALU issue for about half of its 32 cycles).  X and
        // Y take turns as the accumulators; the sums and their order are
        // unchanged.
        auto interleave = [&]() {
#pragma unroll
            for (int i = 0; i < HB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // eight VALU
            }
        };
        auto score_tile = [&](int b, int kc0) {
            const int np = min(kPfChunk / 32, (kend - kc0 + 31) / 32);   // sub-block pairs holding keys
            i32x8 Bc, Bn;
            f32x4 X[HB], Y[HB];
            load_b(b, 0, Bc);
            mma(Bc, 0, X);
#pragma unroll 1
            for (int p = 0; p < np; ++p) {
                const int sb = 2 * p;
                const bool more = p + 1 < np;
                __builtin_amdgcn_sched_barrier(0);
                load_b(b, sb + 1, Bn);
                mma(Bc, 1, Y);
                const float r0 = epi(X, 0);
                interleave();
                __builtin_amdgcn_sched_barrier(0);
                mma(Bn, 0, X);
                const float r1 = epi(Y, 1);
                interleave();
                __builtin_amdgcn_sched_barrier(0);
                load_b(b, more ? sb + 2 : sb, Bc);   // (the last pair: its own again, in bounds)
                mma(Bn, 1, Y);
                const float r2 = epi(X, 0);
                interleave();
                __builtin_amdgcn_sched_barrier(0);
                mma(Bc, 0, X);                           // (after the last pair: discarded)
                const float r3 = epi(Y, 1);
                interleave();
                // X is read only by the next pass: without this use the
                // compiler sinks its products to the top of the loop, out of
                // this stage's interleave
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) asm volatile("" : "+v"(X[hb]));
                __builtin_amdgcn_sched_barrier(0);
                // the four partial sums reduced together: lane group g then
                // holds sub-block sb + g / 2 of row g % 2
                const float part = group_sum4x4(r0, r1, r2, r3);
                const int key = kc0 + sb * 16 + 16 * ls + c16;
                const float sk = tsc[b][(sb + ls) * 16 + c16];
                if (lact && key < lN) {
                    const float v = sk * part;
                    lsrow[key] = v;
                    if (fabsf(v) < INFINITY) {
                        const uint32_t u = score_key(v);
                        kmn = min(kmn, u);
                        kmx = max(kmx, u);
                    }
                }
            }
        };
        auto score_pair = [&](int b, int sb, int kb) {   // sub-blocks sb, sb + 1; kb: the first key of sb
            float p0[2], p1[2];
            partials(b, sb, p0);
            __builtin_amdgcn_sched_barrier(0);           // one sub-block's MFMA results live at a time
            partials(b, sb + 1, p1);
            const float part = group_sum4x4(p0[0], p0[1], p1[0], p1[1]);
            const int key = kb + 16 * ls + c16;
            const float sk = tsc[b][(sb + ls) * 16 + c16];
            if (lact && key < lN) {
                const float v = sk * part;
                lsrow[key] = v;
                if (fabsf(v) < INFINITY) {
                    const uint32_t u = score_key(v);
                    kmn = min(kmn, u);
                    kmx = max(kmx, u);
                }
            }
        };
        // (DMA: every wave waits for its own copies before each tile barrier)
        auto copies_done = [&]() {
            if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        };
        load_tile(kbeg, 0);
        store_tile(0);
        copies_done();
        __syncthreads();
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            const int kc0 = kbeg + c * kPfChunk, b = c & 1;
            if (c + 1 < nch) load_tile(kc0 + kPfChunk, b ^ 1);   // in flight while this tile is scored
            kmn = 0xffffffffu;
            kmx = 0u;
            if constexpr (F4) {
#pragma unroll 1
                for (int sb = 0; sb < kPfChunk / 16; sb += 2) {
                    const int kb = kc0 + sb * 16;
                    if (kb >= kend) break;               // workgroup-uniform
                    score_pair(b, sb, kb);
                }
            } else {
                score_tile(b, kc0);
            }
            // this tile's extremes per row (the record the decode scorer's wave
            // for these keys writes): over the lanes of the row's two lane
            // groups (lane bit 4 is the row), found in lanes 0 and 16
            {
                uint32_t mn = kmn, mx = kmx;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    if (o == 16) continue;
                    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
                    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
                }
                if ((lane & ~16) == 0 && lact && kc0 < lN)
                    wr[(int64_t)(row0 + lrw) * nwr + kc0 / kKeysPerWave] = make_uint2(mn, mx);
            }
            if (c + 1 < nch) store_tile(b ^ 1);
            copies_done();
            __syncthreads();                             // next tile visible; this one free
        }
    }
}

// ---------------------------------------------------------------- top-k
// Exact selection of the min(k, N) largest scores of a query by (score desc,
// index asc), emitted in ascending index order.  The score row is cut into
// segments of kTkSeg scores and the selection runs in four launches, each
// independent of how many queries share it:
//   hist   per segment, a kTkBins histogram of its scores mapped linearly onto
//          the query's finite score range (the scorer records each wave's
//          extremes).  The map is monotone, so bins are ordered by score; NaN
//          lies below every bin and +-inf fall into the end bins;
//   bin    per query, the bin b* holding the k-th largest score, how many
//          elements lie above it (all selected: "sure") and how many remain to
//          be taken from inside it, plus each segment's output offsets;
//   split  per segment, its sure indices and its candidates (elements of b*:
//          key and index) written in index order at those offsets;
//   final  per query, the exact threshold among the candidates (the rem-th
//          largest key; ties go to the lower index) and a merge of the sure
//          list with the chosen candidates.  When b* holds more than
//          kTkCandMax elements the threshold is refined by radix passes over
//          the query's whole score row instead, and the row is compacted
//          directly.
// Every count is an exact integer and every order is fixed, so the result is
// unique.
constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkVec = kTkSeg / (kTkThreads * 4);    // float4 loads per thread and segment
static_assert(kTkVec * kTkThreads * 4 == kTkSeg, "segment = whole float4 rows");
static_assert(kTkBins == kTkThreads * 8, "eight bins per thread");

struct TkArgs {
    Lay L;
    const int32_t *req, *pos;
    int n_req;
    int64_t max_tokens;
    IndexWs ws;
    int32_t *out;
    const int32_t *nvis;    // explicit row lengths (rows of given scores), else from req / pos
    int64_t nvis_max;
};

// Elements of row q: the visible compressed entries of query q, or the given
// row length (0 for an invalid request / position / length).  Split in two so
// that a kernel can issue the two loads together with its others and wait once.
struct TkRowLen {
    int32_t a, b;
};
__device__ __forceinline__ TkRowLen tk_fetch(const TkArgs &A, int q) {
    const int32_t *pa = A.nvis ? A.nvis : A.req;
    const int32_t *pb = A.nvis ? A.nvis : A.pos;
    return TkRowLen{pa[q], pb[q]};
}
__device__ __forceinline__ int64_t tk_count(const TkArgs &A, TkRowLen v) {
    if (A.nvis) return (v.a < 0 || (int64_t)v.a > A.nvis_max) ? 0 : v.a;
    const int r = v.a;
    const int64_t t = v.b;
    if (r < 0 || r >= A.n_req || t < 0 || t >= A.max_tokens) return 0;
    return (t + 1) / A.L.m;
}
__device__ __forceinline__ int64_t tk_visible(const TkArgs &A, int q) { return tk_count(A, tk_fetch(A, q)); }

__device__ __forceinline__ int bit_length(uint32_t x) { return x ? 32 - __clz(x) : 0; }

// Float value of an order-preserving key (key 0, the NaN key, is excluded by callers).
__device__ __forceinline__ float key_value(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Linear map of [fmin, fmax] onto bins 0 .. kTkBins-1 (scale 0 when the range
// is empty, a single value or not finite: every score then lands in bin 0).
__device__ __forceinline__ void tk_map(uint32_t kmin, uint32_t kmax, float &fmin, float &scale) {
    fmin = 0.0f;
    scale = 0.0f;
    if (kmax == 0u || kmin > kmax) return;
    fmin = key_value(kmin);
    const float range = key_value(kmax) - fmin;
    if (range > 0.0f && range < INFINITY) scale = (float)(kTkBins - 1) / range;
}

// Bin of key u: -1 for NaN, else monotone non-decreasing in u.
// (Selects only, no branches.)
__device__ __forceinline__ int tk_digit(uint32_t u, float fmin, float scale) {
    const float y = (key_value(u) - fmin) * scale;
    // y <= 0 also catches -inf and the NaN products of scale 0
    const float yc = y > 0.0f ? (y < (float)(kTkBins - 1) ? y : (float)(kTkBins - 1)) : 0.0f;
    return u == 0u ? -1 : (int)yc;
}

// Wave-wide inclusive scan under an associative op with identity id, on the
// DPP cross-lane paths (no LDS round trips): prefix within each row of 16
// lanes by shifts of 1, 2, 4, 8, then the row totals carried into the rows
// above (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3).
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op) {
    const int i = (int)id;
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(i, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(i, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(i, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(i, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(i, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(i, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) { return wave_scan(x, 0u, OpAdd()); }
__device__ __forceinline__ uint32_t wave_last(uint32_t x) { return (uint32_t)__builtin_amdgcn_readlane((int)x, 63); }
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) { return wave_last(wave_incl_scan(x)); }
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) { return wave_last(wave_scan(x, 0xffffffffu, OpMin())); }
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) { return wave_last(wave_scan(x, 0u, OpMax())); }

// Exclusive prefix (thread order) of NV values per thread at once, and their
// block totals.  wt: LDS scratch of NV * kTkWaves words.  Contains barriers.
template <int NV>
__device__ __forceinline__ void block_excl(uint32_t (&x)[NV], uint32_t (&tot)[NV], uint32_t *wt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        incl[v] = wave_incl_scan(x[v]);
        if (lane == 63) wt[v * kTkWaves + wave] = incl[v];
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        uint32_t base = 0, t = 0;
#pragma unroll
        for (int w = 0; w < kTkWaves; ++w) {
            const uint32_t c = wt[v * kTkWaves + w];
            base += w < wave ? c : 0u;
            t += c;
        }
        x[v] = base + incl[v] - x[v];
        tot[v] = t;
    }
    __syncthreads();
}

// Min / max over the block (all threads get the result).  Contains barriers.
__device__ __forceinline__ void block_minmax(uint32_t &mn, uint32_t &mx, uint32_t *wt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    mn = wave_umin(mn);
    mx = wave_umax(mx);
    if (lane == 0) {
        wt[wave] = mn;
        wt[kTkWaves + wave] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
        mn = min(mn, wt[w]);
        mx = max(mx, wt[kTkWaves + w]);
    }
    __syncthreads();
}

// Over hist[0..nb) (nb <= kTkBins, bins ordered by value), the bin holding the
// rem-th largest element and how many elements lie in higher bins.  bin = -1
// (and before = the total) when fewer than rem elements were counted.
// Contains barriers.
__device__ __forceinline__ void tk_find_bin(const uint32_t *hist, int nb, uint32_t rem, uint32_t *wt,
                                            int *bin_out, uint32_t *before_out) {
    __shared__ int s_bin;
    __shared__ uint32_t s_before;
    const int tid = threadIdx.x;
    uint32_t c[8], sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {                    // reversed bins: largest first
        const int rb = tid * 8 + j;
        c[j] = rb < nb ? hist[nb - 1 - rb] : 0u;
        sum += c[j];
    }
    uint32_t x[1] = {sum}, tot[1];
    block_excl<1>(x, tot, wt);
    if (tid == 0 && tot[0] < rem) {
        s_bin = -1;
        s_before = tot[0];
    }
    uint32_t run = x[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (run < rem && rem <= run + c[j]) {
            s_bin = nb - 1 - (tid * 8 + j);
            s_before = run;
        }
        run += c[j];
    }
    __syncthreads();
    *bin_out = s_bin;
    *before_out = s_before;
    __syncthreads();
}

__device__ __forceinline__ uint32_t shr32(uint32_t v, int s) { return s >= 32 ? 0u : v >> s; }

// Exact rem-th largest among the keys get(p), p < n, that satisfy in(u); all
// such keys lie in [lo_key, hi_key].  Radix passes of up to 11 bits over
// u - lo_key.  Returns the key; *need receives how many keys equal to it are
// among the rem largest.  Contains barriers.
template <typename Get, typename In>
__device__ uint32_t tk_refine(Get get, int64_t n, In in, uint32_t lo_key, uint32_t hi_key, uint32_t rem,
                              uint32_t *hist, uint32_t *wt, uint32_t *need) {
    int hs = bit_length(hi_key - lo_key);
    uint32_t hv = 0;
    while (hs > 0) {
        const int lo = hs > 11 ? hs - 11 : 0;
        const int nb = 1 << (hs - lo);
        for (int b = threadIdx.x; b < kTkBins; b += kTkThreads) hist[b] = 0;
        __syncthreads();
        for (int64_t p = threadIdx.x; p < n; p += kTkThreads) {
            const uint32_t u = get(p);
            if (!in(u)) continue;
            const uint32_t v = u - lo_key;
            if (shr32(v, hs) == hv) atomicAdd(&hist[(v >> lo) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        int fb;
        uint32_t before;
        tk_find_bin(hist, nb, rem, wt, &fb, &before);
        hv = (hv << (hs - lo)) | (uint32_t)fb;       // fb >= 0: the keys in range number >= rem
        rem -= before;
        hs = lo;
    }
    *need = rem;
    return lo_key + hv;
}

// Rows of given scores: grid (nwr / 4, n), one wave per 256 scores records
// the extremes of its finite scores, as the scoring kernel does.
__global__ __launch_bounds__(256) void k_tk_extremes(TkArgs A) {
    const int q = blockIdx.y, lane = threadIdx.x & 63;
    const int64_t k0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kKeysPerWave;
    const int64_t N = tk_visible(A, q);
    if (k0 >= N) return;
    const float4 x = *(const float4 *)(A.ws.scores + (int64_t)q * A.ws.ld + k0 + 4 * lane);
    const float e[4] = {x.x, x.y, x.z, x.w};
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (k0 + 4 * lane + c < N && fabsf(e[c]) < INFINITY) {
            const uint32_t u = score_key(e[c]);
            mn = min(mn, u);
            mx = max(mx, u);
        }
    }
    mn = wave_umin(mn);
    mx = wave_umax(mx);
    if (lane == 0) A.ws.wr[(int64_t)q * A.ws.nwr + k0 / kKeysPerWave] = make_uint2(mn, mx);
}

// Histograms are stored as 16-bit counts (a segment holds at most 4096
// scores): thread t of a pass owns bins [8t, 8t+8), one 16-byte word.
__device__ __forceinline__ void tk_unpack8(const uint4 &h, uint32_t (&c)[8]) {
    c[0] = h.x & 0xffffu; c[1] = h.x >> 16;
    c[2] = h.y & 0xffffu; c[3] = h.y >> 16;
    c[4] = h.z & 0xffffu; c[5] = h.z >> 16;
    c[6] = h.w & 0xffffu; c[7] = h.w >> 16;
}

// Pass 1: grid (s_max, n).  Histogram of one segment.  Every load whose
// address is known up front is issued before the row length is read (rows and
// per-wave extremes are always in bounds), so the kernel waits on memory once.
__global__ __launch_bounds__(kTkThreads) void k_tk_hist(TkArgs A) {
    __shared__ uint32_t hist[kTkBins];
    __shared__ uint32_t wt[2 * kTkWaves];
    const int q = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
    const IndexWs &W = A.ws;
    const float *row = W.scores + (int64_t)q * W.ld + (int64_t)s * kTkSeg;
    float4 x[kTkVec];
#pragma unroll
    for (int v = 0; v < kTkVec; ++v) x[v] = *(const float4 *)(row + v * kTkThreads * 4 + 4 * tid);
    // (clamped indices keep every load unconditional: no branch between them)
    const uint2 e0 = W.wr[(int64_t)q * W.nwr + min(tid, W.nwr - 1)];
    const TkRowLen rl = tk_fetch(A, q);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t N = tk_count(A, rl);
    const int k = A.L.topk;
    if (N <= k || (int64_t)s * kTkSeg >= N) return;
    const int n = (int)min((int64_t)kTkSeg, N - (int64_t)s * kTkSeg);
    // the query's finite score range, from the scoring waves' extremes
    const int nw = (int)((N + kKeysPerWave - 1) / kKeysPerWave);
    uint32_t mn = 0xffffffffu, mx = 0u;
    if (tid < nw && e0.y != 0u) {
        mn = e0.x;
        mx = e0.y;
    }
    for (int i = tid + kTkThreads; i < nw; i += kTkThreads) {
        const uint2 e = W.wr[(int64_t)q * W.nwr + i];
        if (e.y != 0u) {
            mn = min(mn, e.x);
            mx = max(mx, e.y);
        }
    }
    for (int b = tid; b < kTkBins; b += kTkThreads) hist[b] = 0;
    block_minmax(mn, mx, wt);
    float fmin, scale;
    tk_map(mn, mx, fmin, scale);
#pragma unroll
    for (int v = 0; v < kTkVec; ++v) {
        const int p = v * kTkThreads * 4 + 4 * tid;
        const float e[4] = {x[v].x, x[v].y, x[v].z, x[v].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int d = p + c < n ? tk_digit(score_key(e[c]), fmin, scale) : -1;
            if (d >= 0) atomicAdd(&hist[d], 1u);
        }
    }
    __syncthreads();
    const uint32_t *h = hist + 8 * tid;
    *(uint4 *)(W.hist + ((int64_t)q * W.s_max + s) * kTkBins + 8 * tid) =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    if (s == 0 && tid == 0) {
        W.qm[q].fmin = fmin;
        W.qm[q].scale = scale;
    }
}

// Query histogram over segments [0, S) (c) and over segments [0, s_lim) (p),
// bins [8t, 8t+8) of thread t; eight segments' loads in flight at a time.
template <bool PREFIX>
__device__ __forceinline__ void tk_sum_hists(const uint16_t *gh, int S, int s_lim, uint32_t (&c)[8],
                                             uint32_t (&p)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = p[j] = 0;
    for (int s0 = 0; s0 < S; s0 += 8) {
        uint4 h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            h[i] = s0 + i < S ? *(const uint4 *)(gh + (int64_t)(s0 + i) * kTkBins + 8 * threadIdx.x)
                              : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t e[8];
            tk_unpack8(h[i], e);
            const bool before = PREFIX && s0 + i < s_lim;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c[j] += e[j];
                p[j] += before ? e[j] : 0u;
            }
        }
    }
}

// Pass 2 (rows of more than kTkFuseSeg segments): grid (n).  Boundary bin of
// the query and every segment's output offsets.  (With fewer segments the
// split pass derives them itself.)
__global__ __launch_bounds__(kTkThreads) void k_tk_bin(TkArgs A) {
    __shared__ uint32_t hist[kTkBins];
    __shared__ uint32_t wt[3 * kTkWaves];
    __shared__ uint32_t seg_sure[kTkMaxSeg], seg_cand[kTkMaxSeg];
    const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t N = tk_visible(A, q);
    const uint32_t k = (uint32_t)A.L.topk;
    if (N <= (int64_t)k) return;
    const IndexWs &W = A.ws;
    const int S = (int)((N + kTkSeg - 1) / kTkSeg);
    const uint16_t *gh = W.hist + (int64_t)q * W.s_max * kTkBins;
    uint32_t c[8], p[8];
    tk_sum_hists<false>(gh, S, 0, c, p);
#pragma unroll
    for (int j = 0; j < 8; ++j) hist[8 * tid + j] = c[j];
    __syncthreads();
    int bstar;
    uint32_t above;
    tk_find_bin(hist, kTkBins, k, wt, &bstar, &above);
    // per segment: elements above b* and inside b* (NaN scores form the bin
    // below bin 0); wave w takes segments w, w + 4, ..., the loads of four of
    // them at a time in flight (segments past S re-read segment S-1, unused)
    constexpr int SB = 4;
    for (int s0 = wave; s0 < S; s0 += SB * kTkWaves) {
        uint4 hv[SB][4];
#pragma unroll
        for (int b4 = 0; b4 < SB; ++b4) {
            const int s = min(s0 + b4 * kTkWaves, S - 1);
            const uint16_t *h = gh + (int64_t)s * kTkBins + 32 * lane;
#pragma unroll
            for (int j = 0; j < 4; ++j) hv[b4][j] = *(const uint4 *)(h + 8 * j);
        }
#pragma unroll
        for (int b4 = 0; b4 < SB; ++b4) {
            const int s = s0 + b4 * kTkWaves;
            if (s >= S) break;                       // (wave-uniform)
            uint32_t sure = 0, all = 0, inb = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t e[8];
                tk_unpack8(hv[b4][j], e);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int b = 32 * lane + 8 * j + i;
                    all += e[i];
                    sure += b > bstar ? e[i] : 0u;
                    inb += b == bstar ? e[i] : 0u;
                }
            }
            sure = wave_sum(sure);
            all = wave_sum(all);
            inb = wave_sum(inb);
            if (lane == 0) {
                const uint32_t ns = (uint32_t)min((int64_t)kTkSeg, N - (int64_t)s * kTkSeg);
                seg_sure[s] = sure;
                seg_cand[s] = bstar >= 0 ? inb : ns - all;
            }
        }
    }
    __syncthreads();
    uint32_t base_s = 0, base_c = 0;
    for (int s0 = 0; s0 < S; s0 += kTkThreads) {
        const int s = s0 + tid;
        uint32_t x[2] = {s < S ? seg_sure[s] : 0u, s < S ? seg_cand[s] : 0u}, tot[2];
        block_excl<2>(x, tot, wt);
        if (s < S) W.segoff[(int64_t)q * W.s_max + s] = make_int2((int)(base_s + x[0]), (int)(base_c + x[1]));
        base_s += tot[0];
        base_c += tot[1];
    }
    if (tid == 0) {
        W.qm[q].bstar = bstar;
        W.qm[q].rem = (int32_t)(k - base_s);
        W.qm[q].n_sure = (int32_t)base_s;
        W.qm[q].n_cand = (int32_t)base_c;
    }
}

// Pass 3: grid (s_max, n).  Sure indices and candidates of one segment, in
// index order.  FUSED (s_max <= kTkFuseSeg): the boundary bin and this
// segment's offsets come from the histograms directly (every workgroup of the
// query derives the same values; segment 0 records them for the final pass).
// All loads are issued before the row length is known.
template <bool FUSED>
__global__ __launch_bounds__(kTkThreads) void k_tk_split(TkArgs A) {
    __shared__ uint32_t wt[2 * kTkVec * kTkWaves];
    const int q = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
    const IndexWs &W = A.ws;
    const float *row = W.scores + (int64_t)q * W.ld + (int64_t)s * kTkSeg;
    float4 x[kTkVec];
#pragma unroll
    for (int v = 0; v < kTkVec; ++v) x[v] = *(const float4 *)(row + v * kTkThreads * 4 + 4 * tid);
    const float2 map = *(const float2 *)&W.qm[q].fmin;
    uint4 hw[FUSED ? kTkFuseSeg : 1];
    int2 off = make_int2(0, 0);
    int32_t q_bstar = 0, q_ncand = 0;
    if constexpr (FUSED) {
        const uint16_t *gh = W.hist + (int64_t)q * W.s_max * kTkBins + 8 * tid;
        // (clamped indices keep every load unconditional: no branch between them)
#pragma unroll
        for (int i = 0; i < kTkFuseSeg; ++i) hw[i] = *(const uint4 *)(gh + (int64_t)min(i, W.s_max - 1) * kTkBins);
    } else {
        off = W.segoff[(int64_t)q * W.s_max + s];
        q_bstar = W.qm[q].bstar;
        q_ncand = W.qm[q].n_cand;
    }
    const TkRowLen rl = tk_fetch(A, q);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t N = tk_count(A, rl);
    const int k = A.L.topk;
    if (N <= k || (int64_t)s * kTkSeg >= N) return;
    const int n = (int)min((int64_t)kTkSeg, N - (int64_t)s * kTkSeg);
    const float fmin = map.x, scale = map.y;
    int bstar;
    uint32_t sure_off, cand_off, above = 0, n_cand;
    if constexpr (FUSED) {
        __shared__ uint32_t hist[kTkBins];
        const int S = (int)((N + kTkSeg - 1) / kTkSeg);
        uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0}, p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < kTkFuseSeg; ++i) {
            uint32_t e[8];
            tk_unpack8(hw[i], e);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c[j] += i < S ? e[j] : 0u;
                p[j] += i < s ? e[j] : 0u;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) hist[8 * tid + j] = c[j];
        __syncthreads();
        tk_find_bin(hist, kTkBins, (uint32_t)k, wt, &bstar, &above);
        uint32_t r[4] = {0, 0, 0, 0}, tot[4];       // prefix above b*, prefix all, prefix in b*, query all
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int b = 8 * tid + j;
            r[0] += b > bstar ? p[j] : 0u;
            r[1] += p[j];
            r[2] += b == bstar ? p[j] : 0u;
            r[3] += c[j];
        }
        block_excl<4>(r, tot, wt);
        sure_off = tot[0];
        cand_off = bstar >= 0 ? tot[2] : (uint32_t)s * kTkSeg - tot[1];
        n_cand = bstar >= 0 ? hist[bstar] : (uint32_t)N - tot[3];
    } else {
        bstar = q_bstar;
        n_cand = (uint32_t)q_ncand;
        sure_off = (uint32_t)off.x;
        cand_off = (uint32_t)off.y;
    }
    const bool keep = n_cand <= (uint32_t)kTkCandMax;
    uint32_t key[kTkVec][4];
    int dg[kTkVec][4];
    uint32_t cnt[2 * kTkVec];
#pragma unroll
    for (int v = 0; v < kTkVec; ++v) {
        const float e[4] = {x[v].x, x[v].y, x[v].z, x[v].w};
        uint32_t ns = 0, nc = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int p = v * kTkThreads * 4 + 4 * tid + c;
            key[v][c] = score_key(e[c]);
            // beyond the row's end: a bin below every other (never chosen)
            dg[v][c] = p < n ? tk_digit(key[v][c], fmin, scale) : -2;
            ns += dg[v][c] > bstar;
            nc += dg[v][c] == bstar;
        }
        cnt[v] = ns;
        cnt[kTkVec + v] = nc;
    }
    uint32_t tot[2 * kTkVec];
    block_excl<2 * kTkVec>(cnt, tot, wt);
    uint32_t bs = sure_off, bc = cand_off;
    int32_t *sure = W.sure + (int64_t)q * k;
    uint32_t *ck = W.ckey + (int64_t)q * kTkCandMax;
    int32_t *cp = W.cpos + (int64_t)q * kTkCandMax;
    int32_t *cr = W.crank + (int64_t)q * kTkCandMax;
#pragma unroll
    for (int v = 0; v < kTkVec; ++v) {
        uint32_t is = bs + cnt[v], ic = bc + cnt[kTkVec + v];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int32_t idx = (int32_t)((int64_t)s * kTkSeg + v * kTkThreads * 4 + 4 * tid + c);
            if (dg[v][c] > bstar) sure[is++] = idx;
            if (dg[v][c] == bstar && keep) {
                ck[ic] = key[v][c];
                cp[ic] = idx;
                cr[ic] = (int32_t)is;                // sure elements before it
                ++ic;
            }
        }
        bs += tot[v];
        bc += tot[kTkVec + v];
    }
    if (FUSED && s == 0 && tid == 0) {
        W.qm[q].bstar = bstar;
        W.qm[q].rem = (int32_t)((uint32_t)k - above);
        W.qm[q].n_sure = (int32_t)above;
        W.qm[q].n_cand = (int32_t)n_cand;
    }
}

// Pass 4: grid (n).  Exact threshold and the ascending output list.
__global__ __launch_bounds__(kTkThreads) void k_tk_final(TkArgs A) {
    constexpr int kMaxK = 2048;
    __shared__ uint32_t ckey[kTkCandMax];
    __shared__ int32_t cpos[kTkCandMax];
    __shared__ int32_t crk[kTkCandMax];
    __shared__ int32_t sure[kMaxK], slotv[kMaxK];
    __shared__ uint32_t hist[kTkBins];
    __shared__ uint32_t wt[4 * kTkWaves];
    __shared__ uint32_t s_thr, s_need;
    const int q = blockIdx.x, tid = threadIdx.x;
    const int k = A.L.topk;
    const IndexWs &W = A.ws;
    // the first candidates, the sure list and the query's counts, all read
    // before the row length (the workspace rows are always that long)
    const uint32_t ck0 = W.ckey[(int64_t)q * kTkCandMax + tid];
    const int32_t cp0 = W.cpos[(int64_t)q * kTkCandMax + tid];
    const int32_t cr0 = W.crank[(int64_t)q * kTkCandMax + tid];
    int32_t su[kMaxK / kTkThreads];
#pragma unroll
    for (int j = 0; j < kMaxK / kTkThreads; ++j) su[j] = W.sure[(int64_t)q * k + min(tid + j * kTkThreads, k - 1)];
    const TkQuery M = W.qm[q];
    const TkRowLen rl = tk_fetch(A, q);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t N = tk_count(A, rl);
    int32_t *out = A.out + (int64_t)q * k;
    if (N <= k) {                                    // everything visible, ascending, then padding
        for (int i = tid; i < k; i += kTkThreads) out[i] = i < N ? i : -1;
        return;
    }
    const uint32_t rem = (uint32_t)M.rem;
    const int D = M.n_sure;
    const float *row = W.scores + (int64_t)q * W.ld;
    const int bstar = M.bstar;
    auto in_b = [&](uint32_t u) { return tk_digit(u, M.fmin, M.scale) == bstar; };
    uint32_t T, need;
    if (M.n_cand <= kTkCandMax) {
        const int C = M.n_cand;
        if (tid < C) {
            ckey[tid] = ck0;
            cpos[tid] = cp0;
            crk[tid] = cr0;
        }
        for (int i = kTkThreads + tid; i < C; i += kTkThreads) {
            ckey[i] = W.ckey[(int64_t)q * kTkCandMax + i];
            cpos[i] = W.cpos[(int64_t)q * kTkCandMax + i];
            crk[i] = W.crank[(int64_t)q * kTkCandMax + i];
        }
        for (int i = tid; i < k; i += kTkThreads) slotv[i] = -1;
#pragma unroll
        for (int j = 0; j < kMaxK / kTkThreads; ++j)
            if (tid + j * kTkThreads < D) sure[tid + j * kTkThreads] = su[j];
        __syncthreads();
        if (C <= kTkThreads) {
            // rank the candidates: the rem-th largest has fewer than rem
            // candidates above it and at least rem at or above it
            if (tid < C) {
                const uint32_t mine = ck0;
                uint32_t gt = 0, ge = 0;
                for (int j = 0; j < C; ++j) {
                    const uint32_t c = ckey[j];
                    gt += c > mine;
                    ge += c >= mine;
                }
                if (gt < rem && rem <= ge) {         // equal candidates write equal values
                    s_thr = mine;
                    s_need = rem - gt;
                }
            }
            __syncthreads();
            T = s_thr;
            need = s_need;
        } else {
            uint32_t lo = 0xffffffffu, hi = 0u;
            for (int i = tid; i < C; i += kTkThreads) {
                lo = min(lo, ckey[i]);
                hi = max(hi, ckey[i]);
            }
            block_minmax(lo, hi, wt);
            T = tk_refine([&](int64_t p) { return ckey[p]; }, C, [](uint32_t) { return true; }, lo, hi, rem, hist,
                          wt, &need);
        }
        // chosen candidates in index order: above T, then the first `need`
        // equal to T.  The j-th chosen one, with r sure elements before it,
        // takes output slot j + r; the sure elements fill the other slots in order.
        uint32_t ngt = 0, neq = 0;                   // candidates above / equal to T so far
        for (int i0 = 0; i0 < C; i0 += kTkThreads) {
            const int i = i0 + tid;
            const uint32_t u = i < C ? ckey[i] : 0u;
            const bool gt = i < C && u > T, isq = i < C && u == T;
            uint32_t x[2] = {gt ? 1u : 0u, isq ? 1u : 0u}, tx[2];
            block_excl<2>(x, tx, wt);
            const uint32_t eq_before = neq + x[1];
            // chosen ones before i: all above T, and the first `need` equal to T
            const uint32_t j = ngt + x[0] + min(eq_before, need);
            if (gt || (isq && eq_before < need)) slotv[j + crk[i]] = cpos[i];
            ngt += tx[0];
            neq += tx[1];
        }
        __syncthreads();
        uint32_t fr[1] = {0}, tf[1];
        int32_t sv[kMaxK / kTkThreads];
        constexpr int SPT = kMaxK / kTkThreads;      // output slots per thread
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int slot = SPT * tid + j;
            sv[j] = slot < k ? slotv[slot] : 0;
            fr[0] += (slot < k && sv[j] < 0) ? 1u : 0u;
        }
        block_excl<1>(fr, tf, wt);
        uint32_t f = fr[0];
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int slot = SPT * tid + j;
            if (slot < k) out[slot] = sv[j] >= 0 ? sv[j] : sure[f++];
        }
        return;
    }
    // crowded boundary bin: refine over the whole row, then compact it
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int64_t p = tid; p < N; p += kTkThreads) {
        const uint32_t u = score_key(row[p]);
        if (in_b(u)) {
            lo = min(lo, u);
            hi = max(hi, u);
        }
    }
    block_minmax(lo, hi, wt);
    T = tk_refine([&](int64_t p) { return score_key(row[p]); }, N, in_b, lo, hi, rem, hist, wt, &need);
    uint32_t nsel = 0, neq = 0;
    for (int64_t p0 = 0; p0 < N; p0 += 4 * kTkThreads) {
        uint32_t u[4], e = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t p = p0 + 4 * tid + c;
            u[c] = p < N ? score_key(row[p]) : 0u;
            e += (p < N && u[c] == T) ? 1u : 0u;
        }
        uint32_t x[1] = {e}, tx[1];
        block_excl<1>(x, tx, wt);
        bool pick[4];
        uint32_t np = 0, eq = neq + x[0];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t p = p0 + 4 * tid + c;
            const bool isq = p < N && u[c] == T;
            pick[c] = p < N && (u[c] > T || (isq && eq < need));
            eq += isq ? 1u : 0u;
            np += pick[c] ? 1u : 0u;
        }
        uint32_t y[1] = {np}, ty[1];
        block_excl<1>(y, ty, wt);
        uint32_t o = nsel + y[0];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (pick[c]) out[o++] = (int32_t)(p0 + 4 * tid + c);
        nsel += ty[0];
        neq += tx[0];
    }
}

// ---------------------------------------------------------------- launchers
// Workspace layout for n queries whose rows hold ld = Nmax rounded up to whole
// segments: q8 [n][HI][128] | wq [n][HI] | wave extremes [n][ld/256] |
// scores [n][ld] | 16-bit histograms [n][S][2048] | query results [n] |
// segment offsets [n][S] | sure lists [n][k] | candidate keys, indices and
// sure-ranks [n][kTkCandMax] each.
static inline int64_t al256(int64_t x) { return (x + 255) & ~(int64_t)255; }

int64_t index_ws_bytes(const Lay &L, int n, int64_t nmax, IndexWs *w, uint8_t *base, int64_t *scores_off, int64_t *scores_ld) {
    const int64_t ld = (nmax + kTkSeg - 1) / kTkSeg * kTkSeg;
    const int s_max = (int)(ld / kTkSeg);
    const int nwr = (int)(ld / kKeysPerWave);
    int64_t off = 0;
    const int64_t o_q8 = off; off = al256(off + (int64_t)n * L.HI * 128);
    const int64_t o_wq = off; off = al256(off + (int64_t)n * L.HI * 4);
    const int64_t o_wr = off; off = al256(off + (int64_t)n * nwr * 8);
    const int64_t o_sc = off; off = al256(off + (int64_t)n * ld * 4);
    const int64_t o_hi = off; off = al256(off + (int64_t)n * s_max * kTkBins * 2);
    const int64_t o_qm = off; off = al256(off + (int64_t)n * (int64_t)sizeof(TkQuery));
    const int64_t o_sm = off; off = al256(off + (int64_t)n * s_max * 8);
    const int64_t o_su = off; off = al256(off + (int64_t)n * L.topk * 4);
    const int64_t o_ck = off; off = al256(off + (int64_t)n * kTkCandMax * 4);
    const int64_t o_cp = off; off = al256(off + (int64_t)n * kTkCandMax * 4);
    const int64_t o_cr = off; off = al256(off + (int64_t)n * kTkCandMax * 4);
    if (scores_off) *scores_off = o_sc;
    if (scores_ld) *scores_ld = ld;
    if (w) {
        w->q8 = base + o_q8;
        w->wq = (float *)(base + o_wq);
        w->wr = (uint2 *)(base + o_wr);
        w->scores = (float *)(base + o_sc);
        w->hist = (uint16_t *)(base + o_hi);
        w->qm = (TkQuery *)(base + o_qm);
        w->segoff = (int2 *)(base + o_sm);
        w->sure = (int32_t *)(base + o_su);
        w->ckey = (uint32_t *)(base + o_ck);
        w->cpos = (int32_t *)(base + o_cp);
        w->crank = (int32_t *)(base + o_cr);
        w->ld = ld;
        w->nwr = nwr;
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
    const int64_t waves = (rows + kQuantRows - 1) / kQuantRows;
    hipLaunchKernelGGL(k_quant_index_q, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, L, qI, w, rows, ws.q8, ws.wq);
    return hipGetLastError();
}

hipError_t launch_score_decode(const Lay &L, const dsv4_cache &C, const void *qI, const float *w,
                               const int32_t *req, const int32_t *pos, int n, const IndexWs &ws, hipStream_t s) {
    dim3 g((unsigned)((ws.ld + kKeysPerWG - 1) / kKeysPerWG), n);
    const int hb = (L.HI + 15) / 16;
    const bool full = L.dI == 128;
#define DSV4_SCORE(HBV, FV, F4V) \
    hipLaunchKernelGGL((k_index_score_decode<HBV, FV, F4V>), g, dim3(256), 0, s, L, C, qI, w, req, pos, ws.scores, \
                       ws.ld, ws.wr, ws.nwr)
#define DSV4_SCORE_HB(FV, F4V)                \
    do {                                      \
        if (hb == 4) DSV4_SCORE(4, FV, F4V);  \
        else if (hb == 3) DSV4_SCORE(3, FV, F4V); \
        else if (hb == 2) DSV4_SCORE(2, FV, F4V); \
        else DSV4_SCORE(1, FV, F4V);          \
    } while (0)
    if (L.idx_store == DSV4_STORE_MXFP4) {
        if (full) DSV4_SCORE_HB(true, true);
        else DSV4_SCORE_HB(false, true);
    } else {
        if (full) DSV4_SCORE_HB(true, false);
        else DSV4_SCORE_HB(false, false);
    }
#undef DSV4_SCORE_HB
#undef DSV4_SCORE
    return hipGetLastError();
}

hipError_t launch_score_f32(const Lay &L, const dsv4_cache &C, const void *qI, const float *w, const int32_t *req,
                            const int32_t *pos, int n, const IndexWs &ws, hipStream_t s) {
    hipLaunchKernelGGL(k_index_score_f32, dim3((unsigned)(ws.nwr / 4), n), dim3(256), 0, s, L, C, qI, w, req, pos,
                       ws.scores, ws.ld, ws.wr, ws.nwr);
    return hipGetLastError();
}

hipError_t launch_score_prefill(const Lay &L, const dsv4_cache &C, const int32_t *req, const int32_t *pos,
                                int n, const IndexWs &ws, hipStream_t s) {
    dim3 g((unsigned)((ws.ld + kPfKeys - 1) / kPfKeys), (unsigned)((n + kPfRows - 1) / kPfRows));
    const int hb = (L.HI + 15) / 16;
    const bool full = L.dI == 128;
    const size_t dyn = (size_t)score_prefill_dyn_lds(L);
#define DSV4_SCORE(HBV, FV, F4V) \
    hipLaunchKernelGGL((k_index_score_prefill<HBV, FV, F4V>), g, dim3(256), dyn, s, L, C, ws.q8, ws.wq, req, pos, n, \
                       ws.scores, ws.ld, ws.wr, ws.nwr)
#define DSV4_SCORE_HB(FV, F4V)                \
    do {                                      \
        if (hb == 4) DSV4_SCORE(4, FV, F4V);  \
        else if (hb == 3) DSV4_SCORE(3, FV, F4V); \
        else if (hb == 2) DSV4_SCORE(2, FV, F4V); \
        else DSV4_SCORE(1, FV, F4V);          \
    } while (0)
    if (L.idx_store == DSV4_STORE_MXFP4) {
        if (full) DSV4_SCORE_HB(true, true);
        else DSV4_SCORE_HB(false, true);
    } else {
        if (full) DSV4_SCORE_HB(true, false);
        else DSV4_SCORE_HB(false, false);
    }
#undef DSV4_SCORE_HB
#undef DSV4_SCORE
    return hipGetLastError();
}

// n <= 65535 (grid y).  With no segments (empty rows) only the final pass
// runs: it writes the padding.
static void launch_tk_passes(const TkArgs &A, int n, hipStream_t s) {
    const IndexWs &ws = A.ws;
    if (ws.s_max > 0) {
        hipLaunchKernelGGL(k_tk_hist, dim3(ws.s_max, n), dim3(kTkThreads), 0, s, A);
        if (ws.s_max <= kTkFuseSeg) {
            hipLaunchKernelGGL(k_tk_split<true>, dim3(ws.s_max, n), dim3(kTkThreads), 0, s, A);
        } else {
            hipLaunchKernelGGL(k_tk_bin, dim3(n), dim3(kTkThreads), 0, s, A);
            hipLaunchKernelGGL(k_tk_split<false>, dim3(ws.s_max, n), dim3(kTkThreads), 0, s, A);
        }
    }
    hipLaunchKernelGGL(k_tk_final, dim3(n), dim3(kTkThreads), 0, s, A);
}

hipError_t launch_topk(const Lay &L, const dsv4_cache &C, const int32_t *req, const int32_t *pos, int n,
                       const IndexWs &ws, int32_t *out, hipStream_t s) {
    const TkArgs A{L, req, pos, C.n_req, (int64_t)C.max_blocks * kBlockTokens, ws, out, nullptr, 0};
    launch_tk_passes(A, n, s);
    return hipGetLastError();
}

hipError_t launch_topk_rows(const float *scores, int64_t ld, const int32_t *nvis, int n, int64_t max_n, int k,
                            const IndexWs &ws, int32_t *out, hipStream_t s) {
    Lay L;
    memset(&L, 0, sizeof(L));
    L.topk = k;
    L.m = 1;
    const TkArgs A{L, nullptr, nullptr, 0, 0, ws, out, nvis, max_n};
    if (max_n > 0) {
        hipError_t e = hipMemcpy2DAsync(ws.scores, (size_t)ws.ld * 4, scores, (size_t)ld * 4, (size_t)max_n * 4,
                                        n, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_tk_extremes, dim3((unsigned)(ws.nwr / 4), n), dim3(256), 0, s, A);
    }
    launch_tk_passes(A, n, s);
    return hipGetLastError();
}

}  // namespace dsv4
