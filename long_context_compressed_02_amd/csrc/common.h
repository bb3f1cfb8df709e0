// common.h -- internal layout and device helpers of libdsv4attn (gfx950).
// Not part of the public ABI (include/dsv4attn.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4attn.h"

namespace dsv4 {

constexpr int kBlockTokens = DSV4_BLOCK_TOKENS;  // raw tokens per classic-cache block

// Everything a kernel needs to address one layer's cache; built on the host
// from (cfg, kind) and passed by value.
struct Lay {
    int kind;
    int d, dr, dn;          // head dim, RoPE dims (the last dr), non-RoPE dims
    int H, W;               // query heads, raw window
    int m, wc;              // stride and compression window of this layer's compressor
    int epb;                // entries per 128-token block
    int rec_bytes;          // stored KV record stride
    int rope_off;           // FP8 mode: byte offset of the bf16 RoPE dims
    int scale_off;          // FP8 mode: byte offset of the fp32 scale
    int64_t entry_block_bytes;
    int HI, dI;             // indexer heads and dim (CSA)
    int key_bytes;          // one stored index key
    int key_scale_off;      // FP8 index keys: offset of the scales inside a block
    int64_t index_block_bytes;
    int64_t state_bytes;
    int64_t pend_off;       // state: byte offset of the pending ring
    int pend_slots;         // pending ring slots (= wc)
    int pend_tok_floats;    // floats per pending token: kv d, gate d (+ kI dI, gI dI)
    int topk;
    int kv_store, idx_store, act;
    float rope_base, tau;
    double theta[64];       // RoPE frequencies base^(-2i/dr), i < dr/2 (fp64, from the host)
};

// Host: validate a configuration and derive the layout.
dsv4_status make_layout(const dsv4_cfg *cfg, int32_t kind, Lay *out);

// ------------------------------------------------------------------ numerics
// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> OCP E4M3 code, round to nearest even, saturating at +-448 (the
// hardware conversion rounds to nearest even; inputs are clamped first so it
// never sees an out-of-range value).
__device__ __forceinline__ uint32_t fp8_code(float y) {
    if (y != y) return 0x7fu;
    y = fminf(fmaxf(y, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xffu;
}

// OCP MXFP4 (indexer rows): blocks of 32 consecutive values share a
// power-of-two scale 2^x stored as an E8M0 byte x + 127; each value is an
// E2M1 code (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6).
//
// Nearest E2M1 code of y, ties to the even mantissa bit, saturating to +-6:
// inside binade [2^u, 2^(u+1)) (u = 0, 1, 2) the step is 2^(u-1), and below 1
// the step 0.5 of the first binade continues down to 0.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
    const uint32_t s = (__float_as_uint(y) >> 28) & 8u;
    const float a = fabsf(y);
    if (!(a < 6.0f)) return s | 7u;
    const int u = a >= 1.0f ? (int)(__float_as_uint(a) >> 23) - 127 : 0;
    const float q = __builtin_rintf(__builtin_ldexpf(a, 1 - u));   // a / step, exact scaling
    return s | (uint32_t)(2 * u + (int)q);
}

// Shared exponent of a block whose largest magnitude is amax: floor(log2 amax)
// - 2 (2: the exponent of E2M1's largest magnitude, so the block's largest
// value scales into [4, 8)), clamped to the E8M0 range; -127 for a block of
// zeros (and for amax below the smallest normal fp32, where the rule gives
// less than -127 anyway).
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax >= 1.17549435e-38f)) return -127;
    const int x = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 2;
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// One MXFP4 row of at most 128 values held by a wave, two per lane (lane l:
// values 2l and 2l+1; v0, v1 say which are real): the 16 lanes of a DPP row
// hold one 32-value block.  Returns the lane's code byte (value 2l in the low
// nibble); *scales receives the four E8M0 bytes, block b in byte b (blocks
// without real values get byte 0 and all-zero codes).
__device__ __forceinline__ uint32_t mx4_row(float x0, float x1, bool v0, bool v1, uint32_t *scales) {
    float am = fmaxf(v0 ? fabsf(x0) : 0.0f, v1 ? fabsf(x1) : 0.0f);
    const int zero = 0;
    am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(zero, __float_as_int(am), 0x111, 0xf, 0xf, false)));
    am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(zero, __float_as_int(am), 0x112, 0xf, 0xf, false)));
    am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(zero, __float_as_int(am), 0x114, 0xf, 0xf, false)));
    am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(zero, __float_as_int(am), 0x118, 0xf, 0xf, false)));
    // lane 16b+15 now holds block b's largest magnitude
    uint32_t sc = 0, mine = 0;
    const int row = (int)(threadIdx.x & 63) >> 4;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int xb = mx_exponent(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 16 * b + 15)));
        sc |= (uint32_t)(xb + 127) << (8 * b);
        mine = b == row ? (uint32_t)(xb + 127) : mine;
    }
    const int x = (int)mine - 127;
    const uint32_t c0 = v0 ? e2m1_code(__builtin_ldexpf(x0, -x)) : 0u;
    const uint32_t c1 = v1 ? e2m1_code(__builtin_ldexpf(x1, -x)) : 0u;
    *scales = sc;
    return c0 | (c1 << 4);
}

// Activation loads/stores in the configured dtype.
__device__ __forceinline__ float load_act(const void *p, int64_t i, int act) {
    if (act == DSV4_DT_BF16) return bf16_to_f32(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

// cos/sin of the RoPE angle pos * theta_i.  The angle is formed and reduced
// modulo 2*pi in fp64 (Cody-Waite with 2*pi split into three parts whose
// products with the quotient are exact for positions below 2^26), so large
// positions keep full accuracy; the reduced angle's sine and cosine are then
// taken in fp32.
__device__ __forceinline__ void rope_cs_theta(double theta, int64_t pos, float &c, float &s) {
    const double ang = (double)pos * theta;
    const double kq = rint(ang * 0.15915494309189535);          // 1 / (2*pi)
    double r = __fma_rn(-kq, 6.28318530717958623200e+00, ang);  // 2*pi, split in three parts
    r = __fma_rn(-kq, 2.44929359829470641e-16, r);
    r = __fma_rn(-kq, -5.97232958240207e-33, r);
    sincosf((float)r, &s, &c);
}
__device__ __forceinline__ void rope_cs(const Lay &L, int64_t pos, int i, float &c, float &s) {
    rope_cs_theta(L.theta[i], pos, c, s);
}
// theta_l for lane l < n of the wave, read from the argument block with
// uniform (scalar) loads and written into each lane with v_writelane: a
// per-lane indexed read is a vector load, and the wait for it also waits for
// every vector load issued before it (a select chain over the n values, the
// earlier form, was folded back into that load by the compiler or, with the
// values forced uniform, held enough registers to spill).
__device__ __forceinline__ double theta_lane(const Lay &L, int n) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 64; ++k) {
        if (k >= n) break;
        const uint64_t b = (uint64_t)__double_as_longlong(L.theta[k]);
        const uint32_t blo = (uint32_t)b, bhi = (uint32_t)(b >> 32);
        // (register moves only: v_writelane_b32 takes a scalar source and a constant lane)
        asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(lo) : "s"(blo), "i"(k));
        asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(hi) : "s"(bhi), "i"(k));
    }
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Wave-wide max over the 64 lanes, returned to every lane.  Max is exact and
// ignores NaN operands whatever the order, so any reduction tree gives the same
// value; this one runs on the DPP cross-lane paths (no LDS round trips):
// within rows of 16 lanes by shifts of 1, 2, 4, 8, then across rows.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float x) {
    const int ninf = (int)0xff800000u;
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), CTRL, ROW_MASK, 0xf, false)));
}
__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max_step<0x111, 0xf>(v);   // row_shr:1
    v = dpp_max_step<0x112, 0xf>(v);   // row_shr:2
    v = dpp_max_step<0x114, 0xf>(v);   // row_shr:4
    v = dpp_max_step<0x118, 0xf>(v);   // row_shr:8
    v = dpp_max_step<0x142, 0xa>(v);   // row_bcast:15
    v = dpp_max_step<0x143, 0xc>(v);   // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ------------------------------------------------------------------ cache addressing
__device__ __forceinline__ int64_t block_id(const int32_t *bt, int max_blocks, int n_blocks, int r,
                                            int64_t blk) {
    if (blk < 0 || blk >= max_blocks) return -1;
    int b = bt[(int64_t)r * max_blocks + blk];
    return (b >= 0 && b < n_blocks) ? b : -1;
}

// Per-channel gated pooling of one compressor window: softmax over the
// window's tokens of the gate logits, weighted sum of the values.  `get(s, &kv,
// &g)` returns token s of the window (s = 0 .. n-1 in position order).  The
// same operation sequence is used by the decode and prefill paths, so a
// prefilled entry is bitwise equal to one built token by token.
template <typename Get>
__device__ __forceinline__ float pool_channel(int n, Get get) {
    float mx = -INFINITY;
    for (int s = 0; s < n; ++s) {
        float v, g;
        get(s, v, g);
        mx = fmaxf(mx, g);
    }
    float den = 0.0f, num = 0.0f;
    for (int s = 0; s < n; ++s) {
        float v, g;
        get(s, v, g);
        float a = expf(g - mx);
        den = den + a;
        num = num + a * v;
    }
    return num / den;
}

}  // namespace dsv4
