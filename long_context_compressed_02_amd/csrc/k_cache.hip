// k_cache.hip -- dump and reload of one request's cache (vastsailsolution.com
// V4 article, paragraph on the state cache and the classic cache;
// xiaoyuzhoufm.com summary 2.1: an on-disk KV cache for requests that share a
// prefix, with full-cache, periodic-checkpoint and recompute strategies).
//
// A request's cache after n tokens is its state cache (window ring and
// pending ring) plus the classic-cache blocks that cover tokens [0, n): the
// entries, and for a CSA layer the index keys.  The dump is those bytes in a
// fixed order -- state, then the entry blocks in token order, then the index
// blocks -- independent of where the blocks sit in the pool; a reload writes
// them into another request's blocks through its own block table.  Every
// stored byte is copied as it is, so a reloaded prefix continues bit for bit
// like the original.
#include "launch.h"

namespace dsv4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One thread per 16-byte piece of the dump; to_buf: cache -> buffer (else the
// reverse).  Pieces of a block the table does not map read as zeros (dump) or
// are skipped (reload).
__global__ __launch_bounds__(256) void k_cache_xfer(Lay L, dsv4_cache C, int r, int nb, uint8_t *buf,
                                                    int64_t total, int to_buf) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t off = 16 * i;
    uint8_t *c = nullptr;
    if (off < L.state_bytes) {
        c = (uint8_t *)C.state + (int64_t)r * L.state_bytes + off;
    } else {
        int64_t o2 = off - L.state_bytes;
        const int64_t eb = L.entry_block_bytes, ib = L.index_block_bytes;
        int64_t bytes_per = eb;
        uint8_t *pool = (uint8_t *)C.entries;
        if (o2 >= nb * eb) {                                 // index blocks (CSA)
            o2 -= nb * eb;
            bytes_per = ib;
            pool = (uint8_t *)C.index_keys;
        }
        const int b = (int)(o2 / bytes_per);
        const int64_t bid = block_id(C.block_table, C.max_blocks, C.n_blocks, r, b);
        if (bid >= 0) c = pool + bid * bytes_per + o2 % bytes_per;
    }
    u32x4 *bp = (u32x4 *)(buf + off);
    if (to_buf) *bp = c ? *(const u32x4 *)c : (u32x4){0u, 0u, 0u, 0u};
    else if (c) *(u32x4 *)c = *bp;
}

// ---------------------------------------------------------------- read-back
// Value of an OCP E4M3 code (bias 7; exponent 0 subnormal: m/8 * 2^-6;
// S.1111.111 NaN) and of an E2M1 code (bias 1; magnitudes 0, 0.5 .. 6).
// Both are exact in fp64 (and in fp32).
__device__ __forceinline__ double e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    double v;
    if (e == 15u && m == 7u) v = __builtin_nan("");
    else if (e == 0u) v = __builtin_ldexp((double)m, -9);
    else v = __builtin_ldexp((double)(8u + m), (int)e - 10);
    return (c & 0x80u) ? -v : v;
}
__device__ __forceinline__ double e2m1_value(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const double v = e == 0u ? 0.5 * (double)m : __builtin_ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return (c & 8u) ? -v : v;
}

// One thread per value: item i, dim c of the stored vector the target names
// (entry, index key, or window-ring record of a position), decoded from its
// storage format in fp64 (exact: a code's value has at most 4 significant
// bits, its fp32 scale 24) and written as fp64 or rounded to fp32.  Items
// whose request, index or block is out of range are skipped.
__global__ __launch_bounds__(256) void k_read_entries(Lay L, dsv4_cache C, int target, const int32_t *req,
                                                      const int32_t *idx, int n, void *out, int f64) {
    const int dim = target == DSV4_TARGET_INDEX_KEY ? L.dI : L.d;
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gi >= (int64_t)n * dim) return;
    const int64_t it = gi / dim;
    const int c = (int)(gi % dim);
    const int r = req[it];
    const int64_t j = idx[it];
    if (r < 0 || r >= C.n_req || j < 0 || j >= (int64_t)C.max_blocks * kBlockTokens) return;
    double v;
    if (target == DSV4_TARGET_INDEX_KEY) {
        const int64_t bid = block_id(C.block_table, C.max_blocks, C.n_blocks, r, (j * L.m) / kBlockTokens);
        if (bid < 0) return;
        const uint8_t *blk = (const uint8_t *)C.index_keys + bid * L.index_block_bytes;
        const int slot = (int)(j % L.epb);
        const uint8_t *key = blk + (int64_t)slot * L.key_bytes;
        if (L.idx_store == DSV4_STORE_FP32) {
            v = ((const float *)key)[c];
        } else if (L.idx_store == DSV4_STORE_MXFP4) {
            const uint32_t code = (key[c >> 1] >> (4 * (c & 1))) & 15u;
            const uint32_t word = ((const uint32_t *)(blk + L.key_scale_off))[slot];
            const int x = (int)((word >> (8 * (c >> 5))) & 0xffu) - 127;
            v = __builtin_ldexp(e2m1_value(code), x);
        } else {
            v = e4m3_value(key[c]) * (double)((const float *)(blk + L.key_scale_off))[slot];
        }
    } else {
        const uint8_t *rec;
        if (target == DSV4_TARGET_WINDOW) {
            if (L.W <= 0) return;
            rec = (const uint8_t *)C.state + (int64_t)r * L.state_bytes + (j % L.W) * L.rec_bytes;
        } else {
            const int64_t bid = block_id(C.block_table, C.max_blocks, C.n_blocks, r, (j * L.m) / kBlockTokens);
            if (bid < 0) return;
            rec = (const uint8_t *)C.entries + bid * L.entry_block_bytes + (j % L.epb) * L.rec_bytes;
        }
        if (L.kv_store == DSV4_STORE_FP32) v = ((const float *)rec)[c];
        else if (c < L.dn) v = e4m3_value(rec[c]) * (double)*(const float *)(rec + L.scale_off);
        else v = bf16_to_f32(((const uint16_t *)(rec + L.rope_off))[c - L.dn]);
    }
    if (f64) ((double *)out)[gi] = v;
    else ((float *)out)[gi] = (float)v;
}

hipError_t launch_read_entries(const Lay &L, const dsv4_cache &C, int target, const int32_t *req, const int32_t *idx,
                               int n, void *out, bool f64, hipStream_t s) {
    const int dim = target == DSV4_TARGET_INDEX_KEY ? L.dI : L.d;
    const int64_t total = (int64_t)n * dim;
    hipLaunchKernelGGL(k_read_entries, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, L, C, target, req, idx,
                       n, out, f64 ? 1 : 0);
    return hipGetLastError();
}

int64_t cache_dump_bytes(const Lay &L, int nb) {
    return L.state_bytes + (int64_t)nb * (L.entry_block_bytes + L.index_block_bytes);
}

hipError_t launch_cache_xfer(const Lay &L, const dsv4_cache &C, int r, int nb, uint8_t *buf, bool to_buf,
                             hipStream_t s) {
    const int64_t total = cache_dump_bytes(L, nb) / 16;
    hipLaunchKernelGGL(k_cache_xfer, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, L, C, r, nb, buf, total,
                       to_buf ? 1 : 0);
    return hipGetLastError();
}

}  // namespace dsv4
