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
