// k_mx.hip -- linear layers of the indexer's low-precision path for gfx950.
//
// What is computed (vastsailsolution.com V4 article, CSA section: the
// indexer's query is first projected down to d_c = 1024 dims, then up to the
// multi-head index queries; rqlyzj.com article, FP4 QAT section, and
// xiaoyuzhoufm.com summary 2.1: the indexer runs in FP4): out = x . W^T with
//   W [N][K]  weights, stored once as MXFP4 (E2M1 values, one E8M0 power-of-two
//             scale per 32 consecutive k: exponent floor(log2 amax) - 2);
//   x [M][K]  bf16 activations, quantised on the way in to MXFP8 (E4M3 values,
//             one scale per 32 k: exponent floor(log2 amax) - 8);
// summed in fp32 by v_mfma_scale_f32_16x16x128_f8f6f4 (A = FP8, B = FP4, the
// scales applied by the instruction per lane).
//
// Operand order of a 16x16x128 step (measured with a probe on gfx950, every
// other candidate order failing): lane l (g = l/16, c = l%16) supplies
//   B (FP4): row c's k = 32g .. 32g+31, 16 bytes, value 2i in the low nibble
//            of byte i;
//   A (FP8): row c's k = 16g .. 16g+15 in bytes 0..15 and k = 64+16g ..
//            64+16g+15 in bytes 16..31;
//   scales:  one byte per operand, the scale of row c's k-block g (k = 32g ..
//            32g+31), wherever those values sit in the registers.
// So a B lane holds exactly its own MX block, while an A block spreads over two
// lanes: block g's first 16 values go to lane group 2(g%2), its last 16 to
// lane group 2(g%2)+1, in the half g/2 of their 32 bytes.  Both operands are
// written in register order, so every load is a contiguous kilobyte per wave:
//   codes   tile (16-row block, 128-wide k-step): FP8: two 1 KB halves, half h
//           holding bytes 16h .. 16h+15 of each lane at 16l; FP4: one 1 KB
//           piece, lane l's 16 bytes at 16l
//   scales  per (16-row block, group of four k-steps): 64 lanes x 4 bytes,
//           byte j = lane l's scale for k-step 4q+j (0x7f past the last step)
// Rows are padded to a multiple of 16 with zeros (scale byte 0, codes 0).
//
// Batch invariance (m.youleyou.com article, "what was sacrificed": no split-K):
// one wave reduces each output over k in increasing order with the same
// instruction whatever the tiling, so a row's output is bitwise the same in any
// batch.
#include "launch.h"

namespace dsv4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

int64_t mx_pack_bytes(int rows, int K, bool fp8) {
    const int64_t rb = (rows + 15) / 16, nks = K / 128, nq = (nks + 3) / 4;
    return rb * nks * (fp8 ? 2048 : 1024) + rb * nq * 256;
}
__host__ __device__ static inline int64_t mx_code_bytes(int rows, int K, bool fp8) {
    return (int64_t)((rows + 15) / 16) * (K / 128) * (fp8 ? 2048 : 1024);
}

// MXFP8 shared exponent: floor(log2 amax) - 8 (8: the exponent of E4M3's
// largest value 448, so the block's largest magnitude scales into [256, 512)
// and saturates to 448 above it), clamped to the E8M0 range; -127 for a block
// of zeros or below the smallest normal fp32.
__device__ __forceinline__ int mx8_exponent(float amax) {
    if (!(amax >= 1.17549435e-38f)) return -127;
    const int x = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 8;
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// One thread per (16-row block, group of four k-steps, lane (g, c)):
// quantises row c's block g (k = 32g .. 32g+31) of each of the four k-steps,
// writes the codes where the operand order puts them and the lane's scale word.
// STEP1 (small inputs): one thread per (16-row block, k-step, lane) instead,
// writing its scale byte alone -- four times the threads, one memory round
// trip each (the threads of the padding k-steps of the last group write 0x7f).
template <bool F8, bool STEP1>
__global__ __launch_bounds__(256) void k_mx_quant(const uint16_t *X, int rows, int K, uint8_t *P, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int lane = (int)(i & 63), g = lane >> 4;
    const int nks = K / 128, nq = (nks + 3) / 4;
    const int64_t t = i >> 6;
    const int kq = STEP1 ? (int)(t % (4 * nq)) / 4 : (int)(t % nq);
    const int64_t rb = STEP1 ? t / (4 * nq) : t / nq;
    const int64_t row = rb * 16 + (lane & 15);
    const bool live = row < rows;
    uint8_t *scales = P + mx_code_bytes(rows, K, F8);
    uint32_t sw = 0x7f7f7f7fu;
    const int j_lo = STEP1 ? (int)(t % 4) : 0, j_hi = STEP1 ? j_lo + 1 : 4;
#pragma unroll 1
    for (int j = j_lo; j < j_hi; ++j) {
        const int ks = 4 * kq + j;
        if (ks >= nks) break;
        u32x4 raw[4] = {};
        if (live) {
            const u32x4 *src = (const u32x4 *)(X + row * K + 128 * ks + 32 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) raw[v] = src[v];
        }
        float x[32];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                x[8 * v + 2 * w] = __uint_as_float(raw[v][w] << 16);
                x[8 * v + 2 * w + 1] = __uint_as_float(raw[v][w] & 0xffff0000u);
            }
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < 32; ++v) amax = fmaxf(amax, fabsf(x[v]));
        const int e = F8 ? mx8_exponent(amax) : mx_exponent(amax);
        sw = (sw & ~(0xffu << (8 * j))) | ((uint32_t)(e + 127) << (8 * j));
        if constexpr (F8) {
            u32x4 c[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t word = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        word |= fp8_code(__builtin_ldexpf(x[16 * h + 4 * w + b], -e)) << (8 * b);
                    c[h][w] = word;
                }
            // first 16 values -> lane group 2(g%2), last 16 -> 2(g%2)+1, half g/2
            const int l0 = 16 * (2 * (g & 1)) + (lane & 15);
            uint8_t *dst = P + ((rb * nks + ks) * 2 + (g >> 1)) * 1024;
            *(u32x4 *)(dst + 16 * l0) = c[0];
            *(u32x4 *)(dst + 16 * (l0 + 16)) = c[1];
        } else {
            u32x4 c;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t word = 0;
#pragma unroll
                for (int b = 0; b < 8; ++b) word |= e2m1_code(__builtin_ldexpf(x[8 * w + b], -e)) << (4 * b);
                c[w] = word;
            }
            *(u32x4 *)(P + (rb * nks + ks) * 1024 + 16 * lane) = c;
        }
    }
    if constexpr (STEP1)
        scales[(rb * nq + kq) * 256 + 4 * lane + j_lo] = (uint8_t)(sw >> (8 * j_lo));
    else
        ((uint32_t *)(scales + (rb * nq + kq) * 256))[lane] = sw;
}

struct MxArgs {
    const uint8_t *A;       // MXFP8 activations, packed (rows padded to 16)
    const uint8_t *B;       // MXFP4 weights, packed
    void *C;                // [M][ldc] fp32 or bf16
    int64_t a_scale_off, b_scale_off;
    int64_t ldc;
    int M, N, K;
    int c_f32;
    int tiles_x, tiles_y;   // column / row tiles
    int chunk_w;            // column tiles per chunk of the tile order
};

// Workgroup -> tile.  Workgroups are dealt to the 8 XCDs in turn (id % 8), and
// each XCD has its own L2 (4 MB).  The tiles are ordered in column chunks --
// chunk_w column tiles, whose weights fit one L2 -- and row-major inside a
// chunk; XCD x takes the x-th run of consecutive tiles in that order.  So the
// workgroups sharing an L2 sweep a chunk's column tiles over a few row tiles:
// each row tile's activations are fetched into one L2 per chunk, and the
// chunk's weights stay resident there.
__device__ __forceinline__ bool mx_tile(const MxArgs &G, int id, int &ty, int &tx) {
    const int tiles = G.tiles_x * G.tiles_y;
    const int per = (tiles + 7) / 8;
    const int t = (id % 8) * per + id / 8;
    if (t >= tiles) return false;
    const int chunk = t / (G.chunk_w * G.tiles_y);
    const int r = t - chunk * G.chunk_w * G.tiles_y;
    const int w = min(G.chunk_w, G.tiles_x - chunk * G.chunk_w);   // the last chunk may be narrower
    ty = r / w;
    tx = chunk * G.chunk_w + r % w;
    return true;
}

// WM x WN 16x16 blocks per wave, WGM x WGN waves per workgroup (4 in all), D
// k-steps of loads in flight.
template <int WM, int WN, int WGM, int WGN, int D>
__global__ __launch_bounds__(256) void k_mx_gemm(MxArgs G) {
    static_assert(WGM * WGN == 4, "four waves");
    int ty, tx;
    if (!mx_tile(G, blockIdx.x, ty, tx)) return;      // (whole workgroup: the grid is rounded up to 8)
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int nks = G.K / 128, nq = (nks + 3) / 4;
    const int rbs = (G.M + 15) / 16, cbs = G.N / 16;
    const int rb0 = ty * (WGM * WM) + wm * WM;
    const int cb0 = tx * (WGN * WN) + wn * WN;
    // blocks past the matrix read the last one (their results are not stored)
    const uint8_t *ap[WM];
    const uint8_t *bp[WN];
    const uint32_t *asp[WM];
    const uint32_t *bsp[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
        const int64_t rb = rb0 + i < rbs ? rb0 + i : rbs - 1;
        ap[i] = G.A + rb * nks * 2048 + 16 * lane;
        asp[i] = (const uint32_t *)(G.A + G.a_scale_off + rb * nq * 256) + lane;
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
        const int64_t cb = cb0 + j < cbs ? cb0 + j : cbs - 1;
        bp[j] = G.B + cb * nks * 1024 + 16 * lane;
        bsp[j] = (const uint32_t *)(G.B + G.b_scale_off + cb * nq * 256) + lane;
    }
    f32x4 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    i32x4 ra[D][WM][2], rbv[D][WN];
    uint32_t sa[D][WM], sb[D][WN];
    // step s's loads; steps past the end re-read the last step (never used), so
    // every ring slot is refilled on every path and the counter waits stay exact
    auto load = [&](int slot, int s) {
        const int sc = s < nks ? s : nks - 1;
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            ra[slot][i][0] = *(const i32x4 *)(ap[i] + (int64_t)2048 * sc);
            ra[slot][i][1] = *(const i32x4 *)(ap[i] + (int64_t)2048 * sc + 1024);
            sa[slot][i] = asp[i][64 * (sc >> 2)];
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            rbv[slot][j] = *(const i32x4 *)(bp[j] + (int64_t)1024 * sc);
            sb[slot][j] = bsp[j][64 * (sc >> 2)];
        }
    };
    const i32x4 z4 = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, s);
#pragma unroll 1
    for (int s0 = 0; s0 < nks; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int s = s0 + d;
            if (s < nks) {                               // (uniform)
                const int sh = 8 * (s & 3);
#pragma unroll
                for (int i = 0; i < WM; ++i) {
                    i32x8 a;
                    a.lo = ra[d][i][0];
                    a.hi = ra[d][i][1];
#pragma unroll
                    for (int j = 0; j < WN; ++j) {
                        i32x8 b;
                        b.lo = rbv[d][j];
                        b.hi = z4;
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a, b, acc[i][j], 0, 4, 0, (int)(sa[d][i] >> sh), 0, (int)(sb[d][j] >> sh));
                    }
                }
            }
            load(d, s + D);
        }
    }
    // lane (g, c16) holds rows 4g+e, column c16 of each 16x16 block
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int col = 16 * (cb0 + j) + c16;
            if (cb0 + j >= cbs) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * (rb0 + i) + 4 * g + e;
                if (row >= G.M) continue;
                const int64_t off = (int64_t)row * G.ldc + col;
                if (G.c_f32) ((float *)G.C)[off] = acc[i][j][e];
                else ((uint16_t *)G.C)[off] = bf16_bits(acc[i][j][e]);
            }
        }
}

// Large inputs with LDS-staged tiles: a workgroup of 8 waves owns a tile of
// 16 row blocks x CB column blocks (256x256 or, where that leaves compute
// units idle, 256x128), wave (wm, wn) 64 x 8 CB of it (4 x CB/2 blocks).  Per
// k-step all 512 threads copy the tile's operands into one of two LDS stages
// in the packed order (A codes 32 KB, B codes CB KB, the 64 scale words of
// each block), so the copy's stores and the waves' reads are 64 consecutive
// slots; the next k-step's loads are in flight in registers while the current
// one is multiplied.  Each output is still one wave's chain over
// the k-steps in increasing order with the same instruction: bitwise the other
// tilings' result.  Tiles go to the XCDs in contiguous runs, four row tiles
// at a time column by column.
constexpr int kMxLdsRows = 256;                                   // rows of a tile
constexpr int kMxLdsA = 16 * 2048;
template <int CB>
struct MxLds {
    static constexpr int B = CB * 1024, S = (16 + CB) * 256;       // B codes, A and B scale words
    static constexpr int STAGE = kMxLdsA + B + S;
    static constexpr int BYTES = 2 * STAGE;
    static constexpr int NB = CB * 64 / 512;                       // B pieces a thread copies
    static_assert(CB == 8 || CB == 16, "two tile widths");
};

template <int CB>
__global__ __launch_bounds__(512) void k_mx_gemm_lds(MxArgs G, int per) {
    using Ly = MxLds<CB>;
    constexpr int WJ = CB / 2;                                     // column blocks a wave owns
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;                       // 4 x 2 waves
    const int nx = G.tiles_x, ny = G.tiles_y;
    const int T = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (T >= nx * ny) return;
    const int gsz = 4 * nx, fr = (T / gsz) * 4;
    const int rows = ny - fr < 4 ? ny - fr : 4;
    const int ty = fr + (T % gsz) % rows, tx = (T % gsz) / rows;
    const int nks = G.K / 128, nq = (nks + 3) / 4;
    const int rbs = (G.M + 15) / 16;
    const int rb0 = ty * 16, cb0 = tx * CB;
    // the copy: A pieces p = t + 512 u (u < 4) -- block p / 128, 16 bytes at
    // 16 (p mod 128) of its 2 KB; B pieces p = t + 512 u (u < 2) -- block p / 64;
    // scale piece t: 16 bytes of the A (t < 256) or B block's 256-byte word row
    const uint8_t *ga[4];
    const uint8_t *gb[Ly::NB];
    const uint8_t *gs;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int pc = tid + 512 * u;
        const int64_t rb = rb0 + (pc >> 7) < rbs ? rb0 + (pc >> 7) : rbs - 1;   // (past the rows: the last block)
        ga[u] = G.A + rb * nks * 2048 + 16 * (pc & 127);
    }
#pragma unroll
    for (int u = 0; u < Ly::NB; ++u) {
        const int pc = tid + 512 * u;
        gb[u] = G.B + (int64_t)(cb0 + (pc >> 6)) * nks * 1024 + 16 * (pc & 63);
    }
    // scale piece t < 16 (16 + CB): 16 bytes of an A (block t / 16 < 16) or a
    // B block's word row; the other threads copy none
    const bool scopy = tid < 16 * (16 + CB);
    {
        const int blk = tid >> 4, off = 16 * (tid & 15);
        if (blk < 16) {
            const int64_t rb = rb0 + blk < rbs ? rb0 + blk : rbs - 1;
            gs = G.A + G.a_scale_off + rb * nq * 256 + off;
        } else {
            const int cb = scopy ? cb0 + blk - 16 : cb0;
            gs = G.B + G.b_scale_off + (int64_t)cb * nq * 256 + off;
        }
    }
    u32x4 ra[4], rbv[Ly::NB], rs;
    auto fetch = [&](int ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) ra[u] = *(const u32x4 *)(ga[u] + (int64_t)2048 * ks);
#pragma unroll
        for (int u = 0; u < Ly::NB; ++u) rbv[u] = *(const u32x4 *)(gb[u] + (int64_t)1024 * ks);
        rs = *(const u32x4 *)(gs + (int64_t)256 * (ks >> 2));       // (every thread: in bounds)
    };
    auto stash = [&](int st) {
        uint8_t *sp = smem + st * Ly::STAGE;
#pragma unroll
        for (int u = 0; u < 4; ++u) *(u32x4 *)(sp + 16 * (tid + 512 * u)) = ra[u];
#pragma unroll
        for (int u = 0; u < Ly::NB; ++u) *(u32x4 *)(sp + kMxLdsA + 16 * (tid + 512 * u)) = rbv[u];
        if (scopy) *(u32x4 *)(sp + kMxLdsA + Ly::B + 16 * tid) = rs;   // A words, then B words
    };
    f32x4 acc[4][WJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    const i32x4 z4 = {0, 0, 0, 0};
    fetch(0);
    stash(0);
    __syncthreads();
#pragma unroll 1
    for (int ks = 0; ks < nks; ++ks) {
        if (ks + 1 < nks) fetch(ks + 1);                           // (uniform)
        const uint8_t *sp = smem + (ks & 1) * Ly::STAGE;
        const uint32_t *sws = (const uint32_t *)(sp + kMxLdsA + Ly::B);
        const int sh = 8 * (ks & 3);
        i32x4 fb[WJ];
        uint32_t sb[WJ];
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            fb[j] = *(const i32x4 *)(sp + kMxLdsA + ((WJ * wn + j) * 64 + lane) * 16);
            sb[j] = sws[(16 + WJ * wn + j) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            i32x8 a;
            a.lo = *(const i32x4 *)(sp + ((4 * wm + i) * 128 + lane) * 16);
            a.hi = *(const i32x4 *)(sp + ((4 * wm + i) * 128 + 64 + lane) * 16);
            const uint32_t sa = sws[(4 * wm + i) * 64 + lane];
#pragma unroll
            for (int j = 0; j < WJ; ++j) {
                i32x8 b;
                b.lo = fb[j];
                b.hi = z4;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i][j], 0, 4, 0, (int)(sa >> sh), 0,
                                                                            (int)(sb[j] >> sh));
            }
        }
        if (ks + 1 < nks) stash((ks + 1) & 1);                     // the stage read one step ago
        __syncthreads();
    }
    // lane (g, c16) holds rows 4g+e, column c16 of each 16x16 block
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const int col = 16 * (cb0 + WJ * wn + j) + c16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * (rb0 + 4 * wm + i) + 4 * g + e;
                if (row >= G.M) continue;
                const int64_t off = (int64_t)row * G.ldc + col;
                if (G.c_f32) ((float *)G.C)[off] = acc[i][j][e];
                else ((uint16_t *)G.C)[off] = bf16_bits(acc[i][j][e]);
            }
        }
}

// Tilings.  Up to 64 rows: a wave owns all (2 or 4) row blocks of one
// column block and keeps 8 k-steps of loads in flight -- the weights stream
// once.  Larger: 256x256 (or 256x128) tiles staged through LDS where N is a
// multiple of 256 (128), else a wave owns 64x64, a workgroup 128x128,
// straight from memory.
constexpr int kMxSmallRows = 64;

template <int CB>
static hipError_t launch_lds(MxArgs G, hipStream_t s) {
    // (one fixed size, set once: the initialisation of a local static is thread-safe)
    static const hipError_t lds_e = hipFuncSetAttribute((const void *)k_mx_gemm_lds<CB>,
                                                        hipFuncAttributeMaxDynamicSharedMemorySize, MxLds<CB>::BYTES);
    if (lds_e != hipSuccess) return lds_e;
    G.tiles_x = G.N / (16 * CB);
    G.tiles_y = (G.M + kMxLdsRows - 1) / kMxLdsRows;
    const int per = (G.tiles_x * G.tiles_y + 7) / 8;
    hipLaunchKernelGGL(k_mx_gemm_lds<CB>, dim3((unsigned)(8 * per)), dim3(512), (size_t)MxLds<CB>::BYTES, s, G, per);
    return hipGetLastError();
}

hipError_t launch_mx_quant(const uint16_t *X, int rows, int K, bool fp8, uint8_t *P, hipStream_t s) {
    const int nq = (K / 128 + 3) / 4;
    const int64_t rb = (rows + 15) / 16;
    const bool step1 = rows <= 256;                  // small inputs: more threads, one round trip
    const int64_t total = rb * nq * 64 * (step1 ? 4 : 1);
    const dim3 grid((unsigned)((total + 255) / 256));
    if (fp8 && step1) hipLaunchKernelGGL((k_mx_quant<true, true>), grid, dim3(256), 0, s, X, rows, K, P, total);
    else if (fp8) hipLaunchKernelGGL((k_mx_quant<true, false>), grid, dim3(256), 0, s, X, rows, K, P, total);
    else if (step1) hipLaunchKernelGGL((k_mx_quant<false, true>), grid, dim3(256), 0, s, X, rows, K, P, total);
    else hipLaunchKernelGGL((k_mx_quant<false, false>), grid, dim3(256), 0, s, X, rows, K, P, total);
    return hipGetLastError();
}

template <int WM, int WN, int WGM, int WGN, int D>
static void launch_tiled(MxArgs G, hipStream_t s) {
    const int rbs = (G.M + 15) / 16, cbs = G.N / 16;
    G.tiles_x = (cbs + WGN * WN - 1) / (WGN * WN);
    G.tiles_y = (rbs + WGM * WM - 1) / (WGM * WM);
    // weights of one column tile (codes and scales), chunks of at most 4 MB
    const int64_t tile_b = (int64_t)WGN * WN * (G.K / 128) * 1024 + (int64_t)WGN * WN * ((G.K / 128 + 3) / 4) * 256;
    const int64_t nchunks = (tile_b * G.tiles_x + (4 << 20) - 1) / (4 << 20);
    G.chunk_w = (int)((G.tiles_x + nchunks - 1) / nchunks);
    const int tiles = G.tiles_x * G.tiles_y;
    hipLaunchKernelGGL((k_mx_gemm<WM, WN, WGM, WGN, D>), dim3((unsigned)((tiles + 7) / 8 * 8)), dim3(256), 0, s, G);
}

hipError_t launch_mx_gemm(const uint8_t *A, const uint8_t *Bp, int M, int N, int K, void *C, int64_t ldc, int c_f32,
                          hipStream_t s) {
    MxArgs G{A, Bp, C, mx_code_bytes(M, K, true), mx_code_bytes(N, K, false), ldc, M, N, K, c_f32, 0, 0, 0};
    if (M <= 32) launch_tiled<2, 1, 1, 4, 8>(G, s);
    else if (M <= kMxSmallRows) launch_tiled<4, 1, 1, 4, 8>(G, s);
    else if (N % 128 == 0) {
        // 256-wide tiles unless they would leave compute units idle
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        const int64_t wide = (int64_t)(N / 256) * ((M + kMxLdsRows - 1) / kMxLdsRows);
        if (N % 256 == 0 && wide >= cus) return launch_lds<16>(G, s);
        return launch_lds<8>(G, s);
    } else launch_tiled<4, 4, 2, 2, 2>(G, s);
    return hipGetLastError();
}

}  // namespace dsv4
