// k_proj.hip -- the grouped output projection for gfx950.
//
// What is computed (rqlyzj.com article, section on depth compensation: the
// 128 heads' outputs are not projected to the model width in one matrix; the
// heads form 16 groups, each group's output is first condensed into a short
// group summary, and the 16 summaries are projected to the model width):
//     y[t][g] = W1[g] . o[t][g]         o[t][g]: the group's heads, gd = (H/G)*d dims
//                                        y[t][g]: r dims, stored as bf16
//     out[t]  = W2 . concat_g y[t][g]   hidden dims
// Both products are C[z][m][n] = sum_k A[z][m][k] * B[z][n][k] with A the
// activations (rows = tokens, k contiguous) and B the weights (rows = outputs,
// k contiguous), on v_mfma_f32_16x16x32_bf16.
//
// Batch invariance (m.youleyou.com article, "what was sacrificed": no split-K):
// every output element is reduced by one wave, k in steps of 32 in increasing
// order, with the same MFMA instruction whatever the tile; the tiling differs
// only in how many rows / columns a wave and a workgroup own.  So a token's
// output is bitwise the same whether it is one row of a decode batch or of a
// prefill chunk.
//
// The operands go straight from memory into MFMA registers: lane (g, c16) of
// a 16x16x32 step reads 16 bytes -- k = 8g .. 8g+7 of row c16 -- of A and of B.
// The weights are packed once (dsv4_out_proj_pack) in exactly that order: the
// operand of (16-row block, k-step) is one contiguous kilobyte, lane l's 16
// bytes at 16l, so every weight load reads whole lines in sequence (read
// straight from the row-major matrix, each load would touch 16 rows 64 bytes
// apiece, and HBM served that pattern at a quarter of its rate).  A D-deep
// ring of loads per wave keeps bytes in flight: the decode shape (a few dozen
// tokens) streams the weights once and is bound by HBM; the prefill shape
// reuses each loaded operand across a 64x64 wave tile.
#include "launch.h"

namespace dsv4 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint16_t *A;      // [z][M][lda] bf16
    const uint16_t *B;      // [z][N/16][K/32][64 lanes][8] bf16, packed (see k_pack_b)
    void *C;                // [z][M][ldc] bf16 or fp32
    int64_t lda, ldc;       // row strides (elements)
    int64_t sA, sB, sC;     // batch strides (elements)
    int M, N, K;
    int c_f32;              // C in fp32 (else bf16, round to nearest even)
};

// Pack W [z][N][K] (row-major, k contiguous) into the MFMA operand order:
// tile (n/16, k/32) is 512 elements, lane (k%32/8)*16 + n%16 holds the 8
// elements k - k%8 .. +8 of row n.  One thread per 16-byte piece.
__global__ __launch_bounds__(256) void k_pack_b(const uint16_t *W, uint16_t *P, int N, int K, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // piece index in the packed order
    if (i >= total) return;
    const int nk = K / 32;
    const int lane = (int)(i & 63);
    const int64_t tile = i >> 6;
    const int s = (int)(tile % nk);
    const int64_t zb = tile / nk;                  // z * (N/16) + column block
    const int nb16 = N / 16;
    const int64_t z = zb / nb16;
    const int nb = (int)(zb % nb16);
    const int n = 16 * nb + (lane & 15), k = 32 * s + 8 * (lane >> 4);
    *(u32x4 *)(P + 8 * i) = *(const u32x4 *)(W + (z * N + n) * (int64_t)K + k);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    union { u32x4 u; bf16x8 b; } x;
    x.u = v;
    return x.b;
}

// WM x WN 16x16 blocks per wave, WGM x WGN waves per workgroup (4 in all), D
// k-steps of loads in flight.
template <int WM, int WN, int WGM, int WGN, int D>
__global__ __launch_bounds__(256) void k_gemm_nt(GemmArgs G) {
    static_assert(WGM * WGN == 4, "four waves");
    const int z = blockIdx.z;
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int m0 = blockIdx.y * (WGM * WM * 16) + wm * WM * 16;
    const int n0 = blockIdx.x * (WGN * WN * 16) + wn * WN * 16;
    const uint16_t *A = G.A + (int64_t)z * G.sA;
    const uint16_t *B = G.B + (int64_t)z * G.sB;
    // row pointers at k = 8g: rows past M read row M-1 (their results are not stored)
    const uint16_t *ap[WM];
    const uint16_t *bp[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
        const int row = m0 + 16 * i + c16;
        ap[i] = A + (int64_t)(row < G.M ? row : G.M - 1) * G.lda + 8 * g;
    }
    const int nk = G.K / 32;                             // k-steps (K is a multiple of 32)
#pragma unroll
    for (int j = 0; j < WN; ++j) bp[j] = B + (int64_t)((n0 + 16 * j) / 16) * nk * 512 + 8 * lane;
    f32x4 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    u32x4 ra[D][WM], rb[D][WN];
    // step s's loads; steps past the end re-read the last step (never used), so
    // every ring slot is refilled on every path and the counter waits stay exact
    auto load = [&](int slot, int s) {
        const int sc = s < nk ? s : nk - 1;
#pragma unroll
        for (int i = 0; i < WM; ++i) ra[slot][i] = *(const u32x4 *)(ap[i] + 32 * sc);
#pragma unroll
        for (int j = 0; j < WN; ++j) rb[slot][j] = *(const u32x4 *)(bp[j] + (int64_t)512 * sc);
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, s);
#pragma unroll 1
    for (int s0 = 0; s0 < nk; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (s0 + d < nk) {                           // (uniform)
#pragma unroll
                for (int i = 0; i < WM; ++i)
#pragma unroll
                    for (int j = 0; j < WN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[d][i]), as_bf16x8(rb[d][j]),
                                                                            acc[i][j], 0, 0, 0);
            }
            load(d, s0 + d + D);
        }
    }
    // lane (g, c16) holds rows 4g+i, column c16 of each 16x16 block
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + 16 * i + 4 * g + e, col = n0 + 16 * j + c16;
                if (row >= G.M) continue;
                const int64_t off = (int64_t)z * G.sC + (int64_t)row * G.ldc + col;
                if (G.c_f32) ((float *)G.C)[off] = acc[i][j][e];
                else ((uint16_t *)G.C)[off] = bf16_bits(acc[i][j][e]);
            }
}

// Large batches with LDS-staged tiles: a workgroup of 8 waves owns a 256x256
// tile of C, wave (wm, wn) of it 128x64 (8 x 4 blocks of 16x16).  k advances
// in tiles of 64 (two MFMA k-steps): all 512 threads copy the tile's A and B
// operands (32 KB each) from memory into LDS, laid out in MFMA operand order
// -- per (k-step, 16-row block) one kilobyte, lane l's 16 bytes at 16 l -- so
// the copy's stores and the waves' operand reads are both 64 consecutive
// 16-byte slots (no bank conflicts).  Two LDS stages and two register sets:
// tiles t+1 and t+2 are in flight while tile t is multiplied, then tile t+1 is
// stored into the other stage; one barrier per tile.  Each wave's operand bytes are read from LDS
// instead of from the L1 / L2 caches, and each byte fetched from memory feeds
// 256 rows or columns.  Every output element is still one wave's chain of
// 16x16x32 MFMAs over the k-steps in increasing order, so the results are
// bitwise those of the other tilings.
//
// Workgroups are dealt to the 8 XCDs in turn: workgroup id w computes tile
// (w mod 8) * per + w / 8, so each XCD runs a contiguous range of tiles, taken
// in groups of four row tiles column by column (the XCD's concurrent
// workgroups then share their A and B tiles in its L2).
constexpr int kLdsBM = 256, kLdsBN = 256, kLdsBK = 64;
constexpr int kLdsGroupM = 4;
constexpr int kLdsStage = (kLdsBM + kLdsBN) * kLdsBK * 2;     // bytes of one LDS stage
constexpr int kLdsBytes = 2 * kLdsStage;

__global__ __launch_bounds__(512) void k_gemm_nt_lds(GemmArgs G, int nx, int ny, int per) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;                 // 2 x 4 waves
    const int z = blockIdx.y;
    const int w = blockIdx.x;
    const int T = (w & 7) * per + (w >> 3);                  // this workgroup's tile
    if (T >= nx * ny) return;
    const int gsz = kLdsGroupM * nx;                         // tiles of a group of row tiles
    const int fr = (T / gsz) * kLdsGroupM;
    const int rows = ny - fr < kLdsGroupM ? ny - fr : kLdsGroupM;
    const int ty = fr + (T % gsz) % rows, tx = (T % gsz) / rows;
    const int m0 = ty * kLdsBM, n0 = tx * kLdsBN;
    const uint16_t *A = G.A + (int64_t)z * G.sA;
    const uint16_t *B = G.B + (int64_t)z * G.sB;
    const int nk = G.K / 32;                                 // k-steps
    const int nkt = G.K / kLdsBK;                            // k-tiles

    // the copy: thread t moves pieces p = t + 512 u (u < 4) of A and of B, in
    // operand order p = (k-step s, block i, lane l): A row m0 + 16 i + l % 16
    // at k = 32 s + 8 (l / 16) (rows past M read row M-1, never stored); B the
    // packed kilobyte of column block n0 / 16 + i, k-step s
    const uint16_t *ga[4];
    const uint16_t *gb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int p = tid + 512 * u, s = p >> 10, i = (p >> 6) & 15, l = p & 63;
        int row = m0 + 16 * i + (l & 15);
        row = row < G.M ? row : G.M - 1;
        ga[u] = A + (int64_t)row * G.lda + 32 * s + 8 * (l >> 4);
        gb[u] = B + ((int64_t)(n0 / 16 + i) * nk + s) * 512 + 8 * l;
    }
    // two tiles' loads in flight: tile j's in register set j mod 2 (a tile
    // past the end re-reads the last one: every load unconditional, never used)
    u32x4 ra[2][4], rb[2][4];
    auto fetch = [&](int set, int kt) {
        const int kc = kt < nkt ? kt : nkt - 1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ra[set][u] = *(const u32x4 *)(ga[u] + (int64_t)kLdsBK * kc);
            rb[set][u] = *(const u32x4 *)(gb[u] + (int64_t)1024 * kc);   // two packed k-steps a tile
        }
    };
    auto stash = [&](int set, int st) {
        uint8_t *sa = smem + st * kLdsStage, *sb = sa + kLdsBM * kLdsBK * 2;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            *(u32x4 *)(sa + 16 * (tid + 512 * u)) = ra[set][u];
            *(u32x4 *)(sb + 16 * (tid + 512 * u)) = rb[set][u];
        }
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](int st) {
        const uint8_t *sa = smem + st * kLdsStage, *sb = sa + kLdsBM * kLdsBK * 2;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            u32x4 fa[8], fb[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[i] = *(const u32x4 *)(sa + (((s * 16 + 8 * wm + i) * 64) + lane) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = *(const u32x4 *)(sb + (((s * 16 + 4 * wn + j) * 64) + lane) * 16);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j],
                                                                        0, 0, 0);
        }
    };
    // tile kt is multiplied from stage kt mod 2 while tiles kt+1 (set (kt+1)
    // mod 2) and kt+2 are on their way; then tile kt+1 goes into the other
    // stage and its registers take tile kt+3
    fetch(0, 0);
    stash(0, 0);
    fetch(1, 1);
    fetch(0, 2);
    __syncthreads();
#pragma unroll 1
    for (int kt = 0; kt < nkt; kt += 2) {
        compute(0);
        if (kt + 1 < nkt) {                                  // (uniform)
            stash(1, 1);
            fetch(1, kt + 3);
        }
        __syncthreads();
        if (kt + 1 < nkt) {
            compute(1);
            if (kt + 2 < nkt) {
                stash(0, 0);
                fetch(0, kt + 4);
            }
            __syncthreads();
        }
    }
    // lane (g, c16) holds rows 4g+e, column c16 of each 16x16 block
    const int g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + 128 * wm + 16 * i + 4 * g + e, col = n0 + 64 * wn + 16 * j + c16;
                if (row >= G.M) continue;
                const int64_t off = (int64_t)z * G.sC + (int64_t)row * G.ldc + col;
                if (G.c_f32) ((float *)G.C)[off] = acc[i][j][e];
                else ((uint16_t *)G.C)[off] = bf16_bits(acc[i][j][e]);
            }
}

// Tilings.  Small batches: a wave owns one 16x16 block and keeps 8 k-steps of
// loads in flight (the weights are streamed once; parallelism comes from the
// columns).  Large batches: 256x256 workgroup tiles staged through LDS where N
// and K allow (N a multiple of 256, K of 64), else a wave owns 64x64 straight
// from memory, a workgroup 128x128.
constexpr int kProjSmallRows = 256;
constexpr int kSmallTileM = 32, kSmallTileN = 32;
constexpr int kLargeTileM = 128, kLargeTileN = 128;

int proj_tile_n() { return kLargeTileN; }

static hipError_t launch_gemm(const GemmArgs &G, int batch, hipStream_t s) {
    if (G.M <= kProjSmallRows) {
        dim3 grid((unsigned)(G.N / kSmallTileN), (unsigned)((G.M + kSmallTileM - 1) / kSmallTileM), (unsigned)batch);
        hipLaunchKernelGGL((k_gemm_nt<1, 1, 2, 2, 8>), grid, dim3(256), 0, s, G);
    } else if (G.N % kLdsBN == 0 && G.K % kLdsBK == 0) {
        // (one fixed size, set once: the initialisation of a local static is thread-safe)
        static const hipError_t lds_e =
            hipFuncSetAttribute((const void *)k_gemm_nt_lds, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (lds_e != hipSuccess) return lds_e;
        const int nx = G.N / kLdsBN, ny = (G.M + kLdsBM - 1) / kLdsBM;
        const int per = (nx * ny + 7) / 8;
        hipLaunchKernelGGL(k_gemm_nt_lds, dim3((unsigned)(8 * per), (unsigned)batch), dim3(512), (size_t)kLdsBytes, s,
                           G, nx, ny, per);
    } else {
        dim3 grid((unsigned)(G.N / kLargeTileN), (unsigned)((G.M + kLargeTileM - 1) / kLargeTileM), (unsigned)batch);
        hipLaunchKernelGGL((k_gemm_nt<4, 4, 2, 2, 2>), grid, dim3(256), 0, s, G);
    }
    return hipGetLastError();
}

hipError_t launch_out_proj(const uint16_t *o, int T, int H, int d, int groups, int rank, int hidden,
                           const uint16_t *w1p, const uint16_t *w2p, uint16_t *y, void *out, int out_f32,
                           hipStream_t s) {
    const int gd = H / groups * d;
    GemmArgs g1{o, w1p, y, (int64_t)H * d, (int64_t)groups * rank, gd, (int64_t)rank * gd, rank,
                T, rank, gd, 0};
    hipError_t e = launch_gemm(g1, groups, s);
    if (e != hipSuccess) return e;
    GemmArgs g2{y, w2p, out, (int64_t)groups * rank, hidden, 0, 0, 0, T, hidden, groups * rank, out_f32};
    return launch_gemm(g2, 1, s);
}

hipError_t launch_pack_b(const uint16_t *W, uint16_t *P, int batch, int N, int K, hipStream_t s) {
    const int64_t total = (int64_t)batch * N * K / 8;
    hipLaunchKernelGGL(k_pack_b, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W, P, N, K, total);
    return hipGetLastError();
}

}  // namespace dsv4
