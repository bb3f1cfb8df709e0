// launch.h -- internal launchers shared between the kernel files and the C ABI.
#pragma once
#include "common.h"

namespace dsv4 {

hipError_t launch_compress_decode(const Lay &L, const dsv4_cache &C, const void *kv, const void *gate,
                                  const void *kI, const void *gI, const int32_t *req,
                                  const int32_t *pos, int B, hipStream_t s);
hipError_t launch_compress_prefill(const Lay &L, const dsv4_cache &C, const void *kv, const void *gate,
                                   const void *kI, const void *gI, const int32_t *cu,
                                   const int32_t *req, const int32_t *pos0, int n_seq, int total,
                                   uint8_t *win, hipStream_t s);
hipError_t launch_write_entries(const Lay &L, const dsv4_cache &C, int target, const int32_t *req,
                                const int32_t *ent, int n, const float *vals, hipStream_t s);
hipError_t launch_state_tokens(const Lay &L, const dsv4_cache &C, int r, int64_t p0, int n,
                               const void *kv, const void *gate, const void *kI, const void *gI,
                               hipStream_t s);

// Top-k: scores are selected in segments of kTkSeg; a query's boundary bin
// keeps at most kTkCandMax candidates in the workspace (more take a slower
// exact path); a score row spans at most kTkMaxSeg segments.
constexpr int kTkSeg = 4096;
constexpr int kTkBins = 2048;
constexpr int kTkCandMax = 4096;
constexpr int kTkMaxSeg = 1024;
// Rows of at most this many segments skip the separate boundary-bin pass:
// each split workgroup sums the (few) segment histograms itself.
constexpr int kTkFuseSeg = 16;
// Queries (or rows) one indexer / top-k launch takes: the grid's y extent.
constexpr int kMaxGridRows = 65535;
// Per-query outcome of the boundary-bin pass.
struct TkQuery {
    float fmin, scale;      // linear map of the finite scores onto the bins
    int32_t bstar;          // bin holding the k-th largest score (-1: the NaN scores)
    int32_t rem;            // elements still to take from bin bstar
    int32_t n_sure;         // elements above bin bstar (all selected)
    int32_t n_cand;         // elements inside bin bstar
    int32_t pad[2];
};
struct IndexWs {
    uint8_t *q8;
    float *wq;
    uint2 *wr;              // [n][nwr]: per scoring wave, min / max key of its finite scores
    float *scores;          // [n][ld]
    uint16_t *hist;         // [n][s_max][kTkBins] per-segment counts
    TkQuery *qm;            // [n]
    int2 *segoff;           // [n][s_max]: output offsets of a segment's sure / candidate elements
    int32_t *sure;          // [n][k]
    uint32_t *ckey;         // [n][kTkCandMax]
    int32_t *cpos;          // [n][kTkCandMax]
    int32_t *crank;         // [n][kTkCandMax]: sure elements before each candidate
    int64_t ld;
    int nwr, s_max;
};
// Bytes of the indexer's workspace for n queries of at most nmax visible
// entries; with w, its regions carved from base.  scores_off / scores_ld
// (optional): byte offset of the score rows and their stride in floats.
int64_t index_ws_bytes(const Lay &L, int n, int64_t nmax, IndexWs *w, uint8_t *base, int64_t *scores_off = nullptr,
                       int64_t *scores_ld = nullptr);
hipError_t launch_quant_q(const Lay &L, const void *qI, const float *w, int rows, const IndexWs &ws,
                          hipStream_t s);
hipError_t launch_score_decode(const Lay &L, const dsv4_cache &C, const void *qI, const float *w,
                               const int32_t *req, const int32_t *pos, int n, const IndexWs &ws, hipStream_t s);
// The same scores for the packed rows of a prefill chunk (rows of one request
// in index order share their key loads).
hipError_t launch_score_prefill(const Lay &L, const dsv4_cache &C, const int32_t *req, const int32_t *pos,
                                int n, const IndexWs &ws, hipStream_t s);
// fp32 index rows (reference-precision storage): scores from the query rows
// as given, into the same workspace records the top-k passes read.
hipError_t launch_score_f32(const Lay &L, const dsv4_cache &C, const void *qI, const float *w, const int32_t *req,
                            const int32_t *pos, int n, const IndexWs &ws, hipStream_t s);
hipError_t launch_topk(const Lay &L, const dsv4_cache &C, const int32_t *req, const int32_t *pos, int n,
                       const IndexWs &ws, int32_t *out, hipStream_t s);
hipError_t launch_topk_rows(const float *scores, int64_t ld, const int32_t *nvis, int n, int64_t max_n, int k,
                            const IndexWs &ws, int32_t *out, hipStream_t s);
hipError_t launch_expand_queries(const int32_t *cu, const int32_t *req, const int32_t *pos0, int n_seq,
                                 int total, int32_t *req_q, int32_t *pos_q, hipStream_t s);

struct AttnArgs {
    Lay L;
    dsv4_cache C;
    const void *q;
    const int32_t *req;     // decode
    const int32_t *pos;     // decode
    const int32_t *cu;      // prefill
    const int32_t *pos0;    // prefill
    int n_seq;
    const int32_t *topk;    // CSA
    const uint8_t *win;     // prefill window records
    const float *sinks;
    void *out;
    int nq;
    int nhg;                // head groups (ceil(H/16))
};
hipError_t launch_attend(const AttnArgs &A, bool csa, bool prefill, bool hi, hipStream_t s);
// fp32 records (reference-precision storage): one kernel for both policies.
hipError_t launch_attend_f32(const AttnArgs &A, bool csa, bool prefill, hipStream_t s);
// Longest record list one attention query can have, and the LDS the attention
// kernels need for it (the per-query locators live in LDS).
int64_t attend_list_max(const Lay &L, const dsv4_cache &C, bool csa);
int64_t attend_lds_max(const Lay &L, int64_t list_max);
constexpr int64_t kLdsMax = 160 * 1024;   // LDS of one gfx950 workgroup

// Grouped output projection (two batch-invariant bf16 products).
hipError_t launch_out_proj(const uint16_t *o, int T, int H, int d, int groups, int rank, int hidden,
                           const uint16_t *w1p, const uint16_t *w2p, uint16_t *y, void *out, int out_f32,
                           hipStream_t s);
hipError_t launch_pack_b(const uint16_t *W, uint16_t *P, int batch, int N, int K, hipStream_t s);
// Dump / reload of one request's cache (state, then its entry and index blocks).
int64_t mx_pack_bytes(int rows, int K, bool fp8);
hipError_t launch_mx_quant(const uint16_t *X, int rows, int K, bool fp8, uint8_t *P, hipStream_t s);
hipError_t launch_mx_gemm(const uint8_t *A, const uint8_t *Bp, int M, int N, int K, void *C, int64_t ldc, int c_f32,
                          hipStream_t s);
int64_t cache_dump_bytes(const Lay &L, int nb);
// Dequantised read-back of stored entries, index keys or window records.
hipError_t launch_read_entries(const Lay &L, const dsv4_cache &C, int target, const int32_t *req, const int32_t *idx,
                               int n, void *out, bool f64, hipStream_t s);
hipError_t launch_cache_xfer(const Lay &L, const dsv4_cache &C, int r, int nb, uint8_t *buf, bool to_buf,
                             hipStream_t s);

}  // namespace dsv4
