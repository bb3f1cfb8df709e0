// api.cpp -- the C ABI of libdsv4attn: argument validation, layouts, dispatch
// and the optional kernel timers.  Every check runs on the host before any
// launch; a failed check launches nothing.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "launch.h"

using namespace dsv4;

namespace {

bool pow2_divides_128(int v) { return v >= 1 && v <= 128 && (v & (v - 1)) == 0; }
int64_t al(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
hipStream_t S(void *s) { return (hipStream_t)s; }

// ---- timers
struct TimerSlot {
    bool on = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
    double total_ms = 0.0;
    int64_t count = 0;
};
TimerSlot g_timers[DSV4_K_COUNT];
std::mutex g_timer_mu;

struct Timed {
    int id;
    hipStream_t s;
    hipEvent_t a = nullptr, b = nullptr;
    Timed(int id_, hipStream_t s_) : id(id_), s(s_) {   // id -1: never timed
        if (id >= 0 && g_timers[id].on) {
            hipEventCreate(&a);
            hipEventCreate(&b);
            hipEventRecord(a, s);
        }
    }
    ~Timed() {
        if (a) {
            hipEventRecord(b, s);
            std::lock_guard<std::mutex> lk(g_timer_mu);
            g_timers[id].pending.emplace_back(a, b);
        }
    }
};

dsv4_status hip_status(hipError_t e) { return e == hipSuccess ? DSV4_OK : DSV4_ERR_LAUNCH; }

dsv4_status check_cache(const Lay &L, const dsv4_cache *C, int kind) {
    if (!C) return DSV4_ERR_INVALID_ARG;
    if (C->kind != kind) return DSV4_ERR_INVALID_ARG;
    if (C->n_req <= 0 || C->max_blocks <= 0 || C->n_blocks <= 0) return DSV4_ERR_INVALID_ARG;
    if (!C->entries || !C->state || !C->block_table) return DSV4_ERR_INVALID_ARG;
    if (kind == DSV4_CSA && !C->index_keys) return DSV4_ERR_INVALID_ARG;
    if ((int64_t)C->max_blocks * kBlockTokens > (int64_t)1 << 30) return DSV4_ERR_INVALID_ARG;
    if (((uintptr_t)C->entries | (uintptr_t)C->state) & 255) return DSV4_ERR_INVALID_ARG;
    if (C->index_keys && ((uintptr_t)C->index_keys & 255)) return DSV4_ERR_INVALID_ARG;
    (void)L;
    return DSV4_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

int num_cus() {
    // (a function-local static: initialised once, thread-safe, on the device
    // current at the first call)
    static const int cus = [] {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            return prop.multiProcessorCount;
        return 256;
    }();
    return cus;
}

bool pick_hi(int policy, int nq, int nhg) {
    if (policy == DSV4_POLICY_HI) return true;
    if (policy == DSV4_POLICY_LO) return false;
    // LO gives each (query, head group) workgroup 16 waves; once there are
    // enough workgroups to give every compute unit several, HI's 4-wave
    // workgroups keep the same number of waves busy with less LDS each
    return (int64_t)nq * nhg >= 2 * (int64_t)num_cus();
}

}  // namespace

namespace dsv4 {

dsv4_status make_layout(const dsv4_cfg *c, int32_t kind, Lay *out) {
    if (!c || !out) return DSV4_ERR_INVALID_ARG;
    if (kind != DSV4_CSA && kind != DSV4_HCA) return DSV4_ERR_INVALID_ARG;
    if (c->d <= 0 || c->d_rope <= 0 || c->d_rope > c->d || c->d_rope > 128 || (c->d_rope & 1) || (c->d % 16) ||
        (c->d_rope % 16))
        return DSV4_ERR_INVALID_ARG;
    if (c->n_heads < 1 || c->n_heads > 256) return DSV4_ERR_INVALID_ARG;
    if (c->window < 0 || c->window > 1024) return DSV4_ERR_INVALID_ARG;
    if (!pow2_divides_128(c->m_csa) || !(c->w_csa == c->m_csa || c->w_csa == 2 * c->m_csa))
        return DSV4_ERR_INVALID_ARG;
    if (!pow2_divides_128(c->m_hca)) return DSV4_ERR_INVALID_ARG;
    if (c->idx_heads < 1 || c->idx_heads > 64) return DSV4_ERR_INVALID_ARG;
    if (c->idx_dim < 32 || c->idx_dim > 128 || (c->idx_dim % 32)) return DSV4_ERR_INVALID_ARG;
    if (c->topk < 1 || c->topk > 2048) return DSV4_ERR_INVALID_ARG;
    if (c->kv_store != DSV4_STORE_FP8 && c->kv_store != DSV4_STORE_FP32) return DSV4_ERR_INVALID_ARG;
    if (c->idx_store != DSV4_STORE_FP8 && c->idx_store != DSV4_STORE_FP32 && c->idx_store != DSV4_STORE_MXFP4)
        return DSV4_ERR_INVALID_ARG;
    if (c->act_dtype != DSV4_DT_F32 && c->act_dtype != DSV4_DT_BF16) return DSV4_ERR_INVALID_ARG;
    if (!(c->rope_base > 0.0f) || !isfinite(c->rope_base)) return DSV4_ERR_INVALID_ARG;
    if (!(c->softmax_scale > 0.0f) || !isfinite(c->softmax_scale)) return DSV4_ERR_INVALID_ARG;
    const bool shape_built = (c->d == 512 && c->d_rope == 64) || (c->d == 64 && c->d_rope == 16);
    if (!shape_built) return DSV4_ERR_UNSUPPORTED;

    Lay L;
    memset(&L, 0, sizeof(L));
    L.kind = kind;
    L.d = c->d;
    L.dr = c->d_rope;
    L.dn = c->d - c->d_rope;
    L.H = c->n_heads;
    L.W = c->window;
    L.m = kind == DSV4_CSA ? c->m_csa : c->m_hca;
    L.wc = kind == DSV4_CSA ? c->w_csa : c->m_hca;
    L.epb = kBlockTokens / L.m;
    L.kv_store = c->kv_store;
    L.idx_store = c->idx_store;
    L.act = c->act_dtype;
    L.rope_base = c->rope_base;
    L.tau = c->softmax_scale;
    L.topk = c->topk;
    if (c->kv_store == DSV4_STORE_FP8) {
        L.rope_off = L.dn;
        L.scale_off = L.dn + 2 * L.dr;
        L.rec_bytes = (int)al(L.dn + 2 * L.dr + 4, 64);
    } else {
        L.rope_off = 0;
        L.scale_off = 0;
        L.rec_bytes = (int)al(4 * (int64_t)L.d, 64);
    }
    L.entry_block_bytes = (int64_t)L.epb * L.rec_bytes;
    L.HI = c->idx_heads;
    L.dI = c->idx_dim;
    L.key_bytes = c->idx_store == DSV4_STORE_MXFP4 ? L.dI / 2 : c->idx_store == DSV4_STORE_FP8 ? L.dI : 4 * L.dI;
    L.key_scale_off = L.epb * L.key_bytes;
    L.index_block_bytes = kind == DSV4_CSA ? al((int64_t)L.epb * L.key_bytes + (int64_t)L.epb * 4, 256) : 0;
    for (int i = 0; i < L.dr / 2 && i < 64; ++i)
        L.theta[i] = pow((double)c->rope_base, -2.0 * (double)i / (double)L.dr);
    L.pend_slots = L.wc;
    L.pend_tok_floats = 2 * L.d + (kind == DSV4_CSA ? 2 * L.dI : 0);
    L.pend_off = al((int64_t)L.W * L.rec_bytes, 256);
    L.state_bytes = al(L.pend_off + (int64_t)L.pend_slots * L.pend_tok_floats * 4, 256);
    *out = L;
    return DSV4_OK;
}

}  // namespace dsv4

extern "C" {

const char *dsv4_status_string(dsv4_status s) {
    switch (s) {
        case DSV4_OK: return "ok";
        case DSV4_ERR_INVALID_ARG: return "invalid argument";
        case DSV4_ERR_UNSUPPORTED: return "unsupported configuration";
        case DSV4_ERR_WORKSPACE: return "workspace missing or too small";
        case DSV4_ERR_LAUNCH: return "kernel launch failed";
        case DSV4_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

dsv4_status dsv4_get_layout(const dsv4_cfg *cfg, int32_t kind, dsv4_layout *out) {
    if (!out) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, kind, &L);
    if (st != DSV4_OK) return st;
    out->record_bytes = L.rec_bytes;
    out->entries_per_block = L.epb;
    out->entry_block_bytes = L.entry_block_bytes;
    out->index_key_bytes = kind == DSV4_CSA ? L.key_bytes : 0;
    out->index_block_bytes = L.index_block_bytes;
    out->state_bytes = L.state_bytes;
    out->pending_offset = L.pend_off;
    out->pending_slots = L.pend_slots;
    out->pending_token_floats = L.pend_tok_floats;
    return DSV4_OK;
}

dsv4_status dsv4_workspace_bytes(const dsv4_cfg *cfg, int32_t n_queries, int32_t max_entries, int64_t *out) {
    if (!out || n_queries < 0 || max_entries < 0) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, DSV4_CSA, &L);
    if (st != DSV4_OK) return st;
    *out = index_ws_bytes(L, n_queries, max_entries, nullptr, nullptr) + al((int64_t)n_queries * 8, 256);
    return DSV4_OK;
}

dsv4_status dsv4_index_scores_layout(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t n_queries,
                                     int32_t prefill, int64_t *offset, int64_t *ld) {
    if (!offset || !ld || n_queries < 1 || n_queries > kMaxGridRows || (prefill != 0 && prefill != 1))
        return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, DSV4_CSA, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, DSV4_CSA)) != DSV4_OK) return st;
    int64_t off = 0, stride = 0;
    index_ws_bytes(L, n_queries, (int64_t)cache->max_blocks * L.epb, nullptr, nullptr, &off, &stride);
    // a prefill call's workspace starts with its per-query (request, position) rows
    *offset = (prefill ? al((int64_t)n_queries * 8, 256) : 0) + off;
    *ld = stride;
    return DSV4_OK;
}

dsv4_status dsv4_compress_kv_decode(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *kv,
                                    const void *gate, const void *kI, const void *gI, const int32_t *req_dev,
                                    const int32_t *pos_dev, int32_t B, void *stream) {
    if (!cache) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, cache->kind, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, cache->kind)) != DSV4_OK) return st;
    if (B < 0) return DSV4_ERR_INVALID_ARG;
    if (B == 0) return DSV4_OK;
    if (!kv || !gate || !req_dev || !pos_dev) return DSV4_ERR_INVALID_ARG;
    if (cache->kind == DSV4_CSA && (!kI || !gI)) return DSV4_ERR_INVALID_ARG;
    Timed tm(DSV4_K_COMPRESS, S(stream));
    return hip_status(launch_compress_decode(L, *cache, kv, gate, kI, gI, req_dev, pos_dev, B, S(stream)));
}

dsv4_status dsv4_compress_kv_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *kv,
                                     const void *gate, const void *kI, const void *gI,
                                     const int32_t *cu_seqlens_dev, const int32_t *req_dev,
                                     const int32_t *pos0_dev, int32_t n_seq, int32_t total_tokens,
                                     void *win_out_dev, void *stream) {
    if (!cache) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, cache->kind, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, cache->kind)) != DSV4_OK) return st;
    if (n_seq < 0 || total_tokens < 0) return DSV4_ERR_INVALID_ARG;
    if (n_seq == 0 || total_tokens == 0) return DSV4_OK;
    if (!kv || !gate || !cu_seqlens_dev || !req_dev || !pos0_dev || !win_out_dev) return DSV4_ERR_INVALID_ARG;
    if (cache->kind == DSV4_CSA && (!kI || !gI)) return DSV4_ERR_INVALID_ARG;
    if (!aligned16(win_out_dev)) return DSV4_ERR_INVALID_ARG;
    Timed tm(DSV4_K_COMPRESS, S(stream));
    return hip_status(launch_compress_prefill(L, *cache, kv, gate, kI, gI, cu_seqlens_dev, req_dev, pos0_dev,
                                              n_seq, total_tokens, (uint8_t *)win_out_dev, S(stream)));
}

static dsv4_status index_topk_common(const Lay &L, const dsv4_cache *cache, const void *qI, const float *w,
                                     const int32_t *req_q, const int32_t *pos_q, int nq, int32_t *topk_dev,
                                     uint8_t *ws, int64_t ws_bytes, hipStream_t s, bool prefill,
                                     bool timed = true) {
    const int64_t nmax = (int64_t)cache->max_blocks * L.epb;
    IndexWs W;
    const int64_t need = index_ws_bytes(L, nq, nmax, &W, ws);
    if (need > ws_bytes) return DSV4_ERR_WORKSPACE;
    if (W.s_max > kTkMaxSeg) return DSV4_ERR_UNSUPPORTED;
    hipError_t e;
    if (L.idx_store == DSV4_STORE_FP32) {          // fp32 rows: the queries are scored as given
        Timed tm(timed ? DSV4_K_INDEX_SCORE : -1, s);
        e = launch_score_f32(L, *cache, qI, w, req_q, pos_q, nq, W, s);
    } else {
        if (L.epb < 16) return DSV4_ERR_UNSUPPORTED;   // scoring reads 16-key runs inside one block
        if (prefill) {                             // (decode quantises the queries inside the scorer)
            e = launch_quant_q(L, qI, w, nq * L.HI, W, s);
            if (e != hipSuccess) return DSV4_ERR_LAUNCH;
        }
        Timed tm(timed ? DSV4_K_INDEX_SCORE : -1, s);
        e = prefill ? launch_score_prefill(L, *cache, req_q, pos_q, nq, W, s)
                    : launch_score_decode(L, *cache, qI, w, req_q, pos_q, nq, W, s);
    }
    if (e != hipSuccess) return DSV4_ERR_LAUNCH;
    Timed tm(timed ? DSV4_K_TOPK : -1, s);
    return hip_status(launch_topk(L, *cache, req_q, pos_q, nq, W, topk_dev, s));
}

dsv4_status dsv4_index_topk_decode(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *qI,
                                   const float *w_dev, const int32_t *req_dev, const int32_t *pos_dev,
                                   int32_t B, int32_t *topk_dev, void *ws_dev, int64_t ws_bytes,
                                   void *stream) {
    Lay L;
    dsv4_status st = make_layout(cfg, DSV4_CSA, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, DSV4_CSA)) != DSV4_OK) return st;
    if (B < 0) return DSV4_ERR_INVALID_ARG;
    if (B == 0) return DSV4_OK;
    if (B > kMaxGridRows) return DSV4_ERR_UNSUPPORTED;
    if (!qI || !aligned16(qI) || !req_dev || !pos_dev || !topk_dev) return DSV4_ERR_INVALID_ARG;
    if (!ws_dev || ws_bytes <= 0 || ((uintptr_t)ws_dev & 255)) return DSV4_ERR_WORKSPACE;
    return index_topk_common(L, cache, qI, w_dev, req_dev, pos_dev, B, topk_dev, (uint8_t *)ws_dev, ws_bytes,
                             S(stream), false);
}

}  // extern "C"

// ---- the allocation-free decode indexer: its workspace is a file-scope device
// array of kNoAllocScratch bytes, one copy per GPU (held until the process
// ends).  Host code never uses the array's name as an address: each device's
// address is taken once with hipGetSymbolAddress (with that device current)
// and kept.  Every call on a GPU shares that GPU's array, so calls that
// overlap on one GPU race; nothing in it needs to start at zero (every byte
// a call reads was written earlier in the same call).
namespace {
constexpr int64_t kNoAllocScratch = (int64_t)DSV4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratch];
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};

dsv4_status scratch_of_current_device(uint8_t **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSV4_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSV4_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = (uint8_t *)g_scratch_ptr[dev];
    return DSV4_OK;
}
}  // namespace

extern "C" {

dsv4_status dsv4_index_topk_decode_noalloc(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *qI,
                                           const float *w_dev, const int32_t *req_dev, const int32_t *pos_dev,
                                           int32_t B, int32_t *topk_dev, void *stream) {
    Lay L;
    dsv4_status st = make_layout(cfg, DSV4_CSA, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, DSV4_CSA)) != DSV4_OK) return st;
    if (B < 0) return DSV4_ERR_INVALID_ARG;
    if (B == 0) return DSV4_OK;
    if (B > kMaxGridRows) return DSV4_ERR_UNSUPPORTED;
    if (!qI || !aligned16(qI) || !req_dev || !pos_dev || !topk_dev) return DSV4_ERR_INVALID_ARG;
    const int64_t need = index_ws_bytes(L, B, (int64_t)cache->max_blocks * L.epb, nullptr, nullptr);
    if (need > kNoAllocScratch) return DSV4_ERR_WORKSPACE;
    uint8_t *ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != DSV4_OK) return st;
    return index_topk_common(L, cache, qI, w_dev, req_dev, pos_dev, B, topk_dev, ws, kNoAllocScratch, S(stream),
                             false, false);
}

dsv4_status dsv4_index_topk_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *qI,
                                    const float *w_dev, const int32_t *cu_seqlens_dev, const int32_t *req_dev,
                                    const int32_t *pos0_dev, int32_t n_seq, int32_t total_tokens,
                                    int32_t *topk_dev, void *ws_dev, int64_t ws_bytes, void *stream) {
    Lay L;
    dsv4_status st = make_layout(cfg, DSV4_CSA, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, DSV4_CSA)) != DSV4_OK) return st;
    if (n_seq < 0 || total_tokens < 0) return DSV4_ERR_INVALID_ARG;
    if (n_seq == 0 || total_tokens == 0) return DSV4_OK;
    if (!qI || !aligned16(qI) || !cu_seqlens_dev || !req_dev || !pos0_dev || !topk_dev) return DSV4_ERR_INVALID_ARG;
    if (!ws_dev || ws_bytes <= 0 || ((uintptr_t)ws_dev & 255)) return DSV4_ERR_WORKSPACE;
    // per-query (request, position) rows first, then groups of queries that fit
    const int64_t rows_bytes = al((int64_t)total_tokens * 8, 256);
    const int64_t nmax = (int64_t)cache->max_blocks * L.epb;
    const int64_t per1 = index_ws_bytes(L, 1, nmax, nullptr, nullptr);
    if (ws_bytes < rows_bytes + per1) return DSV4_ERR_WORKSPACE;
    uint8_t *ws = (uint8_t *)ws_dev;
    int32_t *req_q = (int32_t *)ws, *pos_q = req_q + total_tokens;
    hipStream_t s = S(stream);
    if (launch_expand_queries(cu_seqlens_dev, req_dev, pos0_dev, n_seq, total_tokens, req_q, pos_q, s) !=
        hipSuccess)
        return DSV4_ERR_LAUNCH;
    int group = total_tokens;
    if (group > kMaxGridRows) group = kMaxGridRows;
    while (group > 1 && rows_bytes + index_ws_bytes(L, group, nmax, nullptr, nullptr) > ws_bytes) group = (group + 1) / 2;
    const int64_t qrow = (int64_t)L.HI * L.dI * (L.act == DSV4_DT_BF16 ? 2 : 4);
    for (int q0 = 0; q0 < total_tokens; q0 += group) {
        const int n = total_tokens - q0 < group ? total_tokens - q0 : group;
        st = index_topk_common(L, cache, (const uint8_t *)qI + q0 * qrow, w_dev ? w_dev + (int64_t)q0 * L.HI : nullptr,
                               req_q + q0, pos_q + q0, n, topk_dev + (int64_t)q0 * L.topk, ws + rows_bytes,
                               ws_bytes - rows_bytes, s, true);
        if (st != DSV4_OK) return st;
    }
    return DSV4_OK;
}

static void rows_layout(int k, Lay *L) {
    memset(L, 0, sizeof(*L));
    L->topk = k;
    L->m = 1;
}

dsv4_status dsv4_topk_rows_ws_bytes(int32_t n_rows, int32_t max_n, int32_t k, int64_t *out) {
    if (!out || n_rows < 0 || max_n < 0 || max_n > (1 << 30) || k < 1 || k > 2048) return DSV4_ERR_INVALID_ARG;
    Lay L;
    rows_layout(k, &L);
    *out = index_ws_bytes(L, n_rows < kMaxGridRows ? n_rows : kMaxGridRows, max_n, nullptr, nullptr);
    return DSV4_OK;
}

dsv4_status dsv4_topk_rows(const float *scores_dev, int64_t ld, const int32_t *n_dev, int32_t n_rows,
                           int32_t max_n, int32_t k, int32_t *out_dev, void *ws_dev, int64_t ws_bytes,
                           void *stream) {
    if (n_rows < 0 || max_n < 0 || max_n > (1 << 30) || k < 1 || k > 2048 || ld < max_n) return DSV4_ERR_INVALID_ARG;
    if (n_rows == 0) return DSV4_OK;
    if (!scores_dev || !n_dev || !out_dev) return DSV4_ERR_INVALID_ARG;
    if (!ws_dev || ((uintptr_t)ws_dev & 255)) return DSV4_ERR_WORKSPACE;
    Lay L;
    rows_layout(k, &L);
    IndexWs W;
    const int chunk = n_rows < kMaxGridRows ? n_rows : kMaxGridRows;
    if (index_ws_bytes(L, chunk, max_n, &W, (uint8_t *)ws_dev) > ws_bytes) return DSV4_ERR_WORKSPACE;
    if (W.s_max > kTkMaxSeg) return DSV4_ERR_UNSUPPORTED;
    Timed tm(DSV4_K_TOPK, S(stream));
    for (int r0 = 0; r0 < n_rows; r0 += chunk) {
        const int n = n_rows - r0 < chunk ? n_rows - r0 : chunk;
        const hipError_t e = launch_topk_rows(scores_dev + (int64_t)r0 * ld, ld, n_dev + r0, n, max_n, k, W,
                                              out_dev + (int64_t)r0 * k, S(stream));
        if (e != hipSuccess) return DSV4_ERR_LAUNCH;
    }
    return DSV4_OK;
}

static dsv4_status attend_common(const dsv4_cfg *cfg, const dsv4_cache *cache, int kind, const void *q,
                                 const int32_t *req, const int32_t *pos, const int32_t *cu, const int32_t *pos0,
                                 int n_seq, int nq, const int32_t *topk, const void *win, const float *sinks,
                                 void *out, int policy, bool prefill, void *stream) {
    Lay L;
    dsv4_status st = make_layout(cfg, kind, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, kind)) != DSV4_OK) return st;
    if (nq < 0 || n_seq < 0) return DSV4_ERR_INVALID_ARG;
    if (policy != DSV4_POLICY_AUTO && policy != DSV4_POLICY_HI && policy != DSV4_POLICY_LO)
        return DSV4_ERR_INVALID_ARG;
    if (nq == 0) return DSV4_OK;
    if (!q || !sinks || !out || !req) return DSV4_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out)) return DSV4_ERR_INVALID_ARG;
    if (prefill && (!cu || !pos0 || n_seq == 0 || (L.W > 0 && !win))) return DSV4_ERR_INVALID_ARG;
    if (!prefill && !pos) return DSV4_ERR_INVALID_ARG;
    if (kind == DSV4_CSA && !topk) return DSV4_ERR_INVALID_ARG;
    AttnArgs A;
    memset(&A, 0, sizeof(A));
    A.L = L;
    A.C = *cache;
    A.q = q;
    A.req = req;
    A.pos = pos;
    A.cu = cu;
    A.pos0 = pos0;
    A.n_seq = n_seq;
    A.topk = topk;
    A.win = (const uint8_t *)win;
    A.sinks = sinks;
    A.out = out;
    A.nq = nq;
    A.nhg = (L.H + 15) / 16;
    if (L.kv_store == DSV4_STORE_FP32) {           // fp32 records: one kernel for both policies
        Timed tm(DSV4_K_ATTEND, S(stream));
        return hip_status(launch_attend_f32(A, kind == DSV4_CSA, prefill, S(stream)));
    }
    if (attend_lds_max(L, attend_list_max(L, *cache, kind == DSV4_CSA)) > kLdsMax) return DSV4_ERR_UNSUPPORTED;
    const bool hi = pick_hi(policy, nq, A.nhg);
    Timed tm(DSV4_K_ATTEND, S(stream));
    return hip_status(launch_attend(A, kind == DSV4_CSA, prefill, hi, S(stream)));
}

dsv4_status dsv4_csa_attend_decode(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                   const int32_t *req_dev, const int32_t *pos_dev, const int32_t *topk_dev,
                                   const float *sinks_dev, void *out, int32_t B, int32_t policy, void *stream) {
    return attend_common(cfg, cache, DSV4_CSA, q, req_dev, pos_dev, nullptr, nullptr, 0, B, topk_dev, nullptr,
                         sinks_dev, out, policy, false, stream);
}

dsv4_status dsv4_hca_attend_decode(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                   const int32_t *req_dev, const int32_t *pos_dev, const float *sinks_dev,
                                   void *out, int32_t B, int32_t policy, void *stream) {
    return attend_common(cfg, cache, DSV4_HCA, q, req_dev, pos_dev, nullptr, nullptr, 0, B, nullptr, nullptr,
                         sinks_dev, out, policy, false, stream);
}

dsv4_status dsv4_csa_attend_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                    const int32_t *cu_seqlens_dev, const int32_t *req_dev, const int32_t *pos0_dev,
                                    int32_t n_seq, int32_t total_tokens, const int32_t *topk_dev,
                                    const void *win_dev, const float *sinks_dev, void *out, void *stream) {
    return attend_common(cfg, cache, DSV4_CSA, q, req_dev, nullptr, cu_seqlens_dev, pos0_dev, n_seq, total_tokens,
                         topk_dev, win_dev, sinks_dev, out, DSV4_POLICY_HI, true, stream);
}

dsv4_status dsv4_hca_attend_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                    const int32_t *cu_seqlens_dev, const int32_t *req_dev, const int32_t *pos0_dev,
                                    int32_t n_seq, int32_t total_tokens, const void *win_dev,
                                    const float *sinks_dev, void *out, void *stream) {
    return attend_common(cfg, cache, DSV4_HCA, q, req_dev, nullptr, cu_seqlens_dev, pos0_dev, n_seq, total_tokens,
                         nullptr, win_dev, sinks_dev, out, DSV4_POLICY_HI, true, stream);
}

dsv4_status dsv4_cache_write_entries(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t target,
                                     const int32_t *req_dev, const int32_t *entry_dev, int32_t n,
                                     const float *values_dev, void *stream) {
    if (!cache) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, cache->kind, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, cache->kind)) != DSV4_OK) return st;
    if (target != DSV4_TARGET_ENTRY && target != DSV4_TARGET_INDEX_KEY) return DSV4_ERR_INVALID_ARG;
    if (target == DSV4_TARGET_INDEX_KEY && cache->kind != DSV4_CSA) return DSV4_ERR_INVALID_ARG;
    if (n < 0) return DSV4_ERR_INVALID_ARG;
    if (n == 0) return DSV4_OK;
    if (!req_dev || !entry_dev || !values_dev) return DSV4_ERR_INVALID_ARG;
    return hip_status(launch_write_entries(L, *cache, target, req_dev, entry_dev, n, values_dev, S(stream)));
}

dsv4_status dsv4_cache_read_entries(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t target,
                                    const int32_t *req_dev, const int32_t *idx_dev, int32_t n, void *out_dev,
                                    int32_t out_dtype, void *stream) {
    if (!cache) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, cache->kind, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, cache->kind)) != DSV4_OK) return st;
    if (target != DSV4_TARGET_ENTRY && target != DSV4_TARGET_INDEX_KEY && target != DSV4_TARGET_WINDOW)
        return DSV4_ERR_INVALID_ARG;
    if (target == DSV4_TARGET_INDEX_KEY && cache->kind != DSV4_CSA) return DSV4_ERR_INVALID_ARG;
    if (out_dtype != DSV4_DT_F32 && out_dtype != DSV4_DT_F64) return DSV4_ERR_INVALID_ARG;
    if (n < 0) return DSV4_ERR_INVALID_ARG;
    if (n == 0) return DSV4_OK;
    if (!req_dev || !idx_dev || !out_dev || !aligned16(out_dev)) return DSV4_ERR_INVALID_ARG;
    return hip_status(launch_read_entries(L, *cache, target, req_dev, idx_dev, n, out_dev,
                                          out_dtype == DSV4_DT_F64, S(stream)));
}

dsv4_status dsv4_state_write_tokens(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t req, int32_t pos0,
                                    int32_t n, const void *kv, const void *gate, const void *kI, const void *gI,
                                    void *stream) {
    if (!cache) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, cache->kind, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, cache->kind)) != DSV4_OK) return st;
    if (req < 0 || req >= cache->n_req || pos0 < 0 || n < 0) return DSV4_ERR_INVALID_ARG;
    if (n == 0) return DSV4_OK;
    if (!kv || !gate) return DSV4_ERR_INVALID_ARG;
    if (cache->kind == DSV4_CSA && (!kI || !gI)) return DSV4_ERR_INVALID_ARG;
    return hip_status(launch_state_tokens(L, *cache, req, pos0, n, kv, gate, kI, gI, S(stream)));
}

dsv4_status dsv4_cache_dump_bytes(const dsv4_cfg *cfg, int32_t kind, int32_t n_tokens, int64_t *out) {
    if (!out || n_tokens < 1) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, kind, &L);
    if (st != DSV4_OK) return st;
    *out = cache_dump_bytes(L, (n_tokens + kBlockTokens - 1) / kBlockTokens);
    return DSV4_OK;
}

static dsv4_status cache_xfer(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t req, int32_t n_tokens,
                              const void *buf, int64_t buf_bytes, bool to_buf, void *stream) {
    if (!cache) return DSV4_ERR_INVALID_ARG;
    Lay L;
    dsv4_status st = make_layout(cfg, cache->kind, &L);
    if (st != DSV4_OK) return st;
    if ((st = check_cache(L, cache, cache->kind)) != DSV4_OK) return st;
    if (req < 0 || req >= cache->n_req || n_tokens < 1) return DSV4_ERR_INVALID_ARG;
    const int nb = (n_tokens + kBlockTokens - 1) / kBlockTokens;
    if (nb > cache->max_blocks) return DSV4_ERR_INVALID_ARG;
    if (!buf || ((uintptr_t)buf & 15) || buf_bytes < cache_dump_bytes(L, nb)) return DSV4_ERR_INVALID_ARG;
    return hip_status(launch_cache_xfer(L, *cache, req, nb, (uint8_t *)buf, to_buf, S(stream)));
}

dsv4_status dsv4_cache_dump(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t req, int32_t n_tokens,
                            void *buf_dev, int64_t buf_bytes, void *stream) {
    return cache_xfer(cfg, cache, req, n_tokens, buf_dev, buf_bytes, true, stream);
}

dsv4_status dsv4_cache_load(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t req, int32_t n_tokens,
                            const void *buf_dev, int64_t buf_bytes, void *stream) {
    return cache_xfer(cfg, cache, req, n_tokens, buf_dev, buf_bytes, false, stream);
}

static dsv4_status proj_shape(const dsv4_cfg *cfg, int32_t groups, int32_t rank, int32_t hidden) {
    if (!cfg) return DSV4_ERR_INVALID_ARG;
    const int H = cfg->n_heads, d = cfg->d;
    if (H < 1 || d < 1 || groups < 1 || H % groups) return DSV4_ERR_INVALID_ARG;
    const int64_t gd = (int64_t)(H / groups) * d;
    if (gd % 32 || gd > (1 << 24)) return DSV4_ERR_INVALID_ARG;
    if (rank < 128 || rank % 128 || hidden < 128 || hidden % 128) return DSV4_ERR_INVALID_ARG;
    if ((int64_t)groups * rank > (1 << 24)) return DSV4_ERR_INVALID_ARG;
    return DSV4_OK;
}

dsv4_status dsv4_out_proj_pack(const dsv4_cfg *cfg, int32_t groups, int32_t rank, int32_t hidden, const void *w1,
                               const void *w2, void *w1p, void *w2p, void *stream) {
    dsv4_status st = proj_shape(cfg, groups, rank, hidden);
    if (st != DSV4_OK) return st;
    if (!w1 || !w2 || !w1p || !w2p) return DSV4_ERR_INVALID_ARG;
    if (((uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)w1p | (uintptr_t)w2p) & 15) return DSV4_ERR_INVALID_ARG;
    const int gd = cfg->n_heads / groups * cfg->d;
    hipError_t e = launch_pack_b((const uint16_t *)w1, (uint16_t *)w1p, groups, rank, gd, S(stream));
    if (e != hipSuccess) return DSV4_ERR_LAUNCH;
    return hip_status(launch_pack_b((const uint16_t *)w2, (uint16_t *)w2p, 1, hidden, groups * rank, S(stream)));
}

dsv4_status dsv4_out_proj(const dsv4_cfg *cfg, int32_t groups, int32_t rank, int32_t hidden, const void *o,
                          const void *w1, const void *w2, void *y_ws, void *out, int32_t T, void *stream) {
    dsv4_status st = proj_shape(cfg, groups, rank, hidden);
    if (st != DSV4_OK) return st;
    const int H = cfg->n_heads, d = cfg->d;
    if (T < 0) return DSV4_ERR_INVALID_ARG;
    if (cfg->act_dtype != DSV4_DT_BF16) return DSV4_ERR_UNSUPPORTED;
    if (T == 0) return DSV4_OK;
    if (!o || !w1 || !w2 || !y_ws || !out) return DSV4_ERR_INVALID_ARG;
    if (((uintptr_t)o | (uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)y_ws | (uintptr_t)out) & 15)
        return DSV4_ERR_INVALID_ARG;
    if ((T + 31) / 32 > 65535) return DSV4_ERR_UNSUPPORTED;
    Timed tm(DSV4_K_PROJ, S(stream));
    return hip_status(launch_out_proj((const uint16_t *)o, T, H, d, groups, rank, hidden, (const uint16_t *)w1,
                                      (const uint16_t *)w2, (uint16_t *)y_ws, out, 0, S(stream)));
}

static bool mx_shape_ok(int64_t M, int64_t N, int64_t K) {
    return M >= 0 && M <= (1 << 20) && N >= 16 && N <= (1 << 20) && N % 16 == 0 && K >= 128 && K <= (1 << 20) &&
           K % 128 == 0;
}

dsv4_status dsv4_mx_pack_bytes(int32_t rows, int32_t K, int32_t fp8, int64_t *out) {
    if (!out || rows < 0 || rows > (1 << 20) || K < 128 || K > (1 << 20) || K % 128) return DSV4_ERR_INVALID_ARG;
    *out = mx_pack_bytes(rows, K, fp8 != 0);
    return DSV4_OK;
}

dsv4_status dsv4_mx_pack_weight(const void *w, int32_t N, int32_t K, void *wp, int64_t wp_bytes, void *stream) {
    if (!mx_shape_ok(0, N, K) || !w || !wp) return DSV4_ERR_INVALID_ARG;
    if (((uintptr_t)w | (uintptr_t)wp) & 15) return DSV4_ERR_INVALID_ARG;
    if (wp_bytes < mx_pack_bytes(N, K, false)) return DSV4_ERR_WORKSPACE;
    return hip_status(launch_mx_quant((const uint16_t *)w, N, K, false, (uint8_t *)wp, S(stream)));
}

static dsv4_status mx_linear(const void *x, int M, int K, const void *wp, int N, uint8_t *ws, void *out, int ldc,
                             int c_f32, hipStream_t s) {
    hipError_t e = launch_mx_quant((const uint16_t *)x, M, K, true, ws, s);
    if (e != hipSuccess) return DSV4_ERR_LAUNCH;
    return hip_status(launch_mx_gemm(ws, (const uint8_t *)wp, M, N, K, out, ldc, c_f32, s));
}

dsv4_status dsv4_mx_linear(const void *x, int32_t M, int32_t K, const void *wp, int32_t N, void *ws,
                           int64_t ws_bytes, void *out, int32_t out_dtype, void *stream) {
    if (!mx_shape_ok(M, N, K)) return DSV4_ERR_INVALID_ARG;
    if (out_dtype != DSV4_DT_F32 && out_dtype != DSV4_DT_BF16) return DSV4_ERR_INVALID_ARG;
    if (M == 0) return DSV4_OK;
    if (!x || !wp || !out) return DSV4_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)wp) & 15) return DSV4_ERR_INVALID_ARG;
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < mx_pack_bytes(M, K, true)) return DSV4_ERR_WORKSPACE;
    if ((M + 127) / 128 > 65535) return DSV4_ERR_UNSUPPORTED;
    Timed tm(DSV4_K_MX, S(stream));
    return mx_linear(x, M, K, wp, N, (uint8_t *)ws, out, N, out_dtype == DSV4_DT_F32, S(stream));
}

static int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

dsv4_status dsv4_index_q_proj_ws_bytes(const dsv4_cfg *cfg, int32_t T, int32_t hidden, int32_t dc, int64_t *out) {
    if (!cfg || !out || T < 0) return DSV4_ERR_INVALID_ARG;
    const int64_t nq = (int64_t)cfg->idx_heads * cfg->idx_dim;
    if (!mx_shape_ok(T, dc, hidden) || !mx_shape_ok(T, nq, dc)) return DSV4_ERR_INVALID_ARG;
    const int64_t a = mx_pack_bytes(T, hidden, true), b = mx_pack_bytes(T, dc, true);
    *out = round256((int64_t)T * dc * 2) + (a > b ? a : b);
    return DSV4_OK;
}

dsv4_status dsv4_index_q_proj(const dsv4_cfg *cfg, const void *x, int32_t T, int32_t hidden, int32_t dc,
                              const void *wdq_p, const void *wuq_p, void *ws, int64_t ws_bytes, void *qI,
                              void *stream) {
    int64_t need = 0;
    dsv4_status st = dsv4_index_q_proj_ws_bytes(cfg, T, hidden, dc, &need);
    if (st != DSV4_OK) return st;
    if (cfg->act_dtype != DSV4_DT_F32 && cfg->act_dtype != DSV4_DT_BF16) return DSV4_ERR_INVALID_ARG;
    if (T == 0) return DSV4_OK;
    if (!x || !wdq_p || !wuq_p || !qI) return DSV4_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)wdq_p | (uintptr_t)wuq_p) & 15) return DSV4_ERR_INVALID_ARG;
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return DSV4_ERR_WORKSPACE;
    if ((T + 127) / 128 > 65535) return DSV4_ERR_UNSUPPORTED;
    const int nq = cfg->idx_heads * cfg->idx_dim;
    uint8_t *cq = (uint8_t *)ws, *act = cq + round256((int64_t)T * dc * 2);
    Timed tm(DSV4_K_MX, S(stream));
    st = mx_linear(x, T, hidden, wdq_p, dc, act, cq, dc, 0, S(stream));
    if (st != DSV4_OK) return st;
    return mx_linear(cq, T, dc, wuq_p, nq, act, qI, nq, cfg->act_dtype == DSV4_DT_F32, S(stream));
}

dsv4_status dsv4_kv_proj_ws_bytes(const dsv4_cfg *cfg, int32_t T, int32_t hidden, int64_t *out) {
    if (!cfg || !out || T < 0) return DSV4_ERR_INVALID_ARG;
    if (!mx_shape_ok(T, 16, hidden)) return DSV4_ERR_INVALID_ARG;
    *out = mx_pack_bytes(T, hidden, true);
    return DSV4_OK;
}

dsv4_status dsv4_kv_proj(const dsv4_cfg *cfg, int32_t kind, const void *x, int32_t T, int32_t hidden,
                         const void *wkv_p, const void *wg_p, const void *wki_p, const void *wgi_p, const void *ww_p,
                         void *kv, void *gate, void *kI, void *gI, float *w, void *ws, int64_t ws_bytes,
                         void *stream) {
    Lay L;
    dsv4_status st = make_layout(cfg, kind, &L);
    if (st != DSV4_OK) return st;
    if (T < 0 || !mx_shape_ok(T, L.d, hidden)) return DSV4_ERR_INVALID_ARG;
    const bool csa = kind == DSV4_CSA;
    if (csa ? (!wki_p || !wgi_p || !kI || !gI) : (wki_p || wgi_p || kI || gI || ww_p || w)) return DSV4_ERR_INVALID_ARG;
    if ((ww_p == nullptr) != (w == nullptr)) return DSV4_ERR_INVALID_ARG;
    if (ww_p && L.HI % 16) return DSV4_ERR_UNSUPPORTED;          // the products take whole 16-row blocks
    if (T == 0) return DSV4_OK;
    if (!x || !wkv_p || !wg_p || !kv || !gate) return DSV4_ERR_INVALID_ARG;
    const void *ptrs[] = {x, wkv_p, wg_p, wki_p, wgi_p, ww_p, kv, gate, kI, gI, w};
    for (const void *q : ptrs)
        if ((uintptr_t)q & 15) return DSV4_ERR_INVALID_ARG;
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < mx_pack_bytes(T, hidden, true)) return DSV4_ERR_WORKSPACE;
    if ((T + 127) / 128 > 65535) return DSV4_ERR_UNSUPPORTED;
    const int of32 = L.act == DSV4_DT_F32;
    hipStream_t s = S(stream);
    Timed tm(DSV4_K_MX, s);
    // x quantised to MXFP8 once, then one product per projection
    uint8_t *act = (uint8_t *)ws;
    if (launch_mx_quant((const uint16_t *)x, T, hidden, true, act, s) != hipSuccess) return DSV4_ERR_LAUNCH;
    struct P { const void *wp; void *out; int n; int f32; } prods[] = {
        {wkv_p, kv, L.d, of32}, {wg_p, gate, L.d, of32}, {wki_p, kI, L.dI, of32}, {wgi_p, gI, L.dI, of32},
        {ww_p, w, L.HI, 1}};
    for (const P &p : prods) {
        if (!p.wp) continue;
        if (launch_mx_gemm(act, (const uint8_t *)p.wp, T, p.n, hidden, p.out, p.n, p.f32, s) != hipSuccess)
            return DSV4_ERR_LAUNCH;
    }
    return DSV4_OK;
}

dsv4_status dsv4_timer_enable(int32_t kernel_id, int32_t on) {
    if (kernel_id < 0 || kernel_id >= DSV4_K_COUNT) return DSV4_ERR_INVALID_ARG;
    g_timers[kernel_id].on = on != 0;
    return DSV4_OK;
}

dsv4_status dsv4_timer_read(int32_t kernel_id, int32_t reset, double *total_ms, int64_t *count) {
    if (kernel_id < 0 || kernel_id >= DSV4_K_COUNT || !total_ms || !count) return DSV4_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_timer_mu);
    TimerSlot &t = g_timers[kernel_id];
    dsv4_status st = DSV4_OK;
    for (auto &pr : t.pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(pr.second) != hipSuccess || hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
            st = DSV4_ERR_HIP;
        t.total_ms += ms;
        t.count += 1;
        hipEventDestroy(pr.first);
        hipEventDestroy(pr.second);
    }
    t.pending.clear();
    *total_ms = t.total_ms;
    *count = t.count;
    if (reset) {
        t.total_ms = 0.0;
        t.count = 0;
    }
    return st;
}

}  // extern "C"
