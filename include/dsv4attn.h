/*
 * dsv4attn.h -- C ABI of libdsv4attn.so: CSA/HCA compressed attention
 * (block compressor, lightning-indexer scoring, top-k, single-KV-head MQA with
 * a raw sliding window and per-head sink) for AMD MI355X (gfx950).
 *
 * Sources for what each call computes (pages as published, sections named):
 *  - vastsailsolution.com article on the DeepSeek-V4 report: section
 *    "CSA -- compressed sparse attention" (data flow: compressor every 4
 *    tokens, lightning indexer producing index keys and scores, top-k of 512 /
 *    1024 entries, MQA over them plus 128 raw window tokens), section "HCA --
 *    heavily compressed attention" (compressor every 128 tokens, no indexer,
 *    dense MQA), and the paragraphs after it: sliding window of the last 128
 *    raw tokens and a learnable per-head sink logit added to the softmax
 *    denominator; RoPE on only the last 64 dims of query and KV; KV cache with
 *    BF16 RoPE dims and FP8 for the rest; a per-request "state cache" (window
 *    tokens plus the not-yet-compressible tail) and a "classic cache" whose
 *    blocks cover lcm(4,128)=128 raw tokens = 32 CSA entries + 1 HCA entry.
 *  - rqlyzj.com "three paradigm innovations" article, section 01: the
 *    overlapping compression windows and the learned weighted merge of a
 *    block's tokens (no decompression).
 *  - hwcomputing.csdn.net "DeepSeek V4 底层逻辑全解析", section 二 (CSA in three
 *    steps with overlap; Top-512 Flash / Top-1024 Pro) and section 四 (batch
 *    invariance: no split-KV; two decode kernels that agree bit for bit).
 *  - m.youleyou.com article on batch invariance, section "what was
 *    sacrificed": split-KV and split-K are dropped; attention decode has one
 *    kernel for a saturated GPU and one for an unsaturated GPU with identical
 *    results.
 *
 * Conventions (all entry points):
 *  - Every function returns a dsv4_status.  Arguments are validated on the
 *    host before anything is launched; a failed check launches nothing.
 *  - The caller owns all memory.  Pointers named *_dev are device pointers
 *    (hipMalloc / torch CUDA tensors); the library never allocates device
 *    memory and never synchronises.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream) in call order.
 *  - Integer index arrays (req, pos, cu_seqlens, block tables, top-k lists)
 *    are device-resident int32.  Their values are not visible to the host:
 *    kernels skip (and leave untouched) any item whose request, position or
 *    block id is out of range instead of faulting.
 *  - Activations (kv, gate, kI, gI, q, qI, out) are row-major in the dtype
 *    given by cfg->act_dtype (bf16 or fp32).  w and sinks are fp32.
 *  - Device pointers must be 16-byte aligned; pools 256-byte aligned.
 *  - The library keeps no state between calls (the optional kernel timers
 *    below excepted).  Results are bitwise deterministic and independent of
 *    the batch (size, order, co-batched requests) and of the decode policy.
 */
#ifndef DSV4ATTN_H
#define DSV4ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dsv4_status;
#define DSV4_OK 0
#define DSV4_ERR_INVALID_ARG 1   /* bad pointer, size, or configuration value */
#define DSV4_ERR_UNSUPPORTED 2   /* valid but not built (e.g. a head dim without a kernel) */
#define DSV4_ERR_WORKSPACE 3     /* workspace missing or smaller than dsv4_workspace_bytes */
#define DSV4_ERR_LAUNCH 4        /* a kernel launch failed (hipGetLastError) */
#define DSV4_ERR_HIP 5           /* another HIP runtime error */

/* layer kinds */
#define DSV4_CSA 0
#define DSV4_HCA 1

/* storage formats */
#define DSV4_STORE_FP32 0        /* records / index keys as fp32 (reference-precision mode: plain
                                    fp32 kernels, both decode policies run the same one) */
#define DSV4_STORE_FP8 1         /* records: E4M3 non-RoPE dims + one fp32 scale + BF16 RoPE dims;
                                    index keys / queries: E4M3 + one fp32 scale per row */
#define DSV4_STORE_MXFP4 2       /* index keys / queries only: OCP MXFP4 -- E2M1 codes, one E8M0
                                    (power-of-two) scale per 32 consecutive dims */

/* activation dtypes (DSV4_DT_F64: read-back output only) */
#define DSV4_DT_F32 0
#define DSV4_DT_BF16 1
#define DSV4_DT_F64 2

/* decode kernel policy (the two kernels give bitwise identical results) */
#define DSV4_POLICY_AUTO 0
#define DSV4_POLICY_HI 1         /* for a saturated GPU: d = 512: per (query, four 16-head groups)
                                    one workgroup of 8 waves (head group x half of the dims) taking
                                    the record subsets in turn, each record loaded and converted to
                                    bf16 once per workgroup; other d: per (query, 16-head group) 2
                                    waves.  Prefill always runs this layout. */
#define DSV4_POLICY_LO 2         /* for an unsaturated GPU: per (query, 16-head group) one workgroup
                                    of 8 waves (record subset x half of the dims; lists up to 2048
                                    records at d = 512) or 4 waves (one per subset, over all dims) */

/* cache-write / read-back targets */
#define DSV4_TARGET_ENTRY 0
#define DSV4_TARGET_INDEX_KEY 1
#define DSV4_TARGET_WINDOW 2     /* read-back only: the window-ring record of a position */

/* Raw tokens covered by one classic-cache block: lcm(4, 128). */
#define DSV4_BLOCK_TOKENS 128

/*
 * Layer configuration.  Defaults in brackets are the V4-Pro shape.
 *   d            head dim of query and the single KV head                 [512]
 *   d_rope       RoPE dims, the LAST d_rope of d (pairs (2i, 2i+1),
 *                angle pos * rope_base^(-2i/d_rope))                      [64]
 *   n_heads      query heads sharing the KV head, multiple of 16           [128]
 *   window       raw sliding window W: query t sees tokens t-W+1 .. t      [128]
 *   m_csa        CSA stride m (entries per block 128/m)                    [4]
 *   w_csa        CSA compression window: entry j pools tokens
 *                [m*j - (w_csa - m), m*j + m - 1] (clipped at 0);
 *                w_csa is m (no overlap) or 2m (overlap with the previous block) [8]
 *   m_hca        HCA stride m' = window (no overlap)                       [128]
 *   idx_heads    lightning-indexer heads (<= 64)                           [64]
 *   idx_dim      indexer head dim (multiple of 32, <= 128)                 [128]
 *   topk         entries kept per CSA query (<= 2048)                      [1024]
 *   kv_store     DSV4_STORE_FP8 (production) or DSV4_STORE_FP32
 *   idx_store    DSV4_STORE_FP8 (production), DSV4_STORE_MXFP4 (the indexer in
 *                FP4: rqlyzj.com section on FP4 QAT -- the indexer's QK
 *                activations cached, loaded and multiplied in FP4;
 *                hwcomputing.csdn.net section 二, CSA step 2) or DSV4_STORE_FP32
 *   act_dtype    DSV4_DT_BF16 or DSV4_DT_F32 for kv/gate/kI/gI/q/qI/out
 *   rope_base    [10000]
 *   softmax_scale tau in tau * q.k                                         [1/sqrt(d)]
 * Built head shapes: (d, d_rope) = (512, 64) and (64, 16).
 */
typedef struct dsv4_cfg {
    int32_t d, d_rope, n_heads, window;
    int32_t m_csa, w_csa, m_hca;
    int32_t idx_heads, idx_dim, topk;
    int32_t kv_store, idx_store, act_dtype;
    float rope_base, softmax_scale;
} dsv4_cfg;

/*
 * One layer's cache (a CSA layer and an HCA layer each have one; they may
 * share block_table).  All memory is caller-allocated, sizes from
 * dsv4_get_layout.
 *   kind         DSV4_CSA or DSV4_HCA
 *   entries      classic cache: [n_blocks][entry_block_bytes]; block b holds the
 *                128/m entries of the 128 raw tokens mapped to b, entry j of a
 *                request at slot j mod (128/m) of block block_table[r][j*m/128]
 *   index_keys   CSA only (NULL for HCA): [n_blocks][index_block_bytes], the
 *                compressed index keys laid out like `entries`
 *   state        state cache: [n_req][state_bytes] -- the W most recent raw
 *                tokens as stored records (ring, slot = pos mod W) and the raw
 *                tail tokens still needed by the compressor (ring of
 *                pending_slots raw fp32 tokens, slot = pos mod pending_slots)
 *   block_table  device int32 [n_req][max_blocks]: physical block id of the
 *                b-th 128-token span of request r
 */
typedef struct dsv4_cache {
    int32_t kind;
    int32_t n_req, max_blocks, n_blocks;
    void *entries;
    void *index_keys;
    void *state;
    const int32_t *block_table;
} dsv4_cache;

/*
 * Byte layout of one layer's cache.
 *  KV record (DSV4_STORE_FP8): bytes [0, d-d_rope) E4M3 codes of the non-RoPE
 *    dims, then d_rope BF16 values (post-RoPE), then one fp32 scale; the value
 *    of a code c is E4M3(c) * scale.  Padded to record_bytes (multiple of 64).
 *  KV record (DSV4_STORE_FP32): d fp32 values (post-RoPE).
 *  Index block: entries_per_block keys of index_key_bytes (E4M3 or fp32)
 *    back to back, then (FP8 only) entries_per_block fp32 scales.
 *  Index block (DSV4_STORE_MXFP4): entries_per_block keys of idx_dim/2 bytes
 *    (dim 2i in the low nibble of byte i), then per key one 32-bit word of
 *    E8M0 bytes, byte b the scale of dims [32b, 32b+32): the value of dim i
 *    is E2M1(code_i) * 2^(byte - 127).
 *  State (per request): window ring of `window` records at offset 0, pending
 *    ring at pending_offset: pending_slots raw tokens, each
 *    [kv d][gate d][kI idx_dim][gI idx_dim] fp32 (kI, gI for CSA only).
 */
typedef struct dsv4_layout {
    int64_t record_bytes;
    int64_t entries_per_block;
    int64_t entry_block_bytes;
    int64_t index_key_bytes;
    int64_t index_block_bytes;
    int64_t state_bytes;
    int64_t pending_offset;
    int64_t pending_slots;
    int64_t pending_token_floats;
} dsv4_layout;

const char *dsv4_status_string(dsv4_status s);

/* Validate cfg for a layer kind and fill *out.  DSV4_ERR_INVALID_ARG for values
 * outside the documented ranges, DSV4_ERR_UNSUPPORTED for a head shape or
 * storage mode without kernels. */
dsv4_status dsv4_get_layout(const dsv4_cfg *cfg, int32_t kind, dsv4_layout *out);

/* Workspace for dsv4_index_topk_{decode,prefill}: n_queries queries whose
 * visible entry count is at most max_entries.  For the prefill call the
 * library processes queries in groups that fit the workspace given, so any
 * size >= dsv4_workspace_bytes(cfg, n_queries = 1, ...) is accepted. */
dsv4_status dsv4_workspace_bytes(const dsv4_cfg *cfg, int32_t n_queries, int32_t max_entries,
                                 int64_t *out);

/* Where dsv4_index_topk_decode (prefill = 0) or dsv4_index_topk_prefill
 * (prefill = 1) leaves the indexer scores I[j] in its workspace, for reading
 * them back (tests, analysis): score j of query i -- i < n_queries, j below
 * the query's visible entry count -- is the fp32 at byte
 * *offset + 4 * (i * *ld + j) of ws_dev, valid until the workspace is used
 * again.  n_queries is the call's B (decode) or total_tokens (prefill); for
 * the prefill call this holds when its workspace fits all its queries at once
 * (ws_bytes >= dsv4_workspace_bytes(cfg, total_tokens, max_blocks*128/m)).
 * Caller-owned outputs; nothing is launched.  DSV4_ERR_INVALID_ARG for null
 * outputs, n_queries outside [1, 65535], prefill not 0 or 1, or an invalid
 * cfg or cache. */
dsv4_status dsv4_index_scores_layout(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t n_queries,
                                     int32_t prefill, int64_t *offset, int64_t *ld);

/*
 * Append + compress, decode: one new token per request.
 * Token b (position pos_dev[b], request req_dev[b]) is RoPE-rotated at its
 * position, stored into the window ring, and pushed into the pending ring.  If
 * it completes a block of the layer's stride (pos+1 divisible by m), the entry
 * of that block is formed: per channel c, softmax over the block's tokens s of
 * gate[s][c], weighted sum of kv[s][c]; RoPE at the block's last token; stored
 * (FP8/BF16).  For a CSA layer the index key is formed the same way from
 * (kI, gI), without RoPE.  Sources: vastsailsolution.com CSA/HCA sections and
 * state/classic cache paragraph; rqlyzj.com section 01 (overlap, weighted
 * merge).
 *   kv, gate   [B][d] act dtype;  kI, gI [B][idx_dim] act dtype (CSA) or NULL (HCA)
 *   req_dev    [B] request rows of the cache; pos_dev [B] new token positions
 * Requests in one call must be distinct.  Run before the attention of the
 * same step: the new token is visible to its own query.
 */
dsv4_status dsv4_compress_kv_decode(const dsv4_cfg *cfg, const dsv4_cache *cache,
                                    const void *kv, const void *gate, const void *kI,
                                    const void *gI, const int32_t *req_dev,
                                    const int32_t *pos_dev, int32_t B, void *stream);

/*
 * Append + compress, prefill of a chunk per sequence (varlen).  Sequence i has
 * tokens cu_seqlens_dev[i] .. cu_seqlens_dev[i+1]-1 of the packed inputs,
 * request req_dev[i], first position pos0_dev[i] (= tokens already cached).
 * Entries completed inside the chunk are formed exactly as in decode (bitwise
 * identical to appending the same tokens one at a time); earlier tail tokens
 * come from the state cache.  Afterwards the state cache holds the chunk's
 * last window / tail tokens.
 *   win_out_dev (required) receives the window records the chunk's queries
 *   need, as stored records: for sequence i, (window + chunk_len_i) records
 *   starting at record (cu_seqlens[i] + i*window) -- first the `window`
 *   records of positions pos0-window .. pos0-1 (from the state cache; slots
 *   for negative positions are left unspecified), then the chunk's tokens.
 *   Size: (total_tokens + n_seq*window) * record_bytes.  Pass it to the
 *   *_attend_prefill calls of the same chunk.
 */
dsv4_status dsv4_compress_kv_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache,
                                     const void *kv, const void *gate, const void *kI,
                                     const void *gI, const int32_t *cu_seqlens_dev,
                                     const int32_t *req_dev, const int32_t *pos0_dev,
                                     int32_t n_seq, int32_t total_tokens, void *win_out_dev,
                                     void *stream);

/*
 * Lightning indexer + top-k, decode (CSA).  For query b at position t =
 * pos_dev[b] over the visible entries j < floor((t+1)/m):
 *   I[j] = sum_h w[b][h] * max(0, qI[b][h] . kI_j)
 * with qI quantised like the index keys (E4M3 with one scale per (query,
 * head), or MXFP4 with one per (query, head, 32 dims)),
 * then the min(k, N) largest I by (score desc, index asc), written ascending
 * to topk_dev[b][0..k), padded with -1.  Sources: vastsailsolution.com CSA
 * section (indexer: query projected into ReLU index heads scored against the
 * compressed index keys; top-k); xiaoyuzhoufm.com 1.1 (CSA applies DSA).
 *   qI [B][idx_heads][idx_dim] act dtype, 16-byte aligned (else
 *   DSV4_ERR_INVALID_ARG);  w_dev [B][idx_heads] fp32 (NULL = all ones)
 *   ws_dev / ws_bytes: workspace of at least
 *   dsv4_workspace_bytes(cfg, B, max_blocks*128/m).
 */
dsv4_status dsv4_index_topk_decode(const dsv4_cfg *cfg, const dsv4_cache *cache,
                                   const void *qI, const float *w_dev, const int32_t *req_dev,
                                   const int32_t *pos_dev, int32_t B, int32_t *topk_dev,
                                   void *ws_dev, int64_t ws_bytes, void *stream);

/*
 * dsv4_index_topk_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with the workspace taken
 * from a library-held device array of DSV4_NOALLOC_SCRATCH_BYTES per GPU
 * (each GPU the library runs on keeps its copy until the process ends).  It
 * calls no allocating routine.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  DSV4_ERR_WORKSPACE when the call would need
 * more than the array (dsv4_workspace_bytes(cfg, B, max_blocks*128/m) >
 * DSV4_NOALLOC_SCRATCH_BYTES); nothing is launched then.
 */
#define DSV4_NOALLOC_SCRATCH_BYTES (32 << 20)
dsv4_status dsv4_index_topk_decode_noalloc(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *qI,
                                           const float *w_dev, const int32_t *req_dev, const int32_t *pos_dev,
                                           int32_t B, int32_t *topk_dev, void *stream);

/* Same for the packed queries of a prefill chunk (positions pos0 + offset);
 * qI is [total_tokens][idx_heads][idx_dim] (16-byte aligned), topk_dev is
 * [total_tokens][k]. */
dsv4_status dsv4_index_topk_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache,
                                    const void *qI, const float *w_dev,
                                    const int32_t *cu_seqlens_dev, const int32_t *req_dev,
                                    const int32_t *pos0_dev, int32_t n_seq, int32_t total_tokens,
                                    int32_t *topk_dev, void *ws_dev, int64_t ws_bytes,
                                    void *stream);

/*
 * Exact top-k selection alone (the selection step of the two calls above), on
 * caller-given fp32 rows.  Row i holds scores_dev[i*ld + j], j < n_dev[i]; its
 * min(k, n) largest elements by (score desc, index asc) are written ascending
 * to out_dev[i][0..k), padded with -1.  NaN ranks below every number, -0
 * equals +0.  A row whose n lies outside [0, max_n] yields all -1.  Sources:
 * vastsailsolution.com CSA section (keep the k most relevant entries).
 *   scores_dev [n_rows][ld] fp32, ld >= max_n;  n_dev [n_rows] int32
 *   k in [1, 2048];  max_n <= 2^30
 *   ws_dev / ws_bytes: at least dsv4_topk_rows_ws_bytes(n_rows, max_n, k),
 *   256-byte aligned.  Returns DSV4_ERR_UNSUPPORTED when max_n exceeds
 *   4,194,304 (1024 segments of 4096).
 */
dsv4_status dsv4_topk_rows_ws_bytes(int32_t n_rows, int32_t max_n, int32_t k, int64_t *out);
dsv4_status dsv4_topk_rows(const float *scores_dev, int64_t ld, const int32_t *n_dev, int32_t n_rows,
                           int32_t max_n, int32_t k, int32_t *out_dev, void *ws_dev, int64_t ws_bytes,
                           void *stream);

/*
 * Sparse CSA attention, decode.  For query b (position t, request r), per head
 * h, over A = {selected entries topk_dev[b][*] (valid, ascending)} followed by
 * the window tokens max(0, t-W+1) .. t:
 *   l_i = tau * qrot_h . v_i,  M = max(z_h, max l_i),
 *   out_h = sum_i e^(l_i-M) v_i / (e^(z_h-M) + sum_i e^(l_i-M))
 * where qrot is q rotated at t on its last d_rope dims and each stored record
 * v_i serves as key and value.  Sources: vastsailsolution.com CSA section
 * (MQA over selected entries + 128 raw window tokens) and sink paragraph.
 *   q [B][n_heads][d] act dtype (un-rotated);  sinks_dev [n_heads] fp32;
 *   out [B][n_heads][d] act dtype;  policy DSV4_POLICY_* (results identical).
 */
dsv4_status dsv4_csa_attend_decode(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                   const int32_t *req_dev, const int32_t *pos_dev,
                                   const int32_t *topk_dev, const float *sinks_dev, void *out,
                                   int32_t B, int32_t policy, void *stream);

/* Dense HCA attention, decode: as above over all complete HCA entries
 * (j < floor((t+1)/m')) followed by the window.  Source: vastsailsolution.com
 * HCA section (no indexer, no top-k, all entries with the window). */
dsv4_status dsv4_hca_attend_decode(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                   const int32_t *req_dev, const int32_t *pos_dev,
                                   const float *sinks_dev, void *out, int32_t B, int32_t policy,
                                   void *stream);

/* Prefill variants: packed queries of a chunk (see dsv4_compress_kv_prefill for
 * cu_seqlens/req/pos0), window records from win_dev (its win_out_dev). */
dsv4_status dsv4_csa_attend_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                    const int32_t *cu_seqlens_dev, const int32_t *req_dev,
                                    const int32_t *pos0_dev, int32_t n_seq, int32_t total_tokens,
                                    const int32_t *topk_dev, const void *win_dev,
                                    const float *sinks_dev, void *out, void *stream);
dsv4_status dsv4_hca_attend_prefill(const dsv4_cfg *cfg, const dsv4_cache *cache, const void *q,
                                    const int32_t *cu_seqlens_dev, const int32_t *req_dev,
                                    const int32_t *pos0_dev, int32_t n_seq, int32_t total_tokens,
                                    const void *win_dev, const float *sinks_dev, void *out,
                                    void *stream);

/*
 * Grouped output projection of the attention output (rqlyzj.com article,
 * section on depth compensation: the heads are split into groups, each
 * group's output is condensed into a short group summary, and the summaries
 * are projected to the model width).  With G = groups, gd = (n_heads/G)*d:
 *   y[t][g][j] = sum_i W1[g][j][i] * o[t][g*gd + i]        (j < rank), rounded to bf16
 *   out[t][n]  = sum_k W2[n][k] * y[t][k]                    (k < G*rank, n < hidden)
 * Each output element is reduced by one wave in a fixed order (k ascending in
 * steps of 32), so a token's result is bitwise independent of T and of the
 * other rows (no split-K).
 *   o     [T][n_heads][d] bf16 (the attention output; cfg->act_dtype must be BF16)
 *   w1p, w2p  the weights as packed by dsv4_out_proj_pack
 *   y_ws  [T][G*rank] bf16 caller-owned workspace (receives the summaries)
 *   out   [T][hidden] bf16
 * n_heads % G == 0, gd % 32 == 0, rank and hidden multiples of 128.
 * DSV4_ERR_UNSUPPORTED for an fp32 act dtype.
 */
dsv4_status dsv4_out_proj(const dsv4_cfg *cfg, int32_t groups, int32_t rank, int32_t hidden, const void *o,
                          const void *w1p, const void *w2p, void *y_ws, void *out, int32_t T, void *stream);

/* Pack the projection weights once (same sizes as the inputs; caller-owned):
 *   w1 [G][rank][gd] bf16 -> w1p,  w2 [hidden][G*rank] bf16 -> w2p.
 * Packed order of a matrix W [N][K]: for each 16-row block n0 and each 32-wide
 * k-step k0, 512 elements in which position 8*l + e (l < 64, e < 8) holds
 * W[n0 + l%16][k0 + 8*(l/16) + e] -- the MFMA operand of that block and step,
 * one contiguous kilobyte. */
dsv4_status dsv4_out_proj_pack(const dsv4_cfg *cfg, int32_t groups, int32_t rank, int32_t hidden, const void *w1,
                               const void *w2, void *w1p, void *w2p, void *stream);

/*
 * Linear layers of the indexer's low-precision path (vastsailsolution.com V4
 * article, CSA section: the indexer's query is projected down to d_c = 1024
 * dims, then up to the multi-head index queries; rqlyzj.com article, FP4 QAT
 * section, and xiaoyuzhoufm.com summary 2.1: the indexer runs in FP4):
 *   out [M][N] = x [M][K] . W [N][K]^T
 * with W stored MXFP4 (E2M1 values, an E8M0 scale 2^(floor(log2 amax) - 2)
 * per 32 consecutive k) and x, bf16, quantised on the way in to MXFP8 (E4M3
 * values, scale 2^(floor(log2 amax) - 8) per 32 k, saturating at 448); the
 * products summed in fp32.  No split-K: a row's output is bitwise the same in
 * any batch.  K a multiple of 128, N of 16; M, N, K at most 2^20.
 *
 * dsv4_mx_pack_bytes  bytes of a packed operand of `rows` rows: fp8 = 0 for
 *                     packed weights (MXFP4), 1 for the activation workspace
 *                     dsv4_mx_linear needs (MXFP8 of x).
 * dsv4_mx_pack_weight quantise and pack W (bf16 [N][K], 16-byte aligned) into
 *                     wp (caller-owned, dsv4_mx_pack_bytes(N, K, 0) bytes):
 *                     per 16-row block and 128-wide k-step, 1 KB in which
 *                     bytes 16l .. 16l+15 hold the E2M1 codes of row l%16,
 *                     k = 32(l/16) .. +31 (value 2i in the low nibble of byte
 *                     i); then per 16-row block and group of four k-steps, 64
 *                     words whose byte j is lane l's scale for k-step 4q+j.
 * dsv4_mx_linear      x bf16 [M][K]; wp packed weights; ws device workspace of
 *                     at least dsv4_mx_pack_bytes(M, K, 1) bytes, 256-byte
 *                     aligned; out [M][N], out_dtype DSV4_DT_F32 or
 *                     DSV4_DT_BF16 (round to nearest even).
 */
dsv4_status dsv4_mx_pack_bytes(int32_t rows, int32_t K, int32_t fp8, int64_t *out);
dsv4_status dsv4_mx_pack_weight(const void *w, int32_t N, int32_t K, void *wp, int64_t wp_bytes, void *stream);
dsv4_status dsv4_mx_linear(const void *x, int32_t M, int32_t K, const void *wp, int32_t N, void *ws,
                           int64_t ws_bytes, void *out, int32_t out_dtype, void *stream);

/*
 * The indexer's query path (same passages): cq = bf16(x . Wdq^T), then
 * qI = cq . Wuq^T, both as dsv4_mx_linear.
 *   x     [T][hidden] bf16
 *   wdq_p Wdq [dc][hidden] packed by dsv4_mx_pack_weight
 *   wuq_p Wuq [idx_heads*idx_dim][dc] packed likewise
 *   qI    [T][idx_heads][idx_dim] in cfg->act_dtype (the input of the index
 *         scoring entry points)
 *   ws    at least dsv4_index_q_proj_ws_bytes bytes, 256-byte aligned
 *         (receives cq, then the MXFP8 activations)
 * hidden and dc multiples of 128, idx_heads*idx_dim a multiple of 16.
 */
dsv4_status dsv4_index_q_proj_ws_bytes(const dsv4_cfg *cfg, int32_t T, int32_t hidden, int32_t dc, int64_t *out);
dsv4_status dsv4_index_q_proj(const dsv4_cfg *cfg, const void *x, int32_t T, int32_t hidden, int32_t dc,
                              const void *wdq_p, const void *wuq_p, void *ws, int64_t ws_bytes, void *qI,
                              void *stream);

/*
 * The per-token projections that feed the compressors and the indexer's head
 * weights, on the same low-precision path as dsv4_index_q_proj (the pages name
 * the indexer's activations FP4 and the prefill configuration "FP4 weights,
 * FP8 activations": rqlyzj.com FP4 QAT section, xiaoyuzhoufm.com 2.1; the
 * compressors take a kv vector and gate logits per token and, for CSA, the
 * indexer's key-side vector and gate: vastsailsolution.com V4 article, CSA and
 * HCA sections).  x is quantised to MXFP8 once; then, each as dsv4_mx_linear
 * (no split-K, a token's outputs bitwise the same in any batch):
 *   kv   = x . Wkv^T   [T][d]        gate = x . Wg^T   [T][d]
 *   kI   = x . WkI^T   [T][idx_dim]  gI   = x . WgI^T  [T][idx_dim]   (CSA only)
 *   w    = x . Ww^T    [T][idx_heads] fp32                           (CSA, optional)
 * kv, gate, kI, gI in cfg->act_dtype (bf16 rounds to nearest even): the
 * inputs of dsv4_compress_kv_{decode,prefill}; w the head weights of
 * dsv4_index_topk_{decode,prefill}.
 *   kind       DSV4_CSA or DSV4_HCA (HCA: wki_p, wgi_p, ww_p, kI, gI, w NULL)
 *   x          [T][hidden] bf16; hidden a multiple of 128, T <= 2^20
 *   w*_p       weights [rows][hidden] bf16 packed by dsv4_mx_pack_weight
 *   ww_p, w    both NULL (no head-weight projection) or both set; idx_heads a
 *              multiple of 16 for it (DSV4_ERR_UNSUPPORTED otherwise)
 *   ws         at least dsv4_kv_proj_ws_bytes bytes, 256-byte aligned
 */
dsv4_status dsv4_kv_proj_ws_bytes(const dsv4_cfg *cfg, int32_t T, int32_t hidden, int64_t *out);
dsv4_status dsv4_kv_proj(const dsv4_cfg *cfg, int32_t kind, const void *x, int32_t T, int32_t hidden,
                         const void *wkv_p, const void *wg_p, const void *wki_p, const void *wgi_p, const void *ww_p,
                         void *kv, void *gate, void *kI, void *gI, float *w, void *ws, int64_t ws_bytes,
                         void *stream);

/*
 * Cache fill (benchmarks, tests, reloading a saved prefix).  Writes n entries
 * (target DSV4_TARGET_ENTRY: a KV record, RoPE at the entry's block-end
 * position m*j+m-1 then stored; DSV4_TARGET_INDEX_KEY: a CSA index key,
 * stored) from fp32 values [n][dim].  Item i goes to request req_dev[i],
 * entry entry_dev[i].  Items must address distinct entries.
 */
dsv4_status dsv4_cache_write_entries(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t target,
                                     const int32_t *req_dev, const int32_t *entry_dev, int32_t n,
                                     const float *values_dev, void *stream);

/*
 * Dequantised read-back of stored vectors (tests, inspection, a host copy of
 * a prefix): item i of request req_dev[i] is decoded from its storage format
 * into out_dev[i][0..dim), fp32 or fp64 (out_dtype DSV4_DT_F32 / DSV4_DT_F64;
 * fp64 holds every stored value exactly, an E4M3 code times its fp32 scale
 * included):
 *   DSV4_TARGET_ENTRY      entry idx_dev[i] of the classic cache, d values as
 *                          stored (post-RoPE): E4M3 code * record scale for the
 *                          first d - d_rope dims, the BF16 (or fp32) values after
 *   DSV4_TARGET_INDEX_KEY  CSA index key idx_dev[i], idx_dim values (E4M3 * key
 *                          scale, E2M1 * 2^(E8M0 - 127) per 32 dims, or fp32)
 *   DSV4_TARGET_WINDOW     the window-ring record of position idx_dev[i] (slot
 *                          idx mod window; whether that slot still holds the
 *                          position is the caller's to know), d values
 * Sources: vastsailsolution.com V4 article, the classic-cache paragraph (blocks
 * of compressed entries), the state-cache paragraph (window records) and the
 * mixed-precision paragraph (BF16 RoPE dims, FP8 rest).  Items whose request,
 * index or block is out of range are skipped (their output left untouched).
 *   out_dev  [n][dim] of out_dtype, device, 16-byte aligned
 */
dsv4_status dsv4_cache_read_entries(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t target,
                                    const int32_t *req_dev, const int32_t *idx_dev, int32_t n, void *out_dev,
                                    int32_t out_dtype, void *stream);

/*
 * Dump and reload of one request's cache (vastsailsolution.com V4 article,
 * state-cache and classic-cache paragraph; xiaoyuzhoufm.com summary 2.1: an
 * on-disk KV cache for requests sharing a prefix, full-cache or periodic
 * checkpoints).  After n_tokens tokens a request's cache is its state cache
 * plus the classic-cache blocks covering tokens [0, n_tokens).  The dump is
 * those bytes in a fixed order, independent of the physical block ids:
 *   [state_bytes] [entry blocks 0 .. nb-1] [index blocks 0 .. nb-1 (CSA)]
 * with nb = ceil(n_tokens / 128); dsv4_cache_dump_bytes gives its size.  A
 * reload writes a dump into request `req` of a cache with the same
 * configuration through that request's block table (other block ids, another
 * pool): decoding then continues bit for bit as it would have on the original.
 * Blocks the table does not map are dumped as zeros and skipped on reload.
 *   buf_dev  device memory of at least dsv4_cache_dump_bytes bytes, 16-byte aligned
 *   (a host copy of it -- disk -- is the caller's)
 * n_tokens >= 1 with ceil(n_tokens / 128) <= the cache's max_blocks, and
 * 0 <= req < n_req; DSV4_ERR_INVALID_ARG otherwise, and for a missing, short
 * or misaligned buffer (nothing is copied then).
 */
dsv4_status dsv4_cache_dump_bytes(const dsv4_cfg *cfg, int32_t kind, int32_t n_tokens, int64_t *out);
dsv4_status dsv4_cache_dump(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t req, int32_t n_tokens,
                            void *buf_dev, int64_t buf_bytes, void *stream);
dsv4_status dsv4_cache_load(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t req, int32_t n_tokens,
                            const void *buf_dev, int64_t buf_bytes, void *stream);

/* Write raw tokens [pos0, pos0+n) of request `req` into its state cache (window
 * ring and pending ring; only the last W resp. pending_slots tokens land), as
 * the appends would have, without forming entries.  kv, gate [n][d] and
 * kI, gI [n][idx_dim] (CSA; NULL for HCA) in the act dtype. */
dsv4_status dsv4_state_write_tokens(const dsv4_cfg *cfg, const dsv4_cache *cache, int32_t req,
                                    int32_t pos0, int32_t n, const void *kv, const void *gate,
                                    const void *kI, const void *gI, void *stream);

/*
 * Optional kernel timers (instrumentation; not thread-safe).  When enabled for
 * a kernel id, every launch of that kernel is bracketed by HIP events on the
 * launch stream; dsv4_timer_read synchronises on the last event and returns
 * the summed elapsed milliseconds and launch count.
 */
#define DSV4_K_COMPRESS 0
#define DSV4_K_INDEX_SCORE 1
#define DSV4_K_TOPK 2
#define DSV4_K_ATTEND 3
#define DSV4_K_PROJ 4
#define DSV4_K_MX 5
#define DSV4_K_COUNT 6
dsv4_status dsv4_timer_enable(int32_t kernel_id, int32_t on);
dsv4_status dsv4_timer_read(int32_t kernel_id, int32_t reset, double *total_ms, int64_t *count);

#ifdef __cplusplus
}
#endif
#endif /* DSV4ATTN_H */
