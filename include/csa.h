/*
 * csa.h — C ABI of the MI355X (gfx950) hybrid compressed attention library
 * (libcsa.so): DeepSeek-V4's CSA and HCA attention layers.
 *
 * Sources (page title, section):
 *  [DD] "DeepSeek-V4 内部机制" (LLM-101-CN deep dive): §1.2 Step 1 (token-level
 *       compressor), Step 2 (Lightning Indexer, top-k, shared-KV MQA), §1.3
 *       (HCA: m' = 128, dense, no indexer), §1.4 table (Q/KV RMSNorm, partial
 *       RoPE with the output rotated at -i, 128-token sliding window,
 *       attention sink and its softmax equation), §1.5 (RoPE channels BF16,
 *       the rest FP8), §6.2 (FP4 indexer QK, BF16 index scores), §7 (state
 *       cache + paged cache whose block holds lcm(m, m') raw tokens).
 *  [YP] yunpan.plus explainer, "CSA / HCA" section, eqs. (6)-(11).
 *  [AD] m.admirer.cn article, CSA/HCA section (k = 512 / 1024, 128-token
 *       window, 64 RoPE channels, block of 128 raw tokens = 32 CSA + 1 HCA
 *       entries, state cache holding the window and the uncompressed tail).
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE memory unless marked [host].  The caller owns all
 *    memory; the library allocates nothing and never synchronises.
 *  - Every compute call enqueues its kernels on `stream` (a hipStream_t passed
 *    as void*, NULL = the default stream) and returns without waiting.
 *  - All arguments are validated on the host before anything is launched.
 *    Return value: CSA_OK (0) or a negative csa_status; csa_last_error()
 *    then holds a message (thread-local).  A launch failure reported by the
 *    HIP runtime returns CSA_EHIP.  No exception crosses the ABI.
 *  - Results are deterministic: every reduction runs in a fixed order that
 *    does not depend on the launch configuration or on timing.
 *  - Calls that share buffers must be ordered by the caller (same stream).
 *
 * The batch: a call processes the new tokens of n_req requests.  Request r
 * owns new tokens cu_new[r] .. cu_new[r+1]-1 (global rows of H, q, ...) at
 * positions start_pos[r], start_pos[r]+1, ...  Its state slot is r (slot r of
 * the state buffer) and its logical block j is physical block
 * block_table[r*max_blocks + j] of each layer's cache pools.
 *
 * Positions and visibility: compressed entry i of a request covers raw
 * tokens m*i .. m*i+m-1; it becomes visible to the query at position t iff
 * m*i+m-1 <= t, so a query sees V_t = floor((t+1)/m) entries.  Its RoPE
 * position is m*i.  Queries are rotated at t and outputs back at -t.
 *
 * Storage layouts (all little-endian, no padding beyond what is stated):
 *  KV block (one pool per layer, block stride csa_sizes.kv_block_bytes):
 *    CSA_KV_F32   epb records of c fp32
 *    CSA_KV_BF16  epb records of c bf16
 *    CSA_KV_FP8   64-byte header (fp32 scale s at byte 0, rest 0), then epb
 *                 records of (c - r) E4M3FN codes followed by r bf16 values
 *                 (the RoPE channels).  FP8 channels decode to code * s.
 *    epb = block_tokens / m entries per block (32 for CSA, 1 for HCA).
 *  Indexer-key block (CSA only, stride csa_sizes.idx_block_bytes):
 *    CSA_IDX_F32 / CSA_IDX_BF16  epb keys of c_idx values
 *    CSA_IDX_MXFP4  epb*c_idx/2 bytes of E2M1 codes (key j at j*c_idx/2, two
 *                   codes per byte, even element in the low nibble), then
 *                   epb*c_idx/32 E8M0 scale bytes (key j at j*c_idx/32), one
 *                   per 32 consecutive elements (OCP MX).
 *  State slot (stride csa_sizes.state_bytes): window ring of win_cap rows x c
 *    in act_fmt (row of position p at slot p mod win_cap), then the
 *    compressor tail ring of R rows x ncols fp32 (R = 2m with overlap, m
 *    without; row of position p at slot p mod R).  The tail holds the
 *    projected rows of the tokens whose entries are not complete yet, plus
 *    (CSA) the previous block that the next entry's b-half reads.
 *  Projection columns (ncols): CSA [C^a | C^b | Z^a | Z^b] (4c) followed by
 *    the indexer's [C^a | C^b | Z^a | Z^b] (4c_idx); HCA [C | Z] (2c).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 3

typedef enum {
    CSA_OK = 0,
    CSA_EINVAL = -1,        /* bad argument (null pointer, size, range) */
    CSA_EUNSUPPORTED = -2,  /* valid but unsupported combination */
    CSA_EWORKSPACE = -3,    /* workspace or output capacity too small */
    CSA_EHIP = -4,          /* HIP runtime reported an error */
    CSA_EINTERNAL = -5
} csa_status;

enum { CSA_KIND_CSA = 0, CSA_KIND_HCA = 1 };
enum { CSA_KV_F32 = 0, CSA_KV_BF16 = 1, CSA_KV_FP8 = 2 };
enum { CSA_IDX_F32 = 0, CSA_IDX_BF16 = 1, CSA_IDX_MXFP4 = 2 };
enum { CSA_FMT_F32 = 0, CSA_FMT_BF16 = 1 };   /* activations, scores, outputs */

/* One attention layer.  [host] */
typedef struct {
    int32_t kind;          /* CSA_KIND_CSA (overlapping 2m window, indexer, top-k) or CSA_KIND_HCA */
    int32_t m;             /* compression ratio: 4 (CSA) or 128 (HCA); block_tokens % m == 0 */
    int32_t c;             /* entry / head width (multiple of 32, <= 512) */
    int32_t rope_dim;      /* r: RoPE on the last r channels (even, 0 < r <= c) */
    int32_t n_heads;       /* query heads sharing the one KV head (multiple of 8, <= 128) */
    int32_t n_idx_heads;   /* CSA: indexer heads (multiple of 4, <= 64) */
    int32_t c_idx;         /* CSA: indexer key width (multiple of 32, <= 128) */
    int32_t top_k;         /* CSA: entries kept per query (1..2048) */
    int32_t n_win;         /* sliding-window rows (the query's own token and the n_win-1 before) */
    int32_t win_cap;       /* window ring rows per state slot: cache_append takes <= win_cap new tokens per request,
                              the attention calls <= win_cap - n_win + 1 */
    int32_t block_tokens;  /* raw tokens per paged block (128 = lcm(4, 128)) */
    int32_t kv_fmt;        /* CSA_KV_* */
    int32_t idx_fmt;       /* CSA_IDX_* */
    int32_t score_fmt;     /* CSA_FMT_*: index scores */
    int32_t act_fmt;       /* CSA_FMT_*: H, W, q, q_idx and the window ring */
    int32_t out_fmt;       /* CSA_FMT_*: attention output */
    float rope_theta;      /* RoPE base (10000) */
    float norm_eps;        /* RMSNorm epsilon (1e-6) */
    int32_t flags;         /* CSA_FLAG_* (0: none) */
} csa_layer_desc;

/* Batch invariance ([YP] "批无关性 & 计算确定性"; [DD] §6.3): every output of a
 * request (entries, keys, window rows, scores, selection, attention output)
 * is bit-identical whatever other requests share its calls.  The projection
 * is computed by the same kernel whatever the number of rows (each row's sums
 * do not depend on the other rows), and the attention always splits a
 * query's rows at the same boundaries (CSA_INVARIANT_SPLIT_ROWS rows per
 * split) and merges the splits in split order, also when a query has a
 * single split.  A request's own chunking (how its tokens are spread over
 * calls) still decides its FP8 block scales (see csa_cache_append).  The
 * indexer and the top-k are batch-invariant in every mode.  Costs: the
 * projection of many rows and the attention of many queries are slower, and
 * the attention workspace grows with the split count. */
#define CSA_FLAG_BATCH_INVARIANT 1
#define CSA_INVARIANT_SPLIT_ROWS 128

/* The requests of one call.  The struct itself is [host]. */
typedef struct {
    int32_t n_req;
    int32_t max_new;               /* [host] >= every request's new-token count */
    int32_t max_ctx;               /* [host] >= every request's start_pos + new-token count */
    int32_t max_blocks;            /* columns of block_table */
    const int32_t* cu_new;         /* [n_req+1] prefix sums of new tokens, cu_new[0] = 0 */
    const int32_t* start_pos;      /* [n_req] position of each request's first new token */
    const int32_t* block_table;    /* [n_req*max_blocks] physical block ids (-1 = unused) */
    int32_t* next_start_pos;       /* [n_req] or NULL.  csa_compress_kv and csa_compress_append write
                                      start_pos[r] + (cu_new[r+1] - cu_new[r]) here (must not alias
                                      start_pos); other calls ignore it.  A decode loop replayed as a
                                      graph alternates two position buffers with it instead of advancing
                                      positions with work of its own. */
} csa_batch;

/* Sizes the caller allocates.  [host] */
typedef struct {
    size_t kv_block_bytes;         /* one KV block */
    size_t idx_block_bytes;        /* one indexer-key block (0 for HCA) */
    size_t state_bytes;            /* one state slot (window ring + tail ring) */
    int32_t entries_per_block;     /* epb */
    int32_t proj_cols;             /* ncols of the projection */
} csa_sizes;

int csa_abi_version(void);
const char* csa_last_error(void);

/* Fill *out for a layer (validates the descriptor). */
int csa_layer_sizes(const csa_layer_desc* layer, csa_sizes* out);

/* Workspace bytes an op needs for n_rows rows (tokens or queries):
 *   CSA_OP_COMPRESS  projection rows [n_rows x ncols] fp32; bf16 activations:
 *                    4 partial products of n_rows rows each (n_rows <= 64, or
 *                    a batch-invariant layer), else max(n_rows, 256) rows, so
 *                    the size never falls as n_rows grows
 *   CSA_OP_TOPK      candidate lists for n_rows score rows of up to max_cols
 *   CSA_OP_ATTENTION split-KV partial results for n_rows queries, max_cols =
 *                    the largest number of rows (entries + window) a query reads
 *   CSA_OP_INDEX_TOPK csa_index_topk for n_rows queries, max_cols = ld (CSA layers) */
enum { CSA_OP_COMPRESS = 0, CSA_OP_TOPK = 1, CSA_OP_ATTENTION = 2, CSA_OP_INDEX_TOPK = 3 };
int csa_workspace_size(const csa_layer_desc* layer, int op, int n_rows, int max_cols, int top_k,
                       size_t* bytes);

/*
 * a1: token-level compressor ([DD] §1.2 Step 1 and §1.3; [YP] eqs. (6),(7),
 * (10),(11)).  Projects the call's new rows, H . W^T, into the workspace;
 * for every token t with (t+1) % m == 0 emits entry i = (t+1)/m - 1:
 *   per channel, softmax over the m logits Z^a + B^a of block i and (CSA,
 *   i >= 1) the m logits Z^b + B^b of block i-1, then the weighted sum of the
 *   matching C rows; entry 0 soft-maxes over its own block only.
 * The main entry is then RMS-normalised (gamma, norm_eps) and its last r
 * channels rotated at m*i ([DD] §1.4).  CSA also emits the indexer key, the
 * same merge over the indexer's own projection, without norm or RoPE.  Every
 * new token also yields its window row: C^a (HCA: C) normalised with gamma
 * and rotated at its position.  Rows of earlier calls come from the tail
 * ring, which is updated at the end of the call.
 *   H         [n_tokens x d] act_fmt           W      [4c x d] (HCA [2c x d]) act_fmt
 *   W_idx     [4c_idx x d] act_fmt (CSA)       B_a, B_b [m x c] fp32 (HCA: B_a only)
 *   B_a_idx, B_b_idx [m x c_idx] fp32 (CSA)    gamma  [c] fp32
 *   state     [n_req slots] read/write (tail ring)
 *   out_entries [max_entries x c] fp32, out_keys [max_entries x c_idx] fp32 (CSA),
 *   out_meta  [max_entries x 2] int32 (request, entry index), out_count [1] int32:
 *             entries in (request, index) order; max_entries must be
 *             >= sum over requests of floor((start+n)/m) - floor(start/m)
 *             (checked on the device: excess entries are dropped and
 *             out_count reports the true total).
 *   out_win   [n_tokens x c] fp32 window rows
 *   ws        >= csa_workspace_size(CSA_OP_COMPRESS, n_tokens)
 */
int csa_compress_kv(void* stream, const csa_layer_desc* layer, const csa_batch* batch,
                    int n_tokens, int d, const void* H, const void* W, const void* W_idx,
                    const float* B_a, const float* B_b, const float* B_a_idx, const float* B_b_idx,
                    const float* gamma, void* state,
                    float* out_entries, float* out_keys, int32_t* out_meta, int32_t* out_count,
                    int max_entries, float* out_win, void* ws, size_t ws_bytes);

/*
 * a2: cache append ([DD] §1.5, §7; [AD] cache section).  Stores the entries,
 * keys and window rows that csa_compress_kv produced:
 *   entry (r, i)  -> slot i % epb of physical block block_table[r][i / epb]
 *                    in kv_cache (format kv_fmt), key likewise in idx_cache;
 *   window row of the token at position p -> ring slot p % win_cap of state r.
 * FP8 block scale, per call and block, all decisions in fp32:
 *   s_old = 0 if the call's first new slot in the block is 0, else the header;
 *   s = max(s_old, amax / 448) with amax over the new entries' FP8 channels;
 *   if s > s_old, earlier slots are re-encoded E4M3(decode(code)*s_old / s);
 *   new entries are encoded E4M3(x / s) (round to nearest even, saturating).
 * bf16 stores round to nearest even; MXFP4 keys use OCP MX rules (E8M0
 * X = floor(log2 amax) - 2, E2M1 nearest-even, saturating at 6).
 *   entries/keys/meta/count as written by csa_compress_kv; win [n_tokens x c] fp32.
 */
int csa_cache_append(void* stream, const csa_layer_desc* layer, const csa_batch* batch,
                     int n_tokens, const float* entries, const float* keys, const int32_t* meta,
                     const int32_t* count, int max_entries, const float* win,
                     void* kv_cache, void* idx_cache, void* state);

/*
 * a1 then a2 in one call ([DD] §7: the new tokens' compressed entries and
 * window rows go to the caches as they are produced).  Same arguments,
 * outputs and errors as csa_compress_kv, plus the caches of
 * csa_cache_append (batch->block_table required, max_new <= win_cap); the
 * caches and state end as after csa_compress_kv followed by
 * csa_cache_append on its outputs, byte for byte.  With batch->max_new <= 1
 * (decode: at most one entry per request and call) the merge and window
 * workgroups store what they produce themselves, in one kernel; otherwise the
 * two calls' kernels run in order.
 */
int csa_compress_append(void* stream, const csa_layer_desc* layer, const csa_batch* batch,
                        int n_tokens, int d, const void* H, const void* W, const void* W_idx,
                        const float* B_a, const float* B_b, const float* B_a_idx, const float* B_b_idx,
                        const float* gamma, void* state,
                        float* out_entries, float* out_keys, int32_t* out_meta, int32_t* out_count,
                        int max_entries, float* out_win, void* kv_cache, void* idx_cache,
                        void* ws, size_t ws_bytes);

/*
 * Prefix reuse, host-memory tier ([DD] §7: the compressed entries of a shared
 * prefix are stored whole; the sliding window by one of three strategies, one
 * of them a checkpoint every p tokens).  Copies between a layer's caches and
 * PINNED host memory (hipHostMalloc, or a torch tensor with pin_memory=True);
 * any other host pointer is rejected with CSA_EINVAL before anything runs.
 *
 * csa_prefix_blocks: the n_blocks physical blocks block_ids[0..n_blocks)
 *   (device int32; negative ids are skipped) of kv_cache and, for CSA, of
 *   idx_cache, to (CSA_TO_HOST) or from (CSA_FROM_HOST) host, packed as
 *   n_blocks x kv_block_bytes followed (CSA) by n_blocks x idx_block_bytes
 *   (csa_prefix_bytes).  One kernel reads or writes the host buffer directly.
 * csa_prefix_state: one state slot (window ring and compressor tail ring,
 *   state_bytes) to or from host, stream-ordered.
 *
 * A request resumes bit-identically (every later output equal to the
 * uninterrupted run's) from its blocks and its state slot saved together
 * after a call that ended at position P.  A block holding only entries
 * below P is final once complete (its FP8 scale changes only when entries
 * are appended to it), so with P a multiple of block_tokens the blocks of a
 * shared prefix can be saved once and the window state checkpointed every p
 * tokens (p a multiple of block_tokens).  Calls sharing buffers must be
 * ordered by the caller; host buffers must not be reused before the stream
 * has reached the copy.
 */
enum { CSA_TO_HOST = 0, CSA_FROM_HOST = 1 };
int csa_prefix_bytes(const csa_layer_desc* layer, int n_blocks, size_t* bytes);
int csa_prefix_blocks(void* stream, const csa_layer_desc* layer, int n_blocks, const int32_t* block_ids,
                      void* kv_cache, void* idx_cache, void* host, int dir);
int csa_prefix_state(void* stream, const csa_layer_desc* layer, void* state_slot, void* host, int dir);

/*
 * The dense projections on either side of the path ([DD] §1.2 Step 2 query
 * side: c^Q_t = h_t . W^DQ, then the indexer queries from c^Q; Step 3:
 * grouped output projection, g groups of head outputs each projected to d_g,
 * concatenated and projected to d; [AD]: d_c = 1024; [DD]: V4-Pro g = 16,
 * d_g = 1024).  The caller composes them (see DESIGN): one GEMM per call,
 * fp32 accumulation on the MFMA, no workspace.
 *
 * csa_linear:         Y[n_rows x N] = X[n_rows x K] . W^T,  W [N x K] (one row per output)
 * csa_grouped_linear: for g < groups:
 *                     Y[:, g*N .. g*N+N) = X[:, g*K .. g*K+K) . W[g]^T,  W [groups x N x K]
 *   X, W in act_fmt (CSA_FMT_BF16 or CSA_FMT_F32), Y in out_fmt (bf16 rounds
 *   to nearest even).  K must be a positive multiple of 128; all pointers
 *   16-byte aligned.
 */
int csa_linear(void* stream, int act_fmt, int out_fmt, int n_rows, int K, int N, const void* X, const void* W,
               void* Y);
int csa_grouped_linear(void* stream, int act_fmt, int out_fmt, int n_rows, int groups, int K, int N, const void* X,
                       const void* W, void* Y);

/*
 * a3: Lightning Indexer scores ([DD] §1.2 Step 2; [YP] eq. (8); [DD] §6.2).
 * For every new token t of the batch (query row g = its global row) and every
 * visible entry s < V_t:
 *   scores[g*ld + s] = round_score_fmt( sum_h w[g][h] * ReLU(q[g][h] . K[s]) )
 * with fp32 accumulation; -0 is stored as +0.  For CSA_IDX_MXFP4 the query
 * heads are first quantised to MXFP4 (same rules as the keys) and the
 * product runs on the dequantised values.  Also writes n_valid[g] = V_t.
 *   q_idx [n_tokens x n_idx_heads x c_idx] act_fmt, w [n_tokens x n_idx_heads] fp32
 *   scores [n_tokens x ld] score_fmt (ld >= the largest V_t; columns >= V_t untouched)
 */
int csa_index_scores(void* stream, const csa_layer_desc* layer, const csa_batch* batch,
                     int n_tokens, const void* q_idx, const float* w, const void* idx_cache,
                     void* scores, int ld, int32_t* n_valid);

/*
 * a3 + a4 fused ([DD] §6.2: FP4 indexer QK, BF16 index scores, top-k selector;
 * the selection of csa_topk_select on the scores of csa_index_scores).  Same
 * arguments, scores and n_valid as csa_index_scores, plus out_idx
 * [n_tokens x top_k] int32 with exactly the selection csa_topk_select would
 * make from those scores (k = layer->top_k: the k largest, ties to the lower
 * index, ascending, -1 padded).  With bf16 scores the selection's first
 * radix digit comes from per-chunk counts of the scores by the top 8 bits of
 * the order-preserving score key (into ws): for decode-shaped calls the
 * indexer's workgroups count their chunk while they stream the keys; for
 * prefill-shaped calls (many new tokens per request; the scan is bound by
 * its MFMAs) a pass over the stored scores counts them per segment.  The
 * selection then needs only a counting and an emitting pass over segments
 * of each row (many workgroups per row), instead of a histogram pipeline of
 * its own.
 * Requires ld % 8 == 0 and 16-byte aligned scores and ws (bf16 scores).
 * fp32 scores run the two calls' kernels in order.
 *   ws >= csa_workspace_size(CSA_OP_INDEX_TOPK, n_tokens, ld): per (query,
 *   chunk of entries) 256 counts and per (query, segment) 258 counts (bf16),
 *   or the top-k candidates (fp32).
 */
int csa_index_topk(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens,
                   const void* q_idx, const float* w, const void* idx_cache, void* scores, int ld,
                   int32_t* n_valid, int32_t* out_idx, void* ws, size_t ws_bytes);

/*
 * a4: top-k selector ([DD] §1.2 Step 2; [AD]: k = 512 / 1024).  For each row
 * g: the k largest of scores[g*ld + 0 .. n_valid[g]-1] (ties: the lower index
 * wins), written to out_idx[g*k ..] in ascending index order, padded with -1
 * when n_valid[g] < k.  Exact (integer radix selection on order-preserving
 * keys).  ws >= csa_workspace_size(CSA_OP_TOPK, n_rows, ld, k).  n_valid[g]
 * above ld is taken as ld (a row never reads past its ld columns).
 */
int csa_topk_select(void* stream, int score_fmt, int n_rows, const void* scores, int ld,
                    const int32_t* n_valid, int k, int32_t* out_idx, void* ws, size_t ws_bytes);

/*
 * csa_topk_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * csa_topk_select; the candidate lists of the two-stage selection (rows
 * longer than one workgroup's share) live in a static device array of
 * CSA_STATIC_TOPK_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends.  A call whose csa_workspace_size(CSA_OP_TOPK, n_rows, ld,
 * k) exceeds it returns CSA_EWORKSPACE before anything runs.  The array's
 * address on the current device is looked up on the first call on that
 * device.  Every call on a GPU shares that GPU's array (it keeps the last
 * call's candidates; nothing in it needs to start at zero): calls that
 * overlap on one GPU (other streams, unordered host threads) race, so the
 * caller must order them.  Allocates nothing.
 */
#define CSA_STATIC_TOPK_SCRATCH_BYTES (8u << 20)
int csa_topk_select_static(void* stream, int score_fmt, int n_rows, const void* scores, int ld,
                           const int32_t* n_valid, int k, int32_t* out_idx);

/*
 * a5: sparse shared-KV MQA with window and sink ([DD] §1.2 Step 2, §1.4
 * table and sink equation; [YP] eq. (9)).  For each new token t (row g) and
 * head h: q = RoPE_t(RMSNorm_gamma_q(q_raw[g][h])); rows X = the entries
 * sel[g][0..top_k) (skipping -1) and the window rows of positions
 * max(0, t-n_win+1) .. t (from the ring, which csa_cache_append has already
 * filled for this call's tokens); z_j = q . X_j / sqrt(c);
 *   o = sum_j exp(z_j) X_j / (sum_j exp(z_j) + exp(sinks[h])), then RoPE_-t.
 *   q [n_tokens x n_heads x c] act_fmt, q_gamma [c] fp32, sinks [n_heads] fp32,
 *   sel [n_tokens x top_k] int32, out [n_tokens x n_heads x c] out_fmt
 *   ws >= csa_workspace_size(CSA_OP_ATTENTION, n_tokens, top_k + n_win)
 */
int csa_sparse_mqa(void* stream, const csa_layer_desc* layer, const csa_batch* batch,
                   int n_tokens, const void* q, const float* q_gamma, const int32_t* sel,
                   const void* kv_cache, const void* state, const float* sinks, void* out,
                   void* ws, size_t ws_bytes);

/*
 * a6: HCA dense MQA ([DD] §1.3; [YP] HCA attention).  As csa_sparse_mqa, with
 * the rows being every visible entry s < V_t followed by the window.
 *   ws >= csa_workspace_size(CSA_OP_ATTENTION, n_tokens, max_ctx/m + n_win)
 */
int csa_hca_attention(void* stream, const csa_layer_desc* layer, const csa_batch* batch,
                      int n_tokens, const void* q, const float* q_gamma, const void* kv_cache,
                      const void* state, const float* sinks, void* out, void* ws, size_t ws_bytes);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
