// C ABI of libcsa.so (declared in include/csa.h): host-side validation,
// workspace sizing and kernel dispatch.  Nothing here allocates device
// memory or synchronises; every call enqueues on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/csa.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return CSA_OK;
    return fail(CSA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, code, ...) \
    do { if (!(cond)) return fail(code, __VA_ARGS__); } while (0)

bool is_csa(const csa_layer_desc* L) { return L->kind == CSA_KIND_CSA; }

int tail_rows(const csa_layer_desc* L) { return is_csa(L) ? 2 * L->m : L->m; }

int proj_cols(const csa_layer_desc* L) { return is_csa(L) ? 4 * L->c + 4 * L->c_idx : 2 * L->c; }
bool invariant(const csa_layer_desc* L) { return (L->flags & CSA_FLAG_BATCH_INVARIANT) != 0; }

size_t kv_record(const csa_layer_desc* L)
{
    if (L->kv_fmt == CSA_KV_F32) return (size_t)L->c * 4;
    if (L->kv_fmt == CSA_KV_BF16) return (size_t)L->c * 2;
    return (size_t)(L->c - L->rope_dim) + 2 * (size_t)L->rope_dim;
}

size_t kv_block(const csa_layer_desc* L)
{
    const int epb = L->block_tokens / L->m;
    return (L->kv_fmt == CSA_KV_FP8 ? 64 : 0) + (size_t)epb * kv_record(L);
}

size_t idx_block(const csa_layer_desc* L)
{
    if (!is_csa(L)) return 0;
    const size_t epb = L->block_tokens / L->m, cI = L->c_idx;
    if (L->idx_fmt == CSA_IDX_F32) return epb * cI * 4;
    if (L->idx_fmt == CSA_IDX_BF16) return epb * cI * 2;
    return epb * (cI / 2 + cI / 32);
}

size_t win_bytes(const csa_layer_desc* L)
{
    return (size_t)L->win_cap * L->c * (L->act_fmt == CSA_FMT_BF16 ? 2 : 4);
}

size_t state_bytes(const csa_layer_desc* L)
{
    size_t w = (win_bytes(L) + 255) & ~(size_t)255;
    return w + (size_t)tail_rows(L) * proj_cols(L) * 4;
}

int check_layer(const csa_layer_desc* L)
{
    REQUIRE(L != nullptr, CSA_EINVAL, "layer descriptor is NULL");
    REQUIRE(L->kind == CSA_KIND_CSA || L->kind == CSA_KIND_HCA, CSA_EINVAL, "kind %d", L->kind);
    REQUIRE(L->m >= 1 && L->block_tokens >= L->m && L->block_tokens % L->m == 0, CSA_EINVAL,
            "m=%d must divide block_tokens=%d", L->m, L->block_tokens);
    REQUIRE(((L->block_tokens / L->m) & (L->block_tokens / L->m - 1)) == 0, CSA_EUNSUPPORTED,
            "entries per block (block_tokens / m = %d) must be a power of two", L->block_tokens / L->m);
    REQUIRE(L->c == 128 || L->c == 256 || L->c == 512, CSA_EUNSUPPORTED, "c=%d (supported: 128, 256, 512)", L->c);
    REQUIRE(L->rope_dim > 0 && L->rope_dim <= L->c && L->rope_dim % 2 == 0 && L->rope_dim <= 512, CSA_EINVAL,
            "rope_dim=%d", L->rope_dim);
    REQUIRE((L->c == 128 && L->rope_dim == 32) || (L->c >= 256 && L->rope_dim == 64), CSA_EUNSUPPORTED,
            "(c, rope_dim) = (%d, %d); supported: (128, 32), (256, 64), (512, 64)", L->c, L->rope_dim);
    REQUIRE(L->n_heads >= 1 && L->n_heads <= 128 && (L->n_heads <= 64 || L->n_heads % 64 == 0), CSA_EUNSUPPORTED,
            "n_heads=%d (1..64, or a multiple of 64 up to 128)", L->n_heads);
    REQUIRE(L->n_heads <= 16 || L->n_heads % 16 == 0, CSA_EUNSUPPORTED, "n_heads=%d must be a multiple of 16 above 16",
            L->n_heads);
    REQUIRE(L->n_win >= 1 && L->win_cap >= L->n_win, CSA_EINVAL, "n_win=%d win_cap=%d", L->n_win, L->win_cap);
    REQUIRE(L->kv_fmt >= CSA_KV_F32 && L->kv_fmt <= CSA_KV_FP8, CSA_EINVAL, "kv_fmt=%d", L->kv_fmt);
    REQUIRE(L->act_fmt == CSA_FMT_F32 || L->act_fmt == CSA_FMT_BF16, CSA_EINVAL, "act_fmt=%d", L->act_fmt);
    REQUIRE(L->out_fmt == CSA_FMT_F32 || L->out_fmt == CSA_FMT_BF16, CSA_EINVAL, "out_fmt=%d", L->out_fmt);
    REQUIRE(L->kv_fmt != CSA_KV_F32 || L->act_fmt == CSA_FMT_F32, CSA_EUNSUPPORTED,
            "fp32 KV needs fp32 activations (window ring)");
    REQUIRE(L->kv_fmt != CSA_KV_F32 || L->c <= 256, CSA_EUNSUPPORTED, "fp32 KV supports c <= 256");
    REQUIRE(L->kv_fmt == CSA_KV_F32 || L->act_fmt == CSA_FMT_BF16, CSA_EUNSUPPORTED,
            "bf16 / fp8 KV needs bf16 activations (window ring)");
    REQUIRE(L->kv_fmt != CSA_KV_FP8 || (L->c - L->rope_dim) % 32 == 0, CSA_EUNSUPPORTED,
            "fp8 KV needs c - rope_dim to be a multiple of 32");
    REQUIRE(L->norm_eps >= 0.0f && L->rope_theta > 0.0f, CSA_EINVAL, "norm_eps / rope_theta");
    REQUIRE((L->flags & ~CSA_FLAG_BATCH_INVARIANT) == 0, CSA_EINVAL, "flags=%d", L->flags);
    if (is_csa(L)) {
        REQUIRE(L->n_idx_heads >= 1 && L->n_idx_heads <= 64, CSA_EUNSUPPORTED, "n_idx_heads=%d (1..64)",
                L->n_idx_heads);
        REQUIRE(L->c_idx == 64 || L->c_idx == 128, CSA_EUNSUPPORTED, "c_idx=%d (64 or 128)", L->c_idx);
        REQUIRE(L->idx_fmt >= CSA_IDX_F32 && L->idx_fmt <= CSA_IDX_MXFP4, CSA_EINVAL, "idx_fmt=%d", L->idx_fmt);
        REQUIRE(L->idx_fmt != CSA_IDX_MXFP4 || L->c_idx == 128, CSA_EUNSUPPORTED, "MXFP4 keys need c_idx=128");
        REQUIRE(L->idx_fmt != CSA_IDX_F32 || L->act_fmt == CSA_FMT_F32, CSA_EUNSUPPORTED,
                "fp32 indexer keys need fp32 queries");
        REQUIRE(L->idx_fmt == CSA_IDX_F32 || L->act_fmt == CSA_FMT_BF16, CSA_EUNSUPPORTED,
                "bf16 / MXFP4 indexer keys need bf16 queries");
        REQUIRE(L->score_fmt == CSA_FMT_F32 || L->score_fmt == CSA_FMT_BF16, CSA_EINVAL, "score_fmt=%d",
                L->score_fmt);
        REQUIRE(L->top_k >= 1 && L->top_k <= 2048, CSA_EUNSUPPORTED, "top_k=%d (1..2048)", L->top_k);
        REQUIRE(2 * L->m <= 512, CSA_EUNSUPPORTED, "overlapping window 2m=%d too large", 2 * L->m);
    }
    return CSA_OK;
}

// win_rule: 0 no window constraint, 1 the call writes the window ring (its new
// rows must not overwrite each other), 2 the call reads the window of every
// new token (the oldest row a query needs must survive the call's writes).
int check_batch(const csa_layer_desc* L, const csa_batch* B, bool need_blocks, int win_rule)
{
    REQUIRE(B != nullptr, CSA_EINVAL, "batch is NULL");
    REQUIRE(B->n_req >= 1, CSA_EINVAL, "n_req=%d", B->n_req);
    REQUIRE(B->cu_new != nullptr && B->start_pos != nullptr, CSA_EINVAL, "cu_new / start_pos is NULL");
    REQUIRE(B->max_new >= 0 && B->max_ctx >= B->max_new, CSA_EINVAL, "max_new=%d max_ctx=%d", B->max_new, B->max_ctx);
    REQUIRE(win_rule != 1 || B->max_new <= L->win_cap, CSA_EINVAL,
            "max_new=%d exceeds win_cap=%d (new window rows would overwrite each other)", B->max_new, L->win_cap);
    REQUIRE(win_rule != 2 || B->max_new <= L->win_cap - L->n_win + 1, CSA_EINVAL,
            "max_new=%d exceeds win_cap - n_win + 1 = %d (the window ring would overwrite rows still needed)",
            B->max_new, L->win_cap - L->n_win + 1);
    if (need_blocks) {
        REQUIRE(B->block_table != nullptr, CSA_EINVAL, "block_table is NULL");
        const int epb = L->block_tokens / L->m;
        const long need = ((long)B->max_ctx / L->m + epb - 1) / epb;
        REQUIRE(B->max_blocks >= need, CSA_EINVAL, "max_blocks=%d < %ld blocks needed for max_ctx=%d", B->max_blocks,
                need, B->max_ctx);
    }
    return CSA_OK;
}

#define CHECK(expr) do { int _rc = (expr); if (_rc != CSA_OK) return _rc; } while (0)

// Workspace of the fused index + top-k: per-chunk score counts (bf16
// scores), or the two-stage top-k's candidates (fp32 scores).
size_t index_topk_hist_bytes(const csa_layer_desc* layer, int n_rows, int ld)
{
    const int chunk = csa::index_min_chunk(layer->idx_fmt);
    const size_t b = (size_t)n_rows * ((ld + chunk - 1) / chunk) * 256 * sizeof(uint16_t);
    return (b + 255) & ~(size_t)255;
}

size_t index_topk_workspace(const csa_layer_desc* layer, int n_rows, int ld)
{
    if (layer->score_fmt != CSA_FMT_BF16) return csa::topk_workspace(n_rows, ld, layer->top_k, false);
    return index_topk_hist_bytes(layer, n_rows, ld) + csa::topk_hist_workspace(n_rows, ld);
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_err; }

int csa_layer_sizes(const csa_layer_desc* layer, csa_sizes* out)
{
    CHECK(check_layer(layer));
    REQUIRE(out != nullptr, CSA_EINVAL, "out is NULL");
    out->kv_block_bytes = kv_block(layer);
    out->idx_block_bytes = idx_block(layer);
    out->state_bytes = state_bytes(layer);
    out->entries_per_block = layer->block_tokens / layer->m;
    out->proj_cols = proj_cols(layer);
    return CSA_OK;
}

int csa_workspace_size(const csa_layer_desc* layer, int op, int n_rows, int max_cols, int top_k, size_t* bytes)
{
    CHECK(check_layer(layer));
    REQUIRE(bytes != nullptr, CSA_EINVAL, "bytes is NULL");
    REQUIRE(n_rows >= 0 && max_cols >= 0, CSA_EINVAL, "n_rows=%d max_cols=%d", n_rows, max_cols);
    switch (op) {
    case CSA_OP_COMPRESS:
        *bytes = csa::compress_workspace(layer->act_fmt == CSA_FMT_BF16, invariant(layer), n_rows, proj_cols(layer));
        return CSA_OK;
    case CSA_OP_TOPK:
        REQUIRE(top_k >= 1, CSA_EINVAL, "top_k=%d", top_k);
        *bytes = csa::topk_workspace(n_rows, max_cols, top_k, layer->score_fmt == CSA_FMT_BF16);
        return CSA_OK;
    case CSA_OP_ATTENTION:
        *bytes = csa::attention_workspace(n_rows, layer->n_heads, layer->c, max_cols, invariant(layer));
        return CSA_OK;
    case CSA_OP_INDEX_TOPK:
        REQUIRE(is_csa(layer), CSA_EINVAL, "index_topk needs a CSA layer");
        REQUIRE(max_cols >= 1, CSA_EINVAL, "max_cols=%d (ld)", max_cols);
        *bytes = index_topk_workspace(layer, n_rows, max_cols);
        return CSA_OK;
    default: return fail(CSA_EINVAL, "op=%d", op);
    }
}

}  // extern "C"

namespace {

// Validates compress_kv's arguments and fills its kernel arguments.
int compress_args(const csa_layer_desc* layer, const csa_batch* batch, int n_tokens, int d, const void* H,
                  const void* W, const void* W_idx, const float* B_a, const float* B_b, const float* B_a_idx,
                  const float* B_b_idx, const float* gamma, void* state, float* out_entries, float* out_keys,
                  int32_t* out_meta, int32_t* out_count, int max_entries, float* out_win, void* ws, size_t ws_bytes,
                  csa::CompressArgs* out)
{
    CHECK(check_layer(layer));
    CHECK(check_batch(layer, batch, false, 0));
    const bool csa = is_csa(layer);
    REQUIRE(n_tokens >= 0 && max_entries >= 0, CSA_EINVAL, "n_tokens=%d max_entries=%d", n_tokens, max_entries);
    REQUIRE(d >= 128 && d % 128 == 0, CSA_EUNSUPPORTED, "d=%d must be a positive multiple of 128", d);
    REQUIRE(n_tokens == 0 || (H != nullptr && W != nullptr && out_win != nullptr), CSA_EINVAL,
            "H / W / out_win is NULL");
    REQUIRE(B_a != nullptr && gamma != nullptr && state != nullptr && out_count != nullptr, CSA_EINVAL,
            "B_a / gamma / state / out_count is NULL");
    REQUIRE(max_entries == 0 || (out_entries != nullptr && out_meta != nullptr), CSA_EINVAL,
            "out_entries / out_meta is NULL");
    if (csa) {
        REQUIRE(B_b != nullptr && B_a_idx != nullptr && B_b_idx != nullptr, CSA_EINVAL, "CSA biases are NULL");
        REQUIRE(n_tokens == 0 || W_idx != nullptr, CSA_EINVAL, "W_idx is NULL");
        REQUIRE(max_entries == 0 || out_keys != nullptr, CSA_EINVAL, "out_keys is NULL");
    }
    const size_t need = n_tokens > 0 ? csa::compress_workspace(layer->act_fmt == CSA_FMT_BF16, invariant(layer),
                                                                n_tokens, proj_cols(layer)) : 0;
    REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), CSA_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
            need);
    csa::CompressArgs& a = *out;
    memset(&a, 0, sizeof(a));
    a.invariant = invariant(layer);
    a.P = (float*)ws;
    a.ncols = proj_cols(layer);
    a.state = state;
    a.state_stride = state_bytes(layer);
    a.tail_off = (win_bytes(layer) + 255) & ~(size_t)255;
    a.R = tail_rows(layer);
    a.cu_new = batch->cu_new;
    a.start_pos = batch->start_pos;
    a.n_req = batch->n_req;
    a.m = layer->m;
    a.overlap = csa ? 1 : 0;
    a.c = layer->c;
    a.c_idx = csa ? layer->c_idx : 0;
    a.r = layer->rope_dim;
    a.B_a = B_a;
    a.B_b = B_b;
    a.B_a_idx = B_a_idx;
    a.B_b_idx = B_b_idx;
    a.gamma = gamma;
    a.eps = layer->norm_eps;
    a.theta = layer->rope_theta;
    a.out_entries = out_entries;
    a.out_keys = out_keys;
    a.out_meta = out_meta;
    a.out_count = out_count;
    a.max_entries = max_entries;
    a.out_win = out_win;
    a.max_new = batch->max_new;
    REQUIRE(batch->next_start_pos == nullptr || (const int32_t*)batch->next_start_pos != batch->start_pos,
            CSA_EINVAL, "next_start_pos must not alias start_pos");
    a.next_pos = batch->next_start_pos;
    return CSA_OK;
}

// Validates cache_append's arguments and fills its kernel arguments.
int append_args(const csa_layer_desc* layer, const csa_batch* batch, int n_tokens, const float* entries,
                const float* keys, const int32_t* meta, const int32_t* count, int max_entries, const float* win,
                void* kv_cache, void* idx_cache, void* state, csa::AppendArgs* out)
{
    CHECK(check_layer(layer));
    CHECK(check_batch(layer, batch, true, 1));
    const bool csa = is_csa(layer);
    REQUIRE(n_tokens >= 0 && max_entries >= 0, CSA_EINVAL, "n_tokens=%d max_entries=%d", n_tokens, max_entries);
    REQUIRE(max_entries == 0 || (entries != nullptr && meta != nullptr && count != nullptr && kv_cache != nullptr),
            CSA_EINVAL, "entries / meta / count / kv_cache is NULL");
    REQUIRE(!csa || max_entries == 0 || (keys != nullptr && idx_cache != nullptr), CSA_EINVAL,
            "keys / idx_cache is NULL");
    REQUIRE(n_tokens == 0 || (win != nullptr && state != nullptr), CSA_EINVAL, "win / state is NULL");
    csa::AppendArgs& a = *out;
    memset(&a, 0, sizeof(a));
    a.entries = entries;
    a.keys = keys;
    a.meta = meta;
    a.count = count;
    a.max_entries = max_entries;
    a.win = win;
    a.n_tokens = n_tokens;
    a.one_per_req = batch->max_new <= 1 && n_tokens == batch->n_req;
    a.cu_new = batch->cu_new;
    a.start_pos = batch->start_pos;
    a.block_table = batch->block_table;
    a.n_req = batch->n_req;
    a.max_blocks = batch->max_blocks;
    a.c = layer->c;
    a.r = layer->rope_dim;
    a.c_idx = csa ? layer->c_idx : 0;
    a.epb = layer->block_tokens / layer->m;
    a.kv_fmt = layer->kv_fmt;
    a.idx_fmt = layer->idx_fmt;
    a.win_bf16 = layer->act_fmt == CSA_FMT_BF16;
    a.kv = kv_cache;
    a.kv_block_bytes = kv_block(layer);
    a.idx = csa ? idx_cache : nullptr;
    a.idx_block_bytes = idx_block(layer);
    a.state = state;
    a.state_stride = state_bytes(layer);
    a.win_cap = layer->win_cap;
    return CSA_OK;
}

hipError_t compress_launch(hipStream_t st, const csa_layer_desc* layer, const csa::CompressArgs& a, const void* H,
                           const void* W, const void* W_idx, int d, int n_tokens, const csa::AppendArgs* app)
{
    const bool csa = is_csa(layer);
    const int n_main = csa ? 4 * layer->c : 2 * layer->c;
    return csa::launch_compress(st, a, H, W, csa ? W_idx : W, n_main, d, layer->act_fmt == CSA_FMT_BF16, n_tokens,
                                app);
}

}  // namespace

extern "C" {

int csa_compress_kv(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens, int d,
                    const void* H, const void* W, const void* W_idx, const float* B_a, const float* B_b,
                    const float* B_a_idx, const float* B_b_idx, const float* gamma, void* state,
                    float* out_entries, float* out_keys, int32_t* out_meta, int32_t* out_count, int max_entries,
                    float* out_win, void* ws, size_t ws_bytes)
{
    csa::CompressArgs a;
    CHECK(compress_args(layer, batch, n_tokens, d, H, W, W_idx, B_a, B_b, B_a_idx, B_b_idx, gamma, state, out_entries,
                        out_keys, out_meta, out_count, max_entries, out_win, ws, ws_bytes, &a));
    return hip_status(compress_launch((hipStream_t)stream, layer, a, H, W, W_idx, d, n_tokens, nullptr),
                      "compress_kv launch");
}

int csa_cache_append(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens,
                     const float* entries, const float* keys, const int32_t* meta, const int32_t* count,
                     int max_entries, const float* win, void* kv_cache, void* idx_cache, void* state)
{
    csa::AppendArgs a;
    CHECK(append_args(layer, batch, n_tokens, entries, keys, meta, count, max_entries, win, kv_cache, idx_cache,
                      state, &a));
    return hip_status(csa::launch_append((hipStream_t)stream, a), "cache_append launch");
}

int csa_compress_append(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens, int d,
                        const void* H, const void* W, const void* W_idx, const float* B_a, const float* B_b,
                        const float* B_a_idx, const float* B_b_idx, const float* gamma, void* state,
                        float* out_entries, float* out_keys, int32_t* out_meta, int32_t* out_count, int max_entries,
                        float* out_win, void* kv_cache, void* idx_cache, void* ws, size_t ws_bytes)
{
    csa::CompressArgs a;
    csa::AppendArgs b;
    CHECK(compress_args(layer, batch, n_tokens, d, H, W, W_idx, B_a, B_b, B_a_idx, B_b_idx, gamma, state, out_entries,
                        out_keys, out_meta, out_count, max_entries, out_win, ws, ws_bytes, &a));
    CHECK(append_args(layer, batch, n_tokens, out_entries, out_keys, out_meta, out_count, max_entries, out_win,
                      kv_cache, idx_cache, state, &b));
    return hip_status(compress_launch((hipStream_t)stream, layer, a, H, W, W_idx, d, n_tokens, &b),
                      "compress_append launch");
}

}  // extern "C"

namespace {

// Validates index_scores' arguments and fills its kernel arguments.
int index_args(const csa_layer_desc* layer, const csa_batch* batch, int n_tokens, const void* q_idx, const float* w,
               const void* idx_cache, void* scores, int ld, int32_t* n_valid, csa::IndexArgs* out)
{
    CHECK(check_layer(layer));
    REQUIRE(is_csa(layer), CSA_EINVAL, "index_scores needs a CSA layer");
    CHECK(check_batch(layer, batch, true, 0));
    REQUIRE(n_tokens >= 0, CSA_EINVAL, "n_tokens=%d", n_tokens);
    const int max_vis = batch->max_ctx / layer->m;
    REQUIRE(ld >= max_vis && ld >= 1, CSA_EINVAL, "ld=%d < largest visible count %d", ld, max_vis);
    REQUIRE(max_vis / 1024 < 65535, CSA_EUNSUPPORTED, "max_ctx / m = %d entries exceeds the decode grid", max_vis);
    REQUIRE(n_tokens == 0 || (q_idx != nullptr && w != nullptr && idx_cache != nullptr && scores != nullptr &&
                              n_valid != nullptr),
            CSA_EINVAL, "NULL pointer argument");
    csa::IndexArgs& a = *out;
    memset(&a, 0, sizeof(a));
    a.q = q_idx;
    a.w = w;
    a.keys = idx_cache;
    a.key_block_bytes = idx_block(layer);
    a.cu_new = batch->cu_new;
    a.start_pos = batch->start_pos;
    a.block_table = batch->block_table;
    a.n_req = batch->n_req;
    a.max_blocks = batch->max_blocks;
    a.m = layer->m;
    a.epb = layer->block_tokens / layer->m;
    a.epb_log2 = __builtin_ctz((unsigned)a.epb);
    a.nh = layer->n_idx_heads;
    a.cI = layer->c_idx;
    a.q_bf16 = layer->act_fmt == CSA_FMT_BF16;
    a.idx_fmt = layer->idx_fmt;
    a.score_bf16 = layer->score_fmt == CSA_FMT_BF16;
    a.scores = scores;
    a.ld = ld;
    a.n_valid = n_valid;
    a.n_tokens = n_tokens;
    return CSA_OK;
}

}  // namespace

extern "C" {

int csa_index_scores(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens,
                     const void* q_idx, const float* w, const void* idx_cache, void* scores, int ld,
                     int32_t* n_valid)
{
    csa::IndexArgs a;
    CHECK(index_args(layer, batch, n_tokens, q_idx, w, idx_cache, scores, ld, n_valid, &a));
    return hip_status(csa::launch_index((hipStream_t)stream, a, batch->max_ctx / layer->m, batch->max_new),
                      "index_scores launch");
}

int csa_index_topk(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens,
                   const void* q_idx, const float* w, const void* idx_cache, void* scores, int ld, int32_t* n_valid,
                   int32_t* out_idx, void* ws, size_t ws_bytes)
{
    csa::IndexArgs a;
    CHECK(index_args(layer, batch, n_tokens, q_idx, w, idx_cache, scores, ld, n_valid, &a));
    const bool bf = layer->score_fmt == CSA_FMT_BF16;
    REQUIRE(n_tokens == 0 || out_idx != nullptr, CSA_EINVAL, "out_idx is NULL");
    REQUIRE(!bf || (ld % 8 == 0 && ((uintptr_t)scores & 15) == 0), CSA_EINVAL,
            "bf16 scores: ld (%d) must be a multiple of 8 and scores 16-byte aligned", ld);
    REQUIRE(bf || csa::topk_supported(ld, layer->top_k, false), CSA_EUNSUPPORTED,
            "rows of %d scores with k=%d exceed the two-stage selector's capacity", ld, layer->top_k);
    const size_t need = index_topk_workspace(layer, n_tokens, ld);
    REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), CSA_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
            need);
    REQUIRE(!bf || ((uintptr_t)ws & 15) == 0, CSA_EINVAL, "workspace must be 16-byte aligned");
    if (n_tokens == 0) return CSA_OK;
    const hipStream_t st = (hipStream_t)stream;
    const int max_vis = batch->max_ctx / layer->m;
    if (!bf) {
        hipError_t e = csa::launch_index(st, a, max_vis, batch->max_new);
        if (e == hipSuccess)
            e = csa::launch_topk(st, 0, n_tokens, scores, ld, n_valid, layer->top_k, out_idx, ws, ld);
        return hip_status(e, "index_topk launch");
    }
    a.hist = (uint16_t*)ws;
    int chunk = 0;
    hipError_t e = csa::launch_index(st, a, max_vis, batch->max_new, &chunk);
    if (e == hipSuccess && chunk == 0)                       // scores stored without their counts
        e = csa::launch_seg_hist(st, n_tokens, scores, ld, n_valid, (uint16_t*)ws, &chunk);
    if (e == hipSuccess)
        e = csa::launch_topk_hist(st, n_tokens, scores, ld, n_valid, (const uint16_t*)ws, (ld + chunk - 1) / chunk,
                                  chunk, layer->top_k, out_idx,
                                  (char*)ws + index_topk_hist_bytes(layer, n_tokens, ld));
    return hip_status(e, "index_topk launch");
}

}  // extern "C"

// The allocation-free top-k keeps its candidate lists in this file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// never uses the array's name as an address: the device address of each
// GPU's copy is looked up once per device (hipGetSymbolAddress with that
// device current) and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[CSA_STATIC_TOPK_SCRATCH_BYTES];

namespace {

// Validates topk_select's arguments; *need = the workspace it uses.
int topk_args(int score_fmt, int n_rows, const void* scores, int ld, const int32_t* n_valid, int k,
              const int32_t* out_idx, size_t* need)
{
    REQUIRE(score_fmt == CSA_FMT_F32 || score_fmt == CSA_FMT_BF16, CSA_EINVAL, "score_fmt=%d", score_fmt);
    REQUIRE(n_rows >= 0 && ld >= 1, CSA_EINVAL, "n_rows=%d ld=%d", n_rows, ld);
    REQUIRE(k >= 1 && k <= 2048, CSA_EUNSUPPORTED, "k=%d (1..2048)", k);
    REQUIRE(n_rows == 0 || (scores != nullptr && n_valid != nullptr && out_idx != nullptr), CSA_EINVAL,
            "NULL pointer argument");
    REQUIRE(csa::topk_supported(ld, k, score_fmt == CSA_FMT_BF16), CSA_EUNSUPPORTED,
            "rows of %d scores with k=%d exceed the two-stage selector's capacity", ld, k);
    *need = csa::topk_workspace(n_rows, ld, k, score_fmt == CSA_FMT_BF16);
    return CSA_OK;
}

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int scratch_address(void** out)
{
    int dev = -1;
    CHECK(hip_status(hipGetDevice(&dev), "hipGetDevice"));
    REQUIRE(dev >= 0 && dev < MAX_DEVICES, CSA_EUNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        CHECK(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
        REQUIRE(p != nullptr, CSA_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return CSA_OK;
}

}  // namespace

extern "C" {

int csa_topk_select(void* stream, int score_fmt, int n_rows, const void* scores, int ld, const int32_t* n_valid,
                    int k, int32_t* out_idx, void* ws, size_t ws_bytes)
{
    size_t need = 0;
    CHECK(topk_args(score_fmt, n_rows, scores, ld, n_valid, k, out_idx, &need));
    REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), CSA_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
            need);
    return hip_status(csa::launch_topk((hipStream_t)stream, score_fmt == CSA_FMT_BF16, n_rows, scores, ld, n_valid, k,
                                       out_idx, ws, ld),
                      "topk_select launch");
}

int csa_topk_select_static(void* stream, int score_fmt, int n_rows, const void* scores, int ld,
                           const int32_t* n_valid, int k, int32_t* out_idx)
{
    size_t need = 0;
    CHECK(topk_args(score_fmt, n_rows, scores, ld, n_valid, k, out_idx, &need));
    REQUIRE(need <= (size_t)CSA_STATIC_TOPK_SCRATCH_BYTES, CSA_EWORKSPACE,
            "candidate lists of %zu bytes exceed the static scratch of %zu bytes", need,
            (size_t)CSA_STATIC_TOPK_SCRATCH_BYTES);
    if (n_rows == 0) return CSA_OK;
    void* ws = nullptr;
    if (need > 0) CHECK(scratch_address(&ws));
    return hip_status(csa::launch_topk((hipStream_t)stream, score_fmt == CSA_FMT_BF16, n_rows, scores, ld, n_valid, k,
                                       out_idx, ws, ld),
                      "topk_select_static launch");
}

static int attention_common(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens,
                            const void* q, const float* q_gamma, const int32_t* sel, const void* kv_cache,
                            const void* state, const float* sinks, void* out, void* ws, size_t ws_bytes)
{
    CHECK(check_batch(layer, batch, true, 2));
    REQUIRE(n_tokens >= 0, CSA_EINVAL, "n_tokens=%d", n_tokens);
    REQUIRE(n_tokens == 0 || (q != nullptr && q_gamma != nullptr && kv_cache != nullptr && state != nullptr &&
                              sinks != nullptr && out != nullptr),
            CSA_EINVAL, "NULL pointer argument");
    const int rows = (sel ? layer->top_k : batch->max_ctx / layer->m) + layer->n_win;
    const size_t need = csa::attention_workspace(n_tokens, layer->n_heads, layer->c, rows, invariant(layer));
    REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), CSA_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
            need);
    csa::AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.invariant = invariant(layer);
    a.q = q;
    a.q_gamma = q_gamma;
    a.sel = sel;
    a.k = sel ? layer->top_k : 0;
    a.kv = kv_cache;
    a.kv_block_bytes = kv_block(layer);
    a.state = state;
    a.state_stride = state_bytes(layer);
    a.win_cap = layer->win_cap;
    a.n_win = layer->n_win;
    a.cu_new = batch->cu_new;
    a.start_pos = batch->start_pos;
    a.block_table = batch->block_table;
    a.n_req = batch->n_req;
    a.max_blocks = batch->max_blocks;
    a.m = layer->m;
    a.epb = layer->block_tokens / layer->m;
    a.epb_log2 = __builtin_ctz((unsigned)a.epb);
    a.c = layer->c;
    a.r = layer->rope_dim;
    a.nh = layer->n_heads;
    a.kv_fmt = layer->kv_fmt;
    a.q_bf16 = layer->act_fmt == CSA_FMT_BF16;
    a.win_bf16 = layer->act_fmt == CSA_FMT_BF16;
    a.out_bf16 = layer->out_fmt == CSA_FMT_BF16;
    a.eps = layer->norm_eps;
    a.theta = layer->rope_theta;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)layer->c));
    a.sinks = sinks;
    a.out = out;
    a.ws = (float*)ws;
    a.n_tokens = n_tokens;
    a.rows_max = rows;
    a.one_per_req = batch->max_new <= 1 && n_tokens == batch->n_req;
    return hip_status(csa::launch_attention((hipStream_t)stream, a), "attention launch");
}

int csa_sparse_mqa(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens, const void* q,
                   const float* q_gamma, const int32_t* sel, const void* kv_cache, const void* state,
                   const float* sinks, void* out, void* ws, size_t ws_bytes)
{
    CHECK(check_layer(layer));
    REQUIRE(is_csa(layer), CSA_EINVAL, "sparse_mqa needs a CSA layer");
    REQUIRE(n_tokens == 0 || sel != nullptr, CSA_EINVAL, "sel is NULL");
    return attention_common(stream, layer, batch, n_tokens, q, q_gamma, sel, kv_cache, state, sinks, out, ws, ws_bytes);
}

int csa_hca_attention(void* stream, const csa_layer_desc* layer, const csa_batch* batch, int n_tokens, const void* q,
                      const float* q_gamma, const void* kv_cache, const void* state, const float* sinks, void* out,
                      void* ws, size_t ws_bytes)
{
    CHECK(check_layer(layer));
    return attention_common(stream, layer, batch, n_tokens, q, q_gamma, nullptr, kv_cache, state, sinks, out, ws,
                            ws_bytes);
}

// ---- dense projections around the path ------------------------------------

int csa_grouped_linear(void* stream, int act_fmt, int out_fmt, int n_rows, int groups, int K, int N, const void* X,
                       const void* W, void* Y)
{
    REQUIRE(act_fmt == CSA_FMT_F32 || act_fmt == CSA_FMT_BF16, CSA_EINVAL, "act_fmt=%d", act_fmt);
    REQUIRE(out_fmt == CSA_FMT_F32 || out_fmt == CSA_FMT_BF16, CSA_EINVAL, "out_fmt=%d", out_fmt);
    REQUIRE(n_rows >= 0 && groups >= 1 && N >= 1, CSA_EINVAL, "n_rows=%d groups=%d N=%d", n_rows, groups, N);
    REQUIRE(K >= 128 && K % 128 == 0, CSA_EUNSUPPORTED, "K=%d must be a positive multiple of 128", K);
    REQUIRE(n_rows <= 65535 * 16 && groups <= 65535, CSA_EUNSUPPORTED, "n_rows=%d groups=%d", n_rows, groups);
    if (n_rows == 0) return CSA_OK;
    REQUIRE(X != nullptr && W != nullptr && Y != nullptr, CSA_EINVAL, "X / W / Y is NULL");
    REQUIRE((((uintptr_t)X | (uintptr_t)W | (uintptr_t)Y) & 15) == 0, CSA_EINVAL, "pointers must be 16-byte aligned");
    return hip_status(csa::launch_linear((hipStream_t)stream, act_fmt == CSA_FMT_BF16, n_rows, K, N, groups, X, W, Y,
                                         out_fmt == CSA_FMT_BF16),
                      "linear launch");
}

int csa_linear(void* stream, int act_fmt, int out_fmt, int n_rows, int K, int N, const void* X, const void* W,
               void* Y)
{
    return csa_grouped_linear(stream, act_fmt, out_fmt, n_rows, 1, K, N, X, W, Y);
}

// ---- prefix reuse (host-memory tier) --------------------------------------

// Device address of a host buffer the device may read and write (pinned host
// memory, or device memory), or null.
static void* device_visible(void* host)
{
    if (host == nullptr) return nullptr;
    hipPointerAttribute_t at;
    const hipError_t e = hipPointerGetAttributes(&at, host);
    if (e != hipSuccess) {
        (void)hipGetLastError();                  // pageable memory: clear the error it leaves
        return nullptr;
    }
    if (at.type != hipMemoryTypeHost && at.type != hipMemoryTypeDevice) return nullptr;
    return at.devicePointer != nullptr ? at.devicePointer : host;
}

int csa_prefix_bytes(const csa_layer_desc* layer, int n_blocks, size_t* bytes)
{
    CHECK(check_layer(layer));
    REQUIRE(n_blocks >= 0 && bytes != nullptr, CSA_EINVAL, "n_blocks=%d / bytes", n_blocks);
    *bytes = (size_t)n_blocks * (kv_block(layer) + idx_block(layer));
    return CSA_OK;
}

int csa_prefix_blocks(void* stream, const csa_layer_desc* layer, int n_blocks, const int32_t* block_ids,
                      void* kv_cache, void* idx_cache, void* host, int dir)
{
    CHECK(check_layer(layer));
    const bool csa = is_csa(layer);
    REQUIRE(dir == CSA_TO_HOST || dir == CSA_FROM_HOST, CSA_EINVAL, "dir=%d", dir);
    REQUIRE(n_blocks >= 0, CSA_EINVAL, "n_blocks=%d", n_blocks);
    if (n_blocks == 0) return CSA_OK;
    REQUIRE(block_ids != nullptr && kv_cache != nullptr && (!csa || idx_cache != nullptr), CSA_EINVAL,
            "block_ids / kv_cache / idx_cache is NULL");
    REQUIRE(kv_block(layer) % 16 == 0 && idx_block(layer) % 16 == 0, CSA_EUNSUPPORTED, "block bytes not 16-aligned");
    char* h = (char*)device_visible(host);
    REQUIRE(h != nullptr && ((uintptr_t)h & 15) == 0, CSA_EINVAL,
            "host buffer must be 16-byte aligned pinned host memory (hipHostMalloc / pin_memory)");
    const hipStream_t st = (hipStream_t)stream;
    hipError_t e = csa::launch_prefix_blocks(st, n_blocks, block_ids, kv_cache, kv_block(layer), h, dir);
    if (e == hipSuccess && csa)
        e = csa::launch_prefix_blocks(st, n_blocks, block_ids, idx_cache, idx_block(layer),
                                      h + (size_t)n_blocks * kv_block(layer), dir);
    return hip_status(e, "prefix_blocks launch");
}

int csa_prefix_state(void* stream, const csa_layer_desc* layer, void* state_slot, void* host, int dir)
{
    CHECK(check_layer(layer));
    REQUIRE(dir == CSA_TO_HOST || dir == CSA_FROM_HOST, CSA_EINVAL, "dir=%d", dir);
    REQUIRE(state_slot != nullptr, CSA_EINVAL, "state_slot is NULL");
    REQUIRE(device_visible(host) != nullptr, CSA_EINVAL,
            "host buffer must be pinned host memory (hipHostMalloc / pin_memory)");
    const size_t n = state_bytes(layer);
    const hipError_t e = dir == CSA_TO_HOST
        ? hipMemcpyAsync(host, state_slot, n, hipMemcpyDeviceToHost, (hipStream_t)stream)
        : hipMemcpyAsync(state_slot, host, n, hipMemcpyHostToDevice, (hipStream_t)stream);
    return hip_status(e, "prefix_state copy");
}

}  // extern "C"
