// Argument blocks and host-side launchers of the gfx950 kernels.  Everything
// here is internal to libcsa.so; the public interface is include/csa.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

struct CompressArgs {
    float* P;                  // projection workspace [n_tokens x ncols]
    int ncols;
    void* state;               // state slots
    size_t state_stride;       // bytes per slot
    size_t tail_off;           // byte offset of the tail ring inside a slot
    int R;                     // tail ring rows
    const int32_t* cu_new;
    const int32_t* start_pos;
    int n_req;
    int m, overlap, c, c_idx, r;
    const float *B_a, *B_b, *B_a_idx, *B_b_idx, *gamma;
    float eps, theta;
    float* out_entries;
    float* out_keys;
    int32_t* out_meta;
    int32_t* out_count;
    int max_entries;
    float* out_win;
    int max_new;               // largest number of new tokens of one request
    int one_per_req;           // set by launch_compress: every request has exactly one new token
    int invariant;             // batch-invariant layer: the projection kernel does not depend on the row count
    int32_t* next_pos;         // [n_req] or null: start_pos + new tokens, written by the post-projection kernel
    int n_psplit;              // set by launch_compress: P holds this many partial products ...
    size_t psplit_stride;      // ... this many floats apart, which readers add in order
};

// Few-row bf16 projections (and every projection of a batch-invariant layer)
// are PROJ_PARTS partial products over equal chunks of the contraction.
constexpr int PROJ_PARTS = 4;
int proj_parts(bool bf16, bool invariant, int n_rows);
// compress_kv's workspace for calls of up to n_rows rows (never less for more rows)
size_t compress_workspace(bool bf16, bool invariant, int n_rows, int ncols);

// Y[M x groups*N] = per group g: X[:, g*K .. g*K+K) . W[g]^T, W [groups x N x K];
// X, W bf16 (bf16) or fp32, Y fp32 or (out_bf16) bf16.
hipError_t launch_linear(hipStream_t st, bool bf16, int M, int K, int N, int groups, const void* X, const void* W,
                         void* Y, bool out_bf16);

struct AppendArgs;

// app: also append the outputs to the caches (one fused decode kernel when
// every request has at most one new token, else the append launch after)
hipError_t launch_compress(hipStream_t st, const CompressArgs& a, const void* H, const void* W, const void* Wi,
                           int n_main, int d, bool bf16, int n_tokens, const AppendArgs* app = nullptr);

struct AppendArgs {
    const float* entries;
    const float* keys;
    const int32_t* meta;
    const int32_t* count;
    int max_entries;
    const float* win;
    int n_tokens;
    const int32_t* cu_new;
    const int32_t* start_pos;
    const int32_t* block_table;
    int n_req, max_blocks;
    int c, r, c_idx, epb;
    int kv_fmt, idx_fmt, win_bf16;
    void* kv;
    size_t kv_block_bytes;
    void* idx;
    size_t idx_block_bytes;
    void* state;
    size_t state_stride;
    int win_cap;
    int one_per_req;           // every request has exactly one new token (token g is request g's)
};

hipError_t launch_append(hipStream_t st, const AppendArgs& a);

struct IndexArgs {
    const void* q;             // [n_tokens x nh x cI] f32 or bf16
    const float* w;            // [n_tokens x nh]
    const void* keys;          // indexer-key pool
    size_t key_block_bytes;
    const int32_t* cu_new;
    const int32_t* start_pos;
    const int32_t* block_table;
    int n_req, max_blocks;
    int m, epb, epb_log2, nh, cI;
    int q_bf16, idx_fmt, score_bf16;
    void* scores;
    int ld;
    int32_t* n_valid;
    int n_tokens;
    int one_per_req;           // set by launch_index: every request has exactly one new token
    uint16_t* hist;            // or null: per (row, chunk of entries) counts of the bf16 scores by the top 8
                               // bits of their order-preserving key, 256 per chunk (the fused top-k's first digit)
    int hist_chunks;           // chunks per row in hist (set by launch_index from the chunk it launches)
};

// *chunk (if not null): entries per histogram chunk of the launch chosen
hipError_t launch_index(hipStream_t st, const IndexArgs& a, int max_visible, int max_new, int* chunk = nullptr);
// Entries per histogram chunk of the smallest chunk any index launch of this key format uses.
int index_min_chunk(int idx_fmt);

// The fused top-k's selection (bf16 scores, ld % 8 == 0): the k-th key's top 8
// bits from the indexer's per-chunk counts, then a counting and an emitting
// pass over segments of each row (many workgroups per row); ws holds the
// per-segment counts (topk_hist_workspace bytes, 16-byte aligned).
hipError_t launch_seg_hist(hipStream_t st, int n_rows, const void* scores, int ld, const int32_t* n_valid,
                           uint16_t* hist, int* chunk);
hipError_t launch_topk_hist(hipStream_t st, int n_rows, const void* scores, int ld, const int32_t* n_valid,
                            const uint16_t* hist, int hist_chunks, int chunk, int k, int32_t* out, void* ws);
size_t topk_hist_workspace(int n_rows, int ld);

hipError_t launch_topk(hipStream_t st, int score_bf16, int n_rows, const void* scores, int ld,
                       const int32_t* n_valid, int k, int32_t* out, void* ws, int max_cols);
size_t topk_workspace(int n_rows, int max_cols, int k, bool bf16);
bool topk_supported(int max_cols, int k, bool bf16);

struct AttnArgs {
    const void* q;             // [n_tokens x nh x c] f32 or bf16
    const float* q_gamma;
    const int32_t* sel;        // [n_tokens x k] or null (dense)
    int k;
    const void* kv;
    size_t kv_block_bytes;
    const void* state;
    size_t state_stride;
    int win_cap, n_win;
    const int32_t* cu_new;
    const int32_t* start_pos;
    const int32_t* block_table;
    int n_req, max_blocks;
    int m, epb, epb_log2, c, r, nh;
    int kv_fmt, q_bf16, win_bf16, out_bf16;
    float eps, theta, scale_log2;
    const float* sinks;
    void* out;
    float* ws;                 // split partials
    int n_tokens;
    int rows_max;              // rows per query (slots): k + n_win, or max entries + n_win
    int n_splits;
    int tiles_per_split;
    int one_per_req;           // every request has exactly one new token (query gq is request gq's)
    int invariant;             // batch-invariant layer: fixed split boundaries, always split partials + combine
    double inv_freq[32];       // RoPE frequencies theta^(-2j/r), j < r/2 (filled by launch_attention)
};

// Prefix reuse: n_blocks blocks (ids, device) of a pool to / from host (dir 0 / 1).
hipError_t launch_prefix_blocks(hipStream_t st, int n_blocks, const int32_t* ids, void* pool, size_t block_bytes,
                                void* host, int dir);

int attention_splits(int n_tokens, int n_heads, int rows_max);
size_t attention_workspace(int n_tokens, int n_heads, int c, int rows_max, bool invariant);
hipError_t launch_attention(hipStream_t st, AttnArgs a);

}  // namespace csa
