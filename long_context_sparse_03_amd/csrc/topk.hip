// a4: exact top-k selection on gfx950 ("DeepSeek-V4 内部机制" §1.2 Step 2:
// keep the k best index scores per query; m.admirer.cn: k = 512 / 1024;
// BF16 scores, §6.2).
//
// Scores become order-preserving unsigned keys (sign-magnitude flip; -0 and
// +0 map to the same key), so selection is integer work and bit-exact.  The
// order is (key descending, index ascending): the k-th element is found by
// an MSB-first radix select with 8-bit digits (histograms in LDS), and the
// selected set is compacted in index order with two block-wide prefix sums,
// which also breaks ties at the threshold toward lower indices.
//
// Rows longer than one chunk run in two stages: each chunk keeps its own
// top-k (in index order) as candidates, and a second pass selects from the
// concatenated candidates.  Every element of the global top-k is in its
// chunk's top-k under the same total order, so the result is the same.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_CHUNK = 16384;        // elements per first-stage workgroup when rows are long

CSA_DEV uint32_t score_key(const void* base, size_t i, bool bf16)
{
    uint32_t u;
    if (bf16) {
        uint32_t b = ((const uint16_t*)base)[i];
        if ((b & 0x7FFFu) == 0u) b = 0u;
        b = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
        return b << 16;
    }
    u = ((const uint32_t*)base)[i];
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block (fixed order); *total gets the sum.
CSA_DEV int block_exscan(int v, int* sh, int* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = v;
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    __syncthreads();
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    int off = 0, tot = 0;
    for (int i = 0; i < nw; ++i) {
        if (i < w) off += sh[i];
        tot += sh[i];
    }
    *total = tot;
    return off + inc - v;
}

// Select the top kk (kk <= n) of keys key(i), i < n, by (key desc, i asc) and
// write the selected positions, ascending, through emit(rank, i).
template <class KeyF, class EmitF>
CSA_DEV void select_top(int n, int kk, int min_shift, KeyF key, EmitF emit)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_prefix, sh_rem;
    __shared__ int scan_sh[32];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (n + nt - 1) / nt;
    const int i0 = tid * per, i1 = min(n, i0 + per);
    uint32_t prefix = 0, mask = 0, rem = (uint32_t)kk;
    const bool all = kk >= n;
    if (!all) {
        for (int shift = 24; shift >= min_shift; shift -= 8) {
            for (int b = tid; b < 256; b += nt) hist[b] = 0;
            __syncthreads();
            for (int i = i0; i < i1; ++i) {
                uint32_t k = key(i);
                if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t cum = 0;
                for (int b = 255; b >= 0; --b) {
                    uint32_t h = hist[b];
                    if (cum + h >= rem) {
                        sh_prefix = prefix | ((uint32_t)b << shift);
                        sh_rem = rem - cum;
                        break;
                    }
                    cum += h;
                }
            }
            __syncthreads();
            prefix = sh_prefix;
            rem = sh_rem;
            mask |= 255u << shift;
            __syncthreads();
        }
    }
    // prefix = threshold key T (keys above T are all taken), rem = how many
    // keys equal to T to take, lowest positions first.
    int eq = 0;
    if (!all)
        for (int i = i0; i < i1; ++i) eq += key(i) == prefix;
    int tot;
    int eq_before = block_exscan(eq, scan_sh, &tot);
    int sel = 0;
    {
        int er = eq_before;
        for (int i = i0; i < i1; ++i) {
            uint32_t k = key(i);
            bool s = all || k > prefix || (k == prefix && (uint32_t)(er++) < rem);
            sel += s;
        }
    }
    int out_before = block_exscan(sel, scan_sh, &tot);
    {
        int er = eq_before, o = out_before;
        for (int i = i0; i < i1; ++i) {
            uint32_t k = all ? 0u : key(i);
            bool s = all || k > prefix || (k == prefix && (uint32_t)(er++) < rem);
            if (s) emit(o++, i);
        }
    }
}

// Stage 1 (or the only stage): chunk blockIdx.x of row blockIdx.y.
__global__ __launch_bounds__(TOPK_THREADS) void topk_chunk_kernel(const void* scores, int ld, int bf16,
                                                                  const int32_t* n_valid, int k, int chunk,
                                                                  int n_chunks, int32_t* out, uint32_t* cand_key,
                                                                  int32_t* cand_idx)
{
    const int row = blockIdx.y, ch = blockIdx.x;
    const int V = n_valid[row];
    const int start = ch * chunk;
    const int n = max(0, min(V, start + chunk) - start);
    const int kk = min(k, n);
    const char* base = (const char*)scores + ((size_t)row * ld + start) * (bf16 ? 2 : 4);
    const bool isbf = bf16 != 0;
    auto key = [&](int i) { return score_key(base, (size_t)i, isbf); };
    if (n_chunks == 1) {
        int32_t* o = out + (size_t)row * k;
        select_top(n, kk, isbf ? 16 : 0, key, [&](int r, int i) { o[r] = start + i; });
        for (int r = kk + threadIdx.x; r < k; r += blockDim.x) o[r] = -1;
    } else {
        uint32_t* ck = cand_key + ((size_t)row * n_chunks + ch) * k;
        int32_t* ci = cand_idx + ((size_t)row * n_chunks + ch) * k;
        select_top(n, kk, isbf ? 16 : 0, key, [&](int r, int i) { ck[r] = key(i); ci[r] = start + i; });
        for (int r = kk + threadIdx.x; r < k; r += blockDim.x) { ck[r] = 0u; ci[r] = -1; }
    }
}

// Stage 2: select from the n_chunks*k candidates of row blockIdx.x.  Invalid
// candidates carry key 0, below every real key.
__global__ __launch_bounds__(TOPK_THREADS) void topk_merge_kernel(const int32_t* n_valid, int k, int n_chunks,
                                                                  const uint32_t* cand_key, const int32_t* cand_idx,
                                                                  int bf16, int32_t* out)
{
    const int row = blockIdx.x;
    const int V = n_valid[row];
    const int kk = min(k, V);
    const int n = n_chunks * k;
    const uint32_t* ck = cand_key + (size_t)row * n;
    const int32_t* ci = cand_idx + (size_t)row * n;
    int32_t* o = out + (size_t)row * k;
    select_top(n, kk, bf16 ? 16 : 0, [&](int i) { return ck[i]; }, [&](int r, int i) { o[r] = ci[i]; });
    for (int r = kk + threadIdx.x; r < k; r += blockDim.x) o[r] = -1;
}

static int chunk_for(int max_cols)
{
    return max_cols <= 2 * TOPK_CHUNK ? (max_cols > 0 ? max_cols : 1) : TOPK_CHUNK;
}

size_t topk_workspace(int n_rows, int max_cols, int k)
{
    int chunk = chunk_for(max_cols);
    int n_chunks = (max_cols + chunk - 1) / chunk;
    if (n_chunks <= 1) return 0;
    return (size_t)n_rows * n_chunks * k * 8;
}

hipError_t launch_topk(hipStream_t st, int score_bf16, int n_rows, const void* scores, int ld,
                       const int32_t* n_valid, int k, int32_t* out, void* ws, int max_cols)
{
    if (n_rows <= 0) return hipSuccess;
    const int chunk = chunk_for(max_cols);
    const int n_chunks = max(1, (max_cols + chunk - 1) / chunk);
    uint32_t* ck = (uint32_t*)ws;
    int32_t* ci = n_chunks > 1 ? (int32_t*)((char*)ws + (size_t)n_rows * n_chunks * k * 4) : nullptr;
    topk_chunk_kernel<<<dim3(n_chunks, n_rows), TOPK_THREADS, 0, st>>>(scores, ld, score_bf16, n_valid, k, chunk,
                                                                       n_chunks, out, ck, ci);
    if (n_chunks > 1)
        topk_merge_kernel<<<n_rows, TOPK_THREADS, 0, st>>>(n_valid, k, n_chunks, ck, ci, score_bf16, out);
    return hipGetLastError();
}

}  // namespace csa
