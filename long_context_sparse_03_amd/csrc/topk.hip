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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int TOPK_THREADS = 1024;
constexpr int MAX_K = 2048;                                  // largest k the entry points accept
constexpr int CAP16 = 40960;             // bf16 keys per workgroup (16-bit keys in LDS)
constexpr int CAP32 = 20480;             // fp32 keys per workgroup

// Order-preserving key of a score: sign-magnitude flip; -0 and +0 share the key.
CSA_DEV uint32_t key16(uint32_t b)
{
    if ((b & 0x7FFFu) == 0u) b = 0u;
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

CSA_DEV uint32_t key32(uint32_t u)
{
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

// Select the top kk of the n keys in LDS (order: key descending, position
// ascending) and emit the selected positions in ascending order through
// emit(rank, position).  BITS = key width (16 or 32).  The threshold is
// found MSB first with an 11-bit first digit (sign, exponent and the top
// mantissa bits, so that clustered scores spread over many bins) and
// histograms kept in four interleaved copies to cut atomic contention.
// Keys below lo are known to lie under the threshold: the histograms skip
// them (the caller guarantees at least kk keys >= lo).
template <int BITS, class KT, class EmitF>
CSA_DEV void select_top(const KT* keys, int n, int kk, EmitF emit, uint32_t lo = 0u)
{
    constexpr int COPIES = 4;
    __shared__ uint32_t hist[2048 * COPIES];
    __shared__ uint32_t sh_prefix, sh_rem;
    __shared__ int scan_sh[32];
    const int tid = threadIdx.x, nt = blockDim.x;
    uint32_t prefix = 0, mask = 0, rem = (uint32_t)kk;
    const bool all = kk >= n;
    if (!all) {
        int hi = BITS;                                          // digits: 11, then 5 (16-bit) or 11, 10 (32-bit)
        while (hi > 0) {
            const int width = hi == BITS ? 11 : (hi > 11 ? 11 : hi);
            const int shift = hi - width;
            const int nb = 1 << width;
            for (int b = tid; b < nb * COPIES; b += nt) hist[b] = 0;
            __syncthreads();
            for (int i = tid; i < n; i += nt) {                 // strided: conflict-free LDS reads
                const uint32_t k = keys[i];
                if (k >= lo && (k & mask) == prefix) atomicAdd(&hist[((k >> shift) & (uint32_t)(nb - 1)) * COPIES + (tid & 3)], 1u);
            }
            __syncthreads();
            // bpt consecutive bins per thread, from the top: thread tid owns
            // bins nb-1-bpt*tid down to nb-bpt*(tid+1)
            const int bpt = (nb + nt - 1) / nt;
            const int btop = nb - 1 - bpt * tid;
            uint32_t cnt = 0;
            for (int j = 0; j < bpt; ++j) {
                const int b = btop - j;
                if (b >= 0)
                    for (int c = 0; c < COPIES; ++c) cnt += hist[b * COPIES + c];
            }
            int tot;
            uint32_t above = (uint32_t)block_exscan((int)cnt, scan_sh, &tot);
            if (above < rem && rem <= above + cnt) {
                for (int j = 0; j < bpt; ++j) {
                    const int b = btop - j;
                    if (b < 0) break;
                    uint32_t cb = 0;
                    for (int c = 0; c < COPIES; ++c) cb += hist[b * COPIES + c];
                    if (rem <= above + cb) {
                        sh_prefix = prefix | ((uint32_t)b << shift);
                        sh_rem = rem - above;
                        break;
                    }
                    above += cb;
                }
            }
            __syncthreads();
            prefix = sh_prefix;
            rem = sh_rem;
            mask |= (uint32_t)(nb - 1) << shift;
            hi = shift;
        }
    }
    // prefix = threshold key T (keys above T are all taken); rem = how many
    // keys equal to T to take, lowest positions first.
    const int per = (n + nt - 1) / nt;
    const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
    int eq = 0;
    if (!all)
        for (int i = i0; i < i1; ++i) eq += (uint32_t)keys[i] == prefix;
    int tot;
    const int eq_before = block_exscan(eq, scan_sh, &tot);
    int sel = 0;
    {
        int er = eq_before;
        for (int i = i0; i < i1; ++i) {
            uint32_t k = keys[i];
            sel += all || k > prefix || (k == prefix && (uint32_t)(er++) < rem);
        }
    }
    const int out_before = block_exscan(sel, scan_sh, &tot);
    {
        int er = eq_before, o = out_before;
        for (int i = i0; i < i1; ++i) {
            uint32_t k = keys[i];
            if (all || k > prefix || (k == prefix && (uint32_t)(er++) < rem)) emit(o++, i);
        }
    }
}

// Stage 1 (or the only stage): chunk blockIdx.x of row blockIdx.y.
template <bool BF16>
__global__ __launch_bounds__(TOPK_THREADS) void topk_chunk_kernel(const void* scores, int ld,
                                                                  const int32_t* n_valid, int k, int chunk,
                                                                  int n_chunks, int32_t* out, uint32_t* cand_key,
                                                                  int32_t* cand_idx)
{
    using KT = typename std::conditional<BF16, uint16_t, uint32_t>::type;
    __shared__ KT keys[BF16 ? CAP16 : CAP32];
    const int row = blockIdx.y, ch = blockIdx.x;
    const int V = n_valid[row];
    const int start = ch * chunk;
    const int n = max(0, min(V, start + chunk) - start);
    const int kk = min(k, n);
    // stage the chunk's keys in LDS; 16-byte loads, four in flight per thread
    const size_t off = (size_t)row * ld + start;
    constexpr int EPL = BF16 ? 8 : 4;                       // scores per 16-byte load
    const int head = (int)min((size_t)n, (EPL - off % EPL) % EPL);   // scalar prologue up to alignment
    const char* base = (const char*)scores + off * (BF16 ? 2 : 4);
    for (int i = threadIdx.x; i < head; i += blockDim.x)
        keys[i] = (KT)(BF16 ? key16(((const uint16_t*)base)[i]) : key32(((const uint32_t*)base)[i]));
    const int nvec = (n - head) / EPL;
    const char* vbase = base + (size_t)head * (BF16 ? 2 : 4);
    for (int v0 = threadIdx.x; v0 < nvec; v0 += 4 * blockDim.x) {
        uint4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = min(v0 + u * (int)blockDim.x, nvec - 1);
            q[u] = ld16(vbase + (size_t)v * 16);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * (int)blockDim.x;
            if (v >= nvec) break;
            const uint32_t w4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
            KT* dst = keys + head + v * EPL;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if (BF16) {
                    dst[2 * h] = (KT)key16(w4[h] & 0xFFFFu);
                    dst[2 * h + 1] = (KT)key16(w4[h] >> 16);
                } else {
                    dst[h] = (KT)key32(w4[h]);
                }
            }
        }
    }
    for (int i = head + nvec * EPL + threadIdx.x; i < n; i += blockDim.x)
        keys[i] = (KT)(BF16 ? key16(((const uint16_t*)base)[i]) : key32(((const uint32_t*)base)[i]));
    __syncthreads();
    // one stage: final indices; first of two: candidates (key, index) per chunk
    const bool single = n_chunks == 1;
    int32_t* o = single ? out + (size_t)row * k : cand_idx + ((size_t)row * n_chunks + ch) * k;
    uint32_t* ck = single ? nullptr : cand_key + ((size_t)row * n_chunks + ch) * k;
    select_top<BF16 ? 16 : 32>(keys, n, kk, [&](int r, int i) {
        o[r] = start + i;
        if (!single) ck[r] = keys[i];
    });
    for (int r = kk + threadIdx.x; r < k; r += blockDim.x) {
        o[r] = -1;
        if (!single) ck[r] = 0u;
    }
}

// Stage 2: select from the n_chunks*k candidates of row blockIdx.x.  Invalid
// candidates carry key 0, below every real key; candidates are in ascending
// index order, so position order is index order.
template <bool BF16>
__global__ __launch_bounds__(TOPK_THREADS) void topk_merge_kernel(const int32_t* n_valid, int k, int n_chunks,
                                                                  const uint32_t* cand_key, const int32_t* cand_idx,
                                                                  int32_t* out)
{
    using KT = typename std::conditional<BF16, uint16_t, uint32_t>::type;
    __shared__ KT keys[BF16 ? CAP16 : CAP32];
    const int row = blockIdx.x;
    const int V = n_valid[row];
    const int kk = min(k, V);
    const int n = n_chunks * k;
    const uint32_t* ck = cand_key + (size_t)row * n;
    const int32_t* ci = cand_idx + (size_t)row * n;
    __shared__ uint32_t floor_sh;
    if (threadIdx.x == 0) floor_sh = 0u;
    for (int i = threadIdx.x; i < n; i += blockDim.x) keys[i] = (KT)ck[i];
    __syncthreads();
    // Each chunk holds k keys >= its smallest candidate key (a chunk with
    // fewer valid keys is padded with key 0), so the row's k-th largest key is
    // at least the largest of these minima: keys below it cannot be selected.
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    for (int c = threadIdx.x >> 6; c < n_chunks; c += nw) {
        uint32_t mn = 0xFFFFFFFFu;
        for (int i = lane; i < k; i += 64) mn = min(mn, (uint32_t)keys[c * k + i]);
        for (int o = 32; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
        if (lane == 0) atomicMax(&floor_sh, mn);
    }
    __syncthreads();
    const uint32_t lo = floor_sh;
    // selected positions go to LDS first, so that the index lookups below
    // are issued together rather than one dependent load after another
    __shared__ int32_t spos[MAX_K];
    select_top<BF16 ? 16 : 32>(keys, n, kk, [&](int r, int i) { spos[r] = i; }, lo);
    __syncthreads();
    int32_t* o = out + (size_t)row * k;
    for (int r = threadIdx.x; r < k; r += blockDim.x) o[r] = r < kk ? ci[spos[r]] : -1;
}

// Chunk length per first-stage workgroup: at most the LDS capacity; when
// there are few rows the chunks shrink (down to 4k keys each) so that more
// workgroups share the work, as long as the candidates still fit one
// second-stage workgroup.
static int chunk_for(int n_rows, int max_cols, int k, bool bf16)
{
    const int cap = bf16 ? CAP16 : CAP32;
    int chunk = max_cols <= cap ? (max_cols > 0 ? max_cols : 1) : cap;
    auto nch = [&](int c) { return (max_cols + c - 1) / c; };
    while ((long)n_rows * nch(chunk) < 256 && chunk / 2 >= 4 * k && (long)nch(chunk / 2) * k <= cap) chunk /= 2;
    return chunk;
}

size_t topk_workspace(int n_rows, int max_cols, int k, bool bf16)
{
    const int chunk = chunk_for(n_rows, max_cols, k, bf16);
    const int n_chunks = (max_cols + chunk - 1) / chunk;
    if (n_chunks <= 1) return 0;
    return (size_t)n_rows * n_chunks * k * 8;
}

bool topk_supported(int max_cols, int k, bool bf16)
{
    const int cap = bf16 ? CAP16 : CAP32;
    const int chunk = max_cols <= cap ? max_cols : cap;
    const int n_chunks = (max_cols + chunk - 1) / chunk;
    return n_chunks <= 1 || (long)n_chunks * k <= cap;
}

hipError_t launch_topk(hipStream_t st, int score_bf16, int n_rows, const void* scores, int ld,
                       const int32_t* n_valid, int k, int32_t* out, void* ws, int max_cols)
{
    if (n_rows <= 0) return hipSuccess;
    const bool bf = score_bf16 != 0;
    const int chunk = chunk_for(n_rows, max_cols, k, bf);
    const int n_chunks = max(1, (max_cols + chunk - 1) / chunk);
    const int threads1 = chunk <= 8192 ? 256 : TOPK_THREADS;
    uint32_t* ck = (uint32_t*)ws;
    int32_t* ci = n_chunks > 1 ? (int32_t*)((char*)ws + (size_t)n_rows * n_chunks * k * 4) : nullptr;
    dim3 g1(n_chunks, n_rows);
    if (bf) topk_chunk_kernel<true><<<g1, threads1, 0, st>>>(scores, ld, n_valid, k, chunk, n_chunks, out, ck, ci);
    else topk_chunk_kernel<false><<<g1, threads1, 0, st>>>(scores, ld, n_valid, k, chunk, n_chunks, out, ck, ci);
    if (n_chunks > 1) {
        if (bf) topk_merge_kernel<true><<<n_rows, TOPK_THREADS, 0, st>>>(n_valid, k, n_chunks, ck, ci, out);
        else topk_merge_kernel<false><<<n_rows, TOPK_THREADS, 0, st>>>(n_valid, k, n_chunks, ck, ci, out);
    }
    return hipGetLastError();
}

}  // namespace csa
