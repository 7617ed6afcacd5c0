// a4: exact top-k selection on gfx950 ("DeepSeek-V4 内部机制" §1.2 Step 2:
// keep the k best index scores per query; m.admirer.cn: k = 512 / 1024;
// BF16 scores, §6.2).
//
// Scores become order-preserving unsigned keys (sign-magnitude flip; -0 and
// +0 map to the same key), so selection is integer work and bit-exact.  The
// order is (key descending, index ascending).  A workgroup holds its keys in
// registers, each thread a run of consecutive positions.  The k-th key is
// found with histograms over the range [smallest, largest] of the keys in
// play (at most 2048 bins, narrowed to the selected bin until bins are single
// keys: one pass when the range spans at most 2048 keys), and the selected
// set is emitted in index order from one block-wide scan, which also breaks
// ties at the threshold toward lower indices.  Before that, a lower bound
// from the per-thread maxima usually leaves only a few per cent of the keys
// in play.
//
// Rows longer than one workgroup run in two stages: each chunk keeps its own
// top-k (in index order) as candidates, and a second pass selects from the
// concatenated candidates.  Every element of the global top-k is in its
// chunk's top-k under the same total order, so the result is the same.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int TOPK_THREADS = 1024;
constexpr int MAX_K = 2048;                   // largest k the entry points accept
constexpr int CAP16 = 40960;                  // bf16 keys per workgroup
constexpr int CAP32 = 20480;                  // fp32 keys per workgroup
constexpr int KPT16 = CAP16 / TOPK_THREADS;   // keys per thread at the capacity
constexpr int KPT32 = CAP32 / TOPK_THREADS;
constexpr int SMALL_NT = 512, SMALL_KPT = 16; // workgroups of up to 8192 keys (512 threads: 9 us for
                                              // 16 rows of 8192, 12 us with 256 x 32)
constexpr int MID_KPT = 16;                   // 1024 threads for up to 16384 keys
constexpr int SURV_CAP = 4096;                // keys kept after the lower bound (1024-thread workgroups)

// Order-preserving key of an fp32 score (key16 for bf16 is in common.hpp):
// sign-magnitude flip; -0 and +0 share the key.
CSA_DEV uint32_t key32(uint32_t u)
{
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave: steps of 1, 2, 4, 8
// within each row of 16 lanes, then the row totals carried across rows
// (DPP row shifts and row broadcasts; lanes without a source add 0).
CSA_DEV uint32_t wave_incl_scan(uint32_t v)
{
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return (uint32_t)x;
}

// Exclusive prefix sums over the workgroup (fixed order, modulo 2^32), one
// barrier each: the wave totals alternate between two LDS slots, and a slot
// is written again only after every wave has passed the barrier of the scan
// in between.
struct BlockScan {
    int parity = 0;
    CSA_DEV uint32_t exscan(uint32_t v, uint32_t* total)
    {
        __shared__ uint32_t part[2][16];
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
        const uint32_t inc = wave_incl_scan(v);
        if (lane == 63) part[parity][w] = inc;
        __syncthreads();
        uint32_t off = 0, tot = 0;
        for (int i = 0; i < nw; ++i) {
            const uint32_t x = part[parity][i];
            tot += x;
            off += i < w ? x : 0u;
        }
        parity ^= 1;
        *total = tot;
        return off + inc - v;
    }
};

constexpr int HIST_COPIES = 4;
__shared__ uint32_t topk_hist[2048 * HIST_COPIES];  // range histograms (four interleaved copies)
__shared__ uint32_t topk_digit[2];                  // chosen bin, remaining rank

// Selection works on keys held in registers: thread tid holds the keys of
// positions tid*KPT .. tid*KPT+KPT-1, so a thread's positions are
// consecutive; positions >= n hold key 0, and every real key is >= 1 (see
// raise_keys), so kk <= n keeps them out of the selection.

// Running maximum / minimum over the lanes of a wave, in DPP steps as in
// wave_incl_scan (lanes without a source see the identity); lane 63 ends
// with the wave's extreme.
CSA_DEV uint32_t wave_max63(uint32_t v)
{
    int x = (int)v;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
    return (uint32_t)x;
}

CSA_DEV uint32_t wave_min63(uint32_t v)
{
    int x = (int)v;
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x111, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x112, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x114, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x118, 0xf, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x142, 0xa, 0xf, false));
    x = (int)min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(-1, x, 0x143, 0xc, 0xf, false));
    return (uint32_t)x;
}

// Largest and smallest value over the workgroup (DPP within waves, then the
// wave results through LDS after one barrier; the slots alternate as in
// BlockScan, whose parity this shares).
CSA_DEV void block_max_min(uint32_t& mx, uint32_t& mn, BlockScan& bs)
{
    __shared__ uint32_t part[2][2][16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint32_t a = wave_max63(mx), b = wave_min63(mn);
    if (lane == 63) {
        part[bs.parity][0][w] = a;
        part[bs.parity][1][w] = b;
    }
    __syncthreads();
    uint32_t x = 0u, y = 0xFFFFFFFFu;
    for (int i = 0; i < nw; ++i) {
        x = max(x, part[bs.parity][0][i]);
        y = min(y, part[bs.parity][1][i]);
    }
    bs.parity ^= 1;
    mx = x;
    mn = y;
}

// Histogram select over the keys in [lo, hi] (others ignored; at least rem
// of them): bins of 2^shift consecutive keys from lo, at most 2048 of them,
// counted with LDS atomics (four interleaved copies).  Returns the bin
// holding the rem-th largest key and updates rem to its rank inside the bin.
// Keys spread over the range, so few lanes hit one counter at a time.
template <int KPT>
CSA_DEV void range_bin(const uint32_t (&kr)[KPT], uint32_t lo, uint32_t hi, int shift, uint32_t& rem, BlockScan& bs,
                       uint32_t& bin)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    const int nb = (int)((hi - lo) >> shift) + 1;              // <= 2048
    for (int b = tid; b < nb * HIST_COPIES; b += nt) topk_hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t k = kr[j];
        if (k >= lo && k <= hi) atomicAdd(&topk_hist[((k - lo) >> shift) * HIST_COPIES + (tid & 3)], 1u);
    }
    __syncthreads();
    // bpt consecutive bins per thread, from the top: thread tid owns bins
    // nb-1-bpt*tid down to nb-bpt*(tid+1)
    const int bpt = (nb + nt - 1) / nt;
    const int btop = nb - 1 - bpt * tid;
    uint32_t cnt = 0;
    for (int j = 0; j < bpt; ++j) {
        const int b = btop - j;
        if (b >= 0)
            for (int c = 0; c < HIST_COPIES; ++c) cnt += topk_hist[b * HIST_COPIES + c];
    }
    uint32_t tot;
    uint32_t above = bs.exscan(cnt, &tot);
    if (above < rem && rem <= above + cnt) {
        for (int j = 0; j < bpt; ++j) {
            const int b = btop - j;
            if (b < 0) break;
            uint32_t cb = 0;
            for (int c = 0; c < HIST_COPIES; ++c) cb += topk_hist[b * HIST_COPIES + c];
            if (rem <= above + cb) {
                topk_digit[0] = (uint32_t)b;
                topk_digit[1] = rem - above;
                break;
            }
            above += cb;
        }
    }
    __syncthreads();
    bin = topk_digit[0];
    rem = topk_digit[1];
}

// Bins of 2^shift keys covering [lo, hi] in at most 2048 bins.
CSA_DEV int range_shift(uint32_t lo, uint32_t hi)
{
    int shift = 0;
    while (((hi - lo) >> shift) >= 2048u) ++shift;
    return shift;
}

// Exact threshold of the top rem keys among those in [lo, hi]: narrow the
// range to the selected bin until bins are single keys (one pass when the
// range spans at most 2048 keys).
template <int KPT>
CSA_DEV void range_threshold(const uint32_t (&kr)[KPT], uint32_t lo, uint32_t hi, uint32_t rem, BlockScan& bs,
                             uint32_t& T, uint32_t& rem_out)
{
    while (true) {
        const int shift = range_shift(lo, hi);
        uint32_t b;
        range_bin<KPT>(kr, lo, hi, shift, rem, bs, b);
        const uint32_t nlo = lo + (b << shift);
        if (shift == 0) {
            T = nlo;
            rem_out = rem;
            return;
        }
        // the selected bin's last key, without wrapping past 2^32 - 1
        hi = nlo + min(hi - nlo, (1u << shift) - 1u);
        lo = nlo;
    }
}

// Emit the keys above T and the first rem keys equal to T, in position
// order, through emit(rank, position, key) (T = 0, rem = 0 takes every real
// key).  Equal keys are taken in position order, so the threads before this
// one took min(eq_before, rem) of them: one scan of the packed counts (gt,
// eq) gives every thread its first output rank.  Equal keys are only counted
// when some are taken (rem > 0, so T >= 1 and the key-0 positions are not
// among them); both counts are then at most 40960, so the packed sums stay
// below 2^32.
template <int KPT, class EmitF>
CSA_DEV void emit_selected(const uint32_t (&kr)[KPT], int kk, uint32_t T, uint32_t rem, BlockScan& bs, EmitF emit)
{
    const int tid = threadIdx.x;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gt += kr[j] > T;
        eq += rem > 0u && kr[j] == T;
    }
    uint32_t tot;
    const uint32_t packed = bs.exscan(gt | (eq << 16), &tot);
    const int gt_before = (int)(packed & 0xFFFFu), eq_before = (int)(packed >> 16);
    int o = gt_before + min(eq_before, (int)rem);
    const int take_eq = min(max((int)rem - eq_before, 0), (int)eq);   // this thread's equal keys taken
    // an opaque copy of T: the compiler recomputes the comparisons instead of
    // keeping 2*KPT lane masks alive (they would spill)
    uint32_t t2 = T;
    asm volatile("" : "+v"(t2));
    int te = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t k = kr[j];
        const bool e = k == t2;
        if ((k > t2 || (e && te < take_eq)) && o < kk) emit(o++, tid * KPT + j, k);   // ranks stay below kk
        te += e;
    }
}

// Select the top kk of n keys and emit the selected positions in ascending
// order through emit(rank, position, key): the threshold by range
// histograms over [smallest, largest] real key.
template <int KPT, class EmitF>
CSA_DEV void select_top(const uint32_t (&kr)[KPT], int n, int kk, BlockScan& bs, EmitF emit)
{
    uint32_t T = 0, rem = 0;
    if (kk < n) {
        uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            kmax = max(kmax, kr[j]);
            kmin = min(kmin, kr[j] > 0u ? kr[j] : 0xFFFFFFFFu);
        }
        block_max_min(kmax, kmin, bs);
        range_threshold<KPT>(kr, kmin, kmax, (uint32_t)kk, bs, T, rem);
    }
    emit_selected<KPT>(kr, kk, T, rem, bs, emit);
}

// Positions >= n get key 0.  With RAISE, keys are raised to at least 1 (only
// the order among NaNs of one sign changes: keys 0 and 1 are both NaN);
// second-stage candidates are already raised, and their padding keeps key 0.
template <bool RAISE, int KPT>
CSA_DEV void raise_keys(int n, uint32_t (&kr)[KPT])
{
    const int nv = n - (int)threadIdx.x * KPT;              // keys of this thread below n
#pragma unroll
    for (int j = 0; j < KPT; ++j) kr[j] = j < nv ? (RAISE ? max(kr[j], 1u) : kr[j]) : 0u;
}

// Unpack one 16-byte vector of scores (BF16: 8 bf16, else 4 fp32) into keys.
template <bool BF16, int KPT>
CSA_DEV void unpack_keys(uint4 q, int at, uint32_t (&kr)[KPT])
{
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        if (BF16) {
            kr[at + 2 * h] = key16(w4[h] & 0xFFFFu);
            kr[at + 2 * h + 1] = key16(w4[h] >> 16);
        } else {
            kr[at + h] = key32(w4[h]);
        }
    }
}

// Scores straight into registers (16-byte aligned run whose last, partial
// vector lies inside the row): thread tid reads the vectors of its KPT
// positions; vectors past the run are clamped to its last one and masked.
template <bool BF16, int KPT>
CSA_DEV void load_keys_direct(const void* scores, size_t off, int n, uint32_t (&kr)[KPT])
{
    constexpr int EPL = BF16 ? 8 : 4, NV = KPT / EPL;
    static_assert(KPT % EPL == 0, "whole vectors per thread");
    const int nvec = (n + EPL - 1) / EPL;
    const char* base = (const char*)scores + off * (BF16 ? 2 : 4);
    uint4 q[NV];
    if (nvec > 0) {                                         // workgroup-uniform
#pragma unroll
        for (int v = 0; v < NV; ++v) q[v] = ld16(base + (size_t)min((int)threadIdx.x * NV + v, nvec - 1) * 16);
    } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) q[v] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) unpack_keys<BF16>(q[v], v * EPL, kr);
}

// Stage n scores (starting at element off of the score array) as keys in
// LDS: 16-byte loads, four in flight per thread, after a scalar prologue up
// to 16-byte alignment.
template <bool BF16, class KT>
CSA_DEV void stage_keys(const void* scores, size_t off, int n, KT* keys)
{
    constexpr int EPL = BF16 ? 8 : 4;                       // scores per 16-byte load
    const int head = (int)min((size_t)n, (EPL - off % EPL) % EPL);
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
}

// Thread tid's KPT consecutive keys from LDS into registers (16-byte reads:
// KPT * sizeof(KT) is a multiple of 16 and the array is 16-byte aligned).
template <int KPT, class KT>
CSA_DEV void keys_to_regs(const KT* keys, uint32_t (&kr)[KPT])
{
    constexpr int PER = 16 / (int)sizeof(KT);
    static_assert(KPT % PER == 0, "whole 16-byte reads");
    const uint4* p = (const uint4*)(keys + threadIdx.x * KPT);
#pragma unroll
    for (int v = 0; v < KPT / PER; ++v) {
        const uint4 q = p[v];
        const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            if (sizeof(KT) == 2) {
                kr[v * PER + 2 * h] = w4[h] & 0xFFFFu;
                kr[v * PER + 2 * h + 1] = w4[h] >> 16;
            } else {
                kr[v * PER + h] = w4[h];
            }
        }
    }
}

// Stage 1 (or the only stage): chunk blockIdx.x of row blockIdx.y, NT
// threads of KPT keys each (chunk <= NT * KPT).
template <bool BF16, int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_chunk_kernel(const void* scores, int ld, const int32_t* n_valid, int k,
                                                        int chunk, int n_chunks, int32_t* out, uint32_t* cand_key,
                                                        int32_t* cand_idx)
{
    using KT = typename std::conditional<BF16, uint16_t, uint32_t>::type;
    constexpr int EPL = BF16 ? 8 : 4;
    const int row = blockIdx.y, ch = blockIdx.x;
    const int V = min(n_valid[row], ld);                    // never past the row
    const int start = ch * chunk;
    const int n = max(0, min(V, start + chunk) - start);
    const int kk = min(k, n);
    const size_t off = (size_t)row * ld + start;
    uint32_t kr[KPT];
    // 16-byte aligned run whose partial last vector stays inside the row:
    // scores straight into registers; otherwise staged through LDS
    const bool aligned = ((uintptr_t)scores + off * (BF16 ? 2 : 4)) % 16 == 0;
    if (aligned && (n % EPL == 0 || start + (n / EPL + 1) * EPL <= ld)) {
        load_keys_direct<BF16, KPT>(scores, off, n, kr);
    } else {
        __shared__ __attribute__((aligned(16))) KT keys[NT * KPT];
        stage_keys<BF16>(scores, off, n, keys);
        __syncthreads();
        keys_to_regs<KPT>(keys, kr);
    }
    raise_keys<true, KPT>(n, kr);
    // one stage: final indices; first of two: candidates (key, index) per chunk
    const bool single = n_chunks == 1;
    int32_t* o = single ? out + (size_t)row * k : cand_idx + ((size_t)row * n_chunks + ch) * k;
    uint32_t* ck = single ? nullptr : cand_key + ((size_t)row * n_chunks + ch) * k;
    auto emit = [&](int r, int i, uint32_t key) {
        o[r] = start + i;
        if (!single) ck[r] = key;
    };
    BlockScan bs;
    bool done = false;
    if constexpr (NT == TOPK_THREADS) {
        // Lower bound first: when kk threads hold a key >= L, the threshold
        // is at least L.  L is the lower edge of the histogram bin (over the
        // range of the per-thread maxima) that holds the kk-th largest
        // maximum.  The keys >= L (typically a few per cent of the row) are
        // compacted in position order and the exact selection runs over them
        // alone, unless there are more than SURV_CAP of them (ties,
        // adversarial rows).
        constexpr int SPT = SURV_CAP / NT;
        __shared__ uint32_t skey[SURV_CAP];
        __shared__ int32_t spos[SURV_CAP];
        if (kk < n && kk <= (n + KPT - 1) / KPT) {          // workgroup-uniform: kk threads hold keys
            uint32_t m = 0u;
#pragma unroll
            for (int j = 0; j < KPT; ++j) m = max(m, kr[j]);
            uint32_t kmax = m, mmin = m > 0u ? m : 0xFFFFFFFFu;   // smallest maximum of a thread with keys
            block_max_min(kmax, mmin, bs);
            uint32_t mr[1] = {m}, remL = (uint32_t)kk, b;
            const int shift = range_shift(mmin, kmax);
            range_bin<1>(mr, mmin, kmax, shift, remL, bs, b);
            const uint32_t L = mmin + (b << shift);
            uint32_t cnt = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) cnt += kr[j] >= L;
            uint32_t S;
            uint32_t at = bs.exscan(cnt, &S);
            if (S <= (uint32_t)SURV_CAP) {                  // workgroup-uniform
#pragma unroll
                for (int j = 0; j < KPT; ++j)
                    if (kr[j] >= L) {
                        skey[at] = kr[j];
                        spos[at] = threadIdx.x * KPT + j;
                        ++at;
                    }
                __syncthreads();
                uint32_t k2[SPT];
#pragma unroll
                for (int q = 0; q < SPT; ++q) {
                    const int i = threadIdx.x * SPT + q;
                    k2[q] = i < (int)S ? skey[i] : 0u;
                }
                uint32_t T = 0, rem = 0;
                if (kk < (int)S) range_threshold<SPT>(k2, L, kmax, (uint32_t)kk, bs, T, rem);
                emit_selected<SPT>(k2, kk, T, rem, bs, [&](int r, int i, uint32_t key) { emit(r, spos[i], key); });
                done = true;
            }
        }
    }
    if (!done) select_top<KPT>(kr, n, kk, bs, emit);
    for (int r = kk + threadIdx.x; r < k; r += blockDim.x) {
        o[r] = -1;
        if (!single) ck[r] = 0u;
    }
}

// Stage 2: select from the n_chunks*k candidates of row blockIdx.x.  Invalid
// candidates carry key 0, below every real key; candidates are in ascending
// index order, so position order is index order.
template <bool BF16, int KPT = (BF16 ? KPT16 : KPT32)>
__global__ __launch_bounds__(TOPK_THREADS) void topk_merge_kernel(const int32_t* n_valid, int ld, int k, int n_chunks,
                                                                  const uint32_t* cand_key, const int32_t* cand_idx,
                                                                  int32_t* out)
{
    using KT = typename std::conditional<BF16, uint16_t, uint32_t>::type;
    __shared__ __attribute__((aligned(16))) KT keys[TOPK_THREADS * KPT];
    const int row = blockIdx.x;
    const int V = min(n_valid[row], ld);
    const int kk = min(k, V);
    const int n = n_chunks * k;
    const uint32_t* ck = cand_key + (size_t)row * n;
    const int32_t* ci = cand_idx + (size_t)row * n;
    __shared__ uint32_t floor_sh;
    if (threadIdx.x == 0) floor_sh = 0u;
    {
        // candidates into LDS: 16-byte loads, four in flight per thread,
        // after a scalar prologue up to 16-byte alignment
        const int head = (int)min((size_t)n, ((16 - (uintptr_t)ck % 16) % 16) / 4);
        for (int i = threadIdx.x; i < head; i += TOPK_THREADS) keys[i] = (KT)ck[i];
        const int nvec = (n - head) / 4;
        const uint32_t* vb = ck + head;
        for (int v0 = threadIdx.x; v0 < nvec; v0 += 4 * TOPK_THREADS) {
            uint4 q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = ld16(vb + 4 * (size_t)min(v0 + u * TOPK_THREADS, nvec - 1));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = v0 + u * TOPK_THREADS;
                if (v < nvec) {
                    KT* dst = keys + head + 4 * v;
                    dst[0] = (KT)q[u].x;
                    dst[1] = (KT)q[u].y;
                    dst[2] = (KT)q[u].z;
                    dst[3] = (KT)q[u].w;
                }
            }
        }
        for (int i = head + 4 * nvec + threadIdx.x; i < n; i += TOPK_THREADS) keys[i] = (KT)ck[i];
    }
    __syncthreads();
    uint32_t kr[KPT];
    keys_to_regs<KPT>(keys, kr);
    raise_keys<false, KPT>(n, kr);
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
    BlockScan bs;
    // the threshold by range histograms over [lo, the largest key] (one pass
    // when the candidates above the floor span at most 2048 keys)
    uint32_t kmax = 0u, dummy_min = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < KPT; ++j) kmax = max(kmax, kr[j]);
    block_max_min(kmax, dummy_min, bs);
    uint32_t T = 0, rem = 0;
    if (kk < n) range_threshold<KPT>(kr, lo, kmax, (uint32_t)kk, bs, T, rem);
    emit_selected<KPT>(kr, kk, T, rem, bs, [&](int r, int i, uint32_t) { spos[r] = i; });
    __syncthreads();
    int32_t* o = out + (size_t)row * k;
    for (int r = threadIdx.x; r < k; r += blockDim.x) o[r] = r < kk ? ci[spos[r]] : -1;
}

// ---------------------------------------------------------------------------
// Fused top-k (bf16 scores): selection from the indexer's counts, over
// segments of each row.
//
// The indexer counted each chunk's scores by the top 8 bits of their
// order-preserving key (csa::key16), so the coarse digit b* of the k-th
// largest key, and its rank r1 inside that bin, come from adding those
// counts without reading a score.  Two kernels then cover each row in
// segments of SEL_ROUND * rounds keys, many workgroups per row:
//   count: each segment counts its keys above bin b* and, for the keys in
//          b*, a histogram of their low 8 bits, stored as suffix sums
//          cum[f] = #(keys in b* with low bits >= f), f = 0..256;
//   emit:  each segment adds every segment's suffix sums, which gives the
//          exact k-th key T = (b*, f*) and how many keys equal to T are
//          taken; the counts of the segments before it give its first
//          output rank, and it emits its keys above T and the first of
//          those equal to T in position order (ties to the lower index).
// No workgroup waits for another: the kernel boundary orders the two passes.
// ---------------------------------------------------------------------------
constexpr int SEL_NT = 256;                   // threads per segment workgroup
constexpr int SEL_KPT = 16;                   // keys per thread and round
constexpr int SEL_ROUND = SEL_NT * SEL_KPT;   // 4096 keys per round
constexpr int SEL_REC = 260;                  // words per (row, segment): keys above b*, cum[0..256], b*, rank

// Two exclusive prefix sums over the workgroup with one barrier (as
// BlockScan::exscan, pairs of wave totals in alternating LDS slots).
CSA_DEV void block_exscan2(uint32_t a, uint32_t b, uint32_t& a_before, uint32_t& b_before, uint32_t& a_total,
                           uint32_t& b_total, int& parity)
{
    __shared__ uint32_t part2[2][2][16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    if (lane == 63) {
        part2[parity][0][w] = ia;
        part2[parity][1][w] = ib;
    }
    __syncthreads();
    uint32_t oa = 0, ob = 0, ta = 0, tb = 0;
    for (int i = 0; i < nw; ++i) {
        const uint32_t xa = part2[parity][0][i], xb = part2[parity][1][i];
        ta += xa;
        tb += xb;
        oa += i < w ? xa : 0u;
        ob += i < w ? xb : 0u;
    }
    parity ^= 1;
    a_before = oa + ia - a;
    b_before = ob + ib - b;
    a_total = ta;
    b_total = tb;
}

// Wave 0: among 256 counts (cnt(b) for bin b), the bin holding the rem-th
// largest key counting from bin 255 down, and the rank of that key inside
// its bin.  Lane l holds bins 255-4l .. 252-4l.
template <class CountF>
CSA_DEV void wave_pick_bin(CountF cnt, uint32_t rem, uint32_t* out_bin, uint32_t* out_rem)
{
    const int lane = threadIdx.x & 63;
    uint32_t c4[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        c4[j] = cnt(255 - 4 * lane - j);
        tot += c4[j];
    }
    const uint32_t inc = wave_incl_scan(tot), exc = inc - tot;
    if (exc < rem && rem <= inc) {
        uint32_t above = exc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (rem <= above + c4[j]) {
                *out_bin = (uint32_t)(255 - 4 * lane - j);
                *out_rem = rem - above;
                break;
            }
            above += c4[j];
        }
    }
}

// Order-preserving keys of two bf16 scores in one word (low half first),
// the sign-magnitude flip of key16 on both halves at once.  The indexer
// stores no -0, so no zero fix-up is needed.
CSA_DEV uint32_t key16x2(uint32_t w)
{
    return w ^ 0x80008000u ^ (((w >> 15) & 0x00010001u) * 0x7FFFu);
}

// The 16 keys of thread t in the round starting at position p0 (positions
// p0 + 16 t .. p0 + 16 t + 15) as two 16-byte vectors of packed bf16 pairs;
// vectors past the row are clamped to its last one (masked by position).
CSA_DEV void sel_load(const uint16_t* sr, int nvec_row, int p0, uint4 (&q)[2])
{
    const int v0 = (p0 + (int)threadIdx.x * SEL_KPT) / 8;
    q[0] = ld16(sr + 8 * (size_t)min(v0, nvec_row - 1));
    q[1] = ld16(sr + 8 * (size_t)min(v0 + 1, nvec_row - 1));
}

// Coarse digit of the k-th largest key of a row from the per-chunk counts
// (all 256 threads): bin b* into pick[0], the rank of the k-th key inside it
// into pick[1].  Thread t adds bins 8 (t mod 32) .. +7 of chunks t/32,
// t/32 + 8, .. (16-byte loads, four chunks in flight), the 8 chunk groups
// meet in LDS.
CSA_DEV void coarse_pick(const uint16_t* hr, int nch, uint32_t k, uint32_t (&part)[8][256], uint32_t (&tot)[256],
                         uint32_t* pick)
{
    const int tid = threadIdx.x, sub = tid & 31, cgrp = tid >> 5;
    uint32_t acc[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    for (int c0 = cgrp; c0 < nch; c0 += 4 * 8) {
        uint4 h[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + 8 * u;
            h[u] = c < nch ? ld16(hr + (size_t)c * 256 + 8 * sub) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t w4[4] = {h[u].x, h[u].y, h[u].z, h[u].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += (w4[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        }
    }
    *(uint4*)&part[cgrp][8 * sub] = make_uint4(acc[0], acc[1], acc[2], acc[3]);
    *(uint4*)&part[cgrp][8 * sub + 4] = make_uint4(acc[4], acc[5], acc[6], acc[7]);
    if (tid == 0) {                                          // defined even if no bin qualifies
        pick[0] = 0u;
        pick[1] = 1u;
    }
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int g2 = 0; g2 < 8; ++g2) t += part[g2][tid];
    tot[tid] = t;
    __syncthreads();
    if (tid < 64) wave_pick_bin([&](int b) { return tot[b]; }, k, &pick[0], &pick[1]);
    __syncthreads();
    if (tid == 0) pick[0] = min(pick[0], 255u);
    __syncthreads();
}

__global__ __launch_bounds__(SEL_NT) void topk_seg_count_kernel(const uint16_t* scores, int ld,
                                                                const int32_t* n_valid, const uint16_t* hist,
                                                                int hist_chunks, int chunk, int k, int rounds,
                                                                int seg_stride, uint32_t* rec)
{
    const int row = blockIdx.y, sgi = blockIdx.x, tid = threadIdx.x;
    const int V = min(n_valid[row], ld);
    const int s0 = sgi * rounds * SEL_ROUND;
    if (V <= k || s0 >= V) return;                           // uniform: nothing of this segment is needed
    __shared__ uint32_t part[8][256];
    __shared__ uint32_t tot[256];
    __shared__ uint32_t fine[256];
    __shared__ uint32_t pick[2];
    const uint16_t* sr = scores + (size_t)row * ld;
    const int nvec_row = ld / 8;
    uint4 q[2];
    sel_load(sr, nvec_row, s0, q);                           // in flight during the coarse sums
    fine[tid] = 0u;
    coarse_pick(hist + (size_t)row * hist_chunks * 256, (V + chunk - 1) / chunk, (uint32_t)k, part, tot, pick);
    const uint32_t bstar = pick[0];
    uint32_t gt = 0;
    for (int rnd = 0; rnd < rounds; ++rnd) {
        const int p0 = s0 + rnd * SEL_ROUND;
        if (p0 >= V) break;                                  // uniform
        if (rnd > 0) sel_load(sr, nvec_row, p0, q);
        const int base = p0 + tid * SEL_KPT;
        const uint32_t w8[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const uint32_t kp = key16x2(w8[h]);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t kv = (kp >> (16 * half)) & 0xFFFFu;
                const bool in = base + 2 * h + half < V;
                gt += in && (kv >> 8) > bstar;
                if (in && (kv >> 8) == bstar) atomicAdd(&fine[kv & 0xFFu], 1u);
            }
        }
    }
    __syncthreads();
    // suffix sums of the fine counts (thread t holds bin 255 - t: an
    // inclusive scan in thread order) and the segment's keys above b*
    BlockScan bs;
    uint32_t gt_tot;
    const uint32_t gt_before = bs.exscan(gt, &gt_tot);
    (void)gt_before;
    uint32_t fin_tot;
    const uint32_t f = fine[255 - tid];
    const uint32_t suffix = bs.exscan(f, &fin_tot) + f;     // cum[255 - t]
    uint32_t* r = rec + ((size_t)row * seg_stride + sgi) * SEL_REC;
    r[1 + (255 - tid)] = suffix;
    if (tid == 0) {
        r[0] = gt_tot;
        r[1 + 256] = 0u;
        r[258] = bstar;                                      // the row's coarse digit and the rank in it
        r[259] = pick[1];                                    // (the same in every segment's record)
    }
}

__global__ __launch_bounds__(SEL_NT) void topk_seg_emit_kernel(const uint16_t* scores, int ld, const int32_t* n_valid,
                                                               int k, int rounds, int seg_stride,
                                                               const uint32_t* rec, int32_t* out)
{
    const int row = blockIdx.y, sgi = blockIdx.x, tid = threadIdx.x;
    const int V = min(n_valid[row], ld);
    int32_t* o = out + (size_t)row * k;
    if (V <= k) {                                            // every visible entry, then -1
        if (sgi == 0)
            for (int r = tid; r < k; r += SEL_NT) o[r] = r < V ? r : -1;
        return;
    }
    const int seg = rounds * SEL_ROUND;
    const int s0 = sgi * seg;
    if (s0 >= V) return;
    const int nseg = (V + seg - 1) / seg;
    __shared__ uint32_t ctot[257];
    __shared__ uint32_t cpre[257];
    __shared__ uint32_t gsum[SEL_NT / 64];
    __shared__ uint32_t pick[2];
    const uint16_t* sr = scores + (size_t)row * ld;
    const int nvec_row = ld / 8;
    uint4 q[2];
    sel_load(sr, nvec_row, s0, q);
    // the coarse digit and the rank in it, from the count kernel's records;
    // suffix sums over every segment of the row and over the segments before
    // this one: thread t adds cum[t] of segments 0, 1, .. (sixteen loads in
    // flight), and the keys above b* of the segments before this one are
    // added up at the same time, so nothing waits for the fine digit below
    const uint32_t* rr = rec + (size_t)row * seg_stride * SEL_REC;
    const uint32_t bstar = min(rr[258], 255u), r1 = rr[259];
    {
        uint32_t g0 = 0;
        for (int i = tid; i < sgi; i += SEL_NT) g0 += rr[(size_t)i * SEL_REC];
        uint32_t c = 0, cp = 0;
        for (int i0 = 0; i0 < nseg; i0 += 16) {
            uint32_t v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = i0 + u < nseg ? rr[(size_t)(i0 + u) * SEL_REC + 1 + tid] : 0u;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                c += v[u];
                cp += i0 + u < sgi ? v[u] : 0u;
            }
        }
        ctot[tid] = c;
        cpre[tid] = cp;
        if (tid == 0) {
            ctot[256] = 0u;
            cpre[256] = 0u;
        }
        g0 = wave_incl_scan(g0);
        if ((tid & 63) == 63) gsum[tid >> 6] = g0;
    }
    if (tid == 0) {                                          // defined even if no bin qualifies
        pick[0] = 0u;
        pick[1] = 0u;
    }
    __syncthreads();
    // the low 8 bits f* of the k-th key: the largest f with ctot[f] >= r1
    if (ctot[tid] >= r1 && ctot[tid + 1] < r1) {
        pick[0] = (uint32_t)tid;
        pick[1] = r1 - ctot[tid + 1];                        // keys equal to T taken
    }
    __syncthreads();
    const uint32_t fstar = min(pick[0], 255u), rem = pick[1];   // fstar indexes cum[0..256]
    const uint32_t T = (bstar << 8) | fstar;
    // outputs of the segments before this one: their keys above T (those
    // above b*, and those of bin b* above f*) and their keys equal to T
    uint32_t gt_before = cpre[fstar + 1];
#pragma unroll
    for (int w = 0; w < SEL_NT / 64; ++w) gt_before += gsum[w];
    const uint32_t eq_before = cpre[fstar] - cpre[fstar + 1];
    int parity = 0;
    uint32_t out_base = gt_before + min(eq_before, rem);
    uint32_t rem_left = rem - min(eq_before, rem);
    for (int rnd = 0; rnd < rounds; ++rnd) {
        const int p0 = s0 + rnd * SEL_ROUND;
        if (p0 >= V) break;                                  // uniform
        if (rnd > 0) sel_load(sr, nvec_row, p0, q);
        const int base = p0 + tid * SEL_KPT;
        const uint32_t w8[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
        uint32_t kp[8];
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            kp[h] = key16x2(w8[h]);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t kv = (kp[h] >> (16 * half)) & 0xFFFFu;
                const bool in = base + 2 * h + half < V;
                gt += in && kv > T;
                eq += in && kv == T;
            }
        }
        uint32_t gtb, eqb, gtt, eqt;
        block_exscan2(gt, eq, gtb, eqb, gtt, eqt, parity);
        int oi = (int)(out_base + gtb + min(eqb, rem_left));
        int take_eq = (int)min(eq, rem_left > eqb ? rem_left - eqb : 0u);
#pragma unroll
        for (int h = 0; h < 8; ++h) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int pos = base + 2 * h + half;
                const uint32_t kv = (kp[h] >> (16 * half)) & 0xFFFFu;
                if (pos < V && (kv > T || (kv == T && take_eq > 0)) && (unsigned)oi < (unsigned)k) {   // ranks below k
                    take_eq -= kv == T;
                    o[oi++] = pos;
                }
            }
        }
        out_base += gtt + min(eqt, rem_left);
        rem_left -= min(eqt, rem_left);
    }
}

// Coarse counts of one segment of a row whose scores were stored without
// them: the 256 bins of the keys' top 8 bits, in the layout of the index
// launches' per-chunk counts (the segment is the chunk).  Each lane counts
// into its own copy of a bin (32 copies, lane mod 32), so the lanes of a
// wave, whose keys mostly fall into a few bins, do not queue on one LDS
// address; the copies are added at the end.
__global__ __launch_bounds__(SEL_NT) void topk_seg_hist_kernel(const uint16_t* scores, int ld, const int32_t* n_valid,
                                                               int rounds, int nseg, uint16_t* hist)
{
    __shared__ uint32_t hc[256 * 32];
    const int row = blockIdx.y, sgi = blockIdx.x, tid = threadIdx.x;
    for (int i = tid; i < 256 * 32; i += SEL_NT) hc[i] = 0u;
    const int V = min(n_valid[row], ld);
    const int s0 = sgi * rounds * SEL_ROUND;
    const uint16_t* sr = scores + (size_t)row * ld;
    const int nvec_row = ld / 8;
    const uint32_t cp = tid & 31;
    __syncthreads();
    if (s0 < V) {                                            // uniform
        uint4 q[2];
        sel_load(sr, nvec_row, s0, q);
        for (int rnd = 0; rnd < rounds; ++rnd) {
            const int p0 = s0 + rnd * SEL_ROUND;
            if (p0 >= V) break;                              // uniform
            uint4 qn[2];                                     // the next round's keys load meanwhile
            if (rnd + 1 < rounds && p0 + SEL_ROUND < V) sel_load(sr, nvec_row, p0 + SEL_ROUND, qn);
            const int base = p0 + tid * SEL_KPT;
            const uint32_t w8[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                const uint32_t kp = key16x2(w8[h]);
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t kv = (kp >> (16 * half)) & 0xFFFFu;
                    if (base + 2 * h + half < V) atomicAdd(&hc[(kv >> 8) * 32 + cp], 1u);
                }
            }
            q[0] = qn[0];
            q[1] = qn[1];
        }
    }
    __syncthreads();
    // thread t adds the 32 copies of bin t (rotated start: fewer bank conflicts)
    uint32_t c = 0;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) c += hc[tid * 32 + ((j + tid) & 31)];
    hist[((size_t)row * nseg + sgi) * 256 + tid] = (uint16_t)c;
}

// Rounds of SEL_ROUND keys per segment: doubled while a launch would have
// more than 4096 segment workgroups, at most 8 (decode rows: one round).
static int sel_rounds(int n_rows, int ld)
{
    const long keys = (long)n_rows * ld;
    int r = 1;
    while (r < 8 && keys / ((long)SEL_ROUND * r) > 4096) r *= 2;
    return r;
}

size_t topk_hist_workspace(int n_rows, int ld)
{
    const int seg = sel_rounds(n_rows, ld) * SEL_ROUND;
    return (size_t)n_rows * ((ld + seg - 1) / seg) * SEL_REC * 4;
}

// The per-segment coarse counts of rows stored without them, in the segments
// launch_topk_hist will use (*chunk: the segment length).
hipError_t launch_seg_hist(hipStream_t st, int n_rows, const void* scores, int ld, const int32_t* n_valid,
                           uint16_t* hist, int* chunk)
{
    const int rounds = sel_rounds(n_rows, ld);
    const int seg = rounds * SEL_ROUND;
    *chunk = seg;
    if (n_rows <= 0) return hipSuccess;
    const int nseg = (ld + seg - 1) / seg;
    topk_seg_hist_kernel<<<dim3(nseg, n_rows), SEL_NT, 0, st>>>((const uint16_t*)scores, ld, n_valid, rounds, nseg,
                                                                hist);
    return hipGetLastError();
}

hipError_t launch_topk_hist(hipStream_t st, int n_rows, const void* scores, int ld, const int32_t* n_valid,
                            const uint16_t* hist, int hist_chunks, int chunk, int k, int32_t* out, void* ws)
{
    if (n_rows <= 0) return hipSuccess;
    const int rounds = sel_rounds(n_rows, ld);
    const int seg = rounds * SEL_ROUND;
    const int nseg = (ld + seg - 1) / seg;
    const dim3 grid(nseg, n_rows);
    uint32_t* rec = (uint32_t*)ws;
    topk_seg_count_kernel<<<grid, SEL_NT, 0, st>>>((const uint16_t*)scores, ld, n_valid, hist, hist_chunks, chunk, k,
                                                   rounds, nseg, rec);
    topk_seg_emit_kernel<<<grid, SEL_NT, 0, st>>>((const uint16_t*)scores, ld, n_valid, k, rounds, nseg, rec, out);
    return hipGetLastError();
}

// Chunk length per first-stage workgroup.  A row that fits one workgroup is
// one chunk (one stage, no candidates).  Longer rows split into chunks of at
// most the capacity; when there are few rows the chunks shrink so that more
// workgroups share the work, as long as the candidates still fit one
// second-stage workgroup: bf16 rows into equal chunks of at most 16384 keys
// (the merge of up to 16384 candidates then also runs 16 keys per thread;
// 4 rows of 262144: 25.8 us, against 29.7 us with 26 chunks of 10240),
// others by halving down to 4k keys.
static int chunk_for(int n_rows, int max_cols, int k, bool bf16)
{
    const int cap = bf16 ? CAP16 : CAP32;
    if (max_cols <= cap) return max_cols > 0 ? max_cols : 1;
    auto nch = [&](int c) { return (max_cols + c - 1) / c; };
    if (bf16 && (long)n_rows * nch(cap) < 256) {
        // few long bf16 rows: equal chunks of at most 16384 keys (1024
        // threads, 16 keys each), a multiple of 64 keys long
        const int n = nch(TOPK_THREADS * MID_KPT);
        const int c = ((max_cols + n - 1) / n + 63) / 64 * 64;
        if (c >= 4 * k && (long)nch(c) * k <= cap) return c;
    }
    int chunk = cap;
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

template <bool BF16>
static void launch_chunks(hipStream_t st, dim3 grid, int chunk, const void* scores, int ld, const int32_t* n_valid,
                          int k, int n_chunks, int32_t* out, uint32_t* ck, int32_t* ci)
{
    if (chunk <= SMALL_NT * SMALL_KPT)
        topk_chunk_kernel<BF16, SMALL_NT, SMALL_KPT><<<grid, SMALL_NT, 0, st>>>(scores, ld, n_valid, k, chunk,
                                                                                n_chunks, out, ck, ci);
    else if (BF16 && chunk <= TOPK_THREADS * MID_KPT)        // faster than 256 threads x 40 keys here
        topk_chunk_kernel<BF16, TOPK_THREADS, BF16 ? MID_KPT : KPT32><<<grid, TOPK_THREADS, 0, st>>>(
            scores, ld, n_valid, k, chunk, n_chunks, out, ck, ci);
    else
        topk_chunk_kernel<BF16, TOPK_THREADS, BF16 ? KPT16 : KPT32><<<grid, TOPK_THREADS, 0, st>>>(
            scores, ld, n_valid, k, chunk, n_chunks, out, ck, ci);
}

hipError_t launch_topk(hipStream_t st, int score_bf16, int n_rows, const void* scores, int ld,
                       const int32_t* n_valid, int k, int32_t* out, void* ws, int max_cols)
{
    if (n_rows <= 0) return hipSuccess;
    const bool bf = score_bf16 != 0;
    const int chunk = chunk_for(n_rows, max_cols, k, bf);
    const int n_chunks = max(1, (max_cols + chunk - 1) / chunk);
    uint32_t* ck = (uint32_t*)ws;
    int32_t* ci = n_chunks > 1 ? (int32_t*)((char*)ws + (size_t)n_rows * n_chunks * k * 4) : nullptr;
    dim3 g1(n_chunks, n_rows);
    if (bf) launch_chunks<true>(st, g1, chunk, scores, ld, n_valid, k, n_chunks, out, ck, ci);
    else launch_chunks<false>(st, g1, chunk, scores, ld, n_valid, k, n_chunks, out, ck, ci);
    if (n_chunks > 1) {
        if (bf && (long)n_chunks * k <= TOPK_THREADS * MID_KPT)   // few candidates: 16 per thread
            topk_merge_kernel<true, MID_KPT><<<n_rows, TOPK_THREADS, 0, st>>>(n_valid, ld, k, n_chunks, ck, ci, out);
        else if (bf && (long)n_chunks * k <= TOPK_THREADS * 24)   // e.g. 17 chunks of 1024 (rows just past 2^18)
            topk_merge_kernel<true, 24><<<n_rows, TOPK_THREADS, 0, st>>>(n_valid, ld, k, n_chunks, ck, ci, out);
        else if (bf) topk_merge_kernel<true><<<n_rows, TOPK_THREADS, 0, st>>>(n_valid, ld, k, n_chunks, ck, ci, out);
        else topk_merge_kernel<false><<<n_rows, TOPK_THREADS, 0, st>>>(n_valid, ld, k, n_chunks, ck, ci, out);
    }
    return hipGetLastError();
}

}  // namespace csa
