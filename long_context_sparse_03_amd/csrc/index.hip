// a3: Lightning Indexer scores on gfx950.
//
// I[t][s] = sum_h w[t][h] * ReLU(q[t][h] . K[s]) over the visible entries
// s < floor((t+1)/m) ("DeepSeek-V4 内部机制" §1.2 Step 2; yunpan.plus eq. (8)),
// rounded to the score format (BF16 scores: "DeepSeek-V4 内部机制" §6.2).
//
// The contraction is an MFMA product with the indexer heads as the M
// dimension and 16 keys as N: lane l of a wave holds head (key) l%16; in the
// decode kernel, step s of the contraction covers 64 bytes of the key and
// lane group l/16 the 16 bytes at 16*(l/16) of them, so the four lanes of a
// key read 64 contiguous bytes per load.  ReLU, the head weights and the head sum
// are applied to the accumulators in registers; the sum over the four lane
// groups is a fixed butterfly, so the result is deterministic.
//
// MXFP4 keys and the MXFP4-quantised query go straight into gfx950's scaled
// FP4 MFMA (16x16x128 with E8M0 block scales): one instruction covers a
// 128-wide key, and the products of E2M1 values and power-of-two scales are
// exact, so only the fp32 accumulation order differs from the definition.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// ReLU as one clamp to [0, FLT_MAX]: the same value as max(x, 0) for every
// finite x, without the canonicalising copy an IEEE-mode max of an MFMA
// result costs
CSA_DEV float relu_clamp(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.40282347e38f); }

// Load EPF elements of a row (f32 or bf16 storage) as one 16-byte fragment of
// the MMA element type (T_MMA_BF16 = bf16 fragments).
template <bool MMA_BF16>
CSA_DEV void load_frags(const void* base, bool src_bf16, int n_frag, int q_elems, uint4* out)
{
    // n_frag fragments covering q_elems consecutive elements
    if (MMA_BF16) {
        if (src_bf16) {
            const uint4* p = (const uint4*)base;
            for (int f = 0; f < n_frag; ++f) out[f] = p[f];
        } else {
            const float4* p = (const float4*)base;
            for (int f = 0; f < n_frag; ++f) {
                float4 a = p[2 * f], b = p[2 * f + 1];
                out[f] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                                    pack_bf16x2(b.z, b.w));
            }
        }
    } else {
        const uint4* p = (const uint4*)base;       // f32 storage, 4 per fragment
        for (int f = 0; f < n_frag; ++f) out[f] = p[f];
    }
}

// Quantise the 32 bf16 values of four fragments (one MX block) to E2M1 codes
// (element 2i in the low nibble of byte i) and return the E8M0 scale code.
CSA_DEV int mx_quant_codes(const uint4 (&f)[4], uint4& codes)
{
    float v[32];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t w4[4] = {f[s].x, f[s].y, f[s].z, f[s].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[8 * s + 2 * h] = bf16_to_f32(w4[h] & 0xFFFF);
            v[8 * s + 2 * h + 1] = bf16_to_f32(w4[h] >> 16);
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const int sc = mx_scale_code(amax);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) w[j / 8] |= f32_to_e2m1(ldexpf(v[j], 127 - sc)) << (4 * (j % 8));
    codes = make_uint4(w[0], w[1], w[2], w[3]);
    return sc;
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// One scaled FP4 MFMA (16x16x128, E2M1 operands with E8M0 block scales): the
// lane's 16 bytes hold its row's (column's) 32-element block l/16, and its
// scale applies to those 32 elements.
CSA_DEV f32x4_t mfma_fp4(uint4 a, int sa, uint4 b, int sb)
{
    const i32x8_t av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero4(), 4, 4, 0, sa, 0, sb);
}

// Decode-shaped launch: one workgroup per (query, EPW entries).  Each wave
// scores 64 entries per iteration as four 16-key tiles and keeps the next
// iteration's key loads in flight while it computes the current one.
// HT = head tiles (<= 4), S = fragments per lane group.
constexpr int IDX_EPW = 2048;                 // entries per workgroup (MXFP4 kernel; 1024: 5 % slower at 1M)
constexpr int IDXD_EPW = 1024;                // entries per workgroup (fp32 / bf16 kernel)
constexpr int IDXD_TPI = 4;                   // 16-key tiles per wave and iteration (fp32 / bf16 kernel)
constexpr int IDXD_ITERS = IDXD_EPW / (64 * IDXD_TPI);   // iterations of 64 * TPI entries
constexpr int IDX_ITERS = IDX_EPW / 256;      // the same for the MXFP4 kernel

template <int IDXF, int S, int TPI>
CSA_DEV void load_keys(const IndexArgs& a, const int* bt, int blk0, int e0, int V, int g, int li, uint4 (&B)[TPI][S])
{
    // Loads are unconditional (entries past V are clamped to V-1): an MFMA
    // column only feeds the score of its own entry, and scores of entries
    // >= V are not stored.  Branch-free loads stay in flight together.
    const int cI = a.cI, quarter = cI / 4;
    const size_t kbytes = IDXF == 0 ? (size_t)cI * 4 : (size_t)cI * 2;
#pragma unroll
    for (int tile = 0; tile < TPI; ++tile) {
        const int e = min(e0 + 16 * tile + li, V - 1);
        const int phys = bt[(e >> a.epb_log2) - blk0];
        const int slot = (e & (a.epb - 1));
        const char* kb = (const char*)a.keys + (size_t)phys * a.key_block_bytes;
        // step s covers 64 bytes of the key, lane group g the 16 bytes at 16g
        // of them: the four lanes of a key read 64 contiguous bytes
        const char* kp = kb + (size_t)slot * kbytes + (size_t)g * 16;
#pragma unroll
        for (int s = 0; s < S; ++s) B[tile][s] = ld16(kp + 64 * s);
    }
}

// bf16 bits with -0 (a tiny negative score that rounds to zero) made +0, as
// the scores are stored and counted
CSA_DEV uint16_t canon_bf16(uint16_t b) { return (b & 0x7FFFu) == 0u ? (uint16_t)0u : b; }

// Fused top-k counts: lanes 4j .. 4j+3 (a quad) hold four consecutive keys,
// which mostly fall into one bin, so the first lane of a quad with a given
// bin adds the quad's count of it; bin ~0 counts nothing.  Every lane of the
// wave calls it (the quad permutes read the other lanes' bins).
CSA_DEV void count_bins_quad(uint32_t* h, uint32_t b)
{
    const int qd = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 3;
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)b, 0xB1, 0xF, 0xF, false);   // lane ^ 1
    const uint32_t b2 = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)b, 0x4E, 0xF, 0xF, false);   // lane ^ 2
    const uint32_t b3 = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)b, 0x1B, 0xF, 0xF, false);   // lane ^ 3
    const bool m1 = b1 == b, m2 = b2 == b, m3 = b3 == b;
    const bool later = (qd == 1 && m1) || (qd == 2 && (m2 || m3)) || (qd == 3 && (m1 || m2 || m3));
    if (b != ~0u && !later) atomicAdd(&h[b], 1u + m1 + m2 + m3);
}

// Fused top-k: the chunk's 256 counts of query row gq (threads 0..255, one
// coalesced 512-byte store), after every wave has counted its scores.  Every
// wave of the workgroup must call it (it holds a barrier when HIST).
template <bool HIST>
CSA_DEV void store_hist(const IndexArgs& a, int gq, int chunk, const uint32_t* hcnt)
{
    if (!HIST) return;
    __syncthreads();
    if (threadIdx.x < 256)
        a.hist[((size_t)gq * a.hist_chunks + chunk) * 256 + threadIdx.x] = (uint16_t)hcnt[threadIdx.x];
}

template <int IDXF, int HT, int S, bool HIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(S <= 4 ? 2 : 1))) void index_decode_kernel(IndexArgs a)
{
    // IDXF 0: fp32 keys and queries; 1: bf16 keys and queries.
    using MMA = typename std::conditional<IDXF == 0, MmaF32, MmaBF16>::type;
    __shared__ int bt[IDXD_EPW + 1];             // physical blocks of this workgroup's entries
    // the query's MFMA fragments, shared by the four waves (in LDS rather than
    // registers, so that two workgroups fit on a compute unit and twice the
    // key bytes are in flight)
    __shared__ uint4 qfrag[HT][S][64];
    __shared__ uint32_t hcnt[256];               // fused top-k: this chunk's scores by key16 >> 8
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    // query fastest in the dispatch order: every query's near-empty last
    // key chunk comes after all full chunks, not among them
    const int gq = blockIdx.x;
    hcnt[threadIdx.x] = 0u;                      // 256 threads, published by the prologue's barrier
    const int wg0 = blockIdx.y * IDXD_EPW;
    const int cI = a.cI, nh = a.nh;
    constexpr int QES = IDXF == 0 ? 4 : 2;      // query element size
    __shared__ int cu_sh[1025];
    int req, tok;
    if (a.one_per_req) {                         // token gq is request gq's only new token
        req = gq;
        tok = 0;
    } else {
        req = find_request_block(a.cu_new, a.n_req, gq, cu_sh);
        tok = gq - (a.n_req < 1024 ? cu_sh[req] : a.cu_new[req]);   // cu_sh is filled only below 1024
    }

    // ---- prologue: position, block-table slice, query fragments and head
    //      weights, all loads issued together (the slice covers every block
    //      the workgroup can touch, clamped to the table row; indices
    //      clamped, values masked afterwards)
    const int blk0 = wg0 >> a.epb_log2;
    const int nbw = ((wg0 + IDXD_EPW - 1) >> a.epb_log2) - blk0 + 1;
    const int sp = a.start_pos[req];
    int btv[(IDXD_EPW + 255) / 256];
#pragma unroll
    for (int i = 0; i < (IDXD_EPW + 255) / 256; ++i) {
        const int j = min(blk0 + min((int)threadIdx.x + 256 * i, nbw - 1), a.max_blocks - 1);
        btv[i] = a.block_table[(size_t)req * a.max_blocks + j];
    }
    // wave ht (< HT) stages head tile ht of the query
    uint4 A[S];
    if (wave < HT) {
        const int head = min(16 * wave + li, nh - 1);
        const char* qp = (const char*)a.q + ((size_t)gq * nh + head) * cI * QES + (size_t)g * 16;
#pragma unroll
        for (int s = 0; s < S; ++s) A[s] = ld16(qp + 64 * s);
    }
    float wv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = a.w[(size_t)gq * nh + min(16 * ht + 4 * g + i, nh - 1)];
    const int t = sp + tok;
    const int V = (t + 1) / a.m;
    if (blockIdx.y == 0 && threadIdx.x == 0) a.n_valid[gq] = V;
    if (wg0 >= V) return;                        // workgroup-uniform
#pragma unroll
    for (int i = 0; i < (IDXD_EPW + 255) / 256; ++i)
        if ((int)threadIdx.x + 256 * i < nbw) bt[threadIdx.x + 256 * i] = btv[i];
    if (wave < HT) {
        const bool hv = 16 * wave + li < nh;
#pragma unroll
        for (int s = 0; s < S; ++s) qfrag[wave][s][lane] = sel16(hv, A[s]);
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = 16 * ht + 4 * g + i < nh ? wv[ht][i] : 0.f;
    __syncthreads();

    // ---- main loop: 256 entries per iteration (64 per wave); the next
    //      iterations' key loads are issued before this one's arithmetic
    constexpr int NB = 2;                       // key buffers (NB-1 iterations in flight)
    constexpr int TPI = IDXD_TPI, EPI = 64 * TPI;           // tiles per wave, entries per iteration
    uint4 B[NB][TPI][S];
    // The loads are unconditional (clamped to the last visible entry): loads
    // under a branch would make the wait counts below pessimistic.
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) {
        if (j < IDXD_ITERS) load_keys<IDXF, S, TPI>(a, bt, blk0, wg0 + EPI * j + wave * 16 * TPI, V, g, li, B[j]);
        __builtin_amdgcn_sched_barrier(0);            // keep the loads in iteration order
    }
#pragma unroll
    for (int it = 0; it < IDXD_ITERS; ++it) {
        const int cur = it % NB;
        const int e_base = wg0 + it * EPI + wave * 16 * TPI;
        if (it + NB - 1 < IDXD_ITERS)
            load_keys<IDXF, S, TPI>(a, bt, blk0, e_base + EPI * (NB - 1), V, g, li, B[(it + NB - 1) % NB]);
        __builtin_amdgcn_sched_barrier(0);
        if (e_base >= V) break;                  // wave-uniform
        // head tiles outermost: each query fragment is read from LDS once
        // per iteration and serves the four key tiles; every tile's score
        // still sums the head tiles in order
        float v[TPI];
#pragma unroll
        for (int tile = 0; tile < TPI; ++tile) v[tile] = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            uint4 qf[S];
#pragma unroll
            for (int s = 0; s < S; ++s) qf[s] = qfrag[ht][s][lane];
#pragma unroll
            for (int tile = 0; tile < TPI; ++tile) {
                f32x4_t acc = zero4();
#pragma unroll
                for (int s = 0; s < S; ++s) acc = MMA::step(qf[s], B[cur][tile][s], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) v[tile] += wv[ht][i] * relu_clamp(acc[i]);
            }
        }
        // sum over the four lane groups, transposed: after the exchange with
        // group g^1 a lane keeps two tiles, after the one with g^2 one tile,
        // (v_g + v_g^1) + (v_g^2 + v_g^3) in every case; lane (g, li) ends
        // with the entry of tile 2 (g & 1) + (g >> 1), so one store per lane
        static_assert(TPI == 4, "four tiles meet four lane groups");
        const bool o1 = g & 1, o2 = g & 2;
        float k0 = o1 ? v[2] : v[0], k1 = o1 ? v[3] : v[1];
        k0 += __shfl_xor(o1 ? v[0] : v[2], 16, 64);
        k1 += __shfl_xor(o1 ? v[1] : v[3], 16, 64);
        float x = o2 ? k1 : k0;
        x += __shfl_xor(o2 ? k0 : k1, 32, 64);
        const int e = e_base + 16 * (2 * (g & 1) + (g >> 1)) + li;
        uint32_t hbin = ~0u;
        if (e < V) {
            if (x == 0.0f) x = 0.0f;                    // -0 is stored as +0
            if (a.score_bf16) {
                const uint16_t b = canon_bf16(f32_to_bf16(x));   // a value rounding to -0 is stored as +0
                ((uint16_t*)a.scores)[(size_t)gq * a.ld + e] = b;
                hbin = key16(b) >> 8;
            } else {
                ((float*)a.scores)[(size_t)gq * a.ld + e] = x;
            }
        }
        if (HIST) count_bins_quad(hcnt, hbin);
    }
    store_hist<HIST>(a, gq, blockIdx.y, hcnt);
}

// Prefill-shaped launch (bf16 keys, 128 channels): eight queries of one
// request per workgroup, one per wave, share every 128-key tile staged in
// LDS, so a key is read from memory once per eight queries.  Tiles are
// double-buffered and go from memory straight into LDS (no register
// staging): the next tile's loads are in flight while the current one is
// multiplied.  A tile row is the key's 16 chunks of 16 bytes, chunk c at
// slot c ^ (row mod 16), so the 16 lanes that read one chunk of 16
// consecutive keys hit 16 different slots (all 64 banks).
constexpr int PF_QPW = 8;                     // queries (waves) per workgroup
constexpr int PF_TILE = 128;                  // keys per LDS tile
constexpr int PF_ECH = 8192;                  // keys per workgroup
constexpr int PF_CI = 128;                    // key channels (16 chunks of 16 bytes)

template <int HT, int S, bool BF16OUT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void index_prefill_kernel(IndexArgs a, int groups_per_req)
{
    static_assert(S * 8 * 4 == PF_CI, "S steps of eight channels in each of four lane groups cover a key");
    static_assert(PF_TILE == 8 * 4 * 4, "each wave brings four 1 KB pieces (four rows each) of a tile");
    // two tile buffers as separate objects, so that reads of one need not
    // wait for the loads in flight into the other
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[PF_TILE * PF_CI];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[PF_TILE * PF_CI];
    __shared__ int bt[PF_ECH / 32 + 2];
    __shared__ int cu_sh[1025];
    const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int req = blockIdx.y / groups_per_req, grp = blockIdx.y % groups_per_req;
    if (a.n_req >= 1024) return;                                    // host dispatch keeps n_req small here
    for (int i = threadIdx.x; i <= a.n_req; i += blockDim.x) cu_sh[i] = a.cu_new[i];
    __syncthreads();
    const int cu = cu_sh[req], n_tok = cu_sh[req + 1] - cu;
    if (PF_QPW * grp >= n_tok) return;                             // whole workgroup
    const int s0 = a.start_pos[req];
    const int qi = min(PF_QPW * grp + wave, n_tok - 1);              // clamped: extra waves help with loads only
    const bool qvalid = PF_QPW * grp + wave < n_tok;
    const int gq = cu + qi;
    const int V = (s0 + qi + 1) / a.m;
    const int Vmax = (s0 + min(PF_QPW * grp + PF_QPW, n_tok)) / a.m;  // of the workgroup's last query
    if (blockIdx.x == 0 && lane == 0 && qvalid) a.n_valid[gq] = V;
    const int e0 = blockIdx.x * PF_ECH;
    if (e0 >= Vmax) return;                                         // whole workgroup
    const int e1 = min(Vmax, e0 + PF_ECH);
    const int nh = a.nh;

    const int blk0 = e0 >> a.epb_log2;
    const int nblk = ((e1 - 1) >> a.epb_log2) - blk0 + 1;
    for (int j = threadIdx.x; j < nblk; j += blockDim.x) bt[j] = a.block_table[(size_t)req * a.max_blocks + blk0 + j];

    // query fragments and head weights of this wave's query
    uint4 A[HT][S];
    float wv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int head = min(16 * ht + li, nh - 1);
        // step s, lane group g: channels 32s + 8g .. +7, the decode kernel's
        // split of the channels into MFMA steps, so both kernels sum in the
        // same order and give identical scores
        const char* qp = (const char*)a.q + ((size_t)gq * nh + head) * PF_CI * 2 + (size_t)g * 16;
#pragma unroll
        for (int s = 0; s < S; ++s) A[ht][s] = ld16(qp + 64 * s);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = a.w[(size_t)gq * nh + min(16 * ht + 4 * g + i, nh - 1)];
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const bool hv = 16 * ht + li < nh;
#pragma unroll
        for (int s = 0; s < S; ++s) A[ht][s] = sel16(hv, A[ht][s]);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = 16 * ht + 4 * g + i < nh ? wv[ht][i] : 0.f;
    }
    __syncthreads();                                                // bt ready

    // one tile into a buffer: wave w fills bytes 1024 (4w + u) .. +1023 for
    // u < 4, i.e. rows 16w + 4u .. +3; lane l brings chunk (l mod 16) ^ (row
    // mod 16) of row 16w + 4u + l/16 (rows past the range repeat the last key)
    auto issue_tile = [&](int t0, uint16_t* buf) {
        // the lane's row and chunk are recomputed here rather than kept
        // across the loop (kept, they were spilled to scratch)
        int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 16 * wave + 4 * u + (ln >> 4);
            const int e = min(t0 + row, e1 - 1);
            const int c = (ln & 15) ^ (row & 15);
            const uint32_t in_blk = (uint32_t)(e & (a.epb - 1)) * (PF_CI * 2) + 16u * (uint32_t)c;
            const char* src = (const char*)a.keys + (size_t)bt[(e >> a.epb_log2) - blk0] * a.key_block_bytes + in_blk;
            __builtin_amdgcn_global_load_lds((const CSA_GLOBAL void*)src,
                                             (CSA_LDS void*)(buf + (16 * wave + 4 * u) * PF_CI), 16, 0, 0);
        }
    };
    // scores of the last tile, stored at the start of the next one (a
    // store issued right before the end-of-tile wait would hold it up)
    float xs[PF_TILE / 64];
    int es = -1;                                                    // first key of those scores (-1: none)
    auto store_scores = [&]() {
        if (es < 0) return;
        // the key offsets are recomputed (a spilled copy's reload would wait
        // for the next tile's loads, issued just before)
        int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int eb = 0; eb < PF_TILE / 64; ++eb) {
            const int e = es + eb * 64 + 16 * (2 * ((ln >> 4) & 1) + (ln >> 5)) + (ln & 15);
            if (e < V) {
                float x = xs[eb];
                if (x == 0.0f) x = 0.0f;                            // -0 is stored as +0
                if constexpr (BF16OUT) {
                    const uint16_t b = canon_bf16(f32_to_bf16(x));   // a value rounding to -0 is stored as +0
                    ((uint16_t*)a.scores)[(size_t)gq * a.ld + e] = b;
                } else {
                    ((float*)a.scores)[(size_t)gq * a.ld + e] = x;
                }
            }
        }
        es = -1;
    };
    auto compute = [&](int t0, const uint16_t* K) {
        if (!(qvalid && t0 < V)) return;
#pragma unroll
        for (int eb = 0; eb < PF_TILE / 64; ++eb) {                 // 64-key blocks
            // v[j]: this lane's partial score of key 64 eb + 16 j + li over
            // heads 4g .. 4g+3 of every head tile
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = eb * 64 + j * 16 + li;              // row mod 16 == li
                uint4 B[S];
#pragma unroll
                for (int s = 0; s < S; ++s) B[s] = *(const uint4*)&K[row * PF_CI + 8 * ((4 * s + g) ^ li)];
                f32x4_t acc[HT];
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc[ht] = zero4();
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) acc[ht] = MmaBF16::step(A[ht][s], B[s], acc[ht]);
                float vj = 0.f;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                    for (int i = 0; i < 4; ++i) vj += wv[ht][i] * relu_clamp(acc[ht][i]);
                v[j] = vj;
            }
            // sum over the four lane groups, transposed: after the exchange
            // with group g^1 a lane keeps two keys, after the one with g^2
            // one key, (v_g + v_g^1) + (v_g^2 + v_g^3) in every case
            const bool o1 = g & 1, o2 = g & 2;
            float k0 = o1 ? v[2] : v[0], k1 = o1 ? v[3] : v[1];
            k0 += __shfl_xor(o1 ? v[0] : v[2], 16, 64);
            k1 += __shfl_xor(o1 ? v[1] : v[3], 16, 64);
            float x = o2 ? k1 : k0;
            x += __shfl_xor(o2 ? k0 : k1, 32, 64);
            xs[eb] = x;
        }
        es = t0;
    };
    // every wave's loads of a tile have landed before the barrier after it
    auto tile_done = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);                         // vmcnt(0)
        __syncthreads();
    };

    const int n_tiles = (e1 - e0 + PF_TILE - 1) / PF_TILE;
    issue_tile(e0, Ks0);
    tile_done();
    for (int it = 0; it < n_tiles; it += 2) {
        const int t0 = e0 + it * PF_TILE;
        // Ks1 was last read in the previous pass, finished before its barrier
        if (it + 1 < n_tiles) issue_tile(t0 + PF_TILE, Ks1);
        store_scores();
        compute(t0, Ks0);
        tile_done();
        if (it + 1 >= n_tiles) break;
        if (it + 2 < n_tiles) issue_tile(t0 + 2 * PF_TILE, Ks0);
        store_scores();
        compute(t0 + PF_TILE, Ks1);
        tile_done();
    }
    store_scores();
}

// MXFP4 decode launch: as the bf16 decode kernel, with the stored key bytes
// fed straight into the scaled FP4 MFMA (one instruction per 16 keys and 16
// heads covers the whole 128-wide key).
template <int HT, bool HIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void index_decode_fp4_kernel(IndexArgs a)
{
    static_assert(HT <= 4, "one wave quantises each head tile");
    __shared__ int bt[IDX_EPW + 1];
    __shared__ int cu_sh[1025];
    __shared__ uint4 qc_sh[HT][64];              // quantised query: E2M1 codes ...
    __shared__ int qs_sh[HT][64];                // ... and E8M0 scales per (head tile, lane)
    __shared__ uint32_t hcnt[256];               // fused top-k: this chunk's scores by key16 >> 8
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int gq = blockIdx.x;                   // query fastest (as the bf16 kernel)
    hcnt[threadIdx.x] = 0u;                      // 256 threads, published by the barrier below
    const int wg0 = blockIdx.y * IDX_EPW;
    const int cI = a.cI, nh = a.nh;                // cI == 128: lane group g holds MX block g
    int req, tok;
    if (a.one_per_req) {                         // token gq is request gq's only new token
        req = gq;
        tok = 0;
    } else {
        req = find_request_block(a.cu_new, a.n_req, gq, cu_sh);
        tok = gq - (a.n_req < 1024 ? cu_sh[req] : a.cu_new[req]);   // cu_sh is filled only below 1024
    }
    // position, block-table slice (every block the workgroup can touch,
    // clamped to the row), query block of this wave's head tile and head
    // weights: all loads issued together
    const int blk0 = wg0 >> a.epb_log2;
    const int nbw = ((wg0 + IDX_EPW - 1) >> a.epb_log2) - blk0 + 1;
    const int sp = a.start_pos[req];
    int btv[(IDX_EPW + 255) / 256];
#pragma unroll
    for (int i = 0; i < (IDX_EPW + 255) / 256; ++i) {
        const int j = min(blk0 + min((int)threadIdx.x + 256 * i, nbw - 1), a.max_blocks - 1);
        btv[i] = a.block_table[(size_t)req * a.max_blocks + j];
    }
    uint4 f[4];
    if (wave < HT) {
        const int head = min(16 * wave + li, nh - 1);
        const char* qp = (const char*)a.q + ((size_t)gq * nh + head) * cI * 2 + (size_t)g * 64;
#pragma unroll
        for (int s = 0; s < 4; ++s) f[s] = ld16(qp + 16 * s);
    }
    float wv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = a.w[(size_t)gq * nh + min(16 * ht + 4 * g + i, nh - 1)];
    const int t = sp + tok;
    const int V = (t + 1) / a.m;
    if (blockIdx.y == 0 && threadIdx.x == 0) a.n_valid[gq] = V;
    if (wg0 >= V) return;                        // workgroup-uniform
#pragma unroll
    for (int i = 0; i < (IDX_EPW + 255) / 256; ++i)
        if ((int)threadIdx.x + 256 * i < nbw) bt[threadIdx.x + 256 * i] = btv[i];
    if (wave < HT) {
        uint4 codes;
        const int sc = mx_quant_codes(f, codes);
        qc_sh[wave][lane] = sel16(16 * wave + li < nh, codes);
        qs_sh[wave][lane] = sc;
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = 16 * ht + 4 * g + i < nh ? wv[ht][i] : 0.f;
    __syncthreads();
    uint4 Aq[HT];
    int sa[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        Aq[ht] = qc_sh[ht][lane];
        sa[ht] = qs_sh[ht][lane];
    }

    // loads are unconditional (entries past V are clamped to V-1, whose
    // scores are not stored), so the wait counts stay exact
    const size_t codes_off = (size_t)a.epb * (cI / 2);
    auto load = [&](int e0, uint4 (&B)[4], uint32_t (&SC)[4]) {
#pragma unroll
        for (int tile = 0; tile < 4; ++tile) {
            const int e = min(e0 + 16 * tile + li, V - 1);
            const char* kb = (const char*)a.keys + (size_t)bt[(e >> a.epb_log2) - blk0] * a.key_block_bytes;
            const int slot = (e & (a.epb - 1));
            B[tile] = ld16(kb + (size_t)slot * (cI / 2) + (size_t)g * 16);
            SC[tile] = (uint8_t)kb[codes_off + (size_t)slot * (cI / 32) + g];
        }
    };
    // NB buffers: NB-1 iterations of keys in flight while one is multiplied
    constexpr int NB = 2;
    uint4 B[NB][4];
    uint32_t SC[NB][4];
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) {
        if (j < IDX_ITERS) load(wg0 + 256 * j + wave * 64, B[j], SC[j]);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int it = 0; it < IDX_ITERS; ++it) {
        const int cur = it % NB;
        const int e_base = wg0 + it * 256 + wave * 64;
        if (it + NB - 1 < IDX_ITERS) load(e_base + 256 * (NB - 1), B[(it + NB - 1) % NB], SC[(it + NB - 1) % NB]);
        __builtin_amdgcn_sched_barrier(0);
        if (e_base >= V) break;                  // wave-uniform
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int tile = 0; tile < 4; ++tile) {
                const f32x4_t acc = mfma_fp4(Aq[ht], sa[ht], B[cur][tile], (int)SC[cur][tile]);
#pragma unroll
                for (int i = 0; i < 4; ++i) v[tile] += wv[ht][i] * relu_clamp(acc[i]);
            }
        // transposed sum over the four lane groups (as the bf16 kernel):
        // lane (g, li) ends with the entry of tile 2 (g & 1) + (g >> 1)
        const bool o1 = g & 1, o2 = g & 2;
        float k0 = o1 ? v[2] : v[0], k1 = o1 ? v[3] : v[1];
        k0 += __shfl_xor(o1 ? v[0] : v[2], 16, 64);
        k1 += __shfl_xor(o1 ? v[1] : v[3], 16, 64);
        float x = o2 ? k1 : k0;
        x += __shfl_xor(o2 ? k0 : k1, 32, 64);
        const int e = e_base + 16 * (2 * (g & 1) + (g >> 1)) + li;
        uint32_t hbin = ~0u;
        if (e < V) {
            if (x == 0.0f) x = 0.0f;                    // -0 is stored as +0
            if (a.score_bf16) {
                const uint16_t b = canon_bf16(f32_to_bf16(x));   // a value rounding to -0 is stored as +0
                ((uint16_t*)a.scores)[(size_t)gq * a.ld + e] = b;
                hbin = key16(b) >> 8;
            } else {
                ((float*)a.scores)[(size_t)gq * a.ld + e] = x;
            }
        }
        if (HIST) count_bins_quad(hcnt, hbin);
    }
    store_hist<HIST>(a, gq, blockIdx.y, hcnt);
}

template <int IDXF, int HT, bool HIST>
static void launch_ht(hipStream_t st, const IndexArgs& a, dim3 grid)
{
    // fragments per lane group: quarter of the key width / elements per fragment
    const int quarter = a.cI / 4;
    const int epf = IDXF == 0 ? 4 : 8;
    const int S = quarter / epf;
    switch (S) {
    case 1: index_decode_kernel<IDXF, HT, 1, HIST><<<grid, 256, 0, st>>>(a); break;
    case 2: index_decode_kernel<IDXF, HT, 2, HIST><<<grid, 256, 0, st>>>(a); break;
    case 4: index_decode_kernel<IDXF, HT, 4, HIST><<<grid, 256, 0, st>>>(a); break;
    case 8: index_decode_kernel<IDXF, HT, 8, HIST><<<grid, 256, 0, st>>>(a); break;
    default: break;
    }
}

template <int IDXF, bool HIST>
static void launch_fmt(hipStream_t st, const IndexArgs& a, dim3 grid)
{
    const int HT = (a.nh + 15) / 16;
    switch (HT) {
    case 1: launch_ht<IDXF, 1, HIST>(st, a, grid); break;
    case 2: launch_ht<IDXF, 2, HIST>(st, a, grid); break;
    case 3: launch_ht<IDXF, 3, HIST>(st, a, grid); break;
    default: launch_ht<IDXF, 4, HIST>(st, a, grid); break;
    }
}

template <bool BF16OUT>
static void launch_prefill(hipStream_t st, const IndexArgs& a, dim3 grid, int groups)
{
    const int HT = (a.nh + 15) / 16;
    if (HT == 4) index_prefill_kernel<4, 4, BF16OUT><<<grid, 512, 0, st>>>(a, groups);
    else if (HT == 3) index_prefill_kernel<3, 4, BF16OUT><<<grid, 512, 0, st>>>(a, groups);
    else if (HT == 2) index_prefill_kernel<2, 4, BF16OUT><<<grid, 512, 0, st>>>(a, groups);
    else index_prefill_kernel<1, 4, BF16OUT><<<grid, 512, 0, st>>>(a, groups);
}

template <bool HIST>
static void launch_fp4(hipStream_t st, const IndexArgs& a, dim3 grid)
{
    const int HT = (a.nh + 15) / 16;
    if (HT == 4) index_decode_fp4_kernel<4, HIST><<<grid, 256, 0, st>>>(a);
    else if (HT == 3) index_decode_fp4_kernel<3, HIST><<<grid, 256, 0, st>>>(a);
    else if (HT == 2) index_decode_fp4_kernel<2, HIST><<<grid, 256, 0, st>>>(a);
    else index_decode_fp4_kernel<1, HIST><<<grid, 256, 0, st>>>(a);
}

int index_min_chunk(int idx_fmt) { return idx_fmt == 2 ? IDX_EPW : IDXD_EPW; }

hipError_t launch_index(hipStream_t st, const IndexArgs& args, int max_visible, int max_new, int* chunk)
{
    if (args.n_tokens <= 0) return hipSuccess;
    IndexArgs a = args;
    // n_tokens tokens over n_req requests with at most one each: one apiece
    a.one_per_req = max_new <= 1 && a.n_tokens == a.n_req;
    // the per-chunk counts of the fused top-k (bf16 scores only)
    const bool hist = a.hist != nullptr && a.score_bf16;
    if (a.idx_fmt == 1 && a.cI == 128 && a.nh <= 64 && max_new >= 2 * PF_QPW && a.n_req < 1024) {
        // MFMA-bound: the counts are left to a pass over the stored scores
        // (*chunk = 0), which costs less than counting here
        if (chunk) *chunk = 0;
        const int groups = (max_new + PF_QPW - 1) / PF_QPW;
        dim3 grid(max_visible > 0 ? (max_visible + PF_ECH - 1) / PF_ECH : 1, a.n_req * groups);
        if (!a.score_bf16) launch_prefill<false>(st, a, grid, groups);
        else launch_prefill<true>(st, a, grid, groups);
        return hipGetLastError();
    }
    const int epw = a.idx_fmt == 2 ? IDX_EPW : IDXD_EPW;
    if (chunk) *chunk = epw;
    a.hist_chunks = (a.ld + epw - 1) / epw;
    dim3 grid(a.n_tokens, max_visible > 0 ? (max_visible + epw - 1) / epw : 1);
    if (a.idx_fmt == 0) {
        if (hist) launch_fmt<0, true>(st, a, grid);
        else launch_fmt<0, false>(st, a, grid);
    } else if (a.idx_fmt == 1) {
        if (hist) launch_fmt<1, true>(st, a, grid);
        else launch_fmt<1, false>(st, a, grid);
    } else {
        if (hist) launch_fp4<true>(st, a, grid);
        else launch_fp4<false>(st, a, grid);
    }
    return hipGetLastError();
}

}  // namespace csa
