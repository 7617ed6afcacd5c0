// a5 / a6: shared-KV MQA over compressed entries plus the raw sliding window,
// with a per-head sink logit, on gfx950.
//
// "DeepSeek-V4 内部机制" §1.2 Step 2 (the selected compressed entries serve as
// both key and value; every head has its own query), §1.3 (HCA: all visible
// entries, no top-k), §1.4 table (RMSNorm of each query head, partial RoPE on
// the last r channels with the output rotated back at -t, the 128-token
// uncompressed window, and the sink logit that only enters the softmax
// denominator); yunpan.plus explainer eq. (9).
//
// Work split: a workgroup of NW waves (8 for c >= 256, two per SIMD, else 4)
// owns one query, a group of 16*HT heads and a contiguous range of 32-row KV
// tiles (a split).  Rows are the query's selected entries (sparse) or all
// visible entries (dense), then its window.
//
// Tile pipeline: while tile n computes, the rows of tile n+1 are loaded as
// stored (FP8 entry record or bf16 / fp32 row) into registers, one row per
// load instruction (16 contiguous bytes per lane), with the FP8 block scale
// of each row; a tile is expanded once into Kt [32][C] (row-major, FP8 codes
// converted exactly to bf16), which serves both as the A operand of
// S^T = K . Q^T and, through the LDS transpose read, as the A operand of
// O^T = V^T . P^T (keys and values are the same rows).  The per-row FP8 block
// scale is applied to the fp32 logits of the FP8 channels and folded into P
// for the FP8 value channels.
//
// The waves split the channels: wave w contracts its C/NW channels for every
// head of the group (each K element is read from LDS once per workgroup), the
// partial logits are summed through LDS in wave order, the softmax of head
// tile h runs on wave h, and wave w then accumulates the output channels of
// its slice for every head.  The rotary channels fill whole waves' slices, so
// each wave's logits are either all FP8-scaled or all not.  Online softmax in
// base 2; splits write (max, sum, O) partials that a combine kernel merges in
// split order, so the output does not depend on scheduling.
#include <type_traits>

#include "csa.h"
#include "common.hpp"
#include "kernels.hpp"

namespace csa {


constexpr float LOG2E = 1.4426950408889634f;

template <int KVF, int C, int R, int HT>
struct AttnCfg {
    static constexpr int NF = C - R;                                     // non-rotary channels
    static constexpr bool F32 = KVF == 0;
    using MMA = typename std::conditional<F32, MmaF32, MmaBF16>::type;
    using ET = typename std::conditional<F32, float, uint16_t>::type;   // LDS element type
    static constexpr int EPF = 16 / sizeof(ET);                          // elements per fragment
    static constexpr int NW = C >= 256 ? 8 : 4;                          // waves
    static constexpr int NT = 64 * NW;                                   // threads
    static constexpr int DW = C / NW;                                    // channels per wave
    static constexpr int KSW = DW / MMA::K;                              // contraction steps per wave
    static constexpr int DTW = DW / 16;                                  // 16-channel output tiles per wave
    static constexpr int NNW = NF / DW;                                  // waves holding non-rotary channels
    static constexpr int RPW = 32 / NW;                                  // tile rows loaded per wave
    static constexpr int KP = C + (F32 ? 4 : 8);                         // Kt row stride (elements)
    static constexpr int WB = C * (F32 ? 4 : 2);                         // bytes of a window row (and of a
                                                                         // bf16 / fp32 entry)
    static constexpr int EB = KVF == 2 ? NF + 2 * R : WB;                // bytes of an entry record
    static constexpr int NCH = NF / 16;                                  // 16-byte chunks of FP8 codes
    // bf16 KV with fp32 accumulation: the normalised query and the softmax
    // weights enter the bf16 MFMAs as hi + lo bf16 pairs (about 16
    // significant bits) instead of one rounded bf16 value
    static constexpr bool SPLIT = KVF == 1 && C <= 256;
    static constexpr int QPARTS = SPLIT ? 2 : 1;
    // P^T fragments per head tile: fp32 two 16-row steps; FP8 plain + scaled
    // (value channels of FP8 entries); bf16 hi (+ lo)
    static constexpr int NPF = F32 ? 2 : (KVF == 2 ? 2 : QPARTS);
    static_assert(KSW >= 1 && DW % MMA::K == 0 && DW % 16 == 0, "channel split");
    static_assert(NF % DW == 0, "the rotary channels fill whole waves' slices");
    static_assert(WB <= 1024, "one 64-lane 16-byte load per row");
    static_assert(KVF != 2 || NF % 16 == 0, "FP8 codes in 16-byte chunks");
    static_assert(HT <= NW, "one softmax wave per head tile");
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int KVF, int C, int R, int HT>
__global__ __launch_bounds__((AttnCfg<KVF, C, R, HT>::NT)) void attn_kernel(AttnArgs a)
{
    using Cfg = AttnCfg<KVF, C, R, HT>;
    using MMA = typename Cfg::MMA;
    using ET = typename Cfg::ET;
    constexpr int EPF = Cfg::EPF, KP = Cfg::KP, DW = Cfg::DW, KSW = Cfg::KSW, DTW = Cfg::DTW;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, RPW = Cfg::RPW, NPF = Cfg::NPF, NNW = Cfg::NNW;
    constexpr int DESC = 256;                                  // rows described at a time
    constexpr int nf = Cfg::NF;

    __shared__ __attribute__((aligned(16))) ET Kt[32 * KP];
    __shared__ __attribute__((aligned(16))) f32x4_t Sbuf[NW][HT][2][64];  // partial logits per wave
    __shared__ __attribute__((aligned(16))) uint4 Pbuf[HT][NPF][64];      // P^T fragments per head tile
    __shared__ float Abuf[HT][16];                             // rescale factor per head
    __shared__ float Mbuf[HT][16], Lbuf[HT][16];               // final (max, sum) per head
    __shared__ float SSbuf[NW][HT][16];                        // partial sums of squares of the query heads
    __shared__ int Rflag[HT];
    __shared__ const char* rptr[DESC];                         // row start (null: masked row)
    __shared__ const char* rblk[DESC];                         // FP8 entry rows: their block (scale at byte 0)
    __shared__ float tscl[32];                                 // the current tile's scales
    __shared__ int tval[32];                                   // ... and valid rows
    __shared__ float rcs[R / 2], rsn[R / 2];
    __shared__ int cu_sh[257];

    const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gq = blockIdx.x;
    const int hbase = blockIdx.y * 16 * HT;
    const int split = blockIdx.z;
    const int dw0 = wave * DW;                                 // first channel of this wave

    // query fragments (B operand of S^T) of head hbase + 16*ht + li, channels
    // dw0 + s*K + g*EPF ..; loaded first, with the norm gains of the same
    // channels, so that their latency overlaps the request lookup
    uint4 QB[HT][KSW];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int head = hbase + 16 * ht + li;
        const char* qp = (const char*)a.q + ((size_t)gq * a.nh + (head < a.nh ? head : 0)) * C * sizeof(ET);
#pragma unroll
        for (int s = 0; s < KSW; ++s) QB[ht][s] = ld16(qp + (size_t)(dw0 + s * MMA::K + g * EPF) * sizeof(ET));
    }
    uint4 GB[KSW][EPF / 4];
#pragma unroll
    for (int s = 0; s < KSW; ++s)
#pragma unroll
        for (int h = 0; h < EPF / 4; ++h) GB[s][h] = ld16(a.q_gamma + dw0 + s * MMA::K + g * EPF + 4 * h);

    const int req = find_request_block(a.cu_new, a.n_req, gq, cu_sh, 256);
    const int t = a.start_pos[req] + (gq - (a.n_req < 256 ? cu_sh[req] : a.cu_new[req]));
    const bool dense = a.sel == nullptr;
    const int V = (t + 1) / a.m;
    const int K0 = dense ? V : a.k;                            // entry slots before the window
    const int nwr = min(a.n_win, t + 1);
    const int w0 = t - nwr + 1;
    const int n_slots = K0 + a.n_win;
    const int n_tiles = (n_slots + 31) / 32;
    const int tile0 = split * a.tiles_per_split;
    const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);

    const size_t win_es = a.win_bf16 ? 2 : 4;
    const size_t rec = KVF == 2 ? (size_t)(nf + 2 * R) : (size_t)C * (KVF == 0 ? 4 : 2);
    const size_t hdr = KVF == 2 ? 64 : 0;
    const char* ring = (const char*)a.state + (size_t)req * a.state_stride;

    // ---- row descriptors of DESC consecutive slots: row start and (FP8
    //      entries) the block whose header holds the scale
    auto describe = [&](int first_slot) {
        for (int j = threadIdx.x; j < DESC; j += NT) {
            const int slot = first_slot + j;
            const char* p = nullptr;
            const char* blk = nullptr;
            if (slot < K0) {
                const int e = dense ? slot : a.sel[(size_t)gq * a.k + slot];
                if (e >= 0 && e < V) {
                    const int phys = a.block_table[(size_t)req * a.max_blocks + (e >> a.epb_log2)];
                    const char* b = (const char*)a.kv + (size_t)phys * a.kv_block_bytes;
                    p = b + hdr + (size_t)(e & (a.epb - 1)) * rec;
                    if (KVF == 2) blk = b;
                }
            } else if (slot < n_slots && slot - K0 < nwr) {
                p = ring + (size_t)((w0 + slot - K0) % a.win_cap) * C * win_es;
            }
            rptr[j] = p;
            rblk[j] = blk;
        }
    };
    // ---- loads of one tile into registers: wave w loads rows w, w+NW, ..,
    //      one row per instruction, lane l the row's bytes 16l..16l+15
    //      (clamped to the row, so the loads are branch-free; masked rows
    //      read a valid dummy row), and each FP8 entry row's block scale
    const char* dummy = (const char*)a.kv;
    auto load_tile = [&](int tile, int drow0, uint4 (&raw)[RPW], float (&rsr)[RPW]) {
        const int slot0 = tile * 32;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = wave + NW * j;
            const char* p = rptr[drow0 + row];
            const int bytes = (slot0 + row < K0) ? Cfg::EB : Cfg::WB;
            raw[j] = ld16((p != nullptr ? p : dummy) + min(lane * 16, bytes - 16));
            if constexpr (KVF == 2) {
                const char* b = rblk[drow0 + row];
                rsr[j] = *(const CSA_GLOBAL float*)(b != nullptr ? b : dummy);
            }
        }
    };
    // ---- expand a loaded tile into Kt (masked rows become zeros) and keep
    //      its row flags and scales
    auto store_tile = [&](int tile, int drow0, const uint4 (&raw)[RPW], const float (&rsr)[RPW]) {
        const int slot0 = tile * 32;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = wave + NW * j;
            const bool ok = rptr[drow0 + row] != nullptr;
            const bool entry = slot0 + row < K0;
            if (lane == 0) {
                tval[row] = ok;
                tscl[row] = (KVF == 2 && ok && entry) ? rsr[j] : 1.0f;
            }
            const uint4 v = sel16(ok, raw[j]);
            ET* kr = Kt + row * KP;
            if (KVF == 2 && entry) {
                // FP8 record: 16 codes per lane, then the bf16 rotary channels
                if (lane < Cfg::NCH) {
                    const uint2 b0 = e4m3x4_to_bf16x4(v.x), b1 = e4m3x4_to_bf16x4(v.y);
                    const uint2 b2 = e4m3x4_to_bf16x4(v.z), b3 = e4m3x4_to_bf16x4(v.w);
                    *(uint4*)(kr + 16 * lane) = make_uint4(b0.x, b0.y, b1.x, b1.y);
                    *(uint4*)(kr + 16 * lane + 8) = make_uint4(b2.x, b2.y, b3.x, b3.y);
                } else if (lane < Cfg::NCH + R / 8) {
                    *(uint4*)(kr + nf + 8 * (lane - Cfg::NCH)) = v;
                }
            } else if (lane * 16 < Cfg::WB) {
                *(uint4*)(kr + lane * EPF) = v;                // 8 bf16 or 4 fp32 channels
            }
        }
    };

    // ---- prologue: RoPE table at +t, the first descriptors and the partial
    //      sums of squares of the query heads over this wave's channels
    for (int j = threadIdx.x; j < R / 2; j += NT) rope_cs_f((double)t, a.inv_freq[j], &rcs[j], &rsn[j]);
    if (tile0 < tile1) describe(tile0 * 32);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            const uint32_t w4[4] = {QB[ht][s].x, QB[ht][s].y, QB[ht][s].z, QB[ht][s].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if constexpr (Cfg::F32) {
                    const float x = __uint_as_float(w4[h]);
                    ss += x * x;
                } else {
                    const float x0 = bf16_to_f32(w4[h] & 0xFFFF), x1 = bf16_to_f32(w4[h] >> 16);
                    ss += x0 * x0 + x1 * x1;
                }
            }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (g == 0) SSbuf[wave][ht][li] = ss;
    }
    __syncthreads();                                           // prologue: table, descriptors, sums ready
    // the first tile's loads are in flight while the query is prepared
    uint4 raw[RPW];
    float rsr[RPW];
    if (tile0 < tile1) load_tile(tile0, 0, raw, rsr);

    // normalised, rotated, scaled query fragments (registers)
    uint4 QF[HT][KSW][Cfg::QPARTS];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float ssum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) ssum += SSbuf[w][ht][li];
        const float inv = (hbase + 16 * ht + li < a.nh) ? 1.0f / sqrtf(ssum / (float)C + a.eps) : 0.f;
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            const int d0 = dw0 + s * MMA::K + g * EPF;
            const uint32_t w4[4] = {QB[ht][s].x, QB[ht][s].y, QB[ht][s].z, QB[ht][s].w};
            const float* gm = (const float*)&GB[s][0];
            float x[EPF];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if constexpr (Cfg::F32) {
                    x[h] = __uint_as_float(w4[h]);
                } else {
                    x[2 * h] = bf16_to_f32(w4[h] & 0xFFFF);
                    x[2 * h + 1] = bf16_to_f32(w4[h] >> 16);
                }
            }
#pragma unroll
            for (int j = 0; j < EPF; ++j) x[j] = gm[j] * (x[j] * inv);
            if (d0 >= nf) {
#pragma unroll
                for (int j = 0; j < EPF; j += 2) {
                    const int p = (d0 + j - nf) >> 1;
                    const float u0 = x[j], u1 = x[j + 1];
                    x[j] = u0 * rcs[p] - u1 * rsn[p];
                    x[j + 1] = u0 * rsn[p] + u1 * rcs[p];
                }
            }
            if constexpr (Cfg::F32) {
                QF[ht][s][0] = make_uint4(__float_as_uint(x[0] * a.scale_log2), __float_as_uint(x[1] * a.scale_log2),
                                          __float_as_uint(x[2] * a.scale_log2), __float_as_uint(x[3] * a.scale_log2));
            } else {
                uint32_t w[4], wl[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float v0 = x[2 * h] * a.scale_log2, v1 = x[2 * h + 1] * a.scale_log2;
                    w[h] = pack_bf16x2(v0, v1);
                    wl[h] = pack_bf16x2(v0 - bf16_to_f32(w[h] & 0xFFFF), v1 - bf16_to_f32(w[h] >> 16));
                }
                QF[ht][s][0] = make_uint4(w[0], w[1], w[2], w[3]);
                if constexpr (Cfg::SPLIT) QF[ht][s][Cfg::QPARTS - 1] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
            }
        }
    }

    f32x4_t O[HT][DTW];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < DTW; ++i) O[ht][i] = zero4();
    // online softmax state of head tile hs (waves < HT), per head li
    const int hs = HT == 1 ? 0 : (wave < HT ? wave : 0);
    const bool softmax_wave = HT == 1 || wave < HT;
    float m_run = -INFINITY, l_run = 0.f;
    uint4 Ploc[NPF];                                           // P^T fragments when HT == 1
    float alpha_loc = 1.f;
    bool raise_loc = false;

    for (int tile = tile0; tile < tile1; ++tile) {
        const int slot0 = tile * 32;
        const int drow0 = ((tile - tile0) * 32) % DESC;
        __syncthreads();                                       // the previous tile is done with Kt
        store_tile(tile, drow0, raw, rsr);
        __syncthreads();                                       // (A) tile in Kt
        // load the next tile while this one computes
        if (tile + 1 < tile1) {
            const int drow = ((tile + 1 - tile0) * 32) % DESC;
            if (drow == 0) {                                   // the next DESC rows
                describe((tile + 1) * 32);
                __syncthreads();
            }
            load_tile(tile + 1, drow, raw, rsr);
        }

        // ---- partial S^T over this wave's channels, rows 16*rt + li of the tile
        f32x4_t acc[HT][2];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) { acc[ht][0] = zero4(); acc[ht][1] = zero4(); }
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            const int d0 = dw0 + s * MMA::K;
            const uint4 ka = *(const uint4*)(Kt + li * KP + d0 + g * EPF);
            const uint4 kb = *(const uint4*)(Kt + (16 + li) * KP + d0 + g * EPF);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int part = 0; part < Cfg::QPARTS; ++part) {
                    acc[ht][0] = MMA::step(ka, QF[ht][s][part], acc[ht][0]);
                    acc[ht][1] = MMA::step(kb, QF[ht][s][part], acc[ht][1]);
                }
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) Sbuf[wave][ht][rt][lane] = acc[ht][rt];
        __syncthreads();                                       // (B) partial logits in LDS

        // ---- softmax of head tile hs: the partials summed in wave order; the
        //      FP8 block scale multiplies the non-rotary waves' sum (window
        //      rows carry scale 1).  Lane holds rows 16*rt + 4g + i of head li.
        if (softmax_wave) {
            float rsc[2][4];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) rsc[rt][i] = KVF == 2 ? tscl[16 * rt + 4 * g + i] : 1.f;
            float sv[8];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4_t vn = Sbuf[0][hs][rt][lane];
#pragma unroll
                for (int w = 1; w < NNW; ++w) vn += Sbuf[w][hs][rt][lane];
                f32x4_t vr = Sbuf[NNW][hs][rt][lane];
#pragma unroll
                for (int w = NNW + 1; w < NW; ++w) vr += Sbuf[w][hs][rt][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = tval[16 * rt + 4 * g + i] != 0;
                    const float v = KVF == 2 ? rsc[rt][i] * vn[i] + vr[i] : vn[i] + vr[i];
                    sv[4 * rt + i] = valid ? v : -INFINITY;
                }
            }
            float mx = sv[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            // The reference max only moves when a logit exceeds it by more than
            // 2^8 (base-2 units), so weights stay <= 256 and the accumulators
            // are rescaled rarely; the final normalisation uses the same
            // reference.
            const bool raise = mx > m_run + 8.0f;
            const bool rescale = raise && m_run != -INFINITY;   // nothing accumulated yet otherwise
            const float m_new = raise ? mx : m_run;
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
            float p[8], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) { p[i] = __builtin_amdgcn_exp2f(sv[i] - m_use); ps += p[i]; }
            ps += __shfl_xor(ps, 16, 64);
            ps += __shfl_xor(ps, 32, 64);
            l_run = l_run * alpha + ps;
            m_run = m_new;
            uint4 pf[NPF];
            if constexpr (Cfg::F32) {
                pf[0] = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3]));
                pf[1] = make_uint4(__float_as_uint(p[4]), __float_as_uint(p[5]), __float_as_uint(p[6]), __float_as_uint(p[7]));
            } else {
                pf[0] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                   pack_bf16x2(p[6], p[7]));
                if constexpr (KVF == 2) {
                    // value channels of FP8 entry rows carry the block scale
                    float q8[8];
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) q8[4 * rt + i] = p[4 * rt + i] * rsc[rt][i];
                    pf[1] = make_uint4(pack_bf16x2(q8[0], q8[1]), pack_bf16x2(q8[2], q8[3]),
                                       pack_bf16x2(q8[4], q8[5]), pack_bf16x2(q8[6], q8[7]));
                } else if constexpr (Cfg::SPLIT) {
                    const uint32_t h4[4] = {pf[0].x, pf[0].y, pf[0].z, pf[0].w};
                    uint32_t l4[4];
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        l4[h] = pack_bf16x2(p[2 * h] - bf16_to_f32(h4[h] & 0xFFFF), p[2 * h + 1] - bf16_to_f32(h4[h] >> 16));
                    pf[NPF - 1] = make_uint4(l4[0], l4[1], l4[2], l4[3]);
                }
            }
            if constexpr (HT == 1) {
#pragma unroll
                for (int v = 0; v < NPF; ++v) Ploc[v] = pf[v];
                alpha_loc = alpha;
                raise_loc = __any(rescale);
            } else {
#pragma unroll
                for (int v = 0; v < NPF; ++v) Pbuf[hs][v][lane] = pf[v];
                if (g == 0) Abuf[hs][li] = alpha;
                const bool any_rescale = __any(rescale);
                if (lane == 0) Rflag[hs] = any_rescale;
            }
        }
        if constexpr (HT > 1) __syncthreads();                 // (C) P^T and rescale factors in LDS

        // ---- O^T += V^T . P^T for this wave's channels and every head tile.
        //      The V^T fragment of lane (li, g) holds channel c0 + li of rows
        //      4g..4g+3 and 16+4g..16+4g+3 (contraction order 8g..8g+7), read
        //      from the row-major tile with two LDS transpose reads; it is
        //      read once and used for all head tiles.
        uint4 pf[HT][NPF];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            bool rz;
            float al;
            if constexpr (HT == 1) {
#pragma unroll
                for (int v = 0; v < NPF; ++v) pf[ht][v] = Ploc[v];
                rz = raise_loc;
                al = alpha_loc;
            } else {
#pragma unroll
                for (int v = 0; v < NPF; ++v) pf[ht][v] = Pbuf[ht][v][lane];
                rz = Rflag[ht] != 0;
                al = Abuf[ht][li];
            }
            if (rz) {
#pragma unroll
                for (int dt = 0; dt < DTW; ++dt) O[ht][dt] *= al;
            }
        }
        // FP8: the non-rotary waves take the scaled weights (a wave-uniform choice)
        auto pv_all = [&](auto sel) {
            constexpr int VSEL = decltype(sel)::value;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) {
                const int c0 = dw0 + 16 * dt;
                if constexpr (Cfg::F32) {
                    float va[4], vb[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        va[j] = Kt[(4 * g + j) * KP + c0 + li];
                        vb[j] = Kt[(16 + 4 * g + j) * KP + c0 + li];
                    }
                    const uint4 fa = make_uint4(__float_as_uint(va[0]), __float_as_uint(va[1]), __float_as_uint(va[2]), __float_as_uint(va[3]));
                    const uint4 fb = make_uint4(__float_as_uint(vb[0]), __float_as_uint(vb[1]), __float_as_uint(vb[2]), __float_as_uint(vb[3]));
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) {
                        O[ht][dt] = MMA::step(fa, pf[ht][0], O[ht][dt]);
                        O[ht][dt] = MMA::step(fb, pf[ht][1], O[ht][dt]);
                    }
                } else {
                    // lane m of a 16-lane group points at 4 channels of one row:
                    // row 4g + m/4 (+16 for the second read), channels c0 + 4*(m%4)
                    const ET* base = Kt + (4 * g + (li >> 2)) * KP + c0 + 4 * (li & 3);
                    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4_t*)base);
                    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4_t*)(base + 16 * KP));
                    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
                    const uint4 va = make_uint4(l2.x, l2.y, h2.x, h2.y);
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) {
                        O[ht][dt] = MMA::step(va, pf[ht][VSEL], O[ht][dt]);
                        if constexpr (Cfg::SPLIT) O[ht][dt] = MMA::step(va, pf[ht][NPF - 1], O[ht][dt]);
                    }
                }
            }
        };
        if (KVF == 2 && dw0 < nf) pv_all(std::integral_constant<int, KVF == 2 ? 1 : 0>());
        else pv_all(std::integral_constant<int, 0>());
    }

    // ---- per-head (max, sum) of every head tile
    if constexpr (HT > 1) {
        if (softmax_wave && g == 0) { Mbuf[hs][li] = m_run; Lbuf[hs][li] = l_run; }
        __syncthreads();
    }
    // lane holds O^T[dw0 + 16*dt + 4g + i][head hbase + 16*ht + li].  Split
    // partial per (query, head, split): max, sum (fp32) at bytes 0 and 4, the
    // C channels from byte 16, in the output format.
    const size_t pstride = a.out_bf16 ? 2 * (size_t)C + 16 : 4 * (size_t)C + 16;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int head = hbase + 16 * ht + li;
        if (head >= a.nh) continue;
        const float mh = HT == 1 ? m_run : Mbuf[ht][li];
        const float lh = HT == 1 ? l_run : Lbuf[ht][li];
        if (a.n_splits == 1 && !a.invariant) {
            const float zs = a.sinks[head] * LOG2E;
            const float M = fmaxf(mh, zs);
            const float sc = exp2f(mh - M);
            const float inv = sc / (lh * sc + exp2f(zs - M));
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) {
                const int d = dw0 + 16 * dt + 4 * g;
                float o[4] = {O[ht][dt][0] * inv, O[ht][dt][1] * inv, O[ht][dt][2] * inv, O[ht][dt][3] * inv};
                if (d >= nf) {
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {           // rotate back at -t
                        const int pj = (d + j - nf) >> 1;
                        const float u0 = o[j], u1 = o[j + 1];
                        o[j] = u0 * rcs[pj] + u1 * rsn[pj];
                        o[j + 1] = -u0 * rsn[pj] + u1 * rcs[pj];
                    }
                }
                if (a.out_bf16) {
                    const uint2 w = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                    *(uint2*)((uint16_t*)a.out + ((size_t)gq * a.nh + head) * C + d) = w;
                } else {
                    *(float4*)((float*)a.out + ((size_t)gq * a.nh + head) * C + d) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        } else {
            char* pp = (char*)a.ws + (((size_t)gq * a.nh + head) * a.n_splits + split) * pstride;
            if (wave == 0 && g == 0) { ((float*)pp)[0] = mh; ((float*)pp)[1] = lh; }
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) {
                const int d = dw0 + 16 * dt + 4 * g;
                if (a.out_bf16)
                    *(uint2*)(pp + 16 + 2 * (size_t)d) = make_uint2(pack_bf16x2(O[ht][dt][0], O[ht][dt][1]),
                                                                    pack_bf16x2(O[ht][dt][2], O[ht][dt][3]));
                else
                    *(float4*)(pp + 16 + 4 * (size_t)d) = make_float4(O[ht][dt][0], O[ht][dt][1], O[ht][dt][2], O[ht][dt][3]);
            }
        }
    }
}

// What a slot of attn_ht_kernel reads when it has no row (past the query's
// entries or window, an entry that is not visible): 1 KB of zeros, and a
// scale word of -1, which marks the slot as masked.  bf16 window rows take
// the scale 1.
static __device__ __attribute__((aligned(16))) uint32_t attn_zero_row[256];
static __device__ float attn_masked_scale = -1.0f;
static __device__ float attn_unit_scale = 1.0f;

// FP8 entry records with bf16 queries (the serving shapes): two waves per
// head tile.  Waves w and w + HT own heads 16w .. 16w+15 of the group and one
// half of the channels each (alternate 32-channel MFMA steps for the logits,
// alternate 16-channel tiles for the output, so that both halves have the
// same mix of FP8 and rotary channels at the same positions): each contracts
// its half of the tile for those heads (S^T = K . Q^T), the two partial
// logits meet in LDS and each wave adds the other's to its own (a two-term
// sum, equal in both waves), both run the same online softmax in
// registers, and each accumulates the output
// of its half of the channels (O^T = V^T . P^T).  Tiles are double-buffered
// in LDS: the rows of the next two tiles are loaded into registers while one
// computes, and two barriers per tile publish a stored tile and the partial
// logits.  Each lane keeps the output of its head for 4 channels of every
// 16-channel tile of its half (C/8 fp32 accumulators).
template <int C, int R, int HT>
__global__ __launch_bounds__(128 * HT) void attn_ht_kernel(AttnArgs a)
{
    constexpr int NWV = 2 * HT;                                // waves
    constexpr int NF = C - R, KP = C + 8, NT = 64 * NWV, RPW = 32 / NWV;
    constexpr int KS = C / 32;                                 // 16x16x32 steps over the channels
    constexpr int KSN = NF / 32;                               // ... of them over FP8 channels
    constexpr int KSH = KS / 2;                                // ... per wave (its half of the channels)
    constexpr int DT = C / 16;                                 // 16-channel output tiles
    constexpr int DTN = NF / 16;                               // ... of them FP8 value channels
    constexpr int DTH = DT / 2;                                // ... per wave (its half of the channels)
    constexpr int WB = 2 * C;                                  // bytes of a window row (bf16)
    constexpr int EB = NF + 2 * R;                             // bytes of an FP8 entry record
    constexpr int NCH = NF / 16;                               // 16-byte chunks of FP8 codes
    constexpr int DESC = NT;                                   // rows described at a time
    static_assert(NF % 32 == 0 && R % 32 == 0 && WB <= 1024 && 32 % NWV == 0 && DESC % NT == 0 && DT % 2 == 0 &&
                  KSN % 2 == 0 && DTN % 2 == 0, "shape");
    // The two waves of a head tile take alternate 32-channel MFMA steps
    // (step 2j + half) and alternate 16-channel output tiles (tile 2j + half):
    // both then meet the FP8 / rotary boundary at the same j, so which
    // accumulator or which P a step uses is known at compile time.

    __shared__ __attribute__((aligned(16))) uint16_t Kt[2][32 * KP];
    __shared__ float tscl[2][32];                              // per buffer: row scales (-1: masked row)
    __shared__ const char* rptr[DESC];                         // row start (the zero row when masked)
    __shared__ const char* rblk[DESC];                         // the row's scale (FP8 entries: block byte 0)
    __shared__ float rcs[R / 2], rsn[R / 2];
    __shared__ int cu_sh[257];
    __shared__ __attribute__((aligned(16))) float gam[C];      // query norm gains times the softmax scale
    __shared__ __attribute__((aligned(16))) f32x4_t Sx[2][HT][2][2][64];  // partial logits per half
    __shared__ float ssx[HT][2][16];                           // partial sums of squares of the query

    const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ht = wave % HT, half = wave / HT;               // head tile, channel half
    for (int j = threadIdx.x; j < C; j += NT) gam[j] = a.q_gamma[j] * a.scale_log2;
    const int gq = blockIdx.x;
    const int head = blockIdx.y * 16 * HT + 16 * ht + li;     // this lane's head
    const bool hvalid = head < a.nh;
    const int split = blockIdx.z;
    const bool dense = a.sel == nullptr;

    // query fragments (B operand of S^T): channels 32s + 8g .. +7 of `head`,
    // loaded first so that their latency overlaps the lookups below
    uint4 QB[KSH];                                             // this wave's steps 2j + half
    {
        const char* qp = (const char*)a.q + ((size_t)gq * a.nh + (hvalid ? head : 0)) * C * 2;
#pragma unroll
        for (int j = 0; j < KSH; ++j) QB[j] = ld16(qp + (size_t)(32 * (2 * j + half) + 8 * g) * 2);
    }
    // selected entries of this workgroup's first rows (independent of the
    // position, so these loads overlap its lookup)
    const int tile0 = split * a.tiles_per_split;
    int esel[DESC / NT];
#pragma unroll
    for (int u = 0; u < DESC / NT; ++u) {
        const int slot = tile0 * 32 + (int)threadIdx.x + u * NT;
        esel[u] = (!dense && slot < a.k) ? a.sel[(size_t)gq * a.k + slot] : -1;
    }
    int req, tok;
    if (a.one_per_req) {
        req = gq;
        tok = 0;
    } else {
        req = find_request_block(a.cu_new, a.n_req, gq, cu_sh, 256);
        tok = gq - (a.n_req < 256 ? cu_sh[req] : a.cu_new[req]);
    }
    // the position and what follows from it are the same for the whole
    // workgroup (scalar registers, so the row-kind tests below are scalar)
    const int t = __builtin_amdgcn_readfirstlane(a.start_pos[req] + tok);
    const int V = (t + 1) / a.m;
    const int K0 = dense ? V : a.k;                            // entry slots before the window
    const int nwr = min(a.n_win, t + 1);
    const int w0 = t - nwr + 1;
    const int n_slots = K0 + a.n_win;
    const int n_tiles = (n_slots + 31) / 32;
    const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);
    const char* ring = (const char*)a.state + (size_t)req * a.state_stride;

    // ---- row descriptors of DESC consecutive slots (e: the entry of a
    //      slot < K0, already loaded for the first window of a sparse query):
    //      where the row starts and where its scale is; a masked slot gets the
    //      zero row and the scale -1
    const char* const zrow = (const char*)attn_zero_row;
    const char* const mscl = (const char*)&attn_masked_scale;
    const char* const uscl = (const char*)&attn_unit_scale;
    auto describe = [&](int first_slot, bool have_e) {
#pragma unroll
        for (int u = 0; u < DESC / NT; ++u) {
            const int j = (int)threadIdx.x + u * NT;
            const int slot = first_slot + j;
            const char* p = zrow;
            const char* blk = mscl;
            if (slot < K0) {
                const int e = dense ? slot : (have_e ? esel[u] : a.sel[(size_t)gq * a.k + slot]);
                if (e >= 0 && e < V) {
                    const int phys = a.block_table[(size_t)req * a.max_blocks + (e >> a.epb_log2)];
                    const char* b = (const char*)a.kv + (size_t)phys * a.kv_block_bytes;
                    p = b + 64 + (size_t)(e & (a.epb - 1)) * EB;
                    blk = b;
                }
            } else if (slot < n_slots && slot - K0 < nwr) {
                p = ring + (size_t)((w0 + slot - K0) % a.win_cap) * WB;
                blk = uscl;
            }
            rptr[j] = p;
            rblk[j] = blk;
        }
    };
    // ---- one tile into registers: wave w loads rows w, w+NWV, .., one row
    //      per instruction, lane l the row's bytes 16l..16l+15 (clamped to
    //      the row), and each row's scale
    auto load_tile = [&](int tile, int drow0, uint4 (&raw)[RPW], float (&rsr)[RPW]) {
        const int slot0 = tile * 32;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = wave + NWV * j;
            const int bytes = (slot0 + row < K0) ? EB : WB;
            raw[j] = ld16(rptr[drow0 + row] + min(lane * 16, bytes - 16));
            rsr[j] = *(const CSA_GLOBAL float*)rblk[drow0 + row];
        }
    };
    // ---- expand a loaded tile into Kt[buf] (masked rows are zeros already)
    //      with its row scales
    auto store_tile = [&](int tile, int buf, const uint4 (&raw)[RPW], const float (&rsr)[RPW]) {
        const int slot0 = tile * 32;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = wave + NWV * j;
            const bool entry = slot0 + row < K0;
            if (lane == 0) tscl[buf][row] = rsr[j];
            const uint4 v = raw[j];
            uint16_t* kr = &Kt[buf][row * KP];
            if (entry) {
                if (lane < NCH) {                              // 16 FP8 codes per lane
                    const uint2 b0 = e4m3x4_to_bf16x4(v.x), b1 = e4m3x4_to_bf16x4(v.y);
                    const uint2 b2 = e4m3x4_to_bf16x4(v.z), b3 = e4m3x4_to_bf16x4(v.w);
                    *(uint4*)(kr + 16 * lane) = make_uint4(b0.x, b0.y, b1.x, b1.y);
                    *(uint4*)(kr + 16 * lane + 8) = make_uint4(b2.x, b2.y, b3.x, b3.y);
                } else if (lane < NCH + R / 8) {               // the bf16 rotary channels
                    *(uint4*)(kr + NF + 8 * (lane - NCH)) = v;
                }
            } else if (lane * 16 < WB) {
                *(uint4*)(kr + 8 * lane) = v;                  // 8 bf16 channels of a window row
            }
        }
    };

    // ---- prologue: RoPE table at +t, the first descriptors and the partial
    //      sums of squares of the query heads over this wave's half
    for (int j = threadIdx.x; j < R / 2; j += NT) rope_cs_f((double)t, a.inv_freq[j], &rcs[j], &rsn[j]);
    if (tile0 < tile1) describe(tile0 * 32, true);
    {
        // sum of squares of this lane's channels: one bf16 dot product per
        // pair of channels
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < KSH; ++j) {
            const uint32_t w4[4] = {QB[j].x, QB[j].y, QB[j].z, QB[j].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w4[h]);
                ss = __builtin_amdgcn_fdot2_f32_bf16(v, v, ss, false);
            }
        }
        ss = xsum32(xsum16(ss));
        if (g == 0) ssx[ht][half][li] = ss;
    }
    __syncthreads();
    // two tiles in flight: the rows of tiles n+1 and n+2 load while tile n
    // computes (slot k of raw / rsr and LDS buffer k serve tiles
    // tile0 + k, tile0 + k + 2, ..)
    static_assert(DESC >= 64, "two tiles per descriptor window");
    uint4 raw[2][RPW];
    float rsr[2][RPW];
    if (tile0 < tile1) load_tile(tile0, 0, raw[0], rsr[0]);
    if (tile0 + 1 < tile1) load_tile(tile0 + 1, 32, raw[1], rsr[1]);

    // normalised, rotated, scaled query fragments of this lane's head (the
    // softmax scale is in gam; the rotation is linear, so it commutes)
    uint4 QF[KSH];
    {
        const float ss = ssx[ht][0][li] + ssx[ht][1][li];     // the same order in both waves
        const float inv = hvalid ? 1.0f / sqrtf(ss / (float)C + a.eps) : 0.f;
#pragma unroll
        for (int j = 0; j < KSH; ++j) {
            const int s = 2 * j + half;
            const int d0 = 32 * s + 8 * g;
            const float4 ga = *(const float4*)(gam + d0), gb = *(const float4*)(gam + d0 + 4);
            const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
            const uint32_t w4[4] = {QB[j].x, QB[j].y, QB[j].z, QB[j].w};
            float x[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                x[2 * h] = gm[2 * h] * (bf16_to_f32(w4[h] & 0xFFFF) * inv);
                x[2 * h + 1] = gm[2 * h + 1] * (bf16_to_f32(w4[h] >> 16) * inv);
            }
            if (j >= KSN / 2) {                                // the rotary steps (compile-time)
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const int pr = (d0 + j - NF) >> 1;
                    const float u0 = x[j], u1 = x[j + 1];
                    x[j] = u0 * rcs[pr] - u1 * rsn[pr];
                    x[j + 1] = u0 * rsn[pr] + u1 * rcs[pr];
                }
            }
            QF[j] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                               pack_bf16x2(x[6], x[7]));
        }
    }

    // lane (g, li): O^T[16 (2j + half) + 4g + i][head li]
    f32x4_t O[DTH];
#pragma unroll
    for (int j = 0; j < DTH; ++j) O[j] = zero4();
    float m_run = -INFINITY, l_run = 0.f;

    auto tile_step = [&](int tile, auto slot) {
        constexpr int buf = decltype(slot)::value;
        // Kt[buf] was last read by tile-2, which every wave finished before
        // the barrier of tile-1
        store_tile(tile, buf, raw[buf], rsr[buf]);
        __syncthreads();                                       // tile in Kt[buf]
        if (tile + 2 < tile1) {
            const int drow = ((tile + 2 - tile0) * 32) % DESC;
            if (drow == 0) {                                   // the next DESC rows (the loads of tile+1
                describe((tile + 2) * 32, false);              // are issued, stores read no descriptors)
                __syncthreads();
            }
            load_tile(tile + 2, drow, raw[buf], rsr[buf]);
        }
        const uint16_t* kt = Kt[buf];

        // ---- S^T (rows 16 rt + 4g + i, head li); FP8 and rotary channels apart
        // K fragments of this wave's half, read QC steps ahead of the MFMAs
        constexpr int QC = 2;
        static_assert(KSH % QC == 0, "whole chunks");
        f32x4_t an[2] = {zero4(), zero4()}, ar[2] = {zero4(), zero4()};
        uint4 kf[2][QC][2];
        auto read_k = [&](int c, uint4 (&f)[QC][2]) {
#pragma unroll
            for (int u = 0; u < QC; ++u) {
                const int s = 2 * (QC * c + u) + half;
                f[u][0] = *(const uint4*)(kt + li * KP + 32 * s + 8 * g);
                f[u][1] = *(const uint4*)(kt + (16 + li) * KP + 32 * s + 8 * g);
            }
        };
        read_k(0, kf[0]);
#pragma unroll
        for (int c = 0; c < KSH / QC; ++c) {
            if (c + 1 < KSH / QC) read_k(c + 1, kf[(c + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < QC; ++u) {
                const int j = QC * c + u;
                if (j < KSN / 2) {                             // compile-time
                    an[0] = MmaBF16::step(kf[c & 1][u][0], QF[j], an[0]);
                    an[1] = MmaBF16::step(kf[c & 1][u][1], QF[j], an[1]);
                } else {
                    ar[0] = MmaBF16::step(kf[c & 1][u][0], QF[j], ar[0]);
                    ar[1] = MmaBF16::step(kf[c & 1][u][1], QF[j], ar[1]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- the two halves' partial logits (FP8 channels scaled by the
        //      row's block scale) meet in LDS (a masked row's zeros give 0
        //      whatever its scale)
        float rsc[8];
        f32x4_t part[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rsc[4 * rt + i] = tscl[buf][16 * rt + 4 * g + i];
                part[rt][i] = rsc[4 * rt + i] * an[rt][i] + ar[rt][i];
            }
            Sx[buf][ht][half][rt][lane] = part[rt];
        }
        __syncthreads();                                       // partial logits of both halves in LDS
        // ---- online softmax of head li over the 32 rows, in base 2; each
        //      wave reads the other half's partials only (a sum of two terms
        //      is the same in either order, so both waves get equal logits)
        float sv[8];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const f32x4_t so = Sx[buf][ht][half ^ 1][rt][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sv[4 * rt + i] = rsc[4 * rt + i] >= 0.f ? part[rt][i] + so[i] : -INFINITY;   // -1: masked
            }
        }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = xmax32(xmax16(mx));
        // the reference max moves only when a logit exceeds it by more than
        // 2^8 (base 2), so weights stay <= 256 and rescales are rare
        const bool raise = mx > m_run + 8.0f;
        const bool rescale = raise && m_run != -INFINITY;
        const float m_new = raise ? mx : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
        float p[8], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
            ps += p[i];
        }
        ps = xsum32(xsum16(ps));
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if (__any(rescale)) {
#pragma unroll
            for (int j = 0; j < DTH; ++j) O[j] *= alpha;
        }
        // P^T: plain weights for the rotary (bf16) channels, weights times the
        // row's block scale for the FP8 value channels
        const uint4 pp = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                    pack_bf16x2(p[6], p[7]));
        const uint4 psc = make_uint4(pack_bf16x2(p[0] * rsc[0], p[1] * rsc[1]), pack_bf16x2(p[2] * rsc[2], p[3] * rsc[3]),
                                     pack_bf16x2(p[4] * rsc[4], p[5] * rsc[5]), pack_bf16x2(p[6] * rsc[6], p[7] * rsc[7]));
        // ---- O^T += V^T . P^T: lane m of a 16-lane group points at 4
        //      channels of one row (row 4g + m/4, +16 for the second read), so
        //      the transpose reads give lane (g, li) channel c0 + li of rows
        //      4g..4g+3 and 16+4g..16+4g+3, the order of P^T's contraction
        // V^T fragments read VC tiles ahead of their MFMAs
        constexpr int VC = 2;
        static_assert(DTH % VC == 0, "whole chunks");
        uint4 vf[2][VC];
        auto read_v = [&](int c, uint4 (&f)[VC]) {
#pragma unroll
            for (int u = 0; u < VC; ++u) {
                const int dt = 2 * (VC * c + u) + half;
                const uint16_t* base = kt + (4 * g + (li >> 2)) * KP + 16 * dt + 4 * (li & 3);
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4_t*)base);
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS s16x4_t*)(base + 16 * KP));
                const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
                f[u] = make_uint4(l2.x, l2.y, h2.x, h2.y);
            }
        };
        read_v(0, vf[0]);
#pragma unroll
        for (int c = 0; c < DTH / VC; ++c) {
            if (c + 1 < DTH / VC) read_v(c + 1, vf[(c + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < VC; ++u) {
                const int j = VC * c + u;
                O[j] = MmaBF16::step(vf[c & 1][u], j < DTN / 2 ? psc : pp, O[j]);   // compile-time choice
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int tile = tile0; tile < tile1; tile += 2) {
        tile_step(tile, std::integral_constant<int, 0>());
        if (tile + 1 < tile1) tile_step(tile + 1, std::integral_constant<int, 1>());
    }

    // ---- output: the normalised result (one split) or the split partial
    //      (max, sum at bytes 0 and 4, the C channels from byte 16)
    if (!hvalid) return;
    if (a.n_splits == 1 && !a.invariant) {
        const float zs = a.sinks[head] * LOG2E;
        const float M = fmaxf(m_run, zs);
        const float sc = exp2f(m_run - M);
        const float inv = sc / (l_run * sc + exp2f(zs - M));
#pragma unroll
        for (int j = 0; j < DTH; ++j) {
            const int d = 16 * (2 * j + half) + 4 * g;
            float o[4] = {O[j][0] * inv, O[j][1] * inv, O[j][2] * inv, O[j][3] * inv};
            if (j >= DTN / 2) {                                // the rotary channels (compile-time)
#pragma unroll
                for (int j = 0; j < 4; j += 2) {               // rotate back at -t
                    const int pj = (d + j - NF) >> 1;
                    const float u0 = o[j], u1 = o[j + 1];
                    o[j] = u0 * rcs[pj] + u1 * rsn[pj];
                    o[j + 1] = -u0 * rsn[pj] + u1 * rcs[pj];
                }
            }
            if (a.out_bf16)
                *(uint2*)((uint16_t*)a.out + ((size_t)gq * a.nh + head) * C + d) =
                    make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            else
                *(float4*)((float*)a.out + ((size_t)gq * a.nh + head) * C + d) = make_float4(o[0], o[1], o[2], o[3]);
        }
    } else {
        const size_t pstride = a.out_bf16 ? 2 * (size_t)C + 16 : 4 * (size_t)C + 16;
        char* pp = (char*)a.ws + (((size_t)gq * a.nh + head) * a.n_splits + split) * pstride;
        if (g == 0 && half == 0) {
            ((float*)pp)[0] = m_run;
            ((float*)pp)[1] = l_run;
        }
#pragma unroll
        for (int j = 0; j < DTH; ++j) {
            const int d = 16 * (2 * j + half) + 4 * g;
            if (a.out_bf16)
                *(uint2*)(pp + 16 + 2 * (size_t)d) = make_uint2(pack_bf16x2(O[j][0], O[j][1]),
                                                                pack_bf16x2(O[j][2], O[j][3]));
            else
                *(float4*)(pp + 16 + 4 * (size_t)d) = make_float4(O[j][0], O[j][1], O[j][2], O[j][3]);
        }
    }
}

// Merge the split partials of one (query, head) in split order, add the sink,
// normalise, rotate back at -t and store.  The weights and the denominator
// come from fixed-order reductions, so the result does not depend on
// scheduling.
// NSUB waves per (query, head), 4 / NSUB (query, head) pairs per workgroup,
// no LDS, no barrier and no exchange between lanes: lane l of sub-wave u
// holds the CPL = 8 / NSUB output channels from 64 CPL u + CPL l and reads
// every split's (max, sum) itself (the same addresses in every lane, one
// memory request per wave), so the reference max M (with the sink), the
// denominator and the weighted sum of the partial outputs are formed in
// split order, alike in every lane.  The loads of a batch of CB splits (their
// (max, sum) and the lane's channels) are all issued before any is used, so
// up to CB splits cost one round trip to memory.  Two waves per pair
// (NSUB = 2, 512 channels) double the waves that keep loads in flight.
template <bool BF, int CB, int NSUB>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a)
{
    constexpr int CPL = 8 / NSUB;                              // channels per lane
    constexpr int W = BF ? CPL / 2 : CPL;                      // 32-bit words per lane and split
    static_assert(W == 2 || W % 4 == 0, "8- or 16-byte pieces");
    // the wave index (so the head, the split rows' addresses and every
    // split's (max, sum)) is uniform in the wave: in scalar registers a
    // split's address is one scalar add, not a 64-bit multiply per lane
    // (batches of up to 16 splits; 32 splits' (max, sum) pairs would not fit
    // the scalar registers)
    const int lane = threadIdx.x & 63;
    const int wv = CB <= 16 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : (int)(threadIdx.x >> 6);
    const int gq = blockIdx.x, head = blockIdx.y * (4 / NSUB) + wv / NSUB, sub = wv % NSUB;
    if (head >= a.nh) return;                                  // wave-uniform
    const int C = a.c, S = a.n_splits, nf = C - a.r;
    const size_t pstride = BF ? 2 * (size_t)C + 16 : 4 * (size_t)C + 16;
    const char* pp = (const char*)a.ws + ((size_t)gq * a.nh + head) * S * pstride;
    const int d0 = 64 * CPL * sub + CPL * lane;
    const bool dv = d0 < C;
    // a batch of CB splits from split s0: (max, sum) and this lane's channels
    float2 ml[CB];
    uint32_t ov[CB][W];
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int sb = 0; sb < CB; ++sb) {
            const char* src = pp + (size_t)min(s0 + sb, S - 1) * pstride;
            ml[sb] = *(const float2*)src;
            const char* cp = src + 16 + (BF ? 2 : 4) * (size_t)d0;
            if constexpr (W == 2) {
                const uint2 u = dv ? *(const uint2*)cp : make_uint2(0u, 0u);
                ov[sb][0] = u.x;
                ov[sb][1] = u.y;
            } else {
#pragma unroll
                for (int h = 0; h < W / 4; ++h) {
                    const uint4 u = dv ? *(const uint4*)(cp + 16 * h) : make_uint4(0u, 0u, 0u, 0u);
                    ov[sb][4 * h] = u.x;
                    ov[sb][4 * h + 1] = u.y;
                    ov[sb][4 * h + 2] = u.z;
                    ov[sb][4 * h + 3] = u.w;
                }
            }
        }
    };
    load_batch(0);
    const float zs = a.sinks[head] * LOG2E;
    // the common reference max (with the sink): the first batch's maxima,
    // then those of any further splits
    float M = zs;
#pragma unroll
    for (int sb = 0; sb < CB; ++sb)
        if (sb < S) M = fmaxf(M, ml[sb].x);
    for (int s0 = CB; s0 < S; s0 += CB) {                       // further maxima, CB loads at a time
        float mb[CB];
#pragma unroll
        for (int sb = 0; sb < CB; ++sb) mb[sb] = *(const float*)(pp + (size_t)min(s0 + sb, S - 1) * pstride);
#pragma unroll
        for (int sb = 0; sb < CB; ++sb) M = fmaxf(M, mb[sb]);
    }
    // the denominator and the weighted sum of the partial outputs, in split order
    float L = 0.f;
    float o[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) o[i] = 0.f;
    auto accum = [&](float2 msl, const uint32_t (&u)[W]) {
        // msl.x - M <= 0: the hardware exp2 (a weight below 2^-126 flushes to 0)
        const float w = msl.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(msl.x - M);
        if (w == 0.f) return;                                  // empty splits add nothing, not even +0
        L += msl.y * w;
        float v[CPL];
        if constexpr (BF) {
#pragma unroll
            for (int i = 0; i < W; ++i) {
                v[2 * i] = bf16_to_f32(u[i] & 0xFFFF);
                v[2 * i + 1] = bf16_to_f32(u[i] >> 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) v[i] = __uint_as_float(u[i]);
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) o[i] += v[i] * w;
    };
#pragma unroll
    for (int sb = 0; sb < CB; ++sb)
        if (sb < S) accum(ml[sb], ov[sb]);
    for (int s0 = CB; s0 < S; s0 += CB) {
        load_batch(s0);
#pragma unroll
        for (int sb = 0; sb < CB; ++sb)
            if (s0 + sb < S) accum(ml[sb], ov[sb]);
    }
    if (!dv) return;
    const float inv = 1.0f / (exp2f(zs - M) + L);
#pragma unroll
    for (int i = 0; i < CPL; ++i) o[i] *= inv;
    // channel pairs (d, d+1) of the RoPE part: nf is even, so pairs never
    // straddle a lane's channels or the RoPE boundary
    if (d0 + CPL > nf) {
        int req, tok;
        if (a.one_per_req) {
            req = gq;
            tok = 0;
        } else {
            req = find_request(a.cu_new, a.n_req, gq);
            tok = gq - a.cu_new[req];
        }
        const int t = a.start_pos[req] + tok;
#pragma unroll
        for (int q = 0; q < CPL / 2; ++q) {
            const int d = d0 + 2 * q;
            if (d >= nf) {
                float cs, sn;
                rope_cs_f((double)t, a.inv_freq[(d - nf) >> 1], &cs, &sn);
                const float u0 = o[2 * q], u1 = o[2 * q + 1];
                o[2 * q] = u0 * cs + u1 * sn;
                o[2 * q + 1] = -u0 * sn + u1 * cs;
            }
        }
    }
    const size_t ob = ((size_t)gq * a.nh + head) * C + d0;
    if constexpr (BF) {
        uint32_t pk[CPL / 2];
#pragma unroll
        for (int i = 0; i < CPL / 2; ++i) pk[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
        if constexpr (CPL == 8) *(uint4*)((uint16_t*)a.out + ob) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        else *(uint2*)((uint16_t*)a.out + ob) = make_uint2(pk[0], pk[1]);
    } else {
#pragma unroll
        for (int i = 0; i < CPL / 4; ++i)
            *(float4*)((float*)a.out + ob + 4 * i) = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
}

// Head tiles per workgroup: 4 (64 heads) when there are that many heads,
// else 1 (16 heads).
static int head_tiles(int n_heads) { return n_heads >= 64 ? 4 : 1; }

// Splits per query: as many as fit one workgroup per compute unit (256 in
// all), each split at least two tiles long, at most 256 splits.  Measured
// (attention + combine, split counts swept): 16 x 128K CSA queries 22.9 us
// at 10 splits (24.4 at 7, 34.1 at 20); 4 x 1M CSA 25.9 at 18 (27.2 at 12);
// 4 x 1M HCA 51.0 at 29 (71.2 at 16, 73.7 at 40: a second round of
// workgroups).
int attention_splits(int n_tokens, int n_heads, int rows_max)
{
    const int ht = head_tiles(n_heads);
    const int hg = (n_heads + 16 * ht - 1) / (16 * ht);
    const int tiles = (rows_max + 31) / 32;
    const long base = (long)n_tokens * hg;
    const long fit = 256 / (base > 0 ? base : 1);
    return (int)max(1L, min(min((long)tiles / 2, fit), 256L));
}

// Splits of a batch-invariant layer: fixed boundaries every
// CSA_INVARIANT_SPLIT_ROWS rows of a query.
static int invariant_splits(int rows_max)
{
    return max(1, (rows_max + CSA_INVARIANT_SPLIT_ROWS - 1) / CSA_INVARIANT_SPLIT_ROWS);
}

// Bytes of split partials (fp32 layout, the larger of the two).
size_t attention_workspace(int n_tokens, int n_heads, int c, int rows_max, bool invariant)
{
    const int s = invariant ? invariant_splits(rows_max) : attention_splits(n_tokens, n_heads, rows_max);
    if (s <= 1 && !invariant) return 0;
    return (size_t)n_tokens * n_heads * s * (4 * (size_t)c + 16);
}

// (c, rope) shapes: (128, 32), (256, 64), (512, 64); fp32 KV up to c = 256
template <int KVF, int HT>
static void launch_c(hipStream_t st, const AttnArgs& a, dim3 grid)
{
    switch (a.c) {
    case 128: attn_kernel<KVF, 128, 32, HT><<<grid, AttnCfg<KVF, 128, 32, HT>::NT, 0, st>>>(a); break;
    case 256: attn_kernel<KVF, 256, 64, HT><<<grid, AttnCfg<KVF, 256, 64, HT>::NT, 0, st>>>(a); break;
    case 512:
        if constexpr (KVF != 0) attn_kernel<KVF, 512, 64, HT><<<grid, AttnCfg<KVF, 512, 64, HT>::NT, 0, st>>>(a);
        break;
    default: break;
    }
}

template <int HT>
static void launch_ht(hipStream_t st, const AttnArgs& a, dim3 grid)
{
    if (a.kv_fmt == 0) launch_c<0, HT>(st, a, grid);
    else if (a.kv_fmt == 1) launch_c<1, HT>(st, a, grid);
    else launch_c<2, HT>(st, a, grid);
}

hipError_t launch_attention(hipStream_t st, AttnArgs a)
{
    if (a.n_tokens <= 0) return hipSuccess;
    const int ht = head_tiles(a.nh);
    const int hg = (a.nh + 16 * ht - 1) / (16 * ht);
    const int tiles = (a.rows_max + 31) / 32;
    if (a.invariant) {                       // the same boundaries in every batch
        a.tiles_per_split = CSA_INVARIANT_SPLIT_ROWS / 32;
        a.n_splits = invariant_splits(a.rows_max);
    } else {
        a.n_splits = attention_splits(a.n_tokens, a.nh, a.rows_max);
        a.tiles_per_split = (tiles + a.n_splits - 1) / a.n_splits;
        // no split left without tiles (20 tiles over 8 splits of 3: seven),
        // so no workgroup writes and no combine reads an empty partial
        a.n_splits = (tiles + a.tiles_per_split - 1) / a.tiles_per_split;
    }
    for (int j = 0; j < a.r / 2 && j < 32; ++j) a.inv_freq[j] = rope_inv_freq(j, a.r, (double)a.theta);
    const dim3 grid(a.n_tokens, hg, a.n_splits);
    if (ht == 4 && a.kv_fmt == 2 && a.c == 512 && a.r == 64 && a.q_bf16 && a.win_bf16)
        attn_ht_kernel<512, 64, 4><<<grid, 512, 0, st>>>(a);     // FP8 serving shapes: two waves per head tile
    else if (ht == 4) launch_ht<4>(st, a, grid);
    else launch_ht<1>(st, a, grid);
    if (a.n_splits > 1 || a.invariant) {
        // 512 channels: two waves per (query, head) (128K: 22.0 -> 21.4 us,
        // 1M CSA 24.3 -> 23.0, 1M HCA 47.3 -> 45.5, attention + combine)
        const dim3 cg(a.n_tokens, (a.nh + 3) / 4), cg2(a.n_tokens, (a.nh + 1) / 2);
        if (a.c == 512) {
            if (a.out_bf16 && a.n_splits > 16) attn_combine_kernel<true, 32, 2><<<cg2, 256, 0, st>>>(a);
            else if (a.out_bf16) attn_combine_kernel<true, 16, 2><<<cg2, 256, 0, st>>>(a);
            else attn_combine_kernel<false, 16, 2><<<cg2, 256, 0, st>>>(a);
        } else if (a.out_bf16 && a.n_splits > 16) attn_combine_kernel<true, 32, 1><<<cg, 256, 0, st>>>(a);
        else if (a.out_bf16) attn_combine_kernel<true, 16, 1><<<cg, 256, 0, st>>>(a);
        else attn_combine_kernel<false, 16, 1><<<cg, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace csa
