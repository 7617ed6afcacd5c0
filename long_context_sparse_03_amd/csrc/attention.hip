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
// Work split: a workgroup owns one query, 16*NW heads (one wave per 16 heads)
// and a contiguous range of 32-row KV tiles (a split).  Rows are the query's
// selected entries (sparse) or all visible entries (dense), then its window.
// Each tile is gathered once into LDS for all heads of the workgroup:
//   Kt [32][C]  row-major (A operand of S^T = K . Q^T),
//   Vt [C][32]  transposed (A operand of O^T = V^T . P^T),
// with FP8 codes expanded exactly to bf16 and the per-row block scale applied
// to the fp32 logits (FP8 channels) and folded into P (FP8 value channels).
// The 32 tile rows are ordered so that each lane's S^T accumulator holds 8
// consecutive rows, which are exactly the rows its P^T fragment needs.
// Online softmax in base 2 with the running max per head; splits write
// (max, sum, O) partials that a combine kernel merges in split order, so the
// output does not depend on scheduling.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr float LOG2E = 1.4426950408889634f;

template <int KVF, int C, int R>
struct AttnCfg {
    static constexpr int NF = C - R;                                     // non-rotary channels
    static constexpr bool F32 = KVF == 0;
    using MMA = typename std::conditional<F32, MmaF32, MmaBF16>::type;
    using ET = typename std::conditional<F32, float, uint16_t>::type;   // LDS element type
    static constexpr int EPF = 16 / sizeof(ET);                          // elements per fragment
    static constexpr int KP = C + (F32 ? 4 : 8);                         // Kt row stride (elements)
    static constexpr int VP = 32 + (F32 ? 4 : 8);                        // Vt row stride (elements)
    static constexpr int QSTEPS = C / MMA::K;                            // fragments of a query head
    static constexpr int DT = C / 16;                                    // 16-dim tiles of the output
    // bf16 KV with fp32 accumulation: the normalised query and the softmax
    // weights enter the bf16 MFMAs as hi + lo bf16 pairs (about 16
    // significant bits) instead of one rounded bf16 value
    static constexpr bool SPLIT = KVF == 1 && C <= 256;
    static constexpr int QPARTS = SPLIT ? 2 : 1;
};

template <int KVF, int C, int R>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a)
{
    using Cfg = AttnCfg<KVF, C, R>;
    using MMA = typename Cfg::MMA;
    using ET = typename Cfg::ET;
    constexpr int EPF = Cfg::EPF, KP = Cfg::KP, VP = Cfg::VP;
    constexpr int DESC = 256;                                  // rows described at a time

    __shared__ __attribute__((aligned(16))) ET Kt[32 * KP];
    __shared__ __attribute__((aligned(16))) ET Vt[C * VP];
    __shared__ const char* rptr[DESC];                         // row start (null: masked row)
    __shared__ float rscl[DESC];                               // fp8 block scale (1 otherwise)
    __shared__ float rcs[256], rsn[256];
    __shared__ float qg[C];
    __shared__ uint4 qf[4][Cfg::QPARTS][Cfg::QSTEPS][64];      // query fragments per wave, fragment order

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int nthr = blockDim.x;
    const int NW = nthr >> 6;
    const int gq = blockIdx.x;
    const int head = (blockIdx.y * NW + wave) * 16 + li;
    const bool hv = head < a.nh;
    const int split = blockIdx.z;
    __shared__ int cu_sh[1025];
    const int req = find_request_block(a.cu_new, a.n_req, gq, cu_sh);
    const int t = a.start_pos[req] + (gq - cu_sh[req]);
    constexpr int nf = Cfg::NF;                               // non-rotary channels
    const bool dense = a.sel == nullptr;
    const int V = (t + 1) / a.m;
    const int K0 = dense ? V : a.k;                            // entry slots before the window
    const int nwr = min(a.n_win, t + 1);
    const int w0 = t - nwr + 1;
    const int n_slots = K0 + a.n_win;
    const int n_tiles = (n_slots + 31) / 32;
    const int tile0 = split * a.tiles_per_split;
    const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);

    // RoPE table at +t and the query norm gains
    for (int j = threadIdx.x; j < R / 2; j += nthr) rope_cs((double)t, j, R, a.theta, &rcs[j], &rsn[j]);
    for (int j = threadIdx.x; j < C; j += nthr) qg[j] = a.q_gamma[j];

    // query fragments (B operand of S^T): head li, channels s*K + g*EPF + j.
    // One load per fragment; the RMS of the head is summed over the four lane
    // groups that hold it.
    {
        uint4 QB[Cfg::QSTEPS];
        const char* qp = (const char*)a.q + ((size_t)gq * a.nh + (hv ? head : 0)) * C * sizeof(ET);
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < Cfg::QSTEPS; ++s) {
            QB[s] = *(const uint4*)(qp + (size_t)(s * MMA::K + g * EPF) * sizeof(ET));
            const uint32_t w4[4] = {QB[s].x, QB[s].y, QB[s].z, QB[s].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if constexpr (Cfg::F32) {
                    float x = __uint_as_float(w4[h]);
                    ss += x * x;
                } else {
                    float x0 = bf16_to_f32(w4[h] & 0xFFFF), x1 = bf16_to_f32(w4[h] >> 16);
                    ss += x0 * x0 + x1 * x1;
                }
            }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float inv = hv ? 1.0f / sqrtf(ss / (float)C + a.eps) : 0.f;
        __syncthreads();                                       // RoPE table and gains ready
#pragma unroll
        for (int s = 0; s < Cfg::QSTEPS; ++s) {
            const int d0 = s * MMA::K + g * EPF;
            const uint32_t w4[4] = {QB[s].x, QB[s].y, QB[s].z, QB[s].w};
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
            for (int j = 0; j < EPF; ++j) x[j] = qg[d0 + j] * (x[j] * inv);
            if (d0 >= nf) {
#pragma unroll
                for (int j = 0; j < EPF; j += 2) {
                    const int p = (d0 + j - nf) >> 1;
                    float u0 = x[j], u1 = x[j + 1];
                    x[j] = u0 * rcs[p] - u1 * rsn[p];
                    x[j + 1] = u0 * rsn[p] + u1 * rcs[p];
                }
            }
            if constexpr (Cfg::F32) {
                QB[s] = make_uint4(__float_as_uint(x[0] * a.scale_log2), __float_as_uint(x[1] * a.scale_log2),
                                   __float_as_uint(x[2] * a.scale_log2), __float_as_uint(x[3] * a.scale_log2));
            } else {
                uint32_t w[4], wl[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float v0 = x[2 * h] * a.scale_log2, v1 = x[2 * h + 1] * a.scale_log2;
                    w[h] = pack_bf16x2(v0, v1);
                    wl[h] = pack_bf16x2(v0 - bf16_to_f32(w[h] & 0xFFFF), v1 - bf16_to_f32(w[h] >> 16));
                }
                QB[s] = make_uint4(w[0], w[1], w[2], w[3]);
                if constexpr (Cfg::SPLIT) qf[wave][Cfg::QPARTS - 1][s][lane] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
            }
            qf[wave][0][s][lane] = QB[s];
        }
    }

    f32x4_t O[Cfg::DT];
#pragma unroll
    for (int i = 0; i < Cfg::DT; ++i) O[i] = zero4();
    float m_run = -INFINITY, l_run = 0.f;

    const size_t win_es = a.win_bf16 ? 2 : 4;
    const size_t rec = KVF == 2 ? (size_t)(nf + 2 * R) : (size_t)C * (KVF == 0 ? 4 : 2);
    const size_t hdr = KVF == 2 ? 64 : 0;
    const char* ring = (const char*)a.state + (size_t)req * a.state_stride;
    constexpr int CH = C / 8;                                  // 8-channel chunks per row

    // ---- row descriptors: source pointer and scale of DESC consecutive slots
    auto describe = [&](int first_slot) {
        for (int j = threadIdx.x; j < DESC; j += nthr) {
            const int slot = first_slot + j;
            const char* p = nullptr;
            float sc = 1.0f;
            if (slot < K0) {
                const int e = dense ? slot : a.sel[(size_t)gq * a.k + slot];
                if (e >= 0 && e < V) {
                    const int phys = a.block_table[(size_t)req * a.max_blocks + (e >> a.epb_log2)];
                    const char* blk = (const char*)a.kv + (size_t)phys * a.kv_block_bytes;
                    p = blk + hdr + (size_t)(e & (a.epb - 1)) * rec;
                    if (KVF == 2) sc = *(const float*)blk;
                }
            } else if (slot < n_slots && slot - K0 < nwr) {
                p = ring + (size_t)((w0 + slot - K0) % a.win_cap) * C * win_es;
            }
            rptr[j] = p;
            rscl[j] = sc;
        }
    };
    // ---- gather: loads of one round (PF items per thread) of a tile, then
    //      conversion into Kt (row-major) and Vt (transposed)
    constexpr int PF = 4;                                      // items per thread per round
    constexpr int NV = Cfg::F32 ? 2 : 1;                       // 16-byte loads per item
    const int items = 32 * CH;
    const int rounds = (items + PF * nthr - 1) / (PF * nthr);
    // Loads are branch-free so that a round's loads stay in flight together:
    // masked rows read a valid dummy address and are zeroed afterwards; an
    // FP8 channel chunk is 8 bytes, every other chunk 16 (two 8-byte halves).
    const char* dummy = (const char*)a.kv;
    auto load_round = [&](int r, int tile, int drow0, uint4 (&raw)[PF][NV]) {
        const int slot0 = tile * 32;
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int idx = threadIdx.x + (r * PF + u) * nthr;
            const int row = idx & 31, d0 = (idx >> 5) * 8;      // rows fastest: Vt writes spread over banks
            const char* p = idx < items ? rptr[drow0 + row] : nullptr;
            const bool ok = p != nullptr;
            const char* base = ok ? p : dummy;
            if constexpr (KVF == 2) {
                const bool entry = slot0 + row < K0;
                const char* a0 = entry ? (d0 < nf ? base + d0 : base + nf + 2 * (size_t)(d0 - nf)) : base + 2 * (size_t)d0;
                const char* a1 = (entry && d0 < nf) ? a0 : a0 + 8;
                const uint2 lo = *(const uint2*)a0, hi = *(const uint2*)a1;
                raw[u][0] = sel16(ok, make_uint4(lo.x, lo.y, hi.x, hi.y));
            } else if constexpr (KVF == 1) {
                raw[u][0] = sel16(ok, ld16(base + 2 * (size_t)d0));
            } else {
                raw[u][0] = sel16(ok, ld16(base + 4 * (size_t)d0));
                raw[u][NV - 1] = sel16(ok, ld16(base + 4 * (size_t)d0 + 16));
            }
        }
    };
    auto store_round = [&](int r, int tile, uint4 (&raw)[PF][NV]) {
        const int slot0 = tile * 32;
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int idx = threadIdx.x + (r * PF + u) * nthr;
            if (idx >= items) break;
            const int row = idx & 31, d0 = (idx >> 5) * 8;      // rows fastest: Vt writes spread over banks
            const bool entry = slot0 + row < K0;
            ET* kr = Kt + row * KP + d0;
            if constexpr (Cfg::F32) {
                *(uint4*)kr = raw[u][0];
                *(uint4*)(kr + 4) = raw[u][NV - 1];
                const float* v = (const float*)&raw[u][0];
                const float* v2 = (const float*)&raw[u][NV - 1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Vt[(d0 + j) * VP + row] = v[j];
                    Vt[(d0 + 4 + j) * VP + row] = v2[j];
                }
            } else {
                uint4 b;
                if (KVF == 2 && entry && d0 < nf) {
                    const uint2 b0 = e4m3x4_to_bf16x4(raw[u][0].x), b1 = e4m3x4_to_bf16x4(raw[u][0].y);
                    b = make_uint4(b0.x, b0.y, b1.x, b1.y);
                } else {
                    b = raw[u][0];
                }
                *(uint4*)kr = b;
                const uint32_t w4[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    Vt[(d0 + 2 * h) * VP + row] = (uint16_t)(w4[h] & 0xFFFF);
                    Vt[(d0 + 2 * h + 1) * VP + row] = (uint16_t)(w4[h] >> 16);
                }
            }
        }
    };

    uint4 raw[PF][NV];
    if (tile0 < tile1) {
        describe(tile0 * 32);
        __syncthreads();
        load_round(0, tile0, 0, raw);
    }
    for (int tile = tile0; tile < tile1; ++tile) {
        const int drow0 = ((tile - tile0) * 32) % DESC;
        const int slot0 = tile * 32;
        store_round(0, tile, raw);
        for (int r = 1; r < rounds; ++r) {
            uint4 more[PF][NV];
            load_round(r, tile, drow0, more);
            store_round(r, tile, more);
        }
        __syncthreads();
        // prefetch the next tile's first round while this one computes
        const bool next_same_window = tile + 1 < tile1 && drow0 + 32 < DESC;
        if (next_same_window) load_round(0, tile + 1, drow0 + 32, raw);

        // ---- S^T = K . Q^T for 32 rows x 16 heads (two 16-row tiles)
        // tile rt, MFMA row r' -> tile row 8*(r'/4) + 4*rt + r'%4
        const int ra = 8 * (li >> 2) + (li & 3);
        const int rb = ra + 4;
        f32x4_t sn0 = zero4(), sn1 = zero4(), sr0 = zero4(), sr1 = zero4();
#pragma unroll
        for (int s = 0; s < Cfg::QSTEPS; ++s) {
            const int d0 = s * MMA::K + g * EPF;
            uint4 ka = *(const uint4*)(Kt + ra * KP + d0);
            uint4 kb = *(const uint4*)(Kt + rb * KP + d0);
#pragma unroll
            for (int part = 0; part < Cfg::QPARTS; ++part) {
                const uint4 qb = qf[wave][part][s][lane];
                if (KVF == 2 && s * MMA::K < nf) {
                    sn0 = MMA::step(ka, qb, sn0);
                    sn1 = MMA::step(kb, qb, sn1);
                } else {
                    sr0 = MMA::step(ka, qb, sr0);
                    sr1 = MMA::step(kb, qb, sr1);
                }
            }
        }
        // lane holds rows 8g + i (i < 4 from tile 0, 4..7 from tile 1) of head li
        float sv[8], rsc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r0 = 8 * g + i, r1 = 8 * g + 4 + i;
            const bool v0 = rptr[drow0 + r0] != nullptr, v1 = rptr[drow0 + r1] != nullptr;
            const bool e0 = slot0 + r0 < K0, e1 = slot0 + r1 < K0;
            rsc[i] = rscl[drow0 + r0];
            rsc[4 + i] = rscl[drow0 + r1];
            sv[i] = v0 ? (KVF == 2 && e0 ? rsc[i] * sn0[i] + sr0[i] : sn0[i] + sr0[i]) : -INFINITY;
            sv[4 + i] = v1 ? (KVF == 2 && e1 ? rsc[4 + i] * sn1[i] + sr1[i] : sn1[i] + sr1[i]) : -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // The reference max only moves when a logit exceeds it by more than
        // 2^8 (base-2 units), so weights stay <= 256 and the accumulators are
        // rescaled rarely; the final normalisation uses the same reference.
        const bool raise = mx > m_run + 8.0f;
        const float m_new = raise ? mx : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = raise ? exp2f(m_run - m_use) : 1.0f;
        float p[8], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) { p[i] = exp2f(sv[i] - m_use); ps += p[i]; }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if (__any(raise)) {
#pragma unroll
            for (int i = 0; i < Cfg::DT; ++i) O[i] *= alpha;
        }

        // ---- O^T += V^T . P^T
        if constexpr (Cfg::F32) {
            uint4 pa = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3]));
            uint4 pb = make_uint4(__float_as_uint(p[4]), __float_as_uint(p[5]), __float_as_uint(p[6]), __float_as_uint(p[7]));
#pragma unroll
            for (int dt = 0; dt < Cfg::DT; ++dt) {
                const ET* vr = Vt + (dt * 16 + li) * VP + 8 * g;
                O[dt] = MMA::step(*(const uint4*)vr, pa, O[dt]);
                O[dt] = MMA::step(*(const uint4*)(vr + 4), pb, O[dt]);
            }
        } else {
            // FP8 value channels of entry rows carry the block scale; window rows do not
            float ps8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) ps8[i] = (KVF == 2 && slot0 + 8 * g + i < K0) ? p[i] * rsc[i] : p[i];
            const uint4 pr = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                        pack_bf16x2(p[6], p[7]));
            const uint4 pn = make_uint4(pack_bf16x2(ps8[0], ps8[1]), pack_bf16x2(ps8[2], ps8[3]),
                                        pack_bf16x2(ps8[4], ps8[5]), pack_bf16x2(ps8[6], ps8[7]));
            uint4 pl = pr;
            if constexpr (Cfg::SPLIT) {
                const uint32_t h4[4] = {pr.x, pr.y, pr.z, pr.w};
                uint32_t l4[4];
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    l4[h] = pack_bf16x2(p[2 * h] - bf16_to_f32(h4[h] & 0xFFFF), p[2 * h + 1] - bf16_to_f32(h4[h] >> 16));
                pl = make_uint4(l4[0], l4[1], l4[2], l4[3]);
            }
#pragma unroll
            for (int dt = 0; dt < Cfg::DT; ++dt) {
                const ET* vr = Vt + (dt * 16 + li) * VP + 8 * g;
                const uint4 va = *(const uint4*)vr;
                O[dt] = MMA::step(va, (KVF == 2 && dt * 16 < nf) ? pn : pr, O[dt]);
                if constexpr (Cfg::SPLIT) O[dt] = MMA::step(va, pl, O[dt]);
            }
        }
        __syncthreads();                                       // Kt, Vt and rptr are rewritten next
        if (tile + 1 < tile1 && !next_same_window) {
            describe((tile + 1) * 32);
            __syncthreads();
            load_round(0, tile + 1, 0, raw);
        }
    }

    // lane holds O^T[16*dt + 4g + i][head li]
    if (a.n_splits == 1) {
        const float zs = (hv ? a.sinks[head] : 0.f) * LOG2E;
        const float M = fmaxf(m_run, zs);
        const float sc = exp2f(m_run - M);
        const float inv = sc / (l_run * sc + exp2f(zs - M));
        if (hv) {
#pragma unroll
            for (int dt = 0; dt < Cfg::DT; ++dt) {
                const int d = dt * 16 + 4 * g;
                float o[4] = {O[dt][0] * inv, O[dt][1] * inv, O[dt][2] * inv, O[dt][3] * inv};
                if (d >= nf) {
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {       // rotate back at -t
                        const int pj = (d + j - nf) >> 1;
                        float u0 = o[j], u1 = o[j + 1];
                        o[j] = u0 * rcs[pj] + u1 * rsn[pj];
                        o[j + 1] = -u0 * rsn[pj] + u1 * rcs[pj];
                    }
                }
                if (a.out_bf16) {
                    uint2 w = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                    *(uint2*)((uint16_t*)a.out + ((size_t)gq * a.nh + head) * C + d) = w;
                } else {
                    *(float4*)((float*)a.out + ((size_t)gq * a.nh + head) * C + d) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    } else if (hv) {
        float* pp = a.ws + (((size_t)gq * a.nh + head) * a.n_splits + split) * (C + 2);
        if (g == 0) { pp[0] = m_run; pp[1] = l_run; }
#pragma unroll
        for (int dt = 0; dt < Cfg::DT; ++dt) {
            const int d = dt * 16 + 4 * g;
            *(float4*)(pp + 2 + d) = make_float4(O[dt][0], O[dt][1], O[dt][2], O[dt][3]);
        }
    }
}

// Merge the split partials of one (query, head) in split order, add the sink,
// normalise, rotate back at -t and store.
__global__ __launch_bounds__(512) void attn_combine_kernel(AttnArgs a)
{
    __shared__ float o_sh[512];
    const int gq = blockIdx.x, head = blockIdx.y;
    const int C = a.c;
    const int req = find_request(a.cu_new, a.n_req, gq);
    const int t = a.start_pos[req] + (gq - a.cu_new[req]);
    const float* pp = a.ws + ((size_t)gq * a.nh + head) * a.n_splits * (C + 2);
    const float zs = a.sinks[head] * LOG2E;
    float M = zs;
    for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, pp[(size_t)s * (C + 2)]);
    float L = exp2f(zs - M);
    for (int s = 0; s < a.n_splits; ++s) L += pp[(size_t)s * (C + 2) + 1] * exp2f(pp[(size_t)s * (C + 2)] - M);
    const float inv = 1.0f / L;
    for (int d = threadIdx.x; d < C; d += blockDim.x) {
        float o = 0.f;
        for (int s = 0; s < a.n_splits; ++s) o += pp[(size_t)s * (C + 2) + 2 + d] * exp2f(pp[(size_t)s * (C + 2)] - M);
        o_sh[d] = o * inv;
    }
    __syncthreads();
    const int nf = C - a.r;
    for (int d = threadIdx.x; d < C; d += blockDim.x) {
        float o = o_sh[d];
        if (d >= nf) {
            const int pj = (d - nf) >> 1;
            float cs, sn;
            rope_cs((double)t, pj, a.r, a.theta, &cs, &sn);
            const float u0 = o_sh[nf + 2 * pj], u1 = o_sh[nf + 2 * pj + 1];
            o = ((d - nf) & 1) ? (-u0 * sn + u1 * cs) : (u0 * cs + u1 * sn);
        }
        if (a.out_bf16) ((uint16_t*)a.out)[((size_t)gq * a.nh + head) * C + d] = f32_to_bf16(o);
        else ((float*)a.out)[((size_t)gq * a.nh + head) * C + d] = o;
    }
}

int attention_splits(int n_tokens, int n_heads, int rows_max)
{
    const int nw = n_heads >= 64 ? 4 : (n_heads + 15) / 16;
    const int hg = (n_heads + 16 * nw - 1) / (16 * nw);
    const int tiles = (rows_max + 31) / 32;
    const long base = (long)n_tokens * hg;
    int splits = 1;
    while (base * splits < 512 && splits * 2 <= tiles / 2) splits *= 2;
    return splits;
}

size_t attention_workspace(int n_tokens, int n_heads, int c, int rows_max)
{
    const int s = attention_splits(n_tokens, n_heads, rows_max);
    if (s <= 1) return 0;
    return (size_t)n_tokens * n_heads * s * (c + 2) * sizeof(float);
}

// (c, rope) shapes: (128, 32), (256, 64), (512, 64); fp32 KV up to c = 256
template <int KVF>
static void launch_c(hipStream_t st, const AttnArgs& a, dim3 grid, int threads)
{
    switch (a.c) {
    case 128: attn_kernel<KVF, 128, 32><<<grid, threads, 0, st>>>(a); break;
    case 256: attn_kernel<KVF, 256, 64><<<grid, threads, 0, st>>>(a); break;
    case 512:
        if constexpr (KVF != 0) attn_kernel<KVF, 512, 64><<<grid, threads, 0, st>>>(a);
        break;
    default: break;
    }
}

hipError_t launch_attention(hipStream_t st, AttnArgs a)
{
    if (a.n_tokens <= 0) return hipSuccess;
    const int nw = a.nh >= 64 ? 4 : (a.nh + 15) / 16;
    const int hg = (a.nh + 16 * nw - 1) / (16 * nw);
    const int tiles = (a.rows_max + 31) / 32;
    a.n_splits = attention_splits(a.n_tokens, a.nh, a.rows_max);
    a.tiles_per_split = (tiles + a.n_splits - 1) / a.n_splits;
    dim3 grid(a.n_tokens, hg, a.n_splits);
    if (a.kv_fmt == 0) launch_c<0>(st, a, grid, 64 * nw);
    else if (a.kv_fmt == 1) launch_c<1>(st, a, grid, 64 * nw);
    else launch_c<2>(st, a, grid, 64 * nw);
    if (a.n_splits > 1) attn_combine_kernel<<<dim3(a.n_tokens, a.nh), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace csa
