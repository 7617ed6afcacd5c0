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

template <int KVF, int C>
struct AttnCfg {
    static constexpr bool F32 = KVF == 0;
    using MMA = typename std::conditional<F32, MmaF32, MmaBF16>::type;
    using ET = typename std::conditional<F32, float, uint16_t>::type;   // LDS element type
    static constexpr int EPF = 16 / sizeof(ET);                          // elements per fragment
    static constexpr int KP = C + 16 / sizeof(ET) * (F32 ? 1 : 1);      // Kt row stride (elements)
    static constexpr int VP = 32 + (F32 ? 4 : 8);                        // Vt row stride (elements)
    static constexpr int QSTEPS = C / MMA::K;                            // fragments of a query head
    static constexpr int DT = C / 16;                                    // 16-dim tiles of the output
};

template <int KVF, int C>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a)
{
    using Cfg = AttnCfg<KVF, C>;
    using MMA = typename Cfg::MMA;
    using ET = typename Cfg::ET;
    constexpr int EPF = Cfg::EPF, KP = Cfg::KP, VP = Cfg::VP;

    __shared__ __attribute__((aligned(16))) ET Kt[32 * KP];
    __shared__ __attribute__((aligned(16))) ET Vt[C * VP];
    __shared__ float rscale[32];
    __shared__ int rvalid[32];
    __shared__ float rcs[256], rsn[256];
    __shared__ float inv_rms[4][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int nthr = blockDim.x;
    const int gq = blockIdx.x;
    const int NW = nthr >> 6;
    const int head = (blockIdx.y * NW + wave) * 16 + li;
    const int split = blockIdx.z;
    const int req = find_request(a.cu_new, a.n_req, gq);
    const int t = a.start_pos[req] + (gq - a.cu_new[req]);
    const int nf = C - a.r;                                   // non-rotary channels
    const bool dense = a.sel == nullptr;
    const int V = (t + 1) / a.m;
    const int K0 = dense ? V : a.k;                            // entry slots before the window
    const int nwr = min(a.n_win, t + 1);
    const int w0 = t - nwr + 1;
    const int n_slots = K0 + a.n_win;
    const int n_tiles = (n_slots + 31) / 32;
    const int tile0 = split * a.tiles_per_split;
    const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);

    // RoPE table at +t
    for (int j = threadIdx.x; j < a.r / 2; j += nthr) rope_cs((double)t, j, a.r, a.theta, &rcs[j], &rsn[j]);

    // per-head RMS of the raw query
    const size_t qes = a.q_bf16 ? 2 : 4;
    for (int hh = 0; hh < 16; ++hh) {
        const int hd = (blockIdx.y * NW + wave) * 16 + hh;
        float ss = 0.f;
        if (hd < a.nh) {
            const char* qp = (const char*)a.q + ((size_t)gq * a.nh + hd) * C * qes;
            for (int d = lane; d < C; d += 64) {
                float x = a.q_bf16 ? bf16_to_f32(((const uint16_t*)qp)[d]) : ((const float*)qp)[d];
                ss += x * x;
            }
        }
        ss = wave_sum(ss);
        if (lane == 0) inv_rms[wave][hh] = 1.0f / sqrtf(ss / (float)C + a.eps);
    }
    __syncthreads();

    // query fragments (B operand of S^T): head li, channels s*K + g*EPF + j
    uint4 QB[Cfg::QSTEPS];
    {
        const float inv = inv_rms[wave][li];
        const bool hv = head < a.nh;
        const char* qp = (const char*)a.q + ((size_t)gq * a.nh + (hv ? head : 0)) * C * qes;
#pragma unroll
        for (int s = 0; s < Cfg::QSTEPS; ++s) {
            const int d0 = s * MMA::K + g * EPF;
            float x[EPF];
#pragma unroll
            for (int j = 0; j < EPF; ++j) {
                float v = a.q_bf16 ? bf16_to_f32(((const uint16_t*)qp)[d0 + j]) : ((const float*)qp)[d0 + j];
                x[j] = hv ? a.q_gamma[d0 + j] * (v * inv) : 0.f;
            }
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
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) w[h] = pack_bf16x2(x[2 * h] * a.scale_log2, x[2 * h + 1] * a.scale_log2);
                QB[s] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }

    f32x4_t O[Cfg::DT];
#pragma unroll
    for (int i = 0; i < Cfg::DT; ++i) O[i] = zero4();
    float m_run = -INFINITY, l_run = 0.f;

    const size_t win_es = a.win_bf16 ? 2 : 4;
    const size_t rec = KVF == 2 ? (size_t)(nf + 2 * a.r) : (size_t)C * (KVF == 0 ? 4 : 2);
    const size_t hdr = KVF == 2 ? 64 : 0;
    const char* ring = (const char*)a.state + (size_t)req * a.state_stride;

    for (int tile = tile0; tile < tile1; ++tile) {
        // ---- gather 32 rows into Kt (row-major), converting to the MMA type
        __syncthreads();
        for (int idx = threadIdx.x; idx < 32 * (C / 8); idx += nthr) {
            const int row = idx / (C / 8), ch = idx % (C / 8), d0 = ch * 8;
            const int slot = tile * 32 + row;
            float v[8];
            bool valid = false;
            float sc = 1.0f;
            if (slot < K0) {
                const int e = dense ? slot : a.sel[(size_t)gq * a.k + slot];
                valid = e >= 0 && e < V;
                if (valid) {
                    const int phys = a.block_table[(size_t)req * a.max_blocks + e / a.epb];
                    const char* rp = (const char*)a.kv + (size_t)phys * a.kv_block_bytes + hdr + (size_t)(e % a.epb) * rec;
                    if constexpr (KVF == 0) {
                        const float4* p = (const float4*)((const float*)rp + d0);
                        float4 x0 = p[0], x1 = p[1];
                        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
                        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
                    } else if constexpr (KVF == 1) {
                        uint4 u = *(const uint4*)((const uint16_t*)rp + d0);
                        uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                        for (int h = 0; h < 4; ++h) { v[2 * h] = bf16_to_f32(w4[h] & 0xFFFF); v[2 * h + 1] = bf16_to_f32(w4[h] >> 16); }
                    } else {
                        if (d0 < nf) {
                            uint2 u = *(const uint2*)(rp + d0);
#pragma unroll
                            for (int j = 0; j < 4; ++j) { v[j] = e4m3_to_f32((u.x >> (8 * j)) & 0xFF); v[4 + j] = e4m3_to_f32((u.y >> (8 * j)) & 0xFF); }
                        } else {
                            uint4 u = *(const uint4*)(rp + nf + 2 * (size_t)(d0 - nf));
                            uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                            for (int h = 0; h < 4; ++h) { v[2 * h] = bf16_to_f32(w4[h] & 0xFFFF); v[2 * h + 1] = bf16_to_f32(w4[h] >> 16); }
                        }
                        if (ch == 0) sc = *(const float*)((const char*)a.kv + (size_t)phys * a.kv_block_bytes);
                    }
                }
            } else {
                const int j = slot - K0;
                valid = j < nwr;
                if (valid) {
                    const int p = w0 + j;
                    const char* rp = ring + (size_t)(p % a.win_cap) * C * win_es;
                    if (a.win_bf16) {
                        uint4 u = *(const uint4*)((const uint16_t*)rp + d0);
                        uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                        for (int h = 0; h < 4; ++h) { v[2 * h] = bf16_to_f32(w4[h] & 0xFFFF); v[2 * h + 1] = bf16_to_f32(w4[h] >> 16); }
                    } else {
                        const float4* p4 = (const float4*)((const float*)rp + d0);
                        float4 x0 = p4[0], x1 = p4[1];
                        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
                        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
                    }
                }
            }
            if (!valid) {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = 0.f;
            }
            ET* kr = Kt + row * KP + d0;
            if constexpr (Cfg::F32) {
                *(float4*)kr = make_float4(v[0], v[1], v[2], v[3]);
                *(float4*)(kr + 4) = make_float4(v[4], v[5], v[6], v[7]);
            } else {
                *(uint4*)kr = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                         pack_bf16x2(v[6], v[7]));
            }
            if (ch == 0) {
                rscale[row] = sc;
                rvalid[row] = valid;
            }
        }
        __syncthreads();
        // ---- transpose into Vt (row index fastest so lanes write neighbouring rows)
        for (int idx = threadIdx.x; idx < 32 * (C / 8); idx += nthr) {
            const int row = idx & 31, d0 = (idx >> 5) * 8;
            const ET* kr = Kt + row * KP + d0;
#pragma unroll
            for (int j = 0; j < 8; ++j) Vt[(d0 + j) * VP + row] = kr[j];
        }
        __syncthreads();

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
            if (KVF == 2 && s * MMA::K < nf) {
                sn0 = MMA::step(ka, QB[s], sn0);
                sn1 = MMA::step(kb, QB[s], sn1);
            } else {
                sr0 = MMA::step(ka, QB[s], sr0);
                sr1 = MMA::step(kb, QB[s], sr1);
            }
        }
        // lane holds rows 8g + i (i < 4 from tile 0, 4..7 from tile 1) of head li
        float sv[8], rsc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r0 = 8 * g + i, r1 = 8 * g + 4 + i;
            rsc[i] = rscale[r0];
            rsc[4 + i] = rscale[r1];
            sv[i] = rvalid[r0] ? (KVF == 2 ? rsc[i] * sn0[i] + sr0[i] : sr0[i]) : -INFINITY;
            sv[4 + i] = rvalid[r1] ? (KVF == 2 ? rsc[4 + i] * sn1[i] + sr1[i] : sr1[i]) : -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float p[8], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) { p[i] = exp2f(sv[i] - m_use); ps += p[i]; }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < Cfg::DT; ++i) O[i] *= alpha;

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
            const uint4 pr = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                        pack_bf16x2(p[6], p[7]));
            uint4 pn = pr;
            if (KVF == 2)
                pn = make_uint4(pack_bf16x2(p[0] * rsc[0], p[1] * rsc[1]), pack_bf16x2(p[2] * rsc[2], p[3] * rsc[3]),
                                pack_bf16x2(p[4] * rsc[4], p[5] * rsc[5]), pack_bf16x2(p[6] * rsc[6], p[7] * rsc[7]));
#pragma unroll
            for (int dt = 0; dt < Cfg::DT; ++dt) {
                const ET* vr = Vt + (dt * 16 + li) * VP + 8 * g;
                O[dt] = MMA::step(*(const uint4*)vr, (KVF == 2 && dt * 16 < nf) ? pn : pr, O[dt]);
            }
        }
    }

    // lane holds O^T[16*dt + 4g + i][head li]
    if (a.n_splits == 1) {
        const float zs = (head < a.nh ? a.sinks[head] : 0.f) * LOG2E;
        const float M = fmaxf(m_run, zs);
        const float sc = exp2f(m_run - M);
        const float inv = sc / (l_run * sc + exp2f(zs - M));
        if (head < a.nh) {
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
    } else if (head < a.nh) {
        float* pp = a.ws + (((size_t)gq * a.nh + head) * a.n_splits + split) * (C + 2);
        if (g == 0) { pp[0] = m_run; pp[1] = l_run; }
#pragma unroll
        for (int dt = 0; dt < Cfg::DT; ++dt) {
            const int d = dt * 16 + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) pp[2 + d + i] = O[dt][i];
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

template <int KVF>
static void launch_c(hipStream_t st, const AttnArgs& a, dim3 grid, int threads)
{
    switch (a.c) {
    case 128: attn_kernel<KVF, 128><<<grid, threads, 0, st>>>(a); break;
    case 256: attn_kernel<KVF, 256><<<grid, threads, 0, st>>>(a); break;
    case 512: attn_kernel<KVF, 512><<<grid, threads, 0, st>>>(a); break;
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
