// a3: Lightning Indexer scores on gfx950.
//
// I[t][s] = sum_h w[t][h] * ReLU(q[t][h] . K[s]) over the visible entries
// s < floor((t+1)/m) ("DeepSeek-V4 内部机制" §1.2 Step 2; yunpan.plus eq. (8)),
// rounded to the score format (BF16 scores: "DeepSeek-V4 内部机制" §6.2).
//
// The contraction is an MFMA product with the indexer heads as the M
// dimension and 16 keys as N: lane l of a wave holds head (key) l%16 and a
// contiguous quarter of the key width, so a wave loads 16 keys as one
// contiguous run of a paged block.  ReLU, the head weights and the head sum
// are applied to the accumulators in registers; the sum over the four lane
// groups is a fixed butterfly, so the result is deterministic.
//
// MXFP4 keys (and the MXFP4-quantised query) are expanded to bf16 in
// registers; every E2M1 value times its power-of-two scale is exact in bf16,
// so the bf16 MFMA computes exactly the dequantised product.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

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

// Quantise 32 values (one MX block) to MXFP4 and return them dequantised as
// four bf16 fragments.
CSA_DEV void mx_quant_frags(const float* v, uint4* out)
{
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const int sc = mx_scale_code(amax);
    const float up = ldexpf(1.0f, sc - 127);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float a = e2m1_to_f32(f32_to_e2m1(ldexpf(v[8 * f + 2 * h], 127 - sc))) * up;
            float b = e2m1_to_f32(f32_to_e2m1(ldexpf(v[8 * f + 2 * h + 1], 127 - sc))) * up;
            w[h] = pack_bf16x2(a, b);
        }
        out[f] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Expand 32 stored E2M1 codes (16 bytes) with their E8M0 scale to four bf16 fragments.
CSA_DEV void mx_expand_frags(uint4 codes, uint32_t scale_code, uint4* out)
{
    const float up = ldexpf(1.0f, (int)scale_code - 127);
    uint32_t c4[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t byte = (c4[f] >> (8 * h)) & 0xFFu;
            w[h] = pack_bf16x2(e2m1_to_f32(byte & 15u) * up, e2m1_to_f32(byte >> 4) * up);
        }
        out[f] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Decode-shaped launch: one workgroup per (query, EPW entries).  Each wave
// scores 64 entries per iteration as four 16-key tiles and keeps the next
// iteration's key loads in flight while it computes the current one.
// HT = head tiles (<= 4), S = fragments per lane group.
constexpr int IDX_EPW = 1024;                 // entries per workgroup
constexpr int IDX_ITERS = IDX_EPW / 256;      // iterations of 256 entries (64 per wave)

template <int IDXF, int S>
CSA_DEV void load_keys(const IndexArgs& a, const int* bt, int blk0, int e0, int V, int g, int li, uint4 (&B)[4][S],
                       uint32_t (&SC)[4])
{
    // Loads are unconditional (entries past V are clamped to V-1): an MFMA
    // column only feeds the score of its own entry, and scores of entries
    // >= V are not stored.  Branch-free loads stay in flight together.
    const int cI = a.cI, quarter = cI / 4;
    const size_t kbytes = IDXF == 0 ? (size_t)cI * 4 : (IDXF == 1 ? (size_t)cI * 2 : (size_t)cI / 2);
#pragma unroll
    for (int tile = 0; tile < 4; ++tile) {
        const int e = min(e0 + 16 * tile + li, V - 1);
        const int phys = bt[e / a.epb - blk0];
        const int slot = e % a.epb;
        const char* kb = (const char*)a.keys + (size_t)phys * a.key_block_bytes;
        if constexpr (IDXF == 2) {
            B[tile][0] = ld16(kb + (size_t)slot * (cI / 2) + (size_t)g * 16);
            SC[tile] = (uint8_t)kb[(size_t)a.epb * (cI / 2) + (size_t)slot * (cI / 32) + g];
        } else {
            const char* kp = kb + (size_t)slot * kbytes + (size_t)g * quarter * (IDXF == 0 ? 4 : 2);
#pragma unroll
            for (int s = 0; s < S; ++s) B[tile][s] = ld16(kp + 16 * s);
        }
    }
}

template <int IDXF, int HT, int S>
__global__ __launch_bounds__(256) void index_decode_kernel(IndexArgs a)
{
    // IDXF 0: fp32 keys and queries; 1: bf16 keys and queries; 2: MXFP4 keys,
    // bf16 queries quantised to MXFP4 here.
    using MMA = typename std::conditional<IDXF == 0, MmaF32, MmaBF16>::type;
    __shared__ int bt[IDX_EPW + 1];             // physical blocks of this workgroup's entries
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int gq = blockIdx.y;
    __shared__ int cu_sh[1025];
    const int req = find_request_block(a.cu_new, a.n_req, gq, cu_sh);
    const int t = a.start_pos[req] + (gq - cu_sh[req]);
    const int V = (t + 1) / a.m;
    if (blockIdx.x == 0 && threadIdx.x == 0) a.n_valid[gq] = V;
    const int wg0 = blockIdx.x * IDX_EPW;
    if (wg0 >= V) return;
    const int cI = a.cI, nh = a.nh, quarter = cI / 4;
    constexpr int QES = IDXF == 0 ? 4 : 2;      // query element size

    // ---- prologue: block-table slice, query fragments and head weights,
    //      all loads issued together (clamped indices, masked afterwards)
    const int blk0 = wg0 / a.epb;
    const int nblk = (min(V, wg0 + IDX_EPW) - 1) / a.epb - blk0 + 1;
    int btv[(IDX_EPW + 255) / 256];
#pragma unroll
    for (int i = 0; i < (IDX_EPW + 255) / 256; ++i) {
        const int j = min((int)threadIdx.x + 256 * i, nblk - 1);
        btv[i] = a.block_table[(size_t)req * a.max_blocks + blk0 + j];
    }
    uint4 A[HT][S];
    float wv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int head = min(16 * ht + li, nh - 1);
        const char* qp = (const char*)a.q + ((size_t)gq * nh + head) * cI * QES + (size_t)g * quarter * QES;
#pragma unroll
        for (int s = 0; s < S; ++s) A[ht][s] = ld16(qp + 16 * s);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = a.w[(size_t)gq * nh + min(16 * ht + 4 * g + i, nh - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < (IDX_EPW + 255) / 256; ++i)
        if ((int)threadIdx.x + 256 * i < nblk) bt[threadIdx.x + 256 * i] = btv[i];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const bool hv = 16 * ht + li < nh;
        if constexpr (IDXF == 2) {
            float v[32];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t w4[4] = {A[ht][s].x, A[ht][s].y, A[ht][s].z, A[ht][s].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[8 * s + 2 * h] = bf16_to_f32(w4[h] & 0xFFFF);
                    v[8 * s + 2 * h + 1] = bf16_to_f32(w4[h] >> 16);
                }
            }
            mx_quant_frags(v, A[ht]);
        }
#pragma unroll
        for (int s = 0; s < S; ++s) A[ht][s] = sel16(hv, A[ht][s]);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = 16 * ht + 4 * g + i < nh ? wv[ht][i] : 0.f;
    }
    __syncthreads();

    // ---- main loop: 256 entries per iteration (64 per wave); the next
    //      iteration's key loads are issued before this one's arithmetic
    uint4 B[2][4][S];
    uint32_t SC[2][4];
    load_keys<IDXF, S>(a, bt, blk0, wg0 + wave * 64, V, g, li, B[0], SC[0]);
#pragma unroll
    for (int it = 0; it < IDX_ITERS; ++it) {
        const int cur = it & 1;
        const int e_base = wg0 + it * 256 + wave * 64;
        if (it + 1 < IDX_ITERS && e_base + 256 < V)
            load_keys<IDXF, S>(a, bt, blk0, e_base + 256, V, g, li, B[cur ^ 1], SC[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (e_base >= V) break;                  // wave-uniform
#pragma unroll
        for (int tile = 0; tile < 4; ++tile) {
            if (e_base + 16 * tile >= V) break;  // wave-uniform: the whole tile is past V
            const int e = e_base + 16 * tile + li;
            uint4 Bt[S];
            if constexpr (IDXF == 2) {
                mx_expand_frags(B[cur][tile][0], SC[cur][tile], Bt);
            } else {
#pragma unroll
                for (int s = 0; s < S; ++s) Bt[s] = B[cur][tile][s];
            }
            float v = 0.f;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                f32x4_t acc = zero4();
#pragma unroll
                for (int s = 0; s < S; ++s) acc = MMA::step(A[ht][s], Bt[s], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) v += wv[ht][i] * fmaxf(acc[i], 0.f);
            }
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (g == 0 && e < V) {
                if (v == 0.0f) v = 0.0f;                // -0 is stored as +0
                if (a.score_bf16) ((uint16_t*)a.scores)[(size_t)gq * a.ld + e] = f32_to_bf16(v);
                else ((float*)a.scores)[(size_t)gq * a.ld + e] = v;
            }
        }
    }
}

template <int IDXF, int HT>
static void launch_ht(hipStream_t st, const IndexArgs& a, dim3 grid)
{
    // fragments per lane group: quarter of the key width / elements per fragment
    const int quarter = a.cI / 4;
    const int epf = IDXF == 0 ? 4 : 8;
    const int S = quarter / epf;
    if constexpr (IDXF == 2) {             // MXFP4: one 32-element MX block per lane group (c_idx = 128)
        index_decode_kernel<IDXF, HT, 4><<<grid, 256, 0, st>>>(a);
    } else {
        switch (S) {
        case 1: index_decode_kernel<IDXF, HT, 1><<<grid, 256, 0, st>>>(a); break;
        case 2: index_decode_kernel<IDXF, HT, 2><<<grid, 256, 0, st>>>(a); break;
        case 4: index_decode_kernel<IDXF, HT, 4><<<grid, 256, 0, st>>>(a); break;
        case 8: index_decode_kernel<IDXF, HT, 8><<<grid, 256, 0, st>>>(a); break;
        default: break;
        }
    }
}

template <int IDXF>
static void launch_fmt(hipStream_t st, const IndexArgs& a, dim3 grid)
{
    const int HT = (a.nh + 15) / 16;
    switch (HT) {
    case 1: launch_ht<IDXF, 1>(st, a, grid); break;
    case 2: launch_ht<IDXF, 2>(st, a, grid); break;
    case 3: launch_ht<IDXF, 3>(st, a, grid); break;
    default: launch_ht<IDXF, 4>(st, a, grid); break;
    }
}

hipError_t launch_index(hipStream_t st, const IndexArgs& a, int max_visible, int max_new)
{
    (void)max_new;
    if (a.n_tokens <= 0) return hipSuccess;
    dim3 grid(max_visible > 0 ? (max_visible + IDX_EPW - 1) / IDX_EPW : 1, a.n_tokens);
    if (a.idx_fmt == 0) launch_fmt<0>(st, a, grid);
    else if (a.idx_fmt == 1) launch_fmt<1>(st, a, grid);
    else launch_fmt<2>(st, a, grid);
    return hipGetLastError();
}

}  // namespace csa
