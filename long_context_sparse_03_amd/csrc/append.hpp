// Stores of one compressed entry, one indexer key and one window row into
// the caches ("DeepSeek-V4 内部机制" §7: state cache + paged cache; §1.5: RoPE
// channels in BF16, the rest in FP8 with a per-block scale; §6.2: FP4 indexer
// keys).  Used by the cache-append kernel, and by the compressor's decode
// kernel when it appends what it has just produced.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// Records slot .. slot+n_new-1 of KV block `block` from rows x (c floats
// each, global or LDS).  FP8: the block scale becomes max(old scale, amax of
// the new rows' FP8 channels / 448); earlier slots are re-encoded when it
// rises.  The whole workgroup calls this (barriers inside).  A caller that
// has read the block's current scale already passes it (have_s_old).
CSA_DEV void store_kv_records(const AppendArgs& a, uint8_t* block, int slot, int n_new, const float* x, float* red,
                              float* s_sh, bool have_s_old = false, float s_old_in = 0.0f)
{
    const int c = a.c;
    if (a.kv_fmt == 0) {                                   // fp32 records
        float* dst = (float*)block + (size_t)slot * c;
        for (int i = threadIdx.x; i < n_new * c; i += blockDim.x) dst[i] = x[i];
        return;
    }
    if (a.kv_fmt == 1) {                                   // bf16 records
        uint16_t* dst = (uint16_t*)block + (size_t)slot * c;
        for (int i = threadIdx.x; i < n_new * c; i += blockDim.x) dst[i] = f32_to_bf16(x[i]);
        return;
    }
    const int nf = c - a.r, rec = nf + 2 * a.r;            // fp8 + bf16 RoPE channels, block scale
    float amax = 0.f;
    for (int j = 0; j < n_new; ++j)
        for (int ch = threadIdx.x; ch < nf; ch += blockDim.x) amax = fmaxf(amax, fabsf(x[(size_t)j * c + ch]));
    amax = block_max(amax, red);
    if (threadIdx.x == 0) {
        float s_old = slot == 0 ? 0.0f : have_s_old ? s_old_in : *(const float*)block;
        float s_new = amax / 448.0f;
        s_sh[0] = s_old;
        s_sh[1] = s_old > s_new ? s_old : s_new;
    }
    __syncthreads();
    const float s_old = s_sh[0], s = s_sh[1];
    if (s > s_old && slot > 0) {                           // re-encode the earlier slots at the raised scale
        if ((nf & 3) == 0 && (rec & 3) == 0) {
            // four codes per 32-bit word, U words per thread loaded before any store
            constexpr int U = 4;
            const int nw = nf >> 2, total = slot * nw;
            for (int b0 = threadIdx.x; b0 < total; b0 += U * blockDim.x) {
                uint32_t v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = b0 + u * blockDim.x;
                    if (i < total) v[u] = *(const uint32_t*)(block + 64 + (size_t)(i / nw) * rec + 4 * (i % nw));
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = b0 + u * blockDim.x;
                    if (i >= total) continue;
                    uint32_t o = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float old = e4m3_to_f32((v[u] >> (8 * k)) & 0xFFu) * s_old;
                        o |= ((uint32_t)f32_to_e4m3(old / s) & 0xFFu) << (8 * k);
                    }
                    *(uint32_t*)(block + 64 + (size_t)(i / nw) * rec + 4 * (i % nw)) = o;
                }
            }
        } else {
            for (int idx = threadIdx.x; idx < slot * nf; idx += blockDim.x) {
                uint8_t* p = block + 64 + (size_t)(idx / nf) * rec + (idx % nf);
                float old = e4m3_to_f32(*p) * s_old;
                *p = (uint8_t)f32_to_e4m3(old / s);
            }
        }
    }
    if (slot == 0)
        for (int i = threadIdx.x; i < 16; i += blockDim.x) ((uint32_t*)block)[i] = 0u;
    __syncthreads();
    if (threadIdx.x == 0) *(float*)block = s;
    for (int j = 0; j < n_new; ++j) {
        uint8_t* recp = block + 64 + (size_t)(slot + j) * rec;
        const float* xj = x + (size_t)j * c;
        for (int ch = threadIdx.x; ch < nf; ch += blockDim.x)
            recp[ch] = s > 0.0f ? (uint8_t)f32_to_e4m3(xj[ch] / s) : (uint8_t)0;
        for (int ch = threadIdx.x; ch < a.r; ch += blockDim.x)
            ((uint16_t*)(recp + nf))[ch] = f32_to_bf16(xj[nf + ch]);
    }
}

// Indexer key kx (c_idx floats) into slot `slot` of indexer block `phys`.
CSA_DEV void store_idx_key(const AppendArgs& a, int phys, int slot, const float* kx)
{
    const int cI = a.c_idx;
    char* kb = (char*)a.idx + (size_t)phys * a.idx_block_bytes;
    if (a.idx_fmt == 0) {
        float* dst = (float*)kb + (size_t)slot * cI;
        for (int ch = threadIdx.x; ch < cI; ch += blockDim.x) dst[ch] = kx[ch];
    } else if (a.idx_fmt == 1) {
        uint16_t* dst = (uint16_t*)kb + (size_t)slot * cI;
        for (int ch = threadIdx.x; ch < cI; ch += blockDim.x) dst[ch] = f32_to_bf16(kx[ch]);
    } else {                                               // MXFP4: one thread per 32-element block
        uint8_t* codes = (uint8_t*)kb + (size_t)slot * (cI / 2);
        uint8_t* scales = (uint8_t*)kb + (size_t)a.epb * (cI / 2) + (size_t)slot * (cI / 32);
        for (int b = threadIdx.x; b < cI / 32; b += blockDim.x) {
            float amax = 0.f;
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(kx[32 * b + j]));
            int sc = mx_scale_code(amax);
            scales[b] = (uint8_t)sc;
            for (int j = 0; j < 32; j += 2) {
                uint32_t lo = f32_to_e2m1(ldexpf(kx[32 * b + j], 127 - sc));
                uint32_t hi = f32_to_e2m1(ldexpf(kx[32 * b + j + 1], 127 - sc));
                codes[(32 * b + j) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

// Window row src (c floats) of request req at position pos into its ring slot.
CSA_DEV void store_window_row(const AppendArgs& a, int req, int pos, const float* src)
{
    const int slot = pos % a.win_cap;
    char* ring = (char*)a.state + (size_t)req * a.state_stride;
    if (a.win_bf16) {
        uint16_t* dst = (uint16_t*)ring + (size_t)slot * a.c;
        for (int ch = threadIdx.x; ch < a.c; ch += blockDim.x) dst[ch] = f32_to_bf16(src[ch]);
    } else {
        float* dst = (float*)ring + (size_t)slot * a.c;
        for (int ch = threadIdx.x; ch < a.c; ch += blockDim.x) dst[ch] = src[ch];
    }
}

}  // namespace csa
