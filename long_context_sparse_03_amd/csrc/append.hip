// a2: cache append on gfx950.
//
// Stores compressed entries into the paged ("classic") cache, indexer keys
// into their pool and window rows into the state ring ("DeepSeek-V4 内部机制"
// §7: state cache + paged cache of lcm(m, m') raw tokens per block; §1.5:
// RoPE channels in BF16, the rest in FP8; §6.2: FP4 indexer keys).
//
// One launch: a workgroup per new entry, then one per new token's window row.
// For the FP8 format the first new entry of each (request, block) leads: it
// applies the block-scale rule to all of that block's new entries of this
// call, in slot order, so the result does not depend on how workgroups are
// scheduled.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

CSA_DEV void append_entry(const AppendArgs& a, int e, float* red, float* s_sh)
{
    const int count = min(*a.count, a.max_entries);
    if (e >= count) return;
    const int req = a.meta[2 * e], ent = a.meta[2 * e + 1];
    const int blk = ent / a.epb, slot = ent % a.epb;
    const int phys = a.block_table[(size_t)req * a.max_blocks + blk];
    const int c = a.c;
    const float* x = a.entries + (size_t)e * c;

    if (a.kv_fmt == 0) {                                   // fp32 records
        float* dst = (float*)((char*)a.kv + (size_t)phys * a.kv_block_bytes) + (size_t)slot * c;
        for (int ch = threadIdx.x; ch < c; ch += blockDim.x) dst[ch] = x[ch];
    } else if (a.kv_fmt == 1) {                            // bf16 records
        uint16_t* dst = (uint16_t*)((char*)a.kv + (size_t)phys * a.kv_block_bytes) + (size_t)slot * c;
        for (int ch = threadIdx.x; ch < c; ch += blockDim.x) dst[ch] = f32_to_bf16(x[ch]);
    } else {                                               // fp8 + bf16 RoPE channels, block scale
        const bool leader = (e == 0) || a.meta[2 * (e - 1)] != req || a.meta[2 * (e - 1) + 1] / a.epb != blk;
        if (leader) {
            int n_new = 1;
            while (e + n_new < count && a.meta[2 * (e + n_new)] == req && a.meta[2 * (e + n_new) + 1] / a.epb == blk)
                ++n_new;
            const int nf = c - a.r, rec = nf + 2 * a.r;
            uint8_t* block = (uint8_t*)a.kv + (size_t)phys * a.kv_block_bytes;
            float amax = 0.f;
            for (int j = 0; j < n_new; ++j)
                for (int ch = threadIdx.x; ch < nf; ch += blockDim.x) amax = fmaxf(amax, fabsf(x[(size_t)j * c + ch]));
            amax = block_max(amax, red);
            if (threadIdx.x == 0) {
                float s_old = slot > 0 ? *(const float*)block : 0.0f;
                float s_new = amax / 448.0f;
                s_sh[0] = s_old;
                s_sh[1] = s_old > s_new ? s_old : s_new;
            }
            __syncthreads();
            const float s_old = s_sh[0], s = s_sh[1];
            if (s > s_old && slot > 0) {                   // re-encode the earlier slots at the raised scale
                for (int idx = threadIdx.x; idx < slot * nf; idx += blockDim.x) {
                    uint8_t* p = block + 64 + (size_t)(idx / nf) * rec + (idx % nf);
                    float old = e4m3_to_f32(*p) * s_old;
                    *p = (uint8_t)f32_to_e4m3(old / s);
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
    }

    if (a.idx != nullptr && a.c_idx > 0) {
        const int cI = a.c_idx;
        const float* kx = a.keys + (size_t)e * cI;
        char* kb = (char*)a.idx + (size_t)phys * a.idx_block_bytes;
        if (a.idx_fmt == 0) {
            float* dst = (float*)kb + (size_t)slot * cI;
            for (int ch = threadIdx.x; ch < cI; ch += blockDim.x) dst[ch] = kx[ch];
        } else if (a.idx_fmt == 1) {
            uint16_t* dst = (uint16_t*)kb + (size_t)slot * cI;
            for (int ch = threadIdx.x; ch < cI; ch += blockDim.x) dst[ch] = f32_to_bf16(kx[ch]);
        } else {                                           // MXFP4: one thread per 32-element block
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
}

CSA_DEV void append_window_row(const AppendArgs& a, int gtok)
{
    const int req = a.one_per_req ? gtok : find_request(a.cu_new, a.n_req, gtok);
    const int pos = a.start_pos[req] + (a.one_per_req ? 0 : gtok - a.cu_new[req]);
    const int slot = pos % a.win_cap;
    const float* src = a.win + (size_t)gtok * a.c;
    char* ring = (char*)a.state + (size_t)req * a.state_stride;
    if (a.win_bf16) {
        uint16_t* dst = (uint16_t*)ring + (size_t)slot * a.c;
        for (int ch = threadIdx.x; ch < a.c; ch += blockDim.x) dst[ch] = f32_to_bf16(src[ch]);
    } else {
        float* dst = (float*)ring + (size_t)slot * a.c;
        for (int ch = threadIdx.x; ch < a.c; ch += blockDim.x) dst[ch] = src[ch];
    }
}

// Blocks [0, max_entries) store entries, the next n_tokens blocks window rows.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a)
{
    __shared__ float red[16];
    __shared__ float s_sh[2];
    if ((int)blockIdx.x < a.max_entries) append_entry(a, blockIdx.x, red, s_sh);
    else append_window_row(a, blockIdx.x - a.max_entries);
}

hipError_t launch_append(hipStream_t st, const AppendArgs& a)
{
    const int nw = (a.n_tokens > 0 && a.win != nullptr) ? a.n_tokens : 0;
    const int me = a.max_entries > 0 ? a.max_entries : 0;
    if (me + nw > 0) append_kernel<<<me + nw, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace csa
