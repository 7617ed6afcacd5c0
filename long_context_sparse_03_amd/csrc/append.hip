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
#include "append.hpp"

namespace csa {

CSA_DEV void append_entry(const AppendArgs& a, int e, float* red, float* s_sh)
{
    const int count = min(*a.count, a.max_entries);
    if (e >= count) return;
    const int req = a.meta[2 * e], ent = a.meta[2 * e + 1];
    const int blk = ent / a.epb, slot = ent % a.epb;
    const int phys = a.block_table[(size_t)req * a.max_blocks + blk];
    uint8_t* block = (uint8_t*)a.kv + (size_t)phys * a.kv_block_bytes;
    const float* x = a.entries + (size_t)e * a.c;
    if (a.kv_fmt != 2) {
        store_kv_records(a, block, slot, 1, x, red, s_sh);
    } else {
        const bool leader = (e == 0) || a.meta[2 * (e - 1)] != req || a.meta[2 * (e - 1) + 1] / a.epb != blk;
        if (leader) {
            int n_new = 1;
            while (e + n_new < count && a.meta[2 * (e + n_new)] == req && a.meta[2 * (e + n_new) + 1] / a.epb == blk)
                ++n_new;
            store_kv_records(a, block, slot, n_new, x, red, s_sh);
        }
    }
    if (a.idx != nullptr && a.c_idx > 0) store_idx_key(a, phys, slot, a.keys + (size_t)e * a.c_idx);
}

CSA_DEV void append_window_row(const AppendArgs& a, int gtok)
{
    const int req = a.one_per_req ? gtok : find_request(a.cu_new, a.n_req, gtok);
    const int pos = a.start_pos[req] + (a.one_per_req ? 0 : gtok - a.cu_new[req]);
    store_window_row(a, req, pos, a.win + (size_t)gtok * a.c);
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
