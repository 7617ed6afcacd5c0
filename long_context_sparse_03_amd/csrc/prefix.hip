// Prefix reuse, host-memory tier: copies of whole cache blocks between a
// layer's pools and pinned host memory ("DeepSeek-V4 内部机制" §7: the shared
// prefix's compressed entries are stored whole).  One workgroup per block
// moves it in 16-byte pieces, reading or writing the host buffer directly
// over the bus (pinned memory is visible to the device), so a prefix of any
// length is one launch.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// Block j of the list: bytes [0, block_bytes) of pool block ids[j] <->
// host + j * block_bytes.  dir 0: to host, 1: from host.  Negative ids are
// skipped.
template <int DIR>
__global__ __launch_bounds__(256) void prefix_blocks_kernel(const int32_t* __restrict__ ids, char* __restrict__ pool,
                                                            size_t block_bytes, char* __restrict__ host)
{
    const int id = ids[blockIdx.x];
    if (id < 0) return;                                          // workgroup-uniform
    uint4* p = (uint4*)(pool + (size_t)id * block_bytes);
    uint4* h = (uint4*)(host + (size_t)blockIdx.x * block_bytes);
    const int n16 = (int)(block_bytes / 16);
    constexpr int U = 4;                                         // pieces per thread in flight
    for (int b = threadIdx.x; b < n16; b += U * blockDim.x) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = b + u * blockDim.x;
            if (i < n16) v[u] = DIR == 0 ? p[i] : h[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = b + u * blockDim.x;
            if (i < n16) (DIR == 0 ? h : p)[i] = v[u];
        }
    }
}

hipError_t launch_prefix_blocks(hipStream_t st, int n_blocks, const int32_t* ids, void* pool, size_t block_bytes,
                                void* host, int dir)
{
    if (n_blocks <= 0 || block_bytes == 0) return hipSuccess;
    if (dir == 0)
        prefix_blocks_kernel<0><<<n_blocks, 256, 0, st>>>(ids, (char*)pool, block_bytes, (char*)host);
    else
        prefix_blocks_kernel<1><<<n_blocks, 256, 0, st>>>(ids, (char*)pool, block_bytes, (char*)host);
    return hipGetLastError();
}

}  // namespace csa
