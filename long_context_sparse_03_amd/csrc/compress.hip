// a1: token-level compressor on gfx950.
//
// Follows "DeepSeek-V4 内部机制" §1.2 Step 1 (CSA: per-channel softmax over
// the overlapping 2m window of Z + B, weighted sum of the C rows) and §1.3
// (HCA: m' rows, no overlap); yunpan.plus explainer eqs. (6)-(7), (10)-(11).
// Entry normalisation and partial RoPE: "DeepSeek-V4 内部机制" §1.4 table.
//
// Kernels, in launch order:
//   proj_*      H . W^T into the workspace (fp32 out), MFMA with fragments
//               loaded straight from global memory (rows are k-contiguous).
//   merge       one workgroup per completed entry: softmax-merge per channel,
//               then RMSNorm + RoPE of the main entry; indexer keys raw.
//   window_rows one workgroup per new token: RMSNorm + RoPE of its C^a row.
//   tail_update copies the newest projected rows into the state's tail ring
//               (after merge has read the old ring contents).
#include "common.hpp"
#include "kernels.hpp"
#include "append.hpp"

namespace csa {

// ---------------------------------------------------------------------------
// projection: P[M x N] = X[M x K] . Wt[N x K]^T, Wt rows n < n_main from W,
// the rest from Wi.  T is float or uint16_t (bf16).  Rows of X are ldx
// elements apart and rows of P ldp apart; P is fp32 or (out_bf16) bf16;
// grid z selects a group: X, W / Wi and P advance by gx, gw and gp elements
// per group (the compressor: one group, ldx = K, ldp = N, fp32).
// ---------------------------------------------------------------------------

struct GemmShape {
    int ldx, ldp, out_bf16;
    size_t gx, gw, gp;
};

CSA_DEV void store_out(void* P, size_t i, int out_bf16, float v)
{
    if (out_bf16) ((uint16_t*)P)[i] = f32_to_bf16(v);
    else ((float*)P)[i] = v;
}

template <class T, class MMA>
__global__ __launch_bounds__(256) void proj_large(const T* __restrict__ X, const T* __restrict__ W,
                                                  const T* __restrict__ Wi, int n_main, int N, int M, int K,
                                                  void* __restrict__ P, GemmShape sh)
{
    constexpr int EPF = 16 / sizeof(T);
    X += blockIdx.z * sh.gx;
    W += blockIdx.z * sh.gw;
    Wi += blockIdx.z * sh.gw;
    const size_t p0 = blockIdx.z * sh.gp;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int m0 = blockIdx.y * 128 + (wave >> 1) * 64;
    const int n0 = blockIdx.x * 128 + (wave & 1) * 64;
    const T* ap[4];
    const T* bp[4];
    bool av[4], bv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        int m = m0 + 16 * t + li;
        av[t] = m < M;
        ap[t] = X + (size_t)(av[t] ? m : 0) * sh.ldx + g * EPF;
        int n = n0 + 16 * t + li;
        bv[t] = n < N;
        int nn = bv[t] ? n : 0;
        bp[t] = (nn < n_main ? W + (size_t)nn * K : Wi + (size_t)(nn - n_main) * K) + g * EPF;
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    for (int k0 = 0; k0 < K; k0 += MMA::K) {
        uint4 a[4], b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a[t] = ld16(ap[t] + k0);        // rows past M / N are clamped, their outputs dropped
            b[t] = ld16(bp[t] + k0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = MMA::step(a[i], b[j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int n = n0 + 16 * j + li;
            if (n >= N) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int m = m0 + 16 * i + 4 * g + q;
                if (m < M) store_out(P, p0 + (size_t)m * sh.ldp + n, sh.out_bf16, acc[i][j][q]);
            }
        }
}

// Many rows, bf16 (prefill chunks): 256 x 160 output tiles (the 4096-row
// compressor projection of 2560 columns is 16 x 16 tiles, one per compute
// unit), four waves of 128 x 80, the contraction in stages of 64 channels
// that go from memory straight into LDS (direct-to-LDS loads), two stages in
// flight: the next stage's loads are issued right after the barrier that
// publishes the current one.  A stage row is the row's 8 chunks of 16 bytes,
// chunk c at slot c ^ ((row / 2) mod 8), so the 16 lanes that read one chunk
// of 16 consecutive rows cover all 64 banks.  Rows past M / N are clamped
// (their outputs dropped); K is a multiple of the stage.
constexpr int PG_BM = 256, PG_BN = 160, PG_BK = 64;

__global__ __launch_bounds__(256) void proj_lds(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                const uint16_t* __restrict__ Wi, int n_main, int N, int M, int K,
                                                void* __restrict__ P, GemmShape sh)
{
    static_assert(PG_BK == 64 && PG_BM == 256 && PG_BN == 160, "8 chunks per stage row; 32 + 20 row blocks of 8");
    // the two stages as separate objects, so that reads of one need not wait
    // for the loads in flight into the other
    __shared__ __attribute__((aligned(16))) uint8_t As0[PG_BM * 128];
    __shared__ __attribute__((aligned(16))) uint8_t As1[PG_BM * 128];
    __shared__ __attribute__((aligned(16))) uint8_t Bs0[PG_BN * 128];
    __shared__ __attribute__((aligned(16))) uint8_t Bs1[PG_BN * 128];
    X += blockIdx.z * sh.gx;
    W += blockIdx.z * sh.gw;
    Wi += blockIdx.z * sh.gw;
    const size_t p0 = blockIdx.z * sh.gp;
    const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bm0 = blockIdx.y * PG_BM, bn0 = blockIdx.x * PG_BN;
    const int wm = wave >> 1, wn = wave & 1;                   // this wave's 128 x 80 sub-tile

    // direct-to-LDS sources: the u-th load of wave w fills row block 4u + w
    // (rows 8 (4u + w) .. +7, 1 KB), lane l the slot l mod 8 of row l / 8,
    // i.e. chunk (l mod 8) ^ ((row / 2) mod 8), the same chunk for every u
    const int rr = lane >> 3;
    const int ch = (lane & 7) ^ ((4 * wave + (rr >> 1)) & 7);
    const uint16_t* asrc[8];
    const uint16_t* bsrc[5];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int m = min(bm0 + 8 * (4 * u + wave) + rr, M - 1);
        asrc[u] = X + (size_t)m * sh.ldx + 8 * ch;
    }
#pragma unroll
    for (int u = 0; u < 5; ++u) {
        const int n = min(bn0 + 8 * (4 * u + wave) + rr, N - 1);
        bsrc[u] = (n < n_main ? W + (size_t)n * K : Wi + (size_t)(n - n_main) * K) + 8 * ch;
    }
    auto issue = [&](int k0, uint8_t* as, uint8_t* bs) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            __builtin_amdgcn_global_load_lds((const CSA_GLOBAL void*)(asrc[u] + k0),
                                             (CSA_LDS void*)(as + (4 * u + wave) * 1024), 16, 0, 0);
#pragma unroll
        for (int u = 0; u < 5; ++u)
            __builtin_amdgcn_global_load_lds((const CSA_GLOBAL void*)(bsrc[u] + k0),
                                             (CSA_LDS void*)(bs + (4 * u + wave) * 1024), 16, 0, 0);
    };

    f32x4_t acc[8][5];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j) acc[i][j] = zero4();
    // stage kb in buffer kb mod 2: wait for this wave's loads of it, a
    // barrier (everyone's have landed, and stage kb-1 is no longer read), the
    // fragments of both steps into registers, then the loads of stage kb+1
    // into the other buffer (issued after this stage's reads, so nothing
    // makes the reads wait for them), then the MFMAs.  Fragment of row li (of
    // a 16-row tile), channels 8 (4s + g) .. +7 of the stage: slot
    // (4s + g) ^ (li / 2) of the row (tile rows start at multiples of 16, so
    // the row's (row / 2) mod 8 is li / 2)
    const int nk = K / PG_BK;
    issue(0, As0, Bs0);
    for (int kb = 0; kb < nk; ++kb) {
        const bool odd = kb & 1;
        const uint8_t* A = (odd ? As1 : As0) + (size_t)(128 * wm) * 128;
        const uint8_t* B = (odd ? Bs1 : Bs0) + (size_t)(80 * wn) * 128;
        __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0)
        __syncthreads();
        uint4 af[2][8], bf[2][5];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int off = li * 128 + 16 * ((4 * s + g) ^ (li >> 1));
#pragma unroll
            for (int i = 0; i < 8; ++i) af[s][i] = *(const uint4*)(A + 16 * i * 128 + off);
#pragma unroll
            for (int j = 0; j < 5; ++j) bf[s][j] = *(const uint4*)(B + 16 * j * 128 + off);
        }
        if (kb + 1 < nk) issue((kb + 1) * PG_BK, odd ? As0 : As1, odd ? Bs0 : Bs1);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 5; ++j) acc[i][j] = MmaBF16::step(af[s][i], bf[s][j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int n = bn0 + 80 * wn + 16 * j + li;
            if (n >= N) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = bm0 + 128 * wm + 16 * i + 4 * g + q;
                if (m < M) store_out(P, p0 + (size_t)m * sh.ldp + n, sh.out_bf16, acc[i][j][q]);
            }
        }
}

// The LDS-staged kernel when the shape suits it: bf16, whole stages, rows
// 16-byte aligned, and enough tiles to fill the compute units.
static bool use_proj_lds(bool bf16, int M, int N, int K, int groups, const void* X, const void* W, const void* Wi,
                         int ldx)
{
    const long tiles = (long)((M + PG_BM - 1) / PG_BM) * ((N + PG_BN - 1) / PG_BN) * groups;
    const uintptr_t al = (uintptr_t)X | (uintptr_t)W | (uintptr_t)Wi;
    return bf16 && K % PG_BK == 0 && ldx % 8 == 0 && al % 16 == 0 && tiles >= 128;
}

// Few rows (decode): a 16 x 16 output tile per workgroup; the NW waves
// split K into contiguous parts (K / NW a multiple of the MMA step), summed
// in wave order.  Sixteen waves keep a whole 16-column slice of the weights
// in flight at once for the decode widths.
template <class T, class MMA, int NW>
__global__ __launch_bounds__(64 * NW) void proj_small(const T* __restrict__ X, const T* __restrict__ W,
                                                      const T* __restrict__ Wi, int n_main, int N, int M, int K,
                                                      void* __restrict__ P, GemmShape sh)
{
    constexpr int EPF = 16 / sizeof(T);
    __shared__ float red[NW][64][4];
    X += blockIdx.z * sh.gx;
    W += blockIdx.z * sh.gw;
    Wi += blockIdx.z * sh.gw;
    const size_t p0 = blockIdx.z * sh.gp;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int m = blockIdx.y * 16 + li, n = blockIdx.x * 16 + li;
    const bool av = m < M, bv = n < N;
    const int kq = K / NW, kb = wave * kq;
    const T* ap = X + (size_t)(av ? m : 0) * sh.ldx + kb + g * EPF;
    int nn = bv ? n : 0;
    const T* bp = (nn < n_main ? W + (size_t)nn * K : Wi + (size_t)(nn - n_main) * K) + kb + g * EPF;
    f32x4_t acc[4] = {zero4(), zero4(), zero4(), zero4()};
    for (int k0 = 0; k0 < kq; k0 += 8 * MMA::K) {          // up to eight fragment pairs in flight
        const int nb = min(8, (kq - k0) / MMA::K);
        uint4 a8[8], b8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int ku = k0 + min(u, nb - 1) * MMA::K;    // clamped: steps past nb are not used
            a8[u] = ld16(ap + ku);                          // clamped rows: only dropped outputs see them
            b8[u] = ld16(bp + ku);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < nb) acc[u & 3] = MMA::step(a8[u], b8[u], acc[u & 3]);
    }
    const f32x4_t acc0 = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const f32x4_t acc1 = zero4();
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][lane][q] = acc0[q] + acc1[q];
    __syncthreads();
    if (wave == 0) {
        const int col = blockIdx.x * 16 + li;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v = red[0][lane][q];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += red[w][lane][q];
            int row = blockIdx.y * 16 + 4 * g + q;
            if (row < M && col < N) store_out(P, p0 + (size_t)row * sh.ldp + col, sh.out_bf16, v);
        }
    }
}

// Few-row bf16 products with both operands staged through LDS.  Wave w owns
// channels [w K/NW, (w+1) K/NW); per batch of up to 256 channels it copies the
// 16 rows of X and the 16 rows of W that its fragments need into its own LDS
// region, row after row (two rows of 512 bytes per instruction: 16-byte
// chunk c of row r lands at slot c ^ r), and reads the MFMA fragments from
// there (fragment lanes of one chunk index sit in 16 different banks).
// Reading the fragments straight from memory makes every load instruction
// touch 16 rows 64 bytes at a time, so the weight stream spreads over 16
// DRAM pages per instruction instead of one or two.  Requires K % (32 NW)
// == 0 and 16-byte aligned rows.
constexpr int PL_NW = 8;                      // waves per workgroup
constexpr int PL_KB = 256;                    // channels per wave and batch (512 bytes of a bf16 row)

__global__ __launch_bounds__(64 * PL_NW) void proj_small_lds(const uint16_t* __restrict__ X,
                                                             const uint16_t* __restrict__ W,
                                                             const uint16_t* __restrict__ Wi, int n_main, int N,
                                                             int M, int K, void* __restrict__ P, GemmShape sh)
{
    constexpr int NW = PL_NW, RB = PL_KB * 2;                  // bytes of a row's batch
    __shared__ __attribute__((aligned(16))) uint16_t Xs[NW][16 * PL_KB];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[NW][16 * PL_KB];
    __shared__ float red[NW][64][4];
    X += blockIdx.z * sh.gx;
    W += blockIdx.z * sh.gw;
    Wi += blockIdx.z * sh.gw;
    const size_t p0 = blockIdx.z * sh.gp;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int kq = K / NW, kb = wave * kq;
    // the two rows this lane copies: r = 2i + lane / 32 for instruction i;
    // rows past M or N read row 0 (their outputs are not stored)
    const char* xr[8];
    const char* wr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 2 * i + (lane >> 5);
        const int m = blockIdx.y * 16 + r, n = blockIdx.x * 16 + r;
        const int mm = m < M ? m : 0, nn = n < N ? n : 0;
        xr[i] = (const char*)(X + (size_t)mm * sh.ldx + kb);
        wr[i] = (const char*)(nn < n_main ? W + (size_t)nn * K : Wi + (size_t)(nn - n_main) * K) + 2 * (size_t)kb;
    }
    f32x4_t acc[4] = {zero4(), zero4(), zero4(), zero4()};
    for (int k0 = 0; k0 < kq; k0 += PL_KB) {
        const int nb = min(8, (kq - k0) / MmaBF16::K);       // 32-channel steps in this batch
        // this wave's fragment reads of the previous batch have completed
        // (their MFMAs consumed them) before its region is refilled
        __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 2 * i + (lane >> 5);
            // chunks past the batch (a short last batch) repeat its last chunk
            const int c = min((lane & 31) ^ r, 4 * nb - 1);
            const size_t off = 2 * (size_t)k0 + 16 * (size_t)c;
            __builtin_amdgcn_global_load_lds((const CSA_GLOBAL void*)(xr[i] + off), (CSA_LDS void*)&Xs[wave][i * RB],
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const CSA_GLOBAL void*)(wr[i] + off), (CSA_LDS void*)&Ws[wave][i * RB],
                                             16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);                    // vmcnt(0): both regions filled
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u < nb) {
                const int slot = (4 * u + g) ^ li;
                const uint4 av = *(const uint4*)&Xs[wave][li * PL_KB + 8 * slot];
                const uint4 bv = *(const uint4*)&Ws[wave][li * PL_KB + 8 * slot];
                acc[u & 3] = MmaBF16::step(av, bv, acc[u & 3]);
            }
        }
    }
    const f32x4_t acc0 = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][lane][q] = acc0[q];
    __syncthreads();
    if (wave == 0) {
        const int col = blockIdx.x * 16 + li;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v = red[0][lane][q];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += red[w][lane][q];
            int row = blockIdx.y * 16 + 4 * g + q;
            if (row < M && col < N) store_out(P, p0 + (size_t)row * sh.ldp + col, sh.out_bf16, v);
        }
    }
}

// Few-row compressor projection as PROJ_PARTS partial products over equal
// chunks of the contraction: chunk s (grid z) of K / PROJ_PARTS channels
// writes P_s [M x N] fp32 at P + s * M * N, and the kernels that read the
// projection add the partials in chunk order.  Splitting the contraction
// gives more workgroups than 16-column blocks (a 1024-column projection has
// only 64), and each wave takes at most PK_KB channels per batch (one batch
// up to K = 4096 with 4 waves, 8192 with 8), so all of a wave's weight bytes
// are in flight at once.  Weight rows go through LDS as coalesced 512-byte
// row pieces (as in proj_small_lds); the few activation rows are read
// straight into MFMA fragments (they stay in the L2 cache).
constexpr int PK_KB = 256;                    // channels per wave and batch

template <int NW>
__global__ __launch_bounds__(64 * NW) void proj_ksplit(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                       const uint16_t* __restrict__ Wi, int n_main, int N, int M,
                                                       int K, float* __restrict__ P)
{
    constexpr int RB = 2 * PK_KB;                              // elements of two rows' batches
    __shared__ __attribute__((aligned(16))) uint16_t Ws[NW][16 * PK_KB];
    __shared__ float red[NW][64][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int kc = K / PROJ_PARTS;                             // channels of a chunk (a multiple of 32)
    const int steps = kc / MmaBF16::K, spw = (steps + NW - 1) / NW;
    const int st0 = min(steps, wave * spw), nst = min(steps, st0 + spw) - st0;   // this wave's 32-channel steps
    const int k0 = blockIdx.z * kc + MmaBF16::K * st0;        // and its first channel
    const int m = blockIdx.y * 16 + li;
    // rows past M or N read row 0 (their outputs are not stored)
    const uint16_t* xr = X + (size_t)(m < M ? m : 0) * K + k0 + 8 * g;
    const char* wr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int n = blockIdx.x * 16 + 2 * i + (lane >> 5), nn = n < N ? n : 0;
        wr[i] = (const char*)(nn < n_main ? W + (size_t)nn * K : Wi + (size_t)(nn - n_main) * K) + 2 * (size_t)k0;
    }
    f32x4_t acc[4] = {zero4(), zero4(), zero4(), zero4()};
    for (int b0 = 0; b0 < nst; b0 += 8) {
        const int nb = min(8, nst - b0);                       // steps in this batch
        // this wave's fragment reads of the previous batch are done before
        // its region is refilled
        __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
        uint4 xf[8];
        // four waves (K up to 4096): a full batch of 8 steps without per-step
        // branches, which otherwise make each fragment read wait before its
        // MFMA (measured: 128K compressor projection 8.6 -> 8.2 us; with
        // eight waves and 7-step batches the same form was slower)
        const bool full = NW == 4 && nb == 8;
        if (full) {
#pragma unroll
            for (int u = 0; u < 8; ++u) xf[u] = *(const uint4*)(xr + MmaBF16::K * (b0 + u));
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u < nb) xf[u] = *(const uint4*)(xr + MmaBF16::K * (b0 + u));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 2 * i + (lane >> 5);
            // chunks past the batch (a short batch) repeat its last chunk
            const int c = min((lane & 31) ^ r, 4 * nb - 1);
            __builtin_amdgcn_global_load_lds((const CSA_GLOBAL void*)(wr[i] + 64 * (size_t)b0 + 16 * c),
                                             (CSA_LDS void*)&Ws[wave][i * RB], 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);                    // vmcnt(0): fragments and the region filled
        if (full) {
            // every fragment read issued before the first MFMA (steps in the
            // same order per accumulator as below)
            uint4 bv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) bv[u] = *(const uint4*)&Ws[wave][li * PK_KB + 8 * ((4 * u + g) ^ li)];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u & 3] = MmaBF16::step(xf[u], bv[u], acc[u & 3]);
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u < nb) {
                    const int slot = (4 * u + g) ^ li;
                    const uint4 bv = *(const uint4*)&Ws[wave][li * PK_KB + 8 * slot];
                    acc[u & 3] = MmaBF16::step(xf[u], bv, acc[u & 3]);
                }
            }
        }
    }
    const f32x4_t acc0 = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][lane][q] = acc0[q];
    __syncthreads();
    // the waves' sums in wave order, one output row per wave
    float* Ps = P + (size_t)blockIdx.z * M * N;
    for (int q = wave; q < 4; q += NW) {
        const int col = blockIdx.x * 16 + li, row = blockIdx.y * 16 + 4 * g + q;
        float v = red[0][lane][q];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][lane][q];
        if (row < M && col < N) Ps[(size_t)row * N + col] = v;
    }
}

// Loads of a projected row for copy_row / token_row: pieces b, b + blockDim,
// .. (U of them) of T (float4 or float), of ns partial planes sst floats
// apart, summed in plane order.  Every load is issued before any is used:
// pieces past the row (n pieces) read the row's last piece instead (never
// stored), so no load sits behind a per-lane branch, which would make each
// of them wait for its data before the next is issued.
template <class T, int U>
CSA_DEV void row_planes(const float* __restrict__ src, int n, int b, int ns, size_t sst, T (&v)[U])
{
    // pieces u whose slot starts past the row in every thread are skipped
    // (a uniform test: b - threadIdx.x is the workgroup's first piece)
    const int b0 = b - (int)threadIdx.x;
    int ic[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ic[u] = min(b + u * (int)blockDim.x, n - 1);
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u == 0 || b0 + u * (int)blockDim.x < n) v[u] = ((const T*)src)[ic[u]];
    if (ns <= 1) return;
    T x[PROJ_PARTS - 1][U];
#pragma unroll
    for (int s = 1; s < PROJ_PARTS; ++s)
        if (s < ns)
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u == 0 || b0 + u * (int)blockDim.x < n) x[s - 1][u] = ((const T*)(src + s * sst))[ic[u]];
#pragma unroll
    for (int s = 1; s < PROJ_PARTS; ++s)
        if (s < ns)
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u == 0 || b0 + u * (int)blockDim.x < n) v[u] += x[s - 1][u];
    for (int s = PROJ_PARTS; s < ns; ++s)                      // (more planes than the projection makes)
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u == 0 || b0 + u * (int)blockDim.x < n) v[u] += ((const T*)(src + s * sst))[ic[u]];
}

// dst[0..n) (and dst2[0..n2), n2 <= n) = the sum of the ns partial planes of
// the row at src, with the threads of the block: 16-byte pieces when every
// pointer is 16-byte aligned and n, n2 are multiples of 4, a batch of pieces
// loaded before any is stored (one memory latency per batch).
CSA_DEV void copy_row(float* __restrict__ dst, const float* __restrict__ src, int n, float* dst2 = nullptr,
                      int n2 = 0, int ns = 1, size_t sst = 0)
{
    constexpr int U = 4;
    if (n <= 0) return;
    if (((n | n2) & 3) == 0 && (sst & 3) == 0 && (((uintptr_t)dst | (uintptr_t)src | (uintptr_t)dst2) & 15) == 0) {
        const int n4 = n >> 2;
        for (int b = threadIdx.x; b < n4; b += U * blockDim.x) {
            float4 v[U];
            row_planes<float4, U>(src, n4, b, ns, sst, v);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = b + u * blockDim.x;
                if (i < n4) ((float4*)dst)[i] = v[u];
                if (4 * i < n2) ((float4*)dst2)[i] = v[u];
            }
        }
    } else {
        for (int b = threadIdx.x; b < n; b += U * blockDim.x) {
            float v[U];
            row_planes<float, U>(src, n, b, ns, sst, v);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = b + u * blockDim.x;
                if (i < n) dst[i] = v[u];
                if (i < n2) dst2[i] = v[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + RoPE of one row held in LDS (xs[0..c)), written to out.
// ---------------------------------------------------------------------------

CSA_DEV void norm_rope_store(float* xs, float* red, int c, int r, const float* gamma, float eps, double pos,
                             float theta, float* out)
{
    float ss = 0.f;
    for (int ch = threadIdx.x; ch < c; ch += blockDim.x) ss += xs[ch] * xs[ch];
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)c + eps);
    __syncthreads();
    for (int ch = threadIdx.x; ch < c; ch += blockDim.x) xs[ch] = gamma[ch] * (xs[ch] * inv);
    __syncthreads();
    for (int j = threadIdx.x; j < r / 2; j += blockDim.x) {
        float cs, sn;
        rope_cs(pos, j, r, theta, &cs, &sn);
        int d = c - r + 2 * j;
        float a = xs[d], b = xs[d + 1];
        xs[d] = a * cs - b * sn;
        xs[d + 1] = a * sn + b * cs;
    }
    __syncthreads();
    for (int ch = threadIdx.x; ch < c; ch += blockDim.x) out[ch] = xs[ch];
}

// ---------------------------------------------------------------------------
// merge: one workgroup per entry completed in this call
// ---------------------------------------------------------------------------

// (request, entry index) of the call's entry e, or request -1 when the call
// completes no more than e entries or e >= max_entries.  Entry 0's
// workgroup also writes the call's entry count.
CSA_DEV int2 locate_entry(const CompressArgs& a, int e)
{
    // locate the entry: requests in order, entries of a request in index
    // order.  The threads take one request each (256 at a time): the entries
    // a request completes, an exclusive scan over the requests, and the
    // thread whose range holds e records (request, entry index).
    __shared__ int wsum[4], loc[2];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) loc[0] = -1;
    int total = 0;
    for (int base = 0; base < a.n_req; base += 256) {
        const int rr = base + (int)threadIdx.x;
        int cnt = 0, s = 0;
        if (rr < a.n_req) {
            s = a.start_pos[rr];
            cnt = (s + a.cu_new[rr + 1] - a.cu_new[rr]) / a.m - s / a.m;
        }
        int inc = cnt;                                          // inclusive scan within the wave
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane == 63) wsum[w] = inc;
        __syncthreads();
        int before = total;
        for (int i = 0; i < 4; ++i) {
            before += i < w ? wsum[i] : 0;
            total += wsum[i];
        }
        before += inc - cnt;
        if (cnt > 0 && e >= before && e < before + cnt) {
            loc[0] = rr;
            loc[1] = s / a.m + (e - before);
        }
        __syncthreads();
    }
    const int req = loc[0], ent = loc[1];
    if (e == 0 && threadIdx.x == 0) *a.out_count = total;
    if (req < 0 || e >= a.max_entries) return make_int2(-1, 0);
    return make_int2(req, ent);
}

// Entry e = entry `ent` of request `req`: out_entries row e (and xs, in LDS),
// out_keys row e (and ks when given), out_meta row e.
CSA_DEV void merge_located(const CompressArgs& a, int e, int req, int ent, float* xs, float* red, float* ks)
{
    const int s0 = a.start_pos[req], cu = a.cu_new[req];
    const float* tail = (const float*)((const char*)a.state + (size_t)req * a.state_stride + a.tail_off);
    const int m = a.m, c = a.c, cI = a.c_idx;
    const bool has_b = a.overlap && ent >= 1;
    const int nch = c + (a.overlap ? cI : 0);
    for (int ch = threadIdx.x; ch < nch; ch += blockDim.x) {
        const bool ix = ch >= c;
        const int cc = ix ? ch - c : ch;
        const int w = ix ? cI : c;
        const int base = ix ? 4 * c : 0;
        const float* Ba = ix ? a.B_a_idx : a.B_a;
        const float* Bb = ix ? a.B_b_idx : a.B_b;
        const int colCa = base + cc;
        const int colCb = base + w + cc;
        const int colZa = base + (a.overlap ? 2 * w : w) + cc;
        const int colZb = base + 3 * w + cc;
        // softmax over the entry's m rows (and the previous entry's m rows
        // with overlap) of Z + B, weights on C; rows go in batches of MB
        // whose loads are all issued before use, with a running maximum
        // across batches
        constexpr int MB = 8;
        const int nrows = has_b ? 2 * m : m;
        float mx = -INFINITY, den = 0.f, acc = 0.f;
        for (int r0 = 0; r0 < nrows; r0 += MB) {
            float z[MB], cv[MB];
            // every load of the batch (a row's Z and C values, the partial
            // planes of rows projected in this call, the bias) is issued
            // before any is used; the planes are then added in plane order
            float zl[MB], cl[MB], bl[MB], zx[MB][PROJ_PARTS - 1], cx[MB][PROJ_PARTS - 1];
            bool nw[MB];
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                const int rr = min(r0 + u, nrows - 1);
                const bool second = rr >= m;                    // a row of the previous entry (overlap)
                const int r = second ? rr - m : rr;
                const int p = m * (second ? ent - 1 : ent) + r;
                const bool new_row = p >= s0;                   // projected in this call (partials)
                const float* row = new_row ? a.P + (size_t)(cu + p - s0) * a.ncols : tail + (size_t)(p % a.R) * a.ncols;
                const int cz = second ? colZb : colZa, cC = second ? colCb : colCa;
                nw[u] = new_row;
                zl[u] = row[cz];
                cl[u] = row[cC];
                bl[u] = (second ? Bb : Ba)[r * w + cc];
                if (new_row) {
#pragma unroll
                    for (int s = 1; s < PROJ_PARTS; ++s) {
                        if (s < a.n_psplit) {
                            zx[u][s - 1] = row[s * a.psplit_stride + cz];
                            cx[u][s - 1] = row[s * a.psplit_stride + cC];
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                float zv = zl[u], cvv = cl[u];
                if (nw[u]) {                                    // (n_psplit <= PROJ_PARTS)
#pragma unroll
                    for (int s = 1; s < PROJ_PARTS; ++s) {
                        if (s < a.n_psplit) {
                            zv += zx[u][s - 1];
                            cvv += cx[u][s - 1];
                        }
                    }
                }
                z[u] = zv + bl[u];
                cv[u] = cvv;
            }
            float cm = -INFINITY;
#pragma unroll
            for (int u = 0; u < MB; ++u)
                if (r0 + u < nrows) cm = fmaxf(cm, z[u]);
            const float nm = fmaxf(mx, cm);
            const float sc = mx == -INFINITY ? 0.f : expf(mx - nm);
            den *= sc;
            acc *= sc;
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                if (r0 + u < nrows) {
                    const float wgt = expf(z[u] - nm);
                    den += wgt;
                    acc += wgt * cv[u];
                }
            }
            mx = nm;
        }
        float v = acc / den;
        if (ix) {
            a.out_keys[(size_t)e * cI + cc] = v;
            if (ks != nullptr) ks[cc] = v;
        } else {
            xs[cc] = v;
        }
    }
    __syncthreads();
    norm_rope_store(xs, red, c, a.r, a.gamma, a.eps, (double)m * (double)ent, a.theta, a.out_entries + (size_t)e * c);
    if (threadIdx.x == 0) {
        a.out_meta[2 * e] = req;
        a.out_meta[2 * e + 1] = ent;
    }
}

// Workgroup 0 of the kernel after the projection writes every request's
// next start position (the caller's position buffer for the following call).
CSA_DEV void write_next_positions(const CompressArgs& a)
{
    if (a.next_pos == nullptr || blockIdx.x != 0) return;
    for (int r = threadIdx.x; r < a.n_req; r += blockDim.x)
        a.next_pos[r] = a.start_pos[r] + (a.cu_new[r + 1] - a.cu_new[r]);
}

CSA_DEV void merge_entry(const CompressArgs& a, int e, float* xs, float* red)
{
    const int2 re = locate_entry(a, e);
    if (re.x >= 0) merge_located(a, e, re.x, re.y, xs, red, nullptr);
}

__global__ __launch_bounds__(256) void merge_kernel(CompressArgs a)
{
    __shared__ __attribute__((aligned(16))) float xs[512];
    __shared__ float red[16];
    write_next_positions(a);
    merge_entry(a, blockIdx.x, xs, red);
}

// window row of new token gtok: its C^a (CSA) or C (HCA) row, normalised and
// rotated at its position
CSA_DEV void window_row(const CompressArgs& a, int gtok, int pos, float* xs, float* red)
{
    copy_row(xs, a.P + (size_t)gtok * a.ncols, a.c, nullptr, 0, a.n_psplit, a.psplit_stride);   // C^a (CSA) or C (HCA)
    __syncthreads();
    norm_rope_store(xs, red, a.c, a.r, a.gamma, a.eps, (double)pos, a.theta, a.out_win + (size_t)gtok * a.c);
}

__global__ __launch_bounds__(256) void window_rows_kernel(CompressArgs a)
{
    __shared__ __attribute__((aligned(16))) float xs[512];
    __shared__ float red[16];
    const int gtok = blockIdx.x;
    const int req = find_request(a.cu_new, a.n_req, gtok);
    window_row(a, gtok, a.start_pos[req] + (gtok - a.cu_new[req]), xs, red);
}

__global__ __launch_bounds__(256) void tail_update_kernel(CompressArgs a)
{
    const int j = blockIdx.x, req = blockIdx.y;
    const int cu = a.cu_new[req], n = a.cu_new[req + 1] - cu, s0 = a.start_pos[req];
    const int keep = n < a.R ? n : a.R;
    if (j >= keep) return;
    const int p = s0 + n - keep + j;
    float* tail = (float*)((char*)a.state + (size_t)req * a.state_stride + a.tail_off);
    copy_row(tail + (size_t)(p % a.R) * a.ncols, a.P + (size_t)(cu + n - keep + j) * a.ncols, a.ncols, nullptr, 0,
             a.n_psplit, a.psplit_stride);
}

// New token gtok of a call with at most one new token per request: the sum
// of its projected row's partial planes goes into the request's tail ring
// (slot pos mod R) and its first c channels (C^a, HCA: C) into xs; returns
// the token's position.  The row's loads do not depend on the position, so
// they are issued before the wait for it (one round trip to memory for both,
// not two in a row).  Threads take 16-byte pieces when the row allows.
CSA_DEV int token_row(const CompressArgs& a, int gtok, float* xs)
{
    const int req = a.one_per_req ? gtok : find_request(a.cu_new, a.n_req, gtok);
    const int pos_raw = a.start_pos[req];
    const float* src = a.P + (size_t)gtok * a.ncols;
    const int n = a.ncols, nc = a.c;
    constexpr int U = 4;
    const bool vec = ((n | nc) & 3) == 0 && (a.psplit_stride & 3) == 0 && (((uintptr_t)src | (uintptr_t)xs) & 15) == 0 &&
                     (((uintptr_t)a.state | a.tail_off | a.state_stride) & 15) == 0;
    if (vec && n > 0 && (n >> 2) <= U * (int)blockDim.x) {      // the whole row in one batch
        const int n4 = n >> 2;
        float4 v[U];
        row_planes<float4, U>(src, n4, (int)threadIdx.x, a.n_psplit, a.psplit_stride, v);
        const int pos = pos_raw + (a.one_per_req ? 0 : gtok - a.cu_new[req]);
        float* tail = (float*)((char*)a.state + (size_t)req * a.state_stride + a.tail_off) + (size_t)(pos % a.R) * n;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = (int)threadIdx.x + u * (int)blockDim.x;
            if (i < n4) ((float4*)tail)[i] = v[u];
            if (4 * i < nc) ((float4*)xs)[i] = v[u];
        }
        return pos;
    }
    const int pos = pos_raw + (a.one_per_req ? 0 : gtok - a.cu_new[req]);
    float* tail = (float*)((char*)a.state + (size_t)req * a.state_stride + a.tail_off);
    copy_row(tail + (size_t)(pos % a.R) * n, src, n, xs, nc, a.n_psplit, a.psplit_stride);
    return pos;
}

// At most one new token per request: the merges, the window rows and the
// tail update in one launch.  Blocks [0, nm) merge entries; block nm + g
// handles token g: its window row, and its projected row into the tail ring.
// The tail slot written (position p) is never one a merge of this call reads:
// an entry completed by the token at p reads positions p-R+1 .. p only.
__global__ __launch_bounds__(256) void post_decode_kernel(CompressArgs a, int nm)
{
    __shared__ __attribute__((aligned(16))) float xs[512];
    __shared__ float red[16];
    write_next_positions(a);
    if ((int)blockIdx.x < nm) {
        merge_entry(a, blockIdx.x, xs, red);
        return;
    }
    const int gtok = blockIdx.x - nm;
    const int pos = token_row(a, gtok, xs);
    __syncthreads();
    norm_rope_store(xs, red, a.c, a.r, a.gamma, a.eps, (double)pos, a.theta, a.out_win + (size_t)gtok * a.c);
}

// post_decode_kernel, then what a cache append of its outputs stores, in the
// same workgroups.  With at most one new token per request a request
// completes at most one entry per call, so each (request, block) receives one
// new record and its merge workgroup applies the block-scale rule alone.  The
// stores take the values this workgroup has just written (held in LDS), so
// they are those the separate append would read back.
__global__ __launch_bounds__(256) void post_decode_append_kernel(CompressArgs a, AppendArgs b, int nm)
{
    __shared__ __attribute__((aligned(16))) float xs[512];
    __shared__ __attribute__((aligned(16))) float ks[128];
    __shared__ float red[16];
    __shared__ float s_sh[2];
    write_next_positions(a);
    if ((int)blockIdx.x < nm) {
        const int2 re = locate_entry(a, blockIdx.x);
        if (re.x < 0) return;
        // the block's address and FP8 scale are loaded before the merge,
        // which does not need them (no other workgroup of this call writes
        // this block: it receives this one record)
        const int blk = re.y / b.epb, slot = re.y % b.epb;
        const int phys = b.block_table[(size_t)re.x * b.max_blocks + blk];
        uint8_t* block = (uint8_t*)b.kv + (size_t)phys * b.kv_block_bytes;
        const float s_old = (b.kv_fmt == 2 && slot > 0) ? *(const float*)block : 0.0f;
        merge_located(a, blockIdx.x, re.x, re.y, xs, red, ks);
        store_kv_records(b, block, slot, 1, xs, red, s_sh, true, s_old);
        // ks was complete at the merge's barrier before normalisation
        if (b.idx != nullptr && b.c_idx > 0) store_idx_key(b, phys, slot, ks);
        return;
    }
    const int gtok = blockIdx.x - nm;
    const int req = a.one_per_req ? gtok : find_request(a.cu_new, a.n_req, gtok);
    const int pos = token_row(a, gtok, xs);
    __syncthreads();
    norm_rope_store(xs, red, a.c, a.r, a.gamma, a.eps, (double)pos, a.theta, a.out_win + (size_t)gtok * a.c);
    store_window_row(b, req, pos, xs);
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------

int proj_parts(bool bf16, bool invariant, int n_rows)
{
    return bf16 && (n_rows <= 64 || invariant) ? PROJ_PARTS : 1;
}

size_t compress_workspace(bool bf16, bool invariant, int n_rows, int ncols)
{
    // a call with fewer rows may take more partials: at least 64 rows' worth
    // of partials whenever a call of up to n_rows rows can split
    const size_t rows = proj_parts(bf16, invariant, n_rows) > 1 ? (size_t)n_rows * PROJ_PARTS
                        : bf16 ? (size_t)max(n_rows, 64 * PROJ_PARTS) : (size_t)n_rows;
    return rows * (size_t)ncols * 4;
}

hipError_t launch_compress(hipStream_t st, const CompressArgs& args, const void* H, const void* W, const void* Wi,
                           int n_main, int d, bool bf16, int n_tokens, const AppendArgs* app)
{
    const int N = args.ncols, M = n_tokens;
    const GemmShape sh{d, N, 0, 0, 0, 0};
    CompressArgs a = args;
    a.n_psplit = 1;
    a.psplit_stride = 0;
    if (M > 0) {
        // batch-invariant layers: one kernel whatever the row count (its sums
        // for a row do not depend on the other rows)
        if (proj_parts(bf16, a.invariant, M) > 1 && d % (PROJ_PARTS * MmaBF16::K) == 0) {
            a.n_psplit = PROJ_PARTS;
            a.psplit_stride = (size_t)M * N;
            const dim3 grid((N + 15) / 16, (M + 15) / 16, PROJ_PARTS);
            if (d <= 4 * PROJ_PARTS * PK_KB)
                proj_ksplit<4><<<grid, 256, 0, st>>>((const uint16_t*)H, (const uint16_t*)W, (const uint16_t*)Wi, n_main,
                                                     N, M, d, a.P);
            else
                proj_ksplit<8><<<grid, 512, 0, st>>>((const uint16_t*)H, (const uint16_t*)W, (const uint16_t*)Wi, n_main,
                                                     N, M, d, a.P);
        } else if (M <= 64 || a.invariant) {
            dim3 grid((N + 15) / 16, (M + 15) / 16);
            if (bf16 && d % (PL_NW * MmaBF16::K) == 0 && d >= PL_NW * PL_KB)   // whole steps, full batches
                proj_small_lds<<<grid, 64 * PL_NW, 0, st>>>((const uint16_t*)H, (const uint16_t*)W, (const uint16_t*)Wi,
                                                            n_main, N, M, d, a.P, sh);
            else if (bf16)
                proj_small<uint16_t, MmaBF16, 4><<<grid, 256, 0, st>>>((const uint16_t*)H, (const uint16_t*)W,
                                                                       (const uint16_t*)Wi, n_main, N, M, d, a.P, sh);
            else
                proj_small<float, MmaF32, 4><<<grid, 256, 0, st>>>((const float*)H, (const float*)W, (const float*)Wi,
                                                                   n_main, N, M, d, a.P, sh);
        } else if (use_proj_lds(bf16, M, N, d, 1, H, W, Wi, d)) {
            dim3 grid((N + PG_BN - 1) / PG_BN, (M + PG_BM - 1) / PG_BM);
            proj_lds<<<grid, 256, 0, st>>>((const uint16_t*)H, (const uint16_t*)W, (const uint16_t*)Wi, n_main, N, M, d,
                                           a.P, sh);
        } else {
            dim3 grid((N + 127) / 128, (M + 127) / 128);
            if (bf16)
                proj_large<uint16_t, MmaBF16><<<grid, 256, 0, st>>>((const uint16_t*)H, (const uint16_t*)W,
                                                                    (const uint16_t*)Wi, n_main, N, M, d, a.P, sh);
            else
                proj_large<float, MmaF32><<<grid, 256, 0, st>>>((const float*)H, (const float*)W, (const float*)Wi,
                                                                n_main, N, M, d, a.P, sh);
        }
    }
    const int nm = a.max_entries > 0 ? a.max_entries : 1;
    if (a.max_new <= 1) {
        CompressArgs b = a;
        b.one_per_req = M == a.n_req;                           // at most one each, n_req of them
        if (app != nullptr)
            post_decode_append_kernel<<<nm + M, 256, 0, st>>>(b, *app, nm);
        else
            post_decode_kernel<<<nm + M, 256, 0, st>>>(b, nm);
        return hipGetLastError();
    }
    merge_kernel<<<nm, 256, 0, st>>>(a);
    if (M > 0) {
        window_rows_kernel<<<M, 256, 0, st>>>(a);
        tail_update_kernel<<<dim3(a.R, a.n_req), 256, 0, st>>>(a);
    }
    if (app != nullptr) {
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        return launch_append(st, *app);
    }
    return hipGetLastError();
}

}  // namespace csa

namespace csa {

// Y[M x N] = X[M x K] . W^T per group (grid z), W [groups x N x K].  Few rows:
// the small-row kernel (16 waves when K allows), else the 128 x 128 tiles.
hipError_t launch_linear(hipStream_t st, bool bf16, int M, int K, int N, int groups, const void* X, const void* W,
                         void* Y, bool out_bf16)
{
    if (M <= 0 || N <= 0 || groups <= 0) return hipSuccess;
    const GemmShape sh{K * groups, N * groups, out_bf16 ? 1 : 0, (size_t)K, (size_t)N * K, (size_t)N};
    if (M <= 64) {
        dim3 grid((N + 15) / 16, (M + 15) / 16, groups);
        // operands through LDS only when each wave gets at least one full batch of K
        if (bf16 && K % (PL_NW * MmaBF16::K) == 0 && K >= PL_NW * PL_KB)
            proj_small_lds<<<grid, 64 * PL_NW, 0, st>>>((const uint16_t*)X, (const uint16_t*)W, (const uint16_t*)W, N,
                                                        N, M, K, Y, sh);
        else if (bf16)
            proj_small<uint16_t, MmaBF16, 4><<<grid, 256, 0, st>>>((const uint16_t*)X, (const uint16_t*)W,
                                                                   (const uint16_t*)W, N, N, M, K, Y, sh);
        else
            proj_small<float, MmaF32, 4><<<grid, 256, 0, st>>>((const float*)X, (const float*)W, (const float*)W, N,
                                                               N, M, K, Y, sh);
    } else if (use_proj_lds(bf16, M, N, K, groups, X, W, W, K * groups)) {
        dim3 grid((N + PG_BN - 1) / PG_BN, (M + PG_BM - 1) / PG_BM, groups);
        proj_lds<<<grid, 256, 0, st>>>((const uint16_t*)X, (const uint16_t*)W, (const uint16_t*)W, N, N, M, K, Y, sh);
    } else {
        dim3 grid((N + 127) / 128, (M + 127) / 128, groups);
        if (bf16)
            proj_large<uint16_t, MmaBF16><<<grid, 256, 0, st>>>((const uint16_t*)X, (const uint16_t*)W,
                                                                (const uint16_t*)W, N, N, M, K, Y, sh);
        else
            proj_large<float, MmaF32><<<grid, 256, 0, st>>>((const float*)X, (const float*)W, (const float*)W, N, N,
                                                            M, K, Y, sh);
    }
    return hipGetLastError();
}

}  // namespace csa
