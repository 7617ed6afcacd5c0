// Device helpers shared by the gfx950 kernels: number formats, MFMA fragment
// steps, RoPE tables, batch bookkeeping and wave/block reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA_DEV __device__ __forceinline__

namespace csa {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

CSA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest even on the dropped 16 bits (inputs are finite).
CSA_DEV uint16_t f32_to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two floats to bf16 (round to nearest even) in one dword, low half first;
// one hardware conversion.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
CSA_DEV uint32_t pack_bf16x2(float a, float b)
{
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Order-preserving 16-bit key of a bf16 score (sign-magnitude flip; -0 and
// +0 share the key): larger scores have larger keys.
CSA_DEV uint32_t key16(uint32_t b)
{
    if ((b & 0x7FFFu) == 0u) b = 0u;
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// OCP E4M3FN -> fp32 (exact).  0x7F/0xFF (NaN) never occur in stored data.
CSA_DEV float e4m3_to_f32(uint32_t q)
{
    uint32_t s = (q & 0x80u) << 24;
    uint32_t E = (q >> 3) & 15u, M = q & 7u;
    float v = (E == 0) ? (float)M * 0.001953125f                                 // M * 2^-9
                       : __uint_as_float(((E + 120u) << 23) | (M << 20));       // 2^(E-7) * (1 + M/8)
    return __uint_as_float(__float_as_uint(v) | s);
}

// Four E4M3FN codes (one dword) to four bf16 values (two dwords), exactly,
// with gfx950's conversion instruction (OCP E4M3; checked against
// e4m3_to_f32 for every finite code).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
CSA_DEV uint2 e4m3x4_to_bf16x4(uint32_t codes)
{
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes, 1.0f, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// E4M3FN code of an fp32 value: round to nearest even, saturate to +-448,
// a zero result is stored as +0.
CSA_DEV uint32_t f32_to_e4m3(float v)
{
    uint32_t s = (__float_as_uint(v) >> 24) & 0x80u;
    float a = fabsf(v);
    if (a >= 448.0f) return s | 0x7Eu;
    if (a < 0.015625f) {                       // below 2^-6: spacing 2^-9
        float m = rintf(a * 512.0f);           // exact scaling, then RNE
        if (m == 0.0f) return 0u;
        return s | (uint32_t)m;                // m == 8 is the smallest normal 0x08
    }
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // a in [2^e, 2^(e+1))
    float m = rintf(ldexpf(a, 3 - e));         // in [8, 16]
    if (m == 16.0f) { m = 8.0f; e += 1; }
    if (e > 8 || (e == 8 && m > 14.0f)) return s | 0x7Eu;
    return s | ((uint32_t)(e + 7) << 3) | ((uint32_t)m - 8u);
}

// OCP E2M1 magnitude table and encoder (round to nearest even, saturate at 6).
CSA_DEV float e2m1_to_f32(uint32_t q)
{
    uint32_t mag = q & 7u;
    float v = (mag < 4u) ? 0.5f * (float)mag : (mag == 4u ? 2.0f : mag == 5u ? 3.0f : mag == 6u ? 4.0f : 6.0f);
    return (q & 8u) ? -v : v;
}

CSA_DEV uint32_t f32_to_e2m1(float v)
{
    float a = fabsf(v);
    uint32_t code;
    if (a >= 6.0f) code = 7u;
    else if (a < 2.0f) code = (uint32_t)rintf(a * 2.0f);                 // 0..4 (4 == 2.0)
    else if (a < 4.0f) { float m = rintf(a); code = m == 2.0f ? 4u : (m == 3.0f ? 5u : 6u); }
    else { float m = rintf(a * 0.5f); code = m == 2.0f ? 6u : 7u; }
    if (code == 0u) return 0u;
    return code | ((v < 0.0f) ? 8u : 0u);
}

// E8M0 code of an MX block whose largest magnitude is amax: the exponent
// floor(log2 amax) - 2 (E2M1's largest binade), biased by 127.
CSA_DEV int mx_scale_code(float amax)
{
    if (!(amax > 0.0f)) return 127;
    int e;
    frexpf(amax, &e);                          // amax in [2^(e-1), 2^e)
    int code = (e - 1) - 2 + 127;
    return code < 0 ? 0 : (code > 254 ? 254 : code);
}

// ---------------------------------------------------------------------------
// MFMA steps.  A "fragment" is 16 bytes per lane: 8 bf16 or 4 fp32 values of
// one row (A) / one column (B).  In a 16x16 tile, lane l holds row (col) l%16
// and lane group g = l/16 holds its own slice of the contraction index; the
// same (g, element) -> k mapping is used for A and B, so the sum covers every
// k once.  The accumulator layout is the hardware's: lane l holds
// D[4*g + i][l % 16], i = 0..3.
// ---------------------------------------------------------------------------

struct MmaBF16 {
    static constexpr int K = 32;               // contraction length of one step (8 per lane group)
    static CSA_DEV f32x4_t step(uint4 a, uint4 b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};

struct MmaF32 {
    static constexpr int K = 16;               // 4 per lane group, one MFMA per element
    static CSA_DEV f32x4_t step(uint4 a, uint4 b, f32x4_t c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
        return c;
    }
};

CSA_DEV f32x4_t zero4() { f32x4_t z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Loads from global memory.  The pointer is cast to the global address space
// so that the load is a global (not flat) instruction even when the address
// was read back from LDS: flat loads also count against the LDS wait
// counter, which would make every LDS wait also wait for them.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#define CSA_GLOBAL __attribute__((address_space(1)))
#define CSA_LDS __attribute__((address_space(3)))

// 16-byte load as one dwordx4 (the address must be 16-byte aligned).
CSA_DEV uint4 ld16(const void* p)
{
    u32x4_t v = *(const CSA_GLOBAL u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 8-byte load (8-byte aligned).
CSA_DEV uint2 ld8(const void* p)
{
    u32x2_t v = *(const CSA_GLOBAL u32x2_t*)p;
    return make_uint2(v.x, v.y);
}

CSA_DEV uint4 sel16(bool keep, uint4 v)
{
    return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

// ---------------------------------------------------------------------------
// batch bookkeeping
// ---------------------------------------------------------------------------

// Request owning global token row g: the largest r with cu_new[r] <= g.
CSA_DEV int find_request(const int32_t* cu_new, int n_req, int g)
{
    int lo = 0, hi = n_req - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu_new[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// reductions (fixed order: butterfly over the wave, then waves in index order)
// ---------------------------------------------------------------------------

// Max / sum of v over lanes l and l ^ 16 (l ^ 32): gfx950's permlane swaps
// hand every lane both values, lower lane first, so both lanes of a pair
// get the same result.
CSA_DEV float xmax16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
CSA_DEV float xsum16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
CSA_DEV float xmax32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
CSA_DEV float xsum32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

CSA_DEV float wave_sum(float v)
{
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

CSA_DEV float wave_max(float v)
{
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Sum over the block (blockDim.x a multiple of 64, <= 1024); every thread gets
// the total.  `red` is LDS scratch of >= 16 floats.
CSA_DEV float block_sum(float v, float* red)
{
    int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}

CSA_DEV float block_max(float v, float* red)
{
    int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = red[0];
    for (int i = 1; i < nw; ++i) t = fmaxf(t, red[i]);
    return t;
}

// RoPE frequency of pair j of r rotary channels, theta^(-2j/r) (the same
// expression is used on the host to fill frequency tables).
__host__ __device__ inline double rope_inv_freq(int j, int r, double theta)
{
    return exp2(-2.0 * (double)j / (double)r * log2(theta));
}

// cos / sin of pos * inv_freq: the angle is formed and reduced to [-pi, pi]
// in double (positions reach millions), then its sine and cosine are taken
// in fp32.
CSA_DEV void rope_cs_f(double pos, double inv_freq, float* cs, float* sn)
{
    double ang = pos * inv_freq;
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
    sincosf((float)ang, sn, cs);
}

// The same for pair j of r rotary channels at position pos.
CSA_DEV void rope_cs(double pos, int j, int r, float theta, float* cs, float* sn)
{
    const double inv_freq = rope_inv_freq(j, r, (double)theta);
    double ang = pos * inv_freq;
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
    sincosf((float)ang, sn, cs);
}

// Request of global token row g, found by all threads of the block together:
// cu_new is staged in LDS (sh, >= n_req + 1 ints when n_req < cap), then
// searched there (in global memory otherwise).  Every thread of the block
// must call it.
CSA_DEV int find_request_block(const int32_t* cu_new, int n_req, int g, int* sh, int cap = 1024)
{
    if (n_req >= cap) return find_request(cu_new, n_req, g);
    for (int i = threadIdx.x; i <= n_req; i += blockDim.x) sh[i] = cu_new[i];
    __syncthreads();
    int lo = 0, hi = n_req - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (sh[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace csa
