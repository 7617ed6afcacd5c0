/*
 * CPU oracle for the DeepSeek-V4 hybrid compressed attention path (CSA / HCA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library: everything here is
 * written from the pages' definitions and from the OCP number-format specs.
 *
 * Arithmetic is fp64 except where a stored format forces a decision (a
 * quantised code, a block scale): those decisions are taken in fp32, exactly
 * as the format rules below state, so that a GPU fed the same fp32 inputs must
 * produce the same bytes.
 *
 * Sources (page title, section):
 *  [DD] "DeepSeek-V4 内部机制" (LLM-101-CN deep dive): §1.2 Steps 1-3 (CSA
 *       compressor, Lightning Indexer, top-k), §1.3 (HCA), §1.4 table and the
 *       sink equation for s_{h,i,j}, §1.5 (mixed-precision KV), §6.2 (FP4
 *       indexer, BF16 scores), §7 (state cache + paged cache, lcm block).
 *  [YP] yunpan.plus explainer, "CSA / HCA" section, eqs. (6)-(11).
 *  [AD] m.admirer.cn article, CSA/HCA section (k=512/1024, 128-token window,
 *       64 RoPE dims, BF16+FP8 KV, lcm(4,128) block with 32 CSA / 1 HCA entries).
 *
 * Parity pins for every function are in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bfloat16: the top 16 bits of an IEEE binary32, rounded to nearest, ties to
 * even on the dropped 16 bits.  Inputs are finite. */
uint16_t orc_bf16_bits(float x)
{
    uint32_t u = f32_bits(x);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

float orc_bf16_value(uint16_t b) { return bits_f32(((uint32_t)b) << 16); }

/* Round a double straight to bfloat16 (one rounding, nearest-even), used for
 * index scores whose exact value the oracle holds in fp64. */
uint16_t orc_bf16_bits_from_double(double v)
{
    if (v == 0.0) return 0; /* -0 and +0 both become +0 */
    int sgn = v < 0;
    double a = fabs(v);
    int e;
    frexp(a, &e);               /* a = f * 2^e, f in [0.5,1) -> a in [2^(e-1), 2^e) */
    int ex = e - 1;             /* a in [2^ex, 2^(ex+1)) */
    if (ex < -126) ex = -126;   /* subnormal spacing */
    double ulp = ldexp(1.0, ex - 7);   /* 8 significant bits */
    double q = a / ulp;         /* exact: power-of-two scaling */
    double fl = floor(q);
    double rem = q - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * ulp;
    float rf = (float)r;        /* exact: r has <= 8 significant bits */
    uint16_t b = (uint16_t)(f32_bits(rf) >> 16);
    return sgn ? (uint16_t)(b | 0x8000u) : b;
}

/* OCP 8-bit FP, E4M3FN variant: bias 7, no infinities, S.1111.111 is NaN,
 * largest finite 448 = 1.75*2^8, subnormals m*2^-9.  Encoding rounds to
 * nearest, ties to even, and saturates to +-448. */
double orc_e4m3_decode(uint8_t q)
{
    int s = q >> 7, E = (q >> 3) & 15, M = q & 7;
    double v;
    if (E == 15 && M == 7) return NAN;
    if (E == 0) v = ldexp((double)M, -9);
    else v = ldexp(1.0 + M / 8.0, E - 7);
    return s ? -v : v;
}

static double round_half_even(double q)
{
    double fl = floor(q), rem = q - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    return fl;
}

uint8_t orc_e4m3_encode(float v)
{
    double a = fabs((double)v);
    uint8_t s = (v < 0) ? 0x80 : 0x00;
    if (a >= 448.0) return (uint8_t)(s | 0x7E);
    int e;
    if (a < ldexp(1.0, -6)) {               /* subnormal range: spacing 2^-9 */
        double m = round_half_even(a / ldexp(1.0, -9));
        if (m >= 8.0) return (uint8_t)(s | 0x08);   /* rounds up to 2^-6 */
        if (m == 0.0) return 0;                     /* -0 is stored as +0 */
        return (uint8_t)(s | (uint8_t)m);
    }
    frexp(a, &e);
    int ex = e - 1;                         /* a in [2^ex, 2^(ex+1)) */
    double m = round_half_even(a / ldexp(1.0, ex - 3));   /* in [8,16] */
    if (m == 16.0) { m = 8.0; ex += 1; }
    double r = m * ldexp(1.0, ex - 3);
    if (r > 448.0) return (uint8_t)(s | 0x7E);
    int E = ex + 7, M = (int)m - 8;
    return (uint8_t)(s | (E << 3) | M);
}

/* OCP E2M1 (FP4): bias 1, values 0,0.5,1,1.5,2,3,4,6; RNE, saturating to 6. */
double orc_e2m1_decode(uint8_t q)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[q & 7];
    return (q & 8) ? -v : v;
}

uint8_t orc_e2m1_encode(float v)
{
    double a = fabs((double)v);
    uint8_t s = (v < 0) ? 8 : 0;
    int code;
    if (a >= 6.0) code = 7;
    else if (a < 2.0) {                    /* spacing 0.5 below 2 */
        double m = round_half_even(a / 0.5);   /* 0..4 */
        code = (int)m;                     /* 0,1,2,3 -> 0,.5,1,1.5 ; 4 -> 2.0 */
    } else if (a < 4.0) {                  /* spacing 1 on [2,4) */
        double m = round_half_even(a);     /* 2,3,4 */
        code = (m == 2.0) ? 4 : (m == 3.0) ? 5 : 6;
    } else {                               /* spacing 2 on [4,6) */
        double m = round_half_even(a / 2.0);   /* 2 or 3 */
        code = (m == 2.0) ? 6 : 7;
    }
    if (code == 0) return 0;
    return (uint8_t)(s | code);
}

/* OCP MX shared scale (E8M0) for an E2M1 block: X = floor(log2(amax)) - 2,
 * where 2 is the exponent of E2M1's largest normal (6 = 1.5*2^2).  Returned
 * as the biased code X+127, clamped to [0,254]; an all-zero block takes
 * code 127 (scale 1). */
int orc_mx_scale_code(float amax)
{
    if (!(amax > 0.0f)) return 127;
    int e;
    frexp((double)amax, &e);    /* amax in [2^(e-1), 2^e) */
    int X = (e - 1) - 2;
    int code = X + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return code;
}

/* Quantise n (multiple of 32) values to MXFP4: 32-element blocks, one E8M0
 * code each, elements E2M1 (two per byte, element 2j in the low nibble). */
void orc_mxfp4_pack(int n, const float* x, uint8_t* codes, uint8_t* scales)
{
    for (int b = 0; b < n / 32; ++b) {
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            float a = fabsf(x[b * 32 + j]);
            if (a > amax) amax = a;
        }
        int sc = orc_mx_scale_code(amax);
        scales[b] = (uint8_t)sc;
        double inv = ldexp(1.0, 127 - sc);
        for (int j = 0; j < 32; j += 2) {
            float v0 = (float)((double)x[b * 32 + j] * inv);      /* exact */
            float v1 = (float)((double)x[b * 32 + j + 1] * inv);
            codes[(b * 32 + j) / 2] = (uint8_t)(orc_e2m1_encode(v0) | (orc_e2m1_encode(v1) << 4));
        }
    }
}

void orc_mxfp4_unpack(int n, const uint8_t* codes, const uint8_t* scales, double* out)
{
    for (int i = 0; i < n; ++i) {
        uint8_t byte = codes[i / 2];
        uint8_t q = (i & 1) ? (byte >> 4) : (byte & 15);
        out[i] = orc_e2m1_decode(q) * ldexp(1.0, (int)scales[i / 32] - 127);
    }
}

/* ------------------------------------------------------------------------ */
/* a1: token-level compressor  ([DD] §1.2 Step 1; [YP] eqs. (6),(7); HCA:   */
/*     [DD] §1.3, [YP] eqs. (10),(11))                                       */
/* ------------------------------------------------------------------------ */

/*
 * One request, raw tokens 0..n-1, projected rows given (row-major [n x c]).
 * Entry i merges the m rows of block i (the "a" half) and, with overlap, the
 * m rows of block i-1 (the "b" half).  For each channel independently the
 * 2m logits Z+B are soft-maxed together and the entry is the S-weighted sum
 * of the matching C rows.  Entry 0 has no block -1: its softmax runs over its
 * m a-rows only.  Without overlap (HCA) only Ca, Za, Ba are read.
 * Writes floor(n/m) entries.
 */
void orc_compress(int n, int c, int m, int overlap,
                  const double* Ca, const double* Cb, const double* Za, const double* Zb,
                  const double* Ba, const double* Bb, double* out)
{
    int ne = n / m;
    double* lg = (double*)malloc(sizeof(double) * 2 * m);
    for (int i = 0; i < ne; ++i) {
        int has_b = overlap && i >= 1;
        for (int ch = 0; ch < c; ++ch) {
            double mx = -INFINITY;
            for (int r = 0; r < m; ++r) {
                lg[r] = Za[(size_t)(m * i + r) * c + ch] + Ba[(size_t)r * c + ch];
                if (lg[r] > mx) mx = lg[r];
            }
            if (has_b)
                for (int r = 0; r < m; ++r) {
                    lg[m + r] = Zb[(size_t)(m * (i - 1) + r) * c + ch] + Bb[(size_t)r * c + ch];
                    if (lg[m + r] > mx) mx = lg[m + r];
                }
            double den = 0.0;
            for (int r = 0; r < (has_b ? 2 * m : m); ++r) den += exp(lg[r] - mx);
            double acc = 0.0;
            for (int r = 0; r < m; ++r)
                acc += exp(lg[r] - mx) / den * Ca[(size_t)(m * i + r) * c + ch];
            if (has_b)
                for (int r = 0; r < m; ++r)
                    acc += exp(lg[m + r] - mx) / den * Cb[(size_t)(m * (i - 1) + r) * c + ch];
            out[(size_t)i * c + ch] = acc;
        }
    }
    free(lg);
}

/* The softmax weights themselves, for the row-stochastic pin:
 * S[i][r][ch] for r < 2m (b-half rows m..2m-1 are 0 when absent). */
void orc_compress_weights(int n, int c, int m, int overlap,
                          const double* Za, const double* Zb, const double* Ba, const double* Bb,
                          double* S)
{
    int ne = n / m;
    for (int i = 0; i < ne; ++i) {
        int has_b = overlap && i >= 1;
        for (int ch = 0; ch < c; ++ch) {
            double lg[512];
            double mx = -INFINITY;
            for (int r = 0; r < m; ++r) {
                lg[r] = Za[(size_t)(m * i + r) * c + ch] + Ba[(size_t)r * c + ch];
                if (lg[r] > mx) mx = lg[r];
            }
            for (int r = 0; r < m; ++r) {
                lg[m + r] = has_b ? Zb[(size_t)(m * (i - 1) + r) * c + ch] + Bb[(size_t)r * c + ch] : -INFINITY;
                if (lg[m + r] > mx) mx = lg[m + r];
            }
            double den = 0.0;
            for (int r = 0; r < 2 * m; ++r) den += exp(lg[r] - mx);
            for (int r = 0; r < 2 * m; ++r)
                S[((size_t)i * 2 * m + r) * c + ch] = exp(lg[r] - mx) / den;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q / KV-entry RMSNorm and partial RoPE ([DD] §1.4 table)                   */
/* ------------------------------------------------------------------------ */

/* y = gamma * x / sqrt(mean(x^2) + eps) over c channels. */
void orc_rmsnorm(int rows, int c, const double* x, const double* gamma, double eps, double* y)
{
    for (int i = 0; i < rows; ++i) {
        double ss = 0.0;
        for (int k = 0; k < c; ++k) ss += x[(size_t)i * c + k] * x[(size_t)i * c + k];
        double inv = 1.0 / sqrt(ss / c + eps);
        for (int k = 0; k < c; ++k) y[(size_t)i * c + k] = gamma[k] * x[(size_t)i * c + k] * inv;
    }
}

/* Rotate the last r channels of each row as r/2 interleaved pairs
 * (c-r+2j, c-r+2j+1) by angle pos[row] * theta^(-2j/r). */
void orc_rope(int rows, int c, int r, const double* pos, double theta, double* x)
{
    for (int i = 0; i < rows; ++i)
        for (int j = 0; j < r / 2; ++j) {
            double ang = pos[i] * pow(theta, -2.0 * j / r);
            double cs = cos(ang), sn = sin(ang);
            double* p = x + (size_t)i * c + (c - r) + 2 * j;
            double a = p[0], b = p[1];
            p[0] = a * cs - b * sn;
            p[1] = a * sn + b * cs;
        }
}

/* ------------------------------------------------------------------------ */
/* a3: Lightning Indexer scores ([DD] §1.2 Step 2; [YP] eq. (8))             */
/* ------------------------------------------------------------------------ */

/*
 * I[t][s] = sum_h w[t][h] * max(0, qI[t][h] . K[s]) for s < n_vis[t], the
 * exact value rounded once to the score format (fmt 0: fp32, 1: bf16, see
 * [DD] §6.2: scores are kept in BF16 because the sort is precision
 * sensitive).  -0 becomes +0.  Entries s >= n_vis[t] are left untouched.
 * One request: queries t share the key array K [E x cI].
 */
void orc_index_scores(int T, int nh, int cI, const double* qI, const double* w,
                      const int* n_vis, int E, const double* K, int fmt, float* out, int ld)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        int V = n_vis[t] < E ? n_vis[t] : E;
        for (int s = 0; s < V; ++s) {
            double I = 0.0;
            for (int h = 0; h < nh; ++h) {
                double d = 0.0;
                const double* q = qI + ((size_t)t * nh + h) * cI;
                const double* k = K + (size_t)s * cI;
                for (int j = 0; j < cI; ++j) d += q[j] * k[j];
                I += w[(size_t)t * nh + h] * (d > 0.0 ? d : 0.0);
            }
            float v;
            if (fmt == 1) v = orc_bf16_value(orc_bf16_bits_from_double(I));
            else v = (float)I;
            if (v == 0.0f) v = 0.0f;
            out[(size_t)t * ld + s] = v;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* a4: top-k selector ([DD] §1.2 Step 2; [AD]: k = 512 Flash, 1024 Pro)      */
/* ------------------------------------------------------------------------ */

typedef struct { float v; int s; } orc_pair;

static int cmp_desc_then_index(const void* a, const void* b)
{
    const orc_pair* x = (const orc_pair*)a;
    const orc_pair* y = (const orc_pair*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s > y->s) - (x->s < y->s);
}

static int cmp_int(const void* a, const void* b)
{
    int x = *(const int*)a, y = *(const int*)b;
    return (x > y) - (x < y);
}

/* Per row: sort s in [0, n_valid) by (score desc, index asc), keep the first
 * min(k, n_valid), emit them in ascending index order, pad with -1. */
void orc_topk(int T, const float* scores, int ld, const int* n_valid, int k, int* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        int V = n_valid[t];
        orc_pair* p = (orc_pair*)malloc(sizeof(orc_pair) * (V > 0 ? V : 1));
        for (int s = 0; s < V; ++s) { p[s].v = scores[(size_t)t * ld + s]; p[s].s = s; }
        qsort(p, V, sizeof(orc_pair), cmp_desc_then_index);
        int kk = V < k ? V : k;
        int* o = out + (size_t)t * k;
        for (int j = 0; j < kk; ++j) o[j] = p[j].s;
        qsort(o, kk, sizeof(int), cmp_int);
        for (int j = kk; j < k; ++j) o[j] = -1;
        free(p);
    }
}

/* ------------------------------------------------------------------------ */
/* a5 / a6: shared-KV MQA with window and sink ([DD] §1.2 Step 2, §1.3,      */
/*          §1.4 table and the s_{h,i,j} equation; [YP] eq. (9))             */
/* ------------------------------------------------------------------------ */

/*
 * One query at position pos with n_h heads.  q_raw [nh x c] is RMS-normalised
 * per head (gamma_q, eps) and rotated at +pos on its last r channels.  The
 * rows X [nrows x c] (selected compressed entries and raw window rows, already
 * in their final normalised/rotated form) are both key and value.  For head h:
 *   z_j = scale * q_h . X_j,   p_j = exp(z_j) / (sum_j' exp(z_j') + exp(sink_h))
 *   o_h = sum_j p_j X_j, then the last r channels rotated at -pos.
 */
void orc_attend(int nh, int c, int r, const double* q_raw, const double* gamma_q, double eps,
                double pos, double theta, double scale, int nrows, const double* X,
                const double* sink, double* out)
{
    double* q = (double*)malloc(sizeof(double) * c);
    double* z = (double*)malloc(sizeof(double) * (nrows > 0 ? nrows : 1));
    for (int h = 0; h < nh; ++h) {
        orc_rmsnorm(1, c, q_raw + (size_t)h * c, gamma_q, eps, q);
        orc_rope(1, c, r, &pos, theta, q);
        double M = sink[h];
        for (int j = 0; j < nrows; ++j) {
            double d = 0.0;
            for (int k = 0; k < c; ++k) d += q[k] * X[(size_t)j * c + k];
            z[j] = scale * d;
            if (z[j] > M) M = z[j];
        }
        double D = exp(sink[h] - M);
        for (int j = 0; j < nrows; ++j) D += exp(z[j] - M);
        double* o = out + (size_t)h * c;
        for (int k = 0; k < c; ++k) o[k] = 0.0;
        for (int j = 0; j < nrows; ++j) {
            double p = exp(z[j] - M) / D;
            for (int k = 0; k < c; ++k) o[k] += p * X[(size_t)j * c + k];
        }
        double npos = -pos;
        orc_rope(1, c, r, &npos, theta, o);
    }
    free(q);
    free(z);
}

/*
 * Batched form over the queries of one request.  For query t the rows are
 * entries[sel[t][0..k)] (skipping -1; dense HCA passes sel == NULL and uses
 * entries 0..n_ent[t]-1) followed by window rows win[j] for
 * max(0, pos_t-n_win+1) <= j <= pos_t.
 */
void orc_attend_batch(int T, int nh, int c, int r, const double* q_raw, const double* gamma_q,
                      double eps, const double* pos, double theta, double scale,
                      const double* entries, const int* sel, int k, const int* n_ent,
                      const double* win, int n_win, const double* sink, double* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        int p = (int)pos[t];
        int w0 = p - n_win + 1 < 0 ? 0 : p - n_win + 1;
        int nsel = 0;
        if (sel) { for (int j = 0; j < k; ++j) if (sel[(size_t)t * k + j] >= 0) ++nsel; }
        else nsel = n_ent[t];
        int nrows = nsel + (p - w0 + 1);
        double* X = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1) * c);
        int row = 0;
        if (sel) {
            for (int j = 0; j < k; ++j) {
                int s = sel[(size_t)t * k + j];
                if (s < 0) continue;
                memcpy(X + (size_t)row * c, entries + (size_t)s * c, sizeof(double) * c);
                ++row;
            }
        } else {
            for (int s = 0; s < nsel; ++s, ++row)
                memcpy(X + (size_t)row * c, entries + (size_t)s * c, sizeof(double) * c);
        }
        for (int j = w0; j <= p; ++j, ++row)
            memcpy(X + (size_t)row * c, win + (size_t)j * c, sizeof(double) * c);
        orc_attend(nh, c, r, q_raw + (size_t)t * nh * c, gamma_q, eps, pos[t], theta, scale,
                   nrows, X, sink, out + (size_t)t * nh * c);
        free(X);
    }
}

/* ------------------------------------------------------------------------ */
/* a2: storage formats of the paged ("classic") cache ([DD] §1.5, §7; [AD])  */
/* ------------------------------------------------------------------------ */

/*
 * Mixed FP8/BF16 entry block: a 64-byte header holding the block's fp32 scale
 * s (bytes 0..3; the rest zero), then epb entry records of (c-r) E4M3FN codes
 * followed by r bf16 values (the RoPE channels).  The fp8 part decodes to
 * code * s.
 *
 * Append rule, applied once per call to the new entries x[0..n_new) landing
 * in slots first..first+n_new-1 of one block (all decisions in fp32):
 *   s_old = 0 if first == 0 (fresh block) else the stored scale;
 *   amax  = max |x| over the new entries' fp8 channels;
 *   s     = max(s_old, amax / 448);
 *   if s > s_old, every earlier slot j < first is re-encoded:
 *       code' = E4M3(E4M3value(code) * s_old / s)   (the product in fp32,
 *       then one fp32 division);
 *   new entries: code = E4M3(x / s) (fp32 division); s == 0 stores code 0.
 * RoPE channels are stored as bf16(x).
 */
void orc_fp8_block_append(int c, int r, int epb, uint8_t* block, int first, int n_new, const float* x)
{
    int nf = c - r;
    int rec = nf + 2 * r;
    float s_old = 0.0f;
    if (first > 0) memcpy(&s_old, block, 4);
    float amax = 0.0f;
    for (int e = 0; e < n_new; ++e)
        for (int k = 0; k < nf; ++k) {
            float a = fabsf(x[(size_t)e * c + k]);
            if (a > amax) amax = a;
        }
    float s_new = amax / 448.0f;
    float s = s_old > s_new ? s_old : s_new;
    if (s > s_old && first > 0) {
        for (int j = 0; j < first; ++j) {
            uint8_t* codes = block + 64 + (size_t)j * rec;
            for (int k = 0; k < nf; ++k) {
                float old = (float)orc_e4m3_decode(codes[k]) * s_old;
                codes[k] = orc_e4m3_encode(old / s);
            }
        }
    }
    if (first == 0) memset(block, 0, 64);
    memcpy(block, &s, 4);
    for (int e = 0; e < n_new; ++e) {
        uint8_t* recp = block + 64 + (size_t)(first + e) * rec;
        for (int k = 0; k < nf; ++k)
            recp[k] = (s > 0.0f) ? orc_e4m3_encode(x[(size_t)e * c + k] / s) : 0;
        for (int k = 0; k < r; ++k) {
            uint16_t b = orc_bf16_bits(x[(size_t)e * c + nf + k]);
            memcpy(recp + nf + 2 * k, &b, 2);
        }
    }
}

/* Decode one mixed FP8/BF16 entry record of a block into fp64. */
void orc_fp8_block_decode(int c, int r, int epb, const uint8_t* block, int slot, double* out)
{
    int nf = c - r;
    int rec = nf + 2 * r;
    float s;
    memcpy(&s, block, 4);
    const uint8_t* recp = block + 64 + (size_t)slot * rec;
    for (int k = 0; k < nf; ++k) out[k] = orc_e4m3_decode(recp[k]) * (double)s;
    for (int k = 0; k < r; ++k) {
        uint16_t b;
        memcpy(&b, recp + nf + 2 * k, 2);
        out[nf + k] = orc_bf16_value(b);
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
