/*
 * halo_oracle.c -- plain, slow CPU oracle for the Hadamard-rotated low-precision
 * linear layer (forward Y = X W^T, backward dX = dY W and dW = dY^T X).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load this library.  It shares no code, header, table or helper
 * with the GPU library, and the GPU library never calls it.
 *
 * Pages followed (cited by title and section):
 *   [QWHA]  "QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术"
 *           s2.1  the Walsh-Hadamard matrix by the Kronecker (Sylvester) recursion, with
 *                 the 1/sqrt(2) factor per level, i.e. an orthonormal transform;
 *           s2.2  the iterative in-place butterfly (half-width h = 1, 2, 4, ...) followed
 *                 by division of every element by sqrt(n); the absmax k-bit quantiser with
 *                 qmax = 2^(bits-1) - 1, round-to-nearest (numpy's, i.e. ties to even)
 *                 and clipping to [-qmax, qmax];
 *           s3.1  the transform applied blockwise to large matrices.
 *           s5    input lengths padded with zeros up to the transform length; stochastic
 *                 rounding (round down, then up with probability equal to the fraction) to
 *                 reduce the quantiser's bias.
 *   [HALO]  "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs"
 *           abstract: Hadamard rotations in the forward and in the backward pass, and every
 *           large matrix product of both passes computed in low precision;
 *           method section, key design 2: the low-precision type is INT8 or FP8.
 *   [P1]    "企业官网建设流程全解析" (a HALO overview) s4.2: every node initialises the Hadamard
 *           matrix from the same random seed, i.e. a randomised transform H D with a seeded
 *           diagonal D of signs.
 *   Philox4x32-10: the counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel
 *           random numbers: as easy as 1, 2, 3" (SC'11), which draws the uniforms of the
 *           stochastic rounding.
 *
 * Readings taken where the pages are garbled or silent (each is listed with its reason
 * in the design notes of the repository):
 *   - the quantiser's garbled expression is read as q = round(x * qmax / absmax);
 *   - one scale per vector: the whole row (or column) along the contraction dimension;
 *   - the transform is block-diagonal over contiguous blocks of `block` indices;
 *   - FP8 uses the OCP formats E4M3FN (max 448) and E5M2 (max 57344) with qmax equal to
 *     the format's largest finite value, round to nearest even, saturating;
 *   - a zero vector gets scale 0 and all-zero codes;
 *   - an element whose scaled value is exactly zero gets the code of +0 (0x00 in every
 *     format): -0 and +0 are one real number, and the sign an fp zero picks up from the
 *     order of the butterflies carries no meaning for the quantiser.  A nonzero value
 *     that rounds to zero keeps its sign, as the OCP conversion rule has it.
 *   - padding: a vector of length L is extended with zeros to Lp = L rounded up to a multiple
 *     of the block, and all Lp rotated values are quantised (the last block mixes the data
 *     with the zeros); for a single block this is the page's padding to a power of two;
 *   - randomised transform: y = (I (x) H_b) D v / sqrt(b) with D = diag(d), d_i = -1 where
 *     bit (i mod 32) of word i / 32 of the sign array is set, else +1.  The array is an
 *     input: the seed only decides how the caller draws it;
 *   - stochastic rounding (codes only): with t the scaled value clamped to [-qmax, qmax]
 *     and s the spacing of the target grid at t (1 for INT8; for FP8 the quantum of |t|'s
 *     binade, the subnormal spacing below the smallest normal), r = t / s, the result is
 *     the grid value s (floor(r) + [u < r - floor(r)]), a zero result taking the +0 code;
 *     u = w / 2^24 with w the top 24 bits of word (p mod 4) of Philox4x32-10(counter =
 *     (p / 4, vector index, c2, c3), key = (k0, k1)) for the element at position p of its
 *     padded vector.
 *
 * Two precisions are offered for the transform + quantisation step:
 *   precision 64: the Kronecker factors of H_b in fp64, from the highest index bit down,
 *                 divide by sqrt(b), q = rne(y * qmax / a) with the quotient taken in long
 *                 double (a real tie stays a tie).
 *   precision 32: the factors in fp32 from index bit 0 up (each sum rounded to fp32), the
 *                 code decided in fp32 from the un-normalised transform output:
 *                 m = fl32(qmax / a), q = rne(y * m) with the product taken exactly
 *                 (INT8) or rounded to fp32 first (FP8).  Where qmax / a overflows (a
 *                 vector of values below about qmax / FLT_MAX) y and a are first scaled
 *                 by 2^64, exactly, and the decision taken on the scaled vector.  The
 *                 1/sqrt(b) factor cancels between y and max|y| in exact arithmetic, so
 *                 both are evaluations of the same formula; precision 32 is the one a
 *                 single-precision device takes its integer decisions in.  Stochastic rounding there starts from
 *                 t = fl32(y * m) and forms r, floor(r), the fraction and the comparison
 *                 with u in fp32 (each of these steps is exact except where the fraction
 *                 of a negative t below 2^-24 in magnitude rounds to 1).
 *   Stochastic rounding in precision 64 takes t = y * qmax / a in long double.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* element types (the oracle's own numbering) */
enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2, OR_E4M3 = 3, OR_E5M2 = 4, OR_F64 = 5 };
/* axis */
enum { OR_ROWS = 0, OR_COLS = 1 };
/* status */
enum { OR_OK = 0, OR_EARG = 1, OR_ENOMEM = 2 };

/* ------------------------------------------------------------------------- */
/* scalar helpers                                                             */
/* ------------------------------------------------------------------------- */

/* round half to even, written out (numpy's np.round semantics); long double keeps the
 * quotients below exact enough that a real tie stays a tie */
static long double rne(long double t)
{
    long double f = floorl(t);
    long double d = t - f; /* exact */
    if (d > 0.5L) return f + 1.0L;
    if (d < 0.5L) return f;
    return (fmodl(f, 2.0L) == 0.0L) ? f : f + 1.0L;
}

static double load_elem(const void* x, int xtype, int64_t idx)
{
    if (xtype == OR_F32) return (double)((const float*)x)[idx];
    /* bf16: the upper 16 bits of an IEEE single */
    uint32_t bits = (uint32_t)((const uint16_t*)x)[idx] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------- */
/* OCP FP8 codec (E4M3FN and E5M2), from the format definitions               */
/* ------------------------------------------------------------------------- */

typedef struct {
    int mbits, bias;
    double maxv;
} fp8_fmt;

static const fp8_fmt FMT_E4M3 = {3, 7, 448.0};
static const fp8_fmt FMT_E5M2 = {2, 15, 57344.0};

static const fp8_fmt* fmt_of(int t) { return t == OR_E4M3 ? &FMT_E4M3 : &FMT_E5M2; }

/* Nearest-even encoding of a finite value, saturating to +-max. */
static uint8_t fp8_encode(long double v, const fp8_fmt* f)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    long double a = fabsl(v);
    int emin = 1 - f->bias; /* exponent of the smallest normal */
    int e;
    if (a < ldexpl(1.0L, emin)) {
        e = emin; /* the subnormal range shares the smallest normal's quantum */
    } else {
        frexpl(a, &e);
        e -= 1; /* a in [2^e, 2^(e+1)) */
    }
    long double quantum = ldexpl(1.0L, e - f->mbits);
    long double r = rne(a / quantum) * quantum; /* exact: quantum is a power of two */
    if (r > (long double)f->maxv) r = (long double)f->maxv;
    if (r == 0.0L) return sign;
    if (r < ldexpl(1.0L, emin)) {
        int mant = (int)(r / ldexpl(1.0L, emin - f->mbits));
        return (uint8_t)(sign | mant);
    }
    int er;
    frexpl(r, &er);
    er -= 1;
    int mant = (int)((r / ldexpl(1.0L, er) - 1.0L) * (long double)(1 << f->mbits));
    return (uint8_t)(sign | ((er + f->bias) << f->mbits) | mant);
}

/* Exact decode; NaN codes decode to NaN, E5M2 infinities to +-inf. */
static double fp8_decode(uint8_t c, const fp8_fmt* f)
{
    int ebits = 7 - f->mbits;
    int ex = (c >> f->mbits) & ((1 << ebits) - 1);
    int mant = c & ((1 << f->mbits) - 1);
    double s = (c & 0x80) ? -1.0 : 1.0;
    if (f == &FMT_E4M3 && ex == 15 && mant == 7) return NAN;
    if (f == &FMT_E5M2 && ex == 31) return mant == 0 ? s * INFINITY : NAN;
    if (ex == 0) return s * ldexp((double)mant, 1 - f->bias - f->mbits);
    return s * ldexp(1.0 + (double)mant / (double)(1 << f->mbits), ex - f->bias);
}

uint8_t hor_fp8_encode(double v, int fmt) { return fp8_encode((long double)v, fmt_of(fmt)); }
double hor_fp8_decode(uint8_t c, int fmt) { return fp8_decode(c, fmt_of(fmt)); }

/* ------------------------------------------------------------------------- */
/* Walsh-Hadamard transform: [QWHA] s2.1 definition, s2.2 normalisation,      */
/* blockwise per s3.1                                                         */
/* ------------------------------------------------------------------------- */

/* The Sylvester matrix of order b = 2^n is the n-fold Kronecker power of
 * H_2 = [[1, 1], [1, -1]] ([QWHA] s2.1 builds it level by level), so entry (i, j) is
 * (-1)^popcount(i & j) and H_b v is the product of n commuting factors, the factor of index
 * bit s acting on every pair of positions that differ only in bit s:
 *     (v_lo, v_hi) <- (v_lo + v_hi, v_lo - v_hi),   lo = i with bit s clear, hi = lo + 2^s.
 * Every factor is exact in real arithmetic and they commute, so any order of the bits gives
 * H_b v; only the rounding of the floating-point sums depends on the order. */
static int log2_of(int64_t b)
{
    int n = 0;
    while (((int64_t)1 << n) < b) ++n;
    return n;
}

static void kron_factor_f64(double* v, int64_t b, int s)
{
    const int64_t d = (int64_t)1 << s;
    for (int64_t lo = 0; lo < b; ++lo) {
        if (lo & d) continue;
        const double a = v[lo], c = v[lo + d];
        v[lo] = a + c;
        v[lo + d] = a - c;
    }
}

static void kron_factor_f32(float* v, int64_t b, int s)
{
    const int64_t d = (int64_t)1 << s;
    for (int64_t lo = 0; lo < b; ++lo) {
        if (lo & d) continue;
        const float a = v[lo], c = v[lo + d];
        v[lo] = a + c;
        v[lo + d] = a - c;
    }
}

/* One block of length b (a power of two), fp64: the factors from the highest index bit down,
 * then the orthonormal scaling 1/sqrt(b) ([QWHA] s2.1: 1/sqrt(2) per level; s2.2: divide by
 * sqrt(n)). */
static void fwht_block_f64(double* v, int64_t b)
{
    for (int s = log2_of(b) - 1; s >= 0; --s) kron_factor_f64(v, b, s);
    double root = sqrt((double)b);
    for (int64_t t = 0; t < b; ++t) v[t] = v[t] / root;
}

/* The same product in fp32, without the scaling, the factors from index bit 0 up (the order
 * of [QWHA] s2.2, whose half-width doubles from 1): the order a single-precision device that
 * rounds after every sum reproduces exactly. */
static void fwht_block_f32_unnorm(float* v, int64_t b)
{
    for (int s = 0; s < log2_of(b); ++s) kron_factor_f32(v, b, s);
}

/* malloc size for n elements, never zero */
static size_t nz(int64_t n) { return (size_t)(n > 0 ? n : 1); }

static int is_pow2(int64_t b) { return b >= 1 && (b & (b - 1)) == 0; }

/* In-place blockwise orthonormal transform of a contiguous fp64 vector. */
int hor_fwht_f64(double* v, int64_t len, int64_t block)
{
    if (!v || !is_pow2(block) || len < 0 || len % block) return OR_EARG;
    for (int64_t j = 0; j < len; j += block) fwht_block_f64(v + j, block);
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): the counter-based       */
/* generator behind the stochastic rounding                                   */
/* ------------------------------------------------------------------------- */

/* Ten rounds on a 4 x 32-bit counter under a 2 x 32-bit key.  A round multiplies words 0
 * and 2 by the two Philox multipliers and forms the new words (hi(2) ^ c1 ^ k0, lo(2),
 * hi(0) ^ c3 ^ k1, lo(0)); the key advances by the two Weyl increments after each round. */
void hor_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p2 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p2 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p2;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Rounding options of a quantisation pass. */
typedef struct {
    int stochastic;  /* 0: nearest even, 1: stochastic */
    uint32_t key[2]; /* Philox key */
    uint32_t chi[2]; /* counter words 2 and 3 */
} rounding_opts;

/* The 24-bit uniform integer w (u = w / 2^24) of the element at position p of vector vid. */
static uint32_t sr_word(const rounding_opts* ro, int64_t vid, int64_t p)
{
    uint32_t ctr[4] = {(uint32_t)(p >> 2), (uint32_t)vid, ro->chi[0], ro->chi[1]};
    uint32_t out[4];
    hor_philox4x32_10(ctr, ro->key, out);
    return out[p & 3] >> 8;
}

/* ------------------------------------------------------------------------- */
/* Quantisation of one rotated vector ([QWHA] s2.2 quantiser, s5 stochastic   */
/* rounding)                                                                  */
/* ------------------------------------------------------------------------- */

static double qmax_of(int qtype)
{
    if (qtype == OR_I8) return 127.0;
    if (qtype == OR_E4M3) return 448.0;
    return 57344.0; /* E5M2 */
}

/* Stochastic rounding of t (|t| <= qmax) to the INT8 or FP8 grid, long double: the grid
 * point below t, plus one grid step when u < the fraction of the way to the next point. */
static long double sr_long(long double t, int qtype, uint32_t w)
{
    long double s = 1.0L;
    if (qtype != OR_I8) {
        const fp8_fmt* f = fmt_of(qtype);
        int emin = 1 - f->bias, e;
        long double a = fabsl(t);
        if (a < ldexpl(1.0L, emin)) {
            e = emin;
        } else {
            frexpl(a, &e);
            e -= 1;
        }
        s = ldexpl(1.0L, e - f->mbits);
    }
    long double r = t / s;
    long double fl = floorl(r);
    long double up = ((long double)w < (r - fl) * 16777216.0L) ? 1.0L : 0.0L;
    long double v = (fl + up) * s;
    return v == 0.0L ? 0.0L : v; /* a zero result takes the +0 code */
}

/* The same steps in fp32 (the step sizes are powers of two, so t / s is exact). */
static float sr_float(float t, int qtype, uint32_t w)
{
    float s = 1.0f;
    if (qtype != OR_I8) {
        const fp8_fmt* f = fmt_of(qtype);
        int emin = 1 - f->bias, e;
        float a = fabsf(t);
        if (a < ldexpf(1.0f, emin)) {
            e = emin;
        } else {
            frexpf(a, &e);
            e -= 1;
        }
        s = ldexpf(1.0f, e - f->mbits);
    }
    float r = t / s;
    float fl = floorf(r);
    float fr = r - fl;
    float v = (fl + (((float)w < fr * 16777216.0f) ? 1.0f : 0.0f)) * s;
    return v == 0.0f ? 0.0f : v;
}

/* fp64: y holds the normalised rotated vector (vector index vid, Lp elements). */
static void quant_vec_f64(const double* y, int64_t L, int qtype, const rounding_opts* ro,
                          int64_t vid, void* q, double* scale)
{
    double a = 0.0;
    for (int64_t i = 0; i < L; ++i)
        if (fabs(y[i]) > a) a = fabs(y[i]);
    double qmax = qmax_of(qtype);
    if (qtype == OR_F64) {
        for (int64_t i = 0; i < L; ++i) ((double*)q)[i] = y[i] == 0.0 ? 0.0 : y[i]; /* +0 */
        *scale = a;
        return;
    }
    if (a == 0.0) {
        memset(q, 0, (size_t)L);
        *scale = 0.0;
        return;
    }
    for (int64_t i = 0; i < L; ++i) {
        /* y * qmax is exact in long double; the quotient is rounded once, at 64 bits */
        long double t = (long double)y[i] * (long double)qmax / (long double)a;
        if (t == 0.0L) t = 0.0L; /* exact zero: the +0 code */
        if (ro->stochastic) {
            if (t > (long double)qmax) t = qmax;
            if (t < -(long double)qmax) t = -qmax;
            long double v = sr_long(t, qtype, sr_word(ro, vid, i));
            if (qtype == OR_I8) ((int8_t*)q)[i] = (int8_t)v;
            else ((uint8_t*)q)[i] = fp8_encode(v, fmt_of(qtype));
            continue;
        }
        if (qtype == OR_I8) {
            long double n = rne(t);
            if (n > 127.0L) n = 127.0L;
            if (n < -127.0L) n = -127.0L;
            ((int8_t*)q)[i] = (int8_t)n;
        } else {
            ((uint8_t*)q)[i] = fp8_encode(t, fmt_of(qtype));
        }
    }
    *scale = a / qmax;
}

/* fp32: yu holds the un-normalised butterfly output of every block of the vector. */
static void quant_vec_f32(const float* yu, int64_t L, int64_t block, int qtype,
                          const rounding_opts* ro, int64_t vid, void* q, double* scale)
{
    float a = 0.0f;
    for (int64_t i = 0; i < L; ++i)
        if (fabsf(yu[i]) > a) a = fabsf(yu[i]);
    if (qtype == OR_F64) {
        float r = (float)(1.0 / sqrt((double)block));
        for (int64_t i = 0; i < L; ++i) {
            float v = yu[i] * r;
            ((double*)q)[i] = v == 0.0f ? 0.0 : (double)v; /* exact zero: +0 */
        }
        *scale = (double)(a * r);
        return;
    }
    float qmax = (float)qmax_of(qtype);
    float denom = (float)((double)qmax * sqrt((double)block));
    if (a == 0.0f) {
        memset(q, 0, (size_t)L);
        *scale = 0.0;
        return;
    }
    /* A vector so small that qmax / a overflows (a below qmax / FLT_MAX) takes its decision
     * on the vector scaled by 2^64: exact for values this small, and the fp32 butterflies
     * (additions only, with gradual underflow) commute with that scaling, so the codes are
     * those of the scaled vector, as the scale invariance of absmax quantisation asks. */
    float pre = 1.0f;
    float m = qmax / a;
    if (isinf(m)) {
        pre = 0x1p64f;
        m = qmax / (a * pre);
    }
    for (int64_t i = 0; i < L; ++i) {
        const float yi = yu[i] * pre; /* exact */
        if (ro->stochastic) {
            float t = yi * m;
            if (t == 0.0f) t = 0.0f;
            t = fminf(fmaxf(t, -qmax), qmax);
            float v = sr_float(t, qtype, sr_word(ro, vid, i));
            if (qtype == OR_I8) ((int8_t*)q)[i] = (int8_t)v;
            else ((uint8_t*)q)[i] = fp8_encode((long double)v, fmt_of(qtype));
            continue;
        }
        if (qtype == OR_I8) {
            long double n = rne((long double)yi * (long double)m); /* exact product */
            if (n > 127.0L) n = 127.0L;
            if (n < -127.0L) n = -127.0L;
            ((int8_t*)q)[i] = (int8_t)n;
        } else {
            float t = yi * m; /* rounded to fp32, then to the fp8 grid */
            if (t == 0.0f) t = 0.0f; /* exact zero: the +0 code */
            ((uint8_t*)q)[i] = fp8_encode((long double)t, fmt_of(qtype));
        }
    }
    *scale = (double)(a / denom);
}

/* Sign d_i of the randomised transform: -1 where bit i of the sign array is set. */
static double sign_of(const uint32_t* signs, int64_t i)
{
    if (!signs) return 1.0;
    return ((signs[i >> 5] >> (i & 31)) & 1u) ? -1.0 : 1.0;
}

/* Padded (rotated) length of a vector of L elements. */
static int64_t padded_len(int64_t L, int64_t block) { return (L + block - 1) / block * block; }

/*
 * Rotate + quantise vectors of a row-major matrix x[rows x cols] (leading dimension ldx).
 *   axis OR_ROWS: vector r is row r, length L = cols.
 *   axis OR_COLS: vector c is column c, length L = rows.
 * Each vector is padded with zeros to Lp = L rounded up to a multiple of block, multiplied
 * by the signs (NULL: none), rotated and quantised with nearest-even (rounding 0) or
 * stochastic (rounding 1; Philox key key[0..1], counter words 2-3 chi[0..1]) rounding.
 * vec_idx (may be NULL = all vectors, in order) selects nvec vectors.
 * q receives nvec x Lp codes, vector-major (int8, fp8 bytes, or doubles for OR_F64 = the
 * normalised rotated values); scale receives nvec scales (absmax/qmax; for OR_F64 the
 * absmax of the normalised vector).
 */
int hor_fwht_quant_ex(const void* x, int xtype, int64_t rows, int64_t cols, int64_t ldx, int axis,
                      int64_t block, int qtype, int precision, const int64_t* vec_idx,
                      int64_t nvec, const uint32_t* signs, int rounding, const uint32_t* key,
                      const uint32_t* chi, void* q, double* scale)
{
    if (!x || !q || !scale) return OR_EARG;
    if (xtype != OR_F32 && xtype != OR_BF16) return OR_EARG;
    if (qtype != OR_I8 && qtype != OR_E4M3 && qtype != OR_E5M2 && qtype != OR_F64) return OR_EARG;
    if (precision != 32 && precision != 64) return OR_EARG;
    if (rounding != 0 && (rounding != 1 || qtype == OR_F64 || !key || !chi)) return OR_EARG;
    if (rows < 0 || cols < 0 || ldx < cols) return OR_EARG;
    int64_t L = axis == OR_ROWS ? cols : rows;
    int64_t total = axis == OR_ROWS ? rows : cols;
    if (!is_pow2(block)) return OR_EARG;
    int64_t Lp = padded_len(L, block);
    if (nvec < 0 || (!vec_idx && nvec > total)) return OR_EARG;
    for (int64_t v = 0; vec_idx && v < nvec; ++v)
        if (vec_idx[v] < 0 || vec_idx[v] >= total) return OR_EARG;
    rounding_opts ro = {rounding, {0, 0}, {0, 0}};
    if (rounding) {
        ro.key[0] = key[0]; ro.key[1] = key[1];
        ro.chi[0] = chi[0]; ro.chi[1] = chi[1];
    }
    size_t qbytes = qtype == OR_F64 ? sizeof(double) : 1;
    int err = OR_OK;

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t v = 0; v < nvec; ++v) {
        int64_t id = vec_idx ? vec_idx[v] : v;
        void* qv = (char*)q + (size_t)v * (size_t)Lp * qbytes;
        if (precision == 64) {
            double* y = (double*)malloc(nz(Lp) * sizeof(double));
            if (!y) { err = OR_ENOMEM; continue; }
            for (int64_t i = 0; i < Lp; ++i) {
                double e = 0.0; /* the zero padding */
                if (i < L) {
                    e = axis == OR_ROWS ? load_elem(x, xtype, id * ldx + i)
                                        : load_elem(x, xtype, i * ldx + id);
                    if (!isfinite(e)) abort(); /* non-finite input is outside the method */
                }
                y[i] = sign_of(signs, i) * e;
            }
            for (int64_t j = 0; j < Lp; j += block) fwht_block_f64(y + j, block);
            quant_vec_f64(y, Lp, qtype, &ro, id, qv, &scale[v]);
            free(y);
        } else {
            float* y = (float*)malloc(nz(Lp) * sizeof(float));
            if (!y) { err = OR_ENOMEM; continue; }
            for (int64_t i = 0; i < Lp; ++i) {
                double e = 0.0;
                if (i < L)
                    e = axis == OR_ROWS ? load_elem(x, xtype, id * ldx + i)
                                        : load_elem(x, xtype, i * ldx + id);
                y[i] = (float)(sign_of(signs, i) * e);
            }
            for (int64_t j = 0; j < Lp; j += block) fwht_block_f32_unnorm(y + j, block);
            quant_vec_f32(y, Lp, block, qtype, &ro, id, qv, &scale[v]);
            free(y);
        }
    }
    return err;
}

/* Nearest-even rounding, no signs. */
int hor_fwht_quant(const void* x, int xtype, int64_t rows, int64_t cols, int64_t ldx, int axis,
                   int64_t block, int qtype, int precision, const int64_t* vec_idx,
                   int64_t nvec, void* q, double* scale)
{
    return hor_fwht_quant_ex(x, xtype, rows, cols, ldx, axis, block, qtype, precision, vec_idx,
                             nvec, NULL, 0, NULL, NULL, q, scale);
}

/* ------------------------------------------------------------------------- */
/* Low-precision products ([HALO] abstract: every large matmul in low precision) */
/* ------------------------------------------------------------------------- */

/* acc[i,j] = sum_k a[i,k] * b[j,k] in int64 (a: m x k, b: n x k, both k-contiguous). */
int hor_gemm_i8(const int8_t* a, const int8_t* b, int64_t m, int64_t n, int64_t k, int64_t* acc)
{
    if ((!a && m * k != 0) || (!b && n * k != 0) || (!acc && m * n != 0) || m < 0 || n < 0 || k < 0) return OR_EARG;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            int64_t s = 0;
            for (int64_t t = 0; t < k; ++t) s += (int64_t)a[i * k + t] * (int64_t)b[j * k + t];
            acc[i * n + j] = s;
        }
    return OR_OK;
}

/* out[i,j] = sum_k dec(a[i,k]) * dec(b[j,k]) in fp64, summed in order of k.  The codes are
 * decoded once into fp64 tables of the two operands (the same exact values), then the sums
 * are taken. */
int hor_gemm_fp8(const uint8_t* a, int afmt, const uint8_t* b, int bfmt, int64_t m, int64_t n,
                 int64_t k, double* out)
{
    if ((!a && m * k != 0) || (!b && n * k != 0) || (!out && m * n != 0) || m < 0 || n < 0 || k < 0) return OR_EARG;
    if ((afmt != OR_E4M3 && afmt != OR_E5M2) || (bfmt != OR_E4M3 && bfmt != OR_E5M2)) return OR_EARG;
    const fp8_fmt* fa = fmt_of(afmt);
    const fp8_fmt* fb = fmt_of(bfmt);
    double ta[256], tb[256];
    for (int c = 0; c < 256; ++c) {
        ta[c] = fp8_decode((uint8_t)c, fa);
        tb[c] = fp8_decode((uint8_t)c, fb);
    }
    double* da = (double*)malloc(nz(m * k) * sizeof(double));
    double* db = (double*)malloc(nz(n * k) * sizeof(double));
    if (!da || !db) {
        free(da);
        free(db);
        return OR_ENOMEM;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m * k; ++i) da[i] = ta[a[i]];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n * k; ++i) db[i] = tb[b[i]];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t t = 0; t < k; ++t) s += da[i * k + t] * db[j * k + t];
            out[i * n + j] = s;
        }
    free(da);
    free(db);
    return OR_OK;
}

/* Exact fp64 product out = A B^T (A: m x k, B: n x k); the unquantised reference. */
int hor_matmul_f64(const double* a, const double* b, int64_t m, int64_t n, int64_t k, double* out)
{
    if ((!a && m * k != 0) || (!b && n * k != 0) || (!out && m * n != 0)) return OR_EARG;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t t = 0; t < k; ++t) s += a[i * k + t] * b[j * k + t];
            out[i * n + j] = s;
        }
    return OR_OK;
}

/* out[i,j] = acc[i,j] * sa[i] * sb[j] in fp64 (the scale dequant). */
void hor_dequant(const double* acc, const double* sa, const double* sb, int64_t m, int64_t n,
                 double* out)
{
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) out[i * n + j] = acc[i * n + j] * sa[i] * sb[j];
}

/* ------------------------------------------------------------------------- */
/* The layer: quantise both operands along the contraction dim, multiply,     */
/* dequantise.                                                               */
/* ------------------------------------------------------------------------- */

/* C[p x q] = dequant(Qa[p x L] . Qb[q x L]^T) for codes of one type pair. */
static int lowp_product(const void* qa, int ta, const double* sa, const void* qb, int tb,
                        const double* sb, int64_t p, int64_t qn, int64_t L, double* out)
{
    double* acc = (double*)malloc(nz(p * qn) * sizeof(double));
    if (!acc) return OR_ENOMEM;
    int rc;
    if (ta == OR_I8) {
        int64_t* iacc = (int64_t*)malloc(nz(p * qn) * sizeof(int64_t));
        if (!iacc) { free(acc); return OR_ENOMEM; }
        rc = hor_gemm_i8((const int8_t*)qa, (const int8_t*)qb, p, qn, L, iacc);
        for (int64_t i = 0; i < p * qn; ++i) acc[i] = (double)iacc[i];
        free(iacc);
    } else {
        rc = hor_gemm_fp8((const uint8_t*)qa, ta, (const uint8_t*)qb, tb, p, qn, L, acc);
    }
    if (rc == OR_OK) hor_dequant(acc, sa, sb, p, qn, out);
    free(acc);
    return rc;
}

/* Quantisation options of one operand of a product. */
typedef struct {
    const uint32_t* signs; /* the randomised transform's signs along the contraction dim */
    int rounding;          /* 0 nearest even, 1 stochastic */
    const uint32_t* key;
    const uint32_t* chi;
} operand_opts;

/* One low-precision product along one contraction dimension:
 * out = dequant(Q(A along L) Q(B along L)^T), where each operand is a row-major matrix
 * given with its axis (the vectors quantised are rows or columns of it).  Both operands are
 * padded to the same Lp and multiplied over all Lp rotated positions. */
static int rotated_product(const void* a, int64_t ar, int64_t ac, int aaxis, int qa_t,
                           const operand_opts* ao, const void* b, int64_t br, int64_t bc,
                           int baxis, int qb_t, const operand_opts* bo, int xtype, int64_t block,
                           int precision, double* out)
{
    if (!is_pow2(block)) return OR_EARG;
    int64_t p = aaxis == OR_ROWS ? ar : ac;
    int64_t L = aaxis == OR_ROWS ? ac : ar;
    int64_t qn = baxis == OR_ROWS ? br : bc;
    int64_t Lp = padded_len(L, block);
    void* qa = malloc(nz(p * Lp));
    void* qb = malloc(nz(qn * Lp));
    double* sa = (double*)malloc(nz(p) * sizeof(double));
    double* sb = (double*)malloc(nz(qn) * sizeof(double));
    int rc = OR_ENOMEM;
    if (qa && qb && sa && sb) {
        rc = hor_fwht_quant_ex(a, xtype, ar, ac, ac, aaxis, block, qa_t, precision, NULL, p,
                               ao->signs, ao->rounding, ao->key, ao->chi, qa, sa);
        if (rc == OR_OK)
            rc = hor_fwht_quant_ex(b, xtype, br, bc, bc, baxis, block, qb_t, precision, NULL, qn,
                                   bo->signs, bo->rounding, bo->key, bo->chi, qb, sb);
        if (rc == OR_OK) rc = lowp_product(qa, qa_t, sa, qb, qb_t, sb, p, qn, Lp, out);
    }
    free(qa); free(qb); free(sa); free(sb);
    return rc;
}

/* Forward: Y[m x n] = X[m x k] W[n x k]^T, both rotated (signs_k: the randomised
 * transform's signs along k, may be NULL) and quantised along k. */
int hor_linear_fwd_ex(const void* x, const void* w, int xtype, int64_t m, int64_t n, int64_t k,
                      int64_t block, int qtype, int precision, const uint32_t* signs_k, double* y)
{
    if (!x || !w || !y || qtype == OR_F64) return OR_EARG;
    operand_opts o = {signs_k, 0, NULL, NULL};
    return rotated_product(x, m, k, OR_ROWS, qtype, &o, w, n, k, OR_ROWS, qtype, &o, xtype,
                           block, precision, y);
}

int hor_linear_fwd(const void* x, const void* w, int xtype, int64_t m, int64_t n, int64_t k,
                   int64_t block, int qtype, int precision, double* y)
{
    return hor_linear_fwd_ex(x, w, xtype, m, n, k, block, qtype, precision, NULL, y);
}

/* Backward: dX[m x k] = dY[m x n] W[n x k]   (contraction over n, signs signs_n),
 *           dW[n x k] = dY^T X               (contraction over m, signs signs_m).
 * dY is quantised with grad_qtype and grad_rounding (stochastic: Philox key key[0..1],
 * counter words chi[0..1] for the rows of dY and (chi[0], chi[1] ^ 2^31) for its columns),
 * X and W with qtype and nearest-even rounding.  Either output may be NULL. */
int hor_linear_bwd_ex(const void* dy, const void* x, const void* w, int xtype, int64_t m,
                      int64_t n, int64_t k, int64_t block, int qtype, int grad_qtype,
                      int precision, const uint32_t* signs_n, const uint32_t* signs_m,
                      int grad_rounding, const uint32_t* key, const uint32_t* chi, double* dx,
                      double* dw)
{
    if (!dy || !x || !w || qtype == OR_F64 || grad_qtype == OR_F64) return OR_EARG;
    if (grad_rounding && (!key || !chi)) return OR_EARG;
    uint32_t chi_cols[2] = {0, 0};
    if (grad_rounding) {
        chi_cols[0] = chi[0];
        chi_cols[1] = chi[1] ^ 0x80000000u;
    }
    int rc = OR_OK;
    if (dx) { /* A = rows of dY (length n), B = columns of W (length n) */
        operand_opts ga = {signs_n, grad_rounding, key, chi};
        operand_opts wb = {signs_n, 0, NULL, NULL};
        rc = rotated_product(dy, m, n, OR_ROWS, grad_qtype, &ga, w, n, k, OR_COLS, qtype, &wb,
                             xtype, block, precision, dx);
    }
    if (rc == OR_OK && dw) { /* A = columns of dY (length m), B = columns of X (length m) */
        operand_opts ga = {signs_m, grad_rounding, key, chi_cols};
        operand_opts xb = {signs_m, 0, NULL, NULL};
        rc = rotated_product(dy, m, n, OR_COLS, grad_qtype, &ga, x, m, k, OR_COLS, qtype, &xb,
                             xtype, block, precision, dw);
    }
    return rc;
}

int hor_linear_bwd(const void* dy, const void* x, const void* w, int xtype, int64_t m, int64_t n,
                   int64_t k, int64_t block, int qtype, int grad_qtype, int precision,
                   double* dx, double* dw)
{
    return hor_linear_bwd_ex(dy, x, w, xtype, m, n, k, block, qtype, grad_qtype, precision, NULL,
                             NULL, 0, NULL, NULL, dx, dw);
}

int hor_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
