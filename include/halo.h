/*
 * halo.h -- C ABI of libhalo.so: the Hadamard-rotated low-precision linear layer on
 * MI355X (gfx950).
 *
 * The method ("HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs", abstract and
 * method section): every large matrix product of a linear layer's forward and backward pass
 * runs in 8-bit precision (INT8 or FP8, key design 2) after a Hadamard rotation of both
 * operands along the contraction dimension, which spreads outlier channels.  The rotation
 * is the orthonormal Walsh-Hadamard transform in natural (Sylvester) order, applied to
 * contiguous blocks of `block` indices ("QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术",
 * s2.1 definition, s2.2 butterfly and 1/sqrt(n), s3.1 blockwise); every rotated vector is
 * quantised with its own absmax scale (s2.2 quantiser, ties to even).  Because the rotation
 * is orthogonal, (X H)(W H)^T = X W^T, so the dequantised product approximates the plain one.
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major with an explicit leading dimension (in elements).
 *   - Every pointer is DEVICE memory owned by the caller.  The library never allocates,
 *     frees or synchronises; work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and the call returns once it is enqueued.
 *   - A pointer may be NULL only when the matrix it describes is empty (a zero size).
 *   - All arguments are validated on the host before anything is launched.  On any error
 *     the call returns a non-zero status, launches nothing and writes no output.  A failed
 *     launch returns HALO_ERR_HIP.  Nothing is printed, and the only state kept between calls
 *     is a per-device cache of launch attributes and occupancy (set once, atomically), so
 *     calls are thread-safe; calls on one stream run in order.
 *   - Columns longer than 4096 rows (halo_fwht_quant's columns axis with a workspace, and
 *     the backward pass when m > 4096 or n > 4096) are split over workgroups that wait for
 *     each other to combine their maxima.  The wait is bounded: after 2^20 polls (each a
 *     device-scope load and a short sleep; the exchange_polls option of the _ex calls sets
 *     another count) a workgroup stops waiting and leaves its part of the column strip
 *     unstored, and a second launch that the call enqueues right after stores every part of
 *     such strips from the completed maxima.  The codes and scales are the same either way:
 *     no result depends on other work that occupies the device.
 *   - Alignment: every pointer 16-byte aligned, every leading dimension a multiple of 16
 *     bytes (HALO_ERR_ALIGN otherwise).
 *   - Scales are fp32 dequant multipliers: the vector's absmax after the orthonormal
 *     rotation divided by qmax (127 for INT8, 448 for E4M3, 57344 for E5M2).  A zero vector
 *     gets scale 0 and all-zero codes.
 *   - Codes are decided in fp32: the un-normalised rotated value y times m = fl32(qmax /
 *     absmax), rounded to the code grid (INT8: from the exact product; FP8: from its fp32
 *     rounding).  A vector so small that m overflows (absmax below about qmax / FLT_MAX,
 *     e.g. subnormal inputs) is first scaled by 2^64, exactly, so its codes are those of the
 *     scaled vector.  Inputs whose fp32 block sums overflow are outside the supported range.
 *   - FP8 is the OCP format pair E4M3 ("FN": max 448, no infinities) and E5M2 (max 57344);
 *     codes are rounded to nearest even and never exceed the format's largest finite value.
 */
#ifndef HALO_H
#define HALO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HALO_OK = 0,
    HALO_ERR_NULL = 1,      /* a required pointer is NULL                                  */
    HALO_ERR_SHAPE = 2,     /* a size is negative, too large, or not a supported multiple  */
    HALO_ERR_BLOCK = 3,     /* block not a power of two in [1, 4096]                       */
    HALO_ERR_DTYPE = 4,     /* unsupported element type or type pair                      */
    HALO_ERR_ALIGN = 5,     /* pointer or leading dimension not 16-byte aligned            */
    HALO_ERR_WORKSPACE = 6, /* workspace NULL or smaller than the size query returns       */
    HALO_ERR_HIP = 7,       /* the HIP runtime refused a launch                            */
    HALO_ERR_OPTION = 8     /* invalid option: unknown rounding mode, or stochastic        */
                            /* rounding asked of the fp32 value mode                       */
} halo_status;

typedef enum {
    HALO_F32 = 0,  /* IEEE binary32                                      */
    HALO_BF16 = 1, /* bfloat16                                           */
    HALO_I8 = 2,   /* signed 8-bit integer codes in [-127, 127]         */
    HALO_E4M3 = 3, /* OCP FP8 E4M3FN codes                              */
    HALO_E5M2 = 4, /* OCP FP8 E5M2 codes                                */
    HALO_I32 = 5   /* signed 32-bit integer (raw INT8 GEMM accumulators) */
} halo_dtype;

typedef enum {
    HALO_ALONG_ROWS = 0, /* vectors are the rows: rotate the contiguous dimension        */
    HALO_ALONG_COLS = 1  /* vectors are the columns: rotate the strided dimension; the   */
                         /* codes are written transposed, one row per column             */
} halo_axis;

/*
 * Rotate and quantise every vector of x[rows x cols] (leading dimension ldx).
 *
 * Defined by: the blockwise orthonormal Walsh-Hadamard transform of each vector (QWHA page
 * s2.1-s2.2, s3.1) followed by the per-vector absmax quantiser (s2.2), i.e. for a vector v
 * of length L, padded with zeros to Lp = L rounded up to a multiple of block (QWHA page s5:
 * lengths padded with zeros for the transform):
 *   y = v (I_{Lp/block} (x) H_block) / sqrt(block),  a = max|y|,
 *   code = round_to_nearest_even(y * qmax / a),  scale = a / qmax.
 * Every one of the Lp rotated positions gets a code (the last block mixes data and zeros).
 *
 *   x_type   HALO_F32 or HALO_BF16.
 *   axis     HALO_ALONG_ROWS: vector r = x[r, :], L = cols (a multiple of 8); q is [rows x Lp]
 *                             (ldq >= Lp) and scale has `rows` entries.
 *            HALO_ALONG_COLS: vector c = x[:, c], L = rows; q is [cols x Lp] (ldq >= Lp),
 *                             i.e. the codes of column c form row c of q; scale has `cols`
 *                             entries.  cols must be a multiple of 8.
 *   block    power of two in [1, 4096]; Lp must be a multiple of 8 (so L too when block < 8).
 *            block 1 is the identity (plain per-vector absmax quantisation).
 *   q_type   HALO_I8, HALO_E4M3, HALO_E5M2: 1-byte codes.
 *            HALO_F32: test mode, q receives the rotated values themselves (fp32) and scale
 *            the absmax of each rotated vector.
 *   ldq      leading dimension of q in elements.
 *   ws       optional device scratch of ws_bytes >= halo_fwht_quant_workspace_bytes(...)
 *            bytes (16-byte aligned), caller-owned; its contents on entry do not matter and
 *            are clobbered.  With it, a columns-axis pass over long columns reads its input
 *            once; with ws NULL (or too small) the pass reads its input twice and gives the
 *            same codes and scales (as does fp32 input with stochastic rounding).  Calls that share one scratch must be ordered on one
 *            stream.  After such a pass completes, the first 32-bit word of ws holds the
 *            number of workgroups that stopped waiting for the exchange (a diagnostic; the
 *            results do not depend on it).
 * Rows-axis vectors: Lp up to 65536 when Lp is a multiple of 64 (one workgroup of Lp / 4096
 * waves holds a row; for stochastic rounding the input must then be bf16), else up to 16384.
 * Codes are decided in fp32: m = qmax / max|b| with b the un-normalised butterfly output and
 * code = round(b * m); the 1/sqrt(block) factor cancels between b and max|b|.
 */
halo_status halo_fwht_quant(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                            int64_t ldx, halo_axis axis, int32_t block, halo_dtype q_type,
                            void* q, int64_t ldq, float* scale, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * Scratch bytes halo_fwht_quant can use for this shape (0 when it needs none: rows axis, or
 * columns short enough for one workgroup; the same for bf16 and fp32 input).  Invalid
 * arguments give 0.
 */
size_t halo_fwht_quant_workspace_bytes(int64_t rows, int64_t cols, halo_axis axis,
                                       int32_t block, halo_dtype x_type);

/*
 * INT8 product with wide accumulation and a fused scale dequant ("HALO: Hadamard-Assisted
 * Lower-Precision Optimization for LLMs", abstract: all large products in low precision):
 *   acc[i, j] = sum_t a[i, t] * b[j, t]   (int32; exact for k <= 133144 with |codes| <= 127)
 *   c[i, j]   = acc[i, j] * sa[i] * sb[j] (c_type HALO_F32 or HALO_BF16, rounded to nearest even)
 *   c[i, j]   = acc[i, j]                 (c_type HALO_I32; sa and sb are not read and may be NULL)
 * a is [m x k] (lda), b is [n x k] (ldb), both contiguous along k; c is [m x n] (ldc).
 * k must be a positive multiple of 16; m and n are arbitrary (>= 0).  Each code operand must
 * span less than 4 GiB ((m - 1) * lda + k < 2^32, likewise for b; HALO_ERR_SHAPE otherwise).
 */
halo_status halo_gemm_i8(const int8_t* a, int64_t lda, const float* sa, const int8_t* b,
                         int64_t ldb, const float* sb, int64_t m, int64_t n, int64_t k, void* c,
                         halo_dtype c_type, int64_t ldc, void* stream);

/*
 * FP8 product (key design 2 of the HALO page: FP8 as the alternative 8-bit type) with fp32
 * accumulation on the CDNA4 FP8 matrix cores and the same fused dequant:
 *   c[i, j] = (sum_t dec(a[i, t]) * dec(b[j, t])) * sa[i] * sb[j]
 * a_type, b_type: HALO_E4M3 or HALO_E5M2 each (any pair); c_type: HALO_F32 or HALO_BF16.
 * Shapes, layouts and the 4 GiB operand span as for halo_gemm_i8; k must be a positive multiple
 * of 32.
 * The sum is the matrix core's: it adds the products of each group of 8 consecutive t in a
 * fixed-point format aligned to the group's largest product (about 15 bits kept below its
 * leading bit, lower bits dropped), then accumulates the group sums in fp32, so the result
 * lies within (2^-10 + g) * sum_t |dec(a) dec(b)| of the exact sum before the dequant,
 * g = n 2^-24 / (1 - n 2^-24) with n = k / 8 + 2 (behaviour measured on gfx950).
 */
halo_status halo_gemm_fp8(const void* a, halo_dtype a_type, int64_t lda, const float* sa,
                          const void* b, halo_dtype b_type, int64_t ldb, const float* sb,
                          int64_t m, int64_t n, int64_t k, void* c, halo_dtype c_type,
                          int64_t ldc, void* stream);

/*
 * Workspace bytes the layer calls need (codes + scales of every quantised operand, each
 * region 256-byte aligned), for every block size (the largest over blocks 1 .. 4096; the
 * block decides the padded contraction lengths).  backward = 0 for halo_linear_fwd, 1 for
 * halo_linear_bwd.  Returns 0 for invalid sizes or types.
 */
size_t halo_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, halo_dtype q_type,
                                   int backward);

/*
 * Forward of the rotated low-precision linear layer: Y[m x n] = X[m x k] W[n x k]^T with
 * both operands rotated along k, quantised per row and multiplied in 8 bits (the HALO
 * page's forward pass; rotation and quantiser per the QWHA page s2.1-s2.2).
 *   io_type  HALO_F32 or HALO_BF16 for x and w (dense, leading dimension k).
 *   q_type   HALO_I8 or HALO_E4M3.
 *   y_type   HALO_F32 or HALO_BF16 (dense, leading dimension n).
 *   ws       caller workspace of at least halo_linear_workspace_bytes(m, n, k, q_type, 0)
 *            (or halo_linear_workspace_bytes_ex(m, n, k, block, q_type, 0)).
 * k must be a multiple of 8 and n a multiple of 16 bytes of y_type; block as for
 * halo_fwht_quant.  When block does not divide k, X and W are padded with zeros along k (QWHA
 * page s5) and the product runs over all padded positions, which equals the product of the
 * padded operands.  The padded k (rounded up to a multiple of block and of 32) is a rows-axis
 * length as in halo_fwht_quant (up to 65536 when a multiple of 64, else 16384), and each code
 * matrix (m or n rows of the padded k) spans less than 4 GiB.
 */
halo_status halo_linear_fwd(const void* x, const void* w, halo_dtype io_type, int64_t m,
                            int64_t n, int64_t k, int32_t block, halo_dtype q_type, void* y,
                            halo_dtype y_type, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the layer (the HALO page: rotations in the backward pass too, both gradient
 * products in 8 bits), each product rotated along its own contraction dimension:
 *   dX[m x k] = dY[m x n] W[n x k]    rows of dY and columns of W rotated along n
 *   dW[n x k] = dY^T X                columns of dY and of X rotated along m
 * Operands are re-quantised from the high-precision x, w and dy.
 *   io_type      HALO_F32 or HALO_BF16 for dy, x, w and the outputs dx, dw (dense).
 *   q_type       codes of X and W: HALO_I8 or HALO_E4M3.
 *   grad_q_type  codes of dY: HALO_I8 (with q_type HALO_I8) or HALO_E5M2 / HALO_E4M3 (with
 *                q_type HALO_E4M3).
 *   dx, dw       outputs; either may be NULL to skip that product.
 *   ws           at least halo_linear_workspace_bytes(m, n, k, q_type, 1) bytes.
 * n and k must be multiples of 8, m >= 1; block as for halo_fwht_quant.  Contraction
 * dimensions that block does not divide are zero-padded as in halo_linear_fwd; when dx is
 * computed the padded n is a rows-axis length as in halo_fwht_quant (with stochastic rounding
 * of fp32 dY: at most 16384), and each code matrix spans less than 4 GiB.
 * With INT8 codes, dW's int32 sums run over the padded m: exact while every partial sum
 * stays within int32, which |codes| <= 127 guarantee up to 133144 terms (as halo_gemm_i8).
 */
halo_status halo_linear_bwd(const void* dy, const void* x, const void* w, halo_dtype io_type,
                            int64_t m, int64_t n, int64_t k, int32_t block, halo_dtype q_type,
                            halo_dtype grad_q_type, void* dx, void* dw, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Options of the extended rotation calls.
 *
 * Randomised transform H D ("企业官网建设流程全解析", a HALO overview, s4.2: every node
 * initialises the Hadamard matrix from one shared random seed): the vector is multiplied by
 * a diagonal of signs before the transform, y = (I (x) H_block) D v / sqrt(block).  `signs`
 * is a device array of ceil(Lp / 32) 32-bit words, bit (i mod 32) of word i / 32 set meaning
 * d_i = -1; all callers that must agree (for instance every rank of a job) draw it from the
 * same seed.  NULL means D = I.  16-byte aligned.
 *
 * Stochastic rounding (QWHA page s5: round down, then up with probability equal to the
 * fraction, to remove the quantiser's bias), for the code types: t = y * qmax / a is clamped
 * to [-qmax, qmax]; with s the grid step at t (1 for INT8; for FP8 the quantum of |t|'s
 * binade, the subnormal quantum below the smallest normal) and r = t / s, the code is the
 * grid value s (floor(r) + [u < r - floor(r)]) (zero takes the +0 code).  The uniform of the
 * element at position p of vector v (its row index for the rows axis, its column index for
 * the columns axis) is u = (w >> 8) / 2^24 with w word p mod 4 of Philox4x32-10 (Salmon et
 * al., "Parallel random numbers: as easy as 1, 2, 3", SC'11) at counter (p / 4, v,
 * counter[0], counter[1]) and key (seed[0], seed[1]).  The decision is taken in fp32 from
 * t = fl32(b * m), b the un-normalised butterfly output and m = fl32(qmax / max|b|).  Draw a
 * fresh counter (or seed) per call for independent rounding.
 */
typedef enum {
    HALO_ROUND_NEAREST_EVEN = 0,
    HALO_ROUND_STOCHASTIC = 1
} halo_rounding;

typedef struct {
    const uint32_t* signs; /* sign bits of D along the rotated dimension, or NULL         */
    int32_t rounding;      /* halo_rounding                                               */
    uint32_t seed[2];      /* Philox key (stochastic rounding)                            */
    uint32_t counter[2];   /* Philox counter words 2 and 3 (stochastic rounding)          */
    uint32_t exchange_polls; /* columns longer than 4096 rows: polls a waiting workgroup  */
                             /* makes before it stops waiting (0 = 2^20); results are the */
                             /* same for every value                                      */
} halo_quant_opts;

/*
 * halo_fwht_quant with options (NULL opts = halo_fwht_quant).  Invalid options give
 * HALO_ERR_OPTION (rounding not a halo_rounding, or stochastic with q_type HALO_F32) or
 * HALO_ERR_ALIGN (signs not 16-byte aligned).
 */
halo_status halo_fwht_quant_ex(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                               int64_t ldx, halo_axis axis, int32_t block, halo_dtype q_type,
                               void* q, int64_t ldq, float* scale, const halo_quant_opts* opts,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Options of the extended layer calls: one sign array per contraction dimension (each covers
 * that dimension's padded length; NULL = plain transform) and the rounding of the dY codes.
 *   signs_k  D along k: the forward product (rows of X and of W).
 *   signs_n  D along n: the dX product (rows of dY, columns of W).
 *   signs_m  D along m: the dW product (columns of dY and of X).
 *   grad_rounding, seed, counter: rounding of the dY codes, as in halo_quant_opts; the rows
 *            of dY draw at counter words (counter[0], counter[1]) and its columns at
 *            (counter[0], counter[1] ^ 0x80000000).  X and W are always rounded to nearest.
 */
typedef struct {
    const uint32_t* signs_k;
    const uint32_t* signs_n;
    const uint32_t* signs_m;
    int32_t grad_rounding;
    uint32_t seed[2];
    uint32_t counter[2];
    uint32_t exchange_polls;  /* as in halo_quant_opts (the backward's columns along m) */
} halo_linear_opts;

/* Workspace bytes of the layer calls for one block size (exact; the block decides the padded
 * contraction lengths).  Returns 0 for invalid arguments. */
size_t halo_linear_workspace_bytes_ex(int64_t m, int64_t n, int64_t k, int32_t block,
                                      halo_dtype q_type, int backward);

/* halo_linear_fwd / halo_linear_bwd with options (NULL opts = the plain calls).  Invalid
 * options give HALO_ERR_OPTION, unaligned sign arrays HALO_ERR_ALIGN. */
halo_status halo_linear_fwd_ex(const void* x, const void* w, halo_dtype io_type, int64_t m,
                               int64_t n, int64_t k, int32_t block, halo_dtype q_type, void* y,
                               halo_dtype y_type, const halo_linear_opts* opts, void* ws,
                               size_t ws_bytes, void* stream);
halo_status halo_linear_bwd_ex(const void* dy, const void* x, const void* w, halo_dtype io_type,
                               int64_t m, int64_t n, int64_t k, int32_t block, halo_dtype q_type,
                               halo_dtype grad_q_type, void* dx, void* dw,
                               const halo_linear_opts* opts, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): halo_fwht_quant_ex with the columns pass's exchange scratch taken
 * from a fixed array inside the library instead of a caller workspace, so that long bf16
 * columns are still read once.  The call allocates and frees nothing, on the host or the
 * device.  The array holds HALO_NOALLOC_SCRATCH_BYTES bytes, one copy per device, kept until
 * the process ends; a pass that needs more (halo_fwht_quant_workspace_bytes(...) larger than
 * that: columns of over 4096 rows with more than about 250,000 columns) is refused with
 * HALO_ERR_WORKSPACE before anything is launched.  Passes that need no scratch run as
 * halo_fwht_quant_ex.  Every call on one device shares the array and clears what it uses at
 * its start, on its stream: calls that may overlap on one device (other streams, other host
 * threads) race on it and must be ordered by the caller.  Other arguments, results and
 * errors as halo_fwht_quant_ex.
 */
#define HALO_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)
halo_status halo_fwht_quant_noalloc(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                                    int64_t ldx, halo_axis axis, int32_t block,
                                    halo_dtype q_type, void* q, int64_t ldq, float* scale,
                                    const halo_quant_opts* opts, void* stream);

/*
 * Both rotation passes of one matrix, from a single read of it where the shape allows: the
 * codes and scales halo_fwht_quant_ex gives along the rows (qr [rows x Lc], leading dimension
 * ldqr, scale_r [rows], options row_opts) and along the columns (qc [cols x Lr], ldqc,
 * scale_c [cols], col_opts), with one block and one code type.  A layer backward needs its
 * gradient dY both ways (rows for dX = dY W, columns for dW = dY^T X: the HALO page's
 * rotations in the backward pass; QWHA page s2.1-s2.2, s3.1 for the transform and the
 * quantiser); the two separate passes read dY twice.
 *   ws   scratch of halo_fwht_quant_dual_workspace_bytes(rows, cols, block, x_type) bytes,
 *        16-byte aligned, clobbered (its first 32-bit word then holds the number of
 *        workgroups that stopped waiting for an exchange, as in halo_fwht_quant).
 * The single read applies when x is bf16, rows and cols are multiples of 256, block <= 256,
 * both passes round to nearest, all (rows / 256) x (cols / 256) tiles fit on the device at
 * once (one per compute unit: up to 4096 x 4096 on 256 CUs) and ws is large enough; every
 * other valid call runs the two passes one after the other, with the same results.  Each
 * argument is validated as halo_fwht_quant_ex validates it for its pass; options as there.
 */
size_t halo_fwht_quant_dual_workspace_bytes(int64_t rows, int64_t cols, int32_t block,
                                            halo_dtype x_type);
halo_status halo_fwht_quant_dual(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                                 int64_t ldx, int32_t block, halo_dtype q_type, void* qr,
                                 int64_t ldqr, float* scale_r, void* qc, int64_t ldqc,
                                 float* scale_c, const halo_quant_opts* row_opts,
                                 const halo_quant_opts* col_opts, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * Measurement aid, not part of the layer: the sustained rate of the matrix-core instruction a
 * product uses, on the whole device, to set the products' measured rates beside what the
 * instruction alone reaches under a sustained load (the published dense peaks assume the
 * 2.4 GHz engine clock).
 *   kind   0: v_mfma_i32_32x32x32_i8 (the INT8 product's), 1: v_mfma_scale_f32_32x32x64_f8f6f4
 *          on E4M3 operands (the FP8 product's), 2: v_mfma_scale_f32_16x16x128_f8f6f4 on E4M3
 *          operands.
 *   iters  MFMA groups per wave, in [2, 1 << 20] (rounded up to even); one group is 8
 *          independent MFMAs (16 for kind 2), one per (a, b) fragment pair of a product's
 *          wave tile, so every MFMA takes a different operand pair; the operands are codes
 *          drawn like the products' (rotated, absmax-scaled data), since how much their bits
 *          toggle sets the clock the chip holds.
 *   ops    receives the operations (2 x multiply-adds) the launch performs.
 * One launch of 256 workgroups of 512 threads (two waves per SIMD, as the products run) on
 * the stream; it reads and writes no caller memory.  Time it with events on that stream.
 * HALO_ERR_SHAPE for kind or iters out of range, HALO_ERR_NULL for ops NULL.
 */
halo_status halo_mfma_rate_probe(int32_t kind, int32_t iters, int64_t* ops, void* stream);

/* Static description of a status code. */
const char* halo_status_str(halo_status s);

#ifdef __cplusplus
}
#endif

#endif /* HALO_H */
