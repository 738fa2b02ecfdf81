// halo_kernels.h -- internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace halo {

// Arguments of one fused rotation + quantisation pass.
struct FqArgs {
  const void* x;       // input, row-major [rows x cols], leading dim ldx (elements)
  int64_t ldx;
  int64_t nvec;        // number of vectors (rows for the rows axis, cols for the cols axis)
  int64_t len;         // rotated length L
  void* q;             // codes [nvec x L], leading dim ldq (elements)
  int64_t ldq;
  float* scale;        // [nvec]
  int64_t vec_per_wg;  // rows kernel: vectors per workgroup (set by the launcher)
  int block;
  float qmax;          // 127, 448, 57344
  float denom;         // fl32(qmax * sqrt(block)): scale = max|b| / denom
  float inv_sqrt_b;    // fl32(1 / sqrt(block)) for the fp32 test mode
  int64_t in_len;      // input elements per vector (<= len); positions [in_len, len) are the
                       // zero padding and are not read
  const uint32_t* signs;  // randomised transform: bit i set negates element i (NULL: none)
  int sr;                 // 1: stochastic rounding of the codes (code types only)
  uint32_t key0, key1;    // Philox4x32-10 key
  uint32_t ctr2, ctr3;    // Philox counter words 2 and 3 (word 0: position / 4, word 1: vector)
  uint32_t polls;         // columns passes that exchange maxima: polls of a waiting task
                          // before it stops waiting (0: the default, 2^20)
};

// in_bf16: 1 for bf16 input, 0 for fp32.  qt: 0 INT8, 1 E4M3, 2 E5M2, 3 fp32 values.
// axis: 0 rows, 1 cols.  ws / ws_bytes: scratch for the single-read columns kernel (may be
// NULL / 0: the columns pass then reads its input twice).
hipError_t launch_fwht_quant(const FqArgs& a, int in_bf16, int qt, int axis, void* ws,
                             size_t ws_bytes, hipStream_t st);

// Scratch bytes the single-read columns kernel needs for columns of `rows` elements (0 when
// it needs none or does not cover the shape), for bf16 and fp32 input alike.
size_t fq_cols2_ws_bytes(int64_t rows, int64_t cols, int block);
// Whether the single-read columns kernel takes the pass (bf16 or fp32 input; fp32 with
// stochastic rounding is not covered) given ws_bytes of scratch.
bool fq_cols2_supported(int64_t rows, int64_t cols, int block, int in_bf16, bool sr,
                        size_t ws_bytes);
hipError_t launch_fq_cols2(const FqArgs& a, int in_bf16, int qt, void* ws, hipStream_t st);

// The rotation passes of a layer backward in one launch (bf16 input): the rows of dY (codes
// qg; may be NULL, else fq_batch_rows_ok(len) must hold) and the single-read column passes of
// W (qw), dY (qg) and X (qw), whose scratch must be zero at launch.  Code type pairs (qg, qw):
// (0, 0), (2, 1), (1, 1).
bool fq_batch_rows_ok(int64_t len);
hipError_t launch_fq_batch(const FqArgs* rows, const FqArgs& cw, void* ws_w, const FqArgs& cdy,
                           void* ws_dy, const FqArgs& cx, void* ws_x, int qg, int qw,
                           hipStream_t st);

// Both passes of one bf16 matrix from a single read (fwht_dual.hip): the rows pass ar and
// the columns pass ac of the same x (same block and code type qt), with one scratch whose
// size fq_dual_ws_bytes gives (0: the shape is not covered: rows and cols multiples of 256,
// block <= 256).  fq_dual_supported also asks that all 256 x 256 tiles fit on the device at
// once and that both passes round to nearest.
size_t fq_dual_ws_bytes(int64_t rows, int64_t cols, int block, int in_bf16);
bool fq_dual_supported(int64_t rows, int64_t cols, int block, int in_bf16, int qt, bool sr_rows,
                       bool sr_cols, size_t ws_bytes);
hipError_t launch_fq_dual(const FqArgs& ar, const FqArgs& ac, void* ws, int qt, int prezeroed,
                          hipStream_t st);

// Zero n floats (also used for 32-bit counters).
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// Wave-per-slice rows kernel: rows of L = 64 j elements with 4096 % L == 0 or 4096 <= L <= 65536.
bool fq_rows2_supported(int64_t len, int block);
hipError_t launch_fq_rows2(const FqArgs& a, int in_bf16, int qt, hipStream_t st);

// Two rows passes of the same row length, block, input and code type in one launch (p1 is
// used when has1 != 0), which also clears `nzero` 32-bit words at `zero` (may be NULL).
struct FqPair {
  FqArgs p0, p1;
  int has1;
  int64_t split;  // set by the launcher
  uint32_t* zero;
  int64_t nzero;
};
hipError_t launch_fq_rows2_pair(const FqPair& a, int in_bf16, int qt, hipStream_t st);

// Up to two single-read column passes over columns of the same length, block, input type
// (in_bf16) and code type in one launch (a1 may be NULL).  prezeroed: the scratch of both was
// cleared earlier on st.
hipError_t launch_fq_cols2_pair(const FqArgs& a0, void* ws0, const FqArgs* a1, void* ws1,
                                int in_bf16, int qt, int prezeroed, hipStream_t st);

// Longest row the single-pass rows kernel takes for this block size.
int64_t fq_rows_max_len(int block);

struct GemmArgs {
  const void* a;  // [m x k], lda (bytes = elements)
  int64_t lda;
  const void* b;  // [n x k], ldb
  int64_t ldb;
  const float* sa;
  const float* sb;
  void* c;        // [m x n], ldc (elements)
  int64_t ldc;
  int64_t m, n, k;
};

// kind: 0 INT8, 1 FP8.  afmt/bfmt (FP8 only): 0 E4M3, 1 E5M2.  out: 0 int32, 1 fp32, 2 bf16.
hipError_t launch_gemm(const GemmArgs& g, int kind, int afmt, int bfmt, int out, hipStream_t st);
// Two products of the same kind, formats and output type in one launch (g1 may be NULL).
hipError_t launch_gemm_pair(const GemmArgs& g, const GemmArgs* g1, int kind, int afmt, int bfmt,
                            int out, hipStream_t st);

// Matrix-core rate probe (mfma_probe.hip): kind 0 INT8 32x32x32, 1 FP8 32x32x64, 2 FP8
// 16x16x128; mfma_probe_ops gives the operations one launch performs.
hipError_t launch_mfma_probe(int kind, int iters, hipStream_t st);
int64_t mfma_probe_ops(int kind, int iters);

// Let `Kernel` launch with `bytes` of dynamic LDS on the current device.  The attribute belongs
// to one kernel on one device, so it is set once per kernel and device (concurrent first calls
// may both set it); a failure is returned, and tried again on the next call.
template <auto Kernel>
hipError_t allow_dynamic_lds(int bytes) {
  static std::atomic<bool> done[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < 64;
  if (cached && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && cached) done[dev].store(true, std::memory_order_release);
  return e;
}

}  // namespace halo
