// gemm.hip -- 8-bit MFMA GEMM with a fused per-row x per-column dequant epilogue (gfx950).
//
// What is computed ("HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs",
// abstract: every large product of the forward and backward pass in low precision; key
// design 2: INT8 or FP8):  acc[i, j] = sum_t a[i, t] b[j, t] with INT8 codes accumulated in
// int32 (v_mfma_i32_32x32x32_i8) or FP8 codes accumulated in fp32 (the CDNA4
// v_mfma_f32_32x32x64_f8f6f4 with a per-operand format select), then
// c[i, j] = acc * sa[i] * sb[j] in fp32, rounded to bf16 or kept in fp32 (or the raw int32).
//
// Tiling.  A 256-thread workgroup (4 wave64s, 2 x 2) owns a 256 x 256 output tile; each wave
// owns 128 x 128 = 4 x 4 MFMA tiles of 32 x 32 with the accumulators resident in registers.
// Each K step moves a 256 x 128-byte slab of each operand global -> registers -> LDS, double
// buffered (2 x 64 KB of the 160 KB LDS): the next slab's global loads are in flight while
// the current slab feeds the matrix cores.  16-byte chunks are XOR-swizzled by the row's low
// 3 bits in LDS so the fragment reads of 8 consecutive rows spread over all banks.
// The product is formed transposed (the MFMA's first operand is the b tile), so each lane
// ends with 4 consecutive output columns of one row: 8- or 16-byte vector stores.
// Workgroups are numbered so that each of the 8 XCDs (workgroup i runs on XCD i % 8) gets a
// contiguous run of tiles, rastered in groups of 4 tile rows, for L2 reuse of both operands.
#include "halo_device.h"
#include "halo_kernels.h"

#include <mutex>

namespace halo {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int STAGE_BYTES = (BM + BN) * BK;  // 64 KB
constexpr int LDS_BYTES = 2 * STAGE_BYTES;   // 128 KB

__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

template <int OUT>
__device__ __forceinline__ void store4(void* c, int64_t ldc, int64_t row, int64_t col,
                                       int64_t n, const float* v, const int* iv) {
  if (col + 3 < n) {
    if constexpr (OUT == 0) {
      *reinterpret_cast<int4*>(reinterpret_cast<int*>(c) + row * ldc + col) =
          make_int4(iv[0], iv[1], iv[2], iv[3]);
    } else if constexpr (OUT == 1) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + row * ldc + col) =
          make_float4(v[0], v[1], v[2], v[3]);
    } else {
      uint2 w;
      w.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
      w.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(c) + row * ldc + col) = w;
    }
  } else {
    for (int i = 0; i < 4; ++i) {
      if (col + i >= n) break;
      if constexpr (OUT == 0)
        reinterpret_cast<int*>(c)[row * ldc + col + i] = iv[i];
      else if constexpr (OUT == 1)
        reinterpret_cast<float*>(c)[row * ldc + col + i] = v[i];
      else
        reinterpret_cast<uint16_t*>(c)[row * ldc + col + i] = (uint16_t)bf16_rne(v[i]);
    }
  }
}

// KIND 0: INT8.  KIND 1: FP8 with formats AF (a) and BF (b): 0 = E4M3, 1 = E5M2.
// OUT 0: int32 accumulators, 1: fp32, 2: bf16.
template <int KIND, int AF, int BF, int OUT>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) char smem[];

  // ---- tile of this workgroup -------------------------------------------------------
  const int tiles_m = (int)((g.m + BM - 1) / BM), tiles_n = (int)((g.n + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int q8 = T / 8, r8 = T % 8, xcd = bid % 8, slot = bid / 8;
  const int tile = xcd < r8 ? xcd * (q8 + 1) + slot : r8 * (q8 + 1) + (xcd - r8) * q8 + slot;
  constexpr int GROUP_M = 4;
  const int per_group = GROUP_M * tiles_n;
  const int first_m = (tile / per_group) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_grp = tile % per_group;
  const int64_t m0 = (int64_t)(first_m + in_grp % gm) * BM;
  const int64_t n0 = (int64_t)(in_grp / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global -> LDS assignment: chunk lc of rows lr + 32 i ------------------------
  const int lc = tid & 7, lr = tid >> 3;
  const char* __restrict__ A = reinterpret_cast<const char*>(g.a);
  const char* __restrict__ Bm = reinterpret_cast<const char*>(g.b);
  int64_t aoff[8], boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t ra = min(m0 + lr + 32 * i, g.m - 1);  // clamped rows feed unused outputs
    const int64_t rb = min(n0 + lr + 32 * i, g.n - 1);
    aoff[i] = ra * g.lda + lc * 16;
    boff[i] = rb * g.ldb + lc * 16;
  }
  uint4 ra_[8], rb_[8];
  auto gload = [&](int kt) {
    const int64_t koff = (int64_t)kt * BK;
    const bool in = koff + lc * 16 < g.k;  // k is a multiple of 16: chunks are all-in or all-out
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra_[i] = in ? *reinterpret_cast<const uint4*>(A + aoff[i] + koff) : make_uint4(0, 0, 0, 0);
      rb_[i] = in ? *reinterpret_cast<const uint4*>(Bm + boff[i] + koff) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    char* sa = smem + buf * STAGE_BYTES;
    char* sb = sa + BM * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<uint4*>(sa + lds_off(lr + 32 * i, lc)) = ra_[i];
      *reinterpret_cast<uint4*>(sb + lds_off(lr + 32 * i, lc)) = rb_[i];
    }
  };

  using Acc = typename std::conditional<KIND == 0, v16i, v16f>::type;
  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  const int fr = lane & 31, fh = lane >> 5;  // fragment row and K half
  auto compute = [&](int buf) {
    const char* sa = smem + buf * STAGE_BYTES;
    const char* sb = sa + BM * BK;
    if constexpr (KIND == 0) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {  // 32 bytes of K per MFMA
        v4i fa[4], fb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int rb = wn * 128 + t * 32 + fr, ra = wm * 128 + t * 32 + fr;
          fb[t] = *reinterpret_cast<const v4i*>(sb + lds_off(rb, ks * 2 + fh));
          fa[t] = *reinterpret_cast<const v4i*>(sa + lds_off(ra, ks * 2 + fh));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[i], fa[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {  // 64 bytes of K per MFMA
        v8i fa[4], fb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int rb = wn * 128 + t * 32 + fr, ra = wm * 128 + t * 32 + fr;
          const int c = ks * 4 + fh * 2;
          v4i b0 = *reinterpret_cast<const v4i*>(sb + lds_off(rb, c));
          v4i b1 = *reinterpret_cast<const v4i*>(sb + lds_off(rb, c + 1));
          v4i a0 = *reinterpret_cast<const v4i*>(sa + lds_off(ra, c));
          v4i a1 = *reinterpret_cast<const v4i*>(sa + lds_off(ra, c + 1));
          fb[t] = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          fa[t] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            // first operand = b tile (format BF), second = a tile (format AF); scales 2^0
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[i], fa[j], acc[i][j], BF, AF, 0, 127, 0, 127);
      }
    }
  };

  // ---- main loop -------------------------------------------------------------------
  const int nk = (int)((g.k + BK - 1) / BK);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute(cur);
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column block (r / 4) * 8 + fh * 4 + [0, 4) of row fr ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t row = m0 + wm * 128 + j * 32 + fr;
    if (row >= g.m) continue;
    const float sar = OUT == 0 ? 0.f : g.sa[row];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int64_t col = n0 + wn * 128 + i * 32 + gq * 8 + fh * 4;
        if (col >= g.n) continue;
        float v[4];
        int iv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (KIND == 0) iv[e] = acc[i][j][gq * 4 + e];
          else iv[e] = 0;
        }
        if constexpr (OUT != 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sbc = col + e < g.n ? g.sb[col + e] : 0.f;
            const float af = KIND == 0 ? (float)iv[e] : (float)acc[i][j][gq * 4 + e];
            v[e] = (af * sar) * sbc;
          }
        }
        store4<OUT>(g.c, g.ldc, row, col, g.n, v, iv);
      }
    }
  }
}

template <int KIND, int AF, int BF, int OUT>
static hipError_t launch_t(const GemmArgs& g, hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<KIND, AF, BF, OUT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<KIND, AF, BF, OUT>), dim3((unsigned)tiles), dim3(256), LDS_BYTES,
                     st, g);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, int kind, int afmt, int bfmt, int out, hipStream_t st) {
  if (kind == 0) {
    switch (out) {
      case 0: return launch_t<0, 0, 0, 0>(g, st);
      case 1: return launch_t<0, 0, 0, 1>(g, st);
      case 2: return launch_t<0, 0, 0, 2>(g, st);
    }
    return hipErrorInvalidValue;
  }
  const int sel = afmt * 2 + bfmt;
#define HALO_FP8_CASE(AFv, BFv)                                       \
  if (sel == AFv * 2 + BFv) {                                         \
    if (out == 1) return launch_t<1, AFv, BFv, 1>(g, st);             \
    if (out == 2) return launch_t<1, AFv, BFv, 2>(g, st);             \
  }
  HALO_FP8_CASE(0, 0)
  HALO_FP8_CASE(0, 1)
  HALO_FP8_CASE(1, 0)
  HALO_FP8_CASE(1, 1)
#undef HALO_FP8_CASE
  return hipErrorInvalidValue;
}

}  // namespace halo
