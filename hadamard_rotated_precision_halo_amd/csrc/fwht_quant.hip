// fwht_quant.hip -- fused blockwise Walsh-Hadamard rotation + per-vector absmax 8-bit
// quantisation on gfx950.
//
// What is computed ("QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术" s2.1-s2.2, s3.1;
// "HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs", key design 2): every
// vector is split into contiguous blocks of B elements, each block goes through the
// natural-order (Sylvester) butterfly network -- stage h = 1, 2, 4, ... pairs index t with
// t + h and replaces them by their sum and difference -- and the vector is quantised with
// one absmax scale.  The 1/sqrt(B) normalisation cancels in the codes (codes depend only on
// y / max|y|), so it is folded into the stored scale.
//
// Register layout.  A "chunk" is 8 consecutive elements along the rotated dimension, so the
// three lowest index bits are in-register butterflies.  The next index bits live across the
// G lanes of a lane group (exchanged with DPP / ds_swizzle / permlane), and the top bits are
// the U chunks a lane holds.  Stages always run in increasing bit order, which is the
// butterfly's own order: the fp32 results are bit-identical to a sequential fp32 butterfly.
//
// Rows kernel (vectors = rows, contiguous): one lane group owns one block of one row; a
// workgroup owns whole rows, so the row absmax is reduced in LDS in the same launch (one HBM
// read, one code write).
// Cols kernel (vectors = columns, strided): each lane loads 8 consecutive rows of NV adjacent
// columns, a free register transpose that turns them into NV chunks along the rotated
// dimension.  The column absmax spans many workgroups, so the kernel runs twice: a first
// sweep reduces the column maxima into the scale array with integer atomics (non-negative
// floats order like their bit patterns), the second recomputes the rotation and writes the
// transposed codes; a last tiny launch turns maxima into scales.
//
// Both kernels also take the options of a pass: the randomised transform's sign bits, zero
// padding past in_len, and stochastic rounding of the codes (store_chunk_opt).
#include "halo_device.h"
#include "halo_kernels.h"

namespace halo {

// ---------------------------------------------------------------------------
// compile-time geometry
// ---------------------------------------------------------------------------

__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Rows kernel: lanes per block and chunks per lane.
template <int B>
struct RowGeo {
  static constexpr int G = B < 8 ? 1 : (B <= 128 ? B / 8 : (B <= 1024 ? 16 : (B == 2048 ? 32 : 64)));
  static constexpr int U = B < 8 ? 1 : B / (8 * G);
  static constexpr int E = 8 * G * U;           // elements per item (= max(B, 8))
  static constexpr int IT = 64 / (8 * U);        // items per lane group
  static constexpr int NGROUPS = 256 / G;
  static constexpr int MAXV = 256;               // vectors per workgroup (LDS slots)
};

// Cols kernel: lanes per block, chunks per lane, columns per lane.
template <int B>
struct ColGeo {
  static constexpr int G = B < 8 ? 1 : (B <= 512 ? B / 8 : 64);
  static constexpr int U = B < 8 ? 1 : B / (8 * G);
  static constexpr int NV = 8 / U;               // 8, 4 (B=1024), 2 (2048), 1 (4096)
  static constexpr int E = 8 * G * U;
  static constexpr int NGROUPS = 256 / G;
  static constexpr int COLS = NGROUPS * NV;      // columns per workgroup
};

// In-chunk butterflies over the low log2(min(B, 8)) index bits.
template <int B>
__device__ __forceinline__ void chunk_butterflies(float* v) {
  if constexpr (B >= 2) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) { float p = v[i], q = v[i + 1]; v[i] = p + q; v[i + 1] = p - q; }
  }
  if constexpr (B >= 4) {
#pragma unroll
    for (int i = 0; i < 8; i += 4)
#pragma unroll
      for (int t = i; t < i + 2; ++t) { float p = v[t], q = v[t + 2]; v[t] = p + q; v[t + 2] = p - q; }
  }
  if constexpr (B >= 8) {
#pragma unroll
    for (int t = 0; t < 4; ++t) { float p = v[t], q = v[t + 4]; v[t] = p + q; v[t + 4] = p - q; }
  }
}

// Cross-lane stages over log2(G) lane bits, applied to n values per lane.
template <int G>
__device__ __forceinline__ void lane_butterflies(float* v, int n, int x) {
  if constexpr (G >= 2) {
    const float c = (x & 1) ? -1.f : 1.f;
    for (int i = 0; i < n; ++i) v[i] = xbutterfly<0>(v[i], c);
  }
  if constexpr (G >= 4) {
    const float c = (x & 2) ? -1.f : 1.f;
    for (int i = 0; i < n; ++i) v[i] = xbutterfly<1>(v[i], c);
  }
  if constexpr (G >= 8) {
    const float c = (x & 4) ? -1.f : 1.f;
    for (int i = 0; i < n; ++i) v[i] = xbutterfly<2>(v[i], c);
  }
  if constexpr (G >= 16) {
    const float c = (x & 8) ? -1.f : 1.f;
    for (int i = 0; i < n; ++i) v[i] = xbutterfly<3>(v[i], c);
  }
  if constexpr (G >= 32) {
    const float c = (x & 16) ? -1.f : 1.f;
    for (int i = 0; i < n; ++i) v[i] = xbutterfly<4>(v[i], c);
  }
  if constexpr (G >= 64) {
    const float c = (x & 32) ? -1.f : 1.f;
    for (int i = 0; i < n; ++i) v[i] = xbutterfly<5>(v[i], c);
  }
}

// Max over the G lanes of a group (all lanes end with the group max).
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2) v = xmax<0>(v);
  if constexpr (G >= 4) v = xmax<1>(v);
  if constexpr (G >= 8) v = xmax<2>(v);
  if constexpr (G >= 16) v = xmax<3>(v);
  if constexpr (G >= 32) v = xmax<4>(v);
  if constexpr (G >= 64) v = xmax<5>(v);
  return v;
}

// Butterflies across the U chunks of a lane (index bits above the lane bits); v is
// laid out as [U][8] for one vector.
template <int U>
__device__ __forceinline__ void chunk_stages(float* v) {
#pragma unroll
  for (int h = 1; h < U; h *= 2)
#pragma unroll
    for (int i = 0; i < U; i += 2 * h)
#pragma unroll
      for (int t = i; t < i + h; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float p = v[t * 8 + e], q = v[(t + h) * 8 + e];
          v[t * 8 + e] = p + q;
          v[(t + h) * 8 + e] = p - q;
        }
}

// Store the 8 codes / values of one chunk.  QT: 0 = INT8, 1 = E4M3, 2 = E5M2, 3 = fp32 values.
template <int QT>
__device__ __forceinline__ void store_chunk(void* dst, const float* y, float m) {
  if constexpr (QT == 0) {
    uint2 w;
    w.x = pack4(i8_code(y[0], m), i8_code(y[1], m), i8_code(y[2], m), i8_code(y[3], m));
    w.y = pack4(i8_code(y[4], m), i8_code(y[5], m), i8_code(y[6], m), i8_code(y[7], m));
    *reinterpret_cast<uint2*>(dst) = w;
  } else if constexpr (QT == 1 || QT == 2) {
    constexpr int F = QT - 1;
    uint2 w;
    w.x = fp8_pair<F>(mulz(y[0], m), mulz(y[1], m)) | (fp8_pair<F>(mulz(y[2], m), mulz(y[3], m)) << 16);
    w.y = fp8_pair<F>(mulz(y[4], m), mulz(y[5], m)) | (fp8_pair<F>(mulz(y[6], m), mulz(y[7], m)) << 16);
    *reinterpret_cast<uint2*>(dst) = w;
  } else {
    float4* d = reinterpret_cast<float4*>(dst);
    d[0] = make_float4(mulz(y[0], m), mulz(y[1], m), mulz(y[2], m), mulz(y[3], m));
    d[1] = make_float4(mulz(y[4], m), mulz(y[5], m), mulz(y[6], m), mulz(y[7], m));
  }
}

template <int QT>
struct CodeSize { static constexpr int value = QT == 3 ? 4 : 1; };

// Store one chunk, with stochastic rounding when the pass asks for it (code types only):
// element pos + e of vector vec rounds by its own Philox uniform.
template <int QT>
__device__ __forceinline__ void store_chunk_opt(void* dst, const float* y, float m, const FqArgs& a,
                                                int64_t vec, int64_t pos) {
  if constexpr (QT != 3) {
    if (a.sr) {
      uint32_t w[8];
      sr_words8(vec, pos, a.key0, a.key1, a.ctr2, a.ctr3, w);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sr_value<QT>(mulz(y[e], m), w[e], a.qmax);
      store_chunk<QT>(dst, v, 1.f);
      return;
    }
  }
  store_chunk<QT>(dst, y, m);
}

// ---------------------------------------------------------------------------
// rows kernel
// ---------------------------------------------------------------------------

template <typename Tin, int B, int QT>
__global__ __launch_bounds__(256) void fq_rows_kernel(FqArgs a) {
  using Geo = RowGeo<B>;
  constexpr int G = Geo::G, U = Geo::U, E = Geo::E, IT = Geo::IT, NG = Geo::NGROUPS;
  __shared__ uint32_t s_max[Geo::MAXV];
  __shared__ float s_mul[Geo::MAXV];
  __shared__ float s_pre[Geo::MAXV];  // factor the values take first (code_mul)

  const int tid = threadIdx.x;
  const int grp = tid / G, x = tid % G;
  const int64_t v0 = (int64_t)blockIdx.x * a.vec_per_wg;
  const int nv = (int)min<int64_t>(a.vec_per_wg, a.nvec - v0);
  const int items_per_vec = (int)(a.len / E);
  const int nitems = nv * items_per_vec;
  for (int i = tid; i < nv; i += 256) s_max[i] = 0u;
  __syncthreads();

  const Tin* __restrict__ xin = reinterpret_cast<const Tin*>(a.x);
  float val[IT][U * 8];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int item = grp + it * NG;
    if (item < nitems) {
      const int vec = item / items_per_vec, blk = item % items_per_vec;
      const Tin* vp = xin + (v0 + vec) * a.ldx;
      const int64_t pos = (int64_t)blk * E + x * 8;
#pragma unroll
      for (int u = 0; u < U; ++u)
        load8_vec<Tin>(vp, pos + u * 8 * G, a.in_len, a.signs, &val[it][u * 8]);
    } else {
#pragma unroll
      for (int i = 0; i < U * 8; ++i) val[it][i] = 0.f;
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
#pragma unroll
    for (int u = 0; u < U; ++u) chunk_butterflies<B>(&val[it][u * 8]);
    lane_butterflies<G>(val[it], U * 8, x);
    chunk_stages<U>(val[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < U * 8; ++i) mx = fmaxf(mx, fabsf(val[it][i]));
    mx = group_max<G>(mx);
    const int item = grp + it * NG;
    if (item < nitems && x == 0) atomicMax(&s_max[item / items_per_vec], __float_as_uint(mx));
  }
  __syncthreads();
  for (int i = tid; i < nv; i += 256) {
    const float amax = __uint_as_float(s_max[i]);
    float mul, sc, pre = 1.f;
    if (QT == 3) {
      mul = a.inv_sqrt_b;
      sc = amax * a.inv_sqrt_b;
    } else {
      mul = code_mul(a.qmax, amax, &pre);
      sc = amax / a.denom;
    }
    s_mul[i] = mul;
    s_pre[i] = pre;
    a.scale[v0 + i] = sc;
  }
  __syncthreads();
  constexpr int CS = CodeSize<QT>::value;
  char* qout = reinterpret_cast<char*>(a.q);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int item = grp + it * NG;
    if (item < nitems) {
      const int vec = item / items_per_vec, blk = item % items_per_vec;
      const float m = s_mul[vec], pre = s_pre[vec];
      if (pre != 1.f) {
#pragma unroll
        for (int i = 0; i < U * 8; ++i) val[it][i] *= pre;
      }
      const int64_t pos = (int64_t)blk * E + x * 8;
      char* p = qout + ((v0 + vec) * a.ldq + pos) * CS;
#pragma unroll
      for (int u = 0; u < U; ++u)
        store_chunk_opt<QT>(p + u * 8 * G * CS, &val[it][u * 8], m, a, v0 + vec, pos + u * 8 * G);
    }
  }
}

// ---------------------------------------------------------------------------
// cols kernels
// ---------------------------------------------------------------------------

// Load the NV columns x 8 rows a lane owns for one chunk, transposed to [NV][8]; rows from
// `nvalid` on are the zero padding and are not read.
template <typename Tin, int NV>
__device__ __forceinline__ void load_cols(const Tin* p, int64_t ldx, int64_t nvalid, float (*o)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e >= nvalid) {
#pragma unroll
      for (int c = 0; c < NV; ++c) o[c][e] = 0.f;
      continue;
    }
    const Tin* r = p + e * ldx;
    if constexpr (sizeof(Tin) == 2) {
      if constexpr (NV == 8) {
        uint4 w = *reinterpret_cast<const uint4*>(r);
        float t[8];
        unpack_bf16x8(w, t);
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c][e] = t[c];
      } else if constexpr (NV == 4) {
        uint2 w = *reinterpret_cast<const uint2*>(r);
        o[0][e] = __uint_as_float(w.x << 16); o[1][e] = __uint_as_float(w.x & 0xffff0000u);
        o[2][e] = __uint_as_float(w.y << 16); o[3][e] = __uint_as_float(w.y & 0xffff0000u);
      } else if constexpr (NV == 2) {
        uint32_t w = *reinterpret_cast<const uint32_t*>(r);
        o[0][e] = __uint_as_float(w << 16); o[1][e] = __uint_as_float(w & 0xffff0000u);
      } else {
        o[0][e] = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(r)) << 16);
      }
    } else {
#pragma unroll
      for (int c = 0; c < NV; ++c) o[c][e] = reinterpret_cast<const float*>(r)[c];
    }
  }
}

// MODE 0: column maxima into the (zeroed) max array.  MODE 1: transposed codes.
template <typename Tin, int B, int QT, int MODE>
__global__ __launch_bounds__(256) void fq_cols_kernel(FqArgs a) {
  using Geo = ColGeo<B>;
  constexpr int G = Geo::G, U = Geo::U, NV = Geo::NV, E = Geo::E;
  const int tid = threadIdx.x;
  const int grp = tid / G, x = tid % G;
  const int64_t c0 = (int64_t)blockIdx.x * Geo::COLS + grp * NV;  // first column of the lane
  const bool live = c0 < a.nvec;
  const Tin* __restrict__ xin = reinterpret_cast<const Tin*>(a.x);
  // blocks of E rows, grid-strided over y (the launcher caps the grid's y size)
  const int64_t nyb = a.len / E;
  for (int64_t yb = blockIdx.y; yb < nyb; yb += gridDim.y) {
    const int64_t r0 = yb * E;  // first row of the block
    float val[NV][U * 8];
    if (live) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float t[NV][8];
        const int64_t rb = r0 + u * 8 * G + x * 8;  // first row of the chunk
        load_cols<Tin, NV>(xin + rb * a.ldx + c0, a.ldx, a.in_len - rb, t);
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          if (a.signs) apply_signs8(t[c], a.signs, rb);
#pragma unroll
          for (int e = 0; e < 8; ++e) val[c][u * 8 + e] = t[c][e];
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NV; ++c)
#pragma unroll
        for (int i = 0; i < U * 8; ++i) val[c][i] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < NV; ++c) {
#pragma unroll
      for (int u = 0; u < U; ++u) chunk_butterflies<B>(&val[c][u * 8]);
      lane_butterflies<G>(val[c], U * 8, x);
      chunk_stages<U>(val[c]);
    }
    uint32_t* colmax = reinterpret_cast<uint32_t*>(a.scale);
    if constexpr (MODE == 0) {
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < U * 8; ++i) mx = fmaxf(mx, fabsf(val[c][i]));
        mx = group_max<G>(mx);
        if (live && x == 0) atomicMax(&colmax[c0 + c], __float_as_uint(mx));
      }
    } else {
      if (!live) return;
      constexpr int CS = CodeSize<QT>::value;
      char* qout = reinterpret_cast<char*>(a.q);
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const float amax = __uint_as_float(colmax[c0 + c]);
        float m = a.inv_sqrt_b, pre = 1.f;
        if constexpr (QT != 3) m = code_mul(a.qmax, amax, &pre);
        if (pre != 1.f) {
#pragma unroll
          for (int i = 0; i < U * 8; ++i) val[c][i] *= pre;
        }
        char* p = qout + ((c0 + c) * a.ldq + r0 + x * 8) * CS;
#pragma unroll
        for (int u = 0; u < U; ++u)
          store_chunk_opt<QT>(p + u * 8 * G * CS, &val[c][u * 8], m, a, c0 + c,
                              r0 + x * 8 + u * 8 * G);
      }
    }
  }
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// maxima (stored in place) -> scales
__global__ void finalize_scale_kernel(float* s, int64_t n, float div, float mul, int use_mul) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) s[i] = use_mul ? s[i] * mul : s[i] / div;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

template <typename Tin, int B, int QT>
static hipError_t launch_rows_t(const FqArgs& a0, hipStream_t st) {
  using Geo = RowGeo<B>;
  FqArgs a = a0;
  const int64_t items_per_vec = a.len / Geo::E;
  int64_t vpw = (int64_t)Geo::NGROUPS * Geo::IT / (items_per_vec > 0 ? items_per_vec : 1);
  if (vpw > Geo::MAXV) vpw = Geo::MAXV;
  if (vpw < 1) vpw = 1;
  a.vec_per_wg = vpw;
  const int64_t grid = (a.nvec + vpw - 1) / vpw;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((fq_rows_kernel<Tin, B, QT>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int B>
int64_t rows_max_len() {
  using Geo = RowGeo<B>;
  return (int64_t)Geo::NGROUPS * Geo::IT * Geo::E;
}

template <typename Tin, int B, int QT>
static hipError_t launch_cols_t(const FqArgs& a, hipStream_t st) {
  using Geo = ColGeo<B>;
  const int64_t ncol = a.nvec;
  if (ncol == 0) return hipSuccess;
  const unsigned zb = (unsigned)((ncol + 255) / 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(zb), dim3(256), 0, st, a.scale, ncol);
  if (a.len > 0) {
    const int64_t nyb = a.len / Geo::E;  // the kernel strides over the rest
    dim3 grid((unsigned)((ncol + Geo::COLS - 1) / Geo::COLS),
              (unsigned)(nyb < 65535 ? nyb : 65535));
    hipLaunchKernelGGL((fq_cols_kernel<Tin, B, QT, 0>), grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((fq_cols_kernel<Tin, B, QT, 1>), grid, dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(finalize_scale_kernel, dim3(zb), dim3(256), 0, st, a.scale, ncol, a.denom,
                     a.inv_sqrt_b, QT == 3 ? 1 : 0);
  return hipGetLastError();
}

template <typename Tin, int QT>
static hipError_t dispatch_block(const FqArgs& a, int axis, hipStream_t st) {
#define HALO_FQ_CASE(BB)                                                            \
  case BB:                                                                          \
    return axis == 0 ? launch_rows_t<Tin, BB, QT>(a, st) : launch_cols_t<Tin, BB, QT>(a, st);
  switch (a.block) {
    HALO_FQ_CASE(1) HALO_FQ_CASE(2) HALO_FQ_CASE(4) HALO_FQ_CASE(8) HALO_FQ_CASE(16)
    HALO_FQ_CASE(32) HALO_FQ_CASE(64) HALO_FQ_CASE(128) HALO_FQ_CASE(256) HALO_FQ_CASE(512)
    HALO_FQ_CASE(1024) HALO_FQ_CASE(2048) HALO_FQ_CASE(4096)
    default: return hipErrorInvalidValue;
  }
#undef HALO_FQ_CASE
}

int64_t fq_rows_max_len(int block) {
  switch (block) {
    case 1: return rows_max_len<1>();       case 2: return rows_max_len<2>();
    case 4: return rows_max_len<4>();       case 8: return rows_max_len<8>();
    case 16: return rows_max_len<16>();     case 32: return rows_max_len<32>();
    case 64: return rows_max_len<64>();     case 128: return rows_max_len<128>();
    case 256: return rows_max_len<256>();   case 512: return rows_max_len<512>();
    case 1024: return rows_max_len<1024>(); case 2048: return rows_max_len<2048>();
    case 4096: return rows_max_len<4096>();
    default: return 0;
  }
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_fwht_quant(const FqArgs& a, int in_bf16, int qt, int axis, void* ws,
                             size_t ws_bytes, hipStream_t st) {
  if (axis == 0 && fq_rows2_supported(a.len, a.block) && (in_bf16 || !a.sr))
    return launch_fq_rows2(a, in_bf16, qt, st);
  if (axis == 1 && fq_cols2_supported(a.len, a.nvec, a.block, in_bf16, a.sr != 0, ws_bytes))
    return launch_fq_cols2(a, in_bf16, qt, ws, st);
  if (in_bf16) {
    switch (qt) {
      case 0: return dispatch_block<uint16_t, 0>(a, axis, st);
      case 1: return dispatch_block<uint16_t, 1>(a, axis, st);
      case 2: return dispatch_block<uint16_t, 2>(a, axis, st);
      case 3: return dispatch_block<uint16_t, 3>(a, axis, st);
    }
  } else {
    switch (qt) {
      case 0: return dispatch_block<float, 0>(a, axis, st);
      case 1: return dispatch_block<float, 1>(a, axis, st);
      case 2: return dispatch_block<float, 2>(a, axis, st);
      case 3: return dispatch_block<float, 3>(a, axis, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace halo
