// fwht_rows.hip -- rotation + quantisation of rows (the contiguous dimension), wave-per-slice
// kernel for gfx950.
//
// What is computed is the same as in fwht_quant.hip ("QWHA方法：基于Walsh-Hadamard变换的高效
// 大模型微调技术" s2.1-s2.2, s3.1: natural-order butterflies over blocks of B contiguous indices,
// one absmax scale per row): this file only changes how the work maps onto the hardware.
//
// A wave owns 4096 consecutive elements of a row (64 per lane), so a row of up to 4096
// elements is rotated, reduced and quantised by one wave with no barrier, and longer rows by
// one workgroup of ceil(L / 4096) waves with a single LDS exchange of wave maxima.  Within a
// block of B >= 64 elements only g = B / 64 lanes take part: a lane holds 8 chunks of 8
// consecutive elements, chunk j of lane lo sitting at block offset (j * g + lo) * 8, so the 3
// low index bits and the 3 high index bits are butterflied in registers and only log2(g)
// stages cross lanes.  The two lowest lane stages are single v_fmac_f32 instructions with a
// DPP quad permutation on the partner value (z <- z + c * z[lane ^ s], c = +1 on the lower and
// -1 on the upper lane; the upper lane then holds the negated difference, a sign folded into
// its quantisation multiplier); higher lane stages use ds_swizzle / permlane.  All stages run
// in increasing index-bit order with the same operand order as a sequential fp32 butterfly,
// so the values are bit-identical to it.
#include "halo_device.h"
#include "halo_kernels.h"

namespace halo {

// z[i] <- z[i] + c * z[i] of lane ^ (1 << S), S = 0 or 1, for 8 values: one v_fmac_f32 with a
// DPP quad permutation of src0 each.  The leading s_nop covers the two wait states a DPP read
// needs after a VALU write of its source; inside the block each source was written earlier.
template <int S>
__device__ __forceinline__ void dpp_fmac8(float* z, float c) {
  if constexpr (S == 0) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]), "+v"(z[4]), "+v"(z[5]), "+v"(z[6]),
          "+v"(z[7])
        : "v"(c));
  } else {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "+v"(z[0]), "+v"(z[1]), "+v"(z[2]), "+v"(z[3]), "+v"(z[4]), "+v"(z[5]), "+v"(z[6]),
          "+v"(z[7])
        : "v"(c));
  }
}

// Butterflies between in-register values at index distance D (the values of one lane are
// v[j * 8 + e]; D is a power of two, the pair is (t, t + D) within groups of 2D).
template <int D>
__device__ __forceinline__ void reg_stage(float* v) {
#pragma unroll
  for (int i = 0; i < 64; i += 2 * D)
#pragma unroll
    for (int t = i; t < i + D; ++t) {
      const float p = v[t], q = v[t + D];
      v[t] = p + q;
      v[t + D] = p - q;
    }
}

// Encoders for 8 consecutive values (one chunk) -> 8 bytes of codes.
template <int QT>
__device__ __forceinline__ uint2 encode8(const float* y, float m) {
  uint2 w;
  if constexpr (QT == 0) {
    uint32_t t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = __float_as_uint(__builtin_fmaf(y[e], m, 12582912.0f));
    // v_perm_b32: byte 0 of each of two dwords -> bytes 0 and 1 (selector 0x0c zeroes)
    const uint32_t p01 = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(t[3], t[2], 0x0c0c0400u);
    const uint32_t p45 = __builtin_amdgcn_perm(t[5], t[4], 0x0c0c0400u);
    const uint32_t p67 = __builtin_amdgcn_perm(t[7], t[6], 0x0c0c0400u);
    w.x = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    w.y = __builtin_amdgcn_perm(p67, p45, 0x05040100u);
  } else {
    // v_cvt_pk_{fp8,bf8}_f32 writes one 16-bit half of its destination and keeps the other
    if constexpr (QT == 1) {
      w.x = __builtin_amdgcn_cvt_pk_fp8_f32(mulz(y[2], m), mulz(y[3], m),
                                            __builtin_amdgcn_cvt_pk_fp8_f32(mulz(y[0], m), mulz(y[1], m), 0, false), true);
      w.y = __builtin_amdgcn_cvt_pk_fp8_f32(mulz(y[6], m), mulz(y[7], m),
                                            __builtin_amdgcn_cvt_pk_fp8_f32(mulz(y[4], m), mulz(y[5], m), 0, false), true);
    } else {
      w.x = __builtin_amdgcn_cvt_pk_bf8_f32(mulz(y[2], m), mulz(y[3], m),
                                            __builtin_amdgcn_cvt_pk_bf8_f32(mulz(y[0], m), mulz(y[1], m), 0, false), true);
      w.y = __builtin_amdgcn_cvt_pk_bf8_f32(mulz(y[6], m), mulz(y[7], m),
                                            __builtin_amdgcn_cvt_pk_bf8_f32(mulz(y[4], m), mulz(y[5], m), 0, false), true);
    }
  }
  return w;
}

// Wave maximum over the lanes whose bits below LB vary (lanes of one row).
__device__ __forceinline__ float lane_max(float v, int lane_bits) {
  if (lane_bits > 0) v = xmax<0>(v);
  if (lane_bits > 1) v = xmax<1>(v);
  if (lane_bits > 2) v = xmax<2>(v);
  if (lane_bits > 3) v = xmax<3>(v);
  if (lane_bits > 4) v = xmax<4>(v);
  if (lane_bits > 5) v = xmax<5>(v);
  return v;
}

// QT: 0 INT8, 1 E4M3, 2 E5M2, 3 fp32 rotated values.
// NW waves per workgroup.  multi = 1: one row per workgroup, wave w owns columns
// [4096 w, 4096 (w + 1)).  multi = 0: 4096 % L == 0, each wave owns 4096 / L whole rows.
template <typename Tin, int B, int QT>
__global__ __launch_bounds__(1024) void fq_rows2_kernel(FqArgs a, int multi) {
  constexpr int G = B >= 64 ? B / 64 : 1;  // lanes per block
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int lo = lane % G, hi = lane / G;

  // element offset of the lane's chunk j within its wave's 4096-element slice
  auto chunk_off = [&](int j) -> int {
    return B >= 64 ? hi * B + (j * G + lo) * 8 : lane * 64 + j * 8;
  };
  int64_t row;
  int col0;  // column of the slice start within the row
  int row_lanes_log2;
  bool valid;
  if (multi) {
    row = blockIdx.x;
    col0 = w * 4096;
    row_lanes_log2 = 6;
    valid = col0 + chunk_off(0) < a.len;  // lanes past the row end idle (a whole lane or none)
  } else {
    const int L = (int)a.len;
    const int rpw = 4096 / L;              // rows per wave
    const int first = (blockIdx.x * nw + w) * rpw;
    const int r_in_wave = chunk_off(0) / L;
    row = (int64_t)first + r_in_wave;
    col0 = -r_in_wave * L;                 // so that col0 + chunk_off(j) is the column
    row_lanes_log2 = 31 - __builtin_clz((unsigned)(L / 64));
    valid = row < a.nvec;
  }
  const Tin* __restrict__ xin = reinterpret_cast<const Tin*>(a.x);
  // idle lanes (past the row end, or past the last row) read the first chunk of row 0
  const Tin* rp = xin + (valid ? row : 0) * a.ldx;

  float v[64];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = valid ? col0 + chunk_off(j) : 0;
    load8<Tin>(rp + c, &v[j * 8]);
  }

  // ---- butterflies, increasing index bits ---------------------------------------------
  // bits 0-2: within each chunk
  if constexpr (B >= 2) reg_stage<1>(v);
  if constexpr (B >= 4) reg_stage<2>(v);
  if constexpr (B >= 8) reg_stage<4>(v);
  float sgn = 1.f;
  if constexpr (B >= 64) {
    // lane stages (bits 3 .. 3 + log2(G) - 1)
    if constexpr (G >= 2) {
      const float c = (lo & 1) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 64; i += 8) dpp_fmac8<0>(&v[i], c);
      sgn *= c;
    }
    if constexpr (G >= 4) {
      const float c = (lo & 2) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 64; i += 8) dpp_fmac8<1>(&v[i], c);
      sgn *= c;
    }
    if constexpr (G >= 8) {
      const float c = (lo & 4) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = xbutterfly<2>(v[i], c);
    }
    if constexpr (G >= 16) {
      const float c = (lo & 8) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = xbutterfly<3>(v[i], c);
    }
    if constexpr (G >= 32) {
      const float c = (lo & 16) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = xbutterfly<4>(v[i], c);
    }
    if constexpr (G >= 64) {
      const float c = (lo & 32) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = xbutterfly<5>(v[i], c);
    }
    // top bits: the 8 chunks of the lane
    reg_stage<8>(v);
    reg_stage<16>(v);
    reg_stage<32>(v);
  } else {
    // blocks of 16 or 32 elements: chunk bits inside the block
    if constexpr (B >= 16) reg_stage<8>(v);
    if constexpr (B >= 32) reg_stage<16>(v);
  }

  // ---- row absmax -----------------------------------------------------------------------
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 64; i += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, fabsf(v[i])), fabsf(v[i + 1]));
  if (!valid) mx = 0.f;
  mx = lane_max(mx, row_lanes_log2);
  if (multi && nw > 1) {
    __shared__ float s_wmax[16];
    if (lane == 0) s_wmax[w] = mx;
    __syncthreads();
    mx = 0.f;
    for (int i = 0; i < nw; ++i) mx = __builtin_fmaxf(mx, s_wmax[i]);
  }

  // ---- quantise and store ---------------------------------------------------------------
  float mul;
  if constexpr (QT == 3) mul = a.inv_sqrt_b;
  else mul = mx > 0.f ? a.qmax / mx : 0.f;
  const bool writer = multi ? (w == 0 && lane == 0) : ((lane & ((1 << row_lanes_log2) - 1)) == 0);
  if (valid && writer) a.scale[row] = QT == 3 ? mx * a.inv_sqrt_b : mx / a.denom;
  if (!valid) return;
  mul *= sgn;
  if constexpr (QT == 3) {
    float* qp = reinterpret_cast<float*>(a.q) + row * a.ldq;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* y = &v[j * 8];
      float4* d = reinterpret_cast<float4*>(qp + col0 + chunk_off(j));
      d[0] = make_float4(mulz(y[0], mul), mulz(y[1], mul), mulz(y[2], mul), mulz(y[3], mul));
      d[1] = make_float4(mulz(y[4], mul), mulz(y[5], mul), mulz(y[6], mul), mulz(y[7], mul));
    }
  } else {
    uint8_t* qp = reinterpret_cast<uint8_t*>(a.q) + row * a.ldq;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint2*>(qp + col0 + chunk_off(j)) = encode8<QT>(&v[j * 8], mul);
  }
}

template <typename Tin, int B, int QT>
static hipError_t launch_rows2_t(const FqArgs& a, hipStream_t st) {
  const int64_t L = a.len;
  if (a.nvec == 0) return hipSuccess;
  if (L >= 4096) {
    const int nw = (int)((L + 4095) / 4096);
    hipLaunchKernelGGL((fq_rows2_kernel<Tin, B, QT>), dim3((unsigned)a.nvec), dim3(64 * nw), 0, st,
                       a, 1);
  } else {
    const int64_t rpw = 4096 / L;
    const int64_t waves = (a.nvec + rpw - 1) / rpw;
    const int nw = 4;
    hipLaunchKernelGGL((fq_rows2_kernel<Tin, B, QT>), dim3((unsigned)((waves + nw - 1) / nw)),
                       dim3(64 * nw), 0, st, a, 0);
  }
  return hipGetLastError();
}

bool fq_rows2_supported(int64_t len, int block) {
  if (len <= 0 || len % 64 != 0 || len > 16 * 4096) return false;
  if (len < 4096 && 4096 % len != 0) return false;
  return block >= 1 && block <= 4096 && len % block == 0;
}

template <typename Tin, int QT>
static hipError_t rows2_block(const FqArgs& a, hipStream_t st) {
#define HALO_R2_CASE(BB) \
  case BB: return launch_rows2_t<Tin, BB, QT>(a, st);
  switch (a.block) {
    HALO_R2_CASE(1) HALO_R2_CASE(2) HALO_R2_CASE(4) HALO_R2_CASE(8) HALO_R2_CASE(16)
    HALO_R2_CASE(32) HALO_R2_CASE(64) HALO_R2_CASE(128) HALO_R2_CASE(256) HALO_R2_CASE(512)
    HALO_R2_CASE(1024) HALO_R2_CASE(2048) HALO_R2_CASE(4096)
    default: return hipErrorInvalidValue;
  }
#undef HALO_R2_CASE
}

hipError_t launch_fq_rows2(const FqArgs& a, int in_bf16, int qt, hipStream_t st) {
  if (in_bf16) {
    switch (qt) {
      case 0: return rows2_block<uint16_t, 0>(a, st);
      case 1: return rows2_block<uint16_t, 1>(a, st);
      case 2: return rows2_block<uint16_t, 2>(a, st);
      case 3: return rows2_block<uint16_t, 3>(a, st);
    }
  } else {
    switch (qt) {
      case 0: return rows2_block<float, 0>(a, st);
      case 1: return rows2_block<float, 1>(a, st);
      case 2: return rows2_block<float, 2>(a, st);
      case 3: return rows2_block<float, 3>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace halo
