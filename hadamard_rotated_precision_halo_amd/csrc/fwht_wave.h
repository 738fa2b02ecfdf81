// fwht_wave.h -- rotation + quantisation with one wave per 4096-element slice, for gfx950:
// rows (the contiguous axis) and columns (the strided axis, codes written transposed).
//
// What is computed is the same as in fwht_quant.hip ("QWHA方法：基于Walsh-Hadamard变换的高效
// 大模型微调技术" s2.1-s2.2, s3.1: natural-order butterflies over blocks of B contiguous indices
// of each vector, one absmax scale per vector): this file only changes how the work maps onto
// the hardware.
//
// Wave slice.  A wave holds 4096 elements of one or more vectors, 64 per lane, as 8 chunks of
// 8 consecutive elements.  For B >= 64, g = B / 64 lanes share a block and chunk j of lane lo
// sits at block offset (j * g + lo) * 8, so the 3 low index bits and the 3 high index bits of
// a block are butterflied in registers and only log2(g) stages cross lanes; for B < 64 a lane
// holds 64 / B whole blocks.  The two lowest lane stages are single v_fmac_f32 instructions
// with a DPP quad permutation on the partner value (z <- z + c * z[lane ^ s], c = +1 on the
// lower and -1 on the upper lane; the upper lane then holds the negated difference, a sign
// folded into its quantisation multiplier); higher lane stages use ds_swizzle / permlane.
// All stages run in increasing index-bit order with the same operand order as a sequential
// fp32 butterfly, so the values are bit-identical to it.
//
// Rows kernel.  A wave reads its slice straight from HBM: 4096 / L whole rows when L <= 4096
// (no barrier), or a workgroup of ceil(L / 4096) waves per row with one LDS exchange of wave
// maxima.
//
// Columns kernel.  A workgroup of 16 waves owns a tile of C = 65536 / R columns by R rows:
// whole columns (R = 4096, C = 16: 32-byte row segments, no exchange) for columns of up to
// 4096 rows, R = 1024 (C = 64: full 128-byte row segments) for longer ones.  Each lane loads 8
// consecutive rows of 8 adjacent columns, transposes them in registers with v_perm_b32 (8 rows
// of one column in one 16-byte word) and writes them to LDS in the order the compute waves
// read them (bank-conflict-free by an XOR swizzle); the waves then run the slice computation
// on column segments of R rows.  fp32 input keeps the tile's geometry and passes it through
// the LDS in two rounds of half the rows each (see cols_load_f32).  When a column is longer than R, the P = rows / R workgroups
// of one column strip combine their partial maxima through device-scope atomics: each
// max-reduces its maxima into the strip's column maxima, increments the strip's arrival
// counter, and waits until all P have arrived.  The tasks of a group of up to 8 strips are
// consecutive workgroups, the parts of each strip 8 apart (one XCD), so the parts of a strip
// normally run side by side and the input is read once and the codes written once.  No
// result depends on that: the wait is bounded, a task that reaches the bound marks its strip
// late and stops without storing, and the repair launch that follows on the stream stores
// every part of a late strip from the then complete maxima (see cols_task), so every call
// ends with the same codes whatever else occupies the device.
//
// Options (every kernel here): the randomised transform's signs ("企业官网建设流程全解析" s4.2,
// one bit per element, applied before the butterflies), zero padding of vectors whose length
// the block does not divide ("QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术" s5: in_len
// input elements, len rotated positions), and stochastic rounding of the codes (the same s5;
// a template parameter, instantiated in fwht_wave_sr.hip).
#pragma once

#include "halo_device.h"
#include "halo_kernels.h"

#include <atomic>

namespace halo {

// ---------------------------------------------------------------------------
// wave-slice helpers
// ---------------------------------------------------------------------------

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

// Lane geometry of a block of B elements inside a wave slice.
template <int B>
struct Slice {
  static constexpr int G = B >= 64 ? B / 64 : 1;  // lanes per block
  // element offset of chunk j of `lane` within the 4096-element slice
  __device__ static __forceinline__ int off(int lane, int j) {
    if constexpr (B >= 64) return (lane / G) * B + (j * G + lane % G) * 8;
    else return lane * 64 + j * 8;
  }
  // inverse: the lane and chunk holding slice offset o (a multiple of 8)
  __device__ static __forceinline__ void where(int o, int& lane, int& j) {
    if constexpr (B >= 64) {
      const int r = (o % B) / 8;
      lane = (o / B) * G + r % G;
      j = r / G;
    } else {
      lane = o / 64;
      j = (o % 64) / 8;
    }
  }
};

// Rotate the 64 values of a lane in place; returns the sign the DPP stages left on them.
template <int B>
__device__ __forceinline__ float rotate64(float* v, int lane) {
  constexpr int G = Slice<B>::G;
  const int lo = lane % G;
  if constexpr (B >= 2) reg_stage<1>(v);
  if constexpr (B >= 4) reg_stage<2>(v);
  if constexpr (B >= 8) reg_stage<4>(v);
  float sgn = 1.f;
  if constexpr (B >= 64) {
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
  return sgn;
}

__device__ __forceinline__ float absmax64(const float* v) {
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 64; i += 2)
    mx = __builtin_fmaxf(__builtin_fmaxf(mx, fabsf(v[i])), fabsf(v[i + 1]));
  return mx;
}

// Maximum over the lanes whose low `lane_bits` lane-index bits vary (the lanes of one vector).
__device__ __forceinline__ float lane_max(float v, int lane_bits) {
  if (lane_bits > 0) v = xmax<0>(v);
  if (lane_bits > 1) v = xmax<1>(v);
  if (lane_bits > 2) v = xmax<2>(v);
  if (lane_bits > 3) v = xmax<3>(v);
  if (lane_bits > 4) v = xmax<4>(v);
  if (lane_bits > 5) v = xmax<5>(v);
  return v;
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

// Store chunk j of the lane (8 values y) at element `idx` of the code array: 8 code bytes, or
// 8 fp32 rotated values for the value mode (QT 3).
template <int QT>
__device__ __forceinline__ void store_chunk8(void* q, int64_t idx, const float* y, float mul) {
  if constexpr (QT == 3) {
    float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(q) + idx);
    d[0] = make_float4(mulz(y[0], mul), mulz(y[1], mul), mulz(y[2], mul), mulz(y[3], mul));
    d[1] = make_float4(mulz(y[4], mul), mulz(y[5], mul), mulz(y[6], mul), mulz(y[7], mul));
  } else {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(q) + idx) = encode8<QT>(y, mul);
  }
}

// The same with stochastic rounding (code types only): element pos + e of vector vec takes
// the grid point below or above y * mul by its own Philox uniform.
template <int QT>
__device__ __forceinline__ void store_chunk8_sr(void* q, int64_t idx, const float* y, float mul,
                                                const FqArgs& a, int64_t vec, int64_t pos) {
  uint32_t w[8];
  sr_words8(vec, pos, a.key0, a.key1, a.ctr2, a.ctr3, w);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = sr_value<QT>(mulz(y[e], mul), w[e], a.qmax);
  *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(q) + idx) = encode8<QT>(v, 1.f);
}

// Store the 8 chunks of a lane: codes of vector vec, whose chunk j sits at position
// pos0 + off(lane, j) of the vector and at element base + off(lane, j) of the code array.
// SR: stochastic rounding (a separate instantiation, so that the nearest-even kernels keep
// their register budget).
template <int B, int QT, bool SR>
__device__ __forceinline__ void store_slice(const FqArgs& a, const float* v, float mul,
                                            int64_t base, int lane, int64_t vec, int64_t pos0) {
  using S = Slice<B>;
  if constexpr (SR && QT != 3) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      store_chunk8_sr<QT>(a.q, base + S::off(lane, j), &v[j * 8], mul, a, vec,
                          pos0 + S::off(lane, j));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) store_chunk8<QT>(a.q, base + S::off(lane, j), &v[j * 8], mul);
  }
}

// Staged code stores.  In the slice layout a store instruction of store_slice writes the
// wave's codes as 16 runs of 32 bytes (chunk j of the lanes of each block); written
// contiguously, 16 bytes per lane and 1 KB per instruction, the same codes leave the CU in
// fewer, whole-line requests.  A wave whose codes form one contiguous run (rows of 4096 or
// more positions) writes its chunks into its own LDS area at their slice offsets and reads
// them back contiguously.  Every 256 bytes of the area are followed by 32 bytes of padding, so
// the 8-byte chunk writes of 32 lanes (8 blocks, 32 contiguous bytes each) and the 16-byte
// read-back both touch all 64 banks once.
constexpr int kStageBytes = 4096 + 16 * 32;  // LDS bytes per wave

__device__ __forceinline__ int stage_off(int b) { return b + (b >> 8) * 32; }

// The 8 codes of chunk j of the lane (nearest, or stochastic rounding as store_chunk8_sr).
template <int QT, bool SR>
__device__ __forceinline__ uint2 chunk_codes(const FqArgs& a, const float* y, float mul,
                                             int64_t vec, int64_t pos) {
  if constexpr (SR) {
    uint32_t w[8];
    sr_words8(vec, pos, a.key0, a.key1, a.ctr2, a.ctr3, w);
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = sr_value<QT>(mulz(y[e], mul), w[e], a.qmax);
    return encode8<QT>(t, 1.f);
  } else {
    return encode8<QT>(y, mul);
  }
}

// store_slice for code types through the wave's LDS area `st`: the codes at slice offsets
// [0, n) (n a multiple of 16; the lanes holding them call this) go to elements base + [0, n)
// of the code array.
template <int B, int QT, bool SR>
__device__ __forceinline__ void store_slice_staged(const FqArgs& a, const float* v, float mul,
                                                   int64_t base, int lane, int64_t vec,
                                                   int64_t pos0, int n, uint8_t* st) {
  using S = Slice<B>;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int o = S::off(lane, j);
    *reinterpret_cast<uint2*>(st + stage_off(o)) =
        chunk_codes<QT, SR>(a, &v[j * 8], mul, vec, pos0 + o);
  }
  // the wave's LDS accesses complete in order: the reads see every lane's writes
  uint8_t* q = reinterpret_cast<uint8_t*>(a.q) + base;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = i * 1024 + lane * 16;
    if (b < n) *reinterpret_cast<uint4*>(q + b) = *reinterpret_cast<const uint4*>(st + stage_off(b));
  }
}

// Load the 8 chunks of a lane: chunk j at position pos0 + off(lane, j) of the vector whose
// element 0 is at vp.  The loads are unconditional (a chunk of the zero padding, at and past
// in_len, reads chunk 0 instead), so they issue back to back; only passes with padding then
// zero those chunks.  Then the transform's signs.
template <typename Tin, int B>
__device__ __forceinline__ void load_slice(const FqArgs& a, const Tin* vp, int64_t pos0, int lane,
                                           bool valid, float* v) {
  using S = Slice<B>;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t pos = pos0 + S::off(lane, j);
    load8<Tin>(vp + (valid && pos < a.in_len ? pos : 0), &v[j * 8]);
  }
  if (a.in_len < a.len) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (pos0 + S::off(lane, j) >= a.in_len) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j * 8 + e] = 0.f;
      }
  }
  if (a.signs) {
#pragma unroll
    for (int j = 0; j < 8; ++j) apply_signs8(&v[j * 8], a.signs, valid ? pos0 + S::off(lane, j) : 0);
  }
}

// Quantisation multiplier from the vector's absmax, for the lane's 64 values v of a vector
// (the rotated values' 1/sqrt(block) in the fp32 value mode): a vector of tiny values has them
// scaled first (code_mul).
template <int QT>
__device__ __forceinline__ float quant_mul_v(const FqArgs& a, float mx, float* v) {
  if constexpr (QT == 3) {
    return a.inv_sqrt_b;
  } else {
    float pre;
    const float m = code_mul(a.qmax, mx, &pre);
    if (pre != 1.f) {
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] *= pre;
    }
    return m;
  }
}
template <int QT>
__device__ __forceinline__ float stored_scale(const FqArgs& a, float mx) {
  return QT == 3 ? mx * a.inv_sqrt_b : mx / a.denom;
}

// ---------------------------------------------------------------------------
// rows kernel
// ---------------------------------------------------------------------------

// One wave's slice of a rows pass with L <= 4096 and 4096 % L == 0: wave `gw` of the pass owns
// rows [gw * 4096 / L, (gw + 1) * 4096 / L).  Lanes past the last row idle.
template <typename Tin, int B, int QT, bool SR>
__device__ __forceinline__ void rows_wave(const FqArgs& a, int64_t gw, int lane) {
  using S = Slice<B>;
  const int L = (int)a.len;
  const int64_t rpw = 4096 / L;              // rows per wave
  const int r_in_wave = S::off(lane, 0) / L;
  const int64_t row = gw * rpw + r_in_wave;
  const int col0 = -r_in_wave * L;           // so that col0 + off(lane, j) is the column
  const int row_lanes_log2 = 31 - __builtin_clz((unsigned)(L / 64));
  const bool valid = row < a.nvec;
  const Tin* __restrict__ xin = reinterpret_cast<const Tin*>(a.x);
  // idle lanes read the first chunk of row 0
  const Tin* rp = xin + (valid ? row : 0) * a.ldx;
  float v[64];
  load_slice<Tin, B>(a, rp, col0, lane, valid, v);
  const float sgn = rotate64<B>(v, lane);
  float mx = valid ? absmax64(v) : 0.f;
  mx = lane_max(mx, row_lanes_log2);
  const bool writer = (lane & ((1 << row_lanes_log2) - 1)) == 0;
  if (!valid) return;
  if (writer) a.scale[row] = stored_scale<QT>(a, mx);
  const float mul = quant_mul_v<QT>(a, mx, v) * sgn;
  store_slice<B, QT, SR>(a, v, mul, row * a.ldq + col0, lane, row, col0);
}

// QT: 0 INT8, 1 E4M3, 2 E5M2, 3 fp32 rotated values.
// multi = 1: one row per workgroup, wave w owns columns [4096 w, 4096 (w + 1)).
// multi = 0: 4096 % L == 0, each wave owns 4096 / L whole rows.
// One launch serves up to two passes of the same geometry (workgroups below pp.split run the
// first), and can clear a scratch range for the column passes that follow it on the stream.
template <typename Tin, int B, int QT, bool SR>
__global__ __launch_bounds__(1024) void fq_rows2_kernel(FqPair pp, int multi) {
  using S = Slice<B>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  // code types: each wave's staging area for contiguous code stores (launched with
  // nw * kStageBytes of dynamic LDS)
  extern __shared__ __attribute__((aligned(16))) uint8_t s_stage[];
  uint8_t* st = s_stage + (int)__builtin_amdgcn_readfirstlane(w) * kStageBytes;
  if (pp.zero) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pp.nzero; i += stride)
      pp.zero[i] = 0u;
  }
  const bool second = (int64_t)blockIdx.x >= pp.split;
  const FqArgs a = second ? pp.p1 : pp.p0;
  const int bid = (int)(blockIdx.x - (second ? pp.split : 0));
  if (!multi) {
    if (QT != 3 && a.len == 4096) {
      // one whole row per wave: its codes are one contiguous run of 4096 bytes
      const int64_t row = (int64_t)bid * nw + w;
      if (row >= a.nvec) return;
      const Tin* rp = reinterpret_cast<const Tin*>(a.x) + row * a.ldx;
      float v[64];
      load_slice<Tin, B>(a, rp, 0, lane, true, v);
      const float sgn = rotate64<B>(v, lane);
      const float mx = lane_max(absmax64(v), 6);
      if (lane == 0) a.scale[row] = stored_scale<QT>(a, mx);
      const float mul = quant_mul_v<QT>(a, mx, v) * sgn;
      store_slice_staged<B, QT, SR>(a, v, mul, row * a.ldq, lane, row, 0, 4096, st);
      return;
    }
    rows_wave<Tin, B, QT, SR>(a, (int64_t)bid * nw + w, lane);
    return;
  }
  const int64_t row = bid;
  const int col0 = w * 4096;
  const bool valid = col0 + S::off(lane, 0) < a.len;  // lanes past the row end idle (whole lanes)
  const Tin* __restrict__ xin = reinterpret_cast<const Tin*>(a.x);
  const Tin* rp = xin + row * a.ldx;
  float v[64];
  load_slice<Tin, B>(a, rp, col0, lane, valid, v);
  const float sgn = rotate64<B>(v, lane);
  float mx = valid ? absmax64(v) : 0.f;
  mx = lane_max(mx, 6);
  if (nw > 1) {
    __shared__ float s_wmax[16];
    if (lane == 0) s_wmax[w] = mx;
    __syncthreads();
    mx = 0.f;
    for (int i = 0; i < nw; ++i) mx = __builtin_fmaxf(mx, s_wmax[i]);
  }
  if (w == 0 && lane == 0) a.scale[row] = stored_scale<QT>(a, mx);
  if constexpr (QT != 3) {
    // the wave's codes: positions [col0, min(col0 + 4096, len)) of the row, contiguous (len is
    // a multiple of 64 here, so the run is a multiple of 16 bytes).  Every lane takes part:
    // the read-back gives bytes to lanes by position, and lanes past the row end write their
    // chunks past the run, which is not stored
    const float mul = quant_mul_v<QT>(a, mx, v) * sgn;
    const int64_t rest = a.len - col0;
    store_slice_staged<B, QT, SR>(a, v, mul, row * a.ldq + col0, lane, row, col0,
                                  (int)(rest < 4096 ? rest : 4096), st);
  } else {
    if (!valid) return;
    const float mul = quant_mul_v<QT>(a, mx, v) * sgn;
    store_slice<B, QT, SR>(a, v, mul, row * a.ldq + col0, lane, row, col0);
  }
}

// Workgroups of one rows pass (0 for an empty one).
static int64_t rows2_grid(const FqArgs& a) {
  if (a.nvec == 0) return 0;
  if (a.len > 4096) return a.nvec;
  const int64_t rpw = 4096 / a.len;
  const int64_t waves = (a.nvec + rpw - 1) / rpw;
  return (waves + 3) / 4;
}

template <typename Tin, int B, int QT, bool SR>
static hipError_t launch_rows2_t(FqPair pp, hipStream_t st) {
  const int64_t L = pp.p0.len;
  const int64_t g0 = rows2_grid(pp.p0), g1 = pp.has1 ? rows2_grid(pp.p1) : 0;
  pp.split = g0;
  const int64_t grid = g0 + g1;
  if (grid == 0) {
    if (pp.zero && pp.nzero > 0) return launch_fill_zero(reinterpret_cast<float*>(pp.zero), pp.nzero, st);
    return hipSuccess;
  }
  // rows of up to 4096 elements: whole rows per wave in 4-wave workgroups (for 4096, this
  // beat one single-wave workgroup per row: 11.74 against 11.43 us per 4096^2 pass)
  const int multi = L > 4096 ? 1 : 0;
  const int nw = multi ? (int)((L + 4095) / 4096) : 4;
  const int lds = QT != 3 && (multi || L == 4096) ? nw * kStageBytes : 0;
  if (lds > 65536) {
    const hipError_t e = allow_dynamic_lds<&fq_rows2_kernel<Tin, B, QT, SR>>(16 * kStageBytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((fq_rows2_kernel<Tin, B, QT, SR>), dim3((unsigned)grid), dim3(64 * nw), lds,
                     st, pp, multi);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// columns kernel
// ---------------------------------------------------------------------------

constexpr int kColsLdsBytes = 16 * 512 * 16;  // 16 waves x 512 chunks of 16 bytes

// LDS chunk (16-byte slot) of chunk j of `lane` in wave w: lane-major per wave, so the compute
// reads are contiguous; the XOR on the low 4 lane bits spreads the transposing writes over all
// 64 banks.
template <int B>
__device__ __forceinline__ int lds_slot(int w, int lane, int j) {
  constexpr int JA = B >= 64 ? B / 64 : 1;
  return w * 512 + j * 64 + (lane ^ (((j * JA) ^ w) & 15));
}

__device__ __forceinline__ uint32_t bf16_pair(uint32_t lo_word, uint32_t hi_word, int half) {
  // column `half` (0: low 16 bits, 1: high 16 bits) of two rows -> one dword, lower row first
  return __builtin_amdgcn_perm(hi_word, lo_word, half ? 0x07060302u : 0x05040100u);
}

// One column pass: its arguments, its geometry (R rows per task, P tasks per strip of C =
// 65536 / R columns) and its scratch (column maxima and per-strip arrival counters, both zero
// at launch; unused when P == 1).
struct ColsProb {
  FqArgs a;
  float* colmax;
  uint32_t* arrive;
  uint32_t* late;  // count of tasks that stopped waiting (their strips go to the repair)
  int R, P, C;
  int gs;          // strips per task group (see cols_task), 1 or 8
  uint32_t spins;  // polls of a waiting task before it stops waiting (see cols_task)
};

// Load part `part` (rows [part R, (part + 1) R)) of the column strip starting at column c0
// into the LDS tile: each thread reads 8 rows of 8 adjacent columns (16 bytes per row),
// transposes them in registers and writes 8 words of 8 rows of one column each.
template <int B>
__device__ __forceinline__ void cols_load(const ColsProb& pr, int64_t c0, int part, int t,
                                          uint4* lds) {
  using S = Slice<B>;
  const FqArgs& a = pr.a;
  const int R = pr.R, C = pr.C;
  const int CC = C / 8;                      // 16-byte column chunks per row of the tile
  const int cpw = 4096 / R;                  // column segments per wave
  const int cc = t % CC, rg = t / CC;        // column chunk, group of 8 rows
  const uint16_t* __restrict__ xin = reinterpret_cast<const uint16_t*>(a.x);
  const int64_t col = c0 + cc * 8;
  const bool cvalid = col < a.nvec;
  const int64_t r0 = (int64_t)part * R + rg * 8;  // first row of the group
  const uint16_t* p = xin + r0 * a.ldx + (cvalid ? col : 0);
  uint4 raw[8];
  // unconditional loads (a row of the zero padding, at and past in_len, reads row 0 instead);
  // only passes with padding then zero those rows
  const uint16_t* p0 = xin + (cvalid ? col : 0);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    raw[i] = *reinterpret_cast<const uint4*>(r0 + i < a.in_len ? p + i * a.ldx : p0);
  if (a.in_len < a.len) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (r0 + i >= a.in_len) raw[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (a.signs) {  // the transform's signs: one bit per row, on the bf16 sign bits
    const uint32_t b = a.signs[r0 >> 5] >> (r0 & 31);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t f = ((b >> i) & 1u) ? 0x80008000u : 0u;
      raw[i].x ^= f; raw[i].y ^= f; raw[i].z ^= f; raw[i].w ^= f;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int cl = cc * 8 + e;             // column within the tile
    const int wr = cl / cpw, ciw = cl % cpw;
    int ln, j;
    S::where(ciw * R + rg * 8, ln, j);
    uint32_t d0, d1, d2, d3;
    if ((e >> 1) == 0) {
      d0 = bf16_pair(raw[0].x, raw[1].x, e & 1); d1 = bf16_pair(raw[2].x, raw[3].x, e & 1);
      d2 = bf16_pair(raw[4].x, raw[5].x, e & 1); d3 = bf16_pair(raw[6].x, raw[7].x, e & 1);
    } else if ((e >> 1) == 1) {
      d0 = bf16_pair(raw[0].y, raw[1].y, e & 1); d1 = bf16_pair(raw[2].y, raw[3].y, e & 1);
      d2 = bf16_pair(raw[4].y, raw[5].y, e & 1); d3 = bf16_pair(raw[6].y, raw[7].y, e & 1);
    } else if ((e >> 1) == 2) {
      d0 = bf16_pair(raw[0].z, raw[1].z, e & 1); d1 = bf16_pair(raw[2].z, raw[3].z, e & 1);
      d2 = bf16_pair(raw[4].z, raw[5].z, e & 1); d3 = bf16_pair(raw[6].z, raw[7].z, e & 1);
    } else {
      d0 = bf16_pair(raw[0].w, raw[1].w, e & 1); d1 = bf16_pair(raw[2].w, raw[3].w, e & 1);
      d2 = bf16_pair(raw[4].w, raw[5].w, e & 1); d3 = bf16_pair(raw[6].w, raw[7].w, e & 1);
    }
    lds[lds_slot<B>(wr, ln, j)] = make_uint4(d0, d1, d2, d3);
  }
}

// fp32 input.  A task keeps the bf16 tile's geometry (R rows x C columns, 65536 values, each
// wave one slice of 4096), but in fp32 the tile is 256 KB, so it goes through the 128 KB LDS
// in two rounds.  Round h holds chunks 4 h .. 4 h + 3 of every lane (the 8-value chunks of
// Slice<B>): the rows whose offset in their column segment has bit HB equal to h, HB being the
// top bit of a block for B >= 64 (the chunk number is the top 3 bits of the offset in a block)
// and bit 5 below that (the chunk number is offset bits 3-5).  Every element is still read
// from HBM once: a thread issues both rounds' loads before the first is staged.
constexpr int lg2c(int v) { return v <= 1 ? 0 : 1 + lg2c(v / 2); }

// Row group (of 8 rows) of index i in round h: the group index with bit HB - 3 set to h.
template <int B>
__device__ __forceinline__ int f32_group(int i, int h) {
  constexpr int SH = lg2c(B >= 64 ? B : 64) - 4;  // HB - 3
  return ((i >> SH) << (SH + 1)) | (h << SH) | (i & ((1 << SH) - 1));
}

// LDS unit (16 bytes) holding half `half` (rows 0-3 or 4-7) of chunk j of `lane` in wave w,
// for the round that holds chunk j: lane-major per (chunk, half), so the compute reads are
// contiguous, with the bf16 tile's XOR on the low lane bits.
template <int B>
__device__ __forceinline__ int lds_unit_f32(int w, int lane, int j, int half) {
  constexpr int JA = B >= 64 ? B / 64 : 1;
  return w * 512 + (j & 3) * 128 + half * 64 + (lane ^ (((j * JA) ^ w) & 15));
}

// Both rounds' loads of part `part` of the strip at column c0: in round h each thread reads 8
// rows (row group f32_group(i, h)) of 4 adjacent columns, 16 bytes per row.
template <int B>
__device__ __forceinline__ void cols_load_f32(const ColsProb& pr, int64_t c0, int part, int t,
                                              uint4 (&raw)[2][8]) {
  const FqArgs& a = pr.a;
  const int R = pr.R, CC = pr.C / 4;         // 16-byte (4-column) chunks per tile row
  const int cc = t % CC, i = t / CC;         // column chunk, row-group index of a round
  const float* __restrict__ xin = reinterpret_cast<const float*>(a.x);
  const int64_t col = c0 + cc * 4;
  const float* p0 = xin + (col < a.nvec ? col : 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t r0 = (int64_t)part * R + f32_group<B>(i, h) * 8;
    const float* p = p0 + r0 * a.ldx;
    // rows of the zero padding read row 0 instead and are zeroed below
#pragma unroll
    for (int e = 0; e < 8; ++e)
      raw[h][e] = *reinterpret_cast<const uint4*>(r0 + e < a.in_len ? p + e * a.ldx : p0);
    if (a.in_len < a.len) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r0 + e >= a.in_len) raw[h][e] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (a.signs) {  // the transform's signs: one bit per row, on the fp32 sign bits
      const uint32_t b = a.signs[r0 >> 5] >> (r0 & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t f = ((b >> e) & 1u) ? 0x80000000u : 0u;
        raw[h][e].x ^= f; raw[h][e].y ^= f; raw[h][e].z ^= f; raw[h][e].w ^= f;
      }
    }
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int e) {
  return e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
}

// Round h into the LDS: each of the thread's 4 columns becomes the two 16-byte halves of one
// chunk (8 consecutive rows of that column).
template <int B>
__device__ __forceinline__ void cols_stage_f32(const ColsProb& pr, int t, int h,
                                               const uint4 (&raw)[8], uint4* lds) {
  using S = Slice<B>;
  const int R = pr.R, CC = pr.C / 4, cpw = 4096 / R;
  const int cc = t % CC, g8 = f32_group<B>(t / CC, h);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int cl = cc * 4 + e;               // column within the tile
    const int wr = cl / cpw, ciw = cl % cpw;
    int ln, j;
    S::where(ciw * R + g8 * 8, ln, j);
    lds[lds_unit_f32<B>(wr, ln, j, 0)] = make_uint4(word_of(raw[0], e), word_of(raw[1], e),
                                                    word_of(raw[2], e), word_of(raw[3], e));
    lds[lds_unit_f32<B>(wr, ln, j, 1)] = make_uint4(word_of(raw[4], e), word_of(raw[5], e),
                                                    word_of(raw[6], e), word_of(raw[7], e));
  }
}

// One task (one R-row part of one column strip) of a column pass, run by a whole workgroup of
// 16 waves.
// REPAIR: the second launch of an exchanging pass (see below): only the tasks of strips marked
// late run, with the column maxima complete by then.
// F32: fp32 input (two LDS rounds, see cols_load_f32); else bf16.
template <int B, int QT, bool SR, bool REPAIR = false, bool F32 = false>
__device__ __forceinline__ void cols_task(const ColsProb& pr, int64_t ltask, uint4* lds) {
  using S = Slice<B>;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const FqArgs& a = pr.a;
  const int R = pr.R, P = pr.P, C = pr.C;
  const int cpw = 4096 / R;                  // column segments per wave
  const int row_lanes_log2 = 31 - __builtin_clz((unsigned)(R / 64));
  float* colmax = pr.colmax;
  uint32_t* arrive = pr.arrive;
  const int64_t ncols = a.nvec;
  // the tasks of a strip group are consecutive (see the launcher); with one task per strip the
  // strips are spread so that each XCD (task i runs on XCD (i + offset) % 8) gets a contiguous
  // run of them: neighbouring strips share 128-byte lines, which its L2 then fetches once
  int64_t strip;
  int part;
  if (P == 1) {
    const int64_t T = (a.nvec + C - 1) / C, q = T / 8, r = T % 8, x = ltask % 8, s = ltask / 8;
    strip = x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
    part = 0;
  } else {
    // groups of gs strips, gs P tasks: part p of strip x of a group is task x + n p (n = the
    // group's strips), so with gs = 8 the P parts of a strip are 8 workgroups apart, on one
    // XCD, and their exchange stays in that XCD (measured faster than parts spread over
    // XCDs); gs = 1 makes them consecutive
    const int64_t gp = (int64_t)pr.gs * P, g = ltask / gp, j = ltask - g * gp;
    const int64_t T = (a.nvec + C - 1) / C, n = T - g * pr.gs < pr.gs ? T - g * pr.gs : pr.gs;
    strip = g * pr.gs + j % n;
    part = (int)(j / n);
  }
  const int64_t c0 = strip * C;
  constexpr uint32_t kMark = 0x80000000u;  // top bit of a strip's arrival count: marked late
  if constexpr (REPAIR) {
    // every task of the exchanging launch has finished, so every part's maxima are in colmax;
    // the tasks of strips marked late quantise and store their part again from them
    if (P == 1) return;
    __shared__ uint32_t s_mark;
    if (t == 0)
      s_mark = __hip_atomic_load(&arrive[strip], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kMark;
    __syncthreads();
    if (!s_mark) return;
  }

  // ---- load R rows x C columns, transposed into LDS, into the wave's slices ---------------
  float v[64];
  if constexpr (F32) {
    uint4 raw[2][8];
    cols_load_f32<B>(pr, c0, part, t, raw);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cols_stage_f32<B>(pr, t, h, raw[h], lds);
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * h + jj;
        const uint4 lo = lds[lds_unit_f32<B>(w, lane, j, 0)];
        const uint4 hi = lds[lds_unit_f32<B>(w, lane, j, 1)];
        v[j * 8 + 0] = __uint_as_float(lo.x); v[j * 8 + 1] = __uint_as_float(lo.y);
        v[j * 8 + 2] = __uint_as_float(lo.z); v[j * 8 + 3] = __uint_as_float(lo.w);
        v[j * 8 + 4] = __uint_as_float(hi.x); v[j * 8 + 5] = __uint_as_float(hi.y);
        v[j * 8 + 6] = __uint_as_float(hi.z); v[j * 8 + 7] = __uint_as_float(hi.w);
      }
      if (h == 0) __syncthreads();  // round 1 overwrites the LDS tile
    }
  } else {
    cols_load<B>(pr, c0, part, t, lds);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) unpack_bf16x8(lds[lds_slot<B>(w, lane, j)], &v[j * 8]);
  }

  // ---- rotate the wave's column segments --------------------------------------------------
  const int seg = S::off(lane, 0) / R;       // column segment of this lane within the wave
  const int64_t pos0 = (int64_t)part * R - (int64_t)seg * R;  // + off(lane, j): row index
  const float sgn = rotate64<B>(v, lane);
  const int64_t col = c0 + w * cpw + seg;
  const bool valid = col < ncols;
  float mx = lane_max(absmax64(v), row_lanes_log2);
  const bool writer = (lane & ((1 << row_lanes_log2) - 1)) == 0;

  // ---- column maxima of a strip split over P tasks -----------------------------------------
  // Device-scope atomics only (they are performed at the device's coherence point, across
  // XCDs): each task max-reduces its partial maxima into colmax (non-negative floats order
  // like their bit patterns) and waits for their returned values; one thread then counts the
  // task in and waits for all P; one thread per column reads the final maximum back with an
  // atomic load and shares it through LDS.  No cache-wide fence is needed.
  if (P > 1) {
    __shared__ float s_cmax[1024];
    uint32_t* cm = reinterpret_cast<uint32_t*>(colmax);
    if constexpr (!REPAIR) {
      __shared__ uint32_t s_late;
      uint32_t seen = 0;
      if (valid && writer)
        seen = __hip_atomic_fetch_max(&cm[col], __float_as_uint(mx), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      // every wave waits for the values its atomics return (so they have been performed at
      // the coherence point) before it reaches the barrier, so the arrival counted below
      // covers them: a workgroup barrier alone does not wait for outstanding memory
      // operations, and an unused return value would let the compiler drop the wait
      asm volatile("s_waitcnt vmcnt(0)" ::"v"(seen) : "memory");
      __syncthreads();
      // The wait is bounded by pr.spins polls.  The parts of a strip are close together in
      // the launch order and normally all resident at once, so the count completes long
      // before the bound; the bound matters only when other work holds the compute units
      // (another such pass on another stream whose tasks wait too).  A task that reaches it
      // marks the strip late and stops without storing; so does every task that finds the
      // mark.  The repair launch that follows on the stream stores every part of a marked
      // strip from the complete maxima: the same codes as an exchange that completes.
      if (t == 0) {
        uint32_t c = __hip_atomic_fetch_add(&arrive[strip], 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) + 1u;
        // the last task to arrive sees the full count at once and does not poll
        for (uint32_t it = 0; (c & ~kMark) < (uint32_t)P && !(c & kMark) && it < pr.spins; ++it) {
          __builtin_amdgcn_s_sleep(2);
          c = __hip_atomic_load(&arrive[strip], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const bool late = (c & kMark) || (c & ~kMark) < (uint32_t)P;
        if (late) {
          if (!(c & kMark))
            __hip_atomic_fetch_or(&arrive[strip], kMark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_fetch_add(pr.late, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        s_late = late ? 1u : 0u;
      }
      __syncthreads();
      if (s_late) return;
    }
    if (t < C && c0 + t < ncols)
      s_cmax[t] = __uint_as_float(__hip_atomic_load(&cm[c0 + t], __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    if (valid) mx = s_cmax[w * cpw + seg];
  }

  // ---- quantise and store the transposed codes ----------------------------------------------
  if (valid) {
    if (part == 0 && writer) a.scale[col] = stored_scale<QT>(a, mx);
    const float mul = quant_mul_v<QT>(a, mx, v) * sgn;
    store_slice<B, QT, SR>(a, v, mul, col * a.ldq + pos0, lane, col, pos0);
  }
}

// REPAIR: the follow-up launch of a pass whose strips are split over several tasks; it
// stores the parts of strips marked late (see cols_task) and returns at once for the rest.
// Whether any task of the passes whose late counters are given stopped waiting (read once by
// one thread of the workgroup and shared): the repair launches return at once when none did.
__device__ __forceinline__ bool any_late(const uint32_t* a, const uint32_t* b, const uint32_t* c) {
  __shared__ uint32_t s_any;
  if (threadIdx.x == 0) {
    uint32_t n = 0;
    if (a) n |= __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (b) n |= __hip_atomic_load(b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c) n |= __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_any = n;
  }
  __syncthreads();
  return s_any != 0;
}

template <int B, int QT, bool SR, bool REPAIR = false, bool F32 = false>
__global__ __launch_bounds__(1024) void fq_cols2_kernel(ColsProb c0, ColsProb c1, int64_t split,
                                                        int64_t tasks) {
  extern __shared__ __attribute__((aligned(16))) uint4 lds[];
  if constexpr (REPAIR) {
    if (!any_late(c0.P > 1 ? c0.late : nullptr, c1.P > 1 ? c1.late : nullptr, nullptr)) return;
  }
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const bool second = task >= split;
    const ColsProb pr = second ? c1 : c0;
    cols_task<B, QT, SR, REPAIR, F32>(pr, task - (second ? split : 0), lds);
    __syncthreads();  // the next task overwrites the LDS tile
  }
}

// The rotation passes of a layer backward in one launch: the rows of dY (codes QG) and the
// columns of W (QW), dY (QG) and X (QW).  The column passes come first, one task per
// workgroup, in that order; the rows pass follows, 16 waves per workgroup: its shorter tasks
// fill the tail of the launch.  All passes read bf16.
struct FqBatch {
  FqArgs rows;
  int64_t rows_wg;
  ColsProb cw, cdy, cx;
  int64_t end_w, end_dy, end_x;  // one past the last workgroup of each column pass
};

// SR: stochastic rounding of the dY codes (the W and X codes are rounded to nearest).
// REPAIR: the follow-up launch of the column passes (rows tasks excluded from its grid).
template <int B, int QG, int QW, bool SR, bool REPAIR = false>
__global__ __launch_bounds__(1024) void fq_batch_kernel(FqBatch fb) {
  extern __shared__ __attribute__((aligned(16))) uint4 lds[];
  if constexpr (REPAIR) {
    // a grid of at most one workgroup per compute unit, striding over the column tasks
    if (!any_late(fb.cw.P > 1 ? fb.cw.late : nullptr, fb.cdy.P > 1 ? fb.cdy.late : nullptr,
                  fb.cx.P > 1 ? fb.cx.late : nullptr))
      return;
    for (int64_t t = blockIdx.x; t < fb.end_w; t += gridDim.x) {
      cols_task<B, QW, false, true>(fb.cw, t, lds);
      __syncthreads();  // the next task overwrites the LDS tile
    }
    for (int64_t t = blockIdx.x; t < fb.end_dy - fb.end_w; t += gridDim.x) {
      cols_task<B, QG, SR, true>(fb.cdy, t, lds);
      __syncthreads();
    }
    for (int64_t t = blockIdx.x; t < fb.end_x - fb.end_dy; t += gridDim.x) {
      cols_task<B, QW, false, true>(fb.cx, t, lds);
      __syncthreads();
    }
    return;
  }
  const int64_t bid = blockIdx.x;
  if (bid < fb.end_w) {
    cols_task<B, QW, false>(fb.cw, bid, lds);
  } else if (bid < fb.end_dy) {
    cols_task<B, QG, SR>(fb.cdy, bid - fb.end_w, lds);
  } else if (bid < fb.end_x) {
    cols_task<B, QW, false>(fb.cx, bid - fb.end_dy, lds);
  } else {
    rows_wave<uint16_t, B, QG, SR>(fb.rows, (bid - fb.end_x) * 16 + (threadIdx.x >> 6),
                                   threadIdx.x & 63);
  }
}

// Rows per task for a column of `rows` elements (a power of two in [64, 4096] dividing rows
// and divisible by the block; 0 when the shape is not covered).  Columns of up to 4096 rows go
// whole into one task (4096 x 16 columns, or a wider tile for shorter columns): no exchange of
// partial maxima at all, and the strips' XCD-aware order keeps their 32-byte row segments
// fetched once per 128-byte line.  Longer columns take 1024-row tasks (64-column strips, full
// 128-byte row segments) and exchange their partial maxima.
static int cols2_rows_per_task(int64_t rows, int block) {
  int R = rows <= 4096 ? 4096 : 1024;
  if (block > R) R = block;
  while (R > rows) R >>= 1;
  while (R >= 64 && rows % R != 0) R >>= 1;
  if (R < 64 || R > 4096 || (R & (R - 1)) != 0) return 0;
  if (rows % R != 0 || R % block != 0) return 0;
  return R;
}

// Workgroups that can be resident at once (one per compute unit: the tile takes 128 KB of
// LDS), queried once per device.  Every kernel asking has the same 1024-thread, 128 KB LDS
// shape, so one cache serves them; concurrent first calls may both query and store the same
// value.
static int cols2_capacity(const void* fn) {
  static std::atomic<int> cap[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int known = cap[dev].load(std::memory_order_relaxed);
  if (known > 0) return known;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 1024, kColsLdsBytes) != hipSuccess)
    return 0;
  cap[dev].store(cus * per_cu, std::memory_order_relaxed);
  return cus * per_cu;
}

// Strips per task group of a pass with P parts per strip: 8 (one XCD per strip) when 8 P
// workgroups fit on the device at once, so that a group's waits can all end (the argument of
// the launchers below, with groups in place of strips); else 1.
static int cols2_group(int P, int capacity) { return P > 1 && 8 * P <= capacity ? 8 : 1; }

// Scratch layout of one pass: the count of tasks that stopped waiting for the other parts of
// their strip (one word, padded to 256 bytes), the arrival counters (padded to 256 bytes),
// then the column maxima.
constexpr size_t kColsLateBytes = 256;
static void cols2_scratch(void* ws, int64_t strips, float** colmax, uint32_t** arrive,
                          uint32_t** late, int64_t* words) {
  const size_t cnt = ((size_t)strips * 4 + 255) & ~(size_t)255;
  char* base = reinterpret_cast<char*>(ws);
  *late = reinterpret_cast<uint32_t*>(base);
  *arrive = reinterpret_cast<uint32_t*>(base + kColsLateBytes);
  *colmax = reinterpret_cast<float*>(base + kColsLateBytes + cnt);
  *words = (int64_t)((kColsLateBytes + cnt) / 4);
}

// Geometry and scratch of one column pass (rows = a.len); tasks = 0 for an empty pass.
static ColsProb cols2_prob(const FqArgs& a, void* ws, int64_t* tasks, int64_t* scratch_words) {
  ColsProb pr{};
  pr.a = a;
  pr.R = cols2_rows_per_task(a.len, a.block);
  pr.P = (int)(a.len / pr.R);
  pr.C = 65536 / pr.R;
  pr.gs = 1;
  const int64_t strips = (a.nvec + pr.C - 1) / pr.C;
  *tasks = (a.nvec == 0 || a.len == 0) ? 0 : strips * pr.P;
  *scratch_words = 0;
  if (pr.P > 1 && *tasks > 0) {
    cols2_scratch(ws, strips, &pr.colmax, &pr.arrive, &pr.late, scratch_words);
    *scratch_words += a.nvec;
    // polls a waiting task makes before it stops waiting and leaves its strip to the repair
    // launch (each an atomic load and s_sleep 2): the caller's count, else 2^20
    pr.spins = a.polls != 0 ? a.polls : (1u << 20);
  }
  return pr;
}

template <int B, int QT, bool SR, bool F32>
static hipError_t launch_cols2_t(const FqArgs& a0, void* ws0, const FqArgs* a1, void* ws1,
                                 int prezeroed, hipStream_t st) {
  auto* fn = &fq_cols2_kernel<B, QT, SR, false, F32>;
  hipError_t e = allow_dynamic_lds<&fq_cols2_kernel<B, QT, SR, false, F32>>(kColsLdsBytes);
  if (e != hipSuccess) return e;
  int64_t t0 = 0, t1 = 0, w0 = 0, w1 = 0;
  ColsProb p0 = cols2_prob(a0, ws0, &t0, &w0);
  ColsProb p1 = a1 ? cols2_prob(*a1, ws1, &t1, &w1) : p0;
  if (!prezeroed) {
    if (w0 > 0 && (e = launch_fill_zero(reinterpret_cast<float*>(ws0), w0, st)) != hipSuccess) return e;
    if (w1 > 0 && (e = launch_fill_zero(reinterpret_cast<float*>(ws1), w1, st)) != hipSuccess) return e;
  }
  if (t0 == 0) {  // keep the first slot filled: the kernel picks by task index
    p0 = p1;
    t0 = t1;
    t1 = 0;
  }
  const int64_t tasks = t0 + t1;
  if (tasks == 0) return hipSuccess;
  // one task per workgroup; the tasks of a group of gs strips (gs P tasks) are consecutive
  // workgroups, so the parts of a strip normally run side by side (one group fits on the
  // device at once: gs P <= the capacity, which cols2_group ensures).  Termination does not
  // rest on the dispatch order: every wait is bounded (see cols_task).
  const int P = p0.P > p1.P ? p0.P : p1.P;
  if (P > 1) {
    const int cap = cols2_capacity(reinterpret_cast<const void*>(fn));
    if (cap < P) return hipErrorInvalidConfiguration;
    p0.gs = p1.gs = cols2_group(P, cap);
  }
  hipLaunchKernelGGL((fq_cols2_kernel<B, QT, SR, false, F32>), dim3((unsigned)tasks), dim3(1024),
                     kColsLdsBytes, st, p0, p1, t0, tasks);
  e = hipGetLastError();
  if (e != hipSuccess || P == 1) return e;
  // the repair launch: stores the strips whose tasks stopped waiting.  Usually there are
  // none, and its workgroups (at most one per compute unit, striding over the tasks) return
  // after reading the late counters.
  e = allow_dynamic_lds<&fq_cols2_kernel<B, QT, SR, true, F32>>(kColsLdsBytes);
  if (e != hipSuccess) return e;
  const int cap = cols2_capacity(reinterpret_cast<const void*>(fn));
  const int64_t rgrid = tasks < cap ? tasks : cap;
  hipLaunchKernelGGL((fq_cols2_kernel<B, QT, SR, true, F32>), dim3((unsigned)rgrid), dim3(1024),
                     kColsLdsBytes, st, p0, p1, t0, tasks);
  return hipGetLastError();
}

template <int QT, bool SR, bool F32 = false>
static hipError_t cols2_block(const FqArgs& a0, void* ws0, const FqArgs* a1, void* ws1,
                              int prezeroed, hipStream_t st) {
#define HALO_C2_CASE(BB) \
  case BB: return launch_cols2_t<BB, QT, SR, F32>(a0, ws0, a1, ws1, prezeroed, st);
  switch (a0.block) {
    HALO_C2_CASE(1) HALO_C2_CASE(2) HALO_C2_CASE(4) HALO_C2_CASE(8) HALO_C2_CASE(16)
    HALO_C2_CASE(32) HALO_C2_CASE(64) HALO_C2_CASE(128) HALO_C2_CASE(256) HALO_C2_CASE(512)
    HALO_C2_CASE(1024) HALO_C2_CASE(2048) HALO_C2_CASE(4096)
    default: return hipErrorInvalidValue;
  }
#undef HALO_C2_CASE
}

// ---------------------------------------------------------------------------
// backward batch
// ---------------------------------------------------------------------------

template <int B, int QG, int QW, bool SR>
static hipError_t launch_batch_t(const FqArgs* rows, const FqArgs& cw, void* ws_w,
                                 const FqArgs& cdy, void* ws_dy, const FqArgs& cx, void* ws_x,
                                 hipStream_t st) {
  auto* fn = &fq_batch_kernel<B, QG, QW, SR>;
  hipError_t e = allow_dynamic_lds<&fq_batch_kernel<B, QG, QW, SR>>(kColsLdsBytes);
  if (e != hipSuccess) return e;
  FqBatch fb{};
  int64_t tw = 0, tdy = 0, tx = 0, scratch = 0;
  if (rows) {
    fb.rows = *rows;
    const int64_t waves = (rows->nvec * rows->len + 4095) / 4096;
    fb.rows_wg = rows->nvec == 0 ? 0 : (waves + 15) / 16;
  }
  fb.cw = cols2_prob(cw, ws_w, &tw, &scratch);
  fb.cdy = cols2_prob(cdy, ws_dy, &tdy, &scratch);
  fb.cx = cols2_prob(cx, ws_x, &tx, &scratch);
  fb.end_w = tw;
  fb.end_dy = fb.end_w + tdy;
  fb.end_x = fb.end_dy + tx;
  const int64_t grid = fb.end_x + fb.rows_wg;
  if (grid == 0) return hipSuccess;
  int P = fb.cw.P;
  if (fb.cdy.P > P) P = fb.cdy.P;
  if (fb.cx.P > P) P = fb.cx.P;
  if (P > 1) {
    const int cap = cols2_capacity(reinterpret_cast<const void*>(fn));
    if (cap < P) return hipErrorInvalidConfiguration;
    fb.cw.gs = cols2_group(fb.cw.P, cap);
    fb.cdy.gs = cols2_group(fb.cdy.P, cap);
    fb.cx.gs = cols2_group(fb.cx.P, cap);
  }
  hipLaunchKernelGGL((fq_batch_kernel<B, QG, QW, SR>), dim3((unsigned)grid), dim3(1024),
                     kColsLdsBytes, st, fb);
  e = hipGetLastError();
  if (e != hipSuccess || P == 1) return e;
  // the repair launch over the column tasks (see launch_cols2_t)
  e = allow_dynamic_lds<&fq_batch_kernel<B, QG, QW, SR, true>>(kColsLdsBytes);
  if (e != hipSuccess) return e;
  const int cap = cols2_capacity(reinterpret_cast<const void*>(fn));
  const int64_t rgrid = fb.end_x < cap ? fb.end_x : cap;
  hipLaunchKernelGGL((fq_batch_kernel<B, QG, QW, SR, true>), dim3((unsigned)rgrid),
                     dim3(1024), kColsLdsBytes, st, fb);
  return hipGetLastError();
}

template <int QG, int QW, bool SR>
static hipError_t batch_block(int block, const FqArgs* rows, const FqArgs& cw, void* ws_w,
                              const FqArgs& cdy, void* ws_dy, const FqArgs& cx, void* ws_x,
                              hipStream_t st) {
#define HALO_B_CASE(BB) \
  case BB: return launch_batch_t<BB, QG, QW, SR>(rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  switch (block) {
    HALO_B_CASE(1) HALO_B_CASE(2) HALO_B_CASE(4) HALO_B_CASE(8) HALO_B_CASE(16)
    HALO_B_CASE(32) HALO_B_CASE(64) HALO_B_CASE(128) HALO_B_CASE(256) HALO_B_CASE(512)
    HALO_B_CASE(1024) HALO_B_CASE(2048) HALO_B_CASE(4096)
    default: return hipErrorInvalidValue;
  }
#undef HALO_B_CASE
}

// ---------------------------------------------------------------------------
// rows dispatch
// ---------------------------------------------------------------------------

template <typename Tin, int QT, bool SR>
static hipError_t rows2_block(const FqPair& a, hipStream_t st) {
#define HALO_R2_CASE(BB) \
  case BB: return launch_rows2_t<Tin, BB, QT, SR>(a, st);
  switch (a.p0.block) {
    HALO_R2_CASE(1) HALO_R2_CASE(2) HALO_R2_CASE(4) HALO_R2_CASE(8) HALO_R2_CASE(16)
    HALO_R2_CASE(32) HALO_R2_CASE(64) HALO_R2_CASE(128) HALO_R2_CASE(256) HALO_R2_CASE(512)
    HALO_R2_CASE(1024) HALO_R2_CASE(2048) HALO_R2_CASE(4096)
    default: return hipErrorInvalidValue;
  }
#undef HALO_R2_CASE
}

// Stochastic-rounding instantiations of the launches (compiled in fwht_wave_sr.hip).
hipError_t cols2_dispatch_sr(const FqArgs& a0, void* ws0, const FqArgs* a1, void* ws1, int qt,
                             int prezeroed, hipStream_t st);
hipError_t batch_dispatch_sr(int qg, int qw, const FqArgs* rows, const FqArgs& cw, void* ws_w,
                             const FqArgs& cdy, void* ws_dy, const FqArgs& cx, void* ws_x,
                             hipStream_t st);
hipError_t rows2_dispatch_sr(const FqPair& a, int qt, hipStream_t st);

}  // namespace halo
