// halo_device.h -- gfx950 device helpers shared by the rotation and GEMM kernels.
//
// Lane exchanges for the cross-lane butterfly stages, bf16/fp32 unpacking, and the 8-bit
// encoders.  Every exchange pairs lane l with lane l ^ (1 << s) inside a wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace halo {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// element loads
// ---------------------------------------------------------------------------

__device__ __forceinline__ void unpack_bf16x8(uint4 w, float* o) {
  o[0] = __uint_as_float(w.x << 16);
  o[1] = __uint_as_float(w.x & 0xffff0000u);
  o[2] = __uint_as_float(w.y << 16);
  o[3] = __uint_as_float(w.y & 0xffff0000u);
  o[4] = __uint_as_float(w.z << 16);
  o[5] = __uint_as_float(w.z & 0xffff0000u);
  o[6] = __uint_as_float(w.w << 16);
  o[7] = __uint_as_float(w.w & 0xffff0000u);
}

// 8 consecutive elements (16 B of bf16 or 32 B of fp32) starting at p.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* o);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* o) {
  unpack_bf16x8(*reinterpret_cast<const uint4*>(p), o);
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* o) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// ---------------------------------------------------------------------------
// cross-lane partner values
// ---------------------------------------------------------------------------

// Value held by lane (l ^ (1 << S)).  S = 0, 1: DPP quad permutations; S = 2, 3, 4:
// ds_swizzle in bit mode (xor within 32 lanes); S = 5: permlane32 swap.
template <int S>
__device__ __forceinline__ float partner(float v) {
  int i = __float_as_int(v);
  if constexpr (S == 0) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false));
  } else if constexpr (S == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false));
  } else if constexpr (S == 2) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x101F));
  } else if constexpr (S == 3) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x201F));
  } else if constexpr (S == 4) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(i, 0x401F));
  } else {
    static_assert(S == 5, "lane exchange stage out of range");
    auto r = __builtin_amdgcn_permlane32_swap(i, i, false, false);
    // lanes 0-31 receive lanes 32-63 in r[1]; lanes 32-63 receive lanes 0-31 in r[0]
    return __int_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

// One butterfly stage across lanes: the lane whose bit S is clear holds the lower index p
// and becomes p + q; its partner holds q and becomes p - q.  `c` is +1 on the lower lane and
// -1 on the upper one, so one fma gives v + o or o - v with a single rounding each -- the
// same association as an in-register butterfly, hence bit-identical to a sequential fp32
// butterfly.
template <int S>
__device__ __forceinline__ float xbutterfly(float v, float c) {
  return __builtin_fmaf(c, v, partner<S>(v));
}

template <int S>
__device__ __forceinline__ float xmax(float v) {
  return fmaxf(v, partner<S>(v));
}

// ---------------------------------------------------------------------------
// encoders
// ---------------------------------------------------------------------------

// Round-to-nearest-even of y * m for |y * m| <= 2^22, returned as the int8 bit pattern in the
// low byte: fma adds 1.5 * 2^23 to the exact product and rounds once, leaving the integer in
// the low mantissa bits.
__device__ __forceinline__ uint32_t i8_code(float y, float m) {
  return __float_as_uint(__builtin_fmaf(y, m, 12582912.0f)) & 0xffu;
}

__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return a | (b << 8) | (c << 16) | (d << 24);
}

// fl32(y * m) with an exact zero product returned as +0: fma adds +0 to the exact product,
// and -0 + +0 = +0 under round to nearest, while every nonzero product is rounded once as by
// a plain multiply.  A zero has one code, +0, whichever sign the butterflies left on it.
__device__ __forceinline__ float mulz(float y, float m) { return __builtin_fmaf(y, m, 0.0f); }

// Two fp32 values to two OCP FP8 codes (round to nearest even), placed in the low 16 bits.
template <int FMT>  // 0: E4M3, 1: E5M2
__device__ __forceinline__ uint32_t fp8_pair(float a, float b) {
  if constexpr (FMT == 0)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false) & 0xffffu;
}

// ---------------------------------------------------------------------------
// randomised transform and stochastic rounding
// ---------------------------------------------------------------------------

// Signs of the randomised transform H D for the 8 consecutive elements starting at position
// pos (a multiple of 8) of a vector: bit i of the packed sign stream negates element i.
__device__ __forceinline__ void apply_signs8(float* v, const uint32_t* signs, int64_t pos) {
  const uint32_t b = signs[pos >> 5] >> (pos & 31);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (((b >> e) & 1u) << 31));
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11): ten rounds, each multiplying counter words 0 and 2 by the Philox constants and
// forming (hi(c2 m1) ^ c1 ^ k0, lo(c2 m1), hi(c0 m0) ^ c3 ^ k1, lo(c0 m0)); the key advances
// by the Weyl increments between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32 x 32 -> 64-bit product each (v_mad_u64_u32 gives both halves at once); each
    // three-way xor is one v_bitop3_b32 (truth table 0x96), the key word in a scalar register
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p2 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p2 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c0 = n0;
    c1 = (uint32_t)p2;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return make_uint4(c0, c1, c2, c3);
}

// Multiplier of the fp32 code decision, m = fl32(qmax / amax) (0 for a zero vector).  For a
// vector of values so small that this overflows (amax below qmax / FLT_MAX) the decision is
// taken on the vector scaled by 2^64: the scaling is exact for values this small, and the
// butterflies (additions with gradual underflow) commute with it, so the codes are those of
// the scaled vector, as absmax quantisation's scale invariance asks.  *pre receives the factor
// the values take before the multiplier (1 or 2^64).
__device__ __forceinline__ float code_mul(float qmax, float amax, float* pre) {
  float m = amax > 0.f ? qmax / amax : 0.f;
  *pre = 1.f;
  if (m > __FLT_MAX__) {
    *pre = 0x1p64f;
    m = qmax / (amax * 0x1p64f);
  }
  return m;
}

// Chunk of 8 elements at position pos (a multiple of 8) of the vector whose element 0 is at
// v0: zeros at and past in_len (the padding, never read), then the transform's signs.
template <typename T>
__device__ __forceinline__ void load8_vec(const T* v0, int64_t pos, int64_t in_len,
                                          const uint32_t* signs, float* o) {
  if (pos < in_len) {
    load8<T>(v0 + pos, o);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
  }
  if (signs) apply_signs8(o, signs, pos);
}

// The 24-bit uniforms w (u = w / 2^24) of positions pos .. pos + 7 (pos a multiple of 8) of
// vector vec: word p % 4 of Philox4x32-10 at counter (p / 4, vec, c2, c3), top 24 bits.
__device__ __forceinline__ void sr_words8(int64_t vec, int64_t pos, uint32_t k0, uint32_t k1,
                                          uint32_t c2, uint32_t c3, uint32_t* w) {
  const uint32_t c0 = (uint32_t)(pos >> 2), c1 = (uint32_t)vec;
  const uint4 r0 = philox4x32_10(c0, c1, c2, c3, k0, k1);
  const uint4 r1 = philox4x32_10(c0 + 1u, c1, c2, c3, k0, k1);
  w[0] = r0.x >> 8; w[1] = r0.y >> 8; w[2] = r0.z >> 8; w[3] = r0.w >> 8;
  w[4] = r1.x >> 8; w[5] = r1.y >> 8; w[6] = r1.z >> 8; w[7] = r1.w >> 8;
}

// Stochastic rounding of t (|t| <= qmax after the clamp; an exact zero already +0) to the grid
// of the code type: the grid point below t plus one step when w / 2^24 is below the fraction
// of the way to the next point.  QT 0: INT8 (step 1); 1: E4M3, 2: E5M2 (step = the quantum
// of |t|'s binade, the subnormal quantum below the smallest normal).  Every step is exact in
// fp32 (the steps are powers of two) except the fraction of a negative t above -2^-24, which
// rounds to 1.  The result is a grid value; a zero result is +0.
template <int QT>
__device__ __forceinline__ float sr_value(float t, uint32_t w, float qmax) {
  t = __builtin_amdgcn_fmed3f(t, -qmax, qmax);  // the clamp in one v_med3_f32 (t is finite)
  float s = 1.f, inv = 1.f;
  if constexpr (QT != 0) {
    constexpr uint32_t MB = QT == 1 ? 3u : 2u;         // mantissa bits
    constexpr uint32_t EMINB = QT == 1 ? 121u : 113u;  // fp32 biased exponent of the min normal
    uint32_t e = (__float_as_uint(t) >> 23) & 0xffu;
    e = e < EMINB ? EMINB : e;
    s = __uint_as_float((e - MB) << 23);
    inv = __uint_as_float((254u - e + MB) << 23);
  }
  const float r = t * inv;
  const float fl = floorf(r);
  const float up = (float)w < (r - fl) * 16777216.0f ? 1.f : 0.f;
  return (fl + up) * s;
}

}  // namespace halo
