// gemm.hip -- 8-bit MFMA GEMM with a fused per-row x per-column dequant epilogue (gfx950).
//
// What is computed ("HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs",
// abstract: every large product of the forward and backward pass in low precision; key
// design 2: INT8 or FP8):  acc[i, j] = sum_t a[i, t] b[j, t] with INT8 codes accumulated in
// int32 (v_mfma_i32_32x32x32_i8) or FP8 codes on the CDNA4 v_mfma_*_32x32x64_f8f6f4 with a
// per-operand format select, then c[i, j] = (acc * sa[i]) * sb[j] in fp32, rounded to bf16 or
// kept in fp32 (or the raw int32 accumulators).
//
// Tiling.  A 256-thread workgroup (4 wave64s, 2 x 2) owns a 256 x 256 output tile; each wave
// owns 128 x 128 = 4 x 4 MFMA tiles of 32 x 32 with the accumulators resident in AGPRs.  K is
// consumed in slabs of BK bytes: a slab (256 rows of each operand) is staged in LDS with
// direct-to-LDS loads (global_load_lds_dwordx4: no VGPR staging, no ds_write) into a ring of
// NSTAGE slabs filling 128 KB of the 160 KB LDS.  One barrier per slab, placed before the
// slab's last MFMA sub-step: by then that sub-step's fragments are already in VGPRs, so the
// slab's ring slot is refilled right after the barrier (with the slab NSTAGE ahead) while the
// MFMAs keep the matrix cores busy, and the next slab's first fragments are read meanwhile.
// Operand fragments are double buffered in VGPRs one sub-step ahead.
//
// LDS layout.  Row r of a slab is BK bytes = BK / 16 chunks of 16 B; logical chunk c is stored
// at physical chunk c ^ swz(r).  A fragment read has the 16 lanes of a phase read 16
// consecutive rows at one logical chunk; the swizzle puts them in 16 distinct bank groups of
// the 64 banks.  Direct-to-LDS loads write 1 KB contiguous per wave instruction, so each lane
// loads the global chunk that belongs in its physical slot.
//
// The product is formed transposed (the MFMA's first operand is the b tile).  The epilogue
// stages each wave's results in LDS and reads them back row-contiguous, so the stores are
// full 256- or 512-byte row runs (bf16 output is dequantised and rounded before staging,
// halving the staged bytes); the scales sa, sb were loaded into LDS at kernel start.
// Workgroups are numbered so that each of the 8 XCDs (workgroup i runs on XCD i % 8) gets a
// contiguous run of tiles, rastered in groups of 4 tile rows, for L2 reuse of both operands.
#include "halo_device.h"
#include "halo_kernels.h"

#include <mutex>

namespace halo {

constexpr int BM = 256, BN = 256;
#ifndef HALO_GEMM_ORDERED
#define HALO_GEMM_ORDERED 1
#endif
constexpr int RING_BYTES = 128 * 1024;          // K-slab ring; the scales follow it
constexpr int LDS_BYTES = RING_BYTES + 2 * 256 * 4;

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t h = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// One 16-byte direct-to-LDS load per lane: the lane's 16 bytes at g land at lds + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, lds_void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// s_waitcnt immediate for vmcnt(n) with expcnt and lgkmcnt unconstrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define HALO_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

// Slab geometry for BK bytes of K per row.
template <int BK>
struct Slab {
  static constexpr int CHUNKS = BK / 16;               // 16-byte chunks per row
  static constexpr int OPER = BM * BK;                 // bytes per operand per slab
  static constexpr int STAGE = 2 * OPER;
  static constexpr int NSTAGE = RING_BYTES / STAGE;    // 4 (BK 64) or 2 (BK 128)
  static constexpr int INST = OPER / (256 * 16);       // loads per thread per operand
  static constexpr int RPI = 1024 / BK;                // rows one wave instruction fills
  // XOR the chunk with the row bits just above the 256-byte bank period.
  __device__ static __forceinline__ int swz(int r) {
    return BK == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7);
  }
  __device__ static __forceinline__ int off(int r, int c) { return r * BK + ((c ^ swz(r)) << 4); }
};

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
      w.x = pack_bf16x2(v[0], v[1]);
      w.y = pack_bf16x2(v[2], v[3]);
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
        reinterpret_cast<uint16_t*>(c)[row * ldc + col + i] = (uint16_t)pack_bf16x2(v[i], 0.f);
    }
  }
}

// KIND 0: INT8.  KIND 1: FP8 with formats AF (a) and BF (b): 0 = E4M3, 1 = E5M2.
// OUT 0: int32 accumulators, 1: fp32, 2: bf16.  MASK: fragments past k are zeroed (needed when
// k is not a multiple of the slab, or when the FP8 loop pads one extra slab).
template <int KIND, int AF, int BF, int OUT, bool MASK, int BK>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs g) {
  using SL = Slab<BK>;
  constexpr int NSTAGE = SL::NSTAGE, INST = SL::INST, RPI = SL::RPI;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  float* s_sa = reinterpret_cast<float*>(smem + RING_BYTES);
  float* s_sb = s_sa + 256;

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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases in SGPRs
  const int wm = wave >> 1, wn = wave & 1;

  // scales of this tile's rows and columns (written to LDS once the prologue loads landed)
  float my_sa = 0.f, my_sb = 0.f;
  if constexpr (OUT != 0) {
    my_sa = g.sa[min(m0 + tid, g.m - 1)];
    my_sb = g.sb[min(n0 + tid, g.n - 1)];
  }

  // ---- direct-to-LDS assignment -----------------------------------------------------
  // Wave w's instruction i fills LDS bytes [(INST w + i) KB, +1 KB) of an operand's slab =
  // rows 64 w + RPI i + [0, RPI); lane l lands in physical chunk l % CHUNKS of row
  // 64 w + RPI i + l / CHUNKS and loads that row's logical chunk (l % CHUNKS) ^ swz(row).
  const char* __restrict__ A = reinterpret_cast<const char*>(g.a);
  const char* __restrict__ Bm = reinterpret_cast<const char*>(g.b);
  uint32_t aoff[INST], boff[INST];  // byte offsets of the lane's rows (operands are < 4 GB)
  uint32_t cbo[INST];               // byte offset of the lane's chunk within a slab row
#pragma unroll
  for (int i = 0; i < INST; ++i) {
    const int r = wave * 64 + i * RPI + lane / SL::CHUNKS;
    cbo[i] = (uint32_t)(((lane % SL::CHUNKS) ^ SL::swz(r)) << 4);
    aoff[i] = (uint32_t)(min(m0 + r, g.m - 1) * g.lda);  // clamped rows feed unused outputs
    boff[i] = (uint32_t)(min(n0 + r, g.n - 1) * g.ldb);
  }
  const int nk = (int)((g.k + BK - 1) / BK);
  constexpr int KS = BK / (KIND == 0 ? 32 : 64);  // MFMA K sub-steps per slab
  constexpr int UNROLL = KS == 1 ? 2 : 1;          // keeps the fragment buffer index constant
  const int nkr = (nk + UNROLL - 1) / UNROLL * UNROLL;
  const uint32_t klast = (uint32_t)g.k - 16;       // last in-bounds chunk of a row

  // Stage slab kt into ring slot kt % NSTAGE: always 2 * INST direct-to-LDS loads per thread,
  // so the vmcnt arithmetic is uniform.  Slabs past the end reload the last slab (never read)
  // and chunks past k read the row's last chunk instead; their fragments are masked to zero.
  // loads [q0, q1) of the slab: load q is operand q % 2, row group q / 2
  auto stage_part = [&](int kt, int q0, int q1) __attribute__((always_inline)) {
    char* sa = smem + (kt % NSTAGE) * SL::STAGE;
    char* sb = sa + SL::OPER;
    const uint32_t kb = (uint32_t)min(kt, nk - 1) * BK;
#pragma unroll
    for (int q = 0; q < 2 * INST; ++q) {
      if (q < q0 || q >= q1) continue;
      const int i = q >> 1;
      uint32_t kc = kb + cbo[i];
      if constexpr (MASK) kc = min(kc, klast);
      if (q & 1) dma16(Bm + boff[i] + kc, (lds_void*)(sb + (wave * INST + i) * 1024));
      else dma16(A + aoff[i] + kc, (lds_void*)(sa + (wave * INST + i) * 1024));
    }
  };
  auto stage = [&](int kt) __attribute__((always_inline)) { stage_part(kt, 0, 2 * INST); };

  using Acc = typename std::conditional<KIND == 0, v16i, v16f>::type;
  using Frag = typename std::conditional<KIND == 0, v4i, v8i>::type;
  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  const int fr = lane & 31, fh = lane >> 5;  // fragment row and K half
  Frag fa[2][4], fb[2][4];
  auto load_frags = [&](int kt, int ks, Frag* da, Frag* db) __attribute__((always_inline)) {
    const char* sa = smem + (kt % NSTAGE) * SL::STAGE;
    const char* sb = sa + SL::OPER;
    const int c0 = KIND == 0 ? ks * 2 + fh : ks * 4 + fh * 2;  // first 16-byte chunk
    int keep0 = -1, keep1 = -1;
    if constexpr (MASK) {
      keep0 = (kt * BK + c0 * 16) < g.k ? -1 : 0;
      keep1 = (kt * BK + c0 * 16 + 16) < g.k ? -1 : 0;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rb = wn * 128 + t * 32 + fr, ra = wm * 128 + t * 32 + fr;
      if constexpr (KIND == 0) {
        db[t] = *reinterpret_cast<const v4i*>(sb + SL::off(rb, c0)) & keep0;
        da[t] = *reinterpret_cast<const v4i*>(sa + SL::off(ra, c0)) & keep0;
      } else {
        v4i b0 = *reinterpret_cast<const v4i*>(sb + SL::off(rb, c0)) & keep0;
        v4i b1 = *reinterpret_cast<const v4i*>(sb + SL::off(rb, c0 + 1)) & keep1;
        v4i a0 = *reinterpret_cast<const v4i*>(sa + SL::off(ra, c0)) & keep0;
        v4i a1 = *reinterpret_cast<const v4i*>(sa + SL::off(ra, c0 + 1)) & keep1;
        db[t] = Frag{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        da[t] = Frag{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
    }
  };
  auto mfma_step = [&](const Frag* da, const Frag* db) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (KIND == 0)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(db[i], da[j], acc[i][j], 0, 0, 0);
        else  // first operand = b tile (format BF), second = a tile (format AF); scales 2^0
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(db[i], da[j], acc[i][j], BF,
                                                                      AF, 0, 127, 0, 127);
      }
  };

  // ---- main loop -------------------------------------------------------------------
  // Sub-steps run in one flat sequence (slab kt, sub-step ks); the next sub-step's fragments
  // are read while the current one's 16 MFMAs issue.  Before the last sub-step of slab kt the
  // wave waits for its own loads of slab kt + 1 (later slabs may stay in flight), the barrier
  // makes every wave's loads visible, and slab kt + NSTAGE is issued into slab kt's slot,
  // which no wave reads any more.  The loop body has no branches, so the accumulators stay in
  // AGPRs; scheduling hints spread reads and loads between the MFMAs.
  constexpr int FRAG_READS = KIND == 0 ? 8 : 16;  // ds_read_b128 per sub-step
  auto hint_reads = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FRAG_READS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 fragment read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  };
  auto hint_reads_loads = [&]() __attribute__((always_inline)) {
    constexpr int LD = 2 * INST;  // slab loads to spread over the 16 MFMAs
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // 1 MFMA
      if (i < LD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // 1 slab load
      if (i < FRAG_READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
#if HALO_GEMM_ORDERED
  // Explicit issue order of a sub-step: MFMA t, then the sub-step's t-th fragment read and
  // t-th slab load (when there are that many); a scheduling barrier after each group keeps
  // the order, so the loads and reads are spread evenly between the MFMAs instead of being
  // issued in a burst that stalls the MFMA issue.
  auto read_one = [&](int kt, int ks, int q, Frag* da, Frag* db) __attribute__((always_inline)) {
    const char* sa = smem + (kt % NSTAGE) * SL::STAGE;
    const char* sb = sa + SL::OPER;
    const int c0 = KIND == 0 ? ks * 2 + fh : ks * 4 + fh * 2;
    if constexpr (KIND == 0) {
      const int t = q >> 1;
      int keep = -1;
      if constexpr (MASK) keep = (kt * BK + c0 * 16) < g.k ? -1 : 0;
      if (q & 1) da[t] = *reinterpret_cast<const v4i*>(sa + SL::off(wm * 128 + t * 32 + fr, c0)) & keep;
      else db[t] = *reinterpret_cast<const v4i*>(sb + SL::off(wn * 128 + t * 32 + fr, c0)) & keep;
    } else {
      const int t = q >> 2, h = q & 1;
      int keep = -1;
      if constexpr (MASK) keep = (kt * BK + (c0 + h) * 16) < g.k ? -1 : 0;
      if (q & 2) {
        const v4i v = *reinterpret_cast<const v4i*>(sa + SL::off(wm * 128 + t * 32 + fr, c0 + h)) & keep;
        if (h) da[t].hi = v; else da[t].lo = v;
      } else {
        const v4i v = *reinterpret_cast<const v4i*>(sb + SL::off(wn * 128 + t * 32 + fr, c0 + h)) & keep;
        if (h) db[t].hi = v; else db[t].lo = v;
      }
    }
  };
  auto load_one = [&](int kt, int q) __attribute__((always_inline)) { stage_part(kt, q, q + 1); };
  auto ordered_step = [&](const Frag* da, const Frag* db, int rkt, int rks, Frag* nda, Frag* ndb,
                          int nread, int lkt, int nload) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = t >> 2, j = t & 3;
      if constexpr (KIND == 0)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(db[i], da[j], acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(db[i], da[j], acc[i][j], BF,
                                                                    AF, 0, 127, 0, 127);
      if (t < nread) read_one(rkt, rks, t, nda, ndb);
      if (t < nload) load_one(lkt, t);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto do_slab = [&](int kt, auto P) __attribute__((always_inline)) {
    constexpr int P0 = decltype(P)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = (P0 + ks) & 1;
      if (ks + 1 < KS) {
        ordered_step(fa[cur], fb[cur], kt, ks + 1, fa[cur ^ 1], fb[cur ^ 1], FRAG_READS, 0, 0);
      } else {
        __builtin_amdgcn_s_waitcnt(HALO_VMCNT(2 * INST * (NSTAGE - 2)));  // slab kt + 1 landed
        __syncthreads();
        ordered_step(fa[cur], fb[cur], kt + 1, 0, fa[cur ^ 1], fb[cur ^ 1], FRAG_READS,
                     kt + NSTAGE, 2 * INST);
      }
    }
  };
#else
  auto do_slab = [&](int kt, auto P) __attribute__((always_inline)) {
    constexpr int P0 = decltype(P)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = (P0 + ks) & 1;
      if (ks + 1 < KS) {
        load_frags(kt, ks + 1, fa[cur ^ 1], fb[cur ^ 1]);
        mfma_step(fa[cur], fb[cur]);
        hint_reads();
      } else {
        __builtin_amdgcn_s_waitcnt(HALO_VMCNT(2 * INST * (NSTAGE - 2)));  // slab kt + 1 landed
        __syncthreads();
        stage(kt + NSTAGE);
        load_frags(kt + 1, 0, fa[cur ^ 1], fb[cur ^ 1]);
        mfma_step(fa[cur], fb[cur]);
        hint_reads_loads();
      }
    }
  };
#endif

#pragma unroll
  for (int t = 0; t < NSTAGE; ++t) stage(t);
  __builtin_amdgcn_s_waitcnt(HALO_VMCNT(2 * INST * (NSTAGE - 1)));  // slab 0 and the scales
  if constexpr (OUT != 0) {
    s_sa[tid] = my_sa;
    s_sb[tid] = my_sb;
  }
  __syncthreads();
  load_frags(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < nkr; kt += UNROLL) {
    do_slab(kt, std::integral_constant<int, 0>{});
    if constexpr (UNROLL == 2) do_slab(kt + 1, std::integral_constant<int, KS & 1>{});
  }
  __builtin_amdgcn_s_waitcnt(HALO_VMCNT(0));  // no LDS write may outlive the workgroup

  // ---- epilogue -----------------------------------------------------------------------
  __syncthreads();  // every wave is done with the K slabs
  if constexpr (OUT == 2) {
    // bf16 output: the dequant (acc * sa[row]) * sb[col] and the rounding to bf16 happen in
    // the accumulator layout (lane (fr, fh) of tile (i, j) holds output row j * 32 + fr and
    // columns i * 32 + g * 8 + fh * 4 + [0, 4), g = 0..3); the packed bf16 are staged in LDS
    // 32 rows at a time (pitch 264 bytes: the 8-byte writes of 32 consecutive rows cover all
    // 64 banks) and read back row-contiguous, 16 bytes per lane, 16 lanes per 128-column row.
    constexpr int BPITCH = 132;  // row pitch in bf16 elements (264 bytes)
    uint16_t* btile = reinterpret_cast<uint16_t*>(smem) + wave * (32 * BPITCH);
    float4 sbq[4][4];  // sb of the lane's columns, per (i, g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        sbq[i][gq] = *reinterpret_cast<const float4*>(s_sb + wn * 128 + i * 32 + gq * 8 + fh * 4);
    const int rrow = lane >> 4, rcol = (lane & 15) * 8;  // read-back position
    const int64_t col0 = n0 + wn * 128 + rcol;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sar = s_sa[wm * 128 + j * 32 + fr];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (KIND == 0) a[e] = (float)acc[i][j][gq * 4 + e];
            else a[e] = acc[i][j][gq * 4 + e];
          }
          const float4 sbv = sbq[i][gq];
          uint2 w;
          w.x = pack_bf16x2((a[0] * sar) * sbv.x, (a[1] * sar) * sbv.y);
          w.y = pack_bf16x2((a[2] * sar) * sbv.z, (a[3] * sar) * sbv.w);
          *reinterpret_cast<uint2*>(btile + fr * BPITCH + i * 32 + gq * 8 + fh * 4) = w;
        }
      // the wave reads back only what it wrote: program order plus the LDS wait suffice
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = t * 4 + rrow;
        const int64_t row = m0 + wm * 128 + j * 32 + r;
        const uint4 w = *reinterpret_cast<const uint4*>(btile + r * BPITCH + rcol);
        if (row >= g.m || col0 >= g.n) continue;
        uint16_t* dst = reinterpret_cast<uint16_t*>(g.c) + row * g.ldc + col0;
        if (col0 + 7 < g.n) {
          *reinterpret_cast<uint4*>(dst) = w;
        } else {
          const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
          for (int e = 0; e < 8 && col0 + e < g.n; ++e)
            dst[e] = (uint16_t)(wv[e >> 1] >> ((e & 1) * 16));
        }
      }
    }
    return;
  }
  // int32 / fp32 output: each wave stages its raw accumulators in LDS, 32 output rows at a
  // time (row pitch 132 words: the 16-byte writes of 16 consecutive rows fall in 16 different
  // bank groups), and reads them back row-contiguous: 32 lanes cover one 128-column row, so
  // stores are 512-byte runs.  The dequant (acc * sa[row]) * sb[col] is applied after the
  // read-back, where each lane owns 4 fixed columns.
  constexpr int PITCH = 132;
  uint32_t* stile = reinterpret_cast<uint32_t*>(smem) + wave * (32 * PITCH);
  const int ecol = (lane & 31) * 4;  // 4 consecutive columns of this lane after read-back
  const int64_t col0 = n0 + wn * 128 + ecol;
  float4 sbv = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (OUT != 0) sbv = *reinterpret_cast<const float4*>(s_sb + wn * 128 + ecol);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // lane (fr, fh) holds row fr, columns i * 32 + gq * 8 + fh * 4 + [0, 4) of this chunk
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint4 w;
        if constexpr (KIND == 0) {  // raw int32; converted after the read-back
          w = make_uint4(acc[i][j][gq * 4 + 0], acc[i][j][gq * 4 + 1], acc[i][j][gq * 4 + 2],
                         acc[i][j][gq * 4 + 3]);
        } else {
          w = make_uint4(__float_as_uint(acc[i][j][gq * 4 + 0]), __float_as_uint(acc[i][j][gq * 4 + 1]),
                         __float_as_uint(acc[i][j][gq * 4 + 2]), __float_as_uint(acc[i][j][gq * 4 + 3]));
        }
        *reinterpret_cast<uint4*>(stile + fr * PITCH + i * 32 + gq * 8 + fh * 4) = w;
      }
    // the wave reads back only what it wrote: program order plus the LDS wait suffice
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int r = t * 2 + (lane >> 5);
      const int64_t row = m0 + wm * 128 + j * 32 + r;
      const uint4 w = *reinterpret_cast<const uint4*>(stile + r * PITCH + ecol);
      if (row >= g.m || col0 >= g.n) continue;
      if constexpr (OUT == 0) {
        const int iv[4] = {(int)w.x, (int)w.y, (int)w.z, (int)w.w};
        store4<0>(g.c, g.ldc, row, col0, g.n, nullptr, iv);
      } else {
        const float sar = s_sa[wm * 128 + j * 32 + r];
        float a[4];
        if constexpr (KIND == 0) {
          a[0] = (float)(int)w.x; a[1] = (float)(int)w.y; a[2] = (float)(int)w.z; a[3] = (float)(int)w.w;
        } else {
          a[0] = __uint_as_float(w.x); a[1] = __uint_as_float(w.y);
          a[2] = __uint_as_float(w.z); a[3] = __uint_as_float(w.w);
        }
        float v[4];
        v[0] = (a[0] * sar) * sbv.x;
        v[1] = (a[1] * sar) * sbv.y;
        v[2] = (a[2] * sar) * sbv.z;
        v[3] = (a[3] * sar) * sbv.w;
        store4<OUT>(g.c, g.ldc, row, col0, g.n, v, nullptr);
      }
    }
  }
}

template <int KIND, int AF, int BF, int OUT, bool MASK, int BK>
static hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_kernel<KIND, AF, BF, OUT, MASK, BK>),
        hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<KIND, AF, BF, OUT, MASK, BK>), dim3((unsigned)tiles), dim3(256),
                     LDS_BYTES, st, g);
  return hipGetLastError();
}

#ifndef HALO_GEMM_BK
#define HALO_GEMM_BK 128
#endif

template <int KIND, int AF, int BF, int OUT>
static hipError_t launch_t(const GemmArgs& g, hipStream_t st) {
  constexpr int BK = HALO_GEMM_BK;
  constexpr int KS = BK / (KIND == 0 ? 32 : 64);
  const int64_t nk = (g.k + BK - 1) / BK;
  const bool mask = (g.k % BK) != 0 || (KS == 1 && (nk & 1));
  return mask ? launch_cfg<KIND, AF, BF, OUT, true, BK>(g, st)
              : launch_cfg<KIND, AF, BF, OUT, false, BK>(g, st);
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
