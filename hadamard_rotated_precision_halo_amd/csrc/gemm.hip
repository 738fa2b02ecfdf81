// gemm.hip -- 8-bit MFMA GEMM with a fused per-row x per-column dequant epilogue (gfx950).
//
// What is computed ("HALO: Hadamard-Assisted Lower-Precision Optimization for LLMs",
// abstract: every large product of the forward and backward pass in low precision; key
// design 2: INT8 or FP8):  acc[i, j] = sum_t a[i, t] b[j, t] with INT8 codes accumulated in
// int32 (v_mfma_i32_32x32x32_i8) or FP8 codes on the CDNA4 v_mfma_*_32x32x64_f8f6f4 with a
// per-operand format select, then c[i, j] = (acc * sa[i]) * sb[j] in fp32, rounded to bf16 or
// kept in fp32 (or the raw int32 accumulators).
//
// Tiling.  A 512-thread workgroup (8 wave64s, 2 x 4) owns a 256 x 256 output tile; each wave
// owns 128 x 64 = 4 x 2 MFMA tiles of 32 x 32 with the accumulators resident in AGPRs.  K is
// consumed in slabs of BK bytes: a slab (256 rows of each operand) is staged in LDS with
// direct-to-LDS loads (buffer_load_dwordx4 ... lds: no VGPR staging, no ds_write) into a ring of
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
// halving the staged bytes); the scales sa, sb were loaded into LDS at kernel start.  The
// output is written once and never read back here, so its full 16-byte stores are
// non-temporal: they stream past the caches instead of evicting the operand slabs that the
// other workgroups on the XCD still read.
// Workgroups are numbered so that each of the 8 XCDs (workgroup i runs on XCD i % 8) gets a
// contiguous run of tiles, rastered in groups of 4 tile rows, for L2 reuse of both operands.
#include "halo_device.h"
#include "halo_kernels.h"



namespace halo {

constexpr int BM = 256, BN = 256;
constexpr int GEMM_WN = 4;                      // waves across a tile's columns (x 2 rows)
constexpr int GEMM_BK = 128;                    // K bytes per slab: a 2-slab ring
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

// One 16-byte direct-to-LDS load per lane (buffer_load_dwordx4 ... lds): the lane's 16 bytes
// at byte offset off of the resource land at lds + 16 * lane.  The buffer form rather than the
// global one (global_load_lds_dwordx4): the compiler counts a global-to-LDS load as both a
// memory load and an LDS access, and then makes every later LDS read wait for all outstanding
// LDS reads (lgkmcnt(0)); the buffer form counts only as a memory load, so the fragment reads
// keep exact lgkmcnt waits and an MFMA starts as soon as its own fragments have landed.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, 0, 0, 0);
}

// Raw buffer resource over [p, p + 4 GiB): no range check below that (the operands' byte spans
// are validated to stay under 4 GiB); dword 3 selects 32-bit data, as gfx9 raw loads need.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, -1, 0x00020000);
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
      const v4i w = {iv[0], iv[1], iv[2], iv[3]};
      __builtin_nontemporal_store(w, reinterpret_cast<v4i*>(reinterpret_cast<int*>(c) + row * ldc + col));
    } else if constexpr (OUT == 1) {
      const v4i w = {(int)__float_as_uint(v[0]), (int)__float_as_uint(v[1]),
                     (int)__float_as_uint(v[2]), (int)__float_as_uint(v[3])};
      __builtin_nontemporal_store(w, reinterpret_cast<v4i*>(reinterpret_cast<float*>(c) + row * ldc + col));
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
// WN: waves along N (2: four waves of 128 x 128, one per SIMD; 4: eight waves of 128 x 64, two
// per SIMD, so one wave's stalls at the barrier or on loads are covered by the other's MFMAs).
// One launch runs up to two products of the same kind and output type (gp.g[1] when
// blockIdx.x >= gp.split): the second product's tiles fill the compute units as the first's
// finish, so its operand loads overlap the first's output stores.
struct GemmPair {
  GemmArgs g[2];
  int64_t split;  // workgroups of the first product
};

template <int KIND, int AF, int BF, int OUT, bool MASK, int BK, int WN>
__global__ __launch_bounds__(128 * WN, 1) void gemm_kernel(GemmPair gp) {
  using SL = Slab<BK>;
  constexpr int NW = 2 * WN, NT = 64 * NW;         // waves, threads
  constexpr int TN = BN / WN;                      // output columns per wave
  constexpr int FA = 4, FB = TN / 32;              // 32-row fragments of a and b per wave
  constexpr int NSTAGE = SL::NSTAGE, RPI = SL::RPI;
  constexpr int INST = SL::OPER / (NT * 16);       // loads per thread per operand per slab
  constexpr int WROWS = INST * RPI;                // slab rows one wave loads per operand
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  float* s_sa = reinterpret_cast<float*>(smem + RING_BYTES);
  float* s_sb = s_sa + 256;

  // ---- product and tile of this workgroup ---------------------------------------------
  const bool second = (int64_t)blockIdx.x >= gp.split;
  const GemmArgs g = second ? gp.g[1] : gp.g[0];
  const int tiles_m = (int)((g.m + BM - 1) / BM), tiles_n = (int)((g.n + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  const int bid = (int)(blockIdx.x - (second ? gp.split : 0));
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
  const int wm = wave / WN, wn = wave % WN;

  // scales of this tile's rows and columns (written to LDS once the prologue loads landed)
  float my_sa = 0.f, my_sb = 0.f;
  if constexpr (OUT != 0) {
    if (tid < 256) {
      my_sa = g.sa[min(m0 + tid, g.m - 1)];
      my_sb = g.sb[min(n0 + tid, g.n - 1)];
    }
  }

  // ---- direct-to-LDS assignment -----------------------------------------------------
  // Wave w's instruction i fills LDS bytes [(INST w + i) KB, +1 KB) of an operand's slab =
  // rows WROWS w + RPI i + [0, RPI); lane l lands in physical chunk l % CHUNKS of row
  // WROWS w + RPI i + l / CHUNKS and loads that row's logical chunk (l % CHUNKS) ^ swz(row).
  const __amdgpu_buffer_rsrc_t ra = raw_rsrc(g.a), rb = raw_rsrc(g.b);
  uint32_t aoff[INST], boff[INST];  // byte offsets of the lane's rows (operands are < 4 GB)
  uint32_t cbo[INST];               // byte offset of the lane's chunk within a slab row
#pragma unroll
  for (int i = 0; i < INST; ++i) {
    const int r = wave * WROWS + i * RPI + lane / SL::CHUNKS;
    cbo[i] = (uint32_t)(((lane % SL::CHUNKS) ^ SL::swz(r)) << 4);
    aoff[i] = (uint32_t)(min(m0 + r, g.m - 1) * g.lda);  // clamped rows feed unused outputs
    boff[i] = (uint32_t)(min(n0 + r, g.n - 1) * g.ldb);
  }
  const int nk = (int)((g.k + BK - 1) / BK);
  constexpr int KS = BK / (KIND == 0 ? 32 : 64);  // MFMA K sub-steps per slab
  constexpr int UNROLL = KS == 1 ? 2 : 1;          // keeps the fragment buffer index constant
  const int nkr = (nk + UNROLL - 1) / UNROLL * UNROLL;
  const uint32_t klast = (uint32_t)g.k - 16;       // last in-bounds chunk of a row

  // Loads [q0, q1) of slab kt into ring slot kt % NSTAGE (load q: operand q % 2, row group
  // q / 2).  A whole slab is always 2 * INST direct-to-LDS loads per thread, so the vmcnt
  // arithmetic is uniform.  Slabs past the end reload the last slab (never read) and chunks
  // past k read the row's last chunk instead; their fragments are masked to zero.
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
      if (q & 1) dma16(rb, boff[i] + kc, (lds_void*)(sb + (wave * INST + i) * 1024));
      else dma16(ra, aoff[i] + kc, (lds_void*)(sa + (wave * INST + i) * 1024));
    }
  };
  auto stage = [&](int kt) __attribute__((always_inline)) { stage_part(kt, 0, 2 * INST); };

  using Acc = typename std::conditional<KIND == 0, v16i, v16f>::type;
  using Frag = typename std::conditional<KIND == 0, v4i, v8i>::type;
  Acc acc[FB][FA];
#pragma unroll
  for (int i = 0; i < FB; ++i)
#pragma unroll
    for (int j = 0; j < FA; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  const int fr = lane & 31, fh = lane >> 5;  // fragment row and K half
  Frag fa[2][FA], fb[2][FB];

  // ---- main loop -------------------------------------------------------------------
  // Sub-steps run in one flat sequence (slab kt, sub-step ks).  Issue order is explicit: MFMA
  // t of a sub-step is followed by its share of the next sub-step's fragment reads and, in the
  // slab's last sub-step, of the next slab loads; a scheduling barrier after each group keeps
  // the order, so reads and loads are spread evenly between the MFMAs (a burst of loads, each
  // needing its own M0, stalls the MFMA issue).  Before the last sub-step of slab kt the wave
  // waits for its own loads of slab kt + 1, the barrier makes every wave's loads visible, and
  // slab kt + NSTAGE is issued into slab kt's slot, which no wave reads any more.  The loop
  // body has no branches, so the accumulators stay in AGPRs.
  constexpr int RPF = KIND == 0 ? 1 : 2;             // ds_read_b128 per fragment
  constexpr int FRAG_READS = (FA + FB) * RPF;        // per sub-step
  constexpr int NMF = FA * FB;                       // MFMAs per sub-step
  // read q of a sub-step: fragment q / RPF (b fragments first), 16-byte half q % RPF
  auto read_one = [&](int kt, int ks, int q, Frag* da, Frag* db) __attribute__((always_inline)) {
    const char* sa = smem + (kt % NSTAGE) * SL::STAGE;
    const char* sb = sa + SL::OPER;
    const int c0 = KIND == 0 ? ks * 2 + fh : ks * 4 + fh * 2;  // first 16-byte chunk
    const int f = q / RPF, h = q % RPF;
    int keep = -1;
    if constexpr (MASK) keep = (kt * BK + (c0 + h) * 16) < g.k ? -1 : 0;
    const bool isb = f < FB;
    const int t = isb ? f : f - FB;
    const char* base = isb ? sb : sa;
    const int row = isb ? wn * TN + t * 32 + fr : wm * 128 + t * 32 + fr;
    const v4i v = *reinterpret_cast<const v4i*>(base + SL::off(row, c0 + h)) & keep;
    Frag* dst = isb ? &db[t] : &da[t];
    if constexpr (KIND == 0) {
      *dst = v;
    } else {
      if (h) dst->hi = v;
      else dst->lo = v;
    }
  };
  // front: every fragment read right after the sub-step's first MFMA instead of one or two
  // per MFMA.  For the sub-step before the slab barrier: the barrier must wait for these
  // reads (the slab's ring slot is refilled after it), so issuing them first gives them the
  // whole sub-step to land (same-box A/Bs: 0.2-0.9 % faster).
  auto ordered_step = [&](const Frag* da, const Frag* db, int rkt, int rks, Frag* nda, Frag* ndb,
                          int lkt, bool loads, bool front) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      const int i = t / FA, j = t % FA;
      if constexpr (KIND == 0)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(db[i], da[j], acc[i][j], 0, 0, 0);
      else  // first operand = b tile (format BF), second = a tile (format AF); scales 2^0
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(db[i], da[j], acc[i][j], BF,
                                                                    AF, 0, 127, 0, 127);
      const int r0 = front ? (t == 0 ? 0 : FRAG_READS) : t * FRAG_READS / NMF;
      const int r1 = front ? FRAG_READS : (t + 1) * FRAG_READS / NMF;
#pragma unroll
      for (int q = r0; q < r1; ++q)
        read_one(rkt, rks, q, nda, ndb);
      if (loads) stage_part(lkt, t * 2 * INST / NMF, (t + 1) * 2 * INST / NMF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto do_slab = [&](int kt, auto P) __attribute__((always_inline)) {
    constexpr int P0 = decltype(P)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = (P0 + ks) & 1;
      if (ks + 1 < KS) {
        ordered_step(fa[cur], fb[cur], kt, ks + 1, fa[cur ^ 1], fb[cur ^ 1], 0, false,
                     ks + 2 == KS);
      } else {
        __builtin_amdgcn_s_waitcnt(HALO_VMCNT(2 * INST * (NSTAGE - 2)));  // slab kt + 1 landed
        __syncthreads();
        ordered_step(fa[cur], fb[cur], kt + 1, 0, fa[cur ^ 1], fb[cur ^ 1], kt + NSTAGE, true,
                     false);
      }
    }
  };

#pragma unroll
  for (int t = 0; t < NSTAGE; ++t) stage(t);
  __builtin_amdgcn_s_waitcnt(HALO_VMCNT(2 * INST * (NSTAGE - 1)));  // slab 0 and the scales
  if constexpr (OUT != 0) {
    if (tid < 256) {
      s_sa[tid] = my_sa;
      s_sb[tid] = my_sb;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < FRAG_READS; ++q) read_one(0, 0, q, fa[0], fb[0]);
  for (int kt = 0; kt < nkr; kt += UNROLL) {
    do_slab(kt, std::integral_constant<int, 0>{});
    if constexpr (UNROLL == 2) do_slab(kt + 1, std::integral_constant<int, KS & 1>{});
  }
  __builtin_amdgcn_s_waitcnt(HALO_VMCNT(0));  // no LDS write may outlive the workgroup

  // ---- epilogue -----------------------------------------------------------------------
  // Lane (fr, fh) of accumulator tile (i, j) holds output row wm * 128 + j * 32 + fr and
  // columns wn * TN + i * 32 + g * 8 + fh * 4 + [0, 4), g = 0..3.  Each wave stages its
  // results in LDS 32 rows at a time and reads them back row-contiguous, 16 bytes per lane.
  __syncthreads();  // every wave is done with the K slabs
  if constexpr (OUT == 2) {
    // bf16: dequant (acc * sa[row]) * sb[col] and rounding in the accumulator layout; the
    // staged row pitch (TN + 4 elements) makes the 8-byte writes of 32 consecutive rows cover
    // all 64 banks.
    constexpr int BPITCH = TN + 4;
    constexpr int LPR = TN / 8, RPIT = 64 / LPR;    // lanes per row, rows per read-back
    uint16_t* btile = reinterpret_cast<uint16_t*>(smem) + wave * (32 * BPITCH);
    float4 sbq[FB][4];
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        sbq[i][gq] = *reinterpret_cast<const float4*>(s_sb + wn * TN + i * 32 + gq * 8 + fh * 4);
    const int rrow = lane / LPR, rcol = (lane % LPR) * 8;
    const int64_t col0 = n0 + wn * TN + rcol;
#pragma unroll
    for (int j = 0; j < FA; ++j) {
      const float sar = s_sa[wm * 128 + j * 32 + fr];
#pragma unroll
      for (int i = 0; i < FB; ++i)
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
      for (int t = 0; t < 32 / RPIT; ++t) {
        const int r = t * RPIT + rrow;
        const int64_t row = m0 + wm * 128 + j * 32 + r;
        const uint4 w = *reinterpret_cast<const uint4*>(btile + r * BPITCH + rcol);
        if (row >= g.m || col0 >= g.n) continue;
        uint16_t* dst = reinterpret_cast<uint16_t*>(g.c) + row * g.ldc + col0;
        if (col0 + 7 < g.n) {
          const v4i wv = {(int)w.x, (int)w.y, (int)w.z, (int)w.w};
          __builtin_nontemporal_store(wv, reinterpret_cast<v4i*>(dst));
        } else {
          const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
          for (int e = 0; e < 8 && col0 + e < g.n; ++e)
            dst[e] = (uint16_t)(wv[e >> 1] >> ((e & 1) * 16));
        }
      }
    }
    return;
  }
  // int32 / fp32: the raw accumulators are staged (row pitch TN + 4 words: the 16-byte writes
  // of 16 consecutive rows fall in 16 different bank groups) and read back 4 columns per lane;
  // the dequant is applied after the read-back, where each lane owns 4 fixed columns.
  constexpr int PITCH = TN + 4;
  constexpr int ELR = TN / 4, ERPIT = 64 / ELR;      // lanes per row, rows per read-back
  uint32_t* stile = reinterpret_cast<uint32_t*>(smem) + wave * (32 * PITCH);
  const int ecol = (lane % ELR) * 4;
  const int64_t col0 = n0 + wn * TN + ecol;
  float4 sbv = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (OUT != 0) sbv = *reinterpret_cast<const float4*>(s_sb + wn * TN + ecol);
#pragma unroll
  for (int j = 0; j < FA; ++j) {
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint4 w;
        if constexpr (KIND == 0) {
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
    for (int t = 0; t < 32 / ERPIT; ++t) {
      const int r = t * ERPIT + lane / ELR;
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
static hipError_t launch_cfg(const GemmArgs& g0, const GemmArgs* g1, hipStream_t st) {
  constexpr int WN = GEMM_WN;
  const hipError_t attr_err =
      allow_dynamic_lds<&gemm_kernel<KIND, AF, BF, OUT, MASK, BK, WN>>(LDS_BYTES);
  if (attr_err != hipSuccess) return attr_err;
  GemmPair gp{};
  gp.g[0] = g0;
  gp.g[1] = g1 ? *g1 : g0;
  gp.split = ((g0.m + BM - 1) / BM) * ((g0.n + BN - 1) / BN);
  const int64_t t1 = g1 ? ((g1->m + BM - 1) / BM) * ((g1->n + BN - 1) / BN) : 0;
  if (gp.split == 0) {  // keep the first slot filled: the kernel picks by workgroup index
    gp.g[0] = gp.g[1];
    gp.split = t1;
    if (t1 == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<KIND, AF, BF, OUT, MASK, BK, WN>), dim3((unsigned)t1),
                       dim3(128 * WN), LDS_BYTES, st, gp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_kernel<KIND, AF, BF, OUT, MASK, BK, WN>),
                     dim3((unsigned)(gp.split + t1)), dim3(128 * WN), LDS_BYTES, st, gp);
  return hipGetLastError();
}

template <int KIND, int BK>
static bool needs_mask(const GemmArgs& g) {
  constexpr int KS = BK / (KIND == 0 ? 32 : 64);
  const int64_t nk = (g.k + BK - 1) / BK;
  return (g.k % BK) != 0 || (KS == 1 && (nk & 1));
}

template <int KIND, int AF, int BF, int OUT>
static hipError_t launch_t(const GemmArgs& g, const GemmArgs* g1, hipStream_t st) {
  constexpr int BK = GEMM_BK;
  const bool mask = needs_mask<KIND, BK>(g) || (g1 && needs_mask<KIND, BK>(*g1));
  return mask ? launch_cfg<KIND, AF, BF, OUT, true, BK>(g, g1, st)
              : launch_cfg<KIND, AF, BF, OUT, false, BK>(g, g1, st);
}

hipError_t launch_gemm_pair(const GemmArgs& g_in, const GemmArgs* g1_in, int kind, int afmt,
                            int bfmt, int out, hipStream_t st) {
  // The product with the longer contraction takes the first workgroups: its tiles run longer,
  // and dispatching the longer tasks first leaves a shorter tail when the two products' tiles
  // do not divide evenly over the compute units (each workgroup's outputs are its own, so the
  // order changes no result).
  const bool swap = g1_in && g1_in->k > g_in.k;
  const GemmArgs& g = swap ? *g1_in : g_in;
  const GemmArgs* g1 = swap ? &g_in : g1_in;
  if (kind == 0) {
    switch (out) {
      case 0: return launch_t<0, 0, 0, 0>(g, g1, st);
      case 1: return launch_t<0, 0, 0, 1>(g, g1, st);
      case 2: return launch_t<0, 0, 0, 2>(g, g1, st);
    }
    return hipErrorInvalidValue;
  }
  const int sel = afmt * 2 + bfmt;
#define HALO_FP8_CASE(AFv, BFv)                                       \
  if (sel == AFv * 2 + BFv) {                                         \
    if (out == 1) return launch_t<1, AFv, BFv, 1>(g, g1, st);         \
    if (out == 2) return launch_t<1, AFv, BFv, 2>(g, g1, st);         \
  }
  HALO_FP8_CASE(0, 0)
  HALO_FP8_CASE(0, 1)
  HALO_FP8_CASE(1, 0)
  HALO_FP8_CASE(1, 1)
#undef HALO_FP8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& g, int kind, int afmt, int bfmt, int out, hipStream_t st) {
  return launch_gemm_pair(g, nullptr, kind, afmt, bfmt, out, st);
}

}  // namespace halo
