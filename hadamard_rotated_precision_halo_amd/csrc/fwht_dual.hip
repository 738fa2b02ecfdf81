// fwht_dual.hip -- both rotation passes of one matrix from a single read of it (gfx950).
//
// What is computed is exactly what the rows pass and the columns pass compute
// ("QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术" s2.1-s2.2, s3.1: blockwise
// natural-order butterflies, one absmax scale per vector): the codes of every row along the
// columns and of every column along the rows.  A layer backward needs a gradient dY both
// ways (its rows for dX = dY W, its columns for dW = dY^T X, "HALO: Hadamard-Assisted
// Lower-Precision Optimization for LLMs", abstract: rotations in the backward pass too), and
// the two passes otherwise read dY twice.
//
// Tiles.  A workgroup of 16 waves owns a 256 x 256 tile (128 KB of bf16): whole blocks along
// both axes for every block of up to 256.  Its columns part loads the tile into LDS with the
// columns kernel's transposing loader, rotates each column segment in the wave-slice layout,
// and exchanges partial column maxima with the other tiles of its tile column; its rows part
// then reads the tile's rows again, from the caches the first read left them in (the whole
// matrix is at most 256 tiles, 32 MiB, and is read by all tiles at once), rotates each
// 256-element row segment, and exchanges partial row maxima with the tiles of its tile row.
// HBM sees one read of the input and one write of each code matrix.
//
// Exchanges.  The same protocol as the columns kernel's (fwht_wave.h, cols_task): device-scope
// returning atomic max of the partial maxima, an arrival count per tile column (tile row), a
// bounded wait.  A task that reaches the bound marks its strip (the top bit of the count),
// counts itself in the late word and skips that part's stores, but goes on with its other
// part, so every task publishes both its partial maxima.  The repair launch that follows
// stores every part of a marked strip from the then complete maxima: the codes never depend
// on what else runs on the device.  Every tile of a launch depends on the others (through its
// row and its column), so the launch is used only when all tiles fit on the device at once.
#include "fwht_wave.h"

namespace halo {

namespace {

constexpr int kTile = 256;
constexpr uint32_t kLateMark = 0x80000000u;

struct DualProb {
  FqArgs ar;           // rows pass: vectors = rows, length = cols
  ColsProb pc;         // columns pass (pc.a: vectors = cols, length = rows) as the columns
                       // loader takes it: 256 x 256 tiles, its signs left out of the load
  const uint32_t* col_signs;  // the columns pass's signs (applied after the LDS round trip)
  uint32_t* rowmax;    // [rows] partial row maxima (float bits), zero at launch
  uint32_t* colmax;    // [cols]
  uint32_t* arrive_r;  // [tile rows] arrival counts
  uint32_t* arrive_c;  // [tile columns]
  uint32_t* late;      // tasks that stopped waiting (either part)
  int64_t tiles_r, tiles_c;
  uint32_t spins;
};

// One exchange of partial maxima: writer lanes max-reduce `mx` into maxima[idx], the task
// counts itself into *arrive and waits (bounded) for all P tasks of the strip.  Returns
// whether the task stopped waiting (workgroup-uniform).
__device__ __forceinline__ bool strip_exchange(uint32_t* maxima, int64_t idx, bool writer,
                                               float mx, uint32_t* arrive, uint32_t* late,
                                               uint32_t P, uint32_t spins) {
  __shared__ uint32_t s_late;
  uint32_t seen = 0;
  if (writer)
    seen = __hip_atomic_fetch_max(&maxima[idx], __float_as_uint(mx), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  // every wave waits for the values its atomics return before the barrier, so the arrival
  // counted below covers them (see cols_task)
  asm volatile("s_waitcnt vmcnt(0)" ::"v"(seen) : "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t c = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    for (uint32_t it = 0; (c & ~kLateMark) < P && !(c & kLateMark) && it < spins; ++it) {
      __builtin_amdgcn_s_sleep(2);
      c = __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const bool lt = (c & kLateMark) || (c & ~kLateMark) < P;
    if (lt) {
      if (!(c & kLateMark))
        __hip_atomic_fetch_or(arrive, kLateMark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(late, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_late = lt ? 1u : 0u;
  }
  __syncthreads();
  return s_late != 0;
}

// The final maxima of the tile's 256 vectors [base, base + 256), read once per vector with
// atomic loads and shared through LDS.
__device__ __forceinline__ void read_maxima(const uint32_t* maxima, int64_t base, float* s_max) {
  if (threadIdx.x < kTile)
    s_max[threadIdx.x] = __uint_as_float(
        __hip_atomic_load(&maxima[base + threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  __syncthreads();
}

// One 256 x 256 tile.  REPAIR: the follow-up launch, which redoes only the parts whose strip
// is marked, from the complete maxima.
template <int B, int QT, bool SR, bool REPAIR>
__device__ __forceinline__ void dual_task(const DualProb& dp, int64_t ltask, uint4* lds) {
  using S = Slice<B>;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t tri = ltask / dp.tiles_c, tci = ltask - tri * dp.tiles_c;
  const int64_t r0 = tri * kTile, c0 = tci * kTile;
  __shared__ float s_max[kTile];
  bool do_cols = true, do_rows = true;
  if constexpr (REPAIR) {
    __shared__ uint32_t s_marks;
    if (t == 0) {
      const uint32_t mc = __hip_atomic_load(&dp.arrive_c[tci], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t mr = __hip_atomic_load(&dp.arrive_r[tri], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_marks = ((mc & kLateMark) ? 1u : 0u) | ((mr & kLateMark) ? 2u : 0u);
    }
    __syncthreads();
    do_cols = (s_marks & 1u) != 0;
    do_rows = (s_marks & 2u) != 0;
    __syncthreads();  // s_marks is read before any task of this workgroup rewrites it
    if (!do_cols && !do_rows) return;
  }
  constexpr int row_lanes_log2 = 2;  // 256-element segments: 4 lanes each
  const bool writer = (lane & 3) == 0;
  float v[64];

  // ---- columns part: the tile transposed into LDS, column segments of 256 rows -----------
  if (do_cols) {
    const FqArgs& ac = dp.pc.a;
    cols_load<B>(dp.pc, c0, (int)tri, t, lds);
    __syncthreads();
    const int seg = S::off(lane, 0) / kTile;           // column segment of the lane in its wave
    const int64_t pos0 = r0 - (int64_t)seg * kTile;     // + off(lane, j): row index
#pragma unroll
    for (int j = 0; j < 8; ++j) unpack_bf16x8(lds[lds_slot<B>(w, lane, j)], &v[j * 8]);
    if (dp.col_signs) {
#pragma unroll
      for (int j = 0; j < 8; ++j) apply_signs8(&v[j * 8], dp.col_signs, pos0 + S::off(lane, j));
    }
    const float sgn = rotate64<B>(v, lane);
    const int64_t col = c0 + w * (4096 / kTile) + seg;
    float mx = lane_max(absmax64(v), row_lanes_log2);
    bool late = false;
    if constexpr (!REPAIR)
      late = strip_exchange(dp.colmax, col, writer, mx, &dp.arrive_c[tci], dp.late,
                            (uint32_t)dp.tiles_r, dp.spins);
    if (!late) {
      read_maxima(dp.colmax, c0, s_max);
      mx = s_max[w * (4096 / kTile) + seg];
      if (tri == 0 && writer) ac.scale[col] = stored_scale<QT>(ac, mx);
      const float mul = quant_mul_v<QT>(ac, mx, v) * sgn;
      store_slice<B, QT, SR>(ac, v, mul, col * ac.ldq + pos0, lane, col, pos0);
    }
    __syncthreads();  // s_max is reused by the rows part
  }

  // ---- rows part: the tile's rows read again (cache-resident), 256-element segments -------
  if (do_rows) {
    const int rseg = S::off(lane, 0) / kTile;           // row segment of the lane in its wave
    const int64_t row = r0 + w * (4096 / kTile) + rseg;
    const int64_t pos0 = c0 - (int64_t)rseg * kTile;    // + off(lane, j): column index
    const uint16_t* xr = reinterpret_cast<const uint16_t*>(dp.ar.x) + row * dp.ar.ldx;
    load_slice<uint16_t, B>(dp.ar, xr, pos0, lane, true, v);
    const float sgn = rotate64<B>(v, lane);
    float mx = lane_max(absmax64(v), row_lanes_log2);
    bool late = false;
    if constexpr (!REPAIR)
      late = strip_exchange(dp.rowmax, row, writer, mx, &dp.arrive_r[tri], dp.late,
                            (uint32_t)dp.tiles_c, dp.spins);
    if (!late) {
      read_maxima(dp.rowmax, r0, s_max);
      mx = s_max[w * (4096 / kTile) + rseg];
      if (tci == 0 && writer) dp.ar.scale[row] = stored_scale<QT>(dp.ar, mx);
      const float mul = quant_mul_v<QT>(dp.ar, mx, v) * sgn;
      store_slice<B, QT, SR>(dp.ar, v, mul, row * dp.ar.ldq + pos0, lane, row, pos0);
    }
  }
}

template <int B, int QT, bool SR, bool REPAIR>
__global__ __launch_bounds__(1024) void fq_dual_kernel(DualProb dp) {
  extern __shared__ __attribute__((aligned(16))) uint4 lds[];
  if constexpr (REPAIR) {
    if (!any_late(dp.late, nullptr, nullptr)) return;
  }
  const int64_t tiles = dp.tiles_r * dp.tiles_c;
  for (int64_t task = blockIdx.x; task < tiles; task += gridDim.x) {
    dual_task<B, QT, SR, REPAIR>(dp, task, lds);
    __syncthreads();  // the next task overwrites the LDS tile and s_max
  }
}

// Scratch: the late count (padded to 256 bytes), the arrival counts of the tile columns and
// of the tile rows (each padded to 256 bytes), the column maxima, the row maxima.
size_t dual_scratch_bytes(int64_t rows, int64_t cols) {
  const size_t ac = ((size_t)(cols / kTile) * 4 + 255) & ~(size_t)255;
  const size_t ar = ((size_t)(rows / kTile) * 4 + 255) & ~(size_t)255;
  return 256 + ac + ar + (size_t)cols * 4 + (size_t)rows * 4;
}

template <int B, int QT, bool SR>
hipError_t launch_dual_t(const FqArgs& ar, const FqArgs& ac, void* ws, int prezeroed,
                         hipStream_t st) {
  hipError_t e = allow_dynamic_lds<&fq_dual_kernel<B, QT, SR, false>>(kColsLdsBytes);
  if (e != hipSuccess) return e;
  e = allow_dynamic_lds<&fq_dual_kernel<B, QT, SR, true>>(kColsLdsBytes);
  if (e != hipSuccess) return e;
  const int64_t rows = ar.nvec, cols = ac.nvec;
  DualProb dp{};
  dp.ar = ar;
  dp.pc.a = ac;
  dp.pc.a.signs = nullptr;
  dp.pc.R = kTile;
  dp.pc.C = kTile;
  dp.col_signs = ac.signs;
  dp.tiles_r = rows / kTile;
  dp.tiles_c = cols / kTile;
  dp.pc.P = (int)dp.tiles_r;
  char* base = reinterpret_cast<char*>(ws);
  const size_t acb = ((size_t)dp.tiles_c * 4 + 255) & ~(size_t)255;
  const size_t arb = ((size_t)dp.tiles_r * 4 + 255) & ~(size_t)255;
  dp.late = reinterpret_cast<uint32_t*>(base);
  dp.arrive_c = reinterpret_cast<uint32_t*>(base + 256);
  dp.arrive_r = reinterpret_cast<uint32_t*>(base + 256 + acb);
  dp.colmax = reinterpret_cast<uint32_t*>(base + 256 + acb + arb);
  dp.rowmax = dp.colmax + cols;
  // polls of a waiting task (each an atomic load and s_sleep 2): the caller's count (of the
  // columns part's options), else 2^20
  dp.spins = ac.polls != 0 ? ac.polls : (1u << 20);
  const int64_t tiles = dp.tiles_r * dp.tiles_c;
  if (tiles == 0) return hipSuccess;
  if (!prezeroed) {
    e = launch_fill_zero(reinterpret_cast<float*>(ws), (int64_t)(dual_scratch_bytes(rows, cols) / 4), st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((fq_dual_kernel<B, QT, SR, false>), dim3((unsigned)tiles), dim3(1024),
                     kColsLdsBytes, st, dp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the repair launch: its workgroups (at most one per compute unit) return at once unless a
  // task stopped waiting
  const int cap = cols2_capacity(reinterpret_cast<const void*>(&fq_dual_kernel<B, QT, SR, false>));
  const int64_t rgrid = tiles < cap ? tiles : (cap > 0 ? cap : 1);
  hipLaunchKernelGGL((fq_dual_kernel<B, QT, SR, true>), dim3((unsigned)rgrid), dim3(1024),
                     kColsLdsBytes, st, dp);
  return hipGetLastError();
}

template <int QT, bool SR>
hipError_t dual_block(const FqArgs& ar, const FqArgs& ac, void* ws, int prezeroed,
                      hipStream_t st) {
#define HALO_DUAL_CASE(BB) \
  case BB: return launch_dual_t<BB, QT, SR>(ar, ac, ws, prezeroed, st);
  switch (ar.block) {
    HALO_DUAL_CASE(1) HALO_DUAL_CASE(2) HALO_DUAL_CASE(4) HALO_DUAL_CASE(8) HALO_DUAL_CASE(16)
    HALO_DUAL_CASE(32) HALO_DUAL_CASE(64) HALO_DUAL_CASE(128) HALO_DUAL_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef HALO_DUAL_CASE
}

}  // namespace

size_t fq_dual_ws_bytes(int64_t rows, int64_t cols, int block, int in_bf16) {
  if (!in_bf16 || rows <= 0 || cols <= 0 || block < 1 || block > kTile) return 0;
  if (rows % kTile != 0 || cols % kTile != 0) return 0;
  return dual_scratch_bytes(rows, cols);
}

bool fq_dual_supported(int64_t rows, int64_t cols, int block, int in_bf16, int qt, bool sr_rows,
                       bool sr_cols, size_t ws_bytes) {
  const size_t need = fq_dual_ws_bytes(rows, cols, block, in_bf16);
  if (need == 0 || ws_bytes < need) return false;
  // stochastic rounding takes the two passes (its Philox draws would push this kernel's
  // registers, already at the 128 of a 16-wave workgroup, into heavy spills)
  if (sr_rows || sr_cols || qt < 0 || qt > 3) return false;
  // every tile waits on the others of its row and of its column: all must be resident at once
  const int cap = cols2_capacity(reinterpret_cast<const void*>(&fq_dual_kernel<256, 0, false, false>));
  return (rows / kTile) * (cols / kTile) <= cap;
}

hipError_t launch_fq_dual(const FqArgs& ar, const FqArgs& ac, void* ws, int qt, int prezeroed,
                          hipStream_t st) {
  if (ar.sr || ac.sr) return hipErrorInvalidValue;
  switch (qt) {
    case 0: return dual_block<0, false>(ar, ac, ws, prezeroed, st);
    case 1: return dual_block<1, false>(ar, ac, ws, prezeroed, st);
    case 2: return dual_block<2, false>(ar, ac, ws, prezeroed, st);
    case 3: return dual_block<3, false>(ar, ac, ws, prezeroed, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace halo
