// fwht_wave.hip -- launch interface of the wave-slice rotation kernels (fwht_wave.h): shape
// support, scratch sizes, and the nearest-even instantiations.  The stochastic-rounding
// instantiations live in fwht_wave_sr.hip, so the two halves compile in parallel.
#include "fwht_wave.h"

namespace halo {

bool fq_rows2_supported(int64_t len, int block) {
  if (len <= 0 || len % 64 != 0 || len > 16 * 4096) return false;
  if (len < 4096 && 4096 % len != 0) return false;
  return block >= 1 && block <= 4096 && len % block == 0;
}

size_t fq_cols2_ws_bytes(int64_t rows, int64_t cols, int block) {
  const int R = cols2_rows_per_task(rows, block);
  if (R == 0) return 0;
  const int64_t P = rows / R;
  if (P <= 1) return 0;
  const int64_t C = 65536 / R;
  const int64_t strips = (cols + C - 1) / C;
  const size_t cnt = ((size_t)strips * 4 + 255) & ~(size_t)255;
  return kColsLateBytes + cnt + (size_t)cols * 4;
}

bool fq_cols2_supported(int64_t rows, int64_t cols, int block, int in_bf16, bool sr,
                        size_t ws_bytes) {
  // fp32 input with stochastic rounding is left to the two-sweep kernel
  if ((!in_bf16 && sr) || rows <= 0 || cols <= 0) return false;
  const int R = cols2_rows_per_task(rows, block);
  if (R == 0) return false;
  if (rows / R == 1) return true;
  // the parts of a strip wait for each other, so all of them must fit on the device at once;
  // longer columns take the two-sweep kernel, which never waits
  const int cap = cols2_capacity(reinterpret_cast<const void*>(&fq_cols2_kernel<256, 0, false>));
  return rows / R <= cap && ws_bytes >= fq_cols2_ws_bytes(rows, cols, block);
}

bool fq_batch_rows_ok(int64_t len) { return len >= 64 && len <= 4096 && 4096 % len == 0; }

hipError_t launch_fq_cols2_pair(const FqArgs& a0, void* ws0, const FqArgs* a1, void* ws1,
                                int in_bf16, int qt, int prezeroed, hipStream_t st) {
  // the two passes of one launch share the rounding mode and the input type
  if (a1 && a1->sr != a0.sr) return hipErrorInvalidValue;
  if (!in_bf16) {
    if (a0.sr) return hipErrorInvalidValue;
    switch (qt) {
      case 0: return cols2_block<0, false, true>(a0, ws0, a1, ws1, prezeroed, st);
      case 1: return cols2_block<1, false, true>(a0, ws0, a1, ws1, prezeroed, st);
      case 2: return cols2_block<2, false, true>(a0, ws0, a1, ws1, prezeroed, st);
      case 3: return cols2_block<3, false, true>(a0, ws0, a1, ws1, prezeroed, st);
    }
    return hipErrorInvalidValue;
  }
  if (a0.sr && qt != 3) return cols2_dispatch_sr(a0, ws0, a1, ws1, qt, prezeroed, st);
  switch (qt) {
    case 0: return cols2_block<0, false>(a0, ws0, a1, ws1, prezeroed, st);
    case 1: return cols2_block<1, false>(a0, ws0, a1, ws1, prezeroed, st);
    case 2: return cols2_block<2, false>(a0, ws0, a1, ws1, prezeroed, st);
    case 3: return cols2_block<3, false>(a0, ws0, a1, ws1, prezeroed, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fq_cols2(const FqArgs& a, int in_bf16, int qt, void* ws, hipStream_t st) {
  return launch_fq_cols2_pair(a, ws, nullptr, nullptr, in_bf16, qt, 0, st);
}

hipError_t launch_fq_batch(const FqArgs* rows, const FqArgs& cw, void* ws_w, const FqArgs& cdy,
                           void* ws_dy, const FqArgs& cx, void* ws_x, int qg, int qw,
                           hipStream_t st) {
  // stochastic rounding applies to the dY passes only
  if (cw.sr || cx.sr || (rows && rows->sr != cdy.sr)) return hipErrorInvalidValue;
  if (cdy.sr) return batch_dispatch_sr(qg, qw, rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  if (qg == 0 && qw == 0) return batch_block<0, 0, false>(cw.block, rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  if (qg == 2 && qw == 1) return batch_block<2, 1, false>(cw.block, rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  if (qg == 1 && qw == 1) return batch_block<1, 1, false>(cw.block, rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  return hipErrorInvalidValue;
}

hipError_t launch_fq_rows2_pair(const FqPair& a, int in_bf16, int qt, hipStream_t st) {
  // the two passes of one launch share the rounding mode
  if (a.has1 && a.p1.sr != a.p0.sr) return hipErrorInvalidValue;
  if (a.p0.sr && qt != 3) {  // stochastic rounding: bf16 input (fp32 takes the older kernel)
    if (!in_bf16) return hipErrorInvalidValue;
    return rows2_dispatch_sr(a, qt, st);
  }
  if (in_bf16) {
    switch (qt) {
      case 0: return rows2_block<uint16_t, 0, false>(a, st);
      case 1: return rows2_block<uint16_t, 1, false>(a, st);
      case 2: return rows2_block<uint16_t, 2, false>(a, st);
      case 3: return rows2_block<uint16_t, 3, false>(a, st);
    }
  } else {
    switch (qt) {
      case 0: return rows2_block<float, 0, false>(a, st);
      case 1: return rows2_block<float, 1, false>(a, st);
      case 2: return rows2_block<float, 2, false>(a, st);
      case 3: return rows2_block<float, 3, false>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fq_rows2(const FqArgs& a, int in_bf16, int qt, hipStream_t st) {
  FqPair pp{};
  pp.p0 = a;
  return launch_fq_rows2_pair(pp, in_bf16, qt, st);
}

}  // namespace halo
