// fwht_wave_sr.hip -- the stochastic-rounding instantiations of the wave-slice rotation
// kernels (fwht_wave.h), for the code types INT8, E4M3 and E5M2 and bf16 input.  Stochastic
// rounding ("QWHA方法：基于Walsh-Hadamard变换的高效大模型微调技术" s5) draws one Philox4x32-10
// uniform per element; see store_chunk8_sr.
#include "fwht_wave.h"

namespace halo {

hipError_t cols2_dispatch_sr(const FqArgs& a0, void* ws0, const FqArgs* a1, void* ws1, int qt,
                             int prezeroed, hipStream_t st) {
  switch (qt) {
    case 0: return cols2_block<0, true>(a0, ws0, a1, ws1, prezeroed, st);
    case 1: return cols2_block<1, true>(a0, ws0, a1, ws1, prezeroed, st);
    case 2: return cols2_block<2, true>(a0, ws0, a1, ws1, prezeroed, st);
  }
  return hipErrorInvalidValue;
}

hipError_t batch_dispatch_sr(int qg, int qw, const FqArgs* rows, const FqArgs& cw, void* ws_w,
                             const FqArgs& cdy, void* ws_dy, const FqArgs& cx, void* ws_x,
                             hipStream_t st) {
  if (qg == 0 && qw == 0) return batch_block<0, 0, true>(cw.block, rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  if (qg == 2 && qw == 1) return batch_block<2, 1, true>(cw.block, rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  if (qg == 1 && qw == 1) return batch_block<1, 1, true>(cw.block, rows, cw, ws_w, cdy, ws_dy, cx, ws_x, st);
  return hipErrorInvalidValue;
}

hipError_t rows2_dispatch_sr(const FqPair& a, int qt, hipStream_t st) {
  switch (qt) {
    case 0: return rows2_block<uint16_t, 0, true>(a, st);
    case 1: return rows2_block<uint16_t, 1, true>(a, st);
    case 2: return rows2_block<uint16_t, 2, true>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace halo
