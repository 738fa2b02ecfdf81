// halo_api.hip -- the C ABI of libhalo.so (declared in include/halo.h).
//
// Host side only: argument validation (every check runs before any HIP call, so invalid
// calls launch nothing and touch no output), workspace carving, and stream-ordered launches
// of the rotation (fwht_quant.hip) and GEMM (gemm.hip) kernels.  The layer entry points
// compose them exactly as the HALO page places the rotations ("HALO: Hadamard-Assisted
// Lower-Precision Optimization for LLMs", abstract: forward and backward, every large
// product in low precision): each product's two operands are rotated and quantised along
// that product's contraction dimension.
#include "../../include/halo.h"
#include "halo_kernels.h"

#include <atomic>
#include <cmath>
#include <cstring>

using namespace halo;

// Scratch of halo_fwht_quant_noalloc: a fixed device array, one copy per device, held until
// the process ends.  In host code its name stands for a host-side shadow, not a device
// address: the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[HALO_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per device (concurrent
// first calls may both look it up and store the same address).  NULL on a HIP error.
void* noalloc_scratch() {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  addr[dev].store(p, std::memory_order_release);
  return p;
}

// Whether an enum argument holds a value in [lo, hi].  A C caller may pass any int in an enum
// parameter, and in C++ loading an enum object whose value lies outside the enum's range is
// undefined, so the value is read through its object representation, before any other use.
// (The argument is taken by reference: passing it by value would itself be such a load.)
template <typename E>
bool enum_in(const E& e, int lo, int hi) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v >= lo && v <= hi;
}
bool dtype_ok(const halo_dtype& t) { return enum_in(t, HALO_F32, HALO_I32); }
bool axis_ok(const halo_axis& a) { return enum_in(a, HALO_ALONG_ROWS, HALO_ALONG_COLS); }

constexpr int64_t kMaxDim = int64_t(1) << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(halo_dtype t) {
  switch (t) {
    case HALO_F32: return 4;
    case HALO_BF16: return 2;
    case HALO_I8: case HALO_E4M3: case HALO_E5M2: return 1;
    case HALO_I32: return 4;
  }
  return 0;
}

bool valid_block(int32_t b) { return b >= 1 && b <= 4096 && (b & (b - 1)) == 0; }

int qt_index(halo_dtype q) {
  switch (q) {
    case HALO_I8: return 0;
    case HALO_E4M3: return 1;
    case HALO_E5M2: return 2;
    case HALO_F32: return 3;
    default: return -1;
  }
}

float qmax_of(halo_dtype q) {
  return q == HALO_I8 ? 127.f : (q == HALO_E4M3 ? 448.f : (q == HALO_E5M2 ? 57344.f : 1.f));
}

halo_status from_hip(hipError_t e) { return e == hipSuccess ? HALO_OK : HALO_ERR_HIP; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Padded (rotated) length of a vector of L elements: a multiple of the block (the zero
// padding of the QWHA page, s5).
int64_t padded_len(int64_t L, int32_t block) { return round_up(L, block); }

// Contraction length of a layer product: the dimension zero-padded to a multiple of the block
// and of 32 (the FP8 matrix cores' k step); blocks past the padded length are all zero and
// get zero codes, so the product equals the one over the padded operands.
int64_t contraction_len(int64_t d, int32_t block) { return round_up(d, block > 32 ? block : 32); }

halo_status check_signs(const uint32_t* signs) {
  return signs && !aligned16(signs) ? HALO_ERR_ALIGN : HALO_OK;
}

// Whether a rows pass over vectors of Lp rotated positions has a kernel: the wave kernel
// (Lp a multiple of 64, one wave per 4096 positions and up to 16 per row; its stochastic
// rounding takes bf16 input), else the older kernel, whose workgroup holds a whole row of up
// to fq_rows_max_len(block) positions.
bool rows_len_ok(int64_t Lp, int32_t block, bool in_bf16, bool sr) {
  return (fq_rows2_supported(Lp, block) && (in_bf16 || !sr)) || Lp <= fq_rows_max_len(block);
}

// Validation of one rotation pass; shared by halo_fwht_quant and the layer calls.
halo_status check_fq(const void* x, halo_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                     halo_axis axis, int32_t block, halo_dtype qt, const void* q, int64_t ldq,
                     const float* scale, const halo_quant_opts* o) {
  if (rows < 0 || cols < 0) return HALO_ERR_SHAPE;
  const bool any = rows > 0 && cols > 0;  // empty matrices may come with NULL pointers
  if ((any && (!x || !q)) || (!scale && (axis == HALO_ALONG_ROWS ? rows : cols) > 0))
    return HALO_ERR_NULL;
  if (xt != HALO_F32 && xt != HALO_BF16) return HALO_ERR_DTYPE;
  if (qt_index(qt) < 0) return HALO_ERR_DTYPE;
  if (axis != HALO_ALONG_ROWS && axis != HALO_ALONG_COLS) return HALO_ERR_SHAPE;
  if (rows >= kMaxDim || cols >= kMaxDim) return HALO_ERR_SHAPE;
  if (ldx < cols || ldx < 1) return HALO_ERR_SHAPE;
  if (!valid_block(block)) return HALO_ERR_BLOCK;
  const int64_t L = axis == HALO_ALONG_ROWS ? cols : rows;
  const int64_t Lp = padded_len(L, block);
  const int64_t nvec = axis == HALO_ALONG_ROWS ? rows : cols;
  if (ldq < Lp || ldq < 1) return HALO_ERR_SHAPE;
  if (Lp % 8 != 0) return HALO_ERR_SHAPE;
  if (axis == HALO_ALONG_ROWS && L % 8 != 0) return HALO_ERR_SHAPE;
  if (axis == HALO_ALONG_COLS && nvec % 8 != 0) return HALO_ERR_SHAPE;
  const bool sr = o && o->rounding == HALO_ROUND_STOCHASTIC;
  if (axis == HALO_ALONG_ROWS && !rows_len_ok(Lp, block, xt == HALO_BF16, sr))
    return HALO_ERR_SHAPE;
  if (o) {
    if (o->rounding != HALO_ROUND_NEAREST_EVEN && o->rounding != HALO_ROUND_STOCHASTIC)
      return HALO_ERR_OPTION;
    if (o->rounding == HALO_ROUND_STOCHASTIC && qt == HALO_F32) return HALO_ERR_OPTION;
  }
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return HALO_ERR_ALIGN;
  if ((ldx * esize(xt)) % 16 != 0 || (ldq * esize(qt)) % 16 != 0) return HALO_ERR_ALIGN;
  if (o && check_signs(o->signs) != HALO_OK) return HALO_ERR_ALIGN;
  return HALO_OK;
}

// Options of one pass: the transform's signs and the rounding of its codes.
struct PassOpts {
  const uint32_t* signs = nullptr;
  int sr = 0;
  uint32_t key0 = 0, key1 = 0, ctr2 = 0, ctr3 = 0;
  uint32_t polls = 0;
};

PassOpts pass_opts(const halo_quant_opts* o) {
  PassOpts p;
  if (!o) return p;
  p.signs = o->signs;
  p.sr = o->rounding == HALO_ROUND_STOCHASTIC ? 1 : 0;
  p.key0 = o->seed[0];
  p.key1 = o->seed[1];
  p.ctr2 = o->counter[0];
  p.ctr3 = o->counter[1];
  p.polls = o->exchange_polls;
  return p;
}

// Arguments of one pass over x[rows x cols]; len: the rotated (padded) length, 0 = the
// vector length padded to a multiple of the block.
FqArgs make_fq(const void* x, int64_t rows, int64_t cols, int64_t ldx, halo_axis axis,
               int32_t block, halo_dtype qt, void* q, int64_t ldq, float* scale,
               const PassOpts& po = PassOpts(), int64_t len = 0) {
  FqArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.nvec = axis == HALO_ALONG_ROWS ? rows : cols;
  a.in_len = axis == HALO_ALONG_ROWS ? cols : rows;
  a.len = len > 0 ? len : padded_len(a.in_len, block);
  a.q = q;
  a.ldq = ldq;
  a.scale = scale;
  a.block = block;
  a.qmax = qmax_of(qt);
  a.denom = (float)((double)a.qmax * std::sqrt((double)block));
  a.inv_sqrt_b = (float)(1.0 / std::sqrt((double)block));
  a.signs = po.signs;
  a.sr = po.sr;
  a.key0 = po.key0;
  a.key1 = po.key1;
  a.ctr2 = po.ctr2;
  a.ctr3 = po.ctr3;
  a.polls = po.polls;
  return a;
}

halo_status run_fa(const FqArgs& a, halo_dtype xt, halo_axis axis, halo_dtype qt, void* ws,
                   size_t ws_bytes, hipStream_t st) {
  return from_hip(launch_fwht_quant(a, xt == HALO_BF16 ? 1 : 0, qt_index(qt), (int)axis, ws,
                                    ws ? ws_bytes : 0, st));
}

halo_status run_fq(const void* x, halo_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                   halo_axis axis, int32_t block, halo_dtype qt, void* q, int64_t ldq,
                   float* scale, void* ws, size_t ws_bytes, hipStream_t st,
                   const PassOpts& po = PassOpts(), int64_t len = 0) {
  const FqArgs a = make_fq(x, rows, cols, ldx, axis, block, qt, q, ldq, scale, po, len);
  return run_fa(a, xt, axis, qt, ws, ws_bytes, st);
}

// Scratch of one rotation pass (the single-read columns kernel's partial maxima and counters);
// len: the rotated (padded) length.
// The same for bf16 and fp32 input.
size_t fq_ws_bytes_len(int64_t len, int64_t nvec, halo_axis axis, int32_t block) {
  if (axis != HALO_ALONG_COLS) return 0;
  return fq_cols2_ws_bytes(len, nvec, block);
}

// The GEMM kernel loads each code operand through a buffer resource of 2^32 - 1 bytes with
// 32-bit byte offsets: an operand of `rows` rows (leading dimension ld bytes, k bytes used per
// row) must end below byte 2^32 - 1 of its base (a load reaching past the resource's size would
// read zeros).  Both ld and k are multiples of 16, so the span is at most 2^32 - 16.
bool operand_fits(int64_t rows, int64_t ld, int64_t k) {
  return rows <= 0 || (rows - 1) * ld + k < (int64_t(1) << 32);
}

halo_status check_gemm(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t m,
                       int64_t n, int64_t k, const void* c, halo_dtype ct, int64_t ldc,
                       const float* sa, const float* sb, int kmult) {
  if (m < 0 || n < 0 || k <= 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim)
    return HALO_ERR_SHAPE;
  // empty operands may come with NULL pointers
  if ((m > 0 && !a) || (n > 0 && !b) || (m > 0 && n > 0 && !c)) return HALO_ERR_NULL;
  if (ct != HALO_I32 && ((m > 0 && !sa) || (n > 0 && !sb))) return HALO_ERR_NULL;
  if (k % kmult != 0) return HALO_ERR_SHAPE;
  if (lda < k || ldb < k || ldc < n || ldc < 1) return HALO_ERR_SHAPE;
  if (!operand_fits(m, lda, k) || !operand_fits(n, ldb, k)) return HALO_ERR_SHAPE;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return HALO_ERR_ALIGN;
  if (lda % 16 != 0 || ldb % 16 != 0 || (ldc * esize(ct)) % 16 != 0) return HALO_ERR_ALIGN;
  return HALO_OK;
}

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }


// Region sizes of the layer workspace, in carve order; the backward's last region is the
// scratch of its three column passes (W, dY, X: one sub-region each, cleared together by the
// first kernel of the call).
struct WsPlan {
  size_t off[9];
  size_t total;
  size_t scratch_off, scratch_bytes;
  size_t scr_w, scr_dy, scr_x;  // sub-region sizes, in this order
};

WsPlan plan_ws(int64_t m, int64_t n, int64_t k, int backward, int32_t block) {
  WsPlan p{};
  size_t sizes[9];
  int cnt = 0;
  const int64_t kq = contraction_len(k, block), nq = contraction_len(n, block),
                mq = contraction_len(m, block);
  if (!backward) {
    sizes[cnt++] = (size_t)m * kq;     // X codes   [m x kq]
    sizes[cnt++] = (size_t)m * 4;      // X scales
    sizes[cnt++] = (size_t)n * kq;     // W codes   [n x kq]
    sizes[cnt++] = (size_t)n * 4;      // W scales
  } else {
    sizes[cnt++] = (size_t)m * nq;     // dY row codes     [m x nq]
    sizes[cnt++] = (size_t)m * 4;
    sizes[cnt++] = (size_t)k * nq;     // W column codes   [k x nq]
    sizes[cnt++] = (size_t)k * 4;
    sizes[cnt++] = (size_t)n * mq;     // dY column codes  [n x mq]
    sizes[cnt++] = (size_t)n * 4;
    sizes[cnt++] = (size_t)k * mq;     // X column codes   [k x mq]
    sizes[cnt++] = (size_t)k * 4;
  }
  size_t o = 0;
  for (int i = 0; i < cnt; ++i) {
    p.off[i] = o;
    o += round256(sizes[i]);
  }
  if (backward) {
    p.scr_w = round256(fq_ws_bytes_len(nq, k, HALO_ALONG_COLS, block));   // W columns along n
    p.scr_dy = round256(fq_ws_bytes_len(mq, n, HALO_ALONG_COLS, block));  // dY columns along m
    p.scr_x = round256(fq_ws_bytes_len(mq, k, HALO_ALONG_COLS, block));   // X columns along m
  }
  p.scratch_off = o;
  p.scratch_bytes = p.scr_w + p.scr_dy + p.scr_x;
  p.total = o + p.scratch_bytes;
  return p;
}

int gemm_kind_fmt(halo_dtype t) { return t == HALO_E5M2 ? 1 : 0; }

halo_status gemm_any(const void* a, halo_dtype at, int64_t lda, const float* sa, const void* b,
                     halo_dtype bt, int64_t ldb, const float* sb, int64_t m, int64_t n, int64_t k,
                     void* c, halo_dtype ct, int64_t ldc, hipStream_t st) {
  GemmArgs g{a, lda, b, ldb, sa, sb, c, ldc, m, n, k};
  const int out = ct == HALO_I32 ? 0 : (ct == HALO_F32 ? 1 : 2);
  if (at == HALO_I8) return from_hip(launch_gemm(g, 0, 0, 0, out, st));
  return from_hip(launch_gemm(g, 1, gemm_kind_fmt(at), gemm_kind_fmt(bt), out, st));
}

bool layer_dims_ok(int64_t m, int64_t n, int64_t k) {
  return m >= 0 && n >= 0 && k >= 0 && m < kMaxDim && n < kMaxDim && k < kMaxDim;
}

}  // namespace

extern "C" {

halo_status halo_mfma_rate_probe(int32_t kind, int32_t iters, int64_t* ops, void* stream) {
  if (!ops) return HALO_ERR_NULL;
  if (kind < 0 || kind > 2 || iters < 2 || iters > (1 << 20)) return HALO_ERR_SHAPE;
  const hipError_t e = launch_mfma_probe(kind, iters, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return HALO_ERR_HIP;
  *ops = mfma_probe_ops(kind, iters);
  return HALO_OK;
}

const char* halo_status_str(halo_status s) {
  if (!enum_in(s, HALO_OK, HALO_ERR_OPTION)) return "unknown status";
  switch (s) {
    case HALO_OK: return "ok";
    case HALO_ERR_NULL: return "a required pointer is NULL";
    case HALO_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case HALO_ERR_BLOCK: return "block must be a power of two in [1, 4096]";
    case HALO_ERR_DTYPE: return "unsupported element type";
    case HALO_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case HALO_ERR_WORKSPACE: return "workspace missing or too small";
    case HALO_ERR_HIP: return "HIP launch failed";
    case HALO_ERR_OPTION: return "invalid rounding option";
  }
  return "unknown status";
}

size_t halo_fwht_quant_workspace_bytes(int64_t rows, int64_t cols, halo_axis axis,
                                       int32_t block, halo_dtype x_type) {
  if (!axis_ok(axis) || !dtype_ok(x_type)) return 0;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim || !valid_block(block))
    return 0;
  if (axis != HALO_ALONG_COLS) return 0;
  return fq_ws_bytes_len(padded_len(rows, block), cols, axis, block);
}

halo_status halo_fwht_quant_ex(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                               int64_t ldx, halo_axis axis, int32_t block, halo_dtype q_type,
                               void* q, int64_t ldq, float* scale, const halo_quant_opts* opts,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(x_type) || !dtype_ok(q_type)) return HALO_ERR_DTYPE;
  if (!axis_ok(axis)) return HALO_ERR_SHAPE;
  halo_status s = check_fq(x, x_type, rows, cols, ldx, axis, block, q_type, q, ldq, scale, opts);
  if (s != HALO_OK) return s;
  if (ws && !aligned16(ws)) return HALO_ERR_ALIGN;
  return run_fq(x, x_type, rows, cols, ldx, axis, block, q_type, q, ldq, scale, ws, ws_bytes,
                (hipStream_t)stream, pass_opts(opts));
}

halo_status halo_fwht_quant(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                            int64_t ldx, halo_axis axis, int32_t block, halo_dtype q_type,
                            void* q, int64_t ldq, float* scale, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!dtype_ok(x_type) || !dtype_ok(q_type)) return HALO_ERR_DTYPE;
  if (!axis_ok(axis)) return HALO_ERR_SHAPE;
  return halo_fwht_quant_ex(x, x_type, rows, cols, ldx, axis, block, q_type, q, ldq, scale,
                            nullptr, ws, ws_bytes, stream);
}

halo_status halo_fwht_quant_noalloc(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                                    int64_t ldx, halo_axis axis, int32_t block,
                                    halo_dtype q_type, void* q, int64_t ldq, float* scale,
                                    const halo_quant_opts* opts, void* stream) {
  if (!dtype_ok(x_type) || !dtype_ok(q_type)) return HALO_ERR_DTYPE;
  if (!axis_ok(axis)) return HALO_ERR_SHAPE;
  halo_status s = check_fq(x, x_type, rows, cols, ldx, axis, block, q_type, q, ldq, scale, opts);
  if (s != HALO_OK) return s;
  const size_t need = halo_fwht_quant_workspace_bytes(rows, cols, axis, block, x_type);
  if (need > HALO_NOALLOC_SCRATCH_BYTES) return HALO_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && !(ws = noalloc_scratch())) return HALO_ERR_HIP;
  return run_fq(x, x_type, rows, cols, ldx, axis, block, q_type, q, ldq, scale, ws,
                ws ? HALO_NOALLOC_SCRATCH_BYTES : 0, (hipStream_t)stream, pass_opts(opts));
}

size_t halo_fwht_quant_dual_workspace_bytes(int64_t rows, int64_t cols, int32_t block,
                                            halo_dtype x_type) {
  if (!dtype_ok(x_type)) return 0;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim || !valid_block(block))
    return 0;
  // the single-read launch's scratch, or, for shapes it does not take, the columns pass's
  const size_t dual = fq_dual_ws_bytes(rows, cols, block, x_type == HALO_BF16 ? 1 : 0);
  const size_t cols_ws = fq_ws_bytes_len(padded_len(rows, block), cols, HALO_ALONG_COLS, block);
  return dual > cols_ws ? dual : cols_ws;
}

halo_status halo_fwht_quant_dual(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                                 int64_t ldx, int32_t block, halo_dtype q_type, void* qr,
                                 int64_t ldqr, float* scale_r, void* qc, int64_t ldqc,
                                 float* scale_c, const halo_quant_opts* row_opts,
                                 const halo_quant_opts* col_opts, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!dtype_ok(x_type) || !dtype_ok(q_type)) return HALO_ERR_DTYPE;
  halo_status s = check_fq(x, x_type, rows, cols, ldx, HALO_ALONG_ROWS, block, q_type, qr, ldqr,
                           scale_r, row_opts);
  if (s != HALO_OK) return s;
  s = check_fq(x, x_type, rows, cols, ldx, HALO_ALONG_COLS, block, q_type, qc, ldqc, scale_c,
               col_opts);
  if (s != HALO_OK) return s;
  if (ws && !aligned16(ws)) return HALO_ERR_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  const FqArgs ar = make_fq(x, rows, cols, ldx, HALO_ALONG_ROWS, block, q_type, qr, ldqr, scale_r,
                            pass_opts(row_opts));
  const FqArgs ac = make_fq(x, rows, cols, ldx, HALO_ALONG_COLS, block, q_type, qc, ldqc, scale_c,
                            pass_opts(col_opts));
  const int inb = x_type == HALO_BF16 ? 1 : 0;
  if (ws && fq_dual_supported(rows, cols, block, inb, qt_index(q_type), ar.sr != 0, ac.sr != 0,
                              ws_bytes))
    return from_hip(launch_fq_dual(ar, ac, ws, qt_index(q_type), 0, st));
  s = run_fa(ar, x_type, HALO_ALONG_ROWS, q_type, nullptr, 0, st);
  if (s != HALO_OK) return s;
  return run_fa(ac, x_type, HALO_ALONG_COLS, q_type, ws, ws ? ws_bytes : 0, st);
}

halo_status halo_gemm_i8(const int8_t* a, int64_t lda, const float* sa, const int8_t* b,
                         int64_t ldb, const float* sb, int64_t m, int64_t n, int64_t k, void* c,
                         halo_dtype c_type, int64_t ldc, void* stream) {
  if (!dtype_ok(c_type)) return HALO_ERR_DTYPE;
  if (c_type != HALO_I32 && c_type != HALO_F32 && c_type != HALO_BF16) return HALO_ERR_DTYPE;
  halo_status s = check_gemm(a, lda, b, ldb, m, n, k, c, c_type, ldc, sa, sb, 16);
  if (s != HALO_OK) return s;
  if (c_type != HALO_I32 && (!aligned16(sa) || !aligned16(sb))) return HALO_ERR_ALIGN;
  return gemm_any(a, HALO_I8, lda, sa, b, HALO_I8, ldb, sb, m, n, k, c, c_type, ldc,
                  (hipStream_t)stream);
}

halo_status halo_gemm_fp8(const void* a, halo_dtype a_type, int64_t lda, const float* sa,
                          const void* b, halo_dtype b_type, int64_t ldb, const float* sb,
                          int64_t m, int64_t n, int64_t k, void* c, halo_dtype c_type,
                          int64_t ldc, void* stream) {
  if (!dtype_ok(a_type) || !dtype_ok(b_type) || !dtype_ok(c_type)) return HALO_ERR_DTYPE;
  if ((a_type != HALO_E4M3 && a_type != HALO_E5M2) || (b_type != HALO_E4M3 && b_type != HALO_E5M2))
    return HALO_ERR_DTYPE;
  if (c_type != HALO_F32 && c_type != HALO_BF16) return HALO_ERR_DTYPE;
  halo_status s = check_gemm(a, lda, b, ldb, m, n, k, c, c_type, ldc, sa, sb, 32);
  if (s != HALO_OK) return s;
  if (!aligned16(sa) || !aligned16(sb)) return HALO_ERR_ALIGN;
  return gemm_any(a, a_type, lda, sa, b, b_type, ldb, sb, m, n, k, c, c_type, ldc,
                  (hipStream_t)stream);
}


size_t halo_linear_workspace_bytes_ex(int64_t m, int64_t n, int64_t k, int32_t block,
                                      halo_dtype q_type, int backward) {
  if (!dtype_ok(q_type)) return 0;
  if (!layer_dims_ok(m, n, k) || !valid_block(block)) return 0;
  if (q_type != HALO_I8 && q_type != HALO_E4M3) return 0;
  return plan_ws(m, n, k, backward ? 1 : 0, block).total;
}

size_t halo_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, halo_dtype q_type,
                                   int backward) {
  if (!dtype_ok(q_type)) return 0;
  size_t most = 0;
  for (int32_t b = 1; b <= 4096; b *= 2) {
    const size_t t = halo_linear_workspace_bytes_ex(m, n, k, b, q_type, backward);
    if (t > most) most = t;
  }
  return most;
}

halo_status halo_linear_fwd_ex(const void* x, const void* w, halo_dtype io_type, int64_t m,
                               int64_t n, int64_t k, int32_t block, halo_dtype q_type, void* y,
                               halo_dtype y_type, const halo_linear_opts* opts, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!dtype_ok(io_type) || !dtype_ok(q_type) || !dtype_ok(y_type)) return HALO_ERR_DTYPE;
  if (!layer_dims_ok(m, n, k) || k == 0) return HALO_ERR_SHAPE;
  if ((m > 0 && !x) || (n > 0 && !w) || (m > 0 && n > 0 && !y)) return HALO_ERR_NULL;
  if (io_type != HALO_F32 && io_type != HALO_BF16) return HALO_ERR_DTYPE;
  if (q_type != HALO_I8 && q_type != HALO_E4M3) return HALO_ERR_DTYPE;
  if (y_type != HALO_F32 && y_type != HALO_BF16) return HALO_ERR_DTYPE;
  if (!valid_block(block)) return HALO_ERR_BLOCK;
  const int64_t kq = contraction_len(k, block);
  if (k % 8 != 0 || !rows_len_ok(kq, block, io_type == HALO_BF16, false)) return HALO_ERR_SHAPE;
  if (!operand_fits(m, kq, kq) || !operand_fits(n, kq, kq)) return HALO_ERR_SHAPE;
  if (opts && (opts->grad_rounding != HALO_ROUND_NEAREST_EVEN &&
               opts->grad_rounding != HALO_ROUND_STOCHASTIC))
    return HALO_ERR_OPTION;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return HALO_ERR_ALIGN;
  if ((n * esize(y_type)) % 16 != 0) return HALO_ERR_ALIGN;
  if (opts && check_signs(opts->signs_k) != HALO_OK) return HALO_ERR_ALIGN;
  const WsPlan p = plan_ws(m, n, k, 0, block);
  if (!ws || ws_bytes < p.total) return HALO_ERR_WORKSPACE;
  if (!aligned16(ws)) return HALO_ERR_ALIGN;
  char* base = static_cast<char*>(ws);
  void* qx = base + p.off[0];
  float* sx = reinterpret_cast<float*>(base + p.off[1]);
  void* qw = base + p.off[2];
  float* sw = reinterpret_cast<float*>(base + p.off[3]);
  hipStream_t st = (hipStream_t)stream;
  PassOpts po;  // X and W: the signs along k, nearest-even codes
  if (opts) po.signs = opts->signs_k;
  const FqArgs ax = make_fq(x, m, k, k, HALO_ALONG_ROWS, block, q_type, qx, kq, sx, po, kq);
  const FqArgs aw = make_fq(w, n, k, k, HALO_ALONG_ROWS, block, q_type, qw, kq, sw, po, kq);
  halo_status s = HALO_OK;
  if (fq_rows2_supported(kq, block)) {  // X and W rows in one launch
    FqPair pp{};
    pp.p0 = ax;
    pp.p1 = aw;
    pp.has1 = 1;
    s = from_hip(launch_fq_rows2_pair(pp, io_type == HALO_BF16 ? 1 : 0, qt_index(q_type), st));
  } else {
    s = run_fa(ax, io_type, HALO_ALONG_ROWS, q_type, nullptr, 0, st);
    if (s == HALO_OK) s = run_fa(aw, io_type, HALO_ALONG_ROWS, q_type, nullptr, 0, st);
  }
  if (s == HALO_OK)
    s = gemm_any(qx, q_type, kq, sx, qw, q_type, kq, sw, m, n, kq, y, y_type, n, st);
  return s;
}

halo_status halo_linear_fwd(const void* x, const void* w, halo_dtype io_type, int64_t m,
                            int64_t n, int64_t k, int32_t block, halo_dtype q_type, void* y,
                            halo_dtype y_type, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(io_type) || !dtype_ok(q_type) || !dtype_ok(y_type)) return HALO_ERR_DTYPE;
  return halo_linear_fwd_ex(x, w, io_type, m, n, k, block, q_type, y, y_type, nullptr, ws,
                            ws_bytes, stream);
}

halo_status halo_linear_bwd_ex(const void* dy, const void* x, const void* w, halo_dtype io_type,
                               int64_t m, int64_t n, int64_t k, int32_t block, halo_dtype q_type,
                               halo_dtype grad_q_type, void* dx, void* dw,
                               const halo_linear_opts* opts, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!dtype_ok(io_type) || !dtype_ok(q_type) || !dtype_ok(grad_q_type)) return HALO_ERR_DTYPE;
  if (!dy || !x || !w) return HALO_ERR_NULL;
  if (io_type != HALO_F32 && io_type != HALO_BF16) return HALO_ERR_DTYPE;
  if (q_type == HALO_I8) {
    if (grad_q_type != HALO_I8) return HALO_ERR_DTYPE;
  } else if (q_type == HALO_E4M3) {
    if (grad_q_type != HALO_E5M2 && grad_q_type != HALO_E4M3) return HALO_ERR_DTYPE;
  } else {
    return HALO_ERR_DTYPE;
  }
  if (!layer_dims_ok(m, n, k) || m == 0 || n == 0 || k == 0) return HALO_ERR_SHAPE;
  if (!valid_block(block)) return HALO_ERR_BLOCK;
  const int64_t nq = contraction_len(n, block), mq = contraction_len(m, block);
  if (n % 8 != 0 || k % 8 != 0) return HALO_ERR_SHAPE;
  const bool sr_dy = opts && opts->grad_rounding == HALO_ROUND_STOCHASTIC;
  if (dx && !rows_len_ok(nq, block, io_type == HALO_BF16, sr_dy)) return HALO_ERR_SHAPE;
  if (!operand_fits(m, nq, nq) || !operand_fits(k, nq, nq) || !operand_fits(n, mq, mq) ||
      !operand_fits(k, mq, mq))
    return HALO_ERR_SHAPE;
  if (opts && (opts->grad_rounding != HALO_ROUND_NEAREST_EVEN &&
               opts->grad_rounding != HALO_ROUND_STOCHASTIC))
    return HALO_ERR_OPTION;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(w)) return HALO_ERR_ALIGN;
  if ((dx && !aligned16(dx)) || (dw && !aligned16(dw))) return HALO_ERR_ALIGN;
  if (opts && (check_signs(opts->signs_n) != HALO_OK || check_signs(opts->signs_m) != HALO_OK))
    return HALO_ERR_ALIGN;
  const WsPlan p = plan_ws(m, n, k, 1, block);
  if (!ws || ws_bytes < p.total) return HALO_ERR_WORKSPACE;
  if (!aligned16(ws)) return HALO_ERR_ALIGN;
  char* base = static_cast<char*>(ws);
  char* scr = base + p.scratch_off;
  void* scr_w = scr;
  void* scr_dy = scr + p.scr_w;
  void* scr_x = scr + p.scr_w + p.scr_dy;
  const int inb = io_type == HALO_BF16 ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  halo_status s = HALO_OK;

  // pass options: the signs along each contraction dimension; the dY codes' rounding (its
  // columns pass draws at counter word 3 ^ 2^31)
  PassOpts on, om, gn, gm;
  if (opts) {
    on.signs = gn.signs = opts->signs_n;
    om.signs = gm.signs = opts->signs_m;
    gn.sr = gm.sr = opts->grad_rounding == HALO_ROUND_STOCHASTIC ? 1 : 0;
    gn.key0 = gm.key0 = opts->seed[0];
    gn.key1 = gm.key1 = opts->seed[1];
    gn.ctr2 = gm.ctr2 = opts->counter[0];
    gn.ctr3 = opts->counter[1];
    gm.ctr3 = opts->counter[1] ^ 0x80000000u;
    on.polls = om.polls = gn.polls = gm.polls = opts->exchange_polls;
  }
  void* qdy = base + p.off[0];
  float* sdy = reinterpret_cast<float*>(base + p.off[1]);
  void* qwt = base + p.off[2];
  float* swt = reinterpret_cast<float*>(base + p.off[3]);
  void* qdyt = base + p.off[4];
  float* sdyt = reinterpret_cast<float*>(base + p.off[5]);
  void* qxt = base + p.off[6];
  float* sxt = reinterpret_cast<float*>(base + p.off[7]);
  // dX = dY W: rows of dY and columns of W along n; dW = dY^T X: columns of dY and X along m
  const FqArgs rows = make_fq(dy, m, n, n, HALO_ALONG_ROWS, block, grad_q_type, qdy, nq, sdy, gn, nq);
  const FqArgs cw = make_fq(w, n, k, k, HALO_ALONG_COLS, block, q_type, qwt, nq, swt, on, nq);
  const FqArgs cdy = make_fq(dy, m, n, n, HALO_ALONG_COLS, block, grad_q_type, qdyt, mq, sdyt, gm, mq);
  const FqArgs cx = make_fq(x, m, k, k, HALO_ALONG_COLS, block, q_type, qxt, mq, sxt, om, mq);

  // the single-read column passes need their scratch cleared: folded into the first kernel
  // when that is a rows pass, else one fill
  bool zero_pending = p.scratch_bytes > 0;
  auto clear_scratch = [&]() {
    if (!zero_pending || s != HALO_OK) return;
    s = from_hip(launch_fill_zero(reinterpret_cast<float*>(scr), (int64_t)(p.scratch_bytes / 4), st));
    zero_pending = false;
  };
  // one column pass: single-read when covered (its scratch already clear), else two reads
  auto cols_pass = [&](const FqArgs& a, halo_dtype qt, void* sws, size_t sbytes) {
    if (s != HALO_OK) return;
    if (fq_cols2_supported(a.len, a.nvec, block, inb, a.sr != 0, sbytes))
      s = from_hip(launch_fq_cols2_pair(a, sws, nullptr, nullptr, inb, qt_index(qt), 1, st));
    else
      s = run_fa(a, io_type, HALO_ALONG_COLS, qt, nullptr, 0, st);
  };
  // the rows pass of dY, clearing the scratch as a side job when it runs as the wave kernel
  auto rows_pass = [&]() {
    if (s != HALO_OK) return;
    if (fq_rows2_supported(nq, block) && (inb || !rows.sr)) {
      FqPair pp{};
      pp.p0 = rows;
      if (zero_pending) {
        pp.zero = reinterpret_cast<uint32_t*>(scr);
        pp.nzero = (int64_t)(p.scratch_bytes / 4);
        zero_pending = false;
      }
      s = from_hip(launch_fq_rows2_pair(pp, inb, qt_index(grad_q_type), st));
    } else {
      s = run_fa(rows, io_type, HALO_ALONG_ROWS, grad_q_type, nullptr, 0, st);
    }
  };
  const int qg = qt_index(grad_q_type), qw = qt_index(q_type);
  const bool pair_ok = (qg == 0 && qw == 0) || (qg == 2 && qw == 1) || (qg == 1 && qw == 1);
  if (dx && dw && inb && pair_ok && fq_cols2_supported(nq, k, block, 1, false, p.scr_w) &&
      fq_cols2_supported(mq, n, block, 1, cdy.sr != 0, p.scr_dy) &&
      fq_cols2_supported(mq, k, block, 1, false, p.scr_x)) {
    // every rotation pass of the backward in one launch (or two, when the dY rows are long):
    // the passes overlap on the device, then the two products
    const bool rows_in = fq_batch_rows_ok(nq);
    if (rows_in) {
      clear_scratch();
    } else {
      rows_pass();
      clear_scratch();
    }
    if (s == HALO_OK)
      s = from_hip(launch_fq_batch(rows_in ? &rows : nullptr, cw, scr_w, cdy, scr_dy, cx, scr_x,
                                   qg, qw, st));
  } else {
    if (dx) rows_pass();
    clear_scratch();
    if (dx) cols_pass(cw, q_type, scr_w, p.scr_w);
    if (dw) {
      const bool c1 = fq_cols2_supported(mq, n, block, inb, cdy.sr != 0, p.scr_dy);
      const bool c2 = fq_cols2_supported(mq, k, block, inb, cx.sr != 0, p.scr_x);
      if (s == HALO_OK && c1 && c2 && grad_q_type == q_type && cdy.sr == cx.sr) {
        // dY and X columns in one launch
        s = from_hip(launch_fq_cols2_pair(cdy, scr_dy, &cx, scr_x, inb, qt_index(q_type), 1, st));
      } else {
        cols_pass(cdy, grad_q_type, scr_dy, p.scr_dy);
        cols_pass(cx, q_type, scr_x, p.scr_x);
      }
    }
  }
  if (s == HALO_OK && dx && dw) {  // both products in one launch
    const GemmArgs gx{qdy, nq, qwt, nq, sdy, swt, dx, k, m, k, nq};
    const GemmArgs gw{qdyt, mq, qxt, mq, sdyt, sxt, dw, k, n, k, mq};
    const int out = io_type == HALO_F32 ? 1 : 2;
    if (grad_q_type == HALO_I8)
      s = from_hip(launch_gemm_pair(gx, &gw, 0, 0, 0, out, st));
    else
      s = from_hip(launch_gemm_pair(gx, &gw, 1, gemm_kind_fmt(grad_q_type), gemm_kind_fmt(q_type),
                                    out, st));
    return s;
  }
  if (s == HALO_OK && dx)
    s = gemm_any(qdy, grad_q_type, nq, sdy, qwt, q_type, nq, swt, m, k, nq, dx, io_type, k, st);
  if (s == HALO_OK && dw)
    s = gemm_any(qdyt, grad_q_type, mq, sdyt, qxt, q_type, mq, sxt, n, k, mq, dw, io_type, k, st);
  return s;
}

halo_status halo_linear_bwd(const void* dy, const void* x, const void* w, halo_dtype io_type,
                            int64_t m, int64_t n, int64_t k, int32_t block, halo_dtype q_type,
                            halo_dtype grad_q_type, void* dx, void* dw, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!dtype_ok(io_type) || !dtype_ok(q_type) || !dtype_ok(grad_q_type)) return HALO_ERR_DTYPE;
  return halo_linear_bwd_ex(dy, x, w, io_type, m, n, k, block, q_type, grad_q_type, dx, dw,
                            nullptr, ws, ws_bytes, stream);
}

}  // extern "C"
