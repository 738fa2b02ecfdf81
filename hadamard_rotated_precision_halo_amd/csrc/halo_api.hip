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

#include <cmath>

using namespace halo;

namespace {

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

// Validation of one rotation pass; shared by halo_fwht_quant and the layer calls.
halo_status check_fq(const void* x, halo_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                     halo_axis axis, int32_t block, halo_dtype qt, const void* q, int64_t ldq,
                     const float* scale) {
  if (rows < 0 || cols < 0) return HALO_ERR_SHAPE;
  const bool any = rows > 0 && cols > 0;  // empty matrices may come with NULL pointers
  if ((any && (!x || !q)) || (!scale && (axis == HALO_ALONG_ROWS ? rows : cols) > 0))
    return HALO_ERR_NULL;
  if (xt != HALO_F32 && xt != HALO_BF16) return HALO_ERR_DTYPE;
  if (qt_index(qt) < 0) return HALO_ERR_DTYPE;
  if (axis != HALO_ALONG_ROWS && axis != HALO_ALONG_COLS) return HALO_ERR_SHAPE;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return HALO_ERR_SHAPE;
  if (ldx < cols || ldx < 1) return HALO_ERR_SHAPE;
  const int64_t L = axis == HALO_ALONG_ROWS ? cols : rows;
  const int64_t nvec = axis == HALO_ALONG_ROWS ? rows : cols;
  if (ldq < L || ldq < 1) return HALO_ERR_SHAPE;
  if (!valid_block(block) || (L % block) != 0) return HALO_ERR_BLOCK;
  if (L % 8 != 0) return HALO_ERR_SHAPE;
  if (axis == HALO_ALONG_COLS && nvec % 8 != 0) return HALO_ERR_SHAPE;
  if (axis == HALO_ALONG_ROWS && L > fq_rows_max_len(block)) return HALO_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return HALO_ERR_ALIGN;
  if ((ldx * esize(xt)) % 16 != 0 || (ldq * esize(qt)) % 16 != 0) return HALO_ERR_ALIGN;
  return HALO_OK;
}

FqArgs make_fq(const void* x, int64_t rows, int64_t cols, int64_t ldx, halo_axis axis,
               int32_t block, halo_dtype qt, void* q, int64_t ldq, float* scale) {
  FqArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.nvec = axis == HALO_ALONG_ROWS ? rows : cols;
  a.len = axis == HALO_ALONG_ROWS ? cols : rows;
  a.q = q;
  a.ldq = ldq;
  a.scale = scale;
  a.block = block;
  a.qmax = qmax_of(qt);
  a.denom = (float)((double)a.qmax * std::sqrt((double)block));
  a.inv_sqrt_b = (float)(1.0 / std::sqrt((double)block));
  return a;
}

halo_status run_fq(const void* x, halo_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                   halo_axis axis, int32_t block, halo_dtype qt, void* q, int64_t ldq,
                   float* scale, void* ws, size_t ws_bytes, hipStream_t st) {
  FqArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.nvec = axis == HALO_ALONG_ROWS ? rows : cols;
  a.len = axis == HALO_ALONG_ROWS ? cols : rows;
  a.q = q;
  a.ldq = ldq;
  a.scale = scale;
  a.block = block;
  a.qmax = qmax_of(qt);
  a.denom = (float)((double)a.qmax * std::sqrt((double)block));
  a.inv_sqrt_b = (float)(1.0 / std::sqrt((double)block));
  return from_hip(launch_fwht_quant(a, xt == HALO_BF16 ? 1 : 0, qt_index(qt), (int)axis, ws,
                                    ws ? ws_bytes : 0, st));
}

// Scratch of one rotation pass (the single-read columns kernel's partial maxima and counters).
size_t fq_ws_bytes(int64_t rows, int64_t cols, halo_axis axis, int32_t block, halo_dtype xt) {
  if (axis != HALO_ALONG_COLS) return 0;
  return fq_cols2_ws_bytes(rows, cols, block, xt == HALO_BF16 ? 1 : 0);
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

WsPlan plan_ws(int64_t m, int64_t n, int64_t k, int backward, int32_t block, halo_dtype io) {
  WsPlan p{};
  size_t sizes[9];
  int cnt = 0;
  if (!backward) {
    sizes[cnt++] = (size_t)m * k;      // X codes   [m x k]
    sizes[cnt++] = (size_t)m * 4;      // X scales
    sizes[cnt++] = (size_t)n * k;      // W codes   [n x k]
    sizes[cnt++] = (size_t)n * 4;      // W scales
  } else {
    sizes[cnt++] = (size_t)m * n;      // dY row codes     [m x n]
    sizes[cnt++] = (size_t)m * 4;
    sizes[cnt++] = (size_t)k * n;      // W column codes   [k x n]
    sizes[cnt++] = (size_t)k * 4;
    sizes[cnt++] = (size_t)n * m;      // dY column codes  [n x m]
    sizes[cnt++] = (size_t)n * 4;
    sizes[cnt++] = (size_t)k * m;      // X column codes   [k x m]
    sizes[cnt++] = (size_t)k * 4;
  }
  size_t o = 0;
  for (int i = 0; i < cnt; ++i) {
    p.off[i] = o;
    o += round256(sizes[i]);
  }
  if (backward) {
    p.scr_w = round256(fq_ws_bytes(n, k, HALO_ALONG_COLS, block, io));   // W columns along n
    p.scr_dy = round256(fq_ws_bytes(m, n, HALO_ALONG_COLS, block, io));  // dY columns along m
    p.scr_x = round256(fq_ws_bytes(m, k, HALO_ALONG_COLS, block, io));   // X columns along m
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

}  // namespace

extern "C" {

const char* halo_status_str(halo_status s) {
  switch (s) {
    case HALO_OK: return "ok";
    case HALO_ERR_NULL: return "a required pointer is NULL";
    case HALO_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case HALO_ERR_BLOCK: return "block must be a power of two in [1, 4096] dividing the rotated length";
    case HALO_ERR_DTYPE: return "unsupported element type";
    case HALO_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case HALO_ERR_WORKSPACE: return "workspace missing or too small";
    case HALO_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t halo_fwht_quant_workspace_bytes(int64_t rows, int64_t cols, halo_axis axis,
                                       int32_t block, halo_dtype x_type) {
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim || !valid_block(block))
    return 0;
  return fq_ws_bytes(rows, cols, axis, block, x_type);
}

halo_status halo_fwht_quant(const void* x, halo_dtype x_type, int64_t rows, int64_t cols,
                            int64_t ldx, halo_axis axis, int32_t block, halo_dtype q_type,
                            void* q, int64_t ldq, float* scale, void* ws, size_t ws_bytes,
                            void* stream) {
  halo_status s = check_fq(x, x_type, rows, cols, ldx, axis, block, q_type, q, ldq, scale);
  if (s != HALO_OK) return s;
  if (ws && !aligned16(ws)) return HALO_ERR_ALIGN;
  return run_fq(x, x_type, rows, cols, ldx, axis, block, q_type, q, ldq, scale, ws, ws_bytes,
                (hipStream_t)stream);
}

halo_status halo_gemm_i8(const int8_t* a, int64_t lda, const float* sa, const int8_t* b,
                         int64_t ldb, const float* sb, int64_t m, int64_t n, int64_t k, void* c,
                         halo_dtype c_type, int64_t ldc, void* stream) {
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
  if ((a_type != HALO_E4M3 && a_type != HALO_E5M2) || (b_type != HALO_E4M3 && b_type != HALO_E5M2))
    return HALO_ERR_DTYPE;
  if (c_type != HALO_F32 && c_type != HALO_BF16) return HALO_ERR_DTYPE;
  halo_status s = check_gemm(a, lda, b, ldb, m, n, k, c, c_type, ldc, sa, sb, 32);
  if (s != HALO_OK) return s;
  if (!aligned16(sa) || !aligned16(sb)) return HALO_ERR_ALIGN;
  return gemm_any(a, a_type, lda, sa, b, b_type, ldb, sb, m, n, k, c, c_type, ldc,
                  (hipStream_t)stream);
}

size_t halo_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, halo_dtype q_type,
                                   int backward) {
  if (m < 0 || n < 0 || k < 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return 0;
  if (q_type != HALO_I8 && q_type != HALO_E4M3) return 0;
  // the block and the input type decide the columns passes' scratch: size it for the most
  // demanding case (bf16 input, the block that needs the most partial maxima)
  size_t most = 0;
  for (int32_t b = 1; b <= 4096; b *= 2) {
    const size_t t = plan_ws(m, n, k, backward ? 1 : 0, b, HALO_BF16).total;
    if (t > most) most = t;
  }
  return most;
}

halo_status halo_linear_fwd(const void* x, const void* w, halo_dtype io_type, int64_t m,
                            int64_t n, int64_t k, int32_t block, halo_dtype q_type, void* y,
                            halo_dtype y_type, void* ws, size_t ws_bytes, void* stream) {
  if (m < 0 || n < 0 || k <= 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim)
    return HALO_ERR_SHAPE;
  if ((m > 0 && !x) || (n > 0 && !w) || (m > 0 && n > 0 && !y)) return HALO_ERR_NULL;
  if (io_type != HALO_F32 && io_type != HALO_BF16) return HALO_ERR_DTYPE;
  if (q_type != HALO_I8 && q_type != HALO_E4M3) return HALO_ERR_DTYPE;
  if (y_type != HALO_F32 && y_type != HALO_BF16) return HALO_ERR_DTYPE;
  if (k % 32 != 0) return HALO_ERR_SHAPE;
  if (!valid_block(block) || k % block != 0) return HALO_ERR_BLOCK;
  if (k > fq_rows_max_len(block)) return HALO_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return HALO_ERR_ALIGN;
  if ((n * esize(y_type)) % 16 != 0) return HALO_ERR_ALIGN;
  const WsPlan p = plan_ws(m, n, k, 0, block, io_type);
  if (!ws || ws_bytes < p.total) return HALO_ERR_WORKSPACE;
  if (!aligned16(ws)) return HALO_ERR_ALIGN;
  char* base = static_cast<char*>(ws);
  void* qx = base + p.off[0];
  float* sx = reinterpret_cast<float*>(base + p.off[1]);
  void* qw = base + p.off[2];
  float* sw = reinterpret_cast<float*>(base + p.off[3]);
  hipStream_t st = (hipStream_t)stream;
  halo_status s = HALO_OK;
  if (fq_rows2_supported(k, block)) {  // X and W rows in one launch
    FqPair pp{};
    pp.p0 = make_fq(x, m, k, k, HALO_ALONG_ROWS, block, q_type, qx, k, sx);
    pp.p1 = make_fq(w, n, k, k, HALO_ALONG_ROWS, block, q_type, qw, k, sw);
    pp.has1 = 1;
    s = from_hip(launch_fq_rows2_pair(pp, io_type == HALO_BF16 ? 1 : 0, qt_index(q_type), st));
  } else {
    s = run_fq(x, io_type, m, k, k, HALO_ALONG_ROWS, block, q_type, qx, k, sx, nullptr, 0, st);
    if (s == HALO_OK)
      s = run_fq(w, io_type, n, k, k, HALO_ALONG_ROWS, block, q_type, qw, k, sw, nullptr, 0, st);
  }
  if (s == HALO_OK) s = gemm_any(qx, q_type, k, sx, qw, q_type, k, sw, m, n, k, y, y_type, n, st);
  return s;
}

halo_status halo_linear_bwd(const void* dy, const void* x, const void* w, halo_dtype io_type,
                            int64_t m, int64_t n, int64_t k, int32_t block, halo_dtype q_type,
                            halo_dtype grad_q_type, void* dx, void* dw, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!dy || !x || !w) return HALO_ERR_NULL;
  if (io_type != HALO_F32 && io_type != HALO_BF16) return HALO_ERR_DTYPE;
  if (q_type == HALO_I8) {
    if (grad_q_type != HALO_I8) return HALO_ERR_DTYPE;
  } else if (q_type == HALO_E4M3) {
    if (grad_q_type != HALO_E5M2 && grad_q_type != HALO_E4M3) return HALO_ERR_DTYPE;
  } else {
    return HALO_ERR_DTYPE;
  }
  if (m <= 0 || n <= 0 || k <= 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim)
    return HALO_ERR_SHAPE;
  if (m % 32 != 0 || n % 32 != 0 || k % 32 != 0) return HALO_ERR_SHAPE;
  if (!valid_block(block) || m % block != 0 || n % block != 0) return HALO_ERR_BLOCK;
  if (dx && n > fq_rows_max_len(block)) return HALO_ERR_SHAPE;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(w)) return HALO_ERR_ALIGN;
  if ((dx && !aligned16(dx)) || (dw && !aligned16(dw))) return HALO_ERR_ALIGN;
  const WsPlan p = plan_ws(m, n, k, 1, block, io_type);
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
  // the single-read column passes need their scratch cleared: folded into the first kernel
  // when that is a rows pass, else one fill
  bool zero_pending = p.scratch_bytes > 0;
  auto clear_scratch = [&]() {
    if (!zero_pending || s != HALO_OK) return;
    s = from_hip(launch_fill_zero(reinterpret_cast<float*>(scr), (int64_t)(p.scratch_bytes / 4), st));
    zero_pending = false;
  };
  // one column pass along the rows of x (length `rows`): single-read when covered
  auto cols_pass = [&](const void* xx, int64_t rows, int64_t cols, halo_dtype qt, void* q,
                       float* sc, void* sws, size_t sbytes) {
    if (s != HALO_OK) return;
    if (fq_cols2_supported(rows, cols, block, inb, sbytes)) {
      const FqArgs a = make_fq(xx, rows, cols, cols, HALO_ALONG_COLS, block, qt, q, rows, sc);
      s = from_hip(launch_fq_cols2_pair(a, sws, nullptr, nullptr, qt_index(qt), 1, st));
    } else {
      s = run_fq(xx, io_type, rows, cols, cols, HALO_ALONG_COLS, block, qt, q, rows, sc, nullptr,
                 0, st);
    }
  };
  const int qg = qt_index(grad_q_type), qw = qt_index(q_type);
  const bool pair_ok = (qg == 0 && qw == 0) || (qg == 2 && qw == 1) || (qg == 1 && qw == 1);
  if (dx && dw && inb && pair_ok && fq_cols2_supported(n, k, block, 1, p.scr_w) &&
      fq_cols2_supported(m, n, block, 1, p.scr_dy) && fq_cols2_supported(m, k, block, 1, p.scr_x)) {
    // every rotation pass of the backward in one launch (or two, when the dY rows are long):
    // the passes overlap on the device, then the two products
    void* qdy = base + p.off[0];
    float* sdy = reinterpret_cast<float*>(base + p.off[1]);
    void* qwt = base + p.off[2];
    float* swt = reinterpret_cast<float*>(base + p.off[3]);
    void* qdyt = base + p.off[4];
    float* sdyt = reinterpret_cast<float*>(base + p.off[5]);
    void* qxt = base + p.off[6];
    float* sxt = reinterpret_cast<float*>(base + p.off[7]);
    const FqArgs rows = make_fq(dy, m, n, n, HALO_ALONG_ROWS, block, grad_q_type, qdy, n, sdy);
    const FqArgs cw = make_fq(w, n, k, k, HALO_ALONG_COLS, block, q_type, qwt, n, swt);
    const FqArgs cdy = make_fq(dy, m, n, n, HALO_ALONG_COLS, block, grad_q_type, qdyt, m, sdyt);
    const FqArgs cx = make_fq(x, m, k, k, HALO_ALONG_COLS, block, q_type, qxt, m, sxt);
    const bool rows_in = fq_batch_rows_ok(n);
    if (rows_in) {
      clear_scratch();
    } else if (fq_rows2_supported(n, block)) {
      FqPair pp{};
      pp.p0 = rows;
      if (zero_pending) {
        pp.zero = reinterpret_cast<uint32_t*>(scr);
        pp.nzero = (int64_t)(p.scratch_bytes / 4);
        zero_pending = false;
      }
      s = from_hip(launch_fq_rows2_pair(pp, inb, qg, st));
    } else {
      s = run_fq(dy, io_type, m, n, n, HALO_ALONG_ROWS, block, grad_q_type, qdy, n, sdy, nullptr,
                 0, st);
      clear_scratch();
    }
    if (s == HALO_OK)
      s = from_hip(launch_fq_batch(rows_in ? &rows : nullptr, cw, scr_w, cdy, scr_dy, cx, scr_x,
                                   qg, qw, st));
    if (s == HALO_OK)
      s = gemm_any(qdy, grad_q_type, n, sdy, qwt, q_type, n, swt, m, k, n, dx, io_type, k, st);
    if (s == HALO_OK)
      s = gemm_any(qdyt, grad_q_type, m, sdyt, qxt, q_type, m, sxt, n, k, m, dw, io_type, k, st);
    return s;
  }
  if (dx) {  // dX[m x k] = dY W: contraction over n
    void* qdy = base + p.off[0];
    float* sdy = reinterpret_cast<float*>(base + p.off[1]);
    void* qwt = base + p.off[2];
    float* swt = reinterpret_cast<float*>(base + p.off[3]);
    if (fq_rows2_supported(n, block)) {
      FqPair pp{};
      pp.p0 = make_fq(dy, m, n, n, HALO_ALONG_ROWS, block, grad_q_type, qdy, n, sdy);
      if (zero_pending) {
        pp.zero = reinterpret_cast<uint32_t*>(scr);
        pp.nzero = (int64_t)(p.scratch_bytes / 4);
        zero_pending = false;
      }
      s = from_hip(launch_fq_rows2_pair(pp, inb, qt_index(grad_q_type), st));
    } else {
      s = run_fq(dy, io_type, m, n, n, HALO_ALONG_ROWS, block, grad_q_type, qdy, n, sdy, nullptr,
                 0, st);
    }
    clear_scratch();
    cols_pass(w, n, k, q_type, qwt, swt, scr_w, p.scr_w);
    if (s == HALO_OK)
      s = gemm_any(qdy, grad_q_type, n, sdy, qwt, q_type, n, swt, m, k, n, dx, io_type, k, st);
  }
  if (s == HALO_OK && dw) {  // dW[n x k] = dY^T X: contraction over m
    void* qdyt = base + p.off[4];
    float* sdyt = reinterpret_cast<float*>(base + p.off[5]);
    void* qxt = base + p.off[6];
    float* sxt = reinterpret_cast<float*>(base + p.off[7]);
    clear_scratch();
    const bool c1 = fq_cols2_supported(m, n, block, inb, p.scr_dy);
    const bool c2 = fq_cols2_supported(m, k, block, inb, p.scr_x);
    if (s == HALO_OK && c1 && c2 && grad_q_type == q_type) {  // dY and X columns in one launch
      const FqArgs a0 = make_fq(dy, m, n, n, HALO_ALONG_COLS, block, grad_q_type, qdyt, m, sdyt);
      const FqArgs a1 = make_fq(x, m, k, k, HALO_ALONG_COLS, block, q_type, qxt, m, sxt);
      s = from_hip(launch_fq_cols2_pair(a0, scr_dy, &a1, scr_x, qt_index(q_type), 1, st));
    } else {
      cols_pass(dy, m, n, grad_q_type, qdyt, sdyt, scr_dy, p.scr_dy);
      cols_pass(x, m, k, q_type, qxt, sxt, scr_x, p.scr_x);
    }
    if (s == HALO_OK)
      s = gemm_any(qdyt, grad_q_type, m, sdyt, qxt, q_type, m, sxt, n, k, m, dw, io_type, k, st);
  }
  return s;
}

}  // extern "C"
