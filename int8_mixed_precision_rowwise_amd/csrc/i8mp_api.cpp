// C ABI of the INT8 mixed-precision linear-layer library (include/i8mp.h).
// Every argument is validated on the host before the first HIP call, so a
// rejected call launches nothing and writes nothing.
#include "../../include/i8mp.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "internal.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 40;  // rejects sizes whose products could overflow

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [begin, end) byte range of a rows x cols matrix with leading dim ld.
struct Range {
  uintptr_t b = 0, e = 0;
};

Range mat_range(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  Range r;
  if (!p || rows <= 0 || cols <= 0) return r;
  r.b = reinterpret_cast<uintptr_t>(p);
  r.e = r.b + (uintptr_t)(((rows - 1) * ld + cols) * elem);
  return r;
}

Range vec_range(const void* p, int64_t n, int64_t elem) { return mat_range(p, 1, n, n, elem); }

bool overlap(Range a, Range b) { return a.b < a.e && b.b < b.e && a.b < b.e && b.b < a.e; }

bool dims_ok(int64_t a, int64_t b = 0, int64_t c = 0) {
  return a >= 0 && b >= 0 && c >= 0 && a < kMaxDim && b < kMaxDim && c < kMaxDim;
}

// Input or output matrix of `elem`-byte elements read/written in 16-byte
// chunks: base 16-aligned, rows 16-aligned, ld >= cols.  A matrix with no
// elements may be NULL.
bool chunked_ok(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  if (rows == 0 || cols == 0) return ld >= 0 && ld < kMaxDim;
  return p && aligned(p, 16) && ld >= cols && ld < kMaxDim && (ld * elem) % 16 == 0;
}

// Output matrix written element by element: natural alignment, ld >= cols.
bool elementwise_ok(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  if (rows == 0 || cols == 0) return ld >= 0 && ld < kMaxDim;
  return p && aligned(p, (uintptr_t)elem) && ld >= cols && ld < kMaxDim;
}

bool vec_ok(const void* p, int64_t n) { return n == 0 || (p && aligned(p, 4)); }

// gfx950 check, cached per device: 0 unknown, 1 ok, 2 not gfx950.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];

i8mp_status device_check() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return I8MP_EDEVICE;
  }
  if (dev < kMaxDevices) {
    const int s = g_device_state[dev].load(std::memory_order_relaxed);
    if (s == 1) return I8MP_OK;
    if (s == 2) return I8MP_EDEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return I8MP_EDEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_device_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? I8MP_OK : I8MP_EDEVICE;
}

i8mp_status hip_status(hipError_t e) { return e == hipSuccess ? I8MP_OK : I8MP_EHIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Storage shapes of the GEMM operands for a layout.
void operand_shapes(int32_t layout, int64_t M, int64_t N, int64_t K, int64_t& ar, int64_t& ac,
                    int64_t& br, int64_t& bc) {
  if (layout == I8MP_NT) {
    ar = M, ac = K, br = N, bc = K;
  } else if (layout == I8MP_NN) {
    ar = M, ac = K, br = K, bc = N;
  } else {
    ar = K, ac = M, br = K, bc = N;
  }
}

i8mp_status validate_mm(int32_t layout, int64_t M, int64_t N, int64_t K, const int8_t* A,
                        int64_t lda, const int8_t* B, int64_t ldb, const void* C, int64_t ldc,
                        int64_t c_elem, const float* sa, const float* sb, bool scaled) {
  if (layout < 0 || layout > 2) return I8MP_EINVAL;
  if (!dims_ok(M, N, K)) return I8MP_EINVAL;
  if (K > I8MP_MAX_CONTRACTION) return I8MP_ERANGE;
  int64_t ar, ac, br, bc;
  operand_shapes(layout, M, N, K, ar, ac, br, bc);
  const bool out = M > 0 && N > 0;  // anything to compute
  if (!chunked_ok(out ? A : nullptr, out ? ar : 0, out ? ac : 0, lda, 1)) return I8MP_EINVAL;
  if (!chunked_ok(out ? B : nullptr, out ? br : 0, out ? bc : 0, ldb, 1)) return I8MP_EINVAL;
  if (!elementwise_ok(C, M, N, ldc, c_elem)) return I8MP_EINVAL;
  if (scaled && out && (!vec_ok(sa, M) || !vec_ok(sb, N))) return I8MP_EINVAL;
  if (!out) return I8MP_OK;
  const Range rc = mat_range(C, M, N, ldc, c_elem);
  if (overlap(rc, mat_range(A, ar, ac, lda, 1)) || overlap(rc, mat_range(B, br, bc, ldb, 1)))
    return I8MP_EINVAL;
  if (scaled && (overlap(rc, vec_range(sa, M, 4)) || overlap(rc, vec_range(sb, N, 4))))
    return I8MP_EINVAL;
  return I8MP_OK;
}

i8mp_status validate_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                           const int8_t* q, int64_t ldq, const float* scale, int64_t nscale,
                           int32_t round) {
  if (round != I8MP_RNE && round != I8MP_SR) return I8MP_EINVAL;
  if (!dims_ok(rows, cols)) return I8MP_EINVAL;
  if (!chunked_ok(x, rows, cols, ldx, 2)) return I8MP_EINVAL;
  if (!chunked_ok(q, rows, cols, ldq, 1)) return I8MP_EINVAL;
  if (!vec_ok(scale, nscale)) return I8MP_EINVAL;
  const Range rx = mat_range(x, rows, cols, ldx, 2), rq = mat_range(q, rows, cols, ldq, 1),
              rs = vec_range(scale, nscale, 4);
  if (overlap(rq, rx) || overlap(rs, rx) || overlap(rs, rq)) return I8MP_EINVAL;
  return I8MP_OK;
}

constexpr size_t kAlign = 256;
size_t up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }
int64_t pad16(int64_t n) { return (n + 15) / 16 * 16; }

// Workspace carving: regions in a fixed order, each 256-byte aligned.
struct Carver {
  char* base;
  size_t used = 0;
  void* take(size_t n) {
    void* p = base ? base + used : nullptr;
    used += up(n);
    return p;
  }
};

struct FwdWs {
  int8_t *qx, *qw;
  float *sx, *sw;
  void *part_x, *part_w;  // slab column maxima of the two row-wise passes
  void* split;            // int32 partial planes of a contraction-split GEMM (or null)
};
size_t carve_fwd(void* ws, int64_t M, int64_t N, int64_t K, FwdWs* out) {
  Carver c{static_cast<char*>(ws)};
  const int64_t kp = pad16(K);
  FwdWs w;
  w.qx = static_cast<int8_t*>(c.take((size_t)(M * kp)));
  w.qw = static_cast<int8_t*>(c.take((size_t)(N * kp)));
  w.sx = static_cast<float*>(c.take((size_t)M * 4));
  w.sw = static_cast<float*>(c.take((size_t)N * 4));
  // slab maxima of a row pass with column maxima, or (FP8 rows over 14336
  // elements) of the column-maxima pass
  w.part_x = c.take(std::max(i8mp::rowwise_colmax_workspace_bytes(M, K), i8mp::colwise_workspace_bytes(M, K)));
  w.part_w = c.take(std::max(i8mp::rowwise_colmax_workspace_bytes(N, K), i8mp::colwise_workspace_bytes(N, K)));
  const size_t split = i8mp::gemm_split_workspace_bytes(I8MP_NT, M, N, K, kp, kp);
  w.split = split ? c.take(split) : nullptr;
  if (out) *out = w;
  return c.used;
}

struct BwdWs {
  int8_t *qdy, *qw, *qx;
  float *sdy, *sw, *sx, *cdy;
  void* col;    // slab column maxima (column-wise passes, dY's row-wise pass)
  void* split;  // int32 partial planes of a contraction-split GEMM (or null)
};
size_t carve_bwd(void* ws, int64_t M, int64_t N, int64_t K, BwdWs* out) {
  Carver c{static_cast<char*>(ws)};
  const int64_t kp = pad16(K), np = pad16(N);
  BwdWs w;
  w.qdy = static_cast<int8_t*>(c.take((size_t)(M * np)));
  w.qw = static_cast<int8_t*>(c.take((size_t)(N * kp)));
  w.qx = static_cast<int8_t*>(c.take((size_t)(M * kp)));
  w.sdy = static_cast<float*>(c.take((size_t)(M > N ? M : N) * 4));
  w.sw = static_cast<float*>(c.take((size_t)K * 4));
  w.sx = static_cast<float*>(c.take((size_t)K * 4));
  w.cdy = static_cast<float*>(c.take((size_t)N * 4));
  size_t col = i8mp::colwise_workspace_bytes(N, K);
  for (size_t n : {i8mp::colwise_workspace_bytes(M, N), i8mp::colwise_workspace_bytes(M, K),
                   i8mp::rowwise_colmax_workspace_bytes(M, N)})
    if (n > col) col = n;
  w.col = c.take(col);
  size_t split = i8mp::gemm_split_workspace_bytes(I8MP_NN, M, K, N, np, kp);
  const size_t s2 = i8mp::gemm_split_workspace_bytes(I8MP_TN, N, K, M, np, kp);
  if (s2 > split) split = s2;
  w.split = split ? c.take(split) : nullptr;
  if (out) *out = w;
  return c.used;
}

uint64_t pass_offset(uint64_t offset, int j) { return offset + ((uint64_t)j << 40); }

}  // namespace

extern "C" {

const char* i8mp_status_str(i8mp_status s) {
  switch (s) {
    case I8MP_OK: return "ok";
    case I8MP_EINVAL: return "invalid argument (null, negative size, misaligned, ld too small or overlapping buffers)";
    case I8MP_ERANGE: return "contraction longer than 133144: int32 accumulation could overflow";
    case I8MP_EDEVICE: return "no current HIP device, or the device is not gfx950";
    case I8MP_EHIP: return "HIP reported an error at launch";
    case I8MP_EWORKSPACE: return "workspace missing, misaligned or too small";
    case I8MP_ESCRATCH: return "problem needs more scratch than the library's static device buffer holds";
  }
  return "unknown status";
}

int32_t i8mp_abi_version(void) { return 4; }

i8mp_status i8mp_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                  int8_t* q, int64_t ldq, float* scale, int32_t round,
                                  uint64_t seed, uint64_t offset, void* stream) {
  i8mp_status st = validate_quant(x, rows, cols, ldx, q, ldq, scale, rows, round);
  if (st != I8MP_OK) return st;
  if (rows == 0) return I8MP_OK;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_quantize_rowwise(x, rows, cols, ldx, q, ldq, scale, round, seed,
                                                  offset, as_stream(stream)));
}

size_t i8mp_quantize_colwise_workspace_bytes(int64_t rows, int64_t cols) {
  if (!dims_ok(rows, cols) || cols == 0) return 0;
  return up(i8mp::colwise_workspace_bytes(rows, cols));
}

i8mp_status i8mp_quantize_colwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                  int8_t* q, int64_t ldq, float* scale, int32_t round,
                                  uint64_t seed, uint64_t offset, void* ws, size_t ws_bytes,
                                  void* stream) {
  i8mp_status st = validate_quant(x, rows, cols, ldx, q, ldq, scale, cols, round);
  if (st != I8MP_OK) return st;
  if (cols == 0) return I8MP_OK;
  const size_t need = i8mp_quantize_colwise_workspace_bytes(rows, cols);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return I8MP_EWORKSPACE;
  const Range rw = vec_range(ws, (int64_t)need, 1);
  if (overlap(rw, mat_range(x, rows, cols, ldx, 2)) || overlap(rw, mat_range(q, rows, cols, ldq, 1)) ||
      overlap(rw, vec_range(scale, cols, 4)))
    return I8MP_EINVAL;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_quantize_colwise(x, rows, cols, ldx, q, ldq, scale, round, seed,
                                                  offset, ws, as_stream(stream)));
}

i8mp_status i8mp_quantize_colwise_noalloc(const uint16_t* x, int64_t rows, int64_t cols,
                                          int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                          int32_t round, uint64_t seed, uint64_t offset,
                                          void* stream) {
  static_assert(I8MP_STATIC_SCRATCH_BYTES == i8mp::kStaticScratchBytes, "one scratch size");
  i8mp_status st = validate_quant(x, rows, cols, ldx, q, ldq, scale, cols, round);
  if (st != I8MP_OK) return st;
  if (cols == 0) return I8MP_OK;
  if (i8mp_quantize_colwise_workspace_bytes(rows, cols) > I8MP_STATIC_SCRATCH_BYTES) return I8MP_ESCRATCH;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_quantize_colwise_static(x, rows, cols, ldx, q, ldq, scale, round, seed,
                                                         offset, as_stream(stream)));
}

size_t i8mp_quantize_rowwise_colmax_workspace_bytes(int64_t rows, int64_t cols) {
  if (!dims_ok(rows, cols) || cols == 0) return 0;
  return up(i8mp::rowwise_colmax_workspace_bytes(rows, cols));
}

i8mp_status i8mp_quantize_rowwise_colmax(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                         float* colmax, int32_t round, uint64_t seed,
                                         uint64_t offset, void* ws, size_t ws_bytes,
                                         void* stream) {
  i8mp_status st = validate_quant(x, rows, cols, ldx, q, ldq, scale, rows, round);
  if (st != I8MP_OK) return st;
  if (!vec_ok(colmax, cols)) return I8MP_EINVAL;
  const Range rx = mat_range(x, rows, cols, ldx, 2), rq = mat_range(q, rows, cols, ldq, 1),
              rs = vec_range(scale, rows, 4), rc = vec_range(colmax, cols, 4);
  if (overlap(rc, rx) || overlap(rc, rq) || overlap(rc, rs)) return I8MP_EINVAL;
  if (cols == 0) {
    if (rows == 0) return I8MP_OK;
    if ((st = device_check()) != I8MP_OK) return st;
    return hip_status(i8mp::launch_quantize_rowwise(x, rows, cols, ldx, q, ldq, scale, round, seed,
                                                    offset, as_stream(stream)));
  }
  const size_t need = i8mp_quantize_rowwise_colmax_workspace_bytes(rows, cols);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return I8MP_EWORKSPACE;
  const Range rw = vec_range(ws, (int64_t)need, 1);
  if (overlap(rw, rx) || overlap(rw, rq) || overlap(rw, rs) || overlap(rw, rc)) return I8MP_EINVAL;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_quantize_rowwise_colmax(x, rows, cols, ldx, q, ldq, scale, colmax,
                                                         round, seed, offset, ws, as_stream(stream)));
}

i8mp_status i8mp_quantize_colwise_given_colmax(const uint16_t* x, int64_t rows, int64_t cols,
                                               int64_t ldx, const float* colmax, int8_t* q,
                                               int64_t ldq, float* scale, int32_t round,
                                               uint64_t seed, uint64_t offset, void* stream) {
  i8mp_status st = validate_quant(x, rows, cols, ldx, q, ldq, scale, cols, round);
  if (st != I8MP_OK) return st;
  if (!vec_ok(colmax, cols)) return I8MP_EINVAL;
  const Range rc = vec_range(colmax, cols, 4);
  if (overlap(rc, mat_range(q, rows, cols, ldq, 1)) || overlap(rc, vec_range(scale, cols, 4)))
    return I8MP_EINVAL;
  if (cols == 0) return I8MP_OK;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_quantize_colwise_given(x, rows, cols, ldx, colmax, q, ldq, scale,
                                                        round, seed, offset, as_stream(stream)));
}

i8mp_status i8mp_int8_scaled_mm(int32_t layout, int64_t M, int64_t N, int64_t K,
                                const int8_t* A, int64_t lda, const float* scale_a,
                                const int8_t* B, int64_t ldb, const float* scale_b, uint16_t* C,
                                int64_t ldc, void* stream) {
  i8mp_status st = validate_mm(layout, M, N, K, A, lda, B, ldb, C, ldc, 2, scale_a, scale_b, true);
  if (st != I8MP_OK) return st;
  if (M == 0 || N == 0) return I8MP_OK;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_gemm(layout, M, N, K, A, lda, scale_a, B, ldb, scale_b, C,
                                      nullptr, ldc, as_stream(stream)));
}

i8mp_status i8mp_int8_mm_i32(int32_t layout, int64_t M, int64_t N, int64_t K, const int8_t* A,
                             int64_t lda, const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc,
                             void* stream) {
  i8mp_status st = validate_mm(layout, M, N, K, A, lda, B, ldb, C, ldc, 4, nullptr, nullptr, false);
  if (st != I8MP_OK) return st;
  if (M == 0 || N == 0) return I8MP_OK;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_gemm(layout, M, N, K, A, lda, nullptr, B, ldb, nullptr, nullptr,
                                      C, ldc, as_stream(stream)));
}

i8mp_status i8mp_philox4x32_10(uint64_t seed, uint64_t offset, int64_t n_blocks, uint32_t* out,
                               void* stream) {
  if (n_blocks < 0 || n_blocks >= kMaxDim) return I8MP_EINVAL;
  if (n_blocks == 0) return I8MP_OK;
  if (!out || !aligned(out, 16)) return I8MP_EINVAL;
  i8mp_status st = device_check();
  if (st != I8MP_OK) return st;
  return hip_status(i8mp::launch_philox(seed, offset, n_blocks, out, as_stream(stream)));
}

i8mp_status i8mp_mfma_rate_probe(const int8_t* codes, int64_t codes_bytes, int64_t rounds,
                                 int32_t* sink, void* stream) {
  if (!codes || !aligned(codes, 16) || codes_bytes < I8MP_MFMA_PROBE_MIN_BYTES || codes_bytes >= kMaxDim)
    return I8MP_EINVAL;
  if (rounds < 0 || rounds > (int64_t(1) << 24)) return I8MP_EINVAL;
  if (!sink || !aligned(sink, 4)) return I8MP_EINVAL;
  if (overlap(vec_range(codes, codes_bytes, 1), vec_range(sink, I8MP_MFMA_PROBE_SINK_INTS, 4))) return I8MP_EINVAL;
  static_assert(I8MP_MFMA_PROBE_SINK_INTS == i8mp::kMfmaProbeWorkgroups * 512, "one int32 per probe thread");
  i8mp_status st = device_check();
  if (st != I8MP_OK) return st;
  return hip_status(i8mp::launch_mfma_rate_probe(codes, codes_bytes, rounds, sink, as_stream(stream)));
}

size_t i8mp_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t backward) {
  if (!dims_ok(M, N, K)) return 0;
  return backward ? carve_bwd(nullptr, M, N, K, nullptr) : carve_fwd(nullptr, M, N, K, nullptr);
}

i8mp_status i8mp_linear_fwd_colmax(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                                   int64_t N, int64_t K, const i8mp_linear_opts* opts,
                                   float* colmax_x, float* colmax_w, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (!opts || (opts->round != I8MP_RNE && opts->round != I8MP_SR)) return I8MP_EINVAL;
  if (!dims_ok(M, N, K)) return I8MP_EINVAL;
  if (K > I8MP_MAX_CONTRACTION) return I8MP_ERANGE;
  if (!chunked_ok(X, M, K, K, 2) || !chunked_ok(W, N, K, K, 2) || !elementwise_ok(Y, M, N, N, 2))
    return I8MP_EINVAL;
  if ((colmax_x && !vec_ok(colmax_x, K)) || (colmax_w && !vec_ok(colmax_w, K))) return I8MP_EINVAL;
  const Range ry = mat_range(Y, M, N, N, 2), rx = mat_range(X, M, K, K, 2),
              rwt = mat_range(W, N, K, K, 2);
  const Range rcx = colmax_x ? vec_range(colmax_x, K, 4) : Range{},
              rcw = colmax_w ? vec_range(colmax_w, K, 4) : Range{};
  if (overlap(ry, rx) || overlap(ry, rwt)) return I8MP_EINVAL;
  for (Range o : {ry, rx, rwt})
    if (overlap(o, rcx) || overlap(o, rcw)) return I8MP_EINVAL;
  if (overlap(rcx, rcw)) return I8MP_EINVAL;
  if (M == 0 || N == 0) return I8MP_OK;
  const size_t need = carve_fwd(nullptr, M, N, K, nullptr);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return I8MP_EWORKSPACE;
  const Range rw = vec_range(ws, (int64_t)need, 1);
  for (Range o : {ry, rx, rwt, rcx, rcw})
    if (overlap(rw, o)) return I8MP_EINVAL;
  i8mp_status st = device_check();
  if (st != I8MP_OK) return st;
  FwdWs w;
  carve_fwd(ws, M, N, K, &w);
  const hipStream_t s = as_stream(stream);
  const int64_t kp = pad16(K);
  const int r = opts->round;
  hipError_t e = hipSuccess;
  i8mp::ColmaxJob side{};  // X's and W's slab maxima, reduced in the GEMM's prologue
  if (colmax_x && colmax_w) {  // both row-wise passes (same width K) in one launch
    e = i8mp::launch_quantize_rowwise_colmax_pair(X, M, K, w.qx, kp, w.sx, colmax_x, pass_offset(opts->offset, 0),
                                                  w.part_x, W, N, K, w.qw, kp, w.sw, colmax_w,
                                                  pass_offset(opts->offset, 1), w.part_w, K, r, opts->seed,
                                                  K == 0, 0, s);
    if (K > 0) {
      side.n = 2;
      side.cols = K;
      side.part[0] = static_cast<const uint16_t*>(w.part_x);
      side.part[1] = static_cast<const uint16_t*>(w.part_w);
      side.colmax[0] = colmax_x;
      side.colmax[1] = colmax_w;
      i8mp::rowwise_colmax_geometry(M, K, r, &side.slabs[0], &side.part_ld);
      i8mp::rowwise_colmax_geometry(N, K, r, &side.slabs[1], &side.part_ld);
    }
  } else {
    e = colmax_x ? i8mp::launch_quantize_rowwise_colmax(X, M, K, K, w.qx, kp, w.sx, colmax_x, r, opts->seed,
                                                        pass_offset(opts->offset, 0), w.part_x, s)
                 : i8mp::launch_quantize_rowwise(X, M, K, K, w.qx, kp, w.sx, r, opts->seed,
                                                 pass_offset(opts->offset, 0), s);
    if (e == hipSuccess)
      e = colmax_w ? i8mp::launch_quantize_rowwise_colmax(W, N, K, K, w.qw, kp, w.sw, colmax_w, r, opts->seed,
                                                          pass_offset(opts->offset, 1), w.part_w, s)
                   : i8mp::launch_quantize_rowwise(W, N, K, K, w.qw, kp, w.sw, r, opts->seed,
                                                   pass_offset(opts->offset, 1), s);
  }
  if (e == hipSuccess)
    e = i8mp::launch_gemm_split(I8MP_NT, M, N, K, w.qx, kp, w.sx, w.qw, kp, w.sw, Y, N, w.split,
                                side.n ? &side : nullptr, 0, s);
  return hip_status(e);
}

i8mp_status i8mp_linear_fwd(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                            int64_t N, int64_t K, const i8mp_linear_opts* opts, void* ws,
                            size_t ws_bytes, void* stream) {
  return i8mp_linear_fwd_colmax(X, W, Y, M, N, K, opts, nullptr, nullptr, ws, ws_bytes, stream);
}

i8mp_status i8mp_linear_bwd_colmax(const uint16_t* dY, const uint16_t* X, const uint16_t* W,
                                   uint16_t* dX, uint16_t* dW, int64_t M, int64_t N, int64_t K,
                                   const i8mp_linear_opts* opts, const float* colmax_x,
                                   const float* colmax_w, void* ws, size_t ws_bytes, void* stream) {
  if (!opts || (opts->round != I8MP_RNE && opts->round != I8MP_SR)) return I8MP_EINVAL;
  if (!dims_ok(M, N, K)) return I8MP_EINVAL;
  if (dX && N > I8MP_MAX_CONTRACTION) return I8MP_ERANGE;
  if (dW && M > I8MP_MAX_CONTRACTION) return I8MP_ERANGE;
  if (!chunked_ok(dY, M, N, N, 2)) return I8MP_EINVAL;
  if (dX && (!chunked_ok(W, N, K, K, 2) || !elementwise_ok(dX, M, K, K, 2))) return I8MP_EINVAL;
  if (dW && (!chunked_ok(X, M, K, K, 2) || !elementwise_ok(dW, N, K, K, 2))) return I8MP_EINVAL;
  if ((colmax_x && !vec_ok(colmax_x, K)) || (colmax_w && !vec_ok(colmax_w, K))) return I8MP_EINVAL;
  if (dX && dW && dX == dW && M * K > 0 && N * K > 0) return I8MP_EINVAL;
  const Range rdy = mat_range(dY, M, N, N, 2), rx = mat_range(X, M, K, K, 2),
              rwt = mat_range(W, N, K, K, 2), rdx = dX ? mat_range(dX, M, K, K, 2) : Range{},
              rdw = dW ? mat_range(dW, N, K, K, 2) : Range{};
  const Range rcx = colmax_x ? vec_range(colmax_x, K, 4) : Range{},
              rcw = colmax_w ? vec_range(colmax_w, K, 4) : Range{};
  for (Range o : {rdx, rdw})
    if (overlap(o, rdy) || overlap(o, rx) || overlap(o, rwt) || overlap(o, rcx) || overlap(o, rcw))
      return I8MP_EINVAL;
  if (overlap(rdx, rdw)) return I8MP_EINVAL;
  const bool want_dx = dX && M > 0 && K > 0, want_dw = dW && N > 0 && K > 0;
  if (!want_dx && !want_dw) return I8MP_OK;
  const size_t need = carve_bwd(nullptr, M, N, K, nullptr);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return I8MP_EWORKSPACE;
  const Range rw = vec_range(ws, (int64_t)need, 1);
  for (Range o : {rdy, rx, rwt, rdx, rdw, rcx, rcw})
    if (overlap(rw, o)) return I8MP_EINVAL;
  i8mp_status st = device_check();
  if (st != I8MP_OK) return st;
  BwdWs w;
  carve_bwd(ws, M, N, K, &w);
  const hipStream_t s = as_stream(stream);
  const int64_t kp = pad16(K), np = pad16(N);
  const int r = opts->round;
  const uint64_t seed = opts->seed;
  // dY's column maxima come from its row-wise pass when both GEMMs run
  const bool dy_colmax = want_dx && want_dw;
  hipError_t e = hipSuccess;
  i8mp::ColmaxJob side{};  // dY's slab maxima, reduced in the grad-input GEMM's prologue
  if (want_dx) {
    // dX = dY @ W: dY row-wise over N, W column-wise over N, NN
    if (dy_colmax && colmax_w) {
      // dY's row pass leaves its slab maxima in w.col; the grad-input GEMM
      // reduces them to dY's column maxima (needed by dY's column pass, after
      // it).  W's column pass rides in the same launch.
      e = i8mp::launch_quantize_rowslabs_colgiven(dY, M, N, N, w.qdy, np, w.sdy, pass_offset(opts->offset, 2), w.col,
                                                  W, N, K, K, colmax_w, w.qw, kp, w.sw, pass_offset(opts->offset, 3),
                                                  r, seed, 0, s);
      side.n = 1;
      side.cols = N;
      side.part[0] = static_cast<const uint16_t*>(w.col);
      side.colmax[0] = w.cdy;
      i8mp::rowwise_colmax_geometry(M, N, r, &side.slabs[0], &side.part_ld);
    } else {
      e = dy_colmax ? i8mp::launch_quantize_rowwise_colmax(dY, M, N, N, w.qdy, np, w.sdy, w.cdy, r, seed,
                                                           pass_offset(opts->offset, 2), w.col, s)
                    : i8mp::launch_quantize_rowwise(dY, M, N, N, w.qdy, np, w.sdy, r, seed,
                                                    pass_offset(opts->offset, 2), s);
      if (e == hipSuccess)
        e = colmax_w ? i8mp::launch_quantize_colwise_given(W, N, K, K, colmax_w, w.qw, kp, w.sw, r, seed,
                                                           pass_offset(opts->offset, 3), s)
                     : i8mp::launch_quantize_colwise(W, N, K, K, w.qw, kp, w.sw, r, seed,
                                                     pass_offset(opts->offset, 3), w.col, s);
    }
    if (e == hipSuccess)
      e = i8mp::launch_gemm_split(I8MP_NN, M, K, N, w.qdy, np, w.sdy, w.qw, kp, w.sw, dX, K, w.split,
                                  side.n ? &side : nullptr, 0, s);
  }
  if (want_dw && e == hipSuccess) {
    // dW = dY.T @ X: dY column-wise over M, X column-wise over M, TN
    if (dy_colmax && colmax_x) {  // both column-wise passes in one launch
      e = i8mp::launch_quantize_colwise_given_pair(dY, M, N, N, w.cdy, w.qdy, np, w.sdy, pass_offset(opts->offset, 4),
                                                   X, M, K, K, colmax_x, w.qx, kp, w.sx, pass_offset(opts->offset, 5),
                                                   r, seed, 0, s);
    } else {
      e = dy_colmax ? i8mp::launch_quantize_colwise_given(dY, M, N, N, w.cdy, w.qdy, np, w.sdy, r, seed,
                                                          pass_offset(opts->offset, 4), s)
                    : i8mp::launch_quantize_colwise(dY, M, N, N, w.qdy, np, w.sdy, r, seed,
                                                    pass_offset(opts->offset, 4), w.col, s);
      if (e == hipSuccess)
        e = colmax_x ? i8mp::launch_quantize_colwise_given(X, M, K, K, colmax_x, w.qx, kp, w.sx, r, seed,
                                                           pass_offset(opts->offset, 5), s)
                     : i8mp::launch_quantize_colwise(X, M, K, K, w.qx, kp, w.sx, r, seed,
                                                     pass_offset(opts->offset, 5), w.col, s);
    }
    if (e == hipSuccess)
      e = i8mp::launch_gemm_split(I8MP_TN, N, K, M, w.qdy, np, w.sdy, w.qx, kp, w.sx, dW, K, w.split, nullptr, 0, s);
  }
  return hip_status(e);
}

i8mp_status i8mp_linear_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                            uint16_t* dW, int64_t M, int64_t N, int64_t K,
                            const i8mp_linear_opts* opts, void* ws, size_t ws_bytes,
                            void* stream) {
  return i8mp_linear_bwd_colmax(dY, X, W, dX, dW, M, N, K, opts, nullptr, nullptr, ws, ws_bytes,
                                stream);
}

// ---- FP8 (E4M3) variant -------------------------------------------------

i8mp_status i8mp_quantize_rowwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* scale, void* stream) {
  const int8_t* q8 = reinterpret_cast<const int8_t*>(q);
  i8mp_status st = validate_quant(x, rows, cols, ldx, q8, ldq, scale, rows, I8MP_RNE);
  if (st != I8MP_OK) return st;
  if (rows == 0) return I8MP_OK;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_quantize_rowwise_fp8(x, rows, cols, ldx, q, ldq, scale, as_stream(stream)));
}

i8mp_status i8mp_quantize_colwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* scale, void* ws,
                                      size_t ws_bytes, void* stream) {
  const int8_t* q8 = reinterpret_cast<const int8_t*>(q);
  i8mp_status st = validate_quant(x, rows, cols, ldx, q8, ldq, scale, cols, I8MP_RNE);
  if (st != I8MP_OK) return st;
  if (cols == 0) return I8MP_OK;
  const size_t need = i8mp_quantize_colwise_workspace_bytes(rows, cols);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return I8MP_EWORKSPACE;
  const Range rw = vec_range(ws, (int64_t)need, 1);
  if (overlap(rw, mat_range(x, rows, cols, ldx, 2)) || overlap(rw, mat_range(q, rows, cols, ldq, 1)) ||
      overlap(rw, vec_range(scale, cols, 4)))
    return I8MP_EINVAL;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_quantize_colwise_fp8(x, rows, cols, ldx, q, ldq, scale, ws,
                                                      as_stream(stream)));
}

// FP8 GEMM shape rules (one kernel, the pipelined one): K a multiple of 16,
// output extents along operands whose contraction runs down their rows (M
// for TN, N for NN and TN) multiples of 4.

i8mp_status i8mp_fp8_scaled_mm(int32_t layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                               int64_t lda, const float* scale_a, const uint8_t* B, int64_t ldb,
                               const float* scale_b, uint16_t* C, int64_t ldc, void* stream) {
  i8mp_status st = validate_mm(layout, M, N, K, reinterpret_cast<const int8_t*>(A), lda,
                               reinterpret_cast<const int8_t*>(B), ldb, C, ldc, 2, scale_a, scale_b,
                               true);
  if (st == I8MP_ERANGE) st = I8MP_OK;  // fp32 accumulation: no integer bound
  if (st != I8MP_OK) return st;
  if (M == 0 || N == 0) return I8MP_OK;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_gemm_fp8(layout, M, N, K, A, lda, scale_a, B, ldb, scale_b, C, nullptr,
                                          ldc, as_stream(stream)));
}

i8mp_status i8mp_fp8_mm_f32(int32_t layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                            int64_t lda, const uint8_t* B, int64_t ldb, float* C, int64_t ldc,
                            void* stream) {
  i8mp_status st = validate_mm(layout, M, N, K, reinterpret_cast<const int8_t*>(A), lda,
                               reinterpret_cast<const int8_t*>(B), ldb, C, ldc, 4, nullptr, nullptr,
                               false);
  if (st == I8MP_ERANGE) st = I8MP_OK;
  if (st != I8MP_OK) return st;
  if (M == 0 || N == 0) return I8MP_OK;
  if ((st = device_check()) != I8MP_OK) return st;
  return hip_status(i8mp::launch_gemm_fp8(layout, M, N, K, A, lda, nullptr, B, ldb, nullptr, nullptr,
                                          C, ldc, as_stream(stream)));
}

i8mp_status i8mp_linear_fwd_fp8_colmax(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                                       int64_t N, int64_t K, float* colmax_x, float* colmax_w, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (!dims_ok(M, N, K)) return I8MP_EINVAL;
  if (!chunked_ok(X, M, K, K, 2) || !chunked_ok(W, N, K, K, 2) || !elementwise_ok(Y, M, N, N, 2))
    return I8MP_EINVAL;
  if ((colmax_x && !vec_ok(colmax_x, K)) || (colmax_w && !vec_ok(colmax_w, K))) return I8MP_EINVAL;
  const Range ry = mat_range(Y, M, N, N, 2), rx = mat_range(X, M, K, K, 2),
              rwt = mat_range(W, N, K, K, 2);
  const Range rcx = colmax_x ? vec_range(colmax_x, K, 4) : Range{},
              rcw = colmax_w ? vec_range(colmax_w, K, 4) : Range{};
  if (overlap(ry, rx) || overlap(ry, rwt)) return I8MP_EINVAL;
  for (Range o : {ry, rx, rwt})
    if (overlap(o, rcx) || overlap(o, rcw)) return I8MP_EINVAL;
  if (overlap(rcx, rcw)) return I8MP_EINVAL;
  if (M == 0 || N == 0) return I8MP_OK;
  const size_t need = carve_fwd(nullptr, M, N, K, nullptr);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return I8MP_EWORKSPACE;
  const Range rw = vec_range(ws, (int64_t)need, 1);
  for (Range o : {ry, rx, rwt, rcx, rcw})
    if (overlap(rw, o)) return I8MP_EINVAL;
  i8mp_status st = device_check();
  if (st != I8MP_OK) return st;
  FwdWs w;
  carve_fwd(ws, M, N, K, &w);
  const hipStream_t s = as_stream(stream);
  const int64_t kp = pad16(K);
  uint8_t* qx = reinterpret_cast<uint8_t*>(w.qx);
  uint8_t* qw = reinterpret_cast<uint8_t*>(w.qw);
  const bool fused = K > 0 && i8mp::rowwise_colmax_fp8_fused(M, K);  // rows of K <= 14336 elements
  hipError_t e = hipSuccess;
  i8mp::ColmaxJob side{};  // X's and W's slab maxima, folded by the GEMM
  if (colmax_x && colmax_w && fused) {  // both row-wise passes (same width K) in one launch
    e = i8mp::launch_quantize_rowwise_colmax_pair(X, M, K, w.qx, kp, w.sx, colmax_x, 0, w.part_x, W, N, K, w.qw, kp,
                                                  w.sw, colmax_w, 0, w.part_w, K, I8MP_RNE, 0, false, 1, s);
    side.n = 2;
    side.cols = K;
    side.part[0] = static_cast<const uint16_t*>(w.part_x);
    side.part[1] = static_cast<const uint16_t*>(w.part_w);
    side.colmax[0] = colmax_x;
    side.colmax[1] = colmax_w;
    i8mp::rowwise_colmax_geometry(M, K, 0, &side.slabs[0], &side.part_ld);
    i8mp::rowwise_colmax_geometry(N, K, 0, &side.slabs[1], &side.part_ld);
  } else {
    const uint16_t* src[2] = {X, W};
    const int64_t rows[2] = {M, N};
    uint8_t* q[2] = {qx, qw};
    float* sc[2] = {w.sx, w.sw};
    float* cm[2] = {colmax_x, colmax_w};
    void* part[2] = {w.part_x, w.part_w};
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
      if (cm[i] && fused) {
        e = i8mp::launch_quantize_rowwise_colmax_fp8(src[i], rows[i], K, K, q[i], kp, sc[i], cm[i], part[i], true, s);
      } else {
        e = i8mp::launch_quantize_rowwise_fp8(src[i], rows[i], K, K, q[i], kp, sc[i], s);
        if (e == hipSuccess && cm[i]) e = i8mp::launch_column_maxima(src[i], rows[i], K, K, cm[i], part[i], s);
      }
    }
  }
  if (e == hipSuccess)
    e = i8mp::launch_gemm_split(I8MP_NT, M, N, K, w.qx, kp, w.sx, w.qw, kp, w.sw, Y, N, w.split,
                                side.n ? &side : nullptr, 1, s);
  return hip_status(e);
}

i8mp_status i8mp_linear_fwd_fp8(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                                int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream) {
  return i8mp_linear_fwd_fp8_colmax(X, W, Y, M, N, K, nullptr, nullptr, ws, ws_bytes, stream);
}

i8mp_status i8mp_linear_bwd_fp8_colmax(const uint16_t* dY, const uint16_t* X, const uint16_t* W,
                                       uint16_t* dX, uint16_t* dW, int64_t M, int64_t N, int64_t K,
                                       const float* colmax_x, const float* colmax_w, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (!dims_ok(M, N, K)) return I8MP_EINVAL;
  if (!chunked_ok(dY, M, N, N, 2)) return I8MP_EINVAL;
  if (dX && (!chunked_ok(W, N, K, K, 2) || !elementwise_ok(dX, M, K, K, 2))) return I8MP_EINVAL;
  if (dW && (!chunked_ok(X, M, K, K, 2) || !elementwise_ok(dW, N, K, K, 2))) return I8MP_EINVAL;
  if ((colmax_x && !vec_ok(colmax_x, K)) || (colmax_w && !vec_ok(colmax_w, K))) return I8MP_EINVAL;
  if (dX && dW && dX == dW && M * K > 0 && N * K > 0) return I8MP_EINVAL;
  const Range rdy = mat_range(dY, M, N, N, 2), rx = mat_range(X, M, K, K, 2),
              rwt = mat_range(W, N, K, K, 2), rdx = dX ? mat_range(dX, M, K, K, 2) : Range{},
              rdw = dW ? mat_range(dW, N, K, K, 2) : Range{};
  const Range rcx = colmax_x ? vec_range(colmax_x, K, 4) : Range{},
              rcw = colmax_w ? vec_range(colmax_w, K, 4) : Range{};
  for (Range o : {rdx, rdw})
    if (overlap(o, rdy) || overlap(o, rx) || overlap(o, rwt) || overlap(o, rcx) || overlap(o, rcw))
      return I8MP_EINVAL;
  if (overlap(rdx, rdw)) return I8MP_EINVAL;
  const bool want_dx = dX && M > 0 && K > 0, want_dw = dW && N > 0 && K > 0;
  if (!want_dx && !want_dw) return I8MP_OK;
  const size_t need = carve_bwd(nullptr, M, N, K, nullptr);
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return I8MP_EWORKSPACE;
  const Range rw = vec_range(ws, (int64_t)need, 1);
  for (Range o : {rdy, rx, rwt, rdx, rdw, rcx, rcw})
    if (overlap(rw, o)) return I8MP_EINVAL;
  i8mp_status st = device_check();
  if (st != I8MP_OK) return st;
  BwdWs w;
  carve_bwd(ws, M, N, K, &w);
  const hipStream_t s = as_stream(stream);
  const int64_t kp = pad16(K), np = pad16(N);
  uint8_t* qdy = reinterpret_cast<uint8_t*>(w.qdy);
  uint8_t* qw = reinterpret_cast<uint8_t*>(w.qw);
  uint8_t* qx = reinterpret_cast<uint8_t*>(w.qx);
  hipError_t e = hipSuccess;
  // with both gradients, dY's column maxima come from its row-wise pass
  // (rows of at most 14336 elements), so its column-wise pass reads it once
  const bool dy_colmax = want_dx && want_dw && i8mp::rowwise_colmax_fp8_fused(M, N);
  i8mp::ColmaxJob side{};  // dY's slab maxima, folded by the grad-input GEMM
  if (want_dx) {
    // dX = dY @ W: dY row-wise over N, W column-wise over N, NN
    if (dy_colmax && colmax_w) {  // dY's row pass and W's column pass in one launch
      e = i8mp::launch_quantize_rowslabs_colgiven(dY, M, N, N, w.qdy, np, w.sdy, 0, w.col, W, N, K, K, colmax_w, w.qw,
                                                  kp, w.sw, 0, I8MP_RNE, 0, 1, s);
      side.n = 1;
      side.cols = N;
      side.part[0] = static_cast<const uint16_t*>(w.col);
      side.colmax[0] = w.cdy;
      i8mp::rowwise_colmax_geometry(M, N, 0, &side.slabs[0], &side.part_ld);
    } else {
      e = dy_colmax ? i8mp::launch_quantize_rowwise_colmax_fp8(dY, M, N, N, qdy, np, w.sdy, w.cdy, w.col, true, s)
                    : i8mp::launch_quantize_rowwise_fp8(dY, M, N, N, qdy, np, w.sdy, s);
      if (e == hipSuccess)
        e = colmax_w ? i8mp::launch_quantize_colwise_given_fp8(W, N, K, K, colmax_w, qw, kp, w.sw, s)
                     : i8mp::launch_quantize_colwise_fp8(W, N, K, K, qw, kp, w.sw, w.col, s);
    }
    if (e == hipSuccess)
      e = i8mp::launch_gemm_split(I8MP_NN, M, K, N, w.qdy, np, w.sdy, w.qw, kp, w.sw, dX, K, w.split,
                                  side.n ? &side : nullptr, 1, s);
  }
  if (want_dw && e == hipSuccess) {
    // dW = dY.T @ X: dY column-wise over M, X column-wise over M, TN
    if (dy_colmax && colmax_x) {  // both column-wise passes in one launch
      e = i8mp::launch_quantize_colwise_given_pair(dY, M, N, N, w.cdy, w.qdy, np, w.sdy, 0, X, M, K, K, colmax_x,
                                                   w.qx, kp, w.sx, 0, I8MP_RNE, 0, 1, s);
    } else {
      e = dy_colmax ? i8mp::launch_quantize_colwise_given_fp8(dY, M, N, N, w.cdy, qdy, np, w.sdy, s)
                    : i8mp::launch_quantize_colwise_fp8(dY, M, N, N, qdy, np, w.sdy, w.col, s);
      if (e == hipSuccess)
        e = colmax_x ? i8mp::launch_quantize_colwise_given_fp8(X, M, K, K, colmax_x, qx, kp, w.sx, s)
                     : i8mp::launch_quantize_colwise_fp8(X, M, K, K, qx, kp, w.sx, w.col, s);
    }
    if (e == hipSuccess)
      e = i8mp::launch_gemm_split(I8MP_TN, N, K, M, w.qdy, np, w.sdy, w.qx, kp, w.sx, dW, K, w.split, nullptr, 1, s);
  }
  return hip_status(e);
}

i8mp_status i8mp_linear_bwd_fp8(const uint16_t* dY, const uint16_t* X, const uint16_t* W,
                                uint16_t* dX, uint16_t* dW, int64_t M, int64_t N, int64_t K,
                                void* ws, size_t ws_bytes, void* stream) {
  return i8mp_linear_bwd_fp8_colmax(dY, X, W, dX, dW, M, N, K, nullptr, nullptr, ws, ws_bytes, stream);
}

}  // extern "C"
