/*
 * CPU oracle for INT8 mixed-precision linear layers with row-wise scaling.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It is a plain, slow,
 * scalar statement of what the method computes, written so that a reader can
 * check it against the source pages by eye.  It shares no code, header or
 * constant table with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [QT]   "Quantized model training" (gau-nernst/quantized-training README),
 *          section "INT8 mixed precision training": INT8 means dynamic
 *          row-wise quantization followed by a scaled INT8 matmul; the table
 *          there lists three independently INT8-able GEMMs (forward,
 *          backward grad input, backward grad weight) and a stochastic
 *          rounding option.  Section "Speed benchmarks > Matmul" names the
 *          three operand layouts A @ B.T, A @ B and A.T @ B.
 *   [TT]   "Integrate INT8 mixed-precision from torchao 0.7" (torchtune PR
 *          #1552), gau-nernst's reply on memory: weights and activations are
 *          quantized dynamically to INT8 with scaling so an INT8 matmul can
 *          run, and the result is scaled back to BF16; weights and
 *          activations stay BF16 between calls.
 *   [QAT]  "Add QAT support for distributed finetuning" (torchtune PR #980),
 *          summary: quantization is a division by a scale followed by a clamp,
 *          dequantization a multiplication by the scale.
 *   Philox4x32-10: J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel Random
 *          Numbers: As Easy as 1, 2, 3", SC'11, section 3 (Philox).
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes): absmax statistic, divisor 127, fp32 scale = RN(amax/127), IEEE fp32
 * quotient x/s, round-half-even, clamp to [-127,127], zero point 0, an
 * all-zero row has scale 0 and codes 0, stochastic rounding is
 * floor(RN(v + u)) with u a 24-bit uniform from one Philox word, int32
 * accumulation checked in int64, epilogue ((float)acc * sa) * sb rounded to
 * bf16 half-even.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off (no FMA contraction, no
 * flush-to-zero), so every float operation below is one IEEE binary32
 * operation rounded to nearest even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_RNE = 0, OR_SR = 1 };
enum { OR_NT = 0, OR_NN = 1, OR_TN = 2 };

/* ---- bf16 <-> fp32 ------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a binary32 to bf16, nearest with ties to even (NaN never reaches
 * here: the inputs are finite and the epilogue of finite values is finite). */
static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xFFFFu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

/* ---- Philox4x32-10 (Salmon et al., SC'11, section 3) ---------------------- */

/* One Philox4x32 block with 10 rounds.  Each round multiplies words 0 and 2
 * by the two round multipliers, takes the 64-bit products apart, and
 * permutes/xors them with words 1 and 3 and the round key; the Weyl key
 * schedule adds the two bump constants between rounds. */
void oracle_philox4x32_10_block(const uint32_t ctr_in[4], const uint32_t key_in[2],
                                uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* Stream of blocks: block i uses counter (lo32(offset+i), hi32(offset+i), 0, 0)
 * and key (lo32(seed), hi32(seed)); out holds 4*n_blocks words. */
void oracle_philox_stream(uint64_t seed, uint64_t offset, int64_t n_blocks, uint32_t* out) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (int64_t i = 0; i < n_blocks; ++i) {
    uint64_t b = offset + (uint64_t)i;
    uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), 0u, 0u};
    oracle_philox4x32_10_block(ctr, key, out + 4 * i);
  }
}

/* The uniform u in [0, 1 - 2^-24] that stochastic rounding adds to element
 * number e (logical row-major index r*cols + c of the source tensor): word
 * e mod 4 of block offset + e/4, top 24 bits, times 2^-24 (exact in fp32). */
static float sr_uniform(uint64_t seed, uint64_t offset, uint64_t e) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint64_t b = offset + (e >> 2);
  uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), 0u, 0u};
  uint32_t w[4];
  oracle_philox4x32_10_block(ctr, key, w);
  uint32_t word = w[e & 3u];
  return (float)(word >> 8) * (1.0f / 16777216.0f);
}

/* ---- quantization ([QT] "INT8 mixed precision training"; [QAT] summary) -- */

/* Scale of one quantization group: s = RN(amax / 127) in binary32. */
static float scale_from_amax(float amax) { return amax / 127.0f; }

/* One int8 code for x under scale s.  s == 0 only for an all-zero group,
 * whose codes are 0. */
static int8_t quantize_one(float x, float s, int round_mode, float u) {
  if (s == 0.0f) return 0;
  float v = x / s; /* IEEE binary32 division */
  float r;
  if (round_mode == OR_SR) {
    float t = v + u;
    r = floorf(t);
  } else {
    r = rintf(v); /* default rounding mode: nearest, ties to even */
  }
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)(int)r;
}

/* The rounding step alone, with the uniforms supplied by the caller: code
 * i is quantize_one(x[i], s, mode, u[i]) (u may be NULL under RNE).  Lets a
 * test enumerate every possible 24-bit uniform for one value. */
void oracle_quantize_given_u(const uint16_t* x, int64_t n, float s, int round_mode,
                             const float* u, int8_t* q) {
  for (int64_t i = 0; i < n; ++i)
    q[i] = quantize_one(bf16_to_float(x[i]), s, round_mode, u ? u[i] : 0.0f);
}

/* Row-wise: one scale per row; the reduction runs over the columns, which
 * are the contraction dimension of a K-contiguous GEMM operand. */
void oracle_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             int8_t* q, int64_t ldq, float* scale, int round_mode,
                             uint64_t seed, uint64_t offset) {
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      float a = fabsf(bf16_to_float(x[r * ldx + c]));
      if (a > amax) amax = a;
    }
    float s = scale_from_amax(amax);
    scale[r] = s;
    for (int64_t c = 0; c < cols; ++c) {
      float u = 0.0f;
      if (round_mode == OR_SR) u = sr_uniform(seed, offset, (uint64_t)(r * cols + c));
      q[r * ldq + c] = quantize_one(bf16_to_float(x[r * ldx + c]), s, round_mode, u);
    }
  }
}

/* Column-wise: one scale per column; the reduction runs over the rows, which
 * are the contraction dimension when the tensor is used transposed (the
 * A @ B and A.T @ B layouts).  Codes stay in the source layout. */
void oracle_quantize_colwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             int8_t* q, int64_t ldq, float* scale, int round_mode,
                             uint64_t seed, uint64_t offset) {
  for (int64_t c = 0; c < cols; ++c) {
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r) {
      float a = fabsf(bf16_to_float(x[r * ldx + c]));
      if (a > amax) amax = a;
    }
    scale[c] = scale_from_amax(amax);
  }
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      float u = 0.0f;
      if (round_mode == OR_SR) u = sr_uniform(seed, offset, (uint64_t)(r * cols + c));
      q[r * ldq + c] = quantize_one(bf16_to_float(x[r * ldx + c]), scale[c], round_mode, u);
    }
  }
}

/* Column maxima alone: out[c] = max over rows of |x[r,c]| (0 when there are
 * no rows), the statistic behind the column-wise scales above
 * (scale[c] = RN(out[c] / 127)), returned by itself so that a row-wise pass
 * that also reports it can be checked. */
void oracle_col_absmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float* out) {
  for (int64_t c = 0; c < cols; ++c) {
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r) {
      float a = fabsf(bf16_to_float(x[r * ldx + c]));
      if (a > amax) amax = a;
    }
    out[c] = amax;
  }
}

/* ---- integer matmul in the three layouts ([QT] "Speed benchmarks") ------ */

/* Element (m,k) of the left operand and (k,n) of the right operand.
 *   NT (A @ B.T): A is M x K, B is N x K.
 *   NN (A @ B):   A is M x K, B is K x N.
 *   TN (A.T @ B): A is K x M, B is K x N.                                   */
static int64_t a_at(int layout, const int8_t* A, int64_t lda, int64_t m, int64_t k) {
  return layout == OR_TN ? A[k * lda + m] : A[m * lda + k];
}
static int64_t b_at(int layout, const int8_t* B, int64_t ldb, int64_t k, int64_t n) {
  return layout == OR_NT ? B[n * ldb + k] : B[k * ldb + n];
}

/* Exact dot product in int64.  Returns 0 and stores the value when it fits
 * int32, the accumulator width of the method; returns 1 otherwise. */
static int dot_i64(int layout, int64_t K, const int8_t* A, int64_t lda, const int8_t* B,
                   int64_t ldb, int64_t m, int64_t n, int32_t* out) {
  int64_t acc = 0;
  for (int64_t k = 0; k < K; ++k) acc += a_at(layout, A, lda, m, k) * b_at(layout, B, ldb, k, n);
  if (acc > INT32_MAX || acc < INT32_MIN) return 1;
  *out = (int32_t)acc;
  return 0;
}

/* Scale back to BF16 ([TT]): ((float)acc * sa) * sb, each product one
 * binary32 rounding, then bf16 half-even. */
static uint16_t epilogue(int32_t acc, float sa, float sb) {
  float y = (float)acc;
  y = y * sa;
  y = y * sb;
  return float_to_bf16_rne(y);
}

/* C[m,n] = sum_k A(m,k) B(k,n) as int32.  Returns the number of outputs
 * whose exact sum did not fit int32 (0 for K <= 133144). */
int64_t oracle_mm_i32(int layout, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                      const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc) {
  int64_t bad = 0;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int32_t v = 0;
      bad += dot_i64(layout, K, A, lda, B, ldb, m, n, &v);
      C[m * ldc + n] = v;
    }
  return bad;
}

/* Scaled INT8 matmul to bf16: sa is indexed by the output row m and sb by
 * the output column n in every layout. */
int64_t oracle_scaled_mm(int layout, int64_t M, int64_t N, int64_t K, const int8_t* A,
                         int64_t lda, const float* sa, const int8_t* B, int64_t ldb,
                         const float* sb, uint16_t* C, int64_t ldc) {
  int64_t bad = 0;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int32_t v = 0;
      bad += dot_i64(layout, K, A, lda, B, ldb, m, n, &v);
      C[m * ldc + n] = epilogue(v, sa[m], sb[n]);
    }
  return bad;
}

/* The same at a list of (m,n) output positions, for spot checks of outputs
 * too large to compute whole.  Writes the int32 sum and the bf16 result. */
int64_t oracle_scaled_mm_at(int layout, int64_t K, const int8_t* A, int64_t lda, const float* sa,
                            const int8_t* B, int64_t ldb, const float* sb, const int64_t* ms,
                            const int64_t* ns, int64_t count, int32_t* acc_out,
                            uint16_t* y_out) {
  int64_t bad = 0;
  for (int64_t i = 0; i < count; ++i) {
    int32_t v = 0;
    bad += dot_i64(layout, K, A, lda, B, ldb, ms[i], ns[i], &v);
    acc_out[i] = v;
    y_out[i] = epilogue(v, sa[ms[i]], sb[ns[i]]);
  }
  return bad;
}

/* ---- one linear layer's three GEMMs ([QT] "INT8 mixed precision training")
 *
 * forward      Y  = X @ W.T : X row-wise (over K), W row-wise (over K), NT
 * grad input   dX = dY @ W  : dY row-wise (over N), W column-wise (over N), NN
 * grad weight  dW = dY.T @ X: dY column-wise (over M), X column-wise (over M), TN
 *
 * Stochastic rounding draws from a separate Philox stream per quantized
 * tensor: pass j uses counter offset `offset + j * 2^40`, j = 0 X row-wise,
 * 1 W row-wise, 2 dY row-wise, 3 W column-wise, 4 dY column-wise,
 * 5 X column-wise.  All tensors are dense row-major (leading dim = cols).  */
static uint64_t pass_offset(uint64_t offset, int j) { return offset + ((uint64_t)j << 40); }

int64_t oracle_linear_fwd(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                          int64_t N, int64_t K, int round_mode, uint64_t seed,
                          uint64_t offset) {
  int8_t* qx = (int8_t*)malloc((size_t)(M * K));
  int8_t* qw = (int8_t*)malloc((size_t)(N * K));
  float* sx = (float*)malloc((size_t)M * sizeof(float));
  float* sw = (float*)malloc((size_t)N * sizeof(float));
  if (!qx || !qw || !sx || !sw) {
    free(qx), free(qw), free(sx), free(sw);
    return -1;
  }
  oracle_quantize_rowwise(X, M, K, K, qx, K, sx, round_mode, seed, pass_offset(offset, 0));
  oracle_quantize_rowwise(W, N, K, K, qw, K, sw, round_mode, seed, pass_offset(offset, 1));
  int64_t bad = oracle_scaled_mm(OR_NT, M, N, K, qx, K, sx, qw, K, sw, Y, N);
  free(qx), free(qw), free(sx), free(sw);
  return bad;
}

/* dX or dW may be NULL to skip that GEMM. */
int64_t oracle_linear_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                          uint16_t* dW, int64_t M, int64_t N, int64_t K, int round_mode,
                          uint64_t seed, uint64_t offset) {
  int64_t bad = 0;
  if (dX) {
    int8_t* qdy = (int8_t*)malloc((size_t)(M * N));
    int8_t* qw = (int8_t*)malloc((size_t)(N * K));
    float* sdy = (float*)malloc((size_t)M * sizeof(float));
    float* sw = (float*)malloc((size_t)K * sizeof(float));
    if (!qdy || !qw || !sdy || !sw) {
      free(qdy), free(qw), free(sdy), free(sw);
      return -1;
    }
    oracle_quantize_rowwise(dY, M, N, N, qdy, N, sdy, round_mode, seed, pass_offset(offset, 2));
    oracle_quantize_colwise(W, N, K, K, qw, K, sw, round_mode, seed, pass_offset(offset, 3));
    bad += oracle_scaled_mm(OR_NN, M, K, N, qdy, N, sdy, qw, K, sw, dX, K);
    free(qdy), free(qw), free(sdy), free(sw);
  }
  if (dW) {
    int8_t* qdy = (int8_t*)malloc((size_t)(M * N));
    int8_t* qx = (int8_t*)malloc((size_t)(M * K));
    float* sdy = (float*)malloc((size_t)N * sizeof(float));
    float* sx = (float*)malloc((size_t)K * sizeof(float));
    if (!qdy || !qx || !sdy || !sx) {
      free(qdy), free(qx), free(sdy), free(sx);
      return -1;
    }
    oracle_quantize_colwise(dY, M, N, N, qdy, N, sdy, round_mode, seed, pass_offset(offset, 4));
    oracle_quantize_colwise(X, M, K, K, qx, K, sx, round_mode, seed, pass_offset(offset, 5));
    bad += oracle_scaled_mm(OR_TN, N, K, M, qdy, N, sdy, qx, K, sx, dW, K);
    free(qdy), free(qx), free(sdy), free(sx);
  }
  return bad;
}

/* ---- row-wise FP8 (E4M3) variant -----------------------------------------
 *
 * The pages name FP8 training with row-wise scales beside INT8 ([FP8]
 * "Can FP8 GEMM be enabled via module hooks instead of module swapping?",
 * the maintainer's reply: float8 primitives with row-wise scales feeding
 * scaled matmuls; [QT] "Speed benchmarks > Matmul" times a Triton FP8
 * matmul in the same three layouts).  They fix no formula; the readings
 * here mirror the INT8 ones: OCP FP8 E4M3, the same absmax statistic with
 * divisor 448 (the largest finite E4M3 value), the IEEE quotient clamped to
 * [-448, 448] and rounded to the nearest E4M3 value with ties to the even
 * code, fp32 accumulation, and the INT8 epilogue.
 *
 * E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 fraction
 * bits, no infinities, S.1111.111 is NaN.  Exponent field e > 0:
 * (1 + f/8) * 2^(e-7); e = 0: f * 2^-9.  The largest finite value is
 * 1.75 * 2^8 = 448.  Every finite value is an integer multiple of 2^-9. */

/* The value of a finite code as an integer count of 2^-9 (exact). */
static int64_t e4m3_units(uint8_t c) {
  const int e = (c >> 3) & 15, f = c & 7;
  const int64_t mag = e == 0 ? f : (int64_t)(8 + f) << (e - 1);
  return (c & 0x80) ? -mag : mag;
}

float oracle_e4m3_to_float(uint8_t c) {
  if ((c & 0x7F) == 0x7F) return NAN;
  const float mag = ldexpf((float)e4m3_units(c & 0x7F), -9);
  return (c & 0x80) ? -mag : mag; /* 0x80 is -0 */
}

/* Nearest E4M3 value to a finite v, ties to the even code, |v| >= 448
 * saturating to +-448; the sign of v (also of a zero result) is kept.  The
 * non-negative finite codes 0..126 have increasing values, so a binary search
 * finds the largest code whose value does not exceed |v|; the answer is that
 * code or the next one, whichever value is nearer (the even code on a tie). */
uint8_t oracle_float_to_e4m3(float v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 126; /* value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (ldexp((double)e4m3_units((uint8_t)mid), -9) <= a)
      lo = mid;
    else
      hi = mid;
  }
  const double dlo = a - ldexp((double)e4m3_units((uint8_t)lo), -9);
  const double dhi = ldexp((double)e4m3_units((uint8_t)hi), -9) - a;
  const int best = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) == 0 ? lo : hi);
  return sign | (uint8_t)best;
}

static float fp8_scale_from_amax(float amax) { return amax / 448.0f; }

/* Code of x under scale s: 0 for an all-zero group or a zero x; else the
 * IEEE quotient, clamped, rounded to E4M3. */
static uint8_t fp8_quantize_one(float x, float s) {
  if (s == 0.0f || x == 0.0f) return 0;
  float v = x / s;
  if (v > 448.0f) v = 448.0f;
  if (v < -448.0f) v = -448.0f;
  return oracle_float_to_e4m3(v);
}

void oracle_quantize_rowwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* scale) {
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      float a = fabsf(bf16_to_float(x[r * ldx + c]));
      if (a > amax) amax = a;
    }
    const float s = fp8_scale_from_amax(amax);
    scale[r] = s;
    for (int64_t c = 0; c < cols; ++c) q[r * ldq + c] = fp8_quantize_one(bf16_to_float(x[r * ldx + c]), s);
  }
}

void oracle_quantize_colwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* scale) {
  for (int64_t c = 0; c < cols; ++c) {
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r) {
      float a = fabsf(bf16_to_float(x[r * ldx + c]));
      if (a > amax) amax = a;
    }
    scale[c] = fp8_scale_from_amax(amax);
  }
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) q[r * ldq + c] = fp8_quantize_one(bf16_to_float(x[r * ldx + c]), scale[c]);
}

static int64_t f8a_at(int layout, const uint8_t* A, int64_t lda, int64_t m, int64_t k) {
  return e4m3_units(layout == OR_TN ? A[k * lda + m] : A[m * lda + k]);
}
static int64_t f8b_at(int layout, const uint8_t* B, int64_t ldb, int64_t k, int64_t n) {
  return e4m3_units(layout == OR_NT ? B[n * ldb + k] : B[k * ldb + n]);
}

/* FP8 scaled matmul, same layouts as oracle_scaled_mm.  The dot product is
 * exact: each code is an integer count of 2^-9, so the sum is an integer
 * count of 2^-18 (|a*b| < 2^36 of those units, so any K < 2^27 fits int64).
 * It is then rounded once to binary32 (acc_out, if non-NULL), and the INT8
 * epilogue follows.  absdot_out (if non-NULL) gets sum_k |a_k * b_k| in
 * binary64 for error bounds of fp32 accumulation. */
void oracle_fp8_scaled_mm(int layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                          int64_t lda, const float* sa, const uint8_t* B, int64_t ldb,
                          const float* sb, uint16_t* C, int64_t ldc, float* acc_out,
                          double* absdot_out) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int64_t sum = 0, abs_sum = 0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t p = f8a_at(layout, A, lda, m, k) * f8b_at(layout, B, ldb, k, n);
        sum += p;
        abs_sum += p < 0 ? -p : p;
      }
      const float acc = ldexpf((float)sum, -18); /* int64 -> float rounds to nearest even */
      if (acc_out) acc_out[m * N + n] = acc;
      if (absdot_out) absdot_out[m * N + n] = ldexp((double)abs_sum, -18);
      float y = acc * sa[m];
      y = y * sb[n];
      C[m * ldc + n] = float_to_bf16_rne(y);
    }
}

/* The same at a list of (m, n) output positions (for outputs too large to
 * compute whole): bf16 result, fp32 accumulator and sum |a*b| per position. */
void oracle_fp8_scaled_mm_at(int layout, int64_t K, const uint8_t* A, int64_t lda, const float* sa,
                             const uint8_t* B, int64_t ldb, const float* sb, const int64_t* ms,
                             const int64_t* ns, int64_t count, uint16_t* y_out, float* acc_out,
                             double* absdot_out) {
  for (int64_t i = 0; i < count; ++i) {
    const int64_t m = ms[i], n = ns[i];
    int64_t sum = 0, abs_sum = 0;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t p = f8a_at(layout, A, lda, m, k) * f8b_at(layout, B, ldb, k, n);
      sum += p;
      abs_sum += p < 0 ? -p : p;
    }
    const float acc = ldexpf((float)sum, -18);
    acc_out[i] = acc;
    absdot_out[i] = ldexp((double)abs_sum, -18);
    float y = acc * sa[m];
    y = y * sb[n];
    y_out[i] = float_to_bf16_rne(y);
  }
}
