/*
 * i8mp.h: INT8 mixed-precision linear layers with row-wise scaling, for AMD
 * MI355X (gfx950).  C ABI.
 *
 * What the library computes ("Quantized model training", section "INT8 mixed
 * precision training"; "Integrate INT8 mixed-precision from torchao 0.7",
 * gau-nernst's reply on memory): every GEMM of a linear layer's training
 * step quantizes both bf16 operands dynamically to int8, with one fp32 scale
 * per row of the contraction dimension, multiplies the codes with int32
 * accumulation, and scales the result back to bf16.  Weights, activations and
 * gradients stay bf16 between calls; nothing is cached.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains memory.  Scratch space comes in
 *     through the `ws` argument of the calls that need it (the one
 *     exception, i8mp_quantize_colwise_noalloc, uses a static device buffer
 *     of the library's own).
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the null stream).  Buffers must stay valid until the stream
 *     work completes.
 *   - bf16 travels as uint16_t bit patterns.  Matrices are row-major with a
 *     leading dimension `ld*` counted in elements.
 *   - Every argument is validated on the host before any HIP call; a call
 *     that fails validation launches nothing and writes nothing.
 *   - Alignment: base pointers of bf16/int8/int32 matrices are 16-byte
 *     aligned and ld * element size is a multiple of 16 bytes; scale vectors
 *     are 4-byte aligned.  Any sizes >= 0 are accepted (up to the stated
 *     contraction bound of the INT8 GEMMs).  Reads of an input
 *     may touch bytes between the end of a row and the next 16-byte boundary
 *     (never outside that aligned 16-byte chunk); outputs are written only
 *     inside their rows.
 *   - Outputs must not overlap inputs.
 *   - The library is stateless and reentrant, except that calls of
 *     i8mp_quantize_colwise_noalloc on one GPU share that GPU's static
 *     scratch.  The device check (gfx950) is cached per device.
 */
#ifndef I8MP_H
#define I8MP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  I8MP_OK = 0,
  I8MP_EINVAL = 1,     /* null pointer, negative size, misalignment, ld too small, overlap */
  I8MP_ERANGE = 2,     /* contraction longer than I8MP_MAX_CONTRACTION (int32 could overflow) */
  I8MP_EDEVICE = 3,    /* no current HIP device, or it is not gfx950 */
  I8MP_EHIP = 4,       /* a HIP launch reported an error */
  I8MP_EWORKSPACE = 5, /* workspace NULL or smaller than the query function returns */
  I8MP_ESCRATCH = 6,   /* the problem needs more scratch than I8MP_STATIC_SCRATCH_BYTES */
} i8mp_status;

/* Rounding of the quantization step.  RNE: round half to even.  SR:
 * stochastic rounding, code = floor(RN32(x/s + u)) with u a 24-bit uniform
 * from Philox4x32-10 ("Quantized model training", section "INT8 mixed
 * precision training": stochastic rounding is an option of each INT8 GEMM's
 * quantization; the pages leave the mechanism open). */
typedef enum { I8MP_RNE = 0, I8MP_SR = 1 } i8mp_round;

/* Operand layouts ("Quantized model training", section "Speed benchmarks >
 * Matmul"): NT = A @ B.T (A is M x K, B is N x K), NN = A @ B (A is M x K,
 * B is K x N), TN = A.T @ B (A is K x M, B is K x N).  C is M x N. */
typedef enum { I8MP_NT = 0, I8MP_NN = 1, I8MP_TN = 2 } i8mp_layout;

/* floor((2^31 - 1) / 127^2): the longest contraction whose int32 sum of
 * int8 x int8 products (|code| <= 127) cannot overflow. */
#define I8MP_MAX_CONTRACTION 133144

/* Stochastic-rounding stream of one linear-layer call.  Quantization pass j
 * of the call uses Philox counter offset `offset + j * 2^40`:
 * j = 0 X row-wise, 1 W row-wise, 2 dY row-wise, 3 W column-wise,
 * 4 dY column-wise, 5 X column-wise.  Callers advance `offset` (or `seed`)
 * between steps.  Ignored under RNE. */
typedef struct {
  int32_t round; /* i8mp_round */
  uint64_t seed;
  uint64_t offset;
} i8mp_linear_opts;

/* A fixed, human-readable description of a status code (never NULL; the
 * string lives as long as the library).  The codes are this library's own
 * error reporting; the pages report errors as Python exceptions
 * ("Integrate INT8 mixed-precision from torchao 0.7", the device guard and
 * the checks the recipe runs before training). */
const char* i8mp_status_str(i8mp_status s);

/* Version of this ABI (incremented on any signature change).  Bindings
 * compare it with the version they were written for. */
int32_t i8mp_abi_version(void);

/*
 * Row-wise dynamic quantization ("Quantized model training", section "INT8
 * mixed precision training"; the quantize step of "Add QAT support for
 * distributed finetuning", summary, with zero point 0):
 *   amax[r]  = max_c |x[r,c]|                 (exact)
 *   scale[r] = RN32(amax[r] / 127)            (0 for an all-zero row)
 *   q[r,c]   = clamp(round(RN32(x[r,c] / scale[r])), -127, 127), 0 if scale 0
 * round = RNE: half to even.  round = SR: floor(RN32(x/s + u)),
 * u = (w >> 8) * 2^-24 where w is word (e mod 4) of Philox4x32-10 block
 * (offset + e/4), e = r*cols + c (the logical index, independent of ld),
 * counter = (lo32(block), hi32(block), 0, 0), key = (lo32(seed), hi32(seed)).
 *   x:     bf16 [rows x cols], leading dim ldx >= cols
 *   q:     int8 [rows x cols], leading dim ldq >= cols (same layout as x)
 *   scale: fp32 [rows]
 */
i8mp_status i8mp_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                  int8_t* q, int64_t ldq, float* scale, int32_t round,
                                  uint64_t seed, uint64_t offset, void* stream);

/*
 * Column-wise dynamic quantization: the same with the reduction over rows,
 * for operands whose contraction runs down the columns (the A @ B and
 * A.T @ B layouts).  scale is fp32 [cols]; q keeps x's layout (no
 * transpose).  Stochastic rounding uses the same element index e = r*cols+c.
 *   ws: scratch of at least i8mp_quantize_colwise_workspace_bytes(rows, cols)
 *       bytes, 256-byte aligned; its contents on entry do not matter.
 */
/* Bytes of scratch i8mp_quantize_colwise needs for rows x cols (the slab
 * column maxima of its first pass); 0 for cols = 0 or invalid sizes. */
size_t i8mp_quantize_colwise_workspace_bytes(int64_t rows, int64_t cols);
i8mp_status i8mp_quantize_colwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                  int8_t* q, int64_t ldq, float* scale, int32_t round,
                                  uint64_t seed, uint64_t offset, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * i8mp_quantize_colwise for callers that cannot allocate memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments and results, with no workspace argument.
 * The column-maxima scratch is a static device buffer of
 * I8MP_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; nothing is allocated or freed by this call.
 * Problems whose scratch, i8mp_quantize_colwise_workspace_bytes(rows, cols),
 * exceeds that size return I8MP_ESCRATCH (about 2 bytes per column: up to
 * some 2 million columns).  Every call on one GPU shares its buffer, so calls
 * that overlap on one GPU (several streams or threads at once) race:
 * serialize them, for instance on one stream.
 */
#define I8MP_STATIC_SCRATCH_BYTES (4u << 20)
i8mp_status i8mp_quantize_colwise_noalloc(const uint16_t* x, int64_t rows, int64_t cols,
                                          int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                          int32_t round, uint64_t seed, uint64_t offset,
                                          void* stream);

/*
 * Row-wise quantization that also returns each column's maximum magnitude,
 *   colmax[c] = max_r |x[r,c]|   (fp32; exact: bf16 values widen exactly),
 * the statistic the column-wise quantization of the same tensor needs
 * (scale[c] = RN32(colmax[c] / 127)).  Codes and scales are those of
 * i8mp_quantize_rowwise.  This is how the linear chains avoid a second read
 * of X, W and dY for their column-wise passes (the pages report dynamic
 * quantization as a cost worth code-generating: "Integrate INT8
 * mixed-precision from torchao 0.7", known limitations).
 *   colmax: fp32 [cols], 4-byte aligned; rows = 0 gives zeros.
 *   ws: scratch of at least i8mp_quantize_rowwise_colmax_workspace_bytes(rows,
 *       cols) bytes, 256-byte aligned; its contents on entry do not matter.
 */
/* Bytes of scratch i8mp_quantize_rowwise_colmax needs for rows x cols (slab
 * column maxima, and for rows over 14336 elements, or under stochastic
 * rounding over 8192 (6144 when cols is not a multiple of 4), the
 * row-segment maxima), enough for either rounding;
 * 0 for cols = 0 or invalid sizes. */
size_t i8mp_quantize_rowwise_colmax_workspace_bytes(int64_t rows, int64_t cols);
i8mp_status i8mp_quantize_rowwise_colmax(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                         float* colmax, int32_t round, uint64_t seed,
                                         uint64_t offset, void* ws, size_t ws_bytes,
                                         void* stream);

/*
 * Column-wise quantization with the column maxima already known (one pass
 * over x, no scratch): scale[c] = RN32(colmax[c] / 127), codes as in
 * i8mp_quantize_colwise.  colmax must hold the column maxima of x (for
 * instance from i8mp_quantize_rowwise_colmax); other values give the codes
 * of the scales they imply, clamped to [-127, 127].
 */
i8mp_status i8mp_quantize_colwise_given_colmax(const uint16_t* x, int64_t rows, int64_t cols,
                                               int64_t ldx, const float* colmax, int8_t* q,
                                               int64_t ldq, float* scale, int32_t round,
                                               uint64_t seed, uint64_t offset, void* stream);

/*
 * Scaled INT8 matmul ("Quantized model training", section "INT8 mixed
 * precision training"; scaled back to BF16 per "Integrate INT8
 * mixed-precision from torchao 0.7"):
 *   acc[m,n] = sum_k A(m,k) * B(k,n)              (int32, exact)
 *   C[m,n]   = bf16_RNE(RN32(RN32(float(acc)) * scale_a[m]) * scale_b[n])
 * with A(m,k), B(k,n) read in the given layout (see i8mp_layout).  scale_a
 * is indexed by the output row m and scale_b by the output column n in
 * every layout.  K <= I8MP_MAX_CONTRACTION, else I8MP_ERANGE.  K = 0 writes
 * zeros.
 *   C: bf16 [M x N], leading dim ldc >= N
 */
i8mp_status i8mp_int8_scaled_mm(int32_t layout, int64_t M, int64_t N, int64_t K,
                                const int8_t* A, int64_t lda, const float* scale_a,
                                const int8_t* B, int64_t ldb, const float* scale_b, uint16_t* C,
                                int64_t ldc, void* stream);

/* The integer accumulators alone, C = int32 [M x N] (same layouts, same
 * kernels without the scale epilogue): the "INT8 matmul" of "Quantized model
 * training", section "Speed benchmarks > Matmul" (int8 x int8 -> int32 in the
 * three layouts), before any scaling.  For checking the int32 sums, which must
 * equal the exact integer dot products (K <= I8MP_MAX_CONTRACTION). */
i8mp_status i8mp_int8_mm_i32(int32_t layout, int64_t M, int64_t N, int64_t K, const int8_t* A,
                             int64_t lda, const int8_t* B, int64_t ldb, int32_t* C, int64_t ldc,
                             void* stream);

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) words as the quantize
 * kernels draw them: out[4*i + j] = word j of block (offset + i) under key
 * seed.  out: uint32 [4 * n_blocks], 16-byte aligned.  For checking draws. */
i8mp_status i8mp_philox4x32_10(uint64_t seed, uint64_t offset, int64_t n_blocks, uint32_t* out,
                               void* stream);

/*
 * Measurement hook: how fast the INT8 matrix cores run the scaled GEMM's
 * multiply-accumulate work alone under the chip's power limit.  The GEMM's
 * launch shape (256 workgroups of 8 waves) and per-wave tile (8 x 4
 * v_mfma_i32_16x16x64_i8 blocks) with operands held in registers: each wave
 * loads 24 KiB of `codes` (two sets of fragments, at its own 1 KiB-aligned
 * origin inside the buffer) once, then issues rounds x 2 x 32 MFMAs,
 * alternating the two sets, i.e. rounds x 2^32 integer operations in total.
 * The codes' bit patterns matter: the chip's power draw, and so its clock,
 * depends on them.  sink receives one int32 per thread (a checksum of the
 * accumulators) so no work is elided.
 *   codes: int8 [codes_bytes], 16-byte aligned, codes_bytes >= I8MP_MFMA_PROBE_MIN_BYTES
 *   rounds: 0 .. 2^24
 *   sink: int32 [I8MP_MFMA_PROBE_SINK_INTS], not overlapping codes
 */
#define I8MP_MFMA_PROBE_MIN_BYTES (24 * 1024)
#define I8MP_MFMA_PROBE_SINK_INTS (256 * 512)
i8mp_status i8mp_mfma_rate_probe(const int8_t* codes, int64_t codes_bytes, int64_t rounds,
                                 int32_t* sink, void* stream);

/*
 * One linear layer, Y = X @ W.T ("Quantized model training", section "INT8
 * mixed precision training": forward).  X: bf16 [M x K], W: bf16 [N x K],
 * Y: bf16 [M x N], all dense (leading dim = columns).  X and W are quantized
 * row-wise over K, then the NT scaled matmul runs.  K <= I8MP_MAX_CONTRACTION.
 * ws: at least i8mp_linear_workspace_bytes(M, N, K, 0) bytes, 256-aligned.
 * The workspace holds the int8 codes, scales and slab maxima of the chain and,
 * for an output of fewer than 128 tiles of 256 x 256 with a contraction of at
 * least 2048, the int32 partial sums of a contraction split (reduced exactly
 * before the fp32 epilogue: results equal i8mp_int8_scaled_mm's).  Its
 * contents on entry do not matter and are not kept.
 */
/* Bytes of workspace the forward (backward = 0) or backward (backward = 1)
 * chain needs for an M x N x K layer (the same for its _colmax and FP8
 * forms); 0 for invalid sizes. */
size_t i8mp_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t backward);
i8mp_status i8mp_linear_fwd(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                            int64_t N, int64_t K, const i8mp_linear_opts* opts, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Backward of the same layer (same section: backward grad input and grad
 * weight, each an INT8 GEMM quantized along its own contraction):
 *   dX = dY @ W     dY row-wise over N, W column-wise over N, NN; dX [M x K]
 *   dW = dY.T @ X   dY column-wise over M, X column-wise over M, TN; dW [N x K]
 * Either output may be NULL to skip its GEMM.  Outputs are overwritten.
 * N <= I8MP_MAX_CONTRACTION when dX is wanted, M <= it when dW is wanted.
 * ws: at least i8mp_linear_workspace_bytes(M, N, K, 1) bytes, 256-aligned.
 */
i8mp_status i8mp_linear_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* W, uint16_t* dX,
                            uint16_t* dW, int64_t M, int64_t N, int64_t K,
                            const i8mp_linear_opts* opts, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * The same forward, also returning the column maxima of X and W (fp32 [K]
 * each, as i8mp_quantize_rowwise_colmax defines them) for the backward's
 * column-wise passes.  Either pointer may be NULL.  Y is identical to
 * i8mp_linear_fwd's.  Same workspace size.
 */
i8mp_status i8mp_linear_fwd_colmax(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                                   int64_t N, int64_t K, const i8mp_linear_opts* opts,
                                   float* colmax_x, float* colmax_w, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * The same backward, taking the column maxima of X and W from the forward
 * (either may be NULL: that pass then reads its tensor twice).  dX and dW
 * are identical to i8mp_linear_bwd's when the maxima are X's and W's.  The
 * column maxima of dY always come from its row-wise pass when both outputs
 * are wanted.  Same workspace size.
 */
i8mp_status i8mp_linear_bwd_colmax(const uint16_t* dY, const uint16_t* X, const uint16_t* W,
                                   uint16_t* dX, uint16_t* dW, int64_t M, int64_t N, int64_t K,
                                   const i8mp_linear_opts* opts, const float* colmax_x,
                                   const float* colmax_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Row-wise FP8 variant.  The pages name FP8 training with row-wise scales
 * beside INT8 ("Can FP8 GEMM be enabled via module hooks instead of module
 * swapping?", the maintainer's reply: row-wise scaled float8 matmuls;
 * "Quantized model training", section "Speed benchmarks > Matmul": FP8
 * matmuls in the same three layouts).  Codes are OCP FP8 E4M3 bytes (1 sign,
 * 4 exponent bits with bias 7, 3 fraction bits, largest finite 448):
 *   scale = RN32(amax / 448), code = E4M3_RNE(clamp(RN32(x / scale), -448, 448))
 * with ties to the even code, a zero x coded +0 and an all-zero group scale 0
 * and codes 0.  Round to nearest only (no stochastic rounding).  Layouts and
 * leading dimensions as for the INT8 entry points.
 */
i8mp_status i8mp_quantize_rowwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* scale, void* stream);
/* ws: at least i8mp_quantize_colwise_workspace_bytes(rows, cols) bytes, 256-aligned. */
i8mp_status i8mp_quantize_colwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* scale, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * FP8 scaled matmul: acc[m,n] = sum_k A(m,k) * B(k,n) over E4M3 values in
 * fp32 (the matrix core's summation: each product is exact, the sums are
 * rounded), then C = bf16_RNE(RN32(RN32(acc) * scale_a[m]) * scale_b[n]).
 * Same layouts, scale indexing and shape rules as i8mp_int8_scaled_mm (any
 * sizes; fp32 accumulation, so no contraction bound).  Shapes the pipelined
 * kernel cannot take (K not a multiple of 16, an output extent read down an
 * operand's rows not a multiple of 4, tile extents past 2^31 bytes) run on a
 * general kernel that issues the same instruction on the same operand
 * placement, so its sums are those of the pipelined kernel.
 */
i8mp_status i8mp_fp8_scaled_mm(int32_t layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                               int64_t lda, const float* scale_a, const uint8_t* B, int64_t ldb,
                               const float* scale_b, uint16_t* C, int64_t ldc, void* stream);

/* The fp32 sums alone, C = float [M x N] (same layouts and kernel without the
 * scale epilogue).  For characterizing the matrix core's FP8 summation. */
i8mp_status i8mp_fp8_mm_f32(int32_t layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                            int64_t lda, const uint8_t* B, int64_t ldb, float* C, int64_t ldc,
                            void* stream);

/*
 * The linear layer's forward and backward with FP8 codes in place of INT8
 * (same passes, layouts, sizes and outputs as i8mp_linear_fwd /
 * i8mp_linear_bwd; workspace sizes from i8mp_linear_workspace_bytes).  The
 * GEMMs are i8mp_fp8_scaled_mm's; a GEMM with few output tiles and a long
 * contraction sums its contraction in slices into fp32 partial planes in the
 * workspace, added in a fixed order (so its output may differ from the
 * unsliced GEMM's by that fp32 rounding, within the same error bound).
 */
i8mp_status i8mp_linear_fwd_fp8(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                                int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream);
i8mp_status i8mp_linear_bwd_fp8(const uint16_t* dY, const uint16_t* X, const uint16_t* W,
                                uint16_t* dX, uint16_t* dW, int64_t M, int64_t N, int64_t K,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * The FP8 forward also returning the column maxima of X and W (fp32 [K]
 * each, either pointer may be NULL), and the FP8 backward taking them (as
 * i8mp_linear_fwd_colmax / i8mp_linear_bwd_colmax for INT8): the backward's
 * column-wise passes of W and X then read their tensors once, and the chains
 * pair their quantize passes in shared launches.  Outputs are identical to
 * i8mp_linear_fwd_fp8's and i8mp_linear_bwd_fp8's when the maxima are X's
 * and W's.  Same workspace sizes.
 */
i8mp_status i8mp_linear_fwd_fp8_colmax(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                                       int64_t N, int64_t K, float* colmax_x, float* colmax_w, void* ws,
                                       size_t ws_bytes, void* stream);
i8mp_status i8mp_linear_bwd_fp8_colmax(const uint16_t* dY, const uint16_t* X, const uint16_t* W,
                                       uint16_t* dX, uint16_t* dW, int64_t M, int64_t N, int64_t K,
                                       const float* colmax_x, const float* colmax_w, void* ws,
                                       size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* I8MP_H */
