// Internal launchers of the gfx950 kernels.  The C ABI in i8mp_api.cpp
// validates every argument before calling any of these; the launchers assume
// valid, aligned arguments and only pick a kernel variant and a grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace i8mp {

// Row-wise quantization (round: 0 = RNE, 1 = SR).
hipError_t launch_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   int8_t* q, int64_t ldq, float* scale, int round, uint64_t seed,
                                   uint64_t offset, hipStream_t stream);

// Column-wise quantization: slab column maxima into ws, then the quantize
// pass (which reduces the slabs to the scales first).
size_t colwise_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_quantize_colwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   int8_t* q, int64_t ldq, float* scale, int round, uint64_t seed,
                                   uint64_t offset, void* ws, hipStream_t stream);

// The column-wise quantization with its slab maxima in the library's static
// device scratch (kStaticScratchBytes per GPU, shared by every call on that
// GPU) instead of a caller workspace; needs colwise_workspace_bytes(rows,
// cols) <= kStaticScratchBytes (hipErrorInvalidValue otherwise).
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
hipError_t launch_quantize_colwise_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                          int8_t* q, int64_t ldq, float* scale, int round,
                                          uint64_t seed, uint64_t offset, hipStream_t stream);

// Row-wise quantization that also writes colmax[c] = max_r |x[r,c]| (fp32),
// via slab maxima in ws.
size_t rowwise_colmax_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_quantize_rowwise_colmax(const uint16_t* x, int64_t rows, int64_t cols,
                                          int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                          float* colmax, int round, uint64_t seed, uint64_t offset,
                                          void* ws, hipStream_t stream);

// The row pass of launch_quantize_rowwise_colmax alone (finalize = false):
// codes, scales and the slab maxima in ws, which a later ColmaxJob reduces
// to colmax.
hipError_t launch_quantize_rowwise_slabs(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                         int8_t* q, int64_t ldq, float* scale, float* colmax,
                                         int round, uint64_t seed, uint64_t offset, void* ws,
                                         bool finalize, hipStream_t stream);

// Column-wise quantization with the column maxima given: one pass.
hipError_t launch_quantize_colwise_given(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ldx, const float* colmax, int8_t* q, int64_t ldq,
                                         float* scale, int round, uint64_t seed, uint64_t offset,
                                         hipStream_t stream);

// Two tensors of the same width quantized row-wise with column maxima in one
// launch (and, with finalize, one reduction launch; without it the slab
// maxima stay in ws_a / ws_b for a later ColmaxJob); each has its own
// workspace of rowwise_colmax_workspace_bytes(rows, cols).  Same results as
// two calls.  fmt 0: INT8 codes; fmt 1: FP8 E4M3 codes (round = 0, rows of at
// most 14336 elements: rowwise_colmax_fp8_fused).
hipError_t launch_quantize_rowwise_colmax_pair(
    const uint16_t* xa, int64_t rows_a, int64_t ldxa, int8_t* qa, int64_t ldqa, float* scale_a,
    float* colmax_a, uint64_t offset_a, void* ws_a, const uint16_t* xb, int64_t rows_b,
    int64_t ldxb, int8_t* qb, int64_t ldqb, float* scale_b, float* colmax_b, uint64_t offset_b,
    void* ws_b, int64_t cols, int round, uint64_t seed, bool finalize, int fmt, hipStream_t stream);

// Two tensors quantized column-wise with their column maxima given, in one
// launch.  Same results as two calls.  fmt as above (FP8: round = 0).
hipError_t launch_quantize_colwise_given_pair(
    const uint16_t* xa, int64_t rows_a, int64_t cols_a, int64_t ldxa, const float* colmax_a,
    int8_t* qa, int64_t ldqa, float* scale_a, uint64_t offset_a, const uint16_t* xb,
    int64_t rows_b, int64_t cols_b, int64_t ldxb, const float* colmax_b, int8_t* qb, int64_t ldqb,
    float* scale_b, uint64_t offset_b, int round, uint64_t seed, int fmt, hipStream_t stream);

// Tensor a's row pass leaving its slab maxima in ws_a (as
// launch_quantize_rowwise_slabs with finalize = false; a's slab geometry is
// rowwise_colmax_geometry(rows_a, cols_a)) and tensor b's column pass with
// its column maxima given (as launch_quantize_colwise_given), in one launch
// where a's rows take 4 or 8 chunks per lane, else in those two launches.
// fmt as above (FP8: round = 0, a's rows of at most 14336 elements).
hipError_t launch_quantize_rowslabs_colgiven(
    const uint16_t* xa, int64_t rows_a, int64_t cols_a, int64_t ldxa, int8_t* qa, int64_t ldqa,
    float* scale_a, uint64_t offset_a, void* ws_a, const uint16_t* xb, int64_t rows_b, int64_t cols_b,
    int64_t ldxb, const float* colmax_b, int8_t* qb, int64_t ldqb, float* scale_b, uint64_t offset_b,
    int round, uint64_t seed, int fmt, hipStream_t stream);

// FP8 (E4M3) quantization, round to nearest: codes q8 in x's layout,
// scales per row (row-wise) or per column (column-wise, slab maxima in ws,
// colwise_workspace_bytes).
hipError_t launch_quantize_rowwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                       uint8_t* q8, int64_t ldq, float* scale, hipStream_t stream);
hipError_t launch_quantize_colwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                       uint8_t* q8, int64_t ldq, float* scale, void* ws,
                                       hipStream_t stream);

// FP8 (E4M3) row-wise quantization that also writes colmax (as
// launch_quantize_rowwise_colmax, or with finalize = false only the slab
// maxima in ws, as launch_quantize_rowwise_slabs; rows of at most 14336
// elements, where rowwise_colmax_fp8_fused holds), and the FP8 column-wise
// pass with the column maxima given.
bool rowwise_colmax_fp8_fused(int64_t rows, int64_t cols);
// Column maxima of x alone (fp32 [cols], as the row passes with maxima give
// them; any width).  ws: colwise_workspace_bytes(rows, cols).
hipError_t launch_column_maxima(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float* colmax,
                                void* ws, hipStream_t stream);
hipError_t launch_quantize_rowwise_colmax_fp8(const uint16_t* x, int64_t rows, int64_t cols,
                                              int64_t ldx, uint8_t* q8, int64_t ldq, float* scale,
                                              float* colmax, void* ws, bool finalize, hipStream_t stream);
hipError_t launch_quantize_colwise_given_fp8(const uint16_t* x, int64_t rows, int64_t cols,
                                            int64_t ldx, const float* colmax, uint8_t* q8,
                                            int64_t ldq, float* scale, hipStream_t stream);

// FP8 (E4M3) scaled GEMM with fp32 accumulation, same layouts, any shape.
// Exactly one of C (bf16, with both scales) or C_f32 (the raw fp32 sums) is
// non-null.
hipError_t launch_gemm_fp8(int layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                           int64_t lda, const float* sa, const uint8_t* B, int64_t ldb,
                           const float* sb, uint16_t* C, float* C_f32, int64_t ldc,
                           hipStream_t stream);

// Column maxima still to be reduced from the slab maxima (bf16 bit patterns,
// [slabs][part_ld]) that row-wise passes left in a workspace: up to two
// tensors of the same width.  colmax[t][c] = max over slabs of part[t][s][c]
// as fp32 (what colmax_finalize computes).
struct ColmaxJob {
  const uint16_t* part[2];
  float* colmax[2];
  int64_t slabs[2];
  int64_t part_ld, cols;
  int n;  // tensors (0: nothing to reduce)
};
// The slab-maxima geometry of a row pass with column maxima over rows x cols
// under rounding `round` (stochastic rounding takes the banded path for rows
// of more than 16 chunks per lane, 12 when the width is not a multiple of 4,
// with its own slab count).
void rowwise_colmax_geometry(int64_t rows, int64_t cols, int round, int64_t* slabs, int64_t* part_ld);
// The reduction as its own launch (colmax_finalize, or colmax_finalize2 for
// two tensors).
hipError_t launch_colmax_finalize(const ColmaxJob& job, hipStream_t stream);

// int8 GEMM in layout 0 = NT, 1 = NN, 2 = TN.  Exactly one of (C_bf16 with
// both scales) or C_i32 is non-null.
hipError_t launch_gemm(int layout, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                       const float* sa, const int8_t* B, int64_t ldb, const float* sb,
                       uint16_t* C_bf16, int32_t* C_i32, int64_t ldc, hipStream_t stream);

// The linear chains' GEMM (bf16 output): a problem with few output tiles and
// a long contraction splits the contraction into partial planes in ws
// (gemm_split_workspace_bytes; 0 when the problem is not split, and then ws
// may be null) and reduces them before the epilogue.  fmt 0: INT8 codes,
// int32 planes added exactly, results as launch_gemm; fmt 1: FP8 E4M3 codes,
// fp32 planes added in plane order (results as launch_gemm_fp8 up to those
// additions' rounding).  lda/ldb as in launch_gemm.
size_t gemm_split_workspace_bytes(int layout, int64_t M, int64_t N, int64_t K, int64_t lda,
                                  int64_t ldb);
// side: column maxima to reduce as well (or null).  The GEMM's workgroups
// fold them after their epilogue stores, from slab rows loaded behind their
// first operand slabs, when the problem allows (pipelined kernel, at most one
// group of 32 columns per workgroup, at most 256 slabs, 128 for 128 x 128
// tiles); otherwise it runs as its own launch first.
hipError_t launch_gemm_split(int layout, int64_t M, int64_t N, int64_t K, const int8_t* A,
                             int64_t lda, const float* sa, const int8_t* B, int64_t ldb,
                             const float* sb, uint16_t* C, int64_t ldc, void* ws,
                             const ColmaxJob* side, int fmt, hipStream_t stream);

hipError_t launch_philox(uint64_t seed, uint64_t offset, int64_t n_blocks, uint32_t* out,
                         hipStream_t stream);

// The matrix-core throughput probe: kMfmaProbeWorkgroups workgroups of 512
// threads; each wave reads 24 KiB of codes at its own origin (a multiple of
// 1 KiB, wrapping within `bytes`, which must be at least 24 KiB) and writes
// one int32 per thread to sink.
constexpr int kMfmaProbeWorkgroups = 256;
hipError_t launch_mfma_rate_probe(const int8_t* codes, int64_t bytes, int64_t rounds, int32_t* sink,
                                  hipStream_t stream);

}  // namespace i8mp
