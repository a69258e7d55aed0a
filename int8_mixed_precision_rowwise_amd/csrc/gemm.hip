// Scaled INT8 GEMM for gfx950 in the three layouts of a linear layer's
// training step ("Quantized model training", section "Speed benchmarks >
// Matmul": A @ B.T, A @ B, A.T @ B; section "INT8 mixed precision training":
// scaled INT8 matmul after dynamic row-wise quantization):
//   acc[m,n] = sum_k A(m,k) B(k,n)   int8 x int8 -> int32 (exact)
//   C[m,n]   = bf16_RNE(RN32(RN32(float(acc)) * sa[m]) * sb[n])
// or the raw int32 accumulators.
//
// Structure: one workgroup of 4 waves per BM x BN output tile, K in steps of
// 64 through double-buffered LDS, v_mfma_i32_32x32x32_i8 on 32 x 32 blocks.
// An operand whose contraction dimension is contiguous in memory (A in NT and
// NN, B in NT) is staged K-major and fed to the MFMA with ds_read_b128; an
// operand whose contraction runs down its rows (B in NN and TN, A in TN) is
// staged in its storage orientation and transposed on the way out of LDS by
// ds_read_b64_tr_b8, so no transposed copy is ever written to memory.
//
// ds_read_b64_tr_b8: within each group of 16 lanes, lane i receives byte j
// from byte (i mod 8) of the 8 bytes addressed by lane 2j + i/8.  When lane
// 2j + h of a group addresses row k0 + j, columns n0 + 8h .. n0 + 8h + 7 of
// a [k][n] tile, lane i therefore receives column n0 + i at rows k0 .. k0+7.
//
// MFMA 32x32x32 i8 operand/result layout: lane l supplies row l % 32 of the
// A block and column l % 32 of the B block with 16 contraction values in
// k order (k = 16 * (l / 32) + 0..15 of the 32-wide step); result register v
// of lane l holds row 8 * (v / 4) + 4 * (l / 32) + v % 4, column l % 32.
#include "internal.h"

namespace i8mp {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int BK = 64;
constexpr int kThreads = 256;

// K-major LDS tile: rows of 64 bytes, 16-byte chunk c of row r stored at
// chunk c ^ ((r >> 1) & 3), so that 8 lanes reading one chunk column of 8
// consecutive rows (the MFMA fragment read) and 8 lanes writing two rows hit
// 8 distinct 16-byte bank groups.
__device__ __forceinline__ int kmajor_off(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 3)) << 4); }

// Storage-orientation LDS tile: BK rows (k) of W bytes, 16-byte chunk c of
// row k stored at chunk c ^ (k & 7): the 8 rows one transpose read touches
// land in 8 distinct bank groups.
template <int W>
__device__ __forceinline__ int mnmajor_off(int k, int c) { return k * W + ((c ^ (k & 7)) << 4); }

// Keep the first n (0..16) bytes of a 16-byte chunk.
__device__ __forceinline__ uint4 keep_bytes(uint4 v, int n) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int left = n - 4 * i;
    const uint32_t mask = left >= 4 ? 0xFFFFFFFFu : left <= 0 ? 0u : ((1u << (8 * left)) - 1u);
    w[i] &= mask;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Global -> register staging of one BK-deep slab of an operand tile.
//   KMAJOR: R rows (output rows or columns) of BK contraction bytes, row r at
//           p[(mn0 + r) * ld + k0 ..]
//   else:   BK rows of R bytes, row k at p[(k0 + k) * ld + mn0 ..]
template <int R, bool KMAJOR>
struct Stager {
  static constexpr int kChunks = R * BK / 16 / kThreads;  // 16-byte chunks per thread
  uint4 v[kChunks];

  __device__ __forceinline__ void load(const int8_t* __restrict__ p, int64_t ld, int64_t mn0,
                                       int64_t MN, int64_t k0, int64_t K, int t) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int id = i * kThreads + t;
      if constexpr (KMAJOR) {
        const int r = id >> 2, c = id & 3;
        const int64_t kk = k0 + 16 * c;
        if (mn0 + r < MN && kk < K) {
          v[i] = *reinterpret_cast<const uint4*>(p + (mn0 + r) * ld + kk);
          if (kk + 16 > K) v[i] = keep_bytes(v[i], (int)(K - kk));
        } else {
          v[i] = make_uint4(0, 0, 0, 0);
        }
      } else {
        constexpr int CPR = R / 16;  // chunks per row
        const int k = id / CPR, c = id % CPR;
        const int64_t mm = mn0 + 16 * c;
        // bytes past MN inside a chunk only reach outputs that are never stored
        if (k0 + k < K && mm < MN)
          v[i] = *reinterpret_cast<const uint4*>(p + (k0 + k) * ld + mm);
        else
          v[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(int8_t* lds, int t) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int id = i * kThreads + t;
      int off;
      if constexpr (KMAJOR) {
        off = kmajor_off(id >> 2, id & 3);
      } else {
        constexpr int CPR = R / 16;
        off = mnmajor_off<R>(id / CPR, id % CPR);
      }
      *reinterpret_cast<uint4*>(lds + off) = v[i];
    }
  }
};

// MFMA operand (16 contraction bytes) for 32-row block `blk0` (row offset
// within the tile) at contraction step kk (0 or 1) of the slab.
template <int R, bool KMAJOR>
__device__ __forceinline__ v4i frag(const int8_t* lds, int blk0, int kk, int lane) {
  if constexpr (KMAJOR) {
    const int r = blk0 + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const v4i*>(lds + kmajor_off(r, c));
  } else {
    const int g = lane >> 4, li = lane & 15;
    const int n16 = blk0 + 16 * (g & 1);      // 16 output rows/cols of this lane group
    const int kb = 32 * kk + 16 * (g >> 1);   // 16 contraction rows of this lane group
    const int krow = kb + (li >> 1);
    const int c = n16 >> 4;
    const int half = (li & 1) << 3;
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_v2i*)(lds + mnmajor_off<R>(krow, c) + half));
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_v2i*)(lds + mnmajor_off<R>(krow + 8, c) + half));
    v4i out;
    out.x = lo.x;
    out.y = lo.y;
    out.z = hi.x;
    out.w = hi.y;
    return out;
  }
}

// Workgroup -> output tile.  Dispatch sends consecutive workgroups to the 8
// XCDs in turn; when the grid is a multiple of 8 the remap gives each XCD a
// contiguous run of tiles, and tiles are ordered in groups of GROUP_M tile
// rows so that the tiles resident on one XCD share A and B panels in its L2.
__device__ __forceinline__ void tile_of(int wg, int nwg, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 4;
  int t = wg;
  if ((nwg & 7) == 0) t = (wg & 7) * (nwg >> 3) + (wg >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = t - group * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, bool OUT_I32>
__global__ __launch_bounds__(kThreads) void gemm_i8(int64_t M, int64_t N, int64_t K,
                                                    const int8_t* __restrict__ A, int64_t lda,
                                                    const float* __restrict__ sa,
                                                    const int8_t* __restrict__ B, int64_t ldb,
                                                    const float* __restrict__ sb,
                                                    void* __restrict__ Cv, int64_t ldc) {
  constexpr int WM = BM / 2, WN = BN / 2;  // 2 x 2 waves
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  __shared__ __attribute__((aligned(16))) int8_t lds[2 * (A_BYTES + B_BYTES)];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16i){};

  Stager<BM, A_KMAJOR> sa_stage;
  Stager<BN, B_KMAJOR> sb_stage;
  const int nk = (int)((K + BK - 1) / BK);
  if (nk > 0) {
    sa_stage.load(A, lda, m0, M, 0, K, t);
    sb_stage.load(B, ldb, n0, N, 0, K, t);
    sa_stage.store(lds, t);
    sb_stage.store(lds + A_BYTES, t);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    int8_t* cur = lds + (kt & 1) * (A_BYTES + B_BYTES);
    int8_t* nxt = lds + ((kt & 1) ^ 1) * (A_BYTES + B_BYTES);
    const bool more = kt + 1 < nk;
    if (more) {
      sa_stage.load(A, lda, m0, M, (int64_t)(kt + 1) * BK, K, t);
      sb_stage.load(B, ldb, n0, N, (int64_t)(kt + 1) * BK, K, t);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      v4i af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = frag<BM, A_KMAJOR>(cur, wm0 + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = frag<BN, B_KMAJOR>(cur + A_BYTES, wn0 + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      sa_stage.store(nxt, t);
      sb_stage.store(nxt + A_BYTES, t);
    }
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = n0 + wn0 + 32 * j + (lane & 31);
    if (n >= N) continue;
    float sbn = 0.0f;
    if constexpr (!OUT_I32) sbn = sb[n];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m >= M) continue;
        if constexpr (OUT_I32) {
          static_cast<int32_t*>(Cv)[m * ldc + n] = acc[i][j][v];
        } else {
          float y = (float)acc[i][j][v];
          y = y * sa[m];
          y = y * sbn;
          const __bf16 h = (__bf16)y;  // round to nearest even
          static_cast<__bf16*>(Cv)[m * ldc + n] = h;
        }
      }
    }
  }
}

template <int BM, int BN, bool AK, bool BKM>
hipError_t run(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const float* sa,
               const int8_t* B, int64_t ldb, const float* sb, uint16_t* Cb, int32_t* Ci,
               int64_t ldc, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  if (Ci)
    gemm_i8<BM, BN, AK, BKM, true><<<grid, kThreads, 0, stream>>>(M, N, K, A, lda, sa, B, ldb, sb, Ci, ldc);
  else
    gemm_i8<BM, BN, AK, BKM, false><<<grid, kThreads, 0, stream>>>(M, N, K, A, lda, sa, B, ldb, sb, Cb, ldc);
  return hipGetLastError();
}

template <bool AK, bool BKM>
hipError_t pick(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const float* sa,
                const int8_t* B, int64_t ldb, const float* sb, uint16_t* Cb, int32_t* Ci,
                int64_t ldc, hipStream_t stream) {
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles >= 200)
    return run<256, 256, AK, BKM>(M, N, K, A, lda, sa, B, ldb, sb, Cb, Ci, ldc, stream);
  return run<128, 128, AK, BKM>(M, N, K, A, lda, sa, B, ldb, sb, Cb, Ci, ldc, stream);
}

}  // namespace

hipError_t launch_gemm(int layout, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                       const float* sa, const int8_t* B, int64_t ldb, const float* sb,
                       uint16_t* C_bf16, int32_t* C_i32, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (layout) {
    case 0:
      return pick<true, true>(M, N, K, A, lda, sa, B, ldb, sb, C_bf16, C_i32, ldc, stream);
    case 1:
      return pick<true, false>(M, N, K, A, lda, sa, B, ldb, sb, C_bf16, C_i32, ldc, stream);
    default:
      return pick<false, false>(M, N, K, A, lda, sa, B, ldb, sb, C_bf16, C_i32, ldc, stream);
  }
}

}  // namespace i8mp
