// Scaled INT8 GEMM for gfx950 in the three layouts of a linear layer's
// training step ("Quantized model training", section "Speed benchmarks >
// Matmul": A @ B.T, A @ B, A.T @ B; section "INT8 mixed precision training":
// scaled INT8 matmul after dynamic row-wise quantization):
//   acc[m,n] = sum_k A(m,k) B(k,n)   int8 x int8 -> int32 (exact)
//   C[m,n]   = bf16_RNE(RN32(RN32(float(acc)) * sa[m]) * sb[n])
// or the raw int32 accumulators.
//
// Structure: one workgroup per BM x BN output tile, K in slabs of 64 bytes
// through LDS.  Two kernels: a pipelined one (slabs loaded memory -> LDS by
// the buffer unit, several slabs in flight; v_mfma_i32_16x16x64_i8 on 16 x 16
// blocks; 8 waves for 256 x 256 tiles, 4 for 128 x 128) for contraction
// lengths that are multiples of 16, and a register-staged double-buffered one
// (4 waves, v_mfma_i32_32x32x32_i8 on 32 x 32 blocks) for every other shape.
// The linear chains may split a long contraction of a few-tile output over
// several copies of the tile grid (int32 partial planes, then splitk_reduce).
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
// MFMA 32x32x32 i8 operand/result layout: lane l supplies row l % 32 of its
// first operand block and column l % 32 of its second with 16 contraction
// values in k order (k = 16 * (l / 32) + 0..15 of the 32-wide step); result
// register v of lane l holds row 8 * (v / 4) + 4 * (l / 32) + v % 4 (an index
// of the first operand), column l % 32 (of the second).
#include "internal.h"

#include <algorithm>

#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set by the slab loads

namespace i8mp {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int BK = 64;
constexpr int kThreads = 256;

// gfx950 LDS: 64 banks of 4 bytes (256 bytes per clock per CU); a 16-byte
// read is served 16 lanes at a time, an 8-byte read 32 lanes at a time, and
// each phase runs at full rate only if its lanes hit 64 distinct banks.
//
// K-major LDS tile: rows of 64 bytes, 16-byte chunk c of row r stored at
// chunk c ^ ((r >> 2) & 3).  The MFMA fragment read has 16 lanes read one
// chunk column of 16 consecutive rows: rows r and r + 4j share the bank
// offset of r * 64 and the swizzle moves them to 4 different 16-byte groups.
__device__ __forceinline__ int kmajor_off(int r, int c) { return r * BK + ((c ^ ((r >> 2) & 3)) << 4); }

// Storage-orientation LDS tile: BK rows (k) of W bytes, 16-byte chunk c of
// row k stored at chunk c ^ s(k).  A transpose read has 32 lanes read 8
// bytes each from 8 consecutive rows in each of two chunks: either two
// adjacent chunks of the same rows (32 x 32 blocks) or one chunk of rows k
// and k + 16 (16 x 16 blocks).  W = 256: every row starts at bank 0 and
// s(k) = 2 (k & 7) ^ ((k >> 4) & 1) sends all 16 chunk reads to distinct
// 16-byte bank groups; W = 128: rows alternate between the two halves of the
// banks and s(k) = (k & 7) ^ ((k >> 4) & 1) does the same.
__device__ __forceinline__ constexpr int mnmajor_swz(int W, int k) {
  return (W >= 256 ? 2 * (k & 7) : (k & 7)) ^ ((k >> 4) & 1);
}
template <int W>
__device__ __forceinline__ int mnmajor_off(int k, int c) { return k * W + ((c ^ mnmajor_swz(W, k)) << 4); }

// Elementwise maximum of two pairs of packed 16-bit unsigned values.
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

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

// Scales of the workgroup's BM rows and BN columns, staged in LDS once so
// the epilogue reads them with ds_read (global loads would have to wait
// behind the output stores, which share the vector-memory counter).
template <int BM, int BN, bool OUT_I32>
__device__ __forceinline__ void stage_scales(float* s_lds, int64_t m0, int64_t n0, int64_t M,
                                             int64_t N, const float* __restrict__ sa,
                                             const float* __restrict__ sb, int t) {
  if constexpr (!OUT_I32) {
    for (int i = t; i < BM + BN; i += kThreads) {
      float v = 0.0f;
      if (i < BM) {
        if (m0 + i < M) v = sa[m0 + i];
      } else if (n0 + (i - BM) < N) {
        v = sb[n0 + (i - BM)];
      }
      s_lds[i] = v;
    }
  }
  __syncthreads();
}

// Epilogue of one wave's TM x TN blocks of 32 x 32 accumulators whose
// top-left output is (mw, nw) = tile origin + (wm, wn).  The MFMAs take the
// B fragment as their first operand, so in block (i, j) lane l holds output
// row m = mw + 32i + l % 32 and register v holds column
// n = nw + 32j + 8(v / 4) + 4(l / 32) + v % 4: four consecutive registers
// are four adjacent outputs of one row, stored together (8 bytes of bf16 or
// 16 bytes of int32) when VEC.  y = RN(RN(float(acc) * sa[m]) * sb[n]).
// s_lds holds sa[tile rows] then sb[tile columns].
template <int BM, int TM, int TN, bool OUT_I32, bool VEC>
__device__ __forceinline__ void store_tile(const v16i (&acc)[TM][TN], int64_t m0, int64_t n0,
                                           int wm, int wn, int64_t M, int64_t N,
                                           const float* s_lds, void* __restrict__ Cv,
                                           int64_t ldc, int lane) {
  const int mr = lane & 31, nq = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm + 32 * i + mr;
      if (m >= M) continue;
      float sam = 0.0f;
      if constexpr (!OUT_I32) sam = s_lds[wm + 32 * i + mr];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cn = wn + 32 * j + 8 * q + nq;  // column within the tile
        const int64_t n4 = n0 + cn;
        if (n4 >= N) continue;
        if constexpr (OUT_I32) {
          int32_t* row = static_cast<int32_t*>(Cv) + m * ldc;
          if (VEC && n4 + 4 <= N) {
            *reinterpret_cast<v4i*>(row + n4) =
                (v4i){acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n4 + e < N) row[n4 + e] = acc[i][j][4 * q + e];
          }
        } else {
          const float4 sbq = *reinterpret_cast<const float4*>(s_lds + BM + cn);
          const float sbv[4] = {sbq.x, sbq.y, sbq.z, sbq.w};
          __bf16 h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y = (float)acc[i][j][4 * q + e];
            y = y * sam;
            y = y * sbv[e];
            h[e] = (__bf16)y;  // round to nearest even
          }
          __bf16* row = static_cast<__bf16*>(Cv) + m * ldc;
          if (VEC && n4 + 4 <= N) {
            *reinterpret_cast<uint2*>(row + n4) = __builtin_bit_cast(uint2, h);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n4 + e < N) row[n4 + e] = h[e];
          }
        }
      }
    }
  }
}

// bf16 output from fp32 accumulators of 32 x 32 blocks (FP8 GEMM), without
// the LDS stage (C not 16-byte aligned, or ldc not a multiple of 8): same
// index map as store_tile, 4 adjacent outputs per group of registers.
template <int BM, int TM, int TN>
__device__ __forceinline__ void store32f_direct(const v16f (&acc)[TM][TN], int64_t m0, int64_t n0,
                                                int wm, int wn, int64_t M, int64_t N,
                                                const float* s_lds, __bf16* __restrict__ C,
                                                int64_t ldc, int lane) {
  const int mr = lane & 31, nq = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm + 32 * i + mr;
    if (m >= M) continue;
    const float sam = s_lds[wm + 32 * i + mr];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cn = wn + 32 * j + 8 * q + nq + e;
          if (n0 + cn >= N) continue;
          float y = acc[i][j][4 * q + e];
          y = y * sam;
          y = y * s_lds[BM + cn];
          C[m * ldc + n0 + cn] = (__bf16)y;  // round to nearest even
        }
  }
}

// The fp32 sums of 32 x 32 blocks themselves (FP8 GEMM without epilogue).
template <int TM, int TN>
__device__ __forceinline__ void store32f_raw(const v16f (&acc)[TM][TN], int64_t m0, int64_t n0,
                                             int wm, int wn, int64_t M, int64_t N,
                                             float* __restrict__ C, int64_t ldc, int lane) {
  const int mr = lane & 31, nq = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm + 32 * i + mr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t n = n0 + wn + 32 * j + 8 * q + nq + e;
          if (n < N) C[m * ldc + n] = acc[i][j][4 * q + e];
        }
  }
}

// bf16 epilogue through LDS: each wave scales its WM x WN accumulators,
// writes them as bf16 into its own LDS region (rows of WN * 2 bytes, 16-byte
// chunk c of row r at chunk c ^ (r mod chunks-per-row)), then reads whole
// rows back 16 bytes per lane and stores them, so every store instruction
// writes complete rows instead of scattered 8-byte pieces.  Needs C 16-byte
// aligned and ldc a multiple of 8; `stage` holds at least 4 * WM * WN * 2
// bytes and no wave reads the slab buffers any more.
template <int BM, int TM, int TN, typename AccV>
__device__ __forceinline__ void store_tile_staged(const AccV (&acc)[TM][TN], int64_t m0, int64_t n0,
                                                  int wm, int wn, int64_t M, int64_t N,
                                                  const float* s_lds, int8_t* stage,
                                                  __bf16* __restrict__ C, int64_t ldc, int lane,
                                                  int wave) {
  constexpr int WM = 32 * TM, WN = 32 * TN;
  constexpr int CPR = WN / 8;           // 16-byte chunks per row
  constexpr int PITCH = WN * 2;         // bytes per row
  int8_t* mine = stage + wave * (WM * PITCH);
  const int mr = lane & 31, half = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = 32 * i + mr;
    const float sam = s_lds[wm + r];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int chunk = 4 * j + q;  // columns 8 * chunk .. + 7 of the wave tile
        const float4 sbq = *reinterpret_cast<const float4*>(s_lds + BM + wn + 8 * chunk + 4 * half);
        const float sbv[4] = {sbq.x, sbq.y, sbq.z, sbq.w};
        __bf16 h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float y = (float)acc[i][j][4 * q + e];
          y = y * sam;
          y = y * sbv[e];
          h[e] = (__bf16)y;  // round to nearest even
        }
        const int off = r * PITCH + ((chunk ^ (r & (CPR - 1))) << 4) + 8 * half;
        *reinterpret_cast<uint2*>(mine + off) = __builtin_bit_cast(uint2, h);
      }
    }
  }
  __syncthreads();
  constexpr int RPI = 64 / CPR;  // rows per read instruction
  const int c = lane % CPR;
#pragma unroll 4
  for (int r0 = 0; r0 < WM; r0 += RPI) {
    const int r = r0 + lane / CPR;
    const uint4 v = *reinterpret_cast<const uint4*>(mine + r * PITCH + ((c ^ (r & (CPR - 1))) << 4));
    const int64_t m = m0 + wm + r;
    const int64_t n = n0 + wn + 8 * c;
    if (m < M) {
      __bf16* dst = C + m * ldc + n;
      if (n + 8 <= N) {
        // streaming store: the output is not read again by this kernel
        __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(dst));
      } else if (n < N) {
        const __bf16* hv = reinterpret_cast<const __bf16*>(&v);
        for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = hv[e];
      }
    }
  }
}

template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, bool OUT_I32, bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_i8_general(int64_t M, int64_t N, int64_t K,
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
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      sa_stage.store(nxt, t);
      sb_stage.store(nxt + A_BYTES, t);
    }
    __syncthreads();
  }

  // every wave has passed its last LDS read of the slabs before any scale lands
  __syncthreads();
  float* s_lds = reinterpret_cast<float*>(lds);
  stage_scales<BM, BN, OUT_I32>(s_lds, m0, n0, M, N, sa, sb, t);
  store_tile<BM, TM, TN, OUT_I32, VEC>(acc, m0, n0, wm0, wn0, M, N, s_lds, Cv, ldc, lane);
}


// ---------------------------------------------------------------------------
// Pipelined kernel, used when the contraction length is a multiple of 16.
// Operand slabs go straight from memory into LDS with buffer_load ... lds
// (16 bytes per lane, one lane-major KiB per instruction), STAGES slabs deep
// and issued STAGES - 1 slabs ahead of use, so no registers stage them and
// the loads of later slabs overlap the MFMAs of the current one.  Each lane
// picks the source of the LDS chunk it lands in, which realizes the LDS
// swizzles above.  Chunks outside the operand (tails of M, N or K) get an
// out-of-range offset, which the buffer unit returns as zeros.  MFMA
// fragments are double-buffered in registers across the 32-wide steps.

constexpr int STAGES = 4;
constexpr uint32_t kOob = 0x7FFFFFF0u;  // offset past every buffer's range
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits until at most `vm` vector-memory operations
// are outstanding and leaves the other counters alone (gfx9 encoding).
constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | (((vm >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

// Workgroup barrier for the pipelined loop: waits for this wave's LDS reads
// (so no wave refills a buffer another wave is still reading) but not for
// the slab loads in flight, whose completion is tracked with waitcnt_vm.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);  // nothing is scheduled across the barrier
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unchanged
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// REBASE (operands read down their rows only): each slab's loads use a
// descriptor based at the slab's first row, so the offsets stay within one
// slab (BK rows) however far the operand extends, beyond 2^31 bytes included.
// Without it the whole operand must lie within 32-bit offsets of one
// descriptor; the launchers take this form only for operands that do not.
template <int R, bool KMAJOR, int NW, bool REBASE = false>
struct Dma {
  static constexpr int kInst = R * BK / 1024 / NW;  // instructions per wave per slab (NW waves)
  v4u rsrc;              // buffer descriptor (scalar registers)
  uint32_t off0[kInst];  // offset of this lane's chunk in slab 0
  int kpos[kInst];       // contraction index of the chunk within a slab (BK: outside the operand)
  uint32_t kstride;      // offset advance per contraction index
  const int8_t* base;    // REBASE: row 0 of the tile's columns
  int64_t bytes;         // REBASE: bytes from base to the operand's end
  int64_t ld_;           // REBASE: leading dimension (bytes)

  // p: operand base, ld: leading dim (bytes), mn0: first output row/col of
  // the tile, MN: output extent along this operand, K: contraction length.
  // Buffer descriptor of `bytes` bytes at `base`, built from wave-uniform
  // values (read from lane 0) so that it lives in scalar registers; out of
  // range offsets read as zero.
  static __device__ __forceinline__ v4u make_rsrc(const int8_t* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4u d;
    d.x = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    d.y = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu;  // stride 0
    d.z = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    d.w = 0x00020000u;
    return d;
  }

  __device__ __forceinline__ void init(const int8_t* p, int64_t ld, int64_t mn0, int64_t MN,
                                       int64_t K, int wave, int lane) {
    if constexpr (KMAJOR) {
      const int64_t rows_in = min((int64_t)R, MN - mn0);
      rsrc = make_rsrc(p + mn0 * ld, rows_in * ld);
      kstride = 1;
#pragma unroll
      for (int j = 0; j < kInst; ++j) {
        const int pc = (wave + NW * j) * 64 + lane;  // chunk index within the LDS tile
        const int r = pc >> 2;
        const int c = (pc & 3) ^ ((r >> 2) & 3);
        kpos[j] = r < rows_in ? 16 * c : BK;  // BK never passes the slab limit
        off0[j] = (uint32_t)(r * ld + 16 * c);
      }
    } else {
      constexpr int CPR = R / 16;
      const int64_t cols_in = min((int64_t)R, MN - mn0);
      if constexpr (REBASE) {
        base = p + mn0;
        bytes = (K - 1) * ld + cols_in;
        ld_ = ld;
        rsrc = make_rsrc(base, min(bytes, (int64_t)kOob));  // for issue_past_end
      } else {
        rsrc = make_rsrc(p + mn0, (K - 1) * ld + cols_in);
      }
      kstride = (uint32_t)ld;
#pragma unroll
      for (int j = 0; j < kInst; ++j) {
        const int pc = (wave + NW * j) * 64 + lane;
        const int k = pc / CPR;
        const int c = (pc % CPR) ^ mnmajor_swz(R, k);
        kpos[j] = 16 * c < cols_in ? k : BK;
        off0[j] = (uint32_t)(k * ld + 16 * c);
      }
    }
  }

  // Load instruction j (one KiB of the tile) of slab `slab` (contraction
  // offset 64 * slab) into the LDS tile `dst`.  `wave` must be wave-uniform
  // so the LDS address stays in scalar registers.
  __device__ __forceinline__ void issue_one(int j, int8_t* dst, int slab, int64_t K, int wave) const {
    const int k0 = BK * slab;
    const int limit = (int)min(K - k0, (int64_t)BK);  // contraction indices left in this slab
    uint32_t o;
    v4u r = rsrc;
    if constexpr (REBASE && !KMAJOR) {
      const int64_t sh = (int64_t)k0 * ld_;
      o = kpos[j] < limit ? off0[j] : kOob;
      r = make_rsrc(base + sh, max((int64_t)0, min(bytes - sh, (int64_t)kOob)));
    } else {
      o = kpos[j] < limit ? off0[j] + (uint32_t)k0 * kstride : kOob;
    }
    const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)(dst + (wave + NW * j) * 1024)));
    // Issued as inline assembly: the compiler then does not treat the LDS
    // write as pending on every later LDS read (which would make it wait for
    // all slabs in flight); arrival is tracked explicitly with waitcnt_vm and
    // the workgroup barrier.
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(l), "v"(o), "s"(r)
                 : "memory", "m0");
  }

  __device__ __forceinline__ void issue(int8_t* dst, int slab, int64_t K, int wave) const {
#pragma unroll
    for (int j = 0; j < kInst; ++j) issue_one(j, dst, slab, K, wave);
  }

  // Instruction j for a slab known to lie past the contraction (only zeros
  // land, into a buffer nobody reads): the same load at the out-of-range
  // offset, so the slab still counts in the waits.  Needs no offset state.
  __device__ __forceinline__ void issue_past_end(int j, int8_t* dst, int wave) const {
    const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)(dst + (wave + NW * j) * 1024)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(l), "v"(kOob), "s"(rsrc)
                 : "memory", "m0");
  }
};

// ---- column maxima reduced in a GEMM's prologue ----------------------------
//
// A linear chain's row-wise passes leave slab maxima of |x| (bf16 bit
// patterns, [slabs][part_ld], see ColmaxJob) that still have to be reduced to
// fp32 column maxima before the backward needs them.  Instead of a launch of
// its own, workgroup g of the following GEMM reduces group g: 32 columns of
// one tensor over all its slabs (at most side_slabs(BM): 256 for the big tile;
// 128 for the 128 x 128 one, whose LDS must stay under half a CU's so two
// workgroups still share a CU).  Its slab rows come into a spare LDS region
// by the same LDS-DMA loads as the operand slabs, issued after the first
// STAGES slabs' loads (off the first slab's critical path), and are folded
// after the epilogue's stores, under the store drain.  Maximum is exact and order-free: the result
// is colmax finalize's.
constexpr int side_slabs(int bm) { return bm >= 256 ? 256 : 128; }

template <int NW, int SLABS>
struct SideJob {
  static constexpr int kBytes = SLABS * 64;          // 32 columns x 2 bytes per slab row
  static constexpr int kInst = kBytes / 1024 / NW;   // 1 KiB loads per wave
  static_assert(kInst >= 1 && kBytes % (1024 * NW) == 0, "whole 1 KiB loads per wave");
  v4u rsrc;
  bool on;          // this workgroup has a group (workgroup-uniform)
  int t;            // tensor of the group
  int64_t c_first;  // first column of the group

  __device__ __forceinline__ void init(const ColmaxJob& j, int64_t g) {
    const int64_t gpt = (j.cols + 31) / 32;
    on = j.n > 0 && g < j.n * gpt;
    if (!on) return;
    t = (int)(g / gpt);
    c_first = (g % gpt) * 32;
    const int64_t slabs = j.slabs[t];
    // exactly the bytes of this group's columns, so nothing past the slab
    // maxima is read: rows of part_ld elements, the last one from c_first on
    const int64_t bytes = slabs > 0 ? ((slabs - 1) * j.part_ld + (j.part_ld - c_first)) * 2 : 0;
    rsrc = Dma<64, true, NW>::make_rsrc(reinterpret_cast<const int8_t*>(j.part[t] + c_first), bytes);
  }

  // Instruction i of this wave: chunk k = (wave + NW i) * 64 + lane is slab row
  // k / 4, 16-byte column chunk k % 4; it lands at side + 16 k.
  __device__ __forceinline__ void issue(int8_t* side, int64_t part_ld, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int k = (wave + NW * i) * 64 + lane;
      const uint32_t o = (uint32_t)((int64_t)(k >> 2) * part_ld * 2 + (k & 3) * 16);
      const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane(
          (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)(side + (wave + NW * i) * 1024)));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(l), "v"(o), "s"(rsrc)
                   : "memory", "m0");
    }
  }

  // After every wave's loads have landed (the caller's wait and barrier):
  // thread tid takes column chunk tid % 4 of slab rows tid / 4, tid / 4 + NT / 4,
  // ...; the 16 lanes of a chunk fold by shuffles, the waves through `red`.
  __device__ __forceinline__ void reduce(const ColmaxJob& j, const int8_t* side, uint4 (*red)[4],
                                         int tid, int wave, int lane) const {
    constexpr int NT = 64 * NW;
    const int chunk = tid & 3;
    uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < SLABS * 4 / NT; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(side + ((tid >> 2) + i * (NT / 4)) * 64 + chunk * 16);
      m[0] = max_u16x2(m[0], v.x), m[1] = max_u16x2(m[1], v.y);
      m[2] = max_u16x2(m[2], v.z), m[3] = max_u16x2(m[3], v.w);
    }
#pragma unroll
    for (int off = 4; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = max_u16x2(m[e], (uint32_t)__shfl_xor((int)m[e], off));
    if (lane < 4) red[wave][lane] = make_uint4(m[0], m[1], m[2], m[3]);
    __syncthreads();
    if (wave == 0 && lane < 4) {
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const uint4 o = red[w][lane];
        m[0] = max_u16x2(m[0], o.x), m[1] = max_u16x2(m[1], o.y);
        m[2] = max_u16x2(m[2], o.z), m[3] = max_u16x2(m[3], o.w);
      }
      const int64_t c0 = c_first + lane * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < j.cols) j.colmax[t][c0 + e] = __uint_as_float(((m[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
    }
  }
};

// MFMA 16x16x64 i8 operand/result layout: lane l supplies row l % 16 of its
// first operand block and column l % 16 of its second, each with 16
// contraction values (here k = 16 (l / 16) + 0..15 of the 64-deep slab; the
// dot product only needs both operands to use the same assignment); result
// register v of lane l holds row 4 (l / 16) + v of the first operand's block
// and column l % 16 of the second's.  Per operation it moves half the
// accumulator register traffic of the 32 x 32 x 32 form, which matters
// because the chip runs int8 matrix work at its power limit.
//
// Operand for 16-row (or column) block blk0 of an operand tile, whole slab.
template <int R, bool KMAJOR>
__device__ __forceinline__ v4i frag16(const int8_t* lds, int blk0, int lane) {
  if constexpr (KMAJOR) {
    return *reinterpret_cast<const v4i*>(lds + kmajor_off(blk0 + (lane & 15), lane >> 4));
  } else {
    const int li = lane & 15;
    const int krow = 16 * (lane >> 4) + (li >> 1);
    const int c = blk0 >> 4;
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

// Epilogue of one wave's TM x TN blocks of 16 x 16 accumulators whose
// top-left output is (m0 + wm, n0 + wn).  The MFMAs take the B fragment as
// their first operand, so in block (i, j) lane l holds output row
// m = 16 i + l % 16 and register v holds column n = 16 j + 4 (l / 16) + v:
// the four registers are four adjacent outputs of one row, stored together
// (8 bytes of bf16 or 16 bytes of int32) when VEC.
// y = RN(RN(float(acc) * sa[m]) * sb[n]); s_lds holds sa[tile rows] then
// sb[tile columns].
template <int BM, int TM, int TN, bool OUT_I32, bool VEC>
__device__ __forceinline__ void store16_direct(const v4i (&acc)[TM][TN], int64_t m0, int64_t n0,
                                               int wm, int wn, int64_t M, int64_t N,
                                               const float* s_lds, void* __restrict__ Cv,
                                               int64_t ldc, int lane) {
  const int mr = lane & 15, nq = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm + 16 * i + mr;
    if (m >= M) continue;
    float sam = 0.0f;
    if constexpr (!OUT_I32) sam = s_lds[wm + 16 * i + mr];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cn = wn + 16 * j + nq;  // first of the 4 columns within the tile
      const int64_t n4 = n0 + cn;
      if (n4 >= N) continue;
      if constexpr (OUT_I32) {
        int32_t* row = static_cast<int32_t*>(Cv) + m * ldc;
        if (VEC && n4 + 4 <= N) {
          *reinterpret_cast<v4i*>(row + n4) = acc[i][j];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n4 + e < N) row[n4 + e] = acc[i][j][e];
        }
      } else {
        const float4 sbq = *reinterpret_cast<const float4*>(s_lds + BM + cn);
        const float sbv[4] = {sbq.x, sbq.y, sbq.z, sbq.w};
        __bf16 h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float y = (float)acc[i][j][e];
          y = y * sam;
          y = y * sbv[e];
          h[e] = (__bf16)y;  // round to nearest even
        }
        __bf16* row = static_cast<__bf16*>(Cv) + m * ldc;
        if (VEC && n4 + 4 <= N) {
          *reinterpret_cast<uint2*>(row + n4) = __builtin_bit_cast(uint2, h);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n4 + e < N) row[n4 + e] = h[e];
        }
      }
    }
  }
}

// bf16 epilogue through LDS for 16 x 16 blocks: each wave scales its
// WM x WN accumulators, writes them as bf16 into its own LDS region (rows of
// WN * 2 bytes, 16-byte chunk c of row r at chunk c ^ (r mod chunks-per-row)),
// then reads whole rows back 16 bytes per lane and stores them, so each
// store instruction writes complete row segments.  Needs C 16-byte aligned
// and ldc a multiple of 8; `stage` holds NW * WM * WN * 2 bytes and no wave
// reads the slab buffers any more.
template <int BM, int TM, int TN>
__device__ __forceinline__ void store16_staged(const v4i (&acc)[TM][TN], int64_t m0, int64_t n0,
                                               int wm, int wn, int64_t M, int64_t N,
                                               const float* s_lds, int8_t* stage,
                                               __bf16* __restrict__ C, int64_t ldc, int lane,
                                               int wave) {
  constexpr int WM = 16 * TM, WN = 16 * TN;
  constexpr int CPR = WN / 8;    // 16-byte chunks per row
  constexpr int PITCH = WN * 2;  // bytes per row
  int8_t* mine = stage + wave * (WM * PITCH);
  const int mr = lane & 15, q = lane >> 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = 16 * i + mr;
    const float sam = s_lds[wm + r];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float4 sbq = *reinterpret_cast<const float4*>(s_lds + BM + wn + 16 * j + 4 * q);
      const float sbv[4] = {sbq.x, sbq.y, sbq.z, sbq.w};
      __bf16 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y = (float)acc[i][j][e];
        y = y * sam;
        y = y * sbv[e];
        h[e] = (__bf16)y;  // round to nearest even
      }
      const int chunk = 2 * j + (q >> 1);  // columns 8 * chunk .. + 7 of the wave tile
      const int off = r * PITCH + ((chunk ^ (r & (CPR - 1))) << 4) + 8 * (q & 1);
      *reinterpret_cast<uint2*>(mine + off) = __builtin_bit_cast(uint2, h);
    }
  }
  __syncthreads();
  constexpr int RPI = 64 / CPR;  // rows per read instruction
  const int c = lane % CPR;
#pragma unroll 4
  for (int r0 = 0; r0 < WM; r0 += RPI) {
    const int r = r0 + lane / CPR;
    const uint4 v = *reinterpret_cast<const uint4*>(mine + r * PITCH + ((c ^ (r & (CPR - 1))) << 4));
    const int64_t m = m0 + wm + r;
    const int64_t n = n0 + wn + 8 * c;
    if (m < M) {
      __bf16* dst = C + m * ldc + n;
      if (n + 8 <= N) {
        // streaming store: the output is not read again by this kernel
        __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(dst));
      } else if (n < N) {
        const __bf16* hv = reinterpret_cast<const __bf16*>(&v);
        for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = hv[e];
      }
    }
  }
}

// Main-loop schedule of one slab (TM x TN MFMAs, A-block major: MFMA m works
// on A block m / TN and B block m % TN).  The first IA * TN MFMAs run before
// the workgroup barrier; after it, each MFMA is followed by at most one
// fragment read of the next slab and at most one slab load.  Fragment reads
// go A blocks 0 .. IA-1 (free since the barrier), then the TN B blocks (into
// the other B register set), then A blocks IA .. TM-1, each no earlier than
// the MFMA that last reads it.  Small tiles run out of MFMAs: whatever is left
// is issued after the last one.
template <int TM, int TN, int PER>
struct SlabSchedule {
  static constexpr int IA = 1;
  static constexpr int HA = IA * TN;        // MFMAs before the barrier
  static constexpr int NM = TM * TN;
  static constexpr int DMA_STEP = (NM - HA) / PER > 0 ? (NM - HA) / PER : 1;
  static constexpr int last(int m) { return m < NM - 1 ? m : NM - 1; }
  static constexpr int a_read(int i) {  // MFMA index after which A block i is read
    return last(i < IA ? HA + i : (HA + TN + i > TN * (i + 1) - 1 ? HA + TN + i : TN * (i + 1) - 1));
  }
  static constexpr int b_read(int j) { return last(HA + IA + j); }
  static constexpr int dma_at(int d) { return last(HA + 1 + DMA_STEP * d); }
  static_assert(TM > IA, "need A blocks after the barrier");
};

// The two MFMA forms.  FMT 0: INT8, v_mfma_i32_16x16x64_i8 on 16 x 16 blocks
// (fragments of 16 bytes per lane, frag16).  FMT 1: FP8 E4M3,
// v_mfma_f32_32x32x64_f8f6f4 on 32 x 32 blocks: lane l supplies row l % 32 of
// its first operand block and column l % 32 of its second with 32
// contraction values (k = 32 (l / 32) + 0..31 of the slab), products summed
// in fp32; the result layout is that of the 32 x 32 blocks described at the
// top (register v of lane l: row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32).
// The FP8 form takes the whole 64-deep slab in one instruction, like the INT8
// one, so the pipeline is shared.

// FP8 operand (32 contraction bytes) for 32-row block blk0, whole slab.
template <int R, bool KMAJOR>
__device__ __forceinline__ v8i frag32f8(const int8_t* lds, int blk0, int lane) {
  v8i out;
  if constexpr (KMAJOR) {
    const int r = blk0 + (lane & 31);
    const int c = 2 * (lane >> 5);
    const v4i lo = *reinterpret_cast<const v4i*>(lds + kmajor_off(r, c));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + kmajor_off(r, c + 1));
    out[0] = lo.x, out[1] = lo.y, out[2] = lo.z, out[3] = lo.w;
    out[4] = hi.x, out[5] = hi.y, out[6] = hi.z, out[7] = hi.w;
  } else {
    const int g = lane >> 4, li = lane & 15;
    const int c = (blk0 + 16 * (g & 1)) >> 4;  // 16 output columns of this lane group
    const int krow = 32 * (g >> 1) + (li >> 1);
    const int half = (li & 1) << 3;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v2i w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i*)(lds + mnmajor_off<R>(krow + 8 * t, c) + half));
      out[2 * t] = w.x, out[2 * t + 1] = w.y;
    }
  }
  return out;
}

template <int FMT>
struct Mma;

template <>
struct Mma<0> {
  static constexpr int BLK = 16;
  typedef v4i Frag;
  typedef v4i Acc;
  template <int R, bool KMAJOR>
  static __device__ __forceinline__ Frag frag(const int8_t* lds, int blk0, int lane) {
    return frag16<R, KMAJOR>(lds, blk0, lane);
  }
  static __device__ __forceinline__ Acc mma(const Frag& b, const Frag& a, const Acc& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Acc zero() { return (v4i){0, 0, 0, 0}; }
};

template <>
struct Mma<1> {
  static constexpr int BLK = 32;
  typedef v8i Frag;
  typedef v16f Acc;
  template <int R, bool KMAJOR>
  static __device__ __forceinline__ Frag frag(const int8_t* lds, int blk0, int lane) {
    return frag32f8<R, KMAJOR>(lds, blk0, lane);
  }
  static __device__ __forceinline__ Acc mma(const Frag& b, const Frag& a, const Acc& c) {
    // operand formats 0, 0: FP8 E4M3 for both; no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, 0, 0, 0);
  }
  static __device__ __forceinline__ Acc zero() {
    v16f z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.0f;
    return z;
  }
};

template <int BM, int BN, int WGN, bool A_KMAJOR, bool B_KMAJOR, bool OUT_I32, bool VEC, int FMT = 0,
          bool SIDE = false, bool REBASE = false>
__global__ __launch_bounds__(128 * WGN) void gemm_i8_pipelined(int64_t M, int64_t N, int64_t K,
                                                              const int8_t* __restrict__ A, int64_t lda,
                                                              const float* __restrict__ sa,
                                                              const int8_t* __restrict__ B, int64_t ldb,
                                                              const float* __restrict__ sb,
                                                              void* __restrict__ Cv, int64_t ldc,
                                                              int64_t kchunk, int64_t split_stride,
                                                              ColmaxJob side) {
  constexpr int NW = 2 * WGN, NT = 64 * NW;  // 2 x WGN waves
  constexpr int WM = BM / 2, WN = BN / WGN;
  typedef Mma<FMT> T;
  typedef typename T::Frag Frag;
  typedef typename T::Acc Acc;
  constexpr int TM = WM / T::BLK, TN = WN / T::BLK;
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, SLAB = A_BYTES + B_BYTES;
  constexpr int NA = Dma<BM, A_KMAJOR, NW>::kInst;
  constexpr int PER = NA + Dma<BN, B_KMAJOR, NW>::kInst;  // loads per wave per slab
  using S = SlabSchedule<TM, TN, PER>;
  static_assert(NW * WM * WN * 2 <= STAGES * SLAB, "epilogue staging fits in the slab buffers");
  __shared__ __attribute__((aligned(1024))) int8_t lds[STAGES * SLAB];

  __shared__ __attribute__((aligned(16))) float s_lds[BM + BN];  // scales of the tile
  constexpr int SIDE_SLABS = side_slabs(BM);
  __shared__ __attribute__((aligned(1024))) int8_t side_lds[SIDE ? SIDE_SLABS * 64 : 16];
  __shared__ uint4 side_red[SIDE ? NW : 1][4];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  SideJob<NW, SIDE_SLABS> sj;
  if constexpr (SIDE) sj.init(side, blockIdx.x);
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  int wg = blockIdx.x, nwg = gridDim.x;
  if constexpr (OUT_I32) {
    // Contraction split: the grid holds `splits` copies of the tile grid and
    // copy s sums contraction indices [s kchunk, (s+1) kchunk) into its own
    // int32 output plane (Cv + s split_stride).  Unsplit: one copy, kchunk = K.
    // Consecutive workgroups take consecutive copies, so the 8 XCDs (which
    // receive workgroups in turn) mostly read disjoint contraction ranges.
    const int tiles = tiles_m * tiles_n;
    const int splits = nwg / tiles;
    const int split = wg % splits;
    const int64_t k0 = (int64_t)split * kchunk;
    wg /= splits;
    nwg = tiles;
    K = min(kchunk, K - k0);
    A += A_KMAJOR ? k0 : k0 * lda;
    B += B_KMAJOR ? k0 : k0 * ldb;
    Cv = static_cast<int32_t*>(Cv) + split * split_stride;
  }
  int tm, tn;
  tile_of(wg, nwg, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  // the epilogue's scales, fetched now so their latency hides under the main loop
  constexpr int NPRE = (BM + BN + NT - 1) / NT;
  float s_pre[NPRE];
#pragma unroll
  for (int r = 0; r < NPRE; ++r) {
    const int i = t + r * NT;
    s_pre[r] = 0.0f;
    if (!OUT_I32 && i < BM + BN) {
      if (i < BM) {
        if (m0 + i < M) s_pre[r] = sa[m0 + i];
      } else if (n0 + (i - BM) < N) {
        s_pre[r] = sb[n0 + (i - BM)];
      }
    }
  }

  Dma<BM, A_KMAJOR, NW, REBASE> da;
  Dma<BN, B_KMAJOR, NW, REBASE> db;
  da.init(A, lda, m0, M, K, wave, lane);
  db.init(B, ldb, n0, N, K, wave, lane);

  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = T::zero();

  const int nk = (int)((K + BK - 1) / BK);
  Frag a[TM], b0[TN], b1[TN];
  // Slabs 0 .. STAGES-1 go out first.  Slabs past the end are still
  // "loaded", with out-of-range offsets (the buffer unit writes zeros into a
  // buffer nobody reads), so every slab costs the same PER loads per wave and
  // the waits below count slabs.
#pragma unroll
  for (int s = 0; s < STAGES; ++s) {
    da.issue(lds + s * SLAB, s, K, wave);
    db.issue(lds + s * SLAB + A_BYTES, s, K, wave);
  }
  // The column-maxima loads (see SideJob) go out behind the first STAGES
  // slabs.  Loads complete in issue order, so each wait below, which counts
  // slab loads only, then waits for at most kInst loads more than it needs
  // in the first slabs and stays exact.
  if constexpr (SIDE) {
    if (sj.on) sj.issue(side_lds, side.part_ld, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((STAGES - 1) * PER));  // slab 0 has landed
  lds_barrier();
#pragma unroll
  for (int i = 0; i < TM; ++i) a[i] = T::template frag<BM, A_KMAJOR>(lds, wm0 + T::BLK * i, lane);
#pragma unroll
  for (int j = 0; j < TN; ++j) b0[j] = T::template frag<BN, B_KMAJOR>(lds + A_BYTES, wn0 + T::BLK * j, lane);

  // One slab: MFMAs on the fragments of slab kt (registers a, bc) while the
  // fragments of slab kt + 1 are read into a and bn and slab kt + STAGES is
  // loaded into slab kt's buffer.  The barrier guarantees that slab kt + 1
  // has landed for every wave and that every wave has finished reading slab
  // kt, whose fragments were read during the previous slab.  A sched_barrier
  // after each step keeps the matrix core fed while the LDS and memory units
  // work.  `tail`: the last slab but one, whose loads (slab kt + STAGES) lie
  // past the contraction; issuing them at the out-of-range offset directly
  // keeps the load offsets dead after the loop (otherwise they are held, or
  // spilled, across it).
  auto slab = [&](Frag (&bc)[TN], Frag (&bn)[TN], int kt, bool tail) __attribute__((always_inline)) {
    const int8_t* nxt = lds + ((kt + 1) % STAGES) * SLAB;
    int8_t* dst = lds + (kt % STAGES) * SLAB;
    const int ns = kt + STAGES;
#pragma unroll
    for (int m = 0; m < S::HA; ++m) {
      acc[m / TN][m % TN] = T::mma(bc[m % TN], a[m / TN], acc[m / TN][m % TN]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // slab kt+1 has landed once only slabs kt+2 .. kt+STAGES-1 are pending
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((STAGES - 2) * PER));
    lds_barrier();
#pragma unroll
    for (int m = S::HA; m < S::NM; ++m) {
      acc[m / TN][m % TN] = T::mma(bc[m % TN], a[m / TN], acc[m / TN][m % TN]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        if (m == S::a_read(i)) a[i] = T::template frag<BM, A_KMAJOR>(nxt, wm0 + T::BLK * i, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if (m == S::b_read(j)) bn[j] = T::template frag<BN, B_KMAJOR>(nxt + A_BYTES, wn0 + T::BLK * j, lane);
#pragma unroll
      for (int d = 0; d < PER; ++d)
        if (m == S::dma_at(d)) {
          if (tail) {
            if (d < NA) da.issue_past_end(d, dst, wave);
            else db.issue_past_end(d - NA, dst + A_BYTES, wave);
          } else {
            if (d < NA) da.issue_one(d, dst, ns, K, wave);
            else db.issue_one(d - NA, dst + A_BYTES, ns, K, wave);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // slabs 0 .. nk-2 in pairs (the B register sets swap roles each slab)
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    slab(b0, b1, kt, false);
    slab(b1, b0, kt + 1, false);
  }
  if (kt + 1 < nk) {  // kt = nk - 2: its loads are of slab nk + STAGES - 2 >= nk
    slab(b0, b1, kt, true);
    ++kt;
  }
  if (nk > 0) {  // slab nk-1, whose fragments are in a and b0 (nk-1 even) or b1
    const bool odd = kt & 1;
#pragma unroll
    for (int m = 0; m < S::NM; ++m)
      acc[m / TN][m % TN] = T::mma(odd ? b1[m % TN] : b0[m % TN], a[m / TN], acc[m / TN][m % TN]);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the trailing zero-fill loads and the scales
#pragma unroll
  for (int r = 0; r < NPRE; ++r)
    if (!OUT_I32 && t + r * NT < BM + BN) s_lds[t + r * NT] = s_pre[r];
  __syncthreads();
  if constexpr (FMT == 1) {
    if constexpr (OUT_I32)  // the raw fp32 sums (C holds floats)
      store32f_raw<TM, TN>(acc, m0, n0, wm0, wn0, M, N, static_cast<float*>(Cv), ldc, lane);
    else if constexpr (VEC)
      store_tile_staged<BM, TM, TN>(acc, m0, n0, wm0, wn0, M, N, s_lds, lds, static_cast<__bf16*>(Cv), ldc, lane, wave);
    else
      store32f_direct<BM, TM, TN>(acc, m0, n0, wm0, wn0, M, N, s_lds, static_cast<__bf16*>(Cv), ldc, lane);
  } else if constexpr (!OUT_I32 && VEC) {
    store16_staged<BM, TM, TN>(acc, m0, n0, wm0, wn0, M, N, s_lds, lds, static_cast<__bf16*>(Cv), ldc, lane, wave);
  } else {
    store16_direct<BM, TM, TN, OUT_I32, VEC>(acc, m0, n0, wm0, wn0, M, N, s_lds, Cv, ldc, lane);
  }
  // The column maxima last: their slab rows landed long ago (every wave waited
  // for all its loads and passed the barrier above), and the reduction runs
  // while the output stores drain.
  if constexpr (SIDE) {
    if (sj.on) sj.reduce(side, side_lds, side_red, t, wave, lane);  // workgroup-uniform
  }
}


// ---- matrix-core throughput probe ------------------------------------------
//
// The INT8 GEMM's matrix-core work with everything else taken away: the
// GEMM's launch shape (256 workgroups of 8 waves, two waves per SIMD) and its
// per-wave tile (8 x 4 blocks of 16 x 16, 128 accumulator registers), with the
// operands in registers.  Each wave loads two slabs' worth of fragments (real
// codes, so the operand bits toggle as in the GEMM) once, then issues
// `rounds` x 2 x 32 v_mfma_i32_16x16x64_i8, alternating the two fragment sets.
// Measures how fast the chip runs this work under its power limit.
__global__ __launch_bounds__(512) void mfma_rate_probe(const int8_t* __restrict__ codes, int64_t span,
                                                       int64_t rounds, int32_t* __restrict__ sink) {
  const int t = threadIdx.x, lane = t & 63;
  const int64_t wave = (int64_t)blockIdx.x * 8 + (t >> 6);
  // this wave's 24 fragments of 1 KiB, consecutive in the codes (wrapping)
  const int8_t* base = codes + (wave * 24 * 1024) % span;
  v4i a0[8], b0[4], a1[8], b1[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = *reinterpret_cast<const v4i*>(base + i * 1024 + lane * 16);
    a1[i] = *reinterpret_cast<const v4i*>(base + (12 + i) * 1024 + lane * 16);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b0[j] = *reinterpret_cast<const v4i*>(base + (8 + j) * 1024 + lane * 16);
    b1[j] = *reinterpret_cast<const v4i*>(base + (20 + j) * 1024 + lane * 16);
  }
  v4i acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4i){0, 0, 0, 0};
  for (int64_t r = 0; r < rounds; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0[j], a0[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1[j], a1[i], acc[i][j], 0, 0, 0);
  }
  int32_t h = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) h ^= acc[i][j].x ^ acc[i][j].y ^ acc[i][j].z ^ acc[i][j].w;
  sink[(int64_t)blockIdx.x * 512 + t] = h;
}

template <int BM, int BN, bool AK, bool BKM, bool OUT_I32, bool VEC>
void launch(bool fast, bool rebase, dim3 grid, int64_t M, int64_t N, int64_t K, const int8_t* A,
            int64_t lda, const float* sa, const int8_t* B, int64_t ldb, const float* sb, void* C,
            int64_t ldc, const ColmaxJob* side, hipStream_t stream) {
  // 256 x 256 tiles: 8 waves (2 per SIMD, 128 x 64 each) so one wave's MFMAs
  // run while the other waits on its slab-load issue; 128 x 128: 4 waves.
  // side (pipelined kernel only) is a column-maxima reduction the caller has
  // checked fits (side_fits).  rebase: the pipelined kernel with per-slab
  // descriptors (rebase_ok; 256 x 256 tiles, packed bf16 output only).
  constexpr int WGN = BM >= 256 ? 4 : 2;
  if (fast && side)
    gemm_i8_pipelined<BM, BN, WGN, AK, BKM, OUT_I32, VEC, 0, true><<<grid, 128 * WGN, 0, stream>>>(M, N, K, A, lda, sa, B, ldb, sb, C, ldc, K, 0, *side);
  else if (fast)
    gemm_i8_pipelined<BM, BN, WGN, AK, BKM, OUT_I32, VEC><<<grid, 128 * WGN, 0, stream>>>(M, N, K, A, lda, sa, B, ldb, sb, C, ldc, K, 0, ColmaxJob{});
  else if (rebase && BM == 256 && !OUT_I32 && VEC && !(AK && BKM)) {
    if constexpr (BM == 256 && !OUT_I32 && VEC && !(AK && BKM))
      gemm_i8_pipelined<BM, BN, WGN, AK, BKM, false, true, 0, false, true><<<grid, 128 * WGN, 0, stream>>>(M, N, K, A, lda, sa, B, ldb, sb, C, ldc, K, 0, ColmaxJob{});
  } else
    gemm_i8_general<BM, BN, AK, BKM, OUT_I32, VEC><<<grid, kThreads, 0, stream>>>(M, N, K, A, lda, sa, B, ldb, sb, C, ldc);
}

// Whether a column-maxima reduction can ride in the prologue of a pipelined
// launch of `wgs` workgroups of BM x BM tiles: one group of 32 columns per
// workgroup at most, at most side_slabs(BM) slabs per tensor.
bool side_fits(const ColmaxJob& j, int64_t wgs, int bm) {
  if (j.n <= 0 || j.n > 2) return false;
  const int64_t max_slabs = side_slabs(bm);
  const int64_t groups = j.n * ((j.cols + 31) / 32);
  for (int t = 0; t < j.n; ++t)
    if (j.slabs[t] > max_slabs) return false;
  return groups <= wgs && j.part_ld * 2 * max_slabs < (int64_t(1) << 31);
}

// Whether the pipelined kernel can take a BM x BN tiling of this problem.
// It addresses each operand tile with 32-bit buffer offsets and zero-fills
// whole 16-byte chunks, so it needs K % 16 == 0 and tile extents below 2^31
// bytes.  An operand whose contraction runs down its rows is range-checked at
// its last byte, and the buffer unit checks whole dwords: its output extent
// must be a multiple of 4 or the last row's final dword would read as zero.
template <int BM, int BN, bool AK, bool BKM>
bool pipelined_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t a_ext = AK ? (int64_t)BM * lda : K * lda;
  const int64_t b_ext = BKM ? (int64_t)BN * ldb : K * ldb;
  const bool mn_ok = (AK || M % 4 == 0) && (BKM || N % 4 == 0);
  return K > 0 && K % 16 == 0 && a_ext < lim - 1024 && b_ext < lim - 1024 && mn_ok;
}

// Whether the pipelined kernel with per-slab descriptors (REBASE) takes a
// problem the plain form cannot because an operand read down its rows spans
// 2^31 bytes or more (e.g. a grad-weight GEMM over a wide output at many
// tokens): 256 x 256 tiles, the same shape rules, and each slab (BK rows of
// such an operand) within 32-bit offsets.
template <int BM, int BN, bool AK, bool BKM>
bool rebase_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  if (BM != 256 || (AK && BKM)) return false;
  const int64_t lim = int64_t(1) << 31;
  const int64_t a_ext = AK ? (int64_t)BM * lda : (int64_t)BK * lda;
  const int64_t b_ext = BKM ? (int64_t)BN * ldb : (int64_t)BK * ldb;
  const bool mn_ok = (AK || M % 4 == 0) && (BKM || N % 4 == 0);
  return K > 0 && K % 16 == 0 && a_ext < lim - 1024 && b_ext < lim - 1024 && mn_ok &&
         !pipelined_ok<BM, BN, AK, BKM>(M, N, K, lda, ldb);
}

template <int BM, int BN, bool AK, bool BKM>
hipError_t run(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const float* sa,
               const int8_t* B, int64_t ldb, const float* sb, uint16_t* Cb, int32_t* Ci,
               int64_t ldc, const ColmaxJob* side, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  const bool fast = pipelined_ok<BM, BN, AK, BKM>(M, N, K, lda, ldb);
  const bool rebase = rebase_ok<BM, BN, AK, BKM>(M, N, K, lda, ldb);
  if (side && (Ci || !(fast && side_fits(*side, tiles, BM)))) {  // as a launch of its own
    const hipError_t e = launch_colmax_finalize(*side, stream);
    if (e != hipSuccess) return e;
    side = nullptr;
  }
  // packed stores of adjacent outputs need 16-byte aligned rows
  const uintptr_t c = Ci ? reinterpret_cast<uintptr_t>(Ci) : reinterpret_cast<uintptr_t>(Cb);
  const bool vec = Ci ? (ldc % 4 == 0 && c % 16 == 0) : (ldc % 8 == 0 && c % 16 == 0);
  if (Ci) {  // the int32 hook: no column maxima ride along
    if (vec) launch<BM, BN, AK, BKM, true, true>(fast, rebase, grid, M, N, K, A, lda, sa, B, ldb, sb, Ci, ldc, nullptr, stream);
    else launch<BM, BN, AK, BKM, true, false>(fast, rebase, grid, M, N, K, A, lda, sa, B, ldb, sb, Ci, ldc, nullptr, stream);
  } else {
    if (vec) launch<BM, BN, AK, BKM, false, true>(fast, rebase, grid, M, N, K, A, lda, sa, B, ldb, sb, Cb, ldc, side, stream);
    else launch<BM, BN, AK, BKM, false, false>(fast, rebase, grid, M, N, K, A, lda, sa, B, ldb, sb, Cb, ldc, side, stream);
  }
  return hipGetLastError();
}

// Tile choice.  A 256 x 256 tile does four times the work of a 128 x 128
// one at about 1.5x its per-operation rate (fewer LDS and memory bytes per
// MFMA), so 256 x 256 wins whenever its tiles fill at least half the 256 CUs;
// below that the 128 x 128 tiling keeps more CUs busy.  (Measured over the
// Llama-1B and Llama-3-8B layer GEMMs: e.g. 176 big tiles at contraction
// 32768 run in 330 us against 505 us as 704 small tiles.)
constexpr int64_t kBigTileMin = 128;
int64_t big_tiles(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256); }

template <bool AK, bool BKM>
hipError_t pick(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda, const float* sa,
                const int8_t* B, int64_t ldb, const float* sb, uint16_t* Cb, int32_t* Ci,
                int64_t ldc, const ColmaxJob* side, hipStream_t stream) {
  if (big_tiles(M, N) >= kBigTileMin)
    return run<256, 256, AK, BKM>(M, N, K, A, lda, sa, B, ldb, sb, Cb, Ci, ldc, side, stream);
  return run<128, 128, AK, BKM>(M, N, K, A, lda, sa, B, ldb, sb, Cb, Ci, ldc, side, stream);
}

// ---- contraction split (the linear chains) -------------------------------
//
// A problem with fewer 256 x 256 tiles than half the CUs and a long
// contraction (the grad-weight GEMM of a narrow layer contracts over all
// tokens) splits the contraction over `splits` copies of the tile grid, when
// that launches at least as many workgroups as its 128 x 128 tiling would.  Each
// copy writes exact int32 partial sums into its own plane; splitk_reduce adds
// the planes (integer addition: exact and order-free, and every partial sum is
// a sum over a subset of the contraction, bounded like the full one) and
// applies the same fp32 epilogue, so the output is bit-identical to the
// unsplit GEMM's.
constexpr int64_t kSplitMinK = 1024;  // contraction per split, at least

struct SplitPlan {
  int splits;      // 1: no split
  int64_t kchunk;  // contraction per copy (whole 64-deep slabs; the last copy takes the rest)
  int64_t ldp;     // row pitch of a partial plane (int32 elements, multiple of 4)
};

template <bool AK, bool BKM>
SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  SplitPlan p{1, K, 0};
  const int64_t t = big_tiles(M, N);
  if (t >= kBigTileMin || !pipelined_ok<256, 256, AK, BKM>(M, N, K, lda, ldb)) return p;
  int64_t s = std::min<int64_t>(256 / t, K / kSplitMinK);
  if (s < 2) return p;
  int64_t kc = (K + s - 1) / s;
  kc = (kc + BK - 1) / BK * BK;
  s = (K + kc - 1) / kc;  // every copy gets a non-empty range; K % 16 == 0 carries to the last
  // Worth it only with at least as many workgroups as the 128 x 128 tiling
  // would launch (4 t), or a full chip: at 2048^3 (64 tiles, 2 copies) the
  // split chain takes 44 + 116 us against 33 + 88 us on 128 x 128 tiles.
  if (s < 2 || s * t < std::min<int64_t>(256, 4 * t)) return p;
  p.splits = (int)s;
  p.kchunk = kc;
  p.ldp = (N + 3) / 4 * 4;
  return p;
}

size_t plan_bytes(const SplitPlan& p, int64_t M) {
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)p.ldp * 4 : 0;
}

// C[m, n] = bf16_RNE(RN32(RN32(float(sum_s P[s][m][n]) * sa[m]) * sb[n]));
// one thread per 4 adjacent outputs of a row, rows over blockIdx.y.  T =
// int32_t: exact integer partial sums (INT8); T = float: fp32 partial sums
// (FP8), added in fp32 in plane order s = 0, 1, ... (a fixed order, so the
// result does not depend on scheduling).
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce(const T* __restrict__ P, int64_t ldp,
                                                     int64_t plane, int splits, int64_t M,
                                                     int64_t N, const float* __restrict__ sa,
                                                     const float* __restrict__ sb,
                                                     __bf16* __restrict__ C, int64_t ldc) {
  typedef T v4t __attribute__((ext_vector_type(4)));
  const int64_t n = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (n >= N) return;
  const bool vec = ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 8 == 0 && n + 4 <= N;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const T* p = P + m * ldp + n;  // columns up to n + 3 < ldp: inside the plane
    v4t acc = *reinterpret_cast<const v4t*>(p);
#pragma unroll 8
    for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const v4t*>(p + s * plane);
    const float sam = sa[m];
    __bf16 h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float y = (float)acc[e];
      y = y * sam;
      y = y * (n + e < N ? sb[n + e] : 0.0f);
      h[e] = (__bf16)y;  // round to nearest even
    }
    __bf16* row = C + m * ldc;
    if (vec) {
      *reinterpret_cast<uint2*>(row + n) = __builtin_bit_cast(uint2, h);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) row[n + e] = h[e];
    }
  }
}

template <int FMT, bool AK, bool BKM>
hipError_t run_split(const SplitPlan& p, int64_t M, int64_t N, int64_t K, const int8_t* A,
                     int64_t lda, const float* sa, const int8_t* B, int64_t ldb, const float* sb,
                     uint16_t* C, int64_t ldc, void* P, const ColmaxJob* side, hipStream_t stream) {
  // partial planes: int32 sums (INT8) or raw fp32 sums (FP8), 4 bytes either way
  const int64_t tiles = big_tiles(M, N);
  const int64_t plane = M * p.ldp;
  const dim3 grid((unsigned)(tiles * p.splits));
  if (side && !side_fits(*side, tiles * p.splits, 256)) {  // as a launch of its own
    const hipError_t e = launch_colmax_finalize(*side, stream);
    if (e != hipSuccess) return e;
    side = nullptr;
  }
  if (side)
    gemm_i8_pipelined<256, 256, 4, AK, BKM, true, true, FMT, true><<<grid, 512, 0, stream>>>(
        M, N, K, A, lda, nullptr, B, ldb, nullptr, P, p.ldp, p.kchunk, plane, *side);
  else
    gemm_i8_pipelined<256, 256, 4, AK, BKM, true, true, FMT><<<grid, 512, 0, stream>>>(
        M, N, K, A, lda, nullptr, B, ldb, nullptr, P, p.ldp, p.kchunk, plane, ColmaxJob{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 rgrid((unsigned)((N + 1023) / 1024), (unsigned)std::min<int64_t>(M, 65535));
  if constexpr (FMT == 1)
    splitk_reduce<float><<<rgrid, 256, 0, stream>>>(static_cast<const float*>(P), p.ldp, plane, p.splits, M, N, sa, sb,
                                                   reinterpret_cast<__bf16*>(C), ldc);
  else
    splitk_reduce<int32_t><<<rgrid, 256, 0, stream>>>(static_cast<const int32_t*>(P), p.ldp, plane, p.splits, M, N, sa,
                                                     sb, reinterpret_cast<__bf16*>(C), ldc);
  return hipGetLastError();
}

// FP8 GEMM for any shape (the pipelined kernel needs K % 16 == 0, and
// output extents that are multiples of 4 where an operand is read down its
// rows).  The INT8 general kernel's structure (register-staged, byte-masked
// loads into the same swizzled LDS tiles, two slabs in LDS) with the
// pipelined FP8 kernel's fragments and instruction: each 64-deep slab is one
// v_mfma_scale_f32_32x32x64_f8f6f4 per 32 x 32 block with the operands placed
// exactly as there, and slabs are accumulated in the same order, so on shapes
// both kernels take the sums are bit-identical.  Contraction indices past K
// are zero in both operands (a product of two zeros has the smallest
// exponent sum, so it changes no group's truncation step).
template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, bool OUT_F32, bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_f8_general(int64_t M, int64_t N, int64_t K,
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

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = Mma<1>::zero();

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
    v8i af[TM], bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = frag32f8<BM, A_KMAJOR>(cur, wm0 + 32 * i, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = frag32f8<BN, B_KMAJOR>(cur + A_BYTES, wn0 + 32 * j, lane);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = Mma<1>::mma(bf[j], af[i], acc[i][j]);
    if (more) {
      sa_stage.store(nxt, t);
      sb_stage.store(nxt + A_BYTES, t);
    }
    __syncthreads();
  }

  if constexpr (OUT_F32) {  // the raw fp32 sums (C holds floats)
    store32f_raw<TM, TN>(acc, m0, n0, wm0, wn0, M, N, static_cast<float*>(Cv), ldc, lane);
  } else {
    // every wave has passed its last LDS read of the slabs before any scale lands
    __syncthreads();
    float* s_lds = reinterpret_cast<float*>(lds);
    stage_scales<BM, BN, false>(s_lds, m0, n0, M, N, sa, sb, t);
    store32f_direct<BM, TM, TN>(acc, m0, n0, wm0, wn0, M, N, s_lds, static_cast<__bf16*>(Cv), ldc, lane);
  }
}

template <int BM, int BN, bool AK, bool BKM>
hipError_t run_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sa,
                   const uint8_t* B, int64_t ldb, const float* sb, uint16_t* C, float* Cf,
                   int64_t ldc, const ColmaxJob* side, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  constexpr int WGN = BM >= 256 ? 4 : 2;
  const bool vec = ldc % 8 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0;
  const int8_t* a = reinterpret_cast<const int8_t*>(A);
  const int8_t* b = reinterpret_cast<const int8_t*>(B);
  const bool fast = pipelined_ok<BM, BN, AK, BKM>(M, N, K, lda, ldb);
  const bool rebase = !Cf && vec && rebase_ok<BM, BN, AK, BKM>(M, N, K, lda, ldb);
  if (side && (Cf || !(fast && side_fits(*side, tiles, BM)))) {  // as a launch of its own
    const hipError_t e = launch_colmax_finalize(*side, stream);
    if (e != hipSuccess) return e;
    side = nullptr;
  }
  if (rebase) {  // an operand read down its rows spans 2^31 bytes or more
    if constexpr (BM == 256 && !(AK && BKM))
      gemm_i8_pipelined<BM, BN, WGN, AK, BKM, false, true, 1, false, true><<<grid, 128 * WGN, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, C, ldc, K, 0, ColmaxJob{});
  } else if (side && vec) {
    gemm_i8_pipelined<BM, BN, WGN, AK, BKM, false, true, 1, true><<<grid, 128 * WGN, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, C, ldc, K, 0, *side);
  } else if (side) {
    gemm_i8_pipelined<BM, BN, WGN, AK, BKM, false, false, 1, true><<<grid, 128 * WGN, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, C, ldc, K, 0, *side);
  } else if (!fast) {
    if (Cf)
      gemm_f8_general<BM, BN, AK, BKM, true, false><<<grid, kThreads, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, Cf, ldc);
    else
      gemm_f8_general<BM, BN, AK, BKM, false, false><<<grid, kThreads, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, C, ldc);
  } else if (Cf) {
    gemm_i8_pipelined<BM, BN, WGN, AK, BKM, true, false, 1><<<grid, 128 * WGN, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, Cf, ldc, K, 0, ColmaxJob{});
  } else if (vec) {
    gemm_i8_pipelined<BM, BN, WGN, AK, BKM, false, true, 1><<<grid, 128 * WGN, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, C, ldc, K, 0, ColmaxJob{});
  } else {
    gemm_i8_pipelined<BM, BN, WGN, AK, BKM, false, false, 1><<<grid, 128 * WGN, 0, stream>>>(M, N, K, a, lda, sa, b, ldb, sb, C, ldc, K, 0, ColmaxJob{});
  }
  return hipGetLastError();
}

template <bool AK, bool BKM>
hipError_t pick_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sa,
                    const uint8_t* B, int64_t ldb, const float* sb, uint16_t* C, float* Cf,
                    int64_t ldc, const ColmaxJob* side, hipStream_t stream) {
  if (big_tiles(M, N) >= kBigTileMin)
    return run_fp8<256, 256, AK, BKM>(M, N, K, A, lda, sa, B, ldb, sb, C, Cf, ldc, side, stream);
  return run_fp8<128, 128, AK, BKM>(M, N, K, A, lda, sa, B, ldb, sb, C, Cf, ldc, side, stream);
}

}  // namespace

hipError_t launch_gemm_fp8(int layout, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                           int64_t lda, const float* sa, const uint8_t* B, int64_t ldb,
                           const float* sb, uint16_t* C, float* C_f32, int64_t ldc,
                           hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (layout) {
    case 0:
      return pick_fp8<true, true>(M, N, K, A, lda, sa, B, ldb, sb, C, C_f32, ldc, nullptr, stream);
    case 1:
      return pick_fp8<true, false>(M, N, K, A, lda, sa, B, ldb, sb, C, C_f32, ldc, nullptr, stream);
    default:
      return pick_fp8<false, false>(M, N, K, A, lda, sa, B, ldb, sb, C, C_f32, ldc, nullptr, stream);
  }
}

namespace {

SplitPlan plan_for(int layout, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  switch (layout) {
    case 0: return plan_split<true, true>(M, N, K, lda, ldb);
    case 1: return plan_split<true, false>(M, N, K, lda, ldb);
    default: return plan_split<false, false>(M, N, K, lda, ldb);
  }
}

}  // namespace

size_t gemm_split_workspace_bytes(int layout, int64_t M, int64_t N, int64_t K, int64_t lda,
                                  int64_t ldb) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return plan_bytes(plan_for(layout, M, N, K, lda, ldb), M);
}

hipError_t launch_gemm_split(int layout, int64_t M, int64_t N, int64_t K, const int8_t* A,
                             int64_t lda, const float* sa, const int8_t* B, int64_t ldb,
                             const float* sb, uint16_t* C, int64_t ldc, void* ws,
                             const ColmaxJob* side, int fmt, hipStream_t stream) {
  if (side && side->n <= 0) side = nullptr;
  if (M == 0 || N == 0) return side ? launch_colmax_finalize(*side, stream) : hipSuccess;
  const SplitPlan p = K > 0 ? plan_for(layout, M, N, K, lda, ldb) : SplitPlan{1, K, 0};
  const uint8_t* a8 = reinterpret_cast<const uint8_t*>(A);
  const uint8_t* b8 = reinterpret_cast<const uint8_t*>(B);
  if (p.splits < 2 || !ws) {
    if (fmt == 1) {
      switch (layout) {
        case 0: return pick_fp8<true, true>(M, N, K, a8, lda, sa, b8, ldb, sb, C, nullptr, ldc, side, stream);
        case 1: return pick_fp8<true, false>(M, N, K, a8, lda, sa, b8, ldb, sb, C, nullptr, ldc, side, stream);
        default: return pick_fp8<false, false>(M, N, K, a8, lda, sa, b8, ldb, sb, C, nullptr, ldc, side, stream);
      }
    }
    switch (layout) {
      case 0: return pick<true, true>(M, N, K, A, lda, sa, B, ldb, sb, C, nullptr, ldc, side, stream);
      case 1: return pick<true, false>(M, N, K, A, lda, sa, B, ldb, sb, C, nullptr, ldc, side, stream);
      default: return pick<false, false>(M, N, K, A, lda, sa, B, ldb, sb, C, nullptr, ldc, side, stream);
    }
  }
  if (fmt == 1) {
    switch (layout) {
      case 0: return run_split<1, true, true>(p, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, ws, side, stream);
      case 1: return run_split<1, true, false>(p, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, ws, side, stream);
      default: return run_split<1, false, false>(p, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, ws, side, stream);
    }
  }
  switch (layout) {
    case 0: return run_split<0, true, true>(p, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, ws, side, stream);
    case 1: return run_split<0, true, false>(p, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, ws, side, stream);
    default: return run_split<0, false, false>(p, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, ws, side, stream);
  }
}

hipError_t launch_mfma_rate_probe(const int8_t* codes, int64_t bytes, int64_t rounds, int32_t* sink,
                                  hipStream_t stream) {
  const int64_t span = (bytes - 24 * 1024) / 1024 * 1024 + 1024;  // fragment origins a wave may take
  mfma_rate_probe<<<dim3(kMfmaProbeWorkgroups), 512, 0, stream>>>(codes, span, rounds, sink);
  return hipGetLastError();
}

hipError_t launch_gemm(int layout, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                       const float* sa, const int8_t* B, int64_t ldb, const float* sb,
                       uint16_t* C_bf16, int32_t* C_i32, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (layout) {
    case 0:
      return pick<true, true>(M, N, K, A, lda, sa, B, ldb, sb, C_bf16, C_i32, ldc, nullptr, stream);
    case 1:
      return pick<true, false>(M, N, K, A, lda, sa, B, ldb, sb, C_bf16, C_i32, ldc, nullptr, stream);
    default:
      return pick<false, false>(M, N, K, A, lda, sa, B, ldb, sb, C_bf16, C_i32, ldc, nullptr, stream);
  }
}

}  // namespace i8mp
