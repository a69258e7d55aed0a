// Dynamic INT8 quantization kernels for gfx950: row-wise (one scale per row)
// and column-wise (one scale per column), round-half-even or stochastic.
//
// Method ("Quantized model training", section "INT8 mixed precision
// training": dynamic row-wise quantization before each scaled INT8 matmul;
// the quantize step of "Add QAT support for distributed finetuning",
// summary: divide by the scale, round, clamp; zero point 0):
//   scale = RN32(absmax / 127), code = clamp(round(RN32(x / scale)), -127, 127)
// An all-zero group has scale 0 and codes 0.  Stochastic rounding takes
// code = floor(RN32(x/scale + u)), u from Philox4x32-10 at the element's
// logical index.
//
// Both passes are HBM-bound streams: 2 bytes read and 1 byte written per
// element.  Every lane moves 16-byte chunks (8 bf16), a wave covers 1 KiB of
// a row per load, and the absmax is taken on bf16 bit patterns with the sign
// cleared (for non-negative IEEE values bit order is value order, so the
// maximum is exact and order-free).
//
// The quotient x / scale is evaluated as in FMA-based division (Markstein,
// IBM J. Res. Dev. 34(1), 1990): with rcp = RN32(1/scale),
//   q0 = RN(x * rcp); e = fma(-q0, scale, x) (exact); v = RN(fma(e, rcp, q0))
// which equals the IEEE quotient RN32(x/scale) when nothing underflows.  For
// scales below 2^-100 the kernels divide directly instead.  The equality is
// checked on the GPU for every bf16 value against every bf16 absmax.
#include "internal.h"
#include "philox.h"

#include <atomic>
#include <mutex>

namespace i8mp {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;

__device__ __forceinline__ us2 as_us2(uint32_t w) { return __builtin_bit_cast(us2, w); }

// Largest |x| bit pattern among the 8 bf16 of a chunk, kept as two halves.
__device__ __forceinline__ us2 absmax_bits(us2 m, uint4 v) {
  m = __builtin_elementwise_max(m, as_us2(v.x & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, as_us2(v.y & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, as_us2(v.z & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, as_us2(v.w & 0x7FFF7FFFu));
  return m;
}

// Zero the bf16 elements at positions >= n (1 <= n < 8) of a chunk.
__device__ __forceinline__ uint4 keep_first(uint4 v, int n) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lo = 2 * i, hi = 2 * i + 1;
    uint32_t mask = (lo < n ? 0x0000FFFFu : 0u) | (hi < n ? 0xFFFF0000u : 0u);
    w[i] &= mask;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Maximum over the 64 lanes of a wave (all lanes active), the same value in
// every lane.  DPP: within each row of 16 lanes DPP moves combine neighbours
// (quad permutes [1,0,3,2] and [2,3,0,1], then the half-row and row
// mirrors) and the four row maxima are read out with readlane, all in VALU /
// SALU latency; otherwise butterfly shuffles through LDS permutes.  Which is
// faster depends on the kernel (measured at 4096 x 4096: the one-row-per-wave
// pass, at 59 VGPRs and 8 waves per SIMD, runs 0.5 us faster with shuffles;
// the pass with column maxima, at 2-3 waves per SIMD, 0.3 us faster with DPP).
template <bool DPP>
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  if constexpr (!DPP) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    return m;
  }
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
  return max(max(a, b), max(c, d));
}

// Scale of one group and how its quotients are evaluated.
struct GroupScale {
  float s;    // RN32(amax / 127)
  float rcp;  // RN32(1 / s)
  int mode;   // 0: all-zero group, 1: FMA quotient, 2: direct division
};

__device__ __forceinline__ GroupScale scale_from_s(float s) {
  GroupScale g;
  g.s = s;
  if (s == 0.0f) {
    g.rcp = 0.0f;
    g.mode = 0;
  } else if (s >= 0x1p-100f) {
    g.rcp = 1.0f / s;  // IEEE division (correctly rounded)
    g.mode = 1;
  } else {
    g.rcp = 0.0f;
    g.mode = 2;
  }
  return g;
}

// Code formats: 0 = INT8 (codes in [-127, 127]), 1 = FP8 E4M3 (OCP "e4m3fn",
// values in [-448, 448]).  The scale divides amax by the largest code.
template <int FMT>
constexpr float code_max() { return FMT == 1 ? 448.0f : 127.0f; }

// amax is the bit pattern of a non-negative bf16; the scale is
// RN32(amax / code max) (an IEEE division, correctly rounded), 0 only for
// amax = 0.
template <int FMT = 0>
__device__ __forceinline__ GroupScale make_scale(uint32_t amax_bits) {
  return scale_from_s(__uint_as_float(amax_bits << 16) / code_max<FMT>());
}

// Quotient x / s under a known evaluation mode (1: FMA form, 2: division).
template <int MODE>
__device__ __forceinline__ float quotient(float x, float s, float rcp) {
  if constexpr (MODE == 1) {
    const float q0 = x * rcp;
    const float e = __builtin_fmaf(-q0, s, x);
    return __builtin_fmaf(e, rcp, q0);
  } else {
    return x / s;
  }
}

// int8 code of x under scale s with a known mode (1 or 2), in the low byte
// of the result (the upper bytes are not part of the code).
//
// Round half to even: rounding is monotone and +-127 are integers, so
// clamping the quotient first gives the same code.  Adding 1.5 * 2^23 to a
// value in [-127, 127] rounds it to an integer n (ties to even: the added
// constant is even), and the sum's bit pattern is that of 1.5 * 2^23 plus n,
// so its low byte is n in two's complement.
//
// Stochastic rounding: u is the uniform in units of 2^-24 (word_uniform_units);
// u * 2^-24 is exact, so the FMA rounds v + u * 2^-24 once, exactly as the
// addition of the uniform would.
template <bool SR, int MODE>
__device__ __forceinline__ uint32_t code_of(float x, float s, float rcp, float u) {
  const float v = quotient<MODE>(x, s, rcp);
  if constexpr (SR) {
    return (uint32_t)(int)__builtin_amdgcn_fmed3f(floorf(__builtin_fmaf(u, 0x1p-24f, v)), -127.0f, 127.0f);
  } else {
    return __float_as_uint(__builtin_amdgcn_fmed3f(v, -127.0f, 127.0f) + 0x1.8p23f);
  }
}

// Any mode, decided per element (0 gives code 0).
template <bool SR>
__device__ __forceinline__ uint32_t code_any(float x, const GroupScale& g, float u) {
  if (g.mode == 1) return code_of<SR, 1>(x, g.s, g.rcp, u);
  if (g.mode == 2) return code_of<SR, 2>(x, g.s, g.rcp, u);
  return 0;
}

// FP8 value of x under scale s with a known mode (1 or 2): the quotient
// clamped to [-448, 448]; a zero x gives +0 (the FMA form already does: the
// quotient of -0 comes out +0).  v_cvt_pk_fp8_f32 then rounds it to the
// nearest E4M3 value, ties to even.
template <int MODE>
__device__ __forceinline__ float f8_value(float x, float s, float rcp) {
  if constexpr (MODE == 2) {
    if (x == 0.0f) return 0.0f;
  }
  return __builtin_amdgcn_fmed3f(quotient<MODE>(x, s, rcp), -448.0f, 448.0f);
}

__device__ __forceinline__ float f8_any(float x, const GroupScale& g) {
  if (g.mode == 1) return f8_value<1>(x, g.s, g.rcp);
  if (g.mode == 2) return f8_value<2>(x, g.s, g.rcp);
  return 0.0f;
}

// Four E4M3 codes, first value in the lowest byte.
__device__ __forceinline__ uint32_t pack_f8x4(float a, float b, float c, float d) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Low bytes of four words, a's in the lowest byte.
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return (a & 0xFFu) | ((b & 0xFFu) << 8) | ((c & 0xFFu) << 16) | (d << 24);
}

__device__ __forceinline__ float elem(const uint4& v, int j) {
  const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
  return (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}

// Uniforms (in units of 2^-24) of the 8 elements starting at logical index
// e0.  ALIGNED4: e0 is a multiple of 4, so the chunk needs exactly two Philox
// blocks.
template <bool ALIGNED4>
__device__ __forceinline__ void chunk_uniforms(uint64_t seed, uint64_t offset, uint64_t e0,
                                               float u[8]) {
  if constexpr (ALIGNED4) {
    const uint64_t b = offset + (e0 >> 2);
    const u32x4 w0 = philox_block(seed, b);
    const u32x4 w1 = philox_block(seed, b + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u[j] = word_uniform_units(w0.w[j]);
      u[4 + j] = word_uniform_units(w1.w[j]);
    }
  } else {
    // Elements e0 .. e0+7 take words s .. s+7 (s = e0 mod 4) of the three
    // consecutive blocks from block offset + e0 / 4 on.  s is the same in
    // every lane of a wave where the callers call this (e0 = row * cols + a
    // multiple of 8); each element selects among its four candidate words,
    // all at constant indices.
    const uint64_t b = offset + (e0 >> 2);
    const u32x4 w0 = philox_block(seed, b), w1 = philox_block(seed, b + 1), w2 = philox_block(seed, b + 2);
    const uint32_t w[12] = {w0.w[0], w0.w[1], w0.w[2], w0.w[3], w1.w[0], w1.w[1],
                            w1.w[2], w1.w[3], w2.w[0], w2.w[1], w2.w[2], w2.w[3]};
    const uint32_t s = (uint32_t)(e0 & 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t word = s == 0 ? w[j] : s == 1 ? w[j + 1] : s == 2 ? w[j + 2] : w[j + 3];
      u[j] = word_uniform_units(word);
    }
  }
}

// Codes of one chunk.  MODE 1 or 2: every element uses that quotient form
// with scale g[0] (g[j] when PER_ELEM_SCALE); MODE -1: each element's own
// GroupScale decides.  Returns 8 bytes.
template <bool SR, bool ALIGNED4, bool PER_ELEM_SCALE, int MODE, int FMT = 0>
__device__ __forceinline__ uint2 quantize_chunk(const uint4& v, const GroupScale* g,
                                                uint64_t seed, uint64_t offset, uint64_t e0) {
  if constexpr (FMT == 1) {  // FP8: round to nearest only
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const GroupScale& gj = g[PER_ELEM_SCALE ? j : 0];
      if constexpr (MODE < 0)
        f[j] = f8_any(elem(v, j), gj);
      else
        f[j] = f8_value<MODE>(elem(v, j), gj.s, gj.rcp);
    }
    return make_uint2(pack_f8x4(f[0], f[1], f[2], f[3]), pack_f8x4(f[4], f[5], f[6], f[7]));
  }
  float u[8];
  if constexpr (SR) {
    chunk_uniforms<ALIGNED4>(seed, offset, e0, u);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = 0.0f;
  }
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const GroupScale& gj = g[PER_ELEM_SCALE ? j : 0];
    if constexpr (MODE < 0)
      c[j] = code_any<SR>(elem(v, j), gj, u[j]);
    else
      c[j] = code_of<SR, MODE>(elem(v, j), gj.s, gj.rcp, u[j]);
  }
  return make_uint2(pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7]));
}

__device__ __forceinline__ void store_partial(int8_t* dst, uint2 codes, int n) {
  const uint64_t all = ((uint64_t)codes.y << 32) | codes.x;
  for (int j = 0; j < n; ++j) dst[j] = (int8_t)(all >> (8 * j));
}

// ---------------------------------------------------------------------------
// Row-wise, one wave per row: the row stays in registers between the absmax
// and the quantize sweep, so it is read from HBM once.  NV chunks per lane
// cover rows of up to NV * 512 elements.  Waves walk rows with a grid stride;
// with PREFETCH the next row's loads are in flight while the current row is
// reduced, quantized and stored.  FULL: the row is exactly NV * 512 elements,
// so no chunk needs a range check.

template <int NV, bool FULL = false>
__device__ __forceinline__ void load_row(uint4 (&v)[NV], const uint16_t* __restrict__ xr,
                                         int64_t cols, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t c0 = (int64_t)(i * 64 + lane) * 8;
    if (FULL || c0 < cols) {
      v[i] = *reinterpret_cast<const uint4*>(xr + c0);
      if (!FULL && c0 + 8 > cols) v[i] = keep_first(v[i], (int)(cols - c0));
    } else {
      v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <int NV, bool SR, bool ALIGNED4, int MODE, int FMT = 0, bool FULL = false>
__device__ __forceinline__ void quantize_row_mode(const uint4 (&v)[NV], const GroupScale& g,
                                                  int64_t r, int64_t cols, int8_t* __restrict__ qr,
                                                  uint64_t seed, uint64_t offset, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t c0 = (int64_t)(i * 64 + lane) * 8;
    if (FULL || c0 < cols) {
      uint2 codes = make_uint2(0, 0);
      if constexpr (MODE > 0)
        codes = quantize_chunk<SR, ALIGNED4, false, MODE, FMT>(v[i], &g, seed, offset, (uint64_t)(r * cols + c0));
      if (FULL || c0 + 8 <= cols)
        *reinterpret_cast<uint2*>(qr + c0) = codes;
      else
        store_partial(qr + c0, codes, (int)(cols - c0));
    }
    // Under stochastic rounding, one chunk's Philox blocks at a time: left
    // free, the scheduler starts the next chunks' blocks early and the live
    // words of several chunks push the register count past 128.
    if constexpr (SR && MODE > 0) __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NV, bool SR, bool ALIGNED4, int FMT = 0, bool FULL = false, bool DPP = false>
__device__ __forceinline__ void quantize_row(const uint4 (&v)[NV], int64_t r, int64_t cols,
                                             int8_t* __restrict__ q, int64_t ldq,
                                             float* __restrict__ scale, uint64_t seed,
                                             uint64_t offset, int lane) {
  us2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < NV; ++i) m2 = absmax_bits(m2, v[i]);
  // the row maximum is the same in every lane: read it from lane 0 so the
  // mode branch below is a scalar branch
  const uint32_t amax = __builtin_amdgcn_readfirstlane(wave_max_u32<DPP>(max((uint32_t)m2.x, (uint32_t)m2.y)));
  const GroupScale g = make_scale<FMT>(amax);
  if (lane == 0) scale[r] = g.s;
  int8_t* qr = q + r * ldq;
  if (g.mode == 1)
    quantize_row_mode<NV, SR, ALIGNED4, 1, FMT, FULL>(v, g, r, cols, qr, seed, offset, lane);
  else if (g.mode == 2)
    quantize_row_mode<NV, SR, ALIGNED4, 2, FMT, FULL>(v, g, r, cols, qr, seed, offset, lane);
  else
    quantize_row_mode<NV, SR, ALIGNED4, 0, FMT, FULL>(v, g, r, cols, qr, seed, offset, lane);
}

template <int NV, bool SR, bool ALIGNED4, bool PREFETCH, int FMT = 0, bool FULL = false>
__global__ __launch_bounds__(kThreads) void quant_rows_wave(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint64_t seed, uint64_t offset) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
  int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (r >= rows) return;
  uint4 v[NV];
  load_row<NV, FULL>(v, x + r * ldx, cols, lane);
  for (; r < rows; r += stride) {
    const int64_t rn = r + stride;
    if constexpr (PREFETCH) {
      uint4 nv[NV];
      if (rn < rows) load_row<NV, FULL>(nv, x + rn * ldx, cols, lane);
      quantize_row<NV, SR, ALIGNED4, FMT, FULL>(v, r, cols, q, ldq, scale, seed, offset, lane);
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = nv[i];
    } else {
      quantize_row<NV, SR, ALIGNED4, FMT, FULL>(v, r, cols, q, ldq, scale, seed, offset, lane);
      if (rn < rows) load_row<NV, FULL>(v, x + rn * ldx, cols, lane);
    }
  }
}

// Row-wise, one block per row, for rows longer than a wave holds: an absmax
// sweep, then a quantize sweep that re-reads the row (from L2 / MALL).
template <bool SR, bool ALIGNED4, int FMT = 0>
__global__ __launch_bounds__(kThreads) void quant_rows_block(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint64_t seed, uint64_t offset) {
  __shared__ uint32_t red[kWavesPerBlock];
  const int64_t r = blockIdx.x;
  const uint16_t* xr = x + r * ldx;
  const int64_t nchunks = (cols + 7) / 8;
  us2 m2 = {0, 0};
  constexpr int U = 4;
  for (int64_t base = threadIdx.x; base < nchunks; base += (int64_t)kThreads * U) {
    uint4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t ch = base + (int64_t)k * kThreads;
      v[k] = ch < nchunks ? *reinterpret_cast<const uint4*>(xr + ch * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t ch = base + (int64_t)k * kThreads;
      if (ch * 8 + 8 > cols && ch < nchunks) v[k] = keep_first(v[k], (int)(cols - ch * 8));
      m2 = absmax_bits(m2, v[k]);
    }
  }
  uint32_t m = wave_max_u32<false>(max((uint32_t)m2.x, (uint32_t)m2.y));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) m = max(m, red[w]);
  const GroupScale g = make_scale<FMT>(__builtin_amdgcn_readfirstlane(m));
  if (threadIdx.x == 0) scale[r] = g.s;
  int8_t* qr = q + r * ldq;
  for (int64_t ch = threadIdx.x; ch < nchunks; ch += kThreads) {
    const int64_t c0 = ch * 8;
    uint4 v = *reinterpret_cast<const uint4*>(xr + c0);
    const uint2 codes =
        g.mode == 1 ? quantize_chunk<SR, ALIGNED4, false, 1, FMT>(v, &g, seed, offset, (uint64_t)(r * cols + c0))
                    : quantize_chunk<SR, ALIGNED4, false, -1, FMT>(v, &g, seed, offset, (uint64_t)(r * cols + c0));
    if (c0 + 8 <= cols)
      *reinterpret_cast<uint2*>(qr + c0) = codes;
    else
      store_partial(qr + c0, codes, (int)(cols - c0));
  }
}

// ---------------------------------------------------------------------------
// Column-wise, two passes.  A column tile is 512 columns: each lane owns 8
// adjacent columns and the 8 waves of a block walk rows.  Pass 1 writes the
// column maxima of each slab of rows (as bf16 bit patterns) to the
// workspace.  Pass 2 starts every block by reducing the slab maxima of its
// column tile into the scales (each block of a tile does this; the first row
// block stores them), then quantizes its rows.

constexpr int kColTile = 512;
constexpr int kColThreads = 512;
constexpr int kColWaves = kColThreads / 64;
constexpr int kColMaxSlabs = 32;
constexpr int kColLoads = 16;  // rows in flight per wave

__device__ __forceinline__ void max_chunk(us2 (&m)[4], uint4 v) {
  m[0] = __builtin_elementwise_max(m[0], as_us2(v.x & 0x7FFF7FFFu));
  m[1] = __builtin_elementwise_max(m[1], as_us2(v.y & 0x7FFF7FFFu));
  m[2] = __builtin_elementwise_max(m[2], as_us2(v.z & 0x7FFF7FFFu));
  m[3] = __builtin_elementwise_max(m[3], as_us2(v.w & 0x7FFF7FFFu));
}

__device__ __forceinline__ uint4 pack_max(const us2 (&m)[4]) {
  return make_uint4(__builtin_bit_cast(uint32_t, m[0]), __builtin_bit_cast(uint32_t, m[1]),
                    __builtin_bit_cast(uint32_t, m[2]), __builtin_bit_cast(uint32_t, m[3]));
}

// Elementwise maximum of the per-wave partial maxima in red (every wave
// computes it; the caller has synchronized after the writes).
__device__ __forceinline__ void reduce_waves(us2 (&m)[4], const uint4 (*red)[64], int lane) {
#pragma unroll
  for (int w = 0; w < kColWaves; ++w) {
    const uint4 o = red[w][lane];
    m[0] = __builtin_elementwise_max(m[0], as_us2(o.x));
    m[1] = __builtin_elementwise_max(m[1], as_us2(o.y));
    m[2] = __builtin_elementwise_max(m[2], as_us2(o.z));
    m[3] = __builtin_elementwise_max(m[3], as_us2(o.w));
  }
}

__global__ __launch_bounds__(kColThreads) void col_absmax_partial(const uint16_t* __restrict__ x,
                                                                  int64_t rows, int64_t cols,
                                                                  int64_t ldx, int64_t rows_per_slab,
                                                                  uint16_t* __restrict__ part,
                                                                  int64_t part_ld) {
  __shared__ uint4 red[kColWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kColTile + lane * 8;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_slab;
  const int64_t r_end = min(rows, r_begin + rows_per_slab);
  us2 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  if (c0 < cols) {
    const bool tail = c0 + 8 > cols;
    const int ntail = (int)(cols - c0);
    constexpr int U = kColLoads;
    int64_t r = r_begin + wave;
    for (; r + (U - 1) * kColWaves < r_end; r += U * kColWaves) {
      uint4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k)
        v[k] = *reinterpret_cast<const uint4*>(x + (r + k * kColWaves) * ldx + c0);
#pragma unroll
      for (int k = 0; k < U; ++k) max_chunk(m, tail ? keep_first(v[k], ntail) : v[k]);
    }
    for (; r < r_end; r += kColWaves) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + r * ldx + c0);
      max_chunk(m, tail ? keep_first(v, ntail) : v);
    }
  }
  red[wave][lane] = pack_max(m);
  __syncthreads();
  if (wave == 0 && c0 < cols) {
    reduce_waves(m, red, lane);
    *reinterpret_cast<uint4*>(part + (int64_t)blockIdx.y * part_ld + c0) = pack_max(m);
  }
}

// Pass 2 of the two-pass column quantize: a block is rows_per_block rows of
// one column tile, its waves interleaved over the rows; it starts by reducing
// the tile's slab maxima (at most kColMaxSlabs slabs) into the scales.
template <bool SR, bool ALIGNED4, int FMT = 0>
__global__ __launch_bounds__(kColThreads) void quant_cols(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ldx,
                                                          int64_t rows_per_block,
                                                          const uint16_t* __restrict__ part,
                                                          int64_t part_ld, int64_t slabs,
                                                          float* __restrict__ scale,
                                                          int8_t* __restrict__ q, int64_t ldq,
                                                          uint64_t seed, uint64_t offset) {
  __shared__ uint4 red[kColWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // row blocks run last-to-first, so the rows pass 1 touched last (still in
  // L2 / MALL) are read first
  const int64_t r_begin = ((int64_t)gridDim.y - 1 - blockIdx.y) * rows_per_block;
  const int64_t r_end = min(rows, r_begin + rows_per_block);
  int64_t r0 = r_begin + wave;
  const int64_t c0 = (int64_t)blockIdx.x * kColTile + lane * 8;
  const bool active = c0 < cols;
  // Loads carry no branches: lanes past the last column read column 0 and
  // rows past the block's end read its last row (values never used), so
  // each wait for a value covers only the loads issued before it.  The slab
  // maxima go out first and are ready while the rows still arrive.
  const int64_t cl = active ? c0 : 0;
  constexpr int kSlabLoads = kColMaxSlabs / kColWaves;
  uint4 pv[kSlabLoads];
  {
    // the workspace holds at least one slab; a slab read twice leaves the
    // maximum unchanged
    const int64_t s_last = max(slabs, (int64_t)1) - 1;
#pragma unroll
    for (int i = 0; i < kSlabLoads; ++i)
      pv[i] = *reinterpret_cast<const uint4*>(part + min((int64_t)(wave + i * kColWaves), s_last) * part_ld + cl);
  }
  GroupScale g[8];
  const int nvalid = active ? (int)min((int64_t)8, cols - c0) : 0;
  auto make_scales = [&]() {
    us2 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
    if (slabs > 0) {
#pragma unroll
      for (int i = 0; i < kSlabLoads; ++i) max_chunk(m, pv[i]);
    }
    red[wave][lane] = pack_max(m);
    __syncthreads();
    reduce_waves(m, red, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t bits = j & 1 ? m[j >> 1].y : m[j >> 1].x;
      g[j] = make_scale<FMT>(j < nvalid ? bits : 0u);
    }
    if (blockIdx.y == 0 && wave == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < nvalid) scale[c0 + j] = g[j].s;
    }
  };
  if (r_end <= r_begin) {  // no rows: only the (zero) scales are stored
    make_scales();
    return;
  }
  constexpr int U = SR ? kColLoads / 2 : kColLoads;  // SR's Philox state needs the registers
  uint4 v[U];
  auto load_rows = [&](int64_t first) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t r = first + (int64_t)k * kColWaves;
      v[k] = *reinterpret_cast<const uint4*>(x + min(r, r_end - 1) * ldx + cl);
    }
  };
  load_rows(r0);
  make_scales();
  if (!active) return;
  // almost always every column of the wave takes the FMA quotient: then no
  // per-element mode test is needed (padding columns give zero codes that are
  // never stored)
  bool mine = true;
#pragma unroll
  for (int j = 0; j < 8; ++j) mine = mine && (j >= nvalid || g[j].mode == 1);
  const bool all_fma = __all(mine);
  for (; r0 < r_end; r0 += (int64_t)U * kColWaves) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t r = r0 + (int64_t)k * kColWaves;
      if (r >= r_end) break;
      const uint64_t e0 = (uint64_t)(r * cols + c0);
      const uint2 codes = all_fma ? quantize_chunk<SR, ALIGNED4, true, 1, FMT>(v[k], g, seed, offset, e0)
                                  : quantize_chunk<SR, ALIGNED4, true, -1, FMT>(v[k], g, seed, offset, e0);
      int8_t* dst = q + r * ldq + c0;
      if (nvalid == 8)
        *reinterpret_cast<uint2*>(dst) = codes;
      else
        store_partial(dst, codes, nvalid);
    }
    const int64_t rn = r0 + (int64_t)U * kColWaves;
    if (rn < r_end) load_rows(rn);
  }
}

// Column-wise with the column maxima given (fp32, one per column).  A block is
// a band of kColBand consecutive rows (blockIdx.x) across kColWaves column
// tiles (blockIdx.y), one 512-column tile per wave, so each block reads one
// contiguous stretch of the tensor.  Measured at 4096 x 4096 on MI355X: bands
// of 4-16 rows run 10.7-11.5 us, against 16.1 us for blocks of 128 rows of
// one tile; the many small blocks keep more waves per CU busy converting
// while the rows arrive.  A wave whose band and tile are whole takes a body
// without range checks (FULL); the ragged edges take the checked one.
constexpr int kColBand = 8;

template <bool FULL, bool SR, bool ALIGNED4, int FMT>
__device__ __forceinline__ void given_band(const uint16_t* __restrict__ x, int64_t cols, int64_t ldx,
                                           const float* __restrict__ colmax,
                                           float* __restrict__ scale, int8_t* __restrict__ q,
                                           int64_t ldq, uint64_t seed, uint64_t offset,
                                           int64_t r_begin, int64_t nrows, int64_t c0,
                                           bool store_scales) {
  const bool active = FULL || c0 < cols;
  const int64_t cl = active ? c0 : 0;  // lanes past the last column read column 0
  uint4 v[kColBand];
  if (FULL || nrows > 0) {
#pragma unroll
    for (int k = 0; k < kColBand; ++k) {
      const int64_t r = r_begin + (FULL ? k : min((int64_t)k, nrows - 1));
      v[k] = *reinterpret_cast<const uint4*>(x + r * ldx + cl);
    }
  }
  float cm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cm[j] = colmax[FULL ? c0 + j : min(c0 + j, cols - 1)];
  const int nvalid = FULL ? 8 : (active ? (int)min((int64_t)8, cols - c0) : 0);
  GroupScale g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) g[j] = scale_from_s(j < nvalid ? cm[j] / code_max<FMT>() : 0.0f);
  if (store_scales) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < nvalid) scale[c0 + j] = g[j].s;
  }
  if (!active) return;
  bool mine = true;
#pragma unroll
  for (int j = 0; j < 8; ++j) mine = mine && (j >= nvalid || g[j].mode == 1);
  const bool all_fma = __all(mine);
#pragma unroll
  for (int k = 0; k < kColBand; ++k) {
    if (!FULL && k >= nrows) break;
    const int64_t r = r_begin + k;
    const uint64_t e0 = (uint64_t)(r * cols + c0);
    const uint2 codes = all_fma ? quantize_chunk<SR, ALIGNED4, true, 1, FMT>(v[k], g, seed, offset, e0)
                                : quantize_chunk<SR, ALIGNED4, true, -1, FMT>(v[k], g, seed, offset, e0);
    int8_t* dst = q + r * ldq + c0;
    if (FULL || nvalid == 8)
      *reinterpret_cast<uint2*>(dst) = codes;
    else
      store_partial(dst, codes, nvalid);
  }
}

template <bool SR, bool ALIGNED4, int FMT>
__device__ __forceinline__ void cols_given_block(const uint16_t* __restrict__ x, int64_t rows,
                                                 int64_t cols, int64_t ldx,
                                                 const float* __restrict__ colmax,
                                                 float* __restrict__ scale, int8_t* __restrict__ q,
                                                 int64_t ldq, uint64_t seed, uint64_t offset,
                                                 int64_t band, int64_t group) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = group * kColWaves + (threadIdx.x >> 6);
  if (tile * kColTile >= cols) return;  // a wave past the last tile
  const int64_t c0 = tile * kColTile + lane * 8;
  const int64_t r_begin = band * kColBand;
  const int64_t nrows = min((int64_t)kColBand, rows - r_begin);  // 0 only when rows == 0
  const bool store_scales = band == 0;
  if (nrows == kColBand && (tile + 1) * kColTile <= cols)
    given_band<true, SR, ALIGNED4, FMT>(x, cols, ldx, colmax, scale, q, ldq, seed, offset, r_begin,
                                        nrows, c0, store_scales);
  else
    given_band<false, SR, ALIGNED4, FMT>(x, cols, ldx, colmax, scale, q, ldq, seed, offset, r_begin,
                                         nrows, c0, store_scales);
}

template <bool SR, bool ALIGNED4, int FMT = 0>
__global__ __launch_bounds__(kColThreads) void quant_cols_given(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    const float* __restrict__ colmax, float* __restrict__ scale, int8_t* __restrict__ q,
    int64_t ldq, uint64_t seed, uint64_t offset) {
  cols_given_block<SR, ALIGNED4, FMT>(x, rows, cols, ldx, colmax, scale, q, ldq, seed, offset,
                                      blockIdx.x, blockIdx.y);
}

// Two tensors in one launch (a linear layer's grad-weight GEMM quantizes dY
// and X column-wise): blockIdx.x in [0, a.blocks) takes a's row bands, the
// rest b's, kPairBands consecutive bands per block (a pair has twice the
// blocks of one tensor and at 84 VGPRs only two blocks fit per CU, so one
// band per block would run in two rounds); blockIdx.y walks the column groups
// of the wider of the two (waves past a tensor's last column tile return).
// Results as two separate launches.
constexpr int kPairBands = 2;

struct ColGivenJob {
  const uint16_t* x;
  int64_t rows, cols, ldx;
  const float* colmax;
  float* scale;
  int8_t* q;
  int64_t ldq;
  uint64_t offset;
  int64_t bands, blocks;
};

template <bool SR, bool ALIGNED4, int FMT = 0>
__global__ __launch_bounds__(kColThreads) void quant_cols_given2(ColGivenJob a, ColGivenJob b,
                                                                 uint64_t seed) {
  const bool second = (int64_t)blockIdx.x >= a.blocks;
  const ColGivenJob j = second ? b : a;
  const int64_t band0 = (second ? (int64_t)blockIdx.x - a.blocks : (int64_t)blockIdx.x) * kPairBands;
  const int64_t band_end = min(band0 + kPairBands, j.bands);
  for (int64_t band = band0; band < band_end; ++band)
    cols_given_block<SR, ALIGNED4, FMT>(j.x, j.rows, j.cols, j.ldx, j.colmax, j.scale, j.q, j.ldq, seed,
                                        j.offset, band, blockIdx.y);
}

// ---------------------------------------------------------------------------
// Row-wise with column maxima.  A block of WAVES waves owns a band of
// rows_per_block rows; wave w quantizes rows band + w, band + w + WAVES, ...
// exactly as quant_rows_wave does.  Each wave also keeps the running maximum
// of |x| of every column in its own LDS region (lane l's chunk i covers
// columns 8 (64 i + l) .. + 7; one 16-byte read-modify-write per chunk and
// row, so the row in registers is all the per-lane state).  At the end the
// block folds its waves' regions and writes one slab of column maxima (bf16
// bit patterns) to the workspace; colmax_finalize reduces the slabs.  So the
// row-wise pass of a tensor also yields what its column-wise pass needs,
// without a second read of the tensor.

template <int NV, int WAVES, bool SR, bool ALIGNED4, bool FULL, int FMT = 0>
__device__ __forceinline__ void rows_colmax_band(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint64_t seed, uint64_t offset, int64_t rows_per_block,
    uint16_t* __restrict__ part, int64_t part_ld, int64_t band, uint4 (*cm)[NV * 64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r_begin = band * rows_per_block;
  const int64_t r_end = min(rows, r_begin + rows_per_block);
#pragma unroll
  for (int i = 0; i < NV; ++i) cm[wave][i * 64 + lane] = make_uint4(0, 0, 0, 0);
  uint4 v[NV];
  int64_t r = r_begin + wave;
  if (r < r_end) load_row<NV, FULL>(v, x + r * ldx, cols, lane);
  for (; r < r_end; r += WAVES) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {  // load_row zeroed the columns past the end
      us2 m[4];
      const uint4 o = cm[wave][i * 64 + lane];
      m[0] = as_us2(o.x), m[1] = as_us2(o.y), m[2] = as_us2(o.z), m[3] = as_us2(o.w);
      max_chunk(m, v[i]);
      cm[wave][i * 64 + lane] = pack_max(m);
    }
    quantize_row<NV, SR, ALIGNED4, FMT, FULL, true>(v, r, cols, q, ldq, scale, seed, offset, lane);
    const int64_t rn = r + WAVES;
    if (rn < r_end) load_row<NV, FULL>(v, x + rn * ldx, cols, lane);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < NV * 64; j += 64 * WAVES) {
    const int64_t c0 = (int64_t)j * 8;
    if (c0 >= cols) continue;
    us2 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
#pragma unroll
    for (int w = 0; w < WAVES; ++w) max_chunk(m, cm[w][j]);
    *reinterpret_cast<uint4*>(part + band * part_ld + c0) = pack_max(m);
  }
}

template <int NV, int WAVES, bool SR, bool ALIGNED4, bool FULL = false, int FMT = 0>
__global__ __launch_bounds__(64 * WAVES) void quant_rows_colmax(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, uint64_t seed, uint64_t offset, int64_t rows_per_block,
    uint16_t* __restrict__ part, int64_t part_ld) {
  __shared__ uint4 cm[WAVES][NV * 64];
  rows_colmax_band<NV, WAVES, SR, ALIGNED4, FULL, FMT>(x, rows, cols, ldx, q, ldq, scale, seed, offset,
                                                       rows_per_block, part, part_ld, blockIdx.x, cm);
}

// Two tensors of the same width in one launch (a linear layer's forward
// quantizes X and W, both along K): blocks [0, a.slabs) take a's bands, the
// rest b's.  Each tensor keeps its own rows, pitches, outputs, Philox offset
// and slab maxima, so the results are those of two separate launches.
struct RowColmaxJob {
  const uint16_t* x;
  int64_t rows, ldx;
  int8_t* q;
  int64_t ldq;
  float* scale;
  uint64_t offset;
  int64_t rows_per_block, slabs;
  uint16_t* part;
};

template <int NV, int WAVES, bool SR, bool ALIGNED4, bool FULL = false, int FMT = 0>
__global__ __launch_bounds__(64 * WAVES) void quant_rows_colmax2(RowColmaxJob a, RowColmaxJob b,
                                                                 int64_t cols, int64_t part_ld,
                                                                 uint64_t seed) {
  __shared__ uint4 cm[WAVES][NV * 64];
  const bool second = (int64_t)blockIdx.x >= a.slabs;
  const RowColmaxJob j = second ? b : a;
  const int64_t band = second ? (int64_t)blockIdx.x - a.slabs : (int64_t)blockIdx.x;
  rows_colmax_band<NV, WAVES, SR, ALIGNED4, FULL, FMT>(j.x, j.rows, cols, j.ldx, j.q, j.ldq, j.scale, seed,
                                                       j.offset, j.rows_per_block, j.part, part_ld, band, cm);
}

// A row pass with slab maxima (tensor a) and a column pass with its column
// maxima given (tensor b) in one launch: the grad-input GEMM of a linear
// layer needs dY row-wise and W column-wise, two independent passes over
// different tensors.  Blocks [0, a.slabs) take a's bands exactly as
// quant_rows_colmax2 does (8 waves, the same bands and slabs); the rest take
// b's row bands kPairBands at a time, column group (blockIdx.x - a.slabs) %
// b_groups, as quant_cols_given2 does.  At NV <= 8 the LDS (8 x NV KiB) lets
// two blocks share a CU, so the two passes overlap instead of following one
// another.  Results as the two separate launches.
template <int NV, bool SR, bool ALIGNED4, bool FULL = false, int FMT = 0>
__global__ __launch_bounds__(kColThreads) void quant_rows_cols_pair(RowColmaxJob a, int64_t a_cols,
                                                                    int64_t part_ld, ColGivenJob b,
                                                                    int64_t b_groups, uint64_t seed) {
  static_assert(kColThreads == 64 * 8, "both halves run 8 waves");
  __shared__ uint4 cm[8][NV * 64];
  if ((int64_t)blockIdx.x < a.slabs) {
    rows_colmax_band<NV, 8, SR, ALIGNED4, FULL, FMT>(a.x, a.rows, a_cols, a.ldx, a.q, a.ldq, a.scale, seed,
                                                     a.offset, a.rows_per_block, a.part, part_ld, blockIdx.x, cm);
    return;
  }
  const int64_t i = (int64_t)blockIdx.x - a.slabs;
  const int64_t group = i % b_groups;
  const int64_t band0 = i / b_groups * kPairBands;
  const int64_t band_end = min(band0 + kPairBands, b.bands);
  for (int64_t band = band0; band < band_end; ++band)
    cols_given_block<SR, ALIGNED4, FMT>(b.x, b.rows, b.cols, b.ldx, b.colmax, b.scale, b.q, b.ldq, seed, b.offset,
                                        band, group);
}

// Row-wise with column maxima for rows longer than 14336 elements (a row no
// longer fits in one wave's registers).  The tensor is cut into tiles of a
// band of rows by a segment of kLongSeg columns; a block of 8 waves walks the
// band's rows, one row segment per wave at a time (8 chunks per lane).
// rows_long_stats reads each tile once and writes the absmax of every row
// segment (bf16 bit patterns, [rows][segments]) and the band's column maxima
// (one slab per band, as quant_rows_colmax does).  rows_long_quant reads the
// tile again, takes each row's absmax as the maximum of its segment maxima
// (order-free, so exact) and quantizes with the same arithmetic as every other
// row-wise pass.  Two reads of the tensor instead of three (row absmax, row
// quantize, column maxima).
constexpr int kLongSeg = 4096;
constexpr int kLongThreads = 512;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kLongNV = kLongSeg / 512;  // 16-byte chunks per lane and row segment

__device__ __forceinline__ void load_segment(uint4 (&v)[kLongNV], const uint16_t* __restrict__ xr,
                                             int64_t c_begin, int64_t cols, int lane) {
#pragma unroll
  for (int i = 0; i < kLongNV; ++i) {
    const int64_t c0 = c_begin + (int64_t)(i * 64 + lane) * 8;
    if (c0 < cols) {
      v[i] = *reinterpret_cast<const uint4*>(xr + c0);
      if (c0 + 8 > cols) v[i] = keep_first(v[i], (int)(cols - c0));
    } else {
      v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kLongThreads) void rows_long_stats(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int64_t rows_per_band,
    uint16_t* __restrict__ segmax, int64_t nseg, uint16_t* __restrict__ part, int64_t part_ld) {
  __shared__ uint4 red[kLongWaves][kLongNV * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seg = blockIdx.x, band = blockIdx.y;
  const int64_t c_begin = seg * kLongSeg;
  const int64_t r_begin = band * rows_per_band;
  const int64_t r_end = min(rows, r_begin + rows_per_band);
  us2 cm[kLongNV][4];
#pragma unroll
  for (int i = 0; i < kLongNV; ++i) cm[i][0] = cm[i][1] = cm[i][2] = cm[i][3] = us2{0, 0};
  for (int64_t r = r_begin + wave; r < r_end; r += kLongWaves) {
    uint4 v[kLongNV];
    load_segment(v, x + r * ldx, c_begin, cols, lane);
    us2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < kLongNV; ++i) {
      m2 = absmax_bits(m2, v[i]);
      max_chunk(cm[i], v[i]);
    }
    const uint32_t amax = wave_max_u32<false>(max((uint32_t)m2.x, (uint32_t)m2.y));
    if (lane == 0) segmax[r * nseg + seg] = (uint16_t)amax;
  }
#pragma unroll
  for (int i = 0; i < kLongNV; ++i) red[wave][i * 64 + lane] = pack_max(cm[i]);
  __syncthreads();
  // one chunk of the segment per thread: fold the 8 waves, write the band's slab
  const int j = threadIdx.x;
  const int64_t c0 = c_begin + (int64_t)j * 8;
  if (c0 < cols) {
    us2 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
#pragma unroll
    for (int w = 0; w < kLongWaves; ++w) max_chunk(m, red[w][j]);
    *reinterpret_cast<uint4*>(part + band * part_ld + c0) = pack_max(m);
  }
}

template <bool SR, bool ALIGNED4>
__global__ __launch_bounds__(kLongThreads) void rows_long_quant(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int64_t rows_per_band,
    const uint16_t* __restrict__ segmax, int64_t nseg, int8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ scale, uint64_t seed, uint64_t offset) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seg = blockIdx.x, band = blockIdx.y;
  const int64_t c_begin = seg * kLongSeg;
  const int64_t r_begin = band * rows_per_band;
  const int64_t r_end = min(rows, r_begin + rows_per_band);
  for (int64_t r = r_begin + wave; r < r_end; r += kLongWaves) {
    uint4 v[kLongNV];
    load_segment(v, x + r * ldx, c_begin, cols, lane);
    uint32_t m = 0;
    for (int64_t k = lane; k < nseg; k += 64) m = max(m, (uint32_t)segmax[r * nseg + k]);
    const GroupScale g = make_scale<0>(__builtin_amdgcn_readfirstlane(wave_max_u32<false>(m)));
    if (seg == 0 && lane == 0) scale[r] = g.s;
    int8_t* qr = q + r * ldq;
#pragma unroll
    for (int i = 0; i < kLongNV; ++i) {
      const int64_t c0 = c_begin + (int64_t)(i * 64 + lane) * 8;
      if (c0 >= cols) continue;
      const uint64_t e0 = (uint64_t)(r * cols + c0);
      const uint2 codes = g.mode == 1 ? quantize_chunk<SR, ALIGNED4, false, 1>(v[i], &g, seed, offset, e0)
                                      : quantize_chunk<SR, ALIGNED4, false, -1>(v[i], &g, seed, offset, e0);
      if (c0 + 8 <= cols)
        *reinterpret_cast<uint2*>(qr + c0) = codes;
      else
        store_partial(qr + c0, codes, (int)(cols - c0));
    }
  }
}

// fp32 column maxima from slab maxima.  A block of 8 waves covers 32
// columns: lane l reads the 16-byte chunk l % 4 (8 columns) of slab l / 4 of
// each group of 16 slabs, so one load instruction of a wave covers 16 slabs;
// wave w takes slab groups w, w + 8, ...  Each lane's first two loads go out
// together.  The 16 lanes sharing a chunk, then the 8 waves, are folded.
constexpr int kFinThreads = 512;
constexpr int kFinWaves = kFinThreads / 64;

__device__ __forceinline__ void finalize_block_at(const uint16_t* __restrict__ part, int64_t part_ld,
                                                  int64_t slabs, int64_t cols,
                                                  float* __restrict__ colmax, uint4 (*red)[4],
                                                  int64_t group) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = lane & 3, sub = lane >> 2;
  const int64_t c0 = group * 32 + chunk * 8;
  us2 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  if (c0 < cols) {
    constexpr int64_t step = (int64_t)kFinWaves * 16;
    const int64_t s0 = (int64_t)wave * 16 + sub;
    uint4 v[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t s = s0 + k * step;
      v[k] = s < slabs ? *reinterpret_cast<const uint4*>(part + s * part_ld + c0) : make_uint4(0, 0, 0, 0);
    }
    max_chunk(m, v[0]);
    max_chunk(m, v[1]);
    for (int64_t s = s0 + 2 * step; s < slabs; s += step)
      max_chunk(m, *reinterpret_cast<const uint4*>(part + s * part_ld + c0));
  }
  // fold the 16 lanes of each chunk (lanes chunk, chunk + 4, ..., chunk + 60)
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t o = (uint32_t)__shfl_xor((int)__builtin_bit_cast(uint32_t, m[k]), off);
      m[k] = __builtin_elementwise_max(m[k], as_us2(o));
    }
  }
  if (sub == 0) red[wave][chunk] = pack_max(m);
  __syncthreads();
  if (wave == 0 && sub == 0 && c0 < cols) {
#pragma unroll
    for (int w = 1; w < kFinWaves; ++w) max_chunk(m, red[w][chunk]);
    const uint32_t b[8] = {m[0].x, m[0].y, m[1].x, m[1].y, m[2].x, m[2].y, m[3].x, m[3].y};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < cols) colmax[c0 + j] = __uint_as_float(b[j] << 16);
  }
}

__device__ __forceinline__ void finalize_block(const uint16_t* __restrict__ part, int64_t part_ld,
                                               int64_t slabs, int64_t cols,
                                               float* __restrict__ colmax, uint4 (*red)[4]) {
  finalize_block_at(part, part_ld, slabs, cols, colmax, red, blockIdx.x);
}

__global__ __launch_bounds__(kFinThreads) void colmax_finalize(const uint16_t* __restrict__ part,
                                                               int64_t part_ld, int64_t slabs,
                                                               int64_t cols,
                                                               float* __restrict__ colmax) {
  __shared__ uint4 red[kFinWaves][4];
  finalize_block(part, part_ld, slabs, cols, colmax, red);
}

// Two tensors of the same width: blockIdx.y picks the tensor.
__global__ __launch_bounds__(kFinThreads) void colmax_finalize2(
    const uint16_t* __restrict__ part_a, int64_t slabs_a, float* __restrict__ colmax_a,
    const uint16_t* __restrict__ part_b, int64_t slabs_b, float* __restrict__ colmax_b,
    int64_t part_ld, int64_t cols) {
  __shared__ uint4 red[kFinWaves][4];
  if (blockIdx.y == 0)
    finalize_block(part_a, part_ld, slabs_a, cols, colmax_a, red);
  else
    finalize_block(part_b, part_ld, slabs_b, cols, colmax_b, red);
}

// Launch shapes: pass 1 has col_tiles x slabs blocks (about 256, at most
// kColMaxSlabs slabs of at least 64 rows); pass 2 has col_tiles x row_blocks
// blocks of at least 128 rows, so each block's re-read of the slab maxima
// (slabs KiB) stays small next to its rows_per_block KiB of input.
struct ColPlan {
  int64_t col_tiles, slabs, rows_per_slab, part_ld, row_blocks, rows_per_block;
};

ColPlan col_plan(int64_t rows, int64_t cols) {
  ColPlan p;
  p.col_tiles = max((int64_t)1, (cols + kColTile - 1) / kColTile);
  int64_t slabs = (256 + p.col_tiles - 1) / p.col_tiles;
  slabs = min(slabs, (int64_t)kColMaxSlabs);
  slabs = min(slabs, max((int64_t)1, (rows + 63) / 64));
  p.rows_per_slab = max((int64_t)1, (rows + slabs - 1) / slabs);
  p.slabs = rows > 0 ? (rows + p.rows_per_slab - 1) / p.rows_per_slab : 0;
  p.part_ld = (cols + 7) / 8 * 8;
  const int64_t want_blocks = (256 + p.col_tiles - 1) / p.col_tiles;
  int64_t rpb = max((int64_t)128, (rows + want_blocks - 1) / want_blocks);
  rpb = max(rpb, (rows + 65534) / 65535);  // grid y limit
  p.rows_per_block = rpb;
  p.row_blocks = max((int64_t)1, (rows + rpb - 1) / rpb);
  return p;
}

// Widest row (16-byte chunks per lane) held in registers under stochastic
// rounding: beyond it the row and the Philox draws beside it no longer fit
// (the 28-chunk kernels spilled the row to scratch and ran 4x slower than
// round to nearest), so those rows take the two-read kernels instead.  Rows
// whose length is not a multiple of 4 draw a third Philox block per chunk:
// for them the limit is 12.
constexpr int kSrFusedChunks = 16;
constexpr int kSrFusedChunksUnaligned = 12;
__host__ __device__ constexpr int64_t widest_in_registers(int round, int64_t cols) {
  return round == 1 ? (cols % 4 == 0 ? kSrFusedChunks : kSrFusedChunksUnaligned) : 28;
}

template <int NV>
void launch_rows_nv(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int8_t* q,
                    int64_t ldq, float* scale, int round, uint64_t seed, uint64_t offset,
                    hipStream_t stream) {
  // one row per wave: every row's loads are issued at once
  const dim3 grid((unsigned)((rows + kWavesPerBlock - 1) / kWavesPerBlock));
  constexpr bool PF = false;
  const bool a4 = (cols % 4) == 0;
  if (round == 1) {
    if constexpr (NV <= kSrFusedChunks) {
      if (cols == NV * 512)
        quant_rows_wave<NV, true, true, PF, 0, true><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
      else if (a4)
        quant_rows_wave<NV, true, true, PF><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
      else if constexpr (NV <= kSrFusedChunksUnaligned)
        quant_rows_wave<NV, true, false, PF><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
    }
  } else if (cols == NV * 512) {
    quant_rows_wave<NV, false, true, PF, 0, true><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
  } else {
    quant_rows_wave<NV, false, true, PF><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
  }
}

// Row-wise with column maxima: 16 waves per block for rows of up to 4096
// elements (8 for rows of 3585 .. 4096 elements with stochastic rounding or a
// range-checked tail), 8 up to 6144 and 4 beyond (per-lane state and LDS
// regions grow with the row), about 256 blocks, each a band of whole rows
// (a multiple of 16 rows, so the bands do not depend on the wave count).
// Rows longer than 14336 elements go through rows_long_stats and
// rows_long_quant (bands of rows by segments of 4096 columns), and so do rows
// wider than widest_in_registers under stochastic rounding.

struct RowColmaxPlan {
  bool fused;
  int waves;
  int64_t rows_per_block, slabs, part_ld;
  int64_t nseg;        // long rows: column segments of kLongSeg
  size_t part_bytes;   // slab maxima; the segment maxima ([rows][nseg] bf16 bits) follow
};

RowColmaxPlan rcm_plan(int64_t rows, int64_t cols, int round = 0) {
  RowColmaxPlan p;
  const int64_t per_lane = (cols + 511) / 512;
  p.fused = per_lane <= widest_in_registers(round, cols);
  p.part_ld = (cols + 7) / 8 * 8;
  if (p.fused) {
    // about one block per CU (a block's registers and LDS fill most of one)
    p.waves = per_lane > 12 ? 4 : (per_lane > 8 ? 8 : 16);
    int64_t rpb = (rows + 255) / 256;
    rpb = (rpb + p.waves - 1) / p.waves * p.waves;
    p.rows_per_block = max(rpb, (int64_t)p.waves);
    p.slabs = (rows + p.rows_per_block - 1) / p.rows_per_block;
    p.nseg = 0;
  } else {
    // bands of whole rows by segments of kLongSeg columns: at most 128 bands
    // (the slab maxima stay small next to the tensor), a multiple of 8 rows
    p.waves = kLongWaves;
    p.nseg = (cols + kLongSeg - 1) / kLongSeg;
    int64_t rpb = (rows + 127) / 128;
    rpb = (rpb + kLongWaves - 1) / kLongWaves * kLongWaves;
    p.rows_per_block = max(rpb, (int64_t)kLongWaves);
    p.slabs = (rows + p.rows_per_block - 1) / p.rows_per_block;
  }
  p.part_bytes = (size_t)(max(p.slabs, (int64_t)1) * p.part_ld * 2);
  return p;
}

// Waves per block of the row pass with column maxima (LDS: waves x NV KiB of
// column maxima).  16 waves (at most 128 VGPRs per lane) hold the
// range-check-free round-to-nearest body of rows of 4096; stochastic rounding
// (two Philox blocks per chunk) and range-checked rows of 8 chunks per lane
// need more registers and take 8 waves instead of spilling.
template <int NV>
struct RcmWaves {
  static constexpr int full = NV >= 16 ? 4 : (NV > 8 ? 8 : 16);
  static constexpr int wide = NV >= 16 ? 4 : (NV >= 8 ? 8 : 16);
};

template <int NV>
void launch_rcm2_nv(const RowColmaxJob& a, const RowColmaxJob& b, int64_t cols, int64_t part_ld,
                    int round, uint64_t seed, int fmt, hipStream_t stream) {
  constexpr int WAVES_WIDE = RcmWaves<NV>::wide;
  const dim3 grid((unsigned)(a.slabs + b.slabs));
  const bool a4 = (cols % 4) == 0;
  if (fmt == 1) {  // FP8: round to nearest only
    if (cols == NV * 512)
      quant_rows_colmax2<NV, WAVES_WIDE, false, true, true, 1><<<grid, 64 * WAVES_WIDE, 0, stream>>>(a, b, cols, part_ld, seed);
    else
      quant_rows_colmax2<NV, WAVES_WIDE, false, true, false, 1><<<grid, 64 * WAVES_WIDE, 0, stream>>>(a, b, cols, part_ld, seed);
  } else if (round == 1) {
    if constexpr (NV <= kSrFusedChunks) {
      if (cols == NV * 512)
        quant_rows_colmax2<NV, WAVES_WIDE, true, true, true><<<grid, 64 * WAVES_WIDE, 0, stream>>>(a, b, cols, part_ld, seed);
      else if (a4)
        quant_rows_colmax2<NV, WAVES_WIDE, true, true><<<grid, 64 * WAVES_WIDE, 0, stream>>>(a, b, cols, part_ld, seed);
      else if constexpr (NV <= kSrFusedChunksUnaligned)
        quant_rows_colmax2<NV, WAVES_WIDE, true, false><<<grid, 64 * WAVES_WIDE, 0, stream>>>(a, b, cols, part_ld, seed);
    }
  } else if (cols == NV * 512) {
    // two tensors' bands: with the 16-wave shape's LDS (WAVES x NV KiB) only one
    // block fits per CU, so a pair would run as two rounds; 8 waves (two rows
    // each) keep both tensors' blocks resident at once
    quant_rows_colmax2<NV, WAVES_WIDE, false, true, true><<<grid, 64 * WAVES_WIDE, 0, stream>>>(a, b, cols, part_ld, seed);
  } else {
    quant_rows_colmax2<NV, WAVES_WIDE, false, true><<<grid, 64 * WAVES_WIDE, 0, stream>>>(a, b, cols, part_ld, seed);
  }
}

template <int NV>
void launch_rcm_nv(const RowColmaxPlan& p, const uint16_t* x, int64_t rows, int64_t cols,
                   int64_t ldx, int8_t* q, int64_t ldq, float* scale, int round, uint64_t seed,
                   uint64_t offset, uint16_t* part, hipStream_t stream) {
  constexpr int WAVES = RcmWaves<NV>::full, WAVES_WIDE = RcmWaves<NV>::wide;
  const dim3 grid((unsigned)p.slabs);
  const bool a4 = (cols % 4) == 0;
  if (round == 1) {
    if constexpr (NV <= kSrFusedChunks) {
      if (cols == NV * 512)
        quant_rows_colmax<NV, WAVES_WIDE, true, true, true><<<grid, 64 * WAVES_WIDE, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset, p.rows_per_block, part, p.part_ld);
      else if (a4)
        quant_rows_colmax<NV, WAVES_WIDE, true, true><<<grid, 64 * WAVES_WIDE, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset, p.rows_per_block, part, p.part_ld);
      else if constexpr (NV <= kSrFusedChunksUnaligned)
        quant_rows_colmax<NV, WAVES_WIDE, true, false><<<grid, 64 * WAVES_WIDE, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset, p.rows_per_block, part, p.part_ld);
    }
  } else if (cols == NV * 512) {
    quant_rows_colmax<NV, WAVES, false, true, true><<<grid, 64 * WAVES, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset, p.rows_per_block, part, p.part_ld);
  } else {
    quant_rows_colmax<NV, WAVES_WIDE, false, true><<<grid, 64 * WAVES_WIDE, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset, p.rows_per_block, part, p.part_ld);
  }
}

// Rows past widest_in_registers chunks per lane: one block per row, the row
// read twice (maximum, then codes).
void launch_rows_block(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int8_t* q,
                       int64_t ldq, float* scale, int round, uint64_t seed, uint64_t offset,
                       hipStream_t stream) {
  const dim3 grid((unsigned)rows);
  if (round == 1) {
    if (cols % 4 == 0)
      quant_rows_block<true, true><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
    else
      quant_rows_block<true, false><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
  } else {
    quant_rows_block<false, true><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, seed, offset);
  }
}

}  // namespace

hipError_t launch_quantize_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   int8_t* q, int64_t ldq, float* scale, int round, uint64_t seed,
                                   uint64_t offset, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t per_lane = (cols + 511) / 512;  // 16-byte chunks per lane
  if (per_lane > widest_in_registers(round, cols))
    launch_rows_block(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else if (per_lane <= 1)
    launch_rows_nv<1>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else if (per_lane <= 2)
    launch_rows_nv<2>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else if (per_lane <= 4)
    launch_rows_nv<4>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else if (per_lane <= 8)
    launch_rows_nv<8>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else if (per_lane == 11)
    launch_rows_nv<11>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else if (per_lane <= 12)
    launch_rows_nv<12>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else if (per_lane <= 16)
    launch_rows_nv<16>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  else
    launch_rows_nv<28>(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, stream);
  return hipGetLastError();
}

namespace {
template <int NV>
void launch_rows_f8_nv(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int8_t* q,
                       int64_t ldq, float* scale, hipStream_t stream) {
  const dim3 grid((unsigned)((rows + kWavesPerBlock - 1) / kWavesPerBlock));
  if (cols == NV * 512)
    quant_rows_wave<NV, false, true, false, 1, true><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, 0, 0);
  else
    quant_rows_wave<NV, false, true, false, 1><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, 0, 0);
}
}  // namespace

hipError_t launch_quantize_rowwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                       uint8_t* q8, int64_t ldq, float* scale, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  int8_t* q = reinterpret_cast<int8_t*>(q8);
  const int64_t per_lane = (cols + 511) / 512;
  if (per_lane <= 1)
    launch_rows_f8_nv<1>(x, rows, cols, ldx, q, ldq, scale, stream);
  else if (per_lane <= 2)
    launch_rows_f8_nv<2>(x, rows, cols, ldx, q, ldq, scale, stream);
  else if (per_lane <= 4)
    launch_rows_f8_nv<4>(x, rows, cols, ldx, q, ldq, scale, stream);
  else if (per_lane <= 8)
    launch_rows_f8_nv<8>(x, rows, cols, ldx, q, ldq, scale, stream);
  else if (per_lane == 11)
    launch_rows_f8_nv<11>(x, rows, cols, ldx, q, ldq, scale, stream);
  else if (per_lane <= 12)
    launch_rows_f8_nv<12>(x, rows, cols, ldx, q, ldq, scale, stream);
  else if (per_lane <= 16)
    launch_rows_f8_nv<16>(x, rows, cols, ldx, q, ldq, scale, stream);
  else if (per_lane <= 28)
    launch_rows_f8_nv<28>(x, rows, cols, ldx, q, ldq, scale, stream);
  else
    quant_rows_block<false, true, 1><<<dim3((unsigned)rows), kThreads, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, 0, 0);
  return hipGetLastError();
}

namespace {
template <int NV>
void launch_rcm_f8_nv(const RowColmaxPlan& p, const uint16_t* x, int64_t rows, int64_t cols,
                      int64_t ldx, int8_t* q, int64_t ldq, float* scale, uint16_t* part,
                      hipStream_t stream) {
  constexpr int WAVES = RcmWaves<NV>::full, WAVES_WIDE = RcmWaves<NV>::wide;
  const dim3 grid((unsigned)p.slabs);
  if (cols == NV * 512)
    quant_rows_colmax<NV, WAVES, false, true, true, 1><<<grid, 64 * WAVES, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, 0, 0, p.rows_per_block, part, p.part_ld);
  else
    quant_rows_colmax<NV, WAVES_WIDE, false, true, false, 1><<<grid, 64 * WAVES_WIDE, 0, stream>>>(x, rows, cols, ldx, q, ldq, scale, 0, 0, p.rows_per_block, part, p.part_ld);
}
}  // namespace

bool rowwise_colmax_fp8_fused(int64_t rows, int64_t cols) { return rcm_plan(rows, cols).fused; }

hipError_t launch_quantize_rowwise_colmax_fp8(const uint16_t* x, int64_t rows, int64_t cols,
                                              int64_t ldx, uint8_t* q8, int64_t ldq, float* scale,
                                              float* colmax, void* ws, bool finalize, hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  const RowColmaxPlan p = rcm_plan(rows, cols);
  if (!p.fused) return hipErrorInvalidValue;  // rows over 14336 elements: not offered
  uint16_t* part = static_cast<uint16_t*>(ws);
  int8_t* q = reinterpret_cast<int8_t*>(q8);
  if (rows > 0) {
    const int64_t per_lane = (cols + 511) / 512;
    if (per_lane <= 1)
      launch_rcm_f8_nv<1>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
    else if (per_lane <= 2)
      launch_rcm_f8_nv<2>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
    else if (per_lane <= 4)
      launch_rcm_f8_nv<4>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
    else if (per_lane <= 8)
      launch_rcm_f8_nv<8>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
    else if (per_lane == 11)
      launch_rcm_f8_nv<11>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
    else if (per_lane <= 12)
      launch_rcm_f8_nv<12>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
    else if (per_lane <= 16)
      launch_rcm_f8_nv<16>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
    else
      launch_rcm_f8_nv<28>(p, x, rows, cols, ldx, q, ldq, scale, part, stream);
  }
  if (finalize)
    colmax_finalize<<<dim3((unsigned)((cols + 31) / 32)), kFinThreads, 0, stream>>>(
        part, p.part_ld, rows > 0 ? p.slabs : 0, cols, colmax);
  return hipGetLastError();
}

hipError_t launch_quantize_colwise_given_fp8(const uint16_t* x, int64_t rows, int64_t cols,
                                            int64_t ldx, const float* colmax, uint8_t* q8,
                                            int64_t ldq, float* scale, hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  const int64_t bands = max((int64_t)1, (rows + kColBand - 1) / kColBand);
  const int64_t groups = (cols + (int64_t)kColTile * kColWaves - 1) / ((int64_t)kColTile * kColWaves);
  if (bands > 0x7FFFFFFF || groups > 65535) return hipErrorInvalidValue;
  quant_cols_given<false, true, 1><<<dim3((unsigned)bands, (unsigned)groups), kColThreads, 0, stream>>>(
      x, rows, cols, ldx, colmax, scale, reinterpret_cast<int8_t*>(q8), ldq, 0, 0);
  return hipGetLastError();
}

hipError_t launch_quantize_colwise_fp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                       uint8_t* q8, int64_t ldq, float* scale, void* ws,
                                       hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  const ColPlan p = col_plan(rows, cols);
  uint16_t* part = static_cast<uint16_t*>(ws);
  if (p.slabs > 0) {
    col_absmax_partial<<<dim3((unsigned)p.col_tiles, (unsigned)p.slabs), kColThreads, 0, stream>>>(
        x, rows, cols, ldx, p.rows_per_slab, part, p.part_ld);
  }
  const dim3 grid((unsigned)p.col_tiles, (unsigned)p.row_blocks);
  quant_cols<false, true, 1><<<grid, kColThreads, 0, stream>>>(
      x, rows, cols, ldx, p.rows_per_block, part, p.part_ld, p.slabs, scale,
      reinterpret_cast<int8_t*>(q8), ldq, 0, 0);
  return hipGetLastError();
}

// Column maxima alone (fp32 [cols]): the first pass of the two-pass column
// quantize and the slab reduction.  ws: colwise_workspace_bytes(rows, cols).
hipError_t launch_column_maxima(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float* colmax,
                                void* ws, hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  const ColPlan p = col_plan(rows, cols);
  uint16_t* part = static_cast<uint16_t*>(ws);
  if (p.slabs > 0) {
    col_absmax_partial<<<dim3((unsigned)p.col_tiles, (unsigned)p.slabs), kColThreads, 0, stream>>>(
        x, rows, cols, ldx, p.rows_per_slab, part, p.part_ld);
  }
  colmax_finalize<<<dim3((unsigned)((cols + 31) / 32)), kFinThreads, 0, stream>>>(part, p.part_ld, p.slabs, cols,
                                                                                  colmax);
  return hipGetLastError();
}

size_t colwise_workspace_bytes(int64_t rows, int64_t cols) {
  const ColPlan p = col_plan(rows, cols);
  return (size_t)(max(p.slabs, (int64_t)1) * p.part_ld * 2);
}

hipError_t launch_quantize_colwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                   int8_t* q, int64_t ldq, float* scale, int round, uint64_t seed,
                                   uint64_t offset, void* ws, hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  const ColPlan p = col_plan(rows, cols);
  uint16_t* part = static_cast<uint16_t*>(ws);
  if (p.slabs > 0) {
    col_absmax_partial<<<dim3((unsigned)p.col_tiles, (unsigned)p.slabs), kColThreads, 0, stream>>>(
        x, rows, cols, ldx, p.rows_per_slab, part, p.part_ld);
  }
  // with no rows the quantize pass only stores the (zero) scales
  const dim3 grid((unsigned)p.col_tiles, (unsigned)p.row_blocks);
  const bool a4 = (cols % 4) == 0;
  if (round == 1) {
    if (a4)
      quant_cols<true, true><<<grid, kColThreads, 0, stream>>>(x, rows, cols, ldx, p.rows_per_block, part, p.part_ld, p.slabs, scale, q, ldq, seed, offset);
    else
      quant_cols<true, false><<<grid, kColThreads, 0, stream>>>(x, rows, cols, ldx, p.rows_per_block, part, p.part_ld, p.slabs, scale, q, ldq, seed, offset);
  } else {
    quant_cols<false, true><<<grid, kColThreads, 0, stream>>>(x, rows, cols, ldx, p.rows_per_block, part, p.part_ld, p.slabs, scale, q, ldq, seed, offset);
  }
  return hipGetLastError();
}


// ---- column-wise quantization without a workspace argument ---------------
//
// The slab column maxima of the two-pass column quantize live in this static
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy until the process ends.  Every call on one GPU shares
// it, so calls that overlap on one GPU (on different streams, or from
// different threads) race.  Nothing in it has to start at zero: the first
// pass writes every slab entry the second pass reads.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: its copy
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_quantize_colwise_static(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                          int8_t* q, int64_t ldq, float* scale, int round,
                                          uint64_t seed, uint64_t offset, hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  if (colwise_workspace_bytes(rows, cols) > kStaticScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_quantize_colwise(x, rows, cols, ldx, q, ldq, scale, round, seed, offset, ws, stream);
}

size_t rowwise_colmax_workspace_bytes(int64_t rows, int64_t cols) {
  size_t need = 0;
  for (int round = 0; round < 2; ++round) {  // either rounding's plan fits
    const RowColmaxPlan p = rcm_plan(rows, cols, round);
    const size_t n = p.fused ? p.part_bytes
                             : (p.part_bytes + 255) / 256 * 256 + (size_t)(max(rows, (int64_t)1) * p.nseg * 2);
    need = max(need, n);
  }
  return need;
}

hipError_t launch_quantize_rowwise_colmax(const uint16_t* x, int64_t rows, int64_t cols,
                                          int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                          float* colmax, int round, uint64_t seed, uint64_t offset,
                                          void* ws, hipStream_t stream) {
  return launch_quantize_rowwise_slabs(x, rows, cols, ldx, q, ldq, scale, colmax, round, seed, offset,
                                       ws, true, stream);
}

hipError_t launch_quantize_rowwise_slabs(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                         int8_t* q, int64_t ldq, float* scale, float* colmax,
                                         int round, uint64_t seed, uint64_t offset, void* ws,
                                         bool finalize, hipStream_t stream) {
  // no columns: no maxima, but every row's scale is still written (0)
  if (cols == 0) return launch_quantize_rowwise(x, rows, 0, ldx, q, ldq, scale, round, seed, offset, stream);
  const RowColmaxPlan p = rcm_plan(rows, cols, round);
  uint16_t* part = static_cast<uint16_t*>(ws);
  if (rows > 0) {
    if (p.fused) {
      const int64_t per_lane = (cols + 511) / 512;
      if (per_lane <= 1)
        launch_rcm_nv<1>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
      else if (per_lane <= 2)
        launch_rcm_nv<2>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
      else if (per_lane <= 4)
        launch_rcm_nv<4>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
      else if (per_lane <= 8)
        launch_rcm_nv<8>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
      else if (per_lane == 11)
        launch_rcm_nv<11>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
      else if (per_lane <= 12)
        launch_rcm_nv<12>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
      else if (per_lane <= 16)
        launch_rcm_nv<16>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
      else
        launch_rcm_nv<28>(p, x, rows, cols, ldx, q, ldq, scale, round, seed, offset, part, stream);
    } else {
      uint16_t* segmax = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + (p.part_bytes + 255) / 256 * 256);
      const dim3 grid((unsigned)p.nseg, (unsigned)p.slabs);
      rows_long_stats<<<grid, kLongThreads, 0, stream>>>(x, rows, cols, ldx, p.rows_per_block, segmax,
                                                         p.nseg, part, p.part_ld);
      const bool a4 = (cols % 4) == 0;
      if (round == 1 && a4)
        rows_long_quant<true, true><<<grid, kLongThreads, 0, stream>>>(x, rows, cols, ldx, p.rows_per_block, segmax, p.nseg, q, ldq, scale, seed, offset);
      else if (round == 1)
        rows_long_quant<true, false><<<grid, kLongThreads, 0, stream>>>(x, rows, cols, ldx, p.rows_per_block, segmax, p.nseg, q, ldq, scale, seed, offset);
      else
        rows_long_quant<false, true><<<grid, kLongThreads, 0, stream>>>(x, rows, cols, ldx, p.rows_per_block, segmax, p.nseg, q, ldq, scale, seed, offset);
    }
  }
  if (finalize)
    colmax_finalize<<<dim3((unsigned)((cols + 31) / 32)), kFinThreads, 0, stream>>>(
        part, p.part_ld, rows > 0 ? p.slabs : 0, cols, colmax);
  return hipGetLastError();
}

hipError_t launch_quantize_colwise_given(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ldx, const float* colmax, int8_t* q, int64_t ldq,
                                         float* scale, int round, uint64_t seed, uint64_t offset,
                                         hipStream_t stream) {
  if (cols == 0) return hipSuccess;
  // bands of kColBand rows (at least one, so the scales are written for an
  // empty tensor too) x groups of kColWaves column tiles
  const int64_t bands = max((int64_t)1, (rows + kColBand - 1) / kColBand);
  const int64_t groups = (cols + (int64_t)kColTile * kColWaves - 1) / ((int64_t)kColTile * kColWaves);
  if (bands > 0x7FFFFFFF || groups > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)bands, (unsigned)groups);
  const bool a4 = (cols % 4) == 0;
  if (round == 1) {
    if (a4)
      quant_cols_given<true, true><<<grid, kColThreads, 0, stream>>>(x, rows, cols, ldx, colmax, scale, q, ldq, seed, offset);
    else
      quant_cols_given<true, false><<<grid, kColThreads, 0, stream>>>(x, rows, cols, ldx, colmax, scale, q, ldq, seed, offset);
  } else {
    quant_cols_given<false, true><<<grid, kColThreads, 0, stream>>>(x, rows, cols, ldx, colmax, scale, q, ldq, seed, offset);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rowwise_colmax_pair(
    const uint16_t* xa, int64_t rows_a, int64_t ldxa, int8_t* qa, int64_t ldqa, float* scale_a,
    float* colmax_a, uint64_t offset_a, void* ws_a, const uint16_t* xb, int64_t rows_b,
    int64_t ldxb, int8_t* qb, int64_t ldqb, float* scale_b, float* colmax_b, uint64_t offset_b,
    void* ws_b, int64_t cols, int round, uint64_t seed, bool finalize, int fmt, hipStream_t stream) {
  if (cols == 0) {  // no maxima; the row scales are still written (0)
    const hipError_t e = launch_quantize_rowwise(xa, rows_a, 0, ldxa, qa, ldqa, scale_a, round, seed, offset_a, stream);
    if (e != hipSuccess) return e;
    return launch_quantize_rowwise(xb, rows_b, 0, ldxb, qb, ldqb, scale_b, round, seed, offset_b, stream);
  }
  const RowColmaxPlan pa = rcm_plan(rows_a, cols, round), pb = rcm_plan(rows_b, cols, round);
  if (!pa.fused || rows_a == 0 || rows_b == 0) {
    if (fmt == 1) {  // rows of at most 14336 elements (the FP8 row pass with maxima)
      const hipError_t e = launch_quantize_rowwise_colmax_fp8(xa, rows_a, cols, ldxa, reinterpret_cast<uint8_t*>(qa),
                                                              ldqa, scale_a, colmax_a, ws_a, finalize, stream);
      if (e != hipSuccess) return e;
      return launch_quantize_rowwise_colmax_fp8(xb, rows_b, cols, ldxb, reinterpret_cast<uint8_t*>(qb), ldqb,
                                                scale_b, colmax_b, ws_b, finalize, stream);
    }
    const hipError_t e = launch_quantize_rowwise_slabs(xa, rows_a, cols, ldxa, qa, ldqa, scale_a, colmax_a,
                                                       round, seed, offset_a, ws_a, finalize, stream);
    if (e != hipSuccess) return e;
    return launch_quantize_rowwise_slabs(xb, rows_b, cols, ldxb, qb, ldqb, scale_b, colmax_b, round, seed,
                                         offset_b, ws_b, finalize, stream);
  }
  const RowColmaxJob a{xa, rows_a, ldxa, qa, ldqa, scale_a, offset_a, pa.rows_per_block, pa.slabs,
                       static_cast<uint16_t*>(ws_a)};
  const RowColmaxJob b{xb, rows_b, ldxb, qb, ldqb, scale_b, offset_b, pb.rows_per_block, pb.slabs,
                       static_cast<uint16_t*>(ws_b)};
  const int64_t per_lane = (cols + 511) / 512;
  if (per_lane <= 1)
    launch_rcm2_nv<1>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  else if (per_lane <= 2)
    launch_rcm2_nv<2>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  else if (per_lane <= 4)
    launch_rcm2_nv<4>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  else if (per_lane <= 8)
    launch_rcm2_nv<8>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  else if (per_lane == 11)
    launch_rcm2_nv<11>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  else if (per_lane <= 12)
    launch_rcm2_nv<12>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  else if (per_lane <= 16)
    launch_rcm2_nv<16>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  else
    launch_rcm2_nv<28>(a, b, cols, pa.part_ld, round, seed, fmt, stream);
  if (finalize)
    colmax_finalize2<<<dim3((unsigned)((cols + 31) / 32), 2), kFinThreads, 0, stream>>>(
        a.part, a.slabs, colmax_a, b.part, b.slabs, colmax_b, pa.part_ld, cols);
  return hipGetLastError();
}

void rowwise_colmax_geometry(int64_t rows, int64_t cols, int round, int64_t* slabs, int64_t* part_ld) {
  const RowColmaxPlan p = rcm_plan(rows, cols, round);
  *slabs = rows > 0 ? p.slabs : 0;
  *part_ld = p.part_ld;
}

hipError_t launch_colmax_finalize(const ColmaxJob& j, hipStream_t stream) {
  if (j.n <= 0 || j.cols == 0) return hipSuccess;
  const dim3 blocks((unsigned)((j.cols + 31) / 32), (unsigned)j.n);
  if (j.n == 1)
    colmax_finalize<<<blocks, kFinThreads, 0, stream>>>(j.part[0], j.part_ld, j.slabs[0], j.cols, j.colmax[0]);
  else
    colmax_finalize2<<<blocks, kFinThreads, 0, stream>>>(j.part[0], j.slabs[0], j.colmax[0], j.part[1], j.slabs[1],
                                                         j.colmax[1], j.part_ld, j.cols);
  return hipGetLastError();
}

hipError_t launch_quantize_colwise_given_pair(
    const uint16_t* xa, int64_t rows_a, int64_t cols_a, int64_t ldxa, const float* colmax_a,
    int8_t* qa, int64_t ldqa, float* scale_a, uint64_t offset_a, const uint16_t* xb,
    int64_t rows_b, int64_t cols_b, int64_t ldxb, const float* colmax_b, int8_t* qb, int64_t ldqb,
    float* scale_b, uint64_t offset_b, int round, uint64_t seed, int fmt, hipStream_t stream) {
  if (cols_a == 0 || cols_b == 0) {
    if (fmt == 1) {
      const hipError_t e = launch_quantize_colwise_given_fp8(xa, rows_a, cols_a, ldxa, colmax_a,
                                                             reinterpret_cast<uint8_t*>(qa), ldqa, scale_a, stream);
      if (e != hipSuccess) return e;
      return launch_quantize_colwise_given_fp8(xb, rows_b, cols_b, ldxb, colmax_b, reinterpret_cast<uint8_t*>(qb),
                                               ldqb, scale_b, stream);
    }
    const hipError_t e = launch_quantize_colwise_given(xa, rows_a, cols_a, ldxa, colmax_a, qa, ldqa, scale_a,
                                                       round, seed, offset_a, stream);
    if (e != hipSuccess) return e;
    return launch_quantize_colwise_given(xb, rows_b, cols_b, ldxb, colmax_b, qb, ldqb, scale_b, round, seed,
                                         offset_b, stream);
  }
  const int64_t span = (int64_t)kColTile * kColWaves;
  const int64_t bands_a = max((int64_t)1, (rows_a + kColBand - 1) / kColBand);
  const int64_t bands_b = max((int64_t)1, (rows_b + kColBand - 1) / kColBand);
  const ColGivenJob a{xa, rows_a, cols_a, ldxa, colmax_a, scale_a, qa, ldqa, offset_a, bands_a,
                      (bands_a + kPairBands - 1) / kPairBands};
  const ColGivenJob b{xb, rows_b, cols_b, ldxb, colmax_b, scale_b, qb, ldqb, offset_b, bands_b,
                      (bands_b + kPairBands - 1) / kPairBands};
  const int64_t groups = max((cols_a + span - 1) / span, (cols_b + span - 1) / span);
  if (a.blocks + b.blocks > 0x7FFFFFFF || groups > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.blocks + b.blocks), (unsigned)groups);
  if (fmt == 1) {
    quant_cols_given2<false, true, 1><<<grid, kColThreads, 0, stream>>>(a, b, seed);
  } else if (round == 1) {
    if (cols_a % 4 == 0 && cols_b % 4 == 0)
      quant_cols_given2<true, true><<<grid, kColThreads, 0, stream>>>(a, b, seed);
    else
      quant_cols_given2<true, false><<<grid, kColThreads, 0, stream>>>(a, b, seed);
  } else {
    quant_cols_given2<false, true><<<grid, kColThreads, 0, stream>>>(a, b, seed);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rowslabs_colgiven(
    const uint16_t* xa, int64_t rows_a, int64_t cols_a, int64_t ldxa, int8_t* qa, int64_t ldqa,
    float* scale_a, uint64_t offset_a, void* ws_a, const uint16_t* xb, int64_t rows_b, int64_t cols_b,
    int64_t ldxb, const float* colmax_b, int8_t* qb, int64_t ldqb, float* scale_b, uint64_t offset_b,
    int round, uint64_t seed, int fmt, hipStream_t stream) {
  const RowColmaxPlan pa = rcm_plan(rows_a, cols_a, round);
  const int64_t per_lane = (cols_a + 511) / 512;
  const int nv = per_lane > 2 && per_lane <= 4 ? 4 : (per_lane > 4 && per_lane <= 8 ? 8 : 0);
  const bool a4 = cols_a % 4 == 0 && cols_b % 4 == 0;
  if (rows_a == 0 || cols_a == 0 || cols_b == 0 || !pa.fused || nv == 0 || (round == 1 && !a4)) {
    if (fmt == 1) {  // rows of at most 14336 elements (the FP8 row pass with maxima)
      const hipError_t e = cols_a == 0 ? launch_quantize_rowwise_fp8(xa, rows_a, 0, ldxa, reinterpret_cast<uint8_t*>(qa),
                                                                     ldqa, scale_a, stream)
                                       : launch_quantize_rowwise_colmax_fp8(xa, rows_a, cols_a, ldxa,
                                                                            reinterpret_cast<uint8_t*>(qa), ldqa,
                                                                            scale_a, nullptr, ws_a, false, stream);
      if (e != hipSuccess) return e;
      return launch_quantize_colwise_given_fp8(xb, rows_b, cols_b, ldxb, colmax_b, reinterpret_cast<uint8_t*>(qb),
                                               ldqb, scale_b, stream);
    }
    const hipError_t e = launch_quantize_rowwise_slabs(xa, rows_a, cols_a, ldxa, qa, ldqa, scale_a, nullptr, round,
                                                       seed, offset_a, ws_a, false, stream);
    if (e != hipSuccess) return e;
    return launch_quantize_colwise_given(xb, rows_b, cols_b, ldxb, colmax_b, qb, ldqb, scale_b, round, seed,
                                         offset_b, stream);
  }
  const RowColmaxJob a{xa, rows_a, ldxa, qa, ldqa, scale_a, offset_a, pa.rows_per_block, pa.slabs,
                       static_cast<uint16_t*>(ws_a)};
  const int64_t bands_b = max((int64_t)1, (rows_b + kColBand - 1) / kColBand);
  const ColGivenJob b{xb, rows_b, cols_b, ldxb, colmax_b, scale_b, qb, ldqb, offset_b, bands_b,
                      (bands_b + kPairBands - 1) / kPairBands};
  const int64_t groups = (cols_b + (int64_t)kColTile * kColWaves - 1) / ((int64_t)kColTile * kColWaves);
  if (a.slabs + b.blocks * groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.slabs + b.blocks * groups));
  const bool full = cols_a == (int64_t)nv * 512;
  if (fmt == 1) {  // FP8: round to nearest only
    if (nv == 4 && full)
      quant_rows_cols_pair<4, false, true, true, 1><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else if (nv == 4)
      quant_rows_cols_pair<4, false, true, false, 1><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else if (full)
      quant_rows_cols_pair<8, false, true, true, 1><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else
      quant_rows_cols_pair<8, false, true, false, 1><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
  } else if (nv == 4) {
    if (round == 1 && full)
      quant_rows_cols_pair<4, true, true, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else if (round == 1)
      quant_rows_cols_pair<4, true, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else if (full)
      quant_rows_cols_pair<4, false, true, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else
      quant_rows_cols_pair<4, false, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
  } else {
    if (round == 1 && full)
      quant_rows_cols_pair<8, true, true, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else if (round == 1)
      quant_rows_cols_pair<8, true, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else if (full)
      quant_rows_cols_pair<8, false, true, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
    else
      quant_rows_cols_pair<8, false, true><<<grid, kColThreads, 0, stream>>>(a, cols_a, pa.part_ld, b, groups, seed);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------

namespace {
__global__ __launch_bounds__(kThreads) void philox_fill(uint64_t seed, uint64_t offset,
                                                        int64_t n_blocks, uint4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_blocks) return;
  const u32x4 w = philox_block(seed, offset + (uint64_t)i);
  out[i] = make_uint4(w.w[0], w.w[1], w.w[2], w.w[3]);
}
}  // namespace

hipError_t launch_philox(uint64_t seed, uint64_t offset, int64_t n_blocks, uint32_t* out,
                         hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  philox_fill<<<dim3((unsigned)((n_blocks + kThreads - 1) / kThreads)), kThreads, 0, stream>>>(
      seed, offset, n_blocks, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace i8mp
