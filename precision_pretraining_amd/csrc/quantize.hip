// Two-level NVFP4 block quantizer for gfx950.
//
// What it computes (Full-Stack FP4, [FS4 §2.1]: the residual is held in NVFP4;
// [FS4 §2.3]: Newton-Schulz operands are NVFP4; format as in fs4.h):
//   s_t  = RNE_fp32(amax_t / 2688)
//   s_b  = E4M3 RNE satfinite(amax_b / (6 s_t)) per 16 elements
//   code = sign | E2M1 RNE(|x| / (s_b s_t)) with the division exact
//
// Two launches:
//   1. amax pass: grid-stride 16-byte loads, max of |x| on the raw bit
//      patterns (monotone for finite values), one partial per workgroup.
//   2. encode pass: every workgroup reduces the (<= 1024) partials itself,
//      stages a 64x64 tile in LDS, then each of its 256 threads encodes one
//      16-element row block and one 16-element column block of the tile.
//
// Exactness of the element decision: with step = s_b s_t (exact in fp64),
// |x| / step lies above midpoint mu iff |x| > mu * step.  mu * step has at most
// 3 + 4 + 24 significant bits, so it is exact in fp64, and rounding it to fp32
// downwards (for "> mu", ties go down) or upwards (for ">= mu", ties go up)
// gives an fp32 threshold that makes the fp32 compare on |x| exact.
#include "fs4_common.h"

namespace fs4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ inline uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[kThreads / 64];
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = r > red[i] ? r : red[i];
  __syncthreads();
  return r;
}

// magnitude bit patterns of the values in one 16-byte word, as fp32 bits
template <bool BF16>
__device__ inline uint32_t word_mag_max(uint32_t w) {
  if constexpr (BF16) {
    uint32_t a = w & 0x7FFFu, b = (w >> 16) & 0x7FFFu;
    return (a > b ? a : b) << 16;
  } else {
    return w & 0x7FFFFFFFu;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const uint4 *__restrict__ x,
                                                                 int64_t nvec,
                                                                 uint32_t *__restrict__ partials) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    const uint4 v = x[i];
    uint32_t a = word_mag_max<BF16>(v.x), b = word_mag_max<BF16>(v.y);
    uint32_t c = word_mag_max<BF16>(v.z), d = word_mag_max<BF16>(v.w);
    a = a > b ? a : b;
    c = c > d ? c : d;
    a = a > c ? a : c;
    m = m > a ? m : a;
  }
  m = block_max_u32(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Encodes 16 values with tensor scale s_t.  Returns the E4M3 scale byte and the
// 16 codes packed two per byte, even element in the low nibble.
__device__ inline uint32_t encode16(const float *v, float s_t, uint2 &packed) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t sb = 0;
  if (s_t > 0.0f) sb = e4m3_rne_satfinite((double)amax / (6.0 * (double)s_t));
  const double step = (double)e4m3_to_float(sb) * (double)s_t;
  uint32_t w[2] = {0u, 0u};
  if (step > 0.0) {
    const float t0 = f32_round_down(0.25 * step);   // ties at 0.25 go down (to index 0)
    const float t1 = f32_round_up(0.75 * step);     // ties at 0.75 go up (to index 2)
    const float t2 = f32_round_down(1.25 * step);
    const float t3 = f32_round_up(1.75 * step);
    const float t4 = f32_round_down(2.5 * step);
    const float t5 = f32_round_up(3.5 * step);
    const float t6 = f32_round_down(5.0 * step);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = fabsf(v[i]);
      uint32_t c = (uint32_t)(a > t0) + (uint32_t)(a >= t1) + (uint32_t)(a > t2) +
                   (uint32_t)(a >= t3) + (uint32_t)(a > t4) + (uint32_t)(a >= t5) +
                   (uint32_t)(a > t6);
      c |= (__builtin_bit_cast(uint32_t, v[i]) >> 28) & 8u;
      w[i >> 3] |= c << (4 * (i & 7));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      w[i >> 3] |= ((__builtin_bit_cast(uint32_t, v[i]) >> 28) & 8u) << (4 * (i & 7));
  }
  packed = make_uint2(w[0], w[1]);
  return sb;
}

template <bool BF16>
__device__ inline void load_tile(const void *x, int64_t rows, int64_t cols, int64_t r0, int64_t c0,
                                 float (*tile)[kTile + 1]) {
  if constexpr (BF16) {
    // 64 rows x 64 bf16 = 64 x 8 chunks of 16 bytes; 256 threads -> 2 passes
    const uint16_t *xb = (const uint16_t *)x;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      const int r = idx >> 3, ch = idx & 7;
      const int64_t gr = r0 + r, gc = c0 + ch * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gr < rows && gc < cols) v = *(const uint4 *)(xb + gr * cols + gc);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tile[r][ch * 8 + 2 * j] = bf16_bits_to_float(wv[j] & 0xFFFFu);
        tile[r][ch * 8 + 2 * j + 1] = bf16_bits_to_float(wv[j] >> 16);
      }
    }
  } else {
    const float *xf = (const float *)x;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      const int r = idx >> 4, ch = idx & 15;
      const int64_t gr = r0 + r, gc = c0 + ch * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gr < rows && gc < cols) v = *(const float4 *)(xf + gr * cols + gc);
      tile[r][ch * 4 + 0] = v.x;
      tile[r][ch * 4 + 1] = v.y;
      tile[r][ch * 4 + 2] = v.z;
      tile[r][ch * 4 + 3] = v.w;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void *__restrict__ x, int64_t rows,
                                                            int64_t cols,
                                                            const uint32_t *__restrict__ partials,
                                                            int npart, fs4_nvfp4 rv, fs4_nvfp4 cv) {
  __shared__ float tile[kTile][kTile + 1];
  // tensor scale from the amax partials (every workgroup reduces them itself)
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npart; i += kThreads) m = m > partials[i] ? m : partials[i];
  m = block_max_u32(m);
  const float amax = __builtin_bit_cast(float, m);
  const float s_t = (float)((double)amax / kTensorDiv);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    if (rv.codes) *rv.tscale = s_t;
    if (cv.codes) *cv.tscale = s_t;
  }

  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
  load_tile<BF16>(x, rows, cols, r0, c0, tile);
  __syncthreads();

  const int t = threadIdx.x;
  if (rv.codes) {
    const int r = t >> 2, blk = t & 3;
    const int64_t gr = r0 + r, gc = c0 + blk * kBlock;
    if (gr < rows && gc < cols) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = tile[r][blk * kBlock + i];
      uint2 packed;
      const uint32_t sb = encode16(v, s_t, packed);
      *(uint2 *)(rv.codes + gr * (cols / 2) + gc / 2) = packed;
      rv.scales[gr * (cols / kBlock) + gc / kBlock] = (uint8_t)sb;
    }
  }
  if (cv.codes) {
    const int c = t & 63, rblk = t >> 6;
    const int64_t gc = c0 + c, gr = r0 + rblk * kBlock;
    if (gc < cols && gr < rows) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = tile[rblk * kBlock + i][c];
      uint2 packed;
      const uint32_t sb = encode16(v, s_t, packed);
      *(uint2 *)(cv.codes + gc * (rows / 2) + gr / 2) = packed;
      cv.scales[gc * (rows / kBlock) + gr / kBlock] = (uint8_t)sb;
    }
  }
}

__global__ void write_zero_scale_kernel(float *a, float *b) {
  if (a) *a = 0.0f;
  if (b) *b = 0.0f;
}

}  // namespace

size_t quantize_ws_bytes() { return kAmaxPartials * sizeof(uint32_t); }

fs4_status launch_quantize(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                           const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise, void *ws,
                           hipStream_t s) {
  const fs4_nvfp4 none = {nullptr, nullptr, nullptr, 0, 0};
  const fs4_nvfp4 rv = rowwise ? *rowwise : none;
  const fs4_nvfp4 cv = colwise ? *colwise : none;
  if (rows == 0 || cols == 0) {
    write_zero_scale_kernel<<<1, 1, 0, s>>>(rv.tscale, cv.tscale);
    return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
  }
  const bool bf16 = dt == FS4_BF16;
  const int64_t n = rows * cols;
  const int64_t nvec = n / (bf16 ? 8 : 4);
  int64_t g = (nvec + kThreads * 8 - 1) / (kThreads * 8);
  const int npart = (int)(g < 1 ? 1 : (g > kAmaxPartials ? kAmaxPartials : g));
  uint32_t *partials = (uint32_t *)ws;
  dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
  if (bf16) {
    amax_partial_kernel<true><<<npart, kThreads, 0, s>>>((const uint4 *)x, nvec, partials);
    quantize_kernel<true><<<grid, kThreads, 0, s>>>(x, rows, cols, partials, npart, rv, cv);
  } else {
    amax_partial_kernel<false><<<npart, kThreads, 0, s>>>((const uint4 *)x, nvec, partials);
    quantize_kernel<false><<<grid, kThreads, 0, s>>>(x, rows, cols, partials, npart, rv, cv);
  }
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
