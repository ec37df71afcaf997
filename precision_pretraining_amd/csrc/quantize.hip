// Two-level NVFP4 block quantizer for gfx950.
//
// What it computes (Full-Stack FP4, [FS4 §2.1]: the residual is held in NVFP4;
// [FS4 §2.3]: Newton-Schulz operands are NVFP4; format as in fs4.h):
//   s_t  = RNE_fp32(amax_t / 2688)
//   s_b  = E4M3 RNE satfinite(amax_b / (6 s_t)) per 16 elements
//   code = sign | E2M1 RNE(|x| / (s_b s_t)) with the division exact
//
// Two launches:
//   1. amax pass: grid-stride 16-byte loads (several in flight per lane), max
//      of |x| on the raw bit patterns (monotone for finite values), one
//      partial per workgroup.
//   2. encode pass (persistent workgroups): each workgroup reduces the
//      partials to s_t once, builds its lookup tables in LDS, then loops over
//      64 x 64 tiles: stage the tile in LDS, and each of the 256 lanes encodes
//      one 16-element row block and one 16-element column block.
//
// Exact decisions with fp32 compares.  With step = s_b s_t (exact in fp64),
// |x| / step lies above an E2M1 midpoint mu iff |x| > mu * step; mu * step has
// at most 3 + 4 + 24 significant bits, so it is exact in fp64.  Rounded to
// fp32 upwards where ties go up (then ">=" decides) and, where ties go down,
// rounded downwards and stepped to the next float (then ">=" decides as well),
// the compare on the fp32 |x| is exact.  The same construction gives the E4M3
// decision thresholds for amax_b against mid * 6 s_t (5 + 3 + 24 bits).
//
// Fast element path.  For each scale code the table holds R_lo < 1/step <
// R_hi, each within 2^-19 of 1/step.  y_lo = |x| R_lo and y_hi = |x| R_hi
// (fp32) bracket |x| / step; the hardware fp32 -> E2M1 conversion
// (v_cvt_scalef32_pk_fp4_f32, round-to-nearest-even, saturating) is monotone,
// so when both give the same 16 codes the exact code is that one.  A block
// where any code differs (an element within ~2^-19 of a midpoint) takes the
// exact threshold path.  Blocks whose 1/step exceeds 2^120 (tiny fp32
// tensors) always take the exact path.
#include "fs4_common.h"

namespace fs4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kEncodeGrid = 1024;     // persistent workgroups of the encode pass
constexpr int kAmaxUnroll = 4;

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ inline uint32_t block_max_u32(uint32_t v, uint32_t *red) {
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

// largest magnitude bit pattern in a 16-byte word, as fp32 bits
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
__device__ inline uint32_t vec_mag_max(const uint4 &v) {
  uint32_t a = word_mag_max<BF16>(v.x), b = word_mag_max<BF16>(v.y);
  uint32_t c = word_mag_max<BF16>(v.z), d = word_mag_max<BF16>(v.w);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const uint4 *__restrict__ x,
                                                                 int64_t nvec,
                                                                 uint32_t *__restrict__ partials) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  // kAmaxUnroll independent 16-byte loads in flight per lane
  for (; i + (kAmaxUnroll - 1) * stride < nvec; i += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const uint32_t a = vec_mag_max<BF16>(v[u]);
      m = m > a ? m : a;
    }
  }
  for (; i < nvec; i += stride) {
    const uint32_t a = vec_mag_max<BF16>(x[i]);
    m = m > a ? m : a;
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// ---- lookup tables (per workgroup, from s_t) ---------------------------------
// e4t[c], c = 0..125: amax_b >= e4t[c] exactly when the E4M3 scale code is at
//   least c + 1.
// rlo[c], rhi[c], c = 0..126: the bracket of 1/(e4m3(c) s_t); rlo < 0 marks a
//   code whose blocks take the exact path; code 0 (step 0) has rlo = rhi = 0.
// eth[c][i], i = 0..6: |x| >= eth[c][i] exactly when the E2M1 index exceeds i
//   for scale code c.
struct Tables {
  float e4t[128];
  float rlo[128], rhi[128];
  float eth[128][8];
};

// mu * scale rounded for an exact ">=" compare on fp32 values: upwards when
// ties go up, else downwards and stepped to the next float (x > t <=> x >= t+)
__device__ inline float ge_threshold(double exact, bool tie_up) {
  if (tie_up) return f32_round_up(exact);
  const float d = f32_round_down(exact);
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, d) + 1u);
}

__device__ inline double e4m3_value(int c) { return (double)e4m3_to_float((uint32_t)c); }

__device__ void build_tables(Tables &t, float s_t) {
  const double st = (double)s_t;
  for (int c = threadIdx.x; c < 128; c += kThreads) {
    if (c < 126) {
      // boundary between codes c and c+1: ties go to the even code
      const double mid = 0.5 * (e4m3_value(c) + e4m3_value(c + 1));
      t.e4t[c] = st > 0.0 ? ge_threshold(mid * 6.0 * st, (c + 1) % 2 == 0) : __builtin_huge_valf();
    } else {
      t.e4t[c] = __builtin_huge_valf();
    }
    const double step = c < 127 ? e4m3_value(c) * st : 0.0;
    if (step > 0.0) {
      const double r = 1.0 / step;
      if (r < 0x1p120) {
        t.rlo[c] = (float)(r * (1.0 - 0x1p-20));
        t.rhi[c] = (float)(r * (1.0 + 0x1p-20));
      } else {
        t.rlo[c] = -1.0f;
        t.rhi[c] = -1.0f;
      }
    } else {
      t.rlo[c] = 0.0f;
      t.rhi[c] = 0.0f;
    }
    // E2M1 midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5; ties go to the even index,
    // i.e. up at 0.75, 1.75 and 3.5
    const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
    for (int i = 0; i < 7; ++i)
      t.eth[c][i] = step > 0.0 ? ge_threshold(mids[i] * step, i == 1 || i == 3 || i == 5)
                               : __builtin_huge_valf();
    t.eth[c][7] = __builtin_huge_valf();
  }
}

// E4M3 scale code of a block.  The estimate rounds q = amax_b / (6 s_t),
// taken in fp32, to 3 mantissa bits (nearest, from the bit pattern; the
// subnormal range on the 2^-9 grid); fp32 rounding of q moves it by at most one
// code from the exact round-to-nearest-even code, which the two table compares
// then give exactly.
__device__ inline uint32_t scale_code(float amax, float inv6st, const Tables &t) {
  if (!(amax > 0.0f) || !(inv6st > 0.0f)) return 0u;
  float q = amax * inv6st;
  q = q < 448.0f ? q : 448.0f;
  int c;
  if (q >= 0.015625f) {
    const uint32_t b = __builtin_bit_cast(uint32_t, q);
    c = (int)((b + (1u << 19)) >> 20) - (120 << 3);   // biased exponent and 3 mantissa bits
  } else {
    c = (int)(q * 512.0f + 0.5f);
  }
  c = c > 126 ? 126 : (c < 0 ? 0 : c);
  if (c < 126 && amax >= t.e4t[c]) ++c;
  else if (c > 0 && amax < t.e4t[c - 1]) --c;
  // exact code c satisfies e4t[c-1] <= amax < e4t[c]; an estimate that was
  // off by more than one (e.g. 1/(6 s_t) overflowed for a subnormal s_t) is
  // redone by binary search over the thresholds
  const bool ok = (c == 0 || amax >= t.e4t[c - 1]) && (c == 126 || amax < t.e4t[c]);
  if (!ok) {
    int lo = 0, hi = 126;                 // number of thresholds <= amax lies in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (amax >= t.e4t[mid]) lo = mid + 1;
      else hi = mid;
    }
    c = lo;
  }
  return (uint32_t)c;
}

// Encodes 16 values; returns the scale code, packs the codes (element 2j in
// the low nibble of byte j).
__device__ inline uint32_t encode16(const float *v, float inv6st, const Tables &t, uint2 &packed) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sb = scale_code(amax, inv6st, t);
  const float rl = t.rlo[sb], rh = t.rhi[sb];
  uint32_t lo0 = 0, lo1 = 0, hi0 = 0, hi1 = 0;
  bool exact = rl < 0.0f;
  if (!exact) {
#define FS4_CVT(W, A, B, R, SEL) W = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(W, (A) * (R), (B) * (R), 1.0f, SEL)
    FS4_CVT(lo0, v[0], v[1], rl, 0); FS4_CVT(lo0, v[2], v[3], rl, 1);
    FS4_CVT(lo0, v[4], v[5], rl, 2); FS4_CVT(lo0, v[6], v[7], rl, 3);
    FS4_CVT(lo1, v[8], v[9], rl, 0); FS4_CVT(lo1, v[10], v[11], rl, 1);
    FS4_CVT(lo1, v[12], v[13], rl, 2); FS4_CVT(lo1, v[14], v[15], rl, 3);
    FS4_CVT(hi0, v[0], v[1], rh, 0); FS4_CVT(hi0, v[2], v[3], rh, 1);
    FS4_CVT(hi0, v[4], v[5], rh, 2); FS4_CVT(hi0, v[6], v[7], rh, 3);
    FS4_CVT(hi1, v[8], v[9], rh, 0); FS4_CVT(hi1, v[10], v[11], rh, 1);
    FS4_CVT(hi1, v[12], v[13], rh, 2); FS4_CVT(hi1, v[14], v[15], rh, 3);
#undef FS4_CVT
    exact = (lo0 != hi0) | (lo1 != hi1);
  }
  if (exact) {
    // exact path: count the thresholds each |x| reaches
    const float *th = t.eth[sb];
    lo0 = lo1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = fabsf(v[i]);
      uint32_t c = 0;
#pragma unroll
      for (int m = 0; m < 7; ++m) c += (uint32_t)(a >= th[m]);
      c |= (__builtin_bit_cast(uint32_t, v[i]) >> 28) & 8u;
      if (i < 8) lo0 |= c << (4 * i);
      else lo1 |= c << (4 * (i - 8));
    }
  }
  packed = make_uint2(lo0, lo1);
  return sb;
}

// stage a 64 x 64 tile as fp32 in LDS (zeros outside the tensor)
template <bool BF16>
__device__ inline void load_tile(const void *x, int64_t rows, int64_t cols, int64_t r0, int64_t c0,
                                 float (*tile)[kTile + 1]) {
  if constexpr (BF16) {
    const uint16_t *xb = (const uint16_t *)x;
    uint4 v[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      const int r = idx >> 3, ch = idx & 7;
      const int64_t gr = r0 + r, gc = c0 + ch * 8;
      v[p] = (gr < rows && gc < cols) ? *(const uint4 *)(xb + gr * cols + gc) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      const int r = idx >> 3, ch = idx & 7;
      const uint32_t wv[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tile[r][ch * 8 + 2 * j] = bf16_bits_to_float(wv[j] & 0xFFFFu);
        tile[r][ch * 8 + 2 * j + 1] = bf16_bits_to_float(wv[j] >> 16);
      }
    }
  } else {
    const float *xf = (const float *)x;
    float4 v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      const int r = idx >> 4, ch = idx & 15;
      const int64_t gr = r0 + r, gc = c0 + ch * 4;
      v[p] = (gr < rows && gc < cols) ? *(const float4 *)(xf + gr * cols + gc)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      const int r = idx >> 4, ch = idx & 15;
      tile[r][ch * 4 + 0] = v[p].x;
      tile[r][ch * 4 + 1] = v[p].y;
      tile[r][ch * 4 + 2] = v[p].z;
      tile[r][ch * 4 + 3] = v[p].w;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void *__restrict__ x, int64_t rows,
                                                            int64_t cols,
                                                            const uint32_t *__restrict__ partials,
                                                            int npart, fs4_nvfp4 rv, fs4_nvfp4 cv) {
  __shared__ float tile[kTile][kTile + 1];
  __shared__ Tables tab;
  __shared__ uint32_t red[kThreads / 64];
  // tensor scale from the amax partials (every workgroup reduces them itself)
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npart; i += kThreads) m = m > partials[i] ? m : partials[i];
  m = block_max_u32(m, red);
  const float amax = __builtin_bit_cast(float, m);
  const float s_t = (float)((double)amax / kTensorDiv);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (rv.codes) *rv.tscale = s_t;
    if (cv.codes) *cv.tscale = s_t;
  }
  build_tables(tab, s_t);
  // 1/(6 s_t) only seeds the scale-code estimate; the tables make it exact
  const float inv6st = s_t > 0.0f ? (float)(1.0 / (6.0 * (double)s_t)) : 0.0f;   // may be inf
  __syncthreads();

  const int64_t tiles_c = (cols + kTile - 1) / kTile, tiles_r = (rows + kTile - 1) / kTile;
  const int t = threadIdx.x;
  for (int64_t tile_id = blockIdx.x; tile_id < tiles_r * tiles_c; tile_id += gridDim.x) {
    const int64_t r0 = (tile_id / tiles_c) * kTile, c0 = (tile_id % tiles_c) * kTile;
    load_tile<BF16>(x, rows, cols, r0, c0, tile);
    __syncthreads();
    // four lanes per row (or column) write 32 contiguous code bytes
    const int line = t >> 2, blk = t & 3;
    if (rv.codes) {
      const int64_t gr = r0 + line, gc = c0 + blk * kBlock;
      if (gr < rows && gc < cols) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = tile[line][blk * kBlock + i];
        uint2 packed;
        const uint32_t sb = encode16(v, inv6st, tab, packed);
        *(uint2 *)(rv.codes + gr * (cols / 2) + gc / 2) = packed;
        rv.scales[gr * (cols / kBlock) + gc / kBlock] = (uint8_t)sb;
      }
    }
    if (cv.codes) {
      const int64_t gc = c0 + line, gr = r0 + blk * kBlock;
      if (gc < cols && gr < rows) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = tile[blk * kBlock + i][line];
        uint2 packed;
        const uint32_t sb = encode16(v, inv6st, tab, packed);
        *(uint2 *)(cv.codes + gc * (rows / 2) + gr / 2) = packed;
        cv.scales[gc * (rows / kBlock) + gr / kBlock] = (uint8_t)sb;
      }
    }
    __syncthreads();
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
  const int64_t g = (nvec + kThreads * kAmaxUnroll * 2 - 1) / (kThreads * kAmaxUnroll * 2);
  const int npart = (int)(g < 1 ? 1 : (g > kAmaxPartials ? kAmaxPartials : g));
  uint32_t *partials = (uint32_t *)ws;
  const int64_t tiles = ((cols + kTile - 1) / kTile) * ((rows + kTile - 1) / kTile);
  const unsigned grid = (unsigned)(tiles < kEncodeGrid ? tiles : kEncodeGrid);
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
