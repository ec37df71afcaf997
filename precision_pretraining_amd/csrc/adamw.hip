// Q-AdamW optimizer-state codecs for gfx950: the second moment first, the
// first moment further below.
//
// Full-Stack FP4 [FS4 §2.2] stores the AdamW second moment v in NVFP4 after
// s = sqrt(v), the removal of a BF16 mean per 16 x 16 tile, and a Hadamard
// transform; decoding inverts the transform and the mean and squares:
//   encode: s = sqrt(v); mu = bf16(mean of s over the tile);
//           h = fp32(H/4 (s - mu)) per 16-element row group; NVFP4(h)
//   decode: s_hat = H/4 dequant(h) + mu; v_hat = fp32(s_hat^2)
// H is the 16-point Sylvester Hadamard matrix (H/4 is orthonormal and its
// own inverse), applied as butterflies (a, b) -> (a + b, a - b) with strides
// 1, 2, 4, 8.  Everything before a rounding to fp32 or BF16 runs in fp64 in
// that fixed order, and a tile's sum is the sum of its 16 row-group sums
// (each the butterflies' first output) in row order, so the fp32 values the
// quantizer sees are determined, and the codes with them.
//
// Encode is two launches: vstate_prep_kernel writes h (fp32 workspace), the
// BF16 means and per-workgroup amax partials of h; the quantizer's encode
// pass then quantizes h row-wise.  Decode is one launch.
#include <atomic>

#include "fs4_common.h"

namespace fs4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroups = 1024;   // within the quantizer's partials budget

__device__ inline void fwht16(double *x) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const double a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

// bf16 bits of the fp64 value x: round to fp32, then to 8 significant bits
// (each to nearest, ties to even)
__device__ inline uint32_t bf16_bits_of(double x) { return float_to_bf16_rne_bits((float)x); }

// One unit = 16 rows x 256 columns (16 tiles side by side); thread (i, j) =
// (t / 16, t % 16) owns the 16-element group of row i in tile j.
__global__ __launch_bounds__(kThreads) void vstate_prep_kernel(const float *__restrict__ v, int64_t R,
                                                               int64_t C, float *__restrict__ h,
                                                               uint16_t *__restrict__ means,
                                                               uint32_t *__restrict__ amax_parts) {
  __shared__ double gsum[16][17];
  __shared__ double mu[16];
  __shared__ uint32_t red[kThreads / 64];
  const int t = threadIdx.x, i = t >> 4, j = t & 15;
  const int64_t tiles_c = C / 16, groups_c = (tiles_c + 15) / 16;
  const int64_t units = (R / 16) * groups_c;
  float amax = 0.0f;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t tr = u / groups_c, tc = (u % groups_c) * 16 + j;
    const bool live = tc < tiles_c;
    const int64_t row = tr * 16 + i;
    double s[16];
    if (live) {
      const float4 *src = (const float4 *)(v + row * C + tc * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 w = src[q];
        s[4 * q] = __builtin_sqrt((double)w.x);
        s[4 * q + 1] = __builtin_sqrt((double)w.y);
        s[4 * q + 2] = __builtin_sqrt((double)w.z);
        s[4 * q + 3] = __builtin_sqrt((double)w.w);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) s[k] = 0.0;
    }
    double y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) y[k] = s[k];
    fwht16(y);
    gsum[i][j] = y[0];                       // the group's sum, in butterfly order
    __syncthreads();
    if (i == 0) {
      double tot = 0.0;
      for (int rr = 0; rr < 16; ++rr) tot += gsum[rr][j];
      const uint32_t b = bf16_bits_of(tot / 256.0);
      mu[j] = (double)bf16_bits_to_float(b);
      if (live) means[tr * tiles_c + tc] = (uint16_t)b;
    }
    __syncthreads();
    if (live) {
      const double m = mu[j];
#pragma unroll
      for (int k = 0; k < 16; ++k) y[k] = s[k] - m;
      fwht16(y);
      float o[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        o[k] = (float)(y[k] * 0.25);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(o[k]));
      }
      float4 *dst = (float4 *)(h + row * C + tc * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
    __syncthreads();   // gsum and mu are rewritten by the next unit
  }
  // workgroup max |h| as fp32 bits (the quantizer's partials format)
  uint32_t ub = __builtin_bit_cast(uint32_t, amax);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)ub, off, 64);
    ub = ub > o ? ub : o;
  }
  if ((t & 63) == 0) red[t >> 6] = ub;
  __syncthreads();
  if (t == 0) {
    uint32_t m = red[0];
    for (int w = 1; w < kThreads / 64; ++w) m = m > red[w] ? m : red[w];
    amax_parts[blockIdx.x] = m;
  }
}

// one thread per 16-element group: v_hat = fp32((H/4 dequant(h) + mu)^2)
__global__ __launch_bounds__(kThreads) void vstate_decode_kernel(const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ tscale,
                                                                 const uint16_t *__restrict__ means,
                                                                 int64_t R, int64_t C, float *__restrict__ out) {
  const int64_t groups_c = C / 16, total = R * groups_c;
  const double st = (double)*tscale;
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < total;
       gi += (int64_t)gridDim.x * kThreads) {
    const int64_t row = gi / groups_c, g = gi % groups_c;
    const uint2 cw = *(const uint2 *)(codes + row * (C / 2) + g * 8);
    const double sb = (double)e4m3_to_float(scales[row * groups_c + g]);
    const double m = (double)bf16_bits_to_float(means[(row / 16) * groups_c + g]);
    double y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t word = k < 8 ? cw.x : cw.y;
      const uint32_t code = (word >> (4 * (k & 7))) & 15u;
      const uint32_t mag = code & 7u;
      // E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
      const double e = mag < 4 ? 0.5 * (double)mag : (double)(2u << ((mag - 4) >> 1)) * ((mag & 1) ? 1.5 : 1.0);
      const double val = (code & 8u) ? -e : e;
      y[k] = val * sb * st;
    }
    fwht16(y);
    float o[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const double sh = y[k] * 0.25 + m;
      o[k] = (float)(sh * sh);
    }
    float4 *dst = (float4 *)(out + row * C + g * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  }
}

// ---- first moment --------------------------------------------------------
// [FS4 §2.2] mixes the first moment with the Hadamard transform, then
// quantizes it with stochastic rounding and adaptive 4/6 block scales:
//   h = fp32(H/4 m) per 16-element group; s_t = RNE_fp32(amax(h) / 2688);
//   per block, s_k = E4M3(amax_b / (k s_t)) for k = 6 and 4, keeping s_4 only
//   when its round-to-nearest squared error (summed over the block in order)
//   is smaller; each element then rounds up from the E2M1 magnitude below
//   y = |h| / (s_b s_t) exactly when u < (y - g_lo) / (g_hi - g_lo), with
//   u = r 2^-32 from the caller's uint32 r (saturating at 6);
//   decode: m_hat = fp32(H/4 dequant).
// Encode is two passes over m: the amax of h, then h again (the same fp64
// butterflies, so the same fp32 values) and its codes.

__device__ inline double e2m1_mag(int i) {
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6: in half units 0 1 2 3 4 6 8 12
  const int h = i < 4 ? i : ((2 | (i & 1)) << ((i >> 1) - 1));
  return 0.5 * (double)h;
}

// Index of the largest E2M1 magnitude <= y, for y >= 0 (an fp64 value): 0
// below 0.5, 1 below 1; from 1 on the magnitudes are the values with one
// mantissa bit, so the index follows from y's exponent e and its top mantissa
// bit b as 2 + 2e + b, capped at 7.
__device__ inline int e2m1_floor_idx(double y) {
  const uint32_t yh = (uint32_t)(__builtin_bit_cast(uint64_t, y) >> 32);
  if (yh < 0x3FE00000u) return 0;
  if (yh < 0x3FF00000u) return 1;
  const int i = 2 + 2 * ((int)(yh >> 20) - 1023) + (int)((yh >> 19) & 1u);
  return i < 7 ? i : 7;
}

// Index of the E2M1 magnitude nearest to mag / step (ties to the even
// index), decided as mag against midpoint * step: both products are exact in
// fp64 (a midpoint has <= 3 significant bits, step = e4m3 * s_t <= 28), and
// since mag has <= 24 significant bits a quotient that is not exactly a
// midpoint lies at least ~2^-31 (relative) away from it, far beyond the
// rounding of an fp64 quotient, so this is the decision the fp64 quotient
// mag / step makes, without the division.
__device__ inline int e2m1_rne_idx_scaled(double mag, double step) {
  int i = 0;
  i += mag > 0.25 * step;    // 0 | 0.5   tie -> 0
  i += mag >= 0.75 * step;   // 0.5 | 1   tie -> 1.0 (index 2)
  i += mag > 1.25 * step;    // 1 | 1.5   tie -> 1.0
  i += mag >= 1.75 * step;   // 1.5 | 2   tie -> 2.0 (index 4)
  i += mag > 2.5 * step;     // 2 | 3     tie -> 2.0
  i += mag >= 3.5 * step;    // 3 | 4     tie -> 4.0 (index 6)
  i += mag > 5.0 * step;     // 4 | 6     tie -> 4.0
  return i;
}

__global__ __launch_bounds__(kThreads) void mstate_prep_kernel(const float *__restrict__ m, int64_t R,
                                                               int64_t C, uint32_t *__restrict__ amax_parts) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t total = R * (C / 16);
  float amax = 0.0f;
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < total;
       gi += (int64_t)gridDim.x * kThreads) {
    const float4 *src = (const float4 *)(m + gi * 16);
    double y[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 w = src[q];
      y[4 * q] = w.x;
      y[4 * q + 1] = w.y;
      y[4 * q + 2] = w.z;
      y[4 * q + 3] = w.w;
    }
    fwht16(y);
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf((float)(y[k] * 0.25)));
  }
  uint32_t ub = __builtin_bit_cast(uint32_t, amax);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)ub, off, 64);
    ub = ub > o ? ub : o;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ub;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t mx = red[0];
    for (int w = 1; w < kThreads / 64; ++w) mx = mx > red[w] ? mx : red[w];
    amax_parts[blockIdx.x] = mx;
  }
}

__global__ __launch_bounds__(kThreads) void mstate_encode_kernel(const float *__restrict__ m, int64_t R, int64_t C,
                                                                 const uint32_t *__restrict__ rnd,
                                                                 const uint32_t *__restrict__ amax_parts,
                                                                 int nparts, fs4_nvfp4 q) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t mx = 0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) mx = mx > amax_parts[i] ? mx : amax_parts[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)mx, off, 64);
    mx = mx > o ? mx : o;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  uint32_t am = red[0];
  for (int w = 1; w < kThreads / 64; ++w) am = am > red[w] ? am : red[w];
  const float s_t = (float)((double)__builtin_bit_cast(float, am) / kTensorDiv);
  if (blockIdx.x == 0 && threadIdx.x == 0) *q.tscale = s_t;
  const double st = (double)s_t;
  const int64_t groups_c = C / 16, total = R * groups_c;
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < total;
       gi += (int64_t)gridDim.x * kThreads) {
    // the random words are loaded first, so that their latency hides behind
    // the transform and the scale choice
    const uint4 rw0 = *(const uint4 *)(rnd + gi * 16), rw1 = *(const uint4 *)(rnd + gi * 16 + 4);
    const uint4 rw2 = *(const uint4 *)(rnd + gi * 16 + 8), rw3 = *(const uint4 *)(rnd + gi * 16 + 12);
    // h of this group, recomputed from m exactly as the first pass did
    const float4 *src = (const float4 *)(m + gi * 16);
    double y[16];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float4 w = src[qq];
      y[4 * qq] = w.x;
      y[4 * qq + 1] = w.y;
      y[4 * qq + 2] = w.z;
      y[4 * qq + 3] = w.w;
    }
    fwht16(y);
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = (float)(y[k] * 0.25);
    double mag[16], amax_b = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      mag[k] = __builtin_fabs((double)x[k]);
      amax_b = amax_b > mag[k] ? amax_b : mag[k];
    }
    uint32_t sb = 0;
    if (st > 0.0) {
      const uint32_t s6 = e4m3_rne_satfinite(amax_b / (6.0 * st));
      const uint32_t s4 = e4m3_rne_satfinite(amax_b / (4.0 * st));
      double err[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const double step = (double)e4m3_to_float(c == 0 ? s6 : s4) * st;
        double tot = 0.0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const double val = step > 0.0 ? e2m1_mag(e2m1_rne_idx_scaled(mag[k], step)) * step : 0.0;
          const double d = mag[k] - val;
          tot = tot + d * d;
        }
        err[c] = tot;
      }
      sb = err[1] < err[0] ? s4 : s6;
    }
    const double step = (double)e4m3_to_float(sb) * st;
    const uint32_t rr[16] = {rw0.x, rw0.y, rw0.z, rw0.w, rw1.x, rw1.y, rw1.z, rw1.w,
                             rw2.x, rw2.y, rw2.z, rw2.w, rw3.x, rw3.y, rw3.z, rw3.w};
    uint32_t lo32 = 0, hi32 = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      uint32_t idx = 0;
      if (step > 0.0) {
        const double y = mag[k] / step;
        const int lo = e2m1_floor_idx(y);
        if (lo < 7) {
          // the gap to the next magnitude is 0.5, 1 or 2: multiplying by its
          // inverse is the division, exactly
          const double glo = e2m1_mag(lo);
          const double inv_gap = lo < 4 ? 2.0 : (lo < 6 ? 1.0 : 0.5);
          const double p = (y - glo) * inv_gap;
          const double u = (double)rr[k] * 0x1p-32;
          idx = (uint32_t)(u < p ? lo + 1 : lo);
        } else {
          idx = 7;
        }
      }
      const uint32_t code = idx | ((__builtin_bit_cast(uint32_t, x[k]) >> 28) & 8u);
      if (k < 8) lo32 |= code << (4 * k);
      else hi32 |= code << (4 * (k - 8));
    }
    const int64_t row = gi / groups_c, g = gi % groups_c;
    *(uint2 *)(q.codes + row * (C / 2) + g * 8) = make_uint2(lo32, hi32);
    q.scales[row * groups_c + g] = (uint8_t)sb;
  }
}

__global__ __launch_bounds__(kThreads) void mstate_decode_kernel(const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ tscale, int64_t R,
                                                                 int64_t C, float *__restrict__ out) {
  const int64_t groups_c = C / 16, total = R * groups_c;
  const double st = (double)*tscale;
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < total;
       gi += (int64_t)gridDim.x * kThreads) {
    const int64_t row = gi / groups_c, g = gi % groups_c;
    const uint2 cw = *(const uint2 *)(codes + row * (C / 2) + g * 8);
    const double sb = (double)e4m3_to_float(scales[row * groups_c + g]);
    double y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t code = ((k < 8 ? cw.x : cw.y) >> (4 * (k & 7))) & 15u;
      const double e = e2m1_mag((int)(code & 7u));
      y[k] = ((code & 8u) ? -e : e) * sb * st;
    }
    fwht16(y);
    float o[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] = (float)(y[k] * 0.25);
    float4 *dst = (float4 *)(out + row * C + g * 16);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) dst[qq] = make_float4(o[4 * qq], o[4 * qq + 1], o[4 * qq + 2], o[4 * qq + 3]);
  }
}

int prep_groups(int64_t R, int64_t C) {
  const int64_t units = (R / 16) * ((C / 16 + 15) / 16);
  return (int)(units < 1 ? 1 : (units > kMaxGroups ? kMaxGroups : units));
}

}  // namespace

size_t vstate_encode_ws_bytes(int64_t R, int64_t C) {
  Carver c(nullptr);
  c.take((size_t)(R * C) * sizeof(float));
  c.take((size_t)kMaxGroups * sizeof(uint32_t));
  return c.off;
}

fs4_status launch_vstate_encode(const float *v, int64_t R, int64_t C, const fs4_nvfp4 &q,
                                uint16_t *means, void *ws, hipStream_t s) {
  Carver c(ws);
  float *h = (float *)c.take((size_t)(R * C) * sizeof(float));
  uint32_t *parts = (uint32_t *)c.take((size_t)kMaxGroups * sizeof(uint32_t));
  const int g = prep_groups(R, C);
  vstate_prep_kernel<<<g, kThreads, 0, s>>>(v, R, C, h, means, parts);
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;
  return launch_quantize_encode(h, FS4_FP32, R, C, &q, nullptr, parts, g, s);
}

size_t mstate_encode_ws_bytes(int64_t, int64_t) { return (size_t)kMaxGroups * sizeof(uint32_t); }

namespace {
// Workgroups of the encode kernel that the current device holds at once (its
// register use allows three waves per SIMD).  A grid of that size runs the
// grid-stride loop in a single batch, where a larger one would leave a
// partial second batch on a fraction of the CUs.  Asked once per device.
int mstate_encode_resident() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kMaxGroups;
  int r = cached[dev].load(std::memory_order_relaxed);
  if (r == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, mstate_encode_kernel, kThreads, 0) == hipSuccess &&
        cus > 0 && per > 0)
      r = cus * per;
    else
      r = kMaxGroups;
    cached[dev].store(r, std::memory_order_relaxed);
  }
  return r;
}
}  // namespace

fs4_status launch_mstate_encode(const float *m, const uint32_t *rnd, int64_t R, int64_t C, const fs4_nvfp4 &q,
                                void *ws, hipStream_t s) {
  uint32_t *parts = (uint32_t *)ws;
  int64_t g = (R * (C / 16) + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > kMaxGroups ? kMaxGroups : g);
  // pass 1: amax of h; pass 2: h again from m, then the codes
  mstate_prep_kernel<<<(unsigned)g, kThreads, 0, s>>>(m, R, C, parts);
  int64_t ge = (R * (C / 16) + kThreads - 1) / kThreads;
  const int64_t res = mstate_encode_resident();
  ge = ge < 1 ? 1 : (ge > res ? res : ge);
  mstate_encode_kernel<<<(unsigned)ge, kThreads, 0, s>>>(m, R, C, rnd, parts, (int)g, q);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

fs4_status launch_mstate_decode(const fs4_nvfp4 &q, int64_t R, int64_t C, float *out, hipStream_t s) {
  int64_t blocks = (R * (C / 16) + kThreads - 1) / kThreads;
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  mstate_decode_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(q.codes, q.scales, q.tscale, R, C, out);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

fs4_status launch_vstate_decode(const fs4_nvfp4 &q, const uint16_t *means, int64_t R, int64_t C, float *out,
                                hipStream_t s) {
  int64_t blocks = (R * (C / 16) + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  vstate_decode_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(q.codes, q.scales, q.tscale, means, R, C, out);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
