// Q-AdamW second-moment state codec for gfx950.
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

fs4_status launch_vstate_decode(const fs4_nvfp4 &q, const uint16_t *means, int64_t R, int64_t C, float *out,
                                hipStream_t s) {
  int64_t blocks = (R * (C / 16) + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  vstate_decode_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(q.codes, q.scales, q.tscale, means, R, C, out);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
