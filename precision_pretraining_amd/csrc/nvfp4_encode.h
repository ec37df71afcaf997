// NVFP4 block encoding from fp32 values, shared by the quantizer and the
// kernels that quantize what they compute (gfx950 device code).
//
//   s_t  = RNE_fp32(amax_t / 2688)            (the caller's)
//   s_b  = E4M3 RNE satfinite(amax_b / (6 s_t)) per 16 elements
//   code = sign | E2M1 RNE(|x| / (s_b s_t)) with the division exact
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
#pragma once
#include "fs4_common.h"

namespace fs4 {

// ---- lookup tables (per workgroup, from s_t) ---------------------------------
// e4p[c] = (e4t[c-1], e4t[c]), c = 0..126, where amax_b >= e4t[c] exactly when
//   the E4M3 scale code is at least c + 1 (e4t[-1] = -inf, e4t[126] = +inf):
//   one 8-byte read checks an estimate against both of its boundaries.
// rr[c] = (rlo, rhi), c = 0..126: the bracket of 1/(e4m3(c) s_t); rlo < 0 marks
//   a code whose blocks take the exact path; code 0 (step 0) has rlo = rhi = 0.
// eth[c][i], i = 0..6: |x| >= eth[c][i] exactly when the E2M1 index exceeds i
//   for scale code c.
struct Tables {
  float2 e4p[128];
  float2 rr[128];
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

template <int NT>
__device__ inline void build_tables_n(Tables &t, float s_t) {
  const double st = (double)s_t;
  // threshold between codes c and c+1 (ties to the even code), c = -1..126
  auto e4t = [&](int c) -> float {
    if (c < 0) return -__builtin_huge_valf();
    if (c >= 126 || !(st > 0.0)) return __builtin_huge_valf();
    const double mid = 0.5 * (e4m3_value(c) + e4m3_value(c + 1));
    return ge_threshold(mid * 6.0 * st, (c + 1) % 2 == 0);
  };
  for (int c = threadIdx.x; c < 128; c += NT) {
    t.e4p[c] = make_float2(e4t(c - 1), e4t(c));
    const double step = c < 127 ? e4m3_value(c) * st : 0.0;
    if (step > 0.0) {
      const double r = 1.0 / step;
      if (r < 0x1p120) t.rr[c] = make_float2((float)(r * (1.0 - 0x1p-20)), (float)(r * (1.0 + 0x1p-20)));
      else t.rr[c] = make_float2(-1.0f, -1.0f);
    } else {
      t.rr[c] = make_float2(0.0f, 0.0f);
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
// taken in fp32 (two roundings), to 3 mantissa bits (nearest, from the bit
// pattern; the subnormal range on the 2^-9 grid): it is within one code of the
// exact round-to-nearest-even code, so one compare against each of its two
// boundaries makes it exact.  When 1/(6 s_t) overflows fp32 (a subnormal s_t)
// the estimate means nothing and a binary search over the boundaries decides.
__device__ inline uint32_t scale_code(float amax, float inv6st, bool inv_finite, const Tables &t) {
  if (!(amax > 0.0f) || !(inv6st > 0.0f)) return 0u;
  if (inv_finite) {
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
    const float2 th = t.e4p[c];
    c += (amax >= th.y) ? 1 : (amax < th.x ? -1 : 0);
    return (uint32_t)c;
  }
  int lo = 0, hi = 126;                 // number of boundaries <= amax lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (amax >= t.e4p[mid].y) lo = mid + 1;
    else hi = mid;
  }
  return (uint32_t)lo;
}

// Encodes the 16 values rd(0..15) (rd reads LDS, and is called again for the
// rare element that needs an exact decision); returns the scale code and packs
// the codes (element 2j in the low nibble of byte j).
template <typename Reader>
__device__ inline uint32_t encode16(const Reader &rd, float inv6st, bool inv_finite, const Tables &t,
                                    uint2 &packed) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = rd(i);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sb = scale_code(amax, inv6st, inv_finite, t);
  const float2 rlh = t.rr[sb];
  const float rl = rlh.x, rh = rlh.y;
  const float *th = t.eth[sb];
  uint32_t lo0 = 0, lo1 = 0;
  if (rl >= 0.0f) {
    uint32_t hi0 = 0, hi1 = 0;
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
    // An element whose two codes differ lies within the bracket of a
    // midpoint; its code is the lower one, or the upper one when |x| reaches
    // the exact threshold above the lower magnitude.  Rare (mostly exact
    // rational ties of low-precision inputs, perturbed by the rounding of
    // s_t), so lanes loop over such elements one at a time.
    uint32_t d0 = lo0 ^ hi0, d1 = lo1 ^ hi1;
    while (d0 | d1) {
      const bool w1 = d0 == 0u;
      const uint32_t d = w1 ? d1 : d0;
      const uint32_t sh = (uint32_t)__builtin_ctz(d) & ~3u;
      const uint32_t lo = w1 ? lo1 : lo0, hi = w1 ? hi1 : hi0;
      const int e = (int)(sh >> 2) + (w1 ? 8 : 0);
      const float a = fabsf(rd(e));
      const uint32_t c = a >= th[(lo >> sh) & 7u] ? (hi >> sh) & 15u : (lo >> sh) & 15u;
      const uint32_t nl = (lo & ~(15u << sh)) | (c << sh);
      if (w1) {
        lo1 = nl;
        d1 &= ~(15u << sh);
      } else {
        lo0 = nl;
        d0 &= ~(15u << sh);
      }
    }
  } else {
    // 1/step beyond fp32's reach (tiny fp32 tensors): count the thresholds
    // each |x| reaches
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

}  // namespace fs4
