// Exact nearest-rank quantile of |x| for gfx950, used for the p99 outlier
// clipping of the NVFP4 Newton-Schulz iterate (Full-Stack FP4 [FS4 §2.3]).
//
// The quantile is the k-th smallest magnitude, k = ceil(q n).  Magnitudes of
// finite floats order like their bit patterns with the sign bit cleared
// (31 bits), so the k-th smallest is found by radix selection over those
// bits, most significant digit first: bits 30..20, then 19..9, then 8..0.
// Each pass histograms the digit of the elements whose higher digits match
// the prefix found so far (LDS histograms per workgroup, added into one
// global histogram), and a one-workgroup scan picks the digit holding rank k
// and subtracts the ranks below it.  Three passes over x; no sorting and no
// floating point, so the result is exact.
#include "fs4_common.h"

namespace fs4 {
namespace {

constexpr int kThreads = 256;
constexpr int kBins = 2048;        // 11-bit digits (the last pass uses 512)
constexpr int kMaxGroups = 1024;

struct SelState {
  uint32_t prefix;    // digits found so far
  uint32_t pad;
  uint64_t krem;      // rank still to find among the elements matching prefix (1-based)
};

__global__ void sel_init_kernel(uint32_t *hist, SelState *st, uint64_t k) {
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) {
    st->prefix = 0;
    st->pad = 0;
    st->krem = k;
  }
}

// digit of magnitude bits b in pass P, and whether b matches the prefix
template <int P>
__device__ inline void digit_of(uint32_t b, uint32_t prefix, bool &match, uint32_t &d) {
  if constexpr (P == 0) {
    match = true;
    d = b >> 20;
  } else if constexpr (P == 1) {
    match = (b >> 20) == prefix;
    d = (b >> 9) & 0x7FFu;
  } else {
    match = (b >> 9) == prefix;
    d = b & 0x1FFu;
  }
}

template <bool BF16, int P>
__global__ __launch_bounds__(kThreads) void sel_hist_kernel(const void *__restrict__ x, int64_t n,
                                                            uint32_t *__restrict__ hist,
                                                            const SelState *__restrict__ st) {
  __shared__ uint32_t h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0;
  __syncthreads();
  const uint32_t prefix = st->prefix;
  constexpr int kPer = BF16 ? 8 : 4;                  // elements per 16-byte word
  const int64_t nvec = n / kPer;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    const uint4 v = ((const uint4 *)x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int hlf = 0; hlf < (BF16 ? 2 : 1); ++hlf) {
        const uint32_t b = BF16 ? (((w[j] >> (16 * hlf)) & 0x7FFFu) << 16) : (w[j] & 0x7FFFFFFFu);
        bool match;
        uint32_t d;
        digit_of<P>(b, prefix, match, d);
        if (match) atomicAdd(&h[d], 1u);
      }
    }
  }
  // the tail past the last whole word
  for (int64_t e = nvec * kPer + (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += stride) {
    const uint32_t b = BF16 ? (((uint32_t)((const uint16_t *)x)[e] & 0x7FFFu) << 16)
                            : (((const uint32_t *)x)[e] & 0x7FFFFFFFu);
    bool match;
    uint32_t d;
    digit_of<P>(b, prefix, match, d);
    if (match) atomicAdd(&h[d], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (h[i]) atomicAdd(&hist[i], h[i]);
}

// One workgroup: the digit d with (count below d) < krem <= (count up to d),
// then krem -= count below d, prefix = prefix << width | d, and the histogram
// is cleared for the next pass.  After the last pass, *out = the value.
__global__ __launch_bounds__(kThreads) void sel_scan_kernel(uint32_t *hist, SelState *st, int width,
                                                            float *out) {
  constexpr int kPerThread = kBins / kThreads;        // 8 consecutive bins per thread
  __shared__ uint64_t csum[kThreads];
  const int t = threadIdx.x;
  const int nb = 1 << width;
  uint64_t mine = 0;
  for (int i = 0; i < kPerThread; ++i) {
    const int bin = t * kPerThread + i;
    if (bin < nb) mine += hist[bin];
  }
  csum[t] = mine;
  __syncthreads();
  // inclusive scan over the 256 chunk sums (Hillis-Steele)
  for (int off = 1; off < kThreads; off <<= 1) {
    const uint64_t v = t >= off ? csum[t - off] : 0;
    __syncthreads();
    csum[t] += v;
    __syncthreads();
  }
  const uint64_t krem = st->krem;
  const uint64_t below_chunk = t ? csum[t - 1] : 0;
  __syncthreads();
  if (below_chunk < krem && krem <= csum[t]) {
    // the crossing is in this thread's chunk
    uint64_t below = below_chunk;
    int d = t * kPerThread;
    for (int i = 0; i < kPerThread; ++i) {
      const int bin = t * kPerThread + i;
      const uint64_t c = bin < nb ? hist[bin] : 0;
      if (below + c >= krem) {
        d = bin;
        break;
      }
      below += c;
    }
    const uint32_t prefix = (st->prefix << width) | (uint32_t)d;
    st->prefix = prefix;
    st->krem = krem - below;
    if (out) *out = __builtin_bit_cast(float, prefix);
  }
  __syncthreads();
  for (int i = t; i < kBins; i += kThreads) hist[i] = 0;
}

}  // namespace

size_t abs_quantile_ws_bytes() {
  Carver c(nullptr);
  c.take(kBins * sizeof(uint32_t));
  c.take(sizeof(SelState));
  return c.off;
}

fs4_status launch_abs_quantile(const void *x, fs4_dtype dt, int64_t n, double q, float *out, void *ws,
                               hipStream_t s) {
  Carver c(ws);
  uint32_t *hist = (uint32_t *)c.take(kBins * sizeof(uint32_t));
  SelState *st = (SelState *)c.take(sizeof(SelState));
  double kd = __builtin_ceil(q * (double)n);
  if (!(kd >= 1.0)) kd = 1.0;
  if (kd > (double)n) kd = (double)n;
  const uint64_t k = (uint64_t)kd;
  const bool bf16 = dt == FS4_BF16;
  const int64_t nvec = n / (bf16 ? 8 : 4);
  int64_t g = (nvec + kThreads - 1) / kThreads;
  g = g < 1 ? 1 : (g > kMaxGroups ? kMaxGroups : g);
  sel_init_kernel<<<1, kThreads, 0, s>>>(hist, st, k);
#define FS4_SEL_PASS(P, W, OUT)                                                                   \
  do {                                                                                            \
    if (bf16) sel_hist_kernel<true, P><<<(unsigned)g, kThreads, 0, s>>>(x, n, hist, st);          \
    else sel_hist_kernel<false, P><<<(unsigned)g, kThreads, 0, s>>>(x, n, hist, st);              \
    sel_scan_kernel<<<1, kThreads, 0, s>>>(hist, st, W, OUT);                                     \
  } while (0)
  FS4_SEL_PASS(0, 11, nullptr);
  FS4_SEL_PASS(1, 11, nullptr);
  FS4_SEL_PASS(2, 9, out);
#undef FS4_SEL_PASS
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
