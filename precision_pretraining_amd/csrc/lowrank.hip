// BF16 low-rank side products of the LoRA-SVD projection and Newton-Schulz
// helpers, for gfx950.
//
// Full-Stack FP4 [FS4 §2.1] keeps the rank-r subspace L2 L1 = U V in BF16.
// The forward needs T = X V^T [M][r]; the backward needs P = dY U [M][r],
// dU = beta dY^T T [N][r] and dV = beta P^T X [r][K].  All are products with
// one output side <= 64 wide, written here as one strided kernel:
//
//   out[a][b] = scale * sum_k P(a, k) Q(b, k)
//   P(a, k) = P[a * p_sa + k * p_sk],  Q(b, k) = Q[b * q_sb + k * q_sk]
//
// Each operand is bf16 or fp32.  An fp32 operand is split into BF16 hi + lo
// parts (x = hi + lo + O(2^-17 |x|)) and runs as two MFMAs, so the products
// keep ~16 significant bits.  The k range is split over the 4 waves of a
// workgroup and over gridDim.y; partial sums go to a workspace and a second
// pass adds them in a fixed order (deterministic).
#include "fs4_common.h"

namespace fs4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

struct SmallGemm {
  const void *P;
  int64_t p_sa, p_sk;
  const void *Q;
  int64_t q_sb, q_sk;
  int64_t Na, Nb, Kc;
  int64_t kchunk;        // k per gridDim.y split (multiple of 64)
  float *partials;       // [S][Na][Nb]
};

__device__ inline bf16x8_t make_frag(const uint32_t *bits) {
  bf16x8_t f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = __builtin_bit_cast(__bf16, (uint16_t)bits[i]);
  return f;
}

// loads 8 consecutive-k values of one row of an operand as fp32
template <bool F32, bool CONTIG>
__device__ inline void load8(const void *base, int64_t row_off, int64_t sk, int64_t k, bool valid,
                             float *out) {
  if (!valid) {
#pragma unroll
    for (int q = 0; q < 8; ++q) out[q] = 0.0f;
    return;
  }
  if constexpr (F32) {
    const float *p = (const float *)base + row_off;
    if constexpr (CONTIG) {
      const float4 a = *(const float4 *)(p + k), b = *(const float4 *)(p + k + 4);
      out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
      out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] = p[(k + q) * sk];
    }
  } else {
    const uint16_t *p = (const uint16_t *)base + row_off;
    if constexpr (CONTIG) {
      const uint4 v = *(const uint4 *)(p + k);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        out[2 * q] = bf16_bits_to_float(w[q] & 0xFFFFu);
        out[2 * q + 1] = bf16_bits_to_float(w[q] >> 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) out[q] = bf16_bits_to_float(p[(k + q) * sk]);
    }
  }
}

template <bool P_F32, bool P_CONTIG, bool Q_F32, bool Q_CONTIG>
__global__ __launch_bounds__(256) void small_gemm_kernel(SmallGemm g) {
  __shared__ float red[3][64][17];
  const int64_t tiles_b = (g.Nb + 31) / 32;
  const int64_t ta = blockIdx.x / tiles_b, tb = blockIdx.x % tiles_b;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t a = ta * 32 + l32, b = tb * 32 + l32;
  const int64_t kw = g.kchunk / 4;
  int64_t kbeg = (int64_t)blockIdx.y * g.kchunk + wave * kw;
  int64_t kend = kbeg + kw;
  if (kend > g.Kc) kend = g.Kc;

  floatx16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;

  for (int64_t k0 = kbeg; k0 < kend; k0 += 16) {
    const int64_t k = k0 + 8 * h;
    float pv[8], qv[8];
    load8<P_F32, P_CONTIG>(g.P, a * g.p_sa, g.p_sk, k, a < g.Na, pv);
    load8<Q_F32, Q_CONTIG>(g.Q, b * g.q_sb, g.q_sk, k, b < g.Nb, qv);
    uint32_t ph[8], pl[8], qh[8], ql[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ph[q] = float_to_bf16_rne_bits(pv[q]);
      qh[q] = float_to_bf16_rne_bits(qv[q]);
      if constexpr (P_F32) pl[q] = float_to_bf16_rne_bits(pv[q] - bf16_bits_to_float(ph[q]));
      if constexpr (Q_F32) ql[q] = float_to_bf16_rne_bits(qv[q] - bf16_bits_to_float(qh[q]));
    }
    const bf16x8_t fph = make_frag(ph), fqh = make_frag(qh);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fph, fqh, acc, 0, 0, 0);
    if constexpr (P_F32) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(make_frag(pl), fqh, acc, 0, 0, 0);
    if constexpr (Q_F32) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fph, make_frag(ql), acc, 0, 0, 0);
  }

  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave - 1][lane][e] = acc[e];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += red[w][lane][e];
    float *out = g.partials + (int64_t)blockIdx.y * g.Na * g.Nb;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t ra = ta * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (ra < g.Na && b < g.Nb) out[ra * g.Nb + b] = acc[e];
    }
  }
}

__global__ void reduce_partials_kernel(const float *__restrict__ partials, int S, int64_t Na,
                                       int64_t Nb, float scale, float *__restrict__ out,
                                       bool transpose_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Na * Nb) return;
  float s = 0.0f;
  for (int p = 0; p < S; ++p) s += partials[(int64_t)p * Na * Nb + i];
  const int64_t ra = i / Nb, cb = i % Nb;
  out[transpose_out ? cb * Na + ra : i] = scale * s;
}

constexpr int64_t kChunkMin = 64;

int64_t pick_splits(int64_t tiles, int64_t Kc, int64_t *kchunk) {
  // aim at >= 1024 workgroups; each wave takes >= 16 k
  int64_t S = (1024 + tiles - 1) / tiles;
  int64_t maxS = (Kc + kChunkMin - 1) / kChunkMin;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  int64_t kc = (Kc + S - 1) / S;
  kc = (kc + kChunkMin - 1) / kChunkMin * kChunkMin;
  *kchunk = kc;
  return (Kc + kc - 1) / kc;
}

template <bool PF, bool PC, bool QF, bool QC>
fs4_status run_small(const SmallGemm &g0, int64_t S, float scale, float *out, bool transpose_out,
                     hipStream_t s) {
  const int64_t tiles = ((g0.Na + 31) / 32) * ((g0.Nb + 31) / 32);
  dim3 grid((unsigned)tiles, (unsigned)S);
  small_gemm_kernel<PF, PC, QF, QC><<<grid, 256, 0, s>>>(g0);
  const int64_t n = g0.Na * g0.Nb;
  reduce_partials_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(g0.partials, (int)S, g0.Na,
                                                                      g0.Nb, scale, out,
                                                                      transpose_out);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

template <bool PF, bool PC, bool QF>
fs4_status dispatch_q(bool qc, const SmallGemm &g, int64_t S, float scale, float *out, bool t,
                      hipStream_t s) {
  return qc ? run_small<PF, PC, QF, true>(g, S, scale, out, t, s)
            : run_small<PF, PC, QF, false>(g, S, scale, out, t, s);
}
template <bool PF, bool PC>
fs4_status dispatch_qf(bool qf, bool qc, const SmallGemm &g, int64_t S, float scale, float *out,
                       bool t, hipStream_t s) {
  return qf ? dispatch_q<PF, PC, true>(qc, g, S, scale, out, t, s)
            : dispatch_q<PF, PC, false>(qc, g, S, scale, out, t, s);
}
fs4_status dispatch_small(bool pf, bool pc, bool qf, bool qc, const SmallGemm &g, int64_t S,
                          float scale, float *out, bool t, hipStream_t s) {
  if (pf) return pc ? dispatch_qf<true, true>(qf, qc, g, S, scale, out, t, s)
                    : dispatch_qf<true, false>(qf, qc, g, S, scale, out, t, s);
  return pc ? dispatch_qf<false, true>(qf, qc, g, S, scale, out, t, s)
            : dispatch_qf<false, false>(qf, qc, g, S, scale, out, t, s);
}

}  // namespace

fs4_status launch_small_gemm(const void *P, bool p_f32, int64_t p_sa, int64_t p_sk, const void *Q,
                             bool q_f32, int64_t q_sb, int64_t q_sk, int64_t Na, int64_t Nb,
                             int64_t Kc, float scale, float *out, bool transpose_out,
                             float *partials, hipStream_t s) {
  if (Na == 0 || Nb == 0) return FS4_OK;
  SmallGemm g;
  g.P = P; g.p_sa = p_sa; g.p_sk = p_sk;
  g.Q = Q; g.q_sb = q_sb; g.q_sk = q_sk;
  g.Na = Na; g.Nb = Nb; g.Kc = Kc; g.partials = partials;
  const int64_t tiles = ((Na + 31) / 32) * ((Nb + 31) / 32);
  const int64_t S = pick_splits(tiles, Kc, &g.kchunk);
  // vector loads along k need unit k-stride and 8-element aligned rows
  const bool pc = p_sk == 1 && (p_sa % 8 == 0 || Na == 1);
  const bool qc = q_sk == 1 && (q_sb % 8 == 0 || Nb == 1);
  return dispatch_small(p_f32, pc, q_f32, qc, g, S, scale, out, transpose_out, s);
}

size_t small_gemm_partials_bytes(int64_t Na, int64_t Nb, int64_t Kc) {
  const int64_t tiles = ((Na + 31) / 32) * ((Nb + 31) / 32);
  int64_t kc;
  const int64_t S = pick_splits(tiles, Kc, &kc);
  return (size_t)(S * Na * Nb) * sizeof(float);
}

// ---------------------------------------------------------------------------
// Newton-Schulz helpers
namespace {

constexpr int kNormParts = 1024;

template <bool BF16>
__device__ inline double load_elem(const void *x, int64_t i) {
  if constexpr (BF16) return (double)bf16_bits_to_float(((const uint16_t *)x)[i]);
  else return (double)((const float *)x)[i];
}

template <bool BF16>
__global__ __launch_bounds__(256) void sumsq_kernel(const void *__restrict__ x, int64_t n,
                                                    double *__restrict__ parts) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const double v = load_elem<BF16>(x, i);
    s += v * v;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) parts[blockIdx.x] = red[0];
}

template <bool BF16>
__global__ __launch_bounds__(256) void scale_kernel(const void *__restrict__ x, int64_t n,
                                                    const double *__restrict__ parts, int nparts,
                                                    double eps, float *__restrict__ out) {
  __shared__ double inv_s;
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int p = 0; p < nparts; ++p) s += parts[p];
    inv_s = 1.0 / (__builtin_sqrt(s) + eps);
  }
  __syncthreads();
  const double inv = inv_s;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = (float)(load_elem<BF16>(x, i) * inv);
}

template <bool BF16>
__global__ __launch_bounds__(256) void copy_kernel(const void *__restrict__ x, int64_t n,
                                                   float *__restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = (float)load_elem<BF16>(x, i);
}

}  // namespace

size_t normalize_ws_bytes() { return kNormParts * sizeof(double); }

fs4_status launch_normalize(const void *G, fs4_dtype dt, int64_t n, float eps, float *X, void *ws,
                            hipStream_t s) {
  double *parts = (double *)ws;
  int64_t g = (n + 256 * 16 - 1) / (256 * 16);
  const int np = (int)(g < 1 ? 1 : (g > kNormParts ? kNormParts : g));
  const unsigned gs = (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  if (dt == FS4_BF16) {
    sumsq_kernel<true><<<np, 256, 0, s>>>(G, n, parts);
    scale_kernel<true><<<gs, 256, 0, s>>>(G, n, parts, np, (double)eps, X);
  } else {
    sumsq_kernel<false><<<np, 256, 0, s>>>(G, n, parts);
    scale_kernel<false><<<gs, 256, 0, s>>>(G, n, parts, np, (double)eps, X);
  }
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

fs4_status launch_copy_f32(const void *src, fs4_dtype dt, int64_t n, float *dst, hipStream_t s) {
  const unsigned gs = (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  if (n == 0) return FS4_OK;
  if (dt == FS4_BF16) copy_kernel<true><<<gs, 256, 0, s>>>(src, n, dst);
  else copy_kernel<false><<<gs, 256, 0, s>>>(src, n, dst);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
