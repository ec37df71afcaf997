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
#include <type_traits>

#include "fs4_common.h"

namespace fs4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

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

// One workgroup: a 32 x 32 tile of `out` over one k chunk, split over its 4
// waves.  Each wave issues the loads of kUnroll 16-k steps before converting
// and multiplying them, so several loads per lane are in flight.  With
// AMAX, the workgroup also writes the largest |P| it loaded (as fp32 bits) to
// amax_parts[its linear id]: when the grid covers P exactly once (one tile
// column), these are the tensor-amax partials of P.
constexpr int kUnroll = 4;

template <bool P_F32, bool P_CONTIG, bool Q_F32, bool Q_CONTIG, bool AMAX>
__global__ __launch_bounds__(256) void small_gemm_kernel(SmallGemm g, uint32_t *amax_parts) {
  __shared__ float red[3][64][17];
  __shared__ uint32_t mred[4];
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
  float pmax = 0.0f;

  for (int64_t k0 = kbeg; k0 < kend; k0 += 16 * kUnroll) {
    float pv[kUnroll][8], qv[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t k = k0 + 16 * u + 8 * h;
      const bool in = k0 + 16 * u < kend;       // kend - kbeg is a multiple of 16
      load8<P_F32, P_CONTIG>(g.P, a * g.p_sa, g.p_sk, k, in && a < g.Na, pv[u]);
      load8<Q_F32, Q_CONTIG>(g.Q, b * g.q_sb, g.q_sk, k, in && b < g.Nb, qv[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (k0 + 16 * u < kend) {
        uint32_t ph[8], pl[8], qh[8], ql[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if constexpr (AMAX) pmax = fmaxf(pmax, fabsf(pv[u][q]));
          ph[q] = float_to_bf16_rne_bits(pv[u][q]);
          qh[q] = float_to_bf16_rne_bits(qv[u][q]);
          if constexpr (P_F32) pl[q] = float_to_bf16_rne_bits(pv[u][q] - bf16_bits_to_float(ph[q]));
          if constexpr (Q_F32) ql[q] = float_to_bf16_rne_bits(qv[u][q] - bf16_bits_to_float(qh[q]));
        }
        const bf16x8_t fph = make_frag(ph), fqh = make_frag(qh);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fph, fqh, acc, 0, 0, 0);
        if constexpr (P_F32) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(make_frag(pl), fqh, acc, 0, 0, 0);
        if constexpr (Q_F32) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fph, make_frag(ql), acc, 0, 0, 0);
      }
    }
  }

  if constexpr (AMAX) {
    // |x| as fp32 bits is monotone; lanes holding no rows contribute 0
    uint32_t mv = __builtin_bit_cast(uint32_t, pmax);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o = __shfl_xor(mv, off, 64);
      mv = mv > o ? mv : o;
    }
    if (lane == 0) mred[wave] = mv;
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
    if constexpr (AMAX) {
      if (lane == 0) {
        uint32_t m = mred[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) m = m > mred[w] ? m : mred[w];
        amax_parts[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
      }
    }
  }
}

// sum over p = 0, 1, .., S - 1 (in that order) of partials[p * stride + i],
// unrolled so that eight loads are in flight
__device__ inline float sum_slots(const float *__restrict__ partials, int S, int64_t stride, int64_t i) {
  float s = 0.0f;
  int p = 0;
  for (; p + 8 <= S; p += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = partials[(int64_t)(p + q) * stride + i];
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
  for (; p < S; ++p) s += partials[(int64_t)p * stride + i];
  return s;
}

__global__ void reduce_partials_kernel(const float *__restrict__ partials, int S, int64_t Na,
                                       int64_t Nb, float scale, float *__restrict__ out,
                                       bool transpose_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Na * Nb) return;
  const float s = sum_slots(partials, S, Na * Nb, i);
  const int64_t ra = i / Nb, cb = i % Nb;
  out[transpose_out ? cb * Na + ra : i] = scale * s;
}

// x = hi + lo as BF16 parts (x - hi rounded to BF16; |lo| <= 2^-9 |x|)
__device__ inline void split_bf16(float x, uint16_t *hi, uint16_t *lo) {
  const uint32_t hb = float_to_bf16_rne_bits(x);
  *hi = (uint16_t)hb;
  *lo = (uint16_t)float_to_bf16_rne_bits(x - bf16_bits_to_float(hb));
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
                     uint32_t *amax_parts, hipStream_t s) {
  const int64_t tiles = ((g0.Na + 31) / 32) * ((g0.Nb + 31) / 32);
  dim3 grid((unsigned)tiles, (unsigned)S);
  if (amax_parts)
    small_gemm_kernel<PF, PC, QF, QC, true><<<grid, 256, 0, s>>>(g0, amax_parts);
  else
    small_gemm_kernel<PF, PC, QF, QC, false><<<grid, 256, 0, s>>>(g0, nullptr);
  const int64_t n = g0.Na * g0.Nb;
  reduce_partials_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(g0.partials, (int)S, g0.Na,
                                                                      g0.Nb, scale, out,
                                                                      transpose_out);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

template <bool PF, bool PC, bool QF>
fs4_status dispatch_q(bool qc, const SmallGemm &g, int64_t S, float scale, float *out, bool t,
                      uint32_t *am, hipStream_t s) {
  return qc ? run_small<PF, PC, QF, true>(g, S, scale, out, t, am, s)
            : run_small<PF, PC, QF, false>(g, S, scale, out, t, am, s);
}
template <bool PF, bool PC>
fs4_status dispatch_qf(bool qf, bool qc, const SmallGemm &g, int64_t S, float scale, float *out,
                       bool t, uint32_t *am, hipStream_t s) {
  return qf ? dispatch_q<PF, PC, true>(qc, g, S, scale, out, t, am, s)
            : dispatch_q<PF, PC, false>(qc, g, S, scale, out, t, am, s);
}
fs4_status dispatch_small(bool pf, bool pc, bool qf, bool qc, const SmallGemm &g, int64_t S,
                          float scale, float *out, bool t, uint32_t *am, hipStream_t s) {
  if (pf) return pc ? dispatch_qf<true, true>(qf, qc, g, S, scale, out, t, am, s)
                    : dispatch_qf<true, false>(qf, qc, g, S, scale, out, t, am, s);
  return pc ? dispatch_qf<false, true>(qf, qc, g, S, scale, out, t, am, s)
            : dispatch_qf<false, false>(qf, qc, g, S, scale, out, t, am, s);
}

// ---------------------------------------------------------------------------
// Skinny products for the rank-r (r <= 64) side of the LoRA-SVD projection,
// shaped for HBM bandwidth: every global load is a 16-byte word of a row
// segment (whole cache lines per wave), operands are staged row-major in LDS
// and the MFMA fragments are read from there.
//
// rowred: part[s][a][j] = sum_{k in chunk s} A[a][k] B[j][k]
//   A bf16 [Na][K], B bf16 [r][K], both contiguous along k.  A workgroup owns
//   64 rows of A and one k chunk, walked in 128-k slabs (the next slab's loads
//   in flight); its 4 waves take 2 row tiles x 2 k halves.  With AMAX it also
//   writes the largest |A| it read (fp32 bits) to amax_parts[its linear id].
// colred: part[s][c][j] = sum_{m in chunk s} A[m][c] Bm[m][j]
//   A bf16 [M][C] row-major; Bm given as its transposed BF16 hi/lo split
//   (bt_hi, bt_lo [r][M]).  A workgroup owns 128 columns and one m chunk,
//   walked in 64-row slabs; wave w takes columns 32w..32w+31 and reads its
//   A fragments down the LDS columns (2-byte reads, conflict-free).
constexpr int kRrRows = 64, kRrK = 128, kRrStride = kRrK + 8;   // 272-byte LDS rows

template <bool AMAX, int NJ>
__global__ __launch_bounds__(256) void rowred_kernel(const uint16_t *__restrict__ A,
                                                     const uint16_t *__restrict__ B, int64_t Na,
                                                     int r, int64_t K, int64_t kchunk,
                                                     float *__restrict__ part,
                                                     uint32_t *__restrict__ amax_parts) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[kRrRows][kRrStride];
  __shared__ __attribute__((aligned(16))) uint16_t sb[NJ * 32][kRrStride];
  __shared__ float red[2][NJ][64][17];
  __shared__ uint32_t mred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int rt = wave & 1, kh = wave >> 1;
  const int64_t a0 = (int64_t)blockIdx.x * kRrRows;
  const int64_t kbeg = (int64_t)blockIdx.y * kchunk;
  const int64_t kend = kbeg + kchunk < K ? kbeg + kchunk : K;
  // slab loads: A 64 x 128 (4 words per thread), B NJ*32 x 128 (2*NJ per thread);
  // 16 threads per 256-byte row segment
  uint4 ga[4], gb[2 * NJ];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = tid + p * 256, row = idx >> 4, seg = idx & 15;
      const int64_t k = k0 + seg * 8;
      ga[p] = (a0 + row < Na && k < kend) ? *(const uint4 *)(A + (a0 + row) * K + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 2 * NJ; ++p) {
      const int idx = tid + p * 256, j = idx >> 4, seg = idx & 15;
      const int64_t k = k0 + seg * 8;
      gb[p] = (j < r && k < kend) ? *(const uint4 *)(B + (int64_t)j * K + k) : make_uint4(0, 0, 0, 0);
    }
  };
  floatx16_t acc[NJ];
#pragma unroll
  for (int t = 0; t < NJ; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
  uint32_t amax = 0;    // bf16 magnitude bits
  if (kbeg < kend) gload(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += kRrK) {
    __syncthreads();          // the previous slab is fully read
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = tid + p * 256, row = idx >> 4, seg = idx & 15;
      *(uint4 *)&sa[row][seg * 8] = ga[p];
      if constexpr (AMAX) {
        const uint32_t w[4] = {ga[p].x, ga[p].y, ga[p].z, ga[p].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = w[q] & 0x7FFFu, hi = (w[q] >> 16) & 0x7FFFu;
          const uint32_t m2 = lo > hi ? lo : hi;
          amax = amax > m2 ? amax : m2;
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 2 * NJ; ++p) {
      const int idx = tid + p * 256, j = idx >> 4, seg = idx & 15;
      *(uint4 *)&sb[j][seg * 8] = gb[p];
    }
    __syncthreads();
    if (k0 + kRrK < kend) gload(k0 + kRrK);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kk = kh * 64 + st * 16 + 8 * h;
      const bf16x8_t fa = *(const bf16x8_t *)&sa[rt * 32 + l32][kk];
#pragma unroll
      for (int t = 0; t < NJ; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, *(const bf16x8_t *)&sb[t * 32 + l32][kk], acc[t], 0, 0, 0);
    }
  }
  if constexpr (AMAX) {
    uint32_t mv = amax << 16;   // bf16 magnitude bits -> fp32 bits
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o = __shfl_xor(mv, off, 64);
      mv = mv > o ? mv : o;
    }
    if (lane == 0) mred[wave] = mv;
  }
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < NJ; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[rt][t][lane][e] = acc[t][e];
  }
  __syncthreads();
  if (kh == 0) {
    float *out = part + (int64_t)blockIdx.y * Na * r;
#pragma unroll
    for (int t = 0; t < NJ; ++t) {
      const int j = t * 32 + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t ra = a0 + rt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (ra < Na && j < r) out[ra * r + j] = acc[t][e] + red[rt][t][lane][e];
      }
    }
  }
  if constexpr (AMAX) {
    if (tid == 0) {
      uint32_t m = mred[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) m = m > mred[w] ? m : mred[w];
      amax_parts[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
    }
  }
}

constexpr int kColBlock = 128;   // columns of A per workgroup (4 waves x 32)
constexpr int kColSlab = 64;     // rows of A per LDS slab
constexpr int kColAStride = kColBlock + 8;   // 272-byte LDS rows
constexpr int kColBStride = kColSlab + 8;    // 144-byte LDS rows

template <int NJ>
__global__ __launch_bounds__(256) void colred_kernel(const uint16_t *__restrict__ A,
                                                     const uint16_t *__restrict__ bt_hi,
                                                     const uint16_t *__restrict__ bt_lo,
                                                     int64_t M, int64_t C, int r, int64_t mchunk,
                                                     float *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[kColSlab][kColAStride];   // A slab [m][c]
  __shared__ __attribute__((aligned(16))) uint16_t sh[NJ * 32][kColBStride];    // Bm^T hi [j][m]
  __shared__ __attribute__((aligned(16))) uint16_t sl[NJ * 32][kColBStride];    // Bm^T lo [j][m]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t c0 = (int64_t)blockIdx.x * kColBlock;
  const int64_t mbeg = (int64_t)blockIdx.y * mchunk;
  const int64_t mend = mbeg + mchunk < M ? mbeg + mchunk : M;
  // slab loads: A 64 x 128 (4 words per thread, 16 threads per row segment);
  // Bm^T hi and lo NJ*32 x 64 (NJ words each per thread, 8 threads per row)
  uint4 ga[4], gh[NJ], gl[NJ];
  auto gload = [&](int64_t m0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = tid + p * 256, row = idx >> 4, seg = idx & 15;
      const int64_t m = m0 + row, c = c0 + seg * 8;
      ga[p] = (m < mend && c < C) ? *(const uint4 *)(A + m * C + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < NJ; ++p) {
      const int idx = tid + p * 256, j = idx >> 3, seg = idx & 7;
      const int64_t m = m0 + seg * 8;
      const bool in = j < r && m < mend;
      gh[p] = in ? *(const uint4 *)(bt_hi + (int64_t)j * M + m) : make_uint4(0, 0, 0, 0);
      gl[p] = in ? *(const uint4 *)(bt_lo + (int64_t)j * M + m) : make_uint4(0, 0, 0, 0);
    }
  };
  floatx16_t acc[NJ];
#pragma unroll
  for (int t = 0; t < NJ; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
  if (mbeg < mend) gload(mbeg);
  const int col = wave * 32 + l32;
  for (int64_t m0 = mbeg; m0 < mend; m0 += kColSlab) {
    __syncthreads();            // the previous slab is fully read
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = tid + p * 256, row = idx >> 4, seg = idx & 15;
      *(uint4 *)&sa[row][seg * 8] = ga[p];
    }
#pragma unroll
    for (int p = 0; p < NJ; ++p) {
      const int idx = tid + p * 256, j = idx >> 3, seg = idx & 7;
      *(uint4 *)&sh[j][seg * 8] = gh[p];
      *(uint4 *)&sl[j][seg * 8] = gl[p];
    }
    __syncthreads();
    if (m0 + kColSlab < mend) gload(m0 + kColSlab);   // next slab in flight during the MFMAs
#pragma unroll
    for (int st = 0; st < kColSlab / 16; ++st) {
      const int mm = st * 16 + 8 * h;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = (uint32_t)sa[mm + 2 * q][col] | ((uint32_t)sa[mm + 2 * q + 1][col] << 16);
      const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
      for (int t = 0; t < NJ; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, *(const bf16x8_t *)&sh[t * 32 + l32][mm], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, *(const bf16x8_t *)&sl[t * 32 + l32][mm], acc[t], 0, 0, 0);
      }
    }
  }
  float *out = part + (int64_t)blockIdx.y * C * r;
#pragma unroll
  for (int t = 0; t < NJ; ++t) {
    const int j = t * 32 + l32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t c = c0 + wave * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (c < C && j < r) out[c * r + j] = acc[t][e];
    }
  }
}

// Bm fp32 [M][r] -> transposed BF16 hi and lo parts [r][M] (Bm = hi + lo +
// O(2^-17 |Bm|))
__global__ void split_transpose_kernel(const float *__restrict__ Bm, int64_t M, int r,
                                       uint16_t *__restrict__ hi, uint16_t *__restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * r) return;
  const int64_t j = i / M, m = i % M;
  split_bf16(Bm[m * r + j], hi + i, lo + i);
}

// U [N][r] -> U^T [r][N] (bf16)
__global__ void transpose_rank_kernel(const uint16_t *__restrict__ U, int64_t N, int r,
                                      uint16_t *__restrict__ Ut) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * r) return;
  const int64_t j = i / N, n = i % N;
  Ut[i] = U[n * r + j];
}

// The operand preparation of the dual pass in one launch: U [N][r] -> U^T
// [r][N] (bf16, the first N r threads) and Bm fp32 [M][r] -> its transposed
// BF16 hi/lo split [r][M] (the next M r).
__global__ void rank_prep_kernel(const uint16_t *__restrict__ U, int64_t N, int r, uint16_t *__restrict__ Ut,
                                 const float *__restrict__ Bm, int64_t M, uint16_t *__restrict__ hi,
                                 uint16_t *__restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, nu = N * r;
  if (i < nu) {
    const int64_t j = i / N, n = i % N;
    Ut[i] = U[n * r + j];
    return;
  }
  const int64_t k = i - nu;
  if (k >= M * r) return;
  const int64_t j = k / M, m = k % M;
  split_bf16(Bm[m * r + j], hi + k, lo + k);
}

// Both reductions of the dual pass in one launch, each in slot order:
// P[m][j] = p_scale sum over its cb slots (the first M r threads), with
// P's transposed BF16 hi/lo split [r][M] when p_hi is given (the operand of
// the later column pass over X), and Q[n][j] = q_scale sum over its rb
// slots (the next N r).
__global__ void dual_reduce_kernel(const float *__restrict__ ppart, int cb, int64_t M, float p_scale,
                                   float *__restrict__ P, uint16_t *__restrict__ p_hi, uint16_t *__restrict__ p_lo,
                                   const float *__restrict__ qpart, int rb, int64_t N, float q_scale,
                                   float *__restrict__ Q, int r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, np = M * r;
  if (i < np) {
    const float v = p_scale * sum_slots(ppart, cb, np, i);
    P[i] = v;
    if (p_hi) {
      const int64_t m = i / r, j = i % r;
      split_bf16(v, p_hi + j * M + m, p_lo + j * M + m);
    }
    return;
  }
  const int64_t k = i - np;
  if (k >= N * r) return;
  Q[k] = q_scale * sum_slots(qpart, rb, N * r, k);
}

// dualred: both rank-r contractions of one bf16 matrix A [M][N] in a single
// read of it (r <= 32):
//   P[m][j]  = sum_n A[m][n] B[j][n]          (along the rows of A)
//   Q[n][j]  = sum_m A[m][n] Bm[m][j]         (down its columns)
// with B bf16 [r][N] and Bm fp32 [M][r], given as its transposed BF16 hi/lo
// split (bt_hi, bt_lo [r][M]).  In the LoRA-SVD backward A = dY, B = U^T and
// Bm = T: P = dY U feeds the dX epilogue and Q = dY^T T is dU.
// A workgroup owns a 512 x 512 block of A, walked in 64-row slabs staged in
// LDS (the next slab's loads in flight), with its 512 columns of B staged
// once.  Per slab, waves 0 and 1 form the slab's two 32-row tiles of P over
// the block's columns and store them to partial slot "column block"; every
// wave adds the slab into the Q rows of its 64 columns, kept in registers
// over the block's 512 rows and stored to partial slot "row block" at the
// end.  Two reductions then add the slots in order (deterministic).  With
// amax_parts, each workgroup also writes the largest |A| of its block (fp32
// bits).
constexpr int kDrCols = 512, kDrRows = 512, kDrSlab = 64;
constexpr int kDrStride = kDrCols + 8;     // 1040-byte LDS rows
constexpr int kDrThreads = 512;
constexpr int kRawBufferWord3 = 0x00020000;   // buffer resource word 3: 32-bit untyped access

__global__ __launch_bounds__(kDrThreads) void dualred_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ bt_hi, const uint16_t *__restrict__ bt_lo, int64_t M, int64_t N,
    int r, float *__restrict__ ppart, float *__restrict__ qpart, uint32_t *__restrict__ amax_parts) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[kDrSlab][kDrStride];      // A slab [m][n]
  __shared__ __attribute__((aligned(16))) uint16_t sb[32][kDrStride];           // B [j][n]
  __shared__ __attribute__((aligned(16))) uint16_t sh[32][kDrSlab + 8];         // Bm^T hi [j][m]
  __shared__ __attribute__((aligned(16))) uint16_t sl[32][kDrSlab + 8];         // Bm^T lo [j][m]
  __shared__ uint32_t smax;
  if (threadIdx.x == 0) smax = 0;   // (published by the first slab's barrier)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * kDrCols, mb0 = (int64_t)blockIdx.y * kDrRows;
  const int64_t mlim = mb0 + kDrRows < M ? mb0 + kDrRows : M;

  // B's 32 x 512 block, once (64 threads per row)
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = tid + p * kDrThreads, j = idx >> 6, seg = idx & 63;
    const int64_t n = n0 + seg * 8;
    const uint4 v = (j < r && n < N) ? *(const uint4 *)(B + (int64_t)j * N + n) : make_uint4(0, 0, 0, 0);
    *(uint4 *)&sb[j][seg * 8] = v;
  }
  // Slab loads: A 64 x 512 (8 words per thread; word p of a thread is slab
  // row wave + 8p at column n0 + 8 lane, so a wave reads 1 KB of one row);
  // Bm^T hi (waves 0-3) or lo (waves 4-7) 32 x 64.  The next slab's loads are
  // in flight while a slab is multiplied (a second slab in flight measured no
  // faster).  Raw buffer loads take the row's byte offset in a scalar
  // register and the column's in a vector one (the launcher keeps M N and M r
  // below 2^30).  Columns past N load the last 8 columns and Bm^T rows past r
  // or M its last row or columns; these are zeroed by a mask where they are
  // stored to LDS (a select right behind the load, or one in a branch, makes
  // the compiler wait for the load there).
  uint4 ga[8], gt;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool col_ok = n0 + lane * 8 < N;
  const int col_off = (int)((col_ok ? n0 + lane * 8 : N - 8) * 2);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, (int)(M * N * 2), kRawBufferWord3);
  const int tj = (tid & 255) >> 3, tseg = tid & 7;
  const __amdgpu_buffer_rsrc_t rt_ = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(wave_u < 4 ? bt_hi : bt_lo), 0, (int)(M * r * 2), kRawBufferWord3);
  const int t_row = (tj < r ? tj : r - 1) * (int)M;
  auto gload = [&](int64_t m0) {
    const int64_t tm = m0 + tseg * 8;
    const int t_off = (t_row + (int)(tm < M ? tm : M - 8)) * 2;
    gt = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rt_, t_off, 0, 0));
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t m = m0 + wave_u + 8 * p;
      const int roff = (int)((m < mlim ? m : mlim - 1) * N * 2);
      ga[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, col_off, roff, 0));
    }
  };

  floatx16_t accq[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) accq[c][e] = 0.0f;
  gload(mb0);
  for (int64_t m0 = mb0; m0 < mlim; m0 += kDrSlab) {
    __syncthreads();          // the previous slab is fully read
    u16x2_t am2 = {0, 0};     // max bf16 magnitude bits, two lanes of 16
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t keep = (col_ok && m0 + wave_u + 8 * p < mlim) ? 0xFFFFFFFFu : 0u;
      const uint4 v = make_uint4(ga[p].x & keep, ga[p].y & keep, ga[p].z & keep, ga[p].w & keep);
      *(uint4 *)&sa[wave + 8 * p][lane * 8] = v;
      am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu));
      am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu));
      am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu));
      am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu));
    }
    if (amax_parts) {
      // the slab's max |A| per wave, folded into the block's in LDS (a value
      // carried in registers across the slabs costs the loop its registers)
      uint32_t mv = am2[0] > am2[1] ? am2[0] : am2[1];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = __shfl_xor(mv, off, 64);
        mv = mv > o ? mv : o;
      }
      if (lane == 0) atomicMax(&smax, mv);
    }
    {
      const uint32_t keep = (tj < r && m0 + tseg * 8 < mlim) ? 0xFFFFFFFFu : 0u;
      *(uint4 *)&(wave_u < 4 ? sh : sl)[tj][tseg * 8] =
          make_uint4(gt.x & keep, gt.y & keep, gt.z & keep, gt.w & keep);
    }
    __syncthreads();
    if (m0 + kDrSlab < mlim) gload(m0 + kDrSlab);
    if (wave < 2) {
      // P: waves 0 and 1 take one 32-row tile each, over all 512 columns (no
      // sum across waves), and store it to the partial slot
      floatx16_t accp;
#pragma unroll
      for (int e = 0; e < 16; ++e) accp[e] = 0.0f;
#pragma unroll
      for (int st = 0; st < kDrCols / 16; ++st) {
        const int kk = st * 16 + 8 * h;
        accp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t *)&sa[wave * 32 + l32][kk],
                                                       *(const bf16x8_t *)&sb[l32][kk], accp, 0, 0, 0);
      }
      float *out = ppart + (int64_t)blockIdx.x * M * r;
      const int j = l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t rw = m0 + wave * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (rw < mlim && j < r) out[rw * r + j] = accp[e];
      }
    }
    // Q: the slab's rows into this wave's 64 columns (A fragments read down
    // the LDS columns)
#pragma unroll
    for (int st = 0; st < kDrSlab / 16; ++st) {
      const int mm = st * 16 + 8 * h;
      const bf16x8_t fh = *(const bf16x8_t *)&sh[l32][mm], fl = *(const bf16x8_t *)&sl[l32][mm];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = wave * 64 + c * 32 + l32;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)sa[mm + 2 * q][col] | ((uint32_t)sa[mm + 2 * q + 1][col] << 16);
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        accq[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fh, accq[c], 0, 0, 0);
        accq[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fl, accq[c], 0, 0, 0);
      }
    }
  }
  {
    float *out = qpart + (int64_t)blockIdx.y * N * r;
    const int j = l32;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t col = n0 + wave * 64 + c * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (col < N && j < r) out[col * r + j] = accq[c][e];
      }
  }
  if (amax_parts) {
    __syncthreads();
    if (tid == 0) amax_parts[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = smax << 16;   // -> fp32 bits
  }
}

int64_t rowred_splits(int64_t Na, int64_t K, int64_t *kchunk) {
  const int64_t blocks = (Na + kRrRows - 1) / kRrRows;
  // >= 1024 workgroups when K allows, chunks of whole 128-k slabs
  int64_t S = (1024 + blocks - 1) / blocks;
  const int64_t maxS = (K + kRrK - 1) / kRrK;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  int64_t kc = (K + S - 1) / S;
  kc = (kc + kRrK - 1) / kRrK * kRrK;
  *kchunk = kc;
  return (K + kc - 1) / kc;
}

int64_t colred_splits(int64_t M, int64_t C, int64_t *mchunk) {
  const int64_t blocks = (C + kColBlock - 1) / kColBlock;
  int64_t S = (1024 + blocks - 1) / blocks;
  const int64_t maxS = (M + kColSlab - 1) / kColSlab;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  int64_t mc = (M + S - 1) / S;
  mc = (mc + kColSlab - 1) / kColSlab * kColSlab;
  *mchunk = mc;
  return (M + mc - 1) / mc;
}

}  // namespace

fs4_status launch_small_gemm(const void *P, bool p_f32, int64_t p_sa, int64_t p_sk, const void *Q,
                             bool q_f32, int64_t q_sb, int64_t q_sk, int64_t Na, int64_t Nb,
                             int64_t Kc, float scale, float *out, bool transpose_out,
                             float *partials, hipStream_t s, uint32_t *amax_parts) {
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
  return dispatch_small(p_f32, pc, q_f32, qc, g, S, scale, out, transpose_out, amax_parts, s);
}

int64_t small_gemm_workgroups(int64_t Na, int64_t Nb, int64_t Kc) {
  const int64_t tiles = ((Na + 31) / 32) * ((Nb + 31) / 32);
  int64_t kc;
  return tiles * pick_splits(tiles, Kc, &kc);
}

size_t rowred_partials_bytes(int64_t Na, int r, int64_t K) {
  int64_t kc;
  return (size_t)(rowred_splits(Na, K, &kc) * Na * r) * sizeof(float);
}
int64_t rowred_workgroups(int64_t Na, int64_t K) {
  int64_t kc;
  return ((Na + kRrRows - 1) / kRrRows) * rowred_splits(Na, K, &kc);
}
fs4_status launch_rowred(const uint16_t *A, const uint16_t *B, int64_t Na, int r, int64_t K,
                         float scale, float *out, float *partials, uint32_t *amax_parts,
                         hipStream_t s) {
  if (Na == 0 || r == 0) return FS4_OK;
  int64_t kc;
  const int64_t S = rowred_splits(Na, K, &kc);
  dim3 grid((unsigned)((Na + kRrRows - 1) / kRrRows), (unsigned)S);
  if (r <= 32) {
    if (amax_parts) rowred_kernel<true, 1><<<grid, 256, 0, s>>>(A, B, Na, r, K, kc, partials, amax_parts);
    else rowred_kernel<false, 1><<<grid, 256, 0, s>>>(A, B, Na, r, K, kc, partials, nullptr);
  } else {
    if (amax_parts) rowred_kernel<true, 2><<<grid, 256, 0, s>>>(A, B, Na, r, K, kc, partials, amax_parts);
    else rowred_kernel<false, 2><<<grid, 256, 0, s>>>(A, B, Na, r, K, kc, partials, nullptr);
  }
  const int64_t n = Na * r;
  reduce_partials_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(partials, (int)S, Na, r, scale,
                                                                      out, false);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}
size_t colred_partials_bytes(int64_t M, int64_t C, int r) {
  int64_t mc;
  return (size_t)(colred_splits(M, C, &mc) * C * r) * sizeof(float);
}
fs4_status launch_colred(const uint16_t *A, const float *Bm, int64_t M, int64_t C, int r,
                         float scale, float *out, bool transpose_out, float *partials,
                         uint16_t *bt, hipStream_t s, bool presplit) {
  if (C == 0 || r == 0) return FS4_OK;
  uint16_t *bt_hi = bt, *bt_lo = bt + M * r;
  const int64_t nb = M * r;
  if (!presplit) split_transpose_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, s>>>(Bm, M, r, bt_hi, bt_lo);
  int64_t mc;
  const int64_t S = colred_splits(M, C, &mc);
  dim3 grid((unsigned)((C + kColBlock - 1) / kColBlock), (unsigned)S);
  if (r <= 32) colred_kernel<1><<<grid, 256, 0, s>>>(A, bt_hi, bt_lo, M, C, r, mc, partials);
  else colred_kernel<2><<<grid, 256, 0, s>>>(A, bt_hi, bt_lo, M, C, r, mc, partials);
  const int64_t n = C * r;
  reduce_partials_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(partials, (int)S, C, r, scale,
                                                                      out, transpose_out);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}
size_t dualred_partials_bytes(int64_t M, int64_t N, int r) {
  const int64_t cb = (N + kDrCols - 1) / kDrCols, rb = (M + kDrRows - 1) / kDrRows;
  return (size_t)((cb * M + rb * N) * r) * sizeof(float);
}
int64_t dualred_workgroups(int64_t M, int64_t N) {
  return ((N + kDrCols - 1) / kDrCols) * ((M + kDrRows - 1) / kDrRows);
}
fs4_status launch_dualred(const uint16_t *A, const uint16_t *U, uint16_t *Ut, const float *Bm, int64_t M,
                          int64_t N, int r, float p_scale, float *P, float q_scale, float *Q,
                          float *partials, uint16_t *bt, uint32_t *amax_parts, uint16_t *p_split,
                          hipStream_t s) {
  if (M == 0 || N == 0 || r == 0) return FS4_OK;
  if (r > 32) return FS4_ERR_RANK;
  if (M * N >= ((int64_t)1 << 30) || M * r >= ((int64_t)1 << 30)) return FS4_ERR_SHAPE;   // 32-bit buffer offsets
  uint16_t *bt_hi = bt, *bt_lo = bt + M * r;
  const int64_t nprep = (N + M) * r;
  rank_prep_kernel<<<(unsigned)((nprep + 255) / 256), 256, 0, s>>>(U, N, r, Ut, Bm, M, bt_hi, bt_lo);
  const int64_t cb = (N + kDrCols - 1) / kDrCols, rb = (M + kDrRows - 1) / kDrRows;
  float *ppart = partials, *qpart = partials + cb * M * r;
  dualred_kernel<<<dim3((unsigned)cb, (unsigned)rb), kDrThreads, 0, s>>>(A, Ut, bt_hi, bt_lo, M, N, r,
                                                                       ppart, qpart, amax_parts);
  // (the dual pass has read bt; p_split may be the same buffer)
  const int64_t nred = (M + N) * r;
  dual_reduce_kernel<<<(unsigned)((nred + 255) / 256), 256, 0, s>>>(
      ppart, (int)cb, M, p_scale, P, p_split, p_split ? p_split + M * r : nullptr, qpart, (int)rb, N, q_scale, Q, r);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}
fs4_status launch_transpose_rank(const uint16_t *U, int64_t N, int r, uint16_t *Ut, hipStream_t s) {
  const int64_t n = N * r;
  if (n == 0) return FS4_OK;
  transpose_rank_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(U, N, r, Ut);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
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
constexpr int kNormBlocks = 2048;   // transpose_scale_kernel workgroups (and amax partials)

// Eight consecutive elements (one 16-byte word of bf16, two of fp32) as double.
template <bool BF16>
__device__ inline void load8d(const void *x, int64_t v, double *o) {
  if constexpr (BF16) {
    const uint4 w = ((const uint4 *)x)[v];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = (double)bf16_bits_to_float(u[q] & 0xFFFFu);
      o[2 * q + 1] = (double)bf16_bits_to_float(u[q] >> 16);
    }
  } else {
    const float4 a = ((const float4 *)x)[2 * v], b = ((const float4 *)x)[2 * v + 1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
}

// Partial sums of squares in fp64 over 8-element words (n % 8 == 0).
template <bool BF16>
__global__ __launch_bounds__(256) void sumsq_kernel(const void *__restrict__ x, int64_t nv,
                                                    double *__restrict__ parts) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nv; v += (int64_t)gridDim.x * 256) {
    double o[8];
    load8d<BF16>(x, v, o);
#pragma unroll
    for (int q = 0; q < 8; ++q) s += o[q] * o[q];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) parts[blockIdx.x] = red[0];
}

// out[c][r] = sc * x[r][c] as fp32 (x bf16 or fp32, rows and cols multiples
// of 16), 64 x 64 tiles through LDS.  NORM: sc = 1 / (||x||_F + eps), every
// workgroup reducing the fp64 partial sums in the same fixed order; each
// element is x * sc in fp64, rounded once to fp32.  Otherwise sc = 1.  With
// amax_parts, each workgroup writes the max |out| of what it wrote.
template <bool BF16, bool NORM>
__global__ __launch_bounds__(256) void transpose_scale_kernel(const void *__restrict__ x, int64_t rows,
                                                              int64_t cols, const double *__restrict__ parts,
                                                              int nparts, double eps, float *__restrict__ out,
                                                              uint32_t *__restrict__ amax_parts) {
  __shared__ float tile[64][65];
  double inv = 1.0;
  if constexpr (NORM) {
    __shared__ double red[256];
    double sum = 0.0;
    for (int p = threadIdx.x; p < nparts; p += 256) sum += parts[p];
    red[threadIdx.x] = sum;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    inv = 1.0 / (__builtin_sqrt(red[0]) + eps);
  }
  const int t = threadIdx.x;
  const int64_t tcols = (cols + 63) / 64, ntiles = ((rows + 63) / 64) * tcols;
  float am = 0.0f;
  for (int64_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const int64_t r0 = tile_id / tcols * 64, c0 = tile_id % tcols * 64;
    // 8-element words: row t/8 (+32), columns 8 (t%8) .. +7
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int rr = t / 8 + 32 * p, cc = 8 * (t % 8);
      const int64_t r = r0 + rr, c = c0 + cc;
      double o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < rows && c < cols) load8d<BF16>(x, (r * cols + c) / 8, o);
#pragma unroll
      for (int q = 0; q < 8; ++q) tile[rr][cc + q] = NORM ? (float)(o[q] * inv) : (float)o[q];
    }
    __syncthreads();
    // output row c0 + t/16 (+16, +32, +48), its columns r0 + 4 (t%16) .. +3
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int oc = t / 16 + 16 * p, q4 = 4 * (t % 16);
      const int64_t c = c0 + oc, r = r0 + q4;
      if (c < cols && r < rows) {
        const float4 v = make_float4(tile[q4][oc], tile[q4 + 1][oc], tile[q4 + 2][oc], tile[q4 + 3][oc]);
        *(float4 *)(out + c * rows + r) = v;
        am = fmaxf(am, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      }
    }
    __syncthreads();          // the tile is rewritten by the next iteration
  }
  if (amax_parts) {
    __shared__ uint32_t bm[256];
    bm[t] = __builtin_bit_cast(uint32_t, am);
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (t < w) bm[t] = bm[t] > bm[t + w] ? bm[t] : bm[t + w];
      __syncthreads();
    }
    if (t == 0) amax_parts[blockIdx.x] = bm[0];
  }
}

}  // namespace

size_t normalize_ws_bytes() { return kNormParts * sizeof(double); }

namespace {
unsigned transpose_grid(int64_t rows, int64_t cols) {
  const int64_t tiles = ((rows + 63) / 64) * ((cols + 63) / 64);
  return (unsigned)(tiles < kNormBlocks ? tiles : kNormBlocks);
}
}  // namespace

fs4_status launch_normalize_t(const void *G, fs4_dtype dt, int64_t rows, int64_t cols, float eps,
                              float *XT, void *ws, hipStream_t s, uint32_t *amax_parts, int *nparts) {
  double *parts = (double *)ws;
  const int64_t nv = rows * cols / 8;
  int64_t g = (nv + 256 * 4 - 1) / (256 * 4);
  const int np = (int)(g < 1 ? 1 : (g > kNormParts ? kNormParts : g));
  const unsigned gs = transpose_grid(rows, cols);
  if (nparts) *nparts = amax_parts ? (int)gs : 0;
  if (rows == 0 || cols == 0) return FS4_OK;
  if (dt == FS4_BF16) {
    sumsq_kernel<true><<<np, 256, 0, s>>>(G, nv, parts);
    transpose_scale_kernel<true, true><<<gs, 256, 0, s>>>(G, rows, cols, parts, np, (double)eps, XT, amax_parts);
  } else {
    sumsq_kernel<false><<<np, 256, 0, s>>>(G, nv, parts);
    transpose_scale_kernel<false, true><<<gs, 256, 0, s>>>(G, rows, cols, parts, np, (double)eps, XT, amax_parts);
  }
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

fs4_status launch_transpose_f32(const void *src, fs4_dtype dt, int64_t rows, int64_t cols, float *dst,
                                hipStream_t s, uint32_t *amax_parts, int *nparts) {
  const unsigned gs = transpose_grid(rows, cols);
  if (nparts) *nparts = amax_parts ? (int)gs : 0;
  if (rows == 0 || cols == 0) return FS4_OK;
  if (dt == FS4_BF16)
    transpose_scale_kernel<true, false><<<gs, 256, 0, s>>>(src, rows, cols, nullptr, 0, 0.0, dst, amax_parts);
  else
    transpose_scale_kernel<false, false><<<gs, 256, 0, s>>>(src, rows, cols, nullptr, 0, 0.0, dst, amax_parts);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}


}  // namespace fs4
