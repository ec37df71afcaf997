// NVFP4 mixed-precision attention forward (Q-Attn) for gfx950.
//
// Full-Stack FP4 [FS4 §2.4] runs Q K^T on NVFP4 operands and keeps the
// softmax-sensitive P V in BF16; the quantized views of Q and K made once
// serve the forward and the backward.  Per sequence g (batch x head):
//   S = s_Q s_K Q_hat K_hat^T / sqrt(D)   (NVFP4 views, blocks along D)
//   P = softmax(S) row by row, causal or not
//   O = P V                                (P rounded to BF16, V BF16)
//   LSE = log sum_j exp(S_ij)
//
// One workgroup takes 128 queries of one sequence, 32 per wave, and walks
// the keys in blocks of 64, flash-attention style (running max and sum per
// query, the output rescaled as the max grows).  The wave computes S^T =
// K Q^T with FP16 MFMA 32x32x16: its Q block is expanded to FP16 once
// (E2M1 code x E4M3 block scale is exact in FP16: <= 6 significant bits)
// and stays in registers; each key block's codes sit in LDS and every wave
// expands the K fragments it multiplies.  In the S^T accumulator layout a
// lane holds 16 keys of one query, so the softmax reductions are in-lane
// plus one exchange with the lane 32 apart.  Those registers, rounded to
// BF16, are directly the B operand of O^T = V^T P^T (BF16 MFMA 32x32x16):
// the keys are contracted in the order the registers hold them, and the V^T
// fragments are read from LDS in that same order (V is staged transposed,
// [D][keys]).
#include "fs4_common.h"

namespace fs4 {
namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kAttnThreads = 256;   // four waves
constexpr int kBQ = 128;            // queries per workgroup, 32 per wave
constexpr int kBK = 64;             // keys per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint8_t *q_codes, *q_scales, *k_codes, *k_scales;
  const float *q_ts, *k_ts;
  const uint16_t *vt;   // bf16 [G][D][S]
  float *o;             // fp32 [G][S][D]
  float *lse;           // fp32 [G][S], nullable
  int64_t G, S;
  float scale;          // softmax scale, 1/sqrt(D)
  int causal;
};

// E4M3 block scale s_b = 2^E F: the power of two as an fp32 (the converter
// reads only its exponent) and F = 1 + m/8 as a pair of FP16.  Every E4M3
// value has at most 4 significant bits, so they are the top bits of its fp32
// significand, subnormal scales included.
struct ScalePair {
  float pow2;
  f16x2_t mant;
};
__device__ inline ScalePair split_scale(uint32_t byte) {
  const uint32_t fb = __builtin_bit_cast(uint32_t, e4m3_to_float(byte & 0x7Fu));
  ScalePair s;
  s.pow2 = __builtin_bit_cast(float, fb & 0x7F800000u);   // 0 for a zero scale
  const uint32_t h = 0x3C00u | (((fb >> 20) & 7u) << 7);
  s.mant = __builtin_bit_cast(f16x2_t, h | (h << 16));
  return s;
}

// 8 E2M1 codes (element 2j in the low nibble of byte j) times s_b, in FP16
__device__ inline f16x8_t expand8(uint32_t codes8, const ScalePair &s) {
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, s.pow2, 0) * s.mant;
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, s.pow2, 1) * s.mant;
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, s.pow2, 2) * s.mant;
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, s.pow2, 3) * s.mant;
  f16x8_t f;
  f[0] = p0[0]; f[1] = p0[1]; f[2] = p1[0]; f[3] = p1[1];
  f[4] = p2[0]; f[5] = p2[1]; f[6] = p3[0]; f[7] = p3[1];
  return f;
}

template <int D>
struct AttnLds {
  static constexpr int kKc = D / 2 + 8;           // K code row stride (bytes): 8-byte aligned, spreads banks
  static constexpr int kKs = D / 16;              // K scale row stride
  static constexpr int kVt = kBK * 2 + 8;         // V^T row stride (bytes), 64 keys of BF16 + pad
  static constexpr int kKcBytes = kBK * kKc, kKsBytes = kBK * kKs, kVtBytes = D * kVt;
  static constexpr int kStage = kKcBytes + kKsBytes + kVtBytes;
  // per-lane staging registers: K codes, K scales, V^T (16-byte words)
  static constexpr int kKcWords = kBK * (D / 2) / 16;    // 256 for D = 128
  static constexpr int kVtWords = D * kBK * 2 / 16;      // 1024 for D = 128
  static constexpr int kKcPer = (kKcWords + kAttnThreads - 1) / kAttnThreads;
  static constexpr int kVtPer = kVtWords / kAttnThreads;
  static_assert(kVtWords % kAttnThreads == 0, "V^T staging");
};

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attention_fwd_kernel(AttnArgs a) {
  using L = AttnLds<D>;
  constexpr int KSTEPS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int DT = D / 32;       // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::kStage];

  const int64_t G = a.G, S = a.S;
  const int64_t nqb = (S + kBQ - 1) / kBQ;
  // the longest query blocks (last, under a causal mask) first
  const int64_t g = blockIdx.x % G;
  const int64_t qb = a.causal ? nqb - 1 - (int64_t)blockIdx.x / G : (int64_t)blockIdx.x / G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int64_t q0 = qb * kBQ;
  const int64_t qw0 = q0 + w * 32;               // this wave's first query
  const int64_t q = qw0 + l32;                   // this lane's query (column of every tile)
  const int64_t qc = q < S ? q : S - 1;          // clamped for the loads

  // ---- this wave's Q block, expanded once (B operand of S^T = K Q^T) ------
  f16x8_t qf[KSTEPS];
  {
    const uint8_t *qrow = a.q_codes + (g * S + qc) * (D / 2);
    const uint8_t *qsc = a.q_scales + (g * S + qc) * (D / 16);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const uint32_t c8 = *(const uint32_t *)(qrow + 8 * t + 4 * h);   // d = 16t + 8h .. +8
      qf[t] = expand8(c8, split_scale(qsc[t]));
    }
  }
  const float c_log2 = (*a.q_ts) * (*a.k_ts) * a.scale * kLog2e;   // S in log2 units

  floatx16_t ot[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) ot[i][e] = 0.0f;
  float m_run = -__builtin_huge_valf(), l_run = 0.0f;

  const int64_t nkb_all = (S + kBK - 1) / kBK;
  const int64_t nkb = a.causal ? ((q0 + kBQ < S ? q0 + kBQ : S) + kBK - 1) / kBK : nkb_all;

  // ---- key-block staging: global -> registers -> LDS ------------------------
  uint4 rk[L::kKcPer], rv[L::kVtPer];
  uint2 rs = make_uint2(0, 0);
  auto load_block = [&](int64_t kb) {
    const int64_t k0 = kb * kBK;
#pragma unroll
    for (int i = 0; i < L::kKcPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      const int row = idx / (D / 32), ch = idx % (D / 32);
      int64_t key = k0 + row;
      key = key < S ? key : S - 1;
      rk[i] = idx < L::kKcWords ? *(const uint4 *)(a.k_codes + (g * S + key) * (D / 2) + ch * 16)
                                : make_uint4(0, 0, 0, 0);
    }
    if (tid < kBK) {
      int64_t key = k0 + tid;
      key = key < S ? key : S - 1;
      if constexpr (D == 128) rs = *(const uint2 *)(a.k_scales + (g * S + key) * 8);
      else rs = make_uint2(*(const uint32_t *)(a.k_scales + (g * S + key) * 4), 0u);
    }
#pragma unroll
    for (int i = 0; i < L::kVtPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      const int d = idx / (kBK / 8), ch = idx % (kBK / 8);     // 8 keys per 16-byte word
      const int64_t key = k0 + ch * 8;
      rv[i] = key < S ? *(const uint4 *)(a.vt + (g * D + d) * S + key) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_block = [&](int st) {
    uint8_t *base = lds + st * L::kStage;
    uint8_t *kc = base, *ks = base + L::kKcBytes, *vt = ks + L::kKsBytes;
#pragma unroll
    for (int i = 0; i < L::kKcPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      if (idx < L::kKcWords) {
        const int row = idx / (D / 32), ch = idx % (D / 32);
        uint2 *p = (uint2 *)(kc + row * L::kKc + ch * 16);
        p[0] = make_uint2(rk[i].x, rk[i].y);
        p[1] = make_uint2(rk[i].z, rk[i].w);
      }
    }
    if (tid < kBK) {
      if constexpr (D == 128) *(uint2 *)(ks + tid * 8) = rs;
      else *(uint32_t *)(ks + tid * 4) = rs.x;
    }
#pragma unroll
    for (int i = 0; i < L::kVtPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      const int d = idx / (kBK / 8), ch = idx % (kBK / 8);
      uint2 *p = (uint2 *)(vt + d * L::kVt + ch * 16);
      p[0] = make_uint2(rv[i].x, rv[i].y);
      p[1] = make_uint2(rv[i].z, rv[i].w);
    }
  };

  load_block(0);
  store_block(0);
  __syncthreads();

  for (int64_t kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) load_block(kb + 1);
    const int64_t k0 = kb * kBK;
    // the wave's queries see some key of this block (wave-uniform)
    const bool live = !a.causal || k0 <= qw0 + 31;
    if (live) {
      const uint8_t *base = lds + (int)(kb & 1) * L::kStage;
      const uint8_t *kc = base, *ks = base + L::kKcBytes, *vt = ks + L::kKsBytes;
      // ---- S^T = K Q^T: two 32-key tiles ------------------------------------
      floatx16_t st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) st[kt][e] = 0.0f;
        const int krow = kt * 32 + l32;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          const uint32_t c8 = *(const uint32_t *)(kc + krow * L::kKc + 8 * t + 4 * h);
          const f16x8_t kf = expand8(c8, split_scale(ks[krow * L::kKs + t]));
          st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[t], st[kt], 0, 0, 0);
        }
      }
      // ---- online softmax in log2 units ------------------------------------
      // register e of tile kt holds key k0 + 32 kt + 8 (e/4) + 4 h + e%4
      const bool mask = (a.causal && k0 + kBK - 1 > qw0) || k0 + kBK > S;
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = st[kt][e] * c_log2;
          if (mask) {
            const int64_t key = k0 + 32 * kt + 8 * (e >> 2) + 4 * h + (e & 3);
            if (key >= S || (a.causal && key > q)) x = -__builtin_huge_valf();
          }
          st[kt][e] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      // m_new is finite from the first block on: key 0 is visible to every query
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float rsum = 0.0f;
      bf16x8_t pb[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(st[kt][e] - m_new);
          rsum += p;
          pb[kt][e >> 3][e & 7] = (__bf16)p;
        }
      rsum += __shfl_xor(rsum, 32);
      l_run = l_run * alpha + rsum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < DT; ++i) ot[i] *= alpha;
      // ---- O^T += V^T P^T, keys in the registers' order --------------------
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint8_t *vrow = vt + (dt * 32 + l32) * L::kVt;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kt = u >> 1, s = u & 1;
          const int kk = 32 * kt + 16 * s + 4 * h;        // keys kk..kk+3 and kk+8..kk+11
          const uint2 v0 = *(const uint2 *)(vrow + kk * 2);
          const uint2 v1 = *(const uint2 *)(vrow + (kk + 8) * 2);
          const uint32_t vw[4] = {v0.x, v0.y, v1.x, v1.y};
          bf16x8_t vf;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vf[2 * i] = __builtin_bit_cast(__bf16, (uint16_t)(vw[i] & 0xFFFFu));
            vf[2 * i + 1] = __builtin_bit_cast(__bf16, (uint16_t)(vw[i] >> 16));
          }
          ot[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kt][s], ot[dt], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkb) store_block((int)((kb + 1) & 1));
    __syncthreads();
  }

  // ---- O = O^T / l, LSE ---------------------------------------------------------
  if (q < S) {
    const float inv = 1.0f / l_run;
    float *orow = a.o + (g * S + q) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = dt * 32 + 8 * c + 4 * h;
        *(float4 *)(orow + d0) = make_float4(ot[dt][4 * c] * inv, ot[dt][4 * c + 1] * inv, ot[dt][4 * c + 2] * inv,
                                             ot[dt][4 * c + 3] * inv);
      }
    if (a.lse && h == 0) a.lse[g * S + q] = (m_run + __builtin_log2f(l_run)) * kLn2;
  }
}

// V [G][S][D] -> V^T [G][D][S] (BF16), 64 x 64 tiles through LDS
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ v, int64_t S, int64_t D,
                                                             uint16_t *__restrict__ vt) {
  __shared__ uint16_t tile[64][66];
  const int64_t g = blockIdx.z;
  const int64_t s0 = (int64_t)blockIdx.x * 64, d0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int64_t s = s0 + r, d = d0 + tx;
    tile[r][tx] = (s < S && d < D) ? v[(g * S + s) * D + d] : (uint16_t)0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t d = d0 + r, s = s0 + tx;
    if (d < D && s < S) vt[(g * D + d) * S + s] = tile[tx][r];
  }
}

}  // namespace

size_t attention_fwd_ws_bytes(int64_t G, int64_t S, int64_t D) {
  return round_up((size_t)(G * S * D) * 2, 256);
}

fs4_status launch_attention_fwd(const fs4_nvfp4 &Q, const fs4_nvfp4 &K, const uint16_t *V, int64_t G, int64_t S,
                                int64_t D, int causal, float *O, float *LSE, uint16_t *Vt, hipStream_t s) {
  const dim3 tg((unsigned)((S + 63) / 64), (unsigned)((D + 63) / 64), (unsigned)G);
  transpose_bf16_kernel<<<tg, 256, 0, s>>>(V, S, D, Vt);
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;
  AttnArgs a;
  a.q_codes = Q.codes; a.q_scales = Q.scales; a.k_codes = K.codes; a.k_scales = K.scales;
  a.q_ts = Q.tscale; a.k_ts = K.tscale;
  a.vt = Vt; a.o = O; a.lse = LSE;
  a.G = G; a.S = S;
  a.scale = (float)(1.0 / __builtin_sqrt((double)D));
  a.causal = causal;
  const int64_t nqb = (S + kBQ - 1) / kBQ;
  const unsigned grid = (unsigned)(G * nqb);
  if (D == 128) attention_fwd_kernel<128><<<grid, kAttnThreads, 0, s>>>(a);
  else attention_fwd_kernel<64><<<grid, kAttnThreads, 0, s>>>(a);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
