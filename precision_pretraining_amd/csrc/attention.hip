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
// and stays in registers; each key block is expanded to FP16 once per
// workgroup as it is staged in LDS, and the waves read its fragments.  In the S^T accumulator layout a
// lane holds 16 keys of one query, so the softmax reductions are in-lane
// plus one exchange with the lane 32 apart.  Those registers, rounded to
// BF16, are directly the B operand of O^T = V^T P^T (BF16 MFMA 32x32x16):
// the keys are contracted in the order the registers hold them, and the V^T
// fragments are read from LDS in that same order (V is staged transposed,
// [D][keys]).
#include "nvfp4_encode.h"

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
  const uint16_t *v;    // bf16 [G][S][D]
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
  static constexpr int kKh = D + 8;               // FP16 per row of the expanded K block
  static constexpr int kVt = kBK * 2 + 8;         // V^T row stride (bytes), 64 keys of BF16 + pad
  static constexpr int kKhBytes = kBK * kKh * 2, kVtBytes = D * kVt;
  static constexpr int kStage = kKhBytes + kVtBytes;
  // staging: each thread expands kEpt K elements (a quarter row) and
  // transposes kVPairs pairs of V words (8 dims of two consecutive keys)
  static constexpr int kEpt = kBK * D / kAttnThreads;    // 32 for D = 128, 16 for D = 64
  static constexpr int kVPairs = (kBK / 2) * (D / 8) / kAttnThreads;   // 2 for D = 128, 1 for D = 64
  static_assert((kBK / 2) * (D / 8) % kAttnThreads == 0, "V staging");
  static_assert(D / kEpt == 4 && kEpt % 16 == 0, "K staging: four threads per key, whole scale blocks");
};

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attention_fwd_kernel(AttnArgs a) {
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
  // K is expanded to FP16 once per workgroup as it is stored, and every wave
  // reads its fragments from LDS
  uint4 rk = make_uint4(0, 0, 0, 0), rv[2 * L::kVPairs];
  uint32_t rks = 0;
  const int krow_s = tid / 4, kc0 = (tid % 4) * L::kEpt;   // the K elements this thread expands
  auto load_block = [&](int64_t kb) {
    const int64_t k0 = kb * kBK;
    {
      int64_t key = k0 + krow_s;
      key = key < S ? key : S - 1;
      const uint8_t *cp = a.k_codes + (g * S + key) * (D / 2) + kc0 / 2;
      const uint8_t *sp = a.k_scales + (g * S + key) * (D / 16) + kc0 / 16;
      if constexpr (L::kEpt == 32) {
        rk = *(const uint4 *)cp;
        rks = *(const uint16_t *)sp;
      } else {
        const uint2 t = *(const uint2 *)cp;
        rk = make_uint4(t.x, t.y, 0u, 0u);
        rks = *sp;
      }
    }
    // V as it sits in memory: word (key, dims 8 dg .. 8 dg + 7); a thread
    // takes keys 2 kp and 2 kp + 1 of one dim group, so that it can write
    // both keys of a dim as one 32-bit word of the transposed LDS rows
#pragma unroll
    for (int j = 0; j < L::kVPairs; ++j) {
      const int idx = tid + j * kAttnThreads;
      const int kp = idx % (kBK / 2), dg = idx / (kBK / 2);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        // (keys past S load the last key and are zeroed where they are
        // stored, not behind the load)
        int64_t key = k0 + 2 * kp + b;
        key = key < S ? key : S - 1;
        rv[2 * j + b] = *(const uint4 *)(a.v + (g * S + key) * D + dg * 8);
      }
    }
  };
  auto store_block = [&](int st, int64_t k0) {
    uint8_t *base = lds + st * L::kStage;
    _Float16 *kh = (_Float16 *)base + krow_s * L::kKh + kc0;
    uint8_t *vt = base + L::kKhBytes;
    const uint32_t cw[4] = {rk.x, rk.y, rk.z, rk.w};
#pragma unroll
    for (int j = 0; j < L::kEpt / 8; ++j)
      *(f16x8_t *)(kh + 8 * j) = expand8(cw[j], split_scale((rks >> (8 * (j / 2))) & 0xFFu));
    // V^T rows [d][keys]: dims 2q, 2q + 1 of each word pair become two 32-bit
    // words (key 2 kp in the low half, 2 kp + 1 in the high half)
#pragma unroll
    for (int j = 0; j < L::kVPairs; ++j) {
      const int idx = tid + j * kAttnThreads;
      const int kp = idx % (kBK / 2), dg = idx / (kBK / 2);
      const uint32_t m0 = k0 + 2 * kp < S ? 0xFFFFFFFFu : 0u, m1 = k0 + 2 * kp + 1 < S ? 0xFFFFFFFFu : 0u;
      const uint32_t w0[4] = {rv[2 * j].x & m0, rv[2 * j].y & m0, rv[2 * j].z & m0, rv[2 * j].w & m0};
      const uint32_t w1[4] = {rv[2 * j + 1].x & m1, rv[2 * j + 1].y & m1, rv[2 * j + 1].z & m1, rv[2 * j + 1].w & m1};
      uint8_t *col = vt + (dg * 8) * L::kVt + 4 * kp;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        *(uint32_t *)(col + (2 * qd) * L::kVt) = __builtin_amdgcn_perm(w1[qd], w0[qd], 0x05040100u);
        *(uint32_t *)(col + (2 * qd + 1) * L::kVt) = __builtin_amdgcn_perm(w1[qd], w0[qd], 0x07060302u);
      }
    }
  };

  load_block(0);
  store_block(0, 0);
  __syncthreads();

  for (int64_t kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) load_block(kb + 1);
    const int64_t k0 = kb * kBK;
    // the wave's queries see some key of this block (wave-uniform)
    const bool live = !a.causal || k0 <= qw0 + 31;
    if (live) {
      const uint8_t *base = lds + (int)(kb & 1) * L::kStage;
      const _Float16 *kh = (const _Float16 *)base;
      const uint8_t *vt = base + L::kKhBytes;
      // ---- S^T = K Q^T: two 32-key tiles ------------------------------------
      floatx16_t st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) st[kt][e] = 0.0f;
        const int krow = kt * 32 + l32;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
          st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8_t *)(kh + krow * L::kKh + 16 * t + 8 * h),
                                                           qf[t], st[kt], 0, 0, 0);
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
    if (kb + 1 < nkb) store_block((int)((kb + 1) & 1), (kb + 1) * kBK);
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

// ---------------------------------------------------------------------------
// Backward.  Per sequence, from the forward's quantized Q and K, its O and
// LSE, and dO:
//   P = exp(S - LSE)                  (S recomputed from the same NVFP4 views)
//   dP = dO V^T, Delta = rowsum(dO * O), dS = P * (dP - Delta)
//   dV = P^T dO                        (P rounded to BF16, dO BF16)
//   dQ = Q(dS) Q_col(K)^T / sqrt(D),  dK = Q(dS^T) Q_col(Q)^T / sqrt(D)
// dS is quantized once, with one tensor scale over all sequences, so the
// keys are walked twice: the softmax-gradient kernel forms dS and dV and
// keeps one partial amax of |dS| per workgroup; a second kernel forms dS
// again, identically, and encodes it into both NVFP4 views with the tensor
// scale those partials give; a batched NVFP4 product kernel forms dQ and dK.
// dS never goes through memory in fp32 (unless the caller asks for it).
//
// The softmax-gradient kernel gives each workgroup 128 keys of one sequence,
// 32 per wave, and walks the queries in blocks of 64.  A wave keeps its keys'
// K (expanded to FP16) and V (BF16) in registers as the B operands of
// S = Q K^T and dP = dO V^T, so both accumulators hold one key per lane and
// 16 queries per lane in registers; P and dS are formed in place.  Those P
// registers, rounded to BF16, are the B operand of dV^T = dO^T P, the
// queries contracted in the order the registers hold them (dO^T is staged
// transposed so the A fragments follow that order).  Each query block's Q
// is expanded to FP16 once per workgroup, into LDS.

constexpr int kBwdKeys = 128;   // keys per workgroup, 32 per wave
constexpr int kBwdQ = 64;       // queries per step: two 32-query tiles

struct AttnBwdArgs {
  const uint8_t *q_codes, *q_scales, *k_codes, *k_scales;
  const float *q_ts, *k_ts;
  const uint16_t *dout;   // bf16 [G][S][D]
  const float *lse;       // [G][S], natural log
  float *dv;              // fp32 [G][S][D]
  int64_t G, S;
  float scale;
  int causal;
};

template <int D>
struct BwdLds {
  static constexpr int kQh = D + 8;       // FP16 per row of the expanded Q block
  static constexpr int kDt = kBwdQ + 8;   // BF16 per row of dO^T
  static constexpr int kQhOff = 0;
  static constexpr int kDtOff = kQhOff + kBwdQ * kQh * 2;
  static constexpr int kLseOff = kDtOff + D * kDt * 2;
  static constexpr int kStage = kLseOff + kBwdQ * 4;
  static constexpr int kEpt = kBwdQ * D / kAttnThreads;                // Q elements a thread expands
  // dO words (8 dims of a query) in pairs of consecutive queries: each pair
  // is stored, transposed, as 32-bit words of dO^T
  static constexpr int kDoPairs = (kBwdQ / 2) * (D / 8) / kAttnThreads;   // 2 for D = 128, 1 for D = 64
  static_assert((kBwdQ / 2) * (D / 8) % kAttnThreads == 0, "dO staging");
  static_assert(D / kEpt == 4 && kEpt % 16 == 0, "Q staging: four threads per row, whole scale blocks");
  static_assert(kStage % 16 == 0, "stage alignment");
};

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attention_bwd_kernel(AttnBwdArgs a) {
  using L = BwdLds<D>;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::kStage];

  const int64_t G = a.G, S = a.S;
  const int64_t g = blockIdx.x % G;
  const int64_t kb = (int64_t)blockIdx.x / G;   // under a causal mask the first keys see the most queries
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int64_t k0 = kb * kBwdKeys;
  const int64_t kend = k0 + kBwdKeys < S ? k0 + kBwdKeys : S;
  const int64_t kw0 = k0 + w * 32;
  const int64_t key = kw0 + l32;
  const bool key_ok = key < S;
  const int64_t keyc = key_ok ? key : S - 1;

  // ---- this wave's keys: K expanded to FP16, the B operand of S ------------
  f16x8_t kf[KSTEPS];
  {
    const uint8_t *krow = a.k_codes + (g * S + keyc) * (D / 2);
    const uint8_t *ksc = a.k_scales + (g * S + keyc) * (D / 16);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
      kf[t] = expand8(*(const uint32_t *)(krow + 8 * t + 4 * h), split_scale(ksc[t]));   // d = 16t + 8h .. +8
  }

  // ---- query-block staging: global -> registers -> LDS ---------------------
  uint4 rq = make_uint4(0, 0, 0, 0);
  uint32_t rqs = 0;
  uint4 rdo[2 * L::kDoPairs];
  float rls = 0.0f;
  const int qrow = tid / 4, qc0 = (tid % 4) * L::kEpt;   // the Q elements this thread expands
  auto load_block = [&](int64_t q0) {
    {
      int64_t qq = q0 + qrow;
      qq = qq < S ? qq : S - 1;
      const uint8_t *cp = a.q_codes + (g * S + qq) * (D / 2) + qc0 / 2;
      const uint8_t *sp = a.q_scales + (g * S + qq) * (D / 16) + qc0 / 16;
      if constexpr (L::kEpt == 32) {
        rq = *(const uint4 *)cp;
        rqs = *(const uint16_t *)sp;
      } else {
        const uint2 t = *(const uint2 *)cp;
        rq = make_uint4(t.x, t.y, 0u, 0u);
        rqs = *sp;
      }
    }
    // (queries past S load the last query and are zeroed where they are
    // stored, not behind the load)
#pragma unroll
    for (int j = 0; j < L::kDoPairs; ++j) {
      const int idx = tid + j * kAttnThreads;
      const int qp = idx % (kBwdQ / 2), dg = idx / (kBwdQ / 2);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        int64_t qq = q0 + 2 * qp + b;
        qq = qq < S ? qq : S - 1;
        rdo[2 * j + b] = *(const uint4 *)(a.dout + (g * S + qq) * D + dg * 8);
      }
    }
    if (tid < kBwdQ) {
      const int64_t qq = q0 + tid;
      rls = qq < S ? a.lse[g * S + qq] * kLog2e : 0.0f;
    }
  };
  auto store_block = [&](int st, int64_t q0) {
    uint8_t *base = lds + st * L::kStage;
    _Float16 *qh = (_Float16 *)(base + L::kQhOff) + qrow * L::kQh + qc0;
    const uint32_t cw[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
    for (int j = 0; j < L::kEpt / 8; ++j)
      *(f16x8_t *)(qh + 8 * j) = expand8(cw[j], split_scale((rqs >> (8 * (j / 2))) & 0xFFu));
#pragma unroll
    for (int j = 0; j < L::kDoPairs; ++j) {
      const int idx = tid + j * kAttnThreads;
      const int qp = idx % (kBwdQ / 2), dg = idx / (kBwdQ / 2);
      const uint32_t m0 = q0 + 2 * qp < S ? 0xFFFFFFFFu : 0u, m1 = q0 + 2 * qp + 1 < S ? 0xFFFFFFFFu : 0u;
      const uint4 w0 = make_uint4(rdo[2 * j].x & m0, rdo[2 * j].y & m0, rdo[2 * j].z & m0, rdo[2 * j].w & m0);
      const uint4 w1 = make_uint4(rdo[2 * j + 1].x & m1, rdo[2 * j + 1].y & m1, rdo[2 * j + 1].z & m1,
                                  rdo[2 * j + 1].w & m1);
      // dO^T rows [d][queries]: dims 2c, 2c + 1 of the pair become two 32-bit
      // words (query 2 qp in the low half, 2 qp + 1 in the high half)
      const uint32_t a0[4] = {w0.x, w0.y, w0.z, w0.w}, a1[4] = {w1.x, w1.y, w1.z, w1.w};
      uint8_t *col = base + L::kDtOff + (dg * 8) * L::kDt * 2 + 4 * qp;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        *(uint32_t *)(col + (2 * c) * L::kDt * 2) = __builtin_amdgcn_perm(a1[c], a0[c], 0x05040100u);
        *(uint32_t *)(col + (2 * c + 1) * L::kDt * 2) = __builtin_amdgcn_perm(a1[c], a0[c], 0x07060302u);
      }
    }
    if (tid < kBwdQ) ((float *)(base + L::kLseOff))[tid] = rls;   // LSE in log2 units
  };

  const float c_log2 = (*a.q_ts) * (*a.k_ts) * a.scale * kLog2e;   // S in log2 units
  floatx16_t dvt[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dvt[i][e] = 0.0f;

  const int64_t nqb = (S + kBwdQ - 1) / kBwdQ;
  const int64_t qb0 = a.causal ? k0 / kBwdQ : 0;
  load_block(qb0 * kBwdQ);
  store_block(0, qb0 * kBwdQ);
  __syncthreads();

  for (int64_t qb = qb0; qb < nqb; ++qb) {
    if (qb + 1 < nqb) load_block((qb + 1) * kBwdQ);
    const int st = (int)((qb - qb0) & 1);
    const uint8_t *base = lds + st * L::kStage;
    const _Float16 *qh = (const _Float16 *)(base + L::kQhOff);
    const uint8_t *dtr = base + L::kDtOff;
    const float *lse2 = (const float *)(base + L::kLseOff);
    const int64_t q0 = qb * kBwdQ;
    bf16x8_t pb[2][2];
    bool live[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int64_t qt0 = q0 + 32 * qt;
      // some query of this tile sees some key of this wave (wave-uniform)
      live[qt] = qt0 < S && (!a.causal || qt0 + 31 >= kw0);
      floatx16_t sacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
      if (live[qt]) {
        const int r = 32 * qt + l32;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8_t *)(qh + r * L::kQh + 16 * t + 8 * h), kf[t],
                                                         sacc, 0, 0, 0);
      }
      // register e holds query q0 + 32 qt + 8 (e/4) + 4 h + e%4 of key `key`;
      // a tile wholly in range and below a causal diagonal needs no masks
      auto form_p = [&](auto masked) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int qi = 32 * qt + 8 * c + 4 * h;
          const float4 l4 = *(const float4 *)(lse2 + qi);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * c + r;
            float p = __builtin_amdgcn_exp2f(sacc[e] * c_log2 - lv[r]);
            if constexpr (decltype(masked)::value) {
              const int64_t query = q0 + qi + r;
              const bool valid = key_ok && query < S && (!a.causal || key <= query);
              p = valid ? p : 0.0f;
            }
            pb[qt][e >> 3][e & 7] = (__bf16)p;
          }
        }
      };
      if (qt0 + 31 < S && kw0 + 31 < S && (!a.causal || kw0 + 31 <= qt0)) form_p(std::false_type{});
      else form_p(std::true_type{});
    }
    // ---- dV^T += dO^T P, queries in the registers' order ---------------------
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint8_t *drow = dtr + (dt * 32 + l32) * L::kDt * 2;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qt = u >> 1, s = u & 1;
        if (!live[qt]) continue;
        const int kk = 32 * qt + 16 * s + 4 * h;   // queries kk..kk+3 and kk+8..kk+11
        const uint2 v0 = *(const uint2 *)(drow + kk * 2);
        const uint2 v1 = *(const uint2 *)(drow + (kk + 8) * 2);
        const uint32_t vw[4] = {v0.x, v0.y, v1.x, v1.y};
        bf16x8_t af;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          af[2 * i] = __builtin_bit_cast(__bf16, (uint16_t)(vw[i] & 0xFFFFu));
          af[2 * i + 1] = __builtin_bit_cast(__bf16, (uint16_t)(vw[i] >> 16));
        }
        dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[qt][s], dvt[dt], 0, 0, 0);
      }
    }
    if (qb + 1 < nqb) store_block(st ^ 1, (qb + 1) * kBwdQ);
    __syncthreads();
  }

  // ---- dV -------------------------------------------------------------------
  if (key_ok) {
    float *vrow = a.dv + (g * S + key) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *(float4 *)(vrow + dt * 32 + 8 * c + 4 * h) =
            make_float4(dvt[dt][4 * c], dvt[dt][4 * c + 1], dvt[dt][4 * c + 2], dvt[dt][4 * c + 3]);
  }
}

// ---- the amax of dS ------------------------------------------------------------
// dS's tensor scale needs max |dS| over all of it before any block is encoded.
// This pass forms S, P, dP and dS query-major, as the forward walks the keys:
// a workgroup takes 128 queries (32 per wave) and walks 64-key blocks, with
// each block's K expanded to FP16 and its V rows staged in LDS, and keeps only
// the maximum (and dS itself when the caller asks for it).  Every product
// takes the same operands in the same roles and order as the key-major
// passes (A = Q or dO, B = K or V, k-steps over D in order), so its dS values
// are bit for bit the ones the second pass encodes.
struct AttnAmaxArgs {
  const uint8_t *q_codes, *q_scales, *k_codes, *k_scales;
  const float *q_ts, *k_ts;
  const uint16_t *v;      // bf16 [G][S][D]
  const uint16_t *dout;   // bf16 [G][S][D]
  const float *lse;       // [G][S], natural log
  const float *delta;     // [G][S]
  float *ds;              // fp32 [G*S][S], nullable: dS for the caller
  uint32_t *amax;         // one max |dS| per workgroup (fp32 bits)
  int64_t G, S;
  float scale;
  int causal;
};

constexpr int kAmK = 32;   // keys per block of the amax pass (one MFMA tile)

template <int D>
struct AmaxLds {
  static constexpr int kKh = D + 8;   // FP16 per row of the expanded K block
  static constexpr int kVr = D + 8;   // BF16 per row of the V block
  static constexpr int kKhBytes = kAmK * kKh * 2, kVBytes = kAmK * kVr * 2;
  static constexpr int kStage = kKhBytes + kVBytes;
  static constexpr int kEpt = kAmK * D / kAttnThreads;           // K elements a thread expands (16 or 8)
  static constexpr int kTpr = D / kEpt;                          // threads per K row (8)
  static constexpr int kVPer = kAmK * D * 2 / 16 / kAttnThreads;  // 16-byte words of V per thread
  static_assert(kEpt % 8 == 0 && kVPer >= 1, "staging");
};

// KEEP: write dS too (the caller asked for it; every key block is walked so
// that its zeros above a causal diagonal are written as well)
template <int D, bool KEEP>
__global__ __launch_bounds__(kAttnThreads, 2) void attention_amax_kernel(AttnAmaxArgs a) {
  using L = AmaxLds<D>;
  constexpr int KSTEPS = D / 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::kStage];
  __shared__ __attribute__((aligned(16))) float qv[2][kBQ];   // LSE (log2 units) and Delta of the queries
  __shared__ uint32_t red[kAttnThreads / 64];

  const int64_t G = a.G, S = a.S;
  const int64_t nqb = (S + kBQ - 1) / kBQ;
  const int64_t g = blockIdx.x % G;
  const int64_t qb = a.causal ? nqb - 1 - (int64_t)blockIdx.x / G : (int64_t)blockIdx.x / G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int64_t q0 = qb * kBQ;
  const int64_t qw0 = q0 + w * 32;
  const int64_t qc = qw0 + l32 < S ? qw0 + l32 : S - 1;   // this lane's A-operand row, clamped

  // ---- the wave's Q (FP16) and dO fragments, A operands -------------------
  f16x8_t qf[KSTEPS];
  bf16x8_t df[KSTEPS];
  {
    const uint8_t *qrow = a.q_codes + (g * S + qc) * (D / 2);
    const uint8_t *qsc = a.q_scales + (g * S + qc) * (D / 16);
    const uint16_t *drow = a.dout + (g * S + qc) * D;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      qf[t] = expand8(*(const uint32_t *)(qrow + 8 * t + 4 * h), split_scale(qsc[t]));   // d = 16t + 8h .. +8
      df[t] = *(const bf16x8_t *)(drow + 16 * t + 8 * h);
    }
  }
  if (tid < kBQ) {
    const int64_t qq = q0 + tid;
    qv[0][tid] = qq < S ? a.lse[g * S + qq] * kLog2e : 0.0f;
    qv[1][tid] = qq < S ? a.delta[g * S + qq] : 0.0f;
  }
  const float c_log2 = (*a.q_ts) * (*a.k_ts) * a.scale * kLog2e;   // S in log2 units

  // ---- key-block staging: K expanded to FP16, V rows as they are -----------
  uint4 rk = make_uint4(0, 0, 0, 0), rv[L::kVPer];
  uint32_t rks = 0;
  const int krow_s = tid / L::kTpr, kc0 = (tid % L::kTpr) * L::kEpt;
  auto load_block = [&](int64_t kb) {
    const int64_t k0 = kb * kAmK;
    {
      int64_t key = k0 + krow_s;
      key = key < S ? key : S - 1;
      const uint8_t *cp = a.k_codes + (g * S + key) * (D / 2) + kc0 / 2;
      const uint8_t *sp = a.k_scales + (g * S + key) * (D / 16) + kc0 / 16;
      if constexpr (L::kEpt == 16) {
        const uint2 t = *(const uint2 *)cp;
        rk = make_uint4(t.x, t.y, 0u, 0u);
        rks = *sp;
      } else {
        rk = make_uint4(*(const uint32_t *)cp, 0u, 0u, 0u);   // half of a scale block
        rks = *sp;
      }
    }
#pragma unroll
    for (int i = 0; i < L::kVPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      int64_t key = k0 + row;
      key = key < S ? key : S - 1;   // rows past S are never visible
      rv[i] = *(const uint4 *)(a.v + (g * S + key) * D + ch * 8);
    }
  };
  auto store_block = [&](int st) {
    uint8_t *base = lds + st * L::kStage;
    _Float16 *kh = (_Float16 *)base + krow_s * L::kKh + kc0;
    const uint32_t cw[4] = {rk.x, rk.y, rk.z, rk.w};
#pragma unroll
    for (int j = 0; j < L::kEpt / 8; ++j)
      *(f16x8_t *)(kh + 8 * j) = expand8(cw[j], split_scale(rks & 0xFFu));   // one scale block
#pragma unroll
    for (int i = 0; i < L::kVPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      *(uint4 *)(base + L::kKhBytes + (row * L::kVr + ch * 8) * 2) = rv[i];
    }
  };

  const int64_t nkb_all = (S + kAmK - 1) / kAmK;
  const int64_t nkb = (a.causal && !KEEP) ? ((q0 + kBQ < S ? q0 + kBQ : S) + kAmK - 1) / kAmK : nkb_all;
  float amax = 0.0f;
  load_block(0);
  store_block(0);
  __syncthreads();
  for (int64_t kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) load_block(kb + 1);
    const int64_t k0 = kb * kAmK;
    const bool live = !a.causal || k0 <= qw0 + 31 || KEEP;   // wave-uniform
    if (live) {
      const uint8_t *base = lds + (int)(kb & 1) * L::kStage;
      const _Float16 *kh = (const _Float16 *)base;
      const uint16_t *vr = (const uint16_t *)(base + L::kKhBytes);
#pragma unroll
      for (int kt = 0; kt < kAmK / 32; ++kt) {
        floatx16_t sacc, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sacc[e] = 0.0f;
          dp[e] = 0.0f;
        }
        const int kr = kt * 32 + l32;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qf[t], *(const f16x8_t *)(kh + kr * L::kKh + 16 * t + 8 * h),
                                                         sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // (the fragments of one product at a time in registers)
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(df[t], *(const bf16x8_t *)(vr + kr * L::kVr + 16 * t + 8 * h),
                                                        dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // register e holds query qw0 + 8 (e/4) + 4 h + e%4 of key `key`; a
        // tile wholly in range and below a causal diagonal needs no masks
        const int64_t key = k0 + kr;
        auto form_ds = [&](auto masked) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int qi = 32 * w + 8 * c + 4 * h;
            const float4 l4 = *(const float4 *)(&qv[0][qi]);
            const float4 d4 = *(const float4 *)(&qv[1][qi]);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int e = 4 * c + r;
              const int64_t query = qw0 + 8 * c + 4 * h + r;
              const float p = __builtin_amdgcn_exp2f(sacc[e] * c_log2 - lv[r]);
              float dsv = p * (dp[e] - dl[r]);
              if constexpr (decltype(masked)::value) {
                const bool valid = key < S && query < S && (!a.causal || key <= query);
                dsv = valid ? dsv : 0.0f;
              }
              amax = fmaxf(amax, fabsf(dsv));
              if constexpr (KEEP) {
                if (key < S && query < S) a.ds[(g * S + query) * S + key] = dsv;
              }
            }
          }
        };
        const int64_t kt0 = k0 + kt * 32;
        if (!KEEP && qw0 + 31 < S && kt0 + 31 < S && (!a.causal || kt0 + 31 <= qw0)) form_ds(std::false_type{});
        else form_ds(std::true_type{});
        __builtin_amdgcn_sched_barrier(0);   // one 32-key tile at a time
      }
    }
    if (kb + 1 < nkb) store_block((int)((kb + 1) & 1));
    __syncthreads();
  }

  uint32_t m = __builtin_bit_cast(uint32_t, amax);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  if (lane == 0) red[w] = m;
  __syncthreads();
  if (tid == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int i = 1; i < kAttnThreads / 64; ++i) r = r > red[i] ? r : red[i];
    a.amax[blockIdx.x] = r;
  }
}

// ---- dS quantized where it is formed ----------------------------------------
// The second pass over the keys: with the amax of dS known from the first
// pass (its per-workgroup partials), each workgroup recomputes S, P, dP and
// dS for its 128 keys exactly as the first pass does (same operands, same
// instruction sequence) and encodes them into dS's two NVFP4 views, so dS
// never goes through memory in fp32.  A wave's 32 x 32 tile of dS is staged
// in its own LDS scratch; each lane then encodes one 16-key block of a query
// (the row-wise view, blocks along keys) and one 16-query block of a key (the
// column-wise view, blocks along queries).  Tiles wholly above a causal
// diagonal are not encoded: the dQ and dK products skip those blocks.
struct AttnDsqArgs {
  const uint8_t *q_codes, *q_scales, *k_codes, *k_scales;
  const float *q_ts, *k_ts;
  const uint16_t *v;      // bf16 [G][S][D]
  const uint16_t *dout;   // bf16 [G][S][D]
  const float *lse;       // [G][S], natural log
  const float *delta;     // [G][S]
  const uint32_t *amax;   // the first pass's partial maxima of |dS| (fp32 bits)
  int npart;
  fs4_nvfp4 row, col;     // dS views: row-wise [G*S][S], column-wise [S][G*S]
  int64_t G, S;
  float scale;
  int causal;
};

template <int D>
struct DsqLds {
  static constexpr int kQh = D + 8;
  static constexpr int kDo = D + 8;
  static constexpr int kQhOff = 0;
  static constexpr int kDoOff = kQhOff + kBwdQ * kQh * 2;
  static constexpr int kLseOff = kDoOff + kBwdQ * kDo * 2;
  static constexpr int kDeltaOff = kLseOff + kBwdQ * 4;
  static constexpr int kStage = kDeltaOff + kBwdQ * 4;
  static constexpr int kEpt = kBwdQ * D / kAttnThreads;
  static constexpr int kDoPer = kBwdQ * D * 2 / 16 / kAttnThreads;
  static constexpr int kT = 33;                       // scratch row stride (floats)
  static_assert(kStage % 16 == 0, "stage alignment");
};

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attention_dsq_kernel(AttnDsqArgs a) {
  using L = DsqLds<D>;
  constexpr int KSTEPS = D / 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kStage];   // one stage: two workgroups fit a CU
  __shared__ float scratch[kAttnThreads / 64][32 * L::kT];
  __shared__ Tables tab;
  __shared__ uint32_t red[kAttnThreads / 64];

  const int64_t G = a.G, S = a.S;
  const int64_t g = blockIdx.x % G;
  const int64_t kb = (int64_t)blockIdx.x / G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int64_t k0 = kb * kBwdKeys;
  const int64_t kw0 = k0 + w * 32;
  const int64_t key = kw0 + l32;
  const bool key_ok = key < S;
  const int64_t keyc = key_ok ? key : S - 1;

  // ---- dS's tensor scale from the first pass's partials; the tables --------
  uint32_t m = 0;
  for (int i = tid; i < a.npart; i += kAttnThreads) m = m > a.amax[i] ? m : a.amax[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(m, off, 64);
    m = m > o ? m : o;
  }
  if (lane == 0) red[w] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < kAttnThreads / 64; ++i) m = m > red[i] ? m : red[i];
  const float s_t = (float)((double)__builtin_bit_cast(float, m) / kTensorDiv);
  if (blockIdx.x == 0 && tid == 0) {
    *a.row.tscale = s_t;
    *a.col.tscale = s_t;
  }
  build_tables_n<kAttnThreads>(tab, s_t);
  const float inv6st = s_t > 0.0f ? (float)(1.0 / (6.0 * (double)s_t)) : 0.0f;   // may be inf
  const bool inv_finite = inv6st < __builtin_huge_valf();

  // ---- this wave's keys: K expanded to FP16 and V, as in the first pass ---
  f16x8_t kf[KSTEPS];
  bf16x8_t vf[KSTEPS];
  {
    const uint8_t *krow = a.k_codes + (g * S + keyc) * (D / 2);
    const uint8_t *ksc = a.k_scales + (g * S + keyc) * (D / 16);
    const uint16_t *vrow = a.v + (g * S + keyc) * D;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      kf[t] = expand8(*(const uint32_t *)(krow + 8 * t + 4 * h), split_scale(ksc[t]));
      vf[t] = *(const bf16x8_t *)(vrow + 16 * t + 8 * h);
    }
  }

  uint4 rq = make_uint4(0, 0, 0, 0);
  uint32_t rqs = 0;
  uint4 rdo[L::kDoPer];
  float rls = 0.0f;
  const int qrow = tid / 4, qc0 = (tid % 4) * L::kEpt;
  auto load_block = [&](int64_t q0) {
    {
      int64_t qq = q0 + qrow;
      qq = qq < S ? qq : S - 1;
      const uint8_t *cp = a.q_codes + (g * S + qq) * (D / 2) + qc0 / 2;
      const uint8_t *sp = a.q_scales + (g * S + qq) * (D / 16) + qc0 / 16;
      if constexpr (L::kEpt == 32) {
        rq = *(const uint4 *)cp;
        rqs = *(const uint16_t *)sp;
      } else {
        const uint2 t = *(const uint2 *)cp;
        rq = make_uint4(t.x, t.y, 0u, 0u);
        rqs = *sp;
      }
    }
#pragma unroll
    for (int i = 0; i < L::kDoPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      const int64_t qq = q0 + row;
      rdo[i] = qq < S ? *(const uint4 *)(a.dout + (g * S + qq) * D + ch * 8) : make_uint4(0, 0, 0, 0);
    }
    if (tid < 2 * kBwdQ) {
      const int64_t qq = q0 + (tid & (kBwdQ - 1));
      rls = qq < S ? (tid < kBwdQ ? a.lse[g * S + qq] * kLog2e : a.delta[g * S + qq]) : 0.0f;
    }
  };
  auto store_block = [&](int st) {
    uint8_t *base = lds + st * L::kStage;
    _Float16 *qh = (_Float16 *)(base + L::kQhOff) + qrow * L::kQh + qc0;
    const uint32_t cw[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
    for (int j = 0; j < L::kEpt / 8; ++j)
      *(f16x8_t *)(qh + 8 * j) = expand8(cw[j], split_scale((rqs >> (8 * (j / 2))) & 0xFFu));
#pragma unroll
    for (int i = 0; i < L::kDoPer; ++i) {
      const int idx = tid + i * kAttnThreads;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      *(uint4 *)(base + L::kDoOff + (row * L::kDo + ch * 8) * 2) = rdo[i];
    }
    if (tid < 2 * kBwdQ) ((float *)(base + L::kLseOff))[tid] = rls;
  };

  const float c_log2 = (*a.q_ts) * (*a.k_ts) * a.scale * kLog2e;
  float *sc = scratch[w];
  const int bi = lane >> 1, bh = lane & 1;   // this lane's blocks: (query bi, keys 16 bh..) and (key bi, queries 16 bh..)
  const int64_t GS = G * S;

  const int64_t nqb = (S + kBwdQ - 1) / kBwdQ;
  const int64_t qb0 = a.causal ? k0 / kBwdQ : 0;
  load_block(qb0 * kBwdQ);
  store_block(0);
  __syncthreads();

  for (int64_t qb = qb0; qb < nqb; ++qb) {
    if (qb + 1 < nqb) load_block((qb + 1) * kBwdQ);
    const uint8_t *base = lds;
    const _Float16 *qh = (const _Float16 *)(base + L::kQhOff);
    const uint16_t *dor = (const uint16_t *)(base + L::kDoOff);
    const float *lse2 = (const float *)(base + L::kLseOff);
    const float *dlt = (const float *)(base + L::kDeltaOff);
    const int64_t q0 = qb * kBwdQ;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int64_t qt0 = q0 + 32 * qt;
      // a tile wholly above the diagonal holds only zeros, which the dS
      // products never read (wave-uniform)
      if (qt0 >= S || (a.causal && qt0 + 31 < kw0)) continue;
      floatx16_t sacc, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[e] = 0.0f;
        dp[e] = 0.0f;
      }
      const int r = 32 * qt + l32;
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8_t *)(qh + r * L::kQh + 16 * t + 8 * h), kf[t],
                                                       sacc, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t *)(dor + r * L::kDo + 16 * t + 8 * h), vf[t],
                                                      dp, 0, 0, 0);
      // dS exactly as the first pass forms it; the tile goes to the scratch
      // as [key][query].  A tile with every (key, query) in range and, when
      // causal, wholly below the diagonal needs no masks (wave-uniform).
      auto form_ds = [&](auto masked) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int qi = 32 * qt + 8 * c + 4 * h;
          const float4 l4 = *(const float4 *)(lse2 + qi);
          const float4 d4 = *(const float4 *)(dlt + qi);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int e = 4 * c + rr;
            const float p = __builtin_amdgcn_exp2f(sacc[e] * c_log2 - lv[rr]);
            float ds = p * (dp[e] - dv[rr]);
            if constexpr (decltype(masked)::value) {
              const int64_t query = q0 + qi + rr;
              const bool valid = key_ok && query < S && (!a.causal || key <= query);
              ds = valid ? ds : 0.0f;
            }
            sc[l32 * L::kT + 8 * c + 4 * h + rr] = ds;
          }
        }
      };
      if (qt0 + 31 < S && kw0 + 31 < S && (!a.causal || kw0 + 31 <= qt0)) form_ds(std::false_type{});
      else form_ds(std::true_type{});
      __builtin_amdgcn_wave_barrier();
      // row-wise view: query bi of the tile, keys 16 bh .. 16 bh + 15
      {
        uint2 pk;
        const float *src = sc + 16 * bh * L::kT + bi;
        const uint32_t sb = encode16([&](int i) { return src[i * L::kT]; }, inv6st, inv_finite, tab, pk);
        const int64_t query = qt0 + bi, k16 = kw0 + 16 * bh;
        if (query < S && k16 < S) {
          *(uint2 *)(a.row.codes + (g * S + query) * (S / 2) + k16 / 2) = pk;
          a.row.scales[(g * S + query) * (S / 16) + k16 / 16] = (uint8_t)sb;
        }
      }
      // column-wise view: key bi of the tile, queries 16 bh .. 16 bh + 15
      {
        uint2 pk;
        const float *src = sc + bi * L::kT + 16 * bh;
        const uint32_t sb = encode16([&](int i) { return src[i]; }, inv6st, inv_finite, tab, pk);
        const int64_t kk = kw0 + bi, q16 = qt0 + 16 * bh;
        if (kk < S && q16 < S) {
          *(uint2 *)(a.col.codes + kk * (GS / 2) + (g * S + q16) / 2) = pk;
          a.col.scales[kk * (GS / 16) + (g * S + q16) / 16] = (uint8_t)sb;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (qb + 1 < nqb) {
      __syncthreads();
      store_block(0);
    }
    __syncthreads();
  }
}

// Delta[row] = sum_d dO[row][d] O[row][d] (fp32), D / 8 lanes per row
template <int D>
__global__ __launch_bounds__(256) void attention_delta_kernel(const uint16_t *__restrict__ dout,
                                                              const float *__restrict__ o, int64_t rows,
                                                              float *__restrict__ delta) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  float acc = 0.0f;
  if (row < rows) {
    const uint4 dw = *(const uint4 *)(dout + row * D + c);
    const float4 o0 = *(const float4 *)(o + row * D + c), o1 = *(const float4 *)(o + row * D + c + 4);
    const uint32_t wv[4] = {dw.x, dw.y, dw.z, dw.w};
    const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += __builtin_bit_cast(float, wv[i] << 16) * ov[2 * i];
      acc += __builtin_bit_cast(float, wv[i] & 0xFFFF0000u) * ov[2 * i + 1];
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && threadIdx.x % TPR == 0) delta[row] = acc;
}

// ---- dQ and dK: batched NT products of NVFP4 views --------------------------
// C_g = s_a s_b scale A_g B_g^T for every sequence g, A_g [S][S] and B_g [D][S]
// NVFP4 views (blocks along the contraction) at a per-sequence offset within
// larger views.  Under a causal mask dS is lower triangular, so dQ's rows
// (queries) contract over the keys up to their block's end, and dK's rows
// (keys) over the queries from their block's start; the skipped products are
// exact zeros.  Each workgroup forms 256 rows x D, 64 rows per wave, with
// both operands expanded to FP16 into LDS 64 columns at a time.
constexpr int kDsBM = 256;
constexpr int kDsKC = 64;

struct DsOperand {
  const uint8_t *codes, *scales;
  int64_t ld, gs;   // bytes of codes: row stride and per-sequence offset (scales: both / 8)
};
struct DsGemmArgs {
  DsOperand a[2], b[2];
  const float *ts_a[2], *ts_b[2];
  float *c[2];      // fp32 [G][S][D]
  int mode[2];      // 0 every column, 1 columns before the row block's end, 2 from its start
  int64_t G, S;
  float scale;
};

template <int D>
__global__ __launch_bounds__(256, 2) void attention_ds_gemm_kernel(DsGemmArgs p) {
  constexpr int TN = D / 32;
  constexpr int TM = 2;
  // An LDS stage holds a chunk's codes and scales as they sit in memory (4
  // bits per element); each wave expands the fragments it multiplies in
  // registers, so the LDS traffic per MFMA is a quarter of FP16 staging.
  constexpr int kCS = kDsKC / 2 + 8;            // code bytes per LDS row (40: 2-way conflicts at most)
  constexpr int kSB = kDsKC / 16;               // scale bytes per row and chunk
  constexpr int A_C = kDsBM * kCS, B_C = D * kCS, A_S = kDsBM * kSB, B_S = D * kSB;
  constexpr int STAGE = A_C + B_C + A_S + B_S;
  // staging unit: one 16-element block of a row (8 code bytes, 1 scale byte)
  constexpr int AU = kDsBM * kSB, BU = D * kSB;
  constexpr int APER = AU / 256, BPER = (BU + 255) / 256;
  static_assert(AU % 256 == 0 && kSB == 4, "staging");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
  __shared__ uint2 lut[128];   // E4M3 byte -> {2^E as fp32 bits, F as two FP16}

  const int z = blockIdx.y;
  const DsOperand A = p.a[z], B = p.b[z];
  const int mode = p.mode[z];
  const int64_t G = p.G, S = p.S;
  const int64_t nrb = (S + kDsBM - 1) / kDsBM;
  const int64_t g = blockIdx.x % G;
  const int64_t rbx = (int64_t)blockIdx.x / G;
  const int64_t rb = mode == 1 ? nrb - 1 - rbx : rbx;   // the longest row blocks first
  const int64_t r0 = rb * kDsBM;
  const int64_t k_lo = mode == 2 ? r0 : 0;
  const int64_t k_hi = mode == 1 ? (r0 + kDsBM < S ? r0 + kDsBM : S) : S;
  const int nkc = (int)((k_hi - k_lo + kDsKC - 1) / kDsKC);
  const uint8_t *ac = A.codes + g * A.gs, *as = A.scales + g * (A.gs / 8);
  const uint8_t *bc = B.codes + g * B.gs, *bs = B.scales + g * (B.gs / 8);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;

  for (int b = tid; b < 128; b += 256) {
    const ScalePair sp = split_scale((uint32_t)b);
    lut[b] = make_uint2(__builtin_bit_cast(uint32_t, sp.pow2), __builtin_bit_cast(uint32_t, sp.mant));
  }

  // A block is zero, and masked to zero (codes and scale) where it is stored,
  // when it lies past S or k_hi or wholly above a causal diagonal: dQ (rows
  // are queries) past the row, dK (rows are keys) before it.  The loads read
  // clamped, in-range blocks, so that none sits in a branch.
  auto a_blk_ok = [&](int64_t rg, int64_t kg) {
    const bool above = (mode == 1 && kg > rg) || (mode == 2 && kg + 15 < rg);
    return rg < S && kg < k_hi && !above;
  };
  uint2 ra[APER], rbv[BPER];
  uint8_t rsa[APER], rsb[BPER];
  auto load = [&](int kc) {
    const int64_t kk0 = k_lo + (int64_t)kc * kDsKC;
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int u = tid + i * 256, row = u / kSB, blk = u % kSB;
      int64_t rg = r0 + row, kg = kk0 + 16 * blk;
      rg = rg < S ? rg : S - 1;
      kg = kg < k_hi ? kg : k_hi - 16;
      ra[i] = *(const uint2 *)(ac + rg * A.ld + kg / 2);
      rsa[i] = as[rg * (A.ld / 8) + kg / 16];
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int u = tid + i * 256, row = (u < BU ? u : 0) / kSB, blk = u % kSB;
      int64_t kg = kk0 + 16 * blk;
      kg = kg < k_hi ? kg : k_hi - 16;
      rbv[i] = *(const uint2 *)(bc + row * B.ld + kg / 2);
      rsb[i] = bs[row * (B.ld / 8) + kg / 16];
    }
  };
  auto store = [&](int st, int kc) {
    const int64_t kk0 = k_lo + (int64_t)kc * kDsKC;
    uint8_t *base = lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int u = tid + i * 256, row = u / kSB, blk = u % kSB;
      const uint32_t m = a_blk_ok(r0 + row, kk0 + 16 * blk) ? 0xFFFFFFFFu : 0u;
      *(uint2 *)(base + row * kCS + 8 * blk) = make_uint2(ra[i].x & m, ra[i].y & m);
      base[A_C + B_C + row * kSB + blk] = (uint8_t)(rsa[i] & m);
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int u = tid + i * 256, row = u / kSB, blk = u % kSB;
      if (u < BU) {
        const uint32_t m = kk0 + 16 * blk < k_hi ? 0xFFFFFFFFu : 0u;
        *(uint2 *)(base + A_C + row * kCS + 8 * blk) = make_uint2(rbv[i].x & m, rbv[i].y & m);
        base[A_C + B_C + A_S + row * kSB + blk] = (uint8_t)(rsb[i] & m);
      }
    }
  };

  floatx16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto lut_pair = [&](uint32_t byte) {
    const uint2 v = lut[byte & 0x7Fu];
    ScalePair sp;
    sp.pow2 = __builtin_bit_cast(float, v.x);
    sp.mant = __builtin_bit_cast(f16x2_t, v.y);
    return sp;
  };
  if (nkc > 0) {
    load(0);
    store(0, 0);
  }
  __syncthreads();   // the table and the first chunk
  for (int kc = 0; kc < nkc; ++kc) {
    if (kc + 1 < nkc) load(kc + 1);
    const uint8_t *base = lds + (kc & 1) * STAGE;
    const uint8_t *a_rows = base + (64 * w + l32) * kCS, *b_rows = base + A_C + l32 * kCS;
    uint32_t sa[TM], sb[TN];   // the chunk's four scale bytes of each fragment row
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = *(const uint32_t *)(base + A_C + B_C + (64 * w + 32 * i + l32) * kSB);
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = *(const uint32_t *)(base + A_C + B_C + A_S + (32 * j + l32) * kSB);
#pragma unroll
    for (int ks = 0; ks < kDsKC / 16; ++ks) {
      f16x8_t af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = expand8(*(const uint32_t *)(a_rows + 32 * i * kCS + 8 * ks + 4 * h), lut_pair(sa[i] >> (8 * ks)));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = expand8(*(const uint32_t *)(b_rows + 32 * j * kCS + 8 * ks + 4 * h), lut_pair(sb[j] >> (8 * ks)));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kc + 1 < nkc) store((kc + 1) & 1, kc + 1);   // that stage was last read in chunk kc - 1
    __syncthreads();
  }

  // ---- C = alpha acc: lane holds column 32 j + l32, rows 8 (e/4) + 4 h + e%4
  const float alpha = (*p.ts_a[z]) * (*p.ts_b[z]) * p.scale;
  float *c = p.c[z] + g * S * D;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = r0 + 64 * w + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
      if (row < S) {
#pragma unroll
        for (int j = 0; j < TN; ++j) c[row * D + 32 * j + l32] = alpha * acc[i][j][e];
      }
    }
}

}  // namespace

size_t attention_fwd_ws_bytes(int64_t, int64_t, int64_t) { return 0; }

fs4_status launch_attention_fwd(const fs4_nvfp4 &Q, const fs4_nvfp4 &K, const uint16_t *V, int64_t G, int64_t S,
                                int64_t D, int causal, float *O, float *LSE, uint16_t *Vt, hipStream_t s) {
  if (Vt) {
    // V^T as a side output, for callers that keep it
    const dim3 tg((unsigned)((S + 63) / 64), (unsigned)((D + 63) / 64), (unsigned)G);
    transpose_bf16_kernel<<<tg, 256, 0, s>>>(V, S, D, Vt);
    if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;
  }
  AttnArgs a;
  a.q_codes = Q.codes; a.q_scales = Q.scales; a.k_codes = K.codes; a.k_scales = K.scales;
  a.q_ts = Q.tscale; a.k_ts = K.tscale;
  a.v = V; a.o = O; a.lse = LSE;
  a.G = G; a.S = S;
  a.scale = (float)(1.0 / __builtin_sqrt((double)D));
  a.causal = causal;
  const int64_t nqb = (S + kBQ - 1) / kBQ;
  const unsigned grid = (unsigned)(G * nqb);
  if (D == 128) attention_fwd_kernel<128><<<grid, kAttnThreads, 0, s>>>(a);
  else attention_fwd_kernel<64><<<grid, kAttnThreads, 0, s>>>(a);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

size_t attention_bwd_ws_bytes(int64_t G, int64_t S, int64_t D) {
  Carver c(nullptr);
  attention_bwd_carve(c, G, S, D);
  return c.off;
}

AttnBwdWs attention_bwd_carve(Carver &c, int64_t G, int64_t S, int64_t D) {
  AttnBwdWs w;
  w.delta = (float *)c.take((size_t)(G * S) * 4);
  static_assert(kBwdKeys == kBQ, "one amax partial per 128 queries and per 128 keys alike");
  w.nwg = G * ((S + kBwdKeys - 1) / kBwdKeys);
  w.amax = (uint32_t *)c.take((size_t)w.nwg * 4);
  w.ds_row = carve_view(c, G * S, S);
  w.ds_col = carve_view(c, S, G * S);
  return w;
}

fs4_status launch_attention_bwd(const fs4_nvfp4 &Qr, const fs4_nvfp4 &Kr, const fs4_nvfp4 &Qc,
                                const fs4_nvfp4 &Kc, const uint16_t *V, const uint16_t *dO, const float *O,
                                const float *LSE, int64_t G, int64_t S, int64_t D, int causal, float *dQ,
                                float *dK, float *dV, float *dS, const AttnBwdWs &w, hipStream_t s) {
  const int64_t rows = G * S;
  const unsigned dgrid = (unsigned)((rows + (256 / (D / 8)) - 1) / (256 / (D / 8)));
  if (D == 128) attention_delta_kernel<128><<<dgrid, 256, 0, s>>>(dO, O, rows, w.delta);
  else attention_delta_kernel<64><<<dgrid, 256, 0, s>>>(dO, O, rows, w.delta);
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;

  const float scale = (float)(1.0 / __builtin_sqrt((double)D));
  // the amax of dS (and dS when asked for), query-major
  AttnAmaxArgs x;
  x.q_codes = Qr.codes; x.q_scales = Qr.scales; x.k_codes = Kr.codes; x.k_scales = Kr.scales;
  x.q_ts = Qr.tscale; x.k_ts = Kr.tscale;
  x.v = V; x.dout = dO; x.lse = LSE; x.delta = w.delta;
  x.ds = dS; x.amax = w.amax;
  x.G = G; x.S = S;
  x.scale = scale;
  x.causal = causal;
  const unsigned xgrid = (unsigned)(G * ((S + kBQ - 1) / kBQ));   // == w.nwg (128 rows either way)
  if (dS) {
    if (D == 128) attention_amax_kernel<128, true><<<xgrid, kAttnThreads, 0, s>>>(x);
    else attention_amax_kernel<64, true><<<xgrid, kAttnThreads, 0, s>>>(x);
  } else {
    if (D == 128) attention_amax_kernel<128, false><<<xgrid, kAttnThreads, 0, s>>>(x);
    else attention_amax_kernel<64, false><<<xgrid, kAttnThreads, 0, s>>>(x);
  }
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;

  // first pass over the keys: dV = P^T dO
  AttnBwdArgs a;
  a.q_codes = Qr.codes; a.q_scales = Qr.scales; a.k_codes = Kr.codes; a.k_scales = Kr.scales;
  a.q_ts = Qr.tscale; a.k_ts = Kr.tscale;
  a.dout = dO; a.lse = LSE; a.dv = dV;
  a.G = G; a.S = S;
  a.scale = scale;
  a.causal = causal;
  if (D == 128) attention_bwd_kernel<128><<<(unsigned)w.nwg, kAttnThreads, 0, s>>>(a);
  else attention_bwd_kernel<64><<<(unsigned)w.nwg, kAttnThreads, 0, s>>>(a);
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;

  // second pass: dS again, encoded into its row-wise (blocks along keys) and
  // column-wise (blocks along queries) views
  AttnDsqArgs q;
  q.q_codes = Qr.codes; q.q_scales = Qr.scales; q.k_codes = Kr.codes; q.k_scales = Kr.scales;
  q.q_ts = Qr.tscale; q.k_ts = Kr.tscale;
  q.v = V; q.dout = dO; q.lse = LSE; q.delta = w.delta;
  q.amax = w.amax; q.npart = (int)w.nwg;
  q.row = w.ds_row; q.col = w.ds_col;
  q.G = G; q.S = S;
  q.scale = scale;
  q.causal = causal;
  if (D == 128) attention_dsq_kernel<128><<<(unsigned)w.nwg, kAttnThreads, 0, s>>>(q);
  else attention_dsq_kernel<64><<<(unsigned)w.nwg, kAttnThreads, 0, s>>>(q);
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;

  DsGemmArgs p;
  // dQ_g = Q(dS_g) Q_col(K_g)^T: dS rows g*S.., K^T columns g*S..
  p.a[0] = {w.ds_row.codes, w.ds_row.scales, S / 2, S * S / 2};
  p.b[0] = {Kc.codes, Kc.scales, G * S / 2, S / 2};
  p.ts_a[0] = w.ds_row.tscale; p.ts_b[0] = Kc.tscale; p.c[0] = dQ; p.mode[0] = causal ? 1 : 0;
  // dK_g = Q(dS_g^T) Q_col(Q_g)^T: dS^T columns g*S.., Q^T columns g*S..
  p.a[1] = {w.ds_col.codes, w.ds_col.scales, G * S / 2, S / 2};
  p.b[1] = {Qc.codes, Qc.scales, G * S / 2, S / 2};
  p.ts_a[1] = w.ds_col.tscale; p.ts_b[1] = Qc.tscale; p.c[1] = dK; p.mode[1] = causal ? 2 : 0;
  p.G = G; p.S = S;
  p.scale = scale;
  const dim3 grid((unsigned)(G * ((S + kDsBM - 1) / kDsBM)), 2);
  if (D == 128) attention_ds_gemm_kernel<128><<<grid, 256, 0, s>>>(p);
  else attention_ds_gemm_kernel<64><<<grid, 256, 0, s>>>(p);
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

}  // namespace fs4
