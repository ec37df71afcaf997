// Block-scaled NVFP4 NT GEMM for gfx950 with a fused epilogue.
//
//   C[m][n] = alpha * s_tA * s_tB * sum_k A_hat[m][k] B_hat[n][k]
//             + sum_j (l_scale * L[m][j]) R(n, j)            (low-rank term)
//             + beta_e * E[m][n]
//
// A_hat = e2m1(code) * e4m3(s_b).  An E2M1 magnitude has <= 2 significant
// bits and an E4M3 scale <= 4, so their product has <= 6 significant bits and
// lies in [2^-10, 2688]: it is exact in FP16.  Packed codes are staged in LDS
// as they sit in memory (4 bits per element) and expanded in registers right
// before FP16 MFMA with fp32 accumulation:
//   - write the scale as 2^E * F with F in [1, 2) (3 mantissa bits);
//   - v_cvt_scalef32_pk_f16_fp4 turns two codes into two FP16 values times a
//     power-of-two scale (the instruction takes only the exponent of its fp32
//     scale operand, so 2^E is passed);
//   - one packed FP16 multiply by F completes code * s_b, exactly.
//
// Full-Stack FP4 [FS4 §2.1] runs the projection GEMMs on NVFP4 operands while
// the rank-r term stays in BF16: L = X V^T arrives in fp32, is split into BF16
// hi + lo parts and runs as extra BF16 MFMA k-steps into the accumulators
// after they have been scaled by alpha s_tA s_tB (operands staged in LDS once
// per workgroup).
//
// On gfx950 a wave's VALU work and its MFMAs do not overlap much (measured),
// so the VALU count per MFMA bounds the kernel: expanding an A fragment once
// serves TN MFMAs and a B fragment TM MFMAs.  Codes are read from LDS one
// 16-element block per k-step pair, and the next step's operands are
// expanded right before the current step's MFMAs are issued.
//
// Tiling: a workgroup of WM x WN waves computes (WM*TM*32) x (WN*TN*32) of C,
// each wave TM x TN accumulators of v_mfma_f32_32x32x16_f16.  The k-tile is
// 128 elements (64 code bytes and 8 scale bytes per row), double-buffered in
// LDS with the next tile prefetched into registers while the current one is
// multiplied.  Within a k-tile, lanes 0-31 of a wave take elements [0, 64)
// and lanes 32-63 take [64, 128): MFMA k-step s uses elements 64h + 8s .. +8
// for lane half h on both operands, so every step pairs equal k (the order of
// summation over k is permuted, the set is not).
//
// Workgroups are ordered XCD-aware: the hardware deals workgroup ids round-
// robin over the 8 XCDs, so ids are remapped to give each XCD a contiguous
// run of tiles, walked in groups of rows so that concurrently running tiles
// share A and B panels in that XCD's L2.
#include <type_traits>

#include "fs4_common.h"

namespace fs4 {
namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;          // k-tile in elements
constexpr int kRowBytes = 64;     // code bytes per row per k-tile
constexpr int kLdsStride = 80;    // padded LDS row stride (conflict-free 16-byte reads)
constexpr int kXcds = 8;
constexpr int kLrStrideMax = 72;  // epilogue LDS row stride (BF16 elements) for rank <= 64
constexpr int kGroupM = 8;

struct GemmArgs {
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  const float *a_ts, *b_ts;
  int64_t M, N, K;
  float alpha, beta_e, l_scale;
  const float *E;
  float *C;
  const float *L;
  const uint16_t *R;
  int64_t r_sn, r_sj;
  int r;
  uint32_t *amax_parts;   // nullable: per-tile max |C| (fp32 bits)
  // sym: C is symmetric (A and B the same view): only tiles with
  // tile_m <= tile_n are computed, each stored at both positions.
  int sym;
  int mirror;   // with sym: store each tile at its mirrored position too
  float *Ct;    // nullable: C is stored transposed, Ct[n][m] (leading dimension M), instead
  // Split-k: tiles [0, t_full) run whole, one workgroup each; every later
  // tile runs as s_tail workgroups over consecutive ranges of whole k-tiles,
  // which store their raw fp32 accumulators to `part` (slot (tile - t_full)
  // * s_tail + split, in accumulator order) and end; split_reduce_kernel
  // then adds them in split order and runs the epilogue.
  int64_t t_full;
  int s_tail;
  float *part;
};

// E4M3 block scale -> (2^E as fp32, F as a pair of FP16) with s_b = 2^E F.
struct ScalePair {
  float pow2;
  f16x2_t mant;
};
__device__ inline ScalePair split_scale(uint32_t byte) {
  const uint32_t fb = __builtin_bit_cast(uint32_t, e4m3_to_float(byte));
  ScalePair s;
  s.pow2 = __builtin_bit_cast(float, fb & 0x7F800000u);    // 0 for a zero scale
  const uint32_t h = 0x3C00u | (((fb >> 20) & 7u) << 7);    // FP16 1 + m/8
  s.mant = __builtin_bit_cast(f16x2_t, h | (h << 16));
  return s;
}

// Fills a 256-entry LDS table: entry b = {bits of 2^E, FP16 pair F} for the
// E4M3 byte b (only 0..0x7E occur; the rest decode to something finite).
__device__ inline void fill_scale_lut(uint2 *lut) {
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    const ScalePair p = split_scale((uint32_t)b & 0x7Fu);
    lut[b] = make_uint2(__builtin_bit_cast(uint32_t, p.pow2), __builtin_bit_cast(uint32_t, p.mant));
  }
}
__device__ inline ScalePair lut_scale(const uint2 *lut, uint32_t byte) {
  const uint2 v = lut[byte];
  ScalePair p;
  p.pow2 = __builtin_bit_cast(float, v.x);
  p.mant = __builtin_bit_cast(f16x2_t, v.y);
  return p;
}

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

__device__ inline bf16x8_t bits_to_bf16x8(const uint32_t *b) {
  bf16x8_t f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = __builtin_bit_cast(__bf16, (uint16_t)b[i]);
  return f;
}

// tile id -> (tile_m, tile_n): XCD-contiguous runs, grouped by kGroupM rows
__device__ inline void tile_coords(int64_t bid, int64_t tiles_m, int64_t tiles_n, int64_t *tm,
                                   int64_t *tn) {
  const int64_t T = tiles_m * tiles_n;
  int64_t L = bid;
  if (T % kXcds == 0) L = (bid % kXcds) * (T / kXcds) + bid / kXcds;
  const int64_t per_group = kGroupM * tiles_n;
  const int64_t group = L / per_group;
  const int64_t first_m = group * kGroupM;
  const int64_t gsz = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int64_t in_group = L - group * per_group;
  *tm = first_m + in_group % gsz;
  *tn = in_group / gsz;
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (a loop whose index
// is a constant expression in the body).
template <int B, int E, class F>
__device__ inline void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Word 3 of a raw buffer resource: 32-bit data format (untyped dword access).
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer store: the non-temporal (streaming) bit.
constexpr int kStoreNT = 2;

// Direct global->LDS loads (gfx950 global_load_lds): lane l's 16 (or 4)
// bytes from `src` land at LDS byte address `lds_dst + 16 l` (or + 4 l);
// lds_dst must be wave-uniform.  Issued as inline assembly so the compiler
// does not guard every later LDS read with a wait for them; the kernel waits
// explicitly (wait_vmcnt) before a barrier publishes a stage.
// M0 (the LDS destination register) is set inside each statement and listed
// as clobbered; the compiler warns that it is a reserved register, and nothing
// else in these kernels uses it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The source is a wave-uniform base (scalar registers) plus a 32-bit per-lane
// byte offset.
__device__ inline void lds_dma16(uint32_t lds_dst, const void *base, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_dst), "v"(off), "s"(base)
               : "memory", "m0");
}
__device__ inline void lds_dma4(uint32_t lds_dst, const void *base, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_dst), "v"(off), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// KFAST: K % 128 == 0 (16-byte code chunks, 8-byte scale chunks, no k tail);
// otherwise K % 16 == 0 with 8-byte code chunks and byte-wise scales.
template <int WM, int WN, int TM, int TN, bool KFAST>
__global__ __launch_bounds__(WM *WN * 64) void gemm_nt_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int A_BYTES = BM * kLdsStride, B_BYTES = BN * kLdsStride;
  constexpr int STAGE = A_BYTES + B_BYTES + BM * 8 + BN * 8;
  // KFAST stages are filled by direct global->LDS loads: unpadded 64-byte code
  // rows (16-byte slots XOR-swizzled by row), then 8 scale bytes per row; four
  // stages, plus 1 KB that idle load instructions write to
  constexpr int STAGE_D = (BM + BN) * (kRowBytes + 8);
  constexpr int MAIN_BYTES = KFAST ? 4 * STAGE_D + 1024 : 2 * STAGE;
  constexpr int LR_BYTES = (2 * BM + BN) * kLrStrideMax * 2;   // rank-r staging in the epilogue
  constexpr int LDS_BYTES = MAIN_BYTES > LR_BYTES ? MAIN_BYTES : LR_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ uint2 scale_lut[256];

  const int64_t tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  // workgroup -> (tile, split)
  const int64_t wu = blockIdx.x;
  int64_t tile = wu;
  int S = 1, sp = 0;
  if (wu >= g.t_full) {
    tile = g.t_full + (wu - g.t_full) / g.s_tail;
    sp = (int)((wu - g.t_full) % g.s_tail);
    S = g.s_tail;
  }
  int64_t tile_m, tile_n;
  if (g.sym) {
    // tile -> (tile_m <= tile_n), row by row of the upper triangle
    int64_t t = tile, tm = 0;
    while (t >= tiles_n - tm) { t -= tiles_n - tm; ++tm; }
    tile_m = tm;
    tile_n = tm + t;
  } else {
    tile_coords(tile, tiles_m, tiles_n, &tile_m, &tile_n);
  }
  const int64_t m0 = tile_m * BM, n0 = tile_n * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // the same value, known uniform
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t K = g.K, kb = K / 2, ks = K / kBlock;
  const int nk_all = (int)((K + kBK - 1) / kBK);
  const int kt_per = (nk_all + S - 1) / S;
  // (uniform values, kept in scalar registers: they form load addresses)
  const int kt0 = __builtin_amdgcn_readfirstlane(sp * kt_per);   // this split's first k-tile
  const int nk = __builtin_amdgcn_readfirstlane((kt0 + kt_per < nk_all ? kt0 + kt_per : nk_all) - kt0);

  // ---- global -> register staging ----------------------------------------
  constexpr int CH = KFAST ? 16 : 8;
  constexpr int PER_ROW = kRowBytes / CH;
  constexpr int A_CH = BM * PER_ROW / NT, B_CH = BN * PER_ROW / NT;
  constexpr int SCH = KFAST ? 8 : 1;                       // scale bytes per load
  constexpr int SA_N = BM * 8 / SCH, SB_N = BN * 8 / SCH;  // scale chunks per tile
  constexpr int SA_CH = (SA_N + NT - 1) / NT, SB_CH = (SB_N + NT - 1) / NT;
  static_assert(A_CH >= 1 && B_CH >= 1 && SA_CH >= 1 && SB_CH >= 1, "tile too small");
  static_assert(BM * PER_ROW % NT == 0 && BN * PER_ROW % NT == 0, "uneven staging");
  typedef typename std::conditional<KFAST, uint4, uint2>::type chunk_t;
  typedef typename std::conditional<KFAST, uint2, uint8_t>::type schunk_t;
  chunk_t ra[A_CH], rb[B_CH];
  schunk_t rsa[SA_CH], rsb[SB_CH];

  auto load_global = [&](int kt) {
    const int64_t kbyte0 = (int64_t)(kt0 + kt) * kRowBytes, ksc0 = (int64_t)(kt0 + kt) * 8;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      const int row = c / PER_ROW, seg = c % PER_ROW;
      const int64_t gm = m0 + row, gb = kbyte0 + seg * CH;
      chunk_t v = {};
      if (gm < g.M && (KFAST || gb < kb)) v = *(const chunk_t *)(g.a_codes + gm * kb + gb);
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT;
      const int row = c / PER_ROW, seg = c % PER_ROW;
      const int64_t gn = n0 + row, gb = kbyte0 + seg * CH;
      chunk_t v = {};
      if (gn < g.N && (KFAST || gb < kb)) v = *(const chunk_t *)(g.b_codes + gn * kb + gb);
      rb[i] = v;
    }
#pragma unroll
    for (int i = 0; i < SA_CH; ++i) {
      const int c = tid + i * NT;
      const int row = c / (8 / SCH), j = (c % (8 / SCH)) * SCH;
      const int64_t gm = m0 + row, gs = ksc0 + j;
      schunk_t v = {};
      if (c < SA_N && gm < g.M && (KFAST || gs < ks)) v = *(const schunk_t *)(g.a_scales + gm * ks + gs);
      rsa[i] = v;
    }
#pragma unroll
    for (int i = 0; i < SB_CH; ++i) {
      const int c = tid + i * NT;
      const int row = c / (8 / SCH), j = (c % (8 / SCH)) * SCH;
      const int64_t gn = n0 + row, gs = ksc0 + j;
      schunk_t v = {};
      if (c < SB_N && gn < g.N && (KFAST || gs < ks)) v = *(const schunk_t *)(g.b_scales + gn * ks + gs);
      rsb[i] = v;
    }
  };
  auto store_lds = [&](int stage) {
    uint8_t *la = lds + stage * STAGE, *lb = la + A_BYTES, *lsa = lb + B_BYTES, *lsb = lsa + BM * 8;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      *(chunk_t *)(la + (c / PER_ROW) * kLdsStride + (c % PER_ROW) * CH) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT;
      *(chunk_t *)(lb + (c / PER_ROW) * kLdsStride + (c % PER_ROW) * CH) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < SA_CH; ++i)
      if (tid + i * NT < SA_N) *(schunk_t *)(lsa + (tid + i * NT) * SCH) = rsa[i];
#pragma unroll
    for (int i = 0; i < SB_CH; ++i)
      if (tid + i * NT < SB_N) *(schunk_t *)(lsb + (tid + i * NT) * SCH) = rsb[i];
  };

  floatx16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  fill_scale_lut(scale_lut);
  const int sw = ((l32 >> 1) ^ (l32 >> 3)) & 3;    // slot swizzle of this lane's rows (KFAST stages)

  // One k-tile from an LDS stage is 8 k-steps of TM x TN MFMAs.  Step s uses
  // the 32-bit code word s%4 of code pair s/4 (a pair is two blocks, 16
  // bytes of a row for this lane half) and the scales of block s/2.  Step
  // s+1's operands are expanded while step s's MFMAs run.  Codes are read
  // in 8-byte halves two steps ahead of their use, into the registers of the
  // half they replace: lo = words 0-1, hi = words 2-3.
  struct Stage { const uint8_t *a, *b, *sa, *sb; };
  uint32_t sa4[TM], sb4[TN];      // the four scale bytes of each row's blocks in this lane half
  uint2 clo_a[TM], clo_b[TN], chi_a[TM], chi_b[TN];
  ScalePair sa[2][TM], sb[2][TN];   // the scales of the blocks in use, by block parity
  f16x8_t av[TM], bv[TN];         // operands of the current k-step
  // half q (0: words 0-1, 1: words 2-3) of code pair p of row r
  auto codes_at = [&](const uint8_t *base, int r, int p, int q) -> uint2 {
    if constexpr (KFAST) return *(const uint2 *)(base + r * kRowBytes + (((2 * h + p) ^ sw) << 4) + q * 8);
    else return *(const uint2 *)(base + r * kLdsStride + h * 32 + p * 16 + q * 8);
  };
  auto read_codes = [&](const Stage &t, int p, int q) {
    uint2 *da = q ? chi_a : clo_a, *db = q ? chi_b : clo_b;
#pragma unroll
    for (int i = 0; i < TM; ++i) da[i] = codes_at(t.a, wm * TM * 32 + i * 32 + l32, p, q);
#pragma unroll
    for (int j = 0; j < TN; ++j) db[j] = codes_at(t.b, wn * TN * 32 + j * 32 + l32, p, q);
  };
  auto read_scales = [&](int blk) {
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[blk & 1][i] = lut_scale(scale_lut, (sa4[i] >> (8 * blk)) & 0xFFu);
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[blk & 1][j] = lut_scale(scale_lut, (sb4[j] >> (8 * blk)) & 0xFFu);
  };
  auto expand_step = [&](int s, f16x8_t *ao, f16x8_t *bo) {
    const int w = s & 3;
    const uint2 *wa = w < 2 ? clo_a : chi_a, *wb = w < 2 ? clo_b : chi_b;
#pragma unroll
    for (int i = 0; i < TM; ++i) ao[i] = expand8((w & 1) ? wa[i].y : wa[i].x, sa[(s >> 1) & 1][i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) bo[j] = expand8((w & 1) ? wb[j].y : wb[j].x, sb[(s >> 1) & 1][j]);
  };
  auto read_scale_bytes = [&](const Stage &t) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sa4[i] = *(const uint32_t *)(t.sa + (wm * TM * 32 + i * 32 + l32) * 8 + h * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sb4[j] = *(const uint32_t *)(t.sb + (wn * TN * 32 + j * 32 + l32) * 8 + h * 4);
  };
  // a stage's scale bytes and first code pair, then its step 0
  auto begin_tile = [&](const Stage &t) {
    read_scale_bytes(t);
    read_codes(t, 0, 0);
    read_codes(t, 0, 1);
    read_scales(0);
    expand_step(0, av, bv);
  };
  // The 8 k-steps of stage t (whose step 0 is already in av/bv, whose
  // pair-0 codes are in clo/chi and whose block-0 scales are in set 0).
  // Reads: pair 1 lo in step 1, pair 1 hi in step 3; the scales of block b
  // (b = 1, 2, 3) in step 2b - 2, one step before the step that expands with
  // them first, so that their LDS latency passes under that step's MFMAs.
  // With CROSS, stage nt's scale bytes (step 5), its block-0 scales (step 6)
  // and its pair 0 (lo in step 5, hi in step 7) are read too, and the last
  // step expands nt's step 0, so no k-step runs without expansion work beside
  // its MFMAs.  mid() runs after step 3, once this wave has issued its last
  // read of t; the reads of nt come after it.
  auto run_tile = [&](const Stage &t, const Stage &nt, auto cross, auto mid) {
    constexpr bool CROSS = decltype(cross)::value;
    static_for<0, 8>([&](auto step) {
      constexpr int s = decltype(step)::value;
      constexpr bool EXPAND = s + 1 < 8 || CROSS;
      f16x8_t an[TM], bn[TN];
      if constexpr (s == 1) read_codes(t, 1, 0);
      if constexpr (s == 3) read_codes(t, 1, 1);
      if constexpr (s == 0 || s == 2 || s == 4) read_scales(s / 2 + 1);
      if constexpr (CROSS && s == 5) {
        read_codes(nt, 0, 0);
        read_scale_bytes(nt);   // this stage's were last decoded in step 4
      }
      if constexpr (CROSS && s == 6) read_scales(0);
      if constexpr (CROSS && s == 7) read_codes(nt, 0, 1);
      if constexpr (s + 1 < 8) expand_step(s + 1, an, bn);
      else if constexpr (CROSS) expand_step(0, an, bn);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      if constexpr (EXPAND) {
        // Interleave: each MFMA (32 cycles in the matrix pipe) is followed by
        // an even share of the next step's expansion, which the SIMD issues
        // while the MFMA runs.  Left to itself the scheduler clusters the
        // conversions into long VALU runs that stall the matrix pipe.
        constexpr int VPM = (8 * (TM + TN) + TM * TN - 1) / (TM * TN);
#pragma unroll
        for (int i = 0; i < TM * TN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0); // VPM VALU
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) av[i] = an[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) bv[j] = bn[j];
      }
      __builtin_amdgcn_sched_barrier(0);   // one scheduling region per k-step
      if constexpr (s == 3) {
        mid();
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };

  if constexpr (KFAST) {
    // Four-stage pipeline of direct global->LDS loads (no staging registers).
    // Tile kt+3's loads are issued as tile kt starts, into the stage of tile
    // kt-1.  One barrier per tile, in its middle: before it each wave has
    // issued its last read of tile kt and waited for its own loads of tile
    // kt+1; after it tile kt+1 is visible to all and tile kt's stage may be
    // refilled (at the start of tile kt+1).  So the last k-step of tile kt
    // can already read and expand tile kt+1.
    // Every wave issues the same number of 64-lane load instructions per tile
    // (idle ones write the spare 1 KB), so "tile kt+1 has landed" is exactly
    // "at most DMA_PER_TILE loads outstanding per tile issued after it".  Rows
    // past M or N load a clamped row: they only feed outputs that are never
    // stored.
    constexpr int NW = NT / 64;
    constexpr int CODE_Q = (BM + BN) * 4, SC_U = (BM + BN) * 2;
    static_assert(CODE_Q % 64 == 0 && SC_U % 64 == 0, "load instructions must be all-real or all-idle");
    constexpr int CODE_I = (CODE_Q + 64 * NW - 1) / (64 * NW), SC_I = (SC_U + 64 * NW - 1) / (64 * NW);
    constexpr int DMA_PER_TILE = CODE_I + SC_I;
    static_assert(2 * DMA_PER_TILE < 64, "vmcnt range");
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;     // LDS byte address of the stages
    // Per load instruction: whether it fills A or B (uniform: the A part is a
    // whole number of instructions) and this lane's byte offset from the
    // start of the A or B codes (scales) at k = 0; 32 bits suffice (the
    // launcher checks).  Idle instructions read offset 0.
    uint32_t coff[CODE_I], soff[SC_I];
#pragma unroll
    for (int j = 0; j < CODE_I; ++j) {
      const int q0 = (j * NW + wave_u) * 64, q = q0 + lane;
      coff[j] = 0;
      if (q0 < CODE_Q) {
        const bool isa = q0 < BM * 4;
        const int qq = isa ? q : q - BM * 4, row = qq >> 2;
        const int logical = (qq & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
        const int64_t lim = isa ? g.M : g.N;
        int64_t gr = (isa ? m0 : n0) + row;
        gr = gr < lim ? gr : lim - 1;
        coff[j] = (uint32_t)(gr * kb + logical * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < SC_I; ++j) {
      const int u0 = (j * NW + wave_u) * 64, u = u0 + lane;
      soff[j] = 0;
      if (u0 < SC_U) {
        const bool isa = u0 < BM * 2;
        const int uu = isa ? u : u - BM * 2, row = uu >> 1;
        const int64_t lim = isa ? g.M : g.N;
        int64_t gr = (isa ? m0 : n0) + row;
        gr = gr < lim ? gr : lim - 1;
        soff[j] = (uint32_t)(gr * ks + (uu & 1) * 4);
      }
    }
    auto issue_tile = [&](int kt, int st) {
      const uint32_t sbase = lds0 + (uint32_t)(st * STAGE_D), spare = lds0 + 4u * STAGE_D;
      const int64_t kbyte0 = (int64_t)(kt0 + kt) * kRowBytes, ksc0 = (int64_t)(kt0 + kt) * 8;
#pragma unroll
      for (int j = 0; j < CODE_I; ++j) {
        const int q0 = (j * NW + wave_u) * 64;
        const bool real = q0 < CODE_Q, isa = q0 < BM * 4;
        const uint8_t *base = (isa || !real ? g.a_codes : g.b_codes) + kbyte0;
        lds_dma16(real ? sbase + (uint32_t)(q0 * 16) : spare, base, coff[j]);
      }
#pragma unroll
      for (int j = 0; j < SC_I; ++j) {
        const int u0 = (j * NW + wave_u) * 64;
        const bool real = u0 < SC_U, isa = u0 < BM * 2;
        const uint8_t *base = (isa || !real ? g.a_scales : g.b_scales) + ksc0;
        lds_dma4(real ? sbase + (uint32_t)((BM + BN) * kRowBytes + u0 * 4) : spare, base, soff[j]);
      }
    };
    auto stage = [&](int st) -> Stage {
      const uint8_t *base = lds + st * STAGE_D;
      return Stage{base, base + BM * kRowBytes, base + (BM + BN) * kRowBytes, base + (BM + BN) * kRowBytes + BM * 8};
    };
    issue_tile(0, 0);
    if (nk > 1) issue_tile(1, 1);
    if (nk > 2) issue_tile(2, 2);
    if (nk > 2) wait_vmcnt<2 * DMA_PER_TILE>();
    else if (nk > 1) wait_vmcnt<DMA_PER_TILE>();
    else wait_vmcnt<0>();
    __syncthreads();
    begin_tile(stage(0));
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 3 < nk) issue_tile(kt + 3, (kt + 3) % 4);
      const int ahead = (kt + 2 < nk) + (kt + 3 < nk);   // tiles issued after kt+1
      run_tile(stage(kt % 4), stage(kt + 1 < nk ? (kt + 1) % 4 : kt % 4), std::true_type{}, [&] {
        if (ahead == 2) wait_vmcnt<2 * DMA_PER_TILE>();     // tile kt+1 has landed
        else if (ahead == 1) wait_vmcnt<DMA_PER_TILE>();
        else wait_vmcnt<0>();
        __syncthreads();
      });
    }
    __syncthreads();           // the epilogue reuses the stages
  } else {
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load_global(kt + 1);
      const uint8_t *la = lds + cur * STAGE;
      const Stage t{la, la + A_BYTES, la + A_BYTES + B_BYTES, la + A_BYTES + B_BYTES + BM * 8};
      begin_tile(t);
      run_tile(t, t, std::false_type{}, [] {});
      if (kt + 1 < nk) store_lds(cur ^ 1);
      __syncthreads();
    }
  }

  if (S > 1) {
    // a split's raw accumulators, coalesced: element e of MFMA tile (i, j) of
    // thread tid at [((i * TN + j) * 16 + e) * NT + tid]
    float *my = g.part + ((tile - g.t_full) * S + sp) * (int64_t)(BM * BN);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) my[((i * TN + j) * 16 + e) * NT + tid] = acc[i][j][e];
    if (g.amax_parts && sp == 0 && tid == 0) g.amax_parts[tile] = 0u;   // the reduce folds into it
    return;
  }

  // ---- epilogue ---------------------------------------------------------------
  // C = alpha s_tA s_tB acc + (rank-r term) + beta_e E, one 32x32 tile at a
  // time.  The rank-r term runs as BF16 MFMA k-steps on the hi/lo split of
  // l_scale * L against R.  The workgroup first stages its L rows (as hi and
  // lo BF16) and R rows, all r <= 64 rank columns, in the LDS the main loop no
  // longer needs, with the loads in flight together; each tile then reads its
  // operands from LDS.
  // 32x32 accumulator layout: register e of lane l holds row
  // 8*(e/4) + 4*(l/32) + e%4, column l%32.
  const float scale = g.alpha * (*g.a_ts) * (*g.b_ts);
  // (buffer offsets are 32-bit: rows up to 32 apart within one base)
  const bool interior = m0 + BM <= g.M && n0 + BN <= g.N && 32 * g.N * 4 + BN * 4 < (int64_t(1) << 31);
  const int wm_u = wave_u / WN;     // wm, known uniform
  float amax = 0.0f;                // max |C| over this thread's stored elements
  const int nchunks = (g.r + 15) / 16;                    // <= 4 (r <= 64)
  const int lrs = (g.r <= 32 ? 32 : 64) + 8;              // 80 or 144 bytes: conflict-free 16-byte reads
  uint16_t *lhi = (uint16_t *)lds, *llo = lhi + BM * lrs, *rt = llo + BM * lrs;
  if (g.r > 0) {
    // 16-byte staging when rows are aligned (the usual case), element-wise otherwise
    const bool vec_l = g.r % 4 == 0 && ((uintptr_t)g.L & 15u) == 0;
    const bool vec_r_rows = g.r_sj == 1 && g.r_sn % 8 == 0 && ((uintptr_t)g.R & 15u) == 0;
    const bool vec_r_cols = g.r_sn == 1 && g.r_sj % 8 == 0 && g.N % 8 == 0 && ((uintptr_t)g.R & 15u) == 0;
    auto put_l = [&](int row, int jj, float x) {
      const uint32_t hb = float_to_bf16_rne_bits(x);
      lhi[row * lrs + jj] = (uint16_t)hb;
      llo[row * lrs + jj] = (uint16_t)float_to_bf16_rne_bits(x - bf16_bits_to_float(hb));
    };
    for (int c0 = 0; c0 < g.r; c0 += 32) {
      if (vec_l) {
        // BM rows x 8 four-column groups, in batches of 4 loads per thread
        constexpr int NL = BM * 8 / NT, NB = NL < 4 ? NL : 4;
        static_assert(NL % NB == 0, "uneven rank-r staging");
#pragma unroll
        for (int q0 = 0; q0 < NL; q0 += NB) {
          float4 v[NB];
#pragma unroll
          for (int q = 0; q < NB; ++q) {
            const int e = tid + (q0 + q) * NT, row = e >> 3, j = c0 + (e & 7) * 4;
            const int64_t m = m0 + row;
            v[q] = (m < g.M && j < g.r) ? *(const float4 *)(g.L + m * g.r + j) : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
          for (int q = 0; q < NB; ++q) {
            const int e = tid + (q0 + q) * NT, row = e >> 3, jj = c0 + (e & 7) * 4;
            put_l(row, jj + 0, v[q].x * g.l_scale);
            put_l(row, jj + 1, v[q].y * g.l_scale);
            put_l(row, jj + 2, v[q].z * g.l_scale);
            put_l(row, jj + 3, v[q].w * g.l_scale);
          }
        }
      } else {
        for (int e = tid; e < BM * 32; e += NT) {
          const int row = e >> 5, jj = c0 + (e & 31);
          const int64_t m = m0 + row;
          put_l(row, jj, (m < g.M && jj < g.r) ? g.L[m * g.r + jj] * g.l_scale : 0.0f);
        }
      }
      // R(n, j) = R[n r_sn + j r_sj], staged as rt[n][j], one 16-byte chunk at a time
      constexpr int NR = BN * 4 / NT;
      static_assert(BN * 4 % NT == 0, "uneven rank-r staging");
      if (vec_r_rows) {
#pragma unroll 1
        for (int q = 0; q < NR; ++q) {
          const int e = tid + q * NT, row = e >> 2, jj = c0 + (e & 3) * 8;
          const int64_t n = n0 + row;
          *(uint4 *)(rt + row * lrs + jj) =
              (n < g.N && jj < g.r) ? *(const uint4 *)(g.R + n * g.r_sn + jj) : make_uint4(0, 0, 0, 0);
        }
      } else if (vec_r_cols) {
        // eight consecutive n for one rank column j, written transposed
#pragma unroll 1
        for (int q = 0; q < NR; ++q) {
          const int e = tid + q * NT, jj = c0 + e / (BN / 8), n8 = (e % (BN / 8)) * 8;
          const int64_t n = n0 + n8;
          const uint4 v = (n < g.N && jj < g.r) ? *(const uint4 *)(g.R + (int64_t)jj * g.r_sj + n) : make_uint4(0, 0, 0, 0);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            rt[(n8 + 2 * t) * lrs + jj] = (uint16_t)(w[t] & 0xFFFFu);
            rt[(n8 + 2 * t + 1) * lrs + jj] = (uint16_t)(w[t] >> 16);
          }
        }
      } else {
        for (int e = tid; e < BN * 32; e += NT) {
          const int row = e >> 5, jj = c0 + (e & 31);
          const int64_t n = n0 + row;
          rt[row * lrs + jj] = (n < g.N && jj < g.r) ? g.R[n * g.r_sn + (int64_t)jj * g.r_sj] : (uint16_t)0;
        }
      }
    }
    __syncthreads();
  }
  // E for a whole 32x32 accumulator tile (16 values per lane) is loaded one
  // tile ahead, so that its latency overlaps the previous tile's stores
  // instead of stalling every four rows.  Tiles are disjoint, so loading E of
  // tile q+1 before storing C of tile q is correct even when C and E are the
  // same buffer.
  const bool e_pipe = g.E != nullptr && interior;
  float ebuf[2][16];
  auto load_e = [&](int i, int j, float *dst) {
    const int64_t base = (m0 + wm_u * TM * 32 + i * 32) * g.N + n0;
    const int nrec = (int)((g.M * g.N - base) * 4 < 0x7FFFFFFF ? (g.M * g.N - base) * 4 : 0x7FFFFFFF);
    const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((float *)g.E + base, 0, nrec, kBufferWord3);
    const int loff = (4 * h * (int)g.N + wn * TN * 32 + j * 32 + l32) * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      dst[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, loff, (8 * (e >> 2) + (e & 3)) * (int)g.N * 4, 0));
  };
  if (e_pipe) load_e(0, 0, ebuf[0]);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int arow = wm * TM * 32 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int brow = wn * TN * 32 + j * 32 + l32;
      const int q = i * TN + j;
      if (e_pipe && q + 1 < TM * TN) load_e((q + 1) / TN, (q + 1) % TN, ebuf[(q + 1) & 1]);
      floatx16_t t = acc[i][j] * scale;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < nchunks) {
          const bf16x8_t ah = *(const bf16x8_t *)(lhi + arow * lrs + c * 16 + 8 * h);
          const bf16x8_t al = *(const bf16x8_t *)(llo + arow * lrs + c * 16 + 8 * h);
          const bf16x8_t rv = *(const bf16x8_t *)(rt + brow * lrs + c * 16 + 8 * h);
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, rv, t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, rv, t, 0, 0, 0);
        }
      }
      float vv[16];   // the stored values (for the mirrored store of a symmetric C)
      if (interior) {
        // Whole tile in range: buffer stores (and loads of E) from a uniform
        // base at row m0 + wm*TM*32 + i*32, column n0, with the row offset of
        // register e in a scalar register and this lane's offset (rows 4h..,
        // column l32) in a vector register: no per-element address work.
        const int64_t base = (m0 + wm_u * TM * 32 + i * 32) * g.N + n0;
        // (with Ct the record count is 0: the hardware drops these stores).
        // C goes out with the non-temporal policy: an output of 100-268 MB
        // would otherwise displace the operands that the kernels after it
        // read from the caches.
        const int nrec = g.Ct ? 0 : (int)((g.M * g.N - base) * 4 < 0x7FFFFFFF ? (g.M * g.N - base) * 4 : 0x7FFFFFFF);
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(g.C + base, 0, nrec, kBufferWord3);
        const int loff = (4 * h * (int)g.N + wn * TN * 32 + j * 32 + l32) * 4;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int soff = (8 * (e >> 2) + (e & 3)) * (int)g.N * 4;
          if (e_pipe) t[e] += g.beta_e * ebuf[q & 1][e];
          const float v = t[e];
          if (g.amax_parts) amax = fmaxf(amax, fabsf(v));
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, loff, soff, kStoreNT);
          vv[e] = v;
        }
      } else {
        const int64_t n = n0 + brow;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + wm * TM * 32 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          vv[e] = 0.0f;
          if (m < g.M && n < g.N) {
            float v = t[e];
            if (g.E) v += g.beta_e * g.E[m * g.N + n];
            if (!g.Ct) g.C[m * g.N + n] = v;   // (non-interior tiles only)
            if (g.amax_parts) amax = fmaxf(amax, fabsf(v));
            vv[e] = v;
          }
        }
      }
      // The transposed store: C^T into Ct, or a symmetric C's mirror image.
      // This lane's column n becomes a row, its rows m (four runs of four)
      // become 16-byte pieces of that row (M % 4 == 0; a symmetric C is
      // square).
      float *ct = g.Ct ? g.Ct : ((g.sym && g.mirror && tile_m != tile_n) ? g.C : nullptr);
      if (ct) {
        const int64_t n = n0 + brow;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t m = m0 + wm * TM * 32 + i * 32 + 8 * q + 4 * h;
          if (n < g.N && m < g.M)
            *(float4 *)(ct + n * g.M + m) = make_float4(vv[4 * q], vv[4 * q + 1], vv[4 * q + 2], vv[4 * q + 3]);
        }
      }
    }
  }
  if (g.amax_parts) {
    // workgroup max (non-negative floats order as their bit patterns)
    __shared__ uint32_t wmax[NT / 64];
    uint32_t u = __builtin_bit_cast(uint32_t, amax);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t v = (uint32_t)__shfl_xor((int)u, o);
      u = u > v ? u : v;
    }
    if (lane == 0) wmax[wave] = u;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = wmax[0];
#pragma unroll
      for (int w = 1; w < NT / 64; ++w) m = m > wmax[w] ? m : wmax[w];
      g.amax_parts[tile] = m;
    }
  }
}

// Adds the split partials of tiles t_full.. in split order and runs the
// epilogue: C = alpha s_tA s_tB sum + beta_e E (no rank-r term), mirrored
// for a symmetric C, and folds each tile's max |C| into amax_parts (which the
// tile's first split set to 0).  One thread per four consecutive partials:
// in accumulator order those are four adjacent lanes of one GEMM thread
// register, i.e. C[m][n .. n+3]; kSplitReduceWg of them per tile.
constexpr int kSplitReduceThreads = 256;
template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(kSplitReduceThreads) void split_reduce_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int WG_PER_TILE = BM * BN / 4 / kSplitReduceThreads;
  static_assert(BM * BN % (4 * kSplitReduceThreads) == 0 && NT % 64 == 0, "reduce mapping");
  const int64_t slot = blockIdx.x / WG_PER_TILE, tile = g.t_full + slot, S = g.s_tail;
  const int64_t tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int64_t tile_m, tile_n;
  if (g.sym) {
    int64_t t = tile, tm = 0;
    while (t >= tiles_n - tm) { t -= tiles_n - tm; ++tm; }
    tile_m = tm;
    tile_n = tm + t;
  } else {
    tile_coords(tile, tiles_m, tiles_n, &tile_m, &tile_n);
  }
  // flat partial index f = ((i * TN + j) * 16 + e) * NT + t  (t: GEMM thread)
  const int f = ((int)(blockIdx.x % WG_PER_TILE) * kSplitReduceThreads + (int)threadIdx.x) * 4;
  const int t = f % NT, ije = f / NT, e = ije % 16, i = ije / 16 / TN, j = ije / 16 % TN;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave / WN, wn = wave % WN, h = lane >> 5, l32 = lane & 31;
  const int64_t m = tile_m * BM + wm * TM * 32 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
  const int64_t n = tile_n * BN + wn * TN * 32 + j * 32 + l32;     // .. n + 3
  const float *base = g.part + slot * S * (int64_t)(BM * BN) + f;
  float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int64_t q = 0; q < S; ++q) {          // in split order
    const float4 p = *(const float4 *)(base + q * (BM * BN));
    sum.x += p.x; sum.y += p.y; sum.z += p.z; sum.w += p.w;
  }
  const float scale = g.alpha * (*g.a_ts) * (*g.b_ts);
  float v[4] = {scale * sum.x, scale * sum.y, scale * sum.z, scale * sum.w};
  float amax = 0.0f;
  if (m < g.M) {
    const int64_t o = m * g.N + n;
    const bool vec = n + 3 < g.N && (((uintptr_t)(g.C + o) | (g.E ? (uintptr_t)(g.E + o) : 0)) & 15u) == 0;
    if (vec) {
      if (g.E) {
        const float4 ev = *(const float4 *)(g.E + o);
        v[0] += g.beta_e * ev.x; v[1] += g.beta_e * ev.y; v[2] += g.beta_e * ev.z; v[3] += g.beta_e * ev.w;
      }
      *(float4 *)(g.C + o) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
      for (int c = 0; c < 4; ++c) amax = fmaxf(amax, fabsf(v[c]));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n + c < g.N) {
          if (g.E) v[c] += g.beta_e * g.E[o + c];
          g.C[o + c] = v[c];
          amax = fmaxf(amax, fabsf(v[c]));
        }
    }
    if (g.sym && g.mirror && tile_m != tile_n) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n + c < g.M && m < g.N) g.C[(n + c) * g.N + m] = v[c];
    }
  }
  if (g.amax_parts) {
    __shared__ uint32_t wmax[kSplitReduceThreads / 64];
    uint32_t u = __builtin_bit_cast(uint32_t, amax);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t w = (uint32_t)__shfl_xor((int)u, o);
      u = u > w ? u : w;
    }
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = u;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mx = wmax[0];
#pragma unroll
      for (int w = 1; w < kSplitReduceThreads / 64; ++w) mx = mx > wmax[w] ? mx : wmax[w];
      // non-negative floats order as their bit patterns
      atomicMax(g.amax_parts + tile, mx);
    }
  }
}

template <int WM, int WN, int TM, int TN>
fs4_status launch_cfg(GemmArgs g, int64_t tiles, int64_t t_full, int s_tail, hipStream_t s, int *nwg) {
  if (nwg) *nwg = (int)tiles;
  g.t_full = t_full;
  g.s_tail = s_tail;
  const int64_t wgs = t_full + (tiles - t_full) * s_tail;
  // the direct-load path addresses operands with 32-bit per-lane offsets
  const int64_t rows = g.M > g.N ? g.M : g.N;
  if (g.K > 0 && g.K % kBK == 0 && rows * (g.K / 2) < (int64_t(1) << 32))
    gemm_nt_kernel<WM, WN, TM, TN, true><<<(unsigned)wgs, WM * WN * 64, 0, s>>>(g);
  else
    gemm_nt_kernel<WM, WN, TM, TN, false><<<(unsigned)wgs, WM * WN * 64, 0, s>>>(g);
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;
  if (s_tail > 1) {
    constexpr int WG_PER_TILE = WM * TM * 32 * WN * TN * 32 / 4 / kSplitReduceThreads;
    split_reduce_kernel<WM, WN, TM, TN>
        <<<(unsigned)((tiles - t_full) * WG_PER_TILE), kSplitReduceThreads, 0, s>>>(g);
    if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;
  }
  return FS4_OK;
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool sym, bool can_split, int64_t split_floats) {
  // Plan: the tile shape and work split with the least estimated time.  One
  // k-tile (128 deep) of a 256 x 256 tile takes ~3.9 us on a CU (measured on
  // MI355X at the 3B shapes); the configurations' relative MFMA throughput:
  //   256 x 256, 8 waves of 128 x 64 (two per SIMD)   1.00
  //   256 x 192, 4 waves of 128 x 96 (one per SIMD)   0.83
  //   128 x 128, 4 waves of 64 x 64                   0.70
  // Tiles run in rounds of 256 workgroups (one per CU), and whole rounds
  // matter: 384 tiles of 256 x 256 (an 8192 x 3072 output) leave half the
  // chip idle in the second round, 512 tiles of 256 x 192 do not.  A
  // symmetric product counts the upper triangle's tiles (square tiles only).
  // With a split workspace (and no rank-r term) the tiles of a last round
  // that fills at most half the chip are split along k so that it fills the
  // chip, for the price of writing and re-reading fp32 partials (counted at
  // 4 TB/s) and a reduce launch (~4 us).
  const int64_t nk_all = (K + kBK - 1) / kBK;
  can_split = can_split && K > 0 && K % kBK == 0;
  auto plan = [&](int cfg, int64_t bm, int64_t bn, double rate) {
    GemmPlan p{cfg, (int)bm, (int)bn, 0, 0, 1, 0.0};
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    p.tiles = sym ? tm * (tm + 1) / 2 : tm * tn;
    p.t_full = p.tiles;
    const double tk = 3.9e-6 * (double)(bm * bn) / 65536.0 / rate;
    p.cost = (double)((p.tiles + 255) / 256) * (double)nk_all * tk;
    const int64_t tail = p.tiles % 256;
    if (can_split && tail > 0 && tail <= 128) {
      int st = (int)(256 / tail);
      if (st > 8) st = 8;
      // every split at least two k-tiles, and none empty
      while (st > 1 && ((nk_all + st - 1) / st < 2 || (nk_all + st - 1) / st * (st - 1) >= nk_all)) --st;
      if (st > 1 && (double)tail * st * bm * bn <= (double)split_floats) {
        const double bytes = 2.0 * (double)tail * st * (double)(bm * bn) * 4.0;
        const double c = (double)(p.tiles / 256) * (double)nk_all * tk +
                         (double)((nk_all + st - 1) / st) * tk + bytes / 4e12 + 4e-6;
        if (c < p.cost) {
          p.cost = c;
          p.t_full = p.tiles - tail;
          p.s_tail = st;
        }
      }
    }
    return p;
  };
  GemmPlan best = plan(0, 256, 256, 1.0);
  if (!sym) {
    const GemmPlan p1 = plan(1, 256, 192, 0.83);
    if (p1.cost < best.cost) best = p1;
  }
  const GemmPlan p2 = plan(2, 128, 128, 0.70);
  if (p2.cost < best.cost) best = p2;
  return best;
}

fs4_status launch_gemm_nt(const fs4_nvfp4 &A, const fs4_nvfp4 &B, float alpha, const float *E,
                          float beta_e, float *C, const LowRankEpilogue &lr, hipStream_t s,
                          uint32_t *amax_parts, int *nwg, bool sym, float *split_ws,
                          int64_t split_floats, bool mirror, float *Ct) {
  GemmArgs g;
  g.mirror = mirror ? 1 : 0;
  g.Ct = Ct;
  g.t_full = 0;
  g.s_tail = 1;
  g.part = split_ws;
  g.amax_parts = amax_parts;
  if (nwg) *nwg = 0;
  g.a_codes = A.codes; g.a_scales = A.scales; g.a_ts = A.tscale;
  g.b_codes = B.codes; g.b_scales = B.scales; g.b_ts = B.tscale;
  g.M = A.rows; g.N = B.rows; g.K = A.cols;
  g.alpha = alpha; g.beta_e = beta_e; g.E = E; g.C = C;
  g.L = lr.L; g.R = lr.R; g.r = lr.L ? lr.r : 0; g.l_scale = lr.l_scale;
  g.r_sn = lr.r_sn; g.r_sj = lr.r_sj;
  // a symmetric product (B the same view as A) stores only the upper
  // triangle's tiles, each at both positions; not with a rank-r term
  g.sym = sym && A.codes == B.codes && A.scales == B.scales && g.M == g.N && g.r == 0 ? 1 : 0;
  if (g.M == 0 || g.N == 0) return FS4_OK;
  if (Ct && (g.sym || g.M % 4)) return FS4_ERR_ARG;
  const GemmPlan best = plan_gemm(g.M, g.N, g.K, g.sym != 0, split_ws && g.r == 0 && !Ct, split_floats);
  if (best.cfg == 0) return launch_cfg<2, 4, 4, 2>(g, best.tiles, best.t_full, best.s_tail, s, nwg);
  if (best.cfg == 1) return launch_cfg<2, 2, 4, 3>(g, best.tiles, best.t_full, best.s_tail, s, nwg);
  return launch_cfg<2, 2, 2, 2>(g, best.tiles, best.t_full, best.s_tail, s, nwg);
}

}  // namespace fs4
