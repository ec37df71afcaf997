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
// The exact block encoding (tables, scale codes, the bracketed fast path) is
// in nvfp4_encode.h.
#include "nvfp4_encode.h"

namespace fs4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
// persistent workgroups of the encode pass (multiples of 128, whole
// super-tiles per XCD).  Fewer than fit on the CUs at once (6 per CU for
// bf16, 4 for fp32): measured on MI355X, 4 (bf16) and 3 (fp32) per CU run
// 3-11% faster (bf16 8192^2: 89 against 100 us; 4096^2: 27.6 against 28.5;
// fp32 3072^2: 24.7 against 26.4), ties elsewhere
constexpr int kEncodeGridBf16 = 1024, kEncodeGridF32 = 768;
constexpr int kAmaxUnroll = 4;

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

template <int NT>
__device__ inline uint32_t block_max_u32_n(uint32_t v, uint32_t *red) {
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = r > red[i] ? r : red[i];
  __syncthreads();
  return r;
}
__device__ inline uint32_t block_max_u32(uint32_t v, uint32_t *red) { return block_max_u32_n<kThreads>(v, red); }

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

// One 64 x 64 tile in registers: bf16 takes two 16-byte words per lane, fp32
// four (zeros outside the tensor).
template <bool BF16>
struct TileRegs {
  static constexpr int kVec = BF16 ? 2 : 4;
  uint4 v[kVec];
};

// Loads are issued for every lane (addresses clamped into the tensor) and the
// padding is zeroed when the tile is staged, so no lane-dependent branch
// surrounds a load.
// A workgroup past its last tile (valid == false) reads the tensor's first
// 16 bytes instead, so the number of loads in flight never depends on the
// data and the waits stay exact.
template <bool BF16>
__device__ inline void tile_gload(const void *x, int64_t rows, int64_t cols, int64_t r0, int64_t c0,
                                  bool valid, TileRegs<BF16> &g) {
  constexpr int kPerRow = BF16 ? 8 : 16;     // 16-byte words per 64-element tile row
  constexpr int kElems = BF16 ? 8 : 4;       // elements per word
  const char *xb = (const char *)x;
  const int64_t esz = BF16 ? 2 : 4;
#pragma unroll
  for (int p = 0; p < TileRegs<BF16>::kVec; ++p) {
    const int idx = threadIdx.x + p * kThreads;
    const int r = idx / kPerRow, ch = idx % kPerRow;
    int64_t gr = r0 + r, gc = c0 + ch * kElems;
    gr = gr < rows ? gr : rows - 1;
    gc = gc < cols ? gc : cols - kElems;
    const int64_t off = valid ? (gr * cols + gc) * esz : 0;
    g.v[p] = *(const uint4 *)(xb + off);
  }
}

// With CLIP, magnitudes above clipv are clipped to it (signs kept).
template <bool BF16, bool CLIP = false>
__device__ inline void tile_store(const TileRegs<BF16> &g, int64_t rows, int64_t cols, int64_t r0,
                                  int64_t c0, float (*tile)[kTile + 1], float clipv = 0.0f) {
  constexpr int kPerRow = BF16 ? 8 : 16;
  constexpr int kElems = BF16 ? 8 : 4;
#pragma unroll
  for (int p = 0; p < TileRegs<BF16>::kVec; ++p) {
    const int idx = threadIdx.x + p * kThreads;
    const int r = idx / kPerRow, ch = idx % kPerRow;
    const bool in = r0 + r < rows && c0 + ch * kElems < cols;
    const uint32_t w[4] = {in ? g.v[p].x : 0u, in ? g.v[p].y : 0u, in ? g.v[p].z : 0u,
                           in ? g.v[p].w : 0u};
    if constexpr (BF16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo = bf16_bits_to_float(w[j] & 0xFFFFu), hi = bf16_bits_to_float(w[j] >> 16);
        if constexpr (CLIP) {
          lo = __builtin_copysignf(__builtin_fminf(__builtin_fabsf(lo), clipv), lo);
          hi = __builtin_copysignf(__builtin_fminf(__builtin_fabsf(hi), clipv), hi);
        }
        tile[r][ch * 8 + 2 * j] = lo;
        tile[r][ch * 8 + 2 * j + 1] = hi;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = __builtin_bit_cast(float, w[j]);
        if constexpr (CLIP) v = __builtin_copysignf(__builtin_fminf(__builtin_fabsf(v), clipv), v);
        tile[r][ch * 4 + j] = v;
      }
    }
  }
}

// Work order.  Tiles are grouped 4 x 4 into 256 x 256 super-tiles; the 16
// tiles of a super-tile go to 16 workgroups of one XCD (consecutive
// dispatches land on different XCDs, round robin over 8), so the partial
// 128-byte lines of both code layouts that neighbouring tiles share are
// completed in one L2.
struct TileOrder {
  // The grid size is a multiple of 16, so a workgroup keeps its position
  // (sub_r, sub_c) inside the super-tile and its super-tile index advances
  // by grid / 16 per step; all of it is wave-uniform 32-bit arithmetic.
  int tiles_r, tiles_c, sct, n_st;   // tile grid, super-tile columns and count
  int sub_r, sub_c;                  // this workgroup's tile inside a super-tile
  int d_r, d_c;                      // per-step advance in super-tile rows / columns
  int upper;                         // only tiles on or above the diagonal
  __device__ TileOrder(int64_t rows, int64_t cols, int upper_only) {
    upper = upper_only;
    tiles_r = (int)((rows + kTile - 1) / kTile);
    tiles_c = (int)((cols + kTile - 1) / kTile);
    sct = (tiles_c + 3) / 4;
    n_st = ((tiles_r + 3) / 4) * sct;
    const int g = (int)gridDim.x, b = (int)blockIdx.x;
    const int v = (g % 8 == 0) ? (b % 8) * (g / 8) + b / 8 : b;   // XCD-major numbering
    sub_r = (v & 15) >> 2;
    sub_c = v & 3;
    d_r = (g / 16) / sct;
    d_c = (g / 16) % sct;
  }
  // Position: super-tile (sr, sc); returns whether a tile is left, moving
  // (sr, sc) forward to the first super-tile whose sub-tile lies inside.
  __device__ bool seek(int &sr, int &sc) const {
    while (sr * sct + sc < n_st) {
      if (sr * 4 + sub_r < tiles_r && sc * 4 + sub_c < tiles_c && (!upper || sr * 4 + sub_r <= sc * 4 + sub_c))
        return true;
      advance(sr, sc);
    }
    return false;
  }
  __device__ void advance(int &sr, int &sc) const {
    sr += d_r;
    sc += d_c;
    if (sc >= sct) {
      sc -= sct;
      ++sr;
    }
  }
  __device__ void start(int &sr, int &sc) const {
    const int g = (int)gridDim.x, b = (int)blockIdx.x;
    const int v = (g % 8 == 0) ? (b % 8) * (g / 8) + b / 8 : b;
    sr = (v >> 4) / sct;
    sc = (v >> 4) % sct;
  }
  __device__ int64_t r0(int sr) const { return (int64_t)(sr * 4 + sub_r) * kTile; }
  __device__ int64_t c0(int sc) const { return (int64_t)(sc * 4 + sub_c) * kTile; }
};

// With CLIP, *clip replaces the tensor amax and every element is clipped to
// magnitude *clip before it is encoded (the partials are not read).  With
// upper_only (a symmetric square x, cv the same view as rv), only the tiles
// on or above the diagonal are read: a tile's column blocks are the row
// blocks of its mirror image, and go there.
template <bool BF16, bool ROW, bool COL, bool CLIP = false>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void *__restrict__ x, int64_t rows,
                                                            int64_t cols,
                                                            const uint32_t *__restrict__ partials,
                                                            int npart, fs4_nvfp4 rv, fs4_nvfp4 cv,
                                                            const float *clip = nullptr, int upper_only = 0) {
  __shared__ float tile[kTile][kTile + 1];
  __shared__ Tables tab;
  __shared__ uint32_t red[kThreads / 64];
  // The amax partials (every workgroup reduces them itself) are loaded first
  // and the first two tiles' loads are issued behind them, so one memory round
  // trip covers both; the tables are built while the tiles are in flight.
  constexpr int kPrePart = 4;
  uint32_t pm[kPrePart] = {};
  float clipv = 0.0f;
  if constexpr (CLIP) {
    clipv = *clip;
  } else {
#pragma unroll
    for (int u = 0; u < kPrePart; ++u) {
      const int i = threadIdx.x + u * kThreads;
      pm[u] = partials[i < npart ? i : npart - 1];   // npart >= 1; a repeat leaves the max unchanged
    }
  }
  const TileOrder order(rows, cols, upper_only);
  int sr, sc;
  order.start(sr, sc);
  int have = order.seek(sr, sc) ? 1 : 0;   // int flags stay in scalar registers
  int sr1 = sr, sc1 = sc;
  if (have) order.advance(sr1, sc1);
  int have1 = (have && order.seek(sr1, sc1)) ? 1 : 0;
  TileRegs<BF16> g0, g1;
  tile_gload<BF16>(x, rows, cols, order.r0(sr), order.c0(sc), have != 0, g0);
  tile_gload<BF16>(x, rows, cols, order.r0(sr1), order.c0(sc1), have1 != 0, g1);
  float amax;
  if constexpr (CLIP) {
    amax = clipv;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < kPrePart; ++u) m = m > pm[u] ? m : pm[u];
    for (int i = threadIdx.x + kPrePart * kThreads; i < npart; i += kThreads)
      m = m > partials[i] ? m : partials[i];
    m = block_max_u32(m, red);
    amax = __builtin_bit_cast(float, m);
  }
  const float s_t = (float)((double)amax / kTensorDiv);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (ROW) *rv.tscale = s_t;
    if (COL) *cv.tscale = s_t;
  }
  build_tables_n<kThreads>(tab, s_t);
  // 1/(6 s_t) only seeds the scale-code estimate; the tables make it exact
  const float inv6st = s_t > 0.0f ? (float)(1.0 / (6.0 * (double)s_t)) : 0.0f;   // may be inf
  const bool inv_finite = inv6st < __builtin_huge_valf();
  tile_store<BF16, CLIP>(g0, rows, cols, order.r0(sr), order.c0(sc), tile, clipv);
  __syncthreads();

  const int t = threadIdx.x;
  const int line = t >> 2, blk = t & 3;     // four lanes per row (or column) of the tile
  // One step: the tile in LDS is (sr, sc); `nxt` holds the loads of the
  // following tile (sr1, sc1); `ahead` is free and receives the tile after
  // that.  The encode runs from LDS while both are in flight; after a barrier
  // `nxt` replaces the tile in LDS (its wait leaves the loads just issued into
  // `ahead` outstanding) and this tile's codes are stored.
  auto step = [&](TileRegs<BF16> &ahead, const TileRegs<BF16> &nxt) {
    const int64_t r0 = order.r0(sr), c0 = order.c0(sc);
    int sr2 = sr1, sc2 = sc1;
    if (have1) order.advance(sr2, sc2);
    const int have2 = (have1 && order.seek(sr2, sc2)) ? 1 : 0;
    tile_gload<BF16>(x, rows, cols, order.r0(sr2), order.c0(sc2), have2 != 0, ahead);
    // zero padding outside the tensor encodes harmlessly; only stores are masked
    uint2 pr = make_uint2(0, 0), pc = make_uint2(0, 0);
    uint32_t sbr = 0, sbc = 0;
    if (ROW) {
      const float *src = &tile[line][blk * kBlock];
      sbr = encode16([&](int i) { return src[i]; }, inv6st, inv_finite, tab, pr);
    }
    if (COL) {
      const float *src = &tile[blk * kBlock][line];
      sbc = encode16([&](int i) { return src[i * (kTile + 1)]; }, inv6st, inv_finite, tab, pc);
    }
    __syncthreads();
    tile_store<BF16, CLIP>(nxt, rows, cols, order.r0(sr1), order.c0(sc1), tile, clipv);   // unread past the last tile
    if (ROW) {
      const int64_t gr = r0 + line, gc = c0 + blk * kBlock;
      if (gr < rows && gc < cols) {
        *(uint2 *)(rv.codes + gr * (cols / 2) + gc / 2) = pr;
        rv.scales[gr * (cols / kBlock) + gc / kBlock] = (uint8_t)sbr;
      }
    }
    if (COL) {
      const int64_t gc = c0 + line, gr = r0 + blk * kBlock;
      if (gc < cols && gr < rows) {
        *(uint2 *)(cv.codes + gc * (rows / 2) + gr / 2) = pc;
        cv.scales[gc * (rows / kBlock) + gr / kBlock] = (uint8_t)sbc;
      }
    }
    __syncthreads();
    have = have1; sr = sr1; sc = sc1;
    have1 = have2; sr1 = sr2; sc1 = sc2;
  };
  while (have) {
    step(g0, g1);
    if (!have) break;
    step(g1, g0);
  }
}

__global__ void write_zero_scale_kernel(float *a, float *b) {
  if (a) *a = 0.0f;
  if (b) *b = 0.0f;
}

}  // namespace

size_t quantize_ws_bytes() { return kAmaxPartials * sizeof(uint32_t); }

fs4_status launch_quantize_encode(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                                  const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise,
                                  const uint32_t *partials, int npart, hipStream_t s,
                                  const float *clip, bool upper_only) {
  const fs4_nvfp4 none = {nullptr, nullptr, nullptr, 0, 0};
  if (upper_only && (rows != cols || !rowwise || colwise || clip)) return FS4_ERR_ARG;
  if (!clip && (!partials || npart < 1)) return FS4_ERR_ARG;
  const fs4_nvfp4 rv = rowwise ? *rowwise : none;
  // a square view's column blocks land at its mirrored row blocks: the same
  // addresses as in a column-wise view of the same shape
  const fs4_nvfp4 cv = upper_only ? *rowwise : (colwise ? *colwise : none);
  const bool bf16 = dt == FS4_BF16;
  // one workgroup per tile slot (4 x 4 tiles per super-tile), at most the cap
  const int64_t slots = ((rows + 4 * kTile - 1) / (4 * kTile)) * ((cols + 4 * kTile - 1) / (4 * kTile)) * 16;
  const int64_t cap = bf16 ? kEncodeGridBf16 : kEncodeGridF32;
  const unsigned grid = (unsigned)(slots < cap ? slots : cap);   // multiple of 16
  static_assert(kEncodeGridBf16 % 128 == 0 && kEncodeGridF32 % 128 == 0,
                "the tile walk needs a multiple of 16, whole super-tiles per XCD a multiple of 128");
  const bool row = rv.codes != nullptr, col = cv.codes != nullptr;
#define FS4_QK(B, R, C)                                                                            \
  do {                                                                                             \
    if (clip)                                                                                      \
      quantize_kernel<B, R, C, true><<<grid, kThreads, 0, s>>>(x, rows, cols, partials, npart, rv, cv, clip); \
    else                                                                                           \
      quantize_kernel<B, R, C><<<grid, kThreads, 0, s>>>(x, rows, cols, partials, npart, rv, cv, nullptr, \
                                                          upper_only ? 1 : 0);                     \
  } while (0)
  if (bf16) {
    if (row && col) FS4_QK(true, true, true);
    else if (row) FS4_QK(true, true, false);
    else FS4_QK(true, false, true);
  } else {
    if (row && col) FS4_QK(false, true, true);
    else if (row) FS4_QK(false, true, false);
    else FS4_QK(false, false, true);
  }
#undef FS4_QK
  return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
}

fs4_status launch_quantize(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                           const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise, void *ws,
                           hipStream_t s) {
  if (rows == 0 || cols == 0) {
    write_zero_scale_kernel<<<1, 1, 0, s>>>(rowwise ? rowwise->tscale : nullptr,
                                             colwise ? colwise->tscale : nullptr);
    return hipGetLastError() == hipSuccess ? FS4_OK : FS4_ERR_HIP;
  }
  const bool bf16 = dt == FS4_BF16;
  const int64_t n = rows * cols;
  const int64_t nvec = n / (bf16 ? 8 : 4);
  const int64_t g = (nvec + kThreads * kAmaxUnroll * 2 - 1) / (kThreads * kAmaxUnroll * 2);
  const int npart = (int)(g < 1 ? 1 : (g > kAmaxPartials ? kAmaxPartials : g));
  uint32_t *partials = (uint32_t *)ws;
  if (bf16) amax_partial_kernel<true><<<npart, kThreads, 0, s>>>((const uint4 *)x, nvec, partials);
  else amax_partial_kernel<false><<<npart, kThreads, 0, s>>>((const uint4 *)x, nvec, partials);
  if (hipGetLastError() != hipSuccess) return FS4_ERR_HIP;
  return launch_quantize_encode(x, dt, rows, cols, rowwise, colwise, partials, npart, s);
}

}  // namespace fs4
