// Grouped expert GEMMs in bf16 on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// float32 accumulation), with the SwiGLU forward and backward fused into the
// epilogues.  These are the "expert FFN compute" that the expert-parallel
// overlap pages hide the token exchange behind (skill card page 1, "What it
// is"), split into activation gradient (dgrad, D) and weight gradient (wgrad,
// W) as the 1F1B note describes (page 2, "MoE 1F1B overlap").
//
// Structure shared by every kernel here:
//  * block tile BM x BN, K step 64, operands staged through LDS in two stages
//    (global -> registers for step k+1 while the matrix cores work on step k);
//  * LDS tiles are [rows][64] bf16 with the 16-byte chunk index XOR-swizzled
//    by the row so that the matrix-core fragment reads hit distinct banks;
//  * an operand that is contiguous along K is copied 16 bytes at a time; an
//    operand contiguous along M/N (weights in dgrad, activations in wgrad) is
//    read as 8 (k) x 4 (m) blocks and transposed in registers on its way to LDS;
//  * the block id is remapped so that consecutive tiles (same expert, same
//    rows) land on the same XCD and share its L2.
// Row-grouped GEMMs (fwd, dgrad) take their (expert, M-tile) from the dispatch
// plan's tile_offsets (tiles of kTileM rows); the grid is sized for the worst
// case on the host and surplus blocks exit.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 64;

// Element offset of 16-byte chunk `ch` (0..7) of row `row` of an LDS tile.
__device__ __forceinline__ int lds_off(int row, int ch) {
  const int s = (row & 7) ^ ((row >> 3) & 1);
  return row * BK + ((ch ^ s) << 3);
}

// Hardware places block b on XCD b % 8.  Map so that each XCD works on a
// contiguous range of logical tile ids.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int xcd = bid & 7, lid = bid >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + lid;
}

// Operand contiguous along K: R rows x 64 k per stage, 16-byte chunks.
// row_ptr(r) gives the address of element k = 0 of tile row r, or nullptr for
// a row outside the matrix (loaded as zeros).  K must be a multiple of 64.
template <int R, int NT>
struct LoadK {
  static constexpr int CH = R * 8 / NT;
  static_assert(CH >= 1 && (R * 8) % NT == 0, "tile/threads mismatch");
  const uint16_t* src[CH];
  int dst[CH];
  uint4 v[CH];
  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr row_ptr, int tid) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int q = c * NT + tid, row = q >> 3, ch = q & 7;
      const uint16_t* p = row_ptr(row);
      src[c] = p ? p + ch * 8 : nullptr;
      dst[c] = lds_off(row, ch);
    }
  }
  __device__ __forceinline__ void load(int k0, int /*k_end*/) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
      v[c] = src[c] ? *(const uint4*)(src[c] + k0) : make_uint4(0u, 0u, 0u, 0u);
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int c = 0; c < CH; ++c) *(uint4*)(lds + dst[c]) = v[c];
  }
};

// Operand contiguous along M/N: element (k, col) at col_ptr(col)[k * ld].
// Each unit is 8 consecutive k x 4 consecutive columns, transposed in
// registers into four 16-byte K-chunks.  col_ptr(c) is nullptr for a group of
// 4 columns outside the matrix; rows k >= k_end load as zeros.
template <int R, int NT>
struct LoadMN {
  static constexpr int U = 2 * R / NT;
  static_assert(U >= 1 && (2 * R) % NT == 0, "tile/threads mismatch");
  const uint16_t* src[U];
  int kg[U];
  int dst_row[U];
  long ld;
  uint2 v[U][8];
  template <class ColPtr>
  __device__ __forceinline__ void init(ColPtr col_ptr, long ld_, int tid) {
    ld = ld_;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = u * NT + tid, mg = q % (R / 4);
      kg[u] = q / (R / 4);
      dst_row[u] = mg * 4;
      src[u] = col_ptr(mg * 4);
    }
  }
  __device__ __forceinline__ void load(int k0, int k_end) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int k = k0 + kg[u] * 8 + kk;
        v[u][kk] = (src[u] && k < k_end) ? *(const uint2*)(src[u] + (long)k * ld)
                                          : make_uint2(0u, 0u);
      }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t e[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const uint32_t w = (i < 2) ? v[u][kk].x : v[u][kk].y;
          e[kk] = (i & 1) ? (w >> 16) : (w & 0xffffu);
        }
        uint4 o;
        o.x = e[0] | (e[1] << 16);
        o.y = e[2] | (e[3] << 16);
        o.z = e[4] | (e[5] << 16);
        o.w = e[6] | (e[7] << 16);
        *(uint4*)(lds + lds_off(dst_row[u] + i, kg[u])) = o;
      }
  }
};

template <int BM_, int BN_, int WGM_, int WGN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * BK;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
};

// Output element held by accumulator register r of 32x32 tile (i, j) in this
// lane: row = wave_row0 + i*32 + out_row(lane, r), col = wave_col0 + j*32 + lane%32.
__device__ __forceinline__ int out_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Two-stage LDS main loop over k in [k_begin, k_end), steps of 64.
template <class TL, class LA, class LB>
__device__ __forceinline__ void mainloop(LA& la, LB& lb, int k_begin, int k_end,
                                         uint16_t* smem, f32x16_t (&acc)[TL::TM][TL::TN]) {
  uint16_t* const sA0 = smem;
  uint16_t* const sA1 = smem + TL::BM * BK;
  uint16_t* const sB0 = smem + 2 * TL::BM * BK;
  uint16_t* const sB1 = sB0 + TL::BN * BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  const int fr = lane & 31, fk = lane >> 5;
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;  // block-uniform
  la.load(k_begin, k_end);
  lb.load(k_begin, k_end);
  la.store(sA0);
  lb.store(sB0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool odd = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(k_begin + (kt + 1) * BK, k_end);
      lb.load(k_begin + (kt + 1) * BK, k_end);
    }
    const uint16_t* A = odd ? sA1 : sA0;
    const uint16_t* B = odd ? sB1 : sB0;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t a[TL::TM], b[TL::TN];
#pragma unroll
      for (int i = 0; i < TL::TM; ++i)
        a[i] = *(const bf16x8_t*)(A + lds_off(wm * TL::WTM + i * 32 + fr, kk * 2 + fk));
#pragma unroll
      for (int j = 0; j < TL::TN; ++j)
        b[j] = *(const bf16x8_t*)(B + lds_off(wn * TL::WTN + j * 32 + fr, kk * 2 + fk));
#pragma unroll
      for (int i = 0; i < TL::TM; ++i)
#pragma unroll
        for (int j = 0; j < TL::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(odd ? sA0 : sA1);
      lb.store(odd ? sB0 : sB1);
    }
    __syncthreads();
  }
}

struct RowTile {
  int e, m0, m_end;
};

// (expert, first row, row end) of M-tile mt; false (block-uniform) past the last tile.
__device__ __forceinline__ bool row_tile(const int32_t* __restrict__ offsets,
                                         const int32_t* __restrict__ tile_offsets, int E_l,
                                         int mt, int* s_to, int* s_off, RowTile& rt) {
  for (int j = threadIdx.x; j <= E_l; j += blockDim.x) {
    s_to[j] = tile_offsets[j];
    s_off[j] = offsets[j];
  }
  __syncthreads();
  if (mt >= s_to[E_l]) return false;
  int lo = 0, hi = E_l;  // s_to[lo] <= mt < s_to[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_to[mid] <= mt) lo = mid;
    else hi = mid;
  }
  rt.e = lo;
  rt.m0 = s_off[lo] + (mt - s_to[lo]) * kTileM;
  rt.m_end = s_off[lo + 1];
  return true;
}

// ---------------------------------------------------------------------------
// forward GEMM1: [g, u] = xp . W_gu[e]^T with the SwiGLU epilogue.
// The B tile pairs gate and up rows: wave wn's 64 tile rows are 32 gate rows
// j and the 32 up rows F + j of the same j, so each lane holds g and u of the
// same output element.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void ffn_gate_up_kernel(
    const uint16_t* __restrict__ xp, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_offsets, const uint16_t* __restrict__ W_gu,
    uint16_t* __restrict__ h, uint16_t* __restrict__ a, int E_l, int d, int F, int n_tiles) {
  using TL = Tile<BM, BN, WGM, WGN>;
  static_assert(BM == kTileM, "row tiles come from the dispatch plan");
  static_assert(TL::WTN == 64, "each wave pairs 32 gate with 32 up columns");
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  __shared__ int s_to[257], s_off[257];
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = lid / n_tiles, nt = lid % n_tiles;
  RowTile rt;
  if (!row_tile(offsets, tile_offsets, E_l, mt, s_to, s_off, rt)) return;
  const int tid = threadIdx.x;
  const int jb = nt * (BN / 2);
  const uint16_t* Wg = W_gu + (size_t)rt.e * 2 * F * d;
  LoadK<BM, TL::NT> la;
  LoadK<BN, TL::NT> lb;
  la.init([&](int r) -> const uint16_t* {
    const int row = rt.m0 + r;
    return row < rt.m_end ? xp + (size_t)row * d : nullptr;
  }, tid);
  lb.init([&](int n) -> const uint16_t* {
    const int j = jb + (n >> 6) * 32 + (n & 31);
    return j < F ? Wg + (size_t)(((n >> 5) & 1) * F + j) * d : nullptr;
  }, tid);
  f32x16_t acc[TL::TM][TL::TN];
  mainloop<TL>(la, lb, 0, d, smem, acc);
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
  const int j = jb + wn * 32 + (lane & 31);
  if (j >= F) return;
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rt.m0 + wm * TL::WTM + i * 32 + out_row(lane, r);
      if (row < rt.m_end) {
        const float g = acc[i][0][r], u = acc[i][1][r];
        h[(size_t)row * 2 * F + j] = f2bf(g);
        h[(size_t)row * 2 * F + F + j] = f2bf(u);
        a[(size_t)row * F + j] = f2bf(silu_f(g) * u);
      }
    }
}

// ---------------------------------------------------------------------------
// forward GEMM2: y_p = a . W_down[e]^T   (A: a rows, K = F; B: W_down rows, K = F)
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void ffn_down_kernel(
    const uint16_t* __restrict__ a, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_offsets, const uint16_t* __restrict__ W_down,
    uint16_t* __restrict__ yp, int E_l, int d, int F, int n_tiles) {
  using TL = Tile<BM, BN, WGM, WGN>;
  static_assert(BM == kTileM, "row tiles come from the dispatch plan");
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  __shared__ int s_to[257], s_off[257];
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = lid / n_tiles, nt = lid % n_tiles;
  RowTile rt;
  if (!row_tile(offsets, tile_offsets, E_l, mt, s_to, s_off, rt)) return;
  const int tid = threadIdx.x;
  const int nb = nt * BN;
  const uint16_t* Wd = W_down + (size_t)rt.e * d * F;
  LoadK<BM, TL::NT> la;
  LoadK<BN, TL::NT> lb;
  la.init([&](int r) -> const uint16_t* {
    const int row = rt.m0 + r;
    return row < rt.m_end ? a + (size_t)row * F : nullptr;
  }, tid);
  lb.init([&](int n) -> const uint16_t* {
    return nb + n < d ? Wd + (size_t)(nb + n) * F : nullptr;
  }, tid);
  f32x16_t acc[TL::TM][TL::TN];
  mainloop<TL>(la, lb, 0, F, smem, acc);
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int j = 0; j < TL::TN; ++j) {
    const int col = nb + wn * TL::WTN + j * 32 + (lane & 31);
    if (col >= d) continue;
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rt.m0 + wm * TL::WTM + i * 32 + out_row(lane, r);
        if (row < rt.m_end) yp[(size_t)row * d + col] = f2bf(acc[i][j][r]);
      }
  }
}

// ---------------------------------------------------------------------------
// dgrad GEMM A: da = dy_p . W_down[e]  (A: dy_p rows, K = d; B: W_down[e] as
// [K = d][N = F], contiguous along N) with the SwiGLU backward epilogue.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void dgrad_act_kernel(
    const uint16_t* __restrict__ dyp, const uint16_t* __restrict__ hbuf,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_offsets,
    const uint16_t* __restrict__ W_down, uint16_t* __restrict__ dh, int E_l, int d, int F,
    int n_tiles) {
  using TL = Tile<BM, BN, WGM, WGN>;
  static_assert(BM == kTileM, "row tiles come from the dispatch plan");
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  __shared__ int s_to[257], s_off[257];
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = lid / n_tiles, nt = lid % n_tiles;
  RowTile rt;
  if (!row_tile(offsets, tile_offsets, E_l, mt, s_to, s_off, rt)) return;
  const int tid = threadIdx.x;
  const int nb = nt * BN;
  const uint16_t* Wd = W_down + (size_t)rt.e * d * F;
  LoadK<BM, TL::NT> la;
  LoadMN<BN, TL::NT> lb;
  la.init([&](int r) -> const uint16_t* {
    const int row = rt.m0 + r;
    return row < rt.m_end ? dyp + (size_t)row * d : nullptr;
  }, tid);
  lb.init([&](int c) -> const uint16_t* { return nb + c < F ? Wd + nb + c : nullptr; },
          (long)F, tid);
  f32x16_t acc[TL::TM][TL::TN];
  mainloop<TL>(la, lb, 0, d, smem, acc);
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int j = 0; j < TL::TN; ++j) {
    const int col = nb + wn * TL::WTN + j * 32 + (lane & 31);
    if (col >= F) continue;
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rt.m0 + wm * TL::WTM + i * 32 + out_row(lane, r);
        if (row < rt.m_end) {
          const float da = acc[i][j][r];
          const float g = bf2f(hbuf[(size_t)row * 2 * F + col]);
          const float u = bf2f(hbuf[(size_t)row * 2 * F + F + col]);
          const float s = sigmoid_f(g);
          dh[(size_t)row * 2 * F + col] = f2bf(da * u * s * (1.0f + g * (1.0f - s)));
          dh[(size_t)row * 2 * F + F + col] = f2bf(da * g * s);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dgrad GEMM B: dxp = dh . W_gu[e]  (A: dh rows, K = 2F; B: W_gu[e] as
// [K = 2F][N = d], contiguous along N)
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void dgrad_in_kernel(
    const uint16_t* __restrict__ dh, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_offsets, const uint16_t* __restrict__ W_gu,
    uint16_t* __restrict__ dxp, int E_l, int d, int F, int n_tiles) {
  using TL = Tile<BM, BN, WGM, WGN>;
  static_assert(BM == kTileM, "row tiles come from the dispatch plan");
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  __shared__ int s_to[257], s_off[257];
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = lid / n_tiles, nt = lid % n_tiles;
  RowTile rt;
  if (!row_tile(offsets, tile_offsets, E_l, mt, s_to, s_off, rt)) return;
  const int tid = threadIdx.x;
  const int nb = nt * BN;
  const uint16_t* Wg = W_gu + (size_t)rt.e * 2 * F * d;
  LoadK<BM, TL::NT> la;
  LoadMN<BN, TL::NT> lb;
  la.init([&](int r) -> const uint16_t* {
    const int row = rt.m0 + r;
    return row < rt.m_end ? dh + (size_t)row * 2 * F : nullptr;
  }, tid);
  lb.init([&](int c) -> const uint16_t* { return nb + c < d ? Wg + nb + c : nullptr; },
          (long)d, tid);
  f32x16_t acc[TL::TM][TL::TN];
  mainloop<TL>(la, lb, 0, 2 * F, smem, acc);
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int j = 0; j < TL::TN; ++j) {
    const int col = nb + wn * TL::WTN + j * 32 + (lane & 31);
    if (col >= d) continue;
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rt.m0 + wm * TL::WTM + i * 32 + out_row(lane, r);
        if (row < rt.m_end) dxp[(size_t)row * d + col] = f2bf(acc[i][j][r]);
      }
  }
}

// ---------------------------------------------------------------------------
// wgrad: per local expert e over its rows [offsets[e], offsets[e+1]):
//   dW_down[e] (d x F)  = dy_p^T . a      (A: dy_p, M = d;  B: a,  N = F)
//   dW_gu[e]   (2F x d) = dh^T   . xp     (A: dh,   M = 2F; B: xp, N = d)
// Both operands are contiguous along M/N (reduction over rows).  One launch
// covers both products of every expert; tiles of one expert are consecutive.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void wgrad_kernel(
    const uint16_t* __restrict__ xp, const uint16_t* __restrict__ abuf,
    const uint16_t* __restrict__ dh, const uint16_t* __restrict__ dyp,
    const int32_t* __restrict__ offsets, float* __restrict__ dW_gu,
    float* __restrict__ dW_down, int d, int F, int accumulate) {
  using TL = Tile<BM, BN, WGM, WGN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  const int tdm = (d + BM - 1) / BM, tdn = (F + BN - 1) / BN;
  const int tgm = (2 * F + BM - 1) / BM, tgn = (d + BN - 1) / BN;
  const int per_e = tdm * tdn + tgm * tgn;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int e = lid / per_e;
  int t = lid % per_e;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const uint16_t *Asrc, *Bsrc;
  int M, N, m0, n0;
  float* out;
  if (t < tdm * tdn) {
    Asrc = dyp;
    Bsrc = abuf;
    M = d;
    N = F;
    m0 = (t / tdn) * BM;
    n0 = (t % tdn) * BN;
    out = dW_down + (size_t)e * d * F;
  } else {
    t -= tdm * tdn;
    Asrc = dh;
    Bsrc = xp;
    M = 2 * F;
    N = d;
    m0 = (t / tgn) * BM;
    n0 = (t % tgn) * BN;
    out = dW_gu + (size_t)e * 2 * F * d;
  }
  const int tid = threadIdx.x;
  LoadMN<BM, TL::NT> la;
  LoadMN<BN, TL::NT> lb;
  la.init([&](int c) -> const uint16_t* { return m0 + c < M ? Asrc + m0 + c : nullptr; },
          (long)M, tid);
  lb.init([&](int c) -> const uint16_t* { return n0 + c < N ? Bsrc + n0 + c : nullptr; },
          (long)N, tid);
  f32x16_t acc[TL::TM][TL::TN];
  mainloop<TL>(la, lb, r0, r1, smem, acc);
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int j = 0; j < TL::TN; ++j) {
    const int col = n0 + wn * TL::WTN + j * 32 + (lane & 31);
    if (col >= N) continue;
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * TL::WTM + i * 32 + out_row(lane, r);
        if (row < M) {
          float* o = out + (size_t)row * N + col;
          *o = accumulate ? *o + acc[i][j][r] : acc[i][j][r];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// router logits: l = x . W_r + bias with W_r given transposed (W_rT [E][d]),
// float32 output.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void router_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W_rT,
    const float* __restrict__ bias, float* __restrict__ logits, int T, int d, int E,
    int n_tiles) {
  using TL = Tile<BM, BN, WGM, WGN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (lid / n_tiles) * BM, n0 = (lid % n_tiles) * BN;
  const int tid = threadIdx.x;
  LoadK<BM, TL::NT> la;
  LoadK<BN, TL::NT> lb;
  la.init([&](int r) -> const uint16_t* {
    return m0 + r < T ? x + (size_t)(m0 + r) * d : nullptr;
  }, tid);
  lb.init([&](int n) -> const uint16_t* {
    return n0 + n < E ? W_rT + (size_t)(n0 + n) * d : nullptr;
  }, tid);
  f32x16_t acc[TL::TM][TL::TN];
  mainloop<TL>(la, lb, 0, d, smem, acc);
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int j = 0; j < TL::TN; ++j) {
    const int col = n0 + wn * TL::WTN + j * 32 + (lane & 31);
    if (col >= E) continue;
    const float b = bias ? bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * TL::WTM + i * 32 + out_row(lane, r);
        if (row < T) logits[(size_t)row * E + col] = acc[i][j][r] + b;
      }
  }
}

// Upper bound on the number of kTileM-row tiles over all local experts.
inline int max_row_tiles(const moe_shape* s) {
  const int64_t cap = s->T * s->K;
  return (int)((cap + s->E_l * (int64_t)(kTileM - 1)) / kTileM);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers (bf16)
// ---------------------------------------------------------------------------
int launch_ffn_fwd_bf16(const moe_shape* s, const void* xp, const int32_t* offsets,
                        const int32_t* tile_offsets, const void* W_gu, const void* W_down,
                        void* h, void* a, void* yp, hipStream_t st) {
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  const int mt = max_row_tiles(s);
  if (mt == 0) return MOE_OK;
  {
    const int nt = (F + 127) / 128;
    MOE_LAUNCH("ffn_gate_up", st,
               ffn_gate_up_kernel<256, 256, 2, 4><<<mt * nt, 512, 0, st>>>(
        (const uint16_t*)xp, offsets, tile_offsets, (const uint16_t*)W_gu, (uint16_t*)h,
        (uint16_t*)a, E_l, d, F, nt));
    if (int rc = check_launch("expert GEMM1 (gate/up + SwiGLU)")) return rc;
  }
  {
    const int nt = (d + 255) / 256;
    MOE_LAUNCH("ffn_down", st,
               ffn_down_kernel<256, 256, 2, 4><<<mt * nt, 512, 0, st>>>(
        (const uint16_t*)a, offsets, tile_offsets, (const uint16_t*)W_down, (uint16_t*)yp, E_l,
        d, F, nt));
    if (int rc = check_launch("expert GEMM2 (down)")) return rc;
  }
  return MOE_OK;
}

int launch_ffn_dgrad_bf16(const moe_shape* s, const void* dyp, const void* h,
                          const int32_t* offsets, const int32_t* tile_offsets, const void* W_gu,
                          const void* W_down, void* dh, void* dxp, hipStream_t st) {
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  const int mt = max_row_tiles(s);
  if (mt == 0) return MOE_OK;
  {
    const int nt = (F + 255) / 256;
    MOE_LAUNCH("dgrad_act", st,
               dgrad_act_kernel<256, 256, 2, 4><<<mt * nt, 512, 0, st>>>(
        (const uint16_t*)dyp, (const uint16_t*)h, offsets, tile_offsets,
        (const uint16_t*)W_down, (uint16_t*)dh, E_l, d, F, nt));
    if (int rc = check_launch("dgrad GEMM (activation)")) return rc;
  }
  {
    const int nt = (d + 255) / 256;
    MOE_LAUNCH("dgrad_in", st,
               dgrad_in_kernel<256, 256, 2, 4><<<mt * nt, 512, 0, st>>>(
        (const uint16_t*)dh, offsets, tile_offsets, (const uint16_t*)W_gu, (uint16_t*)dxp, E_l,
        d, F, nt));
    if (int rc = check_launch("dgrad GEMM (input)")) return rc;
  }
  return MOE_OK;
}

int launch_ffn_wgrad_bf16(const moe_shape* s, const void* xp, const void* a, const void* dh,
                          const void* dyp, const int32_t* offsets, float* dW_gu, float* dW_down,
                          bool accumulate, hipStream_t st) {
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  const int per_e = ((d + 255) / 256) * ((F + 255) / 256) + ((2 * F + 255) / 256) * ((d + 255) / 256);
  MOE_LAUNCH("wgrad", st,
             wgrad_kernel<256, 256, 2, 4><<<E_l * per_e, 512, 0, st>>>(
      (const uint16_t*)xp, (const uint16_t*)a, (const uint16_t*)dh, (const uint16_t*)dyp, offsets,
      dW_gu, dW_down, d, F, accumulate ? 1 : 0));
  return check_launch("wgrad GEMM");
}

int launch_router_logits_bf16(const moe_shape* s, const void* x, const void* W_rT,
                              const float* bias, float* logits, hipStream_t st) {
  const int T = (int)s->T, d = (int)s->d, E = (int)s->E;
  const int nt = (E + 127) / 128, mt = (T + 127) / 128;
  MOE_LAUNCH("router", st,
             router_kernel<128, 128, 2, 2><<<mt * nt, 256, 0, st>>>(
      (const uint16_t*)x, (const uint16_t*)W_rT, bias, logits, T, d, E, nt));
  return check_launch("router GEMM");
}

}  // namespace moe
