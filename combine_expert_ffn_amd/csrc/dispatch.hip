// Dispatch (token -> expert-grouped rows) and combine (rows -> tokens, gate
// weighted), forward and backward: the local halves of the token all-to-all
// that the expert-parallel overlap pages hide behind the expert FFN (skill card
// page 1, "What it is"; 1F1B note page 2, backward chain "combine.backward",
// "dispatch.backward").
//
// The plan is a deterministic stable counting sort of the (token, slot) pairs
// by local expert: per-block LDS histograms, one exclusive scan over
// (expert, block), then an in-block stable rank from per-(wave, expert) LDS
// lane masks and a per-wave LDS prefix.  No global atomics decide positions, so the maps
// are bit-identical run to run.
//
// The copies are token-major: one wave per token reads the token's row once
// and writes (or gathers) its K rows with 16-byte accesses.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// plan step 1: per-block histogram of local expert ids.
// blockcnt[j * NB + b] = number of pairs of block b with local id j.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_hist_kernel(const int32_t* __restrict__ idx,
                                                        long npairs, int e_lo, int E_l, int NB,
                                                        int32_t* __restrict__ blockcnt) {
  __shared__ int cnt[256];
  const int b = blockIdx.x;
  for (int j = threadIdx.x; j < E_l; j += 256) cnt[j] = 0;
  __syncthreads();
  const long p0 = (long)b * kPlanChunk;
  const long p1 = min(npairs, p0 + kPlanChunk);
  for (long p = p0 + threadIdx.x; p < p1; p += 256) {
    const int j = idx[p] - e_lo;
    if (j >= 0 && j < E_l) atomicAdd(&cnt[j], 1);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < E_l; j += 256) blockcnt[(size_t)j * NB + b] = cnt[j];
}

// ---------------------------------------------------------------------------
// plan step 2: one block.  Exclusive scan of blockcnt in (expert, block) order
// -> blockbase; counts, offsets and tile_offsets.
// The block is 256 threads (one wave per SIMD, few registers), so that it fits
// on a CU beside a block of a persistent expert GEMM running on the other
// stream, instead of waiting for one to retire.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 256;
__global__ __launch_bounds__(kScanThreads) void plan_scan_kernel(
    const int32_t* __restrict__ blockcnt, int32_t* __restrict__ blockbase, int E_l, int NB,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_offsets) {
  constexpr int NW = kScanThreads / 64;
  __shared__ int wsum[NW];
  __shared__ int s_off[257];  // E_l <= 256
  const int n = E_l * NB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // wave w scans the contiguous range [b0, b1) (b0 a multiple of 256), 256
  // entries per step: lane l takes entries 4l .. 4l + 3 of the step (one
  // 16-byte load when all four are in range)
  const int per = ((n + NW - 1) / NW + 255) / 256 * 256;
  const int b0 = min(n, w * per), b1 = min(n, b0 + per);
  // the caller's workspace carries no alignment promise: vector loads only
  // when its base is 16-byte aligned (wave-uniform)
  const bool vec = ((uintptr_t)blockcnt & 15) == 0;
  auto load4 = [&](int i, int (&v)[4]) {
    if (vec && i + 3 < b1) {
      const int4 q = *(const int4*)(blockcnt + i);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = i + k < b1 ? blockcnt[i + k] : 0;
    }
  };
  int s = 0;
#pragma unroll 2
  for (int c = b0; c < b1; c += 256) {
    int v[4];
    load4(c + 4 * lane, v);
    s += v[0] + v[1] + v[2] + v[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) wsum[w] = s;
  __syncthreads();
  int carry = 0, total = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    if (u < w) carry += wsum[u];
    total += wsum[u];
  }
  // exclusive prefix: per lane over its four entries, then a wave inclusive
  // scan of the lane sums and the running carry; the start of expert j's
  // segment (entry j * NB) goes to LDS
  for (int c = b0; c < b1; c += 256) {
    const int i = c + 4 * lane;
    int v[4];
    load4(i, v);
    const int t = v[0] + v[1] + v[2] + v[3];
    int incl = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    int ex = carry + incl - t;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (i + k < b1) {
        blockbase[i + k] = ex;
        if ((i + k) % NB == 0) s_off[(i + k) / NB] = ex;
      }
      ex += v[k];
    }
    carry += __shfl(incl, 63, 64);
  }
  if (tid == 0) s_off[E_l] = total;
  if (NB == 0)
    for (int j = tid; j < E_l; j += kScanThreads) s_off[j] = 0;
  __syncthreads();
  // offsets[j] = start of expert j's segment; offsets[E_l] = N
  for (int j = tid; j <= E_l; j += kScanThreads) offsets[j] = s_off[j];
  if (tid == 0) {
    int acc = 0;
    for (int j = 0; j < E_l; ++j) {
      const int c = s_off[j + 1] - s_off[j];
      counts[j] = c;
      if (tile_offsets) tile_offsets[j] = acc;
      acc += (c + kTileM - 1) / kTileM;
    }
    if (tile_offsets) tile_offsets[E_l] = acc;
  }
}

// ---------------------------------------------------------------------------
// plan step 3: stable in-block rank -> row_of_pair, pair_of_row.
// Rounds of 256 pairs; within a wave, pairs with the same expert are ranked by
// a 64-bit LDS lane mask per (wave, expert): each lane ORs in its bit, reads
// the mask back and counts the lower lanes (the cost does not depend on how
// many distinct experts the wave holds); across waves by a per-wave count
// prefix in LDS; across rounds by a running count.
// Also writes -1 into pair_of_row rows [N, cap) of this block's range.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_rank_kernel(const int32_t* __restrict__ idx,
                                                        long npairs, int e_lo, int E_l, int NB,
                                                        const int32_t* __restrict__ blockbase,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ row_of_pair,
                                                        int32_t* __restrict__ pair_of_row) {
  __shared__ int running[256];
  __shared__ int wcnt[4][256];
  __shared__ unsigned long long wmask[4][256];  // lanes of wave w holding expert j
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int j = tid; j < E_l; j += 256) {
    running[j] = blockbase[(size_t)j * NB + b];
    wcnt[0][j] = wcnt[1][j] = wcnt[2][j] = wcnt[3][j] = 0;
    wmask[0][j] = wmask[1][j] = wmask[2][j] = wmask[3][j] = 0ull;
  }
  __syncthreads();
  const long p0 = (long)b * kPlanChunk;
  const long p1 = min(npairs, p0 + kPlanChunk);
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (long base = p0; base < p1; base += 256) {
    const long p = base + tid;
    int j = -1;
    if (p < p1) {
      const int jj = idx[p] - e_lo;
      if (jj >= 0 && jj < E_l) j = jj;
    }
    // stable rank among the wave's lanes with the same expert: each lane sets
    // its bit in its expert's mask, reads the mask back (the LDS operations of
    // one wave complete in order) and counts the lower lanes, then the mask is
    // cleared for the next round; constant work however many experts the wave
    // holds
    int myrank = 0;
    if (j >= 0) {
      atomicOr(&wmask[w][j], 1ull << lane);
      const unsigned long long m = wmask[w][j];
      myrank = __popcll(m & lt_mask);
      wcnt[w][j] = __popcll(m);
      wmask[w][j] = 0ull;
    }
    __syncthreads();
    if (p < p1) {
      if (j >= 0) {
        int row = running[j] + myrank;
        for (int ww = 0; ww < w; ++ww) row += wcnt[ww][j];
        row_of_pair[p] = row;
        if (row < npairs) pair_of_row[row] = (int32_t)p;
      } else {
        row_of_pair[p] = -1;
      }
    }
    __syncthreads();
    for (int jj = tid; jj < E_l; jj += 256) {
      running[jj] += wcnt[0][jj] + wcnt[1][jj] + wcnt[2][jj] + wcnt[3][jj];
      wcnt[0][jj] = wcnt[1][jj] = wcnt[2][jj] = wcnt[3][jj] = 0;
    }
    __syncthreads();
  }
  // rows [N, cap) of this block's row range get -1
  const long N = offsets[E_l];
  const long r0 = max(N, p0);
  for (long r = r0 + tid; r < min(npairs, p0 + (long)kPlanChunk); r += 256) pair_of_row[r] = -1;
}

// The dispatch plan of the shared expert: one expert over all T rows in token
// order: offsets {0, T}, tile_offsets {0, ceil(T / kTileM)}.
__global__ void shared_plan_kernel(int32_t* __restrict__ plan, int T_) {
  if (threadIdx.x == 0) {
    plan[0] = 0;
    plan[1] = T_;
    plan[2] = 0;
    plan[3] = (T_ + kTileM - 1) / kTileM;
  }
}

int launch_shared_plan(int64_t T, int32_t* plan, hipStream_t st) {
  MOE_LAUNCH("shared_plan", st, shared_plan_kernel<<<1, 64, 0, st>>>(plan, (int)T));
  return check_launch("shared plan");
}

int launch_plan(const moe_shape* s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                int32_t* row_of_pair, int32_t* pair_of_row, int32_t* tile_offsets, void* ws,
                hipStream_t st) {
  const long npairs = s->T * s->K;
  const int NB = (int)cdiv(npairs, kPlanChunk);
  int32_t* blockcnt = (int32_t*)ws;
  int32_t* blockbase = blockcnt + (size_t)s->E_l * NB;
  int rc;
  if (NB > 0) {
    MOE_LAUNCH("plan_hist", st,
               plan_hist_kernel<<<NB, 256, 0, st>>>(idx, npairs, (int)s->e_lo, (int)s->E_l, NB, blockcnt));
    if ((rc = check_launch("plan histogram"))) return rc;
  }
  MOE_LAUNCH("plan_scan", st,
             plan_scan_kernel<<<1, kScanThreads, 0, st>>>(blockcnt, blockbase, (int)s->E_l, NB, counts, offsets,
                                       tile_offsets));
  if ((rc = check_launch("plan scan"))) return rc;
  if (NB > 0) {
    MOE_LAUNCH("plan_rank", st,
               plan_rank_kernel<<<NB, 256, 0, st>>>(idx, npairs, (int)s->e_lo, (int)s->E_l, NB, blockbase,
                                         offsets, row_of_pair, pair_of_row));
    if ((rc = check_launch("plan rank"))) return rc;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Token-major kernels (permute, combine and their backwards): one wave per
// token, lane l handles the 16-byte chunks l, l+64, ... of a row.  Row lengths
// are multiples of 8 chunks but not always of 64, so loads use a clamped
// (always valid) chunk index and only the stores are predicated: with no
// branch between them, a row's loads, and those of the next row, are in
// flight together instead of one at a time.
// ---------------------------------------------------------------------------

// The token's local rows: lane k (< K) holds row_of_pair[t*K + k]; the valid
// slots form a wave-uniform bit mask, walked in ascending slot order, and a
// slot's row is read from its lane, so everything stays in scalar registers.
struct LocalRows {
  uint64_t mask;
  int rk;
  __device__ __forceinline__ void load(const int32_t* __restrict__ row_of_pair, int t, int K,
                                       int nrows, int lane) {
    rk = lane < K ? row_of_pair[(size_t)t * K + lane] : -1;
    mask = __ballot(rk >= 0 && rk < nrows);
  }
  __device__ __forceinline__ bool empty() const { return mask == 0; }
  // next valid slot (ascending); the mask must not be empty
  __device__ __forceinline__ int next() {
    const int k = __ffsll((unsigned long long)mask) - 1;
    mask &= mask - 1;
    return k;
  }
  __device__ __forceinline__ int row(int k) const { return __builtin_amdgcn_readlane(rk, k); }
};

// A 16-byte load with the non-temporal cache policy, for the gathered row
// streams (y_p in the combine and its backward, dx_p in the dispatch
// backward): each row is read once per launch, so it should not displace
// what the next kernels read (measured on the 128-expert layer: combine
// 126 -> 106 us).  Stores keep the default policy: their rows (x_p, dy_p) are
// read back by the expert GEMMs that follow.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Keep a loaded chunk in registers where it was loaded: without this the
// compiler may move a side-effect-free load next to each of its uses (into a
// conditional block or a loop), where its latency is no longer overlapped.
__device__ __forceinline__ void pin(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ int uniform_token(int lane_tid_base) {
  return __builtin_amdgcn_readfirstlane(lane_tid_base);
}

// ---------------------------------------------------------------------------
// permute: xp[row_of_pair[t*K+k]] = x[t].  The token row is read once and
// written to each of its local rows.
// ---------------------------------------------------------------------------
template <int MAXC>
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ row_of_pair,
                                                      uint4* __restrict__ xp, int T, int K,
                                                      int nch) {
  const int t = uniform_token((int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6));
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const uint4* src = x + (size_t)t * nch;
  LocalRows lr0;
  lr0.load(row_of_pair, t, K, T * K, lane);
  for (int c0 = 0; c0 < nch; c0 += 64 * MAXC) {
    uint4 v[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = c0 + lane + 64 * i;
      v[i] = src[c < nch ? c : nch - 1];
    }
    // (otherwise the loads are re-issued for every destination row)
#pragma unroll
    for (int i = 0; i < MAXC; ++i) pin(v[i]);
    for (LocalRows lr = lr0; !lr.empty();) {
      uint4* dst = xp + (size_t)lr.row(lr.next()) * nch;
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = c0 + lane + 64 * i;
        if (c < nch) dst[c] = v[i];
      }
    }
  }
}

static inline int row_chunks(const moe_shape* s) {
  return (int)(s->d * (int64_t)elt_bytes(s) / 16);
}

int launch_permute(const moe_shape* s, const void* x, const int32_t* row_of_pair, void* xp,
                   hipStream_t st) {
  if (s->T == 0) return MOE_OK;
  MOE_LAUNCH("permute", st,
             permute_kernel<4><<<(unsigned)cdiv(s->T, 4), 256, 0, st>>>(
      (const uint4*)x, row_of_pair, (uint4*)xp, (int)s->T, (int)s->K, row_chunks(s)));
  return check_launch("permute");
}

// ---------------------------------------------------------------------------
// combine: out[t] = [add[t] +] sum_k gates[t,k] * yp[row(t,k)] over local k
// ascending, float32 accumulation, one rounding.  add (nullable) is a
// token-aligned term such as the shared expert's output.  One wave per token.
// ---------------------------------------------------------------------------
template <typename T, int MAXC>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ row_of_pair,
                                                      const uint4* __restrict__ add,
                                                      uint4* __restrict__ out, int T_, int K,
                                                      int nch, int pairs) {
  constexpr int CN = Chunk<T>::N;
  const int t = uniform_token((int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6));
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  LocalRows lr0;
  lr0.load(row_of_pair, t, K, T_ * K, lane);
  for (int c0 = 0; c0 < nch; c0 += 64 * MAXC) {
    int cc[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = c0 + lane + 64 * i;
      cc[i] = c < nch ? c : nch - 1;
    }
    float acc[MAXC][CN];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      if (add) {  // uniform
        Chunk<T>::unpack(add[(size_t)t * nch + cc[i]], acc[i]);
      } else {
#pragma unroll
        for (int q = 0; q < CN; ++q) acc[i][q] = 0.f;
      }
    }
    // two rows per pass: both rows' loads are issued before the first FMA;
    // the sum still runs over the rows in ascending slot order
    LocalRows lr = lr0;
    while (!lr.empty()) {
      const int k0 = lr.next();
      const bool two = !lr.empty();
      const int k1 = two ? lr.next() : k0;
      // y by dispatched row, or (pairs) by pair: token t's slots are rows
      // t*K .. t*K + K - 1
      const uint4* s0 = yp + (size_t)(pairs ? t * K + k0 : lr.row(k0)) * nch;
      const uint4* s1 = yp + (size_t)(pairs ? t * K + k1 : lr.row(k1)) * nch;
      uint4 v0[MAXC], v1[MAXC];
#pragma unroll
      for (int i = 0; i < MAXC; ++i) v0[i] = load_nt(&s0[cc[i]]);
#pragma unroll
      for (int i = 0; i < MAXC; ++i) v1[i] = load_nt(&s1[cc[i]]);
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        pin(v0[i]);
        pin(v1[i]);
      }
      const float g0 = gates[(size_t)t * K + k0];
      const float g1 = gates[(size_t)t * K + k1];
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        float f[CN];
        Chunk<T>::unpack(v0[i], f);
#pragma unroll
        for (int q = 0; q < CN; ++q) acc[i][q] = fmaf(g0, f[q], acc[i][q]);
      }
      if (two) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          float f[CN];
          Chunk<T>::unpack(v1[i], f);
#pragma unroll
          for (int q = 0; q < CN; ++q) acc[i][q] = fmaf(g1, f[q], acc[i][q]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = c0 + lane + 64 * i;
      if (c < nch) out[(size_t)t * nch + c] = Chunk<T>::pack(acc[i]);
    }
  }
}

template <typename T>
static void combine_t(const moe_shape* s, const void* yp, const float* gates,
                      const int32_t* row_of_pair, const void* add, void* out, hipStream_t st,
                      bool pairs) {
  MOE_LAUNCH("combine", st,
             combine_kernel<T, 4><<<(unsigned)cdiv(s->T, 4), 256, 0, st>>>(
                 (const uint4*)yp, gates, row_of_pair, (const uint4*)add, (uint4*)out, (int)s->T,
                 (int)s->K, row_chunks(s), pairs ? 1 : 0));
}

int launch_combine(const moe_shape* s, const void* yp, const float* gates,
                   const int32_t* row_of_pair, const void* add, void* out, hipStream_t st,
                   bool pairs) {
  if (s->T == 0) return MOE_OK;
  if (s->dtype == MOE_BF16) combine_t<uint16_t>(s, yp, gates, row_of_pair, add, out, st, pairs);
  else if (s->dtype == MOE_F16)
    combine_t<_Float16>(s, yp, gates, row_of_pair, add, out, st, pairs);
  else combine_t<float>(s, yp, gates, row_of_pair, add, out, st, pairs);
  return check_launch("combine");
}

// ---------------------------------------------------------------------------
// combine backward: dyp[r] = g * dout[t]; dgates[t,k] = <dout[t], yp[r]>.
// One wave per token; dout row held in registers.  WRITE_DYP = false: dgates
// only (the fused combine backward: the expert GEMMs gather dout themselves).
// ---------------------------------------------------------------------------
template <typename T, int MAXC, bool WRITE_DYP>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* __restrict__ dout,
                                                          const uint4* __restrict__ yp,
                                                          const float* __restrict__ gates,
                                                          const int32_t* __restrict__ row_of_pair,
                                                          uint4* __restrict__ dyp,
                                                          float* __restrict__ dgates, int T_,
                                                          int K, int nch, int pairs) {
  constexpr int CN = Chunk<T>::N;
  const int t = uniform_token((int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6));
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  // nch <= 64 * MAXC is guaranteed by the launcher (whole dout row in registers)
  float dv[MAXC][CN];
  {
    uint4 raw[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      raw[i] = dout[(size_t)t * nch + (c < nch ? c : nch - 1)];
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      if constexpr (MAXC <= 4) pin(raw[i]);
      Chunk<T>::unpack(raw[i], dv[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
#pragma unroll
    for (int q = 0; q < CN; ++q) dv[i][q] = lane + 64 * i < nch ? dv[i][q] : 0.f;
  for (int k = 0; k < K; ++k) {
    const int r = row_of_pair[(size_t)t * K + k];
    if (r < 0 || r >= T_ * K) {
      if (lane == 0) dgates[(size_t)t * K + k] = 0.f;
      continue;
    }
    const float g = gates[(size_t)t * K + k];
    // y's row: the dispatched row, or (pairs) the pair's own row
    const size_t yr = pairs ? (size_t)t * K + k : (size_t)r;
    float dot = 0.f;
    if constexpr (MAXC <= 4) {
      // the row's chunks are loaded together (clamped indices), then used in
      // chunk order
      uint4 yv[MAXC];
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = lane + 64 * i;
        yv[i] = load_nt(&yp[yr * nch + (c < nch ? c : nch - 1)]);
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) pin(yv[i]);
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
          float y[CN], o[CN];
          Chunk<T>::unpack(yv[i], y);
#pragma unroll
          for (int q = 0; q < CN; ++q) {
            dot = fmaf(dv[i][q], y[q], dot);
            o[q] = g * dv[i][q];
          }
          if constexpr (WRITE_DYP) dyp[(size_t)r * nch + c] = Chunk<T>::pack(o);
        }
      }
    } else {
      // wide rows: the dout row already fills the registers
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
          float y[CN], o[CN];
          Chunk<T>::unpack(load_nt(&yp[yr * nch + c]), y);
#pragma unroll
          for (int q = 0; q < CN; ++q) {
            dot = fmaf(dv[i][q], y[q], dot);
            o[q] = g * dv[i][q];
          }
          if constexpr (WRITE_DYP) dyp[(size_t)r * nch + c] = Chunk<T>::pack(o);
        }
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) dgates[(size_t)t * K + k] = dot;
  }
}

template <typename T, int MAXC>
static void combine_bwd_t(const moe_shape* s, const void* dout, const void* yp,
                          const float* gates, const int32_t* row_of_pair, void* dyp,
                          float* dgates, hipStream_t st, bool pairs) {
  if (dyp)
    MOE_LAUNCH("combine_bwd", st,
               (combine_bwd_kernel<T, MAXC, true><<<(unsigned)cdiv(s->T, 4), 256, 0, st>>>(
                   (const uint4*)dout, (const uint4*)yp, gates, row_of_pair, (uint4*)dyp, dgates,
                   (int)s->T, (int)s->K, row_chunks(s), pairs ? 1 : 0)));
  else
    MOE_LAUNCH("combine_bwd", st,
               (combine_bwd_kernel<T, MAXC, false><<<(unsigned)cdiv(s->T, 4), 256, 0, st>>>(
                   (const uint4*)dout, (const uint4*)yp, gates, row_of_pair, nullptr, dgates,
                   (int)s->T, (int)s->K, row_chunks(s), pairs ? 1 : 0)));
}

int launch_combine_bwd(const moe_shape* s, const void* dout, const void* yp, const float* gates,
                       const int32_t* row_of_pair, void* dyp, float* dgates, hipStream_t st,
                       bool pairs) {
  if (s->T == 0) return MOE_OK;
  const int nch = row_chunks(s);
  // d <= 16384: 16-bit rows <= 2048 chunks, f32 rows <= 4096 chunks
  if (s->dtype == MOE_BF16) {
    if (nch <= 256) combine_bwd_t<uint16_t, 4>(s, dout, yp, gates, row_of_pair, dyp, dgates, st, pairs);
    else combine_bwd_t<uint16_t, 32>(s, dout, yp, gates, row_of_pair, dyp, dgates, st, pairs);
  } else if (s->dtype == MOE_F16) {
    if (nch <= 256) combine_bwd_t<_Float16, 4>(s, dout, yp, gates, row_of_pair, dyp, dgates, st, pairs);
    else combine_bwd_t<_Float16, 32>(s, dout, yp, gates, row_of_pair, dyp, dgates, st, pairs);
  } else {
    if (nch <= 256) combine_bwd_t<float, 4>(s, dout, yp, gates, row_of_pair, dyp, dgates, st, pairs);
    else combine_bwd_t<float, 64>(s, dout, yp, gates, row_of_pair, dyp, dgates, st, pairs);
  }
  return check_launch("combine bwd");
}

// ---------------------------------------------------------------------------
// dispatch backward: dx[t] = [dx[t]] + [add[t]] + sum_k dxp[row(t,k)]
//                            [+ sum_k dlogits[t, e_k] * W_rT[e_k]]   (e_k = idx[t,k])
// float32 accumulation, one rounding.  One wave per token.
// ---------------------------------------------------------------------------
template <typename T, int MAXC>
__global__ __launch_bounds__(256) void dispatch_bwd_kernel(
    const uint4* __restrict__ dxp, const int32_t* __restrict__ row_of_pair,
    const int32_t* __restrict__ idx, const float* __restrict__ dlogits,
    const uint4* __restrict__ W_rT, const uint4* __restrict__ add, uint4* __restrict__ dx,
    int T_, int K, int E, int nch, int accumulate) {
  constexpr int CN = Chunk<T>::N;
  const int t = uniform_token((int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6));
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  LocalRows lr0;
  lr0.load(row_of_pair, t, K, T_ * K, lane);
  for (int c0 = 0; c0 < nch; c0 += 64 * MAXC) {
    int cc[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = c0 + lane + 64 * i;
      cc[i] = c < nch ? c : nch - 1;
    }
    float acc[MAXC][CN];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      if (accumulate) {  // uniform
        Chunk<T>::unpack(dx[(size_t)t * nch + cc[i]], acc[i]);
      } else {
#pragma unroll
        for (int q = 0; q < CN; ++q) acc[i][q] = 0.f;
      }
      if (add) {  // uniform: a token-aligned term (the shared expert's input gradient)
        float f[CN];
        Chunk<T>::unpack(add[(size_t)t * nch + cc[i]], f);
#pragma unroll
        for (int q = 0; q < CN; ++q) acc[i][q] += f[q];
      }
    }
    // two rows per pass, summed in ascending slot order
    LocalRows lr = lr0;
    while (!lr.empty()) {
      const int k0 = lr.next();
      const bool two = !lr.empty();
      const int k1 = two ? lr.next() : k0;
      const uint4* s0 = dxp + (size_t)lr.row(k0) * nch;
      const uint4* s1 = dxp + (size_t)lr.row(k1) * nch;
      uint4 v0[MAXC], v1[MAXC];
#pragma unroll
      for (int i = 0; i < MAXC; ++i) v0[i] = load_nt(&s0[cc[i]]);
#pragma unroll
      for (int i = 0; i < MAXC; ++i) v1[i] = load_nt(&s1[cc[i]]);
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        pin(v0[i]);
        pin(v1[i]);
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        float f[CN];
        Chunk<T>::unpack(v0[i], f);
#pragma unroll
        for (int q = 0; q < CN; ++q) acc[i][q] += f[q];
      }
      if (two) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          float f[CN];
          Chunk<T>::unpack(v1[i], f);
#pragma unroll
          for (int q = 0; q < CN; ++q) acc[i][q] += f[q];
        }
      }
    }
    if (dlogits) {
      // two slots per pass: both W_r rows are loaded before the first FMA;
      // the terms are still added in slot order, and a slot whose expert is
      // out of range is skipped (uniform: one token per wave)
      for (int k = 0; k < K; k += 2) {
        const int e0 = idx[(size_t)t * K + k];
        const int e1 = k + 1 < K ? idx[(size_t)t * K + k + 1] : -1;
        const bool ok0 = e0 >= 0 && e0 < E, ok1 = e1 >= 0 && e1 < E;
        const uint4* w0 = W_rT + (size_t)(ok0 ? e0 : 0) * nch;
        const uint4* w1 = W_rT + (size_t)(ok1 ? e1 : 0) * nch;
        uint4 wv0[MAXC], wv1[MAXC];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) wv0[i] = w0[cc[i]];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) wv1[i] = w1[cc[i]];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          pin(wv0[i]);
          pin(wv1[i]);
        }
        if (ok0) {
          const float gl = dlogits[(size_t)t * E + e0];
#pragma unroll
          for (int i = 0; i < MAXC; ++i) {
            float f[CN];
            Chunk<T>::unpack(wv0[i], f);
#pragma unroll
            for (int q = 0; q < CN; ++q) acc[i][q] = fmaf(gl, f[q], acc[i][q]);
          }
        }
        if (ok1) {
          const float gl = dlogits[(size_t)t * E + e1];
#pragma unroll
          for (int i = 0; i < MAXC; ++i) {
            float f[CN];
            Chunk<T>::unpack(wv1[i], f);
#pragma unroll
            for (int q = 0; q < CN; ++q) acc[i][q] = fmaf(gl, f[q], acc[i][q]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = c0 + lane + 64 * i;
      if (c < nch) dx[(size_t)t * nch + c] = Chunk<T>::pack(acc[i]);
    }
  }
}

template <typename T>
static void dispatch_bwd_t(const moe_shape* s, const void* dxp, const int32_t* row_of_pair,
                           const int32_t* idx, const float* dlogits, const void* W_rT,
                           const void* add, void* dx, bool accumulate, hipStream_t st) {
  MOE_LAUNCH("dispatch_bwd", st,
             dispatch_bwd_kernel<T, 4><<<(unsigned)cdiv(s->T, 4), 256, 0, st>>>(
                 (const uint4*)dxp, row_of_pair, idx, dlogits, (const uint4*)W_rT,
                 (const uint4*)add, (uint4*)dx, (int)s->T, (int)s->K, (int)s->E, row_chunks(s),
                 accumulate ? 1 : 0));
}

int launch_dispatch_bwd(const moe_shape* s, const void* dxp, const int32_t* row_of_pair,
                        const int32_t* idx, const float* dlogits, const void* W_rT,
                        const void* add, void* dx, bool accumulate, hipStream_t st) {
  if (s->T == 0) return MOE_OK;
  if (s->dtype == MOE_BF16)
    dispatch_bwd_t<uint16_t>(s, dxp, row_of_pair, idx, dlogits, W_rT, add, dx, accumulate, st);
  else if (s->dtype == MOE_F16)
    dispatch_bwd_t<_Float16>(s, dxp, row_of_pair, idx, dlogits, W_rT, add, dx, accumulate, st);
  else
    dispatch_bwd_t<float>(s, dxp, row_of_pair, idx, dlogits, W_rT, add, dx, accumulate, st);
  return check_launch("dispatch bwd");
}

}  // namespace moe
