// Grouped expert GEMMs in bf16 or fp16 on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16 / _f16, float32 accumulation), with the SwiGLU forward and backward fused into the
// epilogues.  These are the "expert FFN compute" that the expert-parallel
// overlap pages hide the token exchange behind (skill card page 1, "What it
// is"), split into activation gradient (dgrad, D) and weight gradient (wgrad,
// W) as the 1F1B note describes (page 2, "MoE 1F1B overlap").
//
// Structure shared by every kernel here:
//  * persistent grid (one block per CU); the tiles are split into eight
//    contiguous ranges, one per XCD (the hardware places block b on XCD b % 8),
//    so the tiles running together on an XCD share A rows and expert weights
//    in its L2, and the ranges stay balanced whatever the device-side tile count;
//  * block tile 256 x 256, K step 64, 8 waves (2 per SIMD), each owning a
//    128 x 64 piece as 4 x 2 MFMA 32x32 tiles;
//  * two LDS stages fed through registers: the register stage is written to
//    the free LDS buffer over the first three k slices of a step, each chunk's
//    store followed by the load of the same chunk two stages ahead;
//  * LDS tiles are [rows][64] bf16 with the 16-byte chunk index XOR-swizzled
//    by the row, so matrix-core fragment reads are free of bank conflicts;
//  * the MFMA fragments of the next 16-wide k slice are read while the current
//    slice's MFMAs run (across the stage barrier too), and the instruction
//    order (MFMA / LDS read / LDS write / global load) is fixed per slice with
//    scheduling group barriers, the slices fenced from each other, so the
//    matrix pipe is fed continuously;
//  * loads are branch free: rows or columns outside the matrix read a valid
//    clamped address (their results are discarded, or replaced by zero where
//    they would enter a sum);
//  * operands contiguous along K are copied 16 bytes at a time; dgrad reads
//    its weights from K-contiguous transposed copies made at the start of the
//    call; wgrad, whose operands are contiguous along M/N, stages natural-layout
//    tiles in LDS and transposes on the fragment read (see wgrad_kernel).
// Row-grouped GEMMs (fwd, dgrad) take their (expert, M-tile) from the dispatch
// plan's tile_offsets (tiles of kTileM rows).
#include "moe_internal.h"

#include <type_traits>

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 16-bit element types of the matrix-core path.  Operands travel as raw 16-bit
// patterns (global -> LDS -> registers); only the MFMA and the epilogue's
// conversions depend on the type.
struct BF16 {
  typedef uint16_t elt;  // Chunk<uint16_t> converts bf16
  static __device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
struct F16 {
  typedef _Float16 elt;
  static __device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

constexpr int BK = 64;

// scheduling group masks (instruction classes)
constexpr int SG_MFMA = 0x008, SG_VMEM_R = 0x020, SG_DS_R = 0x100, SG_DS_W = 0x200;
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

// Element offset of 16-byte chunk `ch` (0..7) of row `row` of an LDS tile.
__device__ __forceinline__ int lds_off(int row, int ch) {
  const int s = (row & 7) ^ ((row >> 3) & 1);
  return row * BK + ((ch ^ s) << 3);
}

// Operand contiguous along K: R rows x 64 k per stage, 16-byte chunks, read
// with buffer loads: the operand base is a wave-uniform buffer resource
// (scalar registers), each chunk a 32-bit byte offset in one vector register,
// and the k position the scalar offset.  row_off(r) gives the element offset
// from the base of element k = 0 of tile row r (rows outside the matrix are
// clamped by the caller to valid ones); offsets stay below 2^31 bytes.  K is
// a multiple of 64.
template <int R, int NT>
struct LoadK {
  static constexpr int CH = R * 8 / NT;
  static constexpr int NLOAD = CH, NSTORE = CH;
  static_assert(CH >= 1 && (R * 8) % NT == 0, "tile/threads mismatch");
  // Chunk c of this thread is row c*NT/8 + tid/8, chunk tid%8; with NT a
  // multiple of 128 the swizzle of those rows does not depend on c, so the
  // LDS offsets are one register plus constants.
  static_assert(NT % 128 == 0, "LDS offsets assume NT % 128 == 0");
  static constexpr int DSTEP = NT / 8 * BK;
  u32x4_t v[CH];  // the stage in flight
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[CH];  // bytes
  int dst0;
  template <class RowOff>
  __device__ __forceinline__ void init(const uint16_t* base, RowOff row_off, int tid) {
    // raw buffer (stride 0); the records limit is never reached: every
    // offset is a valid element of the operand
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int c = 0; c < CH; ++c)
      off[c] = (uint32_t)row_off(c * (NT / 8) + (tid >> 3)) * 2u + (uint32_t)(tid & 7) * 16u;
    dst0 = lds_off(tid >> 3, tid & 7);
  }
  __device__ __forceinline__ void load(int k0, int /*k_end*/) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
      v[c] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off[c], k0 * 2, 0);
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int c = 0; c < CH; ++c) *(u32x4_t*)(lds + dst0 + c * DSTEP) = v[c];
  }
  __device__ __forceinline__ void load_c(int c, int k0) {
    v[c] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off[c], k0 * 2, 0);
  }
  __device__ __forceinline__ void store_c(int c, uint16_t* lds) const {
    *(u32x4_t*)(lds + dst0 + c * DSTEP) = v[c];
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
using T256 = Tile<256, 256, 2, 4>;

// Output element held by accumulator register r of 32x32 tile (i, j) in this
// lane: row = wave_row0 + i*32 + out_row(lane, r), col = wave_col0 + j*32 + lane%32.
__device__ __forceinline__ int out_row(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Epilogue staging: the 32 x 64 accumulator block acc[i][2p], acc[i][2p+1]
// of a wave is written to the wave's own LDS area, row-major with EP_LD floats
// per row, and read back by rows, so that the epilogues' global accesses are
// 16 bytes per lane and whole rows per group of lanes: in pass q (0..3) lane l
// takes row 8q + l/8, columns 8(l%8)..+8, and one store instruction writes
// eight 128-byte rows.  The LDS must be free (the main loop ends with a
// barrier); the caller synchronises before the next tile writes it.  LDS
// operations of one wave complete in order, so a lane may read what other
// lanes of its wave wrote just before.
constexpr int EP_LD = 68;  // 64 + 4 floats per staged row
template <class TL>
__device__ __forceinline__ const float* stage_rows(const f32x16_t (&acc)[TL::TM][TL::TN], int i,
                                                   int p, uint16_t* smem, int wave, int lane) {
  static_assert(TL::TN % 2 == 0, "staged blocks are 64 columns wide");
  static_assert(TL::NT / 64 * 32 * EP_LD * 4 <= TL::LDS_ELEMS * 2, "staging exceeds the LDS");
  float* reg = reinterpret_cast<float*>(smem) + wave * 32 * EP_LD;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      reg[out_row(lane, r) * EP_LD + j * 32 + (lane & 31)] = acc[i][2 * p + j][r];
  return reg;
}

// Eight consecutive staged floats.
__device__ __forceinline__ void ld8(const float* p, float* f) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Staged row of pass q for this lane, and its 8-column chunk.
__device__ __forceinline__ int st_row(int q, int lane) { return q * 8 + (lane >> 3); }
__device__ __forceinline__ int st_col(int lane) { return (lane & 7) * 8; }

// Store a staged 32 x 64 block as bf16 rows: out_row0 points at column 0 of
// the block's first row, ld is the row stride, rows at or past n_rows are
// skipped.
template <class E>
__device__ __forceinline__ void store_block(const float* blk, uint16_t* out_row0, size_t ld,
                                            int n_rows, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = st_row(q, lane), c = st_col(lane);
    float f[8];
    ld8(blk + r * EP_LD + c, f);
    if (r < n_rows) *(uint4*)(out_row0 + r * ld + c) = Chunk<typename E::elt>::pack(f);
  }
}

// The same with the staged rows scattered: row r of the block goes to row
// dst[q] of out (out points at the block's first column), where q is the
// pass that holds r for this lane (r = st_row(q, lane)).
template <class E>
__device__ __forceinline__ void store_block_rows(const float* blk, uint16_t* out, size_t ld,
                                                 const int (&dst)[4], int n_rows, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = st_row(q, lane), c = st_col(lane);
    float f[8];
    ld8(blk + r * EP_LD + c, f);
    if (r < n_rows) *(uint4*)(out + (size_t)dst[q] * ld + c) = Chunk<typename E::elt>::pack(f);
  }
}

template <class TL>
struct Frags {
  bf16x8_t a[TL::TM], b[TL::TN];
};

// B fragments first: the first MFMA of a slice needs a[0] and b[0], so with
// B read first it waits for the third read instead of the fifth.
template <class TL>
__device__ __forceinline__ void read_frags(Frags<TL>& f, const uint16_t* A, const uint16_t* B,
                                           int kk, int wm, int wn, int lane) {
  const int fr = lane & 31, ch = kk * 2 + (lane >> 5);
#pragma unroll
  for (int j = 0; j < TL::TN; ++j)
    f.b[j] = *(const bf16x8_t*)(B + lds_off(wn * TL::WTN + j * 32 + fr, ch));
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
    f.a[i] = *(const bf16x8_t*)(A + lds_off(wm * TL::WTM + i * 32 + fr, ch));
}

template <class TL, class E, bool NSIDE = false>
__device__ __forceinline__ void mfmas(const Frags<TL>& f, f32x16_t (&acc)[TL::TM][TL::TN]) {
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j)
      acc[i][j] = NSIDE ? E::mfma(f.b[j], f.a[i], acc[i][j]) : E::mfma(f.a[i], f.b[j], acc[i][j]);
}

// Stage tiles in natural [64 k][256 col] layout (the wgrad operands, which
// are contiguous along M/N while the reduction runs over rows): the MFMA
// operands, 8 consecutive k of one column per lane, are assembled from two
// LDS transpose reads (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane s addresses row k0 + s/4 at columns c0 + 4*(s%4), and lane t receives
// rows k0..k0+3 of column c0 + t.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int WG_ROWB = 256 * 2;  // bytes per natural-layout tile row (256 columns)

// Physical 32-byte chunk of logical chunk c in tile row k: rows k..k+3 of a
// transpose read land in distinct bank groups.
__device__ __forceinline__ int wg_swz(int k) { return ((k & 3) << 1) | ((k >> 2) & 1); }
__device__ __forceinline__ int wg_byte(int k, int col) {
  return k * WG_ROWB + ((((col >> 4) ^ wg_swz(k)) & 15) << 5) + ((col & 15) << 1);
}

// Fragment readers of the main loop.  RowFrags: tiles [rows][64 k] (operands
// contiguous along K), one 16-byte LDS read per MFMA operand.
struct RowFrags {
  static constexpr int READS = 1;       // LDS read instructions per fragment
  static constexpr bool NSIDE = false;  // the MFMA takes the M-side fragment first
  template <class TL>
  __device__ __forceinline__ void read(Frags<TL>& f, const uint16_t* A, const uint16_t* B, int kk,
                                       int wm, int wn, int lane) const {
    read_frags<TL>(f, A, B, kk, wm, wn, lane);
  }
};
// TrFrags: natural-layout tiles read by transpose.  With g = lane / 16 and
// t = lane % 16, half h of the operand for columns [cb, cb + 32) (cb a
// multiple of 32) reads tile row kr = 8 (g / 2) + t / 4 + 4h at physical
// 32-byte chunk ((cb / 16 + g % 2) ^ wg_swz(kr)) and byte 8 (t % 4) in it;
// wg_swz(kr) = 2 (t / 4) + h is below 8 and cb / 16 is even, so the chunk is
// (cb / 16) ^ u_h with the per-lane u_h = (g % 2) ^ wg_swz(kr): each read
// costs one XOR of a block-uniform value with u_h and one shift-add onto the
// per-lane row base.  With HOIST the twelve resulting addresses are left to
// the compiler, which keeps them in registers across the main loop (fewer
// instructions per slice); without, they are formed at each read, which needs
// twelve registers fewer.  The MFMA takes the N-side fragment first, so a
// block of four accumulator registers holds four consecutive columns of one
// output row.
template <class TL, bool HOIST>
struct TrFrags {
  static constexpr int READS = 2;
  static constexpr bool NSIDE = true;
  int rb[2], u[2];  // per half: row byte base + 8 (t % 4), chunk XOR term
  int wm, wn;
  __device__ __forceinline__ static void terms(int lane, int (&r)[2], int (&x)[2]) {
    const int g = lane >> 4, t = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kr = ((g >> 1) << 3) + (t >> 2) + 4 * h;
      r[h] = kr * WG_ROWB + ((t & 3) << 3);
      x[h] = (g & 1) ^ wg_swz(kr);
    }
  }
  __device__ __forceinline__ void init(int wm_, int wn_, int lane) {
    wm = wm_;
    wn = wn_;
    if constexpr (HOIST) terms(lane, rb, u);
  }
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int cb, int kk,
                                                  const int (&rb)[2], const int (&u)[2]) {
    const uint8_t* t8 = (const uint8_t*)tile + kk * 16 * WG_ROWB;
    const int c16 = cb >> 4;  // block-uniform
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(t8 + rb[0] + ((c16 ^ u[0]) << 5)));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(t8 + rb[1] + ((c16 ^ u[1]) << 5)));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
  template <class>
  __device__ __forceinline__ void read(Frags<TL>& f, const uint16_t* A, const uint16_t* B, int kk,
                                       int, int, int) const {
    // without HOIST the per-lane terms are recomputed here from the lane
    // index, made opaque by an empty asm, so neither they nor the addresses
    // occupy registers across the main loop
    int r[2] = {rb[0], rb[1]}, x[2] = {u[0], u[1]};
    if constexpr (!HOIST) {
      int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      asm volatile("" : "+v"(lane));
      terms(lane, r, x);
    }
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) f.b[j] = frag(B, wn * TL::WTN + j * 32, kk, r, x);
#pragma unroll
    for (int i = 0; i < TL::TM; ++i) f.a[i] = frag(A, wm * TL::WTM + i * 32, kk, r, x);
  }
};

// Wave position inside the block tile.  The wave index is moved to a scalar
// register and the lane index is recomputed where it is needed (from the exec
// mask count, made opaque to the optimiser), so addresses derived from it are
// computed next to their use instead of being hoisted out of the tile loop
// and held in vector registers across the main loop.
struct WavePos {
  int lane, wave, wm, wn;
  template <class TL>
  __device__ __forceinline__ static WavePos of() {
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    return {l, w, w / TL::WGN, w % TL::WGN};
  }
};

// Two-stage LDS main loop, steps of 64 k from k_begin, once stage 0 is in LDS
// buffer 0 (published by a barrier) and the loads of stage 1 are in the
// loaders' registers.  The registers hold the stage after the one being
// written to LDS: in step kt, stage kt+1 goes from registers to LDS and the
// loads of stage kt+2 are issued right behind it, so a load has four k slices
// to arrive.  Loads past the last stage re-read it (harmless), so the loop
// body has no branches.  Ends with a barrier: the LDS is free on return.
// One k slice with W chunk stores and V chunk loads: each MFMA is followed by
// up to two LDS reads of the next slice; once the reads are all issued, each
// MFMA is followed by one store and one load (reads first, so the next
// slice's MFMAs do not wait behind the stores in the in-order LDS counter).
template <int NM, int NR, int W, int V>
__device__ __forceinline__ void sched_slice_wv() {
  constexpr int RM = (NR + 1) / 2;  // MFMAs that carry reads
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    SCHED_GROUP(SG_MFMA, 1);
    if (2 * i < NR) SCHED_GROUP(SG_DS_R, 1);
    if (2 * i + 1 < NR) SCHED_GROUP(SG_DS_R, 1);
    if (i >= RM && i - RM < W) SCHED_GROUP(SG_DS_W, 1);
    if (i >= RM && i - RM < V) SCHED_GROUP(SG_VMEM_R, 1);
  }
}

// Store chunks [Q0, Q1) of the register stage (A chunks first, then B) to
// LDS, each followed by the load of the same chunk of the stage after.
template <int Q0, int Q1, class LA, class LB>
__device__ __forceinline__ void store_load(LA& la, LB& lb, uint16_t* An, uint16_t* Bn, int kn) {
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    if (q < LA::CH) {
      la.store_c(q, An);
      la.load_c(q, kn);
    } else {
      lb.store_c(q - LA::CH, Bn);
      lb.load_c(q - LA::CH, kn);
    }
  }
}

template <class TL, class E, class LA, class LB, bool SCHED = true, class FR = RowFrags>
__device__ __forceinline__ void mainloop_steps(LA& la, LB& lb, int k_begin, int nk,
                                               uint16_t* smem, f32x16_t (&acc)[TL::TM][TL::TN],
                                               const FR& fr = FR{}) {
  uint16_t* const sA0 = smem;
  uint16_t* const sA1 = smem + TL::BM * BK;
  uint16_t* const sB0 = smem + 2 * TL::BM * BK;
  uint16_t* const sB1 = sB0 + TL::BN * BK;
  const WavePos w = WavePos::of<TL>();
  const int lane = w.lane, wm = w.wm, wn = w.wn;
#pragma unroll
  for (int i = 0; i < TL::TM; ++i)
#pragma unroll
    for (int j = 0; j < TL::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  constexpr int NM = TL::TM * TL::TN, NR = (TL::TM + TL::TN) * FR::READS;
  constexpr int NQ = LA::CH + LB::CH;  // chunks per stage, spread over slices 0..2
  constexpr int Q1 = NQ / 3, Q2 = 2 * NQ / 3;
  Frags<TL> f0, f1;
  fr.template read<TL>(f0, sA0, sB0, 0, wm, wn, lane);
  for (int kt = 0; kt < nk; ++kt) {
    const bool odd = kt & 1;
    const uint16_t* A = odd ? sA1 : sA0;
    const uint16_t* B = odd ? sB1 : sB0;
    uint16_t* An = odd ? sA0 : sA1;
    uint16_t* Bn = odd ? sB0 : sB1;
    const int kn2 = k_begin + (kt + 2 < nk ? kt + 2 : nk - 1) * BK;
    // slice 0; the other buffer's last readers passed the previous barrier,
    // so the stage in registers can go to it from here on
    fr.template read<TL>(f1, A, B, 1, wm, wn, lane);
    mfmas<TL, E, FR::NSIDE>(f0, acc);
    store_load<0, Q1>(la, lb, An, Bn, kn2);
    if constexpr (SCHED) sched_slice_wv<NM, NR, Q1, Q1>();
    __builtin_amdgcn_sched_barrier(0);
    // slice 1
    fr.template read<TL>(f0, A, B, 2, wm, wn, lane);
    mfmas<TL, E, FR::NSIDE>(f1, acc);
    store_load<Q1, Q2>(la, lb, An, Bn, kn2);
    if constexpr (SCHED) sched_slice_wv<NM, NR, Q2 - Q1, Q2 - Q1>();
    __builtin_amdgcn_sched_barrier(0);
    // slice 2
    fr.template read<TL>(f1, A, B, 3, wm, wn, lane);
    mfmas<TL, E, FR::NSIDE>(f0, acc);
    store_load<Q2, NQ>(la, lb, An, Bn, kn2);
    if constexpr (SCHED) sched_slice_wv<NM, NR, NQ - Q2, NQ - Q2>();
    __builtin_amdgcn_sched_barrier(0);
    // the next stage is complete once every wave passes the barrier; its
    // first fragments are read while the last slice's MFMAs run
    __syncthreads();
    fr.template read<TL>(f0, An, Bn, 0, wm, wn, lane);
    mfmas<TL, E, FR::NSIDE>(f1, acc);
    if constexpr (SCHED) sched_slice_wv<NM, NR, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();  // LDS free for the caller's epilogue / next tile
}

// The whole main loop over k in [k_begin, k_end) (a multiple of 64 long)
// for a tile whose loaders are initialised: stage 0 to LDS, stage 1 to
// registers, then the steps.
template <class TL, class E, class LA, class LB>
__device__ __forceinline__ void mainloop(LA& la, LB& lb, int k_begin, int k_end,
                                         uint16_t* smem, f32x16_t (&acc)[TL::TM][TL::TN]) {
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) {  // block-uniform
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int j = 0; j < TL::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    return;
  }
  la.load(k_begin, k_end);
  lb.load(k_begin, k_end);
  la.store(smem);
  lb.store(smem + 2 * TL::BM * BK);
  const int k1 = k_begin + (nk > 1 ? 1 : 0) * BK;
  la.load(k1, k_end);
  lb.load(k1, k_end);
  __syncthreads();
  mainloop_steps<TL, E>(la, lb, k_begin, nk, smem, acc);
}

// Persistent schedule: the blocks form G = min(8, grid) groups by block % G
// (with G = 8 a group is one XCD); group g owns tiles [g*total/G, (g+1)*total/G),
// handed out to its blocks round robin.  Every group has at least one block,
// so every tile is processed.
struct Sched {
  int t, end, step;
  __device__ __forceinline__ explicit Sched(int total) {
    const int nb = gridDim.x, G = nb < 8 ? nb : 8;
    const int g = blockIdx.x % G, slot = blockIdx.x / G;
    t = (int)((long)total * g / G) + slot;
    end = (int)((long)total * (g + 1) / G);
    step = (nb - g + G - 1) / G;
  }
};

// (expert, first row, row end) of M-tile mt from LDS copies of tile_offsets/offsets.
__device__ __forceinline__ void row_tile(const int* s_to, const int* s_off, int E_l, int mt,
                                         int& e, int& m0, int& m_end) {
  int lo = 0, hi = E_l;  // s_to[lo] <= mt < s_to[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_to[mid] <= mt) lo = mid;
    else hi = mid;
  }
  e = lo;
  m0 = s_off[lo] + (mt - s_to[lo]) * kTileM;
  m_end = s_off[lo + 1];
}
// The same, moved to scalar registers (the values are block-uniform), so the
// operand bases built from them are scalar.
__device__ __forceinline__ void uniform_row_tile(const int* s_to, const int* s_off, int E_l,
                                                 int mt, int& e, int& m0, int& m_end) {
  row_tile(s_to, s_off, E_l, mt, e, m0, m_end);
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  m_end = __builtin_amdgcn_readfirstlane(m_end);
}

// Whether an Op's epilogue takes destination rows loaded before it (ROWS).
template <class Op, class = void>
struct OpRows {
  static constexpr bool value = false;
};
template <class Op>
struct OpRows<Op, std::void_t<decltype(Op::ROWS)>> {
  static constexpr bool value = Op::ROWS;
};

// ---------------------------------------------------------------------------
// Row-grouped GEMM (forward and dgrad): M tiles follow the dispatch plan, N
// tiles are fixed.  Op supplies the loaders (init), the K extent (k_len) and
// the epilogue.  Tiles are software-pipelined across the persistent loop: the
// first two stages of the next tile are loaded before the epilogue of the
// current one issues its stores, so the next main loop does not wait for
// those stores to complete (the vector memory counter retires in order).
// ---------------------------------------------------------------------------
template <class TL, class Op>
__global__ __launch_bounds__(TL::NT) void row_grouped_kernel(Op op,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ tile_offsets,
                                                             int E_l, int n_tiles) {
  static_assert(TL::BM == kTileM, "row tiles come from the dispatch plan");
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  __shared__ int s_to[257], s_off[257];
  for (int j = threadIdx.x; j <= E_l; j += blockDim.x) {
    s_to[j] = tile_offsets[j];
    s_off[j] = offsets[j];
  }
  __syncthreads();
  Sched sc(s_to[E_l] * n_tiles);
  if (sc.t >= sc.end) return;  // block-uniform
  const int tid = threadIdx.x;
  const int nk = (op.k_len() + BK - 1) / BK;  // >= 1: K is a positive multiple of 64
  const int k1 = (nk > 1 ? 1 : 0) * BK;
  LoadK<TL::BM, TL::NT> la;
  LoadK<TL::BN, TL::NT> lb;
  int e, m0, m_end, nt = sc.t % n_tiles;
  uniform_row_tile(s_to, s_off, E_l, sc.t / n_tiles, e, m0, m_end);
  op.template init<TL>(e, m0, m_end, nt, la, lb, tid);
  la.load(0, 0);
  lb.load(0, 0);
  for (;;) {
    la.store(smem);
    lb.store(smem + 2 * TL::BM * BK);
    la.load(k1, 0);
    lb.load(k1, 0);
    __syncthreads();
    f32x16_t acc[TL::TM][TL::TN];
    mainloop_steps<TL, typename Op::Elt>(la, lb, 0, nk, smem, acc);
    const int ce = e, cm0 = m0, cm_end = m_end, cnt = nt;
    // an epilogue that scatters its rows loads their destinations now, ahead
    // of the next tile's loads (the memory counter retires in order)
    int dst[OpRows<Op>::value ? TL::TM : 1][4];
    if constexpr (OpRows<Op>::value) op.template dest_rows<TL>(cm0, cm_end, dst);
    sc.t += sc.step;
    const bool more = sc.t < sc.end;  // block-uniform
    if (more) {
      nt = sc.t % n_tiles;
      uniform_row_tile(s_to, s_off, E_l, sc.t / n_tiles, e, m0, m_end);
      op.template init<TL>(e, m0, m_end, nt, la, lb, tid);
      la.load(0, 0);
      lb.load(0, 0);
    }
    if constexpr (OpRows<Op>::value) op.template epilogue<TL>(acc, ce, cm0, cm_end, cnt, smem, dst);
    else op.template epilogue<TL>(acc, ce, cm0, cm_end, cnt, smem);
    __syncthreads();  // epilogue staging done before the next tile's stage 0 lands in LDS
    if (!more) break;
  }
}


// forward GEMM1: [g, u] = xp . W_gu[e]^T with the SwiGLU epilogue.  The B tile
// pairs gate and up rows: every 64 tile rows are 32 gate rows j and the 32 up
// rows F + j of the same j, so a staged 64-column block holds g and u of 32
// outputs.
//
// With xrows set, the permute is fused into the A loads: xp is the token
// matrix x [T][d] and dispatched row r reads token xrows[r] / K (xrows is the
// dispatch plan's pair_of_row), so the permuted copy of x is never written.
template <class E>
struct GateUpOp {
  typedef E Elt;
  const uint16_t* xp;
  const uint16_t* W_gu;
  uint16_t* h;
  uint16_t* a;
  int d, F;
  const int32_t* xrows;
  int K;
  __device__ __forceinline__ int k_len() const { return d; }
  template <class TL, class LA, class LB>
  __device__ __forceinline__ void init(int e, int m0, int m_end, int nt, LA& la, LB& lb,
                                       int tid) const {
    const int jb = nt * (TL::BN / 2);
    const uint16_t* Wg = W_gu + (size_t)e * 2 * F * d;
    if (xrows)  // block-uniform
      la.init(xp, [&](int r) { return xrows[min(m0 + r, m_end - 1)] / K * d; }, tid);
    else
      la.init(xp + (size_t)m0 * d, [&](int r) { return (min(m0 + r, m_end - 1) - m0) * d; },
              tid);
    lb.init(Wg, [&](int n) {
      const int j = min(jb + (n >> 6) * 32 + (n & 31), F - 1);
      return (((n >> 5) & 1) * F + j) * d;
    }, tid);
  }
  // staged block p: columns 0..31 gate, 32..63 up of the 32 outputs starting
  // at jb + (wn*TN/2 + p)*32; in pass q a lane takes row 16q + l/4 and
  // outputs 8(l%4)..+8 (four lanes cover a row's 64 bytes of each output)
  template <class TL>
  __device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TL::TM][TL::TN], int e, int m0,
                                           int m_end, int nt, uint16_t* smem) const {
    const WavePos w = WavePos::of<TL>();
    const int jb = nt * (TL::BN / 2);
#pragma unroll
    for (int p = 0; p < TL::TN / 2; ++p) {
      const int j0 = jb + (w.wn * (TL::TN / 2) + p) * 32 + (w.lane & 3) * 8;
      const bool col_ok = j0 < F;  // F is a multiple of 64
#pragma unroll
      for (int i = 0; i < TL::TM; ++i) {
        const float* blk = stage_rows<TL>(acc, i, p, smem, w.wave, w.lane);
        const int rb = m0 + w.wm * TL::WTM + i * 32;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int r = q * 16 + (w.lane >> 2);
          float g[8], u[8], av[8];
          ld8(blk + r * EP_LD + (w.lane & 3) * 8, g);
          ld8(blk + r * EP_LD + 32 + (w.lane & 3) * 8, u);
#pragma unroll
          for (int t = 0; t < 8; ++t) av[t] = silu_fast(g[t]) * u[t];
          if (col_ok && rb + r < m_end) {
            const size_t row = (size_t)(rb + r);
            *(uint4*)(h + row * 2 * F + j0) = Chunk<typename E::elt>::pack(g);
            *(uint4*)(h + row * 2 * F + F + j0) = Chunk<typename E::elt>::pack(u);
            *(uint4*)(a + row * F + j0) = Chunk<typename E::elt>::pack(av);
          }
        }
      }
    }
  }
};

// forward GEMM2: y_p = a . W_down[e]^T  (A: a rows, K = F; B: W_down rows, K = F)
//
// SCATTER: the epilogue writes dispatched row r of the product to row
// yrows[r] of yp (yrows is the plan's pair_of_row), so y is laid out by
// (token, slot) pair, and the combine and its backward read a token's K rows
// as one contiguous run.
template <class E, bool SCATTER = false>
struct DownOp {
  typedef E Elt;
  static constexpr bool ROWS = SCATTER;
  const uint16_t* a;
  const uint16_t* W_down;
  uint16_t* yp;
  int d, F;
  const int32_t* yrows;
  // SCATTER: destination row of each staged row this lane stores, per 32-row
  // block i of the wave (rows past the expert's end clamp to its last row)
  template <class TL, int R>
  __device__ __forceinline__ void dest_rows(int m0, int m_end, int (&dst)[R][4]) const {
    const WavePos w = WavePos::of<TL>();
#pragma unroll
    for (int i = 0; i < TL::TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[i][q] = yrows[min(m0 + w.wm * TL::WTM + i * 32 + st_row(q, w.lane), m_end - 1)];
  }
  __device__ __forceinline__ int k_len() const { return F; }
  template <class TL, class LA, class LB>
  __device__ __forceinline__ void init(int e, int m0, int m_end, int nt, LA& la, LB& lb,
                                       int tid) const {
    const int nb = nt * TL::BN;
    const uint16_t* Wd = W_down + (size_t)e * d * F;
    la.init(a + (size_t)m0 * F, [&](int r) { return (min(m0 + r, m_end - 1) - m0) * F; }, tid);
    lb.init(Wd, [&](int n) { return min(nb + n, d - 1) * F; }, tid);
  }
  template <class TL, int R = 1>
  __device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TL::TM][TL::TN], int e, int m0,
                                           int m_end, int nt, uint16_t* smem,
                                           const int (&dst)[R][4] = {}) const {
    const WavePos w = WavePos::of<TL>();
#pragma unroll
    for (int p = 0; p < TL::TN / 2; ++p) {
      const int cb = nt * TL::BN + w.wn * TL::WTN + p * 64;
      if (cb >= d) continue;  // d is a multiple of 64; wave-uniform
#pragma unroll
      for (int i = 0; i < TL::TM; ++i) {
        const int rb = m0 + w.wm * TL::WTM + i * 32;
        const float* blk = stage_rows<TL>(acc, i, p, smem, w.wave, w.lane);
        if constexpr (SCATTER) {
          static_assert(R == TL::TM, "one row set per 32-row block");
          store_block_rows<E>(blk, yp + cb, (size_t)d, dst[i], m_end - rb, w.lane);
        } else {
          store_block<E>(blk, yp + (size_t)rb * d + cb, (size_t)d, m_end - rb, w.lane);
        }
      }
    }
  }
};

// dgrad GEMM A: da = dy_p . W_down[e]  (A: dy_p rows, K = d; B: W_down[e]
// transposed, W_downT[e] [F][d], K-contiguous) with the SwiGLU backward epilogue.
//
// With FUSED (the fused combine backward), dy_p is never materialised:
// dyp is the token matrix dout [T][d], dispatched row r of the A operand is
// token xrows[r] / K (xrows is the plan's pair_of_row), and the gate of the
// row, gates[xrows[r]], scales the float32 product in the epilogue, so
// da = g . (dout . W_down[e]).  The epilogue then also writes
// ag = g . silu(g_h) . u_h from the stored h, the operand that takes the
// gate into the dW_down product of the weight gradient.
template <class E, bool FUSED = false>
struct DgradActOp {
  typedef E Elt;
  const uint16_t* dyp;
  const uint16_t* hbuf;
  const uint16_t* W_downT;
  uint16_t* dh;
  int d, F;
  const int32_t* xrows;
  int K;
  const float* gates;
  uint16_t* ag;
  __device__ __forceinline__ int k_len() const { return d; }
  template <class TL, class LA, class LB>
  __device__ __forceinline__ void init(int e, int m0, int m_end, int nt, LA& la, LB& lb,
                                       int tid) const {
    const int nb = nt * TL::BN;
    const uint16_t* WdT = W_downT + (size_t)e * F * d;
    if constexpr (FUSED)
      la.init(dyp, [&](int r) { return xrows[min(m0 + r, m_end - 1)] / K * d; }, tid);
    else
      la.init(dyp + (size_t)m0 * d, [&](int r) { return (min(m0 + r, m_end - 1) - m0) * d; },
              tid);
    lb.init(WdT, [&](int n) { return min(nb + n, F - 1) * d; }, tid);
  }
  // The h chunks of this lane's rows (16 bytes each, rows clamped to valid
  // ones) are loaded one row block ahead: block 0's before the first block
  // is staged, and block i + 1's pass q into the registers that block i's
  // pass q has just consumed, so each load has a block's work to arrive.
  // FUSED: the gates of all the lane's rows are loaded first, the pair
  // indices of the rows together and then the gates together, so the
  // dependent loads cost two memory waits per tile.
  template <class TL>
  __device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TL::TM][TL::TN], int e, int m0,
                                           int m_end, int nt, uint16_t* smem) const {
    const WavePos w = WavePos::of<TL>();
    const int c = st_col(w.lane);
    float grow[FUSED ? TL::TM : 1][4];
    if constexpr (FUSED) {
      int pr[TL::TM][4];
#pragma unroll
      for (int i = 0; i < TL::TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pr[i][q] = xrows[min(m0 + w.wm * TL::WTM + i * 32 + st_row(q, w.lane), m_end - 1)];
#pragma unroll
      for (int i = 0; i < TL::TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) grow[i][q] = gates[pr[i][q]];
    }
#pragma unroll
    for (int p = 0; p < TL::TN / 2; ++p) {
      const int cb = nt * TL::BN + w.wn * TL::WTN + p * 64;
      if (cb >= F) continue;  // F is a multiple of 64; wave-uniform
      const int rb0 = m0 + w.wm * TL::WTM;
      uint4 gv[4], uv[4];
      auto load_h = [&](int i, int q) {
        const size_t rowc = (size_t)min(rb0 + i * 32 + st_row(q, w.lane), m_end - 1);
        gv[q] = *(const uint4*)(hbuf + rowc * 2 * F + cb + c);
        uv[q] = *(const uint4*)(hbuf + rowc * 2 * F + F + cb + c);
      };
#pragma unroll
      for (int q = 0; q < 4; ++q) load_h(0, q);
#pragma unroll
      for (int i = 0; i < TL::TM; ++i) {
        const int rb = rb0 + i * 32;
        const float* blk = stage_rows<TL>(acc, i, p, smem, w.wave, w.lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = st_row(q, w.lane);
          float da[8], g[8], u[8], dg[8], du[8], av[8];
          ld8(blk + r * EP_LD + c, da);
          Chunk<typename E::elt>::unpack(gv[q], g);
          Chunk<typename E::elt>::unpack(uv[q], u);
          if (i + 1 < TL::TM) load_h(i + 1, q);
          const float gr = FUSED ? grow[FUSED ? i : 0][q] : 1.0f;  // the row's gate
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float sg = sigmoid_fast(g[t]);
            const float dat = FUSED ? da[t] * gr : da[t];
            dg[t] = dat * u[t] * sg * (1.0f + g[t] * (1.0f - sg));
            du[t] = dat * g[t] * sg;
            if constexpr (FUSED) av[t] = gr * (g[t] * sg) * u[t];
          }
          if (rb + r < m_end) {
            const size_t row = (size_t)(rb + r);
            *(uint4*)(dh + row * 2 * F + cb + c) = Chunk<typename E::elt>::pack(dg);
            *(uint4*)(dh + row * 2 * F + F + cb + c) = Chunk<typename E::elt>::pack(du);
            if constexpr (FUSED)
              *(uint4*)(ag + row * F + cb + c) = Chunk<typename E::elt>::pack(av);
          }
        }
      }
    }
  }
};

// dgrad GEMM B: dxp = dh . W_gu[e]  (A: dh rows, K = 2F; B: W_gu[e]
// transposed, W_guT[e] [d][2F], K-contiguous)
template <class E>
struct DgradInOp {
  typedef E Elt;
  const uint16_t* dh;
  const uint16_t* W_guT;
  uint16_t* dxp;
  int d, F;
  __device__ __forceinline__ int k_len() const { return 2 * F; }
  template <class TL, class LA, class LB>
  __device__ __forceinline__ void init(int e, int m0, int m_end, int nt, LA& la, LB& lb,
                                       int tid) const {
    const int nb = nt * TL::BN;
    const uint16_t* WgT = W_guT + (size_t)e * d * 2 * F;
    la.init(dh + (size_t)m0 * 2 * F, [&](int r) { return (min(m0 + r, m_end - 1) - m0) * 2 * F; },
            tid);
    lb.init(WgT, [&](int n) { return min(nb + n, d - 1) * 2 * F; }, tid);
  }
  template <class TL>
  __device__ __forceinline__ void epilogue(const f32x16_t (&acc)[TL::TM][TL::TN], int e, int m0,
                                           int m_end, int nt, uint16_t* smem) const {
    const WavePos w = WavePos::of<TL>();
#pragma unroll
    for (int p = 0; p < TL::TN / 2; ++p) {
      const int cb = nt * TL::BN + w.wn * TL::WTN + p * 64;
      if (cb >= d) continue;  // d is a multiple of 64; wave-uniform
#pragma unroll
      for (int i = 0; i < TL::TM; ++i) {
        const int rb = m0 + w.wm * TL::WTM + i * 32;
        const float* blk = stage_rows<TL>(acc, i, p, smem, w.wave, w.lane);
        store_block<E>(blk, dxp + (size_t)rb * d + cb, (size_t)d, m_end - rb, w.lane);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// wgrad: per local expert e over its rows [offsets[e], offsets[e+1]):
//   dW_down[e] (d x F)  = dy_p^T . a      (A: dy_p, M = d;  B: a,  N = F)
//   dW_gu[e]   (2F x d) = dh^T   . xp     (A: dh,   M = 2F; B: xp, N = d)
// Both operands are contiguous along M/N (the reduction runs over rows), so a
// 64-row stage is copied with 16-byte row-contiguous loads into a natural
// [k][col] LDS tile and read back by transpose (TrFrags).  One launch covers
// both products of every expert.
// ---------------------------------------------------------------------------

// Loader of one wgrad operand: a stage is the [64 k][256 col] tile at rows
// [k0, k0 + 64) of the expert's rows, columns [m0, m0 + 256).  Thread t's
// chunk c is tile row c * 16 + t / 32, columns m0 + 8 (t % 32)..+7, so a wave
// instruction reads two 512-byte row pieces; it is stored to the LDS tile at
// the position frag_at expects.  A direct operand is read through a buffer
// resource rebuilt per stage over rows [k0, rows) of the expert (offsets stay
// small, whatever the operand's size), so rows past the expert's end read as
// zero; columns past M, only in a tile that crosses M, read the next row's
// values and only reach outputs the epilogue does not store.  A gathered
// operand's row k is token rows_of[r0 + k] / K of the token matrix; each
// chunk's token is loaded one stage ahead (when the chunk is loaded for the
// stage before), and a row past the expert's end gets an offset past the
// resource, which reads as zero.  A direct operand may have up to kWgMore
// more segments (segment()): stages from row kB[s] on read rows k - kB[s] of
// another operand's expert rows (the grouped weight gradient: one reduction
// over several micro-batches' rows, each segment padded with zero rows to
// whole stages).
constexpr int kWgMore = 3;  // micro-batches beyond the first in one wgrad launch
template <bool CAN_GATHER, int NT = 512>
struct WgLoad {
  static constexpr int CH = 64 * 32 / NT;  // 16-byte chunks per thread and stage
  static constexpr int NLOAD = CH, NSTORE = CH;
  u32x4_t v[CH];  // the stage in flight
  __amdgpu_buffer_rsrc_t rsrc;  // direct: the current stage's rows
  const uint16_t* base;         // direct: the expert's first row
  long ld;                      // elements per operand row
  int rows;                     // rows of the expert
  uint32_t voff;                // direct: byte offset of chunk 0 within a stage
  int dst0;                     // byte offset of chunk 0 in an LDS tile
  const uint16_t* base2[kWgMore];  // more segments (direct operands): expert's first row
  int rows2[kWgMore], kB[kWgMore];  // their rows, and the first stage row that reads them
  // CAN_GATHER: with gat set (block-uniform) the operand is gathered.  The
  // gathered and the direct offset are both formed and one is selected, so
  // the chunk loads have no branch (a branch around them costs a full wait
  // for every outstanding load where the paths merge).
  bool gat;
  __amdgpu_buffer_rsrc_t rsrc_g;  // the token matrix
  __amdgpu_buffer_rsrc_t rtok;    // rows_of entries [0, n_rows)
  uint32_t coff;                  // byte offset of this thread's columns within a row
  int r0, K, trow;
  // rows_of value of each chunk's row in the next stage loaded (a vector, so
  // that it stays in registers)
  typedef int i32xCH_t __attribute__((ext_vector_type(CH)));
  i32xCH_t tok_next;

  __device__ __forceinline__ void init(const uint16_t* src, long ld_, int m0, int r0_, int r1,
                                       bool gathered, const int32_t* xrows, int K_, int tid,
                                       int n_rows = 0) {
    ld = ld_;
    rows = r1 - r0_;
    trow = tid >> 5;
    coff = (uint32_t)(m0 + 8 * (tid & 31)) * 2u;
    dst0 = wg_byte(trow, 8 * (tid & 31));
    base = src + (size_t)r0_ * ld_;
    voff = (uint32_t)trow * (uint32_t)(ld_ * 2) + coff;
#pragma unroll
    for (int q = 0; q < kWgMore; ++q) kB[q] = 0x7fffffff;
    gat = CAN_GATHER && gathered;
    if constexpr (CAN_GATHER) {
      // every token is a row of the matrix; only the past-the-end marker
      // exceeds the records limit
      rsrc_g = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, 0x7fffffff, 0x00020000);
      rtok = __builtin_amdgcn_make_buffer_rsrc((void*)xrows, (short)0, n_rows * 4, 0x00020000);
      r0 = r0_;
      K = K_;
#pragma unroll
      for (int c = 0; c < CH; ++c) tok_next[c] = token(0, c);
    }
  }
  __device__ __forceinline__ void segment(int q, const uint16_t* src, int r0_, int r1, int kB_) {
    base2[q] = src + (size_t)r0_ * ld;
    rows2[q] = r1 - r0_;
    kB[q] = kB_;
  }
  // rows_of value of chunk c's row in stage k0, read without a branch at an
  // index clamped into the expert's rows (for an expert with none, index
  // r0 - 1, past the resource when r0 = 0, which reads 0); whether the row
  // exists is decided where the value is used
  __device__ __forceinline__ int token(int k0, int c) const {
    const int k = min(k0 + c * 16 + trow, rows - 1);
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rtok, (r0 + k) * 4, 0, 0);
  }
  __device__ __forceinline__ void load_c(int c, int k0) {
    if (c == 0) {  // the direct resource of stage k0 (segments in ascending kB)
      const uint16_t* b = base;
      int k = k0, rw = rows;
#pragma unroll
      for (int q = 0; q < kWgMore; ++q) {
        const bool in = k0 >= kB[q];  // block-uniform
        b = in ? base2[q] : b;
        k = in ? k0 - kB[q] : k;
        rw = in ? rows2[q] : rw;
      }
      const long left = (long)(rw - k) * ld * 2;
      const int nrec = left <= 0 ? 0 : (left > 0x7fffffffL ? 0x7fffffff : (int)left);
      rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(b + (size_t)k * ld), (short)0, nrec,
                                               0x00020000);
    }
    const uint32_t off_d = voff + (uint32_t)(c * 16) * (uint32_t)(ld * 2);
    if constexpr (CAN_GATHER) {
      // the token is consumed before the next one is loaded into its
      // register, so that load needs no copy (and no wait)
      const int t = tok_next[c];
      const uint32_t row_off = ((unsigned)t / (unsigned)K) * (uint32_t)(ld * 2) + coff;
      const uint32_t off_g = k0 + c * 16 + trow < rows ? row_off : 0x80000000u;
      v[c] = __builtin_amdgcn_raw_buffer_load_b128(gat ? rsrc_g : rsrc, (int)(gat ? off_g : off_d),
                                                   0, 0);
      tok_next[c] = token(k0 + 64, c);
    } else {
      v[c] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off_d, 0, 0);
    }
  }
  __device__ __forceinline__ void store_c(int c, uint16_t* lds) const {
    *(u32x4_t*)((uint8_t*)lds + dst0 + c * 16 * WG_ROWB) = v[c];
  }
  __device__ __forceinline__ void load(int k0, int /*k_end*/) {
#pragma unroll
    for (int c = 0; c < CH; ++c) load_c(c, k0);
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int c = 0; c < CH; ++c) store_c(c, lds);
  }
};

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ long long uniform64(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(unsigned long long)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// 256 x 256 output tiles, 8 waves (2 x 4), wave tile 128 x 64, on the main
// loop of the row-grouped GEMMs (two LDS stages of 64 rows, the stage after
// next in registers; see mainloop_steps) with transposed fragment reads.
// Tiles are software-pipelined across the persistent loop like the
// row-grouped GEMMs': the next tile's first stage is loaded before this
// tile's epilogue issues its stores.
//
// With xrows set (the fused permute), xp is the token matrix x [T][d] and the
// dW_gu tiles read dispatched row r from token xrows[r] / K.
//
// ROUTER reuses the kernel for the router weight gradient: the "experts" are
// chunks of rchunk tokens (chunk c = rows [c rchunk, min((c+1) rchunk, rows))),
// only the first product is formed, dyp holds x [T][d], abuf holds the split
// dlogits [T][F] (F = 2E) and dW_down receives one float32 partial [d][F] per
// chunk; offsets, xp, dh and dW_gu are unused.
// GD (the fused combine backward): dy_p is not materialised; dyp is the token
// matrix dout [T][d], the dW_down tiles read dispatched row r of their A
// operand from token xrows[r] / K in the same way, and abuf holds
// ag = gate . a, so dW_down[e] = sum_r dout[t_r] (outer) ag[r].
//
// ACC: add into the existing values of dW (gradient accumulation) instead of
// overwriting them.
// MULTI (the grouped weight gradient, with neither gather): the reduction of
// every tile runs over the expert's rows of up to kWgMore more micro-batches
// too (more: their xp, a, dh, dy_p and offsets), after the first one's, in
// one float32 accumulation, so dW is read and written once for all of them.
struct WgMore {
  int n;  // micro-batches given below (0 .. kWgMore)
  const uint16_t *xp[kWgMore], *abuf[kWgMore], *dh[kWgMore], *dyp[kWgMore];
  const int32_t* offsets[kWgMore];
};
template <bool GATHER, class E, bool ROUTER, bool ACC, bool GD = false, bool MULTI = false>
__global__ __launch_bounds__(512) void wgrad_kernel(
    const uint16_t* __restrict__ xp, const int32_t* __restrict__ xrows, int K,
    const uint16_t* __restrict__ abuf, const uint16_t* __restrict__ dh,
    const uint16_t* __restrict__ dyp, const int32_t* __restrict__ offsets,
    float* __restrict__ dW_gu, float* __restrict__ dW_down, int E_l, int d, int F,
    int rchunk = 0, int rows = 0, WgMore more = WgMore{}) {
  static_assert(!MULTI || !(GATHER || GD || ROUTER), "the grouped wgrad reads direct operands");
  using TL = T256;
  constexpr int WTM = TL::WTM, WTN = TL::WTN, TM = TL::TM, TN = TL::TN;
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  __shared__ long long s_it[257];  // first cost unit of each expert's tiles; s_it[E_l] = W
  const int tdm = (d + 255) / 256, tdn = (F + 255) / 256;
  const int tgm = (2 * F + 255) / 256, tgn = (d + 255) / 256;
  const int per_e = tdm * tdn + (ROUTER ? 0 : tgm * tgn);
  // first row of expert (or token chunk) e; with MULTI, of micro-batch q's
  // expert e among the others
  auto off = [&](int e) { return ROUTER ? min(e * rchunk, rows) : offsets[e]; };
  const int nmore = MULTI ? more.n : 0;
  auto off2 = [&](int q, int e) { return more.offsets[q][e]; };
  // stages of expert e: each segment padded to whole stages
  auto stages = [&](int e) {
    int n = (off(e + 1) - off(e) + BK - 1) / BK;
    if constexpr (MULTI) {
#pragma unroll
      for (int q = 0; q < kWgMore; ++q)
        if (q < nmore) n += (off2(q, e + 1) - off2(q, e) + BK - 1) / BK;
    }
    return n;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / TL::WGN, wn = w % TL::WGN;
  // Work-balanced schedule: a tile costs nk_e = max(1, ceil(rows_e / 64))
  // units (experts' row counts differ) and the W units of all tiles are laid
  // out tile-major.  XCD g (the hardware places block b on XCD b % 8) takes
  // the tiles whose first unit falls in [W*g/8, W*(g+1)/8), so the XCDs get
  // equal work, and its blocks take those tiles round robin, so the tiles
  // running together share operand rows in the XCD's L2.
  if (tid == 0) {
    long long acc_it = 0;
    for (int e = 0; e < E_l; ++e) {
      s_it[e] = acc_it;
      const int nk = stages(e);
      acc_it += (long long)per_e * (nk > 0 ? nk : 1);
    }
    s_it[E_l] = acc_it;
  }
  __syncthreads();
  const int G = gridDim.x, NG = G % 8 == 0 ? 8 : 1;
  const int grp = blockIdx.x % NG, slot = blockIdx.x / NG, nslots = G / NG;
  const long long W = uniform64(s_it[E_l]);
  const long long lo = W * grp / NG, hi = W * (grp + 1) / NG;
  long long gt0;  // first tile (expert-major index) starting at or after lo
  {
    int a = 0, b = E_l;  // s_it[a] <= lo < s_it[b]
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (s_it[mid] <= lo) a = mid;
      else b = mid;
    }
    a = __builtin_amdgcn_readfirstlane(a);
    const long long it0 = uniform64(s_it[a]);
    const long long nk0 = (uniform64(s_it[a + 1]) - it0) / per_e;
    gt0 = (long long)a * per_e + (lo - it0 + nk0 - 1) / nk0;
  }
  // Tile gt of the expert-major order: its expert, operands, output and
  // k-steps; valid = false once the group's range of work is done.
  struct TileJob {
    bool valid, ga, gb;  // gathers a token-indexed operand: A (dW_down), B (dW_gu)
    int r0, r1, M, N, m0, n0, nk;
    const uint16_t *Asrc, *Bsrc;
    float* out;
    // MULTI: micro-batch q's rows and operands among the others, from stage
    // row kB[q] on
    int r0b[kWgMore], r1b[kWgMore], kB[kWgMore];
    const uint16_t *Asrc2[kWgMore], *Bsrc2[kWgMore];
  };
  // Tile t of expert e (the tile index advances by whole slots, so e and t
  // are kept apart and no division runs between tiles: a division needs
  // vector registers, which the accumulators hold there)
  auto job = [&](int e, int t) {
    TileJob j{};
    j.valid = false;
    if (e >= E_l) return j;
    {
      const long long it0 = uniform64(s_it[e]);
      const int nk_e = max(1, stages(e));
      if (it0 + (long long)t * nk_e >= hi) return j;  // uniform
    }
    j.valid = true;
    j.r0 = off(e);
    j.r1 = off(e + 1);
    j.nk = stages(e);
    const bool down = t < tdm * tdn;
    if constexpr (MULTI) {
      int kb = (j.r1 - j.r0 + BK - 1) / BK * BK;
#pragma unroll
      for (int q = 0; q < kWgMore; ++q) {
        if (q >= nmore) break;  // uniform
        j.r0b[q] = off2(q, e);
        j.r1b[q] = off2(q, e + 1);
        j.kB[q] = kb;
        kb += (j.r1b[q] - j.r0b[q] + BK - 1) / BK * BK;
        j.Asrc2[q] = down ? more.dyp[q] : more.dh[q];
        j.Bsrc2[q] = down ? more.abuf[q] : more.xp[q];
      }
    }
    if (down) {
      j.ga = GD;
      j.gb = false;
      j.Asrc = dyp;
      j.Bsrc = abuf;
      j.M = d;
      j.N = F;
      j.m0 = (t / tdn) * 256;
      j.n0 = (t % tdn) * 256;
      j.out = dW_down + (size_t)e * d * F;
    } else {
      t -= tdm * tdn;
      j.Asrc = dh;
      j.Bsrc = xp;
      j.ga = false;
      j.gb = GATHER;
      j.M = 2 * F;
      j.N = d;
      j.m0 = (t / tgn) * 256;
      j.n0 = (t % tgn) * 256;
      j.out = dW_gu + (size_t)e * 2 * F * d;
    }
    return j;
  };
  // the gathering variants hold token registers: addresses formed per read
  using FR = TrFrags<TL, !(GATHER || GD)>;
  // dispatched rows (the token lists' extent)
  const int n_rows = (GATHER || GD) ? __builtin_amdgcn_readfirstlane(off(E_l)) : 0;
  FR fr;
  fr.init(wm, wn, lane);
  WgLoad<GD> la;
  WgLoad<GATHER> lb;
  auto init_loaders = [&](const TileJob& c) {
    la.init(c.Asrc, c.M, c.m0, c.r0, c.r1, c.ga, xrows, K, tid, n_rows);
    lb.init(c.Bsrc, c.N, c.n0, c.r0, c.r1, c.gb, xrows, K, tid, n_rows);
    if constexpr (MULTI) {
#pragma unroll
      for (int q = 0; q < kWgMore; ++q) {
        if (q >= nmore) break;  // uniform
        la.segment(q, c.Asrc2[q], c.r0b[q], c.r1b[q], c.kB[q]);
        lb.segment(q, c.Bsrc2[q], c.r0b[q], c.r1b[q], c.kB[q]);
      }
    }
  };
  int ge = (int)((gt0 + slot) / per_e), gtt = (int)((gt0 + slot) % per_e);
  TileJob cur = job(ge, gtt);
  if (!cur.valid) return;  // block-uniform
  init_loaders(cur);
  la.load(0, 0);
  lb.load(0, 0);
  for (;;) {
    const int nk = cur.nk;
    la.store(smem);
    lb.store(smem + 2 * TL::BM * BK);
    la.load(nk > 1 ? BK : 0, 0);
    lb.load(nk > 1 ? BK : 0, 0);
    __syncthreads();
    f32x16_t acc[TM][TN];
    mainloop_steps<TL, E, WgLoad<GD>, WgLoad<GATHER>, true, FR>(la, lb, 0, nk, smem, acc, fr);
    gtt += nslots;
    while (gtt >= per_e) {  // uniform, a few rounds at most
      gtt -= per_e;
      ++ge;
    }
    const TileJob nxt = job(ge, gtt);
    // the next tile's first stage is loaded during this tile's epilogue,
    // behind the epilogue's first loads and ahead of its stores
    auto next_stage0 = [&]() {
      if (nxt.valid) {  // block-uniform
        init_loaders(nxt);
        la.load(0, 0);
        lb.load(0, 0);
      }
    };
    // Epilogue.  Accumulator block acc[i][j] registers 4q..4q+3 hold output
    // row wm*128 + i*32 + lane%32 of the tile, columns wn*64 + j*32 + 8q +
    // 4*(lane/32) + 0..3 (TrFrags: the N-side fragment is the MFMA's first
    // operand).  Each 32 x 32 piece pc = i*TN + j goes through a 4 KiB slot
    // of the wave's 16 KiB of LDS (all of it is free: the main loop ended
    // with a barrier, and the next tile's first stage is in registers):
    // written as 16-byte chunks, a row's chunks XOR-swizzled by the row, and
    // read back as 8 rows x 128 bytes per instruction, lane l taking row
    // l/8 + 8p, columns 4*(l%8)..+3, so every global access is 16 bytes per
    // lane and 128 contiguous bytes per row.  LDS operations of one wave
    // complete in order, so no barrier is needed between a write and its
    // read-back, or between a slot's read-back and its next write.  dW is
    // touched once per launch: its loads and stores are non-temporal.
    // Global accesses go through a buffer resource over the tile's rows
    // [m0, min(m0 + 256, M)).  No branch decides what is written: an access
    // the tile does not own -- a 32-row piece past M (M - m0 is a multiple
    // of 64, so a piece lies wholly inside or past it) or columns past N --
    // has 2^31 added to its offset, beyond the resource's size, so the
    // buffer range check drops it (a load returns 0).
    const int M = cur.M, N = cur.N, m0 = cur.m0, n0 = cur.n0;
    const int rows_in = min(256, M - m0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cur.out + (size_t)m0 * N), (short)0, rows_in * N * 4, 0x00020000);
    constexpr int NT_ = 2;  // cache policy: non-temporal
    uint8_t* const ep = (uint8_t*)smem + w * 16384;
    auto ep_write = [&](int i, int j, int slot) {
      const int r = lane & 31;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 2 * q + (lane >> 5);
        const f32x4_t v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                           acc[i][j][4 * q + 3]};
        *(f32x4_t*)(ep + slot * 4096 + r * 128 + ((c ^ (r & 7)) << 4)) = v;
      }
    };
    auto ep_read = [&](int p, int slot) {
      const int r = (lane >> 3) + 8 * p, c = lane & 7;
      return *(const f32x4_t*)(ep + slot * 4096 + r * 128 + ((c ^ (r & 7)) << 4));
    };
    auto piece_in = [&](int i) { return (uint32_t)(wm * WTM + i * 32 - rows_in) >> 31; };
    // byte offset of this lane's chunk of piece (i, j), row group p, column e
    // of the chunk (drop bit included)
    auto voff = [&](int i, int j, int p, int e = 0) {
      const int col = n0 + wn * WTN + j * 32 + 4 * (lane & 7) + e;
      const int row = wm * WTM + i * 32 + (lane >> 3) + 8 * p;
      const uint32_t drop = ((uint32_t)(N - 1 - col) >> 31) | (1u - piece_in(i));
      return (int)(((uint32_t)(row * N + col) * 4u) | (drop << 31));
    };
    constexpr int NP = TM * TN;  // pieces
    constexpr int NS = 4;        // LDS slots per wave
    if constexpr (ROUTER) next_stage0();
    // the router's N = 2E need not be a multiple of 4 (block-uniform)
    if (!ROUTER || (N & 3) == 0) {
      // N is a multiple of 4: a chunk of four columns lies wholly inside or
      // past it.  With ACC, pieces 0..NS-1 first go to their LDS slots, which
      // frees their registers for the previous values of PF pieces, all
      // loaded at once; piece pc + PF is loaded into piece pc's registers as
      // soon as those are consumed.  Piece pc is then read back (pieces past
      // NS are staged through the slot of piece pc - NS, already read), added
      // to its previous values and stored.  The next tile's first stage is
      // loaded once half of the pieces are stored.
      constexpr int PF = 5;
      f32x4_t prev[ACC ? PF : 1][4];
      auto load_piece = [&](int pc) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          prev[pc % PF][p] = __builtin_bit_cast(
              f32x4_t,
              __builtin_amdgcn_raw_buffer_load_b128(rs, voff(pc / TN, pc % TN, p), 0, NT_));
      };
      if constexpr (ACC) {
#pragma unroll
        for (int pc = 0; pc < NS; ++pc) ep_write(pc / TN, pc % TN, pc);
#pragma unroll
        for (int pc = 0; pc < PF; ++pc) load_piece(pc);
      } else if constexpr (!ROUTER) {
        next_stage0();
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        const int i = pc / TN, j = pc % TN, slot = pc % NS;
        if (!ACC || pc >= NS) ep_write(i, j, slot);
        f32x4_t v[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          v[p] = ep_read(p, slot);
          if constexpr (ACC) v[p] += prev[pc % PF][p];
        }
        // (ahead of the stores: a load issued after a store could not be
        // waited for without it, vector memory operations complete in order)
        if (ACC && pc + PF < NP) load_piece(pc + PF);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < 4; ++p)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v[p]), rs,
                                                 voff(i, j, p), 0, NT_);
        __builtin_amdgcn_sched_barrier(0);
        if (ACC && pc == NP / 2 - 1) next_stage0();
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // 4-byte stores, each column checked
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        const int i = pc / TN, j = pc % TN;
        ep_write(i, j, 0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f32x4_t v = ep_read(p, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), rs, voff(i, j, p, e), 0, 0);
        }
      }
    }
    __syncthreads();  // staging reads done before the next tile's first stage lands in LDS
    if (!nxt.valid) break;
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// router logits: l = x . W_r + bias with W_r given transposed (W_rT [E][d]),
// float32 output.
// ---------------------------------------------------------------------------
// With splits > 1 the reduction over d is cut into `splits` equal ranges (one
// per block-tile pass) and range s writes its float32 partial, without the
// bias, to partial + s * T * E; the top-k kernel adds the ranges.
template <class TL, class EL>
__global__ __launch_bounds__(TL::NT) void router_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W_rT,
    const float* __restrict__ bias, float* __restrict__ logits, int T, int d, int E,
    int n_tiles, int m_tiles, int splits, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  const int dk = d / splits;  // a multiple of 64
  for (Sched sc(m_tiles * n_tiles * splits); sc.t < sc.end; sc.t += sc.step) {
    const int sp = sc.t % splits, tile = sc.t / splits;
    const int m0 = (tile / n_tiles) * TL::BM, n0 = (tile % n_tiles) * TL::BN;
    LoadK<TL::BM, TL::NT> la;
    LoadK<TL::BN, TL::NT> lb;
    la.init(x + (size_t)m0 * d, [&](int r) { return (min(m0 + r, T - 1) - m0) * d; }, tid);
    lb.init(W_rT + (size_t)n0 * d, [&](int n) { return (min(n0 + n, E - 1) - n0) * d; }, tid);
    f32x16_t acc[TL::TM][TL::TN];
    mainloop<TL, EL>(la, lb, sp * dk, (sp + 1) * dk, smem, acc);
    float* out = splits > 1 ? partial + (size_t)sp * T * E : logits;
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) {
      const int col = n0 + wn * TL::WTN + j * 32 + (lane & 31);
      if (col >= E) continue;
      const float b = (bias && splits == 1) ? bias[col] : 0.f;
#pragma unroll
      for (int i = 0; i < TL::TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * TL::WTM + i * 32 + out_row(lane, r);
          if (row < T) out[(size_t)row * E + col] = acc[i][j][r] + b;
        }
    }
  }
}

// out[b] = in[b]^T for a batch of R x C bf16 matrices (R, C multiples of 64):
// 64 x 64 tiles through LDS, 16-byte global accesses on both sides.
__global__ __launch_bounds__(256) void transpose_batched_kernel(const uint16_t* __restrict__ in,
                                                                uint16_t* __restrict__ out, int R,
                                                                int C) {
  __shared__ uint16_t t[64][64 + 2];
  const size_t mat = (size_t)blockIdx.z * R * C;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int rr = q >> 3, cc = (q & 7) * 8;
    const uint4 v = *(const uint4*)(in + mat + (size_t)(r0 + rr) * C + c0 + cc);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[rr][cc + 2 * i] = (uint16_t)(w[i] & 0xffffu);
      t[rr][cc + 2 * i + 1] = (uint16_t)(w[i] >> 16);
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int cc = q >> 3, rr = (q & 7) * 8;
    uint4 v;
    v.x = t[rr + 0][cc] | ((uint32_t)t[rr + 1][cc] << 16);
    v.y = t[rr + 2][cc] | ((uint32_t)t[rr + 3][cc] << 16);
    v.z = t[rr + 4][cc] | ((uint32_t)t[rr + 5][cc] << 16);
    v.w = t[rr + 6][cc] | ((uint32_t)t[rr + 7][cc] << 16);
    *(uint4*)(out + mat + (size_t)(c0 + cc) * R + r0 + rr) = v;
  }
}

// Upper bound on the number of kTileM-row tiles over all local experts.
inline int max_row_tiles(const moe_shape* s) {
  const int64_t cap = s->T * s->K;
  return (int)((cap + s->E_l * (int64_t)(kTileM - 1)) / kTileM);
}

// Persistent grid: one block per CU of the current device (at most `tiles`).
inline int persistent_grid(long tiles) {
  static int ncu[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (ncu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    ncu[dev] = n;
  }
  return (int)(tiles < ncu[dev] ? (tiles > 0 ? tiles : 1) : ncu[dev]);
}

template <class TL = T256, class Op>
int launch_row_grouped(const char* name, const moe_shape* s, const Op& op,
                       const int32_t* offsets, const int32_t* tile_offsets, int n_tiles,
                       hipStream_t st) {
  const long tiles = (long)max_row_tiles(s) * n_tiles;
  if (tiles == 0) return MOE_OK;
  const int grid = persistent_grid(tiles);
  MOE_LAUNCH(name, st,
             row_grouped_kernel<TL, Op><<<grid, TL::NT, 0, st>>>(
                 op, offsets, tile_offsets, (int)s->E_l, n_tiles));
  return check_launch(name);
}

// ---------------------------------------------------------------------------
// launchers (16-bit types, dispatched on shape->dtype)
// ---------------------------------------------------------------------------
template <class E>
int ffn_fwd_t(const moe_shape* s, const void* xp, const int32_t* xrows, const int32_t* offsets,
              const int32_t* tile_offsets, const void* W_gu, const void* W_down, void* h,
              void* a, void* yp, hipStream_t st, const int32_t* yrows) {
  const int d = (int)s->d, F = (int)s->F;
  GateUpOp<E> g{(const uint16_t*)xp, (const uint16_t*)W_gu, (uint16_t*)h, (uint16_t*)a, d, F,
                xrows, (int)s->K};
  if (int rc = launch_row_grouped("ffn_gate_up", s, g, offsets, tile_offsets,
                                  (F + T256::BN / 2 - 1) / (T256::BN / 2), st))
    return rc;
  const int nt = (d + T256::BN - 1) / T256::BN;
  if (yrows) {
    DownOp<E, true> dn{(const uint16_t*)a, (const uint16_t*)W_down, (uint16_t*)yp, d, F, yrows};
    return launch_row_grouped("ffn_down", s, dn, offsets, tile_offsets, nt, st);
  }
  DownOp<E> dn{(const uint16_t*)a, (const uint16_t*)W_down, (uint16_t*)yp, d, F, nullptr};
  return launch_row_grouped("ffn_down", s, dn, offsets, tile_offsets, nt, st);
}

template <class E>
int ffn_dgrad_t(const moe_shape* s, const void* dyp, const void* h, const int32_t* offsets,
                const int32_t* tile_offsets, void* dh, void* dxp, void* ws, hipStream_t st,
                int parts, const FusedCombineBwd* fc) {
  const int d = (int)s->d, F = (int)s->F;
  const uint16_t* W_downT = (const uint16_t*)((char*)ws + ws_wT_offset(s));
  const uint16_t* W_guT = (const uint16_t*)((const char*)W_downT + ws_wT_down_bytes(s));
  if (parts & kDgradAct) {
    const int nt = (F + T256::BN - 1) / T256::BN;
    if (fc) {
      DgradActOp<E, true> da{(const uint16_t*)dyp, (const uint16_t*)h, W_downT, (uint16_t*)dh,
                             d, F, fc->pair_of_row, (int)s->K, fc->gates, (uint16_t*)fc->ag};
      if (int rc = launch_row_grouped("dgrad_act", s, da, offsets, tile_offsets, nt, st))
        return rc;
    } else {
      DgradActOp<E> da{(const uint16_t*)dyp, (const uint16_t*)h, W_downT, (uint16_t*)dh, d, F,
                       nullptr, 0, nullptr, nullptr};
      if (int rc = launch_row_grouped("dgrad_act", s, da, offsets, tile_offsets, nt, st))
        return rc;
    }
  }
  if (!(parts & kDgradIn)) return MOE_OK;
  DgradInOp<E> di{(const uint16_t*)dh, W_guT, (uint16_t*)dxp, d, F};
  return launch_row_grouped("dgrad_in", s, di, offsets, tile_offsets,
                            (d + T256::BN - 1) / T256::BN, st);
}

template <class E>
void wgrad_t(const moe_shape* s, const void* xp, const int32_t* xrows, const void* a,
             const void* dh, const void* dyp, const int32_t* offsets, float* dW_gu,
             float* dW_down, bool accumulate, hipStream_t st, const int32_t* dyrows) {
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  const long per_e = (long)((d + 255) / 256) * ((F + 255) / 256) +
                     (long)((2 * F + 255) / 256) * ((d + 255) / 256);
  const int grid = persistent_grid(E_l * per_e);
  // both gathers take their token list from the plan's pair_of_row
  const int32_t* rows = xrows ? xrows : dyrows;
  auto go = [&](auto gather, auto gd, auto acc) {
    MOE_LAUNCH("wgrad", st,
               (wgrad_kernel<decltype(gather)::value, E, false, decltype(acc)::value,
                             decltype(gd)::value>
                <<<grid, 512, 0, st>>>((const uint16_t*)xp, rows, (int)s->K,
                                       (const uint16_t*)a, (const uint16_t*)dh,
                                       (const uint16_t*)dyp, offsets, dW_gu, dW_down, E_l, d, F)));
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto acc_ = [&](auto gather, auto gd) {
    if (accumulate) go(gather, gd, T_{});
    else go(gather, gd, F_{});
  };
  if (xrows) {
    if (dyrows) acc_(T_{}, T_{});
    else acc_(T_{}, F_{});
  } else {
    if (dyrows) acc_(F_{}, T_{});
    else acc_(F_{}, F_{});
  }
}

// The grouped weight gradient of n micro-batches (same shape): one launch
// whose reduction runs over every micro-batch's rows of each expert.
template <class E>
void wgrad_multi_t(const moe_shape* s, const WgrOps* ops, int n, float* dW_gu, float* dW_down,
                   bool accumulate, hipStream_t st) {
  static_assert(kWgGroupMax == 1 + kWgMore, "one first micro-batch plus the others");
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  const long per_e = (long)((d + 255) / 256) * ((F + 255) / 256) +
                     (long)((2 * F + 255) / 256) * ((d + 255) / 256);
  const int grid = persistent_grid(E_l * per_e);
  WgMore more{};
  more.n = n - 1;
  for (int q = 0; q + 1 < n; ++q) {
    more.xp[q] = (const uint16_t*)ops[q + 1].xp;
    more.abuf[q] = (const uint16_t*)ops[q + 1].a;
    more.dh[q] = (const uint16_t*)ops[q + 1].dh;
    more.dyp[q] = (const uint16_t*)ops[q + 1].dyp;
    more.offsets[q] = ops[q + 1].offsets;
  }
  const WgrOps& A = ops[0];
  auto go = [&](auto acc) {
    MOE_LAUNCH("wgrad_multi", st,
               (wgrad_kernel<false, E, false, decltype(acc)::value, false, true>
                <<<grid, 512, 0, st>>>((const uint16_t*)A.xp, nullptr, (int)s->K,
                                       (const uint16_t*)A.a, (const uint16_t*)A.dh,
                                       (const uint16_t*)A.dyp, A.offsets, dW_gu, dW_down, E_l, d,
                                       F, 0, 0, more)));
  };
  if (accumulate) go(std::true_type{});
  else go(std::false_type{});
}

template <class E>
void router_t(const moe_shape* s, const void* x, const void* W_rT, const float* bias,
              float* logits, float* partial, hipStream_t st) {
  using TR = Tile<128, 128, 2, 2>;
  const int T = (int)s->T, d = (int)s->d, En = (int)s->E;
  const int nt = (En + TR::BN - 1) / TR::BN, mt = (T + TR::BM - 1) / TR::BM;
  const int splits = router_splits(s);
  const int grid = persistent_grid((long)mt * nt * splits);
  MOE_LAUNCH("router", st,
             router_kernel<TR, E><<<grid, TR::NT, 0, st>>>((const uint16_t*)x,
                                                           (const uint16_t*)W_rT, bias, logits, T,
                                                           d, En, nt, mt, splits, partial));
}

}  // namespace

int launch_ffn_fwd_mfma(const moe_shape* s, const void* xp, const int32_t* xrows,
                        const int32_t* offsets, const int32_t* tile_offsets, const void* W_gu,
                        const void* W_down, void* h, void* a, void* yp, hipStream_t st,
                        const int32_t* yrows) {
  return s->dtype == MOE_F16 ? ffn_fwd_t<F16>(s, xp, xrows, offsets, tile_offsets, W_gu, W_down,
                                              h, a, yp, st, yrows)
                             : ffn_fwd_t<BF16>(s, xp, xrows, offsets, tile_offsets, W_gu,
                                               W_down, h, a, yp, st, yrows);
}

int launch_dgrad_weights_mfma(const moe_shape* s, const void* W_gu, const void* W_down,
                              void* ws, hipStream_t st) {
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  // K-contiguous copies of the weights (16-bit moves, any 16-bit type):
  // W_downT[e] = W_down[e]^T [F][d], W_guT[e] = W_gu[e]^T [d][2F]
  uint16_t* W_downT = (uint16_t*)((char*)ws + ws_wT_offset(s));
  uint16_t* W_guT = (uint16_t*)((char*)W_downT + ws_wT_down_bytes(s));
  MOE_LAUNCH("transpose_w", st,
             transpose_batched_kernel<<<dim3(F / 64, d / 64, E_l), 256, 0, st>>>(
                 (const uint16_t*)W_down, W_downT, d, F));
  if (int rc = check_launch("transpose W_down")) return rc;
  MOE_LAUNCH("transpose_w", st,
             transpose_batched_kernel<<<dim3(d / 64, 2 * F / 64, E_l), 256, 0, st>>>(
                 (const uint16_t*)W_gu, W_guT, 2 * F, d));
  return check_launch("transpose W_gu");
}

int launch_ffn_dgrad_mfma(const moe_shape* s, const void* dyp, const void* h,
                          const int32_t* offsets, const int32_t* tile_offsets, const void* W_gu,
                          const void* W_down, void* dh, void* dxp, void* ws, bool weights_ready,
                          hipStream_t st, int parts, const FusedCombineBwd* fc) {
  if (!weights_ready)
    if (int rc = launch_dgrad_weights_mfma(s, W_gu, W_down, ws, st)) return rc;
  return s->dtype == MOE_F16
             ? ffn_dgrad_t<F16>(s, dyp, h, offsets, tile_offsets, dh, dxp, ws, st, parts, fc)
             : ffn_dgrad_t<BF16>(s, dyp, h, offsets, tile_offsets, dh, dxp, ws, st, parts, fc);
}

int launch_ffn_wgrad_mfma(const moe_shape* s, const void* xp, const int32_t* xrows,
                          const void* a, const void* dh, const void* dyp,
                          const int32_t* offsets, float* dW_gu, float* dW_down, bool accumulate,
                          hipStream_t st, const int32_t* dyrows) {
  if (s->dtype == MOE_F16)
    wgrad_t<F16>(s, xp, xrows, a, dh, dyp, offsets, dW_gu, dW_down, accumulate, st, dyrows);
  else
    wgrad_t<BF16>(s, xp, xrows, a, dh, dyp, offsets, dW_gu, dW_down, accumulate, st, dyrows);
  return check_launch("wgrad GEMM");
}

int launch_ffn_wgrad_multi_mfma(const moe_shape* s, const WgrOps* ops, int n, float* dW_gu,
                                float* dW_down, bool accumulate, hipStream_t st) {
  if (s->dtype == MOE_F16) wgrad_multi_t<F16>(s, ops, n, dW_gu, dW_down, accumulate, st);
  else wgrad_multi_t<BF16>(s, ops, n, dW_gu, dW_down, accumulate, st);
  return check_launch("grouped wgrad GEMM");
}

int launch_router_wgrad_mfma(const moe_shape* s, const void* x, const void* dl_split,
                             float* partial, hipStream_t st) {
  const int d = (int)s->d, N = 2 * (int)s->E, T = (int)s->T;
  const int chunk = (int)router_mfma_chunk(s->T);
  const int nchunks = (int)cdiv(s->T, chunk);
  const long tiles = (long)nchunks * ((d + 255) / 256) * ((N + 255) / 256);
  if (tiles == 0) return MOE_OK;
  const int grid = persistent_grid(tiles);
  MOE_LAUNCH("dwr_mfma", st,
             (wgrad_kernel<false, BF16, true, false><<<grid, 512, 0, st>>>(
                 nullptr, nullptr, 0, (const uint16_t*)dl_split, nullptr, (const uint16_t*)x,
                 nullptr, nullptr, partial, nchunks, d, N, chunk, T)));
  return check_launch("router dW_r GEMM");
}

int launch_router_logits_mfma(const moe_shape* s, const void* x, const void* W_rT,
                              const float* bias, float* logits, float* partial,
                              hipStream_t st) {
  if (s->dtype == MOE_F16) router_t<F16>(s, x, W_rT, bias, logits, partial, st);
  else router_t<BF16>(s, x, W_rT, bias, logits, partial, st);
  return check_launch("router GEMM");
}

}  // namespace moe
