// Internal declarations shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// element types: bf16 is kept as raw 16-bit patterns
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// float32 -> bfloat16, round to nearest even (NaN stays a NaN): gfx950's
// v_cvt_pk_bf16_f32, two values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f2bf(v); }
};

// fp16 (IEEE binary16) is stored as _Float16; the conversions round to
// nearest even (v_cvt_f16_f32 under the default rounding mode).
template <> struct Elt<_Float16> {
  static __device__ __forceinline__ float ld(const _Float16* p) { return (float)*p; }
  static __device__ __forceinline__ void st(_Float16* p, float v) { *p = (_Float16)v; }
};

// Unpack a 16-byte chunk into floats (8 bf16, 8 fp16 or 4 f32).
template <typename T> struct Chunk;
template <> struct Chunk<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    uint4 r;
    r.x = pack_bf2(f[0], f[1]);
    r.y = pack_bf2(f[2], f[3]);
    r.z = pack_bf2(f[4], f[5]);
    r.w = pack_bf2(f[6], f[7]);
    return r;
  }
};
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
template <> struct Chunk<_Float16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    const f16x8_t h = __builtin_bit_cast(f16x8_t, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    f16x8_t h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)f[i];
    return __builtin_bit_cast(uint4, h);
  }
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    uint4 r;
    r.x = __float_as_uint(f[0]);
    r.y = __float_as_uint(f[1]);
    r.z = __float_as_uint(f[2]);
    r.w = __float_as_uint(f[3]);
    return r;
  }
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }
__device__ __forceinline__ float sigmoid_f(float g) { return 1.0f / (1.0f + expf(-g)); }
// The same for the 16-bit matrix-core epilogues, whose results are rounded to
// bf16 / fp16 (8 / 11 significant bits) right away: exp2 and reciprocal on the
// transcendental unit (v_exp_f32, v_rcp_f32, about 1 ulp each), five
// instructions instead of a correctly rounded expf and an IEEE division.
// Limits as above: sigmoid -> 0 and silu -> -0 for g -> -inf.
__device__ __forceinline__ float sigmoid_fast(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_fast(float g) { return g * sigmoid_fast(g); }

// Wave-wide float sum (wave64).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// host-side helpers (defined in abi.cpp)
// ---------------------------------------------------------------------------
int set_error(int code, const char* fmt, ...);
int check_launch(const char* what);

// Brackets one kernel launch with timing events while moe_timing is enabled.
// `name` must outlive the process (a string literal).
struct KernelTimer {
  int slot = -1;
  hipStream_t stream;
  KernelTimer(const char* name, hipStream_t st);
  void stop();
  ~KernelTimer() { stop(); }
};
#define MOE_LAUNCH(name, st, ...)          \
  do {                                     \
    ::moe::KernelTimer kt_(name, st);      \
    __VA_ARGS__;                           \
    kt_.stop();                            \
  } while (0)

// Rows per M-tile of the bf16 grouped GEMMs (tile_offsets are in these units).
constexpr int kTileM = 256;
// Pairs per block of the dispatch-plan kernels.
constexpr int kPlanChunk = 2048;
// Tokens per partial of the router weight-gradient reduction.
constexpr int kRouterChunk = 256;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 16-bit data types (bf16, fp16) take the matrix-core path.
inline bool is16(const moe_shape* s) { return s->dtype != MOE_F32; }
inline size_t elt_bytes(const moe_shape* s) { return is16(s) ? 2 : 4; }

// Workspace layout pieces (bytes).
inline size_t ws_plan_bytes(const moe_shape* s) {
  int64_t nb = cdiv(s->T * s->K, kPlanChunk);
  return align_up((size_t)(2 * s->E_l * nb) * sizeof(int32_t), 256);
}
inline size_t ws_wrt_bytes(const moe_shape* s) {
  return align_up((size_t)(s->E * s->d) * elt_bytes(s), 256);
}
// The 16-bit router weight gradient on the matrix cores (bf16 data): dlogits
// as two bf16 terms per value (hi | lo, [T][2E]), and per chunk of
// router_mfma_chunk(T) tokens a float32 partial [d][2E] of x^T [hi | lo].
inline int64_t router_mfma_chunk(int64_t T) {
  const int64_t c = align_up((size_t)cdiv(T, 32), 64);
  return c > kRouterChunk ? c : kRouterChunk;
}
inline size_t ws_router_split_bytes(const moe_shape* s) {
  return align_up((size_t)(s->T * 2 * s->E) * 2, 256);
}
inline size_t ws_router_partial_bytes(const moe_shape* s) {
  const int64_t nc = cdiv(s->T, kRouterChunk);
  const size_t valu = align_up((size_t)(nc * s->d * s->E) * sizeof(float), 256);
  if (s->dtype != MOE_BF16) return valu;
  const int64_t nm = cdiv(s->T, router_mfma_chunk(s->T));
  const size_t mfma =
      ws_router_split_bytes(s) + align_up((size_t)(nm * s->d * 2 * s->E) * sizeof(float), 256);
  return mfma > valu ? mfma : valu;
}
// Split-K factor of the 16-bit router GEMM (K = d runs through 128 x 128
// tiles one latency-bound k-step at a time; with few tiles the chip idles):
// S <= 8, a power of two dividing d / 64, raised while tiles * S < 256.
// The S float32 partials of the logits [S][T][E] follow the transposed router
// weights in the workspace; top-k sums them.
inline int router_splits(const moe_shape* s) {
  if (!is16(s)) return 1;
  const int64_t tiles = cdiv(s->T, 128) * cdiv(s->E, 128);
  int S = 1;
  while (S < 8 && tiles * S < 256 && (s->d / 64) % (2 * S) == 0) S *= 2;
  return S;
}
inline size_t ws_router_fwd_bytes(const moe_shape* s) {
  const int S = router_splits(s);
  return S > 1 ? align_up((size_t)(S * s->T * s->E) * sizeof(float), 256) : 0;
}
// Transposed expert weights for the 16-bit dgrad: W_downT [E_l][F][d] then
// W_guT [E_l][d][2F].  The float32 dgrad needs none.  They sit after
// the regions of the plan, the transposed router weights and the router
// gradient partials, so a step can write them while the same micro-batch's
// router backward still uses its partials.
inline size_t ws_wT_offset(const moe_shape* s) {
  size_t b = ws_plan_bytes(s);
  if (ws_wrt_bytes(s) + ws_router_fwd_bytes(s) > b) b = ws_wrt_bytes(s) + ws_router_fwd_bytes(s);
  if (ws_router_partial_bytes(s) > b) b = ws_router_partial_bytes(s);
  return align_up(b, 256);
}
inline size_t ws_wT_down_bytes(const moe_shape* s) {
  return is16(s) ? align_up((size_t)(s->E_l * s->F * s->d) * 2, 256) : 0;
}
inline size_t ws_wT_bytes(const moe_shape* s) {
  return is16(s) ? ws_wT_down_bytes(s) + align_up((size_t)(s->E_l * 2 * s->F * s->d) * 2, 256)
                 : 0;
}

// ---------------------------------------------------------------------------
// launchers (each returns MOE_OK or MOE_ERR_HIP)
// ---------------------------------------------------------------------------
// routing
int launch_transpose_wr(const moe_shape* s, const void* W_r, void* W_rT, hipStream_t st);
int launch_router_logits(const moe_shape* s, const void* x, const void* W_r,
                         const void* W_rT, const float* bias, float* logits, hipStream_t st);
// ws: the workspace of a preceding 16-bit router GEMM (finish its split-K
// partials into logits first), or NULL (logits are given)
int launch_topk(const moe_shape* s, float* logits, int32_t* idx, float* gates, const void* ws,
                const float* bias, hipStream_t st);
int launch_force_balance(const moe_shape* s, int32_t* idx, hipStream_t st);
int launch_route_bwd(const moe_shape* s, const float* dgates, const float* gates,
                     const int32_t* idx, const void* x, float* dlogits, float* dW_r,
                     bool accumulate, void* ws, hipStream_t st);
// dispatch / combine
int launch_plan(const moe_shape* s, const int32_t* idx, int32_t* counts, int32_t* offsets,
                int32_t* row_of_pair, int32_t* pair_of_row, int32_t* tile_offsets, void* ws,
                hipStream_t st);
int launch_permute(const moe_shape* s, const void* x, const int32_t* row_of_pair, void* xp,
                   hipStream_t st);
// writes the shared expert's plan: plan[0..1] = offsets {0, T}, plan[2..3] =
// tile_offsets {0, ceil(T / kTileM)}
int launch_shared_plan(int64_t T, int32_t* plan, hipStream_t st);
// add (nullable): a token-aligned [T][d] term summed in before the one rounding.
// pairs: yp is laid out by (token, slot) pair (row t*K + k, written by the
// forward with yrows set) instead of by dispatched row.
int launch_combine(const moe_shape* s, const void* yp, const float* gates,
                   const int32_t* row_of_pair, const void* add, void* out, hipStream_t st,
                   bool pairs = false);
int launch_combine_bwd(const moe_shape* s, const void* dout, const void* yp, const float* gates,
                       const int32_t* row_of_pair, void* dyp, float* dgates, hipStream_t st,
                       bool pairs = false);
int launch_dispatch_bwd(const moe_shape* s, const void* dxp, const int32_t* row_of_pair,
                        const int32_t* idx, const float* dlogits, const void* W_rT,
                        const void* add, void* dx, bool accumulate, hipStream_t st);
// expert GEMMs.  xrows: null, or the plan's pair_of_row for the fused permute,
// in which case xp is the token matrix x and dispatched row r of the GEMM1 (and
// wgrad dW_gu) operand is token xrows[r] / K.  yrows: null, or the plan's
// pair_of_row, in which case GEMM2 writes dispatched row r to row yrows[r] of
// yp (y by pair).
int launch_ffn_fwd(const moe_shape* s, const void* xp, const int32_t* xrows,
                   const int32_t* offsets, const int32_t* tile_offsets, const void* W_gu,
                   const void* W_down, void* h, void* a, void* yp, hipStream_t st,
                   const int32_t* yrows = nullptr);
// The 16-bit dgrad's transposed weight copies (into ws at ws_wT_offset); a
// no-op in float32.
int launch_dgrad_weights(const moe_shape* s, const void* W_gu, const void* W_down, void* ws,
                         hipStream_t st);
// weights_ready: launch_dgrad_weights already ran on this ws (ordered before
// this call), so the copies are not made again.  parts selects the GEMMs:
// kDgradAct (dy_p -> dh, with the SwiGLU backward), kDgradIn (dh -> dx_p), or
// both in that order; a call with kDgradIn alone needs the copies made.
enum { kDgradAct = 1, kDgradIn = 2, kDgradBoth = 3 };
// The fused combine backward: dy_p is not materialised.  The dgrad's first
// GEMM reads its rows from dout through the plan's pair_of_row (dyp is then
// dout [T][d]) and scales each by its pair's gate in float32; it also writes
// ag = gate * silu(g) * u [T*K][F], which the weight gradient's dW_down
// product takes with the gathered dout rows.
struct FusedCombineBwd {
  const int32_t* pair_of_row;
  const float* gates;  // [T*K], indexed by pair t*K + k
  void* ag;            // [T*K][F]
};
int launch_ffn_dgrad(const moe_shape* s, const void* dyp, const void* h, const int32_t* offsets,
                     const int32_t* tile_offsets, const void* W_gu, const void* W_down, void* dh,
                     void* dxp, void* ws, bool weights_ready, hipStream_t st,
                     int parts = kDgradBoth, const FusedCombineBwd* fc = nullptr);
// dyrows: null, or pair_of_row for the fused combine backward, in which case
// dyp is dout [T][d] (row r of the dW_down operand is token dyrows[r] / K) and
// a is ag.
int launch_ffn_wgrad(const moe_shape* s, const void* xp, const int32_t* xrows, const void* a,
                     const void* dh, const void* dyp, const int32_t* offsets, float* dW_gu,
                     float* dW_down, bool accumulate, hipStream_t st,
                     const int32_t* dyrows = nullptr);
// The operands of one micro-batch's weight gradient (materialised xp and dy_p).
struct WgrOps {
  const void *xp, *a, *dh, *dyp;
  const int32_t* offsets;
};
// The grouped weight gradient: dW (+)= the weight gradients of micro-batches
// ops[0 .. n), reduced over all their rows of each expert in one
// accumulation (in that order), so dW is read and written once; 2 <= n <=
// kWgGroupMax.
constexpr int kWgGroupMax = 4;
int launch_ffn_wgrad_multi(const moe_shape* s, const WgrOps* ops, int n, float* dW_gu,
                           float* dW_down, bool accumulate, hipStream_t st);
int launch_ffn_wgrad_multi_mfma(const moe_shape* s, const WgrOps* ops, int n, float* dW_gu,
                                float* dW_down, bool accumulate, hipStream_t st);

}  // namespace moe
