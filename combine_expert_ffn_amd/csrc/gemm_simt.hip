// Expert GEMMs in float32: one thread per output element, float32
// accumulation in k order.  This is the float32 mode of the library (small
// layers, exact-to-1e-5 checks); bf16 and fp16 layers use the matrix-core
// kernels in gemm_mfma.hip.  Same formulas as there: SwiGLU expert FFN forward,
// its activation gradient (D) and weight gradient (W) (1F1B note page 2, "MoE
// 1F1B overlap").
#include "moe_internal.h"

namespace moe {

// Local expert owning permuted row `row` (offsets non-decreasing, row < offsets[E_l]).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E_l,
                                             int row) {
  int lo = 0, hi = E_l;  // offsets[lo] <= row < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

// xrows: null, or pair_of_row for the fused permute (xp is then x and row r
// reads token xrows[r] / K).
__global__ __launch_bounds__(256) void f32_gate_up_kernel(const float* __restrict__ xp,
                                                          const int32_t* __restrict__ xrows,
                                                          int K,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ W_gu,
                                                          float* __restrict__ h,
                                                          float* __restrict__ a, long cap,
                                                          int E_l, int d, int F) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= cap * F) return;
  const int row = (int)(i / F), j = (int)(i % F);
  if (row >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, row);
  const float* xr = xp + (size_t)(xrows ? xrows[row] / K : row) * d;
  const float* wg = W_gu + ((size_t)e * 2 * F + j) * d;
  const float* wu = W_gu + ((size_t)e * 2 * F + F + j) * d;
  float g = 0.f, u = 0.f;
  for (int c = 0; c < d; ++c) {
    g = fmaf(xr[c], wg[c], g);
    u = fmaf(xr[c], wu[c], u);
  }
  h[(size_t)row * 2 * F + j] = g;
  h[(size_t)row * 2 * F + F + j] = u;
  a[(size_t)row * F + j] = silu_f(g) * u;
}

__global__ __launch_bounds__(256) void f32_down_kernel(const float* __restrict__ a,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ W_down,
                                                       float* __restrict__ yp, long cap, int E_l,
                                                       int d, int F,
                                                       const int32_t* __restrict__ yrows) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= cap * d) return;
  const int row = (int)(i / d), c = (int)(i % d);
  if (row >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, row);
  const float* ar = a + (size_t)row * F;
  const float* w = W_down + ((size_t)e * d + c) * F;
  float y = 0.f;
  for (int f = 0; f < F; ++f) y = fmaf(ar[f], w[f], y);
  yp[(size_t)(yrows ? yrows[row] : row) * d + c] = y;
}

// xrows: null, or pair_of_row for the fused combine backward: dyp is then
// dout, row r reads token xrows[r] / K, the product is scaled by the pair's
// gate and ag = gate * silu(g) * u is written too.
__global__ __launch_bounds__(256) void f32_dgrad_act_kernel(
    const float* __restrict__ dyp, const int32_t* __restrict__ xrows, int K,
    const float* __restrict__ gates, float* __restrict__ ag, const float* __restrict__ hbuf,
    const int32_t* __restrict__ offsets, const float* __restrict__ W_down,
    float* __restrict__ dh, long cap, int E_l, int d, int F) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= cap * F) return;
  const int row = (int)(i / F), j = (int)(i % F);
  if (row >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, row);
  const float* dy = dyp + (size_t)(xrows ? xrows[row] / K : row) * d;
  const float* w = W_down + (size_t)e * d * F + j;
  float da = 0.f;
  for (int c = 0; c < d; ++c) da = fmaf(dy[c], w[(size_t)c * F], da);
  const float gate = xrows ? gates[xrows[row]] : 1.f;
  da *= gate;
  const float g = hbuf[(size_t)row * 2 * F + j];
  const float u = hbuf[(size_t)row * 2 * F + F + j];
  const float s = sigmoid_f(g);
  dh[(size_t)row * 2 * F + j] = da * u * s * (1.0f + g * (1.0f - s));
  dh[(size_t)row * 2 * F + F + j] = da * g * s;
  if (xrows) ag[(size_t)row * F + j] = gate * (g * s) * u;
}

__global__ __launch_bounds__(256) void f32_dgrad_in_kernel(const float* __restrict__ dh,
                                                           const int32_t* __restrict__ offsets,
                                                           const float* __restrict__ W_gu,
                                                           float* __restrict__ dxp, long cap,
                                                           int E_l, int d, int F) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= cap * d) return;
  const int row = (int)(i / d), c = (int)(i % d);
  if (row >= offsets[E_l]) return;
  const int e = expert_of_row(offsets, E_l, row);
  const float* g = dh + (size_t)row * 2 * F;
  const float* w = W_gu + (size_t)e * 2 * F * d + c;
  float acc = 0.f;
  for (int m = 0; m < 2 * F; ++m) acc = fmaf(g[m], w[(size_t)m * d], acc);
  dxp[(size_t)row * d + c] = acc;
}

// The micro-batches after the first of a grouped weight gradient.
struct WgrMoreF32 {
  int n;
  WgrOps ops[kWgGroupMax - 1];
};

// dW_down[e][i][f] = sum_r dyp[r][i] a[r][f]; dW_gu[e][m][c] = sum_r dh[r][m] xp[r][c]
// (dyrows set: dyp is dout and row r of it is token dyrows[r] / K)
__global__ __launch_bounds__(256) void f32_wgrad_kernel(
    const float* __restrict__ xp, const int32_t* __restrict__ xrows, int K,
    const float* __restrict__ a, const float* __restrict__ dh,
    const float* __restrict__ dyp, const int32_t* __restrict__ dyrows,
    const int32_t* __restrict__ offsets,
    float* __restrict__ dW_gu, float* __restrict__ dW_down, int E_l, int d, int F,
    int accumulate, WgrMoreF32 more) {
  // more.n > 0: the grouped weight gradient, the sum continuing over the
  // other micro-batches' rows of the expert, in order (materialised operands)
  const long per_e = (long)d * F + 2L * F * d;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_e * E_l) return;
  const int e = (int)(i / per_e);
  long q = i % per_e;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  float acc = 0.f;
  float* o;
  if (q < (long)d * F) {
    const int ii = (int)(q / F), f = (int)(q % F);
    for (int r = r0; r < r1; ++r)
      acc = fmaf(dyp[(size_t)(dyrows ? dyrows[r] / K : r) * d + ii], a[(size_t)r * F + f], acc);
    for (int g = 0; g < more.n; ++g) {
      const float *dy2 = (const float*)more.ops[g].dyp, *a2 = (const float*)more.ops[g].a;
      for (int r = more.ops[g].offsets[e]; r < more.ops[g].offsets[e + 1]; ++r)
        acc = fmaf(dy2[(size_t)r * d + ii], a2[(size_t)r * F + f], acc);
    }
    o = dW_down + (size_t)e * d * F + q;
  } else {
    q -= (long)d * F;
    const int m = (int)(q / d), c = (int)(q % d);
    for (int r = r0; r < r1; ++r)
      acc = fmaf(dh[(size_t)r * 2 * F + m], xp[(size_t)(xrows ? xrows[r] / K : r) * d + c], acc);
    for (int g = 0; g < more.n; ++g) {
      const float *dh2 = (const float*)more.ops[g].dh, *xp2 = (const float*)more.ops[g].xp;
      for (int r = more.ops[g].offsets[e]; r < more.ops[g].offsets[e + 1]; ++r)
        acc = fmaf(dh2[(size_t)r * 2 * F + m], xp2[(size_t)r * d + c], acc);
    }
    o = dW_gu + (size_t)e * 2 * F * d + q;
  }
  *o = accumulate ? *o + acc : acc;
}

int launch_ffn_fwd_mfma(const moe_shape* s, const void* xp, const int32_t* xrows,
                        const int32_t* offsets, const int32_t* tile_offsets, const void* W_gu,
                        const void* W_down, void* h, void* a, void* yp, hipStream_t st,
                        const int32_t* yrows);
int launch_dgrad_weights_mfma(const moe_shape* s, const void* W_gu, const void* W_down,
                              void* ws, hipStream_t st);
int launch_ffn_dgrad_mfma(const moe_shape* s, const void* dyp, const void* h,
                          const int32_t* offsets, const int32_t* tile_offsets, const void* W_gu,
                          const void* W_down, void* dh, void* dxp, void* ws, bool weights_ready,
                          hipStream_t st, int parts, const FusedCombineBwd* fc);
int launch_ffn_wgrad_mfma(const moe_shape* s, const void* xp, const int32_t* xrows,
                          const void* a, const void* dh, const void* dyp,
                          const int32_t* offsets, float* dW_gu, float* dW_down, bool accumulate,
                          hipStream_t st, const int32_t* dyrows);

int launch_ffn_fwd(const moe_shape* s, const void* xp, const int32_t* xrows,
                   const int32_t* offsets, const int32_t* tile_offsets, const void* W_gu,
                   const void* W_down, void* h, void* a, void* yp, hipStream_t st,
                   const int32_t* yrows) {
  if (s->T == 0) return MOE_OK;
  if (is16(s))
    return launch_ffn_fwd_mfma(s, xp, xrows, offsets, tile_offsets, W_gu, W_down, h, a, yp, st,
                               yrows);
  const long cap = s->T * s->K;
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  MOE_LAUNCH("f32_gate_up", st,
             f32_gate_up_kernel<<<(unsigned)cdiv(cap * F, 256), 256, 0, st>>>(
      (const float*)xp, xrows, (int)s->K, offsets, (const float*)W_gu, (float*)h, (float*)a, cap, E_l, d, F));
  if (int rc = check_launch("f32 expert GEMM1")) return rc;
  MOE_LAUNCH("f32_down", st,
             f32_down_kernel<<<(unsigned)cdiv(cap * d, 256), 256, 0, st>>>(
      (const float*)a, offsets, (const float*)W_down, (float*)yp, cap, E_l, d, F, yrows));
  return check_launch("f32 expert GEMM2");
}

int launch_dgrad_weights(const moe_shape* s, const void* W_gu, const void* W_down, void* ws,
                         hipStream_t st) {
  if (s->T == 0 || !is16(s)) return MOE_OK;
  return launch_dgrad_weights_mfma(s, W_gu, W_down, ws, st);
}

int launch_ffn_dgrad(const moe_shape* s, const void* dyp, const void* h, const int32_t* offsets,
                     const int32_t* tile_offsets, const void* W_gu, const void* W_down, void* dh,
                     void* dxp, void* ws, bool weights_ready, hipStream_t st, int parts,
                     const FusedCombineBwd* fc) {
  if (s->T == 0) return MOE_OK;
  if (is16(s))
    return launch_ffn_dgrad_mfma(s, dyp, h, offsets, tile_offsets, W_gu, W_down, dh, dxp, ws,
                                 weights_ready, st, parts, fc);
  const long cap = s->T * s->K;
  const int d = (int)s->d, F = (int)s->F, E_l = (int)s->E_l;
  if (parts & kDgradAct) {
    MOE_LAUNCH("f32_dgrad_act", st,
               f32_dgrad_act_kernel<<<(unsigned)cdiv(cap * F, 256), 256, 0, st>>>(
        (const float*)dyp, fc ? fc->pair_of_row : nullptr, (int)s->K, fc ? fc->gates : nullptr,
        fc ? (float*)fc->ag : nullptr, (const float*)h, offsets, (const float*)W_down,
        (float*)dh, cap, E_l, d, F));
    if (int rc = check_launch("f32 dgrad (activation)")) return rc;
  }
  if (!(parts & kDgradIn)) return MOE_OK;
  MOE_LAUNCH("f32_dgrad_in", st,
             f32_dgrad_in_kernel<<<(unsigned)cdiv(cap * d, 256), 256, 0, st>>>(
      (const float*)dh, offsets, (const float*)W_gu, (float*)dxp, cap, E_l, d, F));
  return check_launch("f32 dgrad (input)");
}

int launch_ffn_wgrad(const moe_shape* s, const void* xp, const int32_t* xrows, const void* a,
                     const void* dh, const void* dyp, const int32_t* offsets, float* dW_gu,
                     float* dW_down, bool accumulate, hipStream_t st, const int32_t* dyrows) {
  if (is16(s))
    return launch_ffn_wgrad_mfma(s, xp, xrows, a, dh, dyp, offsets, dW_gu, dW_down, accumulate,
                                 st, dyrows);
  const long n = s->E_l * (s->d * s->F + 2 * s->F * s->d);
  MOE_LAUNCH("f32_wgrad", st,
             f32_wgrad_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(
      (const float*)xp, xrows, (int)s->K, (const float*)a, (const float*)dh, (const float*)dyp,
      dyrows, offsets, dW_gu, dW_down, (int)s->E_l, (int)s->d, (int)s->F, accumulate ? 1 : 0,
      WgrMoreF32{}));
  return check_launch("f32 wgrad");
}

int launch_ffn_wgrad_multi(const moe_shape* s, const WgrOps* ops, int n, float* dW_gu,
                           float* dW_down, bool accumulate, hipStream_t st) {
  if (is16(s)) return launch_ffn_wgrad_multi_mfma(s, ops, n, dW_gu, dW_down, accumulate, st);
  WgrMoreF32 more{};
  more.n = n - 1;
  for (int g = 0; g + 1 < n; ++g) more.ops[g] = ops[g + 1];
  const WgrOps& A = ops[0];
  const long cnt = s->E_l * (s->d * s->F + 2 * s->F * s->d);
  MOE_LAUNCH("f32_wgrad", st,
             f32_wgrad_kernel<<<(unsigned)cdiv(cnt, 256), 256, 0, st>>>(
      (const float*)A.xp, nullptr, (int)s->K, (const float*)A.a, (const float*)A.dh,
      (const float*)A.dyp, nullptr, A.offsets, dW_gu, dW_down, (int)s->E_l, (int)s->d,
      (int)s->F, accumulate ? 1 : 0, more));
  return check_launch("f32 grouped wgrad");
}

}  // namespace moe
