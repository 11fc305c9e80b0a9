// Routing: router scores, top-K selection with softmax gates, forced balance,
// and the router backward (gate Jacobian and router weight gradient).
//
// Routing is the step in front of the token dispatch the expert-parallel
// overlap pages describe (skill card page 1, "What it is"; "HybridEP benchmark":
// "Routing: force balance").  The pages do not give the routing function; this
// is top-K over router logits with a softmax over the selected logits.
#include "moe_internal.h"

#include <math.h>

namespace moe {

// ---------------------------------------------------------------------------
// W_rT[e][c] = W_r[c][e]: 32x32 tiles through LDS (coalesced both ways).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_wr_kernel(const T* __restrict__ W_r,
                                                           T* __restrict__ W_rT, int d, int E) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, e = e0 + tx;
    if (c < d && e < E) tile[i][tx] = W_r[(size_t)c * E + e];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int e = e0 + i, c = c0 + tx;
    if (c < d && e < E) W_rT[(size_t)e * d + c] = tile[tx][i];
  }
}

int launch_transpose_wr(const moe_shape* s, const void* W_r, void* W_rT, hipStream_t st) {
  dim3 grid((unsigned)cdiv(s->d, 32), (unsigned)cdiv(s->E, 32));
  if (is16(s))  // a 16-bit copy: the same kernel for bf16 and fp16
    MOE_LAUNCH("transpose_wr", st,
               transpose_wr_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)W_r, (uint16_t*)W_rT,
                                                        (int)s->d, (int)s->E));
  else
    MOE_LAUNCH("transpose_wr", st,
               transpose_wr_kernel<float><<<grid, 256, 0, st>>>((const float*)W_r, (float*)W_rT, (int)s->d,
                                                     (int)s->E));
  return check_launch("transpose W_r");
}

// ---------------------------------------------------------------------------
// float32 router logits: one thread per (t, e), float32 accumulation.
// (The 16-bit path uses the MFMA GEMM in gemm_mfma.hip.)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_f32_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ W_r,
                                                                const float* __restrict__ bias,
                                                                float* __restrict__ logits,
                                                                int T, int d, int E) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * d;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(xr[c], W_r[(size_t)c * E + e], acc);
  if (bias) acc += bias[e];
  logits[i] = acc;
}

int launch_router_logits_mfma(const moe_shape* s, const void* x, const void* W_rT,
                              const float* bias, float* logits, float* partial,
                              hipStream_t st);
int launch_router_wgrad_mfma(const moe_shape* s, const void* x, const void* dl_split,
                             float* partial, hipStream_t st);

int launch_router_logits(const moe_shape* s, const void* x, const void* W_r, const void* W_rT,
                         const float* bias, float* logits, hipStream_t st) {
  if (s->T == 0) return MOE_OK;
  // 16-bit: W_rT is the workspace base, the split-K partials follow it (with
  // more than one split the logits are finished by the top-k kernel)
  if (is16(s))
    return launch_router_logits_mfma(s, x, W_rT, bias, logits,
                                     (float*)((char*)W_rT + ws_wrt_bytes(s)), st);
  const long n = s->T * s->E;
  MOE_LAUNCH("router_logits_f32", st,
             router_logits_f32_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(
      (const float*)x, (const float*)W_r, bias, logits, (int)s->T, (int)s->d, (int)s->E));
  return check_launch("router logits f32");
}

// ---------------------------------------------------------------------------
// Top-K + softmax gates: one wave per token.  Each lane holds up to 8 logits
// (E <= 512).  K rounds of a wave-wide argmax; ties go to the lower expert
// index.  Lane k keeps selection k; gates = softmax over the selected logits.
// ---------------------------------------------------------------------------
// With partial set, the logits are first finished here: the sum of the router
// GEMM's split-K partials [splits][T][E] in split order, plus the bias, which
// is also written to logits.
__global__ __launch_bounds__(256) void topk_kernel(float* __restrict__ logits,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ gates, int T, int E,
                                                   int K, const float* __restrict__ partial,
                                                   int splits, const float* __restrict__ bias) {
  const int t = (int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;  // uniform per wave
  float* row = logits + (size_t)t * E;
  float v[8];
  if (partial) {  // uniform
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      if (e < E) {
        float acc = partial[(size_t)t * E + e];
        for (int sp = 1; sp < splits; ++sp) acc += partial[((size_t)sp * T + t) * E + e];
        if (bias) acc += bias[e];
        row[e] = acc;
        v[j] = acc;
      } else {
        v[j] = 0.f;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? row[e] : 0.f;
    }
  }
  unsigned taken = 0;
  float selv = 0.f;
  int seli = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((taken >> j) & 1u)) {
        if (bi == 0x7fffffff || v[j] > bv) {
          bv = v[j];
          bi = e;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == k) {
      selv = bv;
      seli = bi;
    }
  }
  const float m = __shfl(selv, 0, 64);
  const float ex = lane < K ? expf(selv - m) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < K) {
    idx[(size_t)t * K + lane] = seli;
    gates[(size_t)t * K + lane] = ex / sum;
  }
}

int launch_topk(const moe_shape* s, float* logits, int32_t* idx, float* gates,
                const void* ws, const float* bias, hipStream_t st) {
  if (s->T == 0) return MOE_OK;
  // ws set: the logits are the router GEMM's split-K partials (in ws after the
  // transposed router weights) when it ran with more than one split
  const int splits = ws ? router_splits(s) : 1;
  const float* partial =
      splits > 1 ? (const float*)((const char*)ws + ws_wrt_bytes(s)) : nullptr;
  MOE_LAUNCH("topk", st,
             topk_kernel<<<(unsigned)cdiv(s->T, 4), 256, 0, st>>>(
                 logits, idx, gates, (int)s->T, (int)s->E, (int)s->K, partial, splits, bias));
  return check_launch("top-k");
}

__global__ __launch_bounds__(256) void force_balance_kernel(int32_t* __restrict__ idx, long n,
                                                            int E) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p < n) idx[p] = (int32_t)(p % E);  // p = t*K + k
}

int launch_force_balance(const moe_shape* s, int32_t* idx, hipStream_t st) {
  const long n = s->T * s->K;
  if (n == 0) return MOE_OK;
  MOE_LAUNCH("force_balance", st,
             force_balance_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(idx, n, (int)s->E));
  return check_launch("force balance");
}

// ---------------------------------------------------------------------------
// Router backward.
// dlogits: one wave per token; lane k < K holds slot k.  Every lane writes its
// own logits' final value once (0 unless selected).
// ---------------------------------------------------------------------------
// With split set, dlogits is also written as two bf16 terms, split[t][e] =
// hi = bf16(v) and split[t][E + e] = lo = bf16(v - hi), for the matrix-core
// weight gradient (hi + lo carries about 16 significant bits of v).
__global__ __launch_bounds__(256) void dlogits_kernel(const float* __restrict__ dgates,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ idx,
                                                      float* __restrict__ dlogits,
                                                      uint16_t* __restrict__ split, int T, int E,
                                                      int K) {
  const int t = (int)(((long)blockIdx.x * 256 + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  float g = 0.f, dg = 0.f;
  int e_sel = -1;
  if (lane < K) {
    g = gates[(size_t)t * K + lane];
    dg = dgates[(size_t)t * K + lane];
    e_sel = idx[(size_t)t * K + lane];
  }
  const float inner = wave_sum(g * dg);
  const float dsel = g * (dg - inner);
  float* out = dlogits + (size_t)t * E;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    float val = 0.f;
    for (int k = 0; k < K; ++k) {
      const int ek = __shfl(e_sel, k, 64);
      const float dk = __shfl(dsel, k, 64);
      if (ek == e) val += dk;
    }
    if (e < E) {
      out[e] = val;
      if (split) {
        const uint16_t hi = f2bf(val);
        split[(size_t)t * 2 * E + e] = hi;
        split[(size_t)t * 2 * E + E + e] = f2bf(val - bf2f(hi));
      }
    }
  }
}

// dW_r partials: block = 64 columns c x 64 experts e over one chunk of tokens.
// partial[chunk][c][e] = sum_{t in chunk} x[t][c] * dlogits[t][e].  Each
// thread owns a 4 x 4 piece (columns 4*(tid%16).., experts 4*(tid/16)..), so
// a 32-token slab staged in LDS feeds 16 FMAs per two 16-byte LDS reads.
template <typename T>
__global__ __launch_bounds__(256) void dwr_partial_kernel(const T* __restrict__ x,
                                                          const float* __restrict__ dl,
                                                          float* __restrict__ partial, int T_,
                                                          int d, int E) {
  __shared__ __attribute__((aligned(16))) float xs[32][68];
  __shared__ __attribute__((aligned(16))) float ds[32][68];
  const int c0 = blockIdx.x * 64, e0 = blockIdx.z * 64;
  const int chunk = blockIdx.y;
  const int t_begin = chunk * kRouterChunk;
  const int t_end = min(T_, t_begin + kRouterChunk);
  const int tid = threadIdx.x;
  const int ci = (tid & 15) * 4, ei = (tid >> 4) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int t0 = t_begin; t0 < t_end; t0 += 32) {
    for (int i = tid; i < 32 * 64; i += 256) {
      const int tt = i >> 6, cc = i & 63;
      const int t = t0 + tt;
      xs[tt][cc] = (t < t_end && c0 + cc < d) ? Elt<T>::ld(x + (size_t)t * d + c0 + cc) : 0.f;
      ds[tt][cc] = (t < t_end && e0 + cc < E) ? dl[(size_t)t * E + e0 + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int tt = 0; tt < 32; ++tt) {
      const float4 xv = *(const float4*)&xs[tt][ci];
      const float4 dv = *(const float4*)&ds[tt][ei];
      const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
      const float da[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], da[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (c0 + ci + i >= d) continue;
    float* out = partial + ((size_t)chunk * d + c0 + ci + i) * E + e0 + ei;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e0 + ei + j < E) out[j] = acc[i][j];
  }
}

// dW_r from the matrix-core partials: partial[c][i][f], f < 2E, of chunk c;
// dW_r[i][e] = [dW_r] + sum_c (partial[c][i][e] + partial[c][i][E + e]) in
// chunk order.
__global__ __launch_bounds__(256) void dwr_reduce_split_kernel(const float* __restrict__ partial,
                                                               float* __restrict__ dW_r, int d,
                                                               int E, int nchunks,
                                                               int accumulate) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)d * E) return;
  const long row = i / E, e = i % E;
  float acc = accumulate ? dW_r[i] : 0.f;
  for (int ch = 0; ch < nchunks; ++ch) {
    const float* p = partial + ((size_t)ch * d + row) * 2 * E;
    acc += p[e] + p[E + e];
  }
  dW_r[i] = acc;
}

__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float* __restrict__ partial,
                                                         float* __restrict__ dW_r, long n,
                                                         int nchunks, int accumulate) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = accumulate ? dW_r[i] : 0.f;
  for (int ch = 0; ch < nchunks; ++ch) acc += partial[(size_t)ch * n + i];
  dW_r[i] = acc;
}

int launch_route_bwd(const moe_shape* s, const float* dgates, const float* gates,
                     const int32_t* idx, const void* x, float* dlogits, float* dW_r,
                     bool accumulate, void* ws, hipStream_t st) {
  // bf16 data: dW_r = x^T dlogits on the matrix cores from a two-term bf16
  // split of dlogits (the workspace holds the split, then the partials)
  const bool mfma = x && dW_r && s->dtype == MOE_BF16 && s->T > 0;
  uint16_t* split = mfma ? (uint16_t*)ws : nullptr;
  if (s->T > 0) {
    MOE_LAUNCH("dlogits", st,
               dlogits_kernel<<<(unsigned)cdiv(s->T, 4), 256, 0, st>>>(
                   dgates, gates, idx, dlogits, split, (int)s->T, (int)s->E, (int)s->K));
    int rc = check_launch("router dlogits");
    if (rc) return rc;
  }
  if (!x || !dW_r) return MOE_OK;
  if (mfma) {
    float* partial = (float*)((char*)ws + ws_router_split_bytes(s));
    if (int rc = launch_router_wgrad_mfma(s, x, split, partial, st)) return rc;
    const int nchunks = (int)cdiv(s->T, router_mfma_chunk(s->T));
    const long n = s->d * s->E;
    MOE_LAUNCH("dwr_reduce", st,
               dwr_reduce_split_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(
                   partial, dW_r, (int)s->d, (int)s->E, nchunks, accumulate ? 1 : 0));
    return check_launch("router dW_r reduce");
  }
  const int nchunks = (int)cdiv(s->T, kRouterChunk);
  float* partial = (float*)ws;
  if (nchunks > 0) {
    dim3 grid((unsigned)cdiv(s->d, 64), (unsigned)nchunks, (unsigned)cdiv(s->E, 64));
    if (s->dtype == MOE_BF16)
      MOE_LAUNCH("dwr_partial", st,
                 dwr_partial_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, dlogits, partial,
                                                         (int)s->T, (int)s->d, (int)s->E));
    else if (s->dtype == MOE_F16)
      MOE_LAUNCH("dwr_partial", st,
                 dwr_partial_kernel<_Float16><<<grid, 256, 0, st>>>((const _Float16*)x, dlogits,
                                                                    partial, (int)s->T,
                                                                    (int)s->d, (int)s->E));
    else
      MOE_LAUNCH("dwr_partial", st,
                 dwr_partial_kernel<float><<<grid, 256, 0, st>>>((const float*)x, dlogits, partial,
                                                      (int)s->T, (int)s->d, (int)s->E));
    int rc = check_launch("router dW_r partial");
    if (rc) return rc;
  }
  const long n = s->d * s->E;
  MOE_LAUNCH("dwr_reduce", st,
             dwr_reduce_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(partial, dW_r, n, nchunks,
                                                            accumulate ? 1 : 0));
  return check_launch("router dW_r reduce");
}

}  // namespace moe
