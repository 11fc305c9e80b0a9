// libmoe C ABI: host-side validation, launch sequencing and the two-stream
// two-micro-batch step.  Every entry point validates all of its arguments
// before the first launch, so a rejected call writes nothing.
#include "moe_internal.h"

#include <dlfcn.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

namespace moe {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Phase ranges for profilers.  With MOE_ROCTX=1 in the environment (read
// once), each phase of the step (route, dispatch, expert forward, combine and
// their backwards, the weight gradients) is bracketed by a roctx range
// ("moe.<phase>"), which rocprofv3 --marker-trace records: host-side ranges
// around the phase's launches, from which a trace maps each kernel to its
// phase through its launch call.  The roctx library is opened at run time, so
// the library has no link dependency on it; without the variable (or without
// the library) a phase costs one predictable branch.
// ---------------------------------------------------------------------------
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};
static const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx x;
    const char* e = getenv("MOE_ROCTX");
    if (!e || strcmp(e, "1") != 0) return x;
    for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"}) {
      void* h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
      if (!h) continue;
      x.push = (int (*)(const char*))dlsym(h, "roctxRangePushA");
      x.pop = (int (*)())dlsym(h, "roctxRangePop");
      if (x.push && x.pop) return x;
      x = Roctx{};
    }
    return x;
  }();
  return r;
}
struct PhaseRange {
  const bool on;
  explicit PhaseRange(const char* name) : on(roctx().push != nullptr) {
    if (on) roctx().push(name);
  }
  ~PhaseRange() {
    if (on) roctx().pop();
  }
};

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
struct TimingState {
  std::mutex mu;
  bool on = false;
  int cap = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;  // 2 per record
  std::vector<const char*> name;
};
static TimingState g_timing;

KernelTimer::KernelTimer(const char* nm, hipStream_t st) : stream(st) {
  if (!__atomic_load_n(&g_timing.on, __ATOMIC_ACQUIRE)) return;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (!g_timing.on || g_timing.used >= g_timing.cap) return;
  slot = g_timing.used++;
  g_timing.name[slot] = nm;
  if (hipEventRecord(g_timing.ev[2 * slot], st) != hipSuccess) slot = -1;
}

void KernelTimer::stop() {
  if (slot >= 0) (void)hipEventRecord(g_timing.ev[2 * slot + 1], stream);
  slot = -1;
}

static int validate_shape(const moe_shape* s) {
  if (!s) return set_error(MOE_ERR_NULL, "shape is NULL");
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16 && s->dtype != MOE_F16)
    return set_error(MOE_ERR_DTYPE, "dtype %d is not MOE_F32, MOE_BF16 or MOE_F16", s->dtype);
  if (s->reserved != 0) return set_error(MOE_ERR_ARG, "shape.reserved must be 0");
  if (s->T < 0) return set_error(MOE_ERR_SHAPE, "T = %lld < 0", (long long)s->T);
  if (s->E < 1 || s->E > 512)
    return set_error(MOE_ERR_SHAPE, "E = %lld outside [1, 512]", (long long)s->E);
  if (s->K < 1 || s->K > 16 || s->K > s->E)
    return set_error(MOE_ERR_SHAPE, "K = %lld outside [1, min(E, 16)]", (long long)s->K);
  if (s->E_l < 1 || s->E_l > 256 || s->e_lo < 0 || s->e_lo + s->E_l > s->E)
    return set_error(MOE_ERR_SHAPE, "local window [%lld, %lld) invalid for E = %lld",
                     (long long)s->e_lo, (long long)(s->e_lo + s->E_l), (long long)s->E);
  if (s->d < 64 || s->d > 16384 || s->d % 64)
    return set_error(MOE_ERR_SHAPE, "d = %lld must be a multiple of 64 in [64, 16384]",
                     (long long)s->d);
  if (s->F < 64 || s->F > 16384 || s->F % 64)
    return set_error(MOE_ERR_SHAPE, "F = %lld must be a multiple of 64 in [64, 16384]",
                     (long long)s->F);
  if (s->T * s->K >= (1LL << 31) || s->T * s->E >= (1LL << 31))
    return set_error(MOE_ERR_SHAPE, "T*K and T*E must be < 2^31");
  return MOE_OK;
}

#define REQUIRE(p)                                                               \
  do {                                                                           \
    if (!(p)) return set_error(MOE_ERR_NULL, "%s: %s is NULL", __func__, #p);    \
  } while (0)

static size_t ws_one(const moe_shape* s) {
  size_t b = ws_plan_bytes(s);
  if (ws_wrt_bytes(s) > b) b = ws_wrt_bytes(s);
  if (ws_router_partial_bytes(s) > b) b = ws_router_partial_bytes(s);
  if (ws_wT_offset(s) + ws_wT_bytes(s) > b) b = ws_wT_offset(s) + ws_wT_bytes(s);
  return b < 256 ? 256 : b;
}

static int need_ws(const char* fn, size_t have, size_t need) {
  if (have < need)
    return set_error(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu required", fn, have,
                     need);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// unvalidated bodies (arguments checked by the callers)
// ---------------------------------------------------------------------------
static int do_route(const moe_shape* s, int mode, const void* x, const void* W_r,
                    const float* bias, float* logits, int32_t* idx, float* gates, void* ws,
                    hipStream_t st) {
  int rc;
  if (mode == MOE_ROUTE_FORCE_BALANCE) return launch_force_balance(s, idx, st);
  if (mode == MOE_ROUTE_TOPK) {
    if (is16(s) && s->T > 0) {
      if ((rc = launch_transpose_wr(s, W_r, ws, st))) return rc;
    }
    if ((rc = launch_router_logits(s, x, W_r, ws, bias, logits, st))) return rc;
    return launch_topk(s, logits, idx, gates, is16(s) ? ws : nullptr, bias, st);
  }
  return launch_topk(s, logits, idx, gates, nullptr, nullptr, st);
}

// xp == NULL: the plan only (fused permute)
static int do_dispatch(const moe_shape* s, const void* x, const int32_t* idx, int32_t* counts,
                       int32_t* offsets, int32_t* row_of_pair, int32_t* pair_of_row,
                       int32_t* tile_offsets, void* xp, void* ws, hipStream_t st) {
  int rc = launch_plan(s, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets, ws, st);
  if (rc || !xp) return rc;
  return launch_permute(s, x, row_of_pair, xp, st);
}

// The shared expert as a grouped-GEMM shape: one expert over all T rows.
static moe_shape shared_shape(const moe_shape* s, int64_t F_s) {
  moe_shape ss = *s;
  ss.F = F_s;
  ss.E = 1;
  ss.e_lo = 0;
  ss.E_l = 1;
  ss.K = 1;
  return ss;
}
static int validate_shared(int64_t F_s) {
  if (F_s < 64 || F_s > 16384 || F_s % 64)
    return set_error(MOE_ERR_SHAPE, "F_s = %lld must be a multiple of 64 in [64, 16384]",
                     (long long)F_s);
  return MOE_OK;
}
// Shared-expert workspace: its 4-entry plan in the first 256 bytes, then the
// layout of a grouped call on the shared shape (the dgrad's weight copies).
constexpr size_t kSharedPlanBytes = 256;
static size_t ws_shared(const moe_shape* s, int64_t F_s) {
  const moe_shape ss = shared_shape(s, F_s);
  return kSharedPlanBytes + ws_wT_offset(&ss) + ws_wT_bytes(&ss);
}
static int do_shared_fwd(const moe_shape* s, int64_t F_s, const void* x, const void* W_gu_s,
                         const void* W_down_s, void* h_s, void* a_s, void* y_s, void* ws,
                         hipStream_t st) {
  if (s->T == 0) return MOE_OK;
  const moe_shape ss = shared_shape(s, F_s);
  int32_t* plan = (int32_t*)ws;
  if (int rc = launch_shared_plan(s->T, plan, st)) return rc;
  return launch_ffn_fwd(&ss, x, nullptr, plan, plan + 2, W_gu_s, W_down_s, h_s, a_s, y_s, st);
}
static int do_shared_dgrad(const moe_shape* s, int64_t F_s, const void* dout, const void* h_s,
                           const void* W_gu_s, const void* W_down_s, void* dh_s, void* dx_s,
                           void* ws, hipStream_t st) {
  if (s->T == 0) return MOE_OK;
  const moe_shape ss = shared_shape(s, F_s);
  int32_t* plan = (int32_t*)ws;
  if (int rc = launch_shared_plan(s->T, plan, st)) return rc;
  return launch_ffn_dgrad(&ss, dout, h_s, plan, plan + 2, W_gu_s, W_down_s, dh_s, dx_s,
                          (char*)ws + kSharedPlanBytes, false, st);
}
static int do_shared_wgrad(const moe_shape* s, int64_t F_s, const void* x, const void* a_s,
                           const void* dh_s, const void* dout, float* dW_gu_s, float* dW_down_s,
                           bool accumulate, void* ws, hipStream_t st) {
  const moe_shape ss = shared_shape(s, F_s);
  int32_t* plan = (int32_t*)ws;
  if (int rc = launch_shared_plan(s->T, plan, st)) return rc;
  return launch_ffn_wgrad(&ss, x, nullptr, a_s, dh_s, dout, plan, dW_gu_s, dW_down_s, accumulate,
                          st);
}

// The gathering GEMMs (fused permute, fused combine backward) address the
// token matrices x and dout [T][d] with 32-bit byte offsets.
static int check_gather_x(const moe_shape* s, const char* fn) {
  const int64_t es = (int64_t)elt_bytes(s);
  if (s->T * s->d * es >= (1LL << 31))
    return set_error(MOE_ERR_SHAPE,
                     "%s: a [T,d] token matrix is %lld bytes, the gathering GEMMs need < 2^31",
                     fn, (long long)(s->T * s->d * es));
  return MOE_OK;
}

static int do_dispatch_bwd(const moe_shape* s, const void* dxp, const int32_t* row_of_pair,
                           const int32_t* idx, const float* dlogits, const void* W_r, void* dx,
                           bool accumulate, void* ws, hipStream_t st, const void* add = nullptr) {
  if (dlogits && s->T > 0) {
    int rc = launch_transpose_wr(s, W_r, ws, st);
    if (rc) return rc;
  }
  return launch_dispatch_bwd(s, dxp, row_of_pair, idx, dlogits, ws, add, dx, accumulate, st);
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s) {
  if (validate_shape(s)) return 0;
  return ws_one(s);
}

size_t moe_step_workspace_bytes(const moe_shape* s) {
  if (validate_shape(s)) return 0;
  return 2 * ws_one(s);
}

size_t moe_shared_workspace_bytes(const moe_shape* s, int64_t F_s) {
  if (validate_shape(s) || validate_shared(F_s)) return 0;
  return ws_shared(s, F_s);
}

size_t moe_step_workspace_bytes_shared(const moe_shape* s, int64_t F_s) {
  if (validate_shape(s)) return 0;
  if (F_s == 0) return 2 * ws_one(s);
  if (validate_shared(F_s)) return 0;
  return 2 * ws_one(s) + 2 * ws_shared(s, F_s);
}

int moe_tile_m(void) { return kTileM; }

const char* moe_last_error(void) { return g_err; }

int moe_version(void) { return 100; }

int moe_timing_enable(int max_records) {
  if (max_records < 1) return set_error(MOE_ERR_SHAPE, "moe_timing_enable: max_records < 1");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  while ((int)g_timing.name.size() < max_records) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess)
      return set_error(MOE_ERR_HIP, "moe_timing_enable: hipEventCreate failed");
    g_timing.ev.push_back(a);
    g_timing.ev.push_back(b);
    g_timing.name.push_back(nullptr);
  }
  g_timing.cap = max_records;
  __atomic_store_n(&g_timing.on, true, __ATOMIC_RELEASE);
  return MOE_OK;
}

int moe_timing_disable(void) {
  __atomic_store_n(&g_timing.on, false, __ATOMIC_RELEASE);
  return MOE_OK;
}

int moe_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.used = 0;
  return MOE_OK;
}

int moe_timing_report(int i, char* name, size_t name_len, double* total_ms, int* launches) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  std::vector<const char*> names;
  for (int r = 0; r < g_timing.used; ++r) {
    bool seen = false;
    for (const char* n : names) seen |= (strcmp(n, g_timing.name[r]) == 0);
    if (!seen) names.push_back(g_timing.name[r]);
  }
  if (i < 0 || i >= (int)names.size()) return (int)names.size();
  double tot = 0.0;
  int cnt = 0;
  for (int r = 0; r < g_timing.used; ++r) {
    if (strcmp(g_timing.name[r], names[i]) != 0) continue;
    float ms = 0.f;
    if (hipEventSynchronize(g_timing.ev[2 * r + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timing.ev[2 * r], g_timing.ev[2 * r + 1]) != hipSuccess)
      return set_error(MOE_ERR_HIP, "moe_timing_report: event query failed");
    tot += ms;
    ++cnt;
  }
  if (name && name_len) {
    snprintf(name, name_len, "%s", names[i]);
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = cnt;
  return (int)names.size();
}

int moe_route(const moe_shape* s, int mode, const void* x, const void* W_r, const float* bias,
              float* logits, int32_t* idx, float* gates, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(idx);
  switch (mode) {
    case MOE_ROUTE_TOPK:
      REQUIRE(x);
      REQUIRE(W_r);
      REQUIRE(logits);
      REQUIRE(gates);
      if (is16(s)) {
        REQUIRE(ws);
        if (int rc = need_ws(__func__, ws_bytes, ws_wrt_bytes(s) + ws_router_fwd_bytes(s)))
          return rc;
      }
      break;
    case MOE_ROUTE_TOPK_FROM_LOGITS:
      REQUIRE(logits);
      REQUIRE(gates);
      break;
    case MOE_ROUTE_FORCE_BALANCE:
      break;
    default:
      return set_error(MOE_ERR_ARG, "moe_route: unknown mode %d", mode);
  }
  return do_route(s, mode, x, W_r, bias, logits, idx, gates, ws, stream);
}

int moe_dispatch(const moe_shape* s, const void* x, const int32_t* idx, int32_t* counts,
                 int32_t* offsets, int32_t* row_of_pair, int32_t* pair_of_row,
                 int32_t* tile_offsets, void* xp, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (xp) REQUIRE(x);
  REQUIRE(idx);
  REQUIRE(counts);
  REQUIRE(offsets);
  REQUIRE(row_of_pair);
  REQUIRE(pair_of_row);
  REQUIRE(tile_offsets);
  REQUIRE(ws);
  if (int rc = need_ws(__func__, ws_bytes, ws_plan_bytes(s))) return rc;
  return do_dispatch(s, x, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets, xp, ws,
                     stream);
}

int moe_expert_ffn_fwd(const moe_shape* s, const void* xp, const int32_t* offsets,
                       const int32_t* tile_offsets, const void* W_gu, const void* W_down,
                       void* h, void* a, void* yp, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(xp);
  REQUIRE(offsets);
  REQUIRE(tile_offsets);
  REQUIRE(W_gu);
  REQUIRE(W_down);
  REQUIRE(h);
  REQUIRE(a);
  REQUIRE(yp);
  return launch_ffn_fwd(s, xp, nullptr, offsets, tile_offsets, W_gu, W_down, h, a, yp, stream);
}

int moe_expert_ffn_fwd_gather(const moe_shape* s, const void* x, const int32_t* pair_of_row,
                              const int32_t* offsets, const int32_t* tile_offsets,
                              const void* W_gu, const void* W_down, void* h, void* a, void* yp,
                              hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(x);
  REQUIRE(pair_of_row);
  REQUIRE(offsets);
  REQUIRE(tile_offsets);
  REQUIRE(W_gu);
  REQUIRE(W_down);
  REQUIRE(h);
  REQUIRE(a);
  REQUIRE(yp);
  if (int rc = check_gather_x(s, __func__)) return rc;
  return launch_ffn_fwd(s, x, pair_of_row, offsets, tile_offsets, W_gu, W_down, h, a, yp,
                        stream);
}

int moe_combine(const moe_shape* s, const void* yp, const float* gates,
                const int32_t* row_of_pair, void* out, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(yp);
  REQUIRE(gates);
  REQUIRE(row_of_pair);
  REQUIRE(out);
  return launch_combine(s, yp, gates, row_of_pair, nullptr, out, stream);
}

int moe_combine_bwd(const moe_shape* s, const void* dout, const void* yp, const float* gates,
                    const int32_t* row_of_pair, void* dyp, float* dgates, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(dout);
  REQUIRE(yp);
  REQUIRE(gates);
  REQUIRE(row_of_pair);
  REQUIRE(dgates);
  return launch_combine_bwd(s, dout, yp, gates, row_of_pair, dyp, dgates, stream);
}

int moe_expert_ffn_fwd_scatter(const moe_shape* s, const void* xp, const void* x,
                               const int32_t* pair_of_row, const int32_t* offsets,
                               const int32_t* tile_offsets, const void* W_gu, const void* W_down,
                               void* h, void* a, void* yq, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (!xp && !x) return set_error(MOE_ERR_NULL, "%s: xp and x are both NULL", __func__);
  REQUIRE(pair_of_row);
  REQUIRE(offsets);
  REQUIRE(tile_offsets);
  REQUIRE(W_gu);
  REQUIRE(W_down);
  REQUIRE(h);
  REQUIRE(a);
  REQUIRE(yq);
  if (!xp)
    if (int rc = check_gather_x(s, __func__)) return rc;
  return launch_ffn_fwd(s, xp ? xp : x, xp ? nullptr : pair_of_row, offsets, tile_offsets, W_gu,
                        W_down, h, a, yq, stream, pair_of_row);
}

int moe_combine_pairs(const moe_shape* s, const void* yq, const float* gates,
                      const int32_t* row_of_pair, void* out, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(yq);
  REQUIRE(gates);
  REQUIRE(row_of_pair);
  REQUIRE(out);
  return launch_combine(s, yq, gates, row_of_pair, nullptr, out, stream, true);
}

int moe_combine_bwd_pairs(const moe_shape* s, const void* dout, const void* yq,
                          const float* gates, const int32_t* row_of_pair, void* dyp,
                          float* dgates, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(dout);
  REQUIRE(yq);
  REQUIRE(gates);
  REQUIRE(row_of_pair);
  REQUIRE(dgates);
  return launch_combine_bwd(s, dout, yq, gates, row_of_pair, dyp, dgates, stream, true);
}

int moe_ffn_dgrad(const moe_shape* s, const void* dyp, const void* h, const int32_t* offsets,
                  const int32_t* tile_offsets, const void* W_gu, const void* W_down, void* dh,
                  void* dxp, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(dyp);
  REQUIRE(h);
  REQUIRE(offsets);
  REQUIRE(tile_offsets);
  REQUIRE(W_gu);
  REQUIRE(W_down);
  REQUIRE(dh);
  REQUIRE(dxp);
  if (is16(s)) {
    REQUIRE(ws);
    if (int rc = need_ws(__func__, ws_bytes, ws_wT_offset(s) + ws_wT_bytes(s))) return rc;
  }
  return launch_ffn_dgrad(s, dyp, h, offsets, tile_offsets, W_gu, W_down, dh, dxp, ws, false,
                          stream);
}

int moe_ffn_wgrad(const moe_shape* s, const void* xp, const void* a, const void* dh,
                  const void* dyp, const int32_t* offsets, float* dW_gu, float* dW_down,
                  int accumulate, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(xp);
  REQUIRE(a);
  REQUIRE(dh);
  REQUIRE(dyp);
  REQUIRE(offsets);
  REQUIRE(dW_gu);
  REQUIRE(dW_down);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_ffn_wgrad: unknown accumulate bits 0x%x", accumulate);
  return launch_ffn_wgrad(s, xp, nullptr, a, dh, dyp, offsets, dW_gu, dW_down,
                          (accumulate & MOE_ACCUM_DW) != 0, stream);
}

int moe_ffn_wgrad_pair(const moe_shape* s, const void* xp, const void* a, const void* dh,
                       const void* dyp, const int32_t* offsets, const void* xp2,
                       const void* a2, const void* dh2, const void* dyp2,
                       const int32_t* offsets2, float* dW_gu, float* dW_down, int accumulate,
                       hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(xp);
  REQUIRE(a);
  REQUIRE(dh);
  REQUIRE(dyp);
  REQUIRE(offsets);
  REQUIRE(xp2);
  REQUIRE(a2);
  REQUIRE(dh2);
  REQUIRE(dyp2);
  REQUIRE(offsets2);
  REQUIRE(dW_gu);
  REQUIRE(dW_down);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_ffn_wgrad_pair: unknown accumulate bits 0x%x",
                     accumulate);
  const WgrOps ops[2] = {WgrOps{xp, a, dh, dyp, offsets}, WgrOps{xp2, a2, dh2, dyp2, offsets2}};
  return launch_ffn_wgrad_multi(s, ops, 2, dW_gu, dW_down, (accumulate & MOE_ACCUM_DW) != 0,
                                stream);
}

int moe_ffn_wgrad_multi(const moe_shape* s, int n, const moe_wgrad_ops* ops, float* dW_gu,
                        float* dW_down, int accumulate, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(ops);
  REQUIRE(dW_gu);
  REQUIRE(dW_down);
  if (n < 1 || n > kWgGroupMax)
    return set_error(MOE_ERR_ARG, "moe_ffn_wgrad_multi: n = %d outside [1, %d]", n,
                     kWgGroupMax);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_ffn_wgrad_multi: unknown accumulate bits 0x%x",
                     accumulate);
  WgrOps w[kWgGroupMax];
  for (int i = 0; i < n; ++i) {
    const moe_wgrad_ops& o = ops[i];
    if (!o.xp || !o.a || !o.dh || !o.dyp || !o.offsets)
      return set_error(MOE_ERR_NULL, "moe_ffn_wgrad_multi: an operand of micro-batch %d is NULL",
                       i);
    w[i] = WgrOps{o.xp, o.a, o.dh, o.dyp, o.offsets};
  }
  const bool acc = (accumulate & MOE_ACCUM_DW) != 0;
  if (n == 1)
    return launch_ffn_wgrad(s, w[0].xp, nullptr, w[0].a, w[0].dh, w[0].dyp, w[0].offsets, dW_gu,
                            dW_down, acc, stream);
  return launch_ffn_wgrad_multi(s, w, n, dW_gu, dW_down, acc, stream);
}

int moe_ffn_wgrad_gather(const moe_shape* s, const void* x, const int32_t* pair_of_row,
                         const void* a, const void* dh, const void* dyp, const int32_t* offsets,
                         float* dW_gu, float* dW_down, int accumulate, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(x);
  REQUIRE(pair_of_row);
  REQUIRE(a);
  REQUIRE(dh);
  REQUIRE(dyp);
  REQUIRE(offsets);
  REQUIRE(dW_gu);
  REQUIRE(dW_down);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_ffn_wgrad_gather: unknown accumulate bits 0x%x",
                     accumulate);
  if (int rc = check_gather_x(s, __func__)) return rc;
  return launch_ffn_wgrad(s, x, pair_of_row, a, dh, dyp, offsets, dW_gu, dW_down,
                          (accumulate & MOE_ACCUM_DW) != 0, stream);
}

int moe_ffn_dgrad_gather(const moe_shape* s, const void* dout, const int32_t* pair_of_row,
                         const float* gates, const void* h, const int32_t* offsets,
                         const int32_t* tile_offsets, const void* W_gu, const void* W_down,
                         void* dh, void* dxp, void* ag, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(dout);
  REQUIRE(pair_of_row);
  REQUIRE(gates);
  REQUIRE(h);
  REQUIRE(offsets);
  REQUIRE(tile_offsets);
  REQUIRE(W_gu);
  REQUIRE(W_down);
  REQUIRE(dh);
  REQUIRE(dxp);
  REQUIRE(ag);
  if (int rc = check_gather_x(s, __func__)) return rc;
  if (is16(s)) {
    REQUIRE(ws);
    if (int rc = need_ws(__func__, ws_bytes, ws_wT_offset(s) + ws_wT_bytes(s))) return rc;
  }
  const FusedCombineBwd fc{pair_of_row, gates, ag};
  return launch_ffn_dgrad(s, dout, h, offsets, tile_offsets, W_gu, W_down, dh, dxp, ws, false,
                          stream, kDgradBoth, &fc);
}

int moe_ffn_wgrad_fused(const moe_shape* s, const void* xp, const void* x,
                        const int32_t* pair_of_row, const void* ag, const void* dh,
                        const void* dout, const int32_t* offsets, float* dW_gu, float* dW_down,
                        int accumulate, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (!xp) REQUIRE(x);
  REQUIRE(pair_of_row);
  REQUIRE(ag);
  REQUIRE(dh);
  REQUIRE(dout);
  REQUIRE(offsets);
  REQUIRE(dW_gu);
  REQUIRE(dW_down);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_ffn_wgrad_fused: unknown accumulate bits 0x%x",
                     accumulate);
  if (int rc = check_gather_x(s, __func__)) return rc;
  return launch_ffn_wgrad(s, xp ? xp : x, xp ? nullptr : pair_of_row, ag, dh, dout, offsets,
                          dW_gu, dW_down, (accumulate & MOE_ACCUM_DW) != 0, stream, pair_of_row);
}

int moe_shared_expert_fwd(const moe_shape* s, int64_t F_s, const void* x, const void* W_gu_s,
                          const void* W_down_s, void* h_s, void* a_s, void* y_s, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (int rc = validate_shared(F_s)) return rc;
  REQUIRE(x);
  REQUIRE(W_gu_s);
  REQUIRE(W_down_s);
  REQUIRE(h_s);
  REQUIRE(a_s);
  REQUIRE(y_s);
  REQUIRE(ws);
  if (int rc = need_ws(__func__, ws_bytes, ws_shared(s, F_s))) return rc;
  return do_shared_fwd(s, F_s, x, W_gu_s, W_down_s, h_s, a_s, y_s, ws, stream);
}

int moe_shared_expert_dgrad(const moe_shape* s, int64_t F_s, const void* dout, const void* h_s,
                            const void* W_gu_s, const void* W_down_s, void* dh_s, void* dx_s,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (int rc = validate_shared(F_s)) return rc;
  REQUIRE(dout);
  REQUIRE(h_s);
  REQUIRE(W_gu_s);
  REQUIRE(W_down_s);
  REQUIRE(dh_s);
  REQUIRE(dx_s);
  REQUIRE(ws);
  if (int rc = need_ws(__func__, ws_bytes, ws_shared(s, F_s))) return rc;
  return do_shared_dgrad(s, F_s, dout, h_s, W_gu_s, W_down_s, dh_s, dx_s, ws, stream);
}

int moe_shared_expert_wgrad(const moe_shape* s, int64_t F_s, const void* x, const void* a_s,
                            const void* dh_s, const void* dout, float* dW_gu_s,
                            float* dW_down_s, int accumulate, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (int rc = validate_shared(F_s)) return rc;
  REQUIRE(x);
  REQUIRE(a_s);
  REQUIRE(dh_s);
  REQUIRE(dout);
  REQUIRE(dW_gu_s);
  REQUIRE(dW_down_s);
  REQUIRE(ws);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_shared_expert_wgrad: unknown accumulate bits 0x%x",
                     accumulate);
  if (int rc = need_ws(__func__, ws_bytes, ws_shared(s, F_s))) return rc;
  return do_shared_wgrad(s, F_s, x, a_s, dh_s, dout, dW_gu_s, dW_down_s,
                         (accumulate & MOE_ACCUM_DW) != 0, ws, stream);
}

int moe_route_bwd(const moe_shape* s, int mode, const float* dgates, const float* gates,
                  const int32_t* idx, const void* x, float* dlogits, float* dW_r, int accumulate,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (mode == MOE_ROUTE_FORCE_BALANCE)
    return set_error(MOE_ERR_UNSUPPORTED,
                     "moe_route_bwd: forced-balance gates are inputs; their gradient is dgates");
  if (mode != MOE_ROUTE_TOPK && mode != MOE_ROUTE_TOPK_FROM_LOGITS)
    return set_error(MOE_ERR_ARG, "moe_route_bwd: unknown mode %d", mode);
  REQUIRE(dgates);
  REQUIRE(gates);
  REQUIRE(idx);
  REQUIRE(dlogits);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_route_bwd: unknown accumulate bits 0x%x", accumulate);
  const bool with_dw = x && dW_r;
  if (with_dw) {
    REQUIRE(ws);
    if (int rc = need_ws(__func__, ws_bytes, ws_router_partial_bytes(s))) return rc;
  }
  return launch_route_bwd(s, dgates, gates, idx, with_dw ? x : nullptr, dlogits,
                          with_dw ? dW_r : nullptr, (accumulate & MOE_ACCUM_DW) != 0, ws, stream);
}

int moe_dispatch_bwd(const moe_shape* s, const void* dxp, const int32_t* row_of_pair,
                     const int32_t* idx, const float* dlogits, const void* W_r, void* dx,
                     int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  REQUIRE(dxp);
  REQUIRE(row_of_pair);
  REQUIRE(dx);
  if (accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "moe_dispatch_bwd: unknown accumulate bits 0x%x", accumulate);
  if (dlogits) {
    REQUIRE(idx);
    REQUIRE(W_r);
    REQUIRE(ws);
    if (int rc = need_ws(__func__, ws_bytes, ws_wrt_bytes(s))) return rc;
  }
  return do_dispatch_bwd(s, dxp, row_of_pair, idx, dlogits, W_r, dx,
                         (accumulate & MOE_ACCUM_DX) != 0, ws, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// dispatch without a caller workspace: the plan's scratch is a fixed device
// array of this library (one copy per GPU, held until the process ends)
// ---------------------------------------------------------------------------
namespace moe {

constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The array's device address on the current device, looked up once per
// device with that device current.  In host code `scratch` names a host-side
// stand-in, not device memory, so only this address may reach a kernel.
static int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess)
    return set_error(MOE_ERR_HIP, "moe_dispatch_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= 64)
    return set_error(MOE_ERR_UNSUPPORTED, "moe_dispatch_noalloc: device %d >= 64", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(MOE_ERR_HIP, "moe_dispatch_noalloc: hipGetSymbolAddress(scratch): %s",
                       hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOE_OK;
}

}  // namespace moe

extern "C" size_t moe_dispatch_noalloc_max_scratch(void) { return moe::kNoAllocScratchBytes; }

extern "C" int moe_dispatch_noalloc(const moe_shape* s, const void* x, const int32_t* idx,
                                    int32_t* counts, int32_t* offsets, int32_t* row_of_pair,
                                    int32_t* pair_of_row, int32_t* tile_offsets, void* xp,
                                    hipStream_t stream) {
  using namespace moe;
  g_err[0] = 0;
  if (int rc = validate_shape(s)) return rc;
  if (xp) REQUIRE(x);
  REQUIRE(idx);
  REQUIRE(counts);
  REQUIRE(offsets);
  REQUIRE(row_of_pair);
  REQUIRE(pair_of_row);
  REQUIRE(tile_offsets);
  const size_t need = ws_plan_bytes(s);
  if (need > kNoAllocScratchBytes)
    return set_error(MOE_ERR_WORKSPACE,
                     "moe_dispatch_noalloc: the plan needs %zu bytes of scratch (2 * E_l * "
                     "ceil(T*K / %d) * 4), more than the library's fixed %zu; use moe_dispatch "
                     "with a workspace", need, kPlanChunk, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  return do_dispatch(s, x, idx, counts, offsets, row_of_pair, pair_of_row, tile_offsets, xp, ws,
                     stream);
}

// ---------------------------------------------------------------------------
// two-micro-batch step
// ---------------------------------------------------------------------------
namespace moe {

struct StepEvents {
  hipEvent_t start, shared_a, shared_b, end;
};

// One event set per (host thread, device); events are only recorded and waited
// on inside one call, so reuse by the next call of the same thread is safe.
static int step_events(StepEvents** out) {
  static thread_local std::vector<StepEvents*> sets;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_error(MOE_ERR_HIP, "hipGetDevice failed");
  if ((int)sets.size() <= dev) sets.resize(dev + 1, nullptr);
  if (!sets[dev]) {
    StepEvents* e = new StepEvents();
    hipEvent_t* all[] = {&e->start, &e->shared_a, &e->shared_b, &e->end};
    for (hipEvent_t* p : all)
      if (hipEventCreateWithFlags(p, hipEventDisableTiming) != hipSuccess)
        return set_error(MOE_ERR_HIP, "hipEventCreateWithFlags failed");
    sets[dev] = e;
  }
  *out = sets[dev];
  return MOE_OK;
}

static int validate_mb_fwd(const moe_mb* m, int mode, bool fused) {
  REQUIRE(m->x);
  REQUIRE(m->idx);
  REQUIRE(m->counts);
  REQUIRE(m->offsets);
  REQUIRE(m->row_of_pair);
  REQUIRE(m->pair_of_row);
  REQUIRE(m->tile_offsets);
  if (!fused) REQUIRE(m->xp);
  REQUIRE(m->h);
  REQUIRE(m->a);
  REQUIRE(m->yp);
  REQUIRE(m->out);
  REQUIRE(m->gates);
  if (mode != MOE_ROUTE_FORCE_BALANCE) REQUIRE(m->logits);
  return MOE_OK;
}

static int validate_mb_bwd(const moe_mb* m, int mode, bool fused, bool fcb) {
  REQUIRE(m->idx);
  REQUIRE(m->gates);
  REQUIRE(m->offsets);
  REQUIRE(m->tile_offsets);
  REQUIRE(m->row_of_pair);
  if (fused) {
    REQUIRE(m->x);
    REQUIRE(m->pair_of_row);
  } else {
    REQUIRE(m->xp);
  }
  REQUIRE(m->h);
  REQUIRE(m->a);
  REQUIRE(m->yp);
  REQUIRE(m->dout);
  if (fcb) {
    REQUIRE(m->ag);
    REQUIRE(m->pair_of_row);
  } else {
    REQUIRE(m->dyp);
  }
  REQUIRE(m->dgates);
  REQUIRE(m->dh);
  REQUIRE(m->dxp);
  REQUIRE(m->dx);
  if (mode != MOE_ROUTE_FORCE_BALANCE) REQUIRE(m->dlogits);
  return MOE_OK;
}

#define TRY(call)                 \
  do {                            \
    if (int rc_ = (call)) return rc_; \
  } while (0)
#define HIPTRY(call)                                                               \
  do {                                                                             \
    if ((call) != hipSuccess) return set_error(MOE_ERR_HIP, "%s failed", #call);   \
  } while (0)

struct StepCtx {
  const moe_step* st;
  const moe_shape* s;
  void* wsA;
  void* wsB;
  bool router;  // TOPK mode: router weights are differentiated
  bool fused;   // fused permute: no xp, GEMM1 / wgrad gather from x
  bool fcb;     // fused combine backward: no dy_p, dgrad / wgrad gather from dout
  void* wsSA;   // shared-expert workspace of the forward micro-batch
  void* wsSB;   // and of the backward one
  void* wsW;    // non-null: a workspace whose dgrad weight copies are already
                // made (once per moe_overlap_steps call); the dgrad reads them
                // there instead of making its own
  bool scatter;  // fused scatter: GEMM2 writes y by pair, the combine and its
                 // backward read it so
};

static int fwd_route(const StepCtx& c, const moe_mb* A, hipStream_t q) {
  const PhaseRange pr("moe.route");
  return do_route(c.s, c.st->route_mode, A->x, c.st->W_r, c.st->bias, A->logits, A->idx,
                  A->gates, c.wsA, q);
}
static int fwd_dispatch(const StepCtx& c, const moe_mb* A, hipStream_t q) {
  const PhaseRange pr("moe.dispatch");
  return do_dispatch(c.s, A->x, A->idx, A->counts, A->offsets, A->row_of_pair, A->pair_of_row,
                     A->tile_offsets, c.fused ? nullptr : A->xp, c.wsA, q);
}
static int fwd_ffn(const StepCtx& c, const moe_mb* A, hipStream_t q) {
  const PhaseRange pr("moe.expert_ffn_fwd");
  return launch_ffn_fwd(c.s, c.fused ? A->x : A->xp, c.fused ? A->pair_of_row : nullptr,
                        A->offsets, A->tile_offsets, c.st->W_gu, c.st->W_down, A->h, A->a,
                        A->yp, q, c.scatter ? A->pair_of_row : nullptr);
}
static bool has_shared(const StepCtx& c) { return c.st->F_s > 0; }
static int fwd_combine(const StepCtx& c, const moe_mb* A, hipStream_t q) {
  const PhaseRange pr("moe.combine");
  return launch_combine(c.s, A->yp, A->gates, A->row_of_pair, has_shared(c) ? A->y_s : nullptr,
                        A->out, q, c.scatter);
}
static int fwd_shared(const StepCtx& c, const moe_mb* A, hipStream_t q) {
  const PhaseRange pr("moe.shared_fwd");
  return do_shared_fwd(c.s, c.st->F_s, A->x, c.st->W_gu_s, c.st->W_down_s, A->h_s, A->a_s,
                       A->y_s, c.wsSA, q);
}
static int bwd_shared_dgrad(const StepCtx& c, const moe_mb* B, hipStream_t q) {
  const PhaseRange pr("moe.shared_dgrad");
  return do_shared_dgrad(c.s, c.st->F_s, B->dout, B->h_s, c.st->W_gu_s, c.st->W_down_s, B->dh_s,
                         B->dx_s, c.wsSB, q);
}
static int bwd_shared_wgrad(const StepCtx& c, const moe_mb* B, hipStream_t q) {
  const PhaseRange pr("moe.shared_wgrad");
  return do_shared_wgrad(c.s, c.st->F_s, B->x, B->a_s, B->dh_s, B->dout, c.st->dW_gu_s,
                         c.st->dW_down_s, (c.st->accumulate & MOE_ACCUM_DW) != 0, c.wsSB, q);
}
static int bwd_combine(const StepCtx& c, const moe_mb* B, hipStream_t q) {
  const PhaseRange pr("moe.combine_bwd");
  return launch_combine_bwd(c.s, B->dout, B->yp, B->gates, B->row_of_pair,
                            c.fcb ? nullptr : B->dyp, B->dgates, q, c.scatter);
}
static int bwd_route(const StepCtx& c, const moe_mb* B, hipStream_t q) {
  const PhaseRange pr("moe.route_bwd");
  if (c.st->route_mode == MOE_ROUTE_FORCE_BALANCE) return MOE_OK;
  const bool with_dw = c.router && c.st->dW_r;
  return launch_route_bwd(c.s, B->dgates, B->gates, B->idx, with_dw ? B->x : nullptr, B->dlogits,
                          with_dw ? c.st->dW_r : nullptr,
                          (c.st->accumulate & MOE_ACCUM_DW) != 0, c.wsB, q);
}
static int bwd_dgrad(const StepCtx& c, const moe_mb* B, bool weights_ready, hipStream_t q,
                     int parts = kDgradBoth) {
  const PhaseRange pr(parts == kDgradAct  ? "moe.expert_dgrad_act"
                      : parts == kDgradIn ? "moe.expert_dgrad_in"
                                          : "moe.expert_dgrad");
  const FusedCombineBwd fc{B->pair_of_row, B->gates, B->ag};
  return launch_ffn_dgrad(c.s, c.fcb ? B->dout : B->dyp, B->h, B->offsets, B->tile_offsets,
                          c.st->W_gu, c.st->W_down, B->dh, B->dxp, c.wsW ? c.wsW : c.wsB,
                          c.wsW ? true : weights_ready, q, parts, c.fcb ? &fc : nullptr);
}
static int bwd_dispatch(const StepCtx& c, const moe_mb* B, hipStream_t q) {
  const PhaseRange pr("moe.dispatch_bwd");
  return do_dispatch_bwd(c.s, B->dxp, B->row_of_pair, B->idx, c.router ? B->dlogits : nullptr,
                         c.st->W_r, B->dx, false, c.wsB, q,
                         has_shared(c) ? B->dx_s : nullptr);
}
static int bwd_wgrad(const StepCtx& c, const moe_mb* B, hipStream_t q) {
  const PhaseRange pr("moe.expert_wgrad");
  return launch_ffn_wgrad(c.s, c.fused ? B->x : B->xp, c.fused ? B->pair_of_row : nullptr,
                          c.fcb ? B->ag : B->a, B->dh, c.fcb ? B->dout : B->dyp, B->offsets,
                          c.st->dW_gu, c.st->dW_down, (c.st->accumulate & MOE_ACCUM_DW) != 0, q,
                          c.fcb ? B->pair_of_row : nullptr);
}

// The routed experts' weight gradients of the micro-batches deferred by the
// steps before (prev[0 .. np), in step order) and of B in one launch
// (materialised xp and dy_p).  The later steps of a group accumulate (the
// grouping plan requires it), so the sum starts from the previous values
// exactly when the group's first step asked for that: first_acc.
static int bwd_wgrad_group(const StepCtx& c, const moe_mb* const* prev, int np, bool first_acc,
                           const moe_mb* B, hipStream_t q) {
  const PhaseRange pr("moe.expert_wgrad_group");
  WgrOps ops[kWgGroupMax];
  for (int i = 0; i < np; ++i)
    ops[i] = WgrOps{prev[i]->xp, prev[i]->a, prev[i]->dh, prev[i]->dyp, prev[i]->offsets};
  ops[np] = WgrOps{B->xp, B->a, B->dh, B->dyp, B->offsets};
  return launch_ffn_wgrad_multi(c.s, ops, np + 1, c.st->dW_gu, c.st->dW_down, first_acc, q);
}

// Host-side checks of one step description (flags, route mode, buffers,
// workspace); fn names the entry point in the error message.
static int check_step(const moe_step* st, int flags, const char* fn) {
  REQUIRE(st);
  const moe_shape* s = &st->shape;
  if (int rc = validate_shape(s)) return rc;
  if (flags & ~(MOE_STEP_SERIALIZE | MOE_STEP_EAGER_WGRAD | MOE_STEP_SKIP_WGRAD |
                MOE_STEP_FUSED_PERMUTE | MOE_STEP_MID_WGRAD | MOE_STEP_FUSED_COMBINE_BWD |
                MOE_STEP_PAIR_WGRAD | MOE_STEP_FUSED_SCATTER | MOE_STEP_GROUP4_WGRAD))
    return set_error(MOE_ERR_ARG, "%s: unknown flags 0x%x", fn, flags);
  if ((flags & MOE_STEP_PAIR_WGRAD) && (flags & MOE_STEP_GROUP4_WGRAD))
    return set_error(MOE_ERR_ARG, "%s: PAIR_WGRAD and GROUP4_WGRAD exclude each other", fn);
  if ((flags & (MOE_STEP_PAIR_WGRAD | MOE_STEP_GROUP4_WGRAD)) &&
      (flags & (MOE_STEP_FUSED_PERMUTE | MOE_STEP_FUSED_COMBINE_BWD)))
    return set_error(MOE_ERR_UNSUPPORTED,
                     "%s: grouped weight gradients read materialised xp and dy_p: not with "
                     "FUSED_PERMUTE or FUSED_COMBINE_BWD", fn);
  if ((flags & MOE_STEP_EAGER_WGRAD ? 1 : 0) + (flags & MOE_STEP_SKIP_WGRAD ? 1 : 0) +
          (flags & MOE_STEP_MID_WGRAD ? 1 : 0) > 1)
    return set_error(MOE_ERR_ARG, "%s: EAGER_WGRAD, SKIP_WGRAD and MID_WGRAD exclude each other",
                     fn);
  const int mode = st->route_mode;
  if (mode != MOE_ROUTE_TOPK && mode != MOE_ROUTE_TOPK_FROM_LOGITS &&
      mode != MOE_ROUTE_FORCE_BALANCE)
    return set_error(MOE_ERR_ARG, "%s: unknown route mode %d", fn, mode);
  if (st->accumulate & ~(MOE_ACCUM_DX | MOE_ACCUM_DW))
    return set_error(MOE_ERR_ARG, "%s: unknown accumulate bits 0x%x", fn,
                     st->accumulate);
  REQUIRE(st->W_gu);
  REQUIRE(st->W_down);
  if (mode == MOE_ROUTE_TOPK) REQUIRE(st->W_r);
  const moe_mb* A = st->fwd;
  const moe_mb* B = st->bwd;
  const bool fused = (flags & MOE_STEP_FUSED_PERMUTE) != 0;
  const bool fcb = (flags & MOE_STEP_FUSED_COMBINE_BWD) != 0;
  if (fused || fcb) TRY(check_gather_x(s, fn));
  if (A) TRY(validate_mb_fwd(A, mode, fused));
  if (B) {
    TRY(validate_mb_bwd(B, mode, fused, fcb));
    REQUIRE(st->dW_gu);
    REQUIRE(st->dW_down);
    if (mode == MOE_ROUTE_TOPK && st->dW_r) REQUIRE(B->x);
  }
  if (A && B && A == B)
    return set_error(MOE_ERR_ARG, "%s: fwd and bwd micro-batches must differ", fn);
  const bool shared = st->F_s != 0;
  if (shared) {
    TRY(validate_shared(st->F_s));
    REQUIRE(st->W_gu_s);
    REQUIRE(st->W_down_s);
    if (A) {
      REQUIRE(A->h_s);
      REQUIRE(A->a_s);
      REQUIRE(A->y_s);
    }
    if (B) {
      REQUIRE(B->x);
      REQUIRE(B->h_s);
      REQUIRE(B->a_s);
      REQUIRE(B->dh_s);
      REQUIRE(B->dx_s);
      REQUIRE(st->dW_gu_s);
      REQUIRE(st->dW_down_s);
    }
  }
  REQUIRE(st->ws);
  const size_t one = ws_one(s);
  const size_t sh = shared ? ws_shared(s, st->F_s) : 0;
  if (int rc = need_ws(fn, st->ws_bytes, 2 * one + 2 * sh)) return rc;
  return MOE_OK;
}

}  // namespace moe

namespace moe {
// One step (arguments checked by the caller).  wsW: see StepCtx.
static int step_impl(const moe_step* st, hipStream_t s0, hipStream_t s1, int flags, void* wsW) {
  const moe_shape* s = &st->shape;
  const int mode = st->route_mode;
  const moe_mb* A = st->fwd;
  const moe_mb* B = st->bwd;
  const bool fused = (flags & MOE_STEP_FUSED_PERMUTE) != 0;
  const bool shared = st->F_s != 0;
  const size_t one = ws_one(s);
  const size_t sh = shared ? ws_shared(s, st->F_s) : 0;
  StepCtx c{st, s, st->ws, (char*)st->ws + one, mode == MOE_ROUTE_TOPK, fused,
            (flags & MOE_STEP_FUSED_COMBINE_BWD) != 0, (char*)st->ws + 2 * one,
            (char*)st->ws + 2 * one + sh, wsW, (flags & MOE_STEP_FUSED_SCATTER) != 0};
  const bool serial = (flags & MOE_STEP_SERIALIZE) || s0 == s1;
  const bool eager = (flags & MOE_STEP_EAGER_WGRAD) != 0;
  const bool skip_w = (flags & MOE_STEP_SKIP_WGRAD) != 0;
  const bool mid = (flags & MOE_STEP_MID_WGRAD) != 0;

  // B's weight gradients: the routed experts', then the shared expert's
  auto wgrads = [&](hipStream_t q) -> int {
    TRY(bwd_wgrad(c, B, q));
    if (shared) TRY(bwd_shared_wgrad(c, B, q));
    return MOE_OK;
  };
  if (serial) {  // the forward-then-backward order of a non-overlapped layer
    if (A) {
      if (shared) TRY(fwd_shared(c, A, s0));
      TRY(fwd_route(c, A, s0));
      TRY(fwd_dispatch(c, A, s0));
      TRY(fwd_ffn(c, A, s0));
      TRY(fwd_combine(c, A, s0));
    }
    if (B && mid) {
      TRY(bwd_combine(c, B, s0));
      TRY(bwd_route(c, B, s0));
      TRY(bwd_dgrad(c, B, false, s0, kDgradAct));
      TRY(bwd_wgrad(c, B, s0));
      TRY(bwd_dgrad(c, B, true, s0, kDgradIn));
      if (shared) TRY(bwd_shared_dgrad(c, B, s0));
      TRY(bwd_dispatch(c, B, s0));
      if (shared) TRY(bwd_shared_wgrad(c, B, s0));
    } else if (B) {
      TRY(bwd_combine(c, B, s0));
      TRY(bwd_route(c, B, s0));
      TRY(bwd_dgrad(c, B, false, s0));
      if (shared) TRY(bwd_shared_dgrad(c, B, s0));
      if (eager) TRY(wgrads(s0));
      TRY(bwd_dispatch(c, B, s0));
      if (!eager && !skip_w) TRY(wgrads(s0));
    }
    return MOE_OK;
  }

  StepEvents* ev = nullptr;
  TRY(step_events(&ev));
  // s1 starts after everything already queued on s0
  HIPTRY(hipEventRecord(ev->start, s0));
  HIPTRY(hipStreamWaitEvent(s1, ev->start, 0));
  // The micro-batches share no buffers (each has its own half of the
  // workspace), so each runs in order on its own stream and the hardware
  // interleaves the two streams' kernels.
  // A shared expert runs on the stream of the other micro-batch: A's shared
  // forward at the head of s0, B's shared D at the head of s1, each joined
  // where its output is summed in (A's combine, B's dispatch backward).
  if (shared && A) {
    TRY(fwd_shared(c, A, s0));
    HIPTRY(hipEventRecord(ev->shared_a, s0));
  }
  if (shared && B) {
    TRY(bwd_shared_dgrad(c, B, s1));
    HIPTRY(hipEventRecord(ev->shared_b, s1));
  }
  if (A) {  // the forward micro-batch, start to end on s1
    TRY(fwd_route(c, A, s1));
    TRY(fwd_dispatch(c, A, s1));
    TRY(fwd_ffn(c, A, s1));
    if (shared) HIPTRY(hipStreamWaitEvent(s1, ev->shared_a, 0));
    TRY(fwd_combine(c, A, s1));
  }
  if (B && mid) {  // the backward micro-batch on s0, routed W between the two D GEMMs
    TRY(bwd_combine(c, B, s0));
    TRY(bwd_route(c, B, s0));
    TRY(bwd_dgrad(c, B, false, s0, kDgradAct));
    TRY(bwd_wgrad(c, B, s0));
    TRY(bwd_dgrad(c, B, true, s0, kDgradIn));
    if (shared) HIPTRY(hipStreamWaitEvent(s0, ev->shared_b, 0));
    TRY(bwd_dispatch(c, B, s0));
    if (shared) TRY(bwd_shared_wgrad(c, B, s0));
  } else if (B) {  // the backward micro-batch on s0
    TRY(bwd_combine(c, B, s0));
    TRY(bwd_route(c, B, s0));
    TRY(bwd_dgrad(c, B, false, s0));
    if (shared) HIPTRY(hipStreamWaitEvent(s0, ev->shared_b, 0));
    if (eager) TRY(wgrads(s0));
    TRY(bwd_dispatch(c, B, s0));
    if (!eager && !skip_w) TRY(wgrads(s0));
  }
  // s0 ends after everything the step issued on s1
  HIPTRY(hipEventRecord(ev->end, s1));
  HIPTRY(hipStreamWaitEvent(s0, ev->end, 0));
  return MOE_OK;
}
}  // namespace moe

extern "C" int moe_overlap_step(const moe_step* st, hipStream_t s0, hipStream_t s1, int flags) {
  using namespace moe;
  g_err[0] = 0;
  if (int rc = check_step(st, flags, "moe_overlap_step")) return rc;
  if (flags & (MOE_STEP_PAIR_WGRAD | MOE_STEP_GROUP4_WGRAD))
    return set_error(MOE_ERR_ARG, "moe_overlap_step: grouped weight gradients span consecutive "
                                  "steps: use moe_overlap_steps");
  return step_impl(st, s0, s1, flags, nullptr);
}

// ---------------------------------------------------------------------------
// several consecutive steps with the streams' roles alternating
// ---------------------------------------------------------------------------
namespace moe {

struct MultiEvents {
  hipEvent_t start, end, dwr, dw, dws;
  hipEvent_t bend[2];  // end of the backward chain of the steps of each parity
  // grouped weight gradients: the deferred micro-batches' dh are written
  hipEvent_t grp[kWgGroupMax - 1];
};

// One set per (host thread, device), as step_events; every wait of a call is
// on a record issued earlier in the same call.
static int multi_events(MultiEvents** out) {
  static thread_local std::vector<MultiEvents*> sets;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_error(MOE_ERR_HIP, "hipGetDevice failed");
  if ((int)sets.size() <= dev) sets.resize(dev + 1, nullptr);
  if (!sets[dev]) {
    MultiEvents* e = new MultiEvents();
    hipEvent_t* all[] = {&e->start,  &e->end,    &e->dwr,    &e->dw,    &e->dws,
                         &e->bend[0], &e->bend[1], &e->grp[0], &e->grp[1], &e->grp[2]};
    static_assert(kWgGroupMax - 1 == 3, "one event per deferred micro-batch of a group");
    for (hipEvent_t* p : all)
      if (hipEventCreateWithFlags(p, hipEventDisableTiming) != hipSuccess)
        return set_error(MOE_ERR_HIP, "hipEventCreateWithFlags failed");
    sets[dev] = e;
  }
  *out = sets[dev];
  return MOE_OK;
}

static bool same_mb(const moe_mb* a, const moe_mb* b) {
  if (!a || !b) return a == b;
  return a == b || memcmp(a, b, sizeof(moe_mb)) == 0;
}

// Grouped weight gradients: whether the forward of micro-batch A writes into
// any buffer the grouped weight gradient reads from micro-batch B (xp, a, dh,
// dy_p, offsets).
static bool fwd_overwrites_wgrad_inputs(const moe_mb* A, const moe_mb* B) {
  if (!A || !B) return false;
  const void* reads[] = {B->xp, B->a, B->dh, B->dyp, B->offsets};
  const void* writes[] = {A->logits, A->idx,         A->gates,       A->counts, A->offsets,
                          A->row_of_pair, A->pair_of_row, A->tile_offsets, A->xp, A->h,
                          A->a,      A->yp,          A->out,         A->h_s,    A->a_s,
                          A->y_s};
  for (const void* r : reads)
    for (const void* w : writes)
      if (r && r == w) return true;
  return false;
}

// The forward chain of one micro-batch on one stream (its shared expert first).
static int fwd_chain(const StepCtx& c, const moe_mb* A, hipStream_t q) {
  if (has_shared(c)) TRY(fwd_shared(c, A, q));
  TRY(fwd_route(c, A, q));
  TRY(fwd_dispatch(c, A, q));
  TRY(fwd_ffn(c, A, q));
  return fwd_combine(c, A, q);
}

// Which weight-gradient accumulation events this call has recorded.
struct AccumOrder {
  const MultiEvents* ev;
  bool dwr, dw, dws;
};

// The backward chain of one micro-batch on one stream.  Each weight-gradient
// accumulation (router dW_r, routed dW, shared dW) waits for the latest
// earlier accumulation into the same buffer in this call (on either stream),
// and records its own, so the sums happen in step order.  Only events
// recorded in this call are waited on.
// skip: leave the weight gradients (routed and shared) to the caller.
// With grouped weight gradients, rw says what the routed experts' weight
// gradient does: kRwOwn (B's alone), kRwDefer (none: record ev->grp[g.slot]
// once dh is written; the group's last step takes it) or kRwGroup (B's
// together with the g.np micro-batches deferred by the steps before, after
// waiting for their events; g.first_acc is the group's first step's
// accumulate flag).
enum { kRwOwn, kRwDefer, kRwGroup };
struct GroupRole {
  int slot = 0;                                // kRwDefer: its event
  int np = 0;                                  // kRwGroup: deferred micro-batches
  const moe_mb* prev[kWgGroupMax - 1] = {};    // in step order
  bool first_acc = false;
};
static int bwd_chain(const StepCtx& c, const moe_mb* B, hipStream_t q, bool mid, bool eager,
                     bool skip, AccumOrder& ord, int rw = kRwOwn,
                     const GroupRole& g = GroupRole{}) {
  const bool shared = has_shared(c);
  const bool dwr = c.router && c.st->dW_r;
  const MultiEvents* ev = ord.ev;
  auto wait = [&](hipEvent_t e, bool recorded) -> int {
    if (recorded) HIPTRY(hipStreamWaitEvent(q, e, 0));
    return MOE_OK;
  };
  auto routed_w = [&]() -> int {
    if (rw == kRwDefer) return MOE_OK;
    TRY(wait(ev->dw, ord.dw));
    if (rw == kRwGroup) {
      for (int i = 0; i < g.np; ++i) HIPTRY(hipStreamWaitEvent(q, ev->grp[i], 0));
      TRY(bwd_wgrad_group(c, g.prev, g.np, g.first_acc, B, q));
    } else {
      TRY(bwd_wgrad(c, B, q));
    }
    HIPTRY(hipEventRecord(ev->dw, q));
    ord.dw = true;
    return MOE_OK;
  };
  // B's dh is written: the grouped weight gradient of a later step may read it
  auto dh_done = [&]() -> int {
    if (rw == kRwDefer) HIPTRY(hipEventRecord(ev->grp[g.slot], q));
    return MOE_OK;
  };
  auto shared_w = [&]() -> int {
    if (!shared) return MOE_OK;
    TRY(wait(ev->dws, ord.dws));
    TRY(bwd_shared_wgrad(c, B, q));
    HIPTRY(hipEventRecord(ev->dws, q));
    ord.dws = true;
    return MOE_OK;
  };
  TRY(bwd_combine(c, B, q));
  if (dwr) TRY(wait(ev->dwr, ord.dwr));
  TRY(bwd_route(c, B, q));
  if (dwr) {
    HIPTRY(hipEventRecord(ev->dwr, q));
    ord.dwr = true;
  }
  if (mid) {
    TRY(bwd_dgrad(c, B, false, q, kDgradAct));
    TRY(dh_done());
    TRY(routed_w());
    TRY(bwd_dgrad(c, B, true, q, kDgradIn));
    if (shared) TRY(bwd_shared_dgrad(c, B, q));
    TRY(bwd_dispatch(c, B, q));
    return shared_w();
  }
  TRY(bwd_dgrad(c, B, false, q));
  TRY(dh_done());
  if (shared) TRY(bwd_shared_dgrad(c, B, q));
  if (eager) {
    TRY(routed_w());
    TRY(shared_w());
    return bwd_dispatch(c, B, q);
  }
  TRY(bwd_dispatch(c, B, q));
  if (skip) return MOE_OK;
  TRY(routed_w());
  return shared_w();
}

}  // namespace moe

extern "C" int moe_overlap_steps(const moe_step* steps, int n, hipStream_t s0, hipStream_t s1,
                                 int flags) {
  using namespace moe;
  g_err[0] = 0;
  REQUIRE(steps);
  if (n < 1) return set_error(MOE_ERR_ARG, "moe_overlap_steps: n = %d, need at least 1", n);
  for (int j = 0; j < n; ++j) {
    const moe_step* st = &steps[j];
    if (int rc = check_step(st, flags, "moe_overlap_steps")) return rc;
    if (st->fwd && st->bwd && same_mb(st->fwd, st->bwd))
      return set_error(MOE_ERR_ARG,
                       "moe_overlap_steps: step %d forwards and back-propagates the same "
                       "micro-batch", j);
    // each stream owns a fixed half of the one workspace, laid out by the shape
    if (j > 0 && (memcmp(&st->shape, &steps[0].shape, sizeof(moe_shape)) != 0 ||
                  st->ws != steps[0].ws || st->ws_bytes != steps[0].ws_bytes ||
                  st->F_s != steps[0].F_s))
      return set_error(MOE_ERR_ARG,
                       "moe_overlap_steps: step %d differs from step 0 in shape, workspace or "
                       "shared-expert width", j);
    if (j > 0 && !same_mb(st->bwd, steps[j - 1].fwd))
      return set_error(MOE_ERR_ARG,
                       "moe_overlap_steps: step %d must back-propagate the micro-batch that "
                       "step %d forwarded", j, j - 1);
    if (j > 0 && (st->W_gu != steps[0].W_gu || st->W_down != steps[0].W_down))
      return set_error(MOE_ERR_ARG,
                       "moe_overlap_steps: step %d has other expert weights than step 0", j);
  }
  if (flags & (MOE_STEP_PAIR_WGRAD | MOE_STEP_GROUP4_WGRAD)) {
    // A graph-captured run of paired steps ended in a host crash whose cause
    // is not known: grouped steps are issued eagerly only.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s0, &cs) != hipSuccess)
      return set_error(MOE_ERR_HIP, "moe_overlap_steps: hipStreamIsCapturing failed");
    if (cs != hipStreamCaptureStatusNone)
      return set_error(MOE_ERR_UNSUPPORTED,
                       "moe_overlap_steps: grouped weight gradients are not supported under "
                       "stream capture");
  }
  // The expert weights are the same for every step of the call, so the
  // dgrad's transposed copies of them are made once, at the start, into the
  // first half of the workspace, and every step's dgrad on either stream reads
  // them there (no other call writes that region during the call).
  bool any_bwd = false;
  for (int j = 0; j < n; ++j) any_bwd |= steps[j].bwd != nullptr;
  void* wsW = nullptr;
  if (any_bwd) {
    wsW = steps[0].ws;
    const PhaseRange pr("moe.dgrad_weights");
    TRY(launch_dgrad_weights(&steps[0].shape, steps[0].W_gu, steps[0].W_down, wsW, s0));
  }
  const bool serial = (flags & MOE_STEP_SERIALIZE) || s0 == s1;
  // SKIP_WGRAD leaves the weight gradients of the last step's backward
  // micro-batch to the caller; the earlier steps' run as usual
  const bool skip_last = (flags & MOE_STEP_SKIP_WGRAD) != 0;
  // Grouped weight gradients (PAIR_WGRAD: groups of 2 steps, GROUP4_WGRAD:
  // of 4): steps j .. j + G - 1 (all with a backward micro-batch, the later
  // ones accumulating, the last step of the call left out with SKIP_WGRAD)
  // form a group whose routed weight gradients run as one launch in step
  // j + G - 1; groups are formed from the first step on, and a step in no
  // group keeps its own
  const int G = (flags & MOE_STEP_GROUP4_WGRAD) ? 4 : (flags & MOE_STEP_PAIR_WGRAD) ? 2 : 1;
  const bool grouped = G > 1;
  std::vector<int> rw(n, kRwOwn);
  std::vector<GroupRole> role(n);
  if (grouped) {
    const int last = skip_last ? n - 1 : n;  // steps that may be grouped
    for (int j = 0; j + G - 1 < last;) {
      bool ok = true;
      for (int k = 0; k < G; ++k) ok = ok && steps[j + k].bwd != nullptr;
      // the later steps must add to what the earlier ones leave (an
      // overwriting step discards the weight gradients before it), into the
      // same weight-gradient buffers
      for (int k = 1; k < G; ++k)
        ok = ok && (steps[j + k].accumulate & MOE_ACCUM_DW) != 0 &&
             steps[j + k].dW_gu == steps[j].dW_gu && steps[j + k].dW_down == steps[j].dW_down;
      if (!ok) {
        ++j;
        continue;
      }
      // a deferred micro-batch's wgrad inputs must stay intact until the
      // group's last step
      for (int dd = j; dd < j + G - 1; ++dd)
        for (int f = dd + 1; f < j + G; ++f)
          if (fwd_overwrites_wgrad_inputs(steps[f].fwd, steps[dd].bwd))
            return set_error(MOE_ERR_ARG,
                             "moe_overlap_steps: grouped weight gradients: step %d forwards "
                             "into a buffer that the weight gradient of step %d's backward "
                             "micro-batch reads in step %d", f, dd, j + G - 1);
      GroupRole& gl = role[j + G - 1];
      rw[j + G - 1] = kRwGroup;
      gl.np = G - 1;
      gl.first_acc = (steps[j].accumulate & MOE_ACCUM_DW) != 0;
      for (int k = 0; k < G - 1; ++k) {
        rw[j + k] = kRwDefer;
        role[j + k].slot = k;
        gl.prev[k] = steps[j + k].bwd;
      }
      j += G;
    }
  }
  if (serial && !grouped) {
    for (int j = 0; j < n; ++j)
      TRY(step_impl(&steps[j], s0, s0, j == n - 1 ? flags : flags & ~MOE_STEP_SKIP_WGRAD, wsW));
    return MOE_OK;
  }
  // (serialized with grouped weight gradients: the same chains, all on s0, forward then
  // backward, which is the serialized order)
  MultiEvents* ev = nullptr;
  TRY(multi_events(&ev));
  const bool mid = (flags & MOE_STEP_MID_WGRAD) != 0;
  const bool eager = (flags & MOE_STEP_EAGER_WGRAD) != 0;
  const bool fused = (flags & MOE_STEP_FUSED_PERMUTE) != 0;
  HIPTRY(hipEventRecord(ev->start, s0));
  HIPTRY(hipStreamWaitEvent(s1, ev->start, 0));
  AccumOrder ord{ev, false, false, false};
  bool bend_rec[2] = {false, false};  // bend[p] recorded in this call
  for (int j = 0; j < n; ++j) {
    const moe_step* st = &steps[j];
    const moe_shape* s = &st->shape;
    const size_t one = ws_one(s);
    const size_t sh = st->F_s ? ws_shared(s, st->F_s) : 0;
    // Step j runs its forward on P and its backward on Q; the roles swap every
    // step, so the forward of step j follows, on its stream, the backward of
    // step j - 1 (whose micro-batch buffers it may reuse), and the backward of
    // step j follows the forward of the same micro-batch in step j - 1.  Each
    // stream owns one half of the workspace (s1 the first), so no half is
    // used by both streams at once.
    const bool even = (j & 1) == 0;
    hipStream_t P = serial ? s0 : (even ? s1 : s0), Q = serial ? s0 : (even ? s0 : s1);
    char* ws = (char*)st->ws;
    char* half_s1 = ws;
    char* half_s0 = ws + one;
    char* shalf_s1 = ws + 2 * one;
    char* shalf_s0 = ws + 2 * one + sh;
    StepCtx c{st, s, even ? half_s1 : half_s0, even ? half_s0 : half_s1,
              st->route_mode == MOE_ROUTE_TOPK, fused, (flags & MOE_STEP_FUSED_COMBINE_BWD) != 0,
              even ? shalf_s1 : shalf_s0, even ? shalf_s0 : shalf_s1, wsW,
              (flags & MOE_STEP_FUSED_SCATTER) != 0};
    // The forward of step j also waits for the backward of step j - 2 (on
    // the other stream), the last earlier chain not ordered before it by its
    // stream, so a forward may reuse the buffers of any micro-batch
    // back-propagated in an earlier step.  That backward has normally ended
    // long before.
    if (st->fwd) {
      if (bend_rec[j & 1]) HIPTRY(hipStreamWaitEvent(P, ev->bend[j & 1], 0));
      TRY(fwd_chain(c, st->fwd, P));
    }
    if (st->bwd) {
      TRY(bwd_chain(c, st->bwd, Q, mid, eager, skip_last && j == n - 1, ord, rw[j],
                    role[j]));
      HIPTRY(hipEventRecord(ev->bend[j & 1], Q));
      bend_rec[j & 1] = true;
    }
  }
  HIPTRY(hipEventRecord(ev->end, s1));
  HIPTRY(hipStreamWaitEvent(s0, ev->end, 0));
  return MOE_OK;
}
