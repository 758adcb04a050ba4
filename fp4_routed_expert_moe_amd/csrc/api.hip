// C ABI of the MoE layer: validation, workspace carve-up, path choice, kernel enqueue.
// Nothing here synchronises the host with the device.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "api_internal.h"

// Workspace of moe_forward_noalloc: one array per device (each GPU the library runs on holds
// its own copy until the process ends).  In host code this name is only a stand-in: the
// device address comes from hipGetSymbolAddress (scratch_of below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe_api {

thread_local std::string g_last_error;
// set while moe_forward_noalloc runs: its launches record no timing events (no event objects
// are created inside it)
thread_local bool g_no_timing = false;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

constexpr int kGemvMaxTokens = 32;  // AUTO: GEMV up to this many tokens, grouped GEMM above
constexpr int kWarmMinT = 4;        // decode batches from which routing reads the shared expert ahead


// Workspace layout for T tokens; assigns pointers when base != nullptr.  Returns bytes.
size_t carve(const moe::Dims& d, int T, char* base, moe::CallBufs* b) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return p;
  };
  const size_t tk = (size_t)T * d.K;
  const size_t rows = (size_t)T * (d.K + d.S);
  const size_t C = ((size_t)T + moe::kChunk - 1) / moe::kChunk;
  const size_t gnz = std::min<size_t>(d.E, tk) + d.S;
  const size_t mt_bound = (rows + gnz * (moe::kGemmBM - 1)) / moe::kGemmBM + 1;
  moe::CallBufs t{};
  // control words first: their offset must not depend on T (zero between calls)
  t.ctrl = reinterpret_cast<int32_t*>(take((size_t)moe::ctrl_layout(d.H, d.E, d.S, d.I).words * 4));
  // partial scores: the largest slices x tokens over the batch sizes up to T (slices only change
  // at multiples of 64 tokens, and within such a range the product grows with the tokens)
  size_t score_rows = (size_t)T;
  if (!moe::route_fused(d, T))
    for (int t = 64; t <= T + 63; t += 64) {
      const int tt = t < T ? t : T;
      score_rows = std::max(score_rows, (size_t)tt * moe::router_slices(d, tt));
    }
  t.logits = reinterpret_cast<float*>(take(score_rows * d.E * 4));
  t.idx = reinterpret_cast<int32_t*>(take(tk * 4));
  t.w = reinterpret_cast<float*>(take(tk * 4));
  t.counts = reinterpret_cast<int32_t*>(take((size_t)d.E * 4));
  t.offsets = reinterpret_cast<int32_t*>(take((size_t)(d.E + 1) * 4));
  t.perm = reinterpret_cast<int32_t*>(take(tk * 4));
  t.row_w = reinterpret_cast<float*>(take(tk * 4));
  t.gmask = reinterpret_cast<uint64_t*>(take(C * d.E * 8));
  t.cbase = reinterpret_cast<int32_t*>(take(C * d.E * 4));
  t.grp_row0 = reinterpret_cast<int32_t*>(take((size_t)d.G * 4));
  t.grp_rows = reinterpret_cast<int32_t*>(take((size_t)d.G * 4));
  t.grec = reinterpret_cast<moe::GroupRec*>(take((size_t)d.G * sizeof(moe::GroupRec)));
  t.info = reinterpret_cast<int32_t*>(take(16));
  t.mt_group = reinterpret_cast<int32_t*>(take(mt_bound * 4));
  t.mt_row0 = reinterpret_cast<int32_t*>(take(mt_bound * 4));
  t.h = take(rows * d.I * 4);
  t.xq = reinterpret_cast<uint8_t*>(take((size_t)T * d.H * 2 + (size_t)T * moe::kb_pad(d.H)));
  t.staging = reinterpret_cast<float*>(take(rows * d.H * 4));
  if (b) *b = t;
  return off;
}

int mt_bound_of(const moe::Dims& d, int T) {
  const size_t tk = (size_t)T * d.K;
  const size_t rows = (size_t)T * (d.K + d.S);
  const size_t gnz = std::min<size_t>(d.E, tk) + d.S;
  return (int)((rows + gnz * (moe::kGemmBM - 1)) / moe::kGemmBM + 1);
}

// upper bound of the active groups (routed experts hit plus shared experts) of a T-token call
int max_active_of(const moe::Dims& d, int T) {
  return (int)(std::min<size_t>(d.E, (size_t)T * d.K) + d.S);
}


// ---- kernel timing -------------------------------------------------------------------
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
struct TimingAcc {
  const char* name;
  int64_t launches = 0;
  double ms = 0;
};
std::mutex g_tmu;
bool g_tenabled = false;
std::vector<TimingRec> g_trecs;
std::vector<hipEvent_t> g_tpool;
std::map<std::string, TimingAcc> g_tacc;

hipEvent_t take_event() {
  if (!g_tpool.empty()) {
    hipEvent_t e = g_tpool.back();
    g_tpool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain_timing_locked() {
  for (auto& r : g_trecs) {
    float ms = 0.f;
    if (r.b && hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      auto& acc = g_tacc[r.name];
      acc.name = r.name;
      acc.launches += 1;
      acc.ms += ms;
    }
    if (r.a) g_tpool.push_back(r.a);
    if (r.b) g_tpool.push_back(r.b);
  }
  g_trecs.clear();
}

}  // namespace moe_api

using namespace moe_api;

namespace moe {

int timing_begin(const char* name, hipStream_t s) {
  if (!g_tenabled || g_no_timing) return -1;
  std::lock_guard<std::mutex> lk(g_tmu);
  TimingRec r{name, take_event(), take_event()};
  if (!r.a || !r.b) return -1;
  (void)hipEventRecord(r.a, s);
  g_trecs.push_back(r);
  return (int)g_trecs.size() - 1;
}

void timing_end(int token, hipStream_t s) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (token < (int)g_trecs.size()) (void)hipEventRecord(g_trecs[token].b, s);
}

}  // namespace moe

// ---- moe_forward without a caller workspace -----------------------------------------
namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kScratchDevices];  // device address of `scratch` on each device, once looked up

__global__ void clear_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// The device address of this device's scratch array (the current device is `dev`).  The first
// call on a device looks it up and enqueues a kernel on `s` that zeroes the control words at
// its start (a device array starts zeroed; every completed call leaves them at zero again).
int32_t scratch_of(int dev, hipStream_t s, void** out) {
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device %d beyond the %d the library tracks", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "moe_forward_noalloc: hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    const int words = moe::ctrl_layout(0, 0, 0, 0).words;
    clear_words_kernel<<<1, 64, 0, s>>>(static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess)
      return fail(MOE_ERR_HIP, "moe_forward_noalloc: clearing the scratch control words failed: %s",
                  hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}
}  // namespace

namespace moe_api {

int32_t check_call(const moe_layer* L, const uint16_t* x, int32_t T, void* ws, uint64_t ws_bytes,
                          const char* what) {
  if (!L) return fail(MOE_ERR_INVALID, "%s: NULL layer", what);
  if (T < 0 || T > kMaxTokens) return fail(MOE_ERR_INVALID, "%s: tokens=%d out of [0, %d]", what, T, kMaxTokens);
  if (T == 0) return MOE_OK;
  if (!x) return fail(MOE_ERR_INVALID, "%s: NULL input", what);
  if (reinterpret_cast<uintptr_t>(x) & 15u) return fail(MOE_ERR_INVALID, "%s: x must be 16-byte aligned", what);
  const uint64_t need = carve(L->dims, T, nullptr, nullptr);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %p/%llu bytes, need %llu bytes aligned to 256", what, ws,
                (unsigned long long)ws_bytes, (unsigned long long)need);
  return MOE_OK;
}

// Routing; with `forward` set the routing kernels also write the FP8 activation terms the
// expert kernels read, and (for the grouped GEMM) its M-tile list.  route_out: the caller
// reads the routing (idx, weights, counts, offsets, perm), so every table is written.
int32_t enqueue_route(const moe_layer* L, const uint16_t* x, int32_t T, moe::CallBufs& b, hipStream_t s,
                             bool forward, bool gemm, bool route_out, const moe::JoinArgs* join) {
  const moe::Dims& d = L->dims;
  const bool lean = forward && !gemm && !route_out;
  // A forward call on the decode kernels reads the FP4 shared expert's weights right after
  // routing; from kWarmMinT tokens the routing launch reads them ahead (8 tokens: the step
  // 2-2.5 us shorter).  Not at one token, where the extra HBM traffic slows the routing tail by
  // more than it saves, nor for an FP8 shared expert (25 MB: the same).
  moe::Warm warm{};
  const bool use_warm = forward && !gemm && d.S && !d.fp8_shared && T >= kWarmMinT;
  if (use_warm) {
    const moe_layer_desc& w = L->desc;
    const size_t gu_codes = (size_t)d.I * d.H / 2, dn_codes = (size_t)d.H * d.I / 2;
    const size_t gu_sc = moe::scale_slab_bytes(d.I, d.H), dn_sc = moe::scale_slab_bytes(d.H, d.I);
    const uint8_t* base[6] = {w.gate_codes, w.up_codes, w.down_codes, w.gate_scales, w.up_scales, w.down_scales};
    const size_t per[6] = {gu_codes, gu_codes, dn_codes, gu_sc, gu_sc, dn_sc};
    for (int i = 0; i < 6; ++i) {  // the shared expert is group E
      warm.p[i] = base[i] + (size_t)d.E * per[i];
      warm.bytes[i] = (uint32_t)per[i];
    }
  }
  hipError_t e = moe::launch_router_logits(d, x, L->desc.w_router, L->desc.router_bias, b, T, forward,
                                           forward && gemm, lean, s, join, use_warm ? &warm : nullptr);
  if (e == hipSuccess && !moe::route_fused(d, T)) e = moe::launch_route_chunked(d, b, T, s);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "routing launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

void use_route_out(moe::CallBufs& b, const moe_route_out* r) {
  b.idx = r->idx;
  b.w = r->weight;
  b.counts = r->counts;
  b.offsets = r->offsets;
  b.perm = r->perm;
}

bool route_ok(const moe_route_out* r) {
  return r && r->idx && r->weight && r->counts && r->offsets && r->perm;
}

}  // namespace moe_api

// =====================================================================================
extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported device or configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_ALLOC: return "allocation failed";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_device_supported(int32_t device, char* name, int32_t cap) {
  auto put = [&](const char* s) {
    if (name && cap > 0) {
      strncpy(name, s, (size_t)cap - 1);
      name[cap - 1] = '\0';
    }
  };
  // test hook: MOE_FAKE_ARCH names the architecture of every device (no HIP call), so the
  // host-side paths (create, validation, workspace sizing) can be exercised without a GPU
  if (const char* fake = getenv("MOE_FAKE_ARCH")) {
    put(fake);
    return device >= 0 && strncmp(fake, "gfx950", 6) == 0 && (fake[6] == '\0' || fake[6] == ':');
  }
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    put("no HIP device");
    return 0;
  }
  if (device < 0 || device >= n) {
    put("device ordinal out of range");
    return 0;
  }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, device) != hipSuccess) {
    (void)hipGetLastError();
    put("hipGetDeviceProperties failed");
    return 0;
  }
  put(p.gcnArchName);
  return strncmp(p.gcnArchName, "gfx950", 6) == 0 && (p.gcnArchName[6] == '\0' || p.gcnArchName[6] == ':');
}

int32_t moe_layer_create(const moe_layer_desc* d, moe_layer** out) {
  if (out) *out = nullptr;
  if (!d || !out) return fail(MOE_ERR_INVALID, "moe_layer_create: NULL descriptor or output pointer");
  if (d->abi_version != MOE_ABI_VERSION)
    return fail(MOE_ERR_UNSUPPORTED, "moe_layer_create: ABI version %d, library is %d", d->abi_version,
                MOE_ABI_VERSION);
  if (d->hidden < 32 || d->hidden > 8192 || d->hidden % 32)
    return fail(MOE_ERR_INVALID, "hidden=%d must be a multiple of 32 in [32, 8192]", d->hidden);
  if (d->inter < 32 || d->inter > 8192 || d->inter % 32)
    return fail(MOE_ERR_INVALID, "inter=%d must be a multiple of 32 in [32, 8192]", d->inter);
  if (d->n_experts < 1 || d->n_experts > 1024)
    return fail(MOE_ERR_INVALID, "n_experts=%d must be in [1, 1024]", d->n_experts);
  if (d->top_k < 1 || d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID, "top_k=%d must be in [1, n_experts=%d]", d->top_k, d->n_experts);
  if (d->n_shared != 0 && d->n_shared != 1) return fail(MOE_ERR_INVALID, "n_shared=%d must be 0 or 1", d->n_shared);
  if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_GEMM) return fail(MOE_ERR_INVALID, "path=%d unknown", d->path);
  if (d->block != 32) return fail(MOE_ERR_INVALID, "block=%d: FP4 scales cover 32 values", d->block);
  if (d->reserved != 0) return fail(MOE_ERR_INVALID, "reserved=%d must be 0", d->reserved);
  if (!(d->routed_scale > 0.f) || !(d->routed_scale <= 3.402823466e38f))
    return fail(MOE_ERR_INVALID, "routed_scale=%g must be finite and > 0", (double)d->routed_scale);
  if (d->flags & ~(int32_t)MOE_SHARED_FP8) return fail(MOE_ERR_INVALID, "flags=0x%x has unknown bits", d->flags);
  const bool fp8 = (d->flags & MOE_SHARED_FP8) != 0;
  if (!d->w_router || !d->gate_codes || !d->gate_scales || !d->up_codes || !d->up_scales || !d->down_codes ||
      !d->down_scales)
    return fail(MOE_ERR_INVALID, "moe_layer_create: a weight pointer is NULL");
  if (!aligned16(d->w_router) || !aligned16(d->gate_codes) || !aligned16(d->up_codes) ||
      !aligned16(d->down_codes))
    return fail(MOE_ERR_INVALID, "router weights and code arrays must be 16-byte aligned");
  const void* f8[6] = {d->shared_gate_fp8, d->shared_gate_fp8_scales, d->shared_up_fp8,
                       d->shared_up_fp8_scales, d->shared_down_fp8, d->shared_down_fp8_scales};
  if (fp8) {
    if (d->n_shared != 1) return fail(MOE_ERR_INVALID, "MOE_SHARED_FP8 needs n_shared = 1");
    if (d->hidden % 128 || d->inter % 128)
      return fail(MOE_ERR_INVALID, "MOE_SHARED_FP8: hidden=%d and inter=%d must be multiples of 128", d->hidden,
                  d->inter);
    for (int i = 0; i < 6; ++i)
      if (!f8[i]) return fail(MOE_ERR_INVALID, "MOE_SHARED_FP8: a shared-expert FP8 pointer is NULL");
    if (!aligned16(d->shared_gate_fp8) || !aligned16(d->shared_up_fp8) || !aligned16(d->shared_down_fp8))
      return fail(MOE_ERR_INVALID, "FP8 code arrays must be 16-byte aligned");
    for (int i = 1; i < 6; i += 2)
      if (reinterpret_cast<uintptr_t>(f8[i]) & 3u) return fail(MOE_ERR_INVALID, "FP8 scales must be 4-byte aligned");
  } else {
    for (int i = 0; i < 6; ++i)
      if (f8[i]) return fail(MOE_ERR_INVALID, "shared-expert FP8 pointers given without MOE_SHARED_FP8");
  }
  char arch[64];
  if (!moe_device_supported(d->device, arch, sizeof(arch)))
    return fail(MOE_ERR_UNSUPPORTED, "device %d is not a supported gfx950 (%s)", d->device, arch);
  // test hook: MOE_FAIL_ALLOC makes the layer's host allocation fail
  moe_layer* L = getenv("MOE_FAIL_ALLOC") ? nullptr : new (std::nothrow) moe_layer;
  if (!L) return fail(MOE_ERR_ALLOC, "moe_layer_create: out of host memory");
  L->desc = *d;
  L->dims = moe::Dims{d->hidden, d->n_experts, d->top_k, d->n_shared, d->inter, d->n_experts + d->n_shared,
                      fp8, d->routed_scale};
  *out = L;
  return MOE_OK;
}

void moe_layer_destroy(moe_layer* layer) { delete layer; }

uint64_t moe_workspace_bytes(const moe_layer* layer, int32_t max_tokens) {
  if (!layer || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
  return carve(layer->dims, std::max(max_tokens, 1), nullptr, nullptr);
}

int32_t moe_route(const moe_layer* L, const uint16_t* x, int32_t T, const moe_route_out* route, void* ws,
                  uint64_t ws_bytes, void* stream) {
  int32_t st = check_call(L, x, T, ws, ws_bytes, "moe_route");
  if (st != MOE_OK || T == 0) return st;
  if (!route_ok(route)) return fail(MOE_ERR_INVALID, "moe_route: every route_out buffer is required");
  DeviceGuard dg(L->desc.device);
  if (!dg.ok) return fail(MOE_ERR_HIP, "moe_route: hipSetDevice(%d) failed", L->desc.device);
  moe::CallBufs b;
  carve(L->dims, T, static_cast<char*>(ws), &b);
  use_route_out(b, route);
  return enqueue_route(L, x, T, b, static_cast<hipStream_t>(stream), false, false, true);
}

int32_t moe_forward(const moe_layer* L, const uint16_t* x, int32_t T, float* y, const moe_route_out* route,
                    void* ws, uint64_t ws_bytes, void* stream) {
  return forward_impl(L, x, T, y, route, ws, ws_bytes, static_cast<hipStream_t>(stream), nullptr);
}

}  // extern "C"

namespace moe_api {

int32_t forward_impl(const moe_layer* L, const uint16_t* x, int32_t T, float* y, const moe_route_out* route,
                     void* ws, uint64_t ws_bytes, hipStream_t s, const moe::JoinArgs* join) {
  int32_t st = check_call(L, x, T, ws, ws_bytes, "moe_forward");
  if (st != MOE_OK || T == 0) return st;
  if (!y) return fail(MOE_ERR_INVALID, "moe_forward: NULL output");
  if (reinterpret_cast<uintptr_t>(y) & 15u) return fail(MOE_ERR_INVALID, "moe_forward: y must be 16-byte aligned");
  if (route && !route_ok(route)) return fail(MOE_ERR_INVALID, "moe_forward: route_out given with a NULL buffer");
  DeviceGuard dg(L->desc.device);
  if (!dg.ok) return fail(MOE_ERR_HIP, "moe_forward: hipSetDevice(%d) failed", L->desc.device);
  const moe::Dims& d = L->dims;
  moe::CallBufs b;
  carve(d, T, static_cast<char*>(ws), &b);
  if (route) use_route_out(b, route);
  const bool gemv = L->desc.path == MOE_PATH_GEMV || (L->desc.path == MOE_PATH_AUTO && T <= kGemvMaxTokens);
  hipError_t e;
  st = enqueue_route(L, x, T, b, s, true, !gemv, route != nullptr, join);
  if (st != MOE_OK) return st;
  if (gemv) {
    // the down kernel also adds each token's rows into y
    const int na = max_active_of(d, T);
    e = moe::launch_gemv_gateup(d, L->desc, x, b, T, na, s);
    if (e == hipSuccess) e = moe::launch_gemv_down(d, L->desc, b, y, T, na, s);
  } else {
    const int mb = mt_bound_of(d, T);
    e = moe::launch_gemm_gateup(d, L->desc, x, b, T, mb, s);
    if (e == hipSuccess) e = moe::launch_gemm_down(d, L->desc, b, T, mb, s);
    if (e == hipSuccess) e = moe::launch_combine(d, b, y, T, s);
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_forward: launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // namespace moe_api

extern "C" {

int32_t moe_forward_noalloc(const moe_layer* L, const uint16_t* x, int32_t T, float* y, const moe_route_out* route,
                            void* stream) {
  if (!L) return fail(MOE_ERR_INVALID, "moe_forward_noalloc: NULL layer");
  if (T < 0 || T > kMaxTokens)
    return fail(MOE_ERR_INVALID, "moe_forward_noalloc: tokens=%d out of [0, %d]", T, kMaxTokens);
  if (T == 0) return MOE_OK;
  const uint64_t need = carve(L->dims, T, nullptr, nullptr);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE, "moe_forward_noalloc: %d tokens need %llu bytes of scratch; the limit is %llu", T,
                (unsigned long long)need, (unsigned long long)MOE_NOALLOC_SCRATCH_BYTES);
  DeviceGuard dg(L->desc.device);
  if (!dg.ok) return fail(MOE_ERR_HIP, "moe_forward_noalloc: hipSetDevice(%d) failed", L->desc.device);
  void* ws = nullptr;
  int32_t st = scratch_of(L->desc.device, static_cast<hipStream_t>(stream), &ws);
  if (st != MOE_OK) return st;
  g_no_timing = true;
  st = moe_forward(L, x, T, y, route, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
  g_no_timing = false;
  return st;
}

int32_t moe_pack_fp4(const uint8_t* codes_in, const uint8_t* scales_in, uint8_t* codes_out, uint8_t* scales_out,
                     int32_t groups, int32_t rows, int32_t cols, void* stream) {
  if (!codes_in || !scales_in || !codes_out || !scales_out)
    return fail(MOE_ERR_INVALID, "moe_pack_fp4: NULL pointer");
  if (groups < 1 || rows < 1 || cols < 32 || cols % 32)
    return fail(MOE_ERR_INVALID, "moe_pack_fp4: groups=%d rows=%d cols=%d (cols must be a positive multiple of 32)",
                groups, rows, cols);
  if (!aligned16(codes_in) || !aligned16(codes_out))
    return fail(MOE_ERR_INVALID, "moe_pack_fp4: code arrays must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(scales_out) & 3u)
    return fail(MOE_ERR_INVALID, "moe_pack_fp4: scales_out must be 4-byte aligned");
  const size_t cb = (size_t)groups * rows * (cols / 2), sb = (size_t)groups * rows * (cols / 32);
  const size_t sb_out = (size_t)groups * moe::scale_slab_bytes(rows, cols);
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
  };
  if (overlap(codes_in, cb, codes_out, cb) || overlap(scales_in, sb, scales_out, sb_out))
    return fail(MOE_ERR_INVALID, "moe_pack_fp4: output overlaps input");
  const hipError_t e = moe::launch_pack(codes_in, scales_in, codes_out, scales_out, groups, rows, cols,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_pack_fp4: launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

int32_t moe_pack_fp8(const uint8_t* codes_in, uint8_t* codes_out, int32_t groups, int32_t rows, int32_t cols,
                     void* stream) {
  if (!codes_in || !codes_out) return fail(MOE_ERR_INVALID, "moe_pack_fp8: NULL pointer");
  if (groups < 1 || rows < 1 || cols < 128 || cols % 128)
    return fail(MOE_ERR_INVALID, "moe_pack_fp8: groups=%d rows=%d cols=%d (cols must be a positive multiple of 128)",
                groups, rows, cols);
  if (!aligned16(codes_in) || !aligned16(codes_out))
    return fail(MOE_ERR_INVALID, "moe_pack_fp8: code arrays must be 16-byte aligned");
  const size_t n = (size_t)groups * rows * cols;
  const char* a = reinterpret_cast<const char*>(codes_in);
  const char* b = reinterpret_cast<const char*>(codes_out);
  if (a < b + n && b < a + n) return fail(MOE_ERR_INVALID, "moe_pack_fp8: output overlaps input");
  const hipError_t e = moe::launch_pack_fp8(codes_in, codes_out, groups, rows, cols, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_pack_fp8: launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

int32_t moe_residual_rmsnorm(const float* h_src, const float* y, float* h_dst, const float* norm_weight, float eps,
                             uint16_t* x, int32_t T, int32_t H, void* stream) {
  if (T < 0 || T > kMaxTokens || H < 4 || H > (1 << 20) || H % 4)
    return fail(MOE_ERR_INVALID, "moe_residual_rmsnorm: tokens=%d hidden=%d (hidden a multiple of 4)", T, H);
  if (T == 0) return MOE_OK;
  if (!h_src) return fail(MOE_ERR_INVALID, "moe_residual_rmsnorm: NULL h_src");
  if (!y && !x) return fail(MOE_ERR_INVALID, "moe_residual_rmsnorm: neither y nor x given: nothing to do");
  if (!(eps > 0.f) || !(eps <= 3.402823466e38f))
    return fail(MOE_ERR_INVALID, "moe_residual_rmsnorm: eps=%g must be finite and > 0", (double)eps);
  if (!aligned16(h_src) || !aligned16(y) || !aligned16(h_dst) || !aligned16(norm_weight) ||
      (reinterpret_cast<uintptr_t>(x) & 7u))
    return fail(MOE_ERR_INVALID, "moe_residual_rmsnorm: float arrays must be 16-byte and x 8-byte aligned");
  const hipError_t e = moe::launch_residual_rmsnorm(h_src, y, y ? h_dst : nullptr, norm_weight, eps, x, T, H,
                                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_residual_rmsnorm: launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // extern "C"

struct moe_chain {
  int device = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

// Enqueue the chain's work on s (being captured): for each layer the join step and the layer,
// then the final residual add.
int32_t enqueue_chain(const moe_chain_desc* d, const std::vector<moe_route_out>& routes, hipStream_t s) {
  const moe::Dims& dm = d->layers[0]->dims;
  const int T = d->tokens, H = dm.H;
  const size_t plane = (size_t)T * H;
  const bool residual = d->flags & MOE_CHAIN_RESIDUAL;
  for (int l = 0; l < d->n_layers; ++l) {
    uint16_t* x = d->x + l * plane;
    moe::JoinArgs join{};
    bool fused = false;
    if (residual) {
      const float* g = d->norm_weight ? d->norm_weight[l] : nullptr;
      // layer 0 normalises h_in; layer l > 0 first adds y_{l-1} into the running residual
      const float* src = l <= 1 ? d->h_in : d->h_out;
      const float* yp = l == 0 ? nullptr : d->y + (l - 1) * plane;
      join = moe::JoinArgs{src, yp, l == 0 ? nullptr : d->h_out, g, d->eps};
      // small batches: the layer's routing launch does the join itself (the same arithmetic)
      fused = moe::join_fused(d->layers[l]->dims, T);
      if (!fused) {
        const hipError_t e = moe::launch_residual_rmsnorm(src, yp, join.h_dst, g, d->eps, x, T, H, s);
        if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_chain_create: join launch failed: %s", hipGetErrorString(e));
      }
    }
    const int32_t st = forward_impl(d->layers[l], x, T, d->y + l * plane, routes.empty() ? nullptr : &routes[l],
                                    d->workspace, d->workspace_bytes, s, fused ? &join : nullptr);
    if (st != MOE_OK) return st;
  }
  if (residual) {
    const int L = d->n_layers;
    const hipError_t e = moe::launch_residual_rmsnorm(L == 1 ? d->h_in : d->h_out, d->y + (L - 1) * plane,
                                                      d->h_out, nullptr, d->eps, nullptr, T, H, s);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_chain_create: residual launch failed: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

}  // namespace

extern "C" {

int32_t moe_chain_create(const moe_chain_desc* d, moe_chain** out) {
  if (!out) return fail(MOE_ERR_INVALID, "moe_chain_create: NULL out");
  *out = nullptr;
  if (!d) return fail(MOE_ERR_INVALID, "moe_chain_create: NULL descriptor");
  if (d->abi_version != MOE_ABI_VERSION)
    return fail(MOE_ERR_UNSUPPORTED, "moe_chain_create: abi_version %d, library %d", d->abi_version, MOE_ABI_VERSION);
  if (d->n_layers < 1 || d->n_layers > 1024 || !d->layers)
    return fail(MOE_ERR_INVALID, "moe_chain_create: n_layers=%d (1..1024) and a layer array are required", d->n_layers);
  if (d->tokens < 1 || d->tokens > kMaxTokens)
    return fail(MOE_ERR_INVALID, "moe_chain_create: tokens=%d out of [1, %d]", d->tokens, kMaxTokens);
  if (d->flags & ~MOE_CHAIN_RESIDUAL) return fail(MOE_ERR_INVALID, "moe_chain_create: unknown flags 0x%x", d->flags);
  if (d->reserved != 0) return fail(MOE_ERR_INVALID, "moe_chain_create: reserved must be 0");
  const bool residual = d->flags & MOE_CHAIN_RESIDUAL;
  for (int l = 0; l < d->n_layers; ++l) {
    const moe_layer* L = d->layers[l];
    if (!L) return fail(MOE_ERR_INVALID, "moe_chain_create: layer %d is NULL", l);
    if (L->dims.H != d->layers[0]->dims.H || L->desc.device != d->layers[0]->desc.device)
      return fail(MOE_ERR_INVALID, "moe_chain_create: layer %d differs from layer 0 in hidden size or device", l);
    const uint64_t need = carve(L->dims, d->tokens, nullptr, nullptr);
    if (!d->workspace || (reinterpret_cast<uintptr_t>(d->workspace) & 255u) || d->workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "moe_chain_create: layer %d needs %llu workspace bytes aligned to 256", l,
                  (unsigned long long)need);
    if (residual && d->norm_weight && !aligned16(d->norm_weight[l]))
      return fail(MOE_ERR_INVALID, "moe_chain_create: norm_weight[%d] must be 16-byte aligned", l);
    if (d->routes && !route_ok(&d->routes[l]))
      return fail(MOE_ERR_INVALID, "moe_chain_create: routes[%d] has a NULL buffer", l);
  }
  const int H = d->layers[0]->dims.H;
  const size_t plane = (size_t)d->tokens * H;
  if (!d->x || !d->y || !aligned16(d->x) || !aligned16(d->y))
    return fail(MOE_ERR_INVALID, "moe_chain_create: x and y are required and 16-byte aligned");
  if (overlaps(d->x, plane * 2 * d->n_layers, d->y, plane * 4 * d->n_layers))
    return fail(MOE_ERR_INVALID, "moe_chain_create: x and y overlap");
  if (residual) {
    if (!(d->eps > 0.f) || !(d->eps <= 3.402823466e38f))
      return fail(MOE_ERR_INVALID, "moe_chain_create: eps=%g must be finite and > 0", (double)d->eps);
    if (!d->h_in || !d->h_out || !aligned16(d->h_in) || !aligned16(d->h_out))
      return fail(MOE_ERR_INVALID, "moe_chain_create: h_in and h_out are required and 16-byte aligned");
    if (overlaps(d->h_in, plane * 4, d->h_out, plane * 4))
      return fail(MOE_ERR_INVALID, "moe_chain_create: h_in and h_out overlap");
  } else if (d->h_in || d->h_out || d->norm_weight) {
    return fail(MOE_ERR_INVALID, "moe_chain_create: h_in, h_out and norm_weight belong to MOE_CHAIN_RESIDUAL");
  }
  std::vector<moe_route_out> routes;
  if (d->routes) routes.assign(d->routes, d->routes + d->n_layers);

  const int dev = d->layers[0]->desc.device;
  DeviceGuard dg(dev);
  if (!dg.ok) return fail(MOE_ERR_HIP, "moe_chain_create: hipSetDevice(%d) failed", dev);
  moe_chain* c = new (std::nothrow) moe_chain;
  if (!c) return fail(MOE_ERR_ALLOC, "moe_chain_create: out of host memory");
  c->device = dev;
  hipStream_t s = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e != hipSuccess) {
    delete c;
    return fail(MOE_ERR_HIP, "moe_chain_create: hipStreamCreate failed: %s", hipGetErrorString(e));
  }
  int32_t st = MOE_OK;
  e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    st = fail(MOE_ERR_HIP, "moe_chain_create: hipStreamBeginCapture failed: %s", hipGetErrorString(e));
  } else {
    const bool no_timing = g_no_timing;
    g_no_timing = true;  // no timing events inside the graph
    st = enqueue_chain(d, routes, s);
    g_no_timing = no_timing;
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(s, &g);  // always ends the capture, also after a failed enqueue
    c->graph = g;
    if (st == MOE_OK && e != hipSuccess)
      st = fail(MOE_ERR_HIP, "moe_chain_create: hipStreamEndCapture failed: %s", hipGetErrorString(e));
    if (st == MOE_OK) {
      e = hipGraphInstantiate(&c->exec, c->graph, nullptr, nullptr, 0);
      if (e != hipSuccess) st = fail(MOE_ERR_HIP, "moe_chain_create: hipGraphInstantiate failed: %s", hipGetErrorString(e));
    }
  }
  (void)hipStreamDestroy(s);
  if (st != MOE_OK) {
    moe_chain_destroy(c);
    return st;
  }
  *out = c;
  return MOE_OK;
}

int32_t moe_chain_run(const moe_chain* c, void* stream) {
  if (!c || !c->exec) return fail(MOE_ERR_INVALID, "moe_chain_run: NULL chain");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(MOE_ERR_HIP, "moe_chain_run: hipSetDevice(%d) failed", c->device);
  const hipError_t e = hipGraphLaunch(c->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "moe_chain_run: hipGraphLaunch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

void moe_chain_destroy(moe_chain* c) {
  if (!c) return;
  DeviceGuard dg(c->device);
  if (c->exec) (void)hipGraphExecDestroy(c->exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  delete c;
}

int32_t moe_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_tenabled = on != 0;
  return MOE_OK;
}

int32_t moe_timing_read(const char** names, int64_t* launches, double* total_ms, int32_t cap) {
  std::lock_guard<std::mutex> lk(g_tmu);
  drain_timing_locked();
  int32_t i = 0;
  for (auto& kv : g_tacc) {
    if (i < cap) {
      if (names) names[i] = kv.second.name;
      if (launches) launches[i] = kv.second.launches;
      if (total_ms) total_ms[i] = kv.second.ms;
    }
    ++i;
  }
  return i;
}

void moe_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  drain_timing_locked();
  g_tacc.clear();
}

}  // extern "C"
