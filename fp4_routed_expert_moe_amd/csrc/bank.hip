// Partial-residency expert bank: a layer's FP4 experts live in page-locked host memory and are
// brought into n_slots HBM expert slots on demand, route-aware, in refill groups.
//
// The pages' prefill MoE routes on the device, then refills a transient per-layer VRAM expert
// bank in groups the size of its slots from page-locked host slabs, the lookups of group g+1
// overlapping the uploads of group g ("feat(v4/cuda): the CUDA tier wired into the DeepSeek V4
// engine", PR #1055, "What it is", the Prefill MoE item).  Here the lookups are host-side slot
// decisions, the uploads are DMA copies on copy streams of the bank's own, and the expert
// kernels are the grouped GEMM's, which take a group -> slot table and skip the M-tiles of
// groups outside the current refill group.  A slot reused within a call waits (on its copy
// stream) for the kernels of the refill group that last read it.
#include <algorithm>
#include <new>
#include <vector>

#include "api_internal.h"

using namespace moe_api;

namespace {
constexpr int kArrays = 6;  // gate codes, gate scales, up codes, up scales, down codes, down scales
// Copy streams the uploads rotate over, expert by expert: one stream's copies run on one DMA
// engine at a time, several keep more engines busy.
#ifndef MOE_BANK_COPY_STREAMS
#define MOE_BANK_COPY_STREAMS 4
#endif
constexpr int kCopies = MOE_BANK_COPY_STREAMS;
}

struct moe_bank {
  const moe_layer* layer = nullptr;  // host-resident weights
  moe_layer dev{};                   // the same layer over the slot arrays
  int device = 0, n_slots = 0, group = 0, max_groups = 0;
  size_t bytes[kArrays] = {};        // one group of each array
  uint8_t* slots[kArrays] = {};      // device [n_slots][bytes[i]]
  const uint8_t* host[kArrays] = {};
  hipStream_t copy[kCopies] = {};
  std::vector<hipEvent_t> ev_up, ev_done;  // ev_up: [max_groups][kCopies]
  hipEvent_t ev_end = nullptr;       // after the last call's combine
  bool called = false;
  int32_t* counts_host = nullptr;    // page-locked [E]
  int32_t* tables_host = nullptr;    // page-locked [max_groups][G]
  int32_t* tables_dev = nullptr;     // device [max_groups][G]
  std::vector<int> slot_group, group_slot;
  std::vector<int64_t> slot_tick;
  int64_t tick = 0;
  int64_t stats[5] = {};
};

namespace {

void release(moe_bank* k) {
  if (!k) return;
  DeviceGuard dg(k->device);
  for (auto& p : k->slots)
    if (p) (void)hipFree(p);
  for (auto e : k->ev_up)
    if (e) (void)hipEventDestroy(e);
  for (auto e : k->ev_done)
    if (e) (void)hipEventDestroy(e);
  if (k->ev_end) (void)hipEventDestroy(k->ev_end);
  for (auto c : k->copy)
    if (c) (void)hipStreamDestroy(c);
  if (k->counts_host) (void)hipHostFree(k->counts_host);
  if (k->tables_host) (void)hipHostFree(k->tables_host);
  if (k->tables_dev) (void)hipFree(k->tables_dev);
  delete k;
}

bool page_locked_host(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

}  // namespace

extern "C" {

int32_t moe_bank_create(const moe_layer* layer, int32_t n_slots, int32_t group, moe_bank** out) {
  if (!out) return fail(MOE_ERR_INVALID, "moe_bank_create: NULL out");
  *out = nullptr;
  if (!layer) return fail(MOE_ERR_INVALID, "moe_bank_create: NULL layer");
  if (layer->dims.fp8_shared) return fail(MOE_ERR_UNSUPPORTED, "moe_bank_create: an FP8 shared expert is not banked");
  if (group < 1 || n_slots < 2 * group || n_slots > (1 << 16))
    return fail(MOE_ERR_INVALID, "moe_bank_create: n_slots=%d, group=%d (need group >= 1, n_slots >= 2 * group)",
                n_slots, group);
  const moe::Dims& d = layer->dims;
  const moe_layer_desc& w = layer->desc;
  const uint8_t* host[kArrays] = {w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, w.down_codes, w.down_scales};
  DeviceGuard dg(w.device);
  if (!dg.ok) return fail(MOE_ERR_HIP, "moe_bank_create: hipSetDevice(%d) failed", w.device);
  for (int i = 0; i < kArrays; ++i)
    if (!page_locked_host(host[i]))
      return fail(MOE_ERR_INVALID, "moe_bank_create: weight array %d is not page-locked host memory", i);
  moe_bank* k = new (std::nothrow) moe_bank;
  if (!k) return fail(MOE_ERR_ALLOC, "moe_bank_create: out of host memory");
  k->layer = layer;
  k->device = w.device;
  k->n_slots = n_slots;
  k->group = group;
  k->max_groups = (d.G + group - 1) / group;
  const size_t code_bytes = (size_t)d.H * d.I / 2;
  k->bytes[0] = k->bytes[2] = code_bytes;
  k->bytes[1] = k->bytes[3] = moe::scale_slab_bytes(d.I, d.H);
  k->bytes[4] = code_bytes;
  k->bytes[5] = moe::scale_slab_bytes(d.H, d.I);
  hipError_t e = hipSuccess;
  for (int i = 0; i < kArrays && e == hipSuccess; ++i) {
    k->host[i] = host[i];
    e = hipMalloc(reinterpret_cast<void**>(&k->slots[i]), k->bytes[i] * n_slots);
  }
  for (int c = 0; c < kCopies && e == hipSuccess; ++c) e = hipStreamCreateWithFlags(&k->copy[c], hipStreamNonBlocking);
  k->ev_up.assign((size_t)k->max_groups * kCopies, nullptr);
  k->ev_done.assign(k->max_groups, nullptr);
  for (size_t i = 0; i < k->ev_up.size() && e == hipSuccess; ++i)
    e = hipEventCreateWithFlags(&k->ev_up[i], hipEventDisableTiming);
  for (int i = 0; i < k->max_groups && e == hipSuccess; ++i)
    e = hipEventCreateWithFlags(&k->ev_done[i], hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&k->ev_end, hipEventDisableTiming);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&k->counts_host), (size_t)d.E * 4, hipHostMallocDefault);
  const size_t tbytes = (size_t)k->max_groups * d.G * 4;
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&k->tables_host), tbytes, hipHostMallocDefault);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&k->tables_dev), tbytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    release(k);
    return fail(MOE_ERR_ALLOC, "moe_bank_create: device or page-locked allocation failed: %s", hipGetErrorString(e));
  }
  k->dev = *layer;
  k->dev.desc.gate_codes = k->slots[0];
  k->dev.desc.gate_scales = k->slots[1];
  k->dev.desc.up_codes = k->slots[2];
  k->dev.desc.up_scales = k->slots[3];
  k->dev.desc.down_codes = k->slots[4];
  k->dev.desc.down_scales = k->slots[5];
  k->dev.desc.path = MOE_PATH_GEMM;
  k->slot_group.assign(n_slots, -1);
  k->group_slot.assign(d.G, -1);
  k->slot_tick.assign(n_slots, -1);
  *out = k;
  return MOE_OK;
}

int32_t moe_bank_forward(moe_bank* k, const uint16_t* x, int32_t T, float* y, const moe_route_out* route, void* ws,
                         uint64_t ws_bytes, void* stream) {
  if (!k) return fail(MOE_ERR_INVALID, "moe_bank_forward: NULL bank");
  int32_t st = check_call(&k->dev, x, T, ws, ws_bytes, "moe_bank_forward");
  if (st != MOE_OK || T == 0) return st;
  if (!y || !aligned16(y)) return fail(MOE_ERR_INVALID, "moe_bank_forward: y must be given and 16-byte aligned");
  if (route && !route_ok(route)) return fail(MOE_ERR_INVALID, "moe_bank_forward: route_out given with a NULL buffer");
  DeviceGuard dg(k->device);
  if (!dg.ok) return fail(MOE_ERR_HIP, "moe_bank_forward: hipSetDevice(%d) failed", k->device);
  const moe::Dims& d = k->dev.dims;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // after a failed step the slot map may name uploads that never ran: forget every slot
  auto hip_fail = [&](hipError_t e, const char* what) {
    std::fill(k->slot_group.begin(), k->slot_group.end(), -1);
    std::fill(k->group_slot.begin(), k->group_slot.end(), -1);
    (void)hipEventRecord(k->ev_end, s);  // the next call waits for whatever this one enqueued
    k->called = true;
    return fail(MOE_ERR_HIP, "moe_bank_forward: %s: %s", what, hipGetErrorString(e));
  };
  // the previous call's work (on any stream) is done before its tables and slots are rewritten
  hipError_t e = k->called ? hipEventSynchronize(k->ev_end) : hipSuccess;
  if (e != hipSuccess) return hip_fail(e, "waiting for the previous call");

  moe::CallBufs b;
  carve(d, T, static_cast<char*>(ws), &b);
  if (route) use_route_out(b, route);
  st = enqueue_route(&k->dev, x, T, b, s, true, true, route != nullptr);
  if (st != MOE_OK) return st;  // nothing of the bank's state changed yet
  e = hipMemcpyAsync(k->counts_host, b.counts, (size_t)d.E * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the routing counts");

  // the groups with rows, resident ones first (they need no upload)
  std::vector<int> need, miss;
  for (int g = 0; g < d.G; ++g) {
    const bool active = g < d.E ? k->counts_host[g] > 0 : true;  // the shared expert always runs
    if (!active) continue;
    (k->group_slot[g] >= 0 ? need : miss).push_back(g);
  }
  const int hits = (int)need.size();
  need.insert(need.end(), miss.begin(), miss.end());
  std::vector<char> needed(d.G, 0);
  for (int g : need) needed[g] = 1;
  std::vector<int> slot_rg(k->n_slots, -1);  // refill group of this call that last used the slot
  const int n_rg = ((int)need.size() + k->group - 1) / k->group;
  const int mb = mt_bound_of(d, T);
  ++k->stats[0];
  k->stats[1] += hits;
  for (int rg = 0; rg < n_rg; ++rg) {
    const int lo = rg * k->group, hi = std::min((int)need.size(), lo + k->group);
    int32_t* table = k->tables_host + (size_t)rg * d.G;
    std::fill(table, table + d.G, -1);
    bool uploads[kCopies] = {};
    for (int j = lo; j < hi; ++j) {
      const int g = need[j];
      int slot = k->group_slot[g];
      if (slot < 0) {
        // a free slot, else the least recently used slot whose group this call does not need,
        // else the slot of the oldest refill group at least two back (after its kernels)
        int best = -1;
        int64_t best_key = 0;
        for (int c = 0; c < k->n_slots; ++c) {
          const int occ = k->slot_group[c];
          int64_t key;
          if (occ < 0) key = -2;                                     // empty
          else if (!needed[occ]) key = k->slot_tick[c];              // not needed: by age
          else if (slot_rg[c] >= 0 && slot_rg[c] <= rg - 2) key = ((int64_t)1 << 60) + slot_rg[c];
          else continue;                                              // needed now or in flight
          if (best < 0 || key < best_key) best = c, best_key = key;
        }
        if (best < 0) return hip_fail(hipErrorUnknown, "no slot free for a refill group");
        slot = best;
        const int cs = (int)(k->stats[2] % kCopies);  // the copy stream of this upload
        if (slot_rg[slot] >= 0) {
          e = hipStreamWaitEvent(k->copy[cs], k->ev_done[slot_rg[slot]], 0);
          if (e != hipSuccess) return hip_fail(e, "ordering a slot reuse");
        }
        if (k->slot_group[slot] >= 0) k->group_slot[k->slot_group[slot]] = -1;
        k->slot_group[slot] = g;
        k->group_slot[g] = slot;
        for (int i = 0; i < kArrays && e == hipSuccess; ++i)
          e = hipMemcpyAsync(k->slots[i] + (size_t)slot * k->bytes[i], k->host[i] + (size_t)g * k->bytes[i],
                             k->bytes[i], hipMemcpyHostToDevice, k->copy[cs]);
        if (e != hipSuccess) return hip_fail(e, "uploading an expert");
        ++k->stats[2];
        for (int i = 0; i < kArrays; ++i) k->stats[3] += (int64_t)k->bytes[i];
        uploads[cs] = true;
      }
      table[g] = slot;
      slot_rg[slot] = rg;
      k->slot_tick[slot] = ++k->tick;
    }
    for (int c = 0; c < kCopies; ++c) {
      if (!uploads[c]) continue;
      hipEvent_t ev = k->ev_up[(size_t)rg * kCopies + c];
      e = hipEventRecord(ev, k->copy[c]);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, ev, 0);
      if (e != hipSuccess) return hip_fail(e, "ordering the kernels after their uploads");
    }
    int32_t* tdev = k->tables_dev + (size_t)rg * d.G;
    e = hipMemcpyAsync(tdev, table, (size_t)d.G * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = moe::launch_gemm_gateup(d, k->dev.desc, x, b, T, mb, s, tdev);
    if (e == hipSuccess) e = moe::launch_gemm_down(d, k->dev.desc, b, T, mb, s, tdev);
    if (e == hipSuccess) e = hipEventRecord(k->ev_done[rg], s);
    if (e != hipSuccess) return hip_fail(e, "expert kernels of a refill group");
    ++k->stats[4];
  }
  e = moe::launch_combine(d, b, y, T, s);
  if (e == hipSuccess) e = hipEventRecord(k->ev_end, s);
  if (e != hipSuccess) return hip_fail(e, "combine");
  k->called = true;
  return MOE_OK;
}

int32_t moe_bank_stats(const moe_bank* k, int64_t* out) {
  if (!k || !out) return fail(MOE_ERR_INVALID, "moe_bank_stats: NULL argument");
  for (int i = 0; i < 5; ++i) out[i] = k->stats[i];
  return MOE_OK;
}

void moe_bank_destroy(moe_bank* k) { release(k); }

}  // extern "C"
