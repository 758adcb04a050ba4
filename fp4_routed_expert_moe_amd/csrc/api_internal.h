// Internal interface shared by the C-ABI sources (api.hip, bank.hip); not part of the ABI.
#pragma once
#include <cstddef>
#include <cstdint>

#include "common.h"

struct moe_layer {
  moe_layer_desc desc;
  moe::Dims dims;
};

namespace moe_api {

constexpr int kMaxTokens = 1 << 20;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sets the calling thread's last-error message and returns `code`.
int fail(int code, const char* fmt, ...);
// Workspace layout for T tokens; assigns pointers when base != nullptr.  Returns bytes.
size_t carve(const moe::Dims& d, int T, char* base, moe::CallBufs* b);
// Upper bound of the grouped GEMM's M-tiles for T tokens.
int mt_bound_of(const moe::Dims& d, int T);
// Argument and workspace checks of a layer call (MOE_OK, or the failure status).
int32_t check_call(const moe_layer* L, const uint16_t* x, int32_t T, void* ws, uint64_t ws_bytes, const char* what);
// Routing launches; `forward` also writes the FP8 activation terms, `gemm` the M-tile list,
// `route_out` every routing table.
int32_t enqueue_route(const moe_layer* L, const uint16_t* x, int32_t T, moe::CallBufs& b, hipStream_t s,
                      bool forward, bool gemm, bool route_out, const moe::JoinArgs* join = nullptr);
// moe_forward with, optionally, the chained decode's join done by the routing launch (x is
// then written from the residual; moe::join_fused must hold).
int32_t forward_impl(const moe_layer* L, const uint16_t* x, int32_t T, float* y, const moe_route_out* route,
                     void* ws, uint64_t ws_bytes, hipStream_t s, const moe::JoinArgs* join);
void use_route_out(moe::CallBufs& b, const moe_route_out* r);
bool route_ok(const moe_route_out* r);

// Makes `dev` the current device for a scope and restores the previous one.
struct DeviceGuard {
  int old = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&old) != hipSuccess) old = -1;
    if (old != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (old >= 0) (void)hipSetDevice(old);
  }
};

}  // namespace moe_api
