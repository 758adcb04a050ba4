// Host-side checks of the C ABI (include/moe.h), built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library and run on the CPU, with no GPU:
// argument validation, descriptor checks, workspace sizing, the error strings, the test hooks
// (MOE_FAKE_ARCH, MOE_FAIL_ALLOC), create/destroy pairs and the timing calls.  Nothing here
// launches a kernel.  Exit status 0 when every check holds; the sanitizers abort on the first
// memory or undefined-behaviour error (and report leaks at exit).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static moe_layer_desc base_desc(void) {
  moe_layer_desc d;
  memset(&d, 0, sizeof(d));
  d.abi_version = MOE_ABI_VERSION;
  d.hidden = 4096;
  d.n_experts = 256;
  d.top_k = 6;
  d.n_shared = 1;
  d.inter = 2048;
  d.path = MOE_PATH_AUTO;
  d.device = 0;
  d.block = 32;
  d.flags = 0;
  d.routed_scale = 1.0f;
  d.reserved = 0;
  // never dereferenced on the host: the library only keeps and checks these pointers
  d.w_router = (const float*)0x10000;
  d.gate_codes = (const uint8_t*)0x20000;
  d.gate_scales = (const uint8_t*)0x30000;
  d.up_codes = (const uint8_t*)0x40000;
  d.up_scales = (const uint8_t*)0x50000;
  d.down_codes = (const uint8_t*)0x60000;
  d.down_scales = (const uint8_t*)0x70000;
  return d;
}

static int create(const moe_layer_desc* d, moe_layer** out) {
  *out = (moe_layer*)0x1;
  const int st = moe_layer_create(d, out);
  if (st != MOE_OK) CHECK(*out == NULL && moe_last_error()[0] != '\0');
  return st;
}

int main(void) {
  CHECK(moe_abi_version() == MOE_ABI_VERSION);
  for (int s = 0; s < 8; ++s) CHECK(moe_status_string(s) != NULL && moe_status_string(s)[0] != '\0');

  // no GPU here: the real device check fails and names the reason
  unsetenv("MOE_FAKE_ARCH");
  char name[8];
  CHECK(moe_device_supported(0, name, sizeof(name)) == 0);
  CHECK(strlen(name) < sizeof(name));
  CHECK(moe_device_supported(0, NULL, 0) == 0);
  moe_layer_desc d = base_desc();
  moe_layer* L;
  CHECK(create(&d, &L) == MOE_ERR_UNSUPPORTED);

  // fake architecture: host paths without a GPU
  setenv("MOE_FAKE_ARCH", "gfx942", 1);
  CHECK(moe_device_supported(0, name, sizeof(name)) == 0);
  CHECK(create(&d, &L) == MOE_ERR_UNSUPPORTED);
  setenv("MOE_FAKE_ARCH", "gfx950:sramecc+:xnack-", 1);
  char longname[4];
  CHECK(moe_device_supported(0, longname, sizeof(longname)) == 1);
  CHECK(strcmp(longname, "gfx") == 0);  // truncated, NUL-terminated
  CHECK(moe_device_supported(-1, NULL, 0) == 0);

  // descriptor validation
  struct {
    int field, value, status;
  } bad[] = {
      {0, 99, MOE_ERR_UNSUPPORTED}, {1, 100, MOE_ERR_INVALID}, {1, 16, MOE_ERR_INVALID},
      {1, 16384, MOE_ERR_INVALID},  {2, 0, MOE_ERR_INVALID},   {2, 2000, MOE_ERR_INVALID},
      {3, 0, MOE_ERR_INVALID},      {3, 257, MOE_ERR_INVALID}, {4, 2, MOE_ERR_INVALID},
      {5, 48, MOE_ERR_INVALID},     {6, 7, MOE_ERR_INVALID},
  };
  for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
    moe_layer_desc b = base_desc();
    int32_t* f[] = {&b.abi_version, &b.hidden, &b.n_experts, &b.top_k, &b.n_shared, &b.inter, &b.path};
    *f[bad[i].field] = bad[i].value;
    CHECK(create(&b, &L) == bad[i].status);
  }
  {
    moe_layer_desc b = base_desc();
    b.down_codes = NULL;
    CHECK(create(&b, &L) == MOE_ERR_INVALID);
    b = base_desc();
    b.gate_codes = (const uint8_t*)0x20004;
    CHECK(create(&b, &L) == MOE_ERR_INVALID);
    CHECK(moe_layer_create(NULL, &L) == MOE_ERR_INVALID);
    CHECK(moe_layer_create(&b, NULL) == MOE_ERR_INVALID);
  }

  // injected allocation failure: nothing created, nothing leaked
  setenv("MOE_FAIL_ALLOC", "1", 1);
  CHECK(create(&d, &L) == MOE_ERR_ALLOC);
  unsetenv("MOE_FAIL_ALLOC");

  // a layer, its workspace sizes, and calls rejected before anything is enqueued
  CHECK(create(&d, &L) == MOE_OK && L != NULL);
  const uint64_t w1 = moe_workspace_bytes(L, 1), w8 = moe_workspace_bytes(L, 8);
  CHECK(w1 > 0 && w1 <= w8 && w8 <= moe_workspace_bytes(L, 4096));
  CHECK(moe_workspace_bytes(L, 0) == w1);
  CHECK(moe_workspace_bytes(L, -1) == 0 && moe_workspace_bytes(L, (1 << 20) + 1) == 0);
  CHECK(moe_workspace_bytes(NULL, 8) == 0);
  CHECK(moe_workspace_bytes(L, 340) <= MOE_NOALLOC_SCRATCH_BYTES);
  CHECK(moe_workspace_bytes(L, 341) > MOE_NOALLOC_SCRATCH_BYTES);

  const uint16_t* x = (const uint16_t*)0x100000;
  float* y = (float*)0x200000;
  void* ws = (void*)0x300000;
  CHECK(moe_forward(L, x, 0, y, NULL, NULL, 0, NULL) == MOE_OK);  // T = 0: no-op
  CHECK(moe_forward(L, x, -1, y, NULL, ws, w8, NULL) == MOE_ERR_INVALID);
  CHECK(moe_forward(L, NULL, 8, y, NULL, ws, w8, NULL) == MOE_ERR_INVALID);
  CHECK(moe_forward(L, (const uint16_t*)0x100002, 8, y, NULL, ws, w8, NULL) == MOE_ERR_INVALID);
  CHECK(moe_forward(L, x, 8, y, NULL, NULL, w8, NULL) == MOE_ERR_WORKSPACE);
  CHECK(moe_forward(L, x, 8, y, NULL, ws, w8 - 1, NULL) == MOE_ERR_WORKSPACE);
  CHECK(moe_forward(L, x, 8, y, NULL, (void*)0x300010, w8, NULL) == MOE_ERR_WORKSPACE);
  CHECK(moe_forward(L, x, 8, NULL, NULL, ws, w8, NULL) == MOE_ERR_INVALID);
  CHECK(moe_forward(L, x, 8, (float*)0x200004, NULL, ws, w8, NULL) == MOE_ERR_INVALID);
  moe_route_out r;
  memset(&r, 0, sizeof(r));
  CHECK(moe_forward(L, x, 8, y, &r, ws, w8, NULL) == MOE_ERR_INVALID);  // route with NULL buffers
  CHECK(moe_route(L, x, 8, NULL, ws, w8, NULL) == MOE_ERR_INVALID);
  CHECK(moe_route(L, x, 8, &r, ws, w8, NULL) == MOE_ERR_INVALID);
  CHECK(moe_route(NULL, x, 8, &r, ws, w8, NULL) == MOE_ERR_INVALID);
  CHECK(moe_forward_noalloc(L, x, 341, y, NULL, NULL) == MOE_ERR_WORKSPACE);
  CHECK(strstr(moe_last_error(), "scratch") != NULL);
  CHECK(moe_forward_noalloc(L, x, -3, y, NULL, NULL) == MOE_ERR_INVALID);
  CHECK(moe_forward_noalloc(L, x, 0, y, NULL, NULL) == MOE_OK);
  CHECK(moe_forward_noalloc(NULL, x, 8, y, NULL, NULL) == MOE_ERR_INVALID);

  // the join step: rejected on the host
  float* h = (float*)0x800000;
  uint16_t* xo = (uint16_t*)0x900000;
  CHECK(moe_residual_rmsnorm(h, y, h, NULL, 1e-6f, xo, 0, 256, NULL) == MOE_OK);  // T = 0: no-op
  CHECK(moe_residual_rmsnorm(h, y, h, NULL, 1e-6f, xo, -1, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(h, y, h, NULL, 1e-6f, xo, 8, 254, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(NULL, y, h, NULL, 1e-6f, xo, 8, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(h, NULL, h, NULL, 1e-6f, NULL, 8, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(h, y, h, NULL, 0.f, xo, 8, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(h, y, h, NULL, -1.f, xo, 8, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(h + 1, y, h, NULL, 1e-6f, xo, 8, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(h, y, h, (const float*)0x800008, 1e-6f, xo, 8, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_residual_rmsnorm(h, y, h, NULL, 1e-6f, xo + 1, 8, 256, NULL) == MOE_ERR_INVALID);

  // chain descriptors: every rejection leaves *out NULL and leaks nothing
  {
    const moe_layer* layers[2] = {L, L};
    moe_chain_desc c;
    memset(&c, 0, sizeof(c));
    c.abi_version = MOE_ABI_VERSION;
    c.n_layers = 2;
    c.tokens = 8;
    c.flags = MOE_CHAIN_RESIDUAL;
    c.eps = 1e-6f;
    c.layers = layers;
    c.h_in = (const float*)0xa00000;
    c.h_out = (float*)0xb00000;
    c.x = (uint16_t*)0xc00000;
    c.y = (float*)0xd00000;
    c.workspace = ws;
    c.workspace_bytes = w8;
    moe_chain* ch = (moe_chain*)0x1;
    CHECK(moe_chain_create(NULL, &ch) == MOE_ERR_INVALID && ch == NULL);
    CHECK(moe_chain_create(&c, NULL) == MOE_ERR_INVALID);
    struct {
      void (*edit)(moe_chain_desc*);
      int status;
    } bad[] = {
        {[](moe_chain_desc* b) { b->abi_version = 1; }, MOE_ERR_UNSUPPORTED},
        {[](moe_chain_desc* b) { b->n_layers = 0; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->tokens = 0; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->flags = 2; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->reserved = 1; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->layers = NULL; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->workspace_bytes -= 1; }, MOE_ERR_WORKSPACE},
        {[](moe_chain_desc* b) { b->workspace = (char*)b->workspace + 16; }, MOE_ERR_WORKSPACE},
        {[](moe_chain_desc* b) { b->x = NULL; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->y = (float*)((char*)b->x + 64); }, MOE_ERR_INVALID},  // x, y overlap
        {[](moe_chain_desc* b) { b->eps = 0.f; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->h_out = (float*)b->h_in + 16; }, MOE_ERR_INVALID},     // h overlap
        {[](moe_chain_desc* b) { b->h_in = NULL; }, MOE_ERR_INVALID},
        {[](moe_chain_desc* b) { b->flags = 0; }, MOE_ERR_INVALID},  // h_in given without RESIDUAL
    };
    for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
      moe_chain_desc b = c;
      bad[i].edit(&b);
      ch = (moe_chain*)0x1;
      CHECK(moe_chain_create(&b, &ch) == bad[i].status && ch == NULL);
    }
    const moe_layer* with_null[2] = {L, NULL};
    moe_chain_desc b = c;
    b.layers = with_null;
    CHECK(moe_chain_create(&b, &ch) == MOE_ERR_INVALID && ch == NULL);
    // a descriptor that passes every host check reaches the device, which this host lacks
    ch = (moe_chain*)0x1;
    CHECK(moe_chain_create(&c, &ch) == MOE_ERR_HIP && ch == NULL);
    CHECK(moe_chain_run(NULL, NULL) == MOE_ERR_INVALID);
    moe_chain_destroy(NULL);
  }

  // expert bank: argument checks on the host; a well-formed request reaches the device
  {
    moe_bank* bk = (moe_bank*)0x1;
    CHECK(moe_bank_create(L, 4, 2, NULL) == MOE_ERR_INVALID);
    CHECK(moe_bank_create(NULL, 4, 2, &bk) == MOE_ERR_INVALID && bk == NULL);
    bk = (moe_bank*)0x1;
    CHECK(moe_bank_create(L, 3, 2, &bk) == MOE_ERR_INVALID && bk == NULL);  // fewer than 2 * group slots
    bk = (moe_bank*)0x1;
    CHECK(moe_bank_create(L, 4, 0, &bk) == MOE_ERR_INVALID && bk == NULL);
    bk = (moe_bank*)0x1;
    CHECK(moe_bank_create(L, 4, 2, &bk) == MOE_ERR_HIP && bk == NULL);      // no device on this host
    CHECK(moe_bank_forward(NULL, x, 8, y, NULL, ws, w8, NULL) == MOE_ERR_INVALID);
    int64_t st5[5];
    CHECK(moe_bank_stats(NULL, st5) == MOE_ERR_INVALID);
    moe_bank_destroy(NULL);
  }
  moe_layer_destroy(L);
  moe_layer_destroy(NULL);

  // repack argument checks (no launch: every call below is rejected on the host)
  const uint8_t* ci = (const uint8_t*)0x400000;
  const uint8_t* si = (const uint8_t*)0x500000;
  uint8_t* co = (uint8_t*)0x600000;
  uint8_t* so = (uint8_t*)0x700000;
  CHECK(moe_pack_fp4(NULL, si, co, so, 1, 64, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp4(ci, si, co, so, 0, 64, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp4(ci, si, co, so, 1, 64, 48, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp4(ci + 8, si, co, so, 1, 64, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp4(ci, si, co, so + 2, 1, 64, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp4(ci, si, (uint8_t*)ci + 16, so, 1, 64, 256, NULL) == MOE_ERR_INVALID);  // overlap
  CHECK(moe_pack_fp8(NULL, co, 1, 64, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp8(ci, co, 1, 64, 96, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp8(ci, co + 8, 1, 64, 256, NULL) == MOE_ERR_INVALID);
  CHECK(moe_pack_fp8(ci, (uint8_t*)ci + 64, 1, 64, 256, NULL) == MOE_ERR_INVALID);  // overlap

  // the FP8 shared expert's descriptor checks, and routed_scale / block / reserved
  {
    moe_layer_desc b = base_desc();
    b.flags = MOE_SHARED_FP8;
    CHECK(create(&b, &L) == MOE_ERR_INVALID);  // pointers missing
    b.shared_gate_fp8 = (const uint8_t*)0x80000;
    b.shared_gate_fp8_scales = (const float*)0x90000;
    b.shared_up_fp8 = (const uint8_t*)0xa0000;
    b.shared_up_fp8_scales = (const float*)0xb0000;
    b.shared_down_fp8 = (const uint8_t*)0xc0000;
    b.shared_down_fp8_scales = (const float*)0xd0000;
    CHECK(create(&b, &L) == MOE_OK && L != NULL);
    moe_layer_destroy(L);
    b.shared_down_fp8_scales = (const float*)0xd0002;
    CHECK(create(&b, &L) == MOE_ERR_INVALID);  // misaligned scales
    b = base_desc();
    b.routed_scale = -1.0f;
    CHECK(create(&b, &L) == MOE_ERR_INVALID);
    b = base_desc();
    b.block = 64;
    CHECK(create(&b, &L) == MOE_ERR_INVALID);
  }

  // timing calls with nothing recorded
  CHECK(moe_timing_enable(1) == MOE_OK);
  CHECK(moe_timing_read(NULL, NULL, NULL, 0) == 0);
  moe_timing_reset();
  CHECK(moe_timing_enable(0) == MOE_OK);

  unsetenv("MOE_FAKE_ARCH");
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("abi host checks: ok\n");
  return failures ? 1 : 0;
}
