/*
 * moe.h -- C ABI of the routed FP4-expert MoE layer for AMD Instinct MI355X (gfx950).
 *
 * The header includes only <stdint.h> and the caller drives the library, never the
 * other way round: the same shape as the kernel tier on "DeepSeek V4: the CUDA
 * kernels, as a tier rather than an engine" (PR #772, "Why it works as a tier").
 * The caller owns device memory and streams; the library enqueues kernels.
 *
 * The layer (for T tokens of width H, E routed experts, top-k, S shared experts, expert
 * width I):
 *   1. router scores   l[t,e] = sum_h x[t,h] * w_router[e,h] + router_bias[e]   (fp32)
 *   2. top-k per token (score descending, ties to the lower expert index) and weights
 *      w[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected scores
 *   3. rows grouped by expert: counts[e], offsets[e] (exclusive scan, offsets[E] = T*k),
 *      perm[r] = t*k + j for the pair at grouped row r, ascending token within an expert
 *   4. per expert, SwiGLU with FP4 weights dequantised on the fly:
 *      h = silu(x Wg^T) * (x Wu^T),  y_e = h Wd^T
 *   5. the shared expert (S = 1) on every token with weight 1
 *   6. y[t] = y_shared[t] + sum_j w[t,j] * y_{idx[t,j]}[t]
 * Steps 1-3 follow "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine"
 * (PR #1055, "What it is": prefill routes on the device into expert-grouped GEMM rows;
 * decode fuses routed and shared experts).  Step 4's format follows "Add DeepSeek V4 Flash
 * CPU inference with NVMe expert streaming" (PR #165): FP4 E2M1 values with one UE8M0
 * scale per group of 32 along the reduction axis.
 *
 * Weight layouts.  Group g in [0, E+S); the shared expert is group E.  A matrix has N output
 * rows and a reduction axis of K values (gate/up: N = I, K = H; down: N = H, K = I); e2m1
 * codes pack two values per byte (low nibble = even element) and one e8m0 scale covers 32
 * consecutive values of a row.  An e8m0 byte s means the float32 with bit pattern s << 23
 * (s = 0 is +0, s = 255 is +inf), as "DeepSeek V4: the CUDA kernels, as a tier rather than an
 * engine" (PR #772) describes for the MXFP4 decode.
 *   checkpoint layout (row-major):   codes uint8 [E+S][N][K/2],       scales uint8 [E+S][N][K/32]
 *   kernel layout (block-interleaved): codes uint8 [E+S][K/32][N][16],
 *                                      scales uint8 [E+S][ceil(K/128)][ceil(N/64)][16][4][4]
 * In the kernel layout the 16 code bytes of block kb of consecutive rows are adjacent, which
 * is what the decode kernels stream (one lane per row, one contiguous KiB per wave load).
 * Scale byte (i, t, m, q, j) of a group is the scale of row 64t + 16j + m, block 4i + q
 * (0 where that row or block is past the matrix): the four scales one lane needs for a
 * 128-value K step of a 64-row tile share a dword.
 * moe_pack_fp4 converts the first into the second once, at load time; the layer reads the
 * kernel layout only.
 *
 * Errors: every entry point returns a status (MOE_OK = 0).  Argument errors are reported
 * before anything is enqueued; launch errors are read back with hipGetLastError right after
 * the launches; a device fault surfaces at the caller's next synchronisation.  No C++
 * exception crosses this boundary.  moe_last_error() gives a message for the calling
 * thread's last failure, so a caller can log the reason and fall back (the per-stage
 * fallback convention of PR #1055).
 */
#ifndef MOE_FP4_MOE_H
#define MOE_FP4_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* NULL pointer, bad size, inconsistent descriptor */
  MOE_ERR_UNSUPPORTED = 2,  /* no device, device is not gfx950, ABI version mismatch */
  MOE_ERR_WORKSPACE = 3,    /* workspace pointer NULL or smaller than moe_workspace_bytes */
  MOE_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  MOE_ERR_ALLOC = 5         /* the library could not allocate its own small metadata */
};

/* Execution path for the expert products.  AUTO picks by token count: the FP4 GEMV
 * kernels (decode: HBM-bound, few rows per expert) or the FP4 grouped GEMM (prefill); both
 * run on the block-scaled FP8 x FP4 matrix cores.  The two others force one path (A/B
 * testing, the kill-switch pattern of PR #165's AVX2 series). */
enum moe_path { MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_GEMM = 2 };

/* Layer flags. */
enum moe_flags {
  /* The shared expert is stored as FP8 E4M3 with a float32 scale per 128 x 128 block, the dense
   * format of the V4 checkpoints ("Add DeepSeek V4 Flash CPU inference with NVMe expert
   * streaming", PR #165, the question on V4 sizes: "FP8 E4M3 dense with 128x128 block scales").
   * Element (n, k) = E4M3(code) * scale[n / 128][k / 128]; E4M3 has 1 sign, 4 exponent (bias 7)
   * and 3 mantissa bits, subnormals, and NaN at 0x7F / 0xFF.  Requires n_shared = 1 and H, I
   * multiples of 128; the FP4 arrays then hold the E routed experts only. */
  MOE_SHARED_FP8 = 1
};

/* Layer description.  All pointers are device pointers on `device`.  The library BORROWS
 * them: the caller keeps them alive and unchanged until moe_layer_destroy. */
typedef struct moe_layer_desc {
  int32_t abi_version;   /* must be MOE_ABI_VERSION */
  int32_t hidden;        /* H: multiple of 32, 32..8192 */
  int32_t n_experts;     /* E: 1..1024 */
  int32_t top_k;         /* k: 1..E */
  int32_t n_shared;      /* S: 0 or 1 */
  int32_t inter;         /* I: multiple of 32, 32..8192 */
  int32_t path;          /* enum moe_path */
  int32_t device;        /* HIP device ordinal holding the weights */
  int32_t block;         /* values per FP4 scale along the reduction axis: must be 32 */
  int32_t flags;         /* enum moe_flags, OR-ed */
  float routed_scale;    /* the routed experts' sum is multiplied by this (1.0 for V4 Flash);
                            finite and > 0; the shared expert's weight stays 1 */
  int32_t reserved;      /* must be 0 */
  const float* w_router;       /* fp32 [E][H] */
  const float* router_bias;    /* fp32 [E], or NULL for no bias */
  /* FP4 experts, kernel layout (see above); G = E + S groups, or E with MOE_SHARED_FP8 */
  const uint8_t* gate_codes;   /* [G][H/32][I][16] */
  const uint8_t* gate_scales;  /* [G][ceil(H/128)][ceil(I/64)][16][4][4] */
  const uint8_t* up_codes;     /* [G][H/32][I][16] */
  const uint8_t* up_scales;    /* [G][ceil(H/128)][ceil(I/64)][16][4][4] */
  const uint8_t* down_codes;   /* [G][I/32][H][16] */
  const uint8_t* down_scales;  /* [G][ceil(I/128)][ceil(H/64)][16][4][4] */
  /* MOE_SHARED_FP8 only (else NULL): the shared expert in the FP8 kernel layout, codes
   * [K/128][N][128] (the 128 values of reduction step j of row n together, see moe_pack_fp8)
   * and float32 scales [N/128][K/128] as stored; gate/up N = I, K = H; down N = H, K = I */
  const uint8_t* shared_gate_fp8;
  const float* shared_gate_fp8_scales;
  const uint8_t* shared_up_fp8;
  const float* shared_up_fp8_scales;
  const uint8_t* shared_down_fp8;
  const float* shared_down_fp8_scales;
} moe_layer_desc;

/* Routing results (device pointers), written by moe_route / moe_forward. */
typedef struct moe_route_out {
  int32_t* idx;      /* [T][k] expert of slot j of token t, score-descending */
  float* weight;     /* [T][k] renormalised softmax weight of that slot */
  int32_t* counts;   /* [E] rows per expert */
  int32_t* offsets;  /* [E+1] exclusive scan of counts; offsets[E] = T*k */
  int32_t* perm;     /* [T*k] t*k+j at grouped row r, ascending t within an expert */
} moe_route_out;

typedef struct moe_layer moe_layer;

/* MOE_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

/* 1 if HIP device `device` is a gfx950 the library was built for, else 0.  Writes the
 * device's architecture name (or a reason) into name[0..cap-1], NUL-terminated, when
 * name is not NULL and cap > 0.  "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4
 * engine" (PR #1055, "What it is") checks the architecture before anything else runs; this is
 * that check for gfx950.  Test hook: when the environment variable MOE_FAKE_ARCH is set, its
 * value is taken as every device's architecture and no HIP call is made (host-side paths can
 * then be exercised without a GPU). */
int32_t moe_device_supported(int32_t device, char* name, int32_t cap);

/* Validate `desc`, check the device, and create a layer.  On success *out is a new layer
 * (destroy with moe_layer_destroy); on failure *out is NULL and nothing is leaked.  Test hook:
 * with MOE_FAIL_ALLOC set in the environment the layer's host allocation fails
 * (MOE_ERR_ALLOC).
 * Enqueues no work.  A layer is immutable after creation: concurrent calls on different
 * streams are safe when each uses its own workspace. */
int32_t moe_layer_create(const moe_layer_desc* desc, moe_layer** out);

/* Free the layer's own metadata (never the borrowed weights).  NULL is a no-op.  The
 * caller must have synchronised every stream that used the layer. */
void moe_layer_destroy(moe_layer* layer);

/* Bytes of device workspace one call with up to max_tokens tokens needs (0 on bad
 * arguments).  The caller allocates and owns it; it must be 256-byte aligned and filled with
 * zeros before its first use.  Its first bytes are control words (device-scope counters the
 * kernels use to let one workgroup finish a stage for the others; their number is fixed);
 * every call that completes leaves them at zero, so a workspace is zeroed once, not per
 * call, and may serve any layer it is large enough for.
 * A workspace serves one stream at a time: calls that overlap on one workspace race. */
uint64_t moe_workspace_bytes(const moe_layer* layer, int32_t max_tokens);

/* Steps 1-3 for x (bf16 bit patterns, device, [T][H]) into `route` (all five pointers
 * required).  Asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 * T = 0 is a no-op.  No host synchronisation. */
int32_t moe_route(const moe_layer* layer, const uint16_t* x, int32_t tokens,
                  const moe_route_out* route, void* workspace, uint64_t workspace_bytes,
                  void* stream);

/* The whole layer: y (fp32, device, [T][H]; must not overlap x or the workspace) for x
 * (bf16 bit patterns, device, [T][H]).  If `route` is not NULL its five buffers receive
 * the routing (as moe_route); if NULL no routing output is produced, and a small batch then
 * builds only the grouping its own expert kernels read (the output is the same bit for bit).
 * Asynchronous on `stream`; T = 0 is a no-op; no host synchronisation.  Device-side failures
 * are not reported by the return value: a fault surfaces at the caller's next synchronisation,
 * and the small-batch combine, which waits for the other workgroups' rows with a bounded poll
 * (every one of them is dispatched before the combining workgroup, so the bound is never
 * reached in a launch that runs), would leave NaN in the outputs it gave up on. */
int32_t moe_forward(const moe_layer* layer, const uint16_t* x, int32_t tokens, float* y,
                    const moe_route_out* route, void* workspace, uint64_t workspace_bytes,
                    void* stream);

/* Bytes of the scratch array moe_forward_noalloc uses as its workspace, per device. */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same layer, the same kernels and
 * the same result, bit for bit, with the workspace in a scratch array the library holds, one
 * per device (MOE_NOALLOC_SCRATCH_BYTES each, kept until the process ends), instead of a
 * caller-allocated one.  No device memory is allocated or freed.  The first call on a device
 * looks the array up (hipGetSymbolAddress) and enqueues one small kernel on `stream` that
 * zeroes its control words.  Calls whose workspace (moe_workspace_bytes) would exceed the
 * array return MOE_ERR_WORKSPACE before anything is enqueued: at H=4096, E=256, top-6, one
 * shared expert, I=2048 that allows up to 340 tokens.  Every call on a device shares its
 * array: calls that overlap on one device (different streams or threads) race; serialise
 * them.  Kernel timing (moe_timing_*) does not record these calls. */
int32_t moe_forward_noalloc(const moe_layer* layer, const uint16_t* x, int32_t tokens, float* y,
                            const moe_route_out* route, void* stream);

/* Repack `groups` FP4 matrices of `rows` x `cols` (cols = reduction axis, multiple of 32)
 * from the checkpoint layout into the kernel layout (device pointers; codes 16-byte aligned,
 * scales_out 4-byte aligned and groups * ceil(cols/128) * ceil(rows/64) * 256 bytes long;
 * outputs must not overlap inputs).  Asynchronous on `stream` (a hipStream_t, NULL = default
 * stream) of the current device.  "Add DeepSeek V4 Flash CPU inference with NVMe expert
 * streaming" (PR #165) likewise repacks each expert once into its kernels' interleaved layout. */
int32_t moe_pack_fp4(const uint8_t* codes_in, const uint8_t* scales_in, uint8_t* codes_out,
                     uint8_t* scales_out, int32_t groups, int32_t rows, int32_t cols, void* stream);

/* Repack `groups` FP8 E4M3 matrices of `rows` x `cols` (cols = reduction axis, multiple of 128)
 * from the checkpoint layout codes [groups][rows][cols] into the kernel layout
 * [groups][cols/128][rows][128] (device pointers, 16-byte aligned, not overlapping).  Their
 * float32 block scales need no repacking.  Asynchronous on `stream` of the current device. */
int32_t moe_pack_fp8(const uint8_t* codes_in, uint8_t* codes_out, int32_t groups, int32_t rows, int32_t cols,
                     void* stream);

/* ---- chained decode -----------------------------------------------------------------
 * The pages run the MoE stage once per transformer layer in decode ("feat(v4/cuda): the CUDA
 * tier wired into the DeepSeek V4 engine", PR #1055, "What it is"; V4 Flash has 43 layers,
 * "Add DeepSeek V4 Flash CPU inference with NVMe expert streaming", PR #165) and leave the
 * join between layers open.  The library takes the plain pre-norm residual reading, with
 * attention and hyper-connection mixing left to the caller:
 *   x_l = bf16(RMSNorm(h_l) * gamma_l),  y_l = MoE_l(x_l),  h_{l+1} = h_l + y_l,
 *   RMSNorm(v) = v / sqrt(mean(v^2) + eps). */

/* One join step on T rows of width H (device pointers, float4-aligned, H a multiple of 4):
 *   if y is not NULL:  h_dst = h_src + y   (fp32, one rounding per add; h_dst may equal
 *                                            h_src, NULL means h_dst is not written)
 *   if x is not NULL:  x = bf16 round-to-nearest-even of (h * (1/sqrt(mean(h^2) + eps))) *
 *                      norm_weight, h being h_src (+ y); norm_weight NULL means all ones.
 * eps must be finite and > 0.  Asynchronous on `stream` of the current device. */
int32_t moe_residual_rmsnorm(const float* h_src, const float* y, float* h_dst, const float* norm_weight,
                             float eps, uint16_t* x, int32_t tokens, int32_t hidden, void* stream);

enum moe_chain_flags {
  /* layers joined by the residual stream and RMSNorm (above); without it the layers run
   * one after another on inputs the caller wrote into x (a stack of independent calls) */
  MOE_CHAIN_RESIDUAL = 1
};

typedef struct moe_chain_desc {
  int32_t abi_version;              /* MOE_ABI_VERSION */
  int32_t n_layers;                 /* 1 .. 1024 */
  int32_t tokens;                   /* T per layer call, >= 1 */
  int32_t flags;                    /* MOE_CHAIN_RESIDUAL or 0 */
  float eps;                        /* RMSNorm epsilon (RESIDUAL; finite, > 0) */
  int32_t reserved;                 /* 0 */
  const moe_layer* const* layers;   /* host array [n_layers]: same hidden size and device */
  const float* const* norm_weight;  /* host array [n_layers] of device float32 [H] (an entry may
                                       be NULL: all ones), or NULL (all ones); RESIDUAL only */
  const float* h_in;                /* device float32 [T][H]: residual input h_0 (RESIDUAL; read only) */
  float* h_out;                     /* device float32 [T][H]: residual after the last layer, also
                                       the running residual (RESIDUAL; must not overlap h_in) */
  uint16_t* x;                      /* device bf16 [n_layers][T][H]: each layer's input (written
                                       when RESIDUAL, else read) */
  float* y;                         /* device float32 [n_layers][T][H]: each layer's output */
  const moe_route_out* routes;      /* host array [n_layers] (copied at create) or NULL: each
                                       layer's routing, as moe_forward's route argument */
  void* workspace;                  /* one workspace for every layer (sequential on one stream) */
  uint64_t workspace_bytes;         /* >= moe_workspace_bytes(layer, T) for every layer */
} moe_chain_desc;

typedef struct moe_chain moe_chain;

/* Record the whole chain -- for each layer the join step and moe_forward, and the final
 * residual add -- into a HIP graph, once, on a stream of the library's own (no work runs).
 * With RESIDUAL, T <= 16 and H <= 8192 the join runs inside the layer's routing launch, with
 * the same arithmetic as moe_residual_rmsnorm (same x and h bits); otherwise as its own kernel.
 * Every pointer is borrowed and baked into the graph: buffers, weights and layers must stay
 * alive and in place until moe_chain_destroy.  On failure *out is NULL and nothing leaks. */
int32_t moe_chain_create(const moe_chain_desc* desc, moe_chain** out);

/* Replay the recorded chain on `stream` (NULL = default stream): one graph launch.  With
 * RESIDUAL, h_in is only read, so replays with the same h_in give the same results bit for
 * bit.  Replays that overlap (other streams) race on the buffers and the workspace. */
int32_t moe_chain_run(const moe_chain* chain, void* stream);

/* Free the graph.  NULL is a no-op; the caller must have synchronised every replay. */
void moe_chain_destroy(moe_chain* chain);

/* ---- partial-residency expert bank --------------------------------------------------
 * For expert sets larger than the HBM set aside for them.  The pages' prefill MoE routes on
 * the device, then refills a transient per-layer VRAM expert bank route-aware, in groups the
 * size of its slots, from page-locked host slabs, with the lookups of group g+1 overlapping the
 * uploads of group g ("feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine", PR
 * #1055, "What it is", the Prefill MoE item; the decode tier keeps a VRAM-sized FP4 expert
 * mirror cache, refilled in place).  Here a bank is n_slots expert slots in HBM, each holding one
 * group's gate, up and down codes and scales in the kernel layout, filled from the layer's FP4
 * arrays, which live in page-locked host memory. */
typedef struct moe_bank moe_bank;

/* A bank for `layer`: a layer created by moe_layer_create whose six FP4 weight pointers are
 * page-locked host memory (hipHostMalloc) in the kernel layout ([G][...] as moe_pack_fp4 writes
 * it), with its router weights on the device and no FP8 shared expert.  Allocates n_slots
 * expert slots in HBM (n_slots >= 2 * group; one slot is the bytes of one group of all six
 * arrays), four copy streams (default priority), events and small page-locked tables; `group`
 * (>= 1) is the number of experts per refill group.  The bank borrows the layer, which must
 * outlive it.  On failure *out is NULL and nothing leaks. */
int32_t moe_bank_create(const moe_layer* layer, int32_t n_slots, int32_t group, moe_bank** out);

/* The layer's forward with its experts served from the bank.  Routing runs on `stream`; the
 * calling thread then waits for the routing counts (the refill is route-aware, so this call
 * blocks until routing is done), takes the groups with rows (shared expert included) resident
 * ones first, and splits them into refill groups of up to `group` experts.  The experts of
 * refill group i that are not resident are uploaded on the bank's copy streams, expert by
 * expert in turn (into free slots, least recently used ones, or slots of refill groups two or
 * more back, after their kernels);
 * the grouped-GEMM expert kernels of refill group i run on `stream` once its uploads are in,
 * while group i+1 uploads; the combine runs after the last group.  Slots keep their experts
 * between calls.  The result equals moe_forward on the same layer with MOE_PATH_GEMM and
 * resident weights, bit for bit.  Returns with the expert work enqueued on `stream`.  Calls on
 * one bank must not overlap; `workspace` is as for moe_forward. */
int32_t moe_bank_forward(moe_bank* bank, const uint16_t* x, int32_t tokens, float* y,
                         const moe_route_out* route, void* workspace, uint64_t workspace_bytes,
                         void* stream);

/* Counters since creation: [0] calls, [1] experts found resident, [2] experts uploaded,
 * [3] bytes uploaded, [4] refill groups run. */
int32_t moe_bank_stats(const moe_bank* bank, int64_t* out5);

/* Free the bank's slots, streams, events and tables (never the layer).  NULL is a no-op; the
 * caller must have synchronised the streams of its calls. */
void moe_bank_destroy(moe_bank* bank);

/* Static text for a status code. */
const char* moe_status_string(int32_t status);

/* Message of the calling thread's last failed call ("" if none). */
const char* moe_last_error(void);

/* ---- kernel timing (measurement support) ------------------------------------------
 * While enabled, every kernel the library launches is bracketed by a pair of HIP events
 * recorded on the stream it runs on.  moe_timing_read waits for those events and returns,
 * per kernel name, the launch count and summed duration since the last reset.  Process
 * wide; not meant to be toggled while other threads call the library. */
int32_t moe_timing_enable(int32_t on);
/* Number of distinct kernel names recorded; fills up to `cap` entries. names[i] points to
 * static strings. */
int32_t moe_timing_read(const char** names, int64_t* launches, double* total_ms, int32_t cap);
void moe_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP4_MOE_H */
