// Internal declarations shared by the HIP sources of the MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// ---- cross-lane reductions on DPP (no LDS round trips) ------------------------------
// quad_perm [1,0,3,2] and [2,3,0,1], then row_ror 4 and 8: every lane of a 16-lane row holds
// the row's result; the four row results are read from lanes 15, 31, 47, 63 and combined in a
// fixed order, so the outcome is the same on every lane and on every call.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x124>(v));
  v = max(v, dpp_u32<0x128>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 15), b = __builtin_amdgcn_readlane(v, 31);
  const uint32_t c = __builtin_amdgcn_readlane(v, 47), d = __builtin_amdgcn_readlane(v, 63);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x124>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));
  const float a = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 15));
  const float b = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 31));
  const float c = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 47));
  const float d = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
  return ((a + b) + c) + d;
}
// ---- cross-workgroup hand-off inside one kernel ---------------------------------------
// Values another workgroup reads in the same launch are written and read with agent-scope
// relaxed atomics (stores write through the XCD-local L2, loads miss it), the writer waits
// for its stores to complete before it bumps a counter, and the workgroup that brings the
// counter to its final value does the dependent work.  No device-scope fence is used: on
// gfx950 that writes back the whole L2 and costs far more than the data it publishes.
template <class V>
__device__ __forceinline__ void st_agent(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class V>
__device__ __forceinline__ V ld_agent(const V* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int32_t* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Cache-policy bits of buffer loads and stores: sc1 makes them coherent across the XCDs'
// L2 caches (the encoding agent-scope atomics use), for data another workgroup of the
// same launch produces or consumes.
constexpr int kSC1 = 16;
// Wait until this wave's stores (and loads) have completed.
__device__ __forceinline__ void wait_stores() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
}
__device__ __forceinline__ void reset_counter(int32_t* counter) {
  __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Read-only views in the constant address space: uniform loads through them become scalar
// loads (SGPRs), which is how a value shared by every lane of a wave is best fetched.
typedef const __attribute__((address_space(4))) uint32_t c_u32;
typedef const __attribute__((address_space(4))) float c_f32;

// Control area at the start of the workspace (int32 words).  Its size depends only on the
// layer's dims, so its place does not move with the batch size.  A fresh workspace is all
// zero, and every call leaves every word at zero again (a counter is reset by the workgroup
// that brings it to its final value).
struct CtrlLayout {
  static constexpr int kRoute = 0;  // router_kernel: arrival counter of its workgroups
  int words;
};
inline CtrlLayout ctrl_layout(int H, int E, int S, int I) {
  (void)H, (void)E, (void)S, (void)I;
  CtrlLayout c;
  c.words = 64;
  return c;
}

constexpr int kWave = 64;
constexpr int kChunk = 64;        // tokens per routing chunk (one bit per token in a 64-bit mask)
constexpr int kGemmBM = 64;       // grouped-GEMM rows per M-tile

// ---- exact FP8 (e4m3) term splits for the block-scaled MFMA ------------------------
// A 32-value block v is written as S * (t0 + t1/16 + t2/256 + ...), each t an e4m3 value, with
// S = 2^(s-127) a power of two chosen from the block's largest magnitude so that |v/S| < 256
// (e4m3 saturates at 448 and the converts round to nearest even).  Term i carries e8m0 scale
// s - 4i.  Each term keeps 4 significant bits of what the previous terms left, so two terms
// hold a bf16 value exactly and three terms hold 12 significant bits of an fp32 value
// (values below 2^-14 of the block maximum keep fewer).
__device__ __forceinline__ int fp8_block_scale(float amax) {
  if (!(amax > 0.f)) return 127;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  return max(e - 7, 9);
}
__device__ __forceinline__ float fp8_inv_scale(int s) { return __uint_as_float((uint32_t)(254 - s) << 23); }

// Four values -> one dword of e4m3 bytes (value i in byte i).
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}
// One value -> its e4m3 byte, and back.
__device__ __forceinline__ uint32_t fp8_of(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float f32_of_fp8(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }
// 0x7F (e4m3 NaN; OR-ing it into any byte gives a NaN byte) for an infinite or NaN value, else
// 0.  Non-finite activations stay non-finite through the FP8 terms, as they would in the
// float products they stand for (an e8m0 scale byte of 255 means +inf).
constexpr uint32_t kFp8NaN = 0x7Fu;
__device__ __forceinline__ uint32_t fp8_nan_mask(float v) { return fabsf(v) <= 3.402823466e38f ? 0u : kFp8NaN; }

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;


__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// More DPP controls for the helpers below (every lane of the wave active).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i within each half row
constexpr int kRowMirror = 0x140;      // lane i <-> 15 - i within each row
// max of v over the 16 lanes of this lane's row (every lane gets it)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kQuadXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kQuadXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kRowHalfMirror>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(dpp_u32<kRowMirror>(__float_as_uint(v))));
}

// Operands of v_mfma_scale_f32_16x16x128_f8f6f4 (probed lane layout, 16x16 output tile):
// * FP4 operand, lane (n, q) = (lane % 16, lane / 16): the 32 values of K block q of row/column
//   n, i.e. 16 bytes, plus that block's e8m0 scale.
// * FP8 operand, lane (m, q): bytes 16q..16q+15 and 64+16q..64+16q+15 of the 128-value K step
//   of row m; its scale is that of K block q of row m.
// * Result: lane l, element i -> row 4*(l/16) + i, column l % 16.
__device__ __forceinline__ i32x8 fp4_operand(const uint4& c) {
  return i32x8{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};  // FP4 reads the low 4 dwords
}
__device__ __forceinline__ i32x8 fp8_operand(const uint4& lo, const uint4& hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
// acc += A(fp8, scale sa) x B(fp4, scale sb)
__device__ __forceinline__ f32x4 mma_f8f4(const i32x8& a, const i32x8& b, f32x4 acc, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 4, 0, sa, 0, sb);
}
// acc += A(fp8, scale sa) x B(fp8 e4m3, scale byte 127 = 1.0): the FP8 shared expert, whose
// float32 128 x 128 block scales are applied to the product afterwards.  Both operands use the
// FP8 lane layout above.
__device__ __forceinline__ f32x4 mma_f8f8(const i32x8& a, const i32x8& b, f32x4 acc, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, 127);
}
// The same with B's scale taken from byte SELB of the register sb.
template <int SELB>
__device__ __forceinline__ f32x4 mma_f8f4_sb(const i32x8& a, const i32x8& b, f32x4 acc, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 4, 0, sa, SELB, sb);
}

// Token of grouped row r: routed rows carry t*k+j in perm; the shared expert's rows
// (r >= T*k) are the tokens in order.
__device__ __forceinline__ int row_token(const int32_t* perm, int r, int tk, int k) {
  return r < tk ? perm[r] / k : r - tk;
}

// Bytes of one matrix's scales in the kernel layout: [ceil(K/128)][ceil(N/64)][16][4][4].
// Byte (i, t, m, q, j) is the scale of row 64t + 16j + m, K block 4i + q (0 past the matrix),
// so lane (m, q) of a wave finds the scales of its four 16-row column tiles of one 128-value
// K step in one dword, and the 64 lanes' dwords are 256 contiguous bytes.
// Activation scale rows ([rows][kb_pad(K)] e8m0) are padded to whole 128-value K steps; the
// pad bytes hold 127 (a finite scale that only ever meets zero weights).
__host__ __device__ inline int kb_pad(int K) { return (K / 32 + 3) / 4 * 4; }
__host__ __device__ inline size_t scale_slab_bytes(int N, int K) {
  return (size_t)((K / 32 + 3) / 4) * (size_t)((N + 63) / 64) * 256;
}

struct Dims {
  int H, E, K, S, I, G;  // hidden, experts, top-k, shared, inter, groups = E + S
  bool fp8_shared;       // the shared expert (group E) is FP8 E4M3 with 128 x 128 block scales
  float routed_scale;    // multiplies every routed row's routing weight in the combine
};
constexpr int kFp8Block = 128;

// Device buffers of one call, carved from the workspace (and the caller's route buffers).
// Active-group slot of the decode kernels: one 16-byte load gives a workgroup its group, the
// group's rows and the number of active slots (slots past that count hold only the count).
struct alignas(16) GroupRec {
  int32_t group, row0, rows, nact;
};

struct CallBufs {
  float* logits;      // [T][E] scores (fused routing), or [slices][T][E] partial scores
  int32_t* idx;       // [T][k]
  float* w;           // [T][k]
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* perm;      // [T*k]
  float* row_w;       // [T*k] routing weight of grouped row r (= w[perm[r]])
  uint64_t* gmask;    // [C][E] per-chunk token masks
  int32_t* cbase;     // [C][E] rows of expert e in chunks before c
  int32_t* grp_row0;  // [G] first grouped row of group g
  int32_t* grp_rows;  // [G] rows of group g
  GroupRec* grec;     // [G] groups with rows, ascending, shared last; then count-only slots
  int32_t* info;      // [0] = active groups, [1] = GEMM M-tiles, [2] = routed GEMM M-tiles (the shared ones follow)
  int32_t* mt_group;  // [mt_bound]
  int32_t* mt_row0;   // [mt_bound]
  int32_t* ctrl;      // control words (zero between calls): [0] routing arrival counter
  void* h;            // h as FP8 terms [3 decode / 2 prefill][R][I] then e8m0 scales [R][kb_pad(I)]
  uint8_t* xq;        // x as 2 FP8 terms [2][T][H] then e8m0 scales [T][kb_pad(H)]
  float* staging;     // [T(k+S)][H] weighted expert outputs, slot-indexed
};

// ---- kernel timing hooks (api.hip) --------------------------------------------------
int timing_begin(const char* name, hipStream_t s);
void timing_end(int token, hipStream_t s);

// ---- launchers (return hipGetLastError of the launch) ---------------------------------
// Batches routed by the router kernel's last workgroup: one bit per token in a 64-bit mask,
// and every score of the batch held in that workgroup's LDS.
constexpr int kFusedMaxT = 64;
constexpr int kTailScores = 8192;
inline bool route_fused(const Dims& d, int T) { return T <= kFusedMaxT && T * d.E <= kTailScores; }
// Router GEMM of larger batches: the hidden axis is cut into router_slices(T, E) slices, one
// workgroup per (64-token tile, 64-expert tile, slice), so even a few token tiles fill the
// GPU; the slices' partial scores ([slices][T][E]) are added in slice order by the top-k.
constexpr int kRouterMaxSlices = 16;
inline int router_slices(const Dims& d, int T) {
  const int tiles = ((T + 63) / 64) * ((d.E + 63) / 64);
  int ks = (512 + tiles - 1) / tiles;
  ks = ks < 1 ? 1 : (ks > kRouterMaxSlices ? kRouterMaxSlices : ks);
  return ks < d.H / 32 ? ks : d.H / 32;
}
// The chained decode's join (h = h_src + y, x = bf16(RMSNorm(h) * gamma)) done by the routing
// launch of the next layer, for batches route_fused takes and at most kJoinMaxT tokens: every
// router workgroup normalises the rows itself (the same steps as the join kernel) and writes x;
// the last one writes h_dst.
struct JoinArgs {
  const float* h_src;  // residual before the join [T][H]
  const float* y;      // previous layer's output [T][H], or NULL (the first layer)
  float* h_dst;        // residual after the join (may equal h_src), or NULL
  const float* gamma;  // RMSNorm weight [H], or NULL (ones)
  float eps;
};
constexpr int kJoinMaxT = 16;
inline bool join_fused(const Dims& d, int T) { return route_fused(d, T) && T <= kJoinMaxT && d.H <= 8192; }

// Router scores (and, for batches route_fused takes, the whole routing in the same launch).
// quantize_x: also write the FP8 activation terms; mtiles: also the grouped GEMM's M-tile
// list; lean: the caller only runs the decode kernels and reads no routing output, so with
// at most kLeanMaxPicks picks only their tables are built.
constexpr int kLeanMaxPicks = 64;
// Byte ranges the routing launch reads ahead (one word per 128-byte line) once its workgroups
// have published their scores, so that the lines are in the memory-side cache when the expert
// kernels stream them: the always-active shared expert's weights.
struct Warm {
  const uint8_t* p[6];
  uint32_t bytes[6];
};
hipError_t launch_router_logits(const Dims& d, const uint16_t* x, const float* wr, const float* bias,
                                const CallBufs& b, int T, bool quantize_x, bool mtiles, bool lean, hipStream_t s,
                                const JoinArgs* join = nullptr, const Warm* warm = nullptr);
hipError_t launch_route_chunked(const Dims& d, const CallBufs& b, int T, hipStream_t s);

// Decode GEMV kernels (gemv.hip): gate/up + SwiGLU into h, then down + the combine into y.
// They read the routing tables and the FP8 activation terms earlier launches on the stream
// wrote.
// With d.fp8_shared each of these enqueues the FP4 kernel for the routed groups and then the
// FP8 kernel for the shared expert (whose down launch also does the combine, after every
// routed row is in staging).
hipError_t launch_gemv_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b, int T,
                              int max_act, hipStream_t s);
hipError_t launch_gemv_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, float* y, int T, int max_act,
                            hipStream_t s);
// slot_of (NULL: every group at its own index): group g's weights sit at index slot_of[g] of
// w's arrays; the M-tiles of groups with slot_of[g] < 0 are skipped (one expert-bank refill group
// per launch).  FP4 groups only.
hipError_t launch_gemm_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int mt_bound, hipStream_t s, const int32_t* slot_of = nullptr);
hipError_t launch_gemm_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int mt_bound,
                            hipStream_t s, const int32_t* slot_of = nullptr);
hipError_t launch_pack_fp8(const uint8_t* codes_in, uint8_t* codes_out, int groups, int N, int K, hipStream_t s);
// h_dst = h_src + y (y, h_dst may be NULL), x = bf16(RMSNorm(h) * gamma) (x may be NULL)
hipError_t launch_residual_rmsnorm(const float* h_src, const float* y, float* h_dst, const float* gamma, float eps,
                                   uint16_t* x, int T, int H, hipStream_t s);
hipError_t launch_pack(const uint8_t* codes_in, const uint8_t* scales_in, uint8_t* codes_out, uint8_t* scales_out,
                       int groups, int N, int K, hipStream_t s);
hipError_t launch_combine(const Dims& d, const CallBufs& b, float* y, int T, hipStream_t s);

}  // namespace moe
