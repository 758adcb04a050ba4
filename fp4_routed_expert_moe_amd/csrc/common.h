// Internal declarations shared by the HIP sources of the MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Read-only views in the constant address space: uniform loads through them become scalar
// loads (SGPRs), which is how a value shared by every lane of a wave is best fetched.
typedef const __attribute__((address_space(4))) uint32_t c_u32;
typedef const __attribute__((address_space(4))) float c_f32;

constexpr int kWave = 64;
constexpr int kChunk = 64;        // tokens per routing chunk (one bit per token in a 64-bit mask)
constexpr int kGemmBM = 64;       // grouped-GEMM rows per M-tile
constexpr int kGemmBN = 64;       // grouped-GEMM output columns per workgroup

// e8m0 scale byte -> float32 with bit pattern s << 23 (s = 0 gives +0, s = 255 gives +inf).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

// Eight e2m1 codes (one dword; byte q holds elements 2q and 2q+1) -> four bf16 pairs / four
// fp32 pairs, each value multiplied by `scale` by the gfx950 scaled FP4 converts.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t v, float scale, bf16x2 out[4]) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
}
__device__ __forceinline__ void fp4x8_to_f32(uint32_t v, float scale, f32x2 out[4]) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, scale, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, scale, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, scale, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, scale, 3);
}

// Eight e2m1 codes -> one bf16x8 MFMA operand (value i from nibble i), times `scale`.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t v, float scale) {
  bf16x2 p[4];
  fp4x8_to_bf16(v, scale, p);
  bf16x8 r;
  r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
  r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
  return r;
}

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

typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Token of grouped row r: routed rows carry t*k+j in perm; the shared expert's rows
// (r >= T*k) are the tokens in order.
__device__ __forceinline__ int row_token(const int32_t* perm, int r, int tk, int k) {
  return r < tk ? perm[r] / k : r - tk;
}

struct Dims {
  int H, E, K, S, I, G;  // hidden, experts, top-k, shared, inter, groups = E + S
};

// Device buffers of one call, carved from the workspace (and the caller's route buffers).
struct CallBufs {
  float* logits;      // [T][E]
  int32_t* idx;       // [T][k]
  float* w;           // [T][k]
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* perm;      // [T*k]
  uint64_t* gmask;    // [C][E] per-chunk token masks
  int32_t* cbase;     // [C][E] rows of expert e in chunks before c
  int32_t* grp_row0;  // [G] first grouped row of group g
  int32_t* grp_rows;  // [G] rows of group g
  int32_t* act;       // [G] groups with rows, ascending, shared last
  int32_t* info;      // [0] = active groups, [1] = GEMM M-tiles
  int32_t* mt_group;  // [mt_bound]
  int32_t* mt_row0;   // [mt_bound]
  void* h;            // GEMV path: h as FP8 terms + scales (see gemv.hip); GEMM path: bf16 [T(k+S)][I]
  uint8_t* xq;        // GEMV path: x as 2 FP8 terms [2][T][H] then e8m0 scales [T][H/32]
  float* staging;     // [T(k+S)][H] weighted expert outputs, slot-indexed
};

// ---- kernel timing hooks (api.hip) --------------------------------------------------
int timing_begin(const char* name, hipStream_t s);
void timing_end(int token, hipStream_t s);

// ---- launchers (return hipGetLastError of the launch) ---------------------------------
hipError_t launch_router_logits(const Dims& d, const uint16_t* x, const float* wr, const float* bias,
                                float* logits, int T, uint8_t* xq, hipStream_t s);
hipError_t launch_route_small(const Dims& d, const CallBufs& b, int T, hipStream_t s);
hipError_t launch_route_chunked(const Dims& d, const CallBufs& b, int T, hipStream_t s);

hipError_t launch_gemv_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int max_act, hipStream_t s);
hipError_t launch_gemv_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int max_act,
                            hipStream_t s);
hipError_t launch_gemm_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int mt_bound, hipStream_t s);
hipError_t launch_gemm_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int mt_bound,
                            hipStream_t s);
hipError_t launch_pack(const uint8_t* codes_in, const uint8_t* scales_in, uint8_t* codes_out, uint8_t* scales_out,
                       int groups, int N, int K, hipStream_t s);
hipError_t launch_combine(const Dims& d, const CallBufs& b, float* y, int T, hipStream_t s);

}  // namespace moe
