// The chained decode's join between layers, one token row at a time:
//
//   h = h_src + y            (fp32, one rounding per add; y may be absent)
//   x = bf16( h * (1 / sqrt(mean(h^2) + eps)) * gamma )
//
// A row is handled by 256 threads (four waves): thread tid owns the float4s tid + 256 j,
// j < kJoinRegs, holds them in registers, and sums their squares in that order with FMAs; the
// four waves' sums meet through a wave butterfly and a fixed-order sum of the four.  Both the
// join kernel and the routing launch that does the join itself (chain.hip, route.hip) use
// these steps, so a row gives the same bits either way.
#pragma once
#include "common.h"

namespace moe {

constexpr int kJoinThreads = 256;  // threads per row
constexpr int kJoinRegs = 8;       // float4s per thread: rows up to 8192 values

__device__ __forceinline__ uint32_t bf16_bits_rn(float v) {
  const uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN -> quiet NaN
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;         // nearest, ties to even (overflow -> inf)
}

struct JoinRow {
  float4 v[kJoinRegs];
  float ss;  // this thread's sum of squares
};

// Thread tid's part of the row: loads (all at once), the residual add, the residual store
// (h_dst may be NULL) and the sum of squares.
__device__ __forceinline__ void join_load(JoinRow& r, const float* h_src, const float* __restrict__ y, float* h_dst,
                                          int H, int tid) {
  const float4* hs = reinterpret_cast<const float4*>(h_src);
  const float4* ys = reinterpret_cast<const float4*>(y);
  float4* hd = reinterpret_cast<float4*>(h_dst);
  const int n4 = H >> 2;
  float4 d[kJoinRegs];
#pragma unroll
  for (int j = 0; j < kJoinRegs; ++j) {
    const int i = tid + j * kJoinThreads;
    r.v[j] = i < n4 ? hs[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    d[j] = ys && i < n4 ? ys[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kJoinRegs; ++j) {
    const int i = tid + j * kJoinThreads;
    if (i >= n4) break;
    if (ys) {
      r.v[j].x += d[j].x;
      r.v[j].y += d[j].y;
      r.v[j].z += d[j].z;
      r.v[j].w += d[j].w;
    }
    if (hd) hd[i] = r.v[j];
    ss = fmaf(r.v[j].x, r.v[j].x, ss);
    ss = fmaf(r.v[j].y, r.v[j].y, ss);
    ss = fmaf(r.v[j].z, r.v[j].z, ss);
    ss = fmaf(r.v[j].w, r.v[j].w, ss);
  }
  r.ss = ss;
}

__device__ __forceinline__ float join_wave_sum(float ss) { return wave_sum_f32(ss); }

// 1 / sqrt(mean + eps) from the four waves' sums p[0..3] of a row.
__device__ __forceinline__ float join_inv(const float* p, int H, float eps) {
  return 1.0f / sqrtf(((p[0] + p[1]) + (p[2] + p[3])) / (float)H + eps);
}

__device__ __forceinline__ uint2 bf16x4_rn(const float4& v, float inv, const float4& g) {
  const uint32_t b0 = bf16_bits_rn(v.x * inv * g.x), b1 = bf16_bits_rn(v.y * inv * g.y);
  const uint32_t b2 = bf16_bits_rn(v.z * inv * g.z), b3 = bf16_bits_rn(v.w * inv * g.w);
  return make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
}

__device__ __forceinline__ void join_store_x(const JoinRow& r, float inv, const float* __restrict__ gamma,
                                             uint16_t* x, int H, int tid) {
  const float4* gs = reinterpret_cast<const float4*>(gamma);
  uint2* xo = reinterpret_cast<uint2*>(x);
  const int n4 = H >> 2;
#pragma unroll
  for (int j = 0; j < kJoinRegs; ++j) {
    const int i = tid + j * kJoinThreads;
    if (i >= n4) break;
    xo[i] = bf16x4_rn(r.v[j], inv, gs ? gs[i] : make_float4(1.f, 1.f, 1.f, 1.f));
  }
}

}  // namespace moe
