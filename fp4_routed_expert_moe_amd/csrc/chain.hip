// The step between two MoE layers of a chained decode: the residual stream and the next
// layer's RMSNorm, with the normalised row rounded to bf16 as that layer's input.
//
//   h_dst = h_src + y                         (when y is given; fp32, one rounding per add)
//   x     = bf16( h * (1 / sqrt(mean(h^2) + eps)) * gamma )      (when x is given)
//
// The pages run the MoE stage once per layer in decode ("feat(v4/cuda): the CUDA tier wired into
// the DeepSeek V4 engine", PR #1055, "What it is") and leave the join between layers open; this
// is the plain pre-norm residual reading (attention and hyper-connection mixing are not on the
// MoE path).
//
// One workgroup per token row.  Rows up to 8192 values stay in registers between the residual
// add and the normalisation (one memory round trip); longer rows take two passes in which each
// thread owns the same float4 columns, so an in-place update (h_dst == h_src) reads back only
// what the thread itself wrote.  Tiny (T rows of H floats): at decode sizes the launch and one
// memory round trip, not the bytes, are its cost.
#include "common.h"

namespace moe {

namespace {

constexpr int kNormThreads = 256;

__device__ __forceinline__ uint32_t bf16_bits_rn(float v) {
  const uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN -> quiet NaN
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;         // nearest, ties to even (overflow -> inf)
}

constexpr int kNormRegs = 8;  // float4s per thread held in registers (rows up to 8192 values)

// Row sum over the workgroup: wave butterfly, then the four waves' sums in a fixed order.
__device__ __forceinline__ float row_sum(float ss) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) ss += __shfl_xor(ss, m, 64);
  __shared__ float part[kNormThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  return (part[0] + part[1]) + (part[2] + part[3]);
}

__device__ __forceinline__ uint2 bf16x4_rn(const float4& v, float inv, const float4& g) {
  const uint32_t b0 = bf16_bits_rn(v.x * inv * g.x), b1 = bf16_bits_rn(v.y * inv * g.y);
  const uint32_t b2 = bf16_bits_rn(v.z * inv * g.z), b3 = bf16_bits_rn(v.w * inv * g.w);
  return make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
}

// Rows of up to kNormRegs * 256 float4s: every load issued at once and the row kept in
// registers, so the whole step is one memory round trip.  The same arithmetic, in the same
// order, as the two-pass kernel below.
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_regs_kernel(const float* h_src,
                                                                             const float* __restrict__ y,
                                                                             float* h_dst,
                                                                             const float* __restrict__ gamma,
                                                                             uint16_t* __restrict__ x, float eps,
                                                                             int H) {
  const size_t row = (size_t)blockIdx.x * H;
  const float4* hs = reinterpret_cast<const float4*>(h_src + row);
  const float4* ys = y ? reinterpret_cast<const float4*>(y + row) : nullptr;
  float4* hd = h_dst ? reinterpret_cast<float4*>(h_dst + row) : nullptr;
  const int n4 = H >> 2;
  float4 v[kNormRegs], d[kNormRegs];
#pragma unroll
  for (int j = 0; j < kNormRegs; ++j) {
    const int i = threadIdx.x + j * kNormThreads;
    v[j] = i < n4 ? hs[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    d[j] = ys && i < n4 ? ys[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kNormRegs; ++j) {
    const int i = threadIdx.x + j * kNormThreads;
    if (i >= n4) break;
    if (ys) {
      v[j].x += d[j].x;
      v[j].y += d[j].y;
      v[j].z += d[j].z;
      v[j].w += d[j].w;
    }
    if (hd) hd[i] = v[j];
    ss = fmaf(v[j].x, v[j].x, ss);
    ss = fmaf(v[j].y, v[j].y, ss);
    ss = fmaf(v[j].z, v[j].z, ss);
    ss = fmaf(v[j].w, v[j].w, ss);
  }
  if (!x) return;
  const float inv = 1.0f / sqrtf(row_sum(ss) / (float)H + eps);
  const float4* gs = reinterpret_cast<const float4*>(gamma);
  uint2* xo = reinterpret_cast<uint2*>(x + row);
#pragma unroll
  for (int j = 0; j < kNormRegs; ++j) {
    const int i = threadIdx.x + j * kNormThreads;
    if (i >= n4) break;
    xo[i] = bf16x4_rn(v[j], inv, gs ? gs[i] : make_float4(1.f, 1.f, 1.f, 1.f));
  }
}

__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(const float* h_src,
                                                                        const float* __restrict__ y,
                                                                        float* h_dst,
                                                                        const float* __restrict__ gamma,
                                                                        uint16_t* __restrict__ x, float eps, int H) {
  const size_t row = (size_t)blockIdx.x * H;
  const float4* hs = reinterpret_cast<const float4*>(h_src + row);
  const float4* ys = y ? reinterpret_cast<const float4*>(y + row) : nullptr;
  float4* hd = h_dst ? reinterpret_cast<float4*>(h_dst + row) : nullptr;
  const int n4 = H >> 2;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += kNormThreads) {
    float4 v = hs[i];
    if (ys) {
      const float4 d = ys[i];
      v.x += d.x;
      v.y += d.y;
      v.z += d.z;
      v.w += d.w;
    }
    if (hd) hd[i] = v;
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  if (!x) return;
  const float inv = 1.0f / sqrtf(row_sum(ss) / (float)H + eps);
  const float4* gs = reinterpret_cast<const float4*>(gamma);
  uint2* xo = reinterpret_cast<uint2*>(x + row);
  for (int i = threadIdx.x; i < n4; i += kNormThreads) {
    float4 v;
    if (hd) {
      v = hd[i];  // this thread's own store of the first pass
    } else {
      v = hs[i];
      if (ys) {
        const float4 d = ys[i];
        v.x += d.x;
        v.y += d.y;
        v.z += d.z;
        v.w += d.w;
      }
    }
    xo[i] = bf16x4_rn(v, inv, gs ? gs[i] : make_float4(1.f, 1.f, 1.f, 1.f));
  }
}

}  // namespace

static_assert(kNormThreads == 256, "the row sum reduces four waves");

hipError_t launch_residual_rmsnorm(const float* h_src, const float* y, float* h_dst, const float* gamma, float eps,
                                   uint16_t* x, int T, int H, hipStream_t s) {
  const int tk = timing_begin("residual_rmsnorm", s);
  if ((H >> 2) <= kNormRegs * kNormThreads)
    residual_rmsnorm_regs_kernel<<<T, kNormThreads, 0, s>>>(h_src, y, h_dst, gamma, x, eps, H);
  else
    residual_rmsnorm_kernel<<<T, kNormThreads, 0, s>>>(h_src, y, h_dst, gamma, x, eps, H);
  timing_end(tk, s);
  return hipGetLastError();
}

}  // namespace moe
