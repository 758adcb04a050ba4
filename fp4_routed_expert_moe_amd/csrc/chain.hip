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
#include "join_dev.h"

namespace moe {

namespace {

constexpr int kNormThreads = kJoinThreads;
constexpr int kNormRegs = kJoinRegs;  // float4s per thread held in registers (rows up to 8192 values)

// Row sum over the workgroup: wave butterfly, then the four waves' sums in a fixed order.
__device__ __forceinline__ float row_sum(float ss) {
  ss = join_wave_sum(ss);
  __shared__ float part[kNormThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  return (part[0] + part[1]) + (part[2] + part[3]);
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
  JoinRow r;
  join_load(r, h_src + row, y ? y + row : nullptr, h_dst ? h_dst + row : nullptr, H, threadIdx.x);
  if (!x) return;
  __shared__ float part[kNormThreads / 64];
  const float ss = join_wave_sum(r.ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  join_store_x(r, join_inv(part, H, eps), gamma, x + row, H, threadIdx.x);
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
