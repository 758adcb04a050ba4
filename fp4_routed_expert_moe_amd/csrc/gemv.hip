// Decode path: expert-grouped FP4 GEMV.  Few rows per expert, so the work is bound by
// streaming the e2m1 nibbles and e8m0 scales from HBM once.
//
// "feat(dsv4): DeepSeek V4 Flash support -- CUDA/VRAM expert tiering ..." (PR #1031) makes a
// custom FP4 expert-grouped matvec the default GPU expert path, and "Add DeepSeek V4 Flash
// CPU inference with NVMe expert streaming" (PR #165, the NEON rows16 comment) pairs gate
// and up in one "dual" pass.  Here one workgroup owns a tile of output rows of one active
// group: gate and up rows are read together so SwiGLU happens in registers.
//
// Mapping: thread (rsub, b) owns 32-element block b of the reduction axis for the rows
// n = n_base + rsub + rpi*i.  Each thread loads 16 contiguous code bytes per row (a wave
// reads 1 KiB contiguous per row), dequantises in registers with the gfx950 FP4 converts,
// and keeps its slice of the activations in registers across all rows.  The e8m0 scale is
// a power of two, so the 32-element partial sum is scaled once (exact).  Partial sums over
// blocks are reduced through LDS.
#include "common.h"

namespace moe {

constexpr int kGemvRI = 4;   // row iterations per workgroup
constexpr int kGateTT = 4;   // tokens per pass, gate/up
constexpr int kDownTT = 2;   // tokens per pass, down (fp32 activations in registers)

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Threads per reduction task (a power of two <= 64) so that tasks * P <= 256.
__device__ __forceinline__ int reduce_lanes(int tasks) {
  int p = 1;
  while (p < 64 && p * 2 * tasks <= 256) p <<= 1;
  return p;
}

// ------------------------------------------------------------------------------------
// gate/up:  h[row][n] = silu(x_t . Wg[n]) * (x_t . Wu[n])   (fp32 h)
// ------------------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void gateup_pass(const uint16_t* __restrict__ x, const uint8_t* __restrict__ gc,
                                            const uint8_t* __restrict__ gs, const uint8_t* __restrict__ uc,
                                            const uint8_t* __restrict__ us, const int32_t* __restrict__ perm,
                                            float* __restrict__ hout, float* red, int r_first, int tk, int k,
                                            int H, int I, size_t grow, int n_base, int rpi, int KB, int rsub,
                                            int b, bool on) {
  const int tid = threadIdx.x;
  uint4 xr[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int t = row_token(perm, r_first + tt, tk, k);
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * H + b * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) xr[tt][q] = on ? src[q] : make_uint4(0, 0, 0, 0);
  }
  uint4 cg[kGemvRI], cu[kGemvRI];
  uint32_t sg[kGemvRI], su[kGemvRI];
#pragma unroll
  for (int i = 0; i < kGemvRI; ++i) {
    const int n = n_base + rsub + rpi * i;
    if (on && n < I) {
      const size_t row = grow + n;
      cg[i] = *reinterpret_cast<const uint4*>(gc + row * (H >> 1) + b * 16);
      cu[i] = *reinterpret_cast<const uint4*>(uc + row * (H >> 1) + b * 16);
      sg[i] = gs[row * KB + b];
      su[i] = us[row * KB + b];
    } else {
      cg[i] = cu[i] = make_uint4(0, 0, 0, 0);
      sg[i] = su[i] = 0;
    }
  }
#pragma unroll
  for (int i = 0; i < kGemvRI; ++i) {
    float ag[NT], au[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) ag[tt] = au[tt] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x2 wg[4], wu[4];
      fp4x8_to_bf16(u4get(cg[i], q), 1.0f, wg);
      fp4x8_to_bf16(u4get(cu[i], q), 1.0f, wu);
#pragma unroll
      for (int sel = 0; sel < 4; ++sel) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const bf16x2 xp = as_bf16x2(u4get(xr[tt][q], sel));
          ag[tt] = __builtin_amdgcn_fdot2_f32_bf16(wg[sel], xp, ag[tt], false);
          au[tt] = __builtin_amdgcn_fdot2_f32_bf16(wu[sel], xp, au[tt], false);
        }
      }
    }
    const float scg = e8m0_to_f32(sg[i]), scu = e8m0_to_f32(su[i]);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      red[((i * NT + tt) * 2 + 0) * 256 + tid] = ag[tt] * scg;
      red[((i * NT + tt) * 2 + 1) * 256 + tid] = au[tt] * scu;
    }
  }
  __syncthreads();
  const int tasks = kGemvRI * rpi * NT;
  const int P = reduce_lanes(tasks);
  for (int base = 0; base < tasks * P; base += 256) {
    const int id = base + tid;
    const int task = id / P, p = id - (id / P) * P;
    const bool ok = task < tasks;
    float s_g = 0.f, s_u = 0.f;
    int n = 0, tt = 0;
    if (ok) {
      tt = task % NT;
      const int r2 = task / NT;
      const int rs = r2 % rpi, i = r2 / rpi;
      n = n_base + rs + rpi * i;
      const float* rg = red + ((i * NT + tt) * 2) * 256 + rs * KB;
      for (int bb = p; bb < KB; bb += P) {
        s_g += rg[bb];
        s_u += rg[256 + bb];
      }
    }
    for (int m = 1; m < P; m <<= 1) {
      s_g += __shfl_xor(s_g, m, 64);
      s_u += __shfl_xor(s_u, m, 64);
    }
    if (ok && p == 0 && n < I) hout[(size_t)(r_first + tt) * I + n] = silu_f(s_g) * s_u;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void gemv_gateup_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ gc, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ uc, const uint8_t* __restrict__ us, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ act, const int32_t* __restrict__ info, const int32_t* __restrict__ grp_row0,
    const int32_t* __restrict__ grp_rows, float* __restrict__ hout, int T, int k, int H, int I) {
  __shared__ float red[kGemvRI * kGateTT * 2 * 256];
  if ((int)blockIdx.y >= info[0]) return;
  const int g = act[blockIdx.y];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  const int KB = H >> 5;
  const int rpi = 256 / KB;
  const int tid = threadIdx.x;
  const int rsub = tid / KB, b = tid - rsub * KB;
  const bool on = rsub < rpi;
  const int n_base = blockIdx.x * rpi * kGemvRI;
  const int tk = T * k;
  const size_t grow = (size_t)g * I;
  for (int c0 = 0; c0 < rows; c0 += kGateTT) {
    const int nt = min(kGateTT, rows - c0);
    switch (nt) {
      case 1: gateup_pass<1>(x, gc, gs, uc, us, perm, hout, red, row0 + c0, tk, k, H, I, grow, n_base, rpi, KB, rsub, b, on); break;
      case 2: gateup_pass<2>(x, gc, gs, uc, us, perm, hout, red, row0 + c0, tk, k, H, I, grow, n_base, rpi, KB, rsub, b, on); break;
      case 3: gateup_pass<3>(x, gc, gs, uc, us, perm, hout, red, row0 + c0, tk, k, H, I, grow, n_base, rpi, KB, rsub, b, on); break;
      default: gateup_pass<4>(x, gc, gs, uc, us, perm, hout, red, row0 + c0, tk, k, H, I, grow, n_base, rpi, KB, rsub, b, on); break;
    }
  }
}

// ------------------------------------------------------------------------------------
// down:  staging[slot(r)][n] = weight(r) * (h_r . Wd[n])    (fp32 h, fp32 FMA)
// ------------------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void down_pass(const float* __restrict__ hin, const uint8_t* __restrict__ dc,
                                          const uint8_t* __restrict__ ds, const int32_t* __restrict__ perm,
                                          const float* __restrict__ wts, float* __restrict__ staging, float* red,
                                          int r_first, int tk, int H, int I, size_t grow, int n_base, int rpi,
                                          int KB, int rsub, int b, bool on) {
  const int tid = threadIdx.x;
  float4 xr[NT][8];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const float4* src = reinterpret_cast<const float4*>(hin + (size_t)(r_first + tt) * I + b * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) xr[tt][q] = on ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  uint4 cd[kGemvRI];
  uint32_t sd[kGemvRI];
#pragma unroll
  for (int i = 0; i < kGemvRI; ++i) {
    const int n = n_base + rsub + rpi * i;
    if (on && n < H) {
      const size_t row = grow + n;
      cd[i] = *reinterpret_cast<const uint4*>(dc + row * (I >> 1) + b * 16);
      sd[i] = ds[row * KB + b];
    } else {
      cd[i] = make_uint4(0, 0, 0, 0);
      sd[i] = 0;
    }
  }
#pragma unroll
  for (int i = 0; i < kGemvRI; ++i) {
    float a[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) a[tt] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x2 wq[4];
      fp4x8_to_f32(u4get(cd[i], q), 1.0f, wq);
#pragma unroll
      for (int sel = 0; sel < 4; ++sel) {
        const f32x2 wv = wq[sel];
        // elements 8q + 2sel and 8q + 2sel + 1
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const float4 xv = xr[tt][2 * q + (sel >> 1)];
          const float x0 = (sel & 1) ? xv.z : xv.x;
          const float x1 = (sel & 1) ? xv.w : xv.y;
          a[tt] = fmaf(wv.x, x0, a[tt]);
          a[tt] = fmaf(wv.y, x1, a[tt]);
        }
      }
    }
    const float sc = e8m0_to_f32(sd[i]);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) red[(i * NT + tt) * 256 + tid] = a[tt] * sc;
  }
  __syncthreads();
  const int tasks = kGemvRI * rpi * NT;
  const int P = reduce_lanes(tasks);
  for (int base = 0; base < tasks * P; base += 256) {
    const int id = base + tid;
    const int task = id / P, p = id - (id / P) * P;
    const bool ok = task < tasks;
    float s = 0.f;
    int n = 0, tt = 0;
    if (ok) {
      tt = task % NT;
      const int r2 = task / NT;
      const int rs = r2 % rpi, i = r2 / rpi;
      n = n_base + rs + rpi * i;
      const float* rr = red + (i * NT + tt) * 256 + rs * KB;
      for (int bb = p; bb < KB; bb += P) s += rr[bb];
    }
    for (int m = 1; m < P; m <<= 1) s += __shfl_xor(s, m, 64);
    if (ok && p == 0 && n < H) {
      const int r = r_first + tt;
      const int slot = r < tk ? perm[r] : r;
      const float wt = r < tk ? wts[slot] : 1.0f;
      staging[(size_t)slot * H + n] = s * wt;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void gemv_down_kernel(
    const float* __restrict__ hin, const uint8_t* __restrict__ dc, const uint8_t* __restrict__ ds,
    const int32_t* __restrict__ perm, const float* __restrict__ wts, const int32_t* __restrict__ act,
    const int32_t* __restrict__ info, const int32_t* __restrict__ grp_row0, const int32_t* __restrict__ grp_rows,
    float* __restrict__ staging, int T, int k, int H, int I) {
  __shared__ float red[kGemvRI * kDownTT * 256];
  if ((int)blockIdx.y >= info[0]) return;
  const int g = act[blockIdx.y];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  const int KB = I >> 5;
  const int rpi = 256 / KB;
  const int tid = threadIdx.x;
  const int rsub = tid / KB, b = tid - rsub * KB;
  const bool on = rsub < rpi;
  const int n_base = blockIdx.x * rpi * kGemvRI;
  const int tk = T * k;
  const size_t grow = (size_t)g * H;
  for (int c0 = 0; c0 < rows; c0 += kDownTT) {
    if (rows - c0 >= 2)
      down_pass<2>(hin, dc, ds, perm, wts, staging, red, row0 + c0, tk, H, I, grow, n_base, rpi, KB, rsub, b, on);
    else
      down_pass<1>(hin, dc, ds, perm, wts, staging, red, row0 + c0, tk, H, I, grow, n_base, rpi, KB, rsub, b, on);
  }
}

// ------------------------------------------------------------------------------------
hipError_t launch_gemv_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int max_act, hipStream_t s) {
  const int rpi = 256 / (d.H >> 5);
  const int nr = rpi * kGemvRI;
  dim3 grid((d.I + nr - 1) / nr, max_act);
  const int tk = timing_begin("gemv_gateup", s);
  gemv_gateup_kernel<<<grid, 256, 0, s>>>(x, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, b.perm, b.act,
                                          b.info, b.grp_row0, b.grp_rows, static_cast<float*>(b.h), T, d.K, d.H,
                                          d.I);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int max_act,
                            hipStream_t s) {
  const int rpi = 256 / (d.I >> 5);
  const int nr = rpi * kGemvRI;
  dim3 grid((d.H + nr - 1) / nr, max_act);
  const int tk = timing_begin("gemv_down", s);
  gemv_down_kernel<<<grid, 256, 0, s>>>(static_cast<const float*>(b.h), w.down_codes, w.down_scales, b.perm, b.w,
                                        b.act, b.info, b.grp_row0, b.grp_rows, b.staging, T, d.K, d.H, d.I);
  timing_end(tk, s);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// y[t] = staging[shared slot of t] + sum_j staging[t*k + j]
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ st, float* __restrict__ y, int T,
                                                      int H, int k, int S) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (S) acc = *reinterpret_cast<const float4*>(st + ((size_t)T * k + t) * H + c);
  for (int j = 0; j < k; ++j) {
    const float4 v = *reinterpret_cast<const float4*>(st + ((size_t)t * k + j) * H + c);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(y + (size_t)t * H + c) = acc;
}

hipError_t launch_combine(const Dims& d, const CallBufs& b, float* y, int T, hipStream_t s) {
  dim3 grid((d.H / 4 + 255) / 256, T);
  const int tk = timing_begin("combine", s);
  combine_kernel<<<grid, 256, 0, s>>>(b.staging, y, T, d.H, d.K, d.S);
  timing_end(tk, s);
  return hipGetLastError();
}

}  // namespace moe
