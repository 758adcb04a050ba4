// Decode path: expert-grouped FP4 GEMV.  Few rows per expert, so the work is bound by
// streaming the e2m1 nibbles and e8m0 scales from HBM once.
//
// "feat(dsv4): DeepSeek V4 Flash support -- CUDA/VRAM expert tiering ..." (PR #1031) makes a
// custom FP4 expert-grouped matvec the default GPU expert path, and "Add DeepSeek V4 Flash
// CPU inference with NVMe expert streaming" (PR #165, the NEON rows16 comment) computes one
// weight row per vector lane with the columns ascending, and pairs gate and up in one "dual"
// pass.  The gfx950 version keeps both ideas:
//
// * One lane owns one output row (gate and up rows n together, so SwiGLU stays in
//   registers); a workgroup owns 64 rows of one active group.  Weights are in the
//   block-interleaved kernel layout (pack.hip), so the 64 lanes' 16-byte loads of one block
//   are one contiguous KiB.
// * The reduction axis is split over the workgroup's 4 waves; each lane walks its row's
//   32-element blocks in ascending order, 16 code bytes per load, several blocks in flight.
// * The activations are the same for every lane, so they are read with scalar loads into
//   SGPRs and used directly as the shared operand of v_dot2 / v_fma.
// * e2m1 codes are converted with the gfx950 scaled converts, the e8m0 scale applied inside
//   the convert (exact: the scale is a power of two).
// * The 4 wave partials are added in a fixed order through LDS, so a token's result does not
//   depend on which other tokens share its expert.
#include "common.h"

namespace moe {

constexpr int kSplit = 4;     // waves per workgroup = slices of the reduction axis
constexpr int kGateTT = 4;    // tokens per pass, gate/up (bf16 activations: 16 SGPRs per block)
constexpr int kDownTT = 2;    // tokens per pass, down (fp32 activations: 32 SGPRs per block)
constexpr int kUnroll = 4;    // 32-element blocks in flight per lane

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// ------------------------------------------------------------------------------------
// gate/up:  h[row][n] = silu(x_t . Wg[n]) * (x_t . Wu[n])   (fp32 h)
// ------------------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void gateup_pass(const uint16_t* __restrict__ x, const uint8_t* __restrict__ gcr,
                                            const uint8_t* __restrict__ gsr, const uint8_t* __restrict__ ucr,
                                            const uint8_t* __restrict__ usr, const int32_t* __restrict__ perm,
                                            float* __restrict__ hout, float (*red)[2 * kGateTT][64], int r_first,
                                            int tk, int k, int H, int I, int n, bool nok, int kb0, int kb1) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  c_u32* xrow[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int t = row_token(perm, r_first + tt, tk, k);
    xrow[tt] = (c_u32*)(x + (size_t)t * H);
  }
  float ag[NT], au[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) ag[tt] = au[tt] = 0.f;
  for (int kb = kb0; kb < kb1; kb += kUnroll) {
    uint4 cg[kUnroll], cu[kUnroll];
    float sg[kUnroll], su[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int b = min(kb + u, kb1 - 1);  // tail: re-read the last block, contribution skipped
      cg[u] = *reinterpret_cast<const uint4*>(gcr + (size_t)b * I * 16);
      cu[u] = *reinterpret_cast<const uint4*>(ucr + (size_t)b * I * 16);
      sg[u] = e8m0_to_f32(gsr[(size_t)b * I]);
      su[u] = e8m0_to_f32(usr[(size_t)b * I]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (kb + u < kb1) {
        const uint32_t cgw[4] = {cg[u].x, cg[u].y, cg[u].z, cg[u].w};
        const uint32_t cuw[4] = {cu[u].x, cu[u].y, cu[u].z, cu[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x2 wg[4], wu[4];
          fp4x8_to_bf16(cgw[q], sg[u], wg);
          fp4x8_to_bf16(cuw[q], su[u], wu);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            c_u32* xp = xrow[tt] + (size_t)(kb + u) * 16 + 4 * q;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const bf16x2 xv = as_bf16x2(xp[s]);
              ag[tt] = __builtin_amdgcn_fdot2_f32_bf16(wg[s], xv, ag[tt], false);
              au[tt] = __builtin_amdgcn_fdot2_f32_bf16(wu[s], xv, au[tt], false);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    red[wave][2 * tt][lane] = ag[tt];
    red[wave][2 * tt + 1][lane] = au[tt];
  }
  __syncthreads();
  if (wave == 0 && nok) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      float g = red[0][2 * tt][lane], u = red[0][2 * tt + 1][lane];
#pragma unroll
      for (int w = 1; w < kSplit; ++w) {
        g += red[w][2 * tt][lane];
        u += red[w][2 * tt + 1][lane];
      }
      hout[(size_t)(r_first + tt) * I + n] = silu_f(g) * u;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void gemv_gateup_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ gc, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ uc, const uint8_t* __restrict__ us, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ act, const int32_t* __restrict__ info, const int32_t* __restrict__ grp_row0,
    const int32_t* __restrict__ grp_rows, float* __restrict__ hout, int T, int k, int H, int I) {
  __shared__ float red[kSplit][2 * kGateTT][64];
  if ((int)blockIdx.y >= info[0]) return;
  const int g = act[blockIdx.y];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  // readfirstlane: the wave index is uniform, and the compiler must know it for scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool nok = n < I;
  const int KB = H >> 5;
  const int kb0 = wave * KB / kSplit, kb1 = (wave + 1) * KB / kSplit;
  // kernel layout: block kb of row n of group g at ((g*KB + kb)*I + n) 16-byte chunks
  const size_t col = (size_t)g * KB * I + (nok ? n : I - 1);
  const uint8_t* gcr = gc + col * 16;
  const uint8_t* ucr = uc + col * 16;
  const uint8_t* gsr = gs + col;
  const uint8_t* usr = us + col;
  const int tk = T * k;
  for (int c0 = 0; c0 < rows; c0 += kGateTT) {
    switch (min(kGateTT, rows - c0)) {
      case 1: gateup_pass<1>(x, gcr, gsr, ucr, usr, perm, hout, red, row0 + c0, tk, k, H, I, n, nok, kb0, kb1); break;
      case 2: gateup_pass<2>(x, gcr, gsr, ucr, usr, perm, hout, red, row0 + c0, tk, k, H, I, n, nok, kb0, kb1); break;
      case 3: gateup_pass<3>(x, gcr, gsr, ucr, usr, perm, hout, red, row0 + c0, tk, k, H, I, n, nok, kb0, kb1); break;
      default: gateup_pass<4>(x, gcr, gsr, ucr, usr, perm, hout, red, row0 + c0, tk, k, H, I, n, nok, kb0, kb1); break;
    }
  }
}

// ------------------------------------------------------------------------------------
// down:  staging[slot(r)][n] = weight(r) * (h_r . Wd[n])    (fp32 h, fp32 FMA)
// ------------------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void down_pass(const float* __restrict__ hin, const uint8_t* __restrict__ dcr,
                                          const uint8_t* __restrict__ dsr, const int32_t* __restrict__ perm,
                                          const float* __restrict__ wts, float* __restrict__ staging,
                                          float (*red)[kDownTT][64], int r_first, int tk, int H, int I, int n,
                                          bool nok, int kb0, int kb1) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float a[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) a[tt] = 0.f;
  for (int kb = kb0; kb < kb1; kb += kUnroll) {
    uint4 cd[kUnroll];
    float sd[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int b = min(kb + u, kb1 - 1);
      cd[u] = *reinterpret_cast<const uint4*>(dcr + (size_t)b * H * 16);
      sd[u] = e8m0_to_f32(dsr[(size_t)b * H]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (kb + u < kb1) {
        const uint32_t cw[4] = {cd[u].x, cd[u].y, cd[u].z, cd[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x2 wv[4];
          fp4x8_to_f32(cw[q], sd[u], wv);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            c_f32* hp = (c_f32*)(hin + (size_t)(r_first + tt) * I + (size_t)(kb + u) * 32 + 8 * q);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              a[tt] = fmaf(wv[s].x, hp[2 * s], a[tt]);
              a[tt] = fmaf(wv[s].y, hp[2 * s + 1], a[tt]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) red[wave][tt][lane] = a[tt];
  __syncthreads();
  if (wave == 0 && nok) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      float s = red[0][tt][lane];
#pragma unroll
      for (int w = 1; w < kSplit; ++w) s += red[w][tt][lane];
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
  __shared__ float red[kSplit][kDownTT][64];
  if ((int)blockIdx.y >= info[0]) return;
  const int g = act[blockIdx.y];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  // readfirstlane: the wave index is uniform, and the compiler must know it for scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = blockIdx.x * 64 + lane;
  const bool nok = n < H;
  const int KB = I >> 5;
  const int kb0 = wave * KB / kSplit, kb1 = (wave + 1) * KB / kSplit;
  const size_t col = (size_t)g * KB * H + (nok ? n : H - 1);
  const uint8_t* dcr = dc + col * 16;
  const uint8_t* dsr = ds + col;
  const int tk = T * k;
  for (int c0 = 0; c0 < rows; c0 += kDownTT) {
    if (rows - c0 >= 2)
      down_pass<2>(hin, dcr, dsr, perm, wts, staging, red, row0 + c0, tk, H, I, n, nok, kb0, kb1);
    else
      down_pass<1>(hin, dcr, dsr, perm, wts, staging, red, row0 + c0, tk, H, I, n, nok, kb0, kb1);
  }
}

// ------------------------------------------------------------------------------------
hipError_t launch_gemv_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int max_act, hipStream_t s) {
  dim3 grid((d.I + 63) / 64, max_act);
  const int tk = timing_begin("gemv_gateup", s);
  gemv_gateup_kernel<<<grid, 64 * kSplit, 0, s>>>(x, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, b.perm,
                                                  b.act, b.info, b.grp_row0, b.grp_rows, static_cast<float*>(b.h),
                                                  T, d.K, d.H, d.I);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int max_act,
                            hipStream_t s) {
  dim3 grid((d.H + 63) / 64, max_act);
  const int tk = timing_begin("gemv_down", s);
  gemv_down_kernel<<<grid, 64 * kSplit, 0, s>>>(static_cast<const float*>(b.h), w.down_codes, w.down_scales, b.perm,
                                                b.w, b.act, b.info, b.grp_row0, b.grp_rows, b.staging, T, d.K, d.H,
                                                d.I);
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
