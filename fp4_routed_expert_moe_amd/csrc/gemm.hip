// Prefill path: expert-grouped GEMM over the sorted token rows on bf16 MFMA.
//
// "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine" (PR #1055, "What it is",
// prefill MoE) runs expert-grouped GEMM rows after routing on the device.  Here each
// workgroup takes one M-tile (64 grouped rows of one group, listed on the device by the
// routing scan) and 64 output columns; its four waves each own 16 columns and all 64 rows.
//
// * Activation rows (gathered by token for gate/up, contiguous h rows for down) are staged
//   through LDS and shared by the four waves.
// * Weights never touch LDS: the 16x16x32 bf16 MFMA's B operand for one lane is 8
//   consecutive K values of one weight row, i.e. 4 bytes of e2m1 codes plus that row's e8m0
//   scale, so each lane loads one dword and converts it with the gfx950 scaled FP4->bf16
//   converts.  In the block-interleaved kernel layout (pack.hip) a wave's 64 dwords are 256
//   contiguous bytes.  Every dequantised product is exact (e2m1 * 2^(s-127) has 2
//   significant bits).
// * Epilogues: SwiGLU into bf16 h (gate/up); weight * y into the slot-indexed staging rows
//   (down).
#include "common.h"

namespace moe {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 64, LDA = BK + 8;  // LDS row pitch in bf16

__device__ __forceinline__ float silu_g(float g) { return g / (1.0f + expf(-g)); }

// 8 consecutive K values (k % 8 == 0) of one weight row as scaled bf16.  codes_col/scales_col
// point at block 0 of the row in the kernel layout; block kb is N chunks further.
__device__ __forceinline__ bf16x8 load_b_frag(const uint8_t* __restrict__ codes_col,
                                              const uint8_t* __restrict__ scales_col, size_t N, int k) {
  const size_t kb = (size_t)(k >> 5);
  const uint32_t c = *reinterpret_cast<const uint32_t*>(codes_col + kb * N * 16 + ((k & 31) >> 1));
  const float s = e8m0_to_f32(scales_col[kb * N]);
  return fp4x8_to_bf16x8(c, s);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ------------------------------------------------------------------------------------
// gate/up: h[row][n] = bf16( silu(x_t . Wg[n]) * (x_t . Wu[n]) )
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_gateup_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ gc, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ uc, const uint8_t* __restrict__ us, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ info, const int32_t* __restrict__ mt_group, const int32_t* __restrict__ mt_row0,
    const int32_t* __restrict__ grp_row0, const int32_t* __restrict__ grp_rows, uint16_t* __restrict__ hout,
    int T, int k, int H, int I) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
  const int mt = blockIdx.x;
  if (mt >= info[1]) return;
  const int g = mt_group[mt], m0 = mt_row0[mt];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  const int tk = T * k;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ncol = blockIdx.y * BN + wave * 16 + (lane & 15);
  const bool col_ok = ncol < I;
  const size_t col = (size_t)g * (H >> 5) * I + (col_ok ? ncol : I - 1);
  const uint8_t* gcr = gc + col * 16;
  const uint8_t* gsr = gs + col;
  const uint8_t* ucr = uc + col * 16;
  const uint8_t* usr = us + col;
  // activation loader: 64 rows x 4 segments of 16 bf16
  const int arow = tid >> 2, aseg = tid & 3;
  const bool a_ok = m0 + arow < rows;
  const int atok = a_ok ? row_token(perm, row0 + m0 + arow, tk, k) : 0;
  const uint16_t* asrc = x + (size_t)atok * H + aseg * 16;
  const int kq = (lane >> 4) * 8;
  f32x4 accg[4], accu[4];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) accg[ms] = accu[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < H; k0 += BK) {
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (a_ok && k0 + aseg * 16 < H) {
      v0 = *reinterpret_cast<const uint4*>(asrc + k0);
      v1 = *reinterpret_cast<const uint4*>(asrc + k0 + 8);
    }
    __syncthreads();
    *reinterpret_cast<uint4*>(&As[arow * LDA + aseg * 16]) = v0;
    *reinterpret_cast<uint4*>(&As[arow * LDA + aseg * 16 + 8]) = v1;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      if (k0 + kk < H) {
        const bf16x8 bg = load_b_frag(gcr, gsr, I, k0 + kk + kq);
        const bf16x8 bu = load_b_frag(ucr, usr, I, k0 + kk + kq);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[(ms * 16 + (lane & 15)) * LDA + kk + kq]);
          accg[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bg, accg[ms], 0, 0, 0);
          accu[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bu, accu[ms], 0, 0, 0);
        }
      }
    }
  }
  if (!col_ok) return;
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + ms * 16 + (lane >> 4) * 4 + i;
      if (r < rows) {
        const float hv = silu_g(accg[ms][i]) * accu[ms][i];
        hout[(size_t)(row0 + r) * I + ncol] = f32_to_bf16_bits(hv);
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// down: staging[slot(r)][n] = weight(r) * (h_r . Wd[n])
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_down_kernel(
    const uint16_t* __restrict__ hin, const uint8_t* __restrict__ dc, const uint8_t* __restrict__ ds,
    const int32_t* __restrict__ perm, const float* __restrict__ wts, const int32_t* __restrict__ info,
    const int32_t* __restrict__ mt_group, const int32_t* __restrict__ mt_row0, const int32_t* __restrict__ grp_row0,
    const int32_t* __restrict__ grp_rows, float* __restrict__ staging, int T, int k, int H, int I) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
  const int mt = blockIdx.x;
  if (mt >= info[1]) return;
  const int g = mt_group[mt], m0 = mt_row0[mt];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  const int tk = T * k;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ncol = blockIdx.y * BN + wave * 16 + (lane & 15);
  const bool col_ok = ncol < H;
  const size_t col = (size_t)g * (I >> 5) * H + (col_ok ? ncol : H - 1);
  const uint8_t* dcr = dc + col * 16;
  const uint8_t* dsr = ds + col;
  const int arow = tid >> 2, aseg = tid & 3;
  const bool a_ok = m0 + arow < rows;
  const uint16_t* asrc = hin + (size_t)(row0 + (a_ok ? m0 + arow : 0)) * I + aseg * 16;
  const int kq = (lane >> 4) * 8;
  f32x4 acc[4];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) acc[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < I; k0 += BK) {
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (a_ok && k0 + aseg * 16 < I) {
      v0 = *reinterpret_cast<const uint4*>(asrc + k0);
      v1 = *reinterpret_cast<const uint4*>(asrc + k0 + 8);
    }
    __syncthreads();
    *reinterpret_cast<uint4*>(&As[arow * LDA + aseg * 16]) = v0;
    *reinterpret_cast<uint4*>(&As[arow * LDA + aseg * 16 + 8]) = v1;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      if (k0 + kk < I) {
        const bf16x8 bd = load_b_frag(dcr, dsr, H, k0 + kk + kq);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[(ms * 16 + (lane & 15)) * LDA + kk + kq]);
          acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bd, acc[ms], 0, 0, 0);
        }
      }
    }
  }
  if (!col_ok) return;
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + ms * 16 + (lane >> 4) * 4 + i;
      if (r < rows) {
        const int gr = row0 + r;
        const int slot = gr < tk ? perm[gr] : gr;
        const float wt = gr < tk ? wts[slot] : 1.0f;
        staging[(size_t)slot * H + ncol] = acc[ms][i] * wt;
      }
    }
  }
}

// ------------------------------------------------------------------------------------
hipError_t launch_gemm_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int mt_bound, hipStream_t s) {
  dim3 grid(mt_bound, (d.I + BN - 1) / BN);
  const int tk = timing_begin("gemm_gateup", s);
  gemm_gateup_kernel<<<grid, 256, 0, s>>>(x, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, b.perm,
                                          b.info, b.mt_group, b.mt_row0, b.grp_row0, b.grp_rows,
                                          static_cast<uint16_t*>(b.h), T, d.K, d.H, d.I);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int mt_bound,
                            hipStream_t s) {
  dim3 grid(mt_bound, (d.H + BN - 1) / BN);
  const int tk = timing_begin("gemm_down", s);
  gemm_down_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(b.h), w.down_codes, w.down_scales, b.perm,
                                        b.w, b.info, b.mt_group, b.mt_row0, b.grp_row0, b.grp_rows, b.staging, T,
                                        d.K, d.H, d.I);
  timing_end(tk, s);
  return hipGetLastError();
}

}  // namespace moe
