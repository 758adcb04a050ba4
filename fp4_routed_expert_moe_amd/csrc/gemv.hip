// Decode path: expert-grouped FP4 GEMV.  Few rows per expert, so the work is bound by
// streaming the e2m1 nibbles and e8m0 scales from HBM once.
//
// "feat(dsv4): DeepSeek V4 Flash support -- CUDA/VRAM expert tiering ..." (PR #1031) makes a
// custom FP4 expert-grouped matvec the default GPU expert path, and "Add DeepSeek V4 Flash
// CPU inference with NVMe expert streaming" (PR #165, the NEON rows16 comment) pairs gate
// and up in one "dual" pass over interleaved rows.  On gfx950 the products go to the matrix
// cores, so the vector ALU only converts FP4 to bf16 (one convert per code byte):
//
// * Gate and up row n are produced by the same lane, so SwiGLU stays in registers; the
//   tokens of one group are the MFMA's M side, up to 16 per pass -- one pass for every group
//   in decode, whatever its token count.
// * Lane (n, q) loads one whole 16-byte block (32 values) of row n from the block-interleaved
//   kernel layout (a wave reads 4 x 256 contiguous bytes) and feeds it to four
//   16x16x32 bf16 MFMAs, eight values each.  The activation lanes (m, q) supply the same
//   K values of token m, so each MFMA sums one 8-value slice of four blocks; over the four
//   MFMAs every K value is met once.  Each lane scales by its own block's e8m0 inside the
//   convert (exact: a power of two).
// * Products bf16 x bf16 are exact in fp32 and accumulate in fp32.  h leaves gate/up as a
//   bf16 pair hi + lo (hi = bf16(h), lo = bf16(h - hi), 16 significant bits), and the down
//   projection runs one MFMA on each, so h is not rounded to 8 bits.
// * A token's result depends only on its own activations: the K order and the order in
//   which the wave partials are added are fixed, so batch composition never changes a bit.
#include "common.h"

namespace moe {

constexpr int kSkM = 16;  // tokens per pass (MFMA M)

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t u4w(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ------------------------------------------------------------------------------------
// Work split: a workgroup owns 64 rows of one group; its 4 waves take one quarter of the
// reduction axis each and stream all 64 rows (4 MFMA column tiles sharing one activation
// operand), reading 4 contiguous KiB per matrix per step.  The quarters are added through
// LDS in a fixed order, wave w finishing column tile w.
// ------------------------------------------------------------------------------------
constexpr int kTiles = 4;   // 16-row MFMA column tiles per wave
constexpr int kSplit = 4;   // waves per workgroup = reduction-axis quarters

// One step of the gate/up stream: 4 blocks (lane q takes block kb + q) of the
// wave's kTiles column tiles, both matrices, plus the matching activation slice.
struct GateUpStage {
  uint4 cg[kTiles], cu[kTiles], xa[4];
  float sg[kTiles], su[kTiles];
};

__device__ __forceinline__ void load_gateup(GateUpStage& st, const uint8_t* __restrict__ gc,
                                            const uint8_t* __restrict__ gs, const uint8_t* __restrict__ uc,
                                            const uint8_t* __restrict__ us, const uint16_t* __restrict__ xr,
                                            const size_t* col, int kb, int kb_hi, int I, int q, bool mok) {
  const int blk = kb + q;
  const bool bok = blk < kb_hi;
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    st.cg[j] = st.cu[j] = make_uint4(0, 0, 0, 0);
    st.sg[j] = st.su[j] = 0.f;
    if (bok) {
      const size_t c = col[j] + (size_t)blk * I;
      st.cg[j] = *reinterpret_cast<const uint4*>(gc + c * 16);
      st.cu[j] = *reinterpret_cast<const uint4*>(uc + c * 16);
      st.sg[j] = e8m0_to_f32(gs[c]);
      st.su[j] = e8m0_to_f32(us[c]);
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) st.xa[s] = make_uint4(0, 0, 0, 0);
  if (bok && mok) {
    const uint4* xp = reinterpret_cast<const uint4*>(xr + (size_t)blk * 32);
#pragma unroll
    for (int s = 0; s < 4; ++s) st.xa[s] = xp[s];
  }
}

struct DownStage {
  uint4 cd[kTiles], ha[4], la[4];
  float sd[kTiles];
};

__device__ __forceinline__ void load_down(DownStage& st, const uint8_t* __restrict__ dc,
                                          const uint8_t* __restrict__ ds, const uint16_t* __restrict__ hhi,
                                          const uint16_t* __restrict__ hlo, size_t hrow, const size_t* col, int kb,
                                          int kb_hi, int H, int q, bool mok) {
  const int blk = kb + q;
  const bool bok = blk < kb_hi;
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    st.cd[j] = make_uint4(0, 0, 0, 0);
    st.sd[j] = 0.f;
    if (bok) {
      const size_t c = col[j] + (size_t)blk * H;
      st.cd[j] = *reinterpret_cast<const uint4*>(dc + c * 16);
      st.sd[j] = e8m0_to_f32(ds[c]);
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) st.ha[s] = st.la[s] = make_uint4(0, 0, 0, 0);
  if (bok && mok) {
    const uint4* hp = reinterpret_cast<const uint4*>(hhi + hrow + (size_t)blk * 32);
    const uint4* lp = reinterpret_cast<const uint4*>(hlo + hrow + (size_t)blk * 32);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      st.ha[s] = hp[s];
      st.la[s] = lp[s];
    }
  }
}

// gate/up:  h[row][n] = silu(x_t . Wg[n]) * (x_t . Wu[n]), stored as bf16 hi + lo
__global__ __launch_bounds__(256) void gemv_gateup_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ gc, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ uc, const uint8_t* __restrict__ us, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ act, const int32_t* __restrict__ info, const int32_t* __restrict__ grp_row0,
    const int32_t* __restrict__ grp_rows, uint16_t* __restrict__ hhi, uint16_t* __restrict__ hlo, int T, int k,
    int H, int I) {
  __shared__ f32x4 red[kSplit][kTiles][2][64];
  if ((int)blockIdx.y >= info[0]) return;
  const int g = act[blockIdx.y];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * (16 * kTiles);
  const int KB = H >> 5;
  const int kb_lo = wave * KB / kSplit, kb_hi = (wave + 1) * KB / kSplit;
  const size_t gbase = (size_t)g * KB * I;
  size_t col[kTiles];
#pragma unroll
  for (int j = 0; j < kTiles; ++j) col[j] = gbase + min(n0 + 16 * j + m, I - 1);
  const int tk = T * k;
  for (int c0 = 0; c0 < rows; c0 += kSkM) {
    const int nt = min(kSkM, rows - c0);
    const bool mok = m < nt;
    const uint16_t* xr = x + (size_t)(mok ? row_token(perm, row0 + c0 + m, tk, k) : 0) * H;
    f32x4 ag[kTiles], au[kTiles];
#pragma unroll
    for (int j = 0; j < kTiles; ++j) ag[j] = au[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = kb_lo; kb < kb_hi; kb += 4) {
      GateUpStage cur;
      load_gateup(cur, gc, gs, uc, us, xr, col, kb, kb_hi, I, q, mok);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = as_bf16x8(cur.xa[s]);
#pragma unroll
        for (int j = 0; j < kTiles; ++j) {
          ag[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16x8(u4w(cur.cg[j], s), cur.sg[j]), ag[j], 0,
                                                          0, 0);
          au[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fp4x8_to_bf16x8(u4w(cur.cu[j], s), cur.su[j]), au[j], 0,
                                                          0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      red[wave][j][0][lane] = ag[j];
      red[wave][j][1][lane] = au[j];
    }
    __syncthreads();
    {
      const int j = wave;  // wave w finishes column tile w
      f32x4 gsum = red[0][j][0][lane], usum = red[0][j][1][lane];
#pragma unroll
      for (int w = 1; w < kSplit; ++w) {
        gsum += red[w][j][0][lane];
        usum += red[w][j][1][lane];
      }
      const int n = n0 + 16 * j + m;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 4 * q + i;  // lane (n, q) holds tokens 4q .. 4q+3 of row n
        if (n < I && tok < nt) {
          const float hv = silu_f(gsum[i]) * usum[i];
          const uint16_t hi = bf16_bits(hv);
          const size_t o = (size_t)(row0 + c0 + tok) * I + n;
          hhi[o] = hi;
          hlo[o] = bf16_bits(hv - bf16_val(hi));
        }
      }
    }
    __syncthreads();
  }
}

// down:  staging[slot(r)][n] = weight(r) * ((h_hi + h_lo)_r . Wd[n])
__global__ __launch_bounds__(256) void gemv_down_kernel(
    const uint16_t* __restrict__ hhi, const uint16_t* __restrict__ hlo, const uint8_t* __restrict__ dc,
    const uint8_t* __restrict__ ds, const int32_t* __restrict__ perm, const float* __restrict__ wts,
    const int32_t* __restrict__ act, const int32_t* __restrict__ info, const int32_t* __restrict__ grp_row0,
    const int32_t* __restrict__ grp_rows, float* __restrict__ staging, int T, int k, int H, int I) {
  __shared__ f32x4 red[kSplit][kTiles][64];
  if ((int)blockIdx.y >= info[0]) return;
  const int g = act[blockIdx.y];
  const int rows = grp_rows[g], row0 = grp_row0[g];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * (16 * kTiles);
  const int KB = I >> 5;
  const int kb_lo = wave * KB / kSplit, kb_hi = (wave + 1) * KB / kSplit;
  const size_t gbase = (size_t)g * KB * H;
  size_t col[kTiles];
#pragma unroll
  for (int j = 0; j < kTiles; ++j) col[j] = gbase + min(n0 + 16 * j + m, H - 1);
  const int tk = T * k;
  for (int c0 = 0; c0 < rows; c0 += kSkM) {
    const int nt = min(kSkM, rows - c0);
    const bool mok = m < nt;
    const size_t hrow = (size_t)(row0 + c0 + (mok ? m : 0)) * I;
    f32x4 acc[kTiles];
#pragma unroll
    for (int j = 0; j < kTiles; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = kb_lo; kb < kb_hi; kb += 4) {
      DownStage cur;
      load_down(cur, dc, ds, hhi, hlo, hrow, col, kb, kb_hi, H, q, mok);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int j = 0; j < kTiles; ++j) {
          const bf16x8 b = fp4x8_to_bf16x8(u4w(cur.cd[j], s), cur.sd[j]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.ha[s]), b, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.la[s]), b, acc[j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kTiles; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    {
      const int j = wave;
      f32x4 sum = red[0][j][lane];
#pragma unroll
      for (int w = 1; w < kSplit; ++w) sum += red[w][j][lane];
      const int n = n0 + 16 * j + m;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 4 * q + i;
        if (n < H && tok < nt) {
          const int r = row0 + c0 + tok;
          const int slot = r < tk ? perm[r] : r;
          const float wt = r < tk ? wts[slot] : 1.0f;
          staging[(size_t)slot * H + n] = sum[i] * wt;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
hipError_t launch_gemv_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int max_act, hipStream_t s) {
  dim3 grid((d.I + 16 * kTiles - 1) / (16 * kTiles), max_act);
  uint16_t* hhi = static_cast<uint16_t*>(b.h);
  uint16_t* hlo = hhi + (size_t)T * (d.K + d.S) * d.I;
  const int tk = timing_begin("gemv_gateup", s);
  gemv_gateup_kernel<<<grid, 64 * kSplit, 0, s>>>(x, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, b.perm,
                                                  b.act, b.info, b.grp_row0, b.grp_rows, hhi, hlo, T, d.K, d.H, d.I);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int max_act,
                            hipStream_t s) {
  dim3 grid((d.H + 16 * kTiles - 1) / (16 * kTiles), max_act);
  const uint16_t* hhi = static_cast<const uint16_t*>(b.h);
  const uint16_t* hlo = hhi + (size_t)T * (d.K + d.S) * d.I;
  const int tk = timing_begin("gemv_down", s);
  gemv_down_kernel<<<grid, 64 * kSplit, 0, s>>>(hhi, hlo, w.down_codes, w.down_scales, b.perm, b.w, b.act, b.info,
                                                b.grp_row0, b.grp_rows, b.staging, T, d.K, d.H, d.I);
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
