// Decode path: expert-grouped FP4 GEMV.  Few rows per expert, so the work is bound by
// streaming the e2m1 nibbles and e8m0 scales from HBM once.
//
// "feat(dsv4): DeepSeek V4 Flash support -- CUDA/VRAM expert tiering ..." (PR #1031) makes a
// custom FP4 expert-grouped matvec the default GPU expert path, and "Add DeepSeek V4 Flash
// CPU inference with NVMe expert streaming" (PR #165, the NEON rows16 comment) pairs gate
// and up in one "dual" pass over interleaved rows.  On gfx950 the products run on the
// block-scaled matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4), which take the e2m1 codes
// and their e8m0 scales exactly as stored: no convert touches the weights.
//
// * B (weights, FP4): lane (n, q) holds block kb+q of row n -- one 16-byte chunk of the
//   block-interleaved kernel layout (a wave reads 4 x 256 contiguous bytes per column tile)
//   -- through buffer loads; one dword per lane holds the scales of its four column tiles
//   (a wave's scales for a K step are 256 contiguous bytes), picked by the MFMA's byte select.
// * A (activations, FP8 e4m3): lane (m, q) holds 16 values at K offset 16q and 16 at 64+16q
//   of the 128-value step for token m, plus the scale of block kb+q.  Activations arrive as
//   exact FP8 term splits (x: 2 terms = all 8 bf16 bits; h: 3 terms = 12 bits), one MFMA
//   per term, all accumulating in fp32.
// * A wave owns 64 rows (4 column tiles of 16 sharing the activation operand) and one
//   quarter of the reduction axis (whole 128-value iterations, the next one's loads in
//   flight while the current one runs); the 4 quarters are added through LDS in a fixed
//   order.
//   Gate and up row n meet in the same lane, so SwiGLU stays in registers.  The tokens of
//   a group are the MFMA's M side, up to 16 per pass: one pass per group in decode.
// * A token's result depends only on its own activations (fixed K and reduction order), so
//   batch composition never changes a bit of it.
#include <type_traits>

#include "common.h"

namespace moe {

constexpr int kSkM = 16;    // tokens per pass (MFMA M)
#ifndef MOE_GEMV_SPLIT
#define MOE_GEMV_SPLIT 4
#endif
#ifndef MOE_DEC_HTERMS
#define MOE_DEC_HTERMS 3
#endif
constexpr int kHTerms = MOE_DEC_HTERMS;  // FP8 terms of h between gate/up and down (2 or 3)
static_assert(kHTerms == 2 || kHTerms == 3, "h term count");
constexpr int kSplit = MOE_GEMV_SPLIT;  // waves per gate/up workgroup = reduction-axis slices
// TL = 16-row MFMA column tiles per wave (4, or 2 / 1 when few groups are active: more
// workgroups over the same bytes); all TL tiles share one scale dword.

// One K iteration (4 blocks = 128 values) of a wave's operands.  Weights come through buffer
// descriptors spanning one group's matrix: a fixed per-lane offset and the K position as a
// scalar offset; in the last iteration of a K that is not a multiple of 128 the lanes past K
// read zero codes (their packed scales are 0 too).  Activations come from the token rows of
// the pass; past the end of K they read a valid part of the row (multiplied by zero weights).
constexpr int kBufferFlags = 0x00020000;  // raw byte-addressed buffer, 32-bit data format
constexpr int kWeightAux = 2;             // nontemporal: the weights are streamed once
constexpr int kOutOfRange = 1 << 30;      // added to a lane's buffer offset: reads zeros

template <int NM, int NA, int TL>
struct GFrag {
  i32x4 c[NM][TL];
  int s[NM];  // byte sel + j: scale of column tile j
  i32x4 a[NA][2];
  int sa;
};
template <int NM>
struct GSrc {
  __amdgpu_buffer_rsrc_t c[NM], s[NM];
  int voff_c, voff_s;  // column tile 0, K block q, K iteration 0 (tile j is 16 columns on)
  int sel;             // byte of tile 0 in the lane's scale dword
};
// Matrix mtx's columns start at n0 + mtx * col_step (col_step a multiple of 64): gate and up
// use the same columns of two matrices, down two adjacent 64-column blocks of one.
template <int NM>
__device__ __forceinline__ void gsrc_init(GSrc<NM>& src, const uint8_t* const* codes, const uint8_t* const* scales,
                                          int g, int KB, int N, int n0, int m, int q, int col_step) {
  const int slab = (int)scale_slab_bytes(N, 32 * KB);
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx) {
    const int dc = mtx * col_step * 16, dsb = mtx * (col_step >> 6) * 256;
    src.c[mtx] = __builtin_amdgcn_make_buffer_rsrc((void*)(codes[mtx] + (size_t)g * KB * N * 16 + dc), (short)0,
                                                   KB * N * 16 - dc, kBufferFlags);
    src.s[mtx] = __builtin_amdgcn_make_buffer_rsrc((void*)(scales[mtx] + (size_t)g * slab + dsb), (short)0,
                                                   slab - dsb, kBufferFlags);
  }
  // columns past N read other bytes of the group (or zeros past its end); they are not stored
  src.voff_c = (q * N + n0 + m) * 16;
  src.voff_s = (((n0 >> 6) * 16 + m) * 4 + q) * 4;  // n0 is a multiple of 16
  src.sel = (n0 >> 4) & 3;
}
template <int NM, int NA, int TL>
__device__ __forceinline__ void gv_load(GFrag<NM, NA, TL>& f, const GSrc<NM>& src, int N, const uint8_t* const* arow,
                                        const uint8_t* asc, int K, int it, int q) {
  const int kb = 4 * it;
  const int so_c = __builtin_amdgcn_readfirstlane(kb * N * 16);
  const int so_s = __builtin_amdgcn_readfirstlane(it * ((N + 63) >> 6) * 256);
  // Lanes whose block is past K (last iteration only) move their per-lane offset past the
  // descriptor's range: they read zeros and touch no memory.  (The scalar offset is not
  // relied on for the range check.)
  int voff_c = src.voff_c;
  if (kb + 4 > (K >> 5)) voff_c += (kb + q >= (K >> 5)) ? kOutOfRange : 0;
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx) {
#pragma unroll
    for (int j = 0; j < TL; ++j)
      f.c[mtx][j] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(src.c[mtx], voff_c + 256 * j, so_c, kWeightAux));
    f.s[mtx] = __builtin_amdgcn_raw_buffer_load_b32(src.s[mtx], src.voff_s, so_s, kWeightAux);
  }
  int o1 = kb * 32 + 16 * q, o2 = o1 + 64;
  if ((kb + 4) * 32 > K) {  // last iteration of a K that is not a multiple of 128 (uniform)
    o1 = min(o1, K - 16);
    o2 = min(o2, K - 16);
  }
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    f.a[t][0] = *reinterpret_cast<const i32x4*>(arow[t] + o1);
    f.a[t][1] = *reinterpret_cast<const i32x4*>(arow[t] + o2);
  }
  f.sa = asc[min(kb + q, (K >> 5) - 1)];
}
// acc[mtx][j] += sum over the NA terms of A(term) x B(mtx, tile j); term t has scale sa - 4t.
template <int NM, int NA, int TL>
__device__ __forceinline__ void gv_mma(const GFrag<NM, NA, TL>& f, f32x4 (&acc)[NM][TL], int sel) {
  i32x8 a[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) a[t] = __builtin_shufflevector(f.a[t][0], f.a[t][1], 0, 1, 2, 3, 4, 5, 6, 7);
  static_assert(TL == 1 || TL == 2 || TL == 4, "a wave's tiles share one scale dword");
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx) {
    const int sb = TL == 4 ? f.s[mtx] : (int)((uint32_t)f.s[mtx] >> (8 * sel));  // tile j at byte j
    i32x8 b[TL];
#pragma unroll
    for (int j = 0; j < TL; ++j)
      b[j] = __builtin_shufflevector(f.c[mtx][j], f.c[mtx][j], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const int sa = f.sa - 4 * t;
      acc[mtx][0] = mma_f8f4_sb<0>(a[t], b[0], acc[mtx][0], sa, sb);
      if constexpr (TL > 1) acc[mtx][1] = mma_f8f4_sb<1>(a[t], b[1], acc[mtx][1], sa, sb);
      if constexpr (TL > 2) {
        acc[mtx][2] = mma_f8f4_sb<2>(a[t], b[2], acc[mtx][2], sa, sb);
        acc[mtx][3] = mma_f8f4_sb<3>(a[t], b[3], acc[mtx][3], sa, sb);
      }
    }
  }
}
// ---- the FP8 shared expert (e4m3 codes, float32 scale per 128 x 128 block) --------------
// Kernel layout [K/128][N][128]: the 128 codes of reduction step it of row n are together.  In
// the FP8 lane layout (common.h) lane (n, q) takes bytes 16q.. and 64+16q.. of its row's step:
// two 16-byte loads, and across the wave each row's 128 bytes are read once.  A wave's TL tiles
// (16*TL consecutive rows from a multiple of 16*TL) lie in one 128-row scale block, so one
// float32 per matrix and step scales the wave's products (applied after the step's MFMAs).
template <int NM, int NA, int TL>
struct GFrag8 {
  i32x4 c[NM][TL][2];
  float s[NM];
  i32x4 a[NA][2];
  int sa;
};
template <int NM>
struct GSrc8 {
  __amdgpu_buffer_rsrc_t c[NM];
  const float* s[NM];  // this wave's row block of each matrix's scales: s[mtx][it]
  int voff;            // tile 0, step 0
  int sel;             // unused (the FP4 source's byte select)
};
template <int NM>
__device__ __forceinline__ void gsrc8_init(GSrc8<NM>& src, const uint8_t* const* codes, const float* const* scales,
                                           int K, int N, int n0, int m, int q) {
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx) {
    src.c[mtx] = __builtin_amdgcn_make_buffer_rsrc((void*)codes[mtx], (short)0, K * N, kBufferFlags);
    src.s[mtx] = scales[mtx] + (size_t)(n0 / kFp8Block) * (K / kFp8Block);
  }
  src.voff = (n0 + m) * 128 + 16 * q;  // rows past N read other rows (or zeros past the end): not stored
  src.sel = 0;
}
template <int NM, int NA, int TL>
__device__ __forceinline__ void gv_load(GFrag8<NM, NA, TL>& f, const GSrc8<NM>& src, int N, const uint8_t* const* arow,
                                        const uint8_t* asc, int K, int it, int q) {
  const int so = __builtin_amdgcn_readfirstlane(it * N * 128);
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx) {
#pragma unroll
    for (int j = 0; j < TL; ++j) {
      f.c[mtx][j][0] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(src.c[mtx], src.voff + 2048 * j, so, kWeightAux));
      f.c[mtx][j][1] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(src.c[mtx], src.voff + 2048 * j + 64, so, kWeightAux));
    }
    f.s[mtx] = src.s[mtx][it];
  }
  const int o1 = it * 128 + 16 * q, o2 = o1 + 64;  // K is a multiple of 128 here
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    f.a[t][0] = *reinterpret_cast<const i32x4*>(arow[t] + o1);
    f.a[t][1] = *reinterpret_cast<const i32x4*>(arow[t] + o2);
  }
  f.sa = asc[4 * it + q];
}
template <int NM, int NA, int TL>
__device__ __forceinline__ void gv_mma(const GFrag8<NM, NA, TL>& f, f32x4 (&acc)[NM][TL], int sel) {
  (void)sel;
  i32x8 a[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) a[t] = __builtin_shufflevector(f.a[t][0], f.a[t][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx)
#pragma unroll
    for (int j = 0; j < TL; ++j) {
      const i32x8 b = __builtin_shufflevector(f.c[mtx][j][0], f.c[mtx][j][1], 0, 1, 2, 3, 4, 5, 6, 7);
      f32x4 p = mma_f8f8(a[0], b, f32x4{0.f, 0.f, 0.f, 0.f}, f.sa);
#pragma unroll
      for (int t = 1; t < NA; ++t) p = mma_f8f8(a[t], b, p, f.sa - 4 * t);
      acc[mtx][j] += p * f.s[mtx];
    }
}

// The fragment and source types of a weight format.
template <bool FP8, int NM, int NA, int TL>
struct GvFmt {
  using Frag = GFrag<NM, NA, TL>;
  using Src = GSrc<NM>;
};
template <int NM, int NA, int TL>
struct GvFmt<true, NM, NA, TL> {
  using Frag = GFrag8<NM, NA, TL>;
  using Src = GSrc8<NM>;
};

// This wave's K iterations [it_lo, it_hi), the loads of iteration i+1 in flight while
// iteration i runs on the matrix cores.  The steady-state loop body is one block whose loads
// are issued before the matrix work (a scheduling barrier keeps them there), so the wait
// before each step's MFMAs covers only that step's own loads.
template <int NM, int NA, int TL, class Src>
__device__ __forceinline__ void gv_pass(f32x4 (&acc)[NM][TL], const Src& src, int N,
                                        const uint8_t* const* arow, const uint8_t* asc, int K, int it_lo, int it_hi,
                                        int q) {
  if (it_lo >= it_hi) return;
  using Frag = typename GvFmt<std::is_same<Src, GSrc8<NM>>::value, NM, NA, TL>::Frag;
  Frag f0, f1;
  gv_load(f0, src, N, arow, asc, K, it_lo, q);
  int it = it_lo;
  for (; it + 2 < it_hi; it += 2) {
    gv_load(f1, src, N, arow, asc, K, it + 1, q);
    __builtin_amdgcn_sched_barrier(0);
    gv_mma(f0, acc, src.sel);
    gv_load(f0, src, N, arow, asc, K, it + 2, q);
    __builtin_amdgcn_sched_barrier(0);
    gv_mma(f1, acc, src.sel);
  }
  if (it + 1 < it_hi) {
    gv_load(f1, src, N, arow, asc, K, it + 1, q);
    __builtin_amdgcn_sched_barrier(0);
    gv_mma(f0, acc, src.sel);
    gv_mma(f1, acc, src.sel);
  } else {
    gv_mma(f0, acc, src.sel);
  }
}

// ------------------------------------------------------------------------------------
// gate/up:  h[row][n] = silu(x_t . Wg[n]) * (x_t . Wu[n]), written as 3 FP8 terms + scales
// (h8 = [kHTerms][rows][I] bytes, hs = [rows][kb_pad(I)] e8m0).
// ------------------------------------------------------------------------------------
// One tile: column tile bx of active-group slot `slot` (FP4), or column tile bx of the FP8
// shared expert (slot unused).  red: the workgroup's LDS reduction buffer.
#define GATEUP_ARGS                                                                                         \
  const uint8_t *__restrict__ xq, const uint8_t *__restrict__ gc, const uint8_t *__restrict__ gs,           \
      const uint8_t *__restrict__ uc, const uint8_t *__restrict__ us, const uint8_t *__restrict__ g8,       \
      const float *__restrict__ g8s, const uint8_t *__restrict__ u8, const float *__restrict__ u8s,         \
      const int32_t *__restrict__ perm, const GroupRec *__restrict__ grec, uint8_t *__restrict__ h8,        \
      uint32_t *__restrict__ stage_clear, int skip_group, int T, int k, int H, int I, int R
#define GATEUP_PASS xq, gc, gs, uc, us, g8, g8s, u8, u8s, perm, grec, h8, stage_clear, skip_group, T, k, H, I, R
template <int TL, int SPLIT, bool FP8>
__device__ __forceinline__ void gateup_tile(f32x4 (*red)[TL][2][64], int bx, int slot, GATEUP_ARGS) {
  (void)stage_clear;
  static_assert(TL == 2 || TL == 4, "h's FP8 blocks are 32 columns: a workgroup finishes whole blocks");
  int g, row0, rows;
  if constexpr (FP8) {
    g = -1;
    row0 = T * k;
    rows = T;
  } else {
    const int4 rec = *reinterpret_cast<const int4*>(grec + slot);
    if (slot >= rec.w || rec.x == skip_group) return;
    g = __builtin_amdgcn_readfirstlane(rec.x);
    row0 = __builtin_amdgcn_readfirstlane(rec.y);
    rows = __builtin_amdgcn_readfirstlane(rec.z);
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  const int n0 = bx * (16 * TL);
  const int KB = H >> 5;
  const int NI = (KB + 3) >> 2;  // K iterations of 4 blocks
  const int it_lo = wave * NI / SPLIT, it_hi = (wave + 1) * NI / SPLIT;
  typename GvFmt<FP8, 2, 2, TL>::Src src;
  if constexpr (FP8) {
    const uint8_t* codes[2] = {g8, u8};
    const float* scales[2] = {g8s, u8s};
    gsrc8_init<2>(src, codes, scales, H, I, n0, m, q);
  } else {
    const uint8_t* codes[2] = {gc, uc};
    const uint8_t* scales[2] = {gs, us};
    gsrc_init<2>(src, codes, scales, g, KB, I, n0, m, q, 0);
  }
  const uint8_t* x_hi = xq;
  const uint8_t* x_lo = xq + (size_t)T * H;
  const uint8_t* x_sc = xq + (size_t)2 * T * H;
  uint8_t* hs = h8 + (size_t)kHTerms * R * I;
  const int tk = T * k;
  for (int c0 = 0; c0 < rows; c0 += kSkM) {
    const int nt = min(kSkM, rows - c0);
    // lanes past the pass's tokens repeat its first token (their results are dropped)
    const int tok = row_token(perm, row0 + c0 + (m < nt ? m : 0), tk, k);
    const uint8_t* arow[2] = {x_hi + (size_t)tok * H, x_lo + (size_t)tok * H};
    f32x4 acc[2][TL];
#pragma unroll
    for (int j = 0; j < TL; ++j) acc[0][j] = acc[1][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    gv_pass<2, 2, TL>(acc, src, I, arow, x_sc + (size_t)tok * kb_pad(H), H, it_lo, it_hi, q);
    f32x4 (&ag)[TL] = acc[0];
    f32x4 (&au)[TL] = acc[1];
#pragma unroll
    for (int j = 0; j < TL; ++j) {
      red[wave][j][0][lane] = ag[j];
      red[wave][j][1][lane] = au[j];
    }
    __syncthreads();
    if (wave < TL / 2) {
      // wave p finishes column tiles 2p and 2p+1 = one 32-column block of h
      const int p = wave;
      float hv[2][4];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int j = 2 * p + c;
        f32x4 gsum = red[0][j][0][lane], usum = red[0][j][1][lane];
#pragma unroll
        for (int w = 1; w < SPLIT; ++w) {
          gsum += red[w][j][0][lane];
          usum += red[w][j][1][lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[c][i] = silu(gsum[i]) * usum[i];
      }
      const int nb = n0 + 32 * p;  // first column of the block
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // lanes with the same q hold the same 4 tokens: reduce |h| over the 32 columns
        const int sc = fp8_block_scale(row16_max(fmaxf(fabsf(hv[0][i]), fabsf(hv[1][i]))));
        const float inv = fp8_inv_scale(sc);
        const int tok_i = 4 * q + i;
        if (nb < I && tok_i < nt) {
          const size_t r = (size_t)(row0 + c0 + tok_i);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint32_t nanm = fp8_nan_mask(hv[c][i]);  // non-finite h stays NaN in every term
            float v = hv[c][i] * inv;
            const uint32_t t0 = fp8_of(v) | nanm;
            v = (v - f32_of_fp8(t0)) * 16.f;
            const uint32_t t1 = fp8_of(v) | nanm;
            v = (v - f32_of_fp8(t1)) * 16.f;
            const uint32_t t2 = fp8_of(v) | nanm;
            const size_t o = r * I + nb + 16 * c + m;
            h8[o] = (uint8_t)t0;
            h8[(size_t)R * I + o] = (uint8_t)t1;
            if (kHTerms == 3) h8[(size_t)2 * R * I + o] = (uint8_t)t2;
          }
          if (m == 0) {
            hs[r * kb_pad(I) + (nb >> 5)] = (uint8_t)sc;
            if ((nb >> 5) == (I >> 5) - 1)  // pad bytes of the row
              for (int j = I >> 5; j < kb_pad(I); ++j) hs[r * kb_pad(I) + j] = (uint8_t)127;
          }
        }
      }
    }
    __syncthreads();
  }
}

// The staging rows the down kernel fills next (R x H words) start at zero: every workgroup
// of the gate/up launch clears a grid-stride share.
template <int NTH>
__device__ __forceinline__ void clear_stage(uint32_t* stage_clear, int R, int H) {
  if (!stage_clear) return;
  const size_t n = (size_t)R * H;
  const size_t wg = (size_t)blockIdx.y * gridDim.x + blockIdx.x, nwg = (size_t)gridDim.x * gridDim.y;
  for (size_t i = (wg * NTH + threadIdx.x) * 4; i < n; i += nwg * NTH * 4)
    *reinterpret_cast<uint4*>(stage_clear + i) = make_uint4(0u, 0u, 0u, 0u);
}

// FP8: the FP8 shared expert alone (the grid's y dimension is 1; its rows are the T tokens after
// the T*k routed rows).  Otherwise the FP4 groups of the active-group slots, skipping group
// `skip_group` (the shared expert when it is FP8; -1 for none).
template <int TL, int SPLIT, bool FP8>
__global__ __launch_bounds__(64 * SPLIT, SPLIT <= 4 ? 8 / SPLIT : 1) void gemv_gateup_kernel(GATEUP_ARGS) {
  clear_stage<64 * SPLIT>(stage_clear, R, H);
  __shared__ f32x4 red[SPLIT][TL][2][64];
  gateup_tile<TL, SPLIT, FP8>(red, blockIdx.x, blockIdx.y, GATEUP_PASS);
}

// The FP4 groups and an FP8 shared expert in one launch: the first TL/2 rows of the grid are the
// FP8 expert's 32-column tiles (dispatched first, so they overlap the FP4 tiles), the rest the
// FP4 active-group slots (skip_group = the shared expert's FP4 slot).
template <int TL, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT, SPLIT <= 4 ? 8 / SPLIT : 1) void gemv_gateup_mixed_kernel(GATEUP_ARGS) {
  clear_stage<64 * SPLIT>(stage_clear, R, H);
  __shared__ f32x4 red[SPLIT][TL][2][64];
  constexpr int n8 = TL / 2;
  if ((int)blockIdx.y < n8)
    gateup_tile<2, SPLIT, true>(reinterpret_cast<f32x4(*)[2][2][64]>(red), blockIdx.y * gridDim.x + blockIdx.x, 0,
                                GATEUP_PASS);
  else
    gateup_tile<TL, SPLIT, false>(red, blockIdx.x, blockIdx.y - n8, GATEUP_PASS);
}

// ------------------------------------------------------------------------------------
// down:  staging[slot(r)][n] = weight(r) * (h_r . Wd[n]),  h_r from its 3 FP8 terms, and
// y[t][n] = staging[shared slot of t][n] + sum_j staging[t*k + j][n].
// Workgroup (c, a) handles column tile c of active group a.  The workgroup of the last active
// group of each tile also adds the tile's rows, in the combine order of the prefill path,
// once they are all in staging: a staging word is 0 until its row is written (the gate/up
// kernel of the call clears them), so no writer waits for its stores to complete.
// ------------------------------------------------------------------------------------
constexpr int kFlagPolls = 1 << 20;  // bound of each word's wait: never hangs
// Staging words hold a row value's bits XOR kStageKey, so a word is 0 only until written: the
// key is a signalling-NaN pattern, which no arithmetic result has (results are quiet).  The
// gate/up kernel clears the staging rows of the call.
constexpr uint32_t kStageKey = 0x7F800001u;

constexpr int kDnBlocks = 1;  // column blocks (of TL tiles) per down workgroup
#ifndef MOE_DN_SPLIT
#define MOE_DN_SPLIT 4
#endif
constexpr int kDnSplit = MOE_DN_SPLIT;            // waves per down workgroup = reduction-axis slices

// One tile: column tile bx of active-group slot `slot` (FP4), or column tile bx of the FP8 shared
// expert.  comb: which tiles add the call's rows -- for FP4, the slot `comb` places from the
// end (1: the last slot; 2: the last routed slot, when the shared expert's slot is skipped);
// for FP8, every tile when comb != 0.  red: the workgroup's LDS reduction buffer.
#define DOWN_ARGS                                                                                           \
  const uint8_t *__restrict__ h8, const uint8_t *__restrict__ dc, const uint8_t *__restrict__ ds,           \
      const uint8_t *__restrict__ d8, const float *__restrict__ d8s, const int32_t *__restrict__ perm,      \
      const float *__restrict__ row_w, const GroupRec *__restrict__ grec, float *__restrict__ staging,       \
      float *__restrict__ y, int skip_group, float routed_scale, int T, int k, int S, int H, int I, int R
#define DOWN_PASS h8, dc, ds, d8, d8s, perm, row_w, grec, staging, y, skip_group, routed_scale, T, k, S, H, I, R
template <int TL, bool FP8, int SPLIT>
__device__ __forceinline__ void down_tile(f32x4 (*red)[kDnBlocks][TL][64], int bx, int slot, int comb, DOWN_ARGS) {
  constexpr int kDnCols = kDnBlocks * 16 * TL;  // output columns per workgroup
  // column tiles each wave finishes (waves past the last tile only reduce)
  constexpr int kDnPerWave = kDnBlocks * TL > SPLIT ? kDnBlocks * TL / SPLIT : 1;
  static_assert(kDnPerWave * SPLIT >= kDnBlocks * TL, "down workgroup shape");
  int g, row0, rows;
  bool combiner;
  if constexpr (FP8) {
    g = -1;
    row0 = T * k;
    rows = T;
    combiner = comb != 0;
  } else {
    const int4 rec = *reinterpret_cast<const int4*>(grec + slot);
    const int nslots = rec.w;
    if (slot >= nslots || rec.x == skip_group) return;
    g = __builtin_amdgcn_readfirstlane(rec.x);
    row0 = __builtin_amdgcn_readfirstlane(rec.y);
    rows = __builtin_amdgcn_readfirstlane(rec.z);
    combiner = slot == nslots - comb;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  const int n0 = bx * kDnCols;
  const int KB = I >> 5;
  const int NI = (KB + 3) >> 2;
  const int it_lo = wave * NI / SPLIT, it_hi = (wave + 1) * NI / SPLIT;
  typename GvFmt<FP8, kDnBlocks, kHTerms, TL>::Src src;
  if constexpr (FP8) {
    const uint8_t* codes[kDnBlocks] = {d8};
    const float* scales[kDnBlocks] = {d8s};
    gsrc8_init<kDnBlocks>(src, codes, scales, I, H, n0, m, q);
  } else {
    const uint8_t* codes[kDnBlocks] = {dc};
    const uint8_t* scales[kDnBlocks] = {ds};
    gsrc_init<kDnBlocks>(src, codes, scales, g, KB, H, n0, m, q, 16 * TL);
  }
  const uint8_t* hs = h8 + (size_t)kHTerms * R * I;
  const int tk = T * k;
  for (int c0 = 0; c0 < rows; c0 += kSkM) {
    const int nt = min(kSkM, rows - c0);
    const size_t r = (size_t)(row0 + c0 + (m < nt ? m : 0));
    // staging slot and weight of the rows this lane finishes, loaded now (they arrive during the K loop)
    int slot_i[4];
    float wt_i[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = row0 + c0 + min(4 * q + i, nt - 1);
      slot_i[i] = rr < tk ? perm[rr] : rr;
      wt_i[i] = rr < tk ? row_w[rr] * routed_scale : 1.0f;
    }
    const uint8_t* arow[kHTerms] = {h8 + r * I, h8 + (size_t)R * I + r * I
#if MOE_DEC_HTERMS == 3
                                    , h8 + (size_t)2 * R * I + r * I
#endif
    };
    f32x4 acc[kDnBlocks][TL];
#pragma unroll
    for (int c = 0; c < kDnBlocks; ++c)
#pragma unroll
      for (int j = 0; j < TL; ++j) acc[c][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    gv_pass<kDnBlocks, kHTerms, TL>(acc, src, H, arow, hs + r * kb_pad(I), I, it_lo, it_hi, q);
#pragma unroll
    for (int c = 0; c < kDnBlocks; ++c)
#pragma unroll
      for (int j = 0; j < TL; ++j) red[wave][c][j][lane] = acc[c][j];
    __syncthreads();
    // wave w finishes column tiles kDnPerWave*w .. kDnPerWave*w + kDnPerWave - 1
#pragma unroll
    for (int u = 0; u < kDnPerWave; ++u) {
      const int jj = kDnPerWave * wave + u, c = jj / TL, j = jj % TL;
      if (jj >= kDnBlocks * TL) break;
      f32x4 sum = red[0][c][j][lane];
#pragma unroll
      for (int w = 1; w < SPLIT; ++w) sum += red[w][c][j][lane];
      const int n = n0 + 16 * jj + m;
#pragma unroll
      for (int i = 0; i < 4; ++i)  // lane (n, q) holds rows 4q .. 4q+3 of the pass
        if (n < H && 4 * q + i < nt)
          st_agent(reinterpret_cast<uint32_t*>(staging) + (size_t)slot_i[i] * H + n,
                   __float_as_uint(sum[i] * wt_i[i]) ^ kStageKey);
    }
    __syncthreads();
  }
  // The last active group's workgroup of the tile adds the tile's rows once they are all
  // there (a word is 0 until its row is written; the others need not wait for their stores).
  if (!combiner) return;
  // The slots of an output are read 8 at a time with their loads issued together; a word
  // still 0 is polled again on its own.
  const uint32_t* st = reinterpret_cast<const uint32_t*>(staging);
  const int ns = k + S;
  for (int i = threadIdx.x; i < T * kDnCols; i += (64 * SPLIT)) {
    const int t = i / kDnCols, n = n0 + i % kDnCols;
    if (n >= H) continue;
    float sacc = 0.f;
    for (int j0 = 0; j0 < ns; j0 += 8) {
      uint32_t wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const size_t slot = j < S ? (size_t)tk + t : (size_t)t * k + (j - S);
        wv[u] = j < ns ? ld_agent(st + slot * H + n) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j >= ns) break;
        uint32_t w = wv[u];
        if (w == 0u) {
          const size_t slot = j < S ? (size_t)tk + t : (size_t)t * k + (j - S);
          for (int round = 0; w == 0u && round < kFlagPolls; ++round) {
            __builtin_amdgcn_s_sleep(1);
            w = ld_agent(st + slot * H + n);
          }
        }
        const float v = __uint_as_float(w ^ kStageKey);
        sacc = j == 0 ? v : sacc + v;
      }
    }
    y[(size_t)t * H + n] = sacc;
  }
}

// FP8: the FP8 shared expert alone (launched after the FP4 kernel, so every routed row is in
// staging), each workgroup also combining its tile.  Otherwise the FP4 groups, skipping
// skip_group, the last slot's workgroups combining.  A routed row's weight is its routing
// weight times routed_scale.
template <int TL, bool FP8, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT, SPLIT <= 4 ? 8 / SPLIT : 1) void gemv_down_kernel(DOWN_ARGS) {
  __shared__ f32x4 red[SPLIT][kDnBlocks][TL][64];
  down_tile<TL, FP8, SPLIT>(red, blockIdx.x, blockIdx.y, 1, DOWN_PASS);
}

// The FP4 groups and an FP8 shared expert in one launch: the first TL/2 rows of the grid are the
// FP8 expert's 32-column tiles (dispatched first), the rest the FP4 active-group slots, whose last
// routed slot combines (the shared expert's FP4 slot is skip_group, the last slot).
template <int TL, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT, SPLIT <= 4 ? 8 / SPLIT : 1) void gemv_down_mixed_kernel(DOWN_ARGS) {
  __shared__ f32x4 red[SPLIT][kDnBlocks][TL][64];
  constexpr int n8 = TL / 2;
  if ((int)blockIdx.y < n8)
    down_tile<2, true, SPLIT>(reinterpret_cast<f32x4(*)[kDnBlocks][2][64]>(red), blockIdx.y * gridDim.x + blockIdx.x,
                              0, 0, DOWN_PASS);
  else
    down_tile<TL, false, SPLIT>(red, blockIdx.x, blockIdx.y - n8, 2, DOWN_PASS);
}

// ------------------------------------------------------------------------------------
// Few active groups (small batches) get narrower column tiles per workgroup, so the grid
// still covers the GPU several times over.
constexpr int kMinGemvGroups = 512;

hipError_t launch_gemv_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int max_act, hipStream_t s) {
  (void)x;
  const int R = T * (d.K + d.S);
  const bool narrow = (size_t)max_act * ((d.I + 63) / 64) < kMinGemvGroups;
  const int cols = narrow ? 32 : 64;
  const int tk = timing_begin("gemv_gateup", s);
  uint32_t* clear = reinterpret_cast<uint32_t*>(b.staging);
  uint8_t* h = static_cast<uint8_t*>(b.h);
  if (!d.fp8_shared) {
    auto kern = narrow ? gemv_gateup_kernel<2, kSplit, false> : gemv_gateup_kernel<4, kSplit, false>;
    kern<<<dim3((d.I + cols - 1) / cols, max_act), 64 * kSplit, 0, s>>>(
        b.xq, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, nullptr, nullptr, nullptr, nullptr, b.perm,
        b.grec, h, clear, -1, T, d.K, d.H, d.I, R);
  } else {
    // the FP8 shared expert's 32-column tiles (cols/32 grid rows) ahead of the FP4 slots, whose
    // shared-expert slot is skipped
    auto kern = narrow ? gemv_gateup_mixed_kernel<2, kSplit> : gemv_gateup_mixed_kernel<4, kSplit>;
    kern<<<dim3(d.I / cols, max_act + cols / 32), 64 * kSplit, 0, s>>>(
        b.xq, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, w.shared_gate_fp8, w.shared_gate_fp8_scales,
        w.shared_up_fp8, w.shared_up_fp8_scales, b.perm, b.grec, h, clear, d.E, T, d.K, d.H, d.I, R);
  }
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, float* y, int T,
                            int max_act, hipStream_t s) {
  const int R = T * (d.K + d.S);
  // (narrower down tiles measured slower: a down workgroup's bytes are already few)
  constexpr int kCols = kDnBlocks * 16 * 4;
  const int tk = timing_begin("gemv_down", s);
  const uint8_t* h = static_cast<const uint8_t*>(b.h);
  if (!d.fp8_shared) {
    gemv_down_kernel<4, false, kDnSplit><<<dim3((d.H + kCols - 1) / kCols, max_act), 64 * kDnSplit, 0, s>>>(
        h, w.down_codes, w.down_scales, nullptr, nullptr, b.perm, b.row_w, b.grec, b.staging, y, -1, d.routed_scale,
        T, d.K, d.S, d.H, d.I, R);
  } else {
    // the FP8 shared expert's 32-column tiles (two grid rows) ahead of the FP4 slots; the last
    // routed slot's workgroups combine
    gemv_down_mixed_kernel<4, kDnSplit><<<dim3(d.H / kCols, max_act + 2), 64 * kDnSplit, 0, s>>>(
        h, w.down_codes, w.down_scales, w.shared_down_fp8, w.shared_down_fp8_scales, b.perm, b.row_w, b.grec,
        b.staging, y, d.E, d.routed_scale, T, d.K, d.S, d.H, d.I, R);
  }
  timing_end(tk, s);
  return hipGetLastError();
}

}  // namespace moe
