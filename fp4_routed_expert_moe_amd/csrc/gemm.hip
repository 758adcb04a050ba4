// Prefill path: expert-grouped GEMM over the sorted token rows on the block-scaled matrix
// cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine" (PR #1055, "What it is",
// prefill MoE) runs expert-grouped GEMM rows after routing on the device.  Here:
//
// * Weights (B) enter the matrix cores as stored: e2m1 codes with their e8m0 block scales, no
//   convert instruction touches them.  Each wave loads its own weight operands from the
//   block-interleaved kernel layout straight into registers, one K step ahead.
// * Activations (A) are exact FP8 (e4m3) term splits with an e8m0 scale per 32 values: x as
//   two terms (all 8 bf16 significand bits, written by the router kernel), h as two terms
//   (about 8 significant bits, the precision of bf16) written by the gate/up epilogue.  One
//   MFMA per term, all accumulating in fp32.
// * A workgroup takes one M-tile (64 grouped rows of one group, from the device-built M-tile
//   list) and 256 output columns.  Its four waves each own 64 columns of all 64 rows: 4 x 4
//   16x16 tiles, for gate and up at once in the gate/up kernel, so SwiGLU stays in registers.
//   The activation tile of each 256-value K step is staged in LDS (double-buffered) and read
//   by all four waves; 16-row subtiles past the group's last row are skipped.
// * Workgroup b takes N-tile b % NT of M-tile b / NT.  Workgroups reach the 8 XCDs
//   round-robin, so when NT is a multiple of 8 every XCD streams a fixed slice of columns of
//   every expert and no expert's weight tile is fetched by two XCDs.
#include "common.h"

namespace moe {

constexpr int kPM = kGemmBM;      // rows per M-tile (64)
constexpr int kPNW = 64;          // output columns per wave
constexpr int kPN = 4 * kPNW;     // output columns per workgroup
constexpr int kPU = 2;            // MFMA K chunks (128 values each) per step
constexpr int kPK = 128 * kPU;    // K values per step
constexpr int kPKB = kPK / 32;    // K blocks per step
constexpr int kALd = kPK + 16;    // LDS row pitch of the activation tile (bytes)

struct ATile {                    // one K step of the activation tile
  uint8_t v[2][kPM][kALd];        // FP8 terms
  uint8_t s[kPM][kPKB];           // e8m0 scales of the step's K blocks
};

// Activation rows: term planes hi/lo [rows][K] bytes and scales [rows][K/32].
struct ARows {
  const uint8_t* hi;
  const uint8_t* lo;
  const uint8_t* sc;
  int K;
};

// Thread t of 256 moves K blocks u*4 + p (u < kPU, p = t%4) of K step `step` of tile row t/4,
// both terms and scales, into LDS.  `src_row` < 0 marks a row past the group: zeros with
// scale 127 (as are blocks past K).
struct AStage {
  uint4 c[kPU][4];
  uint32_t s[kPU];
};
__device__ __forceinline__ AStage a_fetch(const ARows& a, int src_row, int step, int p) {
  AStage st;
  const int KB = a.K >> 5;
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int u = 0; u < kPU; ++u) {
    const int blk = step * kPKB + 4 * u + p;
    const bool ok = src_row >= 0 && blk < KB;
    const size_t o = (size_t)src_row * a.K + 32 * blk;
    st.c[u][0] = ok ? ld16(a.hi + o) : z;
    st.c[u][1] = ok ? ld16(a.hi + o + 16) : z;
    st.c[u][2] = ok ? ld16(a.lo + o) : z;
    st.c[u][3] = ok ? ld16(a.lo + o + 16) : z;
    st.s[u] = ok ? a.sc[(size_t)src_row * KB + blk] : 127u;
  }
  return st;
}
__device__ __forceinline__ void a_store(ATile& t, const AStage& st, int r, int p) {
#pragma unroll
  for (int u = 0; u < kPU; ++u) {
    const int b = 128 * u + 32 * p;
    *reinterpret_cast<uint4*>(&t.v[0][r][b]) = st.c[u][0];
    *reinterpret_cast<uint4*>(&t.v[0][r][b + 16]) = st.c[u][1];
    *reinterpret_cast<uint4*>(&t.v[1][r][b]) = st.c[u][2];
    *reinterpret_cast<uint4*>(&t.v[1][r][b + 16]) = st.c[u][3];
    t.s[r][4 * u + p] = (uint8_t)st.s[u];
  }
}

// Weight operands of one wave for one K step: kPU chunks x NM matrices x 4 column tiles.
template <int NM>
struct BFrag {
  uint4 c[kPU][NM][4];
  int s[kPU][NM][4];
};
template <int NM>
__device__ __forceinline__ void b_fetch(BFrag<NM>& f, const uint8_t* const* codes, const uint8_t* const* scales,
                                        const size_t* col, int N, int KB, int step, int q) {
#pragma unroll
  for (int u = 0; u < kPU; ++u) {
    const int kb = step * kPKB + 4 * u + q;
    const bool ok = kb < KB;
#pragma unroll
    for (int mtx = 0; mtx < NM; ++mtx)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const size_t o = (size_t)kb * N + col[c];
        f.c[u][mtx][c] = ok ? ld16(codes[mtx] + o * 16) : make_uint4(0, 0, 0, 0);
        f.s[u][mtx][c] = ok ? scales[mtx][o] : 127;
      }
  }
}

// One K step: acc[mtx][rs][c] += A(rs) x B(mtx, c) for both FP8 terms, rs < nsub.
template <int NM>
__device__ __forceinline__ void k_step(const ATile& t, const BFrag<NM>& f, f32x4 (&acc)[NM][4][4], int nsub, int m,
                                       int q) {
#pragma unroll
  for (int u = 0; u < kPU; ++u)
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      if (rs >= nsub) break;
      const int r = 16 * rs + m;
      const int b = 128 * u + 16 * q;
      const i32x8 a0 = fp8_operand(*reinterpret_cast<const uint4*>(&t.v[0][r][b]),
                                   *reinterpret_cast<const uint4*>(&t.v[0][r][b + 64]));
      const i32x8 a1 = fp8_operand(*reinterpret_cast<const uint4*>(&t.v[1][r][b]),
                                   *reinterpret_cast<const uint4*>(&t.v[1][r][b + 64]));
      const int sa = t.s[r][4 * u + q];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int mtx = 0; mtx < NM; ++mtx) {
          const i32x8 bb = fp4_operand(f.c[u][mtx][c]);
          acc[mtx][rs][c] = mma_f8f4(a0, bb, acc[mtx][rs][c], sa, f.s[u][mtx][c]);
          acc[mtx][rs][c] = mma_f8f4(a1, bb, acc[mtx][rs][c], sa - 4, f.s[u][mtx][c]);
        }
    }
}

// ------------------------------------------------------------------------------------
// GATEUP: h[r][n] = silu(x_t(r) . Wg[n]) * (x_t(r) . Wu[n]) as 2 FP8 terms + e8m0 per 32
//         (h8 = [2][R][I] bytes then [R][I/32] scales).
// DOWN:   staging[slot(r)][n] = weight(r) * (h_r . Wd[n]).
// ------------------------------------------------------------------------------------
template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f8f4_kernel(
    ARows a, const uint8_t* __restrict__ c0p, const uint8_t* __restrict__ s0p, const uint8_t* __restrict__ c1p,
    const uint8_t* __restrict__ s1p, const int32_t* __restrict__ perm, const float* __restrict__ wts,
    const int32_t* __restrict__ info, const int32_t* __restrict__ mt_group, const int32_t* __restrict__ mt_row0,
    const int32_t* __restrict__ grp_row0, const int32_t* __restrict__ grp_rows, uint8_t* __restrict__ h8,
    float* __restrict__ staging, int T, int k, int N, int R, int NT) {
  constexpr int NM = GATEUP ? 2 : 1;
  __shared__ ATile tile[2];
  const int mt = blockIdx.x / NT, nt = blockIdx.x - mt * NT;
  if (mt >= info[1]) return;
  const int g = mt_group[mt];
  const int r0 = grp_row0[g] + mt_row0[mt];          // first grouped row of the tile
  const int nrows = min(kPM, grp_rows[g] - mt_row0[mt]);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, q = lane >> 4;
  const int tk = T * k;
  const int KB = a.K >> 5;
  const int nsteps = (a.K + kPK - 1) / kPK;

  // the activation row this thread stages
  const int lr = tid >> 2, lp = tid & 3;
  int src = -1;
  if (lr < nrows) src = GATEUP ? row_token(perm, r0 + lr, tk, k) : r0 + lr;

  // this wave's weight columns (clamped; stores are masked)
  const int n0 = nt * kPN + wave * kPNW;
  const size_t gbase = (size_t)g * KB * N;
  size_t col[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) col[c] = gbase + min(n0 + 16 * c + m, N - 1);
  const uint8_t* codes[2] = {c0p, c1p};
  const uint8_t* scales[2] = {s0p, s1p};
  const int nsub = (nrows + 15) >> 4;

  f32x4 acc[NM][4][4];
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx)
#pragma unroll
    for (int rs = 0; rs < 4; ++rs)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[mtx][rs][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  BFrag<NM> fb[2];
  a_store(tile[0], a_fetch(a, src, 0, lp), lr, lp);
  b_fetch<NM>(fb[0], codes, scales, col, N, KB, 0, q);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    // even step: compute from tile[0] / fb[0], prefetch step s+1 into tile[1] / fb[1]
    {
      const bool more = s + 1 < nsteps;
      AStage st;
      if (more) {
        st = a_fetch(a, src, s + 1, lp);
        b_fetch<NM>(fb[1], codes, scales, col, N, KB, s + 1, q);
      }
      k_step<NM>(tile[0], fb[0], acc, nsub, m, q);
      if (more) a_store(tile[1], st, lr, lp);
      __syncthreads();
      if (!more) break;
    }
    // odd step
    {
      const bool more = s + 2 < nsteps;
      AStage st;
      if (more) {
        st = a_fetch(a, src, s + 2, lp);
        b_fetch<NM>(fb[0], codes, scales, col, N, KB, s + 2, q);
      }
      k_step<NM>(tile[1], fb[1], acc, nsub, m, q);
      if (more) a_store(tile[0], st, lr, lp);
      __syncthreads();
    }
  }

  // ---- epilogue ----
  if constexpr (GATEUP) {
    uint8_t* h_lo = h8 + (size_t)R * N;
    uint8_t* hs = h8 + (size_t)2 * R * N;
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      if (rs >= nsub) break;
#pragma unroll
      for (int p = 0; p < 2; ++p) {  // 32-column block = column tiles 2p, 2p+1
        const int nb = n0 + 32 * p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lrow = 16 * rs + 4 * q + i;
          float hv[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) hv[c] = silu(acc[0][rs][2 * p + c][i]) * acc[1][rs][2 * p + c][i];
          // lanes with the same q hold the same row: |h| max over the block's 32 columns
          float amax = fmaxf(fabsf(hv[0]), fabsf(hv[1]));
#pragma unroll
          for (int msk = 1; msk < 16; msk <<= 1) amax = fmaxf(amax, __shfl_xor(amax, msk, 64));
          const int sc = fp8_block_scale(amax);
          const float inv = fp8_inv_scale(sc);
          if (lrow < nrows && nb < N) {
            const size_t r = (size_t)(r0 + lrow);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const float v = hv[c] * inv;
              const uint32_t t0 = fp8_of(v);
              const uint32_t t1 = fp8_of((v - f32_of_fp8(t0)) * 16.f);
              const size_t o = r * N + nb + 16 * c + m;
              h8[o] = (uint8_t)t0;
              h_lo[o] = (uint8_t)t1;
            }
            if (m == 0) hs[r * (N >> 5) + (nb >> 5)] = (uint8_t)sc;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      if (rs >= nsub) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lrow = 16 * rs + 4 * q + i;
        if (lrow >= nrows) continue;
        const int rr = r0 + lrow;
        const int slot = rr < tk ? perm[rr] : rr;
        const float wt = rr < tk ? wts[slot] : 1.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int n = n0 + 16 * c + m;
          if (n < N) staging[(size_t)slot * N + n] = acc[0][rs][c][i] * wt;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
hipError_t launch_gemm_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int mt_bound, hipStream_t s) {
  (void)x;
  const int NT = (d.I + kPN - 1) / kPN;
  const int R = T * (d.K + d.S);
  const ARows a{b.xq, b.xq + (size_t)T * d.H, b.xq + (size_t)2 * T * d.H, d.H};
  const int tk = timing_begin("gemm_gateup", s);
  gemm_f8f4_kernel<true><<<mt_bound * NT, 256, 0, s>>>(a, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales,
                                                       b.perm, b.w, b.info, b.mt_group, b.mt_row0, b.grp_row0,
                                                       b.grp_rows, static_cast<uint8_t*>(b.h), nullptr, T, d.K, d.I,
                                                       R, NT);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int mt_bound,
                            hipStream_t s) {
  const int NT = (d.H + kPN - 1) / kPN;
  const int R = T * (d.K + d.S);
  const uint8_t* h8 = static_cast<const uint8_t*>(b.h);
  const ARows a{h8, h8 + (size_t)R * d.I, h8 + (size_t)2 * R * d.I, d.I};
  const int tk = timing_begin("gemm_down", s);
  gemm_f8f4_kernel<false><<<mt_bound * NT, 256, 0, s>>>(a, w.down_codes, w.down_scales, w.down_codes, w.down_scales,
                                                        b.perm, b.w, b.info, b.mt_group, b.mt_row0, b.grp_row0,
                                                        b.grp_rows, nullptr, b.staging, T, d.K, d.H, R, NT);
  timing_end(tk, s);
  return hipGetLastError();
}

}  // namespace moe
