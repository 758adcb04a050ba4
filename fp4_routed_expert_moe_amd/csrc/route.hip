// Routing on the device: router scores, top-k with renormalised softmax weights, and the
// stable token->expert grouping (counts, offsets, perm) plus the tables the expert kernels
// read (active groups for the GEMV path, M-tiles for the grouped GEMM).
//
// "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine" (PR #1055, "What it is",
// prefill MoE) routes on the device and feeds expert-grouped GEMM rows; the pages leave the
// scoring rule open, so scores are a plain fp32 dot product (+ optional bias), selection is
// the k largest (ties to the lower index), and the weights are a softmax over the k selected
// scores.
//
// Small batches (route_fused: T <= 64 and T*E <= kTailScores) are routed in one launch: the
// router workgroups publish their scores, and the last one to finish (device-scope counter
// in the workspace, left at zero again) runs top-k, the grouping tables and the scatter.
// Larger batches use a per-chunk top-k kernel, a one-workgroup scan and a per-chunk scatter.
#include "common.h"

namespace moe {

constexpr int kRouterTT = 8;  // tokens per router workgroup

// ------------------------------------------------------------------------------------
// Activations as two exact FP8 terms with a scale per 32-value block (the decode kernels'
// A operand): xq = [2][T][H] e4m3 bytes, then [T][H/32] e8m0 scales.
// ------------------------------------------------------------------------------------
__device__ void quantize_x_block(const uint16_t* __restrict__ src, uint8_t* __restrict__ hi,
                                 uint8_t* __restrict__ lo, uint8_t* __restrict__ sc) {
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = reinterpret_cast<const uint4*>(src)[i];
  const uint32_t* w = reinterpret_cast<const uint32_t*>(raw);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  const int s = fp8_block_scale(amax);
  const float inv = fp8_inv_scale(s);
  uint32_t th[8], tl[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[4] = {bf16_lo(w[2 * i]) * inv, bf16_hi(w[2 * i]) * inv, bf16_lo(w[2 * i + 1]) * inv,
                  bf16_hi(w[2 * i + 1]) * inv};
    th[i] = pack_fp8x4(v[0], v[1], v[2], v[3]);
    float r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (v[j] - f32_of_fp8((th[i] >> (8 * j)) & 0xFFu)) * 16.f;
    tl[i] = pack_fp8x4(r[0], r[1], r[2], r[3]);
  }
  reinterpret_cast<uint4*>(hi)[0] = make_uint4(th[0], th[1], th[2], th[3]);
  reinterpret_cast<uint4*>(hi)[1] = make_uint4(th[4], th[5], th[6], th[7]);
  reinterpret_cast<uint4*>(lo)[0] = make_uint4(tl[0], tl[1], tl[2], tl[3]);
  reinterpret_cast<uint4*>(lo)[1] = make_uint4(tl[4], tl[5], tl[6], tl[7]);
  *sc = (uint8_t)s;
}

// ------------------------------------------------------------------------------------
// Top-k of one token by one wave.
// Each score becomes a 64-bit rank key: high word = order-preserving image of the float
// (+1, so that NaN -> 1 still beats an excluded entry, which is 0), low word = ~index so
// that equal scores prefer the lower expert.  -0 is ranked as +0.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  const uint32_t ord = v != v ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return ((uint64_t)ord + 1ull) << 32 | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
// The score whose key has high word `hi` (-0 comes back as +0).
__device__ __forceinline__ float hi_value(uint32_t hi) {
  const uint32_t ord = hi - 1u;
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Lane l owns experts l, l + 64, ...  (Q = scores per lane, E <= 64*Q).  Each round finds
// the largest remaining key: the wave-wide maximum of the high words on DPP, then the low
// word of the one lane that holds it (a second reduction only when several lanes tie).
// Every pick is wave-uniform, so the per-round bookkeeping is scalar.  At the end the wave
// writes idx[0..k) and w[0..k) of the token (softmax over the k picked scores, summed in a
// fixed order), sets bit `tbit` of mask[e] for each pick and copies the picks to sel when
// sel is not NULL.
template <int Q>
__device__ __forceinline__ void topk_wave(const float* row, int E, int k, int32_t* __restrict__ idx_out,
                                          float* __restrict__ w_out, uint64_t* mask, int tbit, uint16_t* sel) {
  const int lane = threadIdx.x & 63;
  float val[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    val[q] = row[e < E ? e : 0];
  }
  uint64_t key[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    key[q] = e < E ? rank_key(val[q], e) : 0ull;
  }
  int selE[Q];
  float selV[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    selE[q] = 0;
    selV[q] = 0.f;
  }
  float vtop = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int q = 1; q < Q; ++q) m = key[q] > m ? key[q] : m;
    const uint32_t mhi = (uint32_t)(m >> 32), mlo = (uint32_t)m;
    const uint32_t bhi = wave_max_u32(mhi);
    const uint64_t tied = __ballot(mhi == bhi);
    uint32_t blo;
    if (__popcll(tied) == 1)
      blo = __builtin_amdgcn_readlane(mlo, __ffsll((unsigned long long)tied) - 1);
    else
      blo = wave_max_u32(mhi == bhi ? mlo : 0u);
    const int e = (int)(0xFFFFFFFFu - blo);
    const float v = hi_value(bhi);
    if (j == 0) vtop = v;
    const bool owner = (e & 63) == lane;
    const int qe = e >> 6;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (q == qe) key[q] = owner ? 0ull : key[q];
    const bool rec = (j & 63) == lane;
    const int qj = j >> 6;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (q == qj) {
        selE[q] = rec ? e : selE[q];
        selV[q] = rec ? v : selV[q];
      }
  }
  float p[Q];
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = lane + 64 * q;
    p[q] = 0.f;
    if (j < k) {
      p[q] = expf(selV[q] - vtop);
      s += p[q];
    }
  }
  s = wave_sum_f32(s);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = lane + 64 * q;
    if (j < k) {
      idx_out[j] = selE[q];
      w_out[j] = p[q] / s;
      atomicOr(reinterpret_cast<unsigned long long*>(&mask[selE[q]]), 1ull << tbit);
      if (sel) sel[j] = (uint16_t)selE[q];
    }
  }
}

// Tokens [0, T) of scores [T][E] (T <= 64), one token per wave at a time over the NT
// threads of the block.  Token t sets bit t of the expert masks; its picks go to
// sel[t*k ..] when sel != NULL.
template <int NT, int Q>
__device__ __forceinline__ void topk_block(const float* scores, int T, int E, int k, int32_t* idx, float* w,
                                           uint64_t* mask, uint16_t* sel) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t = wave; t < T; t += NT / 64)
    topk_wave<Q>(scores + (size_t)t * E, E, k, idx + (size_t)t * k, w + (size_t)t * k, mask, t,
                 sel ? sel + t * k : nullptr);
}
template <int NT>
__device__ __forceinline__ void topk_block_any(const float* scores, int T, int E, int k, int32_t* idx, float* w,
                                               uint64_t* mask, uint16_t* sel) {
  if (E <= 64)
    topk_block<NT, 1>(scores, T, E, k, idx, w, mask, sel);
  else if (E <= 128)
    topk_block<NT, 2>(scores, T, E, k, idx, w, mask, sel);
  else if (E <= 256)
    topk_block<NT, 4>(scores, T, E, k, idx, w, mask, sel);
  else if (E <= 512)
    topk_block<NT, 8>(scores, T, E, k, idx, w, mask, sel);
  else
    topk_block<NT, 16>(scores, T, E, k, idx, w, mask, sel);
}

// ------------------------------------------------------------------------------------
// Grouping tables, built by one wave (no block barriers) from per-expert row counts
// cnt[0..E) in LDS.  Lane l owns experts [l*J, l*J+J), J = ceil(E/64).  Writes counts,
// offsets, group rows/first rows, the active-group list (shared expert last), the M-tile
// list, and each expert's first grouped row to offs[] (LDS; may be the same array as cnt).
// ------------------------------------------------------------------------------------
// Exclusive prefix sum over the wave on DPP: row_shr 1, 2, 4, 8 scans each 16-lane row, then
// row_bcast 15 and 31 carry the row totals into the rows above (checked lane by lane on the
// device against a serial sum).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWMASK, 0xF, false);
}
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  int x = v;
  x = dpp_add<0x111, 0xF>(x);  // row_shr:1
  x = dpp_add<0x112, 0xF>(x);  // row_shr:2
  x = dpp_add<0x114, 0xF>(x);  // row_shr:4
  x = dpp_add<0x118, 0xF>(x);  // row_shr:8
  x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  *total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

__device__ void build_tables_wave(const int* cnt, int T, int E, int k, int S, const CallBufs& b, int* offs) {
  const int lane = threadIdx.x & 63;
  const int J = (E + 63) >> 6;
  const int e0 = lane * J;
  int rows = 0, acts = 0, mts = 0;
  for (int i = 0; i < J; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int c = cnt[e];
      rows += c;
      acts += c > 0;
      mts += (c + kGemmBM - 1) / kGemmBM;
    }
  }
  int total, nact, nmt;
  int off = wave_excl_scan(rows, &total);
  int apos = wave_excl_scan(acts, &nact);
  int mpos = wave_excl_scan(mts, &nmt);
  for (int i = 0; i < J; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int c = cnt[e];
    b.counts[e] = c;
    b.offsets[e] = off;
    b.grp_row0[e] = off;
    b.grp_rows[e] = c;
    offs[e] = off;
    off += c;
    if (c > 0) b.act[apos++] = e;
    for (int m = 0; m < (c + kGemmBM - 1) / kGemmBM; ++m) {
      b.mt_group[mpos] = e;
      b.mt_row0[mpos++] = m * kGemmBM;
    }
  }
  const int mt_shared = S ? (T + kGemmBM - 1) / kGemmBM : 0;
  for (int i = lane; i < mt_shared; i += 64) {
    b.mt_group[nmt + i] = E;
    b.mt_row0[nmt + i] = i * kGemmBM;
  }
  if (lane == 0) {
    b.offsets[E] = total;
    if (S) {
      b.grp_row0[E] = T * k;
      b.grp_rows[E] = T;
      b.act[nact] = E;
    }
    b.info[0] = nact + S;
    b.info[1] = nmt + mt_shared;
  }
}

// ------------------------------------------------------------------------------------
// The routing tail of a small batch (route_fused), run by the router kernel's last
// workgroup once every score is published: top-k, grouping tables, stable scatter.
// ------------------------------------------------------------------------------------
constexpr int kTailThreads = 1024;

__device__ __forceinline__ void route_tail(const CallBufs& b, int T, int E, int K, int S) {
  __shared__ float sc[kTailScores];
  __shared__ uint16_t sel[kTailScores];  // picks of token t at [t*K, t*K+K); T*K <= T*E
  __shared__ uint64_t mask[1024];        // bit t: token t picked expert e
  __shared__ int offs[1024];
  const int tid = threadIdx.x;
  const int n = T * E;
  // every score in one round of loads, then into LDS
  for (int i0 = 0; i0 < n; i0 += kTailThreads * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kTailThreads + tid;
      v[u] = i < n ? ld_agent(b.logits + i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kTailThreads + tid;
      if (i < n) sc[i] = v[u];
    }
  }
  for (int i = tid; i < E; i += kTailThreads) mask[i] = 0ull;
  __syncthreads();
  topk_block_any<kTailThreads>(sc, T, E, K, b.idx, b.w, mask, sel);
  __syncthreads();
  for (int i = tid; i < E; i += kTailThreads) offs[i] = __popcll(mask[i]);
  __syncthreads();
  if (tid < 64) build_tables_wave(offs, T, E, K, S, b, offs);
  __syncthreads();
  // pick i = t*K + j lands after the rows of lower tokens routed to the same expert
  for (int i = tid; i < T * K; i += kTailThreads) {
    const int t = i / K, e = sel[i];
    b.perm[offs[e] + __popcll(mask[e] & ((1ull << t) - 1ull))] = i;
  }
}

// ------------------------------------------------------------------------------------
// Small batches: router scores l[t][e] = x[t] . W_r[e] + b[e] (fp32 accumulate, bf16
// activations) and the routing tail in one launch.  One workgroup of NT threads per (expert,
// tile of kRouterTT tokens): the threads split the hidden axis (8 values each per step);
// partial sums are added in ascending hidden order per thread, across each wave, then over
// the waves in a fixed order, so a score does not depend on the other tokens of the batch.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kTailThreads) void router_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ wr,
                                                             const float* __restrict__ bias, CallBufs b, int T,
                                                             int E, int H, int K, int S, int quantize) {
  constexpr int NT = kTailThreads;
  constexpr int NW = NT / 64;
  constexpr int U = 1;
  __shared__ float part[NW][kRouterTT];
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterTT;
  const int nt = min(kRouterTT, T - t0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (quantize) {
    // the token tile's nt*KB blocks, an equal slice per expert workgroup (a few per workgroup)
    const int KB = H >> 5;
    const int nb = nt * KB, per = (nb + E - 1) / E;
    uint8_t* xq = b.xq;
    for (int j = e * per + tid; j < min(nb, (e + 1) * per); j += NT) {
      const int t = t0 + j / KB, bb = j % KB;
      quantize_x_block(x + (size_t)t * H + bb * 32, xq + (size_t)t * H + bb * 32,
                       xq + (size_t)(T + t) * H + bb * 32, xq + (size_t)2 * T * H + (size_t)t * KB + bb);
    }
  }
  float acc[kRouterTT];
#pragma unroll
  for (int i = 0; i < kRouterTT; ++i) acc[i] = 0.f;
  const float* wrow = wr + (size_t)e * H;
  const uint16_t* xt = x + (size_t)t0 * H;
  for (int h0 = tid * 8; h0 < H; h0 += NT * 8 * U) {  // H % 32 == 0, so h + 8 <= H
    float4 w[U][2];
    uint4 xv[U][kRouterTT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int h = h0 + u * NT * 8;
      if (h < H) {
        w[u][0] = *reinterpret_cast<const float4*>(wrow + h);
        w[u][1] = *reinterpret_cast<const float4*>(wrow + h + 4);
#pragma unroll
        for (int i = 0; i < kRouterTT; ++i)
          if (i < nt) xv[u][i] = *reinterpret_cast<const uint4*>(xt + (size_t)i * H + h);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (h0 + u * NT * 8 < H) {
        const float4 w0 = w[u][0], w1 = w[u][1];
#pragma unroll
        for (int i = 0; i < kRouterTT; ++i) {
          if (i < nt) {
            const uint4 v = xv[u][i];
            float a = acc[i];
            a = fmaf(bf16_lo(v.x), w0.x, a);
            a = fmaf(bf16_hi(v.x), w0.y, a);
            a = fmaf(bf16_lo(v.y), w0.z, a);
            a = fmaf(bf16_hi(v.y), w0.w, a);
            a = fmaf(bf16_lo(v.z), w1.x, a);
            a = fmaf(bf16_hi(v.z), w1.y, a);
            a = fmaf(bf16_lo(v.w), w1.z, a);
            a = fmaf(bf16_hi(v.w), w1.w, a);
            acc[i] = a;
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRouterTT; ++i) {
    const float v = wave_sum_f32(acc[i]);
    if (lane == 0) part[wave][i] = v;
  }
  __syncthreads();
  if (tid < nt) {
    float v = part[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += part[w][tid];
    st_agent(b.logits + (size_t)(t0 + tid) * E + e, v + (bias ? bias[e] : 0.f));
  }
  // the last workgroup to finish routes the whole batch, then re-arms the counter
  __shared__ int is_last;
  if (!arrive_last(&b.ctrl[0], (int)(gridDim.x * gridDim.y), &is_last)) return;
  route_tail(b, T, E, K, S);
  if (tid == 0) reset_counter(&b.ctrl[0]);
}

// ------------------------------------------------------------------------------------
// Larger batches: router scores on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
// W_r (fp32) is split on the fly into three bf16 terms whose sum is exactly W_r: the top,
// middle and low 8 bits of the 24-bit significand, each remainder exact (it is the float
// minus its own truncation).  x (bf16) times each term is exact in fp32, so a score is the
// fp32 dot product up to summation order, which is fixed per (token, expert).  64 tokens x
// 64 experts per workgroup, 32 x 32 per wave (2 x 2 MFMA tiles, three terms each).
// Operand layout: lane l holds row (token or expert) l % 16, K values 8*(l/16) .. +8 of each
// 32-value step; result lane l, element i -> token 4*(l/16) + i, expert l % 16.
// ------------------------------------------------------------------------------------
constexpr int kRouterGemmTile = 64;

__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {  // (bf16 of a) | (bf16 of b) << 16
  return (a >> 16) | (b & 0xFFFF0000u);
}
// 8 consecutive fp32 weights -> three bf16x8 terms with t0 + t1 + t2 == w exactly.
__device__ __forceinline__ void split3(const float4& p, const float4& r, bf16x8 (&t)[3]) {
  uint32_t w[8] = {__float_as_uint(p.x), __float_as_uint(p.y), __float_as_uint(p.z), __float_as_uint(p.w),
                   __float_as_uint(r.x), __float_as_uint(r.y), __float_as_uint(r.z), __float_as_uint(r.w)};
  uint32_t u[3][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = w[i] & 0xFFFF0000u;
    const float r1 = __uint_as_float(w[i]) - __uint_as_float(a);
    const uint32_t b = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(b);  // at most 8 significant bits: exact in bf16
    u[0][i] = a;
    u[1][i] = b;
    u[2][i] = __float_as_uint(r2);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const uint4 v = make_uint4(hi_halves(u[j][0], u[j][1]), hi_halves(u[j][2], u[j][3]),
                               hi_halves(u[j][4], u[j][5]), hi_halves(u[j][6], u[j][7]));
    t[j] = __builtin_bit_cast(bf16x8, v);
  }
}

__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int T, int E, int H) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * kRouterGemmTile + (wave & 1) * 32;
  const int e0 = blockIdx.y * kRouterGemmTile + (wave >> 1) * 32;
  const uint16_t* xa[2];
  const float* wb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xa[i] = x + (size_t)min(t0 + 16 * i + r, T - 1) * H + 8 * kq;
    wb[i] = wr + (size_t)min(e0 + 16 * i + r, E - 1) * H + 8 * kq;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;  // 32-value K steps loaded together
  for (int k0 = 0; k0 < H; k0 += 32 * U) {
    uint4 xr[U][2];
    float4 wv[U][2][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 32 * u;
      if (k < H) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          xr[u][i] = *reinterpret_cast<const uint4*>(xa[i] + k);
          wv[u][i][0] = *reinterpret_cast<const float4*>(wb[i] + k);
          wv[u][i][1] = *reinterpret_cast<const float4*>(wb[i] + k + 4);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + 32 * u >= H) break;
      bf16x8 bt[2][3];
#pragma unroll
      for (int j = 0; j < 2; ++j) split3(wv[u][j][0], wv[u][j][1], bt[j]);
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xr[u][i]), bt[j][t],
                                                                acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + 16 * j + r;
      if (e >= E) continue;
      const float be = bias ? bias[e] : 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 16 * i + 4 * kq + v;
        if (t < T) logits[(size_t)t * E + e] = acc[i][j][v] + be;
      }
    }
}

// FP8 term split of x for the expert kernels (larger batches; small ones do it in the
// router kernel): one thread per 32-value block.
__global__ __launch_bounds__(256) void quantize_x_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                         int T, int H) {
  const int KB = H >> 5;
  const size_t j = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= (size_t)T * KB) return;
  const size_t t = j / KB, bb = j % KB;
  quantize_x_block(x + t * H + bb * 32, xq + t * H + bb * 32, xq + ((size_t)T + t) * H + bb * 32,
                   xq + (size_t)2 * T * H + t * KB + bb);
}

// ------------------------------------------------------------------------------------
// Any T: per-chunk top-k + masks, one-workgroup table build, per-chunk stable scatter.
// ------------------------------------------------------------------------------------
constexpr int kChunkThreads = 1024;

__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(const float* __restrict__ logits, int T, int E,
                                                                   int k, int32_t* __restrict__ idx,
                                                                   float* __restrict__ w,
                                                                   uint64_t* __restrict__ gmask) {
  __shared__ uint64_t mask[1024];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kChunkThreads) mask[e] = 0ull;
  __syncthreads();
  const size_t t0 = (size_t)c * kChunk;
  topk_block_any<kChunkThreads>(logits + t0 * E, min(kChunk, T - (int)t0), E, k, idx + t0 * k, w + t0 * k, mask,
                                nullptr);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunkThreads) gmask[(size_t)c * E + e] = mask[e];
}

__global__ __launch_bounds__(1024) void route_scan_kernel(CallBufs b, int T, int E, int k, int S, int C) {
  __shared__ int cnt[1024];
  const int e = threadIdx.x;
  if (e < E) {
    int c = 0;
    for (int ch = 0; ch < C; ++ch) {
      b.cbase[(size_t)ch * E + e] = c;
      c += __popcll(b.gmask[(size_t)ch * E + e]);
    }
    cnt[e] = c;
  }
  __syncthreads();
  if (threadIdx.x < 64) build_tables_wave(cnt, T, E, k, S, b, cnt);
}

__global__ __launch_bounds__(64) void route_scatter_kernel(CallBufs b, int T, int E, int k) {
  const int c = blockIdx.x, lane = threadIdx.x, t = c * kChunk + lane;
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int e = b.idx[(size_t)t * k + j];
    const size_t ce = (size_t)c * E + e;
    b.perm[b.offsets[e] + b.cbase[ce] + __popcll(b.gmask[ce] & below)] = t * k + j;
  }
}

// ------------------------------------------------------------------------------------
hipError_t launch_router_logits(const Dims& d, const uint16_t* x, const float* wr, const float* bias,
                                const CallBufs& b, int T, bool quantize_x, hipStream_t s) {
  if (route_fused(d, T)) {
    dim3 grid(d.E, (T + kRouterTT - 1) / kRouterTT);
    const int tk = timing_begin("router_route", s);
    router_kernel<<<grid, kTailThreads, 0, s>>>(x, wr, bias, b, T, d.E, d.H, d.K, d.S, quantize_x ? 1 : 0);
    timing_end(tk, s);
    return hipGetLastError();
  }
  dim3 grid((T + kRouterGemmTile - 1) / kRouterGemmTile, (d.E + kRouterGemmTile - 1) / kRouterGemmTile);
  int tk = timing_begin("router_gemm", s);
  router_gemm_kernel<<<grid, 256, 0, s>>>(x, wr, bias, b.logits, T, d.E, d.H);
  timing_end(tk, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !quantize_x) return e;
  const size_t blocks = (size_t)T * (d.H / 32);
  tk = timing_begin("quantize_x", s);
  quantize_x_kernel<<<(unsigned)((blocks + 255) / 256), 256, 0, s>>>(x, b.xq, T, d.H);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_route_chunked(const Dims& d, const CallBufs& b, int T, hipStream_t s) {
  const int C = (T + kChunk - 1) / kChunk;
  int tk = timing_begin("topk_chunk", s);
  topk_chunk_kernel<<<C, kChunkThreads, 0, s>>>(b.logits, T, d.E, d.K, b.idx, b.w, b.gmask);
  timing_end(tk, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tk = timing_begin("route_scan", s);
  route_scan_kernel<<<1, 1024, 0, s>>>(b, T, d.E, d.K, d.S, C);
  timing_end(tk, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  tk = timing_begin("route_scatter", s);
  route_scatter_kernel<<<C, 64, 0, s>>>(b, T, d.E, d.K);
  timing_end(tk, s);
  return hipGetLastError();
}

}  // namespace moe
