// Routing on the device: router scores, top-k with renormalised softmax weights, and the
// stable token->expert grouping (counts, offsets, perm) plus the tables the expert kernels
// read (active groups for the GEMV path, M-tiles for the grouped GEMM).
//
// "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine" (PR #1055, "What it is",
// prefill MoE) routes on the device and feeds expert-grouped GEMM rows; the pages leave the
// scoring rule open, so scores are a plain fp32 dot product (+ optional bias), selection is
// the k largest (ties to the lower index), and the weights are a softmax over the k selected
// scores.
#include "common.h"

namespace moe {

// ------------------------------------------------------------------------------------
// Router scores l[t][e] = x[t] . W_r[e] + b[e]  (fp32 accumulate, bf16 activations).
// One workgroup per (expert, tile of kRouterTT tokens): the 256 threads split the hidden
// axis (8 values each per step), partial sums are reduced across each wave and then the
// 4 waves in a fixed order, so a score does not depend on the other tokens of the batch.
// ------------------------------------------------------------------------------------
constexpr int kRouterTT = 8;

// When xq is not NULL the workgroups of a token tile also write the tile's activations as
// two exact FP8 terms with a scale per 32-value block (the decode kernels' A operand):
// xq = [2][T][H] e4m3 bytes, then [T][H/32] e8m0 scales.
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

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T, int E,
                                                            int H, uint8_t* __restrict__ xq) {
  __shared__ float part[4][kRouterTT];
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterTT;
  const int nt = min(kRouterTT, T - t0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (xq) {
    const int KB = H >> 5;
    for (int j = e * 256 + tid; j < nt * KB; j += E * 256) {
      const int t = t0 + j / KB, b = j % KB;
      quantize_x_block(x + (size_t)t * H + b * 32, xq + (size_t)t * H + b * 32,
                       xq + (size_t)(T + t) * H + b * 32, xq + (size_t)2 * T * H + (size_t)t * KB + b);
    }
  }
  float acc[kRouterTT];
#pragma unroll
  for (int i = 0; i < kRouterTT; ++i) acc[i] = 0.f;
  const float* wrow = wr + (size_t)e * H;
  for (int h = tid * 8; h < H; h += 256 * 8) {  // H % 32 == 0, so h + 8 <= H
    const float4 w0 = *reinterpret_cast<const float4*>(wrow + h);
    const float4 w1 = *reinterpret_cast<const float4*>(wrow + h + 4);
#pragma unroll
    for (int i = 0; i < kRouterTT; ++i) {
      if (i < nt) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + i) * H + h);
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
#pragma unroll
  for (int i = 0; i < kRouterTT; ++i) {
    float v = acc[i];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0) part[wave][i] = v;
  }
  __syncthreads();
  if (tid < nt) {
    const float v = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
    logits[(size_t)(t0 + tid) * E + e] = v + (bias ? bias[e] : 0.f);
  }
}

// ------------------------------------------------------------------------------------
// Top-k of one token by one wave.
// Each score becomes a 64-bit rank key: high word = order-preserving image of the float
// (+1, so that NaN -> 1 still beats an excluded entry, which is 0), low word = ~index so
// that equal scores prefer the lower expert.  -0 is ranked as +0.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  uint32_t ord;
  if (v != v)
    ord = 0u;
  else
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord + 1ull) << 32 | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = __shfl_xor(v, m, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Writes idx[0..k), w[0..k) of the token and sets bit `tbit` of mask[e] for each pick;
// also copies the picks to sel (LDS) when sel is not NULL.  Q = scores per lane (E <= 64*Q).
template <int Q>
__device__ void topk_token(const float* __restrict__ lrow, int E, int k, int lane,
                           int32_t* __restrict__ idx_out, float* __restrict__ w_out, uint64_t* mask,
                           int tbit, int32_t* sel) {
  uint64_t key[Q];
  float val[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    val[q] = e < E ? lrow[e] : 0.f;
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
    uint64_t best = 0ull;
#pragma unroll
    for (int q = 0; q < Q; ++q) best = key[q] > best ? key[q] : best;
    best = wave_max_u64(best);
    const int e = __builtin_amdgcn_readfirstlane((int)(0xFFFFFFFFu - (uint32_t)best));
    float mine = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (q == (e >> 6)) mine = val[q];
    const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mine), e & 63));
    if (j == 0) vtop = v;
    if ((e & 63) == lane) {
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (q == (e >> 6)) key[q] = 0ull;
    }
    if ((j & 63) == lane) {
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (q == (j >> 6)) {
          selE[q] = e;
          selV[q] = v;
        }
    }
    if (lane == 0) {
      atomicOr(reinterpret_cast<unsigned long long*>(&mask[e]), 1ull << tbit);
      if (sel) sel[j] = e;
    }
  }
  // softmax over the k picked scores; xor-butterfly sums are identical on every lane
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
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = lane + 64 * q;
    if (j < k) {
      idx_out[j] = selE[q];
      w_out[j] = p[q] / s;
    }
  }
}

// Calls topk_token with the smallest Q >= ceil(E/64) among 1, 2, 4, 8, 16.
__device__ __forceinline__ void topk_any(int E, const float* lrow, int k, int lane, int32_t* idx_out,
                                         float* w_out, uint64_t* mask, int tbit, int32_t* sel) {
  if (E <= 64)
    topk_token<1>(lrow, E, k, lane, idx_out, w_out, mask, tbit, sel);
  else if (E <= 128)
    topk_token<2>(lrow, E, k, lane, idx_out, w_out, mask, tbit, sel);
  else if (E <= 256)
    topk_token<4>(lrow, E, k, lane, idx_out, w_out, mask, tbit, sel);
  else if (E <= 512)
    topk_token<8>(lrow, E, k, lane, idx_out, w_out, mask, tbit, sel);
  else
    topk_token<16>(lrow, E, k, lane, idx_out, w_out, mask, tbit, sel);
}

// ------------------------------------------------------------------------------------
// Block-wide exclusive scan over 1024 threads (16 waves).
// ------------------------------------------------------------------------------------
__device__ int scan1024(int v, int* lds16, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds16[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int s = lane < 16 ? lds16[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(s, d, 64);
      if (lane >= d) s += y;
    }
    if (lane < 16) lds16[lane] = s;
  }
  __syncthreads();
  const int base = wave > 0 ? lds16[wave - 1] : 0;
  *total = lds16[15];
  __syncthreads();
  return base + x - v;
}

// Expert tables from per-expert row counts (thread e holds count of expert e; 0 past E).
// Returns the expert's first grouped row.  Requires blockDim.x == 1024 and E <= 1024.
__device__ int build_tables(int cnt, int T, int E, int k, int S, const CallBufs& b, int* lds16) {
  const int tid = threadIdx.x;
  int total;
  const int off = scan1024(cnt, lds16, &total);
  if (tid < E) {
    b.counts[tid] = cnt;
    b.offsets[tid] = off;
    b.grp_row0[tid] = off;
    b.grp_rows[tid] = cnt;
  }
  if (tid == 0) {
    b.offsets[E] = total;
    if (S) {
      b.grp_row0[E] = T * k;
      b.grp_rows[E] = T;
    }
  }
  int nact;
  const int apos = scan1024(cnt > 0 ? 1 : 0, lds16, &nact);
  if (cnt > 0) b.act[apos] = tid;
  if (tid == 0 && S) b.act[nact] = E;
  const int mt = (cnt + kGemmBM - 1) / kGemmBM;
  int nmt;
  const int mpos = scan1024(mt, lds16, &nmt);
  for (int i = 0; i < mt; ++i) {
    b.mt_group[mpos + i] = tid;
    b.mt_row0[mpos + i] = i * kGemmBM;
  }
  const int mts = S ? (T + kGemmBM - 1) / kGemmBM : 0;
  for (int i = tid; i < mts; i += 1024) {
    b.mt_group[nmt + i] = E;
    b.mt_row0[nmt + i] = i * kGemmBM;
  }
  if (tid == 0) {
    b.info[0] = nact + S;
    b.info[1] = nmt + mts;
  }
  return off;
}

// ------------------------------------------------------------------------------------
// Small batches (T <= 64): top-k, tables and scatter in one 1024-thread workgroup.
// ------------------------------------------------------------------------------------
constexpr int kSmallSel = 4096;  // picks kept in LDS by the one-workgroup route (T*k)

__global__ __launch_bounds__(1024) void route_small_kernel(CallBufs b, int T, int E, int k, int S) {
  __shared__ uint64_t mask[1024];
  __shared__ int offs[1024];
  __shared__ int32_t sel[kSmallSel];
  __shared__ int lds16[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool in_lds = T * k <= kSmallSel;
  if (tid < E) mask[tid] = 0ull;
  __syncthreads();
  for (int t = wave; t < T; t += 16)
    topk_any(E, b.logits + (size_t)t * E, k, lane, b.idx + (size_t)t * k, b.w + (size_t)t * k, mask, t,
             in_lds ? sel + t * k : nullptr);
  __syncthreads();
  const int cnt = tid < E ? __popcll(mask[tid]) : 0;
  const int off = build_tables(cnt, T, E, k, S, b, lds16);
  if (tid < E) offs[tid] = off;
  __syncthreads();
  if (tid < T) {
    const uint64_t below = (1ull << tid) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = in_lds ? sel[tid * k + j] : b.idx[tid * k + j];
      b.perm[offs[e] + __popcll(mask[e] & below)] = tid * k + j;
    }
  }
}

// ------------------------------------------------------------------------------------
// Any T: per-chunk top-k + masks, one-workgroup scan, per-chunk stable scatter.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_chunk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ w,
                                                         uint64_t* __restrict__ gmask) {
  __shared__ uint64_t mask[1024];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = wave; i < kChunk; i += 4) {
    const int t = c * kChunk + i;
    if (t >= T) break;
    topk_any(E, logits + (size_t)t * E, k, lane, idx + (size_t)t * k, w + (size_t)t * k, mask, i, nullptr);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) gmask[(size_t)c * E + e] = mask[e];
}

__global__ __launch_bounds__(1024) void route_scan_kernel(CallBufs b, int T, int E, int k, int S, int C) {
  __shared__ int lds16[16];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    for (int c = 0; c < C; ++c) {
      b.cbase[(size_t)c * E + e] = cnt;
      cnt += __popcll(b.gmask[(size_t)c * E + e]);
    }
  }
  build_tables(cnt, T, E, k, S, b, lds16);
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
                                float* logits, int T, uint8_t* xq, hipStream_t s) {
  dim3 grid(d.E, (T + kRouterTT - 1) / kRouterTT);
  const int tk = timing_begin("router_logits", s);
  router_logits_kernel<<<grid, 256, 0, s>>>(x, wr, bias, logits, T, d.E, d.H, xq);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_route_small(const Dims& d, const CallBufs& b, int T, hipStream_t s) {
  const int tk = timing_begin("route_small", s);
  route_small_kernel<<<1, 1024, 0, s>>>(b, T, d.E, d.K, d.S);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_route_chunked(const Dims& d, const CallBufs& b, int T, hipStream_t s) {
  const int C = (T + kChunk - 1) / kChunk;
  int tk = timing_begin("topk_chunk", s);
  topk_chunk_kernel<<<C, 256, 0, s>>>(b.logits, T, d.E, d.K, b.idx, b.w, b.gmask);
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
