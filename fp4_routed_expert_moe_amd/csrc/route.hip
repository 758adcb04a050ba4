// Routing kernels: router scores, top-k with renormalised softmax weights, and the stable
// token->expert grouping (counts, offsets, perm) plus the tables the expert kernels read
// (active groups, M-tiles for the grouped GEMM).  The device steps themselves are in
// route_dev.h, shared with the fused decode kernel.
//
// Small batches (route_fused: T <= 64 and T*E <= kTailScores) are routed in one launch: the
// router workgroups publish their scores, and the last one to finish (device-scope counter
// in the workspace, left at zero again) runs top-k, the grouping tables and the scatter.
// Larger batches score on the matrix cores, then use a per-chunk top-k kernel, a
// one-workgroup scan and a per-chunk scatter.
#include "join_dev.h"
#include "route_dev.h"

namespace moe {

// ------------------------------------------------------------------------------------
// Small batches: router scores l[t][e] = x[t] . W_r[e] + b[e] and the routing tail in one
// launch.  Workgroup (i, j) scores experts 4i .. 4i+3 (four waves each) for tokens
// 4j .. 4j+3 and quantizes an equal slice of the activation blocks when asked; the last
// workgroup to finish routes the whole batch.
// ------------------------------------------------------------------------------------
constexpr int kTailThreads = 1024;
constexpr int kRouterEPB = kTailThreads / 64 / kScoreWaves;  // experts per router workgroup

using RouterTail = TailLayout<1024, kTailScores>;

// flags: kRouteQuantize = also split x into FP8 terms (the workgroups that are not last, after
// publishing their scores, so the split never delays the routing); kRouteMTiles = also build
// the grouped GEMM's M-tile list; kRouteLean = only the tables the decode kernels read (at
// most 64 picks).
// kRouteJoin = first form x from the chained decode's residual (JoinArgs) into the x buffer.
// kRouteWarm = the workgroups that are not last then read one word of every 128-byte line of
// the Warm ranges, one slice each.
constexpr int kRouteQuantize = 1, kRouteMTiles = 2, kRouteLean = 4, kRouteJoin = 8, kRouteWarm = 16;

// Slice `part` of `parts` of the lines of the Warm ranges: one 4-byte load per line, kept
// live only through an empty asm statement.
__device__ __forceinline__ void warm_lines(const Warm& w, int part, int parts) {
  size_t total = 0;
#pragma unroll
  for (int i = 0; i < 6; ++i) total += w.bytes[i] >> 7;
  const size_t per = (total + parts - 1) / parts, lo = (size_t)part * per, hi = min(total, lo + per);
  float acc = 0.f;
  for (size_t l = lo + threadIdx.x; l < hi; l += kTailThreads) {
    size_t r = l;
    int i = 0;
    while (i < 5 && r >= (w.bytes[i] >> 7)) r -= w.bytes[i++] >> 7;
    acc += *reinterpret_cast<const float*>(w.p[i] + (r << 7));
  }
  asm volatile("" ::"v"(acc));
}

// x is not __restrict__: with kRouteJoin this launch writes it before reading it.
__global__ __launch_bounds__(kTailThreads) void router_kernel(const uint16_t* x,
                                                             const float* __restrict__ wr,
                                                             const float* __restrict__ bias, CallBufs b, int T,
                                                             int E, int H, int K, int S, int flags, JoinArgs join,
                                                             Warm warm) {
  __shared__ __align__(16) char lds[RouterTail::kBytes];
  const int wave = threadIdx.x >> 6;
  const int grp = wave / kScoreWaves;
  const int e = blockIdx.x * kRouterEPB + grp;
  if (flags & kRouteJoin) {
    // every workgroup forms all T rows of x itself (identical values), four rows at a time,
    // 256 threads a row, the join kernel's steps; x is then read back as usual
    static_assert(kTailThreads == 4 * kJoinThreads, "four join rows per pass");
    __shared__ float jpart[4][4];
    const int jr = threadIdx.x / kJoinThreads, tid = threadIdx.x % kJoinThreads;
    uint16_t* xo = const_cast<uint16_t*>(x);
    for (int tb = 0; tb < T; tb += 4) {
      const int t = tb + jr;
      JoinRow r;
      float ss = 0.f;
      if (t < T) {
        join_load(r, join.h_src + (size_t)t * H, join.y ? join.y + (size_t)t * H : nullptr, nullptr, H, tid);
        ss = join_wave_sum(r.ss);
      }
      if ((threadIdx.x & 63) == 0) jpart[jr][tid >> 6] = ss;
      __syncthreads();
      if (t < T) join_store_x(r, join_inv(jpart[jr], H, join.eps), join.gamma, xo + (size_t)t * H, H, tid);
      __syncthreads();
    }
  }
  const int t0 = blockIdx.y * kScoreTT;
  const int nt = min(kScoreTT, T - t0);
  __shared__ float part[kRouterEPB][kScoreWaves * kScoreTT];
  score_expert(x, wr, bias, b.logits, t0, nt, e, e < E, E, H, part[grp]);
  // the x split: slice `part` of `parts` of all T*KB blocks
  auto quantize = [&](int slice, int parts) {
    const int KB = H >> 5;
    const int nb = T * KB, per = (nb + parts - 1) / parts;
    uint8_t* xq = b.xq;
    for (int j = slice * per + threadIdx.x; j < min(nb, (slice + 1) * per); j += kTailThreads) {
      const int t = j / KB, bb = j % KB;
      const XBlock q = quantize_x_block(x + (size_t)t * H + bb * 32);
      uint4* hi = reinterpret_cast<uint4*>(xq + (size_t)t * H + bb * 32);
      uint4* lo = reinterpret_cast<uint4*>(xq + (size_t)(T + t) * H + bb * 32);
      hi[0] = q.hi[0];
      hi[1] = q.hi[1];
      lo[0] = q.lo[0];
      lo[1] = q.lo[1];
      uint8_t* xs = xq + (size_t)2 * T * H + (size_t)t * kb_pad(H);
      xs[bb] = (uint8_t)q.s;
      if (bb == KB - 1)  // pad bytes of the row (finite; they only meet zero weights)
        for (int jj = KB; jj < kb_pad(H); ++jj) xs[jj] = (uint8_t)127;
    }
  };
  // The last workgroup to finish routes the whole batch, then re-arms the counter; the others
  // split x, one slice per arrival ticket.
  __shared__ int ticket;
  int32_t* counter = b.ctrl + CtrlLayout::kRoute;
  const int total = (int)(gridDim.x * gridDim.y);
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) ticket = add_agent(counter, 1);
  __syncthreads();
  if (ticket < total - 1) {
    if (flags & kRouteQuantize) quantize(ticket, total - 1);
    if (flags & kRouteWarm) warm_lines(warm, ticket, total - 1);
    return;
  }
  if (flags & kRouteLean)
    route_tail<kTailThreads, 16, 1024, kTailScores, false, true>(b, T, E, K, S, lds);
  else if (flags & kRouteMTiles)
    route_tail<kTailThreads, 16, 1024, kTailScores, true>(b, T, E, K, S, lds);
  else
    route_tail<kTailThreads, 16, 1024, kTailScores, false>(b, T, E, K, S, lds);
  if (threadIdx.x == 0) reset_counter(counter);
  if ((flags & kRouteJoin) && join.h_dst) {
    // the residual after the join: every other workgroup has read h_src (it arrived), so an
    // in-place update is safe; fp32 adds, as in the join kernel
    const size_t n4 = (size_t)T * H / 4;
    const float4* hs = reinterpret_cast<const float4*>(join.h_src);
    const float4* ys = reinterpret_cast<const float4*>(join.y);
    float4* hd = reinterpret_cast<float4*>(join.h_dst);
    for (size_t i = threadIdx.x; i < n4; i += kTailThreads) {
      float4 v = hs[i];
      if (ys) {
        const float4 d = ys[i];
        v.x += d.x;
        v.y += d.y;
        v.z += d.z;
        v.w += d.w;
      }
      hd[i] = v;
    }
  }
  if ((flags & kRouteQuantize) && total == 1) quantize(0, 1);
}

// ------------------------------------------------------------------------------------
// Larger batches: router scores on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
// W_r (fp32) is split on the fly into three bf16 terms whose sum is exactly W_r: the top,
// middle and low 8 bits of the 24-bit significand, each remainder exact (it is the float
// minus its own truncation).  x (bf16) times each term is exact in fp32, so a score is the
// fp32 dot product up to summation order, which is fixed per (token, expert).  64 tokens x
// 64 experts per workgroup, 32 x 32 per wave (2 x 2 MFMA tiles, three terms each).
// Rounding chain of a score: each 32-value step's top-term products go through one MFMA
// that starts from zero (any internal order: at most 31 roundings of that step's products),
// and that step's result is added into the running fp32 sum with one VALU add; the two low
// terms (2^-8 and 2^-16 of the products) accumulate in MFMA chains of their own, added at
// the end.  So a product passes at most 31 + steps + 1 roundings before the slice's partial
// score, plus one per slice when the top-k adds the slices and one for the bias.
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

__global__ __launch_bounds__(256, 2) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, uint8_t* __restrict__ xq,
                                                          uint64_t* __restrict__ gmask, int T, int E, int H) {
  // hidden-axis slice blockIdx.z of gridDim.z (whole 32-value steps); its partial scores go to
  // logits[slice][T][E], the bias into slice 0's
  const int nk = H >> 5, ks = blockIdx.z, KS = gridDim.z;
  const int k_lo = 32 * (ks * nk / KS), k_hi = 32 * ((ks + 1) * nk / KS);
  logits += (size_t)ks * T * E;
  {
    // clear the per-chunk expert masks the top-k ORs its bits into
    const size_t nmask = (size_t)((T + kChunk - 1) / kChunk) * E;
    const size_t wg = ((size_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const size_t nwg = (size_t)gridDim.x * gridDim.y * gridDim.z;
    for (size_t i = wg * 256 + threadIdx.x; i < nmask; i += nwg * 256) gmask[i] = 0ull;
  }
  if (xq) {
    // the FP8 term split of this token tile's x over this slice, shared by the expert tiles
    const int tt0 = blockIdx.x * kRouterGemmTile, ntt = min(kRouterGemmTile, T - tt0);
    const int b_lo = k_lo >> 5, nb = (k_hi - k_lo) >> 5, KB = H >> 5;
    for (int j = blockIdx.y * 256 + threadIdx.x; j < ntt * nb; j += 256 * gridDim.y) {
      const int t = tt0 + j / nb, bb = b_lo + j % nb;
      const XBlock q = quantize_x_block(x + (size_t)t * H + bb * 32);
      uint4* hi = reinterpret_cast<uint4*>(xq + (size_t)t * H + bb * 32);
      uint4* lo = reinterpret_cast<uint4*>(xq + (size_t)(T + t) * H + bb * 32);
      hi[0] = q.hi[0];
      hi[1] = q.hi[1];
      lo[0] = q.lo[0];
      lo[1] = q.lo[1];
      uint8_t* xs = xq + (size_t)2 * T * H + (size_t)t * kb_pad(H);
      xs[bb] = (uint8_t)q.s;
      if (bb == KB - 1)  // pad bytes of the row (finite; they only meet zero weights)
        for (int jj = KB; jj < kb_pad(H); ++jj) xs[jj] = (uint8_t)127;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * kRouterGemmTile + (wave & 1) * 32;
  const int e0 = blockIdx.y * kRouterGemmTile + (wave >> 1) * 32;
  f32x4 acc[2][2], acc_lo[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = acc_lo[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one 32-value step: top term from zero, added into acc; low terms chained in acc_lo
  auto mma_step = [&](const bf16x8 (&xa)[2], const bf16x8 (&wb)[2][3]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x4 hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], wb[j][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc_lo[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], wb[j][1], acc_lo[i][j], 0, 0, 0);
        acc_lo[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], wb[j][2], acc_lo[i][j], 0, 0, 0);
        acc[i][j] += hi;
      }
  };
  // The tile's 64 tokens and 64 experts pass through LDS 64 K values at a time: x as bf16,
  // W_r split into its three bf16 terms once per workgroup (each wave reads the half it
  // needs); the next batch's global loads are in flight while this one runs from LDS.
  constexpr int KBt = 64, PITCH = KBt + 8;  // bf16 per LDS row (16 bytes of padding)
  __shared__ __align__(16) __bf16 xs[2][kRouterGemmTile][PITCH];
  __shared__ __align__(16) __bf16 ws3[2][3][kRouterGemmTile][PITCH];
  // staging: thread t loads 16 K values of tile row t / 4 at column (t % 4) * 16
  const int srow = threadIdx.x >> 2, scol = (threadIdx.x & 3) * 16;
  const uint16_t* xg = x + (size_t)min(blockIdx.x * kRouterGemmTile + srow, T - 1) * H;
  const float* wg = wr + (size_t)min(blockIdx.y * kRouterGemmTile + srow, E - 1) * H;
  struct Stage {
    uint4 x[2];
    float4 w[4];
  };
  auto gload = [&](Stage& st, int k0) {
    const int kk = min(k0 + scol, k_hi - 16);  // past the slice: valid bytes, never used
    st.x[0] = *reinterpret_cast<const uint4*>(xg + kk);
    st.x[1] = *reinterpret_cast<const uint4*>(xg + kk + 8);
#pragma unroll
    for (int v = 0; v < 4; ++v) st.w[v] = *reinterpret_cast<const float4*>(wg + kk + 4 * v);
  };
  auto lstore = [&](int buf, const Stage st) {  // by value: a reference to either stage spilled it
    *reinterpret_cast<uint4*>(&xs[buf][srow][scol]) = st.x[0];
    *reinterpret_cast<uint4*>(&xs[buf][srow][scol + 8]) = st.x[1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 t3[3];
      split3(st.w[2 * h], st.w[2 * h + 1], t3);
#pragma unroll
      for (int t = 0; t < 3; ++t) *reinterpret_cast<bf16x8*>(&ws3[buf][t][srow][scol + 8 * h]) = t3[t];
    }
  };
  auto compute = [&](int buf, int k0) {
#pragma unroll
    for (int u = 0; u < KBt / 32; ++u) {
      if (k0 + 32 * u >= k_hi) break;
      bf16x8 xa[2], wb[2][3];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        xa[i] = *reinterpret_cast<const bf16x8*>(&xs[buf][(wave & 1) * 32 + 16 * i + r][32 * u + 8 * kq]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 3; ++t)
          wb[j][t] = *reinterpret_cast<const bf16x8*>(&ws3[buf][t][(wave >> 1) * 32 + 16 * j + r][32 * u + 8 * kq]);
      mma_step(xa, wb);
    }
  };
  // Global loads run two batches ahead: while batch k0 runs from LDS, batch k0 + KBt waits in
  // registers for the other LDS buffer and batch k0 + 2 KBt is in flight.
  Stage sa, sb;
  gload(sa, k_lo);
  if (k_lo + KBt < k_hi) gload(sb, k_lo + KBt);
  lstore(0, sa);
  __syncthreads();
  // two batches a round: LDS buffer 0 holds batch k0 and sb batch k0 + KBt (sa is free), then
  // buffer 1 holds k0 + KBt and sa k0 + 2 KBt
  for (int k0 = k_lo; k0 < k_hi; k0 += 2 * KBt) {
    if (k0 + 2 * KBt < k_hi) gload(sa, k0 + 2 * KBt);
    __builtin_amdgcn_sched_barrier(0);
    compute(0, k0);
    if (k0 + KBt >= k_hi) break;
    lstore(1, sb);
    __syncthreads();
    if (k0 + 3 * KBt < k_hi) gload(sb, k0 + 3 * KBt);
    __builtin_amdgcn_sched_barrier(0);
    compute(1, k0 + KBt);
    if (k0 + 2 * KBt >= k_hi) break;
    lstore(0, sa);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + 16 * j + r;
      if (e >= E) continue;
      const float be = bias && ks == 0 ? bias[e] : 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 16 * i + 4 * kq + v;
        if (t < T) logits[(size_t)t * E + e] = (acc[i][j][v] + acc_lo[i][j][v]) + be;
      }
    }
}

// ------------------------------------------------------------------------------------
// Any T: per-chunk top-k + masks, one-workgroup table build, per-chunk stable scatter.
// ------------------------------------------------------------------------------------
constexpr int kChunkThreads = 1024;

// One workgroup per kTopkTokens tokens, one wave per token; the tokens' bits of the per-chunk
// expert masks are ORed into gmask (cleared by the router GEMM earlier in the call).
constexpr int kTopkTokens = kChunkThreads / 64;

__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(const float* __restrict__ logits, int KS, int T,
                                                                   int E, int k, int32_t* __restrict__ idx,
                                                                   float* __restrict__ w,
                                                                   uint64_t* __restrict__ gmask) {
  __shared__ uint64_t mask[1024];
  __shared__ uint16_t sel_e[kTopkTokens * 1024];
  __shared__ float sel_w[kTopkTokens * 1024];
  for (int e = threadIdx.x; e < E; e += kChunkThreads) mask[e] = 0ull;
  __syncthreads();
  const size_t t0 = (size_t)blockIdx.x * kTopkTokens;
  const int nt = min(kTopkTokens, T - (int)t0);
  const int wave = threadIdx.x >> 6;
  const int tbit = (int)(t0 % kChunk) + wave;  // bit of this token in its chunk's masks
  if (wave < nt) {
    const float* row = logits + (t0 + wave) * E;
    const size_t st = (size_t)T * E;
    uint16_t* se = sel_e + wave * k;
    float* sw = sel_w + wave * k;
    if (E <= 64)
      topk_wave<1>(row, E, k, se, sw, mask, tbit, KS, st);
    else if (E <= 128)
      topk_wave<2>(row, E, k, se, sw, mask, tbit, KS, st);
    else if (E <= 256)
      topk_wave<4>(row, E, k, se, sw, mask, tbit, KS, st);
    else if (E <= 512)
      topk_wave<8>(row, E, k, se, sw, mask, tbit, KS, st);
    else
      topk_wave<16>(row, E, k, se, sw, mask, tbit, KS, st);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * k; i += kChunkThreads) {
    idx[t0 * k + i] = sel_e[i];
    w[t0 * k + i] = sel_w[i];
  }
  uint64_t* gm = gmask + (t0 / kChunk) * E;
  for (int e = threadIdx.x; e < E; e += kChunkThreads)
    if (mask[e]) atomicOr(reinterpret_cast<unsigned long long*>(gm + e), (unsigned long long)mask[e]);
}

// Per expert: the prefix over the chunks of its pick counts (16 chunks' masks loaded at a
// time), then the grouping tables.
__global__ __launch_bounds__(1024) void route_scan_kernel(CallBufs b, int T, int E, int k, int S, int C) {
  __shared__ int cnt[1024], offs[1024], act[1024], mt_off[1024], part[1024];
  __shared__ GroupScan gs;
  // P threads per expert, each over a contiguous range of the chunks: first their row counts,
  // then (after the counts of the ranges before are known) each chunk's base row
  const int P = E <= 512 ? 1024 / E : 1;
  const int e = threadIdx.x % E, p = threadIdx.x / E;
  const bool on = p < P;
  const int c_lo = p * C / P, c_hi = (p + 1) * C / P;
  const uint64_t* __restrict__ gm = b.gmask;
  int32_t* __restrict__ cb = b.cbase;
  if (on) {
    int c = 0;
    for (int ch0 = c_lo; ch0 < c_hi; ch0 += 16) {
      uint64_t mv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) mv[u] = ch0 + u < c_hi ? gm[(size_t)(ch0 + u) * E + e] : 0ull;
#pragma unroll
      for (int u = 0; u < 16; ++u) c += __popcll(mv[u]);
    }
    part[p * E + e] = c;
  }
  __syncthreads();
  if (on) {
    int base = 0, total = 0;
    for (int q = 0; q < P; ++q) {
      const int v = part[q * E + e];
      base += q < p ? v : 0;
      total += v;
    }
    for (int ch0 = c_lo; ch0 < c_hi; ch0 += 16) {
      uint64_t mv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) mv[u] = ch0 + u < c_hi ? gm[(size_t)(ch0 + u) * E + e] : 0ull;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (ch0 + u < c_hi) cb[(size_t)(ch0 + u) * E + e] = base;
        base += __popcll(mv[u]);
      }
    }
    if (p == 0) {
      cnt[e] = total;
      offs[e] = total;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) group_scan_wave<true>(offs, act, mt_off, &gs, T, E, S);
  __syncthreads();
  write_tables<1024, true>([&](int i) { return cnt[i]; }, offs, act, mt_off, gs, T, E, k, S, b);
}

__global__ __launch_bounds__(64) void route_scatter_kernel(CallBufs b, int T, int E, int k) {
  const int c = blockIdx.x, lane = threadIdx.x, t = c * kChunk + lane;
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int e = b.idx[(size_t)t * k + j];
    const size_t ce = (size_t)c * E + e;
    const int r = b.offsets[e] + b.cbase[ce] + __popcll(b.gmask[ce] & below);
    b.perm[r] = t * k + j;
    b.row_w[r] = b.w[(size_t)t * k + j];
  }
}

// ------------------------------------------------------------------------------------
hipError_t launch_router_logits(const Dims& d, const uint16_t* x, const float* wr, const float* bias,
                                const CallBufs& b, int T, bool quantize_x, bool mtiles, bool lean, hipStream_t s,
                                const JoinArgs* join, const Warm* warm) {
  if (join && !join_fused(d, T)) return hipErrorInvalidValue;  // the caller runs the join kernel instead
  if (route_fused(d, T)) {
    dim3 grid((d.E + kRouterEPB - 1) / kRouterEPB, (T + kScoreTT - 1) / kScoreTT);
    const int tk = timing_begin("router_route", s);
    const int flags = (quantize_x ? kRouteQuantize : 0) | (mtiles ? kRouteMTiles : 0) |
                      (lean && !mtiles && T * d.K <= kLeanMaxPicks ? kRouteLean : 0) | (join ? kRouteJoin : 0) |
                      (warm && grid.x * grid.y > 1 ? kRouteWarm : 0);
    router_kernel<<<grid, kTailThreads, 0, s>>>(x, wr, bias, b, T, d.E, d.H, d.K, d.S, flags,
                                                join ? *join : JoinArgs{nullptr, nullptr, nullptr, nullptr, 0.f},
                                                warm ? *warm : Warm{});
    timing_end(tk, s);
    return hipGetLastError();
  }
  dim3 grid((T + kRouterGemmTile - 1) / kRouterGemmTile, (d.E + kRouterGemmTile - 1) / kRouterGemmTile,
            router_slices(d, T));
  const int tk = timing_begin("router_gemm", s);
  router_gemm_kernel<<<grid, 256, 0, s>>>(x, wr, bias, b.logits, quantize_x ? b.xq : nullptr, b.gmask, T, d.E, d.H);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_route_chunked(const Dims& d, const CallBufs& b, int T, hipStream_t s) {
  const int C = (T + kChunk - 1) / kChunk;
  int tk = timing_begin("topk_chunk", s);
  topk_chunk_kernel<<<(T + kTopkTokens - 1) / kTopkTokens, kChunkThreads, 0, s>>>(b.logits, router_slices(d, T), T,
                                                                                 d.E, d.K, b.idx, b.w, b.gmask);
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
