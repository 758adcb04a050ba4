// Device-side routing steps shared by the routing kernels (route.hip): router scores, the FP8
// term split of the activations, top-k with renormalised softmax weights, and the stable
// token->expert grouping tables.
//
// "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine" (PR #1055, "What it is",
// prefill MoE) routes on the device and feeds expert-grouped GEMM rows; the pages leave the
// scoring rule open, so scores are a plain fp32 dot product (+ optional bias), selection is
// the k largest (ties to the lower index), and the weights are a softmax over the k selected
// scores.
#pragma once

#include "common.h"

namespace moe {

// ------------------------------------------------------------------------------------
// Router score of one expert for up to kScoreTT tokens, computed by a group of four waves:
// wave w of the group adds x[h]*w[h] over its quarter of the hidden axis, lane l taking
// h = w*H/4 + 8l + 512j + i (j ascending, i = 0..7) with fused multiply-adds in that order;
// the lanes are summed in the fixed DPP order of wave_sum_f32 and the four quarters in wave
// order.  The one-launch router (batches route_fused takes) scores with this, so there a
// token's scores do not depend on the batch it comes in.  Larger batches score on the matrix
// cores (router_gemm_kernel) in another summation order: the same fp32 dot product, not the
// same bits.  All of a lane's loads are issued before the first product.
// Rounding chain: a lane's FMAs round once each (8 per 512 values of the quarter), then four
// DPP adds and three lane-total adds, three quarter adds and the bias: a product passes at
// most 8*ceil(H/2048) + 11 roundings.
// ------------------------------------------------------------------------------------
constexpr int kScoreTT = 4;  // tokens per router workgroup (4 measured faster than 8 or 2 at 8 tokens)
constexpr int kScoreWaves = 4;

// Quarter sums of one wave (wq = wave index in the group), same value on every lane.
__device__ __forceinline__ void score_quarter(const uint16_t* x, int nt, const float* __restrict__ w, int H, int wq,
                                              float (&out)[kScoreTT]) {
  const int lane = threadIdx.x & 63;
  const int hq = H / kScoreWaves;  // H % 32 == 0: a multiple of 8
  const int h_end = (wq + 1) * hq;
  float acc[kScoreTT];
#pragma unroll
  for (int i = 0; i < kScoreTT; ++i) acc[i] = 0.f;
  for (int h0 = wq * hq + lane * 8; h0 < h_end; h0 += 1024) {
    // two 512-value steps at once (their loads in flight together)
    float4 wv[2][2];
    uint4 xv[2][kScoreTT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int h = h0 + 512 * u;
      if (h < h_end) {
        wv[u][0] = *reinterpret_cast<const float4*>(w + h);
        wv[u][1] = *reinterpret_cast<const float4*>(w + h + 4);
#pragma unroll
        for (int i = 0; i < kScoreTT; ++i)
          if (i < nt) xv[u][i] = *reinterpret_cast<const uint4*>(x + (size_t)i * H + h);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (h0 + 512 * u >= h_end) break;
      const float4 w0 = wv[u][0], w1 = wv[u][1];
#pragma unroll
      for (int i = 0; i < kScoreTT; ++i) {
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
#pragma unroll
  for (int i = 0; i < kScoreTT; ++i) out[i] = wave_sum_f32(acc[i]);
}

// Scores of expert e for tokens [t0, t0+nt) (nt <= kScoreTT), published to logits[t][e] with
// agent-scope stores (the routing tail may run in another workgroup of the same launch).
// Called by every thread of the block; the group of waves [4g, 4g+4) handles expert e (valid
// false: the group only takes part in the barrier).  part: kScoreWaves * kScoreTT floats of
// LDS per group.
__device__ __forceinline__ void score_expert(const uint16_t* x, const float* __restrict__ wr,
                                            const float* __restrict__ bias, float* logits, int t0, int nt, int e,
                                            bool valid, int E, int H, float* part) {
  const int wq = (threadIdx.x >> 6) % kScoreWaves, lane = threadIdx.x & 63;
  if (valid) {
    float s[kScoreTT];
    score_quarter(x + (size_t)t0 * H, nt, wr + (size_t)e * H, H, wq, s);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kScoreTT; ++i) part[wq * kScoreTT + i] = s[i];
    }
  }
  __syncthreads();
  if (valid && wq == 0 && lane < nt) {
    const float v = ((part[lane] + part[kScoreTT + lane]) + part[2 * kScoreTT + lane]) + part[3 * kScoreTT + lane];
    st_agent(logits + (size_t)(t0 + lane) * E + e, v + (bias ? bias[e] : 0.f));
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------
// Activations as two exact FP8 terms with a scale per 32-value block (the expert kernels'
// A operand): xq = [2][T][H] e4m3 bytes, then [T][kb_pad(H)] e8m0 scales.
// ------------------------------------------------------------------------------------
struct XBlock {
  uint4 hi[2], lo[2];  // 32 e4m3 bytes of each term
  uint32_t s;          // e8m0 scale of term 0 (term 1: s - 4)
};
__device__ __forceinline__ XBlock quantize_x_block(const uint16_t* __restrict__ src) {
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
    // a non-finite value (the convert would saturate an infinity) becomes NaN in both terms
    uint32_t nanm = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) nanm |= fp8_nan_mask(v[j]) << (8 * j);
    th[i] |= nanm;
    tl[i] |= nanm;
  }
  XBlock b;
  b.hi[0] = make_uint4(th[0], th[1], th[2], th[3]);
  b.hi[1] = make_uint4(th[4], th[5], th[6], th[7]);
  b.lo[0] = make_uint4(tl[0], tl[1], tl[2], tl[3]);
  b.lo[1] = make_uint4(tl[4], tl[5], tl[6], tl[7]);
  b.s = (uint32_t)s;
  return b;
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

// Lane l owns experts l, l + 64, ...  (Q = scores per lane, E <= 64*Q) and first sorts its Q
// keys in descending order.  Each round then takes the largest of the lanes' first keys: the
// wave-wide maximum of their high words on DPP, then the low word of the one lane that holds
// it (a second reduction only when several lanes tie), and that lane drops its first key.
// Every pick is wave-uniform.  The picks and their weights (softmax over the k picked scores,
// summed in a fixed order) go to sel_e[0..k) / sel_w[0..k) in LDS, and bit `tbit` of mask[e]
// is set for each pick; the caller writes the results out.
// The score of expert e is row[e] (nparts = 1) or the sum of nparts partial scores
// row[p*stride + e], added in p order.
template <int Q>
__device__ __forceinline__ void topk_wave(const float* row, int E, int k, uint16_t* sel_e, float* sel_w,
                                          uint64_t* mask, int tbit, int nparts = 1, size_t stride = 0) {
  const int lane = threadIdx.x & 63;
  float v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < E ? row[e] : 0.f;
  }
  for (int p0 = 1; p0 < nparts; p0 += 4) {  // four partials' loads in flight at a time
    float pv[4][Q];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        pv[u][q] = p0 + u < nparts && e < E ? row[(p0 + u) * stride + e] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (p0 + u < nparts) v[q] += pv[u][q];
  }
  uint64_t key[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + 64 * q;
    key[q] = e < E ? rank_key(v[q], e) : 0ull;
  }
  // descending order within the lane (odd-even transposition: Q rounds)
#pragma unroll
  for (int r = 0; r < Q; ++r)
#pragma unroll
    for (int q = r & 1; q + 1 < Q; q += 2) {
      const uint64_t a = key[q], b = key[q + 1];
      key[q] = a > b ? a : b;
      key[q + 1] = a > b ? b : a;
    }
  // Each pick is wave-uniform: lane 0 records it in sel_e / sel_w (the score for now) as soon
  // as it is known, and the softmax below reads the picks back.
  const bool lead = lane == 0;
  float vtop = 0.f;
  for (int j = 0; j < k; ++j) {
    const uint32_t mhi = (uint32_t)(key[0] >> 32), mlo = (uint32_t)key[0];
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
    if ((e & 63) == lane) {  // the owner drops its first key
#pragma unroll
      for (int q = 0; q + 1 < Q; ++q) key[q] = key[q + 1];
      key[Q - 1] = 0ull;
    }
    if (lead) {
      sel_e[j] = (uint16_t)e;
      sel_w[j] = v;
    }
  }
  // softmax over the picks: lane l takes picks l, l + 64, ... (the same order of sums as
  // before the picks moved through LDS)
  int selE[Q];
  float p[Q];
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = lane + 64 * q;
    p[q] = 0.f;
    selE[q] = 0;
    if (j < k) {
      selE[q] = sel_e[j];
      p[q] = expf(sel_w[j] - vtop);
      s += p[q];
    }
  }
  s = wave_sum_f32(s);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int j = lane + 64 * q;
    if (j < k) {
      sel_w[j] = p[q] / s;
      atomicOr(reinterpret_cast<unsigned long long*>(&mask[selE[q]]), 1ull << tbit);
    }
  }
}

// Tokens [0, T) of scores [T][E] (T <= 64), one token per wave at a time over the NT
// threads of the block.  Token t sets bit t of the expert masks; its picks go to
// sel_e/sel_w[t*k ..].
template <int NT, int Q>
__device__ __forceinline__ void topk_block(const float* scores, int T, int E, int k, uint16_t* sel_e, float* sel_w,
                                           uint64_t* mask) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t = wave; t < T; t += NT / 64)
    topk_wave<Q>(scores + (size_t)t * E, E, k, sel_e + t * k, sel_w + t * k, mask, t);
}
// Experts up to 64 * QMAX (QMAX = 16 covers the layer's limit of 1024).
template <int NT, int QMAX = 16>
__device__ __forceinline__ void topk_block_any(const float* scores, int T, int E, int k, uint16_t* sel_e,
                                               float* sel_w, uint64_t* mask) {
  if (E <= 64)
    topk_block<NT, 1>(scores, T, E, k, sel_e, sel_w, mask);
  else if (E <= 128 || QMAX < 4)
    topk_block<NT, 2>(scores, T, E, k, sel_e, sel_w, mask);
  else if (E <= 256 || QMAX < 8)
    topk_block<NT, (QMAX < 4 ? 2 : 4)>(scores, T, E, k, sel_e, sel_w, mask);
  else if (E <= 512 || QMAX < 16)
    topk_block<NT, (QMAX < 8 ? 4 : 8)>(scores, T, E, k, sel_e, sel_w, mask);
  else
    topk_block<NT, (QMAX < 16 ? 8 : 16)>(scores, T, E, k, sel_e, sel_w, mask);
}

// ------------------------------------------------------------------------------------
// Grouping tables.  One wave scans the per-expert row counts cnt[0..E) (LDS) into exclusive
// offsets offs[] (LDS; may be the same array as cnt) and the ascending list of experts with
// rows act[] (LDS), with the totals in GroupScan (LDS); it also writes the grouped GEMM's
// M-tile list when asked.  Every thread of the block then writes the tables out with one
// store per entry (write_tables), so no store waits on another.
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

struct GroupScan {
  int nact, total, nmt, nmt_routed;
};

// One wave: rows and M-tiles of each expert -> first grouped row (cnt_offs[e], in place), the
// active-expert list, each expert's first M-tile (mt_off[e], when MTILES) and the totals.
template <bool MTILES>
__device__ __forceinline__ void group_scan_wave(int* cnt_offs, int* act, int* mt_off, GroupScan* gs, int T, int E,
                                                int S) {
  const int lane = threadIdx.x & 63;
  const int J = (E + 63) >> 6;
  const int e0 = lane * J;
  int rows = 0, acts = 0, mts = 0;
  for (int i = 0; i < J; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int c = cnt_offs[e];
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
    const int c = cnt_offs[e];
    cnt_offs[e] = off;
    off += c;
    if (c > 0) act[apos++] = e;
    if (MTILES) {
      mt_off[e] = mpos;
      mpos += (c + kGemmBM - 1) / kGemmBM;
    }
  }
  if (lane == 0) {
    gs->nact = nact;
    gs->total = total;
    gs->nmt = nmt + (MTILES && S ? (T + kGemmBM - 1) / kGemmBM : 0);
    gs->nmt_routed = nmt;
  }
}

// The tables the expert kernels read, from the scan's LDS results (cnt(e) = rows of expert e,
// offs[e] = its first row, mt_off[e] = its first M-tile): counts, offsets, group rows and first
// rows, the active-group slots (shared expert last), the M-tile list (a wave per expert, its lanes
// over the expert's tiles) and the info words.  Only later kernels read them: plain stores.
template <int NT, bool MTILES, class CNT>
__device__ __forceinline__ void write_tables(const CNT& cnt, const int* offs, const int* act, const int* mt_off,
                                             const GroupScan& gs, int T, int E, int K, int S, const CallBufs& b) {
  for (int e = threadIdx.x; e < E; e += NT) {
    const int c = cnt(e), o = offs[e];
    b.counts[e] = c;
    b.offsets[e] = o;
    b.grp_row0[e] = o;
    b.grp_rows[e] = c;
  }
  // every slot of the active list, so a workgroup's one load also tells it whether it has work
  const int G = E + S, nslots = gs.nact + S;
  for (int a = threadIdx.x; a < G; a += NT) {
    GroupRec r{0, 0, 0, nslots};
    if (a < gs.nact) {
      const int e = act[a];
      r.group = e;
      r.row0 = offs[e];
      r.rows = cnt(e);
    } else if (a < nslots) {  // the shared expert
      r.group = E;
      r.row0 = T * K;
      r.rows = T;
    }
    *reinterpret_cast<int4*>(b.grec + a) = make_int4(r.group, r.row0, r.rows, r.nact);
  }
  if (MTILES) {
    const int lane = threadIdx.x & 63;
    for (int e = threadIdx.x >> 6; e < E; e += NT / 64) {
      const int nm = (cnt(e) + kGemmBM - 1) / kGemmBM, m0 = mt_off[e];
      for (int m = lane; m < nm; m += 64) {
        b.mt_group[m0 + m] = e;
        b.mt_row0[m0 + m] = m * kGemmBM;
      }
    }
    for (int i = threadIdx.x; i < gs.nmt - gs.nmt_routed; i += NT) {
      b.mt_group[gs.nmt_routed + i] = E;
      b.mt_row0[gs.nmt_routed + i] = i * kGemmBM;
    }
  }
  if (threadIdx.x == 0) {
    b.offsets[E] = gs.total;
    if (S) {
      b.grp_row0[E] = T * K;
      b.grp_rows[E] = T;
    }
    b.info[0] = gs.nact + S;
    b.info[1] = gs.nmt;
    b.info[2] = gs.nmt_routed;
  }
}

// ------------------------------------------------------------------------------------
// Grouping of at most 64 picks when only the decode kernels read it (perm, row weights and
// the active-group slots; no counts, offsets or per-token lists).  One wave: lane i holds
// pick i = t*K + j with key (expert, token); its rank among the keys is its grouped row
// (experts ascending, tokens ascending within an expert, as the full tables order them).
// The rows that start a new expert, as a ballot, give each group's slot and row count.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void lean_tables(const uint16_t* sel_e, const float* sel_w, int T, int E, int K, int S,
                                            const CallBufs& b) {
  const int lane = threadIdx.x & 63;
  const int np = T * K;  // <= 64
  const bool live = lane < np;
  const int key = live ? (int)sel_e[lane] * 64 + lane / K : 0x7FFFFFFF;
  // the lanes' keys eight at a time (lanes past np hold 0x7FFFFFFF, above every live key, so a
  // whole last group of eight counts right)
  int rank = 0;
  for (int j0 = 0; j0 < np; j0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += __builtin_amdgcn_readlane(key, j0 + u) < key;
  }
  if (!live) rank = lane;  // the rest keep their places: the ranks stay a permutation
  if (live) {
    b.perm[rank] = lane;
    b.row_w[rank] = sel_w[lane];
  }
  // lane r receives the key of rank r, then compares its expert with lane r-1's
  const int skey = __builtin_amdgcn_ds_permute(rank * 4, key);
  const int er = skey >> 6;
  const int eprev = __builtin_amdgcn_ds_bpermute(((lane + 63) & 63) * 4, skey) >> 6;
  const bool first = lane < np && (lane == 0 || er != eprev);
  const uint64_t starts = __ballot(first);
  const int nact = __popcll(starts), nslots = nact + S;
  if (first) {
    const int slot = __popcll(starts & ((1ull << lane) - 1ull));
    const uint64_t after = lane < 63 ? starts >> (lane + 1) : 0ull;
    const int next = after ? lane + 1 + __builtin_ctzll(after) : np;
    *reinterpret_cast<int4*>(b.grec + slot) = make_int4(er, lane, next - lane, nslots);
  }
  for (int a = nact + lane; a < E + S; a += 64)  // the shared expert, then count-only slots
    *reinterpret_cast<int4*>(b.grec + a) = a < nslots ? make_int4(E, np, T, nslots) : make_int4(0, 0, 0, nslots);
}

// ------------------------------------------------------------------------------------
// The routing tail of a small batch (route_fused), run by one workgroup of NT threads once
// every score is published: top-k, grouping tables, stable scatter.  Everything is built in
// LDS and written out at the end.  TailLayout<MAXE, MAXTK> sizes the caller's LDS for up to
// MAXE experts and MAXTK = T*k picks (T*E <= kTailScores always).
// ------------------------------------------------------------------------------------
template <int MAXE, int MAXTK>
struct TailLayout {
  static constexpr int kSc = 0;                           // f32 [kTailScores]
  static constexpr int kSelE = kSc + kTailScores * 4;     // u16 [MAXTK] picks of token t at [t*K, t*K+K)
  static constexpr int kSelW = kSelE + MAXTK * 2;         // f32 [MAXTK] their weights
  static constexpr int kMask = (kSelW + MAXTK * 4 + 7) / 8 * 8;  // u64 [MAXE] bit t: token t picked e
  static constexpr int kOffs = kMask + MAXE * 8;          // i32 [MAXE]
  static constexpr int kAct = kOffs + MAXE * 4;           // i32 [MAXE]
  static constexpr int kMtOff = kAct + MAXE * 4;          // i32 [MAXE]
  static constexpr int kScan = kMtOff + MAXE * 4;         // GroupScan
  static constexpr int kBytes = kScan + 16;
};

template <int NT, int QMAX, int MAXE, int MAXTK, bool MTILES, bool LEAN = false>
__device__ __forceinline__ void route_tail(const CallBufs& b, int T, int E, int K, int S, char* lds) {
  using L = TailLayout<MAXE, MAXTK>;
  float* sc = reinterpret_cast<float*>(lds + L::kSc);
  uint16_t* sel_e = reinterpret_cast<uint16_t*>(lds + L::kSelE);
  float* sel_w = reinterpret_cast<float*>(lds + L::kSelW);
  uint64_t* mask = reinterpret_cast<uint64_t*>(lds + L::kMask);
  int* offs = reinterpret_cast<int*>(lds + L::kOffs);
  int* act = reinterpret_cast<int*>(lds + L::kAct);
  int* mt_off = reinterpret_cast<int*>(lds + L::kMtOff);
  GroupScan* gs = reinterpret_cast<GroupScan*>(lds + L::kScan);
  const int tid = threadIdx.x;
  const int n = T * E;
  // every score in one round of loads, then into LDS
  for (int i0 = 0; i0 < n; i0 += NT * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * NT + tid;
      v[u] = i < n ? ld_agent(b.logits + i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * NT + tid;
      if (i < n) sc[i] = v[u];
    }
  }
  for (int i = tid; i < E; i += NT) mask[i] = 0ull;
  __syncthreads();
  topk_block_any<NT, QMAX>(sc, T, E, K, sel_e, sel_w, mask);
  __syncthreads();
  if constexpr (LEAN) {
    if (tid < 64) lean_tables(sel_e, sel_w, T, E, K, S, b);
    return;
  }
  for (int i = tid; i < E; i += NT) offs[i] = __popcll(mask[i]);
  __syncthreads();
  if (tid < 64) group_scan_wave<MTILES>(offs, act, mt_off, gs, T, E, S);
  __syncthreads();
  write_tables<NT, MTILES>([&](int e) { return __popcll(mask[e]); }, offs, act, mt_off, *gs, T, E, K, S, b);
  // pick i = t*K + j lands after the rows of lower tokens routed to the same expert
  for (int i = tid; i < T * K; i += NT) {
    const int t = i / K, e = sel_e[i];
    const float w = sel_w[i];
    const int r = offs[e] + __popcll(mask[e] & ((1ull << t) - 1ull));
    b.idx[i] = e;
    b.w[i] = w;
    b.perm[r] = (int32_t)i;
    b.row_w[r] = w;
  }
}

}  // namespace moe
