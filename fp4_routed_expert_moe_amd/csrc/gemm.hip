// Prefill path: expert-grouped GEMM over the sorted token rows on the block-scaled matrix
// cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine" (PR #1055, "What it is",
// prefill MoE) runs expert-grouped GEMM rows after routing on the device.  Here:
//
// * Weights (B) enter the matrix cores as stored: e2m1 codes with their e8m0 block scales, no
//   convert instruction touches them.  Each wave loads its own weight operands from the
//   block-interleaved kernel layout straight into registers.
// * Activations (A) are exact FP8 (e4m3) term splits with an e8m0 scale per 32 values: x as
//   two terms (all 8 bf16 significand bits, written by the router kernel), h as two terms
//   (about 8 significant bits, the precision of bf16) written by the gate/up epilogue.  One
//   MFMA per term, all accumulating in fp32.
// * A workgroup takes one M-tile (64 grouped rows of one group, from the device-built M-tile
//   list) and a slice of output columns; four waves each own a column slice of all 64 rows:
//   64 columns (4 16x16 tiles) in the down kernel; 32 or 64 columns of gate and of up at once
//   in the gate/up kernel (so SwiGLU stays in registers), the wider slice when the groups are
//   large enough to keep the matrix cores busy (it halves the LDS reads per MFMA but has one
//   weight step in flight instead of two).  16-row subtiles past the group's last row are
//   skipped.
// * The activation tile of each 128-value K step goes straight from memory into LDS (buffer
//   loads with the LDS flag, no registers), three buffers deep: while step s runs on the
//   matrix cores, step s+2's tile streams in.  LDS rows are 128 bytes with their 16-byte
//   chunks permuted by row (chunk c of row r sits at c ^ (r & 7)), which keeps the matrix-
//   operand reads (16 rows, one chunk each) free of bank conflicts.  Each step ends with one
//   barrier, preceded by a wait for this wave's loads of the next tile only (counted in
//   vector-memory instructions, not a full drain).
// * Workgroups reach the 8 XCDs round-robin (b % 8).  XCD x takes every 8th M-tile (or, for
//   large groups, every 8th run of two consecutive M-tiles, so that a group of two tiles reads
//   its weights into one XCD's L2), every column slice of each in turn: an M-tile's activation
//   rows are fetched into one XCD's L2 only, and with small batches (one M-tile per expert)
//   the XCDs stream different experts.  Blocks of 8 runs come alternately from the front and
//   the back of the tile list, so that skewed batches run their many-tile groups (matrix-core
//   bound) beside their one-tile groups (weight-stream bound).
#include <type_traits>

#include "common.h"

namespace moe {

constexpr int kPM = kGemmBM;      // rows per M-tile (64)

// Per-kernel shape: NW waves of CT 16-column tiles each (PN = NW * CT * 16 columns per
// workgroup); PU = 128-value MFMA K chunks per step; OCC = workgroups per CU the register
// budget targets; BS = weight-operand register stages (their loads run BS - 1 steps ahead).
template <int NW_, int CT_, int PU_, int OCC_, int BS_>
struct GemmShape {
  static constexpr int NW = NW_;
  static constexpr int CT = CT_;
  static constexpr int NTH = 64 * NW;      // threads
  static constexpr int PU = PU_;
  static constexpr int OCC = OCC_;
  static constexpr int BS = BS_;
  static constexpr int PK = 128 * PU;      // K values per step
  static constexpr int PKB = PK / 32;      // K blocks per step
  static constexpr int ALD = PK;           // LDS row pitch of the activation tile (bytes; chunks permuted)
  static constexpr int PN = NW * CT * 16;  // output columns per workgroup
};
using GateUpShape = GemmShape<4, 2, 1, 2, 3>;      // 32 columns of gate and of up per wave
using GateUpWideShape = GemmShape<4, 4, 1, 2, 2>;  // 64 columns of each (256 VGPRs, no spill)
using DownShape = GemmShape<4, 4, 1, 3, 3>;        // three workgroups per CU (164 VGPRs)
// The FP8 shared expert's kernels: the same tiles at one workgroup per CU (its weight operands
// are twice the FP4 ones' registers)
using GateUpShape8 = GemmShape<4, 2, 1, 1, 3>;
using DownShape8 = GemmShape<4, 4, 1, 1, 3>;
// Gate/up takes the wide column slices from this many grouped rows per group on average (the
// measured crossing point at H 4096, I 2048 lies between 30 and 45 rows per group).
constexpr int kWideRowsPerGroup = 40;
inline bool gateup_wide(const Dims& d, int T) {
  return (long long)T * (d.K + d.S) >= (long long)kWideRowsPerGroup * d.G;
}
// Workgroups meet the XCDs in runs of M-tiles: 2 (a group of two M-tiles, common at these
// sizes, then reads its weights into one XCD's L2) when the groups are as large as for the wide
// slices, else 1 (round-robin; a hot expert's tiles spread over all XCDs).  Measured at H 4096,
// I 2048: runs of 2 take 4096 uniform tokens from 1.75 to 1.60 ms per step and 4096 zipf tokens
// from 1.63 to 1.61, and cost about 1% at 512 uniform tokens; runs of 4 or a contiguous eighth
// per XCD did no better.
inline int tile_run_log2(const Dims& d, int T) { return gateup_wide(d, T) ? 1 : 0; }
inline int tile_grid(int tiles, int rl, int NT) { return (tiles + (8 << rl) - 1) / (8 << rl) * (8 << rl) * NT; }

template <class SH>
struct ATile {                    // one K step of the activation tile
  uint8_t v[2][kPM][SH::ALD];     // FP8 terms
  uint8_t s[kPM][SH::PKB];        // e8m0 scales of the step's K blocks
};

// Activation rows: term planes hi/lo [rows][K] bytes and scales [rows][kb_pad(K)].
struct ARows {
  const uint8_t* hi;
  const uint8_t* lo;
  const uint8_t* sc;
  int K;
  int rows;
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// The activation tile is loaded straight into LDS (buffer loads with the LDS flag): one such
// load fills 1 KB, lane l writing bytes 16l..16l+15, i.e. 8 tile rows of one term, lane l
// covering physical chunk l % 8 of row l / 8.  Wave w fills rows 16w..16w+15 of both terms;
// since physical chunk p of row r holds logical chunk p ^ (r & 7), lane l fetches logical
// chunk (l % 8) ^ (l / 8) of its rows 16w + l/8 and 16w + 8 + l/8.  Wave 0 also loads the 64
// rows' scale dwords of the step (lane l: row l).  Chunks past K in the last step (K % 128
// != 0) read the row's last 16 bytes instead; the scale rows are padded to whole steps with
// byte 127 and the weights there read as zero codes, so those products are 0.
struct ADma {
  __amdgpu_buffer_rsrc_t hi, lo, sc;
  int ra, rb;   // byte offsets of this lane's two rows in a term plane
  int rs;       // wave 0: byte offset of row `lane`'s scales
  int lc16;     // 16 * logical chunk
};
template <class SH>
__device__ __forceinline__ void a_dma(ATile<SH>& t, const ADma& d, int K, int step, int wave) {
  int off = 128 * step + d.lc16;
  if (off >= K) off = K - 16;
  lds_u8* base = (lds_u8*)(&t);
  lds_u8* p0 = base + 2048 * wave;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.hi, p0, 16, d.ra + off, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.hi, p0 + 1024, 16, d.rb + off, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.lo, p0 + kPM * 128, 16, d.ra + off, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.lo, p0 + kPM * 128 + 1024, 16, d.rb + off, 0, 0, 0);
  if (wave == 0)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.sc, base + 2 * kPM * 128, 4, d.rs + 4 * step, 0, 0, 0);
}
// Keeps the compiler from moving memory accesses across this point: the waits below count
// vector-memory instructions in issue order.  (The weight pointers reach the kernel without
// __restrict__ for the same reason: loads the compiler may treat as reading invariant memory
// can be moved across such a point.)
__device__ __forceinline__ void mem_order() { asm volatile("" ::: "memory"); }
// Wait until this wave's tile loads issued before the last kNewer vector-memory instructions
// are done, and for its LDS reads, then meet the other waves: the tile those loads filled is
// then complete for every wave, and every wave's reads of the tile being refilled next are over.
template <int kNewer>
__device__ __forceinline__ void tile_barrier() {
  static_assert(kNewer < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kNewer) : "memory");
}

// Weight operands of one wave for one K step: PU chunks x NM matrices x CT column tiles.
// Lane (n, q) reads K block 4u + q of its column: one 16-byte chunk and its scale byte (from
// the kernel scale layout, where a lane's four 16-row tiles share a dword).  The loads go
// through buffer descriptors spanning one group's matrix, so the per-lane offset is fixed and
// the K position is a scalar offset.
template <class SH, int NM>
struct BFrag {
  i32x4 c[SH::PU][NM][SH::CT];
  int s[SH::PU][NM];  // scale dword of the lane's four 16-row tiles
};
template <class SH, int NM>
struct BSrc {
  __amdgpu_buffer_rsrc_t c[NM], s[NM];
  int voff_c;  // column tile 0, K block q, step 0
  int voff_s;  // scale dword of this wave's 64-row tile, K block q, step 0
  int nt64;    // 64-row tiles of the matrix
};
constexpr int kBufferFlags = 0x00020000;  // raw byte-addressed buffer, 32-bit data format
// Steps past the last one (the prefetch runs ahead unconditionally) and lanes whose block is
// past K move their per-lane offsets past the descriptor's range: they read zeros and touch
// no memory.  (The scalar offset is not relied on for the range check.)
constexpr int kOutOfRange = 1 << 30;
template <int AUX, class SH, int NM>
__device__ __forceinline__ void b_fetch_aux(BFrag<SH, NM>& f, const BSrc<SH, NM>& bs, int N, int KB, int step, int q) {
#pragma unroll
  for (int u = 0; u < SH::PU; ++u) {
    const int chunk = step * SH::PU + u;  // 128-value K chunk (uniform; kept in scalar registers)
    const int kb = 4 * chunk;
    const int so_c = __builtin_amdgcn_readfirstlane(kb * N * 16);
    const int so_s = __builtin_amdgcn_readfirstlane(chunk * bs.nt64 * 256);
    int bias_c = 0, bias_s = 0;
    if (kb + 4 > KB) {  // uniform
      bias_c = kb + q >= KB ? kOutOfRange : 0;
      bias_s = kb >= KB ? kOutOfRange : 0;
    }
#pragma unroll
    for (int mtx = 0; mtx < NM; ++mtx) {
#pragma unroll
      for (int c = 0; c < SH::CT; ++c)
        f.c[u][mtx][c] =
            __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(bs.c[mtx], bs.voff_c + bias_c + 256 * c, so_c, AUX));
      f.s[u][mtx] = __builtin_amdgcn_raw_buffer_load_b32(bs.s[mtx], bs.voff_s + bias_s, so_s, AUX);
    }
  }
}
// A group of one M-tile reads each weight byte once per column slice: those loads go through
// as nontemporal (they would only push out lines that other tiles reuse); a group of several
// M-tiles reads its weights once per M-tile and keeps them cached.
constexpr int kStreamAux = 2;  // nontemporal

// One K step: acc[mtx][rs][c] += A(rs) x B(mtx, c) for both FP8 terms, rs < nsub.  sh: the
// bit offset of this wave's first tile in its scale dword (0 or 16 when CT == 2).
template <class SH, int NM>
__device__ __forceinline__ void k_step(const ATile<SH>& t, const BFrag<SH, NM>& f, f32x4 (&acc)[NM][4][SH::CT],
                                       int nsub, int m, int q, int sh) {
#pragma unroll
  for (int u = 0; u < SH::PU; ++u) {
    int sb[NM];
#pragma unroll
    for (int mtx = 0; mtx < NM; ++mtx) sb[mtx] = SH::CT == 4 ? f.s[u][mtx] : (int)((uint32_t)f.s[u][mtx] >> sh);
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      // Down (one matrix): each subtile's LDS reads just before its matrix work.  Gate/up:
      // the reads of all subtiles first (the compiler hoists them out of this form), which
      // measured faster for its eight products per subtile.
      if (rs >= nsub) {
        if constexpr (NM == 1 || SH::CT == 4) continue;
        else break;
      }
      const int r = 16 * rs + m;
      const int b = 128 * u + 16 * (q ^ (m & 7)), b2 = b ^ 64;  // (r & 7 == m & 7)
      const i32x8 a0 = __builtin_shufflevector(*reinterpret_cast<const i32x4*>(&t.v[0][r][b]),
                                               *reinterpret_cast<const i32x4*>(&t.v[0][r][b2]), 0, 1, 2, 3, 4,
                                               5, 6, 7);
      const i32x8 a1 = __builtin_shufflevector(*reinterpret_cast<const i32x4*>(&t.v[1][r][b]),
                                               *reinterpret_cast<const i32x4*>(&t.v[1][r][b2]), 0, 1, 2, 3, 4,
                                               5, 6, 7);
      const int sa = t.s[r][4 * u + q];
#pragma unroll
      for (int c = 0; c < SH::CT; ++c)
#pragma unroll
        for (int mtx = 0; mtx < NM; ++mtx) {
          // FP4 reads the low four registers of the operand; the rest are left undefined
          const i32x8 bb = __builtin_shufflevector(f.c[u][mtx][c], f.c[u][mtx][c], 0, 1, 2, 3, -1, -1, -1, -1);
          f32x4 x = acc[mtx][rs][c];
          switch (c) {  // B's scale: byte c of sb
            case 0: x = mma_f8f4_sb<0>(a0, bb, x, sa, sb[mtx]); x = mma_f8f4_sb<0>(a1, bb, x, sa - 4, sb[mtx]); break;
            case 1: x = mma_f8f4_sb<1>(a0, bb, x, sa, sb[mtx]); x = mma_f8f4_sb<1>(a1, bb, x, sa - 4, sb[mtx]); break;
            case 2: x = mma_f8f4_sb<2>(a0, bb, x, sa, sb[mtx]); x = mma_f8f4_sb<2>(a1, bb, x, sa - 4, sb[mtx]); break;
            default: x = mma_f8f4_sb<3>(a0, bb, x, sa, sb[mtx]); x = mma_f8f4_sb<3>(a1, bb, x, sa - 4, sb[mtx]); break;
          }
          acc[mtx][rs][c] = x;
        }
    }
  }
}

// ---- the FP8 shared expert's weights (e4m3, float32 scale per 128 x 128 block) ----------
// Kernel layout [K/128][N][128]; lane (n, q) takes bytes 16q.. and 64+16q.. of its row's
// 128-value chunk (the FP8 lane layout, the same as the activations').  A wave's CT tiles lie in
// one 128-row scale block, so one float32 per chunk and matrix scales the wave's products,
// applied after the chunk's two MFMAs (one per activation term).
template <class SH, int NM>
struct BFrag8 {
  i32x4 c[SH::PU][NM][SH::CT][2];
  float s[SH::PU][NM];
};
template <class SH, int NM>
struct BSrc8 {
  __amdgpu_buffer_rsrc_t c[NM];
  const float* s[NM];  // the wave's row block of each matrix's scales, indexed by chunk
  int voff;            // column tile 0, chunk 0
};
template <int AUX, class SH, int NM>
__device__ __forceinline__ void b_fetch_aux(BFrag8<SH, NM>& f, const BSrc8<SH, NM>& bs, int N, int KB, int step,
                                            int q) {  // (the FP8 shared expert spans many M-tiles: cached)
  (void)q;
#pragma unroll
  for (int u = 0; u < SH::PU; ++u) {
    const int chunk = step * SH::PU + u;
    const bool past = 4 * chunk >= KB;  // the prefetch runs past the last step: read zeros
    const int so = __builtin_amdgcn_readfirstlane(past ? 0 : chunk * N * 128);
    const int bias = past ? kOutOfRange : 0;
#pragma unroll
    for (int mtx = 0; mtx < NM; ++mtx) {
#pragma unroll
      for (int c = 0; c < SH::CT; ++c) {
        f.c[u][mtx][c][0] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(bs.c[mtx], bs.voff + bias + 2048 * c, so, 0));
        f.c[u][mtx][c][1] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(bs.c[mtx], bs.voff + bias + 2048 * c + 64, so, 0));
      }
      f.s[u][mtx] = past ? 0.f : bs.s[mtx][chunk];
    }
  }
}
template <class SH, int NM>
__device__ __forceinline__ void k_step(const ATile<SH>& t, const BFrag8<SH, NM>& f, f32x4 (&acc)[NM][4][SH::CT],
                                       int nsub, int m, int q, int sh) {
  (void)sh;
#pragma unroll
  for (int u = 0; u < SH::PU; ++u) {
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      if (rs >= nsub) break;
      const int r = 16 * rs + m;
      const int b = 128 * u + 16 * (q ^ (m & 7)), b2 = b ^ 64;  // (r & 7 == m & 7)
      const i32x8 a0 = __builtin_shufflevector(*reinterpret_cast<const i32x4*>(&t.v[0][r][b]),
                                               *reinterpret_cast<const i32x4*>(&t.v[0][r][b2]), 0, 1, 2, 3, 4,
                                               5, 6, 7);
      const i32x8 a1 = __builtin_shufflevector(*reinterpret_cast<const i32x4*>(&t.v[1][r][b]),
                                               *reinterpret_cast<const i32x4*>(&t.v[1][r][b2]), 0, 1, 2, 3, 4,
                                               5, 6, 7);
      const int sa = t.s[r][4 * u + q];
#pragma unroll
      for (int c = 0; c < SH::CT; ++c)
#pragma unroll
        for (int mtx = 0; mtx < NM; ++mtx) {
          const i32x8 bb = __builtin_shufflevector(f.c[u][mtx][c][0], f.c[u][mtx][c][1], 0, 1, 2, 3, 4, 5, 6, 7);
          f32x4 p = mma_f8f8(a0, bb, f32x4{0.f, 0.f, 0.f, 0.f}, sa);
          p = mma_f8f8(a1, bb, p, sa - 4);
          acc[mtx][rs][c] += p * f.s[u][mtx];
        }
    }
  }
}

// 4 x 4 byte transpose within a lane quad: lane u of the quad holds byte i = element (i, u)
// and gets byte c = element (u, c).  Two exchange steps: bytes with the neighbour lane, then
// 16-bit halves with the lane two over.
__device__ __forceinline__ uint32_t quad_byte_transpose(uint32_t w, int u) {
  const uint32_t p = dpp_u32<kQuadXor1>(w);
  const uint32_t n = (u & 1) ? (((p >> 8) & 0x00FF00FFu) | (w & 0xFF00FF00u))
                             : ((w & 0x00FF00FFu) | ((p & 0x00FF00FFu) << 8));
  const uint32_t p2 = dpp_u32<kQuadXor2>(n);
  return (u & 2) ? ((p2 >> 16) | (n & 0xFFFF0000u)) : ((n & 0xFFFFu) | (p2 << 16));
}

// 4 x 4 transpose of dwords within a lane quad: lane u holds v[i] = element (i, u) and gets
// v[c] = element (u, c).  Two exchange steps: elements with the neighbour lane, then pairs of
// elements with the lane two over.
__device__ __forceinline__ void quad_transpose4(float (&v)[4], int u) {
  const bool odd = u & 1;
  const float r0 = __uint_as_float(dpp_u32<kQuadXor1>(__float_as_uint(odd ? v[0] : v[1])));
  const float r1 = __uint_as_float(dpp_u32<kQuadXor1>(__float_as_uint(odd ? v[2] : v[3])));
  if (odd) {
    v[0] = r0;
    v[2] = r1;
  } else {
    v[1] = r0;
    v[3] = r1;
  }
  const bool upper = u & 2;
  const float s0 = __uint_as_float(dpp_u32<kQuadXor2>(__float_as_uint(upper ? v[0] : v[2])));
  const float s1 = __uint_as_float(dpp_u32<kQuadXor2>(__float_as_uint(upper ? v[1] : v[3])));
  if (upper) {
    v[0] = s0;
    v[1] = s1;
  } else {
    v[2] = s0;
    v[3] = s1;
  }
}

// ------------------------------------------------------------------------------------
// GATEUP: h[r][n] = silu(x_t(r) . Wg[n]) * (x_t(r) . Wu[n]) as 2 FP8 terms + e8m0 per 32
//         (h8 = [2][R][I] bytes then [R][kb_pad(I)] scales).
// DOWN:   staging[slot(r)][n] = weight(r) * (h_r . Wd[n])  (wts: weight of grouped row r).
// ------------------------------------------------------------------------------------
// FP8: the M-tiles of the FP8 shared expert (info[2] .. info[1]), weights c0p/c1p as FP8 codes
// and f0p/f1p their float32 block scales.  Otherwise the FP4 M-tiles [0, info[1]), or
// [0, info[2]) when routed_only (the shared expert is FP8 and has its own launch).
// slot_of (FP4 only; NULL = every group at its own index): group g's weights are at index
// slot_of[g] of the weight arrays, and the M-tiles of groups with slot_of[g] < 0 are skipped
// (an expert bank running one refill group of experts per launch).
template <bool GATEUP, class SH, bool FP8 = false>
__global__ __launch_bounds__(SH::NTH, SH::OCC) void gemm_f8f4_kernel(
    ARows a, const uint8_t* c0p, const uint8_t* s0p, const uint8_t* c1p, const uint8_t* s1p,
    const float* __restrict__ f0p, const float* __restrict__ f1p,
    const int32_t* __restrict__ perm, const float* __restrict__ wts,
    const int32_t* __restrict__ info, const int32_t* __restrict__ mt_group, const int32_t* __restrict__ mt_row0,
    const int32_t* __restrict__ grp_row0, const int32_t* __restrict__ grp_rows, const int32_t* __restrict__ slot_of,
    uint8_t* __restrict__ h8, float* __restrict__ staging, int routed_only, float routed_scale, int T, int k, int N,
    int R, int NT, int rl) {
  constexpr int NM = GATEUP ? 2 : 1;
  static_assert(SH::PU == 1 && SH::NW == 4, "tile loads: 4 waves x 16 rows, one 128-value chunk per step");
  __shared__ ATile<SH> tile[3];
  // XCD x (= b % 8) takes runs of 2^rl consecutive M-tiles, every 8th run, all NT column slices
  // of each (the grid holds a whole number of runs per XCD).  The blocks of 8 runs are taken
  // alternately from the front and, backwards, from the back of the launch's tile list, so that
  // the tiles of large groups (matrix-core bound, their weights shared through the caches) run
  // beside those of one-tile groups (bound by their weight stream) instead of before them.
  const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3, it = jj / NT, nt = jj % NT;
  const int base = FP8 ? info[2] : 0, n_mt = (routed_only ? info[2] : info[1]) - base;
  const int nblk = (n_mt + (8 << rl) - 1) >> (rl + 3), blk = it >> rl;
  if (blk >= nblk) return;
  const int blk_f = (blk & 1) ? nblk - 1 - (blk >> 1) : (blk >> 1);
  const int mt_l = (((blk_f << 3) + xcd) << rl) + (it & ((1 << rl) - 1));
  if (mt_l >= n_mt) return;
  const int mt = base + mt_l;
  // tile metadata is the same for every lane: keep it in scalar registers
  const int g = __builtin_amdgcn_readfirstlane(mt_group[mt]);
  const int gw = slot_of ? __builtin_amdgcn_readfirstlane(slot_of[g]) : g;  // weight index of the group
  if (gw < 0) return;
  const int mr0 = __builtin_amdgcn_readfirstlane(mt_row0[mt]);
  const int r0 = __builtin_amdgcn_readfirstlane(grp_row0[g]) + mr0;  // first grouped row of the tile
  const int grp_rows_g = __builtin_amdgcn_readfirstlane(grp_rows[g]);
  const int nrows = min(kPM, grp_rows_g - mr0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, q = lane >> 4;
  const int tk = T * k;
  const int KB = a.K >> 5;
  const int nsteps = (a.K + SH::PK - 1) / SH::PK;

  // this lane's tile rows for the loads (rows past the group repeat the tile's first row)
  ADma ad;
  {
    auto srow_of = [&](int lr) {
      const int gr = r0 + (lr < nrows ? lr : 0);
      return GATEUP ? row_token(perm, gr, tk, k) : gr;
    };
    const int la = 16 * wave + (lane >> 3);
    ad.ra = srow_of(la) * a.K;
    ad.rb = srow_of(la + 8) * a.K;
    ad.rs = wave == 0 ? srow_of(lane) * kb_pad(a.K) : 0;
    ad.lc16 = 16 * ((lane & 7) ^ (lane >> 3));
    // (sizes through readfirstlane: the descriptors must stay in scalar registers)
    const int plane = __builtin_amdgcn_readfirstlane(a.rows * a.K);
    const int scb = __builtin_amdgcn_readfirstlane(a.rows * kb_pad(a.K));
    ad.hi = __builtin_amdgcn_make_buffer_rsrc((void*)a.hi, (short)0, plane, kBufferFlags);
    ad.lo = __builtin_amdgcn_make_buffer_rsrc((void*)a.lo, (short)0, plane, kBufferFlags);
    ad.sc = __builtin_amdgcn_make_buffer_rsrc((void*)a.sc, (short)0, scb, kBufferFlags);
  }

  // this wave's weight columns (columns past N read other bytes of the group or zeros; their
  // results are not stored)
  const int n0 = nt * SH::PN + wave * 16 * SH::CT;
  const uint8_t* codes[2] = {c0p, c1p};
  using BS = typename std::conditional<FP8, BSrc8<SH, NM>, BSrc<SH, NM>>::type;
  using BF = typename std::conditional<FP8, BFrag8<SH, NM>, BFrag<SH, NM>>::type;
  BS bs;
  if constexpr (FP8) {
    const float* fsc[2] = {f0p, f1p};
#pragma unroll
    for (int mtx = 0; mtx < NM; ++mtx) {
      bs.c[mtx] = __builtin_amdgcn_make_buffer_rsrc((void*)codes[mtx], (short)0, a.K * N, kBufferFlags);
      // (a wave wholly past N reads the last row block's scales; its results are not stored)
      bs.s[mtx] = fsc[mtx] + (size_t)min(n0 / kFp8Block, N / kFp8Block - 1) * (a.K / kFp8Block);
    }
    bs.voff = (n0 + m) * 128 + 16 * q;
  } else {
    const uint8_t* scales[2] = {s0p, s1p};
    const int slab = __builtin_amdgcn_readfirstlane((int)scale_slab_bytes(N, a.K));
#pragma unroll
    for (int mtx = 0; mtx < NM; ++mtx) {
      bs.c[mtx] = __builtin_amdgcn_make_buffer_rsrc((void*)(codes[mtx] + (size_t)gw * KB * N * 16), (short)0,
                                                    KB * N * 16, kBufferFlags);
      bs.s[mtx] = __builtin_amdgcn_make_buffer_rsrc((void*)(scales[mtx] + (size_t)gw * slab), (short)0, slab,
                                                    kBufferFlags);
    }
    bs.voff_c = (q * N + n0 + m) * 16;
    bs.nt64 = (N + 63) >> 6;
    bs.voff_s = (((n0 >> 6) * 16 + m) * 4 + q) * 4;
  }
  const int sh = 8 * ((n0 >> 4) & 3);  // CT == 2: this wave's tiles are bytes sh/8 and sh/8 + 1
  static_assert(SH::CT == 2 || SH::CT == 4, "a wave's tiles share one scale dword");
  const int nsub = (nrows + 15) >> 4;

  f32x4 acc[NM][4][SH::CT];
#pragma unroll
  for (int mtx = 0; mtx < NM; ++mtx)
#pragma unroll
    for (int rs = 0; rs < 4; ++rs)
#pragma unroll
      for (int c = 0; c < SH::CT; ++c) acc[mtx][rs][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pipeline: while step s runs on the matrix cores, the activation tile of step s+2 streams
  // into the third LDS buffer and the weight operands of step s+BS-1 into registers.  Per
  // step a wave issues 4 tile loads (wave 0: 5), then NB weight loads (FP4: NM * (CT + 1);
  // FP8 more), so the tile of step s+1, issued in step s-1, is complete once at most
  // 2 NB + 4 newer loads are outstanding (wave 0 waits for one more than it needs).
  // tests/test_gemm_wait_counts_cpu.py checks these counts against the compiled order.
  constexpr int kBS = SH::BS;
  static_assert(kBS == 2 || kBS == 3, "weight stages");
  constexpr int NB = NM * (SH::CT + 1);
  constexpr int kNewer = 2 * NB + 4;
  // The main loop exists twice, once per weight-load policy, chosen per workgroup (a branch
  // inside the loop would make the compiler's waits before the MFMAs drain the loads in flight).
  auto pipeline = [&](auto policy) {
    constexpr int AUX = decltype(policy)::value;
    BF fb[kBS];
    // The loads run ahead unconditionally: past the last step the tile loads repeat the last
    // step (cache hits) and the weights read zeros without memory traffic.
    const int last = nsteps - 1;
    a_dma<SH>(tile[0], ad, a.K, 0, wave);
    mem_order();
    b_fetch_aux<AUX>(fb[0], bs, N, KB, 0, q);
    mem_order();
    a_dma<SH>(tile[1], ad, a.K, min(1, last), wave);
    if constexpr (kBS == 3) {
      mem_order();
      b_fetch_aux<AUX>(fb[1], bs, N, KB, 1, q);
      tile_barrier<kNewer>();
    } else {
      tile_barrier<NB + 4>();
    }
    auto step = [&](int s, ATile<SH>& tc, ATile<SH>& t_far, BF& fc, BF& f_far, auto newer) -> bool {
      a_dma<SH>(t_far, ad, a.K, min(s + 2, last), wave);
      mem_order();
      b_fetch_aux<AUX>(f_far, bs, N, KB, s + kBS - 1, q);
      k_step(tc, fc, acc, nsub, m, q, sh);
      tile_barrier<decltype(newer)::value>();
      return s + 1 < nsteps;
    };
    const std::integral_constant<int, kNewer> steady;
    if constexpr (kBS == 3) {
      for (int s = 0; s < nsteps; s += 3) {
        if (!step(s + 0, tile[0], tile[2], fb[0], fb[2], steady)) break;
        if (!step(s + 1, tile[1], tile[0], fb[1], fb[0], steady)) break;
        if (!step(s + 2, tile[2], tile[1], fb[2], fb[1], steady)) break;
      }
    } else {
      // With one weight stage the prologue ends with step 1's tile loads, so at the end of
      // step 0 only that step's NB + 4 loads are newer: step 0 waits with that count, the
      // following steps (whose next tile came one step earlier, before NB + 4 + NB loads)
      // with 2 NB + 4.
      if (step(0, tile[0], tile[2], fb[0], fb[1], std::integral_constant<int, NB + 4>{})) {
        for (int s = 1; s < nsteps; s += 6) {
          if (!step(s + 0, tile[1], tile[0], fb[1], fb[0], steady)) break;
          if (!step(s + 1, tile[2], tile[1], fb[0], fb[1], steady)) break;
          if (!step(s + 2, tile[0], tile[2], fb[1], fb[0], steady)) break;
          if (!step(s + 3, tile[1], tile[0], fb[0], fb[1], steady)) break;
          if (!step(s + 4, tile[2], tile[1], fb[1], fb[0], steady)) break;
          if (!step(s + 5, tile[0], tile[2], fb[0], fb[1], steady)) break;
        }
      }
    }
  };
  if (!FP8 && mr0 == 0 && nrows == grp_rows_g)
    pipeline(std::integral_constant<int, kStreamAux>{});
  else
    pipeline(std::integral_constant<int, 0>{});
  // no tile load may still be writing LDS when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue ----
  if constexpr (GATEUP) {
    // h leaves through LDS in 16-byte row chunks.  A lane holds column m of rows 4q..4q+3
    // of each 16x16 tile; it packs those four bytes into a dword, a byte transpose within the
    // lane quad turns that into columns 4(m/4)..+3 of row 4q + m%4, and those dwords go to an
    // LDS copy of the workgroup's h rows.  The tile buffers are free once every wave's last
    // tile loads have landed and every wave is past its last barrier.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    constexpr int EPL = SH::PN + 16;  // LDS row pitch of the staged h (bytes; +16: no bank conflicts)
    static_assert(2 * kPM * EPL <= (int)sizeof(tile), "staged h fits the tile buffers");
    uint8_t* hl = reinterpret_cast<uint8_t*>(&tile[0]);
    uint8_t* hs = h8 + (size_t)2 * R * N;
    const int u = m & 3;
    const int lds0 = (4 * q + u) * EPL + wave * 16 * SH::CT + 4 * (m >> 2);  // this lane's dword, subtile 0
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      if (rs >= nsub) break;
#pragma unroll
      for (int p = 0; p < SH::CT / 2; ++p) {  // 32-column block = column tiles 2p, 2p+1
        const int nb = n0 + 32 * p;
        float hv[4][2];  // [row 4q + i][tile]
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 2; ++c) hv[i][c] = silu(acc[0][rs][2 * p + c][i]) * acc[1][rs][2 * p + c][i];
        float inv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // lanes with the same q hold the same row: |h| max over the block's 32 columns
          const int sc = fp8_block_scale(row16_max(fmaxf(fabsf(hv[i][0]), fabsf(hv[i][1]))));
          inv[i] = fp8_inv_scale(sc);
          const int lrow = 16 * rs + 4 * q + i;
          if (m == 0 && lrow < nrows && nb < N) {
            const size_t r = (size_t)(r0 + lrow);
            hs[r * kb_pad(N) + (nb >> 5)] = (uint8_t)sc;
            if ((nb >> 5) == (N >> 5) - 1)  // pad bytes of the row
              for (int j = N >> 5; j < kb_pad(N); ++j) hs[r * kb_pad(N) + j] = (uint8_t)127;
          }
        }
        uint32_t w[2][2];  // [term][tile]: byte i = row 4q + i
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = hv[i][c] * inv[i];
          const uint32_t t0 = pack_fp8x4(v[0], v[1], v[2], v[3]);
          const uint32_t t1 = pack_fp8x4((v[0] - __builtin_amdgcn_cvt_f32_fp8((int)t0, 0)) * 16.f,
                                         (v[1] - __builtin_amdgcn_cvt_f32_fp8((int)t0, 1)) * 16.f,
                                         (v[2] - __builtin_amdgcn_cvt_f32_fp8((int)t0, 2)) * 16.f,
                                         (v[3] - __builtin_amdgcn_cvt_f32_fp8((int)t0, 3)) * 16.f);
          uint32_t nanm = 0;  // non-finite h stays NaN in both terms
#pragma unroll
          for (int i = 0; i < 4; ++i) nanm |= fp8_nan_mask(hv[i][c]) << (8 * i);
          w[0][c] = t0 | nanm;
          w[1][c] = t1 | nanm;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            *reinterpret_cast<uint32_t*>(hl + t * kPM * EPL + lds0 + 16 * rs * EPL + 16 * (2 * p + c)) =
                quad_byte_transpose(w[t][c], u);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    constexpr int CPR = SH::PN / 16;  // 16-byte chunks per staged row
#pragma unroll
    for (int k = tid; k < 2 * kPM * CPR; k += SH::NTH) {
      const int t = k / (kPM * CPR), row = (k / CPR) % kPM, ch = k % CPR;
      const int col = nt * SH::PN + 16 * ch;
      if (row < nrows && col < N)
        *reinterpret_cast<i32x4*>(h8 + (size_t)t * R * N + (size_t)(r0 + row) * N + col) =
            *reinterpret_cast<const i32x4*>(hl + t * kPM * EPL + row * EPL + 16 * ch);
    }
  } else {
    // A 4 x 4 transpose within the lane quad turns column m of rows 4q..4q+3 into columns
    // 4(m/4)..+3 of row 4q + m%4: one 16-byte store per tile and row.  The staging slot and
    // routing weight of the four rows this lane stores, all loads first.
    const int u = m & 3;
    int slot[4];
    float wt[4];
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      const int rr = r0 + min(16 * rs + 4 * q + u, nrows - 1);
      slot[rs] = rr < tk ? perm[rr] : rr;
      wt[rs] = rr < tk ? wts[rr] * routed_scale : 1.0f;
    }
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      if (rs >= nsub) break;
      const bool row_ok = 16 * rs + 4 * q + u < nrows;
#pragma unroll
      for (int c = 0; c < SH::CT; ++c) {
        float v[4] = {acc[0][rs][c][0], acc[0][rs][c][1], acc[0][rs][c][2], acc[0][rs][c][3]};
        quad_transpose4(v, u);
        const int n = n0 + 16 * c + 4 * (m >> 2);
        if (row_ok && n < N)
          *reinterpret_cast<float4*>(&staging[(size_t)slot[rs] * N + n]) =
              make_float4(v[0] * wt[rs], v[1] * wt[rs], v[2] * wt[rs], v[3] * wt[rs]);
      }
    }
  }
}

// ------------------------------------------------------------------------------------
template <class SH>
static void gateup_fp4(const Dims& d, const moe_layer_desc& w, const CallBufs& b, const ARows& a, int T,
                       int mt_bound, hipStream_t s, const int32_t* slot_of) {
  const int NT = (d.I + SH::PN - 1) / SH::PN;
  const int R = T * (d.K + d.S);
  const int rl = tile_run_log2(d, T);
  gemm_f8f4_kernel<true, SH><<<tile_grid(mt_bound, rl, NT), SH::NTH, 0, s>>>(
      a, w.gate_codes, w.gate_scales, w.up_codes, w.up_scales, nullptr, nullptr, b.perm, b.w, b.info, b.mt_group,
      b.mt_row0, b.grp_row0, b.grp_rows, slot_of, static_cast<uint8_t*>(b.h), nullptr, d.fp8_shared, 1.0f, T, d.K,
      d.I, R, NT, rl);
}

hipError_t launch_gemm_gateup(const Dims& d, const moe_layer_desc& w, const uint16_t* x, const CallBufs& b,
                              int T, int mt_bound, hipStream_t s, const int32_t* slot_of) {
  (void)x;
  const ARows a{b.xq, b.xq + (size_t)T * d.H, b.xq + (size_t)2 * T * d.H, d.H, T};
  const int tk = timing_begin("gemm_gateup", s);
  if (gateup_wide(d, T))
    gateup_fp4<GateUpWideShape>(d, w, b, a, T, mt_bound, s, slot_of);
  else
    gateup_fp4<GateUpShape>(d, w, b, a, T, mt_bound, s, slot_of);
  timing_end(tk, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !d.fp8_shared) return e;
  const int NT = (d.I + GateUpShape8::PN - 1) / GateUpShape8::PN;
  const int R = T * (d.K + d.S);
  const int mts = (T + kGemmBM - 1) / kGemmBM;  // the shared expert's M-tiles
  const int tk8 = timing_begin("gemm_gateup_fp8", s);
  gemm_f8f4_kernel<true, GateUpShape8, true><<<tile_grid(mts, 0, NT), GateUpShape8::NTH, 0, s>>>(
      a, w.shared_gate_fp8, nullptr, w.shared_up_fp8, nullptr, w.shared_gate_fp8_scales, w.shared_up_fp8_scales,
      b.perm, b.w, b.info, b.mt_group, b.mt_row0, b.grp_row0, b.grp_rows, nullptr, static_cast<uint8_t*>(b.h),
      nullptr, 0, 1.0f, T, d.K, d.I, R, NT, 0);
  timing_end(tk8, s);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Dims& d, const moe_layer_desc& w, const CallBufs& b, int T, int mt_bound,
                            hipStream_t s, const int32_t* slot_of) {
  const int NT = (d.H + DownShape::PN - 1) / DownShape::PN;
  const int R = T * (d.K + d.S);
  const uint8_t* h8 = static_cast<const uint8_t*>(b.h);
  const ARows a{h8, h8 + (size_t)R * d.I, h8 + (size_t)2 * R * d.I, d.I, R};
  const int tk = timing_begin("gemm_down", s);
  const int rl = tile_run_log2(d, T);
  gemm_f8f4_kernel<false, DownShape><<<tile_grid(mt_bound, rl, NT), DownShape::NTH, 0, s>>>(
      a, w.down_codes, w.down_scales, w.down_codes, w.down_scales, nullptr, nullptr, b.perm, b.row_w, b.info,
      b.mt_group, b.mt_row0, b.grp_row0, b.grp_rows, slot_of, nullptr, b.staging, d.fp8_shared, d.routed_scale, T,
      d.K, d.H, R, NT, rl);
  timing_end(tk, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !d.fp8_shared) return e;
  const int mts = (T + kGemmBM - 1) / kGemmBM;
  const int tk8 = timing_begin("gemm_down_fp8", s);
  gemm_f8f4_kernel<false, DownShape8, true><<<tile_grid(mts, 0, NT), DownShape8::NTH, 0, s>>>(
      a, w.shared_down_fp8, nullptr, w.shared_down_fp8, nullptr, w.shared_down_fp8_scales,
      w.shared_down_fp8_scales, b.perm, b.row_w, b.info, b.mt_group, b.mt_row0, b.grp_row0, b.grp_rows, nullptr,
      nullptr, b.staging, 0, d.routed_scale, T, d.K, d.H, R, NT, 0);
  timing_end(tk8, s);
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
