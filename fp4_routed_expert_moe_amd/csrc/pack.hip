// One-time repack of FP4 expert weights from the checkpoint layout into the layout the
// kernels stream.
//
// Checkpoint layout (row-major, per group g):   codes [N][K/2],       scales [N][K/32]
// Kernel layout (block-interleaved, per group):  codes [K/32][N][16],
//                                                scales [K/128][N/64][16][4][4] (see below)
//
// In the kernel layout the 16 code bytes of block kb of rows n, n+1, ... are adjacent, so a
// wave whose lanes own consecutive rows reads 1 KiB contiguous per instruction, and the
// scales of those rows are 64 contiguous bytes.  "Add DeepSeek V4 Flash CPU inference with
// NVMe expert streaming" (PR #165) repacks pinned experts the same way for its SIMD kernels
// (16 rows interleaved per vector lane, packed once per expert).
//
// Each workgroup transposes a tile of 64 rows x 64 blocks through LDS, reading and writing
// whole 16-byte chunks with consecutive threads on consecutive addresses.
//
// e8m0 edges.  A scale byte s means the float with bit pattern s << 23 ("DeepSeek V4: the
// CUDA kernels, as a tier rather than an engine", PR #772, the note on the MXFP4 decode), so
// s = 0 is +0: every value of such a block is 0.  OCP MX reads byte 0 as 2^-127 instead, so
// the repack writes the 16 code bytes of an s = 0 block as zeros: the block is then exactly 0
// whichever reading the matrix cores take.  s = 255 (+inf here, NaN under OCP MX) is kept:
// either reading makes the block's products non-finite, and the kernels carry non-finite
// intermediate values on as NaN.
#include "common.h"

namespace moe {

constexpr int kPackTile = 64;

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint4* __restrict__ in, const uint8_t* __restrict__ sc,
                                                         uint4* __restrict__ out, int N, int KB, int ntiles) {
  __shared__ uint4 tile[kPackTile][kPackTile + 1];
  const int g = blockIdx.x / ntiles;
  const int n0 = (blockIdx.x - g * ntiles) * kPackTile;
  const int kb0 = blockIdx.y * kPackTile;
  const size_t gin = (size_t)g * N * KB;
  for (int i = threadIdx.x; i < kPackTile * kPackTile; i += 256) {
    const int r = i / kPackTile, c = i % kPackTile;  // c fastest: contiguous chunks of one row
    const int n = n0 + r, kb = kb0 + c;
    if (n < N && kb < KB) {
      const size_t o = gin + (size_t)n * KB + kb;  // chunk o = block kb of row n; its scale is byte o
      tile[r][c] = sc[o] ? in[o] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kPackTile * kPackTile; i += 256) {
    const int c = i / kPackTile, r = i % kPackTile;  // r fastest: contiguous rows of one block
    const int n = n0 + r, kb = kb0 + c;
    if (n < N && kb < KB) out[gin + (size_t)kb * N + n] = tile[r][c];
  }
}

// Scales into the kernel layout [KI][NT][16 m][4 q][4 j] (KI = ceil(K/128), NT = ceil(N/64)):
// byte (i, t, m, q, j) is the scale of row 64t + 16j + m, block 4i + q, or 0 past the matrix.
// One thread per output dword (the four j of one (i, t, m, q)).
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ in, uint32_t* __restrict__ out,
                                                          int N, int KB, int groups) {
  const int KI = (KB + 3) / 4, NT = (N + 63) / 64;
  const size_t per_group = (size_t)KI * NT * 64;  // dwords
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= per_group * groups) return;
  const int g = (int)(id / per_group);
  size_t r = id - (size_t)g * per_group;
  const int q = (int)(r & 3), m = (int)((r >> 2) & 15);
  r >>= 6;
  const int t = (int)(r % NT), i = (int)(r / NT);
  const int kb = 4 * i + q;
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 64 * t + 16 * j + m;
    if (n < N && kb < KB) v |= (uint32_t)in[((size_t)g * N + n) * KB + kb] << (8 * j);
  }
  out[id] = v;
}

// FP8 codes [G][N][K] -> [G][K/128][N][128]: the 128-byte chunks of each row transposed, one
// 16-byte piece per thread (consecutive threads on consecutive output bytes).
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint4* __restrict__ in, uint4* __restrict__ out, int N,
                                                       int KC, size_t total) {
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;  // output piece
  if (id >= total) return;
  const int p = (int)(id & 7);                               // piece of the 128-byte chunk
  size_t r = id >> 3;
  const int n = (int)(r % N);
  r /= N;
  const int kc = (int)(r % KC);
  const size_t g = r / KC;
  out[id] = in[((g * N + n) * KC + kc) * 8 + p];
}

hipError_t launch_pack_fp8(const uint8_t* codes_in, uint8_t* codes_out, int groups, int N, int K, hipStream_t s) {
  const int KC = K / kFp8Block;
  const size_t total = (size_t)groups * N * KC * 8;
  const int tk = timing_begin("pack_fp8", s);
  pack_fp8_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(reinterpret_cast<const uint4*>(codes_in),
                                                                   reinterpret_cast<uint4*>(codes_out), N, KC, total);
  timing_end(tk, s);
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* codes_in, const uint8_t* scales_in, uint8_t* codes_out, uint8_t* scales_out,
                       int groups, int N, int K, hipStream_t s) {
  const int KB = K / 32;
  const int ntiles = (N + kPackTile - 1) / kPackTile;
  dim3 grid(ntiles * groups, (KB + kPackTile - 1) / kPackTile);
  int tk = timing_begin("pack_codes", s);
  pack_codes_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<const uint4*>(codes_in), scales_in,
                                         reinterpret_cast<uint4*>(codes_out), N, KB, ntiles);
  timing_end(tk, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tk = timing_begin("pack_scales", s);
  const size_t dwords = scale_slab_bytes(N, K) / 4 * groups;
  pack_scales_kernel<<<(unsigned)((dwords + 255) / 256), 256, 0, s>>>(scales_in, reinterpret_cast<uint32_t*>(scales_out),
                                                                      N, KB, groups);
  timing_end(tk, s);
  return hipGetLastError();
}

}  // namespace moe
