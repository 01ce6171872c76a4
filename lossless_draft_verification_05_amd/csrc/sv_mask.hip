// sv_mask.hip -- attention masks of a draft tree on gfx950.
//
// Method ("Falcon: Faster and Parallel Inference of Large Language Models
// through Enhanced Semi-Autoregressive Drafting and Custom-Designed Decoding
// Tree", Pith review: "What carries the argument", "Assumptions & free
// parameters"): the target scores every branch of the draft tree in one pass,
// so node i may attend exactly to its ancestors and itself (the tree mask);
// the drafter's relaxed causal mask additionally lets the tokens of one k-token
// block attend to each other.
//
// One 256-thread workgroup per (tree, slab of mask rows). The workgroup loads
// the parent array into LDS; one thread per row of the slab walks from its
// node to the root (parents[j] < j bounds the walk by j steps), setting the
// bits of the row's ancestors in an LDS bitset and counting the depth. The
// slab (at most 64 KB of mask bytes, so at most 8 KB of bits) is then written
// as a flat byte range with 16-byte stores, each built from at most two
// bitset words.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_plan.hpp"

namespace sv {

// Mask byte (i, j) of the slab whose rows start at r0; bits holds W words per row.
__device__ __forceinline__ uint8_t mask_byte(int i, int j, int r0, int W, const uint32_t* bits, const int* blk,
                                             bool relaxed) {
  const bool anc = (bits[(i - r0) * W + (j >> 5)] >> (j & 31)) & 1u;
  if (!relaxed) return anc;
  return anc || (blk[i] >= 0 && blk[i] == blk[j]);
}

// Four mask bits (x in 0..15) as four 0/1 bytes, bit k in byte k: the shifted
// copies of x (by 0, 7, 14, 21) occupy disjoint bit ranges, so the product
// has no carries.
__device__ __forceinline__ uint32_t bits_to_bytes(uint32_t x) { return (x * 0x204081u) & 0x01010101u; }

// Bits j..j+15 of a bitset row of W words (j + 16 <= the row's bit count).
__device__ __forceinline__ uint32_t row_bits16(const uint32_t* row, int j, int W) {
  const int wi = j >> 5;
  const uint64_t two = (uint64_t)row[wi] | ((uint64_t)(wi + 1 < W ? row[wi + 1] : 0u) << 32);
  return (uint32_t)(two >> (j & 31)) & 0xffffu;
}

// Writes bytes [e0, e1) of a tree's [N][N] mask (flat index e = i * N + j < 2^20);
// zero: write zeros (invalid tree). Each thread writes 16-byte vectors; a
// vector inside one row takes its 16 ancestor bits from at most two bitset
// words and, for the relaxed mask, compares its 16 block ids with the row's
// (read 4 at a time when aligned: the lanes' 64-byte strides make single-id
// reads collide in the LDS banks); one that crosses a row end is built byte by
// byte.
__device__ void write_mask_range(uint8_t* out, int e0, int e1, int N, int r0, int W, const uint32_t* bits,
                                 const int* blk, bool relaxed, bool zero) {
  const int tid = threadIdx.x;
  // head: bytes up to the first 16-byte boundary
  int a = (int)((((uintptr_t)(out + e0) + 15) & ~(uintptr_t)15) - (uintptr_t)out);
  if (a > e1) a = e1;
  for (int e = e0 + tid; e < a; e += blockDim.x)
    out[e] = zero ? 0 : mask_byte(e / N, e % N, r0, W, bits, blk, relaxed);
  // body: 16 bytes per thread per iteration
  const int nvec = (e1 - a) / 16;
  for (int v = tid; v < nvec; v += blockDim.x) {
    const int e = a + v * 16;
    uint32_t w[4] = {0, 0, 0, 0};
    if (!zero) {
      const int i = e / N, j = e % N;
      if (j + 16 <= N) {
        uint32_t m = row_bits16(bits + (i - r0) * W, j, W);
        if (relaxed) {
          const int bi = blk[i];
          if (bi >= 0) {
            if ((j & 3) == 0) {
              const int4* q4 = reinterpret_cast<const int4*>(blk + j);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int4 v = q4[q];
                m |= ((uint32_t)(v.x == bi) | (uint32_t)(v.y == bi) << 1 | (uint32_t)(v.z == bi) << 2 |
                      (uint32_t)(v.w == bi) << 3) << (4 * q);
              }
            } else {
#pragma unroll
              for (int k = 0; k < 16; ++k) m |= (uint32_t)(blk[j + k] == bi) << k;
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = bits_to_bytes((m >> (4 * q)) & 0xfu);
      } else {
        int ii = i, jj = j;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          w[k >> 2] |= (uint32_t)mask_byte(ii, jj, r0, W, bits, blk, relaxed) << (8 * (k & 3));
          if (++jj == N) {
            jj = 0;
            ++ii;
          }
        }
      }
    }
    *reinterpret_cast<uint4*>(out + e) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // tail
  for (int e = a + nvec * 16 + tid; e < e1; e += blockDim.x)
    out[e] = zero ? 0 : mask_byte(e / N, e % N, r0, W, bits, blk, relaxed);
}

__global__ __launch_bounds__(kThreads) void sv_mask_kernel(MaskLaunch A) {
  __shared__ int par[kMaxMaskNodes];
  __shared__ __align__(16) int blk[kMaxMaskNodes];
  __shared__ uint32_t bits[kMaskSlabBytes / 32];  // slab rows x W words: ancestors (and the node itself)
  __shared__ int sh_bad;
  const int N = A.N, tid = threadIdx.x;
  const int b = blockIdx.x / A.nslab, slab = blockIdx.x % A.nslab;
  const int32_t* P = A.parents + (int64_t)b * N;
  const int W = (N + 31) >> 5;
  const int r0 = slab * A.rows_per_slab, r1 = min(N, r0 + A.rows_per_slab);
  if (tid == 0) sh_bad = 0;
  for (int k = tid; k < (r1 - r0) * W; k += kThreads) bits[k] = 0;
  __syncthreads();
  for (int j = tid; j < N; j += kThreads) {
    const int p = P[j];
    par[j] = p;
    blk[j] = A.blocks ? A.blocks[(int64_t)b * N + j] : -1;
    if (j == 0 ? p != -1 : (p < 0 || p >= j)) sh_bad = 1;  // same value from every writer
  }
  __syncthreads();
  const bool bad = sh_bad != 0;
  const int e0 = r0 * N, e1 = r1 * N;  // N <= 1024: a tree's mask has at most 2^20 bytes
  if (!bad) {
    // one thread per row: the path to the root. Ancestors strictly decrease,
    // so each bitset word is visited in one run: it is built in a register and
    // stored once when the walk leaves it (the bitset was cleared above).
    for (int i = r0 + tid; i < r1; i += kThreads) {
      uint32_t* row = bits + (i - r0) * W;
      int d = 0, cw = i >> 5;
      uint32_t cur = 0;
      for (int a = i; a >= 0; a = par[a]) {
        if ((a >> 5) != cw) {
          row[cw] = cur;
          cw = a >> 5;
          cur = 0;
        }
        cur |= 1u << (a & 31);
        ++d;
      }
      row[cw] = cur;
      if (A.out_depth) A.out_depth[(int64_t)b * N + i] = d - 1;
    }
  } else if (A.out_depth) {
    for (int i = r0 + tid; i < r1; i += kThreads) A.out_depth[(int64_t)b * N + i] = -1;
  }
  __syncthreads();
  if (A.out_mask)
    write_mask_range(A.out_mask + (int64_t)b * N * N, e0, e1, N, r0, W, bits, blk, false, bad);
  if (A.out_relaxed)
    write_mask_range(A.out_relaxed + (int64_t)b * N * N, e0, e1, N, r0, W, bits, blk, true, bad);
}

hipError_t launch_mask(const MaskLaunch& A, hipStream_t stream) {
  hipLaunchKernelGGL(sv_mask_kernel, dim3((unsigned)((int64_t)A.B * A.nslab)), dim3(kThreads), 0, stream, A);
  return hipGetLastError();
}

}  // namespace sv
