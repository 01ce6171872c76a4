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
// as a flat byte range with 16-byte stores.
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

// Writes bytes [e0, e1) of a tree's [N][N] mask (flat index e = i * N + j);
// zero: write zeros (invalid tree).
__device__ void write_mask_range(uint8_t* out, int64_t e0, int64_t e1, int N, int r0, int W, const uint32_t* bits,
                                 const int* blk, bool relaxed, bool zero) {
  const int tid = threadIdx.x;
  // head: bytes up to the first 16-byte boundary
  int64_t a = (int64_t)(((uintptr_t)(out + e0) + 15) & ~(uintptr_t)15) - (int64_t)(uintptr_t)out;
  if (a > e1) a = e1;
  for (int64_t e = e0 + tid; e < a; e += blockDim.x)
    out[e] = zero ? 0 : mask_byte((int)(e / N), (int)(e % N), r0, W, bits, blk, relaxed);
  // body: 16 bytes per thread per iteration
  const int64_t nvec = (e1 - a) / 16;
  for (int64_t v = tid; v < nvec; v += blockDim.x) {
    const int64_t e = a + v * 16;
    uint32_t w[4] = {0, 0, 0, 0};
    if (!zero) {
      int i = (int)(e / N), j = (int)(e % N);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        w[k >> 2] |= (uint32_t)mask_byte(i, j, r0, W, bits, blk, relaxed) << (8 * (k & 3));
        if (++j == N) {
          j = 0;
          ++i;
        }
      }
    }
    *reinterpret_cast<uint4*>(out + e) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // tail
  for (int64_t e = a + nvec * 16 + tid; e < e1; e += blockDim.x)
    out[e] = zero ? 0 : mask_byte((int)(e / N), (int)(e % N), r0, W, bits, blk, relaxed);
}

__global__ __launch_bounds__(kThreads) void sv_mask_kernel(MaskLaunch A) {
  __shared__ int par[kMaxMaskNodes], blk[kMaxMaskNodes];
  __shared__ uint32_t bits[kMaskSlabBytes / 32];  // slab rows x W words
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
  const int64_t e0 = (int64_t)r0 * N, e1 = (int64_t)r1 * N;
  if (!bad) {
    // one thread per row: the path to the root
    for (int i = r0 + tid; i < r1; i += kThreads) {
      uint32_t* row = bits + (i - r0) * W;
      int d = 0;
      for (int a = i; a >= 0; a = par[a]) {
        row[a >> 5] |= 1u << (a & 31);
        ++d;
      }
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
