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
// the parent array into LDS and derives from it, by pointer doubling, each
// node's 2^m-th ancestor for 2^m up to the L threads it gives each row of the
// slab (L <= 16, as many as fit); thread k of a row starts at the row's k-th
// ancestor and jumps L ancestors at a time to the root (parents[j] < j bounds
// the path by j nodes), so the L threads together set the bits of every
// ancestor of the row in an LDS bitset, and their node counts sum to the
// depth. The slab (at most 16 KB of mask bytes, so at most 2 KB of bits) is
// then written with 16-byte stores, each built from at most two bitset words.
// When N is a multiple of 16 and the outputs are 16-byte aligned, both masks
// come from one pass over the slab's vectors, each inside one row and one
// bitset word. Trees of at most 64 nodes take one wave each instead (mask64,
// below): every row's ancestor set fits a 64-bit register.
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

// Both masks of the slab's rows [r0, r1) when N is a multiple of 16 and both
// outputs are 16-byte aligned: every 16-byte vector lies inside one row, its
// 16 ancestor bits inside one bitset word, and its 16 block ids in four
// aligned int4 reads. Thread t takes vectors t, t + 256, ... of the slab; its
// (row, column) advances by a constant step, so no vector needs a division,
// and each vector's ancestor bits serve both masks. out_t / out_r may be NULL
// (not written); zero: write zeros (invalid tree).
__device__ void write_masks_aligned(uint8_t* out_t, uint8_t* out_r, int N, int r0, int r1, int W,
                                    const uint32_t* bits, const int* blk, bool zero) {
  const int vpr = N >> 4;  // vectors per row, at most 64
  const int nv = (r1 - r0) * vpr;
  const int di = kThreads / vpr, dc = kThreads % vpr;
  int i = r0 + (int)threadIdx.x / vpr, c = (int)threadIdx.x % vpr;
  for (int v = threadIdx.x; v < nv; v += kThreads) {
    const int j = c << 4;
    uint32_t wt[4] = {0, 0, 0, 0}, wr[4] = {0, 0, 0, 0};
    if (!zero) {
      const uint32_t anc = (bits[(i - r0) * W + (j >> 5)] >> (j & 16)) & 0xffffu;
#pragma unroll
      for (int q = 0; q < 4; ++q) wt[q] = bits_to_bytes((anc >> (4 * q)) & 0xfu);
      if (out_r) {
        uint32_t m = anc;
        const int bi = blk[i];
        if (bi >= 0) {
          const int4* q4 = reinterpret_cast<const int4*>(blk + j);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int4 b4 = q4[q];
            m |= ((uint32_t)(b4.x == bi) | (uint32_t)(b4.y == bi) << 1 | (uint32_t)(b4.z == bi) << 2 |
                  (uint32_t)(b4.w == bi) << 3) << (4 * q);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) wr[q] = bits_to_bytes((m >> (4 * q)) & 0xfu);
      }
    }
    const int e = i * N + j;  // < 2^20
    if (out_t) *reinterpret_cast<uint4*>(out_t + e) = make_uint4(wt[0], wt[1], wt[2], wt[3]);
    if (out_r) *reinterpret_cast<uint4*>(out_r + e) = make_uint4(wr[0], wr[1], wr[2], wr[3]);
    c += dc;
    i += di;
    if (c >= vpr) {
      c -= vpr;
      ++i;
    }
  }
}

__global__ __launch_bounds__(kThreads) void sv_mask_kernel(MaskLaunch A) {
  // anc[m][j]: the 2^m-th ancestor of node j (-1 past the root); anc[0] holds
  // the parents. N <= 1024 fits a short.
  __shared__ short anc[kMaskJumpLevels + 1][kMaxMaskNodes];
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
  // every thread's loads of the parent and block arrays first, then the LDS
  // stores (one memory round trip, not one per element)
  constexpr int kPer = kMaxMaskNodes / kThreads;
  int pv[kPer], bv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    pv[k] = 0;
    bv[k] = -1;
    if (j < N) {
      pv[k] = P[j];
      if (A.blocks) bv[k] = A.blocks[(int64_t)b * N + j];
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = tid + k * kThreads;
    if (j < N) {
      const int p = pv[k];
      anc[0][j] = (short)p;  // used only when every parent is checked valid below
      blk[j] = bv[k];
      if (j == 0 ? p != -1 : (p < 0 || p >= j)) sh_bad = 1;  // same value from every writer
    }
  }
  __syncthreads();
  const bool bad = sh_bad != 0;
  const int e0 = r0 * N, e1 = r1 * N;  // N <= 1024: a tree's mask has at most 2^20 bytes
  // L = 2^lg threads per row of the slab, as many as fit, up to 16, and at
  // most about sqrt(N) / 2: every doubling pass costs about two walk steps,
  // which shallow small trees do not recover (measured: a 60-node tree's
  // masks are faster at L = 2 than at 4)
  const int nrows = r1 - r0;
  const int lgcap = min(kMaskJumpLevels, max(0, (31 - __builtin_clz((unsigned)N)) - 2) / 2);
  int lg = 0;
  while (lg < lgcap && (nrows << (lg + 1)) <= kThreads) ++lg;
  if (!bad) {
    // the 2^m-th ancestors, m = 1..lg, of every node a walk can visit (those
    // below r1), one doubling per pass
    for (int m = 1; m <= lg; ++m) {
      for (int j = tid; j < r1; j += kThreads) {
        const int h = anc[m - 1][j];
        anc[m][j] = (short)(h >= 0 ? anc[m - 1][h] : -1);
      }
      __syncthreads();  // `bad` and lg are the same in every thread
    }
    // thread k of row i: ancestors k, k + L, k + 2L, ... of i, each one's bit
    // ORed into the row's bitset (cleared above); the L threads of a row are
    // consecutive lanes of one wave and share the row's trip count
    const int k = tid & ((1 << lg) - 1);
    for (int i = r0 + (tid >> lg); i < r1; i += kThreads >> lg) {
      uint32_t* row = bits + (i - r0) * W;
      int a = i;
      for (int m = 0; m < lg; ++m)
        if (((k >> m) & 1) && a >= 0) a = anc[m][a];
      int cnt = 0;
      for (; a >= 0; a = anc[lg][a]) {
        atomicOr(row + (a >> 5), 1u << (a & 31));
        ++cnt;
      }
      for (int o = 1; o < (1 << lg); o <<= 1) cnt += __shfl_xor(cnt, o, kWave);
      if (k == 0 && A.out_depth) A.out_depth[(int64_t)b * N + i] = cnt - 1;
    }
  } else if (A.out_depth) {
    for (int i = r0 + tid; i < r1; i += kThreads) A.out_depth[(int64_t)b * N + i] = -1;
  }
  __syncthreads();
  uint8_t* mt = A.out_mask ? A.out_mask + (int64_t)b * N * N : nullptr;
  uint8_t* mr = A.out_relaxed ? A.out_relaxed + (int64_t)b * N * N : nullptr;
  if ((N & 15) == 0 && (((uintptr_t)mt | (uintptr_t)mr) & 15) == 0) {
    write_masks_aligned(mt, mr, N, r0, r1, W, bits, blk, bad);
  } else {
    if (mt) write_mask_range(mt, e0, e1, N, r0, W, bits, blk, false, bad);
    if (mr) write_mask_range(mr, e0, e1, N, r0, W, bits, blk, true, bad);
  }
}

// Trees of at most 64 nodes: one wave per tree, row j in lane j. A row's
// ancestors (and itself) are one 64-bit set in a register, built by pointer
// doubling over the parents with __shfl (set |= the ancestor's set, then jump
// to the ancestor's ancestor; six rounds cover any depth below 64), so no LDS
// and no barrier; the depth is its population count minus one. The relaxed
// mask adds, for every node k with the row's block id, bit k (one ballot per
// node). Each lane writes its own rows, four bytes at a time (bytes where N or
// the buffer leaves a row unaligned). An invalid tree's masks are all zero and
// its depths -1, as in the workgroup kernel.
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const unsigned lo = (unsigned)__shfl((int)(unsigned)v, src, kWave);
  const unsigned hi = (unsigned)__shfl((int)(unsigned)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void write_row64(uint8_t* out, int N, uint64_t m, bool words) {
  if (words) {
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    for (int w = 0; w < (N >> 2); ++w) o[w] = bits_to_bytes((uint32_t)(m >> (4 * w)) & 0xfu);
  } else {
    for (int t = 0; t < N; ++t) out[t] = (uint8_t)((m >> t) & 1u);
  }
}

__global__ __launch_bounds__(kWave) void sv_mask64_kernel(MaskLaunch A) {
  const int j = threadIdx.x, b = blockIdx.x, N = A.N;
  const bool in = j < N;
  int p = -1, bl = -1;
  if (in) {
    p = A.parents[(int64_t)b * N + j];
    if (A.blocks) bl = A.blocks[(int64_t)b * N + j];
  }
  const bool ok = (j == 0) ? p == -1 : (p >= 0 && p < j);
  const bool bad = __ballot(in && !ok) != 0ull;  // the same in every lane
  uint64_t anc = 0, rel = 0;
  int depth = -1;
  if (!bad) {
    int up = in ? p : -1;
    anc = in ? ((1ull << j) | (up >= 0 ? 1ull << up : 0ull)) : 0ull;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      const int src = up >= 0 ? up : j;
      const uint64_t a2 = shfl_u64(anc, src);
      const int u2 = __shfl(up, src, kWave);
      if (up >= 0) {
        anc |= a2;
        up = u2;
      }
    }
    depth = in ? __popcll(anc) - 1 : -1;
    rel = anc;
    if (A.out_relaxed) {
      for (int k = 0; k < N; ++k) {
        const int bk = __builtin_amdgcn_readlane(bl, k);
        if (bk >= 0 && bl == bk) rel |= 1ull << k;
      }
    }
  }
  if (!in) return;
  if (A.out_depth) A.out_depth[(int64_t)b * N + j] = depth;
  const int64_t row = (int64_t)b * N * N + (int64_t)j * N;
  if (A.out_mask) {
    uint8_t* o = A.out_mask + row;
    write_row64(o, N, anc, (N & 3) == 0 && ((uintptr_t)A.out_mask & 3) == 0);
  }
  if (A.out_relaxed) {
    uint8_t* o = A.out_relaxed + row;
    write_row64(o, N, rel, (N & 3) == 0 && ((uintptr_t)A.out_relaxed & 3) == 0);
  }
}

hipError_t launch_mask(const MaskLaunch& A, hipStream_t stream) {
  if (A.N <= kWave)
    hipLaunchKernelGGL(sv_mask64_kernel, dim3((unsigned)A.B), dim3(kWave), 0, stream, A);
  else
    hipLaunchKernelGGL(sv_mask_kernel, dim3((unsigned)((int64_t)A.B * A.nslab)), dim3(kThreads), 0, stream, A);
  return hipGetLastError();
}

}  // namespace sv
