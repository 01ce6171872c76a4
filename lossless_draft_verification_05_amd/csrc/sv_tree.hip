// sv_tree.hip -- greedy decoding-tree verify on gfx950.
//
// Method ("Falcon: ... Custom-Designed Decoding Tree", Pith review: "What
// carries the argument" -- the target checks all candidate branches of the
// draft tree in one pass; "Assumptions & free parameters" and Figure 4 --
// greedy decoding must reproduce vanilla autoregressive output): node j is
// accepted iff its parent is accepted and its token is the argmax of the
// parent's target row; the result is the deepest accepted node d (lowest id on
// ties), its root path and the bonus token argmax(row d).
//
// Two kernels on the caller's stream (the launch boundary is the only
// synchronisation; see the sampling kernels for why no intra-kernel handoff):
//  argmax : a workgroup per (sequence, node row, chunk) streams 16-byte units
//           (4 KB per load instruction) and keeps a per-lane (max, first
//           index) pair; one partial per workgroup.
//  tree   : a workgroup per tree merges the row partials and resolves the tree
//           in LDS by pointer jumping over the parent array (log2 N rounds),
//           which also leaves a binary-lifting table for writing the accepted
//           path in parallel; trees of at most 64 nodes take one wave and do
//           the same in registers (tree64).
#include "sv_device.hpp"

namespace sv {

struct ArgState {
  float best;
  int idx;
  bool nan;
};

template <int DT, int NU>
__device__ __forceinline__ void argmax_units(ArgState& st, const Unit<DT> (&un)[NU], const int64_t (&u)[NU]) {
  constexpr int E = Unit<DT>::kEpu;
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    bool nan = false;
#pragma unroll
    for (int k = 0; k < E; k += 2) nan |= __builtin_isunordered(un[j].x[k], un[j].x[k + 1]);
    st.nan |= nan;
    const float gm = unit_max(un[j]);
    if (gm > st.best) {  // strict: earlier (lower) indices win ties inside a lane
      int kk = E - 1;
#pragma unroll
      for (int k = E - 1; k >= 0; --k)
        if (un[j].x[k] == gm) kk = k;
      st.best = gm;
      st.idx = (int)(u[j] * E + kk);
    }
  }
}

// The workgroup streams units [c_begin, c_end); thread t takes units
// c_begin + t + 256 k (one contiguous 4 KB block per load instruction), kU1
// of them per round: every load of a round is issued first (a lane past c_end
// loads the chunk's last unit and skips it), then the units are compared one
// at a time in increasing order, so strict ">" keeps the first index of a tie
// within a thread and only one unit's values are live at once.
template <int DT>
__device__ __forceinline__ void stream_argmax(const char* __restrict__ row, int V, int64_t c_begin, int64_t c_end,
                                              ArgState& st) {
  constexpr int E = Unit<DT>::kEpu;
  const int tid = threadIdx.x;
  const int64_t nu_row = ((int64_t)V + E - 1) / E;
  const bool ragged = (V % E) != 0;
  for (int64_t base = c_begin; base < c_end; base += (int64_t)kThreads * kU1) {
    uint4 w[kU1];
#pragma unroll
    for (int j = 0; j < kU1; ++j) {
      const int64_t u = base + tid + kThreads * j;
      w[j] = load16(row + (u < c_end ? u : c_end - 1) * 16);
    }
#pragma unroll
    for (int j = 0; j < kU1; ++j) {
      int64_t uu[1] = {base + tid + kThreads * j};
      if (uu[0] < c_end) {
        Unit<DT> un[1];
        un[0].unpack(w[j]);
        if (ragged && uu[0] == nu_row - 1) mask_tail(un[0], uu[0], V);
        argmax_units<DT, 1>(st, un, uu);
      }
    }
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void sv_argmax_kernel(TreeLaunch A) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int per_seq = A.N * A.nch;
  const int b = blockIdx.x / per_seq;
  const int r = blockIdx.x % per_seq;
  const int j = r / A.nch, c = r % A.nch;

  ArgState st{-INFINITY, INT_MAX, false};
  {
    const char* row = A.logits + (int64_t)b * A.seq_b + (int64_t)j * A.row_b;
    const int64_t nu = ((int64_t)A.V * Unit<DT>::kEsz + 15) / 16;
    const int64_t u0 = (int64_t)c * A.cu;
    const int64_t u1 = u0 + A.cu < nu ? u0 + A.cu : nu;
    stream_argmax<DT>(row, A.V, u0, u1, st);
  }
  float bv = st.best;
  int bi = st.idx;
  wave_argmax(bv, bi);
  const bool nan = __ballot(st.nan) != 0ull;
  // one partial per workgroup: the waves' results combined in LDS
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves], s_n[kWaves];
  if (lane == 0) {
    s_v[w] = bv;
    s_i[w] = bi;
    s_n[w] = nan ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = s_v[0];
    int i = s_i[0], bad = s_n[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
      arg_combine(v, i, s_v[k], s_i[k]);
      bad |= s_n[k];
    }
    ArgPartial p;
    p.best = v;
    p.idx = i;
    p.bad = bad;
    p.pad = 0;
    A.part[blockIdx.x] = p;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void sv_tree_kernel(TreeLaunch A) {
  __shared__ int s_ok;
  __shared__ int s_key[kWaves];
  // Resolve arrays, sized by N at launch (tree_lds_bytes):
  //   s_g[N] int | s_tk[N] int | s_up[(kLog2MaxNodes+1) * N] short | s_D[2 * N] short | s_A[2 * N] uchar
  extern __shared__ __align__(16) char s_dyn[];
  const int NN = A.N;
  int* s_g = reinterpret_cast<int*>(s_dyn);
  int* s_tk = s_g + NN;  // node tokens
  short* s_upb = reinterpret_cast<short*>(s_tk + NN);
  short* s_Db = s_upb + (kLog2MaxNodes + 1) * NN;
  unsigned char* s_Ab = reinterpret_cast<unsigned char*>(s_Db + 2 * NN);
#define s_up(k, i) s_upb[(k) * NN + (i)]
#define s_D(k, i) s_Db[(k) * NN + (i)]
#define s_A(k, i) s_Ab[(k) * NN + (i)]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & (kWave - 1);
  const int per_seq = A.N * A.nch;
  const int b = blockIdx.x;
  const int N = A.N;
  if (tid == 0) s_ok = 1;
  __syncthreads();
  const ArgPartial* P = A.part + (int64_t)b * per_seq;
  for (int jj = tid; jj < N; jj += kThreads) {
    // the node's parent and token first: their loads do not wait for the partials'
    const int pj = A.parents[(int64_t)b * N + jj];
    const int tk = A.tokens[(int64_t)b * N + jj];
    float v = -INFINITY;
    int i = INT_MAX, bad = 0;
    const ArgPartial* q = P + (int64_t)jj * A.nch;
    // the row's chunk partials, four loads in flight at a time, combined in chunk order
    for (int c0 = 0; c0 < A.nch; c0 += 4) {
      ArgPartial r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c0 + k < A.nch) r[k] = q[c0 + k];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c0 + k < A.nch) {
          arg_combine(v, i, r[k].best, r[k].idx);
          bad |= r[k].bad;
        }
    }
    if (v == INFINITY) bad = 1;  // +inf makes the row unusable
    if (v == -INFINITY) i = 0;   // a row of -inf only: first index
    s_g[jj] = i;
    if (bad) s_ok = 0;
    if (A.out_argmax) A.out_argmax[(int64_t)b * N + jj] = bad ? -1 : i;
    s_tk[jj] = tk;
    const bool node_ok = (jj == 0) ? (pj == -1) : (pj >= 0 && pj < jj && tk >= 0 && tk < A.V);
    if (!node_ok) s_ok = 0;
    s_up(0, jj) = (short)((jj == 0) ? -1 : pj);
  }
  __syncthreads();
  int32_t* opath = A.out_path + (int64_t)b * N;
  if (!s_ok) {
    for (int t = tid; t < N; t += kThreads) opath[t] = -1;
    if (tid == 0) {
      A.out_len[b] = -1;
      A.out_bonus[b] = -1;
    }
    return;
  }
  for (int jj = tid; jj < N; jj += kThreads) {
    const int tk = s_tk[jj];
    s_A(0, jj) = (jj == 0) ? 1 : (unsigned char)(tk == s_g[s_up(0, jj)]);
    s_D(0, jj) = (jj == 0) ? 0 : 1;
  }
  __syncthreads();
  int rounds = 0;
  while ((1 << rounds) < N) ++rounds;
  for (int k = 0; k < rounds; ++k) {
    const int cur = k & 1, nxt = cur ^ 1;
    for (int jj = tid; jj < N; jj += kThreads) {
      const int p = s_up(k, jj);
      if (p >= 0) {
        s_A(nxt, jj) = s_A(cur, jj) & s_A(cur, p);
        s_D(nxt, jj) = (short)(s_D(cur, jj) + s_D(cur, p));
        s_up(k + 1, jj) = s_up(k, p);
      } else {
        s_A(nxt, jj) = s_A(cur, jj);
        s_D(nxt, jj) = s_D(cur, jj);
        s_up(k + 1, jj) = -1;
      }
    }
    __syncthreads();
  }
  const int fin = rounds & 1;
  // deepest accepted node, lowest id on ties: key = depth * 2048 + (2047 - id)
  int key = -1;
  for (int jj = tid; jj < N; jj += kThreads)
    if (s_A(fin, jj)) key = max(key, ((int)s_D(fin, jj) << 11) | (2047 - jj));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, kWave));
  if (lane == 0) s_key[w] = key;
  __syncthreads();
  key = max(max(s_key[0], s_key[1]), max(s_key[2], s_key[3]));
  const int d = 2047 - (key & 2047);
  const int depth = key >> 11;
  for (int t = tid; t < N; t += kThreads) {
    int node = -1;
    if (t <= depth) {
      node = d;
      const int dist = depth - t;
      for (int k = 0; k < rounds && node >= 0; ++k)
        if ((dist >> k) & 1) node = s_up(k, node);
    }
    opath[t] = node;
  }
  if (tid == 0) {
    A.out_len[b] = depth;
    A.out_bonus[b] = s_g[d];
  }
#undef s_up
#undef s_D
#undef s_A
}

// Trees of at most 64 nodes: one wave per tree, node j in lane j, and the
// same resolve as sv_tree_kernel by pointer jumping in registers (ds_bpermute
// reads another lane's value), so no LDS and no barrier: acc, depth and the
// 2^k-th ancestor of every node after k rounds, the deepest accepted node
// (lowest id on ties) by a wave maximum of the same key, then each path entry
// by binary lifting over the saved ancestor registers.
constexpr int kWaveTreeRounds = 6;  // ceil(log2 64)
template <int DT>
__global__ __launch_bounds__(kWave) void sv_tree64_kernel(TreeLaunch A) {
  const int j = threadIdx.x;  // node
  const int b = blockIdx.x;
  const int N = A.N;
  const bool in = j < N;
  const int per_seq = A.N * A.nch;
  int pj = -1, tk = 0;
  if (in) {
    // the node's parent and token first: their loads do not wait for the partials'
    pj = A.parents[(int64_t)b * N + j];
    tk = A.tokens[(int64_t)b * N + j];
  }
  float v = -INFINITY;
  int i = INT_MAX, bad = 0;
  if (in) {
    const ArgPartial* q = A.part + (int64_t)b * per_seq + (int64_t)j * A.nch;
    // the row's chunk partials, four loads in flight at a time, combined in chunk order
    for (int c0 = 0; c0 < A.nch; c0 += 4) {
      ArgPartial r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c0 + k < A.nch) r[k] = q[c0 + k];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c0 + k < A.nch) {
          arg_combine(v, i, r[k].best, r[k].idx);
          bad |= r[k].bad;
        }
    }
    if (v == INFINITY) bad = 1;  // +inf makes the row unusable
    if (v == -INFINITY) i = 0;   // a row of -inf only: first index
    if (A.out_argmax) A.out_argmax[(int64_t)b * N + j] = bad ? -1 : i;
  }
  const bool node_ok = (j == 0) ? (pj == -1) : (pj >= 0 && pj < j && tk >= 0 && tk < A.V);
  int32_t* opath = A.out_path + (int64_t)b * N;
  if (__ballot(in && (bad || !node_ok)) != 0ull) {  // the same in every lane
    if (in) opath[j] = -1;
    if (j == 0) {
      A.out_len[b] = -1;
      A.out_bonus[b] = -1;
    }
    return;
  }
  const int g = i;  // argmax of row j
  int up = (j == 0 || !in) ? -1 : pj;
  const int gp = __shfl(g, up >= 0 ? up : 0, kWave);
  int acc = (j == 0) ? 1 : (in && tk == gp ? 1 : 0);
  int dep = (j == 0 || !in) ? 0 : 1;
  int rounds = 0;
  while ((1 << rounds) < N) ++rounds;
  int ups[kWaveTreeRounds];  // ups[k]: the 2^k-th ancestor (-1 past the root)
#pragma unroll
  for (int k = 0; k < kWaveTreeRounds; ++k) {
    ups[k] = up;
    if (k < rounds) {
      const int src = up >= 0 ? up : j;
      const int a2 = __shfl(acc, src, kWave), d2 = __shfl(dep, src, kWave), u2 = __shfl(up, src, kWave);
      if (up >= 0) {
        acc &= a2;
        dep += d2;
        up = u2;
      }
    }
  }
  // deepest accepted node, lowest id on ties: key = depth * 2048 + (2047 - id)
  int key = (in && acc) ? ((dep << 11) | (2047 - j)) : -1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, kWave));
  const int d = 2047 - (key & 2047);
  const int depth = key >> 11;
  // path entry t = the (depth - t)-th ancestor of d, for t <= depth
  const int dist = depth - j;
  int node = d;
#pragma unroll
  for (int k = 0; k < kWaveTreeRounds; ++k) {
    if (k < rounds) {
      const int nn = __shfl(ups[k], node, kWave);
      if (dist >= 0 && ((dist >> k) & 1)) node = nn;
    }
  }
  if (in) opath[j] = dist >= 0 ? node : -1;
  const int bonus = __shfl(g, d, kWave);
  if (j == 0) {
    A.out_len[b] = depth;
    A.out_bonus[b] = bonus;
  }
}

size_t tree_lds_bytes(int N) {
  return (size_t)N * 8 + (size_t)(kLog2MaxNodes + 1) * N * 2 + (size_t)2 * N * 2 + (size_t)2 * N + 16;
}

// stage 1: per-row argmax partials; stage 2: per-tree resolve
hipError_t launch_tree(const TreeLaunch& A, int dt, int stage, hipStream_t stream) {
  const int64_t grid = (int64_t)A.B * A.N * A.nch;
  if (stage == 1) {
    if (dt == 1)
      hipLaunchKernelGGL((sv_argmax_kernel<1>), dim3((unsigned)grid), dim3(kThreads), 0, stream, A);
    else
      hipLaunchKernelGGL((sv_argmax_kernel<0>), dim3((unsigned)grid), dim3(kThreads), 0, stream, A);
  } else if (A.N <= kWave) {
    if (dt == 1)
      hipLaunchKernelGGL((sv_tree64_kernel<1>), dim3((unsigned)A.B), dim3(kWave), 0, stream, A);
    else
      hipLaunchKernelGGL((sv_tree64_kernel<0>), dim3((unsigned)A.B), dim3(kWave), 0, stream, A);
  } else {
    if (dt == 1)
      hipLaunchKernelGGL((sv_tree_kernel<1>), dim3((unsigned)A.B), dim3(kThreads), tree_lds_bytes(A.N), stream, A);
    else
      hipLaunchKernelGGL((sv_tree_kernel<0>), dim3((unsigned)A.B), dim3(kThreads), tree_lds_bytes(A.N), stream, A);
  }
  return hipGetLastError();
}

}  // namespace sv
