// sv_sample.hip -- speculative-sampling verify on gfx950.
//
// Method ("Fast Inference from Transformers via Speculative Decoding", Pith
// review: "The pith", "What carries the argument", "Desk Editor's Note",
// "Referee Report" Summary/Significance, "Circularity Check"): per sequence,
// p_i = softmax(target_i / T), q_i = softmax(draft_i / T); accept x_i while
// u_i < p_i(x_i) / q_i(x_i); at the first rejection n redraw from
// max(0, p_n - q_n), or after full acceptance draw from p_gamma; the draw is an
// inverse CDF in token order at u_gamma.
//
// Four kernels, each a flat grid of 256-thread workgroups, ordered on the
// caller's stream (kernel boundaries are the only synchronisation: a
// per-workgroup agent-scope release would write back the L2 of its XCD, which
// serialises across the device and costs more than the streaming itself):
//  stats  : one workgroup per (row, chunk) of every target and draft row. It
//           streams 16-byte units, 4 KB per load instruction, and keeps a per-lane
//           tempered sum-exp against a lazily moved reference; one partial per
//           workgroup goes to the workspace.
//  accept : one workgroup per sequence merges its partials, gathers p(x), q(x),
//           runs the accept tests and the first-rejection scan (one ballot) and
//           writes a plan for the draw.
//  resid  : one workgroup per (sequence, chunk) of the one row pair the draw
//           needs (residual) or the bonus row; each wave writes exact masses of
//           2048-token steps and the workgroup a chunk total.
//  draw   : one workgroup per sequence walks chunk totals -> step totals -> one
//           rescanned step to the token whose running mass first exceeds
//           u * total, and writes the outputs.
#include "sv_device.hpp"

namespace sv {

constexpr int kMaxRows = 2 * 64 + 1;

// ---------------------------------------------------------------------------
// streaming tempered sum-exp
// ---------------------------------------------------------------------------
struct SumExp {
  float m_ref;   // terms are exp2((x - m_ref) * kl)
  float m_true;  // running maximum
  double s;
};

template <int DT, int NU>
__device__ __forceinline__ void sumexp_units(SumExp& st, const Unit<DT> (&un)[NU], float kl) {
  constexpr int E = Unit<DT>::kEpu;
  float gm = unit_max(un[0]);
#pragma unroll
  for (int j = 1; j < NU; ++j) gm = fmaxf(gm, unit_max(un[j]));
  st.m_true = fmaxf(st.m_true, gm);
  // The reference only moves when new values would push a term past 2^64, so
  // the rescale below is taken about once per lane and per row.
  if ((gm - st.m_ref) * kl > 64.0f) {
    st.s *= (double)hw_exp2((st.m_ref - gm) * kl);
    st.m_ref = gm;
  }
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    float e[E];
#pragma unroll
    for (int k = 0; k < E; ++k) e[k] = hw_exp2((un[j].x[k] - st.m_ref) * kl);
    float a;
    if constexpr (E == 8)
      a = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    else
      a = (e[0] + e[1]) + (e[2] + e[3]);
    st.s += (double)a;
  }
}

// The workgroup streams units [c_begin, c_end) of a row with V elements; thread
// t takes units c_begin + t + 256 k, so every load instruction of the
// workgroup covers one contiguous 4 KB block.
template <int DT>
__device__ __forceinline__ void stream_sumexp(const char* __restrict__ row, int V, int64_t c_begin, int64_t c_end,
                                              float kl, SumExp& st) {
  constexpr int E = Unit<DT>::kEpu;
  const int tid = threadIdx.x;
  const int64_t nu_row = ((int64_t)V + E - 1) / E;
  const bool ragged = (V % E) != 0;
  int64_t full_end = c_end;
  if (ragged && full_end > nu_row - 1) full_end = nu_row - 1;
  int64_t base = c_begin;
  for (; base + (int64_t)kThreads * kU1 <= full_end; base += (int64_t)kThreads * kU1) {
    uint4 w[kU1];
#pragma unroll
    for (int j = 0; j < kU1; ++j) w[j] = load16(row + (base + tid + kThreads * j) * 16);
    Unit<DT> un[kU1];
#pragma unroll
    for (int j = 0; j < kU1; ++j) un[j].unpack(w[j]);
    sumexp_units<DT, kU1>(st, un, kl);
  }
#pragma unroll
  for (int j = 0; j < kU1; ++j) {
    int64_t u = base + tid + kThreads * j;
    if (u < c_end) {
      Unit<DT> un[1];
      un[0].unpack(load16(row + u * 16));
      if (ragged && u == nu_row - 1) mask_tail(un[0], u, V);
      sumexp_units<DT, 1>(st, un, kl);
    }
  }
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, int v) {
  if constexpr (DT == 1) {
    uint32_t h = *reinterpret_cast<const uint16_t*>(row + (int64_t)v * 2);
    return __uint_as_float(h << 16);
  } else {
    return *reinterpret_cast<const float*>(row + (int64_t)v * 4);
  }
}

// ---------------------------------------------------------------------------
// stats kernel
// ---------------------------------------------------------------------------
template <int TD, int DD>
__global__ __launch_bounds__(kThreads) void sv_stats_kernel(SampleLaunch A) {
  __shared__ float sh_m[kWaves], sh_mt[kWaves];
  __shared__ double sh_s[kWaves];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & (kWave - 1);
  const int64_t wg = blockIdx.x;
  const int b = (int)(wg / A.per_seq);
  const int r = (int)(wg % A.per_seq);
  const float T = A.temps[b];
  const float kl = temp_ok(T) ? log2e_over(T) : 1.0f;
  const int G = A.gamma;
  const int tchunks = (G + 1) * A.nct;

  SumExp st{-FLT_MAX, -INFINITY, 0.0};
  if (r < tchunks) {
    const int row = r / A.nct, c = r % A.nct;
    const char* p = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)row * A.t_row_b;
    const int64_t nu = ((int64_t)A.V * Unit<TD>::kEsz + 15) / 16;
    const int64_t u0 = (int64_t)c * A.cut;
    const int64_t u1 = u0 + A.cut < nu ? u0 + A.cut : nu;
    stream_sumexp<TD>(p, A.V, u0, u1, kl, st);
  } else {
    const int rr = r - tchunks;
    const int row = rr / A.ncd, c = rr % A.ncd;
    const char* p = A.dft + (int64_t)b * A.d_seq_b + (int64_t)row * A.d_row_b;
    const int64_t nu = ((int64_t)A.V * Unit<DD>::kEsz + 15) / 16;
    const int64_t u0 = (int64_t)c * A.cud;
    const int64_t u1 = u0 + A.cud < nu ? u0 + A.cud : nu;
    stream_sumexp<DD>(p, A.V, u0, u1, kl, st);
  }

  // wave -> workgroup merge of (reference, sum, max)
  const float M = wave_max(st.m_ref);
  double s = st.s * (double)hw_exp2((st.m_ref - M) * kl);
  s = wave_sum(s);
  const float mt = wave_max(st.m_true);
  if (lane == 0) {
    sh_m[w] = M;
    sh_s[w] = s;
    sh_mt[w] = mt;
  }
  __syncthreads();
  if (tid == 0) {
    float Mb = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));
    double sb = 0.0;
    for (int k = 0; k < kWaves; ++k) sb += sh_s[k] * exp2(((double)sh_m[k] - (double)Mb) * (double)kl);
    RowPartial rp;
    rp.m_ref = Mb;
    rp.m_true = fmaxf(fmaxf(sh_mt[0], sh_mt[1]), fmaxf(sh_mt[2], sh_mt[3]));
    rp.s = sb;
    A.part[wg] = rp;
  }
}

// ---------------------------------------------------------------------------
// accept kernel: one workgroup per sequence
// ---------------------------------------------------------------------------
template <int TD, int DD>
__global__ __launch_bounds__(kThreads) void sv_accept_kernel(SampleLaunch A) {
  __shared__ float rM[kMaxRows];
  __shared__ double rS[kMaxRows];
  __shared__ int rV[kMaxRows];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & (kWave - 1);
  const int b = blockIdx.x;
  const float T = A.temps[b];
  const bool tv = temp_ok(T);
  const float kl = tv ? log2e_over(T) : 1.0f;
  const int G = A.gamma;
  const int tchunks = (G + 1) * A.nct;

  // merge the chunk partials of every row, in chunk order
  const int nrows = 2 * G + 1;
  for (int t = tid; t < nrows; t += kThreads) {
    int nch, base;
    if (t <= G) {
      nch = A.nct;
      base = t * A.nct;
    } else {
      nch = A.ncd;
      base = tchunks + (t - G - 1) * A.ncd;
    }
    const RowPartial* P = A.part + (int64_t)b * A.per_seq + base;
    float Mr = -FLT_MAX, mtr = -INFINITY;
    for (int c = 0; c < nch; ++c) {
      Mr = fmaxf(Mr, P[c].m_ref);
      mtr = fmaxf(mtr, P[c].m_true);
    }
    double S = 0.0;
    for (int c = 0; c < nch; ++c) S += P[c].s * exp2(((double)P[c].m_ref - (double)Mr) * (double)kl);
    const double St = S * exp2(((double)Mr - (double)mtr) * (double)kl);
    rM[t] = mtr;
    rS[t] = St;
    rV[t] = tv && __builtin_isfinite(St) && St > 0.0 && __builtin_isfinite(mtr);
  }
  __syncthreads();
  if (w != 0) return;

  int code = 1;  // 1 accepted, 0 rejected, 2 invalid
  if (lane < G) {
    const int i = lane;
    const int xi = A.tokens[(int64_t)b * G + i];
    const float ui = A.uniforms[(int64_t)b * (G + 1) + i];
    bool ok = tv && rV[i] && rV[G + 1 + i] && xi >= 0 && xi < A.V && ui >= 0.0f && ui < 1.0f;
    float pxo = __builtin_nanf(""), qxo = __builtin_nanf("");
    if (ok) {
      const float lt = load_elem<TD>(A.tgt + (int64_t)b * A.t_seq_b + (int64_t)i * A.t_row_b, xi);
      const float ld = load_elem<DD>(A.dft + (int64_t)b * A.d_seq_b + (int64_t)i * A.d_row_b, xi);
      if (ld == -INFINITY) ok = false;
      if (ok) {
        const double lp2 = ((double)lt - (double)rM[i]) * (double)kl;
        const double lq2 = ((double)ld - (double)rM[G + 1 + i]) * (double)kl;
        const double Sp = rS[i], Sq = rS[G + 1 + i];
        const double rho = exp2(lp2 - lq2) * (Sq / Sp);
        pxo = (float)(exp2(lp2) / Sp);
        qxo = (float)(exp2(lq2) / Sq);
        code = ((double)ui < rho) ? 1 : 0;
      }
    }
    if (!ok) code = 2;
    if (A.diag_px) A.diag_px[(int64_t)b * G + i] = pxo;
    if (A.diag_qx) A.diag_qx[(int64_t)b * G + i] = qxo;
  }
  const unsigned long long stop = __ballot(code != 1);
  const int n = stop ? (__ffsll((long long)stop) - 1) : G;
  const int code_n = __shfl(code, n < G ? n : 0, kWave);
  if (lane == 0) {
    const float ug = A.uniforms[(int64_t)b * (G + 1) + G];
    bool valid = tv && (n == G || code_n == 0) && ug >= 0.0f && ug < 1.0f;
    if (n == G) valid = valid && rV[G];
    SeqPlan P;
    P.valid = valid;
    P.n = n;
    P.mode = (n == G) ? kModeBonus : kModeResidual;
    P.kl = kl;
    P.mp = rM[n];
    P.sp = rS[n];
    if (n < G) {
      P.mq = rM[G + 1 + n];
      P.sq = rS[G + 1 + n];
      const double kap = P.sp / P.sq;
      P.kap_hi = (float)kap;
      P.kap_lo = (float)(kap - (double)P.kap_hi);
    } else {
      P.mq = 0.0f;
      P.sq = 1.0;
      P.kap_hi = 0.0f;
      P.kap_lo = 0.0f;
    }
    A.plan[b] = P;
  }
}

// ---------------------------------------------------------------------------
// draw kernel
// ---------------------------------------------------------------------------
// Unnormalised mass of the 8 tokens of octet `oct` (token ids 8*oct .. 8*oct+7):
// residual mode r_v = max(0, e^p_v - kappa e^q_v) = Sp * max(0, p_v - q_v);
// bonus mode r_v = e^p_v = Sp * p_v. Tokens at or beyond V get 0.
template <int DT>
__device__ __forceinline__ void load_octet(const char* row, int64_t oct, int V, float (&x)[8]) {
  if constexpr (DT == 1) {
    Unit<1> un;
    un.unpack(load16(row + oct * 16));
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = un.x[k];
  } else {
    Unit<0> a, c;
    a.unpack(load16(row + oct * 32));
    if (oct * 8 + 4 < V) {
      c.unpack(load16(row + oct * 32 + 16));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) c.x[k] = -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a.x[k];
      x[4 + k] = c.x[k];
    }
  }
  if (oct * 8 + 8 > V) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (oct * 8 + k >= V) x[k] = -INFINITY;
  }
}

template <int TD, int DD>
__device__ __forceinline__ void octet_mass(const char* trow, const char* drow, int64_t oct, int V, int mode,
                                           const SeqPlan& P, float (&r)[8]) {
  float xt[8];
  load_octet<TD>(trow, oct, V, xt);
  if (mode == kModeResidual) {
    float xd[8];
    load_octet<DD>(drow, oct, V, xd);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float ep = hw_exp2((xt[k] - P.mp) * P.kl);
      const float eq = hw_exp2((xd[k] - P.mq) * P.kl);
      float d = fmaf(-eq, P.kap_hi, ep);
      d = fmaf(-eq, P.kap_lo, d);
      r[k] = fmaxf(d, 0.0f);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = hw_exp2((xt[k] - P.mp) * P.kl);
  }
}

__device__ __forceinline__ float sum8(const float (&r)[8]) {
  return ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
}

// Chunk c of the draw row(s) of sequence b: per-step masses and the chunk mass.
// Called by a whole workgroup.
template <int TD, int DD>
__device__ void draw_chunk(const SampleLaunch& A, int b, const SeqPlan& P, int c, int mode, double* sh_w) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & (kWave - 1);
  const char* trow = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)P.n * A.t_row_b;
  const char* drow = (mode == kModeResidual) ? A.dft + (int64_t)b * A.d_seq_b + (int64_t)P.n * A.d_row_b : nullptr;
  const int s0 = c * A.spc2;
  const int s1 = min(s0 + A.spc2, A.ns2);
  const int64_t noct = ((int64_t)A.V + 7) / 8;
  double wacc = 0.0;
  for (int s = s0 + w; s < s1; s += kWaves) {
    double lacc = 0.0;
#pragma unroll
    for (int j = 0; j < kU2; ++j) {
      const int64_t oct = (int64_t)s * kStepOctets + kWave * j + lane;
      if (oct < noct) {
        float rr[8];
        octet_mass<TD, DD>(trow, drow, oct, A.V, mode, P, rr);
        lacc += (double)sum8(rr);
      }
    }
    const double tot = wave_sum(lacc);
    if (lane == 0) A.steptot[(int64_t)b * A.ns2 + s] = tot;
    wacc += tot;
  }
  if (lane == 0) sh_w[w] = wacc;
  __syncthreads();
  if (tid == 0) A.chunktot[(int64_t)b * A.nc2 + c] = ((sh_w[0] + sh_w[1]) + sh_w[2]) + sh_w[3];
  __syncthreads();
}

// Wave-wide search over arr[0..len): the first i (in order) whose running mass
// acc + arr[0] + ... + arr[i] exceeds t, with arr[i] > 0. If rounding leaves no
// such i, the last i with arr[i] > 0. On return acc holds the mass before i.
__device__ int wave_find(const double* arr, int len, double t, double& acc, int lane) {
  double run = acc;
  int last_i = -1;
  double last_acc = acc;
  for (int base = 0; base < len; base += kWave) {
    const int i = base + lane;
    const double v = (i < len) ? arr[i] : 0.0;
    const double incl = wave_incl_scan(v, lane);
    double excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0;
    const unsigned long long hit = __ballot(v > 0.0 && run + incl > t);
    if (hit) {
      const int L = __ffsll((long long)hit) - 1;
      acc = run + __shfl(excl, L, kWave);
      return base + L;
    }
    const unsigned long long pos = __ballot(v > 0.0);
    if (pos) {
      const int L = 63 - __clzll((long long)pos);
      last_i = base + L;
      last_acc = run + __shfl(excl, L, kWave);
    }
    run += __shfl(incl, kWave - 1, kWave);
  }
  acc = last_acc;
  return last_i;
}

template <int TD, int DD>
__global__ __launch_bounds__(kThreads) void sv_resid_kernel(SampleLaunch A) {
  __shared__ double sh_w[kWaves];
  const int b = blockIdx.x / A.nc2;
  const int c = blockIdx.x % A.nc2;
  const SeqPlan P = A.plan[b];
  if (P.valid) draw_chunk<TD, DD>(A, b, P, c, P.mode, sh_w);
}

template <int TD, int DD>
__global__ __launch_bounds__(kThreads) void sv_draw_kernel(SampleLaunch A) {
  __shared__ double sh_w[kWaves];
  __shared__ double sh_total;
  __shared__ int sh_y;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & (kWave - 1);
  const int b = blockIdx.x;
  const SeqPlan P = A.plan[b];
  const int G = A.gamma;
  int32_t* otok = A.out_tok + (int64_t)b * (G + 1);
  if (!P.valid) {
    for (int k = tid; k <= G; k += kThreads) otok[k] = -1;
    if (tid == 0) {
      A.out_n[b] = -1;
      if (A.diag_mass) A.diag_mass[b] = __builtin_nanf("");
    }
    return;
  }
  const double* ctot = A.chunktot + (int64_t)b * A.nc2;
  const double* stot = A.steptot + (int64_t)b * A.ns2;
  if (tid == 0) {
    double tot = 0.0;
    for (int k = 0; k < A.nc2; ++k) tot += ctot[k];
    sh_total = tot;
  }
  __syncthreads();
  int mode = P.mode;
  if (!(sh_total > 0.0) && mode == kModeResidual) {
    // Nothing left after the rejection (p_n == q_n up to rounding): draw from p_n.
    // Rare slow path: this workgroup recomputes every chunk of target row n.
    mode = kModeBonus;
    for (int k = 0; k < A.nc2; ++k) draw_chunk<TD, DD>(A, b, P, k, mode, sh_w);
    // draw_chunk ends with a workgroup barrier: every step and chunk mass this
    // workgroup wrote is visible to all of its waves
    if (tid == 0) {
      double tot = 0.0;
      for (int k = 0; k < A.nc2; ++k) tot += ctot[k];
      sh_total = tot;
    }
    __syncthreads();
  }
  const double total = sh_total;
  if (w == 0) {
    const double t = (double)A.uniforms[(int64_t)b * (G + 1) + G] * total;
    double acc = 0.0;
    // wave_find returns -1 only if every mass is zero, which valid rows rule out;
    // clamp anyway so that no index can leave the arrays.
    const int cc = max(wave_find(ctot, A.nc2, t, acc, lane), 0);
    const int s0 = cc * A.spc2;
    const int s1 = min(s0 + A.spc2, A.ns2);
    const int ss = s0 + max(wave_find(stot + s0, s1 - s0, t, acc, lane), 0);
    // rescan the step in token order: octet j-major, then lane, then slot
    const char* trow = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)P.n * A.t_row_b;
    const char* drow = (mode == kModeResidual) ? A.dft + (int64_t)b * A.d_seq_b + (int64_t)P.n * A.d_row_b : nullptr;
    const int64_t noct = ((int64_t)A.V + 7) / 8;
    int y = -1;
    int last_pos = -1;
    for (int j = 0; j < kU2 && y < 0; ++j) {
      const int64_t oct = (int64_t)ss * kStepOctets + kWave * j + lane;
      float rr[8];
      if (oct < noct) {
        octet_mass<TD, DD>(trow, drow, oct, A.V, mode, P, rr);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) rr[k] = 0.0f;
      }
      const double os = (double)sum8(rr);
      const double incl = wave_incl_scan(os, lane);
      double excl = __shfl_up(incl, 1, kWave);
      if (lane == 0) excl = 0.0;
      int lk = -1;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (rr[k] > 0.0f) lk = k;
      if (lk >= 0) last_pos = (int)(oct * 8 + lk);  // later j / lanes have larger ids
      const unsigned long long hit = __ballot(os > 0.0 && acc + incl > t);
      if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        int yy = -1;
        if (lane == L) {
          double run = acc + excl;
          for (int k = 0; k < 8; ++k) {
            if (rr[k] > 0.0f) {
              run += (double)rr[k];
              if (run > t) {
                yy = (int)(oct * 8 + k);
                break;
              }
            }
          }
          if (yy < 0) yy = (int)(oct * 8 + lk);
        }
        y = __shfl(yy, L, kWave);
      } else {
        acc += __shfl(incl, kWave - 1, kWave);
      }
    }
    if (y < 0) {
      // rounding pushed t past the step's rescanned mass: take its last positive token
      int m = last_pos;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
      y = m;
    }
    if (lane == 0) sh_y = y;
  }
  __syncthreads();
  const int y = sh_y;
  const int n = P.n;
  for (int k = tid; k <= G; k += kThreads)
    otok[k] = (k < n) ? A.tokens[(int64_t)b * G + k] : (k == n ? y : -1);
  if (tid == 0) {
    A.out_n[b] = n;
    if (A.diag_mass) A.diag_mass[b] = (float)(total / P.sp);
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int TD, int DD>
static hipError_t launch_pair(const SampleLaunch& A, int stage, hipStream_t stream) {
  switch (stage) {
    case 1:
      hipLaunchKernelGGL((sv_stats_kernel<TD, DD>), dim3((unsigned)((int64_t)A.B * A.per_seq)), dim3(kThreads), 0,
                         stream, A);
      break;
    case 2:
      hipLaunchKernelGGL((sv_accept_kernel<TD, DD>), dim3((unsigned)A.B), dim3(kThreads), 0, stream, A);
      break;
    case 3:
      hipLaunchKernelGGL((sv_resid_kernel<TD, DD>), dim3((unsigned)((int64_t)A.B * A.nc2)), dim3(kThreads), 0,
                         stream, A);
      break;
    default:
      hipLaunchKernelGGL((sv_draw_kernel<TD, DD>), dim3((unsigned)A.B), dim3(kThreads), 0, stream, A);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_sample_stage(const SampleLaunch& A, int tdt, int ddt, int stage, hipStream_t stream) {
  if (tdt == 1 && ddt == 1) return launch_pair<1, 1>(A, stage, stream);
  if (tdt == 1 && ddt == 0) return launch_pair<1, 0>(A, stage, stream);
  if (tdt == 0 && ddt == 1) return launch_pair<0, 1>(A, stage, stream);
  return launch_pair<0, 0>(A, stage, stream);
}

}  // namespace sv
