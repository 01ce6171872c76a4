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
// Two kernels on the caller's stream (no fence-based hand-off between
// workgroups: a per-workgroup agent-scope release would write back the L2 of
// its XCD, which serialises across the device and costs more than the
// streaming itself):
//  stats  : one 256-thread workgroup per (row, chunk of 16-256 KB) of every
//           target and draft row. It streams 16-byte units (4 KB per load
//           instruction, non-temporal) and keeps a per-lane tempered sum-exp
//           against a lazily moved reference; one partial per wave.
//  finish : one 512-thread workgroup per sequence (with fewer sequences than
//           CUs, several per sequence -- 1024-thread ones where each wave
//           streams at most two steps -- that hand their step masses to the
//           last one through relaxed device-scope atomics, no fence and no
//           wait).
//           It merges the partials of the sequence's rows (a wave per row),
//           gathers p(x), q(x), runs the accept tests and the first-rejection
//           ballot, streams the one row (pair) the draw needs -- max(0, p_n -
//           q_n) after a rejection, p_gamma after full acceptance -- writing
//           exact masses of 2048-token steps, then walks step masses -> one
//           rescanned step -> one octet to the token whose running mass first
//           exceeds u_gamma * total, and writes the outputs.
// With V <= 2048 the whole call is one kernel instead (small: one wave per
// sequence; small2: two per wave when V <= 32 and 2 gamma + 1 <= 32). Also
// here: the early-exit statistics kernel (stats_pos) and the one-pass draft
// sampler (draft1).
#include <type_traits>

#include "sv_device.hpp"

namespace sv {

constexpr int kMaxRows = 2 * 64 + 1;

// ---------------------------------------------------------------------------
// streaming tempered sum-exp
// ---------------------------------------------------------------------------
// Per-lane state of the statistics pass (FMA form): s = sum of
// exp2(x * kl - c) over the lane's values so far, against an integer shift c
// (log2 units, a float holding an integer; -inf while every value seen was
// -inf). Each batch -- the lane's kU1 units of one 16 KB block of the row -- is
// summed in fp32 against its own integer shift at or just above the batch's
// maximum, so every term is at most ~1, where an fp32 exponent is finest (the
// only rounding of x * kl - c is that of the FMA's result), and the batch sum
// depends on the batch alone; it is then folded into s by exact powers of two.
// With chunks that start on 16 KB boundaries the batches, and so every fp32
// rounding, are the same however a row is split into chunks: a call's
// statistics do not depend on its batch size, only fp64 additions do.
// The subtract form exp2((x - m) * kl) is used when a shift reaches 2^24
// (tiny temperatures or huge logits), where an fp32 shift no longer holds
// every integer.
struct SumExp {
  float c;
  double s;
  int ovf;  // a batch shift reached 2^24: the chunk is redone in the subtract form
};

// Sum of exp2(x * kl - c) over the NU units of a batch, in a fixed order.
template <int DT, int NU>
__device__ __forceinline__ float terms_fma(const Unit<DT> (&un)[NU], float kl, float c) {
  constexpr int E = Unit<DT>::kEpu;
  float u[NU];
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    float e[E];
#pragma unroll
    for (int k = 0; k < E; ++k) e[k] = hw_exp2(fmaf(un[j].x[k], kl, -c));
    if constexpr (E == 8)
      u[j] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    else
      u[j] = (e[0] + e[1]) + (e[2] + e[3]);
  }
  if constexpr (NU == 8)
    return ((u[0] + u[1]) + (u[2] + u[3])) + ((u[4] + u[5]) + (u[6] + u[7]));
  else if constexpr (NU == 4)
    return (u[0] + u[1]) + (u[2] + u[3]);
  else if constexpr (NU == 2)
    return u[0] + u[1];
  else
    return u[0];
}

// Add a batch sum a taken against shift cb (-inf: an empty batch, a = 0) to
// the lane's sum, moving the lane's shift up to cb if that is larger. Both
// shifts are integers, so the rescaling is exact; a NaN batch (NaN or +inf in
// the row) makes the lane's sum NaN.
__device__ __forceinline__ void fold_batch(SumExp& st, float cb, float a) {
  const float hi = fmaxf(st.c, cb);
  const int e1 = (int)fmaxf(st.c - hi, -1100.0f);  // <= 0; -inf or NaN (no shift yet) -> underflow to 0
  const int e2 = (int)fmaxf(cb - hi, -1100.0f);
  st.s = ldexp(st.s, e1) + ldexp((double)a, e2);
  st.c = hi;
}

template <int DT, int NU>
__device__ __forceinline__ void sumexp_fma(SumExp& st, const Unit<DT> (&un)[NU], float kl) {
  float gm = unit_max(un[0]);
#pragma unroll
  for (int j = 1; j < NU; ++j) gm = fmaxf(gm, unit_max(un[j]));
  // the ceiling of the rounded product is at most half an ulp (<= 1/2 while
  // |c| < 2^24) below gm * kl: every term of the batch is below 2^(1/2)
  const float cb = ceilf(gm * kl);
  if (!(fabsf(cb) < 0x1p24f) && __builtin_isfinite(gm)) st.ovf = 1;
  const float a = (cb == -INFINITY) ? 0.0f : terms_fma<DT, NU>(un, kl, cb);
  fold_batch(st, cb, a);
}

// Subtract form: reference m_ref starts at -FLT_MAX and moves to the batch
// maximum when that exceeds it by more than 64 / kl.
struct SumExpSub {
  float m_ref;
  double s;
};

template <int DT, int NU>
__device__ __forceinline__ void sumexp_sub(SumExpSub& st, const Unit<DT> (&un)[NU], float kl) {
  constexpr int E = Unit<DT>::kEpu;
  float gm = unit_max(un[0]);
#pragma unroll
  for (int j = 1; j < NU; ++j) gm = fmaxf(gm, unit_max(un[j]));
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

// The read-only pass (a measurement of the rate at which the statistics pass
// can read its own bytes): every 32-bit word of every unit is folded into one
// xor, so each 16-byte load is kept whole, and nothing else is computed.
struct ReadXor {
  uint32_t s;
};

template <int DT, int NU, class St>
__device__ __forceinline__ void sumexp(St& st, const Unit<DT> (&un)[NU], float kl) {
  if constexpr (std::is_same<St, SumExp>::value) {
    sumexp_fma<DT, NU>(st, un, kl);
  } else if constexpr (std::is_same<St, ReadXor>::value) {
#pragma unroll
    for (int j = 0; j < NU; ++j)
#pragma unroll
      for (int k = 0; k < Unit<DT>::kEpu; ++k) st.s ^= __float_as_uint(un[j].x[k]);
  } else {
    sumexp_sub<DT, NU>(st, un, kl);
  }
}

// The workgroup streams units [c_begin, c_end) of a row with V elements; thread
// t takes units c_begin + t + 256 k, so every load instruction of the
// workgroup covers one contiguous 4 KB block.
template <int DT, class St>
__device__ __forceinline__ void stream_sumexp(const char* __restrict__ row, int V, int64_t c_begin, int64_t c_end,
                                              float kl, St& st) {
  constexpr int E = Unit<DT>::kEpu;
  const int tid = threadIdx.x;
  const int64_t nu_row = ((int64_t)V + E - 1) / E;
  const bool ragged = (V % E) != 0;
  int64_t full_end = c_end;
  if (ragged && full_end > nu_row - 1) full_end = nu_row - 1;
  int64_t base = c_begin;
  // Whole batches, two buffers deep: the loads of the next batch are in
  // flight while the current one is summed (no buffer is copied: a copy
  // would wait for its loads).
  constexpr int64_t BU = (int64_t)kThreads * kU1;
  const int64_t nb = full_end > base ? (full_end - base) / BU : 0;
  if (nb > 0) {
    auto load_batch = [&](uint4 (&w)[kU1], int64_t at) {
#pragma unroll
      for (int j = 0; j < kU1; ++j) w[j] = load16(row + (at + tid + kThreads * j) * 16);
    };
    auto sum_batch = [&](const uint4 (&w)[kU1]) {
      Unit<DT> un[kU1];
#pragma unroll
      for (int j = 0; j < kU1; ++j) un[j].unpack(w[j]);
      sumexp<DT, kU1>(st, un, kl);
      // the batch is summed before the next loads are issued (else the
      // compiler holds two batches of values in registers at once)
      __asm__ volatile("" : "+v"(st.s)::"memory");
    };
    uint4 a[kU1], b[kU1];
    load_batch(a, base);
    int64_t i = 0;
    for (; i + 2 < nb; i += 2) {
      load_batch(b, base + (i + 1) * BU);
      sum_batch(a);
      load_batch(a, base + (i + 2) * BU);
      sum_batch(b);
    }
    if (i + 1 < nb) {
      load_batch(b, base + (i + 1) * BU);
      sum_batch(a);
      sum_batch(b);
    } else {
      sum_batch(a);
    }
    base += nb * BU;
  }
  // The tail (fewer than kU1 units per thread left): every load is issued
  // before the first term is taken, so the chunk ends one memory round trip
  // later instead of one per unit. A lane past c_end loads the chunk's last
  // unit (in bounds) and skips it.
  if (base < c_end) {
    uint4 w[kU1];
#pragma unroll
    for (int j = 0; j < kU1; ++j) {
      const int64_t u = base + tid + kThreads * j;
      w[j] = load16(row + (u < c_end ? u : c_end - 1) * 16);
    }
#pragma unroll
    for (int j = 0; j < kU1; ++j) {
      const int64_t u = base + tid + kThreads * j;
      if (u < c_end) {
        Unit<DT> un[1];
        un[0].unpack(w[j]);
        if (ragged && u == nu_row - 1) mask_tail(un[0], u, V);
        sumexp<DT, 1>(st, un, kl);
      }
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
// stats kernels
// ---------------------------------------------------------------------------
// Partials of chunk slot r of sequence b: slots [0, (gamma+1) * nct) are the
// target rows' chunks (row r / nct, chunk r % nct), the rest the draft rows'.
// One partial per wave: (reference, sum relative to it, max).
template <int DT, class St>
__device__ __forceinline__ void stream_slot(const SampleLaunch& A, int b, int r, float kl, St& st) {
  const int tchunks = (A.gamma + 1) * A.nct;
  if (r < tchunks) {
    const int row = r / A.nct, c = r % A.nct;
    const char* p = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)row * A.t_row_b;
    const int64_t nu = ((int64_t)A.V * Unit<DT>::kEsz + 15) / 16;
    const int64_t u0 = (int64_t)c * A.cut;
    const int64_t u1 = u0 + A.cut < nu ? u0 + A.cut : nu;
    stream_sumexp<DT>(p, A.V, u0, u1, kl, st);
  } else {
    const int rr = r - tchunks;
    const int row = rr / A.ncd, c = rr % A.ncd;
    const char* p = A.dft + (int64_t)b * A.d_seq_b + (int64_t)row * A.d_row_b;
    const int64_t nu = ((int64_t)A.V * Unit<DT>::kEsz + 15) / 16;
    const int64_t u0 = (int64_t)c * A.cud;
    const int64_t u1 = u0 + A.cud < nu ? u0 + A.cud : nu;
    stream_sumexp<DT>(p, A.V, u0, u1, kl, st);
  }
}

// Partials of chunk slot r of sequence b: slots [0, (gamma+1) * nct) are the
// target rows' chunks (row r / nct, chunk r % nct), the rest the draft rows'.
// One partial per wave. The chunk is streamed in the FMA form; if any lane's
// reference needs the subtract form (|m * kl| >= 2^24: tiny temperatures or
// huge logits), the workgroup streams the chunk again in that form.
template <int TD, int DD>
__device__ __forceinline__ void stats_chunk(const SampleLaunch& A, int b, int r, float kl) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const bool tgt = r < (A.gamma + 1) * A.nct;
  RowPartial rp;
  SumExp st{-INFINITY, 0.0, 0};
  if (tgt)
    stream_slot<TD>(A, b, r, kl, st);
  else
    stream_slot<DD>(A, b, r, kl, st);
  if (!__syncthreads_or(st.ovf)) {
    // the wave's lanes at its largest shift, rescaled by exact powers of two
    const float Mc = wave_max(st.c);
    if (Mc == -INFINITY)
      rp.s = wave_sum(st.s);  // every value -inf (s = 0) or NaN seen
    else
      rp.s = wave_sum(ldexp(st.s, (int)fmaxf(st.c - Mc, -1100.0f)));
    rp.m = Mc;
    rp.form = 1;
  } else {
    SumExpSub ss{-FLT_MAX, 0.0};
    if (tgt)
      stream_slot<TD>(A, b, r, kl, ss);
    else
      stream_slot<DD>(A, b, r, kl, ss);
    const float M = wave_max(ss.m_ref);
    rp.s = wave_sum(ss.s * (double)hw_exp2((ss.m_ref - M) * kl));
    rp.m = M;
    rp.form = 0;
  }
  if (lane == 0) A.part[((int64_t)b * A.per_seq + r) * kWaves + w] = rp;
}

// Statistics of a whole row from its nrec wave partials, computed by one wave
// (every lane gets the result). Used by the finish kernel and by the gate of
// the early-exit stats kernel, which must reach the same accept decisions bit
// for bit; contraction is off so that inlining cannot change the rounding.
// p_v = exp2(x_v * kl - c) / s.
struct RowStat {
  double c;  // shift in log2 units: the largest partial shift
  float m;   // a logit with m * kl near c (the reference of the subtract form)
  double s;  // sum_v exp2(x_v * kl - c)
  int valid;
};
// Shift of a partial in log2 units, exactly as its terms were taken.
__device__ __forceinline__ double partial_shift(const RowPartial& p, float kl) {
  return p.form ? (double)p.m : (double)p.m * (double)kl;
}

// 2^d for d <= 0 in fp64: exact (a power of two) when d is an integer, as it
// is between two FMA-form partials.
__device__ __forceinline__ double pow2_le0(double d) {
  return (d == rint(d)) ? ldexp(1.0, (int)fmax(d, -1100.0)) : exp2(d);
}

__device__ __forceinline__ RowStat row_stat(double Ms, float Mm, double S, float kl, bool tv) {
#pragma clang fp contract(off)
  RowStat r;
  r.c = Ms;
  r.m = (Mm != -INFINITY) ? Mm : (float)(Ms / (double)kl);
  r.s = S;
  r.valid = tv && __builtin_isfinite(S) && S > 0.0 && __builtin_isfinite(Ms);
  return r;
}

// The merge of a row with at most one partial per lane (have: this lane holds
// partial q), taken with the same operations as the general merge below.
__device__ __forceinline__ RowStat merge_row_one(const RowPartial& q, bool have, float kl, bool tv) {
#pragma clang fp contract(off)
  double sh = -INFINITY;
  if (have) sh = partial_shift(q, kl);
  const double Ms = wave_max_f64(sh);
  float Mm = -INFINITY;  // the reference logit of a subtract-form partial at Ms
  if (have && sh == Ms && q.form == 0) Mm = q.m;
  Mm = wave_max(Mm);
  double S = 0.0;
  if (have) S += q.s * pow2_le0(sh - Ms);
  S = wave_sum(S);
  return row_stat(Ms, Mm, S, kl, tv);
}

__device__ __forceinline__ RowStat merge_row(const RowPartial* P, int nrec, float kl, bool tv, int lane) {
#pragma clang fp contract(off)
  if (nrec <= kWave) {
    // at most one partial per lane, loaded once
    const bool have = lane < nrec;
    RowPartial q{};
    if (have) q = P[lane];
    return merge_row_one(q, have, kl, tv);
  }
  double Ms = -INFINITY;
  for (int k = lane; k < nrec; k += kWave) Ms = fmax(Ms, partial_shift(P[k], kl));
  Ms = wave_max_f64(Ms);
  float Mm = -INFINITY;
  for (int k = lane; k < nrec; k += kWave)
    if (P[k].form == 0 && partial_shift(P[k], kl) == Ms) Mm = fmaxf(Mm, P[k].m);
  Mm = wave_max(Mm);
  double S = 0.0;
  for (int k = lane; k < nrec; k += kWave) S += P[k].s * pow2_le0(partial_shift(P[k], kl) - Ms);
  S = wave_sum(S);
  return row_stat(Ms, Mm, S, kl, tv);
}

// Accept test of one position: rho = p(x) / q(x) in the log2 domain in fp64;
// code 1 accepted, 0 rejected, 2 invalid; p(x), q(x) for the diagnostics (NaN
// when invalid).
struct AcceptOut {
  int code;
  float px, qx;
};
// want_p: also p(x) and q(x) (else NaN; the decision is the same either way).
__device__ __forceinline__ AcceptOut accept_test(float lt, float ld, const RowStat& t, const RowStat& d, float kl,
                                                 float u, bool tok_ok, bool tv, bool want_p) {
#pragma clang fp contract(off)
  AcceptOut o;
  o.px = __builtin_nanf("");
  o.qx = __builtin_nanf("");
  const bool ok = tv && t.valid && d.valid && tok_ok && u >= 0.0f && u < 1.0f && ld != -INFINITY;
  if (ok) {
    const double lp2 = (double)lt * (double)kl - t.c;  // the product of two floats is exact
    const double lq2 = (double)ld * (double)kl - d.c;
    const double rho = exp2(lp2 - lq2) * (d.s / t.s);
    if (want_p) {
      o.px = (float)(exp2(lp2) / t.s);
      o.qx = (float)(exp2(lq2) / d.s);
    }
    o.code = ((double)u < rho) ? 1 : 0;
  } else {
    o.code = 2;
  }
  return o;
}

// The finish parts' hand-off state of sequence b before a finish launch: no
// part done, no step mass yet (one workgroup of the sequence calls this).
// (The step sums of sequence b are [4][ns2] in the workspace: masses,
// q-masses and form flags hold -1 until published, signed sums NaN.)
__device__ __forceinline__ void reset_handoff(const SampleLaunch& A, int b) {
  if (threadIdx.x == 0) A.done[b] = 0;
  if (A.parts > 1) {
    double* g = A.steptot + (int64_t)b * 4 * A.ns2;
    for (int s = threadIdx.x; s < A.ns2; s += blockDim.x) {
      g[s] = -1.0;
      g[A.ns2 + s] = -1.0;
      g[2 * A.ns2 + s] = __builtin_nan("");
      g[3 * A.ns2 + s] = -1.0;
    }
  }
}

// One pass: one workgroup per (sequence, chunk slot) over every row.
template <int TD, int DD>
// At most 80 VGPRs: six waves per SIMD keep enough loads in flight (at four,
// a pass over 512 x 11 rows of 256k logits took 727 us instead of 617).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void sv_stats_kernel(SampleLaunch A) {
  const int64_t wg = blockIdx.x;
  const int b = (int)(wg / A.per_seq);
  const int r = (int)(wg % A.per_seq);
  const float T = A.temps[b];
  const float kl = temp_ok(T) ? log2e_over(T) : 1.0f;
  if (r == 0) reset_handoff(A, b);
  stats_chunk<TD, DD>(A, b, r, kl);
}

// The statistics pass's reads alone: the same grid, chunks and loads as
// sv_stats_kernel, with the arithmetic replaced by an xor of the loaded words.
// Writes nothing unless the xor of a workgroup's first thread equals one
// arbitrary constant (then that value to the sequence's finish counter in the
// workspace, which the statistics pass resets before any finish reads it);
// the comparison keeps every thread's loads alive.
template <int TD, int DD>
__global__ __launch_bounds__(kThreads) void sv_read_kernel(SampleLaunch A) {
  const int64_t wg = blockIdx.x;
  const int b = (int)(wg / A.per_seq);
  const int r = (int)(wg % A.per_seq);
  ReadXor st{0u};
  if (r < (A.gamma + 1) * A.nct)
    stream_slot<TD>(A, b, r, 1.0f, st);
  else
    stream_slot<DD>(A, b, r, 1.0f, st);
  if (threadIdx.x == 0 && st.s == 0x9e3779b9u) A.done[b] = (int32_t)st.s;
}

// Early exit: the statistics of positions p0..p1 (target rows, and draft rows
// of positions below gamma), one workgroup per (sequence, chunk of those rows).
// reach[b] = k records that positions 0..k-2 were accepted and rows 0..k-1
// have statistics. For p0 > 0 a workgroup first re-derives the accept decision
// of position p0 - 1 from that position's partials (every workgroup of the
// sequence derives the same one) and streams its chunk only after an
// acceptance, so after a rejection the sequence's later rows are never read.
template <int TD, int DD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void sv_stats_pos_kernel(
    SampleLaunch A, int p0, int p1) {
  __shared__ RowStat sh_rs[2];
  __shared__ float sh_g[2];
  __shared__ int sh_go;
  const int G = A.gamma;
  const int pair = A.nct + A.ncd;
  const int npair = max(0, min(p1, G - 1) - p0 + 1);  // positions below gamma in [p0, p1]
  const int cps = npair * pair + (p1 == G ? A.nct : 0);
  const int64_t wg = blockIdx.x;
  const int b = (int)(wg / cps);
  const int c = (int)(wg % cps);
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float T = A.temps[b];
  const bool tv = temp_ok(T);
  const float kl = tv ? log2e_over(T) : 1.0f;
  if (p0 == 0) {
    if (tid == 0) A.reach[b] = p1 + 1;  // every workgroup of the sequence writes the same value
    if (c == 0) reset_handoff(A, b);
  } else {
    if (A.reach[b] < p0) return;  // the sequence stopped at an earlier position
    const int i = p0 - 1;
    if (w < 2) {
      // wave 0 merges target row i, wave 1 draft row i
      const int nrec = (w == 0 ? A.nct : A.ncd) * kWaves;
      const int base = (w == 0) ? i * A.nct : (G + 1) * A.nct + i * A.ncd;
      const RowStat rs = merge_row(A.part + ((int64_t)b * A.per_seq + base) * kWaves, nrec, kl, tv, lane);
      if (lane == 0) sh_rs[w] = rs;
    } else if (w == 2 && lane == 0) {
      // the two logits of draft token x_i
      const int xi = A.tokens[(int64_t)b * G + i];
      float lt = 0.0f, ld = 0.0f;
      if (xi >= 0 && xi < A.V) {
        lt = load_elem<TD>(A.tgt + (int64_t)b * A.t_seq_b + (int64_t)i * A.t_row_b, xi);
        ld = load_elem<DD>(A.dft + (int64_t)b * A.d_seq_b + (int64_t)i * A.d_row_b, xi);
      }
      sh_g[0] = lt;
      sh_g[1] = ld;
    }
    __syncthreads();
    if (tid == 0) {
      const int xi = A.tokens[(int64_t)b * G + i];
      const float ui = A.uniforms[(int64_t)b * (G + 1) + i];
      const AcceptOut ao = accept_test(sh_g[0], sh_g[1], sh_rs[0], sh_rs[1], kl, ui, xi >= 0 && xi < A.V, tv, false);
      sh_go = ao.code == 1;
      if (ao.code == 1) A.reach[b] = p1 + 1;
    }
    __syncthreads();
    if (!sh_go) return;
  }
  int r;
  if (c < npair * pair) {
    const int pos = p0 + c / pair, cc = c % pair;
    r = (cc < A.nct) ? pos * A.nct + cc : (G + 1) * A.nct + pos * A.ncd + (cc - A.nct);
  } else {
    r = G * A.nct + (c - npair * pair);  // the bonus row
  }
  stats_chunk<TD, DD>(A, b, r, kl);
}

// ---------------------------------------------------------------------------
// draw kernel
// ---------------------------------------------------------------------------
// Octet `oct` of a row holds token ids 8*oct .. 8*oct+7.
//
// Raw words of one octet of a row, loaded with no branch so that the loads of
// several octets are all in flight before the first is used: an octet at or
// past the row's end (oct >= noct) loads the row's last octet instead, and an
// fp32 octet whose second half lies at or past V loads its first half twice.
// to_float() gives the octet's 8 values, -inf at and past V; the values of an
// octet past the end are never used.
template <int DT>
struct OctetIn;
template <>
struct OctetIn<1> {
  uint4 w;
  __device__ __forceinline__ void load(const char* row, int64_t oct, int64_t noct, int V) {
    w = load16(row + (oct < noct ? oct : noct - 1) * 16);
  }
  __device__ __forceinline__ void to_float(int64_t oct, int V, float (&x)[8]) const {
    Unit<1> un;
    un.unpack(w);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = un.x[k];
    if (oct * 8 + 8 > V) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (oct * 8 + k >= V) x[k] = -INFINITY;
    }
  }
};
template <>
struct OctetIn<0> {
  uint4 w0, w1;
  __device__ __forceinline__ void load(const char* row, int64_t oct, int64_t noct, int V) {
    const int64_t o = oct < noct ? oct : noct - 1;
    w0 = load16(row + o * 32);
    w1 = load16(row + o * 32 + (o * 8 + 4 < V ? 16 : 0));
  }
  __device__ __forceinline__ void to_float(int64_t oct, int V, float (&x)[8]) const {
    x[0] = __uint_as_float(w0.x);
    x[1] = __uint_as_float(w0.y);
    x[2] = __uint_as_float(w0.z);
    x[3] = __uint_as_float(w0.w);
    const bool hi = oct * 8 + 4 < V;
    x[4] = hi ? __uint_as_float(w1.x) : -INFINITY;
    x[5] = hi ? __uint_as_float(w1.y) : -INFINITY;
    x[6] = hi ? __uint_as_float(w1.z) : -INFINITY;
    x[7] = hi ? __uint_as_float(w1.w) : -INFINITY;
    if (oct * 8 + 8 > V) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (oct * 8 + k >= V) x[k] = -INFINITY;
    }
  }
};

__device__ __forceinline__ float sum8(const float (&r)[8]) {
  return ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
}

// Raw 16-byte loads of one octet (8 tokens) of a row: bf16 needs one unit,
// fp32 two. Only used where the whole octet lies inside the row.
template <int DT>
struct OctetRaw;
template <>
struct OctetRaw<1> {
  uint4 w;
  __device__ __forceinline__ void load(const char* row, int64_t oct) { w = load16(row + oct * 16); }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
    Unit<1> un;
    un.unpack(w);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = un.x[k];
  }
};
template <>
struct OctetRaw<0> {
  uint4 w0, w1;
  __device__ __forceinline__ void load(const char* row, int64_t oct) {
    w0 = load16(row + oct * 32);
    w1 = load16(row + oct * 32 + 16);
  }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
    x[0] = __uint_as_float(w0.x);
    x[1] = __uint_as_float(w0.y);
    x[2] = __uint_as_float(w0.z);
    x[3] = __uint_as_float(w0.w);
    x[4] = __uint_as_float(w1.x);
    x[5] = __uint_as_float(w1.y);
    x[6] = __uint_as_float(w1.z);
    x[7] = __uint_as_float(w1.w);
  }
};

// 2^x - 1 for x <= 0 (x may be -inf), to a few ulp relative: on [-1/2, 0] as
// x * P(x), P of degree 4 fitted for the smallest maximum relative error
// (Lawson's iteratively reweighted least squares; coefficients from
// fit_expm1_2.py, 2.3 ulp at most in this fp32 Horner form); below -1/2 as
// exp2(x) - 1, which is at least 0.29 in magnitude there, so the subtraction
// keeps it within a few ulp of a faithful exp2.
__device__ __forceinline__ float expm1_2(float x) {
  constexpr float c0 = 6.931471825e-01f, c1 = 2.402256429e-01f, c2 = 5.549040809e-02f, c3 = 9.541280568e-03f,
                  c4 = 1.154452213e-03f;
  float p = fmaf(c4, x, c3);
  p = fmaf(p, x, c2);
  p = fmaf(p, x, c1);
  p = fmaf(p, x, c0);
  const float poly = p * x;
  const float e = hw_exp2(x) - 1.0f;
  return (x >= -0.5f) ? poly : e;
}

// One token of the residual in the FMA form (see SeqPlan): e = max(e_p, e_q)
// and mag = |e_p - e_q| = -e * expm1_2(-|w|), with w = log2(q_v / p_v) formed
// from the logit difference, so mag keeps its relative accuracy however close
// p_v and q_v are; pos: p_v >= q_v (the residual is mag there, else 0).
// Where the target logit is -inf and the draft's is not, e (= e_q) comes out
// NaN; the caller redoes such octets with resid_fix (a NaN octet sum).
struct ResidTerm {
  float e, mag;
  bool pos;
};
__device__ __forceinline__ ResidTerm resid_term(float xt, float xd, const SeqPlan& P) {
  ResidTerm t;
  const float w = fmaf(xd - xt, P.kl, P.dt);
  t.e = hw_exp2(fmaf(xt, P.kl, -P.cp) + fmaxf(w, 0.0f));
  t.mag = -t.e * expm1_2(fminf(-fabsf(w), 0.0f));  // a NaN w (both logits -inf) gives 0
  t.pos = w <= 0.0f;
  return t;
}
// The same token when its target logit is -inf (p_v = 0): e = e_q from the
// draft logit alone.
__device__ __forceinline__ ResidTerm resid_fix(float xt, float xd, const SeqPlan& P) {
  ResidTerm t = resid_term(xt, xd, P);
  if (!(t.e == t.e)) {
    t.e = hw_exp2(fmaf(xd, P.kl, -P.cq) - P.cq_lo);
    t.mag = t.e;
  }
  return t;
}

// Sums over the 8 tokens of an octet in the residual's FMA form: r = the
// residual (mag where p >= q), pe = e_p where p >= q, a = mag everywhere
// (the step's q-mass of the positive residual is pe - r, its signed sum of
// e_p - e_q is 2 r - a). Pairwise fp32 sums, as sum8. FIX: take resid_fix
// (needed only where a target logit of -inf meets a finite draft logit, which
// leaves a NaN in a).
struct ResidSums {
  float r, pe, a;
};
template <bool FIX>
__device__ __forceinline__ ResidSums resid_sums8(const float (&xt)[8], const float (&xd)[8], const SeqPlan& P) {
  float r[8], pe[8], a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const ResidTerm t = FIX ? resid_fix(xt[k], xd[k], P) : resid_term(xt[k], xd[k], P);
    r[k] = t.pos ? t.mag : 0.0f;
    pe[k] = t.pos ? t.e : 0.0f;
    a[k] = t.mag;
  }
  return ResidSums{((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7])),
                   ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7])),
                   ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]))};
}

// resid_sums8 in the streaming loop: the fix is redone only if a NaN shows up
// in the wave (a wave-uniform branch, so its exponentials are not computed
// speculatively for every token).
__device__ __forceinline__ ResidSums resid_sums8_checked(const float (&xt)[8], const float (&xd)[8], const SeqPlan& P) {
  ResidSums o = resid_sums8<false>(xt, xd, P);
  const bool bad = !(o.a == o.a);
  if (__builtin_expect(__ballot(bad) != 0, 0) && bad) o = resid_sums8<true>(xt, xd, P);
  return o;
}

// The residual's cheap form (FMA shifts): e_p and e_q from one exponential
// each (e_q straight from the draft logit, so logits of -inf give 0 and no
// NaN). The draft's shift is the fp32 head cq of cqx; the rest of it is the
// factor cq_s = 2^-(cqx - cq), applied in the difference's FMA: e1 =
// exp2(fma(x_d, kl, -cq)), e_q = cq_s e1, t = e_p - e_q = fma(-cq_s, e1, e_p).
// A token lies on the residual's side where t > 0, and its residual is t there.
// Each exponential carries its own rounding, so t is off by a few units of
// fp32 rounding of e_p wherever p and q are close; a step whose positive
// residual is small next to its q-mass takes the exact form instead
// (cheap_ok).
struct CheapTerm {
  float e1, t;
};
__device__ __forceinline__ CheapTerm cheap_term(float xt, float xd, const SeqPlan& P) {
  CheapTerm c;
  const float ep = hw_exp2(fmaf(xt, P.kl, -P.cp));
  c.e1 = hw_exp2(fmaf(xd, P.kl, -P.cq));
  c.t = fmaf(-P.cq_s, c.e1, ep);
  return c;
}

// Sums over the 8 tokens of an octet in the cheap form: r = the residual, q =
// e_q where t > 0 (the q-mass of the positive residual), d = e_p - e_q over
// all 8 (the signed sum). Pairwise fp32 sums, as sum8.
struct CheapSums {
  float r, q, d;
};
__device__ __forceinline__ CheapSums cheap_sums8(const float (&xt)[8], const float (&xd)[8], const SeqPlan& P) {
  float r[8], q[8], d[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const CheapTerm c = cheap_term(xt[k], xd[k], P);
    r[k] = fmaxf(c.t, 0.0f);
    q[k] = c.t > 0.0f ? c.e1 : 0.0f;
    d[k] = c.t;
  }
  return CheapSums{sum8(r), sum8(q) * P.cq_s, sum8(d)};
}

// Whether a step's cheap sums stand: its positive residual m is at least
// 1 / kCheapRatio of its q-mass q (then the rounding of the two exponentials,
// independent and unbiased per token, is well under 1e-6 of m). Steps where
// p and q are closer, or whose sums are not finite, take the exact form.
constexpr double kCheapRatio = 7.0;
__device__ __forceinline__ bool cheap_ok(double m, double q) { return q <= kCheapRatio * m; }

// A lane's cheap sums over a step, added octet by octet in fp32 and reduced
// over the wave in fp32 (wave_sum_f32): a step's 2048 terms pass about a
// dozen fp32 roundings, well under 1e-6 of the step's mass, and the cheap
// form only stands where the residual is not small next to the terms.
struct CheapAcc {
  float r = 0.0f, q = 0.0f, d = 0.0f;
  __device__ __forceinline__ void add(const CheapSums& o) {
    r += o.r;
    q += o.q;
    d += o.d;
  }
};

// Unnormalised masses of 8 tokens (see SeqPlan for the forms). Residual mode,
// FMA form: r_v = mag - g (e_p - mag) where p_v >= q_v, clamped at 0, else 0:
// F Sp * max(0, p_v - q_v) with the normalisers' ratio corrected to first
// order (g = 0 before the correction is known); subtract form: max(0, e^p_v -
// kappa e^q_v). Bonus mode: r_v = e^p_v = F Sp * p_v. Tokens at or beyond V
// (value -inf) get 0.
template <int MODE, int FORM>
__device__ __forceinline__ void mass8(const float (&xt)[8], const float (&xd)[8], const SeqPlan& P, float (&r)[8]) {
  if constexpr (MODE == kModeResidual && FORM == 1) {
    const float gf = (float)P.g;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const ResidTerm t = resid_term(xt[k], xd[k], P);
      r[k] = t.pos ? fmaxf(fmaf(-gf, t.e - t.mag, t.mag), 0.0f) : 0.0f;
      bad |= !(t.mag == t.mag);
    }
    // a target logit of -inf next to a finite draft logit (a NaN term):
    // redo the octet with resid_fix, in a wave-uniform branch
    if (__builtin_expect(__ballot(bad) != 0, 0) && bad) {
#pragma nounroll
      for (int k = 0; k < 8; ++k) {
        const ResidTerm t = resid_fix(xt[k], xd[k], P);
        r[k] = t.pos ? fmaxf(fmaf(-gf, t.e - t.mag, t.mag), 0.0f) : 0.0f;
      }
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if constexpr (FORM == 1) {
      r[k] = hw_exp2(fmaf(xt[k], P.kl, -P.cp));
    } else {
      const float ep = hw_exp2((xt[k] - P.mp) * P.kl);
      if constexpr (MODE != kModeBonus) {
        const float eq = hw_exp2((xd[k] - P.mq) * P.kl);
        float d = fmaf(-eq, P.kap_hi, ep);
        d = fmaf(-eq, P.kap_lo, d);
        r[k] = fmaxf(d, 0.0f);
      } else {
        r[k] = ep;
      }
    }
  }
}

// The 8 values of octet oct < noct of a row, -inf at and past V, with each
// load made only where the row has the bytes (the same values as OctetIn).
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

// Masses of 8 tokens in the residual's cheap form, corrected to first order
// as in mass8: r_v = max(0, t - g e_q) where t = e_p - e_q > 0, else 0.
__device__ __forceinline__ void mass8_cheap(const float (&xt)[8], const float (&xd)[8], const SeqPlan& P,
                                            float (&r)[8]) {
  const float gs = (float)(P.g * (double)P.cq_s);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const CheapTerm c = cheap_term(xt[k], xd[k], P);
    r[k] = c.t > 0.0f ? fmaxf(fmaf(-gs, c.e1, c.t), 0.0f) : 0.0f;
  }
}

// Masses of 8 tokens in the draw's mode and the plan's form (cheap: the
// residual's cheap form, for a step whose sums took it).
__device__ __forceinline__ void mass8_of(const float (&xt)[8], const float (&xd)[8], int mode, const SeqPlan& P,
                                         float (&r)[8], bool cheap = false) {
  if (mode == kModeResidual) {
    if (P.form == 1 && cheap)
      mass8_cheap(xt, xd, P, r);
    else if (P.form == 1)
      mass8<kModeResidual, 1>(xt, xd, P, r);
    else
      mass8<kModeResidual, 0>(xt, xd, P, r);
  } else {
    if (P.form == 1)
      mass8<kModeBonus, 1>(xt, xd, P, r);
    else
      mass8<kModeBonus, 0>(xt, xd, P, r);
  }
}

// Token masses of step s of the draw row(s) for one wave: rr[j] is octet
// s * kStepOctets + kWave * j + lane, all zero past the row's end. Every load
// of the step is issued before the first mass is taken (one memory round
// trip). cheap: the step's sums took the residual's cheap form (its masses
// are then taken in that form, the ones its mass was summed from).
template <int TD, int DD, bool kCheap>
__device__ __forceinline__ void step_octet_masses_in(const char* trow, const char* drow, int64_t s, int64_t noct,
                                                     int V, int mode, const SeqPlan& P, int lane,
                                                     float (&rr)[kU2][8]) {
  OctetIn<TD> t[kU2];
  OctetIn<DD> d[kU2];
  if (mode != kModeBonus) {
#pragma unroll
    for (int j = 0; j < kU2; ++j) {
      const int64_t oct = s * kStepOctets + kWave * j + lane;
      t[j].load(trow, oct, noct, V);
      d[j].load(drow, oct, noct, V);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kU2; ++j) t[j].load(trow, s * kStepOctets + kWave * j + lane, noct, V);
  }
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      float xt[8], xd[8];
      t[j].to_float(oct, V, xt);
      if (mode != kModeBonus) d[j].to_float(oct, V, xd);
      if constexpr (kCheap)
        mass8_cheap(xt, xd, P, rr[j]);
      else
        mass8_of(xt, xd, mode, P, rr[j]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) rr[j][k] = 0.0f;
    }
  }
}

template <int TD, int DD>
__device__ __forceinline__ void step_octet_masses(const char* trow, const char* drow, int64_t s, int64_t noct, int V,
                                                  int mode, const SeqPlan& P, int lane, bool cheap,
                                                  float (&rr)[kU2][8]) {
  if (mode == kModeResidual && P.form == 1 && cheap)
    step_octet_masses_in<TD, DD, true>(trow, drow, s, noct, V, mode, P, lane, rr);
  else
    step_octet_masses_in<TD, DD, false>(trow, drow, s, noct, V, mode, P, lane, rr);
}

// Per-step sums of the drawn distribution: m its mass; for the residual's
// FMA form also q, the q-mass of its positive part (sum of e_q where
// p_v >= q_v), and d, the signed sum of e_p - e_q over the step (the
// first-order correction of the normalisers' ratio takes both; 0 otherwise);
// c = 1 where the step's sums took the residual's cheap form, else 0.
struct StepSums {
  double m, q, d, c;
};
// Where the steps' sums go: LDS when the steps fit, else the workspace.
struct StepOut {
  double *m, *q, *d, *c;
};

// The wave's sums of a step from its lanes' shares (r: residual, pe: e_p where
// p >= q, a: |e_p - e_q|), every lane gets them.
__device__ __forceinline__ StepSums wave_step_sums(double r, double pe, double a) {
  StepSums o;
  o.m = wave_sum(r);
  o.q = wave_sum(pe) - o.m;
  o.d = 2.0 * o.m - wave_sum(a);
  o.c = 0.0;
  return o;
}

// The wave's cheap sums of a step (c = 1), every lane gets them.
__device__ __forceinline__ StepSums cheap_step_sums(const CheapAcc& a) {
  return StepSums{(double)wave_sum_f32(a.r), (double)wave_sum_f32(a.q), (double)wave_sum_f32(a.d), 1.0};
}

// Raw loads of half a step (1024 tokens) of the draw row(s) for one wave:
// kU2 / 2 octets per lane per row. Only used where the step lies inside the row.
constexpr int kHalfU = kU2 / 2;
template <int TD, int DD, int MODE>
struct HalfStep {
  OctetRaw<TD> t[kHalfU];
  OctetRaw<DD> d[kHalfU];
  // half h (0 or 1) of step s: octets s * kStepOctets + kWave * (h * kHalfU + j) + lane
  __device__ __forceinline__ void load(const char* trow, const char* drow, int64_t s, int h, int lane) {
#pragma unroll
    for (int j = 0; j < kHalfU; ++j) {
      const int64_t oct = s * kStepOctets + kWave * (h * kHalfU + j) + lane;
      t[j].load(trow, oct);
      if constexpr (MODE == kModeResidual) d[j].load(drow, oct);
    }
  }
  // This lane's share of the half step's masses r, added in octet order
  // (bonus mode, or the residual's subtract form).
  template <int FORM>
  __device__ __forceinline__ void sums(const SeqPlan& P, double& r) const {
#pragma unroll
    for (int j = 0; j < kHalfU; ++j) {
      float xt[8], xd[8];
      t[j].unpack(xt);
      if constexpr (MODE == kModeResidual) d[j].unpack(xd);
      float rr[8];
      mass8<MODE, FORM>(xt, xd, P, rr);
      r += (double)sum8(rr);
    }
  }
  // This lane's share of the half step's cheap sums (r, q, d; the residual's
  // FMA form), added in octet order in fp32 (see CheapAcc).
  __device__ __forceinline__ void cheap_sums(const SeqPlan& P, CheapAcc& a) const {
#pragma unroll
    for (int j = 0; j < kHalfU; ++j) {
      float xt[8], xd[8];
      t[j].unpack(xt);
      d[j].unpack(xd);
      a.add(cheap_sums8(xt, xd, P));
    }
  }
};

// The exact-form sums of the octets of step s held in t, d (residual, FMA
// form; octets at or past noct skipped), the NaN fix per octet.
template <int TD, int DD>
__device__ __forceinline__ StepSums exact_step_sums(const OctetIn<TD> (&t)[kU2], const OctetIn<DD> (&d)[kU2], int64_t s,
                                                    int64_t noct, int V, const SeqPlan& P, int lane) {
  double r = 0.0, pe = 0.0, a = 0.0;
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      float xt[8], xd[8];
      t[j].to_float(oct, V, xt);
      d[j].to_float(oct, V, xd);
      ResidSums o = resid_sums8<false>(xt, xd, P);
      if (!(o.a == o.a)) o = resid_sums8<true>(xt, xd, P);
      r += (double)o.r;
      pe += (double)o.pe;
      a += (double)o.a;
    }
  }
  return wave_step_sums(r, pe, a);
}

// The same sums with each octet loaded on its own (the pipelined loop's
// fallback, where a step's loads have left the registers): the same
// operations in the same order, so the same bits, with fewer registers live.
template <int TD, int DD>
__device__ __forceinline__ StepSums exact_step_sums_reload(const char* trow, const char* drow, int64_t s,
                                                           int64_t noct, int V, const SeqPlan& P, int lane) {
  double r = 0.0, pe = 0.0, a = 0.0;
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      float xt[8], xd[8];
      load_octet<TD>(trow, oct, V, xt);
      load_octet<DD>(drow, oct, V, xd);
      ResidSums o = resid_sums8<false>(xt, xd, P);
      if (!(o.a == o.a)) o = resid_sums8<true>(xt, xd, P);
      r += (double)o.r;
      pe += (double)o.pe;
      a += (double)o.a;
    }
  }
  return wave_step_sums(r, pe, a);
}

// The sums of step s of the draw row(s), every load of the step issued before
// the first use, bounds-checked (every lane gets them). Inside the row these
// are the same operations in the same order as the pipelined loop below, so
// both give the same bits for a step. In the residual's FMA form: the cheap
// sums, or the exact ones where cheap_ok rejects them (from the same loads).
template <int TD, int DD, int MODE, int FORM>
__device__ __forceinline__ StepSums direct_step_sums(const char* trow, const char* drow, int64_t s, int64_t noct,
                                                     int V, const SeqPlan& P, int lane) {
  OctetIn<TD> t[kU2];
  OctetIn<DD> d[kU2];
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    t[j].load(trow, oct, noct, V);
    if constexpr (MODE == kModeResidual) d[j].load(drow, oct, noct, V);
  }
  double r = 0.0;
  CheapAcc a;
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      float xt[8], xd[8];
      t[j].to_float(oct, V, xt);
      if constexpr (MODE == kModeResidual) d[j].to_float(oct, V, xd);
      if constexpr (MODE == kModeResidual && FORM == 1) {
        a.add(cheap_sums8(xt, xd, P));
      } else {
        float rr[8];
        mass8<MODE, FORM>(xt, xd, P, rr);
        r += (double)sum8(rr);
      }
    }
  }
  if constexpr (MODE == kModeResidual && FORM == 1) {
    const StepSums v = cheap_step_sums(a);
    if (cheap_ok(v.m, v.q)) return v;
    return exact_step_sums<TD, DD>(t, d, s, noct, V, P, lane);
  }
  return StepSums{wave_sum(r), 0.0, 0.0, 0.0};
}

template <int TD, int DD>
__device__ __forceinline__ StepSums direct_step_sums_of(const char* trow, const char* drow, int64_t s, int64_t noct,
                                                        int V, int mode, const SeqPlan& P, int lane) {
  if (mode == kModeResidual) {
    if (P.form == 1) return direct_step_sums<TD, DD, kModeResidual, 1>(trow, drow, s, noct, V, P, lane);
    return direct_step_sums<TD, DD, kModeResidual, 0>(trow, drow, s, noct, V, P, lane);
  }
  if (P.form == 1) return direct_step_sums<TD, DD, kModeBonus, 1>(trow, drow, s, noct, V, P, lane);
  return direct_step_sums<TD, DD, kModeBonus, 0>(trow, drow, s, noct, V, P, lane);
}

// One step per wave, its loads kept: direct_step_sums (the same operations in
// the same order, so the same bits) with the step's octets left in t and d,
// which the draw then rescans from registers instead of loading them again
// (the rescan's memory round trip is most of the draw's time on short rows).
template <int TD, int DD, int MODE, int FORM>
__device__ __forceinline__ StepSums kept_step_sums(const char* trow, const char* drow, int64_t s, int64_t noct,
                                                   int V, const SeqPlan& P, int lane, OctetIn<TD> (&t)[kU2],
                                                   OctetIn<DD> (&d)[kU2]) {
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    t[j].load(trow, oct, noct, V);
    if constexpr (MODE == kModeResidual) d[j].load(drow, oct, noct, V);
  }
  double r = 0.0;
  CheapAcc a;
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      float xt[8], xd[8];
      t[j].to_float(oct, V, xt);
      if constexpr (MODE == kModeResidual) d[j].to_float(oct, V, xd);
      if constexpr (MODE == kModeResidual && FORM == 1) {
        a.add(cheap_sums8(xt, xd, P));
      } else {
        float rr[8];
        mass8<MODE, FORM>(xt, xd, P, rr);
        r += (double)sum8(rr);
      }
    }
  }
  if constexpr (MODE == kModeResidual && FORM == 1) {
    const StepSums v = cheap_step_sums(a);
    if (cheap_ok(v.m, v.q)) return v;
    return exact_step_sums<TD, DD>(t, d, s, noct, V, P, lane);
  }
  return StepSums{wave_sum(r), 0.0, 0.0, 0.0};
}

template <int TD, int DD>
__device__ __forceinline__ StepSums kept_step_sums_of(const char* trow, const char* drow, int64_t s, int64_t noct,
                                                      int V, int mode, const SeqPlan& P, int lane,
                                                      OctetIn<TD> (&t)[kU2], OctetIn<DD> (&d)[kU2]) {
  if (mode == kModeResidual) {
    if (P.form == 1) return kept_step_sums<TD, DD, kModeResidual, 1>(trow, drow, s, noct, V, P, lane, t, d);
    return kept_step_sums<TD, DD, kModeResidual, 0>(trow, drow, s, noct, V, P, lane, t, d);
  }
  if (P.form == 1) return kept_step_sums<TD, DD, kModeBonus, 1>(trow, drow, s, noct, V, P, lane, t, d);
  return kept_step_sums<TD, DD, kModeBonus, 0>(trow, drow, s, noct, V, P, lane, t, d);
}

// The bonus-mode sums of a kept step (the fallback after a residual of zero
// mass), from the target octets in t.
template <int TD, int DD>
__device__ __forceinline__ StepSums kept_bonus_sums(const OctetIn<TD> (&t)[kU2], int64_t s, int64_t noct, int V,
                                                    const SeqPlan& P, int lane) {
  double r = 0.0;
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      float xt[8], xd[8];
      t[j].to_float(oct, V, xt);
#pragma unroll
      for (int k = 0; k < 8; ++k) xd[k] = 0.0f;
      float rr[8];
      if (P.form == 1)
        mass8<kModeBonus, 1>(xt, xd, P, rr);
      else
        mass8<kModeBonus, 0>(xt, xd, P, rr);
      r += (double)sum8(rr);
    }
  }
  return StepSums{wave_sum(r), 0.0, 0.0, 0.0};
}

// The token masses of a kept step, as step_octet_masses takes them from memory.
template <int TD, int DD>
__device__ __forceinline__ void kept_octet_masses(const OctetIn<TD> (&t)[kU2], const OctetIn<DD> (&d)[kU2], int64_t s,
                                                  int64_t noct, int V, int mode, const SeqPlan& P, int lane,
                                                  bool cheap, float (&rr)[kU2][8]) {
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      float xt[8], xd[8];
      t[j].to_float(oct, V, xt);
      if (mode != kModeBonus) d[j].to_float(oct, V, xd);
      if (mode == kModeResidual && P.form == 1 && cheap)
        mass8_cheap(xt, xd, P, rr[j]);
      else
        mass8_of(xt, xd, mode, P, rr[j]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) rr[j][k] = 0.0f;
    }
  }
}

// A whole step's sums in the pipelined loop from the lane's shares: in the
// residual's FMA form the cheap ones, or, where cheap_ok rejects them, the
// exact ones from the step loaded again (its data has left the registers;
// a rare detour).
template <int TD, int DD>
__device__ __forceinline__ StepSums pipeline_cheap_step_sums(const char* trow, const char* drow, int64_t s,
                                                             int64_t noct, int V, const SeqPlan& P, int lane,
                                                             const CheapAcc& a) {
  const StepSums v = cheap_step_sums(a);
  if (cheap_ok(v.m, v.q)) return v;
  return exact_step_sums_reload<TD, DD>(trow, drow, s, noct, V, P, lane);
}

__device__ __forceinline__ void put_step(const StepOut& out, int s, const StepSums& v) {
  out.m[s] = v.m;
  out.q[s] = v.q;
  out.d[s] = v.d;
  out.c[s] = v.c;
}

// Sums of the draw row(s) of sequence b over all steps; wave w of nw takes
// steps w, w + nw, ... and lane 0 writes each step's sums to out.
// Whole steps run as a two-buffer software pipeline over half steps: the loads
// of the next half are in flight while the wave computes the current one, so
// its memory and arithmetic overlap.
template <int TD, int DD, int MODE, int FORM>
__device__ __forceinline__ void step_masses(const SampleLaunch& A, int b, const SeqPlan& P, int w, int nw,
                                            const StepOut& out) {
  const int lane = threadIdx.x & (kWave - 1);
  const char* trow = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)P.n * A.t_row_b;
  const char* drow = (MODE == kModeResidual) ? A.dft + (int64_t)b * A.d_seq_b + (int64_t)P.n * A.d_row_b : nullptr;
  const int64_t noct = ((int64_t)A.V + 7) / 8;
  const int full_steps = A.V / kStepTokens;  // steps that lie wholly inside the row
  const int nmine = (full_steps > w) ? (full_steps - w + nw - 1) / nw : 0;  // this wave's whole steps
  if (nmine > 0) {
    // every load is unconditional inside its block, so no buffer is copied
    // (a copy would wait for the loads in flight)
    HalfStep<TD, DD, MODE> h0, h1;
    h0.load(trow, drow, w, 0, lane);
    int64_t st = w;
    // the sums of one step from the two halves in its buffers (h1 loaded by
    // the caller just before); NEXT: load the next step's first half into h0
    // between the halves
    auto step = [&](int64_t s, bool next) {
      if constexpr (MODE == kModeResidual && FORM == 1) {
        CheapAcc a;
        h0.cheap_sums(P, a);
        if (next) h0.load(trow, drow, s + nw, 0, lane);
        h1.cheap_sums(P, a);
        return pipeline_cheap_step_sums<TD, DD>(trow, drow, s, noct, A.V, P, lane, a);
      } else {
        double r = 0.0;
        h0.template sums<FORM>(P, r);
        if (next) h0.load(trow, drow, s + nw, 0, lane);
        h1.template sums<FORM>(P, r);
        return StepSums{wave_sum(r), 0.0, 0.0, 0.0};
      }
    };
    for (int i = 0; i + 1 < nmine; ++i, st += nw) {
      h1.load(trow, drow, st, 1, lane);
      const StepSums v = step(st, true);
      if (lane == 0) put_step(out, (int)st, v);
    }
    h1.load(trow, drow, st, 1, lane);
    const StepSums v = step(st, false);
    if (lane == 0) put_step(out, (int)st, v);
  }
  // the ragged last step (if any), octet by octet
  for (int s = w + nmine * nw; s < A.ns2; s += nw) {
    const StepSums v = direct_step_sums<TD, DD, MODE, FORM>(trow, drow, s, noct, A.V, P, lane);
    if (lane == 0) put_step(out, s, v);
  }
}

template <int TD, int DD>
__device__ __forceinline__ void all_step_masses(const SampleLaunch& A, int b, const SeqPlan& P, int mode, int w,
                                                int nw, const StepOut& out) {
  if (mode == kModeResidual) {
    if (P.form == 1)
      step_masses<TD, DD, kModeResidual, 1>(A, b, P, w, nw, out);
    else
      step_masses<TD, DD, kModeResidual, 0>(A, b, P, w, nw, out);
  } else {
    if (P.form == 1)
      step_masses<TD, DD, kModeBonus, 1>(A, b, P, w, nw, out);
    else
      step_masses<TD, DD, kModeBonus, 0>(A, b, P, w, nw, out);
  }
}

// The workspace's step sums of sequence b ([4][ns2]: m, q, d, c).
__device__ __forceinline__ StepOut ws_steps(const SampleLaunch& A, int b) {
  double* g = A.steptot + (int64_t)b * 4 * A.ns2;
  return StepOut{g, g + A.ns2, g + 2 * A.ns2, g + 3 * A.ns2};
}

// Sentinels of a step's sums not yet published (m, q, c >= 0 and d finite
// for every valid row).
__device__ __forceinline__ bool step_published(const StepSums& v) {
  return v.m >= 0.0 && v.q >= 0.0 && v.d == v.d && v.c >= 0.0;
}

// The drawing part's copy of every step's sums of sequence b into LDS (wave w
// of the NW takes 64-step blocks w, w + NW, ...). Steps of other
// parts come from the workspace; one whose sums are not all visible yet still
// holds a sentinel and is recomputed here with the same bits, so no result
// depends on which stores have landed and no part ever waits for another. The
// slots are then reset to the sentinels.
template <int TD, int DD, int NW>
__device__ __forceinline__ void gather_steps(const SampleLaunch& A, int b, const SeqPlan& P, int mode, int part,
                                             const StepOut& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gnw = A.parts * NW;
  const StepOut g = ws_steps(A, b);
  const char* trow = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)P.n * A.t_row_b;
  const char* drow = (mode == kModeResidual) ? A.dft + (int64_t)b * A.d_seq_b + (int64_t)P.n * A.d_row_b : nullptr;
  const int64_t noct = ((int64_t)A.V + 7) / 8;
  for (int base = w * kWave; base < A.ns2; base += NW * kWave) {
    const int s = base + lane;
    const bool in = s < A.ns2;
    const bool mine = (s % gnw) / NW == part;  // computed by this workgroup: already in LDS
    StepSums v{0.0, 0.0, 0.0, 0.0};
    if (in) {
      if (mine) {
        v = StepSums{sh.m[s], sh.q[s], sh.d[s], sh.c[s]};
      } else {
        v.m = __hip_atomic_load(g.m + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v.q = __hip_atomic_load(g.q + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v.d = __hip_atomic_load(g.d + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v.c = __hip_atomic_load(g.c + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    unsigned long long miss = __ballot(in && !step_published(v));
    while (miss) {
      const int L = __ffsll((long long)miss) - 1;
      miss &= miss - 1;
      const StepSums m = direct_step_sums_of<TD, DD>(trow, drow, base + L, noct, A.V, mode, P, lane);
      if (lane == L) v = m;
    }
    if (in) {
      put_step(sh, s, v);
      __hip_atomic_store(g.m + s, -1.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(g.q + s, -1.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(g.d + s, __builtin_nan(""), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(g.c + s, -1.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The first-order correction of the residual, by one wave (FMA form). With the
// plan's ratio of the normalisers off by a factor 2^eta, the true residual of
// token v is e_p - 2^eta e_q, and the signed sum of e_p - e_q over the row is
// F Sp (1 - 2^-eta) (exactly 0 for an exact ratio). So with g = 2^eta - 1 =
// d / (F Sp - d), d that sum, each step's residual mass becomes m - g q
// (terms that change sign under the correction are of second order in eta).
// Corrects the step masses in place (clamped at 0) and returns g; `total` gets
// their sum in the order of wave_total.
__device__ __forceinline__ double correct_steps(const StepOut& st, int ns2, double ptot, int lane, double& total) {
  double dl = 0.0;
  for (int s = lane; s < ns2; s += kWave) dl += st.d[s];
  const double d = wave_sum(dl);
  const double g = d / (ptot - d);
  double acc = 0.0;
  for (int s = lane; s < ns2; s += kWave) {
    const double m = fmax(st.m[s] - g * st.q[s], 0.0);
    st.m[s] = m;
    acc += m;
  }
  total = wave_sum(acc);
  return g;
}

// Sum of arr[0..len) by one wave, in a fixed order.
__device__ __forceinline__ double wave_total(const double* arr, int len, int lane) {
  double acc = 0.0;
  for (int i = lane; i < len; i += kWave) acc += arr[i];
  return wave_sum(acc);
}

// Wave-wide search over arr[0..len): the first i (in order) whose running mass
// acc + arr[0] + ... + arr[i] exceeds t, with arr[i] > 0. If rounding leaves no
// such i, the last i with arr[i] > 0. On return acc holds the mass before i.
__device__ __forceinline__ int wave_find(const double* arr, int len, double t, double& acc, int lane) {
  double run = acc;
  int last_i = -1;
  double last_acc = acc;
  for (int base = 0; base < len; base += kWave) {
    const int i = base + lane;
    const double v = (i < len) ? arr[i] : 0.0;
    const double incl = wave_incl_scan(v, lane);
    const double excl = incl - v;  // only compared against t; exact enough for the search
    const unsigned long long hit = __ballot(v > 0.0 && run + incl > t);
    if (hit) {
      const int L = __ffsll((long long)hit) - 1;
      acc = run + readlane_f64(excl, L);
      return base + L;
    }
    const unsigned long long pos = __ballot(v > 0.0);
    if (pos) {
      const int L = 63 - __clzll((long long)pos);
      last_i = base + L;
      last_acc = run + readlane_f64(excl, L);
    }
    run += readlane_f64(incl, kWave - 1);
  }
  acc = last_acc;
  return last_i;
}

// The scan of one step's token masses rr[j] (octet ss * kStepOctets +
// kWave * j + lane, j < NJ, zero past the row's end) by one wave, in token
// order (octet j-major, then lane, then slot): the first token whose running
// mass acc + ... exceeds t (acc: the mass of the steps before ss). If rounding
// leaves none, the step's last token with positive mass. Every lane returns y.
template <int NJ>
__device__ __forceinline__ int scan_step(const float (&rr)[NJ][8], int ss, double t, double acc, int lane) {
  int y = -1;
  int last_pos = -1;
  for (int j = 0; j < NJ && y < 0; ++j) {
    const int64_t oct = (int64_t)ss * kStepOctets + kWave * j + lane;
    const double os = (double)sum8(rr[j]);
    const double incl = wave_incl_scan(os, lane);
    const double excl = incl - os;
    int lk = -1;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (rr[j][k] > 0.0f) lk = k;
    if (lk >= 0) last_pos = (int)(oct * 8 + lk);  // later j / lanes have larger ids
    const unsigned long long hit = __ballot(os > 0.0 && acc + incl > t);
    if (hit) {
      const int L = __ffsll((long long)hit) - 1;
      int yy = -1;
      if (lane == L) {
        double run = acc + excl;
        for (int k = 0; k < 8; ++k) {
          if (rr[j][k] > 0.0f) {
            run += (double)rr[j][k];
            if (run > t) {
              yy = (int)(oct * 8 + k);
              break;
            }
          }
        }
        if (yy < 0) yy = (int)(oct * 8 + lk);
      }
      y = __builtin_amdgcn_readlane(yy, L);
    } else {
      acc += readlane_f64(incl, kWave - 1);
    }
  }
  if (y < 0) {
    // rounding pushed t past the step's rescanned mass: take its last positive token
    int m = last_pos;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
    y = m;
  }
  return y;
}

// Rescan of step ss of the draw row(s) of sequence b by one wave: its token
// masses, then the scan above.
template <int TD, int DD>
__device__ __forceinline__ int rescan_step(const SampleLaunch& A, int b, const SeqPlan& P, int mode, int ss, double t,
                                           double acc, int lane, bool cheap) {
  const char* trow = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)P.n * A.t_row_b;
  const char* drow = (mode != kModeBonus) ? A.dft + (int64_t)b * A.d_seq_b + (int64_t)P.n * A.d_row_b : nullptr;
  const int64_t noct = ((int64_t)A.V + 7) / 8;
  float rr[kU2][8];
  step_octet_masses<TD, DD>(trow, drow, ss, noct, A.V, mode, P, lane, cheap, rr);
  return scan_step<kU2>(rr, ss, t, acc, lane);
}

// Every output of a valid sequence b once y is drawn, by one wave whose lane
// k < gamma holds draft token k in xi (so the tokens are not loaded again).
template <int TD>
__device__ __forceinline__ void write_outputs(const SampleLaunch& A, int b, const SeqPlan& P, int mode, int y,
                                              double total, int lane, int xi) {
  const int G = A.gamma, n = P.n;
  int32_t* otok = A.out_tok + (int64_t)b * (G + 1);
  if (lane < G) otok[lane] = (lane < n) ? xi : (lane == n ? y : -1);
  if (lane == 0) {
    otok[G] = (n == G) ? y : -1;
    if (A.out_n) A.out_n[b] = n;
    if (A.diag_mass) A.diag_mass[b] = (float)(total / (P.sp * P.fscale));
    if (A.out_py) {
      // p(y) of a bonus-mode draw, from the row's statistics in fp64
      float py = __builtin_nanf("");
      if (mode == kModeBonus) {
        const float x = load_elem<TD>(A.tgt + (int64_t)b * A.t_seq_b + (int64_t)n * A.t_row_b, y);
        py = (float)(exp2((double)x * (double)P.kl - P.ct) / P.sp);
      }
      A.out_py[b] = py;
    }
  }
}

// The outputs of an invalid sequence (every token -1).
__device__ __forceinline__ void write_invalid(const SampleLaunch& A, int b, int t, int t0, int nt) {
  const int G = A.gamma;
  int32_t* otok = A.out_tok + (int64_t)b * (G + 1);
  for (int k = t - t0; k <= G; k += nt) otok[k] = -1;
  if (t == t0) {
    if (A.out_n) A.out_n[b] = -1;
    if (A.out_py) A.out_py[b] = __builtin_nanf("");
    if (A.diag_mass) A.diag_mass[b] = __builtin_nanf("");
  }
}

// Inverse-CDF draw from the step masses stot[0..ns2) (total mass `total`) of
// the draw row(s) of sequence b, then every output of the sequence, by wave 0
// (the other waves return): lane k < gamma of wave 0 holds draft token k in xi.
// scheap: the steps' form flags (null: no step took the cheap form).
template <int TD, int DD>
__device__ __forceinline__ void draw_and_write(const SampleLaunch& A, int b, const SeqPlan& P, int mode, const double* stot,
                                               const double* scheap, double total, int xi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w != 0) return;
  // (5) inverse-CDF search
  const double t = (double)P.ug * total;
  double acc = 0.0;
  // wave_find returns -1 only if every mass is zero, which valid rows rule
  // out; clamp anyway so that no index can leave the arrays.
  const int ss = max(wave_find(stot, A.ns2, t, acc, lane), 0);
  const bool cheap = mode == kModeResidual && scheap && scheap[ss] > 0.5;
  const int y = rescan_step<TD, DD>(A, b, P, mode, ss, t, acc, lane, cheap);
  // (6) outputs
  write_outputs<TD>(A, b, P, mode, y, total, lane, xi);
}

// The plan of the draw of a sequence whose first stop is n (gamma: every
// draft accepted) with accept code code_n there; tn, dn: the statistics of
// target row n and (n < gamma) draft row n. nst: rows with statistics.
__device__ __forceinline__ SeqPlan make_plan(int n, int code_n, int G, int nst, bool tv, float kl, float ug,
                                             const RowStat& tn, const RowStat& dn) {
#pragma clang fp contract(off)
  bool valid = tv && (n == G || code_n == 0) && ug >= 0.0f && ug < 1.0f && n < nst;
  if (n == G) valid = valid && tn.valid;
  SeqPlan Q;
  Q.valid = valid;
  Q.ug = ug;
  Q.n = n;
  Q.mode = (n == G) ? kModeBonus : kModeResidual;
  Q.kl = kl;
  Q.ct = tn.c;
  Q.mp = tn.m;
  Q.sp = tn.s;
  Q.g = 0.0;
  const double kld = (double)kl;
  Q.cp = (float)tn.c;  // exact for the integer shifts of the statistics pass
  const double dp = tn.c - (double)Q.cp;
  // the shifts must round by less than half a log2 unit: |c| < 2^24
  bool fma_ok = fabs(tn.c) < 0x1p24;
  Q.kap_hi = 0.0f;
  Q.kap_lo = 0.0f;
  if (n < G) {
    Q.mq = dn.m;
    Q.sq = dn.s;
    const double cqx = dn.c - log2(Q.sp / Q.sq) - dp;
    Q.cq = (float)cqx;
    Q.cq_lo = (float)(cqx - (double)Q.cq);
    Q.cq_s = (float)exp2((double)Q.cq - cqx);
    Q.dt = (float)((double)Q.cp - cqx);
    fma_ok = fma_ok && fabs(cqx) < 0x1p24;
  } else {
    Q.mq = 0.0f;
    Q.sq = 1.0;
    Q.cq = 0.0f;
    Q.cq_lo = 0.0f;
    Q.cq_s = 1.0f;
    Q.dt = 0.0f;
  }
  Q.form = fma_ok ? 1 : 0;
  if (fma_ok) {
    Q.fscale = (dp == 0.0) ? 1.0 : exp2(dp);  // 1 for the integer shifts of the statistics pass
  } else {
    // subtract form: e_p = exp2((x_t - mp) * kl) = p_v * sp * Fp, kappa = (sp Fp) / (sq Fq)
    const double Fp = exp2(tn.c - (double)tn.m * kld);
    Q.fscale = Fp;
    if (n < G) {
      const double Fq = exp2(dn.c - (double)dn.m * kld);
      const double kap = (Q.sp * Fp) / (Q.sq * Fq);
      Q.kap_hi = (float)kap;
      Q.kap_lo = (float)(kap - (double)Q.kap_hi);
    }
  }
  return Q;
}

// A copy of a plan held in LDS, in scalar registers: the plan is the same for
// the whole workgroup, and reading it word by word through readfirstlane
// tells the compiler so (a plan in vector registers would take 24 of them).
__device__ __forceinline__ SeqPlan uniform_plan(const SeqPlan& src) {
  static_assert(sizeof(SeqPlan) % 4 == 0, "the plan is a whole number of 32-bit words");
  constexpr int kWords = (int)(sizeof(SeqPlan) / 4);
  uint32_t w[kWords];
  __builtin_memcpy(w, &src, sizeof(SeqPlan));
#pragma unroll
  for (int k = 0; k < kWords; ++k) w[k] = __builtin_amdgcn_readfirstlane(w[k]);
  SeqPlan P;
  __builtin_memcpy(&P, w, sizeof(SeqPlan));
  return P;
}

// ---------------------------------------------------------------------------
// finish kernel: one workgroup (512 or 1024 threads) per sequence or part
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 3;  // rows per wave merged from one batch of loads: 2 * gamma + 1 <= 24
// NW: waves per workgroup (kFinWaves, or twice that for split sequences).
// OS: one workgroup per sequence and at most one step per wave: each wave
// keeps its step's octets in registers and the wave whose step holds the
// draw rescans it from there (no second load of the draw row at the end).
template <int TD, int DD, int NW, bool OS>
// At most 128 VGPRs, so that two 8-wave workgroups (one 16-wave one) fit a CU.
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(4))) void sv_finish_kernel(
    SampleLaunch A) {
  constexpr int NT = NW * kWave;
  __shared__ double rC[kMaxRows];
  __shared__ float rM[kMaxRows];
  __shared__ double rS[kMaxRows];
  __shared__ int rV[kMaxRows];
  __shared__ SeqPlan sP;
  __shared__ double sh_total;
  __shared__ double sh_g;
  __shared__ int sh_last;
  // step sums when the row has at most kLdsSteps steps: masses, q-masses of
  // the positive residual, signed sums of e_p - e_q
  __shared__ double sh_steps[kLdsSteps], sh_q[kLdsSteps], sh_d[kLdsSteps], sh_c[kLdsSteps];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so loops over steps stay scalar
  const int K = A.parts;  // workgroups per sequence
  const int b = (int)(blockIdx.x / (unsigned)K);
  const int part = (int)blockIdx.x - b * K;
  const float T = A.temps[b];
  const bool tv = temp_ok(T);
  const float kl = tv ? log2e_over(T) : 1.0f;
  const int G = A.gamma;
  const int tchunks = (G + 1) * A.nct;
  // rows 0..nst-1 (target and draft) have statistics: all of them after the
  // one-pass stats kernel, those up to the first rejection after early exit
  const int nst = A.reach ? min(max(A.reach[b], 0), G + 1) : G + 1;

  // (1) gathers of p(x), q(x) do not depend on the merge: issue them first
  int xi = 0;
  float ui = 0.0f, lt = 0.0f, ld = 0.0f;
  bool tok_ok = false;
  if (w == 0 && lane < G && lane < nst) {
    xi = A.tokens[(int64_t)b * G + lane];
    ui = A.uniforms[(int64_t)b * (G + 1) + lane];
    tok_ok = xi >= 0 && xi < A.V;
    if (tok_ok) {
      lt = load_elem<TD>(A.tgt + (int64_t)b * A.t_seq_b + (int64_t)lane * A.t_row_b, xi);
      ld = load_elem<DD>(A.dft + (int64_t)b * A.d_seq_b + (int64_t)lane * A.d_row_b, xi);
    }
  }

  __shared__ int sh_xi[kWave];  // the draft tokens, for the wave that draws (OS)
  if (OS && w == 0) sh_xi[lane] = xi;

  // (2) merge the partials of every row: one wave per row, lanes over partials.
  // When every row has at most one partial per lane and each wave has at most
  // kMergeRows rows, a wave loads the partials of all its rows before merging
  // any (one memory round trip instead of one per row).
  const int nrows = 2 * G + 1;
  if (A.nct * kWaves <= kWave && A.ncd * kWaves <= kWave && nrows <= kMergeRows * NW) {
    RowPartial q[kMergeRows];
    bool have[kMergeRows];
#pragma unroll
    for (int k = 0; k < kMergeRows; ++k) {
      const int t = w + k * NW;
      const int pos = t <= G ? t : t - G - 1;
      const int nrec = (t <= G ? A.nct : A.ncd) * kWaves;
      const int base = t <= G ? t * A.nct : tchunks + pos * A.ncd;
      have[k] = t < nrows && pos < nst && lane < nrec;
      q[k] = RowPartial{};
      if (have[k]) q[k] = A.part[((int64_t)b * A.per_seq + base) * kWaves + lane];
    }
#pragma unroll
    for (int k = 0; k < kMergeRows; ++k) {
      const int t = w + k * NW;
      if (t >= nrows) break;
      const int pos = t <= G ? t : t - G - 1;
      RowStat rs{0.0, 0.0f, 0.0, 0};
      if (pos < nst) rs = merge_row_one(q[k], have[k], kl, tv);
      if (lane == 0) {
        rC[t] = rs.c;
        rM[t] = rs.m;
        rS[t] = rs.s;
        rV[t] = rs.valid;
      }
    }
  } else {
    for (int t = w; t < nrows; t += NW) {
      int nrec, base, pos;
      if (t <= G) {
        nrec = A.nct * kWaves;
        base = t * A.nct;
        pos = t;
      } else {
        nrec = A.ncd * kWaves;
        base = tchunks + (t - G - 1) * A.ncd;
        pos = t - G - 1;
      }
      if (pos >= nst) {
        if (lane == 0) {
          rC[t] = 0.0;
          rM[t] = 0.0f;
          rS[t] = 0.0;
          rV[t] = 0;
        }
        continue;
      }
      const RowStat rs = merge_row(A.part + ((int64_t)b * A.per_seq + base) * kWaves, nrec, kl, tv, lane);
      if (lane == 0) {
        rC[t] = rs.c;
        rM[t] = rs.m;
        rS[t] = rs.s;
        rV[t] = rs.valid;
      }
    }
  }
  __syncthreads();

  // (3) accept tests and first rejection (wave 0); code 3: position not reached
  // (early exit stopped before it)
  if (w == 0) {
    int code = 1;  // 1 accepted, 0 rejected, 2 invalid
    if (lane < G) {
      const int i = lane;
      float pxo = __builtin_nanf(""), qxo = __builtin_nanf("");
      if (i < nst) {
        const RowStat ts{rC[i], rM[i], rS[i], rV[i]}, ds{rC[G + 1 + i], rM[G + 1 + i], rS[G + 1 + i], rV[G + 1 + i]};
        const AcceptOut ao = accept_test(lt, ld, ts, ds, kl, ui, tok_ok, tv, A.diag_px || A.diag_qx);
        code = ao.code;
        pxo = ao.px;
        qxo = ao.qx;
      } else {
        code = 3;
      }
      if (A.diag_px) A.diag_px[(int64_t)b * G + i] = pxo;
      if (A.diag_qx) A.diag_qx[(int64_t)b * G + i] = qxo;
    }
    const unsigned long long stop = __ballot(code != 1);
    const int n = stop ? (__ffsll((long long)stop) - 1) : G;
    const int code_n = __builtin_amdgcn_readlane(code, n < G ? n : 0);
    if (lane == 0) {
      const RowStat tn{rC[n], rM[n], rS[n], rV[n]};
      const RowStat dn =
          (n < G) ? RowStat{rC[G + 1 + n], rM[G + 1 + n], rS[G + 1 + n], rV[G + 1 + n]} : RowStat{0.0, 0.0f, 1.0, 0};
      sP = make_plan(n, code_n, G, nst, tv, kl, A.uniforms[(int64_t)b * (G + 1) + G], tn, dn);
    }
  }
  __syncthreads();
  const SeqPlan P = uniform_plan(sP);
  if (!P.valid) {
    // every part reaches the same plan; part 0 writes the outputs
    if (part == 0) write_invalid(A, b, tid, 0, NT);
    return;
  }

  if constexpr (OS) {
    // (4') one step per wave, its octets kept (parts == 1, ns2 <= NW)
    int mode = P.mode;
    const StepOut st{sh_steps, sh_q, sh_d, sh_c};
    const char* trow = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)P.n * A.t_row_b;
    const char* drow = (mode == kModeResidual) ? A.dft + (int64_t)b * A.d_seq_b + (int64_t)P.n * A.d_row_b : nullptr;
    const int64_t noct = ((int64_t)A.V + 7) / 8;
    OctetIn<TD> kt[kU2];
    OctetIn<DD> kd[kU2];
    const bool has = w < A.ns2;
    if (has) {
      const StepSums v = kept_step_sums_of<TD, DD>(trow, drow, w, noct, A.V, mode, P, lane, kt, kd);
      if (lane == 0) put_step(st, w, v);
    }
    __syncthreads();
    if (w == 0) {
      double tot, g = 0.0;
      if (mode == kModeResidual && P.form == 1)
        g = correct_steps(st, A.ns2, P.sp * P.fscale, lane, tot);
      else
        tot = wave_total(st.m, A.ns2, lane);
      if (lane == 0) {
        sh_total = tot;
        sh_g = g;
      }
    }
    __syncthreads();
    SeqPlan Pd = P;
    Pd.g = sh_g;
    if (!(sh_total > 0.0) && mode == kModeResidual) {
      // Nothing left after the rejection (p_n == q_n up to rounding): draw from
      // p_n, from the kept target octets.
      mode = kModeBonus;
      Pd.g = 0.0;
      if (has) {
        const StepSums v = kept_bonus_sums<TD, DD>(kt, w, noct, A.V, P, lane);
        if (lane == 0) put_step(st, w, v);
      }
      __syncthreads();
      if (w == 0) {
        const double tot = wave_total(st.m, A.ns2, lane);
        if (lane == 0) sh_total = tot;
      }
      __syncthreads();
    }
    const double total = sh_total;
    // (5) the step that holds the draw (every wave finds the same one), then
    // its rescan by the wave that holds it, and (6) the outputs
    const double t = (double)Pd.ug * total;
    double acc = 0.0;
    const int ss = max(wave_find(st.m, A.ns2, t, acc, lane), 0);
    if (w != ss) return;
    const bool cheap = mode == kModeResidual && sh_c[ss] > 0.5;
    float rr[kU2][8];
    kept_octet_masses<TD, DD>(kt, kd, ss, noct, A.V, mode, Pd, lane, cheap, rr);
    const int y = scan_step<kU2>(rr, ss, t, acc, lane);
    write_outputs<TD>(A, b, Pd, mode, y, total, lane, sh_xi[lane]);
  } else {
  // (4) sums of the drawn distribution's steps, every wave on its steps, into
    // LDS when they fit, else the workspace. (The two calls differ only in the
    // address space of the output, which keeps the stores of the streaming loop
    // out of the generic path: after a generic store every wait for a load
    // would drain all loads in flight.)
    // With K parts the waves of all parts share the steps round-robin: wave w of
    // part p is wave p * NW + w of K * NW (K > 1 only when the
    // steps fit in LDS).
    int mode = P.mode;
    const bool lds_steps = A.ns2 <= kLdsSteps;
    const StepOut sh_out{sh_steps, sh_q, sh_d, sh_c};
    const StepOut st = lds_steps ? sh_out : ws_steps(A, b);
    if (lds_steps)
      all_step_masses<TD, DD>(A, b, P, mode, part * NW + w, K * NW, sh_out);
    else
      all_step_masses<TD, DD>(A, b, P, mode, w, NW, ws_steps(A, b));
    __syncthreads();  // every wave's step sums are visible to the workgroup
    if (K > 1) {
      // Hand-off: each part publishes its step sums (relaxed device-scope
      // atomic stores, which no cache of this XCD holds back) and counts itself
      // done; the part that counts last gathers every step's sums and draws.
      const StepOut g = ws_steps(A, b);
      for (int s = tid; s < A.ns2; s += NT)
        if ((s % (K * NW)) / NW == part) {
          __hip_atomic_store(g.m + s, sh_steps[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(g.q + s, sh_q[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(g.d + s, sh_d[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(g.c + s, sh_c[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      __syncthreads();
      if (tid == 0) sh_last = __hip_atomic_fetch_add(A.done + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == K - 1;
      __syncthreads();
      if (!sh_last) return;
      if (tid == 0) A.done[b] = 0;  // ready for the next finish launch on this workspace
      gather_steps<TD, DD, NW>(A, b, P, mode, part, sh_out);
      __syncthreads();
    }
    if (w == 0) {
      // the residual's first-order correction of the normalisers' ratio (FMA
      // form; g = 0 otherwise), then the total
      double tot, g = 0.0;
      if (mode == kModeResidual && P.form == 1)
        g = correct_steps(st, A.ns2, P.sp * P.fscale, lane, tot);
      else
        tot = wave_total(st.m, A.ns2, lane);
      if (lane == 0) {
        sh_total = tot;
        sh_g = g;
      }
    }
    __syncthreads();
    SeqPlan Pd = P;
    Pd.g = sh_g;
    if (!(sh_total > 0.0) && mode == kModeResidual) {
      // Nothing left after the rejection (p_n == q_n up to rounding): draw from p_n.
      mode = kModeBonus;
      Pd.g = 0.0;
      if (lds_steps)
        all_step_masses<TD, DD>(A, b, P, mode, w, NW, sh_out);
      else
        all_step_masses<TD, DD>(A, b, P, mode, w, NW, ws_steps(A, b));
      __syncthreads();
      if (w == 0) {
        const double tot = wave_total(st.m, A.ns2, lane);
        if (lane == 0) sh_total = tot;
      }
      __syncthreads();
    }
    const double total = sh_total;

    draw_and_write<TD, DD>(A, b, Pd, mode, st.m, st.c, total, xi);
  }
}

// ---------------------------------------------------------------------------
// one-pass draft sampler: one workgroup (512 or 1024 threads) per row (gamma = 0)
// ---------------------------------------------------------------------------
// One pass over the row writes the exact mass of every 2048-token step into
// LDS, each against its own reference: a lane takes its terms against a
// reference that moves lazily (as in the statistics pass), and a step's lanes
// are combined at their largest reference. The draw then merges the step masses
// into the row's total, searches them and rescans one step, so the row is read
// once instead of twice.

// A lane's reference across the steps of its wave (FMA form).
struct LaneRef {
  float m;  // reference logit (-inf while every value seen was -inf)
  float c;  // fp32(m * kl)
  int ovf;  // |c| >= 2^24: the row is redone in the subtract form
};

template <int NO>
__device__ __forceinline__ float octet_terms_fma(const float (&x)[NO][8], float kl, float c) {
  float u[NO];
#pragma unroll
  for (int j = 0; j < NO; ++j) {
    float e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = hw_exp2(fmaf(x[j][k], kl, -c));
    u[j] = sum8(e);
  }
  if constexpr (NO == 2)
    return u[0] + u[1];
  else
    return (u[0] + u[1]) + (u[2] + u[3]);
}

// Sum of the lane's terms over NO octets, moving the reference when a term
// would exceed 2^64 (or on the first finite value, +inf or NaN).
template <int NO>
__device__ __forceinline__ float lane_terms(const float (&x)[NO][8], float kl, LaneRef& R) {
  float a = octet_terms_fma<NO>(x, kl, R.c);
  if (!(a <= 0x1p64f)) {
    float gm = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < NO; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        gm = fmaxf(gm, x[j][k]);
        nan |= x[j][k] != x[j][k];
      }
    if (gm > R.m) {
      const float cn = __fmul_rn(gm, kl);
      if (!(fabsf(cn) < 0x1p24f) && __builtin_isfinite(gm)) R.ovf = 1;
      R.m = gm;
      R.c = cn;
    }
    a = (R.c == -INFINITY) ? 0.0f : octet_terms_fma<NO>(x, kl, R.c);
    if (nan) a = __builtin_nanf("");
  }
  return a;
}

// Step total of one wave from its lanes' sums (FMA form): lane 0 writes the
// step's reference shift, reference logit and mass.
__device__ __forceinline__ void write_step_fma(float a, const LaneRef& R, int s, float* stepC, float* stepM,
                                               double* stepS) {
  const int lane = threadIdx.x & (kWave - 1);
  const float Mc = wave_max(R.c);
  double tot;
  float Mm;
  if (Mc == -INFINITY) {
    tot = wave_sum((double)a);  // every value -inf (0) or NaN seen
    Mm = -INFINITY;
  } else {
    tot = wave_sum((double)a * (double)hw_exp2(R.c - Mc));
    Mm = wave_max(R.c == Mc ? R.m : -INFINITY);
  }
  if (lane == 0) {
    stepC[s] = Mc;
    stepM[s] = Mm;
    stepS[s] = tot;
  }
}

template <int DT>
__device__ __forceinline__ void unpack_half(const HalfStep<DT, DT, kModeBonus>& h, float (&x)[kHalfU][8]) {
#pragma unroll
  for (int j = 0; j < kHalfU; ++j) h.t[j].unpack(x[j]);
}

// The values of step s of a row for one wave: x[j] is octet
// s * kStepOctets + kWave * j + lane, -inf at and past V. Every load is issued
// before the first value is used.
template <int DT>
__device__ __forceinline__ void load_step(const char* row, int64_t s, int64_t noct, int V, int lane,
                                          float (&x)[kU2][8]) {
  OctetIn<DT> o[kU2];
#pragma unroll
  for (int j = 0; j < kU2; ++j) o[j].load(row, s * kStepOctets + kWave * j + lane, noct, V);
#pragma unroll
  for (int j = 0; j < kU2; ++j) {
    const int64_t oct = s * kStepOctets + kWave * j + lane;
    if (oct < noct) {
      o[j].to_float(oct, V, x[j]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[j][k] = -INFINITY;
    }
  }
}

// FMA-form pass: wave w of NW takes steps w, w + NW, ...; whole steps through
// the two-buffer pipeline of the draw, the ragged last step octet by octet.
template <int DT, int NW>
__device__ void draft_pass_fma(const char* row, int V, int ns2, float kl, LaneRef& R, float* stepC, float* stepM,
                               double* stepS) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = NW;
  const int64_t noct = ((int64_t)V + 7) / 8;
  const int full_steps = V / kStepTokens;
  const int nmine = (full_steps > w) ? (full_steps - w + nw - 1) / nw : 0;
  if (nmine > 0) {
    // every load is unconditional inside its block (see step_masses)
    HalfStep<DT, DT, kModeBonus> h0, h1;
    float x0[kHalfU][8], x1[kHalfU][8];
    h0.load(row, nullptr, w, 0, lane);
    int64_t st = w;
    for (int i = 0; i + 1 < nmine; ++i, st += nw) {
      h1.load(row, nullptr, st, 1, lane);
      unpack_half<DT>(h0, x0);
      float a0 = lane_terms<kHalfU>(x0, kl, R);
      const float c0 = R.c;
      h0.load(row, nullptr, st + nw, 0, lane);
      unpack_half<DT>(h1, x1);
      const float a1 = lane_terms<kHalfU>(x1, kl, R);
      if (R.c != c0 && c0 != -INFINITY) a0 *= hw_exp2(c0 - R.c);
      write_step_fma(a0 + a1, R, (int)st, stepC, stepM, stepS);
    }
    h1.load(row, nullptr, st, 1, lane);
    unpack_half<DT>(h0, x0);
    float a0 = lane_terms<kHalfU>(x0, kl, R);
    const float c0 = R.c;
    unpack_half<DT>(h1, x1);
    const float a1 = lane_terms<kHalfU>(x1, kl, R);
    if (R.c != c0 && c0 != -INFINITY) a0 *= hw_exp2(c0 - R.c);
    write_step_fma(a0 + a1, R, (int)st, stepC, stepM, stepS);
  }
  for (int s = w + nmine * nw; s < ns2; s += nw) {
    float x[kU2][8];
    load_step<DT>(row, s, noct, V, lane, x);
    const float a = lane_terms<kU2>(x, kl, R);
    write_step_fma(a, R, s, stepC, stepM, stepS);
  }
}

// Subtract-form pass (|m * kl| >= 2^24 somewhere in the row): each step
// against its own maximum m_s; stepM = m_s, stepS = sum exp2((x - m_s) * kl).
template <int DT, int NW>
__device__ void draft_pass_sub(const char* row, int V, int ns2, float kl, float* stepM, double* stepS) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t noct = ((int64_t)V + 7) / 8;
  for (int s = w; s < ns2; s += NW) {
    float x[kU2][8];
    float gm = -INFINITY;
    bool nan = false;
    load_step<DT>(row, s, noct, V, lane, x);
#pragma unroll
    for (int j = 0; j < kU2; ++j) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        gm = fmaxf(gm, x[j][k]);
        nan |= x[j][k] != x[j][k];
      }
    }
    const float ms = wave_max(gm);
    float a = 0.0f;
    if (ms != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kU2; ++j) {
        float e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = hw_exp2((x[j][k] - ms) * kl);
        a += sum8(e);
      }
    }
    if (nan) a = __builtin_nanf("");
    const double tot = wave_sum((double)a);
    if (lane == 0) {
      stepM[s] = ms;
      stepS[s] = tot;
    }
  }
}

// NW waves per workgroup: 16 when there are at most as many rows as CUs (one
// workgroup per CU then; twice the loads in flight per row), else 8.
template <int DT, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(4))) void sv_draft1_kernel(
    SampleLaunch A) {
  __shared__ float stepC[kLdsSteps], stepM[kLdsSteps];
  __shared__ double stepS[kLdsSteps];
  __shared__ SeqPlan sP;
  __shared__ double sh_total;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  const float T = A.temps[b];
  const bool tv = temp_ok(T);
  const float kl = tv ? log2e_over(T) : 1.0f;
  const char* row = A.tgt + (int64_t)b * A.t_seq_b;
  const int ns2 = A.ns2;

  LaneRef R{-INFINITY, -INFINITY, 0};
  draft_pass_fma<DT, NW>(row, A.V, ns2, kl, R, stepC, stepM, stepS);
  const bool sub = __syncthreads_or(R.ovf) != 0;
  if (sub) {
    draft_pass_sub<DT, NW>(row, A.V, ns2, kl, stepM, stepS);
    __syncthreads();
  }
  // merge the steps into step masses against the row's reference (wave 0)
  if (w == 0) {
    double Ms = -INFINITY;
    for (int s = lane; s < ns2; s += kWave)
      Ms = fmax(Ms, sub ? (double)stepM[s] * (double)kl : (double)stepC[s]);
    Ms = wave_max_f64(Ms);
    float mp = -INFINITY;
    for (int s = lane; s < ns2; s += kWave) {
      const double sh = sub ? (double)stepM[s] * (double)kl : (double)stepC[s];
      if (sh == Ms) mp = fmaxf(mp, stepM[s]);
    }
    mp = wave_max(mp);
    for (int s = lane; s < ns2; s += kWave) {
      const double sh = sub ? (double)stepM[s] * (double)kl : (double)stepC[s];
      stepS[s] = stepS[s] * exp2(sh - Ms);
    }
    const double total = wave_total(stepS, ns2, lane);
    if (lane == 0) {
      const float u = A.uniforms[b];
      SeqPlan Q;
      Q.valid = tv && u >= 0.0f && u < 1.0f && __builtin_isfinite(total) && total > 0.0 &&
                __builtin_isfinite(mp);
      Q.ug = u;
      Q.n = 0;
      Q.mode = kModeBonus;
      Q.form = sub ? 0 : 1;
      Q.kl = kl;
      Q.mp = mp;
      Q.mq = 0.0f;
      Q.kap_hi = Q.kap_lo = 0.0f;
      // the step masses are sums of exp2(x * kl - Ms): in the FMA form Ms is a
      // float (a lane's shift), so e_p = exp2(fma(x, kl, -cp)) with cp = Ms; in
      // the subtract form Ms = mp * kl
      Q.ct = Ms;
      Q.cp = sub ? 0.0f : (float)Ms;
      Q.cq = Q.cq_lo = Q.dt = 0.0f;
      Q.cq_s = 1.0f;
      Q.fscale = 1.0;
      Q.sp = total;
      Q.sq = 1.0;
      Q.g = 0.0;
      sP = Q;
      sh_total = total;
    }
  }
  __syncthreads();
  const SeqPlan P = uniform_plan(sP);
  if (!P.valid) {
    if (tid == 0) {
      A.out_tok[b] = -1;
      if (A.out_py) A.out_py[b] = __builtin_nanf("");
    }
    return;
  }
  draw_and_write<DT, DT>(A, b, P, kModeBonus, stepS, nullptr, sh_total, 0);
}

// ---------------------------------------------------------------------------
// small vocabularies (V <= kStepTokens): one wave per sequence, every step
// ---------------------------------------------------------------------------
// Statistics of one row from this lane's PL values x (value v = lane + 64 k;
// -inf past V) by one wave: the reference is the row's maximum, s = sum_v
// exp2((x_v - m) * kl) with fp32 terms summed in fp64 (each lane's values in
// order, then the wave sum). NaN or +inf values make the row invalid, as in the
// statistics pass.
template <int PL>
__device__ __forceinline__ RowStat small_row_stat(const float (&x)[PL], float kl, bool tv) {
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < PL; ++k) m = fmaxf(m, x[k]);
  m = wave_max(m);
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < PL; ++k) {
    const bool nan = x[k] != x[k];
    if (nan || x[k] != -INFINITY) s += nan ? (double)x[k] : (double)hw_exp2((x[k] - m) * kl);
  }
  s = wave_sum(s);
  RowStat r;
  r.c = (double)m * (double)kl;
  r.m = m;
  r.s = s;
  r.valid = tv && __builtin_isfinite(s) && s > 0.0 && __builtin_isfinite(m);
  return r;
}

// The whole verify of sequences with V <= kStepTokens: wave w of workgroup g
// takes sequence 4 g + w. Row statistics straight from the rows (no
// partials), the accept tests, the plan, the one step's mass, the rescan and
// the outputs, with the same functions as the two-kernel path from the plan
// on. Needs no workspace.
// PL: values of a row per lane (V <= 64 PL); rows are loaded RB at a time, so
// that their loads overlap.
template <int TD, int DD, int PL>
__global__ __launch_bounds__(kThreads) void sv_small_kernel(SampleLaunch A) {
  constexpr int RB = PL == 1 ? 16 : (PL <= 4 ? 4 : 1);
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x * kWaves + w;
  if (b >= A.B) return;  // the whole wave; this kernel has no workgroup barrier
  const float T = A.temps[b];
  const bool tv = temp_ok(T);
  const float kl = tv ? log2e_over(T) : 1.0f;
  const int G = A.gamma;

  // the draft tokens, their uniforms and logits (position = lane)
  int xi = 0;
  float ui = 0.0f, lt = 0.0f, ld = 0.0f;
  bool tok_ok = false;
  if (lane < G) {
    xi = A.tokens[(int64_t)b * G + lane];
    ui = A.uniforms[(int64_t)b * (G + 1) + lane];
    tok_ok = xi >= 0 && xi < A.V;
    if (tok_ok) {
      lt = load_elem<TD>(A.tgt + (int64_t)b * A.t_seq_b + (int64_t)lane * A.t_row_b, xi);
      ld = load_elem<DD>(A.dft + (int64_t)b * A.d_seq_b + (int64_t)lane * A.d_row_b, xi);
    }
  }
  // statistics of target rows 0..G (slots 0..G) and draft rows 0..G-1 (slots
  // G+1..2G <= 128); slot t is kept by lane t % 64 in register set t / 64
  float m0 = 0.0f, m1 = 0.0f, m2 = 0.0f;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0;
  int v0 = 0, v1 = 0, v2 = 0;
  for (int t0 = 0; t0 <= 2 * G; t0 += RB) {
    float x[RB][PL];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + r;
      const char* row = (t <= G) ? A.tgt + (int64_t)b * A.t_seq_b + (int64_t)t * A.t_row_b
                                 : A.dft + (int64_t)b * A.d_seq_b + (int64_t)(t - G - 1) * A.d_row_b;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const int v = lane + kWave * k;
        x[r][k] = -INFINITY;
        if (t <= 2 * G && v < A.V) x[r][k] = (t <= G) ? load_elem<TD>(row, v) : load_elem<DD>(row, v);
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + r;
      if (t > 2 * G) break;
      const RowStat st = small_row_stat<PL>(x[r], kl, tv);
      if (lane == (t & (kWave - 1))) {
        if (t < kWave) {
          m0 = st.m;
          s0 = st.s;
          v0 = st.valid;
        } else if (t < 2 * kWave) {
          m1 = st.m;
          s1 = st.s;
          v1 = st.valid;
        } else {
          m2 = st.m;
          s2 = st.s;
          v2 = st.valid;
        }
      }
    }
  }
  // slot t's statistics: in every lane for a uniform t, from lane j % 64 for a per-lane j
  // the row's reference is its maximum m: shift m * kl (exact in fp64)
  auto stat = [&](float m, double s, int v) { return RowStat{(double)m * (double)kl, m, s, v}; };
  auto slot_uniform = [&](int t) {
    const int l = t & (kWave - 1);
    if (t < kWave) return stat(readlane_f32(m0, l), readlane_f64(s0, l), __builtin_amdgcn_readlane(v0, l));
    if (t < 2 * kWave) return stat(readlane_f32(m1, l), readlane_f64(s1, l), __builtin_amdgcn_readlane(v1, l));
    return stat(readlane_f32(m2, l), readlane_f64(s2, l), __builtin_amdgcn_readlane(v2, l));
  };
  // accept tests (lane i: position i; target slot i is its own) and the first stop
  const int j = G + 1 + lane;  // this lane's draft slot
  const int jl = j & (kWave - 1);
  const float dm0 = __shfl(m0, jl, kWave), dm1 = __shfl(m1, jl, kWave), dm2 = __shfl(m2, jl, kWave);
  const double ds0 = __shfl(s0, jl, kWave), ds1 = __shfl(s1, jl, kWave), ds2 = __shfl(s2, jl, kWave);
  const int dv0 = __shfl(v0, jl, kWave), dv1 = __shfl(v1, jl, kWave), dv2 = __shfl(v2, jl, kWave);
  int code = 1;
  if (lane < G) {
    const RowStat ts = stat(m0, s0, v0);
    const RowStat ds = (j < kWave) ? stat(dm0, ds0, dv0) : (j < 2 * kWave ? stat(dm1, ds1, dv1) : stat(dm2, ds2, dv2));
    const AcceptOut ao = accept_test(lt, ld, ts, ds, kl, ui, tok_ok, tv, A.diag_px || A.diag_qx);
    code = ao.code;
    if (A.diag_px) A.diag_px[(int64_t)b * G + lane] = ao.px;
    if (A.diag_qx) A.diag_qx[(int64_t)b * G + lane] = ao.qx;
  }
  const unsigned long long stop = __ballot(code != 1);
  const int n = stop ? (__ffsll((long long)stop) - 1) : G;
  const int code_n = __builtin_amdgcn_readlane(code, n < G ? n : 0);
  const RowStat tn = slot_uniform(n);
  const RowStat dn = (n < G) ? slot_uniform(G + 1 + n) : RowStat{0.0, 0.0f, 1.0, 0};
  const SeqPlan P = make_plan(n, code_n, G, G + 1, tv, kl, A.uniforms[(int64_t)b * (G + 1) + G], tn, dn);
  if (!P.valid) {
    write_invalid(A, b, lane, 0, kWave);
    return;
  }
  // the drawn distribution's one step, then the draw
  const char* trow = A.tgt + (int64_t)b * A.t_seq_b + (int64_t)n * A.t_row_b;
  const char* drow = (n < G) ? A.dft + (int64_t)b * A.d_seq_b + (int64_t)n * A.d_row_b : nullptr;
  const int64_t noct = ((int64_t)A.V + 7) / 8;
  int mode = P.mode;
  if constexpr (PL <= 4) {
    // Rows of at most 32 octets: a lane holds at most one octet of the step.
    // Its values are loaded once and serve the total, the bonus-mode fallback
    // and the scan (the same operations, in the same order, as the step mass
    // and rescan of longer rows).
    const bool have = lane < noct;
    float xt[8], xd[8], rr[1][8];
#pragma unroll
    for (int k = 0; k < 8; ++k) xd[k] = 0.0f;
    if (have) {
      load_octet<TD>(trow, lane, A.V, xt);
      if (mode == kModeResidual) load_octet<DD>(drow, lane, A.V, xd);
    }
    bool cheap = false;
    auto step_total = [&](int m, const SeqPlan& Q) -> double {
      double lacc = 0.0;
      if (have) {
        mass8_of(xt, xd, m, Q, rr[0], cheap);
        lacc += (double)sum8(rr[0]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) rr[0][k] = 0.0f;
      }
      return wave_sum(lacc);
    };
    SeqPlan Pd = P;
    if (mode == kModeResidual && P.form == 1) {
      // the step's form (see cheap_ok), then the first-order correction of
      // the normalisers' ratio (see correct_steps) from its signed sum
      CheapSums c{0.0f, 0.0f, 0.0f};
      if (have) c = cheap_sums8(xt, xd, P);
      const double cm = wave_sum((double)c.r), cq = wave_sum((double)c.q);
      cheap = cheap_ok(cm, cq);
      double d;
      if (cheap) {
        d = wave_sum((double)c.d);
      } else {
        d = 0.0;
        if (have) {
          ResidSums o = resid_sums8<false>(xt, xd, P);
          if (!(o.a == o.a)) o = resid_sums8<true>(xt, xd, P);
          d = 2.0 * (double)o.r - (double)o.a;
        }
        d = wave_sum(d);
      }
      Pd.g = d / (P.sp * P.fscale - d);
    }
    double total = step_total(mode, Pd);  // the corrected terms, the same ones the scan takes
    if (!(total > 0.0) && mode == kModeResidual) {
      // nothing left after the rejection (p_n == q_n up to rounding): draw from p_n
      mode = kModeBonus;
      Pd.g = 0.0;
      cheap = false;
      total = step_total(mode, Pd);
    }
    const int y = scan_step<1>(rr, 0, (double)P.ug * total, 0.0, lane);
    write_outputs<TD>(A, b, Pd, mode, y, total, lane, xi);
  } else {
    SeqPlan Pd = P;
    double total;
    bool cheap = false;
    if (mode == kModeResidual && P.form == 1) {
      // the first-order correction of the normalisers' ratio (see correct_steps)
      const StepSums v = direct_step_sums<TD, DD, kModeResidual, 1>(trow, drow, 0, noct, A.V, P, lane);
      Pd.g = v.d / (P.sp * P.fscale - v.d);
      total = fmax(v.m - Pd.g * v.q, 0.0);
      cheap = v.c > 0.5;
    } else {
      total = direct_step_sums_of<TD, DD>(trow, drow, 0, noct, A.V, mode, P, lane).m;
    }
    if (!(total > 0.0) && mode == kModeResidual) {
      // nothing left after the rejection (p_n == q_n up to rounding): draw from p_n
      mode = kModeBonus;
      Pd.g = 0.0;
      total = direct_step_sums_of<TD, DD>(trow, drow, 0, noct, A.V, mode, P, lane).m;
      cheap = false;
    }
    const double t = (double)P.ug * total;
    const int y = rescan_step<TD, DD>(A, b, Pd, mode, 0, t, 0.0, lane, cheap);
    write_outputs<TD>(A, b, Pd, mode, y, total, lane, xi);
  }
}

// ---------------------------------------------------------------------------
// tiny vocabularies (V <= 32, 2 gamma + 1 <= 32): two sequences per wave
// ---------------------------------------------------------------------------
// Half-wave reductions: the wave reductions' DPP butterfly within 16-lane
// rows, then rows 0 + 1 (lanes 0-31) and rows 2 + 3 (lanes 32-63) combined
// apart. For a half whose other lanes hold nothing (-inf, 0) these are the
// wave reductions' results bit for bit.
__device__ __forceinline__ float half_max(float v, bool upper) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  const float lo = fmaxf(readlane_f32(v, 0), readlane_f32(v, 16));
  const float hi = fmaxf(readlane_f32(v, 32), readlane_f32(v, 48));
  return upper ? hi : lo;
}
__device__ __forceinline__ double half_sum(double v, bool upper) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppRowRor4>(v);
  v += dpp_f64<kDppRowRor8>(v);
  const double lo = readlane_f64(v, 0) + readlane_f64(v, 16);
  const double hi = readlane_f64(v, 32) + readlane_f64(v, 48);
  return upper ? hi : lo;
}
// Inclusive prefix sum within each half (the wave scan without its step
// from lane 31 into the upper half).
__device__ __forceinline__ double half_incl_scan(double v) {
  v += dpp_f64_masked<kDppRowShr1, 0xf>(v);
  v += dpp_f64_masked<kDppRowShr2, 0xf>(v);
  v += dpp_f64_masked<kDppRowShr4, 0xf>(v);
  v += dpp_f64_masked<kDppRowShr8, 0xf>(v);
  v += dpp_f64_masked<kDppRowBcast15, 0xa>(v);
  return v;
}

// The whole verify of sequences with V <= 32 and 2 gamma + 1 <= 32 rows, two
// per wave: lanes 0-31 take sequence 2 k, lanes 32-63 sequence 2 k + 1 (k the
// wave's index in the grid), half-lane h holding token h of every row and
// row slot h's statistics. The steps and their order are those of the
// one-wave kernel (whose rows of at most 32 tokens leave its upper half
// empty); every wave operation runs with the whole wave active, each half
// taking its own results, and a half past the batch computes on the last
// sequence's rows and writes nothing.
template <int TD, int DD>
__global__ __launch_bounds__(kThreads) void sv_small2_kernel(SampleLaunch A) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool upper = lane >= 32;
  const int hl = lane & 31, base = upper ? 32 : 0;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b0 = (blockIdx.x * kWaves + w) * 2;
  if (b0 >= A.B) return;  // the whole wave; this kernel has no workgroup barrier
  const int b = b0 + (upper ? 1 : 0);
  const bool active = b < A.B;
  const int bl = active ? b : A.B - 1;  // rows read by a half past the batch
  const float T = A.temps[bl];
  const bool tv = temp_ok(T);
  const float kl = tv ? log2e_over(T) : 1.0f;
  const int G = A.gamma;

  // the draft tokens, their uniforms and logits (position = half-lane)
  int xi = 0;
  float ui = 0.0f, lt = 0.0f, ld = 0.0f;
  bool tok_ok = false;
  if (hl < G) {
    xi = A.tokens[(int64_t)bl * G + hl];
    ui = A.uniforms[(int64_t)bl * (G + 1) + hl];
    tok_ok = xi >= 0 && xi < A.V;
    if (tok_ok) {
      lt = load_elem<TD>(A.tgt + (int64_t)bl * A.t_seq_b + (int64_t)hl * A.t_row_b, xi);
      ld = load_elem<DD>(A.dft + (int64_t)bl * A.d_seq_b + (int64_t)hl * A.d_row_b, xi);
    }
  }
  // statistics of target rows 0..G (slots 0..G) and draft rows 0..G-1 (slots
  // G+1..2G <= 30); slot t is kept by half-lane t
  constexpr int RB = 16;
  float m0 = 0.0f;
  double s0 = 0.0;
  int v0 = 0;
  for (int t0 = 0; t0 <= 2 * G; t0 += RB) {
    float x[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + r;
      const char* row = (t <= G) ? A.tgt + (int64_t)bl * A.t_seq_b + (int64_t)t * A.t_row_b
                                 : A.dft + (int64_t)bl * A.d_seq_b + (int64_t)(t - G - 1) * A.d_row_b;
      x[r] = -INFINITY;
      if (t <= 2 * G && hl < A.V) x[r] = (t <= G) ? load_elem<TD>(row, hl) : load_elem<DD>(row, hl);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + r;
      if (t > 2 * G) break;
      // the one-wave kernel's row statistics (reference: the row's maximum)
      const float m = half_max(x[r], upper);
      const bool nan = x[r] != x[r];
      double e = 0.0;
      if (nan || x[r] != -INFINITY) e = nan ? (double)x[r] : (double)hw_exp2((x[r] - m) * kl);
      const double sm = half_sum(e, upper);
      if (hl == t) {
        m0 = m;
        s0 = sm;
        v0 = tv && __builtin_isfinite(sm) && sm > 0.0 && __builtin_isfinite(m);
      }
    }
  }
  auto stat_of = [&](int t) {  // slot t of this half's sequence, in every lane of the half
    const float m = __shfl(m0, base + t, kWave);
    const double sm = __shfl(s0, base + t, kWave);
    const int v = __shfl(v0, base + t, kWave);
    return RowStat{(double)m * (double)kl, m, sm, v};
  };
  // accept tests (half-lane i: position i) and the first stop
  const RowStat ds = stat_of(G + 1 + hl < 32 ? G + 1 + hl : 31);
  int code = 1;
  if (hl < G) {
    const RowStat ts{(double)m0 * (double)kl, m0, s0, v0};
    const AcceptOut ao = accept_test(lt, ld, ts, ds, kl, ui, tok_ok, tv, A.diag_px || A.diag_qx);
    code = ao.code;
    if (active && A.diag_px) A.diag_px[(int64_t)b * G + hl] = ao.px;
    if (active && A.diag_qx) A.diag_qx[(int64_t)b * G + hl] = ao.qx;
  }
  const unsigned long long stopw = __ballot(code != 1);
  const unsigned stop = upper ? (unsigned)(stopw >> 32) : (unsigned)stopw;
  const int n = stop ? (__ffs(stop) - 1) : G;
  const int code_n = __shfl(code, base + (n < G ? n : 0), kWave);
  const RowStat tn = stat_of(n);
  const RowStat dq = stat_of(n < G ? G + 1 + n : 0);
  const RowStat dn = (n < G) ? dq : RowStat{0.0, 0.0f, 1.0, 0};
  const SeqPlan P = make_plan(n, code_n, G, G + 1, tv, kl, A.uniforms[(int64_t)bl * (G + 1) + G], tn, dn);

  // the draw row(s): at most 4 octets, one per half-lane
  const char* trow = A.tgt + (int64_t)bl * A.t_seq_b + (int64_t)n * A.t_row_b;
  const char* drow = (n < G) ? A.dft + (int64_t)bl * A.d_seq_b + (int64_t)n * A.d_row_b : nullptr;
  const int noct = (A.V + 7) / 8;
  int mode = P.mode;
  const bool have = hl < noct;
  float xt[8], xd[8], rr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) xd[k] = 0.0f;
  if (have) {
    load_octet<TD>(trow, hl, A.V, xt);
    if (mode == kModeResidual) load_octet<DD>(drow, hl, A.V, xd);
  }
  bool cheap = false;
  auto step_total = [&](int m, const SeqPlan& Q) -> double {
    double lacc = 0.0;
    if (have) {
      mass8_of(xt, xd, m, Q, rr, cheap);
      lacc = (double)sum8(rr);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) rr[k] = 0.0f;
    }
    return half_sum(lacc, upper);
  };
  SeqPlan Pd = P;
  // the step's form (see cheap_ok), then the first-order correction of the
  // normalisers' ratio (see correct_steps) from its signed sum
  const bool rform = mode == kModeResidual && P.form == 1;
  CheapSums c{0.0f, 0.0f, 0.0f};
  if (have && rform) c = cheap_sums8(xt, xd, P);
  const double cm = half_sum((double)c.r, upper), cq = half_sum((double)c.q, upper);
  const double cd = half_sum((double)c.d, upper);
  cheap = rform && cheap_ok(cm, cq);
  const bool exact = rform && !cheap;
  double d = cd;
  if (__ballot(exact)) {
    double de = 0.0;
    if (have && exact) {
      ResidSums o = resid_sums8<false>(xt, xd, P);
      if (!(o.a == o.a)) o = resid_sums8<true>(xt, xd, P);
      de = 2.0 * (double)o.r - (double)o.a;
    }
    de = half_sum(de, upper);
    if (exact) d = de;
  }
  if (rform) Pd.g = d / (P.sp * P.fscale - d);
  double total = step_total(mode, Pd);  // the corrected terms, the same ones the scan takes
  const bool fb = !(total > 0.0) && mode == kModeResidual;
  if (__ballot(fb)) {
    // nothing left after the rejection (p_n == q_n up to rounding): draw from p_n
    if (fb) {
      mode = kModeBonus;
      Pd.g = 0.0;
      cheap = false;
    }
    const double t2 = step_total(mode, Pd);  // the other half's terms come out unchanged
    if (fb) total = t2;
  }
  // the scan of the step (the one-wave scan within the half)
  const double t = (double)P.ug * total;
  const double os = (double)sum8(rr);
  const double incl = half_incl_scan(os);
  const double excl = incl - os;
  int lk = -1;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (rr[k] > 0.0f) lk = k;
  const unsigned long long hitw = __ballot(os > 0.0 && incl > t);
  const unsigned hit = upper ? (unsigned)(hitw >> 32) : (unsigned)hitw;
  const int L = hit ? (__ffs(hit) - 1) : 0;
  int yy = -1;
  if (hit && hl == L) {
    double run = excl;
    for (int k = 0; k < 8; ++k) {
      if (rr[k] > 0.0f) {
        run += (double)rr[k];
        if (run > t) {
          yy = hl * 8 + k;
          break;
        }
      }
    }
    if (yy < 0) yy = hl * 8 + lk;
  }
  int y = __shfl(yy, base + L, kWave);
  // rounding pushed t past the step's mass: its last positive token
  int lp = lk >= 0 ? hl * 8 + lk : -1;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o, kWave));
  if (!hit) y = lp;
  if (!active) return;
  if (!P.valid)
    write_invalid(A, b, hl, 0, 32);
  else
    write_outputs<TD>(A, b, Pd, mode, y, total, hl, xi);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// The finish keeps each wave's step in registers (OS) unless both rows are
// fp32: their 64 bytes per octet pair would not fit beside the kernel's
// other registers (measured: 64 VGPRs spilled).
template <int TD, int DD>
constexpr bool kKeepSteps = TD == 1 || DD == 1;

template <int TD, int DD>
static hipError_t launch_pair(const SampleLaunch& A, int stage, hipStream_t stream) {
  if (stage == 1)
    hipLaunchKernelGGL((sv_stats_kernel<TD, DD>), dim3((unsigned)((int64_t)A.B * A.per_seq)), dim3(kThreads), 0,
                       stream, A);
  else if (stage == 3)
    hipLaunchKernelGGL((sv_read_kernel<TD, DD>), dim3((unsigned)((int64_t)A.B * A.per_seq)), dim3(kThreads), 0,
                       stream, A);
  else if (kKeepSteps<TD, DD> && A.fin_waves == 2 * kFinWaves && A.parts == 1 && A.ns2 <= 2 * kFinWaves)
    hipLaunchKernelGGL((sv_finish_kernel<TD, DD, 2 * kFinWaves, kKeepSteps<TD, DD>>), dim3((unsigned)A.B),
                       dim3(2 * kFinThreads), 0, stream, A);
  else if (A.fin_waves == 2 * kFinWaves)
    hipLaunchKernelGGL((sv_finish_kernel<TD, DD, 2 * kFinWaves, false>), dim3((unsigned)((int64_t)A.B * A.parts)),
                       dim3(2 * kFinThreads), 0, stream, A);
  else if (kKeepSteps<TD, DD> && A.parts == 1 && A.ns2 <= kFinWaves)
    hipLaunchKernelGGL((sv_finish_kernel<TD, DD, kFinWaves, kKeepSteps<TD, DD>>), dim3((unsigned)A.B),
                       dim3(kFinThreads), 0, stream, A);
  else
    hipLaunchKernelGGL((sv_finish_kernel<TD, DD, kFinWaves, false>), dim3((unsigned)((int64_t)A.B * A.parts)),
                       dim3(kFinThreads), 0, stream, A);
  return hipGetLastError();
}

template <int TD, int DD>
static hipError_t launch_pos(const SampleLaunch& A, int p0, int p1, hipStream_t stream) {
  const int64_t cps = early_chunks(A.gamma, A.nct, A.ncd, p0, p1);
  hipLaunchKernelGGL((sv_stats_pos_kernel<TD, DD>), dim3((unsigned)((int64_t)A.B * cps)), dim3(kThreads), 0, stream,
                     A, p0, p1);
  return hipGetLastError();
}

hipError_t launch_sample_stage(const SampleLaunch& A, int tdt, int ddt, int stage, hipStream_t stream) {
  if (tdt == 1 && ddt == 1) return launch_pair<1, 1>(A, stage, stream);
  if (tdt == 1 && ddt == 0) return launch_pair<1, 0>(A, stage, stream);
  if (tdt == 0 && ddt == 1) return launch_pair<0, 1>(A, stage, stream);
  return launch_pair<0, 0>(A, stage, stream);
}

template <int TD, int DD>
static hipError_t launch_small_t(const SampleLaunch& A, hipStream_t stream) {
  const dim3 grid((unsigned)(((int64_t)A.B + kWaves - 1) / kWaves));
  if (A.V <= 32 && 2 * A.gamma + 1 <= 32)
    hipLaunchKernelGGL((sv_small2_kernel<TD, DD>), dim3((unsigned)(((int64_t)A.B + 2 * kWaves - 1) / (2 * kWaves))),
                       dim3(kThreads), 0, stream, A);
  else if (A.V <= kWave)
    hipLaunchKernelGGL((sv_small_kernel<TD, DD, 1>), grid, dim3(kThreads), 0, stream, A);
  else if (A.V <= 4 * kWave)
    hipLaunchKernelGGL((sv_small_kernel<TD, DD, 4>), grid, dim3(kThreads), 0, stream, A);
  else
    hipLaunchKernelGGL((sv_small_kernel<TD, DD, kStepTokens / kWave>), grid, dim3(kThreads), 0, stream, A);
  return hipGetLastError();
}

hipError_t launch_sample_small(const SampleLaunch& A, int tdt, int ddt, hipStream_t stream) {
  if (tdt == 1 && ddt == 1) return launch_small_t<1, 1>(A, stream);
  if (tdt == 1 && ddt == 0) return launch_small_t<1, 0>(A, stream);
  if (tdt == 0 && ddt == 1) return launch_small_t<0, 1>(A, stream);
  return launch_small_t<0, 0>(A, stream);
}

hipError_t launch_draft_one_pass(const SampleLaunch& A, int dt, hipStream_t stream) {
  const bool wide = A.B <= kDraftWideRows;
  if (dt == 1 && wide)
    hipLaunchKernelGGL((sv_draft1_kernel<1, 16>), dim3((unsigned)A.B), dim3(16 * kWave), 0, stream, A);
  else if (dt == 1)
    hipLaunchKernelGGL((sv_draft1_kernel<1, 8>), dim3((unsigned)A.B), dim3(8 * kWave), 0, stream, A);
  else if (wide)
    hipLaunchKernelGGL((sv_draft1_kernel<0, 16>), dim3((unsigned)A.B), dim3(16 * kWave), 0, stream, A);
  else
    hipLaunchKernelGGL((sv_draft1_kernel<0, 8>), dim3((unsigned)A.B), dim3(8 * kWave), 0, stream, A);
  return hipGetLastError();
}

hipError_t launch_sample_pos(const SampleLaunch& A, int tdt, int ddt, int p0, int p1, hipStream_t stream) {
  if (tdt == 1 && ddt == 1) return launch_pos<1, 1>(A, p0, p1, stream);
  if (tdt == 1 && ddt == 0) return launch_pos<1, 0>(A, p0, p1, stream);
  if (tdt == 0 && ddt == 1) return launch_pos<0, 1>(A, p0, p1, stream);
  return launch_pos<0, 0>(A, p0, p1, stream);
}

}  // namespace sv
