// sv_plan.hpp -- launch descriptors, workspace records and work decomposition
// shared by the host library and the kernels of libspec_verify.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;  // streaming workgroups: 4 wave64
constexpr int kWaves = 4;
constexpr int kFinThreads = 512;  // per-sequence finish workgroup: 8 wave64
constexpr int kFinWaves = 8;
constexpr int kWave = 64;
constexpr int kU1 = 4;                          // 16-byte units per lane per iteration (stats, argmax)
constexpr int kU2 = 4;                          // 8-token octets per lane per residual step
constexpr int kStepOctets = kWave * kU2;        // 256 octets = 2048 tokens per residual step (one wave)
constexpr int kStepTokens = kStepOctets * 8;
constexpr int kLdsSteps = 2048;                 // step masses kept in LDS up to this many steps (V <= 4.19M)
constexpr int64_t kMinChunkBytes = 16 << 10;    // stats / argmax work unit bounds
constexpr int64_t kMaxChunkBytes = 256 << 10;   // measured best for the stats kernel on MI355X (128/256/512 KB)
constexpr int64_t kTargetWGs = 8192;            // ~32 workgroups per CU on 256 CUs
constexpr int kLog2MaxNodes = 10;               // 1024 tree nodes
constexpr int64_t kEarlyChunkBytes = 128 << 10;  // early-exit statistics work unit
constexpr double kEarlyAlpha = 0.7;             // acceptance rate assumed when grouping positions
constexpr double kEarlyLaunchBytes = 64e6;      // bytes moved in about the time one extra launch costs
constexpr int64_t kFinTargetWGs = 256;          // finish: split sequences over parts up to one workgroup per CU
constexpr int64_t kBatchUnits = (int64_t)kThreads * kU1;  // 1024 units = 16 KB: one batch of every thread

enum : int { kModeResidual = 0, kModeBonus = 1 };

// Partial statistics of one wave's share of one chunk of one logits row
// (stats pass):
//   form 1: s = sum of exp2(x * kl - m), where m is an integer number of log2
//           units (a float holding an integer, |m| < 2^24, or -inf when every
//           value was -inf); every term of every batch was taken against an
//           integer shift at or just above that batch's maximum and moved to m
//           by an exact power of two;
//   form 0: s = sum of exp2((x - m) * kl) against a reference logit m (used
//           when a shift would reach 2^24: tiny temperatures or huge logits).
struct RowPartial {
  float m;
  int form;
  double s;
};

// The finish kernel's per-sequence plan for the draw (held in LDS).
//
// Row statistics: p_v = exp2(x_t,v * kl - ct) / sp over target row n and
// q_v = exp2(x_d,v * kl - cd) / sq over draft row n (ct, cd in log2 units,
// fp64). Mass of token v of the drawn distribution, up to one positive factor
// F * sp per sequence:
//  form 1 (shifts folded into one FMA each):
//    e_p = exp2(fma(x_t, kl, -cp)) with cp = fp32(ct) (exact when ct is an
//    integer), F = exp2(ct - cp) (fscale); r = e_p = F sp p_v for the bonus row.
//    After a rejection: w = fma(x_d - x_t, kl, dt) = log2(q_v / p_v) with
//    dt = cp - cqx, cqx = cd - log2(sp / sq) - (ct - cp) (e_q = F sp q_v =
//    exp2(x_d * kl - cqx)); e = e_p where w <= 0, else e_q, taken as
//    exp2(e_p's exponent + w) (as exp2(fma(x_d, kl, -cq) - cq_lo), cq + cq_lo
//    = cqx, where the target logit is -inf); |e_p - e_q| = -e * expm1_2(-|w|),
//    exact to a few ulp however close p and q are, and r = that where p >= q,
//    less g * e_q, g the first-order correction of the normalisers' ratio from
//    the signed sum of e_p - e_q over the row. r = F sp * max(0, p - q).
//    A 2048-token step whose positive residual is not small next to its
//    q-mass takes the cheap form instead: e_p = exp2(fma(x_t, kl, -cp)) and
//    e_q = cq_s * exp2(fma(x_d, kl, -cq)), one exponential each, the token's
//    residual t = e_p - e_q where t > 0 (see cheap_ok in sv_sample.hip).
//  form 0 (used when a shift is 2^24 or more in magnitude, where its fp32
//  rounding would be half a log2 unit or more):
//    e_p = exp2((x_t - mp) * kl), e_q = exp2((x_d - mq) * kl),
//    r = max(0, e_p - kappa e_q) with kappa as a float pair, F = exp2(ct - mp * kl).
struct SeqPlan {
  int valid;   // 0: the sequence is invalid (all outputs -1)
  int n;       // accepted drafts
  int mode;    // kModeResidual (row n pair) or kModeBonus (target row n == gamma)
  int form;    // 1: FMA shifts, 0: subtract-multiply
  float kl;    // log2(e) / T, fp32
  float mp;    // form 0: reference logit of target row n
  float mq;    // form 0: reference logit of draft row n
  float kap_hi;  // form 0: kappa (F * sp) / (F_q * sq) as a float pair (hi + lo)
  float kap_lo;
  float cp, cq;
  float cq_lo;    // cqx - cq
  float cq_s;     // 2^(cq - cqx), fp32: the cheap form's factor of e_q
  float dt;       // fp32(cp - cqx): log2(q_v / p_v) - (x_d - x_t) * kl
  float ug;       // the draw's uniform
  double ct;      // shift of target row n (log2 units)
  double sp;      // sum_v exp2(x_v * kl - ct) over target row n
  double sq;      // sum_v exp2(x_v * kl - cd) over draft row n
  double fscale;  // F
  double g;       // exact pass: first-order correction factor (0 otherwise)
};

// Partial argmax of one wave's share of one chunk of one row (tree pass).
struct ArgPartial {
  float best;
  int idx;
  int bad;  // NaN seen
  int pad;
};

struct SampleLaunch {
  const char* tgt;
  int64_t t_seq_b, t_row_b;  // strides in bytes
  const char* dft;
  int64_t d_seq_b, d_row_b;
  const int32_t* tokens;
  const float* uniforms;
  const float* temps;
  int B, gamma, V;
  int32_t* out_n;    // may be null (draft sampler)
  int32_t* out_tok;
  float* out_py;     // may be null: probability of the drawn token (bonus-mode draws; draft sampler)
  float* diag_px;
  float* diag_qx;
  float* diag_mass;
  // stats pass decomposition
  int nct, ncd;  // chunks per target row / per draft row
  int cut, cud;  // 16-byte units per chunk (multiples of 256)
  int per_seq;   // (gamma + 1) * nct + gamma * ncd
  int ns2;  // 2048-token steps per row (draw)
  int parts;  // finish workgroups per sequence, each streaming a share of the draw's steps
  int fin_waves;  // waves per finish workgroup: kFinWaves, or 2 * kFinWaves for split sequences
  // workspace
  RowPartial* part;  // [B][per_seq][kWaves]
  double* steptot;   // [B][4][ns2] step sums (masses, q-masses, signed sums, form flags) when they exceed
                     // LDS, and the finish parts' hand-off (sentinels -1, -1, NaN, -1 before each finish
                     // launch when parts > 1)
  int32_t* reach;    // [B] early exit only (else null): rows 0..reach-1 have statistics
  int32_t* done;     // [B] finish parts done; zeroed by the statistics pass and by the drawing part
};

struct TreeLaunch {
  const char* logits;
  int64_t seq_b, row_b;
  const int32_t* parents;
  const int32_t* tokens;
  int B, N, V;
  int nch;  // chunks per row
  int cu;   // 16-byte units per chunk (multiple of 256)
  int32_t* out_len;
  int32_t* out_path;
  int32_t* out_bonus;
  int32_t* out_argmax;
  ArgPartial* part;  // [B][N][nch]
};

constexpr int kMaxMaskNodes = 1024;  // tree masks: nodes per tree
constexpr int kMaskJumpLevels = 4;   // tree masks: up to 2^4 threads walk each row
constexpr int64_t kMaskSlabBytes = 16 << 10;  // tree masks: mask bytes per workgroup (measured: 16 KB beat 8, 32 and 64 KB)

struct MaskLaunch {
  const int32_t* parents;  // [B][N]
  const int32_t* blocks;   // [B][N] or null
  int B, N;
  int nslab, rows_per_slab;
  uint8_t* out_mask;     // [B][N][N] or null
  uint8_t* out_relaxed;  // [B][N][N] or null
  int32_t* out_depth;    // [B][N] or null
};

// ---------------------------------------------------------------------------
// host-side decomposition helpers (pure integer arithmetic)
// ---------------------------------------------------------------------------
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Bytes of work per stats/argmax workgroup for a call that streams total_bytes.
// A multiple of 16 KB (one batch of 4 units of every thread), so that every
// chunk starts on a batch boundary of its row: the statistics pass then forms
// the same batches, with the same fp32 arithmetic, whatever the chunking (and
// so whatever the batch size of the call).
inline int64_t chunk_bytes_for(int64_t total_bytes) {
  int64_t c = clamp64(total_bytes / kTargetWGs, kMinChunkBytes, kMaxChunkBytes);
  return round_up(c, kBatchUnits * 16);
}

// Work unit of the tree's argmax kernel: the same rule with its own lower bound.
constexpr int64_t kTreeMinChunkBytes = 16 << 10;
inline int64_t tree_chunk_bytes_for(int64_t total_bytes) {
  int64_t c = clamp64(total_bytes / kTargetWGs, kTreeMinChunkBytes, kMaxChunkBytes);
  return round_up(c, (int64_t)kThreads * 16);
}

// Split a row of V elements of esz bytes into nch chunks of cu 16-byte units,
// cu a multiple of `align` units (chunk_bytes is a multiple of align * 16).
inline void split_row(int64_t V, int esz, int64_t chunk_bytes, int* nch, int* cu, int64_t align = kThreads) {
  int64_t nu = ceil_div(V * esz, 16);
  int64_t per = chunk_bytes / 16;
  int64_t n = ceil_div(nu, per);
  int64_t c = round_up(ceil_div(nu, n), align);
  *nch = (int)ceil_div(nu, c);
  *cu = (int)c;
}

// Upper bound of chunks per row for any dtype (used to size the workspace).
inline int64_t max_chunks_per_row(int64_t V) { return ceil_div(V * 4, kMinChunkBytes); }

inline int64_t align256(int64_t x) { return round_up(x, 256); }

struct SampleLayout {
  int64_t off_part, off_step, off_reach, off_done, total;
};

inline int64_t draw_steps(int64_t V) { return ceil_div(V, kStepTokens); }

// Finish workgroups per sequence. With fewer sequences than CUs, one
// workgroup per sequence leaves most of the GPU idle while each streams its
// draw row(s) alone (a 256k-token residual pair is 1.5 MB), so each sequence's
// steps are split over up to kFinTargetWGs / B parts, at least one step per
// wave each. Every part repeats the (small) merge and accept tests; the part
// that finishes last gathers the step masses into its LDS and draws, so only
// rows whose steps fit in LDS are split. With B at or above the CU count one
// part per sequence is faster (measured: the repeated merges cost more than
// the balance gains).
inline int finish_parts(int64_t B, int64_t ns2) {
  if (ns2 > kLdsSteps) return 1;
  int64_t k = ceil_div(kFinTargetWGs, B);
  const int64_t cap = ns2 / kFinWaves;
  if (k > cap) k = cap;
  return (int)(k < 1 ? 1 : k);
}

// Waves per finish workgroup and parts per sequence. A sequence split into K
// parts of kFinWaves waves whose waves stream at most two steps each runs as
// ceil(K / 2) parts of 2 * kFinWaves waves instead: the same waves (or one
// part's more) with half the repeated merges and accept tests, and no hand-off
// at all for K = 2; its stream is one or two round trips per wave either way
// (measured: 64 sequences of 32k bf16 tokens, gamma 4: 0.0298 -> 0.0287 ms; a
// single 128k or 256k sequence 0.0220 -> 0.0209 and 0.0255 -> 0.0248 ms). With longer streams the workgroups' CUs
// bound the stream, and halving them costs more (64 sequences of 256k: 0.117
// -> 0.127 ms), so they keep kFinWaves.
inline void finish_shape(int64_t B, int64_t ns2, int* parts, int* waves) {
  const int k = finish_parts(B, ns2);
  const bool wide = k >= 2 && ns2 <= (int64_t)2 * k * kFinWaves;
  *waves = wide ? 2 * kFinWaves : kFinWaves;
  *parts = wide ? (k + 1) / 2 : k;
}

// Draft sampler: the one-pass kernel (one workgroup per row) when the row's
// step masses fit its LDS and there are enough rows to fill the GPU (or the
// rows are short enough that two launches would cost more than the pass).
constexpr int64_t kOnePassMinRows = 128;
constexpr int64_t kDraftWideRows = 256;  // one-pass sampler: 16-wave workgroups up to this many rows
constexpr int64_t kOnePassShortRowBytes = 64 << 10;
inline bool draft_one_pass(int64_t B, int64_t V, int esz) {
  return draw_steps(V) <= kLdsSteps && (B >= kOnePassMinRows || V * esz <= kOnePassShortRowBytes);
}

// ---------------------------------------------------------------------------
// early exit
// ---------------------------------------------------------------------------
// Chunks per sequence of one launch over positions p0..p1 (target rows, and
// draft rows of the positions below gamma).
inline int64_t early_chunks(int64_t G, int64_t nct, int64_t ncd, int64_t p0, int64_t p1) {
  const int64_t hi = p1 < G - 1 ? p1 : G - 1;
  const int64_t npair = hi >= p0 ? hi - p0 + 1 : 0;
  return npair * (nct + ncd) + (p1 == G ? nct : 0);
}

// Work unit of the early-exit statistics launches. Smaller than the one-pass
// kernel's largest: a launch over the later positions holds few active
// sequences, and its time is then one workgroup's chain of dependent loads.
// Not much smaller: every workgroup of a gated launch first re-derives an
// accept decision (a few dependent round trips), which a small unit does not
// amortise (measured on MI355X at V = 128k: 64 KB beat 16 and 32 KB by
// 20-30%, 128 KB beat 64 KB by 4% and 256 KB by 20%; at V = 256k 64 and
// 128 KB matched).
inline int64_t early_chunk_bytes() { return kEarlyChunkBytes; }

// First position of the tail group: positions 0..k-1 get a launch each and
// k..gamma share one. Position p gets its own launch while the bytes that its
// gate is expected to save -- sequences still active at p (alpha^p) that
// reject there (1 - alpha) skip the rows of p+1..gamma -- exceed what a launch
// costs in time (kEarlyLaunchBytes at full bandwidth). alpha is an assumed
// acceptance rate, not measured. k = 0 (small batches) is one launch over
// every row, with no gate.
inline int early_tail_start(int64_t B, int64_t G, int64_t V, int et, int ed) {
  const double pair = (double)B * V * (et + ed), bonus = (double)B * V * et;
  double active = 1.0;
  for (int64_t p = 0; p < G; ++p) {
    const double later = (double)(G - p - 1) * pair + bonus;
    if (active * (1.0 - kEarlyAlpha) * later < kEarlyLaunchBytes) return (int)p;
    active *= kEarlyAlpha;
  }
  return (int)G;
}

inline SampleLayout sample_layout(int64_t B, int64_t gamma, int64_t V) {
  SampleLayout L;
  int64_t o = 0;
  L.off_part = o;
  o += align256(B * (2 * gamma + 1) * max_chunks_per_row(V) * kWaves * (int64_t)sizeof(RowPartial));
  L.off_step = o;
  o += align256(B * 4 * draw_steps(V) * 8);
  L.off_reach = o;
  o += align256(B * 4);
  L.off_done = o;
  o += align256(B * 4);
  L.total = o;
  return L;
}

struct TreeLayout {
  int64_t off_part, total;
};

inline TreeLayout tree_layout(int64_t B, int64_t N, int64_t V) {
  TreeLayout L;
  int64_t o = 0;
  L.off_part = o;
  o += align256(B * N * max_chunks_per_row(V) * (int64_t)sizeof(ArgPartial));
  L.total = o;
  return L;
}

}  // namespace sv
