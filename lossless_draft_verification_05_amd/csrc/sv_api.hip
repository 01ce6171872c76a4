// sv_api.hip -- the C ABI of libspec_verify: argument checks on the host, work
// decomposition, workspace layout and kernel launches. Every argument error is
// returned before the first HIP call.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/spec_verify.h"
#include "sv_plan.hpp"

namespace sv {
hipError_t launch_sample_stage(const SampleLaunch& A, int tdt, int ddt, int stage, hipStream_t stream);
hipError_t launch_sample_pos(const SampleLaunch& A, int tdt, int ddt, int p0, int p1, hipStream_t stream);
hipError_t launch_draft_one_pass(const SampleLaunch& A, int dt, hipStream_t stream);
hipError_t launch_sample_small(const SampleLaunch& A, int tdt, int ddt, hipStream_t stream);
hipError_t launch_tree(const TreeLaunch& A, int dt, int stage, hipStream_t stream);
hipError_t launch_mask(const MaskLaunch& A, hipStream_t stream);

static thread_local int g_last_hip_error = 0;

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return SV_OK;
  g_last_hip_error = (int)e;
  return SV_ERR_HIP;
}

static inline int esz_of(int dt) { return dt == SV_BF16 ? 2 : 4; }
static inline bool dtype_ok(int dt) { return dt == SV_F32 || dt == SV_BF16; }
static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Largest byte offset touched by a [B][rows][V] view, or -1 on overflow.
static int64_t extent_bytes(int64_t B, int64_t rows, int64_t V, int64_t seq_stride, int64_t row_stride, int esz) {
  const int64_t lim = INT64_MAX / 8;
  if (seq_stride > lim / (B > 0 ? B : 1) || row_stride > lim / (rows > 0 ? rows : 1)) return -1;
  int64_t e = (B - 1) * seq_stride + (rows - 1) * row_stride + V;
  if (e > lim / esz) return -1;
  return e * esz;
}

static int check_rows(const void* base, int dt, int64_t seq_stride, int64_t row_stride, int64_t B, int64_t rows,
                      int64_t V) {
  if (!dtype_ok(dt)) return SV_ERR_DTYPE;
  if (row_stride < V || seq_stride < 0) return SV_ERR_SHAPE;
  const int esz = esz_of(dt);
  if (extent_bytes(B, rows, V, seq_stride, row_stride, esz) < 0) return SV_ERR_SHAPE;
  if (!aligned(base, 16) || (row_stride * esz) % 16 != 0 || (seq_stride * esz) % 16 != 0) return SV_ERR_ALIGN;
  return SV_OK;
}

struct SampleArgs {
  const void* tgt;
  int tdt;
  int64_t tss, trs;
  const void* dft;
  int ddt;
  int64_t dss, drs;
  const int32_t* tokens;
  const float* uniforms;
  const float* temps;
  int B, gamma, V;
  int32_t* out_n;
  int32_t* out_tok;
  const sv_sample_diag* diag;
  void* ws;
  size_t ws_bytes;
};

static int validate_sample(const SampleArgs& a) {
  if (!a.tgt || !a.dft || !a.tokens || !a.uniforms || !a.temps || !a.out_n || !a.out_tok) return SV_ERR_NULL;
  if (!dtype_ok(a.tdt) || !dtype_ok(a.ddt)) return SV_ERR_DTYPE;
  if (a.B < 1 || a.B > SV_MAX_BATCH || a.gamma < 1 || a.gamma > SV_MAX_GAMMA || a.V < 1 || a.V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  int st = check_rows(a.tgt, a.tdt, a.tss, a.trs, a.B, a.gamma + 1, a.V);
  if (st) return st;
  st = check_rows(a.dft, a.ddt, a.dss, a.drs, a.B, a.gamma, a.V);
  if (st) return st;
  if (!aligned(a.tokens, 4) || !aligned(a.uniforms, 4) || !aligned(a.temps, 4) || !aligned(a.out_n, 4) ||
      !aligned(a.out_tok, 4))
    return SV_ERR_ALIGN;
  if (a.diag && ((a.diag->p_x && !aligned(a.diag->p_x, 4)) || (a.diag->q_x && !aligned(a.diag->q_x, 4)) ||
                 (a.diag->resid_mass && !aligned(a.diag->resid_mass, 4))))
    return SV_ERR_ALIGN;
  if (!a.ws) return SV_ERR_WORKSPACE;
  if (!aligned(a.ws, 256)) return SV_ERR_ALIGN;
  if (a.ws_bytes < (size_t)sample_layout(a.B, a.gamma, a.V).total) return SV_ERR_WORKSPACE;
  return SV_OK;
}

static SampleLaunch plan_sample(const SampleArgs& a, bool early = false) {
  SampleLaunch L;
  memset(&L, 0, sizeof(L));
  const int et = esz_of(a.tdt), ed = esz_of(a.ddt);
  L.tgt = (const char*)a.tgt;
  L.t_seq_b = a.tss * et;
  L.t_row_b = a.trs * et;
  L.dft = (const char*)a.dft;
  L.d_seq_b = a.dss * ed;
  L.d_row_b = a.drs * ed;
  L.tokens = a.tokens;
  L.uniforms = a.uniforms;
  L.temps = a.temps;
  L.B = a.B;
  L.gamma = a.gamma;
  L.V = a.V;
  L.out_n = a.out_n;
  L.out_tok = a.out_tok;
  if (a.diag) {
    L.diag_px = a.diag->p_x;
    L.diag_qx = a.diag->q_x;
    L.diag_mass = a.diag->resid_mass;
  }
  const int64_t G = a.gamma, V = a.V, B = a.B;
  const int64_t total = B * ((G + 1) * V * et + G * V * ed);
  const int64_t cb = early ? early_chunk_bytes() : chunk_bytes_for(total);
  // chunks start on 16 KB batch boundaries of their rows (see chunk_bytes_for)
  split_row(V, et, cb, &L.nct, &L.cut, kBatchUnits);
  split_row(V, ed, cb, &L.ncd, &L.cud, kBatchUnits);
  L.per_seq = (int)((G + 1) * L.nct + G * L.ncd);
  L.ns2 = (int)draw_steps(V);
  finish_shape(B, L.ns2, &L.parts, &L.fin_waves);
  const SampleLayout lay = sample_layout(B, G, V);
  char* ws = (char*)a.ws;
  L.part = (RowPartial*)(ws + lay.off_part);
  L.steptot = (double*)(ws + lay.off_step);
  L.done = (int32_t*)(ws + lay.off_done);
  return L;
}

// stages 1..2 = stats, finish; first..last inclusive
static int run_sample(int first, int last, const SampleArgs& a, hipStream_t stream) {
  int st = validate_sample(a);
  if (st) return st;
  const SampleLaunch L = plan_sample(a);
  // grid sizes fit a 32-bit dimension by construction of the limits; check anyway
  if ((int64_t)L.B * L.per_seq > 0x7fffffffLL) return SV_ERR_SHAPE;
  // the whole call on rows of one draw step: one kernel, a wave per sequence
  if (first == 1 && last == 2 && a.V <= kStepTokens) return hip_status(launch_sample_small(L, a.tdt, a.ddt, stream));
  for (int s = first; s <= last; ++s) {
    st = hip_status(launch_sample_stage(L, a.tdt, a.ddt, s, stream));
    if (st) return st;
  }
  return SV_OK;
}

// Draft-side sampler: the path with gamma = 0 (statistics of one row per
// sequence, then the bonus-mode draw from it).
static int run_draft(int first, int last, const void* logits, int dtype, int64_t row_stride, const float* uniforms,
                     const float* temperature, int B, int V, int32_t* out_tokens, float* out_prob, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (!logits || !uniforms || !temperature || !out_tokens) return SV_ERR_NULL;
  if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
  if (B < 1 || B > SV_MAX_BATCH || V < 1 || V > SV_MAX_VOCAB) return SV_ERR_SHAPE;
  int st = check_rows(logits, dtype, row_stride, row_stride, B, 1, V);
  if (st) return st;
  if (!aligned(uniforms, 4) || !aligned(temperature, 4) || !aligned(out_tokens, 4) || !aligned(out_prob, 4))
    return SV_ERR_ALIGN;
  if (!ws) return SV_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SV_ERR_ALIGN;
  if (ws_bytes < (size_t)sample_layout(B, 0, V).total) return SV_ERR_WORKSPACE;
  SampleArgs a{logits, dtype, row_stride, row_stride, nullptr, dtype, 0, 0, nullptr, uniforms, temperature, B, 0, V,
               nullptr, out_tokens, nullptr, ws, ws_bytes};
  SampleLaunch L = plan_sample(a);
  L.out_py = out_prob;
  if ((int64_t)L.B * L.per_seq > 0x7fffffffLL) return SV_ERR_SHAPE;
  if (first == 0) {
    // rows of one draw step: a wave per row (the verify's one-kernel path with
    // gamma = 0, a bonus-row draw); longer rows: a workgroup per row
    if (V <= kStepTokens) return hip_status(launch_sample_small(L, dtype, dtype, stream));
    return hip_status(launch_draft_one_pass(L, dtype, stream));
  }
  for (int s = first; s <= last; ++s) {
    st = hip_status(launch_sample_stage(L, dtype, dtype, s, stream));
    if (st) return st;
  }
  return SV_OK;
}

// Early exit: statistics launches over positions 0, 1, ..., k-1 and then
// k..gamma together (each gated on the accept decision of the position before
// it), then the finish kernel.
static int run_sample_early(const SampleArgs& a, int tail_start, hipStream_t stream) {
  int st = validate_sample(a);
  if (st) return st;
  if (tail_start > a.gamma) return SV_ERR_ARG;
  SampleLaunch L = plan_sample(a, true);
  if ((int64_t)L.B * L.per_seq > 0x7fffffffLL) return SV_ERR_SHAPE;
  L.reach = (int32_t*)((char*)a.ws + sample_layout(a.B, a.gamma, a.V).off_reach);
  const int k = tail_start >= 0 ? tail_start : early_tail_start(a.B, a.gamma, a.V, esz_of(a.tdt), esz_of(a.ddt));
  // No gated position: every row is read either way, and the one-pass call
  // does it with its own work units (finer for small calls: a single 128k
  // sequence 0.0240 -> 0.0205 ms) or, for rows of one draw step, in one
  // launch (a wave per sequence); its results are the one-pass call's.
  if (k == 0) return run_sample(1, 2, a, stream);
  for (int p0 = 0; p0 <= a.gamma;) {
    const int p1 = (p0 < k) ? p0 : a.gamma;
    st = hip_status(launch_sample_pos(L, a.tdt, a.ddt, p0, p1, stream));
    if (st) return st;
    p0 = p1 + 1;
  }
  return hip_status(launch_sample_stage(L, a.tdt, a.ddt, 2, stream));
}

// ---------------------------------------------------------------------------
// spec_verify_sample_noalloc: the workspace is a static device array
// ---------------------------------------------------------------------------
// One copy per GPU, held until the process ends. In host code `scratch` names a
// host-side stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept here.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The static array's address on the current device (looked up at the first
// call on that device).
static int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return SV_ERR_ARG;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (!p) return SV_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" {

int spec_verify_sample_noalloc(const void* target_logits, int target_dtype, int64_t target_seq_stride,
                               int64_t target_row_stride, const void* draft_logits, int draft_dtype,
                               int64_t draft_seq_stride, int64_t draft_row_stride, const int32_t* draft_tokens,
                               const float* uniforms, const float* temperature, int B, int gamma, int V,
                               int32_t* out_num_accepted, int32_t* out_tokens, const sv_sample_diag* diag,
                               void* stream) {
  // every argument check of spec_verify_sample first (with a stand-in
  // workspace of the array's size and alignment), then the size, then the
  // first HIP call
  SampleArgs a{target_logits, target_dtype, target_seq_stride, target_row_stride, draft_logits, draft_dtype,
               draft_seq_stride, draft_row_stride, draft_tokens, uniforms, temperature, B, gamma, V,
               out_num_accepted, out_tokens, diag, (void*)(uintptr_t)256, (size_t)SV_NOALLOC_SCRATCH_BYTES};
  int st = validate_sample(a);
  if (st == SV_ERR_WORKSPACE) return SV_ERR_SCRATCH;  // the layout exceeds the array
  if (st) return st;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st) return st;
  a.ws = ws;
  return run_sample(1, 2, a, (hipStream_t)stream);
}

size_t sv_sample_workspace_bytes(int B, int gamma, int V) {
  if (B < 1 || B > SV_MAX_BATCH || gamma < 1 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return 0;
  return (size_t)sample_layout(B, gamma, V).total;
}

size_t sv_tree_workspace_bytes(int B, int N, int V) {
  if (B < 1 || B > SV_MAX_BATCH || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB) return 0;
  return (size_t)tree_layout(B, N, V).total;
}

int spec_verify_sample_stage(int stage, const void* target_logits, int target_dtype, int64_t target_seq_stride,
                             int64_t target_row_stride, const void* draft_logits, int draft_dtype,
                             int64_t draft_seq_stride, int64_t draft_row_stride, const int32_t* draft_tokens,
                             const float* uniforms, const float* temperature, int B, int gamma, int V,
                             int32_t* out_num_accepted, int32_t* out_tokens, const sv_sample_diag* diag,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < 1 || stage > 3) return SV_ERR_ARG;
  SampleArgs a{target_logits, target_dtype, target_seq_stride, target_row_stride, draft_logits, draft_dtype,
               draft_seq_stride, draft_row_stride, draft_tokens, uniforms, temperature, B, gamma, V,
               out_num_accepted, out_tokens, diag, workspace, workspace_bytes};
  return run_sample(stage, stage, a, (hipStream_t)stream);
}

int spec_verify_sample(const void* target_logits, int target_dtype, int64_t target_seq_stride,
                       int64_t target_row_stride, const void* draft_logits, int draft_dtype, int64_t draft_seq_stride,
                       int64_t draft_row_stride, const int32_t* draft_tokens, const float* uniforms,
                       const float* temperature, int B, int gamma, int V, int32_t* out_num_accepted,
                       int32_t* out_tokens, const sv_sample_diag* diag, void* workspace, size_t workspace_bytes,
                       void* stream) {
  SampleArgs a{target_logits, target_dtype, target_seq_stride, target_row_stride, draft_logits, draft_dtype,
               draft_seq_stride, draft_row_stride, draft_tokens, uniforms, temperature, B, gamma, V,
               out_num_accepted, out_tokens, diag, workspace, workspace_bytes};
  return run_sample(1, 2, a, (hipStream_t)stream);
}

int spec_verify_sample_early_exit(const void* target_logits, int target_dtype, int64_t target_seq_stride,
                                  int64_t target_row_stride, const void* draft_logits, int draft_dtype,
                                  int64_t draft_seq_stride, int64_t draft_row_stride, const int32_t* draft_tokens,
                                  const float* uniforms, const float* temperature, int B, int gamma, int V,
                                  int32_t* out_num_accepted, int32_t* out_tokens, const sv_sample_diag* diag,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  SampleArgs a{target_logits, target_dtype, target_seq_stride, target_row_stride, draft_logits, draft_dtype,
               draft_seq_stride, draft_row_stride, draft_tokens, uniforms, temperature, B, gamma, V,
               out_num_accepted, out_tokens, diag, workspace, workspace_bytes};
  return run_sample_early(a, -1, (hipStream_t)stream);
}

int spec_verify_sample_early_exit_grouped(int tail_start, const void* target_logits, int target_dtype,
                                          int64_t target_seq_stride, int64_t target_row_stride,
                                          const void* draft_logits, int draft_dtype, int64_t draft_seq_stride,
                                          int64_t draft_row_stride, const int32_t* draft_tokens,
                                          const float* uniforms, const float* temperature, int B, int gamma,
                                          int V, int32_t* out_num_accepted, int32_t* out_tokens,
                                          const sv_sample_diag* diag, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  SampleArgs a{target_logits, target_dtype, target_seq_stride, target_row_stride, draft_logits, draft_dtype,
               draft_seq_stride, draft_row_stride, draft_tokens, uniforms, temperature, B, gamma, V,
               out_num_accepted, out_tokens, diag, workspace, workspace_bytes};
  return run_sample_early(a, tail_start < 0 ? -1 : tail_start, (hipStream_t)stream);
}

int spec_tree_mask(const int32_t* parents, const int32_t* blocks, int B, int N, uint8_t* out_mask,
                   uint8_t* out_relaxed, int32_t* out_depth, void* stream) {
  if (!parents || (out_relaxed && !blocks)) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || N < 1 || N > SV_MAX_TREE_NODES) return SV_ERR_SHAPE;
  if (!aligned(parents, 4) || !aligned(blocks, 4) || !aligned(out_depth, 4)) return SV_ERR_ALIGN;
  if (!out_mask && !out_relaxed && !out_depth) return SV_OK;
  MaskLaunch L;
  L.parents = parents;
  L.blocks = blocks;
  L.B = B;
  L.N = N;
  // rows per workgroup: about kMaskSlabBytes of mask, and their ancestor
  // bitsets (ceil(N / 32) words per row) within the kernel's LDS array
  const int64_t nslab0 = ceil_div((int64_t)N * N, kMaskSlabBytes);
  const int64_t words = ceil_div(N, 32);
  L.rows_per_slab = (int)std::min<int64_t>(ceil_div(N, nslab0), kMaskSlabBytes / 32 / words);
  L.nslab = (int)ceil_div(N, L.rows_per_slab);
  if ((int64_t)B * L.nslab > 0x7fffffffLL) return SV_ERR_SHAPE;
  L.out_mask = out_mask;
  L.out_relaxed = out_relaxed;
  L.out_depth = out_depth;
  return hip_status(launch_mask(L, (hipStream_t)stream));
}

size_t sv_draft_workspace_bytes(int B, int V) {
  if (B < 1 || B > SV_MAX_BATCH || V < 1 || V > SV_MAX_VOCAB) return 0;
  return (size_t)sample_layout(B, 0, V).total;
}

int spec_draft_sample(const void* logits, int dtype, int64_t row_stride, const float* uniforms,
                      const float* temperature, int B, int V, int32_t* out_tokens, float* out_prob, void* workspace,
                      size_t workspace_bytes, void* stream) {
  // one pass (one workgroup per row, or a wave per row of at most one draw
  // step) when the rows keep the GPU busy or are short, and a row's step
  // masses fit the kernel's LDS; else the two kernels
  const bool one_pass = draft_one_pass(B, V, esz_of(dtype));
  return run_draft(one_pass ? 0 : 1, 2, logits, dtype, row_stride, uniforms, temperature, B, V, out_tokens,
                   out_prob, workspace, workspace_bytes, (hipStream_t)stream);
}

int spec_draft_sample_stage(int stage, const void* logits, int dtype, int64_t row_stride, const float* uniforms,
                            const float* temperature, int B, int V, int32_t* out_tokens, float* out_prob,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < 1 || stage > 2) return SV_ERR_ARG;
  return run_draft(stage, stage, logits, dtype, row_stride, uniforms, temperature, B, V, out_tokens, out_prob,
                   workspace, workspace_bytes, (hipStream_t)stream);
}

static int run_tree(int first, int last, const void* target_logits, int dtype, int64_t seq_stride,
                    int64_t row_stride, const int32_t* parents, const int32_t* tokens, int B, int N, int V,
                    int32_t* out_accept_len, int32_t* out_path, int32_t* out_bonus, int32_t* out_argmax,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!target_logits || !parents || !tokens || !out_accept_len || !out_path || !out_bonus) return SV_ERR_NULL;
  if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
  if (B < 1 || B > SV_MAX_BATCH || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB) return SV_ERR_SHAPE;
  int st = check_rows(target_logits, dtype, seq_stride, row_stride, B, N, V);
  if (st) return st;
  if (!aligned(parents, 4) || !aligned(tokens, 4) || !aligned(out_accept_len, 4) || !aligned(out_path, 4) ||
      !aligned(out_bonus, 4) || (out_argmax && !aligned(out_argmax, 4)))
    return SV_ERR_ALIGN;
  if (!workspace) return SV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return SV_ERR_ALIGN;
  const TreeLayout lay = tree_layout(B, N, V);
  if (workspace_bytes < (size_t)lay.total) return SV_ERR_WORKSPACE;

  TreeLaunch L;
  memset(&L, 0, sizeof(L));
  const int esz = esz_of(dtype);
  L.logits = (const char*)target_logits;
  L.seq_b = seq_stride * esz;
  L.row_b = row_stride * esz;
  L.parents = parents;
  L.tokens = tokens;
  L.B = B;
  L.N = N;
  L.V = V;
  const int64_t total = (int64_t)B * N * V * esz;
  split_row(V, esz, tree_chunk_bytes_for(total), &L.nch, &L.cu);
  L.out_len = out_accept_len;
  L.out_path = out_path;
  L.out_bonus = out_bonus;
  L.out_argmax = out_argmax;
  L.part = (ArgPartial*)((char*)workspace + lay.off_part);
  if ((int64_t)B * N * L.nch > 0x7fffffffLL) return SV_ERR_SHAPE;
  for (int s = first; s <= last; ++s) {
    st = hip_status(launch_tree(L, dtype, s, (hipStream_t)stream));
    if (st) return st;
  }
  return SV_OK;
}

int spec_verify_greedy_tree(const void* target_logits, int dtype, int64_t seq_stride, int64_t row_stride,
                            const int32_t* parents, const int32_t* tokens, int B, int N, int V,
                            int32_t* out_accept_len, int32_t* out_path, int32_t* out_bonus, int32_t* out_argmax,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return run_tree(1, 2, target_logits, dtype, seq_stride, row_stride, parents, tokens, B, N, V, out_accept_len,
                  out_path, out_bonus, out_argmax, workspace, workspace_bytes, stream);
}

int spec_verify_greedy_tree_stage(int stage, const void* target_logits, int dtype, int64_t seq_stride,
                                  int64_t row_stride, const int32_t* parents, const int32_t* tokens, int B, int N,
                                  int V, int32_t* out_accept_len, int32_t* out_path, int32_t* out_bonus,
                                  int32_t* out_argmax, void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < 1 || stage > 2) return SV_ERR_ARG;
  return run_tree(stage, stage, target_logits, dtype, seq_stride, row_stride, parents, tokens, B, N, V,
                  out_accept_len, out_path, out_bonus, out_argmax, workspace, workspace_bytes, stream);
}

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "shape out of range (B, gamma, N, V, strides or size overflow)";
    case SV_ERR_DTYPE: return "unknown dtype (use SV_F32 or SV_BF16)";
    case SV_ERR_ALIGN: return "misaligned pointer or stride (rows need 16-byte alignment)";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP launch failed (see sv_last_hip_error)";
    case SV_ERR_ARG: return "invalid argument";
    case SV_ERR_SCRATCH: return "call too large for spec_verify_sample_noalloc's static scratch (32 MiB)";
    default: return "unknown status";
  }
}

int sv_last_hip_error(void) { return g_last_hip_error; }

const char* sv_version(void) { return "spec_verify 0.1.0 (gfx950)"; }

}  // extern "C"
