/*
 * spec_verify.h -- C ABI of libspec_verify.so, the verify step of speculative
 * decoding on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *  [SD]     "Fast Inference from Transformers via Speculative Decoding",
 *           Pith review page (pith.science, arXiv 2211.17192).
 *  [Falcon] "Falcon: Faster and Parallel Inference of Large Language Models
 *           through Enhanced Semi-Autoregressive Drafting and Custom-Designed
 *           Decoding Tree", Pith review page (pith.science, arXiv 2412.12639).
 *
 * Conventions shared by every entry point
 *  - Pointers named *logits, tokens, uniforms, temperature, parents, out_* and
 *    workspace are DEVICE pointers owned by the caller. The library never
 *    allocates, frees or retains them past the call.
 *  - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *    stream). Every call only enqueues work on it and returns; outputs are
 *    valid once the stream reaches that point. No call synchronises.
 *  - Strides are in ELEMENTS of the logits' dtype. Every logits row must start
 *    on a 16-byte boundary: base pointer, row stride and sequence stride times
 *    the element size must all be multiples of 16 bytes (a sequence stride of 0
 *    is allowed and makes every sequence share one block of rows). The kernels
 *    may read the rest of the 16-byte block that holds a row's last element;
 *    those bytes are ignored.
 *  - Return value: SV_OK, or a negative sv_status. Argument errors are found
 *    on the host before any HIP call, so nothing is enqueued when a call fails
 *    that way. Data-dependent problems (bad token, NaN row, ...) do not fail
 *    the call: the affected sequence reports -1 (see each call).
 *  - Workspace: device memory of at least the size the matching *_workspace_bytes
 *    function returns, 256-byte aligned. It needs no initialisation and holds
 *    nothing between calls. Calls that overlap in time must not share one.
 *  - No C++ exception crosses this interface. The library holds no global
 *    mutable state apart from the thread-local last HIP error and the
 *    per-device address of spec_verify_sample_noalloc's static array (set once
 *    per device, under a lock).
 *  - Results are deterministic: the same inputs give the same bits. A
 *    sequence's results barely depend on the batch it is verified in (its
 *    batch size, its place in the batch, the split of its rows into work
 *    chunks): every fp32 rounding of its statistics is taken over fixed 16 KB
 *    blocks of its rows, and only fp64 sums of those blocks' results are
 *    grouped differently. The reported probabilities then differ by fp64
 *    rounding, and a decision or token differs only where a quantity lies
 *    within that rounding of its boundary.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL = -1,      /* a required pointer is NULL */
  SV_ERR_SHAPE = -2,     /* B, gamma, V or N out of range, stride < V, size overflow */
  SV_ERR_DTYPE = -3,     /* dtype is not SV_F32 or SV_BF16 */
  SV_ERR_ALIGN = -4,     /* a logits row does not start on a 16-byte boundary; a
                            4-byte array is not 4-byte aligned; workspace not 256-byte aligned */
  SV_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required */
  SV_ERR_HIP = -6,       /* a HIP launch failed; sv_last_hip_error() gives the hipError_t */
  SV_ERR_ARG = -7,       /* any other invalid argument (e.g. an unknown stage) */
  SV_ERR_SCRATCH = -8    /* spec_verify_sample_noalloc: the call needs more than SV_NOALLOC_SCRATCH_BYTES */
} sv_status;

/* Limits checked on the host. */
#define SV_MAX_GAMMA 64
#define SV_MAX_TREE_NODES 1024
#define SV_MAX_VOCAB (1 << 30)
#define SV_MAX_BATCH (1 << 24)

/* Workspace sizes in bytes (valid for either logits dtype). 0 for shapes
 * outside the limits above. */
size_t sv_sample_workspace_bytes(int B, int gamma, int V);
size_t sv_tree_workspace_bytes(int B, int N, int V);

/* Optional per-position diagnostics of spec_verify_sample; any member may be
 * NULL (not written). Values are fp32 roundings of fp64 results. */
typedef struct {
  float* p_x;        /* [B][gamma]: p_i(x_i), target probability of draft token i */
  float* q_x;        /* [B][gamma]: q_i(x_i), draft probability of draft token i */
  float* resid_mass; /* [B]: mass of the distribution the final token was drawn from,
                        before renormalisation: 1 - alpha_n after a rejection at n
                        (alpha_n = sum_v min(p_n,v, q_n,v)), about 1 for the bonus row */
} sv_sample_diag;

/*
 * spec_verify_sample -- speculative sampling verification of B sequences.
 *
 * Defines: [SD] "The pith" and "What carries the argument" (score gamma drafted
 * tokens in one parallel target pass, keep the longest accepted prefix, emit
 * several tokens per target call); [SD] "Desk Editor's Note" and "Referee
 * Report" (Summary, Significance) (a rejection-sampling correction whose
 * accept probability comes from the target conditional); [SD] abstract, "Core
 * claim" and "Circularity Check" (the output distribution is exactly the
 * target's). For sequence b with temperature T:
 *   p_i = softmax(target row i / T), q_i = softmax(draft row i / T);
 *   accept x_i iff u[b][i] < p_i(x_i) / q_i(x_i), for i = 0, 1, ... until the
 *   first rejection n (n = gamma if all are accepted);
 *   after a rejection draw y from max(0, p_n - q_n) renormalised, otherwise
 *   from p_gamma (the bonus row), by inverse CDF in token-id order at
 *   u[b][gamma] (the smallest v whose running mass exceeds u * total);
 *   out_tokens[b] = x_0 .. x_{n-1}, y, then -1; out_num_accepted[b] = n.
 *
 * target_logits : logical [B][gamma+1][V], dtype target_dtype; row i (i < gamma)
 *                 holds the target's next-token logits after the drafts
 *                 x_0..x_{i-1}; row gamma is the bonus row.
 * draft_logits  : logical [B][gamma][V], dtype draft_dtype; row i is the
 *                 distribution x_i was drawn from.
 * draft_tokens  : [B][gamma] int32, contiguous.
 * uniforms      : [B][gamma+1] float, contiguous, each in [0, 1): u[b][i]
 *                 for the accept test of position i, u[b][gamma] for the draw.
 * temperature   : [B] float, each finite, positive and normal (>= 2^-126).
 * out_num_accepted : [B] int32: n in [0, gamma], or -1 for an invalid sequence.
 * out_tokens    : [B][gamma+1] int32 (all -1 for an invalid sequence).
 * diag          : may be NULL.
 *
 * A sequence is invalid (-1) when its temperature is not usable, or when a
 * position the method reaches (accept tests 0..n, the draw at n or gamma) has a
 * token outside [0, V), a draft token whose draft logit is -inf, a uniform
 * outside [0, 1), or a target/draft row with NaN, +inf or no finite value.
 * Rows after the first rejection are not consulted.
 *
 * Work on `stream`: the statistics kernel then the finish kernel (see
 * spec_verify_sample_stage); with V <= 2048 a single kernel, one wave per
 * sequence (two per wave when V <= 32 and 2 * gamma + 1 <= 32, with the same
 * results). The paths round differently and agree within the parity contract.
 */
int spec_verify_sample(const void* target_logits, int target_dtype, int64_t target_seq_stride,
                       int64_t target_row_stride, const void* draft_logits, int draft_dtype,
                       int64_t draft_seq_stride, int64_t draft_row_stride, const int32_t* draft_tokens,
                       const float* uniforms, const float* temperature, int B, int gamma, int V,
                       int32_t* out_num_accepted, int32_t* out_tokens, const sv_sample_diag* diag,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_sample_noalloc -- spec_verify_sample for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, outputs, kernels and
 * results, without the workspace. The workspace is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends; its
 * address on the current device is looked up once (hipGetSymbolAddress) at the
 * first call on that device. The call allocates nothing.
 *
 * Calls on one GPU share its array: calls that may overlap in time on the
 * same GPU (concurrent streams, or threads) race and must not be made; the
 * array keeps the last call's contents, which no call depends on. The current
 * HIP device must be the GPU that owns the pointers and the stream.
 * Errors: as spec_verify_sample, and SV_ERR_SCRATCH when
 * sv_sample_workspace_bytes(B, gamma, V) exceeds SV_NOALLOC_SCRATCH_BYTES
 * (found before any HIP call).
 */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20)
int spec_verify_sample_noalloc(const void* target_logits, int target_dtype, int64_t target_seq_stride,
                               int64_t target_row_stride, const void* draft_logits, int draft_dtype,
                               int64_t draft_seq_stride, int64_t draft_row_stride, const int32_t* draft_tokens,
                               const float* uniforms, const float* temperature, int B, int gamma, int V,
                               int32_t* out_num_accepted, int32_t* out_tokens, const sv_sample_diag* diag,
                               void* stream);

/*
 * spec_verify_sample_early_exit -- spec_verify_sample ordered by position, so
 * that the rows after a sequence's first rejection need not be read.
 *
 * Defines: [SD] "The pith" (the longest accepted prefix is kept: nothing after
 * the first rejection can change the output). Same arguments, outputs,
 * validity rules, workspace and parity with the definition as
 * spec_verify_sample. The work is ordered by position: statistics launches
 * over positions 0, 1, ..., k-1 one at a time and then k..gamma together (k
 * from the sizes: a position gets its own launch while the bytes its gate is
 * expected to save, at an assumed acceptance rate of 0.7, outweigh a launch;
 * small batches get k = 0, one launch with no gate), then the finish kernel.
 * With k = 0 every row is read in any case, and the call runs
 * spec_verify_sample instead (its work units, or its one-kernel path for
 * V <= 2048; the same results as spec_verify_sample, bit for bit).
 * spec_verify_sample_early_exit_grouped takes k from the caller. In every launch
 * after the first, each workgroup re-derives the accept decision of the
 * position before it and streams its rows only if that position was accepted.
 * Data moved: the rows of positions 0..n (0..gamma for a sequence that reaches
 * the tail group) plus the draw row(s), instead of all 2*gamma+1 rows.
 * Differences from spec_verify_sample: the row statistics are taken in smaller
 * chunks, so results can differ in rounding (an accept decision within ~1e-7
 * of u, p_x and q_x in the last bits); diag p_x, q_x are NaN for positions
 * whose rows were not read; more kernel launches (k + 2 instead of 2). With
 * k = 0 none of these differences apply.
 */
int spec_verify_sample_early_exit(const void* target_logits, int target_dtype, int64_t target_seq_stride,
                                  int64_t target_row_stride, const void* draft_logits, int draft_dtype,
                                  int64_t draft_seq_stride, int64_t draft_row_stride,
                                  const int32_t* draft_tokens, const float* uniforms, const float* temperature,
                                  int B, int gamma, int V, int32_t* out_num_accepted, int32_t* out_tokens,
                                  const sv_sample_diag* diag, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * spec_verify_sample_early_exit_grouped -- spec_verify_sample_early_exit with
 * the grouping of positions chosen by the caller (who may know the
 * acceptance rate): tail_start = k in 0..gamma gives positions 0..k-1 a
 * statistics launch each and k..gamma one together (k = 0: one launch, no
 * gate; k = gamma: every position gated); tail_start < 0 chooses k from the
 * sizes exactly as spec_verify_sample_early_exit. Same definition ([SD] "The
 * pith"), arguments, outputs and parity. Errors: tail_start > gamma ->
 * SV_ERR_ARG, otherwise as spec_verify_sample.
 */
int spec_verify_sample_early_exit_grouped(int tail_start, const void* target_logits, int target_dtype,
                                          int64_t target_seq_stride, int64_t target_row_stride,
                                          const void* draft_logits, int draft_dtype, int64_t draft_seq_stride,
                                          int64_t draft_row_stride, const int32_t* draft_tokens,
                                          const float* uniforms, const float* temperature, int B, int gamma,
                                          int V, int32_t* out_num_accepted, int32_t* out_tokens,
                                          const sv_sample_diag* diag, void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * spec_verify_sample_stage -- one of the two kernels of spec_verify_sample,
 * for callers that want to time or overlap them. Same arguments and meaning as
 * spec_verify_sample; `stage` selects:
 *   1: row statistics: streams every target and draft row once (maximum and
 *      tempered sum-exp per wave and row chunk, into the workspace);
 *   2: finish, one workgroup per sequence (several for small batches of
 *      long rows): merges the statistics, runs the accept tests and the
 *      first-rejection scan, streams the one row (pair) the draw needs, draws
 *      by inverse CDF at u[b][gamma] and writes every output (and diag).
 *   3: the reads of stage 1 alone, for measurement: the same grid, row
 *      chunks and 16-byte loads, with the arithmetic replaced by an xor of
 *      the loaded words. It computes nothing of the method and writes no
 *      output; its time is the rate at which stage 1 could read these bytes.
 *      It may leave one word of the workspace changed (stage 1 resets it).
 * Stage 2 must follow stage 1 on the same stream with the same arguments and
 * workspace. spec_verify_sample enqueues both.
 */
int spec_verify_sample_stage(int stage, const void* target_logits, int target_dtype,
                             int64_t target_seq_stride, int64_t target_row_stride, const void* draft_logits,
                             int draft_dtype, int64_t draft_seq_stride, int64_t draft_row_stride,
                             const int32_t* draft_tokens, const float* uniforms, const float* temperature,
                             int B, int gamma, int V, int32_t* out_num_accepted, int32_t* out_tokens,
                             const sv_sample_diag* diag, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * spec_draft_sample -- draft-side sampler: one token per row from the
 * tempered softmax of the row, by inverse CDF.
 *
 * Defines: [SD] "The pith" and the abstract (the fast approximation model
 * proposes the speculative tokens by sampling from its own distribution q;
 * spec_verify_sample then needs x_i ~ q_i). For row b with temperature T:
 *   q = softmax(logits[b] / T); out_tokens[b] = the smallest v whose running
 *   mass in token-id order exceeds uniforms[b] * (total mass).
 * The same row statistics and draw as spec_verify_sample's bonus-row draw.
 *
 * logits      : [B][V], dtype, rows row_stride elements apart (>= V, 16-byte
 *               aligned rows).
 * uniforms    : [B] float in [0, 1).
 * temperature : [B] float, finite, positive and normal.
 * out_tokens  : [B] int32: the drawn token, or -1 for an invalid row (bad
 *               temperature or uniform, NaN or +inf in the row, no finite value).
 * out_prob    : [B] float or NULL: q(out_token) (fp32 rounding of an fp64
 *               value; NaN for an invalid row).
 * workspace   : at least sv_draft_workspace_bytes(B, V), 256-byte aligned, no
 *               initialisation needed. Errors as for spec_verify_sample.
 */
size_t sv_draft_workspace_bytes(int B, int V);
int spec_draft_sample(const void* logits, int dtype, int64_t row_stride, const float* uniforms,
                      const float* temperature, int B, int V, int32_t* out_tokens, float* out_prob, void* workspace,
                      size_t workspace_bytes, void* stream);

/* One of the two kernels of spec_draft_sample (same arguments): stage 1 row
 * statistics, stage 2 the draw and the outputs; stage 2 must follow stage 1 on
 * the same stream with the same arguments and workspace. */
int spec_draft_sample_stage(int stage, const void* logits, int dtype, int64_t row_stride, const float* uniforms,
                            const float* temperature, int B, int V, int32_t* out_tokens, float* out_prob,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_greedy_tree -- greedy verification of B draft trees.
 *
 * Defines: [Falcon] "What carries the argument" (the drafter proposes a tree of
 * candidate branches that the target verifies in one parallel pass) and
 * [Falcon] "Assumptions & free parameters" with Figure 4 (greedy decoding,
 * temperature 0; the result equals vanilla autoregressive decoding). For tree b:
 *   g_j = argmax_v logits[b][j][v] (lowest v on ties; -0 equals +0);
 *   node 0 (the root) is accepted; node j >= 1 is accepted iff its parent is
 *   accepted and tokens[b][j] == g_{parents[b][j]};
 *   d = the accepted node of largest depth (lowest node id on ties);
 *   out_accept_len[b] = depth(d); out_path[b] = node ids root .. d, then -1;
 *   out_bonus[b] = g_d.
 *
 * target_logits : logical [B][N][V]; row j holds the target's next-token
 *                 logits after node j.
 * parents       : [B][N] int32, contiguous; parents[b][0] = -1 and
 *                 0 <= parents[b][j] < j.
 * tokens        : [B][N] int32, contiguous; tokens[b][0] (the root) is unused,
 *                 tokens[b][j] in [0, V) for j >= 1.
 * out_accept_len: [B] int32: depth of d, or -1 for an invalid tree.
 * out_path      : [B][N] int32.
 * out_bonus     : [B] int32.
 * out_argmax    : [B][N] int32 per-node argmax (-1 for a row with NaN or
 *                 +inf); may be NULL.
 *
 * A tree is invalid (-1 everywhere) if its parent array breaks the rule above,
 * a non-root token is outside [0, V), or any of its rows holds NaN or +inf.
 * A row of -inf only has argmax 0.
 */
int spec_verify_greedy_tree(const void* target_logits, int dtype, int64_t seq_stride, int64_t row_stride,
                            const int32_t* parents, const int32_t* tokens, int B, int N, int V,
                            int32_t* out_accept_len, int32_t* out_path, int32_t* out_bonus,
                            int32_t* out_argmax, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_greedy_tree_stage -- one of the two kernels of
 * spec_verify_greedy_tree (same arguments): stage 1 streams every row and
 * leaves per-row argmax partials in the workspace; stage 2 merges them,
 * resolves each tree and writes every output. Stage 2 must follow stage 1 on
 * the same stream with the same arguments and workspace.
 */
int spec_verify_greedy_tree_stage(int stage, const void* target_logits, int dtype, int64_t seq_stride,
                                  int64_t row_stride, const int32_t* parents, const int32_t* tokens, int B, int N,
                                  int V, int32_t* out_accept_len, int32_t* out_path, int32_t* out_bonus,
                                  int32_t* out_argmax, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_tree_mask -- attention masks and positions of B draft trees.
 *
 * Defines: [Falcon] "What carries the argument" (the target verifies the
 * tree's candidate branches in one parallel pass; the drafter uses a relaxed
 * causal mask under which the tokens of one k-token block attend to each
 * other) and "Assumptions & free parameters" (the relaxed mask must keep the
 * causality verification needs). For tree b with parent array parents[b]
 * (parents[b][0] = -1, 0 <= parents[b][j] < j):
 *   out_mask[b][i][j]    = 1 iff node j is node i or one of its ancestors
 *                          (the target's tree-attention mask), else 0;
 *   out_relaxed[b][i][j] = out_mask[b][i][j] or (blocks[b][i] >= 0 and
 *                          blocks[b][i] == blocks[b][j]) (the drafter's mask);
 *   out_depth[b][i]      = depth of node i (root 0): its position offset.
 * blocks [B][N] int32 (nodes proposed together share an id, -1 = none) is
 * needed only for out_relaxed. Masks are uint8 [B][N][N], row-major, any
 * alignment; int32 arrays 4-byte aligned. Any output may be NULL. A tree with
 * an invalid parent array gets all-zero masks and depth -1. No workspace.
 * Errors: SV_ERR_NULL (parents NULL, or out_relaxed without blocks),
 * SV_ERR_SHAPE (B or N out of range), SV_ERR_ALIGN, SV_ERR_HIP.
 */
int spec_tree_mask(const int32_t* parents, const int32_t* blocks, int B, int N, uint8_t* out_mask,
                   uint8_t* out_relaxed, int32_t* out_depth, void* stream);

/* Text of a status code (static storage). */
const char* sv_status_string(int status);

/* hipError_t of the last failed HIP call made by this thread inside the library (0 = none). */
int sv_last_hip_error(void);

/* Library version string. */
const char* sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
