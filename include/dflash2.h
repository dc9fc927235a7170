/*
 * dflash2.h -- C ABI of the MI355X (gfx950) DFlash 2 path selector.
 *
 * The selector is described on the page "DFlash 2: Keep Drafting Parallel",
 * section "A Lightweight Path Selector": keep the top 16 candidates of the
 * block drafter at every draft position, score every adjacent candidate pair
 * with the selector equation
 *
 *     S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >
 *
 * (U_t is the drafter's own logit, A and B are 256-dimensional token
 * embeddings, H(h_t) a gate computed from the drafter hidden state), and make
 * one walk over the precomputed scores, starting from the last verified
 * token.  This library reads H as a bias-free linear map d -> r,
 * H_t = W_H h_t, and the walk as a max-sum (Viterbi) pass with backtrack;
 * the section's literal greedy walk is available as a second walk mode, and
 * its sampling walk through dflash2_select_sample / dflash2_sample_walk,
 * whose uniforms dflash2_philox_uniforms can draw on the device.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer on the current HIP device,
 *    owned by the caller.  The library reads inputs, writes outputs, keeps no
 *    pointer after the call returns and never frees caller memory.
 *  - Every tensor is dense row-major (C order), last dimension contiguous.
 *  - Work is enqueued on `stream` and the call returns without waiting.
 *  - Scratch memory (top-K partials, gate partials, pair scores, arrival
 *    counters) comes from a cache owned by the library, one buffer per
 *    (device, stream); it grows with hipMalloc outside the launch and is
 *    zero-initialised when allocated.  Calls on the same stream are ordered; calls on different
 *    streams use different scratch.  Warm the cache with one call before
 *    capturing a stream into a HIP graph.
 *  - Argument errors are found on the host, before any launch: the call
 *    returns DF2_EINVAL or DF2_EUNSUPPORTED, enqueues nothing, and
 *    dflash2_last_error() describes the problem.  A failed launch returns
 *    DF2_EHIP.  Out-of-range token ids read on the device (prev_tok, or a
 *    caller's cand_idx, outside [0, V)) are replaced by token 0 and raise a
 *    device flag that dflash2_device_error() reports.
 *  - Non-finite logits (NaN) are outside the contract; +-inf are ordered.
 *  - Top-K order: value descending; equal values (IEEE, -0 == +0) go to the
 *    lower vocabulary index.  Walk ties go to the smaller predecessor rank,
 *    the final pick to the smaller rank.
 *  - The launch plan is chosen from the shapes and the device.  It can be
 *    overridden for measurement only through dflash2_plan_override(); the
 *    library never reads the environment.  The top-K plan never changes a
 *    result; the gate and convolution slice counts change the fp32 summation
 *    order of H and of the corrections (within the documented tolerances;
 *    dflash2_project keeps matching dflash2_select bit for bit).
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of logits, hidden, A_tab, B_tab and W_H (all the same). */
typedef enum { DF2_F32 = 0, DF2_BF16 = 1 } df2_dtype;

/*
 * The walk over the pair scores.
 *   DF2_WALK_VITERBI  max-sum pass plus backtrack: the path with the largest
 *                     total score (ties: smaller predecessor rank, then
 *                     smaller final rank).
 *   DF2_WALK_GREEDY   the greedy walk of the same section: from the last
 *                     verified token, each position takes the best successor
 *                     of the token chosen one step earlier,
 *                     j_0 = argmax_j S_0(prev, j), j_t = argmax_j S_t(j_{t-1}, j)
 *                     (ties: smaller rank); the score is the sum of the chosen
 *                     S_t, added in order of t.
 */
typedef enum { DF2_WALK_VITERBI = 0, DF2_WALK_GREEDY = 1 } df2_walk;

/* Plan knobs that dflash2_plan_override() can pin (0 = automatic). */
typedef enum {
    DF2_PLAN_SEGMENT_WGS = 0,   /* target count of top-K segment workgroups */
    DF2_PLAN_CHUNK_VECTORS = 1, /* 16-byte vectors per lane per chunk: 1, 2 or 4 */
    DF2_PLAN_MERGE_WORDS = 2,   /* most candidate words one row merge takes (<= 1024;
                                   automatic: 768 in dflash2_select, 1024 in dflash2_topk) */
    DF2_PLAN_GATE_SLICES = 3,   /* slices of d of the gate projection (<= 16) */
    DF2_PLAN_CONV_SLICES = 4,   /* k slices of the convolution's correction GEMM */
    DF2_PLAN_LAUNCHES = 5,      /* dflash2_select: 1 = one fused launch, 2 = scan, then
                                   merges, pairs and walk, 3 = scan with the row merges,
                                   then pairs and walk, 4 = as 3 with the walks in a third
                                   launch; automatic: 3, or 4 when the rows exceed one
                                   resident wave of workgroups */
    DF2_PLAN_LM_RANGES = 6,     /* dflash2_lmhead_topk: vocabulary ranges (<= 256) */
    DF2_PLAN_GATE_GIVEUP = 7    /* failure-handling tests only: 1 = in dflash2_select
                                   under launches 1 or 2 (the plans whose row merges
                                   wait for the gate) the row merges wait for one gate
                                   arrival more than will come, give up after 64
                                   sleeps and raise flag bit 2; that call's outputs
                                   are not valid */
} df2_plan_knob;

typedef enum {
    DF2_OK = 0,
    DF2_EINVAL = 1,        /* bad pointer, size or combination of sizes */
    DF2_EUNSUPPORTED = 2,  /* valid request outside what the library handles */
    DF2_EHIP = 3,          /* HIP runtime or launch failure */
    DF2_ENOMEM = 4         /* scratch allocation failed */
} df2_status;

/*
 * Problem sizes.
 *   B  sequences (B >= 0; B == 0 enqueues nothing)
 *   P  draft positions per sequence, the block size minus the verified
 *      token (1 <= P <= 64)
 *   V  vocabulary size (K <= V < 2^31)
 *   d  drafter hidden size (multiple of 32)
 *   r  embedding rank of A, B and H (multiple of 64, <= 512); the pages use 256
 */
typedef struct df2_dims {
    int32_t B, P, V, d, r;
    df2_dtype dtype;
} df2_dims;

/*
 * The whole selector ("A Lightweight Path Selector": top-K, pair scores, one
 * walk from the last verified token), enqueued as two kernel launches: the
 * vocabulary scan with the gate and the row merges, then the pair scores and
 * walks.  The plan knob DF2_PLAN_LAUNCHES can move the row merges into the
 * second launch or fuse everything into one; the results are the same bits
 * in every plan.
 *   logits   [B, P, V]   drafter logits U_t
 *   hidden   [B, P, d]   drafter hidden states h_t
 *   A_tab    [V, r]      predecessor embeddings A(.)
 *   B_tab    [V, r]      candidate embeddings B(.)
 *   W_H      [r, d]      gate map, H_t = W_H h_t
 *   prev_tok [B] int32   last verified token of each sequence
 *   K        candidates per position, 1 <= K <= min(V, 64) (the pages use 16)
 *   out_path  [B, P] int32   selected token at each draft position
 *   out_score [B] float      score of the selected path, sum_t S_t (fp32)
 * Arithmetic: inputs are read exactly; H and S accumulate in fp32.  With
 * bf16 tables the products G = A(a) (.) H_t enter the matrix cores as a bf16
 * high part plus a bf16 low part (about 16 significant bits, a relative
 * error near 2^-16 per product); B(b) is exact.  fp32 tables use the fp32
 * matrix instruction throughout.
 */
df2_status dflash2_select(const df2_dims* dims, const void* logits,
                          const void* hidden, const void* A_tab,
                          const void* B_tab, const void* W_H,
                          const int32_t* prev_tok, int32_t K,
                          int32_t* out_path, float* out_score,
                          hipStream_t stream);

/*
 * dflash2_select with a choice of walk (same section; see df2_walk).
 * Arguments as for dflash2_select; `walk` outside df2_walk is DF2_EINVAL.
 * dflash2_select is this call with DF2_WALK_VITERBI.
 */
df2_status dflash2_select_walk(const df2_dims* dims, const void* logits,
                               const void* hidden, const void* A_tab,
                               const void* B_tab, const void* W_H,
                               const int32_t* prev_tok, int32_t K,
                               df2_walk walk, int32_t* out_path,
                               float* out_score, hipStream_t stream);

/*
 * dflash2_select with the sampling walk (same section: sampling draws from
 * the same scores).  From the last verified token, position t draws its
 * candidate from the softmax of the pair scores of the token chosen at
 * t - 1 (row 0 at t = 0), at the given temperature:
 *     q_t(j) = exp((S_t(i, j) - max_k S_t(i, k)) / temperature) / (sum over k)
 *     j_t    = the first j whose running sum q_t(0) + ... + q_t(j) exceeds
 *              u[b][t] (running sums in rank order; the last j with
 *              q_t(j) > 0 if rounding leaves none).
 *   temperature  > 0 and finite, 1 / temperature finite in fp32 (else DF2_EINVAL)
 *   u         [B, P] float  caller's uniforms in [0, 1) (values outside are
 *                           clamped into it, NaN to 0); the library draws
 *                           no random numbers itself
 *   out_path  [B, P] int32  drawn token at each position
 *   out_q     [B, P] float  q_t(j_t): the draft probability of each drawn
 *                           token, for rejection sampling against the target
 *   out_score [B] float     sum_t S_t(j_{t-1}, j_t), added in order of t
 * Other arguments as for dflash2_select; u and out_q 4-byte aligned.
 * Arithmetic: fp32 (expf); scores must be finite.
 */
df2_status dflash2_select_sample(const df2_dims* dims, const void* logits,
                                 const void* hidden, const void* A_tab,
                                 const void* B_tab, const void* W_H,
                                 const int32_t* prev_tok, int32_t K,
                                 float temperature, const float* u,
                                 int32_t* out_path, float* out_q,
                                 float* out_score, hipStream_t stream);

/*
 * dflash2_select that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid it).  Same arguments, arithmetic and results as
 * dflash2_select (the same kernels), but its scratch is a static device
 * array of 48 MiB (50331648 bytes) that each GPU holds from module load
 * until the process ends; the first call on a device looks up its address.
 * Every call on one GPU shares that array: calls that overlap in time on a
 * GPU (different streams, or threads) race and must be serialised by the
 * caller.  Each call clears the array's arrival counters with a small
 * kernel before its own launches (no memset, no allocation).  A problem
 * whose scratch exceeds 48 MiB returns DF2_EUNSUPPORTED before anything is
 * enqueued (the stress shape B = 256, P = 15, V = 262144, K = 32 needs about
 * 40 MB).  Its device flags are reported by dflash2_device_error().
 */
df2_status dflash2_select_noalloc(const df2_dims* dims, const void* logits,
                                  const void* hidden, const void* A_tab,
                                  const void* B_tab, const void* W_H,
                                  const int32_t* prev_tok, int32_t K,
                                  int32_t* out_path, float* out_score,
                                  hipStream_t stream);

/*
 * Top-K of each row ("keep the top 16 candidates at each position").
 *   logits  [rows, V] (dtype)
 *   out_idx [rows, K] int32  candidate token ids, best first
 *   out_val [rows, K] float  their logits widened to fp32 (a -0 logit is
 *                            returned as +0)
 * 1 <= K <= min(V, 64).  rows == 0 enqueues nothing.
 */
df2_status dflash2_topk(const void* logits, int64_t rows, int32_t V,
                        df2_dtype dtype, int32_t K, int32_t* out_idx,
                        float* out_val, hipStream_t stream);

/*
 * The drafter's LM head fused with top-K ("DFlash 2: Keep Drafting
 * Parallel", section "A Lightweight Path Selector": the selector works on
 * the drafter's own logits and needs no extra LM-head pass).  For each row m
 *     U(m, v) = sum_k W_lm[v][k] * hidden[m][k]      (v = 0 .. V-1)
 * is computed on the matrix cores (bf16 products, exact in fp32, summed in
 * fp32) and only its top K leave the chip: the [M, V] logits are never
 * written to memory.  The outputs are those of dflash2_topk applied to the
 * fp32 logits, and feed dflash2_pair_scores like its outputs do.
 *   hidden  [M, d] bf16   final hidden state of each draft position
 *   W_lm    [V, d] bf16   LM-head weight, one row per token
 *   out_idx [M, K] int32  candidate token ids, best first
 *   out_val [M, K] float  their fp32 logits (a -0 logit is returned as +0)
 * dtype must be DF2_BF16 (DF2_F32 returns DF2_EUNSUPPORTED).  1 <= K <=
 * min(V, 64); V <= 2^29; d a multiple of 64 in [64, 32768]; M <= 2^24
 * (M == 0 enqueues nothing); hidden and W_lm 16-byte aligned, outputs
 * 4-byte aligned.
 * Top-K order as everywhere (value descending, equal values to the lower
 * index); the fp32 sums differ from exact ones by at most a few units in
 * the last place of sum_k |W_lm[v][k] hidden[m][k]|, so near-equal logits at
 * the K-th place may order differently than in exact arithmetic.
 * Non-finite hidden states or weights are outside the contract.  The
 * per-range candidate lists go through the library's scratch.
 */
df2_status dflash2_lmhead_topk(const void* hidden, const void* W_lm, int64_t M, int32_t V,
                               int32_t d, df2_dtype dtype, int32_t K, int32_t* out_idx,
                               float* out_val, hipStream_t stream);

/*
 * Gate projection H = W_H h for M rows ("DFlash 2: Keep Drafting Parallel",
 * section "A Lightweight Path Selector": the context gate H(h_t) of the
 * drafter state, whose formula the page cuts off; read as a bias-free
 * linear map d -> r).
 *   hidden [M, d] (dtype), W_H [r, d] (dtype), out_H [M, r] float
 * d multiple of 32, r multiple of 64 and <= 1024; hidden, W_H and out_H
 * 16-byte aligned.  H is rounded exactly as inside dflash2_select (the same
 * slices of d, summed in the same order).
 */
df2_status dflash2_project(const void* hidden, const void* W_H, int64_t M,
                           int32_t d, int32_t r, df2_dtype dtype, float* out_H,
                           hipStream_t stream);

/*
 * Pair scores of the selector equation for every adjacent candidate pair
 * (same section: S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >, every
 * adjacent pair scored at once).
 *   cand_idx [B, P, K] int32, cand_val [B, P, K] float (from dflash2_topk)
 *   H        [B, P, r] float (from dflash2_project)
 *   A_tab, B_tab [V, r] (dims->dtype), prev_tok [B] int32
 *   out_S    [B, P, K, K] float, out_S[b][t][i][j] = S_t(pred_i, cand_j)
 * The predecessor of rank i at t >= 1 is cand_idx[b][t-1][i]; at t == 0
 * every row uses prev_tok[b], so all K rows of t == 0 are equal.
 * dims->d is ignored.
 */
df2_status dflash2_pair_scores(const df2_dims* dims, const int32_t* cand_idx,
                               const float* cand_val, const float* H,
                               const void* A_tab, const void* B_tab,
                               const int32_t* prev_tok, int32_t K,
                               float* out_S, hipStream_t stream);

/*
 * The walk alone (same section: the one sequential step is a walk over the
 * precomputed scores from the last verified token), read as a max-sum pass
 * over S plus backtrack.
 *   S        [B, P, K, K] float (row 0 of t == 0 is used)
 *   cand_idx [B, P, K] int32
 *   out_path [B, P] int32, out_score [B] float
 */
df2_status dflash2_viterbi(const float* S, const int32_t* cand_idx, int32_t B,
                           int32_t P, int32_t K, int32_t* out_path,
                           float* out_score, hipStream_t stream);

/*
 * The walk alone, either mode (see df2_walk; same section: the walk over
 * the precomputed scores, max-sum or greedy).  Arguments as for
 * dflash2_viterbi, which is this call with DF2_WALK_VITERBI; 1 <= P <= 64,
 * 1 <= K <= 64; S, cand_idx, out_path and out_score 4-byte aligned.
 */
df2_status dflash2_walk(const float* S, const int32_t* cand_idx, int32_t B,
                        int32_t P, int32_t K, df2_walk walk, int32_t* out_path,
                        float* out_score, hipStream_t stream);

/*
 * The sampling walk alone (see dflash2_select_sample; same section:
 * sampling draws from the same scores) over given scores.
 *   S [B, P, K, K] float, cand_idx [B, P, K] int32, as for dflash2_walk;
 *   u [B, P] float uniforms, temperature, out_path [B, P] int32,
 *   out_q [B, P] float, out_score [B] float.
 */
df2_status dflash2_sample_walk(const float* S, const int32_t* cand_idx,
                               const float* u, int32_t B, int32_t P, int32_t K,
                               float temperature, int32_t* out_path,
                               float* out_q, float* out_score,
                               hipStream_t stream);

/*
 * Uniforms for the sampling walk, drawn on the device from a counter-based
 * generator (same section: sampling draws from the same scores, one uniform
 * per draft position), so a serving loop need not bring them from the host.
 * The generator is Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC 2011):
 *     out[i] = (x >> 40) * 2^-24,  x = word (i mod 4) of
 *              Philox4x64-10(counter = (i / 4, offset, 0, 0), key = (seed, 0))
 * exact in fp32 and in [0, 1); the values depend on (seed, offset, i) only.
 * Advance `offset` once per draft-verify cycle and pass the [B, P] result
 * as dflash2_select_sample's u (same stream).  seed and offset are kernel
 * arguments: a call captured into a HIP graph replays the same uniforms
 * every time (dflash2_philox_uniforms_next keeps the offset on the device
 * for that case).
 *   n    number of uniforms, 0 <= n <= 2^31 (n == 0 enqueues nothing;
 *        n < 0 is DF2_EINVAL, n > 2^31 DF2_EUNSUPPORTED)
 *   out  [n] float, device memory owned by the caller, 4-byte aligned
 *        (16-byte alignment lets whole blocks go out in one store)
 */
df2_status dflash2_philox_uniforms(uint64_t seed, uint64_t offset, int64_t n,
                                   float* out, hipStream_t stream);

/*
 * dflash2_philox_uniforms with the offset kept in device memory, for a
 * serving loop that replays a captured HIP graph: the uniforms use the
 * value *offset holds when the launch runs, then a second launch on the same
 * stream adds one to it, so every replay draws the next cycle's uniforms.
 * Nothing is allocated and no memset is enqueued.
 *   offset  [1] uint64, device memory owned by the caller, 8-byte aligned;
 *           calls that share it must be ordered (same stream)
 * Other arguments as for dflash2_philox_uniforms; n == 0 enqueues nothing
 * and leaves *offset as it is.
 */
df2_status dflash2_philox_uniforms_next(uint64_t seed, uint64_t* offset,
                                        int64_t n, float* out,
                                        hipStream_t stream);

/*
 * Two-tap dynamic depthwise convolution of the block drafter ("DFlash 2:
 * Keep Drafting Parallel", section "A Lightweight Local Convolution"),
 * applied around each attention and feed-forward sublayer:
 *     y_t[c] = k_{t,0}[c] x_t[c] + k_{t,1}[c] x_{t-1}[c],   x_{-1} = x_prev,
 *     k_{t,tap}[c] = base[tap][c] + corr_t[tap][c / 16],
 *     corr_t[tap][g] = sum_m W_c[tap][g][m] x_t[m].
 * The pages give a learned base plus a correction from the current hidden
 * state shared by 16 channels; the correction's form is this library's
 * reading (a bias-free linear map of x_t).
 *   x      [B, P, d]     (dtype) sublayer input at the draft positions
 *   x_prev [B, d]        (dtype) the same for the last verified token
 *   base   [2, d]        (dtype) base kernel, tap 0 (current) then tap 1 (previous)
 *   W_c    [2, d/16, d]  (dtype) correction map
 *   out    [B, P, d]     (dtype) y; fp32 arithmetic, bf16 output rounded to
 *                        nearest even; must not overlap x or x_prev
 * B >= 0 (B == 0 enqueues nothing), P >= 1, d a multiple of 512 in
 * [512, 8192]; every pointer 16-byte aligned.  The corrections go through
 * the library's scratch (as dflash2_project's partials do).
 */
df2_status dflash2_conv2(const void* x, const void* x_prev, const void* base,
                         const void* W_c, int32_t B, int32_t P, int32_t d,
                         df2_dtype dtype, void* out, hipStream_t stream);

/*
 * Waits for `stream`, then reports and clears the device-side flags of its
 * scratch buffer and of the current device's no-allocation scratch: *flags
 * receives a bit mask (bit 0: a prev_tok outside
 * [0, V) was replaced by 0; bit 1: a cand_idx entry outside [0, V) was
 * replaced by 0; bit 2: a row merge of dflash2_select gave up waiting for
 * its gate rows (launches 1 or 2 only), which only a fault elsewhere can
 * cause, and its scores are then unreliable).  A raised flag can leave a late gate arrival
 * counted in the stream's scratch, so after reporting one the next call on
 * that stream clears all its arrival counters before it launches.  Returns
 * DF2_OK, or DF2_EHIP.
 */
df2_status dflash2_device_error(hipStream_t stream, uint32_t* flags);

/*
 * Pins one plan knob for every later call of this process (value 0 restores
 * the automatic choice), for measurement and plan-invariance tests.  Values
 * out of a knob's range are clamped to what the shapes allow.  Returns
 * DF2_EINVAL for an unknown knob or a negative value.  Not for use while
 * another thread is enqueueing selector work.
 */
df2_status dflash2_plan_override(df2_plan_knob knob, int32_t value);

/* Frees every scratch buffer the library holds (call with no work in flight). */
df2_status dflash2_release(void);

/* Static description of a status code. */
const char* dflash2_status_string(df2_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* dflash2_last_error(void);

/* Library version, "major.minor.patch". */
const char* dflash2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH2_H */
