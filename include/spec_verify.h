/*
 * spec_verify.h -- C ABI of the speculative-decoding verify round on one AMD
 * MI355X (gfx950).
 *
 * What the calls compute (the pages' definitions):
 *   - "Speculative decoding" (gpillon.github.io/ignis), "One round, step by
 *     step": each lane holds an anchor plus up to k drafts; all lanes' columns
 *     go through the target model once; per lane the longest run of drafts the
 *     model itself would have chosen is kept, plus the model's own next token
 *     (between 1 and k + 1 tokens); the state then moves forward by exactly
 *     that committed run, attention layers keeping every committed column's
 *     keys and recurrent layers replaying only the committed prefix.
 *   - The same page, "The row budget": drafts per lane =
 *     min(draft tokens, rows / lanes - 1), a budget of 0 meaning 8.
 *   - "Draft heads and speculative decoding" (research.strata2signal.com),
 *     "Guess, then check": the greedy walk; the textbook sampled rule it cites
 *     (Leviathan, Kalman & Matias 2022, Def. 3.7 / Thm. 3.8).
 *   - FreeToken tracking issue #828, "Per-request state": the verify forward
 *     only reads the live state and stages scratch; commit rolls the state to
 *     the accepted count; a model whose recurrent state has no buffer is
 *     refused.
 *
 * Conventions shared by every call:
 *   - Status: SPEC_OK (0) or a negative SPEC_E_* code.  All arguments are
 *     validated on the host BEFORE anything is enqueued, so an error leaves
 *     every caller buffer untouched.  A HIP launch failure returns SPEC_E_HIP;
 *     an asynchronous device fault surfaces at the caller's next stream sync.
 *   - Ownership: the caller owns every device buffer (weights, KV pools, block
 *     tables, state, workspace, outputs).  The library never allocates or
 *     frees device memory; it owns only the host-side spec_model object.
 *   - Streams: `stream` is a hipStream_t passed as void*; NULL is the default
 *     stream.  Work is enqueued asynchronously, with no implicit
 *     synchronisation, no memset nodes and no host<->device copies.  The LM
 *     head of a sampled round of a bf16 model is one cooperative launch (one
 *     workgroup per compute unit, all resident at once); every other launch is
 *     an ordinary kernel launch.
 *   - Rows of a round are packed lane-major: lane l owns rows
 *     [row_start(l), row_start(l) + cols[l]) with row_start(l) = sum of cols of
 *     lanes before l; column 0 is the anchor, column j >= 1 is draft d_j.
 *   - Numerics are batch-invariant: every reduction order is fixed by the
 *     model shape and by absolute positions, never by the number of rows or
 *     lanes in the round, so a row's results do not depend on the other rows.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_MAX_ROWS 64   /* rows of one round, summed over lanes */
#define SPEC_MAX_COLS 16   /* columns of one lane: the anchor plus up to 15 drafts */
#define SPEC_MAX_LANES 64
#define SPEC_KV_BLOCK 16   /* tokens per paged-KV block */

enum spec_status {
  SPEC_OK = 0,
  SPEC_E_INVAL = -1,        /* malformed argument */
  SPEC_E_RANGE = -2,        /* the round does not fit the lane's block table */
  SPEC_E_UNSUPPORTED = -3,  /* shape or combination this build does not run */
  SPEC_E_WORKSPACE = -4,    /* workspace missing or too small */
  SPEC_E_HIP = -5,          /* a HIP runtime call failed */
  SPEC_E_SCRATCH = -6       /* the round needs more than the library's static scratch */
};

enum spec_dtype { SPEC_F32 = 0, SPEC_BF16 = 1 };
enum spec_layer_kind { SPEC_LAYER_ATTN = 0, SPEC_LAYER_GDN = 1 };
enum spec_mode { SPEC_GREEDY = 0, SPEC_SAMPLED = 1 };

/* Kernel classes that spec_profile_enable can time. */
enum spec_kernel_class {
  SPEC_K_NONE = -1,
  SPEC_K_PROJ_IN = 0,   /* QKV / gated-delta-rule input projection */
  SPEC_K_ATTN = 1,      /* verify attention */
  SPEC_K_PROJ_O = 2,    /* attention / recurrent output projection */
  SPEC_K_GATE_UP = 3,   /* SwiGLU gate+up projection */
  SPEC_K_DOWN = 4,      /* MLP down projection */
  SPEC_K_LM_HEAD = 5,   /* fused LM head statistics */
  SPEC_K_GDN = 6,       /* gated-delta-rule column recurrence */
  SPEC_K_COUNT = 7
};

/* Weights of one decoder layer.  Device pointers to [out][in] matrices, element
 * type = the model dtype unless noted; borrowed, never freed by the library.
 * An f32 model passes them row-major.  A bf16 model passes every matrix in the
 * fragment layout written by spec_pack_weight (the embedding table excepted).
 *   norm1, norm2: float [hidden] RMSNorm gains.
 *   w_in:   full attention: [(n_q + 2 n_kv) * head_dim][hidden], rows = q heads,
 *           then k heads, then v heads;
 *           gated delta rule: [3 * gdn_heads * gdn_dim + 2 * gdn_heads][hidden],
 *           rows = q, k, v (head-major), then one alpha row and one beta row per head.
 *   w_o:    [hidden][n_q * head_dim]  or  [hidden][gdn_heads * gdn_dim].
 *   w_gate, w_up: [ffn][hidden];  w_down: [hidden][ffn]. */
typedef struct {
  const float* norm1;
  const void* w_in;
  const void* w_o;
  const float* norm2;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
} spec_layer_weights;

/* Model description (copied by spec_model_create; pointers are borrowed).
 * Decoder: RMSNorm -> (GQA attention with rotate-half RoPE | gated delta rule)
 * -> residual; RMSNorm -> SwiGLU MLP -> residual; final RMSNorm -> LM head.
 * Gated delta rule (Yang et al. 2024): alpha = sigmoid(h.w_alpha),
 * beta = sigmoid(h.w_beta), q = q~/|q~| * d^-1/2, k = k~/|k~|,
 * S_t = alpha S + beta (v - alpha S k) k^T, o_t = S_t q_t. */
typedef struct {
  int n_layers;            /* >= 0; 0 = LM head only (spec_verify_head) */
  int hidden;              /* multiple of 4 (bf16: of 256), <= 8192 */
  int n_q_heads, n_kv_heads, head_dim;   /* head_dim 128 (bf16) or <= 128 and a multiple of 8 (f32) */
  int ffn;                 /* multiple of 32 */
  int vocab;               /* multiple of 16 */
  int dtype;               /* SPEC_F32 | SPEC_BF16: weights, KV, stored activations */
  const int32_t* layer_kind;   /* host [n_layers]: SPEC_LAYER_ATTN | SPEC_LAYER_GDN */
  int gdn_heads, gdn_dim;  /* gdn_dim 128 when any layer is SPEC_LAYER_GDN */
  float rms_eps;           /* e.g. 1e-6 */
  float rope_theta;        /* 0 = no positional encoding */
  int kv_block;            /* must be SPEC_KV_BLOCK */
  int attn_chunk;          /* positions per split-KV chunk (multiple of 256, <= 4096); 0 = 512 */
  const void* embed;       /* [vocab][hidden] row-major; may be NULL for a head-only model */
  const void* lm_head;     /* [vocab][hidden]: row-major (f32) or packed (bf16) */
  const float* final_norm; /* [hidden]; may be NULL for a head-only model */
  const spec_layer_weights* layers;   /* host [n_layers] */
  /* Sliding-window targets (FreeToken issue, "Design": sliding-window targets; the
   * Gemma 4 assistant thread): sliding_window = 0 is full attention; W > 0 makes a row
   * at position P of a windowed attention layer attend to positions P - W + 1 .. P
   * only.  window_global_every = g > 0 keeps full attention in attention layers g - 1,
   * 2g - 1, ... (counted among the attention layers); 0 windows every attention layer.
   * Both >= 0, else SPEC_E_INVAL. */
  int sliding_window;
  int window_global_every;
} spec_model_desc;

typedef struct spec_model spec_model;

/* One verify round.  Device buffers are read (and, by spec_commit, written)
 * asynchronously on the stream; host arrays are read during the call only.
 *
 * Paged KV layout (element type = model dtype), per full-attention layer a
 * slice of n_blocks blocks, layers in order:
 *   k_pool [n_attn_layers][n_blocks][n_kv][16 slots][head_dim]
 *   v_pool [n_attn_layers][n_blocks][n_kv][head_dim][16 slots]
 * Token position p of lane l lives in block block_table[l * max_blocks + p/16],
 * slot p % 16.  Block ids must lie in [0, n_blocks); kernels clamp others.
 * Recurrent state (float): gdn_state [lanes][n_gdn_layers][gdn_heads][dv][dk]. */
typedef struct {
  int lanes;                   /* 1 .. SPEC_MAX_LANES */
  const int32_t* cols_host;    /* host [lanes]: k_l + 1 in [1, SPEC_MAX_COLS]; sum <= SPEC_MAX_ROWS */
  const int32_t* tokens;       /* device [R]: anchor then drafts per lane, lane-major */
  int32_t* kv_len;             /* device [lanes]: committed length; the anchor sits at position kv_len */
  const int32_t* kv_len_host;  /* host [lanes] mirror for the capacity check; NULL skips it */
  const int32_t* block_table;  /* device [lanes][max_blocks] */
  int max_blocks;              /* block-table width; capacity = 16 * max_blocks positions */
  void* k_pool;                /* device; NULL iff the model has no attention layer */
  void* v_pool;
  int n_blocks;                /* blocks per layer slice of the pools */
  float* gdn_state;            /* device; NULL iff the model has no recurrent layer */
  int mode;                    /* SPEC_GREEDY | SPEC_SAMPLED */
  float temperature;           /* sampled: > 0; p = softmax(z / T) */
  const float* q_probs;        /* sampled: device [R][vocab], row of column j >= 1 = the
                                  drafter's q for draft d_j (column-0 rows unused) */
  uint64_t seed;               /* Philox4x32-10 key */
  void* workspace;             /* device, >= spec_workspace_bytes; 256-byte aligned */
  size_t workspace_bytes;
  /* Per-row presence and frequency penalties (the FreeToken issue, "Design": per-row
   * penalties in target-side verify).  counts: device int32 [lanes][vocab], each lane's
   * token counts up to and including its anchor, or NULL for no penalties.  Row j of a
   * lane conditions on those tokens and on its drafts d_1 .. d_j, so a token seen c times
   * there loses presence * [c > 0] + frequency * c from its logit before every statistic
   * and decision (argmax, softmax at T, the textbook rule, the residual and bonus draws).
   * With counts, both penalties must be finite and counts 16-byte aligned, else
   * SPEC_E_INVAL.  spec_counts_add
   * keeps counts current after each commit. */
  const int32_t* counts;
  float presence_penalty;
  float frequency_penalty;
} spec_round;

/* Per-row statistics of the LM head (T = 1 in greedy mode). */
typedef struct {
  float max_logit;   /* max_v z_v */
  float lse;         /* log sum_v exp(z_v / T) */
  int32_t argmax;    /* lowest index among the maxima */
  float z_next;      /* z at the row's next draft token; NaN on a lane's last row */
} spec_row_stat;

const char* spec_status_string(int status);

/* Row-budget planner ("The row budget", gpillon.github.io/ignis):
 * returns min(k, max(0, rows / lanes - 1)) with integer division and rows =
 * row_budget, or 8 when row_budget == 0.  Errors (lanes <= 0, k < 0,
 * row_budget < 0) return SPEC_E_INVAL.  Pure host function. */
int spec_plan_drafts(int k, int row_budget, int lanes);

/* Validates and copies a model description into a host object.  No HIP call. */
int spec_model_create(const spec_model_desc* desc, spec_model** out);
void spec_model_destroy(spec_model* model);

/* Workspace bytes for rounds of up to max_lanes lanes, max_cols columns per lane
 * and block tables max_blocks wide.  Returns a negative status on error.  The
 * workspace also carries the staged columns from spec_verify_round to
 * spec_commit: pass the same workspace, unmodified, to the calls of one round. */
int64_t spec_workspace_bytes(const spec_model* model, int max_lanes, int max_cols, int max_blocks);

/* The verify forward: every row through every layer once, then the fused LM
 * head's per-row statistics (logits are never written to memory).  Reads the
 * KV pools and recurrent state, writes neither; stages each column's K/V and
 * recurrent inputs in the workspace.
 * Sampled rounds of a bf16 model: the textbook rule needs a row's whole
 * normaliser before any residual weight is known ("Draft heads and speculative
 * decoding", "Guess, then check").  The LM head is then one cooperative launch
 * whose workgroups keep their vocabulary slices' logits on chip across two grid
 * barriers: they reduce the row statistics, take every lane's accept/reject
 * decision and run each lane's draw (the residual race on a rejected row, the
 * bonus race when every draft is kept) on the logits they still hold; the
 * workspace receives only per-workgroup partials.  This needs vocab / 16 <= 64
 * per compute unit (vocab <= 262144 on 256 compute units) and vocab * hidden * 2
 * <= 2^31, else SPEC_E_UNSUPPORTED.
 * Errors: SPEC_E_INVAL (lanes, cols, NULL buffers, sampled without q_probs or
 * with T <= 0), SPEC_E_RANGE (kv_len_host + cols exceeds 16 * max_blocks),
 * SPEC_E_UNSUPPORTED (recurrent layers with gdn_state == NULL; a lane whose
 * cols x (n_q_heads / n_kv_heads) query rows exceed 64; the sampled bf16 head
 * limits above), SPEC_E_WORKSPACE. */
int spec_verify_round(const spec_model* model, const spec_round* round, void* stream);

/* The LM head and row statistics alone, on caller-given final hidden states
 * `hidden` (device [R][hidden], model dtype; no final norm is applied).  Same
 * round fields as spec_verify_round except the KV/state ones, which are unused. */
int spec_verify_head(const spec_model* model, const spec_round* round, const void* hidden,
                     void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation: spec_verify_head followed by
 * spec_accept in one call, with the library's own static device scratch in place of
 * round->workspace (ignored; may be NULL).  The scratch is one 16 MiB array per GPU,
 * held from the first such call on that GPU until the process ends; a round whose
 * head-only buffers (hidden rows, LM-head and race partials, row statistics) exceed it
 * returns SPEC_E_SCRATCH before anything is enqueued.  Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (several streams or threads at once)
 * race: the caller serialises them.  The call allocates nothing (no hipMalloc, no
 * hipFree).  Arguments and outputs as spec_verify_head and spec_accept; the results
 * equal theirs. */
int spec_verify_head_noalloc(const spec_model* model, const spec_round* round, const void* hidden,
                             int32_t* committed, int32_t* out_tokens, spec_row_stat* row_stats,
                             void* stream);

/* Acceptance.  Greedy: per lane the longest prefix of drafts equal to the
 * argmax of the row before, then the argmax at the first mismatch (or after the
 * last draft).  Sampled: draft d_i is kept iff u * q_i(d_i) < p_{i-1}(d_i), with
 * u the Philox uniform at (seed, position kv_len + i, lane); on the first
 * rejection the token is drawn from max(0, p - q) by an exponential race;
 * with every draft kept the bonus token is drawn from p_k.
 * Outputs (device): committed[lanes] in [1, cols]; out_tokens[lanes][SPEC_MAX_COLS]
 * holds the committed run (kept drafts, then the model's token); row_stats
 * [R] (may be NULL).  Must follow spec_verify_round / spec_verify_head of the
 * same round and workspace.  In a sampled round of a bf16 model the head has
 * already decided (see spec_verify_round) and this call only gathers the
 * outcome; committed[l] = 0 there marks a round whose head could not
 * synchronise its workgroups (a bounded grid-barrier wait ran out, which a
 * cooperative launch with every workgroup resident does not reach): the
 * round's outputs are invalid and must be discarded. */
int spec_accept(const spec_model* model, const spec_round* round, int32_t* committed,
                int32_t* out_tokens, spec_row_stat* row_stats, void* stream);

/* Commit: for each lane copies the staged K/V of columns 0 .. committed-1 into
 * the paged cache at positions kv_len .. kv_len + committed - 1, replays the
 * same columns through the recurrent state, then kv_len += committed.
 * committed is read on the device (no host round trip); values are clamped to
 * [1, cols].  Rejected columns leave no trace. */
int spec_commit(const spec_model* model, const spec_round* round, const int32_t* committed,
                void* stream);

/* Tests only: the verify forward, then the full logits float [R][vocab]. */
int spec_debug_logits(const spec_model* model, const spec_round* round, float* logits,
                      void* stream);

/* Tests and measurement: the skinny projection kernel alone, Y[R][N] = X[R][K] W[N][K]^T
 * (Y float), with the split and launch shape the round uses for an [N][K]
 * weight.  X is row-major in the model dtype and taken as exact (one bf16
 * plane; inside a round a bf16 model's float32 activations enter the same
 * kernel as two planes).  W: packed (bf16) or row-major (f32).
 * R <= SPEC_MAX_ROWS; bf16 needs K % 256 == 0.  A bf16 model needs a workspace
 * of at least 32 ceil(R / 16) K + 4 S R N bytes (S <= K / 256 the split, 256-byte
 * aligned), else SPEC_E_WORKSPACE. */
int spec_debug_gemm(const spec_model* model, const void* X, const void* W, float* Y, int R,
                    int N, int K, void* workspace, size_t workspace_bytes, void* stream);

/* Weight fragment layout of a bf16 model.  A row-major bf16 matrix [N][K]
 * (K % 256 == 0) is stored as 1 KB fragments of 16 rows x 32 consecutive k:
 * fragment (g, s) (g = row tile, s = k / 32) starts at element (g * K/32 + s) * 512,
 * and within it lane i (0..63) holds the 8 elements
 * [16 g + i % 16][32 s + 8 (i / 16) + e], e = 0..7 -- exactly the operand one
 * lane feeds to a 16x16x32 bf16 MFMA, so a wave loads it as 1 KB contiguous.
 * Rows past N are zero.  spec_packed_weight_bytes returns the size
 * (32 ceil(N / 16) K bytes) or SPEC_E_INVAL; spec_pack_weight converts
 * device src (row-major) into device dst (distinct buffers, the caller's) on
 * the stream. */
int64_t spec_packed_weight_bytes(int N, int K);
int spec_pack_weight(const void* src, void* dst, int N, int K, void* stream);

/* Out-of-window frees of a sliding-window target (FreeToken issue, "Design": each
 * request frees the slots whose interval has slid out of the window).  Returns the
 * first cache block (index into the lane's block_table row) that a verify round at
 * committed length kv_len reads in an attention layer of window W > 0; the round never
 * reads or dereferences the table entries below it, and since kv_len only grows they
 * stay unread, so the caller may release and reuse those blocks -- when every attention
 * layer of the model is windowed and shares that table.  Rejected columns never reach
 * the cache (spec_commit writes only committed ones), so rejection frees nothing.
 * window == 0: returns 0 (nothing may be freed).  kv_len < 0 or window < 0:
 * SPEC_E_INVAL.  Host only. */
int spec_window_live_block(int kv_len, int window);

/* counts[l][t] += 1 for every token t of lane l's committed run, out_tokens[l][0 ..
 * committed[l]) (device, row stride out_stride), after spec_accept: the counts that
 * spec_round.counts expects for the next round (tokens up to the new anchor).  Tokens
 * outside [0, vocab) are skipped.  Device buffers, the caller's; lanes in [1,
 * SPEC_MAX_LANES], vocab >= 1, out_stride >= 1, else SPEC_E_INVAL. */
int spec_counts_add(int32_t* counts, int vocab, int lanes, const int32_t* committed,
                    const int32_t* out_tokens, int out_stride, void* stream);

/* Copy-from-the-conversation drafter (n-gram prompt lookup): "Speculative decoding",
 * mashbox docs, "Where it runs" (--speculation ngram: the drafter looks up the last few
 * tokens earlier in the request and proposes the tokens that followed them there).
 * history: device int32 [lanes][max_len], lane l's tokens so far in history[l][0 ..
 * hist_len[l]), the last one being the lane's anchor (the token at position kv_len).
 * For n = n_max down to n_min the suffix of length n is looked up; the most recent
 * earlier occurrence (largest p with p + n < len) of the longest suffix that recurs is
 * copied: draft i is the token at p + n + i of the history extended by the drafts (a
 * copy that reaches the end goes on over what it has just proposed).  Output, device:
 * tokens [lanes][k + 1] = the anchor, then k drafts (the anchor repeated when no suffix
 * recurs, so every lane keeps k + 1 columns), lane-major as spec_round.tokens expects;
 * n_match [lanes] = the matched n, 0 for none.  A lane with hist_len < 1 gets token 0
 * columns.  1 <= lanes <= SPEC_MAX_LANES, 0 <= k < SPEC_MAX_COLS,
 * 1 <= n_min <= n_max <= SPEC_MAX_NGRAM, max_len >= 1, else SPEC_E_INVAL.  All buffers
 * are the caller's; the call only enqueues work on the stream. */
#define SPEC_MAX_NGRAM 8
int spec_ngram_draft(const int32_t* history, const int32_t* hist_len, int lanes, int max_len, int k,
                     int n_max, int n_min, int32_t* tokens, int32_t* n_match, void* stream);

/* The history update of a multi-round loop (the round's committed run, "One round, step
 * by step", ignis, step 5): after spec_accept and spec_commit, lane l's out_tokens[l][0
 * .. committed[l]) (device, row stride out_stride) are appended to history[l] and
 * hist_len[l] grows by committed[l], both capped at max_len.  Device buffers, the
 * caller's; lanes in [1, SPEC_MAX_LANES], out_stride >= 1, else SPEC_E_INVAL.  With
 * spec_ngram_draft this makes a loop of rounds that never waits for the host. */
int spec_history_append(int32_t* history, int32_t* hist_len, int lanes, int max_len,
                        const int32_t* committed, const int32_t* out_tokens, int out_stride,
                        void* stream);

/* Per-request miss back-off of a drafter, host side ("Speculative decoding", mashbox
 * docs, "What it does for you": a request whose guesses keep missing stops guessing for
 * a while).  The engine runs several passes (verify rounds) per device call and decides
 * once per call who guesses:
 *  - spec_backoff_call at the start of a call: a request may guess unless it is waiting;
 *    the call speculates (returns 1, else 0) when some request may guess and the row
 *    budget (spec_plan_drafts(k, row_budget, n), n counting every active request)
 *    leaves it a draft; drafts[i] = that plan for a request that may guess in a call that
 *    speculates, 0 otherwise;
 *  - spec_backoff_pass after each pass of the call, kept[i] = the request's drafts the
 *    model kept (committed - 1).  In a call that speculates, every pass counts for each
 *    request that may guess: 4 passes in a row that keep nothing start a wait of 16
 *    passes (the count starts again), each further such 4 double it up to 256, and a pass
 *    that keeps a guess clears the count and sets the wait back to 16 -- unless the
 *    request is waiting: the rest of the call in which a wait began still guesses and
 *    its passes count toward the wait.  Every other pass only shortens a running wait.
 * States are caller-owned host memory, n in [1, SPEC_MAX_LANES]; spec_backoff_init sets
 * them to "not waiting, next wait 16".  Pure host functions (no device work); bad
 * arguments return SPEC_E_INVAL and change nothing. */
typedef struct {
  int32_t miss_run;    /* counted passes in a row that kept nothing, since the last wait began */
  int32_t wait_len;    /* length of the next wait, 16 .. 256 */
  int32_t wait_left;   /* passes of the current wait still to go, 0 when not waiting */
  int32_t may_guess;   /* 1 if the request may guess in the current call */
} spec_backoff;
int spec_backoff_init(spec_backoff* states, int n);
int spec_backoff_call(spec_backoff* states, int n, int k, int row_budget, int32_t* drafts);
int spec_backoff_pass(spec_backoff* states, int n, const int32_t* kept, int speculates);

/* Measurement: record HIP events around launches 0, every, 2 every, ... of one
 * kernel class, counted from this call (SPEC_K_NONE stops recording; every >= 1,
 * else SPEC_E_INVAL), and read back the summed duration and the number of the
 * launches recorded since the last enable (synchronises on those events).  Each
 * recorded launch pays for its two event records (a few microseconds of queue
 * gap), so a sparse stride keeps the measurement from slowing what it measures. */
int spec_profile_enable(spec_model* model, int kernel_class, int every);
int spec_profile_collect(spec_model* model, double* total_ms, int* launches);

/* Tests only: the number of polls a workgroup of the sampled bf16 head's cooperative
 * launch makes at each grid barrier before it gives up (default about a second of
 * polling; >= 0, else SPEC_E_INVAL).  A small limit lets a test force the failure path
 * from the host: a workgroup that gives up raises the launch's error flag and goes on,
 * every wave ends, and spec_accept reports committed[l] = 0 for every lane. */
int spec_debug_barrier_spin(spec_model* model, int polls);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
