/*
 * spec_verify.h -- C ABI of the block speculative-verification library
 * (MI355X / gfx950, HIP).
 *
 * The step it implements: a target model checks k_b draft tokens of every
 * sequence b in one pass over T_b = k_b + 1 verify tokens (the last committed
 * token followed by the drafts) and then keeps only the accepted prefix.
 * Sources: "InternLM/lmdeploy pull request 5019" (feature list: block
 * speculative verification with paged verification attention and gated
 * delta-rule verify / commit kernels; "Two fixes" item 2: the recurrent-state
 * commit after acceptance), "microsoft/onnxruntime-genai pull request 2457"
 * (commit messages: packed varlen operators with cu_seqlens, V-major fp32
 * GatedDeltaNet state, CommitPrefix of the accepted prefix with no snapshot,
 * one device argmax readback), "InternLM/lmdeploy pull request 3945" (review
 * of reject_sampler.py: output [batch, max_spec_len + 1] padded with -1).
 *
 * Conventions shared by every call
 *   - Every pointer is a DEVICE pointer unless marked "host".  The caller owns
 *     all memory; the library allocates nothing, keeps no state between calls
 *     and never synchronises the stream.  Every call only enqueues work on
 *     `stream` and returns; results are valid once the stream has run them.
 *   - Packed varlen rows: sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1
 *     of every [total_T, ...] tensor; its k_b = T_b - 1 drafts (and the per-
 *     draft uniforms / draft logits) are packed at rows cu_seqlens[b] - b ...
 *   - Host validation returns a status and never aborts; the text of the last
 *     non-OK status of the calling thread is sv_last_error().
 *   - `err` (nullable, device int32): kernels OR an SV_DERR_* bit into it when
 *     they meet bad device-resident input (a page id outside the pool, a
 *     context that overflows the block table, T_b outside 1..max_T, a commit
 *     length outside 0..T_b, a draft token outside 0..V-1, a state slot
 *     outside the bank); the affected
 *     sequence is then skipped: attention, GDN and short-conv calls leave its
 *     outputs, pages and states untouched (a bad page id anywhere in a
 *     sequence's block-table range skips the whole sequence, append
 *     included); acceptance writes accept_len -1, a row of -1 and commit
 *     length 0 for it and leaves its ctx_lens entry, so a commit or deferred
 *     replay that follows keeps its recurrent state.  The caller clears the
 *     word (sv_clear_device_error) and reads it (sv_read_device_error).
 *   - Calls that run on the same buffers must be ordered on one stream; two
 *     calls that share a workspace or a state / cache buffer must not overlap.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of this header are the only ones the library exports. */
#define SV_API __attribute__((visibility("default")))

typedef enum {
  SV_OK = 0,
  SV_EINVAL = 1,      /* a bad argument (null pointer, size, shape) */
  SV_EDTYPE = 2,      /* unsupported dtype / head size combination */
  SV_ECAPACITY = 3,   /* a size beyond what the kernels support */
  SV_EWORKSPACE = 4,  /* workspace missing or smaller than required */
  SV_EHIP = 5         /* the HIP runtime refused a launch */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1, SV_F16 = 2 /* GDN state only */ } sv_dtype;

/* Device error bits (see `err` above). */
#define SV_DERR_PAGE      1   /* block_table entry outside [0, num_pages) */
#define SV_DERR_CAPACITY  2   /* ctx_len + T_b > max_pages_per_seq * page_size */
#define SV_DERR_SEQLEN    4   /* T_b < 1 or T_b > max_T, or rows past total_T */
#define SV_DERR_COMMIT    8   /* commit length outside 0..T_b */
#define SV_DERR_TOKEN    16   /* draft token outside 0..V-1 */
#define SV_DERR_SLOT     32   /* state_slot entry outside [0, num_slots) */

/* One batch of packed varlen verify rows. */
typedef struct {
  int32_t B;                   /* host: number of sequences, >= 1 */
  int32_t max_T;               /* host: bound on every T_b, 1..8 */
  int32_t total_T;             /* host: cu_seqlens[B] */
  const int32_t* cu_seqlens;   /* [B+1], cu_seqlens[0] = 0 */
} sv_batch;

/* ------------------------------------------------------------------------
 * Paged verification attention with KV write-through.
 *
 * lmdeploy #5019 feature list (paged verification attention over a fixed
 * draft chain); lmdeploy #3945 review of flatten_kv_cache.py (paged K/V of a
 * sequence read back as a dense state).  For every sequence b, query head h,
 * verify token j < T_b and the GQA head g = h * Hkv / Hq:
 *   o[cu_b + j, h] = sum_p softmax_p(scale * q[cu_b+j, h] . K_b[p, g]) V_b[p, g]
 * over the L_b = ctx_lens[b] cached positions and the in-flight positions
 * L_b .. L_b + j (a chain: plain causal mask).  Logical position p of
 * sequence b lives in page block_table[b * max_pages_per_seq + p / page_size]
 * at slot p % page_size.  With write_kv = 1 the in-flight rows k_new / v_new
 * are also stored at positions L_b .. L_b + T_b - 1 (ctx_lens is NOT changed
 * here: the KV commit is the length update done after acceptance).
 *
 *   q            [total_T, Hq, D]           dtype
 *   k_new, v_new [total_T, Hkv, D]          dtype
 *   k_cache,
 *   v_cache      [num_pages, Hkv, page_size, D]  dtype, updated in place
 *   block_table  int32 [B, max_pages_per_seq]; entries past a sequence's
 *                last page are never read
 *   ctx_lens     int32 [B]
 *   out          [total_T, Hq, D]           dtype
 * dtype SV_BF16 (fp32 accumulation; D = 64 or 128; page_size a power of two
 * >= 16; Hq/Hkv * max_T <= 64) or SV_F32 (D <= 128).  scale = 0 means
 * 1/sqrt(D).  Workspace: spec_verify_attention_workspace_bytes(); it holds
 * the split-KV partials (fp32) and is scratch between calls.
 * ------------------------------------------------------------------------ */
SV_API size_t spec_verify_attention_workspace_bytes(int32_t B, int32_t total_T,
    int32_t Hq, int32_t Hkv, int32_t D, int32_t max_pages_per_seq,
    int32_t page_size, sv_dtype dtype);

SV_API sv_status spec_verify_attention(const sv_batch* batch,
    const void* q, const void* k_new, const void* v_new,
    void* k_cache, void* v_cache,
    const int32_t* block_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* ctx_lens, void* out,
    int32_t Hq, int32_t Hkv, int32_t D, sv_dtype dtype, float scale,
    int32_t write_kv, void* workspace, size_t workspace_bytes,
    int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The same verification attention over INT8 pages.
 *
 * onnxruntime-genai #2457, commit message on the MTP head and INT8 KV: the
 * main model's cache uses kv_cache_quant_type = int8_per_channel with scales
 * calibrated per attention layer.  Symmetric per-channel codes with a static
 * fp32 scale for every (KV head, channel), one set for K and one for V:
 *   code = clamp(round_half_even(x / s), -127, 127),   x ~ s * code
 * where x / s is the correctly rounded fp32 quotient of the row value (bf16,
 * widened exactly) and the scale.  The result is the attention of
 * spec_verify_attention over the dequantized cache; the in-flight rows are
 * ALWAYS written (their codes at L_b .. L_b + T_b - 1) and read back like
 * every other position, so they enter as their codes too.
 *
 *   q, k_new, v_new, out  bf16, shapes as above
 *   k_cache, v_cache      int8 [num_pages, Hkv, page_size, D], updated in place
 *   k_scale, v_scale      fp32 [Hkv, D], positive and finite (a zero or
 *                         non-finite scale gives saturated codes, no error)
 * Limits as for the bf16 path; every tensor 16-byte aligned.  Workspace:
 * spec_verify_attention_workspace_bytes(..., SV_BF16).
 * ------------------------------------------------------------------------ */
SV_API sv_status spec_verify_attention_kv8(const sv_batch* batch,
    const void* q, const void* k_new, const void* v_new,
    int8_t* k_cache, int8_t* v_cache, const float* k_scale, const float* v_scale,
    const int32_t* block_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* ctx_lens, void* out,
    int32_t Hq, int32_t Hkv, int32_t D, float scale,
    void* workspace, size_t workspace_bytes, int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gated delta-net recurrent state: verify and commit.
 *
 * Gated delta rule (Yang, Kautz & Hatamizadeh, ICLR 2025), per (b, h), state
 * S = state[slot_b, h] of shape [dv, dk] stored V-major in fp32
 * (onnxruntime-genai #2457, GatedDeltaNet state), gates pre-cast to fp32:
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   o_t = S_t q_t
 * Commit (lmdeploy #5019 "Two fixes" item 2; onnxruntime-genai #2457
 * CommitPrefix): with c_b = commit_len[b] in 0..T_b, the stored state becomes
 * S after the first c_b tokens (c_b = 0 leaves it as it was) -- the state a run
 * over only those tokens would leave.  No snapshot is taken.
 *
 *   mode SV_GDN_VERIFY_COMMIT  o for all T_b tokens; state stored at c_b
 *        SV_GDN_VERIFY_ONLY    o for all T_b tokens; commit_len unused
 *        SV_GDN_COMMIT_ONLY    first c_b tokens applied and stored; q, out unused
 *   state       [num_slots, H, dv, dk], updated in place, state_dtype SV_F32
 *               or SV_F16 (lmdeploy #5019 "Two fixes" item 2: the commit
 *               kernel takes a half-precision state and computes in float);
 *               all arithmetic is fp32, an fp16 state is rounded to nearest
 *               even once per store
 *   state_slot  int32 [B] (slot of sequence b) or NULL (slot b)
 *   q, k        [total_T, H, dk]  io_dtype;   v [total_T, H, dv] io_dtype
 *   alpha, beta fp32 [total_T, H]
 *   commit_len  int32 [B]
 *   out         [total_T, H, dv]  io_dtype
 *   pending     NULL, or the tokens a previous step accepted but did not yet
 *               write (deferred commit): its first pending->commit_len[b]
 *               tokens of sequence b are applied to the state before this
 *               call's tokens, and the state is then stored even in
 *               VERIFY_ONLY mode.  It must describe the same B sequences.
 * dk = 64 or 128; dv a multiple of 64 up to 256.  state, q, k, v (and the
 * pending k, v) must be 16-byte aligned; SV_EINVAL otherwise.
 * ------------------------------------------------------------------------ */
typedef enum {
  SV_GDN_VERIFY_COMMIT = 0,
  SV_GDN_VERIFY_ONLY = 1,
  SV_GDN_COMMIT_ONLY = 2
} sv_gdn_mode;

typedef struct {
  sv_batch batch;              /* the pending step's batch (same B) */
  const void* k;               /* [batch.total_T, H, dk] io_dtype */
  const void* v;               /* [batch.total_T, H, dv] io_dtype */
  const float* alpha;          /* [batch.total_T, H] */
  const float* beta;           /* [batch.total_T, H] */
  const int32_t* commit_len;   /* [B], 0..T_b of the pending step */
} sv_gdn_pending;

SV_API sv_status gdn_verify_commit(const sv_batch* batch, sv_gdn_mode mode,
    void* state, sv_dtype state_dtype, const int32_t* state_slot, int32_t num_slots,
    const void* q, const void* k, const void* v, sv_dtype io_dtype,
    const float* alpha, const float* beta, const int32_t* commit_len,
    void* out, int32_t H, int32_t dk, int32_t dv,
    const sv_gdn_pending* pending, int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Short causal convolution of the linear-attention layers: verify and commit.
 *
 * The packed varlen operator keeps a rolling state of the last K-1 inputs
 * per sequence and publishes the state after every token (onnxruntime-genai
 * #2457, VarlenCausalConvWithState prefix states: slot j is the state after
 * local token j).  Per channel c, with z = [state rows, x_0 .. x_{T_b-1}]
 * (oldest first):
 *   y_t[c] = act( sum_{i<K} weight[c][i] * z_{t+i}[c] + bias[c] )
 * so weight[c][K-1] multiplies the newest input; act is the identity
 * (SV_ACT_NONE) or SiLU (SV_ACT_SILU).  Commit keeps the last K-1 rows of
 * [state, x_0 .. x_{c_b - 1}] -- the state a run over only the accepted
 * prefix leaves (c_b = 0 keeps it).  Modes as for gdn_verify_commit.
 *   state      [num_slots, K-1, C] io_dtype, oldest first, updated in place
 *   state_slot int32 [B] or NULL (slot b)
 *   x, out     [total_T, C] io_dtype (out unused by COMMIT_ONLY)
 *   weight     fp32 [C, K];   bias fp32 [C] or NULL
 *   commit_len int32 [B] (unused by VERIFY_ONLY)
 *   pending    NULL, or the previous step's inputs and commit lengths
 *              (deferred commit): the window first advances over the first
 *              pending->commit_len[b] pending inputs and that state is
 *              stored, then this call's tokens run from it.
 * K in 2..8, C >= 1.  Stored states are copies of inputs (exact).
 * ------------------------------------------------------------------------ */
#define SV_ACT_NONE 0
#define SV_ACT_SILU 1

typedef struct {
  sv_batch batch;              /* the pending step's batch (same B) */
  const void* x;               /* [batch.total_T, C] io_dtype */
  const int32_t* commit_len;   /* [B], 0..T_b of the pending step */
} sv_conv_pending;

SV_API sv_status short_conv_verify_commit(const sv_batch* batch, sv_gdn_mode mode,
    void* state, const int32_t* state_slot, int32_t num_slots, const void* x,
    const float* weight, const float* bias, sv_dtype io_dtype, int32_t activation,
    const int32_t* commit_len, void* out, int32_t C, int32_t K,
    const sv_conv_pending* pending, int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Acceptance.
 *
 * Greedy (onnxruntime-genai #2457, greedy MTP step and device argmax of the
 * verify rows): g_i = argmax of target row cu_b + i (lowest index on ties);
 * a_b = leading run with draft_i == g_i; y = g_{a_b}.
 * Rejection sampling (Leviathan et al. 2023, Algorithm 1; Chen et al. 2023),
 * temperature 1: p_i / q_i are the softmaxes of target row cu_b + i / draft
 * row cu_b - b + i (fp64 normalisers); draft x_i is accepted iff
 * u_accept[cu_b - b + i] * q_i(x_i) < p_i(x_i); at the first rejection y is
 * drawn from max(0, p_i - q_i) (p_i if that is all zero) and if every draft
 * passes from p_{k_b}, by inverse CDF in vocabulary order with u_final[b]
 * (first y whose running sum exceeds u_final * total).
 *
 *   target_logits  [total_T, V] logit_dtype
 *   draft_logits   [total_T - B, V] logit_dtype; unused by greedy.  NULL in
 *                  rejection mode: each draft distribution is the point mass
 *                  on its draft token (lmdeploy #3945 reject_sampler.py with
 *                  draft_probs = None): x_i passes iff u_accept < p_i(x_i) and
 *                  the residual is p_i without x_i
 *   draft_tokens   int32 [total_T - B]
 *   u_accept       fp32 [total_T - B], u_final fp32 [B] (rejection only)
 *   result         int32 [B * (1 + max_T)]: accept_len[B] followed by the
 *                  rows out[B][max_T] = x_1 .. x_a, y, -1 ... (lmdeploy #3945
 *                  reject_sampler.py layout), one buffer for one readback
 *   commit_len_out int32 [B] = accept_len + 1, or NULL
 *   ctx_lens_inout int32 [B] += accept_len + 1 (the KV commit), or NULL
 *   bonus_tokens   (spec_accept_args only) int32 [B] or NULL: when every
 *                  draft of sequence b passes, bonus_tokens[b] is emitted in
 *                  place of the last row's argmax / draw (pre-sampled
 *                  bonus_token_ids of the same file); an id outside 0..V-1
 *                  flags SV_DERR_TOKEN and skips the sequence
 * Workspace: spec_accept_workspace_bytes().
 * ------------------------------------------------------------------------ */
typedef enum { SV_ACCEPT_GREEDY = 0, SV_ACCEPT_REJECTION = 1 } sv_accept_mode;

SV_API size_t spec_accept_workspace_bytes(int32_t B, int32_t total_T, int32_t V,
                                   sv_accept_mode mode);

/* The acceptance inputs of spec_accept_args and spec_verify_step. */
typedef struct {
  sv_accept_mode mode;
  sv_dtype logit_dtype;
  int32_t V;
  const void* target_logits; const void* draft_logits;
  const int32_t* draft_tokens; const float* u_accept; const float* u_final;
  const int32_t* bonus_tokens;   /* [B] or NULL */
} sv_accept_args;

SV_API sv_status spec_accept_args(const sv_batch* batch, const sv_accept_args* acc,
    int32_t* result, int32_t* commit_len_out, int32_t* ctx_lens_inout,
    void* workspace, size_t workspace_bytes, int32_t* err, hipStream_t stream);

/* The same acceptance for callers that cannot allocate or pass a workspace
 * (code under graph capture, tight serving loops, hosts that forbid device
 * allocation): the scratch is a device array inside the library, 8 MiB on
 * every GPU it runs on, held until the process ends.  A batch whose
 * spec_accept_workspace_bytes() exceeds 8 MiB (2^23 bytes) is refused with
 * SV_ECAPACITY.  It calls no allocator; its first call on a GPU looks up that
 * GPU's scratch address (make it outside a graph capture).  Every call on one
 * GPU shares the scratch: calls that overlap on one GPU (two streams, two
 * threads) race and must be ordered by the caller.  Results are those of
 * spec_accept_args with the same arguments. */
SV_API sv_status spec_accept_noalloc(const sv_batch* batch, const sv_accept_args* acc,
    int32_t* result, int32_t* commit_len_out, int32_t* ctx_lens_inout, int32_t* err,
    hipStream_t stream);

SV_API sv_status spec_accept(const sv_batch* batch, sv_accept_mode mode,
    const void* target_logits, const void* draft_logits, sv_dtype logit_dtype,
    int32_t V, const int32_t* draft_tokens, const float* u_accept,
    const float* u_final, int32_t* result, int32_t* commit_len_out,
    int32_t* ctx_lens_inout, void* workspace, size_t workspace_bytes,
    int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Checkpoint-series commit (the pages' other rollback, for comparison with
 * the replay commit above).
 *
 * onnxruntime-genai #2457, commit messages on the per-token state series and
 * CommitPrefix: during the step the operators publish the state after every
 * token into a window of `window` slots (window >= max_T) per sequence;
 * GatedDeltaNet writes slot window - 1 after the last token (token j of a
 * T_b-token sequence -> slot window - T_b + j), the short convolution writes
 * slot j after local token j.  After acceptance, CommitPrefix copies the
 * slot of the accepted prefix (c_b tokens kept; c_b = 0 keeps the state)
 * into the sequence's state slot.  Slots no token maps to are not written.
 * The verify calls leave the state bank untouched and take no pending
 * tokens; outputs are those of VERIFY_ONLY.
 *
 *   checkpoints    [B, window, H, dv, dk] in state_dtype
 *   prefix_states  [B, window, K-1, C] in io_dtype
 * Other arguments as for gdn_verify_commit / short_conv_verify_commit.
 * Device errors: SEQLEN, SLOT and (CommitPrefix) COMMIT bits; the sequence
 * is skipped.
 * ------------------------------------------------------------------------ */
SV_API sv_status gdn_verify_checkpoint(const sv_batch* batch,
    const void* state, sv_dtype state_dtype, const int32_t* state_slot, int32_t num_slots,
    const void* q, const void* k, const void* v, sv_dtype io_dtype,
    const float* alpha, const float* beta, void* out,
    void* checkpoints, int32_t window, int32_t H, int32_t dk, int32_t dv,
    int32_t* err, hipStream_t stream);

SV_API sv_status gdn_commit_prefix(const sv_batch* batch,
    void* state, sv_dtype state_dtype, const int32_t* state_slot, int32_t num_slots,
    const void* checkpoints, int32_t window, const int32_t* commit_len,
    int32_t H, int32_t dk, int32_t dv, int32_t* err, hipStream_t stream);

SV_API sv_status short_conv_verify_checkpoint(const sv_batch* batch,
    const void* state, const int32_t* state_slot, int32_t num_slots,
    const void* x, const float* weight, const float* bias, sv_dtype io_dtype,
    int32_t activation, void* out, void* prefix_states, int32_t window,
    int32_t C, int32_t K, int32_t* err, hipStream_t stream);

SV_API sv_status short_conv_commit_prefix(const sv_batch* batch,
    void* state, const int32_t* state_slot, int32_t num_slots,
    const void* prefix_states, int32_t window, const int32_t* commit_len,
    sv_dtype io_dtype, int32_t C, int32_t K, int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The whole step over a hybrid stack, in dependency order (lmdeploy #5019:
 * target pass, then the speculative round whose recurrent-state commit runs
 * after acceptance):
 *   1. every layer in model order: attention layers run
 *      spec_verify_attention (write_kv = 1), or spec_verify_attention_kv8
 *      when acfg->kv_format is SV_KV_INT8; GDN layers run their verify pass
 *      (deferred schedule: applying the pending tokens first and storing),
 *      and, with gcfg->conv_C > 0, their short convolution's verify pass in
 *      the same launch (the pages keep the two as separate operators, each
 *      with its own state: the step takes both operators' inputs and
 *      neither reads the other's output);
 *   2. spec_accept -> result, commit_len = accept_len + 1;
 *   3. two-phase schedule: one launch applies the first commit_len tokens of
 *      every GDN layer (and its convolution) and stores the states (deferred
 *      schedule: nothing, the next step's verify pass does it, or
 *      spec_verify_flush);
 *   4. ctx_lens += commit_len.
 * Attention layers share block_table / ctx_lens; GDN layers share
 * state_slot.  `layer_kind` (host) holds 0 = GDN, 1 = attention, in model
 * order; `attn` / `gdn` (host arrays) hold the attention / GDN layers in the
 * order they appear.  Workspace: spec_verify_step_workspace_bytes().
 * ------------------------------------------------------------------------ */
typedef enum { SV_SCHEDULE_TWO_PHASE = 0, SV_SCHEDULE_DEFERRED = 1 } sv_schedule;

typedef enum { SV_KV_PLAIN = 0, SV_KV_INT8 = 1 } sv_kv_format;

typedef struct {
  const void* q; const void* k_new; const void* v_new;
  void* k_cache; void* v_cache; void* out;
  const float* k_scale; const float* v_scale;  /* SV_KV_INT8 only */
} sv_attn_layer;

typedef struct {
  void* state; const void* q; const void* k; const void* v;
  const float* alpha; const float* beta; void* out;
  /* the layer's short convolution (used when sv_gdn_config.conv_C > 0; see
   * short_conv_verify_commit): rolling state [num_slots, K-1, C] in the io
   * dtype (updated in place, slots as for `state`), inputs conv_x and
   * outputs conv_out [total_T, C], taps fp32 [C, K], bias fp32 [C] or NULL */
  void* conv_state; const void* conv_x; void* conv_out;
  const float* conv_weight; const float* conv_bias;
} sv_gdn_layer;

typedef struct {
  int32_t Hq, Hkv, D, page_size, num_pages, max_pages_per_seq;
  const int32_t* block_table;  /* [B, max_pages_per_seq] */
  sv_dtype dtype;
  float scale;                 /* 0 => 1/sqrt(D) */
  sv_kv_format kv_format;      /* SV_KV_INT8: int8 pools, dtype SV_BF16 */
} sv_attn_config;

typedef struct {
  int32_t H, dk, dv, num_slots;
  const int32_t* state_slot;   /* [B] or NULL */
  sv_dtype io_dtype;
  sv_dtype state_dtype;        /* SV_F32 or SV_F16 */
  /* the short convolution of every GDN layer: channels (0: none), width
   * 2..8, activation SV_ACT_NONE / SV_ACT_SILU; its state and inputs use
   * io_dtype and the GDN layers' state slots */
  int32_t conv_C, conv_K, conv_activation;
} sv_gdn_config;



/* Pending tokens of every GDN layer for the deferred schedule (host struct;
 * `layers` is a host array of n_gdn entries whose k, v, alpha, beta (and
 * conv_x) point at the previous step's inputs; the other pointers are
 * unused). */
typedef struct {
  sv_batch batch;
  const sv_gdn_layer* layers;
  const int32_t* commit_len;   /* [B] */
} sv_step_pending;

SV_API size_t spec_verify_step_workspace_bytes(const sv_batch* batch,
    const sv_attn_config* acfg, const sv_accept_args* acc);

SV_API sv_status spec_verify_step(const sv_batch* batch, int32_t n_layers,
    const uint8_t* layer_kind,
    const sv_attn_config* acfg, const sv_attn_layer* attn,
    const sv_gdn_config* gcfg, const sv_gdn_layer* gdn,
    const sv_accept_args* acc, int32_t* ctx_lens, int32_t* result,
    int32_t* commit_len, sv_schedule schedule, const sv_step_pending* pending,
    void* workspace, size_t workspace_bytes, int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Flush of the deferred schedule: the commit the next step's verify pass
 * would have done, without a next step (the state of a sequence that
 * leaves, or every state before it is read).  For each of the n_gdn layers
 * of `pending` (their state, k, v, alpha, beta and, with gcfg->conv_C > 0,
 * conv_state and conv_x are read; gcfg as given to the step), the first
 * pending->commit_len[b] tokens of sequence b are applied to its state (and
 * convolution window) and the result is stored: the stored state is the one
 * the two-phase schedule would have left (onnxruntime-genai #2457:
 * CommitPrefix of the accepted prefix; lmdeploy #5019 "Two fixes" item 2:
 * the commit runs after acceptance).  The layers are committed in batched
 * launches, as the two-phase step commits; no workspace.  Every argument of
 * every layer is checked before the first launch.  Device errors as for
 * gdn_verify_commit (a bad commit length, T_b or slot skips the sequence).
 * Calling it twice applies the tokens twice: a flushed `pending` must not
 * be passed to a later step.
 * ------------------------------------------------------------------------ */
SV_API sv_status spec_verify_flush(int32_t n_gdn, const sv_gdn_config* gcfg,
    const sv_step_pending* pending, int32_t* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sizing and errors.
 *
 * sv_workspace_bytes: one workspace size that serves every call of a batch
 * of at most B sequences of at most max_T verify tokens (attention of either
 * page format with up to Hq KV heads of head size D over block tables of
 * max_pages_per_seq pages, acceptance of either mode over V entries, and the
 * step).  0 for a size outside the limits.  The per-call queries above give
 * tighter sizes.
 *
 * sv_read_device_error: the value of the caller's device error word `err`
 * (the SV_DERR_* bits the kernels OR into it) once `stream` has run the work
 * enqueued before the call.  It copies the word to the host and waits for
 * the stream, so it is the one call that blocks and must not be made while
 * the stream is being captured.  Returns the bits (>= 0), or -1 if the copy
 * failed (sv_last_error() says why).
 *
 * sv_clear_device_error: enqueues a kernel that zeroes the error word (no
 * memset node, so it may be captured into a graph with the step).
 * ------------------------------------------------------------------------ */
SV_API size_t sv_workspace_bytes(int32_t B, int32_t max_T, int32_t Hq, int32_t D, int32_t V,
                                 int32_t max_pages_per_seq);
SV_API int32_t sv_read_device_error(const int32_t* err, hipStream_t stream);
SV_API sv_status sv_clear_device_error(int32_t* err, hipStream_t stream);

/* Host: text of the calling thread's last non-OK status ("" if none). */
SV_API const char* sv_last_error(void);

/* Host: library version string. */
SV_API const char* sv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
