/*
 * pg_lmhead.h - C ABI of the fused tied LM head + logit softcap cross-entropy -> bits-per-byte
 * library for AMD Instinct MI355X (gfx950).
 *
 * The path scores a small GPT by compression, as the Parameter Golf challenge does:
 *   logits      z[t,v] = sum_d H[t,d] * E[v,d]      tied head: the input embedding E is the output
 *                                                    projection (trios issue #19, approach table,
 *                                                    "Tied embeddings"; parameter-golf README
 *                                                    leaderboard, "Naive Baseline": TiedEmbeddings)
 *   softcap     s = c * tanh(z / c), c = 0: s = z    (a fused softcapped cross-entropy kernel: HYDRA Golf site
 *                                                    stack list; README leaderboard, PR #1787 row)
 *   loss        nats[t] = logsumexp_v s[t,v] - s[t,y[t]]   (trios issue, "Контекст": cross-entropy)
 *   metric      bpb = sum nats / (ln 2 * sum bytes(y[t])) over scored rows   (README introduction:
 *                                                    the challenge scores compression, in bits per byte)
 *   backward    dZ = g (softmax(s) - onehot(y)) * (1 - (s/c)^2), dH = dZ E, dE = dZ^T H
 *                                                    (repo-explainer, "The Baseline Is a Map":
 *                                                    the backward pass of the baseline's loss)
 *
 * Conventions for every entry point:
 *   - Array pointers are DEVICE pointers (hipMalloc'ed or equivalent), row-major and contiguous,
 *     16-byte aligned. H is [T, D], E is [V, D]; D is the fastest axis of both.
 *   - bf16 arrays hold raw bfloat16 bit patterns (uint16). f32 arrays are IEEE binary32.
 *   - The caller owns every buffer, including the workspace. The library allocates no device
 *     memory and keeps no caller pointer after a call returns. Its only global state is a
 *     per-device cache of the device check and, for pg_lmhead_ce_fwd_noalloc, a static device
 *     array per GPU (part of the loaded code object) with its cached address; that array keeps
 *     the last such call's contents.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream) and never
 *     synchronises the host. Buffers must stay alive until the stream's work is done.
 *   - Arguments are validated on the host before anything is launched; a non-zero status means
 *     nothing was enqueued. Data errors found on the device (a target outside [0, V) on a scored
 *     row, NaN/Inf inputs) are not reported as codes: they turn the affected nats into NaN, which
 *     propagates into the bits-per-byte, and in the backward into that row of dhidden and, since
 *     every entry of dembed sums over the rows, into all of dembed (the loss itself is NaN then).
 *   - nats >= 0 on every scored row: the target's logit is taken from the same accumulation that
 *     forms the log-sum-exp, so p(target) <= 1 holds in floating point too (a one-entry vocabulary
 *     gives exactly 0; the last step, a difference of two hardware log2 values, is floored at 0).
 *   - Unscored rows (score_mask[t] == 0) get nats = lse = 0, zero dH rows, and add nothing to any
 *     sum. A NULL score_mask scores every row.
 */
#ifndef PG_LMHEAD_H
#define PG_LMHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pg_status;

enum {
  PG_OK = 0,
  PG_ERR_NULL = -1,      /* a required pointer is NULL */
  PG_ERR_SHAPE = -2,     /* T < 0, D < 1, V < 1, or a size beyond the supported range */
  PG_ERR_DTYPE = -3,     /* unknown dtype code */
  PG_ERR_SOFTCAP = -4,   /* softcap negative or not finite; grad_scale not finite */
  PG_ERR_WORKSPACE = -5, /* workspace smaller than pg_workspace_bytes() asks for */
  PG_ERR_ALIGN = -6,     /* a pointer is not 16-byte aligned */
  PG_ERR_DEVICE = -7,    /* no HIP device, or the current device is not gfx950 */
  PG_ERR_HIP = -8,       /* a HIP runtime call or kernel launch failed */
  PG_ERR_SCRATCH = -9    /* pg_lmhead_ce_fwd_noalloc: the shape needs more than its static scratch */
};

enum { PG_DTYPE_BF16 = 0, PG_DTYPE_F32 = 1 }; /* dtype of H and E (they share one) */
enum { PG_OP_FWD = 0, PG_OP_BWD = 1, PG_OP_BPB = 2, PG_OP_FWD_Q8 = 3, PG_OP_FWD_BWD = 4 };

/* Largest supported sizes: T rows up to 2^31 - 256 (each row index fits an int32, and one launch
 * of 512-thread workgroups over 256-row tiles stays within 2^32 - 1 work items), V and D up to
 * 2^20. The backward entry points on the MFMA path also need their dhidden product's grid of
 * 256 x 256 output tiles to fit one launch: T < 2^30 at D = 512, T < 2^31 - 256 at D <= 256.
 * Beyond these, PG_ERR_SHAPE (and pg_workspace_bytes returns 0). bf16 with D in
 * {32, 64, 128, 256, 512} runs the MFMA kernels; any other D, and f32 inputs, run a plain vector
 * kernel with the same results up to rounding. */

/*
 * Forward: per-row softcapped cross-entropy, without ever writing the T x V logits to memory.
 *   hidden      [T, D] bf16 or f32 - final hidden states (input of the tied head)
 *   embed       [V, D] same dtype  - tied embedding, used as the output projection
 *   target      [T] int32          - next-token ids (the caller has already shifted x -> y)
 *   score_mask  [T] uint8 or NULL  - 1 = scored row (sliding-window evaluation scores only the
 *                                    last `stride` rows of each window: README leaderboard,
 *                                    "Sliding Window Eval", stride 64)
 *   softcap     c >= 0; c = 0 disables the cap
 *   nats        [T] f32 out        - -ln p(target) per row; 0 on unscored rows
 *   lse         [T] f32 out or NULL - logsumexp of the capped logits; 0 on unscored rows
 *                                    (pg_lmhead_ce_bwd needs it)
 *   workspace   device scratch of at least pg_workspace_bytes(PG_OP_FWD, T, D, V) bytes
 */
pg_status pg_lmhead_ce_fwd(const void* hidden, const void* embed, int32_t dtype,
                           const int32_t* target, const uint8_t* score_mask,
                           int64_t T, int32_t D, int32_t V, float softcap,
                           float* nats, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * pg_lmhead_ce_fwd without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation. It computes
 * exactly what pg_lmhead_ce_fwd computes (the same kernels) and allocates nothing: its scratch is a
 * static device array of 16 MiB + 256 B that each GPU the library runs on holds until the process
 * ends, which covers T <= 2^20 rows for any D and V (pg_workspace_bytes(PG_OP_FWD, T, D, V) must
 * fit; otherwise PG_ERR_SCRATCH, nothing enqueued). Every call on one GPU shares that GPU's array,
 * so calls that may overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller; calls in one stream are safe. Arguments and other errors as for
 * pg_lmhead_ce_fwd.
 */
pg_status pg_lmhead_ce_fwd_noalloc(const void* hidden, const void* embed, int32_t dtype,
                                   const int32_t* target, const uint8_t* score_mask,
                                   int64_t T, int32_t D, int32_t V, float softcap,
                                   float* nats, float* lse, void* stream);

/*
 * Backward of L = grad_scale * sum over scored rows of nats (mean cross-entropy: grad_scale =
 * 1 / number of scored rows). The logits are recomputed from hidden and embed; lse must be the
 * output of pg_lmhead_ce_fwd on the same inputs.
 *   dhidden     [T, D] f32 out, overwritten; rows of unscored positions are zero. NULL leaves
 *               dH out (its product is not run): for callers that train the embedding alone, such
 *               as score-first test-time training of the tied embedding
 *   dembed      [V, D] f32 out, overwritten; the LM-head part of the tied embedding's gradient
 *               only (the caller adds the gradient of the input lookup)
 *   workspace   at least pg_workspace_bytes(PG_OP_BWD, T, D, V) bytes (holds bf16 dZ [T, V])
 */
pg_status pg_lmhead_ce_bwd(const void* hidden, const void* embed, int32_t dtype,
                           const int32_t* target, const uint8_t* score_mask, const float* lse,
                           int64_t T, int32_t D, int32_t V, float softcap, float grad_scale,
                           float* dhidden, float* dembed,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward and backward in one call: the outputs of pg_lmhead_ce_fwd (nats, lse) and of
 * pg_lmhead_ce_bwd (dhidden, dembed) for the same arguments, the training step of the head
 * (repo-explainer, baseline listing: the loss, then its backward pass). For bf16
 * with D in {32, 64, 128, 256, 512} and 0 < softcap <= 40 the logits are computed once: the forward
 * also stores the gradient of every logit with the fixed shift of its log-sum-exp in place of the
 * not yet known lse, and the row factor that corrects it is applied when lse is known (in the dH
 * product, and to the hidden rows that feed dE, rounded to bf16 there). Any other input runs
 * pg_lmhead_ce_fwd then pg_lmhead_ce_bwd. Results agree with those two calls up to rounding.
 *   lse         [T] f32 out, required here
 *   workspace   at least pg_workspace_bytes(PG_OP_FWD_BWD, T, D, V) bytes
 * Other arguments and errors as for the two calls.
 */
pg_status pg_lmhead_ce_fwd_bwd(const void* hidden, const void* embed, int32_t dtype,
                               const int32_t* target, const uint8_t* score_mask,
                               int64_t T, int32_t D, int32_t V, float softcap, float grad_scale,
                               float* nats, float* lse, float* dhidden, float* dembed,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Asymmetric softcap variants: s = cap_pos * tanh(z / cap_pos) for z >= 0 and
 * s = cap_neg * tanh(z / cap_neg) for z < 0 (ds/dz = 1 - (s / cap)^2 on each side; a cap of 0 leaves
 * that side uncapped). The pages name an "AsymLogit" change to the head (HYDRA Golf site,
 * leaderboard table, entries #1 and #4; README leaderboard, PR #2135 and PR #1945 rows) without
 * defining it; separate caps for positive and negative logits is the reading taken here. With
 * cap_pos == cap_neg these equal pg_lmhead_ce_fwd / pg_lmhead_ce_bwd / pg_lmhead_ce_fwd_bwd.
 * Arguments, workspace sizes and errors are those of the symmetric entry points; either cap
 * negative or not finite gives PG_ERR_SOFTCAP. pg_lmhead_ce_fwd_bwd_asym computes the logits once
 * when both caps lie in (0, 40] (bf16, D as for pg_lmhead_ce_fwd_bwd); otherwise it runs the two
 * asymmetric calls.
 */
pg_status pg_lmhead_ce_fwd_asym(const void* hidden, const void* embed, int32_t dtype,
                                const int32_t* target, const uint8_t* score_mask,
                                int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                                float* nats, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

pg_status pg_lmhead_ce_bwd_asym(const void* hidden, const void* embed, int32_t dtype,
                                const int32_t* target, const uint8_t* score_mask, const float* lse,
                                int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg, float grad_scale,
                                float* dhidden, float* dembed,
                                void* workspace, size_t workspace_bytes, void* stream);

pg_status pg_lmhead_ce_fwd_bwd_asym(const void* hidden, const void* embed, int32_t dtype,
                                    const int32_t* target, const uint8_t* score_mask,
                                    int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                                    float grad_scale, float* nats, float* lse, float* dhidden, float* dembed,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Quantised tied head. The model is quantised to fit the artifact (trios issue #19, approach
 * table, "Квантование": INT4/INT8; README leaderboard, GPTQ and LQER rows), and the tied embedding
 * then serves as both input lookup and output head. The pages define no format; this library uses
 * per-row symmetric int8:
 *   scale[v] = max_d |E[v,d]| / 127                      (float32, correctly rounded)
 *   q[v,d]   = round_half_even(E[v,d] / scale[v])         (int8 in [-127, 127]; 0 if scale is 0)
 *   E'[v,d]  = bf16_round_half_even(float32(q[v,d]) * scale[v])   (what the head computes with)
 * D must be a multiple of 8 (PG_ERR_SHAPE otherwise).
 *
 * pg_quantize_q8: embed [V, D] (bf16 or f32, dtype as above) -> embed_q8 [V, D] int8 and
 *   embed_scale [V] f32, all device arrays. Needs no workspace.
 * pg_lmhead_ce_fwd_q8: the forward of pg_lmhead_ce_fwd (bf16 hidden) on the head E' of
 *   (embed_q8, embed_scale). At D = 512 with one cap in (0, 40], calls with a score mask or at
 *   most 8192 rows read the int8 rows in the forward itself, which forms E' tile by tile on chip;
 *   other calls first write E' into the workspace. Either way the workspace must hold
 *   pg_workspace_bytes(PG_OP_FWD_Q8, T, D, V) bytes, and the results are the same bits. nats and
 *   lse as for pg_lmhead_ce_fwd.
 */
pg_status pg_quantize_q8(const void* embed, int32_t dtype, int32_t V, int32_t D, int8_t* embed_q8,
                         float* embed_scale, void* stream);

pg_status pg_lmhead_ce_fwd_q8(const void* hidden, const int8_t* embed_q8, const float* embed_scale,
                              const int32_t* target, const uint8_t* score_mask,
                              int64_t T, int32_t D, int32_t V, float softcap,
                              float* nats, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bits per byte over the scored rows (tproger article, "Правила и метрика": the score counts
 * compression in bytes, independent of the tokenizer).
 *   nats          [T] f32 from pg_lmhead_ce_fwd
 *   target        [T] int32 - used to look up byte_len; a scored row whose target is outside
 *                 [0, V) adds no bytes (pg_lmhead_ce_fwd gives such a row NaN nats)
 *   byte_len      [V] int32 - UTF-8 bytes of each vocabulary entry (BOS / specials = 0)
 *   byte_per_pos  [T] int32 or NULL - per-position byte counts that replace byte_len (README
 *                 leaderboard, PR #1736 row: byte counts carried per position beside the tokens)
 *   out           [4] double, device: sum_nats, sum_bytes, n_scored, bits_per_byte
 *                 (0/0 = NaN for an empty mask, x/0 = +inf for zero bytes)
 * The sums use a fixed reduction order, so the result is bitwise reproducible.
 */
pg_status pg_bpb_reduce(const float* nats, const int32_t* target, const uint8_t* score_mask,
                        const int32_t* byte_len, const int32_t* byte_per_pos,
                        int64_t T, int32_t V, double* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * pg_bpb_reduce that adds to running sums instead of overwriting them: out[0..2] (sum_nats,
 * sum_bytes, n_scored) must hold the sums of the earlier calls (zeros before the first), this call's
 * sums are added in a fixed order and out[3] becomes the bits per byte of the running sums. Calls
 * in one stream therefore accumulate an evaluation that spans many batches, such as the sliding
 * windows below. Arguments, workspace and errors as for pg_bpb_reduce.
 */
pg_status pg_bpb_accumulate(const float* nats, const int32_t* target, const uint8_t* score_mask,
                            const int32_t* byte_len, const int32_t* byte_per_pos,
                            int64_t T, int32_t V, double* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sliding-window evaluation of a token stream (parameter-golf README leaderboard, "Sliding Window
 * Eval" row: windows advancing by a stride of 64 tokens, so that each scored token sees a long context), with
 * score-first test-time training (README leaderboard, "Legal Score-First TTT" rows, and the row that
 * trains in phases on validation chunks already scored; HYDRA Golf site, leaderboard entry #2).
 *
 * Schedule. tokens[0 .. n_tokens) is the stream; prediction p (p = 0 .. n_tokens - 2) is token
 * p + 1 given tokens 0 .. p. Window w covers input positions [w stride, w stride + window).
 * Window 0 scores predictions [0, window); window w >= 1 scores [w stride + window - stride,
 * w stride + window): the predictions it adds, each with at least window - stride tokens of
 * context. Every prediction is scored exactly once; stride <= window.
 *
 * pg_window_count: the number of windows that cover the stream (0 when n_tokens < 2).
 * pg_window_scored: the number of predictions that windows first_window .. first_window +
 *   n_windows - 1 score (windows past the last one score none). Both are host arithmetic (no
 *   device, no stream) and return PG_ERR_SHAPE (negative) for n_tokens < 0 or > 2^40,
 *   window < 1, stride < 1, stride > window, first_window < 0 or > pg_window_count, or
 *   n_windows < 0.
 * pg_window_rows: the rows of a batch of windows, laid out as n_windows x window rows, row
 *   (b, r) being input position (first_window + b) stride + r: target [n_windows * window] int32
 *   gets token p + 1 of each row's position p (0 past the stream), score_mask the same count of
 *   uint8 (1 where that window scores the row). The caller supplies the hidden states of the same
 *   rows (the model run on each window) and passes target and score_mask on to pg_lmhead_ce_fwd
 *   (or pg_lmhead_ce_fwd_bwd) and pg_bpb_accumulate. tokens is a device array; a token outside
 *   [0, V) poisons its row as in the forward. Errors: PG_ERR_SHAPE (as above, n_windows < 1, or more
 *   rows than the forward takes), PG_ERR_NULL, PG_ERR_ALIGN, PG_ERR_DEVICE, PG_ERR_HIP.
 * pg_sgd_step_bf16: one SGD step of score-first test-time training on the tied embedding, kept as
 *   float32 master weights with a bf16 copy that the head reads: for i < n,
 *   master[i] = fl(master[i] - fl(lr * grad[i])) (two float32 roundings, no fused multiply-add)
 *   and embed_bf16[i] = bf16_round_half_even(master[i]). grad is dembed from the training entry
 *   points on an already-scored batch, so a later batch is scored with the updated embedding and
 *   no batch with one trained on itself. PG_ERR_SOFTCAP for a non-finite lr.
 */
int64_t pg_window_count(int64_t n_tokens, int32_t window, int32_t stride);

int64_t pg_window_scored(int64_t n_tokens, int32_t window, int32_t stride, int64_t first_window,
                         int32_t n_windows);

pg_status pg_window_rows(const int32_t* tokens, int64_t n_tokens, int32_t window, int32_t stride,
                         int64_t first_window, int32_t n_windows, int32_t* target, uint8_t* score_mask,
                         void* stream);

pg_status pg_sgd_step_bf16(float* master, const float* grad, float lr, int64_t n, void* embed_bf16,
                           void* stream);

/* Workspace bytes an entry point needs for these sizes (0 for invalid sizes). */
size_t pg_workspace_bytes(int32_t op, int64_t T, int32_t D, int32_t V);

/* Static, NUL-terminated description of a status code. */
const char* pg_status_str(pg_status s);

/* ABI version of this header (bumped on any incompatible change). */
int32_t pg_abi_version(void);

#define PG_ABI_VERSION 1

#ifdef __cplusplus
}
#endif
#endif /* PG_LMHEAD_H */
