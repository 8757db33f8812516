/*
 * streambp_head.h -- C interface of the MI355X (gfx950) library for
 * StreamBP's sequence-chunked exact forward and backward through a
 * language-model head.
 *
 * Method: "StreamBP: Memory-Efficient Exact Backpropagation for Long Sequence
 * Training of LLMs".  LM-head paragraph of the news-article page: for SFT and
 * GRPO the logits of different positions enter the objective independently,
 * so the sequence is cut into chunks and the loss gradient is formed one chunk
 * at a time; only one chunk's logits and logits gradient are ever stored.
 * DPO paragraph of the same page: the sigmoid couples positions, but the
 * logits gradient still separates along the sequence; this library does it in
 * two passes (sequence log-probabilities first, then the chunked backward with
 * the pair factor).  Abstract (chatpaper / fugumt pages): the result is the
 * exact backpropagation gradient.
 *
 * Shapes: H [T x D] hidden states, W [V x D] head weight (nn.Linear layout,
 * no bias), labels [T] int32 already aligned with the rows of H (the caller
 * does any next-token shift).  A label of STREAMBP_IGNORE_INDEX (-100) drops
 * its row from the objective.  For each chunk of C rows the library computes
 * Z_c = H_c W^T, lse_t = log sum_v exp Z_tv, logp_t = Z_{t,y_t} - lse_t and
 * G_c = diag(w) (softmax(Z_c) - onehot(y)), then dH_c = G_c W and
 * dW += G_c^T H_c.  w_t is the per-token cross-entropy weight of the objective.
 *
 * Conventions shared by every entry point
 *  - All array pointers are DEVICE pointers on the handle's device, row-major
 *    and contiguous, 16-byte aligned.  H and W are float32 or bfloat16 bit
 *    patterns (uint16), as the handle's dtype says.  dH and dW are float32,
 *    losses and sequence sums are float64.
 *  - The library never allocates device memory in a call.  The caller passes
 *    `workspace` (device memory, 256-byte aligned) of at least
 *    streambp_head_workspace_bytes() bytes.  The workspace must not overlap
 *    any input or output; its contents are undefined after the call.  Peak
 *    workspace is O(C*V): one C x V logits buffer, reused in place for the
 *    logits gradient, plus O(T) and O(C*D) vectors.
 *  - Every kernel is enqueued on `stream` (a hipStream_t; NULL means the null
 *    stream).  Calls return before the GPU finishes; inputs must stay valid
 *    until the stream passes the call.  A handle serves one host thread at a
 *    time.  Results are bitwise deterministic from run to run.
 *  - Argument, shape, alignment and workspace errors are detected on the host
 *    before anything is enqueued; the call then returns the error code and
 *    streambp_head_last_error() describes it.  A failed kernel launch returns
 *    STREAMBP_ERR_HIP.
 *  - Label values outside [0, V) other than -100 are treated as ignored, and
 *    the device word `*status` is set to STREAMBP_ERR_LABEL_RANGE; sequence
 *    offsets that do not run from 0 to T without decreasing set it to
 *    STREAMBP_ERR_INVALID_ARGUMENT (every token then gets weight 0).
 *    Otherwise *status is STREAMBP_OK.  NaN and Inf inputs propagate.
 *  - `accumulate_dW` = 0 overwrites dW; 1 adds this call's gradient to it.
 */
#ifndef STREAMBP_HEAD_H
#define STREAMBP_HEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STREAMBP_IGNORE_INDEX (-100)

#ifndef STREAMBP_API
#define STREAMBP_API __attribute__((visibility("default")))
#endif

typedef struct streambp_head_s* streambp_head;

typedef enum {
  STREAMBP_OK = 0,
  STREAMBP_ERR_INVALID_ARGUMENT = 1,
  STREAMBP_ERR_UNSUPPORTED = 2,
  STREAMBP_ERR_WORKSPACE_TOO_SMALL = 3,
  STREAMBP_ERR_HIP = 4,
  STREAMBP_ERR_LABEL_RANGE = 5
} streambp_status;

typedef enum { STREAMBP_F32 = 0, STREAMBP_BF16 = 1 } streambp_dtype;

/* Create a handle for a head of width D and vocabulary V processed in chunks
 * of `chunk` rows on HIP device `device`.  Requires D > 0 with D % 8 == 0
 * (else STREAMBP_ERR_UNSUPPORTED), V > 0, chunk > 0, all below 2^31.  The
 * handle holds host state only.  A device index beyond the visible devices is
 * rejected; when no HIP device can be queried at all the handle is still
 * created (argument checks work) and calls fail with STREAMBP_ERR_HIP. */
STREAMBP_API streambp_status streambp_head_create(streambp_head* out, int64_t D, int64_t V, int64_t chunk,
                                     streambp_dtype dtype, int device);

/* Release a handle (NULL is accepted). */
STREAMBP_API streambp_status streambp_head_destroy(streambp_head h);

/* Chunk-size suggestion.  The summary page's partition-count ablations and
 * limitations note that small partitions cost HBM traffic and launch overhead
 * while larger ones mainly cost memory; here the dW read-modify-write (4 B per
 * weight per chunk) makes that concrete.  Returns in *chunk_out the largest C
 * among 256, 512, ..., 16384 (and no larger than T rounded up to 256) whose
 * workspace for (T, n_seq) fits in budget_bytes; STREAMBP_ERR_WORKSPACE_TOO_SMALL
 * (and *chunk_out = 0) when not even C = 256 fits.  Host only; no device is
 * touched.  D, V, dtype as for streambp_head_create, T >= 0, n_seq >= 1. */
STREAMBP_API streambp_status streambp_head_suggest_chunk(int64_t D, int64_t V, int64_t T, int32_t n_seq,
                                            streambp_dtype dtype, size_t budget_bytes, int64_t* chunk_out);

/* Workspace bytes needed for a call over T rows split into n_seq sequences
 * (n_seq = 1 for SFT).  Grows as C*V + C*D + T + n_seq, plus V*D bf16 for the
 * tiled copy of W while the tiled logits operands are on (see
 * streambp_head_set_tiled_logits); 0 for a NULL handle. */
STREAMBP_API size_t streambp_head_workspace_bytes(streambp_head h, int64_t T, int32_t n_seq);

/* Text of the last error on this handle ("" if none).  Owned by the handle. */
STREAMBP_API const char* streambp_head_last_error(streambp_head h);

/* Library version string, static storage. */
STREAMBP_API const char* streambp_head_version(void);

/* SFT (LM-head paragraph): loss = (1/N) sum over valid t of (lse_t - Z_{t,y_t}),
 * N = number of valid labels, i.e. w_t = 1/N.  N = 0 gives loss 0, dH = 0 and
 * no change to dW beyond the overwrite/accumulate rule.
 * Outputs: dH [T x D], dW [V x D], loss [1] (float64), n_valid [1] (int64),
 * status [1] (int32).  n_valid may be NULL. */
STREAMBP_API streambp_status streambp_head_sft(streambp_head h, int64_t T, const void* H, const void* W,
                                  const int32_t* labels, float* dH, float* dW, int accumulate_dW,
                                  double* loss, int64_t* n_valid, int32_t* status,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * streambp_head_sft without the workspace argument.  The workspace is a
 * fixed device array of STREAMBP_STATIC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends (its address on a device
 * is looked up when a handle is created there); the call allocates nothing
 * and creates no events (the per-kernel timer does not cover it).  A call
 * whose streambp_head_workspace_bytes(h, T, 1) exceeds that size returns
 * STREAMBP_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  Every call
 * on one device shares the array: calls that can overlap on one device (on
 * different streams, or from different threads) race on it and must be
 * serialised by the caller.  Nothing in the array needs to start at zero.
 * Arguments, outputs and errors are otherwise those of streambp_head_sft. */
#define STREAMBP_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
STREAMBP_API streambp_status streambp_head_sft_noalloc(streambp_head h, int64_t T, const void* H, const void* W,
                                                      const int32_t* labels, float* dH, float* dW,
                                                      int accumulate_dW, double* loss, int64_t* n_valid,
                                                      int32_t* status, void* stream);

/* On-policy GRPO (LM-head paragraph; ratio 1, no KL, so clipping is inactive):
 * tokens form n_seq packed sequences, sequence s = rows [seq_offsets[s],
 * seq_offsets[s+1]).  The objective weights log pi_t by -adv[s]/len_s, len_s =
 * valid labels of sequence s, i.e. w_t = adv[s]/len_s.
 * loss = sum_t (-adv[s]/len_s) logp_t.  seq_offsets [n_seq+1] int32 and
 * adv [n_seq] float32 are device arrays.  logp [T] (float32 per-token
 * log-probability, 0 on ignored rows) may be NULL. */
STREAMBP_API streambp_status streambp_head_grpo(streambp_head h, int64_t T, const void* H, const void* W,
                                   const int32_t* labels, const int32_t* seq_offsets, int32_t n_seq,
                                   const float* adv, float* logp, float* dH, float* dW,
                                   int accumulate_dW, double* loss, int32_t* status,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Off-policy head: PPO (listed among StreamBP's objectives in the news
 * article) or off-policy GRPO with a KL penalty.  Per valid token t of
 * sequence s, with logp_t from this call:
 *   r_t = exp(logp_t - logp_old[t]),  a_t = adv[s]/len_s,  d_t = logp_ref[t] - logp_t,
 *   L_t = -min(r_t a_t, clip(r_t, 1-clip_eps, 1+clip_eps) a_t)
 *         + (beta_kl/len_s) (exp(d_t) - d_t - 1);
 * loss = sum_t L_t (float64).  The gradient takes the slope of the unclipped
 * product where it is the minimum (ties included) and 0 where the clipped one
 * is strictly smaller.  Each token's loss depends only on its own logits, so
 * the same chunk loop runs, with the weight formed in the row pass right
 * after logp_t.  logp_old and logp_ref are float32 [T] device arrays aligned
 * with H's rows (logp_ref may be NULL when beta_kl == 0); seq_offsets and adv
 * as for GRPO; logp [T] may be NULL.  clip_eps must be finite and >= 0,
 * beta_kl finite.  Errors as for the other calls. */
STREAMBP_API streambp_status streambp_head_ppo(streambp_head h, int64_t T, const void* H, const void* W,
                                  const int32_t* labels, const int32_t* seq_offsets, int32_t n_seq,
                                  const float* adv, const float* logp_old, const float* logp_ref,
                                  double clip_eps, double beta_kl, float* logp, float* dH, float* dW,
                                  int accumulate_dW, double* loss, int32_t* status,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* DPO pass 1 (DPO paragraph): seq_logp[s] = sum of logp_t over the valid
 * tokens of sequence s, accumulated in float64.  A forward pass only; dH and
 * dW are not touched.  seq_logp [n_seq] float64 device array.  token_lse
 * (may be NULL): float32 [T] device array that receives each token's
 * log-sum-exp over the vocabulary (entries of ignored tokens are unspecified
 * under masked-row compaction); pass it to streambp_head_dpo_bwd. */
STREAMBP_API streambp_status streambp_head_dpo_logp(streambp_head h, int64_t T, const void* H, const void* W,
                                       const int32_t* labels, const int32_t* seq_offsets,
                                       int32_t n_seq, double* seq_logp, float* token_lse, int32_t* status,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* DPO pass 2 (DPO paragraph): n_seq = 2P sequences, 0..P-1 chosen and P..2P-1
 * rejected, pair i = (i, P+i).  With Delta_i = (S_i - R_i) - (S_{P+i} - R_{P+i})
 * from seq_logp S (pass 1 output) and ref_logp R (both float64 [n_seq]):
 * loss = (1/P) sum_i softplus(-beta Delta_i); chosen tokens get
 * w_t = +(beta/P) sigmoid(-beta Delta_i), rejected tokens the negative.  The
 * factors are formed on the device; the chunked backward then runs with them.
 * token_lse (may be NULL): the per-token log-sum-exp that pass 1 wrote for
 * the same H, W and labels (and the same compaction setting).  On a bf16
 * handle the logits GEMM then writes the gradient of each chunk's logits
 * directly from the fp32 logits, and the separate row pass is skipped; results
 * agree with the NULL path to bf16 rounding (the softmax is taken from the
 * fp32 rather than the bf16-rounded logits).  fp32 handles ignore it. */
STREAMBP_API streambp_status streambp_head_dpo_bwd(streambp_head h, int64_t T, const void* H, const void* W,
                                      const int32_t* labels, const int32_t* seq_offsets,
                                      int32_t n_seq, const double* seq_logp, const double* ref_logp,
                                      double beta, const float* token_lse, float* dH, float* dW,
                                      int accumulate_dW, double* loss, int32_t* status, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Masked-row compaction (a performance option, off by default; bf16 handles
 * only, else STREAMBP_ERR_UNSUPPORTED).  Rows whose label is ignored carry
 * zero weight in every objective, so their logits need not be formed: when
 * enabled, the label scan lists the valid rows on the device and the chunk
 * loop runs over them only (C valid rows per chunk; each chunk's rows of H are
 * first copied into a dense workspace buffer).  Results equal those of the
 * plain loop up to the fp32 summation order of dW; dH rows of ignored tokens
 * are written as 0.  The number of valid rows stays on the device: the host
 * still enqueues ceil(T/C) chunks and the kernels of chunks past the valid
 * rows exit at once, so calls stay asynchronous.  The setting changes
 * streambp_head_workspace_bytes(): T x 4 bytes of row indices, a C x D bf16
 * buffer and split-K slabs more. */
STREAMBP_API streambp_status streambp_head_set_row_compaction(streambp_head h, int enable);

/* Tiled logits operands (a performance option of bf16 handles, off by
 * default; enabling it on an fp32 handle returns STREAMBP_ERR_UNSUPPORTED,
 * disabling always succeeds).  The logits GEMM reduces over D along rows of W
 * and of the chunk's H, whose k-stages are scattered 64-byte pieces of
 * row-major storage.  bf16 handles always copy each chunk's rows of H into
 * contiguous 256 x 32 tiles (zero-padded; C*D bf16 of workspace); with the
 * option each call also copies W into such tiles first, so that every stage
 * of both operands is one contiguous run.  Results are bit-for-bit those of
 * the plain path (same summation order).  Costs: V*D bf16 of workspace for
 * the copy of W (rounded up to whole tiles), and one extra read and write of
 * W per call. */
STREAMBP_API streambp_status streambp_head_set_tiled_logits(streambp_head h, int enable);

/* Per-kernel timing, for measurement tools.  While enabled, every kernel the
 * library launches is bracketed by a pair of HIP events recorded on the
 * call's stream (events are created by the library; no device memory).
 * streambp_head_kernel_times() waits for the recorded events, adds their
 * elapsed times to per-kind totals and returns the totals for `kind`
 * (0 <= kind < streambp_head_kernel_kinds()).  Enabling or disabling resets
 * the totals.  Returns STREAMBP_ERR_INVALID_ARGUMENT for a bad kind. */
STREAMBP_API streambp_status streambp_head_set_timing(streambp_head h, int enable);
STREAMBP_API int streambp_head_kernel_kinds(void);
STREAMBP_API const char* streambp_head_kernel_name(int kind);
STREAMBP_API streambp_status streambp_head_kernel_times(streambp_head h, int kind, double* total_ms,
                                                        int64_t* launches);

/* Measurement aid, not part of the head computation: the dense bf16 MFMA
 * rate this GPU sustains for the instruction the GEMMs use.  Enqueues on
 * `stream` (the current device) one launch of `blocks` blocks of 4 waves,
 * each wave issuing iters x 8 independent v_mfma_f32_32x32x16_bf16 on
 * operands held in registers (no memory traffic; nothing observable is
 * written): the same pair in every instruction, or with changing_operands
 * != 0 pseudo-random pairs that change from one instruction to the next, as
 * in a GEMM.  *flops (may be NULL) receives the launch's flop count,
 * blocks x 4 x iters x 8 x 32768; the caller times the stream around it.
 * STREAMBP_ERR_INVALID_ARGUMENT unless 1 <= blocks <= 2^31 - 1 and
 * iters >= 1; STREAMBP_ERR_HIP if the launch fails. */
STREAMBP_API streambp_status streambp_head_mfma_probe(int64_t blocks, int32_t iters, int changing_operands,
                                                      double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAMBP_HEAD_H */
