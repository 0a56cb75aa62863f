/*
 * domino.h — C ABI of the Domino draft-head engine for AMD Instinct MI355X (gfx950).
 *
 * The engine turns the hidden states that a parallel draft backbone produces
 * for a block of K positions into a K-token draft, as the Domino head does:
 * frozen LM head -> base logits for every position in one pass; then, position
 * by position, a GRU causal encoder over the previously chosen tokens, a
 * low-rank logit correction added to the base logits, and a token pick.
 * A separate call scores a draft against verification targets.
 *
 * Sources (pages on the Domino paper, cited by title and section):
 *   [notes]     "完全开源的语言模型学习记录--推理加速Domino" (gsyq.cn)
 *   [explainer] the yhxrc.cn article on the Domino paper (sections 一 … 七, Q&A)
 *
 * Conventions shared by every call
 *   - Every tensor pointer is caller-owned DEVICE memory, contiguous and
 *     row-major, unless stated otherwise.  The library keeps no pointer after
 *     a call returns and allocates no device memory of its own.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream).  Nothing synchronises the host.
 *   - Argument errors are reported as a negative domino_status before any work
 *     is enqueued.  A failed kernel launch returns DOMINO_ERR_HIP.  No call
 *     throws across this interface.
 *   - Preconditions not checked on the host: token ids lie in [0, vocab);
 *     every floating-point input is finite.  Violations give unspecified
 *     results (never out-of-bounds accesses for token ids: the kernels clamp).
 *   - Thread safety: calls may be made from several host threads on different
 *     streams; each concurrent draft_block call needs its own workspace.
 *   - domino_draft_block's single-block schedule (one block per call, or two,
 *     with a GRU input table at the pages' shapes) runs one workgroup on every
 *     compute unit, and those workgroups wait on one another.  The library
 *     orders every such launch of a process after the previous one on the same
 *     device, whatever streams they are issued on, so they never share the
 *     compute units (under stream capture the graph's own order applies).
 *     Work of other processes can still hold compute units; every wait of the
 *     loop is bounded (about a second), and a loop that gives up reports it
 *     through domino_draft_status and leaves -1 in its block's tokens.
 */
#ifndef DOMINO_H_
#define DOMINO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DOMINO_OK = 0,
  DOMINO_ERR_NULL = -1,        /* a required pointer is NULL                      */
  DOMINO_ERR_SHAPE = -2,       /* a size is out of range or not a multiple of 32  */
  DOMINO_ERR_DTYPE = -3,       /* unknown dtype code                              */
  DOMINO_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                */
  DOMINO_ERR_ARG = -5,         /* a scalar argument is invalid (e.g. T < 0, NaN)  */
  DOMINO_ERR_WORKSPACE = -6,   /* workspace missing, too small or not 256-aligned */
  DOMINO_ERR_HIP = -7,         /* the HIP runtime reported an error               */
  DOMINO_ERR_UNSUPPORTED = -8  /* valid request outside the library's limits     */
} domino_status;

typedef enum { DOMINO_F32 = 0, DOMINO_BF16 = 1 } domino_dtype;

/*
 * The Domino head: frozen LM head and input embedding of the target model,
 * and the trained GRU + low-rank correction parameters ([notes] §二.1(2);
 * [explainer] §四).  Weight layouts are [out, in], row-major.
 *
 *   d          hidden size of the backbone / LM head input      (multiple of 32)
 *   vocab      V, vocabulary size                               (1 … 2^24 - 1)
 *   gru_hidden H, GRU state size (1024 in the pages)             (multiple of 32)
 *   rank       r, correction bottleneck (256 in the pages)       (multiple of 32)
 *   block      K, positions per draft block (16 in the pages)    (1 … 64)
 *   dtype      element type of every weight, bias and hidden state
 *
 *   lm_head [V, d]      frozen LM head (no bias)
 *   embed   [V, d]      token embedding read by the GRU; may equal lm_head (tied)
 *   w_ih    [3H, d]     GRU input weights, gate rows ordered r | z | n
 *   w_hh    [3H, H]     GRU recurrent weights, rows r | z | n
 *   b_ih, b_hh [3H]     GRU biases (NULL = zero)
 *   w1      [r, d + H]  first correction projection; columns 0 … d-1 multiply
 *                       the hidden state, columns d … d+H-1 the GRU state
 *   b1      [r]         (NULL = zero)
 *   w2      [V, r]      second correction projection to the vocabulary
 *   b2      [V]         (NULL = zero)
 *   gru_input_table [V, 3H] float32, or NULL: T[v] = W_ih embed[v] + b_ih,
 *                       the GRU's input pre-activation for every token, filled
 *                       by domino_prepare_gru_table.  Both factors are frozen,
 *                       so the table is a per-head constant; when it is given,
 *                       domino_draft_block reads T[token] instead of
 *                       multiplying by W_ih at every position.
 *
 * Limits of the library: d * sizeof(element) <= 8192 bytes (bf16: d <= 4096,
 * f32: d <= 2048); H <= 4096; r <= 1024; batch <= 128.
 */
typedef struct {
  int32_t d;
  int32_t vocab;
  int32_t gru_hidden;
  int32_t rank;
  int32_t block;
  int32_t dtype; /* domino_dtype */
  const void *lm_head;
  const void *embed;
  const void *w_ih;
  const void *w_hh;
  const void *b_ih;
  const void *b_hh;
  const void *w1;
  const void *b1;
  const void *w2;
  const void *b2;
  const float *gru_input_table;
} domino_head;

/* Library version, as major * 10000 + minor * 100 + patch. */
int domino_version(void);

/* Static text for a domino_status code. */
const char *domino_status_string(int status);

/* Host-only check of a head descriptor (sizes, dtype, pointers, alignment).
 * Touches no device memory and makes no HIP call. */
int domino_check_head(const domino_head *head);

/* Bytes of the head's GRU input table: vocab * 3 * gru_hidden * 4. */
int domino_gru_table_size(const domino_head *head, size_t *bytes);

/*
 * Fills table[v, :] = W_ih embed[v] + b_ih for every v (the GRU input
 * pre-activation of each token, [notes] §二.1(2) item 1), as float32 with the
 * products accumulated in float32.  table: caller-owned device buffer of
 * domino_gru_table_size() bytes, 16-byte aligned.  Run once per head; the
 * result is then passed as head->gru_input_table.
 */
int domino_prepare_gru_table(const domino_head *head, float *table, void *stream);

/* Bytes of device workspace that domino_draft_block needs for `batch` blocks. */
int domino_workspace_size(const domino_head *head, int32_t batch, size_t *bytes);

/*
 * Base logits of every position of every block, in one pass over the frozen
 * LM head ([notes] §二.1(1); [explainer] §三):
 *     base_logits[b, i, v] = sum_k hidden[b, i, k] * lm_head[v, k]
 * hidden      [batch, K, d] (head dtype), 16-byte aligned
 * base_logits [batch, K, V] float32 (output)
 * Products are accumulated in float32.  batch == 0 is a no-op.
 */
int domino_base_logits(const domino_head *head, int32_t batch, const void *hidden,
                       float *base_logits, void *stream);

/*
 * One draft block per batch row: the Domino head's serial causal-correction
 * loop ([notes] §二.1(2) items 1-3; [explainer] §四):
 *   g_{-1} = 0;  for i = 0 … K-1:
 *     g_i  = GRU(embed[prev_i], g_{i-1})      prev_0 = x_t[b];
 *                                              prev_i = tokens[b, i-1], or
 *                                              teacher[b, i-1] when teacher != NULL
 *     L_i  = base_logits[b, i] + W2 SiLU(W1 [hidden[b, i] ; g_i] + b1) + b2
 *     tokens[b, i] = argmax_v L_i[v]                      (temperature == 0)
 *                  = argmax_v L_i[v] / T + G[b, i, v]     (temperature T > 0)
 *   Ties go to the lowest index.  G = -ln(-ln U) with U from Philox4x32-10:
 *   counter (v >> 2, i, b, offset), key (seed low 32 bits, seed high 32 bits),
 *   word = output lane (v & 3), U = ((word >> 9) + 0.5) * 2^-23.
 *
 * hidden      [batch, K, d] head dtype          base_logits [batch, K, V] float32, or NULL
 * x_t         [batch] int32                     teacher     [batch, K] int32 or NULL
 * tokens      [batch, K] int32 (output)
 * logits      [batch, K, V] float32 or NULL (output: the corrected logits L_i)
 * gru_states  [batch, K, H] float32 or NULL (output: g_i)
 * workspace   device scratch of at least domino_workspace_size() bytes,
 *             256-byte aligned; its contents are overwritten.
 * base_logits == NULL: the call forms base_logits[b, i] = lm_head hidden[b, i]
 *   itself, inside the draft loop (the LM head is read once, and the base
 *   logits never reach device memory).  Only for batch == 1, K <= 16, a bf16
 *   head with its GRU input table, d = 2560 or 4096, H = 1024, r = 256, on a
 *   device of at least 200 compute units; otherwise DOMINO_ERR_UNSUPPORTED
 *   (shapes: before anything is enqueued).  The products are summed in another
 *   order than domino_base_logits': the logits agree to float32 rounding.
 * Arithmetic: float32 throughout; bf16 weights are multiplied in bf16 by the
 * matrix cores with float32 accumulation, and float32 activations are fed to
 * them as a bf16 (high, low) pair so they keep about 16 significant bits.
 * Completion: the schedules whose workgroups wait on one another (see the
 * conventions above) give up a wait after about a second; the call's status
 * word (domino_draft_status) is then 1 and every token of the block whose
 * loop gave up is -1, which is never a valid token id.  A call that returns
 * DOMINO_OK and whose status word reads 0 drafted every block.
 */
int domino_draft_block(const domino_head *head, int32_t batch, const void *hidden,
                       const float *base_logits, const int32_t *x_t, const int32_t *teacher,
                       float temperature, uint64_t seed, uint32_t offset, int32_t *tokens,
                       float *logits, float *gru_states, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * For callers that cannot allocate device memory (code under stream capture,
 * serving loops or harnesses that forbid allocation): domino_draft_block with
 * the same arguments except the workspace.  Its scratch is a fixed device
 * array of 16 MiB inside the library (one per device, held until the process
 * ends), enough for up to 32 blocks of a Qwen3-8B-shaped head; a call whose
 * domino_workspace_size exceeds 16 MiB returns DOMINO_ERR_UNSUPPORTED before
 * anything is enqueued.  The call allocates nothing.  Every call on a device
 * shares that device's array: calls that overlap on one device (different
 * streams, or host threads, without ordering between them) race and give
 * undefined results.  Each call clears what must start at zero.  Outputs,
 * arguments and errors are those of domino_draft_block; a loop that gives up
 * leaves -1 in its block's tokens.
 */
int domino_draft_block_noalloc(const domino_head *head, int32_t batch, const void *hidden,
                               const float *base_logits, const int32_t *x_t, const int32_t *teacher,
                               float temperature, uint64_t seed, uint32_t offset, int32_t *tokens, float *logits,
                               float *gru_states, void *stream);

/*
 * Status of the last domino_draft_block call that used `workspace` for `batch`
 * blocks of this head: enqueues on `stream` a copy of the call's status word
 * into status[0] (device memory, int32): 0 = every block's loop completed,
 * 1 = a loop gave up a wait (its block's tokens are -1).  Stream-ordered after
 * the draft call when issued on the same stream; the workspace must not have
 * been reused in between.
 */
int domino_draft_status(const domino_head *head, int32_t batch, const void *workspace, size_t workspace_bytes,
                        int32_t *status, void *stream);

/*
 * Acceptance length of each draft row ([notes] §一.1 item 1): the number of
 * leading positions j with draft[b, j] == target[b, j], in 0 … block.
 * draft, target [batch, block] int32; accept [batch] int32 (output).
 * block in 1 … 1024; batch == 0 is a no-op.
 */
int domino_accept_len(int32_t batch, int32_t block, const int32_t *draft, const int32_t *target,
                      int32_t *accept, void *stream);

/*
 * Verification of a sampled draft.  The pages report sampled decoding at T = 1
 * ([notes] §三.2(1)) and have the target model verify the drafted block in
 * parallel without giving the acceptance rule; this call applies the published
 * speculative-sampling rule (Leviathan, Kalman, Matias, ICML 2023, Algorithm 1;
 * Chen et al. 2023), which keeps the output distributed as the target's.  With
 * p_t = softmax(target_logits[b, i] / T) and p_d = softmax(draft_logits[b, i] / T):
 *   position i = 0, 1, ... is accepted while U_i * p_d(y_i) < p_t(y_i),
 *   U_i = ((word >> 9) + 0.5) * 2^-23 with word = the Philox4x32-10 output lane 0
 *   at counter (0, i, b, offset), key (seed lo, seed hi);
 *   accept[b] = n, the first rejected position (block if none);
 *   next_token[b] = argmax_v log max(0, p_t(v) - p_d(v)) + G(v) at position n
 *   (log 0 = -inf), or argmax_v target_logits[b, block, v] / T + G(v) when
 *   n == block; G is the Gumbel noise of domino_draft_block at counter offset
 *   offset + 1, block b, position n.  Ties go to the lowest index.
 * The caller passes an offset whose streams (offset, offset + 1) the drafter
 * does not use for the same blocks.
 *
 * target_logits [batch, block + 1, vocab] float32 (4-byte aligned)
 * draft_logits  [batch, block, vocab] float32 (4-byte aligned): the logits the
 *               draft tokens were sampled from
 * draft         [batch, block] int32; ids outside [0, vocab) are clamped
 * temperature   T > 0 and finite (else DOMINO_ERR_ARG)
 * accept, next_token  [batch] int32 (outputs)
 * workspace     device scratch of at least domino_verify_workspace_size()
 *               bytes, 256-byte aligned; its contents are overwritten.
 * batch in 0 … 2^20 (0 is a no-op), block in 1 … 255, vocab in 1 … 2^24 - 1.
 * Arithmetic: float32 (log-sum-exp normalisers merged over vocabulary slices).
 */
int domino_verify_sampled(int32_t batch, int32_t block, int32_t vocab, const float *target_logits,
                          const float *draft_logits, const int32_t *draft, float temperature, uint64_t seed,
                          uint32_t offset, int32_t *accept, int32_t *next_token, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Workspace bytes domino_verify_sampled needs (0 for sizes out of range). */
size_t domino_verify_workspace_size(int32_t batch, int32_t block, int32_t vocab);

/*
 * Base-only drafting, the head-off configuration the pages measure Domino
 * against: the parallel backbone's block drafted from its base logits alone
 * ([notes] §二.1(1); the head ablation of [notes] §三 and [explainer] §六).
 * With no causal correction L_i = L_i^base, so every position is picked
 * independently, with the sampler of domino_draft_block:
 *   tokens[b, i] = argmax_v base_logits[b, i, v]                 (temperature == 0)
 *                = argmax_v base_logits[b, i, v] / T + G[b, i, v] (temperature T > 0)
 * G is the Gumbel noise of domino_draft_block (same counter layout), so a head
 * whose correction is identically zero drafts the same tokens through either
 * call.  Ties go to the lowest index.
 *
 * base_logits [batch, block, vocab] float32 (4-byte aligned)
 * tokens      [batch, block] int32 (output)
 * temperature >= 0 and finite (else DOMINO_ERR_ARG)
 * workspace   device scratch of at least domino_base_draft_workspace_size()
 *             bytes, 256-byte aligned; its contents are overwritten.
 * batch in 0 … 2^20 (0 is a no-op), block in 1 … 1024, vocab in 1 … 2^24 - 1.
 */
int domino_base_draft(int32_t batch, int32_t block, int32_t vocab, const float *base_logits, float temperature,
                      uint64_t seed, uint32_t offset, int32_t *tokens, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Workspace bytes domino_base_draft needs (0 for sizes out of range). */
size_t domino_base_draft_workspace_size(int32_t batch, int32_t block);

/*
 * Base-anchored curriculum loss of the head's teacher-forced training
 * ([notes] §二.2): with CE_x[b, i] = logsumexp(x[b, i, :]) - x[b, i, targets[b, i]]
 * for x = base_logits and final_logits (the final logits of a teacher-forced
 * domino_draft_block call, whose GRU read the same reference tokens),
 *   loss = Σ_b Σ_i w_i ((1 - lambda) CE_final[b, i] + lambda CE_base[b, i]) / (B Σ_i w_i),
 *   w_i = gamma^i (weights decaying along the block).
 * lambda is the curriculum weight λ_t, annealed by the caller from 1 to 0 over
 * training; the pages fix neither the decay rate nor the normalisation: gamma
 * is a parameter and the weighted mean above is this library's reading.
 * Optional outputs: ce_base, ce_final [batch, block] (the per-position
 * cross-entropies) and grad_base, grad_final [batch, block, vocab], the
 * gradients of loss with respect to each logit tensor,
 *   coef (softmax(x[b, i]) - onehot(targets[b, i])),
 *   coef = lambda w_i / (B Σw) for base, (1 - lambda) w_i / (B Σw) for final.
 * A gradient may be written over its own logits (grad_final == final_logits).
 *
 * base_logits, final_logits [batch, block, vocab] float32 (4-byte aligned)
 * targets     [batch, block] int32; ids outside [0, vocab) are clamped
 * loss        one float32 in device memory (output)
 * lambda in [0, 1], gamma in (0, 1], both finite (else DOMINO_ERR_ARG)
 * workspace   device scratch of at least domino_curriculum_loss_workspace_size()
 *             bytes, 256-byte aligned; its contents are overwritten.
 * batch in 0 … 2^20 (0 is a no-op that leaves loss untouched), block in
 * 1 … 1024, vocab in 1 … 2^24 - 1.  Arithmetic: float32; the loss is summed
 * in a fixed order, so repeated calls give the same bits.
 */
int domino_curriculum_loss(int32_t batch, int32_t block, int32_t vocab, const float *base_logits,
                           const float *final_logits, const int32_t *targets, float lambda, float gamma,
                           float *loss, float *ce_base, float *ce_final, float *grad_base, float *grad_final,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes domino_curriculum_loss needs (0 for sizes out of range). */
size_t domino_curriculum_loss_workspace_size(int32_t batch, int32_t block, int32_t vocab);

/*
 * Backward through the low-rank correction head ([notes] §二.1(2) items 2-3)
 * for training: given G = grad_final, the gradient of a loss with respect to
 * the final logits of every block and position (domino_curriculum_loss writes
 * it), and the teacher-forced GRU states g (domino_draft_block's gru_states),
 * with x_i = [hidden_i ; g_i], z_i = W1 x_i + b1, u_i = SiLU(z_i):
 *   d_w2 = Σ_i G_i u_iᵀ  [V, r]        d_b2 = Σ_i G_i      [V]   (NULL: skipped)
 *   d_w1 = Σ_i dz_i x_iᵀ [r, d + H]    d_b1 = Σ_i dz_i     [r]   (NULL: skipped)
 *   d_states_i = W1[:, d:]ᵀ dz_i [batch, block, H]                (NULL: skipped)
 * where dz_i = (W2ᵀ G_i) ⊙ SiLU'(z_i) and the sums run over every block and
 * position.  The base logits carry no head parameter, so G reaches the head
 * through the correction only; d_states is where the GRU's own backward
 * through time would start.  Outputs are overwritten, not accumulated.
 *
 * hidden      [batch, block, d] head dtype, 16-byte aligned
 * gru_states  [batch, block, H] float32;  grad_final [batch, block, V] float32
 * outputs     float32, 4-byte aligned
 * workspace   device scratch of domino_correction_backward_workspace_size()
 *             bytes, 256-byte aligned.
 * batch in 0 … 128 (0 is a no-op), rank ≤ 512 (else DOMINO_ERR_UNSUPPORTED).
 * Arithmetic: float32, every sum in a fixed order (repeatable bits).
 */
int domino_correction_backward(const domino_head *head, int32_t batch, const void *hidden,
                               const float *gru_states, const float *grad_final, float *d_w2, float *d_b2,
                               float *d_w1, float *d_b1, float *d_states, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Workspace bytes domino_correction_backward needs for `batch` blocks. */
int domino_correction_backward_workspace_size(const domino_head *head, int32_t batch, size_t *bytes);

/*
 * Backward through time of the teacher-forced GRU causal encoder ([notes]
 * §二.1(2) item 1, §二.2(1)).  The forward it differentiates is the one
 * domino_draft_block runs with `teacher`: g_{-1} = 0, g_i = GRU(E[tok_i], g_{i-1}),
 * tok_0 = x_t[b], tok_i = teacher[b, i - 1].  Given d_states, the gradient of a
 * loss with respect to every g_i from outside the recurrence (the d_states of
 * domino_correction_backward), it writes the gradients of W_ih [3H, d],
 * W_hh [3H, H] and (NULL: skipped) b_ih, b_hh [3H], summed over every block
 * and position; the embedding table is frozen.  Outputs are overwritten.
 *
 * x_t [batch] and teacher [batch, block] int32 (ids outside [0, V) are
 * clamped); gru_states [batch, block, H] float32, the forward states;
 * d_states [batch, block, H] float32; outputs float32, 4-byte aligned.
 * workspace   device scratch of domino_gru_backward_workspace_size() bytes,
 *             256-byte aligned.
 * batch in 0 … 128 (0 is a no-op).  Arithmetic: float32, every sum in a
 * fixed order; for bf16 heads the input pre-activations W_ih e, and from
 * 128 rows (batch x block) on the two weight gradients, run on the matrix
 * cores, float32 factors split as bf16 hi + lo (the lo·lo term dropped, about
 * 2^-16 relative).
 */
int domino_gru_backward(const domino_head *head, int32_t batch, const int32_t *x_t, const int32_t *teacher,
                        const float *gru_states, const float *d_states, float *d_w_ih, float *d_w_hh,
                        float *d_b_ih, float *d_b_hh, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes domino_gru_backward needs for `batch` blocks. */
int domino_gru_backward_workspace_size(const domino_head *head, int32_t batch, size_t *bytes);

/*
 * Calibration hook: reads `bytes` bytes at `buf` (device memory) once, the way
 * the LM-head streams read (16-byte non-temporal loads, several in flight per
 * thread, a contiguous range for each of 2048 workgroups), and stores into
 * sink[j] (device memory, 2048 uint32) the XOR of the 32-bit words workgroup
 * j read, so the XOR of the 2048 entries is the XOR of the buffer.  Timing it
 * gives the read bandwidth a plain stream reaches on the device, the practical
 * ceiling of the HBM-bound kernels.  buf 16-byte aligned, bytes a multiple of
 * 16 (0 … 2^40).
 */
int domino_debug_read_stream(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/*
 * Test hook: out[j] = the Philox word that domino_draft_block uses for
 * vocabulary entry v0 + j of position pos of block b (see above).
 * out: device buffer of n uint32.  n in 0 … 2^26.
 */
int domino_debug_philox(uint64_t seed, uint32_t offset, int32_t b, int32_t pos, int32_t v0, int32_t n,
                        uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DOMINO_H_ */
