/*
 * flce.h -- fused linear cross-entropy + entropy for the LM output head, on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (all from the pages on fusing the LM head with
 * cross-entropy and entropy):
 *
 *   z   = hidden[N,H] x weight[H,V]                       (logits, never stored)
 *   z'  = c * tanh(z / c) if softcap c > 0, else z          (Gemma2 cap)
 *   lse_i     = log sum_j exp(z'_ij)
 *   logprob_i = z'_{i,y_i} - lse_i                          (minus the cross-entropy)
 *   entropy_i = lse_i - sum_j p_ij z'_ij,  p_ij = exp(z'_ij - lse_i)
 *
 * and the gradients of  sum_i gbar_i logprob_i + ebar_i entropy_i  with respect
 * to hidden and weight. The extended entry points (flce_forward_ex,
 * flce_backward_ex) add two per-token outputs with their gradients:
 *
 *   uniform_ce_i = lse_i - (1/V) sum_j z'_ij    (cross-entropy against the uniform
 *                                                distribution: with weight eps,
 *                                                (1-eps)(-logprob) + eps uniform_ce
 *                                                is the label-smoothed cross-entropy)
 *   z_loss_i     = lam * lse_i^2                (z-loss with scale lam)
 *
 * a "sum" reduction, and fp32 gradient outputs. flce_forward_backward
 * returns the outputs and the gradients of one batch in a single call when
 * the upstream gradients are known in advance (the logit gradient formed from
 * logits kept during the forward, no recompute).
 *
 * Sources: verl pull request #462 (memory-efficient linear_cross_entropy),
 * sections "Equivalent compute logic" (the definition above, and that logprobs
 * are the negated cross-entropy) and "API" (hidden is [num_tokens,
 * hidden_size], weight is [hidden_size, vocab_size], labels are integer token
 * ids, a `reduction` argument); Liger-Kernel pull request #551 "[Verl] Add
 * entropy loss to cross_entropy_loss and fused_linear_cross_entropy_loss"
 * (Summary: both outputs without materialising the logits; review thread: the
 * mean divides by the number of non-ignored tokens); Liger-Kernel pull
 * request #435 "Fix LigerCrossEntropyLoss Reduction Behavior for 'None' Mode"
 * (Summary: reduction "none" returns the per-example vector; "Why we pass
 * gradient to output.backward()": a per-element upstream gradient for
 * non-scalar outputs); Liger-Kernel issue #127 "[feat] FusedLinearCrossEntropy
 * support for Gemma2" (proposal: an optional softcap applied after the head
 * matmul; discussion: tanh cap, gradients of hidden and weight by the chain
 * rule).
 *
 * The review thread of Liger-Kernel pull request #551 names a fused z-loss,
 * label smoothing and a sum reduction among the options of such a head,
 * without formulas; the definitions above are the usual ones (the smoothed
 * cross-entropy as torch.nn.functional.cross_entropy defines label_smoothing).
 *
 * Readings where those pages are silent:
 *   - A token whose label equals ignore_index gets every per-token output 0
 *     and no gradient, and is not counted by the mean.
 *   - reduction MEAN reduces each output over the n non-ignored tokens (n = 0
 *     gives 0), SUM sums them; the per-token vectors are written under every
 *     reduction.
 *   - A label that is neither ignore_index nor in [0, V) is treated as ignored
 *     and counted in the workspace status word (see flce_get_status).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers; the caller owns every
 *     buffer, including the workspace. The library allocates no device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     device work is enqueued on it; no call synchronises the device except
 *     flce_get_status and flce_profile_read, which say so.
 *   - Matrices are dense and row-major. bf16 means IEEE bfloat16 bits (uint16).
 *   - Alignment: hidden, weight, grad_hidden, grad_weight and the workspace
 *     must be 16-byte aligned, and H must be a multiple of 8
 *     (FLCE_ERR_MISALIGNED otherwise). V may take any value; when it is not a
 *     multiple of 8 the weight is read from a copy with 16-byte aligned rows
 *     and dW is formed in a buffer of that row stride and copied out (both in
 *     the workspace; flce_workspace_size and flce_fused_workspace_size count
 *     them). N, H and V need no other multiple.
 *   - Argument errors are detected on the host before anything is enqueued;
 *     then nothing is launched and no output is touched. A failed launch
 *     returns FLCE_ERR_HIP. No C++ exception crosses this interface.
 *   - Concurrent calls on different streams need distinct workspaces.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_NULL_POINTER = 1,      /* a required pointer is NULL */
  FLCE_ERR_BAD_SHAPE = 2,         /* N < 0, H < 1, V < 1, or a size beyond the limits below */
  FLCE_ERR_BAD_REDUCTION = 3,     /* reduction not FLCE_REDUCTION_NONE / _MEAN / _SUM */
  FLCE_ERR_MISALIGNED = 4,        /* see "Alignment" above */
  FLCE_ERR_WORKSPACE_TOO_SMALL = 5,
  FLCE_ERR_BAD_SOFTCAP = 6,       /* softcap is NaN or infinite */
  FLCE_ERR_HIP = 7,               /* a HIP runtime call or kernel launch failed */
  FLCE_ERR_INVALID_LABEL = 8,     /* reported only by flce_get_status */
  FLCE_ERR_BAD_OPTION = 9,        /* z_loss_scale negative or not finite, unknown grad_dtype,
                                   * class_weight under NONE, entropy_per_token not 0 or 1 */
  FLCE_ERR_TOO_LARGE = 10         /* flce_forward_noalloc: the shape needs more scratch than
                                   * FLCE_NOALLOC_SCRATCH_BYTES */
} flce_status_t;

enum { FLCE_REDUCTION_NONE = 0, FLCE_REDUCTION_MEAN = 1, FLCE_REDUCTION_SUM = 2 };
enum { FLCE_GRAD_BF16 = 0, FLCE_GRAD_F32 = 1 };

/* Size limits: N <= 2^21, H <= 2^20, V <= 2^22 - 256, and V <= 2^21 with
 * fp32 gradient outputs (FLCE_ERR_BAD_SHAPE beyond). */

/* Workspace bytes needed by the forward (*fwd_bytes) and backward
 * (*bwd_bytes) entry points for this shape and reduction. Host only; either
 * out-pointer may be NULL. The forward size is about 16 * N * ceil(V/256) +
 * 2 * N * H bytes (one partial softmax state per token and 256-wide
 * vocabulary tile, and a re-laid-out copy of hidden). The backward size holds
 * a slice of Vc vocabulary columns of the logit gradient in two bf16 layouts
 * (4 * Np * Vc bytes, Np = 256*ceil(N/256); independent of V): Vc fills
 * 1 GiB while that gives at least 16384 columns, is 16384 up to 4 GiB, and
 * beyond that whatever fits in 4 GiB, down to a floor of 2048 columns. Then
 * re-laid-out copies of hidden and of the weight slice, and, when the slice
 * does not cover the whole vocabulary or dH is K-split, fp32 accumulators of
 * N*H*4 bytes each. */
flce_status_t flce_workspace_size(int64_t N, int64_t H, int64_t V, int reduction,
                                  size_t* fwd_bytes, size_t* bwd_bytes);

/* Forward. The call shape of the API example of verl pull request #462
 * (section "API": hidden [num_tokens, hidden_size], weight [hidden_size,
 * vocab_size], integer labels, a reduction argument, two outputs), with the
 * outputs of its section "Equivalent compute logic" (per-token entropy and the
 * label log-probability, the negated cross-entropy) and the cap of
 * Liger-Kernel issue #127 (proposal: applied after the head matmul).
 *   hidden   device bf16 [N,H]        weight  device bf16 [H,V]
 *   labels   device int64 [N]         ignore_index: label value that marks a skipped token
 *   softcap  c > 0 caps logits as c*tanh(z/c); c <= 0 disables the cap
 *   lse, logprob, entropy   device fp32 [N] outputs (always written).
 *                           Keep lse and entropy for flce_backward.
 *   logprob_mean, entropy_mean  device fp32 [1] outputs; required when
 *                           reduction is MEAN (the means) or SUM (the sums),
 *                           ignored under NONE.
 *   workspace  device scratch of at least the forward size from
 *              flce_workspace_size; its first 256 bytes hold the status word.
 */
flce_status_t flce_forward(const void* hidden, const void* weight, const int64_t* labels,
                           int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                           float softcap, int reduction,
                           float* lse, float* logprob, float* entropy,
                           float* logprob_mean, float* entropy_mean,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Backward: writes grad_hidden = dL/dhidden (device bf16 [N,H]) and
 * grad_weight = dL/dweight (device bf16 [H,V]) for
 *   L = sum_i gbar_i logprob_i + ebar_i entropy_i.
 * Liger-Kernel pull request #435 ("Why we pass gradient to output.backward()")
 * fixes the convention: an unreduced output takes one upstream gradient per
 * element, a reduced one a scalar; the review thread of Liger-Kernel pull
 * request #551 fixes the mean's divisor (the non-ignored tokens) and issue #127
 * (discussion) the cap's chain rule into both gradients.
 * hidden, weight, labels, N, H, V, ignore_index, softcap and reduction must be
 * those of the matching flce_forward; lse and entropy are its outputs.
 *   reduction NONE: grad_logprob, grad_entropy are device fp32 [N]
 *                   (gbar_i = grad_logprob[i]).
 *   reduction MEAN: they are device fp32 [1], the gradients of the two means
 *                   (gbar_i = grad_logprob[0] / n on non-ignored tokens).
 *   reduction SUM:  device fp32 [1], the gradients of the two sums
 *                   (gbar_i = grad_logprob[0] on non-ignored tokens).
 * Either gradient pointer may be NULL, meaning zero. Ignored tokens get zero
 * rows in grad_hidden. The logit gradient is recomputed, not stored by the
 * forward.
 */
flce_status_t flce_backward(const void* hidden, const void* weight, const int64_t* labels,
                            int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                            float softcap, int reduction,
                            const float* lse, const float* entropy,
                            const float* grad_logprob, const float* grad_entropy,
                            void* grad_hidden, void* grad_weight,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Arguments, outputs and errors as flce_forward, minus
 * the workspace: the call runs in a scratch array of FLCE_NOALLOC_SCRATCH_BYTES
 * that the library holds in every device it runs on until the process ends
 * (its address is looked up once per device, on the first call with that
 * device current; `stream` must belong to the current device). Shapes whose
 * forward workspace (flce_workspace_size) exceeds that size are refused with
 * FLCE_ERR_TOO_LARGE before anything is enqueued (about N * (16 ceil(V/256) +
 * 2 H) bytes must fit, e.g. N = 2048 at H = 4096, V = 128256; a vocabulary
 * that is not a multiple of 8 adds 2 H V). The call allocates nothing,
 * enqueues kernels only, and writes every scratch byte it reads before
 * reading it. All calls on one device share that device's array: calls that
 * overlap in time on one device (two streams, two threads) race and give
 * wrong results; serialise them. The invalid-label count of these calls is
 * not reported (flce_get_status needs a workspace); such labels are treated
 * as ignored as in flce_forward. */
#define FLCE_NOALLOC_SCRATCH_BYTES (64u << 20)
flce_status_t flce_forward_noalloc(const void* hidden, const void* weight, const int64_t* labels,
                                   int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                                   float softcap, int reduction,
                                   float* lse, float* logprob, float* entropy,
                                   float* logprob_mean, float* entropy_mean, void* stream);

/* Options of the extended entry points. class_weight was added in version
 * 211 (flce_version), entropy_per_token in version 212; the struct grew from
 * 24 to 32 and then to 40 bytes, so callers built against an older header must
 * be rebuilt. A zero-initialised tail keeps the earlier behaviour. */
typedef struct flce_options {
  int64_t ignore_index;  /* label value that marks a skipped token */
  float softcap;         /* c > 0: z' = c*tanh(z/c); c <= 0: no cap; must be finite */
  int reduction;         /* FLCE_REDUCTION_NONE, _MEAN or _SUM */
  float z_loss_scale;    /* lam >= 0 (finite) of z_loss = lam * lse^2 */
  int grad_dtype;        /* FLCE_GRAD_BF16 or FLCE_GRAD_F32: type of grad_hidden/grad_weight */
  const float* class_weight; /* NULL, or device fp32 [V] (the whole vocabulary; 4-byte
                              * aligned, finite values): target weights of the MEAN and
                              * SUM reductions, see below; FLCE_ERR_BAD_OPTION under NONE */
  int entropy_per_token; /* 0: the entropy follows `reduction` like the other outputs;
                          * 1: under MEAN or SUM the entropy is taken per token while the
                          * other outputs are reduced, so the backward's grad_entropy is
                          * device fp32 [N] (ebar_i = grad_entropy[i], no class weight) and
                          * the other upstream gradients stay [1]; the verl pull request
                          * #462 "Equivalent compute logic" returns entropy per token beside
                          * a reduced logprob. Any other value: FLCE_ERR_BAD_OPTION. The
                          * forward writes the per-token entropy under every reduction
                          * (reduced[1] is still the entropy's reduction). */
} flce_options_t;

/* Target (class) weights. The Liger-Kernel PR #551 review ("[Verl] Add
 * entropy loss to cross_entropy_loss and fused_linear_cross_entropy_loss")
 * lists target weights among the fused options and normalises the weighted
 * case by the weight of the non-ignored tokens instead of their count. With
 * class_weight set, a valid token t carries w_t = class_weight[labels[t]]:
 *   MEAN  reduced[k] = sum_t w_t x_t / sum_t w_t  (0 when the weight sum is 0),
 *         and the scalar upstream gradient g of output k reaches token t as
 *         g * w_t / sum_t w_t;
 *   SUM   reduced[k] = sum_t w_t x_t, gradient g * w_t,
 * for all four outputs x (logprob, entropy, uniform_ce, z_loss). For the
 * cross-entropy this is torch.nn.functional.cross_entropy(weight=...). The
 * per-token vectors stay unweighted. The weight sum is accumulated in
 * float64 in a fixed order. The sharded calls take the same weights (over
 * V_total) in flce_merge_shards and flce_backward_shard; flce_forward_shard
 * ignores them. */

/* Extended forward. As flce_forward, plus
 *   uniform_ce, z_loss  device fp32 [N] outputs, each optional (NULL = not
 *                       written);
 *   reduced             device fp32 [4]: the reductions (MEAN: means over the
 *                       n non-ignored tokens; SUM: sums) of logprob, entropy,
 *                       uniform_ce and z_loss, in that order; required unless
 *                       reduction is NONE, ignored then.
 * The workspace size is the forward size of flce_workspace_size. */
flce_status_t flce_forward_ex(const void* hidden, const void* weight, const int64_t* labels,
                              int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                              float* lse, float* logprob, float* entropy,
                              float* uniform_ce, float* z_loss, float* reduced,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Extended backward: grad_hidden [N,H] and grad_weight [H,V] (device; bf16
 * or fp32 as opt->grad_dtype says) of
 *   L = sum_i gbar_i logprob_i + ebar_i entropy_i + gu_i uniform_ce_i + gz_i z_loss_i,
 * with the four upstream gradients given as for flce_backward (device fp32,
 * [N] under NONE, [1] under MEAN and SUM; NULL means zero). opt and the
 * tensors must be those of the matching flce_forward_ex. The workspace size is
 * the backward size of flce_workspace_size. */
flce_status_t flce_backward_ex(const void* hidden, const void* weight, const int64_t* labels,
                               int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                               const float* lse, const float* entropy,
                               const float* grad_logprob, const float* grad_entropy,
                               const float* grad_uniform_ce, const float* grad_z_loss,
                               void* grad_hidden, void* grad_weight,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---- Vocabulary-sharded head ------------------------------------------------
 * The vocabulary is split into slices [v_begin, v_begin + Vs) of V_total
 * classes, each with its own weight slice weight_shard [H,Vs] (row-major, the
 * columns v_begin .. v_begin+Vs-1 of the full [H,V_total] weight), e.g. one per
 * GPU under tensor parallelism. Labels stay global class ids.
 *
 *   1. flce_forward_shard per slice: the per-token online-softmax state of the
 *      slice, {m, s, u, sum z'} with lse_slice = m + ln s, and the label logit
 *      (0 when the label lies in another slice). 20 bytes per token.
 *   2. Gather the S slices' states into [S,N,4] and label logits into [S,N]
 *      (an all-gather across GPUs) and call flce_merge_shards once: it merges
 *      them in slice order with the same combine as the unsharded forward and
 *      writes the outputs of flce_forward_ex.
 *   3. flce_backward_shard per slice with the merged lse and entropy: the
 *      slice's grad_weight [H,Vs] and its partial grad_hidden [N,H]; the sum
 *      over slices of the partials is grad_hidden (an all-reduce across GPUs;
 *      fp32 partials, opt->grad_dtype = FLCE_GRAD_F32, keep that sum exact to
 *      fp32 rounding).
 * The slice calls need Vs, v_begin within V_total (FLCE_ERR_BAD_SHAPE
 * otherwise); Vs follows the rules of V above; v_begin has no alignment rule.
 */

/* Slice forward. hidden, labels as flce_forward_ex; opt->reduction is ignored.
 *   state        device fp32 [N,4], 16-byte aligned: per token {m, s, u, sum z'}
 *                of the slice (natural-log units; {-1e30, 0, 0, 0} for ignored
 *                tokens)
 *   label_logit  device fp32 [N]: the capped label logit if the label lies in
 *                this slice, else 0
 * Workspace: the forward size of flce_workspace_size(N, H, Vs, ...). */
flce_status_t flce_forward_shard(const void* hidden, const void* weight_shard,
                                 const int64_t* labels, int64_t N, int64_t H, int64_t Vs,
                                 int64_t v_begin, int64_t V_total, const flce_options_t* opt,
                                 float* state, float* label_logit, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Workspace bytes of flce_merge_shards for N tokens (host only). */
flce_status_t flce_merge_workspace_size(int64_t N, size_t* bytes);

/* Merge of S slices: states device fp32 [S,N,4] and label_logits device fp32
 * [S,N] from flce_forward_shard (slice s at offset s*N*4 / s*N; any slice
 * order, merged in array order). Outputs as flce_forward_ex (lse, logprob,
 * entropy required when N > 0; uniform_ce, z_loss optional; reduced [4]
 * required unless reduction is NONE). 1 <= S <= 65536. */
flce_status_t flce_merge_shards(const float* states, const float* label_logits, int64_t S,
                                const int64_t* labels, int64_t N, int64_t V_total,
                                const flce_options_t* opt, float* lse, float* logprob,
                                float* entropy, float* uniform_ce, float* z_loss, float* reduced,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Slice backward: arguments as flce_backward_ex with lse and entropy from
 * flce_merge_shards; writes grad_weight_shard [H,Vs] (the slice's columns of
 * grad_weight) and grad_hidden_partial [N,H], this slice's share of
 * grad_hidden. Workspace: the backward size of flce_workspace_size(N, H, Vs,
 * ...). */
flce_status_t flce_backward_shard(const void* hidden, const void* weight_shard,
                                  const int64_t* labels, int64_t N, int64_t H, int64_t Vs,
                                  int64_t v_begin, int64_t V_total, const flce_options_t* opt,
                                  const float* lse, const float* entropy,
                                  const float* grad_logprob, const float* grad_entropy,
                                  const float* grad_uniform_ce, const float* grad_z_loss,
                                  void* grad_hidden_partial, void* grad_weight_shard,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---- Fused forward + backward (gradient in the forward) ----------------------
 * When the upstream gradients are known before the forward runs (a terminal
 * loss such as the mean cross-entropy, or per-token weights fixed in
 * advance), the logit gradient can be formed from logits kept during the
 * forward instead of recomputing them in the backward: this is how the fused
 * linear cross-entropy of Liger-Kernel pull request #551 (item 1 of its
 * description) produces the loss and its input gradient in one pass. Here the
 * tokens are taken in chunks; per chunk the capped logits of the whole
 * vocabulary are kept as z' - m in bf16 (m: the maximum over 128 vocabulary
 * rows, so the rounding error is relative to the distance from the maximum),
 * and the gradient is formed from them once the chunk's logsumexp is known.
 * Compared with flce_forward_ex + flce_backward_ex this saves the backward's
 * logit GEMM (2*N*H*V flops) and costs workspace and HBM traffic:
 *   chunk images  4 * 256*ceil(Nc/256) * 256*ceil(V/256) bytes,
 *   the weight re-laid out, 2 * H * 256*ceil(V/256) bytes,
 *   with more than one chunk and bf16 gradients, an fp32 dW accumulator of
 *   4 * H * V bytes (fp32 gradients accumulate in grad_weight itself).
 * The results agree with flce_forward_ex followed by flce_backward_ex to the
 * rounding of the kept logits (bf16 of z' - m), not bit for bit.
 *
 * chunk_tokens: tokens per chunk Nc (rounded up to 256); 0 picks the largest
 * multiple of 256 whose chunk images fit in 1 GiB (the budget of the
 * backward's logit-gradient images; at least 256 tokens), e.g. 2048 tokens at
 * V = 128256. A larger chunk saves passes over the fp32 dW accumulator at the
 * price of memory; chunk_tokens >= N keeps every logit of the call (4 bytes
 * each) in one chunk. V <= 2^21.
 * Workspace bytes for this shape, options and chunk_tokens (host only): */
flce_status_t flce_fused_workspace_size(int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                                        int64_t chunk_tokens, size_t* bytes);

/* The outputs of flce_forward_ex (lse, logprob, entropy required when N > 0;
 * uniform_ce, z_loss optional; reduced [4] required unless reduction is NONE)
 * and the gradients of flce_backward_ex (grad_hidden [N,H], grad_weight [H,V],
 * bf16 or fp32 as opt->grad_dtype says) for the upstream gradients given here
 * as for flce_backward_ex ([N] under NONE, [1] under MEAN and SUM, NULL =
 * zero). Under MEAN the scalar gradients are divided by the number of valid
 * tokens counted by this call. Errors as flce_backward_ex; FLCE_ERR_BAD_SHAPE
 * also for V > 2^21 or chunk_tokens < 0. */
flce_status_t flce_forward_backward(const void* hidden, const void* weight, const int64_t* labels,
                                    int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                                    int64_t chunk_tokens, const float* grad_logprob,
                                    const float* grad_entropy, const float* grad_uniform_ce,
                                    const float* grad_z_loss, float* lse, float* logprob,
                                    float* entropy, float* uniform_ce, float* z_loss,
                                    float* reduced, void* grad_hidden, void* grad_weight,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Reads the status word that the last flce_forward / flce_backward /
 * flce_forward_backward on this workspace left, after synchronising `stream`. *invalid_labels (may be NULL)
 * receives the number of labels that were neither ignore_index nor in [0, V);
 * returns FLCE_ERR_INVALID_LABEL if that number is not 0, else FLCE_OK. */
flce_status_t flce_get_status(const void* workspace, int64_t* invalid_labels, void* stream);

/* Static English text for a status code. */
const char* flce_status_string(flce_status_t status);

/* Library version, major*10000 + minor*100 + patch. */
int flce_version(void);

/* Measurement hooks. When enabled, every kernel the library launches is
 * bracketed by a pair of hipEvents recorded on the launch stream; the host
 * side keeps one table per kernel kind. Host state, not thread-safe; meant for
 * benchmarks. */
flce_status_t flce_profile_enable(int enable);
flce_status_t flce_profile_reset(void);
/* Number of kernel kinds in the table. */
int flce_profile_kinds(void);
/* Synchronises the recorded events, then returns the name, the number of
 * launches and the summed duration (ms) of kernel kind `kind`. */
flce_status_t flce_profile_read(int kind, const char** name, int64_t* launches, double* total_ms);

/* Measurement hook, for context in benchmarks: the bf16 MFMA rate (TFLOP/s,
 * in *tflops) that this device sustains in the GEMM kernels' wave tile: one
 * 512-thread block per CU (two waves per SIMD), each wave running `steps`
 * (4 <= steps <= 2^24, rounded down to a multiple of 4) 16-wide K steps of
 * 4 x 2 v_mfma_f32_32x32x16_bf16, with the GEMM kernels' data movement added
 * by `mode`:
 *   0  operands held in registers, pseudo-random bf16 in [-2, 2);
 *   1  the same with zero operands;
 *   2  mode 0 with each step's six operand fragments read from LDS
 *      (ds_read_b128);
 *   3  mode 2 plus the global -> LDS DMA of a 256 x 256 block tile (32 KiB per
 *      block per 32-deep K block) from a 2 MiB window that stays in L2.
 * The published dense peak assumes a clock that the matrix cores hold on
 * zero operands but not under the power they draw on varying data; modes 2
 * and 3 show what the LDS and L2 traffic of the tile costs on top.
 * workspace: device, 16-byte aligned, at least 256 * 512 * 4 bytes (results)
 * plus 2 MiB for mode 3 (the DMA window, filled here). Synchronises `stream`.
 * FLCE_ERR_BAD_OPTION for another mode. */
flce_status_t flce_probe_mfma_rate(int mode, int64_t steps, double* tflops, void* workspace,
                                   size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
