/*
 * flce.h -- C ABI of the MI355X (gfx950) fused linear cross-entropy library.
 *
 * The operation is the one the trl-lib "fused-linear-ce" kernel card
 * defines ("Full signature", "Metrics for free", "Algorithm"):
 *
 *   raw  = hidden @ weight^T                  (N x V, never stored)
 *   z    = c * tanh(s * (raw + bias) / c)     (bias optional; cap only if softcap > 0)
 *   lse  = log sum_j exp(z_ij)
 *   loss_i = lse_i - z_{i,t_i}   for rows whose target t_i != ignore_index, else 0
 *   loss = mean over non-ignored rows | sum | per-row vector   (reduction)
 *   metrics = { mean token accuracy (first-index argmax of z == target, over
 *               non-ignored rows), mean softmax entropy in nats (same rows) }
 *
 * and its gradients (card: "Algorithm"): with G = (softmax(z) - onehot(t))
 * scaled by the reduction and the upstream gradient and by dz/draw,
 *   grad_hidden = G @ weight,  grad_weight = G^T @ hidden,  grad_bias = sum_i G_i.
 *
 * Readings of points the card leaves open: the transform applies bias, then
 * logit_scale (a multiplier), then the soft cap c*tanh(x/c); "mean" divides
 * by the number of non-ignored rows; with no such row the mean loss and both
 * metrics are NaN and every gradient is 0; ignored rows have per-row loss 0.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and dense:
 *     hidden (N,H), weight (V,H), bias (V), targets (N) int64, grad_hidden
 *     (N,H), grad_weight (V,H), grad_bias (V); hidden and targets may
 *     instead follow the strided token layout of flce_problem_t.  hidden, weight, grad_hidden,
 *     grad_weight must be 16-byte aligned.  hidden/weight/bias and the
 *     gradient outputs share the problem's dtype; loss, lse, metrics and
 *     grad_loss are fp32.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream) and never synchronises the host.
 *   - The library never allocates, frees or retains device memory.  The
 *     caller owns every buffer, including `workspace`, which must hold at
 *     least the byte count the matching *_workspace_size function returns
 *     and must not be used by anything else until the call's work on
 *     `stream` has finished.  Calls that share a workspace must be ordered.
 *   - Host-detectable errors return a status before anything is launched;
 *     flce_last_error() then gives a thread-local message.  FLCE_ERR_HIP
 *     reports a HIP runtime failure (including "no device").
 *   - Out-of-range targets (not ignore_index, outside [0,V)) cannot be seen
 *     without a sync.  The forward gives such a row a NaN loss, so a mean or
 *     sum loss is NaN, and sets bit 0 of the device status word (read it with
 *     flce_forward_status); its lse and every other row's loss are unaffected.
 *     The backward gives the row's softmax-minus-one-hot row a NaN factor,
 *     so its grad_hidden row is NaN and, since grad_weight and grad_bias
 *     contract over every row, every entry of grad_weight and grad_bias is
 *     NaN too; the other rows of grad_hidden are unaffected.  (The Liger
 *     FLCE pull request's contract refuses bad input loudly rather than
 *     silently mis-scaling; a NaN that reaches every parameter gradient is
 *     this library's loud form of that, since it cannot raise without a sync.)
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FLCE_F32 = 0, FLCE_F16 = 1, FLCE_BF16 = 2 } flce_dtype_t;

typedef enum { FLCE_MEAN = 0, FLCE_SUM = 1, FLCE_NONE = 2 } flce_reduction_t;

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad size or option   */
  FLCE_ERR_UNSUPPORTED = 2,      /* valid but not handled (e.g. H not a multiple of 16 bytes) */
  FLCE_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required     */
  FLCE_ERR_HIP = 4               /* HIP runtime error (launch failure, no device)  */
} flce_status_t;

/* Problem description (card: "Full signature").  Plain data; the library
 * keeps no pointer to it after a call returns. */
typedef struct flce_problem {
  int64_t n_tokens;      /* N >= 0 rows of hidden / targets                         */
  int64_t hidden;        /* H >= 1; H * sizeof(dtype) must be a multiple of 16      */
  int64_t vocab;         /* V >= 1 rows of weight; N, V < 2^31                      */
  int64_t ignore_index;  /* rows with this target are ignored (default -100)        */
  int32_t dtype;         /* flce_dtype_t of hidden, weight, bias and gradients      */
  int32_t reduction;     /* flce_reduction_t                                        */
  float logit_scale;     /* s, finite (default 1.0)                                 */
  float softcap;         /* c: 0 = no cap; > 0 enables c*tanh(x/c); < 0, inf, NaN invalid */
  int32_t return_metrics;/* 0 / 1: also compute {accuracy, entropy}                 */
  int32_t has_bias;      /* 0 / 1: bias (V) present                                 */
  /* Plan overrides (0 = automatic).  They change the partition of the work,
   * not the result beyond fp32 summation order. */
  int32_t fwd_tiles_per_split; /* vocabulary tiles (256 ids) per forward split      */
  int32_t bwd_vocab_chunk;     /* vocabulary ids per backward chunk (multiple of 256) */
  /* Cross-entropy variants on the same vocabulary sweep (textbook
   * definitions, not the card's; 0 / NULL = plain cross-entropy, bit for bit):
   *   label_smoothing eps in [0, 1]: target (1 - eps) one-hot + eps/V uniform,
   *     row loss lse - (1 - eps) z_t - (eps/V) sum_j z_j;
   *   z_loss zl (finite): row loss += zl * lse^2;
   *   class_weight: device fp32 [V] or NULL: row i's whole loss times
   *     w[t_i]; the mean divides by the sum of w[t_i] over non-ignored rows
   *     (metrics stay unweighted).  Weights must be finite; not read for
   *     ignored rows or out-of-range targets. */
  float label_smoothing;
  float z_loss;
  const float* class_weight;
  /* Optional forward output: device int64 [N], each row's predicted token
   * (the first-index argmax of z, the one the accuracy metric uses; written
   * for ignored rows too), or NULL.  Requires return_metrics = 1. */
  int64_t* predictions;
  /* 1: grad_weight and grad_bias are written as fp32 arrays whatever the
   * input dtype (master-weight trainers); 0: in the input dtype. */
  int32_t grad_weight_fp32;
  /* Token layout; all zero means hidden (N,H) and targets (N,) contiguous.
   * Token n = s * seq_len + t (0 <= t < seq_len; N a multiple of seq_len)
   * has its hidden row at element s * hidden_seq_stride + t *
   * hidden_row_stride of hidden and its target at element s *
   * targets_seq_stride + t * targets_stride of targets, so that views such
   * as hidden[:, :-1, :] and labels[:, 1:] of an (S, T+1) batch are taken as
   * they are.  Zero selects the default: seq_len N, hidden_row_stride H,
   * hidden_seq_stride seq_len * hidden_row_stride, targets_stride 1,
   * targets_seq_stride seq_len * targets_stride.  Strides are >= 0 and
   * below 2^40 elements; the two hidden strides times sizeof(dtype) are
   * multiples of 16 bytes.  Outputs indexed by token (lse, loss rows,
   * predictions, grad_hidden) stay contiguous in n.  Hidden rows that are not contiguous are gathered
   * into the workspace first (2 N H sizeof(dtype) bytes moved), and so are
   * targets that are not (16 N bytes). */
  int64_t seq_len;
  int64_t hidden_row_stride;
  int64_t hidden_seq_stride;
  int64_t targets_stride;
  int64_t targets_seq_stride;
  /* Vocabulary shard: one device's share of a vocabulary split across
   * devices, the vocabulary-parallel FLCE that the Liger FusedLinearKLDivLoss
   * pull request (#1423, its rebase comment) names as #1428.  vocab_total =
   * 0: no shard (vocab_offset must be 0).  Otherwise weight, bias,
   * grad_weight and grad_bias hold ids [vocab_offset, vocab_offset + vocab)
   * of a vocabulary of vocab_total ids, while targets stay ids of the whole
   * vocabulary: a target inside the shard is its own, one inside
   * [0, vocab_total) but outside the shard belongs to another shard (no
   * target term here), one outside [0, vocab_total) is out of range (the
   * NaN behaviour above).  Used by flce_forward_shard and flce_backward;
   * flce_forward, flce_forward_noalloc and flce_forward_backward refuse it.
   * Not combined with label_smoothing, z_loss, class_weight or predictions
   * (FLCE_ERR_UNSUPPORTED); metrics come from flce_combine_shards. */
  int64_t vocab_offset;
  int64_t vocab_total;
  /* 1: flce_backward writes grad_hidden as an fp32 array whatever the input
   * dtype (for example one shard's part of grad_hidden, summed over the
   * shards in fp32); 0: in the input dtype. */
  int32_t grad_hidden_fp32;
} flce_problem_t;

/* Bytes of workspace flce_forward / flce_backward need for problem *p
 * (0 if *p is invalid; never fails otherwise).  Pure host function.
 * The caller allocates it: every entry point only writes to memory the
 * caller preallocated, the contract the tdt-loss pull request
 * (huggingface/kernels-community #882, its torch.compile comment) states for
 * the fake implementations of its ops. */
size_t flce_forward_workspace_size(const flce_problem_t* p);
size_t flce_backward_workspace_size(const flce_problem_t* p);

/* The forward's vocabulary splits for problem *p (card: "Algorithm", the
 * online log-sum-exp over tiles, and "Metrics for free"): each row's
 * vocabulary is swept in *n_splits runs of *tiles_per_split 256-id tiles (the
 * last run may be shorter), each ending in one partial state per row, merged
 * in a fixed order by the combine.  The split size depends on V only (or on
 * fwd_tiles_per_split), so a row's result does not depend on N.
 * *splits_per_workgroup consecutive splits of one 256-token tile are walked
 * by one workgroup; that grouping depends on N and changes no result.
 * Small fp32 problems (see flce_backward_plan) take no splits:
 * *tiles_per_split = *n_splits = *splits_per_workgroup = 0.
 * Pure host function; any output pointer may be NULL.
 * FLCE_ERR_INVALID_ARGUMENT or FLCE_ERR_UNSUPPORTED for an invalid *p. */
flce_status_t flce_forward_plan(const flce_problem_t* p, int32_t* tiles_per_split, int32_t* n_splits,
                                int32_t* splits_per_workgroup);

/* The backward's vocabulary chunking for problem *p (card: "Algorithm",
 * backward: each logit tile is recomputed; here the vocabulary is swept in
 * chunks of *chunk ids, the last one *last_chunk ids, *n_chunks in all, each
 * chunk's grad_weight rows complete after it).  *one_launch_per_chunk is 1
 * when each chunk's recompute and the previous chunk's two contractions run
 * in one launch (n_chunks + 1 launches of the GEMM kernel; 16-bit inputs
 * whose operand offsets fit 32 bits), else 0 (three kernels per chunk).
 * The default plan depends on H and V only (bwd_vocab_chunk overrides it).
 * fp32 problems of at most 256 tokens, 8192 ids and a hidden size of 1024
 * with the default plan run a small path without chunks (one workgroup per
 * token or per 8 vocabulary rows, plain fp32 FMAs): *chunk = V, *n_chunks = 1.
 * Pure host function; any output pointer may be NULL.
 * FLCE_ERR_INVALID_ARGUMENT or FLCE_ERR_UNSUPPORTED for an invalid *p. */
flce_status_t flce_backward_plan(const flce_problem_t* p, int64_t* chunk, int64_t* n_chunks,
                                 int64_t* last_chunk, int32_t* one_launch_per_chunk);

/* Forward pass (card: "Algorithm", forward; "Metrics for free").
 *   hidden, weight, targets, bias (NULL iff !has_bias): inputs as above.
 *   loss:    out, [1] for MEAN/SUM, [N] for NONE.
 *   lse:     out, [N] per-row log-sum-exp of z, the state the backward pass
 *            consumes; may be NULL when no backward follows.
 *   metrics: out, [2] = {mean_token_accuracy, entropy}; NULL iff !return_metrics.
 * The loss and lse are bit-identical whether or not metrics are requested. */
flce_status_t flce_forward(const flce_problem_t* p, const void* hidden, const void* weight,
                           const int64_t* targets, const void* bias, float* loss, float* lse,
                           float* metrics, void* workspace, size_t workspace_bytes,
                           void* stream);

/* The forward pass without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and results as
 * flce_forward (bit for bit), but the workspace is a fixed array of 32 MiB
 * per device inside the library, held until the process ends; the call
 * allocates nothing.  Problems whose forward workspace
 * (flce_forward_workspace_size) exceeds 32 MiB return FLCE_ERR_WORKSPACE
 * before anything is launched (e.g. a strided hidden layout that must be
 * gathered at N*H*sizeof(dtype) > ~30 MiB).  `stream` must belong to the
 * current device.  Every call on a device shares that device's array: calls
 * that overlap on one device (other streams, other threads) race and must
 * be ordered by the caller.  The device status word it writes lives in that
 * array, so flce_forward_status cannot read it; an out-of-range target still
 * shows as a NaN row loss. */
flce_status_t flce_forward_noalloc(const flce_problem_t* p, const void* hidden, const void* weight,
                                   const int64_t* targets, const void* bias, float* loss, float* lse,
                                   float* metrics, void* stream);

/* Backward pass (card: "Algorithm", backward: recompute each logit tile,
 * form p - onehot, accumulate the three gradients).
 *   lse:        in, [N] from flce_forward with the same problem and inputs.
 *   grad_loss:  in, device fp32 upstream gradient of the loss, [1] for
 *               MEAN/SUM, [N] for NONE; NULL means 1.
 *   grad_hidden (N,H), grad_weight (V,H), grad_bias (V): outputs, each may
 *               be NULL when not wanted (grad_bias requires has_bias).  They
 *               are overwritten, not accumulated into.  grad_weight and
 *               grad_bias are fp32 when grad_weight_fp32 = 1, grad_hidden
 *               when grad_hidden_fp32 = 1.
 * With a vocabulary shard (vocab_total > 0): lse is the whole vocabulary's
 * (flce_combine_shards), the mean divides by the non-ignored rows of the
 * whole batch, grad_weight and grad_bias are the shard's rows, and
 * grad_hidden is the shard's part: the sum over the shards is the gradient.
 * FLCE_ERR_UNSUPPORTED when n_tokens or the vocabulary chunk times
 * sizeof(dtype) reaches 16 MiB (the operand tiles use 32-bit offsets). */
flce_status_t flce_backward(const flce_problem_t* p, const void* hidden, const void* weight,
                            const int64_t* targets, const void* bias, const float* lse,
                            const float* grad_loss, void* grad_hidden, void* grad_weight,
                            void* grad_bias, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Forward and backward in one call, for callers that know the upstream
 * gradient when they compute the loss (the gradient-in-forward use of the
 * Liger FLCE pull requests, Summary: loss and gradients from one fused
 * call).  Same arguments as the two calls above; lse may be NULL (it is
 * then kept in the workspace), grad_loss as in flce_backward (NULL = 1; a
 * per-row [N] gradient with reduction NONE).  One workspace of
 * flce_forward_backward_workspace_size bytes serves both passes; the
 * forward's region comes first, so flce_forward_status reads it afterwards.
 * Results are bit-identical to flce_forward followed by flce_backward. */
size_t flce_forward_backward_workspace_size(const flce_problem_t* p);
flce_status_t flce_forward_backward(const flce_problem_t* p, const void* hidden, const void* weight,
                                    const int64_t* targets, const void* bias, float* loss, float* lse,
                                    float* metrics, const float* grad_loss, void* grad_hidden,
                                    void* grad_weight, void* grad_bias, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* One shard's part of the forward (vocabulary-parallel; p->vocab_total > 0,
 * see flce_problem_t): the card's "Algorithm" forward over the shard's ids
 * only.  For every row n:
 *   shard_lse[n]    = log sum over the shard's ids j of e^{z_nj};
 *   target_logit[n] = z_{n,t_n} if t_n is one of the shard's ids, else 0
 *                     (ignored rows and targets of other shards; NaN for a
 *                     target outside [0, vocab_total)).
 * Both outputs are device fp32 [N].  With return_metrics (card: "Metrics
 * for free"), also per row: shard_max[n] the largest logit over the shard's
 * ids, shard_argmax[n] its first id (an id of the whole vocabulary, int64),
 * shard_entropy[n] the entropy of the softmax over the shard's ids (nats);
 * these three are NULL iff !return_metrics.  p->reduction is not applied
 * here: flce_combine_shards turns the shards' outputs into the loss and the
 * metrics.  The workspace is flce_forward_workspace_size(p) bytes; the
 * status word is set as by flce_forward. */
flce_status_t flce_forward_shard(const flce_problem_t* p, const void* hidden, const void* weight,
                                 const int64_t* targets, const void* bias, float* shard_lse,
                                 float* target_logit, float* shard_max, int64_t* shard_argmax,
                                 float* shard_entropy, void* workspace, size_t workspace_bytes, void* stream);

/* The loss of a vocabulary split into n_shards shards, from the shards'
 * flce_forward_shard outputs brought together (what each device does after
 * gathering the per-row partials; on one device, the shards' calls in a
 * row).  p describes the whole problem: vocab is the whole vocabulary,
 * vocab_offset and vocab_total 0, and its reduction, ignore_index and token
 * layout, return_metrics and predictions apply; no loss variants.  The
 * shard arrays are device [n_shards][N] (shard-major, contiguous), the
 * shards in the order of their ids.  Writes
 *   lse[n]  = log sum_k e^{shard_lse[k][n]} (fp32, k in order, after the
 *             largest is taken out): the input of flce_backward;
 *   loss    = per p->reduction of the rows lse[n] - sum_k target_logit[k][n]
 *             (0 for ignored rows), as flce_forward would ([1] or [N]);
 *   metrics = {mean token accuracy, mean entropy} over non-ignored rows, from
 *             the argmax of the first shard holding the largest shard_max
 *             (the first id on ties) and H = lse - sum_k e^{lse_k - lse}
 *             (lse_k - shard_entropy_k); p->predictions gets that argmax.
 * lse may be NULL; shard_max, shard_argmax, shard_entropy and metrics are
 * NULL iff !return_metrics.  The workspace is
 * flce_combine_shards_workspace_size(p) bytes (its status word is readable
 * with flce_forward_status). */
size_t flce_combine_shards_workspace_size(const flce_problem_t* p);
flce_status_t flce_combine_shards(const flce_problem_t* p, int32_t n_shards, const float* shard_lse,
                                  const float* target_logit, const float* shard_max,
                                  const int64_t* shard_argmax, const float* shard_entropy,
                                  const int64_t* targets, float* loss, float* lse, float* metrics,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Synchronously reads the device status word the last flce_forward call
 * left in `workspace` (bit 0: a non-ignored target outside [0,V)).
 * Waits for `stream`.  Debug helper, not for hot loops. */
flce_status_t flce_forward_status(const flce_problem_t* p, const void* workspace,
                                  uint32_t* status_out, void* stream);

/* Host-side validation and refusal (the Liger FLCE pull request #1287,
 * Summary: host-side validation and by-design-refusal contracts, refusing
 * loudly): every entry point checks its arguments on the host before
 * anything is enqueued and returns a status instead of raising.
 * flce_status_str names a status ("FLCE_OK", ...; "FLCE_ERR_UNKNOWN" for
 * other values); flce_last_error returns this thread's message for the last
 * non-OK status (valid until this thread's next failing call; "" if none).
 * Both strings are owned by the library. */
const char* flce_status_str(flce_status_t s);
const char* flce_last_error(void);
const char* flce_version(void);
/* sizeof(flce_problem_t) as this library was built, for bindings that lay
 * the struct out themselves. */
size_t flce_problem_size(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
