/*
 * kd_fused_kl.h — C ABI of the fused, chunked top-K KL distillation loss on
 * AMD MI355X (gfx950).
 *
 * Source pages (cited by title and section):
 *  [P1] "Distilação de LLMs mais barata: top-K offline e KL fundida cortam
 *       VRAM em até 15x" (imasters.com.br)
 *  [P3] "Destilación de LLMs: Multiverse Computing reduce memoria 15× con
 *       1 GPU" (ecosistemastartup.com)
 *  [P4] "Hugging Face：让知识蒸馏廉价到可大规模运行" (feinterview.poetries.top)
 *  [P5] "Chunkovaná KL strata umožnila destilovať LLM s 32-tisícovým
 *       kontextom na jednom H200" (aifeed.sk)
 *
 * What the library computes. Student hidden states H[N,d] are projected
 * through the output head W[V,d] one chunk of positions at a time; the logits
 * of a chunk are folded into an accumulated loss and discarded, and the
 * backward pass recomputes them instead of storing them ([P1] "As duas
 * mudanças"; [P4] 为什么蒸馏恢复代价高昂, "Fused chunked KL" paragraph). The
 * teacher side is an offline top-K cache: for each position, K token ids and
 * their log-probabilities, not renormalised ([P4] 离线蒸馏; [P5] "Čo dopĺňajú
 * podrobnejšie experimenty"). With z = H Wᵀ, lse_r = log Σ_j exp z_rj over the
 * full vocabulary, p_rk = exp(logp_rk) and S_r = Σ_k p_rk:
 *
 *   loss_tok[r] = Σ_k p_rk (logp_rk − z_r,idx_rk + lse_r)   (forward KL)
 *   loss_sum    = Σ_r loss_tok[r]                          (sum over rows)
 *   dlogits_rj  = g (S_r exp(z_rj − lse_r) − Σ_k p_rk [j = idx_rk])
 *   dH = dlogits W,  dW = dlogitsᵀ H
 *
 * which is the dense KL of the pages' correctness baseline rewritten so that
 * no N×V grid exists ([P4], the three variants are mathematically
 * equivalent). Chunk size is the caller's memory/speed knob ([P3]
 * "Implementación práctica").
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller, row-major
 *    and contiguous. H, W and dH rows must start on 16-byte boundaries
 *    (d*sizeof(element) % 16 == 0 and 16-byte aligned base pointers).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously on it; the library never allocates,
 *    frees, synchronises or prints.
 *  - `workspace` is a caller-owned device buffer of at least
 *    kd_fused_kl_workspace_bytes(...) bytes, 256-byte aligned; its contents
 *    on entry are irrelevant and on exit unspecified.
 *  - Invalid arguments are reported by the return value BEFORE anything is
 *    enqueued. A failed launch returns KD_ERR_HIP.
 *  - Preconditions not checked on the hot path: teacher ids are distinct
 *    within a row; logp values are <= 0 and finite or −inf (−inf means p = 0
 *    and the entry contributes nothing). Ids outside [0, V) are skipped by
 *    the kernels (never dereferenced) and count as p = 0.
 *    kd_fused_kl_check_inputs checks all three on request.
 *  - Results are deterministic: every reduction runs in a fixed order.
 *  - Calls that share one workspace must not overlap.
 */
#ifndef KD_FUSED_KL_H
#define KD_FUSED_KL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
  KD_OK = 0,
  KD_ERR_INVALID_ARG = 1, /* a size, pointer, alignment or flag is invalid */
  KD_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels take  */
  KD_ERR_WORKSPACE = 3,   /* workspace NULL, misaligned or too small        */
  KD_ERR_HIP = 4          /* a kernel launch failed                         */
} kd_status;

/* Element type of H, W and dH. */
typedef enum { KD_F32 = 0, KD_BF16 = 1 } kd_dtype;

/* Which pass a workspace query is for. */
typedef enum {
  KD_PASS_FWD = 0,
  KD_PASS_BWD = 1,
  KD_PASS_TEACHER = 2,
  KD_PASS_FWD_BWD = 3 /* kd_fused_kl_fwd_bwd: loss and gradients in one call */
} kd_pass;

/* How per-position losses are accumulated (the _ex entry points). */
typedef enum { KD_REDUCE_SUM = 0, KD_REDUCE_MEAN = 1 } kd_reduction;

/* Human-readable name of a status code; never NULL. */
const char* kd_status_str(int status);

/*
 * Bytes of workspace kd_fused_kl_fwd (pass = KD_PASS_FWD), kd_fused_kl_bwd
 * (pass = KD_PASS_BWD), kd_teacher_topk (KD_PASS_TEACHER) or
 * kd_fused_kl_fwd_bwd (KD_PASS_FWD_BWD) needs for these sizes. Returns 0 if the sizes are
 * invalid (the same checks the entry points make). The backward workspace
 * holds the dlogits of a window of consecutive chunks, window × chunk × V
 * elements of `dtype` (padded to the kernel tile), where the window is
 * min(4, max(1, 4096 / chunk)) chunks; dW is contracted once per window. It
 * grows with the chunk, never with N × V. The forward and backward passes
 * also bucket the cached entries of up to 65,536 positions at a time (about
 * 8·K bytes per position). One launch of the forward's logit GEMM covers up
 * to 16,384 positions (whole chunks, at least one), and the forward holds
 * their logsumexp partials (8 bytes per position and 256 vocabulary entries)
 * and, in bf16, their transposed rows of H (2·d bytes per position); the
 * backward holds the transposed rows of one window. KD_PASS_FWD_BWD needs
 * the backward's window and one chunk of float32 logits (chunk × V × 4
 * bytes), and no buckets.
 */
size_t kd_fused_kl_workspace_bytes(int pass, int64_t N, int64_t d, int64_t V, int64_t K,
                                   int64_t chunk, int dtype);

/*
 * Forward: loss of every position, the saved log-normaliser, and their sum.
 *
 *  H         [N, d] of `dtype` — student hidden states.
 *  W         [V, d] of `dtype` — output head (student projection).
 *  topk_idx  [N, K] int32 — cached teacher token ids.
 *  topk_logp [N, K] float32 — cached teacher log-probabilities.
 *  N, d, V, K, chunk — sizes; 1 <= K <= V, chunk >= 1, N >= 0.
 *  loss_tok  [N] float32 or NULL — per-position loss.
 *  lse       [N] float32 — log Σ_j exp z_rj, saved for the backward pass.
 *  loss_sum  [1] float32 — Σ_r loss_tok[r], reduced in a fixed order.
 *
 * N = 0 writes loss_sum = 0. Rows are processed `chunk` at a time; one
 * launch of the logit GEMM projects the chunks of up to 16,384 rows.
 *
 * Returns KD_ERR_UNSUPPORTED for sizes the kernels do not take: K > 16383,
 * d > 2^20, N >= 2^31, a padded vocabulary row of 8 MiB or more
 * (V > 4,194,048 in bf16, V > 2,096,896 in float32), or a chunk so large
 * that one launch would need 2^24 workgroups or more (the logit tiles of a
 * chunk, ⌈chunk/256⌉·⌈V/256⌉; the dH or dW tiles of a window; one
 * workgroup per row of a chunk).
 */
int kd_fused_kl_fwd(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                    const float* topk_logp, int64_t N, int64_t d, int64_t V, int64_t K,
                    int64_t chunk, float* loss_tok, float* lse, float* loss_sum, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Backward: recomputes each chunk's logits from H and W (they are never
 * stored between passes), forms dlogits in registers, writes them once for
 * the chunk, and contracts them into dH and dW.
 *
 *  H, W, topk_idx, topk_logp, N, d, V, K, chunk — as in the forward pass.
 *  lse        [N] float32 — the forward pass's output for the same inputs.
 *  grad_loss  [1] float32, DEVICE pointer — g = ∂objective/∂loss_sum (a
 *             mean over tokens is g = 1/N); read by the kernels, so no host
 *             synchronisation is needed.
 *  dH         [N, d] of `dtype`, or NULL to skip — overwritten.
 *  dW         [V, d] float32, or NULL to skip — overwritten when
 *             dW_accumulate == 0, added to when dW_accumulate == 1.
 */
int kd_fused_kl_bwd(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                    const float* topk_logp, const float* lse, int64_t N, int64_t d, int64_t V,
                    int64_t K, int64_t chunk, const float* grad_loss, void* dH, float* dW,
                    int dW_accumulate, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-position weights or masks, and the mean reduction, for packed
 * sequences. The Hugging Face post on cheap distillation lists sequence
 * packing among the paper's ablations (section 得到的 student). Packing
 * needs a weight or mask per position. Its reading here:
 *
 *   loss = Σ_r w_r L_r                  (reduction = KD_REDUCE_SUM)
 *   loss = Σ_r w_r L_r / Σ_r w_r        (reduction = KD_REDUCE_MEAN; 0 if Σ w = 0)
 *
 * with L_r the per-position KL of kd_fused_kl_fwd and the gradient scaled per
 * row accordingly: dlogits_r = g · w_r / den · (S_r q_r − p_r), where den is
 * Σ_r w_r for the mean and 1 for the sum.
 *
 *  weight     [N] float32 device pointer, or NULL for w_r = 1 (then the
 *             mean divides by N). Any finite values; 0 masks a position.
 *  reduction  KD_REDUCE_SUM or KD_REDUCE_MEAN; anything else is
 *             KD_ERR_INVALID_ARG.
 *  loss       [1] float32 — the reduced loss (the `loss_sum` of
 *             kd_fused_kl_fwd).
 *  loss_tok   stays the unweighted L_r.
 *
 * The other arguments, the workspace and the errors are those of
 * kd_fused_kl_fwd / kd_fused_kl_bwd, which are these calls with
 * weight = NULL and KD_REDUCE_SUM. Pass the same weight and reduction to
 * both passes.
 */
int kd_fused_kl_fwd_ex(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                       const float* topk_logp, const float* weight, int reduction, int64_t N,
                       int64_t d, int64_t V, int64_t K, int64_t chunk, float* loss_tok, float* lse,
                       float* loss, void* workspace, size_t workspace_bytes, void* stream);

int kd_fused_kl_bwd_ex(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                       const float* topk_logp, const float* weight, int reduction, const float* lse,
                       int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                       const float* grad_loss, void* dH, float* dW, int dW_accumulate,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward pass without a workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, and harnesses that forbid allocation.
 *
 * Arguments, results and errors are those of kd_fused_kl_fwd_ex with the
 * workspace left out. The scratch the forward needs (the bucketed cache of a
 * group of chunks, the transposed chunks of H, the tile partials, and the
 * per-position losses when loss_tok is NULL) lives instead in a device array
 * held by the library: KD_NOALLOC_SCRATCH_BYTES bytes on every GPU the
 * library runs on, kept until the process ends. When the forward workspace,
 * kd_fused_kl_workspace_bytes(KD_PASS_FWD, ...), exceeds it, the call
 * projects one chunk per launch of the logit GEMM instead of a group of
 * chunks: the same results bit for bit, from a smaller scratch. Sizes that
 * exceed it even so are rejected with KD_ERR_WORKSPACE before anything is
 * enqueued. 64 MiB holds the forward of the 8K-token head (17 MiB one chunk
 * per launch), of 32,768 tokens at d = 3072, V = 128,256, K = 100, chunk
 * 2048 (46 MiB) and of the 201,088-token head at the same N (50 MiB); from
 * 65,536 tokens at K = 100 the bucketed cache alone takes 52 MiB and the call
 * is rejected. The stream must belong to the current device
 * (KD_ERR_INVALID_ARG otherwise).
 *
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress); make it once outside graph capture. No call
 * allocates or frees device memory or calls hipMemset; the scratch is
 * cleared by fill kernels. Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (two streams, or two host threads) race and give
 * undefined results. Kernel timing (kd_timing_enable) is not recorded for
 * this call, since recording it would create events.
 */
#define KD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kd_fused_kl_fwd_noalloc(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                            const float* topk_logp, const float* weight, int reduction,
                            int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                            float* loss_tok, float* lse, float* loss, void* stream);

/*
 * Loss and gradients in one call, for callers that know the upstream
 * gradient g when they compute the loss (g = 1 for a loss that is the
 * objective, or a fixed scale).
 *
 * The two-pass calls above follow the pages' schedule: the forward discards
 * each chunk's logits and the backward recomputes them ("Distilação de LLMs
 * mais barata ...", section "As duas mudanças": the projection is done twice).
 * Here each chunk's logits are projected once. They are kept in float32 in
 * the workspace only until that chunk's lse is known, turned into dlogits by
 * a streaming pass, and then discarded. The workspace grows by chunk × V × 4
 * bytes, still never with N × V, and the logit GEMM runs three times per
 * chunk instead of four.
 *
 * The result equals kd_fused_kl_fwd_ex followed by kd_fused_kl_bwd_ex with
 * the same arguments: the same logits, lse, losses and reductions, and the
 * dlogits formed by the same float32 expressions. Arguments are those of the
 * two calls:
 *  - loss_tok, lse and loss as in kd_fused_kl_fwd_ex (lse is still written);
 *  - grad_loss, dH, dW and dW_accumulate as in kd_fused_kl_bwd_ex.
 * The workspace is kd_fused_kl_workspace_bytes(KD_PASS_FWD_BWD, ...). The
 * errors are those of the two calls.
 *
 * Duplicate ids within a row are outside the contract, as for every entry
 * point; the dlogits entry at a duplicated id may keep only one of the
 * duplicates' corrections.
 */
int kd_fused_kl_fwd_bwd(const void* H, const void* W, int dtype, const int32_t* topk_idx,
                        const float* topk_logp, const float* weight, int reduction, int64_t N,
                        int64_t d, int64_t V, int64_t K, int64_t chunk, const float* grad_loss,
                        float* loss_tok, float* lse, float* loss, void* dH, float* dW,
                        int dW_accumulate, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The offline teacher cache: run the teacher's output head once and keep,
 * for every position, the K most probable tokens with their log-probabilities
 * under the full softmax, not renormalised. Sources:
 *  - "Distilação de LLMs mais barata: top-K offline e KL fundida cortam VRAM
 *    em até 15x", section "As duas mudanças";
 *  - "Hugging Face：让知识蒸馏廉价到可大规模运行", paragraph 离线蒸馏;
 *  - "Chunkovaná KL strata ...", section "Čo dopĺňajú podrobnejšie
 *    experimenty".
 * The output is the topk_idx / topk_logp input of the loss.
 *
 *  Ht         [N, d] of `dtype` — teacher hidden states (final layer).
 *  Wt         [V, d] of `dtype` — teacher output head.
 *  N, d, V, K, chunk — sizes; 1 <= K <= min(V, 2048), chunk >= 1, N >= 0.
 *  topk_idx   [N, K] int32 out — ids by logit, largest first; equal logits
 *             are ordered by the lower id first.
 *  topk_logp  [N, K] float32 out — z_r,idx − lse_r.
 *  lse        [N] float32 out, or NULL — log Σ_j exp z_rj of every row.
 *
 * Rows are processed `chunk` at a time with one pass of the logit GEMM and
 * no [N, V] grid: the chunk's float32 logits are kept until its candidates
 * (logits at or above a per-row threshold that bounds the K-th largest) are
 * collected. The workspace (kd_fused_kl_workspace_bytes with
 * KD_PASS_TEACHER) holds those logits and per-row candidate lists of up to V
 * entries of 8 bytes, so it is about chunk × V × 12 bytes. The selection is
 * exact on the float32 logits the kernels compute. Errors as for
 * kd_fused_kl_fwd; K > 2048 is KD_ERR_UNSUPPORTED.
 */
int kd_teacher_topk(const void* Ht, const void* Wt, int dtype, int64_t N, int64_t d, int64_t V,
                    int64_t K, int64_t chunk, int32_t* topk_idx, float* topk_logp, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Debug check of the cache preconditions the loss does not check on its hot
 * path (not needed for correct inputs, and not called by the loss):
 * every id in [0, V), the ids of a row distinct, every log-probability ≤ 0
 * or −inf (never positive, +inf or NaN). The cache holds log-probabilities
 * of the teacher's full softmax, kept without renormalisation ("Chunkovaná KL
 * strata ...", section "Čo dopĺňajú podrobnejšie experimenty").
 *
 *  topk_idx  [N, K] int32, topk_logp [N, K] float32 — device pointers.
 *  flags     [1] int32, DEVICE pointer — overwritten with the OR of
 *            KD_CHECK_* bits of every violation found (0: all hold). Read it
 *            after the stream reaches this call; nothing here synchronises.
 *
 * 1 <= K <= min(V, 16383), N >= 0; otherwise KD_ERR_INVALID_ARG.
 */
enum { KD_CHECK_ID_RANGE = 1, KD_CHECK_DUPLICATE = 2, KD_CHECK_LOGP = 4 };
int kd_fused_kl_check_inputs(const int32_t* topk_idx, const float* topk_logp, int64_t N,
                             int64_t K, int64_t V, int32_t* flags, void* stream);

/*
 * x[i] *= s for n values in place, x of `dtype` (KD_F32 or KD_BF16; bf16
 * values are scaled in float32 and rounded to nearest even), s a float32
 * DEVICE scalar. When s == 1 the kernel leaves x untouched and costs only
 * its launch. For callers that obtain the gradients of kd_fused_kl_fwd_bwd
 * at g = 1 and learn the upstream gradient later (an autograd backward):
 * scaling by g afterwards gives the gradients at g, bitwise those of the
 * two-pass calls when g == 1. Device pointers; n >= 0.
 */
int kd_scale(void* x, int dtype, int64_t n, const float* s, void* stream);

/*
 * Element-wise float32 -> bfloat16 (round to nearest even) of n values, for
 * callers that keep W in bf16 and want dW in W's dtype. Device pointers;
 * src and dst must not overlap.
 */
int kd_cast_f32_to_bf16(const float* src, void* dst, int64_t n, void* stream);

/*
 * Kernel timing, for benchmarks. Not part of the loss.
 *
 * kd_timing_enable(1) makes every later loss or teacher-cache call bracket
 * its kernel launches with HIP events on the caller's stream
 * (kd_timing_enable(0) stops it). kd_timing_read waits for the recorded
 * events, writes per kernel class the summed milliseconds
 * (total_ms[KD_KERNEL_CLASSES]) and launch counts
 * (launches[KD_KERNEL_CLASSES]), and clears the record. A "launch" of
 * KD_KERNEL_PREP is the two prep kernels of one group of chunks, or the
 * transpose of the chunks of H one logit launch reads. The logit pass of the teacher cache and of
 * kd_fused_kl_fwd_bwd, which also store the logits, count as
 * KD_KERNEL_FWD_LOGITS; their streaming passes over the stored logits as
 * KD_KERNEL_DL_STREAM. Global state, not thread-safe; this is the one entry
 * point that synchronises (with its own events).
 */
enum {
  KD_KERNEL_PREP = 0,         /* bucket top-K entries; transpose chunks of H  */
  KD_KERNEL_FWD_LOGITS = 1,   /* fused logit tile + logsumexp partials        */
  KD_KERNEL_BWD_DLOGITS = 2,  /* recomputed logit tile -> dlogits             */
  KD_KERNEL_BWD_DH = 3,       /* dH = dlogits W                               */
  KD_KERNEL_BWD_DW = 4,       /* dW (+)= dlogitsᵀ H                           */
  KD_KERNEL_OTHER = 5,        /* combine, split reduce, teacher select/finish */
  KD_KERNEL_DL_STREAM = 6,    /* stored logits -> dlogits, or teacher candidates */
  KD_KERNEL_CLASSES = 7
};
int kd_timing_enable(int enable);
int kd_timing_read(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* KD_FUSED_KL_H */
