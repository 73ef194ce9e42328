/*
 * pi.h -- C ABI of the neuron-aware sparse FFN library (libpi.so) for AMD MI355X (gfx950).
 *
 * The library computes the FFN of a ReLU / ReGLU transformer layer by predicting which
 * FFN neurons fire for the current token(s), compacting their indices, and reading and
 * multiplying only those neurons' up/gate rows and down columns. This is the hot path of
 * PowerInfer as described on the pages
 *   P1 "Tüketici sınıfı GPU takılı PC'lerde yüksek hızlı büyük dil modeli serving",
 *   P2 "PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU" (КПД),
 *   P3 "PowerInfer: Mesin Inferensi LLM Cepat dengan GPU Konsumen" (unite.ai).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller, 16-byte aligned, row-major.
 *    The library never frees them. A pi_ffn borrows its weight pointers until destroyed.
 *  - Compute entry points enqueue work on the context's HIP stream and return without
 *    host synchronisation. Device faults surface at the caller's next synchronisation.
 *  - Argument errors are detected on the host before anything is enqueued: the call
 *    returns PI_ERR_INVALID (or PI_ERR_UNSUPPORTED) and enqueues nothing. HIP launch
 *    failures return PI_ERR_HIP. pi_last_error(ctx) gives a human-readable reason.
 *  - Compute entry points allocate nothing: every scratch buffer (activations, partial
 *    sums, mask words, staging) belongs to the pi_ctx and is sized at pi_ctx_create.
 *  - No C++ exception crosses this boundary. A pi_ctx is used by one host thread at a time,
 *    and the work of one context must not run concurrently with itself (its scratch is
 *    shared between calls): keep a context's calls on one stream, or order them.
 *  - Neuron index space: the "stored" order of the layer's rows. With a hot-first layout
 *    (pi_permute_rows), neuron_table[k] maps stored row k back to its original neuron.
 */
#ifndef PI_H
#define PI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PI_ABI_VERSION 2

typedef enum {
  PI_OK = 0,
  PI_ERR_INVALID = 1,      /* bad argument: null pointer, bad shape, misalignment, too large */
  PI_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. batch size outside a path)     */
  PI_ERR_OOM = 3,          /* device allocation failed in pi_ctx_create                      */
  PI_ERR_HIP = 4           /* a HIP runtime call failed; see pi_last_error                    */
} pi_status;

/* Activation families the method supports (P1 header bullets, «Kısıtlar ve SSS»):
 * ReLU a = max(h, 0); ReGLU a = max(g, 0) * u; Squared-ReLU a = max(h, 0)^2. ReLU and
 * Squared-ReLU read one row per neuron (w_up, masked on h > 0); ReGLU reads two (w_gate,
 * masked on g > 0, and w_up). */
typedef enum { PI_ACT_RELU = 0, PI_ACT_REGLU = 1, PI_ACT_SQRELU = 2 } pi_act;

/* Weight storage. PI_W_Q4_0: each block of 32 consecutive elements of a row stores an fp16
 * scale s and 32 4-bit codes q; the weight is (q - 8) * s (P1 «Kuantizasyon ve uyumluluk»).
 * Layout is struct-of-arrays: codes uint8 [rows][d/32][16], byte j of a block holding
 * element j in its low nibble and element j+16 in its high nibble; scales fp16 [rows][d/32]. */
typedef enum { PI_W_F32 = 0, PI_W_F16 = 1, PI_W_Q4_0 = 2 } pi_wtype;

typedef struct pi_ctx pi_ctx;
typedef struct pi_ffn pi_ffn;

/* One FFN layer (borrowed device pointers). Neuron-major layout: row i of w_up / w_gate is
 * neuron i's input row, row i of w_down_t is neuron i's output column (W_down transposed),
 * so an active neuron's weights are contiguous rows (P3 «Operator yang Sadar Neuron»).
 *   d        model width, multiple of 8 (of 32 for Q4_0)
 *   ffn      number of FFN neurons, multiple of 64
 *   rank     predictor rank r (multiple of 8, at most 1024; fp16 / Q4_0 layers only), or 0:
 *            no predictor, the mask is the true pre-activation of the masked projection
 *            (> threshold)
 *   act      pi_act. ReLU and Squared-ReLU mask the up projection; ReGLU masks the gate.
 *   wtype    pi_wtype of w_up / w_gate / w_down_t
 *   threshold decision threshold on the predictor logit (0 == "sigmoid > 0.5")
 *   w_up, w_gate, w_down_t   [ffn][d] (fp32 / fp16) or Q4_0 codes; w_gate NULL unless ReGLU
 *   s_up, s_gate, s_down     Q4_0 fp16 scales [ffn][d/32]; NULL otherwise
 *   b        fp32 [ffn] bias of the masked projection (gate for ReGLU, else up)
 *   p_w1     fp16 [rank][d], p_w2 fp16 [ffn][rank], p_b fp32 [ffn]: the low-rank predictor
 *            logit = p_w2 (p_w1 x) + p_b (P3 «Prediktor Kepadatan Adaptif»); NULL if rank 0
 *   neuron_table  int32 [ffn] stored row -> original neuron id, or NULL (identity).
 *            Informational: outputs are in stored order.
 *   hot_prefix  H in [0, ffn]: the first H stored neurons are taken for every token without
 *            a prediction (their predictor rows are not read, their decision value is +inf)
 *            and the activation itself zeroes those that do not fire: the hot neurons
 *            PowerInfer keeps resident and always computes (P1 header bullets and «CPU/GPU
 *            hibrit çıkarım yöntemi»; P3 «Penempatan dan Pengelolaan Neuron»), on a hot-first
 *            layout. Predictor layers only (rank > 0); 0 for none.
 *   y_center fp32 [d] or NULL: this layer's expected output, subtracted from its y before the
 *            normalisation that feeds the next layer of a stack (pi_stack_run, pi_glue). */
typedef struct pi_ffn_desc {
  int32_t d, ffn, rank;
  int32_t act;
  int32_t wtype;
  float threshold;
  const void *w_up, *w_gate, *w_down_t;
  const uint16_t *s_up, *s_gate, *s_down;
  const float *b;
  const uint16_t *p_w1, *p_w2;
  const float *p_b;
  const int32_t *neuron_table;
  int32_t hot_prefix;
  const float *y_center;
} pi_ffn_desc;

int32_t pi_abi_version(void);
const char *pi_status_str(pi_status s);
/* Reason of the last failed call on ctx (empty string if none). Valid until the next call. */
const char *pi_last_error(const pi_ctx *ctx);

/* Create a context bound to `device` and the HIP stream `hip_stream` (hipStream_t, may be
 * NULL for the default stream). Sizes the scratch for batches up to max_batch tokens and
 * layers up to max_d x max_ffn with predictor rank up to max_rank. Allocates device memory. */
pi_status pi_ctx_create(int32_t device, void *hip_stream, int32_t max_batch, int32_t max_d,
                        int32_t max_ffn, int32_t max_rank, pi_ctx **out);
void pi_ctx_destroy(pi_ctx *ctx);
/* Rebind the context to another stream on the same device. */
pi_status pi_ctx_set_stream(pi_ctx *ctx, void *hip_stream);

/* Validate a layer description against the context and wrap it. Copies the descriptor,
 * not the weights. */
pi_status pi_ffn_create(pi_ctx *ctx, const pi_ffn_desc *desc, pi_ffn **out);
void pi_ffn_destroy(pi_ffn *ffn);

/* Masking of a batch of B > 1 tokens in pi_layer, pi_stack_run and pi_stack_profile:
 *  PI_MASK_UNION      (default) every token gets the activations of every neuron in the
 *                     union of the batch's masks (ReLU zeroes the neurons it does not
 *                     itself activate)
 *  PI_MASK_PER_TOKEN  each token gets only its own predicted neurons, a_t,i = 0 where bit i
 *                     of token t's mask is clear: the operator of P3 «Operator yang Sadar
 *                     Neuron» applied one token at a time with the mask P3 «Prediktor
 *                     Kepadatan Adaptif» gives that token.
 * The same rows are read either way (those of the union). The mode is a property of the
 * context; pi_sparse_ffn (one list for all tokens) does not depend on it. */
typedef enum { PI_MASK_UNION = 0, PI_MASK_PER_TOKEN = 1 } pi_mask_mode;

/* Set the context's masking of batches; PI_ERR_INVALID for another value. Work already
 * enqueued keeps the mode it was enqueued with. */
pi_status pi_ctx_set_mask_mode(pi_ctx *ctx, int32_t mode);

/* Predict the active neurons of B tokens (P3 «Fase Online», «Prediktor Kepadatan Adaptif»).
 *   x         [B][d] fp16 (fp32 when wtype == PI_W_F32)
 *   mask      [B][ffn/64] uint64 per-token bits: bit j of word w is neuron 64w+j, set when
 *             the decision value (predictor logit, or true pre-activation if rank 0) is
 *             strictly above the threshold
 *   idx       [ffn] int32: ascending indices of the UNION of the B masks (the token's own
 *             list when B == 1); entries at and beyond n_active are unspecified
 *   n_active  device int32 scalar: length of idx
 *   logits_out nullable fp32 [B][ffn]: the decision values themselves (for checking)
 *   B         1..max_batch (at most 64); 1..8 run on the vector units, 9..64 on the
 *             matrix cores (fp16 weights, d and rank multiples of 16); mask words are then
 *             written as 32-bit halves (same bit layout) */
pi_status pi_predict(pi_ctx *ctx, const pi_ffn *ffn, const void *x, int32_t B, uint64_t *mask,
                     int32_t *idx, int32_t *n_active, float *logits_out);

/* The neuron-aware sparse FFN on a given index list (P3 «Operator yang Sadar Neuron»): for
 * every listed neuron i, a_t,i = relu(w_up[i].x_t + b_i) (ReLU), its square (Squared-ReLU)
 * or relu(w_gate[i].x_t + b_i) * (w_up[i].x_t) (ReGLU), and y_t = sum_i a_t,i w_down_t[i].
 * The one list applies to all B tokens.
 *   idx, n_active  device [ffn] int32 (each entry < ffn, no duplicates) and device int32
 *   y         [B][d] fp32 output (overwritten) */
pi_status pi_sparse_ffn(pi_ctx *ctx, const pi_ffn *ffn, const void *x, int32_t B,
                        const int32_t *idx, const int32_t *n_active, float *y);

/* One FFN layer for B tokens (P3 «Fase Online»: the predictor marks the neurons likely to
 * fire, inactive ones are skipped, active ones computed): pi_predict followed by
 * pi_sparse_ffn on its union list, as three or four fused kernels. mask, idx and n_active
 * are nullable outputs (context scratch is used when NULL). */
pi_status pi_layer(pi_ctx *ctx, const pi_ffn *ffn, const void *x, int32_t B, float *y,
                   uint64_t *mask, int32_t *idx, int32_t *n_active);

/* pi_layer for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no pi_ctx, and no allocation at
 * all. Its scratch (predictor stage 1 output, mask words, index list, activations, partial
 * sums) is one fixed device array of the library, 26.1 MiB, which each GPU it runs on
 * holds until the process ends. Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (several streams or threads) race; order them. No part of the array
 * needs to start at zero. Limits: B <= 8 tokens, d <= 12288, ffn <= 49152, rank <= 1024
 * (PI_ERR_UNSUPPORTED beyond them); otherwise the arguments, outputs, errors and kernels are
 * those of pi_layer on a context of the same stream in union masking (the result is bitwise
 * the same). PI_ERR_INVALID for a bad argument or description (no reason is kept: there is
 * no context). Work is enqueued on hip_stream (NULL: the default stream) of `device`, which
 * becomes the current device. */
pi_status pi_layer_noalloc(int32_t device, void *hip_stream, const pi_ffn_desc *desc, const void *x,
                           int32_t B, float *y, uint64_t *mask, int32_t *idx, int32_t *n_active);

/* Threshold + compaction alone, on caller-provided decision values v [B][ffn] fp32:
 * the same device code pi_predict uses after computing v (P3 «Prediktor Kepadatan Adaptif»:
 * neurons predicted active are processed; P3 «Operator yang Sadar Neuron»: they are then
 * addressed directly, with no dense conversion). B is 1..8. */
pi_status pi_compact(pi_ctx *ctx, const float *v, int32_t B, int32_t ffn, float threshold,
                     uint64_t *mask, int32_t *idx, int32_t *n_active);

/* Chain between stacked layers, so that each token passes through every layer before the
 * next token (P3 introduction). The pages define no layer between FFNs; this one keeps every
 * layer's input at the scale its calibration assumes: u_t = y_t - c, x_out_t = round(u_t /
 * sqrt(mean(u_t^2))) to x's storage type (fp16, or fp32 when x_is_f32), or x_prev_t
 * unchanged when y_t (or u_t) is all zero.
 *   y [B][d] fp32, center c fp32 [d] or NULL (zero), x_prev [B][d], x_out [B][d] */
pi_status pi_glue(pi_ctx *ctx, const float *y, const float *center, const void *x_prev, int32_t B,
                  int32_t d, int32_t x_is_f32, void *x_out);

/* Run L layers over T tokens, B tokens per step (T % B == 0), one step at a time: step s
 * feeds x_tokens[s*B..s*B+B) to layer 0, each layer's y (through pi_glue, with that layer's
 * y_center) to the next, and writes the last layer's y to y_out[s*B..]. Token-by-token
 * decode (P3 intro) at B == 1.
 *   layers     host array of L layer handles with equal d and activation/weight types
 *   x_tokens   [T][d] fp16 (fp32 for PI_W_F32 stacks); y_out [T][d] fp32
 *   n_active_log nullable device int32 [T/B][L]: n_active of every (step, layer)
 *   use_graph  nonzero: each step's L layers run as one captured HIP graph */
pi_status pi_stack_run(pi_ctx *ctx, const pi_ffn *const *layers, int32_t L, const void *x_tokens,
                       int32_t T, int32_t B, float *y_out, int32_t *n_active_log, int32_t use_graph);

/* What pi_stack_run_dump records of every (step, layer); each pointer is DEVICE memory or
 * NULL (not recorded). With S = T/B steps, slot (s, l) is at index s*L + l:
 *   x     [S][L][B][d] in x's storage type: the layer's input as its kernels read it
 *   mask  [S][L][B][ffn_stride/64] uint64: the tokens' predicted mask words
 *   idx   [S][L][ffn_stride] int32: the ascending union list (entries past n unspecified)
 *   n     [S][L] int32: the union count
 *   y     [S][L][B][d] fp32: the layer's output (its partial sums added)
 *   ffn_stride  >= every layer's ffn, a multiple of 64 */
typedef struct pi_stack_dump {
  void *x;
  uint64_t *mask;
  int32_t *idx;
  int32_t *n;
  float *y;
  int32_t ffn_stride;
} pi_stack_dump;

/* pi_stack_run with every layer's input, mask, index list, count and output recorded, for
 * checking a whole stack layer by layer against a reference that takes each layer's
 * recorded input (P3 «Fase Online»: per layer, predict, skip the inactive, compute the
 * active). Runs the same kernels in the same order as pi_stack_run, eagerly (no graph),
 * with copies and sums of partials into the dump between layers; y_out and n_active_log are
 * therefore bitwise those of pi_stack_run. Other arguments as for pi_stack_run. */
pi_status pi_stack_run_dump(pi_ctx *ctx, const pi_ffn *const *layers, int32_t L, const void *x_tokens,
                            int32_t T, int32_t B, float *y_out, int32_t *n_active_log,
                            const pi_stack_dump *dump);

/* Kernel classes of pi_stack_profile's outputs, in this order:
 * predictor stage 1 (with the glue); predictor stage 2 + threshold + the activations of the
 * workgroup's active neurons; true-mask threshold GEMV + activations; gathered up/gate GEMV
 * (index-list entry point; the separate, column-sliced GEMV that 1..8 tokens take instead
 * of stage 2's activations when x is above 64 KiB, for Q4_0, d >= 8192 or 5..8 tokens; the
 * matrix-core path's gathered GEMM);
 * down projection (with the index scan) into partial sums; the small kernels: sum of
 * partial sums into y, activations from the column slices' partial sums, glue between
 * layers of several tokens, compaction and predictor hi/lo split of the matrix-core path. */
#define PI_KERNEL_CLASSES 6

/* pi_stack_run without a graph, every kernel dispatched with a pair of hipEvents
 * (hipExtLaunchKernelGGL) on the context's stream, so each pair times that kernel's own
 * execution: the per-kernel time of the generation speed the pages measure end to end
 * in tokens/s (P1 «Performans değerlendirmesi ve demo»). Blocks until the work is done,
 * then writes the summed event time in milliseconds (ms_out[PI_KERNEL_CLASSES], host) and
 * the number of launches (launches_out[PI_KERNEL_CLASSES], host) of each kernel class.
 * Other arguments as for pi_stack_run. For measurement. */
pi_status pi_stack_profile(pi_ctx *ctx, const pi_ffn *const *layers, int32_t L, const void *x_tokens,
                           int32_t T, int32_t B, float *y_out, int32_t *n_active_log, double *ms_out,
                           int64_t *launches_out);

/* Q4_0 rows to fp32 with the kernels' own in-register unpacking (P1 «Kuantizasyon ve
 * uyumluluk»: 4-bit weights in 32-element blocks with a 16-bit scale): out[i][c] =
 * (q - 8) * s for every row i < rows and column c < d, where block b of row i is the 16
 * code bytes codes[(i * d/32 + b) * 16 ...] (byte j: element j in the low nibble, element
 * j + 16 in the high nibble) and its scale is the fp16 scales[i * d/32 + b]. (q - 8) is
 * rebuilt exactly in fp16 and multiplied by the scale in fp32, which is exact (a 4-bit by an
 * 11-bit significand), so the result is bitwise the dequantised weight. Device pointers:
 * codes [rows][d/2] bytes, scales [rows][d/32] fp16, out [rows][d] fp32. d % 32 == 0. For
 * checking the dequantisation against a plain implementation. */
pi_status pi_q4_dequant(pi_ctx *ctx, const uint8_t *codes, const uint16_t *scales, int32_t rows, int32_t d,
                        float *out);

/* Hot-first neuron order (P3 «Penempatan dan Pengelolaan Neuron»): perm[k] = the neuron
 * with the k-th largest activation probability, ties in ascending neuron order. HOST
 * pointers: p double [ffn], perm int32 [ffn]. */
pi_status pi_hot_first_order(const double *p, int32_t ffn, int32_t *perm);

/* Gather rows on the device: dst[k] = src[perm[k]] for k < rows, each row_bytes long
 * (a multiple of 4). Used to store a layer's neuron-indexed arrays in hot-first order
 * (P3 «Penempatan dan Pengelolaan Neuron»: neurons placed by hotness, with a table back to
 * their original positions).
 * perm is a device int32 [rows] permutation; src and dst must not overlap. */
pi_status pi_permute_rows(pi_ctx *ctx, const void *src, void *dst, const int32_t *perm,
                          int32_t rows, int64_t row_bytes);

#ifdef __cplusplus
}
#endif

#endif /* PI_H */
