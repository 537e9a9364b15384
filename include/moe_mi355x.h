/*
 * moe_mi355x.h -- C ABI of the routed-expert MoE FFN library for MI355X (gfx950).
 *
 * One MoE layer's routed experts compute, for every token t routed to the k
 * experts e_tj with weights w_tj,
 *
 *     y_t = sum_j w_tj * Wd[e_tj] ( SiLU(Wg[e_tj] x_t) * Wu[e_tj] x_t )
 *
 * (SwiGLU experts and the weighted top-k combine: warp-decode post, sections on
 * the traditional MoE path and on how the two kernels work).  Two regimes:
 *
 *  - decode (output-centric, small batches): moe_gate_up + moe_down.  Every
 *    output scalar is produced by exactly one 64-lane wavefront that streams
 *    the expert weight rows it needs, converts the stored format in registers
 *    and keeps FP32 accumulators (warp-decode post: the two kernels, warp
 *    independence);
 *  - grouped (expert-centric, large batches): moe_align_sort and
 *    moe_quant_rows, then moe_grouped_gate_up, moe_grouped_down, moe_combine
 *    on gfx950 block-scaled matrix cores (align-and-sort article: background,
 *    D-C-P algorithm, CK fused-MoE section on online FP8 quantisation and on
 *    the sort feeding the GEMM).
 *
 * moe_layer runs either regime, or picks one (moe_choose_path).
 *
 * Conventions for every entry point:
 *  - Pointers named as device memory must be device memory of the current
 *    HIP device; the caller owns all of it.  The library never allocates,
 *    frees or synchronises; every call enqueues kernels on `stream` (a
 *    hipStream_t passed as void*, NULL = the default stream) and returns.
 *  - Every shape / pointer / enum problem is detected on the host before any
 *    launch and returns an error with nothing enqueued.  A launch failure
 *    reported by the HIP runtime returns MOE_ERR_HIP.  No exceptions, no exit.
 *  - Preconditions NOT checked (they would need a device read): expert ids in
 *    [0, num_experts); finite weights and scales; outputs not aliasing inputs.
 *    Every kernel reads an id outside [0, num_experts) as expert 0, so such an
 *    id never takes an access outside the caller's buffers; moe_check_routing
 *    finds such ids on the device when a caller wants them checked.
 *  - The library keeps no mutable global state apart from a per-device cache
 *    of the compute-unit count; calls are thread-safe.  Calls may be captured
 *    in a HIP graph: they record kernels only.
 *
 * Weight storage (per expert e in [0, E+S), S = num_shared in {0, 1}; the
 * shared expert is stored as index E):
 *   w13 [E+S][2][I][H*]  gate rows (index 0) then up rows (index 1), [out][in]
 *   w2  [E+S][H][I*]     down rows, [out][in]
 *   MOE_W_F32        : float32 values, no scales.
 *   MOE_W_MXFP8      : E4M3FN bytes; scales E8M0 bytes, one per 32 consecutive
 *                      input elements: w13_scale [E+S][2][I][H/32],
 *                      w2_scale [E+S][H][I/32].
 *   MOE_W_MXFP4      : E2M1 nibbles, two per byte, even element in the low
 *                      nibble (rows are H/2 resp. I/2 bytes); E8M0 scales as MXFP8.
 *   MOE_W_FP8_BLK128 : E4M3FN bytes; float32 scale per 128x128 tile of each
 *                      [out][in] matrix: w13_scale [E+S][2][I/128][H/128],
 *                      w2_scale [E+S][H/128][I/128].
 * Routing: topk_ids [T][k] int32 and topk_weights [T][k] float32 list the
 * routed slots; with S = 1 every token also runs slot k on expert E with
 * weight 1.0.  "slots" below means k + S.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,        /* bad pointer, size or enum value          */
  MOE_ERR_UNSUPPORTED = 2,        /* valid but not implemented combination    */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* the HIP runtime reported an error        */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_W_F32 = 0,
  MOE_W_MXFP8 = 1,
  MOE_W_MXFP4 = 2,
  MOE_W_FP8_BLK128 = 3
} moe_weight_format;

typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_GROUPED = 2 } moe_path;

/* One layer's expert weights.  A host struct holding device pointers. */
typedef struct {
  int32_t hidden;        /* H                                              */
  int32_t inter;         /* I                                              */
  int32_t num_experts;   /* E, routed experts                              */
  int32_t num_shared;    /* S in {0, 1}; the shared expert is index E      */
  int32_t format;        /* moe_weight_format                              */
  const void* w13;       /* device, layout above                           */
  const void* w13_scale; /* device, NULL for MOE_W_F32                     */
  const void* w2;        /* device                                         */
  const void* w2_scale;  /* device, NULL for MOE_W_F32                     */
} moe_weights;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* ABI version of this header (incremented on incompatible change). */
int32_t moe_abi_version(void);

/* ------------------------------------------------------------------ */
/* Decode regime (output-centric).                                     */
/* ------------------------------------------------------------------ */

/* Largest T * slots the decode kernels accept (the routed ids of one call
 * are staged on chip). */
int32_t moe_decode_max_entries(void);

/*
 * moe_gate_up: h[t][j][n] = SiLU(g) * u with g = Wg[e_tj][n,:] . x_t and
 * u = Wu[e_tj][n,:] . x_t, for every token t < T, slot j < slots, neuron n < I
 * (warp-decode post, section on how the two kernels work: one wavefront per
 * intermediate neuron of a (token, routed expert) pair, gate and up rows
 * streamed with the activation read once for both, SiLU(gate) * up applied
 * after the wave reduction).  A wavefront owns neuron rows of one expert and
 * produces those neurons for every slot routed to that expert in the batch, so
 * each weight row is read once per call; every h scalar is written exactly
 * once and its reduction order does not depend on the batch.
 *   x        device, [T][H], x_dtype (MOE_DT_F32 only with MOE_W_F32 weights)
 *   topk_ids device, [T][k] int32
 *   h        device, [T][slots][I], h_dtype (MOE_W_F32 weights take MOE_DT_F32
 *            only: MOE_ERR_UNSUPPORTED otherwise, as in moe_down)
 * T == 0 is a no-op.  T * slots must not exceed moe_decode_max_entries().
 */
moe_status moe_gate_up(const moe_weights* W, const void* x, int32_t x_dtype,
                       const int32_t* topk_ids, int32_t T, int32_t k,
                       void* h, int32_t h_dtype, void* stream);

/* Launch shapes of moe_down (identical bits, with the MXFP4 exception below). */
typedef enum {
  MOE_DOWN_AUTO = 0,          /* token-major for small batches, expert-major from
                                 a number of routed entries on (see moe_down);
                                 expert-major at every T for MXFP4 rows that fit
                                 the matrix-core kernel (see below)             */
  MOE_DOWN_TOKEN_MAJOR = 1,   /* a wavefront owns (token, rows); no buffer        */
  MOE_DOWN_EXPERT_MAJOR = 2   /* a wavefront owns (expert, rows); slot buffer in
                                 the workspace and a combine kernel               */
} moe_down_variant;

/*
 * moe_down: y[t][d] = sum_j w_tj * (Wd[e_tj][d,:] . h[t][j][:]) for every
 * token t < T and output d < H (warp-decode post, section on how the two
 * kernels work: one wavefront per output dimension of a token walks all of
 * the token's experts, folds each routing weight in and finishes with a
 * butterfly reduction; the combine is part of the projection).
 * Each slot's dot product is computed by a fixed group of lanes in a fixed
 * order, multiplied by w_tj, and the slots are added in slot order, so every
 * launch shape gives identical bits:
 *   MOE_DOWN_TOKEN_MAJOR   a wavefront owns (token, output rows) and sums the
 *                          slots in registers (the page's form); nothing is
 *                          buffered;
 *   MOE_DOWN_EXPERT_MAJOR  a wavefront owns (expert, output rows), reads those
 *                          rows once for all tokens routed to the expert and
 *                          stores w * dot per (token, slot) in the workspace;
 *                          a combine kernel adds them in slot order.
 *   MOE_DOWN_AUTO          token-major below a number of routed entries
 *                          (T * slots), expert-major from it on, measured
 *                          faster on each side of that line: 112 entries
 *                          when a W_down row spans fewer than 32 lanes (I up
 *                          to about 1024 with BF16 h), 18 from 32 lanes on.
 * The exception: MXFP4 weights with BF16 h, I a multiple of 256 and H of 32.
 * Their expert-major shape runs on the matrix cores (the expert's routed
 * entries as the columns of v_mfma_f32_16x16x32_bf16): the same exact
 * products summed in another FP32 order, so its bits differ from the
 * token-major shape's.  AUTO takes it at every T for such weights, so y still
 * does not depend on the batch.
 *   h            device, [T][slots][I], h_dtype (MOE_DT_F32 only with
 *                MOE_W_F32 weights)
 *   topk_ids     device, [T][k] int32; topk_weights device, [T][k] float32
 *   y            device, [T][H], y_dtype
 *   variant      moe_down_variant
 *   workspace    device, at least moe_down_workspace_bytes(W, T, k) bytes,
 *                16-byte aligned, when the variant run is expert-major;
 *                ignored (may be NULL) otherwise
 * slots must be <= 64; the expert-major shape takes at most
 * moe_decode_max_entries() entries (MOE_ERR_UNSUPPORTED otherwise, before
 * any launch).
 */
size_t moe_down_workspace_bytes(const moe_weights* W, int32_t T, int32_t k);

moe_status moe_down(const moe_weights* W, const void* h, int32_t h_dtype,
                    const int32_t* topk_ids, const float* topk_weights,
                    int32_t T, int32_t k, void* y, int32_t y_dtype, int32_t variant,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* Align-and-sort (expert-centric front end).                          */
/* ------------------------------------------------------------------ */

/* Padded capacity: n + (E+S)*(BS-1) with n = T*(k+S). */
size_t moe_align_sort_capacity(int32_t T, int32_t k, int32_t num_experts,
                               int32_t num_shared, int32_t block_size);

/* Bytes of device scratch moe_align_sort needs. */
size_t moe_align_sort_workspace_bytes(int32_t T, int32_t k, int32_t num_experts,
                                      int32_t num_shared, int32_t block_size);

/*
 * moe_align_sort: groups the n = T*(k+S) (token, slot) entries by expert and
 * pads every expert's run to a multiple of block_size (align-and-sort article:
 * background -- sort by expert id, align to the grouped GEMM's block;
 * D-C-P section -- distributed counting, cumulative sum of the aligned counts,
 * parallel placement).  Entry i = t*(k+S) + j; with S = 1 the entry of slot k
 * is expert E.  Results (bit-exact, deterministic):
 *   expert_offsets[e]   exclusive prefix of the padded counts, e in [0, E+S]
 *   *num_tokens_post_padded = expert_offsets[E+S]  (device scalar)
 *   sorted_token_ids[expert_offsets[e] + r] = r-th smallest entry of expert e
 *                          (ascending, i.e. stable); the padding tail of each
 *                          run holds the sentinel n
 *   expert_ids[b]       expert of block b, b < num_tokens_post_padded/block_size
 * Only the first num_tokens_post_padded entries of sorted_token_ids and the
 * first num_tokens_post_padded/block_size of expert_ids are written.
 *   topk_ids          device [T][k] int32
 *   sorted_token_ids  device [capacity] int32
 *   expert_ids        device [capacity / block_size] int32
 *   expert_offsets    device [E+S+1] int32
 *   num_tokens_post_padded device [1] int32
 *   workspace         device, >= moe_align_sort_workspace_bytes(...)
 * block_size must be 1..1024; E+S must be 1..1024; k <= num_experts
 * (MOE_ERR_INVALID_ARG otherwise).
 */
moe_status moe_align_sort(const int32_t* topk_ids, int32_t T, int32_t k,
                          int32_t num_experts, int32_t num_shared, int32_t block_size,
                          int32_t* sorted_token_ids, int32_t* expert_ids,
                          int32_t* expert_offsets, int32_t* num_tokens_post_padded,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* Grouped regime steps (expert-centric, block-scaled MFMA).           */
/* ------------------------------------------------------------------ */

/*
 * moe_quant_rows: MX-quantises each of the T rows of x once, per 32
 * consecutive elements: shared exponent floor(log2 amax) - 8 (clamped to
 * [-127, 127], -127 for a zero block), scale byte = exponent + 127, elements
 * divided by 2^exponent, saturated to +-448 and rounded to the nearest E4M3
 * value, ties to even (align-and-sort article, CK section: online FP8
 * quantisation of the tokens ahead of the grouped GEMM).  A token is
 * quantised once however many slots route it; moe_grouped_gate_up reads each
 * sorted row's activations from its token's row, so no per-slot gathered copy
 * exists (warp-decode post, buffer section: the expert-major activation copy
 * is a cost of the expert-centric path).
 *   x    device [T][H], x_dtype (BF16 or F32)
 *   xq   device [T][H] E4M3 bytes;  xs device [T][H/32] E8M0 bytes
 * H must be a multiple of 32 and T*H at most 2^31 - 1.
 */
moe_status moe_quant_rows(const void* x, int32_t x_dtype, int32_t T, int32_t H, uint8_t* xq,
                          uint8_t* xs, void* stream);

/*
 * moe_grouped_gate_up: for every block b < *num_tokens_post_padded/block_size
 * with expert e = expert_ids[b], G = A[b] Wg[e]^T and U = A[b] Wu[e]^T on
 * block-scaled MFMA with FP32 accumulation, where row r of A[b] is token row
 * sorted_token_ids[r] / slots of xq (the matrix-core loads follow the sort;
 * a padding row reads token 0 and its results are never used), then
 * h = SiLU(G) * U requantised per 32 consecutive neurons as two MXFP8 terms,
 * hi = Q(h) and lo = Q(h - hi), with the rule of moe_quant_rows (GC-MoE
 * abstract: grouped GEMM with SwiGLU and requantisation fused in the
 * epilogue).  The second term absorbs the code flips a single requantisation
 * would take from the matrix core's accumulation error.
 *   xq/xs   device [T][H] and [T][H/32], from moe_quant_rows
 *   T, k    tokens and routed slots of the sort (slots = k + num_shared)
 *   sorted_token_ids, expert_ids, num_tokens_post_padded: from moe_align_sort
 *   hq      device [2][capacity][I] E4M3 (hi rows, then lo rows)
 *   hs      device [2][capacity][I/32] E8M0
 * Weight formats: MOE_W_MXFP8, MOE_W_MXFP4, MOE_W_FP8_BLK128.
 * block_size in {32, 64, 128}; H and I multiples of 128 (MOE_ERR_UNSUPPORTED
 * otherwise).
 */
moe_status moe_grouped_gate_up(const moe_weights* W, const uint8_t* xq, const uint8_t* xs,
                               int32_t T, int32_t k, const int32_t* sorted_token_ids,
                               const int32_t* expert_ids,
                               const int32_t* num_tokens_post_padded, int32_t capacity,
                               int32_t block_size, uint8_t* hq, uint8_t* hs, void* stream);

/*
 * moe_grouped_down: for every block b with expert e, O = (Hhi[b] + Hlo[b]) Wd[e]^T
 * on block-scaled MFMA (one MFMA per term into the same accumulator), with
 * hq/hs laid out as moe_grouped_gate_up writes them; row r of O is multiplied
 * by the routing weight of entry
 * i = sorted_token_ids[r] (1.0 for the shared slot) and stored to
 * slot_out[i][:], rounded once to BF16 (round to nearest even); sentinel rows
 * are dropped (warp-decode post, buffer section: the per-expert output buffer
 * of the expert-centric path, 2-byte values).
 *   slot_out device [T*slots][H] BF16 bit patterns
 */
moe_status moe_grouped_down(const moe_weights* W, const uint8_t* hq, const uint8_t* hs,
                            const int32_t* sorted_token_ids, const int32_t* expert_ids,
                            const int32_t* num_tokens_post_padded, int32_t capacity,
                            int32_t block_size, const float* topk_weights, int32_t T,
                            int32_t k, uint16_t* slot_out, void* stream);

/*
 * moe_combine: y[t][d] = sum_{j < slots} slot_out[t*slots + j][d], summed in
 * slot order in FP32 (deterministic; warp-decode post, traditional path: the
 * final combine of per-expert outputs).
 *   slot_out device [T*slots][H] BF16 bit patterns (as moe_grouped_down writes)
 *   y device [T][H], y_dtype
 */
moe_status moe_combine(const uint16_t* slot_out, int32_t T, int32_t slots, int32_t H,
                       void* y, int32_t y_dtype, void* stream);

/* ------------------------------------------------------------------ */
/* Router front-end (the step before the path).                         */
/* ------------------------------------------------------------------ */

/*
 * moe_topk_route: routing from gating scores (align-and-sort article,
 * background section: experts are activated by their top-k gating scores,
 * with a per-expert bias added for the selection in DeepSeek V3/R1;
 * FasterTransformer section: the fused top-k gating softmax and its biased
 * variant).  For every token t:
 *   key[e]             = scores[t][e] + bias[e], in float32 (bias may be NULL)
 *   topk_ids[t][0..k)  = the experts of the k largest keys, largest first;
 *                        equal keys go to the lower expert index
 *   topk_weights[t][j] = exp(s_j - max s) / sum_i exp(s_i - max s) with
 *                        s_j = scores[t][topk_ids[t][j]] (a softmax over the
 *                        selected raw scores: the renormalised top-k of a
 *                        softmax over all experts)
 *   scores device [T][E] float32, bias device [E] float32 or NULL;
 *   topk_ids device [T][k] int32 and topk_weights device [T][k] float32 are
 *   written (caller-owned; they are the inputs of the routed-expert layer).
 * Sizes: T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 64).  Scores and bias must
 * be finite (not checked).  Errors: MOE_ERR_INVALID_ARG for bad sizes or null
 * pointers (nothing enqueued); T == 0 is a no-op.
 */
moe_status moe_topk_route(const float* scores, const float* bias, int32_t T, int32_t E,
                          int32_t k, int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * moe_check_routing: checks on the device the one precondition the layer's
 * entry points take on trust: every routed id is the index of one of the E
 * experts the router chooses among (align-and-sort article, background
 * section: each token activates k of the E experts), i.e. lies in
 * [0, num_experts).  Writes
 *   result[0] = the number of entries of topk_ids outside [0, num_experts)
 *   result[1] = the first such entry, t*k + j, or -1 if there is none
 *   topk_ids device [T][k] int32; result device int32[2] (caller-owned).
 * One kernel of one workgroup; nothing is read back to the host and nothing
 * needs clearing first, so it can be enqueued (or captured) ahead of the
 * layer and its result read whenever the caller synchronises.
 * Sizes: T >= 0, k >= 1, num_experts >= 1; T*k <= 2^31 - 1, else
 * MOE_ERR_UNSUPPORTED.  Errors: MOE_ERR_INVALID_ARG for bad sizes or a null
 * pointer (nothing enqueued).  T == 0 writes {0, -1}.
 */
moe_status moe_check_routing(const int32_t* topk_ids, int32_t T, int32_t k, int32_t num_experts,
                             int32_t* result, void* stream);

/* ------------------------------------------------------------------ */
/* The whole layer.                                                     */
/* ------------------------------------------------------------------ */

/*
 * moe_choose_path: the regime moe_layer(MOE_PATH_AUTO) runs for T tokens
 * (warp-decode post, last section: output-centric decode wins while the work
 * each expert shares is small; prefill and large batches favour expert-centric
 * packing).  Returns MOE_PATH_DECODE or MOE_PATH_GROUPED.
 */
int32_t moe_choose_path(const moe_weights* W, int32_t T, int32_t k);

/* Workspace bytes moe_layer needs for this path (AUTO resolved as above). */
size_t moe_layer_workspace_bytes(const moe_weights* W, int32_t T, int32_t k,
                                 int32_t path, int32_t block_size);

/*
 * moe_layer: y = the routed-expert FFN of the layer for T tokens.
 *   x           device, [T][H], x_dtype: MOE_DT_BF16, or MOE_DT_F32 with
 *               MOE_W_F32 weights only (MOE_ERR_UNSUPPORTED otherwise, on
 *               either path, before any launch)
 *   path        MOE_PATH_AUTO / DECODE / GROUPED
 *   block_size  grouped path M block (32, 64 or 128), or 0: the library picks
 *               by the expected entries per expert (32 up to 48, 64 up to
 *               160, else 128; the same rule in moe_layer_workspace_bytes);
 *               ignored for decode
 *   chosen      host, nullable: receives the path that ran
 *   workspace   device, >= moe_layer_workspace_bytes(W, T, k, path, block_size)
 * The decode path keeps activations exact (BF16/FP32 in, FP32 accumulate);
 * the grouped path quantises x and h to MXFP8 for the matrix cores and holds
 * each slot's weighted output in BF16 before the combine.
 */
moe_status moe_layer(const moe_weights* W, const void* x, int32_t x_dtype,
                     const int32_t* topk_ids, const float* topk_weights,
                     int32_t T, int32_t k, void* y, int32_t y_dtype,
                     int32_t path, int32_t block_size,
                     void* workspace, size_t workspace_bytes,
                     int32_t* chosen, void* stream);

/*
 * moe_layer_noalloc: moe_layer with no caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a device array
 * inside the library, moe_layer_noalloc_max_bytes() bytes (32 MiB), one copy
 * per GPU, held from the library's load until the process ends.  Nothing is
 * allocated or freed by the call; the caller still owns x, the routing and y.
 *   Arguments and results as moe_layer.
 *   MOE_ERR_WORKSPACE_TOO_SMALL (nothing enqueued) when
 *   moe_layer_workspace_bytes(W, T, k, path, block_size) exceeds the array,
 *   e.g. the grouped path at prefill sizes.
 * All calls on one GPU share its array and leave their contents in it (no
 * step of the layer needs it cleared): calls that overlap on one GPU --
 * different streams, or threads enqueueing at the same time -- race and must
 * be serialised by the caller.
 */
size_t moe_layer_noalloc_max_bytes(void);

moe_status moe_layer_noalloc(const moe_weights* W, const void* x, int32_t x_dtype,
                             const int32_t* topk_ids, const float* topk_weights,
                             int32_t T, int32_t k, void* y, int32_t y_dtype,
                             int32_t path, int32_t block_size, int32_t* chosen, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
