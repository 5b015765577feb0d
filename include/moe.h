/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts layer hot path:
 * router + top-K, sparse dispatch, grouped SiLU-gated expert MLP, weighted
 * combine, and a two-microbatch overlapped forward.
 *
 * Sources of the operations (page titles and sections):
 *   [PPLX] "Efficient and portable mixture-of-experts communication"
 *          (Perplexity, 2025-04-02): Introduction, Sharding and Parallelism,
 *          Portable Kernels, Dispatch, Combine.
 *   [DBO]  "Dual Batch Overlap" (vLLM design doc): Introduction (overlap
 *          schedule), UBatchRunner (midpoint split), Interfaces (compute and
 *          communication streams), Limitations and UBatchWrapper (the
 *          overlapped forward is captured whole as a graph and replayed),
 *          Running with DBO (token thresholds).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer (HBM of the current HIP
 *     device) unless marked "host".  The library never allocates, frees or
 *     keeps device memory: inputs, outputs and workspaces are caller-owned and
 *     may be reused from call to call (as the pages' buffers are reused across
 *     layers, [PPLX] Portable Kernels).  (The graph entry points create a HIP
 *     graph, whose runtime resources last until moe_graph_destroy.)
 *   - All matrices are dense row-major.  Expert weights use the [out, in]
 *     layout, so both operands of every product are contiguous along the
 *     reduction dimension.
 *   - Calls are asynchronous: the host validates arguments, then only enqueues
 *     kernels on the given stream; pointers must stay valid until that work has
 *     completed.  No call synchronises with the host or reads device data on
 *     the host.
 *   - On any status other than MOE_OK nothing has been enqueued (except
 *     MOE_ERR_HIP, returned when a launch itself fails).
 *   - Results are deterministic: no floating-point atomics, fixed reduction
 *     orders, a stable dispatch order.  Repeated calls give identical bits.
 *   - Stateless and re-entrant; calls on different streams are independent as
 *     long as their buffers do not overlap.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, bad size, bad expert range   */
  MOE_ERR_WORKSPACE_TOO_SMALL = 2,
  MOE_ERR_UNSUPPORTED = 3,        /* valid but not implemented (dtype, shape)  */
  MOE_ERR_HIP = 4                 /* a HIP runtime call or launch failed       */
} moe_status_t;

/* The configuration's enumerated fields are int32_t holding these constants
 * (the size of a C enum type is up to the compiler; a field of fixed width
 * keeps moe_config_t's layout the same for every caller). */
/* Element types of activations and weights. */
enum { MOE_F32 = 0, MOE_BF16 = 1 };
/* Router score functions. */
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
/* Layouts of the bf16 expert weight stacks (moe_config_t.weight_layout). */
enum { MOE_WEIGHTS_ROW_MAJOR = 0, MOE_WEIGHTS_PACKED = 1 };
/* Where a whole-layer call runs the shared experts (moe_config_t.shared_placement). */
enum { MOE_SHARED_FUSED = 0, MOE_SHARED_BESIDE_COMBINE = 1 };
/* Workspace kinds for moe_workspace_bytes. */
enum { MOE_WS_ROUTE = 0, MOE_WS_DISPATCH = 1, MOE_WS_EXPERT_MLP = 2, MOE_WS_FORWARD = 3,
       MOE_WS_FORWARD_DBO = 4 };

#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 16
#define MOE_MAX_SHARED 4
#define MOE_MAX_TOKENS (1 << 26)

/* One layer's shape.  Limits (else MOE_ERR_INVALID_ARGUMENT):
 *   1 <= num_tokens, num_tokens * top_k < 2^31;
 *   1 <= num_experts <= MOE_MAX_EXPERTS; 1 <= top_k <= min(num_experts, MOE_MAX_TOPK);
 *   0 <= expert_begin < expert_end <= num_experts;
 *   0 <= num_shared <= MOE_MAX_SHARED; score in MOE_SCORE_*; dtype in MOE_F32/MOE_BF16;
 *   hidden and intermediate >= 1.
 *   weight_layout in MOE_WEIGHTS_*.
 * Shapes the kernels do not cover return MOE_ERR_UNSUPPORTED:
 *   bf16: hidden and intermediate multiples of 64;  f32: multiples of 16;
 *   MOE_WEIGHTS_PACKED: bf16 only, hidden and intermediate multiples of 128;
 *   num_tokens >= MOE_MAX_TOKENS (the router, scatter and combine run one
 *   64-lane wave per token, and a launch holds fewer than 2^32 work-items);
 *   shapes whose grouped expert GEMM launch would reach 2^32 work-items. */
typedef struct moe_config {
  int32_t num_tokens;    /* T: tokens in this call                                    */
  int32_t hidden;        /* d: model width                                            */
  int32_t num_experts;   /* E: routed experts of the whole layer (all GPUs)           */
  int32_t top_k;         /* K: experts chosen per token                               */
  int32_t intermediate;  /* I: expert MLP width                                       */
  int32_t expert_begin;  /* this GPU hosts experts [expert_begin, expert_end)         */
  int32_t expert_end;
  int32_t num_shared;    /* always-applied shared experts, each of width I            */
  int32_t score;         /* MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID                    */
  int32_t renormalize;   /* 1: weights = selected scores / their sum; 0: raw scores   */
  int32_t dtype;         /* MOE_F32 or MOE_BF16, for activations and weights          */
  int32_t weight_layout; /* MOE_WEIGHTS_ROW_MAJOR, or MOE_WEIGHTS_PACKED: every bf16
                            expert weight stack (w_gate, w_up, w_down, ws_*) passed in
                            the layout moe_pack_weights writes                        */
  int32_t shared_placement; /* whole-layer calls with shared experts (moe_forward,
                            moe_forward_dbo, their graph captures):
                            MOE_SHARED_FUSED: the shared experts are extra groups of
                              the routed expert-MLP launches and the combine adds
                              their rows;
                            MOE_SHARED_BESIDE_COMBINE: [DBO] Introduction's
                              schedule -- each microbatch's shared-expert MLP is a
                              launch of its own on the compute stream, beside that
                              microbatch's routed combine on the communication
                              stream (which keeps its fp32 sums in the workspace);
                              a last pass adds the shared rows to those sums in the
                              same order and rounds once.
                            Both give the same bits.  The per-stage calls
                            (moe_expert_mlp, moe_combine) do not read it.           */
} moe_config_t;

/* A hipStream_t handle; NULL means the default (null) stream. */
typedef void* moe_stream_t;

/*
 * moe_route -- router projection, scoring and top-K selection.
 * [PPLX] Introduction: the router is a small linear layer whose output is a
 * probability distribution over experts; the K best-scoring experts are kept
 * and weighted by values derived from that distribution.
 *
 *   z[t,e] = sum_i x[t,i] * w_router[e,i] + (bias ? bias[e] : 0)   (fp32 accumulate)
 *   score  = softmax over all E of z[t,:]  (MOE_SCORE_SOFTMAX)
 *          | 1 / (1 + exp(-z[t,e]))       (MOE_SCORE_SIGMOID)
 *   topk_ids[t,:]     = the K experts with the largest z (both scores are
 *                       increasing in z), in descending order of z; equal z
 *                       go to the lower expert id first;
 *   topk_weights[t,k] = score of topk_ids[t,k], divided by the sum of the K
 *                       selected scores when cfg->renormalize is set.
 * Arguments:
 *   x            [T, d]  dtype            tokens
 *   w_router     [E, d]  dtype            router weight ([out, in])
 *   bias         [E]     fp32 or NULL     added to the logits (used for selection and score)
 *   topk_ids     [T, K]  int32  (out)
 *   topk_weights [T, K]  fp32   (out)
 *   logits       [T, E]  fp32   (out, optional: NULL to skip) the z above
 *   workspace    >= moe_workspace_bytes(cfg, MOE_WS_ROUTE) bytes, 256-byte aligned
 *                (that size is 0 for fp32 layers, where workspace may be NULL)
 */
moe_status_t moe_route(const moe_config_t* cfg, const void* x, const void* w_router,
                       const float* bias, int32_t* topk_ids, float* topk_weights,
                       float* logits, void* workspace, size_t workspace_bytes,
                       moe_stream_t stream);

/*
 * moe_dispatch -- count tokens per expert and copy routed tokens into
 * expert-contiguous rows, recording where each row came from.
 * [PPLX] Dispatch: per-destination-expert token counts; tokens unpacked into a
 * contiguous per-expert buffer that feeds the grouped GEMM; source indices
 * stored in a buffer shared with the combine.  Unlike the pages' receive
 * kernel, the row order here is stable (expert ascending, then token
 * ascending), so the layout is unique and deterministic.
 *
 *   expert_counts[e]  = #{(t,k) : topk_ids[t,k] == e}  for all E experts
 *   expert_offsets[j] = sum of expert_counts[expert_begin + i] for i < j,
 *                       j = 0..E_loc (so expert_offsets[E_loc] = N_loc, the local rows)
 *   for local expert e (ascending), token t (ascending) with topk_ids[t,k] == e:
 *       row = expert_offsets[e - expert_begin] + (rank of t among such tokens)
 *       x_sorted[row,:] = x[t,:] (bit copy); src_index[row] = t*K + k; row_of[t*K+k] = row
 *   row_of[t*K+k] = -1 for assignments to non-local or invalid experts.
 * Ids outside [0, E) are skipped and counted into the int32 at the start of
 * the workspace ("n_invalid", valid after the stream reaches this point).
 * Arguments:
 *   x              [T, d]     dtype
 *   topk_ids       [T, K]     int32
 *   expert_counts  [E]        int32 (out)
 *   expert_offsets [E_loc+1]  int32 (out)
 *   x_sorted       [T*K, d]   dtype (out; rows >= N_loc untouched)
 *   src_index      [T*K]      int32 (out; entries >= N_loc untouched)
 *   row_of         [T*K]      int32 (out)
 *   workspace      >= moe_workspace_bytes(cfg, MOE_WS_DISPATCH) bytes, 256-byte aligned
 */
moe_status_t moe_dispatch(const moe_config_t* cfg, const void* x, const int32_t* topk_ids,
                          int32_t* expert_counts, int32_t* expert_offsets, void* x_sorted,
                          int32_t* src_index, int32_t* row_of, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate device
 * memory (code being captured into a HIP graph, tight serving loops, hosts
 * that forbid hipMalloc): the same kernels and the same results (counts,
 * offsets, x_sorted, src_index, row_of, bit for bit), with the scratch those
 * kernels need taken from a 4 MiB array the library holds on each GPU instead
 * of a workspace argument.  The call allocates nothing.
 *   n_invalid  [1] int32 (out, device) -- the count of ids outside [0, E), or
 *              NULL when the caller does not want it
 * Limits: moe_workspace_bytes(cfg, MOE_WS_DISPATCH) <= 4 MiB (T*K up to about
 * 900k assignments at E = 256), else MOE_ERR_UNSUPPORTED.  Every call on a GPU
 * uses that GPU's one array: calls that may overlap on one GPU (different
 * streams, or graphs replayed concurrently) race and must be serialised by the
 * caller.  The array needs no clearing: each call writes every entry it reads.
 */
moe_status_t moe_dispatch_noalloc(const moe_config_t* cfg, const void* x, const int32_t* topk_ids,
                                  int32_t* expert_counts, int32_t* expert_offsets, void* x_sorted,
                                  int32_t* src_index, int32_t* row_of, int32_t* n_invalid,
                                  moe_stream_t stream);

/*
 * moe_expert_mlp -- grouped SiLU-gated MLP over the expert-contiguous rows,
 * plus optional shared experts over all tokens.
 * [PPLX] Introduction (experts are small MLPs), Dispatch (the contiguous
 * buffer feeds a downstream grouped GEMM); [DBO] Introduction (shared
 * expert "S" in the overlap schedule).
 *
 *   for local expert j, rows r in [expert_offsets[j], expert_offsets[j+1]):
 *     h[r,:]        = SiLU(x_sorted[r,:] . w_gate[j]^T) * (x_sorted[r,:] . w_up[j]^T)
 *     y_sorted[r,:] = h[r,:] . w_down[j]^T,         SiLU(z) = z / (1 + exp(-z))
 *   for shared expert s < num_shared: the same MLP on every token of x,
 *     weights ws_*[s], result in y_shared[s].
 * fp32 accumulation; bf16 configs keep h in bf16 and write bf16 outputs.
 * Row counts are read on the device from expert_offsets (no host sync).
 * Arguments:
 *   x_sorted       [T*K, d]      dtype   (from moe_dispatch)
 *   expert_offsets [E_loc+1]     int32   (from moe_dispatch)
 *   w_gate, w_up   [E_loc, I, d] dtype
 *   w_down         [E_loc, d, I] dtype
 *   y_sorted       [T*K, d]      dtype (out; rows >= N_loc untouched)
 *   x              [T, d]        dtype, shared experts' input (NULL iff num_shared == 0)
 *   ws_gate, ws_up [num_shared, I, d], ws_down [num_shared, d, I]  (NULL iff num_shared == 0)
 *   y_shared       [num_shared, T, d] dtype (out; NULL iff num_shared == 0)
 *   workspace      >= moe_workspace_bytes(cfg, MOE_WS_EXPERT_MLP) bytes, 256-byte aligned
 */
moe_status_t moe_expert_mlp(const moe_config_t* cfg, const void* x_sorted,
                            const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                            const void* w_down, void* y_sorted, const void* x,
                            const void* ws_gate, const void* ws_up, const void* ws_down,
                            void* y_shared, void* workspace, size_t workspace_bytes,
                            moe_stream_t stream);

/*
 * moe_combine -- weighted sum of each token's expert outputs, back in token order.
 * [PPLX] Introduction (output = weighted sum of the selected experts'
 * outputs), Sharding and Parallelism (the accumulation fused into the gather),
 * Combine (router weights applied on the receiving side; the result written to
 * an externally allocated tensor).
 *
 *   out[t,:] = round( sum_{k=0..K-1, row_of[t*K+k] >= 0} topk_weights[t,k] * y_sorted[row_of[t*K+k],:]
 *                     + sum_{s=0..num_shared-1} y_shared[s,t,:] )
 * accumulated in fp32 in exactly that order, rounded once to dtype.
 * Assignments with row_of = -1 (experts hosted elsewhere) contribute nothing:
 * out is this GPU's partial sum.
 * Arguments:
 *   y_sorted     [T*K, d]           dtype
 *   row_of       [T*K]              int32 (from moe_dispatch)
 *   topk_weights [T, K]             fp32  (from moe_route)
 *   y_shared     [num_shared, T, d] dtype, or NULL iff num_shared == 0
 *   out          [T, d]             dtype (out)
 */
moe_status_t moe_combine(const moe_config_t* cfg, const void* y_sorted, const int32_t* row_of,
                         const float* topk_weights, const void* y_shared, void* out,
                         moe_stream_t stream);

/* Scale layouts of moe_quantize_mxfp8. */
enum { MOE_MX_ROWS = 0, MOE_MX_MFMA = 1 };

/*
 * moe_pack_weights -- rearranges a stack of bf16 expert weight matrices once
 * (offline, like a checkpoint conversion) into the layout the expert GEMM
 * streams in order.  The grouped GEMM ([PPLX] Dispatch: the expert-contiguous
 * rows feed a grouped GEMM) reads each weight matrix as k-tiles of 64
 * columns over blocks of 128 rows; row-major storage spreads such a k-tile
 * over 128 rows 2*cols bytes apart, the packed layout stores it as 16 KB in
 * a row, the k-tiles of a row block one after another:
 *   in [n, rows, cols] bf16 (row-major)  ->  packed [n, rows/128, cols/64, 128, 64] bf16,
 *   packed element (m, r / 128, c / 64, r % 128, c % 64) = in[m, r, c].
 * The packed stack has the same size; layers whose config has weight_layout
 * = MOE_WEIGHTS_PACKED take w_gate and w_up ([E_loc, I, d]: rows = I,
 * cols = d), w_down ([E_loc, d, I]: rows = d, cols = I) and the shared
 * stacks in this layout; results are bit-identical to the row-major layer's
 * (the same products in the same order).
 * Requirements: n >= 0 (0: nothing to do), rows a multiple of 128, cols a
 * multiple of 64, n*rows*cols < 2^35 (one work-item per 8 elements, fewer
 * than 2^32 in the launch; else MOE_ERR_UNSUPPORTED); in and packed 16-byte
 * aligned, not overlapping (MOE_ERR_INVALID_ARGUMENT otherwise).
 */
moe_status_t moe_pack_weights(int32_t n, int32_t rows, int32_t cols, const void* in, void* packed,
                              moe_stream_t stream);

/*
 * moe_quantize_mxfp8 -- block-scaled 8-bit encoding of the rows of a matrix,
 * the form in which [PPLX] Dispatch sends token payloads (activations with
 * per-block scaling factors; the page fixes no format).  Format: OCP MX-FP8,
 * the operand format of gfx950's scaled MFMA.  Each run of 32 consecutive
 * elements of a row shares one scale 2^s with s = floor(log2 max|x|) - 8,
 * kept within [-127, 127] (s = -127 for an all-zero block), stored as the
 * E8M0 byte s + 127; each element becomes x / 2^s, clamped to +-448 and
 * rounded to the nearest E4M3 (fn) value, ties to even.  A decoded element is
 * e4m3(code) * 2^(scale - 127).  Inputs must be finite.
 * Arguments:
 *   rows, cols    rows >= 0; cols > 0, a multiple of 32 (of 512 for
 *                 MOE_MX_MFMA)
 *   dtype         MOE_BF16 or MOE_F32
 *   in            [rows, ld] dtype: the first cols elements of each row are
 *                 encoded; 16-byte aligned, ld >= cols, ld * element size a
 *                 multiple of 16 bytes
 *   scale_layout  where the scale of block q (elements 32q .. 32q + 31) of
 *                 row r goes in `scales` (rows * cols / 32 bytes either way):
 *                 MOE_MX_ROWS: byte r * cols/32 + q;
 *                 MOE_MX_MFMA: with q = 16g + m, m = 8d + 4j + 2s + h (each of
 *                 d, j, s, h 0 or 1), byte 2j + s of 32-bit word
 *                 ((2g + d) * rows + r) * 2 + h -- the layout that
 *                 moe_expert_mlp_mxfp8 reads
 *   codes         [rows, cols] uint8 E4M3 (out), 8-byte aligned
 *   scales        uint8 E8M0 (out), 4-byte aligned
 * The result is bit-exact and independent of the launch.  rows == 0 enqueues
 * nothing and reads no pointer.  rows * cols / 8 must stay below 2^32 - 256
 * (one work-item per 8 elements; MOE_ERR_UNSUPPORTED otherwise).
 */
moe_status_t moe_quantize_mxfp8(int32_t rows, int32_t cols, int32_t dtype, const void* in,
                                int64_t ld, int32_t scale_layout, uint8_t* codes,
                                uint8_t* scales, moe_stream_t stream);

/*
 * moe_expert_mlp_mxfp8 -- moe_expert_mlp with MX-FP8 operands: the dispatched
 * payload reaches the grouped GEMM with block scaling factors ([PPLX]
 * Dispatch) and the expert outputs return in 16 bits ([PPLX] Combine).  For
 * each local expert e and each of its rows,
 *   h = SiLU(D(xq) D(gq_e)^T) * (D(xq) D(uq_e)^T)   accumulated in fp32,
 *   y = h' W'_e^T                                   accumulated in fp32,
 *                                                   rounded to bf16,
 * with D() the decoding of moe_quantize_mxfp8 (every product of two decoded
 * elements is exact in fp32) and, for the down projection, either
 *   - bf16 weights (w_down given): h' = h rounded to bf16, W'_e = w_down[e]; or
 *   - MX-FP8 weights (wq_down and wq_down_scales given): h' = D(MX-FP8 encoding
 *     of h, blocks of 32 along I, from the fp32 values), W'_e = D(wq_down[e]);
 *     requires cfg->intermediate to be a multiple of 512.
 * Exactly one of the two must be given.  Requires cfg->dtype == MOE_BF16,
 * cfg->num_shared == 0 (the block-scaled shared experts run inside
 * moe_forward_mxfp8) and cfg->hidden a multiple of 512 (MOE_ERR_UNSUPPORTED
 * otherwise).
 * Arguments (T = num_tokens, K = top_k, d = hidden, I = intermediate,
 * E_loc = expert_end - expert_begin):
 *   xq_sorted       [T*K, d] E4M3 codes of the dispatched rows
 *   xq_scales       their scales, MOE_MX_MFMA layout with rows = T*K
 *   expert_offsets  [E_loc + 1] int32 (from moe_dispatch)
 *   wq_gate, wq_up  [E_loc, I, d] E4M3 codes
 *   wq_gate_scales, wq_up_scales
 *                   scales of the [E_loc * I, d] stacks, MOE_MX_MFMA layout
 *                   with rows = E_loc * I
 *   w_down          [E_loc, d, I] bf16, or NULL
 *   wq_down         [E_loc, d, I] E4M3 codes, or NULL
 *   wq_down_scales  scales of the [E_loc * d, I] stack, MOE_MX_MFMA layout with
 *                   rows = E_loc * d, or NULL
 *   y_sorted        [T*K, d] bf16 (out); rows past the local count untouched
 *   workspace       >= moe_workspace_bytes(cfg, MOE_WS_EXPERT_MLP) bytes,
 *                   256-byte aligned
 * Code arrays and bf16 arrays 16-byte aligned, scale arrays 4-byte aligned.
 */
moe_status_t moe_expert_mlp_mxfp8(const moe_config_t* cfg, const uint8_t* xq_sorted,
                                  const uint8_t* xq_scales, const int32_t* expert_offsets,
                                  const uint8_t* wq_gate, const uint8_t* wq_gate_scales,
                                  const uint8_t* wq_up, const uint8_t* wq_up_scales,
                                  const void* w_down, const uint8_t* wq_down,
                                  const uint8_t* wq_down_scales, void* y_sorted, void* workspace,
                                  size_t workspace_bytes, moe_stream_t stream);

/*
 * moe_dispatch_mxfp8 -- moe_dispatch with the block-scaled payload of [PPLX]
 * Dispatch: each routed token row is encoded once as MX-FP8 (the rule of
 * moe_quantize_mxfp8) and its codes and scales are written to every local
 * row of the token.  expert_counts, expert_offsets, src_index, row_of and
 * n_invalid are exactly those of moe_dispatch; the codes and scales of row r
 * are moe_quantize_mxfp8 of row r of moe_dispatch's x_sorted.  Requires
 * cfg->dtype == MOE_BF16 and cfg->hidden a multiple of 512
 * (MOE_ERR_UNSUPPORTED otherwise).
 * Arguments as moe_dispatch, with x_sorted replaced by
 *   xq_sorted  [T*K, d] uint8 E4M3 (out; rows >= N_loc untouched), 16-byte
 *              aligned
 *   xq_scales  T*K*d/32 bytes (out), MOE_MX_MFMA layout with rows = T*K
 *              (entries of rows >= N_loc untouched), 4-byte aligned
 */
moe_status_t moe_dispatch_mxfp8(const moe_config_t* cfg, const void* x, const int32_t* topk_ids,
                                int32_t* expert_counts, int32_t* expert_offsets,
                                uint8_t* xq_sorted, uint8_t* xq_scales, int32_t* src_index,
                                int32_t* row_of, void* workspace, size_t workspace_bytes,
                                moe_stream_t stream);

/* Tensors of a whole-layer call (moe_forward, moe_forward_dbo). */
typedef struct moe_layer_tensors {
  const void* x;             /* [T, d] dtype                                     */
  const void* w_router;      /* [E, d] dtype                                     */
  const float* bias;         /* [E] fp32 or NULL                                 */
  const void* w_gate;        /* [E_loc, I, d] dtype                              */
  const void* w_up;          /* [E_loc, I, d] dtype                              */
  const void* w_down;        /* [E_loc, d, I] dtype                              */
  const void* ws_gate;       /* [num_shared, I, d] dtype or NULL                 */
  const void* ws_up;         /* [num_shared, I, d] dtype or NULL                 */
  const void* ws_down;       /* [num_shared, d, I] dtype or NULL                 */
  void* out;                 /* [T, d] dtype (out)                               */
  int32_t* topk_ids;         /* [T, K] int32 (out)                               */
  float* topk_weights;       /* [T, K] fp32 (out)                                */
} moe_layer_tensors_t;

/*
 * moe_forward -- the whole layer on one stream: moe_route, moe_dispatch,
 * moe_expert_mlp, moe_combine, with every intermediate (x_sorted, y_sorted,
 * maps, counts, h, y_shared) carved from the caller's workspace of at least
 * moe_workspace_bytes(cfg, MOE_WS_FORWARD) bytes (256-byte aligned).
 */
moe_status_t moe_forward(const moe_config_t* cfg, const moe_layer_tensors_t* tensors,
                         void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Tensors of a block-scaled whole-layer call (moe_forward_mxfp8). */
typedef struct moe_layer_tensors_mxfp8 {
  const void* x;                /* [T, d] bf16                                      */
  const void* w_router;         /* [E, d] bf16                                      */
  const float* bias;            /* [E] fp32 or NULL                                 */
  const uint8_t* wq_gate;       /* [E_loc, I, d] E4M3 codes                         */
  const uint8_t* wq_gate_scales;/* MOE_MX_MFMA scales of the [E_loc*I, d] stack     */
  const uint8_t* wq_up;         /* [E_loc, I, d] E4M3 codes                         */
  const uint8_t* wq_up_scales;  /* MOE_MX_MFMA scales of the [E_loc*I, d] stack     */
  const void* w_down;           /* [E_loc, d, I] bf16, or NULL                      */
  const uint8_t* wq_down;       /* [E_loc, d, I] E4M3 codes, or NULL                */
  const uint8_t* wq_down_scales;/* MOE_MX_MFMA scales of the [E_loc*d, I] stack     */
  /* Shared experts (cfg->num_shared = S > 0; all NULL when S == 0): encoded
   * like the routed ones, the down weights in the routed experts' form.     */
  const uint8_t* wsq_gate;       /* [S, I, d] E4M3 codes                             */
  const uint8_t* wsq_gate_scales;/* MOE_MX_MFMA scales of the [S*I, d] stack         */
  const uint8_t* wsq_up;         /* [S, I, d] E4M3 codes                             */
  const uint8_t* wsq_up_scales;  /* MOE_MX_MFMA scales of the [S*I, d] stack         */
  const void* ws_down;           /* [S, d, I] bf16 (with w_down), else NULL          */
  const uint8_t* wsq_down;       /* [S, d, I] E4M3 codes (with wq_down), else NULL   */
  const uint8_t* wsq_down_scales;/* MOE_MX_MFMA scales of the [S*d, I] stack         */
  void* out;                    /* [T, d] bf16 (out)                                */
  int32_t* topk_ids;            /* [T, K] int32 (out)                               */
  float* topk_weights;          /* [T, K] fp32 (out)                                */
} moe_layer_tensors_mxfp8_t;

/*
 * moe_forward_mxfp8 -- the whole layer with the block-scaled payload on one
 * stream: moe_route, moe_dispatch_mxfp8, moe_expert_mlp_mxfp8, moe_combine,
 * the intermediates carved from a workspace of at least
 * moe_workspace_bytes(cfg, MOE_WS_FORWARD) bytes (256-byte aligned).  The
 * gate and up weights are passed encoded (moe_quantize_mxfp8 of the
 * [E_loc*I, d] stacks, MOE_MX_MFMA layout, done once, offline), the down
 * weights either in bf16 (w_down) or encoded too (wq_down, wq_down_scales;
 * the other NULL), as for moe_expert_mlp_mxfp8, with the same requirements
 * except that shared experts are allowed (as in moe_expert_mlp: [DBO]
 * Introduction's shared expert, applied to every token with weight one).
 * A shared expert s reads the token rows encoded by the same rule (D(xq)
 * below is the decoding of x's moe_quantize_mxfp8; wsq_* are its weights):
 *   h_s = SiLU(D(xq) D(gsq_s)^T) * (D(xq) D(usq_s)^T)   in fp32,
 *   y_s = h_s' W'_s^T                                   in fp32, to bf16,
 * with h_s' and W'_s as for the routed experts (ws_down, or the encoded h_s
 * and wsq_down); the combine adds the y_s as moe_combine adds y_shared.
 */
moe_status_t moe_forward_mxfp8(const moe_config_t* cfg,
                               const moe_layer_tensors_mxfp8_t* tensors, void* workspace,
                               size_t workspace_bytes, moe_stream_t stream);

/*
 * moe_forward_dbo -- the layer as two microbatches on two streams of one GPU.
 * [DBO] UBatchRunner: the token count is padded up to a multiple of 256 and
 * split at the midpoint: microbatch 0 = tokens [0, min(mid, T)), microbatch 1
 * = [mid, T) (no work when empty).  [DBO] Introduction and Interfaces: one
 * microbatch's dispatch/combine runs on the communication stream while the
 * other microbatch's expert compute runs on the compute stream:
 *     compute: route0, route1, mlp0, mlp1
 *     comm:    dispatch0, dispatch1, combine0, combine1
 * with events ordering each microbatch's steps, so dispatch1 overlaps mlp0
 * and combine0 overlaps mlp1.  With shared experts and cfg->shared_placement
 * = MOE_SHARED_BESIDE_COMBINE the compute stream runs each microbatch's
 * shared-expert MLP right after its routed MLP, beside its combine:
 *     compute: route0, route1, mlp0, shared0, mlp1, shared1
 *     comm:    dispatch0, dispatch1, combine0, finish0, combine1, finish1
 * (finish = the shared rows added to the combine's sums).  Every output row
 * depends only on its own token, so the result is bitwise equal to
 * moe_forward's.
 * If T < min_tokens_to_split (or microbatch 1 is empty) the unsplit forward
 * runs on `compute`.  On return, work enqueued later on `compute` waits for
 * both microbatches; `comm` may be the same stream as `compute`.
 * workspace >= moe_workspace_bytes(cfg, MOE_WS_FORWARD_DBO) bytes.
 */
moe_status_t moe_forward_dbo(const moe_config_t* cfg, const moe_layer_tensors_t* tensors,
                             void* workspace, size_t workspace_bytes,
                             int32_t min_tokens_to_split, moe_stream_t compute,
                             moe_stream_t comm);

/*
 * moe_forward_dbo_at -- moe_forward_dbo with the cut given: microbatch 0 =
 * tokens [0, split), microbatch 1 = [split, T); split <= 0 or >= T runs the
 * unsplit forward on `compute`.  Same schedule, streams and result (bitwise
 * equal to moe_forward's for every split).  workspace >=
 * moe_workspace_bytes(cfg, MOE_WS_FORWARD_DBO) bytes, which covers every cut.
 */
moe_status_t moe_forward_dbo_at(const moe_config_t* cfg, const moe_layer_tensors_t* tensors,
                                void* workspace, size_t workspace_bytes, int32_t split,
                                moe_stream_t compute, moe_stream_t comm);

/*
 * moe_dbo_plan_split -- whether and where to cut a batch of num_tokens tokens
 * (pure host function).  [DBO] Running with DBO: a batch is split only when it
 * has at least `decode_threshold` tokens (a batch of decodes only) or
 * `prefill_threshold` tokens (a batch with at least one prefill; has_prefill
 * != 0).  [DBO] UBatchRunner: the cut is moe_dbo_split_point's midpoint of the
 * padded count, except that a uniform batch of multi-token queries (no
 * prefill, uniform_query_len = q > 1 tokens per request, num_tokens a
 * multiple of q) is cut on the request boundary nearest that midpoint (the
 * lower of two equally near ones), so both halves stay uniform.  Returns the
 * first token of microbatch 1, or 0 for "do not split" (below the threshold,
 * or microbatch 1 would be empty); pass the result to moe_forward_dbo_at.
 */
int32_t moe_dbo_plan_split(int32_t num_tokens, int32_t has_prefill, int32_t decode_threshold,
                           int32_t prefill_threshold, int32_t uniform_query_len);

/*
 * Graph capture of a whole-layer call.  [DBO] Limitations and UBatchWrapper:
 * the overlapped forward is captured whole, as one graph, and a captured graph
 * replays with no host work between its kernels.
 *
 * moe_graph_capture_forward / moe_graph_capture_forward_dbo record every
 * launch of one moe_forward / moe_forward_dbo call (same arguments and
 * checks) into an executable HIP graph, on private streams of the current
 * device (created and destroyed inside the call, default priority); nothing
 * runs during the capture.  The tensor and workspace pointers are fixed in the
 * graph: each moe_graph_launch recomputes the layer from what those buffers
 * hold at that time and writes the same outputs, so the buffers must outlive
 * the graph.  moe_graph_launch enqueues a replay on `stream` (asynchronous;
 * replays on one stream run in order; replays of one graph must not overlap).
 * moe_graph_destroy releases the graph (after its replays have completed, or
 * the runtime defers the release).  *graph is written only on MOE_OK.
 */
typedef struct moe_graph* moe_graph_t;

moe_status_t moe_graph_capture_forward(const moe_config_t* cfg,
                                       const moe_layer_tensors_t* tensors, void* workspace,
                                       size_t workspace_bytes, moe_graph_t* graph);
moe_status_t moe_graph_capture_forward_dbo(const moe_config_t* cfg,
                                           const moe_layer_tensors_t* tensors, void* workspace,
                                           size_t workspace_bytes, int32_t min_tokens_to_split,
                                           moe_graph_t* graph);
/* The same for one moe_forward_mxfp8 call (block-scaled layer). */
moe_status_t moe_graph_capture_forward_mxfp8(const moe_config_t* cfg,
                                             const moe_layer_tensors_mxfp8_t* tensors,
                                             void* workspace, size_t workspace_bytes,
                                             moe_graph_t* graph);
moe_status_t moe_graph_launch(moe_graph_t graph, moe_stream_t stream);
moe_status_t moe_graph_destroy(moe_graph_t graph);

/* Bytes of workspace needed by a call of the given kind (MOE_WS_*), or 0 for
 * an invalid configuration.  Pure host function. */
size_t moe_workspace_bytes(const moe_config_t* cfg, int32_t kind);

/* Token index at which moe_forward_dbo splits T tokens (pure host function). */
int32_t moe_dbo_split_point(int32_t num_tokens);

/* Static description of a status code (host). */
const char* moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
