/*
 * moe_w4a16.h -- fused Mixture-of-Experts layer with 4-bit expert weights and
 * bf16 activations (W4A16) for AMD MI355X (gfx950).
 *
 * The layer, step by step (the steps of the fused MoE call that the
 * "moe_wna16_marlin_gemm applies wrong per-row topk weights" page replays):
 *
 *   moe_route        router logits -> top-k expert ids and routing weights
 *   moe_align        flat slots sorted by expert, each expert padded to block_m
 *   moe_w4a16_gemm1  grouped GEMM with the gate/up weights (w13), bias and the
 *                    swigluoai or ReLU^2 activation fused in the epilogue
 *   moe_w4a16_gemm2  grouped GEMM with the down weights (w2), bias and the
 *                    per-row routing weight fused in the epilogue
 *   moe_forward      all of the above plus the sum of each token's top-k rows
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is device memory owned by the caller (global
 *   memory of the GPU current on the calling thread), contiguous, row-major.
 *   The library allocates nothing, never synchronises, never reads device
 *   memory from the host and keeps no state between calls (one exception:
 *   moe_forward_noalloc keeps its scratch array's address per device): all
 *   work is enqueued on `stream` (a hipStream_t; NULL is the default stream).
 * - bf16 values are passed as uint16_t bit patterns.
 * - A "flat slot" is f = t*top_k + j (token t, choice j).  The padding id in
 *   sorted_ids is the sentinel size_m*top_k.
 * - Every call validates its arguments on the host before launching
 *   anything and returns a status; no C++ exception crosses this boundary.
 *   A non-MOE_OK status means nothing was enqueued, except MOE_ERR_HIP,
 *   which reports a launch failure (work enqueued before it may have run).
 * - Device data conventions: expert ids outside [0, E) are not routed (align
 *   gives them no slot; the sum skips them).  NaN scales propagate to every
 *   output they reach (e4m3 0x7F and 0xFF, e8m0 0xFF, NaN fp16 scales and
 *   global scales); e8m0 0x00 is 2^-127.  Dequantised weights beyond the bf16
 *   range become infinities.
 * - Sizes: K (the reduction length) must be a multiple of 32 and of the
 *   group size; N must be a multiple of 16 (32 for the gated GEMM1, whose
 *   rows pair up).  K and N tails are handled exactly: no buffer is padded
 *   (hidden 2880 stays 2880; "gpt-oss-120b MXFP4 + --enable-expert-parallel
 *   crashes", root cause: the op's output is the unpadded width).
 * - Base pointers of qweight, scales, zeros, x/a and outputs must be 16-byte
 *   aligned (bias: 2-byte).
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* sizes are inconsistent or out of range */
  MOE_ERR_UNSUPPORTED = 3, /* a format / activation / option combination that is not built */
  MOE_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned */
  MOE_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  MOE_ERR_WORKSPACE = 6,   /* workspace smaller than moe_forward_workspace_bytes() */
  MOE_ERR_TOO_LARGE = 7    /* moe_forward_noalloc: the call needs more than its fixed scratch */
} moe_status_t;

/* 4-bit weight storage formats.
 * NVFP4: e2m1 codes + fp8-e4m3fn scale per 16 along K + fp32 global scale per
 *   expert; w = e2m1 * scale * global ("moe_wna16_marlin_gemm applies wrong
 *   per-row topk weights", minimal repro: ModelOpt NVFP4 layout and its
 *   dequantised reference).
 * MXFP4: e2m1 codes + e8m0 shared exponent per 32 along K; w = e2m1 * 2^(s-127)
 *   ("gpt-oss-120b MXFP4 ..." page names the format; the block layout is the
 *   OCP microscaling one).
 * INT4_GPTQ: asymmetric uint4 with uint4 zero points and fp16 scales per
 *   group along K; w = (q - z) * s (OneCompression "GPT-OSS (mixed_gptq)",
 *   sections 1 and "Why GPT-OSS needs special handling": group size 64 for
 *   hidden 2880, 45 groups). */
typedef enum { MOE_W_NVFP4 = 0, MOE_W_MXFP4 = 1, MOE_W_INT4_GPTQ = 2 } moe_wfmt_t;

/* Epilogue of GEMM1.
 * SWIGLUOAI: gpt-oss clamped SwiGLU over interleaved rows (row 2i = gate,
 *   2i+1 = up): g = min(gate, limit), u = clamp(up, -limit, limit),
 *   a = g * sigmoid(alpha * g) * (u + beta) ("gpt-oss-20b NVFP4 inference is
 *   broken", Gap 3: alpha/beta/clamp limit, biases, interleaved gate/up).
 * RELU2: non-gated a = max(h, 0)^2 (Nemotron-3-Nano page, summary and
 *   environment: non-gated ReLU^2 MoE).
 * NONE: a = h (the raw pre-activation; for testing GEMM1 alone). */
typedef enum { MOE_ACT_SWIGLUOAI = 0, MOE_ACT_RELU2 = 1, MOE_ACT_NONE = 2 } moe_act_t;

/* Router.
 * SOFTMAX: topk(softmax(logits)) ("moe_wna16_marlin_gemm ..." repro, routing
 *   step); selection on the raw logits, descending, ties to the lower id.
 * SIGMOID_BIAS: score = sigmoid(l) + bias[e] in fp32 (sigmoid evaluated in
 *   double and rounded once), top-k of the scores with n_group = 1, weights =
 *   the selected *unbiased* sigmoids (Nemotron-3-Nano page, Analysis item 3). */
typedef enum { MOE_ROUTE_SOFTMAX = 0, MOE_ROUTE_SIGMOID_BIAS = 1 } moe_route_t;

/* One family of 4-bit expert weights; logical W_e is [N][K] (out x reduce). */
typedef struct {
  moe_wfmt_t fmt;
  int group_size;             /* NVFP4: 16, MXFP4: 32, GPTQ: 32/64/128; must divide K */
  const void* qweight;        /* NVFP4/MXFP4: uint8 [E][N][K/2], even k in the low nibble.
                                 GPTQ: int32 [E][K/8][N], nibble i holds k%8 == i.
                                 NVFP4/MXFP4 may pass NULL here and in `scales` when both
                                 copies by K chunk (qweight_kc, scales_kc) are given: every
                                 kernel then reads those, so a caller holds one copy of the
                                 codes ("chunked-only" family).  Otherwise required. */
  const void* scales;         /* NVFP4: e4m3fn uint8 [E][N][K/16]; MXFP4: e8m0 uint8 [E][N][K/32];
                                 GPTQ: fp16 [E][K/G][N].  NULL only in a chunked-only family */
  const void* zeros;          /* GPTQ: int32 [E][K/G][N/8], nibble i holds n%8 == i. Else NULL */
  const float* global_scale;  /* NVFP4: fp32 [E]. Else NULL */
  const int32_t* g_idx;       /* GPTQ group of each row, int32 [E][K] (4-byte aligned), or NULL
                                 for group = k / group_size.  The kernels read groups as runs
                                 of group_size rows, so the only map they take is that
                                 identity: each workgroup checks its expert's map on the
                                 device, and a map that differs anywhere turns every output
                                 that expert's weights produce into NaN (a visible failure).
                                 Act-order maps are first put in group order by
                                 moe_gptq_act_order_sort (whose weights come with k_perm and
                                 g_idx = NULL; both set is MOE_ERR_UNSUPPORTED).  Other formats:
                                 must be NULL. */
  const uint16_t* bias;       /* bf16 [E][N], or NULL for no bias */
  const int32_t* k_perm;      /* GPTQ act-order: NULL, or int32 [E][K] from moe_gptq_act_order_sort
                                 (row k of the stored weight multiplies input channel
                                 k_perm[e][k]; 16-byte aligned, K <= 8192).  Only moe_forward
                                 accepts it (it gathers the GEMM inputs through it); the
                                 single GEMM calls return MOE_ERR_UNSUPPORTED: gather with
                                 moe_permute_slots and call them in the top_k = 1 view. */
  const uint8_t* scales_kc;   /* optional load-time copy of the scales laid out by K chunk.  The
                                 64/128-row (streaming) GEMM kernel then streams each chunk's
                                 scales with its codes instead of holding the tile's scales
                                 for the whole K on chip, so two workgroups share a CU; every
                                 other kernel reads it in place of `scales` too.  NVFP4: uint8
                                 [E][K/64][N][4] from moe_nvfp4_scales_by_chunk (K a multiple of
                                 64).  MXFP4: uint8 [E][ceil(K/128)][N][4] from
                                 moe_mxfp4_scales_by_chunk.  16-byte aligned.  GPTQ: must be
                                 NULL. */
  const uint8_t* qweight_kc;  /* optional load-time copy of the codes laid out by K chunk, so the
                                 copy of one chunk of a 32-row block is one contiguous piece
                                 instead of 32 row pieces; every kernel reads it in place of
                                 `qweight` when given.  NVFP4, only together with scales_kc:
                                 uint8 [E][K/64][N][32] (moe_nvfp4_codes_by_chunk).  MXFP4: uint8
                                 [E][ceil(K/128)][N][64] (moe_mxfp4_codes_by_chunk), alone or
                                 with scales_kc.  16-byte aligned. */
} moe_wq_t;

/* Kernel for the grouped GEMMs over blocks of 16 or 32 rows (few tokens per
 * expert).  AUTO: the library's choice from the launch size.  SPLITK: the
 * split-K kernel (32 weight rows per workgroup, K split over its waves).
 * WIDE: 128 weight rows per workgroup with the A rows shared through on-chip
 * memory (the split-K kernel where its scale tile would not fit).  The results
 * agree to the rounding of the fp32 accumulation order.  Blocks of 64/128 rows
 * always run the streaming prefill kernel.  Taken by the _ex entry points; the
 * plain ones use AUTO.  Any other value is MOE_ERR_UNSUPPORTED. */
typedef enum { MOE_KERNEL_AUTO = 0, MOE_KERNEL_SPLITK = 1, MOE_KERNEL_WIDE = 2 } moe_kernel_t;

/* Length of sorted_ids for T tokens: T*top_k + min(E, T*top_k)*(block_m-1),
 * rounded up to block_m (every expert that can receive a slot pads to
 * block_m).  expert_ids has moe_align_capacity()/block_m entries. */
size_t moe_align_capacity(int T, int top_k, int E, int block_m);

/* Route T tokens over E experts.
 *   logits      fp32 [T][E]
 *   expert_bias fp32 [E] for SIGMOID_BIAS, ignored (may be NULL) for SOFTMAX
 *   renormalize 1: weights divided by their sum over the selected k
 *   topk_ids    out int32 [T][top_k], descending score, ties to lower id
 *   topk_w      out fp32 [T][top_k]
 * Limits: 1 <= top_k <= min(E, 16), E <= 1024, T >= 0 (T = 0 is a no-op). */
moe_status_t moe_route(const float* logits, int T, int E, int top_k, moe_route_t kind,
                       const float* expert_bias, int renormalize,
                       int32_t* topk_ids, float* topk_w, moe_stream_t stream);

/* Stable sort of the T*top_k flat slots by expert id, each expert's run
 * padded to a multiple of block_m with the sentinel T*top_k ("moe_align_block_size"
 * in the repro; the reference loop reads blocks with expert id < 0 as empty).
 *   topk_ids     int32 [T*top_k]
 *   sorted_ids   out int32 [moe_align_capacity()]: experts ascending, slots
 *                ascending within an expert, sentinel in padding and past the end
 *   expert_ids   out int32 [capacity/block_m]: expert of each block, -1 past the end
 *   num_post_pad out int32 [1]: padded length actually used
 * block_m in {16, 32, 64, 128}; E <= 1024; T*top_k < 2^24. */
moe_status_t moe_align(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
                       int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post_pad,
                       moe_stream_t stream);

/* The same sort (same outputs, bit for bit) spread over 16 workgroups, for
 * large batches: a counting launch writes each workgroup's per-expert counts
 * to `counts`, a placing launch reads them.  moe_forward uses it from 8192
 * slots on, with the counts in its workspace.
 *   counts  int32 scratch of moe_align_large_scratch_bytes(E) bytes (16*E
 *           ints), caller-owned, overwritten; no alignment beyond 4 bytes.
 * Other arguments and limits as moe_align. */
moe_status_t moe_align_large(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
                             int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post_pad,
                             int32_t* counts, moe_stream_t stream);
/* Bytes of moe_align_large's counts for E experts (0 if E is out of range). */
size_t moe_align_large_scratch_bytes(int E);

/* moe_route followed by moe_align on its ids, with the same outputs as the
 * two calls (all five written).  Small batches run both steps in one launch
 * (the routed ids pass through on-chip memory); larger ones run the two
 * kernels back to back.  Limits are those of moe_route and moe_align. */
moe_status_t moe_route_align(const float* logits, int T, int E, int top_k, moe_route_t kind,
                             const float* expert_bias, int renormalize, int block_m,
                             int32_t* topk_ids, float* topk_w, int32_t* sorted_ids,
                             int32_t* expert_ids, int32_t* num_post_pad, moe_stream_t stream);

/* Grouped GEMM1 over aligned blocks.  For every real entry f of block b
 * (expert e = expert_ids[b]):
 *   h   = W13_e . x[f / top_k] (+ bias13_e)           fp32 accumulate
 *         (with mul_topk_weights: W13_e . (topk_w[f] x[f / top_k]) + bias13_e,
 *          the routing weight applied on the input, "apply_router_weight_on_input"
 *          on the "moe_wna16_marlin_gemm applies wrong per-row topk weights" page;
 *          topk_w fp32 [size_m*top_k], may be NULL when the flag is 0)
 *   out[f][:] = act(h)  bf16 (round to nearest even)
 *   x    bf16 [size_m][K]
 *   N    rows of W13 (2*intermediate when gated, intermediate for RELU2/NONE)
 *   out  bf16 [size_m*top_k][N/2] for SWIGLUOAI, [size_m*top_k][N] otherwise;
 *        rows of slots that no block covers are left untouched.
 * sorted_ids / expert_ids / num_post_pad come from moe_align with the same
 * block_m, size_m and top_k. */
moe_status_t moe_w4a16_gemm1(const uint16_t* x, int size_m, int top_k, int K, int N, int E,
                             const moe_wq_t* w13, moe_act_t act, float alpha, float beta,
                             float limit, const float* topk_w, int mul_topk_weights,
                             const int32_t* sorted_ids, const int32_t* expert_ids,
                             const int32_t* num_post_pad, int block_m, uint16_t* out,
                             moe_stream_t stream);

/* Grouped GEMM2.  For every real entry f of block b (expert e):
 *   y[f][:] = (W2_e . a[f / top_k] (+ bias2_e)) * (mul_topk_weights ? topk_w[f] : 1)
 * The layer calls it in the top_k = 1 view (size_m = T*top_k, one A row per
 * flat slot), as the "moe_wna16_marlin_gemm applies wrong per-row topk
 * weights" page's repro calls its gemm2 step; top_k > 1 shares one A row
 * between top_k slots, as GEMM1 does.  The routing weight is read from topk_w
 * at the row's own flat slot (that page's fix: each row gets its own weight).
 *   a      bf16 [size_m][K]
 *   topk_w fp32 [size_m*top_k]      (may be NULL when mul_topk_weights = 0)
 *   y      bf16 [size_m*top_k][N]; rows no block covers are left untouched.
 * sorted_ids / expert_ids / num_post_pad come from moe_align with the same
 * block_m, size_m and top_k (sentinel size_m*top_k). */
moe_status_t moe_w4a16_gemm2(const uint16_t* a, int size_m, int top_k, int K, int N, int E,
                             const moe_wq_t* w2, const float* topk_w, int mul_topk_weights,
                             const int32_t* sorted_ids, const int32_t* expert_ids,
                             const int32_t* num_post_pad, int block_m, uint16_t* y,
                             moe_stream_t stream);

/* moe_w4a16_gemm1 and moe_w4a16_gemm2 with the kernel for 16/32-row blocks
 * chosen by the caller (moe_kernel_t; for tuning and for testing each kernel). */
moe_status_t moe_w4a16_gemm1_ex(const uint16_t* x, int size_m, int top_k, int K, int N, int E,
                                const moe_wq_t* w13, moe_act_t act, float alpha, float beta,
                                float limit, const float* topk_w, int mul_topk_weights,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_post_pad, int block_m, uint16_t* out,
                                moe_kernel_t kernel, moe_stream_t stream);
moe_status_t moe_w4a16_gemm2_ex(const uint16_t* a, int size_m, int top_k, int K, int N, int E,
                                const moe_wq_t* w2, const float* topk_w, int mul_topk_weights,
                                const int32_t* sorted_ids, const int32_t* expert_ids,
                                const int32_t* num_post_pad, int block_m, uint16_t* y,
                                moe_kernel_t kernel, moe_stream_t stream);

/* GPTQ act-order preparation, run once when the weights are loaded.  A GPTQ
 * checkpoint quantised in activation order stores its rows in input-channel
 * order with the group of each row in g_idx (the per-expert qweight / qzeros /
 * scales / g_idx tensors of the OneCompression "GPT-OSS (mixed_gptq)" page,
 * section 1); the dequantised weight is w[k][n] = (q[k][n] - z[g_idx[k]][n]) *
 * s[g_idx[k]][n].  Per expert e this computes
 *   k_perm[e]          the rows sorted by group, ascending k within a group
 *   qweight_sorted[e]  row j = row k_perm[e][j] of qweight[e] (same packing)
 *   status[e]          0, or 1 when g_idx[e] is not an act-order map (a value
 *                      outside [0, K/G) or a group without exactly G rows);
 *                      k_perm[e] is then the identity and the expert must not
 *                      be used with k_perm.
 * With status 0 everywhere, {qweight_sorted, the same scales and zeros,
 * g_idx = NULL, k_perm} describes the same weights as {qweight, g_idx}.
 *   qweight         int32 [E][K/8][N] (the moe_wq_t GPTQ packing)
 *   g_idx           int32 [E][K]
 *   qweight_sorted  out int32 [E][K/8][N]; must not overlap qweight
 *   k_perm          out int32 [E][K];  status  out int32 [E]
 * group_size in {32, 64, 128}, K a multiple of it, K <= 8192, E <= 1024.
 * The statuses are written on the device: read them after the stream. */
moe_status_t moe_gptq_act_order_sort(const int32_t* qweight, const int32_t* g_idx, int E, int K,
                                     int N, int group_size, int32_t* qweight_sorted,
                                     int32_t* k_perm, int32_t* status, moe_stream_t stream);

/* NVFP4 scales re-laid by K chunk, run once when the weights are loaded:
 *   out[e][c][n][j] = scales[e][n][4c + j]   (c < K/64, j < 4)
 * i.e. the four e4m3 group scales of each 64-deep chunk of each weight row,
 * rows of one chunk contiguous.  scales uint8 [E][N][K/16] (the moe_wq_t NVFP4
 * layout); out uint8 [E][K/64][N][4]; K % 64 == 0; both 16-byte aligned. */
moe_status_t moe_nvfp4_scales_by_chunk(const uint8_t* scales, int E, int N, int K, uint8_t* out,
                                       moe_stream_t stream);

/* NVFP4 codes re-laid by K chunk, run once when the weights are loaded:
 *   out[e][c][n][j] = qweight[e][n][32c + j]   (c < K/64, j < 32)
 * i.e. the 32 code bytes (64 packed values) of each 64-deep chunk of each
 * weight row, rows of one chunk contiguous.  qweight uint8 [E][N][K/2] (the
 * moe_wq_t NVFP4 layout); out uint8 [E][K/64][N][32], a separate buffer;
 * K % 64 == 0; both 16-byte aligned.  Costs a second copy of the codes: the
 * 1..64-token kernels keep reading qweight. */
moe_status_t moe_nvfp4_codes_by_chunk(const uint8_t* qweight, int E, int N, int K, uint8_t* out,
                                      moe_stream_t stream);

/* MXFP4 codes re-laid by 128-deep K chunk for the MX kernels, run once when
 * the weights are loaded:
 *   out[e][c][n][j] = qweight[e][n][64c + j] for 64c + j < K/2, else 0
 *   (c < ceil(K/128), j < 64)
 * qweight uint8 [E][N][K/2]; out uint8 [E][ceil(K/128)][N][64], a separate
 * buffer; K % 32 == 0; both 16-byte aligned.  A second copy of the codes (the
 * bf16-activation kernels keep reading qweight). */
moe_status_t moe_mxfp4_codes_by_chunk(const uint8_t* qweight, int E, int N, int K, uint8_t* out,
                                      moe_stream_t stream);

/* MXFP4 scales re-laid by 128-deep K chunk, run once when the weights are
 * loaded:
 *   out[e][c][n][j] = scales[e][n][4c + j] for 4c + j < K/32, else 0
 *   (c < ceil(K/128), j < 4)
 * i.e. the four e8m0 group scales of each 128-deep chunk of each weight row,
 * rows of one chunk contiguous.  scales uint8 [E][N][K/32] (the moe_wq_t MXFP4
 * layout); out uint8 [E][ceil(K/128)][N][4], a separate buffer, 16-byte
 * aligned; K % 32 == 0.  Pass as moe_wq_t.scales_kc. */
moe_status_t moe_mxfp4_scales_by_chunk(const uint8_t* scales, int E, int N, int K, uint8_t* out,
                                       moe_stream_t stream);

/* Gather of GEMM input rows through an act-order permutation, one row per
 * flat slot f < size_m*top_k, permuted by the slot's own expert:
 *   dst[f][k] = src[f / top_k][k_perm[e][k]],  e = topk_ids[f]
 * Rows of slots whose expert is outside [0, E) are left untouched (moe_align
 * gives them no block).  k_perm values outside [0, K) read channel K-1.
 *   src  bf16 [size_m][K];  dst  bf16 [size_m*top_k][K]
 * dst may equal src when top_k is 1 (each row is read whole before it is
 * written); other overlaps are not allowed.  K a multiple of 8, K <= 8192;
 * src, dst and k_perm 16-byte aligned. */
moe_status_t moe_permute_slots(const uint16_t* src, int size_m, int top_k, int K, int E,
                               const int32_t* k_perm, const int32_t* topk_ids, uint16_t* dst,
                               moe_stream_t stream);

/* The block_m moe_forward uses for T tokens, from the average number of slots
 * per expert a = T*top_k/E: 16 for a <= 8 (the decode kernels), 64 for
 * a <= 56, else 128 (the streaming kernel); callers that run the steps one by
 * one can use it to get the same tiling. */
int moe_forward_block_m(int T, int top_k, int E);

/* Bytes of scratch moe_forward needs (routing results, align metadata and
 * the two intermediates act [T*top_k][inter] and y [T*top_k][hidden] in bf16). */
size_t moe_forward_workspace_bytes(int T, int E, int top_k, int hidden, int inter);

/* The whole layer: route -> align -> gemm1 -> gemm2 -> sum over each token's
 * top_k rows (fp32, j ascending, one bf16 rounding).
 *   x          bf16 [T][hidden]
 *   logits     fp32 [T][E]
 *   w13        N = 2*inter (SWIGLUOAI) or inter (RELU2), K = hidden
 *   w2         N = hidden, K = inter
 *   w13/w2 k_perm (act-order, optional): GEMM1 then reads one gathered
 *              copy of x per slot (placed in the workspace's y region) and
 *              GEMM2's input rows are permuted in place before it runs
 *   mul_topk_weights  0: routing weights not applied; 1: each GEMM2 output row
 *              times its own weight (mul_topk_weights=True on the pages); 2: each
 *              GEMM1 input row times its weight instead (apply_router_weight_on_input;
 *              top_k must be 1, else MOE_ERR_SHAPE)
 *   workspace  device scratch of at least moe_forward_workspace_bytes(), 256-byte aligned
 *   out        bf16 [T][hidden] (the unpadded width)
 * block_m is chosen by the library from T*top_k/E. */
moe_status_t moe_forward(const uint16_t* x, const float* logits, int T, int E, int top_k,
                         int hidden, int inter, moe_route_t kind, const float* expert_bias,
                         int renormalize, const moe_wq_t* w13, const moe_wq_t* w2,
                         moe_act_t act, float alpha, float beta, float limit,
                         int mul_topk_weights, void* workspace, size_t workspace_bytes,
                         uint16_t* out, moe_stream_t stream);

/* Size of the fixed scratch of moe_forward_noalloc, per GPU (64 MiB). */
#define MOE_FORWARD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid it.  The
 * workspace is a fixed array in the library, MOE_FORWARD_NOALLOC_SCRATCH_BYTES
 * per GPU, held by every GPU the library runs on until the process ends; the
 * first call on a device looks up that device's copy (hipGetSymbolAddress) and
 * keeps its address.  Calls whose moe_forward_workspace_bytes() exceeds the
 * scratch return MOE_ERR_TOO_LARGE before anything is enqueued (for the
 * gpt-oss-20b shape, E=32 top-4 2880/2880, up to about 1450 tokens).  The
 * call allocates nothing; every call on one GPU uses that GPU's one array, so
 * calls that overlap on one GPU (other streams, other threads) race: order
 * them.  The caller still passes x, logits and out; everything else is as
 * moe_forward (kernel choice automatic). */
moe_status_t moe_forward_noalloc(const uint16_t* x, const float* logits, int T, int E, int top_k,
                                 int hidden, int inter, moe_route_t kind, const float* expert_bias,
                                 int renormalize, const moe_wq_t* w13, const moe_wq_t* w2,
                                 moe_act_t act, float alpha, float beta, float limit,
                                 int mul_topk_weights, uint16_t* out, moe_stream_t stream);

/* moe_forward with the kernel for 16/32-row blocks chosen by the caller
 * (moe_kernel_t), for both GEMMs. */
moe_status_t moe_forward_ex(const uint16_t* x, const float* logits, int T, int E, int top_k,
                            int hidden, int inter, moe_route_t kind, const float* expert_bias,
                            int renormalize, const moe_wq_t* w13, const moe_wq_t* w2,
                            moe_act_t act, float alpha, float beta, float limit,
                            int mul_topk_weights, void* workspace, size_t workspace_bytes,
                            uint16_t* out, moe_kernel_t kernel, moe_stream_t stream);

/* ---- MXFP8 activations (MXFP4 weights x MXFP8 activations) ----
 * The variant of the layer with MXFP8 activations ("gpt-oss-120b MXFP4 +
 * --enable-expert-parallel crashes", sections "Actual behavior" and "Why the
 * mxfp8 workaround is not a fix": the activation option switches the MoE to
 * MXFP8 activations).  Encoding (OCP microscaling): per block of 32
 * consecutive values of a row, shared e8m0 exponent floor(log2(amax)) - 8,
 * elements value / 2^exponent rounded to the nearest e4m3fn value (ties to
 * even, saturating at 448); an all-zero block has exponent byte 0; a block
 * with a NaN or an infinity has exponent byte 0xFF and NaN elements.
 * Operand layout: codes uint8 [rows][lda], lda = K rounded up to 128, zero
 * past K; scales uint8 [rows][lds], lds = K/32 rounded up to 16, zero past
 * K/32. */

/* Quantise bf16 rows [rows][K] (K % 32 == 0).  Any of codes, scales and
 * dequant may be NULL (not all three): dequant receives the MXFP8 values as
 * bf16 [rows][K] (exact except below 2^-133) and may be x itself. */
moe_status_t moe_mxfp8_quantize(const uint16_t* x, int rows, int K, uint8_t* codes, uint8_t* scales,
                                uint16_t* dequant, moe_stream_t stream);

/* moe_w4a16_gemm1 with the input rows in MXFP8 ([size_m] rows in the layout
 * above) and MXFP4 weights, on the MX-scaled matrix cores (e4m3 x e2m1 with
 * both e8m0 scales applied per 32-deep block, fp32 accumulate).  block_m must
 * be 64 or 128.  With the weight scales by K chunk (scales_kc) both scale
 * tiles stream with the K chunks and any K is taken; otherwise both must fit
 * the kernel's 56 KB of resident LDS (256*K/32 + block_m*lds bytes, each
 * rounded up to 1 KB; K <= ~4600), else MOE_ERR_UNSUPPORTED.  No routing
 * weight on the input. */
moe_status_t moe_mx_gemm1(const uint8_t* x_codes, const uint8_t* x_scales, int size_m, int top_k,
                          int K, int N, int E, const moe_wq_t* w13, moe_act_t act, float alpha,
                          float beta, float limit, const int32_t* sorted_ids,
                          const int32_t* expert_ids, const int32_t* num_post_pad, int block_m,
                          uint16_t* out, moe_stream_t stream);

/* moe_w4a16_gemm2 with MXFP8 input rows (one per flat slot); limits as
 * moe_mx_gemm1. */
moe_status_t moe_mx_gemm2(const uint8_t* a_codes, const uint8_t* a_scales, int size_m, int K, int N,
                          int E, const moe_wq_t* w2, const float* topk_w, int mul_topk_weights,
                          const int32_t* sorted_ids, const int32_t* expert_ids,
                          const int32_t* num_post_pad, int block_m, uint16_t* y,
                          moe_stream_t stream);

/* Workspace of moe_forward_mxfp8: that of moe_forward plus the MXFP8 copies
 * of x and of the activation. */
size_t moe_forward_mxfp8_workspace_bytes(int T, int E, int top_k, int hidden, int inter);

/* moe_forward with MXFP8 activations: x is quantised to MXFP8 before GEMM1,
 * GEMM1's bf16 output before GEMM2; both weight families must be MXFP4
 * (else MOE_ERR_UNSUPPORTED); mul_topk_weights 0 or 1; no k_perm.  Blocks of
 * 64/128 rows run the MX-scaled kernels; smaller blocks (few tokens per
 * expert) feed the MXFP8 values, dequantised to bf16 exactly, to the bf16
 * kernels -- the same products, summed in fp32. */
moe_status_t moe_forward_mxfp8(const uint16_t* x, const float* logits, int T, int E, int top_k,
                               int hidden, int inter, moe_route_t kind, const float* expert_bias,
                               int renormalize, const moe_wq_t* w13, const moe_wq_t* w2,
                               moe_act_t act, float alpha, float beta, float limit,
                               int mul_topk_weights, void* workspace, size_t workspace_bytes,
                               uint16_t* out, moe_stream_t stream);

/* Static description of a status code. */
const char* moe_status_str(moe_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
