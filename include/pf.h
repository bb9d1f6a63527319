/*
 * pf.h — C ABI of libpf: PackForcing per-block context attention on MI355X (gfx950).
 *
 * The current block's queries attend over a bounded three-partition KV cache
 *   C = C_sink || C_mid || C_rc
 * [PackForcing digest (paper.rainbus.top), 方法步骤详情 (5); PackForcing arXiv
 * HTML, "Bounded Attention Context"]. The sink and recent/current partitions are
 * full resolution; the mid partition is the top-k of a pool of compressed blocks,
 * chosen by query-key affinity [digest, 方法步骤详情 (3); arXiv HTML, "Compressed
 * Mid Tokens"], whose keys are re-aligned by a temporal-only RoPE rotation
 * [digest, 方法步骤详情 (4); arXiv HTML, "Incremental RoPE adjustment"].
 *
 * Conventions shared by every call:
 *  - K, V, Q and O are bfloat16, passed as raw 16-bit patterns (pf_bf16).
 *  - Layout is row-major [rows][n_heads][128]: one row per token, row stride
 *    n_heads*128 elements. The head dimension is fixed at 128
 *    (44 temporal + 42 height + 42 width RoPE dims [digest, 前置知识 RoPE]).
 *  - A pool of compressed blocks is [n_blocks*n_c][n_heads][128]; block j owns
 *    rows j*n_c .. j*n_c + n_c - 1.
 *  - Every data pointer is a DEVICE pointer and must be 16-byte aligned.
 *    Ownership stays with the caller; libpf allocates nothing and keeps no
 *    device state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work and return; there is no host synchronisation.
 *  - Arguments are validated on the host before anything is enqueued. On error
 *    nothing is enqueued, the call returns a pf_status other than PF_OK, and
 *    pf_last_error_message() describes it. Faults inside a kernel surface at
 *    the caller's next synchronisation.
 *  - Index arrays that live on the device (ids, block lists) cannot be checked
 *    on the host; the kernels skip out-of-range entries instead of reading out
 *    of bounds, as documented per call.
 *  - Calls on disjoint buffers may run concurrently. pf_rope_shift and
 *    pf_selection_deltas write in place: order them against readers of the same
 *    buffers on the caller's streams.
 */
#ifndef PF_H_
#define PF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PF_ABI_VERSION 1
#define PF_HEAD_DIM 128
#define PF_TEMPORAL_DIMS 44
#define PF_MAX_HEADS 32
#define PF_MAX_BLOCKS 4096   /* pool blocks scored by pf_score_select */
#define PF_MAX_TOPK 256      /* top_k of pf_score_select */
#define PF_MAX_SELECTED 1024 /* n_sel of pf_partition_attn */
#define PF_MAX_BATCH 65535   /* n_batch of the _batched calls */
#define PF_HR_STAGES 4       /* strided stages of the HR branch before the projection */

typedef uint16_t pf_bf16;

typedef enum pf_status {
  PF_OK = 0,
  PF_ERR_NULL = 1,        /* a required pointer is NULL */
  PF_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
  PF_ERR_UNSUPPORTED = 3, /* a size beyond the limits above */
  PF_ERR_MISALIGNED = 4,  /* a data pointer is not 16-byte aligned */
  PF_ERR_RANGE = 5,       /* a count outside its allowed range (top_k, n_sel, ...) */
  PF_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the query function says */
  PF_ERR_HIP = 7          /* the HIP runtime refused a launch; the message names the error */
} pf_status;

/* PF_ABI_VERSION of the loaded library. */
int pf_abi_version(void);

/* Static name of a status code ("PF_OK", ...); "PF_UNKNOWN" for other values. */
const char* pf_status_name(int status);

/* Message of the last failed call on this host thread (empty after a success).
 * The string is owned by libpf and valid until the thread's next pf_* call. */
const char* pf_last_error_message(void);

/* ------------------------------------------------------------------------- *
 * Dynamic context selection
 * [PackForcing digest, 方法步骤详情 (3): top-K over the compressed mid blocks by
 *  query-key affinity phi_j = sum_i q_i^T k_j / sqrt(d), N_top = 16;
 *  arXiv HTML, "Compressed Mid Tokens" and "Implementation Details"]
 *
 * The pages leave the pooling open; this library computes, per pool block j,
 *   s_j = (1/H) sum_h < mean_i Q[i,h,:], mean_{r<n_c} K[j*n_c + r,h,:] > / sqrt(128)
 * which ranks blocks exactly as the double sum over queries and block keys does.
 * The k largest s_j are selected, ties going to the lower block index, and
 * written to ids_out[0..top_k) in ascending block order.
 *
 *   q           [n_q][n_heads][128] bf16 — the current block's queries.
 *   pool_k      [n_blocks*n_c][n_heads][128] bf16 — compressed mid keys.
 *   ids_out     int32[top_k] (device) — selected block ids, ascending.
 *   scores_out  float[n_blocks] (device) or NULL — s_j in fp32.
 *   workspace   device scratch of at least pf_score_select_workspace_bytes(...)
 *               bytes; its contents need no initialisation.
 * Limits: 1 <= n_heads <= PF_MAX_HEADS, 1 <= n_blocks <= PF_MAX_BLOCKS,
 *         1 <= top_k <= min(n_blocks, PF_MAX_TOPK), n_q >= 1, n_c >= 1.
 * Arithmetic: bf16 inputs, fp32 sums in a fixed order (repeatable bit for bit).
 * ------------------------------------------------------------------------- */
size_t pf_score_select_workspace_bytes(int64_t n_q, int n_heads, int n_blocks, int n_c);

pf_status pf_score_select(const pf_bf16* q, int64_t n_q, int n_heads,
                          const pf_bf16* pool_k, int n_blocks, int n_c, int top_k,
                          int32_t* ids_out, float* scores_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Sub-sampled scoring: the same score computed from query rows 0, q_step,
 * 2*q_step, ... and heads 0, head_step, 2*head_step, ... only. The pages run
 * selection only at each block's first denoising step [digest, 方法步骤详情 (3)]
 * and speed it up further by scoring with a subsample of the query tokens and
 * half of the attention heads [digest, 局限与改进]; q_step = head_step = 1 is
 * pf_score_select. The means run over the rows and heads that are used.
 * Limits as pf_score_select, plus q_step >= 1 and 1 <= head_step <= n_heads. */
size_t pf_score_select_sub_workspace_bytes(int64_t n_q, int n_heads, int q_step, int head_step, int n_blocks,
                                           int n_c);

pf_status pf_score_select_sub(const pf_bf16* q, int64_t n_q, int n_heads, int q_step, int head_step,
                              const pf_bf16* pool_k, int n_blocks, int n_c, int top_k,
                              int32_t* ids_out, float* scores_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Batched form: n_batch independent caches (for example the same layer of
 * several videos, or layers whose queries are already known) in one launch
 * sequence. Cache b reads q + b*q_batch_stride and pool_k + b*pool_batch_stride
 * (strides in elements, multiples of 8, each at least one cache's rows; ignored
 * when n_batch == 1) and writes ids_out[b*top_k ..] and scores_out[b*n_blocks ..].
 * Every cache gets bit for bit the result of a single call on it.
 * Limits as above, plus 1 <= n_batch <= PF_MAX_BATCH. */
size_t pf_score_select_batched_workspace_bytes(int64_t n_q, int n_heads, int n_blocks, int n_c, int n_batch);

pf_status pf_score_select_batched(const pf_bf16* q, int64_t q_batch_stride, int64_t n_q, int n_heads,
                                  const pf_bf16* pool_k, int64_t pool_batch_stride, int n_blocks, int n_c,
                                  int top_k, int n_batch, int32_t* ids_out, float* scores_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Random selection, the pages' weakest baseline against dynamic selection
 * [digest, 实验结果 (dynamic vs FIFO vs random); arXiv HTML, "FIFO vs. Dynamic
 * Context Selection"]. The pages name no generator; this library draws k
 * distinct blocks with Floyd's sampling algorithm (Bentley and Floyd, CACM
 * 1987): step r (r = 0..top_k-1) takes j = n_blocks - top_k + r and
 * t = floor(hi32(x_{r+1}) * (j + 1) / 2^32), keeping t unless it was kept
 * already, else j. x_i is draw i of a counter-based SplitMix64 stream
 * (Steele, Lea and Flood, OOPSLA 2014):
 *   x_i = mix(seed + (c * 2^32 + i) * 0x9E3779B97F4A7C15)   (mod 2^64)
 * with c = counter + b for cache b of the batch. ids_out[b*top_k ..] gets the
 * ids in ascending order. The FIFO baseline needs no kernel: it keeps blocks
 * n_blocks - top_k .. n_blocks - 1.
 * Limits: 1 <= n_blocks <= PF_MAX_BLOCKS, 1 <= top_k <= min(n_blocks,
 * PF_MAX_TOPK), 1 <= n_batch <= PF_MAX_BATCH. */
pf_status pf_select_random(int n_blocks, int top_k, uint64_t seed, uint64_t counter, int n_batch,
                           int32_t* ids_out, void* stream);

/* ------------------------------------------------------------------------- *
 * Placement of the selected blocks -> per-block temporal shift delta
 * [PackForcing arXiv HTML, "The Position Misalignment Problem" and
 *  "Incremental RoPE adjustment"; openbayes summary, "Method": the remaining
 *  tokens are shifted to continuous indices]
 *
 * pos_tags[m] is the first latent frame that pool block m's keys currently
 * encode. The selected blocks ids[0] < ... < ids[top_k-1] are laid end to end
 * just before the recent block, whose first frame is recent_first_frame:
 *   target_r   = recent_first_frame - (top_k - r) * block_frames
 *   deltas[r]  = target_r - pos_tags[ids[r]]      (signed, latent frames)
 *   pos_tags[ids[r]] = target_r                   (updated in place)
 *
 *   ids         int32[top_k] (device), ascending and distinct.
 *   pos_tags    int32[n_blocks] (device), read and updated.
 *   deltas_out  int32[top_k] (device).
 * An id outside [0, n_blocks) gets delta 0 and leaves pos_tags untouched.
 * Limits: 1 <= top_k <= PF_MAX_TOPK, top_k <= n_blocks, block_frames >= 1.
 * ------------------------------------------------------------------------- */
pf_status pf_selection_deltas(const int32_t* ids, int top_k, int32_t* pos_tags, int n_blocks,
                              int32_t recent_first_frame, int32_t block_frames,
                              int32_t* deltas_out, void* stream);

/* Batched form: cache b uses ids[b*top_k ..], pos_tags[b*n_blocks ..] and
 * deltas_out[b*top_k ..]; all caches share top_k, n_blocks and the frames.
 * Limits as above, plus 1 <= n_batch <= PF_MAX_BATCH. */
pf_status pf_selection_deltas_batched(const int32_t* ids, int top_k, int32_t* pos_tags, int n_blocks,
                                      int32_t recent_first_frame, int32_t block_frames, int n_batch,
                                      int32_t* deltas_out, void* stream);

/* ------------------------------------------------------------------------- *
 * Selection and placement in one call
 * [the two passages above: digest 方法步骤详情 (3), arXiv HTML "Compressed Mid
 *  Tokens"; arXiv HTML "The Position Misalignment Problem", "Incremental RoPE
 *  adjustment"]
 *
 * Same results as pf_score_select followed by pf_selection_deltas with the same
 * arguments (ids, deltas, updated pos_tags and scores are bit-identical), with
 * one launch fewer: the workgroup that selects a cache's top-k also places
 * them. Workspace: pf_score_select_workspace_bytes
 * (batched: pf_score_select_batched_workspace_bytes); concurrent calls must not
 * share a workspace. Arguments and limits as for the two calls; pos_tags and
 * deltas_out must not be NULL.
 * ------------------------------------------------------------------------- */
pf_status pf_select_place(const pf_bf16* q, int64_t n_q, int n_heads, const pf_bf16* pool_k, int n_blocks,
                          int n_c, int top_k, int32_t* pos_tags, int32_t recent_first_frame,
                          int32_t block_frames, int32_t* ids_out, int32_t* deltas_out, float* scores_out,
                          void* workspace, size_t workspace_bytes, void* stream);

pf_status pf_select_place_batched(const pf_bf16* q, int64_t q_batch_stride, int64_t n_q, int n_heads,
                                  const pf_bf16* pool_k, int64_t pool_batch_stride, int n_blocks, int n_c,
                                  int top_k, int32_t* pos_tags, int32_t recent_first_frame, int32_t block_frames,
                                  int n_batch, int32_t* ids_out, int32_t* deltas_out, float* scores_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * Incremental temporal RoPE shift, in place
 * [PackForcing digest, 前置知识 RoPE (k^(p) = k_raw e^{i theta p}, and
 *  e^{i theta p} e^{i theta delta} = e^{i theta (p+delta)}) and 方法步骤详情 (4);
 *  arXiv HTML, "Incremental RoPE adjustment": k' = k e^{i(theta_t delta, 1_h, 1_w)}]
 *
 * For every row of each listed block and every head, the 22 temporal complex
 * pairs (dims 2j, 2j+1 for j < 22) are multiplied by e^{+i theta_j delta} with
 * theta_j = rope_base^(-2j/44); dims 44..127 keep their bits (dims 44..63 are
 * stored back unchanged, so that whole 128-byte lines are written, and no
 * other writer may update them concurrently), V is never touched, and a zero delta leaves the
 * block's bits unchanged. The angle, its
 * cos/sin and the rotation are fp64; the result is rounded once to bf16
 * (round to nearest even).
 *
 *   k           [n_blocks*rows_per_block][n_heads][128] bf16, updated in place.
 *   block_ids   int32[n_shift] (device) — blocks to shift; NULL means blocks
 *               0..n_shift-1 (e.g. a contiguous sink slab as one block).
 *   deltas      int32[n_shift] (device) — shift of each listed block, frames.
 * Entries whose block id is outside [0, n_blocks) are skipped. Each block may
 * be listed at most once per call: two entries for one block rotate the same
 * keys concurrently and leave them undefined.
 * Limits: 1 <= n_heads <= PF_MAX_HEADS, rows_per_block >= 1, n_shift >= 0
 *         (0 enqueues nothing), n_shift <= n_blocks when block_ids is NULL,
 *         rope_base > 1.
 * ------------------------------------------------------------------------- */
pf_status pf_rope_shift(pf_bf16* k, int n_heads, int64_t rows_per_block, int64_t n_blocks,
                        const int32_t* block_ids, const int32_t* deltas, int n_shift,
                        double rope_base, void* stream);

/* Batched form: cache b shifts k + b*k_batch_stride (elements, a multiple of 8,
 * at least one cache's n_blocks*rows_per_block rows; ignored when n_batch == 1)
 * using block_ids[b*n_shift ..] (or blocks 0..n_shift-1 when NULL) and
 * deltas[b*n_shift ..]. Limits as above, plus 1 <= n_batch <= PF_MAX_BATCH. */
pf_status pf_rope_shift_batched(pf_bf16* k, int64_t k_batch_stride, int n_heads, int64_t rows_per_block,
                                int64_t n_blocks, const int32_t* block_ids, const int32_t* deltas, int n_shift,
                                int n_batch, double rope_base, void* stream);

/* ------------------------------------------------------------------------- *
 * Partition attention over the bounded context
 * [PackForcing digest, 前置知识 KV缓存 (Attn(Q_i, C) = softmax(Q_i K^T / sqrt(d_h)) V)
 *  and 方法步骤详情 (5); arXiv HTML, "Bounded Attention Context"]
 *
 *   O[i,h,:] = sum_t softmax_t(scale * Q[i,h,:] . K[t,h,:]) V[t,h,:]
 * with one softmax over the virtual concatenation
 *   K = sink || pool[mid_ids[0]] || ... || pool[mid_ids[n_sel-1]] || recent || cur
 * (V follows the same row map). The selected pool blocks are read in place
 * through mid_ids, never copied. There is no mask: the current block attends
 * to itself in full.
 *
 *   q                    [n_q][n_heads][128] bf16.
 *   sink_k/v  [n_sink]   recent_k/v [n_recent]   cur_k/v [n_cur] — row counts
 *                        may be 0 (then the pointers may be NULL).
 *   pool_k/v             [n_blocks*n_c][n_heads][128]; read only if n_sel > 0.
 *   mid_ids              int32[n_sel] (device). An id outside [0, n_blocks)
 *                        contributes no keys (its rows are masked out).
 *   scale                softmax scale; <= 0 selects 1/sqrt(128).
 *   o                    [n_q][n_heads][128] bf16 output (round to nearest even).
 *   lse                  float[n_heads][n_q] natural-log sum-exp of the scaled
 *                        scores, or NULL.
 *   workspace            device scratch of pf_partition_attn_workspace_bytes(...)
 *                        bytes (may be NULL when that is 0).
 * Limits: 1 <= n_heads <= PF_MAX_HEADS, n_q >= 1, 0 <= n_sel <= PF_MAX_SELECTED,
 *         n_sel <= n_blocks, the total key count must be >= 1 and < 2^31,
 *         and the pool's K (and V) must span less than 2 GiB, because its
 *         rows, scattered by mid_ids, are addressed with 32-bit byte offsets
 *         from the pool's start; PF_ERR_UNSUPPORTED otherwise. The sink,
 *         recent and current partitions may be larger: their tiles are
 *         addressed from each tile's own first row.
 * Arithmetic: bf16 MFMA products with fp32 accumulation; the online softmax is
 * fp32; probabilities are rounded to bf16 before the P.V product.
 * ------------------------------------------------------------------------- */
size_t pf_partition_attn_workspace_bytes(int64_t n_q, int n_heads, int64_t n_keys);

pf_status pf_partition_attn(const pf_bf16* q, int64_t n_q, int n_heads,
                            const pf_bf16* sink_k, const pf_bf16* sink_v, int64_t n_sink,
                            const pf_bf16* pool_k, const pf_bf16* pool_v, int n_blocks, int n_c,
                            const int32_t* mid_ids, int n_sel,
                            const pf_bf16* recent_k, const pf_bf16* recent_v, int64_t n_recent,
                            const pf_bf16* cur_k, const pf_bf16* cur_v, int64_t n_cur,
                            float scale, pf_bf16* o, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* pf_partition_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results as pf_partition_attn, with no
 * workspace argument. The partial results that a workspace would hold go to a
 * fixed 40 MiB device array inside the library, one per GPU, kept until the
 * process ends; the call itself allocates nothing. Its device address is
 * looked up once per device, on the first call with that device current.
 * Shapes whose partials exceed the array (the size
 * pf_partition_attn_workspace_bytes reports, at most 34 MB on a 256-CU
 * MI355X) return PF_ERR_UNSUPPORTED before anything is enqueued. The array is
 * shared by every call on a GPU and keeps the last call's contents (no call
 * reads a partial it did not write first): calls that overlap on one GPU,
 * on any streams, race and must be ordered by the caller. Other arguments,
 * limits and errors as pf_partition_attn. */
pf_status pf_partition_attn_noalloc(const pf_bf16* q, int64_t n_q, int n_heads,
                                    const pf_bf16* sink_k, const pf_bf16* sink_v, int64_t n_sink,
                                    const pf_bf16* pool_k, const pf_bf16* pool_v, int n_blocks, int n_c,
                                    const int32_t* mid_ids, int n_sel,
                                    const pf_bf16* recent_k, const pf_bf16* recent_v, int64_t n_recent,
                                    const pf_bf16* cur_k, const pf_bf16* cur_v, int64_t n_cur,
                                    float scale, pf_bf16* o, float* lse, void* stream);

/* ------------------------------------------------------------------------- *
 * Roll-in of a compressed block into the mid pool
 * [PackForcing arXiv HTML, "Dual-Resolution Shifting Mechanism": when a block
 *  leaves the recent window its reduced-resolution backup joins the mid buffer]
 *
 * Copies block_k/block_v ([n_c][n_heads][128]) into pool rows
 * slot*n_c .. slot*n_c + n_c - 1 and sets pos_tags[slot] = first_frame (the
 * frame the block's keys start at; pos_tags may be NULL). The pool must have
 * room for the slot; nothing else is touched, so the call can run on a stream
 * of its own while attention reads the other slots.
 * Batched form: cache b uses pool_k/v + b*pool_batch_stride, pos_tags +
 * b*tags_batch_stride and block_k/v + b*block_batch_stride (ignored when
 * n_batch == 1). Limits: 1 <= n_heads <= PF_MAX_HEADS, n_c >= 1, slot >= 0,
 * 1 <= n_batch <= PF_MAX_BATCH.
 * ------------------------------------------------------------------------- */
pf_status pf_rollin(pf_bf16* pool_k, pf_bf16* pool_v, int32_t* pos_tags, int n_heads, int n_c, int slot,
                    const pf_bf16* block_k, const pf_bf16* block_v, int32_t first_frame, void* stream);

pf_status pf_rollin_batched(pf_bf16* pool_k, pf_bf16* pool_v, int64_t pool_batch_stride,
                            int32_t* pos_tags, int tags_batch_stride, int n_heads, int n_c, int slot,
                            const pf_bf16* block_k, const pf_bf16* block_v, int64_t block_batch_stride,
                            int32_t first_frame, int n_batch, void* stream);

/* ------------------------------------------------------------------------- *
 * HR branch of the compressor
 * [PackForcing arXiv HTML, "HR Branch: Progressive 3D Convolution": strided 3D
 *  convolutions with SiLU halve time once and space three times (2x8x8 =
 *  128x volume reduction), then a 1x1x1 projection reaches the hidden width;
 *  "Feature Fusion": N_c = floor(T/2) floor(H/8) floor(W/8) tokens;
 *  digest (paper.rainbus.top), 前置知识 3D卷积]
 *
 * pf_hr_conv: one strided 3D convolution whose kernel equals its stride (no
 * padding; each output dimension is floor(input / kernel)), plus bias and,
 * when act != 0, SiLU:
 *   y[b][t][h][w][n] = act(bias[n] + sum_{dt,dh,dw,c} w[n][dt][dh][dw][c] *
 *                      x[b][kt*t+dt][kh*h+dh][kw*w+dw][c])
 * x: [n_batch][T][H][W][c_in] bf16 (channels last); w: [c_out][kt][kh][kw][c_in]
 * bf16; bias: [c_out] fp32 or NULL; y: [n_batch][T/kt][H/kh][W/kw][c_out] bf16
 * (round to nearest even of the fp32 result). Accumulation is fp32 in a fixed
 * order, so results are bit-reproducible. All device pointers, owned by the
 * caller; x, w, y and workspace 16-byte aligned, bias 4-byte aligned.
 * Deep stages with few output positions split the reduction and need a
 * workspace of pf_hr_conv_workspace_bytes(...) bytes (0: none needed; the
 * size depends on the device's CU count).
 * Limits: n_batch >= 1; 1 <= kt, kh, kw with kt*kh*kw <= 64 and the input at
 * least one kernel in every dimension; c_in and c_out multiples of 16 in
 * [16, 65536]. Errors are returned before anything is enqueued.
 *
 * pf_hr_branch: the whole branch on a latent block z [n_batch][T][H][W][c_in]:
 * stage 0 has kernel 2x1x1, stages 1..3 kernel 1x2x2, each with SiLU and
 * widths[s] output channels, then the linear projection proj_w
 * [hidden][widths[3]] (+ proj_b) to out [n_batch][N_c][hidden] with
 * N_c = (T/2)(H/8)(W/8) tokens numbered t-major. stage_w, stage_b and widths
 * are HOST arrays of PF_HR_STAGES entries (the weight and bias pointers they
 * hold are device pointers; stage_b entries may be NULL). The intermediate
 * activations live in the caller's workspace of
 * pf_hr_branch_workspace_bytes(...) bytes. Limits: T >= 2, H >= 8, W >= 8 and
 * those of pf_hr_conv for every stage.
 * ------------------------------------------------------------------------- */
size_t pf_hr_conv_workspace_bytes(int n_batch, int T, int H, int W, int c_in, int kt, int kh, int kw, int c_out);

pf_status pf_hr_conv(const pf_bf16* x, int n_batch, int T, int H, int W, int c_in, int kt, int kh, int kw,
                     const pf_bf16* w, const float* bias, int c_out, int act, pf_bf16* y,
                     void* workspace, size_t workspace_bytes, void* stream);

size_t pf_hr_branch_workspace_bytes(int n_batch, int T, int H, int W, int c_in, const int* widths, int hidden);

/* Tokens per block that pf_hr_branch writes for a T x H x W latent block:
 * the product of the dimensions left after the stages' kernels, which is
 * N_c = floor(T/2) floor(H/8) floor(W/8); 0 when the block is smaller than
 * 2 x 8 x 8. The caller sizes `out` as [n_batch][this][hidden]. */
int64_t pf_hr_branch_out_tokens(int T, int H, int W);

pf_status pf_hr_branch(const pf_bf16* z, int n_batch, int T, int H, int W, int c_in,
                       const pf_bf16* const* stage_w, const float* const* stage_b, const int* widths,
                       const pf_bf16* proj_w, const float* proj_b, int hidden, pf_bf16* out,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PF_H_ */
