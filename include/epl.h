/*
 * epl.h -- C ABI of libepl.so: MoE expert-parallel token layout, dispatch
 * into an expert-contiguous ragged buffer, and weighted combine, for one
 * rank on an MI355X (gfx950) GPU.
 *
 * The calls follow the problem statement of the pages:
 *   1. layout   -- per-expert / per-rank token counts and the token->rank
 *                  mask, computed from topk_idx on the GPU
 *                  ("[MoE] Deepseek的All-to-all通信: DeepEP代码解读", section
 *                  Dispatch, get_dispatch_layout);
 *   2. scan     -- exclusive prefix sum of the counts: where each expert's
 *                  block starts and the exact buffer size
 *                  ("高性能专家并行（EP）内核解剖学解读", high-throughput part,
 *                  subsections 3 and 5);
 *   3. scatter  -- copy each routed token row (and its scale row) into its
 *                  expert's block, writing m_indices and output_index
 *                  ("参考sglang代码，重构vllm021中EP高吞吐代码，消除空泡问题",
 *                  sections 2.2 and 3.3, ep_scatter and its outputs);
 *   4. combine  -- gather the expert-output rows back into token order as a
 *                  top-k-weighted sum ("高性能专家并行（EP）内核解剖学解读",
 *                  section 任务设定与数据流: results return to where the
 *                  tokens came from; sglang section 2.2 keeps topk ids,
 *                  weights and output_index for that step).
 * epl_dispatch runs 1-3 in one call with no host round-trip.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are DEVICE pointers to row-major, densely packed
 *   arrays, except `total_host` (pinned host memory, see epl_scan).
 * - The caller owns every buffer, including the workspace. The library
 *   allocates no memory and keeps no global state between calls, except
 *   the static workspace of epl_dispatch_static (a device array of
 *   EPL_STATIC_WORKSPACE_BYTES per GPU, part of the loaded library).
 * - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *   enqueues work on that stream; none synchronises it except epl_status.
 * - Return value: EPL_OK (0) or a negative EPL_E* code. Argument errors are
 *   detected on the host before anything is enqueued (EPL_EINVAL).
 *   Data errors that only the GPU can see (an expert id outside [-1, E), too
 *   few capacity rows, an output_index beyond the expert output) are
 *   recorded in a status word inside the workspace and returned by
 *   epl_status; the offending slot is then treated as "no selection", and
 *   nothing is ever written out of bounds.
 * - Ownership of experts by virtual ranks: rank r owns the contiguous
 *   experts [r*E/R, (r+1)*E/R); E must be a multiple of R.
 * - Row order inside an expert's block: by token, then by top-k slot. The
 *   result is therefore deterministic (bit-identical from run to run).
 * - Send side and receive side. On the send side topk_idx holds global
 *   expert ids and the layout's per-rank outputs say where tokens go. On
 *   the receive side (the batch a rank holds after the dispatch) topk_idx
 *   holds the rank's local expert ids, 0 .. E/R - 1, with -1 for the slots
 *   whose experts live on other ranks; the same calls then run with
 *   num_experts = the local expert count and num_ranks = 1, and scatter
 *   and combine touch only the local experts' rows, with no id remapping
 *   (the direct local-id path of "参考sglang代码，重构vllm021中EP高吞吐代码，
 *   消除空泡问题", section 7; DeepEP's received top-k ids, section Dispatch
 *   of "[MoE] Deepseek的All-to-all通信: DeepEP代码解读"). The combine then
 *   yields each received token's partial sum over the rank's experts.
 */
#ifndef EPL_H
#define EPL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define EPL_OK          0
#define EPL_EINVAL    (-1)  /* bad problem, NULL or misaligned pointer, bad size */
#define EPL_ERANGE    (-2)  /* device: a topk id outside [-1, E), or an
                               output_index at or beyond expert_rows */
#define EPL_ECAPACITY (-3)  /* device: routed rows exceed capacity_rows */
#define EPL_EHIP      (-4)  /* a HIP runtime call or kernel launch failed */

/* ---- combine output types ---------------------------------------------- */
#define EPL_OUT_F32   0     /* y is float32 [T, H] */
#define EPL_OUT_BF16  1     /* y is bf16 [T, H], round to nearest even of the f32 sum */

/* ---- scale formats of the FP8 calls -------------------------------------- */
#define EPL_SCALE_NONE  0   /* no scale rows                                     */
#define EPL_SCALE_F32   1   /* x_scale fp32 [T, S] -> out_scale fp32 [capacity, S]
                               (row-major, as in the bf16 calls)                  */
#define EPL_SCALE_UE8M0 2   /* x_scale int32 [T, W], W = ceil(S/4), each word four
                               packed 8-bit power-of-two exponents (moved as
                               opaque bits) -> out_scale int32 column-major
                               [W, capacity]: word j of row p at
                               out_scale[j * capacity + p], the transposed layout
                               sglang allocates for UE8M0 scales ("参考sglang代码，
                               重构vllm021中EP高吞吐代码，消除空泡问题", section 2.2) */

/* ---- problem description ----------------------------------------------- */
typedef struct epl_problem {
    int64_t num_tokens;   /* T >= 0                                           */
    int32_t num_topk;     /* K, 1 <= K <= 64                                  */
    int32_t num_experts;  /* E, 1 <= E <= 2048                                */
    int32_t num_ranks;    /* R >= 1, E % R == 0                               */
    int32_t hidden;       /* H >= 8, H % 8 == 0 (16-byte rows of bf16)        */
    int32_t scale_cols;   /* S: 0 (no scales) or H / 128 (needs H % 128 == 0) */
    int32_t expert_alignment; /* a: 0 or 1 = no padding; a > 1 (<= 65536): each
                             expert's block is padded to a multiple of a rows
                             (the grouped GEMM's block_m; DeepEP's
                             expert_alignment). Padding rows get m_indices = -1
                             and are otherwise not written.               */
    int32_t ranks_per_node; /* G: GPUs per node, for num_tokens_per_rdma_rank.
                             0 or G >= R: one node, that output is not
                             produced; 1 <= G < R: R % G == 0, rank r sits on
                             node r / G and the layout counts the tokens
                             bound for each of the R / G nodes.            */
    int32_t reserved;     /* must be 0                                        */
} epl_problem;
/* Also required: T * K + E * (a - 1) <= INT32_MAX (row indices are int32). */

/* Host-only check of a problem description. Needs no GPU. */
int epl_validate(const epl_problem *p);

/* Bytes of device workspace that the calls below need for problem `p`
 * (0 if `p` is invalid). The workspace carries the per-block counts that
 * make the row order deterministic, the per-slot ranks, the device copy of
 * the total row count and the status word. It needs no initialisation;
 * epl_layout / epl_dispatch write every byte that later calls read. Its
 * address must be 256-byte aligned. Host-only; needs no GPU.
 * The calls take the workspace as a bare pointer and cannot check its size:
 * the layout, scan and scatter calls need all epl_workspace_bytes(p) bytes
 * for the same problem (a smaller one is written past its end), while
 * epl_combine, epl_expert_scale, epl_status and epl_total touch only its
 * first 256 bytes (status word and total). The Python binding checks the
 * size before every call. */
size_t epl_workspace_bytes(const epl_problem *p);

/* Rows that always suffice for the ragged buffer of problem `p`: T * K
 * without alignment, else round_up(T * K + E * (a - 1), a) (the bound of the
 * vLLM fork's compute_aligned_M in "参考sglang代码，重构vllm021中EP高吞吐代码，
 * 消除空泡问题", section 4). -1 if `p` is invalid. Host-only. */
int64_t epl_capacity_rows(const epl_problem *p);

/* Step 1 -- layout. Reads topk_idx [T, K] int64 (-1 = no selection).
 * Writes num_tokens_per_expert [E] int32 (routed slots per expert),
 * num_tokens_per_rank [R] int32 (tokens sent to each rank, a token counted
 * once per rank however many of its experts live there),
 * num_tokens_per_rdma_rank [R / G] int32 when the problem spans several
 * nodes (1 <= ranks_per_node = G < R): tokens sent to each node's RDMA
 * rank, a token counted once per node however many of the node's ranks it
 * goes to ("[MoE] Deepseek的All-to-all通信: DeepEP代码解读", section Dispatch,
 * get_dispatch_layout's second output; NULL is accepted, and the pointer
 * ignored, when the problem fits one node), and is_token_in_rank [T, R]
 * uint8 (1 if any valid slot of the token goes to the rank, else 0). Also
 * fills the workspace for epl_scatter and resets the status word (bit for
 * out-of-range ids set if any was seen; such an id counts as -1). */
int epl_layout(const epl_problem *p, const int64_t *topk_idx,
               int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
               int32_t *num_tokens_per_rdma_rank, uint8_t *is_token_in_rank,
               void *workspace, void *stream);

/* Step 2 -- scan. expert_start_loc[e] = sum of block sizes of experts e' < e
 * (exclusive, expert_start_loc[0] = 0), where an expert's block size is its
 * count, rounded up to a multiple of the expert alignment when a > 1 ("高性能
 * 专家并行（EP）内核解剖学解读", high-throughput part, subsections 3 and 5).
 * The total N = sum of all block sizes (the ragged buffer's row count) is
 * stored in the workspace and, if `total_host` is not NULL, copied
 * asynchronously to *total_host, which must be pinned host memory
 * (hipHostMalloc / torch pin_memory). *total_host is valid once the stream
 * has reached this point (after any later synchronisation of the stream). */
int epl_scan(const epl_problem *p, const int32_t *num_tokens_per_expert,
             int32_t *expert_start_loc, int32_t *total_host,
             void *workspace, void *stream);

/* Step 3 -- scatter. For every valid slot (t, k) with expert e:
 *   row = expert_start_loc[e] + (number of valid slots of expert e that come
 *         before (t, k) in (token, k) order)
 *   out[row, :] = x[t, :] (bit copy, H bf16 values), out_scale[row, :] =
 *   x_scale[t, :] (S floats) when S > 0, m_indices[row] = e,
 *   output_index[t, k] = row. Slots with -1 get output_index = -1. With an
 *   expert alignment a > 1 the rows between an expert's last row and the
 *   end of its padded block get m_indices = -1 (nothing else is written).
 * `out` / `out_scale` / `m_indices` have room for `capacity_rows` rows
 * (capacity_rows >= N; epl_capacity_rows() always suffices); rows >= N are
 * not written.
 * If N > capacity_rows the rows past the capacity are skipped and the
 * status word records EPL_ECAPACITY: a slot whose row would fall at or past
 * capacity_rows (or before row 0, with a caller-made expert_start_loc) is
 * not placed -- nothing is written for it and its output_index is -1, the
 * marker of an unplaced slot ("参考sglang代码，重构vllm021中EP高吞吐代码，
 * 消除空泡问题", section 3.3) -- and alignment padding rows outside the
 * buffer are skipped likewise. Requires that epl_layout and then
 * epl_scan (with the counts epl_layout produced) ran on the same
 * workspace and stream. x / out: 16-byte aligned; x_scale / out_scale may be
 * NULL iff S == 0. */
int epl_scatter(const epl_problem *p, const uint16_t *x, const float *x_scale,
                const int64_t *topk_idx, const int32_t *expert_start_loc,
                void *workspace, int64_t capacity_rows,
                uint16_t *out, float *out_scale, int32_t *m_indices,
                int32_t *output_index, void *stream);

/* Steps 1-3 in one call, all on `stream`, with no host wait between them:
 * layout, scan (the total is copied to *total_host if it is not NULL) and
 * scatter, with the arguments and results described above. Decode-sized
 * batches (at most 2048 (token, k) slots) run all three steps in one launch,
 * and batches of a few thousand tokens run the scan inside the scatter
 * launch; the results, and the workspace left for later epl_scatter /
 * epl_scatter_fp8 calls, are the same. */
int epl_dispatch(const epl_problem *p, const int64_t *topk_idx,
                 const uint16_t *x, const float *x_scale, int64_t capacity_rows,
                 int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                 int32_t *num_tokens_per_rdma_rank,
                 uint8_t *is_token_in_rank, int32_t *expert_start_loc,
                 int32_t *total_host, uint16_t *out, float *out_scale,
                 int32_t *m_indices, int32_t *output_index,
                 void *workspace, void *stream);

/* epl_dispatch for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, work and results as epl_dispatch, except that there is no
 * workspace argument: the call uses a static workspace, a device array of
 * EPL_STATIC_WORKSPACE_BYTES that the library holds on each GPU it runs on
 * (one per GPU, the current device's) until the process ends, and that this
 * call neither allocates nor frees (no hipMalloc / hipFree, no allocating
 * library routine). Limit: problems whose epl_workspace_bytes exceed
 * EPL_STATIC_WORKSPACE_BYTES are rejected with EPL_EINVAL before anything
 * touches the GPU (8 MiB holds the per-slot ranks of about two million
 * (token, k) slots, e.g. 65536 tokens at top-8 with room to spare). If
 * `workspace_used` is not NULL it receives the device address of the static
 * workspace used, which the caller may pass as `workspace` to epl_status,
 * epl_total, epl_expert_scale and epl_combine like any workspace. Every call
 * on one GPU shares that GPU's static workspace and it keeps the last call's
 * contents: calls that overlap on one GPU (several streams or host threads
 * at once) race and must be ordered by the caller; the status word and
 * total read afterwards are those of the last dispatch. No part of the
 * static workspace needs to start at zero. */
#define EPL_STATIC_WORKSPACE_BYTES ((size_t)8 << 20)
int epl_dispatch_static(const epl_problem *p, const int64_t *topk_idx,
                        const uint16_t *x, const float *x_scale, int64_t capacity_rows,
                        int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                        int32_t *num_tokens_per_rdma_rank,
                        uint8_t *is_token_in_rank, int32_t *expert_start_loc,
                        int32_t *total_host, uint16_t *out, float *out_scale,
                        int32_t *m_indices, int32_t *output_index,
                        void **workspace_used, void *stream);

/* Steps 3 and 1-3 for an FP8 (e4m3) payload, as DeepEP dispatches it
 * ("[MoE] Deepseek的All-to-all通信: DeepEP代码解读", section Dispatch: x as a
 * (fp8 [T, H], fp32 [T, H/128]) tuple): rows are H bytes (requires
 * H % 16 == 0), moved bit for bit like the bf16 rows; the scale rows follow
 * in `scale_format` (EPL_SCALE_*; with a format other than NONE the problem
 * needs scale_cols = H/128 and the scale pointers must be 4-byte aligned).
 * Everything else (row placement, m_indices, output_index, alignment
 * padding, status) is as in epl_scatter / epl_dispatch. */
int epl_scatter_fp8(const epl_problem *p, const uint8_t *x, const void *x_scale,
                    int scale_format, const int64_t *topk_idx,
                    const int32_t *expert_start_loc, void *workspace, int64_t capacity_rows,
                    uint8_t *out, void *out_scale, int32_t *m_indices, int32_t *output_index,
                    void *stream);
int epl_dispatch_fp8(const epl_problem *p, const int64_t *topk_idx, const uint8_t *x,
                     const void *x_scale, int scale_format, int64_t capacity_rows,
                     int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                     int32_t *num_tokens_per_rdma_rank,
                     uint8_t *is_token_in_rank, int32_t *expert_start_loc,
                     int32_t *total_host, uint8_t *out, void *out_scale,
                     int32_t *m_indices, int32_t *output_index, void *workspace,
                     void *stream);

/* Low-latency dispatch into a fixed rectangle (strategy A of "高性能专家并行
 * （EP）内核解剖学解读", high-throughput part, subsection 3: room for the
 * worst case, no count exchange; laid out like the low-latency receive
 * buffers of "[MoE] Deepseek的All-to-all通信: DeepEP代码解读", section
 * low_latency, with the FP8 cast the low-latency dispatch does on the way).
 * The T tokens arrive as T / M source segments of M = tokens_per_segment
 * tokens (segment s = tokens [s*M, (s+1)*M); T % M == 0; tokens of a short
 * segment are padded with all -1 slots). Expert e owns rows
 * [e*cap, (e+1)*cap) of `out`, cap = rows_per_expert (the worst case is M
 * times the number of segments); its slots fill them from the first one in
 * (token, k) order, so the valid rows of e are its first recv_count[e]
 * rows, grouped by segment. Each placed row holds the token's row cast to
 * FP8 e4m3 per 128-column group: scale = amax / 448, codes = e4m3(x *
 * (448 / amax)) rounded to nearest even (binary32 steps; an all-zero group
 * has scale 0 and zero codes). Outputs, all device memory:
 *   out           uint8 [E, cap, H]   e4m3 codes (rows past recv_count untouched)
 *   out_scale     float [E, S, cap]   scale of group g of row j at (e*S + g)*cap + j
 *                                     (column-major per expert), S = H / 128
 *   recv_count    int32 [E]           rows placed for each expert
 *   src_info      int32 [E, cap]      token index within its segment, per placed row
 *   layout_range  int32 [E, T/M, 2]   (begin, count) of segment s's rows in e's block
 *   output_index  int32 [T, K]        e*cap + j, or -1 (no selection, or no room)
 * A slot that finds its expert's rectangle full is not placed and sets
 * EPL_ECAPACITY in the status word. Requires H % 128 == 0, scale_cols ==
 * H / 128, no expert alignment, E * cap <= INT32_MAX; num_ranks and
 * ranks_per_node are not used. x: bf16 [T, H], 16-byte aligned; out 16-byte
 * aligned. The workspace must have epl_ll_workspace_bytes(p, M) bytes
 * (256-byte aligned); the call runs on `stream` the layout and the
 * cast-and-place kernel (with a per-block reduction between them when the
 * layout has more than 64 blocks), or, for a decode-sized batch (T * K <=
 * 4096 and (T / M) * E <= 14336), one kernel that does it all, always with
 * the same results. Receive side: pass local expert ids (-1 for other ranks'
 * experts) and E = the local expert count. */
size_t epl_ll_workspace_bytes(const epl_problem *p, int32_t tokens_per_segment);
int epl_ll_dispatch(const epl_problem *p, int32_t tokens_per_segment, int64_t rows_per_expert,
                    const int64_t *topk_idx, const uint16_t *x, uint8_t *out,
                    float *out_scale, int32_t *recv_count, int32_t *src_info,
                    int32_t *layout_range, int32_t *output_index, void *workspace,
                    void *stream);

/* Step 4 -- combine. For every token t:
 *   y[t, :] = sum over k ascending with output_index[t, k] >= 0 of
 *             topk_weights[t, k] * expert_out[output_index[t, k], :]
 * accumulated in fp32 from +0 (a token with no valid slot gets zeros).
 * expert_out is bf16 [expert_rows, H] (it may be the scatter's `out`);
 * topk_weights is fp32 [T, K]; y is fp32 or bf16 [T, H] per `out_dtype`.
 * An output_index >= expert_rows is skipped and, if `workspace` is not
 * NULL, recorded as EPL_ERANGE in its status word. expert_out / y: 16-byte
 * aligned; output_index / topk_weights: 4-byte aligned; y must not overlap
 * any input. */
int epl_combine(const epl_problem *p, const uint16_t *expert_out,
                int64_t expert_rows, const int32_t *output_index,
                const float *topk_weights, int out_dtype, void *y,
                void *workspace, void *stream);

/* The synthetic expert of the large-batch workload (not a step of the
 * dispatch path; it stands in for the grouped GEMM between scatter and
 * combine): rows_out[p, :] = bf16_rne(float(rows_in[p, :]) * (1 + m_indices[p]/256))
 * for p < min(N, capacity_rows) with m_indices[p] >= 0 (padding rows are
 * skipped), N being the total that the last epl_scan / epl_dispatch on
 * `workspace` stored. rows_in may equal rows_out. */
int epl_expert_scale(const epl_problem *p, const uint16_t *rows_in,
                     const int32_t *m_indices, int64_t capacity_rows,
                     uint16_t *rows_out, const void *workspace, void *stream);

/* Synchronises `stream`, then returns the status recorded in `workspace`
 * since the last epl_layout / epl_dispatch: EPL_OK, EPL_ERANGE or
 * EPL_ECAPACITY (EPL_ERANGE first if both occurred), or EPL_EHIP. */
int epl_status(const void *workspace, void *stream);

/* Synchronises `stream` and returns the total row count N stored in
 * `workspace` by the last scan, or a negative EPL_E* code. */
int64_t epl_total(const void *workspace, void *stream);

/* Static text for a status code. */
const char *epl_strerror(int code);

/* Library version, e.g. 0x000300 for 0.3.0. */
int epl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EPL_H */
