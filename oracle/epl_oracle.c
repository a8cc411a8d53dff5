/*
 * CPU oracle for MoE expert-parallel layout / scan / scatter / combine.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this file. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg use it. It shares no code, header, table
 * or helper with the HIP library: every routine below is written out from
 * the definitions, plainly, single-threaded, with no blocking or fusion.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fPIC -shared (see build.py).
 *
 * Sources (page title, section):
 *   [DEEPEP]  "[MoE] Deepseek的All-to-all通信: DeepEP代码解读" (hqwc.cn),
 *             section "Dispatch": get_dispatch_layout returns, per expert and
 *             per rank, how many tokens go there, and a [tokens, ranks]
 *             boolean telling whether a token goes to a rank; topk_idx is
 *             int64 [tokens, topk] with -1 meaning "no selection".
 *   [ANATOMY] "高性能专家并行（EP）内核解剖学解读" (aimsg.uk), part on the
 *             high-throughput path, subsections 1 (dispatch gathers the rows
 *             bound for each expert into one dense buffer for the grouped
 *             GEMM), 3 (exact allocation sized by the real counts) and 5
 *             (buffer layout by prefix sum: the first source starts at 0,
 *             each next one where the previous ended); section
 *             "任务设定与数据流" (results are brought back to where they
 *             came from).
 *   [SGLANG]  "参考sglang代码，重构vllm021中EP高吞吐代码，消除空泡问题"
 *             (rkmt.cn), section 2.2 (ep_scatter writes the ragged buffer,
 *             its scales, m_indices and output_index; the total row count is
 *             the sum of the counts) and section 3.3 (output_index / inv_perm
 *             is int32 with -1 for slots that are not placed; m_indices holds
 *             the expert id of every row).
 *
 * Readings where the pages leave a step open:
 *   - rank r owns the contiguous experts [r*E/R, (r+1)*E/R);
 *   - per-rank counts count tokens, once per rank, not slots;
 *   - within an expert, rows are ordered by (token, k) ascending;
 *   - the prefix sum is exclusive and starts at 0;
 *   - combine: y[t] = sum over valid k, ascending, of w[t,k] * row, where the
 *     row is the expert output at output_index[t,k]. Evaluated here in fp64.
 *
 * Parity pins (tests/test_oracle_pins.py): worked examples from the pages,
 * an O((TK)^2) brute force of the placement definition, numpy's stable
 * argsort, closed forms for combine on exactly representable values,
 * torch's float->bf16 and float->float8_e4m3fn rounding for the two
 * encoders, the quantiser redone with numpy binary32 arithmetic, the
 * fixed-rectangle layout against the (pinned) prefix-sum layout, and
 * invariants.
 */
#define _POSIX_C_SOURCE 200809L   /* clock_gettime, for the timing harness at the end */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ERANGE (-2)

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 is the upper half of an IEEE binary32: widen by appending 16 zero
 * bits, then convert the float exactly to double. */
double epl_oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, and return its
 * bit pattern. Written from the number format: bf16 keeps 8 significant
 * bits (exponent range of binary32), so a finite value is a multiple of
 * 2^(e-7) where 2^e <= |v| < 2^(e+1), or of 2^-133 in the subnormal range.
 * nearbyint() rounds the scaled value to an integer with ties to even under
 * the default rounding mode. */
uint16_t epl_oracle_bf16_from_double(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    int e2;
    (void)frexp(a, &e2);              /* a = m * 2^e2, 0.5 <= m < 1 */
    int quantum = (e2 - 1) - 7;       /* spacing of bf16 values in this binade */
    if (quantum < -133)
        quantum = -133;               /* subnormal spacing */
    double q = nearbyint(ldexp(a, -quantum));
    double r = ldexp(q, quantum);
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);   /* overflow to infinity */
    float f = (float)r;               /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* -------------------------------------------------------------- layout -- */

static int check_shape(int64_t T, int32_t K, int32_t E, int32_t R)
{
    if (T < 0 || K < 1 || E < 1 || R < 1 || E % R != 0)
        return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* [DEEPEP] get_dispatch_layout: counts per expert, the token/rank mask and
 * the number of tokens each rank receives. A token that picks two experts of
 * the same rank is sent to that rank once. Ids outside [-1, E) are rejected. */
int epl_oracle_layout(int64_t T, int32_t K, int32_t E, int32_t R,
                      const int64_t *topk_idx,
                      int32_t *num_tokens_per_expert,
                      int32_t *num_tokens_per_rank,
                      uint8_t *is_token_in_rank)
{
    if (check_shape(T, K, E, R) != ORACLE_OK)
        return ORACLE_EINVAL;
    int64_t experts_per_rank = E / R;

    for (int64_t i = 0; i < T * (int64_t)K; ++i)
        if (topk_idx[i] < -1 || topk_idx[i] >= E)
            return ORACLE_ERANGE;

    for (int32_t e = 0; e < E; ++e)
        num_tokens_per_expert[e] = 0;
    for (int32_t r = 0; r < R; ++r)
        num_tokens_per_rank[r] = 0;
    for (int64_t i = 0; i < T * (int64_t)R; ++i)
        is_token_in_rank[i] = 0;

    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0)
                continue;                       /* -1: no selection */
            num_tokens_per_expert[e] += 1;
            is_token_in_rank[t * R + e / experts_per_rank] = 1;
        }
    }
    for (int64_t t = 0; t < T; ++t)
        for (int32_t r = 0; r < R; ++r)
            num_tokens_per_rank[r] += is_token_in_rank[t * R + r];
    return ORACLE_OK;
}

/* [DEEPEP] Dispatch, get_dispatch_layout: with ranks spread over nodes of
 * G GPUs each, the tokens bound for each RDMA rank, i.e. for each node
 * (rank r sits on node r / G; a token reaches another node through the peer
 * with the same GPU index there). A token counts once for a node if it goes
 * to any rank of that node. The page gives no value for the single-node
 * case; callers take it as "not produced". */
int epl_oracle_rdma_counts(int64_t T, int32_t R, int32_t G,
                           const uint8_t *is_token_in_rank,
                           int32_t *num_tokens_per_rdma_rank)
{
    if (T < 0 || R < 1 || G < 1 || R % G != 0)
        return ORACLE_EINVAL;
    int32_t nodes = R / G;
    for (int32_t n = 0; n < nodes; ++n) {
        int32_t tokens = 0;
        for (int64_t t = 0; t < T; ++t) {
            int any = 0;
            for (int32_t r = n * G; r < (n + 1) * G; ++r)
                if (is_token_in_rank[t * R + r])
                    any = 1;
            tokens += any;
        }
        num_tokens_per_rdma_rank[n] = tokens;
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- scan -- */

/* [ANATOMY] subsection 5 / [SGLANG] section 2.2: each expert's block starts
 * where the previous one ended, the first at 0; the buffer holds the sum of
 * all block sizes. With an alignment a > 1 ([DEEPEP] Dispatch, the
 * expert_alignment argument; [SGLANG] section 3.3, block_m for the grouped
 * GEMM) an expert's block size is its count rounded up to a multiple of a;
 * a <= 1 means no rounding. */
int epl_oracle_scan(int32_t E, const int32_t *num_tokens_per_expert, int32_t alignment,
                    int32_t *expert_start_loc, int64_t *total)
{
    if (E < 1 || alignment < 0)
        return ORACLE_EINVAL;
    int64_t a = alignment > 1 ? alignment : 1;
    int64_t running = 0;
    for (int32_t e = 0; e < E; ++e) {
        if (num_tokens_per_expert[e] < 0)
            return ORACLE_EINVAL;
        expert_start_loc[e] = (int32_t)running;
        int64_t c = num_tokens_per_expert[e];
        int64_t blocks = c / a + (c % a != 0);
        running += blocks * a;
    }
    *total = running;
    return ORACLE_OK;
}

/* ------------------------------------------------------------- scatter -- */

/* [ANATOMY] subsection 1, [SGLANG] sections 2.2 and 3.3: every valid slot
 * (t, k) gets its own row in its expert's block, in (t, k) order (a counting
 * sort: a cursor per expert starts at the expert's offset and advances by
 * one per placed row). The row receives a bit copy of x[t] and, when scales
 * are present, of x_scale[t]; m_indices[row] = expert; output_index[t, k] =
 * row, or -1 for a -1 slot. A row of the total_rows that receives no slot
 * (alignment padding at the end of an expert's block) has m_indices = -1,
 * the marker the grouped GEMM skips ([SGLANG] section 3.3). Any of out /
 * out_scale may be NULL to skip the row copies (used when only the indices
 * are compared). */
int epl_oracle_scatter(int64_t T, int32_t K, int32_t E, int32_t H, int32_t S,
                       const uint16_t *x, const float *x_scale,
                       const int64_t *topk_idx, const int32_t *expert_start_loc,
                       int64_t total_rows, uint16_t *out, float *out_scale,
                       int32_t *m_indices, int32_t *output_index)
{
    if (T < 0 || K < 1 || E < 1 || H < 0 || S < 0 || total_rows < 0)
        return ORACLE_EINVAL;
    for (int64_t p = 0; p < total_rows; ++p)
        m_indices[p] = -1;
    int64_t *cursor = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    if (!cursor)
        return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e)
        cursor[e] = expert_start_loc[e];

    int rc = ORACLE_OK;
    for (int64_t t = 0; t < T && rc == ORACLE_OK; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < -1 || e >= E) {
                rc = ORACLE_ERANGE;
                break;
            }
            if (e < 0) {
                output_index[t * K + k] = -1;
                continue;
            }
            int64_t row = cursor[e];
            cursor[e] += 1;
            output_index[t * K + k] = (int32_t)row;
            m_indices[row] = (int32_t)e;
            if (out)
                memcpy(out + row * (int64_t)H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);
            if (out_scale && S > 0)
                memcpy(out_scale + row * (int64_t)S, x_scale + t * (int64_t)S, sizeof(float) * (size_t)S);
        }
    }
    free(cursor);
    return rc;
}

/* Scale formats of the byte-row scatter. */
#define ORACLE_SCALE_NONE 0
#define ORACLE_SCALE_ROWS 1   /* W words per row, row-major in and out            */
#define ORACLE_SCALE_COLS 2   /* W words per token row-major in; out column-major */

/* The scatter for rows given as raw bytes: an FP8 (e4m3) payload of H bytes
 * per row, as DeepEP dispatches it ([DEEPEP] Dispatch, the x argument's
 * tuple form), with per-row scale words. Placement is the same counting sort
 * as epl_oracle_scatter. Scale rows of W 4-byte words follow their row:
 * ORACLE_SCALE_ROWS writes them row-major ([rows, W]); ORACLE_SCALE_COLS
 * writes the layout sglang allocates for UE8M0 scales ([SGLANG] section 2.2:
 * an int32 [ceil(S/4), rows] buffer viewed transposed), i.e. word j of row p
 * at out_scale[j * scale_ld + p], scale_ld being the buffer's row capacity.
 * The words are moved as opaque bits. Rows that receive no slot get
 * m_indices = -1. */
int epl_oracle_scatter_rows(int64_t T, int32_t K, int32_t E, int64_t row_bytes,
                            const uint8_t *x, int32_t scale_format, int32_t scale_words,
                            const uint32_t *x_scale, const int64_t *topk_idx,
                            const int32_t *expert_start_loc, int64_t total_rows,
                            int64_t scale_ld, uint8_t *out, uint32_t *out_scale,
                            int32_t *m_indices, int32_t *output_index)
{
    if (T < 0 || K < 1 || E < 1 || row_bytes < 0 || scale_words < 0 || total_rows < 0)
        return ORACLE_EINVAL;
    if (scale_format == ORACLE_SCALE_COLS && scale_ld < total_rows)
        return ORACLE_EINVAL;
    for (int64_t p = 0; p < total_rows; ++p)
        m_indices[p] = -1;              /* rows without a slot: padding */
    int64_t *next = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    if (!next)
        return ORACLE_EINVAL;
    for (int32_t e = 0; e < E; ++e)
        next[e] = expert_start_loc[e];

    int rc = ORACLE_OK;
    for (int64_t t = 0; t < T && rc == ORACLE_OK; ++t) {
        for (int32_t k = 0; k < K; ++k) {   /* the token's slots in order */
            int64_t e = topk_idx[t * K + k];
            if (e < -1 || e >= E) {
                rc = ORACLE_ERANGE;
                break;
            }
            if (e == -1) {
                output_index[t * K + k] = -1;   /* no selection: no row */
                continue;
            }
            int64_t p = next[e]++;
            output_index[t * K + k] = (int32_t)p;
            m_indices[p] = (int32_t)e;
            if (out)
                memcpy(out + p * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            if (out_scale && scale_format == ORACLE_SCALE_ROWS) {
                for (int32_t j = 0; j < scale_words; ++j)
                    out_scale[p * scale_words + j] = x_scale[t * scale_words + j];
            } else if (out_scale && scale_format == ORACLE_SCALE_COLS) {
                for (int32_t j = 0; j < scale_words; ++j)
                    out_scale[j * scale_ld + p] = x_scale[t * scale_words + j];
            }
        }
    }
    free(next);
    return rc;
}

/* ------------------------------------------------ FP8 e4m3 quantisation -- */

/* Round a double to the nearest FP8 e4m3 value (the OCP "fn" encoding: 1 sign
 * bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, largest
 * finite value 448), ties to even, and return its byte. Written from the
 * number format like the bf16 encoder: a value in [2^(e-1), 2^e) is a
 * multiple of 2^(e-4); below the smallest normal 2^-6 the spacing is 2^-9.
 * Magnitudes that round above 448 saturate to 448 (the quantiser below never
 * produces them). NaN gives 0x7F. */
uint8_t epl_oracle_e4m3_from_double(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);              /* a = m * 2^e2, 0.5 <= m < 1 */
    int quantum = e2 - 4;
    if (quantum < -9)
        quantum = -9;                 /* subnormal spacing */
    double r = ldexp(nearbyint(ldexp(a, -quantum)), quantum);
    if (r > 448.0)
        r = 448.0;
    if (r < ldexp(1.0, -6))           /* subnormal (or zero): r = m * 2^-9 */
        return (uint8_t)(sign | (uint8_t)ldexp(r, 9));
    int e;
    double m = frexp(r, &e);          /* r = m * 2^e, 0.5 <= m < 1 */
    int exp_field = e + 6;            /* (e - 1) + bias 7 */
    int mant = (int)ldexp(m * 2.0 - 1.0, 3);
    return (uint8_t)(sign | (uint8_t)(exp_field << 3) | (uint8_t)mant);
}

/* Round a double to binary32's 24-bit significand, ties to even, with no
 * exponent limits (no overflow, no subnormal range): the value binary32
 * arithmetic gives when its result is in the normal range, and beyond it
 * the value it would give with a wider exponent. Zero and non-finite values
 * pass through. */
static double round_to_24_bits(double v)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    double m = frexp(v, &e);                  /* v = m * 2^e, 0.5 <= |m| < 1 */
    return ldexp(nearbyint(ldexp(m, 24)), e - 24);
}

/* The low-latency dispatch sends FP8 rows with one fp32 scale per 128
 * hidden columns ([DEEPEP] low_latency mode: the dispatch casts to FP8 on
 * the way, and returns scales of shape [..., hidden / 128]). The pages do
 * not give the cast; reading: per 128-column group of a token,
 *   amax = max |x|, scale = amax / 448, inv = 448 / amax (0 if amax = 0),
 *   q = e4m3(x * inv),
 * with round to nearest at binary32's precision at every step (scale in
 * binary32 proper; inv and the product x * inv rounded to 24 significant
 * bits before the e4m3 rounding), so that the group's largest magnitude
 * lands on 448 and q * scale approximates x. inv and the product use no
 * exponent limits: bf16 keeps binary32's exponent range, and for a group
 * whose amax is below 448 / FLT_MAX (about 1.3e-36) binary32's 448 / amax
 * would overflow to infinity, turning every zero of the group into a NaN
 * code and every other value into +-448; without the limit the group
 * encodes like the same group scaled by a power of two. (Where binary32 has
 * the range -- every other group -- this is exactly binary32 arithmetic:
 * the quotient is rounded once from the double quotient, which for a
 * division is the same as rounding the exact quotient, since 53 >= 2 * 24
 * + 2; the product of an 8-bit and a 24-bit significand is exact in double;
 * a product below binary32's normal range would round to zero in e4m3
 * either way.) x is bf16 [T, H], H a multiple of 128; q is [T, H] bytes,
 * scale [T, H / 128]. */
int epl_oracle_quantize_e4m3(int64_t T, int32_t H, const uint16_t *x, uint8_t *q, float *scale)
{
    if (T < 0 || H < 0 || H % 128 != 0)
        return ORACLE_EINVAL;
    int32_t S = H / 128;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t g = 0; g < S; ++g) {
            const uint16_t *xg = x + t * (int64_t)H + (int64_t)g * 128;
            float amax = 0.0f;
            for (int32_t i = 0; i < 128; ++i) {
                float v = fabsf((float)epl_oracle_bf16_to_double(xg[i]));
                if (v > amax)
                    amax = v;
            }
            float s = amax / 448.0f;
            double inv = amax > 0.0f ? round_to_24_bits(448.0 / (double)amax) : 0.0;
            scale[t * (int64_t)S + g] = s;
            for (int32_t i = 0; i < 128; ++i) {
                double p = round_to_24_bits(epl_oracle_bf16_to_double(xg[i]) * inv);
                q[t * (int64_t)H + (int64_t)g * 128 + i] = epl_oracle_e4m3_from_double(p);
            }
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------- low-latency rectangle -- */

/* Strategy A of [ANATOMY] high-throughput part, subsection 3 (a fixed
 * rectangle sized for the worst case, no count exchange), in the shape of
 * DeepEP's low-latency receive buffers ([DEEPEP] low_latency mode): every
 * expert e owns rows [e * cap, (e + 1) * cap) of a [E * cap, H] FP8 buffer,
 * with cap = (source segments) x (tokens per segment) in the worst case. The
 * T tokens arrive as T / M source segments of M tokens each (segment s =
 * tokens [s * M, (s + 1) * M), padding tokens carry only -1 slots). An
 * expert's slots fill its rows from the first one in (token, k) order, so
 * the valid rows of e are its first recv_count[e] rows, grouped by source
 * segment; the row holds the token's quantised row (epl_oracle_quantize_e4m3)
 * and its scales go to out_scale[(e * S + g) * cap + j], column-major in the
 * last two dimensions as DeepEP returns them. src_info of the row is the
 * token's index within its segment; layout_range[e][s] = (rows of e from
 * segments before s, rows of e from segment s), i.e. where segment s's rows
 * start within e's block and how many there are; output_index[t, k] is the
 * row (e * cap + j) or -1. A slot beyond cap rows is not placed
 * (output_index -1, not counted in recv_count) and *overflow is set to 1.
 * Rows of an expert past its recv_count are left untouched. With x NULL
 * only the indices are produced. */
int epl_oracle_ll_dispatch(int64_t T, int32_t K, int32_t E, int32_t H, int32_t M, int64_t cap,
                           const uint16_t *x, const int64_t *topk_idx, uint8_t *out,
                           float *out_scale, int32_t *recv_count, int32_t *src_info,
                           int32_t *layout_range, int32_t *output_index, int32_t *overflow)
{
    if (T < 0 || K < 1 || E < 1 || H < 0 || H % 128 != 0 || M < 1 || T % M != 0 || cap < 0)
        return ORACLE_EINVAL;
    int32_t S = H / 128;
    int64_t nseg = T / M;
    uint8_t *qrow = (uint8_t *)malloc((size_t)H + 1);
    float *srow = (float *)malloc(sizeof(float) * ((size_t)S + 1));
    if (!qrow || !srow) {
        free(qrow);
        free(srow);
        return ORACLE_EINVAL;
    }
    *overflow = 0;
    for (int32_t e = 0; e < E; ++e) {
        recv_count[e] = 0;
        for (int64_t s = 0; s < nseg; ++s) {
            layout_range[(e * nseg + s) * 2 + 0] = 0;
            layout_range[(e * nseg + s) * 2 + 1] = 0;
        }
    }
    int rc = ORACLE_OK;
    for (int64_t t = 0; t < T && rc == ORACLE_OK; ++t) {
        int64_t seg = t / M;
        int quantised = 0;
        for (int32_t k = 0; k < K; ++k) {      /* slots in k order */
            int64_t e = topk_idx[t * K + k];
            if (e < -1 || e >= E) {
                rc = ORACLE_ERANGE;
                break;
            }
            if (e == -1) {
                output_index[t * K + k] = -1;  /* not selected */
                continue;
            }
            int64_t j = recv_count[e];
            if (j >= cap) {                    /* the rectangle is full */
                *overflow = 1;
                output_index[t * K + k] = -1;  /* dropped */
                continue;
            }
            recv_count[e] += 1;
            layout_range[(e * nseg + seg) * 2 + 1] += 1;
            int64_t row = e * cap + j;
            output_index[t * K + k] = (int32_t)row;
            src_info[row] = (int32_t)(t - seg * M);
            if (!x)
                continue;                      /* indices only */
            if (!quantised) {
                epl_oracle_quantize_e4m3(1, H, x + t * (int64_t)H, qrow, srow);
                quantised = 1;
            }
            if (out)
                memcpy(out + row * (int64_t)H, qrow, (size_t)H);
            if (out_scale)
                for (int32_t g = 0; g < S; ++g)
                    out_scale[(e * (int64_t)S + g) * cap + j] = srow[g];
        }
    }
    for (int32_t e = 0; e < E; ++e) {
        int32_t before = 0;                    /* rows of e from earlier segments */
        for (int64_t s = 0; s < nseg; ++s) {
            layout_range[(e * nseg + s) * 2 + 0] = before;
            before += layout_range[(e * nseg + s) * 2 + 1];
        }
    }
    free(qrow);
    free(srow);
    return rc;
}

/* ------------------------------------------------------- expert stand-in -- */

/* The synthetic expert of the large-batch workload: expert e multiplies its
 * row by (1 + e/256) and the result is stored as bf16 (nearest, ties to even).
 * The product is exact in double, so the only rounding is the final one. */
int epl_oracle_expert_scale(int64_t N, int32_t H, const uint16_t *rows,
                            const int32_t *m_indices, uint16_t *expert_out)
{
    if (N < 0 || H < 0)
        return ORACLE_EINVAL;
    for (int64_t p = 0; p < N; ++p) {
        double factor = 1.0 + (double)m_indices[p] / 256.0;
        for (int32_t h = 0; h < H; ++h) {
            double v = epl_oracle_bf16_to_double(rows[p * (int64_t)H + h]);
            expert_out[p * (int64_t)H + h] = epl_oracle_bf16_from_double(v * factor);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------- combine -- */

/* [ANATOMY] "任务设定与数据流" / [SGLANG] section 2.2 (the state kept for the
 * way back: topk ids, topk weights, output_index): for each token t,
 *     y[t, :] = sum over valid k (ascending) of w[t, k] * expert_out[output_index[t, k], :]
 * accumulated in double from +0. A token with no valid slot yields zeros.
 * ``tokens`` (length n_tokens) selects which tokens to evaluate; NULL means
 * all T in order. y has one H-wide row per evaluated token. */
int epl_oracle_combine(int64_t T, int32_t K, int32_t H,
                       const uint16_t *expert_out, int64_t expert_rows,
                       const int32_t *output_index, const float *topk_weights,
                       const int64_t *tokens, int64_t n_tokens, double *y)
{
    if (T < 0 || K < 1 || H < 0 || expert_rows < 0)
        return ORACLE_EINVAL;
    int64_t count = tokens ? n_tokens : T;
    for (int64_t i = 0; i < count; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        if (t < 0 || t >= T)
            return ORACLE_EINVAL;
        double *yrow = y + i * (int64_t)H;
        for (int32_t h = 0; h < H; ++h)
            yrow[h] = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            int64_t row = output_index[t * K + k];
            if (row < 0)
                continue;
            if (row >= expert_rows)
                return ORACLE_ERANGE;
            double w = (double)topk_weights[t * K + k];
            const uint16_t *src = expert_out + row * (int64_t)H;
            for (int32_t h = 0; h < H; ++h)
                yrow[h] = yrow[h] + w * epl_oracle_bf16_to_double(src[h]);
        }
    }
    return ORACLE_OK;
}

/* ----------------------------------------------------- timing harness -- */

/* Not part of the method: a wall-clock harness for the CPU baseline of the
 * benchmark. Runs one pass of the oracle's steps above on buffers the caller
 * allocated once -- layout, scan, the byte-row scatter (rows of row_bytes
 * bytes: 2H for bf16, H for FP8; W scale words per row in scale_format),
 * then the combine -- timing each step with the monotonic clock. The
 * combine's expert rows depend on expert_mode: 0 = the scattered rows
 * themselves (bf16, row_bytes = 2H), 1 = the large workload's expert
 * stand-in applied to them into expert_out, 2 = expert_out as given (a bf16
 * stand-in for an FP8 payload's expert output). Step durations in
 * nanoseconds: ns[0] layout, ns[1] scan, ns[2] scatter, ns[3] expert (0
 * unless expert_mode is 1), ns[4] combine. Buffers: cnt [E], per_rank [R],
 * in_rank [T, R], start [E], out [cap, row_bytes], out_scale for cap rows
 * (NULL without scales), m_indices [cap], output_index [T, K], expert_out
 * [cap, H] bf16 (modes 1 and 2), y [T, H] double; cap must be at least the
 * buffer's row count (routed rows, plus the padding of an expert alignment
 * a > 1). */
static int64_t monotonic_ns(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (int64_t)ts.tv_sec * 1000000000LL + (int64_t)ts.tv_nsec;
}

int epl_oracle_time_pass(int64_t T, int32_t K, int32_t E, int32_t R, int32_t H,
                         int64_t row_bytes, const uint8_t *x, int32_t scale_format,
                         int32_t scale_words, const uint32_t *x_scale, const int64_t *topk_idx,
                         const float *topk_weights, int32_t alignment, int64_t cap, int32_t *cnt,
                         int32_t *per_rank, uint8_t *in_rank, int32_t *start, uint8_t *out,
                         uint32_t *out_scale, int32_t *m_indices, int32_t *output_index,
                         int32_t expert_mode, uint16_t *expert_out, double *y, int64_t *ns)
{
    if (expert_mode < 0 || expert_mode > 2 || (expert_mode == 0 && row_bytes != 2 * (int64_t)H) ||
        (expert_mode > 0 && !expert_out))
        return ORACLE_EINVAL;
    int64_t t0 = monotonic_ns();
    int rc = epl_oracle_layout(T, K, E, R, topk_idx, cnt, per_rank, in_rank);
    int64_t t1 = monotonic_ns();
    if (rc != ORACLE_OK)
        return rc;
    int64_t total = 0;
    rc = epl_oracle_scan(E, cnt, alignment, start, &total);
    int64_t t2 = monotonic_ns();
    if (rc != ORACLE_OK)
        return rc;
    if (total > cap)
        return ORACLE_EINVAL;
    rc = epl_oracle_scatter_rows(T, K, E, row_bytes, x, scale_format, scale_words, x_scale,
                                 topk_idx, start, total, cap, out, out_scale, m_indices,
                                 output_index);
    int64_t t3 = monotonic_ns();
    if (rc != ORACLE_OK)
        return rc;
    const uint16_t *rows = expert_mode == 0 ? (const uint16_t *)(const void *)out : expert_out;
    if (expert_mode == 1)
        rc = epl_oracle_expert_scale(total, H, (const uint16_t *)(const void *)out, m_indices,
                                     expert_out);
    int64_t t4 = monotonic_ns();
    if (rc != ORACLE_OK)
        return rc;
    rc = epl_oracle_combine(T, K, H, rows, total, output_index, topk_weights, NULL, T, y);
    int64_t t5 = monotonic_ns();
    ns[0] = t1 - t0;
    ns[1] = t2 - t1;
    ns[2] = t3 - t2;
    ns[3] = expert_mode == 1 ? t4 - t3 : 0;
    ns[4] = t5 - t4;
    return rc;
}

/* The same harness for the low-latency step: epl_oracle_ll_dispatch into the
 * caller's rectangle buffers, then the combine over the experts' bf16 output
 * rows given compactly (expert_out [n_rows, H], the row of slot (t, k) being
 * output_index_compact[t, k], prepared by the caller from a previous pass:
 * the placement is deterministic). ns[0] dispatch, ns[1] combine. */
int epl_oracle_time_ll_pass(int64_t T, int32_t K, int32_t E, int32_t H, int32_t M, int64_t cap,
                            const uint16_t *x, const int64_t *topk_idx, uint8_t *out,
                            float *out_scale, int32_t *recv_count, int32_t *src_info,
                            int32_t *layout_range, int32_t *output_index, int32_t *overflow,
                            const uint16_t *expert_out, int64_t n_rows,
                            const int32_t *output_index_compact, const float *topk_weights,
                            double *y, int64_t *ns)
{
    int64_t t0 = monotonic_ns();
    int rc = epl_oracle_ll_dispatch(T, K, E, H, M, cap, x, topk_idx, out, out_scale, recv_count,
                                    src_info, layout_range, output_index, overflow);
    int64_t t1 = monotonic_ns();
    if (rc != ORACLE_OK)
        return rc;
    rc = epl_oracle_combine(T, K, H, expert_out, n_rows, output_index_compact, topk_weights, NULL,
                            T, y);
    int64_t t2 = monotonic_ns();
    ns[0] = t1 - t0;
    ns[1] = t2 - t1;
    return rc;
}
