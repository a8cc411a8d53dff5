// libepl.so host side: argument validation, workspace carving and kernel
// launches for the C ABI declared in include/epl.h. Every entry point
// checks its arguments on the host before it enqueues anything, then only
// enqueues on the caller's stream (epl_status / epl_total synchronise it).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "epl.h"
#include "epl_kernels.h"

namespace {

using epl::WsHeader;

constexpr size_t kWsAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int alignment_of(const epl_problem &p) { return p.expert_alignment > 1 ? p.expert_alignment : 1; }

// Nodes whose token counts the layout produces: R / G when the ranks span
// several nodes of G, else 0 (one node: not produced).
int nodes_of(const epl_problem &p)
{
    const int G = p.ranks_per_node;
    return (G > 0 && G < p.num_ranks) ? p.num_ranks / G : 0;
}

// Rows that always suffice: T*K, or round_up(T*K + E*(a-1), a) with padding.
int64_t capacity_bound(const epl_problem &p)
{
    const int64_t a = alignment_of(p);
    const int64_t rows = p.num_tokens * (int64_t)p.num_topk + (int64_t)p.num_experts * (a - 1);
    return (rows + a - 1) / a * a;
}

bool problem_ok(const epl_problem *p)
{
    if (!p)
        return false;
    if (p->num_tokens < 0 || p->num_topk < 1 || p->num_topk > epl::kMaxTopk)
        return false;
    if (p->num_experts < 1 || p->num_experts > epl::kMaxExperts)
        return false;
    if (p->num_ranks < 1 || p->num_ranks > p->num_experts || p->num_experts % p->num_ranks != 0)
        return false;
    if (p->hidden < 8 || p->hidden % 8 != 0)
        return false;
    if (p->scale_cols != 0 && (p->hidden % 128 != 0 || p->scale_cols != p->hidden / 128))
        return false;
    if (p->expert_alignment < 0 || p->expert_alignment > epl::kMaxAlignment)
        return false;
    if (p->ranks_per_node < 0 || p->reserved != 0)
        return false;
    if (p->ranks_per_node > 0 && p->ranks_per_node < p->num_ranks &&
        p->num_ranks % p->ranks_per_node != 0)
        return false;
    if (capacity_bound(*p) > (int64_t)INT32_MAX)
        return false;
    return true;
}

// FP8 rows are H bytes (16-byte vectors need H % 16 == 0); scales, when
// requested, need a problem with scale_cols > 0.
bool fp8_problem_ok(const epl_problem *p, int scale_format)
{
    if (!problem_ok(p) || p->hidden % 16 != 0)
        return false;
    if (scale_format == EPL_SCALE_NONE)
        return true;
    return (scale_format == EPL_SCALE_F32 || scale_format == EPL_SCALE_UE8M0) && p->scale_cols > 0;
}

#ifndef EPL_LAYOUT_BLOCKS
#define EPL_LAYOUT_BLOCKS 64       // blocks the layout aims for
#endif
#ifndef EPL_LAYOUT_MIN_TOKENS
#define EPL_LAYOUT_MIN_TOKENS 16   // smallest block
#endif

#ifndef EPL_LAYOUT_MATRIX_BUDGET
#define EPL_LAYOUT_MATRIX_BUDGET 65536
#endif

// Tokens per layout block for 256-thread workgroups (expert counts too wide
// for the 1024-thread layout): enough blocks to spread the work (about 64),
// but at most 256 tokens (one per thread) and at most 2048 slots (the LDS
// key buffer), and at least 16 tokens so the per-block count matrix stays
// small. With many tokens, blocks stay at 64 tokens (else 128) while the
// matrix the scan reduces, blocks x (experts + rank and node columns), holds
// at most EPL_LAYOUT_MATRIX_BUDGET entries: smaller blocks rank their slots
// sooner, but a larger matrix makes the single-workgroup scan longer.
// Measured with 256-thread workgroups on layout + reduce: 29765 tokens with
// 8 local experts 20.6 -> 14.9 us (64), 16384 tokens with 256 experts 25.2
// -> 22.9 us (128), while 65536 tokens with 256 experts keep 256 (128 would
// take 35.3 -> 42.9 us).
#ifndef EPL_LAYOUT_BLOCKS_WIDE
#define EPL_LAYOUT_BLOCKS_WIDE 32
#endif

// When the per-wave counters of 16 waves fit in LDS (up to ~512 experts),
// the layout runs 1024-thread workgroups on about 32 blocks of at most 256
// tokens: each block ranks its slots with 4x the waves, and the scan
// reduces a matrix of fewer blocks. Layout + reduce: 4096 tokens of hidden
// 7168 15.2 -> 13.8 us, 16384 tokens 22.8 -> 16.6 us, 65536 tokens 35.2 ->
// 28.3 us; the receive side (29765 tokens, 8 experts) unchanged. Wider
// expert counts keep 256-thread workgroups and the block rule below.
bool wide_layout(const epl_problem &p)
{
    const int bmax = std::min(256, epl::kMaxSlotsPerBlock / p.num_topk);
    return epl::layout_lds_bytes(bmax, p.num_topk, p.num_experts, p.num_ranks + nodes_of(p),
                                 epl::kLayoutThreadsWide / epl::kWave) <= epl::kLayoutLdsBytes;
}

int layout_block_tokens(const epl_problem &p)
{
    if (wide_layout(p)) {
        const int64_t cap = std::min(256, epl::kMaxSlotsPerBlock / p.num_topk);
        const int64_t want = (p.num_tokens + EPL_LAYOUT_BLOCKS_WIDE - 1) / EPL_LAYOUT_BLOCKS_WIDE;
        return (int)std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(EPL_LAYOUT_MIN_TOKENS, want), cap));
    }
    int64_t cap = std::min<int64_t>(epl::kLayoutThreads, epl::kMaxSlotsPerBlock / p.num_topk);
    const int64_t cols = (int64_t)p.num_experts + p.num_ranks + nodes_of(p);
    for (int64_t b : {64, 128}) {
        if ((p.num_tokens + b - 1) / b * cols <= EPL_LAYOUT_MATRIX_BUDGET) {
            cap = std::min(cap, b);
            break;
        }
    }
    // the LDS bound: keys and ranks take 8 bytes per slot, plus a pad word per token
    const size_t fixed =
        epl::layout_lds_bytes(0, p.num_topk, p.num_experts, p.num_ranks + nodes_of(p));
    cap = std::min<int64_t>(cap, (int64_t)((epl::kLayoutLdsBytes - fixed) / (8 * (size_t)p.num_topk + 4)));
    int64_t want = (p.num_tokens + EPL_LAYOUT_BLOCKS - 1) / EPL_LAYOUT_BLOCKS;
    want = std::max<int64_t>(EPL_LAYOUT_MIN_TOKENS, want);
    return (int)std::max<int64_t>(1, std::min<int64_t>(want, cap));
}

// The low-latency layout reads per-segment offsets off the per-block ones,
// so its blocks must tile the source segments of M tokens: the largest
// divisor of M not above the usual block size.
int ll_block_tokens(const epl_problem &p, int32_t M)
{
    int b = (int)std::min<int64_t>(layout_block_tokens(p), M);
    while (b > 1 && M % b != 0)
        --b;
    return std::max(b, 1);
}

struct WsLayout {
    int block_tokens;
    int64_t num_blocks;
    size_t counts, block_count, block_base, block_rank, block_err, slot_rank, bytes;
};

WsLayout ws_layout(const epl_problem &p, int block_tokens)
{
    WsLayout w{};
    w.block_tokens = block_tokens;
    w.num_blocks = (p.num_tokens + w.block_tokens - 1) / w.block_tokens;
    size_t off = round_up(sizeof(WsHeader), kWsAlign);
    w.counts = off;
    off += round_up((size_t)p.num_experts * 4, kWsAlign);
    w.block_count = off;
    off += round_up((size_t)w.num_blocks * (size_t)p.num_experts * 4, kWsAlign);
    w.block_base = off;
    off += round_up((size_t)w.num_blocks * (size_t)p.num_experts * 4, kWsAlign);
    w.block_rank = off;
    off += round_up((size_t)w.num_blocks * (size_t)(p.num_ranks + nodes_of(p)) * 4, kWsAlign);
    w.block_err = off;
    off += round_up((size_t)w.num_blocks * 4, kWsAlign);
    w.slot_rank = off;
    off += round_up((size_t)p.num_tokens * (size_t)p.num_topk * 4, kWsAlign);
    w.bytes = off;
    return w;
}

// Batches that one workgroup lays out and scans by itself (see
// ep_layout_scan_kernel): all their tokens form a single block.
bool fused_layout(const epl_problem &p)
{
    return p.num_tokens >= 1 && p.num_tokens * (int64_t)p.num_topk <= epl::kFusedMaxSlots &&
           p.num_experts <= epl::kFusedMaxExperts &&
           p.num_ranks + nodes_of(p) <= epl::kFusedMaxCols;
}

WsLayout ws_layout(const epl_problem &p)
{
    return ws_layout(p, fused_layout(p) ? (int)p.num_tokens : layout_block_tokens(p));
}

template <typename T>
T *at(void *ws, size_t off)
{
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

int launch_status() { return hipGetLastError() == hipSuccess ? EPL_OK : EPL_EHIP; }

// Workgroups for a row kernel: min(items, limit), and never more than 2^22:
// the dispatch packet counts work-items in 32 bits, and 2^22 workgroups of
// up to 1024 threads stay below 2^32. The kernels stride over any items
// beyond the grid.
constexpr int64_t kMaxRowGrid = int64_t(1) << 22;
unsigned row_grid(int64_t items, int64_t limit)
{
    return (unsigned)std::min<int64_t>(items, std::min<int64_t>(limit, kMaxRowGrid));
}

// row_grid for kernels with XCD-aware token ranges (epl::token_range): a
// grid of one workgroup per item, below kXcdRoundBelow items, is rounded up
// to a multiple of the 8 XCDs, without which token_range falls back to
// plain striding (the extra workgroups, at most 7, find no item). At 257 and
// 300 DeepSeek-V3-shaped tokens (1799 and 2100 scatter items, 1028 and 1200
// combine items) the step went 37.5 -> 30.6 and 43.0 -> 32.7 us; with one
// workgroup per token at 29765 tokens the XCD ranges made scatter and
// combine 4-5% slower, so larger grids keep their size. Capped, striding
// grids keep theirs too.
constexpr int64_t kXcdRoundBelow = 8192;

// Grids of at least this many workgroups (one item each) walk their items
// round-robin over the XCDs (workgroup w takes item w) instead of in
// XCD-contiguous ranges: 4096 tokens of hidden 7168 (16384 combine items)
// combine in 98.7-99.3 instead of 104.0-104.3 us, 16384 tokens in 392
// instead of 410 us; from 257 to 2048 tokens (1028-4096 items) the ranges
// are as fast or faster (at 300 tokens, 9.2 against 10.5 us).
#ifndef EPL_COMBINE_XCD_BELOW
#define EPL_COMBINE_XCD_BELOW 8192
#endif
#ifndef EPL_SCATTER_XCD_BELOW
#define EPL_SCATTER_XCD_BELOW 8192
#endif
unsigned xcd_grid(int64_t items, int64_t limit)
{
    const unsigned g = row_grid(items, limit);
    if (g < (unsigned)epl::kNumXcd || (int64_t)g < items || items >= kXcdRoundBelow)
        return g;
    const int64_t r = ((int64_t)g + epl::kNumXcd - 1) / epl::kNumXcd * epl::kNumXcd;
    return (unsigned)std::min<int64_t>(r, kMaxRowGrid);
}

int enqueue_layout(const epl_problem &p, const WsLayout &w, const int64_t *topk, uint8_t *in_rank,
                   void *ws, hipStream_t s)
{
    if (w.num_blocks == 0)
        return EPL_OK;
    const bool vec16 = (p.num_ranks % 16 == 0) && aligned(in_rank, 16);
    const int Rn = nodes_of(p);
    auto launch = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)w.num_blocks), dim3(threads),
                           epl::layout_lds_bytes(w.block_tokens, p.num_topk, p.num_experts,
                                                 p.num_ranks + Rn, threads / epl::kWave),
                           s, topk, p.num_tokens, p.num_topk, p.num_experts, p.num_ranks,
                           p.num_experts / p.num_ranks, epl::div_magic(p.num_experts / p.num_ranks),
                           p.ranks_per_node, epl::div_magic(std::max(p.ranks_per_node, 1)), Rn,
                           w.block_tokens, in_rank, vec16, at<int32_t>(ws, w.block_count),
                           at<int32_t>(ws, w.block_rank), at<uint32_t>(ws, w.block_err),
                           at<int32_t>(ws, w.slot_rank), &at<WsHeader>(ws, 0)->status,
                           &at<WsHeader>(ws, 0)->dense);
    };
    if (wide_layout(p))
        launch(epl::ep_layout_kernel<epl::kLayoutThreadsWide>, epl::kLayoutThreadsWide);
    else
        launch(epl::ep_layout_kernel<epl::kLayoutThreads>, epl::kLayoutThreads);
    return launch_status();
}

// The device address through which a kernel can store straight into the
// caller's pinned host word, or null if the runtime cannot map it (then the
// total is copied with hipMemcpyAsync after the scan).
int32_t *mapped_host_word(int32_t *host)
{
    if (!host)
        return nullptr;
    void *dev = nullptr;
    if (hipHostGetDevicePointer(&dev, host, 0) != hipSuccess) {
        (void)hipGetLastError();   // not mapped: clear the error, use the copy
        return nullptr;
    }
    return static_cast<int32_t *>(dev);
}

// Arguments of the one-workgroup layout + scan; `capacity` >= 0 also
// flags N > capacity in the status word.
epl::LayoutScanArgs layout_scan_args(const epl_problem &p, const WsLayout &w, const int64_t *topk,
                                     uint8_t *in_rank, int32_t *cnt, int32_t *per_rank,
                                     int32_t *per_node, int32_t *start, void *ws,
                                     int32_t *total_mapped, int64_t capacity)
{
    epl::LayoutScanArgs a{};
    a.topk = topk;
    a.T = p.num_tokens;
    a.K = p.num_topk;
    a.E = p.num_experts;
    a.R = p.num_ranks;
    a.experts_per_rank = p.num_experts / p.num_ranks;
    a.epr_magic = epl::div_magic(p.num_experts / p.num_ranks);
    a.G = p.ranks_per_node;
    a.node_magic = epl::div_magic(std::max(p.ranks_per_node, 1));
    a.Rn = nodes_of(p);
    a.alignment = alignment_of(p);
    a.in_rank = in_rank;
    a.in_rank_vec16 = (p.num_ranks % 16 == 0) && aligned(in_rank, 16);
    a.cnt = cnt;
    a.per_rank = per_rank;
    a.per_node = per_node;
    a.start = start;
    a.block_base = at<int32_t>(ws, w.block_base);
    a.slot_rank = at<int32_t>(ws, w.slot_rank);
    a.ws_counts = at<int32_t>(ws, w.counts);
    a.hdr = at<WsHeader>(ws, 0);
    a.total_out = total_mapped;
    a.capacity = capacity;
    return a;
}

// Layout and scan of a small batch in one launch (fused_layout(p)). With
// `start` null only the layout's outputs are produced (epl_layout); with it,
// also expert_start_loc and N, copied to *total_host if that is not null.
int enqueue_fused(const epl_problem &p, const WsLayout &w, const int64_t *topk, uint8_t *in_rank,
                  int32_t *cnt, int32_t *per_rank, int32_t *per_node, int32_t *start,
                  int32_t *total_host, void *ws, hipStream_t s)
{
    int32_t *mapped = start ? mapped_host_word(total_host) : nullptr;
    hipLaunchKernelGGL(epl::ep_layout_scan_kernel, dim3(1), dim3(epl::kFusedThreads), 0, s,
                       layout_scan_args(p, w, topk, in_rank, cnt, per_rank, per_node, start, ws,
                                        mapped, -1));
    int rc = launch_status();
    if (rc != EPL_OK)
        return rc;
    if (start && total_host && !mapped) {
        if (hipMemcpyAsync(total_host, &at<WsHeader>(ws, 0)->total, sizeof(int32_t),
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            return EPL_EHIP;
    }
    return EPL_OK;
}

int enqueue_scan(const epl_problem &p, const WsLayout &w, int mode, int32_t *cnt, int32_t *per_rank,
                 int32_t *per_node, int32_t *start, int32_t *total_host, void *ws, hipStream_t s)
{
    int32_t *mapped = (mode & epl::kScanPrefix) ? mapped_host_word(total_host) : nullptr;
    hipLaunchKernelGGL(epl::ep_scan_kernel, dim3(1), dim3(epl::kScanThreads), 0, s, mode,
                       w.num_blocks, p.num_experts, p.num_ranks, nodes_of(p), alignment_of(p),
                       at<const int32_t>(ws, w.block_count), at<int32_t>(ws, w.block_base),
                       at<int32_t>(ws, w.block_rank),
                       at<uint32_t>(ws, w.block_err), cnt, per_rank, per_node, start,
                       at<int32_t>(ws, w.counts), at<WsHeader>(ws, 0), mapped);
    int rc = launch_status();
    if (rc != EPL_OK)
        return rc;
    if ((mode & epl::kScanPrefix) && total_host && !mapped) {
        if (hipMemcpyAsync(total_host, &at<WsHeader>(ws, 0)->total, sizeof(int32_t),
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            return EPL_EHIP;
    }
    return EPL_OK;
}

// What the scatter moves per token: the row as opaque bytes, and optional
// scale words in one of the kernel's layouts.
struct RowArgs {
    const uint8_t *x;
    int64_t row_bytes;
    int scale_mode;            // epl::kScaleNone / kScaleRows / kScaleCols
    const uint32_t *x_scale;
    int words;                 // scale words per row
    int64_t scale_ld;          // leading dimension of the column-major layout
    uint8_t *out;
    uint32_t *out_scale;
};

// Work split of the scatter: one workgroup per token from kScatterGridFrom
// tokens on; below, a striding grid of kScatterGridLong (rows of at least
// kScatterLongRowBytes) or kScatterGrid workgroups; and with fewer tokens
// than that grid, each row cut into column parts (decode-sized batches).
struct ScatterSplit {
    int parts;
    unsigned grid;
    int grid_dense;     // > 0: workgroups kept when the layout found dense routing
};

ScatterSplit scatter_split(const epl_problem &p, int64_t row_bytes)
{
    const int64_t T = p.num_tokens;
    if (T >= epl::kScatterGridFrom)
        return {1, xcd_grid(T, T), 0};
    // Long rows: kScatterGrid workgroups, of which the kernel keeps
    // kScatterGridLong when the layout found the batch's first slots densely
    // routed (WsHeader::dense; the measured best for rows with many
    // destinations, while rows with one or two, as on a receive side, run
    // faster with the whole grid)
    const bool long_rows = row_bytes >= epl::kScatterLongRowBytes;
    if (long_rows && T >= epl::kScatterGridLong)
        return {1, xcd_grid(std::min<int64_t>(T, epl::kScatterGrid), epl::kScatterGrid),
                epl::kScatterGridLong};
    if (!long_rows && T >= epl::kScatterGrid)
        return {1, row_grid(T, epl::kScatterGrid), 0};
    const int64_t nvec = row_bytes / 16;
    const int64_t by_items = (epl::kScatterSmallItems + T - 1) / std::max<int64_t>(T, 1);
    const int64_t by_width = nvec / epl::kScatterThreads;
    const int parts = (int)std::max<int64_t>(
        1, std::min<int64_t>({(int64_t)epl::kScatterMaxParts, by_items, by_width}));
    return {parts, xcd_grid(T * parts, T * parts), 0};
}

// The scan's work done by the scatter of a dispatch (epl::ScanInScatter):
// for layouts of several blocks whose per-block count matrix every
// workgroup of a striding scatter grid can read (at most
// EPL_SCAN_IN_SCATTER_ENTRIES words), with the LDS rows of per-block
// offsets that one workgroup's token range needs. Saves the scan launch
// between layout and scatter. 0 turns it off.
#ifndef EPL_SCAN_IN_SCATTER_ENTRIES
#define EPL_SCAN_IN_SCATTER_ENTRIES 16384
#endif
// At most this many LDS rows of per-block offsets per workgroup (blocks
// beyond them are summed from the count matrix by the slot's own thread).
#ifndef EPL_SCAN_IN_SCATTER_ROWS
#define EPL_SCAN_IN_SCATTER_ROWS 64
#endif
constexpr size_t kScanInScatterLds = 32768;

struct ScanPlan {
    bool on = false;
    int nbl = 0;        // LDS rows of per-block offsets
    size_t lds = 0;     // dynamic LDS bytes
};

ScanPlan scan_in_scatter(const epl_problem &p, const WsLayout &w, const ScatterSplit &sp)
{
    ScanPlan plan;
    const int64_t T = p.num_tokens, E = p.num_experts, nb = w.num_blocks;
    if (fused_layout(p) || T == 0 || nb == 0 || sp.parts != 1 ||
        sp.grid > (unsigned)epl::kScatterGrid || nb * E > EPL_SCAN_IN_SCATTER_ENTRIES)
        return plan;
    // the kernel reads the count matrix in 16-byte pieces: E / 4 expert
    // quads, each over kScatterThreads / (E / 4) segments of at most 16 blocks
    if (E % 4 != 0 || E / 4 > epl::kScatterThreads)
        return plan;
    const int64_t segs = epl::kScatterThreads / (E / 4);
    if ((nb + segs - 1) / segs > 16)
        return plan;
    // Blocks one workgroup's tokens can touch (the kernel's token_range):
    // with the XCD-aware ranges tokens of a contiguous eighth of the batch,
    // per = ceil(T / 8) tokens, which meet at most ceil((per - 1) / B) + 1
    // blocks of B tokens; else any block.
    int64_t nbl = nb;
    if (EPL_XCD_MAP && sp.grid % epl::kNumXcd == 0 && sp.grid >= (unsigned)epl::kNumXcd &&
        (int64_t)sp.grid < EPL_SCATTER_XCD_BELOW) {
        const int64_t per = (T + epl::kNumXcd - 1) / epl::kNumXcd;
        nbl = std::min<int64_t>(nb, (per - 1 + w.block_tokens - 1) / w.block_tokens + 1);
    }
    nbl = std::min<int64_t>(nbl, EPL_SCAN_IN_SCATTER_ROWS);
    const size_t lds = ((size_t)(2 + nbl) * (size_t)E + epl::kScanSegWords) * 4;
    if (lds > kScanInScatterLds)
        return plan;
    plan.on = true;
    plan.nbl = (int)nbl;
    plan.lds = lds;
    return plan;
}

// Where the scatter of a dispatch stores the scan's results.
struct ScanOuts {
    int32_t *cnt, *per_rank, *per_node, *start, *total_mapped;
};

template <int VPT>
void launch_scatter(const epl_problem &p, const WsLayout &w, const RowArgs &ra,
                    const int64_t *topk, const int32_t *start, void *ws, int64_t cap,
                    int32_t *m_idx, int32_t *oi, const ScatterSplit &sp, const ScanPlan &plan,
                    const ScanOuts &so, hipStream_t s)
{
    const bool vec16 = ra.scale_mode == epl::kScaleRows && ra.words % 4 == 0 &&
                       aligned(ra.x_scale, 16) && aligned(ra.out_scale, 16);
    epl::ScanInScatter sc{};
    if (plan.on) {
        sc.block_count = at<const int32_t>(ws, w.block_count);
        sc.block_rank = at<const int32_t>(ws, w.block_rank);
        sc.block_err = at<const uint32_t>(ws, w.block_err);
        sc.nb = w.num_blocks;
        sc.R = p.num_ranks;
        sc.Rn = nodes_of(p);
        sc.nbl = plan.nbl;
        sc.cnt = so.cnt;
        sc.per_rank = so.per_rank;
        sc.per_node = so.per_node;
        sc.start = so.start;
        sc.ws_counts = at<int32_t>(ws, w.counts);
        sc.block_base = at<int32_t>(ws, w.block_base);
        sc.hdr = at<WsHeader>(ws, 0);
        sc.total_out = so.total_mapped;
    }
    auto kernel = plan.on ? epl::ep_scatter_kernel<VPT, false, true>
                  : sp.parts > 1 ? epl::ep_scatter_kernel<VPT, true, false>
                                 : epl::ep_scatter_kernel<VPT, false, false>;
    hipLaunchKernelGGL(kernel, dim3(sp.grid), dim3(epl::kScatterThreads), plan.lds, s, ra.x,
                       ra.row_bytes, ra.scale_mode, ra.x_scale, ra.words, vec16,
                       ra.scale_ld, topk, start, at<const int32_t>(ws, w.block_base),
                       at<const int32_t>(ws, w.slot_rank), p.num_tokens, p.num_topk,
                       p.num_experts, w.block_tokens, alignment_of(p),
                       at<const int32_t>(ws, w.counts), cap, sp.parts,
                       (int64_t)sp.grid < EPL_SCATTER_XCD_BELOW, ra.out, ra.out_scale, m_idx, oi,
                       &at<WsHeader>(ws, 0)->status, sc,
                       sp.grid_dense > 0 ? &at<WsHeader>(ws, 0)->dense : nullptr, sp.grid_dense);
}

// The scatter launch. With plan.on (a dispatch whose scan launch was left
// out, see scan_in_scatter) it also does the scan's work and stores its
// results where `outs` says; else the scan has run before it.
int enqueue_scatter(const epl_problem &p, const WsLayout &w, const RowArgs &ra,
                    const int64_t *topk, const int32_t *start, void *ws, int64_t cap,
                    int32_t *m_idx, int32_t *oi, hipStream_t s, const ScanPlan &plan = ScanPlan{},
                    const ScanOuts &outs = ScanOuts{})
{
    if (p.num_tokens == 0)
        return EPL_OK;
    const ScatterSplit sp = scatter_split(p, ra.row_bytes);
    const int64_t nvec = ra.row_bytes / 16;
    const int64_t pvec = (nvec + sp.parts - 1) / sp.parts;
    const int vpt = (int)std::min<int64_t>(8, (pvec + epl::kScatterThreads - 1) / epl::kScatterThreads);
    switch (std::max(vpt, 1)) {
#define EPL_SCATTER_CASE(V)                                                                        \
    case V:                                                                                        \
        launch_scatter<V>(p, w, ra, topk, start, ws, cap, m_idx, oi, sp, plan, outs, s);           \
        break;
        EPL_SCATTER_CASE(1)
        EPL_SCATTER_CASE(2)
        EPL_SCATTER_CASE(3)
        EPL_SCATTER_CASE(4)
        EPL_SCATTER_CASE(5)
        EPL_SCATTER_CASE(6)
        EPL_SCATTER_CASE(7)
        EPL_SCATTER_CASE(8)
#undef EPL_SCATTER_CASE
    default:
        return EPL_EINVAL;
    }
    return launch_status();
}

RowArgs bf16_rows(const epl_problem &p, const uint16_t *x, const float *xs, uint16_t *out,
                  float *out_scale)
{
    return RowArgs{reinterpret_cast<const uint8_t *>(x), 2 * (int64_t)p.hidden,
                   p.scale_cols > 0 ? epl::kScaleRows : epl::kScaleNone,
                   reinterpret_cast<const uint32_t *>(xs), p.scale_cols, 0,
                   reinterpret_cast<uint8_t *>(out), reinterpret_cast<uint32_t *>(out_scale)};
}

// FP8 rows: H bytes; scales per the caller's format (see epl.h).
RowArgs fp8_rows(const epl_problem &p, const uint8_t *x, const void *xs, int scale_format,
                 int64_t cap, uint8_t *out, void *out_scale)
{
    RowArgs ra{x, (int64_t)p.hidden, epl::kScaleNone, static_cast<const uint32_t *>(xs), 0, cap,
               out, static_cast<uint32_t *>(out_scale)};
    if (scale_format == EPL_SCALE_F32) {
        ra.scale_mode = epl::kScaleRows;
        ra.words = p.scale_cols;
    } else if (scale_format == EPL_SCALE_UE8M0) {
        ra.scale_mode = epl::kScaleCols;
        ra.words = (p.scale_cols + 3) / 4;
    }
    return ra;
}

// Decode-sized dispatches (fused_layout) in one launch: workgroup 0 lays
// out and scans, workgroups 1 .. T place and copy one token each
// (epl::ep_dispatch_decode_kernel). 0 turns it off (layout + scan launch,
// then the scatter launch).
#ifndef EPL_DECODE_DISPATCH
#define EPL_DECODE_DISPATCH 1
#endif

int enqueue_decode_dispatch(const epl_problem &p, const WsLayout &w, const RowArgs &ra,
                            const int64_t *topk, int64_t cap, uint8_t *in_rank, int32_t *cnt,
                            int32_t *per_rank, int32_t *per_node, int32_t *start,
                            int32_t *total_host, int32_t *m_idx, int32_t *oi, void *ws,
                            hipStream_t s)
{
    int32_t *mapped = mapped_host_word(total_host);
    const epl::LayoutScanArgs a =
        layout_scan_args(p, w, topk, in_rank, cnt, per_rank, per_node, start, ws, mapped, cap);
    epl::DecodeRows d{};
    d.x = ra.x;
    d.row_bytes = ra.row_bytes;
    d.scale_mode = ra.scale_mode;
    d.x_scale = ra.x_scale;
    d.W = ra.words;
    d.scale_vec16 = ra.scale_mode == epl::kScaleRows && ra.words % 4 == 0 &&
                    aligned(ra.x_scale, 16) && aligned(ra.out_scale, 16);
    d.scale_ld = ra.scale_ld;
    d.capacity = cap;
    d.out = ra.out;
    d.out_scale = ra.out_scale;
    d.m_indices = m_idx;
    d.output_index = oi;
    hipLaunchKernelGGL(epl::ep_dispatch_decode_kernel, dim3((unsigned)(p.num_tokens + 1)),
                       dim3(epl::kFusedThreads), 0, s, a, d);
    int rc = launch_status();
    if (rc == EPL_OK && total_host && !mapped) {
        if (hipMemcpyAsync(total_host, &at<WsHeader>(ws, 0)->total, sizeof(int32_t),
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            rc = EPL_EHIP;
    }
    return rc;
}

// Pointer checks shared by the scatter entry points.
bool rows_args_ok(const epl_problem &p, const RowArgs &ra, const int64_t *topk, int64_t cap,
                  int32_t *m_idx, int32_t *oi)
{
    const bool any_tokens = p.num_tokens > 0;
    if (cap < 0 || ra.row_bytes % 16 != 0)
        return false;
    if (any_tokens && (!topk || !aligned(topk, 8) || !oi || !aligned(oi, 4) || !ra.x ||
                       !aligned(ra.x, 16)))
        return false;
    if (cap > 0 && (!ra.out || !aligned(ra.out, 16) || !m_idx || !aligned(m_idx, 4)))
        return false;
    if (ra.scale_mode != epl::kScaleNone) {
        if (ra.words < 1)
            return false;
        if (any_tokens && (!ra.x_scale || !aligned(ra.x_scale, 4)))
            return false;
        if (cap > 0 && (!ra.out_scale || !aligned(ra.out_scale, 4)))
            return false;
    }
    return true;
}

// The per-node output is required (and 4-byte aligned) exactly when the
// problem spans several nodes.
bool per_node_ok(const epl_problem &p, const int32_t *per_node)
{
    return nodes_of(p) == 0 || (per_node && aligned(per_node, 4));
}

// Low-latency problems: scales are produced (H % 128 == 0, S = H / 128), no
// alignment, T a whole number of segments of M tokens, row ids int32.
bool ll_ok(const epl_problem *p, int32_t M, int64_t cap)
{
    if (!problem_ok(p) || p->hidden % 128 != 0 || p->scale_cols != p->hidden / 128)
        return false;
    if (p->expert_alignment > 1 || M < 1 || p->num_tokens % M != 0 || cap < 0)
        return false;
    return (int64_t)p->num_experts * cap <= (int64_t)INT32_MAX;
}

// Decode-sized low-latency dispatches (at most kLLDecodeMaxSlots slots, and
// at most kLLDecodeMaxCounts (segment, expert) counters, whose 56 KB of LDS
// keep the workgroup within 64 KB) in one launch (epl::ep_ll_decode_kernel).
// 0 turns it off (layout, reduction and cast launches).
#ifndef EPL_LL_DECODE
#define EPL_LL_DECODE 1
#endif
constexpr int64_t kLLDecodeMaxCounts = 14336;

bool ll_decode(const epl_problem &p, int32_t M)
{
    return EPL_LL_DECODE && p.num_tokens >= 1 &&
           p.num_tokens * (int64_t)p.num_topk <= epl::kLLDecodeMaxSlots &&
           (p.num_tokens / M) * (int64_t)p.num_experts <= kLLDecodeMaxCounts;
}

// Low-latency dispatches of 1 to EPL_LL_SUMMED_BLOCKS layout blocks run no
// reduction launch: the cast kernel sums the per-block offsets it needs from
// the layout's per-block counts (ep_ll_scatter_kernel, SUMMED). Without
// tokens the reduction still runs: it is what resets the status word then.
// 0 turns it off.
#ifndef EPL_LL_SUMMED_BLOCKS
#define EPL_LL_SUMMED_BLOCKS 64
#endif

// (Column parts per row of the low-latency cast kernel, at most; 1 turns
// them off.)
#ifndef EPL_LL_MAX_PARTS
#define EPL_LL_MAX_PARTS 8
#endif

bool ll_summed(const WsLayout &w)
{
    return w.num_blocks >= 1 && w.num_blocks <= EPL_LL_SUMMED_BLOCKS;
}

template <int VPT>
void launch_ll_scatter(const epl_problem &p, const WsLayout &w, int32_t M, int64_t cap,
                       const uint16_t *x, const int64_t *topk, void *ws, uint8_t *out,
                       float *out_scale, int32_t *recv_count, int32_t *src_info,
                       int32_t *layout_range, int32_t *output_index, hipStream_t s)
{
    // kLLGrid workgroups striding over the items (fewer with fewer items),
    // and at least enough for the recv_count / layout_range entries (also
    // when there are no tokens). With fewer tokens than kLLGrid each row is
    // cut into column parts (whole 128-column groups, at most
    // EPL_LL_MAX_PARTS), so that about kLLGrid (token, part) items exist.
    int parts = 1;
    if (p.num_tokens > 0 && p.num_tokens < epl::kLLGrid)
        parts = (int)std::min<int64_t>({(int64_t)EPL_LL_MAX_PARTS, p.hidden / 128,
                                        (epl::kLLGrid + p.num_tokens - 1) / p.num_tokens});
    const int64_t items = p.num_tokens * parts;
    const int64_t entries = (int64_t)p.num_experts * std::max<int64_t>(1, p.num_tokens / M);
    const int64_t need = (entries + epl::kScatterThreads - 1) / epl::kScatterThreads;
    const unsigned grid =
        xcd_grid(std::max<int64_t>(std::min<int64_t>(items, epl::kLLGrid), need), 1 << 30);
    auto kernel = ll_summed(w) ? epl::ep_ll_scatter_kernel<VPT, true>
                               : epl::ep_ll_scatter_kernel<VPT, false>;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(epl::kScatterThreads), 0, s,
                       x, p.hidden, topk, at<const int32_t>(ws, w.block_base),
                       at<const int32_t>(ws, w.slot_rank), at<const int32_t>(ws, w.counts),
                       p.num_tokens, p.num_topk, p.num_experts, w.block_tokens, M, cap, out,
                       out_scale, recv_count, src_info, layout_range, output_index,
                       &at<WsHeader>(ws, 0)->status, at<const int32_t>(ws, w.block_count),
                       at<const uint32_t>(ws, w.block_err), w.num_blocks, parts);
}

// The workspace of epl_dispatch_static: a device array that the library
// holds on every GPU it runs on until the process ends, for callers that
// cannot allocate. The dispatch writes every byte of it that it later reads,
// so no part needs to start at zero. In host code `scratch` only stands for
// the symbol: its device address on each GPU comes from hipGetSymbolAddress
// (taken once per device, with that device current) and only that address is
// handed to kernels.
constexpr size_t kStaticWorkspaceBytes = size_t(8) << 20;
static_assert(kStaticWorkspaceBytes == EPL_STATIC_WORKSPACE_BYTES, "header and library agree");
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// This GPU's copy of `scratch` (the current device's), looked up on the
// device's first call.
int static_workspace(void **ws)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return EPL_EHIP;
    if (dev < 0 || dev >= kMaxDevices)
        return EPL_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr ||
            !aligned(ptr, kWsAlign)) {
            (void)hipGetLastError();
            return EPL_EHIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *ws = g_scratch_ptr[dev];
    return EPL_OK;
}

}  // namespace

extern "C" {

int epl_version(void) { return 0x000300; }

int epl_validate(const epl_problem *p) { return problem_ok(p) ? EPL_OK : EPL_EINVAL; }

int64_t epl_capacity_rows(const epl_problem *p) { return problem_ok(p) ? capacity_bound(*p) : -1; }

size_t epl_workspace_bytes(const epl_problem *p)
{
    if (!problem_ok(p))
        return 0;
    return ws_layout(*p).bytes;
}

const char *epl_strerror(int code)
{
    switch (code) {
    case EPL_OK:
        return "success";
    case EPL_EINVAL:
        return "invalid argument (problem, pointer, alignment or size)";
    case EPL_ERANGE:
        return "index out of range (topk id outside [-1, E) or output_index beyond expert rows)";
    case EPL_ECAPACITY:
        return "routed rows exceed the capacity of the output buffers";
    case EPL_EHIP:
        return "HIP runtime error";
    default:
        return "unknown status code";
    }
}

int epl_layout(const epl_problem *p, const int64_t *topk_idx, int32_t *num_tokens_per_expert,
               int32_t *num_tokens_per_rank, int32_t *num_tokens_per_rdma_rank,
               uint8_t *is_token_in_rank, void *workspace, void *stream)
{
    if (!problem_ok(p))
        return EPL_EINVAL;
    if (!workspace || !aligned(workspace, kWsAlign) || !num_tokens_per_expert ||
        !aligned(num_tokens_per_expert, 4) || !num_tokens_per_rank || !aligned(num_tokens_per_rank, 4))
        return EPL_EINVAL;
    if (!per_node_ok(*p, num_tokens_per_rdma_rank))
        return EPL_EINVAL;
    if (p->num_tokens > 0 && (!topk_idx || !aligned(topk_idx, 8) || !is_token_in_rank))
        return EPL_EINVAL;
    const WsLayout w = ws_layout(*p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fused_layout(*p))
        return enqueue_fused(*p, w, topk_idx, is_token_in_rank, num_tokens_per_expert,
                             num_tokens_per_rank, nodes_of(*p) ? num_tokens_per_rdma_rank : nullptr,
                             nullptr, nullptr, workspace, s);
    int rc = enqueue_layout(*p, w, topk_idx, is_token_in_rank, workspace, s);
    if (rc != EPL_OK)
        return rc;
    return enqueue_scan(*p, w, epl::kScanReduce, num_tokens_per_expert, num_tokens_per_rank,
                        nodes_of(*p) ? num_tokens_per_rdma_rank : nullptr, nullptr, nullptr,
                        workspace, s);
}

int epl_scan(const epl_problem *p, const int32_t *num_tokens_per_expert, int32_t *expert_start_loc,
             int32_t *total_host, void *workspace, void *stream)
{
    if (!problem_ok(p))
        return EPL_EINVAL;
    if (!workspace || !aligned(workspace, kWsAlign) || !num_tokens_per_expert ||
        !aligned(num_tokens_per_expert, 4) || !expert_start_loc || !aligned(expert_start_loc, 4) ||
        (total_host && !aligned(total_host, 4)))
        return EPL_EINVAL;
    const WsLayout w = ws_layout(*p);
    return enqueue_scan(*p, w, epl::kScanPrefix, const_cast<int32_t *>(num_tokens_per_expert),
                        nullptr, nullptr, expert_start_loc, total_host, workspace,
                        static_cast<hipStream_t>(stream));
}

int epl_scatter(const epl_problem *p, const uint16_t *x, const float *x_scale,
                const int64_t *topk_idx, const int32_t *expert_start_loc, void *workspace,
                int64_t capacity_rows, uint16_t *out, float *out_scale, int32_t *m_indices,
                int32_t *output_index, void *stream)
{
    if (!problem_ok(p))
        return EPL_EINVAL;
    if (!workspace || !aligned(workspace, kWsAlign) || !expert_start_loc ||
        !aligned(expert_start_loc, 4))
        return EPL_EINVAL;
    const RowArgs ra = bf16_rows(*p, x, x_scale, out, out_scale);
    if (!rows_args_ok(*p, ra, topk_idx, capacity_rows, m_indices, output_index))
        return EPL_EINVAL;
    const WsLayout w = ws_layout(*p);
    return enqueue_scatter(*p, w, ra, topk_idx, expert_start_loc, workspace, capacity_rows,
                           m_indices, output_index, static_cast<hipStream_t>(stream));
}

int epl_scatter_fp8(const epl_problem *p, const uint8_t *x, const void *x_scale, int scale_format,
                    const int64_t *topk_idx, const int32_t *expert_start_loc, void *workspace,
                    int64_t capacity_rows, uint8_t *out, void *out_scale, int32_t *m_indices,
                    int32_t *output_index, void *stream)
{
    if (!fp8_problem_ok(p, scale_format))
        return EPL_EINVAL;
    if (!workspace || !aligned(workspace, kWsAlign) || !expert_start_loc ||
        !aligned(expert_start_loc, 4))
        return EPL_EINVAL;
    const RowArgs ra = fp8_rows(*p, x, x_scale, scale_format, capacity_rows, out, out_scale);
    if (!rows_args_ok(*p, ra, topk_idx, capacity_rows, m_indices, output_index))
        return EPL_EINVAL;
    const WsLayout w = ws_layout(*p);
    return enqueue_scatter(*p, w, ra, topk_idx, expert_start_loc, workspace, capacity_rows,
                           m_indices, output_index, static_cast<hipStream_t>(stream));
}

// layout + scan + scatter on one stream, shared by both payload types
static int dispatch_rows(const epl_problem *p, const int64_t *topk_idx, const RowArgs &ra,
                         int64_t capacity_rows, int32_t *num_tokens_per_expert,
                         int32_t *num_tokens_per_rank, int32_t *num_tokens_per_rdma_rank,
                         uint8_t *is_token_in_rank, int32_t *expert_start_loc,
                         int32_t *total_host, int32_t *m_indices, int32_t *output_index,
                         void *workspace, void *stream)
{
    if (!workspace || !aligned(workspace, kWsAlign) || !num_tokens_per_expert ||
        !aligned(num_tokens_per_expert, 4) || !num_tokens_per_rank ||
        !aligned(num_tokens_per_rank, 4) || !expert_start_loc || !aligned(expert_start_loc, 4) ||
        (total_host && !aligned(total_host, 4)))
        return EPL_EINVAL;
    if (p->num_tokens > 0 && !is_token_in_rank)
        return EPL_EINVAL;
    if (!per_node_ok(*p, num_tokens_per_rdma_rank))
        return EPL_EINVAL;
    if (!rows_args_ok(*p, ra, topk_idx, capacity_rows, m_indices, output_index))
        return EPL_EINVAL;
    const WsLayout w = ws_layout(*p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t *per_node = nodes_of(*p) ? num_tokens_per_rdma_rank : nullptr;
    if (EPL_DECODE_DISPATCH && fused_layout(*p))
        return enqueue_decode_dispatch(*p, w, ra, topk_idx, capacity_rows, is_token_in_rank,
                                       num_tokens_per_expert, num_tokens_per_rank, per_node,
                                       expert_start_loc, total_host, m_indices, output_index,
                                       workspace, s);
    const ScanPlan plan = scan_in_scatter(*p, w, scatter_split(*p, ra.row_bytes));
    int rc;
    if (fused_layout(*p)) {
        rc = enqueue_fused(*p, w, topk_idx, is_token_in_rank, num_tokens_per_expert,
                           num_tokens_per_rank, per_node, expert_start_loc, total_host,
                           workspace, s);
    } else {
        rc = enqueue_layout(*p, w, topk_idx, is_token_in_rank, workspace, s);
        if (rc == EPL_OK && !plan.on)
            rc = enqueue_scan(*p, w, epl::kScanReduce | epl::kScanPrefix, num_tokens_per_expert,
                              num_tokens_per_rank, per_node, expert_start_loc, total_host,
                              workspace, s);
    }
    if (rc != EPL_OK)
        return rc;
    if (!plan.on)
        return enqueue_scatter(*p, w, ra, topk_idx, expert_start_loc, workspace, capacity_rows,
                               m_indices, output_index, s);
    int32_t *mapped = mapped_host_word(total_host);
    rc = enqueue_scatter(*p, w, ra, topk_idx, nullptr, workspace, capacity_rows, m_indices,
                         output_index, s, plan,
                         ScanOuts{num_tokens_per_expert, num_tokens_per_rank, per_node,
                                  expert_start_loc, mapped});
    if (rc == EPL_OK && total_host && !mapped) {
        if (hipMemcpyAsync(total_host, &at<WsHeader>(workspace, 0)->total, sizeof(int32_t),
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            rc = EPL_EHIP;
    }
    return rc;
}

int epl_dispatch(const epl_problem *p, const int64_t *topk_idx, const uint16_t *x,
                 const float *x_scale, int64_t capacity_rows, int32_t *num_tokens_per_expert,
                 int32_t *num_tokens_per_rank, int32_t *num_tokens_per_rdma_rank,
                 uint8_t *is_token_in_rank, int32_t *expert_start_loc, int32_t *total_host,
                 uint16_t *out, float *out_scale,
                 int32_t *m_indices, int32_t *output_index, void *workspace, void *stream)
{
    if (!problem_ok(p))
        return EPL_EINVAL;
    return dispatch_rows(p, topk_idx, bf16_rows(*p, x, x_scale, out, out_scale), capacity_rows,
                         num_tokens_per_expert, num_tokens_per_rank, num_tokens_per_rdma_rank,
                         is_token_in_rank, expert_start_loc, total_host, m_indices, output_index,
                         workspace, stream);
}

int epl_dispatch_static(const epl_problem *p, const int64_t *topk_idx, const uint16_t *x,
                        const float *x_scale, int64_t capacity_rows,
                        int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                        int32_t *num_tokens_per_rdma_rank, uint8_t *is_token_in_rank,
                        int32_t *expert_start_loc, int32_t *total_host, uint16_t *out,
                        float *out_scale, int32_t *m_indices, int32_t *output_index,
                        void **workspace_used, void *stream)
{
    // host checks first: nothing touches the GPU for a problem that does not fit
    if (!problem_ok(p) || ws_layout(*p).bytes > kStaticWorkspaceBytes)
        return EPL_EINVAL;
    void *ws = nullptr;
    const int rc = static_workspace(&ws);
    if (rc != EPL_OK)
        return rc;
    if (workspace_used)
        *workspace_used = ws;
    return dispatch_rows(p, topk_idx, bf16_rows(*p, x, x_scale, out, out_scale), capacity_rows,
                         num_tokens_per_expert, num_tokens_per_rank, num_tokens_per_rdma_rank,
                         is_token_in_rank, expert_start_loc, total_host, m_indices, output_index,
                         ws, stream);
}

int epl_dispatch_fp8(const epl_problem *p, const int64_t *topk_idx, const uint8_t *x,
                     const void *x_scale, int scale_format, int64_t capacity_rows,
                     int32_t *num_tokens_per_expert, int32_t *num_tokens_per_rank,
                     int32_t *num_tokens_per_rdma_rank, uint8_t *is_token_in_rank,
                     int32_t *expert_start_loc, int32_t *total_host, uint8_t *out,
                     void *out_scale, int32_t *m_indices, int32_t *output_index,
                     void *workspace, void *stream)
{
    if (!fp8_problem_ok(p, scale_format))
        return EPL_EINVAL;
    return dispatch_rows(p, topk_idx,
                         fp8_rows(*p, x, x_scale, scale_format, capacity_rows, out, out_scale),
                         capacity_rows, num_tokens_per_expert, num_tokens_per_rank,
                         num_tokens_per_rdma_rank, is_token_in_rank, expert_start_loc, total_host,
                         m_indices, output_index, workspace, stream);
}

size_t epl_ll_workspace_bytes(const epl_problem *p, int32_t tokens_per_segment)
{
    if (!ll_ok(p, tokens_per_segment, 0))
        return 0;
    return ws_layout(*p, ll_block_tokens(*p, tokens_per_segment)).bytes;
}

int epl_ll_dispatch(const epl_problem *p, int32_t tokens_per_segment, int64_t rows_per_expert,
                    const int64_t *topk_idx, const uint16_t *x, uint8_t *out, float *out_scale,
                    int32_t *recv_count, int32_t *src_info, int32_t *layout_range,
                    int32_t *output_index, void *workspace, void *stream)
{
    const int32_t M = tokens_per_segment;
    const int64_t cap = rows_per_expert;
    if (!ll_ok(p, M, cap))
        return EPL_EINVAL;
    if (!workspace || !aligned(workspace, kWsAlign) || !recv_count || !aligned(recv_count, 4))
        return EPL_EINVAL;
    if (p->num_tokens > 0 && (!topk_idx || !aligned(topk_idx, 8) || !x || !aligned(x, 16) ||
                              !output_index || !aligned(output_index, 4) || !layout_range ||
                              !aligned(layout_range, 4)))
        return EPL_EINVAL;
    if (cap > 0 && (!out || !aligned(out, 16) || !out_scale || !aligned(out_scale, 4) ||
                    !src_info || !aligned(src_info, 4)))
        return EPL_EINVAL;
    const WsLayout w = ws_layout(*p, ll_block_tokens(*p, M));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (ll_decode(*p, M)) {
        const epl::LLArgs a{x, (int)p->hidden, topk_idx, p->num_tokens, p->num_topk,
                            p->num_experts, M, cap, out, out_scale, recv_count, src_info,
                            layout_range, output_index, &at<WsHeader>(workspace, 0)->status};
        const size_t lds = sizeof(int32_t) * (size_t)(p->num_tokens / M) * p->num_experts;
        const bool wide = p->num_tokens * (int64_t)p->num_topk > epl::kFusedMaxSlots;
        auto kernel = wide ? epl::ep_ll_decode_kernel<epl::kLLDecodeMaxSlots / epl::kFusedThreads>
                           : epl::ep_ll_decode_kernel<epl::kFusedMaxSlots / epl::kFusedThreads>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)(1 + p->num_tokens)), dim3(epl::kFusedThreads),
                           lds, s, a);
        return launch_status();
    }
    int rc = enqueue_layout(*p, w, topk_idx, nullptr, workspace, s);
    if (rc == EPL_OK && !ll_summed(w))
        rc = enqueue_scan(*p, w, epl::kScanReduce, nullptr, nullptr, nullptr, nullptr, nullptr,
                          workspace, s);
    if (rc != EPL_OK)
        return rc;
    const int64_t npair = p->hidden / 16;     // 16 bf16 values per thread and step
    const int vpt = (int)std::min<int64_t>(8, (npair + epl::kScatterThreads - 1) / epl::kScatterThreads);
    switch (std::max(vpt, 1)) {
#define EPL_LL_CASE(V)                                                                             \
    case V:                                                                                        \
        launch_ll_scatter<V>(*p, w, M, cap, x, topk_idx, workspace, out, out_scale, recv_count,    \
                             src_info, layout_range, output_index, s);                             \
        break;
        EPL_LL_CASE(1)
        EPL_LL_CASE(2)
        EPL_LL_CASE(3)
        EPL_LL_CASE(4)
        EPL_LL_CASE(5)
        EPL_LL_CASE(6)
        EPL_LL_CASE(7)
        EPL_LL_CASE(8)
#undef EPL_LL_CASE
    default:
        return EPL_EINVAL;
    }
    return launch_status();
}

int epl_combine(const epl_problem *p, const uint16_t *expert_out, int64_t expert_rows,
                const int32_t *output_index, const float *topk_weights, int out_dtype, void *y,
                void *workspace, void *stream)
{
    if (!problem_ok(p))
        return EPL_EINVAL;
    if (out_dtype != EPL_OUT_F32 && out_dtype != EPL_OUT_BF16)
        return EPL_EINVAL;
    if (expert_rows < 0 || (workspace && !aligned(workspace, kWsAlign)))
        return EPL_EINVAL;
    if (p->num_tokens == 0)
        return EPL_OK;
    if (!output_index || !aligned(output_index, 4) || !topk_weights || !aligned(topk_weights, 4) ||
        !y || !aligned(y, 16) || (expert_rows > 0 && (!expert_out || !aligned(expert_out, 16))))
        return EPL_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *status = workspace ? &at<WsHeader>(workspace, 0)->status : nullptr;
    const bool bf16 = out_dtype == EPL_OUT_BF16;
    const int64_t y_bytes = p->num_tokens * (int64_t)p->hidden * (bf16 ? 2 : 4);
    const bool y_nt = y_bytes > epl::kYNtBytes;
    constexpr int th = epl::kCombineThreads;
    const bool few = p->num_tokens < epl::kCombineFewBelow;
    const int unroll = few ? epl::kCombineUnrollFew : epl::kCombineUnroll;
    // Column parts per token: as many as make one pass of the workgroup's
    // threads cover a part.
    const int64_t units = p->hidden / epl::combine_unit_cols(bf16);
    const int64_t per_pass = (int64_t)th * epl::combine_units_per_thread(bf16, unroll);
    const int parts =
        (int)std::max<int64_t>(1, std::min<int64_t>(epl::kCombineMaxParts, (units + per_pass - 1) / per_pass));
    const int64_t items = p->num_tokens * parts;
    const dim3 grid(xcd_grid(items, epl::kCombineGrid));
    const bool xcd_ranges = items < EPL_COMBINE_XCD_BELOW;
    auto launch = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, expert_out, expert_rows,
                           output_index, topk_weights, p->num_tokens, p->num_topk, p->hidden,
                           parts, xcd_ranges, y, status);
    };
    constexpr int u1 = epl::kCombineUnrollFew, u2 = epl::kCombineUnroll;
    if (bf16) {
        if (y_nt)
            few ? launch(epl::ep_combine_kernel<true, true, th, u1>, th)
                : launch(epl::ep_combine_kernel<true, true, th, u2>, th);
        else
            few ? launch(epl::ep_combine_kernel<true, false, th, u1>, th)
                : launch(epl::ep_combine_kernel<true, false, th, u2>, th);
    } else {
        if (y_nt)
            few ? launch(epl::ep_combine_kernel<false, true, th, u1>, th)
                : launch(epl::ep_combine_kernel<false, true, th, u2>, th);
        else
            few ? launch(epl::ep_combine_kernel<false, false, th, u1>, th)
                : launch(epl::ep_combine_kernel<false, false, th, u2>, th);
    }
    return launch_status();
}

int epl_expert_scale(const epl_problem *p, const uint16_t *rows_in, const int32_t *m_indices,
                     int64_t capacity_rows, uint16_t *rows_out, const void *workspace,
                     void *stream)
{
    if (!problem_ok(p) || capacity_rows < 0 || !workspace || !aligned(workspace, kWsAlign))
        return EPL_EINVAL;
    if (capacity_rows == 0)
        return EPL_OK;
    if (!rows_in || !aligned(rows_in, 16) || !rows_out || !aligned(rows_out, 16) || !m_indices ||
        !aligned(m_indices, 4))
        return EPL_EINVAL;
    const unsigned grid = (unsigned)std::min<int64_t>(capacity_rows, 1 << 16);
    hipLaunchKernelGGL(epl::ep_expert_scale_kernel, dim3(grid), dim3(epl::kRowThreads), 0,
                       static_cast<hipStream_t>(stream), rows_in, m_indices, capacity_rows,
                       static_cast<const WsHeader *>(workspace), p->hidden, rows_out);
    return launch_status();
}

int epl_status(const void *workspace, void *stream)
{
    if (!workspace || !aligned(workspace, kWsAlign))
        return EPL_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t st = 0;
    if (hipMemcpyAsync(&st, &static_cast<const WsHeader *>(workspace)->status, sizeof st,
                       hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return EPL_EHIP;
    if (st & (epl::kStatusBadExpert | epl::kStatusBadRow))
        return EPL_ERANGE;
    if (st & epl::kStatusCapacity)
        return EPL_ECAPACITY;
    return EPL_OK;
}

int64_t epl_total(const void *workspace, void *stream)
{
    if (!workspace || !aligned(workspace, kWsAlign))
        return EPL_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t total = 0;
    if (hipMemcpyAsync(&total, &static_cast<const WsHeader *>(workspace)->total, sizeof total,
                       hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return EPL_EHIP;
    return total;
}

}  // extern "C"
