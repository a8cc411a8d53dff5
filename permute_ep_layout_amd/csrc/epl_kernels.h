// Device kernels of libepl.so: MoE expert-parallel layout, scan, scatter and
// combine for gfx950 (CDNA4, 64-lane wavefronts). Host entry points that
// validate arguments and launch these kernels live in epl.hip.
//
// The four steps follow the problem statement of the pages:
//   layout  -- "[MoE] Deepseek的All-to-all通信: DeepEP代码解读", section
//              Dispatch (get_dispatch_layout: counts per expert and per rank,
//              token-in-rank mask, -1 = no selection);
//   scan    -- "高性能专家并行（EP）内核解剖学解读", high-throughput part,
//              subsection 5 (blocks laid out by a prefix sum starting at 0);
//   scatter -- "参考sglang代码，重构vllm021中EP高吞吐代码，消除空泡问题",
//              section 2.2 (ep_scatter: rows into expert-contiguous blocks,
//              scales, m_indices, output_index), section 3.3 (-1 markers);
//   combine -- the way back to token order, weighted by topk_weights
//              ("高性能专家并行（EP）内核解剖学解读", 任务设定与数据流).
// The low-latency variant (ep_ll_scatter_kernel) places rows into a fixed
// rectangle per expert instead (strategy A of the EP anatomy page, high-
// throughput part subsection 3; the receive buffers of the DeepEP page's
// low_latency section) and casts them to FP8 on the way.
//
// Determinism. Counts are integer sums, so atomics would already give exact
// counts; row positions are another matter. Here nothing about positions
// depends on timing: the layout kernel splits the tokens into fixed blocks
// and, inside a block, ranks every slot among the earlier slots of the same
// expert in (token, k) order with wavefront ballots; the scan kernel turns
// the per-block counts into per-block offsets (a prefix over blocks per
// expert); the scatter kernel adds expert offset + block offset + rank.
// For a dispatch of a few thousand tokens the scatter computes the offsets
// itself from the per-block counts (ScanInScatter), so no scan launch sits
// between layout and scatter. Decode-sized batches (at most 2048 slots) take
// ep_layout_scan_kernel in the layout / scan calls (one workgroup, one
// block) and ep_dispatch_decode_kernel in a dispatch (one launch, each token
// placed by its own workgroup from the routing of all slots); the
// low-latency dispatch does the same up to 4096 slots (ep_ll_decode_kernel)
// and, up to 64 layout blocks, sums its block offsets in the cast kernel
// instead of running the scan's reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace epl {

constexpr int kWave = 64;
constexpr int kLayoutThreads = 256;       // any number of experts
constexpr int kLayoutThreadsWide = 1024;  // when its per-wave counters fit in LDS
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kMaxSlotsPerBlock = 2048;   // B * K per layout block
constexpr int kMaxTopk = 64;
constexpr int kMaxExperts = 2048;
constexpr int kMaxAlignment = 65536;
constexpr int kScanThreads = 1024;
constexpr int kRowThreads = 128;          // expert-scale workgroup

// Launch shape of the two bandwidth kernels. Build-time knobs (-D...) so the
// shape can be swept on the target; the defaults are the measured best on
// MI355X for hidden 7168.
#ifndef EPL_SCATTER_THREADS
#define EPL_SCATTER_THREADS 128
#endif
#ifndef EPL_COMBINE_THREADS
#define EPL_COMBINE_THREADS 256
#endif
#ifndef EPL_COMBINE_UNROLL
#define EPL_COMBINE_UNROLL 2
#endif
#ifndef EPL_COMBINE_UNROLL_FEW
#define EPL_COMBINE_UNROLL_FEW 1
#endif
#ifndef EPL_COMBINE_FEW_BELOW
#define EPL_COMBINE_FEW_BELOW 8192
#endif
#ifndef EPL_SCATTER_GRID
#define EPL_SCATTER_GRID 1024
#endif
#ifndef EPL_SCATTER_GRID_FROM
#define EPL_SCATTER_GRID_FROM 8192
#endif
#ifndef EPL_SCATTER_GRID_LONG
#define EPL_SCATTER_GRID_LONG 512
#endif
#ifndef EPL_SCATTER_LONG_ROW_BYTES
#define EPL_SCATTER_LONG_ROW_BYTES 12288
#endif
#ifndef EPL_COMBINE_GRID
#define EPL_COMBINE_GRID (1 << 30)
#endif
constexpr int kScatterThreads = EPL_SCATTER_THREADS;
constexpr int kCombineThreads = EPL_COMBINE_THREADS;

// Status word bits (workspace header).
constexpr uint32_t kStatusBadExpert = 1u;      // topk id outside [-1, E)
constexpr uint32_t kStatusCapacity = 2u;       // routed rows > capacity rows
constexpr uint32_t kStatusBadRow = 4u;         // combine: output_index >= expert rows

constexpr int kScanReduce = 1;   // per-block counts -> per-block offsets, totals
constexpr int kScanPrefix = 2;   // totals -> expert_start_loc and N

struct WsHeader {
    uint32_t status;
    int32_t total;
    // 1 when at least half of the batch's first 64 slots name an expert
    // (dense routing, as in a global dispatch), 0 when most are -1 (a receive
    // side's local ids): the long-row scatter's grid size follows it
    int32_t dense;
    int32_t pad[61];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

// The dense-routing hint from the validity ballot of the first min(ns, 64)
// slots (bit i: slot i names an expert).
__device__ __forceinline__ int32_t dense_sample(uint64_t valid, int ns)
{
    return 2 * (int)__popcll(valid) >= min(ns, 64) ? 1 : 0;
}

__device__ __forceinline__ uint64_t wave_ballot(bool pred)
{
    return __builtin_amdgcn_ballot_w64(pred);
}

__device__ __forceinline__ int lane_id()
{
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Workgroup barrier that orders LDS accesses only. __syncthreads() also
// orders global memory, which on CDNA makes every wave wait for all of its
// outstanding global stores (they share the vmcnt counter with loads) before
// the barrier. No kernel here hands data between its threads through global
// memory (the outputs are read by later kernels), so every barrier is this
// one: the row kernels keep their stores streaming across tokens, and the
// layout and scan kernels do not wait for their own output stores (in the
// layout, waiting for the token->rank mask stores had cost ~5 us).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// --------------------------------------------------------------- layout --

// n / d for n, d < 2^16 without a division: the high word of n * magic with
// magic = ceil(2^32 / d) (the error n * (magic - 2^32/d) / 2^32 < 2^-16 stays
// below the 1/d distance to the next integer); d = 1 is the identity.
__host__ __device__ inline uint32_t div_magic(uint32_t d)
{
    return d > 1 ? (uint32_t)((((uint64_t)1 << 32) + d - 1) / d) : 0u;
}
__device__ __forceinline__ int div_small(uint32_t n, int d, uint32_t magic)
{
    return d > 1 ? (int)__umulhi(n, magic) : (int)n;
}

// Writes the 0/1 bytes of `n` (<= 64) mask bits to dst; `vec16` says that
// dst is 16-byte aligned and n is a multiple of 16.
__device__ __forceinline__ void store_mask_bytes(uint8_t *dst, uint64_t mask, int n, bool vec16)
{
    if (vec16) {
        for (int j = 0; j < n; j += 16) {
            uint32_t w[4];
            for (int q = 0; q < 4; ++q) {
                const uint32_t nib = (uint32_t)(mask >> (j + 4 * q)) & 0xFu;
                w[q] = (nib & 1u) | ((nib >> 1) & 1u) << 8 | ((nib >> 2) & 1u) << 16 |
                       ((nib >> 3) & 1u) << 24;
            }
            *reinterpret_cast<uint4 *>(dst + j) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        for (int j = 0; j < n; ++j)
            dst[j] = (uint8_t)((mask >> j) & 1u);
    }
}

// Dynamic LDS of the layout kernel for E experts, RC token-count columns
// (R ranks, then the nodes if asked for), B tokens of K slots. Kept <=
// kLayoutLdsBytes by the host's choice of B.
constexpr size_t kLayoutLdsBytes = 65536;
__host__ __device__ constexpr size_t layout_lds_bytes(int B, int K, int E, int RC,
                                                      int waves = kLayoutWaves)
{
    return sizeof(int32_t) * ((size_t)B * (K + 1) + (size_t)B * K   // keys (padded), ranks
                              + (size_t)waves * E             // running count per wave and expert
                              + (size_t)waves * ((E + 3) / 4) // per-chunk byte counters
                              + (size_t)RC + 1);              // tokens per rank / node, error flag
}

// One workgroup of THREADS threads (kLayoutThreads, or kLayoutThreadsWide
// when the per-wave counters fit) per block of B tokens (B <= THREADS, B * K <=
// kMaxSlotsPerBlock). Outputs: in_rank rows of the block's tokens;
// block_count[b][e] (slots of expert e in block b); block_rank[b][c] (tokens
// of block b sent to rank c for c < R, to node c - R for R <= c < R + Rn,
// a node being G consecutive ranks); block_err[b]; slot_rank[t*K+k] = rank
// of slot (t,k) among the block's earlier slots of the same expert, or -1
// for an invalid slot. Block 0 also clears the status word, for the
// kernels that only OR bits into it later in the chain, and stores the
// dense-routing hint (dense_sample).
template <int THREADS>
__global__ __launch_bounds__(THREADS) void ep_layout_kernel(
    const int64_t *__restrict__ topk, int64_t T, int K, int E, int R, int experts_per_rank,
    uint32_t epr_magic, int G, uint32_t node_magic, int Rn, int B, uint8_t *__restrict__ in_rank,
    bool in_rank_vec16,
    int32_t *__restrict__ block_count, int32_t *__restrict__ block_rank,
    uint32_t *__restrict__ block_err, int32_t *__restrict__ slot_rank,
    uint32_t *__restrict__ status, int32_t *__restrict__ dense)
{
    constexpr int WAVES = THREADS / kWave;
    extern __shared__ int32_t lds[];
    const int max_slots = B * K;
    const int cwords = (E + 3) / 4;
    // keys of slot s = (t, k) at t * (K + 1) + k: a token's K keys followed by
    // one unused word, so that in the mask step, where thread t reads its
    // token's keys, the lanes stride by K + 1 words, odd and so co-prime with
    // the LDS bank count (a stride of K = 8 words put a wave's lanes on a few
    // banks: 43 K of 72 K LDS-active cycles in bank conflicts at 4096 tokens
    // of top-8, 32 K of 61 K with the pad; the rest are the histogram and
    // rank-count atomics)
    const uint32_t kmagic = div_magic((uint32_t)K);
    auto kidx = [&](int s) { return s + div_small((uint32_t)s, K, kmagic); };
    int32_t *keys = lds;                                   // [B*(K+1)] key | owner << 16, or -1
    int32_t *lrank = keys + B * (K + 1);                   // [B*K] rank within the owning wave
    int32_t *wave_cnt = lrank + max_slots;                 // [waves][E]
    uint32_t *chunk_cnt = reinterpret_cast<uint32_t *>(wave_cnt + WAVES * E);  // [waves][E/4]
    int32_t *rank_cnt = reinterpret_cast<int32_t *>(chunk_cnt + WAVES * cwords); // [R+Rn]
    const int RC = R + Rn;
    int32_t *s_err = rank_cnt + RC;                        // [1]

    const int64_t b = blockIdx.x;
    const int64_t t0 = b * B;
    const int nt = (int)min((int64_t)B, T - t0);
    const int ns = nt * K;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;

    for (int i = tid; i < WAVES * E; i += THREADS)
        wave_cnt[i] = 0;
    for (int i = tid; i < WAVES * cwords; i += THREADS)
        chunk_cnt[i] = 0;
    for (int i = tid; i < RC; i += THREADS)
        rank_cnt[i] = 0;
    if (tid == 0)
        *s_err = 0;

    // Keys of the block's slots, in (token, k) order, packed with the owning
    // rank; bad ids become -1.
    const int64_t *src = topk + t0 * K;
    bool bad = false;
    for (int s = tid; s < ns; s += THREADS) {
        const int64_t e = src[s];
        int packed = -1;
        if (e >= 0 && e < E)
            packed = (int)e | (div_small((uint32_t)e, experts_per_rank, epr_magic) << 16);
        else if (e != -1)
            bad = true;
        keys[kidx(s)] = packed;
    }
    lds_barrier();
    if (bad)
        atomicOr(reinterpret_cast<uint32_t *>(s_err), 1u);

    // Rank of each slot among the earlier slots with the same key. Wave w
    // owns a contiguous run of 64-slot chunks and walks it in order. For a
    // chunk, each lane first counts its key in a per-wave byte histogram
    // (a key occurs at most 64 times in a chunk); lanes whose key occurs
    // once have in-chunk rank 0, and only the repeated keys go through the
    // ballot loop, where a lane's rank is the number of lower lanes holding
    // its key. Then every lane adds the wave's running count for its key, and
    // the lowest lane of each key advances that count and clears the byte.
    //
    // The mask step below does not depend on the ranks: in 1024-thread
    // blocks of at most 128 tokens the token waves (one thread per token)
    // do only the mask step and the other 14 or 15 waves rank, side by side
    // (layout kernel 7.4 -> 6.8 us at 4096 tokens of top-8, 6.0 -> 5.3 us
    // at 2048 tokens of top-6). With 256-token blocks (four token waves,
    // three chunks per ranking wave instead of two) it was 0.1-0.3 us slower.
    const int nchunks = (ns + kWave - 1) / kWave;
    const int mask_waves = (nt + kWave - 1) / kWave;
    const int rw0 = WAVES >= 8 && mask_waves <= 2 ? mask_waves : 0;   // first ranking wave
    const int cpw = (nchunks + (WAVES - rw0) - 1) / (WAVES - rw0);
    if (wave >= rw0) {
        int32_t *my_cnt = wave_cnt + wave * E;
        uint32_t *my_chunk = chunk_cnt + wave * cwords;
        const int rw = wave - rw0;
        const int c_end = min(nchunks, (rw + 1) * cpw);
        const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
        for (int c = rw * cpw; c < c_end; ++c) {
            const int s = c * kWave + lane;
            const int packed = (s < ns) ? keys[kidx(s)] : -1;
            const bool valid = packed >= 0;
            const int k16 = valid ? (packed & 0xFFFF) : 0;
            const int shift = 8 * (k16 & 3);
            if (valid)
                atomicAdd(&my_chunk[k16 >> 2], 1u << shift);
            const int group = valid ? (int)((my_chunk[k16 >> 2] >> shift) & 0xFFu) : 0;
            int rank = 0;
            uint64_t todo = wave_ballot(group > 1);
            while (todo) {
                const int leader = (int)__builtin_ctzll(todo);
                const int lkey = __builtin_amdgcn_readlane(k16, leader);
                const uint64_t same = wave_ballot(valid && k16 == lkey);
                if (valid && k16 == lkey)
                    rank = __popcll(same & lower);
                todo &= ~same;
            }
            if (valid) {
                const int base = my_cnt[k16];
                lrank[s] = base + rank;
                if (rank == 0) {
                    my_cnt[k16] = base + group;
                    atomicAnd(&my_chunk[k16 >> 2], ~(0xFFu << shift));
                }
            }
        }
    }

    // Token -> rank mask (one thread per token), tokens per rank and tokens
    // per node, one 64-wide window at a time. A token adds one to the count
    // of each rank (node) in its mask: at most K LDS atomics per token (a
    // ballot per rank had cost ~3.4 us at 32 ranks).
    if (tid < nt) {
        for (int w0 = 0; w0 < R; w0 += 64) {
            const int wr = min(64, R - w0);
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int packed = keys[tid * (K + 1) + k];
                if (packed >= 0) {
                    const int r = (packed >> 16) - w0;
                    if (r >= 0 && r < wr)
                        mask |= 1ull << r;
                }
            }
            if (in_rank)
                store_mask_bytes(in_rank + (t0 + tid) * R + w0, mask, wr, in_rank_vec16);
            for (uint64_t m = mask; m; m &= m - 1)
                atomicAdd(&rank_cnt[w0 + __builtin_ctzll(m)], 1);
        }
        // a token counts once for a node (G consecutive ranks) whichever of
        // its ranks it reaches; node = rank / G
        for (int n0 = 0; n0 < Rn; n0 += 64) {
            const int wn = min(64, Rn - n0);
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int packed = keys[tid * (K + 1) + k];
                if (packed >= 0) {
                    const int n = div_small((uint32_t)packed >> 16, G, node_magic) - n0;
                    if (n >= 0 && n < wn)
                        mask |= 1ull << n;
                }
            }
            for (uint64_t m = mask; m; m &= m - 1)
                atomicAdd(&rank_cnt[R + n0 + __builtin_ctzll(m)], 1);
        }
    }
    lds_barrier();

    // Per expert: exclusive prefix over the waves (in place) and block total.
    for (int e = tid; e < E; e += THREADS) {
        int run = 0;
        for (int w = 0; w < WAVES; ++w) {
            const int c = wave_cnt[w * E + e];
            wave_cnt[w * E + e] = run;
            run += c;
        }
        block_count[b * E + e] = run;
    }
    for (int r = tid; r < RC; r += THREADS)
        block_rank[b * RC + r] = rank_cnt[r];
    lds_barrier();
    if (tid == 0) {
        block_err[b] = (uint32_t)*s_err;
        if (b == 0)
            *status = 0u;
    }
    if (b == 0 && tid < kWave) {
        // the dense-routing hint from the batch's first 64 slots
        const uint64_t m = wave_ballot(tid < ns && keys[kidx(tid)] >= 0);
        if (tid == 0)
            *dense = dense_sample(m, ns);
    }

    for (int s = tid; s < ns; s += THREADS) {
        const int packed = keys[kidx(s)];
        const int w = rw0 + (s / kWave) / cpw;
        slot_rank[t0 * K + s] = packed >= 0 ? lrank[s] + wave_cnt[w * E + (packed & 0xFFFF)] : -1;
    }
}

// ----------------------------------------------------------------- scan --

// Inclusive prefix sum over a workgroup of THREADS threads (s_wave holds
// THREADS / 64 words).
template <int THREADS = kScanThreads>
__device__ __forceinline__ int block_inclusive_scan(int v, int *s_wave)
{
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d)
            v += o;
    }
    if (lane == kWave - 1)
        s_wave[wave] = v;
    lds_barrier();
    if (wave == 0) {
        constexpr int nw = THREADS / kWave;
        int x = lane < nw ? s_wave[lane] : 0;
        for (int d = 1; d < nw; d <<= 1) {
            const int o = __shfl_up(x, d, kWave);
            if (lane >= d)
                x += o;
        }
        if (lane < nw)
            s_wave[lane] = x;
    }
    lds_barrier();
    return v + (wave > 0 ? s_wave[wave - 1] : 0);
}

// Sums of one column segment [b0, b1) of a row-major [nb, ncols] matrix,
// loading 16 rows at a time so the loads of a batch are in flight together.
__device__ __forceinline__ int segment_sum(const int32_t *m, int ncols, int col, int64_t b0,
                                           int64_t b1)
{
    int sum = 0;
    for (int64_t bb = b0; bb < b1; bb += 16) {
        int v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] = (bb + j < b1) ? m[(bb + j) * ncols + col] : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            sum += v[j];
    }
    return sum;
}

// Single workgroup. kScanReduce: column sums of block_count / block_rank
// give num_tokens_per_expert / num_tokens_per_rank (and, for the Rn node
// columns after the R rank columns, num_tokens_per_rdma_rank), block_base
// receives the exclusive prefix of block_count over blocks (block_count
// itself stays as the layout wrote it), and the status word is reset to the
// layout's error bits. kScanPrefix: exclusive prefix of the per-expert block
// sizes (the counts, read from `cnt` unless kScanReduce produced them,
// rounded up to a multiple of `alignment`) into expert_start_loc, total into
// the header and, if `total_out` is not null, into that (host-mapped) word
// too. Either mode keeps a copy of the counts in `ws_counts` for the
// scatter's padding rows.
//
// The columns are split into P segments of L blocks each so that all 1024
// threads have work: thread (column, segment) sums its segment, a short
// per-column scan over the P segment sums gives each segment's offset, and
// the thread then rewrites its segment as a running prefix.
__global__ __launch_bounds__(kScanThreads) void ep_scan_kernel(
    int mode, int64_t nb, int E, int R, int Rn, int alignment,
    const int32_t *__restrict__ block_count, int32_t *__restrict__ block_base,
    const int32_t *__restrict__ block_rank, const uint32_t *__restrict__ block_err,
    int32_t *__restrict__ cnt, int32_t *__restrict__ per_rank, int32_t *__restrict__ per_node,
    int32_t *__restrict__ start,
    int32_t *__restrict__ ws_counts, WsHeader *__restrict__ hdr, int32_t *__restrict__ total_out)
{
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_seg[kMaxExperts];
    __shared__ int s_rseg[2 * kMaxExperts];   // rank and node column totals
    __shared__ int s_wave[kScanThreads / kWave];
    __shared__ uint32_t s_err;
    const int tid = threadIdx.x;

    if (mode & kScanReduce) {
        if (tid == 0)
            s_err = 0;
        // segments per column: enough to occupy the threads, but never more
        // than there are blocks (each segment sum is later added serially)
        const int P = (int)max((int64_t)1, min((int64_t)(E <= kScanThreads ? kScanThreads / E : 1), nb));
        const int64_t L = (nb + P - 1) / P;
        const int RC = R + Rn;      // rank columns, then node columns
        for (int r = tid; r < RC; r += kScanThreads)
            s_rseg[r] = 0;
        lds_barrier();
        // When every thread owns at most one segment of at most 16 blocks,
        // the segment stays in registers between the sum and the rewrite.
        const bool held = E * P <= kScanThreads && L <= 16;
        int seg[16];
        for (int col = tid; col < E * P; col += kScanThreads) {
            const int e = col % E, q = col / E;
            const int64_t b0 = q * L, b1 = min(nb, b0 + L);
            if (held) {
                int sum = 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    seg[j] = (b0 + j < b1) ? block_count[(b0 + j) * E + e] : 0;
                    sum += seg[j];
                }
                s_seg[q * E + e] = sum;
            } else {
                s_seg[q * E + e] = segment_sum(block_count, E, e, b0, b1);
            }
        }
        // Rank and node columns only need their totals: every element of
        // the [nb, RC] matrix is added into its column in LDS (integer adds,
        // exact in any order), four loads in flight per thread.
        const int64_t nrc = nb * RC;
        for (int64_t i0 = tid; i0 < nrc; i0 += 4 * kScanThreads) {
            int v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = i0 + (int64_t)j * kScanThreads;
                v[j] = i < nrc ? block_rank[i] : 0;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = i0 + (int64_t)j * kScanThreads;
                if (v[j])
                    atomicAdd(&s_rseg[i % RC], v[j]);
            }
        }
        uint32_t err = 0;
        for (int64_t bb = tid; bb < nb; bb += kScanThreads)
            err |= block_err[bb];
        lds_barrier();
        if (err)
            atomicOr(&s_err, err);
        if (E * P <= kScanThreads) {
            // Exclusive prefix over the P segments of each column, one
            // segment per thread (thread q * E + e): log2(P) steps of
            // Hillis-Steele in LDS instead of a serial walk of P dependent
            // LDS round trips (P is 117 for 8 experts over 117 blocks).
            const int col = tid, e = col % E, q = col / E;
            const bool mine = col < E * P;
            const int v = mine ? s_seg[col] : 0;
            int incl = v;
            for (int d = 1; d < P; d *= 2) {
                const int add = mine && q >= d ? s_seg[col - d * E] : 0;
                lds_barrier();
                incl += add;
                if (mine)
                    s_seg[col] = incl;
                lds_barrier();
            }
            if (mine) {
                s_seg[col] = incl - v;
                if (q == P - 1) {
                    s_cnt[e] = incl;
                    if (cnt)
                        cnt[e] = incl;
                    ws_counts[e] = incl;
                }
            }
        } else {
            for (int e = tid; e < E; e += kScanThreads) {
                int run = 0;
                for (int q = 0; q < P; ++q) {
                    const int v = s_seg[q * E + e];
                    s_seg[q * E + e] = run;
                    run += v;
                }
                s_cnt[e] = run;
                if (cnt)
                    cnt[e] = run;
                ws_counts[e] = run;
            }
        }
        for (int r = tid; r < RC; r += kScanThreads) {
            const int run = s_rseg[r];
            if (r < R) {
                if (per_rank)
                    per_rank[r] = run;
            } else if (per_node) {
                per_node[r - R] = run;
            }
        }
        lds_barrier();
        // block_base = exclusive prefix of block_count over blocks.
        for (int col = tid; col < E * P; col += kScanThreads) {
            const int e = col % E, q = col / E;
            const int64_t b0 = q * L, b1 = min(nb, b0 + L);
            int run = s_seg[q * E + e];
            if (held) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (b0 + j < b1) {
                        block_base[(b0 + j) * E + e] = run;
                        run += seg[j];
                    }
                }
                continue;
            }
            for (int64_t bb = b0; bb < b1; bb += 16) {
                int v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    v[j] = (bb + j < b1) ? block_count[(bb + j) * E + e] : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (bb + j < b1) {
                        block_base[(bb + j) * E + e] = run;
                        run += v[j];
                    }
                }
            }
        }
        if (tid == 0)
            hdr->status = s_err ? kStatusBadExpert : 0u;
    } else if (mode & kScanPrefix) {
        for (int e = tid; e < E; e += kScanThreads) {
            s_cnt[e] = cnt[e];
            ws_counts[e] = s_cnt[e];
        }
        lds_barrier();
    }

    if (mode & kScanPrefix) {
        // Two consecutive experts per thread (E <= 2 * kScanThreads).
        const int i0 = 2 * tid, i1 = 2 * tid + 1;
        auto block = [alignment](int c) { return (c + alignment - 1) / alignment * alignment; };
        const int a0 = i0 < E ? block(s_cnt[i0]) : 0;
        const int a1 = i1 < E ? block(s_cnt[i1]) : 0;
        const int incl = block_inclusive_scan(a0 + a1, s_wave);
        const int excl = incl - (a0 + a1);
        if (i0 < E)
            start[i0] = excl;
        if (i1 < E)
            start[i1] = excl + a0;
        if (tid == kScanThreads - 1) {
            hdr->total = incl;
            if (total_out)
                *total_out = incl;
        }
    }
}

// ------------------------------------------------- layout + scan, fused --

// Decode-sized batches (at most kFusedMaxSlots slots, kFusedMaxExperts experts
// and kFusedMaxCols rank + node columns) run layout and scan in one workgroup:
// the slots need no per-block offsets, so the per-block count matrix and the
// second launch that reduces it go away. The results are those of
// ep_layout_kernel + ep_scan_kernel with a single block of all T tokens:
// block_base (one row of E zeros), slot_rank = rank of slot (t, k) among
// all earlier slots of its expert, per-expert / per-rank / per-node counts,
// the token -> rank mask, the counts copy for the padding rows, the status
// word, and, if `start` is not null, expert_start_loc and N (header, and the
// caller's host-mapped word if `total_out` is not null).
//
// Ranking: wave w owns a contiguous run of 64-slot chunks and walks it in
// order, as in ep_layout_kernel; each lane keeps its chunks' keys and
// in-wave ranks in registers (at most kFusedChunksPerWave per lane), a
// prefix over the 16 waves per expert then turns them into global ranks.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;
// At DeepSeek-V3 dimensions (top-8 of 256 experts) one workgroup beats the
// two launches up to 2048 slots (dispatch 2.1-2.7 us faster at 64-256
// tokens), ties at 4096 and loses beyond (8192 slots: +4 us; 12288 slots
// at hidden 4096: layout 11 -> 30 us), as the waves walk their chunks in turn.
#ifndef EPL_FUSED_MAX_SLOTS
#define EPL_FUSED_MAX_SLOTS 2048
#endif
constexpr int kFusedMaxSlots = EPL_FUSED_MAX_SLOTS;
static_assert(kFusedMaxSlots % kFusedThreads == 0, "whole slots per thread");
constexpr int kFusedChunksPerWave = kFusedMaxSlots / kWave / kFusedWaves;
constexpr int kFusedMaxExperts = 256;
constexpr int kFusedMaxCols = 256;
static_assert(kFusedThreads == kScanThreads, "the fused kernel reuses the scan's block scan");

// Arguments of the one-workgroup layout + scan.
struct LayoutScanArgs {
    const int64_t *topk;
    int64_t T;
    int K, E, R, experts_per_rank;
    uint32_t epr_magic;
    int G;
    uint32_t node_magic;
    int Rn, alignment;
    uint8_t *in_rank;
    bool in_rank_vec16;
    int32_t *cnt, *per_rank, *per_node, *start, *block_base, *slot_rank, *ws_counts;
    WsHeader *hdr;
    int32_t *total_out;
    int64_t capacity;   // < 0: none; else N > capacity also sets the capacity bit
};

// The whole layout + scan by one workgroup of kFusedThreads threads (the
// body of ep_layout_scan_kernel, also run by workgroup 0 of
// ep_dispatch_decode_kernel).
__device__ __forceinline__ void layout_scan_block(const LayoutScanArgs &a)
{
    const int64_t *__restrict__ topk = a.topk;
    const int64_t T = a.T;
    const int K = a.K, E = a.E, R = a.R, experts_per_rank = a.experts_per_rank;
    const uint32_t epr_magic = a.epr_magic, node_magic = a.node_magic;
    const int G = a.G, Rn = a.Rn, alignment = a.alignment;
    uint8_t *__restrict__ in_rank = a.in_rank;
    const bool in_rank_vec16 = a.in_rank_vec16;
    int32_t *__restrict__ cnt = a.cnt;
    int32_t *__restrict__ per_rank = a.per_rank;
    int32_t *__restrict__ per_node = a.per_node;
    int32_t *__restrict__ start = a.start;
    int32_t *__restrict__ block_base = a.block_base;
    int32_t *__restrict__ slot_rank = a.slot_rank;
    int32_t *__restrict__ ws_counts = a.ws_counts;
    WsHeader *__restrict__ hdr = a.hdr;
    int32_t *__restrict__ total_out = a.total_out;
    __shared__ int32_t wave_cnt[kFusedWaves][kFusedMaxExperts];
    __shared__ uint32_t chunk_cnt[kFusedWaves][kFusedMaxExperts / 4];
    __shared__ int32_t rank_cnt[kFusedMaxCols];
    __shared__ int s_wave[kFusedWaves];
    __shared__ uint32_t s_err;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int ns = (int)(T * K);
    const int RC = R + Rn;

    for (int i = tid; i < kFusedWaves * kFusedMaxExperts; i += kFusedThreads)
        (&wave_cnt[0][0])[i] = 0;
    for (int i = tid; i < kFusedWaves * (kFusedMaxExperts / 4); i += kFusedThreads)
        (&chunk_cnt[0][0])[i] = 0u;
    for (int i = tid; i < RC; i += kFusedThreads)
        rank_cnt[i] = 0;
    if (tid == 0)
        s_err = 0u;
    lds_barrier();

    // Keys of this lane's slots, one per chunk of the wave's run.
    const int nchunks = (ns + kWave - 1) / kWave;
    const int cpw = (nchunks + kFusedWaves - 1) / kFusedWaves;
    const int c0 = wave * cpw;
    int key[kFusedChunksPerWave];
    int lrank[kFusedChunksPerWave];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kFusedChunksPerWave; ++i) {
        const int s = (c0 + i) * kWave + lane;
        int64_t e = -1;
        if (i < cpw && s < ns)
            e = topk[s];
        bad |= (e < -1 || e >= E);
        key[i] = (e >= 0 && e < E) ? (int)e : -1;
        lrank[i] = 0;
    }
    if (bad)
        atomicOr(&s_err, 1u);
    if (wave == 0) {
        // wave 0's first chunk is the batch's first 64 slots
        const uint64_t m = wave_ballot(key[0] >= 0);
        if (lane == 0)
            hdr->dense = dense_sample(m, ns);
    }

    // In-wave ranks, chunk by chunk in order (see ep_layout_kernel).
    {
        int32_t *my_cnt = wave_cnt[wave];
        uint32_t *my_chunk = chunk_cnt[wave];
        const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
        for (int i = 0; i < kFusedChunksPerWave; ++i) {
            // chunks past the wave's run hold only -1 keys: no-ops
            const int k16 = key[i] >= 0 ? key[i] : 0;
            const bool valid = key[i] >= 0;
            const int shift = 8 * (k16 & 3);
            if (valid)
                atomicAdd(&my_chunk[k16 >> 2], 1u << shift);
            const int group = valid ? (int)((my_chunk[k16 >> 2] >> shift) & 0xFFu) : 0;
            int rank = 0;
            uint64_t todo = wave_ballot(group > 1);
            while (todo) {
                const int leader = (int)__builtin_ctzll(todo);
                const int lkey = __builtin_amdgcn_readlane(k16, leader);
                const uint64_t same = wave_ballot(valid && k16 == lkey);
                if (valid && k16 == lkey)
                    rank = __popcll(same & lower);
                todo &= ~same;
            }
            if (valid) {
                const int base = my_cnt[k16];
                lrank[i] = base + rank;
                if (rank == 0) {
                    my_cnt[k16] = base + group;
                    atomicAnd(&my_chunk[k16 >> 2], ~(0xFFu << shift));
                }
            }
        }
    }

    // Token -> rank mask and tokens per rank / node (one thread per token,
    // keys read again from topk_idx).
    for (int64_t t = tid; t < T; t += kFusedThreads) {
        const int64_t *row = topk + t * K;
        for (int w0 = 0; w0 < R; w0 += 64) {
            const int wr = min(64, R - w0);
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int64_t e = row[k];
                if (e >= 0 && e < E) {
                    const int r = div_small((uint32_t)e, experts_per_rank, epr_magic) - w0;
                    if (r >= 0 && r < wr)
                        mask |= 1ull << r;
                }
            }
            if (in_rank)
                store_mask_bytes(in_rank + t * R + w0, mask, wr, in_rank_vec16);
            for (uint64_t m = mask; m; m &= m - 1)
                atomicAdd(&rank_cnt[w0 + __builtin_ctzll(m)], 1);
        }
        for (int n0 = 0; n0 < Rn; n0 += 64) {
            const int wn = min(64, Rn - n0);
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int64_t e = row[k];
                if (e >= 0 && e < E) {
                    const int r = div_small((uint32_t)e, experts_per_rank, epr_magic);
                    const int n = div_small((uint32_t)r, G, node_magic) - n0;
                    if (n >= 0 && n < wn)
                        mask |= 1ull << n;
                }
            }
            for (uint64_t m = mask; m; m &= m - 1)
                atomicAdd(&rank_cnt[R + n0 + __builtin_ctzll(m)], 1);
        }
    }
    lds_barrier();

    // Per expert: exclusive prefix over the waves (in place) and the total.
    int blk = 0;
    if (tid < E) {
        int run = 0;
        for (int w = 0; w < kFusedWaves; ++w) {
            const int c = wave_cnt[w][tid];
            wave_cnt[w][tid] = run;
            run += c;
        }
        if (cnt)
            cnt[tid] = run;
        ws_counts[tid] = run;
        block_base[tid] = 0;
        blk = (run + alignment - 1) / alignment * alignment;
    }
    for (int r = tid; r < RC; r += kFusedThreads) {
        if (r < R) {
            if (per_rank)
                per_rank[r] = rank_cnt[r];
        } else if (per_node) {
            per_node[r - R] = rank_cnt[r];
        }
    }
    // expert_start_loc and N (the block scan has its own barriers, which
    // also order the wave_cnt rewrite above before the slot ranks below)
    const int incl = block_inclusive_scan(blk, s_wave);
    if (start) {
        if (tid < E)
            start[tid] = incl - blk;
        if (tid == kFusedThreads - 1) {
            hdr->total = incl;
            if (total_out)
                *total_out = incl;
        }
    }
    if (tid == kFusedThreads - 1)
        hdr->status = (s_err ? kStatusBadExpert : 0u) |
                      (a.capacity >= 0 && incl > a.capacity ? kStatusCapacity : 0u);

    // Global rank of every slot.
#pragma unroll
    for (int i = 0; i < kFusedChunksPerWave; ++i) {
        const int s = (c0 + i) * kWave + lane;
        if (i < cpw && s < ns)
            slot_rank[s] = key[i] >= 0 ? lrank[i] + wave_cnt[wave][key[i]] : -1;
    }
}

__global__ __launch_bounds__(kFusedThreads) void ep_layout_scan_kernel(LayoutScanArgs a)
{
    layout_scan_block(a);
}

// -------------------------------------------------------------- scatter --

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Workgroup counts of the row kernels. Combine: one workgroup per token (the
// dispatcher starts a new workgroup as soon as one retires, which balances
// better than striding). Scatter: also one per token from
// kScatterGridFrom tokens on; below that, kScatterGrid workgroups striding
// over the tokens, which measured faster at a few thousand tokens, of which
// only kScatterGridLong work for rows of at least kScatterLongRowBytes when
// the layout found dense routing (WsHeader::dense). Below kScatterGridFrom
// tokens the batch (at most ~120 MB at hidden 7168) stays in the Infinity
// Cache between steps, so the writes bound the kernel, and with 14 KB rows of
// eight destinations fewer rows in flight write more efficiently (4096
// tokens of hidden 7168: 96.7 -> 93.2 us, five runs each), while rows of one
// or two destinations (a receive side) want more tokens in flight (6000
// tokens: step 130 -> 108 us with the whole grid); with 7-8 KB rows 512 and
// 1024 workgroups tie.
// Decode-sized batches: column parts per row so that about kScatterSmallItems
// (token, part) items exist, each part at least one pass of the workgroup
// (kScatterThreads 16-byte vectors), at most kScatterMaxParts parts. Aiming
// at 4096 rather than 2048 items gives as many parts as the row has whole
// passes (7 of 128 vectors at hidden 7168 up to 585 tokens, 4 at hidden
// 4096) instead of fewer, uneven ones with a ragged second pass: 384 tokens of
// hidden 7168 38.4 -> 36.2 us per step, 1000 tokens of hidden 4096 40.0 ->
// 37.7 us, no shape slower.
#ifndef EPL_SCATTER_SMALL_ITEMS
#define EPL_SCATTER_SMALL_ITEMS 4096
#endif
constexpr int64_t kScatterSmallItems = EPL_SCATTER_SMALL_ITEMS;
constexpr int kScatterMaxParts = 8;
constexpr int kScatterGrid = EPL_SCATTER_GRID;
constexpr int kScatterGridLong = EPL_SCATTER_GRID_LONG;
constexpr int64_t kScatterLongRowBytes = EPL_SCATTER_LONG_ROW_BYTES;
constexpr int64_t kScatterGridFrom = EPL_SCATTER_GRID_FROM;
constexpr int kCombineGrid = EPL_COMBINE_GRID;

// Combine outputs above this size (half of MI355X's 256 MB Infinity Cache)
// are written with non-temporal stores.
#ifndef EPL_Y_NT_BYTES
#define EPL_Y_NT_BYTES (128ll << 20)
#endif
constexpr int64_t kYNtBytes = EPL_Y_NT_BYTES;

#ifndef EPL_XCD_MAP
#define EPL_XCD_MAP 1
#endif
#ifndef EPL_SCALE_NT
#define EPL_SCALE_NT 0
#endif
#ifndef EPL_ROW_NT
#define EPL_ROW_NT 1
#endif
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroup i runs on XCD i % 8

// Tokens of one workgroup of a grid-stride row kernel of G active workgroups
// (the launch's grid unless the kernel retires some): first, first + stride,
// ... below end. With the XCD-aware mapping (xcd_ranges, and a grid that is a
// multiple of 8) each XCD owns one contiguous range of ceil(T / 8) tokens, so
// rows written for neighbouring tokens (the neighbouring rows of an
// expert's block, their scale rows and m_indices entries) meet in the same
// L2, where partial-line writes can merge before they reach HBM. Otherwise
// workgroup w takes items w, w + G, ...: round-robin over the XCDs, which
// the host picks for large one-item-per-workgroup grids (there, all XCDs
// then work on a narrow window of neighbouring tokens, and the combine's
// output rows are written close to one another in time).
struct TokenRange {
    int64_t first, stride, end;
};

__device__ __forceinline__ TokenRange token_range(int64_t T, bool xcd_ranges = true,
                                                  int64_t G = gridDim.x)
{
    const int64_t w = blockIdx.x;
    if (xcd_ranges && EPL_XCD_MAP && G % kNumXcd == 0 && G >= kNumXcd) {
        const int64_t per = (T + kNumXcd - 1) / kNumXcd;
        const int64_t xcd = w % kNumXcd;
        return {xcd * per + w / kNumXcd, G / kNumXcd, min(T, (xcd + 1) * per)};
    }
    return {w, G, T};
}

// Scale rows are small (S floats): written back through L2 by default so that
// the partial lines of neighbouring rows can merge there.
template <typename V>
__device__ __forceinline__ void store_scale(V *dst, const V &v)
{
    if (EPL_SCALE_NT)
        __builtin_nontemporal_store(v, dst);
    else
        *dst = v;
}

// Scale layouts of the scatter.
constexpr int kScaleNone = 0;
constexpr int kScaleRows = 1;   // W words per row, row-major ([rows, W])
constexpr int kScaleCols = 2;   // W words per row, column-major: word j of row p at j * ld + p

// One workgroup per token row, grid-stride over tokens. A row is row_bytes
// of opaque payload (bf16: 2H bytes, FP8: H bytes), read once as 16-byte
// vectors (VPT per thread per pass) and stored to each of the token's K
// destination rows with non-temporal stores: the buffer is written once and
// read much later, so the stores should not displace cached data. The
// token's W scale words are fetched together with the row and follow it,
// row-major (fp32 scales) or column-major (the transposed packed-UE8M0
// layout of the FP8 grouped GEMM).
//
// Destination rows come from two dependent lookups per slot (expert id and
// slot rank, then expert offset and block offset). The first K threads run
// them ahead of the data: while token t streams, they already hold the
// offsets of token t + G and the ids of token t + 2G (G = grid size), so no
// token waits for its own lookups. The rows live in a double-buffered LDS
// table, so one barrier per token suffices: a thread can only overwrite a
// buffer after every thread has passed the barrier of the token in between,
// i.e. has finished reading that buffer.
//
// Batches with fewer tokens than the striding grid has workgroups (decode
// sizes) split each row into `parts` column ranges, one work item per
// (token, part): more workgroups share a token's bytes and the launch ends
// sooner (the first part of a token also writes its indices and scale row).
// SPLIT: the launch may cut rows into parts (parts > 1 only then; without
// it every item is a whole token and the part arithmetic folds away).
//
// OFFSETS: the scatter of a dispatch also does the scan's work, so the
// chain needs no scan launch between layout and scatter (see ScanInScatter).
// Every workgroup reads the layout's per-block counts (nb x E words, from
// L2), sums each expert's column, scans the aligned sums into the expert
// offsets and keeps in LDS the offsets and the per-block offsets of the
// blocks its tokens fall in, so its slot lookups then read LDS instead of
// global memory. Workgroup 0 also stores the scan's results (counts,
// expert_start_loc, N, the per-block offsets for later scatter calls, the
// layout's error bits into the status word, which the layout reset) and
// workgroup 1 (or 0 in a one-workgroup grid) the per-rank and per-node
// totals. Their values are those of ep_scan_kernel in reduce + prefix mode.
// LDS words of the per-segment column sums (E / 4 expert quads x
// kScatterThreads / (E / 4) segments, 4 words each).
constexpr int kScanSegWords = 4 * kScatterThreads;

struct ScanInScatter {
    const int32_t *block_count;   // [nb, E] slots per layout block and expert
    const int32_t *block_rank;    // [nb, R + Rn] tokens per block and rank / node
    const uint32_t *block_err;    // [nb] error bits per block
    int64_t nb;                   // layout blocks
    int R, Rn;                    // rank columns, node columns
    int nbl;                      // LDS rows of per-block offsets per workgroup
    int32_t *cnt;                 // [E] num_tokens_per_expert (or null)
    int32_t *per_rank;            // [R] (or null)
    int32_t *per_node;            // [Rn] (or null)
    int32_t *start;               // [E] expert_start_loc
    int32_t *ws_counts;           // [E] the workspace's copy of the counts
    int32_t *block_base;          // [nb, E] exclusive prefix of block_count over blocks
    WsHeader *hdr;                // total
    int32_t *total_out;           // host-mapped word for N (or null)
};

// Blocks of B tokens that the tokens of one grid-stride range touch: from
// the first token's block to the last one's (b_hi < b_lo when it has none).
__device__ __forceinline__ void range_blocks(const TokenRange &tr, int B, int64_t &b_lo,
                                             int64_t &b_hi)
{
    b_lo = 0;
    b_hi = -1;
    if (tr.first < tr.end) {
        const int64_t last = tr.first + (tr.end - 1 - tr.first) / tr.stride * tr.stride;
        b_lo = tr.first / B;
        b_hi = last / B;
    }
}

template <int VPT, bool SPLIT, bool OFFSETS>
__global__ __launch_bounds__(kScatterThreads) void ep_scatter_kernel(
    const uint8_t *__restrict__ x, int64_t row_bytes, int scale_mode,
    const uint32_t *__restrict__ x_scale, int W, bool scale_vec16, int64_t scale_ld,
    const int64_t *__restrict__ topk, const int32_t *__restrict__ start,
    const int32_t *__restrict__ block_base, const int32_t *__restrict__ slot_rank, int64_t T,
    int K, int E, int B, int alignment, const int32_t *__restrict__ counts, int64_t capacity,
    int parts_arg, bool xcd_ranges, uint8_t *__restrict__ out, uint32_t *__restrict__ out_scale,
    int32_t *__restrict__ m_indices, int32_t *__restrict__ output_index,
    uint32_t *__restrict__ status, ScanInScatter sc, const int32_t *__restrict__ dense,
    int grid_dense)
{
    static_assert(!(SPLIT && OFFSETS), "the scan-in-scatter launch has whole-token items");
    // Active workgroups: the grid, or its first grid_dense workgroups when the
    // layout found dense routing (`dense` null: always the grid). Rows with
    // many destinations write best with fewer of them in flight, rows with
    // one or two need more tokens in flight; the results are the same.
    int G = gridDim.x;
    if (dense != nullptr && *dense == 1)
        G = grid_dense;
    if ((int)blockIdx.x >= G)
        return;
    __shared__ int64_t s_row[2][kMaxTopk];
    extern __shared__ __align__(16) int32_t s_off[];   // OFFSETS only, see below
    const int tid = threadIdx.x;
    const int parts = SPLIT ? parts_arg : 1;
    const int nvec = (int)(row_bytes >> 4);
    const int pvec = SPLIT ? (nvec + parts - 1) / parts : nvec;   // 16-byte vectors per part
    // Work items: (token, column part) pairs, item i = token i / parts, part
    // i % parts (parts = 1 except for batches too small to fill the GPU).
    const TokenRange tr = token_range(T * parts, xcd_ranges, G);
    const int64_t step = tr.stride, i_end = tr.end;
    const bool lead = tid < K;
    auto token_of = [=](int64_t item) { return SPLIT ? item / parts : item; };

    // Lookup pipeline of the first K threads (slot tid of the item's token):
    //   (e1, r1): expert id and block rank for the next item;
    //   (e0, r0, s0, b0): expert id, block rank, expert offset and block offset
    //   for the current one. The two offsets are kept apart (and added only
    //   when used, one item later) so that no wave waits for them early. The
    //   first item's offsets are loaded only after its row loads are issued,
    //   so that a workgroup with a single item waits for one lookup round
    //   trip before its row load instead of two.
    int64_t e0 = -1, e1 = -1;
    int r0 = 0, r1 = 0, s0 = 0, b0 = 0;
    auto valid = [E](int64_t e) { return e >= 0 && e < E; };
    if (lead && tr.first < i_end) {
        const int64_t t = token_of(tr.first);
        e0 = topk[t * K + tid];
        r0 = slot_rank[t * K + tid];
        if (tr.first + step < i_end) {
            const int64_t tn = token_of(tr.first + step);
            e1 = topk[tn * K + tid];
            r1 = slot_rank[tn * K + tid];
        }
    }

    // OFFSETS LDS: [E] expert offsets, [E] counts, [kScanSegWords] segment
    // sums, [nbl, E] per-block offsets of this workgroup's blocks
    int32_t *s_start = s_off, *s_cnt = s_off + E, *s_seg = s_off + 2 * E;
    int32_t *s_base = s_seg + kScanSegWords;
    int64_t b_lo = 0, b_hi = -1;
    u32x4 v[VPT];
    if (OFFSETS) {
        __shared__ int s_wave[kScatterThreads / kWave];
        __shared__ int s_part[kScatterThreads];
        range_blocks(tr, B, b_lo, b_hi);
        b_hi = min(b_hi, b_lo + sc.nbl - 1);   // LDS rows held (the launch sizes nbl to cover the range)
        const bool first_wg = blockIdx.x == 0;
        // The count matrix in 16-byte pieces: thread (c, q) takes experts
        // 4c .. 4c + 3 over the q-th segment of L blocks (the launch
        // guarantees E % 4 == 0, E <= 4 * kScatterThreads and L <= 16), so
        // all of a thread's loads are in flight at once and every workgroup
        // waits for a single round trip.
        const int nq4 = E >> 2;
        const int Q = kScatterThreads / nq4;
        const int64_t L = (sc.nb + Q - 1) / Q;
        const int c = tid % nq4, q = tid / nq4;
        const bool seg_thread = q < Q;
        const int64_t sb0 = (int64_t)q * L, sb1 = min(sc.nb, sb0 + L);
        const i32x4 *bc4 = reinterpret_cast<const i32x4 *>(sc.block_count);
        i32x4 held[16];
        i32x4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            held[j] = i32x4{0, 0, 0, 0};
            if (seg_thread && sb0 + j < sb1)
                held[j] = bc4[(sb0 + j) * nq4 + c];
        }
        // The first item's row loads go out now, behind the count loads, so
        // that they travel while this prologue computes (the loop does not
        // load them again).
        if (tr.first < i_end) {
            const u32x4 *xrow = reinterpret_cast<const u32x4 *>(x + tr.first * row_bytes);
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = i * kScatterThreads + tid;
                if (idx < nvec)
                    v[i] = xrow[idx];
            }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            sum += held[j];
        if (seg_thread)
            reinterpret_cast<i32x4 *>(s_seg)[q * nq4 + c] = sum;
        lds_barrier();
        // Segment offsets and column totals, then the running prefix over
        // the held blocks: into LDS for this workgroup's blocks and, from
        // workgroup 0, into the workspace for later scatter calls.
        if (seg_thread) {
            i32x4 run = {0, 0, 0, 0}, tot = {0, 0, 0, 0};
            for (int g = 0; g < Q; ++g) {
                const i32x4 seg = reinterpret_cast<const i32x4 *>(s_seg)[g * nq4 + c];
                if (g < q)
                    run += seg;
                tot += seg;
            }
            if (q == 0)
                reinterpret_cast<i32x4 *>(s_cnt)[c] = tot;
            i32x4 *bb4 = reinterpret_cast<i32x4 *>(sc.block_base);
            i32x4 *sbase4 = reinterpret_cast<i32x4 *>(s_base);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t b = sb0 + j;
                if (b < sb1) {
                    if (b >= b_lo && b <= b_hi)
                        sbase4[(b - b_lo) * nq4 + c] = run;
                    if (first_wg)
                        bb4[b * nq4 + c] = run;
                    run += held[j];
                }
            }
        }
        // Per-rank and per-node totals (workgroup 1, or 0 in a one-workgroup
        // grid): thread (r, g) sums column r over the g-th of P block segments
        // (16 loads in flight per pass), the P partial sums meet in LDS.
        const bool rank_wg = (int)blockIdx.x == min(1, G - 1);
        const int RC = sc.R + sc.Rn;
        const int P = RC < kScatterThreads ? kScatterThreads / RC : 1;
        if (rank_wg) {
            const int64_t PL = (sc.nb + P - 1) / P;
            for (int i = tid; i < RC * P; i += kScatterThreads) {
                const int r = i % RC, g = i / RC;
                const int64_t g0 = (int64_t)g * PL, g1 = min(sc.nb, g0 + PL);
                int part = 0;
                for (int64_t bb = g0; bb < g1; bb += 16) {
                    int rv[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        rv[j] = bb + j < g1 ? sc.block_rank[(bb + j) * RC + r] : 0;
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        part += rv[j];
                }
                if (P > 1)
                    s_part[i] = part;
                else if (r < sc.R) {
                    if (sc.per_rank)
                        sc.per_rank[r] = part;
                } else if (sc.per_node) {
                    sc.per_node[r - sc.R] = part;
                }
            }
        }
        lds_barrier();
        if (rank_wg && P > 1) {
            for (int r = tid; r < RC; r += kScatterThreads) {
                int tot = 0;
                for (int g = 0; g < P; ++g)
                    tot += s_part[g * RC + r];
                if (r < sc.R) {
                    if (sc.per_rank)
                        sc.per_rank[r] = tot;
                } else if (sc.per_node) {
                    sc.per_node[r - sc.R] = tot;
                }
            }
        }
        // Expert offsets: exclusive prefix of the block sizes (counts rounded
        // up to the alignment); thread i owns experts [i * per, (i + 1) * per).
        const int per = (E + kScatterThreads - 1) / kScatterThreads;
        const int e_lo = min(E, tid * per), e_hi = min(E, e_lo + per);
        auto block = [alignment](int n) { return (n + alignment - 1) / alignment * alignment; };
        int own = 0;
        for (int e = e_lo; e < e_hi; ++e)
            own += block(s_cnt[e]);
        const int incl = block_inclusive_scan<kScatterThreads>(own, s_wave);
        int run = incl - own;
        for (int e = e_lo; e < e_hi; ++e) {
            s_start[e] = run;
            if (first_wg) {
                sc.start[e] = run;
                sc.ws_counts[e] = s_cnt[e];
                if (sc.cnt)
                    sc.cnt[e] = s_cnt[e];
            }
            run += block(s_cnt[e]);
        }
        if (first_wg && tid == kScatterThreads - 1) {
            sc.hdr->total = incl;
            if (sc.total_out)
                *sc.total_out = incl;
        }
        if (first_wg) {
            uint32_t err = 0;
            for (int64_t bb = tid; bb < sc.nb; bb += kScatterThreads)
                err |= sc.block_err[bb];
            if (err)
                atomicOr(status, kStatusBadExpert);
        }
        lds_barrier();
    }
    auto expert_start = [&](int64_t e) { return OFFSETS ? s_start[e] : start[e]; };
    auto expert_count = [&](int64_t e) { return OFFSETS ? s_cnt[e] : counts[e]; };
    auto block_offset = [&](int64_t t, int64_t e) {
        if (!OFFSETS)
            return block_base[(t / B) * E + e];
        const int64_t b = t / B;
        if (b >= b_lo && b <= b_hi)
            return s_base[(b - b_lo) * E + e];
        // not reached when nbl covers the range (the launch sizes it so);
        // kept so that a block outside it still gets its exact offset
        int run = 0;
        for (int64_t bb = 0; bb < b; ++bb)
            run += sc.block_count[bb * E + e];
        return run;
    };

    // Padding rows of the aligned blocks: between an expert's last row and
    // the end of its block, marked -1 (workgroup w takes experts w, w + G, ...).
    if (alignment > 1) {
        for (int e = blockIdx.x; e < E; e += G) {
            const int64_t c = expert_count(e);
            const int64_t p0 = (int64_t)expert_start(e) + c;
            const int64_t p1 = (int64_t)expert_start(e) + (c + alignment - 1) / alignment * alignment;
            for (int64_t p = p0 + tid; p < p1; p += kScatterThreads) {
                if (p >= 0 && p < capacity)
                    m_indices[p] = -1;
                else
                    atomicOr(status, kStatusCapacity);
            }
        }
    }
    // scale words prefetched with the row: 16-byte pieces (row-major, W % 4 == 0)
    // or single words (column-major)
    const int nq = scale_mode == kScaleRows && scale_vec16 ? (W >> 2) : 0;
    const int nw = scale_mode == kScaleCols ? W : 0;

    int it = 0;
    for (int64_t item = tr.first; item < i_end; item += step, ++it) {
        const int64_t t = token_of(item);
        const int q = (int)(item - t * parts);
        const int v0 = q * pvec, v1 = min(nvec, v0 + pvec);
        const bool first_part = q == 0;   // writes the indices and the scale row
        int64_t *rows = s_row[it & 1];
        const u32x4 *xrow = reinterpret_cast<const u32x4 *>(x + t * row_bytes);
        if (!OFFSETS || it > 0) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = v0 + i * kScatterThreads + tid;
                if (idx < v1)
                    v[i] = xrow[idx];
            }
        }
        u32x4 sv = {0u, 0u, 0u, 0u};
        uint32_t sw = 0u;
        if (first_part && tid < nq)
            sv = reinterpret_cast<const u32x4 *>(x_scale + t * W)[tid];
        if (first_part && tid < nw)
            sw = x_scale[t * W + tid];

        if (lead && it == 0 && valid(e0)) {
            s0 = expert_start(e0);
            b0 = block_offset(t, e0);
        }
        if (lead) {
            int pos = -1;
            int64_t row = -1;
            if (valid(e0)) {
                // a slot whose row falls outside the buffer is not placed:
                // output_index -1, like a slot with no selection
                const int64_t p = (int64_t)s0 + b0 + r0;
                if (p >= 0 && p < capacity) {
                    row = p;
                    pos = (int)p;
                    if (first_part)
                        m_indices[p] = (int32_t)e0;
                } else {
                    atomicOr(status, kStatusCapacity);
                }
            }
            if (first_part)
                output_index[t * K + tid] = pos;
            rows[tid] = row;
            // advance the pipeline: offsets for the next item, ids for the one after
            e0 = e1;
            r0 = r1;
            s0 = 0;
            b0 = 0;
            if (item + step < i_end && valid(e0)) {
                s0 = expert_start(e0);
                b0 = block_offset(token_of(item + step), e0);
            }
            e1 = -1;
            if (item + 2 * step < i_end) {
                const int64_t t2 = token_of(item + 2 * step);
                e1 = topk[t2 * K + tid];
                r1 = slot_rank[t2 * K + tid];
            }
        }
        lds_barrier();
        for (int base = v0;;) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kScatterThreads + tid;
                if (idx < v1) {
                    for (int k = 0; k < K; ++k) {
                        const int64_t row = rows[k];
                        if (row >= 0) {
                            u32x4 *dst = reinterpret_cast<u32x4 *>(out + row * row_bytes) + idx;
                            if (EPL_ROW_NT)
                                __builtin_nontemporal_store(v[i], dst);
                            else
                                *dst = v[i];
                        }
                    }
                }
            }
            base += kScatterThreads * VPT;
            if (base >= v1)
                break;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kScatterThreads + tid;
                if (idx < v1)
                    v[i] = xrow[idx];
            }
        }
        if (!first_part)
            continue;
        if (nq > 0) {
            // 16-byte pieces of the scale row (W % 4 == 0 and 16-byte aligned
            // bases); threads past the first kScatterThreads pieces take the rest.
            for (int j = tid; j < nq; j += kScatterThreads) {
                const u32x4 f = j == tid ? sv : reinterpret_cast<const u32x4 *>(x_scale + t * W)[j];
                for (int k = 0; k < K; ++k) {
                    const int64_t row = rows[k];
                    if (row >= 0)
                        store_scale(reinterpret_cast<u32x4 *>(out_scale + row * W) + j, f);
                }
            }
        } else if (scale_mode == kScaleRows) {
            for (int j = tid; j < W; j += kScatterThreads) {
                const uint32_t f = x_scale[t * W + j];
                for (int k = 0; k < K; ++k) {
                    const int64_t row = rows[k];
                    if (row >= 0)
                        store_scale(out_scale + row * W + j, f);
                }
            }
        } else if (scale_mode == kScaleCols) {
            // word j of every destination row lands in column j of the
            // transposed buffer; rows of one expert are neighbours there
            for (int j = tid; j < W; j += kScatterThreads) {
                const uint32_t f = j == tid ? sw : x_scale[t * W + j];
                for (int k = 0; k < K; ++k) {
                    const int64_t row = rows[k];
                    if (row >= 0)
                        store_scale(out_scale + (int64_t)j * scale_ld + row, f);
                }
            }
        }
    }
}

// ------------------------------------------------ decode-sized dispatch --

// Top-k up to which ep_dispatch_decode_kernel keeps the token's experts in
// registers for its slot counts.
constexpr int kDecodeFastTopk = 8;

// Rows and outputs of ep_dispatch_decode_kernel (as in ep_scatter_kernel).
struct DecodeRows {
    const uint8_t *x;
    int64_t row_bytes;
    int scale_mode;
    const uint32_t *x_scale;
    int W;
    bool scale_vec16;
    int64_t scale_ld;
    int64_t capacity;
    uint8_t *out;
    uint32_t *out_scale;
    int32_t *m_indices;
    int32_t *output_index;
};

// The counts side of a decode-sized dispatch, by one workgroup of
// kFusedThreads threads: per-expert counts (and the workspace's copy), the
// zero per-block offsets of the single layout block, expert_start_loc and
// N, tokens per rank and per node, and the status word (out-of-range ids;
// N > capacity, which is exactly when a slot row or a padding row would
// fall outside the buffer). The token -> rank mask and the per-slot ranks
// come from the token workgroups of ep_dispatch_decode_kernel.
__device__ __forceinline__ void decode_counts_block(const LayoutScanArgs &a)
{
    __shared__ int32_t s_hist[kFusedMaxExperts];
    __shared__ int32_t s_rc[kFusedMaxCols];
    __shared__ int s_wave[kFusedWaves];
    __shared__ uint32_t s_err;
    const int tid = threadIdx.x;
    const int K = a.K, E = a.E, R = a.R, Rn = a.Rn;
    const int RC = R + Rn;
    const int ns = (int)(a.T * K);
    int64_t e_in[kFusedMaxSlots / kFusedThreads];
#pragma unroll
    for (int i = 0; i < kFusedMaxSlots / kFusedThreads; ++i) {
        const int sl = i * kFusedThreads + tid;
        e_in[i] = sl < ns ? a.topk[sl] : -1;
    }
    for (int e = tid; e < E; e += kFusedThreads)
        s_hist[e] = 0;
    for (int r = tid; r < RC; r += kFusedThreads)
        s_rc[r] = 0;
    if (tid == 0)
        s_err = 0u;
    lds_barrier();
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kFusedMaxSlots / kFusedThreads; ++i) {
        const int64_t e = e_in[i];
        bad |= (e < -1 || e >= E);
        if (e >= 0 && e < E)
            atomicAdd(&s_hist[e], 1);
    }
    if (bad)
        atomicOr(&s_err, 1u);
    if (tid < kWave) {
        // the dense-routing hint from the first 64 slots (wave 0's e_in[0])
        const uint64_t m = wave_ballot(e_in[0] >= 0 && e_in[0] < E);
        if (tid == 0)
            a.hdr->dense = dense_sample(m, ns);
    }
    // Tokens per rank and per node: one thread per token, a token counted
    // once per rank (node) that any of its valid slots goes to.
    for (int64_t t = tid; t < a.T; t += kFusedThreads) {
        const int64_t *row = a.topk + t * K;
        for (int w0 = 0; w0 < R; w0 += 64) {
            const int wr = min(64, R - w0);
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int64_t e = row[k];
                if (e >= 0 && e < E) {
                    const int r = div_small((uint32_t)e, a.experts_per_rank, a.epr_magic) - w0;
                    if (r >= 0 && r < wr)
                        mask |= 1ull << r;
                }
            }
            for (uint64_t m = mask; m; m &= m - 1)
                atomicAdd(&s_rc[w0 + __builtin_ctzll(m)], 1);
        }
        for (int n0 = 0; n0 < Rn; n0 += 64) {
            const int wn = min(64, Rn - n0);
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int64_t e = row[k];
                if (e >= 0 && e < E) {
                    const int r = div_small((uint32_t)e, a.experts_per_rank, a.epr_magic);
                    const int n = div_small((uint32_t)r, a.G, a.node_magic) - n0;
                    if (n >= 0 && n < wn)
                        mask |= 1ull << n;
                }
            }
            for (uint64_t m = mask; m; m &= m - 1)
                atomicAdd(&s_rc[R + n0 + __builtin_ctzll(m)], 1);
        }
    }
    lds_barrier();
    int blk = 0;
    if (tid < E) {
        const int c = s_hist[tid];
        if (a.cnt)
            a.cnt[tid] = c;
        a.ws_counts[tid] = c;
        a.block_base[tid] = 0;
        blk = (c + a.alignment - 1) / a.alignment * a.alignment;
    }
    for (int r = tid; r < RC; r += kFusedThreads) {
        if (r < R) {
            if (a.per_rank)
                a.per_rank[r] = s_rc[r];
        } else if (a.per_node) {
            a.per_node[r - R] = s_rc[r];
        }
    }
    const int incl = block_inclusive_scan(blk, s_wave);
    if (tid < E)
        a.start[tid] = incl - blk;
    if (tid == kFusedThreads - 1) {
        a.hdr->total = incl;
        if (a.total_out)
            *a.total_out = incl;
        a.hdr->status = (s_err ? kStatusBadExpert : 0u) | (incl > a.capacity ? kStatusCapacity : 0u);
    }
}

// Layout, scan and scatter of a decode-sized batch (the batches that
// ep_layout_scan_kernel lays out alone) in one launch of T + 1 workgroups.
// Workgroup 0 produces the counts side (decode_counts_block). Workgroup
// 1 + t places and copies token t without waiting for it: with its row
// loads in flight it takes, for each slot (t, k) of expert e, the number of
// valid slots of experts below e and of earlier slots of expert e (wave
// ballots over all slots; with an expert alignment, the histogram of all
// slots and its aligned prefix instead of the first number). Their sum is
// the slot's row -- the same row as expert_start_loc[e] + the slot's rank
// in (token, k) order -- and the second number is its rank, stored for
// later scatter calls on the workspace. It also stores the token's row of
// the token -> rank mask. Padding rows of expert e are marked by the
// workgroup of token e mod T. Rows at or past the capacity are skipped (the
// status bit comes from workgroup 0).
__global__ __launch_bounds__(kFusedThreads) void ep_dispatch_decode_kernel(LayoutScanArgs a,
                                                                           DecodeRows d)
{
    if (blockIdx.x == 0) {
        decode_counts_block(a);
        return;
    }
    constexpr int kSlotsPerThread = kFusedMaxSlots / kFusedThreads;
    __shared__ int32_t s_tok[kMaxTopk];                  // the token's expert ids (-1: none)
    __shared__ int32_t s_less[kMaxTopk][kFusedWaves];    // per wave: valid slots of lower experts
    __shared__ int32_t s_same[kMaxTopk][kFusedWaves];    // per wave: earlier slots of the expert
    __shared__ int32_t s_hist[kFusedMaxExperts];         // aligned batches: slots per expert
    __shared__ int32_t s_start[kFusedMaxExperts];        // aligned batches: expert offsets
    __shared__ int64_t s_rows[kMaxTopk];
    __shared__ int s_wave[kFusedWaves];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int64_t t = blockIdx.x - 1;
    const int K = a.K, E = a.E, alignment = a.alignment;
    const int ns = (int)(a.T * K);
    const int nvec = (int)(d.row_bytes >> 4);
    const bool aligned_blocks = alignment > 1;

    // The token's first pass of its row and its scale words go out first,
    // with the routing of every slot.
    const u32x4 *xrow = reinterpret_cast<const u32x4 *>(d.x + t * d.row_bytes);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tid < nvec)
        v = xrow[tid];
    const int nq = d.scale_mode == kScaleRows && d.scale_vec16 ? (d.W >> 2) : 0;
    const int nw = nq == 0 && d.scale_mode != kScaleNone ? d.W : 0;
    u32x4 sv = {0u, 0u, 0u, 0u};
    uint32_t sw = 0u;
    if (tid < nq)
        sv = reinterpret_cast<const u32x4 *>(d.x_scale + t * d.W)[tid];
    if (tid < nw)
        sw = d.x_scale[t * d.W + tid];
    int my_key[kSlotsPerThread];
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
        const int sl = i * kFusedThreads + tid;
        const int64_t e = sl < ns ? a.topk[sl] : -1;
        my_key[i] = (e >= 0 && e < E) ? (int)e : -1;
    }
    if (tid < K) {
        const int64_t e = a.topk[t * K + tid];
        s_tok[tid] = (e >= 0 && e < E) ? (int)e : -1;
    }
    if (aligned_blocks) {
        for (int e = tid; e < E; e += kFusedThreads)
            s_hist[e] = 0;
    }
    lds_barrier();
    if (aligned_blocks) {
#pragma unroll
        for (int i = 0; i < kSlotsPerThread; ++i)
            if (my_key[i] >= 0)
                atomicAdd(&s_hist[my_key[i]], 1);
    }
    // The token's row of the token -> rank mask.
    for (int r = tid; r < a.R; r += kFusedThreads) {
        uint8_t hit = 0;
        for (int k = 0; k < K; ++k) {
            const int e = s_tok[k];
            if (e >= 0 && div_small((uint32_t)e, a.experts_per_rank, a.epr_magic) == r)
                hit = 1;
        }
        a.in_rank[t * a.R + r] = hit;
    }
    auto count_slot = [&](int k, int ek) {
        const int sk = (int)t * K + k;
        int less = 0, same = 0;
#pragma unroll
        for (int i = 0; i < kSlotsPerThread; ++i) {
            const int sl = i * kFusedThreads + tid;
            const int mk = my_key[i];
            if (!aligned_blocks)
                less += __popcll(wave_ballot(mk >= 0 && mk < ek));
            same += __popcll(wave_ballot(ek >= 0 && mk == ek && sl < sk));
        }
        if (lane == 0) {
            s_less[k][tid / kWave] = less;
            s_same[k][tid / kWave] = same;
        }
    };
    if (K <= kDecodeFastTopk) {
        // the token's experts read from LDS all at once, then the slots in
        // turn without an LDS round trip between them
        int tok[kDecodeFastTopk];
#pragma unroll
        for (int k = 0; k < kDecodeFastTopk; ++k)
            tok[k] = k < K ? s_tok[k] : -1;
#pragma unroll
        for (int k = 0; k < kDecodeFastTopk; ++k)
            if (k < K)
                count_slot(k, tok[k]);
    } else {
        for (int k = 0; k < K; ++k)
            count_slot(k, s_tok[k]);
    }
    if (aligned_blocks) {
        // expert offsets: exclusive prefix of the aligned counts
        lds_barrier();
        const int blk = tid < E ? (s_hist[tid] + alignment - 1) / alignment * alignment : 0;
        const int incl = block_inclusive_scan(blk, s_wave);
        if (tid < E)
            s_start[tid] = incl - blk;
    }
    lds_barrier();
    // Slot k's row: its two counts summed over the 16 waves (a serial sum
    // by thread k measured faster than a shuffle reduction over 16 lanes).
    if (tid < K) {
        int less = 0, rank = 0;
        for (int w = 0; w < kFusedWaves; ++w) {
            less += s_less[tid][w];
            rank += s_same[tid][w];
        }
        const int e = s_tok[tid];
        int64_t row = -1;
        if (e >= 0) {
            const int64_t p = (aligned_blocks ? (int64_t)s_start[e] : (int64_t)less) + rank;
            if (p < d.capacity) {
                row = p;
                d.m_indices[p] = e;
            }
        }
        a.slot_rank[t * K + tid] = e >= 0 ? rank : -1;
        d.output_index[t * K + tid] = (int32_t)row;
        s_rows[tid] = row;
    }
    lds_barrier();

    // Row copies: the first pass from registers, then any further passes.
    for (int idx = tid; idx < nvec; idx += kFusedThreads) {
        if (idx != tid)
            v = xrow[idx];
        for (int k = 0; k < K; ++k) {
            const int64_t row = s_rows[k];
            if (row >= 0) {
                u32x4 *dst = reinterpret_cast<u32x4 *>(d.out + row * d.row_bytes) + idx;
                if (EPL_ROW_NT)
                    __builtin_nontemporal_store(v, dst);
                else
                    *dst = v;
            }
        }
    }
    if (nq > 0) {
        for (int j = tid; j < nq; j += kFusedThreads) {
            const u32x4 f = j == tid ? sv : reinterpret_cast<const u32x4 *>(d.x_scale + t * d.W)[j];
            for (int k = 0; k < K; ++k) {
                const int64_t row = s_rows[k];
                if (row >= 0)
                    store_scale(reinterpret_cast<u32x4 *>(d.out_scale + row * d.W) + j, f);
            }
        }
    } else if (nw > 0) {
        for (int j = tid; j < nw; j += kFusedThreads) {
            const uint32_t f = j == tid ? sw : d.x_scale[t * d.W + j];
            for (int k = 0; k < K; ++k) {
                const int64_t row = s_rows[k];
                if (row < 0)
                    continue;
                if (d.scale_mode == kScaleRows)
                    store_scale(d.out_scale + row * d.W + j, f);
                else
                    store_scale(d.out_scale + (int64_t)j * d.scale_ld + row, f);
            }
        }
    }
    // Padding rows of the aligned blocks of experts t, t + T, ...
    if (aligned_blocks) {
        for (int64_t e = t; e < E; e += a.T) {
            const int64_t c = s_hist[e];
            const int64_t p0 = (int64_t)s_start[e] + c;
            const int64_t p1 = (int64_t)s_start[e] + (c + alignment - 1) / alignment * alignment;
            for (int64_t p = p0 + tid; p < p1 && p < d.capacity; p += kFusedThreads)
                d.m_indices[p] = -1;
        }
    }
}

// ------------------------------------------- low-latency fixed rectangle --

// e4m3 (OCP "fn": bias 7, max 448, no infinities) of a binary32 value, round
// to nearest even; magnitudes that round above 448 (infinities too) give 448,
// and a NaN of either sign gives the code 0x7F. Both cases are computed and
// one is selected (no divergent branch per element): normal results
// (|p| >= 2^-6) round the 23-bit mantissa to 3 bits on the bit pattern (a
// carry moves into the exponent as it should) and rebias the exponent from
// 127 to 7; smaller magnitudes are multiples of 2^-9, rounded with rint
// (which may give 8 = 2^-6, the smallest normal code).
__device__ __forceinline__ uint32_t e4m3_rne(float p)
{
    const uint32_t u = __float_as_uint(p);
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    const uint32_t normal = min((r >> 20) - (120u << 3), 0x7Eu);      // exponent 127 -> 7
    const uint32_t sub = (uint32_t)rintf(__uint_as_float(a) * 512.0f); // multiples of 2^-9
    const uint32_t code = ((u >> 24) & 0x80u) | (a >= 0x3C800000u ? normal : sub);  // 2^-6
    return a > 0x7F800000u ? 0x7Fu : code;
}

// Maximum over the 8 lanes of a half DPP row (lanes 8m .. 8m+7), returned
// to every one of them: mirror within the half row (lane i meets lane 7-i,
// so each quad then holds all four pair maxima), then two quad permutes.
__device__ __forceinline__ float half_row_max(float v)
{
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    return v;
}

// e4m3 codes of 4 binary32 values packed little-endian into a word.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    return e4m3_rne(a) | (e4m3_rne(b) << 8) | (e4m3_rne(c) << 16) | (e4m3_rne(d) << 24);
}

// FP8 cast of the 16 bf16 values one lane holds (two 16-byte vectors, 8
// values each) as part of a 128-column group spread over the 8 lanes of a
// half DPP row, all of which must be active: codes = e4m3(x * (448 / amax))
// packed four to a word, zero codes for an all-zero group, and the group's
// scale amax / 448, the same in each of its lanes.
struct Cast16 {
    u32x4 codes;
    float scale;
};
__device__ __forceinline__ Cast16 cast_e4m3_16(const u32x4 (&v)[2])
{
    float f[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[8 * h + 2 * q] = __uint_as_float(v[h][q] << 16);
            f[8 * h + 2 * q + 1] = __uint_as_float(v[h][q] & 0xFFFF0000u);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
        amax = fmaxf(amax, fabsf(f[q]));
    amax = half_row_max(amax);
    const float scale = amax / 448.0f;
    // 448 / amax overflows binary32 for amax below ~1.3e-36 (bf16 keeps
    // binary32's exponent range): such a group is first scaled by 2^64, which
    // changes no rounding (a power of two, the values stay normal), so the
    // codes are those of binary32 arithmetic with an unbounded exponent
    const float pre = amax < 0x1p-64f ? 0x1p64f : 1.0f;
    const float inv = amax > 0.0f ? 448.0f / (amax * pre) : 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
        f[q] *= pre;
    Cast16 c;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        c.codes[q] = e4m3x4(f[4 * q] * inv, f[4 * q + 1] * inv, f[4 * q + 2] * inv, f[4 * q + 3] * inv);
    c.scale = scale;
    return c;
}

#ifndef EPL_LL_GRID
#define EPL_LL_GRID 2048
#endif
constexpr int kLLGrid = EPL_LL_GRID;

// Strategy A (a fixed rectangle, no count exchange) in the shape of the
// low-latency receive buffers: expert e owns rows [e * cap, (e + 1) * cap)
// of the FP8 buffer; its slots fill them from the first in (token, k)
// order, j = block offset + in-block rank (the same per-expert position as
// the prefix-sum layout, without the prefix over experts).
//
// Workgroups stride over the tokens (XCD-aware ranges) -- or, with fewer
// tokens than the grid, over (token, column part) items, a part being a run
// of whole 128-column groups -- one item ahead: while an item is cast and
// stored, its workgroup already loads the next item's row (if that token
// selects any expert) and the first K threads place the next token's slots (output_index = e * cap + j, src_info[row] =
// t mod M, or -1 past the rectangle with the capacity bit in the status
// word); the placements reach the other threads through a double-buffered
// LDS table and one LDS-only barrier per token. A thread owns 16
// consecutive values of the row (two 16-byte loads) per step, so a
// 128-column group spans the 8 lanes of a half DPP row, which reduce |x|
// to amax with lane permutes; scale = amax / 448 and codes = e4m3(x *
// (448 / amax)) (zero codes for an all-zero group; a group too small for
// binary32's 448 / amax is cast like the same group scaled by 2^64). Each
// thread's 16 codes go to every placed row as one 16-byte non-temporal
// store, and each group's scale to out_scale[(e * S + g) * cap + j]
// (column-major per expert), the 8 lanes of the group sharing the slots.
// Before its tokens every workgroup also writes a share of recv_count and
// layout_range (begin, count per expert and source segment of M tokens),
// read off the per-block offsets: blocks of B tokens with B dividing M, so
// segment s starts at block s * M / B. VPT = steps of 16
// values per thread per pass over the row.
//
// SUMMED: no reduction launch ran before this kernel; the per-block offsets
// it would have produced are summed here from the layout's per-block counts
// (nb blocks). A slot's offset is its expert's count over the blocks before
// the token's block, summed by 8 lanes of the first wave (lane l takes blocks
// l, l + 8, ...) and combined with lane shuffles, one token ahead like the
// lookups it replaces; each (expert, segment) entry of layout_range is summed by one
// thread; workgroup 0 ORs the layout's error bits into the status word,
// which layout block 0 has cleared.
template <int VPT, bool SUMMED>
__global__ __launch_bounds__(kScatterThreads) void ep_ll_scatter_kernel(
    const uint16_t *__restrict__ x, int H, const int64_t *__restrict__ topk,
    const int32_t *__restrict__ block_base, const int32_t *__restrict__ slot_rank,
    const int32_t *__restrict__ counts, int64_t T, int K, int E, int B, int M, int64_t cap,
    uint8_t *__restrict__ out, float *__restrict__ out_scale, int32_t *__restrict__ recv_count,
    int32_t *__restrict__ src_info, int32_t *__restrict__ layout_range,
    int32_t *__restrict__ output_index, uint32_t *__restrict__ status,
    const int32_t *__restrict__ block_count, const uint32_t *__restrict__ block_err, int64_t nb,
    int parts)
{
    __shared__ int32_t s_e[2][kMaxTopk];      // expert of each placed slot, -1 if none
    __shared__ int32_t s_j[2][kMaxTopk];      // row within the expert's block
    const int tid = threadIdx.x;
    const int S = H / 128;                    // 128-column groups: 8 pairs of 16-byte vectors
    // Work items: (token, column part) pairs, item i = token i / parts, part
    // i % parts; a part is a run of whole 128-column groups (8 pairs each).
    const int gpp = (S + parts - 1) / parts;  // groups per part
    auto item_token = [&](int64_t i) { return (int64_t)((uint64_t)i / (uint32_t)parts); };
    auto item_pairs = [&](int64_t i, int &p0, int &p1) {
        const int q = (int)((uint64_t)i % (uint32_t)parts);
        p0 = 8 * min(S, q * gpp);
        p1 = 8 * min(S, (q + 1) * gpp);
    };

    // recv_count and layout_range
    {
        const int64_t nseg = T / M;
        const int64_t bps = M / B;
        const int64_t n = (int64_t)E * nseg;
        const int64_t g0 = (int64_t)blockIdx.x * kScatterThreads + tid;
        const int64_t gs = (int64_t)gridDim.x * kScatterThreads;
        if (SUMMED) {
            // entry (e, sg): expert e's counts over the blocks before segment
            // sg and through it; the last segment's end is e's total
            for (int64_t i = g0; i < n; i += gs) {
                const int e = (int)(i / nseg);
                const int64_t sg = i % nseg;
                const int64_t bb0 = sg * bps, bb1 = bb0 + bps;
                int before = 0, within = 0;
#pragma unroll 8
                for (int64_t bb = 0; bb < bb1; ++bb) {
                    const int c = block_count[bb * E + e];
                    if (bb < bb0)
                        before += c;
                    else
                        within += c;
                }
                const int64_t b0 = min((int64_t)before, cap);
                const int64_t b1 = min((int64_t)before + within, cap);
                layout_range[2 * i] = (int32_t)b0;
                layout_range[2 * i + 1] = (int32_t)(b1 - b0);
                if (sg == nseg - 1)
                    recv_count[e] = (int32_t)b1;
            }
            if (blockIdx.x == 0) {
                uint32_t err = 0;
                for (int64_t bb = tid; bb < nb; bb += kScatterThreads)
                    err |= block_err[bb];
                if (err)
                    atomicOr(status, kStatusBadExpert);
            }
        } else {
            for (int64_t e = g0; e < E; e += gs)
                recv_count[e] = (int32_t)min((int64_t)counts[e], cap);
            for (int64_t i = g0; i < n; i += gs) {
                const int e = (int)(i / nseg);
                const int64_t sg = i % nseg;
                const int64_t b0 = min((int64_t)block_base[(sg * bps) * E + e], cap);
                const int64_t b1 = sg + 1 < nseg ? min((int64_t)block_base[((sg + 1) * bps) * E + e], cap)
                                                 : min((int64_t)counts[e], cap);
                layout_range[2 * i] = (int32_t)b0;
                layout_range[2 * i + 1] = (int32_t)(b1 - b0);
            }
        }
    }

    // slot `tid` of token t: place it and publish (expert, row) in the table;
    // the token's first part also stores its indices
    auto place = [&](int64_t t, bool first, int32_t *se, int32_t *sj) {
        const int64_t e = topk[t * K + tid];
        int32_t pe = -1, pj = 0, oi = -1;
        if (e >= 0 && e < E) {
            const uint32_t tu = (uint32_t)t;   // T * K <= INT32_MAX
            const int64_t j = (int64_t)block_base[(int64_t)(tu / (uint32_t)B) * E + e] +
                              slot_rank[t * K + tid];
            if (j < cap) {
                const int64_t row = e * cap + j;
                pe = (int32_t)e;
                pj = (int32_t)j;
                oi = (int32_t)row;
                if (first)
                    src_info[row] = (int32_t)(tu % (uint32_t)M);
            } else if (first) {
                atomicOr(status, kStatusCapacity);
            }
        }
        if (first)
            output_index[t * K + tid] = oi;
        se[tid] = pe;
        sj[tid] = pj;
    };
    // SUMMED: the first wave places token t, 8 lanes per slot (slots k0 +
    // lane / 8), while the other waves go on to the current token's cast
    auto place_summed = [&](int64_t t, bool first, int32_t *se, int32_t *sj) {
        if (tid >= kWave)
            return;
        const int l = tid & 7;
        const uint32_t tu = (uint32_t)t;   // T * K <= INT32_MAX
        const int64_t b = tu / (uint32_t)B;
        for (int k0 = 0; k0 < K; k0 += kWave / 8) {
            const int k = k0 + tid / 8;
            if (k >= K)                     // whole 8-lane groups drop out together
                break;
            const int64_t e = topk[t * K + k];
            const bool ok = e >= 0 && e < E;
            const int r = ok && l == 0 ? slot_rank[t * K + k] : 0;
            int part = 0;
            if (ok)
                for (int64_t bb = l; bb < b; bb += 8)
                    part += block_count[bb * E + e];
            part += __shfl_xor(part, 4, 8);
            part += __shfl_xor(part, 2, 8);
            part += __shfl_xor(part, 1, 8);
            if (l == 0) {
                int32_t pe = -1, pj = 0, oi = -1;
                if (ok) {
                    const int64_t j = (int64_t)part + r;
                    if (j < cap) {
                        const int64_t row = e * cap + j;
                        pe = (int32_t)e;
                        pj = (int32_t)j;
                        oi = (int32_t)row;
                        if (first)
                            src_info[row] = (int32_t)(tu % (uint32_t)M);
                    } else if (first) {
                        atomicOr(status, kStatusCapacity);
                    }
                }
                if (first)
                    output_index[t * K + k] = oi;
                se[k] = pe;
                sj[k] = pj;
            }
        }
    };
    // whether token t has a slot at all (uniform: every wave reads the ids)
    auto has_slot = [&](int64_t t) {
        bool any = false;
        for (int k = 0; k < K; ++k) {
            const int64_t e = topk[t * K + k];
            any |= e >= 0 && e < E;
        }
        return any;
    };
    // pass `base` (in pairs) of token t's row; ordinary loads, as in the
    // scatter (non-temporal loads of the token rows were slower here: 80.7
    // against 71.9 us with the batch in the Infinity Cache, 81.6 against
    // 80.3 us without)
    // pairs [p0 + base, p1) of token t's row, VPT steps of the workgroup;
    // ordinary loads, as in the scatter (non-temporal loads of the token rows
    // were slower here: 80.7 against 71.9 us with the batch in the Infinity
    // Cache, 81.6 against 80.3 us without)
    auto load_row = [&](int64_t t, int p0, int p1, int base, u32x4 (*v)[2]) {
        const u32x4 *xrow = reinterpret_cast<const u32x4 *>(x + t * (int64_t)H);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int pi = p0 + base + i * kScatterThreads + tid;
            if (pi < p1) {
                v[i][0] = xrow[2 * pi];
                v[i][1] = xrow[2 * pi + 1];
            }
        }
    };

    const TokenRange tr = token_range(T * parts);
    const bool lead = tid < K;
    u32x4 v[VPT][2], vn[VPT][2];
    bool any = false;
    int p0 = 0, p1 = 0;
    if (tr.first < tr.end) {
        const int64_t t = item_token(tr.first);
        const bool first = t * parts == tr.first;
        item_pairs(tr.first, p0, p1);
        if (!SUMMED && lead)
            place(t, first, s_e[0], s_j[0]);
        any = has_slot(t);
        if (any)
            load_row(t, p0, p1, 0, v);
        if (SUMMED)
            place_summed(t, first, s_e[0], s_j[0]);
    }
    int it = 0;
    for (int64_t item = tr.first; item < tr.end; item += tr.stride, ++it) {
        lds_barrier();
        const int64_t t = item_token(item);
        const int32_t *se = s_e[it & 1], *sj = s_j[it & 1];
        // the next item: its row loads and its placements overlap this
        // item's cast and stores
        const int64_t in = item + tr.stride;
        const int64_t tn = in < tr.end ? item_token(in) : 0;
        const bool first_next = tn * parts == in;
        int q0 = 0, q1 = 0;
        if (in < tr.end)
            item_pairs(in, q0, q1);
        const bool any_next = in < tr.end && has_slot(tn);
        if (any_next)
            load_row(tn, q0, q1, 0, vn);
        if (SUMMED && in < tr.end)
            place_summed(tn, first_next, s_e[(it + 1) & 1], s_j[(it + 1) & 1]);
        else if (lead && in < tr.end)
            place(tn, first_next, s_e[(it + 1) & 1], s_j[(it + 1) & 1]);

        for (int base = 0; any;) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int pi = p0 + base + i * kScatterThreads + tid;
                if (pi >= p1)         // whole 8-lane groups drop out together (p0, p1 % 8 == 0)
                    continue;
                const Cast16 c = cast_e4m3_16(v[i]);
                const u32x4 codes = c.codes;
                const float scale = c.scale;
                const int g = pi / 8;
                for (int k = 0; k < K; ++k) {
                    const int e = se[k];
                    if (e < 0)
                        continue;
                    const int64_t j = sj[k];
                    const int64_t row = (int64_t)e * cap + j;
                    __builtin_nontemporal_store(codes, reinterpret_cast<u32x4 *>(out + row * H) + pi);
                }
                // every lane of the group holds the scale: lane q stores it
                // for slots q, q + 8, ... (one store instruction for 8 slots)
                for (int k = tid & 7; k < K; k += 8) {
                    const int e = se[k];
                    if (e < 0)
                        continue;
                    out_scale[((int64_t)e * S + g) * cap + sj[k]] = scale;
                }
            }
            base += kScatterThreads * VPT;
            if (p0 + base >= p1)
                break;
            load_row(t, p0, p1, base, v);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            v[i][0] = vn[i][0];
            v[i][1] = vn[i][1];
        }
        any = any_next;
        p0 = q0;
        p1 = q1;
    }
}

// ------------------------------- low-latency dispatch of decode sizes --

// Arguments of ep_ll_decode_kernel (those of the three-launch path).
struct LLArgs {
    const uint16_t *x;
    int H;
    const int64_t *topk;
    int64_t T;
    int K, E, M;
    int64_t cap;
    uint8_t *out;
    float *out_scale;
    int32_t *recv_count;
    int32_t *src_info;
    int32_t *layout_range;
    int32_t *output_index;
    uint32_t *status;
};

// Slots of a low-latency batch dispatched in one launch, at most: twice the
// bf16 decode limit, since the cast (one row in, K rows out, all by one
// workgroup) gains more from the one launch than the bf16 copy does (512
// DeepSeek-V3-shaped tokens: step 39.0 -> 30.9 us, where the bf16 dispatch
// got slower at 4096 slots).
constexpr int kLLDecodeMaxSlots = 2 * kFusedMaxSlots;

// Workgroup 0 of ep_ll_decode_kernel: slots per (source segment, expert) in
// LDS ([T / M][E] words of dynamic LDS), then per expert a running sum over
// the segments clipped to the rectangle gives layout_range and recv_count.
// The status word gets the id error bit and the capacity bit, set exactly
// when an expert has more slots than rows, i.e. when some slot finds no row.
__device__ __forceinline__ void ll_decode_counts_block(const LLArgs &a)
{
    extern __shared__ int32_t s_seg_cnt[];
    __shared__ uint32_t s_err;
    const int tid = threadIdx.x;
    const int K = a.K, E = a.E;
    const int64_t nseg = a.T / a.M;
    const int64_t n = nseg * E;
    const int ns = (int)(a.T * K);
    for (int64_t i = tid; i < n; i += kFusedThreads)
        s_seg_cnt[i] = 0;
    if (tid == 0)
        s_err = 0u;
    lds_barrier();
    bool bad = false;
    for (int sl = tid; sl < ns; sl += kFusedThreads) {
        const int64_t e = a.topk[sl];
        bad |= (e < -1 || e >= E);
        if (e >= 0 && e < E)
            atomicAdd(&s_seg_cnt[(int64_t)(sl / K / a.M) * E + e], 1);
    }
    if (bad)
        atomicOr(&s_err, kStatusBadExpert);
    lds_barrier();
    bool over = false;
    for (int e = tid; e < E; e += kFusedThreads) {
        int64_t run = 0;
        for (int64_t sg = 0; sg < nseg; ++sg) {
            const int64_t b0 = min(run, a.cap);
            run += s_seg_cnt[sg * E + e];
            const int64_t i = (int64_t)e * nseg + sg;
            a.layout_range[2 * i] = (int32_t)b0;
            a.layout_range[2 * i + 1] = (int32_t)(min(run, a.cap) - b0);
        }
        a.recv_count[e] = (int32_t)min(run, a.cap);
        over |= run > a.cap;
    }
    if (over)
        atomicOr(&s_err, kStatusCapacity);
    lds_barrier();
    if (tid == 0)
        *a.status = s_err;
}

// The low-latency dispatch of a decode-sized batch (at most kLLDecodeMaxSlots
// slots; SLOTS_PER_THREAD = 2 up to 2048 slots, 4 up to 4096) in one launch
// of 1 + T workgroups of kFusedThreads threads, with the
// outputs of the layout, reduction and ep_ll_scatter_kernel launches.
// Workgroup 0 writes recv_count, layout_range and the status word
// (ll_decode_counts_block). Workgroup 1 + t issues token t's row loads, then
// counts for each of its K slots, with wave ballots over all slots, the
// earlier slots of the same expert in (token, k) order: that count is the
// slot's row j in its expert's block. It stores output_index and src_info,
// casts the row (16 values per thread, a 128-column group over 8 lanes, as in
// ep_ll_scatter_kernel) and stores the codes and scales to every placed row.
template <int SLOTS_PER_THREAD>
__global__ __launch_bounds__(kFusedThreads) void ep_ll_decode_kernel(LLArgs a)
{
    if (blockIdx.x == 0) {
        ll_decode_counts_block(a);
        return;
    }
    constexpr int kSlotsPerThread = SLOTS_PER_THREAD;
    __shared__ int32_t s_tok[kMaxTopk];                  // the token's expert ids (-1: none)
    __shared__ int32_t s_same[kMaxTopk][kFusedWaves];    // per wave: earlier slots of the expert
    __shared__ int32_t s_e[kMaxTopk];                    // expert of each placed slot, -1 if none
    __shared__ int32_t s_j[kMaxTopk];                    // its row within the expert's block
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int64_t t = blockIdx.x - 1;
    const int K = a.K, E = a.E;
    const int S = a.H / 128;
    const int ns = (int)(a.T * K);
    const int npair = a.H / 16;                          // 16 bf16 values per thread and pass

    const u32x4 *xrow = reinterpret_cast<const u32x4 *>(a.x + t * (int64_t)a.H);
    u32x4 v[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (tid < npair) {
        v[0] = xrow[2 * tid];
        v[1] = xrow[2 * tid + 1];
    }
    int my_key[kSlotsPerThread];
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
        const int sl = i * kFusedThreads + tid;
        const int64_t e = sl < ns ? a.topk[sl] : -1;
        my_key[i] = (e >= 0 && e < E) ? (int)e : -1;
    }
    if (tid < K) {
        const int64_t e = a.topk[t * K + tid];
        s_tok[tid] = (e >= 0 && e < E) ? (int)e : -1;
    }
    lds_barrier();
    auto count_slot = [&](int k, int ek) {
        const int sk = (int)t * K + k;
        int same = 0;
#pragma unroll
        for (int i = 0; i < kSlotsPerThread; ++i) {
            const int sl = i * kFusedThreads + tid;
            same += __popcll(wave_ballot(ek >= 0 && my_key[i] == ek && sl < sk));
        }
        if (lane == 0)
            s_same[k][tid / kWave] = same;
    };
    if (K <= kDecodeFastTopk) {
        int tok[kDecodeFastTopk];
#pragma unroll
        for (int k = 0; k < kDecodeFastTopk; ++k)
            tok[k] = k < K ? s_tok[k] : -1;
#pragma unroll
        for (int k = 0; k < kDecodeFastTopk; ++k)
            if (k < K)
                count_slot(k, tok[k]);
    } else {
        for (int k = 0; k < K; ++k)
            count_slot(k, s_tok[k]);
    }
    lds_barrier();
    if (tid < K) {
        int j = 0;
        for (int w = 0; w < kFusedWaves; ++w)
            j += s_same[tid][w];
        const int e = s_tok[tid];
        int32_t oi = -1;
        int pe = -1;
        if (e >= 0 && j < a.cap) {
            const int64_t row = (int64_t)e * a.cap + j;
            oi = (int32_t)row;
            pe = e;
            a.src_info[row] = (int32_t)(t % a.M);
        }
        a.output_index[t * K + tid] = oi;
        s_e[tid] = pe;
        s_j[tid] = j;
    }
    lds_barrier();

    // whole 8-lane groups are active or idle together (npair % 8 == 0)
    for (int pi = tid; pi < npair; pi += kFusedThreads) {
        if (pi != tid) {
            v[0] = xrow[2 * pi];
            v[1] = xrow[2 * pi + 1];
        }
        const Cast16 c = cast_e4m3_16(v);
        const int g = pi / 8;
        for (int k = 0; k < K; ++k) {
            const int e = s_e[k];
            if (e < 0)
                continue;
            const int64_t row = (int64_t)e * a.cap + s_j[k];
            __builtin_nontemporal_store(c.codes, reinterpret_cast<u32x4 *>(a.out + row * a.H) + pi);
        }
        for (int k = tid & 7; k < K; k += 8) {
            const int e = s_e[k];
            if (e < 0)
                continue;
            a.out_scale[((int64_t)e * S + g) * a.cap + s_j[k]] = c.scale;
        }
    }
}

// -------------------------------------------------------------- combine --

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return ((u >> 16) | 0x40u) & 0xFFFFu;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Column vectors per thread per pass (the combine's unroll): kCombineUnroll
// from kCombineFewBelow tokens on, kCombineUnrollFew below. With few tokens
// the smaller unroll cuts each token into more, smaller column parts, so the
// launch's last workgroups finish sooner (about 1% at 4096 tokens of hidden
// 7168, 5% at 2048 tokens of hidden 4096); from 16384 tokens on the extra
// per-part overhead costs more than the shorter tail saves (0.5-0.7%).
constexpr int kCombineUnroll = EPL_COMBINE_UNROLL;
constexpr int kCombineUnrollFew = EPL_COMBINE_UNROLL_FEW;
constexpr int64_t kCombineFewBelow = EPL_COMBINE_FEW_BELOW;
constexpr int kCombineMaxParts = 64;                  // column parts per token, at most

#ifndef EPL_COMBINE_LOAD_NT
#define EPL_COMBINE_LOAD_NT 1
#endif
// The gathered expert-output rows are read once: non-temporal loads.
template <typename V>
__device__ __forceinline__ V load_row_vec(const V *p)
{
    if (EPL_COMBINE_LOAD_NT)
        return __builtin_nontemporal_load(p);
    return *p;
}

// The combine's output rows: write-back stores while y fits comfortably in
// the Infinity Cache (the host decides, see kYNtBytes), so the step that
// follows finds them there; non-temporal stores for a larger y, which would
// only be evicted again and drain during the next kernels.
// (A template parameter, not a run-time flag: the compiler would merge the
// two stores of a run-time branch into one plain store.)
template <bool NT, typename V>
__device__ __forceinline__ void store_y(V *dst, const V &v)
{
    if (NT)
        __builtin_nontemporal_store(v, dst);
    else
        *dst = v;
}

// Column units of the combine: 8 columns (16-byte loads) for a bf16 y, whose
// 8 outputs are again 16 bytes; 4 columns (8-byte loads) for an fp32 y, so
// that each 16-byte store of 4 outputs sits next to its neighbour lane's and
// a store instruction covers one contiguous span (8 columns per lane would
// leave every other 16 bytes of a span to a second instruction, which
// non-temporal stores write to memory as partial lines).
__host__ __device__ constexpr int combine_unit_cols(bool out_bf16) { return out_bf16 ? 8 : 4; }
// Units a thread covers in one pass.
__host__ __device__ constexpr int combine_units_per_thread(bool out_bf16, int unroll)
{
    return out_bf16 ? unroll : 2 * unroll;
}

// One work item per (token, column part), grid-stride over the items:
// y[t] = sum over valid k (ascending) of w[t,k] * expert_out[output_index[t,k]],
// fp32 accumulation, item t * parts + q covering the q-th of `parts` equal
// column ranges of row t. The host picks parts so that a workgroup covers
// its range in one pass: the work per workgroup shrinks and the last
// workgroups of a launch finish sooner. Each thread issues the loads of up to
// 8 gathered rows for all of its units before accumulating. The gathered rows
// are read once, so the loads are non-temporal. The first wave fetches the
// next item's output_index / weights while the current one streams; the
// compacted slot table is double-buffered in LDS (see ep_scatter_kernel).
template <bool OUT_BF16, bool Y_NT, int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void ep_combine_kernel(
    const uint16_t *__restrict__ expert_out, int64_t rows, const int32_t *__restrict__ oi,
    const float *__restrict__ w, int64_t T, int K, int H, int parts, bool xcd_ranges,
    void *__restrict__ y, uint32_t *__restrict__ status)
{
    __shared__ int64_t s_row[2][kMaxTopk];
    __shared__ float s_w[2][kMaxTopk];
    __shared__ int s_n[2];
    const int tid = threadIdx.x;
    const TokenRange tr = token_range(T * parts, xcd_ranges);
    const int64_t step = tr.stride, i_end = tr.end;

    int64_t p_next = -1;
    float w_next = 0.0f;
    if (tid < K && tr.first < i_end) {
        p_next = oi[(tr.first / parts) * K + tid];
        w_next = w[(tr.first / parts) * K + tid];
    }

    constexpr int CW = combine_unit_cols(OUT_BF16);
    constexpr int UU = combine_units_per_thread(OUT_BF16, UNROLL);
    using In = typename std::conditional<CW == 8, u32x4, u32x2>::type;
    const int nunit_row = H / CW;
    const int part_units = (nunit_row + parts - 1) / parts;

    int it = 0;
    for (int64_t item = tr.first; item < i_end; item += step, ++it) {
        const int64_t t = item / parts;
        const int q = (int)(item - t * parts);
        const int buf = it & 1;
        if (tid < kWave) {
            // Compact the valid slots, keeping ascending k: lane k finds its
            // place among the lower valid lanes with one ballot (K <= 64).
            int64_t p = p_next;
            const float wt = w_next;
            if (tid < K && item + step < i_end) {
                p_next = oi[((item + step) / parts) * K + tid];
                w_next = w[((item + step) / parts) * K + tid];
            }
            if (p >= rows) {
                if (status)
                    atomicOr(status, kStatusBadRow);
                p = -1;
            }
            const bool ok = p >= 0;
            const uint64_t valid = wave_ballot(ok);
            const uint64_t lower = (tid == 0) ? 0ull : (~0ull >> (kWave - tid));
            if (ok) {
                const int slot = __popcll(valid & lower);
                s_row[buf][slot] = p;
                s_w[buf][slot] = wt;
            }
            if (tid == 0)
                s_n[buf] = __popcll(valid);
        }
        lds_barrier();
        const int n = s_n[buf];
        const int64_t *srow = s_row[buf];
        const float *sw = s_w[buf];

        // this item's units: [q * part_units, nunit)
        const int nunit = min(nunit_row, (q + 1) * part_units);
        for (int base = q * part_units + tid; base < nunit; base += THREADS * UU) {
            float acc[UU][CW];
#pragma unroll
            for (int u = 0; u < UU; ++u)
#pragma unroll
                for (int j = 0; j < CW; ++j)
                    acc[u][j] = 0.0f;
            for (int g = 0; g < n; g += 8) {
                In v[UU][8];
#pragma unroll
                for (int u = 0; u < UU; ++u) {
                    const int idx = base + u * THREADS;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (g + j < n && idx < nunit)
                            v[u][j] = load_row_vec(
                                reinterpret_cast<const In *>(expert_out + srow[g + j] * H) + idx);
                }
#pragma unroll
                for (int u = 0; u < UU; ++u)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (g + j < n) {
                            const float wj = sw[g + j];
#pragma unroll
                            for (int pr = 0; pr < CW / 2; ++pr) {
                                acc[u][2 * pr] = fmaf(wj, bf16_lo(v[u][j][pr]), acc[u][2 * pr]);
                                acc[u][2 * pr + 1] =
                                    fmaf(wj, bf16_hi(v[u][j][pr]), acc[u][2 * pr + 1]);
                            }
                        }
            }
#pragma unroll
            for (int u = 0; u < UU; ++u) {
                const int idx = base + u * THREADS;
                if (idx >= nunit)
                    continue;
                if (OUT_BF16) {
                    u32x4 o = {pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3]),
                               pack_bf16x2(acc[u][4], acc[u][5]), pack_bf16x2(acc[u][6], acc[u][7])};
                    store_y<Y_NT>(reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(y) + t * H) + idx, o);
                } else {
                    store_y<Y_NT>(reinterpret_cast<f32x4 *>(static_cast<float *>(y) + t * H) + idx,
                                  f32x4{acc[u][0], acc[u][1], acc[u][2], acc[u][3]});
                }
            }
        }
    }
}

// --------------------------------------------------------- expert stand-in --

// rows_out[p] = bf16_rne(rows_in[p] * (1 + m_indices[p] / 256)) for
// p < min(total, capacity). The factor has 9 significant bits and a bf16
// value 8, so the fp32 product is exact and only the final rounding remains.
__global__ __launch_bounds__(kRowThreads) void ep_expert_scale_kernel(
    const uint16_t *__restrict__ in, const int32_t *__restrict__ m_indices, int64_t capacity,
    const WsHeader *__restrict__ hdr, int H, uint16_t *__restrict__ out)
{
    const int64_t n = min((int64_t)hdr->total, capacity);
    const int nvec = H >> 3;
    for (int64_t p = blockIdx.x; p < n; p += gridDim.x) {
        if (m_indices[p] < 0)
            continue;   // padding row of an aligned block
        const float f = 1.0f + (float)m_indices[p] * (1.0f / 256.0f);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(in + p * H);
        u32x4 *dst = reinterpret_cast<u32x4 *>(out + p * H);
        for (int idx = threadIdx.x; idx < nvec; idx += kRowThreads) {
            const u32x4 v = src[idx];
            dst[idx] = u32x4{pack_bf16x2(bf16_lo(v.x) * f, bf16_hi(v.x) * f),
                             pack_bf16x2(bf16_lo(v.y) * f, bf16_hi(v.y) * f),
                             pack_bf16x2(bf16_lo(v.z) * f, bf16_hi(v.z) * f),
                             pack_bf16x2(bf16_lo(v.w) * f, bf16_hi(v.w) * f)};
        }
    }
}

}  // namespace epl
