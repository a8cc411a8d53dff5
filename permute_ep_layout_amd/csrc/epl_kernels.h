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
//
// Determinism. Counts are integer sums, so atomics would already give exact
// counts; row positions are another matter. Here nothing about positions
// depends on timing: the layout kernel splits the tokens into fixed blocks
// and, inside a block, ranks every slot among the earlier slots of the same
// expert in (token, k) order with wavefront ballots; the scan kernel turns
// the per-block counts into per-block offsets (a prefix over blocks per
// expert); the scatter kernel adds expert offset + block offset + rank.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epl {

constexpr int kWave = 64;
constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kMaxSlotsPerBlock = 2048;   // B * K per layout block
constexpr int kMaxTopk = 64;
constexpr int kMaxExperts = 2048;
constexpr int kScanThreads = 1024;
constexpr int kRowThreads = 128;          // scatter / combine / expert-scale workgroup

// Status word bits (workspace header).
constexpr uint32_t kStatusBadExpert = 1u;      // topk id outside [-1, E)
constexpr uint32_t kStatusCapacity = 2u;       // routed rows > capacity rows
constexpr uint32_t kStatusBadRow = 4u;         // combine: output_index >= expert rows

constexpr int kScanReduce = 1;   // per-block counts -> per-block offsets, totals
constexpr int kScanPrefix = 2;   // totals -> expert_start_loc and N

struct WsHeader {
    uint32_t status;
    int32_t total;
    int32_t pad[62];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

__device__ __forceinline__ uint64_t wave_ballot(bool pred)
{
    return __builtin_amdgcn_ballot_w64(pred);
}

__device__ __forceinline__ int lane_id()
{
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// --------------------------------------------------------------- layout --

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

// One workgroup per block of B tokens (B * K <= kMaxSlotsPerBlock).
// Outputs: in_rank rows of the block's tokens; block_count[b][e] (slots of
// expert e in block b); block_rank[b][r] (tokens of block b sent to rank r);
// block_err[b]; slot_rank[t*K+k] = rank of slot (t,k) among the block's
// earlier slots of the same expert, or -1 for an invalid slot.
__global__ __launch_bounds__(kLayoutThreads) void ep_layout_kernel(
    const int64_t *__restrict__ topk, int64_t T, int K, int E, int R, int experts_per_rank,
    int B, uint8_t *__restrict__ in_rank, bool in_rank_vec16,
    int32_t *__restrict__ block_count, int32_t *__restrict__ block_rank,
    uint32_t *__restrict__ block_err, int32_t *__restrict__ slot_rank)
{
    extern __shared__ int32_t lds[];
    const int max_slots = B * K;
    int32_t *keys = lds;                                  // [B*K]
    int32_t *lrank = keys + max_slots;                    // [B*K] rank within the owning wave
    int32_t *wave_cnt = lrank + max_slots;                // [waves][E]
    int32_t *rank_cnt = wave_cnt + kLayoutWaves * E;      // [R]
    int32_t *s_err = rank_cnt + R;                        // [1]

    const int64_t b = blockIdx.x;
    const int64_t t0 = b * B;
    const int nt = (int)min((int64_t)B, T - t0);
    const int ns = nt * K;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;

    for (int i = tid; i < kLayoutWaves * E; i += kLayoutThreads)
        wave_cnt[i] = 0;
    for (int i = tid; i < R; i += kLayoutThreads)
        rank_cnt[i] = 0;
    if (tid == 0)
        *s_err = 0;

    // Keys of the block's slots, in (token, k) order; bad ids become -1.
    const int64_t *src = topk + t0 * K;
    bool bad = false;
    for (int s = tid; s < ns; s += kLayoutThreads) {
        const int64_t e = src[s];
        int key = (int)e;
        if (e < -1 || e >= E) {
            bad = true;
            key = -1;
        }
        keys[s] = key;
    }
    __syncthreads();
    if (bad)
        atomicOr(reinterpret_cast<uint32_t *>(s_err), 1u);

    // Rank of each slot among the earlier slots with the same key. Wave w
    // owns a contiguous run of 64-slot chunks and walks it in order; inside a
    // chunk, lanes holding the same key are found with one ballot per
    // distinct key, and a lane's rank is the number of lower lanes in that
    // ballot plus the wave's running count for the key.
    const int nchunks = (ns + kWave - 1) / kWave;
    const int cpw = (nchunks + kLayoutWaves - 1) / kLayoutWaves;
    {
        int32_t *my_cnt = wave_cnt + wave * E;
        const int c_end = min(nchunks, (wave + 1) * cpw);
        const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
        for (int c = wave * cpw; c < c_end; ++c) {
            const int s = c * kWave + lane;
            const int key = (s < ns) ? keys[s] : -1;
            uint64_t todo = wave_ballot(key >= 0);
            while (todo) {
                const int leader = (int)__builtin_ctzll(todo);
                const int lkey = __builtin_amdgcn_readlane(key, leader);
                const uint64_t same = wave_ballot(key == lkey);
                const int base = my_cnt[lkey];
                if (key == lkey)
                    lrank[s] = base + __popcll(same & lower);
                if (lane == leader)
                    my_cnt[lkey] = base + __popcll(same);
                todo &= ~same;
            }
        }
    }

    // Token -> rank mask (one thread per token) and tokens per rank, one
    // 64-rank window at a time; rank counts are summed with ballots.
    {
        const bool tok = tid < nt;
        for (int w0 = 0; w0 < R; w0 += 64) {
            const int wr = min(64, R - w0);
            uint64_t mask = 0;
            if (tok) {
                for (int k = 0; k < K; ++k) {
                    const int e = keys[tid * K + k];
                    if (e >= 0) {
                        const int r = e / experts_per_rank - w0;
                        if (r >= 0 && r < wr)
                            mask |= 1ull << r;
                    }
                }
                store_mask_bytes(in_rank + (t0 + tid) * R + w0, mask, wr, in_rank_vec16);
            }
            for (int r = 0; r < wr; ++r) {
                const uint64_t has = wave_ballot((mask >> r) & 1u);
                if (lane == 0 && has)
                    atomicAdd(&rank_cnt[w0 + r], __popcll(has));
            }
        }
    }
    __syncthreads();

    // Per expert: exclusive prefix over the waves (in place) and block total.
    for (int e = tid; e < E; e += kLayoutThreads) {
        int run = 0;
        for (int w = 0; w < kLayoutWaves; ++w) {
            const int c = wave_cnt[w * E + e];
            wave_cnt[w * E + e] = run;
            run += c;
        }
        block_count[b * E + e] = run;
    }
    for (int r = tid; r < R; r += kLayoutThreads)
        block_rank[b * R + r] = rank_cnt[r];
    __syncthreads();
    if (tid == 0)
        block_err[b] = (uint32_t)*s_err;

    for (int s = tid; s < ns; s += kLayoutThreads) {
        const int key = keys[s];
        const int w = (s / kWave) / cpw;
        slot_rank[t0 * K + s] = key >= 0 ? lrank[s] + wave_cnt[w * E + key] : -1;
    }
}

// ----------------------------------------------------------------- scan --

// Inclusive prefix sum over the workgroup (kScanThreads threads).
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
    __syncthreads();
    if (wave == 0) {
        constexpr int nw = kScanThreads / kWave;
        int x = lane < nw ? s_wave[lane] : 0;
        for (int d = 1; d < nw; d <<= 1) {
            const int o = __shfl_up(x, d, kWave);
            if (lane >= d)
                x += o;
        }
        if (lane < nw)
            s_wave[lane] = x;
    }
    __syncthreads();
    return v + (wave > 0 ? s_wave[wave - 1] : 0);
}

// Single workgroup. kScanReduce: column sums of block_count / block_rank
// give num_tokens_per_expert / num_tokens_per_rank, block_count is replaced
// by its exclusive prefix over blocks, and the status word is reset to the
// layout's error bits. kScanPrefix: exclusive prefix of the per-expert
// counts (read from `cnt` unless kScanReduce produced them) into
// expert_start_loc, total into the header.
__global__ __launch_bounds__(kScanThreads) void ep_scan_kernel(
    int mode, int64_t nb, int E, int R, int32_t *__restrict__ block_count,
    const int32_t *__restrict__ block_rank, const uint32_t *__restrict__ block_err,
    int32_t *__restrict__ cnt, int32_t *__restrict__ per_rank, int32_t *__restrict__ start,
    WsHeader *__restrict__ hdr)
{
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_seg[kScanThreads > kMaxExperts ? kScanThreads : kMaxExperts];
    __shared__ int s_wave[kScanThreads / kWave];
    __shared__ uint32_t s_err;
    const int tid = threadIdx.x;

    if (mode & kScanReduce) {
        if (tid == 0)
            s_err = 0;
        // Columns split into P segments of blocks so all threads have work.
        const int P = E <= kScanThreads ? kScanThreads / E : 1;
        const int64_t L = (nb + P - 1) / P;
        for (int col = tid; col < E * P; col += kScanThreads) {
            const int e = col % E;
            const int q = col / E;
            const int64_t b0 = q * L, b1 = min(nb, b0 + L);
            int sum = 0;
            for (int64_t bb = b0; bb < b1; ++bb)
                sum += block_count[bb * E + e];
            s_seg[q * E + e] = sum;
        }
        uint32_t err = 0;
        for (int64_t bb = tid; bb < nb; bb += kScanThreads)
            err |= block_err[bb];
        __syncthreads();
        if (err)
            atomicOr(&s_err, err);
        for (int e = tid; e < E; e += kScanThreads) {
            int run = 0;
            for (int q = 0; q < P; ++q) {
                const int v = s_seg[q * E + e];
                s_seg[q * E + e] = run;
                run += v;
            }
            s_cnt[e] = run;
            cnt[e] = run;
        }
        __syncthreads();
        // Rewrite block_count as the exclusive prefix over blocks; loads of
        // a batch are issued together before its stores.
        for (int col = tid; col < E * P; col += kScanThreads) {
            const int e = col % E;
            const int q = col / E;
            const int64_t b0 = q * L, b1 = min(nb, b0 + L);
            int run = s_seg[q * E + e];
            for (int64_t bb = b0; bb < b1; bb += 16) {
                int v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    v[j] = (bb + j < b1) ? block_count[(bb + j) * E + e] : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (bb + j < b1) {
                        block_count[(bb + j) * E + e] = run;
                        run += v[j];
                    }
                }
            }
        }
        for (int r = tid; r < R; r += kScanThreads) {
            int sum = 0;
            for (int64_t bb = 0; bb < nb; ++bb)
                sum += block_rank[bb * R + r];
            per_rank[r] = sum;
        }
        __syncthreads();
        if (tid == 0)
            hdr->status = s_err ? kStatusBadExpert : 0u;
    } else if (mode & kScanPrefix) {
        for (int e = tid; e < E; e += kScanThreads)
            s_cnt[e] = cnt[e];
        __syncthreads();
    }

    if (mode & kScanPrefix) {
        // Two consecutive experts per thread (E <= 2 * kScanThreads).
        const int i0 = 2 * tid, i1 = 2 * tid + 1;
        const int a0 = i0 < E ? s_cnt[i0] : 0;
        const int a1 = i1 < E ? s_cnt[i1] : 0;
        const int incl = block_inclusive_scan(a0 + a1, s_wave);
        const int excl = incl - (a0 + a1);
        if (i0 < E)
            start[i0] = excl;
        if (i1 < E)
            start[i1] = excl + a0;
        if (tid == kScanThreads - 1)
            hdr->total = incl;
    }
}

// -------------------------------------------------------------- scatter --

// One workgroup per token row. The row is read once (16-byte vectors, VPT
// per thread per pass) and written to each of the token's K destination
// rows; the scale row follows it; m_indices and output_index are written by
// the first K threads.
template <int VPT>
__global__ __launch_bounds__(kRowThreads) void ep_scatter_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ x_scale,
    const int64_t *__restrict__ topk, const int32_t *__restrict__ start,
    const int32_t *__restrict__ block_base, const int32_t *__restrict__ slot_rank, int K,
    int E, int H, int S, int B, int64_t capacity, uint16_t *__restrict__ out,
    float *__restrict__ out_scale, int32_t *__restrict__ m_indices,
    int32_t *__restrict__ output_index, uint32_t *__restrict__ status)
{
    __shared__ int64_t s_row[kMaxTopk];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;

    if (tid < K) {
        const int64_t e = topk[t * K + tid];
        const int r = slot_rank[t * K + tid];
        int pos = -1;
        int64_t row = -1;
        if (e >= 0 && e < E) {
            const int64_t p = (int64_t)start[e] + block_base[(t / B) * E + e] + r;
            pos = (int)p;
            if (p >= 0 && p < capacity) {
                row = p;
                m_indices[p] = (int32_t)e;
            } else {
                atomicOr(status, kStatusCapacity);
            }
        }
        output_index[t * K + tid] = pos;
        s_row[tid] = row;
    }

    const int nvec = H >> 3;
    const uint4 *xrow = reinterpret_cast<const uint4 *>(x + t * H);
    bool first = true;
    for (int base = 0; base < nvec; base += kRowThreads * VPT) {
        uint4 v[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = base + i * kRowThreads + tid;
            if (idx < nvec)
                v[i] = xrow[idx];
        }
        if (first) {
            __syncthreads();
            first = false;
        }
        for (int k = 0; k < K; ++k) {
            const int64_t row = s_row[k];
            if (row < 0)
                continue;
            uint4 *orow = reinterpret_cast<uint4 *>(out + row * H);
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kRowThreads + tid;
                if (idx < nvec)
                    orow[idx] = v[i];
            }
        }
    }
    if (first)
        __syncthreads();
    for (int j = tid; j < S; j += kRowThreads) {
        const float f = x_scale[t * S + j];
        for (int k = 0; k < K; ++k) {
            const int64_t row = s_row[k];
            if (row >= 0)
                out_scale[row * S + j] = f;
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

// One workgroup per token: y[t] = sum over valid k (ascending) of
// w[t,k] * expert_out[output_index[t,k]], fp32 accumulation. Each thread
// owns 8 columns at a time and keeps up to 8 gathered rows in flight.
template <bool OUT_BF16>
__global__ __launch_bounds__(kRowThreads) void ep_combine_kernel(
    const uint16_t *__restrict__ expert_out, int64_t rows, const int32_t *__restrict__ oi,
    const float *__restrict__ w, int K, int H, void *__restrict__ y, uint32_t *__restrict__ status)
{
    __shared__ int64_t s_row[kMaxTopk];
    __shared__ float s_w[kMaxTopk];
    __shared__ int s_n;
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;

    if (tid < kWave) {
        // Compact the valid slots, keeping ascending k: lane k finds its
        // place among the lower valid lanes with one ballot (K <= 64).
        int64_t p = -1;
        float wt = 0.0f;
        if (tid < K) {
            p = oi[t * K + tid];
            wt = w[t * K + tid];
            if (p >= rows) {
                if (status)
                    atomicOr(status, kStatusBadRow);
                p = -1;
            }
        }
        const bool ok = p >= 0;
        const uint64_t valid = wave_ballot(ok);
        const uint64_t lower = (tid == 0) ? 0ull : (~0ull >> (kWave - tid));
        if (ok) {
            const int slot = __popcll(valid & lower);
            s_row[slot] = p;
            s_w[slot] = wt;
        }
        if (tid == 0)
            s_n = __popcll(valid);
    }
    __syncthreads();
    const int n = s_n;
    const int nvec = H >> 3;

    for (int idx = tid; idx < nvec; idx += kRowThreads) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = 0.0f;
        for (int g = 0; g < n; g += 8) {
            uint4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (g + j < n)
                    v[j] = reinterpret_cast<const uint4 *>(expert_out + s_row[g + j] * H)[idx];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (g + j < n) {
                    const float wt = s_w[g + j];
                    const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        acc[2 * c] = fmaf(wt, bf16_lo(q[c]), acc[2 * c]);
                        acc[2 * c + 1] = fmaf(wt, bf16_hi(q[c]), acc[2 * c + 1]);
                    }
                }
            }
        }
        if (OUT_BF16) {
            uint4 o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                 pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
            reinterpret_cast<uint4 *>(static_cast<uint16_t *>(y) + t * H)[idx] = o;
        } else {
            float4 *yr = reinterpret_cast<float4 *>(static_cast<float *>(y) + t * H);
            yr[2 * idx] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            yr[2 * idx + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
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
        const float f = 1.0f + (float)m_indices[p] * (1.0f / 256.0f);
        const uint4 *src = reinterpret_cast<const uint4 *>(in + p * H);
        uint4 *dst = reinterpret_cast<uint4 *>(out + p * H);
        for (int idx = threadIdx.x; idx < nvec; idx += kRowThreads) {
            const uint4 v = src[idx];
            dst[idx] = make_uint4(pack_bf16x2(bf16_lo(v.x) * f, bf16_hi(v.x) * f),
                                  pack_bf16x2(bf16_lo(v.y) * f, bf16_hi(v.y) * f),
                                  pack_bf16x2(bf16_lo(v.z) * f, bf16_hi(v.z) * f),
                                  pack_bf16x2(bf16_lo(v.w) * f, bf16_hi(v.w) * f));
        }
    }
}

}  // namespace epl
