// Streaming-bandwidth probes (libepl_probe.so): plain kernels that move
// fixed read:write mixes of 16-byte words, used by bench.py --ceilings to put
// the library's kernels next to the rate the same traffic mix reaches when
// it is perfectly sequential. Not part of the dispatch / combine path.
//
//   mix: out[i] = xor of in[r * ld + i] over r < ratio   (ratio reads : 1 write)
//   fan: out[f * ld + i] = in[i] for f < fan             (1 read : fan writes)
//
// for i < n; ld >= n is the distance between streams, so that the streams
// need not start at addresses that are multiples of a large power of two
// (which would put their words in the same DRAM banks at the same time).
// Loads are non-temporal (each word is read once); stores are write-back or
// non-temporal per the caller's flag. Workgroups of 256 threads stride over i.
//
//   pieces: out is cut into pieces of `piece` words, one workgroup per piece
//           (no striding), its threads storing the piece's words in order;
//           the pieces go in address order or, with `xcd`, each XCD (workgroup
//           i runs on XCD i mod 8) takes one contiguous eighth of them. This
//           measures how the bytes one workgroup writes, and which XCD writes
//           them, set the HBM write rate.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 2;

template <bool NT>
__device__ __forceinline__ void put(u32x4 *p, const u32x4 &v)
{
    if (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <int RATIO, bool NT>
__global__ __launch_bounds__(kThreads) void mix_kernel(const u32x4 *__restrict__ in,
                                                       u32x4 *__restrict__ out, int64_t n,
                                                       int64_t ld)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t i0 = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i0 < n;
         i0 += stride) {
        u32x4 v[kUnroll][RATIO];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int r = 0; r < RATIO; ++r) {
                const int64_t i = i0 + u * kThreads;
                if (i < n)
                    v[u][r] = __builtin_nontemporal_load(in + r * ld + i);
            }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + u * kThreads;
            if (i >= n)
                continue;
            u32x4 a = v[u][0];
#pragma unroll
            for (int r = 1; r < RATIO; ++r)
                a ^= v[u][r];
            put<NT>(out + i, a);
        }
    }
}

template <int FAN, bool NT>
__global__ __launch_bounds__(kThreads) void fan_kernel(const u32x4 *__restrict__ in,
                                                       u32x4 *__restrict__ out, int64_t n,
                                                       int64_t ld)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kThreads) {
        const u32x4 v = __builtin_nontemporal_load(in + i);
#pragma unroll
        for (int f = 0; f < FAN; ++f)
            put<NT>(out + f * ld + i, v);
    }
}

template <bool NT, bool XCD>
__global__ __launch_bounds__(1024) void pieces_kernel(u32x4 *__restrict__ out, int64_t n,
                                                      int64_t piece, int64_t npieces)
{
    int64_t r = blockIdx.x;
    if (XCD) {
        const int64_t per = (npieces + 7) / 8;
        r = (r % 8) * per + r / 8;
    }
    if (r >= npieces)
        return;
    const int64_t b0 = r * piece, b1 = min(n, b0 + piece);
    for (int64_t i = b0 + threadIdx.x; i < b1; i += blockDim.x)
        put<NT>(out + i, u32x4{(uint32_t)i, (uint32_t)r, 1u, 2u});
}

template <int R>
int launch_mix(const void *in, void *out, int64_t n, int64_t ld, int nt, unsigned grid,
               hipStream_t s)
{
    if (nt)
        hipLaunchKernelGGL((mix_kernel<R, true>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), n, ld);
    else
        hipLaunchKernelGGL((mix_kernel<R, false>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), n, ld);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <int F>
int launch_fan(const void *in, void *out, int64_t n, int64_t ld, int nt, unsigned grid,
               hipStream_t s)
{
    if (nt)
        hipLaunchKernelGGL((fan_kernel<F, true>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), n, ld);
    else
        hipLaunchKernelGGL((fan_kernel<F, false>), dim3(grid), dim3(kThreads), 0, s,
                           static_cast<const u32x4 *>(in), static_cast<u32x4 *>(out), n, ld);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

bool args_ok(const void *in, const void *out, int64_t n, int64_t ld, unsigned grid)
{
    return in && out && n > 0 && ld >= n && grid > 0 && grid <= (1u << 22) &&
           reinterpret_cast<uintptr_t>(in) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
}

}  // namespace

extern "C" {

// `in` holds ratio * ld 16-byte words, `out` n words. ratio in {1, 2, 4, 8}.
// Returns 0, -1 for bad arguments, -4 if the launch failed.
int epl_probe_mix(const void *in, void *out, int64_t n, int64_t ld, int ratio, int nt_stores,
                  unsigned grid, void *stream)
{
    if (!args_ok(in, out, n, ld, grid))
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (ratio) {
    case 1: return launch_mix<1>(in, out, n, ld, nt_stores, grid, s);
    case 2: return launch_mix<2>(in, out, n, ld, nt_stores, grid, s);
    case 4: return launch_mix<4>(in, out, n, ld, nt_stores, grid, s);
    case 8: return launch_mix<8>(in, out, n, ld, nt_stores, grid, s);
    default: return -1;
    }
}

// `in` holds n 16-byte words, `out` fan * ld words. fan in {1, 4, 8}.
int epl_probe_fan(const void *in, void *out, int64_t n, int64_t ld, int fan, int nt_stores,
                  unsigned grid, void *stream)
{
    if (!args_ok(in, out, n, ld, grid))
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (fan) {
    case 1: return launch_fan<1>(in, out, n, ld, nt_stores, grid, s);
    case 4: return launch_fan<4>(in, out, n, ld, nt_stores, grid, s);
    case 8: return launch_fan<8>(in, out, n, ld, nt_stores, grid, s);
    default: return -1;
    }
}

// `out` holds n 16-byte words, cut into pieces of `piece` words, one
// workgroup of `threads` threads (64 .. 1024, a multiple of 64) per piece.
// Returns 0, -1 for bad arguments, -4 if the launch failed.
int epl_probe_pieces(void *out, int64_t n, int64_t piece, int threads, int nt_stores, int xcd,
                     void *stream)
{
    if (!out || n <= 0 || piece <= 0 || threads < 64 || threads > 1024 || threads % 64 != 0 ||
        reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return -1;
    const int64_t npieces = (n + piece - 1) / piece;
    const int64_t grid = xcd ? (npieces + 7) / 8 * 8 : npieces;
    if (grid > (int64_t(1) << 22))
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    u32x4 *o = static_cast<u32x4 *>(out);
    const dim3 g((unsigned)grid), b((unsigned)threads);
    if (nt_stores && xcd)
        hipLaunchKernelGGL((pieces_kernel<true, true>), g, b, 0, s, o, n, piece, npieces);
    else if (nt_stores)
        hipLaunchKernelGGL((pieces_kernel<true, false>), g, b, 0, s, o, n, piece, npieces);
    else if (xcd)
        hipLaunchKernelGGL((pieces_kernel<false, true>), g, b, 0, s, o, n, piece, npieces);
    else
        hipLaunchKernelGGL((pieces_kernel<false, false>), g, b, 0, s, o, n, piece, npieces);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// The runtime's own fill of n 32-bit words (for comparison with the pieces).
int epl_probe_fill32(void *out, int64_t n, uint32_t value, void *stream)
{
    if (!out || n <= 0 || reinterpret_cast<uintptr_t>(out) % 4 != 0)
        return -1;
    return hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(out), (int)value, (size_t)n,
                             static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : -4;
}

}  // extern "C"
