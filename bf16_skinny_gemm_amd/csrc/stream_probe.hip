// libskinny_stream_probe.so: one pass over a device buffer with 16-byte buffer
// loads and nothing else, to measure the read rate HBM gives a plain streaming
// kernel on this device (include/skinny_stream_probe.h). Measurement only.
#include "skinny_stream_probe.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                                   // 16-byte loads per thread per chunk
constexpr unsigned kChunk = kThreads * 16u * kUnroll;        // 32 KiB

// The buffer is cut into 32 KiB chunks dealt to the blocks round-robin (chunk c
// to block c mod grid), the order in which the GEMV's persistent blocks take
// their tiles, so the blocks sweep the buffer side by side. Each chunk is read
// through a buffer resource over exactly its bytes (the last chunk's loads past
// the end read zeros, the XOR identity), and the next chunk's loads are issued
// before the current chunk is consumed, as the GEMV's tile prefetch does.
template <bool NT>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint8_t *buf, unsigned long long bytes,
                                                              uint32_t *sink)
{
    const unsigned long long nchunks = (bytes + kChunk - 1) / kChunk;
    const unsigned off = threadIdx.x * 16u;
    auto issue = [&](unsigned long long c, skg::u32x4 (&v)[kUnroll]) {
        const unsigned long long start = c * kChunk;
        unsigned len = 0;
        if (c < nchunks) {
            const unsigned long long rest = bytes - start;
            len = (unsigned)(rest < kChunk ? rest : kChunk);
        }
        const __amdgpu_buffer_rsrc_t r = skg::make_rsrc(buf + (c < nchunks ? start : 0), len);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = skg::load16<NT>(r, off + u * kThreads * 16u);
    };
    skg::u32x4 acc = {0u, 0u, 0u, 0u};
    skg::u32x4 a[kUnroll], b[kUnroll];
    auto consume = [&](const skg::u32x4 (&v)[kUnroll]) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc ^= v[u];
    };
    unsigned long long c = blockIdx.x;
    const unsigned long long step = gridDim.x;
    if (c < nchunks)
        issue(c, a);
    while (c < nchunks) {
        issue(c + step, b);  // an empty resource past the last chunk: no data moves
        consume(a);
        c += step;
        if (c >= nchunks)
            break;
        issue(c + step, a);
        consume(b);
        c += step;
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// v ^ (v of the lane the DPP control names); rows outside ROW_MASK take 0 and keep v.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ unsigned dpp_xor(unsigned v)
{
    return v ^ (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// One block per tile: block b reads bytes [b*T, (b+1)*T) of the buffer, T = waves
// * LOADS KiB. Wave w of the block takes LOADS consecutive KiB, each one 16-byte
// load per lane (1 KiB per instruction), all issued before any is consumed: the
// load schedule of the GEMV's one-block-per-tile plans at M = 1 (a wave's row
// slice of LOADS chunks), without the arithmetic. The tile's buffer resource ends
// at the buffer's end, so a ragged last tile reads zeros past it. Each wave XORs
// what it read into one word, stored by lane 0 to sink[b * waves + w].
template <int LOADS, bool NT>
__global__ __launch_bounds__(1024) void read_tiles_kernel(const uint8_t *buf, unsigned long long bytes,
                                                          uint32_t *sink)
{
    const unsigned waves = blockDim.x >> 6;
    const unsigned wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const unsigned long long tile = (unsigned long long)waves * LOADS * 1024u;
    const unsigned long long start = (unsigned long long)blockIdx.x * tile;
    const unsigned long long rest = bytes - start;
    const unsigned len = (unsigned)(rest < tile ? rest : tile);
    const __amdgpu_buffer_rsrc_t r = skg::make_rsrc(buf + start, len);
    skg::u32x4 v[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
        v[u] = skg::load16<NT>(r, ((wave * LOADS + u) * 64u + lane) * 16u);
    skg::u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
        acc ^= v[u];
    // XOR across the wave with DPP moves (the butterfly the GEMV's row sums take),
    // so a wave retires as soon after its last load as the GEMV's do; lane 63
    // ends with the wave's XOR
    unsigned w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    w = dpp_xor<0xB1>(w);       // quad_perm [1,0,3,2]
    w = dpp_xor<0x4E>(w);       // quad_perm [2,3,0,1]
    w = dpp_xor<0x141>(w);      // row_half_mirror
    w = dpp_xor<0x140>(w);      // row_mirror
    w = dpp_xor<0x142, 0xA>(w); // row_bcast:15 into rows 1 and 3
    w = dpp_xor<0x143, 0xC>(w); // row_bcast:31 into rows 2 and 3
    if (lane == 63)
        sink[(size_t)blockIdx.x * waves + wave] = w;
}

// Does nothing: the cost of one launch of `grid` blocks, for the per-launch floor.
__global__ void empty_kernel() {}

template <int LOADS>
const void *tiles_fn(bool nt)
{
    return nt ? reinterpret_cast<const void *>(&read_tiles_kernel<LOADS, true>)
              : reinterpret_cast<const void *>(&read_tiles_kernel<LOADS, false>);
}

bool tiles_shape_ok(int loads, int threads)
{
    return (loads == 2 || loads == 4 || loads == 8 || loads == 16) && threads >= 64 && threads <= 1024 &&
           threads % 64 == 0;
}

}  // namespace

extern "C" size_t skinny_probe_tiles_sink_words(size_t bytes, int loads, int threads)
{
    if (!tiles_shape_ok(loads, threads))
        return 0;
    const size_t tile = (size_t)(threads / 64) * loads * 1024;
    return (bytes + tile - 1) / tile * (size_t)(threads / 64);
}

extern "C" int skinny_probe_read_tiles(const void *buf, size_t bytes, int nontemporal, int loads, int threads,
                                       uint32_t *sink, hipStream_t stream)
{
    if (!tiles_shape_ok(loads, threads) || !sink || bytes % 16 != 0 || bytes == 0 || !buf ||
        ((uintptr_t)buf % 16) != 0 || ((uintptr_t)sink % 4) != 0)
        return -1;
    const size_t tile = (size_t)(threads / 64) * loads * 1024;
    const size_t blocks = (bytes + tile - 1) / tile;
    if (blocks > 0x7FFFFFFFu)
        return -1;
    const uintptr_t s0 = (uintptr_t)sink, s1 = s0 + skinny_probe_tiles_sink_words(bytes, loads, threads) * 4;
    const uintptr_t b0 = (uintptr_t)buf, b1 = b0 + bytes;
    if (s0 < b1 && b0 < s1)
        return -1;
    const uint8_t *p = (const uint8_t *)buf;
    unsigned long long nbytes = bytes;
    void *args[] = {&p, &nbytes, &sink};
    const bool nt = nontemporal != 0;
    const void *fn = loads == 2 ? tiles_fn<2>(nt) : loads == 4 ? tiles_fn<4>(nt) : loads == 8 ? tiles_fn<8>(nt)
                                                                                             : tiles_fn<16>(nt);
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3((unsigned)threads), args, 0, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return -4;
    }
    return 0;
}

extern "C" int skinny_probe_empty(int grid_blocks, int threads, hipStream_t stream)
{
    if (grid_blocks < 1 || grid_blocks > (1 << 24) || threads < 64 || threads > 1024 || threads % 64 != 0)
        return -1;
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&empty_kernel), dim3((unsigned)grid_blocks),
                                         dim3((unsigned)threads), nullptr, 0, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return -4;
    }
    return 0;
}

extern "C" size_t skinny_probe_sink_words(int grid_blocks)
{
    return grid_blocks > 0 ? (size_t)grid_blocks * kThreads : 0;
}

extern "C" int skinny_probe_read(const void *buf, size_t bytes, int nontemporal, int grid_blocks,
                                 uint32_t *sink, hipStream_t stream)
{
    if (!sink || grid_blocks < 1 || grid_blocks > 65536 || bytes % 16 != 0 ||
        (bytes != 0 && !buf) || ((uintptr_t)buf % 16) != 0 || ((uintptr_t)sink % 4) != 0)
        return -1;
    const uintptr_t s0 = (uintptr_t)sink, s1 = s0 + skinny_probe_sink_words(grid_blocks) * 4;
    const uintptr_t b0 = (uintptr_t)buf, b1 = b0 + bytes;
    if (bytes != 0 && s0 < b1 && b0 < s1)
        return -1;
    const uint8_t *p = (const uint8_t *)buf;
    unsigned long long nbytes = bytes;
    void *args[] = {&p, &nbytes, &sink};
    const void *fn = nontemporal ? reinterpret_cast<const void *>(&read_probe_kernel<true>)
                                 : reinterpret_cast<const void *>(&read_probe_kernel<false>);
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid_blocks), dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return -4;
    }
    return 0;
}
