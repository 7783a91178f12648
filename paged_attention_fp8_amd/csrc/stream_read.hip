// stream_read.hip -- a bare streaming read of device memory, for measurement.
// It reads every byte once with the loads the attention kernels use for KV
// (16 bytes per lane, non-temporal), keeping a wave's next 16 KiB tile in
// flight while it consumes the current one, and does nothing else.  Its time
// is what the memory system delivers for that many bytes under the same
// timing, so an HBM-bound kernel's time can be set beside it as well as
// beside the published peak.
#include "pafp8_device.hpp"
#include "pafp8_internal.hpp"

namespace pafp8 {
namespace {

constexpr int kReadWaves = 4;
constexpr int kReadLoads = 16;   // 16-byte loads per lane per tile: 16 KiB per wave
static_assert(kReadLoads * 64 * 16 == kStreamReadTile, "tile size");
static_assert(kReadWaves * 64 == kStreamReadThreads, "work-group size");

// Work-group g takes tiles [g * per_group, (g + 1) * per_group) of the
// buffer; its waves take every kReadWaves-th of them.  Each thread stores the
// XOR of the 32-bit words it read, so the XOR over sink equals the XOR over
// the buffer.
__global__ __launch_bounds__(kReadWaves * 64) void stream_read_kernel(const uint8_t *src,
                                                                       int64_t tiles,
                                                                       int64_t per_group,
                                                                       uint32_t *sink)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * per_group;
    const int64_t end = first + per_group < tiles ? first + per_group : tiles;
    uint32_t acc = 0;
    u32x4 cur[kReadLoads], nxt[kReadLoads];
    auto load = [&](u32x4 *r, int64_t t) {
        const uint8_t *base = src + t * (kReadLoads * 1024) + lane * 16;
#pragma unroll
        for (int k = 0; k < kReadLoads; ++k)
            r[k] = load16_stream(base + k * 1024);
    };
    auto fold = [&](const u32x4 *r) {
#pragma unroll
        for (int k = 0; k < kReadLoads; ++k)
            acc ^= r[k][0] ^ r[k][1] ^ r[k][2] ^ r[k][3];
    };
    int64_t t = first + wave;
    if (t < end)
        load(cur, t);
    for (; t < end; t += 2 * kReadWaves) {
        if (t + kReadWaves < end)
            load(nxt, t + kReadWaves);
        fold(cur);
        if (t + 2 * kReadWaves < end)
            load(cur, t + 2 * kReadWaves);
        if (t + kReadWaves < end)
            fold(nxt);
    }
    sink[static_cast<int64_t>(blockIdx.x) * (kReadWaves * 64) + threadIdx.x] = acc;
}

// The same read, and for every 16 KiB tile read a 16/R KiB tile written to
// dst with plain 16-byte stores: lane l's k-th store is the XOR of its loads
// kR .. kR + R - 1, at dst tile offset k * 1024 + l * 16.
template <int R>
__global__ __launch_bounds__(kReadWaves * 64) void stream_read_write_kernel(const uint8_t *src,
                                                                             uint8_t *dst, int64_t tiles,
                                                                             int64_t per_group)
{
    constexpr int KW = kReadLoads / R;   // stores per lane per tile
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * per_group;
    const int64_t end = first + per_group < tiles ? first + per_group : tiles;
    u32x4 cur[kReadLoads], nxt[kReadLoads];
    auto load = [&](u32x4 *r, int64_t t) {
        const uint8_t *base = src + t * kStreamReadTile + lane * 16;
#pragma unroll
        for (int k = 0; k < kReadLoads; ++k)
            r[k] = load16_stream(base + k * 1024);
    };
    auto put = [&](const u32x4 *r, int64_t t) {
        uint8_t *base = dst + t * (kStreamReadTile / R) + lane * 16;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            u32x4 v = r[k * R];
#pragma unroll
            for (int q = 1; q < R; ++q)
                v ^= r[k * R + q];
            store16(base + k * 1024, v);
        }
    };
    int64_t t = first + wave;
    if (t < end)
        load(cur, t);
    for (; t < end; t += 2 * kReadWaves) {
        if (t + kReadWaves < end)
            load(nxt, t + kReadWaves);
        put(cur, t);
        if (t + 2 * kReadWaves < end)
            load(cur, t + 2 * kReadWaves);
        if (t + kReadWaves < end)
            put(nxt, t + kReadWaves);
    }
}

}  // namespace

hipError_t launch_stream_read_write(const void *src, int64_t src_bytes, void *dst, int ratio,
                                    int work_groups, hipStream_t stream)
{
    const int64_t tiles = src_bytes / kStreamReadTile;
    const int64_t per = (tiles + work_groups - 1) / work_groups;
    const dim3 grid(work_groups), block(kReadWaves * 64);
    const uint8_t *s = static_cast<const uint8_t *>(src);
    uint8_t *d = static_cast<uint8_t *>(dst);
    if (ratio == 1)
        hipLaunchKernelGGL(stream_read_write_kernel<1>, grid, block, 0, stream, s, d, tiles, per);
    else if (ratio == 2)
        hipLaunchKernelGGL(stream_read_write_kernel<2>, grid, block, 0, stream, s, d, tiles, per);
    else
        hipLaunchKernelGGL(stream_read_write_kernel<4>, grid, block, 0, stream, s, d, tiles, per);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *src, int64_t bytes, int work_groups, uint32_t *sink,
                              hipStream_t stream)
{
    const int64_t tiles = bytes / kStreamReadTile;
    const int64_t per = (tiles + work_groups - 1) / work_groups;
    hipLaunchKernelGGL(stream_read_kernel, dim3(work_groups), dim3(kReadWaves * 64), 0, stream,
                       static_cast<const uint8_t *>(src), tiles, per, sink);
    return hipGetLastError();
}

}  // namespace pafp8
