// HBM read ceilings of the device, measured with two plain kernels, so that
// the decode's bandwidth can be stated as a fraction of what a read-only
// kernel reaches on the same box (besides the vendor peak).  Built into
// libpka_calib.so, apart from the library: nothing in the attention path
// calls it.
//
//   stream: every byte of a buffer once, in contiguous 4 KiB pieces, two
//           pieces (eight 16-byte loads per lane) in flight per wave;
//   gather: whole tiles of tile_bytes at the positions an index array lists
//           (random order), one wave per tile at a time -- the access pattern
//           of a block-table walk over a shuffled pool.
//
// Both fold what they read into one word per lane and store it only when it
// equals a value the host never plants, so no load is dead and nearly
// nothing is written.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr uint32_t kNever = 0x9e3779b9u;

// Wave w reads the 4 KiB pieces w, w + waves, ... of the buffer, two pieces
// (eight 1 KiB wave loads) in flight per iteration.
__global__ __launch_bounds__(256) void stream_read(const uint4 *__restrict__ p, int64_t n16,
                                                   uint32_t *sink)
{
    const int lane = threadIdx.x % 64;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
    const int64_t pieces = n16 / 256;  // 4 KiB = 256 uint4
    uint32_t acc = 0;
    int64_t c = wave;
    for (; c + waves < pieces; c += 2 * waves) {
        const uint4 *a = p + c * 256, *b = p + (c + waves) * 256;
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[u] = a[u * 64 + lane];
            v[4 + u] = b[u * 64 + lane];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc ^= v[u].x ^ v[u].w;
    }
    if (c < pieces) {
        const uint4 *a = p + c * 256;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc ^= a[u * 64 + lane].y;
    }
    // the last partial piece, if any
    for (int64_t i = pieces * 256 + (int64_t)wave * 64 + lane; i < n16; i += waves * 64)
        acc ^= p[i].z;
    if (acc == kNever)
        sink[threadIdx.x] = acc;
}

// tile_bytes a multiple of 1024; tiles[t] in [0, num_tiles_in_pool)
__global__ __launch_bounds__(256) void gather_read(const uint4 *__restrict__ pool,
                                                   const int32_t *__restrict__ tiles,
                                                   int64_t num_tiles, int tile_bytes,
                                                   uint32_t *sink)
{
    const int lane = threadIdx.x % 64;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
    const int per_tile = tile_bytes / 1024;  // 1 KiB wave loads per tile
    uint32_t acc = 0;
    for (int64_t t = wave; t < num_tiles; t += waves) {
        const uint4 *base = pool + (int64_t)tiles[t] * (tile_bytes / 16);
        for (int k = 0; k < per_tile; k += 4) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = base[(k + (k + u < per_tile ? u : 0)) * 64 + lane];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc ^= v[u].x ^ v[u].w;
        }
    }
    if (acc == kNever)
        sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16) at src once; grid workgroups of 256 lanes.
int pka_calib_stream_read(const void *src, int64_t bytes, void *sink, int grid, void *stream)
{
    if (!src || !sink || bytes <= 0 || bytes % 16 || grid <= 0)
        return 1;
    hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), bytes / 16, static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Reads num_tiles tiles of tile_bytes (a multiple of 1024) of pool, tile
// tiles[t] at byte tiles[t] * tile_bytes; the caller keeps every index
// inside the pool.
int pka_calib_gather_read(const void *pool, const int32_t *tiles, int64_t num_tiles,
                          int tile_bytes, void *sink, int grid, void *stream)
{
    if (!pool || !tiles || !sink || num_tiles <= 0 || tile_bytes <= 0 || tile_bytes % 1024 ||
        grid <= 0)
        return 1;
    hipLaunchKernelGGL(gather_read, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(pool), tiles, num_tiles, tile_bytes,
                       static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
