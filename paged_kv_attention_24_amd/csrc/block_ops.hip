// Whole-block movement in the paged KV pools, for preemption and paging
// between GPU and CPU memory (PhotonInfer README, Korean translation,
// "Continuous batching scheduler": requests can be PREEMPTED; JackerLab
// "vllm" tag page, PagedAttention: KV pages move between GPU and CPU memory).
//
// A block is the contiguous run of block_bytes bytes that one physical
// block holds in a pool laid out [num_blocks][num_kv_heads][block_size]
// [head_dim].  Three bit copies share one kernel:
//   copy     block dst of both pools <- block src (pairs [n][2]);
//   gather   packed[i] = (K block ids[i], V block ids[i]), [n][2][block_bytes];
//   scatter  K, V block ids[i] <- packed[i].
// An id outside [0, num_blocks) skips its entry.  A copy launch reads its
// sources and writes its destinations concurrently, so no block may be both
// (the caller's contract).  Host transfers are left to the runtime: a swap
// is a gather into a device buffer and one copy to host memory (or the
// reverse), so the kernel only ever touches device memory.
//
// Grid: (entry, tensor K/V, 16 KiB piece of the block); 256 threads move
// 16 bytes each, four times, with coalesced loads and stores.  The bound is
// HBM: block_bytes read and written per entry and tensor.

#include <hip/hip_runtime.h>

#include "pka_internal.h"

namespace pka {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kPiece = (int64_t)kThreads * 16 * kUnroll;  // bytes per workgroup

__global__ __launch_bounds__(kThreads) void move_blocks_kernel(BlockMoveArgs a)
{
    const int64_t i = blockIdx.x;
    const int tensor = blockIdx.y;  // 0 K, 1 V
    char *pool = static_cast<char *>(tensor == 0 ? a.k_cache : a.v_cache);
    const char *src;
    char *dst;
    if (a.mode == BlockMove::Copy) {
        const int64_t s = a.ids[2 * i], d = a.ids[2 * i + 1];
        if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks)
            return;
        src = pool + s * a.block_bytes;
        dst = pool + d * a.block_bytes;
    } else {
        const int64_t b = a.ids[i];
        if (b < 0 || b >= a.num_blocks)
            return;
        char *packed = static_cast<char *>(a.packed) + (2 * i + tensor) * a.block_bytes;
        if (a.mode == BlockMove::Gather) {
            src = pool + b * a.block_bytes;
            dst = packed;
        } else {
            src = packed;
            dst = pool + b * a.block_bytes;
        }
    }
    const int64_t base = (int64_t)blockIdx.z * kPiece + threadIdx.x * 16;
    uint4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const int64_t o = base + (int64_t)k * kThreads * 16;
        if (o < a.block_bytes)
            v[k] = *reinterpret_cast<const uint4 *>(src + o);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        const int64_t o = base + (int64_t)k * kThreads * 16;
        if (o < a.block_bytes)
            *reinterpret_cast<uint4 *>(dst + o) = v[k];
    }
}

}  // namespace

hipError_t launch_move_blocks(const BlockMoveArgs &a, hipStream_t stream)
{
    if (a.num_entries == 0)
        return hipSuccess;
    const dim3 grid((unsigned)a.num_entries, 2u, (unsigned)((a.block_bytes + kPiece - 1) / kPiece));
    hipLaunchKernelGGL(move_blocks_kernel, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pka
