// Batched multi-sequence KV-cache write for gfx950.
//
// One launch stores the new K and V rows of every token in the batch,
// whatever sequence it belongs to, into the block pools (PhotonInfer README,
// Korean translation, "Technical details > Paged attention": batched cache
// operations done by a single kernel for the K/V writes of many sequences).
//
// Work decomposition: one lane moves one 16-byte piece of one (token, kv
// head) row of K and the matching piece of V.  Consecutive lanes take
// consecutive pieces of a row and then consecutive heads, so a wavefront
// reads a contiguous run of the source rows and writes whole rows (head_dim
// * element bytes = 128 or 256 bytes) of the destination tiles.  The slot is
// read once per lane (it is the same for all lanes of a token and stays in
// the cache).  Pool layout [block][kv_head][offset][head_dim].

#include "pka_internal.h"

namespace pka {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_cache_write_kernel(
    const char *__restrict__ k, const char *__restrict__ v, int64_t k_token_bytes,
    int64_t v_token_bytes, const int64_t *__restrict__ slot_mapping, int32_t num_tokens,
    char *__restrict__ k_cache, char *__restrict__ v_cache, int64_t num_slots,
    int32_t block_size, int32_t num_kv_heads, int32_t row_bytes, int32_t pieces_per_row)
{
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t per_token = (int64_t)num_kv_heads * pieces_per_row;
    const int64_t token = gid / per_token;
    if (token >= num_tokens)
        return;
    const int32_t rem = (int32_t)(gid - token * per_token);
    const int32_t head = rem / pieces_per_row;
    const int32_t piece = rem - head * pieces_per_row;

    const int64_t slot = slot_mapping[token];
    if (slot < 0 || slot >= num_slots)  // padding, or outside the pool: skip
        return;
    const int64_t block = slot / block_size;
    const int32_t offset = (int32_t)(slot - block * block_size);

    const int64_t dst =
        ((block * num_kv_heads + head) * block_size + offset) * (int64_t)row_bytes + piece * 16;
    const int64_t src_k = token * k_token_bytes + (int64_t)head * row_bytes + piece * 16;
    const int64_t src_v = token * v_token_bytes + (int64_t)head * row_bytes + piece * 16;

    const uint4 kval = *reinterpret_cast<const uint4 *>(k + src_k);
    const uint4 vval = *reinterpret_cast<const uint4 *>(v + src_v);
    *reinterpret_cast<uint4 *>(k_cache + dst) = kval;
    *reinterpret_cast<uint4 *>(v_cache + dst) = vval;
}

}  // namespace

hipError_t launch_kv_cache_write(const WriteArgs &a, hipStream_t stream)
{
    if (a.num_tokens == 0)
        return hipSuccess;
    const int elt = dtype_bytes(a.dtype);
    const int32_t row_bytes = a.head_dim * elt;
    const int32_t pieces = row_bytes / 16;
    const int64_t lanes = (int64_t)a.num_tokens * a.num_kv_heads * pieces;
    const int64_t blocks = (lanes + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(kv_cache_write_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const char *>(a.k), static_cast<const char *>(a.v),
                       a.k_token_stride * elt, a.v_token_stride * elt, a.slot_mapping,
                       a.num_tokens, static_cast<char *>(a.k_cache),
                       static_cast<char *>(a.v_cache),
                       (int64_t)a.num_blocks * a.block_size, a.block_size, a.num_kv_heads,
                       row_bytes, pieces);
    return hipGetLastError();
}

}  // namespace pka
