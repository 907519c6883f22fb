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

#include "cdna4.h"
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

// The same write with the rotary position embedding applied to the new keys
// (same README, "Key features > GPU-optimised kernels": batched RoPE among
// the fused operations).  Token i at position p = positions[i] (skipped if
// outside the table) has each K row x stored as y, for j < R/2:
//   y[j] = x[j] c_j - x[j + R/2] s_j,   y[j + R/2] = x[j + R/2] c_j + x[j] s_j,
// c_j = cos_sin[p][j], s_j = cos_sin[p][R/2 + j], in fp32 with every product
// and sum rounded (no fused multiply-add), then rounded to nearest even into
// the pool dtype; dims >= R and the V row are copied.  Same lanes as above:
// a lane whose piece starts below R/2 also produces the piece R/2 further
// on, lanes of the second rotated half have nothing to do.
template <int ELT>
__device__ __forceinline__ void unpack(const uint4 &u, float (&x)[16 / ELT])
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if constexpr (ELT == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = __builtin_bit_cast(float, w[i]);
    }
}
__device__ __forceinline__ void unpack_half(const uint4 &u, float (&x)[8], bool bf16)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t lo = (uint16_t)(w[i] & 0xffffu), hi = (uint16_t)(w[i] >> 16);
        if (bf16) {
            x[2 * i] = __builtin_bit_cast(float, (uint32_t)lo << 16);
            x[2 * i + 1] = __builtin_bit_cast(float, (uint32_t)hi << 16);
        } else {
            x[2 * i] = (float)__builtin_bit_cast(_Float16, lo);
            x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, hi);
        }
    }
}
__device__ __forceinline__ uint4 pack_half(const float (&y)[8], bool bf16)
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t lo = bf16 ? f32_to_bf16_rne(y[2 * i])
                                 : __builtin_bit_cast(uint16_t, (_Float16)y[2 * i]);
        const uint16_t hi = bf16 ? f32_to_bf16_rne(y[2 * i + 1])
                                 : __builtin_bit_cast(uint16_t, (_Float16)y[2 * i + 1]);
        w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int N>
__device__ __forceinline__ void rotate(const float (&x1)[N], const float (&x2)[N],
                                       const float *c, const float *s, float (&y1)[N],
                                       float (&y2)[N])
{
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float a = x1[e] * c[e], b = x2[e] * s[e];
        const float g = x2[e] * c[e], f = x1[e] * s[e];
        y1[e] = a - b;
        y2[e] = g + f;
    }
}

template <int ELT>
__global__ __launch_bounds__(kThreads) void kv_cache_write_rope_kernel(
    const char *__restrict__ k, const char *__restrict__ v, int64_t k_token_bytes,
    int64_t v_token_bytes, const int64_t *__restrict__ slot_mapping,
    const int32_t *__restrict__ positions, const float *__restrict__ cos_sin,
    int32_t max_position, int32_t rotary_dim, int32_t num_tokens, char *__restrict__ k_cache,
    char *__restrict__ v_cache, int64_t num_slots, int32_t block_size, int32_t num_kv_heads,
    int32_t row_bytes, int32_t pieces_per_row, bool bf16)
{
    constexpr int VEC = 16 / ELT;  // elements per 16-byte piece
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t per_token = (int64_t)num_kv_heads * pieces_per_row;
    const int64_t token = gid / per_token;
    if (token >= num_tokens)
        return;
    const int32_t rem = (int32_t)(gid - token * per_token);
    const int32_t head = rem / pieces_per_row;
    const int32_t piece = rem - head * pieces_per_row;

    const int64_t slot = slot_mapping[token];
    const int32_t pos = positions[token];
    if (slot < 0 || slot >= num_slots || pos < 0 || pos >= max_position)
        return;
    const int64_t block = slot / block_size;
    const int32_t offset = (int32_t)(slot - block * block_size);
    const int64_t dst_row = ((block * num_kv_heads + head) * block_size + offset) * (int64_t)row_bytes;
    const int64_t src_k = token * k_token_bytes + (int64_t)head * row_bytes;
    const int64_t src_v = token * v_token_bytes + (int64_t)head * row_bytes;

    *reinterpret_cast<uint4 *>(v_cache + dst_row + piece * 16) =
        *reinterpret_cast<const uint4 *>(v + src_v + piece * 16);

    const int d0 = piece * VEC, half = rotary_dim / 2;
    if (d0 >= rotary_dim) {  // past the rotated dims: a copy
        *reinterpret_cast<uint4 *>(k_cache + dst_row + piece * 16) =
            *reinterpret_cast<const uint4 *>(k + src_k + piece * 16);
        return;
    }
    if (d0 >= half)  // produced by the lane of dims d0 - R/2
        return;
    const int partner = piece + half / VEC;
    const uint4 u1 = *reinterpret_cast<const uint4 *>(k + src_k + piece * 16);
    const uint4 u2 = *reinterpret_cast<const uint4 *>(k + src_k + partner * 16);
    const float *cs = cos_sin + (int64_t)pos * rotary_dim;
    float c[VEC], sn[VEC], x1[VEC], x2[VEC], y1[VEC], y2[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        c[e] = cs[d0 + e];
        sn[e] = cs[half + d0 + e];
    }
    uint4 o1, o2;
    if constexpr (ELT == 4) {
        unpack<4>(u1, x1);
        unpack<4>(u2, x2);
        rotate<VEC>(x1, x2, c, sn, y1, y2);
        o1 = make_uint4(__builtin_bit_cast(uint32_t, y1[0]), __builtin_bit_cast(uint32_t, y1[1]),
                        __builtin_bit_cast(uint32_t, y1[2]), __builtin_bit_cast(uint32_t, y1[3]));
        o2 = make_uint4(__builtin_bit_cast(uint32_t, y2[0]), __builtin_bit_cast(uint32_t, y2[1]),
                        __builtin_bit_cast(uint32_t, y2[2]), __builtin_bit_cast(uint32_t, y2[3]));
    } else {
        unpack_half(u1, x1, bf16);
        unpack_half(u2, x2, bf16);
        rotate<VEC>(x1, x2, c, sn, y1, y2);
        o1 = pack_half(y1, bf16);
        o2 = pack_half(y2, bf16);
    }
    *reinterpret_cast<uint4 *>(k_cache + dst_row + piece * 16) = o1;
    *reinterpret_cast<uint4 *>(k_cache + dst_row + partner * 16) = o2;
}

}  // namespace

hipError_t launch_kv_cache_write(const WriteArgs &a, hipStream_t stream)
{
    if (a.num_tokens == 0)
        return hipSuccess;
    if (a.positions) {
        const int elt = dtype_bytes(a.dtype);
        const int32_t row_bytes = a.head_dim * elt;
        const int32_t pieces = row_bytes / 16;
        const int64_t lanes = (int64_t)a.num_tokens * a.num_kv_heads * pieces;
        const int64_t blocks = (lanes + kThreads - 1) / kThreads;
        auto kernel = elt == 4 ? kv_cache_write_rope_kernel<4> : kv_cache_write_rope_kernel<2>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           static_cast<const char *>(a.k), static_cast<const char *>(a.v),
                           a.k_token_stride * elt, a.v_token_stride * elt, a.slot_mapping,
                           a.positions, a.cos_sin, a.max_position, a.rotary_dim, a.num_tokens,
                           static_cast<char *>(a.k_cache), static_cast<char *>(a.v_cache),
                           (int64_t)a.num_blocks * a.block_size, a.block_size, a.num_kv_heads,
                           row_bytes, pieces, a.dtype == DType::BF16);
        return hipGetLastError();
    }
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
