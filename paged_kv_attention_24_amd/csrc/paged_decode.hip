// Batched paged-attention decode for gfx950 (CDNA4).
//
// What is computed (PhotonInfer README, Korean translation, "Key features >
// GPU-optimised kernels" and "Technical details > Paged attention"): for
// every sequence b and query head hq, one query row attends over the
// sequence's L_b cached tokens, found block by block through its block
// table, with a numerically stable softmax:
//     out[b,hq,:] = sum_t softmax_t(scale * q[b,hq,:] . K_t) V_t.
//
// Design (CDNA4-first; the README's float4 loads and CUB block reductions
// are prior art for another GPU, not the blueprint):
//
//  * Work item = (partition j, kv head h, sequence b): the tokens
//    [j*P, min((j+1)*P, L_b)) of one kv head.  All G = Hq/Hkv query heads of
//    the group are served by the same K/V reads, so every KV byte is read
//    from HBM exactly once.
//  * One workgroup of NW wave64s per work item.  The partition is cut into
//    chunks of CT tokens (4 coalesced 1 KiB loads per chunk per tensor);
//    chunks are dealt round-robin to the waves.
//  * Lane layout of a load: a (block, kv head) tile is a contiguous
//    [block_size][head_dim] run, so one wave load of 64 lanes x 16 bytes
//    covers TPL = 64 / LPR whole token rows, LPR = head_dim*elt/16 lanes per
//    row.  Lane l holds 16 bytes (VEC elements) of token l / LPR.
//  * Pass 1 streams K: partial dot products with v_dot2_f32_{f16,bf16} (or
//    fp32 FMA), a DPP butterfly over the LPR lanes of a row, the scale and
//    log2(e) folded in; logits go to LDS, a running max stays in registers.
//  * Pass 2 streams V: p = exp2(s - m_wave) and o += p * V with
//    v_fma_mix-style mixed-precision FMAs into fp32 accumulators.  Because
//    each wave knows its maximum before pass 2, nothing is ever rescaled in
//    the loop.
//  * Merge: per-lane partial sums (token groups x waves) are combined in LDS
//    with each wave's maximum (log-sum-exp), once per work item.
//  * Partitions: with more than one partition per sequence each work item
//    writes (max, sum, normalised row) to the workspace and counts itself
//    done; the last one of its (sequence, kv head) merges all of them into
//    the output (log-sum-exp) and resets the counter.  One launch per call.
//  * Every K/V load is issued one chunk ahead of its use (register double
//    buffering), so each wave keeps up to 8 KiB in flight.
//  * Tokens >= L (the tail of the last block) are excluded by selects, never
//    by multiplying with 0, so stale or NaN slot contents cannot leak.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "pka_internal.h"

namespace pka {
namespace {

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;
#ifndef PKA_LOADS_PER_CHUNK
#define PKA_LOADS_PER_CHUNK 4
#endif
#ifndef PKA_PREFETCH_DEPTH
#define PKA_PREFETCH_DEPTH 1
#endif
constexpr int kLoadsPerChunk = PKA_LOADS_PER_CHUNK;  // 1 KiB wave loads per chunk per tensor
constexpr int kPrefetchDepth = PKA_PREFETCH_DEPTH;   // chunks in flight ahead of the one processed

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

struct TF32 {
    static constexpr int kBytes = 4;
};
struct TF16 {
    static constexpr int kBytes = 2;
};
struct TBF16 {
    static constexpr int kBytes = 2;
};

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }

// c ? a : b per component (a ternary on the struct type would select
// addresses and keep register arrays in memory)
__device__ __forceinline__ uint4 select4(bool c, const uint4 &a, const uint4 &b)
{
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// acc + (16 bytes of q) . (16 bytes of k), fp32 accumulation.
__device__ __forceinline__ float dot16(TF32, const uint4 &q, const uint4 &k, float acc)
{
    acc = fmaf(as_f(q.x), as_f(k.x), acc);
    acc = fmaf(as_f(q.y), as_f(k.y), acc);
    acc = fmaf(as_f(q.z), as_f(k.z), acc);
    acc = fmaf(as_f(q.w), as_f(k.w), acc);
    return acc;
}
__device__ __forceinline__ float dot16(TF16, const uint4 &q, const uint4 &k, float acc)
{
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.x), __builtin_bit_cast(half2_t, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.y), __builtin_bit_cast(half2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.z), __builtin_bit_cast(half2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.w), __builtin_bit_cast(half2_t, k.w), acc, false);
    return acc;
}
__device__ __forceinline__ float dot16(TBF16, const uint4 &q, const uint4 &k, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.x), __builtin_bit_cast(bf162_t, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.y), __builtin_bit_cast(bf162_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.z), __builtin_bit_cast(bf162_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.w), __builtin_bit_cast(bf162_t, k.w), acc, false);
    return acc;
}

// o[0..VEC) += p * (16 bytes of v), fp32 accumulation.
__device__ __forceinline__ void axpy16(TF32, float p, const uint4 &v, float *o)
{
    o[0] = fmaf(p, as_f(v.x), o[0]);
    o[1] = fmaf(p, as_f(v.y), o[1]);
    o[2] = fmaf(p, as_f(v.z), o[2]);
    o[3] = fmaf(p, as_f(v.w), o[3]);
}
__device__ __forceinline__ void axpy_h2(float p, uint32_t w, float *o)
{
    half2_t h = __builtin_bit_cast(half2_t, w);
    o[0] = fmaf(p, (float)h.x, o[0]);
    o[1] = fmaf(p, (float)h.y, o[1]);
}
__device__ __forceinline__ void axpy16(TF16, float p, const uint4 &v, float *o)
{
    axpy_h2(p, v.x, o + 0);
    axpy_h2(p, v.y, o + 2);
    axpy_h2(p, v.z, o + 4);
    axpy_h2(p, v.w, o + 6);
}
__device__ __forceinline__ void axpy_b2(float p, uint32_t w, float *o)
{
    o[0] = fmaf(p, as_f(w << 16), o[0]);
    o[1] = fmaf(p, as_f(w & 0xffff0000u), o[1]);
}
__device__ __forceinline__ void axpy16(TBF16, float p, const uint4 &v, float *o)
{
    axpy_b2(p, v.x, o + 0);
    axpy_b2(p, v.y, o + 2);
    axpy_b2(p, v.z, o + 4);
    axpy_b2(p, v.w, o + 6);
}

// ---- matrix-core pieces (fp16 / bf16 KV) --------------------------------
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// S^T tile += K rows (16 tokens x 32 dims) * q^T (32 dims x 16 heads).
// Lane l supplies K[token l%16][dims 8(l/16)..+7] and q[head l%16][same dims];
// it receives S^T[token 4(l/16)+i][head l%16], i = 0..3.
__device__ __forceinline__ float4_t mma_qk(TF16, const uint4 &k, const uint4 &q, float4_t acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, k),
                                                  __builtin_bit_cast(half8_t, q), acc, 0, 0, 0);
}
__device__ __forceinline__ float4_t mma_qk(TBF16, const uint4 &k, const uint4 &q, float4_t acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                   __builtin_bit_cast(bf16x8_t, q), acc, 0, 0, 0);
}
// O^T tile += V^T (16 dims x 16 tokens) * P^T (16 tokens x 16 heads).
// Lane l supplies V[tokens 4(l/16)..+3][dim l%16] and P[same tokens][head l%16];
// it accumulates O^T[dim 4(l/16)+i][head l%16].
__device__ __forceinline__ float4_t mma_pv(TF16, const uint2 &v, const uint2 &pr, float4_t acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, v),
                                                 __builtin_bit_cast(half4_t, pr), acc, 0, 0, 0);
}
__device__ __forceinline__ float4_t mma_pv(TBF16, const uint2 &v, const uint2 &pr, float4_t acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, v),
                                                     __builtin_bit_cast(short4_t, pr), acc, 0, 0, 0);
}

// 16 bytes per lane straight from global memory into LDS at base + 16*lane.
__device__ __forceinline__ void load_to_lds(const char *g, char *lds_base)
{
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(lds_base), 16, 0, 0);
}

// Transposing LDS read: within each group of 16 lanes, the four 16-bit
// values read by lanes 4r..4r+3 become element r of the lanes, one column
// per lane (lane i receives value i%4 of lane 4r + i/4).
__device__ __forceinline__ uint2 lds_read_tr16(const char *p)
{
    typedef __attribute__((address_space(3))) short4_t lds_short4;
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(p)));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xF, 0xF, true));
}

__device__ __forceinline__ float swz_xor16(float x)
{
    // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

// Sum over aligned groups of N consecutive lanes (N = 1..32); every lane of
// the group receives the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror: other quad of 8
    if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror: other half of 16
    if constexpr (N >= 32) x += swz_xor16(x);  // other row of 32
    return x;
}

// group_sum over N lanes applied to CNT independent values, one butterfly
// stage at a time for all of them: consecutive DPP instructions never read
// a register written by the instruction just before (no hazard stalls).
template <int N, int CNT>
__device__ __forceinline__ void group_sum_all(float (&x)[CNT])
{
    if constexpr (N >= 2) {
#pragma unroll
        for (int c = 0; c < CNT; ++c) x[c] += dpp<0xB1>(x[c]);
    }
    if constexpr (N >= 4) {
#pragma unroll
        for (int c = 0; c < CNT; ++c) x[c] += dpp<0x4E>(x[c]);
    }
    if constexpr (N >= 8) {
#pragma unroll
        for (int c = 0; c < CNT; ++c) x[c] += dpp<0x141>(x[c]);
    }
    if constexpr (N >= 16) {
#pragma unroll
        for (int c = 0; c < CNT; ++c) x[c] += dpp<0x140>(x[c]);
    }
    if constexpr (N >= 32) {
#pragma unroll
        for (int c = 0; c < CNT; ++c) x[c] += swz_xor16(x[c]);
    }
}

// Sum over the lanes that share (lane % LPR), i.e. over a wave's token
// groups (lane ^ LPR, lane ^ 2*LPR, ... up to lane ^ 32).
__device__ __forceinline__ float xor32(float x)
{
    const int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2,
                                                                  __builtin_bit_cast(int, x)));
}
template <int LPR>
__device__ __forceinline__ float token_group_sum(float x)
{
    if constexpr (LPR <= 8) x += dpp<0x128>(x);  // row_ror:8 = lane ^ 8 within 16
    if constexpr (LPR <= 16) x += swz_xor16(x);
    x += xor32(x);
    return x;
}

// Max over the whole wave, returned as a wave-uniform value.
__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    x = fmaxf(x, swz_xor16(x));
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    return fmaxf(lo, hi);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void *out, int64_t idx, float x, int out_kind)
{
    if (out_kind == 0)
        static_cast<float *>(out)[idx] = x;
    else if (out_kind == 1)
        static_cast<_Float16 *>(out)[idx] = (_Float16)x;
    else
        static_cast<uint16_t *>(out)[idx] = f32_to_bf16_rne(x);
}

// Agent-scope relaxed accesses: plain loads/stores with the coherence bit,
// so partial rows written on one XCD are read correctly on another without
// flushing or invalidating any L2.
__device__ __forceinline__ void coherent_store(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left free): every vector memory
// access of this wave has completed (loads landed, stores acknowledged).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left free
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

struct PartitionParams {
    void *out;
    int out_kind;  // 0 f32, 1 f16, 2 bf16
    const char *q, *k_cache, *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
    int32_t num_q_heads, num_kv_heads, num_blocks;
    float scale_log2;  // scale * log2(e)
    int32_t partition_size, num_partitions, len_cap;
    float *ws_o, *ws_ml;  // per (b, hq, partition): normalised row; (max, sum)
    const int2 *items;    // work list {b, j} (null: dense grid over (j, h, b))
    int32_t *wl_header;   // [0] next dynamic item, [1] number of {b, j} items
    int32_t *counters;    // per (b, kv head): partitions done; zero between calls
    // appended token per sequence (k_new null: plain decode)
    const char *k_new, *v_new;
    int64_t k_new_stride, v_new_stride;  // bytes between sequences
    const int64_t *slots;
    char *k_store, *v_store;             // the pools, written at slots[b]
    int64_t num_slots;
};

template <class T, int D, int BS, int G, int W>
struct Shape {
    static constexpr int ELT = T::kBytes;
    static constexpr int VEC = 16 / ELT;           // elements per lane load
    static constexpr int LPR = D / VEC;            // lanes per token row
    static constexpr int TPL = kWave / LPR;        // tokens per wave load
    static constexpr int NL = kLoadsPerChunk;      // loads per chunk per tensor
    static constexpr int CT = NL * TPL;            // tokens per chunk
    static constexpr int TILE = BS * D * ELT;      // bytes of one (block, head) tile
    // half-precision KV runs QK^T and PV on the matrix cores, with K and V
    // staged through LDS; fp32 KV stays on the vector ALUs
    static constexpr bool MFMA = !std::is_same<T, TF32>::value;
    static constexpr int NW = W;                   // waves per workgroup
    static constexpr int STAGE = MFMA ? 2 * 2 * NL * 1024 : 0;  // LDS bytes per wave: 2 chunks of K and V
    static_assert(LPR >= 1 && LPR <= 32 && TPL * LPR == kWave, "row must fit a wave");
    static_assert(BS % TPL == 0, "a wave load must stay inside one block");
};

// LDS of a workgroup.  The dynamic area holds, on the vector-ALU path,
// [NW][G][D] wave rows, then [NW][G] sums and [NW][G] maxima; on the matrix
// path only the sums and maxima.  Two ints (work-list slot, merge flag)
// follow it.  The matrix path has a static staging buffer, two chunks of K
// and V per wave; once a wave has finished streaming, its rows for the merge
// reuse the start of its part.
struct Lds {
    float *smem;
    char *sb[1];
};
template <class T, int D, int BS, int G, int W>
__host__ __device__ constexpr size_t lds_bytes()
{
    using S = Shape<T, D, BS, G, W>;
    return S::MFMA ? (size_t)S::NW * G * 2 * 4 : (size_t)S::NW * G * (D + 2) * 4;
}
template <class T, int D, int BS, int G, int W>
__device__ __forceinline__ float *wave_rows(const Lds &lds, int ww)
{
    using S = Shape<T, D, BS, G, W>;
    return S::MFMA ? reinterpret_cast<float *>(lds.sb[0] + (size_t)ww * S::STAGE)
                   : lds.smem + (size_t)ww * G * D;
}
template <class T, int D, int BS, int G, int W>
__device__ __forceinline__ float *wave_sums(const Lds &lds)
{
    using S = Shape<T, D, BS, G, W>;
    return S::MFMA ? lds.smem : lds.smem + (size_t)S::NW * G * D;
}

template <class T, int D, int BS, int G, int W>
__global__ void partition_kernel(PartitionParams p);

// Compute units of the current device (cached per device ordinal).
inline int device_compute_units()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        cached[dev] = cus > 0 ? cus : 256;
    }
    return cached[dev];
}

// Workgroups of partition_kernel<...> that fit the device at once.
template <class T, int D, int BS, int G, int W>
int resident_workgroups()
{
    static int cached[64];  // per device ordinal; 0 = not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 1024;
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, partition_kernel<T, D, BS, G, W>, Shape<T, D, BS, G, W>::NW * kWave,
            lds_bytes<T, D, BS, G, W>() + 16);  // static staging buffers are counted by the runtime
        cached[dev] = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
    }
    return cached[dev];
}

// One wave's share of a work item on the matrix cores (fp16 / bf16 KV).
// The wave's chunks of K and V go straight from HBM into its LDS staging
// area (two chunk buffers: chunk k+1 is in flight while chunk k is
// computed).  Per 16-token tile:
//   S^T (16 tokens x 16 heads) = K_tile . q^T     D/32 MFMAs 16x16x32
//   online softmax on S^T, in the registers the MFMA wrote
//   O^T (16 dims x 16 heads) += V_tile^T . P^T      D/16 MFMAs 16x16x16
// Lane l holds S^T[token 4(l/16)+i][head l%16], which is exactly the P^T
// operand of the second product; V_tile^T comes from the transposing LDS
// load.  Heads l%16 >= G are padding (zero q, results discarded).  P enters
// the product as fp16 for fp16 KV, and as a bf16 hi + lo pair (two MFMAs, 16
// significant bits) for bf16 KV.  The softmax reference maximum of a head
// only moves when a logit exceeds it by more than 8 (log2 units); the sum
// and O always use the same reference, so the lazy update is exact.  Ends by
// writing the wave's rows, sums and maxima for the merge.
template <class T, int D, int BS, int G, int W, class LoadNew, class StoreNew>
__device__ __forceinline__ void wave_mfma(const PartitionParams &p, int b, int h, int t_begin,
                                          int t_end, int nk, int last_blk, int pb0, int ids,
                                          int64_t head_off, int64_t block_stride, float c,
                                          uint32_t qflip, bool app, int k_last, int w_last,
                                          int row_app, const LoadNew &load_new,
                                          const StoreNew &store_new, const Lds &lds, float *lred,
                                          float *mred)
{
    using S = Shape<T, D, BS, G, W>;
    constexpr int NW = S::NW, LPR = S::LPR, TPL = S::TPL, NL = S::NL, CT = S::CT;
    constexpr int R = D * S::ELT;     // bytes per token row
    constexpr int TPC = CT / 16;      // 16-token tiles per chunk
    constexpr int KS = D / 32;        // 32-dim steps of the QK product
    constexpr int MT = D / 16;        // 16-dim tiles of the output
    constexpr int CHUNK = NL * 1024;  // bytes of one tensor's chunk
    constexpr float kSlack = 8.0f;    // log2 units a logit may exceed the reference max by
    static_assert(CT % 16 == 0 && TPC >= 1, "a chunk holds whole 16-token tiles");
    static_assert(G <= 16 && (size_t)G * D * 4 <= (size_t)CHUNK, "merge rows fit the staging area");

    const int lane = threadIdx.x % kWave;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tg = lane / LPR, cl = lane % LPR;
    const int n = lane % 16, quad = lane / 16;
    const bool head_ok = n < G;
    char *stage = lds.sb[0] + (size_t)w * S::STAGE;  // this wave's [2 buffers][K, V][CHUNK]

    // XOR swizzles of a staged row's 16-byte units, so that the operand reads
    // below hit distinct LDS banks: physical unit = logical unit ^ sw(row).
    auto swk = [](int r) { return (D == 64 ? r >> 1 : r) & (LPR - 1); };
    auto swv = [](int r) { return ((D == 64 ? r >> 1 : r) & (LPR / 2 - 1)) << 1; };

    // this lane's operand offsets inside a staged chunk
    uint32_t kofs[TPC][KS], vofs[TPC][MT];
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const int r = 16 * t + n, u = quad + 4 * st;
            kofs[t][st] = r * R + 16 * (u ^ swk(r));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int r = 16 * t + lane / 4, u = 2 * mt + (lane % 4) / 2;
            vofs[t][mt] = r * R + 16 * (u ^ swv(r)) + 8 * (lane % 2);
        }
    }

    // chunk k of this wave -> buffer kd: NL 1 KiB loads of K and of V, each
    // covering TPL whole rows of one block; lane l fills physical unit l%LPR
    // of row l/LPR, i.e. reads that row's logical unit (l%LPR) ^ sw(row)
    auto stage_chunk = [&](int k, char *kd) {
        const int tc = t_begin + (w + k * NW) * CT;
        char *vd = kd + CHUNK;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t0 = tc + i * TPL;
            int rb = t0 / BS - pb0;
            rb = rb < last_blk ? rb : last_blk;
            const int blk = __builtin_amdgcn_readlane(ids, rb);
            const int64_t row = (int64_t)blk * block_stride + head_off + (t0 % BS) * R;
            const int rr = i * TPL + tg;
            load_to_lds(p.k_cache + row + tg * R + 16 * (cl ^ swk(rr)), kd + i * 1024);
            load_to_lds(p.v_cache + row + tg * R + 16 * (cl ^ swv(rr)), vd + i * 1024);
        }
    };

    float4_t O[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        O[mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float mref = -INFINITY, lsum = 0.0f;

    // The first chunk's loads go out before anything else is requested.
    if (nk > 0)
        stage_chunk(0, stage);
    // q^T operand: head n, dims 8*quad + 32*st (zero for padding heads)
    uint4 qop[KS];
    {
        const int nn = head_ok ? n : G - 1;
        const char *qrow =
            p.q + (((int64_t)b * p.num_q_heads + h * G + nn) * D + 8 * quad) * S::ELT;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            uint4 v = *reinterpret_cast<const uint4 *>(qrow + 32 * st * S::ELT);
            v.x ^= qflip;
            v.y ^= qflip;
            v.z ^= qflip;
            v.w ^= qflip;
            qop[st] = select4(head_ok, v, make_uint4(0, 0, 0, 0));
        }
    }
    uint4 knew = make_uint4(0, 0, 0, 0), vnew = make_uint4(0, 0, 0, 0);
    if (app)
        load_new(knew, vnew);

    for (int k = 0; k < nk; ++k) {
        char *kd = stage + (k & 1) * (2 * CHUNK);
        char *vd = kd + CHUNK;
        const int tc = t_begin + (w + k * NW) * CT;
        wait_vmem();  // chunk k is in LDS; nothing newer has been issued yet
        const bool full = tc + CT <= t_end;
        if (!full) {
            // rows past the end: zero V (stale or NaN slots must not reach the sum)
#pragma unroll
            for (int i = 0; i < NL; ++i)
                if (tc + i * TPL + tg >= t_end)
                    *reinterpret_cast<uint4 *>(vd + i * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
        }
        if (app && k == k_last && w == w_last && lane < LPR) {
            // position L-1 takes the new K/V, not the pool
            *reinterpret_cast<uint4 *>(kd + row_app * R + 16 * (lane ^ swk(row_app))) = knew;
            *reinterpret_cast<uint4 *>(vd + row_app * R + 16 * (lane ^ swv(row_app))) = vnew;
        }
        uint4 kop[TPC][KS];
        uint2 vop[TPC][MT];
#pragma unroll
        for (int t = 0; t < TPC; ++t) {
#pragma unroll
            for (int st = 0; st < KS; ++st)
                kop[t][st] = *reinterpret_cast<const uint4 *>(kd + kofs[t][st]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                vop[t][mt] = lds_read_tr16(vd + vofs[t][mt]);
        }
        // next chunk into the other buffer (read in the previous iteration)
        if (k + 1 < nk)
            stage_chunk(k + 1, stage + ((k + 1) & 1) * (2 * CHUNK));

#pragma unroll
        for (int t = 0; t < TPC; ++t) {
            float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < KS; ++st)
                sacc = mma_qk(T{}, kop[t][st], qop[st], sacc);
            const int tok0 = tc + 16 * t + 4 * quad;
            bool ok[4];
            float sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ok[i] = full || tok0 + i < t_end;
                sv[i] = ok[i] ? sacc[i] : -INFINITY;
            }
            const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            if (__builtin_amdgcn_ballot_w64(head_ok && mx * c > mref * c + kSlack)) {
                // new reference: the head's maximum over its four lanes
                float mh = fmaxf(mx, swz_xor16(mx));
                mh = fmaxf(mh, xor32(mh));
                const float mnew = fmaxf(mref, mh);
                const float corr =
                    mref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mref - mnew) * c);
                lsum *= corr;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    O[mt] *= corr;
                mref = mnew;
            }
            const float nmc = mref == -INFINITY ? 0.0f : -mref * c;
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pr[i] = ok[i] ? __builtin_amdgcn_exp2f(fmaf(sv[i], c, nmc)) : 0.0f;
            if constexpr (std::is_same<T, TF16>::value) {
                const half2_t h01 = {(_Float16)pr[0], (_Float16)pr[1]};
                const half2_t h23 = {(_Float16)pr[2], (_Float16)pr[3]};
                const uint2 ph = make_uint2(__builtin_bit_cast(uint32_t, h01),
                                            __builtin_bit_cast(uint32_t, h23));
                lsum += ((float)h01.x + (float)h01.y) + ((float)h23.x + (float)h23.y);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    O[mt] = mma_pv(T{}, vop[t][mt], ph, O[mt]);
            } else {
                const bf162_t h01 = {(__bf16)pr[0], (__bf16)pr[1]};
                const bf162_t h23 = {(__bf16)pr[2], (__bf16)pr[3]};
                const bf162_t l01 = {(__bf16)(pr[0] - (float)h01.x), (__bf16)(pr[1] - (float)h01.y)};
                const bf162_t l23 = {(__bf16)(pr[2] - (float)h23.x), (__bf16)(pr[3] - (float)h23.y)};
                const uint2 ph = make_uint2(__builtin_bit_cast(uint32_t, h01),
                                            __builtin_bit_cast(uint32_t, h23));
                const uint2 pl = make_uint2(__builtin_bit_cast(uint32_t, l01),
                                            __builtin_bit_cast(uint32_t, l23));
                lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    O[mt] = mma_pv(T{}, vop[t][mt], ph, O[mt]);
                    O[mt] = mma_pv(T{}, vop[t][mt], pl, O[mt]);
                }
            }
        }
    }
    if (app)
        store_new(knew, vnew);

    // The head's sum over its four lanes; its rows into this wave's (now
    // idle) staging area: lane l holds dims 16*mt + 4*quad + i of head n.
    float lh = lsum + swz_xor16(lsum);
    lh += xor32(lh);
    float *rows = wave_rows<T, D, BS, G, W>(lds, w);
    if (head_ok) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            *reinterpret_cast<float4_t *>(rows + n * D + 16 * mt + 4 * quad) = O[mt];
    }
    if (lane < G) {
        lred[w * G + lane] = lh;
        mred[w * G + lane] = mref;
    }
}

// One work item: the tokens [j*P, min((j+1)*P, L_b)) of kv head h of
// sequence b, for all G query heads of the group.  Called by every thread
// of the workgroup with the same (b, h, j).
template <class T, int D, int BS, int G, int W>
__device__ __forceinline__ void work_item(const PartitionParams &p, int b, int h, int j,
                                          const Lds &lds)
{
    float *smem = lds.smem;
    using S = Shape<T, D, BS, G, W>;
    constexpr int NW = S::NW, LPR = S::LPR, TPL = S::TPL, NL = S::NL, CT = S::CT, VEC = S::VEC;

    const int lane = threadIdx.x % kWave;
    // wave index, provably uniform: block ids and chunk bounds stay scalar
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tg = lane / LPR, cl = lane % LPR;
    const int P = p.partition_size;
    const int t_begin = j * P;
    const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks_per_seq;

    // The partition's block ids (P / BS <= 64 of them), one per lane,
    // requested together with the length.  Row indices are clamped into the
    // table and ids into the pool, so every later access stays in bounds.
    static_assert(kMaxPartition / BS <= kWave, "a partition's block ids must fit one wave");
    const int pb0 = t_begin / BS;
    int ids;
    {
        const int idx = pb0 + lane;
        ids = bt[idx < p.max_blocks_per_seq ? idx : p.max_blocks_per_seq - 1];
        ids = ids < 0 ? 0 : (ids > p.num_blocks - 1 ? p.num_blocks - 1 : ids);
    }
    int L = p.context_lens[b];
    L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
    if (t_begin >= L && !(L == 0 && j == 0))
        return;  // uniform over the workgroup
    const int t_end = min(t_begin + P, L);
    const int nchunks = (t_end - t_begin + CT - 1) / CT;
    const int nk = nchunks > w ? (nchunks - w + NW - 1) / NW : 0;  // chunks of this wave
    const int last_blk = t_end > 0 ? (t_end - 1) / BS - pb0 : 0;   // partition-relative

    // Appended token: the item holding position L-1 stores the new K/V row
    // at slots[b] and uses it from registers for that position, so no other
    // workgroup ever has to see the store.
    const bool app = p.k_new != nullptr && L > 0 && t_end == L;
    int k_last = -1, w_last = -1, i_last = 0, tg_last = 0;
    const int rel_app = L - 1 - t_begin;
    if (app) {
        const int c_last = rel_app / CT;
        w_last = c_last % NW;
        k_last = c_last / NW;
        i_last = (rel_app % CT) / TPL;
        tg_last = rel_app % TPL;
    }
    // this lane's 16 bytes of the appended K/V row, and their store at slots[b]
    // by the first wave (the pool copy is for later steps; this item uses
    // the registers)
    auto load_new = [&](uint4 &kn, uint4 &vn) {
        const int64_t hoff = (int64_t)h * D * S::ELT + cl * 16;
        kn = *reinterpret_cast<const uint4 *>(p.k_new + b * p.k_new_stride + hoff);
        vn = *reinterpret_cast<const uint4 *>(p.v_new + b * p.v_new_stride + hoff);
    };
    auto store_new = [&](const uint4 &kn, const uint4 &vn) {
        const int64_t slot = p.slots[b];
        if (w == 0 && tg == 0 && slot >= 0 && slot < p.num_slots) {
            const int64_t blk = slot / BS;
            const int64_t dst = (blk * p.num_kv_heads + h) * S::TILE + (slot - blk * BS) * (D * S::ELT) +
                                cl * 16;
            *reinterpret_cast<uint4 *>(p.k_store + dst) = kn;
            *reinterpret_cast<uint4 *>(p.v_store + dst) = vn;
        }
    };

    // Softmax runs on raw dot products scaled by c = |scale| * log2(e) >= 0
    // inside the exponent; a negative scale flips the sign of q instead (exact).
    const float c = fabsf(p.scale_log2);
    const uint32_t qflip = p.scale_log2 < 0.0f ? (S::ELT == 4 ? 0x80000000u : 0x80008000u) : 0u;
    const int64_t head_off = (int64_t)h * S::TILE;
    const int64_t block_stride = (int64_t)p.num_kv_heads * S::TILE;
    float *lred = wave_sums<T, D, BS, G, W>(lds);   // [NW][G] softmax sums
    float *mred = lred + (size_t)NW * G;         // [NW][G] maxima, raw dot units

    if constexpr (!S::MFMA) {
    uint4 knew = make_uint4(0, 0, 0, 0), vnew = make_uint4(0, 0, 0, 0);
    if (app) {
        load_new(knew, vnew);
        store_new(knew, vnew);
    }
    // query rows of the group: 16 bytes per lane per head
    uint4 qr[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        qr[g] = *reinterpret_cast<const uint4 *>(
            p.q + (((int64_t)b * p.num_q_heads + h * G + g) * D + cl * VEC) * S::ELT);
        qr[g].x ^= qflip;
        qr[g].y ^= qflip;
        qr[g].z ^= qflip;
        qr[g].w ^= qflip;
    }

    const uint32_t lane_off = lane * 16;

    // K and V of chunk k of this wave: NL wave loads each, issued without
    // conditions (so the compiler's wait counts stay exact).  Loads past the
    // partition's last token re-read its last block; those tokens are masked
    // when the chunk is processed.
    auto load_chunk = [&](int k, uint4 *kr, uint4 *vr) {
        const int tc = t_begin + (w + k * NW) * CT;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t0 = tc + i * TPL;
            int rb = t0 / BS - pb0;
            rb = rb < last_blk ? rb : last_blk;
            const int blk = __builtin_amdgcn_readlane(ids, rb);
            // wave-uniform row address (scalar registers) + this lane's 16 B
            const int64_t row = (int64_t)blk * block_stride + head_off + (t0 % BS) * (D * S::ELT);
            kr[i] = *reinterpret_cast<const uint4 *>(p.k_cache + row + lane_off);
            vr[i] = *reinterpret_cast<const uint4 *>(p.v_cache + row + lane_off);
        }
    };

    // Online softmax per lane (each lane sees one token of every load).
    float m[G], l[G], o[G][VEC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            o[g][e] = 0.0f;
    }

    // One chunk: NL wave loads of K and V, each lane one token of each.
    // FULL chunks lie entirely before t_end; the partial one masks with
    // selects (never 0 * value, so stale or NaN slots cannot leak).
    auto process = [&](auto full_tag, int k, const uint4 *kr, uint4 *vr) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int tc = t_begin + (w + k * NW) * CT;
        float s[NL * G];
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
            for (int g = 0; g < G; ++g)
                s[i * G + g] = dot16(T{}, qr[g], kr[i], 0.0f);
        group_sum_all<LPR>(s);
        bool valid[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            valid[i] = FULL || tc + i * TPL + tg < t_end;
            if constexpr (!FULL) {
                vr[i].x = valid[i] ? vr[i].x : 0u;
                vr[i].y = valid[i] ? vr[i].y : 0u;
                vr[i].z = valid[i] ? vr[i].z : 0u;
                vr[i].w = valid[i] ? vr[i].w : 0u;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float cm = valid[0] ? s[g] : -INFINITY;
#pragma unroll
            for (int i = 1; i < NL; ++i)
                cm = fmaxf(cm, valid[i] ? s[i * G + g] : -INFINITY);
            const float m_new = fmaxf(m[g], cm);
            const float nmc = -(m_new == -INFINITY ? 0.0f : m_new) * c;
            const float corr = m[g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(m[g], c, nmc));
            l[g] *= corr;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                o[g][e] *= corr;
            m[g] = m_new;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                float pw = __builtin_amdgcn_exp2f(fmaf(s[i * G + g], c, nmc));
                if constexpr (!FULL)
                    pw = valid[i] ? pw : 0.0f;
                l[g] += pw;
                axpy16(T{}, pw, vr[i], o[g]);
            }
        }
    };
    auto process_any = [&](int k, uint4 *kr, uint4 *vr) {
        if (app && k == k_last && w == w_last) {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                if (i == i_last) {
                    const bool mine = tg == tg_last;
                    kr[i].x = mine ? knew.x : kr[i].x;
                    kr[i].y = mine ? knew.y : kr[i].y;
                    kr[i].z = mine ? knew.z : kr[i].z;
                    kr[i].w = mine ? knew.w : kr[i].w;
                    vr[i].x = mine ? vnew.x : vr[i].x;
                    vr[i].y = mine ? vnew.y : vr[i].y;
                    vr[i].z = mine ? vnew.z : vr[i].z;
                    vr[i].w = mine ? vnew.w : vr[i].w;
                }
            }
        }
        if (t_begin + (w + k * NW) * CT + CT <= t_end)
            process(std::true_type{}, k, kr, vr);
        else
            process(std::false_type{}, k, kr, vr);
    };

    // Software pipeline: a ring of kPrefetchDepth + 1 chunk buffers; the
    // loads of chunks k+1 .. k+kPrefetchDepth are in flight while chunk k is
    // processed.  Every load is issued unconditionally (past the wave's last
    // chunk the index is clamped to it, a cache hit), so the compiler's wait
    // counts stay exact.
    if (nk > 0) {
        constexpr int NBUF = kPrefetchDepth + 1;
        uint4 kbuf[NBUF][NL], vbuf[NBUF][NL];
#pragma unroll
        for (int d = 0; d < kPrefetchDepth; ++d)
            load_chunk(d < nk ? d : nk - 1, kbuf[d], vbuf[d]);
        for (int k0 = 0; k0 < nk; k0 += NBUF) {
#pragma unroll
            for (int r = 0; r < NBUF; ++r) {
                const int k = k0 + r;
                if (k >= nk)
                    break;
                const int kn = k + kPrefetchDepth < nk ? k + kPrefetchDepth : nk - 1;
                load_chunk(kn, kbuf[(r + kPrefetchDepth) % NBUF], vbuf[(r + kPrefetchDepth) % NBUF]);
                process_any(k, kbuf[r], vbuf[r]);
            }
        }
    }

    // Rescale every lane to the wave's maximum, then sum the token groups
    // in registers (lanes that hold the same dims of different tokens).
    float mw[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mw[g] = wave_max(m[g]);
        const float f = m[g] == -INFINITY ? 0.0f
                        : __builtin_amdgcn_exp2f((m[g] - mw[g]) * c);
        l[g] = token_group_sum<LPR>(l[g] * f);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            o[g][e] = token_group_sum<LPR>(o[g][e] * f);
    }

    // this wave's rows for the merge in LDS
    if (tg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float *dst = wave_rows<T, D, BS, G, W>(lds, w) + (size_t)g * D + cl * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                dst[e] = o[g][e];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            lred[w * G + g] = l[g];
            mred[w * G + g] = mw[g];
        }
    }
    } else {
        wave_mfma<T, D, BS, G, W>(p, b, h, t_begin, t_end, nk, last_blk, pb0, ids, head_off,
                               block_stride, c, qflip, app, k_last, w_last, rel_app % CT,
                               load_new, store_new, lds, lred, mred);
    }
    __syncthreads();

    // ---- merge the waves in LDS (log-sum-exp with the wave maxima) ------

    const int nparts_b = L == 0 ? 1 : (L + P - 1) / P;
    for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
        const int g = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            M = fmaxf(M, mred[ww * G + g]);
        float acc = 0.0f, den = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mv = mred[ww * G + g];
            const float sc = mv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mv - M) * c);
            acc = fmaf(wave_rows<T, D, BS, G, W>(lds, ww)[(size_t)g * D + d], sc, acc);
            den = fmaf(lred[ww * G + g], sc, den);
        }
        M = M == -INFINITY ? M : M * c;  // log2 units for the partition merge
        const float res = den > 0.0f ? acc / den : 0.0f;
        const int hq = h * G + g;
        if (nparts_b == 1) {
            store_out(p.out, ((int64_t)b * p.num_q_heads + hq) * D + d, res, p.out_kind);
        } else {
            // coherent (agent-scope) stores: the merging workgroup may run on
            // another XCD, whose L2 does not see this one's write-back lines
            const int64_t row = ((int64_t)b * p.num_q_heads + hq) * p.num_partitions + j;
            coherent_store(&p.ws_o[row * D + d], res);
            if (d == 0) {
                coherent_store(&p.ws_ml[row * 2 + 0], M);
                coherent_store(&p.ws_ml[row * 2 + 1], den);
            }
        }
    }
    if (nparts_b == 1)
        return;

    // ---- the last partition of (b, h) to finish merges all of them --------
    // With m_j in log2 units: w_j = l_j * 2^(m_j - max m),
    // out = sum_j w_j o_j / sum_j w_j (exact rescaling, log-sum-exp).
    // Publication without an L2 flush: the rows above were written with
    // coherent stores; waiting for their acknowledgement before the
    // workgroup barrier orders them before the counter increment, and the
    // merging workgroup reads them back with coherent loads.
    int *flag = reinterpret_cast<int *>(smem + lds_bytes<T, D, BS, G, W>() / 4) + 1;
    int32_t *counter = p.counters + (int64_t)b * p.num_kv_heads + h;
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0)
        *flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                nparts_b - 1;
    __syncthreads();
    if (!*flag)
        return;
    for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
        const int g = idx / D, d = idx % D;
        const int64_t row0 = ((int64_t)b * p.num_q_heads + h * G + g) * p.num_partitions;
        float M = -INFINITY;
        for (int jj = 0; jj < nparts_b; ++jj)
            M = fmaxf(M, coherent_load(&p.ws_ml[(row0 + jj) * 2]));
        float acc = 0.0f, den = 0.0f;
        for (int jj = 0; jj < nparts_b; ++jj) {
            const float wgt = coherent_load(&p.ws_ml[(row0 + jj) * 2 + 1]) *
                              __builtin_amdgcn_exp2f(coherent_load(&p.ws_ml[(row0 + jj) * 2]) - M);
            den += wgt;
            acc = fmaf(wgt, coherent_load(&p.ws_o[(row0 + jj) * D + d]), acc);
        }
        store_out(p.out, ((int64_t)b * p.num_q_heads + h * G + g) * D + d, acc / den, p.out_kind);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T, int D, int BS, int G, int W>
__global__ __launch_bounds__((Shape<T, D, BS, G, W>::NW * kWave)) void partition_kernel(PartitionParams p)
{
    using S = Shape<T, D, BS, G, W>;
    extern __shared__ float smem[];
    __shared__ __attribute__((aligned(1024))) char sb0[S::MFMA ? S::STAGE * S::NW : 16];
    const Lds lds{smem, {sb0}};
    if (p.items == nullptr) {
        work_item<T, D, BS, G, W>(p, blockIdx.z, blockIdx.y, blockIdx.x, lds);
        return;
    }
    // Work-list mode (skewed batches): a persistent grid.  Workgroup g starts
    // with item g and then takes the next unclaimed item from the counter the
    // plan kernel initialised to the grid size.
    int *slot = reinterpret_cast<int *>(smem + lds_bytes<T, D, BS, G, W>() / 4);
    const int hkv = p.num_kv_heads;
    const int total = p.wl_header[1] * hkv;
    int u = blockIdx.x;
    while (u < total) {
        int next = 0;
        if (threadIdx.x == 0)
            next = atomicAdd(&p.wl_header[0], 1);  // consumed after the item
        const int sidx = u / hkv;
        const int2 it = p.items[sidx];
        work_item<T, D, BS, G, W>(p, it.x, u - sidx * hkv, it.y, lds);
        if (threadIdx.x == 0)
            *slot = next;
        __syncthreads();
        u = __builtin_amdgcn_readfirstlane(*slot);
        __syncthreads();
    }
}

// Build the work list of a skewed batch: every sequence b contributes
// max(1, ceil(L_b / P)) items {b, j}, in batch order.  One workgroup.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *context_lens, int32_t num_seqs,
                                                    int32_t partition_size, int32_t len_cap,
                                                    int2 *items, int32_t *header,
                                                    int32_t first_dynamic)
{
    __shared__ int wave_tot[1024 / kWave];
    __shared__ int wave_off[1024 / kWave];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    int carry = 0;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int i = base + threadIdx.x;
        int n = 0;
        if (i < num_seqs) {
            int L = context_lens[i];
            L = L < 0 ? 0 : (L > len_cap ? len_cap : L);
            n = L == 0 ? 1 : (L + partition_size - 1) / partition_size;
        }
        int x = n;  // inclusive scan within the wave
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(x, off, kWave);
            if (lane >= off)
                x += y;
        }
        if (lane == kWave - 1)
            wave_tot[wv] = x;
        __syncthreads();
        if (threadIdx.x == 0) {
            int acc = 0;
            for (int k = 0; k < 1024 / kWave; ++k) {
                wave_off[k] = acc;
                acc += wave_tot[k];
            }
        }
        __syncthreads();
        const int start = carry + wave_off[wv] + x - n;
        for (int jj = 0; jj < n; ++jj)
            items[start + jj] = make_int2(i, jj);
        carry += wave_off[1024 / kWave - 1] + wave_tot[1024 / kWave - 1];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        header[0] = first_dynamic;
        header[1] = carry;
    }
}

template <class T, int D, int BS, int G, int W>
hipError_t launch_waves(const DecodeArgs &a, hipStream_t stream)
{
    using S = Shape<T, D, BS, G, W>;
    PartitionParams p;
    p.out = a.out;
    p.out_kind = (int)a.out_dtype;
    p.q = static_cast<const char *>(a.q);
    p.k_cache = static_cast<const char *>(a.k_cache);
    p.v_cache = static_cast<const char *>(a.v_cache);
    p.block_tables = a.block_tables;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.context_lens = a.context_lens;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.num_blocks = a.num_blocks;
    p.scale_log2 = a.scale * kLog2e;
    p.partition_size = a.partition_size;
    p.num_partitions = a.num_partitions;
    const int64_t cap_table = (int64_t)a.max_blocks_per_seq * a.block_size;
    const int64_t cap_grid = (int64_t)a.num_partitions * a.partition_size;
    const int64_t cap = cap_table < cap_grid ? cap_table : cap_grid;
    p.len_cap = (int32_t)(cap > INT32_MAX ? INT32_MAX : cap);
    p.ws_o = a.ws_o;
    p.ws_ml = a.ws_ml;
    p.items = a.items;
    p.wl_header = a.wl_header;
    p.counters = a.counters;
    p.k_new = static_cast<const char *>(a.k_new);
    p.v_new = static_cast<const char *>(a.v_new);
    p.k_new_stride = a.k_new_token_stride * dtype_bytes(a.kv_dtype);
    p.v_new_stride = a.v_new_token_stride * dtype_bytes(a.kv_dtype);
    p.slots = a.slot_mapping;
    p.k_store = static_cast<char *>(const_cast<void *>(a.k_cache));
    p.v_store = static_cast<char *>(const_cast<void *>(a.v_cache));
    p.num_slots = (int64_t)a.num_blocks * a.block_size;

    const size_t lds = lds_bytes<T, D, BS, G, W>() + 16;
    hipError_t e;
    if (a.items) {
        const int64_t dense = (int64_t)a.num_partitions * a.num_kv_heads * a.num_seqs;
        const int64_t res = resident_workgroups<T, D, BS, G, W>();
        const int grid = (int)(dense < res ? dense : res);
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.context_lens,
                           a.num_seqs, a.partition_size, p.len_cap, a.items, a.wl_header, grid);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL((partition_kernel<T, D, BS, G, W>), dim3(grid), dim3(S::NW * kWave), lds,
                           stream, p);
    } else {
        const dim3 grid((unsigned)a.num_partitions, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
        hipLaunchKernelGGL((partition_kernel<T, D, BS, G, W>), grid, dim3(S::NW * kWave), lds, stream,
                           p);
    }
    return hipGetLastError();
}

// Waves per workgroup.  fp32 KV (vector ALUs): 4, or 2 where the register
// state of a wave is large.  Half KV (matrix cores): 8 when the grid of work
// items is no larger than the number of compute units (a short batch is
// latency-bound, so each item gets more waves), else 4 (more items resident
// per compute unit).
template <class T, int D, int BS, int G>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s)
{
    if constexpr (std::is_same<T, TF32>::value) {
        constexpr int TPL = kWave / (D * 4 / 16);
        return launch_waves<T, D, BS, G, (G * D * TPL * 4 * 4 > 48 * 1024) ? 2 : 4>(a, s);
    } else {
        const int64_t items = (int64_t)a.num_partitions * a.num_kv_heads * a.num_seqs;
        if (a.items == nullptr && items <= device_compute_units())
            return launch_waves<T, D, BS, G, 8>(a, s);
        return launch_waves<T, D, BS, G, 4>(a, s);
    }
}

template <class T, int D, int BS>
hipError_t dispatch_group(const DecodeArgs &a, hipStream_t s)
{
    switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_typed<T, D, BS, 1>(a, s);
    case 2: return launch_typed<T, D, BS, 2>(a, s);
    case 4: return launch_typed<T, D, BS, 4>(a, s);
    case 8: return launch_typed<T, D, BS, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

template <class T, int D>
hipError_t dispatch_block(const DecodeArgs &a, hipStream_t s)
{
    switch (a.block_size) {
    case 16: return dispatch_group<T, D, 16>(a, s);
    case 32: return dispatch_group<T, D, 32>(a, s);
    }
    return hipErrorInvalidValue;
}

template <class T>
hipError_t dispatch_dim(const DecodeArgs &a, hipStream_t s)
{
    switch (a.head_dim) {
    case 64: return dispatch_block<T, 64>(a, s);
    case 128: return dispatch_block<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(DType kv, int head_dim, int block_size, int group)
{
    (void)kv;
    return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.num_seqs == 0)
        return hipSuccess;
    switch (a.kv_dtype) {
    case DType::F32: return dispatch_dim<TF32>(a, stream);
    case DType::F16: return dispatch_dim<TF16>(a, stream);
    case DType::BF16: return dispatch_dim<TBF16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pka
