// Device primitives for CDNA4 (gfx950) shared by the attention kernels:
// dtype tags, 16-byte dot products and axpys on the vector ALUs, the two
// matrix-core products of the attention tiles, LDS staging by DMA, the
// transposing LDS read, cross-lane reductions, output conversion and the
// wait-count helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pka {

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;

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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// fp32 KV: the same two tile products on v_mfma_f32_16x16x4f32, four
// products per 16-byte operand.  Score step: lane l supplies 4 consecutive
// dims of K[token l%16] and of q[head l%16] (one 16-byte unit); product j
// takes dim j of the unit as its k = l/16.  PV: lane l supplies V[token
// 4(l/16)+j][dim l%16] and P[same token][head l%16] in element j; product j
// takes k = l/16 <-> token 4(l/16)+j.
__device__ __forceinline__ float4_t mma_qk(TF32, const uint4 &k, const uint4 &q, float4_t acc)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(k.x), as_f(q.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(k.y), as_f(q.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(k.z), as_f(q.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(k.w), as_f(q.w), acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ float4_t mma_pv(TF32, const uint4 &v, const uint4 &pr, float4_t acc)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(v.x), as_f(pr.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(v.y), as_f(pr.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(v.z), as_f(pr.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(v.w), as_f(pr.w), acc, 0, 0, 0);
    return acc;
}

// A wave-uniform int32 read through the scalar data cache (the address must
// be wave-uniform and the memory unchanged for the whole kernel).  Scalar
// loads count on lgkmcnt, so waiting for one never waits for the vector
// loads in flight.
__device__ __forceinline__ int32_t scalar_load(const int32_t *base, int64_t i)
{
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    return ((const const_i32 *)(uintptr_t)base)[i];
}

// 16 bytes per lane straight from global memory into LDS at byte address
// lds_base + 16*lane (lds_base is wave-uniform: it goes to M0).
__device__ __forceinline__ void load_to_lds(const char *g, uint32_t lds_base)
{
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(uintptr_t)lds_base, 16, 0, 0);
}
// LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    typedef __attribute__((address_space(3))) const char lds_char;
    return (uint32_t)(uintptr_t)(lds_char *)p;
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

// Sum over the whole wave, returned as a wave-uniform value.
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    x += swz_xor16(x);
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    return lo + hi;
}

// Sums / maxima over the whole wave of N values at once, returned
// wave-uniform: the stages of the N reductions are interleaved, so their
// latencies overlap instead of adding up.
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&x)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp<0xB1>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp<0x4E>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp<0x141>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp<0x140>(x[i]);
    float t[N];
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = swz_xor16(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        x[i] += t[i];
        const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x[i]), 0));
        const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x[i]), 32));
        x[i] = lo + hi;
    }
}
template <int N>
__device__ __forceinline__ void wave_max_n(float (&x)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = fmaxf(x[i], dpp<0xB1>(x[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = fmaxf(x[i], dpp<0x4E>(x[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = fmaxf(x[i], dpp<0x141>(x[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = fmaxf(x[i], dpp<0x140>(x[i]));
    float t[N];
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = swz_xor16(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        x[i] = fmaxf(x[i], t[i]);
        const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x[i]), 0));
        const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x[i]), 32));
        x[i] = fmaxf(lo, hi);
    }
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

// Four consecutive output elements out[idx .. idx+3] (idx a multiple of 4)
// in one vector store.
__device__ __forceinline__ void store_out4(void *out, int64_t idx, float4_t x, int out_kind)
{
    if (out_kind == 0) {
        *reinterpret_cast<float4_t *>(static_cast<float *>(out) + idx) = x;
    } else if (out_kind == 1) {
        const half2_t a = {(_Float16)x[0], (_Float16)x[1]};
        const half2_t b = {(_Float16)x[2], (_Float16)x[3]};
        *reinterpret_cast<uint2 *>(static_cast<_Float16 *>(out) + idx) =
            make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
    } else {
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + idx) =
            make_uint2(f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16),
                       f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16));
    }
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
// Raw buffer view of `bytes` bytes at `base` (wave-uniform), for the 16-byte
// coherent accesses below; accesses past `bytes` read zero / write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
// Cache policy of the buffer accesses: sc1, the coherence bit that the
// agent-scope relaxed accesses above carry.
constexpr int kCoherentPolicy = 16;
// 16 bytes at a 16-byte aligned byte offset, with the coherence of
// coherent_store / coherent_load: one access for four consecutive floats.
__device__ __forceinline__ void coherent_store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset,
                                                 float4_t v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_offset, 0,
                                           kCoherentPolicy);
}
__device__ __forceinline__ float4_t coherent_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset)
{
    return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0,
                                                                              kCoherentPolicy));
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left free): every vector memory
// access of this wave has completed (loads landed, stores acknowledged).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left free): this wave's LDS
// accesses have completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left free
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }
// Every vector memory access of this wave except the n most recent has
// completed (n is wave-uniform, 0..63; vector memory accesses complete in
// issue order for this count).
__device__ __forceinline__ void wait_vmem_keep(int n)
{
    switch (n) {
#define PKA_KEEP(k) \
    case k: __builtin_amdgcn_s_waitcnt(vmcnt_imm(k)); break;
#define PKA_KEEP8(k) PKA_KEEP(k) PKA_KEEP(k + 1) PKA_KEEP(k + 2) PKA_KEEP(k + 3) \
    PKA_KEEP(k + 4) PKA_KEEP(k + 5) PKA_KEEP(k + 6) PKA_KEEP(k + 7)
    PKA_KEEP(1) PKA_KEEP(2) PKA_KEEP(3) PKA_KEEP(4) PKA_KEEP(5) PKA_KEEP(6) PKA_KEEP(7)
    PKA_KEEP8(8) PKA_KEEP8(16) PKA_KEEP8(24) PKA_KEEP8(32) PKA_KEEP8(40) PKA_KEEP8(48)
    PKA_KEEP8(56)
#undef PKA_KEEP8
#undef PKA_KEEP
    default: wait_vmem();
    }
}

// ---- LDS accesses the compiler does not see ------------------------------
// Staged chunks arrive by LDS DMA, which the compiler tracks only as "some
// LDS write pending": before any LDS access it would wait for every vector
// memory access in flight, stores included.  The operand reads and the few
// staging writes of the attention loop are therefore written here in
// assembly, each block complete (its own lgkmcnt(0)) before it ends, and the
// loop waits for exactly the DMA it needs.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four 16-byte reads and eight transposing 8-byte reads (one chunk's K and
// V operands of the fp16/bf16 tiles) at LDS byte addresses ka[] + OFF,
// va[] + OFF (OFF selects the chunk buffer without per-lane adds).
template <int OFF>
__device__ __forceinline__ void lds_read_chunk(u32x4 (&k)[4], u32x2 (&v)[8], const uint32_t (&ka)[4],
                                               const uint32_t (&va)[8])
{
    asm volatile(
        "ds_read_b128 %0, %12 offset:%24\n\t"
        "ds_read_b128 %1, %13 offset:%24\n\t"
        "ds_read_b128 %2, %14 offset:%24\n\t"
        "ds_read_b128 %3, %15 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %10, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %11, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]),
          "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
          "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]), "i"(OFF)
        : "memory");
}
// One 16-byte LDS write, complete before the block ends.
// 16 bytes from LDS byte address addr, waited for in the same block (the
// compiler does not track it, so it never waits for LDS DMA on its behalf).
__device__ __forceinline__ uint4 lds_read16(uint32_t addr)
{
    u32x4 d;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(d) : "v"(addr) : "memory");
    return make_uint4(d[0], d[1], d[2], d[3]);
}
__device__ __forceinline__ void lds_write16(uint32_t addr, const uint4 &x)
{
    const u32x4 d = {x.x, x.y, x.z, x.w};
    asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(d) : "memory");
}

}  // namespace pka
