// Group-quantised INT8 KV cache for gfx950: the quantising batched write
// and the paged decode over it.
//
// What is stored (PhotonInfer README, Korean translation, "Key features >
// GPU-optimised kernels" and "Technical details > INT8 quantisation":
// INT8 quantisation in groups of a configurable size, 32, 64 or 128; the
// README quantises weights, this library applies the scheme to the KV rows):
// each new token's row of one kv head is cut into groups of GS consecutive
// dims; a group keeps one float32 scale s = amax / 127 and codes
// c = rint(x / s) in [-127, 127], and stands for c * s.
//
// Layouts.  One physical block of one kv head is a contiguous run of each
// array.  The BS * D codes of a block run are ordered for the matrix cores:
// tokens in tiles of 16 (offset = 16 * tile + row), and lane L = 16 * j + r
// of a wave owns the D / 4 bytes at (tile * 64 + L) * D / 4:
//   K: for each 32-dim slab c, dims 32c + 8j .. +7 of token row r
//      (the A operand of the score MFMA);
//   V: for each 16-dim block m, tokens 4j .. 4j+3 of dim 16m + r
//      (the A operand of the PV MFMA).
//   k_scales, v_scales  f32 [NB][Hkv][BS][D/GS]   token-major
//
// Decode design (CDNA4-first):
//  * Work unit = (sequence, partition, kv head), one wave each; the G query
//    heads of the kv head share every code and scale read.  Four waves per
//    workgroup run four independent units; no LDS.
//  * The wave streams its tokens in steps of 16-token tiles straight into
//    registers.  Per tile each lane loads its own contiguous D / 4 bytes of
//    K codes and of V codes (the wave's loads are fully coalesced: 1 KiB or
//    2 KiB per instruction) and the scales of its 4 tokens.
//  * Codes become fp16 exactly (1024 + (c + 128) is an fp16 whose low byte
//    is the offset code), so both products run as fp16 MFMAs with fp32
//    accumulation.  bf16 queries are brought into fp16 by a per-head power
//    of two (exact), folded back into the score multiplier.
//  * Scores: one 16x16x32 MFMA per slab gives S^T (16 tokens x 16 heads);
//    slabs of a group accumulate together, then each group is multiplied by
//    its K scale.  The softmax is online in log2 units.
//  * PV: the V scale varies per token inside the reduction, so it goes into
//    the probability operand: P'' = p * s_v * r_g, with r_g a power of two
//    per work unit and group (from a first pass over the unit's V scales)
//    that keeps s_v * r_g in [0, 2) for fp16; O is divided by r_g (exactly)
//    at the end.  The softmax reference max is lazy (p <= 2^8), so the MFMAs
//    accumulate straight into O and a rescale is rare.
//  * One partition per sequence: the wave writes the output.  2 to 8: one
//    workgroup per (sequence, kv head), wave w on partition w, and the
//    workgroup merges the waves' (max, sum, O / sum) rows in LDS.  More: a
//    persistent grid deals the (sequence, partition) items, found in a
//    prefix each workgroup builds in LDS (up to 4096 sequences) or listed by
//    a one-workgroup planning launch; the units write their rows to the
//    workspace and a merge launch combines them.
//  * Fused append (pka_paged_attention_decode_append_int8): the unit that
//    holds position L_b - 1 quantises the new K/V rows of its kv head,
//    stores them, and takes their codes and scales from its registers where
//    it would read them back, so the result is that of the write followed
//    by the decode and nothing waits for the stores.
//  * Tokens past the unit's end are excluded by selects (scores to -inf,
//    probabilities and scales to 0), so poisoned scales never reach O.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "cdna4.h"
#include "pka_internal.h"

namespace pka {
namespace {

constexpr int kI8Waves = 4;             // waves (independent units) per workgroup
constexpr int kI8Tiles = 2;                   // 16-token tiles per step
constexpr int kI8Step = 16 * kI8Tiles;        // tokens per step
constexpr int kI8PlanThreads = 1024;    // planning workgroup
// Up to this many partitions per sequence the decode launches one wave per
// (sequence, partition, kv head) and no planning launch.
constexpr int kI8DenseMaxPartitions = 8;
// With 2..kI8DenseMaxPartitions partitions, one workgroup per (sequence, kv
// head) whose wave w takes partition w merges the partitions' rows in LDS
// (no merge launch, no partial rows in HBM).
// Persistent grids over at most this many sequences plan their work in each
// workgroup's LDS (a prefix of partition counts) instead of a planning launch.
constexpr int kI8PlanInKernelSeqs = 4096;

// ---- quantising write ------------------------------------------------------

template <int N>
__device__ __forceinline__ float lanes_max(float x)
{
    // max over aligned groups of N consecutive lanes (N = 16, 32 or 64)
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    if constexpr (N >= 32) x = fmaxf(x, swz_xor16(x));
    if constexpr (N >= 64) x = fmaxf(x, xor32(x));
    return x;
}

__device__ __forceinline__ float load_as_f32(TF32, const void *p, int64_t i)
{
    return static_cast<const float *>(p)[i];
}
__device__ __forceinline__ float load_as_f32(TF16, const void *p, int64_t i)
{
    return (float)static_cast<const _Float16 *>(p)[i];
}
__device__ __forceinline__ float load_as_f32(TBF16, const void *p, int64_t i)
{
    return as_f((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
}

// One token's row of one kv head, quantised by one wave: lane l holds dims
// [l*E, l*E + E), E = D / 64.  load_row reads the D elements of type T at
// src[src_row ..]; quantise_row takes the group's amax over the GS / E
// lanes holding it, s = amax / 127 (IEEE division), codes rint(x / s), and
// returns the lane's group scale; store_row stores codes and scale at
// (block blk, offset off) of a pool in its layout.
template <class T, int D>
__device__ __forceinline__ void load_row(const void *src, int64_t src_row, int lane,
                                         float (&x)[D / kWave])
{
#pragma unroll
    for (int e = 0; e < D / kWave; ++e)
        x[e] = load_as_f32(T{}, src, src_row + lane * (D / kWave) + e);
}

template <int D, int GS>
__device__ __forceinline__ float quantise_row(const float (&x)[D / kWave], int8_t (&c)[D / kWave])
{
    constexpr int E = D / kWave;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e)
        amax = fmaxf(amax, fabsf(x[e]));
    amax = lanes_max<GS / E>(amax);
    const float s = amax / 127.0f;  // IEEE division (correctly rounded)
#pragma unroll
    for (int e = 0; e < E; ++e) {
        float q = s > 0.0f ? rintf(x[e] / s) : 0.0f;
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        c[e] = (int8_t)q;
    }
    return s;
}

template <int D, int GS>
__device__ __forceinline__ void store_row(const int8_t (&c)[D / kWave], float s, bool is_value,
                                          int8_t *codes_pool, float *scales_pool,
                                          int num_kv_heads, int block_size, int64_t blk, int h,
                                          int off, int lane)
{
    constexpr int E = D / kWave;
    constexpr int NG = D / GS;
    const int64_t run = blk * num_kv_heads + h;  // this block's run of codes
    int8_t *codes = codes_pool + run * block_size * D;
    const int tl = off / 16, row = off % 16;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int d = lane * E + e;
        const int64_t pos =
            is_value ? ((int64_t)(tl * 64 + 16 * (row / 4) + d % 16) * (D / 16) + d / 16) * 4 + row % 4
                     : ((int64_t)(tl * 64 + 16 * ((d % 32) / 8) + row) * (D / 32) + d / 32) * 8 + d % 8;
        codes[pos] = c[e];
    }
    if ((lane * E) % GS == 0)
        scales_pool[(run * block_size + off) * NG + lane * E / GS] = s;
}

// The lane's codes in one dword (byte e: dim l*E + e).
template <int E>
__device__ __forceinline__ uint32_t pack_codes(const int8_t (&c)[E])
{
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
        w |= (uint32_t)(uint8_t)c[e] << (8 * e);
    return w;
}

template <class T, int D, int GS>
__device__ __forceinline__ void quantize_store_row(const void *src, int64_t src_row, bool is_value,
                                                   int8_t *codes_pool, float *scales_pool,
                                                   int num_kv_heads, int block_size, int64_t blk,
                                                   int h, int off, int lane)
{
    float x[D / kWave];
    int8_t c[D / kWave];
    load_row<T, D>(src, src_row, lane, x);
    const float s = quantise_row<D, GS>(x, c);
    store_row<D, GS>(c, s, is_value, codes_pool, scales_pool, num_kv_heads, block_size, blk, h,
                     off, lane);
}

// One wave per (new token, kv head, tensor).
template <class T, int D, int GS>
__global__ __launch_bounds__(256) void quantize_write_kernel(Int8WriteArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t rows = (int64_t)a.num_tokens * a.num_kv_heads;
    if (wid >= 2 * rows)
        return;
    const int is_value = (int)(wid / rows);
    const int64_t r = wid % rows;
    const int64_t i = r / a.num_kv_heads;
    const int h = (int)(r % a.num_kv_heads);
    const int64_t slot = a.slot_mapping[i];
    if (slot < 0 || slot >= (int64_t)a.num_blocks * a.block_size)
        return;
    const void *src = is_value ? a.v : a.k;
    const int64_t src_row = i * (is_value ? a.v_token_stride : a.k_token_stride) + (int64_t)h * D;
    quantize_store_row<T, D, GS>(src, src_row, is_value, is_value ? a.v_codes : a.k_codes,
                                 is_value ? a.v_scales : a.k_scales, a.num_kv_heads, a.block_size,
                                 slot / a.block_size, h, (int)(slot % a.block_size), lane);
}

// ---- decode ----------------------------------------------------------------

// 4 codes (one dword, token or dim order kept) -> 4 fp16 values, exact, by
// the well-known exponent-bias ("magic number") integer-to-float conversion:
// the byte c + 128 under the exponent byte 0x64 is the fp16 1024 + c + 128,
// and subtracting 1152 leaves c.
__device__ __forceinline__ uint2 codes_to_f16(uint32_t w)
{
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const half2_t a = __builtin_bit_cast(half2_t, lo) - bias;
    const half2_t b = __builtin_bit_cast(half2_t, hi) - bias;
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b)
{
    const half2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// max over the four lanes that share lane % 16 (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float column_max(float x)
{
    x = fmaxf(x, swz_xor16(x));
    return fmaxf(x, xor32(x));
}
__device__ __forceinline__ float column_sum(float x)
{
    x += swz_xor16(x);
    return x + xor32(x);
}

// Exact power-of-two normaliser of a non-negative bound sigma: r with
// sigma * r in [0, 2) (or smaller when sigma is tiny), and 1 / r exactly.
__device__ __forceinline__ void pow2_normaliser(float sigma, float &r, float &inv_r)
{
    int e = (int)((__builtin_bit_cast(uint32_t, sigma) >> 23) & 0xff);
    e = e < 1 ? 1 : (e > 253 ? 253 : e);
    r = as_f((uint32_t)(254 - e) << 23);
    inv_r = as_f((uint32_t)e << 23);
}

template <int D, int NG>
struct StepRegs {
    uint4 k[kI8Tiles][D / 64];  // per tile: the lane's D/4 bytes of K codes (8 per slab)
    uint4 v[kI8Tiles][D / 64];  // per tile: the lane's D/4 bytes of V codes (4 per dim block)
    float4 ks[kI8Tiles][NG];       // per tile: K scales of tokens 4j..4j+3 ([token][group])
    float4 vs[kI8Tiles][NG];
};

template <int D, int BS, int GS>
struct I8Shape {
    static constexpr int NG = D / GS;
    static constexpr int SLABS = D / 32;
    static constexpr int DB = D / 16;  // 16-dim blocks of the output
    static constexpr int SLABS_PER_GROUP = GS / 32;
};

// Issue the loads of the two tiles starting at token ts (the block of a
// tile is ids lane (t0 - t_part0) / BS).  A tile past the unit's end is
// loaded too, from a block the lanes past the partition's last id repeat
// (in bounds; its tokens are masked when computed), so that the number of
// loads in flight is the same on every path and the waits stay exact.
template <int D, int BS, int GS>
__device__ __forceinline__ void load_step(const Int8DecodeArgs &a, StepRegs<D, D / GS> &R,
                                          int ids, int t_part0, int ts, int t_end, int h,
                                          int lane)
{
    using S = I8Shape<D, BS, GS>;
    const int j = lane >> 4;
#pragma unroll
    for (int tile = 0; tile < kI8Tiles; ++tile) {
        const int t0 = ts + 16 * tile;
        const int blk = __builtin_amdgcn_readfirstlane(
            __builtin_amdgcn_readlane(ids, (t0 - t_part0) / BS));
        const int off0 = t0 % BS;
        const int64_t tile_idx = (int64_t)blk * a.num_kv_heads + h;
        const int64_t mine = tile_idx * BS * D + (int64_t)((off0 / 16) * 64 + lane) * (D / 4);
        const uint4 *kp = reinterpret_cast<const uint4 *>(a.k_codes + mine);
        const uint4 *vp = reinterpret_cast<const uint4 *>(a.v_codes + mine);
#pragma unroll
        for (int q = 0; q < D / 64; ++q) {
            R.k[tile][q] = kp[q];
            R.v[tile][q] = vp[q];
        }
        const int64_t srow = (tile_idx * BS + off0 + 4 * j) * S::NG;
#pragma unroll
        for (int g = 0; g < S::NG; ++g) {
            R.ks[tile][g] = reinterpret_cast<const float4 *>(a.k_scales + srow)[g];
            R.vs[tile][g] = reinterpret_cast<const float4 *>(a.v_scales + srow)[g];
        }
    }
}

__device__ __forceinline__ uint32_t u4(const uint4 &v, int i)
{
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float f4(const float4 &v, int i)
{
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ void set_u4(uint4 &v, int i, uint32_t x)
{
    if (i == 0)
        v.x = x;
    else if (i == 1)
        v.y = x;
    else if (i == 2)
        v.z = x;
    else
        v.w = x;
}

__device__ __forceinline__ void set_f4(float4 &v, int i, float x)
{
    if (i == 0)
        v.x = x;
    else if (i == 1)
        v.y = x;
    else if (i == 2)
        v.z = x;
    else
        v.w = x;
}

// Scale of token 4j+i of a tile, group g, from the [token][group] rows a
// lane holds (NG float4 = 4 tokens x NG groups).
template <int NG>
__device__ __forceinline__ float scale_of(const float4 (&rows)[NG], int i, int g)
{
    const int flat = i * NG + g;
    return f4(rows[flat / 4], flat % 4);
}

template <int D, int BS, int GS>
struct UnitState {
    float4_t o[D / 16];  // O^T[dim 16m + 4j + i][head lane%16], times r of its group
    float m;             // reference max (log2 units) of head lane%16
    float l;             // this lane's share of the running sum
    float r[D / GS];     // per group: power of two that brings the unit's V scales into [0, 2)
};

// Compute one step (kI8Tiles tiles starting at ts) from loaded registers;
// FULL: every token of the step lies before t_end (no masking).
template <int D, int BS, int GS, bool FULL>
__device__ __forceinline__ void compute_step(const StepRegs<D, D / GS> &R,
                                             UnitState<D, BS, GS> &st, const uint4 (&qf)[D / 32],
                                             float qmul, int ts, int t_end, int lane)
{
    using S = I8Shape<D, BS, GS>;
    constexpr int NG = S::NG;
    const int j = lane >> 4;
    float s[kI8Tiles][4];
#pragma unroll
    for (int tile = 0; tile < kI8Tiles; ++tile) {
        float4_t acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            acc[g] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = g * S::SLABS_PER_GROUP; c < (g + 1) * S::SLABS_PER_GROUP; ++c) {
                const uint4 &w = R.k[tile][c / 2];
                const uint2 lo = codes_to_f16(c % 2 ? w.z : w.x);
                const uint2 hi = codes_to_f16(c % 2 ? w.w : w.y);
                acc[g] = mma_qk(TF16{}, make_uint4(lo.x, lo.y, hi.x, hi.y), qf[c], acc[g]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = acc[0][i] * scale_of<NG>(R.ks[tile], i, 0);
#pragma unroll
            for (int g = 1; g < NG; ++g)
                x = fmaf(acc[g][i], scale_of<NG>(R.ks[tile], i, g), x);
            const bool valid = FULL || ts + 16 * tile + 4 * j + i < t_end;
            s[tile][i] = valid ? x * qmul : -INFINITY;
        }
    }
    // Lazy online softmax: a head's reference max moves only when a logit
    // exceeds it by more than 8 (log2 units), so p <= 2^8; sum and O always
    // share one reference, so the result is exact.  Moves are rare after
    // the first step, and the rescale is skipped by the whole wave then.
    float mx = s[0][0];
#pragma unroll
    for (int tile = 0; tile < kI8Tiles; ++tile)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mx = fmaxf(mx, s[tile][i]);
    mx = column_max(mx);
    const bool move = mx > st.m + 8.0f;
    if (__builtin_amdgcn_ballot_w64(move)) {
        const float m_new = move ? mx : st.m;
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
        st.m = m_new;
        st.l *= alpha;
#pragma unroll
        for (int m = 0; m < S::DB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st.o[m][i] *= alpha;
    }
    uint2 pp[kI8Tiles][NG];
#pragma unroll
    for (int tile = 0; tile < kI8Tiles; ++tile) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(s[tile][i] - st.m);
            st.l += p[i];
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = FULL || ts + 16 * tile + 4 * j + i < t_end;
                w[i] = valid ? p[i] * (scale_of<NG>(R.vs[tile], i, g) * st.r[g]) : 0.0f;
            }
            pp[tile][g] = make_uint2(pack_f16(w[0], w[1]), pack_f16(w[2], w[3]));
        }
    }
#pragma unroll
    for (int m = 0; m < S::DB; ++m) {
        const int g = (16 * m) / GS;
#pragma unroll
        for (int tile = 0; tile < kI8Tiles; ++tile)
            st.o[m] = mma_pv(TF16{}, codes_to_f16(u4(R.v[tile][m / 4], m % 4)), pp[tile][g],
                             st.o[m]);
    }
}

// q operand of the score MFMAs for head lane%16 (zero past G) as fp16, and
// the multiplier that turns the MFMA result into log2-unit scores.
template <class QT, int D, int G>
__device__ __forceinline__ float load_query(const Int8DecodeArgs &a, int b, int h, int lane,
                                            uint4 (&qf)[D / 32])
{
    const int n = lane & 15, j = lane >> 4;
    const bool live = n < G;
    const int hq = h * G + (live ? n : 0);
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((int64_t)b * a.num_q_heads + hq) * D + 8 * j;
    uint4 raw[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        raw[c] = *reinterpret_cast<const uint4 *>(qp + 32 * c);
        if (!live)
            raw[c] = make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (std::is_same<QT, TF16>::value) {
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
            qf[c] = raw[c];
        return a.scale_log2;
    } else {
        // bf16: widen, bring the head's largest magnitude into [1, 2) by a
        // power of two (exact), round to fp16
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                amax = fmaxf(amax, fabsf(as_f(w[k] << 16)));
                amax = fmaxf(amax, fabsf(as_f(w[k] & 0xffff0000u)));
            }
        }
        amax = column_max(amax);
        float r, inv_r;
        pow2_normaliser(amax, r, inv_r);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = pack_f16(as_f(w[k] << 16) * r, as_f(w[k] & 0xffff0000u) * r);
            qf[c] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        return a.scale_log2 * inv_r;
    }
}

__device__ __forceinline__ int clamped_len(const Int8DecodeArgs &a, int b)
{
    int L = a.context_lens[b];
    const int cap = a.len_cap;
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Put a token's codes and scales, as quantise_store_row produced them
// (k_pk / v_pk: each lane's packed codes, k_s / v_s: its group's scales),
// into a loaded step's registers at step position rel, where the loads may
// have found the pool before or after that row's store.  The layouts are
// the operand orders of load_step: K byte 8s + i of lane 16p + row holds
// dim 32s + 8p + i; V byte 4m + row % 4 of lane 16 (row / 4) + c holds dim
// c + 16m; scales of tokens 4j..4j+3 sit in the lanes 16j..16j+15.
template <int D, int GS>
__device__ __forceinline__ void patch_new_token(StepRegs<D, D / GS> &R, int rel, uint32_t k_pk,
                                                uint32_t v_pk, float k_s, float v_s, int lane)
{
    constexpr int E = D / kWave;
    constexpr int NG = D / GS;
    const int tile_of = rel / 16, row = rel % 16;
    // dword of dims 4c..4c+3 in the lane holding dim 4c
    uint32_t w;
    if constexpr (E == 1)
        w = k_pk | (__shfl_down(k_pk, 1) << 8) | (__shfl_down(k_pk, 2) << 16) |
            (__shfl_down(k_pk, 3) << 24);
    else
        w = k_pk | (__shfl_down(k_pk, 2 / E) << 16);
    const bool k_lane = (lane & 15) == row;
    const bool q_lane = (lane >> 4) == row / 4;  // V codes and the scales
    const int p = lane >> 4, c = lane & 15, sh = 8 * (row % 4);
    uint32_t kd[D / 16], vd[D / 16];  // the lane's new dwords, in load order
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            kd[2 * s + hh] = __shfl(w, (32 * s + 8 * p + 4 * hh) / E);
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
        vd[m] = (__shfl(v_pk, (c + 16 * m) / E) >> (8 * (c % E))) & 0xffu;
    float ksn[NG], vsn[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        ksn[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, k_s),
                                                                      g * GS / E));
        vsn[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v_s),
                                                                      g * GS / E));
    }
#pragma unroll
    for (int t = 0; t < kI8Tiles; ++t) {
        if (t != tile_of)
            continue;
#pragma unroll
        for (int q = 0; q < D / 64; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t kv = u4(R.k[t][q], e), vv = u4(R.v[t][q], e);
                set_u4(R.k[t][q], e, k_lane ? kd[4 * q + e] : kv);
                set_u4(R.v[t][q], e,
                       q_lane ? ((vv & ~(0xffu << sh)) | (vd[4 * q + e] << sh)) : vv);
            }
#pragma unroll
        for (int f = 0; f < NG; ++f)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int flat = 4 * f + e;  // token flat / NG of the quad, group flat % NG
                const bool hit = q_lane && flat / NG == row % 4;
                set_f4(R.ks[t][f], e, hit ? ksn[flat % NG] : f4(R.ks[t][f], e));
                set_f4(R.vs[t][f], e, hit ? vsn[flat % NG] : f4(R.vs[t][f], e));
            }
    }
}

// Tokens [jp * P, min((jp+1) * P, L)) of sequence b, kv head h; APPEND:
// the new token's row is quantised and stored (a plain decode compiles
// without it).
// A partial result (L > P) goes to the workspace rows, or with lds_o set to
// LDS: o / l at lds_o[n * D + d] and (max, sum) at lds_ml[n] for head n < G.
template <class QT, int D, int BS, int G, int GS, bool APPEND>
__device__ __forceinline__ void run_unit(const Int8DecodeArgs &a, int b, int jp, int h, int L,
                                         int lane, float *lds_o = nullptr,
                                         float2 *lds_ml = nullptr)
{
    const int P = a.partition_size;
    const int t_begin = jp * P;
    const int t_end = min(t_begin + P, L);
    // Fused append: the unit that holds position L - 1 quantises the
    // sequence's new K/V rows of this kv head and stores them at their slot.
    // Its V-scale pass and its last step take the new codes and scales from
    // the registers, the values a decode after the write would read, so
    // nothing waits for the stores.  The rows are loaded together with the
    // unit's other first loads.
    constexpr int E = D / kWave;
    const bool appending = APPEND && jp == (L - 1) / P;
    int64_t slot = -1;
    float xk[E], xv[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        xk[e] = xv[e] = 0.0f;
    if (appending) {
        slot = a.slot_mapping[b];
        load_row<QT, D>(a.k_new, (int64_t)b * a.k_new_stride + (int64_t)h * D, lane, xk);
        load_row<QT, D>(a.v_new, (int64_t)b * a.v_new_stride + (int64_t)h * D, lane, xv);
    }
    // the partition's block ids, one per lane (clamped into the table row
    // and into the pool, so every access stays in bounds)
    const int nb = (t_end - t_begin + BS - 1) / BS;
    const int col = t_begin / BS + (lane < nb ? lane : nb - 1);
    int ids = a.block_tables[(int64_t)b * a.max_blocks_per_seq + col];
    ids = ids < 0 ? 0 : (ids >= a.num_blocks ? a.num_blocks - 1 : ids);

    uint4 qf[D / 32];
    const float qmul = load_query<QT, D, G>(a, b, h, lane, qf);

    UnitState<D, BS, GS> st;
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
        st.o[m] = float4_t{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.0f;
    const bool stored = appending && slot >= 0 && slot < (int64_t)a.num_blocks * BS;
    // The new token is position L - 1 only when its length was not cut short
    // (a host hint below the real length): only then do the registers take
    // it; otherwise the row is stored and positions 0 .. L - 1 come from the
    // pool, as in a write followed by a decode.
    const bool patched = stored && a.context_lens[b] == L;
    int8_t ck[E], cv[E];
    float new_ks = 0.0f, new_vs = 0.0f;  // this lane's group's scales of the new rows
    if (stored) {
        new_ks = quantise_row<D, GS>(xk, ck);
        new_vs = quantise_row<D, GS>(xv, cv);
    }
    // The unit's V-scale normalisers: lane l reads the scales of the
    // partition's block l (tokens past t_end masked), a wave max per group.
    {
        constexpr int NG = D / GS;
        float sig[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            sig[g] = 0.0f;
        if (lane < nb) {
            const float4 *vsp = reinterpret_cast<const float4 *>(
                a.v_scales + ((int64_t)ids * a.num_kv_heads + h) * BS * NG);
            const int t0 = t_begin + lane * BS;
#pragma unroll
            for (int k4 = 0; k4 < BS * NG / 4; ++k4) {
                const float4 v = vsp[k4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int flat = 4 * k4 + e;
                    // position L - 1 of an appending unit: its new scale below
                    const bool valid = t0 + flat / NG < (patched ? t_end - 1 : t_end);
                    sig[flat % NG] = fmaxf(sig[flat % NG], valid ? f4(v, e) : 0.0f);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float m = wave_max(sig[g]);
            if (patched)  // the lanes of group g hold its scale: lane g * GS / (D / 64)
                m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                           __builtin_bit_cast(int, new_vs),
                                                           g * GS / (D / kWave))));
            float inv_r;
            pow2_normaliser(m, st.r[g], inv_r);
        }
    }
    uint32_t new_kc = 0, new_vc = 0;  // this lane's codes of the new rows
    if (stored) {
        const int64_t blk = slot / BS;
        const int off = (int)(slot % BS);
        store_row<D, GS>(ck, new_ks, false, const_cast<int8_t *>(a.k_codes),
                         const_cast<float *>(a.k_scales), a.num_kv_heads, BS, blk, h, off, lane);
        store_row<D, GS>(cv, new_vs, true, const_cast<int8_t *>(a.v_codes),
                         const_cast<float *>(a.v_scales), a.num_kv_heads, BS, blk, h, off, lane);
        new_kc = pack_codes<E>(ck);
        new_vc = pack_codes<E>(cv);
    }

    // the step starting at ts holds position L - 1: its registers get the
    // new token
    auto patch = [&](StepRegs<D, D / GS> &R, int ts) __attribute__((always_inline)) {
        if (patched && ts <= L - 1 && L - 1 < ts + kI8Step)
            patch_new_token<D, GS>(R, L - 1 - ts, new_kc, new_vc, new_ks, new_vs, lane);
    };
    // One step in flight per wave; the waves resident on a compute unit
    // overlap each other's loads and arithmetic.
    StepRegs<D, D / GS> A;
    int ts = t_begin;
    for (; ts + kI8Step <= t_end; ts += kI8Step) {
        load_step<D, BS, GS>(a, A, ids, t_begin, ts, t_end, h, lane);
        patch(A, ts);
        compute_step<D, BS, GS, true>(A, st, qf, qmul, ts, t_end, lane);
    }
    if (ts < t_end) {
        load_step<D, BS, GS>(a, A, ids, t_begin, ts, t_end, h, lane);
        patch(A, ts);
        compute_step<D, BS, GS, false>(A, st, qf, qmul, ts, t_end, lane);
    }

    const float l = column_sum(st.l);
    const int n = lane & 15, j = lane >> 4;
    if (n >= G)
        return;
    const int hq = h * G + n;
    // O was accumulated times r of its group (a power of two): undo it
    // exactly together with the division by the sum
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        const float u = 1.0f / st.r[(16 * m) / GS];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st.o[m][i] *= u;
    }
    const float inv_l = 1.0f / l;
    if (lds_o != nullptr && L > P) {
        float *o = lds_o + n * D + 4 * j;
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
            *reinterpret_cast<float4 *>(o + 16 * m) =
                make_float4(st.o[m][0] * inv_l, st.o[m][1] * inv_l, st.o[m][2] * inv_l,
                            st.o[m][3] * inv_l);
        if (j == 0)
            lds_ml[n] = make_float2(st.m, l);
    } else if (a.num_partitions == 1 || L <= P) {
        const int64_t base = ((int64_t)b * a.num_q_heads + hq) * D + 4 * j;
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store_out(a.out, base + 16 * m + i, st.o[m][i] * inv_l, a.out_kind);
    } else {
        const int64_t row = ((int64_t)b * a.num_q_heads + hq) * a.num_partitions + jp;
        float *o = a.ws_o + row * D + 4 * j;
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
            *reinterpret_cast<float4 *>(o + 16 * m) =
                make_float4(st.o[m][0] * inv_l, st.o[m][1] * inv_l, st.o[m][2] * inv_l,
                            st.o[m][3] * inv_l);
        if (j == 0)
            *reinterpret_cast<float2 *>(a.ws_ml + 2 * row) = make_float2(st.m, l);
    }
}

__device__ __forceinline__ void store_zero_rows(const Int8DecodeArgs &a, int b, int h, int G,
                                                int D, int lane)
{
    for (int e = lane; e < G * D; e += kWave)
        store_out(a.out, ((int64_t)b * a.num_q_heads + h * G) * D + e, 0.0f, a.out_kind);
}

// Exclusive prefix of the sequences' partition counts, prefix[b] = sum over
// b' < b of ceil(L_b' / P), b = 0..B, in LDS; every thread of the workgroup
// (NT of them) takes part.  wsum: NT / 64 ints of LDS.
template <int NT>
__device__ __forceinline__ void build_prefix(const Int8DecodeArgs &a, int *prefix, int *wsum)
{
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    int base = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += NT) {
        const int b = b0 + t;
        const int n = b < a.num_seqs ? (clamped_len(a, b) + a.partition_size - 1) / a.partition_size
                                     : 0;
        int x = n;  // inclusive scan within the wave, then across waves
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(x, d, kWave);
            if (lane >= d)
                x += y;
        }
        if (lane == kWave - 1)
            wsum[wave] = x;
        __syncthreads();
        int before = base;
        for (int w = 0; w < wave; ++w)
            before += wsum[w];
        if (b < a.num_seqs)
            prefix[b] = before + x - n;
        int total = base;
        for (int w = 0; w < NT / kWave; ++w)
            total += wsum[w];
        __syncthreads();
        base = total;
    }
    if (t == 0)
        prefix[a.num_seqs] = base;
    __syncthreads();
}

// One workgroup (batches of more than kI8PlanInKernelSeqs sequences): items
// (b, jp) for jp < ceil(L_b / P), sequences in order, written to a.items;
// their count to a.wl_header[0].
__global__ __launch_bounds__(kI8PlanThreads) void int8_plan_kernel(Int8DecodeArgs a)
{
    __shared__ int wsum[kI8PlanThreads / kWave];
    __shared__ int chunk[kI8PlanThreads + 1];
    const int t = threadIdx.x;
    int base = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += kI8PlanThreads) {
        const int cnt = min(kI8PlanThreads, a.num_seqs - b0);
        Int8DecodeArgs sub = a;
        sub.num_seqs = cnt;
        sub.context_lens = a.context_lens + b0;
        build_prefix<kI8PlanThreads>(sub, chunk, wsum);
        if (t < cnt) {
            const int start = base + chunk[t];
            const int n = chunk[t + 1] - chunk[t];
            for (int k = 0; k < n; ++k)
                a.items[start + k] = make_int2(b0 + t, k);
        }
        base += chunk[cnt];
        __syncthreads();
    }
    if (t == 0)
        a.wl_header[0] = base;
}

// MODE 0, dense (at most kI8DenseMaxPartitions partitions per sequence):
// wave u handles unit (b, jp, h), u = (b * NP + jp) * Hkv + h, and exits at
// once when partition jp starts past the sequence's end.  MODE 1 and 2, a
// persistent grid: the items (b, jp), crossed with the kv heads, are dealt
// round-robin to all waves of the grid; MODE 1 reads them from the list a
// planning launch wrote, MODE 2 (at most kI8PlanInKernelSeqs sequences)
// finds them in a prefix of partition counts each workgroup builds in LDS.
// MODE 3 (2..kI8DenseMaxPartitions partitions): workgroup (b, h) of
// num_partitions waves, wave w on partition w; the workgroup merges the
// partitions' rows in LDS with the exact log-sum-exp weights.
template <class QT, int D, int BS, int G, int GS, int MODE, bool APPEND>
__global__ __launch_bounds__(MODE == 3 ? kI8DenseMaxPartitions * kWave : kI8Waves * kWave)
void int8_decode_kernel(Int8DecodeArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t w0 = (int64_t)blockIdx.x * kI8Waves + wave;
    if constexpr (MODE == 0) {
        const int64_t per_seq = (int64_t)a.num_partitions * a.num_kv_heads;
        if (w0 >= (int64_t)a.num_seqs * per_seq)
            return;
        const int b = (int)(w0 / per_seq);
        const int jp = (int)(w0 % per_seq / a.num_kv_heads);
        const int h = (int)(w0 % a.num_kv_heads);
        const int L = clamped_len(a, b);
        if (L == 0) {
            if (jp == 0)
                store_zero_rows(a, b, h, G, D, lane);
            return;
        }
        if (jp * a.partition_size >= L)
            return;
        run_unit<QT, D, BS, G, GS, APPEND>(a, b, jp, h, L, lane);
    } else if constexpr (MODE == 3) {
        extern __shared__ int i8_lds[];
        const int nw = a.num_partitions;  // waves of the workgroup
        const int b = (int)(blockIdx.x / a.num_kv_heads);
        const int h = (int)(blockIdx.x % a.num_kv_heads);
        const int L = clamped_len(a, b);
        if (L == 0) {  // the whole workgroup leaves
            if (wave == 0)
                store_zero_rows(a, b, h, G, D, lane);
            return;
        }
        float *lo = reinterpret_cast<float *>(i8_lds);               // [nw][G][D]
        float2 *lml = reinterpret_cast<float2 *>(lo + nw * G * D);  // [nw][G]
        const int P = a.partition_size;
        if (wave * P < L)
            run_unit<QT, D, BS, G, GS, APPEND>(a, b, wave, h, L, lane, lo + wave * G * D,
                                               lml + wave * G);
        const int np = (L + P - 1) / P;
        if (np <= 1)  // written by wave 0; the same for every wave
            return;
        __syncthreads();
        for (int e = threadIdx.x; e < G * D; e += nw * kWave) {
            const int n = e / D, d = e % D;
            float M = -INFINITY;
            for (int w = 0; w < np; ++w)
                M = fmaxf(M, lml[w * G + n].x);
            float acc = 0.0f, den = 0.0f;
            for (int w = 0; w < np; ++w) {
                const float2 ml = lml[w * G + n];
                const float wk = ml.y * __builtin_amdgcn_exp2f(ml.x - M);
                acc = fmaf(wk, lo[(w * G + n) * D + d], acc);
                den += wk;
            }
            store_out(a.out, ((int64_t)b * a.num_q_heads + h * G + n) * D + d,
                      acc * (1.0f / den), a.out_kind);
        }
    } else if constexpr (MODE == 1) {
        const int64_t units = (int64_t)__builtin_amdgcn_readfirstlane(a.wl_header[0]) *
                              a.num_kv_heads;
        const int64_t stride = (int64_t)gridDim.x * kI8Waves;
        for (int64_t u = w0; u < units; u += stride) {
            const int2 it = a.items[u / a.num_kv_heads];
            const int b = __builtin_amdgcn_readfirstlane(it.x);
            const int jp = __builtin_amdgcn_readfirstlane(it.y);
            const int h = (int)(u % a.num_kv_heads);
            run_unit<QT, D, BS, G, GS, APPEND>(a, b, jp, h, clamped_len(a, b), lane);
        }
    } else {
        extern __shared__ int i8_lds[];
        int *wsum = i8_lds;                      // [kI8Waves]
        int *prefix = i8_lds + kI8Waves;         // [B + 1]
        build_prefix<kI8Waves * kWave>(a, prefix, wsum);
        const int64_t units = (int64_t)prefix[a.num_seqs] * a.num_kv_heads;
        const int64_t stride = (int64_t)gridDim.x * kI8Waves;
        for (int64_t u = w0; u < units; u += stride) {
            const int item = (int)(u / a.num_kv_heads);
            int lo = 0, hi = a.num_seqs;  // the last b with prefix[b] <= item
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (prefix[mid] <= item)
                    lo = mid;
                else
                    hi = mid;
            }
            const int b = __builtin_amdgcn_readfirstlane(lo);
            const int jp = __builtin_amdgcn_readfirstlane(item - prefix[lo]);
            const int h = (int)(u % a.num_kv_heads);
            run_unit<QT, D, BS, G, GS, APPEND>(a, b, jp, h, clamped_len(a, b), lane);
        }
    }
}

// acc[e] += sum_{k < cnt} w_k o[k * stride + e], w_k held by lane k: the
// loads of all N rows are issued before the first is used (rows past cnt
// repeat the last one and get weight 0).
template <int N, int E>
__device__ __forceinline__ void accumulate_rows(const float *o, int stride, int cnt, float w,
                                                float (&acc)[E])
{
    float v[N][E];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int kk = k < cnt ? k : cnt - 1;
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[k][e] = o[(int64_t)kk * stride + e];
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float wk = k < cnt ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                 __builtin_bit_cast(int, w), k))
                                 : 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] = fmaf(wk, v[k][e], acc[e]);
    }
}

// out[b][hq] from the partition rows of sequence b: exact log-sum-exp
// merge; zero rows for L_b = 0; nothing for one partition (written by the
// decode).  One wave per (b, hq) row, kI8Waves rows per workgroup: lane k
// takes partition k of a batch of 64 (its max, sum and weight), and every
// lane accumulates its D / 64 dims over the batch with the weights read
// from the lanes; batches merge with a running maximum.
template <int D>
__global__ __launch_bounds__(kI8Waves *kWave) void int8_merge_kernel(Int8DecodeArgs a)
{
    constexpr int E = D / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t r = (int64_t)blockIdx.x * kI8Waves + threadIdx.x / kWave;
    if (r >= (int64_t)a.num_seqs * a.num_q_heads)
        return;
    const int b = (int)(r / a.num_q_heads);
    const int L = clamped_len(a, b);
    const int n = (L + a.partition_size - 1) / a.partition_size;
    if (L == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            store_out(a.out, r * D + lane * E + e, 0.0f, a.out_kind);
        return;
    }
    if (n <= 1)
        return;
    const int64_t row0 = r * a.num_partitions;
    float M = -INFINITY, den = 0.0f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.0f;
    for (int base = 0; base < n; base += kWave) {
        const int cnt = min(kWave, n - base);
        float2 ml = make_float2(-INFINITY, 0.0f);
        if (lane < cnt)
            ml = *reinterpret_cast<const float2 *>(a.ws_ml + 2 * (row0 + base + lane));
        const float Mn = fmaxf(M, wave_max(ml.x));
        const float alpha = __builtin_amdgcn_exp2f(M - Mn);
        M = Mn;
        const float w = lane < cnt ? ml.y * __builtin_amdgcn_exp2f(ml.x - M) : 0.0f;
        float wsum = w;
        wsum += dpp<0xB1>(wsum);
        wsum += dpp<0x4E>(wsum);
        wsum += dpp<0x141>(wsum);
        wsum += dpp<0x140>(wsum);
        wsum += swz_xor16(wsum);
        wsum += xor32(wsum);
        den = den * alpha + wsum;
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] *= alpha;
        const float *o = a.ws_o + (row0 + base) * D + lane * E;
        if (cnt <= 8)
            accumulate_rows<8, E>(o, D, cnt, w, acc);
        else if (cnt <= 16)
            accumulate_rows<16, E>(o, D, cnt, w, acc);
        else if (cnt <= 32)
            accumulate_rows<32, E>(o, D, cnt, w, acc);
        else
            accumulate_rows<kWave, E>(o, D, cnt, w, acc);
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int e = 0; e < E; ++e)
        store_out(a.out, r * D + lane * E + e, acc[e] * inv, a.out_kind);
}

int compute_units()
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

template <class QT, int D, int BS, int G, int GS, bool APPEND>
hipError_t launch_decode_t(const Int8DecodeArgs &a, hipStream_t stream)
{
    if (a.num_partitions > 1 && a.num_partitions <= kI8DenseMaxPartitions) {
        const int64_t groups = (int64_t)a.num_seqs * a.num_kv_heads;
        if (groups > 0x7fffffff)
            return hipErrorInvalidValue;
        const size_t lds = (size_t)a.num_partitions * G * (D * 4 + 8);
        hipLaunchKernelGGL((int8_decode_kernel<QT, D, BS, G, GS, 3, APPEND>),
                           dim3((unsigned)groups), dim3(a.num_partitions * kWave), lds, stream, a);
        return hipGetLastError();  // merged in the launch
    }
    if (a.num_partitions <= kI8DenseMaxPartitions) {
        const int64_t waves = (int64_t)a.num_seqs * a.num_partitions * a.num_kv_heads;
        const int64_t grid = (waves + kI8Waves - 1) / kI8Waves;
        hipLaunchKernelGGL((int8_decode_kernel<QT, D, BS, G, GS, 0, APPEND>), dim3((unsigned)grid),
                           dim3(kI8Waves * kWave), 0, stream, a);
    } else {
        const bool in_kernel = a.num_seqs <= kI8PlanInKernelSeqs;
        const size_t lds = in_kernel ? (size_t)(kI8Waves + a.num_seqs + 1) * 4 : 0;
        if (!in_kernel)
            hipLaunchKernelGGL(int8_plan_kernel, dim3(1), dim3(kI8PlanThreads), 0, stream, a);
        static int per_cu_cache[64][2];  // per device and plan kind, per instantiation
        int dev = 0;
        (void)hipGetDevice(&dev);
        const int kind = in_kernel ? 1 : 0;
        int per_cu = dev >= 0 && dev < 64 ? per_cu_cache[dev][kind] : 0;
        if (per_cu == 0) {
            // the largest in-kernel plan (kI8PlanInKernelSeqs sequences) sizes
            // the cached figure, so it holds for every smaller batch
            if (in_kernel)
                (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &per_cu, int8_decode_kernel<QT, D, BS, G, GS, 2, APPEND>, kI8Waves * kWave,
                    (size_t)(kI8Waves + kI8PlanInKernelSeqs + 1) * 4);
            else
                (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &per_cu, int8_decode_kernel<QT, D, BS, G, GS, 1, APPEND>, kI8Waves * kWave, 0);
            per_cu = per_cu > 0 ? per_cu : 1;
            if (dev >= 0 && dev < 64)
                per_cu_cache[dev][kind] = per_cu;
        }
        const int64_t max_units = (int64_t)a.num_seqs * a.num_partitions * a.num_kv_heads;
        int64_t grid = (int64_t)compute_units() * per_cu;
        const int64_t need = (max_units + kI8Waves - 1) / kI8Waves;
        grid = grid < need ? grid : need;
        if (in_kernel)
            hipLaunchKernelGGL((int8_decode_kernel<QT, D, BS, G, GS, 2, APPEND>), dim3((unsigned)grid),
                               dim3(kI8Waves * kWave), lds, stream, a);
        else
            hipLaunchKernelGGL((int8_decode_kernel<QT, D, BS, G, GS, 1, APPEND>), dim3((unsigned)grid),
                               dim3(kI8Waves * kWave), 0, stream, a);
    }
    if (a.num_partitions > 1) {
        const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
        hipLaunchKernelGGL(int8_merge_kernel<D>, dim3((unsigned)((rows + kI8Waves - 1) / kI8Waves)),
                           dim3(kI8Waves * kWave), 0, stream, a);
    }
    return hipGetLastError();
}

template <class QT, int D, int BS, int G>
hipError_t dispatch_gs(const Int8DecodeArgs &a, hipStream_t s)
{
    switch (a.group_size) {
    case 32:
        return a.k_new ? launch_decode_t<QT, D, BS, G, 32, true>(a, s)
                       : launch_decode_t<QT, D, BS, G, 32, false>(a, s);
    case 64:
        return a.k_new ? launch_decode_t<QT, D, BS, G, 64, true>(a, s)
                       : launch_decode_t<QT, D, BS, G, 64, false>(a, s);
    case 128:
        if constexpr (D >= 128)
            return a.k_new ? launch_decode_t<QT, D, BS, G, 128, true>(a, s)
                           : launch_decode_t<QT, D, BS, G, 128, false>(a, s);
        break;
    }
    return hipErrorInvalidValue;
}

template <class QT, int D, int BS>
hipError_t dispatch_g(const Int8DecodeArgs &a, hipStream_t s)
{
    switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return dispatch_gs<QT, D, BS, 1>(a, s);
    case 2: return dispatch_gs<QT, D, BS, 2>(a, s);
    case 4: return dispatch_gs<QT, D, BS, 4>(a, s);
    case 8: return dispatch_gs<QT, D, BS, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

template <class QT, int D>
hipError_t dispatch_bs(const Int8DecodeArgs &a, hipStream_t s)
{
    return a.block_size == 16 ? dispatch_g<QT, D, 16>(a, s) : dispatch_g<QT, D, 32>(a, s);
}

template <class QT>
hipError_t dispatch_d(const Int8DecodeArgs &a, hipStream_t s)
{
    return a.head_dim == 64 ? dispatch_bs<QT, 64>(a, s) : dispatch_bs<QT, 128>(a, s);
}

template <class T, int D>
hipError_t launch_write_t(const Int8WriteArgs &a, hipStream_t stream)
{
    const int64_t waves = 2 * (int64_t)a.num_tokens * a.num_kv_heads;
    const int64_t grid = (waves + 3) / 4;
    switch (a.group_size) {
    case 32:
        hipLaunchKernelGGL((quantize_write_kernel<T, D, 32>), dim3((unsigned)grid), dim3(256), 0,
                           stream, a);
        break;
    case 64:
        hipLaunchKernelGGL((quantize_write_kernel<T, D, 64>), dim3((unsigned)grid), dim3(256), 0,
                           stream, a);
        break;
    default:
        if constexpr (D >= 128) {
            hipLaunchKernelGGL((quantize_write_kernel<T, D, 128>), dim3((unsigned)grid), dim3(256),
                               0, stream, a);
            break;
        }
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class T>
hipError_t launch_write_d(const Int8WriteArgs &a, hipStream_t s)
{
    return a.head_dim == 64 ? launch_write_t<T, 64>(a, s) : launch_write_t<T, 128>(a, s);
}

}  // namespace

hipError_t launch_kv_cache_write_int8(const Int8WriteArgs &a, hipStream_t stream)
{
    if (a.num_tokens == 0)
        return hipSuccess;
    if ((int64_t)a.num_tokens * a.num_kv_heads * 2 > (int64_t)4 * 0x7fffffff)
        return hipErrorInvalidValue;
    switch (a.dtype) {
    case DType::F32: return launch_write_d<TF32>(a, stream);
    case DType::F16: return launch_write_d<TF16>(a, stream);
    case DType::BF16: return launch_write_d<TBF16>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_int8(const Int8DecodeArgs &a, hipStream_t stream)
{
    if (a.num_seqs == 0)
        return hipSuccess;
    return a.q_dtype == DType::F16 ? dispatch_d<TF16>(a, stream) : dispatch_d<TBF16>(a, stream);
}

}  // namespace pka
