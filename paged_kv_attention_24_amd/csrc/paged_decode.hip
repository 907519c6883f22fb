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
//  * Work space.  The tokens of every (sequence b, kv head h) pair are cut
//    into chunks of CT tokens.  Every chunk costs kUnitsPerChunk work units
//    and every pair with tokens kUnitsPerPair more (its fixed cost: block
//    ids, q, first request, result); the pairs' units, in (b, h) order,
//    form one flat index space of U units, cut into N equal ranges, one per
//    active wave.  A chunk belongs to the wave whose range holds its
//    anchor, so every wave streams about the same bytes and pays about the
//    same fixed costs whatever the mix of lengths (no tail of long
//    sequences).  All G = Hq/Hkv query heads of a pair are served by the
//    same K/V reads, so every KV byte is read from HBM once.
//  * Pair mode, for small batches (pairs at most one per compute unit,
//    every sequence at most kPairModeMaxTokens long): one workgroup of
//    kPairWaves waves per pair, the waves taking contiguous runs of its
//    chunks and combining their parts through LDS; no workspace.
//  * Planning happens in the kernel: each workgroup scans the lengths into
//    a prefix of work units in LDS (one barrier); each wave then finds the
//    pair its range starts in with two ballots over that prefix.
//  * Segments.  A wave's range is a run of segments, one per pair it
//    touches: whole pairs in the middle, possibly part of a pair at either
//    end.  A whole pair's result is normalised and stored; a part stores
//    (max, sum, unnormalised O) to the workspace with coherent stores, and
//    the last wave to report on that pair (a counter per pair, one per
//    128-byte line) combines its parts by log-sum-exp, stores the result
//    and clears the counter.
//  * Data path of a wave: its chunks of K and V go straight from HBM into
//    the wave's own LDS area (global_load_lds, XOR-swizzled rows), one chunk
//    ahead of the one computed; the next segment's first chunk, query rows
//    and appended row (also DMA'd into LDS) are requested while the current
//    segment's last chunk is computed, so the stream runs on across segment
//    boundaries.  Per 16-token tile, matrix-core products give the scores
//    of all G heads (K tile times q^T); the online softmax runs in the
//    registers the product wrote; a second product accumulates
//    O^T += V^T P^T, V^T coming from the transposing LDS read (fp16/bf16)
//    or from column reads (fp32); for fp16 one more product with an
//    all-ones V^T gives the softmax sums.
//  * Fused append: for pka_paged_attention_decode_append the wave that
//    holds position L_b - 1 stores the sequence's new K/V row in its slot
//    and takes that position's K/V from the row's LDS copy, so nothing waits
//    for the store.
//  * Tokens >= L (the tail of the last block) are excluded by selects, never
//    by multiplying with 0, so stale or NaN slot contents cannot leak.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "cdna4.h"
#include "pka_internal.h"

namespace pka {
namespace {

constexpr int kWaves = 4;  // waves per workgroup (each wave works alone after planning)
// Pair mode (small batches): one workgroup of kPairWaves waves per (sequence,
// kv head) pair, the waves splitting its chunks and combining in LDS.  Used
// while pairs fit one per compute unit and sequences are at most
// kPairModeMaxTokens long (a longer pair would keep one compute unit busy
// while the others idle).
constexpr int kPairWaves = 8;
constexpr int64_t kPairModeMaxTokens = 2048;
constexpr size_t kPairModeMaxLds = 160 * 1024;

struct DecodeParams {
    void *out;
    int out_kind;  // 0 f32, 1 f16, 2 bf16
    const char *q, *k_cache, *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
    int32_t num_seqs, num_q_heads, num_kv_heads, num_blocks;
    float scale_log2;     // scale * log2(e)
    int32_t len_cap;      // lengths are clamped to [0, len_cap]
    int32_t min_chunks;   // an active wave takes at least this many chunks
    float *parts;         // [2 * grid waves] partial results of decode_part_floats(G, D)
    int32_t *counters;    // [num_seqs][num_kv_heads] reports per split pair, kCounterStride apart; zero between calls
    // appended token per sequence (k_new null: plain decode)
    const char *k_new, *v_new;
    int64_t k_new_stride, v_new_stride;  // bytes between sequences
    const int64_t *slots;
    char *k_store, *v_store;             // the pools, written at slots[b]
    int64_t num_slots;
};

template <class T, int D, int BS, int G>
struct Shape {
    static constexpr int ELT = T::kBytes;
    static constexpr bool F32 = std::is_same<T, TF32>::value;
    static constexpr int R = D * ELT;              // bytes per token row
    static constexpr int LPR = R / 16;             // lanes per token row (16-byte units)
    static constexpr int TPL = kWave / LPR;        // token rows per 1 KiB wave load
    static constexpr int NL = 16 * R / 1024 > 4 ? 16 * R / 1024 : 4;  // wave loads per chunk and tensor
    static constexpr int CT = NL * TPL;            // tokens per chunk
    static constexpr int TPC = CT / 16;            // 16-token tiles per chunk
    static constexpr int CHUNK = NL * 1024;        // bytes of one tensor's chunk
    static constexpr int QROWS = G * R;            // bytes of a pair's G query rows
    static constexpr int QA = (QROWS + 2 * R + 1023) / 1024 * 1024;  // q rows, new K row, new V row
    static constexpr int STAGE = 2 * 2 * CHUNK + QA;  // LDS per wave: 2 buffers of K and V, then QA
    static constexpr int TILE = BS * R;            // bytes of one (block, head) tile
    static constexpr int KS = D * ELT / 64;        // 16-byte steps of the score product
    static constexpr int MT = D / 16;              // 16-dim tiles of the output
    static constexpr int PART = (int)decode_part_floats(G, D);  // floats of one partial result
    static_assert(LPR >= 1 && LPR <= 32 && TPL * LPR == kWave, "row must fit a wave");
    static_assert(BS % TPL == 0, "a wave load must stay inside one block");
    static_assert(CT % 16 == 0 && (CT % BS == 0 || BS % CT == 0), "chunks hold whole tiles");
};

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

__device__ __forceinline__ int clamp_len(const DecodeParams &p, int L)
{
    return L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
}
// Length of sequence bb (wave-uniform bb), clamped, through the scalar cache.
__device__ __forceinline__ int seq_len_uniform(const DecodeParams &p, int bb)
{
    return clamp_len(p, scalar_load(p.context_lens, bb));
}

// prefix[i] = kv heads * (chunks of the sequences before sequence i), for
// i = 0..B, in LDS; every thread of the workgroup takes part (one barrier
// at the end).  wsum: kWaves ints of scratch.  The counts are work units:
// kUnitsPerChunk per chunk and kUnitsPerPair per (sequence, kv head) pair
// that has tokens.
template <int CT>
__device__ __forceinline__ void build_prefix(const DecodeParams &p, int *prefix, int *wsum)
{
    constexpr int NT = kWaves * kWave;
    const int B = p.num_seqs;
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int per = (B + NT - 1) / NT;
    const int b0 = threadIdx.x * per, b1 = min(b0 + per, B);
    auto chunks = [&](int bb) {
        const int L = clamp_len(p, p.context_lens[bb]);
        const int nch = (L + CT - 1) / CT;
        return nch > 0 ? (kUnitsPerChunk * nch + kUnitsPerPair) * p.num_kv_heads : 0;
    };
    // the first sequence's count stays in a register for the second pass
    // (the common case of one sequence per thread reads context_lens once)
    const int first = b0 < b1 ? chunks(b0) : 0;
    int local = first;
    for (int bb = b0 + 1; bb < b1; ++bb)
        local += chunks(bb);
    // inclusive scan within the wave by DPP: shifts inside each row of 16
    // lanes, then the two row broadcasts (a lane whose source lies outside
    // its row, or a row the mask leaves out, adds the 0 of `old`)
    int x = local;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
    if (lane == kWave - 1)
        wsum[wv] = x;
    __syncthreads();
    int run = x - local;
    for (int ww = 0; ww < wv; ++ww)
        run += wsum[ww];
    if (b0 < b1) {
        prefix[b0] = run;
        run += first;
    }
    for (int bb = b0 + 1; bb < b1; ++bb) {
        prefix[bb] = run;
        run += chunks(bb);
    }
    if (b0 < B && b1 == B)
        prefix[B] = run;
    if (B == 0 && threadIdx.x == 0)
        prefix[0] = 0;
    __syncthreads();
}

// Largest b in [0, B) with prefix[b] <= c (c < prefix[B]): a 64-way ballot
// step over the sequences, then the exact one.  Uniform result.
__device__ __forceinline__ int find_seq(const int *prefix, int B, int64_t c)
{
    const int lane = threadIdx.x % kWave;
    const int st = (B + kWave - 1) / kWave;
    const int s0 = lane * st < B ? lane * st : B;
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(lane * st < B && prefix[s0] <= c);
    const int base = (kWave - 1 - __builtin_clzll(m0)) * st;
    const int s1 = base + lane;
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(lane < st && s1 < B && prefix[s1] <= c);
    return __builtin_amdgcn_readfirstlane(base + (kWave - 1 - __builtin_clzll(m1)));
}

// floor(num / den) for 0 <= num < 2^52, 0 < den < 2^31: an fp64 quotient
// corrected to the exact integer (a few instructions instead of the long
// 64-bit integer division).
__device__ __forceinline__ int64_t floor_div(int64_t num, int64_t den)
{
    int64_t q = (int64_t)((double)num / (double)den);
    q -= q * den > num ? 1 : 0;
    q += (q + 1) * den <= num ? 1 : 0;
    return q;
}
// First chunk of wave `a` of n over c chunks: floor(a * c / n).
__device__ __forceinline__ int64_t range_start(int64_t a, int64_t c, int64_t n)
{
    return floor_div(a * c, n);
}
// The wave whose range holds chunk x: the largest a with range_start(a) <= x.
__device__ __forceinline__ int64_t wave_of(int64_t x, int64_t c, int64_t n)
{
    return floor_div((x + 1) * n - 1, c);
}

// One segment of a wave's range: chunks [k0, k1) of pair (b, h), whose
// sequence has L tokens (nch chunks); pu0 is the pair's first work unit.
struct Segment {
    int b, h, k0, k1, nch, L;
    int64_t pu0;
    bool first;  // the first segment of the wave's range
};

template <class T, int D, int BS, int G, bool PAIR>
__global__ __launch_bounds__((PAIR ? kPairWaves : kWaves) * kWave, PAIR ? 1 : 2)
void decode_kernel(DecodeParams p)
{
    using S = Shape<T, D, BS, G>;
    constexpr int R = S::R, LPR = S::LPR, TPL = S::TPL, NL = S::NL, CT = S::CT, TPC = S::TPC;
    constexpr int CHUNK = S::CHUNK, KS = S::KS, MT = S::MT;
    constexpr float kSlack = 8.0f;  // log2 units a logit may exceed the reference max by
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int lane = threadIdx.x % kWave;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tg = lane / LPR, cl = lane % LPR;
    const int n = lane % 16, quad = lane / 16;
    const bool head_ok = n < G;
    const int B = p.num_seqs, Hkv = p.num_kv_heads;

    // ---- plan: work-unit prefix over the sequences, then this wave's range --
    // The pairs' chunks are laid end to end, each pair led by kUnitsPerPair
    // units for its fixed cost; the U units are cut into N equal ranges,
    // and chunk k of a pair starting at unit s belongs to the wave whose
    // range holds its anchor s + kUnitsPerPair + kUnitsPerChunk * k.  N
    // keeps every range at least min_chunks chunks (and one chunk) long,
    // so every wave between the first and the last of a split pair holds
    // one of its chunks.  (Pair mode: the workgroup's pair, no plan.)
    int *prefix = reinterpret_cast<int *>(smem + kWaves * S::STAGE) + kWaves;
    auto pre = [&](int bb) { return __builtin_amdgcn_readfirstlane(prefix[bb]); };
    int64_t U = 0, N = 1, a = 0, u0 = 0, u1 = 0;
    if constexpr (!PAIR) {
        build_prefix<CT>(p, prefix, prefix - kWaves);
        U = pre(B);
        const int64_t launched = (int64_t)gridDim.x * kWaves;
        const int64_t want = floor_div(U, (int64_t)kUnitsPerChunk * p.min_chunks);
        N = want < 1 ? 1 : (want < launched ? want : launched);
        a = (int64_t)w * gridDim.x + blockIdx.x;  // active waves spread over the CUs

        // Sequences with no token: zero rows (any wave of the grid, by stride).
        for (int bb = (int)a; bb < B; bb += (int)launched) {
            if (prefix[bb + 1] != prefix[bb])
                continue;
            for (int e = lane; e < p.num_q_heads * D; e += kWave)
                store_out(p.out, (int64_t)bb * p.num_q_heads * D + e, 0.0f, p.out_kind);
        }
        if (a >= N || U == 0)
            return;
        u0 = range_start(a, U, N);
        u1 = range_start(a + 1, U, N);
    }

    const float c = fabsf(p.scale_log2);
    // softmax runs on raw dots scaled by c = |scale| log2(e) inside the
    // exponent; a negative scale flips the sign of q instead (exact)
    const uint32_t qflip = p.scale_log2 < 0.0f ? (S::F32 ? 0x80000000u : 0x80008000u) : 0u;
    const int64_t block_stride = (int64_t)Hkv * S::TILE;
    char *stage = smem + (size_t)w * S::STAGE;  // this wave's [2 buffers][K, V][CHUNK]
    const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(lds_address(stage));

    // XOR swizzles of a staged row's 16-byte units (16-bit KV), so that the
    // operand reads below hit distinct LDS banks: physical unit = logical
    // unit ^ sw(row).  fp32 rows are stored unswizzled.
    auto swk = [](int r) { return S::F32 ? 0 : ((D == 64 ? r >> 1 : r) & (LPR - 1)); };
    auto swv = [](int r) { return S::F32 ? 0 : (((D == 64 ? r >> 1 : r) & (LPR / 2 - 1)) << 1); };

    // ---- segment iterator --------------------------------------------------
    auto seq_chunks = [&](int bb) {
        const int d = (pre(bb + 1) - pre(bb)) / Hkv;  // units of one pair
        return d > 0 ? (d - kUnitsPerPair) / kUnitsPerChunk : 0;
    };
    // chunks of the pair starting at unit s whose anchors lie below u
    auto anchors_below = [&](int64_t s, int64_t u, int nch) {
        const int64_t r = u - s - kUnitsPerPair;
        const int64_t k = r <= 0 ? 0 : (r + kUnitsPerChunk - 1) / kUnitsPerChunk;
        return (int)(k < nch ? k : nch);
    };
    // the pair (b, h) starting at unit s as a segment of [u0, u1)
    auto segment = [&](int b, int h, int nch, int L, int64_t s, bool first) {
        Segment sg;
        sg.b = b;
        sg.h = h;
        sg.nch = nch;
        sg.L = L;
        sg.pu0 = s;
        sg.k0 = anchors_below(s, u0, nch);
        sg.k1 = anchors_below(s, u1, nch);
        sg.first = first;
        return sg;
    };
    // the pair after s, if it has a chunk in the range (false at its end)
    auto advance = [&](const Segment &s, Segment &nx) {
        if constexpr (PAIR)
            return false;
        const int64_t start = s.pu0 + (int64_t)kUnitsPerChunk * s.nch + kUnitsPerPair;
        if (start + kUnitsPerPair >= u1)
            return false;
        if (s.h + 1 < Hkv) {
            nx = segment(s.b, s.h + 1, s.nch, s.L, start, false);
        } else {
            int bb = s.b + 1;
            while (pre(bb + 1) == pre(bb))  // skip empty sequences (start < U)
                ++bb;
            nx = segment(bb, 0, seq_chunks(bb), seq_len_uniform(p, bb), start, false);
        }
        return true;
    };
    Segment cur;
    bool empty_range = false;  // pair mode: this wave has no chunk of the pair
    if constexpr (PAIR) {
        const int b = (int)(blockIdx.x / (unsigned)Hkv), h = (int)(blockIdx.x % (unsigned)Hkv);
        const int L = seq_len_uniform(p, b);
        if (L == 0) {  // the same for the whole workgroup: zero rows, nothing else
            for (int e = w * kWave + lane; e < G * D; e += kPairWaves * kWave)
                store_out(p.out, ((int64_t)b * p.num_q_heads + h * G) * D + e, 0.0f, p.out_kind);
            return;
        }
        const int nch = (L + CT - 1) / CT;
        cur.b = b;
        cur.h = h;
        cur.nch = nch;
        cur.L = L;
        cur.pu0 = 0;
        cur.first = true;
        cur.k0 = w * nch / kPairWaves;
        cur.k1 = (w + 1) * nch / kPairWaves;
        if (cur.k0 >= cur.k1) {
            // no chunk here: stream the pair's first chunk anyway (in bounds,
            // result discarded) so that the wave reaches the combine below
            empty_range = true;
            cur.k0 = 0;
            cur.k1 = 1;
        }
    } else {
        const int b0 = find_seq(prefix, B, u0);
        const int nch = seq_chunks(b0);
        const int64_t pu = (int64_t)kUnitsPerChunk * nch + kUnitsPerPair;
        const int h0 = (int)floor_div(u0 - pre(b0), pu);
        // the length is read once the first chunk is requested (below): a
        // scalar load here would be waited for by the next LDS access and
        // delay the block-id loads behind it
        cur = segment(b0, h0, nch, 0, pre(b0) + h0 * pu, true);
        if (cur.k0 >= cur.k1) {
            cur.L = seq_len_uniform(p, b0);
            // u0 lies past the pair's last anchor: the range starts with the
            // next pair, if any of its chunks lies in the range
            Segment nx;
            if (!advance(cur, nx))
                return;
            cur = nx;
            cur.first = true;
        }
    }

    // this lane's operand offsets inside a staged chunk
    uint32_t kofs[TPC][KS], vofs[TPC][MT][S::F32 ? 4 : 1];
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const int r = 16 * t + n, u = quad + 4 * st;
            kofs[t][st] = r * R + 16 * (u ^ swk(r));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (S::F32) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * t + 4 * quad + i, d = 16 * mt + n;
                    vofs[t][mt][i] = r * R + 4 * d;
                }
            } else {
                const int r = 16 * t + lane / 4, u = 2 * mt + (lane % 4) / 2;
                vofs[t][mt][0] = r * R + 16 * (u ^ swv(r)) + 8 * (lane % 2);
            }
        }
    }

    // the 16-bit operand reads' LDS addresses in chunk buffer 0 (buffer 1 is
    // 2 CHUNK further, an immediate offset of the reads)
    uint32_t ka0[4], va0[8];
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
#pragma unroll
        for (int st = 0; st < KS; ++st)
            ka0[(t * KS + st) % 4] = stage_lds + kofs[t][st];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            va0[(t * MT + mt) % 8] = stage_lds + CHUNK + vofs[t][mt][0];
    }

    // Block ids of chunk k of pair (b, h): NB table entries through the scalar
    // cache, clamped into the table row and into the pool.  Entries past the
    // sequence's last block may be read; the rows they give are masked.
    constexpr int NB = CT > BS ? CT / BS : 1;  // blocks a chunk touches
    struct Ids {
        int v[NB];
    };
    auto load_ids = [&](const Segment &s, int k) __attribute__((always_inline)) {
        Ids r;
        const int32_t *bt = p.block_tables + (int64_t)s.b * p.max_blocks_per_seq;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int bi = (k * CT) / BS + j;
            r.v[j] = scalar_load(bt, bi < p.max_blocks_per_seq ? bi : p.max_blocks_per_seq - 1);
        }
        return r;
    };

    // chunk k of pair (b, h) -> buffer buf: NL 1 KiB loads of K and of V,
    // each covering TPL whole rows of one block; lane l fills physical unit
    // l%LPR of row l/LPR, i.e. reads that row's logical unit (l%LPR) ^ sw(row).
    // Rows past the sequence end are masked when the chunk is used.
    auto stage_chunk = [&](const Segment &s, int k, int buf, const Ids &ids)
                           __attribute__((always_inline)) {
        const int tc = k * CT;
        const int64_t head_off = (int64_t)s.h * S::TILE;
        const uint32_t kd = __builtin_amdgcn_readfirstlane(stage_lds + buf * (2 * CHUNK));
        const uint32_t vd = kd + CHUNK;
        int blks[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
            blks[j] = ids.v[j] < 0 ? 0 : (ids.v[j] > p.num_blocks - 1 ? p.num_blocks - 1 : ids.v[j]);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t0 = tc + i * TPL;
            const int blk = blks[(i * TPL) / BS < NB ? (i * TPL) / BS : NB - 1];
            const int64_t row = (int64_t)blk * block_stride + head_off + (t0 % BS) * R;
            const int rr = i * TPL + tg;
            // a wave-uniform base plus an unsigned 32-bit lane offset: the
            // load's scalar-base form, with no 64-bit address add per lane
            load_to_lds(p.k_cache + row + (uint32_t)(tg * R + 16 * (cl ^ swk(rr))), kd + i * 1024);
            load_to_lds(p.v_cache + row + (uint32_t)(tg * R + 16 * (cl ^ swv(rr))), vd + i * 1024);
        }
    };

    // the segment's first chunk into buffer buf, its q^T operand (head n,
    // 16-byte unit quad + 4 st) and, when it holds position L - 1 of an
    // appending call, the new K/V row (lanes < LPR, unit cl)
    // The pair's q rows (and, when the segment holds position L - 1 of an
    // appending call, the new K and V rows) go to this wave's QA area by
    // DMA ahead of the chunk, so the wait for the chunk covers them and no
    // register load is in flight across the loop (which would make the
    // compiler wait for every access, stores included, before using it).
    const uint32_t qa_lds = stage_lds + 4 * CHUNK;
    auto prime = [&](const Segment &s, int64_t &pool_slot, int buf, const Ids &ids)
                     __attribute__((always_inline)) {
        const char *qsrc = p.q + ((int64_t)s.b * p.num_q_heads + s.h * G) * R;
#pragma unroll
        for (int i = 0; i < (S::QROWS + 1023) / 1024; ++i)
            if (i * 1024 + lane * 16 < S::QROWS)
                load_to_lds(qsrc + i * 1024 + lane * 16, qa_lds + i * 1024);
        if (p.k_new != nullptr && s.k1 == s.nch) {
            if (lane < LPR) {
                const int64_t hoff = (int64_t)s.h * R + lane * 16;
                load_to_lds(p.k_new + s.b * p.k_new_stride + hoff, qa_lds + S::QROWS);
                load_to_lds(p.v_new + s.b * p.v_new_stride + hoff, qa_lds + S::QROWS + R);
            }
            const int32_t *slot_words = reinterpret_cast<const int32_t *>(p.slots);
            const uint32_t lo = (uint32_t)scalar_load(slot_words, 2 * (int64_t)s.b);
            const uint32_t hi = (uint32_t)scalar_load(slot_words, 2 * (int64_t)s.b + 1);
            pool_slot = (int64_t)(((uint64_t)hi << 32) | lo);
        }
        stage_chunk(s, s.k0, buf, ids);
    };

    // partial results: slot s holds S::PART floats at byte s * 4 * S::PART
    // (two slots per launched wave)
    const __amdgpu_buffer_rsrc_t parts_view =
        buffer_view(p.parts, (uint32_t)(2u * gridDim.x * kWaves * S::PART * 4u));
    auto part_byte = [&](int64_t slot) { return (uint32_t)(slot * (S::PART * 4)); };

    uint4 knew = make_uint4(0, 0, 0, 0), vnew = make_uint4(0, 0, 0, 0);
    int64_t pool_slot = -1;
    prime(cur, pool_slot, 0, load_ids(cur, cur.k0));
    if constexpr (!PAIR)
        cur.L = seq_len_uniform(p, cur.b);
    int par = 0;  // chunk buffer of the current segment's first chunk
    // split segments of this range (at most the first and the last), reported
    // once the whole range is done: {b, h, first flat chunk of the pair}
    int sp_b[2] = {-1, -1}, sp_h[2] = {0, 0};
    int64_t sp_pu0[2] = {0, 0};

    // A finished segment's stores wait in registers until the next chunk's
    // operands have been read from LDS, so that no wait for those operands
    // (the compiler waits for every access in flight before an LDS read) is
    // a wait for store acknowledgements.
    struct Pending {
        bool valid, whole, app;
        int b, h;
        int64_t part_slot, pool_slot;  // partial-result slot; pool slot of the new row
        float4_t O[MT];
        float l, m;
        uint4 knew, vnew;
    } pend;
    pend.valid = false;
    int younger = 0;  // vector memory instructions issued after the last chunk request
    auto flush = [&]() __attribute__((always_inline)) {
        if (!pend.valid)
            return;
        pend.valid = false;
        // (at least) this many stores join the accesses in flight
        younger += pend.whole ? MT : MT + 2;
        if (pend.whole) {
            const float inv = pend.l > 0.0f ? 1.0f / pend.l : 0.0f;
            if (head_ok) {
                const int64_t orow = ((int64_t)pend.b * p.num_q_heads + pend.h * G + n) * D;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    store_out4(p.out, orow + 16 * mt + 4 * quad, pend.O[mt] * inv, p.out_kind);
            }
        } else if (head_ok) {
            // partial: (unnormalised O, max in log2 units, sum) with stores
            // that another XCD reads back
            const uint32_t pb = part_byte(pend.part_slot);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                coherent_store16(parts_view, pb + 4 * (n * D + 16 * mt + 4 * quad), pend.O[mt]);
            if (quad == 0) {
                float *pf = p.parts + pend.part_slot * S::PART;
                coherent_store(pf + G * D + n, pend.m);
                coherent_store(pf + G * D + G + n, pend.l);
            }
        }
        if (pend.app && lane < LPR) {
            // the new row into its slot, for later steps (this call used it
            // from registers)
            const int64_t slot = pend.pool_slot;
            if (slot >= 0 && slot < p.num_slots) {
                const int64_t blk = slot / BS;
                const int64_t dst = (blk * Hkv + pend.h) * S::TILE + (slot - blk * BS) * R + lane * 16;
                *reinterpret_cast<uint4 *>(p.k_store + dst) = pend.knew;
                *reinterpret_cast<uint4 *>(p.v_store + dst) = pend.vnew;
            }
        }
    };

    // Block ids run one chunk ahead of the chunk requested next: ids_a holds
    // those of the next chunk to request (the next chunk of this segment, or
    // the next segment's first chunk); the segment after next and the ids
    // following the next segment's first chunk are found while that chunk is
    // requested, so no scalar load is waited for at a segment boundary.
    Segment nxt;
    bool has_next = advance(cur, nxt);
    auto ids_following = [&](const Segment &s, bool more, const Segment &after)
                             __attribute__((always_inline)) {
        Ids r{};
        if (s.k0 + 1 < s.k1)
            r = load_ids(s, s.k0 + 1);
        else if (more)
            r = load_ids(after, after.k0);
        return r;
    };
    Ids ids_a = ids_following(cur, has_next, nxt);
    for (;;) {
        Segment nxt2;
        bool has_next2 = false;
        Ids ids_carry{};
        int64_t pool_slotn = -1;
        auto ids_after = [&](int k) __attribute__((always_inline)) {
            Ids r{};
            if (k < cur.k1)
                r = load_ids(cur, k);
            else if (has_next)
                r = load_ids(nxt, nxt.k0);
            return r;
        };
        const bool app = p.k_new != nullptr && cur.k1 == cur.nch && !empty_range;
        const int k_app = cur.nch - 1;                 // chunk of position L - 1
        const int row_app = cur.L - 1 - k_app * CT;    // its row in that chunk

        // q^T operand (head n, 16-byte unit quad + 4 st) from QA, read once
        // the segment's first chunk (DMA'd after it) has landed: sign of the
        // scale applied, padding heads zero
        uint4 qs[KS];
        auto read_q = [&]() __attribute__((always_inline)) {
            const int nn = head_ok ? n : G - 1;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                uint4 v = lds_read16(qa_lds + nn * R + 16 * (quad + 4 * st));
                v.x ^= qflip;
                v.y ^= qflip;
                v.z ^= qflip;
                v.w ^= qflip;
                qs[st] = select4(head_ok, v, make_uint4(0, 0, 0, 0));
            }
        };
        float4_t O[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            O[mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float mref = -INFINITY, lsum = 0.0f;
        // fp16 KV: the sums of the rounded probabilities come from one more
        // product per tile with an all-ones V^T operand (every row of the
        // result is the head's sum over the tile's tokens), off the vector ALUs
        constexpr bool kSumByMfma = std::is_same<T, TF16>::value;
        float4_t lacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const int nk = cur.k1 - cur.k0;
        // one chunk: wait for it, read its operands, request the next chunk
        // (or, for the segment's last chunk, the next segment's first one),
        // then the tile math.  The last chunk is a separate instance, so the
        // next segment's registers are only written there.
        auto run_chunk = [&](int kk, auto last_tag) __attribute__((always_inline)) {
            constexpr bool LAST = decltype(last_tag)::value;
            const int k = cur.k0 + kk;
            char *kd = stage + ((par + kk) & 1) * (2 * CHUNK);
            char *vd = kd + CHUNK;
            const uint32_t kdl = __builtin_amdgcn_readfirstlane(lds_address(kd));
            const uint32_t vdl = kdl + CHUNK;
            const int tc = k * CT;
            // chunk k is in LDS: it is the last DMA requested, and only the
            // `younger` stores issued after it may still be in flight
            if constexpr (S::F32)
                wait_vmem();
            else
                wait_vmem_keep(younger);
            // only a segment's last chunk can hold the pair's end; every
            // other chunk is full, which the compiler then knows (not used
            // at head_dim 128, where the schedule of the specialised loop
            // exceeds 256 registers and spills)
            const bool full = (!LAST && D == 64) || tc + CT <= cur.L;
            if (!full) {
                // rows past the end: zero V (stale or NaN slots must not reach the sum)
#pragma unroll
                for (int i = 0; i < NL; ++i)
                    if (tc + i * TPL + tg >= cur.L) {
                        if constexpr (S::F32)
                            *reinterpret_cast<uint4 *>(vd + i * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
                        else
                            lds_write16(vdl + i * 1024 + lane * 16, make_uint4(0, 0, 0, 0));
                    }
            }
            if (kk == 0)
                read_q();
            if (app && k == k_app && lane < LPR) {
                // position L-1 takes the new K/V (from QA), not the pool
                knew = lds_read16(qa_lds + S::QROWS + 16 * lane);
                vnew = lds_read16(qa_lds + S::QROWS + R + 16 * lane);
                const uint32_t ko = row_app * R + 16 * (lane ^ swk(row_app));
                const uint32_t vo = row_app * R + 16 * (lane ^ swv(row_app));
                if constexpr (S::F32) {
                    *reinterpret_cast<uint4 *>(kd + ko) = knew;
                    *reinterpret_cast<uint4 *>(vd + vo) = vnew;
                } else {
                    lds_write16(kdl + ko, knew);
                    lds_write16(vdl + vo, vnew);
                }
            }
            uint4 kop[TPC][KS];
            uint4 vop[TPC][MT];  // fp16/bf16: .x/.y hold the operand
            if constexpr (S::F32) {
#pragma unroll
                for (int t = 0; t < TPC; ++t) {
#pragma unroll
                    for (int st = 0; st < KS; ++st)
                        kop[t][st] = *reinterpret_cast<const uint4 *>(kd + kofs[t][st]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        vop[t][mt].x = *reinterpret_cast<const uint32_t *>(vd + vofs[t][mt][0]);
                        vop[t][mt].y = *reinterpret_cast<const uint32_t *>(vd + vofs[t][mt][1]);
                        vop[t][mt].z = *reinterpret_cast<const uint32_t *>(vd + vofs[t][mt][2]);
                        vop[t][mt].w = *reinterpret_cast<const uint32_t *>(vd + vofs[t][mt][3]);
                    }
                }
            } else {
                static_assert(TPC * KS == 4 && TPC * MT == 8, "one chunk: 4 + 8 operand reads");
                u32x4 kr[4];
                u32x2 vr[8];
                if ((par + kk) & 1)
                    lds_read_chunk<2 * CHUNK>(kr, vr, ka0, va0);
                else
                    lds_read_chunk<0>(kr, vr, ka0, va0);
#pragma unroll
                for (int t = 0; t < TPC; ++t) {
#pragma unroll
                    for (int st = 0; st < KS; ++st) {
                        const u32x4 x = kr[t * KS + st];
                        kop[t][st] = make_uint4(x[0], x[1], x[2], x[3]);
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const u32x2 x = vr[t * MT + mt];
                        vop[t][mt] = make_uint4(x[0], x[1], 0, 0);
                    }
                }
            }
            // the next chunk into the other buffer (read in the previous
            // iteration), or the next segment's first chunk; then the
            // previous segment's stores, which stay in flight behind it
            const int nbuf = (par + kk + 1) & 1;
            if constexpr (!LAST) {
                stage_chunk(cur, k + 1, nbuf, ids_a);
                ids_a = ids_after(k + 2);
            } else if (has_next) {
                prime(nxt, pool_slotn, nbuf, ids_a);
                has_next2 = advance(nxt, nxt2);
                ids_carry = ids_following(nxt, has_next2, nxt2);
            }
            asm volatile("" ::: "memory");  // the stores below are issued after the DMA
            younger = 0;
            flush();

#pragma unroll
            for (int t = 0; t < TPC; ++t) {
                float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < KS; ++st)
                    sacc = mma_qk(T{}, kop[t][st], qs[st], sacc);
                const int tok0 = tc + 16 * t + 4 * quad;
                bool ok[4];
                float sv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ok[i] = full || tok0 + i < cur.L;
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
                    if constexpr (kSumByMfma)
                        lacc *= corr;
                    else
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
                if constexpr (S::F32) {
                    const uint4 pf = make_uint4(__builtin_bit_cast(uint32_t, pr[0]),
                                                __builtin_bit_cast(uint32_t, pr[1]),
                                                __builtin_bit_cast(uint32_t, pr[2]),
                                                __builtin_bit_cast(uint32_t, pr[3]));
                    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        O[mt] = mma_pv(T{}, vop[t][mt], pf, O[mt]);
                } else if constexpr (std::is_same<T, TF16>::value) {
                    const half2_t h01 = {(_Float16)pr[0], (_Float16)pr[1]};
                    const half2_t h23 = {(_Float16)pr[2], (_Float16)pr[3]};
                    const uint2 ph = make_uint2(__builtin_bit_cast(uint32_t, h01),
                                                __builtin_bit_cast(uint32_t, h23));
                    lacc = mma_pv(T{}, make_uint2(0x3C003C00u, 0x3C003C00u), ph, lacc);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        O[mt] = mma_pv(T{}, make_uint2(vop[t][mt].x, vop[t][mt].y), ph, O[mt]);
                } else {
                    // bf16 P as a hi + lo pair: 16 significant bits
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
                        const uint2 v2 = make_uint2(vop[t][mt].x, vop[t][mt].y);
                        O[mt] = mma_pv(T{}, v2, ph, O[mt]);
                        O[mt] = mma_pv(T{}, v2, pl, O[mt]);
                    }
                }
            }
        };
        for (int kk = 0; kk + 1 < nk; ++kk)
            run_chunk(kk, std::false_type{});
        run_chunk(nk - 1, std::true_type{});

        // ---- the segment's result (stored by flush()) -----------------------
        float lh;
        if constexpr (kSumByMfma) {
            lh = lacc[0];  // already the head's sum over all its tokens
        } else {
            lh = lsum + swz_xor16(lsum);  // the head's sum over its four lanes
            lh += xor32(lh);
        }
        pend.valid = true;
        pend.whole = cur.k0 == 0 && cur.k1 == cur.nch;
        pend.app = app;
        pend.b = cur.b;
        pend.h = cur.h;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            pend.O[mt] = O[mt];
        pend.l = lh;
        pend.m = mref == -INFINITY ? mref : mref * c;
        pend.knew = knew;
        pend.vnew = vnew;
        pend.part_slot = 2 * a + (cur.first ? 0 : 1);
        pend.pool_slot = app ? pool_slot : -1;
        if (!pend.whole) {
            if (cur.first) {
                sp_b[0] = cur.b;
                sp_h[0] = cur.h;
                sp_pu0[0] = cur.pu0;
            } else {
                sp_b[1] = cur.b;
                sp_h[1] = cur.h;
                sp_pu0[1] = cur.pu0;
            }
        }
        if (!has_next)
            break;
        par = (par + nk) & 1;
        cur = nxt;
        nxt = nxt2;
        has_next = has_next2;
        ids_a = ids_carry;
        pool_slot = pool_slotn;
    }

    if constexpr (PAIR) {
        // the new row into its slot (the fused write), then this wave's part
        // (unnormalised O, max in log2 units, sum) into its own staging
        // area, free now; after the barrier the waves combine the parts
        if (pend.app && lane < LPR) {
            const int64_t slot = pend.pool_slot;
            if (slot >= 0 && slot < p.num_slots) {
                const int64_t blk = slot / BS;
                const int64_t dst = (blk * Hkv + pend.h) * S::TILE + (slot - blk * BS) * R + lane * 16;
                *reinterpret_cast<uint4 *>(p.k_store + dst) = pend.knew;
                *reinterpret_cast<uint4 *>(p.v_store + dst) = pend.vnew;
            }
        }
        float *mine = reinterpret_cast<float *>(stage);
        if (head_ok) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<float4_t *>(mine + n * D + 16 * mt + 4 * quad) =
                    empty_range ? float4_t{0.0f, 0.0f, 0.0f, 0.0f} : pend.O[mt];
            if (quad == 0) {
                mine[G * D + n] = empty_range ? -INFINITY : pend.m;
                mine[G * D + G + n] = empty_range ? 0.0f : pend.l;
            }
        }
        __syncthreads();
        // out = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w over the waves
        const int64_t orow = ((int64_t)pend.b * p.num_q_heads + pend.h * G) * D;
        for (int e = w * kWave + lane; e < G * D; e += kPairWaves * kWave) {
            const int g = e / D;
            float mw[kPairWaves], M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < kPairWaves; ++ww) {
                mw[ww] = reinterpret_cast<const float *>(smem + ww * S::STAGE)[G * D + g];
                M = fmaxf(M, mw[ww]);
            }
            float num = 0.0f, den = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kPairWaves; ++ww) {
                const float *part = reinterpret_cast<const float *>(smem + ww * S::STAGE);
                const float wt = mw[ww] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[ww] - M);
                num = fmaf(wt, part[e], num);
                den = fmaf(wt, part[G * D + G + g], den);
            }
            store_out(p.out, orow + e, den > 0.0f ? num / den : 0.0f, p.out_kind);
        }
        return;
    }
    flush();  // the last segment's stores
    // ---- report the split pairs; the last wave of a pair combines it -------
    if (sp_b[0] < 0 && sp_b[1] < 0)
        return;
    wait_vmem();  // this wave's partial stores are acknowledged
    // both reports in one round trip: lane si reports split pair si
    int64_t wf_[2], wl_[2];
    int nseg_[2];
#pragma unroll
    for (int si = 0; si < 2; ++si) {
        // the waves holding the pair's first and last chunk anchors
        const int64_t fa = sp_pu0[si] + kUnitsPerPair;
        const int64_t la = sp_b[si] < 0 ? fa : fa + (int64_t)kUnitsPerChunk * (seq_chunks(sp_b[si]) - 1);
        wf_[si] = wave_of(fa, U, N);
        wl_[si] = wave_of(la, U, N);
        nseg_[si] = (int)(wl_[si] - wf_[si] + 1);
    }
    int old = -1;
    const int rb = lane == 0 ? sp_b[0] : sp_b[1], rh = lane == 0 ? sp_h[0] : sp_h[1];
    if (lane < 2 && rb >= 0)
        old = __hip_atomic_fetch_add(p.counters + ((int64_t)rb * Hkv + rh) * kCounterStride, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    const bool last0 = __builtin_amdgcn_readlane(old, 0) == nseg_[0] - 1 && sp_b[0] >= 0;
    const bool last1 = __builtin_amdgcn_readlane(old, 1) == nseg_[1] - 1 && sp_b[1] >= 0;
    // out = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j over a pair's
    // parts, 64 parts at a time with a running maximum.  Lane j of a batch
    // reads part j's (max, sum) block (2G floats, 16-byte loads); each lane
    // accumulates its output elements e = lane + 64 i (head (64 i) / D, the
    // same in all lanes) over the parts, BJ parts' rows at a time, the first
    // rows requested with the (max, sum) blocks.  One copy of this code
    // serves both split pairs (a loop that is not unrolled): it runs once per
    // combine, where its instruction fetches are on the critical path.
    constexpr int E = G * D / kWave;      // output elements per lane
    constexpr int BJ = 8;                 // parts per batch of row loads
    constexpr int MLV = (2 * G + 3) / 4;  // 16-byte loads of one (max, sum) block
#pragma unroll 1
    for (int si = 0; si < 2; ++si) {
        if (!(si == 0 ? last0 : last1))
            continue;
        const int bb = si == 0 ? sp_b[0] : sp_b[1], hh = si == 0 ? sp_h[0] : sp_h[1];
        const int64_t wf = si == 0 ? wf_[0] : wf_[1];
        const int nseg = si == 0 ? nseg_[0] : nseg_[1];
        // part of wave ww: the first contributing wave holds it in its second
        // slot when the pair starts inside that wave's range (the previous
        // pair's last anchor, kUnitsPerChunk below the pair's start, is in
        // it); every later wave's range starts inside the pair, so there it
        // is the first slot
        const int64_t ps = si == 0 ? sp_pu0[0] : sp_pu0[1];
        const int64_t slot_wf = 2 * wf + (ps > 0 && ps - kUnitsPerChunk >= range_start(wf, U, N) ? 1 : 0);
        auto slot_of = [&](int64_t ww) { return ww == wf ? slot_wf : 2 * ww; };
        float Mrun[G], den[G], acc[E];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            Mrun[g] = -INFINITY;
            den[g] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < E; ++i)
            acc[i] = 0.0f;
        for (int j0 = 0; j0 < nseg; j0 += kWave) {
            const int nb = nseg - j0 < kWave ? nseg - j0 : kWave;
            const bool mine = lane < nb;
            float o[BJ][E];
            auto load_rows = [&](int jj) __attribute__((always_inline)) {
#pragma unroll
                for (int u = 0; u < BJ; ++u) {
                    const int j = jj + u < nb ? jj + u : nb - 1;
                    const float *pr = p.parts + slot_of(wf + j0 + j) * S::PART;
#pragma unroll
                    for (int i = 0; i < E; ++i)
                        o[u][i] = coherent_load(pr + kWave * i + lane);
                }
            };
            float4_t ml[MLV];
            {
                const uint32_t pb = part_byte(slot_of(wf + j0 + (mine ? lane : nb - 1)));
#pragma unroll
                for (int v = 0; v < MLV; ++v)
                    ml[v] = coherent_load16(parts_view, pb + 4 * (G * D + 4 * v));
            }
            load_rows(0);
            // the G heads' weights (lanes past the last part weigh 0)
            float mj[G], lj[G], mx[G], wj[G], sw[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                mj[g] = mine ? ml[g / 4][g % 4] : -INFINITY;
                lj[g] = mine ? ml[(G + g) / 4][(G + g) % 4] : 0.0f;
                mx[g] = mj[g];
            }
            wave_max_n(mx);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float Mb = fmaxf(Mrun[g], mx[g]);
                const float rs = Mrun[g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Mrun[g] - Mb);
                wj[g] = mj[g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mj[g] - Mb);
                sw[g] = wj[g] * lj[g];
                den[g] *= rs;
#pragma unroll
                for (int i = 0; i < E; ++i)
                    if ((kWave * i) / D == g)
                        acc[i] *= rs;
                Mrun[g] = Mb;
            }
            wave_sum_n(sw);
#pragma unroll
            for (int g = 0; g < G; ++g)
                den[g] += sw[g];
            for (int jj = 0; jj < nb; jj += BJ) {
                if (jj > 0)
                    load_rows(jj);
                float wgt[BJ][G];
#pragma unroll
                for (int u = 0; u < BJ; ++u)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        wgt[u][g] = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj[g]), jj + u));
#pragma unroll
                for (int u = 0; u < BJ; ++u)
#pragma unroll
                    for (int i = 0; i < E; ++i)
                        acc[i] = fmaf(wgt[u][(kWave * i) / D], o[u][i], acc[i]);
            }
        }
        float res[E];
        int64_t idx[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const int g = (kWave * i) / D, d = kWave * i + lane - g * D;
            res[i] = den[g] > 0.0f ? acc[i] / den[g] : 0.0f;
            idx[i] = ((int64_t)bb * p.num_q_heads + hh * G + g) * D + d;
        }
        if (p.out_kind == 0) {
#pragma unroll
            for (int i = 0; i < E; ++i)
                store_out(p.out, idx[i], res[i], 0);
        } else if (p.out_kind == 1) {
#pragma unroll
            for (int i = 0; i < E; ++i)
                store_out(p.out, idx[i], res[i], 1);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                store_out(p.out, idx[i], res[i], 2);
        }
        if (lane == 0)
            __hip_atomic_store(p.counters + ((int64_t)bb * Hkv + hh) * kCounterStride, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <class T, int D, int BS, int G>
size_t decode_lds_bytes(int num_seqs)
{
    using S = Shape<T, D, BS, G>;
    return (size_t)kWaves * S::STAGE + (size_t)(kWaves + num_seqs + 1) * 4;
}

// Workgroups of decode_kernel<...> resident on the device at once for a
// dynamic LDS size (cached per device and LDS size class).
template <class T, int D, int BS, int G>
int resident_workgroups(size_t lds)
{
    static int cached[64][2];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    const int cls = lds > decode_lds_bytes<T, D, BS, G>(kMaxSeqsPerLaunch / 2) ? 1 : 0;
    if (cached[dev][cls] == 0) {
        (void)hipFuncSetAttribute((const void *)decode_kernel<T, D, BS, G, false>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)decode_lds_bytes<T, D, BS, G>(kMaxSeqsPerLaunch));
        const size_t probe = decode_lds_bytes<T, D, BS, G>(cls ? kMaxSeqsPerLaunch : kMaxSeqsPerLaunch / 2);
        int per_cu = 0;
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<T, D, BS, G, false>,
                                                           kWaves * kWave, probe);
        per_cu = per_cu < 1 ? 1 : (per_cu > kMaxWorkgroupsPerCU ? kMaxWorkgroupsPerCU : per_cu);
        cached[dev][cls] = device_compute_units() * per_cu;
    }
    return cached[dev][cls];
}

template <class T, int D, int BS, int G>
hipError_t launch_group(const DecodeArgs &a, hipStream_t stream)
{
    using S = Shape<T, D, BS, G>;
    DecodeParams p;
    p.out = a.out;
    p.out_kind = (int)a.out_dtype;
    p.q = static_cast<const char *>(a.q);
    p.k_cache = static_cast<const char *>(a.k_cache);
    p.v_cache = static_cast<const char *>(a.v_cache);
    p.block_tables = a.block_tables;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.context_lens = a.context_lens;
    p.num_seqs = a.num_seqs;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.num_blocks = a.num_blocks;
    p.scale_log2 = a.scale * kLog2e;
    const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
    p.len_cap = (int32_t)(cap > INT32_MAX ? INT32_MAX : cap);
    const int min_tokens = a.partition_size > 0 ? a.partition_size : kDefaultRangeTokens;
    p.min_chunks = (min_tokens + S::CT - 1) / S::CT;
    p.parts = a.parts;
    p.counters = a.counters;
    p.k_new = static_cast<const char *>(a.k_new);
    p.v_new = static_cast<const char *>(a.v_new);
    p.k_new_stride = a.k_new_token_stride * dtype_bytes(a.kv_dtype);
    p.v_new_stride = a.v_new_token_stride * dtype_bytes(a.kv_dtype);
    p.slots = a.slot_mapping;
    p.k_store = static_cast<char *>(const_cast<void *>(a.k_cache));
    p.v_store = static_cast<char *>(const_cast<void *>(a.v_cache));
    p.num_slots = (int64_t)a.num_blocks * a.block_size;
    if constexpr (!S::F32) {
        // Pair mode, when the library picks the split: as many (sequence,
        // kv head) pairs as compute units and sequences short enough (by the
        // table width, or the caller's hint) for kPairWaves waves of one
        // compute unit to stream each pair: no planning and no partial
        // results in HBM.
        constexpr size_t pair_lds = (size_t)kPairWaves * S::STAGE;
        const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
        const int64_t longest = a.context_hint > 0 && a.context_hint < cap ? a.context_hint : cap;
        if (a.partition_size == 0 && pair_lds <= kPairModeMaxLds &&
            pairs <= device_compute_units() && longest <= kPairModeMaxTokens) {
            static bool attr_set[64];
            int dev = 0;
            (void)hipGetDevice(&dev);
            if (dev >= 0 && dev < 64 && !attr_set[dev]) {
                (void)hipFuncSetAttribute((const void *)decode_kernel<T, D, BS, G, true>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)pair_lds);
                attr_set[dev] = true;
            }
            hipLaunchKernelGGL((decode_kernel<T, D, BS, G, true>), dim3((unsigned)pairs),
                               dim3(kPairWaves * kWave), pair_lds, stream, p);
            return hipGetLastError();
        }
    }
    const size_t lds = decode_lds_bytes<T, D, BS, G>(a.num_seqs);
    int grid = resident_workgroups<T, D, BS, G>(lds);
    if ((int64_t)grid * kWaves > a.max_waves)
        grid = (int)(a.max_waves / kWaves);
    if (grid < 1)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_kernel<T, D, BS, G, false>), dim3(grid), dim3(kWaves * kWave), lds,
                       stream, p);
    return hipGetLastError();
}

template <class T, int D, int BS>
hipError_t dispatch_group(const DecodeArgs &a, hipStream_t s)
{
    switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_group<T, D, BS, 1>(a, s);
    case 2: return launch_group<T, D, BS, 2>(a, s);
    case 4: return launch_group<T, D, BS, 4>(a, s);
    case 8: return launch_group<T, D, BS, 8>(a, s);
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

int decode_max_waves()
{
    return device_compute_units() * kMaxWorkgroupsPerCU * kWaves;
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
