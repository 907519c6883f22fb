// Multi-token causal paged attention for gfx950 (CDNA4): the chunked
// prefill of a prompt, or the check of drafted tokens.
//
// What is computed (PhotonInfer README, Korean translation: "Continuous
// batching scheduler", where a request advances token by token through
// num_computed_tokens, and the speculative-decoding item of its "Roadmap";
// JackerLab "vllm" tag page, "Speculative Decoding": a large model checks
// several proposed tokens at once).  Sequence b brings T_b new query tokens,
// rows query_start[b] .. query_start[b+1] - 1 of q, whose K/V are already in
// the block-wise cache; with L_b = context_lens[b] (those new tokens
// included), new token i sits at position p = L_b - T_b + i and
//     out[row, hq, :] = sum_{t <= p} softmax_t(scale * q[row, hq, :] . K_t) V_t.
//
// Design.  A workgroup of four wave64s takes one (query block, kv head,
// sequence).  Its 64 columns are (new token, query head) pairs: G heads of
// 64 / G consecutive new tokens, 16 columns per wave.  It streams the
// sequence's K and V from position 0 to the block's last position in chunks
// (8 KiB of K and of V: two 1 KiB loads per wave and tensor, the measured
// best against one and four), which the waves copy by DMA (global_load_lds)
// into two LDS buffers shared by the workgroup, one chunk ahead.  Per 16-token tile
// each wave computes
//   S^T (16 tokens x 16 columns) = K_tile . Q^T        D/32 MFMAs 16x16x32
//   the online softmax on S^T, with the causal bound t <= p applied per
//   element by selects,
//   O^T (16 dims x 16 columns) += V_tile^T . P^T        D/16 MFMAs 16x16x16,
// the layout of the decode kernel with columns in place of heads.  Every K/V
// byte a workgroup reads serves 64 columns.  A wave whose columns all end
// before a chunk skips its arithmetic but keeps staging its share.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "cdna4.h"
#include "pka_internal.h"

namespace pka {
namespace {

struct PrefillParams {
    void *out;
    int out_kind;  // 0 f32, 1 f16, 2 bf16
    const char *q, *k_cache, *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
    const int32_t *query_start;
    int32_t num_query_tokens, num_q_heads, num_kv_heads, num_blocks;
    int32_t len_cap;  // max_blocks_per_seq * block_size
    float scale_log2;  // scale * log2(e)
    int32_t num_qblocks;  // workgroups (query blocks) per (sequence, kv head) pair
    int64_t num_pairs;    // num_seqs * num_kv_heads
};

// Workgroups are dealt to the XCDs in turn (workgroup i to XCD i % kXcds),
// and each XCD has its own L2.  The grid is numbered so that all query
// blocks of one (sequence, kv head) pair land on one XCD, one after another:
// they read the same K/V, which the first fetches into that L2 for the rest
// (spread over the XCDs, every L2 would fetch it again).  Workgroup i goes
// to XCD x = i % kXcds and takes item k = i / kXcds of that XCD's list: pair
// (k / nqb) * kXcds + x, query block k % nqb.
constexpr int kXcds = 8;

template <class T, int D, int BS, int G>
struct PShape {
    static constexpr int ELT = T::kBytes;
    static constexpr int LPR = D * ELT / 16;  // lanes per token row
    static constexpr int TPL = kWave / LPR;   // token rows per 1 KiB wave load
    static constexpr int NW = 4;              // waves per workgroup
    static constexpr int LPW = 2;             // 1 KiB loads per tensor per wave per chunk
    static constexpr int NL = NW * LPW;       // 1 KiB loads per tensor per chunk
    static constexpr int CT = NL * TPL;       // tokens per chunk
    static constexpr int TPC = CT / 16;       // 16-token tiles per chunk
    static constexpr int KS = D / 32;         // 32-dim steps of QK^T
    static constexpr int MT = D / 16;         // 16-dim tiles of O
    static constexpr int R = D * ELT;         // bytes per token row
    static constexpr int CHUNK = NL * 1024;   // bytes of one tensor's chunk
    static constexpr int TILE = BS * D * ELT; // bytes of one (block, head) tile
    static constexpr int NCT = 1;             // 16-column tiles per wave
    static constexpr int QB = NW * NCT * 16 / G;  // new tokens per workgroup
    static_assert(TPC >= 1 && CT % 16 == 0, "a chunk holds whole 16-token tiles");
    static_assert(BS % TPL == 0, "a wave load stays inside one block");
};

template <class T, int D, int BS, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p)
{
    using S = PShape<T, D, BS, G>;
    constexpr int LPR = S::LPR, TPL = S::TPL, TPC = S::TPC, KS = S::KS, MT = S::MT, CT = S::CT;
    constexpr int R = S::R, CHUNK = S::CHUNK, NCT = S::NCT;
    constexpr float kSlack = 8.0f;  // log2 units a logit may exceed the reference max by
    __shared__ __attribute__((aligned(1024))) char stage[2 * 2 * CHUNK];  // [buffer][K, V]

    const uint32_t xcd = blockIdx.x % kXcds, item = blockIdx.x / kXcds;
    const int64_t pair = (int64_t)(item / (uint32_t)p.num_qblocks) * kXcds + xcd;
    if (pair >= p.num_pairs)
        return;
    const int b = (int)(pair / p.num_kv_heads), h = (int)(pair % p.num_kv_heads);
    const int q0 = (int)(item % (uint32_t)p.num_qblocks) * S::QB;
    const int lane = threadIdx.x % kWave;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n = lane % 16, quad = lane / 16;
    const int tg = lane / LPR, cl = lane % LPR;

    // the sequence's new tokens (malformed offsets: nothing to do)
    const int r0 = __builtin_amdgcn_readfirstlane(p.query_start[b]);
    const int r1 = __builtin_amdgcn_readfirstlane(p.query_start[b + 1]);
    if (r0 < 0 || r1 < r0 || r1 > p.num_query_tokens)
        return;
    const int nq = r1 - r0;  // new tokens of the sequence
    if (q0 >= nq)
        return;
    int L = __builtin_amdgcn_readfirstlane(p.context_lens[b]);
    L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
    const int base = L - nq;  // position of new token 0

    // This lane's columns, one per column tile ct of the wave: new token
    // qi[ct], query head h*G + g[ct], position pos[ct].
    int qi[NCT], pos[NCT];
    bool col_ok[NCT];
    int64_t orow[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int col = 16 * (w * NCT + ct) + n;
        qi[ct] = q0 + col / G;
        pos[ct] = base + qi[ct];
        col_ok[ct] = qi[ct] < nq && pos[ct] >= 0;
        orow[ct] = ((int64_t)(r0 + qi[ct]) * p.num_q_heads + h * G + col % G) * D;
    }
    // last position of the workgroup and of this wave (wave-uniform)
    const int qlast = (q0 + S::QB < nq ? q0 + S::QB : nq) - 1;
    const int n_tok = base + qlast + 1;  // tokens the workgroup streams
    const int wq1 = q0 + (16 * NCT * (w + 1) - 1) / G;
    const int wave_last = base + (wq1 < nq ? wq1 : nq - 1);
    const bool wave_any = q0 + (16 * NCT * w) / G < nq;

    if (n_tok <= 0) {
        // no token precedes any of these queries (more new tokens than cached
        // ones): zero rows
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            if (qi[ct] < nq)
                for (int d = 4 * quad; d < D; d += 16)
                    for (int i = 0; i < 4; ++i)
                        store_out(p.out, orow[ct] + d + i, 0.0f, p.out_kind);
        return;
    }
    const int nch = (n_tok + CT - 1) / CT;
    const int last_blk = (n_tok - 1) / BS;

    // Softmax on raw dot products scaled by c = |scale| * log2(e) inside the
    // exponent; a negative scale flips the sign of q instead (exact).
    const float c = fabsf(p.scale_log2);
    const uint32_t qflip = p.scale_log2 < 0.0f ? 0x80008000u : 0u;

    // Q^T operands: column n of each tile, dims 32 st + 8 quad .. + 7
    // (columns without a query read row 0, in bounds, and are zeroed)
    uint4 qop[NCT][KS];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const char *qrow = p.q + ((col_ok[ct] ? orow[ct] : 0) + 8 * quad) * S::ELT;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            uint4 v = *reinterpret_cast<const uint4 *>(qrow + 32 * st * S::ELT);
            v.x ^= qflip;
            v.y ^= qflip;
            v.z ^= qflip;
            v.w ^= qflip;
            qop[ct][st] = select4(col_ok[ct], v, make_uint4(0, 0, 0, 0));
        }
    }

    // XOR swizzles of a staged row's 16-byte units (physical = logical ^ sw)
    auto swk = [](int r) { return (D == 64 ? r >> 1 : r) & (LPR - 1); };
    auto swv = [](int r) { return ((D == 64 ? r >> 1 : r) & (LPR / 2 - 1)) << 1; };
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

    // Block ids: a window of 64 consecutive entries of the block table, one
    // per lane, read again when a chunk leaves it (ids clamped to the pool).
    const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
    int win0 = -2 * kWave, ids = 0;  // no window loaded yet
    auto block_id = [&](int bi) __attribute__((always_inline)) {
        if (bi < win0 || bi >= win0 + kWave) {  // wave-uniform
            win0 = bi;
            const int e = win0 + lane < p.max_blocks_per_seq ? win0 + lane : p.max_blocks_per_seq - 1;
            const int id = bt[e];
            ids = id < 0 ? 0 : (id > p.num_blocks - 1 ? p.num_blocks - 1 : id);
        }
        return __builtin_amdgcn_readlane(ids, bi - win0);
    };

    // This wave's share of chunk k: its LPW loads of K and of V (token rows
    // [k CT + li TPL, + TPL) for load li) into buffer buf; lane l fills
    // physical unit l % LPR of its row.
    const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(lds_address(stage));
    const int64_t head_off = (int64_t)h * S::TILE;
    const int64_t block_stride = (int64_t)p.num_kv_heads * S::TILE;
    auto stage_share = [&](int k, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int l = 0; l < S::LPW; ++l) {
            const int li = w * S::LPW + l;  // this load's index in the chunk
            const int t0 = k * CT + li * TPL;
            int bi = t0 / BS;
            bi = bi < last_blk ? bi : last_blk;  // rows past the end re-read the last block
            const int blk = block_id(bi);
            const int64_t row = (int64_t)blk * block_stride + head_off + (t0 % BS) * R;
            const int rr = li * TPL + tg;
            const uint32_t kd = stage_lds + buf * (2 * CHUNK) + li * 1024;
            load_to_lds(p.k_cache + row + tg * R + 16 * (cl ^ swk(rr)), kd);
            load_to_lds(p.v_cache + row + tg * R + 16 * (cl ^ swv(rr)), kd + CHUNK);
        }
    };

    float4_t O[NCT][MT];
    float mref[NCT], lsum[NCT];
    // fp16 KV: the sums of the rounded probabilities come from one more
    // product per tile with an all-ones V^T operand (every row of the result
    // is the column's sum over the tile's tokens), off the vector ALUs
    constexpr bool kSumByMfma = std::is_same<T, TF16>::value;
    float4_t lacc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        mref[ct] = -INFINITY;
        lsum[ct] = 0.0f;
        lacc[ct] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            O[ct][mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    stage_share(0, 0);
    for (int k = 0; k < nch; ++k) {
        const int buf = k & 1;
        char *kd = stage + buf * (2 * CHUNK);
        char *vd = kd + CHUNK;
        const int tc = k * CT;
        wait_vmem();  // this wave's share of chunk k is in LDS
        if (tc + CT > L) {
            // rows at or past L hold stale or NaN slots: zero their V (K is
            // masked by selects); each wave clears the rows it staged
#pragma unroll
            for (int l = 0; l < S::LPW; ++l) {
                const int li = w * S::LPW + l;
                if (tc + li * TPL + tg >= L)
                    *reinterpret_cast<uint4 *>(vd + li * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
            }
        }
        __syncthreads();  // every share landed; chunk k - 1's buffer is free
        const bool work = wave_any && tc <= wave_last;
        uint4 kop[TPC][KS];
        uint2 vop[TPC][MT];
        if (work) {
#pragma unroll
            for (int t = 0; t < TPC; ++t) {
#pragma unroll
                for (int st = 0; st < KS; ++st)
                    kop[t][st] = *reinterpret_cast<const uint4 *>(kd + kofs[t][st]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    vop[t][mt] = lds_read_tr16(vd + vofs[t][mt]);
            }
        }
        if (k + 1 < nch)
            stage_share(k + 1, buf ^ 1);
        if (!work)
            continue;
#pragma unroll
        for (int t = 0; t < TPC; ++t) {
            const int tok0 = tc + 16 * t + 4 * quad;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < KS; ++st)
                    sacc = mma_qk(T{}, kop[t][st], qop[ct][st], sacc);
                bool ok[4];
                float sv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ok[i] = col_ok[ct] && tok0 + i <= pos[ct];
                    sv[i] = ok[i] ? sacc[i] : -INFINITY;
                }
                const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                if (__builtin_amdgcn_ballot_w64(mx * c > mref[ct] * c + kSlack)) {
                    // new reference: the column's maximum over its four lanes
                    float mh = fmaxf(mx, swz_xor16(mx));
                    mh = fmaxf(mh, xor32(mh));
                    const float mnew = fmaxf(mref[ct], mh);
                    const float corr = mref[ct] == -INFINITY
                                           ? 0.0f
                                           : __builtin_amdgcn_exp2f((mref[ct] - mnew) * c);
                    if constexpr (kSumByMfma)
                        lacc[ct] *= corr;
                    else
                        lsum[ct] *= corr;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        O[ct][mt] *= corr;
                    mref[ct] = mnew;
                }
                const float nmc = mref[ct] == -INFINITY ? 0.0f : -mref[ct] * c;
                float pr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pr[i] = ok[i] ? __builtin_amdgcn_exp2f(fmaf(sv[i], c, nmc)) : 0.0f;
                if constexpr (std::is_same<T, TF16>::value) {
                    const half2_t h01 = {(_Float16)pr[0], (_Float16)pr[1]};
                    const half2_t h23 = {(_Float16)pr[2], (_Float16)pr[3]};
                    const uint2 ph = make_uint2(__builtin_bit_cast(uint32_t, h01),
                                                __builtin_bit_cast(uint32_t, h23));
                    lacc[ct] = mma_pv(T{}, make_uint2(0x3C003C00u, 0x3C003C00u), ph, lacc[ct]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        O[ct][mt] = mma_pv(T{}, vop[t][mt], ph, O[ct][mt]);
                } else {
                    // P as a bf16 hi + lo pair: 16 significant bits
                    const bf162_t h01 = {(__bf16)pr[0], (__bf16)pr[1]};
                    const bf162_t h23 = {(__bf16)pr[2], (__bf16)pr[3]};
                    const bf162_t l01 = {(__bf16)(pr[0] - (float)h01.x),
                                         (__bf16)(pr[1] - (float)h01.y)};
                    const bf162_t l23 = {(__bf16)(pr[2] - (float)h23.x),
                                         (__bf16)(pr[3] - (float)h23.y)};
                    const uint2 ph = make_uint2(__builtin_bit_cast(uint32_t, h01),
                                                __builtin_bit_cast(uint32_t, h23));
                    const uint2 pl = make_uint2(__builtin_bit_cast(uint32_t, l01),
                                                __builtin_bit_cast(uint32_t, l23));
                    lsum[ct] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        O[ct][mt] = mma_pv(T{}, vop[t][mt], ph, O[ct][mt]);
                        O[ct][mt] = mma_pv(T{}, vop[t][mt], pl, O[ct][mt]);
                    }
                }
            }
        }
    }

    // each column's sum over its four lanes, then the normalised rows: the
    // lane holds dims 16 mt + 4 quad + i of its columns
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        float lh;
        if constexpr (kSumByMfma) {
            lh = lacc[ct][0];  // already the column's sum over all its tokens
        } else {
            lh = lsum[ct] + swz_xor16(lsum[ct]);
            lh += xor32(lh);
        }
        if (qi[ct] < nq) {
            const float inv = col_ok[ct] && lh > 0.0f ? 1.0f / lh : 0.0f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int64_t o = orow[ct] + 16 * mt + 4 * quad;
                if (p.out_kind == 0) {
                    *reinterpret_cast<float4_t *>(static_cast<float *>(p.out) + o) = O[ct][mt] * inv;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        store_out(p.out, o + i, O[ct][mt][i] * inv, p.out_kind);
                }
            }
        }
    }
}

template <class T, int D, int BS, int G>
hipError_t launch_prefill_typed(const PrefillArgs &a, hipStream_t stream)
{
    using S = PShape<T, D, BS, G>;
    PrefillParams p;
    p.out = a.out;
    p.out_kind = (int)a.out_dtype;
    p.q = static_cast<const char *>(a.q);
    p.k_cache = static_cast<const char *>(a.k_cache);
    p.v_cache = static_cast<const char *>(a.v_cache);
    p.block_tables = a.block_tables;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.context_lens = a.context_lens;
    p.query_start = a.query_start;
    p.num_query_tokens = a.num_query_tokens;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.num_blocks = a.num_blocks;
    const int64_t cap = (int64_t)a.max_blocks_per_seq * BS;
    p.len_cap = (int32_t)(cap > INT32_MAX ? INT32_MAX : cap);
    p.scale_log2 = a.scale * kLog2e;
    p.num_qblocks = (a.max_query_len + S::QB - 1) / S::QB;
    p.num_pairs = (int64_t)a.num_seqs * a.num_kv_heads;
    const int64_t groups = (p.num_pairs + kXcds - 1) / kXcds * kXcds * p.num_qblocks;
    if (groups > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<T, D, BS, G>), dim3((unsigned)groups), dim3(S::NW * kWave),
                       0, stream, p);
    return hipGetLastError();
}

template <class T, int D, int BS>
hipError_t prefill_group(const PrefillArgs &a, hipStream_t s)
{
    switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefill_typed<T, D, BS, 1>(a, s);
    case 2: return launch_prefill_typed<T, D, BS, 2>(a, s);
    case 4: return launch_prefill_typed<T, D, BS, 4>(a, s);
    case 8: return launch_prefill_typed<T, D, BS, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

template <class T, int D>
hipError_t prefill_block(const PrefillArgs &a, hipStream_t s)
{
    switch (a.block_size) {
    case 16: return prefill_group<T, D, 16>(a, s);
    case 32: return prefill_group<T, D, 32>(a, s);
    }
    return hipErrorInvalidValue;
}

template <class T>
hipError_t prefill_dim(const PrefillArgs &a, hipStream_t s)
{
    switch (a.head_dim) {
    case 64: return prefill_block<T, 64>(a, s);
    case 128: return prefill_block<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(DType kv, int head_dim, int block_size, int group)
{
    return kv != DType::F32 && (head_dim == 64 || head_dim == 128) &&
           (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_paged_prefill(const PrefillArgs &a, hipStream_t stream)
{
    if (a.num_seqs == 0 || a.num_query_tokens == 0 || a.max_query_len == 0)
        return hipSuccess;
    switch (a.kv_dtype) {
    case DType::F16: return prefill_dim<TF16>(a, stream);
    case DType::BF16: return prefill_dim<TBF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pka
