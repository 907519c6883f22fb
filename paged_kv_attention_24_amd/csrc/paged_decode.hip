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
//  * A workgroup of NW wave64s works on an item; the partition is cut into
//    chunks that are dealt round-robin to the waves, and the waves' (max,
//    sum, O) are merged in LDS with log-sum-exp once per item.
//  * Lane layout of a load: a (block, kv head) tile is a contiguous
//    [block_size][head_dim] run, so one wave load of 64 lanes x 16 bytes
//    covers TPL = 64 / LPR whole token rows, LPR = head_dim*elt/16 lanes per
//    row.  Lane l moves 16 bytes (VEC elements) of token l / LPR.
//  * fp16 / bf16 KV run on the matrix cores (mfma_items): each wave copies
//    its chunks of K and V straight from HBM into LDS (global_load_lds,
//    XOR-swizzled rows), one chunk ahead of the one computed.  Per 16-token
//    tile, 16x16x32 MFMAs give the scores of all G heads (K tile times q^T),
//    the online softmax runs in the registers the MFMA wrote, and 16x16x16
//    MFMAs accumulate O^T += V^T P^T, V^T coming from the transposing LDS
//    read.
//  * fp32 KV runs on the vector ALUs (work_item): fp32 FMAs and a DPP
//    butterfly over the LPR lanes of a row give the scores, a single-pass
//    online softmax rescales once per chunk, and o += p V accumulates in
//    fp32; the K and V loads of chunk k+1 are in flight while chunk k is
//    processed.  (A build with PKA_MATRIX_CORES=0 runs half KV this way too,
//    with v_dot2_f32_{f16,bf16} products; it exists to measure against.)
//  * Grids.  With at most kDenseMaxPartitions partitions per sequence, one
//    workgroup per item (a dense grid); when a sequence has several
//    partitions each item writes (max, sum, normalised row) to the workspace
//    and the last one of its (sequence, kv head) to finish, found with a
//    counter, merges them into the output.  With more, a persistent grid of
//    as many workgroups as fit the GPU claims (item, kv head) units from a
//    counter, over a work list planned in each workgroup's LDS (matrix path,
//    up to kPlanInKernelSeqs sequences) or by a one-workgroup plan_kernel;
//    on the matrix path merge_kernel then combines the partitions.
//  * Fused append: for pka_paged_attention_decode_append the item that holds
//    position L_b - 1 stores the sequence's new K/V row in its slot and uses
//    it from registers for that position.
//  * Tokens >= L (the tail of the last block) are excluded by selects, never
//    by multiplying with 0, so stale or NaN slot contents cannot leak.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "cdna4.h"
#include "pka_internal.h"

namespace pka {
namespace {

#ifndef PKA_LOADS_PER_CHUNK
#define PKA_LOADS_PER_CHUNK 4
#endif
#ifndef PKA_PREFETCH_DEPTH
#define PKA_PREFETCH_DEPTH 1
#endif
constexpr int kLoadsPerChunk = PKA_LOADS_PER_CHUNK;  // 1 KiB wave loads per chunk per tensor
constexpr int kPrefetchDepth = PKA_PREFETCH_DEPTH;   // chunks in flight ahead of the one processed
#ifndef PKA_MFMA_CHUNK_KIB
#define PKA_MFMA_CHUNK_KIB 4
#endif
constexpr int kMfmaChunkKiB = PKA_MFMA_CHUNK_KIB;  // KiB of K (and of V) per chunk, matrix path
#ifndef PKA_SPLIT_MERGE
#define PKA_SPLIT_MERGE 1
#endif
constexpr int kSplitMerge = PKA_SPLIT_MERGE;  // persistent grid: merge partitions in a second launch
#ifndef PKA_PERSISTENT_WAVES
#define PKA_PERSISTENT_WAVES 4
#endif
constexpr int kPersistentWaves = PKA_PERSISTENT_WAVES;  // waves per workgroup of the persistent grid
#ifndef PKA_MATRIX_CORES
#define PKA_MATRIX_CORES 1
#endif
// fp16/bf16 KV on the matrix cores (1) or, like fp32 KV, on the vector ALUs
// (0: the build that the matrix path is measured against)
constexpr bool kMatrixCores = PKA_MATRIX_CORES != 0;

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
    int mode;             // 0 dense grid over (j, h, b); 1 persistent grid, work list
                          // planned in the kernel; 2 persistent grid, work list in items
    int32_t num_seqs;
    const int2 *items;    // mode 2: work list {b, j}
    int32_t *wl_header;   // mode 2: [0] next dynamic item, [1] number of {b, j} items
    int32_t *counters;    // per (b, kv head): partitions done; zero between calls
    int32_t *sched;       // modes 1, 2 (matrix path): [0] next unit, [1] finished workgroups
    int split;            // 1: partitions of multi-partition items only store their rows;
                          // merge_kernel combines them after this launch
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
    // half-precision KV runs QK^T and PV on the matrix cores, with K and V
    // staged through LDS; fp32 KV stays on the vector ALUs
    static constexpr bool MFMA = kMatrixCores && !std::is_same<T, TF32>::value;
    // loads per chunk per tensor: kLoadsPerChunk on the vector-ALU path;
    // kMfmaChunkKiB on the matrix path, but at least one 16-token tile
    static constexpr int NL = !MFMA ? kLoadsPerChunk
                              : (kMfmaChunkKiB > 16 * D * ELT / 1024 ? kMfmaChunkKiB : 16 * D * ELT / 1024);
    static constexpr int CT = NL * TPL;            // tokens per chunk
    static constexpr int TILE = BS * D * ELT;      // bytes of one (block, head) tile
    static constexpr int NW = W;                   // waves per workgroup
    static constexpr int STAGE = MFMA ? 2 * 2 * NL * 1024 : 0;  // LDS bytes per wave: 2 chunks of K and V
    static_assert(LPR >= 1 && LPR <= 32 && TPL * LPR == kWave, "row must fit a wave");
    static_assert(BS % TPL == 0, "a wave load must stay inside one block");
};

// LDS of a workgroup.  The dynamic area holds, on the vector-ALU path,
// [NW][G][D] wave rows, then [NW][G] sums and [NW][G] maxima; on the matrix
// path only the sums and maxima.  Two ints (work-list slot, merge flag)
// follow it.  The matrix path has a static staging buffer, two chunks of K
// and V per wave, and merge rows of their own when W <= 4 (a persistent
// workgroup streams the next item's first chunk while it merges); with
// W = 8 (dense grid only) a wave's rows reuse its second chunk buffer.
struct Lds {
    float *smem;
    char *sb[1];
    float *rows;  // matrix path with W <= 4: [NW][G][D] merge rows of their own
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
    if constexpr (!S::MFMA)
        return lds.smem + (size_t)ww * G * D;
    else if constexpr (W <= 4)
        return lds.rows + (size_t)ww * G * D;
    else
        return reinterpret_cast<float *>(lds.sb[0] + (size_t)ww * S::STAGE + S::STAGE / 2);
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

// Workgroups of partition_kernel<...> that fit the device at once with
// `dyn` bytes of dynamic LDS (static staging buffers are counted by the
// runtime); `kind` keys the cache, one entry per distinct `dyn`.
template <class T, int D, int BS, int G, int W>
int resident_workgroups(size_t dyn, int kind)
{
    static int cached[64][2];  // per device ordinal and kind; 0 = not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || kind < 0 || kind > 1)
        return 1024;
    if (cached[dev][kind] == 0) {
        int per_cu = 0;
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, partition_kernel<T, D, BS, G, W>, Shape<T, D, BS, G, W>::NW * kWave, dyn);
        cached[dev][kind] = device_compute_units() * (per_cu > 0 ? per_cu : 1);
    }
    return cached[dev][kind];
}

// Where a work item's tokens lie, as seen by wave w: the tokens
// [j*P, min((j+1)*P, L)) of one (sequence, kv head), cut into chunks of CT
// tokens dealt round-robin to the NW waves.
struct ItemGeom {
    int t_begin, t_end, pb0, last_blk, nk, nparts;
    bool empty;           // no token (and not the lone item of an empty sequence)
    bool app;             // holds position L-1 of a step that appends a token
    int k_last, w_last;   // chunk and wave of position L-1
    int row_app;          // its row inside that chunk
};

template <class T, int D, int BS, int G, int W>
__device__ __forceinline__ ItemGeom item_geom(const PartitionParams &p, int j, int L, int w)
{
    using S = Shape<T, D, BS, G, W>;
    ItemGeom g;
    const int P = p.partition_size;
    g.t_begin = j * P;
    g.pb0 = g.t_begin / BS;
    g.empty = g.t_begin >= L && !(L == 0 && j == 0);
    g.t_end = min(g.t_begin + P, L);
    const int nchunks = g.t_end > g.t_begin ? (g.t_end - g.t_begin + S::CT - 1) / S::CT : 0;
    g.nk = nchunks > w ? (nchunks - w + S::NW - 1) / S::NW : 0;
    g.last_blk = g.t_end > 0 ? (g.t_end - 1) / BS - g.pb0 : 0;
    g.nparts = L == 0 ? 1 : (L + P - 1) / P;
    g.app = !g.empty && p.k_new != nullptr && L > 0 && g.t_end == L;
    const int rel = L - 1 - g.t_begin;
    g.k_last = g.app ? rel / S::CT / S::NW : -1;
    g.w_last = g.app ? rel / S::CT % S::NW : -1;
    g.row_app = g.app ? rel % S::CT : 0;
    // every field is the same in all lanes: keep them in scalar registers
    auto u = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    g.t_begin = u(g.t_begin);
    g.t_end = u(g.t_end);
    g.pb0 = u(g.pb0);
    g.last_blk = u(g.last_blk);
    g.nk = u(g.nk);
    g.nparts = u(g.nparts);
    g.empty = u(g.empty);
    g.app = u(g.app);
    g.k_last = u(g.k_last);
    g.w_last = u(g.w_last);
    g.row_app = u(g.row_app);
    return g;
}

// The partition's block ids (P / BS <= 64 of them), one per lane.  Row
// indices are clamped into the table and ids into the pool, so every later
// access stays in bounds.
__device__ __forceinline__ int load_block_ids(const PartitionParams &p, int b, int pb0)
{
    static_assert(kMaxPartition / 16 <= kWave, "a partition's block ids must fit one wave");
    const int lane = threadIdx.x % kWave;
    const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
    const int idx = pb0 + lane;
    const int id = bt[idx < p.max_blocks_per_seq ? idx : p.max_blocks_per_seq - 1];
    return id < 0 ? 0 : (id > p.num_blocks - 1 ? p.num_blocks - 1 : id);
}

__device__ __forceinline__ int load_len(const PartitionParams &p, int b)
{
    const int L = p.context_lens[b];
    return L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
}

// Store of this lane's 16 bytes of the appended K/V row at slots[b] by the
// first wave (the pool copy is for later steps; the item itself uses the
// row from registers).
template <class T, int D, int BS, int G, int W>
__device__ __forceinline__ void store_new_row(const PartitionParams &p, int b, int h,
                                              const uint4 &kn, const uint4 &vn)
{
    using S = Shape<T, D, BS, G, W>;
    const int lane = threadIdx.x % kWave;
    const int64_t slot = p.slots[b];
    if (threadIdx.x / kWave == 0 && lane / S::LPR == 0 && slot >= 0 && slot < p.num_slots) {
        const int64_t blk = slot / BS;
        const int64_t dst = (blk * p.num_kv_heads + h) * S::TILE + (slot - blk * BS) * (D * S::ELT) +
                            (lane % S::LPR) * 16;
        *reinterpret_cast<uint4 *>(p.k_store + dst) = kn;
        *reinterpret_cast<uint4 *>(p.v_store + dst) = vn;
    }
}

// One output element from the nparts partition rows starting at row0
// (m_j in log2 units): out = sum_j w_j o_j / sum_j w_j with
// w_j = l_j 2^(m_j - max m), as an online merge over batches of 16
// partitions whose loads are all issued before any is used.
struct Combined {
    float m, acc, den;  // running max (log2 units), weighted row sum, weight sum
};
// The nparts partition rows starting at row0, element d: an online merge
// over batches of 16 partitions whose loads are all issued before any is
// used.
template <int D, bool COHERENT>
__device__ __forceinline__ Combined combine_rows(const PartitionParams &p, int64_t row0, int nparts,
                                                 int d)
{
    constexpr int KB = 16;
    auto ld = [&](const float *a) { return COHERENT ? coherent_load(a) : *a; };
    Combined r{-INFINITY, 0.0f, 0.0f};
    for (int j0 = 0; j0 < nparts; j0 += KB) {
        float m[KB], l[KB], o[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int jj = j0 + i;
            const int64_t rr = row0 + (jj < nparts ? jj : nparts - 1);
            m[i] = ld(&p.ws_ml[rr * 2]);
            l[i] = ld(&p.ws_ml[rr * 2 + 1]);
            o[i] = ld(&p.ws_o[rr * D + d]);
        }
        float Mb = r.m;
#pragma unroll
        for (int i = 0; i < KB; ++i)
            Mb = j0 + i < nparts ? fmaxf(Mb, m[i]) : Mb;
        const float sc = r.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(r.m - Mb);
        r.acc *= sc;
        r.den *= sc;
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const float wgt = (j0 + i < nparts && m[i] != -INFINITY)
                                  ? l[i] * __builtin_amdgcn_exp2f(m[i] - Mb)
                                  : 0.0f;
            r.den += wgt;
            r.acc = fmaf(wgt, o[i], r.acc);
        }
        r.m = Mb;
    }
    return r;
}


// The end of a work item, after every wave has written its rows, sums and
// maxima to LDS and the workgroup has passed a barrier: merge the waves
// (log-sum-exp with the wave maxima); with one partition the result is the
// output, else it becomes the partition's row in the workspace and the last
// partition of (b, h) to finish merges all of them.  `issue` runs once the
// item's results have been stored (before the wait that publishes them) and
// returns how many vector memory accesses it issued; those stay in flight.
template <class T, int D, int BS, int G, int W, class Issue>
__device__ __forceinline__ void item_merge(const PartitionParams &p, const Lds &lds, int b, int h,
                                           int j, int nparts_b, float c, const Issue &issue)
{
    using S = Shape<T, D, BS, G, W>;
    constexpr int NW = S::NW;
    const float *lred = wave_sums<T, D, BS, G, W>(lds);
    const float *mred = lred + (size_t)NW * G;
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
    asm volatile("" ::: "memory");  // the stores above stay ahead of issue()'s accesses
    const int issued = issue();
    if (nparts_b == 1 || p.split)
        return;

    // ---- the last partition of (b, h) to finish merges all of them --------
    // With m_j in log2 units: w_j = l_j * 2^(m_j - max m),
    // out = sum_j w_j o_j / sum_j w_j (exact rescaling, log-sum-exp).
    // Publication without an L2 flush: the rows above were written with
    // coherent stores; waiting for their acknowledgement before the
    // workgroup barrier orders them before the counter increment, and the
    // merging workgroup reads them back with coherent loads.
    int *flag = reinterpret_cast<int *>(lds.smem + lds_bytes<T, D, BS, G, W>() / 4) + 2;
    int32_t *counter = p.counters + (int64_t)b * p.num_kv_heads + h;
    wait_vmem_keep(issued);  // this wave's stored rows are acknowledged
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
        const Combined r = combine_rows<D, true>(p, row0, nparts_b, d);
        store_out(p.out, ((int64_t)b * p.num_q_heads + h * G + g) * D + d, r.acc / r.den, p.out_kind);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// prefix[i] = number of work items (partitions) of the sequences before
// sequence i, i = 0..B, in LDS; every thread of the workgroup takes part.
template <int NT>
__device__ __forceinline__ void build_item_prefix(const PartitionParams &p, int *prefix, int *wsum)
{
    const int B = p.num_seqs, P = p.partition_size;
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int per = (B + NT - 1) / NT;
    const int b0 = threadIdx.x * per, b1 = min(b0 + per, B);
    auto parts = [&](int bb) {
        const int L = load_len(p, bb);
        return L == 0 ? 1 : (L + P - 1) / P;
    };
    int local = 0;
    for (int bb = b0; bb < b1; ++bb)
        local += parts(bb);
    int x = local;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off, kWave);
        if (lane >= off)
            x += y;
    }
    if (lane == kWave - 1)
        wsum[wv] = x;
    __syncthreads();
    int run = x - local;
    for (int ww = 0; ww < wv; ++ww)
        run += wsum[ww];
    for (int bb = b0; bb < b1; ++bb) {
        prefix[bb] = run;
        run += parts(bb);
    }
    if (b0 < B && b1 == B)
        prefix[B] = run;
    __syncthreads();
}

// One wave's share of work items on the matrix cores (fp16 / bf16 KV).
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
// and O always use the same reference, so the lazy update is exact.
//
// Mode 0 runs the single item (blockIdx.z, blockIdx.y, blockIdx.x).  Modes 1
// and 2 run a persistent workgroup over a work list of units (item, kv
// head), claimed from a counter; while one item streams, the next one's
// coordinates, length and block ids are fetched, and its first chunk, q and
// appended row are requested before the current item's merge.
template <class T, int D, int BS, int G, int W>
__device__ __forceinline__ void mfma_items(const PartitionParams &p, const Lds &lds)
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
    static_assert(G <= 16 && (size_t)G * D * 4 <= (size_t)CHUNK, "merge rows fit a chunk buffer");

    const int lane = threadIdx.x % kWave;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tg = lane / LPR, cl = lane % LPR;
    const int n = lane % 16, quad = lane / 16;
    const bool head_ok = n < G;
    char *stage = lds.sb[0] + (size_t)w * S::STAGE;  // this wave's [2 buffers][K, V][CHUNK]
    const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(lds_address(stage));
    float *lred = wave_sums<T, D, BS, G, W>(lds);     // [NW][G] softmax sums
    float *mred = lred + (size_t)NW * G;             // [NW][G] maxima, raw dot units
    // Softmax runs on raw dot products scaled by c = |scale| * log2(e) >= 0
    // inside the exponent; a negative scale flips the sign of q instead (exact).
    const float c = fabsf(p.scale_log2);
    const uint32_t qflip = p.scale_log2 < 0.0f ? 0x80008000u : 0u;
    const int64_t block_stride = (int64_t)p.num_kv_heads * S::TILE;

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

    // chunk k of an item -> buffer kd: NL 1 KiB loads of K and of V, each
    // covering TPL whole rows of one block; lane l fills physical unit l%LPR
    // of row l/LPR, i.e. reads that row's logical unit (l%LPR) ^ sw(row)
    auto stage_chunk = [&](int h, const ItemGeom &g, int ids, int k, int buf)
                           __attribute__((always_inline)) {
        const int tc = __builtin_amdgcn_readfirstlane(g.t_begin + (w + k * NW) * CT);
        const int64_t head_off = (int64_t)h * S::TILE;
        const uint32_t kd = __builtin_amdgcn_readfirstlane(stage_lds + buf * (2 * CHUNK));
        const uint32_t vd = kd + CHUNK;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t0 = tc + i * TPL;
            int rb = t0 / BS - g.pb0;
            rb = rb < g.last_blk ? rb : g.last_blk;
            const int blk = __builtin_amdgcn_readlane(ids, rb);
            const int64_t row = (int64_t)blk * block_stride + head_off + (t0 % BS) * R;
            const int rr = i * TPL + tg;
            load_to_lds(p.k_cache + row + tg * R + 16 * (cl ^ swk(rr)), kd + i * 1024);
            load_to_lds(p.v_cache + row + tg * R + 16 * (cl ^ swv(rr)), vd + i * 1024);
        }
    };

    // The first chunk of an item (into chunk buffer buf), then its q^T
    // operand (head n, dims 8*quad + 32*st) and appended row.  Nothing here
    // waits: q gets its sign and padding in stream(), once the first chunk
    // has landed.
    auto prime = [&](int b, int h, const ItemGeom &g, int ids, uint4 (&qop)[KS], uint4 &knew,
                     uint4 &vnew, int buf) __attribute__((always_inline)) {
        int issued = KS + (g.app ? 2 : 0);
        if (g.nk > 0) {
            stage_chunk(h, g, ids, 0, buf);
            issued += 2 * NL;
        }
        const int nn = head_ok ? n : G - 1;
        const char *qrow =
            p.q + (((int64_t)b * p.num_q_heads + h * G + nn) * D + 8 * quad) * S::ELT;
#pragma unroll
        for (int st = 0; st < KS; ++st)
            qop[st] = *reinterpret_cast<const uint4 *>(qrow + 32 * st * S::ELT);
        if (g.app) {
            const int64_t hoff = (int64_t)h * R + cl * 16;
            knew = *reinterpret_cast<const uint4 *>(p.k_new + b * p.k_new_stride + hoff);
            vnew = *reinterpret_cast<const uint4 *>(p.v_new + b * p.v_new_stride + hoff);
        }
        asm volatile("" ::: "memory");  // nothing else joins these accesses
        return issued;
    };

    // Stream an item whose first chunk prime() requested into buffer par;
    // chunk k sits in buffer (par + k) & 1.  last(buf) runs once, in the last
    // chunk's slot for requesting another (or first, with no chunk): it may
    // request the next item's first chunk into buffer buf.  Then write this
    // wave's rows (head n's dims 16*mt + 4*quad + i), sum and maximum.
    auto stream = [&](int h, const ItemGeom &g, int ids, const uint4 (&qraw)[KS], const uint4 &knew,
                      const uint4 &vnew, int par, const auto &last) __attribute__((always_inline)) {
        if (g.nk == 0)
            last(par);
        // q (loaded with the first chunk): sign of the scale, zero padding heads
        uint4 qop[KS];
        if (g.nk > 0)
            wait_vmem();
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            uint4 v = qraw[st];
            v.x ^= qflip;
            v.y ^= qflip;
            v.z ^= qflip;
            v.w ^= qflip;
            qop[st] = select4(head_ok, v, make_uint4(0, 0, 0, 0));
        }
        float4_t O[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            O[mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float mref = -INFINITY, lsum = 0.0f;
        for (int k = 0; k < g.nk; ++k) {
            char *kd = stage + ((par + k) & 1) * (2 * CHUNK);
            char *vd = kd + CHUNK;
            const int tc = g.t_begin + (w + k * NW) * CT;
            wait_vmem();  // chunk k is in LDS; nothing newer has been issued yet
            const bool full = tc + CT <= g.t_end;
            if (!full) {
                // rows past the end: zero V (stale or NaN slots must not reach the sum)
#pragma unroll
                for (int i = 0; i < NL; ++i)
                    if (tc + i * TPL + tg >= g.t_end)
                        *reinterpret_cast<uint4 *>(vd + i * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
            }
            if (g.app && k == g.k_last && w == g.w_last && lane < LPR) {
                // position L-1 takes the new K/V, not the pool
                *reinterpret_cast<uint4 *>(kd + g.row_app * R + 16 * (lane ^ swk(g.row_app))) = knew;
                *reinterpret_cast<uint4 *>(vd + g.row_app * R + 16 * (lane ^ swv(g.row_app))) = vnew;
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
            if (k + 1 < g.nk)
                stage_chunk(h, g, ids, k + 1, (par + k + 1) & 1);
            else
                last((par + k + 1) & 1);

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
                    ok[i] = full || tok0 + i < g.t_end;
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
        // the head's sum over its four lanes; rows into chunk buffer 1
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
    };

    uint4 qop[KS], knew = make_uint4(0, 0, 0, 0), vnew = make_uint4(0, 0, 0, 0);
    if (p.mode == 0) {
        const int b = blockIdx.z, h = blockIdx.y, j = blockIdx.x;
        const int ids = load_block_ids(p, b, j * p.partition_size / BS);
        const int L = load_len(p, b);
        const ItemGeom g = item_geom<T, D, BS, G, W>(p, j, L, w);
        if (g.empty)
            return;  // uniform over the workgroup
        (void)prime(b, h, g, ids, qop, knew, vnew, 0);
        stream(h, g, ids, qop, knew, vnew, 0, [](int) {});
        if (g.app)
            store_new_row<T, D, BS, G, W>(p, b, h, knew, vnew);
        __syncthreads();
        item_merge<T, D, BS, G, W>(p, lds, b, h, j, g.nparts, c, [] { return 0; });
        return;
    }

    // ---- persistent workgroup over the work list --------------------------
    int *slot = reinterpret_cast<int *>(lds.smem + lds_bytes<T, D, BS, G, W>() / 4);  // [2] next unit
    const int hkv = p.num_kv_heads;
    int total;  // units = items * kv heads
    int *prefix = slot + 4;
    if (p.mode == 1) {
        build_item_prefix<NW * kWave>(p, prefix + NW, prefix);  // [NW] wave sums, then [B+1]
        prefix += NW;
        total = prefix[p.num_seqs] * hkv;
    } else {
        total = p.wl_header[1] * hkv;
    }
    // unit -> (sequence, kv head, partition)
    auto locate = [&](int u, int &b, int &h, int &j) __attribute__((always_inline)) {
        const int i = u / hkv;
        h = u - i * hkv;
        if (p.mode == 1) {
            // largest b with prefix[b] <= i: a 64-way step, then the exact one
            const int B = p.num_seqs;
            const int st = (B + kWave - 1) / kWave;
            const int s0 = lane * st < B ? lane * st : B;
            const uint64_t m0 = __builtin_amdgcn_ballot_w64(prefix[s0] <= i);
            const int base = (kWave - 1 - __builtin_clzll(m0)) * st;
            const int s1 = base + lane < B ? base + lane : B;
            const uint64_t m1 = __builtin_amdgcn_ballot_w64(lane < st && prefix[s1] <= i);
            b = base + (kWave - 1 - __builtin_clzll(m1));
            j = i - prefix[b];
        } else {
            const int2 it = p.items[i];
            b = it.x;
            j = it.y;
        }
        b = __builtin_amdgcn_readfirstlane(b);
        j = __builtin_amdgcn_readfirstlane(j);
    };

    int u = blockIdx.x;
    if (u < total) {
        if (threadIdx.x == 0)
            slot[0] = atomicAdd(&p.sched[0], 1) + (int)gridDim.x;
        int b, h, j;
        locate(u, b, h, j);
        int ids = load_block_ids(p, b, j * p.partition_size / BS);
        int L = load_len(p, b);
        ItemGeom g = item_geom<T, D, BS, G, W>(p, j, L, w);
        int par = 0;  // chunk buffer of the current item's first chunk
        (void)prime(b, h, g, ids, qop, knew, vnew, par);
        __syncthreads();
        int un = __builtin_amdgcn_readfirstlane(slot[0]);
        for (int it = 0;; ++it) {
            const bool has_next = un < total;
            // the unit after the next one (published at the end of this item)
            int after = 0;
            if (threadIdx.x == 0 && has_next)
                after = atomicAdd(&p.sched[0], 1) + (int)gridDim.x;
            // the next item's coordinates, length and block ids
            int bn = 0, hn = 0, jn = 0, idsn = 0, Ln = 0;
            if (has_next) {
                locate(un, bn, hn, jn);
                idsn = load_block_ids(p, bn, jn * p.partition_size / BS);
                Ln = load_len(p, bn);
            }
            // The next item's first chunk, q and appended row are requested
            // in this item's last chunk slot, so the chunk stream runs on
            // across the merge below.
            ItemGeom gn = g;
            uint4 qopn[KS], knewn = make_uint4(0, 0, 0, 0), vnewn = make_uint4(0, 0, 0, 0);
            int parn = par;
            auto request_next = [&](int buf) __attribute__((always_inline)) {
                parn = buf;
                if (!has_next)
                    return;
                gn = item_geom<T, D, BS, G, W>(p, jn, Ln, w);
                (void)prime(bn, hn, gn, idsn, qopn, knewn, vnewn, buf);
            };
            if (!g.empty) {
                stream(h, g, ids, qop, knew, vnew, par, request_next);
                if (g.app)
                    store_new_row<T, D, BS, G, W>(p, b, h, knew, vnew);
                __syncthreads();
                // (the next item's accesses are older than this item's
                // stores, so a publishing wait covers them too)
                item_merge<T, D, BS, G, W>(p, lds, b, h, j, g.nparts, c, [] { return 0; });
            } else {
                request_next(par);
            }
            if (threadIdx.x == 0 && has_next)
                slot[(it + 1) & 1] = after;
            __syncthreads();
            if (!has_next)
                break;
            un = __builtin_amdgcn_readfirstlane(slot[(it + 1) & 1]);
            b = bn;
            h = hn;
            j = jn;
            ids = idsn;
            L = Ln;
            g = gn;
            par = __builtin_amdgcn_readfirstlane(parn);
#pragma unroll
            for (int st = 0; st < KS; ++st)
                qop[st] = qopn[st];
            knew = knewn;
            vnew = vnewn;
        }
    }
    // The last workgroup to finish resets the scheduler for the next call.
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(&p.sched[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            (int)gridDim.x - 1) {
        __hip_atomic_store(&p.sched[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.sched[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One work item on the vector ALUs (fp32 KV): the tokens
// [j*P, min((j+1)*P, L_b)) of kv head h of sequence b, for all G query heads
// of the group.  Called by every thread of the workgroup with the same
// (b, h, j).
template <class T, int D, int BS, int G, int W>
__device__ __forceinline__ void work_item(const PartitionParams &p, int b, int h, int j,
                                          const Lds &lds)
{
    using S = Shape<T, D, BS, G, W>;
    constexpr int NW = S::NW, LPR = S::LPR, TPL = S::TPL, NL = S::NL, CT = S::CT, VEC = S::VEC;

    const int lane = threadIdx.x % kWave;
    // wave index, provably uniform: block ids and chunk bounds stay scalar
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tg = lane / LPR, cl = lane % LPR;
    const int P = p.partition_size;
    const int t_begin = j * P;
    const int pb0 = t_begin / BS;
    const int ids = load_block_ids(p, b, pb0);  // requested together with the length
    const int L = load_len(p, b);
    const ItemGeom gm = item_geom<T, D, BS, G, W>(p, j, L, w);
    if (gm.empty)
        return;  // uniform over the workgroup
    const int t_end = gm.t_end;
    const int nk = gm.nk;
    const int last_blk = gm.last_blk;

    // Appended token: the item holding position L-1 stores the new K/V row
    // at slots[b] and uses it from registers for that position, so no other
    // workgroup ever has to see the store.
    const bool app = gm.app;
    int k_last = -1, w_last = -1, i_last = 0, tg_last = 0;
    if (app) {
        k_last = gm.k_last;
        w_last = gm.w_last;
        i_last = gm.row_app / TPL;
        tg_last = gm.row_app % TPL;
    }
    auto load_new = [&](uint4 &kn, uint4 &vn) {
        const int64_t hoff = (int64_t)h * D * S::ELT + cl * 16;
        kn = *reinterpret_cast<const uint4 *>(p.k_new + b * p.k_new_stride + hoff);
        vn = *reinterpret_cast<const uint4 *>(p.v_new + b * p.v_new_stride + hoff);
    };
    auto store_new = [&](const uint4 &kn, const uint4 &vn) {
        store_new_row<T, D, BS, G, W>(p, b, h, kn, vn);
    };

    // Softmax runs on raw dot products scaled by c = |scale| * log2(e) >= 0
    // inside the exponent; a negative scale flips the sign of q instead (exact).
    const float c = fabsf(p.scale_log2);
    const uint32_t qflip = p.scale_log2 < 0.0f ? (S::ELT == 4 ? 0x80000000u : 0x80008000u) : 0u;
    const int64_t head_off = (int64_t)h * S::TILE;
    const int64_t block_stride = (int64_t)p.num_kv_heads * S::TILE;
    float *lred = wave_sums<T, D, BS, G, W>(lds);  // [NW][G] softmax sums
    float *mred = lred + (size_t)NW * G;          // [NW][G] maxima, raw dot units

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
    __syncthreads();
    item_merge<T, D, BS, G, W>(p, lds, b, h, j, gm.nparts, c, [] { return 0; });
}

template <class T, int D, int BS, int G, int W>
// (the matrix path asks the compiler for two waves per SIMD: 8 / W workgroups per CU)
__global__ __launch_bounds__((Shape<T, D, BS, G, W>::NW * kWave),
                             (Shape<T, D, BS, G, W>::MFMA ? 8 / W : 1)) void partition_kernel(PartitionParams p)
{
    using S = Shape<T, D, BS, G, W>;
    extern __shared__ float smem[];
    __shared__ __attribute__((aligned(1024))) char sb0[S::MFMA ? S::STAGE * S::NW : 16];
    __shared__ __attribute__((aligned(16))) float rows0[S::MFMA && W <= 4 ? W * G * D : 4];
    const Lds lds{smem, {sb0}, rows0};
    if constexpr (S::MFMA) {
        mfma_items<T, D, BS, G, W>(p, lds);
        return;
    }
    if (p.mode == 0) {
        work_item<T, D, BS, G, W>(p, blockIdx.z, blockIdx.y, blockIdx.x, lds);
        return;
    }
    // Work-list mode on the vector ALUs: a persistent grid.  Workgroup g
    // starts with item g and then takes the next unclaimed item from the
    // counter the plan kernel initialised to the grid size.
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

// Combine the partition rows of every (sequence, kv head) with more than one
// partition (log-sum-exp, as in item_merge): one workgroup per (h, b), one
// thread per (query head of the group, dim).
template <int D, int G>
__global__ __launch_bounds__(G * D) void merge_kernel(PartitionParams p)
{
    const int h = blockIdx.x, b = blockIdx.y;
    const int L = load_len(p, b);
    const int nparts_b = L == 0 ? 1 : (L + p.partition_size - 1) / p.partition_size;
    if (nparts_b == 1)
        return;  // written by its only partition
    const int g = threadIdx.x / D, d = threadIdx.x % D;
    const int64_t row0 = ((int64_t)b * p.num_q_heads + h * G + g) * p.num_partitions;
    const Combined r = combine_rows<D, false>(p, row0, nparts_b, d);
    store_out(p.out, ((int64_t)b * p.num_q_heads + h * G + g) * D + d, r.acc / r.den, p.out_kind);
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
    p.num_seqs = a.num_seqs;
    p.sched = a.counters + kMaxCompletionCounters;
    p.mode = 0;
    p.split = 0;

    // dynamic LDS: sums and maxima, then 4 ints (next-unit slots, merge flag),
    // then (in-kernel plan) NW wave sums and the item prefix of B + 1 ints
    const size_t lds = lds_bytes<T, D, BS, G, W>() + 16;
    const size_t lds_plan = lds + (size_t)(S::NW + kPlanInKernelSeqs + 1) * 4;
    hipError_t e;
    if (a.items) {
        const int64_t dense = (int64_t)a.num_partitions * a.num_kv_heads * a.num_seqs;
        if (S::MFMA && W > 4)
            return hipErrorInvalidValue;  // persistent grids stream across items: W <= 4
        if (S::MFMA && a.num_seqs <= kPlanInKernelSeqs) {
            // persistent grid, work list planned in the kernel; partitions
            // only store their rows and merge_kernel combines them
            p.mode = 1;
            p.split = kSplitMerge;
            const int64_t res = resident_workgroups<T, D, BS, G, W>(lds_plan, 1);
            const int grid = (int)(dense < res ? dense : res);
            hipLaunchKernelGGL((partition_kernel<T, D, BS, G, W>), dim3(grid), dim3(S::NW * kWave),
                               lds + (size_t)(S::NW + a.num_seqs + 1) * 4, stream, p);
            e = hipGetLastError();
            if (e != hipSuccess || !p.split)
                return e;
            hipLaunchKernelGGL((merge_kernel<D, G>), dim3(a.num_kv_heads, a.num_seqs), dim3(G * D), 0,
                               stream, p);
            return hipGetLastError();
        }
        p.mode = 2;
        p.split = S::MFMA ? kSplitMerge : 0;
        const int64_t res = resident_workgroups<T, D, BS, G, W>(lds, 0);
        const int grid = (int)(dense < res ? dense : res);
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.context_lens,
                           a.num_seqs, a.partition_size, p.len_cap, a.items, a.wl_header, grid);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL((partition_kernel<T, D, BS, G, W>), dim3(grid), dim3(S::NW * kWave), lds,
                           stream, p);
        e = hipGetLastError();
        if (e != hipSuccess || !p.split)
            return e;
        hipLaunchKernelGGL((merge_kernel<D, G>), dim3(a.num_kv_heads, a.num_seqs), dim3(G * D), 0,
                           stream, p);
    } else {
        const dim3 grid((unsigned)a.num_partitions, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
        hipLaunchKernelGGL((partition_kernel<T, D, BS, G, W>), grid, dim3(S::NW * kWave), lds, stream,
                           p);
    }
    return hipGetLastError();
}

// Waves per workgroup.  fp32 KV (and half KV in a vector-ALU build): 4, or 2
// where the register state of a wave is large.  Half KV (matrix cores): 8 when the grid of work
// items is no larger than the number of compute units (a short batch is
// latency-bound, so each item gets more waves), else 4 (more items resident
// per compute unit).
template <class T, int D, int BS, int G>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s)
{
    if constexpr (std::is_same<T, TF32>::value || !kMatrixCores) {
        constexpr int TPL = kWave / (D * T::kBytes / 16);
        return launch_waves<T, D, BS, G, (G * D * TPL * 4 * 4 > 48 * 1024) ? 2 : 4>(a, s);
    } else {
        const int64_t items = (int64_t)a.num_partitions * a.num_kv_heads * a.num_seqs;
        if (a.items == nullptr && items <= device_compute_units())
            return launch_waves<T, D, BS, G, 8>(a, s);
        if (a.items != nullptr)
            return launch_waves<T, D, BS, G, kPersistentWaves>(a, s);
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
