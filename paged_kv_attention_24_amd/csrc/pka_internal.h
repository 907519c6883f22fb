// Internal interface between the C-ABI layer (abi.cpp) and the kernel
// translation units.  Not installed; the public surface is include/pka.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pka {

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

inline int dtype_bytes(DType t) { return t == DType::F32 ? 4 : 2; }

struct WriteArgs {
    const void *k, *v;
    int64_t k_token_stride, v_token_stride;  // elements
    const int64_t *slot_mapping;
    int32_t num_tokens;
    void *k_cache, *v_cache;
    int32_t num_blocks, block_size, num_kv_heads, head_dim;
    DType dtype;
    // rotary embedding of the new keys (positions null: a plain write)
    const int32_t *positions = nullptr;  // [num_tokens]
    const float *cos_sin = nullptr;      // [max_position][rotary_dim]: cos, then sin
    int32_t max_position = 0, rotary_dim = 0;
};

hipError_t launch_kv_cache_write(const WriteArgs &a, hipStream_t stream);

struct DecodeArgs {
    void *out;
    DType out_dtype;
    const void *q, *k_cache, *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
    int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
    int32_t num_blocks, block_size;
    float scale;
    DType kv_dtype;
    int32_t partition_size;   // smallest number of tokens one wave takes; 0: library default
    int32_t context_hint;     // caller's bound on the lengths (max_context_len; 0: none):
                              // picks the launch shape only, never cuts a sequence short
    float *parts;             // [2 * max_waves] partial results of decode_part_floats(G, D)
    int32_t *counters;        // [num_seqs][num_kv_heads] report counters (kCounterStride apart), zero before and after
    int64_t max_waves;        // waves the partial-result slots cover
    // optional appended token per sequence (k_new null: plain decode)
    const void *k_new, *v_new;
    int64_t k_new_token_stride, v_new_token_stride;  // elements
    const int64_t *slot_mapping;
};

// The decode plans its work in the kernel from a prefix of chunk counts per
// sequence kept in LDS, so one launch takes at most this many sequences;
// the C ABI cuts longer batches into launches of this size.
constexpr int kMaxSeqsPerLaunch = 2040;
// Decode workgroups resident per compute unit (LDS staging of 4 waves x
// 16 KiB, plus the prefix) and the waves the partial-result slots cover.
constexpr int kMaxWorkgroupsPerCU = 2;
// Smallest number of tokens (of any mix of pairs) one decode wave takes by
// default: fewer, longer ranges mean fewer partial results to combine.
constexpr int kDefaultRangeTokens = 64;
// Work units of the decode's split.  A chunk weighs kUnitsPerChunk and each
// (sequence, kv head) pair adds kUnitsPerPair for its fixed cost (staging q,
// finishing and publishing the result), so a wave whose range touches many
// short pairs takes fewer chunks.  One chunk's weight per pair measured best
// on a log-uniform mix of lengths (half a chunk and three quarters were 2%
// slower there; long uniform pairs are indifferent).
constexpr int kUnitsPerChunk = 4;
constexpr int kUnitsPerPair = 4;

// Floats of one decode partial result: the unnormalised output [G][D], then
// the running maxima [G] and sums [G], padded to 16 bytes so that every
// partial result and output row starts 16-byte aligned.
constexpr int64_t decode_part_floats(int64_t group, int64_t head_dim)
{
    return group * head_dim + (2 * group + 3) / 4 * 4;
}

// Waves of the decode grid on the current device (2 slots of partial
// results each).
int decode_max_waves();

// The decode workspace starts with this many bytes of report counters (one
// int32 per (sequence, kv head) of a launch), zero before and after every
// call; a fixed size keeps them in place whatever the shapes, so one
// workspace serves calls of any shape.  Partial results follow.  Each
// counter has a 128-byte line to itself: atomics on one line are served one
// after another, so counters sharing a line would queue behind each other.
constexpr int64_t kCounterBytes = 4 << 20;
constexpr int64_t kCounterStride = 32;  // int32s between counters (128 bytes)
constexpr int64_t kMaxCounters = kCounterBytes / 4 / kCounterStride;

// Byte offsets of the decode workspace: report counters, then partial
// results (256-byte aligned starts).
struct WorkspaceLayout {
    size_t counter_offset, parts_offset, total;
};
WorkspaceLayout decode_workspace_layout(int64_t num_seqs, int64_t num_q_heads,
                                        int64_t num_kv_heads, int64_t head_dim, int64_t max_waves);

// Whether (dtype, head_dim, block_size, group) has a compiled kernel.
bool decode_supported(DType kv, int head_dim, int block_size, int group);

// Largest partition the INT8 kernels accept (bounds their LDS use).
constexpr int kMaxPartition = 1024;

hipError_t launch_paged_decode(const DecodeArgs &a, hipStream_t stream);

// Multi-token causal paged attention (chunked prefill, drafted-token check).
struct PrefillArgs {
    void *out;
    DType out_dtype;
    const void *q, *k_cache, *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
    const int32_t *query_start;  // [num_seqs + 1], device
    int32_t num_seqs, num_query_tokens, max_query_len;
    int32_t num_q_heads, num_kv_heads, head_dim;
    int32_t num_blocks, block_size;
    float scale;
    DType kv_dtype;
};

bool prefill_supported(DType kv, int head_dim, int block_size, int group);
hipError_t launch_paged_prefill(const PrefillArgs &a, hipStream_t stream);

// Whole-block copies between and inside the pools (preemption, paging).
enum class BlockMove : int { Copy = 0, Gather = 1, Scatter = 2 };
struct BlockMoveArgs {
    BlockMove mode;
    void *k_cache, *v_cache;
    void *packed;          // gather: written, scatter: read; [n][2][block_bytes]
    const int64_t *ids;    // copy: [n][2] (src, dst); gather, scatter: [n]
    int64_t num_entries;   // n
    int64_t num_blocks;
    int64_t block_bytes;   // multiple of 16
};

hipError_t launch_move_blocks(const BlockMoveArgs &a, hipStream_t stream);

// Group-quantised INT8 pools: k_codes, v_codes int8 [NB][Hkv][BS * D] (each
// block's run of codes in 16-token tiles, ordered as the matrix-core
// products read them; the order is spelled out in pka.h), k_scales /
// v_scales f32 [NB][Hkv][BS][D / group_size].
struct Int8WriteArgs {
    const void *k, *v;
    int64_t k_token_stride, v_token_stride;  // elements
    DType dtype;                              // of k and v
    const int64_t *slot_mapping;
    int32_t num_tokens;
    int8_t *k_codes, *v_codes;
    float *k_scales, *v_scales;
    int32_t num_blocks, block_size, num_kv_heads, head_dim, group_size;
};

hipError_t launch_kv_cache_write_int8(const Int8WriteArgs &a, hipStream_t stream);

struct Int8DecodeArgs {
    void *out;
    int out_kind;  // 0 f32, 1 f16, 2 bf16
    const void *q;
    DType q_dtype;  // F16 or BF16
    const int8_t *k_codes, *v_codes;
    const float *k_scales, *v_scales;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
    int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, group_size;
    float scale_log2;         // scale * log2(e)
    int32_t len_cap;          // lengths are clamped to [0, len_cap]
    int32_t partition_size;   // tokens, multiple of block_size, <= kMaxPartition
    int32_t num_partitions;   // ceil(max length / partition_size)
    // workspace (num_partitions > 1)
    float *ws_o;              // [B][Hq][num_partitions][D]
    float *ws_ml;             // [B][Hq][num_partitions][2]: max (log2 units), sum
    int2 *items;              // [B * num_partitions] planned (b, partition)
    int32_t *wl_header;       // [0]: item count
    // fused append (k_new null: plain decode): rows [B][Hkv][D] of q_dtype
    const void *k_new = nullptr, *v_new = nullptr;
    int64_t k_new_stride = 0, v_new_stride = 0;  // elements
    const int64_t *slot_mapping = nullptr;
};

// Byte offsets of the INT8 decode workspace (zero total for one partition).
struct Int8WorkspaceLayout {
    size_t header_offset, items_offset, ml_offset, o_offset, total;
};
Int8WorkspaceLayout int8_workspace_layout(int64_t num_seqs, int64_t num_q_heads,
                                          int64_t head_dim, int64_t num_partitions);

hipError_t launch_paged_decode_int8(const Int8DecodeArgs &a, hipStream_t stream);

}  // namespace pka
