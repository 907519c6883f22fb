/*
 * pka.h -- C ABI of the paged KV attention library for AMD Instinct MI355X
 * (gfx950).
 *
 * Operations described in the PhotonInfer README (Korean translation):
 *   - "Technical details > Paged attention": the KV cache is managed in
 *     fixed-size blocks without fragmentation, each sequence keeps its own
 *     cache offsets, and one kernel performs the K/V writes of many
 *     sequences at once  ->  pka_kv_cache_write.
 *   - "Key features > GPU-optimised kernels": batched paged attention over
 *     that block-wise cache, with a numerically stable softmax
 *     ->  pka_paged_attention_decode (and, fused with the write of one new
 *     token per sequence, pka_paged_attention_decode_append).
 *   - Its multi-token form, for prompts admitted chunk by chunk and for
 *     drafted tokens ("Continuous batching scheduler", "Roadmap")
 *     ->  pka_paged_attention_prefill.
 *   - "Key features > GPU-optimised kernels" also lists batched RoPE among
 *     the fused operations  ->  pka_kv_cache_write_rope.
 *   - Block movement for preempted requests and paging
 *     ->  pka_copy_blocks, pka_gather_blocks, pka_scatter_blocks.
 *   - "Technical details > INT8 quantisation" (group-wise INT8 with groups
 *     of 32, 64 or 128), applied to the KV cache
 *     ->  pka_kv_cache_write_int8, pka_paged_attention_decode_int8,
 *     pka_paged_attention_decode_append_int8.
 *
 * Conventions (same README, "Modern C++20 architecture": explicit error
 * results instead of exceptions, zero-copy borrowed buffers):
 *   - Every pointer named "device" is a device (HBM) pointer owned by the
 *     caller; the library never frees or retains it.  The library allocates
 *     no device memory: the decode's scratch workspace is passed in.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     default stream) and returns without synchronising.
 *   - Every call returns a pka_status.  Argument problems that the host can
 *     see are reported before anything is launched; a failed launch returns
 *     PKA_ERR_HIP.  pka_last_error() then gives a thread-local message.
 *   - The contents of device buffers (block ids, lengths, slots) are the
 *     caller's contract and are not validated on the hot path; the kernels
 *     clamp them so that no access ever leaves the buffers described by the
 *     arguments (see each call).
 *
 * KV pool layout (both pools, one layout):
 *   k_cache, v_cache: [num_blocks][num_kv_heads][block_size][head_dim],
 *   row-major, contiguous, 16-byte aligned.  Token t of a sequence whose
 *   block table row is bt[] lives in physical block bt[t / block_size], at
 *   offset t % block_size.  A slot number names one token position of the
 *   pool: slot = block * block_size + offset.
 *
 * Query heads are grouped contiguously onto kv heads: query head hq reads
 * kv head hq / (num_q_heads / num_kv_heads).
 */
#ifndef PKA_H
#define PKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKA_ABI_VERSION 8

/* Both enums are 32-bit codes.  The *_RANGE_* members are not values to
 * pass: they make every int32 a value of the type, so that a code the
 * library does not know (reported as such) is still a defined value. */
typedef enum pka_status {
    PKA_OK = 0,
    PKA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, shape or alignment */
    PKA_ERR_UNSUPPORTED = 2,        /* valid but outside the compiled set */
    PKA_ERR_WORKSPACE_TOO_SMALL = 3,
    PKA_ERR_HIP = 4,                /* the HIP runtime reported an error */
    PKA_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
    PKA_STATUS_RANGE_MAX_ = 0x7fffffff
} pka_status;

typedef enum pka_dtype {
    PKA_F32 = 0,
    PKA_F16 = 1,   /* IEEE binary16 */
    PKA_BF16 = 2,  /* bfloat16 */
    PKA_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
    PKA_DTYPE_RANGE_MAX_ = 0x7fffffff
} pka_dtype;

/*
 * pka_kv_cache_write -- store the K and V rows of num_tokens new tokens,
 * belonging to any number of sequences, into the block pools in one launch.
 *
 * For each token i with s = slot_mapping[i] and 0 <= s < num_blocks *
 * block_size: for every kv head h, the head_dim elements
 * k[i * k_token_stride + h * head_dim + d] (d < head_dim) are copied bit for
 * bit to k_cache[s / block_size][h][s % block_size][d]; likewise v into
 * v_cache.  No dtype conversion happens.  A negative slot marks padding and
 * is skipped; a slot at or beyond num_blocks * block_size is skipped as well
 * (nothing outside the pools is ever written).  Two tokens with the same
 * slot race: which one lands is unspecified.  Every other byte of both pools
 * is left untouched.
 *
 *   k, v            device, [num_tokens][num_kv_heads][head_dim] with token
 *                   strides k_token_stride / v_token_stride (in elements,
 *                   >= num_kv_heads * head_dim); heads are head_dim apart.
 *                   Base pointers 16-byte aligned; token strides times the
 *                   element size multiples of 16 bytes.
 *   slot_mapping    device, int64 [num_tokens].
 *   k_cache,v_cache device, written in place (layout above).
 *   dtype           element type of k, v and both pools.
 * Supported: head_dim in {64, 128}; block_size in {16, 32}; any num_kv_heads
 * >= 1; num_tokens >= 0 (0 launches nothing).
 */
pka_status pka_kv_cache_write(const void *k, const void *v, int64_t k_token_stride,
                              int64_t v_token_stride, const int64_t *slot_mapping,
                              int32_t num_tokens, void *k_cache, void *v_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_dim, pka_dtype dtype, void *stream);

/*
 * pka_kv_cache_write_rope -- pka_kv_cache_write with the rotary position
 * embedding applied to the new keys on their way into the pool (PhotonInfer
 * README, Korean translation, "Key features > GPU-optimised kernels":
 * batched RoPE among the fused operations).  Token i at position
 * p = positions[i] has each K row x stored as y, for j < R/2
 * (R = rotary_dim):
 *   y[j]       = x[j] c_j - x[j + R/2] s_j,
 *   y[j + R/2] = x[j + R/2] c_j + x[j] s_j,
 *   c_j = cos_sin[p][j], s_j = cos_sin[p][R/2 + j],
 * computed in fp32 (each product and sum rounded, no fused multiply-add) and
 * rounded to nearest even into the pool dtype; dims >= R and the V rows are
 * stored unchanged.  The table is the caller's, so the angle schedule (base,
 * frequency scaling) is too.
 *   positions   device, int32 [num_tokens].  A position outside
 *               [0, max_position) skips the token (nothing is stored).
 *   cos_sin     device, float [max_position][rotary_dim]: per position the
 *               R/2 cosines, then the R/2 sines.
 *   rotary_dim  even, <= head_dim, a multiple of 16 (fp16/bf16) or 8 (fp32).
 * Everything else as for pka_kv_cache_write.
 */
pka_status pka_kv_cache_write_rope(const void *k, const void *v, int64_t k_token_stride,
                                   int64_t v_token_stride, const int64_t *slot_mapping,
                                   const int32_t *positions, int32_t num_tokens,
                                   const float *cos_sin, int32_t max_position, int32_t rotary_dim,
                                   void *k_cache, void *v_cache, int32_t num_blocks,
                                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                   pka_dtype dtype, void *stream);

/*
 * pka_decode_partition_size -- the default of pka_paged_attention_decode's
 * partition_size argument: the fewest tokens (summed over the (sequence, kv
 * head) pairs it touches) that one wave of the decode takes.  Pure host
 * function of the shapes.
 */
int32_t pka_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                  int32_t max_context_len);

/*
 * pka_decode_workspace_bytes -- bytes of device scratch
 * pka_paged_attention_decode (and _append) needs for these shapes on the
 * current device: 4 MiB of report counters (one per 128-byte line), then
 * two partial-result slots
 * per wave of the decode grid, each of G * head_dim output floats and 2 G
 * (max, sum) floats padded to a multiple of 4 (G = num_q_heads /
 * num_kv_heads).  It does not depend on the context lengths.  0 when
 * num_seqs <= 0.
 */
size_t pka_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim);

/*
 * pka_paged_attention_decode -- one query token per sequence attends over
 * that sequence's cached tokens, for the whole batch:
 *
 *   out[b][hq][:] = sum_{t < L_b} softmax_t(scale * q[b][hq][:] . K_t) V_t
 *
 * with L_b = context_lens[b], K_t/V_t the rows of token t of sequence b in
 * kv head hq / (num_q_heads / num_kv_heads), found through block_tables[b].
 * Softmax is computed stably (running max subtracted, fp32 throughout);
 * products and sums accumulate in fp32.  L_b <= 0 yields a zero row.
 *
 * How the work is split (split-context partitions): the tokens of all
 * (sequence, kv head) pairs form one flat sequence of chunks, and every wave
 * of the grid takes a contiguous share of equal work (each chunk, plus a
 * fixed cost per pair it touches), so long sequences are cut into
 * partitions wherever the shares end.  A wave that holds only part
 * of a pair leaves its running max, sum and unnormalised output in the
 * workspace; the last wave to finish with that pair combines the parts
 * exactly (log-sum-exp) in the same launch.  The result does not depend on
 * the split beyond fp32 rounding.  Batches of more than 2040 sequences run as
 * several launches on `stream`.  Small batches take the pair mode described
 * under partition_size.
 *
 *   out             device, [num_seqs][num_q_heads][head_dim], contiguous,
 *                   of out_dtype (PKA_F32, or the KV dtype: rounded to
 *                   nearest even).
 *   q               device, [num_seqs][num_q_heads][head_dim], contiguous,
 *                   of the KV dtype.
 *   k_cache,v_cache device pools (layout above), of kv_dtype.
 *   block_tables    device, int32 [num_seqs][max_blocks_per_seq].  Entries
 *                   at index >= ceil(L_b / block_size) are never used.  A
 *                   used entry outside [0, num_blocks) is clamped into range
 *                   (the row's result is then meaningless, but no access
 *                   leaves the pools).
 *   context_lens    device, int32 [num_seqs].  Lengths are clamped on the
 *                   device to [0, max_blocks_per_seq * block_size].
 *   scale           multiplier of the dot products (typically 1/sqrt(D)); any
 *                   finite value (NaN and +-inf give PKA_ERR_INVALID_ARGUMENT)
 *                   whose products scale * q . K stay within float32 range.
 *                   0 gives the plain mean of V over the tokens, a negative
 *                   value flips the logits.
 *   max_context_len optional host bound on the lengths (<= 0: none).  It
 *                   only helps pick the launch shape: no length is ever cut
 *                   short by it (a length above it is still computed).
 *   partition_size  0: the library picks the split: with at most as many
 *                   (sequence, kv head) pairs as compute units and lengths
 *                   of at most 2048 tokens (by max_context_len, else by the
 *                   table width), each pair gets one workgroup whose waves
 *                   share its chunks and combine in LDS (no workspace
 *                   traffic); otherwise the flat split below with
 *                   pka_decode_partition_size() tokens.  Else a positive
 *                   multiple of block_size: the flat split, the fewest
 *                   tokens one wave takes (fewer, longer shares leave fewer parts to
 *                   combine).
 *   workspace       device scratch of workspace_bytes >=
 *                   pka_decode_workspace_bytes(...), 256-byte aligned.  Its
 *                   leading report counters must be zero before the first
 *                   call using this workspace: zero-fill a new workspace
 *                   once.  Every call leaves them zero again, so a workspace
 *                   can be reused by later calls of any shape on the same
 *                   stream (or in a captured graph); calls that share one
 *                   workspace on different streams race.  The rest is
 *                   overwritten by each call.
 * Supported: kv_dtype in {F32, F16, BF16}; head_dim in {64, 128};
 * block_size in {16, 32}; num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 */
pka_status pka_paged_attention_decode(void *out, pka_dtype out_dtype, const void *q,
                                      const void *k_cache, const void *v_cache,
                                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t num_blocks, int32_t block_size, float scale,
                                      pka_dtype kv_dtype, int32_t max_context_len,
                                      int32_t partition_size, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * pka_paged_attention_decode_noalloc -- pka_paged_attention_decode without
 * a workspace argument and without any device allocation, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * The report counters and partial results live in a static device array of
 * PKA_DECODE_STATIC_SCRATCH_BYTES bytes that the library holds on every GPU
 * it runs on until the process ends.  The first call on a device takes that
 * array's address and clears its counters (a fill kernel on `stream`); each
 * call leaves them zero again.  All calls on one GPU share the array: calls
 * that overlap on one GPU (different streams, or threads without ordering)
 * race and give unspecified results.  Arguments and results are those of
 * pka_paged_attention_decode (same kernels, bit-identical output).
 * Returns PKA_ERR_WORKSPACE_TOO_SMALL when the shapes need more scratch than
 * the array holds (pka_decode_workspace_bytes() above the limit: not the
 * case for any supported shape on a GPU of up to 256 compute units), and
 * PKA_ERR_HIP when the array's address cannot be obtained.
 */
#define PKA_DECODE_STATIC_SCRATCH_BYTES (22u << 20)
pka_status pka_paged_attention_decode_noalloc(
    void *out, pka_dtype out_dtype, const void *q, const void *k_cache, const void *v_cache,
    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, int32_t block_size, float scale, pka_dtype kv_dtype,
    int32_t max_context_len, int32_t partition_size, void *stream);

/*
 * pka_paged_attention_decode_append -- one decode step of a batch in a
 * single launch: for every sequence b, store its new token's K/V rows
 * (k_new[b], v_new[b]) at slot_mapping[b] and attend over its L_b tokens,
 * the last of which (position L_b - 1) is that new token:
 *
 *   out[b][hq] = sum_{t < L_b} softmax_t(scale * q[b][hq] . K_t) V_t,
 *   K_t, V_t from the pools for t < L_b - 1 and from k_new[b], v_new[b]
 *   for t = L_b - 1.
 *
 * This is the batched write of the PhotonInfer README ("Technical details >
 * Paged attention": one kernel for the K/V writes of many sequences) fused
 * with the batched decode ("Key features > GPU-optimised kernels").  When
 * slot_mapping[b] is the slot of position L_b - 1 of sequence b (the usual
 * decode step), the pools and the output are bit-identical to
 * pka_kv_cache_write followed by pka_paged_attention_decode.
 *
 *   q, out, pools, block_tables, context_lens, scale, max_context_len,
 *   partition_size, workspace: as for pka_paged_attention_decode (the pools
 *   are written, so they are not const here).
 *   k_new, v_new    device, [num_seqs][num_kv_heads][head_dim] of kv_dtype,
 *                   token strides k_new_token_stride / v_new_token_stride
 *                   (elements, >= num_kv_heads * head_dim, rows 16-byte
 *                   aligned), heads head_dim apart.
 *   slot_mapping    device, int64 [num_seqs].  A negative slot, or one at or
 *                   beyond num_blocks * block_size, stores nothing (the new
 *                   token still takes part in the attention).  Sequences
 *                   with L_b <= 0 store nothing and yield a zero row.  A slot
 *                   that this call reads for another position of any
 *                   sequence races with the store (unspecified result).
 * Supported: as for pka_paged_attention_decode.
 */
pka_status pka_paged_attention_decode_append(
    void *out, pka_dtype out_dtype, const void *q, const void *k_new, const void *v_new,
    int64_t k_new_token_stride, int64_t v_new_token_stride, const int64_t *slot_mapping,
    void *k_cache, void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_blocks, int32_t block_size, float scale, pka_dtype kv_dtype,
    int32_t max_context_len, int32_t partition_size, void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * pka_paged_attention_prefill -- multi-token causal attention over the
 * block-wise cache: the prefill of a chunk of a prompt, or the check of
 * several drafted tokens, for a batch of sequences in one launch.  The
 * PhotonInfer README (Korean translation) schedules requests token by token
 * ("Continuous batching scheduler": num_computed_tokens) and lists
 * speculative decoding on its "Roadmap"; the JackerLab "vllm" tag page
 * ("Speculative Decoding") describes a large model checking several proposed
 * tokens at once.  Sequence b brings T_b = query_start[b+1] - query_start[b]
 * new tokens whose K/V are already in the pools (pka_kv_cache_write with
 * T_b tokens); L_b = context_lens[b] counts the cached tokens including
 * them, so new token i sits at position p = L_b - T_b + i and
 *
 *   out[query_start[b] + i][hq] =
 *       sum_{t <= p} softmax_t(scale * q[query_start[b] + i][hq] . K_t) V_t.
 *
 *   out             device, [num_query_tokens][num_q_heads][head_dim] of
 *                   out_dtype (F32, or the KV dtype, rounded to nearest
 *                   even), 16-byte aligned.  Rows of new tokens with p < 0
 *                   (T_b > L_b: a caller error) are zero.
 *   q               device, [num_query_tokens][num_q_heads][head_dim] of
 *                   kv_dtype, 16-byte aligned.
 *   k_cache, v_cache, block_tables, max_blocks_per_seq, num_blocks,
 *   block_size, scale: as for pka_paged_attention_decode.
 *   context_lens    device, int32 [num_seqs]; values are clamped to
 *                   [0, max_blocks_per_seq * block_size].
 *   query_start     device, int32 [num_seqs + 1], non-decreasing from 0 to
 *                   num_query_tokens.  A sequence whose two entries are out
 *                   of order or out of [0, num_query_tokens] is skipped
 *                   (its rows are left unwritten).
 *   max_query_len   host hint: an upper bound of T_b (sizes the grid); <= 0
 *                   means num_query_tokens.  New tokens past it are not
 *                   computed.
 * Supported: kv_dtype in {F16, BF16} (matrix cores; F32 returns
 * PKA_ERR_UNSUPPORTED); head_dim in {64, 128}; block_size in {16, 32};
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}.  No workspace.
 */
pka_status pka_paged_attention_prefill(void *out, pka_dtype out_dtype, const void *q,
                                       const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, const int32_t *query_start,
                                       int32_t num_seqs, int32_t num_query_tokens,
                                       int32_t max_query_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                       int32_t block_size, float scale, pka_dtype kv_dtype,
                                       void *stream);

/*
 * Whole-block movement for preemption and paging between GPU and CPU memory
 * (PhotonInfer README, Korean translation, "Continuous batching scheduler":
 * requests can be PREEMPTED; JackerLab "vllm" tag page, PagedAttention: KV
 * pages move between GPU and CPU memory).  A block is the contiguous run of
 * block_bytes = num_kv_heads * block_size * head_dim * element-size bytes
 * that one physical block holds in each pool.  All three are bit copies on
 * `stream`; an id outside [0, num_blocks) skips its entry; block_bytes must
 * be a multiple of 16 and every buffer 16-byte aligned.  Host transfers are
 * not done here: a swap-out is pka_gather_blocks into a device buffer
 * followed by one copy of that buffer to (pinned) host memory, a swap-in the
 * reverse followed by pka_scatter_blocks.
 *
 * pka_copy_blocks   block_pairs: device int64 [num_pairs][2] (src, dst).
 *                   Block dst of both pools becomes a copy of block src.
 *                   Destinations must be distinct and no block may be both
 *                   a source and a destination (else unspecified).
 * pka_gather_blocks packed: device [num_ids][2][block_bytes] (K, then V),
 *                   written; block_ids: device int64 [num_ids].  Entries with
 *                   invalid ids are left unwritten.
 * pka_scatter_blocks the inverse: block ids[i] of both pools take packed[i].
 *                   Ids must be distinct (else unspecified).
 */
pka_status pka_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_pairs,
                           int32_t num_pairs, int32_t num_blocks, int64_t block_bytes,
                           void *stream);
pka_status pka_gather_blocks(void *packed, const void *k_cache, const void *v_cache,
                             const int64_t *block_ids, int32_t num_ids, int32_t num_blocks,
                             int64_t block_bytes, void *stream);
pka_status pka_scatter_blocks(void *k_cache, void *v_cache, const void *packed,
                              const int64_t *block_ids, int32_t num_ids, int32_t num_blocks,
                              int64_t block_bytes, void *stream);

/*
 * Group-quantised INT8 KV cache.  The PhotonInfer README (Korean
 * translation), "Key features > GPU-optimised kernels" and "Technical
 * details > INT8 quantisation", quantises to INT8 group by group with a
 * configurable group size of 32, 64 or 128; it does so for weights, and
 * these calls apply the same scheme to the KV rows (a reading: the pages do
 * not quantise KV).  Each new token's row of one kv head is cut into
 * head_dim / group_size groups of consecutive elements; a group stores
 *   s = amax / 127          (amax = largest |x| of the group; float32
 *                            division, correctly rounded)
 *   c = rint(x / s)         (float32 division, ties to even), c in [-127, 127]
 * (s = 0 stores c = 0) and stands for c * s.  Inputs must be finite.
 *
 * INT8 pool layout (four arrays, each 16-byte aligned, one physical block
 * of one kv head contiguous in each):
 *   k_codes, v_codes  int8 [num_blocks][num_kv_heads][block_size * head_dim]
 *   k_scales, v_scales
 *             float32 [num_blocks][num_kv_heads][block_size][head_dim / group_size]
 * Inside a block's run of codes the tokens go in tiles of 16 (token offset
 * = 16 * tile + row) and the codes are in the order the matrix-core
 * products consume them (each lane of a 64-lane wave reads one contiguous
 * run of head_dim / 4 bytes per tile):
 *   K code of (offset, d) at ((tile * 64 + 16 * ((d % 32) / 8) + row)
 *                             * (head_dim / 32) + d / 32) * 8 + d % 8,
 *   V code of (offset, d) at ((tile * 64 + 16 * (row / 4) + d % 16)
 *                             * (head_dim / 16) + d / 16) * 4 + row % 4.
 * The scales are token-major: scale of (offset, group g) at
 * [offset][g].
 * Slots and block tables address tokens exactly as for the other pools.
 * Supported: head_dim in {64, 128}; block_size in {16, 32}; group_size in
 * {32, 64, 128} and <= head_dim.
 */

/*
 * pka_kv_cache_write_int8 -- quantise and store the K and V rows of
 * num_tokens new tokens of any number of sequences in one launch.  For each
 * token i with s = slot_mapping[i] in [0, num_blocks * block_size) (others
 * are skipped: padding), every kv head's rows k[i * k_token_stride + h *
 * head_dim + d] and v[...] (dtype elements) are quantised group by group
 * and stored at block s / block_size, offset s % block_size of the four
 * arrays; every other byte is left untouched.  Two tokens with one slot race.
 *   k, v          device, [num_tokens][num_kv_heads][head_dim] of dtype
 *                 (F32, F16 or BF16), token strides in elements (>=
 *                 num_kv_heads * head_dim), heads head_dim apart; aligned to
 *                 the element size.
 *   slot_mapping  device, int64 [num_tokens].
 *   k_codes, v_codes, k_scales, v_scales: device INT8 pools (layout above),
 *                 written in place.
 */
pka_status pka_kv_cache_write_int8(const void *k, const void *v, int64_t k_token_stride,
                                   int64_t v_token_stride, pka_dtype dtype,
                                   const int64_t *slot_mapping, int32_t num_tokens,
                                   int8_t *k_codes, int8_t *v_codes, float *k_scales,
                                   float *v_scales, int32_t num_blocks, int32_t block_size,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t group_size,
                                   void *stream);

/*
 * pka_decode_int8_partition_size -- the partition length (tokens, a
 * multiple of block_size) pka_paged_attention_decode_int8 uses when its
 * partition_size argument is 0.  Pure host function of the shapes.
 */
int32_t pka_decode_int8_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t block_size, int32_t max_context_len);

/*
 * pka_decode_int8_workspace_bytes -- device scratch of the INT8 decode for
 * these shapes and this (resolved) partition length; 0 when every sequence
 * fits one partition.  The workspace needs no initialisation: each call
 * writes everything it reads.  Its first 4 MiB are left untouched, so one
 * buffer (zero-filled once) can also serve as the workspace of
 * pka_paged_attention_decode, whose report counters live there.
 */
size_t pka_decode_int8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size);

/*
 * pka_paged_attention_decode_int8 -- pka_paged_attention_decode over INT8
 * pools: every cached K and V element is code * scale, and
 *
 *   out[b][hq][:] = sum_{t < L_b} softmax_t(scale * q[b][hq][:] . K_t) V_t
 *
 * with the stable softmax and fp32 accumulation.  Products run on the
 * matrix cores in fp16 (codes are exact in fp16; bf16 queries are scaled by
 * a power of two per head so that they are exact in fp16 too; the
 * probabilities times the V scales enter the second product rounded to fp16).
 * L_b <= 0 yields a zero row.  Long sequences are cut into partitions that
 * separate waves process, and their rows are combined exactly (log-sum-exp):
 * up to 8 partitions per sequence, the waves of one workgroup per (sequence,
 * kv head) take one partition each and merge in that workgroup; past 8 a
 * persistent grid takes the (sequence, partition) items, planned in each
 * workgroup's LDS up to 4096 sequences and by a one-workgroup planning
 * launch beyond, and a merge launch on `stream` combines the rows.
 *   out           device [num_seqs][num_q_heads][head_dim] of out_dtype (F32,
 *                 or q_dtype rounded to nearest even), 16-byte aligned.
 *   q             device [num_seqs][num_q_heads][head_dim] of q_dtype (F16 or
 *                 BF16; F32 returns PKA_ERR_UNSUPPORTED), 16-byte aligned.
 *   block_tables, max_blocks_per_seq, context_lens, num_blocks, block_size,
 *   scale, max_context_len: as for pka_paged_attention_decode (used table
 *                 entries are clamped into [0, num_blocks); lengths into
 *                 [0, min(max_blocks_per_seq * block_size, the partitions
 *                 that max_context_len spans)]).
 *   partition_size 0: pka_decode_int8_partition_size(); else a positive
 *                 multiple of block_size, at most 1024.
 *   workspace     device, >= pka_decode_int8_workspace_bytes(...) bytes,
 *                 256-byte aligned; may be NULL when that is 0.  Calls that
 *                 share a workspace on different streams race.
 * Supported: as for the INT8 pools above, num_q_heads / num_kv_heads in
 * {1, 2, 4, 8}.
 */
pka_status pka_paged_attention_decode_int8(
    void *out, pka_dtype out_dtype, const void *q, pka_dtype q_dtype, const int8_t *k_codes,
    const int8_t *v_codes, const float *k_scales, const float *v_scales,
    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, int32_t block_size, int32_t group_size, float scale,
    int32_t max_context_len, int32_t partition_size, void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * pka_paged_attention_decode_append_int8 -- one decode step over INT8 pools
 * in one launch (two past 8 partitions per sequence: the merge): for every
 * sequence b with L_b >= 1, its new token's K/V rows (k_new[b], v_new[b],
 * [num_seqs][num_kv_heads][head_dim] of q_dtype) are quantised and stored
 * at slot_mapping[b], and the decode then attends over L_b tokens, as
 * pka_kv_cache_write_int8 followed by pka_paged_attention_decode_int8 would
 * (bit-identical pools and output).  slot_mapping[b] must be the slot of
 * position L_b - 1 (a negative slot, or one past the pool, stores nothing
 * and position L_b - 1 is read from the pool as it is); a slot that this
 * call reads for another position races with the store.  Sequences with
 * L_b <= 0 store nothing and yield a zero row.  The PhotonInfer README's
 * batched write ("Technical details > Paged attention") fused with its
 * batched decode, over the INT8 cache of "Technical details > INT8
 * quantisation".
 *   k_new, v_new   device, token strides k_new_token_stride /
 *                  v_new_token_stride (elements, >= num_kv_heads * head_dim),
 *                  heads head_dim apart, of q_dtype.
 *   slot_mapping   device, int64 [num_seqs].
 * Everything else as for pka_paged_attention_decode_int8 (the pools are
 * written, so they are not const here).
 */
pka_status pka_paged_attention_decode_append_int8(
    void *out, pka_dtype out_dtype, const void *q, pka_dtype q_dtype, const void *k_new,
    const void *v_new, int64_t k_new_token_stride, int64_t v_new_token_stride,
    const int64_t *slot_mapping, int8_t *k_codes, int8_t *v_codes, float *k_scales,
    float *v_scales, const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t group_size, float scale,
    int32_t max_context_len, int32_t partition_size, void *workspace, size_t workspace_bytes,
    void *stream);

/* Static English name of a status code. */
const char *pka_status_string(pka_status status);

/* Thread-local detail of the last non-OK status returned on this thread
 * ("" if none).  Valid until the next call on the same thread. */
const char *pka_last_error(void);

/* PKA_ABI_VERSION of the loaded library. */
int32_t pka_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKA_H */
