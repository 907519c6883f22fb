// C ABI of the library (declared in include/pka.h): argument validation,
// the partition-length heuristic, workspace sizing and dispatch to the
// kernel launchers.  Everything the host can check is checked here, before
// any HIP call, and reported as a pka_status with a thread-local message.

#include "pka.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "pka_internal.h"

namespace {

thread_local char g_last_error[512] = "";

pka_status fail(pka_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

pka_status ok()
{
    g_last_error[0] = '\0';
    return PKA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(pka_dtype d) { return d == PKA_F32 || d == PKA_F16 || d == PKA_BF16; }

pka::DType to_internal(pka_dtype d) { return static_cast<pka::DType>(static_cast<int>(d)); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool finite(float x) { return std::isfinite(x); }

// The scale handed to the kernels.  They scale the logits by |scale| log2(e)
// inside the exponent and compare them with a running maximum in those
// units, so an exact 0 (or a subnormal that the arithmetic flushes to 0)
// would turn the initial "no maximum" (-inf) into NaN and leave every part of
// a split (sequence, kv head) pair weightless.  Magnitudes below 1e-30 are
// passed on as +-1e-30 instead: for any finite logit the weights then differ
// from the uniform ones that such a scale defines by far less than float32
// rounding.
float kernel_scale(float scale)
{
    return std::fabs(scale) < 1e-30f ? std::copysign(1e-30f, scale) : scale;
}

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

constexpr int64_t kDefaultPartition = 512;

// Compute units of the current device (256 on MI355X; fewer on a partitioned
// GPU), so that host heuristics match what the kernels see.
int64_t compute_units()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}

}  // namespace

pka::WorkspaceLayout pka::decode_workspace_layout(int64_t num_seqs, int64_t num_q_heads,
                                                  int64_t num_kv_heads, int64_t head_dim,
                                                  int64_t max_waves)
{
    WorkspaceLayout w{0, 0, 0};
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_waves <= 0)
        return w;
    const int64_t group = num_q_heads / num_kv_heads;
    // a fixed counter region, so that one workspace serves calls of any shape
    w.counter_offset = 0;
    w.parts_offset = (size_t)kCounterBytes;
    w.total = w.parts_offset + (size_t)round256(2 * max_waves * decode_part_floats(group, head_dim) * 4);
    return w;
}

extern "C" {

const char *pka_status_string(pka_status s)
{
    switch (s) {
    case PKA_OK: return "ok";
    case PKA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PKA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PKA_ERR_HIP: return "HIP runtime error";
    default: break;
    }
    return "unknown status";
}

const char *pka_last_error(void) { return g_last_error; }

int32_t pka_abi_version(void) { return PKA_ABI_VERSION; }

pka_status pka_kv_cache_write(const void *k, const void *v, int64_t k_token_stride,
                              int64_t v_token_stride, const int64_t *slot_mapping,
                              int32_t num_tokens, void *k_cache, void *v_cache,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_dim, pka_dtype dtype, void *stream)
{
    if (num_tokens < 0)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (!valid_dtype(dtype))
        return fail(PKA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
    if (num_blocks <= 0 || num_kv_heads <= 0)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_blocks and num_kv_heads must be positive");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
    if (block_size != 16 && block_size != 32)
        return fail(PKA_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", block_size);
    if (!k_cache || !v_cache)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null cache pointer");
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKA_ERR_INVALID_ARGUMENT, "caches must be 16-byte aligned");
    if (num_tokens == 0)
        return ok();
    if (!k || !v || !slot_mapping)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null k, v or slot_mapping");
    const int elt = pka::dtype_bytes(to_internal(dtype));
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (k_token_stride < row || v_token_stride < row)
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "token strides (%lld, %lld) must be >= num_kv_heads * head_dim = %lld",
                    (long long)k_token_stride, (long long)v_token_stride, (long long)row);
    if (!aligned16(k) || !aligned16(v) || (k_token_stride * elt) % 16 || (v_token_stride * elt) % 16)
        return fail(PKA_ERR_INVALID_ARGUMENT, "k/v rows must be 16-byte aligned");
    pka::WriteArgs a{k, v, k_token_stride, v_token_stride, slot_mapping, num_tokens,
                     k_cache, v_cache, num_blocks, block_size, num_kv_heads, head_dim,
                     to_internal(dtype)};
    hipError_t e = pka::launch_kv_cache_write(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKA_ERR_HIP, "kv_cache_write launch: %s", hipGetErrorString(e));
    return ok();
}

pka_status pka_kv_cache_write_rope(const void *k, const void *v, int64_t k_token_stride,
                                   int64_t v_token_stride, const int64_t *slot_mapping,
                                   const int32_t *positions, int32_t num_tokens,
                                   const float *cos_sin, int32_t max_position, int32_t rotary_dim,
                                   void *k_cache, void *v_cache, int32_t num_blocks,
                                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                   pka_dtype dtype, void *stream)
{
    if (valid_dtype(dtype)) {
        const int vec = 16 / pka::dtype_bytes(to_internal(dtype));
        if (rotary_dim <= 0 || rotary_dim > head_dim || rotary_dim % (2 * vec))
            return fail(PKA_ERR_INVALID_ARGUMENT,
                        "rotary_dim %d must be in (0, head_dim] and a multiple of %d", rotary_dim,
                        2 * vec);
    }
    if (max_position <= 0)
        return fail(PKA_ERR_INVALID_ARGUMENT, "max_position must be positive");
    // the checks of the plain write (they come first for the shapes)
    const pka_status st = pka_kv_cache_write(nullptr, nullptr, k_token_stride, v_token_stride,
                                             nullptr, 0, k_cache, v_cache, num_blocks,
                                             block_size, num_kv_heads, head_dim, dtype, stream);
    if (st != PKA_OK)
        return st;
    if (num_tokens < 0)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (num_tokens == 0)
        return ok();
    if (!k || !v || !slot_mapping || !positions || !cos_sin)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null k, v, slot_mapping, positions or cos_sin");
    const int elt = pka::dtype_bytes(to_internal(dtype));
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (k_token_stride < row || v_token_stride < row)
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "token strides (%lld, %lld) must be >= num_kv_heads * head_dim = %lld",
                    (long long)k_token_stride, (long long)v_token_stride, (long long)row);
    if (!aligned16(k) || !aligned16(v) || (k_token_stride * elt) % 16 || (v_token_stride * elt) % 16)
        return fail(PKA_ERR_INVALID_ARGUMENT, "k/v rows must be 16-byte aligned");
    pka::WriteArgs a{k, v, k_token_stride, v_token_stride, slot_mapping, num_tokens,
                     k_cache, v_cache, num_blocks, block_size, num_kv_heads, head_dim,
                     to_internal(dtype)};
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.max_position = max_position;
    a.rotary_dim = rotary_dim;
    hipError_t e = pka::launch_kv_cache_write(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKA_ERR_HIP, "kv_cache_write_rope launch: %s", hipGetErrorString(e));
    return ok();
}

int32_t pka_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                  int32_t max_context_len)
{
    // The decode spreads the flat (sequence, kv head, chunk) space evenly
    // over the GPU's waves; partition_size only sets how short a wave's
    // range may get.  64 tokens by default: a shorter range spends more of
    // its time on its first request and on the partial result it leaves.
    (void)num_seqs;
    (void)num_kv_heads;
    (void)max_context_len;
    if (block_size <= 0)
        return 0;
    return (int32_t)(ceil_div(pka::kDefaultRangeTokens, block_size) * block_size);
}

size_t pka_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim)
{
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return 0;
    return pka::decode_workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        pka::decode_max_waves())
        .total;
}

}  // extern "C"

// Workspace of pka_paged_attention_decode_noalloc: report counters, then
// partial results, as in a caller's decode workspace.  Each device holds its
// own copy; host code uses only the per-device address from
// hipGetSymbolAddress, never this name.
static_assert(PKA_DECODE_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[PKA_DECODE_STATIC_SCRATCH_BYTES];

__global__ void zero_words(int32_t *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address, set up (address taken, counters
// cleared on `stream`) by the first call on that device.
pka_status static_scratch(void **ptr, hipStream_t stream)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(PKA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKA_ERR_UNSUPPORTED, "device %d beyond the %d the static scratch serves", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(PKA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        // the counters must read zero before the first decode (a kernel
        // rather than a memset, so that a captured first call stays valid)
        constexpr int64_t n = pka::kCounterBytes / 4;
        hipLaunchKernelGGL(zero_words, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           static_cast<int32_t *>(p), n);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKA_ERR_HIP, "clearing the static scratch: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PKA_OK;
}

}  // namespace

static pka_status decode_impl(void *out, pka_dtype out_dtype, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t num_blocks, int32_t block_size,
                              float scale, pka_dtype kv_dtype, int32_t max_context_len,
                              int32_t partition_size, void *workspace, size_t workspace_bytes,
                              void *stream, const void *k_new, const void *v_new,
                              int64_t k_new_token_stride, int64_t v_new_token_stride,
                              const int64_t *slot_mapping, bool static_workspace = false)
{
    if (!valid_dtype(kv_dtype) || !valid_dtype(out_dtype))
        return fail(PKA_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (out_dtype != PKA_F32 && out_dtype != kv_dtype)
        return fail(PKA_ERR_INVALID_ARGUMENT, "out dtype must be F32 or the KV dtype");
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0)
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "num_seqs >= 0 and positive num_q_heads, num_kv_heads, num_blocks, "
                    "max_blocks_per_seq required");
    if (num_q_heads % num_kv_heads)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_q_heads %d not a multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    const int group = num_q_heads / num_kv_heads;
    if (!pka::decode_supported(to_internal(kv_dtype), head_dim, block_size, group))
        return fail(PKA_ERR_UNSUPPORTED,
                    "head_dim %d / block_size %d / group %d outside {64,128} x {16,32} x {1,2,4,8}",
                    head_dim, block_size, group);
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return fail(PKA_ERR_UNSUPPORTED, "num_seqs and num_kv_heads must be <= 65535");
    if (!finite(scale))
        return fail(PKA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (partition_size < 0 || (partition_size > 0 && partition_size % block_size))
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "partition_size %d must be 0 or a positive multiple of block_size %d",
                    partition_size, block_size);
    // max_context_len only picks the launch shape: no length is cut short by it
    if (num_seqs == 0)
        return ok();
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKA_ERR_INVALID_ARGUMENT, "out, q and the caches must be 16-byte aligned");
    const int elt = pka::dtype_bytes(to_internal(kv_dtype));
    if (k_new || v_new || slot_mapping) {
        if (!k_new || !v_new || !slot_mapping)
            return fail(PKA_ERR_INVALID_ARGUMENT, "null k_new, v_new or slot_mapping");
        const int64_t row = (int64_t)num_kv_heads * head_dim;
        if (k_new_token_stride < row || v_new_token_stride < row)
            return fail(PKA_ERR_INVALID_ARGUMENT,
                        "new-token strides (%lld, %lld) must be >= num_kv_heads * head_dim = %lld",
                        (long long)k_new_token_stride, (long long)v_new_token_stride,
                        (long long)row);
        if (!aligned16(k_new) || !aligned16(v_new) || (k_new_token_stride * elt) % 16 ||
            (v_new_token_stride * elt) % 16)
            return fail(PKA_ERR_INVALID_ARGUMENT, "k_new/v_new rows must be 16-byte aligned");
    }
    // One launch plans its sequences in LDS and counts work units (per
    // chunk of 16 tokens or more, and per pair) in int32: cut the batch into
    // launches that respect both.
    const int64_t table_cap = (int64_t)max_blocks_per_seq * block_size;
    const int64_t units_per_seq =
        (pka::kUnitsPerChunk * ceil_div(table_cap, 16) + pka::kUnitsPerPair) * num_kv_heads;
    if (units_per_seq >= INT32_MAX)
        return fail(PKA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size too large");
    int64_t per_launch = pka::kMaxSeqsPerLaunch;
    if (per_launch * units_per_seq >= INT32_MAX)
        per_launch = (INT32_MAX - 1) / units_per_seq;
    if (per_launch * num_kv_heads > pka::kMaxCounters)
        per_launch = pka::kMaxCounters / num_kv_heads;
    if (per_launch < 1)
        return fail(PKA_ERR_UNSUPPORTED, "num_kv_heads %d exceeds the report counters",
                    num_kv_heads);
    const int64_t max_waves = pka::decode_max_waves();
    const size_t need = pka::decode_workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                     max_waves)
                            .total;
    if (static_workspace) {
        if (need > sizeof(scratch))
            return fail(PKA_ERR_WORKSPACE_TOO_SMALL,
                        "decode needs %zu bytes of scratch; the static scratch holds %zu", need,
                        sizeof(scratch));
        const pka_status s = static_scratch(&workspace, static_cast<hipStream_t>(stream));
        if (s != PKA_OK)
            return s;
        workspace_bytes = sizeof(scratch);
    }
    if (!workspace)
        return fail(PKA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes required, got NULL", need);
    if (workspace_bytes < need)
        return fail(PKA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes required, got %zu", need,
                    workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(PKA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    const pka::WorkspaceLayout wl =
        pka::decode_workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_waves);
    char *base = static_cast<char *>(workspace);
    const int out_elt = pka::dtype_bytes(to_internal(out_dtype));
    for (int64_t b0 = 0; b0 < num_seqs; b0 += per_launch) {
        const int64_t nb = num_seqs - b0 < per_launch ? num_seqs - b0 : per_launch;
        pka::DecodeArgs a{};
        a.out = static_cast<char *>(out) + b0 * num_q_heads * head_dim * out_elt;
        a.out_dtype = to_internal(out_dtype);
        a.q = static_cast<const char *>(q) + b0 * num_q_heads * head_dim * elt;
        a.k_cache = k_cache;
        a.v_cache = v_cache;
        a.block_tables = block_tables + b0 * max_blocks_per_seq;
        a.max_blocks_per_seq = max_blocks_per_seq;
        a.context_lens = context_lens + b0;
        a.num_seqs = (int32_t)nb;
        a.num_q_heads = num_q_heads;
        a.num_kv_heads = num_kv_heads;
        a.head_dim = head_dim;
        a.num_blocks = num_blocks;
        a.block_size = block_size;
        a.scale = kernel_scale(scale);
        a.kv_dtype = to_internal(kv_dtype);
        a.partition_size = partition_size;
        a.context_hint = max_context_len > 0 ? max_context_len : 0;
        a.counters = reinterpret_cast<int32_t *>(base + wl.counter_offset);
        a.parts = reinterpret_cast<float *>(base + wl.parts_offset);
        a.max_waves = max_waves;
        if (k_new) {
            a.k_new = static_cast<const char *>(k_new) + b0 * k_new_token_stride * elt;
            a.v_new = static_cast<const char *>(v_new) + b0 * v_new_token_stride * elt;
            a.k_new_token_stride = k_new_token_stride;
            a.v_new_token_stride = v_new_token_stride;
            a.slot_mapping = slot_mapping + b0;
        }
        hipError_t e = pka::launch_paged_decode(a, static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(PKA_ERR_HIP, "paged_attention_decode launch: %s", hipGetErrorString(e));
    }
    return ok();
}


extern "C" {

pka_status pka_paged_attention_decode(void *out, pka_dtype out_dtype, const void *q,
                                      const void *k_cache, const void *v_cache,
                                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t num_blocks, int32_t block_size, float scale,
                                      pka_dtype kv_dtype, int32_t max_context_len,
                                      int32_t partition_size, void *workspace,
                                      size_t workspace_bytes, void *stream)
{
    return decode_impl(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                       block_size, scale, kv_dtype, max_context_len, partition_size, workspace,
                       workspace_bytes, stream, nullptr, nullptr, 0, 0, nullptr);
}

pka_status pka_paged_attention_decode_noalloc(
    void *out, pka_dtype out_dtype, const void *q, const void *k_cache, const void *v_cache,
    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, int32_t block_size, float scale, pka_dtype kv_dtype,
    int32_t max_context_len, int32_t partition_size, void *stream)
{
    return decode_impl(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                       block_size, scale, kv_dtype, max_context_len, partition_size, nullptr, 0,
                       stream, nullptr, nullptr, 0, 0, nullptr, /*static_workspace=*/true);
}

pka_status pka_paged_attention_decode_append(
    void *out, pka_dtype out_dtype, const void *q, const void *k_new, const void *v_new,
    int64_t k_new_token_stride, int64_t v_new_token_stride, const int64_t *slot_mapping,
    void *k_cache, void *v_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_blocks, int32_t block_size, float scale, pka_dtype kv_dtype,
    int32_t max_context_len, int32_t partition_size, void *workspace, size_t workspace_bytes,
    void *stream)
{
    if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
        return fail(PKA_ERR_INVALID_ARGUMENT, "null k_new, v_new or slot_mapping");
    return decode_impl(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                       block_size, scale, kv_dtype, max_context_len, partition_size, workspace,
                       workspace_bytes, stream, k_new, v_new, k_new_token_stride,
                       v_new_token_stride, slot_mapping);
}

pka_status pka_paged_attention_prefill(void *out, pka_dtype out_dtype, const void *q,
                                       const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, const int32_t *query_start,
                                       int32_t num_seqs, int32_t num_query_tokens,
                                       int32_t max_query_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                       int32_t block_size, float scale, pka_dtype kv_dtype,
                                       void *stream)
{
    if (!valid_dtype(kv_dtype) || !valid_dtype(out_dtype))
        return fail(PKA_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (out_dtype != PKA_F32 && out_dtype != kv_dtype)
        return fail(PKA_ERR_INVALID_ARGUMENT, "out dtype must be F32 or the KV dtype");
    if (num_seqs < 0 || num_query_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "num_seqs, num_query_tokens >= 0 and positive num_q_heads, num_kv_heads, "
                    "num_blocks, max_blocks_per_seq required");
    if (num_q_heads % num_kv_heads)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_q_heads %d not a multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    const int group = num_q_heads / num_kv_heads;
    if (!pka::prefill_supported(to_internal(kv_dtype), head_dim, block_size, group))
        return fail(PKA_ERR_UNSUPPORTED,
                    "multi-token attention needs F16/BF16 KV, head_dim in {64,128}, block_size "
                    "in {16,32}, group in {1,2,4,8} (got dtype %d, %d, %d, %d)",
                    (int)kv_dtype, head_dim, block_size, group);
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return fail(PKA_ERR_UNSUPPORTED, "num_seqs and num_kv_heads must be <= 65535");
    if (!finite(scale))
        return fail(PKA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (num_seqs == 0 || num_query_tokens == 0)
        return ok();
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKA_ERR_INVALID_ARGUMENT, "out, q and the caches must be 16-byte aligned");
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
        return fail(PKA_ERR_UNSUPPORTED, "context length beyond int32");
    pka::PrefillArgs a{};
    a.out = out;
    a.out_dtype = to_internal(out_dtype);
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.query_start = query_start;
    a.num_seqs = num_seqs;
    a.num_query_tokens = num_query_tokens;
    a.max_query_len =
        max_query_len > 0 && max_query_len < num_query_tokens ? max_query_len : num_query_tokens;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.scale = kernel_scale(scale);
    a.kv_dtype = to_internal(kv_dtype);
    hipError_t e = pka::launch_paged_prefill(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKA_ERR_HIP, "paged_attention_prefill launch: %s", hipGetErrorString(e));
    return ok();
}

static pka_status move_blocks(pka::BlockMove mode, void *k_cache, void *v_cache, void *packed,
                              const int64_t *ids, int32_t n, int32_t num_blocks,
                              int64_t block_bytes, void *stream, const char *what)
{
    if (n < 0 || num_blocks <= 0 || block_bytes <= 0)
        return fail(PKA_ERR_INVALID_ARGUMENT, "%s: n >= 0, num_blocks > 0, block_bytes > 0 required",
                    what);
    if (block_bytes % 16)
        return fail(PKA_ERR_INVALID_ARGUMENT, "%s: block_bytes %lld is not a multiple of 16", what,
                    (long long)block_bytes);
    if ((block_bytes + 16383) / 16384 > 65535)
        return fail(PKA_ERR_UNSUPPORTED, "%s: blocks larger than 1 GiB", what);
    if (n == 0)
        return ok();
    if (!k_cache || !v_cache || !ids || (mode != pka::BlockMove::Copy && !packed))
        return fail(PKA_ERR_INVALID_ARGUMENT, "%s: null pointer argument", what);
    if (!aligned16(k_cache) || !aligned16(v_cache) || (packed && !aligned16(packed)))
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "%s: pools and the packed buffer must be 16-byte aligned", what);
    pka::BlockMoveArgs a{};
    a.mode = mode;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.packed = packed;
    a.ids = ids;
    a.num_entries = n;
    a.num_blocks = num_blocks;
    a.block_bytes = block_bytes;
    hipError_t e = pka::launch_move_blocks(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

pka_status pka_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_pairs,
                           int32_t num_pairs, int32_t num_blocks, int64_t block_bytes, void *stream)
{
    return move_blocks(pka::BlockMove::Copy, k_cache, v_cache, nullptr, block_pairs, num_pairs,
                       num_blocks, block_bytes, stream, "copy_blocks");
}

pka_status pka_gather_blocks(void *packed, const void *k_cache, const void *v_cache,
                             const int64_t *block_ids, int32_t num_ids, int32_t num_blocks,
                             int64_t block_bytes, void *stream)
{
    return move_blocks(pka::BlockMove::Gather, const_cast<void *>(k_cache),
                       const_cast<void *>(v_cache), packed, block_ids, num_ids, num_blocks,
                       block_bytes, stream, "gather_blocks");
}

pka_status pka_scatter_blocks(void *k_cache, void *v_cache, const void *packed,
                              const int64_t *block_ids, int32_t num_ids, int32_t num_blocks,
                              int64_t block_bytes, void *stream)
{
    return move_blocks(pka::BlockMove::Scatter, k_cache, v_cache, const_cast<void *>(packed),
                       block_ids, num_ids, num_blocks, block_bytes, stream, "scatter_blocks");
}

}  // extern "C"


// ---------------------------------------------------------------------------
// Group-quantised INT8 KV cache
// ---------------------------------------------------------------------------

pka::Int8WorkspaceLayout pka::int8_workspace_layout(int64_t num_seqs, int64_t num_q_heads,
                                                    int64_t head_dim, int64_t num_partitions)
{
    Int8WorkspaceLayout w{0, 0, 0, 0, 0};
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_partitions <= 1)
        return w;
    const int64_t rows = num_seqs * num_q_heads * num_partitions;
    // the first kCounterBytes stay untouched: there the fp16/bf16/fp32 decode
    // keeps counters that must read zero, so one buffer can serve both decodes
    w.header_offset = (size_t)kCounterBytes;
    w.items_offset = w.header_offset + 256;
    w.ml_offset = w.items_offset + (size_t)round256(num_seqs * num_partitions * 8);
    w.o_offset = w.ml_offset + (size_t)round256(rows * 2 * 4);
    w.total = w.o_offset + (size_t)round256(rows * head_dim * 4);
    return w;
}

namespace {

bool int8_group_ok(int32_t head_dim, int32_t group_size)
{
    return (group_size == 32 || group_size == 64 || group_size == 128) && group_size <= head_dim;
}

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

pka_status pka_kv_cache_write_int8(const void *k, const void *v, int64_t k_token_stride,
                                   int64_t v_token_stride, pka_dtype dtype,
                                   const int64_t *slot_mapping, int32_t num_tokens,
                                   int8_t *k_codes, int8_t *v_codes, float *k_scales,
                                   float *v_scales, int32_t num_blocks, int32_t block_size,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t group_size,
                                   void *stream)
{
    if (num_tokens < 0)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (!valid_dtype(dtype))
        return fail(PKA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
    if (num_blocks <= 0 || num_kv_heads <= 0)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_blocks and num_kv_heads must be positive");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
    if (block_size != 16 && block_size != 32)
        return fail(PKA_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", block_size);
    if (!int8_group_ok(head_dim, group_size))
        return fail(PKA_ERR_UNSUPPORTED, "group_size %d not in {32, 64, 128} or above head_dim %d",
                    group_size, head_dim);
    if (!k_codes || !v_codes || !k_scales || !v_scales)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null code or scale array");
    if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) || !aligned16(v_scales))
        return fail(PKA_ERR_INVALID_ARGUMENT, "code and scale arrays must be 16-byte aligned");
    if (num_tokens == 0)
        return ok();
    if (!k || !v || !slot_mapping)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null k, v or slot_mapping");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (k_token_stride < row || v_token_stride < row)
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "token strides (%lld, %lld) must be >= num_kv_heads * head_dim = %lld",
                    (long long)k_token_stride, (long long)v_token_stride, (long long)row);
    const int elt = pka::dtype_bytes(to_internal(dtype));
    if (elt == 4 ? (!aligned4(k) || !aligned4(v)) : ((reinterpret_cast<uintptr_t>(k) |
                                                      reinterpret_cast<uintptr_t>(v)) & 1u))
        return fail(PKA_ERR_INVALID_ARGUMENT, "k/v not aligned to their element size");
    pka::Int8WriteArgs a{k, v, k_token_stride, v_token_stride, to_internal(dtype), slot_mapping,
                         num_tokens, k_codes, v_codes, k_scales, v_scales, num_blocks,
                         block_size, num_kv_heads, head_dim, group_size};
    hipError_t e = pka::launch_kv_cache_write_int8(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKA_ERR_HIP, "kv_cache_write_int8 launch: %s", hipGetErrorString(e));
    return ok();
}

int32_t pka_decode_int8_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t block_size, int32_t max_context_len)
{
    // One partition (no merge launch) while the longest sequence fits 256
    // tokens; else 512 tokens, halved down to 128 while the (sequence, kv
    // head, partition) units would number fewer than 32 per compute unit
    // (measured: mixed batch of 64, 128-token partitions 20.0 us against
    // 22.3 us with 256).
    if (block_size <= 0)
        return 0;
    const int64_t pairs = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
    const int64_t lmax = max_context_len > 0 ? max_context_len : 1;
    if (lmax <= 256)
        return (int32_t)(ceil_div(lmax, block_size) * block_size);
    int64_t P = kDefaultPartition;
    while (P > 128 && pairs * ceil_div(lmax, P) < 32 * compute_units())
        P /= 2;
    return (int32_t)(ceil_div(P, block_size) * block_size);
}

size_t pka_decode_int8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size)
{
    if (partition_size <= 0 || max_context_len <= partition_size)
        return 0;
    return pka::int8_workspace_layout(num_seqs, num_q_heads, head_dim,
                                      ceil_div(max_context_len, partition_size))
        .total;
}

}  // extern "C"

static pka_status decode_int8_impl(
    void *out, pka_dtype out_dtype, const void *q, pka_dtype q_dtype, const int8_t *k_codes,
    const int8_t *v_codes, const float *k_scales, const float *v_scales,
    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, int32_t block_size, int32_t group_size, float scale,
    int32_t max_context_len, int32_t partition_size, void *workspace, size_t workspace_bytes,
    void *stream, const void *k_new, const void *v_new, int64_t k_new_stride,
    int64_t v_new_stride, const int64_t *slot_mapping)
{
    if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype))
        return fail(PKA_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (q_dtype == PKA_F32)
        return fail(PKA_ERR_UNSUPPORTED, "INT8 decode takes F16 or BF16 queries");
    if (out_dtype != PKA_F32 && out_dtype != q_dtype)
        return fail(PKA_ERR_INVALID_ARGUMENT, "out dtype must be F32 or the query dtype");
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0)
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "num_seqs >= 0 and positive num_q_heads, num_kv_heads, num_blocks, "
                    "max_blocks_per_seq required");
    if (num_q_heads % num_kv_heads)
        return fail(PKA_ERR_INVALID_ARGUMENT, "num_q_heads %d not a multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    const int group = num_q_heads / num_kv_heads;
    if ((head_dim != 64 && head_dim != 128) || (block_size != 16 && block_size != 32) ||
        (group != 1 && group != 2 && group != 4 && group != 8))
        return fail(PKA_ERR_UNSUPPORTED,
                    "head_dim %d / block_size %d / group %d outside {64,128} x {16,32} x {1,2,4,8}",
                    head_dim, block_size, group);
    if (!int8_group_ok(head_dim, group_size))
        return fail(PKA_ERR_UNSUPPORTED, "group_size %d not in {32, 64, 128} or above head_dim %d",
                    group_size, head_dim);
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return fail(PKA_ERR_UNSUPPORTED, "num_seqs and num_kv_heads must be <= 65535");
    if (!finite(scale))
        return fail(PKA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (partition_size < 0 || (partition_size > 0 && partition_size % block_size))
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "partition_size %d must be 0 or a positive multiple of block_size %d",
                    partition_size, block_size);
    if (partition_size > pka::kMaxPartition)
        return fail(PKA_ERR_UNSUPPORTED, "partition_size %d exceeds %d", partition_size,
                    pka::kMaxPartition);
    if (num_seqs == 0)
        return ok();
    if (!out || !q || !k_codes || !v_codes || !k_scales || !v_scales || !block_tables ||
        !context_lens)
        return fail(PKA_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) ||
        !aligned16(k_scales) || !aligned16(v_scales))
        return fail(PKA_ERR_INVALID_ARGUMENT,
                    "out, q, the code and the scale arrays must be 16-byte aligned");
    const int64_t table_cap = (int64_t)max_blocks_per_seq * block_size;
    int64_t lmax = max_context_len > 0 ? max_context_len : table_cap;
    if (lmax > table_cap)
        lmax = table_cap;
    if (lmax > INT32_MAX / 2)
        return fail(PKA_ERR_UNSUPPORTED, "context length beyond 2^30");
    if (partition_size == 0)
        partition_size = pka_decode_int8_partition_size(num_seqs, num_kv_heads, block_size,
                                                        (int32_t)lmax);
    if (partition_size > pka::kMaxPartition)
        partition_size = pka::kMaxPartition / block_size * block_size;
    const int64_t parts = lmax > 0 ? ceil_div(lmax, partition_size) : 1;
    if ((int64_t)num_seqs * parts > 0x7fffffff / 8)
        return fail(PKA_ERR_UNSUPPORTED, "too many (sequence, partition) items");
    const size_t need = pka_decode_int8_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                        (int32_t)lmax, partition_size);
    if (need > 0) {
        if (!workspace)
            return fail(PKA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes required, got NULL", need);
        if (workspace_bytes < need)
            return fail(PKA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes required, got %zu",
                        need, workspace_bytes);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(PKA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    }
    pka::Int8DecodeArgs a{};
    a.out = out;
    a.out_kind = out_dtype == PKA_F32 ? 0 : (out_dtype == PKA_F16 ? 1 : 2);
    a.q = q;
    a.q_dtype = to_internal(q_dtype);
    a.k_codes = k_codes;
    a.v_codes = v_codes;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.group_size = group_size;
    a.scale_log2 = kernel_scale(scale) * 1.44269504088896340736f;
    a.partition_size = partition_size;
    a.num_partitions = (int32_t)parts;
    a.len_cap = (int32_t)(parts * partition_size < table_cap ? parts * partition_size : table_cap);
    if (need > 0) {
        const pka::Int8WorkspaceLayout w =
            pka::int8_workspace_layout(num_seqs, num_q_heads, head_dim, parts);
        char *base = static_cast<char *>(workspace);
        a.wl_header = reinterpret_cast<int32_t *>(base + w.header_offset);
        a.items = reinterpret_cast<int2 *>(base + w.items_offset);
        a.ws_ml = reinterpret_cast<float *>(base + w.ml_offset);
        a.ws_o = reinterpret_cast<float *>(base + w.o_offset);
    }
    if (k_new || v_new || slot_mapping) {
        if (!k_new || !v_new || !slot_mapping)
            return fail(PKA_ERR_INVALID_ARGUMENT, "null k_new, v_new or slot_mapping");
        const int64_t row = (int64_t)num_kv_heads * head_dim;
        if (k_new_stride < row || v_new_stride < row)
            return fail(PKA_ERR_INVALID_ARGUMENT,
                        "new-token strides (%lld, %lld) must be >= num_kv_heads * head_dim = %lld",
                        (long long)k_new_stride, (long long)v_new_stride, (long long)row);
        if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 1u)
            return fail(PKA_ERR_INVALID_ARGUMENT, "k_new/v_new not aligned to their element size");
        a.k_new = k_new;
        a.v_new = v_new;
        a.k_new_stride = k_new_stride;
        a.v_new_stride = v_new_stride;
        a.slot_mapping = slot_mapping;
    }
    hipError_t e = pka::launch_paged_decode_int8(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKA_ERR_HIP, "paged_attention_decode_int8 launch: %s", hipGetErrorString(e));
    return ok();
}

extern "C" {

pka_status pka_paged_attention_decode_int8(
    void *out, pka_dtype out_dtype, const void *q, pka_dtype q_dtype, const int8_t *k_codes,
    const int8_t *v_codes, const float *k_scales, const float *v_scales,
    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, int32_t block_size, int32_t group_size, float scale,
    int32_t max_context_len, int32_t partition_size, void *workspace, size_t workspace_bytes,
    void *stream)
{
    return decode_int8_impl(out, out_dtype, q, q_dtype, k_codes, v_codes, k_scales, v_scales,
                            block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, num_blocks, block_size, group_size, scale,
                            max_context_len, partition_size, workspace, workspace_bytes, stream,
                            nullptr, nullptr, 0, 0, nullptr);
}

pka_status pka_paged_attention_decode_append_int8(
    void *out, pka_dtype out_dtype, const void *q, pka_dtype q_dtype, const void *k_new,
    const void *v_new, int64_t k_new_token_stride, int64_t v_new_token_stride,
    const int64_t *slot_mapping, int8_t *k_codes, int8_t *v_codes, float *k_scales,
    float *v_scales, const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t group_size, float scale,
    int32_t max_context_len, int32_t partition_size, void *workspace, size_t workspace_bytes,
    void *stream)
{
    if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
        return fail(PKA_ERR_INVALID_ARGUMENT, "null k_new, v_new or slot_mapping");
    return decode_int8_impl(out, out_dtype, q, q_dtype, k_codes, v_codes, k_scales, v_scales,
                            block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                            num_kv_heads, head_dim, num_blocks, block_size, group_size, scale,
                            max_context_len, partition_size, workspace, workspace_bytes, stream,
                            k_new, v_new, k_new_token_stride, v_new_token_stride, slot_mapping);
}

}  // extern "C"
