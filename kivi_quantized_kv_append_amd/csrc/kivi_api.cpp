// Host side of the C ABI: configuration checks (fail fast on anything the
// kernels do not implement), pool layout, argument checks, error reporting.
// No device memory is allocated here; only kivi_check_device_errors waits on
// the device.

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <climits>
#include <limits>
#include <string>

#include <hip/hip_runtime.h>

#include "kivi_internal.h"

namespace {

thread_local std::string g_last_error;

kivi_status fail(kivi_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

kivi_status ok() {
    g_last_error.clear();
    return KIVI_OK;
}

uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255u); }

constexpr uint64_t kStatusBytes = 256;  // the status word's sub-array (one 32-bit word used)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks every field; fills the layout on success.
kivi_status check_config(const kivi_cache_config* cfg, kivi_layout* lay) {
    if (!cfg) return fail(KIVI_ERR_INVALID_ARG, "config is NULL");
    const kivi_cache_config& c = *cfg;
    if (c.head_dim != kivi::kHeadDim)
        return fail(KIVI_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", c.head_dim);
    if (c.bits != 2 && c.bits != 4 && c.bits != 8)
        return fail(KIVI_ERR_UNSUPPORTED, "bits %d unsupported (2, 4, or 8 for FP8 E4M3)", c.bits);
    if (c.scale_per_head != 0 && c.scale_per_head != 1)
        return fail(KIVI_ERR_UNSUPPORTED, "scale_per_head %d unsupported (0 or 1)", c.scale_per_head);
    if (c.bits != 8 && c.scale_per_head)
        return fail(KIVI_ERR_UNSUPPORTED, "scale_per_head applies to the FP8 cache (bits 8) only");
    if (c.num_kv_heads < 1 || c.num_kv_heads > 1024)
        return fail(KIVI_ERR_UNSUPPORTED, "num_kv_heads %d outside [1, 1024]", c.num_kv_heads);
    if (c.block_size < 16 || c.block_size > 1024 || c.block_size % 16)
        return fail(KIVI_ERR_UNSUPPORTED, "block_size %d must be a multiple of 16 in [16, 1024]",
                    c.block_size);
    if ((c.block_size & (c.block_size - 1)) || (c.k_group & (c.k_group - 1)))
        return fail(KIVI_ERR_UNSUPPORTED, "block_size %d and k_group %d must be powers of two", c.block_size,
                    c.k_group);
    if (c.bits == 8) {
        // FP8: every token is encoded on append; no groups, no residual
        if (c.k_group || c.v_group || c.residual || c.v_flush)
            return fail(KIVI_ERR_UNSUPPORTED,
                        "the FP8 cache has no groups or residual: k_group, v_group, residual and v_flush "
                        "must be 0");
        if (c.num_blocks < 1) return fail(KIVI_ERR_INVALID_ARG, "num_blocks %d < 1", c.num_blocks);
        if (c.max_seqs < 1) return fail(KIVI_ERR_INVALID_ARG, "max_seqs %d < 1", c.max_seqs);
        if (c.kv_dtype != KIVI_F16 && c.kv_dtype != KIVI_BF16)
            return fail(KIVI_ERR_UNSUPPORTED, "kv_dtype %d unsupported", c.kv_dtype);
        const uint64_t H = (uint64_t)c.num_kv_heads;
        kivi_layout L{};
        L.code_bytes = (uint64_t)c.block_size * kivi::kHeadDim;
        uint64_t off = 0;
        L.k_codes = off; off += align256((uint64_t)c.num_blocks * H * L.code_bytes);
        L.v_codes = off; off += align256((uint64_t)c.num_blocks * H * L.code_bytes);
        L.k_meta = L.v_meta = L.k_ring = L.v_ring = off;
        L.status = off;  off += kStatusBytes;
        L.total_bytes = off;
        if ((uint64_t)c.num_blocks * H * L.code_bytes >= (1ull << 32))
            return fail(KIVI_ERR_UNSUPPORTED, "code sub-array of %llu bytes exceeds 4 GiB",
                        (unsigned long long)((uint64_t)c.num_blocks * H * L.code_bytes));
        if (lay) *lay = L;
        return KIVI_OK;
    }
    if (c.k_group < c.block_size || c.k_group % c.block_size || c.k_group > 256)
        return fail(KIVI_ERR_UNSUPPORTED,
                    "k_group %d must be a multiple of block_size %d and at most 256", c.k_group,
                    c.block_size);
    {
        int pages = c.k_group / c.block_size;
        if (kivi::kHeadDim % pages || (kivi::kHeadDim / pages) % 8)
            return fail(KIVI_ERR_UNSUPPORTED,
                        "k_group/block_size = %d must divide 128 into runs of >= 8 channels", pages);
    }
    if (c.v_group != 16 && c.v_group != 32 && c.v_group != 64 && c.v_group != 128)
        return fail(KIVI_ERR_UNSUPPORTED, "v_group %d unsupported (16, 32, 64 or 128)", c.v_group);
    if (c.residual < c.k_group || c.residual % c.k_group || c.residual > 8192)
        return fail(KIVI_ERR_UNSUPPORTED,
                    "residual %d must be a multiple of k_group %d and at most 8192", c.residual,
                    c.k_group);
    if (c.num_blocks < 1) return fail(KIVI_ERR_INVALID_ARG, "num_blocks %d < 1", c.num_blocks);
    if (c.max_seqs < 1) return fail(KIVI_ERR_INVALID_ARG, "max_seqs %d < 1", c.max_seqs);
    if (c.kv_dtype != KIVI_F16 && c.kv_dtype != KIVI_BF16)
        return fail(KIVI_ERR_UNSUPPORTED, "kv_dtype %d unsupported", c.kv_dtype);
    if (c.v_flush != 0 && c.v_flush != 1)
        return fail(KIVI_ERR_UNSUPPORTED, "v_flush %d unsupported (0 or 1)", c.v_flush);

    const uint64_t H = (uint64_t)c.num_kv_heads;
    kivi_layout L{};
    L.code_bytes = (uint64_t)c.block_size * kivi::kHeadDim * c.bits / 8;
    L.k_meta_bytes = 4ull * kivi::kHeadDim * c.block_size / c.k_group;
    L.v_meta_bytes = 4ull * c.block_size * (kivi::kHeadDim / c.v_group);
    L.ring_bytes = 2ull * c.residual * kivi::kHeadDim;
    uint64_t off = 0;
    L.k_codes = off; off += align256((uint64_t)c.num_blocks * H * L.code_bytes);
    L.v_codes = off; off += align256((uint64_t)c.num_blocks * H * L.code_bytes);
    L.k_meta = off;  off += align256((uint64_t)c.num_blocks * H * L.k_meta_bytes);
    L.v_meta = off;  off += align256((uint64_t)c.num_blocks * H * L.v_meta_bytes);
    L.k_ring = off;  off += align256((uint64_t)c.max_seqs * H * L.ring_bytes);
    L.v_ring = off;  off += align256((uint64_t)c.max_seqs * H * L.ring_bytes);
    L.status = off;  off += kStatusBytes;
    L.total_bytes = off;
    // decode addresses code pages with 32-bit offsets
    if ((uint64_t)c.num_blocks * H * L.code_bytes >= (1ull << 32))
        return fail(KIVI_ERR_UNSUPPORTED, "code sub-array of %llu bytes exceeds 4 GiB",
                    (unsigned long long)((uint64_t)c.num_blocks * H * L.code_bytes));
    if (lay) *lay = L;
    return KIVI_OK;
}

kivi_status check_cache(const kivi_cache* c) {
    if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
    return KIVI_OK;
}

kivi_status device_status(int err, const char* what) {
    if (err != (int)hipSuccess)
        return fail(KIVI_ERR_DEVICE, "%s: %s", what, hipGetErrorString((hipError_t)err));
    return ok();
}

uint32_t* status_word(const kivi_cache* c) { return reinterpret_cast<uint32_t*>(c->pool + c->layout.status); }

// The first call that launches work on a cache clears its status word first,
// on the same stream (the pool's initial contents are arbitrary).
int prepare_status(const kivi_cache* c, void* stream) {
    if (c->status_cleared.load(std::memory_order_acquire)) return 0;
    if (c->status_cleared.exchange(true, std::memory_order_acq_rel)) return 0;
    const int err = kivi::launch_status_clear(status_word(c), stream);
    if (err != 0) c->status_cleared.store(false, std::memory_order_release);
    return err;
}

// Compute units of the current device (the decode split plan fills one round
// of resident work groups); 256, an MI355X's count, when it cannot be read.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < 64) {
        const int known = cache[dev].load(std::memory_order_relaxed);
        if (known > 0) return known;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace

namespace kivi {

CacheView view_of(const kivi_cache* c) {
    CacheView v{};
    const kivi_layout& L = c->layout;
    v.k_codes = c->pool + L.k_codes;
    v.v_codes = c->pool + L.v_codes;
    v.k_meta = c->pool + L.k_meta;
    v.v_meta = c->pool + L.v_meta;
    v.k_ring = reinterpret_cast<uint16_t*>(c->pool + L.k_ring);
    v.v_ring = reinterpret_cast<uint16_t*>(c->pool + L.v_ring);
    v.status = reinterpret_cast<uint32_t*>(c->pool + L.status);
    v.H = c->cfg.num_kv_heads;
    v.bits = c->cfg.bits;
    v.G = c->cfg.k_group;
    v.Gv = c->cfg.v_group;
    v.R = c->cfg.residual;
    v.Bk = c->cfg.block_size;
    v.num_blocks = c->cfg.num_blocks;
    v.max_seqs = c->cfg.max_seqs;
    v.dtype = c->cfg.kv_dtype;
    v.vflush = c->cfg.v_flush;
    v.code_bytes = (int)L.code_bytes;
    v.k_meta_bytes = (int)L.k_meta_bytes;
    v.v_meta_bytes = (int)L.v_meta_bytes;
    v.ring_elems = (int)(L.ring_bytes / 2);
    return v;
}

DecodePlan decode_plan(const kivi_cache* c, int num_seqs, int num_q_heads, int max_seq_len) {
    const int R = c->cfg.residual;
    const int H = c->cfg.num_kv_heads;
    const int gqa = std::max(1, std::min(kMaxGqa, num_q_heads / H));
    const int main_tiles = std::max(0, max_seq_len - R) / kTile;
    const int pairs = std::max(1, num_seqs * H);
    // one round of resident work groups (one 8-wave work group per compute
    // unit), at least kMinSplitTiles main tiles per split
    const int resident = device_cus();
    int n_splits = std::max(1, (resident + pairs / 2) / pairs);
    n_splits = std::min(n_splits, std::max(1, (main_tiles + kMinSplitTiles - 1) / kMinSplitTiles));
    n_splits = std::max(1, std::min(n_splits, 256));
    DecodePlan p;
    p.n_splits = n_splits;
    p.lds_bytes = decode_lds_bytes(gqa);
    p.ws_bytes = n_splits > 1 ? (size_t)num_seqs * num_q_heads * n_splits * kPartialStride * sizeof(float) : 0;
    return p;
}

}  // namespace kivi

namespace {

// Calls of the KIVI codes (bits 2, 4) and of the FP8 cache (bits 8) take only
// their own kind of cache.
kivi_status check_kivi_cache(const kivi_cache* cache) {
    kivi_status s = check_cache(cache);
    if (s != KIVI_OK) return s;
    if (cache->cfg.bits == 8)
        return fail(KIVI_ERR_UNSUPPORTED, "an FP8 cache (bits 8) takes the kivi_fp8_* calls");
    return KIVI_OK;
}
kivi_status check_fp8_cache(const kivi_cache* cache) {
    kivi_status s = check_cache(cache);
    if (s != KIVI_OK) return s;
    if (cache->cfg.bits != 8) return fail(KIVI_ERR_UNSUPPORTED, "not an FP8 cache (bits %d)", cache->cfg.bits);
    return KIVI_OK;
}

kivi_status check_heads(const kivi_cache* cache, int32_t num_q_heads) {
    const int H = cache->cfg.num_kv_heads;
    if (num_q_heads < 1) return fail(KIVI_ERR_INVALID_ARG, "num_q_heads %d < 1", num_q_heads);
    if (num_q_heads % H)
        return fail(KIVI_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    num_q_heads, H);
    if (num_q_heads / H > kivi::kMaxGqa)
        return fail(KIVI_ERR_UNSUPPORTED, "%d query heads per KV head (at most %d)",
                    num_q_heads / H, kivi::kMaxGqa);
    return KIVI_OK;
}

kivi_status prefill_common(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads, const void* d_q,
                           const int32_t* d_cu_q, int32_t max_q_len, const int32_t* d_slot_ids,
                           const int32_t* d_seq_lens, int32_t max_seq_len, const void* d_k_chunk,
                           const void* d_v_chunk, const int32_t* d_block_table, int32_t bt_stride,
                           float softmax_scale, int32_t causal, void* d_out, void* stream, bool raw_chunk) {
    kivi_status s = check_kivi_cache(cache);
    if (s != KIVI_OK) return s;
    s = check_heads(cache, num_q_heads);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0 || max_q_len < 0 || max_seq_len < 0)
        return fail(KIVI_ERR_INVALID_ARG, "bad sizes");
    if (causal != 0 && causal != 1) return fail(KIVI_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (num_seqs == 0 || max_q_len == 0) return ok();
    if (!d_q || !d_cu_q || !d_slot_ids || !d_seq_lens || !d_block_table || !d_out)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (raw_chunk && (!d_k_chunk || !d_v_chunk))
        return fail(KIVI_ERR_INVALID_ARG, "k_new / v_new is NULL");
    if (!aligned(d_q, 16) || !aligned(d_out, 16))
        return fail(KIVI_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (raw_chunk && (!aligned(d_k_chunk, 16) || !aligned(d_v_chunk, 16)))
        return fail(KIVI_ERR_INVALID_ARG, "k_new / v_new must be 16-byte aligned");
    if (!aligned(d_cu_q, 4) || !aligned(d_slot_ids, 4) || !aligned(d_seq_lens, 4) ||
        !aligned(d_block_table, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 array is not 4-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (!(softmax_scale == softmax_scale) || softmax_scale == std::numeric_limits<float>::infinity() ||
        softmax_scale == -std::numeric_limits<float>::infinity())
        return fail(KIVI_ERR_INVALID_ARG, "softmax_scale is not finite");
    if ((int64_t)max_q_len * (num_q_heads / cache->cfg.num_kv_heads) > (int64_t)INT32_MAX / 2)
        return fail(KIVI_ERR_UNSUPPORTED, "max_q_len %d too large", max_q_len);
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    int err = kivi::launch_prefill(kivi::view_of(cache), num_seqs, num_q_heads, d_q, d_cu_q, max_q_len,
                                   d_slot_ids, d_seq_lens, max_seq_len, raw_chunk ? d_k_chunk : nullptr,
                                   raw_chunk ? d_v_chunk : nullptr, d_block_table, bt_stride, softmax_scale,
                                   causal, d_out, stream);
    return device_status(err, "prefill launch");
}

}  // namespace

extern "C" {

const char* kivi_last_error(void) { return g_last_error.c_str(); }

kivi_status kivi_check_device_errors(const kivi_cache* cache, void* stream, uint32_t* flags) {
    if (flags) *flags = 0;
    kivi_status s = check_cache(cache);
    if (s != KIVI_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!cache->status_cleared.load(std::memory_order_acquire)) {
        // nothing has run on this cache yet: clear the word for later calls
        if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
        return ok();
    }
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, status_word(cache), sizeof word, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return device_status((int)e, "status word read");
    if (word == 0) return ok();
    if (int err = kivi::launch_status_clear(status_word(cache), stream)) return device_status(err, "status word clear");
    if (flags) *flags = word;
    std::string what;
    if (word & KIVI_DEVERR_PAGE) what += " page-table entry outside [0, num_blocks);";
    if (word & KIVI_DEVERR_SLOT) what += " slot id outside [0, max_seqs);";
    if (word & KIVI_DEVERR_LENGTH) what += " negative length or row count, or a position past the page table;";
    if (word & KIVI_DEVERR_QUERY) what += " prefill query span longer than max_q_len or its sequence;";
    if (word & ~0xFu) what += " unknown bits;";
    return fail(KIVI_ERR_DEVICE_ASSERT, "device-side errors (0x%x):%s those sequences' results are unspecified",
                word, what.c_str());
}

const char* kivi_status_string(kivi_status s) {
    switch (s) {
        case KIVI_OK: return "KIVI_OK";
        case KIVI_ERR_INVALID_ARG: return "KIVI_ERR_INVALID_ARG";
        case KIVI_ERR_UNSUPPORTED: return "KIVI_ERR_UNSUPPORTED";
        case KIVI_ERR_POOL_TOO_SMALL: return "KIVI_ERR_POOL_TOO_SMALL";
        case KIVI_ERR_WORKSPACE: return "KIVI_ERR_WORKSPACE";
        case KIVI_ERR_DEVICE: return "KIVI_ERR_DEVICE";
        case KIVI_ERR_DEVICE_ASSERT: return "KIVI_ERR_DEVICE_ASSERT";
    }
    return "KIVI_ERR_UNKNOWN";
}

kivi_status kivi_cache_pool_bytes(const kivi_cache_config* cfg, size_t* bytes) {
    if (!bytes) return fail(KIVI_ERR_INVALID_ARG, "bytes is NULL");
    kivi_layout L;
    kivi_status s = check_config(cfg, &L);
    if (s != KIVI_OK) return s;
    if (L.total_bytes > (uint64_t)std::numeric_limits<size_t>::max())
        return fail(KIVI_ERR_UNSUPPORTED, "pool size overflows size_t");
    *bytes = (size_t)L.total_bytes;
    return ok();
}

kivi_status kivi_cache_capacity(const kivi_cache_config* cfg, size_t budget_bytes, int32_t* num_blocks,
                                int64_t* kv_tokens) {
    if (!num_blocks || !kv_tokens) return fail(KIVI_ERR_INVALID_ARG, "output pointer is NULL");
    if (!cfg) return fail(KIVI_ERR_INVALID_ARG, "config is NULL");
    kivi_cache_config c = *cfg;
    c.num_blocks = 1;
    kivi_layout L;
    kivi_status s = check_config(&c, &L);
    if (s != KIVI_OK) return s;
    // largest block count whose pool fits the budget (and the 4 GiB code sub-array)
    const uint64_t H = (uint64_t)c.num_kv_heads;
    int64_t lo = 0, hi = std::min<int64_t>(INT32_MAX, (int64_t)(((1ull << 32) - 1) / (H * L.code_bytes)));
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        c.num_blocks = (int32_t)mid;
        kivi_layout M;
        if (check_config(&c, &M) == KIVI_OK && M.total_bytes <= (uint64_t)budget_bytes) lo = mid;
        else hi = mid - 1;
    }
    *num_blocks = (int32_t)lo;
    *kv_tokens = lo * (int64_t)c.block_size;
    return ok();
}

kivi_status kivi_cache_create(const kivi_cache_config* cfg, void* d_pool, size_t pool_bytes,
                              kivi_cache** out) {
    if (!out) return fail(KIVI_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    kivi_layout L;
    kivi_status s = check_config(cfg, &L);
    if (s != KIVI_OK) return s;
    if (!d_pool) return fail(KIVI_ERR_INVALID_ARG, "pool is NULL");
    if (!aligned(d_pool, 256)) return fail(KIVI_ERR_INVALID_ARG, "pool is not 256-byte aligned");
    if (pool_bytes < L.total_bytes)
        return fail(KIVI_ERR_POOL_TOO_SMALL, "pool has %zu bytes, needs %llu", pool_bytes,
                    (unsigned long long)L.total_bytes);
    kivi_cache* c = new (std::nothrow) kivi_cache;
    if (!c) return fail(KIVI_ERR_INVALID_ARG, "out of host memory");
    c->cfg = *cfg;
    c->layout = L;
    c->pool = static_cast<uint8_t*>(d_pool);
    *out = c;
    return ok();
}

void kivi_cache_destroy(kivi_cache* cache) { delete cache; }

kivi_status kivi_cache_layout(const kivi_cache* cache, kivi_layout* out) {
    kivi_status s = check_cache(cache);
    if (s != KIVI_OK) return s;
    if (!out) return fail(KIVI_ERR_INVALID_ARG, "out is NULL");
    *out = cache->layout;
    return ok();
}

kivi_status kivi_append_tokens(kivi_cache* cache, int32_t num_seqs, const int32_t* d_slot_ids,
                               const int32_t* d_seq_lens_before, const int32_t* d_cu_new,
                               int32_t max_new, const void* d_k_new, const void* d_v_new,
                               const int32_t* d_block_table, int32_t bt_stride, void* stream) {
    kivi_status s = check_kivi_cache(cache);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0) return fail(KIVI_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (max_new < 0) return fail(KIVI_ERR_INVALID_ARG, "max_new %d < 0", max_new);
    if (num_seqs == 0 || max_new == 0) return ok();
    if (!d_slot_ids || !d_seq_lens_before || !d_cu_new || !d_k_new || !d_v_new || !d_block_table)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_slot_ids, 4) || !aligned(d_seq_lens_before, 4) || !aligned(d_cu_new, 4) ||
        !aligned(d_block_table, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 array is not 4-byte aligned");
    if (!aligned(d_k_new, 16) || !aligned(d_v_new, 16))
        return fail(KIVI_ERR_INVALID_ARG, "k_new / v_new must be 16-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    int err = kivi::launch_append(kivi::view_of(cache), num_seqs, d_slot_ids, d_seq_lens_before,
                                  d_cu_new, max_new, d_k_new, d_v_new, d_block_table, bt_stride,
                                  stream);
    return device_status(err, "append launch");
}

kivi_status kivi_decode_workspace_bytes(const kivi_cache* cache, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_seq_len, size_t* bytes) {
    kivi_status s = check_cache(cache);
    if (s != KIVI_OK) return s;
    if (!bytes) return fail(KIVI_ERR_INVALID_ARG, "bytes is NULL");
    if (num_seqs < 0 || num_q_heads < 1 || max_seq_len < 0)
        return fail(KIVI_ERR_INVALID_ARG, "bad sizes (num_seqs %d, num_q_heads %d, max_seq_len %d)",
                    num_seqs, num_q_heads, max_seq_len);
    *bytes = cache->cfg.bits == 8
                 ? kivi::fp8_decode_plan(num_seqs, cache->cfg.num_kv_heads, num_q_heads, max_seq_len).ws_bytes
                 : kivi::decode_plan(cache, num_seqs, num_q_heads, max_seq_len).ws_bytes;
    return ok();
}

kivi_status kivi_decode_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                  const void* d_q, const int32_t* d_slot_ids,
                                  const int32_t* d_seq_lens, int32_t max_seq_len,
                                  const int32_t* d_block_table, int32_t bt_stride,
                                  float softmax_scale, void* d_out, void* d_ws, size_t ws_bytes,
                                  void* stream) {
    kivi_status s = check_kivi_cache(cache);
    if (s != KIVI_OK) return s;
    s = check_heads(cache, num_q_heads);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0) return fail(KIVI_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (max_seq_len < 0) return fail(KIVI_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
    if (num_seqs == 0) return ok();
    if (!d_q || !d_slot_ids || !d_seq_lens || !d_block_table || !d_out)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_q, 16) || !aligned(d_out, 16))
        return fail(KIVI_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!aligned(d_slot_ids, 4) || !aligned(d_seq_lens, 4) || !aligned(d_block_table, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 array is not 4-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (!(softmax_scale == softmax_scale) || softmax_scale == std::numeric_limits<float>::infinity() ||
        softmax_scale == -std::numeric_limits<float>::infinity())
        return fail(KIVI_ERR_INVALID_ARG, "softmax_scale is not finite");
    kivi::DecodePlan plan = kivi::decode_plan(cache, num_seqs, num_q_heads, max_seq_len);
    if (plan.ws_bytes > 0 && (!d_ws || ws_bytes < plan.ws_bytes))
        return fail(KIVI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", d_ws ? ws_bytes : 0,
                    plan.ws_bytes);
    if (d_ws && !aligned(d_ws, 16)) return fail(KIVI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    int err = kivi::launch_decode(kivi::view_of(cache), num_seqs, num_q_heads, d_q, d_slot_ids,
                                  d_seq_lens, d_block_table, bt_stride, softmax_scale, d_out,
                                  static_cast<float*>(d_ws), plan, stream);
    return device_status(err, "decode launch");
}

kivi_status kivi_decode_attention_noalloc(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                          const void* d_q, const int32_t* d_slot_ids, const int32_t* d_seq_lens,
                                          int32_t max_seq_len, const int32_t* d_block_table, int32_t bt_stride,
                                          float softmax_scale, void* d_out, void* stream) {
    kivi_status s = check_kivi_cache(cache);
    if (s != KIVI_OK) return s;
    s = check_heads(cache, num_q_heads);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0) return fail(KIVI_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (max_seq_len < 0) return fail(KIVI_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
    if (num_seqs == 0) return ok();
    if (!d_q || !d_slot_ids || !d_seq_lens || !d_block_table || !d_out)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_q, 16) || !aligned(d_out, 16))
        return fail(KIVI_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!aligned(d_slot_ids, 4) || !aligned(d_seq_lens, 4) || !aligned(d_block_table, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 array is not 4-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (!(softmax_scale == softmax_scale) || softmax_scale == std::numeric_limits<float>::infinity() ||
        softmax_scale == -std::numeric_limits<float>::infinity())
        return fail(KIVI_ERR_INVALID_ARG, "softmax_scale is not finite");
    kivi::DecodePlan plan = kivi::decode_plan(cache, num_seqs, num_q_heads, max_seq_len);
    if (plan.ws_bytes > kivi::kNoAllocScratchBytes)
        return fail(KIVI_ERR_WORKSPACE, "the split partials need %zu bytes, more than the %zu-byte static scratch",
                    plan.ws_bytes, kivi::kNoAllocScratchBytes);
    float* partials = nullptr;
    if (plan.ws_bytes > 0) {
        if (int e = kivi::noalloc_scratch(&partials)) return device_status(e, "static scratch address");
    }
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    int err = kivi::launch_decode(kivi::view_of(cache), num_seqs, num_q_heads, d_q, d_slot_ids, d_seq_lens,
                                  d_block_table, bt_stride, softmax_scale, d_out, partials, plan, stream);
    return device_status(err, "decode launch");
}

kivi_status kivi_decode_step(kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads, const void* d_q,
                             const int32_t* d_slot_ids, const int32_t* d_seq_lens_before, const void* d_k_new,
                             const void* d_v_new, int32_t max_seq_len, const int32_t* d_block_table,
                             int32_t bt_stride, float softmax_scale, void* d_out, void* d_ws, size_t ws_bytes,
                             void* stream) {
    kivi_status s = check_kivi_cache(cache);
    if (s != KIVI_OK) return s;
    s = check_heads(cache, num_q_heads);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0) return fail(KIVI_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (max_seq_len < 0) return fail(KIVI_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
    if (num_seqs == 0) return ok();
    if (!d_q || !d_slot_ids || !d_seq_lens_before || !d_k_new || !d_v_new || !d_block_table || !d_out)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_q, 16) || !aligned(d_out, 16) || !aligned(d_k_new, 16) || !aligned(d_v_new, 16))
        return fail(KIVI_ERR_INVALID_ARG, "q / out / k_new / v_new must be 16-byte aligned");
    if (!aligned(d_slot_ids, 4) || !aligned(d_seq_lens_before, 4) || !aligned(d_block_table, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 array is not 4-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (!(softmax_scale == softmax_scale) || softmax_scale == std::numeric_limits<float>::infinity() ||
        softmax_scale == -std::numeric_limits<float>::infinity())
        return fail(KIVI_ERR_INVALID_ARG, "softmax_scale is not finite");
    kivi::DecodePlan plan = kivi::decode_plan(cache, num_seqs, num_q_heads, max_seq_len);
    if (plan.ws_bytes > 0 && (!d_ws || ws_bytes < plan.ws_bytes))
        return fail(KIVI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", d_ws ? ws_bytes : 0,
                    plan.ws_bytes);
    if (d_ws && !aligned(d_ws, 16)) return fail(KIVI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    const kivi::CacheView view = kivi::view_of(cache);
    if (view.vflush) {
        // Values flush with the Keys: a flush step quantises R Value tokens,
        // which the append kernel spreads over its work group; the attention
        // follows on the same stream over the seq_lens_before + 1 tokens.
        int err = kivi::launch_append(view, num_seqs, d_slot_ids, d_seq_lens_before, nullptr, 1, d_k_new,
                                      d_v_new, d_block_table, bt_stride, stream);
        if (err == 0)
            err = kivi::launch_decode(view, num_seqs, num_q_heads, d_q, d_slot_ids, d_seq_lens_before,
                                      d_block_table, bt_stride, softmax_scale, d_out, static_cast<float*>(d_ws),
                                      plan, stream, 1);
        return device_status(err, "decode step launch");
    }
    int err = kivi::launch_decode_step(view, num_seqs, num_q_heads, d_q, d_slot_ids, d_seq_lens_before, d_k_new,
                                       d_v_new, d_block_table, bt_stride, softmax_scale, d_out,
                                       static_cast<float*>(d_ws), plan, stream);
    return device_status(err, "decode step launch");
}

kivi_status kivi_fp8_append_tokens(kivi_cache* cache, int32_t num_seqs, const int32_t* d_seq_lens_before,
                                   const int32_t* d_cu_new, int32_t max_new, const void* d_k_new,
                                   const void* d_v_new, const float* d_k_scale, const float* d_v_scale,
                                   const int32_t* d_block_table, int32_t bt_stride, void* stream) {
    kivi_status s = check_fp8_cache(cache);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0) return fail(KIVI_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (max_new < 0) return fail(KIVI_ERR_INVALID_ARG, "max_new %d < 0", max_new);
    if (num_seqs == 0 || max_new == 0) return ok();
    if (!d_seq_lens_before || !d_cu_new || !d_k_new || !d_v_new || !d_k_scale || !d_v_scale || !d_block_table)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_seq_lens_before, 4) || !aligned(d_cu_new, 4) || !aligned(d_block_table, 4) ||
        !aligned(d_k_scale, 4) || !aligned(d_v_scale, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 or float array is not 4-byte aligned");
    if (!aligned(d_k_new, 2) || !aligned(d_v_new, 2))
        return fail(KIVI_ERR_INVALID_ARG, "k_new / v_new must be 2-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    int err = kivi::launch_fp8_append(kivi::view_of(cache), cache->cfg.scale_per_head, num_seqs, d_seq_lens_before,
                                      d_cu_new, max_new, d_k_new, d_v_new, d_k_scale, d_v_scale, d_block_table,
                                      bt_stride, stream);
    return device_status(err, "FP8 append launch");
}

kivi_status kivi_fp8_decode_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                      const void* d_q, const int32_t* d_seq_lens, int32_t max_seq_len,
                                      const float* d_k_scale, const float* d_v_scale,
                                      const int32_t* d_block_table, int32_t bt_stride, float softmax_scale,
                                      void* d_out, void* d_ws, size_t ws_bytes, void* stream) {
    kivi_status s = check_fp8_cache(cache);
    if (s != KIVI_OK) return s;
    s = check_heads(cache, num_q_heads);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0) return fail(KIVI_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (max_seq_len < 0) return fail(KIVI_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
    if (num_seqs == 0) return ok();
    if (!d_q || !d_seq_lens || !d_k_scale || !d_v_scale || !d_block_table || !d_out)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_q, 16) || !aligned(d_out, 16))
        return fail(KIVI_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!aligned(d_seq_lens, 4) || !aligned(d_block_table, 4) || !aligned(d_k_scale, 4) || !aligned(d_v_scale, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 or float array is not 4-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (!(softmax_scale == softmax_scale) || softmax_scale == std::numeric_limits<float>::infinity() ||
        softmax_scale == -std::numeric_limits<float>::infinity())
        return fail(KIVI_ERR_INVALID_ARG, "softmax_scale is not finite");
    const kivi::Fp8Plan plan = kivi::fp8_decode_plan(num_seqs, cache->cfg.num_kv_heads, num_q_heads, max_seq_len);
    if (plan.ws_bytes > 0 && (!d_ws || ws_bytes < plan.ws_bytes))
        return fail(KIVI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", d_ws ? ws_bytes : 0, plan.ws_bytes);
    if (d_ws && !aligned(d_ws, 16)) return fail(KIVI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    int err = kivi::launch_fp8_decode(kivi::view_of(cache), cache->cfg.scale_per_head, num_seqs, num_q_heads, d_q,
                                      d_seq_lens, d_k_scale, d_v_scale, d_block_table, bt_stride, softmax_scale,
                                      d_out, static_cast<float*>(d_ws), plan, stream);
    return device_status(err, "FP8 decode launch");
}

kivi_status kivi_fp8_decode_step(kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads, const void* d_q,
                                 const int32_t* d_seq_lens_before, const void* d_k_new, const void* d_v_new,
                                 int32_t max_seq_len, const float* d_k_scale, const float* d_v_scale,
                                 const int32_t* d_block_table, int32_t bt_stride, float softmax_scale, void* d_out,
                                 void* d_ws, size_t ws_bytes, void* stream) {
    kivi_status s = check_fp8_cache(cache);
    if (s != KIVI_OK) return s;
    s = check_heads(cache, num_q_heads);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0) return fail(KIVI_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (max_seq_len < 0) return fail(KIVI_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
    if (num_seqs == 0) return ok();
    if (!d_q || !d_seq_lens_before || !d_k_new || !d_v_new || !d_k_scale || !d_v_scale || !d_block_table || !d_out)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_q, 16) || !aligned(d_out, 16))
        return fail(KIVI_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!aligned(d_k_new, 2) || !aligned(d_v_new, 2))
        return fail(KIVI_ERR_INVALID_ARG, "k_new / v_new must be 2-byte aligned");
    if (!aligned(d_seq_lens_before, 4) || !aligned(d_block_table, 4) || !aligned(d_k_scale, 4) ||
        !aligned(d_v_scale, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 or float array is not 4-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (!(softmax_scale == softmax_scale) || softmax_scale == std::numeric_limits<float>::infinity() ||
        softmax_scale == -std::numeric_limits<float>::infinity())
        return fail(KIVI_ERR_INVALID_ARG, "softmax_scale is not finite");
    const kivi::Fp8Plan plan = kivi::fp8_decode_plan(num_seqs, cache->cfg.num_kv_heads, num_q_heads, max_seq_len);
    if (plan.ws_bytes > 0 && (!d_ws || ws_bytes < plan.ws_bytes))
        return fail(KIVI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", d_ws ? ws_bytes : 0, plan.ws_bytes);
    if (d_ws && !aligned(d_ws, 16)) return fail(KIVI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    // the append (one row per sequence), then the attention over T + 1 tokens
    const kivi::CacheView view = kivi::view_of(cache);
    int err = kivi::launch_fp8_append(view, cache->cfg.scale_per_head, num_seqs, d_seq_lens_before, nullptr, 1,
                                      d_k_new, d_v_new, d_k_scale, d_v_scale, d_block_table, bt_stride, stream);
    if (err != 0) return device_status(err, "FP8 decode step append launch");
    err = kivi::launch_fp8_decode(view, cache->cfg.scale_per_head, num_seqs, num_q_heads, d_q, d_seq_lens_before,
                                  d_k_scale, d_v_scale, d_block_table, bt_stride, softmax_scale, d_out,
                                  static_cast<float*>(d_ws), plan, stream, 1);
    return device_status(err, "FP8 decode step attention launch");
}

kivi_status kivi_fp8_prefill_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                       const void* d_q, const int32_t* d_cu_q, int32_t max_q_len,
                                       const int32_t* d_seq_lens, int32_t max_seq_len, const float* d_k_scale,
                                       const float* d_v_scale, const int32_t* d_block_table, int32_t bt_stride,
                                       float softmax_scale, int32_t causal, void* d_out, void* stream) {
    kivi_status s = check_fp8_cache(cache);
    if (s != KIVI_OK) return s;
    s = check_heads(cache, num_q_heads);
    if (s != KIVI_OK) return s;
    if (num_seqs < 0 || max_q_len < 0 || max_seq_len < 0) return fail(KIVI_ERR_INVALID_ARG, "bad sizes");
    if (causal != 0 && causal != 1) return fail(KIVI_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (num_seqs == 0 || max_q_len == 0) return ok();
    if (!d_q || !d_cu_q || !d_seq_lens || !d_k_scale || !d_v_scale || !d_block_table || !d_out)
        return fail(KIVI_ERR_INVALID_ARG, "a device pointer is NULL");
    if (!aligned(d_q, 16) || !aligned(d_out, 16))
        return fail(KIVI_ERR_INVALID_ARG, "q / out must be 16-byte aligned");
    if (!aligned(d_cu_q, 4) || !aligned(d_seq_lens, 4) || !aligned(d_block_table, 4) || !aligned(d_k_scale, 4) ||
        !aligned(d_v_scale, 4))
        return fail(KIVI_ERR_INVALID_ARG, "an int32 or float array is not 4-byte aligned");
    if (bt_stride < 1) return fail(KIVI_ERR_INVALID_ARG, "bt_stride %d < 1", bt_stride);
    if (!(softmax_scale == softmax_scale) || softmax_scale == std::numeric_limits<float>::infinity() ||
        softmax_scale == -std::numeric_limits<float>::infinity())
        return fail(KIVI_ERR_INVALID_ARG, "softmax_scale is not finite");
    const int g = num_q_heads / cache->cfg.num_kv_heads;
    if ((int64_t)max_q_len * g > (int64_t)INT32_MAX / 2)
        return fail(KIVI_ERR_UNSUPPORTED, "max_q_len %d too large", max_q_len);
    if (int e = prepare_status(cache, stream)) return device_status(e, "status word clear");
    int err = kivi::launch_fp8_prefill(kivi::view_of(cache), cache->cfg.scale_per_head, num_seqs, num_q_heads, d_q,
                                       d_cu_q, max_q_len, d_seq_lens, d_k_scale, d_v_scale, d_block_table, bt_stride,
                                       softmax_scale, causal, d_out, stream);
    return device_status(err, "FP8 prefill launch");
}

kivi_status kivi_prefill_workspace_bytes(const kivi_cache* cache, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t max_q_len,
                                         int32_t max_seq_len, size_t* bytes) {
    kivi_status s = check_cache(cache);
    if (s != KIVI_OK) return s;
    if (!bytes) return fail(KIVI_ERR_INVALID_ARG, "bytes is NULL");
    if (num_seqs < 0 || num_q_heads < 1 || max_q_len < 0 || max_seq_len < 0)
        return fail(KIVI_ERR_INVALID_ARG, "bad sizes");
    *bytes = 0;
    return ok();
}

kivi_status kivi_prefill_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                   const void* d_q, const int32_t* d_cu_q, int32_t max_q_len,
                                   const int32_t* d_slot_ids, const int32_t* d_seq_lens,
                                   int32_t max_seq_len, const int32_t* d_block_table,
                                   int32_t bt_stride, float softmax_scale, int32_t causal,
                                   void* d_out, void* d_ws, size_t ws_bytes, void* stream) {
    (void)d_ws;
    (void)ws_bytes;
    return prefill_common(cache, num_seqs, num_q_heads, d_q, d_cu_q, max_q_len, d_slot_ids, d_seq_lens,
                          max_seq_len, nullptr, nullptr, d_block_table, bt_stride, softmax_scale, causal,
                          d_out, stream, false);
}

kivi_status kivi_prefill_attention_raw_chunk(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                             const void* d_q, const int32_t* d_cu_q, int32_t max_q_len,
                                             const int32_t* d_slot_ids, const int32_t* d_seq_lens_before,
                                             const void* d_k_new, const void* d_v_new, int32_t max_seq_len,
                                             const int32_t* d_block_table, int32_t bt_stride,
                                             float softmax_scale, int32_t causal, void* d_out, void* d_ws,
                                             size_t ws_bytes, void* stream) {
    (void)d_ws;
    (void)ws_bytes;
    return prefill_common(cache, num_seqs, num_q_heads, d_q, d_cu_q, max_q_len, d_slot_ids, d_seq_lens_before,
                          max_seq_len, d_k_new, d_v_new, d_block_table, bt_stride, softmax_scale, causal,
                          d_out, stream, true);
}

}  // extern "C"
