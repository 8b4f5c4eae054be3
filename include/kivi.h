/*
 * kivi.h - C ABI of a KIVI-style low-bit KV cache with paged attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("4.4 KV Cache 量化", sections 3.1 and 3.2):
 *   - Key is quantised per channel: for each channel, G consecutive tokens
 *     share one (scale, zero-point) pair.
 *   - Value is quantised per token: for each token, Gv consecutive channels
 *     share one pair.
 *   - Inside a group the map is min/max asymmetric with b in {2, 4} bits:
 *       scale = (max - min) / (2^b - 1), zero = min, both stored as fp16,
 *       code  = clamp(round_half_even((x - zero) / scale), 0, 2^b - 1),
 *     computed in IEEE single precision against the stored fp16 pair.
 *   - New tokens first enter a full-precision residual. Key tokens are
 *     quantised in one batch of R tokens (R/G groups) once R have gathered.
 *     Value keeps the newest R tokens; each new token pushes the oldest one
 *     out, and that token is quantised.
 *   - Attention reads the quantised history and the residual together and
 *     restores values on read ("给 KV cache 减肥", section 3.1;
 *     "4.4 KV Cache 量化", section 2: P = softmax(Q K^T / sqrt(d)), out = P V).
 * After T tokens a sequence holds T_K = R*floor(T/R) quantised Key tokens and
 * T_V = max(0, T - R) quantised Value tokens; the rest is residual.
 *
 * Conventions
 *   - Pointers named d_* are device memory on the current HIP device. All
 *     other pointers are host memory.
 *   - `stream` is a hipStream_t passed as void* (0 = the null stream). Calls
 *     that launch work are asynchronous on that stream and return once the
 *     launches are queued.
 *   - Every argument check happens before any launch; a call that returns an
 *     argument or configuration error (INVALID_ARG, UNSUPPORTED,
 *     POOL_TOO_SMALL, WORKSPACE) has launched nothing and changed nothing.
 *     KIVI_ERR_DEVICE means a launch failed; the calls that make two
 *     launches (kivi_fp8_decode_step, and kivi_decode_step on a v_flush
 *     cache) may then have run the first one (the append) already.
 *   - Values read from device memory (slot ids, page ids, lengths, row
 *     offsets) are range-checked in the kernels in every build. One outside
 *     its range is skipped, so no memory outside the pool, the inputs and
 *     the outputs is touched, and the kernel sets a bit in the pool's status
 *     word (kivi_device_error). The results for that sequence are then
 *     unspecified; the other sequences of the call are unaffected.
 *     kivi_check_device_errors() reports and clears the word: a serving loop
 *     calls it when it synchronises anyway, so a bad page table fails fast
 *     instead of serving wrong output.
 *   - Only head_dim 128 is supported (the product pages restrict their
 *     backend to head_dim 128 standard attention and fail fast otherwise);
 *     anything else is KIVI_ERR_UNSUPPORTED, never silently ignored.
 *   - Thread safety: calls on different caches may run concurrently. Calls
 *     on one cache must not overlap on the device in ways that race on the
 *     same sequence (the caller orders them, e.g. on one stream).
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kivi_status {
    KIVI_OK = 0,
    KIVI_ERR_INVALID_ARG = 1,    /* null/misaligned pointer, negative count, bad stride */
    KIVI_ERR_UNSUPPORTED = 2,    /* configuration outside what the library implements */
    KIVI_ERR_POOL_TOO_SMALL = 3, /* pool_bytes below kivi_cache_pool_bytes() */
    KIVI_ERR_WORKSPACE = 4,      /* workspace missing or smaller than required */
    KIVI_ERR_DEVICE = 5,         /* a HIP call or kernel launch failed */
    KIVI_ERR_DEVICE_ASSERT = 6   /* a kernel met an out-of-range id or length
                                    (kivi_check_device_errors) */
} kivi_status;

/* Bits of the pool's status word, set by kernels that skip what they cannot
 * use (see kivi_check_device_errors).                                       */
typedef enum kivi_device_error {
    KIVI_DEVERR_PAGE = 1,    /* a page-table entry outside [0, num_blocks) for a
                                position the call reads or writes */
    KIVI_DEVERR_SLOT = 2,    /* a residual slot id outside [0, max_seqs) */
    KIVI_DEVERR_LENGTH = 4,  /* a negative length or row count, or a position
                                past the page table (bt_stride pages) */
    KIVI_DEVERR_QUERY = 8    /* a prefill query span longer than max_q_len or
                                than its sequence */
} kivi_device_error;

typedef enum kivi_dtype {
    KIVI_F16 = 0,  /* IEEE binary16 */
    KIVI_BF16 = 1  /* bfloat16 (values must lie in the fp16 range: the
                      scale and zero-point are stored as fp16) */
} kivi_dtype;

/* Cache configuration (one attention layer).
 *   num_kv_heads  H_KV >= 1
 *   head_dim      must be 128
 *   bits          2 or 4 (KIVI codes), or 8: the FP8 cache ("4.4 KV Cache 量化",
 *                 section 4: K and V stored as FP8 E4M3, the format ROCm
 *                 supports, with no groups and no residual; k_group,
 *                 v_group, residual and v_flush must then be 0, and only the
 *                 kivi_fp8_* calls and kivi_decode_workspace_bytes take it)
 *   k_group       G: Key tokens per (channel) group; a multiple of block_size,
 *                 and 128 must be divisible by G/block_size
 *   v_group       Gv: Value channels per (token) group: 16, 32, 64 or 128
 *   residual      R: residual length in tokens; a multiple of G
 *   block_size    Bk: tokens per physical page; a multiple of 16
 *   num_blocks    physical pages in the pool (>= 1)
 *   max_seqs      residual slots (>= 1); a sequence uses the slot the caller
 *                 assigns it
 *   kv_dtype      kivi_dtype of the K/V tokens, the residual and q/out
 *   v_flush       when Value tokens leave the residual ("4.4 KV Cache 量化",
 *                 section 3.2 gives the window; the other is its open
 *                 variant): 0 = sliding window, the oldest of the R newest
 *                 tokens is quantised as each new token arrives, so the
 *                 Value boundary is max(0, T - R); 1 = with the Keys, the R
 *                 residual tokens are quantised (each per token over Gv
 *                 channels) at every Key flush, so the boundary is
 *                 R*floor(T/R) for both. Any other value is
 *                 KIVI_ERR_UNSUPPORTED. A zero-initialised config takes 0.
 *   scale_per_head FP8 scale granularity (section 4.2 of the same page): 0 =
 *                 one Key and one Value scale for the tensor, 1 = one of each
 *                 per KV head. Must be 0 when bits is 2 or 4.               */
typedef struct kivi_cache_config {
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t bits;
    int32_t k_group;
    int32_t v_group;
    int32_t residual;
    int32_t block_size;
    int32_t num_blocks;
    int32_t max_seqs;
    int32_t kv_dtype;
    int32_t v_flush;
    int32_t scale_per_head;
} kivi_cache_config;

/* Byte offsets of the sub-arrays inside the pool (each 256-byte aligned) and
 * their strides. The pool layout (all multi-byte fields little-endian):
 *
 *   K codes  [num_blocks][H_KV][code_bytes]   code_bytes = Bk*128*b/8
 *   V codes  [num_blocks][H_KV][code_bytes]
 *   K meta   [num_blocks][H_KV][k_meta_bytes] k_meta_bytes = 4*128*Bk/G
 *   V meta   [num_blocks][H_KV][Bk][128/Gv][2] fp16 (scale, zero)
 *   K ring   [max_seqs][H_KV][R][128]  kv_dtype, token-major
 *   V ring   [max_seqs][H_KV][R/4][128][4]  kv_dtype: quads of 4 ring rows,
 *            channel-major inside a quad
 *   status   256 bytes; the first 32-bit word holds kivi_device_error bits
 *
 * A token at position p of a sequence lives in page block_table[p / Bk], row
 * p % Bk; in the residual it lives in ring row r = p % R: K ring row r, V
 * ring quad r / 4, element [channel][r % 4].
 *
 * K meta: the G/Bk pages of Key group j (tokens jG .. jG+G-1) each hold the
 * pairs of nch = 128*Bk/G channels: page i of the group holds channels
 * [i*nch, (i+1)*nch) as fp16 scale[nch] followed by fp16 zero[nch].
 *
 * Code chunk of one (page, head): Bk/16 sub-tiles of 16 tokens, each
 * 16*128*b/8 bytes. With L = m + 16*j (m, j integers, 0 <= m < 16,
 * 0 <= j < 4), sub-tile lane slot L is the (4*b)-byte run at offset 4*b*L:
 *   int4 K: slot L = token m; 32-bit word w (w = 0..3) holds channels
 *           c0 = 32w + 8j .. c0+7: even channels c0+2e in bits 4e..4e+3,
 *           odd channels c0+2e+1 in bits 16+4e..16+4e+3 (e = 0..3).
 *   int4 V: slot L = channels {16t + m : t = 0..7}, tokens 4j..4j+3; word w
 *           covers channels a = 32w + m and c = 32w + 16 + m. Nibble at bit
 *           4e: e=0 (a,4j) 1 (a,4j+2) 2 (c,4j) 3 (c,4j+2) 4 (a,4j+1)
 *           5 (a,4j+3) 6 (c,4j+1) 7 (c,4j+3).
 *   int2 K: slot L = token m; word w (w = 0..1) holds channel groups
 *           c0 = 64w + 8j (fields 0..3 and 8..11) and c1 = 64w + 32 + 8j
 *           (fields 4..7 and 12..15), 2-bit field f at bits 2f: field f<8
 *           holds channel base + 2(f%4), field 8+f holds base + 2(f%4) + 1,
 *           base = c0 for f%8 < 4 else c1.
 *   int2 V: slot L = channels {16t + m}, tokens 4j..4j+3; word w (w = 0..1)
 *           covers channel tiles t = 4w .. 4w+3; field f (f = 0..7) of the
 *           low half holds (tile 4w + f/2, token 4j + 2(f%2)) and field 8+f
 *           holds (tile 4w + f/2, token 4j + 2(f%2) + 1).
 * The layout lets a lane turn a 32-bit word into fp16 pairs with one
 * AND-OR per pair (the fp16 bias-exponent trick) and feed matrix cores
 * directly.
 *
 * FP8 cache (bits 8): only K codes, V codes and the status word,
 * code_bytes = Bk*128, one E4M3 byte per element; the meta and ring
 * sub-arrays are empty. Each
 * 16-token sub-tile (2 KiB) is 64 lane slots of 32 bytes:
 *   K: slot L = token m, byte 8i + e holds channel 32i + 8j + e
 *      (i = 0..3, e = 0..7);
 *   V: slot L = channels {16t + m : t = 0..7}, tokens 4j..4j+3; byte
 *      4t + r holds (channel 16t + m, token 4j + r).
 * An E4M3 byte b read as the fp16 bits ((b & 0x80) << 8) | ((b & 0x7F) << 7)
 * is its value times 2^-8, subnormals included.                              */
typedef struct kivi_layout {
    uint64_t k_codes, v_codes, k_meta, v_meta, k_ring, v_ring;
    uint64_t total_bytes;
    uint64_t code_bytes;     /* per (page, head) */
    uint64_t k_meta_bytes;   /* per (page, head) */
    uint64_t v_meta_bytes;   /* per (page, head) */
    uint64_t ring_bytes;     /* per (slot, head), K and V alike */
    uint64_t status;         /* offset of the 256-byte status sub-array */
} kivi_layout;

typedef struct kivi_cache kivi_cache;

/* Pool size for `cfg` in bytes. Host only; validates exactly as create.
 * Errors: INVALID_ARG (null), UNSUPPORTED (see kivi_cache_config).            */
kivi_status kivi_cache_pool_bytes(const kivi_cache_config* cfg, size_t* bytes);

/* Capacity of a memory budget: the largest num_blocks whose pool (with
 * cfg's other fields; cfg->num_blocks is ignored) fits in budget_bytes, and
 * the tokens those pages hold (num_blocks * block_size, per layer, all KV
 * heads). This is the density the product pages sell ("S4 KV": about three
 * times the fp16 KV tokens per GPU for int4) and the M_KV estimate of
 * "4.4 KV Cache 量化", section 1, with this layout's group metadata and
 * residual rings included. Host only, no device work.
 * A Key or Value code sub-array is limited to 4 GiB (32-bit page offsets),
 * which caps num_blocks for very large budgets.
 * Outputs: *num_blocks (0 when not even the rings fit), *kv_tokens.
 * Errors: INVALID_ARG (null), UNSUPPORTED (as kivi_cache_pool_bytes).       */
kivi_status kivi_cache_capacity(const kivi_cache_config* cfg, size_t budget_bytes, int32_t* num_blocks,
                                int64_t* kv_tokens);

/* Bind a cache to the caller's device pool. The caller allocates and owns
 * d_pool (256-byte aligned, at least kivi_cache_pool_bytes()) and frees it
 * after kivi_cache_destroy(). The handle holds host metadata only: no device
 * allocation, no device work, no synchronisation. The pool's initial
 * contents do not matter; a sequence's state is given by its length. The
 * first call that launches work on the cache also clears the status word
 * (one small kernel on that call's stream, queued before its own kernels).
 * Errors: INVALID_ARG, UNSUPPORTED, POOL_TOO_SMALL.                          */
kivi_status kivi_cache_create(const kivi_cache_config* cfg, void* d_pool, size_t pool_bytes,
                              kivi_cache** out);

/* Release the handle (NULL-safe). Never touches the pool.                    */
void kivi_cache_destroy(kivi_cache* cache);

/* Offsets and strides of the pool's sub-arrays.                              */
kivi_status kivi_cache_layout(const kivi_cache* cache, kivi_layout* out);

/* Append new tokens ("4.4 KV Cache 量化", section 3.2; "给 KV cache 减肥",
 * section 3.1: quantise before writing).
 *   num_seqs            sequences in this call (0 is a no-op)
 *   d_slot_ids[S]       residual slot of each sequence (distinct in a call)
 *   d_seq_lens_before[S] tokens already in each sequence
 *   d_cu_new[S+1]       sequence s appends rows d_cu_new[s] .. d_cu_new[s+1]-1
 *   max_new             host upper bound of d_cu_new[s+1] - d_cu_new[s]
 *   d_k_new, d_v_new    [total_new][H_KV][128] kv_dtype
 *   d_block_table       [S][bt_stride] int32 page ids; pages must exist for
 *                       every position < seq_len_before + n_new
 * The result equals appending the rows one at a time: Value tokens leaving
 * the R-token window are quantised per token, the new rows enter the
 * residual, and every time a sequence's Key residual reaches R tokens those
 * R tokens are quantised per channel as R/G groups. The library keeps no
 * per-sequence length: lengths are the caller's.
 * Errors: INVALID_ARG, DEVICE.                                               */
kivi_status kivi_append_tokens(kivi_cache* cache, int32_t num_seqs, const int32_t* d_slot_ids,
                               const int32_t* d_seq_lens_before, const int32_t* d_cu_new,
                               int32_t max_new, const void* d_k_new, const void* d_v_new,
                               const int32_t* d_block_table, int32_t bt_stride, void* stream);

/* Workspace bytes kivi_decode_attention needs for these sizes (0 when no
 * sequence is split across work groups). The workspace holds the per-split
 * partial results between the attention kernel and the merge kernel of one
 * call; it needs no initialisation. Calls that share a workspace must not
 * overlap on the device.                                                    */
kivi_status kivi_decode_workspace_bytes(const kivi_cache* cache, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_seq_len, size_t* bytes);

/* Decode attention: one query per sequence ("4.4 KV Cache 量化", section 2,
 * over the quantised history plus the residual, section 3.2).
 *   d_q[S][H_Q][128]    kv_dtype; query head hq reads KV head hq / (H_Q/H_KV)
 *   d_seq_lens[S]       tokens in each sequence (after its append); the query
 *                       attends all of them
 *   max_seq_len         host upper bound of d_seq_lens
 *   softmax_scale       multiplies q.k (1/sqrt(128) for standard attention)
 *   d_out[S][H_Q][128]  kv_dtype; a sequence of length 0 gets zeros
 *   d_ws, ws_bytes      device workspace of kivi_decode_workspace_bytes()
 *                       bytes (may be NULL when that is 0)
 * H_Q must be a multiple of H_KV with H_Q/H_KV <= 16 (else UNSUPPORTED).
 * Split plan: a long sequence's tokens may be cut over several work groups
 * whose partial results a second kernel merges; how many depends on the
 * whole call (num_seqs * H_KV against the device's compute units) and on
 * max_seq_len. A sequence's output therefore may differ in its last bits
 * (within the attention tolerance) between batches of different size or
 * devices of different size; the same call on the same device gives the
 * same bits every time.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE.                        */
kivi_status kivi_decode_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                  const void* d_q, const int32_t* d_slot_ids,
                                  const int32_t* d_seq_lens, int32_t max_seq_len,
                                  const int32_t* d_block_table, int32_t bt_stride,
                                  float softmax_scale, void* d_out, void* d_ws, size_t ws_bytes,
                                  void* stream);

/* kivi_decode_attention for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments and results as kivi_decode_attention without the
 * workspace: the split partials live in a static device array of 4 MiB per
 * GPU, held from the first call on a device until the process ends. The
 * call allocates nothing; on its first call on a device it looks up that
 * device's copy of the array. Every call on one device shares the array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be ordered by the caller. Nothing in the array needs to start at zero.
 * A call whose partials need more than 4 MiB (num_seqs * H_Q * splits * 528
 * bytes, see kivi_decode_workspace_bytes) returns KIVI_ERR_WORKSPACE.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE.                       */
kivi_status kivi_decode_attention_noalloc(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                          const void* d_q, const int32_t* d_slot_ids, const int32_t* d_seq_lens,
                                          int32_t max_seq_len, const int32_t* d_block_table, int32_t bt_stride,
                                          float softmax_scale, void* d_out, void* stream);

/* One decode step in one launch: append one token per sequence (as
 * kivi_append_tokens with one row each: the Value eviction, the Key flush
 * when the residual fills, the residual write; "4.4 KV Cache 量化", section
 * 3.2) and then attend with that token's query over the sequence's T + 1
 * tokens (as kivi_decode_attention). The cache state and the outputs are
 * those of the two calls in a row. A cache with v_flush = 1 (a flush step
 * quantises R Value tokens) runs the step as those two launches.
 *   d_seq_lens_before[S]  tokens before this step (the query sits at position T)
 *   d_k_new, d_v_new      [S][H_KV][128] kv_dtype, row s is sequence s's token
 *   max_seq_len           host upper bound of d_seq_lens_before + 1 (also
 *                         for kivi_decode_workspace_bytes)
 * Other arguments as kivi_decode_attention; slot ids must be distinct.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE.                        */
kivi_status kivi_decode_step(kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads, const void* d_q,
                             const int32_t* d_slot_ids, const int32_t* d_seq_lens_before, const void* d_k_new,
                             const void* d_v_new, int32_t max_seq_len, const int32_t* d_block_table,
                             int32_t bt_stride, float softmax_scale, void* d_out, void* d_ws, size_t ws_bytes,
                             void* stream);

/* Append to an FP8 cache (bits 8): every new K/V element x is stored as
 * E4M3(x / scale), with x / scale rounded in single precision, saturated to
 * +-448 and rounded to the nearest E4M3 value, ties to even ("4.4 KV Cache
 * 量化", section 4.2: the scale brings values into FP8's range).
 *   d_seq_lens_before[S], d_cu_new[S+1], max_new, d_k_new, d_v_new,
 *   d_block_table, bt_stride   as for kivi_append_tokens (no residual slots)
 *   d_k_scale, d_v_scale       device float32 scales, positive and finite:
 *                              1 value each, or H_KV when scale_per_head
 * The caller guarantees pages for positions < seq_len_before + n_new.
 * Errors: INVALID_ARG, UNSUPPORTED (not an FP8 cache), DEVICE.               */
kivi_status kivi_fp8_append_tokens(kivi_cache* cache, int32_t num_seqs, const int32_t* d_seq_lens_before,
                                   const int32_t* d_cu_new, int32_t max_new, const void* d_k_new,
                                   const void* d_v_new, const float* d_k_scale, const float* d_v_scale,
                                   const int32_t* d_block_table, int32_t bt_stride, void* stream);

/* Decode attention over an FP8 cache ("4.4 KV Cache 量化", sections 2 and
 * 4.5: values are restored, value * scale, before attention uses them; the
 * attention itself runs in fp32). One query row per sequence at position
 * T - 1, attending over all T = d_seq_lens[s] tokens.
 *   d_q[S][H_Q][128] kv_dtype, d_out[S][H_Q][128] kv_dtype
 *   d_k_scale, d_v_scale       as for kivi_fp8_append_tokens
 *   d_ws, ws_bytes             kivi_decode_workspace_bytes of this cache
 * Other arguments as for kivi_decode_attention (no slot ids). A row with
 * T = 0 writes zeros.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE.                       */
kivi_status kivi_fp8_decode_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                      const void* d_q, const int32_t* d_seq_lens, int32_t max_seq_len,
                                      const float* d_k_scale, const float* d_v_scale,
                                      const int32_t* d_block_table, int32_t bt_stride, float softmax_scale,
                                      void* d_out, void* d_ws, size_t ws_bytes, void* stream);

/* One decode step on an FP8 cache: append one token per sequence (as
 * kivi_fp8_append_tokens with one row each) and then attend with that
 * token's query over the sequence's T + 1 tokens (as
 * kivi_fp8_decode_attention), in two launches on the stream. The cache
 * bytes and the outputs are those of the two calls in a row.
 *   d_seq_lens_before[S]  tokens before this step (the query sits at position T)
 *   d_k_new, d_v_new      [S][H_KV][128] kv_dtype, row s is sequence s's token
 *   max_seq_len           host upper bound of d_seq_lens_before + 1 (also
 *                         for kivi_decode_workspace_bytes)
 * Other arguments as kivi_fp8_decode_attention. The caller guarantees a page
 * for position d_seq_lens_before[s].
 * Errors: INVALID_ARG, UNSUPPORTED (not an FP8 cache), WORKSPACE, DEVICE.    */
kivi_status kivi_fp8_decode_step(kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads, const void* d_q,
                                 const int32_t* d_seq_lens_before, const void* d_k_new, const void* d_v_new,
                                 int32_t max_seq_len, const float* d_k_scale, const float* d_v_scale,
                                 const int32_t* d_block_table, int32_t bt_stride, float softmax_scale, void* d_out,
                                 void* d_ws, size_t ws_bytes, void* stream);

/* Chunked prefill attention over an FP8 cache ("4.4 KV Cache 量化", sections
 * 2 and 4.5: values restored, value * scale, attention in fp32), after the
 * chunk's tokens were appended with kivi_fp8_append_tokens.
 *   d_q[total_q][H_Q][128] kv_dtype; rows of sequence s are d_cu_q[s] ..
 *                       d_cu_q[s+1]-1 and row i sits at position
 *                       seq_len_s - n_q,s + i
 *   causal              1: row i attends positions 0..its own; 0: all
 *   d_out[total_q][H_Q][128] kv_dtype (a row that sees no token gets zeros)
 *   d_k_scale, d_v_scale as for kivi_fp8_append_tokens
 * Other arguments as for kivi_fp8_decode_attention; no workspace.
 * Errors: INVALID_ARG, UNSUPPORTED, DEVICE.                                   */
kivi_status kivi_fp8_prefill_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                       const void* d_q, const int32_t* d_cu_q, int32_t max_q_len,
                                       const int32_t* d_seq_lens, int32_t max_seq_len, const float* d_k_scale,
                                       const float* d_v_scale, const int32_t* d_block_table, int32_t bt_stride,
                                       float softmax_scale, int32_t causal, void* d_out, void* stream);

/* Workspace bytes kivi_prefill_attention needs (0 today; reserved).          */
kivi_status kivi_prefill_workspace_bytes(const kivi_cache* cache, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t max_q_len,
                                         int32_t max_seq_len, size_t* bytes);

/* Chunked prefill attention ("4.4 KV Cache 量化", section 2) over the cache
 * as stored, after the chunk's tokens were appended.
 *   d_q[total_q][H_Q][128] kv_dtype; rows of sequence s are d_cu_q[s] ..
 *                       d_cu_q[s+1]-1 and row i sits at position
 *                       seq_len_s - n_q,s + i
 *   causal              1: row i attends positions 0..its own; 0: all
 *   max_q_len           host upper bound of every span d_cu_q[s+1] - d_cu_q[s];
 *                       max_q_len * (H_Q/H_KV) must stay below 2^30
 *                       (else UNSUPPORTED). A span longer than max_q_len or
 *                       than its sequence sets KIVI_DEVERR_QUERY, and its
 *                       rows are not all written
 *   d_out[total_q][H_Q][128] kv_dtype
 * Other arguments as for kivi_decode_attention.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, DEVICE.                        */
kivi_status kivi_prefill_attention(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                   const void* d_q, const int32_t* d_cu_q, int32_t max_q_len,
                                   const int32_t* d_slot_ids, const int32_t* d_seq_lens,
                                   int32_t max_seq_len, const int32_t* d_block_table,
                                   int32_t bt_stride, float softmax_scale, int32_t causal,
                                   void* d_out, void* d_ws, size_t ws_bytes, void* stream);

/* Chunked prefill in which the chunk is quantised for storage only: its rows
 * attend over the history as the cache holds it (section 2 of "4.4 KV Cache
 * 量化" over the quantised tokens plus the section 3.2 residual) followed by
 * the chunk's own Keys and Values exactly as given (the pages leave the
 * prefill open; this is the reading in which the newest tokens, here the
 * whole chunk, keep full precision). Call it BEFORE kivi_append_tokens stores
 * the same chunk, on the same stream: the append may quantise and overwrite
 * the residual this call reads.
 *   d_seq_lens_before[S]  tokens in the cache before the chunk; row i of
 *                         sequence s sits at position seq_len_before_s + i
 *   d_k_new, d_v_new      [total_q][H_KV][128] kv_dtype, the chunk's rows
 *                         indexed like d_q (the arrays kivi_append_tokens
 *                         then takes with d_cu_new = d_cu_q); 16-byte aligned
 *   causal                1: row i sees positions 0..its own; 0: the whole
 *                         history and chunk
 *   d_block_table         pages must exist for positions < seq_len_before
 *                         (the chunk's pages are not read)
 * Other arguments as kivi_prefill_attention; the workspace is unused.
 * Errors: INVALID_ARG, UNSUPPORTED, DEVICE.                                  */
kivi_status kivi_prefill_attention_raw_chunk(const kivi_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                             const void* d_q, const int32_t* d_cu_q, int32_t max_q_len,
                                             const int32_t* d_slot_ids, const int32_t* d_seq_lens_before,
                                             const void* d_k_new, const void* d_v_new, int32_t max_seq_len,
                                             const int32_t* d_block_table, int32_t bt_stride,
                                             float softmax_scale, int32_t causal, void* d_out, void* d_ws,
                                             size_t ws_bytes, void* stream);

/* Device-side errors since the last check ("S4 KV": an unsupported input
 * fails fast rather than giving wrong output; "给 KV cache 减肥", section 3.2:
 * nothing the caller asked for is silently ignored). Waits for `stream`,
 * reads the pool's status word, clears it (a small kernel queued on
 * `stream`) and stores its kivi_device_error bits in *flags (flags may be
 * NULL). Kernels on other streams that still run may set bits after the
 * read; order them before the call.
 * Returns KIVI_OK when no bit was set, KIVI_ERR_DEVICE_ASSERT (the message
 * names the errors) when one was, INVALID_ARG, or DEVICE (a HIP call
 * failed).                                                                  */
kivi_status kivi_check_device_errors(const kivi_cache* cache, void* stream, uint32_t* flags);

/* Message for the last failure on the calling thread ("" if none).           */
const char* kivi_last_error(void);

/* Static name of a status code.                                              */
const char* kivi_status_string(kivi_status status);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H */
