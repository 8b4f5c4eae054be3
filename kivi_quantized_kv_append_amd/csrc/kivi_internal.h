// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <atomic>
#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "kivi.h"

struct kivi_cache {
    kivi_cache_config cfg;
    kivi_layout layout;
    uint8_t* pool;   // caller-owned device memory
    // set once the first launching call has queued the clear of the pool's
    // status word (the pool's initial contents are arbitrary)
    mutable std::atomic<bool> status_cleared{false};
};

namespace kivi {

constexpr int kHeadDim = 128;
constexpr int kTile = 16;          // tokens per matrix-core tile
constexpr int kMaxGqa = 16;        // query heads per KV head (matrix-core N dimension)

// Launch-time view of a cache: plain values and device pointers.
struct CacheView {
    uint8_t* k_codes;
    uint8_t* v_codes;
    uint8_t* k_meta;
    uint8_t* v_meta;
    uint16_t* k_ring;
    uint16_t* v_ring;
    uint32_t* status;  // kivi_device_error bits, set with vector atomics
    int H, bits, G, Gv, R, Bk, num_blocks, max_seqs, dtype;
    int code_bytes, k_meta_bytes, v_meta_bytes, ring_elems;
    int vflush;  // 0: sliding Value window; 1: Values flush with the Keys
};

// Element (position p, channel c) of a Value ring of R tokens: ring rows in
// quads, each quad [128 channels][4 tokens], so a channel's 4 tokens of a
// quad are 8 contiguous bytes and one token's 128 channels span 1 KiB.
__host__ __device__ inline size_t vring_index(int R, int p, int c) {
    const int r = p % R;
    return (size_t)(r >> 2) * (kHeadDim * 4) + (size_t)c * 4 + (size_t)(r & 3);
}

// Value tokens quantised after T appends: the window keeps the R newest
// tokens; with vflush the Values share the Key boundary R*floor(T/R).
__host__ __device__ inline int value_boundary(const CacheView& v, int T) {
    return v.vflush ? v.R * (T / v.R) : (T > v.R ? T - v.R : 0);
}

CacheView view_of(const kivi_cache* c);

// Split plan for decode: the grid has n_splits work groups per (sequence,
// KV head); a sequence uses min(n_splits, ceil(main tiles / kMinSplitTiles))
// of them (at least one). With more than one split the workspace holds the
// partials and a merge kernel follows.
constexpr int kMinSplitTiles = 64;
struct DecodePlan {
    int n_splits;
    size_t lds_bytes;   // dynamic LDS of one decode work group
    size_t ws_bytes;
};
DecodePlan decode_plan(const kivi_cache* c, int num_seqs, int num_q_heads, int max_seq_len);
size_t decode_lds_bytes(int gqa);

constexpr int kPartialStride = 132;  // floats per partial: m, l, pad, pad, o[128]

// Static split-partial array of kivi_decode_attention_noalloc (per device).
constexpr size_t kNoAllocScratchBytes = 4u << 20;
constexpr int kMaxDevices = 64;
// The calling thread's current device's copy of that array (its address is
// looked up once per device); returns a hipError_t as int.
int noalloc_scratch(float** out);

// Work groups per (sequence, KV head) for the quantisation phase of an
// append of up to max_new rows per sequence: one part per 64 new rows, at
// most 64 parts. One part runs the whole append in a single launch.
inline int append_parts(int max_new) {
    const int p = (max_new + 63) / 64;
    return p < 1 ? 1 : (p > 64 ? 64 : p);
}

// Zero the status word (one thread of one work group), on `stream`.
int launch_status_clear(uint32_t* status, void* stream);

// Kernel launchers (return a hipError_t as int).
int launch_append(const CacheView& v, int num_seqs, const int32_t* slot_ids,
                  const int32_t* seq_lens_before, const int32_t* cu_new, int max_new,
                  const void* k_new, const void* v_new, const int32_t* block_table, int bt_stride,
                  void* stream);

// Append one token per sequence and attend, in one launch (plus the merge
// when sequences are split). seq_lens_before: lengths before the token.
int launch_decode_step(const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                       const int32_t* slot_ids, const int32_t* seq_lens_before, const void* k_new,
                       const void* v_new, const int32_t* block_table, int bt_stride, float softmax_scale,
                       void* out, float* partials, const DecodePlan& plan, void* stream);

// len_add: tokens an earlier launch on the stream appended after seq_lens
// was taken (0 or 1).
int launch_decode(const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                  const int32_t* slot_ids, const int32_t* seq_lens, const int32_t* block_table,
                  int bt_stride, float softmax_scale, void* out, float* partials,
                  const DecodePlan& plan, void* stream, int len_add = 0);

int launch_prefill(const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                   const int32_t* cu_q, int max_q_len, const int32_t* slot_ids,
                   const int32_t* seq_lens, int max_seq_len, const void* k_chunk,
                   const void* v_chunk, const int32_t* block_table, int bt_stride,
                   float softmax_scale, int causal, void* out, void* stream);

// FP8 (E4M3) cache: decode split plan and the kernel launchers.
struct Fp8Plan {
    int n_splits;
    size_t ws_bytes;
};
Fp8Plan fp8_decode_plan(int num_seqs, int num_kv_heads, int num_q_heads, int max_seq_len);
int launch_fp8_append(const CacheView& v, int per_head, int num_seqs, const int32_t* seq_lens_before,
                      const int32_t* cu_new, int max_new, const void* k_new, const void* v_new,
                      const float* k_scale, const float* v_scale, const int32_t* block_table, int bt_stride,
                      void* stream);
int launch_fp8_prefill(const CacheView& v, int per_head, int num_seqs, int num_q_heads, const void* q,
                       const int32_t* cu_q, int max_q_len, const int32_t* seq_lens, const float* k_scale,
                       const float* v_scale, const int32_t* block_table, int bt_stride, float softmax_scale,
                       int causal, void* out, void* stream);
int launch_fp8_decode(const CacheView& v, int per_head, int num_seqs, int num_q_heads, const void* q,
                      const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                      const int32_t* block_table, int bt_stride, float softmax_scale, void* out, float* partials,
                      const Fp8Plan& plan, void* stream, int len_add = 0);

}  // namespace kivi
