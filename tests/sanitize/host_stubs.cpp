// Stand-ins for the device side of libkivi, for a host-only build of the C ABI
// under AddressSanitizer / UndefinedBehaviorSanitizer: the kernel launchers
// check what the host code hands them and launch nothing, and the few HIP
// runtime calls the host code makes report "no device" (nothing here touches a
// GPU, whatever machine runs it).
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "kivi_internal.h"

namespace {
void need(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "host stub: %s\n", what);
        std::abort();
    }
}
void view_ok(const kivi::CacheView& v) {
    need(v.k_codes && v.v_codes && v.status, "cache view pointers");
    need(v.H >= 1 && v.Bk >= 16 && v.num_blocks >= 1 && v.max_seqs >= 1, "cache view sizes");
}
}  // namespace

namespace kivi {

int launch_status_clear(uint32_t* status, void*) {
    need(status != nullptr, "status word");
    return 0;
}
int launch_append(const CacheView& v, int num_seqs, const int32_t* slot_ids, const int32_t* seq_lens_before,
                  const int32_t*, int max_new, const void* k_new, const void* v_new, const int32_t* block_table,
                  int bt_stride, void*) {
    view_ok(v);
    need(num_seqs > 0 && max_new > 0 && slot_ids && seq_lens_before && k_new && v_new && block_table &&
             bt_stride > 0, "append arguments");
    return 0;
}
int launch_decode_step(const CacheView& v, int num_seqs, int num_q_heads, const void* q, const int32_t* slot_ids,
                       const int32_t* seq_lens_before, const void* k_new, const void* v_new,
                       const int32_t* block_table, int bt_stride, float, void* out, float* partials,
                       const DecodePlan& plan, void*) {
    view_ok(v);
    need(num_seqs > 0 && num_q_heads % v.H == 0 && q && slot_ids && seq_lens_before && k_new && v_new &&
             block_table && bt_stride > 0 && out, "decode step arguments");
    need(plan.n_splits >= 1 && (plan.n_splits == 1 || partials), "decode step plan");
    return 0;
}
int launch_decode(const CacheView& v, int num_seqs, int num_q_heads, const void* q, const int32_t* slot_ids,
                  const int32_t* seq_lens, const int32_t* block_table, int bt_stride, float, void* out,
                  float* partials, const DecodePlan& plan, void*, int len_add) {
    view_ok(v);
    need(num_seqs > 0 && num_q_heads % v.H == 0 && q && slot_ids && seq_lens && block_table && bt_stride > 0 &&
             out && (len_add == 0 || len_add == 1), "decode arguments");
    need(plan.n_splits >= 1 && (plan.n_splits == 1 || partials), "decode plan");
    return 0;
}
int launch_prefill(const CacheView& v, int num_seqs, int num_q_heads, const void* q, const int32_t* cu_q,
                   int max_q_len, const int32_t* slot_ids, const int32_t* seq_lens, int, const void*,
                   const void*, const int32_t* block_table, int bt_stride, float, int causal, void* out, void*) {
    view_ok(v);
    need(num_seqs > 0 && num_q_heads % v.H == 0 && q && cu_q && max_q_len > 0 && slot_ids && seq_lens &&
             block_table && bt_stride > 0 && out && (causal == 0 || causal == 1), "prefill arguments");
    return 0;
}
Fp8Plan fp8_decode_plan(int num_seqs, int, int num_q_heads, int) {
    Fp8Plan p;
    p.n_splits = 2;
    p.ws_bytes = (size_t)num_seqs * num_q_heads * 2 * kPartialStride * sizeof(float);
    return p;
}
size_t decode_lds_bytes(int g) { return (size_t)g * 4096; }
int launch_fp8_append(const CacheView& v, int per_head, int num_seqs, const int32_t* seq_lens_before,
                      const int32_t*, int max_new, const void* k_new, const void* v_new, const float* k_scale,
                      const float* v_scale, const int32_t* block_table, int bt_stride, void*) {
    view_ok(v);
    need((per_head == 0 || per_head == 1) && num_seqs > 0 && max_new > 0 && seq_lens_before && k_new && v_new &&
             k_scale && v_scale && block_table && bt_stride > 0, "FP8 append arguments");
    return 0;
}
int launch_fp8_prefill(const CacheView& v, int, int num_seqs, int num_q_heads, const void* q, const int32_t* cu_q,
                       int max_q_len, const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                       const int32_t* block_table, int bt_stride, float, int, void* out, void*) {
    view_ok(v);
    need(num_seqs > 0 && num_q_heads % v.H == 0 && q && cu_q && max_q_len > 0 && seq_lens && k_scale && v_scale &&
             block_table && bt_stride > 0 && out, "FP8 prefill arguments");
    return 0;
}
int launch_fp8_decode(const CacheView& v, int, int num_seqs, int num_q_heads, const void* q, const int32_t* seq_lens,
                      const float* k_scale, const float* v_scale, const int32_t* block_table, int bt_stride, float,
                      void* out, float* partials, const Fp8Plan& plan, void*, int) {
    view_ok(v);
    need(num_seqs > 0 && num_q_heads % v.H == 0 && q && seq_lens && k_scale && v_scale && block_table &&
             bt_stride > 0 && out && (plan.n_splits == 1 || partials), "FP8 decode arguments");
    return 0;
}
int noalloc_scratch(float** out) {
    static float host_stand_in[16];
    *out = host_stand_in;
    return 0;
}

}  // namespace kivi

extern "C" {
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
const char* hipGetErrorString(hipError_t) { return "no device (host-only build)"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void*, size_t bytes, hipMemcpyKind, hipStream_t) {
    std::memset(dst, 0, bytes);  // a clean status word
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}
