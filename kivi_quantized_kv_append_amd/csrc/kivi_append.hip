// Append kernel: one work group of 256 threads per (sequence, KV head), or
// gridDim.y parts of one for a bulk append (a prefill chunk): Key groups and
// Value token quads are dealt round-robin, every unit writes disjoint code
// words and metadata, and phase B (the new residual rows, dealt round-robin
// over the same parts) then runs as a second launch on the same stream, after
// every part has read the ring. The work of
// one (sequence, head) is append_body (kivi_append_body.h).

#include "kivi_append_body.h"

namespace kivi {
namespace {

constexpr int kAppendThreads = 256;

template <int BITS, int DT>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
    __shared__ AppendShared<kAppendThreads> sm;
    const int s = blockIdx.x / a.v.H, h = blockIdx.x % a.v.H;
    // no row offsets: one row per sequence, in sequence order
    const int row0 = a.cu_new ? a.cu_new[s] : s;
    const int n = a.cu_new ? a.cu_new[s + 1] - row0 : 1;
    append_body<BITS, DT, kAppendThreads>(a, s, h, row0, n, threadIdx.x, blockIdx.y, gridDim.y, sm);
}

__global__ __launch_bounds__(64) void status_clear_kernel(uint32_t* status) {
    if (threadIdx.x == 0) status[0] = 0u;
}

}  // namespace

int launch_status_clear(uint32_t* status, void* stream) {
    hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), status);
    return (int)hipGetLastError();
}

int launch_append(const CacheView& v, int num_seqs, const int32_t* slot_ids,
                  const int32_t* seq_lens_before, const int32_t* cu_new, int max_new,
                  const void* k_new, const void* v_new, const int32_t* block_table, int bt_stride,
                  void* stream) {
    AppendArgs a;
    a.v = v;
    a.slot_ids = slot_ids;
    a.seq_lens_before = seq_lens_before;
    a.cu_new = cu_new;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto launch = [&](int mode, int parts) {
        a.mode = mode;
        dim3 grid((unsigned)(num_seqs * v.H), (unsigned)parts), block(kAppendThreads);
        if (v.bits == 4) {
            if (v.dtype == kF16) hipLaunchKernelGGL((append_kernel<4, kF16>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((append_kernel<4, kBF16>), grid, block, 0, st, a);
        } else {
            if (v.dtype == kF16) hipLaunchKernelGGL((append_kernel<2, kF16>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((append_kernel<2, kBF16>), grid, block, 0, st, a);
        }
    };
    // max_new only sizes the split; every part count covers every unit
    const int parts = append_parts(max_new);
    if (parts <= 1) {
        launch(0, 1);
    } else {
        launch(1, parts);
        launch(2, parts);
    }
    return (int)hipGetLastError();
}

}  // namespace kivi
