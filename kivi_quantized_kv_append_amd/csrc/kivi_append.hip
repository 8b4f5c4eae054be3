// Append / quantise-on-flush kernel ("4.4 KV Cache 量化", sections 3.1-3.2;
// "给 KV cache 减肥", section 3.1: quantise before writing).
//
// One work group per (sequence, KV head). For a sequence with T0 tokens that
// receives n new rows (T1 = T0 + n) the group computes the final state
// directly, which equals n single-token appends:
//   * Key: tokens [R*floor(T0/R), R*floor(T1/R)) are quantised per channel,
//     G tokens per group (the residual reached R tokens that many times);
//   * Value: tokens [max(0,T0-R), max(0,T1-R)) left the R-token window and
//     are quantised per token, Gv channels per group;
//   * the residual ring receives the new rows that stay full precision.
// Phase A (all quantisation) reads the old ring and the new rows; a barrier
// separates it from phase B (ring writes), which may overwrite ring slots
// phase A read. Distinct sequences touch disjoint pages and ring slots.
//
// Bulk appends (a prefill chunk) split phase A over gridDim.y parts per
// (sequence, head): Key groups and Value token quads are dealt round-robin,
// every unit writes disjoint code words and metadata, and phase B then runs
// as a second launch on the same stream, after every part has read the ring.

#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kMaxG = 256;

struct AppendArgs {
    CacheView v;
    const int32_t* slot_ids;
    const int32_t* seq_lens_before;
    const int32_t* cu_new;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int32_t* block_table;
    int bt_stride;
    int mode;  // 0: phases A and B; 1: phase A only (split over gridDim.y); 2: phase B only
};

template <int BITS, int DT>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;  // one 16-token sub-tile
    constexpr int SLOT_BYTES = 4 * BITS;                     // bytes per lane slot
    const CacheView& V = a.v;
    const int H = V.H;
    const int s = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int tid = threadIdx.x;
    const int part = blockIdx.y, nparts = gridDim.y;

    const int slot = a.slot_ids[s];
    const int T0 = a.seq_lens_before[s];
    const int row0 = a.cu_new[s];
    const int n = a.cu_new[s + 1] - row0;
    if (slot < 0 || slot >= V.max_seqs || T0 < 0 || n <= 0) return;
    const int T1 = T0 + n;
    const int R = V.R, G = V.G, Gv = V.Gv, Bk = V.Bk;
    const int TK0 = R * (T0 / R), TK1 = R * (T1 / R);
    const int TV0 = max(0, T0 - R), TV1 = max(0, T1 - R);
    const int32_t* bt = a.block_table + (size_t)s * a.bt_stride;
    const int bt_len = a.bt_stride;

    uint16_t* ringK = V.k_ring + ((size_t)slot * H + h) * V.ring_elems;  // [R][128]
    uint16_t* ringV = V.v_ring + ((size_t)slot * H + h) * V.ring_elems;  // [128][R]
    const size_t in_stride = (size_t)H * kHeadDim;
    const uint16_t* inK = a.k_new + (size_t)row0 * in_stride + (size_t)h * kHeadDim;
    const uint16_t* inV = a.v_new + (size_t)row0 * in_stride + (size_t)h * kHeadDim;

    auto page_of = [&](int p) -> int {
        int bi = p / Bk;
        if (bi >= bt_len) return -1;
        int blk = bt[bi];
        return (blk >= 0 && blk < V.num_blocks) ? blk : -1;
    };
    auto kval = [&](int p, int c) -> float {
        uint16_t u = p < T0 ? ringK[(size_t)(p % R) * kHeadDim + c] : inK[(size_t)(p - T0) * in_stride + c];
        return canon(to_f32<DT>(u));
    };
    auto vval = [&](int p, int c) -> float {
        uint16_t u = p < T0 ? ringV[(size_t)c * R + (p % R)] : inV[(size_t)(p - T0) * in_stride + c];
        return canon(to_f32<DT>(u));
    };

    // A one-row append (a decode step) loads its new row here, so the load
    // travels with phase A's ring reads instead of after them.
    const bool one_row = (n == 1);
    uint4 row_k = {0, 0, 0, 0};
    uint16_t row_v = 0;
    if (one_row) {
        if (tid < 16) row_k = *reinterpret_cast<const uint4*>(inK + 8 * tid);
        if (tid < kHeadDim) row_v = inV[tid];
    }

    __shared__ float sm_min[2][kHeadDim], sm_max[2][kHeadDim];
    __shared__ float sm_S[kHeadDim], sm_Z[kHeadDim];
    __shared__ uint8_t sm_codes[kMaxG * kHeadDim];
    __shared__ float sm_v[4][4][kHeadDim];
    __shared__ float sm_vp[4][4][8][2];

    if (a.mode != 2) {
    // ---------------- phase A1: Key flush, one group at a time ----------------
    {
        const int c = tid & (kHeadDim - 1);
        const int half = tid >> 7;
        const int nch = kHeadDim * Bk / G;  // channels per K-meta page slot
        for (int j = TK0 / G + part; j < TK1 / G; j += nparts) {
            const int base = j * G;
            const int lo = half * (G / 2), hi = lo + G / 2;
            float mn = INFINITY, mx = -INFINITY;
            for (int i = lo; i < hi; ++i) {
                float x = kval(base + i, c);
                mn = fminf(mn, x);
                mx = fmaxf(mx, x);
            }
            sm_min[half][c] = mn;
            sm_max[half][c] = mx;
            __syncthreads();
            if (half == 0) {
                mn = fminf(sm_min[0][c], sm_min[1][c]);
                mx = fmaxf(sm_max[0][c], sm_max[1][c]);
                uint16_t s16, z16;
                float S, Z;
                group_params(mn, mx, QMAX, s16, z16, S, Z);
                sm_S[c] = S;
                sm_Z[c] = Z;
                int blk = page_of(base + (c / nch) * Bk);
                if (blk >= 0) {
                    uint16_t* meta = reinterpret_cast<uint16_t*>(V.k_meta + ((size_t)blk * H + h) * V.k_meta_bytes);
                    meta[c % nch] = s16;
                    meta[nch + c % nch] = z16;
                }
            }
            __syncthreads();
            {
                const float S = sm_S[c], Z = sm_Z[c];
                for (int i = lo; i < hi; ++i)
                    sm_codes[i * kHeadDim + c] = (uint8_t)group_code(kval(base + i, c), S, Z, QMAX);
            }
            __syncthreads();
            // pack the group's code words (every word of these tokens is written)
            constexpr int WPT = kHeadDim * BITS / 32;  // 32-bit words per token
            for (int q = tid; q < G * WPT; q += kAppendThreads) {
                const int i = q / WPT, wi = q % WPT;
                const int p = base + i;
                const int blk = page_of(p);
                if (blk < 0) continue;
                const int sub = (p % Bk) / kTile, m = p % kTile;
                const uint8_t* cd = &sm_codes[i * kHeadDim];
                uint32_t word = 0;
                int jj, w;
                if constexpr (BITS == 4) {
                    jj = wi >> 2; w = wi & 3;
                    const int c0 = 32 * w + 8 * jj;
                    for (int e = 0; e < 4; ++e) {
                        word |= (uint32_t)cd[c0 + 2 * e] << (4 * e);
                        word |= (uint32_t)cd[c0 + 2 * e + 1] << (16 + 4 * e);
                    }
                } else {
                    jj = wi >> 1; w = wi & 1;
                    const int c0 = 64 * w + 8 * jj, c1 = c0 + 32;
                    for (int f = 0; f < 8; ++f) {
                        const int b = (f < 4 ? c0 : c1) + 2 * (f & 3);
                        word |= (uint32_t)cd[b] << (2 * f);
                        word |= (uint32_t)cd[b + 1] << (16 + 2 * f);
                    }
                }
                const int L = m + 16 * jj;
                uint8_t* dst = V.k_codes + ((size_t)blk * H + h) * V.code_bytes + sub * TILE_BYTES +
                               SLOT_BYTES * L + 4 * w;
                *reinterpret_cast<uint32_t*>(dst) = word;
            }
            __syncthreads();
        }
    }

    // ---------------- phase A2: Value evictions, one token quad per wave ----------------
    {
        const int wave = tid >> 6, lane = tid & 63;
        const int ng = kHeadDim / Gv;
        const int gw = Gv / 2;  // lanes per channel group (two channels per lane)
        const int q_lo = TV0 / 4, q_hi = (TV1 + 3) / 4;
        const int rounds = TV1 > TV0 ? (q_hi - q_lo + 3) / 4 : 0;
        for (int rd = part; rd < rounds; rd += nparts) {
            const int qd = q_lo + rd * 4 + wave;
            const bool active = qd < q_hi;
            const int p0 = 4 * qd;
            if (active) {
                for (int r = 0; r < 4; ++r) {
                    const int p = p0 + r;
                    if (p < TV0 || p >= TV1) continue;
                    const float x0 = vval(p, 2 * lane), x1 = vval(p, 2 * lane + 1);
                    sm_v[wave][r][2 * lane] = x0;
                    sm_v[wave][r][2 * lane + 1] = x1;
                    const float mn = group_min(fminf(x0, x1), gw);
                    const float mx = group_max(fmaxf(x0, x1), gw);
                    if ((lane % gw) == 0) {
                        const int g = (2 * lane) / Gv;
                        uint16_t s16, z16;
                        float S, Z;
                        group_params(mn, mx, QMAX, s16, z16, S, Z);
                        sm_vp[wave][r][g][0] = S;
                        sm_vp[wave][r][g][1] = Z;
                        const int blk = page_of(p);
                        if (blk >= 0) {
                            uint16_t* meta = reinterpret_cast<uint16_t*>(
                                V.v_meta + ((size_t)blk * H + h) * V.v_meta_bytes) + ((p % Bk) * ng + g) * 2;
                            meta[0] = s16;
                            meta[1] = z16;
                        }
                    }
                }
            }
            __syncthreads();
            if (active) {
                const int blk = page_of(p0);
                const int sub = (p0 % Bk) / kTile, jq = (p0 % kTile) / 4;
                auto code_at = [&](int r, int ch) -> uint32_t {
                    const int g = ch / Gv;
                    return group_code(sm_v[wave][r][ch], sm_vp[wave][r][g][0], sm_vp[wave][r][g][1], QMAX);
                };
                bool in[4];
                for (int r = 0; r < 4; ++r) in[r] = (p0 + r >= TV0) && (p0 + r < TV1);
                const int words = (BITS == 4) ? 64 : 32;
                // The call that writes a quad's first token stores whole words
                // (fields of later tokens zero); later calls OR their fields in,
                // so no word is read back.
                const bool fresh = p0 >= TV0;
                if (blk >= 0 && lane < words) {
                    const int m = lane & 15, w = lane >> 4;
                    const int L = m + 16 * jq;
                    uint32_t* dst = reinterpret_cast<uint32_t*>(V.v_codes + ((size_t)blk * H + h) * V.code_bytes +
                                                                sub * TILE_BYTES + SLOT_BYTES * L + 4 * w);
                    uint32_t word = 0u;
                    if constexpr (BITS == 4) {
                        const int ca = 32 * w + m, cc = ca + 16;
                        // nibble e: (a,0) (a,2) (c,0) (c,2) (a,1) (a,3) (c,1) (c,3)
                        const int ech[8] = {ca, ca, cc, cc, ca, ca, cc, cc};
                        const int etk[8] = {0, 2, 0, 2, 1, 3, 1, 3};
                        for (int e = 0; e < 8; ++e) {
                            const int r = etk[e];
                            if (!in[r]) continue;
                            word |= code_at(r, ech[e]) << (4 * e);
                        }
                    } else {
                        // field f (low half) = (tile 4w + f/2, token 2(f%2)); field 8+f = token + 1
                        for (int f = 0; f < 16; ++f) {
                            const int ff = f & 7;
                            const int ch = 16 * (4 * w + ff / 2) + m;
                            const int r = 2 * (ff & 1) + (f >> 3);
                            if (!in[r]) continue;
                            word |= code_at(r, ch) << (2 * f);
                        }
                    }
                    if (fresh) *dst = word;
                    else __hip_atomic_fetch_or(dst, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __syncthreads();
        }
    }

    }  // phase A
    if (a.mode == 1) return;
    __syncthreads();

    // ---------------- phase B: new rows that stay in the residual ----------------
    {
        const int k_first = max(TK1, T0), v_first = max(TV1, T0);
        const int nk = T1 - k_first, nv = T1 - v_first;
        if (one_row) {  // the row is at position T0 (nk, nv <= 1)
            if (nk > 0 && tid < 16) *reinterpret_cast<uint4*>(ringK + (size_t)(T0 % R) * kHeadDim + 8 * tid) = row_k;
            if (nv > 0 && tid < kHeadDim) ringV[(size_t)tid * R + (T0 % R)] = row_v;
            return;
        }
        // Key ring: token-major rows, 16-byte chunks
        for (int q = tid; q < nk * 16; q += kAppendThreads) {
            const int p = k_first + q / 16, ch = (q % 16) * 8;
            const uint4 val = *reinterpret_cast<const uint4*>(inK + (size_t)(p - T0) * in_stride + ch);
            *reinterpret_cast<uint4*>(ringK + (size_t)(p % R) * kHeadDim + ch) = val;
        }
        // Value ring: channel-major
        for (int q = tid; q < nv * kHeadDim; q += kAppendThreads) {
            const int ch = q / nv, p = v_first + q % nv;
            ringV[(size_t)ch * R + (p % R)] = inV[(size_t)(p - T0) * in_stride + ch];
        }
    }
}

}  // namespace

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
        launch(2, 1);
    }
    return (int)hipGetLastError();
}

}  // namespace kivi
