// Split-K paged decode attention over the KIVI cache, dequantising on read
// ("4.4 KV Cache 量化", section 2: P = softmax(Q K^T / sqrt(d)), out = P V;
// section 3.2: the residual takes part next to the quantised history;
// "给 KV cache 减肥", section 3.1: values are restored when the query reads
// them).
//
// Work: one work group (4 waves) per (sequence, KV head, split). Splits cover
// "main" 16-token tiles whose Key and Value are both quantised; one extra
// split per (sequence, KV head) covers the tail tiles that touch the
// residual. A partial (running max m, sum l, unnormalised o) per query head
// and split goes to the workspace; the combine kernel merges them.
//
// Per main tile (16 tokens), per wave:
//   scores  S^T[16 tok][16 q-heads] = K_codes[16][128] x Q'^T[128][16]
//           on matrix cores (v_mfma_f32_16x16x32_f16), with the Key scale
//           folded into the query (Q' = q * scale, per channel and group) and
//           the zero-point folded into a per-group bias (sum_c q_c zero_c);
//   softmax online, per query head, in registers (exp2 domain);
//   values  O^T[128][16] += V_codes^T[128][16 tok] x W[16 tok][16]
//           (one v_mfma_f32_16x16x32_f16 per 16-channel tile), with
//           W = p * scale_V per token and sum_t p_t zero_t kept apart.
// Folded operands (Q' and W) carry about 22 bits: each is split into an fp16
// head and an fp16 tail (x = hi + lo). Codes are exact small integers in
// fp16, so the products lose nothing beyond fp32 accumulation. The Key side
// runs the tile twice (hi, lo); the Value side fills the MFMA's 32-deep K
// dimension with (codes, codes) against (W_hi, W_lo).
// Codes become fp16 integers with one AND-OR per pair (bits placed in an
// fp16 mantissa under the exponent of 1024) and one packed subtract.
// Query heads of a KV head (GQA) are the matrix N dimension (<= 16).

#include <algorithm>

#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kHalf = 2;  // tiles per load buffer; two buffers per wave
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
    CacheView v;
    const uint16_t* q;
    const int32_t* slot_ids;
    const int32_t* seq_lens;
    const int32_t* block_table;
    int bt_stride;
    int num_q_heads;
    int gqa;
    float scale_log2;
    float* partials;
    int* counters;    // one per (sequence, KV head); zero between calls
    int n_splits;
    int tiles_per_split;
    int lds_groups;   // Key groups whose query tables fit the work group's LDS
    int tpg_shift;    // log2(tiles per Key group)
    int tpp_shift;    // log2(tiles per page)
    uint32_t code_array_bytes, vmeta_array_bytes;
    uint16_t* out;
};

// fp16 pair (1024 + x_lo, 1024 + x_hi) from two code fields placed in the
// low mantissa bits of each half: one AND-OR with the exponent of 1024. The
// 1024 offsets are taken out later from accumulated sums (query-side bias,
// value-side weight sum), not per element.
__device__ __forceinline__ uint32_t magic_pair(uint32_t x, uint32_t mask) {
    uint32_t r;
    const uint32_t magic = 0x64006400u;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
    return r;
}

// Exact fp16 pair (x_lo, x_hi): the magic pair less 1024 in each half.
__device__ __forceinline__ uint32_t exact_pair(uint32_t x, uint32_t mask) {
    h2 v = __builtin_bit_cast(h2, magic_pair(x, mask));
    v = v - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ h8 make_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(h8, (u4){a, b, c, d});
}
__device__ __forceinline__ h4 make_h4(uint32_t a, uint32_t b) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(h4, (u2){a, b});
}

// x = hi + lo with both parts fp16 (about 22 significant bits together)
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}

__device__ __forceinline__ h8 dup_h8(h4 a) { return (h8){a[0], a[1], a[2], a[3], a[0], a[1], a[2], a[3]}; }

// Reductions over the four lanes n, n+16, n+32, n+48 (one query head):
// gfx950 row swaps exchange 16-lane rows and 32-lane halves in one VALU op.
__device__ __forceinline__ float xor_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float xor_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Raw buffer loads: a uniform byte offset (scalar) plus the lane's offset.
// Reads past the buffer's size return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const u4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return (uint4){v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint2 buf_b64(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    const u2v v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    return (uint2){v.x, v.y};
}

// Key A-operands of the 4 score MFMAs from this lane's code slot, as exact
// fp16 integers (a rounding in the scores is amplified by the exponential).
// int4: word i covers channels 32i+8j..+7 (even in the low half, odd in the
// high half), pair factors 1,16,1,16. int2: word w covers MFMAs 2w (fields
// 0..3) and 2w+1 (fields 4..7), pair factors 1,4,16,64.
template <int BITS>
__device__ __forceinline__ void unpack_k(const uint32_t* kw, h8 A[4]) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = kw[i], w8 = w >> 8;
            A[i] = make_h8(exact_pair(w, 0x000F000Fu), exact_pair(w, 0x00F000F0u),
                           exact_pair(w8, 0x000F000Fu), exact_pair(w8, 0x00F000F0u));
        }
    } else {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t x = kw[w], x8 = x >> 8;
            A[2 * w] = make_h8(exact_pair(x, 0x00030003u), exact_pair(x, 0x000C000Cu),
                               exact_pair(x, 0x00300030u), exact_pair(x, 0x00C000C0u));
            A[2 * w + 1] = make_h8(exact_pair(x8, 0x00030003u), exact_pair(x8, 0x000C000Cu),
                                   exact_pair(x8, 0x00300030u), exact_pair(x8, 0x00C000C0u));
        }
    }
}

// Value A-operands of the 8 PV MFMAs (one per 16-channel tile). int4 keeps
// the 1024 offsets (taken out through the weight sums at the merge); int2
// codes are small next to 1024, so they are made exact here.
// int4: word i covers tiles 2i, 2i+1; pair factors (t0,t1)=1, (t2,t3)=16.
// int2: word w covers tiles 4w..4w+3; even tiles factors (1,4), odd (16,64).
template <int BITS>
__device__ __forceinline__ void unpack_v(const uint32_t* vw, h4 A[8]) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = vw[i], w8 = w >> 8;
            A[2 * i] = make_h4(magic_pair(w, 0x000F000Fu), magic_pair(w, 0x00F000F0u));
            A[2 * i + 1] = make_h4(magic_pair(w8, 0x000F000Fu), magic_pair(w8, 0x00F000F0u));
        }
    } else {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t x = vw[w], x8 = x >> 8;
            A[4 * w + 0] = make_h4(exact_pair(x, 0x00030003u), exact_pair(x, 0x000C000Cu));
            A[4 * w + 1] = make_h4(exact_pair(x, 0x00300030u), exact_pair(x, 0x00C000C0u));
            A[4 * w + 2] = make_h4(exact_pair(x8, 0x00030003u), exact_pair(x8, 0x000C000Cu));
            A[4 * w + 3] = make_h4(exact_pair(x8, 0x00300030u), exact_pair(x8, 0x00C000C0u));
        }
    }
}

// Plain code of (tile t, token r) of a Value slot, and of (MFMA i, k e) of a
// Key slot (used on the tail path).
template <int BITS>
__device__ __forceinline__ uint32_t v_code_at(const uint32_t* vw, int t, int r) {
    if constexpr (BITS == 4) {
        const int e = (t & 1) * 2 + (r & 1) * 4 + (r >> 1);
        return (vw[t >> 1] >> (4 * e)) & 0xFu;
    } else {
        const int q = t & 3;
        const int f = 2 * q + (r >> 1) + 8 * (r & 1);
        return (vw[t >> 2] >> (2 * f)) & 0x3u;
    }
}

// 1 / (pair factor) of k-index e of score MFMA (Key side).
template <int BITS>
__device__ __forceinline__ float k_inv_factor(int e) {
    if constexpr (BITS == 4) return ((e >> 1) & 1) ? 0.0625f : 1.0f;
    else return 1.0f / (float)(1 << (2 * (e >> 1)));
}
// 1 / (pair factor) of token r of PV tile t (Value side).
template <int BITS>
__device__ __forceinline__ float v_inv_factor(int t, int r) {
    if constexpr (BITS == 4) return (r >> 1) ? 0.0625f : 1.0f;
    else return 1.0f / (float)(1 << (2 * (2 * (t & 1) + (r >> 1))));
}

// LDS layout of one work group (dynamic shared memory), in fp16 rows of
// kQRow elements (272 bytes: the 16-byte pad spreads rows over banks):
//   zero row | q[g] | per group: table[g][hi, lo] rows, Z[128], bias[16] f32
// The merge buffers of the epilogue reuse the same memory.
constexpr int kQRow = 136;
constexpr int kRowBytes = kQRow * 2;

__host__ __device__ constexpr int group_lds_bytes(int g) { return g * 2 * kRowBytes + 256 + 64; }
__host__ __device__ constexpr int head_lds_bytes(int g) { return kRowBytes * (g + 1); }
constexpr int kMergeBytes = kWaves * 16 * 4 * 2 + kWaves * 16 * kHeadDim * 4;

template <int BITS, int NG>
struct TileRegs {
    uint32_t k[BITS];
    uint32_t v[BITS];
    uint32_t vm[4 * NG];
};

template <int BITS, int NG>
__device__ __forceinline__ void load_tile(TileRegs<BITS, NG>& r, const uint8_t* kslot, const uint8_t* vslot,
                                          const uint32_t* vmeta) {
    if constexpr (BITS == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(kslot);
        const uint4 b = *reinterpret_cast<const uint4*>(vslot);
        r.k[0] = a.x; r.k[1] = a.y; r.k[2] = a.z; r.k[3] = a.w;
        r.v[0] = b.x; r.v[1] = b.y; r.v[2] = b.z; r.v[3] = b.w;
    } else {
        const uint2 a = *reinterpret_cast<const uint2*>(kslot);
        const uint2 b = *reinterpret_cast<const uint2*>(vslot);
        r.k[0] = a.x; r.k[1] = a.y;
        r.v[0] = b.x; r.v[1] = b.y;
    }
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        const uint4 m = reinterpret_cast<const uint4*>(vmeta)[q];
        r.vm[4 * q + 0] = m.x; r.vm[4 * q + 1] = m.y; r.vm[4 * q + 2] = m.z; r.vm[4 * q + 3] = m.w;
    }
}

// Shared state of one work group: the sequence, the KV head, its lengths.
struct WgCtx {
    int s, h, g, T, TK, TV, n_main, slot;
    const int32_t* bt;
    int bt_len;
};

__device__ __forceinline__ WgCtx make_ctx(const DecodeArgs& a, int s, int h) {
    const CacheView& V = a.v;
    WgCtx c;
    c.s = s;
    c.h = h;
    c.g = a.gqa;
    int T = a.seq_lens[s];
    c.slot = a.slot_ids[s];
    if (c.slot < 0 || c.slot >= V.max_seqs || T < 0) T = 0;
    c.T = T;
    c.TK = V.R * (T / V.R);
    c.TV = max(0, T - V.R);
    c.n_main = c.TV / kTile;
    c.bt = a.block_table + (size_t)s * a.bt_stride;
    c.bt_len = a.bt_stride;
    return c;
}

__device__ __forceinline__ int page_of_tile(const DecodeArgs& a, const WgCtx& c, int t) {
    const int bi = t / (a.v.Bk / kTile);
    if (bi >= c.bt_len) return -1;
    const int blk = c.bt[bi];
    return (blk >= 0 && blk < a.v.num_blocks) ? blk : -1;
}

// q of the g query heads as fp16 rows after a zero row (padding heads read the
// zero row); bf16 queries convert exactly within the fp16 range.
// q of the g query heads as fp16 rows after a zero row (bf16 queries convert
// exactly within the fp16 range). Loaded to registers first, stored later,
// so the load overlaps other round trips. Rows hold 16 chunks of 8 channels.
constexpr int kQueryRounds = 2;  // (16 + 1) rows x 16 chunks <= 2 x 256 threads
struct QueryLoads {
    uint4 v[kQueryRounds];
};

template <int DT>
__device__ __forceinline__ void query_load(const DecodeArgs& a, const WgCtx& c, QueryLoads& ql) {
#pragma unroll
    for (int r = 0; r < kQueryRounds; ++r) {
        const int idx = threadIdx.x + r * kThreads;
        const int hn = idx / 16 - 1, k = idx % 16;
        ql.v[r] = (uint4){0, 0, 0, 0};
        if (hn >= 0 && hn < c.g)
            ql.v[r] = *reinterpret_cast<const uint4*>(a.q + ((size_t)c.s * a.num_q_heads + c.h * c.g + hn) * kHeadDim +
                                                      8 * k);
    }
}

template <int DT>
__device__ __forceinline__ void query_store(const WgCtx& c, const QueryLoads& ql, uint16_t* lds_zero) {
#pragma unroll
    for (int r = 0; r < kQueryRounds; ++r) {
        const int idx = threadIdx.x + r * kThreads;
        if (idx >= (c.g + 1) * 16) continue;
        const int row = idx / 16, k = idx % 16;
        uint4 out = ql.v[r];
        if constexpr (DT == kBF16) {
            const uint32_t w[4] = {out.x, out.y, out.z, out.w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const _Float16 lo = (_Float16)bf16_bits_to_f32((uint16_t)(w[e] & 0xFFFFu));
                const _Float16 hi = (_Float16)bf16_bits_to_f32((uint16_t)(w[e] >> 16));
                o[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            out = {o[0], o[1], o[2], o[3]};
        }
        *reinterpret_cast<uint4*>(lds_zero + row * kQRow + 8 * k) = out;
    }
}

constexpr int kTableRounds = 4;  // 8-channel chunks per thread: up to 64 groups per table

// Key-group tables are built in three phases so that their two memory round
// trips (page ids, then the scale/zero runs) overlap with other loads:
//   table_pages -> (other loads) -> table_meta -> (other loads) -> table_fill.
struct TableLoads {
    int blk[kTableRounds];
    uint4 sv[kTableRounds], zv[kTableRounds];
};

template <class GroupOf>
__device__ __forceinline__ void table_pages(const DecodeArgs& a, const WgCtx& c, int n_groups, GroupOf group_of,
                                            TableLoads& tl) {
    const CacheView& V = a.v;
    const int tpg = V.G / kTile, tpp = V.Bk / kTile;
    const int nch = kHeadDim * V.Bk / V.G;
#pragma unroll
    for (int r = 0; r < kTableRounds; ++r) {
        const int q = threadIdx.x + r * kThreads;  // 8-channel chunk q % 16 of table slot q / 16
        const int ch = 8 * (q % 16);
        const int gi = q < n_groups * 16 ? group_of(q / 16) : -1;
        tl.blk[r] = gi >= 0 ? page_of_tile(a, c, gi * tpg + (ch / nch) * tpp) : -1;
    }
}

__device__ __forceinline__ void table_meta(const DecodeArgs& a, const WgCtx& c, TableLoads& tl) {
    const CacheView& V = a.v;
    const int nch = kHeadDim * V.Bk / V.G;
#pragma unroll
    for (int r = 0; r < kTableRounds; ++r) {
        const int ch = 8 * ((threadIdx.x + r * kThreads) % 16);
        const size_t base = (size_t)(tl.blk[r] >= 0 ? tl.blk[r] : 0) * V.H + c.h;
        const uint16_t* meta = reinterpret_cast<const uint16_t*>(V.k_meta + base * V.k_meta_bytes);
        tl.sv[r] = *reinterpret_cast<const uint4*>(meta + (ch % nch));
        tl.zv[r] = *reinterpret_cast<const uint4*>(meta + nch + (ch % nch));
    }
}

// Writes the tables of groups g_first .. g_first+n_groups-1 into slots
// 0 .. n_groups-1; lds_q must be visible to every thread (barrier before).
// Ends with a barrier; call it with every thread of the work group.
template <int BITS>
__device__ __forceinline__ void table_fill(const WgCtx& c, int n_groups, const TableLoads& tl, const uint16_t* lds_q,
                                           uint8_t* lds_groups) {
    const int g = c.g, tid = threadIdx.x;
    const int gbytes = group_lds_bytes(g);
#pragma unroll
    for (int r = 0; r < kTableRounds; ++r) {
        const int q = tid + r * kThreads;
        if (q >= n_groups * 16) continue;
        const int gl = q / 16, ch = 8 * (q % 16);
        const bool ok = tl.blk[r] >= 0;
        const uint4 sv = ok ? tl.sv[r] : (uint4){0, 0, 0, 0};
        const uint4 zv = ok ? tl.zv[r] : (uint4){0, 0, 0, 0};
        uint8_t* gb = lds_groups + gl * gbytes;
        *reinterpret_cast<uint4*>(gb + g * 2 * kRowBytes + 2 * ch) = zv;
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
        h2 sf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // pair factor of channel pair e of this 8-channel run
            const float f = (BITS == 4) ? ((e & 1) ? 0.0625f : 1.0f) : 1.0f / (float)(1 << (2 * e));
            sf[e] = __builtin_bit_cast(h2, sw[e]) * (h2){(_Float16)f, (_Float16)f};
        }
        for (int hn = 0; hn < g; ++hn) {
            const uint4 qu = *reinterpret_cast<const uint4*>(lds_q + hn * kQRow + ch);
            const uint32_t qw[4] = {qu.x, qu.y, qu.z, qu.w};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const h2 qv = __builtin_bit_cast(h2, qw[e]);
                // hi = fp16(q s f); lo = fp16(q s f - hi), the fused residual
                const h2 hi = qv * sf[e];
                const h2 lo = __builtin_elementwise_fma(qv, sf[e], -hi);
                hw[e] = __builtin_bit_cast(uint32_t, hi);
                lw[e] = __builtin_bit_cast(uint32_t, lo);
            }
            *reinterpret_cast<uint4*>(gb + (hn * 2 + 0) * kRowBytes + 2 * ch) = (uint4){hw[0], hw[1], hw[2], hw[3]};
            *reinterpret_cast<uint4*>(gb + (hn * 2 + 1) * kRowBytes + 2 * ch) = (uint4){lw[0], lw[1], lw[2], lw[3]};
        }
    }
    __syncthreads();
    for (int idx = tid; idx < n_groups * g; idx += kThreads) {
        const int gl = idx / g, hn = idx % g;
        const uint8_t* gb = lds_groups + gl * gbytes;
        float zq = 0.0f;  // sum_c q_c zero_c (exact products, fp32 sum)
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const uint4 zu = *reinterpret_cast<const uint4*>(gb + g * 2 * kRowBytes + 16 * k);
            const uint4 qu = *reinterpret_cast<const uint4*>(lds_q + hn * kQRow + 8 * k);
            zq = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, qu.x), __builtin_bit_cast(h2, zu.x), zq, false);
            zq = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, qu.y), __builtin_bit_cast(h2, zu.y), zq, false);
            zq = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, qu.z), __builtin_bit_cast(h2, zu.z), zq, false);
            zq = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, qu.w), __builtin_bit_cast(h2, zu.w), zq, false);
        }
        *reinterpret_cast<float*>(lds_groups + gl * gbytes + g * 2 * kRowBytes + 256 + 4 * hn) = zq;
    }
    __syncthreads();
}

// Per-lane online-softmax state of query head (lane & 15) and its output
// accumulators O^T[16 t + 4 (lane >> 4) + r][head] held in O[t][r].
// wsum[gg][vb] sums the value-side weights (hi + lo) of channel group gg and
// pair-factor variant vb: the codes carry a 1024 offset, so every output
// channel holds 1024 * wsum too much until the merge takes it out.
template <int NG, int NB>
struct Acc {
    float m_run, l_acc, zacc[NG], wsum[NG][NB];
    f4 O[8];
    __device__ __forceinline__ void init() {
        m_run = -INFINITY;
        l_acc = 0.0f;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            zacc[gg] = 0.0f;
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) wsum[gg][vb] = 0.0f;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) O[t] = (f4){0.f, 0.f, 0.f, 0.f};
    }
    // Scores of tokens 4j..4j+3 of one tile (exp2 domain) -> weights p.
    __device__ __forceinline__ void update(const float sc[4], float p[4]) {
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = xor_max(mx);
        if (mx > m_run) {
            const float f = __builtin_amdgcn_exp2f(m_run - mx);
            l_acc *= f;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                zacc[gg] *= f;
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) wsum[gg][vb] *= f;
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) O[t] *= f;
            m_run = mx;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m_run);
        l_acc += (p[0] + p[1]) + (p[2] + p[3]);
    }
};

// Scale-folded query B-operands of one Key group for this lane (head n,
// k-slice j), read from the LDS table.
struct GroupOps {
    h8 Bh[4], Bl[4];
    float biasl2;
    int cur;
    __device__ __forceinline__ void load(const uint8_t* lds_groups, const uint16_t* lds_zero, int gbytes, int g,
                                         int gl, int gi, int n, int j, float sl2) {
        const uint8_t* gb = lds_groups + gl * gbytes;
        const bool ok = n < g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = 2 * (32 * i + 8 * j);
            const uint8_t* rh = ok ? gb + (n * 2 + 0) * kRowBytes + off : reinterpret_cast<const uint8_t*>(lds_zero);
            const uint8_t* rl = ok ? gb + (n * 2 + 1) * kRowBytes + off : reinterpret_cast<const uint8_t*>(lds_zero);
            Bh[i] = *reinterpret_cast<const h8*>(rh);
            Bl[i] = *reinterpret_cast<const h8*>(rl);
        }
        biasl2 = ok ? reinterpret_cast<const float*>(gb + g * 2 * kRowBytes + 256)[n] * sl2 : 0.0f;
        cur = gi;
    }
};

// Scores (exp2 domain) of a 16-token tile whose Keys are quantised.
template <int BITS>
__device__ __forceinline__ void code_scores(const uint32_t* kw, const GroupOps& go, float sl2, float sc[4]) {
    h8 A[4];
    unpack_k<BITS>(kw, A);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], go.Bh[i], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], go.Bl[i], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = acc[r] * sl2 + go.biasl2;
}

// Same, reading the group's B-operands straight from the LDS table (no
// register copy of the table); two accumulation chains (hi, lo). `row` is
// the lane's byte offset into a group table: head row of (n, or n mod g for
// padding lanes, whose results are never used) plus the k-slice 16 j.
template <int BITS>
__device__ __forceinline__ void code_scores_lds(const uint32_t* kw, const uint8_t* gb, int row, int bias_off,
                                                float sl2, float sc[4]) {
    h8 A[4];
    unpack_k<BITS>(kw, A);
    f4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h8 bh = *reinterpret_cast<const h8*>(gb + row + 64 * i);
        const h8 bl = *reinterpret_cast<const h8*>(gb + row + kRowBytes + 64 * i);
        ah = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], bh, ah, 0, 0, 0);
        al = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], bl, al, 0, 0, 0);
    }
    const float biasl2 = *reinterpret_cast<const float*>(gb + bias_off) * sl2;
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (ah[r] + al[r]) * sl2 + biasl2;
}

// Write the 4 waves' states to LDS: m, l per (wave, head) and
// o = O + sum_t p_t zero_t per (wave, head, channel). Every thread calls it.
template <int NG, int NB, bool kValueOffset>
__device__ __forceinline__ void stash_waves(Acc<NG, NB>& st, uint8_t* smem) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, j = lane >> 4;
    const float l_tot = xor_sum(st.l_acc);
    float zt[NG][NB];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
        const float z = xor_sum(st.zacc[gg]);
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) zt[gg][vb] = z - (kValueOffset ? 1024.0f * xor_sum(st.wsum[gg][vb]) : 0.0f);
    }
    __syncthreads();  // LDS tables no longer read
    float* sm_m = reinterpret_cast<float*>(smem);  // [kWaves][16]
    float* sm_l = sm_m + kWaves * 16;              // [kWaves][16]
    float* sm_o = sm_l + kWaves * 16;              // [kWaves][16][128]
    if (j == 0) {
        sm_m[wave * 16 + n] = st.m_run;
        sm_l[wave * 16 + n] = l_tot;
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int chn = 16 * tt + 4 * j + r;
            sm_o[(wave * 16 + n) * kHeadDim + chn] = st.O[tt][r] + zt[chn / (kHeadDim / NG)][tt % NB];
        }
    __syncthreads();
}

// One work group per (sequence, KV head, split). Splits cover the "main"
// 16-token tiles, whose Keys and Values are both quantised; the last split
// of a sequence also covers the tail tiles that touch the residual. Each
// wave takes a contiguous tile range with one buffer of tiles in flight
// while it computes the other. Every split writes a partial (m, l, o); the
// last work group of a (sequence, KV head) to finish merges them:
// m = max m_i, l = sum l_i 2^(m_i - m), o = sum o_i 2^(m_i - m) / l.
template <int BITS, int DT, int NG>
__global__ __launch_bounds__(kThreads, (NG == 1 ? 3 : 2)) void decode_kernel(DecodeArgs a) {
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;
    constexpr int SLOT_BYTES = 4 * BITS;
    constexpr int NB = (BITS == 2) ? 2 : 1;  // Value pair-factor variants
    extern __shared__ __align__(16) uint8_t smem[];
    const CacheView& V = a.v;
    const int H = V.H;
    const int split = blockIdx.x % a.n_splits;
    const int sh = blockIdx.x / a.n_splits;
    const WgCtx c = make_ctx(a, sh / H, sh % H);
    const int tps = a.tiles_per_split;
    const int nvalid = c.n_main > 0 ? min(a.n_splits, (c.n_main + tps - 1) / tps) : 1;
    if (split >= nvalid) return;
    const bool last = split == nvalid - 1;
    const int t_begin = split * tps;
    const int t_end = last ? c.n_main : t_begin + tps;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int n = lane & 15, j = lane >> 4;
    const int g = c.g;
    const int R = V.R;
    const int T = c.T, TV = c.TV;
    const int tk_tiles = c.TK / kTile;
    const float sl2 = a.scale_log2;
    const int HQ = a.num_q_heads;

    uint16_t* lds_zero = reinterpret_cast<uint16_t*>(smem);
    uint16_t* lds_q = lds_zero + kQRow;
    uint8_t* lds_groups = smem + head_lds_bytes(g);
    const int gbytes = group_lds_bytes(g);
    {
        QueryLoads ql;
        query_load<DT>(a, c, ql);
        query_store<DT>(c, ql, lds_zero);
    }
    const int nr = n < g ? n : n % g;
    const int lane_row = nr * 2 * kRowBytes + 16 * j;
    const int lane_bias = g * 2 * kRowBytes + 256 + 4 * nr;
    const uint32_t lane_code_off = SLOT_BYTES * lane;
    const uint32_t lane_meta_off = 16 * NG * j;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(V.k_codes, a.code_array_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V.v_codes, a.code_array_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(V.v_meta, a.vmeta_array_bytes);
    const uint16_t* ringK = V.k_ring + ((size_t)max(c.slot, 0) * H + c.h) * V.ring_elems;
    const uint16_t* ringV = V.v_ring + ((size_t)max(c.slot, 0) * H + c.h) * V.ring_elems;

    Acc<NG, NB> st;
    st.init();
    const int chunk_tiles = max(1, (a.lds_groups - 1) << a.tpg_shift);

    // ---------------- main tiles ----------------
    for (int c0 = t_begin; c0 < t_end; c0 += chunk_tiles) {
        const int c1 = min(t_end, c0 + chunk_tiles);
        const int g_first = c0 >> a.tpg_shift;
        const int n_groups = ((c1 - 1) >> a.tpg_shift) - g_first + 1;
        const int nt = c1 - c0;
        const int per_wave = (nt + kWaves - 1) / kWaves;
        const int w_begin = c0 + wave * per_wave;
        const int w_end = min(c1, w_begin + per_wave);
        int my_page = (w_begin + lane < w_end) ? page_of_tile(a, c, w_begin + lane) : -1;
        // Loads of a tile are unconditional (a missing page or a tile past
        // the range reads page 0 and is not computed), so a buffer of tiles
        // is one straight run of loads that the wait counts can follow.
        // Offsets: scalar per tile, per lane fixed.
        auto issue = [&](int t, TileRegs<BITS, NG>& r) -> bool {
            const int blk = __builtin_amdgcn_readlane(my_page, (t - w_begin) & 63);
            const bool valid = blk >= 0 && t < w_end;
            const uint32_t chk = (uint32_t)(valid ? blk : 0) * (uint32_t)H + (uint32_t)c.h;
            const uint32_t sub = (uint32_t)t & ((1u << a.tpp_shift) - 1u);
            const uint32_t coff = chk * (uint32_t)V.code_bytes + sub * TILE_BYTES;
            const uint32_t moff = chk * (uint32_t)V.v_meta_bytes + sub * (kTile * NG * 4);
            if constexpr (BITS == 4) {
                const uint4 k4 = buf_b128(rk, lane_code_off, coff);
                const uint4 v4 = buf_b128(rv, lane_code_off, coff);
                r.k[0] = k4.x; r.k[1] = k4.y; r.k[2] = k4.z; r.k[3] = k4.w;
                r.v[0] = v4.x; r.v[1] = v4.y; r.v[2] = v4.z; r.v[3] = v4.w;
            } else {
                const uint2 k2 = buf_b64(rk, lane_code_off, coff);
                const uint2 v2 = buf_b64(rv, lane_code_off, coff);
                r.k[0] = k2.x; r.k[1] = k2.y;
                r.v[0] = v2.x; r.v[1] = v2.y;
            }
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const uint4 m = buf_b128(rm, lane_meta_off + 16 * q, moff);
                r.vm[4 * q + 0] = m.x; r.vm[4 * q + 1] = m.y; r.vm[4 * q + 2] = m.z; r.vm[4 * q + 3] = m.w;
            }
            return valid;
        };
        auto compute = [&](const TileRegs<BITS, NG>& cur, int t) {
            const uint8_t* gb = lds_groups + ((t >> a.tpg_shift) - g_first) * gbytes;
            float sc[4], p[4];
            code_scores_lds<BITS>(cur.k, gb, lane_row, lane_bias, sl2, sc);
            st.update(sc, p);
            // Value side: W = p * scale (hi, lo) per channel group and pair-factor variant
            h8 Bv[NG][NB];
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                float Sv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t mw = cur.vm[r * NG + gg];
                    Sv[r] = f16_bits_to_f32((uint16_t)(mw & 0xFFFFu));
                    st.zacc[gg] += p[r] * f16_bits_to_f32((uint16_t)(mw >> 16));
                }
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    float ws = 0.0f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float wv = p[r] * Sv[r] * v_inv_factor<BITS>(vb, r);
                        _Float16 hi, lo;
                        split_f16(wv, hi, lo);
                        Bv[gg][vb][r] = hi;
                        Bv[gg][vb][4 + r] = lo;
                        ws += wv;
                    }
                    st.wsum[gg][vb] += ws;
                }
            }
            h4 Av[8];
            unpack_v<BITS>(cur.v, Av);
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const int gg = (16 * tt) / (kHeadDim / NG);
                st.O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dup_h8(Av[tt]), Bv[gg][tt % NB], st.O[tt], 0, 0, 0);
            }
        };
        TableLoads tl;
        table_pages(a, c, n_groups, [&](int k) { return g_first + k; }, tl);
        table_meta(a, c, tl);
        __syncthreads();  // query rows stored; previous chunk's tables no longer read
        table_fill<BITS>(c, n_groups, tl, lds_q, lds_groups);
        // two buffers of kHalf tiles: one buffer's loads are in flight while
        // the other's tiles are computed
        TileRegs<BITS, NG> ra[kHalf], rb[kHalf];
        bool oka[kHalf], okb[kHalf];
        auto issue_half = [&](int t, TileRegs<BITS, NG>* r, bool* ok) {
            if (((t - w_begin) & 63) == 0 && t != w_begin)
                my_page = (t + lane < w_end) ? page_of_tile(a, c, t + lane) : -1;
#pragma unroll
            for (int b = 0; b < kHalf; ++b) ok[b] = issue(t + b, r[b]);
        };
        auto compute_half = [&](int t, const TileRegs<BITS, NG>* r, const bool* ok) {
#pragma unroll
            for (int b = 0; b < kHalf; ++b)
                if (ok[b]) compute(r[b], t + b);
        };
        issue_half(w_begin, ra, oka);
        for (int t0 = w_begin; t0 < w_end; t0 += 2 * kHalf) {
            issue_half(t0 + kHalf, rb, okb);
            compute_half(t0, ra, oka);
            if (t0 + kHalf >= w_end) break;
            issue_half(t0 + 2 * kHalf, ra, oka);
            compute_half(t0 + kHalf, rb, okb);
        }
    }

    // ---------------- tail tiles ----------------
    // Tiles that touch the residual (Keys from codes or the residual; each
    // Value token from codes (< TV), the residual (< T) or masked) are dealt
    // out over the valid splits: split i takes tail tiles i, i + nvalid, ...,
    // one per wave per round.
    const int n_tail = (T + kTile - 1) / kTile - c.n_main;
    const int my_tail = n_tail > split ? (n_tail - split + nvalid - 1) / nvalid : 0;
    for (int r0 = 0; r0 < my_tail; r0 += kWaves) {
        // this round's tiles: k = r0 .. r0+3 of this split's list; the Key groups
        // of code tiles get one table slot per wave
        __syncthreads();
        int gsel[kWaves];  // table slot w: Key group of wave w's tile, or none
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int kq = r0 + w;
            const int tw = c.n_main + split + kq * nvalid;
            gsel[w] = (kq < my_tail && tw < tk_tiles) ? (tw >> a.tpg_shift) : -1;
        }
        TableLoads tl;
        table_pages(a, c, kWaves, [&](int k) { return gsel[k]; }, tl);
        table_meta(a, c, tl);
        table_fill<BITS>(c, kWaves, tl, lds_q, lds_groups);
        const int kq = r0 + wave;
        const int w_begin = c.n_main + split + kq * nvalid;
        const int w_end = kq < my_tail ? w_begin + 1 : w_begin;
        for (int t = w_begin; t < w_end; ++t) {
            const int p0 = t * kTile;
            const int blk = page_of_tile(a, c, t);
            if (blk < 0) continue;
            const uint32_t chk = (uint32_t)blk * (uint32_t)H + (uint32_t)c.h;
            const uint32_t sub = (uint32_t)t & ((1u << a.tpp_shift) - 1u);
            const uint32_t coff = chk * (uint32_t)V.code_bytes + sub * TILE_BYTES;
            const uint32_t moff = chk * (uint32_t)V.v_meta_bytes + sub * (kTile * NG * 4);
            const bool kcode = t < tk_tiles;
            const bool vcode = p0 < TV;
            // ---- every load of the tile first ----
            uint32_t kw[BITS], vw[BITS], vm[4 * NG];
            uint4 kr[4];
            uint2 vr[8];
#pragma unroll
            for (int k = 0; k < BITS; ++k) kw[k] = vw[k] = 0;
#pragma unroll
            for (int k = 0; k < 4 * NG; ++k) vm[k] = 0;
            if (kcode) {
                if constexpr (BITS == 4) {
                    const uint4 u = buf_b128(rk, lane_code_off, coff);
                    kw[0] = u.x; kw[1] = u.y; kw[2] = u.z; kw[3] = u.w;
                } else {
                    const uint2 u = buf_b64(rk, lane_code_off, coff);
                    kw[0] = u.x; kw[1] = u.y;
                }
            } else {
                const int pk = min(p0 + n, T - 1);  // A row: token n of the tile
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    kr[i] = *reinterpret_cast<const uint4*>(ringK + (size_t)(pk % R) * kHeadDim + 32 * i + 8 * j);
            }
            if (vcode) {
                if constexpr (BITS == 4) {
                    const uint4 u = buf_b128(rv, lane_code_off, coff);
                    vw[0] = u.x; vw[1] = u.y; vw[2] = u.z; vw[3] = u.w;
                } else {
                    const uint2 u = buf_b64(rv, lane_code_off, coff);
                    vw[0] = u.x; vw[1] = u.y;
                }
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const uint4 m = buf_b128(rm, lane_meta_off + 16 * q, moff);
                    vm[4 * q + 0] = m.x; vm[4 * q + 1] = m.y; vm[4 * q + 2] = m.z; vm[4 * q + 3] = m.w;
                }
            }
            // residual Values: positions 4j..4j+3 of a channel are adjacent in the
            // channel-major ring (R is a multiple of 16, so they never wrap)
            const int pq = p0 + 4 * j;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
                vr[tt] = *reinterpret_cast<const uint2*>(ringV + (size_t)(16 * tt + n) * R + (pq % R));

            // ---- scores ----
            float sc[4];
            if (kcode) {
                const uint8_t* gb = lds_groups + wave * gbytes;
                code_scores_lds<BITS>(kw, gb, lane_row, lane_bias, sl2, sc);
            } else {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                const uint8_t* qrow = reinterpret_cast<const uint8_t*>(lds_q + nr * kQRow);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h8 A;
                    const uint32_t ws[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) A[e] = (_Float16)to_f32<DT>((uint16_t)(ws[e >> 1] >> (16 * (e & 1))));
                    const h8 B = *reinterpret_cast<const h8*>(qrow + 2 * (32 * i + 8 * j));
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[r] = (p0 + 4 * j + r < T) ? acc[r] * sl2 : -INFINITY;
            }
            float p[4];
            st.update(sc, p);
            // ---- values ----
            float Sv[4][NG];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool code_tok = pq + r < TV;
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) {
                    const uint32_t mw = code_tok ? vm[r * NG + gg] : 0u;
                    Sv[r][gg] = f16_bits_to_f32((uint16_t)(mw & 0xFFFFu));
                    st.zacc[gg] += p[r] * f16_bits_to_f32((uint16_t)(mw >> 16));
                }
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const int gg = (16 * tt) / (kHeadDim / NG);
                const uint32_t rw[2] = {vr[tt].x, vr[tt].y};
                h4 A;
                h8 B;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int pr = pq + r;
                    float av = 0.0f, wv = 0.0f;
                    if (pr < TV) {
                        av = (float)v_code_at<BITS>(vw, tt, r);
                        wv = p[r] * Sv[r][gg];
                    } else if (pr < T) {
                        av = to_f32<DT>((uint16_t)(rw[r >> 1] >> (16 * (r & 1))));
                        wv = p[r];
                    }
                    A[r] = (_Float16)av;
                    _Float16 hi, lo;
                    split_f16(wv, hi, lo);
                    B[r] = hi;
                    B[4 + r] = lo;
                }
                st.O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dup_h8(A), B, st.O[tt], 0, 0, 0);
            }
        }
    }

    // ---------------- this split's partial ----------------
    stash_waves<NG, NB, BITS == 4>(st, smem);
    const float* sm_m = reinterpret_cast<const float*>(smem);
    const float* sm_l = sm_m + kWaves * 16;
    const float* sm_o = sm_l + kWaves * 16;
    for (int idx = tid; idx < g * kHeadDim; idx += kThreads) {
        const int hn = idx / kHeadDim, chn = idx % kHeadDim;
        float mstar = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm_m[w * 16 + hn]);
        float lsum = 0.0f, osum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm_m[w * 16 + hn];
            const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - mstar);
            lsum += f * sm_l[w * 16 + hn];
            osum += f * sm_o[(w * 16 + hn) * kHeadDim + chn];
        }
        float* part = a.partials + (((size_t)c.s * HQ + c.h * g + hn) * a.n_splits + split) * kPartialStride;
        if (chn == 0) {
            part[0] = mstar;
            part[1] = lsum;
        }
        part[4 + chn] = osum;
    }

    // ---------------- the last work group of this (sequence, KV head) merges ----------------
    __shared__ int sm_last;
    __syncthreads();  // every partial store of this work group precedes the release below
    if (tid == 0) {
        int* ctr = a.counters + (size_t)c.s * H + c.h;
        const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = (prev == nvalid - 1);
        if (sm_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!sm_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every thread sees the other partials
    for (int idx = tid; idx < g * kHeadDim; idx += kThreads) {
        const int hn = idx / kHeadDim, chn = idx % kHeadDim;
        const int hq = c.h * g + hn;
        const float* base = a.partials + ((size_t)c.s * HQ + hq) * a.n_splits * kPartialStride;
        float mstar = -INFINITY;
        for (int i = 0; i < nvalid; ++i) mstar = fmaxf(mstar, base[(size_t)i * kPartialStride]);
        float lsum = 0.0f, osum = 0.0f;
        if (mstar != -INFINITY) {
            for (int i = 0; i < nvalid; ++i) {
                const float* pp = base + (size_t)i * kPartialStride;
                const float mi = pp[0];
                if (mi == -INFINITY) continue;
                const float f = __builtin_amdgcn_exp2f(mi - mstar);
                lsum += f * pp[1];
                osum += f * pp[4 + chn];
            }
        }
        const float o = lsum > 0.0f ? osum / lsum : 0.0f;
        a.out[((size_t)c.s * HQ + hq) * kHeadDim + chn] = from_f32<DT>(o);
    }
}

template <int BITS, int DT>
void launch_bits_dt(const DecodeArgs& a, int ng, dim3 grid, size_t lds, hipStream_t st) {
    dim3 block(kThreads);
    switch (ng) {
        case 1: hipLaunchKernelGGL((decode_kernel<BITS, DT, 1>), grid, block, lds, st, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<BITS, DT, 2>), grid, block, lds, st, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<BITS, DT, 4>), grid, block, lds, st, a); break;
        default: hipLaunchKernelGGL((decode_kernel<BITS, DT, 8>), grid, block, lds, st, a); break;
    }
}

}  // namespace

int launch_decode(const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                  const int32_t* slot_ids, const int32_t* seq_lens, const int32_t* block_table,
                  int bt_stride, float softmax_scale, void* out, float* partials,
                  const DecodePlan& plan, void* stream) {
    DecodeArgs a;
    a.v = v;
    a.q = static_cast<const uint16_t*>(q);
    a.slot_ids = slot_ids;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.num_q_heads = num_q_heads;
    a.gqa = num_q_heads / v.H;
    a.scale_log2 = softmax_scale * kLog2e;
    a.counters = reinterpret_cast<int*>(partials);
    a.partials = partials + plan.counter_floats;
    a.n_splits = plan.n_splits;
    a.tiles_per_split = plan.tiles_per_split;
    a.lds_groups = plan.lds_groups;
    a.tpg_shift = __builtin_ctz((unsigned)(v.G / kTile));
    a.tpp_shift = __builtin_ctz((unsigned)(v.Bk / kTile));
    a.code_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.code_bytes);
    a.vmeta_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.v_meta_bytes);
    a.out = static_cast<uint16_t*>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int ng = kHeadDim / v.Gv;
    dim3 grid((unsigned)(num_seqs * v.H * plan.n_splits));
    const size_t lds = plan.lds_bytes;
    if (v.bits == 4) {
        if (v.dtype == kF16) launch_bits_dt<4, kF16>(a, ng, grid, lds, st);
        else launch_bits_dt<4, kBF16>(a, ng, grid, lds, st);
    } else {
        if (v.dtype == kF16) launch_bits_dt<2, kF16>(a, ng, grid, lds, st);
        else launch_bits_dt<2, kBF16>(a, ng, grid, lds, st);
    }
    return (int)hipGetLastError();
}

// LDS budget of one decode work group (three work groups per compute unit).
int decode_lds_groups(int g) {
    const int budget = 52 * 1024;
    return std::min(kTableRounds * kThreads / 16, std::max(kWaves, (budget - head_lds_bytes(g)) / group_lds_bytes(g)));
}
size_t decode_lds_bytes(int g, int groups) {
    return std::max((size_t)kMergeBytes, (size_t)head_lds_bytes(g) + (size_t)groups * group_lds_bytes(g));
}

}  // namespace kivi
