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
    int n_splits;
    int tiles_per_split;
    uint16_t* out;
};

// fp16 pair from two code fields already placed in the low bits of each
// half: (1024 + x) - 1024, exact.
__device__ __forceinline__ uint32_t code_pair(uint32_t fields) {
    h2 v = __builtin_bit_cast(h2, fields | 0x64006400u);
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

__device__ __forceinline__ float xor_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}
__device__ __forceinline__ float xor_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}

// Key A-operands of the 4 score MFMAs from this lane's code slot.
// int4: word i covers channels 32i+8j..+7 (even in the low half, odd in the
// high half), pair factors 1,16,1,16. int2: word w covers MFMAs 2w (fields
// 0..3) and 2w+1 (fields 4..7), pair factors 1,4,16,64.
template <int BITS>
__device__ __forceinline__ void unpack_k(const uint32_t* kw, h8 A[4]) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = kw[i], w8 = w >> 8;
            A[i] = make_h8(code_pair(w & 0x000F000Fu), code_pair(w & 0x00F000F0u),
                           code_pair(w8 & 0x000F000Fu), code_pair(w8 & 0x00F000F0u));
        }
    } else {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t x = kw[w], x8 = x >> 8;
            A[2 * w] = make_h8(code_pair(x & 0x00030003u), code_pair(x & 0x000C000Cu),
                               code_pair(x & 0x00300030u), code_pair(x & 0x00C000C0u));
            A[2 * w + 1] = make_h8(code_pair(x8 & 0x00030003u), code_pair(x8 & 0x000C000Cu),
                                   code_pair(x8 & 0x00300030u), code_pair(x8 & 0x00C000C0u));
        }
    }
}

// Value A-operands of the 8 PV MFMAs (one per 16-channel tile).
// int4: word i covers tiles 2i, 2i+1; pair factors (t0,t1)=1, (t2,t3)=16.
// int2: word w covers tiles 4w..4w+3; even tiles factors (1,4), odd (16,64).
template <int BITS>
__device__ __forceinline__ void unpack_v(const uint32_t* vw, h4 A[8]) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = vw[i], w8 = w >> 8;
            A[2 * i] = make_h4(code_pair(w & 0x000F000Fu), code_pair(w & 0x00F000F0u));
            A[2 * i + 1] = make_h4(code_pair(w8 & 0x000F000Fu), code_pair(w8 & 0x00F000F0u));
        }
    } else {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t x = vw[w], x8 = x >> 8;
            A[4 * w + 0] = make_h4(code_pair(x & 0x00030003u), code_pair(x & 0x000C000Cu));
            A[4 * w + 1] = make_h4(code_pair(x & 0x00300030u), code_pair(x & 0x00C000C0u));
            A[4 * w + 2] = make_h4(code_pair(x8 & 0x00030003u), code_pair(x8 & 0x000C000Cu));
            A[4 * w + 3] = make_h4(code_pair(x8 & 0x00300030u), code_pair(x8 & 0x00C000C0u));
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

template <int BITS, int DT, int NG>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;
    constexpr int SLOT_BYTES = 4 * BITS;
    constexpr int SLOT_WORDS = BITS;  // 32-bit words per lane slot
    const CacheView& V = a.v;
    const int H = V.H;
    const int nsp = a.n_splits + 1;
    const int split = blockIdx.x % nsp;
    const int sh = blockIdx.x / nsp;
    const int h = sh % H;
    const int s = sh / H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, j = lane >> 4;
    const int g = a.gqa;
    const int HQ = a.num_q_heads;
    const int R = V.R, G = V.G, Bk = V.Bk, Gv = V.Gv;

    int T = a.seq_lens[s];
    const int slot = a.slot_ids[s];
    if (slot < 0 || slot >= V.max_seqs || T < 0) T = 0;
    const int TK = R * (T / R);
    const int TV = max(0, T - R);
    const int n_main = TV / kTile;
    const bool tail = split == a.n_splits;
    int t_begin, t_end;
    if (!tail) {
        t_begin = split * a.tiles_per_split;
        t_end = (split == a.n_splits - 1) ? n_main : min(n_main, t_begin + a.tiles_per_split);
        if (t_begin >= t_end) return;
    } else {
        t_begin = n_main;
        t_end = (T + kTile - 1) / kTile;
    }
    const int nt = t_end - t_begin;
    const int per_wave = (nt + kWaves - 1) / kWaves;
    const int w_begin = t_begin + wave * per_wave;
    const int w_end = min(t_end, w_begin + per_wave);

    const int32_t* bt = a.block_table + (size_t)s * a.bt_stride;
    auto page_of = [&](int p) -> int {
        const int bi = p / Bk;
        if (bi >= a.bt_stride) return -1;
        const int blk = bt[bi];
        return (blk >= 0 && blk < V.num_blocks) ? blk : -1;
    };

    // query of head n (zero for padding heads): channels 32i + 8j + e
    const bool head_ok = n < g;
    const int hq = h * g + (head_ok ? n : 0);
    float qf[32];
    {
        const uint16_t* qrow = a.q + ((size_t)s * HQ + hq) * kHeadDim;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * i + 8 * j);
            const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = to_f32<DT>((uint16_t)(ws[e >> 1] >> (16 * (e & 1))));
                qf[8 * i + e] = head_ok ? x : 0.0f;
            }
        }
    }

    // running state of this lane's query head over this wave's tiles
    float m_run = -INFINITY, l_acc = 0.0f;
    float zacc[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zacc[gg] = 0.0f;
    f4 O[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] = (f4){0.f, 0.f, 0.f, 0.f};

    int cur_group = -1;
    h8 Bhi[4], Blo[4];
    float bias = 0.0f;
    const int nch = kHeadDim * Bk / G;

    auto load_group = [&](int gi) {
        float bpart = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 32 * i + 8 * j;
            const int blk = page_of(gi * G + (c / nch) * Bk);
            uint4 su = {0, 0, 0, 0}, zu = {0, 0, 0, 0};
            if (blk >= 0) {
                const uint16_t* meta = reinterpret_cast<const uint16_t*>(
                    V.k_meta + ((size_t)blk * H + h) * V.k_meta_bytes);
                su = *reinterpret_cast<const uint4*>(meta + (c % nch));
                zu = *reinterpret_cast<const uint4*>(meta + nch + (c % nch));
            }
            const uint32_t sw[4] = {su.x, su.y, su.z, su.w};
            const uint32_t zw[4] = {zu.x, zu.y, zu.z, zu.w};
            h8 bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float S = f16_bits_to_f32((uint16_t)(sw[e >> 1] >> (16 * (e & 1))));
                const float Z = f16_bits_to_f32((uint16_t)(zw[e >> 1] >> (16 * (e & 1))));
                _Float16 hi, lo;
                split_f16(qf[8 * i + e] * S * k_inv_factor<BITS>(e), hi, lo);
                bh[e] = hi;
                bl[e] = lo;
                bpart += qf[8 * i + e] * Z;
            }
            Bhi[i] = bh;
            Blo[i] = bl;
        }
        bias = xor_sum(bpart);
        cur_group = gi;
    };

    // online softmax update with this tile's 4 scores (tokens 4j..4j+3)
    auto softmax_update = [&](const float sc[4], float p[4]) {
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = xor_max(mx);
        if (mx > m_run) {
            const float f = __builtin_amdgcn_exp2f(m_run - mx);
            l_acc *= f;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) zacc[gg] *= f;
#pragma unroll
            for (int t = 0; t < 8; ++t) O[t] *= f;
            m_run = mx;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m_run);
        l_acc += (p[0] + p[1]) + (p[2] + p[3]);
    };

    const float sl2 = a.scale_log2;

    for (int t = w_begin; t < w_end; ++t) {
        const int p0 = t * kTile;
        const int blk = page_of(p0);
        if (blk < 0) continue;
        const int sub = (p0 % Bk) / kTile;
        const int row0 = p0 % Bk;
        const size_t chunk = ((size_t)blk * H + h);
        const uint8_t* kslot = V.k_codes + chunk * V.code_bytes + sub * TILE_BYTES + SLOT_BYTES * lane;
        const uint8_t* vslot = V.v_codes + chunk * V.code_bytes + sub * TILE_BYTES + SLOT_BYTES * lane;
        const uint32_t* vmeta = reinterpret_cast<const uint32_t*>(
            V.v_meta + chunk * V.v_meta_bytes + (size_t)(row0 + 4 * j) * NG * 4);

        // ---- scores ----
        float sc[4];
        if (p0 < TK) {
            const int gi = p0 / G;
            if (gi != cur_group) load_group(gi);
            uint32_t kw[SLOT_WORDS];
            if constexpr (BITS == 4) {
                const uint4 u = *reinterpret_cast<const uint4*>(kslot);
                kw[0] = u.x; kw[1] = u.y; kw[2] = u.z; kw[3] = u.w;
            } else {
                const uint2 u = *reinterpret_cast<const uint2*>(kslot);
                kw[0] = u.x; kw[1] = u.y;
            }
            h8 A[4];
            unpack_k<BITS>(kw, A);
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], Bhi[i], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], Blo[i], acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = (acc[r] + bias) * sl2;
        } else {
            // Key residual rows (full precision) against the plain query
            const uint16_t* ringK = V.k_ring + ((size_t)slot * H + h) * V.ring_elems;
            const int p = p0 + n;  // A row = token n of the tile
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h8 A, B;
                uint4 u = {0, 0, 0, 0};
                if (p < T) u = *reinterpret_cast<const uint4*>(ringK + (size_t)(p % R) * kHeadDim + 32 * i + 8 * j);
                const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    A[e] = (_Float16)to_f32<DT>((uint16_t)(ws[e >> 1] >> (16 * (e & 1))));
                    B[e] = (_Float16)qf[8 * i + e];
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = (p0 + 4 * j + r < T) ? acc[r] * sl2 : -INFINITY;
        }

        float p[4];
        softmax_update(sc, p);

        // ---- values ----
        if (!tail || p0 + kTile <= TV) {
            // all 16 tokens quantised
            uint32_t vw[SLOT_WORDS];
            if constexpr (BITS == 4) {
                const uint4 u = *reinterpret_cast<const uint4*>(vslot);
                vw[0] = u.x; vw[1] = u.y; vw[2] = u.z; vw[3] = u.w;
            } else {
                const uint2 u = *reinterpret_cast<const uint2*>(vslot);
                vw[0] = u.x; vw[1] = u.y;
            }
            h4 A[8];
            unpack_v<BITS>(vw, A);
            float Sv[4][NG], Zv[4][NG];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) {
                    const uint32_t mw = vmeta[r * NG + gg];
                    Sv[r][gg] = f16_bits_to_f32((uint16_t)(mw & 0xFFFFu));
                    Zv[r][gg] = f16_bits_to_f32((uint16_t)(mw >> 16));
                }
#pragma unroll
            for (int gg = 0; gg < NG; ++gg)
#pragma unroll
                for (int r = 0; r < 4; ++r) zacc[gg] += p[r] * Zv[r][gg];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const int gg = (16 * tt) / Gv < NG ? (16 * tt) / Gv : NG - 1;
                h8 B;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    _Float16 hi, lo;
                    split_f16(p[r] * Sv[r][gg] * v_inv_factor<BITS>(tt, r), hi, lo);
                    B[r] = hi;
                    B[4 + r] = lo;
                }
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dup_h8(A[tt]), B, O[tt], 0, 0, 0);
            }
        } else {
            // tail tile: each token from the codes (< TV), the residual (< T) or masked
            const uint16_t* ringV = V.v_ring + ((size_t)slot * H + h) * V.ring_elems;
            uint32_t vw[SLOT_WORDS];
#pragma unroll
            for (int k = 0; k < SLOT_WORDS; ++k) vw[k] = 0;
            if (p0 < TV) {
                if constexpr (BITS == 4) {
                    const uint4 u = *reinterpret_cast<const uint4*>(vslot);
                    vw[0] = u.x; vw[1] = u.y; vw[2] = u.z; vw[3] = u.w;
                } else {
                    const uint2 u = *reinterpret_cast<const uint2*>(vslot);
                    vw[0] = u.x; vw[1] = u.y;
                }
            }
            float Sv[4][NG], Zv[4][NG];
            int kind[4];  // 0 code, 1 residual, 2 masked
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pr = p0 + 4 * j + r;
                kind[r] = pr < TV ? 0 : (pr < T ? 1 : 2);
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) {
                    const uint32_t mw = kind[r] == 0 ? vmeta[r * NG + gg] : 0u;
                    Sv[r][gg] = f16_bits_to_f32((uint16_t)(mw & 0xFFFFu));
                    Zv[r][gg] = f16_bits_to_f32((uint16_t)(mw >> 16));
                }
            }
#pragma unroll
            for (int gg = 0; gg < NG; ++gg)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (kind[r] == 0) zacc[gg] += p[r] * Zv[r][gg];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const int gg = (16 * tt) / Gv < NG ? (16 * tt) / Gv : NG - 1;
                const int ch = 16 * tt + n;
                h4 A;
                h8 B;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int pr = p0 + 4 * j + r;
                    float wv = 0.0f;
                    if (kind[r] == 0) {
                        A[r] = (_Float16)(float)v_code_at<BITS>(vw, tt, r);
                        wv = p[r] * Sv[r][gg];
                    } else if (kind[r] == 1) {
                        A[r] = (_Float16)to_f32<DT>(ringV[(size_t)ch * R + (pr % R)]);
                        wv = p[r];
                    } else {
                        A[r] = (_Float16)0.0f;
                    }
                    _Float16 hi, lo;
                    split_f16(wv, hi, lo);
                    B[r] = hi;
                    B[4 + r] = lo;
                }
                O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dup_h8(A), B, O[tt], 0, 0, 0);
            }
        }
    }

    // ---- merge the 4 waves through LDS, then write this split's partial ----
    __shared__ float sm_m[kWaves][16], sm_l[kWaves][16];
    __shared__ float sm_o[kWaves][16][kHeadDim];
    const float l_tot = xor_sum(l_acc);
    float zt[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) zt[gg] = xor_sum(zacc[gg]);
    if (j == 0) {
        sm_m[wave][n] = m_run;
        sm_l[wave][n] = l_tot;
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ch = 16 * tt + 4 * j + r;
            sm_o[wave][n][ch] = O[tt][r] + zt[ch / Gv < NG ? ch / Gv : NG - 1];
        }
    __syncthreads();
    for (int idx = tid; idx < g * kHeadDim; idx += kThreads) {
        const int hn = idx / kHeadDim, ch = idx % kHeadDim;
        float mstar = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm_m[w][hn]);
        float lsum = 0.0f, osum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm_m[w][hn];
            const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - mstar);
            lsum += f * sm_l[w][hn];
            osum += f * sm_o[w][hn][ch];
        }
        float* part = a.partials + (((size_t)s * HQ + h * g + hn) * nsp + split) * kPartialStride;
        if (ch == 0) {
            part[0] = mstar;
            part[1] = lsum;
        }
        part[4 + ch] = osum;
    }
}

// Cross-split log-sum-exp merge: m = max m_i, l = sum l_i 2^(m_i - m),
// o = sum o_i 2^(m_i - m) / l (exp2 domain, as the partials are).
template <int DT>
__global__ __launch_bounds__(kHeadDim) void combine_kernel(DecodeArgs a) {
    const CacheView& V = a.v;
    const int HQ = a.num_q_heads;
    const int s = blockIdx.x / HQ;
    const int hq = blockIdx.x % HQ;
    const int ch = threadIdx.x;
    const int nsp = a.n_splits + 1;
    int T = a.seq_lens[s];
    const int slot = a.slot_ids[s];
    if (slot < 0 || slot >= V.max_seqs || T < 0) T = 0;
    const int n_main = max(0, T - V.R) / kTile;
    int nvalid = (n_main + a.tiles_per_split - 1) / a.tiles_per_split;
    nvalid = min(nvalid, a.n_splits);
    const float* base = a.partials + ((size_t)s * HQ + hq) * nsp * kPartialStride;
    float mstar = -INFINITY;
    for (int i = 0; i <= nvalid; ++i) {
        const int sp = i < nvalid ? i : a.n_splits;
        mstar = fmaxf(mstar, base[(size_t)sp * kPartialStride]);
    }
    float lsum = 0.0f, osum = 0.0f;
    if (mstar != -INFINITY) {
        for (int i = 0; i <= nvalid; ++i) {
            const int sp = i < nvalid ? i : a.n_splits;
            const float* p = base + (size_t)sp * kPartialStride;
            const float mi = p[0];
            if (mi == -INFINITY) continue;
            const float f = __builtin_amdgcn_exp2f(mi - mstar);
            lsum += f * p[1];
            osum += f * p[4 + ch];
        }
    }
    const float o = lsum > 0.0f ? osum / lsum : 0.0f;
    a.out[((size_t)s * HQ + hq) * kHeadDim + ch] = from_f32<DT>(o);
}

template <int BITS, int DT>
void launch_bits_dt(const DecodeArgs& a, int ng, dim3 grid, hipStream_t st) {
    dim3 block(kThreads);
    switch (ng) {
        case 1: hipLaunchKernelGGL((decode_kernel<BITS, DT, 1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<BITS, DT, 2>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<BITS, DT, 4>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((decode_kernel<BITS, DT, 8>), grid, block, 0, st, a); break;
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
    a.partials = partials;
    a.n_splits = plan.n_splits;
    a.tiles_per_split = plan.tiles_per_split;
    a.out = static_cast<uint16_t*>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int ng = kHeadDim / v.Gv;
    dim3 grid((unsigned)(num_seqs * v.H * (plan.n_splits + 1)));
    if (v.bits == 4) {
        if (v.dtype == kF16) launch_bits_dt<4, kF16>(a, ng, grid, st);
        else launch_bits_dt<4, kBF16>(a, ng, grid, st);
    } else {
        if (v.dtype == kF16) launch_bits_dt<2, kF16>(a, ng, grid, st);
        else launch_bits_dt<2, kBF16>(a, ng, grid, st);
    }
    int err = (int)hipGetLastError();
    if (err) return err;
    dim3 cgrid((unsigned)(num_seqs * num_q_heads)), cblock(kHeadDim);
    if (v.dtype == kF16) hipLaunchKernelGGL((combine_kernel<kF16>), cgrid, cblock, 0, st, a);
    else hipLaunchKernelGGL((combine_kernel<kBF16>), cgrid, cblock, 0, st, a);
    return (int)hipGetLastError();
}

// Prefill is implemented in its own file; until then a stub keeps the ABI.
}  // namespace kivi
