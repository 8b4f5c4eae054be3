// Device building blocks shared by the decode and prefill attention kernels
// (dequantise-on-read attention over the KIVI cache: "4.4 KV Cache 量化",
// sections 2 and 3; "给 KV cache 减肥", section 3).
#pragma once

#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {
namespace attn {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Query rows and Key-group tables live in LDS as fp16 rows of kQRow elements
// (272 bytes: the 16-byte pad spreads rows over banks).
constexpr int kQRow = 136;
constexpr int kRowBytes = kQRow * 2;

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

// x = hi + lo with both parts fp16 (about 22 significant bits together).
// x is pinned to a register first: the compiler may otherwise fold the
// product that makes x into a single-rounding conversion for one use of hi
// and not for another, and then hi + lo misses x by an fp16 ulp of hi.
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
    asm volatile("" : "+v"(x));
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
// kFold: keep the 1024 offsets (one and-or per pair, no subtract); the table
// built with the same kFold takes 1024 sum_c Q'[n][c] out of the bias instead.
template <int BITS, bool kFold = false>
__device__ __forceinline__ void unpack_k(const uint32_t* kw, h8 A[4]) {
    auto pr = [](uint32_t x, uint32_t m) -> uint32_t { return kFold ? magic_pair(x, m) : exact_pair(x, m); };
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = kw[i], w8 = w >> 8;
            A[i] = make_h8(pr(w, 0x000F000Fu), pr(w, 0x00F000F0u), pr(w8, 0x000F000Fu), pr(w8, 0x00F000F0u));
        }
    } else {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t x = kw[w], x8 = x >> 8;
            A[2 * w] = make_h8(pr(x, 0x00030003u), pr(x, 0x000C000Cu), pr(x, 0x00300030u), pr(x, 0x00C000C0u));
            A[2 * w + 1] = make_h8(pr(x8, 0x00030003u), pr(x8, 0x000C000Cu), pr(x8, 0x00300030u),
                                   pr(x8, 0x00C000C0u));
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
            A[4 * w + 0] = make_h4(magic_pair(x, 0x00030003u), magic_pair(x, 0x000C000Cu));
            A[4 * w + 1] = make_h4(magic_pair(x, 0x00300030u), magic_pair(x, 0x00C000C0u));
            A[4 * w + 2] = make_h4(magic_pair(x8, 0x00030003u), magic_pair(x8, 0x000C000Cu));
            A[4 * w + 3] = make_h4(magic_pair(x8, 0x00300030u), magic_pair(x8, 0x00C000C0u));
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

// Sum over the 16 lanes of a row (lanes 16r .. 16r+15), every lane gets it.
__device__ __forceinline__ float row_sum16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row mirror
    return x;
}

// Byte offset into the Key meta array of this lane's 8-channel run (channels
// 8 (lane & 15) .. +7) of a Key group, given the physical page holding them.
__device__ __forceinline__ uint32_t k_meta_off(const CacheView& V, int h, int page, int nch) {
    const int ch = 8 * (threadIdx.x & 15);
    return ((uint32_t)max(page, 0) * (uint32_t)V.H + (uint32_t)h) * (uint32_t)V.k_meta_bytes + 2u * (uint32_t)(ch % nch);
}

// Query table of one Key group, built by one wave into its own LDS rows:
//   hi/lo rows: Q'[n][c] = sgn q[n][c] s[c] f(c) as an fp16 pair (hi + lo),
//   where f(c) is the inverse place value of channel c's field in the code
//   words and sgn the sign of the softmax scale;
//   bias[n] = sgn sum_c q[n][c] z[c] (fp16 products, fp32 sums).
// Lane (k = lane & 15, r = lane >> 4) covers channels 8k..8k+7 of heads
// r, r+4, r+8, r+12. sv/zv: the lane's 8 scales and zero-points. Returns
// bias[nr] for this lane's score row nr: the start of its score chains.
template <int BITS, bool kFold = false>
__device__ __forceinline__ float build_table(int g, uint4 sv, uint4 zv, const uint16_t* lq, uint8_t* lt, float* lbias,
                                             int nr, float sgn) {
    const int lane = threadIdx.x & 63, k = lane & 15, r = lane >> 4;
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
    h2 sf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float f = sgn * ((BITS == 4) ? ((e & 1) ? 0.0625f : 1.0f) : 1.0f / (float)(1 << (2 * e)));
        sf[e] = __builtin_bit_cast(h2, sw[e]) * (h2){(_Float16)f, (_Float16)f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (4 * u >= g) break;  // uniform
        const int hn = r + 4 * u;
        const bool ok = hn < g;
        const uint4 qu = *reinterpret_cast<const uint4*>(lq + (ok ? hn : 0) * kQRow + 8 * k);
        const uint32_t qw[4] = {qu.x, qu.y, qu.z, qu.w};
        uint32_t hw[4], lw[4];
        float zq = 0.0f, qs = 0.0f;
        const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const h2 qv = __builtin_bit_cast(h2, qw[e]);
            const h2 hi = qv * sf[e];
            const h2 lo = __builtin_elementwise_fma(qv, sf[e], -hi);  // fp16(q s f - hi)
            hw[e] = __builtin_bit_cast(uint32_t, hi);
            lw[e] = __builtin_bit_cast(uint32_t, lo);
            zq = __builtin_amdgcn_fdot2(qv, __builtin_bit_cast(h2, zw[e]), zq, false);
            if constexpr (kFold) {  // the table entries exactly as the MFMAs multiply them
                qs = __builtin_amdgcn_fdot2(hi, one, qs, false);
                qs = __builtin_amdgcn_fdot2(lo, one, qs, false);
            }
        }
        zq = row_sum16(ok ? zq : 0.0f);
        if constexpr (kFold) qs = row_sum16(ok ? qs : 0.0f);
        if (ok) {
            *reinterpret_cast<uint4*>(lt + (2 * hn + 0) * kRowBytes + 16 * k) = (uint4){hw[0], hw[1], hw[2], hw[3]};
            *reinterpret_cast<uint4*>(lt + (2 * hn + 1) * kRowBytes + 16 * k) = (uint4){lw[0], lw[1], lw[2], lw[3]};
            if (k == 0) lbias[hn] = kFold ? __builtin_fmaf(-1024.0f, qs, sgn * zq) : sgn * zq;
        }
    }
    // LDS operations of one wave complete in order; the fence keeps the
    // compiler from moving the reads below above the writes.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    return lbias[nr];
}

__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }
__device__ __forceinline__ float max4(f4 x) { return max2(max2(x[0], x[1]), max2(x[2], x[3])); }

// Per-lane online-softmax state of query head (lane & 15). Scores are kept in
// raw units (sgn q.k~); the weight of a score x is 2^((x - m) |scale| log2 e).
// The running max m moves only when a score passes it by more than
// kLazyLog2 / (|scale| log2 e): weights stay below 2^kLazyLog2 and the
// rescale of the accumulators is rare.
// O[t][r] holds O^T[16 t + 4 (lane >> 4) + r][head]; wsum[gg][vb] sums the
// Value-side weights of channel group gg and pair-factor variant vb (codes
// that carry a 1024 offset leave each output channel 1024 wsum too much
// until the merge takes it out).
constexpr float kLazyLog2 = 2.0f;

template <int NG, int NB>
struct Acc {
    float m_run, mneg, l_acc, zacc[NG], wsum[NG][NB];
    f4 O[8];
    __device__ __forceinline__ void init() {
        m_run = -INFINITY;
        mneg = 0.0f;
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
    // mx: this lane's largest new score (already reduced over the head's
    // lanes). The branch is taken by the whole wave or not at all.
    __device__ __forceinline__ void rescale(float mx, float sl2, float thr) {
        if (__builtin_amdgcn_ballot_w64(mx > m_run + thr) != 0) {
            const float mnew = max2(m_run, mx);
            const float f = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_run - mnew) * sl2);
            l_acc *= f;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                zacc[gg] *= f;
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) wsum[gg][vb] *= f;
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) O[t] *= f;
            m_run = mnew;
            mneg = -mnew * sl2;
        }
    }
    __device__ __forceinline__ float weight(float x, float sl2) const {
        return __builtin_amdgcn_exp2f(__builtin_fmaf(x, sl2, mneg));
    }
    // Take the 1024 offsets accumulated so far out of O (main-range Value codes
    // of int4 and int2 enter as 1024 + field). An accumulator that carries
    // them is ~137 times larger than its useful part for int4 (fields of
    // 0..15 under 1024), ~680 times for int2,
    // so fp32 rounding in the MFMA sums grows with the tokens summed;
    // flushing every few hundred tokens bounds it. Wave-uniform call.
    template <int BITS>
    __device__ __forceinline__ void flush_offsets() {
        {
            float c[NG][NB];
#pragma unroll
            for (int gg = 0; gg < NG; ++gg)
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    c[gg][vb] = -1024.0f * xor_sum(wsum[gg][vb]);
                    wsum[gg][vb] = 0.0f;
                }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const float x = c[(16 * tt) / (kHeadDim / NG)][tt % NB];
                O[tt] += (f4){x, x, x, x};
            }
        }
    }
};

// Main-loop iterations (each 2 kHalf tiles) between two offset flushes: about
// 16 tile pairs.
template <int kHalf>
constexpr int flush_period() { return 16 / kHalf > 0 ? 16 / kHalf : 1; }

// Raw scores of a 16-token tile whose Keys are quantised: one accumulation
// chain that starts at the zero-point bias and takes the group's hi and lo
// B-operands from the wave's LDS table. `row`: the lane's byte offset into
// the table (head row nr, k-slice 16 j).
template <int BITS, bool kFold = false>
__device__ __forceinline__ f4 code_scores(const uint32_t* kw, const uint8_t* lt, int row, float bias) {
    h8 A[4];
    unpack_k<BITS, kFold>(kw, A);
    f4 acc = {bias, bias, bias, bias};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h8 bh = *reinterpret_cast<const h8*>(lt + row + 64 * i);
        const h8 bl = *reinterpret_cast<const h8*>(lt + row + kRowBytes + 64 * i);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], bl, acc, 0, 0, 0);
    }
    return acc;
}

// fp16 pair of the low (scale) or high (zero-point) halves of two meta words.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }

// Value side of two main tiles (A, B): one MFMA per 16-channel tile covers
// both, with k = (tile A tokens 4j..4j+3, tile B tokens 4j..4j+3) in each
// lane; its A-operand holds the codes, its B-operand the fp16 weights
// p * scale / F (F: the place value of the token's code field). Zero-points
// go through zacc. A tile that is not computed (oka / okb false: outside the
// wave's range, or without a page) has zero weights, and its metadata, loaded
// from whatever page 0 holds, is replaced by zeros: 0 times a NaN or infinite
// scale left in an unused page would otherwise poison the accumulators.
template <int BITS, int NG, int NB>
__device__ __forceinline__ void value_pair(Acc<NG, NB>& st, const uint32_t* vwa, const uint32_t* vma_in,
                                           const uint32_t* vwb, const uint32_t* vmb_in, const float pa[4],
                                           const float pb[4], bool oka, bool okb) {
    uint32_t vma[4 * NG], vmb[4 * NG];
#pragma unroll
    for (int k = 0; k < 4 * NG; ++k) {
        vma[k] = oka ? vma_in[k] : 0u;
        vmb[k] = okb ? vmb_in[k] : 0u;
    }
    constexpr float kF23 = (BITS == 4) ? 0.0625f : 0.25f;  // 1/F of tokens r = 2, 3
    const h2 qa01 = {(_Float16)pa[0], (_Float16)pa[1]};
    const h2 qa23 = {(_Float16)(pa[2] * kF23), (_Float16)(pa[3] * kF23)};
    const h2 qb01 = {(_Float16)pb[0], (_Float16)pb[1]};
    const h2 qb23 = {(_Float16)(pb[2] * kF23), (_Float16)(pb[3] * kF23)};
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    uint32_t Bw[NG][NB][4];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
        const h2 wa01 = qa01 * __builtin_bit_cast(h2, lo_halves(vma[0 * NG + gg], vma[1 * NG + gg]));
        const h2 wa23 = qa23 * __builtin_bit_cast(h2, lo_halves(vma[2 * NG + gg], vma[3 * NG + gg]));
        const h2 wb01 = qb01 * __builtin_bit_cast(h2, lo_halves(vmb[0 * NG + gg], vmb[1 * NG + gg]));
        const h2 wb23 = qb23 * __builtin_bit_cast(h2, lo_halves(vmb[2 * NG + gg], vmb[3 * NG + gg]));
        Bw[gg][0][0] = __builtin_bit_cast(uint32_t, wa01);
        Bw[gg][0][1] = __builtin_bit_cast(uint32_t, wa23);
        Bw[gg][0][2] = __builtin_bit_cast(uint32_t, wb01);
        Bw[gg][0][3] = __builtin_bit_cast(uint32_t, wb23);
        // the exact fp16 weights the MFMA multiplies the 1024 offsets with
        float ws = __builtin_amdgcn_fdot2(wa01, one, st.wsum[gg][0], false);
        ws = __builtin_amdgcn_fdot2(wa23, one, ws, false);
        ws = __builtin_amdgcn_fdot2(wb01, one, ws, false);
        st.wsum[gg][0] = __builtin_amdgcn_fdot2(wb23, one, ws, false);
        if constexpr (BITS == 2) {
            // odd channel tiles: fields 4 places up (factor 1/16)
            const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
            const h2 sa01 = wa01 * k16, sa23 = wa23 * k16, sb01 = wb01 * k16, sb23 = wb23 * k16;
            Bw[gg][1][0] = __builtin_bit_cast(uint32_t, sa01);
            Bw[gg][1][1] = __builtin_bit_cast(uint32_t, sa23);
            Bw[gg][1][2] = __builtin_bit_cast(uint32_t, sb01);
            Bw[gg][1][3] = __builtin_bit_cast(uint32_t, sb23);
            float w1 = __builtin_amdgcn_fdot2(sa01, one, st.wsum[gg][1], false);
            w1 = __builtin_amdgcn_fdot2(sa23, one, w1, false);
            w1 = __builtin_amdgcn_fdot2(sb01, one, w1, false);
            st.wsum[gg][1] = __builtin_amdgcn_fdot2(sb23, one, w1, false);
        }
        float z = st.zacc[gg];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            z += pa[r] * f16_bits_to_f32((uint16_t)(vma[r * NG + gg] >> 16));
            z += pb[r] * f16_bits_to_f32((uint16_t)(vmb[r * NG + gg] >> 16));
        }
        st.zacc[gg] = z;
    }
    h4 Aa[8], Ab[8];
    unpack_v<BITS>(vwa, Aa);
    unpack_v<BITS>(vwb, Ab);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const int gg = (16 * tt) / (kHeadDim / NG);
        const uint32_t* bw = Bw[gg][tt % NB];
        const h8 Bv = make_h8(bw[0], bw[1], bw[2], bw[3]);
        const h8 Av = (h8){Aa[tt][0], Aa[tt][1], Aa[tt][2], Aa[tt][3], Ab[tt][0], Ab[tt][1], Ab[tt][2], Ab[tt][3]};
        st.O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av, Bv, st.O[tt], 0, 0, 0);
    }
}

template <int BITS, int NG>
struct TileRegs {
    uint32_t k[BITS];
    uint32_t v[BITS];
    uint32_t vm[4 * NG];
};

}  // namespace attn
}  // namespace kivi
