// FP8 (E4M3) KV cache: encode on append and split-K decode attention that
// restores values on read ("4.4 KV Cache 量化", section 4: the cache stored as
// FP8, E4M3 on ROCm, with one scale per tensor or per KV head; section 4.5 and
// "给 KV cache 减肥", section 3: values are restored before attention uses
// them). There are no groups and no residual: every token is encoded as it is
// appended.
//
// Append: 128-thread work groups per (sequence, KV head), each taking every
// gridDim.y-th new row, one thread per channel: y = x / scale in single
// precision, saturated to +-448 and rounded to the nearest E4M3 value (ties
// to even), stored as one byte in the lane slot layout the decode kernel
// reads.
//
// Decode: one work group of 8 waves per (sequence, KV head, split); each wave
// streams a contiguous run of 16-token tiles, one buffer of kF8BufTiles tiles
// in flight while it computes the other. Two E4M3 bytes become the fp16 numbers
// value*2^-8 in one conversion instruction (exact, subnormals included), so the
// scores S[16 tok][16 heads] = K x q^T are 4 v_mfma_f32_16x16x32_f16 and the
// values O^T[128][16] += V^T x P are 8 more, P split into fp16 hi + lo; the
// running max moves lazily, as in the KIVI decode kernel. The
// Key scale (times 2^8) folds into the softmax scale and the Value scale into
// the output. The waves merge (m, l, o) in LDS; with several splits a merge
// kernel combines the partials.

#include <algorithm>

#include "kivi_attn.h"

namespace kivi {
namespace {

using namespace attn;

constexpr int kF8DecWaves = 8;  // decode work groups: 8 waves (4 waves measured ~4 % slower, 16 no faster)
constexpr int kF8DecThreads = 64 * kF8DecWaves;
constexpr int kF8TileBytes = kTile * kHeadDim;  // 2 KiB: 64 lane slots of 32 bytes
constexpr int kF8MinSplitTiles = 32;
// 8-wave decode work groups launched at once: one per CU. Two per CU (twice
// the splits, so a merge launch on the Llama-3-8B shape) measured slower.
constexpr int kF8ResidentGroups = 256;
constexpr int kF8BufTiles = 1;  // tiles per load buffer (two buffers per wave); 2 and 4 measured slower

// ---------------------------------------------------------------- append ---

// E4M3 code of y: saturate at 448, then round to nearest even by the binary32
// fields (steps of 2^-9 below 2^-6, 3 fraction bits above). NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
#pragma clang fp contract(off)
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t c;
    if (a != a) {
        c = 0x7Fu;
    } else if (!(a < 448.0f)) {
        c = 0x7Eu;
    } else if (a < 0.015625f) {
        c = (uint32_t)__builtin_rintf(a * 512.0f);  // 8 is the smallest normal, 2^-6
    } else {
        const uint32_t u = __float_as_uint(a);
        const uint32_t m = u & 0x7FFFFFu;
        c = (((u >> 23) - 120u) << 3) | (m >> 20);  // exponent bias 127 -> 7
        const uint32_t rem = m & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (c & 1u))) c += 1u;
    }
    return sign | c;
}

struct F8AppendArgs {
    uint8_t* k_codes;
    uint8_t* v_codes;
    uint32_t* status;  // kivi_device_error bits
    int H, Bk, num_blocks, per_head;
    uint32_t code_bytes;
    const int32_t* seq_lens_before;
    const int32_t* cu_new;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_table;
    int bt_stride;
};

template <int DT>
__global__ __launch_bounds__(kHeadDim) void fp8_append_kernel(F8AppendArgs a) {
#pragma clang fp contract(off)
    const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
    // without cu_new, one row per sequence: row s (a decode step)
    const int row0 = a.cu_new ? a.cu_new[s] : s;
    const int n = a.cu_new ? a.cu_new[s + 1] - row0 : 1;
    const int T0 = a.seq_lens_before[s];
    if (T0 < 0 || n < 0) {  // skipped, and reported
        if (threadIdx.x == 0 && blockIdx.y == 0) report_error(a.status, KIVI_DEVERR_LENGTH);
        return;
    }
    const int c = threadIdx.x;
    const float ks = a.k_scale[a.per_head ? h : 0];
    const float vs = a.v_scale[a.per_head ? h : 0];
    for (int i = blockIdx.y; i < n; i += gridDim.y) {  // rows of the sequence's new tokens
        const int p = T0 + i;
        const int bi = p / a.Bk;
        if (bi >= a.bt_stride) {
            if (c == 0) report_error(a.status, KIVI_DEVERR_LENGTH);
            break;
        }
        const int blk = a.block_table[(size_t)s * a.bt_stride + bi];
        if (blk < 0 || blk >= a.num_blocks) {
            if (c == 0) report_error(a.status, KIVI_DEVERR_PAGE);
            continue;
        }
        const size_t src = ((size_t)(row0 + i) * a.H + h) * kHeadDim + c;
        const uint32_t ck = e4m3_code(to_f32<DT>(a.k_new[src]) / ks);
        const uint32_t cv = e4m3_code(to_f32<DT>(a.v_new[src]) / vs);
        const size_t tile = ((size_t)blk * a.H + h) * a.code_bytes + (size_t)((p % a.Bk) / kTile) * kF8TileBytes;
        const int m = p % kTile;
        // K: slot m + 16 ((c % 32) / 8), byte 8 (c / 32) + c % 8
        a.k_codes[tile + 32 * (m + 16 * ((c & 31) >> 3)) + 8 * (c >> 5) + (c & 7)] = (uint8_t)ck;
        // V: slot c % 16 + 16 (m / 4), byte 4 (c / 16) + m % 4
        a.v_codes[tile + 32 * ((c & 15) + 16 * (m >> 2)) + 4 * (c >> 4) + (m & 3)] = (uint8_t)cv;
    }
}

// ---------------------------------------------------------------- decode ---

struct F8DecodeArgs {
    const uint8_t* k_codes;
    const uint8_t* v_codes;
    uint32_t* status;  // kivi_device_error bits
    int H, Bk, num_blocks, per_head;
    uint32_t code_bytes, code_array_bytes;
    const uint16_t* q;
    const int32_t* seq_lens;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_table;
    int bt_stride;
    int num_q_heads, gqa, n_splits;
    int len_add;       // tokens appended since seq_lens (1 in a decode step)
    float scale_log2;  // softmax scale * log2(e)
    float* partials;   // [S][H_Q][n_splits][kPartialStride] when n_splits > 1
    uint16_t* out;
};

// fp16 pair (value(b0) 2^-8, value(b1) 2^-8) of E4M3 bytes 0 and 1 of w, or of
// bytes 2 and 3 (kHigh): one gfx950 v_cvt_scalef32_pk_f16_fp8. Its scale acts
// as a power of two, so 2^-8 is exact; every E4M3 value times 2^-8 is an fp16
// number (the smallest, 2^-17, an fp16 subnormal). A one-off device run over
// all 256 codes matched the E4M3 definition. It replaces a byte permute and two
// masks that built the same bits: 20 % off the prefill, 2 % off the decode.
template <bool kHigh>
__device__ __forceinline__ uint32_t f8_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 0.00390625f, kHigh));
}

// Value bytes of tokens at or past T (a sequence's last, partial tile) are
// never written and may hold an E4M3 NaN; their weights are 0, and 0 times NaN
// is NaN, so they are cleared: byte r of each word is token p0 + r.
__device__ __forceinline__ void mask_past_end(uint32_t vw[8], int p0, int T) {
    uint32_t keep = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (p0 + r < T) keep |= 0xFFu << (8 * r);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) vw[tt] &= keep;
}

struct F8Tile {
    uint4 k[2], v[2];
    bool ok;
};

// The bound of 512 threads lets the compiler keep every value in VGPRs (117);
// under the default bound of 1024 threads the accumulators are parked in
// AGPRs and copied back each tile.
template <int DT>
__global__ __launch_bounds__(kF8DecThreads, 1) void fp8_decode_kernel(F8DecodeArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int split = blockIdx.x % a.n_splits;
    const int sh = blockIdx.x / a.n_splits;
    const int s = sh / a.H, h = sh % a.H;
    const int g = a.gqa, HQ = a.num_q_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, j = lane >> 4;
    const int T = a.seq_lens[s] < 0 ? 0 : a.seq_lens[s] + a.len_add;
    const int n_tiles = (T + kTile - 1) / kTile;
    // device-side errors this wave met (wave-uniform), reported once at the end
    uint32_t err = 0;
    if (split == 0 && tid < 64 &&
        (a.seq_lens[s] < 0 || (long long)T > (long long)a.bt_stride * a.Bk))
        err = KIVI_DEVERR_LENGTH;
    // this split's tiles, then this wave's contiguous share of them
    const int s_begin = (int)((long long)n_tiles * split / a.n_splits);
    const int s_end = (int)((long long)n_tiles * (split + 1) / a.n_splits);
    const int w_begin = s_begin + (s_end - s_begin) * wave / kF8DecWaves;
    const int w_end = s_begin + (s_end - s_begin) * (wave + 1) / kF8DecWaves;

    const float ks = a.k_scale[a.per_head ? h : 0];
    const float vs = a.v_scale[a.per_head ? h : 0];
    const float xs = a.scale_log2 * ks * 256.0f;  // log2-unit score of q . (value 2^-8)

    // query operand: lane (n, j) holds q[head n][32 i + 8 j .. + 7], i = 0..3
    h8 Bq[4];
    {
        const uint16_t* qrow = a.q + ((size_t)s * HQ + h * g + min(n, g - 1)) * kHeadDim + 8 * j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * i);
            if (n >= g) u = (uint4){0, 0, 0, 0};
            if constexpr (DT == kBF16) {
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const _Float16 lo = (_Float16)bf16_bits_to_f32((uint16_t)(w[e] & 0xFFFFu));
                    const _Float16 hi = (_Float16)bf16_bits_to_f32((uint16_t)(w[e] >> 16));
                    o[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                u = (uint4){o[0], o[1], o[2], o[3]};
            }
            Bq[i] = make_h8(u.x, u.y, u.z, u.w);
        }
    }

    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_codes, a.code_array_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_codes, a.code_array_bytes);
    const int32_t* bt = a.block_table + (size_t)s * a.bt_stride;
    const int tpp_shift = __builtin_ctz((unsigned)(a.Bk / kTile));
    auto page_ids = [&](int t0) -> int {  // lane l: page of tile t0 + l (-1 past the table)
        const int bi = (t0 + lane) >> tpp_shift;
        return (t0 + lane < w_end && bi < a.bt_stride) ? bt[bi] : -1;
    };
    int base = w_begin;
    int my_page = page_ids(base);
    int next_page = page_ids(base + 64);
    const uint32_t lane_off = 32u * (uint32_t)lane;

    auto issue = [&](int t, F8Tile& x) {
        if (t - base >= 64) {
            base += 64;
            my_page = next_page;
            next_page = page_ids(base + 64);
        }
        const int pg = __builtin_amdgcn_readlane(my_page, (t - base) & 63);
        x.ok = t < w_end && pg >= 0 && pg < a.num_blocks;
        if (t < w_end && !x.ok) err |= KIVI_DEVERR_PAGE;
        const uint32_t off = ((uint32_t)(x.ok ? pg : 0) * (uint32_t)a.H + (uint32_t)h) * a.code_bytes +
                             (uint32_t)(t & ((1 << tpp_shift) - 1)) * kF8TileBytes;
        x.k[0] = buf_b128(rk, lane_off, off);
        x.k[1] = buf_b128(rk, lane_off + 16u, off);
        x.v[0] = buf_b128(rv, lane_off, off);
        x.v[1] = buf_b128(rv, lane_off + 16u, off);
    };

    float m_run = -INFINITY, l_acc = 0.0f;
    f4 O[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] = (f4){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const F8Tile& x, int t) {
        if (!x.ok) return;
        const uint32_t kw[8] = {x.k[0].x, x.k[0].y, x.k[0].z, x.k[0].w, x.k[1].x, x.k[1].y, x.k[1].z, x.k[1].w};
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h8 A = make_h8(f8_pair<false>(kw[2 * i]), f8_pair<true>(kw[2 * i]),
                                 f8_pair<false>(kw[2 * i + 1]), f8_pair<true>(kw[2 * i + 1]));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bq[i], acc, 0, 0, 0);
        }
        // acc[r]: token 16 t + 4 j + r, head n
        const int p0 = kTile * t + 4 * j;
        float xr[4], mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xr[r] = p0 + r < T ? acc[r] * xs : -INFINITY;
            mx = fmaxf(mx, xr[r]);
        }
        // The running max moves only when a score passes it by more than
        // kLazyLog2 (weights stay below 2^kLazyLog2), so the accumulators are
        // rescaled rarely; the branch is taken by the whole wave or not at all.
        const float mt = xor_max(mx);  // finite: the tile holds a token < T
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazyLog2) != 0) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run is -inf
            l_acc *= alpha;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) O[tt] *= alpha;
            m_run = m_new;
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(xr[r] - m_run);
        l_acc += (p[0] + p[1]) + (p[2] + p[3]);
        h8 B;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            _Float16 hi, lo;
            split_f16(p[r], hi, lo);
            B[r] = hi;
            B[4 + r] = lo;
        }
        uint32_t vw[8] = {x.v[0].x, x.v[0].y, x.v[0].z, x.v[0].w, x.v[1].x, x.v[1].y, x.v[1].z, x.v[1].w};
        if (kTile * t + kTile > T) mask_past_end(vw, p0, T);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            const h4 A = make_h4(f8_pair<false>(vw[tt]), f8_pair<true>(vw[tt]));
            O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dup_h8(A), B, O[tt], 0, 0, 0);
        }
    };

    if (w_begin < w_end) {
        constexpr int NB = kF8BufTiles;
        F8Tile xa[NB], xb[NB];
#pragma unroll
        for (int e = 0; e < NB; ++e) issue(w_begin + e, xa[e]);
        for (int t = w_begin; t < w_end; t += 2 * NB) {
#pragma unroll
            for (int e = 0; e < NB; ++e) issue(t + NB + e, xb[e]);
#pragma unroll
            for (int e = 0; e < NB; ++e) compute(xa[e], t + e);
            if (t + NB >= w_end) break;
#pragma unroll
            for (int e = 0; e < NB; ++e) issue(t + 2 * NB + e, xa[e]);
#pragma unroll
            for (int e = 0; e < NB; ++e) compute(xb[e], t + NB + e);
        }
    }

    // ---- merge the waves in LDS: m (log2 units), l, o per query head ----
    const float l_tot = xor_sum(l_acc);
    float* sm_m = reinterpret_cast<float*>(smem);  // [kF8DecWaves][g]
    float* sm_l = sm_m + kF8DecWaves * g;              // [kF8DecWaves][g]
    float* sm_o = sm_l + kF8DecWaves * g;              // [kF8DecWaves][g][128]
    if (n < g) {
        if (j == 0) {
            sm_m[wave * g + n] = m_run;
            sm_l[wave * g + n] = l_tot;
        }
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm_o[(wave * g + n) * kHeadDim + 16 * tt + 4 * j + r] = O[tt][r];
    }
    __syncthreads();
    if (err != 0 && lane == 0) report_error(a.status, err);
    const float vsc = vs * 256.0f;
    for (int idx = tid; idx < g * kHeadDim; idx += kF8DecThreads) {
        const int hn = idx / kHeadDim, chn = idx % kHeadDim;
        float mstar = -INFINITY;
#pragma unroll
        for (int w = 0; w < kF8DecWaves; ++w) mstar = fmaxf(mstar, sm_m[w * g + hn]);
        float lsum = 0.0f, osum = 0.0f;
#pragma unroll
        for (int w = 0; w < kF8DecWaves; ++w) {
            const float mw = sm_m[w * g + hn];
            const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - mstar);
            lsum += f * sm_l[w * g + hn];
            osum += f * sm_o[(w * g + hn) * kHeadDim + chn];
        }
        const size_t row = (size_t)s * HQ + h * g + hn;
        if (a.n_splits == 1) {
            a.out[row * kHeadDim + chn] = from_f32<DT>(lsum > 0.0f ? osum * vsc / lsum : 0.0f);
        } else {
            float* part = a.partials + (row * a.n_splits + split) * kPartialStride;
            if (chn == 0) {
                part[0] = mstar;
                part[1] = lsum;
            }
            part[4 + chn] = osum * vsc;
        }
    }
}

// Merge of the split partials of one (sequence, query head), one thread per
// channel: m = max m_i, l = sum l_i 2^(m_i - m), o = sum o_i 2^(m_i - m) / l;
// splits without tokens carry m_i = -inf.
template <int DT>
__global__ __launch_bounds__(kHeadDim) void fp8_merge_kernel(const float* partials, int n_splits, uint16_t* out) {
    const int row = blockIdx.x, chn = threadIdx.x;
    const float* pb = partials + (size_t)row * n_splits * kPartialStride;
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    for (int i = 0; i < n_splits; ++i) {
        const float* pp = pb + (size_t)i * kPartialStride;
        const float mi = pp[0];
        if (mi == -INFINITY) continue;
        const float mn = fmaxf(m, mi);
        const float fo = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        const float fi = __builtin_amdgcn_exp2f(mi - mn);
        l = l * fo + pp[1] * fi;
        o = o * fo + pp[4 + chn] * fi;
        m = mn;
    }
    out[(size_t)row * kHeadDim + chn] = from_f32<DT>(l > 0.0f ? o / l : 0.0f);
}

// ---------------------------------------------------------------- prefill ---
//
}  // namespace

Fp8Plan fp8_decode_plan(int num_seqs, int num_kv_heads, int num_q_heads, int max_seq_len) {
    const int pairs = std::max(1, num_seqs * num_kv_heads);
    const int tiles = (std::max(0, max_seq_len) + kTile - 1) / kTile;
    // about one 8-wave work group per CU on 256 CUs, at least
    // kF8MinSplitTiles tiles per split
    int n_splits = std::max(1, (kF8ResidentGroups + pairs / 2) / pairs);
    n_splits = std::min(n_splits, std::max(1, (tiles + kF8MinSplitTiles - 1) / kF8MinSplitTiles));
    n_splits = std::max(1, std::min(n_splits, 256));
    Fp8Plan p;
    p.n_splits = n_splits;
    p.ws_bytes = n_splits > 1 ? (size_t)num_seqs * num_q_heads * n_splits * kPartialStride * sizeof(float) : 0;
    return p;
}

int launch_fp8_append(const CacheView& v, int per_head, int num_seqs, const int32_t* seq_lens_before,
                      const int32_t* cu_new, int max_new, const void* k_new, const void* v_new,
                      const float* k_scale, const float* v_scale, const int32_t* block_table, int bt_stride,
                      void* stream) {
    F8AppendArgs a;
    a.k_codes = v.k_codes;
    a.v_codes = v.v_codes;
    a.status = v.status;
    a.H = v.H;
    a.Bk = v.Bk;
    a.num_blocks = v.num_blocks;
    a.per_head = per_head;
    a.code_bytes = (uint32_t)v.code_bytes;
    a.seq_lens_before = seq_lens_before;
    a.cu_new = cu_new;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    hipStream_t st = static_cast<hipStream_t>(stream);
    dim3 grid((unsigned)(num_seqs * v.H), (unsigned)std::min(max_new, 1024));
    if (v.dtype == kF16) hipLaunchKernelGGL((fp8_append_kernel<kF16>), grid, dim3(kHeadDim), 0, st, a);
    else hipLaunchKernelGGL((fp8_append_kernel<kBF16>), grid, dim3(kHeadDim), 0, st, a);
    return (int)hipGetLastError();
}

int launch_fp8_decode(const CacheView& v, int per_head, int num_seqs, int num_q_heads, const void* q,
                      const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                      const int32_t* block_table, int bt_stride, float softmax_scale, void* out, float* partials,
                      const Fp8Plan& plan, void* stream, int len_add) {
    F8DecodeArgs a;
    a.k_codes = v.k_codes;
    a.v_codes = v.v_codes;
    a.status = v.status;
    a.H = v.H;
    a.Bk = v.Bk;
    a.num_blocks = v.num_blocks;
    a.per_head = per_head;
    a.code_bytes = (uint32_t)v.code_bytes;
    a.code_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.code_bytes);
    a.q = static_cast<const uint16_t*>(q);
    a.seq_lens = seq_lens;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.num_q_heads = num_q_heads;
    a.gqa = num_q_heads / v.H;
    a.n_splits = plan.n_splits;
    a.len_add = len_add;
    a.scale_log2 = softmax_scale * kLog2e;
    a.partials = partials;
    a.out = static_cast<uint16_t*>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    dim3 grid((unsigned)(num_seqs * v.H * plan.n_splits));
    const size_t lds = (size_t)kF8DecWaves * a.gqa * (kHeadDim + 2) * sizeof(float);
    if (v.dtype == kF16) hipLaunchKernelGGL((fp8_decode_kernel<kF16>), grid, dim3(kF8DecThreads), lds, st, a);
    else hipLaunchKernelGGL((fp8_decode_kernel<kBF16>), grid, dim3(kF8DecThreads), lds, st, a);
    if (plan.n_splits > 1) {
        dim3 mgrid((unsigned)(num_seqs * num_q_heads));
        if (v.dtype == kF16)
            hipLaunchKernelGGL((fp8_merge_kernel<kF16>), mgrid, dim3(kHeadDim), 0, st, partials, plan.n_splits,
                               a.out);
        else
            hipLaunchKernelGGL((fp8_merge_kernel<kBF16>), mgrid, dim3(kHeadDim), 0, st, partials, plan.n_splits,
                               a.out);
    }
    return (int)hipGetLastError();
}

}  // namespace kivi
