// Chunked-prefill attention over the KIVI cache as stored, after the chunk
// was appended ("4.4 KV Cache 量化", section 2: P = softmax(Q K^T / sqrt(d)),
// out = P V; section 3.2: quantised history plus the full-precision
// residual; "给 KV cache 减肥", section 3: values restored on read).
//
// Rows: the (query position, query head) pairs of one (sequence, KV head),
// row r = i * g + head for chunk query i. A work group of 8 waves owns 256
// consecutive rows, 32 per wave, and walks the 64-token tiles its rows can
// see. Each tile is restored once per work group: each of its 512 threads
// takes half of a 16-byte lane slot of Key codes and half of one of Value
// codes and writes the restored values to LDS, Keys as [token][channel],
// Values as [channel][token]. A restored Key k = code * scale + zero is kept
// as an fp16 pair hi + lo (hi = fp16(k), lo = fp16(k - hi), about 22 bits):
// outlier channels reach |k| of tens, where one fp16 rounding alone moves a
// score by more than the attention tolerance allows. Values are restored to
// fp16 with one packed FMA per pair (their rounding is averaged out).
// Two LDS stages: the next tile is restored while the current tile's score
// products run, from codes loaded half a tile earlier; one barrier per tile.
// Per wave and tile, on matrix cores (v_mfma_f32_32x32x16_f16, fp32 sums):
//   S^T[64 tokens][32 rows] = (K_hi + K_lo)[64][128] Q^T[128][32]   32 MFMAs
//   online softmax per row (one lane pair per row; the running max moves
//   per tile), weights as fp16
//   O^T[128][32] += V^T[128][64] P^T[64][32]                        16 MFMAs
// The k-order of the P^T V MFMAs is the order in which the score MFMAs leave
// the weights in the lanes; the Value rows in LDS are stored in that order.
// Tiles that reach the residual, the end of the sequence or (second reading
// below) the chunk are restored from the right source per token.
//
// The FP8 cache ("4.4 KV Cache 量化", section 4) runs the same kernel with
// BITS = 8: each tile's E4M3 bytes become exact fp16 values (value times 2^-8)
// in one conversion per pair, so the Keys need no lo part (32 products per
// tile instead of 48); the Key scale folds into the softmax scale, the Value
// scale multiplies the normalised output, and there is no residual.
//
// Second reading of the prefill (the pages leave it open): with a chunk given
// at full precision, the call comes before the chunk is stored; seq_lens are
// the lengths P before it, the chunk's rows sit at positions P .. P + n_q - 1,
// and their Keys and Values are read from the chunk's own input rows instead
// of the cache, so only the history is dequantised.

#include <algorithm>

#include "kivi_attn.h"

namespace kivi {
namespace {

using namespace attn;

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kRowsWave = 32;                 // query rows per wave (the N of the 32x32 MFMAs)
constexpr int kRowsWg = kRowsWave * kPWaves;  // 256
constexpr int kTileTok = 64;                  // tokens per KV tile: 4 sub-tiles of 16
constexpr int kXcds = 8;                      // accelerator complex dies of an MI355X, each with its own L2
// LDS rows of one stage (fp16), padded by 16 bytes so that the 8 lanes a
// 16-byte read serves per cycle fall on distinct banks:
//   Key hi, Key lo  [64 tokens][128 channels + 8] each
//   Value [128 channels][64 tokens + 8], the tokens of each 16-token k-step
//         in the order the weights sit in the lanes (v_pos)
constexpr int kKRow = kHeadDim + 8;
constexpr int kVRow = kTileTok + 8;
constexpr int kKHalfs = kTileTok * kKRow;     // one Key part
constexpr int kVOff = 2 * kKHalfs;            // the Value rows within a stage
constexpr int kStageHalfs = 2 * kKHalfs + kHeadDim * kVRow;
// Key scales and zero-points of a tile, per 16-token sub-tile: [4][2][128] fp16
// (the group of each sub-tile), in two stages of their own
constexpr int kMetaHalfs = 4 * 2 * kHeadDim;
constexpr size_t kPrefillLds = (2 * kStageHalfs + 2 * kMetaHalfs) * sizeof(_Float16);
// Running-max threshold (log2 units): weights stay below 2^kLazy, rescales are rare
constexpr float kLazy = 2.0f;

struct PrefillArgs {
    CacheView v;
    const uint16_t* q;
    const uint16_t* k_chunk;  // chunk rows at full precision, or null
    const uint16_t* v_chunk;
    const int32_t* cu_q;
    const int32_t* slot_ids;
    const int32_t* seq_lens;
    const int32_t* block_table;
    int bt_stride;
    int num_q_heads;
    int gqa;
    float scale_log2;  // softmax scale * log2(e)
    int causal;
    int max_q_len;     // the caller's bound of every query span
    int wg_per_sh;     // work groups per (sequence, KV head)
    const float* k_scale;  // FP8 cache: per-tensor or per-KV-head scales
    const float* v_scale;
    int per_head;
    uint16_t* out;
};

// Position of token 4a + r of a 16-token k-step in a Value row: the lanes of
// half h of a P^T V MFMA hold tokens 4h .. 4h + 3 and 8 + 4h .. 8 + 4h + 3 of
// the k-step (in that order) as their 8 k-values, so blocks of 4 tokens are
// stored in the order a = 0, 2, 1, 3.
__device__ __forceinline__ int v_pos(int a) { return 8 * (a & 1) + 4 * (a >> 1); }

// Exact fp16 pair of the two code fields at bit `sh` of each half of x.
template <int BITS>
__device__ __forceinline__ h2 code_pair(uint32_t x, int sh) {
    const uint32_t m = magic_pair(x >> sh, BITS == 4 ? 0x000F000Fu : 0x00030003u);
    return __builtin_bit_cast(h2, m) - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
}
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
// fp16 pair (value 2^-8) of E4M3 bytes 0, 1 of w, or of bytes 2, 3 (kHigh):
// one gfx950 v_cvt_scalef32_pk_f16_fp8; the scale acts as a power of two, so
// the pair is exact
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 0.00390625f, kHigh));
}
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// The codes a thread restores for one tile: half of its Key slot and of its
// Value slot of sub-tile u, and the Value metadata of the slot's 4 tokens for
// the groups of its channels.
template <int BITS, int NGP>
struct SlotRegs {
    uint32_t k[BITS / 2], v[BITS / 2];
    uint32_t vm[4 * NGP];
};

template <int BITS, int DT, int NG>
__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(PrefillArgs a) {
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;
    constexpr int SLOT_BYTES = 4 * BITS;
    extern __shared__ __align__(16) _Float16 lds[];
    const CacheView& V = a.v;
    const int H = V.H;
    // Work groups are dealt to the 8 XCDs in turn (block b to XCD b % 8). The
    // blocks of one XCD take consecutive work items, so the work groups of one
    // (sequence, KV head), which all read its cache, share that XCD's L2.
    const int nblk = (int)gridDim.x, xcd = (int)blockIdx.x % kXcds, per = nblk / kXcds, extra = nblk % kXcds;
    const int item = xcd * per + min(xcd, extra) + (int)blockIdx.x / kXcds;
    const int wg = item % a.wg_per_sh;
    const int sh = item / a.wg_per_sh;
    const int s = sh / H, h = sh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = a.gqa;
    const int HQ = a.num_q_heads;

    // ---- the sequence ----
    const int q0 = a.cu_q[s];
    const int nq = a.cu_q[s + 1] - q0;
    int P = a.seq_lens[s];  // tokens in the cache (before the chunk when it comes raw)
    constexpr bool kF8 = BITS == 8;  // FP8 cache: no slots, no residual, no Key metadata
    const int slot = kF8 ? 0 : a.slot_ids[s];
    const bool bad = slot < 0 || slot >= V.max_seqs || P < 0;
    const bool raw_chunk = a.k_chunk != nullptr;
    if (wg == 0 && wave == 0) {  // device-side errors of this sequence, reported once
        uint32_t e = (!kF8 && (slot < 0 || slot >= V.max_seqs) ? KIVI_DEVERR_SLOT : 0u) |
                     (P < 0 ? KIVI_DEVERR_LENGTH : 0u);
        if (nq < 0 || nq > a.max_q_len || (!raw_chunk && !bad && nq > P)) e |= KIVI_DEVERR_QUERY;
        if (!bad && (long long)P + (raw_chunk ? max(nq, 0) : 0) > (long long)a.bt_stride * V.Bk)
            e |= KIVI_DEVERR_LENGTH;
        if (e != 0 && lane == 0) report_error(V.status, e);
    }
    if (bad) P = 0;
    const int T = bad ? 0 : P + (raw_chunk ? nq : 0);  // tokens the rows attend over
    const int nrows = max(nq, 0) * g;
    const int row0_wg = wg * kRowsWg;
    if (row0_wg >= nrows) return;  // no rows for this work group (uniform)
    const int R = V.R;
    // quantised in the cache (the whole sequence in an FP8 cache)
    const int TK = kF8 ? P : R * (P / R), TV = kF8 ? P : value_boundary(V, P);

    // ---- this lane's row: column l % 32 of the wave's 32 rows ----
    const int half = lane >> 5, col = lane & 31;
    const int row = row0_wg + kRowsWave * wave + col;
    const bool row_ok = row < nrows && T > 0;
    const int qi = row_ok ? row / g : 0, qh = row_ok ? row % g : 0;
    const int my_pos = T - nq + qi;
    const int my_last = row_ok ? (a.causal ? min(my_pos, T - 1) : T - 1) : -1;
    // extents: the work group's last visible token, the wave's smallest
    int wave_min = row_ok ? my_last : 0x7fffffff, wave_max = my_last;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        wave_min = min(wave_min, __shfl_xor(wave_min, d));
        wave_max = max(wave_max, __shfl_xor(wave_max, d));
    }
    wave_min = __builtin_amdgcn_readfirstlane(wave_min);
    wave_max = __builtin_amdgcn_readfirstlane(wave_max);
    __shared__ int wg_max_sh[kPWaves];
    if (lane == 0) wg_max_sh[wave] = wave_max;
    __syncthreads();
    int wg_max = wg_max_sh[0];
#pragma unroll
    for (int w = 1; w < kPWaves; ++w) wg_max = max(wg_max, wg_max_sh[w]);
    const int n_tiles = wg_max >= 0 ? (wg_max + kTileTok) / kTileTok : 0;

    // ---- query operand: lane (col, half) holds q[row][16 ks + 8 half .. + 7] ----
    // FP8: Keys enter as value * 2^-8, so the Key scale times 2^8 joins the softmax scale
    const float xs = kF8 ? a.scale_log2 * a.k_scale[a.per_head ? h : 0] * 256.0f : a.scale_log2;
    const float sgn = xs < 0.0f ? -1.0f : 1.0f;  // scores kept as sgn q.k
    // weight 2^(x - m), x = score * c2; a zero scale (uniform weights) is
    // taken as the smallest normal one, so that -inf * c2 stays -inf
    const float c2 = fmaxf(fabsf(xs), 1.17549435e-38f);
    h8 Qb[8];
    {
        const uint16_t* qrow = a.q + ((size_t)(q0 + qi) * HQ + h * g + qh) * kHeadDim + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const uint4 w = row_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks) : (uint4){0, 0, 0, 0};
            const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h2 p2;
                if constexpr (DT == kBF16) {
                    p2 = (h2){(_Float16)bf16_bits_to_f32((uint16_t)(w4[e] & 0xFFFFu)),
                              (_Float16)bf16_bits_to_f32((uint16_t)(w4[e] >> 16))};
                } else {
                    p2 = as_h2(w4[e]);
                }
                if (sgn < 0.0f) p2 = -p2;
                Qb[ks][2 * e] = p2[0];
                Qb[ks][2 * e + 1] = p2[1];
            }
        }
    }

    // ---- the thread's part of a tile: half pt of Key slot and of Value slot
    // L of sub-tile u. Key: channel runs r = 2 pt, 2 pt + 1 (channels
    // 32 r + 8 j .. + 7) of token m; Value: channel tiles t = 4 pt .. 4 pt + 3
    // (channels 16 t + m) of tokens 4 j .. 4 j + 3 ----
    const int pt = __builtin_amdgcn_readfirstlane(tid >> 8);       // per wave
    const int u = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // per wave
    const int L = lane, m = L & 15, j = L >> 4;
    const int32_t* bt = a.block_table + (size_t)s * a.bt_stride;
    const uint16_t* ringK = kF8 ? nullptr : V.k_ring + ((size_t)max(slot, 0) * H + h) * V.ring_elems;
    const uint16_t* ringV = kF8 ? nullptr : V.v_ring + ((size_t)max(slot, 0) * H + h) * V.ring_elems;
    // Pages per Key group (G / Bk) and the Key channels whose metadata one
    // page holds (128 Bk / G) are powers of two: G / Bk divides 128. Bk is a
    // multiple of 16, usually a power of two as well.
    const int gpb_lg = kF8 ? 0 : __builtin_ctz((unsigned)(V.G / V.Bk));
    const int nch_lg = __builtin_ctz((unsigned)kHeadDim) - gpb_lg, nch = 1 << nch_lg;
    const bool bk_pow2 = (V.Bk & (V.Bk - 1)) == 0;
    const int bk_lg = __builtin_ctz((unsigned)V.Bk);
    auto div_bk = [&](int p) { return bk_pow2 ? p >> bk_lg : p / V.Bk; };
    auto mod_bk = [&](int p) { return bk_pow2 ? p & (V.Bk - 1) : p % V.Bk; };
    uint32_t err = 0;                       // pages this thread could not read
    auto page_at = [&](int bi) -> int {     // page of table entry bi, -1 (noted) when the table has none
        const int blk = bi < a.bt_stride ? bt[bi] : -1;
        if (blk >= 0 && blk < V.num_blocks) return blk;
        err |= KIVI_DEVERR_PAGE;
        return -1;
    };
    auto page_of = [&](int p) -> int { return page_at(div_bk(p)); };  // page of position p
    // Key metadata of tile k, staged in LDS: thread (u, L) of the first 256
    // loads the (scale, zero) pairs of channels 2L, 2L + 1 of sub-tile u's
    // group (two 4-byte loads), two tiles ahead, and stores them after the
    // current tile's computation; the restore of that tile reads them after a
    // barrier.
    _Float16* const meta_lds = lds + 2 * kStageHalfs;
    auto issue_meta = [&](int k, uint32_t& ms, uint32_t& mz) {
        ms = mz = 0;
        if constexpr (kF8) return;
        const int p_sub = kTileTok * k + 16 * u;
        if (pt == 0 && k < n_tiles && p_sub < TK) {
            // group jg = p_sub / G; channel ch's pair sits on page jg G / Bk + ch / nch
            const int ch = 2 * L;
            const int blk = page_at(((div_bk(p_sub) >> gpb_lg) << gpb_lg) + (ch >> nch_lg));
            if (blk >= 0) {
                const uint8_t* mp = V.k_meta + ((size_t)blk * H + h) * V.k_meta_bytes + 2 * (ch & (nch - 1));
                ms = *reinterpret_cast<const uint32_t*>(mp);
                mz = *reinterpret_cast<const uint32_t*>(mp + 2 * nch);
            }
        }
    };
    auto store_meta = [&](int k, uint32_t ms, uint32_t mz) {
        if (kF8 || pt != 0) return;
        _Float16* mt = meta_lds + (k & 1) * kMetaHalfs + u * 2 * kHeadDim;
        *reinterpret_cast<uint32_t*>(mt + 2 * L) = ms;
        *reinterpret_cast<uint32_t*>(mt + kHeadDim + 2 * L) = mz;
    };
    // the thread's code words of a sub-tile whose tokens are quantised, and the
    // Value metadata of its 4 tokens for the groups of its channel tiles
    constexpr int KW = BITS / 2;                 // code words per half slot
    constexpr int NGP = NG == 1 ? 1 : NG / 2;    // Value groups per half slot
    auto load_slot_k = [&](int blk, int p_sub, SlotRegs<BITS, NGP>& x) {
        const uint8_t* base = V.k_codes + ((size_t)blk * H + h) * V.code_bytes +
                              (mod_bk(p_sub) / kTile) * TILE_BYTES + SLOT_BYTES * L + 4 * KW * pt;
        if constexpr (KW == 4) {
            const uint4 w = *reinterpret_cast<const uint4*>(base);
            x.k[0] = w.x; x.k[1] = w.y; x.k[2] = w.z; x.k[3] = w.w;
        } else if constexpr (KW == 2) {
            const uint2 w = *reinterpret_cast<const uint2*>(base);
            x.k[0] = w.x; x.k[1] = w.y;
        } else {
            x.k[0] = *reinterpret_cast<const uint32_t*>(base);
        }
    };
    auto load_slot_v = [&](int blk, int p_sub, SlotRegs<BITS, NGP>& x) {
        const uint8_t* base = V.v_codes + ((size_t)blk * H + h) * V.code_bytes +
                              (mod_bk(p_sub) / kTile) * TILE_BYTES + SLOT_BYTES * L + 4 * KW * pt;
        if constexpr (KW == 4) {
            const uint4 w = *reinterpret_cast<const uint4*>(base);
            x.v[0] = w.x; x.v[1] = w.y; x.v[2] = w.z; x.v[3] = w.w;
            return;  // no Value metadata in an FP8 cache
        } else if constexpr (KW == 2) {
            const uint2 w = *reinterpret_cast<const uint2*>(base);
            x.v[0] = w.x; x.v[1] = w.y;
        } else {
            x.v[0] = *reinterpret_cast<const uint32_t*>(base);
        }
        // (scale, zero) of tokens 4j .. 4j + 3: all of a token's groups are one
        // row of NG words; this half needs groups pt NG / 2 .. + NGP - 1
        const uint8_t* mb = V.v_meta + ((size_t)blk * H + h) * V.v_meta_bytes + (size_t)(mod_bk(p_sub) + 4 * j) * NG * 4;
        if constexpr (NG == 1) {
            const uint4 w = *reinterpret_cast<const uint4*>(mb);
            x.vm[0] = w.x; x.vm[1] = w.y; x.vm[2] = w.z; x.vm[3] = w.w;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint8_t* mr = mb + (size_t)r * NG * 4 + 4 * NGP * pt;
                if constexpr (NGP == 1) {
                    x.vm[r] = *reinterpret_cast<const uint32_t*>(mr);
                } else if constexpr (NGP == 2) {
                    const uint2 w = *reinterpret_cast<const uint2*>(mr);
                    x.vm[2 * r] = w.x; x.vm[2 * r + 1] = w.y;
                } else {
                    const uint4 w = *reinterpret_cast<const uint4*>(mr);
                    x.vm[4 * r] = w.x; x.vm[4 * r + 1] = w.y; x.vm[4 * r + 2] = w.z; x.vm[4 * r + 3] = w.w;
                }
            }
        }
    };

    // ---- restore into LDS ----
    // Keys of sub-tile u, token m, the thread's 2 channel runs, from codes, with
    // the tile's Key metadata (stage k & 1): hi = fp16(k), lo = fp16(k - hi),
    // k = code * scale + zero; t = code * scale + zero is formed in single
    // precision (the product is exact), and t - hi is exact before its
    // rounding to fp16
    auto store_k_codes = [&](_Float16* st, int k, const uint32_t* kw) {
        if constexpr (kF8) {  // exact values: no lo part (the products skip it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int off = (16 * u + m) * kKRow + 32 * (2 * pt + rr) + 8 * j;
                *reinterpret_cast<uint4*>(st + off) =
                    (uint4){e4m3_pair<false>(kw[2 * rr]), e4m3_pair<true>(kw[2 * rr]),
                            e4m3_pair<false>(kw[2 * rr + 1]), e4m3_pair<true>(kw[2 * rr + 1])};
            }
            return;
        }
        const _Float16* mt = meta_lds + (k & 1) * kMetaHalfs + u * 2 * kHeadDim;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * pt + rr;
            const uint4 sv = *reinterpret_cast<const uint4*>(mt + 32 * r + 8 * j);
            const uint4 zv = *reinterpret_cast<const uint4*>(mt + kHeadDim + 32 * r + 8 * j);
            const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w}, zw[4] = {zv.x, zv.y, zv.z, zv.w};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h2 c;
                if constexpr (BITS == 4) c = code_pair<4>(kw[rr], 4 * e);
                else c = code_pair<2>(kw[0], 2 * (e + 4 * rr));
                const h2 sc = as_h2(sw[e]), zc = as_h2(zw[e]);
                const h2 hi = __builtin_elementwise_fma(c, sc, zc);
                h2 lo;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float t = __builtin_fmaf((float)c[q], (float)sc[q], (float)zc[q]);
                    lo[q] = (_Float16)__builtin_fmaf((float)hi[q], -1.0f, t);
                }
                hw[e] = as_u32(hi);
                lw[e] = as_u32(lo);
            }
            const int off = (16 * u + m) * kKRow + 32 * r + 8 * j;
            *reinterpret_cast<uint4*>(st + off) = (uint4){hw[0], hw[1], hw[2], hw[3]};
            *reinterpret_cast<uint4*>(st + kKHalfs + off) = (uint4){lw[0], lw[1], lw[2], lw[3]};
        }
    };
    // fp16 pair of tokens (4j + 2k, 4j + 2k + 1) of channel 16 (4 pt + tt) + m,
    // from codes (tt = 0..3: the thread's tiles; every index below is a
    // compile-time constant, so the registers stay registers)
    auto v_from_codes = [&](const SlotRegs<BITS, NGP>& x, int tt, int k) -> h2 {
        h2 c;
        if constexpr (BITS == 4) c = code_pair<4>(x.v[tt >> 1], 4 * (2 * (tt & 1) + k));
        else c = code_pair<2>(x.v[0], 2 * (2 * tt + k));
        // the channel's group (Gv >= 16 > m), counted from this half's first
        const int gg = NG == 1 ? 0 : (tt * NG) / 8;
        const uint32_t w0 = x.vm[(2 * k) * NGP + gg], w1 = x.vm[(2 * k + 1) * NGP + gg];
        const h2 sc = as_h2(__builtin_amdgcn_perm(w1, w0, 0x05040100u));  // scales of the two tokens
        const h2 zc = as_h2(__builtin_amdgcn_perm(w1, w0, 0x07060302u));  // zero-points
        return __builtin_elementwise_fma(c, sc, zc);
    };
    auto store_v = [&](_Float16* st, int t, uint32_t lo, uint32_t hi) {
        *reinterpret_cast<uint2*>(st + kVOff + (16 * t + m) * kVRow + 16 * u + v_pos(j)) = (uint2){lo, hi};
    };

    // A tile whose 64 tokens have quantised Keys and Values, restored from
    // registers loaded before the previous tile's computation.
    auto fill_pure = [&](_Float16* st, int k, const SlotRegs<BITS, NGP>& x) {
        store_k_codes(st, k, x.k);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            if constexpr (kF8)  // byte r of the word: token 4j + r of channel 16 (4 pt + tt) + m
                store_v(st, 4 * pt + tt, e4m3_pair<false>(x.v[tt]), e4m3_pair<true>(x.v[tt]));
            else
                store_v(st, 4 * pt + tt, as_u32(v_from_codes(x, tt, 0)), as_u32(v_from_codes(x, tt, 1)));
        }
    };
    // Any tile: per sub-tile (Keys; TK is a multiple of 16) and per token
    // (Values) from codes, the residual ring, the raw chunk, or zeros past the
    // sequence. Synchronous; only the last tiles of a sequence take it.
    auto fill_any = [&](_Float16* st, int k) {
        const int t0 = kTileTok * k;
        const int p_sub = t0 + 16 * u;
        if constexpr (kF8) {
            // bytes of tokens at or past T were never written and may hold an
            // E4M3 NaN (0 times NaN is NaN): they become zeros
            const int blk = p_sub < T ? page_of(p_sub) : -1;
            SlotRegs<BITS, NGP> x;
#pragma unroll
            for (int q = 0; q < KW; ++q) x.k[q] = x.v[q] = 0;
            if (blk >= 0) {
                load_slot_k(blk, p_sub, x);
                load_slot_v(blk, p_sub, x);
            }
            if (p_sub + m >= T) {
#pragma unroll
                for (int q = 0; q < KW; ++q) x.k[q] = 0;
            }
            uint32_t keep = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (p_sub + 4 * j + r < T) keep |= 0xFFu << (8 * r);
#pragma unroll
            for (int q = 0; q < KW; ++q) x.v[q] &= keep;
            fill_pure(st, k, x);
            return;
        }
        const int blk = (p_sub < TV || p_sub < TK) ? page_of(p_sub) : -1;
        SlotRegs<BITS, NGP> x;
#pragma unroll
        for (int q = 0; q < KW; ++q) x.k[q] = x.v[q] = 0;
#pragma unroll
        for (int q = 0; q < 4 * NGP; ++q) x.vm[q] = 0;
        if (blk >= 0 && p_sub < TK) load_slot_k(blk, p_sub, x);
        if (blk >= 0 && p_sub < TV) load_slot_v(blk, p_sub, x);
        // Keys: token p = p_sub + m (full-precision values: hi = value, lo = 0)
        const int p = p_sub + m;
        if (p_sub < TK) {
            store_k_codes(st, k, x.k);
        } else {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int r = 2 * pt + rr;
                uint4 w = {0, 0, 0, 0};
                if (p < T) {
                    const uint16_t* src = p < P ? ringK + (size_t)(p % R) * kHeadDim
                                                : a.k_chunk + ((size_t)(q0 + p - P) * H + h) * kHeadDim;
                    w = *reinterpret_cast<const uint4*>(src + 32 * r + 8 * j);
                }
                if constexpr (DT == kBF16) {
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
                    uint32_t o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = as_u32((h2){(_Float16)bf16_bits_to_f32((uint16_t)(ws[e] & 0xFFFFu)),
                                           (_Float16)bf16_bits_to_f32((uint16_t)(ws[e] >> 16))});
                    w = (uint4){o[0], o[1], o[2], o[3]};
                }
                const int off = (16 * u + m) * kKRow + 32 * r + 8 * j;
                *reinterpret_cast<uint4*>(st + off) = w;
                *reinterpret_cast<uint4*>(st + kKHalfs + off) = (uint4){0, 0, 0, 0};
            }
        }
        // Values: tokens pv .. pv + 3, one quad of the ring (R is a multiple of 16)
        const int pv = p_sub + 4 * j;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 4 * pt + tt;
            const int ch = 16 * t + m;
            uint32_t code_w[2] = {0, 0};
            if (pv < TV) {
                code_w[0] = as_u32(v_from_codes(x, tt, 0));
                code_w[1] = as_u32(v_from_codes(x, tt, 1));
            }
            uint2 ring_w = {0, 0};
            if (pv + 3 >= TV && pv < min(T, P)) ring_w = *reinterpret_cast<const uint2*>(ringV + vring_index(R, pv, ch));
            uint16_t val[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pr = pv + r;
                uint16_t bits = 0;
                if (pr < TV) {
                    bits = (uint16_t)(code_w[r >> 1] >> (16 * (r & 1)));
                } else if (pr < min(T, P)) {
                    bits = (uint16_t)((r < 2 ? ring_w.x : ring_w.y) >> (16 * (r & 1)));
                    if constexpr (DT == kBF16) bits = __builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(bits));
                } else if (pr < T) {
                    bits = a.v_chunk[((size_t)(q0 + pr - P) * H + h) * kHeadDim + ch];
                    if constexpr (DT == kBF16) bits = __builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(bits));
                }
                val[r] = bits;
            }
            store_v(st, t, (uint32_t)val[0] | ((uint32_t)val[1] << 16), (uint32_t)val[2] | ((uint32_t)val[3] << 16));
        }
    };
    auto pure = [&](int k) -> bool { return kTileTok * (k + 1) <= TV && kTileTok * (k + 1) <= TK; };
    // loads of a pure tile's codes
    auto issue_pure = [&](int k, SlotRegs<BITS, NGP>& x) {
        const int p_sub = kTileTok * k + 16 * u;
        const int blk = page_of(p_sub);
        load_slot_k(max(blk, 0), p_sub, x);
        load_slot_v(max(blk, 0), p_sub, x);
        if (blk < 0) {  // no page: its slot restores to zero values
#pragma unroll
            for (int q = 0; q < 4 * NGP; ++q) x.vm[q] = 0;
            if constexpr (kF8) {
#pragma unroll
                for (int q = 0; q < KW; ++q) x.k[q] = x.v[q] = 0;
            }
        }
    };

    // ---- per-wave state: O^T[channel][row] in 4 blocks of 32 channels ----
    f16v O[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) O[cb] = (f16v){};
    float m_run = -INFINITY, l_acc = 0.0f;

    // ---- per tile and wave (the lane holds row col; tokens
    // t0 + 32 b + 8 (v / 4) + 4 half + v % 4 of block b) ----
    // Scores S^T[token][row] of the tile's two 32-token blocks, Keys as hi + lo
    // (the two blocks' accumulations alternate, so that no product waits for
    // the one before it).
    auto qk = [&](const _Float16* st, f16v& S0, f16v& S1) {
        S0 = (f16v){};
        S1 = (f16v){};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int o0 = col * kKRow + 16 * ks + 8 * half, o1 = o0 + 32 * kKRow;
            const h8 a0 = *reinterpret_cast<const h8*>(st + o0), a1 = *reinterpret_cast<const h8*>(st + o1);
            S0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, Qb[ks], S0, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, Qb[ks], S1, 0, 0, 0);
            if constexpr (!kF8) {  // FP8 Keys are exact in fp16
                const h8 b0 = *reinterpret_cast<const h8*>(st + kKHalfs + o0);
                const h8 b1 = *reinterpret_cast<const h8*>(st + kKHalfs + o1);
                S0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, Qb[ks], S0, 0, 0, 0);
                S1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, Qb[ks], S1, 0, 0, 0);
            }
        }
    };
    // Tile k's scores (from stage cur) interleaved with the restore of pure
    // tile k + 1 into stage nxt: 8 steps, one per 16-channel k-step of the
    // products; step i issues the k-step's 4 products (operands read one step
    // ahead), restores pair e = i % 4 of Key channel run 2 pt + i / 4 and
    // Value pair i % 2 of channel tile 4 pt + i / 2, and ends at a scheduling
    // barrier, so that the products and the vector work stay mixed.
    auto qk_fill = [&](const _Float16* st, f16v& S0, f16v& S1, _Float16* nst, int kn,
                       const SlotRegs<BITS, NGP>& x) {
        S0 = (f16v){};
        S1 = (f16v){};
        const _Float16* mt = meta_lds + (kn & 1) * kMetaHalfs + u * 2 * kHeadDim;
        uint32_t sw[2][4], zw[2][4];
        if constexpr (!kF8) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const uint4 sv = *reinterpret_cast<const uint4*>(mt + 32 * (2 * pt + rr) + 8 * j);
                const uint4 zv = *reinterpret_cast<const uint4*>(mt + kHeadDim + 32 * (2 * pt + rr) + 8 * j);
                sw[rr][0] = sv.x; sw[rr][1] = sv.y; sw[rr][2] = sv.z; sw[rr][3] = sv.w;
                zw[rr][0] = zv.x; zw[rr][1] = zv.y; zw[rr][2] = zv.z; zw[rr][3] = zv.w;
            }
        }
        auto operands = [&](int ks, h8& a0, h8& a1, h8& b0, h8& b1) {
            const int o0 = col * kKRow + 16 * ks + 8 * half, o1 = o0 + 32 * kKRow;
            a0 = *reinterpret_cast<const h8*>(st + o0);
            a1 = *reinterpret_cast<const h8*>(st + o1);
            if constexpr (!kF8) {
                b0 = *reinterpret_cast<const h8*>(st + kKHalfs + o0);
                b1 = *reinterpret_cast<const h8*>(st + kKHalfs + o1);
            }
        };
        h8 A0, A1, B0, B1;
        operands(0, A0, A1, B0, B1);
        uint32_t hw[4], lw[4], vv[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const h8 a0 = A0, a1 = A1, b0 = B0, b1 = B1;
            if (i < 7) operands(i + 1, A0, A1, B0, B1);
            S0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, Qb[i], S0, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, Qb[i], S1, 0, 0, 0);
            if constexpr (!kF8) {
                S0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, Qb[i], S0, 0, 0, 0);
                S1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, Qb[i], S1, 0, 0, 0);
            }
            // Keys: pair e of channel run r (as store_k_codes)
            const int rr = i >> 2, e = i & 3, r = 2 * pt + rr;
            if constexpr (kF8) {
                if (e == 3) {
                    const int off = (16 * u + m) * kKRow + 32 * r + 8 * j;
                    *reinterpret_cast<uint4*>(nst + off) =
                        (uint4){e4m3_pair<false>(x.k[2 * rr]), e4m3_pair<true>(x.k[2 * rr]),
                                e4m3_pair<false>(x.k[2 * rr + 1]), e4m3_pair<true>(x.k[2 * rr + 1])};
                }
            } else {
                h2 c;
                if constexpr (BITS == 4) c = code_pair<4>(x.k[rr], 4 * e);
                else c = code_pair<2>(x.k[0], 2 * (e + 4 * rr));
                const h2 sc = as_h2(sw[rr][e]), zc = as_h2(zw[rr][e]);
                const h2 hi = __builtin_elementwise_fma(c, sc, zc);
                h2 lo;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float t = __builtin_fmaf((float)c[q], (float)sc[q], (float)zc[q]);
                    lo[q] = (_Float16)__builtin_fmaf((float)hi[q], -1.0f, t);
                }
                hw[e] = as_u32(hi);
                lw[e] = as_u32(lo);
                if (e == 3) {
                    const int off = (16 * u + m) * kKRow + 32 * r + 8 * j;
                    *reinterpret_cast<uint4*>(nst + off) = (uint4){hw[0], hw[1], hw[2], hw[3]};
                    *reinterpret_cast<uint4*>(nst + kKHalfs + off) = (uint4){lw[0], lw[1], lw[2], lw[3]};
                }
            }
            // Values: pair i % 2 of channel tile 4 pt + i / 2
            const int tt = i >> 1, kv = i & 1;
            if constexpr (kF8) {
                if (kv == 1) store_v(nst, 4 * pt + tt, e4m3_pair<false>(x.v[tt]), e4m3_pair<true>(x.v[tt]));
            } else {
                vv[kv] = as_u32(v_from_codes(x, tt, kv));
                if (kv == 1) store_v(nst, 4 * pt + tt, vv[0], vv[1]);
            }
#pragma unroll
            for (int q = 0; q < (kF8 ? 2 : 4); ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, kF8 ? 2 : 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Online softmax, per tile: scores of tokens past the row's last become
    // -inf (only on tiles some row of the wave does not see whole; c2 > 0, so
    // their weights are 0); the tile's maximum (log2 units) moves the running
    // maximum only when it passes it by kLazy.
    auto tile_max = [&](f16v& S0, f16v& S1, int t0) {
        if (t0 + kTileTok - 1 > wave_min) {  // uniform
            const int lim = my_last - t0 - 4 * half;  // the row sees v with 8 (v / 4) + v % 4 <= lim
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if (8 * (v >> 2) + (v & 3) > lim) S0[v] = -INFINITY;
                if (32 + 8 * (v >> 2) + (v & 3) > lim) S1[v] = -INFINITY;
            }
        }
        float mx = fmaxf(S0[0], S1[0]);
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(S0[v], S1[v]));
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float mxl = mx * c2;  // -inf when the row sees none of the tile
        if (__builtin_amdgcn_ballot_w64(mxl > m_run + kLazy) != 0) {  // rare: move the running max
            const float mnew = fmaxf(m_run, mxl);
            const float f = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mnew);
            l_acc *= f;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) O[cb] *= f;
            m_run = mnew;
        }
    };
    // Weights 2^(score c2 - m) of one block into two fp16 B operands (k-steps
    // 2 b, 2 b + 1), rounded to nearest; their sum joins l.
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    auto weights = [&](const f16v& S, h8* Pb) {
        const float mneg = m_run == -INFINITY ? 0.0f : -m_run;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 8 * kk + 2 * e;
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[v], c2, mneg));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[v + 1], c2, mneg));
                const h2 pp = {(_Float16)p0, (_Float16)p1};  // round to nearest (one v_cvt_pk_f16_f32)
                l_acc = __builtin_amdgcn_fdot2(pp, one, l_acc, false);
                Pb[kk][2 * e] = pp[0];
                Pb[kk][2 * e + 1] = pp[1];
            }
    };
    // O^T[128][32] += V^T[128][32 tokens of block b] P^T
    auto pv = [&](const _Float16* vst, int b, const h8* Pb) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const h8 av = *reinterpret_cast<const h8*>(vst + (32 * cb + col) * kVRow + 16 * (2 * b + kk) + 8 * half);
                O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, Pb[kk], O[cb], 0, 0, 0);
            }
    };

    // ---- the tile loop: two LDS stages, one barrier per tile ----
    // Vector work issued between a wave's own matrix products overlaps them;
    // the matrix products of one wave and the vector work of the other wave on
    // the same SIMD hardly do (measured on MI355X: 903 cycles for both against
    // 527 + 408 apart; 553 against 527 for the same work interleaved in one
    // wave). So every wave interleaves: iteration k
    //   (1) tile k's score products with the restore of tile k + 1 (from codes
    //       loaded in the iteration before), one block of straight-line code;
    //   (2) the loads of tile k + 2's codes and Key metadata;
    //   (3) the tile's maximum (and, rarely, a rescale);
    //   (4) block 0's weights, block 0's P V products interleaved with block
    //       1's weights, block 1's P V products;
    // then the metadata store and a barrier. A tile that is not pure is
    // restored after the computation.
    if (n_tiles > 0) {
        SlotRegs<BITS, (NG == 1 ? 1 : NG / 2)> nx;
        uint32_t ms, mz;
        issue_meta(0, ms, mz);
        store_meta(0, ms, mz);
        issue_meta(1, ms, mz);
        store_meta(1, ms, mz);
        __syncthreads();
        if (pure(0)) {
            issue_pure(0, nx);
            fill_pure(lds, 0, nx);
        } else {
            fill_any(lds, 0);
        }
        if (n_tiles > 1 && pure(1)) issue_pure(1, nx);
        __syncthreads();
        for (int k = 0; k < n_tiles; ++k) {
            const _Float16* cur = lds + (k & 1) * kStageHalfs;
            _Float16* nxt = lds + ((k + 1) & 1) * kStageHalfs;
            const bool more = k + 1 < n_tiles;
            const bool nxt_pure = more && pure(k + 1);
            f16v S0, S1;
            if (nxt_pure) {
                qk_fill(cur, S0, S1, nxt, k + 1, nx);
            } else {
                qk(cur, S0, S1);
            }
            if (k + 2 < n_tiles && pure(k + 2)) issue_pure(k + 2, nx);
            issue_meta(k + 2, ms, mz);
            tile_max(S0, S1, kTileTok * k);
            const _Float16* vst = cur + kVOff;
            h8 P0[2], P1[2];
            weights(S0, P0);
            pv(vst, 0, P0);
            weights(S1, P1);
            pv(vst, 1, P1);
            // block 0's weights with the Value reads; block 0's products with
            // block 1's weights; block 1's products
            __builtin_amdgcn_sched_group_barrier(0x002, 40, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 16, 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
            if (more && !nxt_pure) fill_any(nxt, k + 1);
            store_meta(k + 2, ms, mz);
            __syncthreads();
        }
    }
    if (err != 0) report_error(V.status, err);

    // ---- output: lane (col, half) holds channels 32 cb + 8 (v / 4) + 4 half + v % 4 ----
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_acc), __float_as_uint(l_acc), false, false);
        l_acc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (!(row < nrows)) return;
    // FP8: the Values entered as value * 2^-8
    const float vsc = kF8 ? a.v_scale[a.per_head ? h : 0] * 256.0f : 1.0f;
    const float inv = l_acc > 0.0f ? vsc / l_acc : 0.0f;
    uint16_t* orow = a.out + ((size_t)(q0 + qi) * HQ + h * g + qh) * kHeadDim;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int ch = 32 * cb + 8 * b + 4 * half;
            const uint32_t w0 =
                (uint32_t)from_f32<DT>(O[cb][4 * b] * inv) | ((uint32_t)from_f32<DT>(O[cb][4 * b + 1] * inv) << 16);
            const uint32_t w1 = (uint32_t)from_f32<DT>(O[cb][4 * b + 2] * inv) |
                                ((uint32_t)from_f32<DT>(O[cb][4 * b + 3] * inv) << 16);
            *reinterpret_cast<uint2*>(orow + ch) = (uint2){w0, w1};
        }
}

template <int BITS, int DT>
void launch_pf(const PrefillArgs& a, int ng, dim3 grid, hipStream_t st) {
    dim3 block(kPThreads);
    if constexpr (BITS == 8) {  // no Value groups in an FP8 cache
        hipLaunchKernelGGL((prefill_kernel<8, DT, 1>), grid, block, kPrefillLds, st, a);
    } else {
        switch (ng) {
            case 1: hipLaunchKernelGGL((prefill_kernel<BITS, DT, 1>), grid, block, kPrefillLds, st, a); break;
            case 2: hipLaunchKernelGGL((prefill_kernel<BITS, DT, 2>), grid, block, kPrefillLds, st, a); break;
            case 4: hipLaunchKernelGGL((prefill_kernel<BITS, DT, 4>), grid, block, kPrefillLds, st, a); break;
            default: hipLaunchKernelGGL((prefill_kernel<BITS, DT, 8>), grid, block, kPrefillLds, st, a); break;
        }
    }
}

}  // namespace

int launch_prefill(const CacheView& v, int num_seqs, int num_q_heads, const void* q, const int32_t* cu_q,
                   int max_q_len, const int32_t* slot_ids, const int32_t* seq_lens, int max_seq_len,
                   const void* k_chunk, const void* v_chunk, const int32_t* block_table, int bt_stride,
                   float softmax_scale, int causal, void* out, void* stream) {
    (void)max_seq_len;
    PrefillArgs a;
    a.v = v;
    a.q = static_cast<const uint16_t*>(q);
    a.k_chunk = static_cast<const uint16_t*>(k_chunk);
    a.v_chunk = static_cast<const uint16_t*>(v_chunk);
    a.cu_q = cu_q;
    a.slot_ids = slot_ids;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.num_q_heads = num_q_heads;
    a.gqa = num_q_heads / v.H;
    a.scale_log2 = softmax_scale * kLog2e;
    a.causal = causal;
    a.max_q_len = max_q_len;
    const long long rows = (long long)max_q_len * a.gqa;
    a.wg_per_sh = (int)((rows + kRowsWg - 1) / kRowsWg);
    a.out = static_cast<uint16_t*>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int ng = kHeadDim / v.Gv;
    dim3 grid((unsigned)((size_t)num_seqs * v.H * a.wg_per_sh));
    if (v.bits == 4) {
        if (v.dtype == kF16) launch_pf<4, kF16>(a, ng, grid, st);
        else launch_pf<4, kBF16>(a, ng, grid, st);
    } else {
        if (v.dtype == kF16) launch_pf<2, kF16>(a, ng, grid, st);
        else launch_pf<2, kBF16>(a, ng, grid, st);
    }
    return (int)hipGetLastError();
}

int launch_fp8_prefill(const CacheView& v, int per_head, int num_seqs, int num_q_heads, const void* q,
                       const int32_t* cu_q, int max_q_len, const int32_t* seq_lens, const float* k_scale,
                       const float* v_scale, const int32_t* block_table, int bt_stride, float softmax_scale,
                       int causal, void* out, void* stream) {
    PrefillArgs a{};
    a.v = v;
    a.q = static_cast<const uint16_t*>(q);
    a.k_chunk = nullptr;
    a.v_chunk = nullptr;
    a.cu_q = cu_q;
    a.slot_ids = nullptr;  // an FP8 cache has no residual slots
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.num_q_heads = num_q_heads;
    a.gqa = num_q_heads / v.H;
    a.scale_log2 = softmax_scale * kLog2e;
    a.causal = causal;
    a.max_q_len = max_q_len;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.per_head = per_head;
    const long long rows = (long long)max_q_len * a.gqa;
    a.wg_per_sh = (int)((rows + kRowsWg - 1) / kRowsWg);
    a.out = static_cast<uint16_t*>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    dim3 grid((unsigned)((size_t)num_seqs * v.H * a.wg_per_sh));
    if (v.dtype == kF16) launch_pf<8, kF16>(a, 1, grid, st);
    else launch_pf<8, kBF16>(a, 1, grid, st);
    return (int)hipGetLastError();
}

}  // namespace kivi
