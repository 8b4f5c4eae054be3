// Append / quantise-on-flush of one (sequence, KV head) ("4.4 KV Cache 量化",
// sections 3.1-3.2; "给 KV cache 减肥", section 3.1: quantise before writing).
//
// For a sequence with T0 tokens that receives n new rows (T1 = T0 + n) the
// work group computes the final state directly, which equals n single-token
// appends:
//   * Key: tokens [R*floor(T0/R), R*floor(T1/R)) are quantised per channel,
//     G tokens per group (the residual reached R tokens that many times);
//   * Value: tokens [TV(T0), TV(T1)) leave the residual and are quantised
//     per token, Gv channels per group; TV(T) = max(0, T-R) for the sliding
//     window, R*floor(T/R) when Values flush with the Keys;
//   * the residual ring receives the new rows that stay full precision.
// Phase A (all quantisation) reads the old ring and the new rows; a barrier
// separates it from phase B (ring writes), which may overwrite ring slots
// phase A read. Distinct sequences touch disjoint pages and ring slots.
//
// Used by the append kernel (256 threads per work group) and by the fused
// decode step (the decode work group's 512 threads, before it attends).
#pragma once

#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

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
    int mode;  // 0: phases A and B; 1: phase A only (split over parts); 2: phase B only
};

// Shared scratch of append_body for NT threads.
template <int NT>
struct AppendShared {
    float mn[NT / 128][kHeadDim], mx[NT / 128][kHeadDim];
    float S[kHeadDim], Z[kHeadDim];
    uint8_t codes[kMaxG * kHeadDim];
    float v[NT / 64][4][kHeadDim];
    float vp[NT / 64][4][8][2];
};

// The append of one (sequence, KV head) by NT threads (a multiple of 128):
// rows [row0, row0 + n) of the input arrays are the sequence's new tokens.
// Part `part` of `nparts` does every nparts-th Key group and Value quad of
// phase A (mode 1), or everything (mode 0, nparts = 1); mode 2 does phase B
// only. Every thread of the work group calls it (it holds barriers); the
// shared scratch may alias memory the caller uses afterwards.
template <int BITS, int DT, int NT>
__device__ __forceinline__ void append_body(const AppendArgs& a, int s, int h, int row0, int n, int tid, int part,
                                            int nparts, AppendShared<NT>& sm) {
    static_assert(NT % 128 == 0, "two or more channel sweeps");
    constexpr int NQ = NT / 128;  // threads per channel in the Key flush
    constexpr int NW = NT / 64;   // waves
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;  // one 16-token sub-tile
    constexpr int SLOT_BYTES = 4 * BITS;                     // bytes per lane slot
    const CacheView& V = a.v;
    const int H = V.H;

    const int slot = a.slot_ids[s];
    const int T0 = a.seq_lens_before[s];
    if (n == 0) return;
    if (slot < 0 || slot >= V.max_seqs || T0 < 0 || n < 0) {  // skipped, and reported
        if (tid == 0)
            report_error(V.status, (slot < 0 || slot >= V.max_seqs ? KIVI_DEVERR_SLOT : 0u) |
                                       (T0 < 0 || n < 0 ? KIVI_DEVERR_LENGTH : 0u));
        return;
    }
    const int T1 = T0 + n;
    const int R = V.R, G = V.G, Gv = V.Gv, Bk = V.Bk;
    const int TK0 = R * (T0 / R), TK1 = R * (T1 / R);
    const int TV0 = value_boundary(V, T0), TV1 = value_boundary(V, T1);
    const int32_t* bt = a.block_table + (size_t)s * a.bt_stride;
    const int bt_len = a.bt_stride;

    uint16_t* ringK = V.k_ring + ((size_t)slot * H + h) * V.ring_elems;  // [R][128]
    uint16_t* ringV = V.v_ring + ((size_t)slot * H + h) * V.ring_elems;  // [R/4][128][4]
    const size_t in_stride = (size_t)H * kHeadDim;
    const uint16_t* inK = a.k_new + (size_t)row0 * in_stride + (size_t)h * kHeadDim;
    const uint16_t* inV = a.v_new + (size_t)row0 * in_stride + (size_t)h * kHeadDim;

    // page of position p, or -1 (reported) when the table has none for it
    auto page_of = [&](int p) -> int {
        int bi = p / Bk;
        if (bi >= bt_len) {
            report_error(V.status, KIVI_DEVERR_LENGTH);
            return -1;
        }
        int blk = bt[bi];
        if (blk >= 0 && blk < V.num_blocks) return blk;
        report_error(V.status, KIVI_DEVERR_PAGE);
        return -1;
    };
    auto kval = [&](int p, int c) -> float {
        uint16_t u = p < T0 ? ringK[(size_t)(p % R) * kHeadDim + c] : inK[(size_t)(p - T0) * in_stride + c];
        return canon(to_f32<DT>(u));
    };
    auto vval = [&](int p, int c) -> float {
        uint16_t u = p < T0 ? ringV[vring_index(R, p, c)] : inV[(size_t)(p - T0) * in_stride + c];
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

    auto& sm_min = sm.mn;
    auto& sm_max = sm.mx;
    auto& sm_S = sm.S;
    auto& sm_Z = sm.Z;
    auto& sm_codes = sm.codes;
    auto& sm_v = sm.v;
    auto& sm_vp = sm.vp;

    if (a.mode != 2) {
    // ---------------- phase A1: Key flush, one group at a time ----------------
    {
        const int c = tid & (kHeadDim - 1);
        const int half = tid >> 7;  // which 1/NQ of the group's tokens
        const int nch = kHeadDim * Bk / G;  // channels per K-meta page slot
        for (int j = TK0 / G + part; j < TK1 / G; j += nparts) {
            const int base = j * G;
            const int lo = half * (G / NQ), hi = lo + G / NQ;
            float mn = INFINITY, mx = -INFINITY;
            // unrolled so that several tokens' loads are in flight at once
#pragma unroll 8
            for (int i = lo; i < hi; ++i) {
                float x = kval(base + i, c);
                mn = fminf(mn, x);
                mx = fmaxf(mx, x);
            }
            sm_min[half][c] = mn;
            sm_max[half][c] = mx;
            __syncthreads();
            if (half == 0) {
                mn = sm_min[0][c];
                mx = sm_max[0][c];
#pragma unroll
                for (int qq = 1; qq < NQ; ++qq) {
                    mn = fminf(mn, sm_min[qq][c]);
                    mx = fmaxf(mx, sm_max[qq][c]);
                }
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
#pragma unroll 8
                for (int i = lo; i < hi; ++i)
                    sm_codes[i * kHeadDim + c] = (uint8_t)group_code(kval(base + i, c), S, Z, QMAX);
            }
            __syncthreads();
            // pack the group's code words (every word of these tokens is written)
            constexpr int WPT = kHeadDim * BITS / 32;  // 32-bit words per token
            for (int q = tid; q < G * WPT; q += NT) {
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
        const int rounds = TV1 > TV0 ? (q_hi - q_lo + NW - 1) / NW : 0;
        for (int rd = part; rd < rounds; rd += nparts) {
            const int qd = q_lo + rd * NW + wave;
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
            if (nv > 0 && tid < kHeadDim) ringV[vring_index(R, T0, tid)] = row_v;
            return;
        }
        // Phase B is split over the parts like phase A (mode 2 with nparts
        // parts; mode 0 is a single part). Loops are unrolled so that several
        // loads are in flight per thread.
        const int tq = tid + NT * part, step = NT * nparts;
        // Key ring: token-major rows, 16-byte chunks
#pragma unroll 4
        for (int q = tq; q < nk * 16; q += step) {
            const int p = k_first + q / 16, ch = (q % 16) * 8;
            const uint4 val = *reinterpret_cast<const uint4*>(inK + (size_t)(p - T0) * in_stride + ch);
            *reinterpret_cast<uint4*>(ringK + (size_t)(p % R) * kHeadDim + ch) = val;
        }
        // Value ring: quads of [128 channels][4 tokens]; a quad that the new
        // rows fill whole is one 8-byte store per channel, the (at most two)
        // partial quads at the ends take single elements
        const int qa = (v_first + 3) / 4, qb = T1 / 4;  // whole quads [4 qa, 4 qb)
        if (qb > qa) {
#pragma unroll 4
            for (int q = tq; q < (qb - qa) * kHeadDim; q += step) {
                const int p0 = 4 * (qa + q / kHeadDim), ch = q % kHeadDim;
                const uint16_t* src = inV + (size_t)(p0 - T0) * in_stride + ch;
                const uint32_t v0 = src[0], v1 = src[in_stride], v2 = src[2 * in_stride], v3 = src[3 * in_stride];
                *reinterpret_cast<uint2*>(ringV + vring_index(R, p0, ch)) = (uint2){v0 | (v1 << 16), v2 | (v3 << 16)};
            }
        }
        for (int q = tq; q < nv * kHeadDim; q += step) {
            const int p = v_first + q / kHeadDim, ch = q % kHeadDim;
            if (qb > qa && p >= 4 * qa && p < 4 * qb) continue;  // written as a whole quad
            ringV[vring_index(R, p, ch)] = inV[(size_t)(p - T0) * in_stride + ch];
        }
    }
}


}  // namespace kivi

namespace kivi {

// ---------------------------------------------------------------------------
// One-token append of one (sequence, KV head) done by single waves, with no
// work-group barrier, so it can run beside other waves' attention (the fused
// decode step). The result is that of append_body with n = 1:
//   append_token_value_wave: the Value token leaving the window (quantised
//     per Gv-channel group) and the new token's residual writes; one wave,
//     channels 2 lane and 2 lane + 1.
//   append_token_key_wave: when the Key residual fills, its R tokens' Key
//     groups for channels [64 half, 64 half + 64); two waves (half 0 and 1).
// The caller waits for the stores to complete and synchronises before any
// wave reads what these write.
// ---------------------------------------------------------------------------
struct TokenAppend {
    const CacheView* V;
    int H, h, slot, T0, R, G, Gv, Bk;
    const int32_t* bt;
    int bt_len;
    uint16_t* ringK;
    uint16_t* ringV;
    const uint16_t* inK;
    const uint16_t* inV;
    bool ok;
    // page of position p, or -1 (reported) when the table has none for it
    __device__ int page_of(int p) const {
        const int bi = p / Bk;
        if (bi >= bt_len) {
            report_error(V->status, KIVI_DEVERR_LENGTH);
            return -1;
        }
        const int blk = bt[bi];
        if (blk >= 0 && blk < V->num_blocks) return blk;
        report_error(V->status, KIVI_DEVERR_PAGE);
        return -1;
    }
};

__device__ __forceinline__ TokenAppend token_append_ctx(const AppendArgs& a, int s, int h) {
    TokenAppend t;
    const CacheView& V = a.v;
    t.V = &a.v;
    t.H = V.H;
    t.h = h;
    t.slot = a.slot_ids[s];
    t.T0 = a.seq_lens_before[s];
    t.ok = !(t.slot < 0 || t.slot >= V.max_seqs || t.T0 < 0);
    t.R = V.R;
    t.G = V.G;
    t.Gv = V.Gv;
    t.Bk = V.Bk;
    t.bt = a.block_table + (size_t)s * a.bt_stride;
    t.bt_len = a.bt_stride;
    const int sl = t.ok ? t.slot : 0;
    t.ringK = V.k_ring + ((size_t)sl * t.H + h) * V.ring_elems;
    t.ringV = V.v_ring + ((size_t)sl * t.H + h) * V.ring_elems;
    t.inK = a.k_new + ((size_t)s * t.H + h) * kHeadDim;  // row s: one new token per sequence
    t.inV = a.v_new + ((size_t)s * t.H + h) * kHeadDim;
    return t;
}

template <int BITS, int DT>
__device__ __forceinline__ void append_token_value_wave(const AppendArgs& a, int s, int h, int lane) {
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;
    constexpr int SLOT_BYTES = 4 * BITS;
    const TokenAppend t = token_append_ctx(a, s, h);
    if (!t.ok) return;
    const CacheView& V = *t.V;
    const int T0 = t.T0, T1 = T0 + 1, R = t.R;
    const int TK1 = R * (T1 / R);
    // sliding window only: a cache whose Values flush with the Keys never
    // takes the fused step
    const int TV0 = max(0, T0 - R), TV1 = max(0, T1 - R);
    const int slot_new = T0 % R;
    const uint32_t kv = *reinterpret_cast<const uint32_t*>(t.inK + 2 * lane);
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(t.inV + 2 * lane);
    if (TV1 > TV0) {  // token p leaves the window (its ring slot is the new token's)
        const int p = TV0;
        const float x0 = canon(to_f32<DT>(t.ringV[vring_index(R, p, 2 * lane)]));
        const float x1 = canon(to_f32<DT>(t.ringV[vring_index(R, p, 2 * lane + 1)]));
        const int gw = t.Gv / 2;  // lanes per channel group
        const float mn = group_min(fminf(x0, x1), gw);
        const float mx = group_max(fmaxf(x0, x1), gw);
        uint16_t s16, z16;
        float S, Z;
        group_params(mn, mx, QMAX, s16, z16, S, Z);
        const int ng = kHeadDim / t.Gv;
        const int blk = t.page_of(p);
        if (blk >= 0 && (lane % gw) == 0) {
            uint16_t* meta = reinterpret_cast<uint16_t*>(V.v_meta + ((size_t)blk * t.H + h) * V.v_meta_bytes) +
                             ((p % t.Bk) * ng + (2 * lane) / t.Gv) * 2;
            meta[0] = s16;
            meta[1] = z16;
        }
        const uint32_t packed = group_code(x0, S, Z, QMAX) | (group_code(x1, S, Z, QMAX) << 8);
        auto code_of = [&](int ch) -> uint32_t {  // code of channel ch (held by lane ch / 2)
            const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (ch >> 1), (int)packed);
            return (w >> (8 * (ch & 1))) & 0xFFu;
        };
        const int r = p & 3, jq = (p % kTile) >> 2, sub = (p % t.Bk) / kTile;
        const int m = lane & 15, w = lane >> 4;
        uint32_t word = 0;
        if constexpr (BITS == 4) {
            // nibble e of a word: (a,0) (a,2) (c,0) (c,2) (a,1) (a,3) (c,1) (c,3)
            const int ea = (r & 1) * 4 + (r >> 1), ec = ea + 2;
            const int ca = 32 * w + m, cc = ca + 16;
            const uint32_t codeA = code_of(ca), codeC = code_of(cc);
            word = (codeA << (4 * ea)) | (codeC << (4 * ec));
        } else {
            // field f: tile 4 w' + (f & 7) / 2, token 2 ((f & 7) & 1) + (f >> 3)
#pragma unroll
            for (int tq = 0; tq < 4; ++tq) {
                const int ff = 2 * tq + (r >> 1), f = ff + 8 * (r & 1);
                const int ch = 16 * (4 * (w & 1) + tq) + m;
                word |= code_of(ch) << (2 * f);
            }
        }
        const int words = (BITS == 4) ? 64 : 32;
        if (blk >= 0 && lane < words) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(V.v_codes + ((size_t)blk * t.H + h) * V.code_bytes +
                                                        sub * TILE_BYTES + SLOT_BYTES * (m + 16 * jq) + 4 * w);
            if (r == 0) *dst = word;  // the quad's first token: whole word, later tokens OR in
            else __hip_atomic_fetch_or(dst, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // residual writes (after the read above of the same Value slot)
    if (TK1 <= T0) *reinterpret_cast<uint32_t*>(t.ringK + (size_t)slot_new * kHeadDim + 2 * lane) = kv;
    t.ringV[vring_index(R, slot_new, 2 * lane)] = (uint16_t)(vv & 0xFFFFu);
    t.ringV[vring_index(R, slot_new, 2 * lane + 1)] = (uint16_t)(vv >> 16);
}

// Key flush of one wave: channels [64 half, 64 half + 64) of every Key group
// the token completes. Lane (u = lane / 8, c = lane % 8) holds channels
// 8 (8 half + c) .. + 7 of tokens u, u + 8, ...: one 16-byte load per token
// and lane, a chunk of up to 64 tokens (and its page ids) in flight together,
// so the residual is read in one round trip per chunk rather than one per
// token. A group longer than a chunk is read twice (min / max, then codes).
// Eight consecutive channels of one token are exactly one int4 code word of
// the Key layout (slot (token, j), word w with 32 w + 8 j = the chunk's first
// channel); an int2 word joins the chunks c and c ^ 4 of lanes lane and
// lane ^ 4.
template <int BITS, int DT>
__device__ __forceinline__ void append_token_key_wave(const AppendArgs& a, int s, int h, int half, int lane) {
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;
    constexpr int SLOT_BYTES = 4 * BITS;
    constexpr int kChunk = 64;        // tokens loaded together
    constexpr int kHeld = kChunk / 8;  // of them per lane
    const TokenAppend t = token_append_ctx(a, s, h);
    if (!t.ok) return;
    const CacheView& V = *t.V;
    const int T0 = t.T0, T1 = T0 + 1, R = t.R, G = t.G, Bk = t.Bk;
    const int TK0 = R * (T0 / R), TK1 = R * (T1 / R);
    if (TK1 == TK0) return;
    const int u = lane >> 3, cl = lane & 7;
    const int chunk = 8 * half + cl;  // channels 8 chunk .. 8 chunk + 7
    const int c0 = 8 * chunk;
    const int nch = kHeadDim * Bk / G;
    const int cw = G < kChunk ? G : kChunk;  // tokens per chunk (G is a power of two)
    const int nheld = cw / 8;
    uint4 held[kHeld];
    int pg = -1;
    // tokens c_start + u + 8 i of one chunk, and its page ids (lane l < cw / Bk:
    // the page of position c_start + l Bk)
    auto load_chunk = [&](int c_start) {
#pragma unroll
        for (int i = 0; i < kHeld; ++i) {
            if (i >= nheld) break;
            const int p = c_start + u + 8 * i;
            const uint16_t* src = p < T0 ? t.ringK + (size_t)(p % R) * kHeadDim + c0 : t.inK + c0;
            held[i] = *reinterpret_cast<const uint4*>(src);
        }
        pg = lane * Bk < cw ? t.page_of(c_start + lane * Bk) : -1;
    };
    auto value = [&](const uint4& w, int e) -> float {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        return canon(to_f32<DT>((uint16_t)(ws[e >> 1] >> (16 * (e & 1)))));
    };
    for (int base = TK0; base < TK1; base += G) {
        float mn[8], mx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            mn[e] = INFINITY;
            mx[e] = -INFINITY;
        }
        for (int c_start = base; c_start < base + G; c_start += cw) {
            load_chunk(c_start);
#pragma unroll
            for (int i = 0; i < kHeld; ++i) {
                if (i >= nheld) break;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = value(held[i], e);
                    mn[e] = fminf(mn[e], x);
                    mx[e] = fmaxf(mx[e], x);
                }
            }
        }
        // over the chunk's 8 lanes (cl + 8 u), then the group's parameters
        float S[8], Z[8];
        uint32_t sp[4], zp[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int o = 8; o < 64; o <<= 1) {
                mn[e] = fminf(mn[e], __shfl_xor(mn[e], o, 64));
                mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], o, 64));
            }
            uint16_t s16, z16;
            group_params(mn[e], mx[e], QMAX, s16, z16, S[e], Z[e]);
            if (e & 1) {
                sp[e >> 1] |= (uint32_t)s16 << 16;
                zp[e >> 1] |= (uint32_t)z16 << 16;
            } else {
                sp[e >> 1] = s16;
                zp[e >> 1] = z16;
            }
        }
        // the chunk's 8 scales and 8 zero-points, contiguous in the Key meta of
        // the group's page that holds them (nch is a multiple of 8)
        if (u == 0) {
            const int mblk = t.page_of(base + (c0 / nch) * Bk);
            if (mblk >= 0) {
                uint16_t* meta = reinterpret_cast<uint16_t*>(V.k_meta + ((size_t)mblk * t.H + h) * V.k_meta_bytes);
                *reinterpret_cast<uint4*>(meta + c0 % nch) = (uint4){sp[0], sp[1], sp[2], sp[3]};
                *reinterpret_cast<uint4*>(meta + nch + c0 % nch) = (uint4){zp[0], zp[1], zp[2], zp[3]};
            }
        }
        for (int c_start = base; c_start < base + G; c_start += cw) {
            if (cw < G) load_chunk(c_start);  // else the chunk is still held
#pragma unroll
            for (int i = 0; i < kHeld; ++i) {
                if (i >= nheld) break;
                const int p = c_start + u + 8 * i;
                uint32_t q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = group_code(value(held[i], e), S[e], Z[e], QMAX);
                const int blk = __shfl(pg, (p - c_start) / Bk, 64);
                const int sub = (p % Bk) / kTile, m = p % kTile;
                uint32_t word;
                int w, jj;
                bool store = blk >= 0;
                if constexpr (BITS == 4) {
                    // even channels in bits 4e, odd channels in bits 16 + 4e
                    word = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) word |= (q[2 * e] << (4 * e)) | (q[2 * e + 1] << (16 + 4 * e));
                    w = chunk >> 2;
                    jj = chunk & 3;
                } else {
                    // this chunk's fields: channel 8 chunk + 2 e + {0, 1} in fields e + 4 hi
                    // and 8 + e + 4 hi (hi: the chunk is the word's second channel group)
                    const int hi = (chunk >> 2) & 1;
                    uint32_t part = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        part |= (q[2 * e] << (2 * (e + 4 * hi))) | (q[2 * e + 1] << (2 * (8 + e + 4 * hi)));
                    word = part | (uint32_t)__shfl_xor((int)part, 4, 64);
                    w = chunk >> 3;
                    jj = chunk & 3;
                    store = store && hi == 0;
                }
                if (store) {
                    uint8_t* dst = V.k_codes + ((size_t)blk * t.H + h) * V.code_bytes + sub * TILE_BYTES +
                                   SLOT_BYTES * (m + 16 * jj) + 4 * w;
                    *reinterpret_cast<uint32_t*>(dst) = word;
                }
            }
        }
    }
}

}  // namespace kivi
