// Chunked-prefill attention over the KIVI cache as stored, after the chunk
// was appended ("4.4 KV Cache 量化", section 2: P = softmax(Q K^T / sqrt(d)),
// out = P V; section 3.2: quantised history plus the full-precision
// residual; "给 KV cache 减肥", section 3: values restored on read).
//
// Rows: the (query position, query head) pairs of one (sequence, KV head),
// row r = i * g + head for chunk query i. A wave owns 16 consecutive rows
// (one matrix-core row tile, the N dimension of the score MFMA) and streams
// every Key/Value tile its rows can see: 16-token tiles of codes on matrix
// cores exactly as in decode (Key scale folded into a per-group query table
// split fp16 hi + lo, zero-point as the bias that starts the chain; Values in
// pairs of tiles against fp16 weights p * scale / F), then the tiles that
// touch the residual. Causal rows see tokens 0 .. their own position; the
// mask is applied per row only on tiles past the smallest row position.
// Work groups hold 4 independent waves; each wave writes its rows' output.
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

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kRowsPerWave = 16;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X, each with its own L2
// Main-loop Key codes keep their 1024 offsets, taken out through the table's
// bias (saves a packed subtract per code pair); the tail stays exact.
constexpr bool kFoldK = true;

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
    float scale_log2;
    int causal;
    int max_q_len;   // the caller's bound of every query span
    int wg_per_sh;   // work groups per (sequence, KV head)
    int tpg_shift;   // log2(tiles per Key group)
    int tpp_shift;   // log2(tiles per page)
    uint32_t code_array_bytes, vmeta_array_bytes, kmeta_array_bytes;
    uint16_t* out;
};

// LDS of one wave: q rows [16] | Key-group table rows [16][hi, lo] | bias [16]
__host__ __device__ constexpr int prefill_wave_lds_bytes() { return 3 * kRowsPerWave * kRowBytes + 64; }

// Tiles per load buffer (two buffers per wave), as in decode.
template <int NG>
constexpr int max_buffer_tiles_pf() { return NG == 1 ? 4 : (NG <= 4 ? 2 : 1); }

template <int BITS, int DT, int NG, int kHalf>
__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(PrefillArgs a) {
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;
    constexpr int SLOT_BYTES = 4 * BITS;
    constexpr int NB = (BITS == 2) ? 2 : 1;
    extern __shared__ __align__(16) uint8_t smem[];
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
    const int n = lane & 15, j = lane >> 4;
    const int g = a.gqa;
    const int HQ = a.num_q_heads;

    // ---- the sequence and this wave's rows ----
    const int q0 = a.cu_q[s];
    const int nq = a.cu_q[s + 1] - q0;
    // P tokens come from the cache; with a full-precision chunk its nq tokens follow them
    int P = a.seq_lens[s];
    const int slot = a.slot_ids[s];
    const bool bad = slot < 0 || slot >= V.max_seqs || P < 0;
    const bool raw_chunk = a.k_chunk != nullptr;
    // device-side errors this wave met (wave-uniform), reported before the output
    uint32_t err = 0;
    if (wg == 0 && wave == 0) {
        err = (slot < 0 || slot >= V.max_seqs ? KIVI_DEVERR_SLOT : 0u) | (P < 0 ? KIVI_DEVERR_LENGTH : 0u);
        if (nq < 0 || nq > a.max_q_len || (!raw_chunk && !bad && nq > P)) err |= KIVI_DEVERR_QUERY;
        if (!bad && (long long)P + (raw_chunk ? max(nq, 0) : 0) > (long long)a.bt_stride * V.Bk)
            err |= KIVI_DEVERR_LENGTH;
        if (err != 0 && lane == 0) report_error(V.status, err);
        err = 0;
    }
    if (bad) P = 0;
    const int T = bad ? 0 : P + (raw_chunk ? nq : 0);  // tokens the rows attend over
    const int row0 = (wg * kPWaves + wave) * kRowsPerWave;
    if (nq <= 0 || row0 >= nq * g) return;  // no rows for this wave
    const int TK = V.R * (P / V.R), TV = value_boundary(V, P);
    const int n_main = TV / kTile;
    const int tk_tiles = TK / kTile;
    const int R = V.R;
    const int row = row0 + n;  // this lane's row
    const bool row_ok = row < nq * g && T > 0;
    const int qi = row / g, qh = row % g;
    // position of the row's query; the last visible token
    const int my_pos = row_ok ? T - nq + qi : -1;
    const int my_last = row_ok ? (a.causal ? min(my_pos, T - 1) : T - 1) : -1;
    // extent over the wave's rows (lanes of one 16-lane row hold all 16 rows)
    int last_max = my_last, last_min = row_ok ? my_last : 0x7fffffff;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        last_max = max(last_max, __shfl_xor(last_max, d));
        last_min = min(last_min, __shfl_xor(last_min, d));
    }
    last_max = __builtin_amdgcn_readfirstlane(last_max);
    last_min = __builtin_amdgcn_readfirstlane(last_min);
    const int n_tiles = (last_max + 1 + kTile - 1) / kTile;  // tiles any row sees
    const int m_end = min(n_main, n_tiles);                   // main tiles
    const int full_tiles = (last_min + 1) / kTile;            // tiles every row sees whole

    const int tpg = 1 << a.tpg_shift, tpp = 1 << a.tpp_shift;
    const int nch = kHeadDim * V.Bk / V.G;
    const int meta_tile = (8 * (lane & 15) / nch) * tpp;
    const float sgn = a.scale_log2 < 0.0f ? -1.0f : 1.0f;
    const float sl2 = fabsf(a.scale_log2);
    const float thr = sl2 > 0.0f ? kLazyLog2 / sl2 : 0.0f;

    uint8_t* wl = smem + wave * prefill_wave_lds_bytes();
    uint16_t* lq = reinterpret_cast<uint16_t*>(wl);
    uint8_t* lt = wl + kRowsPerWave * kRowBytes;
    float* lbias = reinterpret_cast<float*>(lt + 2 * kRowsPerWave * kRowBytes);
    const int lane_row = n * 2 * kRowBytes + 16 * j;
    const uint32_t lane_code_off = SLOT_BYTES * lane;
    const uint32_t lane_meta_off = 16 * NG * j;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(V.k_codes, a.code_array_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V.v_codes, a.code_array_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(V.v_meta, a.vmeta_array_bytes);
    const __amdgpu_buffer_rsrc_t rkm = make_rsrc(V.k_meta, a.kmeta_array_bytes);
    const uint16_t* ringK = V.k_ring + ((size_t)max(slot, 0) * H + h) * V.ring_elems;
    const uint16_t* ringV = V.v_ring + ((size_t)max(slot, 0) * H + h) * V.ring_elems;
    const int32_t* bt = a.block_table + (size_t)s * a.bt_stride;
    auto page_of = [&](int t) -> int {  // block-table entry of tile t, unchecked
        const int bi = t >> a.tpp_shift;
        return (t < 0 || bi >= a.bt_stride) ? -1 : bt[bi];
    };
    auto valid_pg = [&](int blk) -> int { return (blk >= 0 && blk < V.num_blocks) ? blk : -1; };

    // ---- query rows to LDS (fp16), zero rows past the chunk ----
    int my_page = page_of(lane);
    int next_page = page_of(64 + lane);
    {
        uint4 qv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // 16 rows x 16 chunks of 8 channels
            const int idx = lane + 64 * r, rr = idx >> 4, k = idx & 15;
            const int rw = row0 + rr;
            qv[r] = (uint4){0, 0, 0, 0};
            if (rw < nq * g)
                qv[r] = *reinterpret_cast<const uint4*>(
                    a.q + ((size_t)(q0 + rw / g) * HQ + h * g + rw % g) * kHeadDim + 8 * k);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = lane + 64 * r, rr = idx >> 4, k = idx & 15;
            uint4 o = qv[r];
            if constexpr (DT == kBF16) {
                const uint32_t w[4] = {o.x, o.y, o.z, o.w};
                uint32_t cv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const _Float16 lo = (_Float16)bf16_bits_to_f32((uint16_t)(w[e] & 0xFFFFu));
                    const _Float16 hi = (_Float16)bf16_bits_to_f32((uint16_t)(w[e] >> 16));
                    cv[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                o = {cv[0], cv[1], cv[2], cv[3]};
            }
            *reinterpret_cast<uint4*>(lq + rr * kQRow + 8 * k) = o;
        }
    }

    Acc<NG, NB> st;
    st.init();

    // ---- main tiles [0, m_end): the decode pipeline, masked near the diagonal ----
    struct Buf {
        TileRegs<BITS, NG> t[kHalf];
        bool ok[kHalf];
        uint4 ms, mz;
    };
    int base = 0;
    auto issue = [&](int t0, Buf& b) {
        if (t0 - base >= 64) {
            base += 64;
            my_page = next_page;
            next_page = page_of(base + 64 + lane);
        }
#pragma unroll
        for (int e = 0; e < kHalf; ++e) {
            const int t = t0 + e;
            const int blk = valid_pg(__builtin_amdgcn_readlane(my_page, (t - base) & 63));
            b.ok[e] = blk >= 0 && t < m_end;
            if (blk < 0 && t < m_end) err |= KIVI_DEVERR_PAGE;
            const uint32_t chk = (uint32_t)(b.ok[e] ? blk : 0) * (uint32_t)H + (uint32_t)h;
            const uint32_t sub = (uint32_t)t & ((1u << a.tpp_shift) - 1u);
            const uint32_t coff = chk * (uint32_t)V.code_bytes + sub * TILE_BYTES;
            const uint32_t moff = chk * (uint32_t)V.v_meta_bytes + sub * (kTile * NG * 4);
            if constexpr (BITS == 4) {
                const uint4 k4 = buf_b128(rk, lane_code_off, coff);
                const uint4 v4 = buf_b128(rv, lane_code_off, coff);
                b.t[e].k[0] = k4.x; b.t[e].k[1] = k4.y; b.t[e].k[2] = k4.z; b.t[e].k[3] = k4.w;
                b.t[e].v[0] = v4.x; b.t[e].v[1] = v4.y; b.t[e].v[2] = v4.z; b.t[e].v[3] = v4.w;
            } else {
                const uint2 k2 = buf_b64(rk, lane_code_off, coff);
                const uint2 v2 = buf_b64(rv, lane_code_off, coff);
                b.t[e].k[0] = k2.x; b.t[e].k[1] = k2.y;
                b.t[e].v[0] = v2.x; b.t[e].v[1] = v2.y;
            }
#pragma unroll
            for (int qd = 0; qd < NG; ++qd) {
                const uint4 m = buf_b128(rm, lane_meta_off + 16 * qd, moff);
                b.t[e].vm[4 * qd + 0] = m.x; b.t[e].vm[4 * qd + 1] = m.y;
                b.t[e].vm[4 * qd + 2] = m.z; b.t[e].vm[4 * qd + 3] = m.w;
            }
        }
        const int gt = ((t0 + kHalf - 1) >> a.tpg_shift) << a.tpg_shift;
        const int mp = valid_pg(__builtin_amdgcn_ds_bpermute(4 * ((gt + meta_tile - base) & 63), my_page));
        const uint32_t mo = k_meta_off(V, h, mp, nch);
        b.ms = buf_b128(rkm, mo, 0);
        b.mz = buf_b128(rkm, mo + 2u * (uint32_t)nch, 0);
    };
    float bias = 0.0f;
    auto compute = [&](const Buf& b, int t0) {
#pragma unroll
        for (int e = 0; e < kHalf; e += 2) {
            const int t = t0 + e;
            constexpr bool kPair = kHalf > 1;
            const bool oka = b.ok[e], okb = kPair ? b.ok[kPair ? e + 1 : e] : false;
            if (!oka && !okb) continue;
            if ((t & (tpg - 1)) == 0 && t != 0) bias = build_table<BITS, kFoldK>(kRowsPerWave, b.ms, b.mz, lq, lt, lbias, n, sgn);
            const TileRegs<BITS, NG>& ta = b.t[e];
            const TileRegs<BITS, NG>& tb = b.t[kPair ? e + 1 : e];
            f4 ra = code_scores<BITS, kFoldK>(ta.k, lt, lane_row, bias);
            f4 rb = ra;
            if (kPair) rb = code_scores<BITS, kFoldK>(tb.k, lt, lane_row, bias);
            float pa[4], pb[4];
            if (oka && okb && t + 1 < full_tiles) {  // both tiles seen whole by every row (uniform)
                const float mx = max2(max4(ra), max4(rb));
                st.rescale(xor_max(mx), sl2, thr);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pa[r] = st.weight(ra[r], sl2);
                    pb[r] = st.weight(rb[r], sl2);
                }
            } else {
                // visibility of token 16 t' + 4 j + r to this lane's row
                bool va[4], vb[4];
                const bool full_a = t < full_tiles, full_b = t + 1 < full_tiles;  // uniform
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    va[r] = oka && (full_a || 16 * t + 4 * j + r <= my_last);
                    vb[r] = okb && (full_b || 16 * (t + 1) + 4 * j + r <= my_last);
                }
                float mx = -INFINITY;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (va[r]) mx = max2(mx, ra[r]);
                    if (vb[r]) mx = max2(mx, rb[r]);
                }
                st.rescale(xor_max(mx), sl2, thr);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pa[r] = va[r] ? st.weight(ra[r], sl2) : 0.0f;
                    pb[r] = vb[r] ? st.weight(rb[r], sl2) : 0.0f;
                }
            }
            st.l_acc += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
            value_pair<BITS, NG, NB>(st, ta.v, ta.vm, tb.v, tb.vm, pa, pb, oka, okb);
        }
    };
    if (m_end > 0) {
        Buf ba, bb;
        issue(0, ba);
        const int mp = valid_pg(__builtin_amdgcn_ds_bpermute(4 * meta_tile, my_page));
        const uint32_t mo = k_meta_off(V, h, mp, nch);
        const uint4 ms0 = buf_b128(rkm, mo, 0);
        const uint4 mz0 = buf_b128(rkm, mo + 2u * (uint32_t)nch, 0);
        bias = build_table<BITS, kFoldK>(kRowsPerWave, ms0, mz0, lq, lt, lbias, n, sgn);
        int it = 0;
        for (int t0 = 0; t0 < m_end; t0 += 2 * kHalf) {
            issue(t0 + kHalf, bb);
            compute(ba, t0);
            if (t0 + kHalf >= m_end) break;
            issue(t0 + 2 * kHalf, ba);
            compute(bb, t0 + kHalf);
            if (++it == flush_period<kHalf>()) {
                it = 0;
                st.template flush_offsets<BITS>();
            }
        }
    }

    // ---- tiles that touch the residual: [n_main, n_tiles) ----
    for (int t = max(n_main, 0); t < n_tiles; ++t) {
        const int tb0 = (t >> a.tpg_shift) << a.tpg_shift;
        const int tpage = page_of(tb0 + lane);
        const int blk = valid_pg(__builtin_amdgcn_readlane(tpage, t - tb0));
        const int p0 = t * kTile, pq = p0 + 4 * j;
        if (blk < 0 && (t < tk_tiles || p0 < TV)) {  // codes without a page
            err |= KIVI_DEVERR_PAGE;
            continue;
        }
        const uint32_t chk = (uint32_t)blk * (uint32_t)H + (uint32_t)h;
        const uint32_t sub = (uint32_t)t & ((1u << a.tpp_shift) - 1u);
        const uint32_t coff = chk * (uint32_t)V.code_bytes + sub * TILE_BYTES;
        const uint32_t moff = chk * (uint32_t)V.v_meta_bytes + sub * (kTile * NG * 4);
        f4 raw;
        if (t < tk_tiles) {
            uint32_t kw[BITS];
            if constexpr (BITS == 4) {
                const uint4 u = buf_b128(rk, lane_code_off, coff);
                kw[0] = u.x; kw[1] = u.y; kw[2] = u.z; kw[3] = u.w;
            } else {
                const uint2 u = buf_b64(rk, lane_code_off, coff);
                kw[0] = u.x; kw[1] = u.y;
            }
            const int mp = valid_pg(__builtin_amdgcn_ds_bpermute(4 * meta_tile, tpage));
            const uint32_t mo = k_meta_off(V, h, mp, nch);
            const uint4 ms = buf_b128(rkm, mo, 0);
            const uint4 mz = buf_b128(rkm, mo + 2u * (uint32_t)nch, 0);
            const float tbias = build_table<BITS>(kRowsPerWave, ms, mz, lq, lt, lbias, n, sgn);
            raw = code_scores<BITS>(kw, lt, lane_row, tbias);
        } else {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            const uint8_t* qrow = reinterpret_cast<const uint8_t*>(lq + n * kQRow);
            const int pk = min(p0 + n, T - 1);  // A row: token n of the tile
            const uint16_t* krow = pk < P ? ringK + (size_t)(pk % R) * kHeadDim
                                          : a.k_chunk + ((size_t)(q0 + pk - P) * H + h) * kHeadDim;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 kr = *reinterpret_cast<const uint4*>(krow + 32 * i + 8 * j);
                const uint32_t ws[4] = {kr.x, kr.y, kr.z, kr.w};
                h8 A;
#pragma unroll
                for (int e = 0; e < 8; ++e) A[e] = (_Float16)to_f32<DT>((uint16_t)(ws[e >> 1] >> (16 * (e & 1))));
                const h8 B = *reinterpret_cast<const h8*>(qrow + 2 * (32 * i + 8 * j));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc, 0, 0, 0);
            }
            raw = acc * sgn;
        }
        uint32_t vw[BITS], vm[4 * NG];
#pragma unroll
        for (int k = 0; k < BITS; ++k) vw[k] = 0;
#pragma unroll
        for (int k = 0; k < 4 * NG; ++k) vm[k] = 0;
        if (p0 < TV) {
            if constexpr (BITS == 4) {
                const uint4 u = buf_b128(rv, lane_code_off, coff);
                vw[0] = u.x; vw[1] = u.y; vw[2] = u.z; vw[3] = u.w;
            } else {
                const uint2 u = buf_b64(rv, lane_code_off, coff);
                vw[0] = u.x; vw[1] = u.y;
            }
#pragma unroll
            for (int qd = 0; qd < NG; ++qd) {
                const uint4 m = buf_b128(rm, lane_meta_off + 16 * qd, moff);
                vm[4 * qd + 0] = m.x; vm[4 * qd + 1] = m.y; vm[4 * qd + 2] = m.z; vm[4 * qd + 3] = m.w;
            }
        }
        uint2 vr[8];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
            vr[tt] = *reinterpret_cast<const uint2*>(ringV + vring_index(R, pq, 16 * tt + n));
        if (raw_chunk && p0 + kTile > P) {  // chunk tokens replace their ring halves (uniform test)
            bool inc[4];
            const uint16_t* vrow[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                inc[r] = pq + r >= P && pq + r < T;
                vrow[r] = a.v_chunk + ((size_t)(q0 + (inc[r] ? pq + r - P : 0)) * H + h) * kHeadDim + n;
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                uint32_t w[2] = {vr[tt].x, vr[tt].y};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (inc[r]) {
                        const uint32_t sh16 = 16u * (uint32_t)(r & 1);
                        w[r >> 1] = (w[r >> 1] & ~(0xFFFFu << sh16)) | ((uint32_t)vrow[r][16 * tt] << sh16);
                    }
                vr[tt] = make_uint2(w[0], w[1]);
            }
        }
        float p[4], mx = -INFINITY;
        bool vis[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vis[r] = pq + r < T && pq + r <= my_last;
            if (vis[r]) mx = max2(mx, raw[r]);
        }
        st.rescale(xor_max(mx), sl2, thr);
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = vis[r] ? st.weight(raw[r], sl2) : 0.0f;
        st.l_acc += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            const int gg = (16 * tt) / (kHeadDim / NG);
            const bool first_of_group = (16 * tt) % (kHeadDim / NG) == 0;
            const uint32_t rw[2] = {vr[tt].x, vr[tt].y};
            h4 A;
            h8 B;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pr = pq + r;
                const bool is_code = pr < TV, is_raw = !is_code && pr < T;  // ring or chunk
                const uint32_t mw = is_code ? vm[r * NG + gg] : 0u;
                if (first_of_group) st.zacc[gg] += p[r] * f16_bits_to_f32((uint16_t)(mw >> 16));
                const float code_v = (float)v_code_at<BITS>(vw, tt, r);
                const float raw_v = to_f32<DT>((uint16_t)(rw[r >> 1] >> (16 * (r & 1))));
                const float av = is_code ? code_v : (is_raw ? raw_v : 0.0f);
                const float wv = is_code ? p[r] * f16_bits_to_f32((uint16_t)(mw & 0xFFFFu)) : (is_raw ? p[r] : 0.0f);
                A[r] = (_Float16)av;
                _Float16 hi, lo;
                split_f16(wv, hi, lo);
                B[r] = hi;
                B[4 + r] = lo;
            }
            st.O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dup_h8(A), B, st.O[tt], 0, 0, 0);
        }
    }

    // ---- output of this wave's rows ----
    const float l_tot = xor_sum(st.l_acc);
    float zt[NG][NB];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
        const float z = xor_sum(st.zacc[gg]);
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) zt[gg][vb] = z - (BITS == 4 ? 1024.0f * xor_sum(st.wsum[gg][vb]) : 0.0f);
    }
    if (err != 0 && lane == 0) report_error(V.status, err);
    if (!(row < nq * g)) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* orow = a.out + ((size_t)(q0 + qi) * HQ + h * g + qh) * kHeadDim;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int chn = 16 * tt + 4 * j + r;
            orow[chn] = from_f32<DT>((st.O[tt][r] + zt[chn / (kHeadDim / NG)][tt % NB]) * inv);
        }
}

template <int BITS, int DT, int NG>
void launch_pf_ng(const PrefillArgs& a, int tpg, dim3 grid, size_t lds, hipStream_t st) {
    dim3 block(kPThreads);
    constexpr int kMax = max_buffer_tiles_pf<NG>();
    const int kh = std::min(kMax, tpg);
    if (kh >= 4 && kMax >= 4)
        hipLaunchKernelGGL((prefill_kernel<BITS, DT, NG, (kMax >= 4 ? 4 : 1)>), grid, block, lds, st, a);
    else if (kh >= 2 && kMax >= 2)
        hipLaunchKernelGGL((prefill_kernel<BITS, DT, NG, (kMax >= 2 ? 2 : 1)>), grid, block, lds, st, a);
    else
        hipLaunchKernelGGL((prefill_kernel<BITS, DT, NG, 1>), grid, block, lds, st, a);
}

template <int BITS, int DT>
void launch_pf(const PrefillArgs& a, int ng, int tpg, dim3 grid, size_t lds, hipStream_t st) {
    switch (ng) {
        case 1: launch_pf_ng<BITS, DT, 1>(a, tpg, grid, lds, st); break;
        case 2: launch_pf_ng<BITS, DT, 2>(a, tpg, grid, lds, st); break;
        case 4: launch_pf_ng<BITS, DT, 4>(a, tpg, grid, lds, st); break;
        default: launch_pf_ng<BITS, DT, 8>(a, tpg, grid, lds, st); break;
    }
}

}  // namespace

size_t prefill_lds_bytes() { return (size_t)kPWaves * prefill_wave_lds_bytes(); }

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
    const int rows = max_q_len * a.gqa;
    const int wave_tiles = (rows + kRowsPerWave - 1) / kRowsPerWave;
    a.wg_per_sh = (wave_tiles + kPWaves - 1) / kPWaves;
    a.tpg_shift = __builtin_ctz((unsigned)(v.G / kTile));
    a.tpp_shift = __builtin_ctz((unsigned)(v.Bk / kTile));
    a.code_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.code_bytes);
    a.vmeta_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.v_meta_bytes);
    a.kmeta_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.k_meta_bytes);
    a.out = static_cast<uint16_t*>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int ng = kHeadDim / v.Gv;
    const int tpg = v.G / kTile;
    dim3 grid((unsigned)((size_t)num_seqs * v.H * a.wg_per_sh));
    const size_t lds = prefill_lds_bytes();
    if (v.bits == 4) {
        if (v.dtype == kF16) launch_pf<4, kF16>(a, ng, tpg, grid, lds, st);
        else launch_pf<4, kBF16>(a, ng, tpg, grid, lds, st);
    } else {
        if (v.dtype == kF16) launch_pf<2, kF16>(a, ng, tpg, grid, lds, st);
        else launch_pf<2, kBF16>(a, ng, tpg, grid, lds, st);
    }
    return (int)hipGetLastError();
}

}  // namespace kivi
