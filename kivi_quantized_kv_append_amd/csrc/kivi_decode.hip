// Split-K paged decode attention over the KIVI cache, dequantising on read
// ("4.4 KV Cache 量化", section 2: P = softmax(Q K^T / sqrt(d)), out = P V;
// section 3.2: the residual takes part next to the quantised history;
// "给 KV cache 减肥", section 3: values are restored when the query reads
// them).
//
// Work: one work group of 8 waves per (sequence, KV head, split). The main
// 16-token tiles (Key and Value both quantised) of a (sequence, KV head) are
// cut into contiguous wave ranges; the tail tiles, which touch the residual,
// are dealt out one per wave. The waves merge in LDS; with one split the
// work group writes the output, with several it writes a partial (running
// max m, sum l, unnormalised o) per query head and a merge kernel follows.
//
// Per pair of main tiles (16 tokens each), per wave:
//   scores  S^T[16 tok][16 q-heads] = K_codes[16][128] x Q'^T[128][16] on
//           matrix cores (v_mfma_f32_16x16x32_f16), with the Key scale folded
//           into the query (Q' = q * scale / F, per channel and group, as an
//           fp16 hi + lo pair) and the zero-point into a per-group bias
//           (sum_c q_c zero_c) that starts the accumulation chain;
//   softmax online, per query head, in registers, with a lazily moved max;
//   values  O^T[128][16] += V_codes^T[128][32 tok] x W[32 tok][16] (one
//           MFMA per 16-channel tile for both tiles), W = p * scale_V / F.
// Codes become fp16 numbers with one AND-OR per pair (fields placed in an
// fp16 mantissa under the exponent of 1024); Key codes also get a packed
// subtract so they are exact integers. Query heads of a KV head (GQA) are
// the matrix N dimension (<= 16).
//
// Fused decode step (kivi_decode_step): the same kernel first appends one
// token per sequence. In split 0 of each (sequence, KV head), wave 7
// quantises the Value token that leaves the window and writes the residual,
// and, when the Key residual fills, waves 5 and 6 quantise its Key groups;
// all of this runs beside the other waves' attention. Main tiles lie below
// the old Value boundary, so the append writes nothing they read; the tile
// of the evicted token is read by the wave that wrote it, and a flush step
// reads its tail tiles after a barrier.

#include <mutex>

#include "kivi_append_body.h"
#include "kivi_attn.h"

namespace kivi {
namespace {

using namespace attn;

constexpr int kThreads = 512;
constexpr int kBtPre = 1024;  // page-table entries a work group can hold in LDS
constexpr int kWaves = 8;
// Main tiles of a SIMD's older wave, in percent of an even split (the
// younger wave takes 200 minus this): measured best at 110 on MI355X with
// 4-tile blocks (130 with 2-tile buffers); an even split is slowest.
constexpr int kOldShare = 110;
constexpr int kAppendShare = 70;  // main-tile share of the appending wave (20-70 measure alike)
// Main-tile weight of each of the two Key-flush waves on a step that flushes
// (an even share is 300; their share goes to waves 0-3): the flush keeps them
// busy for a third of the step (measured 52.8 us per Llama flush step against
// 61.0 us at the plain share, 43.5 us with no flush arithmetic at all).
constexpr int kFlushShare = 40;
static_assert((4 * (200 - kOldShare) - kAppendShare - kFlushShare) % 2 == 0, "waves 0-3 split the rest evenly");
// Main tiles keep the 1024 offsets of the Key codes (one and-or per pair, no
// subtract) and take 1024 sum_c Q'[n][c] out of the table's bias; the tail
// tiles, whose tables are built apart, use exact codes.
constexpr bool kFoldK = true;
// 4-tile blocks: load buffers per wave (blocks in flight while one is
// computed: kQuadBuffers - 1), and whether the tail tiles come first (their
// loads overlap the first block's) or after the main range.
constexpr int kQuadBuffers = 2;
constexpr bool kTailFirst = false;
// Tiles per load buffer (two buffers per wave): deeper for the lighter
// Value metadata of wide Value groups, and never more than the tiles of a
// Key group (so at most one group begins inside a buffer).
template <int NG>
__host__ __device__ constexpr int max_buffer_tiles() { return NG <= 2 ? 2 : 1; }

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
    float* partials;  // [S][H_Q][n_splits] partials when n_splits > 1
    int n_splits;
    int tpg_shift;    // log2(tiles per Key group)
    int tpp_shift;    // log2(tiles per page)
    uint32_t code_array_bytes, vmeta_array_bytes, kmeta_array_bytes;
    uint16_t* out;
    // Fused decode step: seq_lens holds the lengths before this step's token;
    // split 0 of each (sequence, KV head) appends the token (rows of app.k_new
    // / app.v_new in sequence order) before it attends over T + 1 tokens.
    int fuse;
    // Tokens appended by an earlier launch on the stream after seq_lens was
    // taken (0 or 1): the sequence holds seq_lens[s] + len_add tokens.
    int len_add;
    AppendArgs app;
};

// Per-wave LDS (dynamic shared memory, one region per wave), fp16 rows of
// kQRow elements (272 bytes: the 16-byte pad spreads rows over banks):
//   q rows [g] | Key-group table rows [g][hi, lo] | bias [16] f32 | zero rows [hi, lo]
// (the zero rows are the off-diagonal blocks of the 4-tile tables). The
// epilogue reuses the whole work group's memory for the wave merge.
__host__ __device__ constexpr int wave_lds_bytes(int g) { return 3 * g * kRowBytes + 64 + 2 * kRowBytes; }

// Row rotation inside each 16-lane row (DPP row_ror).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}
// Sum over the lanes n, n + 4, n + 8, n + 12 of each 16-lane row.
__device__ __forceinline__ float quad_fold(float x) {
    x += row_ror<4>(x);
    return x + row_ror<8>(x);
}
__host__ __device__ constexpr int merge_lds_bytes(int g) { return kWaves * g * (kHeadDim + 2) * 4; }

// Shared state of one work group: the sequence, the KV head, its lengths.
struct WgCtx {
    int s, h, g, T, TK, TV, n_main, slot;
    const int32_t* bt;
    int bt_len;
    uint32_t err;  // kivi_device_error bits of the sequence's slot and length
};

__device__ __forceinline__ WgCtx make_ctx(const DecodeArgs& a, int s, int h) {
    const CacheView& V = a.v;
    WgCtx c;
    c.s = s;
    c.h = h;
    c.g = a.gqa;
    const int T_in = a.seq_lens[s];
    int T = T_in + a.fuse + a.len_add;
    c.slot = a.slot_ids[s];
    c.err = (c.slot < 0 || c.slot >= V.max_seqs ? KIVI_DEVERR_SLOT : 0u) | (T_in < 0 ? KIVI_DEVERR_LENGTH : 0u);
    if (c.err) T = 0;  // the sequence is skipped
    else if ((long long)T > (long long)a.bt_stride * V.Bk) c.err = KIVI_DEVERR_LENGTH;  // past the page table
    c.T = T;
    c.TK = V.R * (T / V.R);
    c.TV = value_boundary(V, T);
    // main tiles: Key and Value both quantised before this call (a fused step
    // writes only at or past the old Value boundary; both boundaries are
    // multiples of 16 or past the Key one)
    c.n_main = value_boundary(V, max(0, T - a.fuse)) / kTile;
    c.bt = a.block_table + (size_t)s * a.bt_stride;
    c.bt_len = a.bt_stride;
    return c;
}

// Block-table entry of tile t (unchecked; -1 past the table). Entries are
// checked where they are used (valid_page), so the load is not waited on
// here.
__device__ __forceinline__ int page_of_tile(const DecodeArgs& a, const WgCtx& c, int t) {
    const int bi = t >> a.tpp_shift;
    if (t < 0 || bi >= c.bt_len) return -1;
    return c.bt[bi];
}
// The page, or -1 when the entry names no block of the pool (tile skipped).
__device__ __forceinline__ int valid_page(const DecodeArgs& a, int blk) {
    return (blk >= 0 && blk < a.v.num_blocks) ? blk : -1;
}

// The g query rows of this KV head, converted to fp16 (bf16 queries are
// exact in fp16 inside its range), into the wave's q rows.
template <int DT>
__device__ __forceinline__ void load_query(const DecodeArgs& a, const WgCtx& c, uint16_t* lq) {
    const int lane = threadIdx.x & 63;
    uint4 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // 16 chunks of 8 channels per row, up to 16 rows
        const int idx = lane + 64 * r, hn = idx >> 4, k = idx & 15;
        v[r] = (uint4){0, 0, 0, 0};
        if (hn < c.g)
            v[r] = *reinterpret_cast<const uint4*>(a.q + ((size_t)c.s * a.num_q_heads + c.h * c.g + hn) * kHeadDim +
                                                   8 * k);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int idx = lane + 64 * r, hn = idx >> 4, k = idx & 15;
        if (hn >= c.g) continue;
        uint4 out = v[r];
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
        *reinterpret_cast<uint4*>(lq + hn * kQRow + 8 * k) = out;
    }
}

// Loads of one tail tile (a tile that touches the residual): Keys from codes
// (t < TK / 16) or from the fp16 residual, Value tokens from codes (< TV) or
// the residual.
template <int BITS, int NG>
struct TailRegs {
    uint32_t kw[BITS], vw[BITS], vm[4 * NG];
    uint4 kr[4];
    uint2 vr[8];
    uint4 ms, mz;
    int blk;
};

// One work group of kWaves waves per (sequence, KV head, split). The main
// tiles (Key and Value both quantised) of a (sequence, KV head) are cut into
// kWaves x n_valid contiguous wave ranges, weighted by wave age; the tail tiles
// (touching the residual) are dealt out one per wave. Each wave streams its
// range on its own: page ids of a 64-tile window, one buffer of tiles in
// flight while the other is computed, and the query table of each Key group
// built in its own LDS rows when the group begins (scales and zero-points
// travel with the tile loads). The waves merge in LDS into the output, or,
// when the sequence is split, into one partial (m, l, o) per query head that
// merge_kernel combines: m = max m_i, l = sum l_i 2^(m_i - m),
// o = sum o_i 2^(m_i - m) / l.
template <int BITS, int DT, int NG, int kHalf>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
    constexpr int TILE_BYTES = kTile * kHeadDim * BITS / 8;
    constexpr int SLOT_BYTES = 4 * BITS;
    constexpr int NB = (BITS == 2) ? 2 : 1;  // Value pair-factor variants
    extern __shared__ __align__(16) uint8_t smem[];
    const CacheView& V = a.v;
    const int H = V.H;
    const int split = blockIdx.x % a.n_splits;
    const int sh = blockIdx.x / a.n_splits;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    uint8_t* wl = smem + wave * wave_lds_bytes(a.gqa);
    uint16_t* lq = reinterpret_cast<uint16_t*>(wl);
    // First round trip, all at once: the sequence's length and slot, the
    // query rows and, when it fits in LDS, the whole page-table row (then the
    // first windows of page ids need no round trip of their own; later
    // windows are loaded one window ahead).
    __shared__ int bt_pre[kBtPre];
    // (16-channel Value groups leave it out: their registers are full)
    const bool bt_fits = NG < 8 && a.bt_stride <= kBtPre;  // uniform
    int pre[kBtPre / kThreads];
#pragma unroll
    for (int e = 0; e < kBtPre / kThreads; ++e) {
        const int idx = tid + e * kThreads;
        pre[e] = bt_fits && idx < a.bt_stride ? a.block_table[(size_t)(sh / H) * a.bt_stride + idx] : -1;
    }
    const WgCtx c = make_ctx(a, sh / H, sh % H);
    load_query<DT>(a, c, lq);
    if (bt_fits) {
#pragma unroll
        for (int e = 0; e < kBtPre / kThreads; ++e) bt_pre[tid + e * kThreads] = pre[e];
        __syncthreads();
    }
    auto first_page = [&](int t) -> int {  // page_of_tile, from LDS when the row is there
        if (!bt_fits) return page_of_tile(a, c, t);
        const int bi = t >> a.tpp_shift;
        return (t < 0 || bi >= c.bt_len) ? -1 : bt_pre[bi];
    };
    // at least kMinSplitTiles main tiles per split when there are that many
    const int nvalid = min(a.n_splits, max(1, (c.n_main + kMinSplitTiles - 1) / kMinSplitTiles));
    // device-side errors this wave met (wave-uniform), reported once at the end
    uint32_t err = split == 0 && tid < 64 ? c.err : 0u;
    if (split >= nvalid) {  // no work: an empty partial for the merge
        if (tid < c.g)
            a.partials[(((size_t)c.s * a.num_q_heads + c.h * c.g + tid) * a.n_splits + split) * kPartialStride] =
                -INFINITY;
        return;
    }
    const int n = lane & 15, j = lane >> 4;
    const int g = c.g;
    const int R = V.R;
    const int T = c.T, TV = c.TV;
    const int tk_tiles = c.TK / kTile;
    const int tpg = 1 << a.tpg_shift, tpp = 1 << a.tpp_shift;
    const int nch = kHeadDim * V.Bk / V.G;  // Key channels whose meta one page holds
    const int meta_tile = (8 * (lane & 15) / nch) * tpp;  // tile (in its group) whose page holds this lane's meta
    // weights 2^(x |scale| log2 e) of raw scores x = sgn q.k (sgn folded into the tables)
    const float sgn = a.scale_log2 < 0.0f ? -1.0f : 1.0f;
    const float sl2 = fabsf(a.scale_log2);
    const float thr = sl2 > 0.0f ? kLazyLog2 / sl2 : 0.0f;  // lazy-max threshold in raw units
    const int HQ = a.num_q_heads;

    const int nslots = kWaves * nvalid;
    // main range: contiguous per wave, in split-major order. Waves 0-3 (one
    // per SIMD, dispatched first) win issue over waves 4-7 on their SIMD, so
    // they take the larger share and the pair ends together.
    // In a fused step the last wave also appends, so it takes kAppendShare
    // and waves 4-6 share the rest of the younger half.
    const bool flush_step = a.fuse && T > 0 && T % R == 0;  // this step fills the Key residual (uniform)
    auto weight = [&](int wv) -> int {
        if (flush_step && wv >= kWaves - 3 && wv < kWaves - 1) return kFlushShare;
        if (flush_step && wv < 4) return 3 * kOldShare + (4 * (200 - kOldShare) - kAppendShare - kFlushShare) / 2;
        if (wv < 4) return 3 * kOldShare;
        if (!a.fuse) return 3 * (200 - kOldShare);
        return wv == kWaves - 1 ? 3 * kAppendShare : 4 * (200 - kOldShare) - kAppendShare;
    };
    auto slot_start = [&](int ws) -> int {
        const int sp = ws / kWaves, wv = ws % kWaves;
        long long before = (long long)sp * kWaves * 300;
        for (int w = 0; w < wv; ++w) before += weight(w);
        const int t = (int)((before * c.n_main) / ((long long)nslots * 300));
        if constexpr (kHalf == 4) {  // 4-tile blocks: ranges start on block boundaries
            if (ws >= nslots) return c.n_main;
            return min(c.n_main, (t + 2) & ~3);
        }
        return t;
    };
    const int wslot = split * kWaves + wave;
    const int m_begin = slot_start(wslot);
    const int m_end = slot_start(wslot + 1);
    const int n_tail = (T + kTile - 1) / kTile - c.n_main;
    // tail tiles: rank, rank + step, ...; a fused step leaves them to split 0,
    // the work group that wrote them
    // Fused step (split 0 only): without a Key flush only the tile of the
    // Value token leaving the window (t_evict) depends on the append; the
    // appending wave takes it, the other waves the rest in the prologue. A
    // flush step takes every tail tile after a barrier at the end.
    const int t_evict = (a.fuse && T - 1 >= R) ? (T - 1 - R) / kTile : -1;
    const bool skip_evict = a.fuse && !flush_step && t_evict >= 0;
    const int n_tail_dealt = n_tail - (skip_evict ? 1 : 0);
    int tail_step, tail_rank;
    if (!a.fuse) {
        tail_step = nslots;
        tail_rank = wave * nvalid + split;
    } else if (split != 0 || (!flush_step && wave == kWaves - 1)) {
        tail_step = kWaves;
        tail_rank = n_tail_dealt;  // none
    } else {
        tail_step = flush_step ? kWaves : kWaves - 1;
        tail_rank = wave;
    }
    const int my_tail = n_tail_dealt > tail_rank ? (n_tail_dealt - tail_rank + tail_step - 1) / tail_step : 0;
    auto tail_tile = [&](int k) -> int { return c.n_main + k + ((skip_evict && c.n_main + k >= t_evict) ? 1 : 0); };

    uint8_t* lt = wl + g * kRowBytes;
    float* lbias = reinterpret_cast<float*>(lt + 2 * g * kRowBytes);
    const int nr = n < g ? n : n % g;  // padding lanes mirror a real head; their results are unused
    const int lane_row = nr * 2 * kRowBytes + 16 * j;
    // 4-tile blocks (kHalf == 4, g in {1, 2, 4}): column n of the score and
    // PV products is (tile n / 4 of the block, query head n % 4), and the
    // table's B operand is block diagonal: lane (j, n) reads its head's row
    // when j == n / 4 (the lane's k block holds tile j's channels), else the
    // zero rows
    constexpr bool kQuad = kHalf == 4;
    const int nr4 = (n & 3) & (g - 1);
    const int lane_row4 = j == (n >> 2) ? nr4 * 2 * kRowBytes : 2 * g * kRowBytes + 64;
    const uint32_t lane_code_off = SLOT_BYTES * lane;
    const uint32_t lane_meta_off = 16 * NG * j;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(V.k_codes, a.code_array_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V.v_codes, a.code_array_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(V.v_meta, a.vmeta_array_bytes);
    const __amdgpu_buffer_rsrc_t rkm = make_rsrc(V.k_meta, a.kmeta_array_bytes);
    const uint16_t* ringK = V.k_ring + ((size_t)max(c.slot, 0) * H + c.h) * V.ring_elems;
    const uint16_t* ringV = V.v_ring + ((size_t)max(c.slot, 0) * H + c.h) * V.ring_elems;

    // ---- first round trip: query rows, page ids of the first two windows
    // and of the first tail tile's Key group ----
    const int base0 = (m_begin >> a.tpg_shift) << a.tpg_shift;  // windows start on a group
    int my_page = first_page(base0 + lane);
    int next_page = first_page(base0 + 64 + lane);
    const int tail0 = tail_tile(tail_rank);
    const int tail_base0 = (tail0 >> a.tpg_shift) << a.tpg_shift;
    int tail_page = my_tail > 0 ? first_page(tail_base0 + lane) : -1;
    if constexpr (kQuad) {  // this wave's zero rows
        if (lane < 2 * kRowBytes / 16)
            *reinterpret_cast<uint4*>(lt + 2 * g * kRowBytes + 64 + 16 * lane) = (uint4){0, 0, 0, 0};
    }

    Acc<NG, NB> st;
    st.init();

    // ---- tail tiles ----
    auto tail_issue = [&](int t, int tpage, TailRegs<BITS, NG>& x) {
        const int tb = (t >> a.tpg_shift) << a.tpg_shift;
        x.blk = valid_page(a, __builtin_amdgcn_readlane(tpage, t - tb));
        if (x.blk < 0) err |= KIVI_DEVERR_PAGE;  // every tail tile holds a token < T
        const int blk = max(x.blk, 0);
        const uint32_t chk = (uint32_t)blk * (uint32_t)H + (uint32_t)c.h;
        const uint32_t sub = (uint32_t)t & ((1u << a.tpp_shift) - 1u);
        const uint32_t coff = chk * (uint32_t)V.code_bytes + sub * TILE_BYTES;
        const uint32_t moff = chk * (uint32_t)V.v_meta_bytes + sub * (kTile * NG * 4);
        const int p0 = t * kTile;
#pragma unroll
        for (int k = 0; k < BITS; ++k) x.kw[k] = x.vw[k] = 0;
#pragma unroll
        for (int k = 0; k < 4 * NG; ++k) x.vm[k] = 0;
        x.ms = x.mz = (uint4){0, 0, 0, 0};
        if (t < tk_tiles) {
            if constexpr (BITS == 4) {
                const uint4 u = buf_b128(rk, lane_code_off, coff);
                x.kw[0] = u.x; x.kw[1] = u.y; x.kw[2] = u.z; x.kw[3] = u.w;
            } else {
                const uint2 u = buf_b64(rk, lane_code_off, coff);
                x.kw[0] = u.x; x.kw[1] = u.y;
            }
            const int mp = valid_page(a, __builtin_amdgcn_ds_bpermute(4 * meta_tile, tpage));
            const uint32_t mo = k_meta_off(V, c.h, mp, nch);
            x.ms = buf_b128(rkm, mo, 0);
            x.mz = buf_b128(rkm, mo + 2u * (uint32_t)nch, 0);
        } else {
            const int pk = min(p0 + n, T - 1);  // A row: token n of the tile
            // a fused step's own token comes from its input row
            const uint16_t* krow = (a.fuse && pk == T - 1)
                                       ? a.app.k_new + ((size_t)c.s * H + c.h) * kHeadDim
                                       : ringK + (size_t)(pk % R) * kHeadDim;
#pragma unroll
            for (int i = 0; i < 4; ++i) x.kr[i] = *reinterpret_cast<const uint4*>(krow + 32 * i + 8 * j);
        }
        if (p0 < TV) {
            if constexpr (BITS == 4) {
                const uint4 u = buf_b128(rv, lane_code_off, coff);
                x.vw[0] = u.x; x.vw[1] = u.y; x.vw[2] = u.z; x.vw[3] = u.w;
            } else {
                const uint2 u = buf_b64(rv, lane_code_off, coff);
                x.vw[0] = u.x; x.vw[1] = u.y;
            }
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const uint4 m = buf_b128(rm, lane_meta_off + 16 * q, moff);
                x.vm[4 * q + 0] = m.x; x.vm[4 * q + 1] = m.y; x.vm[4 * q + 2] = m.z; x.vm[4 * q + 3] = m.w;
            }
        }
        // residual Values: positions 4j..4j+3 of a channel are adjacent in the
        // ring's quads (R is a multiple of 16, so they never wrap)
        const int pq = p0 + 4 * j;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
            x.vr[tt] = *reinterpret_cast<const uint2*>(ringV + vring_index(R, pq, 16 * tt + n));
        if (a.fuse && pq <= T - 1 && T - 1 < pq + 4) {  // a fused step's own token from its input row
            const uint16_t* vrow = a.app.v_new + ((size_t)c.s * H + c.h) * kHeadDim;
            const int r = T - 1 - pq, sh16 = 16 * (r & 1);
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const uint32_t val = vrow[16 * tt + n];
                if (r < 2) x.vr[tt].x = (x.vr[tt].x & ~(0xFFFFu << sh16)) | (val << sh16);
                else x.vr[tt].y = (x.vr[tt].y & ~(0xFFFFu << sh16)) | (val << sh16);
            }
        }
    };
    auto tail_compute = [&](int t, const TailRegs<BITS, NG>& x) {
        if (x.blk < 0) return;
        const int p0 = t * kTile, pq = p0 + 4 * j;
        f4 raw;
        if (t < tk_tiles) {
            const float bias = build_table<BITS>(g, x.ms, x.mz, lq, lt, lbias, nr, sgn);
            raw = code_scores<BITS>(x.kw, lt, lane_row, bias);
        } else {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            const uint8_t* qrow = reinterpret_cast<const uint8_t*>(lq + nr * kQRow);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h8 A;
                const uint32_t ws[4] = {x.kr[i].x, x.kr[i].y, x.kr[i].z, x.kr[i].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) A[e] = (_Float16)to_f32<DT>((uint16_t)(ws[e >> 1] >> (16 * (e & 1))));
                const h8 B = *reinterpret_cast<const h8*>(qrow + 2 * (32 * i + 8 * j));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc, 0, 0, 0);
            }
            raw = acc * sgn;
        }
        // tokens at or past T take no part (weight 0, not in the max)
        float p[4], mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (pq + r < T) mx = max2(mx, raw[r]);
        st.rescale(xor_max(mx), sl2, thr);
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = (pq + r < T) ? st.weight(raw[r], sl2) : 0.0f;
        st.l_acc += (p[0] + p[1]) + (p[2] + p[3]);
        // (16-channel Value groups keep the general path: their tail tiles
        // already fill the registers)
        if (NG < 8 && p0 >= TV && p0 + kTile <= T) {  // uniform: every Value token from the residual
            h8 B;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                _Float16 hi, lo;
                split_f16(p[r], hi, lo);
                B[r] = hi;
                B[4 + r] = lo;
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                h4 A;
                if constexpr (DT == kF16) {
                    A = make_h4(x.vr[tt].x, x.vr[tt].y);
                } else {
                    const uint32_t rw[2] = {x.vr[tt].x, x.vr[tt].y};
#pragma unroll
                    for (int r = 0; r < 4; ++r) A[r] = (_Float16)to_f32<DT>((uint16_t)(rw[r >> 1] >> (16 * (r & 1))));
                }
                st.O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dup_h8(A), B, st.O[tt], 0, 0, 0);
            }
            return;
        }
        // Value token r: code (< TV), residual (< T) or masked, chosen by
        // selects (no divergent branches)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            const int gg = (16 * tt) / (kHeadDim / NG);
            const bool first_of_group = (16 * tt) % (kHeadDim / NG) == 0;
            const uint32_t rw[2] = {x.vr[tt].x, x.vr[tt].y};
            h4 A;
            h8 B;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pr = pq + r;
                const bool is_code = pr < TV, is_raw = !is_code && pr < T;
                const uint32_t mw = is_code ? x.vm[r * NG + gg] : 0u;
                if (first_of_group) st.zacc[gg] += p[r] * f16_bits_to_f32((uint16_t)(mw >> 16));
                const float code_v = (float)v_code_at<BITS>(x.vw, tt, r);
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
    };

    // ---- main tiles ----
    // Loads of a tile are unconditional (a missing page or a tile past the
    // range reads page 0 and is not computed), so a buffer is one straight
    // run of loads that the wait counts can follow. Each buffer also loads
    // the scales and zero-points of the Key group of its last tile: the only
    // group that can begin inside a buffer, as groups span >= kHalf tiles.
    struct Buf {
        TileRegs<BITS, NG> t[kHalf];
        bool ok[kHalf];
        uint4 ms, mz;
    };
    int base = base0;
    auto issue = [&](int t0, Buf& b) {
        if (t0 - base >= 64) {  // next window of page ids (loaded one window ahead)
            base += 64;
            my_page = next_page;
            next_page = page_of_tile(a, c, base + 64 + lane);
        }
#pragma unroll
        for (int e = 0; e < kHalf; ++e) {
            const int t = t0 + e;
            const int blk = valid_page(a, __builtin_amdgcn_readlane(my_page, (t - base) & 63));
            const bool mine = t >= m_begin && t < m_end;
            b.ok[e] = blk >= 0 && mine;
            if (blk < 0 && mine) err |= KIVI_DEVERR_PAGE;
            const uint32_t chk = (uint32_t)(b.ok[e] ? blk : 0) * (uint32_t)H + (uint32_t)c.h;
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
            for (int q = 0; q < NG; ++q) {
                const uint4 m = buf_b128(rm, lane_meta_off + 16 * q, moff);
                b.t[e].vm[4 * q + 0] = m.x; b.t[e].vm[4 * q + 1] = m.y;
                b.t[e].vm[4 * q + 2] = m.z; b.t[e].vm[4 * q + 3] = m.w;
            }
        }
        // Key group of tile t0 + kHalf - 1 (its pages are in the window:
        // windows start on groups)
        const int gt = ((t0 + kHalf - 1) >> a.tpg_shift) << a.tpg_shift;
        const int mp = valid_page(a, __builtin_amdgcn_ds_bpermute(4 * ((gt + meta_tile - base) & 63), my_page));
        const uint32_t mo = k_meta_off(V, c.h, mp, nch);
        b.ms = buf_b128(rkm, mo, 0);
        b.mz = buf_b128(rkm, mo + 2u * (uint32_t)nch, 0);
    };
    float bias = 0.0f;
    // Tiles are taken in pairs (slots e, e + 1 of a buffer; both in one Key
    // group, as pairs start an even number of tiles after a group start).
    auto compute = [&](const Buf& b, int t0) {
#pragma unroll
        for (int e = 0; e < kHalf; e += 2) {
            const int t = t0 + e;
            constexpr bool kPair = kHalf > 1;
            const bool oka = b.ok[e], okb = kPair ? b.ok[kPair ? e + 1 : e] : false;
            if (!oka && !okb) continue;
            if ((t & (tpg - 1)) == 0 && t != m_begin)
                bias = build_table<BITS, kFoldK>(g, b.ms, b.mz, lq, lt, lbias, nr, sgn);
            const TileRegs<BITS, NG>& ta = b.t[e];
            const TileRegs<BITS, NG>& tb = b.t[kPair ? e + 1 : e];
            const f4 ra = code_scores<BITS, kFoldK>(ta.k, lt, lane_row, bias);
            f4 rb = ra;
            if (kPair) rb = code_scores<BITS, kFoldK>(tb.k, lt, lane_row, bias);
            float mx = oka ? max4(ra) : -INFINITY;
            if (okb) mx = max2(mx, max4(rb));
            st.rescale(xor_max(mx), sl2, thr);
            float pa[4], pb[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pa[r] = oka ? st.weight(ra[r], sl2) : 0.0f;
                pb[r] = okb ? st.weight(rb[r], sl2) : 0.0f;
            }
            st.l_acc += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
            value_pair<BITS, NG, NB>(st, ta.v, ta.vm, tb.v, tb.vm, pa, pb, oka, okb);
        }
    };

    // ---- second round trip: the first main buffer and the first group's
    // meta (narrow Value groups, whose tail tiles hold many registers, finish
    // the tail first; wide ones take it after the main range) ----
    // pre: the first tail tile's registers when they were loaded ahead
    auto run_tail = [&](const TailRegs<BITS, NG>* pre) {
        for (int i = 0; i < my_tail; ++i) {
            const int t = tail_tile(tail_rank + i * tail_step);
            if (i == 0 && pre) {
                tail_compute(t, *pre);
                continue;
            }
            if (i > 0) {
                const int tb = (t >> a.tpg_shift) << a.tpg_shift;
                tail_page = page_of_tile(a, c, tb + lane);
            }
            TailRegs<BITS, NG> x;
            tail_issue(t, tail_page, x);
            tail_compute(t, x);
        }
    };
    if constexpr (NG >= 4) {
        if (!flush_step) run_tail(nullptr);
    }
    // buffers start a multiple of kHalf tiles after the window base, so
    // window boundaries fall between buffers (tiles before m_begin may ride
    // along, not computed)
    const int t_first = m_begin - ((m_begin - base0) & (kHalf - 1));

    // ---- 4-tile blocks (kQuad) ----
    // Loads of block t0 .. t0 + 3: Value codes as in a 2-tile buffer (the
    // lane's slot of each tile); Key codes of tile t0 + j only, all four slots
    // (n, 0..3) of the lane's token n, so the lane holds the token's 128
    // channels; Value metadata of tile t0 + n / 4, tokens 4j .. 4j + 3 (the
    // lane's score column); the Key group's scales and zero-points.
    struct Quad {
        uint32_t k[4][BITS];  // slot jp of tile t0 + j: channels 32 i + 8 jp .. + 7 in word i (int4)
        uint32_t v[4][BITS];  // tile t0 + e: the lane's Value slot
        uint32_t vm[4 * NG];  // [token][group] of the lane's column tile
        uint4 ms, mz;
        uint32_t okm;         // bit e: tile t0 + e is computed (uniform)
    };
    auto issue4 = [&](int t0, Quad& b) {
        if (t0 - base >= 64) {  // next window of page ids (loaded one window ahead)
            base += 64;
            my_page = next_page;
            next_page = page_of_tile(a, c, base + 64 + lane);
        }
        uint32_t coff[4], moff[4], okm = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + e;
            const int blk = valid_page(a, __builtin_amdgcn_readlane(my_page, (t - base) & 63));
            const bool mine = t >= m_begin && t < m_end;
            const bool ok = blk >= 0 && mine;
            if (blk < 0 && mine) err |= KIVI_DEVERR_PAGE;
            okm |= ok ? 1u << e : 0u;
            const uint32_t chk = (uint32_t)(ok ? blk : 0) * (uint32_t)H + (uint32_t)c.h;
            const uint32_t sub = (uint32_t)t & ((1u << a.tpp_shift) - 1u);
            coff[e] = chk * (uint32_t)V.code_bytes + sub * TILE_BYTES;
            moff[e] = chk * (uint32_t)V.v_meta_bytes + sub * (kTile * NG * 4);
            if constexpr (BITS == 4) {
                const uint4 u = buf_b128(rv, lane_code_off, coff[e]);
                b.v[e][0] = u.x; b.v[e][1] = u.y; b.v[e][2] = u.z; b.v[e][3] = u.w;
            } else {
                const uint2 u = buf_b64(rv, lane_code_off, coff[e]);
                b.v[e][0] = u.x; b.v[e][1] = u.y;
            }
        }
        b.okm = okm;
        const uint32_t kc = j == 0 ? coff[0] : j == 1 ? coff[1] : j == 2 ? coff[2] : coff[3];
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
            const uint32_t vo = kc + (uint32_t)(SLOT_BYTES * (n + 16 * jp));
            if constexpr (BITS == 4) {
                const uint4 u = buf_b128(rk, vo, 0);
                b.k[jp][0] = u.x; b.k[jp][1] = u.y; b.k[jp][2] = u.z; b.k[jp][3] = u.w;
            } else {
                const uint2 u = buf_b64(rk, vo, 0);
                b.k[jp][0] = u.x; b.k[jp][1] = u.y;
            }
        }
        const int tn = n >> 2;
        const uint32_t mo = (tn == 0 ? moff[0] : tn == 1 ? moff[1] : tn == 2 ? moff[2] : moff[3]) + lane_meta_off;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const uint4 m = buf_b128(rm, mo + 16 * q, 0);
            b.vm[4 * q + 0] = m.x; b.vm[4 * q + 1] = m.y; b.vm[4 * q + 2] = m.z; b.vm[4 * q + 3] = m.w;
        }
        // the Key group of the block (blocks never straddle a group)
        const int gt = (t0 >> a.tpg_shift) << a.tpg_shift;
        const int mp = valid_page(a, __builtin_amdgcn_ds_bpermute(4 * ((gt + meta_tile - base) & 63), my_page));
        const uint32_t mko = k_meta_off(V, c.h, mp, nch);
        b.ms = buf_b128(rkm, mko, 0);
        b.mz = buf_b128(rkm, mko + 2u * (uint32_t)nch, 0);
    };
    const uint32_t diag_w[4] = {(n >> 2) == 0 ? ~0u : 0u, (n >> 2) == 1 ? ~0u : 0u, (n >> 2) == 2 ? ~0u : 0u,
                                (n >> 2) == 3 ? ~0u : 0u};
    auto diag = [&](uint32_t w) -> h8 {  // w in the dword of the lane's column tile, zeros elsewhere
        return make_h8(w & diag_w[0], w & diag_w[1], w & diag_w[2], w & diag_w[3]);
    };
    auto compute4 = [&](const Quad& b, int t0) {
        if ((t0 & (tpg - 1)) == 0 && t0 != t_first)
            bias = build_table<BITS, kFoldK>(g, b.ms, b.mz, lq, lt, lbias, nr4, sgn);
        const bool okc = (b.okm >> (n >> 2)) & 1u;
        // scores of column (tile n / 4, head n % 4), tokens 4j .. 4j + 3:
        // one k-step per 8 channels (k = 8 tile + e), two chains (table hi, lo)
        f4 sh = {bias, bias, bias, bias}, sl = {0.f, 0.f, 0.f, 0.f};
        const uint8_t* trow = lt + lane_row4;
#pragma unroll
        for (int c8 = 0; c8 < 16; ++c8) {
            const int jp = c8 & 3, i = c8 >> 2;
            h8 A;
            if constexpr (BITS == 4) {
                const uint32_t w = b.k[jp][i], w8 = w >> 8;
                A = make_h8(magic_pair(w, 0x000F000Fu), magic_pair(w, 0x00F000F0u), magic_pair(w8, 0x000F000Fu),
                            magic_pair(w8, 0x00F000F0u));
            } else {
                const uint32_t x = b.k[jp][i >> 1], xs = (i & 1) ? x >> 8 : x;
                A = make_h8(magic_pair(xs, 0x00030003u), magic_pair(xs, 0x000C000Cu), magic_pair(xs, 0x00300030u),
                            magic_pair(xs, 0x00C000C0u));
            }
            const h8 bh = *reinterpret_cast<const h8*>(trow + 16 * c8);
            const h8 bl = *reinterpret_cast<const h8*>(trow + kRowBytes + 16 * c8);
            sh = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh, sh, 0, 0, 0);
            sl = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl, sl, 0, 0, 0);
        }
        const f4 raw = sh + sl;
        // the head's largest score over the block: lanes n + 16 r, and the
        // four tiles n % 4 + 4 e
        float mx = okc ? max4(raw) : -INFINITY;
        mx = xor_max(mx);
        mx = max2(mx, row_ror<4>(mx));
        mx = max2(mx, row_ror<8>(mx));
        st.rescale(mx, sl2, thr);
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = okc ? st.weight(raw[r], sl2) : 0.0f;
        const h2 pp01 = {(_Float16)p[0], (_Float16)p[1]};  // round to nearest (one v_cvt_pk_f16_f32)
        const h2 pp23 = {(_Float16)p[2], (_Float16)p[3]};
        const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
        st.l_acc = __builtin_amdgcn_fdot2(pp23, one, __builtin_amdgcn_fdot2(pp01, one, st.l_acc, false), false);
        // Value weights W = p * scale / F (F: the place value of tokens 2, 3's
        // fields), zero-point sums, and the PV B operands (the lane's dword of
        // k-step h holds its tokens 2h, 2h + 1)
        constexpr float kF23 = (BITS == 4) ? 0.0625f : 0.25f;
        const h2 f23 = {(_Float16)kF23, (_Float16)kF23};
        h8 Bq[NG][NB][2];
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            const uint32_t m0 = okc ? b.vm[0 * NG + gg] : 0u, m1 = okc ? b.vm[1 * NG + gg] : 0u;
            const uint32_t m2 = okc ? b.vm[2 * NG + gg] : 0u, m3 = okc ? b.vm[3 * NG + gg] : 0u;
            const h2 w01 = pp01 * __builtin_bit_cast(h2, lo_halves(m0, m1));
            const h2 w23 = (pp23 * f23) * __builtin_bit_cast(h2, lo_halves(m2, m3));
            float z = __builtin_amdgcn_fdot2(pp01, __builtin_bit_cast(h2, __builtin_amdgcn_perm(m1, m0, 0x07060302u)),
                                             st.zacc[gg], false);
            st.zacc[gg] = __builtin_amdgcn_fdot2(pp23, __builtin_bit_cast(h2, __builtin_amdgcn_perm(m3, m2, 0x07060302u)),
                                                 z, false);
            // the Value codes enter as 1024 + field (int4 and int2 alike): the
            // 1024 offsets come out later as 1024 times the weights' sum
            st.wsum[gg][0] =
                __builtin_amdgcn_fdot2(w23, one, __builtin_amdgcn_fdot2(w01, one, st.wsum[gg][0], false), false);
            Bq[gg][0][0] = diag(__builtin_bit_cast(uint32_t, w01));
            Bq[gg][0][1] = diag(__builtin_bit_cast(uint32_t, w23));
            if constexpr (NB == 2) {  // odd channel tiles: fields 4 places up (factor 1/16)
                const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
                const h2 w01s = w01 * k16, w23s = w23 * k16;
                st.wsum[gg][1] =
                    __builtin_amdgcn_fdot2(w23s, one, __builtin_amdgcn_fdot2(w01s, one, st.wsum[gg][1], false), false);
                Bq[gg][NB - 1][0] = diag(__builtin_bit_cast(uint32_t, w01s));
                Bq[gg][NB - 1][1] = diag(__builtin_bit_cast(uint32_t, w23s));
            }
        }
        // PV: channel tile tt, k-step h: k = 8 jj + 2 e + q holds tile e's
        // token 4 jj + 2 h + q (jj: the lane's k block)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            const int gg = (16 * tt) / (kHeadDim / NG);
            uint32_t a0[4], a1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (BITS == 4) {
                    const uint32_t w = b.v[e][tt >> 1], ws = (tt & 1) ? w >> 8 : w;
                    a0[e] = magic_pair(ws, 0x000F000Fu);
                    a1[e] = magic_pair(ws, 0x00F000F0u);
                } else {
                    const uint32_t x = b.v[e][tt >> 2], xs = (tt & 2) ? x >> 8 : x;
                    a0[e] = magic_pair(xs, (tt & 1) ? 0x00300030u : 0x00030003u);
                    a1[e] = magic_pair(xs, (tt & 1) ? 0x00C000C0u : 0x000C000Cu);
                }
            }
            st.O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(make_h8(a0[0], a0[1], a0[2], a0[3]),
                                                              Bq[gg][tt % NB][0], st.O[tt], 0, 0, 0);
            st.O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(make_h8(a1[0], a1[1], a1[2], a1[3]),
                                                              Bq[gg][tt % NB][1], st.O[tt], 0, 0, 0);
        }
    };
    // back to one column per query head: sums over the block's four tiles
    auto quad_to_heads = [&]() {
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.O[tt][r] = quad_fold(st.O[tt][r]);
        st.l_acc = quad_fold(st.l_acc);
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            st.zacc[gg] = quad_fold(st.zacc[gg]);
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) st.wsum[gg][vb] = quad_fold(st.wsum[gg][vb]);
        }
    };

    Buf ba, bb;
    Quad qa, qb;
    uint4 ms0 = {0, 0, 0, 0}, mz0 = {0, 0, 0, 0};
    if (m_begin < m_end) {
        if constexpr (kQuad) {
            issue4(t_first, qa);
        } else {
            issue(t_first, ba);
            const int mp = valid_page(a, __builtin_amdgcn_ds_bpermute(4 * meta_tile, my_page));
            const uint32_t mo = k_meta_off(V, c.h, mp, nch);
            ms0 = buf_b128(rkm, mo, 0);
            mz0 = buf_b128(rkm, mo + 2u * (uint32_t)nch, 0);
        }
    }
    // the tile of the Value token that leaves the window, taken by the wave
    // that wrote it (its own stores complete first)
    auto evict_tile = [&]() {
        __builtin_amdgcn_s_waitcnt(0);
        const int tb = (t_evict >> a.tpg_shift) << a.tpg_shift;
        const int tpage = page_of_tile(a, c, tb + lane);
        TailRegs<BITS, NG> x;
        tail_issue(t_evict, tpage, x);
        tail_compute(t_evict, x);
    };
    // Fused step: split 0 appends this step's token with three waves while the
    // others stream (wave 7: Value eviction and residual writes; waves 5 and 6:
    // the Key flush when the residual fills). Main tiles lie below the old
    // Value boundary, so nothing they read is written here.
    if (a.fuse && split == 0) {
        if (wave == kWaves - 1) {
            append_token_value_wave<BITS, DT>(a.app, c.s, c.h, lane);
            if (!kQuad && skip_evict) evict_tile();  // 4-tile blocks: after the main range
        } else if (wave >= kWaves - 3) {
            // the flush is on the step's critical path: the flush waves, younger
            // than the streaming wave on their SIMD, take issue priority for it
            __builtin_amdgcn_s_setprio(3);
            append_token_key_wave<BITS, DT>(a.app, c.s, c.h, wave - (kWaves - 3), lane);
            __builtin_amdgcn_s_setprio(0);
        }
    }
    if constexpr (kQuad) {
        // tail tiles first (per-head columns), then the state moves to the
        // block columns: lanes n >= 4 clear their sums, so that the fold over
        // the four tiles counts the tail once (a flush step reads its tail
        // only after the flush)
        if (kTailFirst && !flush_step) {
            run_tail(nullptr);
            if (n >= 4) {
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) st.O[tt] = (f4){0.f, 0.f, 0.f, 0.f};
                st.l_acc = 0.0f;
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) {
                    st.zacc[gg] = 0.0f;
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) st.wsum[gg][vb] = 0.0f;
                }
            }
        }
        if (m_begin < m_end) {
            bias = build_table<BITS, kFoldK>(g, qa.ms, qa.mz, lq, lt, lbias, nr4, sgn);
            int it = 0;
            if constexpr (kQuadBuffers == 3) {
                Quad qc;
                issue4(t_first + 4, qb);
                for (int t0 = t_first; t0 < m_end; t0 += 12) {
                    issue4(t0 + 8, qc);
                    compute4(qa, t0);
                    if (t0 + 4 >= m_end) break;
                    issue4(t0 + 12, qa);
                    compute4(qb, t0 + 4);
                    if (t0 + 8 >= m_end) break;
                    issue4(t0 + 16, qb);
                    compute4(qc, t0 + 8);
                    if (++it == 3) {
                        it = 0;
                        st.template flush_offsets<BITS>();
                    }
                }
            } else {
                for (int t0 = t_first; t0 < m_end; t0 += 8) {
                    issue4(t0 + 4, qb);
                    compute4(qa, t0);
                    if (t0 + 4 >= m_end) break;
                    issue4(t0 + 8, qa);
                    compute4(qb, t0 + 4);
                    // int2 fields are smaller against the 1024 offset: flush twice as often
                    if (++it == (BITS == 2 ? flush_period<kHalf>() / 2 : flush_period<kHalf>())) {
                        it = 0;
                        st.template flush_offsets<BITS>();
                    }
                }
            }
        }
        quad_to_heads();
        if (a.fuse && split == 0 && wave == kWaves - 1 && skip_evict) evict_tile();
        if (!kTailFirst && !flush_step) run_tail(nullptr);
    } else if (m_begin < m_end) {
        bias = build_table<BITS, kFoldK>(g, ms0, mz0, lq, lt, lbias, nr, sgn);
        int it = 0;
        for (int t0 = t_first; t0 < m_end; t0 += 2 * kHalf) {
            issue(t0 + kHalf, bb);
            compute(ba, t0);
            if (t0 + kHalf >= m_end) break;
            issue(t0 + 2 * kHalf, ba);
            compute(bb, t0 + kHalf);
            // int2 fields are smaller against the 1024 offset: flush twice as often
            if (++it == (BITS == 2 ? (flush_period<kHalf>() + 1) / 2 : flush_period<kHalf>())) {
                it = 0;
                st.template flush_offsets<BITS>();
            }
        }
    }

    // Wide Value groups take their tail tiles after the main range, so every
    // wave starts streaming at once (a fused step gained 1.4 us per call).
    // The tail reads nothing this launch
    // writes but the evicted token's tile, which stays with the appending wave.
    if constexpr (NG < 4 && !kQuad) {
        if (!flush_step) run_tail(nullptr);
    }
    if (flush_step) {
        // the append's stores complete, then split 0 takes the tail tiles,
        // which hold what it wrote (the step's own token comes from its row)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        run_tail(nullptr);
    }
    // ---------------- merge the waves in LDS ----------------
    {
        const float l_tot = xor_sum(st.l_acc);
        float zt[NG][NB];
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            const float z = xor_sum(st.zacc[gg]);
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) zt[gg][vb] = z - 1024.0f * xor_sum(st.wsum[gg][vb]);
        }
        __syncthreads();  // every wave is done with its LDS rows
        float* sm_m = reinterpret_cast<float*>(smem);  // [kWaves][g]
        float* sm_l = sm_m + kWaves * g;               // [kWaves][g]
        float* sm_o = sm_l + kWaves * g;               // [kWaves][g][128]
        if (n < g) {
            if (j == 0) {  // the running max in log2 units
                sm_m[wave * g + n] = st.m_run == -INFINITY ? -INFINITY : st.m_run * sl2;
                sm_l[wave * g + n] = l_tot;
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int chn = 16 * tt + 4 * j + r;
                    sm_o[(wave * g + n) * kHeadDim + chn] = st.O[tt][r] + zt[chn / (kHeadDim / NG)][tt % NB];
                }
        }
        __syncthreads();
    }
    if (err != 0 && lane == 0) report_error(V.status, err);
    const float* sm_m = reinterpret_cast<const float*>(smem);
    const float* sm_l = sm_m + kWaves * g;
    const float* sm_o = sm_l + kWaves * g;
    for (int idx = tid; idx < g * kHeadDim; idx += kThreads) {
        const int hn = idx / kHeadDim, chn = idx % kHeadDim;
        float mstar = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm_m[w * g + hn]);
        float lsum = 0.0f, osum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm_m[w * g + hn];
            const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - mstar);
            lsum += f * sm_l[w * g + hn];
            osum += f * sm_o[(w * g + hn) * kHeadDim + chn];
        }
        if (a.n_splits == 1) {  // no split anywhere: final output
            a.out[((size_t)c.s * HQ + c.h * g + hn) * kHeadDim + chn] = from_f32<DT>(lsum > 0.0f ? osum / lsum : 0.0f);
        } else {
            float* part = a.partials + (((size_t)c.s * HQ + c.h * g + hn) * a.n_splits + split) * kPartialStride;
            if (chn == 0) {
                part[0] = mstar;
                part[1] = lsum;
            }
            part[4 + chn] = osum;
        }
    }
}

// Merge of the split partials of one (sequence, query head): one work group
// of 128 threads (one per channel), one pass with a running maximum:
// m = max m_i, l = sum l_i 2^(m_i - m), o = sum o_i 2^(m_i - m) / l.
// Splits without work left m_i = -inf. A separate launch, so the partials of
// every split are visible.
template <int DT>
__global__ __launch_bounds__(kHeadDim) void merge_kernel(DecodeArgs a) {
    constexpr int kBatch = 8;
    const int row = blockIdx.x;  // s * H_Q + hq
    const int chn = threadIdx.x;
    const int ns = a.n_splits;
    const float* pbase = a.partials + (size_t)row * ns * kPartialStride;
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    for (int i0 = 0; i0 < ns; i0 += kBatch) {
        float mi[kBatch], li[kBatch], oi[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {  // independent loads, issued together
            const float* pp = pbase + (size_t)min(i0 + k, ns - 1) * kPartialStride;
            mi[k] = i0 + k < ns ? pp[0] : -INFINITY;
            li[k] = pp[1];
            oi[k] = pp[4 + chn];
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (mi[k] == -INFINITY) continue;
            const float mn = fmaxf(m, mi[k]);
            const float fo = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
            const float fi = __builtin_amdgcn_exp2f(mi[k] - mn);
            l = l * fo + li[k] * fi;
            o = o * fo + oi[k] * fi;
            m = mn;
        }
    }
    a.out[(size_t)row * kHeadDim + chn] = from_f32<DT>(l > 0.0f ? o / l : 0.0f);
}

template <int BITS, int DT, int NG>
void launch_ng(const DecodeArgs& a, int tpg, dim3 grid, size_t lds, hipStream_t st) {
    dim3 block(kThreads);
    constexpr int kMax = max_buffer_tiles<NG>();
    const int kh = std::min(kMax, tpg);
    // 4-tile blocks: at most 4 query heads per KV head (a power of two), Key
    // groups of 4 tiles or more, Value groups of 64 channels or more
    const bool quad = tpg >= 4 && (a.gqa == 1 || a.gqa == 2 || a.gqa == 4);
    if (NG <= 2 && quad)
        hipLaunchKernelGGL((decode_kernel<BITS, DT, NG, (NG <= 2 ? 4 : 1)>), grid, block, lds, st, a);
    else if (kh >= 2 && kMax >= 2)
        hipLaunchKernelGGL((decode_kernel<BITS, DT, NG, (kMax >= 2 ? 2 : 1)>), grid, block, lds, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<BITS, DT, NG, 1>), grid, block, lds, st, a);
}

template <int BITS, int DT>
void launch_bits_dt(const DecodeArgs& a, int ng, int tpg, dim3 grid, size_t lds, hipStream_t st) {
    switch (ng) {
        case 1: launch_ng<BITS, DT, 1>(a, tpg, grid, lds, st); break;
        case 2: launch_ng<BITS, DT, 2>(a, tpg, grid, lds, st); break;
        case 4: launch_ng<BITS, DT, 4>(a, tpg, grid, lds, st); break;
        default: launch_ng<BITS, DT, 8>(a, tpg, grid, lds, st); break;
    }
}

}  // namespace

namespace {
int launch_decode_args(DecodeArgs& a, const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                       const int32_t* slot_ids, const int32_t* seq_lens, const int32_t* block_table,
                       int bt_stride, float softmax_scale, void* out, float* partials,
                       const DecodePlan& plan, size_t lds, void* stream);
}  // namespace

int launch_decode(const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                  const int32_t* slot_ids, const int32_t* seq_lens, const int32_t* block_table,
                  int bt_stride, float softmax_scale, void* out, float* partials,
                  const DecodePlan& plan, void* stream, int len_add) {
    DecodeArgs a{};
    a.fuse = 0;
    a.len_add = len_add;
    return launch_decode_args(a, v, num_seqs, num_q_heads, q, slot_ids, seq_lens, block_table, bt_stride,
                              softmax_scale, out, partials, plan, plan.lds_bytes, stream);
}

int launch_decode_step(const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                       const int32_t* slot_ids, const int32_t* seq_lens_before, const void* k_new,
                       const void* v_new, const int32_t* block_table, int bt_stride, float softmax_scale,
                       void* out, float* partials, const DecodePlan& plan, void* stream) {
    DecodeArgs a{};
    a.fuse = 1;
    a.app.v = v;
    a.app.slot_ids = slot_ids;
    a.app.seq_lens_before = seq_lens_before;
    a.app.cu_new = nullptr;  // one row per sequence, in sequence order
    a.app.k_new = static_cast<const uint16_t*>(k_new);
    a.app.v_new = static_cast<const uint16_t*>(v_new);
    a.app.block_table = block_table;
    a.app.bt_stride = bt_stride;
    a.app.mode = 0;
    return launch_decode_args(a, v, num_seqs, num_q_heads, q, slot_ids, seq_lens_before, block_table, bt_stride,
                              softmax_scale, out, partials, plan, plan.lds_bytes, stream);
}

namespace {
int launch_decode_args(DecodeArgs& a, const CacheView& v, int num_seqs, int num_q_heads, const void* q,
                       const int32_t* slot_ids, const int32_t* seq_lens, const int32_t* block_table,
                       int bt_stride, float softmax_scale, void* out, float* partials,
                       const DecodePlan& plan, size_t lds, void* stream) {
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
    a.tpg_shift = __builtin_ctz((unsigned)(v.G / kTile));
    a.tpp_shift = __builtin_ctz((unsigned)(v.Bk / kTile));
    a.code_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.code_bytes);
    a.vmeta_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.v_meta_bytes);
    a.kmeta_array_bytes = (uint32_t)((uint64_t)v.num_blocks * v.H * v.k_meta_bytes);
    a.out = static_cast<uint16_t*>(out);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int ng = kHeadDim / v.Gv;
    dim3 grid((unsigned)(num_seqs * v.H * plan.n_splits));
    const int tpg = v.G / kTile;
    if (v.bits == 4) {
        if (v.dtype == kF16) launch_bits_dt<4, kF16>(a, ng, tpg, grid, lds, st);
        else launch_bits_dt<4, kBF16>(a, ng, tpg, grid, lds, st);
    } else {
        if (v.dtype == kF16) launch_bits_dt<2, kF16>(a, ng, tpg, grid, lds, st);
        else launch_bits_dt<2, kBF16>(a, ng, tpg, grid, lds, st);
    }
    if (plan.n_splits > 1) {
        dim3 mgrid((unsigned)(num_seqs * num_q_heads));
        if (v.dtype == kF16) hipLaunchKernelGGL((merge_kernel<kF16>), mgrid, dim3(kHeadDim), 0, st, a);
        else hipLaunchKernelGGL((merge_kernel<kBF16>), mgrid, dim3(kHeadDim), 0, st, a);
    }
    return (int)hipGetLastError();
}
}  // namespace

// Split partials of kivi_decode_attention_noalloc: one array per device,
// held until the process ends, shared by every call on that device.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

int noalloc_scratch(float** out) {
    static std::mutex mu;
    static float* ptrs[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        // the device's own copy of the array (the current device is `dev`)
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        ptrs[dev] = static_cast<float*>(p);
    }
    *out = ptrs[dev];
    return 0;
}

size_t decode_lds_bytes(int g) {
    return std::max((size_t)kWaves * wave_lds_bytes(g), (size_t)merge_lds_bytes(g));
}

}  // namespace kivi
