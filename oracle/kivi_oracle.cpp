// KIVI oracle: a plain, slow, scalar CPU implementation of KIVI-style
// KV-cache quantisation and of attention over the quantised cache.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
// this file. Only the test suite, the smoke check and the CPU-baseline leg of
// the benchmark use it. It shares no code, header, table or helper with the
// HIP library: it is written from the method's description alone.
//
// Build: g++ -std=c++17 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
// (no -march flags: x86-64 SSE2 scalar float, IEEE single rounding, no FMA).
//
// Sources ("pages") followed here:
//  * "4.4 KV Cache 量化" (infra-guide, module 4, chapter 4):
//      - section 1: the KV memory formula M_KV = 2 L B T H_KV d b;
//      - section 2: attention P = softmax(Q K^T / sqrt(d)), output P V;
//      - section 3.1: Key grouped per channel along G consecutive tokens, Value
//        grouped per token along channels, min/max asymmetric mapping inside a
//        group;
//      - section 3.2: full-precision residual; Key tokens are quantised in a
//        batch once enough have accumulated, Value keeps a sliding window of
//        the newest tokens and quantises the oldest one as each new one comes;
//      - section 4: the FP8 cache (E4M3 on ROCm) with per-tensor or per-KV-head
//        scales.
//  * "给 KV cache 减肥" (ai-reference-codex, section 3.1): each K/V pair is
//    compressed before it is written and restored before the query uses it.
// Where the pages leave a constant open (rounding, scale formula, dtypes) the
// oracle takes: fp32 min/max, scale = (max-min)/(2^b-1), scale and zero-point
// stored as fp16 (round to nearest even), codes computed against the stored
// fp16 parameters with IEEE single-precision subtract and divide, round half
// to even, clamp to [0, 2^b-1]; -0 is read as +0.
//
// Every function below names the passage it follows.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <vector>
#include <thread>
#include <atomic>
#include <algorithm>

namespace {

// ---------------------------------------------------------------------------
// Number formats. IEEE 754 binary16 and bfloat16, written from the format
// definitions (sign, biased exponent, fraction), rounding to nearest even.
// ---------------------------------------------------------------------------

float bits_to_f32(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
uint32_t f32_to_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

// binary16 -> binary32 (exact).
float f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t exp = (h >> 10) & 0x1fu;
    uint32_t frac = h & 0x3ffu;
    if (exp == 0) {
        // zero or subnormal: value = frac * 2^-24, exact in binary32
        float mag = (float)frac * bits_to_f32(0x33800000u);  // 2^-24
        return sign ? -mag : mag;
    }
    if (exp == 31) return bits_to_f32(sign | 0x7f800000u | (frac << 13));
    return bits_to_f32(sign | ((exp + 112u) << 23) | (frac << 13));
}

// binary32 -> binary16, round to nearest, ties to even (normal, subnormal,
// overflow to infinity).
uint16_t f32_to_f16(float f) {
    uint32_t x = f32_to_bits(f);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u)  // inf / nan
        return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
    uint32_t e = ax >> 23;                     // biased binary32 exponent
    if (e >= 113) {                            // >= 2^-14: binary16 normal range
        uint32_t frac = ax & 0x7fffffu;
        uint32_t h = ((e - 112u) << 10) | (frac >> 13);
        uint32_t rem = frac & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;  // carry may reach inf
        if (h >= 0x7c00u) h = 0x7c00u;
        return (uint16_t)(sign | h);
    }
    if (ax < 0x33000000u) return sign;        // below 2^-25 (2^-25 itself ties to 0)
    // subnormal result: k * 2^-24
    uint32_t m = (ax & 0x7fffffu) | 0x800000u; // 24-bit significand
    uint32_t shift = 126u - e;                 // 14 .. 24
    uint32_t k = m >> shift;
    uint32_t rem = m & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (k & 1u))) k += 1u;
    return (uint16_t)(sign | k);               // k == 0x400 is the smallest normal
}

// bfloat16 -> binary32 (exact): the upper half of a binary32.
float bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

enum { DT_F16 = 0, DT_BF16 = 1 };

float load_elem(uint16_t raw, int dtype) {
    return dtype == DT_BF16 ? bf16_to_f32(raw) : f16_to_f32(raw);
}

// ---------------------------------------------------------------------------
// Group quantiser: min/max asymmetric mapping inside one group
// ("4.4 KV Cache 量化", section 3.1, last paragraph: the in-group encoding is
// an asymmetric map built from the group's minimum and maximum).
// ---------------------------------------------------------------------------

// Quantise n values x[i*stride] to b-bit codes with one (scale, zero) pair.
void quantize_group(const float* x, long n, long stride, int bits,
                    uint8_t* codes, long code_stride, uint16_t* s16_out, uint16_t* z16_out) {
    const float qmax = (float)((1 << bits) - 1);
    // 1. read in fp32, -0 read as +0
    // 2. group minimum and maximum
    float mn = 0.0f, mx = 0.0f;
    for (long i = 0; i < n; ++i) {
        float v = x[i * stride];
        if (v == 0.0f) v = 0.0f;
        if (i == 0 || v < mn) mn = v;
        if (i == 0 || v > mx) mx = v;
    }
    // 3. scale = (max - min) / (2^b - 1), IEEE single subtract and divide
    float range = mx - mn;
    float scale32 = range / qmax;
    // 4. stored parameters: fp16 scale and fp16 zero-point (= group minimum)
    uint16_t s16 = f32_to_f16(scale32);
    uint16_t z16 = f32_to_f16(mn);
    *s16_out = s16;
    *z16_out = z16;
    // 5. codes against the stored fp16 parameters
    float S = f16_to_f32(s16);
    float Z = f16_to_f32(z16);
    for (long i = 0; i < n; ++i) {
        float v = x[i * stride];
        if (v == 0.0f) v = 0.0f;
        uint8_t q = 0;
        if (S != 0.0f) {
            float diff = v - Z;
            float t = diff / S;
            float r = std::nearbyint(t);           // default mode: ties to even
            if (r < 0.0f) r = 0.0f;
            if (r > qmax) r = qmax;
            q = (uint8_t)r;
        }
        codes[i * code_stride] = q;
    }
}

// Restore one element: x_hat = code * S + Z, two IEEE single roundings, no FMA
// ("给 KV cache 减肥", section 3.1: restored before the query multiplies it).
float dequant(uint8_t code, uint16_t s16, uint16_t z16) {
    float S = f16_to_f32(s16);
    float Z = f16_to_f32(z16);
    float prod = (float)code * S;
    float r = prod + Z;
    return r;
}

// ---------------------------------------------------------------------------
// Per-sequence cache (one layer, one request, all KV heads).
// "4.4 KV Cache 量化", section 3.2: Key tokens wait in a full-precision
// residual and are quantised together once R of them have accumulated (R a
// multiple of the Key group G, so the flush covers R/G whole groups). Value
// keeps the newest R tokens in full precision; each arriving token pushes the
// oldest one out, and that token is quantised per token over channel groups
// of Gv (section 3.1).
// The raw stream of every appended token is kept; tokens at positions not yet
// quantised are the residual.
// Value flush variant (vflush = 1): section 3.2 fixes the sliding Value
// window above and leaves open a cache that empties its Value residual when
// the Key residual flushes. Read plainly: at every Key flush the same R tokens
// also leave the Value residual, each still quantised per token over channel
// groups of Gv (section 3.1), so Keys and Values share one boundary
// TV = TK = R floor(T/R).
// ---------------------------------------------------------------------------

struct SeqCache {
    int H, d, bits, G, Gv, R, dtype, Tmax;
    int vflush;   // 0: sliding Value window; 1: Values flush with the Keys
    int T = 0;    // tokens appended
    int TK = 0;   // Key tokens quantised (a multiple of R)
    int TV = 0;   // Value tokens quantised (max(0, T - R); TK when vflush)
    std::vector<uint16_t> k_raw, v_raw;  // [H][Tmax][d] input bits
    std::vector<uint8_t> k_code, v_code; // [H][Tmax][d] one code per element
    std::vector<uint16_t> k_s, k_z;      // [H][Tmax/G][d]
    std::vector<uint16_t> v_s, v_z;      // [H][Tmax][d/Gv]

    SeqCache(int H_, int d_, int bits_, int G_, int Gv_, int R_, int dtype_, int Tmax_, int vflush_)
        : H(H_), d(d_), bits(bits_), G(G_), Gv(Gv_), R(R_), dtype(dtype_), Tmax(Tmax_), vflush(vflush_),
          k_raw((size_t)H_ * Tmax_ * d_), v_raw((size_t)H_ * Tmax_ * d_),
          k_code((size_t)H_ * Tmax_ * d_), v_code((size_t)H_ * Tmax_ * d_),
          k_s((size_t)H_ * (Tmax_ / G_ + 1) * d_), k_z((size_t)H_ * (Tmax_ / G_ + 1) * d_),
          v_s((size_t)H_ * Tmax_ * (d_ / Gv_)), v_z((size_t)H_ * Tmax_ * (d_ / Gv_)) {}

    size_t tok(int h, int t) const { return ((size_t)h * Tmax + t) * d; }

    // Quantise Value token t of head h: one group per Gv consecutive channels.
    void quantize_value_token(int h, int t) {
        std::vector<float> x(d);
        for (int c = 0; c < d; ++c) x[c] = load_elem(v_raw[tok(h, t) + c], dtype);
        int ng = d / Gv;
        for (int g = 0; g < ng; ++g) {
            size_t m = ((size_t)h * Tmax + t) * ng + g;
            quantize_group(&x[g * Gv], Gv, 1, bits, &v_code[tok(h, t) + g * Gv], 1, &v_s[m], &v_z[m]);
        }
    }

    // Quantise Key group j of head h: for each channel, G consecutive tokens.
    void quantize_key_group(int h, int j) {
        std::vector<float> x(G);
        for (int c = 0; c < d; ++c) {
            for (int i = 0; i < G; ++i) x[i] = load_elem(k_raw[tok(h, j * G + i) + c], dtype);
            std::vector<uint8_t> q(G);
            size_t m = ((size_t)h * (Tmax / G + 1) + j) * d + c;
            quantize_group(x.data(), G, 1, bits, q.data(), 1, &k_s[m], &k_z[m]);
            for (int i = 0; i < G; ++i) k_code[tok(h, j * G + i) + c] = q[i];
        }
    }

    // Append one token (all heads): k, v are [H][d] raw bits.
    // Order: Value eviction of the token leaving the window (sliding window
    // only), then the new token enters the residual, then the Key flush if
    // the residual is full (with the vflush variant, the Value flush of the
    // same R tokens).
    void append_one(const uint16_t* k, const uint16_t* v) {
        int t = T;
        for (int h = 0; h < H; ++h) {
            if (!vflush && t >= R) quantize_value_token(h, t - R);
            std::memcpy(&k_raw[tok(h, t)], k + (size_t)h * d, d * sizeof(uint16_t));
            std::memcpy(&v_raw[tok(h, t)], v + (size_t)h * d, d * sizeof(uint16_t));
        }
        if (!vflush && t >= R) TV = t - R + 1;
        if ((t + 1) % R == 0) {
            for (int h = 0; h < H; ++h)
                for (int j = (t + 1 - R) / G; j < (t + 1) / G; ++j) quantize_key_group(h, j);
            TK = t + 1;
            if (vflush) {
                for (int h = 0; h < H; ++h)
                    for (int p = t + 1 - R; p <= t; ++p) quantize_value_token(h, p);
                TV = t + 1;
            }
        }
        T = t + 1;
    }

    // Reconstructed Key / Value element: the restored code if quantised, else
    // the residual's full-precision value.
    float k_tilde(int h, int t, int c) const {
        if (t < TK) {
            size_t m = ((size_t)h * (Tmax / G + 1) + t / G) * d + c;
            return dequant(k_code[tok(h, t) + c], k_s[m], k_z[m]);
        }
        return load_elem(k_raw[tok(h, t) + c], dtype);
    }
    float v_tilde(int h, int t, int c) const {
        if (t < TV) {
            size_t m = ((size_t)h * Tmax + t) * (d / Gv) + c / Gv;
            return dequant(v_code[tok(h, t) + c], v_s[m], v_z[m]);
        }
        return load_elem(v_raw[tok(h, t) + c], dtype);
    }
};

// ---------------------------------------------------------------------------
// FP8 KV cache ("4.4 KV Cache 量化", section 4: the cache is stored as FP8;
// ROCm supports the E4M3 format; a scale brings the values into FP8's range,
// one per tensor or one per KV head, and is 1.0 when uncalibrated; section
// 4.5 and "给 KV cache 减肥" section 3: the stored value is restored before
// attention uses it). No groups and no residual: every token is encoded as it
// is appended.
// Readings: E4M3 is the OCP "E4M3FN" layout (sign, 4 exponent bits with bias
// 7, 3 fraction bits, no infinities, S.1111.111 is NaN, largest finite 448);
// a stored value is y = fl32(x / scale), saturated to [-448, 448] and rounded
// to the nearest E4M3 value (ties to the even code); the restored value is
// fl32(fp8 value * scale).
// ---------------------------------------------------------------------------

// E4M3 code -> binary32 (exact), from the layout above.
float e4m3_value(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? m * std::ldexp(1.0, -9) : (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
    return (float)(sign ? -mag : mag);
}

// The 256 values, built once from e4m3_value.
const std::vector<float>& e4m3_table() {
    static const std::vector<float> t = [] {
        std::vector<float> v(256);
        for (int c = 0; c < 256; ++c) v[c] = e4m3_value((uint8_t)c);
        return v;
    }();
    return t;
}
float e4m3_to_f32(uint8_t c) { return e4m3_table()[c]; }

// binary32 -> E4M3: saturate, then the nearest of the non-negative finite
// values (codes 0..0x7E, increasing with the code), ties to the even code,
// then the sign. NaN -> 0x7F.
uint8_t f32_to_e4m3(float y) {
    if (y != y) return 0x7F;
    uint8_t sign = std::signbit(y) ? 0x80 : 0x00;
    float a = std::fabs(y);
    if (a > 448.0f) a = 448.0f;
    const float* v = e4m3_table().data();
    int hi = (int)(std::lower_bound(v, v + 0x7F, a) - v);  // first value >= a
    int best = hi;
    if (hi > 0) {
        double below = (double)a - v[hi - 1], above = (double)v[hi] - a;
        if (below < above || (below == above && ((hi - 1) & 1) == 0)) best = hi - 1;
    }
    return (uint8_t)(sign | best);
}

struct Fp8SeqCache {
    int H, d, dtype, Tmax;
    int T = 0;
    std::vector<float> ks, vs;              // [H] scales (one value repeated per tensor)
    std::vector<uint8_t> k_code, v_code;    // [H][Tmax][d]

    Fp8SeqCache(int H_, int d_, int dtype_, int Tmax_, const float* k_scales, const float* v_scales, int per_head)
        : H(H_), d(d_), dtype(dtype_), Tmax(Tmax_), ks(H_), vs(H_),
          k_code((size_t)H_ * Tmax_ * d_), v_code((size_t)H_ * Tmax_ * d_) {
        for (int h = 0; h < H; ++h) {
            ks[h] = k_scales[per_head ? h : 0];
            vs[h] = v_scales[per_head ? h : 0];
        }
    }
    size_t tok(int h, int t) const { return ((size_t)h * Tmax + t) * d; }

    // Append one token (all heads), k and v [H][d] raw bits: each element is
    // divided by its head's scale in single precision and encoded.
    void append_one(const uint16_t* k, const uint16_t* v) {
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < d; ++c) {
                float xk = load_elem(k[(size_t)h * d + c], dtype);
                float xv = load_elem(v[(size_t)h * d + c], dtype);
                k_code[tok(h, T) + c] = f32_to_e4m3(xk / ks[h]);
                v_code[tok(h, T) + c] = f32_to_e4m3(xv / vs[h]);
            }
        ++T;
    }
    float k_hat(int h, int t, int c) const { return e4m3_to_f32(k_code[tok(h, t) + c]) * ks[h]; }
    float v_hat(int h, int t, int c) const { return e4m3_to_f32(v_code[tok(h, t) + c]) * vs[h]; }
};

// ---------------------------------------------------------------------------
// Attention over the reconstructed cache ("4.4 KV Cache 量化", section 2:
// P = softmax(Q K^T / sqrt(d)), output P V; the residual takes part next to
// the quantised history, section 3.2). fp64 accumulation of fp32 inputs.
// One query row: position pos in its sequence; it attends tokens 0..pos.
// GQA: query head hq reads KV head hq / (H_Q / H_KV).
// ---------------------------------------------------------------------------

// Softmax attention of one query over n tokens whose Keys and Values come
// from kf(t, ch) and vf(t, ch).
template <class KF, class VF>
void attend_tokens(int d, const float* q, int n, KF kf, VF vf, double sigma, double* out) {
    std::vector<double> score(n);
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double s = 0.0;
        for (int ch = 0; ch < d; ++ch) s += (double)q[ch] * (double)kf(t, ch);
        s *= sigma;
        score[t] = s;
        if (s > m) m = s;
    }
    double l = 0.0;
    for (int t = 0; t < n; ++t) { score[t] = std::exp(score[t] - m); l += score[t]; }
    for (int ch = 0; ch < d; ++ch) out[ch] = 0.0;
    for (int t = 0; t < n; ++t)
        for (int ch = 0; ch < d; ++ch) out[ch] += score[t] * (double)vf(t, ch);
    for (int ch = 0; ch < d; ++ch) out[ch] /= l;
}

void attend_row(const SeqCache& c, const float* q, int hq, int H_Q, int pos,
                double sigma, double* out) {
    int h = hq / (H_Q / c.H);
    attend_tokens(c.d, q, pos + 1, [&](int t, int ch) { return c.k_tilde(h, t, ch); },
                  [&](int t, int ch) { return c.v_tilde(h, t, ch); }, sigma, out);
}

// Prefill reading in which a chunk is quantised for storage only: the query
// rows of a chunk see the reconstructed history the cache held before the
// chunk (positions 0..P-1, quantised codes plus the residual of section 3.2)
// and the chunk's own Keys and Values as given, at full precision (the
// residual's rule that the newest tokens keep their precision, applied to the
// whole chunk). kc, vc point at chunk row 0 of this request, rows of H*d
// elements; the row sits at position P + i and sees n_chunk chunk tokens.
void attend_row_raw_chunk(const SeqCache& c, const float* q, int hq, int H_Q, int n_chunk,
                          const uint16_t* kc, const uint16_t* vc, double sigma, double* out) {
    int h = hq / (H_Q / c.H);
    int P = c.T;
    size_t row = (size_t)c.H * c.d;
    attend_tokens(c.d, q, P + n_chunk,
                  [&](int t, int ch) {
                      return t < P ? c.k_tilde(h, t, ch)
                                   : load_elem(kc[(size_t)(t - P) * row + (size_t)h * c.d + ch], c.dtype);
                  },
                  [&](int t, int ch) {
                      return t < P ? c.v_tilde(h, t, ch)
                                   : load_elem(vc[(size_t)(t - P) * row + (size_t)h * c.d + ch], c.dtype);
                  },
                  sigma, out);
}

}  // namespace

extern "C" {

// --- formats ---------------------------------------------------------------
uint16_t orc_f16_from_f32(float f) { return f32_to_f16(f); }
float orc_f32_from_f16(uint16_t h) { return f16_to_f32(h); }
float orc_f32_from_bf16(uint16_t b) { return bf16_to_f32(b); }
void orc_f16_from_f32_array(const float* x, uint16_t* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = f32_to_f16(x[i]);
}
void orc_f32_from_f16_array(const uint16_t* x, float* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = f16_to_f32(x[i]);
}

// --- memory formula ("4.4 KV Cache 量化", section 1) -----------------------
// M_KV = 2 * L * B * T * H_KV * d * b, with b given in bits per element here
// (the page counts b in bytes; bits/8 is the same quantity).
double orc_m_kv_bytes(double L, double B, double T, double H_KV, double d, double bits) {
    return 2.0 * L * B * T * H_KV * d * (bits / 8.0);
}

// --- one group --------------------------------------------------------------
void orc_quantize_group(const float* x, long n, int bits, uint8_t* codes,
                        uint16_t* s16, uint16_t* z16) {
    quantize_group(x, n, 1, bits, codes, 1, s16, z16);
}
float orc_dequant(int code, uint16_t s16, uint16_t z16) { return dequant((uint8_t)code, s16, z16); }
void orc_dequant_array(const uint8_t* codes, const uint16_t* s16, const uint16_t* z16, float* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = dequant(codes[i], s16[i], z16[i]);
}

// --- sequence cache -----------------------------------------------------------
void* orc_cache_new(int H, int d, int bits, int G, int Gv, int R, int dtype, int Tmax, int vflush) {
    if (H <= 0 || d <= 0 || (bits != 2 && bits != 4) || G <= 0 || Gv <= 0 || d % Gv ||
        R <= 0 || R % G || Tmax < 0 || (dtype != DT_F16 && dtype != DT_BF16) || (vflush != 0 && vflush != 1))
        return nullptr;
    return new SeqCache(H, d, bits, G, Gv, R, dtype, Tmax, vflush);
}
void orc_cache_free(void* p) { delete static_cast<SeqCache*>(p); }

// Append n tokens one at a time: k, v are [n][H][d] raw bits.
int orc_cache_append(void* p, int n, const uint16_t* k, const uint16_t* v) {
    SeqCache* c = static_cast<SeqCache*>(p);
    if (c->T + n > c->Tmax) return -1;
    for (int i = 0; i < n; ++i)
        c->append_one(k + (size_t)i * c->H * c->d, v + (size_t)i * c->H * c->d);
    return 0;
}

// Lengths and pointers to the logical state (valid while the cache lives).
void orc_cache_state(void* p, int* T, int* TK, int* TV) {
    SeqCache* c = static_cast<SeqCache*>(p);
    *T = c->T; *TK = c->TK; *TV = c->TV;
}
void orc_cache_arrays(void* p, uint8_t** k_code, uint8_t** v_code, uint16_t** k_s, uint16_t** k_z,
                      uint16_t** v_s, uint16_t** v_z, uint16_t** k_raw, uint16_t** v_raw) {
    SeqCache* c = static_cast<SeqCache*>(p);
    *k_code = c->k_code.data(); *v_code = c->v_code.data();
    *k_s = c->k_s.data(); *k_z = c->k_z.data();
    *v_s = c->v_s.data(); *v_z = c->v_z.data();
    *k_raw = c->k_raw.data(); *v_raw = c->v_raw.data();
}

// Reconstructed K~ and V~ of head h, tokens [0, T): [T][d] fp32 each.
void orc_cache_reconstruct(void* p, int h, float* k_out, float* v_out) {
    SeqCache* c = static_cast<SeqCache*>(p);
    for (int t = 0; t < c->T; ++t)
        for (int ch = 0; ch < c->d; ++ch) {
            k_out[(size_t)t * c->d + ch] = c->k_tilde(h, t, ch);
            v_out[(size_t)t * c->d + ch] = c->v_tilde(h, t, ch);
        }
}

// Attention for selected (query row, query head) items.
//  caches[S]: one cache per request; q: [total_q][H_Q][d] raw bits in q_dtype;
//  cu_q[S+1]: query rows of request s are cu_q[s] .. cu_q[s+1]-1, and row i of
//  request s sits at position T_s - n_q + i (decode: one row per request at
//  T_s - 1). causal = 0 lets every row see all T_s tokens.
//  rows[n_items], heads[n_items]: which outputs to compute; out: [n_items][d].
//  Independent items are spread over `threads` std::threads.
int orc_attention(void** caches, int S, int H_Q, const uint16_t* q, int q_dtype, const int* cu_q,
                  double sigma, int causal, const int* rows, const int* heads, long n_items,
                  double* out, int threads) {
    if (S <= 0 || n_items < 0) return -1;
    const SeqCache* c0 = static_cast<const SeqCache*>(caches[0]);
    int d = c0->d;
    for (int s = 0; s < S; ++s) {
        const SeqCache* c = static_cast<const SeqCache*>(caches[s]);
        if (c->d != d || H_Q % c->H) return -1;
    }
    std::atomic<long> next(0);
    auto work = [&]() {
        std::vector<float> qf(d);
        for (;;) {
            long it = next.fetch_add(1);
            if (it >= n_items) break;
            int r = rows[it], hq = heads[it];
            int s = 0;
            while (s + 1 <= S && cu_q[s + 1] <= r) ++s;
            const SeqCache* c = static_cast<const SeqCache*>(caches[s]);
            int nq = cu_q[s + 1] - cu_q[s];
            int pos = causal ? c->T - nq + (r - cu_q[s]) : c->T - 1;
            for (int ch = 0; ch < d; ++ch)
                qf[ch] = load_elem(q[((size_t)r * H_Q + hq) * d + ch], q_dtype);
            if (pos < 0) { for (int ch = 0; ch < d; ++ch) out[it * d + ch] = 0.0; continue; }
            attend_row(*c, qf.data(), hq, H_Q, pos, sigma, &out[it * d]);
        }
    };
    int nt = threads > 0 ? threads : 1;
    std::vector<std::thread> pool;
    for (int i = 1; i < nt; ++i) pool.emplace_back(work);
    work();
    for (auto& th : pool) th.join();
    return 0;
}

// Attention of chunks whose own tokens take part at full precision (see
// attend_row_raw_chunk). caches[s] hold each request's tokens before its
// chunk (P_s = their length); k_chunk, v_chunk: [total_q][H][d] raw bits in
// the caches' dtype, indexed like q. Row i of request s sits at position
// P_s + i and sees 0..P_s + i (causal) or 0..P_s + n_q,s - 1.
int orc_attention_raw_chunk(void** caches, int S, int H_Q, const uint16_t* q, int q_dtype, const int* cu_q,
                            const uint16_t* k_chunk, const uint16_t* v_chunk, double sigma, int causal,
                            const int* rows, const int* heads, long n_items, double* out, int threads) {
    if (S <= 0 || n_items < 0) return -1;
    const SeqCache* c0 = static_cast<const SeqCache*>(caches[0]);
    int d = c0->d, H = c0->H;
    for (int s = 0; s < S; ++s) {
        const SeqCache* c = static_cast<const SeqCache*>(caches[s]);
        if (c->d != d || c->H != H || H_Q % c->H) return -1;
    }
    std::atomic<long> next(0);
    auto work = [&]() {
        std::vector<float> qf(d);
        for (;;) {
            long it = next.fetch_add(1);
            if (it >= n_items) break;
            int r = rows[it], hq = heads[it];
            int s = 0;
            while (s + 1 <= S && cu_q[s + 1] <= r) ++s;
            const SeqCache* c = static_cast<const SeqCache*>(caches[s]);
            int nq = cu_q[s + 1] - cu_q[s];
            int i = r - cu_q[s];
            int n_chunk = causal ? i + 1 : nq;
            for (int ch = 0; ch < d; ++ch)
                qf[ch] = load_elem(q[((size_t)r * H_Q + hq) * d + ch], q_dtype);
            size_t base = (size_t)cu_q[s] * H * d;
            attend_row_raw_chunk(*c, qf.data(), hq, H_Q, n_chunk, k_chunk + base, v_chunk + base, sigma,
                                 &out[it * d]);
        }
    };
    int nt = threads > 0 ? threads : 1;
    std::vector<std::thread> pool;
    for (int i = 1; i < nt; ++i) pool.emplace_back(work);
    work();
    for (auto& th : pool) th.join();
    return 0;
}

// --- FP8 cache ---------------------------------------------------------------
float orc_e4m3_to_f32(int c) { return e4m3_to_f32((uint8_t)c); }
int orc_f32_to_e4m3(float y) { return f32_to_e4m3(y); }

void* orc_fp8_cache_new(int H, int d, int dtype, int Tmax, const float* k_scales, const float* v_scales,
                        int per_head) {
    if (H <= 0 || d <= 0 || Tmax < 0 || (dtype != DT_F16 && dtype != DT_BF16) || !k_scales || !v_scales)
        return nullptr;
    return new Fp8SeqCache(H, d, dtype, Tmax, k_scales, v_scales, per_head);
}
void orc_fp8_cache_free(void* p) { delete static_cast<Fp8SeqCache*>(p); }
int orc_fp8_cache_append(void* p, int n, const uint16_t* k, const uint16_t* v) {
    Fp8SeqCache* c = static_cast<Fp8SeqCache*>(p);
    if (c->T + n > c->Tmax) return -1;
    for (int i = 0; i < n; ++i) c->append_one(k + (size_t)i * c->H * c->d, v + (size_t)i * c->H * c->d);
    return 0;
}
int orc_fp8_cache_len(void* p) { return static_cast<Fp8SeqCache*>(p)->T; }
void orc_fp8_cache_arrays(void* p, uint8_t** k_code, uint8_t** v_code) {
    Fp8SeqCache* c = static_cast<Fp8SeqCache*>(p);
    *k_code = c->k_code.data();
    *v_code = c->v_code.data();
}

// Decode attention over FP8 caches: one query row per request at position
// T_s - 1, every query head; q [S][H_Q][d] raw bits; out [S][H_Q][d].
int orc_fp8_attention(void** caches, int S, int H_Q, const uint16_t* q, int q_dtype, double sigma, double* out,
                      int threads) {
    if (S <= 0) return -1;
    for (int s = 0; s < S; ++s) {
        const Fp8SeqCache* c = static_cast<const Fp8SeqCache*>(caches[s]);
        if (H_Q % c->H) return -1;
    }
    std::atomic<long> next(0);
    const long n_items = (long)S * H_Q;
    auto work = [&]() {
        for (;;) {
            long it = next.fetch_add(1);
            if (it >= n_items) break;
            int s = (int)(it / H_Q), hq = (int)(it % H_Q);
            const Fp8SeqCache* c = static_cast<const Fp8SeqCache*>(caches[s]);
            int d = c->d, h = hq / (H_Q / c->H);
            std::vector<float> qf(d);
            for (int ch = 0; ch < d; ++ch) qf[ch] = load_elem(q[((size_t)s * H_Q + hq) * d + ch], q_dtype);
            double* o = &out[it * d];
            if (c->T == 0) { for (int ch = 0; ch < d; ++ch) o[ch] = 0.0; continue; }
            attend_tokens(d, qf.data(), c->T, [&](int t, int ch) { return c->k_hat(h, t, ch); },
                          [&](int t, int ch) { return c->v_hat(h, t, ch); }, sigma, o);
        }
    };
    int nt = threads > 0 ? threads : 1;
    std::vector<std::thread> pool;
    for (int i = 1; i < nt; ++i) pool.emplace_back(work);
    work();
    for (auto& th : pool) th.join();
    return 0;
}

// Prefill over FP8 caches: q [total_q][H_Q][d] raw bits, cu_q [S+1]; row i of
// request s sits at position T_s - n_q,s + i and sees positions 0..itself
// (causal) or all T_s tokens; a row that sees no token is zero.
// out [total_q][H_Q][d].
int orc_fp8_attention_rows(void** caches, int S, int H_Q, const uint16_t* q, int q_dtype, const int* cu_q,
                           double sigma, int causal, double* out, int threads) {
    if (S <= 0) return -1;
    for (int s = 0; s < S; ++s)
        if (H_Q % static_cast<const Fp8SeqCache*>(caches[s])->H) return -1;
    const long n_items = (long)cu_q[S] * H_Q;
    std::atomic<long> next(0);
    auto work = [&]() {
        for (;;) {
            long it = next.fetch_add(1);
            if (it >= n_items) break;
            int r = (int)(it / H_Q), hq = (int)(it % H_Q);
            int s = 0;
            while (s + 1 <= S && cu_q[s + 1] <= r) ++s;
            const Fp8SeqCache* c = static_cast<const Fp8SeqCache*>(caches[s]);
            int d = c->d, h = hq / (H_Q / c->H);
            int nq = cu_q[s + 1] - cu_q[s];
            int pos = c->T - nq + (r - cu_q[s]);
            int n = causal ? std::min(pos + 1, c->T) : c->T;
            double* o = &out[it * d];
            if (n <= 0) { for (int ch = 0; ch < d; ++ch) o[ch] = 0.0; continue; }
            std::vector<float> qf(d);
            for (int ch = 0; ch < d; ++ch) qf[ch] = load_elem(q[((size_t)r * H_Q + hq) * d + ch], q_dtype);
            attend_tokens(d, qf.data(), n, [&](int t, int ch) { return c->k_hat(h, t, ch); },
                          [&](int t, int ch) { return c->v_hat(h, t, ch); }, sigma, o);
        }
    };
    int nt = threads > 0 ? threads : 1;
    std::vector<std::thread> pool;
    for (int i = 1; i < nt; ++i) pool.emplace_back(work);
    work();
    for (auto& th : pool) th.join();
    return 0;
}

int orc_hardware_threads() { return (int)std::thread::hardware_concurrency(); }

}  // extern "C"
