// Host-side exercise of the C ABI (kivi.h) and of the CPU oracle, built with
// AddressSanitizer and UndefinedBehaviorSanitizer: every configuration check,
// layout, capacity search and argument check of every call, the split plans,
// the status-word paths, and the oracle's quantiser, caches (both Value flush
// rules, fp16 and bf16, FP8) and attention on small seeded inputs. The device
// side is replaced by host stubs (host_stubs.cpp); nothing here touches a GPU.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "kivi.h"

extern "C" {
void orc_quantize_group(const float* x, long n, int bits, uint8_t* codes, uint16_t* s16, uint16_t* z16);
float orc_dequant(int code, uint16_t s16, uint16_t z16);
uint16_t orc_f16_from_f32(float f);
void* orc_cache_new(int H, int d, int bits, int G, int Gv, int R, int dtype, int Tmax, int vflush);
void orc_cache_free(void* p);
int orc_cache_append(void* p, int n, const uint16_t* k, const uint16_t* v);
void orc_cache_state(void* p, int* T, int* TK, int* TV);
void orc_cache_reconstruct(void* p, int h, float* k_out, float* v_out);
int orc_attention(void** caches, int S, int H_Q, const uint16_t* q, int q_dtype, const int* cu_q, double sigma,
                  int causal, const int* rows, const int* heads, long n_items, double* out, int threads);
void* orc_fp8_cache_new(int H, int d, int dtype, int Tmax, const float* k_scales, const float* v_scales,
                        int per_head);
void orc_fp8_cache_free(void* p);
int orc_fp8_cache_append(void* p, int n, const uint16_t* k, const uint16_t* v);
int orc_fp8_attention(void** caches, int S, int H_Q, const uint16_t* q, int q_dtype, double sigma, double* out,
                      int threads);
}

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static kivi_cache_config cfg(int H, int bits, int G, int Gv, int R, int Bk, int nb, int ms, int dt, int vf = 0) {
    kivi_cache_config c{};
    c.num_kv_heads = H; c.head_dim = 128; c.bits = bits; c.k_group = G; c.v_group = Gv; c.residual = R;
    c.block_size = Bk; c.num_blocks = nb; c.max_seqs = ms; c.kv_dtype = dt; c.v_flush = vf;
    return c;
}

static void abi() {
    // configurations: valid and invalid, pool sizes, layouts, capacities
    const int bits_list[] = {2, 4, 8, 3};
    const int groups[] = {16, 32, 64, 128, 256, 48};
    for (int bits : bits_list)
        for (int G : groups)
            for (int Gv : {16, 128, 48})
                for (int R : {G, 2 * G, 8192, 96})
                    for (int Bk : {16, 64}) {
                        kivi_cache_config c = bits == 8 ? cfg(8, 8, 0, 0, 0, Bk, 100, 4, KIVI_F16)
                                                        : cfg(8, bits, G, Gv, R, Bk, 100, 4, KIVI_BF16);
                        size_t n = 0;
                        const kivi_status s = kivi_cache_pool_bytes(&c, &n);
                        int32_t nb = 0;
                        int64_t tok = 0;
                        EXPECT(kivi_cache_capacity(&c, (size_t)1 << 30, &nb, &tok) == s);
                        if (s != KIVI_OK) continue;
                        EXPECT(tok == (int64_t)nb * Bk);
                        kivi_cache* h = nullptr;
                        EXPECT(kivi_cache_create(&c, (void*)(uintptr_t)(1u << 20), n - 1, &h) == KIVI_ERR_POOL_TOO_SMALL);
                        EXPECT(kivi_cache_create(&c, (void*)(uintptr_t)(1u << 20), n, &h) == KIVI_OK);
                        kivi_layout L{};
                        EXPECT(kivi_cache_layout(h, &L) == KIVI_OK && L.total_bytes == n && L.status + 256 == n);
                        kivi_cache_destroy(h);
                    }
    size_t big = 0;
    kivi_cache_config huge = cfg(1024, 4, 64, 128, 128, 1024, 1 << 20, 1, KIVI_F16);
    EXPECT(kivi_cache_pool_bytes(&huge, &big) == KIVI_ERR_UNSUPPORTED);
    EXPECT(kivi_cache_pool_bytes(nullptr, &big) == KIVI_ERR_INVALID_ARG);
    kivi_cache_destroy(nullptr);

    // calls: argument checks and, past them, the host plans (the launchers are stubs)
    kivi_cache_config c = cfg(8, 4, 64, 128, 128, 16, 8192, 32, KIVI_F16);
    size_t n = 0;
    EXPECT(kivi_cache_pool_bytes(&c, &n) == KIVI_OK);
    kivi_cache* h = nullptr;
    EXPECT(kivi_cache_create(&c, (void*)(uintptr_t)(1u << 20), n, &h) == KIVI_OK);
    void* D = (void*)(uintptr_t)(1u << 20);
    const int32_t* I = (const int32_t*)D;
    uint32_t flags = 7;
    EXPECT(kivi_check_device_errors(h, nullptr, &flags) == KIVI_OK && flags == 0);  // clears, nothing ran
    EXPECT(kivi_append_tokens(h, 32, I, I, I, 1, D, D, I, 256, nullptr) == KIVI_OK);
    EXPECT(kivi_append_tokens(h, 32, I, I, I, 1, (char*)D + 2, D, I, 256, nullptr) == KIVI_ERR_INVALID_ARG);
    for (int S : {1, 4, 32, 300})
        for (int T : {0, 100, 4096, 32768}) {
            size_t ws = 0;
            EXPECT(kivi_decode_workspace_bytes(h, S, 32, T, &ws) == KIVI_OK);
            EXPECT(kivi_decode_attention(h, S, 32, D, I, I, T, I, 256, 0.088f, D, ws ? D : nullptr, ws, nullptr) ==
                   KIVI_OK);
            if (ws)
                EXPECT(kivi_decode_attention(h, S, 32, D, I, I, T, I, 256, 0.088f, D, D, ws - 1, nullptr) ==
                       KIVI_ERR_WORKSPACE);
            EXPECT(kivi_decode_step(h, S, 32, D, I, I, D, D, T, I, 256, 0.088f, D, ws ? D : nullptr, ws, nullptr) ==
                   KIVI_OK);
            EXPECT(kivi_decode_attention_noalloc(h, S, 32, D, I, I, T, I, 256, 0.088f, D, nullptr) == KIVI_OK);
        }
    EXPECT(kivi_decode_attention(h, 4, 30, D, I, I, 64, I, 1, 0.1f, D, D, 1 << 20, nullptr) == KIVI_ERR_UNSUPPORTED);
    EXPECT(kivi_decode_attention(h, 4, 32, D, I, I, 64, I, 1, NAN, D, D, 1 << 20, nullptr) == KIVI_ERR_INVALID_ARG);
    EXPECT(kivi_prefill_attention(h, 2, 32, D, I, 16, I, I, 4096, I, 1, 0.1f, 1, D, nullptr, 0, nullptr) == KIVI_OK);
    EXPECT(kivi_prefill_attention(h, 2, 32, D, I, 1 << 28, I, I, 4096, I, 1, 0.1f, 1, D, nullptr, 0, nullptr) ==
           KIVI_ERR_UNSUPPORTED);
    EXPECT(kivi_prefill_attention_raw_chunk(h, 2, 32, D, I, 16, I, I, D, D, 4096, I, 1, 0.1f, 0, D, nullptr, 0,
                                            nullptr) == KIVI_OK);
    EXPECT(kivi_fp8_append_tokens(h, 2, I, I, 1, D, D, (const float*)D, (const float*)D, I, 1, nullptr) ==
           KIVI_ERR_UNSUPPORTED);
    EXPECT(kivi_check_device_errors(h, nullptr, &flags) == KIVI_OK && flags == 0);
    EXPECT(kivi_check_device_errors(nullptr, nullptr, &flags) == KIVI_ERR_INVALID_ARG);
    kivi_cache_destroy(h);

    kivi_cache_config f = cfg(8, 8, 0, 0, 0, 16, 2048, 1, KIVI_BF16);
    f.scale_per_head = 1;
    EXPECT(kivi_cache_pool_bytes(&f, &n) == KIVI_OK);
    EXPECT(kivi_cache_create(&f, D, n, &h) == KIVI_OK);
    const float* F = (const float*)D;
    EXPECT(kivi_fp8_append_tokens(h, 2, I, I, 3, D, D, F, F, I, 8, nullptr) == KIVI_OK);
    size_t ws = 0;
    EXPECT(kivi_decode_workspace_bytes(h, 4, 32, 4096, &ws) == KIVI_OK);
    EXPECT(kivi_fp8_decode_attention(h, 4, 32, D, I, 4096, F, F, I, 256, 0.088f, D, D, ws, nullptr) == KIVI_OK);
    EXPECT(kivi_fp8_decode_step(h, 4, 32, D, I, D, D, 4096, F, F, I, 256, 0.088f, D, D, ws, nullptr) == KIVI_OK);
    EXPECT(kivi_fp8_prefill_attention(h, 2, 32, D, I, 64, I, 4096, F, F, I, 256, 0.088f, 1, D, nullptr) == KIVI_OK);
    EXPECT(kivi_decode_attention(h, 4, 32, D, I, I, 64, I, 1, 0.1f, D, D, 1 << 20, nullptr) == KIVI_ERR_UNSUPPORTED);
    kivi_cache_destroy(h);
    for (int s = 0; s <= 7; ++s) EXPECT(kivi_status_string((kivi_status)s) != nullptr);
    EXPECT(kivi_last_error() != nullptr);
}

static void oracle_paths() {
    std::mt19937 rng(5);
    std::normal_distribution<float> nd(0.0f, 1.0f);
    // quantiser: random, constant and grid groups, both widths
    for (int bits : {2, 4})
        for (int n : {1, 16, 64, 256}) {
            std::vector<float> x(n);
            std::vector<uint8_t> q(n);
            for (auto& v : x) v = nd(rng) * 3.0f;
            uint16_t s16 = 0, z16 = 0;
            orc_quantize_group(x.data(), n, bits, q.data(), &s16, &z16);
            for (int i = 0; i < n; ++i) EXPECT(q[i] <= (1 << bits) - 1 && std::isfinite(orc_dequant(q[i], s16, z16)));
            for (auto& v : x) v = 0.75f;
            orc_quantize_group(x.data(), n, bits, q.data(), &s16, &z16);
            EXPECT(s16 == 0);
        }
    // caches (fp16 and bf16, both Value rules), then decode and causal prefill rows
    const int H = 2, HQ = 6, d = 128;
    for (int dtype : {0, 1})
        for (int vf : {0, 1}) {
            const int Tn[2] = {150, 77};
            void* caches[2];
            for (int s = 0; s < 2; ++s) {
                caches[s] = orc_cache_new(H, d, 4, 32, 32, 64, dtype, Tn[s] + 4, vf);
                EXPECT(caches[s] != nullptr);
                std::vector<uint16_t> k((size_t)Tn[s] * H * d), v(k.size());
                for (size_t i = 0; i < k.size(); ++i) {
                    k[i] = dtype ? (uint16_t)0x3f80 : orc_f16_from_f32(nd(rng));
                    v[i] = orc_f16_from_f32(nd(rng));
                }
                // in two calls: 50 tokens, then the rest (the rows of one call are consecutive)
                EXPECT(orc_cache_append(caches[s], 50, k.data(), v.data()) == 0);
                EXPECT(orc_cache_append(caches[s], Tn[s] - 50, k.data() + (size_t)50 * H * d,
                                        v.data() + (size_t)50 * H * d) == 0);
                int T = 0, TK = 0, TV = 0;
                orc_cache_state(caches[s], &T, &TK, &TV);
                EXPECT(T == Tn[s] && TK == 64 * (T / 64) && TV == (vf ? TK : T - 64));
                std::vector<float> kr((size_t)T * d), vr(kr.size());
                orc_cache_reconstruct(caches[s], 1, kr.data(), vr.data());
                EXPECT(orc_cache_append(caches[s], 1000, k.data(), v.data()) == -1);  // past Tmax
            }
            const int rows_n = 3;
            std::vector<uint16_t> q((size_t)rows_n * HQ * d);
            for (auto& x : q) x = orc_f16_from_f32(nd(rng) * 0.1f);
            const int cu[3] = {0, 2, 3};
            std::vector<int> rows, heads;
            for (int r = 0; r < rows_n; ++r)
                for (int hq = 0; hq < HQ; ++hq) {
                    rows.push_back(r);
                    heads.push_back(hq);
                }
            std::vector<double> out(rows.size() * d);
            for (int causal : {0, 1})
                EXPECT(orc_attention(caches, 2, HQ, q.data(), 0, cu, 0.088, causal, rows.data(), heads.data(),
                                     (long)rows.size(), out.data(), 2) == 0);
            for (double o : out) EXPECT(std::isfinite(o));
            for (void* c : caches) orc_cache_free(c);
        }
    // FP8 cache and decode
    const float ks[2] = {0.01f, 0.02f}, vs[2] = {0.01f, 0.03f};
    void* c8 = orc_fp8_cache_new(H, d, 0, 40, ks, vs, 1);
    std::vector<uint16_t> k(40 * H * d), v(k.size());
    for (size_t i = 0; i < k.size(); ++i) {
        k[i] = orc_f16_from_f32(nd(rng) * 8.0f);
        v[i] = orc_f16_from_f32(nd(rng));
    }
    EXPECT(orc_fp8_cache_append(c8, 40, k.data(), v.data()) == 0);
    std::vector<uint16_t> q(HQ * d);
    for (auto& x : q) x = orc_f16_from_f32(nd(rng));
    std::vector<double> out(HQ * d);
    EXPECT(orc_fp8_attention(&c8, 1, HQ, q.data(), 0, 0.088, out.data(), 1) == 0);
    orc_fp8_cache_free(c8);
}

int main() {
    abi();
    oracle_paths();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host sanitizer run: all checks passed\n");
    return 0;
}
