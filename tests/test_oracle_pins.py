"""Pins of the CPU oracle against what the pages and the mathematics fix.

No test here compares the oracle with itself: each one checks it against a
printed value of the pages, a closed form, a library routine (numpy's binary16
conversion, numpy float64 softmax), an invariant of min/max mapping, or brute
force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import DT_BF16, DT_F16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(x):
    return np.asarray(x, dtype=np.float16)


def f16bits(x):
    return f16(x).view(np.uint16)


# ---------------------------------------------------------------------------
# number formats (binary16 round-to-nearest-even vs numpy's conversion)
# ---------------------------------------------------------------------------

def test_f16_from_f32_matches_numpy():
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(200000).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 17, 200000),
        rng.uniform(-65600, 65600, 20000).astype(np.float32),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, 2.0 ** -25, 2.0 ** -24,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -26, np.inf, -np.inf], dtype=np.float32),
    ]
    # exact binary16 ties: midpoints between neighbouring binary16 values
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    parts.append(-((lo + hi) / 2).astype(np.float32))
    x = np.concatenate(parts).astype(np.float32)
    got = oracle.f16_bits_from_f32(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f32_from_f16_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (h & 0x7C00) != 0x7C00
    got = oracle.f32_from_f16_bits(h)
    want = h.view(np.float16).astype(np.float32)
    assert np.array_equal(got[finite].view(np.uint32), want[finite].view(np.uint32))


# ---------------------------------------------------------------------------
# M_KV formula: the page's worked example ("4.4 KV Cache 量化", section 1)
# ---------------------------------------------------------------------------

def test_m_kv_worked_example():
    with open(os.path.join(GOLDEN, "m_kv_worked_example.json")) as f:
        g = json.load(f)
    i = g["inputs"]
    for case in g["cases"]:
        got = oracle.m_kv_bytes(i["L"], i["B"], i["T"], i["H_KV"], i["d"], case["bits_per_element"])
        assert got == case["bytes"]
    assert oracle.m_kv_bytes(32, 1, 32768, 8, 128, 16) == 4 * 2 ** 30


# ---------------------------------------------------------------------------
# group quantiser
# ---------------------------------------------------------------------------

def _rand_group(rng, n, spread=1.0, loc=0.0):
    return f16(rng.standard_normal(n) * spread + loc).astype(np.float32)


@pytest.mark.parametrize("bits", [2, 4])
def test_code_range_and_endpoints(bits):
    """2-bit has exactly 4 codes ("4.4 KV Cache 量化" section 3.1); min -> 0, max -> 2^b-1."""
    rng = np.random.default_rng(2)
    Q = 2 ** bits - 1
    for n in (4, 32, 64, 128):
        for _ in range(200):
            x = _rand_group(rng, n, spread=10.0 ** rng.uniform(-3, 2), loc=rng.uniform(-5, 5))
            codes, s, z = oracle.quantize_group(x, bits)
            assert codes.max() <= Q
            if s == 0:
                continue
            assert codes[np.argmin(x)] == 0
            assert codes[np.argmax(x)] == Q
            # zero-point is the group minimum (fp16 inputs: exact)
            assert np.float16(x.min()).view(np.uint16) == z


@pytest.mark.parametrize("bits", [2, 4])
def test_round_trip_bound_and_nearest_grid_point(bits):
    """Min/max mapping puts every element within half a step of its restored value."""
    rng = np.random.default_rng(3)
    Q = 2 ** bits - 1
    for n in (8, 32, 128):
        for _ in range(300):
            x = _rand_group(rng, n, spread=10.0 ** rng.uniform(-2, 1.5), loc=rng.uniform(-8, 8))
            codes, s, z = oracle.quantize_group(x, bits)
            S = float(np.uint16(s).view(np.float16))
            Z = float(np.uint16(z).view(np.float16))
            if S == 0 or S < 2.0 ** -14:
                continue
            xh = oracle.dequant(codes, s, z).astype(np.float64)
            xd = x.astype(np.float64)
            slack = 2.0 ** -22 * (Q * S + abs(Z) + np.abs(xd))
            assert np.all(np.abs(xd - xh) <= S / 2 + slack)
            # no other code in [0, Q] restores closer (beyond rounding slack)
            for delta in (-1, 1):
                alt = codes.astype(np.int64) + delta
                ok = (alt >= 0) & (alt <= Q)
                xa = oracle.dequant(np.clip(alt, 0, Q).astype(np.uint8), s, z).astype(np.float64)
                assert np.all(np.abs(xd - xh)[ok] <= np.abs(xd - xa)[ok] + slack[ok])


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("dtype", [DT_F16, DT_BF16])
def test_constant_group_exact(bits, dtype):
    rng = np.random.default_rng(4)
    for v in [0.0, -0.0, 1.5, -3.25, 1000.0, 6.1e-5, -2.0 ** -20]:
        x = np.full(16, v, dtype=np.float32)
        if dtype == DT_BF16:
            x = oracle.f32_from_bf16_bits((x.view(np.uint32) >> 16).astype(np.uint16))
        else:
            x = f16(x).astype(np.float32)
        codes, s, z = oracle.quantize_group(x, bits)
        assert s == 0 and np.all(codes == 0)
        xh = oracle.dequant(codes, s, z)
        assert np.array_equal(xh, np.where(x == 0, np.float32(0), x))
    del rng


@pytest.mark.parametrize("bits", [2, 4])
def test_grid_exact_groups_closed_form(bits):
    """x = z + k 2^e with k in 0..Q (0 and Q present) -> s16 = 2^e, z16 = z, codes = k."""
    rng = np.random.default_rng(5)
    Q = 2 ** bits - 1
    for _ in range(500):
        e = int(rng.integers(-8, 3))
        z = float(f16(rng.uniform(-4, 4)))
        z = math.floor(z / 2.0 ** e) * 2.0 ** e
        n = int(rng.choice([8, 32, 64]))
        k = rng.integers(0, Q + 1, n)
        k[rng.integers(n)] = 0
        k[(rng.integers(n - 1) + 1 + np.argmin(k)) % n] = Q
        x = (z + k * 2.0 ** e).astype(np.float32)
        assert np.array_equal(f16(x).astype(np.float32), x)
        codes, s, zz = oracle.quantize_group(x, bits)
        assert s == f16bits(2.0 ** e)
        assert zz == (f16bits(z) if z != 0 else 0)
        assert np.array_equal(codes, k.astype(np.uint8))


@pytest.mark.parametrize("bits", [2, 4])
def test_ties_round_to_even(bits):
    rng = np.random.default_rng(6)
    Q = 2 ** bits - 1
    e = -3
    z = -1.0
    for k in range(Q):
        ties = z + (k + 0.5) * 2.0 ** e
        x = np.array([z, z + Q * 2.0 ** e, ties, ties], dtype=np.float32)
        rng.shuffle(x)
        codes, s, _ = oracle.quantize_group(x, bits)
        assert s == f16bits(2.0 ** e)
        want = k if k % 2 == 0 else k + 1
        assert np.all(codes[x == np.float32(ties)] == want)


@pytest.mark.parametrize("bits", [2, 4])
def test_power_of_two_equivariance(bits):
    rng = np.random.default_rng(7)
    for _ in range(300):
        x = _rand_group(rng, 32, spread=rng.uniform(0.5, 2), loc=rng.uniform(-2, 2))
        c0, s0, z0 = oracle.quantize_group(x, bits)
        m = int(rng.integers(-4, 5))
        c1, s1, z1 = oracle.quantize_group((x * np.float32(2.0 ** m)).astype(np.float32), bits)
        assert np.array_equal(c0, c1)
        assert float(np.uint16(s1).view(np.float16)) == float(np.uint16(s0).view(np.float16)) * 2.0 ** m
        assert float(np.uint16(z1).view(np.float16)) == float(np.uint16(z0).view(np.float16)) * 2.0 ** m


@pytest.mark.parametrize("bits", [2, 4])
def test_order_invariance(bits):
    rng = np.random.default_rng(8)
    for _ in range(200):
        x = _rand_group(rng, 64)
        p = rng.permutation(64)
        c0, s0, z0 = oracle.quantize_group(x, bits)
        c1, s1, z1 = oracle.quantize_group(x[p], bits)
        assert (s0, z0) == (s1, z1)
        assert np.array_equal(c0[p], c1)


def test_negative_zero_reads_as_positive_zero():
    x = np.array([-0.0, 0.5, 1.0, 0.25], dtype=np.float32)
    _, _, z = oracle.quantize_group(x, 4)
    assert z == 0


# ---------------------------------------------------------------------------
# sequence cache: grouping directions and residual semantics
# ("4.4 KV Cache 量化", sections 3.1 and 3.2)
# ---------------------------------------------------------------------------

def _stream(rng, T, H, d, dtype=DT_F16, kscale=None):
    k = rng.standard_normal((T, H, d))
    if kscale is not None:
        k = k * kscale
    v = rng.standard_normal((T, H, d))
    if dtype == DT_F16:
        return f16(k).view(np.uint16), f16(v).view(np.uint16)
    to = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731
    return to(k), to(v)


def _as_f32(bits, dtype):
    return oracle.f32_from_bf16_bits(bits) if dtype == DT_BF16 else oracle.f32_from_f16_bits(bits)


@pytest.mark.parametrize("bits,G,Gv,R", [(4, 4, 4, 4), (2, 4, 8, 8), (4, 8, 16, 16), (2, 32, 32, 64)])
@pytest.mark.parametrize("dtype", [DT_F16, DT_BF16])
@pytest.mark.parametrize("v_flush", [0, 1])
def test_cache_state_is_direct_grouping_of_stream(bits, G, Gv, R, dtype, v_flush):
    """After T tokens: T_K = R floor(T/R), T_V = max(0, T-R) (T_V = T_K when Values flush
    with the Keys); Key group j of channel c is the quantisation of tokens jG..jG+G-1 of
    that channel alone; Value token t group g is the quantisation of channels
    gGv..gGv+Gv-1 of that token alone."""
    rng = np.random.default_rng(9)
    H, d, T = 2, 32, 3 * R + R // 2 + 1
    kb, vb = _stream(rng, T, H, d, dtype)
    c = oracle.SeqCache(H, d, bits, G, Gv, R, dtype, T, v_flush=v_flush)
    t = 0
    while t < T:  # appends of random sizes
        n = int(min(T - t, rng.integers(1, 2 * R)))
        c.append(kb[t:t + n], vb[t:t + n])
        t += n
        Tn, TK, TV = c.state()
        assert (Tn, TK, TV) == (t, R * (t // R), R * (t // R) if v_flush else max(0, t - R))
    a = c.arrays()
    kf, vf = _as_f32(kb, dtype), _as_f32(vb, dtype)
    Tn, TK, TV = c.state()
    for h in range(H):
        for j in range(TK // G):
            for ch in range(d):
                codes, s, z = oracle.quantize_group(kf[j * G:(j + 1) * G, h, ch], bits)
                assert np.array_equal(a["k_code"][h, j * G:(j + 1) * G, ch], codes)
                assert a["k_s"][h, j, ch] == s and a["k_z"][h, j, ch] == z
        for tt in range(TV):
            for g in range(d // Gv):
                codes, s, z = oracle.quantize_group(vf[tt, h, g * Gv:(g + 1) * Gv], bits)
                assert np.array_equal(a["v_code"][h, tt, g * Gv:(g + 1) * Gv], codes)
                assert a["v_s"][h, tt, g] == s and a["v_z"][h, tt, g] == z
        # residual keeps the input bits
        assert np.array_equal(a["k_raw"][h, TK:T], kb[TK:T, h])
        assert np.array_equal(a["v_raw"][h, TV:T], vb[TV:T, h])


def _dequant_f32(codes, s16, z16):
    """x = fl32(fl32(code * S) + Z), two single-precision roundings."""
    S = np.asarray(s16, np.uint16).view(np.float16).astype(np.float32)
    Z = np.asarray(z16, np.uint16).view(np.float16).astype(np.float32)
    return (codes.astype(np.float32) * S).astype(np.float32) + Z


def test_value_flush_variant_keeps_keys_and_early_values():
    """Flushing Values with the Keys changes only when Value tokens leave the residual:
    Key state is the same as with the sliding window, and every Value token both caches
    have quantised carries the same codes and parameters (per-token quantisation does
    not depend on when it runs)."""
    rng = np.random.default_rng(21)
    H, d, G, Gv, R, T = 2, 16, 4, 8, 8, 45
    kb, vb = _stream(rng, T, H, d)
    cw = oracle.SeqCache(H, d, 4, G, Gv, R, DT_F16, T)
    cu = oracle.SeqCache(H, d, 4, G, Gv, R, DT_F16, T, v_flush=1)
    for t in range(T):
        cw.append(kb[t:t + 1], vb[t:t + 1])
        cu.append(kb[t:t + 1], vb[t:t + 1])
        _, TKw, TVw = cw.state()
        _, TKu, TVu = cu.state()
        assert TKw == TKu == TVu and TVw == max(0, t + 1 - R)
    aw, au = cw.arrays(), cu.arrays()
    _, TK, TVu = cu.state()
    TVw = cw.state()[2]
    for name in ("k_code", "k_s", "k_z", "k_raw"):
        assert np.array_equal(aw[name], au[name]), name
    for name in ("v_code", "v_s", "v_z"):
        assert np.array_equal(aw[name][:, :TVw], au[name][:, :TVw]), name
    assert TVu == 40 and TVw == 37  # tokens 37..39 are codes in one cache, residual in the other


def test_value_flush_variant_attention_brute_force():
    """Attention over a cache whose Values flush with the Keys, against numpy float64
    softmax over K and V reconstructed by hand: codes of tokens below T_K = T_V restored
    as code * S + Z, the R-floor(T/R) newest tokens at full precision."""
    rng = np.random.default_rng(22)
    H, HQ, d, G, Gv, R, T = 1, 2, 16, 4, 8, 8, 27
    kb, vb = _stream(rng, T, H, d)
    c = oracle.SeqCache(H, d, 4, G, Gv, R, DT_F16, T, v_flush=1)
    c.append(kb, vb)
    assert c.state() == (T, 24, 24)
    kf, vf = _as_f32(kb, DT_F16)[:, 0], _as_f32(vb, DT_F16)[:, 0]
    K, V = kf.copy(), vf.copy()
    for j in range(24 // G):
        for ch in range(d):
            codes, s, z = oracle.quantize_group(kf[j * G:(j + 1) * G, ch], 4)
            K[j * G:(j + 1) * G, ch] = _dequant_f32(codes, s, z)
    for t in range(24):
        for g in range(d // Gv):
            codes, s, z = oracle.quantize_group(vf[t, g * Gv:(g + 1) * Gv], 4)
            V[t, g * Gv:(g + 1) * Gv] = _dequant_f32(codes, s, z)
    assert not np.array_equal(V[16:24], vf[16:24])  # the flushed tokens are restored codes
    qb = f16(rng.standard_normal((1, HQ, d))).view(np.uint16)
    q = qb.view(np.float16).astype(np.float64)
    out = oracle.attention_all([c], HQ, qb, DT_F16, [0, 1], 0.25, False)
    for hq in range(HQ):
        want = _numpy_attention(q[0, hq], K, V, 0.25)
        np.testing.assert_allclose(out[0, hq], want, rtol=1e-12, atol=1e-13)


def test_key_outlier_channel_isolated():
    """An outlier channel changes only its own Key group parameters (section 3.1)."""
    rng = np.random.default_rng(10)
    H, d, G, R, T = 1, 16, 8, 8, 32
    kb, vb = _stream(rng, T, H, d)
    c0 = oracle.SeqCache(H, d, 4, G, 16, R, DT_F16, T)
    c0.append(kb, vb)
    kf = kb.view(np.float16).astype(np.float32)
    kf[:, :, 5] *= 20
    c1 = oracle.SeqCache(H, d, 4, G, 16, R, DT_F16, T)
    c1.append(f16(kf).view(np.uint16), vb)
    a0, a1 = c0.arrays(), c1.arrays()
    others = [ch for ch in range(d) if ch != 5]
    assert np.array_equal(a0["k_code"][..., others], a1["k_code"][..., others])
    assert np.array_equal(a0["k_s"][..., others], a1["k_s"][..., others])
    assert np.array_equal(a0["k_z"][..., others], a1["k_z"][..., others])
    assert not np.array_equal(a0["k_s"][0, :T // G, 5], a1["k_s"][0, :T // G, 5])
    assert np.array_equal(a0["v_code"], a1["v_code"])


# ---------------------------------------------------------------------------
# attention ("4.4 KV Cache 量化", section 2)
# ---------------------------------------------------------------------------

def _numpy_attention(q, K, V, sigma):
    s = (K.astype(np.float64) @ q.astype(np.float64)) * sigma
    p = np.exp(s - s.max())
    return (p[:, None] * V.astype(np.float64)).sum(0) / p.sum()


def test_residual_only_equals_textbook_attention():
    """T < R: nothing is quantised, attention is plain softmax attention on the inputs."""
    rng = np.random.default_rng(11)
    H, HQ, d, R, T = 2, 6, 32, 16, 15
    kb, vb = _stream(rng, T, H, d)
    c = oracle.SeqCache(H, d, 4, 8, 16, R, DT_F16, T)
    c.append(kb, vb)
    assert c.state() == (T, 0, 0)
    qb = f16(rng.standard_normal((1, HQ, d))).view(np.uint16)
    sigma = 1 / math.sqrt(d)
    out = oracle.attention_all([c], HQ, qb, DT_F16, [0, 1], sigma, False)
    K = kb.view(np.float16).astype(np.float64)
    V = vb.view(np.float16).astype(np.float64)
    q = qb.view(np.float16).astype(np.float64)
    for hq in range(HQ):
        want = _numpy_attention(q[0, hq], K[:, hq // 3], V[:, hq // 3], sigma)
        np.testing.assert_allclose(out[0, hq], want, rtol=1e-12, atol=1e-13)


def _grid_exact_stream(rng, T, H, d, G, Gv, bits):
    """K with every (token-group, channel) grid-exact and V with every (token, channel-group)
    grid-exact, so quantisation reproduces the inputs exactly."""
    Q = 2 ** bits - 1
    K = np.zeros((T, H, d))
    V = np.zeros((T, H, d))
    for h in range(H):
        for j in range((T + G - 1) // G):
            n = min(G, T - j * G)
            for ch in range(d):
                e = int(rng.integers(-5, 0))
                z = float(rng.integers(-16, 16)) * 2.0 ** e
                k = rng.integers(0, Q + 1, n)
                if n >= 2:
                    k[0], k[-1] = 0, Q
                K[j * G:j * G + n, h, ch] = z + k * 2.0 ** e
        for t in range(T):
            for g in range(d // Gv):
                e = int(rng.integers(-5, 0))
                z = float(rng.integers(-16, 16)) * 2.0 ** e
                k = rng.integers(0, Q + 1, Gv)
                k[0], k[-1] = 0, Q
                V[t, h, g * Gv:(g + 1) * Gv] = z + k * 2.0 ** e
    return f16(K).view(np.uint16), f16(V).view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4])
def test_grid_exact_cache_attention_equals_textbook(bits):
    rng = np.random.default_rng(12)
    H, HQ, d, G, Gv, R, T = 2, 4, 16, 4, 8, 8, 37
    kb, vb = _grid_exact_stream(rng, T, H, d, G, Gv, bits)
    c = oracle.SeqCache(H, d, bits, G, Gv, R, DT_F16, T)
    c.append(kb, vb)
    _, TK, TV = c.state()
    assert TK == 32 and TV == 29
    for h in range(H):
        k, v = c.reconstruct(h)
        assert np.array_equal(k, kb[:, h].view(np.float16).astype(np.float32))
        assert np.array_equal(v, vb[:, h].view(np.float16).astype(np.float32))
    qb = f16(rng.standard_normal((1, HQ, d))).view(np.uint16)
    out = oracle.attention_all([c], HQ, qb, DT_F16, [0, 1], 0.3, False)
    K = kb.view(np.float16).astype(np.float64)
    V = vb.view(np.float16).astype(np.float64)
    q = qb.view(np.float16).astype(np.float64)
    for hq in range(HQ):
        want = _numpy_attention(q[0, hq], K[:, hq // 2], V[:, hq // 2], 0.3)
        np.testing.assert_allclose(out[0, hq], want, rtol=1e-12, atol=1e-13)


def test_tiny_brute_force_decode_and_causal_prefill():
    """d=8, G=4, R=4 (the grouping figure's sizes): oracle vs numpy float64 softmax over the
    oracle's own reconstruction, decode and causal prefill rows, GQA 2."""
    rng = np.random.default_rng(13)
    H, HQ, d, G, Gv, R = 2, 4, 8, 4, 4, 4
    lens = [11, 4, 9]
    caches, Ks, Vs = [], [], []
    for T in lens:
        kb, vb = _stream(rng, T, H, d, kscale=np.where(np.arange(d) == 3, 20.0, 1.0))
        c = oracle.SeqCache(H, d, 4, G, Gv, R, DT_F16, T)
        c.append(kb, vb)
        caches.append(c)
        rec = [c.reconstruct(h) for h in range(H)]
        Ks.append([r[0] for r in rec])
        Vs.append([r[1] for r in rec])
    sigma = 1 / math.sqrt(d)
    # decode: one row per request, attends every token
    qd = f16(rng.standard_normal((3, HQ, d))).view(np.uint16)
    out = oracle.attention_all(caches, HQ, qd, DT_F16, [0, 1, 2, 3], sigma, False)
    for s in range(3):
        for hq in range(HQ):
            want = _numpy_attention(qd[s, hq].view(np.float16), Ks[s][hq // 2], Vs[s][hq // 2], sigma)
            np.testing.assert_allclose(out[s, hq], want, rtol=1e-12, atol=1e-13)
    # prefill: n_q rows per request at positions T - n_q + i, causal
    nq = [3, 4, 1]
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qp = f16(rng.standard_normal((cu[-1], HQ, d))).view(np.uint16)
    outp = oracle.attention_all(caches, HQ, qp, DT_F16, cu, sigma, True)
    for s in range(3):
        for i in range(nq[s]):
            pos = lens[s] - nq[s] + i
            for hq in range(HQ):
                want = _numpy_attention(qp[cu[s] + i, hq].view(np.float16),
                                        Ks[s][hq // 2][:pos + 1], Vs[s][hq // 2][:pos + 1], sigma)
                np.testing.assert_allclose(outp[cu[s] + i, hq], want, rtol=1e-12, atol=1e-13)


def test_gqa_equals_independent_mha():
    """H_Q = g H_KV is g independent single-head problems per KV head, query heads grouped
    consecutively."""
    rng = np.random.default_rng(14)
    H, g, d, T = 3, 4, 16, 40
    kb, vb = _stream(rng, T, H, d)
    full = oracle.SeqCache(H, d, 4, 8, 8, 16, DT_F16, T)
    full.append(kb, vb)
    qb = f16(rng.standard_normal((1, H * g, d))).view(np.uint16)
    out = oracle.attention_all([full], H * g, qb, DT_F16, [0, 1], 0.25, False)
    for h in range(H):
        one = oracle.SeqCache(1, d, 4, 8, 8, 16, DT_F16, T)
        one.append(np.ascontiguousarray(kb[:, h:h + 1]), np.ascontiguousarray(vb[:, h:h + 1]))
        o1 = oracle.attention_all([one], g, np.ascontiguousarray(qb[:, h * g:(h + 1) * g]), DT_F16,
                                  [0, 1], 0.25, False)
        assert np.array_equal(o1[0], out[0, h * g:(h + 1) * g])


def test_empty_sequence_row_is_zero():
    c = oracle.SeqCache(1, 8, 4, 4, 4, 4, DT_F16, 4)
    q = np.zeros((1, 1, 8), dtype=np.uint16)
    out = oracle.attention_all([c], 1, q, DT_F16, [0, 1], 1.0, False)
    assert np.all(out == 0)


# ---------------------------------------------------------------------------
# prefill with the chunk at full precision (the chunk is quantised for storage
# only; its rows see the history as stored before the chunk plus the chunk's
# own Keys and Values as given)
# ---------------------------------------------------------------------------

def _f64(bits):
    return bits.view(np.float16).astype(np.float64)


def test_raw_chunk_history_in_residual_equals_textbook():
    """History shorter than R is all full precision, so every row is plain softmax attention
    over the input stream, although the chunk (20 rows, R = 16) is long enough that storing
    it first would quantise some of its own tokens."""
    rng = np.random.default_rng(21)
    H, HQ, d, G, Gv, R, P, nq = 2, 4, 16, 8, 8, 16, 10, 20
    kb, vb = _stream(rng, P + nq, H, d)
    c = oracle.SeqCache(H, d, 4, G, Gv, R, DT_F16, P + nq)
    c.append(kb[:P], vb[:P])
    qb = f16(rng.standard_normal((nq, HQ, d))).view(np.uint16)
    sigma = 1 / math.sqrt(d)
    cu = [0, nq]
    out = oracle.attention_raw_chunk([c], HQ, qb, DT_F16, cu, kb[P:], vb[P:], sigma, True)
    K, V = _f64(kb), _f64(vb)
    for i in range(nq):
        for hq in range(HQ):
            want = _numpy_attention(_f64(qb)[i, hq], K[:P + i + 1, hq // 2], V[:P + i + 1, hq // 2], sigma)
            np.testing.assert_allclose(out[i, hq], want, rtol=1e-12, atol=1e-13)
    # the stored reading of the same chunk differs (its oldest chunk tokens were quantised)
    c.append(kb[P:], vb[P:])
    assert c.state()[1] > P
    stored = oracle.attention_all([c], HQ, qb, DT_F16, cu, sigma, True)
    assert not np.allclose(stored[-1], out[-1], rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("bits", [2, 4])
def test_raw_chunk_grid_exact_history_equals_textbook(bits):
    """Quantised history that reproduces its inputs exactly, followed by a chunk of arbitrary
    values: causal and non-causal rows equal softmax attention over the input stream."""
    rng = np.random.default_rng(22)
    H, HQ, d, G, Gv, R, P, nq = 2, 4, 16, 4, 8, 8, 37, 9
    kh, vh = _grid_exact_stream(rng, P, H, d, G, Gv, bits)
    kc, vc = _stream(rng, nq, H, d)
    c = oracle.SeqCache(H, d, bits, G, Gv, R, DT_F16, P)
    c.append(kh, vh)
    assert c.state() == (37, 32, 29)
    K, V = _f64(np.concatenate([kh, kc])), _f64(np.concatenate([vh, vc]))
    qb = f16(rng.standard_normal((nq, HQ, d))).view(np.uint16)
    for causal in (True, False):
        out = oracle.attention_raw_chunk([c], HQ, qb, DT_F16, [0, nq], kc, vc, 0.3, causal)
        for i in range(nq):
            n = P + i + 1 if causal else P + nq
            for hq in range(HQ):
                want = _numpy_attention(_f64(qb)[i, hq], K[:n, hq // 2], V[:n, hq // 2], 0.3)
                np.testing.assert_allclose(out[i, hq], want, rtol=1e-12, atol=1e-13)


def test_raw_chunk_brute_force_ragged():
    """Three requests with ragged history and chunk lengths (one with no history) and GQA 2:
    every row equals numpy softmax over the reconstructed history followed by the raw chunk,
    and selected items equal the corresponding full outputs."""
    rng = np.random.default_rng(23)
    H, HQ, d, G, Gv, R = 2, 4, 8, 4, 4, 4
    hist, nq = [11, 0, 6], [3, 5, 1]
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    caches, Ks, Vs, kcs, vcs = [], [], [], [], []
    for P, n in zip(hist, nq):
        kb, vb = _stream(rng, P + n, H, d, kscale=np.where(np.arange(d) == 3, 20.0, 1.0))
        c = oracle.SeqCache(H, d, 2, G, Gv, R, DT_F16, P + n)
        c.append(kb[:P], vb[:P])
        caches.append(c)
        rec = [c.reconstruct(h) for h in range(H)]
        Ks.append([np.concatenate([r[0], _f64(kb[P:, h])]) for h, r in enumerate(rec)])
        Vs.append([np.concatenate([r[1], _f64(vb[P:, h])]) for h, r in enumerate(rec)])
        kcs.append(kb[P:])
        vcs.append(vb[P:])
    kc, vc = np.concatenate(kcs), np.concatenate(vcs)
    qb = f16(rng.standard_normal((cu[-1], HQ, d))).view(np.uint16)
    sigma = 1 / math.sqrt(d)
    out = oracle.attention_raw_chunk(caches, HQ, qb, DT_F16, cu, kc, vc, sigma, True)
    for s in range(3):
        for i in range(nq[s]):
            n = hist[s] + i + 1
            for hq in range(HQ):
                want = _numpy_attention(_f64(qb)[cu[s] + i, hq], Ks[s][hq // 2][:n], Vs[s][hq // 2][:n], sigma)
                np.testing.assert_allclose(out[cu[s] + i, hq], want, rtol=1e-12, atol=1e-13)
    rows = np.array([8, 0, 3, 3], np.int32)
    heads = np.array([1, 3, 0, 2], np.int32)
    sel = oracle.attention_raw_chunk(caches, HQ, qb, DT_F16, cu, kc, vc, sigma, True, rows, heads)
    assert np.array_equal(sel, out[rows, heads])


def test_raw_chunk_single_token_without_history_is_its_value():
    """One chunk token and no history: the softmax has one term, the output is that token's
    Value for every query head."""
    rng = np.random.default_rng(24)
    H, HQ, d = 2, 6, 16
    c = oracle.SeqCache(H, d, 4, 4, 4, 4, DT_F16, 1)
    kb, vb = _stream(rng, 1, H, d)
    qb = f16(rng.standard_normal((1, HQ, d))).view(np.uint16)
    out = oracle.attention_raw_chunk([c], HQ, qb, DT_F16, [0, 1], kb, vb, 0.7, False)
    for hq in range(HQ):
        assert np.array_equal(out[0, hq], _f64(vb)[0, hq // 3])
