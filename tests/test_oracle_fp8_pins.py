"""Pins of the oracle's FP8 (E4M3) cache ("4.4 KV Cache 量化", section 4: the KV cache
stored as FP8, E4M3 on ROCm, with one scale per tensor or per KV head).

The E4M3 conversions are checked against torch's float8_e4m3fn (a library routine
written from the OCP definition), the cache against element-wise encoding done with
that routine, and the attention against numpy float64 softmax over values restored
by hand."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import DT_BF16, DT_F16


def _torch_e4m3(y):
    """torch's float32 -> E4M3FN codes (round to nearest even; NaN above 464)."""
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_matches_library_for_every_code():
    codes = np.arange(256)
    got = oracle.e4m3_to_f32(codes)
    want = _torch_e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))  # signed zeros too
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_library_in_range():
    rng = np.random.default_rng(31)
    vals = [rng.standard_normal(3000) * sc for sc in (1e-3, 0.02, 1.0, 30.0, 200.0)]
    grid = _torch_e4m3_value(np.arange(0x7F)).astype(np.float64)
    mids = (grid[1:] + grid[:-1]) / 2  # exact ties between neighbours (exact in float32)
    vals += [mids, -mids, grid, -grid, [0.0, -0.0, 464.0, -464.0, 463.99, 2.0 ** -10, 3 * 2.0 ** -11]]
    y = np.concatenate([np.asarray(v, np.float64) for v in vals]).astype(np.float32)
    y = y[np.abs(y) <= 464.0]
    got = oracle.f32_to_e4m3(y)
    want = _torch_e4m3(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (y[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_saturates_beyond_the_largest_value():
    """Reading of the pages' 'scale into range': values past 448 store +-448."""
    y = np.array([465.0, 480.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert list(oracle.f32_to_e4m3(y)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_round_trip_within_half_spacing():
    rng = np.random.default_rng(32)
    y = (rng.standard_normal(5000) * rng.choice([0.01, 1.0, 100.0], 5000)).astype(np.float32)
    y = np.clip(y, -448, 448)
    back = oracle.e4m3_to_f32(oracle.f32_to_e4m3(y)).astype(np.float64)
    a = np.abs(y.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half = np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
    assert np.all(np.abs(back - y) <= half)


def _stream(rng, T, H, d, dtype):
    k = rng.standard_normal((T, H, d)) * 3.0
    v = rng.standard_normal((T, H, d))
    if dtype == DT_F16:
        return k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16)
    to = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731
    return to(k), to(v)


def _as_f32(bits, dtype):
    return oracle.f32_from_bf16_bits(bits) if dtype == DT_BF16 else oracle.f32_from_f16_bits(bits)


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("dtype", [DT_F16, DT_BF16])
def test_fp8_cache_codes_are_elementwise_encoding(per_head, dtype):
    """Every stored code is E4M3(x / scale) of its own element, with its head's scale."""
    rng = np.random.default_rng(33)
    H, d, T = 3, 32, 41
    kb, vb = _stream(rng, T, H, d, dtype)
    ks = np.array([0.01, 0.5, 2.0] if per_head else [0.25], np.float32)
    vs = np.array([0.01, 1.0, 0.125] if per_head else [0.02], np.float32)
    c = oracle.Fp8SeqCache(H, d, dtype, T, ks, vs, per_head)
    c.append(kb[:7], vb[:7])
    c.append(kb[7:], vb[7:])
    assert len(c) == T
    a = c.arrays()
    kf, vf = _as_f32(kb, dtype), _as_f32(vb, dtype)
    for h in range(H):
        sk, sv = (ks[h], vs[h]) if per_head else (ks[0], vs[0])
        yk = (kf[:, h] / sk).astype(np.float32)
        yv = (vf[:, h] / sv).astype(np.float32)
        if per_head and h == 0:
            assert np.abs(yk).max() > 464  # saturation takes part
        ck = np.where(np.abs(yk) > 448, np.where(yk > 0, 0x7E, 0xFE), _torch_e4m3(np.clip(yk, -448, 448)))
        cv = np.where(np.abs(yv) > 448, np.where(yv > 0, 0x7E, 0xFE), _torch_e4m3(np.clip(yv, -448, 448)))
        assert np.array_equal(a["k_code"][h, :T], ck.astype(np.uint8))
        assert np.array_equal(a["v_code"][h, :T], cv.astype(np.uint8))


def _numpy_attention(q, K, V, sigma):
    s = (K.astype(np.float64) @ q.astype(np.float64)) * sigma
    p = np.exp(s - s.max())
    return (p[:, None] * V.astype(np.float64)).sum(0) / p.sum()


@pytest.mark.parametrize("per_head", [False, True])
def test_fp8_attention_brute_force(per_head):
    """Decode attention (GQA 3) over restored values value(E4M3(x/s)) * s, computed by hand
    with torch's conversion, against numpy float64 softmax."""
    rng = np.random.default_rng(34)
    H, HQ, d, T = 2, 6, 16, 37
    kb, vb = _stream(rng, T, H, d, DT_F16)
    ks = np.array([0.02, 0.07] if per_head else [0.03], np.float32)
    vs = np.array([0.005, 0.011] if per_head else [0.008], np.float32)
    c = oracle.Fp8SeqCache(H, d, DT_F16, T, ks, vs, per_head)
    c.append(kb, vb)
    qb = (rng.standard_normal((1, HQ, d)) / math.sqrt(d)).astype(np.float16).view(np.uint16)
    out = oracle.fp8_attention([c], HQ, qb, DT_F16, 0.7)
    kf, vf = _as_f32(kb, DT_F16), _as_f32(vb, DT_F16)
    q = qb.view(np.float16).astype(np.float64)
    for hq in range(HQ):
        h = hq // 3
        sk, sv = (ks[h], vs[h]) if per_head else (ks[0], vs[0])
        K = (_torch_e4m3_value(_torch_e4m3(np.clip(kf[:, h] / sk, -448, 448))) * sk).astype(np.float32)
        V = (_torch_e4m3_value(_torch_e4m3(np.clip(vf[:, h] / sv, -448, 448))) * sv).astype(np.float32)
        np.testing.assert_allclose(out[0, hq], _numpy_attention(q[0, hq], K, V, 0.7), rtol=1e-12, atol=1e-13)


def test_fp8_grid_inputs_restore_exactly():
    """Inputs that are E4M3 values times a power-of-two scale are stored without loss: the
    attention equals textbook softmax attention over the inputs themselves."""
    rng = np.random.default_rng(35)
    H, HQ, d, T = 1, 2, 16, 29
    grid = _torch_e4m3_value(np.arange(0x7F)).astype(np.float64)
    grid = grid[grid <= 16]
    signs = rng.choice([-1.0, 1.0], (T, H, d, 2))
    k = rng.choice(grid, (T, H, d)) * signs[..., 0] * 0.125
    v = rng.choice(grid, (T, H, d)) * signs[..., 1] * 2.0 ** -5
    kb, vb = k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16)
    assert np.array_equal(kb.view(np.float16).astype(np.float64), k)
    c = oracle.Fp8SeqCache(H, d, DT_F16, T, [0.125], [2.0 ** -5], False)
    c.append(kb, vb)
    qb = rng.standard_normal((1, HQ, d)).astype(np.float16).view(np.uint16)
    out = oracle.fp8_attention([c], HQ, qb, DT_F16, 0.2)
    q = qb.view(np.float16).astype(np.float64)
    for hq in range(HQ):
        np.testing.assert_allclose(out[0, hq], _numpy_attention(q[0, hq], k[:, 0], v[:, 0], 0.2),
                                   rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill_rows_brute_force(causal):
    """Prefill rows (GQA 2, two requests, one with more rows than tokens) against numpy float64
    softmax over values restored by hand with torch's conversion; rows that see no token are zero."""
    rng = np.random.default_rng(36)
    H, HQ, d = 2, 4, 16
    lens, nqs = [23, 5], [6, 7]
    ks, vs = np.array([0.03, 0.05], np.float32), np.array([0.01, 0.02], np.float32)
    caches, kv = [], []
    for T in lens:
        kb, vb = _stream(rng, T, H, d, DT_F16)
        c = oracle.Fp8SeqCache(H, d, DT_F16, T, ks, vs, True)
        c.append(kb, vb)
        caches.append(c)
        kv.append((_as_f32(kb, DT_F16), _as_f32(vb, DT_F16)))
    cu = np.concatenate([[0], np.cumsum(nqs)])
    qb = (rng.standard_normal((int(cu[-1]), HQ, d)) / math.sqrt(d)).astype(np.float16).view(np.uint16)
    out = oracle.fp8_attention_rows(caches, HQ, qb, DT_F16, cu, 0.6, causal)
    q = qb.view(np.float16).astype(np.float64)
    for s, (T, nq) in enumerate(zip(lens, nqs)):
        kf, vf = kv[s]
        for i in range(nq):
            r = cu[s] + i
            n = min(T - nq + i + 1, T) if causal else T
            for hq in range(HQ):
                h = hq // 2
                if n <= 0:
                    assert np.all(out[r, hq] == 0)
                    continue
                K = (_torch_e4m3_value(_torch_e4m3(np.clip(kf[:n, h] / ks[h], -448, 448))) * ks[h]).astype(np.float32)
                V = (_torch_e4m3_value(_torch_e4m3(np.clip(vf[:n, h] / vs[h], -448, 448))) * vs[h]).astype(np.float32)
                np.testing.assert_allclose(out[r, hq], _numpy_attention(q[r, hq], K, V, 0.6), rtol=1e-12, atol=1e-13)


def test_fp8_empty_sequence_row_is_zero():
    c = oracle.Fp8SeqCache(1, 16, DT_F16, 4, [1.0], [1.0], False)
    out = oracle.fp8_attention([c], 2, np.zeros((1, 2, 16), np.uint16), DT_F16, 0.25)
    assert np.all(out == 0)
