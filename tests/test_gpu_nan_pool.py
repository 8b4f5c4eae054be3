"""A pool whose unwritten bytes are all 0xFF (every unwritten fp16, bf16 and E4M3 value
is a NaN): pages that no sequence owns, page 0 included, the tail of a sequence's last
page, stale residual rows. Nothing the method has not written may reach an output, so
decode, the fused step and prefill (int4, int2, FP8) match the oracle with no NaN.
Pages are shuffled over a 1.5x pool, lengths are not multiples of the 16-token tile,
and a sequence's main range is cut unevenly over its waves (tiles outside a wave's range
ride along in its load buffers with zero weights)."""
import numpy as np
import pytest

from kivi_quantized_kv_append_amd import inputs
from harness import (SCALE, Fp8GpuCache, GpuCache, amax_scales, check_attention, fp8_oracle_caches,
                     oracle_caches)
import oracle

pytestmark = pytest.mark.gpu


def _w(bits=4, **kw):
    base = dict(num_seqs=5, seq_lens=[700, 1290, 63, 2047, 385], extra_tokens=20, shuffle=True, pool_factor=1.5)
    base.update(kw)
    return inputs.config(2, bits=bits, **base)


@pytest.mark.parametrize("bits", [4, 2])
def test_kivi_paths_on_a_nan_pool(bits):
    w = _w(bits)
    gc = GpuCache(w, fill_byte=0xFF)
    S = w.num_seqs
    T0 = w.seq_lens.astype(np.int64)
    rk, rv = zip(*[w.kv_stream(s, 0, int(T0[s])) for s in range(S)])
    gc.append(list(rk), list(rv))
    orcs = oracle_caches(w)
    q = w.q_decode(0)
    got = gc.decode(q, SCALE)
    assert not np.isnan(inputs.bits_to_float(got, w.dtype)).any()
    check_attention(got, oracle.attention_all(orcs, w.num_q_heads, q, w.dtype, np.arange(S + 1), SCALE, False),
                    w.dtype, label=f"int{bits} decode on a NaN pool")
    for i in range(3):  # fused steps (seq 3 flushes at the first)
        k = np.stack([w.kv_stream(s, int(gc.lens[s]), int(gc.lens[s]) + 1)[0][0] for s in range(S)])
        v = np.stack([w.kv_stream(s, int(gc.lens[s]), int(gc.lens[s]) + 1)[1][0] for s in range(S)])
        got = gc.decode_step(k, v, w.q_decode(1 + i), SCALE)
        for s in range(S):
            orcs[s].append(k[s:s + 1], v[s:s + 1])
        ref = oracle.attention_all(orcs, w.num_q_heads, w.q_decode(1 + i), w.dtype, np.arange(S + 1), SCALE, False)
        check_attention(got, ref, w.dtype, label=f"int{bits} fused step {i} on a NaN pool")
    n = 17
    rk, rv = zip(*[w.kv_stream(s, int(gc.lens[s]), int(gc.lens[s]) + n) for s in range(S)])
    gc.append(list(rk), list(rv))
    for s in range(S):
        orcs[s].append(rk[s], rv[s])
    cu = np.arange(0, (S + 1) * n, n)
    qp = inputs.to_bits(np.random.default_rng(4).standard_normal((S * n, w.num_q_heads, 128)), w.dtype)
    got = gc.prefill(qp, cu, SCALE, causal=True)
    check_attention(got, oracle.attention_all(orcs, w.num_q_heads, qp, w.dtype, cu, SCALE, True, threads=8),
                    w.dtype, label=f"int{bits} prefill on a NaN pool")


def test_fp8_paths_on_a_nan_pool():
    w = _w(4)
    ks, vs = amax_scales(w, per_head=True)
    g8 = Fp8GpuCache(w, ks, vs, per_head=True, fill_byte=0xFF)
    S = w.num_seqs
    T0 = w.seq_lens.astype(np.int64)
    rk, rv = zip(*[w.kv_stream(s, 0, int(T0[s])) for s in range(S)])
    g8.append(list(rk), list(rv))
    o8 = fp8_oracle_caches(w, ks, vs, True)
    q = w.q_decode(0)
    got = g8.decode(q, SCALE)
    check_attention(got, oracle.fp8_attention(o8, w.num_q_heads, q, w.dtype, SCALE), w.dtype,
                    label="fp8 decode on a NaN pool")
    k = np.stack([w.kv_stream(s, int(T0[s]), int(T0[s]) + 1)[0][0] for s in range(S)])
    v = np.stack([w.kv_stream(s, int(T0[s]), int(T0[s]) + 1)[1][0] for s in range(S)])
    got = g8.step(w.q_decode(1), k, v, SCALE)
    for s in range(S):
        o8[s].append(k[s:s + 1], v[s:s + 1])
    check_attention(got, oracle.fp8_attention(o8, w.num_q_heads, w.q_decode(1), w.dtype, SCALE), w.dtype,
                    label="fp8 step on a NaN pool")
    cu = np.array([0, 1, 2, 3, 4, 5])
    got = g8.prefill(w.q_decode(2), cu, SCALE, causal=True)
    ref = oracle.fp8_attention_rows(o8, w.num_q_heads, w.q_decode(2), w.dtype, cu, SCALE, True)
    check_attention(got, ref, w.dtype, label="fp8 prefill on a NaN pool")
