"""GPU parity of prefill with the chunk at full precision (kivi_prefill_attention_raw_chunk)
against the CPU oracle, through the C ABI.

The cache holds each request's history; the call comes before the chunk is stored, the
chunk's rows sit after the history and take part with their own Keys and Values as given.
The oracle's caches hold the same history and get the same chunk rows."""
import numpy as np
import pytest

from kivi_quantized_kv_append_amd import inputs
from harness import SCALE, GpuCache, check_attention, oracle_caches
import oracle

pytestmark = pytest.mark.gpu


def _chunk_rows(w, chunk_lens):
    """The chunk rows of every request (the stream tokens after its history), concatenated."""
    ks, vs = [], []
    for s, n in enumerate(chunk_lens):
        P = int(w.seq_lens[s])
        k, v = w.kv_stream(s, P, P + n)
        ks.append(k)
        vs.append(v)
    return np.concatenate(ks), np.concatenate(vs)


def _raw_chunk_case(w, chunk_lens, causal, seed=9, check_pool=False):
    gc = GpuCache(w)
    rk, rv = zip(*[w.kv_stream(s, 0, int(w.seq_lens[s])) for s in range(w.num_seqs)])
    gc.append(list(rk), list(rv))
    orc = oracle_caches(w)  # the history only
    cu = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int64)
    kc, vc = _chunk_rows(w, chunk_lens)
    q = inputs.to_bits(np.random.default_rng(seed).standard_normal((int(cu[-1]), w.num_q_heads, 128))
                       * w.q_scale, w.dtype)
    before = gc.pool.clone() if check_pool else None
    got = gc.prefill_raw_chunk(q, cu, kc, vc, SCALE, causal=causal)
    if check_pool:
        assert bool((gc.pool == before).all()), "the call wrote to the cache"
    ref = oracle.attention_raw_chunk(orc, w.num_q_heads, q, w.dtype, cu, kc, vc, SCALE, causal, threads=8)
    check_attention(got, ref, w.dtype, label=f"{w.name} raw-chunk prefill causal={causal}")
    return gc, q, cu, kc, vc


def test_raw_chunk_qwen_shape_causal():
    """Qwen2.5-7B head shape (28 Q / 4 KV, bf16, G=R=128), reduced lengths; the call leaves
    the cache untouched."""
    w = inputs.config(5, num_seqs=2, seq_lens=[700, 333], extra_tokens=64, shuffle=True, pool_factor=1.5)
    _raw_chunk_case(w, [64, 64], causal=True, check_pool=True)


def test_raw_chunk_ragged_int2():
    w = inputs.config(1, bits=2, num_seqs=3, num_kv_heads=2, num_q_heads=6, k_group=32, v_group=32,
                      residual=64, seq_lens=[150, 400, 37], extra_tokens=90, shuffle=True, pool_factor=1.5)
    _raw_chunk_case(w, [90, 17, 1], causal=True)
    _raw_chunk_case(w, [90, 17, 1], causal=False)
    _raw_chunk_case(w, [0, 17, 90], causal=True)  # a request with no rows in this call


def test_raw_chunk_without_history_and_longer_than_residual():
    """One request has no history (the rows see only the chunk); chunks of 300 tokens with
    R = 128, so storing them first would have quantised most of their own tokens."""
    w = inputs.config(5, num_seqs=2, seq_lens=[0, 250], extra_tokens=300, shuffle=True, pool_factor=1.5)
    _raw_chunk_case(w, [300, 300], causal=True)


@pytest.mark.parametrize("g", [1, 16])
def test_raw_chunk_gqa_extremes(g):
    w = inputs.config(2, num_seqs=2, num_kv_heads=2, num_q_heads=2 * g, seq_lens=[500, 260],
                      extra_tokens=40, shuffle=True, pool_factor=1.25)
    _raw_chunk_case(w, [40, 25], causal=True)


def test_raw_chunk_then_store_then_decode():
    """The call order the entry point documents: attend with the chunk at full precision,
    then store the chunk, then decode over the stored cache; the decode matches the oracle
    cache that holds history and chunk."""
    w = inputs.config(1, num_seqs=3, num_kv_heads=2, num_q_heads=8, seq_lens=[200, 63, 129], extra_tokens=70,
                      shuffle=True, pool_factor=1.5)
    gc, _, _, kc, vc = _raw_chunk_case(w, [70, 70, 70], causal=True)
    gc.append([kc[70 * s:70 * (s + 1)] for s in range(3)], [vc[70 * s:70 * (s + 1)] for s in range(3)])
    orc = oracle_caches(w, lens=w.final_lens)
    qd = inputs.to_bits(np.random.default_rng(4).standard_normal((3, w.num_q_heads, 128)) * w.q_scale, w.dtype)
    got = gc.decode(qd, SCALE)
    ref = oracle.attention_all(orc, w.num_q_heads, qd, w.dtype, np.arange(4), SCALE, False, threads=8)
    check_attention(got, ref, w.dtype, label="decode after raw-chunk prefill and store")


def test_raw_chunk_qwen_full_size_sampled():
    """Full Qwen2.5-7B prefill workload (8 requests x 16384 cached + a 512-token chunk, bf16,
    int4 G=R=128) with the chunk at full precision: every output is computed, a sample of
    (row, head) outputs, including every request's first and last row, is checked."""
    w = inputs.config(5)
    S, C, P = w.num_seqs, w.extra_tokens, int(w.seq_lens[0])
    gc = GpuCache(w)
    rk, rv = zip(*[w.kv_stream(s, 0, P) for s in range(S)])
    gc.append(list(rk), list(rv))
    orc = oracle_caches(w)
    cu = np.arange(0, (S + 1) * C, C)
    kc, vc = _chunk_rows(w, [C] * S)
    q = inputs.to_bits(np.random.default_rng(7).standard_normal((S * C, w.num_q_heads, 128)), w.dtype)
    got = gc.prefill_raw_chunk(q, cu, kc, vc, SCALE, causal=True)
    rng = np.random.default_rng(5)
    rows = np.concatenate([np.arange(0, S * C, C), np.arange(C - 1, S * C, C),
                           rng.integers(0, S * C, 200)]).astype(np.int32)
    heads = rng.integers(0, w.num_q_heads, rows.size).astype(np.int32)
    ref = oracle.attention_raw_chunk(orc, w.num_q_heads, q, w.dtype, cu, kc, vc, SCALE, True, rows, heads,
                                     threads=8)
    check_attention(got[rows, heads], ref, w.dtype, label="qwen full-size raw-chunk prefill (sampled)")
