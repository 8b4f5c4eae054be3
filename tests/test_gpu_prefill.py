"""GPU parity of chunked-prefill attention against the CPU oracle, through the C ABI.

The cache is built by appending every sequence's cached tokens plus its chunk
(the chunk is appended before it attends); the chunk's queries then attend over
the stored cache, causally (row i at position T - n_q + i sees tokens 0..its own)
or over all T tokens."""
import numpy as np
import pytest

from kivi_quantized_kv_append_amd import inputs
from harness import SCALE, GpuCache, check_attention, compare_seq_state, oracle_caches
import oracle

pytestmark = pytest.mark.gpu


def _prefill_case(w, chunk_lens, causal, seed=7):
    """Append the streams, run prefill for the given chunk lengths (<= the
    workload's extra tokens), compare every output with the oracle."""
    gc = GpuCache(w)
    rk, rv = zip(*[w.kv_stream(s) for s in range(w.num_seqs)])
    gc.append(list(rk), list(rv))
    orc = oracle_caches(w, lens=w.final_lens)
    cu = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int64)
    rng = np.random.default_rng(seed)
    q = inputs.to_bits(rng.standard_normal((int(cu[-1]), w.num_q_heads, 128)) * w.q_scale, w.dtype)
    got = gc.prefill(q, cu, SCALE, causal=causal)
    ref = oracle.attention_all(orc, w.num_q_heads, q, w.dtype, cu, SCALE, causal, threads=8)
    return check_attention(got, ref, w.dtype, label=f"{w.name} prefill causal={causal}")


def test_prefill_qwen_shape_causal():
    """Qwen2.5-7B head shape (28 Q / 4 KV, bf16, G=R=128), reduced lengths."""
    w = inputs.config(5, num_seqs=2, seq_lens=[700, 333], extra_tokens=64, shuffle=True, pool_factor=1.5)
    _prefill_case(w, [64, 64], causal=True)


def test_prefill_ragged_chunks_int2():
    w = inputs.config(1, bits=2, num_seqs=3, num_kv_heads=2, num_q_heads=6, k_group=32, v_group=32,
                      residual=64, seq_lens=[150, 400, 37], extra_tokens=90, shuffle=True, pool_factor=1.5)
    _prefill_case(w, [90, 17, 1], causal=True)
    _prefill_case(w, [90, 17, 1], causal=False)
    _prefill_case(w, [0, 17, 90], causal=True)  # a request with no rows in this call


def test_prefill_chunk_longer_than_residual():
    """A chunk of 300 tokens with R = 128: most of the chunk's own Keys and
    Values are already quantised when it attends; one sequence is all chunk."""
    w = inputs.config(5, num_seqs=2, seq_lens=[0, 250], extra_tokens=300, shuffle=True, pool_factor=1.5)
    _prefill_case(w, [300, 300], causal=True)


@pytest.mark.parametrize("g", [1, 16])
def test_prefill_gqa_extremes(g):
    w = inputs.config(2, num_seqs=2, num_kv_heads=2, num_q_heads=2 * g, seq_lens=[500, 260],
                      extra_tokens=40, shuffle=True, pool_factor=1.25)
    _prefill_case(w, [40, 25], causal=True)


def test_prefill_qwen_full_size():
    """Full Qwen2.5-7B prefill workload (8 requests x 16384 cached + a 512-token
    chunk, bf16, int4 G=R=128), in the launch configuration the benchmark times:
    the chunk is bulk-appended in one call (split over parts), after which the
    whole cache state of every (request, KV head) is compared bit for bit with
    the oracle; every output is computed, every (row, head) output of one
    request (all 512 rows, all 28 heads) is checked against the oracle, and a
    sample across the other requests, including the first and last row of
    every request."""
    w = inputs.config(5)
    S, C, P = w.num_seqs, w.extra_tokens, int(w.seq_lens[0])
    gc = GpuCache(w)
    rk, rv = zip(*w.kv_streams(16))
    gc.append([r[:P] for r in rk], [r[:P] for r in rv])
    gc.append([r[P:] for r in rk], [r[P:] for r in rv])
    orc = oracle_caches(w, lens=w.final_lens)
    pv = gc.pool_view()
    for s in range(S):
        for h in range(w.num_kv_heads):
            st = pv.seq_state(gc.bt_np[s], s, int(w.final_lens[s]), h)
            compare_seq_state(st, orc[s], h, label=f"qwen full-size cache seq {s} head {h}")
    del pv
    print("[qwen full size] cache state bit-exact for every (request, KV head)", flush=True)
    cu = np.arange(0, (S + 1) * C, C)
    q = inputs.to_bits(np.random.default_rng(7).standard_normal((S * C, w.num_q_heads, 128)), w.dtype)
    got = gc.prefill(q, cu, SCALE, causal=True)
    # one whole request: every row and head
    s_full = 5
    rows = np.repeat(np.arange(s_full * C, (s_full + 1) * C, dtype=np.int32), w.num_q_heads)
    heads = np.tile(np.arange(w.num_q_heads, dtype=np.int32), C)
    ref = oracle.attention(orc, w.num_q_heads, q, w.dtype, cu, SCALE, True, rows, heads, threads=16)
    check_attention(got[rows, heads], ref, w.dtype, label=f"qwen full-size prefill, request {s_full}, every output")
    print(f"[qwen full size] request {s_full}: all {C} x {w.num_q_heads} outputs within tolerance", flush=True)
    rng = np.random.default_rng(5)
    rows = np.concatenate([np.arange(0, S * C, C), np.arange(C - 1, S * C, C),
                           rng.integers(0, S * C, 200)]).astype(np.int32)
    heads = rng.integers(0, w.num_q_heads, rows.size).astype(np.int32)
    ref = oracle.attention(orc, w.num_q_heads, q, w.dtype, cu, SCALE, True, rows, heads, threads=16)
    check_attention(got[rows, heads], ref, w.dtype, label="qwen full-size prefill (sampled)")


def test_prefill_large_pages():
    """64-token pages under the Qwen head shape (G = 128: a Key group spans two pages)."""
    w = inputs.config(5, num_seqs=2, seq_lens=[900, 333], extra_tokens=100, block_size=64, shuffle=True,
                      pool_factor=1.5)
    _prefill_case(w, [100, 100], causal=True)


def test_prefill_one_subtile_key_groups_narrow_value_groups():
    """G = 16 (each 16-token sub-tile of a 64-token tile has its own Key scales)
    and Gv = 16 (8 Value groups per token), fp16, R = 32, with the chunk spilling
    past the residual."""
    w = inputs.config(2, num_seqs=3, num_kv_heads=2, num_q_heads=8, k_group=16, v_group=16, residual=32,
                      seq_lens=[213, 64, 5], extra_tokens=70, shuffle=True, pool_factor=1.5)
    _prefill_case(w, [70, 33, 70], causal=True)


def test_prefill_widest_key_groups_int2_32_token_pages():
    """G = 256 over 32-token pages (8 pages per Key group), Gv = 64, int2, bf16,
    non-causal and causal."""
    w = inputs.config(5, bits=2, num_seqs=2, num_kv_heads=2, num_q_heads=6, k_group=256, v_group=64,
                      residual=256, block_size=32, seq_lens=[1100, 300], extra_tokens=120, shuffle=True,
                      pool_factor=1.5)
    _prefill_case(w, [120, 57], causal=True)
    _prefill_case(w, [120, 57], causal=False)
