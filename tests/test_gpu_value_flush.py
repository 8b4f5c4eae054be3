"""GPU parity of a cache whose Values leave the residual together with the Keys
(v_flush = 1: at each Key flush the R residual tokens are also quantised per
token, so both boundaries are R*floor(T/R)) against the CPU oracle, through the
C ABI: appends bit for bit, decode, the decode step and both prefill calls
within the attention tolerance."""
import numpy as np
import pytest

from kivi_quantized_kv_append_amd import inputs
from harness import SCALE, GpuCache, check_attention, compare_seq_state, oracle_caches
import oracle
from test_gpu_decode_step import _run as _decode_step_run
from test_gpu_parity import _append_and_compare
from test_gpu_prefill import _prefill_case
from test_gpu_prefill_raw_chunk import _raw_chunk_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", [4, 2])
def test_value_flush_append_stream_bitexact_and_decode(bits):
    """The tiny single-head case (G = Gv = R = 32): single tokens across flushes and bulk
    appends of several residuals, state compared after every call, decode after each."""
    w = inputs.config(1, bits=bits, v_flush=1)
    plan = [1] * 40 + [7, 33, 64, 1, 1, 110]
    _append_and_compare(w, plan, decode_every=True)


@pytest.mark.parametrize("bits,G,Gv,R,Bk,H,dtype", [
    (4, 16, 16, 48, 16, 2, inputs.F16),
    (2, 64, 128, 128, 32, 3, inputs.BF16),
])
def test_value_flush_append_variants_bitexact(bits, G, Gv, R, Bk, H, dtype):
    w = inputs.config(1, bits=bits, k_group=G, v_group=Gv, residual=R, block_size=Bk, num_kv_heads=H,
                      num_q_heads=4 * H, dtype=dtype, num_seqs=3, seq_lens=[700, 333, 517], shuffle=True,
                      pool_factor=1.5, n_outlier=2, v_flush=1)
    _append_and_compare(w, [1, 1, 5, 16, 63, 1, 1, 128, 200, 3, 300], decode_every=True)


@pytest.mark.parametrize("bits", [4, 2])
def test_value_flush_decode_ragged_llama_shape(bits):
    """32 Q / 8 KV heads, lengths on both sides of residual multiples (an empty residual
    at 128 and 256, a full one at 255)."""
    lens = [0, 1, 127, 128, 129, 255, 256, 1000, 2049]
    w = inputs.config(2, bits=bits, num_seqs=len(lens), seq_lens=lens, shuffle=True, pool_factor=1.25,
                      v_flush=1)
    gc = GpuCache(w)
    orc = oracle_caches(w)
    rk, rv = zip(*[w.kv_stream(s) for s in range(w.num_seqs)])
    gc.append(list(rk), list(rv))
    pv = gc.pool_view()
    for s in range(w.num_seqs):
        for h in (0, 7):
            compare_seq_state(pv.seq_state(gc.bt_np[s], s, int(w.seq_lens[s]), h), orc[s], h,
                              label=f"seq {s} head {h}")
    q = w.q_decode(0)
    got = gc.decode(q, SCALE)
    ref = oracle.attention_all(orc, w.num_q_heads, q, w.dtype, np.arange(w.num_seqs + 1), SCALE, False,
                               threads=8)
    check_attention(got, ref, w.dtype, label="value-flush ragged decode")
    assert np.all(got[0] == 0)


def test_value_flush_decode_step_across_flushes():
    """kivi_decode_step on a v_flush cache (an append launch, then the attention over
    T + 1 tokens): 40 steps with R = 32 cross every sequence's flush at least once."""
    w = inputs.config(1, bits=4, k_group=32, v_group=32, residual=32, num_kv_heads=2, num_q_heads=8,
                      num_seqs=6, seq_lens=[0, 1, 31, 32, 95, 300], extra_tokens=40, shuffle=True,
                      pool_factor=1.5, n_outlier=2, v_flush=1)
    _decode_step_run(w, 40)


def test_value_flush_decode_step_with_splits():
    w = inputs.config(3, num_seqs=2, seq_lens=[5000, 8191], extra_tokens=4, shuffle=True, pool_factor=1.25,
                      v_flush=1)
    _decode_step_run(w, 4, check_every=3)


def test_value_flush_prefill():
    """Chunks appended then attended (causal and over all tokens), with chunks shorter and
    longer than the residual."""
    w = inputs.config(1, bits=4, num_seqs=3, num_kv_heads=2, num_q_heads=6, k_group=32, v_group=32,
                      residual=64, seq_lens=[150, 400, 37], extra_tokens=90, shuffle=True, pool_factor=1.5,
                      v_flush=1)
    _prefill_case(w, [90, 17, 1], causal=True)
    _prefill_case(w, [90, 17, 1], causal=False)
    w5 = inputs.config(5, num_seqs=2, seq_lens=[0, 250], extra_tokens=300, shuffle=True, pool_factor=1.5,
                       v_flush=1)
    _prefill_case(w5, [300, 300], causal=True)


def test_value_flush_raw_chunk_prefill():
    """The chunk at full precision over a v_flush history (histories of 150, 256 and 37
    tokens: a partial residual, an empty one, no quantised tokens)."""
    w = inputs.config(1, bits=2, num_seqs=3, num_kv_heads=2, num_q_heads=6, k_group=32, v_group=32,
                      residual=64, seq_lens=[150, 256, 37], extra_tokens=90, shuffle=True, pool_factor=1.5,
                      v_flush=1)
    _raw_chunk_case(w, [90, 17, 1], causal=True, check_pool=True)
    _raw_chunk_case(w, [90, 17, 1], causal=False)
