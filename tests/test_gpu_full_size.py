"""GPU parity at the workloads' full sizes, through the C ABI.

* Long-context decode (4 requests x 32768 tokens, int4 and int2, G = R = 128, pages in
  a seeded random order over a 1.25x pool): the whole cache state bit for bit, and
  every decode output against the oracle.
* Ragged streaming batch (256 requests, lengths uniform in [128, 8192], int4, G = R = 64):
  64 fused decode steps (kivi_decode_step: one new token per request appended and
  attended in one launch, the call the benchmark times); after every step every byte the step
  changed (evicted Value token pages, flushed Key groups and their metadata, all
  residual windows) is compared bit for bit with the oracle, decode outputs of 16
  requests per step (all 256 over four passes) against the oracle; after the last step
  the whole state of every request.
"""
import time

import numpy as np
import pytest

from kivi_quantized_kv_append_amd import inputs
from harness import (SCALE, GpuCache, PoolMirror, check_attention, check_decode_step_state,
                     compare_seq_state)
import oracle

pytestmark = pytest.mark.gpu

THREADS = 16


def _log(msg):
    print(f"[full-size] {msg}", flush=True)


def _oracle_fill(w, streams, lens):
    caches = []
    for s in range(w.num_seqs):
        c = oracle.SeqCache(w.num_kv_heads, 128, w.bits, w.k_group, w.v_group, w.residual, w.dtype,
                            int(w.final_lens[s]))
        c.append(streams[s][0][:lens[s]], streams[s][1][:lens[s]])
        caches.append(c)
    return caches


def _full_state(gc, orcs, lens, label):
    pv = gc.pool_view()
    for s in range(len(orcs)):
        for h in range(gc.w.num_kv_heads):
            st = pv.seq_state(gc.bt_np[s], s, int(lens[s]), h)
            compare_seq_state(st, orcs[s], h, label=f"{label} seq {s} head {h}")


@pytest.mark.parametrize("bits", [4, 2])
def test_long_context_decode_full_size(bits):
    w = inputs.config(3, bits=bits, extra_tokens=1)
    t = time.time()
    streams = w.kv_streams(THREADS)
    T0 = w.seq_lens.astype(np.int64)
    gc = GpuCache(w)
    gc.append([streams[s][0][:T0[s]] for s in range(w.num_seqs)],
              [streams[s][1][:T0[s]] for s in range(w.num_seqs)])
    orcs = _oracle_fill(w, streams, T0)
    _log(f"long context int{bits}: built in {time.time() - t:.1f} s")
    _full_state(gc, orcs, T0, f"long context int{bits}")
    q = w.q_decode(0)
    got = gc.decode(q, SCALE)
    ref = oracle.attention_all(orcs, w.num_q_heads, q, w.dtype, np.arange(w.num_seqs + 1), SCALE, False,
                               threads=THREADS)
    check_attention(got, ref, w.dtype, label=f"long context int{bits} decode")
    # one more token: the Value eviction and a residual that is no longer full
    gc.append([streams[s][0][T0[s]:T0[s] + 1] for s in range(w.num_seqs)],
              [streams[s][1][T0[s]:T0[s] + 1] for s in range(w.num_seqs)])
    for s in range(w.num_seqs):
        orcs[s].append(streams[s][0][T0[s]:T0[s] + 1], streams[s][1][T0[s]:T0[s] + 1])
    q = w.q_decode(1)
    got = gc.decode(q, SCALE)
    ref = oracle.attention_all(orcs, w.num_q_heads, q, w.dtype, np.arange(w.num_seqs + 1), SCALE, False,
                               threads=THREADS)
    check_attention(got, ref, w.dtype, label=f"long context int{bits} decode after append")
    _log(f"long context int{bits}: done in {time.time() - t:.1f} s")


@pytest.mark.timeout(900)
def test_ragged_stream_64_steps_full_size():
    w = inputs.config(4)
    S, R = w.num_seqs, w.residual
    t = time.time()
    streams = w.kv_streams(THREADS)
    T0 = w.seq_lens.astype(np.int64)
    gc = GpuCache(w)
    gc.append([streams[s][0][:T0[s]] for s in range(S)], [streams[s][1][:T0[s]] for s in range(S)])
    orcs = _oracle_fill(w, streams, T0)
    mirror = PoolMirror(gc)
    _log(f"ragged stream: built in {time.time() - t:.1f} s")
    lens = T0.copy()
    for step in range(w.extra_tokens):
        before = lens.copy()
        ks = [streams[s][0][lens[s]:lens[s] + 1] for s in range(S)]
        vs = [streams[s][1][lens[s]:lens[s] + 1] for s in range(S)]
        q = w.q_decode(step)
        # the call the benchmark times: append and attention in one launch
        got = gc.decode_step(np.concatenate(ks), np.concatenate(vs), q, SCALE)
        for s in range(S):
            orcs[s].append(ks[s], vs[s])
        lens += 1
        pages = []
        for s in range(S):
            tv0 = max(0, int(before[s]) - R)
            if lens[s] - R > tv0:
                pages.append(gc.bt_np[s, tv0 // w.block_size])
            tk0, tk1 = R * (int(before[s]) // R), R * (int(lens[s]) // R)
            pages.extend(gc.bt_np[s, tk0 // w.block_size: tk1 // w.block_size].tolist())
        mirror.refresh(pages)
        check_decode_step_state(mirror, gc.bt_np, orcs, before, lens, label=f"ragged stream step {step}")
        sample = [(16 * step + i) % S for i in range(16)]
        ref = oracle.attention_all([orcs[s] for s in sample], w.num_q_heads, q[sample], w.dtype,
                                   np.arange(len(sample) + 1), SCALE, False, threads=THREADS)
        check_attention(got[sample], ref, w.dtype, label=f"ragged stream step {step} decode")
        if step % 16 == 15:
            _log(f"ragged stream: step {step + 1} checked at {time.time() - t:.1f} s")
    _full_state(gc, orcs, lens, "ragged stream after 64 steps")
    _log(f"ragged stream: done in {time.time() - t:.1f} s")
