"""kivi_decode_attention_noalloc (split partials in a static device array, no
workspace argument) against kivi_decode_attention with a caller workspace,
through the C ABI: bit-identical outputs on two calls in a row, the second with
a smaller batch (a different split plan over the same array), and both within
the attention tolerance of the oracle."""
import numpy as np
import pytest

from kivi_quantized_kv_append_amd import inputs, kivi
from harness import SCALE, GpuCache, check_attention, oracle_caches
import oracle

pytestmark = pytest.mark.gpu


def _noalloc(gc, q_bits, seqs):
    torch, w = gc.torch, gc.w
    HQ = w.num_q_heads
    out = torch.full((len(seqs), HQ, 128), -1, dtype=torch.int16, device=gc.device)
    bt = gc.t(gc.bt_np[seqs])
    kivi.kivi_decode_attention_noalloc(gc.handle, len(seqs), HQ, gc.t(np.ascontiguousarray(q_bits).view(np.int16)),
                                       gc.t(np.asarray(seqs, np.int32)), gc.t(gc.lens[seqs].astype(np.int32)),
                                       int(gc.lens[seqs].max()), bt, bt.shape[1], SCALE, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def test_noalloc_matches_workspace_call_twice():
    # few long sequences: every sequence is split, so the partials go through the static array
    w = inputs.config(3, num_seqs=3, seq_lens=[20000, 9000, 4100], extra_tokens=0, shuffle=True, pool_factor=1.25)
    gc = GpuCache(w)
    rk, rv = zip(*w.kv_streams(8))
    gc.append(list(rk), list(rv))
    orcs = oracle_caches(w)
    assert kivi.kivi_decode_workspace_bytes(gc.handle, 3, w.num_q_heads, 20000) > 0
    for call, seqs in enumerate(([0, 1, 2], [2])):  # the second call is smaller
        q = w.q_decode(call)[seqs]
        want = gc.decode(q, SCALE, seqs=seqs)
        got = _noalloc(gc, q, seqs)
        assert np.array_equal(got, want), f"call {call}: {int((got != want).sum())} elements differ"
        ref = oracle.attention_all([orcs[s] for s in seqs], w.num_q_heads, q, w.dtype, np.arange(len(seqs) + 1),
                                   SCALE, False, threads=8)
        check_attention(got, ref, w.dtype, label=f"no-alloc decode, call {call}")
