"""Host-only checks of the C ABI library: it loads, exports every symbol the
header declares, sizes pools by the documented layout, and fails fast on
unsupported configurations and bad arguments (no device work)."""
import os
import re

import pytest

import oracle
from kivi_quantized_kv_append_amd import kivi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "kivi.h")).read()
    return sorted(set(re.findall(r"\b(kivi_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = kivi.load()
    declared = _declared_symbols()
    assert set(declared) == set(kivi.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def cfg(**kw):
    base = dict(num_kv_heads=8, bits=4, k_group=64, v_group=128, residual=128, block_size=16,
                num_blocks=8192, max_seqs=32, kv_dtype=kivi.KIVI_F16)
    base.update(kw)
    return kivi.make_config(**base)


def test_pool_bytes_matches_layout_formula():
    c = cfg()
    n = kivi.kivi_cache_pool_bytes(c)
    H, NB, S, Bk, G, R = 8, 8192, 32, 16, 64, 128
    codes = NB * H * Bk * 128 * 4 // 8
    kmeta = NB * H * 4 * 128 * Bk // G
    vmeta = NB * H * Bk * 1 * 4
    ring = S * H * R * 128 * 2
    status = 256  # the status word's sub-array (device-side error bits)
    assert n == 2 * codes + kmeta + vmeta + 2 * ring + status


@pytest.mark.parametrize("bits,budget", [(4, 1 << 30), (2, 1 << 30), (4, 70 << 30), (4, 3 << 20), (4, 1000)])
def test_capacity_is_the_largest_pool_that_fits(bits, budget):
    c = cfg(bits=bits)
    nb, tokens = kivi.kivi_cache_capacity(c, budget)
    assert tokens == nb * 16
    if nb == 0:
        assert kivi.kivi_cache_pool_bytes(cfg(bits=bits, num_blocks=1)) > budget
        return
    assert kivi.kivi_cache_pool_bytes(cfg(bits=bits, num_blocks=nb)) <= budget
    try:
        assert kivi.kivi_cache_pool_bytes(cfg(bits=bits, num_blocks=nb + 1)) > budget
    except kivi.KiviError as e:  # one more block passes the 4 GiB code sub-array limit
        assert e.status == kivi.KIVI_ERR_UNSUPPORTED and "4 GiB" in str(e)


def test_capacity_density_against_fp16():
    """Tokens per byte against an fp16 cache of the same budget, whose size is the
    M_KV formula at 16 bits ("4.4 KV Cache 量化", section 1). The codes alone give
    4x at int4 (8x at int2); group metadata and the residual rings take some of it
    back. The product pages quote about 3x for their int4 backend."""
    budget = 8 << 30
    fp16_tokens = budget // oracle.m_kv_bytes(1, 1, 1, 8, 128, 16)
    for bits, lo, hi in ((4, 3.0, 4.0), (2, 5.0, 8.0)):
        _, tokens = kivi.kivi_cache_capacity(cfg(bits=bits, max_seqs=256), budget)
        ratio = tokens / fp16_tokens
        assert lo < ratio < hi, (bits, ratio)
    # with Key groups of 64 tokens and 128-channel Value groups: codes 128 B, Key
    # meta 8 B, Value meta 4 B per token and head, against 512 B in fp16
    _, tokens = kivi.kivi_cache_capacity(cfg(bits=4, max_seqs=1), budget)
    assert abs(tokens / fp16_tokens - 512 / 140) < 0.01


@pytest.mark.parametrize("bits", [2, 4])
def test_code_payload_equals_m_kv(bits):
    """The code sub-arrays hold exactly M_KV = 2 L B T H_KV d b bytes for the tokens their
    pages cover ("4.4 KV Cache 量化", section 1), with L = 1 layer and B*T = pages*Bk."""
    c = cfg(bits=bits, num_blocks=2048)
    h = kivi.kivi_cache_create(c, 1 << 20, 1 << 40)
    try:
        lay = kivi.kivi_cache_layout(h)
        payload = lay["v_codes"] - lay["k_codes"] + lay["code_bytes"] * 2048 * 8
        assert payload == oracle.m_kv_bytes(1, 1, 2048 * 16, 8, 128, bits)
        assert lay["code_bytes"] * 2048 * 8 * 2 == oracle.m_kv_bytes(1, 1, 2048 * 16, 8, 128, bits)
    finally:
        kivi.kivi_cache_destroy(h)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(head_dim=256), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(bits=3), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(bits=8), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(residual=96), kivi.KIVI_ERR_UNSUPPORTED),       # R % G != 0
    (dict(k_group=24), kivi.KIVI_ERR_UNSUPPORTED),        # G % Bk != 0
    (dict(k_group=48), kivi.KIVI_ERR_UNSUPPORTED),        # G/Bk = 3 does not divide 128
    (dict(v_group=48), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(block_size=8), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(v_flush=2), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(v_flush=-1), kivi.KIVI_ERR_UNSUPPORTED),
    (dict(num_blocks=0), kivi.KIVI_ERR_INVALID_ARG),
    (dict(max_seqs=0), kivi.KIVI_ERR_INVALID_ARG),
])
def test_fail_fast_configs(over, status):
    hd = over.pop("head_dim", 128)
    c = cfg(**over)
    c.head_dim = hd
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_pool_bytes(c)
    assert e.value.status == status
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_create(c, 1 << 20, 1 << 40)
    assert e.value.status == status


def test_create_checks_pool():
    c = cfg()
    n = kivi.kivi_cache_pool_bytes(c)
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_create(c, 1 << 20, n - 1)
    assert e.value.status == kivi.KIVI_ERR_POOL_TOO_SMALL
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_create(c, 0, n)
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_create(c, (1 << 20) + 16, n)
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    kivi.kivi_cache_destroy(None)


def test_call_argument_checks_launch_nothing():
    c = cfg()
    h = kivi.kivi_cache_create(c, 1 << 20, 1 << 40)
    D = 1 << 20  # fake aligned device address: no call below may reach a launch
    try:
        # zero sequences: a no-op
        kivi.kivi_append_tokens(h, 0, None, None, None, 0, None, None, None, 1)
        kivi.kivi_decode_attention(h, 0, 32, None, None, None, 0, None, 1, 0.1, None, None, 0)
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_append_tokens(h, -1, D, D, D, 1, D, D, D, 1)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_append_tokens(h, 2, D, D, None, 1, D, D, D, 1)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_append_tokens(h, 2, D, D, D, 1, D + 2, D, D, 1)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_append_tokens(h, 2, D, D, D, 1, D, D, D, 0)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        # decode: head ratio, workspace, pointers
        ws = kivi.kivi_decode_workspace_bytes(h, 4, 32, 4096)
        assert ws > 0  # 32 (sequence, KV head) pairs: split, partials in the workspace
        assert kivi.kivi_decode_workspace_bytes(h, 32, 32, 4096) == 0  # one work group per CU already
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_decode_attention(h, 4, 30, D, D, D, 4096, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_decode_attention(h, 4, 8 * 17, D, D, D, 4096, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_decode_attention(h, 4, 32, D, D, D, 4096, D, 1, 0.1, D, D, ws - 1)
        assert e.value.status == kivi.KIVI_ERR_WORKSPACE
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_decode_attention(h, 4, 32, D, D, D, 4096, D, 1, 0.1, D, None, ws)
        assert e.value.status == kivi.KIVI_ERR_WORKSPACE
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_decode_attention(h, 4, 32, None, D, D, 4096, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_decode_attention(h, 4, 32, D, D, D, 4096, D, 1, float("nan"), D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_prefill_attention(h, 2, 32, D, D, 16, D, D, 4096, D, 1, 0.1, 2, D)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        assert "causal" in kivi.kivi_last_error()
        # prefill with the chunk at full precision: the chunk's rows are required and aligned
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_prefill_attention_raw_chunk(h, 2, 32, D, D, 16, D, D, None, D, 4096, D, 1, 0.1, 1, D)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        assert "k_new" in kivi.kivi_last_error()
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_prefill_attention_raw_chunk(h, 2, 32, D, D, 16, D, D, D, D + 8, 4096, D, 1, 0.1, 1, D)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_prefill_attention_raw_chunk(h, 2, 30, D, D, 16, D, D, D, D, 4096, D, 1, 0.1, 1, D)
        assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
        kivi.kivi_prefill_attention_raw_chunk(h, 0, 32, None, None, 0, None, None, None, None, 0, None, 1, 0.1, 1,
                                              None)  # no sequences: a no-op
    finally:
        kivi.kivi_cache_destroy(h)


def test_fp8_config_and_layout():
    """bits 8 is the FP8 (E4M3) cache: no groups, no residual; its code payload is the
    M_KV formula at 8 bits."""
    c = kivi.make_fp8_config(8, 16, 2048, scale_per_head=1)
    n = kivi.kivi_cache_pool_bytes(c)
    assert n == 2 * 2048 * 8 * 16 * 128 + 256  # codes and the status word
    assert n - 256 == oracle.m_kv_bytes(1, 1, 2048 * 16, 8, 128, 8)
    h = kivi.kivi_cache_create(c, 1 << 20, n)
    try:
        lay = kivi.kivi_cache_layout(h)
        assert lay["code_bytes"] == 16 * 128 and lay["total_bytes"] == n
        assert lay["k_meta"] == lay["v_meta"] == lay["k_ring"] == lay["v_ring"] == lay["status"] == n - 256
    finally:
        kivi.kivi_cache_destroy(h)
    # density of a 1 GiB budget against fp16 K/V: exactly 2x
    nb, tokens = kivi.kivi_cache_capacity(kivi.make_fp8_config(8, 16, 1), 1 << 30)
    assert tokens == ((1 << 30) - 256) // (2 * 8 * 128 * 16) * 16


@pytest.mark.parametrize("over", [dict(k_group=64), dict(v_group=128), dict(residual=128), dict(v_flush=1),
                                  dict(scale_per_head=2)])
def test_fp8_fail_fast_configs(over):
    base = dict(num_kv_heads=8, bits=8, k_group=0, v_group=0, residual=0, block_size=16, num_blocks=64,
                max_seqs=1, kv_dtype=kivi.KIVI_F16)
    base.update(over)
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_pool_bytes(kivi.make_config(**base))
    assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED


def test_scale_granularity_is_fp8_only():
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_pool_bytes(cfg(scale_per_head=1))
    assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED


def test_each_cache_kind_takes_only_its_calls():
    D = 1 << 20
    h8 = kivi.kivi_cache_create(kivi.make_fp8_config(8, 16, 64), D, 1 << 40)
    h4 = kivi.kivi_cache_create(cfg(), D, 1 << 40)
    try:
        for call in (lambda: kivi.kivi_append_tokens(h8, 2, D, D, D, 1, D, D, D, 1),
                     lambda: kivi.kivi_decode_attention(h8, 2, 32, D, D, D, 64, D, 1, 0.1, D, D, 1 << 20),
                     lambda: kivi.kivi_decode_step(h8, 2, 32, D, D, D, D, D, 64, D, 1, 0.1, D, D, 1 << 20),
                     lambda: kivi.kivi_prefill_attention(h8, 2, 32, D, D, 16, D, D, 64, D, 1, 0.1, 1, D),
                     lambda: kivi.kivi_fp8_append_tokens(h4, 2, D, D, 1, D, D, D, D, D, 1),
                     lambda: kivi.kivi_fp8_decode_attention(h4, 2, 32, D, D, 64, D, D, D, 1, 0.1, D, D, 1 << 20),
                     lambda: kivi.kivi_fp8_decode_step(h4, 2, 32, D, D, D, D, 64, D, D, D, 1, 0.1, D, D, 1 << 20),
                     lambda: kivi.kivi_fp8_prefill_attention(h4, 2, 32, D, D, 16, D, 64, D, D, D, 1, 0.1, 1, D)):
            with pytest.raises(kivi.KiviError) as e:
                call()
            assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
        # FP8 argument checks before any launch
        kivi.kivi_fp8_append_tokens(h8, 0, None, None, 0, None, None, None, None, None, 1)  # no-op
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_append_tokens(h8, 2, D, D, 1, D, D, None, D, D, 1)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_prefill_attention(h8, 2, 32, D, D, 16, D, 64, D, D, D, 1, 0.1, 2, D)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG and "causal" in kivi.kivi_last_error()
        kivi.kivi_fp8_prefill_attention(h8, 0, 32, None, None, 0, None, 0, None, None, None, 1, 0.1, 1, None)
        ws = kivi.kivi_decode_workspace_bytes(h8, 4, 32, 32768)
        assert ws > 0
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_decode_attention(h8, 4, 32, D, D, 32768, D, D, D, 1, 0.1, D, D, ws - 1)
        assert e.value.status == kivi.KIVI_ERR_WORKSPACE
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_decode_attention(h8, 4, 30, D, D, 32768, D, D, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_decode_attention(h8, 4, 32, D + 8, D, 32768, D, D, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        # the FP8 decode step: same checks, before either launch
        kivi.kivi_fp8_decode_step(h8, 0, 32, None, None, None, None, 0, None, None, None, 1, 0.1, None)  # no-op
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_decode_step(h8, 4, 32, D, D, D, D, 32768, D, D, D, 1, 0.1, D, D, ws - 1)
        assert e.value.status == kivi.KIVI_ERR_WORKSPACE
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_decode_step(h8, 4, 32, D, D, D + 1, D, 32768, D, D, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_decode_step(h8, 4, 32, D, D, D, D, 32768, None, D, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_fp8_decode_step(h8, 4, 30, D, D, D, D, 32768, D, D, D, 1, 0.1, D, D, ws)
        assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
    finally:
        kivi.kivi_cache_destroy(h8)
        kivi.kivi_cache_destroy(h4)


def test_status_strings():
    for s in range(7):
        assert kivi.kivi_status_string(s).startswith("KIVI_")
    assert kivi.kivi_status_string(kivi.KIVI_ERR_DEVICE_ASSERT) == "KIVI_ERR_DEVICE_ASSERT"


def test_status_word_in_layout():
    """The 256-byte status sub-array follows the rings, 256-byte aligned, and ends the pool."""
    c = cfg()
    h = kivi.kivi_cache_create(c, 1 << 20, 1 << 40)
    try:
        lay = kivi.kivi_cache_layout(h)
        assert lay["status"] % 256 == 0 and lay["status"] >= lay["v_ring"] + 32 * 8 * lay["ring_bytes"]
        assert lay["total_bytes"] == lay["status"] + 256 == kivi.kivi_cache_pool_bytes(c)
        with pytest.raises(kivi.KiviError) as e:
            kivi.kivi_check_device_errors(None)
        assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    finally:
        kivi.kivi_cache_destroy(h)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark is one-GPU only: --gpus above 1 exits with a message, before touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_capacity_report_pins_to_m_kv():
    """The capacity report of every workload layout: a sequence's code bytes are the
    M_KV formula at b bits for its pages ("4.4 KV Cache 量化", section 1), its group
    metadata is 4 bytes per (Key group, channel) and per (token, Value group), its
    residual ring is 2 R H 128 bytes per tensor; the residual and metadata share falls
    as the context grows ("4.4 KV Cache 量化", section 3.2) and density approaches
    16 / (b + metadata bits) against fp16."""
    import bench
    from kivi_quantized_kv_append_amd import inputs
    for cfg_id in (1, 2, 3, 4, 5):
        w = inputs.config(cfg_id)
        H, Bk = w.num_kv_heads, w.block_size
        prev = None
        for T in (128, 512, 4096, 32768):
            b = bench.sequence_bytes(kivi, w, T)
            pages = -(-T // Bk)
            assert b["codes"] == oracle.m_kv_bytes(1, 1, pages * Bk, H, 128, w.bits)
            groups = -(-pages * Bk // w.k_group)
            assert b["meta"] == H * (groups * 128 * 4 + pages * Bk * (128 // w.v_group) * 4)
            assert b["residual"] == 2 * H * w.residual * 128 * 2
            share = (b["meta"] + b["residual"]) / b["total"]
            if prev is not None:
                assert share < prev
            prev = share
    rep = bench.capacity_report(kivi, inputs)
    assert set(rep) == {inputs.config(i).name for i in (1, 2, 3, 4, 5)}
    llama = rep[inputs.config(2).name]
    assert 3.0 < llama["density_vs_fp16"] < 4.0
    assert llama["per_sequence"][-1]["density_vs_fp16"] > llama["per_sequence"][0]["density_vs_fp16"]
