"""Python binding of the ``libkivi.so`` C ABI (argument marshalling only).

Every function has the name and argument order of its C counterpart in
``include/kivi.h``. Device pointers may be given as integers or as objects
with ``data_ptr()`` (e.g. torch tensors); ``stream`` as an integer handle,
``None`` (the null stream) or an object with ``cuda_stream``. A non-OK status
raises :class:`KiviError` carrying the library's message. There is no
fallback: if the HIP library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# KIVI_LIB may name another build of the same library (e.g. an instrumented one)
LIB_PATH = os.environ.get("KIVI_LIB") or os.path.join(_HERE, "libkivi.so")

KIVI_OK = 0
KIVI_ERR_INVALID_ARG = 1
KIVI_ERR_UNSUPPORTED = 2
KIVI_ERR_POOL_TOO_SMALL = 3
KIVI_ERR_WORKSPACE = 4
KIVI_ERR_DEVICE = 5
KIVI_ERR_DEVICE_ASSERT = 6

KIVI_DEVERR_PAGE = 1
KIVI_DEVERR_SLOT = 2
KIVI_DEVERR_LENGTH = 4
KIVI_DEVERR_QUERY = 8

KIVI_F16 = 0
KIVI_BF16 = 1

EXPORTED = [
    "kivi_cache_pool_bytes", "kivi_cache_capacity", "kivi_cache_create", "kivi_cache_destroy", "kivi_cache_layout",
    "kivi_append_tokens", "kivi_decode_workspace_bytes", "kivi_decode_attention", "kivi_decode_attention_noalloc",
    "kivi_decode_step",
    "kivi_prefill_workspace_bytes", "kivi_prefill_attention", "kivi_prefill_attention_raw_chunk",
    "kivi_fp8_append_tokens", "kivi_fp8_decode_attention", "kivi_fp8_decode_step", "kivi_fp8_prefill_attention",
    "kivi_check_device_errors", "kivi_last_error",
    "kivi_status_string",
]


class KiviError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class kivi_cache_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_kv_heads", "head_dim", "bits", "k_group", "v_group", "residual", "block_size",
        "num_blocks", "max_seqs", "kv_dtype", "v_flush", "scale_per_head")]


class kivi_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "k_codes", "v_codes", "k_meta", "v_meta", "k_ring", "v_ring", "total_bytes",
        "code_bytes", "k_meta_bytes", "v_meta_bytes", "ring_bytes", "status")]


_lock = threading.Lock()
_lib = None


def load():
    """Load libkivi.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python kivi_quantized_kv_append_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        P, I32, S = c.c_void_p, c.c_int32, c.c_size_t
        CFG = c.POINTER(kivi_cache_config)
        L.kivi_cache_pool_bytes.argtypes = [CFG, c.POINTER(S)]
        L.kivi_cache_capacity.argtypes = [CFG, S, c.POINTER(c.c_int32), c.POINTER(c.c_int64)]
        L.kivi_cache_create.argtypes = [CFG, P, S, c.POINTER(P)]
        L.kivi_cache_destroy.argtypes = [P]
        L.kivi_cache_destroy.restype = None
        L.kivi_cache_layout.argtypes = [P, c.POINTER(kivi_layout)]
        L.kivi_append_tokens.argtypes = [P, I32, P, P, P, I32, P, P, P, I32, P]
        L.kivi_decode_workspace_bytes.argtypes = [P, I32, I32, I32, c.POINTER(S)]
        L.kivi_decode_attention.argtypes = [P, I32, I32, P, P, P, I32, P, I32, c.c_float, P, P, S, P]
        L.kivi_decode_attention_noalloc.argtypes = [P, I32, I32, P, P, P, I32, P, I32, c.c_float, P, P]
        L.kivi_decode_step.argtypes = [P, I32, I32, P, P, P, P, P, I32, P, I32, c.c_float, P, P, S, P]
        L.kivi_prefill_workspace_bytes.argtypes = [P, I32, I32, I32, I32, c.POINTER(S)]
        L.kivi_prefill_attention.argtypes = [P, I32, I32, P, P, I32, P, P, I32, P, I32, c.c_float,
                                             I32, P, P, S, P]
        L.kivi_prefill_attention_raw_chunk.argtypes = [P, I32, I32, P, P, I32, P, P, P, P, I32, P, I32,
                                                       c.c_float, I32, P, P, S, P]
        L.kivi_fp8_append_tokens.argtypes = [P, I32, P, P, I32, P, P, P, P, P, I32, P]
        L.kivi_fp8_decode_attention.argtypes = [P, I32, I32, P, P, I32, P, P, P, I32, c.c_float, P, P, S, P]
        L.kivi_fp8_decode_step.argtypes = [P, I32, I32, P, P, P, P, I32, P, P, P, I32, c.c_float, P, P, S, P]
        L.kivi_fp8_prefill_attention.argtypes = [P, I32, I32, P, P, I32, P, I32, P, P, P, I32, c.c_float, I32, P, P]
        L.kivi_check_device_errors.argtypes = [P, P, c.POINTER(c.c_uint32)]
        L.kivi_last_error.argtypes = []
        L.kivi_last_error.restype = c.c_char_p
        L.kivi_status_string.argtypes = [c.c_int]
        L.kivi_status_string.restype = c.c_char_p
        for name in EXPORTED:
            if name not in ("kivi_cache_destroy", "kivi_last_error", "kivi_status_string"):
                getattr(L, name).restype = c.c_int
        _lib = L
        return L


def _status_name(status: int) -> str:
    try:
        return load().kivi_status_string(status).decode()
    except Exception:
        return str(status)


def _check(status: int):
    if status != KIVI_OK:
        raise KiviError(status, load().kivi_last_error().decode())


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def make_config(num_kv_heads, bits, k_group, v_group, residual, block_size, num_blocks, max_seqs,
                kv_dtype=KIVI_F16, head_dim=128, v_flush=0, scale_per_head=0) -> kivi_cache_config:
    return kivi_cache_config(num_kv_heads, head_dim, bits, k_group, v_group, residual, block_size,
                             num_blocks, max_seqs, kv_dtype, v_flush, scale_per_head)


def make_fp8_config(num_kv_heads, block_size, num_blocks, max_seqs=1, kv_dtype=KIVI_F16,
                    scale_per_head=0) -> kivi_cache_config:
    """Configuration of an FP8 (E4M3) cache: bits 8, no groups, no residual."""
    return make_config(num_kv_heads, 8, 0, 0, 0, block_size, num_blocks, max_seqs, kv_dtype,
                       scale_per_head=scale_per_head)


def kivi_cache_pool_bytes(cfg: kivi_cache_config) -> int:
    out = ctypes.c_size_t()
    _check(load().kivi_cache_pool_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def kivi_cache_capacity(cfg: kivi_cache_config, budget_bytes: int):
    """(num_blocks, kv_tokens) that fit in budget_bytes (cfg.num_blocks is ignored)."""
    nb, tok = ctypes.c_int32(), ctypes.c_int64()
    _check(load().kivi_cache_capacity(ctypes.byref(cfg), int(budget_bytes), ctypes.byref(nb), ctypes.byref(tok)))
    return nb.value, tok.value


def kivi_cache_create(cfg: kivi_cache_config, d_pool, pool_bytes: int) -> int:
    out = ctypes.c_void_p()
    _check(load().kivi_cache_create(ctypes.byref(cfg), _ptr(d_pool), pool_bytes, ctypes.byref(out)))
    return out.value


def kivi_cache_destroy(cache: int | None):
    load().kivi_cache_destroy(cache)


def kivi_cache_layout(cache: int) -> dict:
    lay = kivi_layout()
    _check(load().kivi_cache_layout(cache, ctypes.byref(lay)))
    return {n: int(getattr(lay, n)) for n, _ in kivi_layout._fields_}


def kivi_append_tokens(cache, num_seqs, d_slot_ids, d_seq_lens_before, d_cu_new, max_new, d_k_new,
                       d_v_new, d_block_table, bt_stride, stream=None):
    _check(load().kivi_append_tokens(cache, num_seqs, _ptr(d_slot_ids), _ptr(d_seq_lens_before),
                                     _ptr(d_cu_new), max_new, _ptr(d_k_new), _ptr(d_v_new),
                                     _ptr(d_block_table), bt_stride, _stream(stream)))


def kivi_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_seq_len) -> int:
    out = ctypes.c_size_t()
    _check(load().kivi_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_seq_len,
                                              ctypes.byref(out)))
    return out.value


def kivi_decode_attention(cache, num_seqs, num_q_heads, d_q, d_slot_ids, d_seq_lens, max_seq_len,
                          d_block_table, bt_stride, softmax_scale, d_out, d_ws, ws_bytes, stream=None):
    _check(load().kivi_decode_attention(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_slot_ids),
                                        _ptr(d_seq_lens), max_seq_len, _ptr(d_block_table), bt_stride,
                                        float(softmax_scale), _ptr(d_out), _ptr(d_ws), ws_bytes,
                                        _stream(stream)))


def kivi_decode_attention_noalloc(cache, num_seqs, num_q_heads, d_q, d_slot_ids, d_seq_lens, max_seq_len,
                                  d_block_table, bt_stride, softmax_scale, d_out, stream=None):
    _check(load().kivi_decode_attention_noalloc(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_slot_ids),
                                                _ptr(d_seq_lens), max_seq_len, _ptr(d_block_table), bt_stride,
                                                float(softmax_scale), _ptr(d_out), _stream(stream)))


def kivi_decode_step(cache, num_seqs, num_q_heads, d_q, d_slot_ids, d_seq_lens_before, d_k_new, d_v_new,
                     max_seq_len, d_block_table, bt_stride, softmax_scale, d_out, d_ws=None, ws_bytes=0,
                     stream=None):
    _check(load().kivi_decode_step(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_slot_ids),
                                   _ptr(d_seq_lens_before), _ptr(d_k_new), _ptr(d_v_new), max_seq_len,
                                   _ptr(d_block_table), bt_stride, float(softmax_scale), _ptr(d_out), _ptr(d_ws),
                                   ws_bytes, _stream(stream)))


def kivi_prefill_workspace_bytes(cache, num_seqs, num_q_heads, max_q_len, max_seq_len) -> int:
    out = ctypes.c_size_t()
    _check(load().kivi_prefill_workspace_bytes(cache, num_seqs, num_q_heads, max_q_len, max_seq_len,
                                               ctypes.byref(out)))
    return out.value


def kivi_prefill_attention(cache, num_seqs, num_q_heads, d_q, d_cu_q, max_q_len, d_slot_ids,
                           d_seq_lens, max_seq_len, d_block_table, bt_stride, softmax_scale, causal,
                           d_out, d_ws=None, ws_bytes=0, stream=None):
    _check(load().kivi_prefill_attention(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_cu_q),
                                         max_q_len, _ptr(d_slot_ids), _ptr(d_seq_lens), max_seq_len,
                                         _ptr(d_block_table), bt_stride, float(softmax_scale),
                                         int(causal), _ptr(d_out), _ptr(d_ws), ws_bytes,
                                         _stream(stream)))


def kivi_prefill_attention_raw_chunk(cache, num_seqs, num_q_heads, d_q, d_cu_q, max_q_len, d_slot_ids,
                                     d_seq_lens_before, d_k_new, d_v_new, max_seq_len, d_block_table, bt_stride,
                                     softmax_scale, causal, d_out, d_ws=None, ws_bytes=0, stream=None):
    _check(load().kivi_prefill_attention_raw_chunk(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_cu_q),
                                                   max_q_len, _ptr(d_slot_ids), _ptr(d_seq_lens_before),
                                                   _ptr(d_k_new), _ptr(d_v_new), max_seq_len,
                                                   _ptr(d_block_table), bt_stride, float(softmax_scale),
                                                   int(causal), _ptr(d_out), _ptr(d_ws), ws_bytes,
                                                   _stream(stream)))


def kivi_fp8_append_tokens(cache, num_seqs, d_seq_lens_before, d_cu_new, max_new, d_k_new, d_v_new,
                           d_k_scale, d_v_scale, d_block_table, bt_stride, stream=None):
    _check(load().kivi_fp8_append_tokens(cache, num_seqs, _ptr(d_seq_lens_before), _ptr(d_cu_new), max_new,
                                         _ptr(d_k_new), _ptr(d_v_new), _ptr(d_k_scale), _ptr(d_v_scale),
                                         _ptr(d_block_table), bt_stride, _stream(stream)))


def kivi_fp8_decode_attention(cache, num_seqs, num_q_heads, d_q, d_seq_lens, max_seq_len, d_k_scale, d_v_scale,
                              d_block_table, bt_stride, softmax_scale, d_out, d_ws=None, ws_bytes=0,
                              stream=None):
    _check(load().kivi_fp8_decode_attention(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_seq_lens),
                                            max_seq_len, _ptr(d_k_scale), _ptr(d_v_scale), _ptr(d_block_table),
                                            bt_stride, float(softmax_scale), _ptr(d_out), _ptr(d_ws), ws_bytes,
                                            _stream(stream)))


def kivi_fp8_decode_step(cache, num_seqs, num_q_heads, d_q, d_seq_lens_before, d_k_new, d_v_new, max_seq_len,
                         d_k_scale, d_v_scale, d_block_table, bt_stride, softmax_scale, d_out, d_ws=None, ws_bytes=0,
                         stream=None):
    _check(load().kivi_fp8_decode_step(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_seq_lens_before),
                                       _ptr(d_k_new), _ptr(d_v_new), max_seq_len, _ptr(d_k_scale), _ptr(d_v_scale),
                                       _ptr(d_block_table), bt_stride, float(softmax_scale), _ptr(d_out), _ptr(d_ws),
                                       ws_bytes, _stream(stream)))


def kivi_fp8_prefill_attention(cache, num_seqs, num_q_heads, d_q, d_cu_q, max_q_len, d_seq_lens, max_seq_len,
                               d_k_scale, d_v_scale, d_block_table, bt_stride, softmax_scale, causal, d_out,
                               stream=None):
    _check(load().kivi_fp8_prefill_attention(cache, num_seqs, num_q_heads, _ptr(d_q), _ptr(d_cu_q), max_q_len,
                                             _ptr(d_seq_lens), max_seq_len, _ptr(d_k_scale), _ptr(d_v_scale),
                                             _ptr(d_block_table), bt_stride, float(softmax_scale), int(causal),
                                             _ptr(d_out), _stream(stream)))


def kivi_check_device_errors(cache, stream=None) -> int:
    """The status word's kivi_device_error bits (0 when none was set; the word is
    cleared). Raises KiviError (KIVI_ERR_DEVICE_ASSERT) when a bit was set; the
    exception carries the bits as ``flags``."""
    flags = ctypes.c_uint32()
    st = load().kivi_check_device_errors(cache, _stream(stream), ctypes.byref(flags))
    if st != KIVI_OK:
        e = KiviError(st, load().kivi_last_error().decode())
        e.flags = flags.value
        raise e
    return flags.value


def kivi_last_error() -> str:
    return load().kivi_last_error().decode()


def kivi_status_string(status: int) -> str:
    return load().kivi_status_string(status).decode()
