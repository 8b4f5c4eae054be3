"""KIVI oracle (test infrastructure only).

A ctypes wrapper around ``kivi_oracle.cpp``: a plain, slow, scalar CPU
implementation of KIVI-style KV-cache quantisation and of attention over the
quantised cache. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product library
never does, and this package imports nothing from it.

Sources (the pages): "4.4 KV Cache 量化" sections 1, 2, 3.1 and 3.2, and
"给 KV cache 减肥" section 3.1. The C++ file names the passage each function
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kivi_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DT_F16 = 0
DT_BF16 = 1

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (scalar, IEEE single rounding, no FMA)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", _SRC, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            c = ctypes
            P = c.c_void_p
            L.orc_f16_from_f32.argtypes = [c.c_float]
            L.orc_f16_from_f32.restype = c.c_uint16
            L.orc_f32_from_f16.argtypes = [c.c_uint16]
            L.orc_f32_from_f16.restype = c.c_float
            L.orc_f32_from_bf16.argtypes = [c.c_uint16]
            L.orc_f32_from_bf16.restype = c.c_float
            L.orc_f16_from_f32_array.argtypes = [P, P, c.c_long]
            L.orc_f32_from_f16_array.argtypes = [P, P, c.c_long]
            L.orc_m_kv_bytes.argtypes = [c.c_double] * 6
            L.orc_m_kv_bytes.restype = c.c_double
            L.orc_quantize_group.argtypes = [P, c.c_long, c.c_int, P, P, P]
            L.orc_dequant.argtypes = [c.c_int, c.c_uint16, c.c_uint16]
            L.orc_dequant.restype = c.c_float
            L.orc_dequant_array.argtypes = [P, P, P, P, c.c_long]
            L.orc_cache_new.argtypes = [c.c_int] * 9
            L.orc_cache_new.restype = P
            L.orc_cache_free.argtypes = [P]
            L.orc_cache_append.argtypes = [P, c.c_int, P, P]
            L.orc_cache_append.restype = c.c_int
            L.orc_cache_state.argtypes = [P, P, P, P]
            L.orc_cache_arrays.argtypes = [P] + [c.POINTER(P)] * 8
            L.orc_cache_reconstruct.argtypes = [P, c.c_int, P, P]
            L.orc_attention.argtypes = [P, c.c_int, c.c_int, P, c.c_int, P, c.c_double, c.c_int,
                                        P, P, c.c_long, P, c.c_int]
            L.orc_attention.restype = c.c_int
            L.orc_attention_raw_chunk.argtypes = [P, c.c_int, c.c_int, P, c.c_int, P, P, P, c.c_double,
                                                  c.c_int, P, P, c.c_long, P, c.c_int]
            L.orc_attention_raw_chunk.restype = c.c_int
            L.orc_hardware_threads.restype = c.c_int
            L.orc_e4m3_to_f32.argtypes = [c.c_int]
            L.orc_e4m3_to_f32.restype = c.c_float
            L.orc_f32_to_e4m3.argtypes = [c.c_float]
            L.orc_f32_to_e4m3.restype = c.c_int
            L.orc_fp8_cache_new.argtypes = [c.c_int, c.c_int, c.c_int, c.c_int, P, P, c.c_int]
            L.orc_fp8_cache_new.restype = P
            L.orc_fp8_cache_free.argtypes = [P]
            L.orc_fp8_cache_append.argtypes = [P, c.c_int, P, P]
            L.orc_fp8_cache_append.restype = c.c_int
            L.orc_fp8_cache_len.argtypes = [P]
            L.orc_fp8_cache_len.restype = c.c_int
            L.orc_fp8_cache_arrays.argtypes = [P, c.POINTER(P), c.POINTER(P)]
            L.orc_fp8_attention.argtypes = [P, c.c_int, c.c_int, P, c.c_int, c.c_double, P, c.c_int]
            L.orc_fp8_attention.restype = c.c_int
            L.orc_fp8_attention_rows.argtypes = [P, c.c_int, c.c_int, P, c.c_int, P, c.c_double, c.c_int, P, c.c_int]
            L.orc_fp8_attention_rows.restype = c.c_int
            _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# --- number formats ---------------------------------------------------------

def f16_bits_from_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f16_from_f32_array(_ptr(x), _ptr(out), x.size)
    return out


def f32_from_f16_bits(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_f32_from_f16_array(_ptr(h), _ptr(out), h.size)
    return out


def f32_from_bf16_bits(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def hardware_threads() -> int:
    return int(lib().orc_hardware_threads())


# --- memory formula ------------------------------------------------------------

def m_kv_bytes(L, B, T, H_KV, d, bits) -> float:
    """M_KV = 2 L B T H_KV d b ("4.4 KV Cache 量化", section 1); b in bits."""
    return float(lib().orc_m_kv_bytes(L, B, T, H_KV, d, bits))


# --- one group -----------------------------------------------------------------

def quantize_group(x, bits: int):
    """Min/max asymmetric quantisation of one group -> (codes u8, s16 bits, z16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    codes = np.empty(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint16)
    z = np.zeros(1, dtype=np.uint16)
    lib().orc_quantize_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0])


def dequant(codes, s16, z16) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(np.broadcast_to(np.asarray(s16, dtype=np.uint16), codes.shape))
    z = np.ascontiguousarray(np.broadcast_to(np.asarray(z16, dtype=np.uint16), codes.shape))
    out = np.empty(codes.shape, dtype=np.float32)
    lib().orc_dequant_array(_ptr(codes), _ptr(s), _ptr(z), _ptr(out), codes.size)
    return out


# --- sequence cache ------------------------------------------------------------

class SeqCache:
    """One request's cache (one layer, all KV heads), grown by sequential appends.

    Arrays exposed by :meth:`arrays` (numpy views into the oracle's memory):
      k_code, v_code: [H][Tmax][d] uint8, one code per element
      k_s, k_z: [H][Tmax//G + 1][d] fp16 bits (group j covers tokens jG..jG+G-1)
      v_s, v_z: [H][Tmax][d//Gv] fp16 bits
      k_raw, v_raw: [H][Tmax][d] input bits (the residual is read from here)

    v_flush=0 keeps the sliding Value window of the newest R tokens; v_flush=1 quantises
    the Value tokens of the residual together with the Keys at every Key flush.
    """

    def __init__(self, H, d, bits, G, Gv, R, dtype, Tmax, v_flush=0):
        self.H, self.d, self.bits, self.G, self.Gv, self.R, self.dtype, self.Tmax = \
            H, d, bits, G, Gv, R, dtype, Tmax
        self.v_flush = v_flush
        self._h = lib().orc_cache_new(H, d, bits, G, Gv, R, dtype, Tmax, v_flush)
        if not self._h:
            raise ValueError("oracle: unsupported cache parameters")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_cache_free(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray):
        """k_bits, v_bits: [n][H][d] uint16 raw input bits."""
        k = np.ascontiguousarray(k_bits, dtype=np.uint16)
        v = np.ascontiguousarray(v_bits, dtype=np.uint16)
        assert k.shape == v.shape and k.shape[1:] == (self.H, self.d)
        if lib().orc_cache_append(self._h, k.shape[0], _ptr(k), _ptr(v)) != 0:
            raise ValueError("oracle: append beyond Tmax")

    def state(self):
        T, TK, TV = (ctypes.c_int(), ctypes.c_int(), ctypes.c_int())
        lib().orc_cache_state(self._h, ctypes.byref(T), ctypes.byref(TK), ctypes.byref(TV))
        return T.value, TK.value, TV.value

    def arrays(self) -> dict:
        ptrs = [ctypes.c_void_p() for _ in range(8)]
        lib().orc_cache_arrays(self._h, *[ctypes.byref(p) for p in ptrs])
        H, Tm, d, G, Gv = self.H, self.Tmax, self.d, self.G, self.Gv

        def view(p, shape, dt):
            n = int(np.prod(shape))
            if n == 0:
                return np.zeros(shape, dtype=dt)
            buf = (ctypes.c_char * (n * np.dtype(dt).itemsize)).from_address(p.value)
            return np.frombuffer(buf, dtype=dt).reshape(shape)

        return {
            "k_code": view(ptrs[0], (H, Tm, d), np.uint8),
            "v_code": view(ptrs[1], (H, Tm, d), np.uint8),
            "k_s": view(ptrs[2], (H, Tm // G + 1, d), np.uint16),
            "k_z": view(ptrs[3], (H, Tm // G + 1, d), np.uint16),
            "v_s": view(ptrs[4], (H, Tm, d // Gv), np.uint16),
            "v_z": view(ptrs[5], (H, Tm, d // Gv), np.uint16),
            "k_raw": view(ptrs[6], (H, Tm, d), np.uint16),
            "v_raw": view(ptrs[7], (H, Tm, d), np.uint16),
        }

    def reconstruct(self, h: int):
        """(K~, V~) of head h over tokens [0, T): [T][d] fp32 each."""
        T, _, _ = self.state()
        k = np.empty((T, self.d), dtype=np.float32)
        v = np.empty((T, self.d), dtype=np.float32)
        lib().orc_cache_reconstruct(self._h, h, _ptr(k), _ptr(v))
        return k, v


def attention(caches, H_Q: int, q_bits: np.ndarray, q_dtype: int, cu_q, sigma: float,
              causal: bool, rows, heads, threads: int = 1) -> np.ndarray:
    """Attention outputs for the (row, head) items, [n_items][d] float64.

    q_bits: [total_q][H_Q][d] raw bits. cu_q: [S+1] row offsets per request;
    row i of request s sits at position T_s - n_q,s + i (with causal) or sees
    all T_s tokens (without).
    """
    S = len(caches)
    arr = (ctypes.c_void_p * S)(*[c.handle for c in caches])
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_q, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    assert rows.shape == heads.shape and cu.shape == (S + 1,)
    d = caches[0].d
    out = np.zeros((rows.size, d), dtype=np.float64)
    rc = lib().orc_attention(ctypes.cast(arr, ctypes.c_void_p), S, H_Q, _ptr(q), q_dtype, _ptr(cu),
                             float(sigma), 1 if causal else 0, _ptr(rows), _ptr(heads), rows.size,
                             _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad attention arguments")
    return out


def attention_all(caches, H_Q, q_bits, q_dtype, cu_q, sigma, causal, threads=1) -> np.ndarray:
    """Every (row, head) output: [total_q][H_Q][d] float64."""
    total = int(cu_q[-1])
    rows = np.repeat(np.arange(total, dtype=np.int32), H_Q)
    heads = np.tile(np.arange(H_Q, dtype=np.int32), total)
    out = attention(caches, H_Q, q_bits, q_dtype, cu_q, sigma, causal, rows, heads, threads)
    return out.reshape(total, H_Q, caches[0].d)


def attention_raw_chunk(caches, H_Q: int, q_bits: np.ndarray, q_dtype: int, cu_q, k_bits: np.ndarray,
                        v_bits: np.ndarray, sigma: float, causal: bool, rows=None, heads=None,
                        threads: int = 1) -> np.ndarray:
    """Prefill outputs when each chunk's own Keys and Values take part at full
    precision: caches hold each request's tokens BEFORE its chunk (P_s), the
    chunk's rows k_bits / v_bits ([total_q][H][d] raw bits, indexed like q)
    follow them, and row i of request s sits at position P_s + i.
    rows / heads select items ([n][d] float64); None means every (row, head),
    returned as [total_q][H_Q][d]."""
    S = len(caches)
    total = int(cu_q[-1])
    full = rows is None
    if full:
        rows = np.repeat(np.arange(total, dtype=np.int32), H_Q)
        heads = np.tile(np.arange(H_Q, dtype=np.int32), total)
    arr = (ctypes.c_void_p * S)(*[c.handle for c in caches])
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_q, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    H, d = caches[0].H, caches[0].d
    assert rows.shape == heads.shape and cu.shape == (S + 1,)
    assert k.shape == (total, H, d) and v.shape == (total, H, d)
    out = np.zeros((rows.size, d), dtype=np.float64)
    rc = lib().orc_attention_raw_chunk(ctypes.cast(arr, ctypes.c_void_p), S, H_Q, _ptr(q), q_dtype, _ptr(cu),
                                       _ptr(k), _ptr(v), float(sigma), 1 if causal else 0, _ptr(rows),
                                       _ptr(heads), rows.size, _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad attention arguments")
    return out.reshape(total, H_Q, d) if full else out


# --- FP8 (E4M3) cache ("4.4 KV Cache 量化", section 4) -----------------------

def e4m3_to_f32(codes) -> np.ndarray:
    """float32 value of each E4M3 code (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64).ravel()
    return np.array([lib().orc_e4m3_to_f32(int(x)) for x in c], dtype=np.float32).reshape(np.shape(codes))


def f32_to_e4m3(y) -> np.ndarray:
    """E4M3 code of each float32 value: saturated to +-448, nearest value, ties to the even code."""
    a = np.asarray(y, dtype=np.float32).ravel()
    return np.array([lib().orc_f32_to_e4m3(float(x)) for x in a], dtype=np.uint8).reshape(np.shape(y))


class Fp8SeqCache:
    """One request's FP8 cache (one layer, all KV heads): every appended element is stored
    as E4M3(x / scale) and restored as value * scale. k_scales / v_scales hold one value
    (per_head=False) or one per KV head."""

    def __init__(self, H, d, dtype, Tmax, k_scales, v_scales, per_head: bool):
        self.H, self.d, self.dtype, self.Tmax = H, d, dtype, Tmax
        self._ks = np.ascontiguousarray(k_scales, dtype=np.float32).ravel()
        self._vs = np.ascontiguousarray(v_scales, dtype=np.float32).ravel()
        n = H if per_head else 1
        assert self._ks.size >= n and self._vs.size >= n
        self._h = lib().orc_fp8_cache_new(H, d, dtype, Tmax, _ptr(self._ks), _ptr(self._vs), 1 if per_head else 0)
        if not self._h:
            raise ValueError("oracle: unsupported FP8 cache parameters")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_fp8_cache_free(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def __len__(self):
        return lib().orc_fp8_cache_len(self._h)

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray):
        """k_bits, v_bits: [n][H][d] uint16 raw input bits."""
        k = np.ascontiguousarray(k_bits, dtype=np.uint16)
        v = np.ascontiguousarray(v_bits, dtype=np.uint16)
        assert k.shape == v.shape and k.shape[1:] == (self.H, self.d)
        if lib().orc_fp8_cache_append(self._h, k.shape[0], _ptr(k), _ptr(v)) != 0:
            raise ValueError("oracle: append beyond Tmax")

    def arrays(self) -> dict:
        """k_code, v_code: [H][Tmax][d] uint8 views (valid while the cache lives)."""
        kp, vp = ctypes.c_void_p(), ctypes.c_void_p()
        lib().orc_fp8_cache_arrays(self._h, ctypes.byref(kp), ctypes.byref(vp))
        n = self.H * self.Tmax * self.d
        shape = (self.H, self.Tmax, self.d)
        out = {}
        for name, p in (("k_code", kp), ("v_code", vp)):
            buf = (ctypes.c_uint8 * n).from_address(p.value) if n else None
            out[name] = (np.frombuffer(buf, dtype=np.uint8) if n else np.zeros(0, np.uint8)).reshape(shape)
        return out


def fp8_attention(caches, H_Q: int, q_bits: np.ndarray, q_dtype: int, sigma: float, threads: int = 1):
    """Decode attention over FP8 caches, one query row per request at its last position:
    q_bits [S][H_Q][d] raw bits -> [S][H_Q][d] float64."""
    S = len(caches)
    arr = (ctypes.c_void_p * S)(*[c.handle for c in caches])
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    d = caches[0].d
    assert q.shape == (S, H_Q, d)
    out = np.zeros((S, H_Q, d), dtype=np.float64)
    rc = lib().orc_fp8_attention(ctypes.cast(arr, ctypes.c_void_p), S, H_Q, _ptr(q), q_dtype, float(sigma),
                                 _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad FP8 attention arguments")
    return out


def fp8_attention_rows(caches, H_Q: int, q_bits: np.ndarray, q_dtype: int, cu_q, sigma: float, causal: bool,
                       threads: int = 1):
    """Prefill over FP8 caches: q_bits [total_q][H_Q][d]; row i of request s sits at position
    T_s - n_q,s + i and sees positions up to itself (causal) or all T_s tokens; a row that sees
    no token is zero. Returns [total_q][H_Q][d] float64."""
    S = len(caches)
    arr = (ctypes.c_void_p * S)(*[c.handle for c in caches])
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_q, dtype=np.int32)
    d = caches[0].d
    out = np.zeros((int(cu[-1]), H_Q, d), dtype=np.float64)
    rc = lib().orc_fp8_attention_rows(ctypes.cast(arr, ctypes.c_void_p), S, H_Q, _ptr(q), q_dtype, _ptr(cu),
                                      float(sigma), 1 if causal else 0, _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("oracle: bad FP8 attention arguments")
    return out
