"""Seeded synthetic workloads for the KIVI KV-cache path.

This module only draws random inputs and page tables. It holds none of the
method's arithmetic (no quantisation, no attention), so both the HIP path and
the CPU oracle can be fed from it.

Recipe (numpy ``Generator(PCG64)``, one stream per tensor and request, drawn
in float64 and rounded to the cache dtype):
  * K ~ N(0, 1) with a fixed set of outlier channels per KV head multiplied
    before rounding (Keys carry channel outliers, Values do not: "4.4 KV Cache
    量化", section 3.1);
  * V ~ N(0, 1); q ~ N(0, 1) (times ``q_scale`` when a workload says so);
  * pages: in-order or a seeded permutation of a pool of ``pool_factor`` times
    the blocks the final lengths need.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F16 = 0
BF16 = 1


def _bits_f16(x64: np.ndarray) -> np.ndarray:
    return x64.astype(np.float16).view(np.uint16)


def _bits_bf16(x64: np.ndarray) -> np.ndarray:
    # float64 -> float32 -> bfloat16, each step round-to-nearest-even
    u = x64.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def to_bits(x64: np.ndarray, dtype: int) -> np.ndarray:
    return _bits_bf16(x64) if dtype == BF16 else _bits_f16(x64)


def bits_to_float(b: np.ndarray, dtype: int) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    if dtype == BF16:
        return (b.astype(np.uint32) << 16).view(np.float32)
    return b.view(np.float16).astype(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    bits: int
    k_group: int
    v_group: int
    residual: int
    block_size: int
    dtype: int
    seq_lens: np.ndarray          # [S] tokens in the cache before the timed work
    extra_tokens: int             # tokens appended later (decode steps or a prefill chunk)
    n_outlier: int
    outlier_scale: float
    q_scale: float
    shuffle: bool
    pool_factor: float
    seed: int = 0
    cfg_id: int = 0
    v_flush: int = 0              # 1: Values leave the residual with the Keys

    # ---- pages ---------------------------------------------------------------
    @property
    def final_lens(self) -> np.ndarray:
        return self.seq_lens + self.extra_tokens

    @property
    def blocks_per_seq(self) -> np.ndarray:
        return (self.final_lens + self.block_size - 1) // self.block_size

    @property
    def max_blocks(self) -> int:
        return int(self.blocks_per_seq.max()) if self.num_seqs else 0

    @property
    def num_blocks(self) -> int:
        need = int(self.blocks_per_seq.sum())
        return int(math.ceil(need * self.pool_factor)) if self.shuffle else need

    def block_table(self) -> np.ndarray:
        """[S][max_blocks] int32 physical block ids (-1 past a sequence's end)."""
        S, mb = self.num_seqs, self.max_blocks
        bt = np.full((S, max(mb, 1)), -1, dtype=np.int32)
        if self.shuffle:
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, self.cfg_id, 4])))
            ids = rng.permutation(self.num_blocks).astype(np.int32)
        else:
            ids = np.arange(self.num_blocks, dtype=np.int32)
        pos = 0
        for s in range(S):
            n = int(self.blocks_per_seq[s])
            bt[s, :n] = ids[pos:pos + n]
            pos += n
        return bt

    # ---- tensors -------------------------------------------------------------
    def _rng(self, *tag) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, self.cfg_id, *tag])))

    def outlier_channels(self) -> np.ndarray:
        """[H_KV][n_outlier] channel ids, drawn without replacement per KV head."""
        rng = self._rng(5)
        return np.stack([rng.choice(self.head_dim, size=self.n_outlier, replace=False)
                         for _ in range(self.num_kv_heads)]) if self.n_outlier else \
            np.zeros((self.num_kv_heads, 0), dtype=np.int64)

    def kv_stream(self, s: int, t0: int = 0, t1: int | None = None):
        """Token stream of request s, positions [t0, t1): (k_bits, v_bits), [n][H_KV][d] uint16."""
        T = int(self.final_lens[s])
        t1 = T if t1 is None else t1
        H, d = self.num_kv_heads, self.head_dim
        k = self._rng(0, s).standard_normal((T, H, d))[t0:t1]
        v = self._rng(1, s).standard_normal((T, H, d))[t0:t1]
        if self.n_outlier:
            oc = self.outlier_channels()
            for h in range(H):
                k[:, h, oc[h]] *= self.outlier_scale
        return to_bits(k, self.dtype), to_bits(v, self.dtype)

    def kv_streams(self, threads: int = 8) -> list:
        """kv_stream(s) for every request, drawn on a thread pool (numpy's generators
        release the GIL while filling); identical to the serial calls."""
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max(1, threads)) as ex:
            return list(ex.map(self.kv_stream, range(self.num_seqs)))

    def q_decode(self, step: int = 0) -> np.ndarray:
        """Decode queries for one step: [S][H_Q][d] uint16."""
        x = self._rng(2, step).standard_normal((self.num_seqs, self.num_q_heads, self.head_dim))
        return to_bits(x * self.q_scale, self.dtype)

    def q_prefill(self) -> np.ndarray:
        """Prefill chunk queries: [S * extra_tokens][H_Q][d] uint16 (request-major)."""
        x = self._rng(3).standard_normal((self.num_seqs * self.extra_tokens, self.num_q_heads, self.head_dim))
        return to_bits(x * self.q_scale, self.dtype)


def config(cfg_id: int, bits: int | None = None, **over) -> Workload:
    """The five workloads (sizes as the method's target deployments use them).

    1  tiny: 1 request, 4 query heads over 1 KV head, T=256, G=32, Gv=32, R=32, int4 or int2
    2  Llama-3-8B-shaped decode: 32 requests x 4096 tokens, 32 Q / 8 KV heads, G=64, Gv=128, R=128, int4
    3  long context: 4 requests x 32768 tokens, G=128, Gv=128, R=128, int4 or int2, shuffled 1.25x pool
    4  ragged stream: 256 requests, T ~ U{128..8192}, 64 decode steps, G=64, Gv=128, R=64, int4, shuffled
    5  Qwen2.5-7B-shaped chunked prefill: 8 requests x 16384 cached + 512-token chunk, 28 Q / 4 KV, bf16
    """
    d = 128
    if cfg_id == 1:
        w = Workload("tiny-1x4q1kv-T256", 1, 4, 1, d, bits or 4, 32, 32, 32, 16, F16,
                     np.array([256]), 0, 4, 20.0, 1.0 / math.sqrt(d), False, 1.0)
    elif cfg_id == 2:
        w = Workload("llama3-8b-decode-b32-T4096", 32, 32, 8, d, bits or 4, 64, 128, 128, 16, F16,
                     np.full(32, 4096), 0, 3, 15.0, 1.0, False, 1.0)
    elif cfg_id == 3:
        w = Workload("long-context-b4-T32768", 4, 32, 8, d, bits or 4, 128, 128, 128, 16, F16,
                     np.full(4, 32768), 0, 3, 15.0, 1.0, True, 1.25)
    elif cfg_id == 4:
        lens = np.random.default_rng(0).integers(128, 8193, 256)
        w = Workload("ragged-stream-b256", 256, 32, 8, d, bits or 4, 64, 128, 64, 16, F16,
                     lens, 64, 3, 15.0, 1.0, True, 1.25)
    elif cfg_id == 5:
        w = Workload("qwen2.5-7b-prefill-b8-16384+512", 8, 28, 4, d, bits or 4, 128, 128, 128, 16, BF16,
                     np.full(8, 16384), 512, 4, 20.0, 1.0, False, 1.0)
    else:
        raise ValueError(cfg_id)
    w.cfg_id = cfg_id
    for k, v in over.items():
        if k == "seq_lens":
            v = np.asarray(v)
        setattr(w, k, v)
    w.seq_lens = np.asarray(w.seq_lens, dtype=np.int64)
    if "num_seqs" in over and "seq_lens" not in over:
        w.seq_lens = w.seq_lens[:w.num_seqs] if len(w.seq_lens) >= w.num_seqs else \
            np.resize(w.seq_lens, w.num_seqs)
    return w
