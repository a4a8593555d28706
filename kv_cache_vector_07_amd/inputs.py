"""Seeded synthetic workloads for the TurboQuant KV cache.

This module only draws random inputs and describes shapes; it holds none of
the method's arithmetic. Tests, the benchmark and the CPU reference all take
their inputs from here, so both sides of every comparison see the same bytes.

Every array is drawn chunk by chunk from numpy's PCG64 seeded with
(data_seed, stream tag, sequence, chunk), so any token range can be generated
without drawing the whole cache, and the same range always yields the same
values. Values are float64 normals, scaled, cast to float32 and, for bfloat16
workloads, rounded to bfloat16 (round-to-nearest-even); the returned float32
arrays hold exactly the values the kernels receive.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096          # tokens per generation chunk (any range is a union of chunks)
QJL_SEED = 12345
_TAG = {"k": 1, "v": 2, "q": 3, "scale": 4, "lens": 5}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16"
    k_dist: str                     # "normal" or "outlier"
    data_seed: int
    fixed_len: int = 0              # context length when all sequences are equal
    len_range: tuple = ()           # (lo, hi) inclusive, drawn per sequence
    n_q: int = 1                    # query tokens per sequence per decode step
    page_size: int = 256
    decode_steps: int = 1
    append_per_step: int = 0        # tokens appended (encoded) per sequence per step
    prefill_chunk: int = 0          # append granularity of the initial cache build
    qjl_seed: int = QJL_SEED
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def workload(n: int) -> Workload:
    """The five synthetic workloads (1-based)."""
    table = {
        1: Workload("tiny_ref", 1, 1, 1, 128, "f32", "normal", 1, fixed_len=1024,
                    note="1 KV head, 1 query head, d=128, L=1024, fp32 N(0,1)"),
        2: Workload("gqa_32k", 1, 32, 8, 128, "bf16", "outlier", 2, fixed_len=32768,
                    decode_steps=256, append_per_step=1,
                    note="B=1, 32 q heads / 8 KV heads, d=128, L=32768, bf16"),
        3: Workload("long_100k", 1, 16, 8, 128, "bf16", "outlier", 3, fixed_len=100000,
                    decode_steps=256, append_per_step=1,
                    note="B=1, 16 q heads / 8 KV heads, d=128, L=100000, bf16"),
        4: Workload("batched_paged", 32, 32, 8, 128, "bf16", "normal", 4,
                    len_range=(4096, 16384), decode_steps=256, append_per_step=1,
                    note="B=32, L~U[4096,16384], 32/8 heads, d=128, 256-token pages"),
        5: Workload("prefill_verify", 4, 32, 8, 256, "bf16", "outlier", 5, fixed_len=131072,
                    n_q=4, decode_steps=64, prefill_chunk=4096,
                    note="B=4, L=131072, 32/8 heads, d=256, 4 query tokens, 4096-token chunks"),
    }
    return table[n]


def seq_lens(w: Workload) -> np.ndarray:
    """Context length of each sequence (int64 [B])."""
    if w.fixed_len:
        return np.full(w.batch, w.fixed_len, dtype=np.int64)
    lo, hi = w.len_range
    rng = np.random.default_rng([w.data_seed, _TAG["lens"]])
    return rng.integers(lo, hi + 1, size=w.batch).astype(np.int64)


def round_to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> the nearest value of `dtype` (returned as float32)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that are exact bfloat16 values."""
    return (np.ascontiguousarray(x32, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def k_channel_scales(w: Workload) -> np.ndarray:
    """Per-(KV head, channel) scale of K: [Hkv][d] float64.

    "outlier": log-uniform in [0.5, 2] per channel, and 4 channels per head,
    chosen without replacement, multiplied by 20. "normal": all ones.
    Shared by every token and sequence.
    """
    if w.k_dist == "normal":
        return np.ones((w.n_kv_heads, w.head_dim))
    rng = np.random.default_rng([w.data_seed, _TAG["scale"]])
    s = np.exp(rng.uniform(np.log(0.5), np.log(2.0), size=(w.n_kv_heads, w.head_dim)))
    for h in range(w.n_kv_heads):
        s[h, rng.choice(w.head_dim, size=4, replace=False)] *= 20.0
    return s


def _chunk(w: Workload, which: str, b: int, c: int, scales) -> np.ndarray:
    rng = np.random.default_rng([w.data_seed, _TAG[which], b, c])
    z = rng.standard_normal((CHUNK, w.n_kv_heads, w.head_dim))
    if which == "k":
        z = z * scales[None]
    return round_to_dtype(z.astype(np.float32), w.dtype)


def kv_tokens(w: Workload, which: str, b: int, t0: int, t1: int) -> np.ndarray:
    """K or V of tokens t0..t1-1 of sequence b: float32 [t1-t0][Hkv][d]."""
    scales = k_channel_scales(w) if which == "k" else None
    parts = []
    for c in range(t0 // CHUNK, (max(t1, t0 + 1) - 1) // CHUNK + 1):
        lo, hi = max(t0, c * CHUNK), min(t1, (c + 1) * CHUNK)
        if hi <= lo:
            continue
        parts.append(_chunk(w, which, b, c, scales)[lo - c * CHUNK:hi - c * CHUNK])
    if not parts:
        return np.zeros((0, w.n_kv_heads, w.head_dim), np.float32)
    return np.concatenate(parts, axis=0)


def queries(w: Workload, step: int) -> np.ndarray:
    """Queries of decode step `step`: float32 [B][n_q][Hq][d], N(0, 1)."""
    rng = np.random.default_rng([w.data_seed, _TAG["q"], step])
    z = rng.standard_normal((w.batch, w.n_q, w.n_q_heads, w.head_dim)).astype(np.float32)
    return round_to_dtype(z, w.dtype)


def page_table(w: Workload, lens: np.ndarray, extra_tokens: int = 0, shuffle: bool = True):
    """A block table [B][max_pages] mapping each sequence's pages to physical
    pages of one shared pool, plus the pool size. Pages are handed out in a
    seeded random order so that logical neighbours are not physical neighbours."""
    P = w.page_size
    need = [(int(L) + extra_tokens + P - 1) // P for L in lens]
    total = int(sum(need))
    order = np.arange(total, dtype=np.int32)
    if shuffle:
        np.random.default_rng([w.data_seed, 99]).shuffle(order)
    max_pages = max(need) if need else 1
    table = np.zeros((len(lens), max(max_pages, 1)), dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = order[pos:pos + n]
        pos += n
    return table, total
