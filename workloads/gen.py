"""Seeded synthetic inputs for the ZHA workloads.

This module only draws random numbers and rounds them to the storage precision; it holds
none of the method's arithmetic.  Both the CPU oracle side (tests) and the GPU side
(tests, bench) take their inputs from here, so both see identical bits.

Recipe
------
* Generator: NumPy ``Generator(Philox)`` seeded with
  ``SeedSequence([2026, cfg_id, stream, slot, chunk])``.
  Streams: 0 = keys, 1 = values, 2 = reference queries, 3 = planted-key counts and
  indices, 4 = query noise.  For keys and values ``slot`` is the KV head and ``chunk``
  indexes 2^20-token chunks, so any chunk can be regenerated on its own and every size of
  one workload family is a prefix of the same token sequence.  Tokens appended during
  decode are the continuation of that same sequence (token ``n_tokens + t`` at step t).
* Values are standard normals drawn in float32, then (bf16 workloads) rounded to bfloat16
  with round-to-nearest-even.  Reference queries and decode queries are rounded the same
  way, so every bf16 x bf16 product in the GPU path is exact.
* Planted queries: for step t and query head h, m ~ U{plant_min..plant_max} distinct
  token indices drawn uniformly from the tokens present at that step, of the head's KV
  head (head h reads KV head h // group); q = plant_scale * sqrt(d) * u / |u| with u the
  sum of those keys, plus N(0, I) noise when ``noise`` is set.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from .configs import Workload

CHUNK = 1 << 20
STREAM_K, STREAM_V, STREAM_REF, STREAM_PLANT, STREAM_NOISE = 0, 1, 2, 3, 4


def rng(cfg_id: int, stream: int, slot: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([2026, cfg_id, stream, slot, chunk])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values exactly representable in the workload's storage dtype."""
    x = np.asarray(x, dtype=np.float32)
    return bf16_to_f32(bf16_bits(x)) if dtype == "bf16" else x


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunk_rows(cfg_id: int, stream: int, head: int, chunk: int, upto: int, d: int) -> np.ndarray:
    g = rng(cfg_id, stream, head, chunk)
    return g.standard_normal(upto * d, dtype=np.float32).reshape(upto, d)


def token_rows(w: Workload, stream: int, head: int, start: int, stop: int) -> np.ndarray:
    """float32 rows [stop-start, d] of keys (stream 0) or values (stream 1), storage-rounded."""
    d = w.head_dim
    out = np.empty((stop - start, d), dtype=np.float32)
    jobs = []
    c0, c1 = start // CHUNK, (stop - 1) // CHUNK if stop > start else start // CHUNK - 1
    for c in range(c0, c1 + 1):
        lo, hi = max(start, c * CHUNK), min(stop, (c + 1) * CHUNK)
        jobs.append((c, lo, hi))

    def run(job):
        c, lo, hi = job
        rows = _chunk_rows(w.cfg_id, stream, head, c, hi - c * CHUNK, d)[lo - c * CHUNK:]
        out[lo - start:hi - start] = round_storage(rows, w.dtype)

    if len(jobs) > 1:
        with cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return out


def iter_kv_chunks(w: Workload, n: int | None = None, workers: int | None = None):
    """Yields (stream, kv_head, start, stop, float32 rows [stop-start, d]) for every chunk of
    the K (stream 0) and V (stream 1) caches over tokens [0, n), generated in parallel with a
    bounded number of chunks alive at once.  Same values as kv_cache()."""
    n = w.capacity if n is None else n
    jobs = [(s, h, c) for s in (STREAM_K, STREAM_V) for h in range(w.num_kv_heads)
            for c in range(0, -(-n // CHUNK))]
    workers = workers or _workers()

    def run(job):
        s, h, c = job
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rows = round_storage(_chunk_rows(w.cfg_id, s, h, c, hi - lo, w.head_dim), w.dtype)
        return s, h, lo, hi, rows

    with cf.ThreadPoolExecutor(workers) as ex:
        pending = []
        for job in jobs:
            pending.append(ex.submit(run, job))
            if len(pending) >= 2 * workers:
                yield pending.pop(0).result()
        for f in pending:
            yield f.result()


def kv_cache(w: Workload, n: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """K, V as float32 arrays [Hkv, n, d] (n defaults to the capacity), storage-rounded."""
    n = w.capacity if n is None else n
    jobs = [(s, h) for s in (STREAM_K, STREAM_V) for h in range(w.num_kv_heads)]
    res = {}

    def run(job):
        s, h = job
        res[job] = token_rows(w, s, h, 0, n)

    with cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    K = np.stack([res[(STREAM_K, h)] for h in range(w.num_kv_heads)])
    V = np.stack([res[(STREAM_V, h)] for h in range(w.num_kv_heads)])
    return K, V


def ref_queries(w: Workload) -> np.ndarray:
    """Reference queries [Hkv, R, d] (random N(0,1) stand-ins for the learned ones)."""
    out = [rng(w.cfg_id, STREAM_REF, h, 0).standard_normal(w.num_ref * w.head_dim, dtype=np.float32)
           for h in range(w.num_kv_heads)]
    return round_storage(np.stack(out).reshape(w.num_kv_heads, w.num_ref, w.head_dim), w.dtype)


def planted_query(w: Workload, step: int, q_head: int, n_present: int, fetch_rows) -> tuple[np.ndarray, np.ndarray]:
    """One decode query for ``q_head`` at ``step``; returns (q [d] float32, planted indices).

    ``fetch_rows(kv_head, idx)`` must return the stored key rows (float32 [len(idx), d]).
    """
    g = rng(w.cfg_id, STREAM_PLANT, q_head, step)
    m = int(g.integers(w.plant_min, w.plant_max + 1))
    m = min(m, n_present)
    idx = np.sort(g.choice(n_present, size=m, replace=False))
    kv = q_head // w.group
    u = np.asarray(fetch_rows(kv, idx), dtype=np.float64).sum(axis=0)
    nrm = np.linalg.norm(u)
    q = w.plant_scale * np.sqrt(w.head_dim) * (u / nrm if nrm > 0 else u)
    if w.noise:
        q = q + rng(w.cfg_id, STREAM_NOISE, q_head, step).standard_normal(w.head_dim)
    return round_storage(q.astype(np.float32), w.dtype), idx


def step_queries(w: Workload, step: int, n_present: int, fetch_rows) -> np.ndarray:
    """All query heads' decode queries for one step: float32 [Hq, d]."""
    return np.stack([planted_query(w, step, h, n_present, fetch_rows)[0] for h in range(w.num_q_heads)])


def host_fetch(K: np.ndarray):
    """``fetch_rows`` over a host cache [Hkv, N, d]."""
    return lambda kv, idx: K[kv, idx]
