"""Seeded synthetic inputs for observation-window KV selection.

This module only draws inputs.  It contains none of the selection arithmetic,
imports nothing else from this package, and is the one module that both the
HIP path's callers and the CPU oracle's tests use, so that both consume the
same bytes.

Recipe (frozen; tests/test_workloads.py hashes a sample of the bytes):
  * one numpy PCG64 stream per (sequence, layer, head):
    ``default_rng(SeedSequence(seed, spawn_key=(seq, layer, head)))``;
  * per head, draws happen in this order:
      1. Qwin  [W, D]  standard normal (float32 ziggurat),
      2. K     [L, D]  standard normal, or for the "codebook" recipe a
                       [16, D] normal codebook followed by L uniform codes,
      3. V     [L, D]  standard normal,
      4. key modifiers: "lognorm" draws ln n_j ~ N(0, 0.5^2) for every
         position and scales row j by n_j; "spike" (also applied after the
         codebook) picks floor(frac * P) distinct prefix positions and sets
         k_j = 3 * mean_i(Qwin_i) + N(0, I), the mean taken in float64 over the
         head's W stored (already rounded) window queries;
  * bf16 workloads round each float32 value once to bfloat16 with
    round-to-nearest-even, after the modifiers (which run in float64 and are
    rounded to float32 first);
  * ragged batches draw their prompt lengths first, from
    ``default_rng(seed)``, uniform on [L_min, L_max] inclusive; the budget of
    sequence b is floor(L_b / 10) (compression 0.9, the budget includes the
    window).

The workloads stand in for the long-prompt settings the pages discuss (a 32
query-head layer with a 32-token window over 16K prompts, a 1024-token budget,
compression 0.9 over 8K-64K inputs, max pooling of width 5); no dataset or
model weights are involved.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import List, Optional, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    heads: int
    W: int
    D: int
    dtype: str            # "f32" or "bf16"
    kernel: int
    pooling: str          # "avg" or "max"
    L: int = 0            # prompt length (single-length workloads)
    C: int = 0            # budget including the window (single-length)
    layers: int = 1       # independent layers, one selection call each
    batch: int = 1        # sequences in a ragged batch
    L_min: int = 0        # ragged: inclusive length range
    L_max: int = 0
    keys: str = "normal"  # "normal" | "lognorm" | "spike" | "codebook"
    spike_frac: float = 0.0
    codebook: int = 16
    lognorm_sigma: float = 0.5

    @property
    def ragged(self) -> bool:
        return self.batch > 1 or self.L_min > 0


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp32_h1_l1k", seed=1, heads=1, L=1024, W=32, C=256, D=64,
                 dtype="f32", kernel=3, pooling="avg"),
        Workload("lognorm_h32_l16k", seed=2, heads=32, L=16384, W=32, C=2048, D=128,
                 dtype="bf16", kernel=5, pooling="avg", keys="lognorm"),
        Workload("spike_l32x_h32_l32k", seed=3, heads=32, layers=32, L=32768, W=32, C=1024,
                 D=128, dtype="bf16", kernel=5, pooling="max", keys="spike", spike_frac=0.01),
        Workload("ragged_b8_h32_l4k_64k", seed=4, heads=32, batch=8, L_min=4096, L_max=65536,
                 W=32, D=128, dtype="bf16", kernel=7, pooling="avg"),
        Workload("tied_h64_l128k", seed=5, heads=64, L=131072, W=64, C=4096, D=128,
                 dtype="bf16", kernel=5, pooling="avg", keys="codebook", spike_frac=0.005),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def reduced(w: Workload, **changes) -> Workload:
    """A smaller variant of a workload (same recipe, other sizes)."""
    name = changes.pop("name", None) or (w.name + "_reduced")
    return replace(w, name=name, **changes)


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 upcast of stored fp32 values or bf16 bit patterns."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored, dtype=np.float32).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


# ---------------------------------------------------------------- lengths

def seq_lengths(w: Workload) -> List[int]:
    if not w.ragged:
        return [w.L]
    rng = np.random.default_rng(w.seed)
    return [int(x) for x in rng.integers(w.L_min, w.L_max, size=w.batch, endpoint=True)]


def budgets(w: Workload) -> List[int]:
    if not w.ragged:
        return [w.C]
    return [L // 10 for L in seq_lengths(w)]


# ---------------------------------------------------------------- one head

def head_arrays(w: Workload, head: int, layer: int = 0, seq: int = 0,
                L: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(Qwin [W, D], K [L, D], V [L, D]) of one head in storage form: float32
    for "f32" workloads, uint16 bf16 bit patterns for "bf16"."""
    if L is None:
        L = seq_lengths(w)[seq]
    W, D = w.W, w.D
    rng = np.random.default_rng(np.random.SeedSequence(w.seed, spawn_key=(seq, layer, head)))
    q32 = rng.standard_normal((W, D), dtype=np.float32)
    q = _store(q32, w.dtype)
    if w.keys == "codebook":
        book = rng.standard_normal((w.codebook, D), dtype=np.float32)
        codes = rng.integers(0, w.codebook, size=L)
        k32 = book[codes]
    else:
        k32 = rng.standard_normal((L, D), dtype=np.float32)
    v32 = rng.standard_normal((L, D), dtype=np.float32)
    if w.keys == "lognorm":
        scale = np.exp(rng.normal(0.0, w.lognorm_sigma, size=L))
        k32 = (k32.astype(np.float64) * scale[:, None]).astype(np.float32)
    if w.spike_frac > 0.0:
        P = L - W
        count = int(np.floor(w.spike_frac * P))
        if count > 0:
            where = rng.choice(P, size=count, replace=False)
            mean_q = to_float64(q, w.dtype).mean(axis=0)
            noise = rng.standard_normal((count, D))
            k32 = np.array(k32, copy=True)
            k32[where] = (3.0 * mean_q[None, :] + noise).astype(np.float32)
    return q, _store(k32, w.dtype), _store(v32, w.dtype)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_arrays(w: Workload, layer: int = 0, seq: int = 0, heads: Optional[Sequence[int]] = None,
                 threads: Optional[int] = None):
    """Stacked (Qwin [H, W, D], K [H, L, D], V [H, L, D]) of one layer of one
    sequence in storage form, heads drawn in parallel threads."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    L = seq_lengths(w)[seq]
    store_t = np.uint16 if w.dtype == "bf16" else np.float32
    Q = np.empty((len(heads), w.W, w.D), dtype=store_t)
    K = np.empty((len(heads), L, w.D), dtype=store_t)
    V = np.empty((len(heads), L, w.D), dtype=store_t)

    def fill(i_h):
        i, h = i_h
        Q[i], K[i], V[i] = head_arrays(w, h, layer=layer, seq=seq, L=L)

    with ThreadPoolExecutor(max_workers=threads or _threads()) as ex:
        list(ex.map(fill, enumerate(heads)))
    return Q, K, V


def ragged_arrays(w: Workload, layer: int = 0, threads: Optional[int] = None):
    """Packed ragged batch: Qwin [B, H, W, D]; K and V as one flat array in
    which sequence b occupies [H, L_b, D] starting at element H * cu_L[b] * D;
    returns (Qwin, K, V, lengths, budgets, cu_L)."""
    lengths = seq_lengths(w)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    store_t = np.uint16 if w.dtype == "bf16" else np.float32
    Q = np.empty((len(lengths), w.heads, w.W, w.D), dtype=store_t)
    K = np.empty(w.heads * int(cu[-1]) * w.D, dtype=store_t)
    V = np.empty_like(K)
    for b, L in enumerate(lengths):
        q, k, v = layer_arrays(w, layer=layer, seq=b, threads=threads)
        Q[b] = q
        lo, hi = w.heads * int(cu[b]) * w.D, w.heads * int(cu[b + 1]) * w.D
        K[lo:hi] = k.reshape(-1)
        V[lo:hi] = v.reshape(-1)
    return Q, K, V, lengths, budgets(w), cu


# ---------------------------------------------------------------- Jacap events

def jacap_arrays(seed: int, heads: int, N: int, D: int, mu_scale: float = 1.0, separate_u: bool = False):
    """Inputs of one Jacap eviction event over N cached tokens per head:
    (K, V, U) [heads, N, D] as bf16 bit patterns, mu_q and lambda_q [heads, D]
    float32.  Per head one PCG64 stream, ``default_rng(SeedSequence(seed,
    spawn_key=(head,)))``, draws in this order: K standard normal, V standard
    normal, U standard normal when `separate_u` (a stand-in for W_O v; else
    U = V, the cheaper proxy), mu_q normal with standard deviation mu_scale,
    lambda_q uniform on [0.1, 2) (a diagonal second moment with the floor
    already applied)."""
    K = np.empty((heads, N, D), dtype=np.uint16)
    V = np.empty_like(K)
    U = np.empty_like(K)
    mu = np.empty((heads, D), dtype=np.float32)
    lam = np.empty((heads, D), dtype=np.float32)
    for h in range(heads):
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(h,)))
        K[h] = f32_to_bf16_bits(rng.standard_normal((N, D), dtype=np.float32))
        V[h] = f32_to_bf16_bits(rng.standard_normal((N, D), dtype=np.float32))
        U[h] = f32_to_bf16_bits(rng.standard_normal((N, D), dtype=np.float32)) if separate_u else V[h]
        mu[h] = (mu_scale * rng.standard_normal(D)).astype(np.float32)
        lam[h] = rng.uniform(0.1, 2.0, size=D).astype(np.float32)
    return K, V, U, mu, lam
