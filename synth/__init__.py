"""Seeded synthetic inputs for attention tests and benchmarks.

This module holds no attention arithmetic.  It draws i.i.d. normal Q, K, V (the
pages' experiments reuse one set of randomly initialised query, key and value
tensors and state no distribution, so N(0, 1) is used), rounds them to the
storage type, and returns both the stored bits and their exact fp64 widening.
Both the HIP library (through the stored bits) and the CPU oracle (through the
widened copy) consume the same values; neither side imports the other.

Recipe:
  rng = numpy.random.default_rng([config_id, N, variant])
  Q, K, V = three successive standard_normal draws of shape [B, H, N, d]
  multiply Q and K by qk_factor and V by v_factor (in float64)
  round to float32 (round-to-nearest-even), then to the storage type with
  round-to-nearest-even (bf16: own routine below; fp16: numpy's conversion).
  Masks come from default_rng([config_id, N, 99]).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bits.

    Finite inputs only (the generators never produce inf or NaN).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def to_storage(x64: np.ndarray, dtype: str):
    """Round a float64 array to the storage type.

    Returns (stored, widened): `stored` is float32 / float16 / uint16 (bf16 bits),
    `widened` is the exact float64 value of what is stored.
    """
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "f16":
        h = x32.astype(np.float16)
        return h, h.astype(np.float64)
    if dtype == "bf16":
        b = f32_to_bf16_bits(x32)
        return b, bf16_bits_to_f64(b)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class QKV:
    """One seeded problem: stored tensors, their fp64 widening, and metadata."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q64: np.ndarray
    k64: np.ndarray
    v64: np.ndarray
    dtype: str
    seed: tuple


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, config_id: int, variant: int = 0,
             qk_factor: float = 1.0, v_factor: float = 1.0) -> QKV:
    """Seeded i.i.d. N(0,1) Q, K, V of shape [B, H, N, d], rounded to `dtype`."""
    seed = (int(config_id), int(N), int(variant))
    rng = np.random.default_rng(list(seed))
    shape = (B, H, N, d)
    q = rng.standard_normal(shape) * qk_factor
    k = rng.standard_normal(shape) * qk_factor
    v = rng.standard_normal(shape) * v_factor
    qs, q64 = to_storage(q, dtype)
    ks, k64 = to_storage(k, dtype)
    vs, v64 = to_storage(v, dtype)
    return QKV(qs, ks, vs, q64, k64, v64, dtype, seed)


def qkv_from_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: str) -> QKV:
    """Wrap hand-built float64 tensors (already representable or not) as a problem."""
    qs, q64 = to_storage(q, dtype)
    ks, k64 = to_storage(k, dtype)
    vs, v64 = to_storage(v, dtype)
    return QKV(qs, ks, vs, q64, k64, v64, dtype, ("explicit",))


def padding_mask(B: int, N: int, config_id: int, lengths) -> np.ndarray:
    """[B, N] uint8 key-padding mask: keys j >= lengths[b] are padded (1).

    `lengths[b]` may be an int, or None for a length drawn from U{1..N} using the
    mask stream default_rng([config_id, N, 99]).
    """
    rng = np.random.default_rng([int(config_id), int(N), 99])
    m = np.zeros((B, N), np.uint8)
    for b in range(B):
        L = lengths[b]
        if L is None:
            L = int(rng.integers(1, N + 1))
        m[b, int(L):] = 1
    return m


def c2_mask(B: int, N: int, config_id: int = 2) -> np.ndarray:
    """Key-padding mask of the B4 H16 N1024 d64 causal workload.

    Batch 0 has a random valid length in U{1..N} (one of four sequences, 25%),
    batch 1 is fully padded (every one of its query rows is fully masked), the
    remaining batches are unpadded.
    """
    lengths: list[Optional[int]] = [N] * B
    if B > 0:
        lengths[0] = None
    if B > 1:
        lengths[1] = 0
    return padding_mask(B, N, config_id, lengths)


def to_torch(arr: np.ndarray, dtype: str, device: str = "cuda"):
    """Copy stored values to a torch tensor of the storage type (bf16 from its bits)."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr, np.float16)).to(device)
    bits = np.ascontiguousarray(arr, np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(device).view(torch.bfloat16)


def upload(p: QKV, device: str = "cuda"):
    """(q, k, v) of a problem as device tensors."""
    return to_torch(p.q, p.dtype, device), to_torch(p.k, p.dtype, device), to_torch(p.v, p.dtype, device)


def sample_rows(B: int, H: int, N: int, per_head: int = 24, seed: int = 0) -> np.ndarray:
    """Flat row indices (b*H + h)*N + i for checks at full size: for every
    (b, h) the first rows, the rows around the first 32-row boundary, the middle
    and last rows, plus `per_head` rows drawn uniformly."""
    rng = np.random.default_rng([4242, B, H, N, seed])
    rows = []
    for bh in range(B * H):
        pick = {0, 1, min(31, N - 1), min(32, N - 1), N // 2, max(N - 2, 0), N - 1}
        pick.update(int(x) for x in rng.integers(0, N, size=per_head))
        rows.extend(bh * N + i for i in sorted(pick) if 0 <= i < N)
    return np.array(rows, np.int64)


def block_mask(B: int, H: int, N: int, block: int, config_id: int, pattern: str = "random",
               density: float = 0.5, band: int = 1, n_global: int = 1) -> np.ndarray:
    """[B, H, nb, nb] uint8 block flags (1 = the block of pairs is attended),
    nb = ceil(N / block), for the block-sparse forward.

    pattern "random": each flag i.i.d. Bernoulli(density) from the stream
    default_rng([config_id, N, 98]).  pattern "local_global": block (i, j) is on
    if |i - j| <= band (a sliding window of blocks) or i < n_global or
    j < n_global (global rows and columns), the same for every (b, h).
    """
    nb = (int(N) + int(block) - 1) // int(block)
    if pattern == "random":
        rng = np.random.default_rng([int(config_id), int(N), 98])
        return (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    if pattern == "local_global":
        i = np.arange(nb)[:, None]
        j = np.arange(nb)[None, :]
        on = (np.abs(i - j) <= band) | (i < n_global) | (j < n_global)
        return np.broadcast_to(on.astype(np.uint8), (B, H, nb, nb)).copy()
    raise ValueError(f"unknown pattern {pattern!r}")
