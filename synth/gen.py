"""Counter-based random streams and the input generators built on them.

Random bits come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used counter-style: draw i of
stream key k is mix(k + (i + 1) * GAMMA).  Normals use the Box-Muller
transform (one normal from two uniforms).  Everything is vectorised numpy and
fully determined by (seed, tags).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "GAMMA", "mix64", "stream_key", "u64", "uniform01", "normal", "randint",
    "to_bf16_bits", "bf16_bits_to_f32",
    "tree_depth_capped", "tree_bushy", "tree_chain", "tree_star", "tree_relabel",
    "logits_with_designated_top", "plant_drafts", "prefix_lengths",
    "commit_pattern_bits",
]

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def mix64(z):
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, *tags: int) -> np.uint64:
    """Derive an independent stream key from a seed and integer tags."""
    k = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    for t in tags:
        with np.errstate(over="ignore"):
            k = mix64(k ^ mix64(np.uint64(t & 0xFFFFFFFFFFFFFFFF) + GAMMA))
    return np.uint64(k)


def u64(key, n: int, start: int = 0) -> np.ndarray:
    """Draws start .. start+n-1 of the stream with key `key`."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + i * GAMMA)


def uniform01(key, n: int, start: int = 0) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (u64(key, n, start) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(key, n: int, sigma: float = 1.0) -> np.ndarray:
    """n standard normals times sigma (float64), Box-Muller on draws 2i, 2i+1."""
    r = u64(key, 2 * n)
    u1 = ((r[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)
    u2 = (r[1::2] >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2) * sigma


def randint(key, n: int, lo: int, hi: int, start: int = 0) -> np.ndarray:
    """Uniform integers in [lo, hi] (inclusive), by multiply-shift on 32 bits."""
    span = np.uint64(hi - lo + 1)
    r = u64(key, n, start) >> np.uint64(32)
    return (lo + ((r * span) >> np.uint64(32)).astype(np.int64)).astype(np.int64)


def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns the uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Trees.  A tree of M draft nodes is a parent array of length T = M + 1 whose
# row 0 is the root and holds 0 (no negative sentinel).
# --------------------------------------------------------------------------
def tree_depth_capped(key, M: int, depth_cap: int) -> np.ndarray:
    """Node i picks its parent uniformly among earlier nodes of depth < cap."""
    par = np.zeros(M + 1, dtype=np.int32)
    dep = np.zeros(M + 1, dtype=np.int64)
    u = uniform01(key, max(M, 1))
    for i in range(1, M + 1):
        cand = np.nonzero(dep[:i] < depth_cap)[0]
        j = cand[min(int(u[i - 1] * len(cand)), len(cand) - 1)]
        par[i] = j
        dep[i] = dep[j] + 1
    return par


def tree_bushy(key, M: int, depth_cap: int = 10, wide: int = 4, narrow: int = 2,
               wide_depth: int = 1) -> np.ndarray:
    """Wide near the root: a node of depth <= wide_depth takes up to `wide`
    children, deeper nodes up to `narrow`; depth stays below depth_cap."""
    par = np.zeros(M + 1, dtype=np.int32)
    dep = np.zeros(M + 1, dtype=np.int64)
    kids = np.zeros(M + 1, dtype=np.int64)
    u = uniform01(key, max(M, 1))
    for i in range(1, M + 1):
        limit = np.where(dep[:i] <= wide_depth, wide, narrow)
        cand = np.nonzero((dep[:i] < depth_cap) & (kids[:i] < limit))[0]
        j = cand[min(int(u[i - 1] * len(cand)), len(cand) - 1)]
        par[i] = j
        dep[i] = dep[j] + 1
        kids[j] += 1
    return par


def tree_chain(M: int) -> np.ndarray:
    return np.concatenate([[0], np.arange(M)]).astype(np.int32)


def tree_star(M: int) -> np.ndarray:
    return np.zeros(M + 1, dtype=np.int32)


def tree_relabel(key, par: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Relabel nodes 1..M by a seeded permutation (root stays 0).  Returns the
    relabelled parent array and perm, where old node i becomes perm[i]."""
    M = len(par) - 1
    order = np.argsort(u64(key, M), kind="stable") + 1
    perm = np.zeros(M + 1, dtype=np.int64)
    perm[1:] = order
    new = np.zeros(M + 1, dtype=np.int32)
    for i in range(1, M + 1):
        new[perm[i]] = perm[par[i]]
    return new, perm


# --------------------------------------------------------------------------
# Logits and drafts.
# --------------------------------------------------------------------------
def logits_with_designated_top(key, rows: int, V: int, clamp: float = 6.0,
                               top: float = 10.0) -> tuple[np.ndarray, np.ndarray]:
    """float32 logits, N(0,1) truncated to [-clamp, clamp], with one seeded
    token per row lifted to `top` (> clamp), so that the row's greedy token is
    known by construction.  Returns (logits [rows][V], designated [rows])."""
    x = np.clip(normal(stream_key(int(key), 1), rows * V), -clamp, clamp).astype(np.float32)
    x = x.reshape(rows, V)
    des = randint(stream_key(int(key), 2), rows, 0, V - 1)
    x[np.arange(rows), des] = np.float32(top)
    return x, des.astype(np.int32)


def plant_drafts(key, parents: np.ndarray, parent_top: np.ndarray, V: int,
                 p: float) -> np.ndarray:
    """Draft tokens for one tree: the root token is uniform; node i >= 1 takes
    parent_top[parents[i]] with probability p, else a uniform token."""
    T = len(parents)
    u = uniform01(stream_key(int(key), 1), T)
    r = randint(stream_key(int(key), 2), T, 0, V - 1)
    tok = r.astype(np.int32).copy()
    for i in range(1, T):
        if u[i] < p:
            tok[i] = parent_top[parents[i]]
    return tok


def prefix_lengths(key, B: int, lo: int, hi: int) -> np.ndarray:
    return randint(key, B, lo, hi).astype(np.int32)


def commit_pattern_bits(slab: np.ndarray, col: np.ndarray, elem: np.ndarray) -> np.ndarray:
    """16-bit integer hash of (slab, column, element), used as raw cache
    contents in commit tests (covers every bit pattern, NaN payloads
    included).  Written with int64 arithmetic that never overflows for
    slab < 2**16, col < 2**17, elem < 2**8, so torch can evaluate the same
    formula on the device."""
    h = (np.asarray(slab, np.int64) * 1000003 + np.asarray(col, np.int64)) * 131 + np.asarray(elem, np.int64)
    h = h ^ (h >> 13)
    h = (h * 40503) & 0xFFFFFFFF
    h = h ^ (h >> 16)
    return (h & 0xFFFF).astype(np.uint16)
