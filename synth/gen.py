"""Counter-based random streams and the input generators built on them.

The bulk generators run in a small C core (fastgen.c, same definitions).
Random bits come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used counter-style: draw i of
stream key k is mix(k + (i + 1) * GAMMA).  Normals use the Box-Muller
transform (one normal from the two 32-bit halves of one draw).  Everything is vectorised numpy and
fully determined by (seed, tags).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fastgen.c")
# SVT_SANITIZE=1 selects an AddressSanitizer + UBSan build (clang's runtime,
# which the process must preload), kept apart from the normal library.
SANITIZE = os.environ.get("SVT_SANITIZE", "0") not in ("", "0")
_LIB = os.path.join(_HERE, "libsynth_san.so" if SANITIZE else "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C generator core with gcc (ISO C11, no fast-math), or with
    clang and AddressSanitizer + UBSan when SVT_SANITIZE=1."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        if SANITIZE:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-std=c11", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-shared-libasan", "-shared",
                   "-fPIC", _SRC, "-lm", "-o", tmp]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", _SRC, "-lm", "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _c():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, u64_, i64_, d_ = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        L.synth_u64.argtypes = [u64_, i64_, i64_, P]
        L.synth_normal_f64.argtypes = [u64_, i64_, d_, P]
        L.synth_normal_f32.argtypes = [u64_, i64_, d_, P]
        L.synth_normal_bf16.argtypes = [u64_, i64_, d_, P]
        L.synth_commit_pattern.argtypes = [P, i64_, i64_, i64_, P]
        _lib = L
    return _lib

__all__ = [
    "GAMMA", "mix64", "stream_key", "u64", "uniform01", "normal", "normal_f32", "normal_bf16", "randint",
    "to_bf16_bits", "bf16_bits_to_f32",
    "tree_depth_capped", "tree_bushy", "tree_chain", "tree_star", "tree_relabel",
    "logits_with_designated_top", "plant_drafts", "prefix_lengths",
    "commit_pattern_bits", "commit_pattern_slabs", "commit_pattern_torch",
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
    out = np.empty(n, dtype=np.uint64)
    if n:
        _c().synth_u64(int(key), start, n, out.ctypes.data_as(ctypes.c_void_p))
    return out


def uniform01(key, n: int, start: int = 0) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (u64(key, n, start) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal(key, n: int, sigma: float = 1.0) -> np.ndarray:
    """n standard normals times sigma (float64).  Box-Muller on the two 32-bit
    halves of draw i: u1 = (hi + 1) / 2^32 in (0, 1], u2 = lo / 2^32."""
    out = np.empty(n, dtype=np.float64)
    if n:
        _c().synth_normal_f64(int(key), n, float(sigma), out.ctypes.data_as(ctypes.c_void_p))
    return out


def normal_f32(key, n: int, sigma: float = 1.0) -> np.ndarray:
    """Same values as normal(), rounded to float32."""
    out = np.empty(n, dtype=np.float32)
    if n:
        _c().synth_normal_f32(int(key), n, float(sigma), out.ctypes.data_as(ctypes.c_void_p))
    return out


def normal_bf16(key, n: int, sigma: float = 1.0) -> np.ndarray:
    """Same values as normal_f32(), rounded to bfloat16 (nearest-even); uint16 bits."""
    out = np.empty(n, dtype=np.uint16)
    if n:
        _c().synth_normal_bf16(int(key), n, float(sigma), out.ctypes.data_as(ctypes.c_void_p))
    return out


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


def tree_layered(key, M: int, depth: int) -> np.ndarray:
    """M nodes spread as evenly as possible over levels 1..min(depth, M) (lower
    levels take the remainder); a node picks its parent uniformly among the
    nodes of the level above (the root is level 0).  Node ids grow with level."""
    D = max(1, min(depth, M))
    per = [M // D + (1 if k < M % D else 0) for k in range(D)]
    par = np.zeros(M + 1, dtype=np.int32)
    u = uniform01(key, max(M, 1))
    prev = [0]
    i = 1
    for k in range(D):
        cur = []
        for _ in range(per[k]):
            par[i] = prev[min(int(u[i - 1] * len(prev)), len(prev) - 1)]
            cur.append(i)
            i += 1
        prev = cur
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


def commit_pattern_slabs(slabs, ncol: int, nel: int) -> np.ndarray:
    """commit_pattern_bits for whole slabs: out[i][c][e] for slab slabs[i]."""
    sl = np.ascontiguousarray(np.asarray(slabs, dtype=np.int64).reshape(-1))
    out = np.empty((len(sl), ncol, nel), dtype=np.uint16)
    if out.size:
        _c().synth_commit_pattern(sl.ctypes.data_as(ctypes.c_void_p), len(sl), ncol, nel,
                                  out.ctypes.data_as(ctypes.c_void_p))
    return out


def commit_pattern_torch(slab, col, elem):
    """The same hash on torch int64 tensors (any device), returned as int16
    bits; used to fill large caches directly in device memory."""
    h = (slab * 1000003 + col) * 131 + elem
    h = h ^ (h >> 13)
    h = (h * 40503) & 0xFFFFFFFF
    h = h ^ (h >> 16)
    h = h & 0xFFFF
    return (h - ((h >> 15) << 16)).to(dtype=__import__("torch").int16)
