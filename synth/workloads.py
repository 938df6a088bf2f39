"""The five synthetic workloads of the tree-verification step and their
seeded materialisation.

Each workload fixes batch size, dtype, head layout, head dim, prefix-length
range, tree budget and shape rule, vocabulary, draft planting probability and
the number of cache layers a commit moves.  `instance()` draws one round of
inputs from the workload's seed; every tensor comes from its own stream, so a
test can regenerate any single tensor without the others.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import gen

SEED_BASE = 0x5EED0000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    dtype: str            # "fp32" or "bf16"
    Hq: int
    Hkv: int
    D: int
    len_lo: int
    len_hi: int
    M: int
    depth_cap: int
    tree: str             # "capped" or "bushy"
    V: int
    p_plant: float
    layers: int           # cache layers moved by one commit
    qkv_sigma: float
    seed: int

    @property
    def T(self) -> int:
        return self.M + 1

    @property
    def W(self) -> int:
        return (self.T + 63) // 64

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "fp32" else 2


WORKLOADS = [
    Workload("b1-fp32-h4kv1-d64-L128-M8", 1, "fp32", 4, 1, 64, 128, 128, 8, 4, "capped",
             1000, 0.7, 1, 1.0, SEED_BASE + 0),
    Workload("b1-bf16-h32kv8-d128-L2048-M16", 1, "bf16", 32, 8, 128, 2048, 2048, 16, 10, "capped",
             32000, 0.7, 32, 1.0 / math.sqrt(128), SEED_BASE + 1),
    Workload("b8-ragged-bf16-h32kv32-d128-L512to4096-M16", 8, "bf16", 32, 32, 128, 512, 4096, 16, 10,
             "capped", 32000, 0.7, 1, 1.0 / math.sqrt(128), SEED_BASE + 2),
    Workload("b1-long-bf16-h32kv2-d128-L32768-M64", 1, "bf16", 32, 2, 128, 32768, 32768, 64, 10,
             "bushy", 151552, 0.6, 1, 1.0 / math.sqrt(128), SEED_BASE + 3),
    Workload("b32-ragged-bf16-h32kv8-d128-L1024to8192-M32", 32, "bf16", 32, 8, 128, 1024, 8192, 32, 10,
             "capped", 32000, 0.75, 36, 1.0 / math.sqrt(128), SEED_BASE + 4),
]


def workload(key) -> Workload:
    """Look a workload up by position or by name."""
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS:
        if w.name == key:
            return w
    raise KeyError(key)


# Stream tags (one per tensor kind).
TAG_LEN, TAG_TREE, TAG_LOGITS, TAG_TOKENS, TAG_Q, TAG_KC, TAG_VC, TAG_KT, TAG_VT = range(1, 10)


def trees(w: Workload, seed: int | None = None) -> np.ndarray:
    s = w.seed if seed is None else seed
    out = np.zeros((w.B, w.T), dtype=np.int32)
    for b in range(w.B):
        k = gen.stream_key(s, TAG_TREE, b)
        if w.tree == "bushy":
            out[b] = gen.tree_bushy(k, w.M, depth_cap=w.depth_cap)
        else:
            out[b] = gen.tree_depth_capped(k, w.M, w.depth_cap)
    return out


def lengths(w: Workload, seed: int | None = None) -> np.ndarray:
    s = w.seed if seed is None else seed
    return gen.prefix_lengths(gen.stream_key(s, TAG_LEN), w.B, w.len_lo, w.len_hi)


def logits_and_drafts(w: Workload, parents: np.ndarray, seed: int | None = None):
    """Returns (logits [B][T][V] float32, tokens [B][T] int32, designated [B][T])."""
    s = w.seed if seed is None else seed
    logits, des = gen.logits_with_designated_top(gen.stream_key(s, TAG_LOGITS), w.B * w.T, w.V)
    des = des.reshape(w.B, w.T)
    tok = np.zeros((w.B, w.T), dtype=np.int32)
    for b in range(w.B):
        tok[b] = gen.plant_drafts(gen.stream_key(s, TAG_TOKENS, b), parents[b], des[b], w.V, w.p_plant)
    return logits.reshape(w.B, w.T, w.V), tok, des


def _values(w: Workload, key, shape) -> np.ndarray:
    """Gaussian values of the workload's dtype: float32 array for fp32, uint16
    bfloat16 bits for bf16."""
    n = int(np.prod(shape))
    if w.dtype == "fp32":
        return gen.normal_f32(key, n, w.qkv_sigma).reshape(shape)
    return gen.normal_bf16(key, n, w.qkv_sigma).reshape(shape)


def poison_value(w: Workload):
    """A NaN of the workload's dtype, written into cache columns outside the
    content so that a read of them shows up in the output."""
    return np.float32(np.nan) if w.dtype == "fp32" else np.uint16(0x7FC1)


def attention_inputs(w: Workload, lens: np.ndarray, cap: int, seed: int | None = None,
                     poison: bool = True):
    """q [B][T][Hq][D], k/v cache [B][Hkv][cap][D] (content right-aligned at
    lmax = max(lens)), k/v tree [B][Hkv][T][D].  Columns outside each
    sequence's content hold NaN when `poison`."""
    s = w.seed if seed is None else seed
    lmax = int(lens.max()) if len(lens) else 0
    q = _values(w, gen.stream_key(s, TAG_Q), (w.B, w.T, w.Hq, w.D))
    kt = _values(w, gen.stream_key(s, TAG_KT), (w.B, w.Hkv, w.T, w.D))
    vt = _values(w, gen.stream_key(s, TAG_VT), (w.B, w.Hkv, w.T, w.D))
    dt = np.float32 if w.dtype == "fp32" else np.uint16
    kc = np.empty((w.B, w.Hkv, cap, w.D), dtype=dt)
    vc = np.empty((w.B, w.Hkv, cap, w.D), dtype=dt)
    fill = poison_value(w) if poison else dt(0)
    for b in range(w.B):
        L = int(lens[b])
        kc[b].fill(fill)
        vc[b].fill(fill)
        if L:
            kc[b][:, lmax - L:lmax] = _values(w, gen.stream_key(s, TAG_KC, b), (w.Hkv, L, w.D))
            vc[b][:, lmax - L:lmax] = _values(w, gen.stream_key(s, TAG_VC, b), (w.Hkv, L, w.D))
    return q, kc, vc, kt, vt


def as_f32(w: Workload, x: np.ndarray) -> np.ndarray:
    """Exact float32 view of a generated tensor (bf16 bits are upcast)."""
    return x if w.dtype == "fp32" else gen.bf16_bits_to_f32(x)
