"""Cross-batch scheduling over a pool of sequences.

Batch Speculative Decoding Done Right (gist.science ko summary, section 2
Methodology) gives two ways to keep a batch of speculative sequences
consistent after each verification round:

- EQSPEC: a fixed batch; after every round each sequence appends what it
  accepted and the batch is re-padded so that padding plus content equals the
  batch maximum for every sequence (svt_commit, SVT_COMMIT_REPAD).  Sequences
  whose padding changes move in the cache: the realignment overhead.
- EXSPEC: a pool of sequences; each round the scheduler groups sequences of
  equal length, whose batch needs no realignment (svt_commit,
  SVT_COMMIT_APPEND: only the accepted rows are written), and falls back to
  EQSPEC's alignment (svt_realign, then a re-pad commit) when no group is
  large enough.

`SequencePool` holds the pool's cache, token and position rows on the device
and each sequence's length and end column on the host; the batch choice is
svt_pool_pick.  `PoolRound` runs one round (mask, attention over every
layer, accept, commit) for a batch of pool slots through the slot map of the
library calls.  Every step runs in libsvt; torch only allocates.
"""
from __future__ import annotations

import numpy as np
import torch

from . import svt


class SequencePool:
    """`n_slots` sequences of an `n_layers`-layer cache [layers][2][slots][Hkv][cap][D].

    Sequence s occupies columns [end[s] - len[s], end[s]) of its row."""

    def __init__(self, n_slots: int, Hkv: int, D: int, n_layers: int, cap: int, dtype: torch.dtype,
                 device="cuda"):
        dev = torch.device(device)
        self.n_slots, self.Hkv, self.D, self.n_layers, self.cap = n_slots, Hkv, D, n_layers, cap
        self.kv = torch.empty(n_layers, 2, n_slots, Hkv, cap, D, dtype=dtype, device=dev)
        self.tokens = torch.zeros(n_slots, cap, dtype=torch.int32, device=dev)
        self.pos = torch.zeros(n_slots, cap, dtype=torch.int32, device=dev)
        self.len = np.zeros(n_slots, np.int32)
        self.end = np.zeros(n_slots, np.int32)
        self.active = np.zeros(n_slots, np.int32)
        self._lmax = torch.zeros(1, dtype=torch.int32, device=dev)
        self._status = torch.zeros(1, dtype=torch.int32, device=dev)

    def place(self, slot: int, length: int, end: int | None = None):
        """Record that sequence `slot` holds `length` rows ending at `end`
        (default: no padding, end = length)."""
        self.len[slot] = length
        self.end[slot] = length if end is None else end
        self.active[slot] = 1

    def pick(self, max_batch: int, min_group: int):
        """(equal_ends, slots) of the next batch (svt_pool_pick)."""
        rc, slots = svt.svt_pool_pick(self.end, self.active, max_batch, min_group)
        if rc < 0:
            raise RuntimeError(f"svt_pool_pick failed: {svt.status_string(rc)}")
        return rc == 1, slots

    def realign(self, slots: np.ndarray, slot_t: torch.Tensor, len_t: torch.Tensor, end_t: torch.Tensor) -> int:
        """Moves the batch's sequences to a common end (the largest); returns it.
        slot_t / len_t / end_t: device copies of slots, len[slots], end[slots]."""
        a = svt.realign_args(self.kv, len_t, end_t, self._lmax, self._status, tokens_main=self.tokens,
                             pos_ids=self.pos, seq_slot=slot_t)
        rc = svt.svt_realign(a)
        if rc != svt.SVT_OK:
            raise RuntimeError(f"svt_realign failed: {svt.status_string(rc)}")
        e = int(self.end[slots].max()) if len(slots) else 0
        self.end[slots] = e
        return e

    def committed(self, slots: np.ndarray, accept_len: np.ndarray, lmax_before: int, mode: int):
        """Host bookkeeping after a commit of the batch `slots` (lengths grow by
        accept_len + 1; ends follow the commit mode)."""
        A = accept_len.astype(np.int32) + 1
        self.len[slots] += A
        if mode == svt.SVT_COMMIT_APPEND:
            self.end[slots] = lmax_before + A
        else:
            self.end[slots] = int(self.len[slots].max()) if len(slots) else 0


class PoolRound:
    """Per-batch device buffers (up to `max_batch` sequences) and one round of
    the four calls on a batch of pool slots."""

    def __init__(self, pool: SequencePool, max_batch: int, M: int, Hq: int, V: int, attn_layers: int,
                 device="cuda"):
        dev = torch.device(device)
        self.pool, self.B, self.M, self.T, self.Hq, self.V = pool, max_batch, M, M + 1, Hq, V
        self.attn_layers = attn_layers
        T, B, D, Hkv, L = self.T, max_batch, pool.D, pool.Hkv, pool.n_layers
        W = (T + 63) // 64
        i32 = dict(dtype=torch.int32, device=dev)
        dt = pool.kv.dtype
        self.parents = torch.zeros(B, T, **i32)
        self.tree_tokens = torch.zeros(B, T, **i32)
        self.logits = torch.zeros(B, T, V, dtype=torch.float32, device=dev)
        self.mask = torch.zeros(B, T, W, dtype=torch.int64, device=dev)
        self.depth = torch.zeros(B, T, **i32)
        self.status = torch.zeros(B, **i32)
        self.seq_status = torch.zeros(B, **i32)
        self.q = torch.zeros(attn_layers, B, T, Hq, D, dtype=dt, device=dev)
        self.out = torch.zeros(attn_layers, B, T, Hq, D, dtype=dt, device=dev)
        self._kvb = torch.zeros(L * 2 * B * Hkv * T * D, dtype=dt, device=dev)
        self.amax = torch.zeros(B, T, **i32)
        self.accept_len = torch.zeros(B, **i32)
        self.path = torch.zeros(B, T, **i32)
        self.bonus = torch.zeros(B, **i32)
        self.commit_status = torch.zeros(1, **i32)
        self.slot = torch.zeros(B, **i32)
        self.len = torch.zeros(B, **i32)
        self.end = torch.zeros(B, **i32)
        self.lmax = torch.zeros(1, **i32)
        # the accept workspace of a smaller batch can be larger (more chunks per
        # row keep the chip busy): size it for every batch size up to B
        need = max(svt.svt_accept_workspace(self._accept_args(n)) for n in range(1, B + 1))
        self.accept_ws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
        self._attn_ws = torch.empty(1, dtype=torch.uint8, device=dev)

    def kv_branch(self, n: int) -> torch.Tensor:
        p = self.pool
        return self._kvb[: p.n_layers * 2 * n * p.Hkv * self.T * p.D].view(p.n_layers, 2, n, p.Hkv, self.T, p.D)

    def _attn_args(self, n: int, layer: int, bound: int, ws=None):
        p, kvb = self.pool, self.kv_branch(n)
        return svt.attn_args(self.q[layer, :n], p.kv[layer, 0], p.kv[layer, 1], self.len[:n], self.lmax, bound,
                             kvb[layer, 0], kvb[layer, 1], self.mask[:n], self.out[layer, :n],
                             status=self.status[:n], seq_status=self.seq_status[:n], workspace=ws,
                             seq_slot=self.slot[:n])

    def _accept_args(self, n: int):
        return svt.accept_args(self.logits[:n], self.tree_tokens[:n], self.parents[:n], self.mask[:n],
                               self.depth[:n], self.amax[:n], self.accept_len[:n], self.path[:n], self.bonus[:n],
                               status=self.status[:n], workspace=getattr(self, "accept_ws", None))

    def _commit_args(self, n: int, mode: int):
        p = self.pool
        return svt.commit_args(p.kv, self.kv_branch(n), self.len[:n], self.lmax, self.path[:n],
                               self.accept_len[:n], self.commit_status, tokens_main=p.tokens,
                               tree_tokens=self.tree_tokens[:n], pos_ids=p.pos, status=self.status[:n],
                               seq_slot=self.slot[:n], mode=mode)

    def load_batch(self, slots: np.ndarray):
        """Copies the batch's slot map, lengths and ends to the device."""
        n = len(slots)
        self.slot[:n].copy_(torch.from_numpy(np.ascontiguousarray(slots, np.int32)))
        self.len[:n].copy_(torch.from_numpy(self.pool.len[slots]))
        self.end[:n].copy_(torch.from_numpy(self.pool.end[slots]))

    def verify(self, n: int, lmax: int) -> int:
        """Mask, attention over every layer and accept for the first n batch rows;
        the batch's content ends at column lmax."""
        self.lmax.fill_(lmax)
        need = svt.svt_verify_attention_workspace(self._attn_args(n, 0, lmax))
        if need > self._attn_ws.numel():
            self._attn_ws = torch.empty(need, dtype=torch.uint8, device=self.q.device)
        rc = svt.svt_build_mask(self.parents[:n], self.M, self.mask[:n], self.depth[:n], self.status[:n])
        for layer in range(self.attn_layers):
            rc = rc or svt.svt_verify_attention(self._attn_args(n, layer, lmax, self._attn_ws))
        return rc or svt.svt_accept(self._accept_args(n))

    def commit(self, n: int, mode: int) -> int:
        return svt.svt_commit(self._commit_args(n, mode))
