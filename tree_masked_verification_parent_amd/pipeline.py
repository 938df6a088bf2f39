"""Multi-layer round skeleton: the commit of one round overlapped, layer by
layer, with the attention of the next.

EAGLE-Pangu (gist.science ko summary, section 2; nl summary, section 2.C)
verifies all speculative tokens of a round in one batched teacher forward
over every layer.  Layer l of round k + 1 only needs layer l of round k
committed, so the commit's cache moves for layers l + 1, l + 2, ... (one
stream) can run while the attention of layer l of the next round runs (the
other stream).  The teacher's projections between the layers need trained
weights and are not part of this skeleton: each layer's queries and branch
keys/values are given.

Layout: the main cache, token rows, position ids and the lengths are shared;
everything a round produces or reads once (tree, drafts, logits, queries,
branch KV, mask, accept results) lives in one of two buffer sets, used by
rounds of alternating parity, and the lengths ping-pong between two arrays
(round k reads lens[k % 2]; its commit writes lens[(k + 1) % 2] through the
commit's len_out / lmax_out, so the per-layer commit calls all read unchanged
lengths).  Every step runs in libsvt; torch allocates, orders streams and
captures graphs.
"""
from __future__ import annotations

import torch

from . import svt


class _RoundSet:
    def __init__(self, B, M, Hq, Hkv, D, V, L, dtype, dev):
        T, W = M + 1, (M + 64) // 64
        i32 = dict(dtype=torch.int32, device=dev)
        self.parents = torch.zeros(B, T, **i32)
        self.tree_tokens = torch.zeros(B, T, **i32)
        self.logits = torch.zeros(B, T, V, dtype=torch.float32, device=dev)
        self.q = torch.zeros(L, B, T, Hq, D, dtype=dtype, device=dev)
        self.out = torch.zeros(L, B, T, Hq, D, dtype=dtype, device=dev)
        self.kv_branch = torch.zeros(L, 2, B, Hkv, T, D, dtype=dtype, device=dev)
        self.mask = torch.zeros(B, T, W, dtype=torch.int64, device=dev)
        self.depth = torch.zeros(B, T, **i32)
        self.status = torch.zeros(B, **i32)
        self.seq_status = torch.zeros(B, **i32)
        self.amax = torch.zeros(B, T, **i32)
        self.accept_len = torch.zeros(B, **i32)
        self.path = torch.zeros(B, T, **i32)
        self.bonus = torch.zeros(B, **i32)


class RoundPipeline:
    def __init__(self, B: int, M: int, Hq: int, Hkv: int, D: int, V: int, cap: int, n_layers: int,
                 dtype: torch.dtype, device="cuda", attn_form: int = svt.SVT_ATTN_AUTO):
        dev = torch.device(device)
        self._args = {}
        self._attn_form = attn_form
        self.B, self.M, self.T, self.L, self.cap = B, M, M + 1, n_layers, cap
        i32 = dict(dtype=torch.int32, device=dev)
        self.kv_main = torch.zeros(n_layers, 2, B, Hkv, cap, D, dtype=dtype, device=dev)
        self.tokens_main = torch.zeros(B, cap, **i32)
        self.pos_ids = torch.zeros(B, cap, **i32)
        self.lens = [torch.zeros(B, **i32), torch.zeros(B, **i32)]
        self.lmax = [torch.zeros(1, **i32), torch.zeros(1, **i32)]
        self.commit_status = torch.zeros(1, **i32)
        self._scratch_len = torch.zeros(B, **i32)       # per-layer calls write their (equal) results here
        self._scratch_lmax = torch.zeros(1, **i32)
        self._scratch_status = torch.zeros(1, **i32)
        self.sets = [_RoundSet(B, M, Hq, Hkv, D, V, n_layers, dtype, dev) for _ in range(2)]
        self.lmax_bound = 0
        self.side = torch.cuda.Stream(device=dev)       # default priority
        self._layer_done = [torch.cuda.Event() for _ in range(n_layers)]
        acc = self._accept_args(self.sets[0])
        self.accept_ws = torch.empty(max(1, svt.svt_accept_workspace(acc)), dtype=torch.uint8, device=dev)
        self.attn_ws = torch.empty(1, dtype=torch.uint8, device=dev)
        self._args = {}  # argument structs by (call, round parity[, layer]): built once, reused

    # ---- argument structs ---------------------------------------------------
    @property
    def attn_form(self) -> int:
        return self._attn_form

    @attn_form.setter
    def attn_form(self, form: int):
        self._attn_form = form
        self._args = {}  # the cached attention structs carry the form

    def _cached(self, key, make):
        a = self._args.get(key)
        if a is None:
            a = self._args[key] = make()
        return a

    def _attn_args(self, s: _RoundSet, k: int, layer: int, ws=None):
        return svt.attn_args(s.q[layer], self.kv_main[layer, 0], self.kv_main[layer, 1], self.lens[k % 2],
                             self.lmax[k % 2], self.lmax_bound, s.kv_branch[layer, 0], s.kv_branch[layer, 1],
                             s.mask, s.out[layer], status=s.status, seq_status=s.seq_status, workspace=ws,
                             form=self.attn_form)

    def _accept_args(self, s: _RoundSet):
        return svt.accept_args(s.logits, s.tree_tokens, s.parents, s.mask, s.depth, s.amax, s.accept_len, s.path,
                               s.bonus, status=s.status, workspace=getattr(self, "accept_ws", None))

    def _commit_args(self, s: _RoundSet, k: int, layer=None):
        """Commit of round k: all layers and the token rows (layer None), or
        one layer's cache only (results to scratch)."""
        src, dst = k % 2, (k + 1) % 2
        if layer is None:
            return svt.commit_args(self.kv_main, s.kv_branch, self.lens[src], self.lmax[src], s.path, s.accept_len,
                                   self.commit_status, tokens_main=self.tokens_main, tree_tokens=s.tree_tokens,
                                   pos_ids=self.pos_ids, status=s.status, len_out=self.lens[dst],
                                   lmax_out=self.lmax[dst])
        if layer < 0:   # token rows and lengths only (no cache layer)
            return svt.commit_args(self.kv_main[:0], s.kv_branch[:0], self.lens[src], self.lmax[src], s.path,
                                   s.accept_len, self.commit_status, tokens_main=self.tokens_main,
                                   tree_tokens=s.tree_tokens, pos_ids=self.pos_ids, status=s.status,
                                   len_out=self.lens[dst], lmax_out=self.lmax[dst])
        return svt.commit_args(self.kv_main[layer:layer + 1], s.kv_branch[layer:layer + 1], self.lens[src],
                               self.lmax[src], s.path, s.accept_len, self._scratch_status, status=s.status,
                               len_out=self._scratch_len, lmax_out=self._scratch_lmax)

    def set_lmax_bound(self, bound: int):
        self.lmax_bound = int(bound)
        need = svt.svt_verify_attention_workspace(self._attn_args(self.sets[0], 0, 0))
        if need > self.attn_ws.numel():
            self.attn_ws = torch.empty(need, dtype=torch.uint8, device=self.kv_main.device)
        self._args = {}

    # ---- rounds -----------------------------------------------------------------
    def verify(self, k: int, stream=None) -> int:
        """Mask, attention over every layer and accept of round k (buffer set k % 2)."""
        s = self.sets[k % 2]
        rc = svt.svt_build_mask(s.parents, self.M, s.mask, s.depth, s.status, 0, stream)
        for layer in range(self.L):
            rc = rc or svt.svt_verify_attention(self._attn(s, k, layer), stream)
        return rc or svt.svt_accept(self._cached(("accept", k % 2), lambda: self._accept_args(s)), stream)

    def _attn(self, s, k, layer):
        return self._cached(("attn", k % 2, layer), lambda: self._attn_args(s, k, layer, self.attn_ws))

    def _commit(self, s, k, layer=None):
        return self._cached(("commit", k % 2, layer), lambda: self._commit_args(s, k, layer))

    def commit(self, k: int, stream=None) -> int:
        """The whole commit of round k in one call."""
        return svt.svt_commit(self._commit(self.sets[k % 2], k), 0, stream)

    def sequential_step(self, k: int) -> int:
        """Round k in order on the current stream: verify, then commit."""
        return self.verify(k) or self.commit(k)

    def pipelined_step(self, k: int) -> int:
        """Commit of round k - 1 overlapped with round k: the token rows and the
        new lengths first (current stream), the cache layers one by one on the
        side stream, and the attention of layer l of round k once layer l is
        committed.  Round 0 has nothing to commit before it."""
        main = torch.cuda.current_stream()
        rc = 0
        if k > 0:
            prev = self.sets[(k - 1) % 2]
            rc = svt.svt_commit(self._commit(prev, k - 1, -1), 0, main)
            self.side.wait_stream(main)
            for layer in range(self.L):
                rc = rc or svt.svt_commit(self._commit(prev, k - 1, layer), 0, self.side)
                self._layer_done[layer].record(self.side)
        s = self.sets[k % 2]
        rc = rc or svt.svt_build_mask(s.parents, self.M, s.mask, s.depth, s.status, 0, main)
        for layer in range(self.L):
            if k > 0:
                main.wait_event(self._layer_done[layer])
            rc = rc or svt.svt_verify_attention(self._attn(s, k, layer), main)
        rc = rc or svt.svt_accept(self._cached(("accept", k % 2), lambda: self._accept_args(s)), main)
        if k > 0:
            main.wait_stream(self.side)
        return rc

    def capture(self, k: int) -> torch.cuda.CUDAGraph:
        """HIP graph of pipelined_step(k) (k >= 1); replaying it runs the step for
        every round of the same parity as k."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rc = self.pipelined_step(k)
        if rc != 0:
            raise RuntimeError(f"capture of a pipelined step failed: {svt.status_string(rc)}")
        return g
