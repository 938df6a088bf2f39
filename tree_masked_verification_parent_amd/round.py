"""Device buffers for one verification round and the four library calls.

`VerifyRound` owns the GPU tensors of a batch (parents, draft tokens, logits,
Q, the layered main cache and branch cache, lengths) and runs
svt_build_mask -> svt_verify_attention (per layer) -> svt_accept ->
svt_commit on the current stream.  Tensors come from torch (memory and
streams only); all computation happens in libsvt.
"""
from __future__ import annotations

import torch

from . import svt


class VerifyRound:
    def __init__(self, B: int, M: int, Hq: int, Hkv: int, D: int, V: int, cap: int, n_layers: int,
                 dtype: torch.dtype, device="cuda", attn_layers: int | None = None, attn_split_keys: int = 0):
        """attn_split_keys > 0 (a multiple of 64) runs attention in the split form
        with splits of that many content keys, so that each sequence's output is
        bitwise independent of the rest of the batch; 0 lets the library choose."""
        self.B, self.M, self.T, self.Hq, self.Hkv, self.D, self.V = B, M, M + 1, Hq, Hkv, D, V
        self.attn_split_keys = int(attn_split_keys)
        self.cap, self.n_layers, self.dtype = cap, n_layers, dtype
        self.attn_layers = n_layers if attn_layers is None else attn_layers
        W = (self.T + 63) // 64
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        T = self.T
        self.parents = torch.zeros(B, T, **i32)
        self.tree_tokens = torch.zeros(B, T, **i32)
        self.mask = torch.zeros(B, T, W, dtype=torch.int64, device=dev)
        self.depth = torch.zeros(B, T, **i32)
        self.status = torch.zeros(B, **i32)
        self.seq_status = torch.zeros(B, **i32)
        self.logits = torch.zeros(B, T, V, dtype=torch.float32, device=dev)
        self.q = torch.zeros(self.attn_layers, B, T, Hq, D, dtype=dtype, device=dev)
        self.out = torch.zeros(self.attn_layers, B, T, Hq, D, dtype=dtype, device=dev)
        self.kv_main = torch.zeros(n_layers, 2, B, Hkv, cap, D, dtype=dtype, device=dev)
        self.kv_branch = torch.zeros(n_layers, 2, B, Hkv, T, D, dtype=dtype, device=dev)
        self.tokens_main = torch.zeros(B, cap, **i32)
        self.pos_ids = torch.zeros(B, cap, **i32)
        self.len = torch.zeros(B, **i32)
        self.lmax = torch.zeros(1, **i32)
        self.amax = torch.zeros(B, T, **i32)
        self.accept_len = torch.zeros(B, **i32)
        self.path = torch.zeros(B, T, **i32)
        self.bonus = torch.zeros(B, **i32)
        self.commit_status = torch.zeros(1, **i32)
        self.lmax_bound = 0
        acc = self._accept_args()
        self.accept_ws = torch.empty(max(1, svt.svt_accept_workspace(acc)), dtype=torch.uint8, device=dev)
        self._attn_ws = None
        # Argument structs are built once and reused: the tensors above are
        # filled in place, never rebound, so their pointers stay valid.  (Per
        # call, building them costs more host time than a short kernel takes.)
        self._attn_cache = {}
        self._accept_cache = None
        self._commit_cache = None

    # ---- argument structs -------------------------------------------------
    def _attn_args(self, layer: int):
        return svt.attn_args(self.q[layer], self.kv_main[layer, 0], self.kv_main[layer, 1], self.len, self.lmax,
                             self.lmax_bound, self.kv_branch[layer, 0], self.kv_branch[layer, 1], self.mask,
                             self.out[layer], status=self.status, seq_status=self.seq_status,
                             workspace=self._attn_ws, split_keys=self.attn_split_keys)

    def _accept_args(self):
        return svt.accept_args(self.logits, self.tree_tokens, self.parents, self.mask, self.depth, self.amax,
                               self.accept_len, self.path, self.bonus, status=self.status,
                               workspace=getattr(self, "accept_ws", None))

    def _commit_args(self):
        return svt.commit_args(self.kv_main, self.kv_branch, self.len, self.lmax, self.path, self.accept_len,
                               self.commit_status, tokens_main=self.tokens_main, tree_tokens=self.tree_tokens,
                               pos_ids=self.pos_ids, status=self.status)

    def set_lmax_bound(self, bound: int):
        """Host upper bound of the batch length; sizes the attention grid."""
        self.lmax_bound = int(bound)
        self._attn_cache = {}
        need = svt.svt_verify_attention_workspace(self._attn_args(0))
        if need and (self._attn_ws is None or self._attn_ws.numel() < need):
            self._attn_ws = torch.empty(need, dtype=torch.uint8, device=self.q.device)
        self._attn_cache = {}

    # ---- the four calls -----------------------------------------------------
    def build_mask(self, flags: int = 0) -> int:
        return svt.svt_build_mask(self.parents, self.M, self.mask, self.depth, self.status, flags)

    def attention(self, layer: int = 0) -> int:
        a = self._attn_cache.get(layer)
        if a is None:
            a = self._attn_cache[layer] = self._attn_args(layer)
        return svt.svt_verify_attention(a)

    def accept(self) -> int:
        if self._accept_cache is None:
            self._accept_cache = self._accept_args()
        return svt.svt_accept(self._accept_cache)

    def commit(self, flags: int = 0) -> int:
        if self._commit_cache is None:
            self._commit_cache = self._commit_args()
        return svt.svt_commit(self._commit_cache, flags)

    def step(self) -> int:
        """One full round: mask, attention over every attention layer, accept, commit."""
        rc = self.build_mask()
        for layer in range(self.attn_layers):
            rc = rc or self.attention(layer)
        rc = rc or self.accept()
        rc = rc or self.commit()
        return rc
