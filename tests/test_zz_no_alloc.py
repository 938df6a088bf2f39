"""svt_accept_noalloc (the accept call with the library's static scratch in
place of a caller workspace) against svt_accept on the same inputs, bit for
bit, on two calls in a row (the second with a smaller input, so it runs on
the scratch the first left behind), plus the size limit: a shape that needs
more than SVT_ACCEPT_NOALLOC_SCRATCH bytes of scratch is refused before
anything is launched, and one that needs exactly that much runs.  Results
are also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tree_masked_verification_parent_amd import svt

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(x):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=DEV)


def _case(B, M, V, seed):
    T = M + 1
    par = np.stack([gen.tree_depth_capped(gen.stream_key(seed, 1, b), M, 10) for b in range(B)]).astype(np.int32)
    logits, des = gen.logits_with_designated_top(gen.stream_key(seed, 2), B * T, V)
    des = des.reshape(B, T)
    tok = np.stack([gen.plant_drafts(gen.stream_key(seed, 3, b), par[b], des[b], V, 0.75)
                    for b in range(B)]).astype(np.int32)
    return par, logits.reshape(B, T, V), tok


class _Bufs:
    def __init__(self, par, logits, tok, M):
        B, T, V = logits.shape
        self.M = M
        self.lg = torch.as_tensor(logits, device=DEV)
        self.tk, self.pr = _i32(tok), _i32(par)
        W = (T + 63) // 64
        self.mk = torch.zeros(B, T, W, dtype=torch.int64, device=DEV)
        self.dp = torch.zeros(B, T, dtype=torch.int32, device=DEV)
        self.st = torch.zeros(B, dtype=torch.int32, device=DEV)
        assert svt.svt_build_mask(self.pr, M, self.mk, self.dp, self.st) == 0

    def outs(self):
        B, T = self.tk.shape
        return (torch.full((B, T), -1, dtype=torch.int32, device=DEV), torch.full((B,), -1, dtype=torch.int32, device=DEV),
                torch.full((B, T), -1, dtype=torch.int32, device=DEV), torch.full((B,), -1, dtype=torch.int32, device=DEV))

    def args(self, outs, workspace=None):
        return svt.accept_args(self.lg, self.tk, self.pr, self.mk, self.dp, *outs, status=self.st, workspace=workspace)


def _run_both(par, logits, tok, M):
    bufs = _Bufs(par, logits, tok, M)
    ref_out = bufs.outs()
    a = bufs.args(ref_out)
    need = svt.svt_accept_workspace(a)
    assert 0 < need <= svt.SVT_ACCEPT_NOALLOC_SCRATCH
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    assert svt.svt_accept(bufs.args(ref_out, ws)) == 0
    na_out = bufs.outs()
    assert svt.svt_accept_noalloc(bufs.args(na_out)) == 0
    torch.cuda.synchronize()
    for r, n in zip(ref_out, na_out):
        assert torch.equal(r, n)
    am = oracle.argmax(logits)
    _, ost = oracle.validate(par, M)
    al, path, bonus = oracle.accept(am, tok, par, M, ost)
    got = [t.cpu().numpy() for t in na_out]
    assert np.array_equal(got[0], am) and np.array_equal(got[1], al)
    assert np.array_equal(got[2], path) and np.array_equal(got[3], bonus)
    return need


def test_accept_noalloc_equals_accept_twice_second_smaller():
    print("noalloc call 1: B=32 M=32 V=32000", flush=True)
    n1 = _run_both(*_case(32, 32, 32000, 9600), 32)
    print("noalloc call 2: B=3 M=64 V=151552 (smaller)", flush=True)
    n2 = _run_both(*_case(3, 64, 151552, 9601), 64)
    print("noalloc call 3: B=2 M=8 V=1000 (smaller still)", flush=True)
    n3 = _run_both(*_case(2, 8, 1000, 9602), 8)
    assert n1 > n2 > n3


def test_accept_noalloc_size_limit():
    # V = 1: one chunk per row, so the scratch holds one 8-byte key per row;
    # 2048 trees of 256 rows fill the 4 MiB exactly, 2049 trees exceed it
    M, V = 255, 1
    for B, ok in [(2049, False), (2048, True)]:
        print(f"noalloc size limit B={B}", flush=True)
        T = M + 1
        par = np.stack([gen.tree_depth_capped(gen.stream_key(9700, b), M, 10) for b in range(B)]).astype(np.int32)
        logits = np.zeros((B, T, V), np.float32)
        tok = (gen.randint(gen.stream_key(9701), B * T, 0, 2).astype(np.int32) % 2).reshape(B, T)
        bufs = _Bufs(par, logits, tok, M)
        outs = bufs.outs()
        a = bufs.args(outs)
        need = svt.svt_accept_workspace(a)
        assert (need <= svt.SVT_ACCEPT_NOALLOC_SCRATCH) == ok, need
        rc = svt.svt_accept_noalloc(a)
        torch.cuda.synchronize()
        if not ok:
            assert rc == svt.SVT_ERR_WORKSPACE
            assert (outs[1] == -1).all()        # nothing was launched
            continue
        assert rc == 0
        am = oracle.argmax(logits)
        _, ost = oracle.validate(par, M)
        al, path, bonus = oracle.accept(am, tok, par, M, ost)
        assert np.array_equal(outs[0].cpu().numpy(), am) and np.array_equal(outs[1].cpu().numpy(), al)
        assert np.array_equal(outs[2].cpu().numpy(), path) and np.array_equal(outs[3].cpu().numpy(), bonus)
