"""Pins for the oracle's dense 4D tree mask and length-based commit.

The dense mask is pinned by a hand-worked tree, by invariants (open count per
row = prefix content + depth + 1), and by the library routine it exists for:
torch's scaled_dot_product_attention over [prefix cache columns, tree rows]
with the mask as its additive attn_mask reproduces the oracle's attention.
The length-based commit is pinned by a hand-worked case on the commit.json
initial state.  No GPU is needed."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import gen
from synth import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_dense_mask_hand_worked():
    # EAGLE-Pangu nl summary 2.C: k attends j only when j is an ancestor of k
    # (reflexive reading); the prefix content [lmax - len, lmax) is visible to
    # every node.  Tree: 1 <- 0, 2 <- 1, 3 <- 0; len 2, lmax 3.
    codes, op = oracle.expand_mask(np.array([[0, 0, 1, 0]], np.int32), [2], 3)
    want = [[0, 1, 1, 1, 0, 0, 0],
            [0, 1, 1, 1, 1, 0, 0],
            [0, 1, 1, 1, 1, 1, 0],
            [0, 1, 1, 1, 0, 0, 1]]
    assert codes.tolist() == [0] and op[0].astype(int).tolist() == want


def _trees(B, M, seed):
    return np.stack([gen.tree_depth_capped(gen.stream_key(seed, 3, b), M, 6) for b in range(B)]).astype(np.int32)


def test_dense_mask_invariants_and_codes():
    B, M, lmax = 4, 40, 30
    par = _trees(B, M, 41)
    lens = np.array([30, 0, 12, 31], np.int32)          # the last breaks len <= lmax
    st = np.array([0, 0, -5, 0], np.int32)
    codes, op = oracle.expand_mask(par, lens, lmax, st)
    assert codes.tolist() == [0, 0, -5, oracle.ERR_LENGTH]
    assert not op[2].any() and not op[3].any()
    _, ost = oracle.validate(par, M)
    mk, dp = oracle.mask(par, M, ost)
    for b in (0, 1):
        L = lens[b]
        assert not op[b, :, :lmax - L].any() and op[b, :, lmax - L:lmax].all()
        assert (op[b].sum(axis=1) == L + dp[b] + 1).all()
        for i in range(M + 1):                           # tree part = the ancestor bitmask
            bits = [(int(mk[b, i, j // 64]) >> (j % 64)) & 1 for j in range(M + 1)]
            assert op[b, i, lmax:].astype(int).tolist() == bits


@pytest.mark.parametrize("lens", [[20, 0, 7], [1, 1, 1]])
def test_dense_mask_drives_library_attention_to_the_oracle(lens):
    import dataclasses
    w = dataclasses.replace(wl.workload(0), B=3, Hq=4, Hkv=2, D=64, M=12)
    lens = np.asarray(lens, np.int32)
    lmax = int(lens.max())
    q, kc, vc, kt, vt = wl.attention_inputs(w, lens, lmax + 5, 4321, poison=False)
    par = wl.trees(w, 4321)
    _, st = oracle.validate(par, w.M)
    mk, _ = oracle.mask(par, w.M, st)
    rc, ref = oracle.attention(q, kc, vc, kt, vt, mk, lens, lmax, st)
    assert rc == 0
    _, op = oracle.expand_mask(par, lens, lmax, st)
    add = torch.from_numpy(np.where(op, 0.0, -np.inf))                  # [B][T][lmax + T]
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // w.G
            K = torch.from_numpy(np.concatenate([kc[b, g, :lmax], kt[b, g]]).astype(np.float64))
            V = torch.from_numpy(np.concatenate([vc[b, g, :lmax], vt[b, g]]).astype(np.float64))
            Q = torch.from_numpy(q[b, :, h].astype(np.float64))
            out = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=add[b][None],
                                                 scale=1.0 / np.sqrt(w.D))[0]
            assert np.abs(out.numpy() - ref[b, :, h]).max() < 1e-9, (b, h)


def test_length_based_commit_hand_worked():
    # EAGLE-Pangu nl summary 2.A, length-based mode: keep the prefix and append
    # the first A steps of the chosen branch (branch rows 0..A-1), then re-pad.
    with open(os.path.join(GOLDEN, "commit.json")) as f:
        ini = json.load(f)["initial"]
    cap = ini["cap"]
    km = np.zeros((1, 2, 2, 1, cap, 1), np.int32)
    km[0, 0, :, 0, :, 0] = ini["k_main"]
    km[0, 1, :, 0, :, 0] = ini["v_main"]
    kb = np.zeros((1, 2, 2, 1, 3, 1), np.int32)
    kb[0, 0, :, 0, :, 0] = ini["k_branch"]
    kb[0, 1, :, 0, :, 0] = ini["v_branch"]
    tm = np.array(ini["tokens_main"], np.int32)
    rc, km2, tm2, ln2, lm2, pos = oracle.commit(km, kb, ini["M"], tm, ini["tree_tokens"], ini["lens"], ini["lmax"],
                                                None, np.array([1, 0], np.int32))
    assert rc == 0 and ln2.tolist() == [5, 2] and lm2 == 5
    assert km2[0, 0, 0, 0, :5, 0].tolist() == [10, 11, 12, 30, 31]
    assert km2[0, 1, 1, 0, 3:5, 0].tolist() == [120, 140]
    assert tm2[0, :5].tolist() == [5, 6, 7, 50, 51] and tm2[1, 3:5].tolist() == [8, 60]
    assert pos[:, :5].tolist() == [[0, 1, 2, 3, 4], [0, 0, 0, 0, 1]]
    # append mode: nothing moves, rows at [lmax, lmax + A)
    rc, km3, *_ = oracle.commit(km, kb, ini["M"], tm, ini["tree_tokens"], ini["lens"], ini["lmax"], None,
                                np.array([1, 0], np.int32), mode=1)
    assert rc == 0 and km3[0, 0, 1, 0, :4, 0].tolist() == [99, 99, 20, 40]
