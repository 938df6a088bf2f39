"""Pins for the append-only commit, the realignment and the slot map of the
oracle (cross-batch scheduling), and checks of the host pool picker.

Oracle pins: hand-worked fixtures (tests/golden/commit_append.json,
tests/golden/realign.json), the identity of append and re-pad when every
sequence accepts the same count (their layouts coincide by definition), the
slot map against an explicit gather / scatter, and invariants.  No GPU is
needed."""
import json
import os

import numpy as np
import pytest

import oracle
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _check_rows(got, want, label):
    for b, row in enumerate(want):
        for c, v in enumerate(row):
            if v is not None:
                assert got[b, c] == v, (label, b, c)


def test_golden_commit_append():
    g = _load("commit_append.json")
    ini = g["initial"]
    for case in g["cases"]:
        cap = case.get("cap_override", ini["cap"])
        km = np.zeros((1, 2, 2, 1, cap, 1), np.int32)
        km[0, 0, :, 0, :, 0] = np.array(ini["k_main"])[:, :cap]
        km[0, 1, :, 0, :, 0] = np.array(ini["v_main"])[:, :cap]
        kb = np.zeros((1, 2, 2, 1, 3, 1), np.int32)
        kb[0, 0, :, 0, :, 0] = ini["k_branch"]
        kb[0, 1, :, 0, :, 0] = ini["v_branch"]
        tm = np.array(ini["tokens_main"], np.int32)[:, :cap]
        rc, km2, tm2, ln2, lm2, pos = oracle.commit(km, kb, ini["M"], tm, ini["tree_tokens"], ini["lens"],
                                                    ini["lmax"], case["path"], case["accept_len"], mode=1)
        assert rc == case["rc"], case["name"]
        if rc:
            assert np.array_equal(km2, km) and np.array_equal(tm2, tm) and ln2.tolist() == ini["lens"]
            continue
        assert ln2.tolist() == case["lens"] and lm2 == case["lmax"], case["name"]
        _check_rows(km2[0, 0, :, 0, :, 0], case["k_main"], "k")
        _check_rows(km2[0, 1, :, 0, :, 0], case["v_main"], "v")
        _check_rows(tm2, case["tokens_main"], "tokens")
        for b, e in enumerate(case["ends"]):
            assert pos[b, :e].tolist() == case["pos_ids"][b], (case["name"], b)


def test_golden_realign():
    g = _load("realign.json")
    ini = g["initial"]
    cap = ini["cap"]
    km = np.zeros((1, 2, 3, 1, cap, 1), np.int32)
    km[0, 0, :, 0, :, 0] = ini["k_main"]
    km[0, 1, :, 0, :, 0] = ini["v_main"]
    tm = np.array(ini["tokens_main"], np.int32)
    for case in g["cases"]:
        ends = case.get("ends_override", ini["ends"])
        rc, km2, tm2, lm, pos = oracle.realign(km, ini["lens"], ends, tokens_main=tm)
        assert rc == case["rc"], case["name"]
        if rc:
            assert np.array_equal(km2, km) and np.array_equal(tm2, tm)
            continue
        assert lm == case["lmax"]
        _check_rows(km2[0, 0, :, 0, :, 0], case["k_main"], "k")
        _check_rows(km2[0, 1, :, 0, :, 0], case["v_main"], "v")
        _check_rows(tm2, case["tokens_main"], "tokens")
        assert pos[:, :lm].tolist() == case["pos_ids"]


def _random_trees(B, M, seed):
    out = np.zeros((B, M + 1), np.int32)
    for b in range(B):
        out[b] = gen.tree_depth_capped(gen.stream_key(seed, 77, b), M, 6)
    return out


def _case(B, rows, Hkv, L, M, lens, cap, seed, el=3):
    T = M + 1
    lens = np.asarray(lens, np.int32)
    slab = np.arange(L * 2 * rows * Hkv).reshape(L, 2, rows, Hkv, 1, 1)
    km = gen.commit_pattern_bits(slab, np.arange(cap).reshape(1, 1, 1, 1, cap, 1), np.arange(el).reshape(1, 1, 1, 1, 1, el))
    bsl = np.arange(L * 2 * B * Hkv).reshape(L, 2, B, Hkv, 1, 1) + 9000
    kb = gen.commit_pattern_bits(bsl, np.arange(T).reshape(1, 1, 1, 1, T, 1), np.arange(el).reshape(1, 1, 1, 1, 1, el))
    trees = _random_trees(B, M, seed)
    amax = gen.randint(gen.stream_key(seed, 1), B * T, 0, 2).astype(np.int32).reshape(B, T)
    tok = gen.randint(gen.stream_key(seed, 2), B * T, 0, 2).astype(np.int32).reshape(B, T)
    al, path, _ = oracle.accept(amax, tok, trees, M)
    tm = gen.randint(gen.stream_key(seed, 3), rows * cap, 0, 1000).astype(np.int32).reshape(rows, cap)
    return km, kb, tm, tok, lens, path, al


def test_append_equals_repad_when_counts_equal():
    B, Hkv, L, M, cap = 4, 2, 2, 6, 30
    km, kb, tm, tok, lens, path, _ = _case(B, B, Hkv, L, M, [9, 4, 0, 12], cap, 31)
    lmax = 12
    al = np.full(B, 3, np.int32)
    chain = np.tile(np.arange(M + 1, dtype=np.int32), (B, 1))
    r1 = oracle.commit(km, kb, M, tm, tok, lens, lmax, chain, al, mode=0)
    r2 = oracle.commit(km, kb, M, tm, tok, lens, lmax, chain, al, mode=1)
    assert r1[0] == r2[0] == 0
    for x, y in zip(r1[1:], r2[1:]):
        assert np.array_equal(np.asarray(x), np.asarray(y))


def test_append_moves_nothing():
    B, Hkv, L, M, cap = 5, 1, 2, 8, 40
    km, kb, tm, tok, lens, path, al = _case(B, B, Hkv, L, M, [17, 3, 0, 25, 9], cap, 33)
    lmax = 25
    rc, km2, tm2, ln2, lm2, pos = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al, mode=1)
    assert rc == 0
    A = al + 1
    assert lm2 == lmax + A.max() and (ln2 == lens + A).all()
    assert np.array_equal(km2[..., :lmax, :], km[..., :lmax, :])             # nothing before lmax changes
    assert np.array_equal(tm2[:, :lmax], tm[:, :lmax])
    for b in range(B):
        e = lmax + A[b]
        assert np.array_equal(km2[:, :, b, :, lmax:e], kb[:, :, b][:, :, :, path[b, :A[b]]])
        assert np.array_equal(km2[:, :, b, :, e:], km[:, :, b, :, e:])       # past the new end untouched
        start = lmax - lens[b]
        assert pos[b, start:e].tolist() == list(range(ln2[b])) and not pos[b, :start].any()


@pytest.mark.parametrize("mode", [0, 1])
def test_slot_map_equals_gather_scatter(mode):
    B, rows, Hkv, L, M, cap = 3, 6, 2, 2, 5, 24
    km, kb, tm, tok, lens, path, al = _case(B, rows, Hkv, L, M, [7, 2, 11], cap, 35)
    lmax = 11
    slot = np.array([4, 0, 2], np.int32)
    rc, km2, tm2, ln2, lm2, pos = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al, mode=mode, slot=slot)
    rcg, kg, tg, lg, mg, pg = oracle.commit(km[:, :, slot], kb, M, tm[slot], tok, lens, lmax, path, al, mode=mode)
    assert rc == rcg == 0 and lm2 == mg and np.array_equal(ln2, lg)
    assert np.array_equal(km2[:, :, slot], kg) and np.array_equal(tm2[slot], tg) and np.array_equal(pos[slot], pg)
    other = [r for r in range(rows) if r not in slot]
    assert np.array_equal(km2[:, :, other], km[:, :, other]) and np.array_equal(tm2[other], tm[other])
    assert not pos[other].any()
    bad = np.array([4, 6, 2], np.int32)
    rc, km3, *_ = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al, mode=mode, slot=bad)
    assert rc == oracle.ERR_ARG and np.array_equal(km3, km)
    # a pool row named by two sequences of the batch: refused, nothing written
    for dup in ([4, 0, 4], [2, 2, 0]):
        rc, km4, tm4, ln4, lm4, _ = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al, mode=mode,
                                                  slot=np.array(dup, np.int32))
        assert rc == oracle.ERR_ARG and np.array_equal(km4, km) and np.array_equal(tm4, tm)
        assert np.array_equal(ln4, lens) and lm4 == lmax


def test_realign_identity_rectangle_and_slots():
    rows, Hkv, L, cap = 5, 2, 2, 20
    km, _, tm, _, _, _, _ = _case(1, rows, Hkv, L, 1, [1], cap, 37)
    lens = np.array([3, 7, 0, 5], np.int32)
    slot = np.array([1, 4, 0, 3], np.int32)
    # already aligned: nothing changes
    rc, k1, t1, lm, pos = oracle.realign(km, lens, [9, 9, 9, 9], tokens_main=tm, slot=slot)
    assert rc == 0 and lm == 9 and np.array_equal(k1, km) and np.array_equal(t1, tm)
    # mixed ends: every content ends at the largest end, in order
    ends = np.array([3, 12, 4, 8], np.int32)
    rc, k2, t2, lm, pos = oracle.realign(km, lens, ends, tokens_main=tm, slot=slot)
    assert rc == 0 and lm == 12
    for b, r in enumerate(slot):
        assert np.array_equal(k2[:, :, r, :, 12 - lens[b]:12], km[:, :, r, :, ends[b] - lens[b]:ends[b]])
        assert np.array_equal(t2[r, 12 - lens[b]:12], tm[r, ends[b] - lens[b]:ends[b]])
        assert pos[r, 12 - lens[b]:12].tolist() == list(range(lens[b])) and not pos[r, :12 - lens[b]].any()
        assert np.array_equal(k2[:, :, r, :, 12:], km[:, :, r, :, 12:])
    assert np.array_equal(k2[:, :, 2], km[:, :, 2])                         # row not in the batch
    rc, k3, *_ = oracle.realign(km, lens, ends, slot=np.array([1, 4, 5, 3], np.int32))
    assert rc == oracle.ERR_ARG and np.array_equal(k3, km)
    rc, k4, *_ = oracle.realign(km, lens, ends, slot=np.array([1, 4, 1, 3], np.int32))   # row 1 twice
    assert rc == oracle.ERR_ARG and np.array_equal(k4, km)
    rc, *_ = oracle.realign(km, np.array([-1, 7, 0, 5], np.int32), ends, slot=slot)
    assert rc == oracle.ERR_LENGTH
