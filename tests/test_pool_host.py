"""Host pool picker of cross-batch scheduling (svt_pool_pick, library host
code): hand-worked pools, the documented rule on random pools, argument
errors, and a short run of equal-length rounds on the oracle showing that a
pool stored without padding never needs realignment.  No GPU is needed."""
import numpy as np
import pytest

import oracle
from tree_masked_verification_parent_amd import svt
from test_oracle_pool import _case


def test_exspec_rounds_keep_zero_padding():
    """A pool stored without padding, batched by equal length and committed
    with append, never realigns: every content keeps starting at column 0."""
    rows, Hkv, L, M, cap = 6, 1, 1, 4, 40
    km, kb1, tm, _, _, _, _ = _case(1, rows, Hkv, L, M, [1], cap, 39)
    lens = np.array([6, 6, 9, 6, 9, 4], np.int32)
    for rnd in range(4):
        rc, pick = svt.svt_pool_pick(lens, np.ones(rows, np.int32), 8, 2)
        assert rc == 1
        B = len(pick)
        _, kb, _, tok, _, path, al = _case(B, rows, Hkv, L, M, [1] * B, cap, 40 + rnd)
        lm = int(lens[pick[0]])
        rc, km, tm, ln2, lm2, pos = oracle.commit(km, kb, M, tm, tok, lens[pick], lm, path, al, mode=1, slot=pick)
        assert rc == 0
        for b, r in enumerate(pick):
            assert pos[r, :ln2[b]].tolist() == list(range(ln2[b]))          # starts at 0: no padding
        lens[pick] = ln2


# ---------------------------------------------------------------- host pool picker
@pytest.mark.parametrize("ends,active,mb,mg,rc,want", [
    ([5, 5, 3, 5, 3, 9], [1] * 6, 4, 2, 1, [0, 1, 3]),
    ([5, 5, 3, 5, 3, 9], [1] * 6, 4, 4, 0, [0, 1, 2, 3]),
    ([5, 5, 3, 5, 3, 9], [1] * 6, 2, 4, 1, [0, 1]),
    ([4, 4, 7, 7], [1] * 4, 8, 1, 1, [0, 1]),
    ([1, 1, 1, 2], [1, 0, 1, 1], 3, 2, 1, [0, 2]),
    ([8, 2, 5], [1, 1, 1], 3, 2, 0, [0, 1, 2]),
    ([3, 3], [0, 0], 4, 1, 1, []),
])
def test_pool_pick_examples(ends, active, mb, mg, rc, want):
    got_rc, got = svt.svt_pool_pick(np.array(ends), np.array(active), mb, mg)
    assert got_rc == rc and got.tolist() == want


def test_pool_pick_rule_on_random_pools():
    rng = np.random.default_rng(7)
    for _ in range(300):
        n = int(rng.integers(1, 40))
        ends = rng.integers(0, 6, n).astype(np.int32)
        act = (rng.random(n) < 0.8).astype(np.int32)
        mb, mg = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        rc, pick = svt.svt_pool_pick(ends, act, mb, mg)
        live = np.flatnonzero(act)
        if len(live) == 0:
            assert rc == 1 and len(pick) == 0
            continue
        assert list(pick) == sorted(set(pick.tolist())) and all(act[p] for p in pick)
        assert len(pick) == min(len(live), mb) or rc == 1
        vals, counts = np.unique(ends[live], return_counts=True)
        e0 = vals[np.argmax(counts)]                                  # first max = smallest end
        group = [s for s in live if ends[s] == e0]
        assert rc == (1 if len(set(ends[pick].tolist())) == 1 else 0)
        if len(group) >= min(mb, mg):
            assert pick.tolist() == group[:mb]
        else:
            assert set(group) <= set(pick.tolist()) and len(pick) == min(len(live), mb)
            far = max(abs(int(ends[p]) - int(e0)) for p in pick)
            for s in live:
                if s not in pick:
                    assert abs(int(ends[s]) - int(e0)) >= far


def test_pool_pick_argument_errors():
    e, a = np.array([1, 2], np.int32), np.array([1, 1], np.int32)
    assert svt.svt_pool_pick(e, a, 0, 1)[0] == svt.SVT_ERR_ARG
    assert svt.svt_pool_pick(e, a, 2, 0)[0] == svt.SVT_ERR_ARG
