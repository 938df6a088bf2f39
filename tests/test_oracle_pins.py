"""Pins for the CPU oracle, checked against things other than the oracle itself:
hand-worked fixtures (tests/golden), library routines that the method reduces
to in special cases (torch scaled_dot_product_attention, numpy argmax), brute
force on tiny inputs, closed forms and invariants.  No GPU is needed."""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(fname):
    with open(os.path.join(GOLDEN, fname)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            yield [c.strip() for c in line.split("|")]


def _ints(s):
    return [int(x) for x in s.split(",")]


# ---------------------------------------------------------------- validation / mask
TREE_ROWS = list(_rows("trees.txt"))


@pytest.mark.parametrize("row", TREE_ROWS, ids=[r[0] for r in TREE_ROWS])
def test_golden_trees(row):
    name, M, par, status, depths, masks = row
    M = int(M)
    par = np.array(_ints(par), dtype=np.int64).astype(np.int32)
    first, st = oracle.validate(par[None], M)
    assert st[0] == int(status) and first == int(status)
    mk, dp = oracle.mask(par[None], M, st)
    if depths == "-":
        assert not mk.any() and not dp.any()  # invalid trees give zeros
    else:
        assert dp[0].tolist() == _ints(depths)
        assert [int(m) for m in mk[0, :, 0]] == [int(x, 16) for x in masks.split(",")]


def _brute_status(par, M):
    """Independent check: ROOT / RANGE by inspection, CYCLE by following
    parents with a visited set."""
    if par[0] != 0:
        return -3
    for i in range(1, M + 1):
        if not (0 <= par[i] <= M) or par[i] == i:
            return -4
    for i in range(1, M + 1):
        seen, u = set(), i
        while u != 0:
            if u in seen:
                return -5
            seen.add(u)
            u = par[u]
    return 0


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_validate_exhaustive_small(M):
    # every parent array with entries in [-1, M+1] for rows 1..M, root 0 or 1
    vals = range(-1, M + 2)
    cases = []
    for root in (0, 1):
        for tail in itertools.product(vals, repeat=M):
            cases.append([root, *tail])
    par = np.array(cases, dtype=np.int32)
    _, st = oracle.validate(par, M)
    want = [_brute_status(list(p), M) for p in cases]
    assert st.tolist() == want


def _ancestors(par, i):
    out, u = [int(i)], int(i)
    while u != 0:
        u = int(par[u])
        out.append(u)
    return out


def _random_trees(n, M, seed):
    out = []
    for k in range(n):
        key = gen.stream_key(seed, k)
        if k % 3 == 0:
            p = gen.tree_depth_capped(key, M, 10)
        elif k % 3 == 1:
            p = gen.tree_bushy(key, M)
        else:
            p, _ = gen.tree_relabel(key, gen.tree_depth_capped(key, M, 4))
        out.append(p)
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("M", [0, 1, 8, 16, 63, 64, 65, 127, 200, 255])
def test_mask_invariants(M):
    par = _random_trees(6, M, 1000 + M)
    first, st = oracle.validate(par, M)
    assert first == 0
    mk, dp = oracle.mask(par, M, st)
    T, W = M + 1, (M + 64) // 64
    for b in range(par.shape[0]):
        p = par[b]

        def bit(i, j):
            return (int(mk[b, i, j // 64]) >> (j % 64)) & 1

        for i in range(T):
            anc = _ancestors(p, i)
            # brute-force ancestor walk
            want = [0] * W
            for j in anc:
                want[j // 64] |= 1 << (j % 64)
            assert [int(x) for x in mk[b, i]] == want
            assert dp[b, i] == len(anc) - 1
            assert bit(i, i) == 1 and bit(i, 0) == 1             # reflexive, root everywhere
            if i:
                pw = [int(x) for x in mk[b, p[i]]]               # transitive along the chain
                assert [pw[w] | ((1 << (i % 64)) if w == i // 64 else 0) for w in range(W)] == \
                    [int(x) for x in mk[b, i]]
            assert sum(bin(int(x)).count("1") for x in mk[b, i]) == dp[b, i] + 1
        # antisymmetric; siblings' subtrees share nothing but common ancestors
        for i in range(1, T):
            for j in range(1, T):
                if i != j and bit(i, j):
                    assert not bit(j, i)
        kids = {}
        for i in range(1, T):
            kids.setdefault(int(p[i]), []).append(i)
        for parent, ch in kids.items():
            for x, y in itertools.combinations(ch, 2):
                common = [int(a) & int(c) for a, c in zip(mk[b, x], mk[b, y])]
                pmask = [int(a) for a in mk[b, parent]]
                assert common == pmask  # no cross-branch entries


def test_mask_special_shapes():
    M = 64  # T = 65: the second word is used
    mk, dp = oracle.mask(gen.tree_chain(M)[None], M)
    full = np.tril(np.ones((M + 1, M + 1), dtype=np.int64))
    got = np.array([[(int(mk[0, i, j // 64]) >> (j % 64)) & 1 for j in range(M + 1)] for i in range(M + 1)])
    assert (got == full).all()  # chain = lower triangular (causal)
    assert int(mk[0, 64, 1]) == 1 and int(mk[0, 64, 0]) == 0xFFFFFFFFFFFFFFFF
    mk, dp = oracle.mask(gen.tree_star(M)[None], M)
    got = np.array([[(int(mk[0, i, j // 64]) >> (j % 64)) & 1 for j in range(M + 1)] for i in range(M + 1)])
    want = np.eye(M + 1, dtype=np.int64)
    want[:, 0] = 1
    assert (got == want).all()  # star = identity + root column


# ---------------------------------------------------------------- attention
def _sdpa(q, k, v, scale, mask=None, causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)[0, 0].numpy()


def _attn_case(B, M, Hq, Hkv, D, lens, cap, seed, parents=None, sigma=1.0):
    T = M + 1
    key = lambda t, b=0: gen.stream_key(seed, t, b)
    if parents is None:
        parents = np.stack([gen.tree_depth_capped(key(1, b), M, 4) for b in range(B)])
    lens = np.asarray(lens, np.int32)
    lmax = int(lens.max())
    q = gen.normal(key(2), B * T * Hq * D, sigma).astype(np.float32).reshape(B, T, Hq, D)
    kc = np.full((B, Hkv, cap, D), np.nan, np.float32)
    vc = np.full((B, Hkv, cap, D), np.nan, np.float32)
    for b in range(B):
        L = int(lens[b])
        kc[b, :, lmax - L:lmax] = gen.normal(key(3, b), Hkv * L * D, sigma).astype(np.float32).reshape(Hkv, L, D)
        vc[b, :, lmax - L:lmax] = gen.normal(key(4, b), Hkv * L * D).astype(np.float32).reshape(Hkv, L, D)
    kt = gen.normal(key(5), B * Hkv * T * D, sigma).astype(np.float32).reshape(B, Hkv, T, D)
    vt = gen.normal(key(6), B * Hkv * T * D).astype(np.float32).reshape(B, Hkv, T, D)
    mk, _ = oracle.mask(parents, M)
    return dict(parents=parents, lens=lens, lmax=lmax, q=q, kc=kc, vc=vc, kt=kt, vt=vt, mk=mk)


def test_attention_chain_is_causal():
    """A chain-shaped tree equals causal attention over [prefix; chain]."""
    B, M, Hq, Hkv, D, L = 1, 12, 4, 2, 32, 20
    c = _attn_case(B, M, Hq, Hkv, D, [L], 24, 7, parents=gen.tree_chain(M)[None])
    rc, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"])
    assert rc == 0
    scale = 1 / np.sqrt(D)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        kseq = np.concatenate([c["kc"][0, g, c["lmax"] - L:c["lmax"]], c["kt"][0, g]])
        vseq = np.concatenate([c["vc"][0, g, c["lmax"] - L:c["lmax"]], c["vt"][0, g]])
        # full causal sequence; the prefix positions get dummy queries
        qseq = np.concatenate([np.zeros((L, D), np.float32), c["q"][0, :, h]])
        ref = _sdpa(qseq, kseq, vseq, scale, causal=True)[L:]
        np.testing.assert_allclose(out[0, :, h], ref, rtol=1e-12, atol=1e-12)


def test_attention_single_node_is_decode():
    """M = 0 (root only) equals plain decode attention over prefix + root."""
    B, M, Hq, Hkv, D = 3, 0, 8, 2, 64
    lens = [5, 0, 17]
    c = _attn_case(B, M, Hq, Hkv, D, lens, 20, 11, parents=np.zeros((B, 1), np.int32))
    rc, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"])
    assert rc == 0
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            k = np.concatenate([c["kc"][b, g, c["lmax"] - L:c["lmax"]], c["kt"][b, g, :1]])
            v = np.concatenate([c["vc"][b, g, c["lmax"] - L:c["lmax"]], c["vt"][b, g, :1]])
            ref = _sdpa(c["q"][b, :, h], k, v, 1 / np.sqrt(D))
            np.testing.assert_allclose(out[b, :, h], ref, rtol=1e-12, atol=1e-12)


def test_attention_per_node_path_equivalence():
    """Row i equals decode attention over prefix + the tree rows on i's root path."""
    B, M, Hq, Hkv, D = 2, 10, 6, 3, 16
    lens = [9, 4]
    c = _attn_case(B, M, Hq, Hkv, D, lens, 12, 13)
    rc, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"])
    for b in range(B):
        L = lens[b]
        for i in range(M + 1):
            anc = sorted(_ancestors(c["parents"][b], i))
            for h in range(Hq):
                g = h // (Hq // Hkv)
                k = np.concatenate([c["kc"][b, g, c["lmax"] - L:c["lmax"]], c["kt"][b, g, anc]])
                v = np.concatenate([c["vc"][b, g, c["lmax"] - L:c["lmax"]], c["vt"][b, g, anc]])
                ref = _sdpa(c["q"][b, i, h][None], k, v, 1 / np.sqrt(D))[0]
                np.testing.assert_allclose(out[b, i, h], ref, rtol=1e-12, atol=1e-12)


def test_attention_no_leakage_and_padding_unread():
    """Changing K/V of non-ancestors leaves a row bitwise unchanged; NaN in the
    padding columns never reaches the output."""
    B, M, Hq, Hkv, D = 1, 14, 2, 1, 8
    c = _attn_case(B, M, Hq, Hkv, D, [6], 10, 17)
    _, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"])
    assert np.isfinite(out).all()
    for i in range(M + 1):
        anc = set(_ancestors(c["parents"][0], i))
        others = [j for j in range(M + 1) if j not in anc]
        kt2, vt2 = c["kt"].copy(), c["vt"].copy()
        kt2[0, :, others] += 3.0
        vt2[0, :, others] -= 5.0
        _, out2 = oracle.attention(c["q"], c["kc"], c["vc"], kt2, vt2, c["mk"], c["lens"], c["lmax"])
        assert np.array_equal(out2[0, i], out[0, i])


def test_attention_relabel_permutes():
    B, M, Hq, Hkv, D = 1, 9, 2, 1, 8
    c = _attn_case(B, M, Hq, Hkv, D, [5], 5, 19)
    _, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"])
    par2, perm = gen.tree_relabel(gen.stream_key(3), c["parents"][0])
    inv = np.argsort(perm)
    q2, kt2, vt2 = c["q"][:, inv], c["kt"][:, :, inv], c["vt"][:, :, inv]
    mk2, _ = oracle.mask(par2[None], M)
    _, out2 = oracle.attention(q2, c["kc"], c["vc"], kt2, vt2, mk2, c["lens"], c["lmax"])
    np.testing.assert_allclose(out2[0], out[0, inv], rtol=1e-13, atol=1e-14)


def test_attention_batch_equals_alone():
    """A ragged left-padded batch equals each sequence run alone."""
    B, M, Hq, Hkv, D = 3, 6, 4, 2, 16
    lens = [11, 3, 7]
    c = _attn_case(B, M, Hq, Hkv, D, lens, 14, 23)
    _, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"])
    for b in range(B):
        L = lens[b]
        kc1 = c["kc"][b:b + 1, :, c["lmax"] - L:c["lmax"]]
        vc1 = c["vc"][b:b + 1, :, c["lmax"] - L:c["lmax"]]
        _, o1 = oracle.attention(c["q"][b:b + 1], kc1, vc1, c["kt"][b:b + 1], c["vt"][b:b + 1],
                                 c["mk"][b:b + 1], [L], L)
        assert np.array_equal(o1[0], out[b])


def test_attention_rows_threads_equal_serial():
    """The threaded row driver returns exactly the serial driver's rows (the
    same C routine per row, in any thread order), for any thread count and
    with a bf16-style converter applied slab by slab."""
    c = _attn_case(3, 20, 8, 2, 64, [50, 0, 130], 140, 21)
    _, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"])
    rows = [(b, i, h) for b in range(3) for i in range(21) for h in range(8)][::3]
    want = np.stack([out[b, i, h] for b, i, h in rows])
    for th in (1, 4, 7):
        got = oracle.attention_rows(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"],
                                    rows, threads=th)
        assert np.array_equal(got, want), th
    bits = lambda x: gen.to_bf16_bits(np.asarray(x, np.float32))
    up = gen.bf16_bits_to_f32
    _, out16 = oracle.attention(up(bits(c["q"])), up(bits(c["kc"])), up(bits(c["vc"])), up(bits(c["kt"])),
                                up(bits(c["vt"])), c["mk"], c["lens"], c["lmax"])
    got16 = oracle.attention_rows(bits(c["q"]), bits(c["kc"]), bits(c["vc"]), bits(c["kt"]), bits(c["vt"]),
                                  c["mk"], c["lens"], c["lmax"], rows, threads=5, to_f32=up)
    assert np.array_equal(got16, np.stack([out16[b, i, h] for b, i, h in rows]))


def test_attention_closed_forms():
    B, M, Hq, Hkv, D = 2, 7, 4, 1, 8
    c = _attn_case(B, M, Hq, Hkv, D, [5, 2], 6, 29)
    # all V rows equal to a constant vector -> output is that vector
    cst = np.arange(D, dtype=np.float32) - 3.5
    vc = np.broadcast_to(cst, c["vc"].shape).copy()
    vt = np.broadcast_to(cst, c["vt"].shape).copy()
    _, out = oracle.attention(c["q"], c["kc"], vc, c["kt"], vt, c["mk"], c["lens"], c["lmax"])
    np.testing.assert_allclose(out, np.broadcast_to(cst, out.shape), rtol=0, atol=1e-12)
    # all K equal -> uniform weights -> mean of the attended V rows
    kc = np.ones_like(c["kc"])
    kt = np.ones_like(c["kt"])
    _, out = oracle.attention(c["q"], kc, c["vc"], kt, c["vt"], c["mk"], c["lens"], c["lmax"])
    for b in range(B):
        L = int(c["lens"][b])
        for i in range(M + 1):
            anc = sorted(_ancestors(c["parents"][b], i))
            rows = np.concatenate([c["vc"][b, 0, c["lmax"] - L:c["lmax"]], c["vt"][b, 0, anc]]).astype(np.float64)
            np.testing.assert_allclose(out[b, i, 0], rows.mean(0), rtol=1e-12, atol=1e-12)


def test_attention_invalid_sequences_zero():
    B, M = 2, 3
    c = _attn_case(B, M, 2, 1, 8, [3, 3], 4, 31)
    st = np.array([0, -5], np.int32)
    rc, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], c["lens"], c["lmax"], status=st)
    assert rc == 0 and not out[1].any() and np.abs(out[0]).sum() > 0
    rc, out = oracle.attention(c["q"], c["kc"], c["vc"], c["kt"], c["vt"], c["mk"], [5, 3], 3)
    assert rc == oracle.ERR_LENGTH and not out[0].any()


# ---------------------------------------------------------------- argmax / accept
def test_argmax_matches_numpy_with_ties_and_nan():
    key = gen.stream_key(41)
    x = np.round(gen.normal(key, 64 * 300) * 2) / 2  # quantised: many ties at the top
    x = x.astype(np.float32).reshape(64, 300)
    x[3, [10, 20, 30]] = np.nan                       # first NaN wins
    x[4, :] = -0.0
    x[4, 7] = 0.0                                     # -0.0 == +0.0: index 0 wins
    x[5, :] = -np.inf
    x[6, 299] = np.inf
    got = oracle.argmax(x)
    assert got.tolist() == np.argmax(x, axis=1).tolist()
    assert got[3] == 10 and got[4] == 0 and got[5] == 0 and got[6] == 299


ACCEPT_ROWS = list(_rows("accept.txt"))


@pytest.mark.parametrize("row", ACCEPT_ROWS, ids=[r[0] for r in ACCEPT_ROWS])
def test_golden_accept(row):
    name, am, tok, al, path, bonus = row
    par = np.array([0, 0, 0, 1, 1, 3], np.int32)
    a, p, bo = oracle.accept(np.array(_ints(am)), np.array(_ints(tok)), par, 5)
    assert a[0] == int(al) and p[0].tolist() == _ints(path) and bo[0] == int(bonus)


def _brute_accept(par, amax, tok):
    """Enumerate every root path by DFS over children, keep paths whose edges
    all hold tok[child] == amax[parent]; longest wins, then lowest end index."""
    T = len(par)
    kids = {i: [] for i in range(T)}
    for i in range(1, T):
        kids[int(par[i])].append(i)
    best = (0, 0, [0])  # (depth, -end, path)
    stack = [[0]]
    while stack:
        pth = stack.pop()
        end = pth[-1]
        cand = (len(pth) - 1, -end, pth)
        if cand[:2] > best[:2]:
            best = cand
        for ch in kids[end]:
            if tok[ch] == amax[end]:
                stack.append(pth + [ch])
    return best[0], best[2], amax[best[2][-1]]


@pytest.mark.parametrize("M", [1, 2, 4, 6, 8])
def test_accept_brute_force_exhaustive(M):
    trees = _random_trees(6, M, 500 + M)
    V = 5
    for t, par in enumerate(trees):
        amax = gen.randint(gen.stream_key(600 + M, t), M + 1, 0, V - 1).astype(np.int32)
        for pattern in range(1 << M):  # every planted / unplanted pattern
            tok = np.full(M + 1, 0, np.int32)
            for i in range(1, M + 1):
                planted = (pattern >> (i - 1)) & 1
                tok[i] = amax[par[i]] if planted else (amax[par[i]] + 1) % V
            a, p, bo = oracle.accept(amax, tok, par, M)
            ba, bp, bb = _brute_accept(par, amax, tok)
            assert a[0] == ba and p[0, :ba + 1].tolist() == bp and not p[0, ba + 1:].any() and bo[0] == bb


def test_accept_properties():
    M = 32
    trees = _random_trees(8, M, 777)
    mk, dp = oracle.mask(trees, M)
    amax = gen.randint(gen.stream_key(778), trees.size, 0, 3).astype(np.int32).reshape(trees.shape)
    tok = gen.randint(gen.stream_key(779), trees.size, 0, 3).astype(np.int32).reshape(trees.shape)
    al, path, bonus = oracle.accept(amax, tok, trees, M)
    for b in range(trees.shape[0]):
        assert al[b] <= dp[b].max()
        for k in range(al[b]):
            assert trees[b, path[b, k + 1]] == path[b, k]
            assert dp[b, path[b, k + 1]] == k + 1
    # chain with every draft planted accepts everything
    ch = gen.tree_chain(M)
    am = np.arange(M + 1, dtype=np.int32)
    tk = np.concatenate([[0], am[:-1]]).astype(np.int32)
    al, path, bonus = oracle.accept(am, tk, ch, M)
    assert al[0] == M and path[0].tolist() == list(range(M + 1)) and bonus[0] == M
    # no depth-1 node correct -> nothing accepted, bonus is the root's greedy token
    st = gen.tree_star(M)
    al, path, bonus = oracle.accept(am, am + 1, st, M)
    assert al[0] == 0 and not path.any() and bonus[0] == am[0]
    # invalid status
    al, path, bonus = oracle.accept(am, tk, ch, M, status=np.array([-5], np.int32))
    assert al[0] == 0 and not path.any() and bonus[0] == am[0]


# ---------------------------------------------------------------- commit
def test_golden_commit():
    with open(os.path.join(GOLDEN, "commit.json")) as f:
        g = json.load(f)
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
                                                    ini["lmax"], case["path"], case["accept_len"])
        assert rc == case["rc"], case["name"]
        if rc:
            assert np.array_equal(km2, km) and np.array_equal(tm2, tm) and ln2.tolist() == ini["lens"]
            continue
        assert ln2.tolist() == case["lens"] and lm2 == case["lmax"]
        for name, got in (("k_main", km2[0, 0, :, 0, :, 0]), ("v_main", km2[0, 1, :, 0, :, 0]),
                          ("tokens_main", tm2)):
            for b, want in enumerate(case[name]):
                for c, v in enumerate(want):
                    if v is not None:
                        assert got[b, c] == v, (case["name"], name, b, c)
        assert pos[:, :case["lmax"]].tolist() == case["pos_ids"]
        u = case["untouched_from"]
        assert (km2[..., u:, :] == km[..., u:, :]).all() and (tm2[:, u:] == tm[:, u:]).all()


def _commit_case(B, Hkv, L, M, lens, cap, seed, row_elems=4):
    T = M + 1
    lens = np.asarray(lens, np.int32)
    lmax = int(lens.max())
    slab = np.arange(L * 2 * B * Hkv).reshape(L, 2, B, Hkv, 1, 1)
    col = np.arange(cap).reshape(1, 1, 1, 1, cap, 1)
    el = np.arange(row_elems).reshape(1, 1, 1, 1, 1, row_elems)
    km = gen.commit_pattern_bits(slab, col, el)
    kb = gen.commit_pattern_bits(slab + 5000, np.arange(T).reshape(1, 1, 1, 1, T, 1), el)
    trees = _random_trees(B, M, seed)
    amax = gen.randint(gen.stream_key(seed, 1), B * T, 0, 2).astype(np.int32).reshape(B, T)
    tok = gen.randint(gen.stream_key(seed, 2), B * T, 0, 2).astype(np.int32).reshape(B, T)
    al, path, _ = oracle.accept(amax, tok, trees, M)
    tm = gen.randint(gen.stream_key(seed, 3), B * cap, 0, 1000).astype(np.int32).reshape(B, cap)
    return km, kb, tm, tok, lens, lmax, path, al


def test_commit_batch_equals_alone_and_invariants():
    B, Hkv, L, M, cap = 5, 2, 2, 12, 40
    lens = [17, 3, 0, 25, 9]
    km, kb, tm, tok, lens, lmax, path, al = _commit_case(B, Hkv, L, M, lens, cap, 91)
    rc, km2, tm2, ln2, lm2, pos = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al)
    assert rc == 0
    A = al + 1
    assert (ln2 == lens + A).all() and lm2 == int((lens + A).max())
    for b in range(B):
        pad = lm2 - ln2[b]
        assert pad + ln2[b] == lm2                                    # rectangular alignment
        assert pos[b, pad:lm2].tolist() == list(range(ln2[b]))        # contiguous from 0
        assert not pos[b, :pad].any()
        # content = old content followed by the accepted branch rows, in path order
        old = km[:, :, b, :, lmax - lens[b]:lmax]
        new = km2[:, :, b, :, pad:lm2]
        assert np.array_equal(new[:, :, :, :lens[b]], old)
        assert np.array_equal(new[:, :, :, lens[b]:], kb[:, :, b][:, :, :, path[b, :A[b]]])
        assert tm2[b, pad:lm2].tolist() == tm[b, lmax - lens[b]:lmax].tolist() + tok[b, path[b, :A[b]]].tolist()
        # each sequence committed alone (B = 1, no padding) gives the same content
        rc1, k1, t1, l1, m1, _ = oracle.commit(km[:, :, b:b + 1, :, lmax - lens[b]:],
                                               kb[:, :, b:b + 1], M, tm[b:b + 1, lmax - lens[b]:], tok[b:b + 1],
                                               lens[b:b + 1], lens[b], path[b:b + 1], al[b:b + 1])
        assert rc1 == 0 and np.array_equal(k1[:, :, 0, :, :ln2[b]], new)
    assert np.array_equal(km2[..., lm2:, :], km[..., lm2:, :])        # beyond new lmax untouched


def test_commit_b1_is_append_and_chain_is_length_based():
    M, cap = 8, 30
    km, kb, tm, tok, lens, lmax, path, al = _commit_case(1, 1, 1, M, [12], cap, 93)
    rc, km2, tm2, ln2, lm2, _ = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al)
    A = int(al[0]) + 1
    # fast reorder: prefix untouched, new rows appended at [len, len + A)
    assert np.array_equal(km2[..., :12, :], km[..., :12, :])
    assert np.array_equal(km2[0, :, 0, :, 12:12 + A], kb[0, :, 0][:, :, path[0, :A]])
    # chain path [0..A): equals keeping the prefix and appending the first A branch steps
    chain_path = np.arange(M + 1, dtype=np.int32)[None]
    acc = np.array([5], np.int32)
    rc, km3, _, _, _, _ = oracle.commit(km, kb, M, None, tok, lens, lmax, chain_path, acc)
    assert rc == 0 and np.array_equal(km3[..., 12:18, :], kb[..., :6, :])


def test_commit_invalid_and_errors():
    B, M, cap = 3, 5, 20
    km, kb, tm, tok, lens, lmax, path, al = _commit_case(B, 1, 1, M, [4, 9, 6], cap, 95)
    st = np.array([0, -4, 0], np.int32)
    rc, km2, tm2, ln2, lm2, pos = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al, status=st)
    assert rc == 0 and ln2[1] == 9   # invalid sequence appends nothing
    pad1 = lm2 - 9
    assert np.array_equal(km2[:, :, 1, :, pad1:lm2], km[:, :, 1, :, lmax - 9:lmax])  # but is re-aligned
    # capacity overflow changes nothing
    rc, km3, tm3, ln3, lm3, _ = oracle.commit(km[..., :lmax + 1, :], kb, M, tm[:, :lmax + 1], tok, lens, lmax,
                                              path, np.array([5, 5, 5], np.int32))
    assert rc == oracle.ERR_CAPACITY and np.array_equal(km3, km[..., :lmax + 1, :]) and ln3.tolist() == lens.tolist()
    # out-of-range accept length is an argument error
    rc, *_ = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, np.array([0, M + 1, 0], np.int32))
    assert rc == oracle.ERR_ARG
