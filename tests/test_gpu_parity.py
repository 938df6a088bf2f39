"""GPU parity: every libsvt call against the CPU oracle on seeded inputs.

Integer outputs (masks, depths, statuses, argmax, accept results, committed
cache bytes, tokens, position ids) must match bit for bit; attention must be
within the contract tolerance (1e-4 max-abs for fp32 inputs, 2e-2 for bf16)
and within the normalised bound of tests/harness.py.  Sizes span several
tiles and ragged tails; the full-size workloads are in test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from synth import gen
from synth import workloads as wl
from tree_masked_verification_parent_amd import svt

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _i32(x):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=DEV)


# ------------------------------------------------------------------ mask
def _trees(B, M, seed, kind="mixed"):
    out = []
    for b in range(B):
        k = gen.stream_key(seed, b)
        if kind == "chain":
            p = gen.tree_chain(M)
        elif kind == "star":
            p = gen.tree_star(M)
        elif b % 3 == 0:
            p = gen.tree_depth_capped(k, M, 10)
        elif b % 3 == 1:
            p = gen.tree_bushy(k, M)
        else:
            p, _ = gen.tree_relabel(k, gen.tree_depth_capped(k, M, 4))
        out.append(p)
    return np.array(out, dtype=np.int32).reshape(B, M + 1)


def _run_mask(par, M, flags=0):
    B = par.shape[0]
    T, W = M + 1, (M + 64) // 64
    p = _i32(par)
    mk = torch.full((B, T, W), -1, dtype=torch.int64, device=DEV)
    dp = torch.full((B, T), -7, dtype=torch.int32, device=DEV)
    st = torch.full((B,), 99, dtype=torch.int32, device=DEV)
    rc = svt.svt_build_mask(p, M, mk, dp, st, flags)
    torch.cuda.synchronize()
    return rc, H.from_dev(mk).view(np.uint64), H.from_dev(dp), H.from_dev(st)


@pytest.mark.parametrize("M", [0, 1, 8, 16, 32, 63, 64, 65, 127, 128, 200, 255])
@pytest.mark.parametrize("kind", ["mixed", "chain", "star"])
def test_build_mask_parity(M, kind):
    par = _trees(7, M, 4000 + M, kind)
    rc, mk, dp, st = _run_mask(par, M)
    assert rc == 0
    first, ost = oracle.validate(par, M)
    omk, odp = oracle.mask(par, M, ost)
    assert np.array_equal(st, ost)
    assert np.array_equal(mk, omk)
    assert np.array_equal(dp, odp)


def test_build_mask_invalid_trees_and_sync_check():
    M = 70
    base = _trees(8, M, 4242)
    bad = base.copy()
    bad[1, 0] = 5                                  # root
    bad[2, 33] = M + 1                             # range
    bad[3, 9] = -1                                 # range
    bad[4, 40] = 40                                # self loop -> range
    bad[5, 66], bad[5, 67] = 67, 66                # 2-cycle across the word boundary
    bad[6, 10] = 0x7FFFFFFF
    rc, mk, dp, st = _run_mask(bad, M, flags=svt.SVT_SYNC_CHECK)
    first, ost = oracle.validate(bad, M)
    omk, odp = oracle.mask(bad, M, ost)
    assert st.tolist() == ost.tolist() == [0, -3, -4, -4, -4, -5, -4, 0]
    assert rc == first == -3
    assert np.array_equal(mk, omk) and np.array_equal(dp, odp)


def test_build_mask_exhaustive_small():
    M = 3
    import itertools
    cases = [[r, *t] for r in (0, 1) for t in itertools.product(range(-1, M + 2), repeat=M)]
    par = np.array(cases, dtype=np.int32)
    rc, mk, dp, st = _run_mask(par, M)
    _, ost = oracle.validate(par, M)
    omk, odp = oracle.mask(par, M, ost)
    assert np.array_equal(st, ost) and np.array_equal(mk, omk) and np.array_equal(dp, odp)


# ------------------------------------------------------------------ accept
def _run_accept(logits, tokens, par, M, status=None):
    B, T, V = logits.shape
    lg = torch.as_tensor(logits, device=DEV)
    tk, pr = _i32(tokens), _i32(par)
    st = _i32(np.zeros(B) if status is None else status)
    W = (T + 63) // 64
    mk = torch.zeros(B, T, W, dtype=torch.int64, device=DEV)
    dp = torch.zeros(B, T, dtype=torch.int32, device=DEV)
    st_mask = torch.zeros(B, dtype=torch.int32, device=DEV)
    assert svt.svt_build_mask(pr, M, mk, dp, st_mask) == 0
    if status is not None:
        st_use = st
    else:
        st_use = st_mask
    am = torch.full((B, T), -1, dtype=torch.int32, device=DEV)
    al = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    path = torch.full((B, T), -1, dtype=torch.int32, device=DEV)
    bo = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    args = svt.accept_args(lg, tk, pr, mk, dp, am, al, path, bo, status=st_use)
    ws = torch.empty(svt.svt_accept_workspace(args), dtype=torch.uint8, device=DEV)
    args = svt.accept_args(lg, tk, pr, mk, dp, am, al, path, bo, status=st_use, workspace=ws)
    rc = svt.svt_accept(args)
    torch.cuda.synchronize()
    return rc, H.from_dev(am), H.from_dev(al), H.from_dev(path), H.from_dev(bo)


def _oracle_accept(logits, tokens, par, M, status=None):
    am = oracle.argmax(logits)
    if status is None:
        _, status = oracle.validate(par, M)
    al, path, bo = oracle.accept(am, tokens, par, M, status)
    return am, al, path, bo


@pytest.mark.parametrize("B,M,V", [(1, 8, 1000), (3, 16, 32000), (5, 33, 4099), (2, 64, 151552),
                                   (4, 100, 777), (2, 255, 96), (6, 0, 50)])
def test_accept_parity_planted(B, M, V):
    par = _trees(B, M, 5000 + M)
    logits, des = gen.logits_with_designated_top(gen.stream_key(5100 + M), B * (M + 1), V)
    logits = logits.reshape(B, M + 1, V)
    des = des.reshape(B, M + 1)
    tok = np.stack([gen.plant_drafts(gen.stream_key(5200 + M, b), par[b], des[b], V, 0.8) for b in range(B)])
    rc, am, al, path, bo = _run_accept(logits, tok, par, M)
    assert rc == 0
    oam, oal, opath, obo = _oracle_accept(logits, tok, par, M)
    assert np.array_equal(am, oam)
    assert np.array_equal(al, oal) and np.array_equal(path, opath) and np.array_equal(bo, obo)


def test_accept_ties_nan_and_signed_zero():
    B, M, V = 4, 20, 3000
    par = _trees(B, M, 5300)
    x = np.round(gen.normal(gen.stream_key(5301), B * (M + 1) * V) * 1.5).astype(np.float32)
    x = x.reshape(B, M + 1, V)             # quantised: ties at the top everywhere
    x[0, 3, [7, 1500, 2999]] = np.nan      # first NaN wins
    x[1, 2, :] = -0.0
    x[1, 2, [5, 9]] = 0.0
    x[2, 4, :] = -np.inf
    x[2, 5, :] = np.float32(1e30)
    x[3, 6, 2999] = np.inf
    am0 = oracle.argmax(x)
    tok = np.zeros((B, M + 1), np.int32)
    for b in range(B):                      # plant on the oracle's argmax to get long paths
        for i in range(1, M + 1):
            tok[b, i] = am0[b, par[b, i]] if (i % 4) else (am0[b, par[b, i]] + 1) % V
    rc, am, al, path, bo = _run_accept(x, tok, par, M)
    oam, oal, opath, obo = _oracle_accept(x, tok, par, M)
    assert np.array_equal(am, oam)
    assert am[0, 3] == 7 and am[1, 2] == 0 and am[2, 4] == 0 and am[2, 5] == 0 and am[3, 6] == 2999
    assert np.array_equal(al, oal) and np.array_equal(path, opath) and np.array_equal(bo, obo)


def test_accept_vocab_not_multiple_of_4_and_invalid_status():
    B, M, V = 3, 12, 1001
    par = _trees(B, M, 5400)
    logits, des = gen.logits_with_designated_top(gen.stream_key(5401), B * (M + 1), V)
    logits = logits.reshape(B, M + 1, V)
    tok = np.stack([gen.plant_drafts(gen.stream_key(5402, b), par[b], des.reshape(B, -1)[b], V, 0.9)
                    for b in range(B)])
    st = np.array([0, -5, 0], np.int32)
    rc, am, al, path, bo = _run_accept(logits, tok, par, M, status=st)
    oam, oal, opath, obo = _oracle_accept(logits, tok, par, M, status=st)
    assert np.array_equal(am, oam)
    assert np.array_equal(al, oal) and np.array_equal(path, opath) and np.array_equal(bo, obo)
    assert al[1] == 0 and not path[1].any() and bo[1] == am[1, 0]


# ------------------------------------------------------------------ commit
def _commit_inputs(B, Hkv, L, M, D, lens, cap, seed, esize):
    T = M + 1
    lens = np.asarray(lens, np.int32)
    lmax = int(lens.max()) if B else 0
    el = D * esize // 2
    slab = np.arange(L * 2 * B * Hkv).reshape(L, 2, B, Hkv, 1, 1)
    km = gen.commit_pattern_bits(slab, np.arange(cap).reshape(1, 1, 1, 1, cap, 1),
                                 np.arange(el).reshape(1, 1, 1, 1, 1, el))
    kb = gen.commit_pattern_bits(slab + 9000, np.arange(T).reshape(1, 1, 1, 1, T, 1),
                                 np.arange(el).reshape(1, 1, 1, 1, 1, el))
    trees = _trees(B, M, seed)
    am = gen.randint(gen.stream_key(seed, 1), B * T, 0, 1).astype(np.int32).reshape(B, T)
    tok = gen.randint(gen.stream_key(seed, 2), B * T, 0, 1).astype(np.int32).reshape(B, T)
    al, path, _ = oracle.accept(am, tok, trees, M)
    tm = gen.randint(gen.stream_key(seed, 3), B * cap, 0, 10 ** 6).astype(np.int32).reshape(B, cap)
    return km, kb, tm, tok, lens, lmax, path, al


def _run_commit(km, kb, tm, tok, lens, lmax, path, al, D, esize, status=None, flags=0):
    dt = torch.float32 if esize == 4 else torch.bfloat16
    km_t = torch.from_numpy(km.view(np.int16).copy()).to(DEV).view(dt)
    kb_t = torch.from_numpy(kb.view(np.int16).copy()).to(DEV).view(dt)
    shape = km.shape[:5] + (D,)
    km_t = km_t.reshape(shape)
    kb_t = kb_t.reshape(kb.shape[:5] + (D,))
    B, cap = tm.shape
    tm_t, tok_t = _i32(tm), _i32(tok)
    ln_t, lm_t = _i32(lens), _i32([lmax])
    pos = torch.full((B, cap), -3, dtype=torch.int32, device=DEV)
    cst = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    st_t = None if status is None else _i32(status)
    args = svt.commit_args(km_t, kb_t, ln_t, lm_t, _i32(path), _i32(al), cst, tokens_main=tm_t,
                           tree_tokens=tok_t, pos_ids=pos, status=st_t)
    rc = svt.svt_commit(args, flags)
    torch.cuda.synchronize()
    got_km = km_t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(km.shape)
    return (rc, got_km, H.from_dev(tm_t), H.from_dev(ln_t), int(H.from_dev(lm_t)[0]), H.from_dev(pos),
            int(H.from_dev(cst)[0]))


def _check_commit(km, kb, tm, tok, lens, lmax, path, al, D, esize, status=None):
    M = kb.shape[4] - 1
    rc, gkm, gtm, gln, glm, gpos, gcst = _run_commit(km, kb, tm, tok, lens, lmax, path, al, D, esize, status)
    orc, okm, otm, oln, olm, opos = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al, status)
    assert rc == 0 and gcst == orc
    if orc != 0:
        assert np.array_equal(gkm, km) and np.array_equal(gtm, tm)
        assert gln.tolist() == list(lens) and glm == lmax
        return orc
    assert np.array_equal(gln, oln) and glm == olm
    for b in range(km.shape[2]):
        pad = olm - oln[b]
        assert np.array_equal(gkm[:, :, b, :, pad:olm], okm[:, :, b, :, pad:olm]), f"kv b={b}"
        assert np.array_equal(gtm[b, pad:olm], otm[b, pad:olm]), f"tokens b={b}"
        assert np.array_equal(gpos[b, :olm], opos[b, :olm]), f"pos b={b}"
        assert (gpos[b, olm:] == -3).all()
    assert np.array_equal(gkm[..., olm:, :], km[..., olm:, :])  # beyond new lmax untouched
    assert np.array_equal(gtm[:, olm:], tm[:, olm:])
    return orc


@pytest.mark.parametrize("esize,D", [(2, 128), (2, 64), (4, 64), (4, 128)])
def test_commit_parity_ragged(esize, D):
    B, Hkv, L, M = 6, 3, 2, 20
    lens = [700, 5, 0, 1234, 333, 1234]     # long rows: many 16 KB chunks, both shift signs
    cap = 1300
    args = _commit_inputs(B, Hkv, L, M, D, lens, cap, 6000 + D + esize, esize)
    assert _check_commit(*args, D, esize) == 0


@pytest.mark.parametrize("M,al_list", [(40, [0, 40, 3, 40, 17]), (255, [255, 0, 9, 200, 128])])
def test_commit_shift_sizes_and_invalid_sequences(M, al_list):
    # |delta| below and (M = 255: up to 256 rows = 64 KB) above the 16 KB chunk,
    # both signs, an invalid sequence that is only re-aligned
    B, Hkv, L, D = 5, 2, 1, 128
    lens = [4000, 3960, 10, 4000, 2000]
    cap = 4300
    km, kb, tm, tok, ln, lmax, path, al = _commit_inputs(B, Hkv, L, M, D, lens, cap, 6100 + M, 2)
    al = np.array(al_list, np.int32)
    path = np.zeros((B, M + 1), np.int32)
    for b in range(B):
        path[b, :al[b] + 1] = np.arange(al[b] + 1)   # chain paths are valid path indices
    st = np.array([0, 0, -4, 0, 0], np.int32)
    assert _check_commit(km, kb, tm, tok, ln, lmax, path, al, D, 2, status=st) == 0


def test_commit_capacity_and_bad_args_write_nothing():
    B, Hkv, L, M, D = 3, 2, 2, 10, 64
    km, kb, tm, tok, ln, lmax, path, al = _commit_inputs(B, Hkv, L, M, D, [50, 60, 55], 62, 6200, 2)
    al = np.array([3, 5, 1], np.int32)
    assert _check_commit(km, kb, tm, tok, ln, lmax, path, al, D, 2) == oracle.ERR_CAPACITY
    bad = al.copy()
    bad[1] = M + 1
    assert _check_commit(km, kb, tm, tok, ln, lmax, path, bad, D, 2) == oracle.ERR_ARG
    # SYNC_CHECK returns the device status
    rc = _run_commit(km, kb, tm, tok, ln, lmax, path, al, D, 2, flags=svt.SVT_SYNC_CHECK)[0]
    assert rc == svt.SVT_ERR_CAPACITY


def test_commit_b1_is_pure_append():
    B, Hkv, L, M, D = 1, 4, 3, 16, 128
    km, kb, tm, tok, ln, lmax, path, al = _commit_inputs(B, Hkv, L, M, D, [2048], 2100, 6300, 2)
    rc, gkm, gtm, gln, glm, _, _ = _run_commit(km, kb, tm, tok, ln, lmax, path, al, D, 2)
    A = int(al[0]) + 1
    assert glm == 2048 + A
    assert np.array_equal(gkm[..., :2048, :], km[..., :2048, :])   # prefix bytes untouched
    assert np.array_equal(gkm[:, :, 0, :, 2048:2048 + A], kb[:, :, 0][:, :, :, path[0, :A]])


# ------------------------------------------------------------------ attention
def _attn_case(w, lens, cap, seed, parents=None, poison=True):
    lens = np.asarray(lens, np.int32)
    q, kc, vc, kt, vt = wl.attention_inputs(w, lens, cap, seed, poison=poison)
    if parents is None:
        parents = wl.trees(w, seed)
    return q, kc, vc, kt, vt, parents, lens


def _run_attn(w, q, kc, vc, kt, vt, parents, lens, lmax_bound=None, status=None, scale=0.0, form=0, split_keys=0):
    return H.run_attention(q, kc, vc, kt, vt, parents, lens, lmax_bound=lmax_bound, status=status, scale=scale,
                           form=form, split_keys=split_keys)


def _small_w(base, **kw):
    import dataclasses
    return dataclasses.replace(wl.workload(base), **kw)


ATTN_CASES = [
    # name, workload overrides, lens
    ("fp32-d64-gqa4", dict(B=1, dtype="fp32", Hq=4, Hkv=1, D=64, M=8), [128]),
    ("fp32-d128-ragged", dict(B=3, dtype="fp32", Hq=6, Hkv=2, D=128, M=20), [300, 0, 77]),
    ("bf16-d128-mha-2tiles", dict(B=3, dtype="bf16", Hq=4, Hkv=4, D=128, M=16), [700, 513, 64]),
    ("bf16-d128-gqa4-M32", dict(B=2, dtype="bf16", Hq=8, Hkv=2, D=128, M=32), [1500, 37]),
    ("bf16-d128-gqa16-M64", dict(B=1, dtype="bf16", Hq=32, Hkv=2, D=128, M=64, tree="bushy"), [2100]),
    ("bf16-d64-gqa2-M100", dict(B=2, dtype="bf16", Hq=4, Hkv=2, D=64, M=100), [90, 1]),
    ("bf16-d128-M255", dict(B=1, dtype="bf16", Hq=2, Hkv=1, D=128, M=255), [200]),
    ("bf16-d128-M0-decode", dict(B=4, dtype="bf16", Hq=8, Hkv=8, D=128, M=0), [5000, 1, 64, 65]),
    ("bf16-lenzero", dict(B=2, dtype="bf16", Hq=8, Hkv=4, D=128, M=12), [0, 0]),
    ("bf16-gqa8-qw3", dict(B=2, dtype="bf16", Hq=16, Hkv=2, D=128, M=20), [4100, 999]),
    ("bf16-gqa4-qw2", dict(B=2, dtype="bf16", Hq=8, Hkv=2, D=128, M=24), [3000, 2999]),
    # 3 and 5-6 query tiles per KV head: the four- and six-wave stream forms
    ("bf16-d128-gqa4-3tiles", dict(B=3, dtype="bf16", Hq=8, Hkv=2, D=128, M=11), [1000, 64, 301]),
    ("bf16-d64-gqa4-5tiles", dict(B=2, dtype="bf16", Hq=8, Hkv=2, D=64, M=16), [2000, 129]),
    ("bf16-d128-gqa2-6tiles", dict(B=2, dtype="bf16", Hq=4, Hkv=2, D=128, M=47), [777, 1500]),
    # head dim 64 with 2, 4 and 12 query tiles per KV head (the other D=64 stream forms)
    ("bf16-d64-mha-2tiles", dict(B=3, dtype="bf16", Hq=2, Hkv=2, D=64, M=20), [650, 3, 1200]),
    ("bf16-d64-gqa2-4tiles", dict(B=2, dtype="bf16", Hq=4, Hkv=2, D=64, M=31), [900, 2500]),
    ("bf16-d64-gqa16-12tiles", dict(B=2, dtype="bf16", Hq=16, Hkv=1, D=64, M=11), [1700, 400]),
    # fewer units than CUs: at most 8 query tiles per unit, the eight-wave
    # stream form; 13 tiles per KV head split 6 + 7 over two units
    ("bf16-d128-gqa4-8tiles", dict(B=1, dtype="bf16", Hq=8, Hkv=2, D=128, M=31), [2300]),
    ("bf16-d64-gqa4-13tiles", dict(B=2, dtype="bf16", Hq=8, Hkv=2, D=64, M=51), [1900, 333]),
    # at least as many units as CUs: up to 12 query tiles per unit, the nine-
    # and twelve-wave stream forms at both head dims
    ("bf16-d64-b32-9tiles", dict(B=32, dtype="bf16", Hq=32, Hkv=8, D=64, M=32),
     [64 + (37 * i) % 600 for i in range(32)]),
    ("bf16-d128-b32-12tiles", dict(B=32, dtype="bf16", Hq=32, Hkv=8, D=128, M=47),
     [1 + (53 * i) % 700 for i in range(32)]),
    ("bf16-d64-b32-12tiles", dict(B=32, dtype="bf16", Hq=32, Hkv=8, D=64, M=44),
     [(71 * i) % 650 for i in range(31)] + [650]),
    # one sequence long enough that every range of its whole-ranges-per-unit
    # grid holds tiles: the stream combine takes the pieces without a list
    ("bf16-d128-b1-wholeranges", dict(B=1, dtype="bf16", Hq=8, Hkv=8, D=128, M=127), [8200]),
    ("bf16-d64-b1-wholeranges", dict(B=1, dtype="bf16", Hq=16, Hkv=4, D=64, M=31), [17000]),
]


FORMS = [svt.SVT_ATTN_AUTO, svt.SVT_ATTN_SPLIT, svt.SVT_ATTN_STREAM]
FORM_IDS = ["auto", "split", "stream"]


def _stream_ok(w):
    return w.dtype == "bf16" and w.B <= 1024


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("name,over,lens", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_parity(name, over, lens, form):
    w = _small_w(1, **over)
    lens = np.asarray(lens, np.int32)
    cap = int(lens.max()) + 40
    q, kc, vc, kt, vt, par, lens = _attn_case(w, lens, cap, 7000 + len(name))
    rc, out, mk, st, sst = _run_attn(w, q, kc, vc, kt, vt, par, lens, form=form)
    if form == svt.SVT_ATTN_STREAM and not _stream_ok(w):
        assert rc == svt.SVT_ERR_UNSUPPORTED
        return
    assert rc == 0 and (sst == 0).all()
    orc, ref = oracle.attention(wl.as_f32(w, q), wl.as_f32(w, kc), wl.as_f32(w, vc), wl.as_f32(w, kt),
                                wl.as_f32(w, vt), mk, lens, int(lens.max()), st)
    H.check_attention(w, H.out_f32(w, out), ref, name)


MANY_CASES = [
    # more sequences than the stream form's workgroup has threads (its per-sequence
    # prefix scan runs in several passes), one query tile per KV head
    ("b300-decode-1wave", dict(B=300, dtype="bf16", Hq=2, Hkv=2, D=64, M=0), 150),
    ("b1024-M3-1wave", dict(B=1024, dtype="bf16", Hq=1, Hkv=1, D=64, M=3), 80),
    # MHA with at most 64 query rows per KV head and four (sequence, KV head)
    # pairs per CU: the automatic choice takes the split form
    ("b64-mha16-M16", dict(B=64, dtype="bf16", Hq=16, Hkv=16, D=128, M=16), 300),
]


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("name,over,lmax", MANY_CASES, ids=[c[0] for c in MANY_CASES])
def test_attention_many_sequences(name, over, lmax, form):
    w = _small_w(1, **over)
    rng = np.random.default_rng(8100 + len(name))
    lens = rng.integers(0, lmax + 1, size=w.B).astype(np.int32)
    lens[0] = lmax  # the longest sequence fixes lmax
    lens[1] = 0
    cap = lmax + 8
    q, kc, vc, kt, vt, par, lens = _attn_case(w, lens, cap, 8200 + len(name))
    rc, out, mk, st, sst = _run_attn(w, q, kc, vc, kt, vt, par, lens, form=form)
    assert rc == 0 and (sst == 0).all()
    orc, ref = oracle.attention(wl.as_f32(w, q), wl.as_f32(w, kc), wl.as_f32(w, vc), wl.as_f32(w, kt),
                                wl.as_f32(w, vt), mk, lens, int(lens.max()), st)
    H.check_attention(w, H.out_f32(w, out), ref, name)


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_attention_deterministic_and_no_leakage(form):
    w = _small_w(1, B=2, dtype="bf16", Hq=8, Hkv=2, D=128, M=40)
    lens = np.array([2500, 1800], np.int32)
    q, kc, vc, kt, vt, par, lens = _attn_case(w, lens, 2600, 7100)
    _, o1, mk, _, _ = _run_attn(w, q, kc, vc, kt, vt, par, lens, form=form)
    _, o2, _, _, _ = _run_attn(w, q, kc, vc, kt, vt, par, lens, form=form)
    a1, a2 = H.from_dev(o1), H.from_dev(o2)
    assert np.array_equal(a1, a2)  # bitwise run to run
    # perturb the K/V rows of every non-ancestor of node i: row i is unchanged bit for bit
    for b, i in [(0, 17), (1, 40), (0, 0)]:
        anc = [j for j in range(w.T) if (int(mk[b, i, j // 64]) >> (j % 64)) & 1]
        others = [j for j in range(w.T) if j not in anc]
        kt2, vt2 = kt.copy(), vt.copy()
        noise = gen.to_bf16_bits(gen.normal(gen.stream_key(7101, b, i), kt[b][:, others].size).astype(np.float32))
        kt2[b][:, others] = noise.reshape(kt[b][:, others].shape)
        vt2[b][:, others] = noise.reshape(vt[b][:, others].shape)[..., ::-1]
        _, o3, _, _, _ = _run_attn(w, q, kc, vc, kt2, vt2, par, lens, form=form)
        a3 = H.from_dev(o3)
        assert np.array_equal(a3[b, i], a1[b, i])


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_attention_batch_equals_alone(form):
    w = _small_w(1, B=3, dtype="bf16", Hq=8, Hkv=2, D=128, M=16)
    lens = np.array([1000, 130, 700], np.int32)
    q, kc, vc, kt, vt, par, lens = _attn_case(w, lens, 1000, 7200)
    _, out, _, _, _ = _run_attn(w, q, kc, vc, kt, vt, par, lens, form=form)
    full = H.from_dev(out)
    for b in range(3):
        L = int(lens[b])
        sl = slice(1000 - L, 1000)
        w1 = _small_w(1, B=1, dtype="bf16", Hq=8, Hkv=2, D=128, M=16)
        _, o1, _, _, _ = _run_attn(w1, q[b:b + 1], np.ascontiguousarray(kc[b:b + 1, :, sl]),
                                   np.ascontiguousarray(vc[b:b + 1, :, sl]), kt[b:b + 1], vt[b:b + 1],
                                   par[b:b + 1], lens[b:b + 1], form=form)
        if form == svt.SVT_ATTN_SPLIT:
            # same keys, same split boundaries relative to the content: identical bits
            assert np.array_equal(H.from_dev(o1)[0], full[b])
        else:
            # The stream partition spans the batch, so the rounding of the
            # partial merge may differ between the batch and the lone sequence;
            # leakage between sequences would be far larger.
            alone = H.out_f32(w1, o1)[0]
            err = np.abs(alone - H.out_f32(w, out)[b]).max()
            assert err <= 1e-2 * np.abs(alone).max() + 1e-3, (b, err)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_attention_fixed_split_size_is_batch_invariant(dtype):
    """With split_keys fixed, a sequence's output is bitwise the same in a
    ragged batch (a grid sized for a larger bound, a skipped empty sequence
    beside it) as computed alone: batching must not change a sequence's
    output (Batch Speculative Decoding Done Right, ko summary, section 4).
    The batch is also checked against the oracle.  Without split_keys a
    batch of 40 sequences of 4000 keys gets 640-key splits and a lone such
    sequence 256-key ones, so the fixed size is what makes the bits agree."""
    w = _small_w(1, B=5, dtype=dtype, Hq=8, Hkv=2, D=128 if dtype == "bf16" else 64, M=16)
    lens = np.array([2100, 1, 700, 0, 1333], np.int32)
    q, kc, vc, kt, vt, par, lens = _attn_case(w, lens, 2300, 7400)
    for sk in (64, 512):
        rc, out, mk, ost, _ = _run_attn(w, q, kc, vc, kt, vt, par, lens, lmax_bound=2300, split_keys=sk)
        assert rc == 0
        full = H.from_dev(out)
        _, ref = oracle.attention(wl.as_f32(w, q), wl.as_f32(w, kc), wl.as_f32(w, vc), wl.as_f32(w, kt),
                                  wl.as_f32(w, vt), mk, lens, 2100, ost)
        H.check_attention(w, H.out_f32(w, out), ref, f"split-keys-{sk}")
        for b in range(len(lens)):
            L = int(lens[b])
            sl = slice(2100 - L, 2100) if L else slice(0, 1)  # an empty prefix: one unread column
            w1 = _small_w(1, B=1, dtype=dtype, Hq=8, Hkv=2, D=w.D, M=16)
            rc1, o1, _, _, _ = _run_attn(w1, q[b:b + 1], np.ascontiguousarray(kc[b:b + 1, :, sl]),
                                         np.ascontiguousarray(vc[b:b + 1, :, sl]), kt[b:b + 1], vt[b:b + 1],
                                         par[b:b + 1], lens[b:b + 1], split_keys=sk)
            assert rc1 == 0 and np.array_equal(H.from_dev(o1)[0], full[b]), (sk, b)
    # the property needs a fixed size: the shape-derived ones differ with the
    # batch (split count from the partials' workspace, [B][Hkv][splits][R][D + 2] fp32)
    def splits(B_):
        a = svt.AttnArgs()
        a.B, a.M, a.Hq, a.Hkv, a.D, a.dtype, a.cap, a.lmax_bound = B_, 16, 8, 2, 128, svt.SVT_BF16, 4000, 4000
        a.form = svt.SVT_ATTN_SPLIT
        return svt.svt_verify_attention_workspace(a) // (B_ * 2 * 68 * 130 * 4)
    assert (splits(40), splits(1)) == (7, 16)


def test_verify_round_split_keys_matches_direct_call():
    """VerifyRound(attn_split_keys=K) runs the same attention as a direct
    svt_verify_attention call with split_keys=K: identical bits."""
    from tree_masked_verification_parent_amd.round import VerifyRound
    w = _small_w(1, B=3, dtype="bf16", Hq=8, Hkv=2, D=128, M=16)
    cap = 1000
    q, kc, vc, kt, vt, par, lens = _attn_case(w, np.array([900, 17, 400], np.int32), cap, 7600)
    rc, ref, _, _, _ = _run_attn(w, q, kc, vc, kt, vt, par, lens, lmax_bound=cap, split_keys=512)
    assert rc == 0
    r = VerifyRound(w.B, w.M, w.Hq, w.Hkv, w.D, 64, cap, 1, torch.bfloat16, attn_split_keys=512)
    r.q[0].copy_(H.to_dev(q))
    r.kv_main[0, 0].copy_(H.to_dev(kc))
    r.kv_main[0, 1].copy_(H.to_dev(vc))
    r.kv_branch[0, 0].copy_(H.to_dev(kt))
    r.kv_branch[0, 1].copy_(H.to_dev(vt))
    r.parents.copy_(torch.from_numpy(par))
    r.len.copy_(torch.from_numpy(lens))
    r.lmax.fill_(int(lens.max()))
    r.set_lmax_bound(cap)
    assert r.build_mask() == 0 and r.attention(0) == 0
    torch.cuda.synchronize()
    assert np.array_equal(H.from_dev(r.out[0]), H.from_dev(ref))


def test_attention_split_keys_arguments():
    """split_keys must be 0 or a positive multiple of 64, and selects the split
    form: with SVT_ATTN_STREAM it is an argument error, found before any launch."""
    w = _small_w(1, B=2, dtype="bf16", Hq=8, Hkv=2, D=128, M=8)
    lens = np.array([300, 200], np.int32)
    q, kc, vc, kt, vt, par, lens = _attn_case(w, lens, 320, 7500)
    for sk, form in ((100, svt.SVT_ATTN_AUTO), (-64, svt.SVT_ATTN_SPLIT), (256, svt.SVT_ATTN_STREAM)):
        rc, out, _, _, sst = _run_attn(w, q, kc, vc, kt, vt, par, lens, form=form, split_keys=sk)
        assert rc == svt.SVT_ERR_ARG, (sk, form, rc)
    rc, _, _, _, sst = _run_attn(w, q, kc, vc, kt, vt, par, lens, split_keys=256)  # AUTO: the split form
    assert rc == 0 and (sst == 0).all()


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_attention_invalid_sequences_and_length_errors(form):
    w = _small_w(1, B=3, dtype="bf16", Hq=8, Hkv=2, D=128, M=10)  # 44 query rows per KV head: 3 tiles
    lens = np.array([300, 200, 100], np.int32)
    q, kc, vc, kt, vt, par, lens = _attn_case(w, lens, 320, 7300)
    st = np.array([0, -5, 0], np.int32)
    rc, out, mk, _, sst = _run_attn(w, q, kc, vc, kt, vt, par, lens, status=st, form=form)
    got = H.out_f32(w, out)
    assert rc == 0 and sst.tolist() == [0, -5, 0] and not got[1].any()
    _, ref = oracle.attention(wl.as_f32(w, q), wl.as_f32(w, kc), wl.as_f32(w, vc), wl.as_f32(w, kt),
                              wl.as_f32(w, vt), mk, lens, 300, st)
    H.check_attention(w, got, ref, "invalid-status")
    # device lmax above the host bound: the sequence is refused, not read out of range
    rc, out, _, _, sst = _run_attn(w, q, kc, vc, kt, vt, par, lens, lmax_bound=250, form=form)
    assert rc == 0 and (sst == svt.SVT_ERR_LENGTH).all() and not H.out_f32(w, out).any()


def test_workspace_missing_small_or_misaligned_is_rejected():
    """Attention needs a 16-byte aligned workspace of svt_verify_attention_workspace
    bytes and accept an 8-byte aligned one of svt_accept_workspace bytes; anything
    else returns SVT_ERR_WORKSPACE before a kernel is launched."""
    w = _small_w(1, B=2, dtype="bf16", Hq=8, Hkv=2, D=128, M=8)
    q, kc, vc, kt, vt, par, lens = _attn_case(w, [300, 41], 340, 7450)
    tq = H.to_dev(q)
    mk = torch.zeros(2, 9, 1, dtype=torch.int64, device=DEV)
    dp = torch.zeros(2, 9, dtype=torch.int32, device=DEV)
    st = torch.zeros(2, dtype=torch.int32, device=DEV)
    assert svt.svt_build_mask(_i32(par), 8, mk, dp, st) == 0
    out = torch.empty_like(tq)
    a = svt.attn_args(tq, H.to_dev(kc), H.to_dev(vc), _i32(lens), _i32([300]), 300, H.to_dev(kt), H.to_dev(vt),
                      mk, out, status=st, form=svt.SVT_ATTN_STREAM)
    need = svt.svt_verify_attention_workspace(a)
    assert need > 0
    ws = torch.empty(need + 64, dtype=torch.uint8, device=DEV)
    base = ws.data_ptr()
    print("attention workspace checks", flush=True)
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_WORKSPACE  # none
    a.workspace, a.workspace_bytes = base, need - 1
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_WORKSPACE  # too small
    a.workspace, a.workspace_bytes = base + 8, need
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_WORKSPACE  # 8-byte aligned only
    a.workspace, a.workspace_bytes = base + 16, need
    assert svt.svt_verify_attention(a) == svt.SVT_OK
    torch.cuda.synchronize()

    logits = np.random.default_rng(7451).standard_normal((2, 9, 1000)).astype(np.float32)
    lg = torch.as_tensor(logits, device=DEV)
    tk = _i32(np.zeros((2, 9)))
    am, path = (torch.zeros(2, 9, dtype=torch.int32, device=DEV) for _ in range(2))
    al, bo = (torch.zeros(2, dtype=torch.int32, device=DEV) for _ in range(2))
    acc = svt.accept_args(lg, tk, _i32(par), mk, dp, am, al, path, bo, status=st)
    need = svt.svt_accept_workspace(acc)
    wsa = torch.empty(need + 64, dtype=torch.uint8, device=DEV)
    base = wsa.data_ptr()
    print("accept workspace checks", flush=True)
    assert svt.svt_accept(acc) == svt.SVT_ERR_WORKSPACE
    acc.workspace, acc.workspace_bytes = base, need - 1
    assert svt.svt_accept(acc) == svt.SVT_ERR_WORKSPACE
    acc.workspace, acc.workspace_bytes = base + 4, need
    assert svt.svt_accept(acc) == svt.SVT_ERR_WORKSPACE
    acc.workspace, acc.workspace_bytes = base + 8, need
    assert svt.svt_accept(acc) == svt.SVT_OK
    torch.cuda.synchronize()
    al_ref, _, _ = oracle.accept(oracle.argmax(logits), np.zeros((2, 9), np.int32), par, 8, np.zeros(2, np.int32))
    assert np.array_equal(H.from_dev(al), al_ref)


def test_attention_host_argument_errors():
    w = _small_w(1, B=1, dtype="bf16", Hq=4, Hkv=2, D=128, M=4)
    q, kc, vc, kt, vt, par, lens = _attn_case(w, [10], 16, 7400)
    tq = H.to_dev(q)
    args = svt.attn_args(tq, H.to_dev(kc), H.to_dev(vc), _i32(lens), _i32([10]), 10, H.to_dev(kt),
                         H.to_dev(vt), torch.zeros(1, 5, 1, dtype=torch.int64, device=DEV), torch.empty_like(tq))
    a = args
    a.D = 96
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_UNSUPPORTED
    a.D = 128
    a.Hq = 3
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_ARG
    a.Hq = 4
    a.lmax_bound = 17
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_ARG
    a.lmax_bound = 10
    a.form = 7
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_ARG
    a.form = svt.SVT_ATTN_STREAM  # the stream form is bf16 only
    a.dtype = svt.SVT_FP32
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_UNSUPPORTED
    a.dtype = svt.SVT_BF16
    a.form = 0
    a.q = None
    assert svt.svt_verify_attention(a) == svt.SVT_ERR_ARG
