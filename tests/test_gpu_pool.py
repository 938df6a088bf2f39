"""GPU parity of cross-batch scheduling: the append-only commit, the slot map
of commit and attention, and the realignment, against the CPU oracle on
seeded inputs.  Cache bytes, tokens, position ids, lengths and statuses must
match bit for bit; attention must meet the tolerance of tests/harness.py."""
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


def _pool(rows, Hkv, L, D, cap, esize, seed):
    el = D * esize // 2
    slab = np.arange(L * 2 * rows * Hkv).reshape(L, 2, rows, Hkv, 1, 1) + seed
    km = gen.commit_pattern_bits(slab, np.arange(cap).reshape(1, 1, 1, 1, cap, 1), np.arange(el).reshape(1, 1, 1, 1, 1, el))
    tm = gen.randint(gen.stream_key(seed, 3), rows * cap, 0, 10 ** 6).astype(np.int32).reshape(rows, cap)
    return km, tm


def _round_inputs(B, Hkv, L, M, D, esize, seed):
    T = M + 1
    el = D * esize // 2
    slab = np.arange(L * 2 * B * Hkv).reshape(L, 2, B, Hkv, 1, 1) + 50000 + seed
    kb = gen.commit_pattern_bits(slab, np.arange(T).reshape(1, 1, 1, 1, T, 1), np.arange(el).reshape(1, 1, 1, 1, 1, el))
    trees = np.stack([gen.tree_depth_capped(gen.stream_key(seed, 9, b), M, 8) for b in range(B)]).astype(np.int32)
    am = gen.randint(gen.stream_key(seed, 1), B * T, 0, 1).astype(np.int32).reshape(B, T)
    tok = gen.randint(gen.stream_key(seed, 2), B * T, 0, 1).astype(np.int32).reshape(B, T)
    al, path, _ = oracle.accept(am, tok, trees, M)
    return kb, tok, al, path


def _dev_rows(x, D, esize):
    dt = torch.float32 if esize == 4 else torch.bfloat16
    return torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(dt).reshape(x.shape[:5] + (D,))


def _host_rows(t, shape):
    return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(shape)


def _run_commit(km, kb, tm, tok, lens, lmax, path, al, D, esize, mode, slot=None, status=None):
    km_t, kb_t = _dev_rows(km, D, esize), _dev_rows(kb, D, esize)
    rows, cap = tm.shape
    tm_t, ln_t, lm_t = _i32(tm), _i32(lens), _i32([lmax])
    pos = torch.full((rows, cap), -3, dtype=torch.int32, device=DEV)
    cst = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    args = svt.commit_args(km_t, kb_t, ln_t, lm_t, _i32(path), _i32(al), cst, tokens_main=tm_t, tree_tokens=_i32(tok),
                           pos_ids=pos, status=None if status is None else _i32(status),
                           seq_slot=None if slot is None else _i32(slot), mode=mode)
    rc = svt.svt_commit(args)
    torch.cuda.synchronize()
    return (rc, _host_rows(km_t, km.shape), H.from_dev(tm_t), H.from_dev(ln_t), int(H.from_dev(lm_t)[0]),
            H.from_dev(pos), int(H.from_dev(cst)[0]))


def _starts_ends(mode, lens, lmax, ln2, lm2):
    """(start, end) of each sequence's content after the commit."""
    if mode == svt.SVT_COMMIT_APPEND:
        st = lmax - np.asarray(lens)
        return st, st + ln2
    return lm2 - ln2, np.full(len(ln2), lm2)


@pytest.mark.parametrize("mode", [svt.SVT_COMMIT_REPAD, svt.SVT_COMMIT_APPEND], ids=["repad", "append"])
@pytest.mark.parametrize("esize,D", [(2, 128), (4, 64)])
def test_commit_modes_with_slots(mode, esize, D):
    B, rows, Hkv, L, M = 4, 7, 2, 2, 24
    lens = np.array([1500, 3, 0, 1500], np.int32)
    lmax, cap = 1500, 1560
    km, tm = _pool(rows, Hkv, L, D, cap, esize, 11)
    kb, tok, al, path = _round_inputs(B, Hkv, L, M, D, esize, 12)
    slot = np.array([5, 0, 3, 6], np.int32)
    print(f"commit mode={mode} esize={esize} D={D}", flush=True)
    rc, gkm, gtm, gln, glm, gpos, gcst = _run_commit(km, kb, tm, tok, lens, lmax, path, al, D, esize, mode, slot)
    orc, okm, otm, oln, olm, opos = oracle.commit(km, kb, M, tm, tok, lens, lmax, path, al, mode=mode, slot=slot)
    assert rc == 0 and gcst == orc == 0
    assert np.array_equal(gln, oln) and glm == olm
    starts, ends = _starts_ends(mode, lens, lmax, oln, olm)
    for b, r in enumerate(slot):
        s, e = starts[b], ends[b]
        assert np.array_equal(gkm[:, :, r, :, s:e], okm[:, :, r, :, s:e]), f"kv b={b}"
        assert np.array_equal(gtm[r, s:e], otm[r, s:e]) and np.array_equal(gpos[r, :e], opos[r, :e]), f"b={b}"
        assert (gpos[r, e:] == -3).all()
        assert np.array_equal(gkm[:, :, r, :, e:], km[:, :, r, :, e:])        # past the new end untouched
    for r in sorted(set(range(rows)) - set(slot.tolist())):                  # rows outside the batch
        assert np.array_equal(gkm[:, :, r], km[:, :, r]) and np.array_equal(gtm[r], tm[r])
        assert (gpos[r] == -3).all()


def test_commit_append_equal_length_batch_moves_nothing():
    """An equal-length batch (the EXSPEC case): content bytes are untouched."""
    B, rows, Hkv, L, M, D = 6, 6, 4, 3, 32, 128
    lens = np.full(B, 2048, np.int32)
    km, tm = _pool(rows, Hkv, L, D, 2100, 2, 13)
    kb, tok, al, path = _round_inputs(B, Hkv, L, M, D, 2, 14)
    rc, gkm, gtm, gln, glm, gpos, gcst = _run_commit(km, kb, tm, tok, lens, 2048, path, al, D, 2,
                                                     svt.SVT_COMMIT_APPEND)
    assert rc == 0 and gcst == 0 and glm == 2048 + int(al.max()) + 1
    assert np.array_equal(gkm[..., :2048, :], km[..., :2048, :])
    for b in range(B):
        A = int(al[b]) + 1
        assert np.array_equal(gkm[:, :, b, :, 2048:2048 + A], kb[:, :, b][:, :, :, path[b, :A]])
        assert gpos[b, :2048 + A].tolist() == list(range(2048 + A))


def test_commit_slot_and_capacity_errors_write_nothing():
    B, rows, Hkv, L, M, D = 3, 4, 1, 1, 10, 64
    lens = np.array([50, 60, 55], np.int32)
    km, tm = _pool(rows, Hkv, L, D, 64, 2, 15)
    kb, tok, al, path = _round_inputs(B, Hkv, L, M, D, 2, 16)
    for mode, slot, acc, want in [(svt.SVT_COMMIT_APPEND, [0, 4, 1], al, oracle.ERR_ARG),
                                  (svt.SVT_COMMIT_REPAD, [0, -1, 1], al, oracle.ERR_ARG),
                                  (svt.SVT_COMMIT_REPAD, [1, 3, 1], al, oracle.ERR_ARG),     # row 1 twice
                                  (svt.SVT_COMMIT_APPEND, [2, 2, 0], al, oracle.ERR_ARG),    # row 2 twice
                                  (svt.SVT_COMMIT_APPEND, [0, 2, 1], np.array([0, 4, 0], np.int32),
                                   oracle.ERR_CAPACITY)]:
        slot = np.array(slot, np.int32)
        rc, gkm, gtm, gln, glm, gpos, gcst = _run_commit(km, kb, tm, tok, lens, 60, path, acc, D, 2, mode, slot)
        orc = oracle.commit(km, kb, M, tm, tok, lens, 60, path, acc, mode=mode, slot=slot)[0]
        assert rc == 0 and gcst == orc == want
        assert np.array_equal(gkm, km) and np.array_equal(gtm, tm) and gln.tolist() == lens.tolist() and glm == 60
        assert (gpos == -3).all()
    # host checks: unknown mode, slot map without a pool size
    km_t, kb_t = _dev_rows(km, D, 2), _dev_rows(kb, D, 2)
    args = svt.commit_args(km_t, kb_t, _i32(lens), _i32([60]), _i32(path), _i32(al), _i32([0]),
                           seq_slot=_i32([0, 1, 2]), mode=5)
    assert svt.svt_commit(args) == svt.SVT_ERR_ARG
    args.mode, args.n_slots = 0, 0
    assert svt.svt_commit(args) == svt.SVT_ERR_ARG


def test_commit_slots_with_equal_residue_are_distinct():
    """The device's duplicate check hashes slots into a 32768-bit table; slots
    that share a bit but differ are accepted, a slot named twice is not."""
    B, Hkv, L, M, D, cap = 3, 1, 1, 6, 64, 16
    rows = 32768 + 8
    km, tm = _pool(rows, Hkv, L, D, cap, 2, 23)
    kb, tok, al, path = _round_inputs(B, Hkv, L, M, D, 2, 24)
    lens = np.array([5, 0, 3], np.int32)
    for slot, want in [([5, 5 + 32768, 7], 0), ([5, 5 + 32768, 5 + 32768], oracle.ERR_ARG)]:
        slot = np.array(slot, np.int32)
        print(f"commit slots {slot.tolist()}", flush=True)
        rc, gkm, gtm, gln, glm, gpos, gcst = _run_commit(km, kb, tm, tok, lens, 5, path, al, D, 2,
                                                         svt.SVT_COMMIT_REPAD, slot)
        orc, okm, otm, oln, olm, opos = oracle.commit(km, kb, M, tm, tok, lens, 5, path, al, slot=slot)
        assert rc == 0 and gcst == orc == want
        if want:
            assert np.array_equal(gkm, km) and np.array_equal(gtm, tm) and (gpos == -3).all()
            continue
        assert np.array_equal(gln, oln) and glm == olm
        for b, r in enumerate(slot):
            s0 = olm - oln[b]
            assert np.array_equal(gkm[:, :, r, :, s0:olm], okm[:, :, r, :, s0:olm])
            assert np.array_equal(gtm[r, s0:olm], otm[r, s0:olm]) and np.array_equal(gpos[r, :olm], opos[r, :olm])


def _run_realign(km, tm, lens, ends, D, esize, slot=None):
    km_t = _dev_rows(km, D, esize)
    rows, cap = tm.shape
    tm_t = _i32(tm)
    pos = torch.full((rows, cap), -3, dtype=torch.int32, device=DEV)
    lm = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    rst = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    args = svt.realign_args(km_t, _i32(lens), _i32(ends), lm, rst, tokens_main=tm_t, pos_ids=pos,
                            seq_slot=None if slot is None else _i32(slot))
    rc = svt.svt_realign(args)
    torch.cuda.synchronize()
    return rc, _host_rows(km_t, km.shape), H.from_dev(tm_t), int(H.from_dev(lm)[0]), H.from_dev(pos), int(H.from_dev(rst)[0])


@pytest.mark.parametrize("esize,D", [(2, 128), (4, 128), (2, 64)])
def test_realign_parity(esize, D):
    rows, Hkv, L, cap = 6, 2, 2, 4400
    km, tm = _pool(rows, Hkv, L, D, cap, esize, 17)
    lens = np.array([4000, 12, 0, 3000, 4100], np.int32)      # moves of 0, a few rows and many 16 KB chunks
    ends = np.array([4100, 3000, 7, 3000, 4100], np.int32)
    slot = np.array([2, 5, 0, 1, 4], np.int32)
    print(f"realign esize={esize} D={D}", flush=True)
    rc, gkm, gtm, glm, gpos, grs = _run_realign(km, tm, lens, ends, D, esize, slot)
    orc, okm, otm, olm, opos = oracle.realign(km, lens, ends, tokens_main=tm, slot=slot)
    assert rc == 0 and grs == orc == 0 and glm == olm == 4100
    for b, r in enumerate(slot):
        s = olm - lens[b]
        assert np.array_equal(gkm[:, :, r, :, s:olm], okm[:, :, r, :, s:olm]), f"kv b={b}"
        assert np.array_equal(gtm[r, s:olm], otm[r, s:olm]) and np.array_equal(gpos[r, :olm], opos[r, :olm])
        assert np.array_equal(gkm[:, :, r, :, olm:], km[:, :, r, :, olm:])
    assert np.array_equal(gkm[:, :, 3], km[:, :, 3]) and (gpos[3] == -3).all()   # row not in the batch


def test_realign_errors_write_nothing():
    rows, Hkv, L, D, cap = 3, 1, 1, 64, 40
    km, tm = _pool(rows, Hkv, L, D, cap, 2, 19)
    lens = np.array([5, 9, 2], np.int32)
    for ends, slot, want in [([5, 41, 3], None, oracle.ERR_LENGTH), ([4, 20, 3], None, oracle.ERR_LENGTH),
                             ([5, 20, 3], [0, 3, 1], oracle.ERR_ARG), ([5, 20, 3], [2, 0, 2], oracle.ERR_ARG)]:
        sl = None if slot is None else np.array(slot, np.int32)
        rc, gkm, gtm, glm, gpos, grs = _run_realign(km, tm, lens, np.array(ends, np.int32), D, 2, sl)
        orc = oracle.realign(km, lens, ends, tokens_main=tm, slot=sl)[0]
        assert rc == 0 and grs == orc == want
        assert np.array_equal(gkm, km) and np.array_equal(gtm, tm) and (gpos == -3).all() and glm == -1


@pytest.mark.parametrize("form", [svt.SVT_ATTN_SPLIT, svt.SVT_ATTN_STREAM], ids=["split", "stream"])
def test_attention_seq_slot(form):
    """Cache rows taken through the slot map equal the gathered batch."""
    import dataclasses
    w = dataclasses.replace(wl.workload(1), B=3, Hq=8, Hkv=2, M=32)
    lens = np.array([1200, 77, 513], np.int32)
    lmax, cap, rows = 1200, 1240, 5
    q, kc, vc, kt, vt = wl.attention_inputs(w, lens, cap, 8100)
    par = wl.trees(w, 8100)
    slot = np.array([3, 0, 4], np.int32)
    pk = np.full((rows,) + kc.shape[1:], wl.poison_value(w), kc.dtype)
    pv = np.full((rows,) + vc.shape[1:], wl.poison_value(w), vc.dtype)
    pk[slot], pv[slot] = kc, vc
    T = w.T
    mk = torch.zeros(w.B, T, 1, dtype=torch.int64, device=DEV)
    dp = torch.zeros(w.B, T, dtype=torch.int32, device=DEV)
    st = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    assert svt.svt_build_mask(_i32(par), w.M, mk, dp, st) == 0
    tq, tk, tv, tkt, tvt = (H.to_dev(x) for x in (q, pk, pv, kt, vt))
    out = torch.full(tq.shape, float("nan"), dtype=tq.dtype, device=DEV)
    sst = torch.full((w.B,), 55, dtype=torch.int32, device=DEV)
    sl_t, ln_t, lm_t = _i32(slot), _i32(lens), _i32([lmax])   # the args hold raw pointers: keep these alive
    args = svt.attn_args(tq, tk, tv, ln_t, lm_t, lmax, tkt, tvt, mk, out, status=st, seq_status=sst, form=form,
                         seq_slot=sl_t)
    ws = torch.empty(max(1, svt.svt_verify_attention_workspace(args)), dtype=torch.uint8, device=DEV)
    args = svt.attn_args(tq, tk, tv, ln_t, lm_t, lmax, tkt, tvt, mk, out, status=st, seq_status=sst, form=form,
                         seq_slot=sl_t, workspace=ws)
    print(f"attention seq_slot form={form}", flush=True)
    assert svt.svt_verify_attention(args) == 0
    torch.cuda.synchronize()
    assert (H.from_dev(sst) == 0).all()
    f = lambda x: wl.as_f32(w, x)
    _, ost = oracle.validate(par, w.M)
    omk, _ = oracle.mask(par, w.M, ost)
    assert np.array_equal(H.from_dev(mk).view(np.uint64), omk) and np.array_equal(H.from_dev(st), ost)
    orc, ref = oracle.attention(f(q), f(kc), f(vc), f(kt), f(vt), omk, lens, lmax, ost)
    H.check_attention(w, H.out_f32(w, out), ref, f"seq_slot form={form}")
    # a slot outside the pool (on the long sequence, which the split form cuts
    # into several key splits): it reports SVT_ERR_ARG and gets zeros; the
    # others are unchanged
    good = H.out_f32(w, out)
    bad = _i32([rows, 0, 4])
    sl_t.copy_(bad)
    assert svt.svt_verify_attention(args) == 0
    torch.cuda.synchronize()
    assert H.from_dev(sst).tolist() == [svt.SVT_ERR_ARG, 0, 0]
    got = H.out_f32(w, out)
    assert not got[0].any()
    for b in (1, 2):
        assert np.abs(got[b] - good[b]).max() <= 1e-2 * max(1.0, np.abs(good[b]).max()) + 1e-3


def test_exspec_rounds_match_oracle():
    """Several scheduling rounds through SequencePool / PoolRound (equal-length
    batches appended, mixed batches realigned and re-padded) leave the pool
    exactly as the oracle replaying the same decisions."""
    from tree_masked_verification_parent_amd.sched import PoolRound, SequencePool
    P, B, L, Hkv, D, M, V, cap = 10, 4, 2, 2, 64, 8, 64, 160
    T = M + 1
    pool = SequencePool(P, Hkv, D, L, cap, torch.bfloat16)
    km, tm = _pool(P, Hkv, L, D, cap, 2, 21)
    pool.kv.copy_(_dev_rows(km, D, 2))
    pool.tokens.copy_(_i32(tm))
    lens0 = [20, 20, 20, 33, 33, 7, 20, 33, 12, 12]
    for s, n in enumerate(lens0):
        pool.place(s, n)
    pr = PoolRound(pool, B, M, 4, V, attn_layers=1)
    opos = np.zeros((P, cap), np.int32)
    kinds = []
    for rnd in range(8):
        same, slots = pool.pick(B, 3)
        n = len(slots)
        seed = 9300 + rnd
        trees = np.stack([gen.tree_depth_capped(gen.stream_key(seed, 5, b), M, 5) for b in range(n)]).astype(np.int32)
        logits, des = gen.logits_with_designated_top(gen.stream_key(seed, 6), n * T, V)
        des = des.reshape(n, T)
        tok = np.stack([gen.plant_drafts(gen.stream_key(seed, 7, b), trees[b], des[b], V, 0.8)
                        for b in range(n)]).astype(np.int32)
        el = D
        bsl = np.arange(L * 2 * n * Hkv).reshape(L, 2, n, Hkv, 1, 1) + 70000 + 100 * rnd
        kb = gen.commit_pattern_bits(bsl, np.arange(T).reshape(1, 1, 1, 1, T, 1), np.arange(el).reshape(1, 1, 1, 1, 1, el))
        pr.parents[:n].copy_(_i32(trees))
        pr.tree_tokens[:n].copy_(_i32(tok))
        pr.logits[:n].copy_(torch.from_numpy(logits.reshape(n, T, V)).to(DEV))
        pr.kv_branch(n).copy_(_dev_rows(kb, D, 2))
        pr.load_batch(slots)
        lens_b, ends_b = pool.len[slots].copy(), pool.end[slots].copy()
        print(f"round {rnd}: slots {slots.tolist()} equal_ends={same} lens {lens_b.tolist()} ends {ends_b.tolist()}",
              flush=True)
        if not same:
            E = pool.realign(slots, pr.slot[:n], pr.len[:n], pr.end[:n])
            orc, km, tm, oE, pos = oracle.realign(km, lens_b, ends_b, tokens_main=tm, slot=slots)
            assert orc == 0 and oE == E
            opos[slots] = pos[slots]
        else:
            E = int(ends_b[0])
        assert pr.verify(n, E) == 0
        mode = svt.SVT_COMMIT_APPEND if same else svt.SVT_COMMIT_REPAD
        assert pr.commit(n, mode) == 0
        torch.cuda.synchronize()
        assert pr.commit_status.item() == 0
        al = H.from_dev(pr.accept_len[:n])
        oal, opath, _ = oracle.accept(oracle.argmax(logits.reshape(n, T, V)), tok, trees, M)
        assert np.array_equal(al, oal) and np.array_equal(H.from_dev(pr.path[:n]), opath)
        orc, km, tm, oln, olm, pos = oracle.commit(km, kb, M, tm, tok, lens_b, E, opath, oal, mode=mode, slot=slots)
        assert orc == 0
        opos[slots] = pos[slots]
        pool.committed(slots, al, E, mode)
        assert np.array_equal(pool.len[slots], oln)
        kinds.append(mode)
    assert svt.SVT_COMMIT_APPEND in kinds and svt.SVT_COMMIT_REPAD in kinds   # both paths were taken
    gkm = _host_rows(pool.kv, km.shape)
    gtm, gpos = H.from_dev(pool.tokens), H.from_dev(pool.pos)
    for s in range(P):
        a, e = pool.end[s] - pool.len[s], pool.end[s]
        assert np.array_equal(gkm[:, :, s, :, a:e], km[:, :, s, :, a:e]), f"slot {s}"
        assert np.array_equal(gtm[s, a:e], tm[s, a:e]), f"tokens slot {s}"
        if a or e != lens0[s]:   # rows that some call wrote position ids for
            assert np.array_equal(gpos[s, :e], opos[s, :e]), f"pos slot {s}"


def test_pool_calls_degenerate_shapes():
    """Empty batches, zero-length contents and a single-node tree."""
    D, Hkv, L, cap = 64, 1, 1, 32
    km, tm = _pool(3, Hkv, L, D, cap, 2, 23)
    # realign of an empty batch: nothing moves, the common end is 0
    km_t = _dev_rows(km, D, 2)
    lm = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    rst = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    e32 = torch.zeros(0, dtype=torch.int32, device=DEV)
    args = svt.realign_args(km_t[:, :, :0], e32, e32, lm, rst)
    assert svt.svt_realign(args, svt.SVT_SYNC_CHECK) == 0
    assert int(H.from_dev(lm)[0]) == 0 and int(H.from_dev(rst)[0]) == 0
    # realign where every content is empty: ends move, no bytes do
    rc, gkm, gtm, glm, gpos, grs = _run_realign(km, tm, np.array([0, 0], np.int32), np.array([5, 9], np.int32), D, 2,
                                                np.array([2, 0], np.int32))
    assert rc == 0 and grs == 0 and glm == 9 and np.array_equal(gkm, km) and np.array_equal(gtm, tm)
    assert (gpos[[0, 2], :9] == 0).all()
    # append commit with M = 0 (a tree of the root alone) on zero-length contents
    M = 0
    kb = gen.commit_pattern_bits(np.arange(2 * 2).reshape(1, 2, 2, 1, 1, 1) + 777,
                                 np.arange(1).reshape(1, 1, 1, 1, 1, 1), np.arange(D).reshape(1, 1, 1, 1, 1, D))
    tok = np.array([[5], [6]], np.int32)
    lens = np.array([0, 0], np.int32)
    al = np.zeros(2, np.int32)
    path = np.zeros((2, 1), np.int32)
    slot = np.array([1, 2], np.int32)
    rc, gkm, gtm, gln, glm, gpos, gcst = _run_commit(km, kb, tm, tok, lens, 0, path, al, D, 2, svt.SVT_COMMIT_APPEND,
                                                     slot)
    orc, okm, otm, oln, olm, opos = oracle.commit(km, kb, M, tm, tok, lens, 0, path, al, mode=1, slot=slot)
    assert rc == 0 and gcst == orc == 0 and gln.tolist() == oln.tolist() == [1, 1] and glm == olm == 1
    for b, r in enumerate(slot):
        assert np.array_equal(gkm[:, :, r, :, :1], okm[:, :, r, :, :1]) and gtm[r, 0] == otm[r, 0] == tok[b, 0]
        assert gpos[r, 0] == 0


def test_commit_empty_batch_is_a_no_op():
    """B = 0: nothing moves; re-pad leaves lmax 0, append keeps it (as the oracle)."""
    D = 64
    km = torch.zeros(1, 2, 0, 1, 8, D, dtype=torch.bfloat16, device=DEV)
    kb = torch.zeros(1, 2, 0, 1, 3, D, dtype=torch.bfloat16, device=DEV)
    e32 = torch.zeros(0, dtype=torch.int32, device=DEV)
    for mode in (svt.SVT_COMMIT_REPAD, svt.SVT_COMMIT_APPEND):
        lm = _i32([4])
        cst = torch.full((1,), 77, dtype=torch.int32, device=DEV)
        args = svt.commit_args(km, kb, e32, lm, torch.zeros(0, 3, dtype=torch.int32, device=DEV), e32, cst, mode=mode)
        assert svt.svt_commit(args, svt.SVT_SYNC_CHECK) == 0
        orc, _, _, _, olm, _ = oracle.commit(np.zeros((1, 2, 0, 1, 8, D), np.uint16), np.zeros((1, 2, 0, 1, 3, D), np.uint16),
                                             2, None, np.zeros((0, 3), np.int32), [], 4, np.zeros((0, 3), np.int32),
                                             np.zeros(0, np.int32), mode=mode)
        assert int(H.from_dev(cst)[0]) == orc == 0 and int(H.from_dev(lm)[0]) == olm
