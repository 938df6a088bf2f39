"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark uses.

- mask, argmax and accept: every output, bit for bit;
- attention (one layer): every row of every workload, each recomputed by the
  oracle from the oracle's own mask (the GPU's mask must equal it), plus
  finite output although the padding holds NaN and bitwise run-to-run
  determinism;
- commit (all layers): a sample of (layer, KV head) slabs, plane K and V,
  against the oracle, plus tokens, position ids, lengths; columns beyond the
  new length untouched.
"""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from synth import gen
from synth import workloads as wl
from tree_masked_verification_parent_amd import svt

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"
WIDS = list(range(len(wl.WORKLOADS)))


def _i32(x):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=DEV)


def _mask_on_gpu(w, parents):
    mk = torch.zeros(w.B, w.T, w.W, dtype=torch.int64, device=DEV)
    dp = torch.zeros(w.B, w.T, dtype=torch.int32, device=DEV)
    st = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    assert svt.svt_build_mask(_i32(parents), w.M, mk, dp, st, svt.SVT_SYNC_CHECK) == 0
    return mk, dp, st


@pytest.mark.parametrize("wi", WIDS, ids=[w.name for w in wl.WORKLOADS])
def test_workload_mask_and_accept(wi):
    w = wl.workload(wi)
    print(f"[{w.name}] mask + accept", flush=True)
    parents = wl.trees(w)
    logits, tokens, _ = wl.logits_and_drafts(w, parents)
    mk, dp, st = _mask_on_gpu(w, parents)
    _, ost = oracle.validate(parents, w.M)
    omk, odp = oracle.mask(parents, w.M, ost)
    assert np.array_equal(H.from_dev(mk).view(np.uint64), omk) and np.array_equal(H.from_dev(dp), odp)
    am = torch.zeros(w.B, w.T, dtype=torch.int32, device=DEV)
    al = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    path = torch.zeros(w.B, w.T, dtype=torch.int32, device=DEV)
    bo = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    lg = torch.from_numpy(logits).to(DEV)
    args = svt.accept_args(lg, _i32(tokens), _i32(parents), mk, dp, am, al, path, bo, status=st)
    ws = torch.empty(svt.svt_accept_workspace(args), dtype=torch.uint8, device=DEV)
    args = svt.accept_args(lg, _i32(tokens), _i32(parents), mk, dp, am, al, path, bo, status=st, workspace=ws)
    assert svt.svt_accept(args) == 0
    torch.cuda.synchronize()
    oam = oracle.argmax(logits)
    oal, opath, obo = oracle.accept(oam, tokens, parents, w.M, ost)
    assert np.array_equal(H.from_dev(am), oam)
    assert np.array_equal(H.from_dev(al), oal) and np.array_equal(H.from_dev(path), opath)
    assert np.array_equal(H.from_dev(bo), obo)
    print(f"[{w.name}] accept lengths {oal.tolist()[:8]} mean {oal.mean():.2f}", flush=True)


@pytest.mark.parametrize("wi", WIDS, ids=[w.name for w in wl.WORKLOADS])
def test_workload_attention(wi):
    w = wl.workload(wi)
    print(f"[{w.name}] attention inputs", flush=True)
    parents = wl.trees(w)
    lens = wl.lengths(w)
    lmax = int(lens.max())
    cap = lmax + 64
    q, kc, vc, kt, vt = wl.attention_inputs(w, lens, cap)      # padding columns hold NaN
    mk, dp, st = _mask_on_gpu(w, parents)
    # the oracle's own mask and status (the GPU's must equal them)
    _, ost = oracle.validate(parents, w.M)
    omk, _ = oracle.mask(parents, w.M, ost)
    assert np.array_equal(H.from_dev(mk).view(np.uint64), omk) and np.array_equal(H.from_dev(st), ost)
    tq, tkc, tvc, tkt, tvt = (H.to_dev(x) for x in (q, kc, vc, kt, vt))
    out = torch.full(tq.shape, float("nan"), dtype=tq.dtype, device=DEV)
    sst = torch.full((w.B,), 55, dtype=torch.int32, device=DEV)
    ln, lm = _i32(lens), _i32([lmax])
    args = svt.attn_args(tq, tkc, tvc, ln, lm, lmax, tkt, tvt, mk, out, status=st, seq_status=sst)
    ws = torch.empty(max(1, svt.svt_verify_attention_workspace(args)), dtype=torch.uint8, device=DEV)
    args = svt.attn_args(tq, tkc, tvc, ln, lm, lmax, tkt, tvt, mk, out, status=st, seq_status=sst, workspace=ws)
    print(f"[{w.name}] attention run", flush=True)
    assert svt.svt_verify_attention(args) == 0
    torch.cuda.synchronize()
    first = H.from_dev(out)
    assert svt.svt_verify_attention(args) == 0
    torch.cuda.synchronize()
    assert np.array_equal(H.from_dev(out), first), "not bitwise deterministic"
    assert (H.from_dev(sst) == 0).all()
    got = H.out_f32(w, out)
    assert np.isfinite(got).all(), "NaN padding leaked into the output"
    del tq, tkc, tvc, tkt, tvt
    # every row, each recomputed by the oracle (rows run side by side on the
    # host's cores); with the stream form this includes every row of the
    # units that range ends cut, which go through the partial merge
    rows = [(b, i, h) for b in range(w.B) for i in range(w.T) for h in range(w.Hq)]
    if w.dtype == "bf16" and w.B <= 1024:
        units = H.stream_units(w.B, w.T, w.Hq, w.Hkv, lens, H.cu_count(), D=w.D)
        print(f"[{w.name}] {sum(1 for u in units if u.cuts)} of {len(units)} stream units are cut", flush=True)
    print(f"[{w.name}] oracle on all {len(rows)} rows, {oracle.default_threads()} threads", flush=True)
    ref = oracle.attention_rows(q, kc, vc, kt, vt, omk, lens, lmax, rows, to_f32=lambda x: wl.as_f32(w, x))
    sel = got.reshape(-1, w.D)     # rows in (b, i, h) order
    err = H.check_attention(w, sel, ref, w.name)
    print(f"[{w.name}] max-abs error {err:.3e} over {len(rows)} rows", flush=True)


def _fill_pattern(t, slab_base_fn, ncol):
    """Fill t[L][2][B][Hkv][ncol][D] (bf16/fp32 viewed as int16 pairs) with the
    commit pattern on the device, layer by layer."""
    L, two, B, Hkv = t.shape[:4]
    raw = t.view(torch.int16).view(L, two, B, Hkv, ncol, -1)
    el = raw.shape[-1]
    dev = t.device
    col = torch.arange(ncol, device=dev, dtype=torch.int64).view(1, 1, 1, ncol, 1)
    e = torch.arange(el, device=dev, dtype=torch.int64).view(1, 1, 1, 1, el)
    for l in range(L):
        slab = slab_base_fn(l).view(two, B, Hkv, 1, 1)
        raw[l].copy_(gen.commit_pattern_torch(slab, col, e))


@pytest.mark.parametrize("wi", WIDS, ids=[w.name for w in wl.WORKLOADS])
def test_workload_commit(wi):
    w = wl.workload(wi)
    parents = wl.trees(w)
    logits, tokens, _ = wl.logits_and_drafts(w, parents)
    _, ost = oracle.validate(parents, w.M)
    al, path, _ = oracle.accept(oracle.argmax(logits), tokens, parents, w.M, ost)   # inputs from the oracle
    del logits
    lens = wl.lengths(w)
    lmax = int(lens.max())
    cap = lmax + w.T + 8
    L = w.layers
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    print(f"[{w.name}] commit: {L} layers, cache {L * 2 * w.B * w.Hkv * cap * w.D * w.esize / 2**30:.1f} GiB",
          flush=True)
    km = torch.empty(L, 2, w.B, w.Hkv, cap, w.D, dtype=dt, device=DEV)
    kb = torch.empty(L, 2, w.B, w.Hkv, w.T, w.D, dtype=dt, device=DEV)
    idx = torch.arange(2 * w.B * w.Hkv, device=DEV, dtype=torch.int64)
    _fill_pattern(km, lambda l: l * 2 * w.B * w.Hkv + idx, cap)
    _fill_pattern(kb, lambda l: 10 ** 6 + l * 2 * w.B * w.Hkv + idx, w.T)
    tm = gen.randint(gen.stream_key(w.seed, 555), w.B * cap, 0, w.V - 1).astype(np.int32).reshape(w.B, cap)
    tm_t, tok_t = _i32(tm), _i32(tokens)
    ln_t, lm_t = _i32(lens), _i32([lmax])
    pos = torch.full((w.B, cap), -3, dtype=torch.int32, device=DEV)
    cst = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    args = svt.commit_args(km, kb, ln_t, lm_t, _i32(path), _i32(al), cst, tokens_main=tm_t, tree_tokens=tok_t,
                           pos_ids=pos, status=_i32(ost))
    assert svt.svt_commit(args, svt.SVT_SYNC_CHECK) == 0
    torch.cuda.synchronize()
    # oracle on a sample of slabs: (layer, KV head) pairs, both planes, every sequence
    layers = sorted({0, L // 2, L - 1})
    heads = sorted({0, w.Hkv - 1})
    el = w.D * w.esize // 2
    def slabs(off, l):
        return np.array([[[off + ((l * 2 + p) * w.B + b) * w.Hkv + h for h in heads] for b in range(w.B)]
                         for p in range(2)], dtype=np.int64)
    hm = np.stack([gen.commit_pattern_slabs(slabs(0, l), cap, el).reshape(2, w.B, len(heads), cap, el)
                   for l in layers])
    hb = np.stack([gen.commit_pattern_slabs(slabs(10 ** 6, l), w.T, el).reshape(2, w.B, len(heads), w.T, el)
                   for l in layers])
    orc, okm, otm, oln, olm, opos = oracle.commit(hm, hb, w.M, tm, tokens, lens, lmax, path, al, ost)
    assert orc == 0 and int(H.from_dev(cst)[0]) == 0
    assert np.array_equal(H.from_dev(ln_t), oln) and int(H.from_dev(lm_t)[0]) == olm
    got_tm, got_pos = H.from_dev(tm_t), H.from_dev(pos)
    for li, l in enumerate(layers):
        for hi, h in enumerate(heads):
            g = km[l, :, :, h].view(torch.int16).cpu().numpy().view(np.uint16).reshape(2, w.B, cap, el)
            for b in range(w.B):
                pad = olm - oln[b]
                assert np.array_equal(g[:, b, pad:olm], okm[li, :, b, hi, pad:olm]), (l, h, b)
            assert np.array_equal(g[:, :, olm:], hm[li, :, :, hi, olm:])     # beyond new lmax untouched
    for b in range(w.B):
        pad = olm - oln[b]
        assert np.array_equal(got_tm[b, pad:olm], otm[b, pad:olm])
        assert np.array_equal(got_pos[b, :olm], opos[b, :olm])
    moved = int(((lmax - lens) != (olm - oln)).sum())
    print(f"[{w.name}] commit ok: lmax {lmax}->{olm}, {moved}/{w.B} sequences re-padded", flush=True)
