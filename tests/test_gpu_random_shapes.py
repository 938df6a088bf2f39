"""Attention parity over seeded random shapes: head dims, GQA groups, tree
sizes, batch sizes, ragged and empty prefixes, grid bounds above the batch
length, value scales from near-uniform to sharp softmax, in every form that
applies.  Each configuration is checked against the oracle (EAGLE-Pangu, nl
summary section 2.C: node u attends the prefix and its tree ancestors) on two
nodes of every (sequence, query head), so that every (sequence, KV head,
query block) of the stream form, cut or whole, has rows in the comparison.

The configurations come from a fixed seed, so a failure names a case that
reruns as it failed; the stream-form cuts they reach are listed by the
harness's host mirror of the cut rule."""
import dataclasses

import numpy as np
import pytest

import harness as H
import oracle
from synth import workloads as wl
from tree_masked_verification_parent_amd import svt

pytestmark = pytest.mark.gpu

N_CASES = 40
SEED = 20261203


def _cases():
    rng = np.random.default_rng(SEED)
    cases = []
    for k in range(N_CASES):
        dtype = "fp32" if k % 5 == 4 else "bf16"
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 8, 16]))
        while G * Hkv > 64:
            G //= 2
        M = int(rng.choice([0, 1, 5, 15, 16, 31, 32, 33, 47, 63, 64, 100]))
        B = int(rng.integers(1, 41))
        lmax_hi = int(rng.choice([64, 500, 2000, 5000]))
        lmax_hi = max(1, min(lmax_hi, 200_000 // (B * Hkv)))  # keep the host arrays small
        lens = rng.integers(0, lmax_hi + 1, size=B)
        lens[rng.random(B) < 0.15] = 0
        whole = rng.random(B) < 0.15
        lens[whole] = 64 * (lens[whole] // 64)  # prefixes of whole key tiles
        if not lens.any():
            lens[0] = lmax_hi
        extra = int(rng.choice([0, 0, 63, 700]))
        sigma = float(rng.choice([0.0883883, 0.5, 1.0]))
        cases.append((f"case{k}-{dtype}-B{B}-Hq{G * Hkv}kv{Hkv}-D{D}-M{M}-L{int(lens.max())}+{extra}-s{sigma:g}",
                      dict(B=B, dtype=dtype, Hq=G * Hkv, Hkv=Hkv, D=D, M=M), lens.astype(np.int32), extra, sigma,
                      1000 + k))
    return cases


CASES = _cases()


@pytest.mark.parametrize("name,over,lens,extra,sigma,seed", CASES, ids=[c[0] for c in CASES])
def test_attention_random_shape(name, over, lens, extra, sigma, seed):
    w = dataclasses.replace(wl.workload(1), qkv_sigma=sigma, **over)
    lmax = int(lens.max())
    bound = lmax + extra
    q, kc, vc, kt, vt = wl.attention_inputs(w, lens, bound + 16, seed)
    par = wl.trees(w, seed)
    forms = [svt.SVT_ATTN_SPLIT] if w.dtype == "fp32" else [svt.SVT_ATTN_AUTO, svt.SVT_ATTN_SPLIT, svt.SVT_ATTN_STREAM]
    rng = np.random.default_rng(seed)
    rows = [(b, int(i), h) for b in range(w.B) for h in range(w.Hq)
            for i in rng.choice(w.T, size=min(2, w.T), replace=False)]
    ref = None
    for form in forms:
        print(f"[{name}] form {form}", flush=True)
        rc, out, omk, ost, sst = H.run_attention(q, kc, vc, kt, vt, par, lens, lmax_bound=bound, form=form)
        assert rc == 0 and (sst == 0).all(), (form, rc, sst)
        got = H.out_f32(w, out)
        assert np.isfinite(got).all(), f"{name} form {form}: padding leaked"
        if ref is None:
            ref = oracle.attention_rows(q, kc, vc, kt, vt, omk, lens, lmax, rows,
                                        to_f32=lambda x: wl.as_f32(w, x))
        sel = np.stack([got[b, i, h] for b, i, h in rows])
        H.check_attention(w, sel, ref, f"{name} form {form}")


def test_attention_few_units_large_kv():
    """Fewer units than CUs with K/V beyond the bound where units of 8 query
    tiles pay off (here 268 MB of K and V): the stream form keeps units of up
    to 12 tiles, each spread over many ranges; two nodes of every (sequence,
    query head) against the oracle, in every form."""
    w = dataclasses.replace(wl.workload(1), B=4, dtype="bf16", Hq=32, Hkv=8, D=128, M=32)
    lens = np.array([16384, 12000, 9000, 3000], np.int32)
    assert 4 * 8 * 16384 * 128 * 4 > (192 << 20)
    nqb, _, nw, _ = H.stream_plan(w.B, w.T, w.Hq, w.Hkv, H.cu_count(), 16384, w.D)
    assert (nqb, nw) == (1, 9)
    q, kc, vc, kt, vt = wl.attention_inputs(w, lens, 16384 + 16, 2100)
    par = wl.trees(w, 2100)
    rng = np.random.default_rng(2101)
    rows = [(b, int(i), h) for b in range(w.B) for h in range(w.Hq) for i in rng.choice(w.T, 2, replace=False)]
    ref = None
    for form in (svt.SVT_ATTN_AUTO, svt.SVT_ATTN_SPLIT, svt.SVT_ATTN_STREAM):
        print(f"[few-units-large-kv] form {form}", flush=True)
        rc, out, omk, ost, sst = H.run_attention(q, kc, vc, kt, vt, par, lens, form=form)
        assert rc == 0 and (sst == 0).all()
        got = H.out_f32(w, out)
        if ref is None:
            ref = oracle.attention_rows(q, kc, vc, kt, vt, omk, lens, 16384, rows, to_f32=lambda x: wl.as_f32(w, x))
        H.check_attention(w, np.stack([got[b, i, h] for b, i, h in rows]), ref, f"form {form}")
