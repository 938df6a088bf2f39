"""The multi-layer round skeleton: rounds run sequentially (verify, then
commit) and rounds whose commit overlaps the next round's attention layer by
layer (two streams; eager and replayed from HIP graphs).  The rounds are
replayed on the oracle alone (its own masks, argmax, accept results and
commits); every schedule's attention of every round and layer must match it
within the contract tolerance, its argmax and accept results and its final
cache, token rows, position ids and lengths bit for bit; and the schedules
must agree with each other bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import harness as H
import oracle
from synth import gen
from synth import workloads as wl
from tree_masked_verification_parent_amd import svt
from tree_masked_verification_parent_amd.pipeline import RoundPipeline

pytestmark = pytest.mark.gpu
DEV = "cuda"
B, M, Hq, Hkv, D, V, L = 4, 12, 8, 2, 128, 96, 3
T = M + 1


def _make(lens0, cap):
    p = RoundPipeline(B, M, Hq, Hkv, D, V, cap, L, torch.bfloat16)
    g = torch.Generator(device=DEV)
    g.manual_seed(1234)
    p.kv_main.normal_(0.0, 0.1, generator=g)
    p.tokens_main.random_(0, V, generator=g)
    lmax0 = int(lens0.max())
    p.lens[0].copy_(torch.from_numpy(lens0))
    p.lmax[0].fill_(lmax0)
    for si, s in enumerate(p.sets):
        seed = 5000 + si
        par = np.stack([gen.tree_depth_capped(gen.stream_key(seed, 1, b), M, 5) for b in range(B)]).astype(np.int32)
        logits, des = gen.logits_with_designated_top(gen.stream_key(seed, 2), B * T, V)
        des = des.reshape(B, T)
        tok = np.stack([gen.plant_drafts(gen.stream_key(seed, 3, b), par[b], des[b], V, 0.8)
                        for b in range(B)]).astype(np.int32)
        s.parents.copy_(torch.from_numpy(par))
        s.tree_tokens.copy_(torch.from_numpy(tok))
        s.logits.copy_(torch.from_numpy(logits.reshape(B, T, V)))
        s.q.normal_(0.0, 0.1, generator=g)
        s.kv_branch.normal_(0.0, 0.1, generator=g)
    p.set_lmax_bound(cap)
    return p


def _state(p, k):
    km = p.kv_main.view(torch.int16).cpu().numpy()
    return km, H.from_dev(p.tokens_main), H.from_dev(p.pos_ids), H.from_dev(p.lens[k % 2]), int(H.from_dev(p.lmax[k % 2])[0])


def _oracle_rounds(p, K):
    """The K rounds replayed on the oracle alone from the rounds' inputs and the
    initial cache: per round, every layer's attention (the oracle's mask and
    status from the parent arrays), argmax and accept, then the commit of the
    oracle's own accept results.  Returns per-round references and the final
    (cache, tokens, lengths, lmax, position ids)."""
    w = dataclasses.replace(wl.workload(1), B=B, M=M, Hq=Hq, Hkv=Hkv, D=D, V=V)
    up = gen.bf16_bits_to_f32
    sets = []
    for s in p.sets:
        par = H.from_dev(s.parents)
        _, ost = oracle.validate(par, M)
        omk, _ = oracle.mask(par, M, ost)
        sets.append(dict(par=par, ost=ost, omk=omk, tok=H.from_dev(s.tree_tokens), logits=H.from_dev(s.logits),
                         q=H.from_dev(s.q), kb=s.kv_branch.view(torch.int16).cpu().numpy().view(np.uint16)))
    km = p.kv_main.view(torch.int16).cpu().numpy().view(np.uint16)
    tm = H.from_dev(p.tokens_main)
    lens, lmax = H.from_dev(p.lens[0]).copy(), int(H.from_dev(p.lmax[0])[0])
    refs = []
    for k in range(K):
        s = sets[k % 2]
        att = [oracle.attention(up(s["q"][l]), up(km[l, 0]), up(km[l, 1]), up(s["kb"][l, 0]), up(s["kb"][l, 1]),
                                s["omk"], lens, lmax, s["ost"])[1] for l in range(L)]
        am = oracle.argmax(s["logits"])
        al, path, bonus = oracle.accept(am, s["tok"], s["par"], M, s["ost"])
        refs.append(dict(att=att, am=am, al=al, path=path, bonus=bonus))
        orc, km, tm, lens, lmax, pos = oracle.commit(km, s["kb"], M, tm, s["tok"], lens, lmax, path, al, s["ost"])
        assert orc == 0
    return w, refs, (km, tm, lens, lmax, pos)


def _check_round(w, name, k, p, ref):
    s = p.sets[k % 2]
    for l in range(L):
        H.check_attention(w, gen.bf16_bits_to_f32(H.from_dev(s.out[l])), ref["att"][l], f"{name} round {k} layer {l}")
    assert np.array_equal(H.from_dev(s.amax), ref["am"]), (name, k)
    assert np.array_equal(H.from_dev(s.accept_len), ref["al"]), (name, k)
    assert np.array_equal(H.from_dev(s.path), ref["path"]) and np.array_equal(H.from_dev(s.bonus), ref["bonus"])


def _check_final(name, p, K, fin):
    km, tm, lens, lmax, pos = fin
    gkm, gtm, gpos, glen, glmax = _state(p, K)
    assert np.array_equal(glen, lens) and glmax == lmax, name
    gkm = gkm.view(np.uint16)
    for b in range(B):
        a = lmax - lens[b]
        assert np.array_equal(gkm[:, :, b, :, a:lmax], km[:, :, b, :, a:lmax]), (name, b)
        assert np.array_equal(gtm[b, a:lmax], tm[b, a:lmax]) and np.array_equal(gpos[b, :lmax], pos[b, :lmax])


def test_pipelined_and_graph_rounds_equal_sequential():
    K = 6
    lens0 = np.array([300, 17, 0, 411], np.int32)
    cap = 411 + (K + 2) * T + 16
    seq, pip, gra = _make(lens0, cap), _make(lens0, cap), _make(lens0, cap)
    w, refs, fin = _oracle_rounds(seq, K)
    outs = {"seq": [], "pip": [], "gra": []}
    for k in range(K):
        print(f"sequential round {k}", flush=True)
        assert seq.sequential_step(k) == 0
        torch.cuda.synchronize()
        assert seq.commit_status.item() == 0
        _check_round(w, "sequential", k, seq, refs[k])
        outs["seq"].append(H.from_dev(seq.sets[k % 2].out))
    _check_final("sequential", seq, K, fin)
    # pipelined, eager
    for k in range(K):
        print(f"pipelined round {k}", flush=True)
        assert pip.pipelined_step(k) == 0
        torch.cuda.synchronize()
        _check_round(w, "pipelined", k, pip, refs[k])
        outs["pip"].append(H.from_dev(pip.sets[k % 2].out))
    assert pip.commit(K - 1) == 0
    torch.cuda.synchronize()
    # pipelined, two eager steps then graphs of both parities replayed in turn
    for k in range(2):
        assert gra.pipelined_step(k) == 0
        torch.cuda.synchronize()
        _check_round(w, "graph (eager start)", k, gra, refs[k])
        outs["gra"].append(H.from_dev(gra.sets[k % 2].out))
    graphs = {0: gra.capture(2), 1: gra.capture(3)}
    for k in range(2, K):
        print(f"graph replay round {k}", flush=True)
        graphs[k % 2].replay()
        torch.cuda.synchronize()
        assert gra.commit_status.item() == 0
        _check_round(w, "graph replay", k, gra, refs[k])
        outs["gra"].append(H.from_dev(gra.sets[k % 2].out))
        _ = H.from_dev(gra.lens[k % 2])            # eager work between replays
    assert gra.commit(K - 1) == 0
    torch.cuda.synchronize()
    for name, p in (("pipelined", pip), ("graph", gra)):
        _check_final(name, p, K, fin)
    # and the schedules agree with each other bit for bit
    for name in ("pip", "gra"):
        for k in range(K):
            assert np.array_equal(outs[name][k].view(np.uint16), outs["seq"][k].view(np.uint16)), (name, k)
