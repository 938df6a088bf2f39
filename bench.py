"""Benchmark of one tree-verification round on one MI355X.

A step is one full round over one batch of the B=32 ragged workload (GQA
32/8 heads, head dim 128, prefix lengths uniform in [1024, 8192], M=32 draft
nodes per tree, vocabulary 32000, 36 cache layers):
    svt_build_mask -> svt_verify_attention for each of the 36 layers ->
    svt_accept over the vocabulary -> svt_commit of all 36 layers.
Inputs are resident in HBM before timing starts.  Each step starts from the
same lengths (a device-to-device copy of 132 bytes restores len/lmax), so
every timed step moves exactly the workload's bytes.

Prints one JSON line.  `value` is verified tree nodes per second of the full
step (B*M nodes per round).  Per-call durations come from HIP events recorded
on the stream the library launches on; the `roofline` object is for the
dominant call, `roofline_attention` for the attention call.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "tree-verify attn GB/s (% HBM peak) + verified tree nodes/s; commit µs/round"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="4", help="workload index or name (default: the B=32 ragged round)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--sched", action="store_true",
                    help="measure the realignment overhead of EQSPEC (fixed batch, re-pad every round) against "
                         "EXSPEC (sequence pool, equal-length batches append) instead of the round benchmark")
    ap.add_argument("--sched-rounds", type=int, default=24)
    ap.add_argument("--sweep", action="store_true",
                    help="cost of one round against the tree budget: M in {8..255} x depth in {4..10} on the "
                         "B=32 workload's shapes, instead of the round benchmark")
    ap.add_argument("--interop", action="store_true",
                    help="time the reference-mode calls (dense 4D mask expansion, length-based commit) on the "
                         "B=32 workload instead of the round benchmark")
    ap.add_argument("--pipeline", action="store_true",
                    help="round time of the B=32 workload with the commit of each round overlapped layer by layer "
                         "with the next round's attention (eager and HIP graph) against sequential rounds")
    ap.add_argument("--attn-sweep", action="store_true",
                    help="attention alone over batch sizes and prefix-length ranges (GQA 32/8, D=128, M=32, "
                         "bf16, inputs cycled so that none is cached), in the automatic, split and stream forms")
    ap.add_argument("--eager", action="store_true",
                    help="time steps launched call by call from the host (per-call events then include any time "
                         "the GPU waits for the next launch) instead of replays of one HIP graph of the step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 3 times (reference for the HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["attn.hip", "commit.hip", "accept.hip", "mask.hip"]


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tree_masked_verification_parent_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernels, workload):
    """HBM bytes per launch of the given kernels from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel factors), or
    None when the summary is missing, was taken on another workload, or the
    kernel sources changed since."""
    import json as _json
    try:
        with open(TRAFFIC_FILE) as f:
            t = _json.load(f)
    except OSError:
        return None
    if t.get("sources_digest") != sources_digest() or t.get("workload", "").split(" ")[0] != workload:
        return None
    total = 0.0
    for k in kernels:
        if k not in t["kernels"]:
            return None
        e = t["kernels"][k]
        total += e["fetch_kib"] * 1024 / t["copy_factor"]["fetch"] + e["write_kib"] * 1024 / t["copy_factor"]["write"]
    return total


def device_copy_gbps(torch, nbytes=1 << 30, reps=5):
    """Read + write rate of a plain device-to-device copy of nbytes (median of
    reps, HIP events): the practical HBM ceiling the kernels are compared with
    besides the 8 TB/s peak."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / float(np.median(ts)) / 1e9


MALL_BYTES = 256 << 20  # MI355X Infinity Cache


def cold_attention(torch, svt, r, len0, lmax0_t, attn_bytes, attn_flops, total=1 << 30, max_copies=256,
                   eager=False, form=0):
    """Attention timed over copies of one layer's inputs (Q, prefix and tree
    K/V, output) totalling at least `total` bytes of attention reads, cycled
    so that no call finds its inputs in the Infinity Cache.  The round above
    reuses its per-layer inputs every step; when they fit in the cache this
    is the number that reads them from HBM."""
    r.len.copy_(len0)
    r.lmax.copy_(lmax0_t)
    n = int(min(max_copies, max(2, -(-total // int(attn_bytes)))))
    keep, args = [], []
    for _ in range(n):
        q = r.q[0].clone()
        kv = r.kv_main[0].clone()
        br = r.kv_branch[0].clone()
        out = torch.empty_like(r.out[0])
        keep.append((q, kv, br, out))
        args.append(svt.attn_args(q, kv[0], kv[1], r.len, r.lmax, r.lmax_bound, br[0], br[1], r.mask, out,
                                  status=r.status, seq_status=r.seq_status, workspace=r._attn_ws, form=form))
    for a in args:  # one untimed pass
        assert svt.svt_verify_attention(a) == 0
    passes = max(1, -(-64 // n))
    # the calls are replayed from one HIP graph (unless eager), so the GPU
    # does not wait for the host between calls
    g = None
    if not eager:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for a in args:
                assert svt.svt_verify_attention(a) == 0
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(passes):
        if g is not None:
            g.replay()
        else:
            for a in args:
                svt.svt_verify_attention(a)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (passes * n)
    del g
    del keep, args
    torch.cuda.empty_cache()
    return {"copies": n, "calls": passes * n, "us_per_call": t * 1e6, "GBps": attn_bytes / t / 1e9,
            "frac_hbm": attn_bytes / t / 1e9 / HBM_PEAK_GBPS,
            "mfma_frac": attn_flops / t / 1e12 / BF16_PEAK_TFLOPS}


def algorithmic_bytes_attention(w, lens, T):
    e = w.esize
    q = w.B * T * w.Hq * w.D * e
    kv = int(lens.sum()) * w.Hkv * w.D * e * 2
    tree = w.B * w.Hkv * T * w.D * e * 2
    mask = w.B * T * ((T + 63) // 64) * 8
    return q + kv + tree + q + mask


def flops_attention(w, lens, depth):
    # 4 * Hq * D per (query, key) pair actually attended: prefix keys plus ancestors
    T = w.T
    pairs = int(lens.sum()) * T + int((depth + 1).sum())
    return 4 * w.Hq * w.D * pairs


def algorithmic_bytes_commit(w, lens, A, n_layers):
    row = w.D * w.esize
    lmax = int(lens.max())
    new_len = lens + A
    new_lmax = int(new_len.max())
    moved = (lmax - lens) != (new_lmax - new_len)
    kv = 0
    for b in range(w.B):
        if moved[b]:
            kv += 2 * int(lens[b]) * row          # read + write of the shifted content
        kv += 2 * int(A[b]) * row                 # gather: read branch row, write main row
    kv *= n_layers * 2 * w.Hkv
    tok = sum(2 * int(lens[b]) * 4 for b in range(w.B) if moved[b]) + 2 * int(A.sum()) * 4
    pos = w.B * new_lmax * 4
    return kv + tok + pos


def algorithmic_bytes_accept(w):
    return w.B * w.T * w.V * 4


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, parents, lens, logits, tokens, seed, budget_s):
    """Time the oracle (plain C, double precision, unchanged) on a bounded
    sample of the same workload and scale it to one full step, twice: on one
    thread, and with the sampled attention rows and commit slabs spread over
    the host's cores (oracle.attention_rows: the same C row routine, rows run
    side by side; commit slabs as independent oracle calls side by side).
    Mask and accept are single-threaded in both legs (they are a small part)."""
    import concurrent.futures as cf

    import oracle
    from synth import gen
    from synth import workloads as wl

    t_all = time.perf_counter()
    nthreads = oracle.default_threads()
    lmax = int(lens.max())
    # mask + validate: whole batch
    t0 = time.perf_counter()
    _, st = oracle.validate(parents, w.M)
    mk, dp = oracle.mask(parents, w.M, st)
    t_mask = time.perf_counter() - t0
    # argmax + accept: whole batch (the logits the GPU also read)
    t0 = time.perf_counter()
    am = oracle.argmax(logits)
    al, path, _ = oracle.accept(am, tokens, parents, w.M, st)
    t_accept = time.perf_counter() - t0
    # attention: whole sequences of one layer, in a seeded order, until the
    # one-thread sample has used about 60 % of the budget; then the same
    # sequences again with their rows over `nthreads` threads
    order = np.argsort(gen.u64(gen.stream_key(seed, 991), w.B))
    picked, t_attn_sample, keys_sample, inputs = [], 0.0, 0, []
    t_part = time.perf_counter()
    sub = wl.Workload(**{**w.__dict__, "B": 1})
    f = lambda x: wl.as_f32(sub, x)
    for b in order:
        if picked and time.perf_counter() - t_part > 0.6 * budget_s:
            break
        Lb = int(lens[b])
        q, kc, vc, kt, vt = wl.attention_inputs(sub, np.array([Lb], np.int32), Lb, seed + 1000 + int(b),
                                                poison=False)
        args = (f(q), f(kc), f(vc), f(kt), f(vt), mk[b:b + 1], np.array([Lb], np.int32), Lb)
        t0 = time.perf_counter()
        oracle.attention(*args)
        t_attn_sample += time.perf_counter() - t0
        keys_sample += Lb
        picked.append(int(b))
        inputs.append(args)
    t0 = time.perf_counter()
    rows = [(0, i, h) for i in range(w.T) for h in range(w.Hq)]
    for args in inputs:
        oracle.attention_rows(*args[:7], args[7], rows, threads=nthreads)
    t_attn_sample_mt = time.perf_counter() - t0
    del inputs
    t_attn_layer = t_attn_sample * float(lens.sum()) / max(keys_sample, 1)
    t_attn_layer_mt = t_attn_sample_mt * float(lens.sum()) / max(keys_sample, 1)
    # commit: one layer and one KV head per oracle call (every layer, plane
    # and head moves the same way; the bytes moved do not depend on their
    # values); nthreads such calls side by side for the threaded leg
    T = w.T
    cap = lmax + T + 8
    row_el = w.D * w.esize // 2
    km = (np.arange(2 * w.B * cap * row_el, dtype=np.uint32) & 0xFFFF).astype(np.uint16)
    km = km.reshape(1, 2, w.B, 1, cap, row_el)
    kb = np.ones((1, 2, w.B, 1, T, row_el), np.uint16)
    tm = np.zeros((w.B, cap), np.int32)
    t0 = time.perf_counter()
    oracle.commit(km, kb, w.M, tm, tokens, lens, lmax, path, al, st)
    t_commit_slab = time.perf_counter() - t0
    n_slabs = w.layers * w.Hkv
    t_commit = t_commit_slab * n_slabs
    par_calls = min(nthreads, n_slabs)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=par_calls) as ex:
        list(ex.map(lambda _: oracle.commit(km, kb, w.M, tm, tokens, lens, lmax, path, al, st), range(par_calls)))
    t_commit_mt = (time.perf_counter() - t0) * -(-n_slabs // par_calls)
    step_s = t_mask + w.layers * t_attn_layer + t_accept + t_commit
    step_s_mt = t_mask + w.layers * t_attn_layer_mt + t_accept + t_commit_mt
    sample = (f"oracle (fp64 C, unchanged) on the same workload: mask+accept for all {w.B} sequences "
              f"(1 thread); one-layer attention for sequences {picked} ({keys_sample} of {int(lens.sum())} "
              f"prefix keys), scaled by keys and by {w.layers} layers; commit of one layer and one KV head per "
              f"call, scaled by {w.layers} layers x {w.Hkv} heads; {time.perf_counter() - t_all:.1f} s wall")
    one = {"value": w.B * w.M / step_s, "cores": 1, "est_step_s": step_s,
           "est_parts_s": {"mask": t_mask, "attention_per_layer": t_attn_layer, "accept": t_accept,
                           "commit": t_commit}}
    return {
        "value": w.B * w.M / step_s_mt,
        "unit": "verified tree nodes/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": sample + f"; attention rows and commit calls over {nthreads} threads",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "est_step_s": step_s_mt,
        "est_parts_s": {"mask": t_mask, "attention_per_layer": t_attn_layer_mt, "accept": t_accept,
                        "commit": t_commit_mt},
        "single_thread": one,
    }


def sched_bench(args):
    """EQSPEC against EXSPEC on the B=32 workload's shapes (36 layers, GQA 32/8,
    D=128, M=32): per round, realignment (svt_realign, EXSPEC fallback only),
    verification (mask, attention over every layer, accept) and commit (re-pad
    for EQSPEC and the fallback, append for equal-length EXSPEC batches), each
    timed with HIP events.  Prints one JSON line."""
    import torch
    from synth import workloads as wl
    from tree_masked_verification_parent_amd import svt
    from tree_masked_verification_parent_amd.sched import PoolRound, SequencePool

    w = wl.workload(4)
    L, R = w.layers, args.sched_rounds
    buckets = [1024, 1536, 2048]              # prompt lengths: few distinct values (bucketed prompts)
    dev = torch.device("cuda")
    gen_t = torch.Generator(device=dev)
    gen_t.manual_seed(w.seed)
    n_sets = 3
    sets = []
    for k in range(n_sets):                   # seeded trees / drafts / logits for up to 32 sequences
        par = wl.trees(w, w.seed + 100 + k)
        logits, tokens, _ = wl.logits_and_drafts(w, par, w.seed + 100 + k)
        sets.append((torch.from_numpy(par).to(dev), torch.from_numpy(tokens).to(dev),
                     torch.from_numpy(logits).to(dev)))
    results = []
    for B in (8, 16, 32):
        for mode in ("eqspec", "exspec"):
            P = B if mode == "eqspec" else 8 * B
            cap = max(buckets) + (R + 4) * w.T + 64
            pool = SequencePool(P, w.Hkv, w.D, L, cap, torch.bfloat16)
            for layer in range(L):
                pool.kv[layer].normal_(0.0, w.qkv_sigma, generator=gen_t)
            lens = np.array([buckets[s % len(buckets)] for s in range(P)], np.int32)
            for s in range(P):
                pool.place(s, int(lens[s]), max(buckets) if mode == "eqspec" else None)
            pr = PoolRound(pool, B, w.M, w.Hq, w.V, L)
            pr.q.normal_(0.0, w.qkv_sigma, generator=gen_t)
            pr._kvb.normal_(0.0, w.qkv_sigma, generator=gen_t)
            stream = torch.cuda.current_stream()
            rows = []
            for rnd in range(R + 2):
                if mode == "eqspec":
                    same, slots = True, np.arange(B, dtype=np.int32)
                else:
                    same, slots = pool.pick(B, max(1, B // 2))
                n = len(slots)
                par, tok, lg = sets[rnd % n_sets]
                pr.parents[:n].copy_(par[:n])
                pr.tree_tokens[:n].copy_(tok[:n])
                pr.logits[:n].copy_(lg[:n])
                pr.load_batch(slots)
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                ev[0].record(stream)
                realigned = mode == "exspec" and not same
                E = pool.realign(slots, pr.slot[:n], pr.len[:n], pr.end[:n]) if realigned else int(pool.end[slots[0]])
                ev[1].record(stream)
                rc_v = pr.verify(n, E)
                ev[2].record(stream)
                cmode = svt.SVT_COMMIT_APPEND if (mode == "exspec" and same) else svt.SVT_COMMIT_REPAD
                rc_c = pr.commit(n, cmode)
                ev[3].record(stream)
                torch.cuda.synchronize()
                assert rc_v == 0 and rc_c == 0 and pr.commit_status.item() == 0, \
                    (mode, B, rnd, n, rc_v, rc_c, pr.commit_status.item())
                al = pr.accept_len[:n].cpu().numpy()
                pool.committed(slots, al, E, cmode)
                if rnd >= 2:
                    rows.append((ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]), ev[2].elapsed_time(ev[3]),
                                 int(n), int((al + 1).sum()), bool(realigned), cmode))
            t_realign = sum(r[0] for r in rows) * 1e-3
            t_verify = sum(r[1] for r in rows) * 1e-3
            t_commit = sum(r[2] for r in rows) * 1e-3
            t_total = t_realign + t_verify + t_commit
            t_move = t_realign + sum(r[2] for r in rows if r[6] == svt.SVT_COMMIT_REPAD) * 1e-3
            t_append = sum(r[2] for r in rows if r[6] == svt.SVT_COMMIT_APPEND) * 1e-3
            toks = sum(r[4] for r in rows)
            results.append({
                "B": B, "mode": mode, "pool": P, "rounds": len(rows),
                "mean_batch": float(np.mean([r[3] for r in rows])),
                "append_rounds": sum(1 for r in rows if r[6] == svt.SVT_COMMIT_APPEND),
                "realign_rounds": sum(1 for r in rows if r[5]),
                "ms_realign": t_realign * 1e3, "ms_verify": t_verify * 1e3, "ms_commit": t_commit * 1e3,
                "ms_commit_append": t_append * 1e3,
                "realign_frac": t_move / t_total,
                "tokens_per_s": toks / t_total,
                "accepted_tokens": toks,
            })
            print(f"[sched] B={B} {mode}: realign {t_realign*1e3:.1f} ms, verify {t_verify*1e3:.1f} ms, "
                  f"commit {t_commit*1e3:.1f} ms, realignment {t_move / t_total:.1%}, "
                  f"{toks / t_total:.0f} tokens/s", file=sys.stderr, flush=True)
            del pool, pr
            torch.cuda.empty_cache()
    out = {
        "metric": "realignment overhead fraction of the verification round, EQSPEC vs EXSPEC",
        "unit": "fraction of round time", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
        "data": "synthetic (seeded trees, drafts, logits; device-seeded normal caches; prompt lengths "
                f"from {buckets})",
        "config": {"workload": w.name + " shapes, pool scheduling", "layers": L, "rounds": R,
                   "pool_factor_exspec": 8, "min_group": "B/2"},
        "results": results,
    }
    print(json.dumps(out), flush=True)


def sweep_bench(args):
    """Round cost against the tree budget: for M draft nodes and a depth cap,
    layered trees (nodes spread evenly over the levels) on the B=32 workload's
    shapes (prefix U[1024, 8192], GQA 32/8, D=128, V=32000, 36 layers).  Per
    call times from HIP events over 5 steps after 2 warm-up steps; every step
    restores the lengths, so it moves the same bytes.  Prints one JSON line."""
    import torch
    from synth import gen
    from synth import workloads as wl
    from tree_masked_verification_parent_amd import svt
    from tree_masked_verification_parent_amd.round import VerifyRound

    w = wl.workload(4)
    L = w.layers
    lens0 = wl.lengths(w)
    lmax0 = int(lens0.max())
    dev = torch.device("cuda")
    gen_t = torch.Generator(device=dev)
    gen_t.manual_seed(w.seed)
    len0 = torch.from_numpy(lens0).to(dev)
    stream = torch.cuda.current_stream()
    steps, warm = 5, 2
    rows = []
    for M in (8, 16, 32, 64, 128, 255):
        T = M + 1
        cap = lmax0 + T + 64
        r = VerifyRound(w.B, M, w.Hq, w.Hkv, w.D, w.V, cap, L, torch.bfloat16, attn_layers=L)
        for layer in range(L):
            r.kv_main[layer].normal_(0.0, w.qkv_sigma, generator=gen_t)
            r.kv_branch[layer].normal_(0.0, w.qkv_sigma, generator=gen_t)
            r.q[layer].normal_(0.0, w.qkv_sigma, generator=gen_t)
        logits, des = gen.logits_with_designated_top(gen.stream_key(w.seed, 900, M), w.B * T, w.V)
        r.logits.copy_(torch.from_numpy(logits.reshape(w.B, T, w.V)))
        des = des.reshape(w.B, T)
        del logits
        for depth in sorted({min(d, M) for d in (4, 6, 8, 10)}):
            par = np.stack([gen.tree_layered(gen.stream_key(w.seed, 901, M, depth, b), M, depth)
                            for b in range(w.B)]).astype(np.int32)
            tok = np.stack([gen.plant_drafts(gen.stream_key(w.seed, 902, M, depth, b), par[b], des[b], w.V,
                                             w.p_plant) for b in range(w.B)]).astype(np.int32)
            r.parents.copy_(torch.from_numpy(par))
            r.tree_tokens.copy_(torch.from_numpy(tok))
            r.len.copy_(len0)
            r.lmax.fill_(lmax0)
            r.set_lmax_bound(lmax0)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
            for k in range(warm + steps):
                r.len.copy_(len0)
                r.lmax.fill_(lmax0)
                ev = evs[k - warm] if k >= warm else None
                if ev:
                    ev[0].record(stream)
                rc = r.build_mask()
                if ev:
                    ev[1].record(stream)
                for layer in range(L):
                    rc = rc or r.attention(layer)
                if ev:
                    ev[2].record(stream)
                rc = rc or r.accept()
                if ev:
                    ev[3].record(stream)
                rc = rc or r.commit()
                if ev:
                    ev[4].record(stream)
                assert rc == 0, (M, depth, rc)
            torch.cuda.synchronize()
            assert r.commit_status.item() == 0 and (r.status.cpu().numpy() == 0).all()
            A = r.accept_len.cpu().numpy() + 1

            def dur(i, j):
                return float(np.median([e[i].elapsed_time(e[j]) for e in evs])) * 1e3

            t = {"mask_us": dur(0, 1), "attn_us": dur(1, 2), "accept_us": dur(2, 3), "commit_us": dur(3, 4)}
            t_round = sum(t.values())
            rows.append({"M": M, "depth": depth, **t, "attn_us_per_layer": t["attn_us"] / L,
                         "round_us": t_round, "mean_accept_len": float(np.mean(A - 1)),
                         "us_per_verified_node": t_round / (w.B * M),
                         "us_per_accepted_token": t_round / float(A.sum())})
            print(f"[sweep] M={M:3d} depth={depth:2d}: round {t_round:8.1f} us (mask {t['mask_us']:.1f}, "
                  f"attention {t['attn_us'] / L:.1f}/layer, accept {t['accept_us']:.1f}, commit "
                  f"{t['commit_us']:.1f}); accept_len {np.mean(A - 1):.2f}; "
                  f"{t_round / float(A.sum()):.2f} us per accepted token", file=sys.stderr, flush=True)
        del r
        torch.cuda.empty_cache()
    out = {"metric": "verification round cost against tree budget (M, depth)", "unit": "us per round",
           "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
           "data": "synthetic (layered trees, planted drafts p=%.2f, seeded logits; device-seeded normal caches)"
                   % w.p_plant,
           "config": {"workload": w.name + " shapes, budget sweep", "layers": L, "steps": steps, "warmup": warm},
           "results": rows}
    print(json.dumps(out), flush=True)


def attn_sweep_bench(args):
    """svt_verify_attention alone over batch sizes and prefix-length ranges on
    the B=32 workload's head shapes (GQA 32/8, D=128, M=32, bf16): per call,
    HIP events over copies of the inputs cycled so that none is read from the
    Infinity Cache (as bench.py's cold attention), in the automatic choice and
    in each form forced.  Prints one JSON line."""
    import dataclasses

    import torch
    from synth import workloads as wl
    from tree_masked_verification_parent_amd import svt
    from tree_masked_verification_parent_amd.round import VerifyRound

    base = wl.workload(4)
    dev = torch.device("cuda")
    grid = [((1024, 8192), (1, 2, 4, 8, 16, 32, 64)), ((128, 1024), (32, 64, 128, 256, 512))]
    forms = [("auto", svt.SVT_ATTN_AUTO), ("split", svt.SVT_ATTN_SPLIT), ("stream", svt.SVT_ATTN_STREAM)]
    rows = []
    for (lo, hi), bs in grid:
        for B in bs:
            w = dataclasses.replace(base, B=B, len_lo=lo, len_hi=hi)
            lens0 = wl.lengths(w)
            lmax0 = int(lens0.max())
            r = VerifyRound(B, w.M, w.Hq, w.Hkv, w.D, 64, lmax0 + w.T + 64, 1, torch.bfloat16, attn_layers=1)
            gen_t = torch.Generator(device=dev)
            gen_t.manual_seed(w.seed + B)
            r.kv_main.normal_(0.0, w.qkv_sigma, generator=gen_t)
            r.kv_branch.normal_(0.0, w.qkv_sigma, generator=gen_t)
            r.q.normal_(0.0, w.qkv_sigma, generator=gen_t)
            r.parents.copy_(torch.from_numpy(wl.trees(w)))
            len0 = torch.from_numpy(lens0).to(dev)
            lmax0_t = torch.tensor([lmax0], dtype=torch.int32, device=dev)
            r.len.copy_(len0)
            r.lmax.copy_(lmax0_t)
            assert r.build_mask() == 0
            nbytes = algorithmic_bytes_attention(w, lens0, w.T)
            res = {"B": B, "len_range": [lo, hi], "sum_len": int(lens0.sum()), "attn_bytes": nbytes}
            r.set_lmax_bound(lmax0)
            # one discarded measurement first: the clock ramps up after the set-up
            cold_attention(torch, svt, r, len0, lmax0_t, nbytes, 0.0)
            for name, form in forms:
                a = r._attn_args(0)
                a.form = form
                need = svt.svt_verify_attention_workspace(a)
                if need == 0 and form == svt.SVT_ATTN_STREAM:
                    res[name] = None   # the stream form does not take this batch
                    continue
                if need > (0 if r._attn_ws is None else r._attn_ws.numel()):
                    r._attn_ws = torch.empty(need, dtype=torch.uint8, device=dev)
                c = cold_attention(torch, svt, r, len0, lmax0_t, nbytes, 0.0, form=form)
                res[name] = {"us_per_call": c["us_per_call"], "GBps": c["GBps"], "frac_hbm": c["frac_hbm"]}
            rows.append(res)
            best = min((v["us_per_call"], k) for k, v in res.items() if isinstance(v, dict))
            print(f"[attn-sweep] B={B:4d} len U[{lo},{hi}]: " + ", ".join(
                f"{k} {v['us_per_call']:.1f} us ({v['frac_hbm']:.0%})" for k, v in res.items() if isinstance(v, dict))
                + f"; fastest {best[1]}", file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()
    out = {"metric": "attention alone: us per call and fraction of 8 TB/s, cold, by batch size and prefix length",
           "unit": "us per call", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
           "data": "synthetic (seeded trees and lengths; device-seeded normal Q/K/V)",
           "config": {"workload": "B=32 workload head shapes (GQA 32/8, D=128, M=32), B and lengths varied"},
           "results": rows}
    print(json.dumps(out), flush=True)


def interop_bench(args):
    """svt_expand_mask (three output kinds) and svt_commit_length against
    svt_commit on the B=32 workload (M=32, prefix U[1024, 8192], 36 layers).
    HIP events over 20 calls after 3 warm-up calls; the commit calls restore
    the lengths before each call.  Prints one JSON line."""
    import torch
    from synth import workloads as wl
    from tree_masked_verification_parent_amd import svt
    from tree_masked_verification_parent_amd.round import VerifyRound

    w = wl.workload(4)
    dev = torch.device("cuda")
    parents = wl.trees(w)
    lens0 = wl.lengths(w)
    lmax0 = int(lens0.max())
    logits, tokens, _ = wl.logits_and_drafts(w, parents)
    L = w.layers
    r = VerifyRound(w.B, w.M, w.Hq, w.Hkv, w.D, w.V, lmax0 + w.T + 64, L, torch.bfloat16, attn_layers=1)
    gen_t = torch.Generator(device=dev)
    gen_t.manual_seed(w.seed)
    for layer in range(L):
        r.kv_main[layer].normal_(0.0, w.qkv_sigma, generator=gen_t)
        r.kv_branch[layer].normal_(0.0, w.qkv_sigma, generator=gen_t)
    r.parents.copy_(torch.from_numpy(parents))
    r.tree_tokens.copy_(torch.from_numpy(tokens))
    r.logits.copy_(torch.from_numpy(logits))
    len0 = torch.from_numpy(lens0).to(dev)
    r.len.copy_(len0)
    r.lmax.fill_(lmax0)
    r.set_lmax_bound(lmax0)
    assert r.build_mask(svt.SVT_SYNC_CHECK) == 0 and r.accept() == 0
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    n, warm = 20, 3

    def timed(fn, before=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for k in range(warm + n):
            if before:
                before()
            if k >= warm:
                evs[k - warm][0].record(stream)
            assert fn() == 0
            if k >= warm:
                evs[k - warm][1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3

    res = {}
    T = w.T
    for kind, dt, name in [(svt.SVT_MASK_ADD_FP32, torch.float32, "add_fp32"),
                           (svt.SVT_MASK_ADD_BF16, torch.bfloat16, "add_bf16"), (svt.SVT_MASK_BOOL, torch.uint8, "bool")]:
        out = torch.empty(w.B, 1, T, lmax0 + T, dtype=dt, device=dev)
        us = timed(lambda: svt.svt_expand_mask(r.mask, r.status, r.len, w.M, lmax0, out, kind))
        nbytes = out.numel() * out.element_size()
        res["expand_" + name] = {"us": us, "bytes_written": nbytes, "GBps": nbytes / us / 1e3,
                                 "frac_hbm": nbytes / us / 1e3 / HBM_PEAK_GBPS}
        del out

    def restore():
        r.len.copy_(len0)
        r.lmax.fill_(lmax0)

    us_path = timed(lambda: svt.svt_commit(r._commit_args()), restore)
    us_len = timed(lambda: svt.svt_commit_length(r._commit_args()), restore)
    A = r.accept_len.cpu().numpy().astype(np.int64) + 1
    cbytes = algorithmic_bytes_commit(w, lens0, A, L)
    res["commit_path_us"] = us_path
    res["commit_length_us"] = us_len
    res["commit_GBps"] = {"path": cbytes / us_path / 1e3, "length": cbytes / us_len / 1e3}
    out = {"metric": "reference-mode interop: dense 4D mask expansion GB/s, length-based commit us",
           "unit": "see fields", "n_gpus": 1, "dtype": "bf16", "data": "synthetic (B=32 ragged workload)",
           "config": {"workload": w.name, "lmax": lmax0, "T": T, "layers": L}, "results": res}
    for k, v in res.items():
        print(f"[interop] {k}: {v}", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def pipeline_bench(args):
    """Steady-state round time of the B=32 workload (36 layers): sequential
    rounds (verify, then a 36-layer commit) against rounds whose commit runs
    layer by layer on a second stream while the next round's attention waits
    only for its own layer, eager and replayed from HIP graphs.  The two
    buffer sets carry different trees, drafts and logits, so the accept
    lengths differ between rounds and the commits move data.  Prints one
    JSON line."""
    import torch
    from synth import workloads as wl
    from tree_masked_verification_parent_amd import svt
    from tree_masked_verification_parent_amd.pipeline import RoundPipeline

    w = wl.workload(4)
    L, R, warm = w.layers, 8, 2
    lens0 = wl.lengths(w)
    lmax0 = int(lens0.max())
    cap = lmax0 + (4 * (R + warm) + 8) * w.T + 64
    dev = torch.device("cuda")
    p = RoundPipeline(w.B, w.M, w.Hq, w.Hkv, w.D, w.V, cap, L, torch.bfloat16)
    gen_t = torch.Generator(device=dev)
    gen_t.manual_seed(w.seed)
    for layer in range(L):
        p.kv_main[layer].normal_(0.0, w.qkv_sigma, generator=gen_t)
    for si, st in enumerate(p.sets):
        par = wl.trees(w, w.seed + 10 + si)
        logits, tokens, _ = wl.logits_and_drafts(w, par, w.seed + 10 + si)
        st.parents.copy_(torch.from_numpy(par))
        st.tree_tokens.copy_(torch.from_numpy(tokens))
        st.logits.copy_(torch.from_numpy(logits))
        st.q.normal_(0.0, w.qkv_sigma, generator=gen_t)
        st.kv_branch.normal_(0.0, w.qkv_sigma, generator=gen_t)
    p.lens[0].copy_(torch.from_numpy(lens0))
    p.lmax[0].fill_(lmax0)
    p.set_lmax_bound(cap)
    stream = torch.cuda.current_stream()

    def run(step, k0, n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        evs[0].record(stream)
        for i in range(n):
            assert step(k0 + i) == 0
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        assert p.commit_status.item() == 0
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]

    k = 0
    run(p.sequential_step, k, warm)
    k += warm
    t_seq = run(p.sequential_step, k, R)
    k += R
    assert p.verify(k) == 0                  # verified, not committed: the next pipelined step commits it
    k += 1
    run(p.pipelined_step, k, warm)
    k += warm
    t_pip = run(p.pipelined_step, k, R)
    k += R
    p.attn_form = svt.SVT_ATTN_SPLIT         # the split form schedules many small workgroups
    p.set_lmax_bound(cap)                    # its workspace differs
    t_pip_split = run(p.pipelined_step, k, R)
    k += R
    p.attn_form = svt.SVT_ATTN_AUTO
    graphs = {0: p.capture(k + (k % 2)), 1: p.capture(k + 1 - (k % 2))}

    def replay(kk):
        graphs[kk % 2].replay()
        return 0

    run(replay, k, warm)
    k += warm
    t_gra = run(replay, k, R)
    k += R
    assert p.commit(k - 1) == 0
    torch.cuda.synchronize()
    res = {"sequential_ms": float(np.median(t_seq)), "pipelined_ms": float(np.median(t_pip)),
           "pipelined_split_attention_ms": float(np.median(t_pip_split)),
           "pipelined_graph_ms": float(np.median(t_gra))}
    res["speedup_pipelined"] = res["sequential_ms"] / res["pipelined_ms"]
    res["speedup_graph"] = res["sequential_ms"] / res["pipelined_graph_ms"]
    out = {"metric": "verification round time, sequential vs commit overlapped with the next round's attention",
           "unit": "ms per round", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
           "data": "synthetic (two alternating seeded rounds; device-seeded normal caches)",
           "config": {"workload": w.name, "layers": L, "rounds": R, "warmup": warm}, "results": res,
           "per_round_ms": {"sequential": t_seq, "pipelined": t_pip, "pipelined_split_attention": t_pip_split,
                            "pipelined_graph": t_gra}}
    print(f"[pipeline] {res}", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(collectives and sharding are out of its scope); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    # Python's cyclic collector stays off for the whole run, as in timeit: a
    # full collection over torch's object heap takes about 40 ms, and it would
    # land inside whichever timed round or step crosses the threshold (one
    # such pause tripled the B=8 EXSPEC verify total of the scheduling run).
    gc.collect()
    gc.disable()
    if args.sched:
        sched_bench(args)
        return
    if args.sweep:
        sweep_bench(args)
        return
    if args.interop:
        interop_bench(args)
        return
    if args.pipeline:
        pipeline_bench(args)
        return
    if args.attn_sweep:
        attn_sweep_bench(args)
        return

    import torch
    from synth import workloads as wl
    from tree_masked_verification_parent_amd import svt
    from tree_masked_verification_parent_amd.round import VerifyRound

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}))
        return
    wkey = int(args.workload) if args.workload.isdigit() else args.workload
    w = wl.workload(wkey)
    dtype = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    seed = w.seed
    parents = wl.trees(w, seed)
    lens0 = wl.lengths(w, seed)
    lmax0 = int(lens0.max())
    logits, tokens, _ = wl.logits_and_drafts(w, parents, seed)
    cap = lmax0 + w.T + 64
    L = w.layers

    r = VerifyRound(w.B, w.M, w.Hq, w.Hkv, w.D, w.V, cap, L, dtype, attn_layers=L)
    dev = r.q.device
    r.parents.copy_(torch.from_numpy(parents))
    r.tree_tokens.copy_(torch.from_numpy(tokens))
    r.logits.copy_(torch.from_numpy(logits))
    gen_t = torch.Generator(device=dev)
    gen_t.manual_seed(seed)
    sig = w.qkv_sigma
    for layer in range(L):  # seeded device-side normals for the large tensors
        r.kv_main[layer].normal_(0.0, sig, generator=gen_t)
        r.kv_branch[layer].normal_(0.0, sig, generator=gen_t)
        r.q[layer].normal_(0.0, sig, generator=gen_t)
    r.tokens_main.random_(0, w.V, generator=gen_t)
    len0 = torch.from_numpy(lens0).to(dev)
    lmax0_t = torch.tensor([lmax0], dtype=torch.int32, device=dev)
    r.len.copy_(len0)
    r.lmax.copy_(lmax0_t)
    r.set_lmax_bound(lmax0)
    torch.cuda.synchronize()

    # first round (untimed): learn the accept lengths, which fix every later round
    assert r.build_mask(svt.SVT_SYNC_CHECK) == 0
    assert r.step() == 0
    assert r.commit_status.item() == 0
    A = r.accept_len.cpu().numpy().astype(np.int64) + 1
    depth = r.depth.cpu().numpy()

    stream = torch.cuda.current_stream()
    # five events per step: before the mask, after it, after the last
    # attention layer, after accept, after commit (the mean per attention layer
    # is the attention interval over L: per-layer events would give the same
    # mean and cost host time on the launch-bound small rounds)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]

    def one_step(ev=None):
        r.len.copy_(len0)
        r.lmax.copy_(lmax0_t)
        if ev:
            ev[0].record(stream)
        rc = r.build_mask()
        if ev:
            ev[1].record(stream)
        for layer in range(L):
            rc = rc or r.attention(layer)
        if ev:
            ev[2].record(stream)
        rc = rc or r.accept()
        if ev:
            ev[3].record(stream)
        rc = rc or r.commit()
        if ev:
            ev[4].record(stream)
        return rc

    for _ in range(args.warmup):
        assert one_step() == 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        rc = one_step(evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert rc == 0 and r.commit_status.item() == 0
    assert np.array_equal(r.len.cpu().numpy(), lens0 + A)

    def per_step(i, j, div=1):
        return np.array([evs[k][i].elapsed_time(evs[k][j]) for k in range(args.steps)]) * 1e-3 / div

    def dist_us(x):
        x = np.asarray(x) * 1e6
        return {"mean": float(x.mean()), "p10": float(np.percentile(x, 10)), "p50": float(np.median(x)),
                "p90": float(np.percentile(x, 90)), "min": float(x.min()), "max": float(x.max())}

    # launched call by call: the distribution over the timed steps of each
    # call type (attention: the step's mean per layer) and of the whole step
    # between its first and last event
    timing_eager = {"mode": "eager", "steps": args.steps, "mask_us": dist_us(per_step(0, 1)),
                    "attention_us_per_layer": dist_us(per_step(1, 2, L)), "accept_us": dist_us(per_step(2, 3)),
                    "commit_us": dist_us(per_step(3, 4)), "step_us": dist_us(per_step(0, 4)),
                    "ms_per_step": elapsed / args.steps * 1e3}
    if args.eager:
        ms_per_step = elapsed / args.steps * 1e3
        timing = timing_eager
        t_mask, t_attn, t_accept, t_commit = (float(np.mean(per_step(i, i + 1, L if i == 1 else 1)))
                                              for i in range(4))
    else:
        # The step as one HIP graph (the library allocates nothing and never
        # synchronises, so every call captures): a serving loop launches a
        # round this way, and the GPU never waits for the host between calls.
        # Per-call times come from graphs of n back-to-back calls of one kind
        # (events around each replay, on the stream the kernels run on); the
        # commit's graph restores the lengths before each call, and a graph of
        # the restores alone is subtracted.
        def capture(fn, n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(n):
                    assert fn() == 0
            return g

        def graph_s(fn, n, reps=7):
            """Seconds per call of fn, one value per replay of a graph of n calls."""
            g = capture(fn, n)
            g.replay()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in ev:
                a.record(stream)
                g.replay()
                b.record(stream)
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3 / n

        def reps_for(t_est, calls=1):
            # about 2 ms of work per replay
            return int(max(1, min(200, np.ceil(2e-3 / max(t_est * calls, 1e-7)))))

        g_step = capture(one_step, 1)
        for _ in range(args.warmup):
            g_step.replay()
        torch.cuda.synchronize()
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for k in range(args.steps):
            sev[k][0].record(stream)
            g_step.replay()
            sev[k][1].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        assert r.commit_status.item() == 0
        assert np.array_equal(r.len.cpu().numpy(), lens0 + A)
        ms_per_step = elapsed / args.steps * 1e3
        step_s = np.array([a.elapsed_time(b) for a, b in sev]) * 1e-3

        def restore():
            r.len.copy_(len0)
            r.lmax.copy_(lmax0_t)
            return 0

        def restore_commit():
            restore()
            return r.commit()

        def layers():
            rc = 0
            for layer in range(L):
                rc = rc or r.attention(layer)
            return rc

        restore()  # the lengths the timed calls start from (a step leaves them committed)
        x_mask = graph_s(r.build_mask, reps_for(float(np.mean(per_step(0, 1)))))
        x_attn = graph_s(layers, reps_for(float(np.mean(per_step(1, 2, L))), L)) / L
        x_accept = graph_s(r.accept, reps_for(float(np.mean(per_step(2, 3)))))
        n_c = reps_for(float(np.mean(per_step(3, 4))))
        x_commit = graph_s(restore_commit, n_c) - float(np.median(graph_s(restore, n_c)))
        assert r.commit_status.item() == 0
        restore()
        t_mask, t_attn, t_accept, t_commit = (float(np.mean(x)) for x in (x_mask, x_attn, x_accept, x_commit))
        timing = {"mode": "graph", "steps": args.steps, "mask_us": dist_us(x_mask),
                  "attention_us_per_layer": dist_us(x_attn), "accept_us": dist_us(x_accept),
                  "commit_us": dist_us(x_commit), "step_us": dist_us(step_s),
                  "ms_per_step_gpu": float(np.mean(step_s)) * 1e3,
                  "per_call": "one value per replay of a graph of back-to-back calls of that kind, divided by the calls"}

    attn_bytes = algorithmic_bytes_attention(w, lens0, w.T)
    attn_flops = flops_attention(w, lens0, depth)
    commit_bytes = algorithmic_bytes_commit(w, lens0, A, L)
    acc_bytes = algorithmic_bytes_accept(w)
    attn_gbps = attn_bytes / t_attn / 1e9
    commit_gbps = commit_bytes / t_commit / 1e9
    totals = {"attention": t_attn * L, "commit": t_commit, "accept": t_accept, "mask": t_mask}
    dominant = max(totals, key=totals.get)

    def roof(kind):
        if kind == "commit":
            a = commit_gbps
            return {"kernel": "commit_move_kernel (+ commit_finalize_kernel)", "bound": "hbm", "achieved": a,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": a / HBM_PEAK_GBPS,
                    "traffic": measured_traffic(["commit_move_kernel"], w.name),
                    "bytes_per_launch": commit_bytes, "avg_launch_us": t_commit * 1e6}
        if kind == "attention":
            a = attn_gbps
            return {"kernel": "attn_bf16_stream_kernel (+ attn_stream_combine_kernel)", "bound": "hbm",
                    "achieved": a, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": a / HBM_PEAK_GBPS,
                    "traffic": measured_traffic(["attn_bf16_stream_kernel", "attn_stream_combine_kernel"], w.name),
                    "bytes_per_launch": attn_bytes, "avg_launch_us": t_attn * 1e6,
                    "mfma_tflops": attn_flops / t_attn / 1e12,
                    "mfma_frac": attn_flops / t_attn / 1e12 / BF16_PEAK_TFLOPS}
        if kind == "accept":
            a = acc_bytes / t_accept / 1e9
            return {"kernel": "argmax_partial_kernel (+ accept_kernel)", "bound": "hbm", "achieved": a,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": a / HBM_PEAK_GBPS,
                    "traffic": measured_traffic(["argmax_partial_kernel", "accept_kernel"], w.name),
                    "bytes_per_launch": acc_bytes, "avg_launch_us": t_accept * 1e6}
        return {"kernel": "build_mask_kernel", "bound": "latency", "achieved": None, "peak": None,
                "unit": None, "frac": None, "traffic": None, "avg_launch_us": t_mask * 1e6}

    out = {
        "metric": METRIC,
        "value": w.B * w.M / (ms_per_step * 1e-3),
        "unit": "verified tree nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded trees, drafts, logits; device-seeded normal caches)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "M": w.M, "V": w.V,
                   "prefix_len": [w.len_lo, w.len_hi], "layers": L, "sum_len": int(lens0.sum()),
                   "mean_accept_len": float(np.mean(A - 1))},
        "attn_GBps": attn_gbps,
        "attn_frac_hbm": attn_gbps / HBM_PEAK_GBPS,
        "attn_us_per_layer": t_attn * 1e6,
        "commit_us_per_round": t_commit * 1e6,
        "commit_GBps": commit_gbps,
        "accept_us": t_accept * 1e6,
        "mask_us": t_mask * 1e6,
        "verified_nodes_per_s_one_layer": w.B * w.M / (t_mask + t_attn + t_accept),
        "timing": timing,
        "timing_eager": timing_eager,
        "dominant": dominant,
        "roofline": roof(dominant),
        "roofline_attention": roof("attention"),
    }
    # context: the same rates against a live device copy (read + write), and
    # whether one round's attention inputs (distinct per layer) could stay in
    # the Infinity Cache between rounds
    copy = device_copy_gbps(torch)
    out["copy_GBps"] = copy
    out["attn_frac_copy"] = attn_gbps / copy
    out["commit_frac_copy"] = commit_gbps / copy
    out["attn_bytes_per_round_MB"] = attn_bytes * L / 1e6
    out["attn_inputs_fit_infinity_cache"] = bool(attn_bytes * L <= MALL_BYTES)
    if attn_bytes * L < (1 << 30):
        out["attention_cold"] = cold_attention(torch, svt, r, len0, lmax0_t, attn_bytes, attn_flops, eager=args.eager)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, parents, lens0, logits, tokens, seed, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
