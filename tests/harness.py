"""Shared helpers for the GPU parity tests and the smoke check: build one
seeded round of inputs, run it through libsvt, run the oracle on the same
inputs, compare.  Inputs come only from `synth`; expected values only from
`oracle`."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
from synth import gen
from synth import workloads as wl

# Tolerances (max-abs) of the attention output against the oracle.
TOL_FP32 = 1e-4
TOL_BF16 = 2e-2
# Normalised bound for bf16 (the contract's 2e-2 alone would pass an all-zero
# output when the outputs are small): 1e-2 of the output scale plus 1e-3.
REL_BF16 = 1e-2
ABS_BF16 = 1e-3


@dataclasses.dataclass
class Instance:
    w: wl.Workload
    parents: np.ndarray
    tokens: np.ndarray
    logits: np.ndarray
    lens: np.ndarray
    lmax: int
    cap: int
    q: np.ndarray
    kc: np.ndarray
    vc: np.ndarray
    kt: np.ndarray
    vt: np.ndarray
    tokens_main: np.ndarray


def make_instance(w: wl.Workload, cap_margin: int = 64, seed: int | None = None, poison: bool = True,
                  with_logits: bool = True) -> Instance:
    s = w.seed if seed is None else seed
    parents = wl.trees(w, s)
    lens = wl.lengths(w, s)
    lmax = int(lens.max())
    cap = lmax + cap_margin
    if with_logits:
        logits, tokens, _ = wl.logits_and_drafts(w, parents, s)
    else:
        logits = np.zeros((w.B, w.T, 1), np.float32)
        tokens = np.zeros((w.B, w.T), np.int32)
    q, kc, vc, kt, vt = wl.attention_inputs(w, lens, cap, s, poison=poison)
    tm = gen.randint(gen.stream_key(s, 77), w.B * cap, 0, w.V - 1).astype(np.int32).reshape(w.B, cap)
    return Instance(w, parents, tokens, logits, lens, lmax, cap, q, kc, vc, kt, vt, tm)


def torch_dtype(w: wl.Workload):
    return torch.float32 if w.dtype == "fp32" else torch.bfloat16


def to_dev(x: np.ndarray, w: wl.Workload | None = None, dev="cuda"):
    """numpy -> device tensor; uint16 arrays are bfloat16 bits."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    if x.dtype == np.uint64:
        return torch.from_numpy(x.view(np.int64).copy()).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def out_f32(w: wl.Workload, t: torch.Tensor) -> np.ndarray:
    x = from_dev(t)
    return x.astype(np.float32) if w.dtype == "fp32" else gen.bf16_bits_to_f32(x)


def attn_error(w: wl.Workload, got: np.ndarray, ref: np.ndarray):
    """(max-abs error, allowed max-abs, normalised bound) of an attention output."""
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if got.size else 0.0
    tol = TOL_FP32 if w.dtype == "fp32" else TOL_BF16
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    norm = (1e-5 + 1e-4 * scale) if w.dtype == "fp32" else (REL_BF16 * scale + ABS_BF16)
    return err, tol, norm


def check_attention(w: wl.Workload, got: np.ndarray, ref: np.ndarray, what: str = ""):
    err, tol, norm = attn_error(w, got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"
    assert err <= norm, f"{what}: max-abs error {err:.3e} > normalised bound {norm:.3e}"
    return err


# --------------------------------------------------------------------------
# Where the stream form of svt_verify_attention cuts the batch.  The kernel
# concatenates the key tiles of every (sequence, KV head, query block) unit
# (prefix tiles, then tree tiles) and gives each of `grid` workgroups one
# range of equal cost, a unit costing its tiles plus a set-up charge.  This
# mirrors that rule on the host so that a test can put inputs right after a
# cut; the expected values still come from the oracle alone.
# --------------------------------------------------------------------------
KT = 64


@dataclasses.dataclass
class StreamUnit:
    b: int
    g: int
    qb: int
    base: int          # first stream tile
    ntl: int           # tiles (prefix + tree)
    n_prefix: int      # prefix tiles
    row_lo: int        # query rows [row_lo, row_hi) of the KV head (r = hl * T + i)
    row_hi: int
    cuts: list         # stream tiles inside (base, base + ntl) where a range starts


def stream_plan(B, T, Hq, Hkv, cus, lmax_bound=0, D=128):
    """(nqb, qb_rows, compute waves, set-up charge) of the stream form: at
    most 12 query tiles per unit, 8 when the batch has fewer units than CUs
    and its K/V bound (B Hkv lmax_bound rows of K and V, bf16) is at most
    192 MiB; the units of a KV head split its tiles as evenly as whole tiles
    allow."""
    R = (Hq // Hkv) * T
    nqt = (R + 15) // 16
    few = B * Hkv * ((nqt + 11) // 12) < cus and B * Hkv * lmax_bound * D * 4 <= (192 << 20)
    cap = 8 if few else 12
    nqb = (nqt + cap - 1) // cap
    tpb = (nqt + nqb - 1) // nqb
    nw = tpb if tpb <= 2 else 4 if tpb <= 4 else 6 if tpb <= 6 else 8 if tpb <= 8 else 9 if tpb <= 9 else 12
    pc = 5 if nw >= 9 else 2
    return nqb, tpb * 16, nw, pc


def unit_rows(nqt, nqb, qb, R):
    """Query rows [lo, hi) of query block qb of a KV head."""
    return 16 * ((qb * nqt) // nqb), min(R, 16 * (((qb + 1) * nqt) // nqb))


def stream_grid(B, T, Hq, Hkv, cus, lmax_bound=0, D=128):
    """Ranges of the stream form: one per CU, or for a single sequence the
    largest whole number of ranges per unit that leaves at most a tenth of
    the CUs idle."""
    nqb, _, _, _ = stream_plan(B, T, Hq, Hkv, cus, lmax_bound, D)
    units = Hkv * nqb
    if B == 1 and units <= cus and 10 * units * (cus // units) >= 9 * cus:
        return units * (cus // units)
    return cus


def stream_units(B, T, Hq, Hkv, lens, cus, status=None, lmax_bound=None, D=128):
    """Units of the stream form in stream order, each with the range starts
    that fall strictly inside it (a unit with cuts is merged from partials),
    for a device of `cus` compute units (lmax_bound: the call's host bound,
    by default the longest length)."""
    G = Hq // Hkv
    R = G * T
    bound = (int(np.max(lens)) if len(lens) else 0) if lmax_bound is None else int(lmax_bound)
    grid = stream_grid(B, T, Hq, Hkv, cus, bound, D)
    nqb, qb_rows, nw, pc = stream_plan(B, T, Hq, Hkv, cus, bound, D)
    nqt = (R + 15) // 16
    ntree = (T + KT - 1) // KT
    tiles = []
    for b in range(B):
        ok = status is None or int(status[b]) == 0
        tiles.append((int(lens[b]) + KT - 1) // KT + ntree if ok else 0)
    pref = [0]
    npref = [0]
    for b in range(B):
        pref.append(pref[-1] + tiles[b])
        npref.append(npref[-1] + (1 if tiles[b] > 0 else 0))
    upb = Hkv * nqb
    N = upb * pref[B]

    def seq_cost(b):
        return upb * (pref[b] + pc * npref[b])

    CT = seq_cost(B)

    def cost_to_tile(p):
        if p >= CT:
            return N
        lo, hi = 0, B
        while hi - lo > 1:
            m = (lo + hi) // 2
            if seq_cost(m) <= p:
                lo = m
            else:
                hi = m
        ntl = pref[lo + 1] - pref[lo]
        off = p - seq_cost(lo)
        j, r = divmod(off, ntl + pc)
        return upb * pref[lo] + j * ntl + max(0, r - pc)

    starts = sorted({cost_to_tile((c * CT) // grid) for c in range(grid)})
    units = []
    for b in range(B):
        ntl = tiles[b]
        if ntl == 0:
            continue
        for j in range(upb):
            base = upb * pref[b] + j * ntl
            g, qb = divmod(j, nqb)
            cuts = [x for x in starts if base < x < base + ntl]
            units.append(StreamUnit(b, g, qb, base, ntl, ntl - ntree, *unit_rows(nqt, nqb, qb, R), cuts))
    return units


def run_attention(q, kc, vc, kt, vt, parents, lens, lmax_bound=None, status=None, scale=0.0, form=0, dev="cuda",
                  split_keys=0):
    """svt_build_mask then svt_verify_attention on host arrays (bf16 as uint16
    bits).  The mask and tree status handed back for the comparison are the
    oracle's own, built from the parent arrays, after asserting that the GPU's
    equal them bit for bit; `status`, when given, overrides the tree status
    that attention sees (and is handed back).  Returns (rc, out tensor, mask,
    status, seq_status)."""
    from tree_masked_verification_parent_amd import svt

    def i32(x):
        return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=dev)

    lens = np.asarray(lens, np.int32)
    lmax = int(lens.max()) if len(lens) else 0
    B, T = parents.shape
    M = T - 1
    Wd = (T + 63) // 64
    mk = torch.zeros(B, T, Wd, dtype=torch.int64, device=dev)
    dp = torch.zeros(B, T, dtype=torch.int32, device=dev)
    st_mask = torch.zeros(B, dtype=torch.int32, device=dev)
    assert svt.svt_build_mask(i32(parents), M, mk, dp, st_mask) == 0
    st = st_mask if status is None else i32(status)
    tq, tkc, tvc, tkt, tvt = (to_dev(x, dev=dev) for x in (q, kc, vc, kt, vt))
    out = torch.full(tq.shape, float("nan"), dtype=tq.dtype, device=dev)
    sst = torch.full((B,), 55, dtype=torch.int32, device=dev)
    ln_t, lm_t = i32(lens), i32([lmax])
    bound = lmax if lmax_bound is None else lmax_bound
    args = svt.attn_args(tq, tkc, tvc, ln_t, lm_t, bound, tkt, tvt, mk, out, status=st, seq_status=sst,
                         scale=scale, form=form, split_keys=split_keys)
    need = svt.svt_verify_attention_workspace(args)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = svt.attn_args(tq, tkc, tvc, ln_t, lm_t, bound, tkt, tvt, mk, out, status=st, seq_status=sst,
                         scale=scale, workspace=ws, form=form, split_keys=split_keys)
    rc = svt.svt_verify_attention(args)
    torch.cuda.synchronize()
    _, ost = oracle.validate(parents, M)
    omk, _ = oracle.mask(parents, M, ost)
    assert np.array_equal(from_dev(mk).view(np.uint64), omk), "GPU mask differs from the oracle's"
    assert np.array_equal(from_dev(st_mask), ost), "GPU tree status differs from the oracle's"
    return rc, out, omk, (ost if status is None else np.asarray(status, np.int32)), from_dev(sst)


def accept_chunking(rows: int, V: int):
    """(chunks per row, entries per chunk) of svt_accept's argmax pass, as its
    plan cuts a row: the fewer of chunks of >= 4096 entries and ~2048
    workgroups over the chip, then more chunks so none exceeds 5120 entries,
    chunk length rounded up to a multiple of 4."""
    nchunk = 1
    if rows > 0:
        by_size = (V + 4095) // 4096
        by_par = (2048 + rows - 1) // rows
        by_cap = (V + 5119) // 5120
        nchunk = max(min(by_size, by_par), by_cap, 1)
    chunk = (V + nchunk - 1) // nchunk
    chunk = (chunk + 3) & ~3
    return (V + chunk - 1) // chunk, chunk


def cu_count(dev=0) -> int:
    return int(torch.cuda.get_device_properties(dev).multi_processor_count)
