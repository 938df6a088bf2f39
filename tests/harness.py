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
