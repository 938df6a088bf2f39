"""Python binding of libsvt: argument marshalling only.

Each function here has the name of a C entry point declared in include/svt.h,
takes torch tensors for the device buffers, passes their data pointers and the
current HIP stream to the library, and returns the library's status code.
PyTorch only provides device memory and streams; every step of the path runs
in libsvt's kernels.  There is no fallback: if the library is missing or the
tensors are not on the GPU, these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SVT_SANITIZE=1 loads the build whose host code carries AddressSanitizer and
# UBSan (see build.py); the device code is the same.
LIB_PATH = os.path.join(_HERE, "libsvt_san.so" if os.environ.get("SVT_SANITIZE", "0") not in ("", "0")
                        else "libsvt.so")

SVT_OK = 0
SVT_ERR_ARG = -1
SVT_ERR_UNSUPPORTED = -2
SVT_ERR_TREE_ROOT = -3
SVT_ERR_TREE_RANGE = -4
SVT_ERR_TREE_CYCLE = -5
SVT_ERR_CAPACITY = -6
SVT_ERR_WORKSPACE = -7
SVT_ERR_HIP = -8
SVT_ERR_LENGTH = -9
SVT_FP32 = 0
SVT_BF16 = 1
SVT_SYNC_CHECK = 1
SVT_ATTN_AUTO, SVT_ATTN_SPLIT, SVT_ATTN_STREAM = 0, 1, 2
SVT_COMMIT_REPAD, SVT_COMMIT_APPEND = 0, 1
SVT_MASK_ADD_FP32, SVT_MASK_ADD_BF16, SVT_MASK_BOOL = 0, 1, 2

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class AttnArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("M", _I32), ("Hq", _I32), ("Hkv", _I32), ("D", _I32), ("dtype", _I32),
                ("scale", ctypes.c_float), ("q", _P), ("k_cache", _P), ("v_cache", _P), ("cap", _I64),
                ("len", _P), ("lmax", _P), ("lmax_bound", _I32), ("k_tree", _P), ("v_tree", _P), ("mask", _P),
                ("status", _P), ("out", _P), ("seq_status", _P), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t), ("form", _I32), ("seq_slot", _P), ("n_slots", _I32),
                ("split_keys", _I32)]


class AcceptArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("M", _I32), ("V", _I32), ("logits", _P), ("tree_tokens", _P), ("parents", _P),
                ("mask", _P), ("depth", _P), ("status", _P), ("amax", _P), ("accept_len", _P), ("path", _P),
                ("bonus", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class CommitArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("M", _I32), ("Hkv", _I32), ("D", _I32), ("n_layers", _I32), ("dtype", _I32),
                ("cap", _I64), ("kv_main", _P), ("kv_branch", _P), ("tokens_main", _P), ("tree_tokens", _P),
                ("len", _P), ("lmax", _P), ("pos_ids", _P), ("path", _P), ("accept_len", _P), ("status", _P),
                ("commit_status", _P), ("seq_slot", _P), ("n_slots", _I32), ("mode", _I32), ("len_out", _P),
                ("lmax_out", _P)]


class RealignArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("Hkv", _I32), ("D", _I32), ("n_layers", _I32), ("dtype", _I32), ("cap", _I64),
                ("kv_main", _P), ("tokens_main", _P), ("pos_ids", _P), ("seq_slot", _P), ("n_slots", _I32),
                ("len", _P), ("end", _P), ("lmax", _P), ("realign_status", _P)]


EXPORTS = ["svt_build_mask", "svt_expand_mask", "svt_verify_attention_workspace", "svt_verify_attention",
           "svt_accept_workspace", "svt_accept", "svt_accept_noalloc", "svt_commit", "svt_commit_length",
           "svt_realign", "svt_pool_pick", "svt_check_status", "svt_status_string", "svt_version"]

_lib = None


def lib():
    """Load libsvt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m tree_masked_verification_parent_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.svt_build_mask.argtypes = [_P, _I32, _I32, _P, _P, _P, _I32, _P]
        L.svt_build_mask.restype = ctypes.c_int
        L.svt_verify_attention_workspace.argtypes = [ctypes.POINTER(AttnArgs)]
        L.svt_verify_attention_workspace.restype = ctypes.c_size_t
        L.svt_verify_attention.argtypes = [ctypes.POINTER(AttnArgs), _P]
        L.svt_verify_attention.restype = ctypes.c_int
        L.svt_accept_workspace.argtypes = [ctypes.POINTER(AcceptArgs)]
        L.svt_accept_workspace.restype = ctypes.c_size_t
        L.svt_accept.argtypes = [ctypes.POINTER(AcceptArgs), _P]
        L.svt_accept.restype = ctypes.c_int
        L.svt_accept_noalloc.argtypes = [ctypes.POINTER(AcceptArgs), _P]
        L.svt_accept_noalloc.restype = ctypes.c_int
        L.svt_commit.argtypes = [ctypes.POINTER(CommitArgs), _I32, _P]
        L.svt_commit.restype = ctypes.c_int
        L.svt_commit_length.argtypes = [ctypes.POINTER(CommitArgs), _I32, _P]
        L.svt_commit_length.restype = ctypes.c_int
        L.svt_expand_mask.argtypes = [_P, _P, _P, _I32, _I32, _I32, _P, _I32, _P, _P]
        L.svt_expand_mask.restype = ctypes.c_int
        L.svt_realign.argtypes = [ctypes.POINTER(RealignArgs), _I32, _P]
        L.svt_realign.restype = ctypes.c_int
        L.svt_pool_pick.argtypes = [_P, _P, _I32, _I32, _I32, _P, _P]
        L.svt_pool_pick.restype = ctypes.c_int
        L.svt_check_status.argtypes = [_P, _I32, _P]
        L.svt_check_status.restype = ctypes.c_int
        L.svt_status_string.argtypes = [ctypes.c_int]
        L.svt_status_string.restype = ctypes.c_char_p
        L.svt_version.argtypes = []
        L.svt_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("libsvt buffers must be GPU tensors")
    if not t.is_contiguous():
        raise ValueError("libsvt buffers must be contiguous")
    return t.data_ptr()


def _keep(args, *tensors):
    """The argument structs hold raw device pointers; keep the tensors they
    point into alive for as long as the struct is."""
    args._tensors = tuple(t for t in tensors if t is not None)
    return args


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def status_string(code: int) -> str:
    return lib().svt_status_string(int(code)).decode()


def version() -> str:
    return lib().svt_version().decode()


def svt_build_mask(parents, M: int, mask, depth, status, flags: int = 0, stream=None) -> int:
    B = parents.shape[0] if parents.dim() > 1 else 1
    return lib().svt_build_mask(_ptr(parents), B, M, _ptr(mask), _ptr(depth), _ptr(status), flags, _stream(stream))


def svt_expand_mask(mask, status, lens, M: int, lmax: int, out, kind: int, seq_status=None, stream=None) -> int:
    """out: [B][1][T][lmax + T] of float32 (SVT_MASK_ADD_FP32), bfloat16
    (SVT_MASK_ADD_BF16) or uint8 (SVT_MASK_BOOL)."""
    B = mask.shape[0]
    want = {SVT_MASK_ADD_FP32: torch.float32, SVT_MASK_ADD_BF16: torch.bfloat16, SVT_MASK_BOOL: torch.uint8}
    if kind in want and (out.dtype != want[kind] or out.numel() != B * (M + 1) * (lmax + M + 1)):
        raise ValueError("out must be [B][1][T][lmax + T] of the kind's dtype")
    return lib().svt_expand_mask(_ptr(mask), _ptr(status), _ptr(lens), B, M, int(lmax), _ptr(out), int(kind),
                                 _ptr(seq_status), _stream(stream))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return SVT_FP32
    if t.dtype == torch.bfloat16:
        return SVT_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def attn_args(q, k_cache, v_cache, lens, lmax, lmax_bound: int, k_tree, v_tree, mask, out, status=None,
              seq_status=None, scale: float = 0.0, workspace=None, form: int = 0, seq_slot=None,
              split_keys: int = 0) -> AttnArgs:
    B, T, Hq, D = q.shape
    a = AttnArgs()
    a.B, a.M, a.Hq, a.Hkv, a.D = B, T - 1, Hq, k_cache.shape[1], D
    a.dtype = _dtype_code(q)
    a.scale = scale
    a.q, a.k_cache, a.v_cache = _ptr(q), _ptr(k_cache), _ptr(v_cache)
    a.cap = k_cache.shape[2]
    a.len, a.lmax, a.lmax_bound = _ptr(lens), _ptr(lmax), int(lmax_bound)
    a.k_tree, a.v_tree, a.mask = _ptr(k_tree), _ptr(v_tree), _ptr(mask)
    a.status, a.out, a.seq_status = _ptr(status), _ptr(out), _ptr(seq_status)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.form = int(form)
    a.seq_slot = _ptr(seq_slot)
    a.n_slots = k_cache.shape[0] if seq_slot is not None else 0
    a.split_keys = int(split_keys)
    return _keep(a, q, k_cache, v_cache, lens, lmax, k_tree, v_tree, mask, out, status, seq_status, workspace, seq_slot)


def svt_verify_attention_workspace(args: AttnArgs) -> int:
    return lib().svt_verify_attention_workspace(ctypes.byref(args))


def svt_verify_attention(args: AttnArgs, stream=None) -> int:
    return lib().svt_verify_attention(ctypes.byref(args), _stream(stream))


def accept_args(logits, tree_tokens, parents, mask, depth, amax, accept_len, path, bonus, status=None,
                workspace=None) -> AcceptArgs:
    B, T, V = logits.shape
    a = AcceptArgs()
    a.B, a.M, a.V = B, T - 1, V
    a.logits, a.tree_tokens, a.parents = _ptr(logits), _ptr(tree_tokens), _ptr(parents)
    a.mask, a.depth, a.status = _ptr(mask), _ptr(depth), _ptr(status)
    a.amax, a.accept_len, a.path, a.bonus = _ptr(amax), _ptr(accept_len), _ptr(path), _ptr(bonus)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _keep(a, logits, tree_tokens, parents, mask, depth, status, amax, accept_len, path, bonus, workspace)


def svt_accept_workspace(args: AcceptArgs) -> int:
    return lib().svt_accept_workspace(ctypes.byref(args))


def svt_accept(args: AcceptArgs, stream=None) -> int:
    return lib().svt_accept(ctypes.byref(args), _stream(stream))


SVT_ACCEPT_NOALLOC_SCRATCH = 4 << 20


def svt_accept_noalloc(args: AcceptArgs, stream=None) -> int:
    """svt_accept with the library's static scratch (args.workspace ignored)."""
    return lib().svt_accept_noalloc(ctypes.byref(args), _stream(stream))


def commit_args(kv_main, kv_branch, lens, lmax, path, accept_len, commit_status, tokens_main=None,
                tree_tokens=None, pos_ids=None, status=None, seq_slot=None, mode: int = SVT_COMMIT_REPAD,
                len_out=None, lmax_out=None) -> CommitArgs:
    Lyr, two, rows, Hkv, cap, D = kv_main.shape
    B = kv_branch.shape[2]
    if seq_slot is None and rows != B:
        raise ValueError("kv_main and kv_branch disagree on the batch size (pass seq_slot for a pool)")
    a = CommitArgs()
    a.B, a.M, a.Hkv, a.D, a.n_layers = B, kv_branch.shape[4] - 1, Hkv, D, Lyr
    a.dtype = _dtype_code(kv_main)
    a.cap = cap
    a.kv_main, a.kv_branch = _ptr(kv_main), _ptr(kv_branch)
    a.tokens_main, a.tree_tokens = _ptr(tokens_main), _ptr(tree_tokens)
    a.len, a.lmax, a.pos_ids = _ptr(lens), _ptr(lmax), _ptr(pos_ids)
    a.path, a.accept_len, a.status, a.commit_status = _ptr(path), _ptr(accept_len), _ptr(status), _ptr(commit_status)
    a.seq_slot = _ptr(seq_slot)
    a.n_slots = rows if seq_slot is not None else 0
    a.mode = int(mode)
    a.len_out, a.lmax_out = _ptr(len_out), _ptr(lmax_out)
    return _keep(a, kv_main, kv_branch, tokens_main, tree_tokens, lens, lmax, pos_ids, path, accept_len, status,
                 commit_status, seq_slot, len_out, lmax_out)


def svt_commit(args: CommitArgs, flags: int = 0, stream=None) -> int:
    return lib().svt_commit(ctypes.byref(args), flags, _stream(stream))


def svt_commit_length(args: CommitArgs, flags: int = 0, stream=None) -> int:
    return lib().svt_commit_length(ctypes.byref(args), flags, _stream(stream))


def svt_check_status(status, n: int, stream=None) -> int:
    return lib().svt_check_status(_ptr(status), n, _stream(stream))


def realign_args(kv_main, lens, end, lmax, realign_status, tokens_main=None, pos_ids=None,
                 seq_slot=None) -> RealignArgs:
    Lyr, two, rows, Hkv, cap, D = kv_main.shape
    B = lens.shape[0]
    if seq_slot is None and rows != B:
        raise ValueError("kv_main rows differ from the batch size (pass seq_slot for a pool)")
    a = RealignArgs()
    a.B, a.Hkv, a.D, a.n_layers = B, Hkv, D, Lyr
    a.dtype = _dtype_code(kv_main)
    a.cap = cap
    a.kv_main, a.tokens_main, a.pos_ids = _ptr(kv_main), _ptr(tokens_main), _ptr(pos_ids)
    a.seq_slot = _ptr(seq_slot)
    a.n_slots = rows if seq_slot is not None else 0
    a.len, a.end, a.lmax, a.realign_status = _ptr(lens), _ptr(end), _ptr(lmax), _ptr(realign_status)
    return _keep(a, kv_main, tokens_main, pos_ids, seq_slot, lens, end, lmax, realign_status)


def svt_realign(args: RealignArgs, flags: int = 0, stream=None) -> int:
    return lib().svt_realign(ctypes.byref(args), flags, _stream(stream))


def svt_pool_pick(end_host, active_host, max_batch: int, min_group: int):
    """Host call.  end_host / active_host: int32 numpy arrays of the pool.
    Returns (rc, slots): rc 1 = equal ends, 0 = mixed, < 0 = error."""
    import numpy as np
    end = np.ascontiguousarray(end_host, dtype=np.int32)
    act = np.ascontiguousarray(active_host, dtype=np.int32)
    if end.shape != act.shape:
        raise ValueError("end and active differ in length")
    out = np.zeros(max(1, max_batch), dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    rc = lib().svt_pool_pick(end.ctypes.data, act.ctypes.data, end.shape[0], int(max_batch), int(min_group),
                             out.ctypes.data, n.ctypes.data)
    return rc, out[: int(n[0])].copy()
