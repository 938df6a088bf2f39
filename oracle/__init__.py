"""CPU oracle for tree-masked verification (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It wraps the plain C oracle in `svt_oracle.c` with
numpy-friendly functions; it never touches the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svt_oracle.c")
# SVT_SANITIZE=1 selects an AddressSanitizer + UBSan build (clang's runtime,
# which the process must preload), kept apart from the normal library.
SANITIZE = os.environ.get("SVT_SANITIZE", "0") not in ("", "0")
_LIB = os.path.join(_HERE, "libsvt_oracle_san.so" if SANITIZE else "libsvt_oracle.so")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
             "-shared-libasan"]

OK, ERR_ARG, ERR_TREE_ROOT, ERR_TREE_RANGE, ERR_TREE_CYCLE, ERR_CAPACITY, ERR_LENGTH = 0, -1, -3, -4, -5, -6, -9


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (ISO C11: no FMA contraction, no fast-math),
    or with clang and AddressSanitizer + UBSan when SVT_SANITIZE=1."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        if SANITIZE:
            cmd = [CLANG, "-O1", "-std=c11", "-Wall", "-Wextra", *SAN_FLAGS, "-shared", "-fPIC", _SRC, "-lm",
                   "-o", tmp]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-lm", "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_validate.argtypes = [P, i32, i32, P]
        L.oracle_validate.restype = ctypes.c_int
        L.oracle_mask.argtypes = [P, i32, i32, P, P, P]
        L.oracle_mask.restype = None
        L.oracle_attention.argtypes = [P, P, P, P, P, P, P, i32, i64, P, i32, i32, i32, i32, i32, dbl, P]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_attention_row.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, dbl, P]
        L.oracle_attention_row.restype = None
        L.oracle_argmax.argtypes = [P, i64, i32, P]
        L.oracle_argmax.restype = None
        L.oracle_accept.argtypes = [P, P, P, P, i32, i32, P, P, P]
        L.oracle_accept.restype = None
        L.oracle_commit.argtypes = [P, P, i32, i32, i32, i64, i32, i32, P, P, P, P, P, P, P, P, i32, P, i32]
        L.oracle_commit.restype = ctypes.c_int
        L.oracle_realign.argtypes = [P, i32, i32, i32, i64, i32, P, P, P, i32, P, P, P]
        L.oracle_realign.restype = ctypes.c_int
        L.oracle_expand_mask.argtypes = [P, P, P, i32, i32, i32, P, P]
        L.oracle_expand_mask.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def validate(parents: np.ndarray, M: int):
    par = _c(parents, np.int32).reshape(-1, M + 1)
    st = np.zeros(par.shape[0], dtype=np.int32)
    first = lib().oracle_validate(_p(par), par.shape[0], M, _p(st))
    return first, st


def mask(parents: np.ndarray, M: int, status=None):
    par = _c(parents, np.int32).reshape(-1, M + 1)
    B, T = par.shape
    W = (T + 63) // 64
    mk = np.zeros((B, T, W), dtype=np.uint64)
    dp = np.zeros((B, T), dtype=np.int32)
    st = None if status is None else _c(status, np.int32)
    lib().oracle_mask(_p(par), B, M, _p(st), _p(mk), _p(dp))
    return mk, dp


def attention(q, k_cache, v_cache, k_tree, v_tree, mk, lens, lmax: int, status=None,
              scale: float | None = None):
    """All tensor inputs float32 (exact upcasts).  Returns (rc, out float64)."""
    q = _c(q, np.float32)
    B, T, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    kc, vc = _c(k_cache, np.float32), _c(v_cache, np.float32)
    kt, vt = _c(k_tree, np.float32), _c(v_tree, np.float32)
    mk = _c(mk, np.uint64)
    ln = _c(lens, np.int32)
    st = None if status is None else _c(status, np.int32)
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    sc = (1.0 / np.sqrt(D)) if scale is None else scale
    rc = lib().oracle_attention(_p(q), _p(kc), _p(vc), _p(kt), _p(vt), _p(mk), _p(ln), int(lmax), cap,
                                _p(st), B, T - 1, Hq, Hkv, D, float(sc), _p(out))
    return rc, out


def attention_row(q_row, k_cache_bh, v_cache_bh, k_tree_bh, v_tree_bh, mask_row, len_b: int,
                  lmax: int, scale: float):
    q_row = _c(q_row, np.float32)
    D = q_row.shape[0]
    kc, vc = _c(k_cache_bh, np.float32), _c(v_cache_bh, np.float32)
    kt, vt = _c(k_tree_bh, np.float32), _c(v_tree_bh, np.float32)
    mr = _c(mask_row, np.uint64)
    out = np.zeros(D, dtype=np.float64)
    lib().oracle_attention_row(_p(q_row), _p(kc), _p(vc), _p(kt), _p(vt), _p(mr), int(len_b), int(lmax),
                               kt.shape[0], D, float(scale), _p(out))
    return out


def default_threads() -> int:
    """Threads for the row-parallel drivers: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def attention_rows(q, k_cache, v_cache, k_tree, v_tree, mk, lens, lmax: int, rows, scale: float | None = None,
                   threads: int | None = None, to_f32=None):
    """oracle_attention_row for the listed (b, i, h) rows, run on `threads`
    threads (ctypes releases the GIL during each call; the C function keeps
    no shared state).  Array inputs in the layouts of `attention`: float32
    (exact upcasts), or any dtype that `to_f32` maps exactly to float32 (it is
    applied to each (sequence, KV head) slab and query row as it is used, so
    a large bf16 cache is never upcast whole).  Returns float64
    [len(rows)][D].  Every row is computed by the same single-threaded C
    routine; the threads only run rows side by side."""
    import concurrent.futures as cf

    B, T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = (1.0 / np.sqrt(D)) if scale is None else float(scale)
    mk = _c(mk, np.uint64)
    out = np.zeros((len(rows), D), dtype=np.float64)
    groups: dict = {}
    for k, (b, i, h) in enumerate(rows):
        groups.setdefault((int(b), int(h) // G), []).append((k, int(i), int(h)))

    f = (lambda x: x) if to_f32 is None else to_f32
    import threading

    n = default_threads() if threads is None else max(1, int(threads))
    # tasks: chunks of one group's rows, enough of them to keep every thread busy
    per = max(1, -(-n // max(1, len(groups))))
    tasks = []
    for key, lst in groups.items():
        step = max(1, -(-len(lst) // per))
        for s0 in range(0, len(lst), step):
            tasks.append((key, lst[s0:s0 + step]))
    left = {key: sum(1 for k2, _ in tasks if k2 == key) for key in groups}
    slabs: dict = {}
    locks = {key: threading.Lock() for key in groups}

    def get_slabs(key):
        # each (sequence, KV head) slab is converted once and dropped after its last chunk
        with locks[key]:
            if key not in slabs:
                b, g = key
                slabs[key] = tuple(_c(f(x[b, g]), np.float32) for x in (k_cache, v_cache, k_tree, v_tree))
            return slabs[key]

    def done(key):
        with locks[key]:
            left[key] -= 1
            if left[key] == 0:
                slabs.pop(key, None)

    def run(task):
        key, lst = task
        b, _ = key
        kc, vc, kt, vt = get_slabs(key)
        for k, i, h in lst:
            qr = _c(f(q[b, i, h]), np.float32)
            lib().oracle_attention_row(_p(qr), _p(kc), _p(vc), _p(kt), _p(vt), _p(mk[b, i]), int(lens[b]),
                                       int(lmax), T, D, sc, _p(out[k]))
        done(key)

    lib()  # load once, before any thread calls it
    if n == 1:
        for t in tasks:
            run(t)
    else:
        with cf.ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(run, tasks))
    return out


def argmax(logits: np.ndarray):
    x = _c(logits, np.float32)
    V = x.shape[-1]
    rows = x.size // V
    am = np.zeros(rows, dtype=np.int32)
    lib().oracle_argmax(_p(x), rows, V, _p(am))
    return am.reshape(x.shape[:-1])


def accept(amax, tree_tokens, parents, M: int, status=None):
    am = _c(amax, np.int32).reshape(-1, M + 1)
    tok = _c(tree_tokens, np.int32).reshape(-1, M + 1)
    par = _c(parents, np.int32).reshape(-1, M + 1)
    B = par.shape[0]
    st = None if status is None else _c(status, np.int32)
    al = np.zeros(B, dtype=np.int32)
    path = np.zeros((B, M + 1), dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    lib().oracle_accept(_p(am), _p(tok), _p(par), _p(st), B, M, _p(al), _p(path), _p(bonus))
    return al, path, bonus


def commit(kv_main: np.ndarray, kv_branch: np.ndarray, M: int, tokens_main, tree_tokens, lens,
           lmax: int, path, accept_len, status=None, want_pos_ids: bool = True, mode: int = 0, slot=None):
    """kv_main [L][2][rows][Hkv][cap][...] and kv_branch [L][2][B][Hkv][T][...] of
    any dtype (raw bytes are moved); rows = B unless `slot` maps each sequence
    to a pool row.  mode 0 re-pads (EQSPEC), 1 appends (EXSPEC).  path None is
    the length-based commit (branch rows [0, A) in step order).  Works on
    copies; returns (rc, kv_main', tokens_main', lens', lmax', pos_ids)."""
    km = np.array(kv_main, copy=True, order="C")
    kb = _c(kv_branch, kv_branch.dtype)
    L, _, rows, Hkv, cap = km.shape[:5]
    B = len(lens)
    row_bytes = km[0, 0, 0, 0, 0].nbytes if km.size else 0
    tm = None if tokens_main is None else np.array(tokens_main, dtype=np.int32, copy=True, order="C")
    tt = _c(tree_tokens, np.int32)
    ln = np.array(lens, dtype=np.int32, copy=True)
    lm = np.array([lmax], dtype=np.int32)
    pos = np.zeros((rows, cap), dtype=np.int32) if want_pos_ids else None
    st = None if status is None else _c(status, np.int32)
    sl = None if slot is None else _c(slot, np.int32)
    rc = lib().oracle_commit(_p(km.view(np.uint8)), _p(kb.view(np.uint8)), L, B, Hkv, cap, row_bytes, M,
                             _p(tm), _p(tt), _p(ln), _p(lm), _p(pos), _p(None if path is None else _c(path, np.int32)),
                             _p(_c(accept_len, np.int32)), _p(st), int(mode), _p(sl), rows)
    return rc, km, tm, ln, int(lm[0]), pos


def realign(kv_main: np.ndarray, lens, ends, tokens_main=None, slot=None, want_pos_ids: bool = True):
    """Moves each sequence's content [end_b - len_b, end_b) to end at the
    largest end.  kv_main [L][2][rows][Hkv][cap][...].  Works on copies;
    returns (rc, kv_main', tokens_main', lmax', pos_ids)."""
    km = np.array(kv_main, copy=True, order="C")
    L, _, rows, Hkv, cap = km.shape[:5]
    B = len(lens)
    row_bytes = km[0, 0, 0, 0, 0].nbytes if km.size else 0
    tm = None if tokens_main is None else np.array(tokens_main, dtype=np.int32, copy=True, order="C")
    pos = np.zeros((rows, cap), dtype=np.int32) if want_pos_ids else None
    sl = None if slot is None else _c(slot, np.int32)
    lm = np.zeros(1, dtype=np.int32)
    rc = lib().oracle_realign(_p(km.view(np.uint8)), L, B, Hkv, cap, row_bytes, _p(tm), _p(pos), _p(sl), rows,
                              _p(_c(lens, np.int32)), _p(_c(ends, np.int32)), _p(lm))
    return rc, km, tm, int(lm[0]), pos


def expand_mask(parents, lens, lmax: int, status=None):
    """Dense tree mask from the parent arrays: (codes [B], open [B][T][lmax+T] bool)."""
    par = _c(parents, np.int32)
    B, T = par.shape
    openm = np.zeros((B, T, lmax + T), dtype=np.uint8)
    codes = np.zeros(B, dtype=np.int32)
    lib().oracle_expand_mask(_p(par), _p(_c(lens, np.int32)), _p(None if status is None else _c(status, np.int32)),
                             B, T - 1, int(lmax), _p(openm), _p(codes))
    return codes, openm.astype(bool)
