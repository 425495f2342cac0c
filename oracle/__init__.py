"""ctypes wrapper of the fp64 C oracle of the QSA layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package's smoke check
and the CPU-baseline leg of the benchmark, never by the product path.  It
shares no code with the HIP library; inputs come from the ``synth`` module.
Parity unpinned by the pages for end-to-end values: the pages print no worked
example, so the oracle is pinned by closed forms, brute force and invariants
(see tests/test_oracle_*.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_oracle.so")
# A test that plants a mistake in the oracle builds a mutated copy and points
# this variable at it (tests/test_oracle_mutations.py).
_LIB_OVERRIDE = os.environ.get("QSA_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``libqsa_oracle.so`` (gcc, -O2, OpenMP over query rows)."""
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = f"{_LIB_PATH}.tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.qsa_oracle_rope.argtypes = [vp, vp, i64, i32, i32, i32, dbl, i64, vp]
        lib.qsa_oracle_rope.restype = None
        lib.qsa_oracle_compress.argtypes = [vp, i64, i32, i32, i32, vp]
        lib.qsa_oracle_compress_ext.argtypes = [vp, i64, i32, i32, i32, vp, i32, dbl, i64, vp]
        lib.qsa_oracle_compress_ext.restype = None
        lib.qsa_oracle_compress.restype = None
        lib.qsa_oracle_num_complete.argtypes = [i64, i32]
        lib.qsa_oracle_num_threads.restype = i32
        lib.qsa_oracle_num_threads.argtypes = []
        lib.qsa_oracle_num_complete.restype = i64
        lib.qsa_oracle_scores_row.argtypes = [vp, vp, i64, i64, i32, i32, i32, i32, vp]
        lib.qsa_oracle_scores_row.restype = i64
        lib.qsa_oracle_topk_row.argtypes = [vp, i64, i32, vp, vp, vp]
        lib.qsa_oracle_topk_row.restype = i32
        lib.qsa_oracle_token_set.argtypes = [vp, i32, i64, i32, vp]
        lib.qsa_oracle_token_set.restype = i64
        lib.qsa_oracle_token_set_reuse.argtypes = [vp, i32, i64, i64, i32, vp]
        lib.qsa_oracle_token_set_reuse.restype = i64
        lib.qsa_oracle_attend_row.argtypes = [vp, vp, vp, i32, i32, i32, vp, i64, vp, vp, vp]
        lib.qsa_oracle_attend_row.restype = None
        lib.qsa_oracle_qsa_rows.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32,
                                            i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp,
                                            vp, vp]
        lib.qsa_oracle_qsa_rows.restype = None
        lib.qsa_oracle_qsa_rows_at.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, i32, i32, i32,
                                               i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp,
                                               vp]
        lib.qsa_oracle_qsa_rows_at.restype = None
        lib.qsa_oracle_sparse_attn_rows.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, i32,
                                                    vp, i64, vp, vp, vp, vp]
        lib.qsa_oracle_sparse_attn_rows.restype = None
        lib.qsa_oracle_sparse_attn_rows_at.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                       i64, vp, vp, vp, vp]
        lib.qsa_oracle_sparse_attn_rows_at.restype = None
        lib.qsa_oracle_select_rows.argtypes = [vp, vp, i64, i64, i32, i32, i32, i32, i32, vp,
                                               i64, vp, i64, vp, vp, vp, vp]
        lib.qsa_oracle_select_rows.restype = None
        lib.qsa_oracle_dense_rows.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, i64, vp, vp]
        lib.qsa_oracle_dense_rows.restype = None
        lib.qsa_oracle_distill_row.argtypes = [vp, vp, i32, i32, i32, i64, i32, vp, vp, vp]
        lib.qsa_oracle_distill_row.restype = dbl
        lib.qsa_oracle_distill_rows.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32,
                                                i32, i32, vp, i64, vp]
        lib.qsa_oracle_distill_rows.restype = None
        lib.qsa_oracle_sparse_kl_row.argtypes = [vp, vp, i32, i32, i32, i64, i32, vp, i32, vp,
                                                 vp, vp]
        lib.qsa_oracle_sparse_kl_row.restype = dbl
        lib.qsa_oracle_sparse_kl_rows.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32,
                                                  i32, i32, i32, i32, vp, i64, vp, vp, vp]
        lib.qsa_oracle_sparse_kl_rows.restype = None
        lib.qsa_oracle_f64_to_bf16.argtypes = [dbl]
        lib.qsa_oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.qsa_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.qsa_oracle_bf16_to_f64.restype = dbl
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data


def _check_rows(name, rows, n_rows, positions, Tk, sel=None, nsel=None, r=4):
    """Reject inputs that would make the C loops read outside the arrays:
    rows outside the query array, positions outside the key array, selected
    blocks that are not complete blocks of their row's position."""
    if rows is not None and rows.size and (rows.min() < 0 or rows.max() >= n_rows):
        raise ValueError(f"{name}: a row lies outside the {n_rows} query rows")
    if positions.size and (positions.min() < 0 or positions.max() >= Tk):
        raise ValueError(f"{name}: a query position lies outside the {Tk} keys")
    if sel is not None:
        if nsel.size != positions.size or sel.shape[0] != positions.size:
            raise ValueError(f"{name}: selection rows do not match the query rows")
        if nsel.size and (nsel.min() < 0 or nsel.max() > sel.shape[1]):
            raise ValueError(f"{name}: a selection count exceeds the budget")
        nc = (positions + 1) // r
        for i in range(positions.size):
            b = sel[i, :nsel[i]]
            if b.size and (b.min() < 0 or b.max() >= nc[i]):
                raise ValueError(f"{name}: row {i} selects a block that is not complete at "
                                 f"position {positions[i]}")


MODE_MAXHEAD, MODE_RELUSUM = 0, 1
KBAR_MEAN, KBAR_RMSNORM = 0, 1


def f64_to_bf16(x: float) -> int:
    return int(_load().qsa_oracle_f64_to_bf16(float(x)))


def bf16_to_f64(h: int) -> float:
    return float(_load().qsa_oracle_bf16_to_f64(int(h)))


def rope(x: np.ndarray, rope_dim: int = 64, theta: float = 1e7, pos0: int = 0,
         pos: np.ndarray | None = None) -> np.ndarray:
    """x [T, nheads, head_dim] bf16 bits -> rotated copy (bf16 bits)."""
    x = _c(x, np.uint16)
    T, nh, hd = x.shape
    y = np.empty_like(x)
    pa = None if pos is None else _c(pos, np.int64)
    _load().qsa_oracle_rope(_p(x), _p(y), T, nh, hd, rope_dim, theta, pos0, _p(pa))
    return y


def compress(k: np.ndarray, r: int = 4, mode: int = KBAR_MEAN, gain: np.ndarray | None = None,
             rope_dim: int = 0, theta: float = 1e7, block0: int = 0) -> np.ndarray:
    """k [Tk, Di] bf16 bits -> kbar [Tk // r, Di] bf16 bits.  gain: bf16 [Di]
    RMSNorm gain (mode 1); rope_dim > 0 rotates the pooled keys at the block
    start positions r * (block0 + b)."""
    k = _c(k, np.uint16)
    Tk, Di = k.shape
    out = np.empty((Tk // r, Di), dtype=np.uint16)
    if gain is None and rope_dim == 0:
        _load().qsa_oracle_compress(_p(k), Tk, Di, r, mode, _p(out))
    else:
        g = None if gain is None else _c(gain, np.uint16)
        _load().qsa_oracle_compress_ext(_p(k), Tk, Di, r, mode, _p(g), rope_dim, theta, block0,
                                        _p(out))
    return out


def num_threads() -> int:
    """Threads of the oracle's OpenMP loops."""
    return int(_load().qsa_oracle_num_threads())


def num_complete(p: int, r: int = 4) -> int:
    return int(_load().qsa_oracle_num_complete(p, r))


def scores_row(qi_row: np.ndarray, kbar: np.ndarray, p: int, r: int = 4,
               mode: int = MODE_MAXHEAD) -> np.ndarray:
    """qi_row [Hi, Di], kbar [nb, Di] -> s [nc] (fp64)."""
    qi_row = _c(qi_row, np.uint16)
    kbar = _c(kbar, np.uint16)
    Hi, Di = qi_row.shape
    nc_full = max(num_complete(p, r), 1)
    s = np.empty(nc_full, dtype=np.float64)
    nc = _load().qsa_oracle_scores_row(_p(qi_row), _p(kbar), kbar.shape[0], p, Hi, Di, r, mode,
                                       _p(s))
    return s[:nc].copy()


def topk_row(s: np.ndarray, K: int):
    """-> (ascending selected blocks, rank-K score, rank-K+1 score)."""
    s = _c(s, np.float64)
    blk = np.full(max(K, 1), -1, dtype=np.int32)
    sK = np.zeros(1)
    sK1 = np.zeros(1)
    n = _load().qsa_oracle_topk_row(_p(s), s.size, K, _p(blk), _p(sK), _p(sK1))
    return blk[:n].copy(), float(sK[0]), float(sK1[0])


def token_set(blk: np.ndarray, p: int, r: int = 4) -> np.ndarray:
    blk = _c(blk, np.int32)
    tok = np.empty(blk.size * r + r, dtype=np.int64)
    n = _load().qsa_oracle_token_set(_p(blk), blk.size, p, r, _p(tok))
    return tok[:n].copy()


def token_set_reuse(blk: np.ndarray, p_sel: int, p: int, r: int = 4) -> np.ndarray:
    """Tokens of a query at position p >= p_sel that reuses the selection blk
    made for position p_sel (speculative steps with index reuse): the blocks
    expanded, then every token from r * nc(p_sel) through p."""
    blk = _c(blk, np.int32)
    tail = max(0, p - num_complete(p_sel, r) * r + 1)
    tok = np.empty(blk.size * r + tail + 1, dtype=np.int64)
    n = _load().qsa_oracle_token_set_reuse(_p(blk), blk.size, p_sel, p, r, _p(tok))
    return tok[:n].copy()


def attend_row(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, tokens: np.ndarray):
    """q_row [H, D], K/V [Tk, Hkv, D] bf16 bits -> (O [H, D], lse [H], wsum_err)."""
    q_row = _c(q_row, np.uint16)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    H, D = q_row.shape
    Hkv = K.shape[1]
    tokens = _c(tokens, np.int64)
    if tokens.size and (tokens.min() < 0 or tokens.max() >= min(K.shape[0], V.shape[0])):
        raise ValueError("attend_row: a token lies outside the key array")
    O = np.empty((H, D))
    lse = np.empty(H)
    err = np.zeros(1)
    _load().qsa_oracle_attend_row(_p(q_row), _p(K), _p(V), H, Hkv, D, _p(tokens), tokens.size,
                                  _p(O), _p(lse), _p(err))
    return O, lse, float(err[0])


def qsa_rows(Q, K, V, qi, kbar, rows, pos0: int = 0, Kbudget: int = 512, r: int = 4,
             mode: int = MODE_MAXHEAD):
    """End-to-end QSA of selected query rows (inputs post-RoPE / post-compress).

    Returns dict with O [n,H,D], lse [n,H], sel [n,K], nsel [n], sK, sK1,
    wsum_err.
    """
    Q, K, V, qi, kbar = (_c(a, np.uint16) for a in (Q, K, V, qi, kbar))
    rows = _c(rows, np.int64)
    n = rows.size
    _, H, D = Q.shape
    Hkv = K.shape[1]
    Hi, Di = qi.shape[1], qi.shape[2]
    _check_rows("qsa_rows", rows, min(Q.shape[0], qi.shape[0]), pos0 + rows, K.shape[0])
    O = np.empty((n, H, D))
    lse = np.empty((n, H))
    sel = np.empty((n, Kbudget), dtype=np.int32)
    nsel = np.empty(n, dtype=np.int32)
    sK = np.empty(n)
    sK1 = np.empty(n)
    err = np.empty(n)
    _load().qsa_oracle_qsa_rows(_p(Q), _p(K), _p(V), _p(qi), _p(kbar), kbar.shape[0], pos0, H,
                                Hkv, D, Hi, Di, r, Kbudget, mode, _p(rows), n, _p(O), _p(lse),
                                _p(sel), _p(nsel), _p(sK), _p(sK1), _p(err))
    return dict(O=O, lse=lse, sel=sel, nsel=nsel, sK=sK, sK1=sK1, wsum_err=err)


def qsa_rows_at(Q_rows, K, V, qi_rows, kbar, positions, Kbudget: int = 512, r: int = 4,
                mode: int = MODE_MAXHEAD):
    """End-to-end QSA of compact query rows: Q_rows [n,H,D] (post-RoPE) and
    qi_rows [n,Hi,Di] are the queries at absolute positions positions[i]."""
    Q_rows, K, V, qi_rows, kbar = (_c(a, np.uint16) for a in (Q_rows, K, V, qi_rows, kbar))
    positions = _c(positions, np.int64)
    n = positions.size
    _, H, D = Q_rows.shape
    Hkv = K.shape[1]
    Hi, Di = qi_rows.shape[1], qi_rows.shape[2]
    if Q_rows.shape[0] < n or qi_rows.shape[0] < n:
        raise ValueError("qsa_rows_at: fewer query rows than positions")
    _check_rows("qsa_rows_at", None, n, positions, K.shape[0])
    O = np.empty((n, H, D))
    lse = np.empty((n, H))
    sel = np.empty((n, Kbudget), dtype=np.int32)
    nsel = np.empty(n, dtype=np.int32)
    sK = np.empty(n)
    sK1 = np.empty(n)
    err = np.empty(n)
    _load().qsa_oracle_qsa_rows_at(_p(Q_rows), _p(K), _p(V), _p(qi_rows), _p(kbar), kbar.shape[0],
                                   _p(positions), H, Hkv, D, Hi, Di, r, Kbudget, mode, n, _p(O),
                                   _p(lse), _p(sel), _p(nsel), _p(sK), _p(sK1), _p(err))
    return dict(O=O, lse=lse, sel=sel, nsel=nsel, sK=sK, sK1=sK1, wsum_err=err)


def sparse_attn_rows(Q, K, V, rows, sel, nsel, pos0: int = 0, r: int = 4):
    """Attention of rows over a given selection sel [n, Kbudget] / nsel [n]."""
    Q, K, V = (_c(a, np.uint16) for a in (Q, K, V))
    rows = _c(rows, np.int64)
    sel = _c(sel, np.int32)
    nsel = _c(nsel, np.int32)
    n = rows.size
    _, H, D = Q.shape
    Hkv = K.shape[1]
    _check_rows("sparse_attn_rows", rows, Q.shape[0], pos0 + rows, K.shape[0], sel, nsel, r)
    O = np.empty((n, H, D))
    lse = np.empty((n, H))
    _load().qsa_oracle_sparse_attn_rows(_p(Q), _p(K), _p(V), pos0, H, Hkv, D, r, sel.shape[1],
                                        _p(rows), n, _p(sel), _p(nsel), _p(O), _p(lse))
    return O, lse


def sparse_attn_rows_at(Q_rows, K, V, positions, sel, nsel, r: int = 4):
    """Attention of compact query rows over a given selection: Q_rows [n,H,D]
    (post-RoPE) are the queries at absolute positions positions[i], with
    selection row sel[i] / nsel[i]."""
    Q_rows, K, V = (_c(a, np.uint16) for a in (Q_rows, K, V))
    positions = _c(positions, np.int64)
    sel = _c(sel, np.int32)
    nsel = _c(nsel, np.int32)
    n = positions.size
    _, H, D = Q_rows.shape
    if Q_rows.shape[0] < n:
        raise ValueError("sparse_attn_rows_at: fewer query rows than positions")
    _check_rows("sparse_attn_rows_at", None, n, positions, K.shape[0], sel, nsel, r)
    O = np.empty((n, H, D))
    lse = np.empty((n, H))
    _load().qsa_oracle_sparse_attn_rows_at(_p(Q_rows), _p(K), _p(V), _p(positions), H, K.shape[1],
                                           D, r, sel.shape[1], n, _p(sel), _p(nsel), _p(O),
                                           _p(lse))
    return O, lse


def select_rows(qi, kbar, rows, pos0: int = 0, Kbudget: int = 512, r: int = 4,
                mode: int = MODE_MAXHEAD, want_scores: bool = False):
    """Scores + top-K of rows.  Returns dict(sel, nsel, sK, sK1[, s])."""
    qi, kbar = (_c(a, np.uint16) for a in (qi, kbar))
    rows = _c(rows, np.int64)
    n = rows.size
    Hi, Di = qi.shape[1], qi.shape[2]
    nb = kbar.shape[0]
    if rows.size and (rows.min() < 0 or rows.max() >= qi.shape[0]):
        raise ValueError(f"select_rows: a row lies outside the {qi.shape[0]} indexer rows")
    s = np.empty((n, nb)) if want_scores else None
    sel = np.empty((n, Kbudget), dtype=np.int32)
    nsel = np.empty(n, dtype=np.int32)
    sK = np.empty(n)
    sK1 = np.empty(n)
    _load().qsa_oracle_select_rows(_p(qi), _p(kbar), nb, pos0, Hi, Di, r, Kbudget, mode,
                                   _p(rows), n, _p(s), nb, _p(sel), _p(nsel), _p(sK), _p(sK1))
    out = dict(sel=sel, nsel=nsel, sK=sK, sK1=sK1)
    if want_scores:
        out["s"] = s
    return out


def decode_reuse_rows(Q_rows, K, V, qi_first, kbar, seq_len: int, Kbudget: int = 512,
                      r: int = 4, mode: int = MODE_MAXHEAD):
    """Decode of the n = Q_rows.shape[0] newest queries of one sequence of
    seq_len tokens (query i at seq_len - n + i; Q_rows post-RoPE) that share
    the selection made for the first of them from its indexer query qi_first
    [Hi, Di] (speculative steps with index reuse).  A query at a position
    below 0 sees no token: O = 0, lse = -inf.
    Returns dict(O [n,H,D], lse [n,H], sel, nsel, s, sK, sK1, wsum_err [n])."""
    Q_rows = _c(Q_rows, np.uint16)
    n, H, D = Q_rows.shape
    p0 = seq_len - n
    sr = select_rows(qi_first[None], kbar, np.array([0]), pos0=p0, Kbudget=Kbudget, r=r,
                     mode=mode, want_scores=True)
    blk = sr["sel"][0, :sr["nsel"][0]]
    O = np.zeros((n, H, D))
    lse = np.full((n, H), -np.inf)
    err = np.zeros(n)
    for i in range(n):
        p = p0 + i
        if p < 0:
            continue
        O[i], lse[i], err[i] = attend_row(Q_rows[i], K, V, token_set_reuse(blk, p0, p, r))
    return dict(O=O, lse=lse, sel=sr["sel"][0], nsel=int(sr["nsel"][0]), s=sr["s"][0],
                sK=float(sr["sK"][0]), sK1=float(sr["sK1"][0]), wsum_err=err)


def dense_rows(Q, K, V, rows, pos0: int = 0):
    """Dense causal attention of rows: O [n,H,D], lse [n,H]."""
    Q, K, V = (_c(a, np.uint16) for a in (Q, K, V))
    rows = _c(rows, np.int64)
    n = rows.size
    _, H, D = Q.shape
    Hkv = K.shape[1]
    _check_rows("dense_rows", rows, Q.shape[0], pos0 + rows, K.shape[0])
    O = np.empty((n, H, D))
    lse = np.empty((n, H))
    _load().qsa_oracle_dense_rows(_p(Q), _p(K), _p(V), pos0, H, Hkv, D, _p(rows), n, _p(O),
                                  _p(lse))
    return O, lse


def distill_row(q_row, K, p: int, s: np.ndarray, r: int = 4):
    """Stage-1 distillation of one query at position p: q_row [H, D] and K
    post-RoPE, s the indexer scores of its nc(p) complete blocks.
    Returns (KL, teacher T [nc], ln S [nc])."""
    q_row = _c(q_row, np.uint16)
    K = _c(K, np.uint16)
    H, D = q_row.shape
    nc = num_complete(p, r)
    s = _c(s[:nc], np.float64)
    T = np.zeros(max(nc, 1))
    lS = np.zeros(max(nc, 1))
    kl = _load().qsa_oracle_distill_row(_p(q_row), _p(K), H, K.shape[1], D, p, r, _p(s), _p(T),
                                        _p(lS))
    return float(kl), T[:nc], lS[:nc]


def distill_rows(Q, K, qi, kbar, rows, pos0: int = 0, r: int = 4, mode: int = MODE_MAXHEAD):
    """KL of stage-1 distillation for query rows (Q, K post-RoPE; qi, kbar the
    indexer inputs) -> [n]."""
    Q, K, qi, kbar = (_c(a, np.uint16) for a in (Q, K, qi, kbar))
    rows = _c(rows, np.int64)
    _, H, D = Q.shape
    _check_rows("distill_rows", rows, min(Q.shape[0], qi.shape[0]), pos0 + rows, K.shape[0])
    kl = np.empty(rows.size)
    _load().qsa_oracle_distill_rows(_p(Q), _p(K), _p(qi), _p(kbar), kbar.shape[0], pos0, H,
                                    K.shape[1], D, qi.shape[1], qi.shape[2], r, mode, _p(rows),
                                    rows.size, _p(kl))
    return kl


def sparse_kl_row(q_row, K, p: int, blk, s_sel, r: int = 4):
    """Distillation KL of one query at position p under the sparse pattern:
    blk the selected blocks (ascending), s_sel their indexer scores.
    Returns (KL, teacher T [nsel], ln S [nsel])."""
    q_row = _c(q_row, np.uint16)
    K = _c(K, np.uint16)
    H, D = q_row.shape
    blk = _c(blk, np.int32)
    ns = blk.size
    s_sel = _c(np.asarray(s_sel, dtype=np.float64).reshape(-1)[:ns], np.float64)
    T = np.zeros(max(ns, 1))
    lS = np.zeros(max(ns, 1))
    kl = _load().qsa_oracle_sparse_kl_row(_p(q_row), _p(K), H, K.shape[1], D, p, r,
                                          _p(blk if ns else np.zeros(1, np.int32)), ns,
                                          _p(s_sel if ns else np.zeros(1)), _p(T), _p(lS))
    return float(kl), T[:ns], lS[:ns]


def sparse_kl_rows(Q, K, qi, kbar, rows, sel, nsel, pos0: int = 0, r: int = 4,
                   mode: int = MODE_MAXHEAD):
    """Distillation KL under the sparse pattern for query rows over a given
    selection sel [n, Kbudget] / nsel [n] -> [n]."""
    Q, K, qi, kbar = (_c(a, np.uint16) for a in (Q, K, qi, kbar))
    rows = _c(rows, np.int64)
    sel = _c(sel, np.int32)
    nsel = _c(nsel, np.int32)
    _, H, D = Q.shape
    _check_rows("sparse_kl_rows", rows, min(Q.shape[0], qi.shape[0]), pos0 + rows, K.shape[0],
                sel, nsel, r)
    if (pos0 + rows).size and ((pos0 + rows + 1) // r).max() > kbar.shape[0]:
        raise ValueError("sparse_kl_rows: fewer pooled keys than complete blocks")
    kl = np.empty(rows.size)
    _load().qsa_oracle_sparse_kl_rows(_p(Q), _p(K), _p(qi), _p(kbar), kbar.shape[0], pos0, H,
                                      K.shape[1], D, qi.shape[1], qi.shape[2], r, mode,
                                      sel.shape[1], _p(rows), rows.size, _p(sel), _p(nsel),
                                      _p(kl))
    return kl
