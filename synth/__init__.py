"""Seeded synthetic inputs for the QSA layer (host side, numpy).

Both the fp64 oracle and the GPU path are fed from this module.  It holds
none of the layer's arithmetic: only the counter-based N(0,1) generator
(SplitMix64 words -> Box-Muller -> bf16, defined in ``synth.c``), the needle
block sets, and the recipes that lay the five workloads out as tensors.

bf16 values are carried as ``numpy.uint16`` bit patterns throughout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_synth.so")
# A test that runs the generator under the sanitizers points this variable at
# an instrumented build (tests/test_sanitizers.py).
_LIB_OVERRIDE = os.environ.get("QSA_SYNTH_LIB")

STREAM_Q, STREAM_K, STREAM_V, STREAM_QIDX, STREAM_KIDX, STREAM_NEEDLE = 1, 2, 3, 4, 5, 6

_lib = None


def build(force: bool = True) -> str:
    """Compile ``libqsa_synth.so`` with gcc (OpenMP)."""
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
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        lib.synth_fill_normal_bf16.argtypes = [u64, u64, u64, i64, vp]
        lib.synth_fill_normal_bf16.restype = None
        lib.synth_fill_normal_bf16_rows.argtypes = [u64, u64, u64, i64, i64, i64, i64, vp]
        lib.synth_fill_normal_bf16_rows.restype = None
        lib.synth_needle_blocks.argtypes = [u64, i64, i32, i32, vp]
        lib.synth_needle_blocks.restype = i32
        lib.synth_scale_rows_x4.argtypes = [vp, vp, i64, i64, i64]
        lib.synth_scale_rows_x4.restype = None
        lib.synth_normal_f64.argtypes = [u64, u64, u64]
        lib.synth_normal_f64.restype = ctypes.c_double
        lib.synth_uniform.argtypes = [u64, u64, u64]
        lib.synth_uniform.restype = ctypes.c_double
        lib.synth_word.argtypes = [u64, u64, u64]
        lib.synth_word.restype = u64
        _lib = lib
    return _lib


def normal_bf16(stream: int, shape, seed: int = 0, first: int = 0, out=None) -> np.ndarray:
    """N(0,1) bf16 bits for elements first..first+prod(shape) of a stream."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    if n:
        _load().synth_fill_normal_bf16(seed, stream, first, n, out.ctypes.data)
    return out


def normal_bf16_rows(stream: int, first: int, nrows: int, row_len: int, src_stride: int,
                     seed: int = 0) -> np.ndarray:
    """Rows j of ``row_len`` stream elements starting at first + j*src_stride."""
    out = np.empty((nrows, row_len), dtype=np.uint16)
    if nrows and row_len:
        _load().synth_fill_normal_bf16_rows(seed, stream, first, nrows, row_len, src_stride,
                                            row_len, out.ctypes.data)
    return out


def normal_f64(stream: int, e: int, seed: int = 0) -> float:
    return _load().synth_normal_f64(seed, stream, e)


def uniform(stream: int, counter: int, seed: int = 0) -> float:
    return _load().synth_uniform(seed, stream, counter)


def word(stream: int, counter: int, seed: int = 0) -> int:
    return _load().synth_word(seed, stream, counter)


def needle_blocks(n_blocks: int, n_sets: int, per_set: int, seed: int = 0) -> np.ndarray:
    """[n_sets, per_set] distinct ascending block ids per set (stream 6)."""
    out = np.empty((n_sets, per_set), dtype=np.int64)
    rc = _load().synth_needle_blocks(seed, n_blocks, n_sets, per_set, out.ctypes.data)
    if rc != 0:
        raise ValueError("needle set larger than the block count")
    return out


def scale_rows_x4(data: np.ndarray, rows: np.ndarray, row_len: int, row_stride: int) -> None:
    """data.flat[r*row_stride : r*row_stride+row_len] *= 4 (exact) for r in rows."""
    assert data.dtype == np.uint16 and data.flags.c_contiguous
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size:
        assert int(rows.max()) * row_stride + row_len <= data.size
        _load().synth_scale_rows_x4(data.ctypes.data, rows.ctypes.data, rows.size, row_len,
                                    row_stride)


# --------------------------------------------------------------------------
# Workload recipes.  Head shapes are those of the QSA layer on the pages'
# model summary: 24 query heads / 2 KV heads of dim 256 for attention, 4 query
# heads / 1 key head of dim 128 for the indexer, micro-blocks of 4 tokens.
# --------------------------------------------------------------------------
H, HKV, D, HI, DI, R = 24, 2, 256, 4, 128, 4


@dataclass
class PrefillInputs:
    """Pre-RoPE prefill tensors of one sequence (bf16 bits).

    Q [Tq,H,D] for queries at positions pos0..pos0+Tq-1; K,V [Tk,HKV,D] for
    positions 0..Tk-1 (Tk = pos0+Tq); qi [Tq,HI,DI]; ki [Tk,DI].
    ``k_is_rotated`` tells whether K already carries RoPE (a cache) or not.
    """
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    qi: np.ndarray
    ki: np.ndarray
    pos0: int
    needles: np.ndarray | None
    k_is_rotated: bool


def apply_needles(K: np.ndarray, ki: np.ndarray, needles: np.ndarray) -> None:
    """Scale the planted needle blocks by 4 in place.

    needles[g] lists the blocks planted for KV head g: K[4b..4b+3, g, :] are
    scaled; the indexer keys ki[4b..4b+3, :] are scaled for every needle block
    of any head, so that the indexer can see them.
    """
    Tk = K.shape[0]
    for g in range(needles.shape[0]):
        toks = (needles[g][:, None] * R + np.arange(R)[None, :]).reshape(-1)
        toks = toks[toks < Tk]
        rows = toks * HKV + g  # K viewed as rows of D elements
        scale_rows_x4(K, rows, D, D)
    allb = np.unique(needles.reshape(-1))
    toks = (allb[:, None] * R + np.arange(R)[None, :]).reshape(-1)
    toks = toks[toks < ki.shape[0]]
    scale_rows_x4(ki, toks, DI, DI)


def prefill_inputs(Tq: int, pos0: int = 0, seed: int = 0, needles_per_head: int = 0,
                   k_is_rotated: bool | None = None) -> PrefillInputs:
    """Seeded inputs for a prefill of Tq queries ending a context of pos0+Tq tokens."""
    Tk = pos0 + Tq
    Q = normal_bf16(STREAM_Q, (Tq, H, D), seed)
    K = normal_bf16(STREAM_K, (Tk, HKV, D), seed)
    V = normal_bf16(STREAM_V, (Tk, HKV, D), seed)
    qi = normal_bf16(STREAM_QIDX, (Tq, HI, DI), seed)
    ki = normal_bf16(STREAM_KIDX, (Tk, DI), seed)
    nd = None
    if needles_per_head:
        nd = needle_blocks(Tk // R, HKV, needles_per_head, seed)
        apply_needles(K, ki, nd)
    if k_is_rotated is None:
        k_is_rotated = pos0 > 0
    return PrefillInputs(Q, K, V, qi, ki, pos0, nd, k_is_rotated)


@dataclass
class DecodeSeq:
    """One decode sequence: new query at position L-1 over a cache of L tokens.

    q [H,D] pre-RoPE; qi [HI,DI]; K,V [L,HKV,D] post-RoPE cache; ki [L,DI].
    """
    q: np.ndarray
    qi: np.ndarray
    K: np.ndarray
    V: np.ndarray
    ki: np.ndarray
    L: int


def decode_seq(b: int, L: int, Lmax: int, seed: int = 0, needles_per_head: int = 0) -> DecodeSeq:
    """Sequence b of a decode batch whose caches are [B, Lmax, ...] tensors.

    Element numbering follows the batched tensor (sequence b starts at
    b*Lmax*row), so one sequence can be regenerated alone.
    """
    q = normal_bf16(STREAM_Q, (H, D), seed, first=b * H * D)
    qi = normal_bf16(STREAM_QIDX, (HI, DI), seed, first=b * HI * DI)
    K = normal_bf16(STREAM_K, (L, HKV, D), seed, first=b * Lmax * HKV * D)
    V = normal_bf16(STREAM_V, (L, HKV, D), seed, first=b * Lmax * HKV * D)
    ki = normal_bf16(STREAM_KIDX, (L, DI), seed, first=b * Lmax * DI)
    if needles_per_head:
        nd = needle_blocks(L // R, HKV, needles_per_head, seed + 1000003 * (b + 1))
        apply_needles(K, ki, nd)
    return DecodeSeq(q, qi, K, V, ki, L)


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (x.astype(np.uint32) << 16).view(np.float32)
