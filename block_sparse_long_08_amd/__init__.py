"""Python binding of libqsa, the MI355X (gfx950) QSA layer.

Argument marshalling only: every function here has the name of the C entry
point it calls (include/qsa.h), takes torch tensors as device memory, passes
their data pointers and the current HIP stream, and raises QSAError on a
non-zero status.  All arithmetic runs in the HIP kernels of libqsa.so; there
is no CPU or PyTorch fallback, and importing fails loudly when the library is
missing.

bf16 tensors may be torch.bfloat16 or 16-bit integer views of the same bits.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(hipcc --offload-arch=gfx950); the QSA path has no fallback")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _dbl, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                              ctypes.c_size_t)


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_lib_status_string = _sig("qsa_status_string", ctypes.c_char_p, _i32)
_sig("qsa_version", _i32)
_sig("qsa_check_device", _i32)
_sig("qsa_rope_bf16", _i32, _vp, _vp, _i64, _i32, _i32, _i32, _dbl, _i64, _vp, _i32, _vp)
_sig("qsa_compress_keys", _i32, _vp, _i32, _i64, _i64, _i32, _i32, _i32, _vp, _i32, _dbl, _i64,
     _vp, _i64, _vp, _vp)
_sig("qsa_index_scores", _i32, _vp, _vp, _i32, _i64, _i64, _vp, _i64, _i32, _i32, _i32, _i32,
     _vp, _i64, _vp, _vp)
_sig("qsa_topk_workspace_bytes", _sz, _i32, _i64, _i64, _i32)
_sig("qsa_topk_blocks", _i32, _vp, _i32, _i64, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _vp,
     _sz, _vp)
_sig("qsa_select_workspace_bytes", _sz, _i32, _i64, _i64, _i32)
_sig("qsa_select_blocks", _i32, _vp, _vp, _i32, _i64, _i64, _vp, _i64, _i32, _i32, _i32, _i32,
     _i32, _vp, _vp, _vp, _sz, _vp, _vp)
_sig("qsa_sparse_attn_prefill", _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
     _i32, _i32, _vp, _vp, _vp, _vp)
_sig("qsa_sparse_attn_prefill_rope", _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32,
     _i32, _i32, _i32, _i32, _dbl, _vp, _vp, _vp, _vp)
_sig("qsa_decode_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _i32, _i32)
_sig("qsa_sparse_attn_decode", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i32, _i32,
     _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp, _vp)
_sig("qsa_sparse_attn_decode_rope", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i32,
     _i32, _i32, _i32, _i32, _i32, _dbl, _vp, _vp, _vp, _sz, _vp, _vp)
_sig("qsa_decode_noalloc_max_bytes", _sz)
_sig("qsa_sparse_attn_decode_noalloc", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i32,
     _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp)
_sig("dense_attn_workspace_bytes", _sz, _i32, _i64, _i64, _i32, _i32, _i32)
_sig("dense_attn", _i32, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _i32, _i32, _vp, _vp,
     _vp, _sz, _vp, _vp)
_sig("qsa_distill_workspace_bytes", _sz, _i64, _i64)
_sig("qsa_distill_kl", _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
     _i32, _i32, _i32, _vp, _vp, _sz, _vp)
_sig("qsa_sparse_attn_prefill_kl", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
     _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp)
_sig("qsa_sparse_attn_prefill_concurrency", _i32, _i32, _i32, _i32, _i32)
_sig("qsa_sparse_attn_prefill_kl_staged_workspace_bytes", _sz, _i64, _i32)
_sig("qsa_sparse_attn_prefill_kl_staged", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
     _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _dbl, _vp, _vp, _vp, _vp, _sz,
     _vp)

EXPORTED = ["qsa_status_string", "qsa_version", "qsa_check_device", "qsa_rope_bf16",
            "qsa_compress_keys", "qsa_index_scores", "qsa_topk_workspace_bytes",
            "qsa_topk_blocks", "qsa_select_workspace_bytes", "qsa_select_blocks",
            "qsa_sparse_attn_prefill", "qsa_sparse_attn_prefill_rope",
            "qsa_decode_workspace_bytes", "qsa_sparse_attn_decode", "qsa_sparse_attn_decode_rope",
            "qsa_decode_noalloc_max_bytes", "qsa_sparse_attn_decode_noalloc",
            "dense_attn_workspace_bytes", "dense_attn", "qsa_distill_workspace_bytes",
            "qsa_distill_kl", "qsa_sparse_attn_prefill_kl", "qsa_sparse_attn_prefill_concurrency",
            "qsa_sparse_attn_prefill_kl_staged_workspace_bytes",
            "qsa_sparse_attn_prefill_kl_staged"]

SCORE_MAXHEAD, SCORE_RELUSUM = 0, 1
KBAR_MEAN, KBAR_RMSNORM = 0, 1
H, HKV, D, HI, DI, R = 24, 2, 256, 4, 128, 4


class QSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {qsa_status_string(status)}")
        self.status = status


def qsa_status_string(status: int) -> str:
    return _lib_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# Host-side checks before a call: each tensor argument must be a GPU tensor
# with the element size the call reads, holding at least the bytes the call's
# own size arguments imply from its first element to the end of its storage
# (strided views of a larger tensor are fine).  The C library cannot see
# extents, and an access past them would fault the GPU.  Raw addresses
# (ints) and None pass unchecked.
_REQUIRE_GPU = True


def _req(fn: str, arg: str, t, elsize: int, nbytes: int) -> None:
    if t is None or isinstance(t, int):
        return
    if _REQUIRE_GPU and not t.is_cuda:
        raise ValueError(f"{fn}: {arg} is not a GPU tensor")
    if t.element_size() != elsize:
        raise ValueError(f"{fn}: {arg} has {t.element_size()}-byte elements, the call reads "
                         f"{elsize}-byte ones")
    span = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    if nbytes > span:
        raise ValueError(f"{fn}: {arg} holds {span} bytes from its first element; the call "
                         f"needs {nbytes}")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _call(name, *args):
    st = getattr(_lib, name)(*args)
    if st != 0:
        raise QSAError(name, st)


class Pages(ctypes.Structure):
    """qsa_pages: a page table (device int32 tensor [B, table_stride]) and the
    page size in tokens; the cache arguments of a call are then page pools."""
    _fields_ = [("table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
                ("page_tokens", ctypes.c_int)]

    def __init__(self, table, page_tokens: int):
        _req("Pages", "table", table, 4, table.numel() * 4)
        if table.dim() != 2 or not table.is_contiguous():
            raise ValueError("Pages: table must be a contiguous [B, table_stride] int32 tensor")
        super().__init__(ctypes.c_void_p(table.data_ptr()), table.shape[-1], page_tokens)
        self._table = table  # keeps the tensor alive


def _pages(p):
    return None if p is None else ctypes.byref(p)


def qsa_version() -> int:
    return int(_lib.qsa_version())


def qsa_check_device() -> None:
    st = _lib.qsa_check_device()
    if st != 0:
        raise QSAError("qsa_check_device", st)


def qsa_rope_bf16(x, y, T: int, nheads: int, head_dim: int, rope_dim: int = 64,
                  theta: float = 1e7, pos0: int = 0, seq_len=None, next_n: int = 1,
                  stream=None) -> None:
    f = "qsa_rope_bf16"
    _req(f, "x", x, 2, T * nheads * head_dim * 2)
    _req(f, "y", y, 2, T * nheads * head_dim * 2)
    _req(f, "seq_len", seq_len, 8, (T // max(next_n, 1)) * 8)
    _call("qsa_rope_bf16", _ptr(x), _ptr(y), T, nheads, head_dim, rope_dim, theta, pos0,
          _ptr(seq_len), next_n, _stream(stream))


def qsa_compress_keys(k, B: int, Tk: int, k_seq_stride: int, Di: int, r: int, kbar_mode: int,
                      kbar, kbar_seq_stride: int, stream=None, gain=None, rope_dim: int = 0,
                      theta: float = 1e7, block0: int = 0, pages=None) -> None:
    f = "qsa_compress_keys"
    _req(f, "k", k, 2, ((B - 1) * k_seq_stride + Tk * Di) * 2)
    _req(f, "kbar", kbar, 2, 2 if pages is not None else ((B - 1) * kbar_seq_stride + (Tk // r) * Di) * 2)
    _req(f, "gain", gain, 2, Di * 2)
    _call("qsa_compress_keys", _ptr(k), B, Tk, k_seq_stride, Di, r, kbar_mode, _ptr(gain),
          rope_dim, theta, block0, _ptr(kbar), kbar_seq_stride, _pages(pages), _stream(stream))


def qsa_index_scores(q_idx, kbar, B: int, Tq: int, pos0: int, seq_len, nb_max: int, Hi: int,
                     Di: int, r: int, score_mode: int, scores, ld: int, stream=None,
                     pages=None) -> None:
    f = "qsa_index_scores"
    rows = B if seq_len is not None else B * Tq
    _req(f, "q_idx", q_idx, 2, B * Tq * Hi * Di * 2)
    _req(f, "kbar", kbar, 2, 2 if pages is not None else B * nb_max * Di * 2)
    _req(f, "seq_len", seq_len, 8, B * 8)
    _req(f, "scores", scores, 4, rows * ld * 4)
    _call("qsa_index_scores", _ptr(q_idx), _ptr(kbar), B, Tq, pos0, _ptr(seq_len), nb_max, Hi, Di,
          r, score_mode, _ptr(scores), ld, _pages(pages), _stream(stream))


def qsa_topk_workspace_bytes(B: int, Tq: int, nb_max: int, K: int) -> int:
    return int(_lib.qsa_topk_workspace_bytes(B, Tq, nb_max, K))


def qsa_topk_blocks(scores, B: int, Tq: int, ld: int, pos0: int, seq_len, nb_max: int, r: int,
                    K: int, blk_idx, n_sel, ws=None, ws_bytes: int = 0, stream=None) -> None:
    f = "qsa_topk_blocks"
    rows = B if seq_len is not None else B * Tq
    _req(f, "scores", scores, 4, rows * ld * 4)
    _req(f, "seq_len", seq_len, 8, B * 8)
    _req(f, "blk_idx", blk_idx, 4, rows * K * 4)
    _req(f, "n_sel", n_sel, 4, rows * 4)
    _req(f, "ws", ws, 1, ws_bytes)
    _call("qsa_topk_blocks", _ptr(scores), B, Tq, ld, pos0, _ptr(seq_len), nb_max, r, K,
          _ptr(blk_idx), _ptr(n_sel), _ptr(ws), ws_bytes, _stream(stream))


def qsa_select_workspace_bytes(B: int, Tq: int, nb_max: int, K: int) -> int:
    return int(_lib.qsa_select_workspace_bytes(B, Tq, nb_max, K))


def qsa_select_blocks(q_idx, kbar, B: int, Tq: int, pos0: int, seq_len, nb_max: int, Hi: int,
                      Di: int, r: int, score_mode: int, K: int, blk_idx, n_sel, ws,
                      ws_bytes: int, stream=None, pages=None) -> None:
    f = "qsa_select_blocks"
    rows = B if seq_len is not None else B * Tq
    _req(f, "q_idx", q_idx, 2, B * Tq * Hi * Di * 2)
    _req(f, "kbar", kbar, 2, 2 if pages is not None else B * nb_max * Di * 2)
    _req(f, "seq_len", seq_len, 8, B * 8)
    _req(f, "blk_idx", blk_idx, 4, rows * K * 4)
    _req(f, "n_sel", n_sel, 4, rows * 4)
    _req(f, "ws", ws, 1, ws_bytes)
    _call("qsa_select_blocks", _ptr(q_idx), _ptr(kbar), B, Tq, pos0, _ptr(seq_len), nb_max, Hi,
          Di, r, score_mode, K, _ptr(blk_idx), _ptr(n_sel), _ptr(ws), ws_bytes, _pages(pages),
          _stream(stream))


def qsa_sparse_attn_prefill(Q, K, V, blk_idx, n_sel, Tq: int, Tk: int, pos0: int, H: int,
                            Hkv: int, D: int, r: int, Kbudget: int, O, lse=None,
                            stream=None, pages=None) -> None:
    f = "qsa_sparse_attn_prefill"
    _req(f, "Q", Q, 2, Tq * H * D * 2)
    _req(f, "K", K, 2, 2 if pages is not None else Tk * Hkv * D * 2)
    _req(f, "V", V, 2, 2 if pages is not None else Tk * Hkv * D * 2)
    _req(f, "blk_idx", blk_idx, 4, Tq * Kbudget * 4)
    _req(f, "n_sel", n_sel, 4, Tq * 4)
    _req(f, "O", O, 4, Tq * H * D * 4)
    _req(f, "lse", lse, 4, Tq * H * 4)
    _call("qsa_sparse_attn_prefill", _ptr(Q), _ptr(K), _ptr(V), _ptr(blk_idx), _ptr(n_sel), Tq,
          Tk, pos0, H, Hkv, D, r, Kbudget, _ptr(O), _ptr(lse), _pages(pages), _stream(stream))


def qsa_sparse_attn_prefill_rope(Q, K, V, blk_idx, n_sel, Tq: int, Tk: int, pos0: int, H: int,
                                 Hkv: int, D: int, r: int, Kbudget: int, rope_dim: int,
                                 theta: float, O, lse=None, stream=None, pages=None) -> None:
    """qsa_sparse_attn_prefill with Q before RoPE: the kernel rotates it on load."""
    f = "qsa_sparse_attn_prefill_rope"
    _req(f, "Q", Q, 2, Tq * H * D * 2)
    _req(f, "K", K, 2, 2 if pages is not None else Tk * Hkv * D * 2)
    _req(f, "V", V, 2, 2 if pages is not None else Tk * Hkv * D * 2)
    _req(f, "blk_idx", blk_idx, 4, Tq * Kbudget * 4)
    _req(f, "n_sel", n_sel, 4, Tq * 4)
    _req(f, "O", O, 4, Tq * H * D * 4)
    _req(f, "lse", lse, 4, Tq * H * 4)
    _call(f, _ptr(Q), _ptr(K), _ptr(V), _ptr(blk_idx), _ptr(n_sel), Tq, Tk, pos0, H, Hkv, D, r,
          Kbudget, rope_dim, float(theta), _ptr(O), _ptr(lse), _pages(pages), _stream(stream))


def qsa_decode_workspace_bytes(B: int, Tq: int, H: int, Hkv: int, D: int, Kbudget: int) -> int:
    return int(_lib.qsa_decode_workspace_bytes(B, Tq, H, Hkv, D, Kbudget))


def qsa_sparse_attn_decode(q, Kc, Vc, seq_len, blk_idx, n_sel, B: int, Tq: int, Lmax: int,
                           H: int, Hkv: int, D: int, r: int, Kbudget: int, O, lse, ws,
                           ws_bytes: int, stream=None, pages=None) -> None:
    f = "qsa_sparse_attn_decode"
    _req(f, "q", q, 2, B * Tq * H * D * 2)
    _req(f, "Kc", Kc, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "Vc", Vc, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "seq_len", seq_len, 8, B * 8)
    _req(f, "blk_idx", blk_idx, 4, B * Kbudget * 4)
    _req(f, "n_sel", n_sel, 4, B * 4)
    _req(f, "O", O, 4, B * Tq * H * D * 4)
    _req(f, "lse", lse, 4, B * Tq * H * 4)
    _req(f, "ws", ws, 1, ws_bytes)
    _call("qsa_sparse_attn_decode", _ptr(q), _ptr(Kc), _ptr(Vc), _ptr(seq_len), _ptr(blk_idx),
          _ptr(n_sel), B, Tq, Lmax, H, Hkv, D, r, Kbudget, _ptr(O), _ptr(lse), _ptr(ws),
          ws_bytes, _pages(pages), _stream(stream))


def qsa_sparse_attn_decode_rope(q, Kc, Vc, seq_len, blk_idx, n_sel, B: int, Tq: int, Lmax: int,
                                H: int, Hkv: int, D: int, r: int, Kbudget: int, rope_dim: int,
                                theta: float, O, lse, ws, ws_bytes: int, stream=None,
                                pages=None) -> None:
    """qsa_sparse_attn_decode with q before RoPE: the kernel rotates it on load."""
    f = "qsa_sparse_attn_decode_rope"
    _req(f, "q", q, 2, B * Tq * H * D * 2)
    _req(f, "Kc", Kc, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "Vc", Vc, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "seq_len", seq_len, 8, B * 8)
    _req(f, "blk_idx", blk_idx, 4, B * Kbudget * 4)
    _req(f, "n_sel", n_sel, 4, B * 4)
    _req(f, "O", O, 4, B * Tq * H * D * 4)
    _req(f, "lse", lse, 4, B * Tq * H * 4)
    _req(f, "ws", ws, 1, ws_bytes)
    _call(f, _ptr(q), _ptr(Kc), _ptr(Vc), _ptr(seq_len), _ptr(blk_idx), _ptr(n_sel), B, Tq, Lmax,
          H, Hkv, D, r, Kbudget, rope_dim, float(theta), _ptr(O), _ptr(lse), _ptr(ws), ws_bytes,
          _pages(pages), _stream(stream))


def qsa_decode_noalloc_max_bytes() -> int:
    return int(_lib.qsa_decode_noalloc_max_bytes())


def qsa_sparse_attn_decode_noalloc(q, Kc, Vc, seq_len, blk_idx, n_sel, B: int, Tq: int,
                                   Lmax: int, H: int, Hkv: int, D: int, r: int, Kbudget: int, O,
                                   lse=None, stream=None, pages=None) -> None:
    f = "qsa_sparse_attn_decode_noalloc"
    _req(f, "q", q, 2, B * Tq * H * D * 2)
    _req(f, "Kc", Kc, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "Vc", Vc, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "seq_len", seq_len, 8, B * 8)
    _req(f, "blk_idx", blk_idx, 4, B * Kbudget * 4)
    _req(f, "n_sel", n_sel, 4, B * 4)
    _req(f, "O", O, 4, B * Tq * H * D * 4)
    _req(f, "lse", lse, 4, B * Tq * H * 4)
    _call("qsa_sparse_attn_decode_noalloc", _ptr(q), _ptr(Kc), _ptr(Vc), _ptr(seq_len),
          _ptr(blk_idx), _ptr(n_sel), B, Tq, Lmax, H, Hkv, D, r, Kbudget, _ptr(O), _ptr(lse),
          _pages(pages), _stream(stream))


def dense_attn_workspace_bytes(B: int, Tq: int, Lmax: int, H: int, Hkv: int, D: int) -> int:
    return int(_lib.dense_attn_workspace_bytes(B, Tq, Lmax, H, Hkv, D))


def dense_attn(Q, K, V, B: int, Tq: int, Lmax: int, pos0: int, seq_len, H: int, Hkv: int, D: int,
               O, lse=None, ws=None, ws_bytes: int = 0, stream=None, pages=None) -> None:
    f = "dense_attn"
    _req(f, "Q", Q, 2, B * Tq * H * D * 2)
    _req(f, "K", K, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "V", V, 2, 2 if pages is not None else B * Lmax * Hkv * D * 2)
    _req(f, "seq_len", seq_len, 8, B * 8)
    _req(f, "O", O, 4, B * Tq * H * D * 4)
    _req(f, "lse", lse, 4, B * Tq * H * 4)
    _req(f, "ws", ws, 1, ws_bytes)
    _call("dense_attn", _ptr(Q), _ptr(K), _ptr(V), B, Tq, Lmax, pos0, _ptr(seq_len), H, Hkv, D,
          _ptr(O), _ptr(lse), _ptr(ws), ws_bytes, _pages(pages), _stream(stream))


def qsa_distill_workspace_bytes(Tq: int, Tk: int) -> int:
    return int(_lib.qsa_distill_workspace_bytes(Tq, Tk))


def qsa_distill_kl(Q, K, lse, q_idx, kbar, Tq: int, Tk: int, pos0: int, H: int, Hkv: int, D: int,
                   Hi: int, Di: int, r: int, score_mode: int, kl, ws=None, ws_bytes: int = 0,
                   stream=None) -> None:
    f = "qsa_distill_kl"
    _req(f, "Q", Q, 2, Tq * H * D * 2)
    _req(f, "K", K, 2, Tk * Hkv * D * 2)
    _req(f, "lse", lse, 4, Tq * H * 4)
    _req(f, "q_idx", q_idx, 2, Tq * Hi * Di * 2)
    _req(f, "kbar", kbar, 2, (Tk // r) * Di * 2)
    _req(f, "kl", kl, 4, Tq * 4)
    _req(f, "ws", ws, 1, ws_bytes)
    _call("qsa_distill_kl", _ptr(Q), _ptr(K), _ptr(lse), _ptr(q_idx), _ptr(kbar), Tq, Tk, pos0,
          H, Hkv, D, Hi, Di, r, score_mode, _ptr(kl), _ptr(ws), ws_bytes, _stream(stream))


def qsa_sparse_attn_prefill_kl(Q, K, V, q_idx, kbar, blk_idx, n_sel, Tq: int, Tk: int,
                               pos0: int, H: int, Hkv: int, D: int, Hi: int, Di: int, r: int,
                               Kbudget: int, score_mode: int, O, lse, kl, stream=None) -> None:
    f = "qsa_sparse_attn_prefill_kl"
    _req(f, "Q", Q, 2, Tq * H * D * 2)
    _req(f, "K", K, 2, Tk * Hkv * D * 2)
    _req(f, "V", V, 2, Tk * Hkv * D * 2)
    _req(f, "q_idx", q_idx, 2, Tq * Hi * Di * 2)
    _req(f, "kbar", kbar, 2, (Tk // r) * Di * 2)
    _req(f, "blk_idx", blk_idx, 4, Tq * Kbudget * 4)
    _req(f, "n_sel", n_sel, 4, Tq * 4)
    _req(f, "O", O, 4, Tq * H * D * 4)
    _req(f, "lse", lse, 4, Tq * H * 4)
    _req(f, "kl", kl, 4, Tq * 4)
    _call("qsa_sparse_attn_prefill_kl", _ptr(Q), _ptr(K), _ptr(V), _ptr(q_idx), _ptr(kbar),
          _ptr(blk_idx), _ptr(n_sel), Tq, Tk, pos0, H, Hkv, D, Hi, Di, r, Kbudget, score_mode,
          _ptr(O), _ptr(lse), _ptr(kl), _stream(stream))


def qsa_sparse_attn_prefill_kl_staged_workspace_bytes(Tq: int, Kbudget: int) -> int:
    return int(_lib.qsa_sparse_attn_prefill_kl_staged_workspace_bytes(Tq, Kbudget))


def qsa_sparse_attn_prefill_kl_staged(Q, K, V, q_idx, kbar, blk_idx, n_sel, Tq: int, Tk: int,
                                      pos0: int, H: int, Hkv: int, D: int, Hi: int, Di: int,
                                      r: int, Kbudget: int, score_mode: int, O, lse, kl, ws=None,
                                      ws_bytes: int = 0, rope_dim: int = 0, theta: float = 1e7,
                                      stream=None) -> None:
    """The fused KL form in two launches (plain attention writing block
    maxima, then the KL); rope_dim > 0: Q before RoPE, rotated on load."""
    f = "qsa_sparse_attn_prefill_kl_staged"
    _req(f, "Q", Q, 2, Tq * H * D * 2)
    _req(f, "K", K, 2, Tk * Hkv * D * 2)
    _req(f, "V", V, 2, Tk * Hkv * D * 2)
    _req(f, "q_idx", q_idx, 2, Tq * Hi * Di * 2)
    _req(f, "kbar", kbar, 2, (Tk // r) * Di * 2)
    _req(f, "blk_idx", blk_idx, 4, Tq * Kbudget * 4)
    _req(f, "n_sel", n_sel, 4, Tq * 4)
    _req(f, "O", O, 4, Tq * H * D * 4)
    _req(f, "lse", lse, 4, Tq * H * 4)
    _req(f, "kl", kl, 4, Tq * 4)
    _req(f, "ws", ws, 1, ws_bytes)
    _call(f, _ptr(Q), _ptr(K), _ptr(V), _ptr(q_idx), _ptr(kbar), _ptr(blk_idx), _ptr(n_sel), Tq,
          Tk, pos0, H, Hkv, D, Hi, Di, r, Kbudget, score_mode, rope_dim, float(theta), _ptr(O),
          _ptr(lse), _ptr(kl), _ptr(ws), ws_bytes, _stream(stream))


def qsa_sparse_attn_prefill_concurrency(Hkv: int, Kbudget: int, with_kl: bool = False,
                                        paged: bool = False) -> int:
    """Queries whose sparse-prefill workgroups the current device holds at
    once (0: unsupported arguments, or the runtime cannot say)."""
    return int(_lib.qsa_sparse_attn_prefill_concurrency(Hkv, Kbudget, int(with_kl), int(paged)))


from .layer import QSAPrefill, QSADecode  # noqa: E402  (chains of the calls above)
