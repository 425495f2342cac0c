"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments on the host (before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")
LIB = os.path.join(ROOT, "block_sparse_long_08_amd", "libqsa.so")
# tests/test_sanitizers.py runs this file against a host-instrumented build
LIB_OVERRIDE = os.environ.get("QSA_ABI_LIB")


@pytest.fixture(scope="module")
def lib():
    if LIB_OVERRIDE:
        return ctypes.CDLL(LIB_OVERRIDE)
    if not os.path.exists(LIB):
        from block_sparse_long_08_amd import _build
        _build.build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text,
                       flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["qsa_compress_keys", "qsa_index_scores", "qsa_topk_blocks",
              "qsa_sparse_attn_prefill", "qsa_sparse_attn_decode", "dense_attn",
              "qsa_rope_bf16", "qsa_select_blocks"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"libqsa.so does not export {n}"


@pytest.mark.skipif(bool(LIB_OVERRIDE), reason="checks the Python binding, not the library")
def test_binding_names_match_header():
    import block_sparse_long_08_amd as qsa
    assert sorted(qsa.EXPORTED) == declared_functions()
    for n in qsa.EXPORTED:
        assert callable(getattr(qsa, n))


def test_status_strings(lib):
    lib.qsa_status_string.restype = ctypes.c_char_p
    for st in range(10):
        s = lib.qsa_status_string(st).decode()
        assert s.startswith("QSA_")
    assert lib.qsa_version() >= 100


# ---------------------------------------------------------------------------
# Host-side validation.  Host buffers stand in for device pointers: every call
# below fails a check before the library touches HIP.
# ---------------------------------------------------------------------------
BUF = np.zeros(1 << 16, dtype=np.uint8)
P = BUF.ctypes.data + (-BUF.ctypes.data) % 16  # 16-byte aligned
MIS = P + 2                                     # misaligned
I64 = ctypes.c_int64
OK, NULL, SHAPE, UNSUP, ALIGN, OVERFLOW, WORKSPACE = 0, 1, 2, 3, 4, 5, 6


def vp(x):
    return ctypes.c_void_p(x)


def rope(lib, x=P, y=P, T=4, nh=24, hd=256, rd=64, theta=1e7, pos0=0, lens=None, next_n=1):
    return lib.qsa_rope_bf16(vp(x), vp(y), I64(T), nh, hd, rd, ctypes.c_double(theta), I64(pos0),
                             lens, next_n, None)


def test_rope_validation(lib):
    assert rope(lib, x=0) == NULL
    assert rope(lib, T=-1) == SHAPE
    assert rope(lib, rd=65) == SHAPE
    assert rope(lib, rd=300) == SHAPE
    assert rope(lib, hd=96) == UNSUP
    assert rope(lib, theta=-1.0) == SHAPE
    assert rope(lib, x=MIS) == ALIGN
    assert rope(lib, next_n=0) == SHAPE
    assert rope(lib, next_n=17) == SHAPE
    assert rope(lib, T=6, lens=vp(P), next_n=4) == SHAPE   # rows not whole sequences


def compress(lib, k=P, B=1, Tk=16, ks=16 * 128, Di=128, r=4, mode=0, kb=P, kbs=4 * 128,
             gain=None, rope_dim=0, theta=1e7, block0=0, pages=None):
    return lib.qsa_compress_keys(vp(k), B, I64(Tk), I64(ks), Di, r, mode, gain, rope_dim,
                                 ctypes.c_double(theta), I64(block0), vp(kb), I64(kbs), pages,
                                 None)


def test_compress_validation(lib):
    assert compress(lib, kb=0) == NULL
    assert compress(lib, B=0) == SHAPE
    assert compress(lib, mode=2) == SHAPE
    assert compress(lib, Di=96) == UNSUP
    assert compress(lib, r=32) == UNSUP
    assert compress(lib, B=2, ks=8) == SHAPE
    assert compress(lib, k=MIS) == ALIGN
    assert compress(lib, rope_dim=48) == UNSUP        # partner chunk by xor: power of two
    assert compress(lib, rope_dim=8) == UNSUP
    assert compress(lib, rope_dim=256) == SHAPE       # more than Di
    assert compress(lib, rope_dim=64, theta=0.0) == SHAPE
    assert compress(lib, block0=-1) == SHAPE
    assert compress(lib, mode=1, gain=vp(MIS)) == ALIGN


def scores(lib, q=P, kb=P, B=1, Tq=8, pos0=0, sl=None, nb=4, Hi=4, Di=128, r=4, mode=0, out=P,
           ld=4, pages=None):
    return lib.qsa_index_scores(vp(q), vp(kb), B, I64(Tq), I64(pos0), sl, I64(nb), Hi, Di, r,
                                mode, vp(out), I64(ld), pages, None)


def test_index_scores_validation(lib):
    assert scores(lib, q=0) == NULL
    assert scores(lib, out=0) == NULL
    assert scores(lib, Tq=-1) == SHAPE
    assert scores(lib, mode=3) == SHAPE
    assert scores(lib, ld=2) == SHAPE
    assert scores(lib, Hi=8) == UNSUP
    assert scores(lib, r=8) == UNSUP
    assert scores(lib, sl=vp(P), Tq=17) == SHAPE          # decode form: at most 16 queries
    assert scores(lib, sl=vp(P), Tq=0) == SHAPE
    assert scores(lib, nb=1 << 33, ld=1 << 33) == OVERFLOW
    assert scores(lib, kb=MIS) == ALIGN


def topk(lib, s=P, B=1, Tq=8, ld=4, pos0=0, nb=4, r=4, K=2, blk=P, ns=P):
    return lib.qsa_topk_blocks(vp(s), B, I64(Tq), I64(ld), I64(pos0), None, I64(nb), r, K,
                               vp(blk), vp(ns), None, ctypes.c_size_t(0), None)


def test_topk_validation(lib):
    assert topk(lib, blk=0) == NULL
    assert topk(lib, K=0) == SHAPE
    assert topk(lib, ld=2) == SHAPE
    assert topk(lib, K=4096) == UNSUP
    assert topk(lib, s=MIS) == ALIGN
    assert topk(lib, nb=5, ld=6) == SHAPE               # rows must be 16-byte strided
    # rows longer than one segment need candidate lists in the workspace
    lib.qsa_topk_workspace_bytes.restype = ctypes.c_size_t
    assert lib.qsa_topk_workspace_bytes(1, I64(8192), I64(32768), 512) == 0
    assert lib.qsa_topk_workspace_bytes(32, I64(1), I64(65536), 512) > 0
    assert topk(lib, B=32, Tq=1, nb=65536, ld=65536) == WORKSPACE


def test_select_validation(lib):
    lib.qsa_select_workspace_bytes.restype = ctypes.c_size_t
    # prefill form: scores of one chunk of rows (at most 8 GiB) and their
    # 16-block group maxima (1/16 of that) in the workspace
    need = lib.qsa_select_workspace_bytes(1, I64(131072), I64(32768), 512)
    assert (1 << 32) <= need <= (1 << 33) * 17 // 16 + (1 << 20)
    assert lib.qsa_select_workspace_bytes(1, I64(1 << 20), I64(1 << 18), 512) <= \
        (1 << 33) * 17 // 16 + (1 << 20)
    st = lib.qsa_select_blocks(vp(P), vp(P), 1, I64(131072), I64(0), None, I64(32768), 4, 128, 4,
                               0, 512, vp(P), vp(P), vp(P), ctypes.c_size_t(need - 1), None,
                               None)
    assert st == WORKSPACE
    # decode form keeps one score row per sequence
    need = lib.qsa_select_workspace_bytes(32, I64(1), I64(65536), 512)
    assert need >= 32 * 65536 * 4
    st = lib.qsa_select_blocks(vp(P), vp(P), 32, I64(1), I64(0), vp(P), I64(65536), 4, 128, 4, 0,
                               512, vp(P), vp(P), vp(P), ctypes.c_size_t(16), None, None)
    assert st == WORKSPACE
    st = lib.qsa_select_blocks(vp(P), vp(P), 1, I64(1000), I64(0), None, I64(250), 4, 128, 4, 0,
                               64, vp(P), vp(0), None, ctypes.c_size_t(0), None, None)
    assert st == NULL
    st = lib.qsa_select_blocks(vp(P), vp(P), 1, I64(1000), I64(0), None, I64(250), 4, 128, 4, 0,
                               4096, vp(P), vp(P), None, ctypes.c_size_t(0), None, None)
    assert st == UNSUP


def sparse_prefill(lib, Q=P, Kt=P, V=P, blk=P, ns=P, Tq=8, Tk=8, pos0=0, H=24, Hkv=2, D=256, r=4,
                   Kb=4, O=P, pages=None):
    return lib.qsa_sparse_attn_prefill(vp(Q), vp(Kt), vp(V), vp(blk), vp(ns), I64(Tq), I64(Tk),
                                       I64(pos0), H, Hkv, D, r, Kb, vp(O), None, pages,
                                       None)


def test_sparse_prefill_validation(lib):
    assert sparse_prefill(lib, O=0) == NULL
    assert sparse_prefill(lib, Tk=7) == SHAPE           # keys must cover every query
    assert sparse_prefill(lib, Tq=8, Tk=12, pos0=5) == SHAPE
    assert sparse_prefill(lib, H=25) == SHAPE
    assert sparse_prefill(lib, D=128) == UNSUP
    assert sparse_prefill(lib, H=48, Hkv=2) == UNSUP    # 24 heads per KV head
    assert sparse_prefill(lib, Hkv=3, H=24) == UNSUP
    assert sparse_prefill(lib, r=2) == UNSUP
    assert sparse_prefill(lib, Kb=0) == SHAPE
    assert sparse_prefill(lib, Kb=4096) == UNSUP
    assert sparse_prefill(lib, V=MIS) == ALIGN


def sparse_prefill_rope(lib, Q=P, Kt=P, V=P, blk=P, ns=P, Tq=8, Tk=8, pos0=0, H=24, Hkv=2,
                        D=256, r=4, Kb=4, rope_dim=64, theta=1e7, O=P, pages=None):
    f = lib.qsa_sparse_attn_prefill_rope
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_int] * 6 + [
        ctypes.c_double] + [ctypes.c_void_p] * 4
    return f(vp(Q), vp(Kt), vp(V), vp(blk), vp(ns), Tq, Tk, pos0, H, Hkv, D, r, Kb, rope_dim,
             theta, vp(O), None, pages, None)


def test_sparse_prefill_rope_validation(lib):
    """The RoPE-on-load form: its own arguments, then every check of the
    plain form (each call fails on the host)."""
    assert sparse_prefill_rope(lib, rope_dim=0) == SHAPE
    assert sparse_prefill_rope(lib, theta=0.0) == SHAPE
    assert sparse_prefill_rope(lib, theta=float("nan")) == SHAPE
    assert sparse_prefill_rope(lib, rope_dim=32) == UNSUP   # pairs across lanes
    assert sparse_prefill_rope(lib, rope_dim=96) == UNSUP
    assert sparse_prefill_rope(lib, rope_dim=256) == UNSUP
    assert sparse_prefill_rope(lib, rope_dim=128, O=0) == NULL
    assert sparse_prefill_rope(lib, Q=0) == NULL
    assert sparse_prefill_rope(lib, Tk=7) == SHAPE
    assert sparse_prefill_rope(lib, H=25) == SHAPE
    assert sparse_prefill_rope(lib, D=128) == UNSUP
    assert sparse_prefill_rope(lib, Kb=4096) == UNSUP
    assert sparse_prefill_rope(lib, Q=MIS) == ALIGN
    assert sparse_prefill_rope(lib, pages=pages(page_tokens=48)) == UNSUP


def test_decode_validation(lib):
    lib.qsa_decode_workspace_bytes.restype = ctypes.c_size_t
    need = lib.qsa_decode_workspace_bytes(32, 1, 24, 2, 256, 512)
    assert need > 0
    # speculative queries: three column tiles of 16 (query, head) pairs per KV head
    assert lib.qsa_decode_workspace_bytes(4, 4, 24, 2, 256, 512) > 0
    assert lib.qsa_decode_workspace_bytes(4, 17, 24, 2, 256, 512) == 0
    args = [vp(P)] * 6
    st = lib.qsa_sparse_attn_decode(*args, 32, 1, I64(1024), 24, 2, 256, 4, 512, vp(P), None,
                                    vp(P), ctypes.c_size_t(need - 1), None, None)
    assert st == WORKSPACE
    st = lib.qsa_sparse_attn_decode(vp(P), vp(P), vp(P), None, vp(P), vp(P), 32, 1, I64(1024), 24,
                                    2, 256, 4, 512, vp(P), None, vp(P), ctypes.c_size_t(need), None,
                                    None)
    assert st == NULL
    for tq in (0, 17):
        st = lib.qsa_sparse_attn_decode(*args, 32, tq, I64(1024), 24, 2, 256, 4, 512, vp(P), None,
                                        vp(P), ctypes.c_size_t(1 << 30), None, None)
        assert st == SHAPE


def decode_rope(lib, q=P, seq=P, Tq=1, H=24, Hkv=2, Kb=512, rope_dim=64, theta=1e7, O=P,
                ws_bytes=1 << 30, pages=None):
    f = lib.qsa_sparse_attn_decode_rope
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 2 + [ctypes.c_int64] + [
        ctypes.c_int] * 6 + [ctypes.c_double] + [ctypes.c_void_p] * 3 + [ctypes.c_size_t] + [
        ctypes.c_void_p] * 2
    return f(vp(q), vp(P), vp(P), vp(seq), vp(P), vp(P), 32, Tq, 1024, H, Hkv, 256, 4, Kb,
             rope_dim, theta, vp(O), None, vp(P), ws_bytes, pages, None)


def test_decode_rope_validation(lib):
    """The decode form that rotates on load: its own arguments, then the
    plain decode's checks (each call fails on the host)."""
    assert decode_rope(lib, rope_dim=0) == SHAPE
    assert decode_rope(lib, theta=-1.0) == SHAPE
    assert decode_rope(lib, rope_dim=32) == UNSUP
    assert decode_rope(lib, rope_dim=256) == UNSUP
    assert decode_rope(lib, seq=0) == NULL
    assert decode_rope(lib, rope_dim=128, O=0) == NULL
    assert decode_rope(lib, Tq=17) == SHAPE
    assert decode_rope(lib, H=48) == UNSUP
    assert decode_rope(lib, Kb=4096) == UNSUP
    assert decode_rope(lib, q=MIS) == ALIGN
    assert decode_rope(lib, ws_bytes=16) == WORKSPACE
    assert decode_rope(lib, pages=pages(page_tokens=48)) == UNSUP


def test_dense_validation(lib):
    st = lib.dense_attn(vp(P), vp(P), vp(P), 1, I64(16), I64(15), I64(0), None, 24, 2, 256,
                        vp(P), None, None, ctypes.c_size_t(0), None, None)
    assert st == SHAPE                                   # pos0 + Tq > Lmax
    st = lib.dense_attn(vp(P), vp(P), vp(P), 1, I64(17), I64(16), I64(0), vp(P), 24, 2, 256,
                        vp(P), None, None, ctypes.c_size_t(0), None, None)
    assert st == SHAPE                                   # decode form: at most 16 queries
    st = lib.dense_attn(vp(P), vp(P), vp(P), 1, I64(4), I64(16), I64(0), vp(P), 24, 2, 256,
                        vp(P), None, None, ctypes.c_size_t(0), None, None)
    assert st == WORKSPACE                               # 4 speculative queries need records
    lib.dense_attn_workspace_bytes.restype = ctypes.c_size_t
    need = lib.dense_attn_workspace_bytes(4, I64(1), I64(1 << 20), 24, 2, 256)
    st = lib.dense_attn(vp(P), vp(P), vp(P), 4, I64(1), I64(1 << 20), I64(0), vp(P), 24, 2, 256,
                        vp(P), None, vp(P), ctypes.c_size_t(need - 16), None, None)
    assert st == WORKSPACE


class Pages(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
                ("page_tokens", ctypes.c_int)]


def pages(table=P, stride=64, page_tokens=64):
    return ctypes.byref(Pages(table, stride, page_tokens))


def test_pages_validation(lib):
    """Paged caches: a table, a power-of-two page of 16 .. 4096 tokens, and a
    table row that covers the call's longest cache."""
    assert sparse_prefill(lib, pages=pages(table=None)) == NULL
    assert sparse_prefill(lib, pages=pages(page_tokens=48)) == UNSUP
    assert sparse_prefill(lib, pages=pages(page_tokens=8)) == UNSUP
    assert sparse_prefill(lib, pages=pages(page_tokens=8192)) == UNSUP
    assert sparse_prefill(lib, Tk=8, Tq=8, pages=pages(stride=0)) == SHAPE
    assert compress(lib, Tk=4096, ks=4096 * 128, pages=pages(stride=63, page_tokens=64)) == SHAPE
    assert compress(lib, Tk=16, block0=100, pages=pages(stride=6, page_tokens=64)) == SHAPE
    assert scores(lib, nb=1024, ld=1024, pages=pages(stride=63, page_tokens=64)) == SHAPE
    args = [vp(P)] * 6
    st = lib.qsa_sparse_attn_decode(*args, 32, 1, I64(1 << 20), 24, 2, 256, 4, 512, vp(P), None,
                                    vp(P), ctypes.c_size_t(1 << 30), pages(stride=100), None)
    assert st == SHAPE
    st = lib.dense_attn(vp(P), vp(P), vp(P), 1, I64(8), I64(4096), I64(0), None, 24, 2, 256,
                        vp(P), None, None, ctypes.c_size_t(0), pages(stride=1, page_tokens=64),
                        None)
    assert st == SHAPE


def distill(lib, Q=P, K=P, lse=P, qi=P, kb=P, Tq=8, Tk=64, pos0=0, H=24, Hkv=2, D=256, Hi=4,
            Di=128, r=4, mode=0, kl=P, ws=P, wsb=1 << 30):
    return lib.qsa_distill_kl(vp(Q), vp(K), vp(lse), vp(qi), vp(kb), I64(Tq), I64(Tk), I64(pos0),
                              H, Hkv, D, Hi, Di, r, mode, vp(kl), vp(ws), ctypes.c_size_t(wsb),
                              None)


def test_prefill_concurrency_validation(lib):
    """Unsupported arguments return 0 before any runtime call."""
    f = lib.qsa_sparse_attn_prefill_concurrency
    assert f(3, 512, 0, 0) == 0          # Hkv not 1, 2 or 4
    assert f(2, 0, 0, 0) == 0            # empty budget
    assert f(2, 2049, 0, 0) == 0         # budget above 2,048
    assert f(2, 512, 1, 1) == 0          # the fused KL runs on contiguous caches
    assert f(1, 512, 1, 0) == 0          # ... over 2 KV heads
    assert f(2, 1025, 1, 0) == 0         # ... at budgets up to 1,024


def test_distill_validation(lib):
    lib.qsa_distill_workspace_bytes.restype = ctypes.c_size_t
    need = lib.qsa_distill_workspace_bytes(I64(8), I64(64))
    assert need >= 8 * 16 * 4                          # the chunk's indexer scores
    assert lib.qsa_distill_workspace_bytes(I64(0), I64(64)) == 0
    assert lib.qsa_distill_workspace_bytes(I64(8), I64(3)) == 0   # no complete block
    # one chunk of rows stays within 8 GiB however long the context
    assert lib.qsa_distill_workspace_bytes(I64(1 << 20), I64(1 << 20)) <= (1 << 33)
    assert distill(lib, lse=0) == NULL
    assert distill(lib, kb=0) == NULL
    assert distill(lib, kl=0) == NULL
    assert distill(lib, Tq=8, Tk=7) == SHAPE            # keys must cover every query
    assert distill(lib, pos0=60) == SHAPE
    assert distill(lib, H=16, Hkv=2) == UNSUP           # 24 query heads over 2 KV heads only
    assert distill(lib, H=12, Hkv=1) == UNSUP
    assert distill(lib, D=128) == UNSUP
    assert distill(lib, Hi=8) == UNSUP
    assert distill(lib, mode=3) == SHAPE
    assert distill(lib, Q=MIS) == ALIGN
    assert distill(lib, kb=MIS) == ALIGN
    assert distill(lib, ws=0) == WORKSPACE
    assert distill(lib, wsb=need - 1) == WORKSPACE
    assert distill(lib, ws=MIS) == ALIGN
    assert distill(lib, Tq=0, ws=0, wsb=0) == OK        # nothing to do, nothing enqueued


def attn_kl(lib, Q=P, K=P, V=P, qi=P, kb=P, blk=P, ns=P, Tq=8, Tk=64, pos0=0, H=24, Hkv=2, D=256,
            Hi=4, Di=128, r=4, Kb=512, mode=0, O=P, lse=P, kl=P):
    return lib.qsa_sparse_attn_prefill_kl(vp(Q), vp(K), vp(V), vp(qi), vp(kb), vp(blk), vp(ns),
                                          I64(Tq), I64(Tk), I64(pos0), H, Hkv, D, Hi, Di, r, Kb,
                                          mode, vp(O), vp(lse), vp(kl), None)


def test_sparse_attn_prefill_kl_validation(lib):
    assert attn_kl(lib, V=0) == NULL
    assert attn_kl(lib, qi=0) == NULL
    assert attn_kl(lib, kb=0) == NULL
    assert attn_kl(lib, kl=0) == NULL
    assert attn_kl(lib, blk=0) == NULL
    assert attn_kl(lib, Tq=8, Tk=7) == SHAPE             # keys must cover every query
    assert attn_kl(lib, Kb=0) == SHAPE
    assert attn_kl(lib, Kb=1025) == UNSUP                 # block maxima of 24 heads in LDS
    assert attn_kl(lib, H=16) == UNSUP
    assert attn_kl(lib, H=12, Hkv=1) == UNSUP
    assert attn_kl(lib, D=128) == UNSUP
    assert attn_kl(lib, Hi=8) == UNSUP
    assert attn_kl(lib, mode=2) == SHAPE
    assert attn_kl(lib, Q=MIS) == ALIGN
    assert attn_kl(lib, qi=MIS) == ALIGN
    assert attn_kl(lib, O=MIS) == ALIGN
    assert attn_kl(lib, Tq=0) == OK                      # nothing to do, nothing enqueued
    assert attn_kl(lib, Tq=0, lse=0) == OK               # lse is optional


def attn_kl_staged(lib, Q=P, K=P, V=P, qi=P, kb=P, blk=P, ns=P, Tq=8, Tk=64, pos0=0, H=24,
                   Hkv=2, D=256, Hi=4, Di=128, r=4, Kb=512, mode=0, rope_dim=0, theta=1e7, O=P,
                   lse=P, kl=P, ws=P, wsb=None):
    f = lib.qsa_sparse_attn_prefill_kl_staged
    f.argtypes = ([ctypes.c_void_p] * 7 + [ctypes.c_int64] * 3 + [ctypes.c_int] * 9 +
                  [ctypes.c_double] + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p])
    if wsb is None:
        wsb = Tq * (2 * Kb * 12 + 24) * 4
    return f(vp(Q), vp(K), vp(V), vp(qi), vp(kb), vp(blk), vp(ns), Tq, Tk, pos0, H, Hkv, D, Hi,
             Di, r, Kb, mode, rope_dim, theta, vp(O), vp(lse), vp(kl), vp(ws), wsb, None)


def test_sparse_attn_prefill_kl_staged_validation(lib):
    """The two-launch KL form: its workspace, RoPE and budget arguments,
    then the checks it shares with the one-kernel form (each call fails on
    the host, or has nothing to do)."""
    wsb = lib.qsa_sparse_attn_prefill_kl_staged_workspace_bytes
    wsb.restype, wsb.argtypes = ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int]
    assert wsb(8, 512) == 8 * (2 * 512 * 12 + 24) * 4    # block maxima, then lse2
    assert wsb(1536, 2048) == 1536 * (2 * 2048 * 12 + 24) * 4
    assert wsb(8, 0) == 0 and wsb(8, 2049) == 0 and wsb(-1, 512) == 0
    assert wsb(0, 512) == 0
    assert attn_kl_staged(lib, ws=0) == WORKSPACE
    assert attn_kl_staged(lib, wsb=8 * (2 * 512 * 12 + 24) * 4 - 1) == WORKSPACE
    assert attn_kl_staged(lib, ws=MIS) == ALIGN
    assert attn_kl_staged(lib, rope_dim=32) == UNSUP
    assert attn_kl_staged(lib, rope_dim=96) == UNSUP
    assert attn_kl_staged(lib, rope_dim=-64) == SHAPE
    assert attn_kl_staged(lib, rope_dim=64, theta=0.0) == SHAPE
    assert attn_kl_staged(lib, Kb=2049) == UNSUP           # above every form's budget
    assert attn_kl_staged(lib, Kb=0) == SHAPE
    assert attn_kl_staged(lib, kl=0) == NULL
    assert attn_kl_staged(lib, qi=0) == NULL
    assert attn_kl_staged(lib, Tq=8, Tk=7) == SHAPE
    assert attn_kl_staged(lib, H=16) == UNSUP
    assert attn_kl_staged(lib, D=128) == UNSUP
    assert attn_kl_staged(lib, mode=2) == SHAPE
    assert attn_kl_staged(lib, Q=MIS) == ALIGN
    assert attn_kl_staged(lib, Tq=0, ws=0, wsb=0) == OK    # nothing to do, nothing enqueued


def noalloc(lib, q=P, Kc=P, Vc=P, sl=P, blk=P, ns=P, B=2, Tq=1, Lmax=64, H=24, Hkv=2, D=256,
            r=4, K=8, O=P, lse=P, pages=None):
    return lib.qsa_sparse_attn_decode_noalloc(vp(q), vp(Kc), vp(Vc), vp(sl), vp(blk), vp(ns), B,
                                              Tq, I64(Lmax), H, Hkv, D, r, K, vp(O), vp(lse),
                                              pages, None)


def test_decode_noalloc_validation(lib):
    """The no-allocation decode checks its arguments like the workspace form,
    and rejects a call whose split records exceed its static scratch
    (QSA_ERR_SCRATCH) before any HIP call."""
    lib.qsa_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.qsa_decode_workspace_bytes.restype = ctypes.c_size_t
    assert lib.qsa_decode_noalloc_max_bytes() == 64 << 20
    assert noalloc(lib, q=0) == NULL
    assert noalloc(lib, O=0) == NULL
    assert noalloc(lib, sl=0) == NULL
    assert noalloc(lib, B=0) == SHAPE
    assert noalloc(lib, Tq=0) == SHAPE and noalloc(lib, Tq=17) == SHAPE
    assert noalloc(lib, K=0) == SHAPE and noalloc(lib, K=4096) == UNSUP
    assert noalloc(lib, H=25) == SHAPE and noalloc(lib, D=128) == UNSUP
    assert noalloc(lib, q=MIS) == ALIGN
    SCRATCH = 9
    # 4,000 sequences: one split each, 8,000 records of 16.9 KB > 64 MiB
    big = lib.qsa_decode_workspace_bytes(4000, 1, 24, 2, 256, 512)
    assert big > lib.qsa_decode_noalloc_max_bytes()
    assert noalloc(lib, B=4000, K=512) == SCRATCH
    assert noalloc(lib, B=70000, K=512) == OVERFLOW
