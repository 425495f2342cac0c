"""Decode with speculative queries that reuse one block selection (the
next_n newest queries of a sequence share the selection made for the first
of them; each adds its own causal tail).  The HIP path runs through the C
ABI; the fp64 oracle checks every query.  Inputs: seeded N(0,1) bf16 rows;
windows at ragged lengths, across block boundaries, before position 0,
within the budget (dense equivalence) and far beyond it."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, check_selection, dev, host_u16, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import torch
    import block_sparse_long_08_amd as q
    assert torch.cuda.is_available()
    q.qsa_check_device()
    return q


def _torch():
    import torch
    return torch


def test_rope_decode_form_with_speculative_queries(qsa):
    torch = _torch()
    B, n = 4, 4
    lens = np.array([2, 5, 4099, 1048576], dtype=np.int64)
    x = synth.normal_bf16(1, (B * n, 24, 256), seed=31)
    y = torch.empty((B * n, 24, 256), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_rope_bf16(dev(x), y, B * n, 24, 256, 64, 1e7, 0, dev(lens), n)
    torch.cuda.synchronize()
    pos = np.maximum(np.repeat(lens - n, n) + np.tile(np.arange(n), B), 0)
    ref = oracle.rope(x, pos=pos)
    assert np.abs(host_u16(y).astype(np.int32) - ref.astype(np.int32)).max() <= 1


@pytest.mark.parametrize("n", [2, 4, 7])
def test_decode_attention_with_reused_selection(qsa, n):
    """Attention of the n newest queries over a given selection (made for the
    first of them), checked per query against the oracle's token sets."""
    torch = _torch()
    B, Lmax, K = 7, 3000, 64
    lens = np.array([1, 3, 6, 257, 1023, 1024, 2999], dtype=np.int64)
    Kc = synth.normal_bf16(2, (B, Lmax, 2, 256), seed=32)
    Vc = synth.normal_bf16(3, (B, Lmax, 2, 256), seed=32)
    q = synth.normal_bf16(1, (B, n, 24, 256), seed=32 + n)
    rng = np.random.default_rng(n)
    sel = np.full((B, K), -1, dtype=np.int32)
    nsel = np.zeros(B, dtype=np.int32)
    for b in range(B):
        nc = oracle.num_complete(int(lens[b]) - n)
        m = min(K, nc)
        sel[b, :m] = np.sort(rng.choice(nc, size=m, replace=False)) if m else []
        nsel[b] = m
    wsb = qsa.qsa_decode_workspace_bytes(B, n, 24, 2, 256, K)
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    O = torch.empty((B, n, 24, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, n, 24), dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_decode(dev(q), dev(Kc), dev(Vc), dev(lens), dev(sel), dev(nsel), B, n,
                               Lmax, 24, 2, 256, 4, K, O, lse, ws, wsb)
    torch.cuda.synchronize()
    Og, lg = O.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        L = int(lens[b])
        p0 = L - n
        for i in range(n):
            p = p0 + i
            if p < 0:
                assert np.all(Og[b, i] == 0) and np.all(np.isneginf(lg[b, i])), (b, i)
                continue
            tok = oracle.token_set_reuse(sel[b, :nsel[b]], p0, p)
            Oref, lref, _ = oracle.attend_row(q[b, i], Kc[b, :L], Vc[b, :L], tok)
            assert_close(Og[b, i], Oref, f"seq {b} (L={L}) query {i} O")
            assert_close(lg[b, i], lref, f"seq {b} query {i} lse")


def test_dense_decode_form_with_speculative_queries(qsa):
    torch = _torch()
    B, n, Lmax = 3, 4, 700
    lens = np.array([3, 301, 700], dtype=np.int64)
    Kc = synth.normal_bf16(2, (B, Lmax, 2, 256), seed=33)
    Vc = synth.normal_bf16(3, (B, Lmax, 2, 256), seed=33)
    q = synth.normal_bf16(1, (B, n, 24, 256), seed=33)
    wsb = qsa.dense_attn_workspace_bytes(B, n, Lmax, 24, 2, 256)
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    O = torch.empty((B, n, 24, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, n, 24), dtype=torch.float32, device="cuda")
    qsa.dense_attn(dev(q), dev(Kc), dev(Vc), B, n, Lmax, 0, dev(lens), 24, 2, 256, O, lse, ws,
                   wsb)
    torch.cuda.synchronize()
    Og, lg = O.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        L = int(lens[b])
        for i in range(n):
            p = L - n + i
            if p < 0:
                assert np.all(Og[b, i] == 0)
                continue
            Oref, lref, _ = oracle.attend_row(q[b, i], Kc[b, :L], Vc[b, :L], np.arange(p + 1))
            assert_close(Og[b, i], Oref, f"dense seq {b} query {i} O")
            assert_close(lg[b, i], lref, f"dense seq {b} query {i} lse")


def _decode_case(B, L, n, seed, needles=0):
    """Caches of B sequences of L tokens (post-RoPE K), pooled keys, and the
    n newest queries of each (raw q, indexer queries)."""
    seqs = [synth.decode_seq(b, L, L, needles_per_head=needles, seed=seed) for b in range(B)]
    Kc = np.stack([s.K for s in seqs])
    Vc = np.stack([s.V for s in seqs])
    kb = np.stack([oracle.compress(s.ki) for s in seqs])
    q = synth.normal_bf16(1, (B, n, 24, 256), seed=seed + 100)
    qi = synth.normal_bf16(4, (B, n, 4, 128), seed=seed + 100)
    return Kc, Vc, kb, q, qi


@pytest.mark.parametrize("L,K,mode", [(3001, 64, 0), (3003, 64, 1), (150, 64, 0),
                                      (20000, 512, 0)])
def test_decode_layer_reuse_end_to_end(qsa, L, K, mode):
    """QSADecode with next_n = 4: the selection equals the oracle's for the
    first query (tie band), and every query's output the oracle's attention
    over that selection and its own tail (and end to end where the sets
    agree).  L = 150 keeps every block in the budget: dense attention."""
    torch = _torch()
    B, n = 3, 4
    Kc, Vc, kb, q, qi = _decode_case(B, L, n, seed=L)
    lens = np.full(B, L, dtype=np.int64)
    dec = qsa.QSADecode(B, L, budget=K, score_mode=mode, next_n=n)
    O, lse = dec(dev(q), dev(qi), dev(Kc), dev(Vc), dev(kb), dev(lens))
    torch.cuda.synchronize()
    Og, lg = O.cpu().numpy(), lse.cpu().numpy()
    blk, ns = dec.blk_idx.cpu().numpy(), dec.n_sel.cpu().numpy()
    p0 = L - n
    for b in range(B):
        qr = oracle.rope(q[b], pos0=p0)
        ref = oracle.decode_reuse_rows(qr, Kc[b], Vc[b], qi[b, 0], kb[b], L, Kbudget=K, mode=mode)
        nc = oracle.num_complete(p0)
        exempt = check_selection(ref["s"][:nc], K, ref["sK"], ref["sK1"], blk[b], int(ns[b]))
        for i in range(n):
            tok = oracle.token_set_reuse(blk[b, :ns[b]], p0, p0 + i)
            Oi, li, _ = oracle.attend_row(qr[i], Kc[b], Vc[b], tok)
            assert_close(Og[b, i], Oi, f"seq {b} query {i} O on the GPU selection")
            assert_close(lg[b, i], li, f"seq {b} query {i} lse")
        if not exempt:
            assert_close(Og[b], ref["O"], f"seq {b} O end to end")
        if L == 150:
            Od, _ = oracle.dense_rows(qr, Kc[b], Vc[b], np.arange(n), pos0=p0)
            assert_close(Og[b], Od, f"seq {b} within budget: dense")
        log(f"  seq {b}: selection {'in the tie band' if exempt else 'exact'}")


def test_decode_select_reuse_matches_single_query_form(qsa):
    """The selection for next_n queries is the one-query selection at the
    first query's position, bit for bit (long rows: filter pass)."""
    torch = _torch()
    B, n, nb_max, K = 3, 4, 40000, 512
    lens = np.array([4 * nb_max, 4 * nb_max - 2, 4 * 30001 + 1], dtype=np.int64)
    qi = synth.normal_bf16(4, (B, n, 4, 128), seed=34)
    kb = synth.normal_bf16(5, (B, nb_max, 128), seed=34)
    outs = []
    for form in ("reuse", "single"):
        m = n if form == "reuse" else 1
        ln = lens if form == "reuse" else lens - n + 1
        qq = qi if form == "reuse" else np.ascontiguousarray(qi[:, 0])
        blk = torch.full((B, K), 7, dtype=torch.int32, device="cuda")
        ns = torch.full((B,), 7, dtype=torch.int32, device="cuda")
        wsb = qsa.qsa_select_workspace_bytes(B, m, nb_max, K)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device="cuda")
        qsa.qsa_select_blocks(dev(qq), dev(kb), B, m, 0, dev(ln), nb_max, 4, 128, 4, 0, K, blk,
                              ns, ws, wsb)
        torch.cuda.synchronize()
        outs.append((blk.cpu().numpy(), ns.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    for b in range(B):
        p0 = int(lens[b]) - n
        ref = oracle.select_rows(qi[b, :1], kb[b], np.array([0]), pos0=p0, Kbudget=K,
                                 want_scores=True)
        nc = oracle.num_complete(p0)
        check_selection(ref["s"][0, :nc], K, ref["sK"][0], ref["sK1"][0], outs[0][0][b],
                        int(outs[0][1][b]))
