"""Parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times.  The HIP path runs the whole workload through
the C ABI; the fp64 oracle checks query rows one by one:

  - selection: the GPU set against the oracle's scores (tie-band rule);
  - attention: the GPU output against the oracle's attention over the GPU's
    (validated) selection;
  - end to end: against the oracle's own selection where the sets agree.

Every row at 32K; at 128K and at the 1M-context chunks, at least 256 rows
that include the first row whose context exceeds the budget, the first and
last row of every 4,096-row chunk the layer pipelines on, and rows of every
trailing-block length.  Decode: every sequence, each regenerated on the host
for the oracle.  Inputs: the seeded N(0,1) bf16 recipes of the workloads
(needle blocks where the workload plants them)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (assert_close, check_prefill_rows, check_selection, dev, log,
                         sample_prefill_rows, score_chunk_rows)

# the oracle's side of these checks runs on the host cores for up to a few
# minutes per test (it prints a progress line per chunk of rows)
pytestmark = [pytest.mark.gpu, pytest.mark.big, pytest.mark.timeout(900)]


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


def _run_prefill(qsa, x, budget, pages=None):
    """The QSA layer as bench.py runs it: a fresh context, or a chunk against
    a post-RoPE cache whose pooled keys are built first; pages = a page size
    in tokens lays the cache out in randomly permuted pages of a pool."""
    torch = _torch()
    Tq, pos0 = x.Q.shape[0], x.pos0
    fresh = pos0 == 0
    Q, K, V, qi, ki = map(dev, (x.Q, x.K, x.V, x.qi, x.ki))
    Tk = pos0 + Tq
    kbar = None
    pg = None
    if pages:
        P = pages
        g = torch.Generator().manual_seed(1)
        perm = torch.randperm(Tk // P, generator=g)
        table = perm.view(1, Tk // P).to(torch.int32).cuda()
        perm = perm.cuda()
        pg = qsa.Pages(table, P)

        def pool(c):
            rows = c.reshape(Tk // P, -1)
            out = torch.empty_like(rows)
            out.index_copy_(0, perm, rows)
            return out.view(c.shape)
        K, V = pool(K), pool(V)
        kbar = torch.empty((Tk // 4, 128), dtype=torch.bfloat16, device="cuda")
        qsa.qsa_compress_keys(ki, 1, pos0, pos0 * 128, 128, 4, 0, kbar, 0, pages=pg)
    elif not fresh:
        kbar = torch.empty((Tk // 4, 128), dtype=torch.bfloat16, device="cuda")
        qsa.qsa_compress_keys(ki, 1, pos0, pos0 * 128, 128, 4, 0, kbar, (pos0 // 4) * 128)
    layer = qsa.QSAPrefill(Tq, pos0=pos0, budget=budget, fresh=fresh, pages=pg)
    O, lse = layer(Q, K, V, qi, ki, kbar)
    torch.cuda.synchronize()
    out = (O.cpu().numpy(), lse.cpu().numpy(), layer.blk_idx.cpu().numpy(),
           layer.n_sel.cpu().numpy(), layer.attn_rows)
    del layer, Q, K, V, qi, ki, kbar, pg
    torch.cuda.empty_cache()
    return out


def _check_full_size(qsa, Tq, pos0, needles, nrows, pages=None):
    log(f"prefill Tq={Tq} pos0={pos0} needles={needles} pages={pages}: generating inputs")
    x = synth.prefill_inputs(Tq, pos0=pos0, seed=0, needles_per_head=needles)
    log("  running the HIP path")
    O, lse, blk, nsel, attn_rows = _run_prefill(qsa, x, 512, pages=pages)
    # every row: a full ascending selection of min(512, nc) blocks
    nc = np.minimum((pos0 + np.arange(Tq) + 1) // 4, (pos0 + Tq) // 4)
    assert np.array_equal(nsel, np.minimum(nc, 512))
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    # edges of the attention launches the layer made and of the score chunks
    edges = (attn_rows, score_chunk_rows(Tq, (pos0 + Tq) // 4))
    rows = (np.arange(Tq, dtype=np.int64) if nrows is None
            else sample_prefill_rows(Tq, pos0, 512, nrows, seed=Tq, chunk_rows=edges))
    log(f"  attention launches of {attn_rows} rows, score chunks of {edges[1]} rows")
    log(f"  oracle check of {rows.size} rows")
    Kr = x.K if x.k_is_rotated else oracle.rope(x.K)
    kb = oracle.compress(x.ki)
    check_prefill_rows(O, lse, blk, nsel, x.Q, Kr, x.V, x.qi, kb, rows, pos0, 512)


def test_prefill_32k_every_row(qsa):
    """prefill_32k: all 32,768 rows against the oracle."""
    _check_full_size(qsa, 32768, 0, 0, None)


@pytest.mark.parametrize("Tq,pos0,needles", [(131072, 0, 64), (8192, 1048576 - 8192, 64)])
def test_prefill_full_size_sampled(qsa, Tq, pos0, needles):
    """prefill_128k and the 8,192-query chunk at 1M: 256 structured rows."""
    _check_full_size(qsa, Tq, pos0, needles, 256)


def test_prefill_1m_chunk16k_paged(qsa):
    """The report's prefill condition (chlience "Result 2": batch 1, 16K-token
    chunks, a paged cache): 16,384 queries at 1,032,192 .. 1,048,575 over a
    1,048,576-token cache in randomly permuted 64-token pages, as bench.py
    times it; 256 structured rows against the oracle on the contiguous
    arrays."""
    _check_full_size(qsa, 16384, 1048576 - 16384, 64, 256, pages=64)


def test_dense_prefill_32k_sampled(qsa):
    """The dense baseline as bench.py times it (32,768 queries)."""
    torch = _torch()
    T = 32768
    log("dense prefill T=32768")
    x = synth.prefill_inputs(T, seed=0)
    Kr = oracle.rope(x.K)
    Qr = oracle.rope(x.Q)
    O = torch.empty((T, 24, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, 24), dtype=torch.float32, device="cuda")
    qsa.dense_attn(dev(Qr), dev(Kr), dev(x.V), 1, T, T, 0, None, 24, 2, 256, O, lse)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 2047, T - 1],
                                     np.random.default_rng(1).choice(T, 60, replace=False)]))
    Oref, lref = oracle.dense_rows(Qr, Kr, x.V, rows)
    assert_close(O.cpu().numpy()[rows], Oref, "dense O at 32K")
    assert_close(lse.cpu().numpy()[rows], lref, "dense lse at 32K")


@pytest.mark.parametrize("B,L,needles", [(32, 262144, 0), (4, 1048576, 64)])
def test_decode_full_size(qsa, B, L, needles):
    """decode_256k_b32 and decode_1m_b4: every sequence against the oracle
    (each sequence regenerated on the host after the GPU run)."""
    torch = _torch()
    log(f"decode B={B} L={L}: generating caches")
    Kc = torch.empty((B, L, 2, 256), dtype=torch.int16, device="cuda")
    Vc = torch.empty((B, L, 2, 256), dtype=torch.int16, device="cuda")
    kbar = torch.empty((B, L // 4, 128), dtype=torch.int16, device="cuda")
    qh = np.empty((B, 24, 256), dtype=np.uint16)
    qih = np.empty((B, 4, 128), dtype=np.uint16)
    for b in range(B):
        s = synth.decode_seq(b, L, L, needles_per_head=needles)
        Kc[b].copy_(dev(s.K))
        Vc[b].copy_(dev(s.V))
        qsa.qsa_compress_keys(dev(s.ki), 1, L, L * 128, 128, 4, 0, kbar[b], (L // 4) * 128)
        qh[b], qih[b] = s.q, s.qi
        torch.cuda.synchronize()
        del s
    seq_len = torch.full((B,), L, dtype=torch.int64, device="cuda")
    log("  running the HIP path")
    dec = qsa.QSADecode(B, L, budget=512)
    O, lse = dec(dev(qh), dev(qih), Kc, Vc, kbar, seq_len)
    torch.cuda.synchronize()
    Og, lg = O.cpu().numpy(), lse.cpu().numpy()
    blk, nsel = dec.blk_idx.cpu().numpy(), dec.n_sel.cpu().numpy()
    del Kc, Vc, kbar, dec
    torch.cuda.empty_cache()
    assert np.all(nsel == 512)
    p = L - 1
    Orefs, lrefs, exempt, e2e_g, e2e_r = [], [], 0, [], []
    for b in range(B):
        s = synth.decode_seq(b, L, L, needles_per_head=needles)
        kb = oracle.compress(s.ki)
        ref = oracle.select_rows(s.qi[None], kb, np.array([0]), pos0=p, Kbudget=512,
                                 want_scores=True)
        ex = check_selection(ref["s"][0], 512, ref["sK"][0], ref["sK1"][0], blk[b], nsel[b],
                             strict=ref["sel"][0, :ref["nsel"][0]])
        exempt += int(ex)
        Qr = oracle.rope(s.q[None], pos0=p)
        Or, lr = oracle.sparse_attn_rows_at(Qr, s.K, s.V, np.array([p]), blk[b:b + 1],
                                            nsel[b:b + 1])
        Orefs.append(Or[0])
        lrefs.append(lr[0])
        if not ex and len(e2e_g) < 4:
            e2e = oracle.qsa_rows_at(Qr, s.K, s.V, s.qi[None], kb, np.array([p]), Kbudget=512)
            e2e_g.append(Og[b])
            e2e_r.append(e2e["O"][0])
        del s, kb
        log(f"  sequence {b + 1}/{B} checked")
    log(f"  {B} sequences: {exempt} selections differ inside the tie band")
    assert_close(Og, np.stack(Orefs), "decode O on the GPU selection")
    assert_close(lg, np.stack(lrefs), "decode lse on the GPU selection")
    if e2e_g:
        assert_close(np.stack(e2e_g), np.stack(e2e_r), "decode O end to end")
