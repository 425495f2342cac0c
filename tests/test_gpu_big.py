"""Parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times.  The HIP path runs the whole workload through
the C ABI; the fp64 oracle checks sampled query rows one by one:

  - selection: the GPU set against the oracle's scores (tie-band rule);
  - attention: the GPU output against the oracle's attention over the GPU's
    (validated) selection;
  - end to end: against the oracle's own selection where the sets agree.

Rows always include the first row whose context exceeds the budget and the
last row.  Inputs: the seeded N(0,1) bf16 recipes of the workloads (needle
blocks where the workload plants them)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, check_selection, dev, log

pytestmark = [pytest.mark.gpu, pytest.mark.big]


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


def _rows(Tq, pos0, budget, n, seed):
    """Sampled query rows: the first row with nc > budget, the last row, and
    n seeded random rows past the first sparse one."""
    first = max(0, 4 * (budget + 1) - 1 - pos0)
    rng = np.random.default_rng(seed)
    extra = rng.choice(np.arange(first, Tq), size=min(n, Tq - first), replace=False)
    return np.unique(np.concatenate([[first, Tq - 1], extra])).astype(np.int64)


def _check_prefill_rows(O, lse, blk, nsel, Q, Kr, V, qi, kb, rows, pos0, budget):
    """Oracle check of compact rows t (absolute positions pos0 + t)."""
    exempt, Orefs, lrefs = [], [], []
    for t in rows:
        p = int(pos0 + t)
        ref = oracle.select_rows(qi[t:t + 1], kb, np.array([0]), pos0=p, Kbudget=budget,
                                 want_scores=True)
        nc = min((p + 1) // 4, kb.shape[0])
        if check_selection(ref["s"][0, :nc], budget, ref["sK"][0], ref["sK1"][0], blk[t],
                           nsel[t]):
            exempt.append(int(t))
        Qr = oracle.rope(Q[t:t + 1], pos0=p)
        Or, lr = oracle.sparse_attn_rows(Qr, Kr, V, np.array([0]), blk[t:t + 1], nsel[t:t + 1],
                                         pos0=p)
        Orefs.append(Or[0])
        lrefs.append(lr[0])
    log(f"  {rows.size} rows: {len(exempt)} differ inside the tie band")
    assert_close(O[rows], np.stack(Orefs), "O vs oracle on the GPU selection")
    assert_close(lse[rows], np.stack(lrefs), "lse vs oracle on the GPU selection")
    same = np.array([int(t) not in set(exempt) for t in rows])
    if same.any():
        rs = rows[same]
        Qr = np.stack([oracle.rope(Q[t:t + 1], pos0=int(pos0 + t))[0] for t in rs])
        e2e = oracle.qsa_rows_at(Qr, Kr, V, qi[rs], kb, pos0 + rs, Kbudget=budget)
        assert_close(O[rs], e2e["O"], "O vs oracle end to end")
        assert np.all(e2e["wsum_err"] < 1e-12)


def _run_prefill(qsa, x, budget):
    """The QSA layer as bench.py runs it (fresh context or a chunk against a
    post-RoPE cache whose pooled keys are built first)."""
    torch = _torch()
    Tq, pos0 = x.Q.shape[0], x.pos0
    fresh = pos0 == 0
    Q, K, V, qi, ki = map(dev, (x.Q, x.K, x.V, x.qi, x.ki))
    Tk = pos0 + Tq
    kbar = None
    if not fresh:
        kbar = torch.empty((Tk // 4, 128), dtype=torch.bfloat16, device="cuda")
        qsa.qsa_compress_keys(ki, 1, pos0, pos0 * 128, 128, 4, 0, kbar, (pos0 // 4) * 128)
    layer = qsa.QSAPrefill(Tq, pos0=pos0, budget=budget, fresh=fresh)
    O, lse = layer(Q, K, V, qi, ki, kbar)
    torch.cuda.synchronize()
    out = (O.cpu().numpy(), lse.cpu().numpy(), layer.blk_idx.cpu().numpy(),
           layer.n_sel.cpu().numpy())
    del layer, Q, K, V, qi, ki, kbar
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("Tq,pos0,needles,nrows", [(32768, 0, 0, 14), (131072, 0, 64, 12),
                                                   (8192, 1048576 - 8192, 64, 10)])
def test_prefill_full_size(qsa, Tq, pos0, needles, nrows):
    log(f"prefill Tq={Tq} pos0={pos0} needles={needles}: generating inputs")
    x = synth.prefill_inputs(Tq, pos0=pos0, seed=0, needles_per_head=needles)
    log("  running the HIP path")
    O, lse, blk, nsel = _run_prefill(qsa, x, 512)
    rows = _rows(Tq, pos0, 512, nrows, seed=Tq)
    Kr = x.K if x.k_is_rotated else oracle.rope(x.K)
    kb = oracle.compress(x.ki)
    _check_prefill_rows(O, lse, blk, nsel, x.Q, Kr, x.V, x.qi, kb, rows, pos0, 512)
    # every row: a full ascending selection of min(512, nc) blocks
    nc = np.minimum((pos0 + np.arange(Tq) + 1) // 4, (pos0 + Tq) // 4)
    assert np.array_equal(nsel, np.minimum(nc, 512))
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))


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
                                     np.random.default_rng(1).choice(T, 6, replace=False)]))
    Oref, lref = oracle.dense_rows(Qr, Kr, x.V, rows)
    assert_close(O.cpu().numpy()[rows], Oref, "dense O at 32K")
    assert_close(lse.cpu().numpy()[rows], lref, "dense lse at 32K")


@pytest.mark.parametrize("B,L,needles,check", [(32, 262144, 0, (0, 17, 31)),
                                               (4, 1048576, 64, (0, 3))])
def test_decode_full_size(qsa, B, L, needles, check):
    torch = _torch()
    log(f"decode B={B} L={L}: generating caches")
    Kc = torch.empty((B, L, 2, 256), dtype=torch.int16, device="cuda")
    Vc = torch.empty((B, L, 2, 256), dtype=torch.int16, device="cuda")
    kbar = torch.empty((B, L // 4, 128), dtype=torch.int16, device="cuda")
    qh = np.empty((B, 24, 256), dtype=np.uint16)
    qih = np.empty((B, 4, 128), dtype=np.uint16)
    kept = {}
    for b in range(B):
        s = synth.decode_seq(b, L, L, needles_per_head=needles)
        Kc[b].copy_(dev(s.K))
        Vc[b].copy_(dev(s.V))
        qsa.qsa_compress_keys(dev(s.ki), 1, L, L * 128, 128, 4, 0, kbar[b], (L // 4) * 128)
        qh[b], qih[b] = s.q, s.qi
        if b in check:
            kept[b] = s
        torch.cuda.synchronize()
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
    for b in check:
        s = kept[b]
        p = L - 1
        kb = oracle.compress(s.ki)
        ref = oracle.select_rows(s.qi[None], kb, np.array([0]), pos0=p, Kbudget=512,
                                 want_scores=True)
        ex = check_selection(ref["s"][0], 512, ref["sK"][0], ref["sK1"][0], blk[b], nsel[b])
        Qr = oracle.rope(s.q[None], pos0=p)
        Or, lr = oracle.sparse_attn_rows(Qr, s.K, s.V, np.array([0]), blk[b:b + 1],
                                         nsel[b:b + 1], pos0=p)
        assert_close(Og[b], Or[0], f"decode seq {b} O on the GPU selection")
        assert_close(lg[b], lr[0], f"decode seq {b} lse")
        if not ex:
            e2e = oracle.qsa_rows_at(Qr, s.K, s.V, s.qi[None], kb, np.array([p]), Kbudget=512)
            assert_close(Og[b], e2e["O"][0], f"decode seq {b} O end to end")
