"""Paged KV and pooled-key caches: the same workload laid out in randomly
permuted pages of a pool (page table per sequence) must give bit for bit the
results of the contiguous layout, and the paged results are checked against
the fp64 oracle on the contiguous arrays (selection by the tie-band rule,
attention over the GPU's selection, dense attention).  Pages no sequence
owns are filled with NaN, so a read of a page the table does not hand out
would show in the outputs."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, check_prefill_rows, check_selection, dev, host_u16, log

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


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


def page_layout(lens, Lmax, P, seed):
    """Random page assignment: table [B, ceil(Lmax/P)] int32 (entries past a
    sequence's pages point at a spare NaN page), and the pool size."""
    rng = np.random.default_rng(seed)
    npg = [-(-int(max(l, 1)) // P) for l in lens]
    total = sum(npg) + 1
    perm = rng.permutation(total).astype(np.int32)
    stride = -(-Lmax // P)
    table = np.full((len(lens), stride), perm[-1], dtype=np.int32)
    k = 0
    for b, n in enumerate(npg):
        table[b, :n] = perm[k:k + n]
        k += n
    return table, total


def to_pool(cache, table, total, rows_per_page, valid=None):
    """cache [B, Lrows, ...] (uint16) -> pool [total * rows_per_page, ...];
    only the first valid[b] rows of sequence b (its own pages) are placed."""
    B, L = cache.shape[:2]
    pool = np.full((total * rows_per_page,) + cache.shape[2:], NAN_BF16, dtype=np.uint16)
    for b in range(B):
        vb = L if valid is None else min(L, int(valid[b]))
        for i in range(table.shape[1]):
            r0 = i * rows_per_page
            if r0 >= vb:
                break
            r1 = min(r0 + rows_per_page, L)
            pid = int(table[b, i])
            pool[pid * rows_per_page:pid * rows_per_page + r1 - r0] = cache[b, r0:r1]
    return pool


def _decode_inputs(B, Lmax, n, seed):
    Kc = synth.normal_bf16(2, (B, Lmax, 2, 256), seed=seed)
    Vc = synth.normal_bf16(3, (B, Lmax, 2, 256), seed=seed)
    ki = synth.normal_bf16(5, (B, Lmax, 128), seed=seed)
    q = synth.normal_bf16(1, (B, n, 24, 256), seed=seed)
    qi = synth.normal_bf16(4, (B, n, 4, 128), seed=seed)
    return Kc, Vc, ki, q, qi


@pytest.mark.parametrize("P,n,budget,idx_rope", [(16, 1, 64, 0), (64, 4, 64, 64),
                                                 (256, 1, 512, 0), (4096, 2, 512, 0)])
def test_paged_decode_equals_contiguous(qsa, P, n, budget, idx_rope):
    """QSADecode (pooling into the pages, selection, sparse attention) and the
    dense decode over paged caches equal the contiguous runs exactly."""
    torch = _torch()
    B, Lmax = 3, 60000
    lens = np.array([60000, 33331, 2050], dtype=np.int64)
    Kc, Vc, ki, q, qi = _decode_inputs(B, Lmax, n, seed=50 + P)
    table, total = page_layout(lens, Lmax, P, seed=P)
    pg = qsa.Pages(dev(table), P)
    ln = dev(lens)
    outs = []
    for paged in (False, True):
        dec = qsa.QSADecode(B, Lmax, budget=budget, next_n=n, idx_rope_dim=idx_rope,
                            pages=pg if paged else None)
        if paged:
            kbar = torch.full((total * P // 4, 128), -1, dtype=torch.int16, device="cuda")
            kc = dev(to_pool(Kc, table, total, P, valid=lens))
            vc = dev(to_pool(Vc, table, total, P, valid=lens))
        else:
            kbar = torch.full((B, Lmax // 4, 128), -1, dtype=torch.int16, device="cuda")
            kc, vc = dev(Kc), dev(Vc)
        dec.pool_keys(dev(ki), kbar)
        O, lse = dec(dev(q), dev(qi), kc, vc, kbar, ln)
        Od = torch.empty((B, n, 24, 256), dtype=torch.float32, device="cuda")
        wsb = qsa.dense_attn_workspace_bytes(B, n, Lmax, 24, 2, 256)
        ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
        qsa.dense_attn(dec.qr, kc, vc, B, n, Lmax, 0, ln, 24, 2, 256, Od, None, ws, wsb,
                       pages=pg if paged else None)
        torch.cuda.synchronize()
        outs.append([x.cpu().numpy().copy() for x in (dec.blk_idx, dec.n_sel, O, lse, Od)])
        del dec, kbar, kc, vc
    for name, a, b in zip(("blk_idx", "n_sel", "O", "lse", "dense O"), *outs):
        assert np.array_equal(a, b, equal_nan=False), name
    assert np.all(np.isfinite(outs[1][2])) and np.all(np.isfinite(outs[1][4]))
    # the paged results against the oracle: the selection made for the first
    # of each sequence's n queries (indexer RoPE at its position when on), each
    # query over the shared selection plus its own causal tail, dense attention
    blk, nsel, O, lse, Od = outs[1]
    O, lse = O.reshape(B, n, 24, 256), lse.reshape(B, n, 24)   # next_n = 1 returns [B, H, ...]
    Og, lg, Or, lr, Odg, Odr = [], [], [], [], [], []
    exempt = 0
    for b in range(B):
        L = int(lens[b])
        p0 = L - n
        kb = oracle.compress(ki[b, :L], rope_dim=idx_rope)
        q0 = qi[b, :1]
        if idx_rope:
            q0 = oracle.rope(q0, rope_dim=idx_rope, pos=np.array([p0]))
        ref = oracle.select_rows(q0, kb, np.array([0]), pos0=p0, Kbudget=budget,
                                 want_scores=True)
        exempt += int(check_selection(ref["s"][0], budget, ref["sK"][0], ref["sK1"][0], blk[b],
                                      nsel[b], strict=ref["sel"][0, :ref["nsel"][0]]))
        Qr = oracle.rope(q[b], pos=p0 + np.arange(n))
        sel_b = blk[b, :nsel[b]]
        for i in range(n):
            o, l, _ = oracle.attend_row(Qr[i], Kc[b], Vc[b], oracle.token_set_reuse(sel_b, p0,
                                                                                     p0 + i))
            Og.append(O[b, i])
            lg.append(lse[b, i])
            Or.append(o)
            lr.append(l)
        od, _ = oracle.dense_rows(Qr, Kc[b], Vc[b], np.arange(n), pos0=p0)
        Odg.append(Od[b])
        Odr.append(od)
    log(f"  paged decode P={P} next_n={n}: {exempt} of {B} selections differ inside the tie band")
    assert_close(np.stack(Og), np.stack(Or), "paged decode O vs oracle on the GPU selection")
    assert_close(np.stack(lg), np.stack(lr), "paged decode lse vs oracle")
    assert_close(np.concatenate(Odg), np.concatenate(Odr), "paged dense decode O vs oracle")


@pytest.mark.parametrize("P", [16, 128])
def test_paged_prefill_chunk_equals_contiguous(qsa, P):
    """A prefill chunk against a paged post-RoPE cache (the chunk's indexer
    keys pooled into the pages), and the dense prefill over the same pages,
    equal the contiguous runs exactly."""
    torch = _torch()
    pos0, Tq, K = 6000, 1100, 512
    Tk = pos0 + Tq
    x = synth.prefill_inputs(Tq, pos0=pos0, seed=60 + P, k_is_rotated=True)
    table, total = page_layout([Tk], Tk, P, seed=P + 1)
    pg = qsa.Pages(dev(table), P)
    outs = []
    for paged in (False, True):
        if paged:
            kc = dev(to_pool(x.K[None], table, total, P))
            vc = dev(to_pool(x.V[None], table, total, P))
            kbar = torch.full((total * P // 4, 128), -1, dtype=torch.int16, device="cuda")
            qsa.qsa_compress_keys(dev(x.ki), 1, pos0, pos0 * 128, 128, 4, 0, kbar, 0, pages=pg)
        else:
            kc, vc = dev(x.K), dev(x.V)
            kbar = torch.full((Tk // 4, 128), -1, dtype=torch.int16, device="cuda")
            qsa.qsa_compress_keys(dev(x.ki), 1, pos0, pos0 * 128, 128, 4, 0, kbar,
                                  (pos0 // 4) * 128)
        layer = qsa.QSAPrefill(Tq, pos0=pos0, budget=K, fresh=False,
                               pages=pg if paged else None)
        O, lse = layer(dev(x.Q), kc, vc, dev(x.qi), dev(x.ki), kbar)
        Od = torch.empty((1, Tq, 24, 256), dtype=torch.float32, device="cuda")
        qsa.dense_attn(layer.Qr, kc, vc, 1, Tq, Tk, pos0, None, 24, 2, 256, Od,
                       pages=pg if paged else None)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (layer.blk_idx, layer.n_sel, O, lse, Od)])
        del layer, kc, vc, kbar
    for name, a, b in zip(("blk_idx", "n_sel", "O", "lse", "dense O"), *outs):
        assert np.array_equal(a, b), name
    # every row of the paged chunk against the oracle on the contiguous arrays
    blk, nsel, O, lse, Od = outs[1]
    kb = oracle.compress(x.ki)
    check_prefill_rows(O, lse, blk, nsel, x.Q, x.K, x.V, x.qi, kb, np.arange(Tq), pos0, K)
    rows = np.array([0, 1, 2, 3, 517, Tq - 2, Tq - 1])
    Qr = oracle.rope(x.Q[rows], pos=pos0 + rows)
    Odr = np.stack([oracle.dense_rows(Qr[i:i + 1], x.K, x.V, np.array([0]),
                                      pos0=pos0 + int(t))[0][0] for i, t in enumerate(rows)])
    assert_close(Od[0, rows], Odr, f"paged dense prefill O vs oracle (P={P})")


def test_paged_compress_and_scores(qsa):
    """Pooling into pages from block0 > 0, and the indexer scores (decode and
    prefill forms) over paged pooled keys, equal the contiguous layout."""
    torch = _torch()
    P, B, Lmax = 32, 2, 8192
    ki = synth.normal_bf16(5, (B, Lmax, 128), seed=70)
    lens = np.array([8192, 5001], dtype=np.int64)   # the scores' sequence lengths
    table, total = page_layout([Lmax, Lmax], Lmax, P, seed=70)
    pg = qsa.Pages(dev(table), P)
    nb = Lmax // 4
    cont = torch.zeros((B, nb, 128), dtype=torch.int16, device="cuda")
    pool = torch.zeros((total * P // 4, 128), dtype=torch.int16, device="cuda")
    # two appends: blocks 0..999, then 1000..2047
    for b0, nblk in ((0, 1000), (1000, nb - 1000)):
        src = dev(np.ascontiguousarray(ki[:, 4 * b0:4 * (b0 + nblk)]))
        qsa.qsa_compress_keys(src, B, 4 * nblk, 4 * nblk * 128, 128, 4, 1, cont[:, b0], nb * 128,
                              rope_dim=64, block0=b0)
        qsa.qsa_compress_keys(src, B, 4 * nblk, 4 * nblk * 128, 128, 4, 1, pool, 0,
                              rope_dim=64, block0=b0, pages=pg)
    torch.cuda.synchronize()
    got = host_u16(pool)
    want = host_u16(cont)
    for b in range(B):
        for j in range(nb):
            row = int(table[b, (4 * j) // P]) * (P // 4) + j % (P // 4)
            assert np.array_equal(got[row], want[b, j]), (b, j)
    qi = synth.normal_bf16(4, (B, 4, 128), seed=71)
    ld = nb
    s1 = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    s2 = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    qsa.qsa_index_scores(dev(qi), cont, B, 1, 0, dev(lens), nb, 4, 128, 4, 0, s1, ld)
    qsa.qsa_index_scores(dev(qi), pool, B, 1, 0, dev(lens), nb, 4, 128, 4, 0, s2, ld, pages=pg)
    torch.cuda.synchronize()
    for b in range(B):
        nc = int(lens[b]) // 4
        assert np.array_equal(s1[b, :nc].cpu().numpy(), s2[b, :nc].cpu().numpy())
    # prefill form over sequence 0's pages: 700 queries ending at 8191
    qp = synth.normal_bf16(4, (700, 4, 128), seed=72)
    p0 = Lmax - 700
    t1 = torch.empty((700, ld), dtype=torch.float32, device="cuda")
    t2 = torch.empty((700, ld), dtype=torch.float32, device="cuda")
    qsa.qsa_index_scores(dev(qp), cont[0], 1, 700, p0, None, nb, 4, 128, 4, 0, t1, ld)
    qsa.qsa_index_scores(dev(qp), pool, 1, 700, p0, None, nb, 4, 128, 4, 0, t2, ld, pages=pg)
    torch.cuda.synchronize()
    a, c = t1.cpu().numpy(), t2.cpu().numpy()
    for t in range(0, 700, 37):
        nc = (p0 + t + 1) // 4
        assert np.array_equal(a[t, :nc], c[t, :nc]), t
