"""Kernels of the library running concurrently on two streams give the same
bits as when run alone.  A workgroup barrier that publishes LDS data must
wait for the wave's own LDS stores first: without that wait the prefill
indexer once read pooled-key rows still being written whenever LDS-DMA
kernels on another stream loaded the CU (the decode scan, the sparse
attention), and its scores changed.  These tests run the fixed kernels under
that load and are meant to pass."""
import numpy as np
import pytest

import synth
from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import torch
    import block_sparse_long_08_amd as q
    assert torch.cuda.is_available()
    q.qsa_check_device()
    return q


def test_prefill_scores_with_a_concurrent_decode_scan(qsa):
    """4,096 prefill rows at 61,440 (nc up to 16,383 blocks) scored while 32
    decode scans of 65,536 pooled keys run on a second stream: every score
    equals the one computed alone."""
    import torch
    r0, n = 61440, 4096
    Tk = r0 + n
    nb = Tk // 4
    qi = dev(synth.normal_bf16(4, (n, 4, 128), seed=90))
    kb = dev(synth.normal_bf16(5, (nb, 128), seed=90))
    kbd = dev(synth.normal_bf16(5, (32, 65536, 128), seed=91))
    qd = dev(synth.normal_bf16(4, (32, 4, 128), seed=91))
    lens = torch.full((32,), 262144, dtype=torch.int64, device="cuda")
    sd = torch.empty((32, 65536), dtype=torch.float32, device="cuda")
    ref = torch.empty((n, nb), dtype=torch.float32, device="cuda")
    qsa.qsa_index_scores(qi, kb, 1, n, r0, None, nb, 4, 128, 4, 0, ref, nb)
    torch.cuda.synchronize()
    nc = (torch.arange(r0, r0 + n, device="cuda")[:, None] + 1) // 4  # complete blocks per row
    mask = torch.arange(nb, device="cuda")[None, :] < nc
    side = torch.cuda.Stream()
    bad = 0
    for trial in range(4):
        got = torch.full((n, nb), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(40):
                qsa.qsa_index_scores(qd, kbd, 32, 1, 0, lens, 65536, 4, 128, 4, 0, sd, 65536)
        for _ in range(3):
            qsa.qsa_index_scores(qi, kb, 1, n, r0, None, nb, 4, 128, 4, 0, got, nb)
        torch.cuda.synchronize()
        bad += int(((got != ref) & mask).any(dim=1).sum())
    log(f"  rows with a differing score over 4 trials: {bad}")
    assert bad == 0


def test_pipelined_prefill_equals_sequential(qsa):
    """The prefill layer with selection and attention overlapped on two
    streams (attention of a row chunk while the next chunk is selected)
    equals the layer run one stage after the other, bit for bit."""
    import torch
    T = 24576
    x = synth.prefill_inputs(T, seed=92, needles_per_head=8)
    ins = [dev(a) for a in (x.Q, x.K, x.V, x.qi, x.ki)]
    outs = []
    for rows in (0, 2048):
        layer = qsa.QSAPrefill(T, budget=512, pipeline_rows=rows)
        O, lse = layer(*ins)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (layer.blk_idx, layer.n_sel, O, lse)])
        del layer
    for name, a, b in zip(("blk_idx", "n_sel", "O", "lse"), *outs):
        assert np.array_equal(a, b), name


@pytest.mark.parametrize("P", [0, 64])
def test_pipelined_chunk_over_a_cache_equals_sequential(qsa, P):
    """A prefill chunk against a post-RoPE cache (contiguous, or in 64-token
    pages): the pipelined layer (256-row chunks) equals the stages run in
    turn, bit for bit."""
    import torch
    from test_gpu_paged import page_layout, to_pool
    pos0, Tq = 9000, 1800
    Tk = pos0 + Tq
    x = synth.prefill_inputs(Tq, pos0=pos0, seed=93, k_is_rotated=True)
    pages = None
    if P:
        table, total = page_layout([Tk], Tk, P, seed=93)
        pages = qsa.Pages(dev(table), P)
        kc, vc = dev(to_pool(x.K[None], table, total, P)), dev(to_pool(x.V[None], table, total, P))
    else:
        kc, vc = dev(x.K), dev(x.V)
    outs = []
    for rows in (0, 256):
        if P:
            kbar = torch.full((total * P // 4, 128), -1, dtype=torch.int16, device="cuda")
            qsa.qsa_compress_keys(dev(x.ki), 1, pos0, pos0 * 128, 128, 4, 0, kbar, 0, pages=pages)
        else:
            kbar = torch.full((Tk // 4, 128), -1, dtype=torch.int16, device="cuda")
            qsa.qsa_compress_keys(dev(x.ki), 1, pos0, pos0 * 128, 128, 4, 0, kbar, (pos0 // 4) * 128)
        layer = qsa.QSAPrefill(Tq, pos0=pos0, budget=512, fresh=False, pages=pages,
                               pipeline_rows=rows)
        O, lse = layer(dev(x.Q), kc, vc, dev(x.qi), dev(x.ki), kbar)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (layer.blk_idx, layer.n_sel, O, lse)])
        del layer, kbar
    for name, a, b in zip(("blk_idx", "n_sel", "O", "lse"), *outs):
        assert np.array_equal(a, b), name
