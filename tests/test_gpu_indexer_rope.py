"""The indexer with partial RoPE after pooling and an RMSNorm gain on the
pooled keys (chlience section 6: keys are average-pooled first and partial
RoPE is applied after; k-bar = RMSNorm(AvgPool(k))).  Pooled keys rotate at
their block's first token, indexer queries at their own positions.  The HIP
path runs through the C ABI; the fp64 oracle checks it."""
import dataclasses

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


@pytest.mark.parametrize("mode,rope_dim,block0,with_gain", [(0, 64, 0, False),
                                                            (0, 32, 12345, False),
                                                            (1, 64, 3, True),
                                                            (1, 128, 0, True),
                                                            (1, 0, 0, True)])
def test_compress_rope_and_gain_parity(qsa, mode, rope_dim, block0, with_gain):
    torch = _torch()
    B, Tk = 3, 4 * 1000 + 3
    k = synth.normal_bf16(5, (B, Tk, 128), seed=41)
    gain = None
    if with_gain:
        gain = synth.normal_bf16(6, (128,), seed=41)
    nb = Tk // 4
    out = torch.empty((B, nb, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_compress_keys(dev(k), B, Tk, Tk * 128, 128, 4, mode, out, nb * 128,
                          gain=None if gain is None else dev(gain), rope_dim=rope_dim,
                          block0=block0)
    torch.cuda.synchronize()
    got = host_u16(out)
    for b in range(B):
        ref = oracle.compress(k[b], mode=mode, gain=gain, rope_dim=rope_dim, block0=block0)
        d = np.abs(got[b].astype(np.int32) - ref.astype(np.int32))
        # one fp64 computation rounded once on both sides: a 1-ulp flip at most
        assert d.max() <= 1 and (d > 0).sum() <= got[b].size * 1e-4, (b, int(d.max()))


def test_prefill_with_indexer_rope_all_rows(qsa):
    """QSAPrefill with a 64-dim partial RoPE on the indexer, T = 2048, budget
    64: selection against the oracle's scores of rotated queries and pooled
    keys (tie band), outputs against the oracle's attention."""
    torch = _torch()
    T, K = 2048, 64
    x = synth.prefill_inputs(T, seed=42)
    layer = qsa.QSAPrefill(T, budget=K, idx_rope_dim=64)
    O, lse = layer(dev(x.Q), dev(x.K), dev(x.V), dev(x.qi), dev(x.ki))
    torch.cuda.synchronize()
    O, lse = O.cpu().numpy(), lse.cpu().numpy()
    qi_r = oracle.rope(x.qi, rope_dim=64)
    kb = oracle.compress(x.ki, rope_dim=64)
    Qr, Kr = oracle.rope(x.Q), oracle.rope(x.K)
    rows = np.arange(T)
    sel_g, ns_g = layer.blk_idx.cpu().numpy(), layer.n_sel.cpu().numpy()
    ref = oracle.select_rows(qi_r, kb, rows, Kbudget=K, want_scores=True)
    exempt = 0
    for t in rows:
        nc = (t + 1) // 4
        exempt += check_selection(ref["s"][t, :nc], K, ref["sK"][t], ref["sK1"][t], sel_g[t],
                                  ns_g[t])
    log(f"  {exempt} rows differ inside the tie band")
    Oref, lref = oracle.sparse_attn_rows(Qr, Kr, x.V, rows, sel_g, ns_g)
    assert_close(O, Oref, "O vs oracle on the GPU selection")
    assert_close(lse, lref, "lse vs oracle on the GPU selection")
    # the rotation changes the selection (it is not a no-op)
    plain = oracle.select_rows(x.qi, oracle.compress(x.ki), rows[-64:], Kbudget=K)
    assert not np.array_equal(plain["sel"], sel_g[-64:])


def test_chunked_prefill_with_indexer_rope(qsa):
    """Two chunks against a cache (the second pools its own blocks at
    block0 = pos0 / 4) reproduce the one-shot prefill with indexer RoPE."""
    torch = _torch()
    T, K, split = 2000, 64, 1200
    x = synth.prefill_inputs(T, seed=43)
    full = qsa.QSAPrefill(T, budget=K, idx_rope_dim=64)
    O, _ = full(dev(x.Q), dev(x.K), dev(x.V), dev(x.qi), dev(x.ki))
    torch.cuda.synchronize()
    O = O.cpu().numpy().copy()
    kbar = torch.zeros((T // 4, 128), dtype=torch.bfloat16, device="cuda")
    outs = []
    for p0, n in [(0, split), (split, T - split)]:
        ch = qsa.QSAPrefill(n, pos0=p0, budget=K, fresh=False, idx_rope_dim=64)
        Oc, _ = ch(dev(x.Q[p0:p0 + n]), full.Kr[:p0 + n], dev(x.V[:p0 + n]),
                   dev(x.qi[p0:p0 + n]), dev(x.ki), kbar)
        torch.cuda.synchronize()
        outs.append(Oc.cpu().numpy().copy())
    assert np.array_equal(np.concatenate(outs), O)


@pytest.mark.parametrize("n", [1, 4])
def test_decode_with_indexer_rope(qsa, n):
    torch = _torch()
    B, L, K = 2, 3001, 64
    seqs = [synth.decode_seq(b, L, L, seed=44) for b in range(B)]
    Kc = np.stack([s.K for s in seqs])
    Vc = np.stack([s.V for s in seqs])
    ki = np.stack([s.ki for s in seqs])
    q = synth.normal_bf16(1, (B, n, 24, 256), seed=45)
    qi = synth.normal_bf16(4, (B, n, 4, 128), seed=45)
    dec = qsa.QSADecode(B, L, budget=K, next_n=n, idx_rope_dim=64)
    kbar = torch.empty((B, L // 4, 128), dtype=torch.bfloat16, device="cuda")
    dec.pool_keys(dev(ki[:, :4 * (L // 4)]), kbar)
    lens = np.full(B, L, dtype=np.int64)
    O, _ = dec(dev(q), dev(qi), dev(Kc), dev(Vc), kbar, dev(lens))
    torch.cuda.synchronize()
    Og = O.cpu().numpy().reshape(B, n, 24, 256)
    blk, ns = dec.blk_idx.cpu().numpy(), dec.n_sel.cpu().numpy()
    p0 = L - n
    for b in range(B):
        kb = oracle.compress(ki[b], rope_dim=64)
        qi0 = oracle.rope(qi[b, :1], rope_dim=64, pos0=p0)[0]
        qr = oracle.rope(q[b], pos0=p0)
        ref = oracle.decode_reuse_rows(qr, Kc[b], Vc[b], qi0, kb, L, Kbudget=K)
        nc = oracle.num_complete(p0)
        ex = check_selection(ref["s"][:nc], K, ref["sK"], ref["sK1"], blk[b], int(ns[b]))
        for i in range(n):
            tok = oracle.token_set_reuse(blk[b, :ns[b]], p0, p0 + i)
            Oi, _, _ = oracle.attend_row(qr[i], Kc[b], Vc[b], tok)
            assert_close(Og[b, i], Oi, f"seq {b} query {i} O")
        if not ex:
            assert_close(Og[b], ref["O"], f"seq {b} O end to end")
