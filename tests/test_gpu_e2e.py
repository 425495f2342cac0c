"""End-to-end parity of the QSA layer (HIP path through the C ABI) with the
fp64 oracle, plus consistency properties.  Inputs follow the workload recipes
of the synth module (N(0,1) bf16, needles where the workload plants them)."""
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


def run_prefill(qsa, x, budget, mode=0, kbar_mode=0):
    torch = _torch()
    T = x.Q.shape[0]
    layer = qsa.QSAPrefill(T, pos0=0, budget=budget, score_mode=mode, kbar_mode=kbar_mode)
    O, lse = layer(dev(x.Q), dev(x.K), dev(x.V), dev(x.qi), dev(x.ki))
    torch.cuda.synchronize()
    return layer, O.cpu().numpy(), lse.cpu().numpy()


def check_rows(x, layer, O, lse, rows, budget, mode=0, kbar_mode=0, Qr=None, Kr=None, kb=None,
               pos0=0):
    """Oracle check of sampled rows: selection by the tie-band rule, outputs
    against the oracle's attention over the GPU's (validated) selection and,
    where the sets agree, the oracle's own end-to-end result."""
    Qr = oracle.rope(x.Q, pos0=pos0) if Qr is None else Qr
    Kr = oracle.rope(x.K) if Kr is None else Kr
    kb = oracle.compress(x.ki, mode=kbar_mode) if kb is None else kb
    sel_g = layer.blk_idx.cpu().numpy()[rows]
    ns_g = layer.n_sel.cpu().numpy()[rows]
    ref = oracle.select_rows(x.qi, kb, rows, pos0=pos0, Kbudget=budget, mode=mode,
                             want_scores=True)
    exempt = []
    for i, t in enumerate(rows):
        nc = min((pos0 + t + 1) // 4, kb.shape[0])
        if check_selection(ref["s"][i, :nc], budget, ref["sK"][i], ref["sK1"][i], sel_g[i],
                           ns_g[i]):
            exempt.append(int(t))
    log(f"  selection: {len(rows)} rows checked, {len(exempt)} differ inside the tie band")
    Oref, lref = oracle.sparse_attn_rows(Qr, Kr, x.V, rows, sel_g, ns_g, pos0=pos0)
    assert_close(O[rows], Oref, "O vs oracle on the GPU selection")
    assert_close(lse[rows], lref, "lse vs oracle on the GPU selection")
    same = np.array([t not in set(exempt) for t in rows])
    if same.any():
        e2e = oracle.qsa_rows(Qr, Kr, x.V, x.qi, kb, rows[same], pos0=pos0, Kbudget=budget,
                              mode=mode)
        assert_close(O[rows[same]], e2e["O"], "O vs oracle end to end")
        assert np.all(e2e["wsum_err"] < 1e-12)
    return exempt


# ------------------------------------------------ the small workload, full
@pytest.mark.parametrize("mode,kbar_mode", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_prefill_T2048_budget64_all_rows(qsa, mode, kbar_mode):
    """Single QSA layer prefill, T = 2048, budget 64 blocks, every row."""
    log(f"prefill T=2048 budget=64 score_mode={mode} kbar_mode={kbar_mode}")
    x = synth.prefill_inputs(2048, seed=0)
    layer, O, lse = run_prefill(qsa, x, 64, mode, kbar_mode)
    check_rows(x, layer, O, lse, np.arange(2048), 64, mode, kbar_mode)


def test_prefill_within_budget_is_dense(qsa):
    """Rows with nc <= K: QSA output equals the GPU dense kernel's (a
    different kernel, fp16 P.V, so to the parity tolerance)."""
    torch = _torch()
    T, K = 600, 64
    x = synth.prefill_inputs(T, seed=1)
    layer, O, _ = run_prefill(qsa, x, K)
    Od = torch.empty((T, 24, 256), dtype=torch.float32, device="cuda")
    Kr = layer.Kr
    qsa.dense_attn(layer.Qr, Kr, dev(x.V), 1, T, T, 0, None, 24, 2, 256, Od, None)
    torch.cuda.synchronize()
    n_dense = 4 * K + 3  # p < 259 -> nc(p) <= 64
    assert_close(O[:n_dense], Od.cpu().numpy()[:n_dense], "rows within budget: QSA vs dense")


@pytest.mark.parametrize("T,K", [(1, 1), (2, 1), (3, 1), (4, 1), (5, 1), (9, 2), (17, 3),
                                 (1029, 64)])
def test_prefill_edge_sizes(qsa, T, K):
    x = synth.prefill_inputs(T, seed=T)
    layer, O, lse = run_prefill(qsa, x, K)
    check_rows(x, layer, O, lse, np.arange(T), K)


def test_value_ones_give_ones(qsa):
    x = synth.prefill_inputs(700, seed=2)
    ones = np.full(x.V.shape, 0x3F80, dtype=np.uint16)
    x.V[...] = ones
    _, O, _ = run_prefill(qsa, x, 32)
    assert np.abs(O - 1.0).max() < 1e-6


def test_deterministic(qsa):
    x = synth.prefill_inputs(1500, seed=4)
    _, O1, l1 = run_prefill(qsa, x, 64)
    _, O2, l2 = run_prefill(qsa, x, 64)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def test_launch_sizes_give_the_same_bits(qsa):
    """The layer's default attention launch (the device's resident
    workgroups: CUs times the kernel's workgroups per CU) and other launch
    sizes, including one launch of all rows, give the same O and lse bits;
    so does the layer that rotates Q in a kernel of its own (rope_on_load
    off), whose stored Qr equals the one the default layer computes on
    demand."""
    torch = _torch()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    c = qsa.qsa_sparse_attn_prefill_concurrency(2, 64)
    assert c > 0 and c % cus == 0
    ckl = qsa.qsa_sparse_attn_prefill_concurrency(2, 64, with_kl=True)
    assert 0 < ckl <= c and ckl % cus == 0
    assert qsa.qsa_sparse_attn_prefill_concurrency(2, 64, paged=True) % cus == 0
    log(f"  resident workgroups: {c} plain, {ckl} with the KL ({cus} CUs)")
    T = 5000
    x = synth.prefill_inputs(T, seed=8)
    outs, qrs = [], []
    for rows, on_load in ((None, True), (0, True), (1000, True), (3333, True), (None, False)):
        layer = qsa.QSAPrefill(T, budget=64, attn_rows=rows, rope_on_load=on_load)
        assert layer.rope_on_load == on_load
        if rows is None:
            assert layer.attn_rows == c
        O, lse = layer(dev(x.Q), dev(x.K), dev(x.V), dev(x.qi), dev(x.ki))
        torch.cuda.synchronize()
        outs.append((O.cpu().numpy().copy(), lse.cpu().numpy().copy()))
        if rows is None:
            qrs.append(host_u16(layer.Qr))
    for O, lse in outs[1:]:
        assert np.array_equal(O, outs[0][0]) and np.array_equal(lse, outs[0][1])
    assert np.array_equal(qrs[0], qrs[1])


def test_chunked_prefill_matches_one_shot(qsa):
    """Two chunks against a post-RoPE cache reproduce the one-shot prefill."""
    torch = _torch()
    T, K, split = 2000, 64, 1200
    x = synth.prefill_inputs(T, seed=5)
    full, O, lse = run_prefill(qsa, x, K)
    Kr = full.Kr                       # post-RoPE cache of all positions
    kbar = torch.zeros((T // 4, 128), dtype=torch.bfloat16, device="cuda")
    outs = []
    for p0, n in [(0, split), (split, T - split)]:
        ch = qsa.QSAPrefill(n, pos0=p0, budget=K, fresh=False)
        Oc, _ = ch(dev(x.Q[p0:p0 + n]), Kr[:p0 + n], dev(x.V[:p0 + n]), dev(x.qi[p0:p0 + n]),
                   dev(x.ki), kbar)
        torch.cuda.synchronize()
        outs.append(Oc.cpu().numpy().copy())
    Ochunk = np.concatenate(outs)
    assert np.array_equal(Ochunk, O)


def test_decode_matches_last_prefill_row(qsa):
    torch = _torch()
    L, K = 3001, 64
    x = synth.prefill_inputs(L, seed=6)
    full, O, _ = run_prefill(qsa, x, K)
    kbar = full.kbar.view(1, L // 4, 128)
    dec = qsa.QSADecode(1, L, budget=K)
    sl = torch.tensor([L], dtype=torch.int64, device="cuda")
    Od, _ = dec(dev(x.Q[L - 1:L]), dev(x.qi[L - 1:L]), full.Kr[None], dev(x.V)[None], kbar, sl)
    torch.cuda.synchronize()
    assert np.array_equal(dec.blk_idx.cpu().numpy()[0], full.blk_idx.cpu().numpy()[L - 1])
    d = np.abs(Od.cpu().numpy()[0] - O[L - 1]).max()
    log(f"  decode vs prefill last row: max diff {d:.2e}")
    assert d < 1e-5
